// Pure streaming read of a large buffer: the achievable HBM read ceiling
// that the weight pass is measured against, beside the 8 TB/s data-sheet
// peak (the veloGB10 docs' "--probe-bandwidth", "Probes (diagnostics)",
// reports its GB10 read ceiling the same way).
//
// Each lane issues 16-byte nontemporal loads, four in flight per iteration,
// over a grid-stride walk; a workgroup writes one float so the loads cannot
// be removed.  Workgroups are spread over every CU (a multiple of the CU
// count), so consecutive blocks land on different XCDs.
#include "launch.h"
#include "nvfp4_device.h"

namespace vg {
namespace {

constexpr int kBlock = 256;
constexpr int kBlocksPerCU = 8;

__global__ __launch_bounds__(kBlock) void bwprobe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         float* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = ld_stream(p + i), b = ld_stream(p + i + stride);
    const u32x4 c = ld_stream(p + i + 2 * stride), d = ld_stream(p + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = ld_stream(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ unsigned red[kBlock / kWave];
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (float)(red[0] ^ red[1] ^ red[2] ^ red[3]);
}

int probe_blocks() {
  static int blocks = 0;
  if (!blocks) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    blocks = cus * kBlocksPerCU;
  }
  return blocks;
}

}  // namespace

size_t bwprobe_sink_floats() { return 4096; }

hipError_t launch_bwprobe(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  int blocks = probe_blocks();
  if ((size_t)blocks > bwprobe_sink_floats()) blocks = (int)bwprobe_sink_floats();
  hipLaunchKernelGGL(bwprobe_kernel, dim3(blocks), dim3(kBlock), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace vg

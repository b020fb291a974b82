// Pure streaming read of a large buffer: the achievable HBM read ceiling
// that the weight pass is measured against, beside the 8 TB/s data-sheet
// peak (the veloGB10 docs' "--probe-bandwidth", "Probes (diagnostics)",
// reports its GB10 read ceiling the same way).
//
// The load structure is the step kernel's: one 512-thread workgroup per CU
// streams one contiguous region of the buffer; each wave reads kPieces
// consecutive 1-KB pieces per round (lane i the 16 bytes at 16 i of each),
// nontemporal buffer loads whose range is exactly the region, the waves of
// a workgroup interleaved piece group by piece group.  Measured on MI355X
// over 8 GiB: 7.2 TB/s, against 6.3 TB/s for a grid-stride walk with four
// loads in flight per lane (both shapes swept: 1-16 pieces per round,
// 1-8 workgroups per CU, cached or nontemporal, software-pipelined or not:
// all within 7.0-7.2 TB/s except the cached forms, 6.1-6.2 TB/s).
#include "launch.h"
#include "nvfp4_device.h"

namespace vg {
namespace {

constexpr int kBlock = 512;
constexpr int kPieces = 4;   // 1-KB pieces per wave per round
constexpr int kNT = 2;       // buffer-load cache policy: nontemporal
constexpr size_t kMaxRegion = size_t(1) << 31;  // bytes per workgroup (32-bit buffer offsets)

__global__ __launch_bounds__(kBlock) void bwprobe_kernel(const unsigned char* __restrict__ buf, size_t bytes,
                                                         float* __restrict__ sink) {
  // region of this workgroup: whole 1-KB pieces (the regions cover every
  // byte; the last ones may be shorter or empty)
  const size_t per = ((bytes + gridDim.x - 1) / gridDim.x + 1023) & ~size_t(1023);
  const size_t beg = per * blockIdx.x;
  unsigned acc = 0;
  if (beg < bytes) {
    const size_t len = beg + per <= bytes ? per : bytes - beg;
    const __amdgpu_buffer_rsrc_t r = rsrc_uniform(buf + beg, (unsigned)len);
    const unsigned lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = kBlock / kWave;
    for (size_t base = (size_t)w * kPieces * 1024; base < len; base += (size_t)nw * kPieces * 1024) {
      u32x4 v[kPieces];
      // offsets past the region read zeros without touching memory
#pragma unroll
      for (int u = 0; u < kPieces; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (unsigned)(base + u * 1024 + 16 * lane), 0, kNT);
#pragma unroll
      for (int u = 0; u < kPieces; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
  }
  __shared__ unsigned red[kBlock / kWave];
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned v = 0;
    for (int i = 0; i < kBlock / kWave; ++i) v ^= red[i];
    sink[blockIdx.x] = (float)v;
  }
}

int probe_blocks() {
  static int blocks = 0;
  if (!blocks) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    blocks = cus;
  }
  return blocks;
}

}  // namespace

size_t bwprobe_sink_floats() { return 4096; }

hipError_t launch_bwprobe(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  int blocks = probe_blocks();
  if ((size_t)blocks > bwprobe_sink_floats()) blocks = (int)bwprobe_sink_floats();
  // more workgroups for buffers whose per-CU region would not fit 32-bit offsets
  while ((size_t)blocks < bwprobe_sink_floats() && bytes / (size_t)blocks >= kMaxRegion) blocks *= 2;
  if (bytes / (size_t)blocks >= kMaxRegion) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwprobe_kernel, dim3(blocks), dim3(kBlock), 0, stream, static_cast<const unsigned char*>(buf),
                     bytes, sink);
  return hipGetLastError();
}

}  // namespace vg

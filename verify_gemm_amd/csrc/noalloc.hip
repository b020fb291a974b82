// nvfp4_gemm_noalloc: nvfp4_gemm_ex for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The workspace nvfp4_gemm_ex takes from its caller --
// the K-slice sums of a narrow matrix's blocks and the per-block counters --
// is a file-scope device array here, `scratch`, of a fixed size per GPU
// (held by each GPU the library runs on until the process ends).
//
// In host code `scratch` names a host-side stand-in, not device memory:
// its device address is looked up once per device (hipGetSymbolAddress,
// with that device current) on the entry point's first call there, and only
// that address is ever handed to a kernel.  The same first call clears the
// whole array with a fill kernel on the caller's stream (no memset), ahead
// of its GEMM; every GEMM launch leaves the counters it used at zero again.
// Nothing here allocates: no hipMalloc, no hipFree, no allocating library
// routine.
//
// Every call on one GPU shares that GPU's array: calls that overlap in time
// on one GPU (other streams, or graph replays running concurrently) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "vgemm.h"

namespace {

static_assert(VG_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");

static __device__ __align__(256) unsigned char scratch[VG_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};
bool g_cleared[kMaxDevices] = {};

// Zeroes n 16-byte words (grid-stride).
__global__ void clear_scratch(uint4* p, unsigned n) {
  for (unsigned i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The device address of `scratch` on the current device (set up on the
// first call there), or nullptr if the lookup fails.  The first call also
// queues the clear on `stream`, ahead of the GEMM that follows.
void* scratch_ptr(hipStream_t stream, int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = VG_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = VG_ERR_HIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  if (!g_cleared[dev]) {
    const unsigned n = VG_NOALLOC_SCRATCH_BYTES / 16;
    hipLaunchKernelGGL(clear_scratch, dim3(1024), dim3(256), 0, stream, static_cast<uint4*>(g_ptr[dev]), n);
    if (hipGetLastError() != hipSuccess) {
      *status = VG_ERR_HIP;
      return nullptr;
    }
    g_cleared[dev] = true;
  }
  *status = VG_OK;
  return g_ptr[dev];
}

}  // namespace

extern "C" int nvfp4_gemm_noalloc(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float gscale,
                                  int M, int N, int K, float* Y, void* stream) {
  // arguments first, exactly as nvfp4_gemm checks them (no HIP call yet)
  if (!X || !Wq || !Ws || !Y) return VG_ERR_NULL;
  if (M < 1 || N < 1 || K < 16 || (K % 16) != 0) return VG_ERR_SHAPE;
  if (M > VG_MAX_M) return VG_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Wq) | reinterpret_cast<uintptr_t>(Ws)) & 15u)
    return VG_ERR_ALIGN;
  const size_t need = vg_gemm_workspace_bytes(M, N, K);
  if (need > (size_t)VG_NOALLOC_SCRATCH_BYTES) return VG_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (need == 0)  // not sliced: nvfp4_gemm_ex ignores a workspace for this shape
    return nvfp4_gemm_ex(X, Wq, Ws, gscale, M, N, K, Y, nullptr, 0, stream);
  int st = VG_OK;
  void* ptr = scratch_ptr(s, &st);
  if (!ptr) return st;
  return nvfp4_gemm_ex(X, Wq, Ws, gscale, M, N, K, Y, ptr, (size_t)VG_NOALLOC_SCRATCH_BYTES, stream);
}

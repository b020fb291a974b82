// Internal launcher interface between the C-ABI layer (api.cpp) and the
// kernels.  Every launcher assumes its arguments were validated by the
// caller and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vg {

// Split-K bookkeeping of the MFMA GEMM: how many K-splits a shape uses and
// how the caller's workspace is carved up.
struct GemmPlan {
  int mt;          // 16-row M-tiles (1..5)
  int nt;          // 16-row N-tiles per wave
  int ntiles;      // N-tiles of 16*nt rows
  int splits;      // K-splits (1 = no workspace)
  int kchunk;      // K elements per split (multiple of 128 unless splits == 1)
  size_t counter_bytes;
  size_t partial_bytes;
  size_t workspace_bytes() const { return splits > 1 ? counter_bytes + partial_bytes : 0; }
};
GemmPlan plan_gemm(int M, int N, int K);

// Workspace of the lm_head pass: arg-max keys + an arrival counter.
struct LmheadWorkspace {
  unsigned long long keys[128];
  unsigned counter;
  unsigned pad[63];
};

hipError_t launch_gemv_m1(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int N,
                          int K, float* Y, hipStream_t stream);
hipError_t launch_gemm_mfma(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int M,
                            int N, int K, float* Y, void* workspace, const GemmPlan& plan,
                            hipStream_t stream);
hipError_t launch_lmhead_m1(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int K,
                            int V, const int32_t* drafts, int32_t* argmax, int32_t* accept_len,
                            LmheadWorkspace* ws, hipStream_t stream);
hipError_t launch_lmhead_mfma(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g,
                              int M, int K, int V, int T, const int32_t* drafts, int32_t* argmax,
                              int32_t* accept_len, LmheadWorkspace* ws, hipStream_t stream);
hipError_t launch_bwprobe(const void* buf, size_t bytes, float* sink, hipStream_t stream);
size_t bwprobe_sink_floats();

}  // namespace vg

// The end of the lm_head verify pass, shared by the M = 1 and MFMA kernels.
//
// Each workgroup has found, for every row m, its best (logit, index) over
// the vocabulary rows it owns.  It publishes that as one 64-bit key per row
// with an unsigned atomic max (order independent, so the result does not
// depend on which workgroup finishes first), then counts itself in.  The
// last workgroup to arrive reads the winning keys, writes argmax[M], runs
// the greedy accept rule per sequence (TandemLLM README, introduction: keep
// the longest prefix the target agrees with; at the first wrong guess the
// target's own token is emitted), and resets the keys and the counter so
// the workspace is zero again for the next call (no host memset, so the
// pass can be replayed from a graph).
#pragma once

#include "launch.h"
#include "nvfp4_device.h"

namespace vg {

// best_v / best_i: [waves_per_block][M] in LDS, filled by every wave.
__device__ __forceinline__ void lmhead_finish(const float* best_v, const int* best_i,
                                              int waves_per_block, int M, int T,
                                              const int32_t* drafts, int32_t* argmax,
                                              int32_t* accept_len, LmheadWorkspace* ws,
                                              int* lds_am /* [M] */, int* lds_last) {
  const int tid = threadIdx.x;
  if (tid < M) {
    float v = best_v[tid];
    int i = best_i[tid];
    for (int w = 1; w < waves_per_block; ++w) {
      float vw = best_v[w * M + tid];
      int iw = best_i[w * M + tid];
      if (better(vw, iw, v, i)) { v = vw; i = iw; }
    }
    if (i >= 0)
      __hip_atomic_fetch_max(&ws->keys[tid], argmax_key(v, (unsigned)i), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    unsigned prev = __hip_atomic_fetch_add(&ws->counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *lds_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!*lds_last) return;
  __threadfence();
  if (tid < M) {
    unsigned long long key = __hip_atomic_load(&ws->keys[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int am = (int)key_index(key);
    lds_am[tid] = am;
    argmax[tid] = am;
    __hip_atomic_store(&ws->keys[tid], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int S = M / T;
  if (tid < S) {
    int L = 0;
    const int32_t* d = drafts + (size_t)tid * (T - 1);
    while (L < T - 1 && d[L] == lds_am[tid * T + L]) ++L;
    accept_len[tid] = L;
  }
  if (tid == 0) __hip_atomic_store(&ws->counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace vg

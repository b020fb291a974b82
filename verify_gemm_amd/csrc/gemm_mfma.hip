// M >= 2: the speculative-verify GEMM (M = 17: 16 drafts + 1; up to 68 =
// 4 sequences x 17) and its lm_head pass on the matrix cores.
//
// At 17+ rows every weight element feeds 17+ products, too many for the
// vector ALU at HBM speed, so the product runs on MFMA
// (v_mfma_f32_16x16x32_bf16).  The E4M3 x E2M1 product has at most 6
// significant bits, so dequantising to bf16 is exact and the only rounding
// is the fp32 accumulation -- the same bar as the M = 1 path.  The veloGB10
// docs ("Unique aspects") describe the GB10 engine's block-scaled
// tensor-core GEMM; this is the CDNA4 counterpart, not a translation.
//
// Work decomposition (one wave = one work item, 4 independent waves per
// workgroup):
//   * a wave owns NT N-tiles of 16 weight rows (16*NT rows) and a K-range;
//     lane (c = lane % 16, g = lane / 16) streams the 16-byte code chunk
//     [kwin/2 + 16g, +16) of row n0 + 16*nt + c per 128-element window, i.e.
//     64 contiguous bytes per row and instruction, nontemporal;
//   * code dword t of that chunk is the B operand of MFMA step t: the K
//     positions kwin + 32g + 8t + j, so X is read in the same permuted
//     order (a consistent permutation of K leaves the dot product intact);
//   * every X fragment (16 B per lane per M-tile and step) is reused by the
//     NT N-tiles of the wave;
//   * rows m >= M of the last M-tile are zero operands and are not stored;
//   * when one wave per N-tile would leave the GPU idle, K is split S ways;
//     each split writes an unscaled partial tile to the workspace, and the
//     last of the S waves to arrive (an agent-scope counter) sums the S
//     partials in split order 0..S-1 -- a fixed order, so results are
//     bitwise repeatable -- scales by g, stores Y and resets its counter.
//     The eight XCDs have separate L2 caches, so partials are written and
//     read with agent-scope accesses (coherent across XCDs); plain accesses
//     could hit a line another XCD's L2 still holds from an earlier call.
#include "launch.h"
#include "lmhead_finish.h"
#include "nvfp4_device.h"

namespace vg {
namespace {

constexpr int kBlock = 256;  // 4 independent waves
constexpr int kNT = 4;       // 64 weight rows per wave
// K is split only for shapes with fewer N-tiles than this; it also sizes the
// fixed counter region at the start of a GEMM workspace.
constexpr int kMaxSplitTiles = 1024;

template <int MT, int NT>
struct Tile {
  f32x4 acc[MT][NT];
};

// One 128-element K window, all loads predicated (any K % 16 == 0, any
// alignment of rows).  Elements at or past kend contribute zero.
template <int MT, int NT>
__device__ __forceinline__ void window_guarded(const uint16_t* __restrict__ X, int M, int K,
                                               const uint8_t* const (&wrow)[NT],
                                               const uint8_t* const (&srow)[NT], int kwin, int kend,
                                               Tile<MT, NT>& t) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int e0 = kwin + 32 * g + 8 * st;
    const bool ok = e0 < kend;
    bf16x8 b[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      unsigned w = 0;
      float s = 0.0f;
      if (ok) {
        w = ld_stream(reinterpret_cast<const unsigned*>(wrow[nt] + (e0 >> 1)));
        s = e4m3x2_lo(ld_stream(srow[nt] + (e0 >> 4)))[0];
      }
      b[nt] = dequant8_bf16(w, s);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + c;
      u32x4 a = {0u, 0u, 0u, 0u};
      if (ok && m < M) a = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + e0);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        t.acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b[nt],
                                                                t.acc[mt][nt], 0, 0, 0);
    }
  }
}

// Accumulate the K-range [kb, ke) of the wave's tile.  ALIGNED: K % 32 == 0
// (16-byte code chunks and 2-byte scale pairs are aligned); full 128-element
// windows then take the fast path and only a trailing partial window is
// guarded.
template <int MT, int NT, bool ALIGNED>
__device__ __forceinline__ void mfma_tile(const uint16_t* __restrict__ X, int M, int K,
                                          const uint8_t* __restrict__ Wq,
                                          const uint8_t* __restrict__ Ws, int N, int n0, int kb,
                                          int ke, Tile<MT, NT>& t) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const uint8_t* wrow[NT];
  const uint8_t* srow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int n = n0 + 16 * nt + c;
    n = n < N ? n : N - 1;  // rows past N re-read the last row; never stored
    wrow[nt] = Wq + (size_t)n * (size_t)(K >> 1);
    srow[nt] = Ws + (size_t)n * (size_t)(K >> 4);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) t.acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int kwin = kb;
  if (ALIGNED) {
    const u32x4* xrow[MT];
    bool mok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + c;
      mok[mt] = m < M;
      xrow[mt] = reinterpret_cast<const u32x4*>(X + (size_t)(mok[mt] ? m : 0) * K);
    }
    for (; kwin + 128 <= ke; kwin += 128) {
      u32x4 q[NT];
      unsigned short sc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        q[nt] = ld_stream(reinterpret_cast<const u32x4*>(wrow[nt] + (kwin >> 1)) + g);
        sc[nt] = ld_stream(reinterpret_cast<const unsigned short*>(srow[nt] + (kwin >> 4)) + g);
      }
      u32x4 xa[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          xa[mt][st] = mok[mt] ? xrow[mt][((kwin + 32 * g) >> 3) + st] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 b[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f32x2 s = e4m3x2_lo(sc[nt]);
          b[nt] = dequant8_bf16(q[nt][st], st < 2 ? s[0] : s[1]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            t.acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xa[mt][st]), b[nt], t.acc[mt][nt], 0, 0, 0);
      }
    }
  }
  for (; kwin < ke; kwin += 128) window_guarded<MT, NT>(X, M, K, wrow, srow, kwin, ke, t);
}

// ---- GEMM -------------------------------------------------------------------
template <int MT, int NT, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void gemm_mfma_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    float g, int M, int N, int K, float* __restrict__ Y, int ntiles, int splits, int kchunk,
    unsigned* __restrict__ counters, float* __restrict__ partials) {
  const int item = (blockIdx.x * kBlock + threadIdx.x) >> 6;
  if (item >= ntiles * splits) return;
  // consecutive items of one tile land on consecutive waves of a block and
  // consecutive blocks, keeping a tile's splits close in time
  const int tile = item / splits, split = item % splits;
  const int n0 = tile * 16 * NT;
  const int kb = split * kchunk;
  const int ke = split == splits - 1 ? K : kb + kchunk;
  Tile<MT, NT> t;
  mfma_tile<MT, NT, ALIGNED>(X, M, K, Wq, Ws, N, n0, kb, ke, t);

  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  if (splits == 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * gq + r;
        if (m < M) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int n = n0 + 16 * nt + c;
            if (n < N) Y[(size_t)m * N + n] = t.acc[mt][nt][r] * g;
          }
        }
      }
    return;
  }
  // split-K: publish the partial tile, the last arrival reduces in order
  constexpr int TN = 16 * NT;
  float* part = partials + ((size_t)tile * splits) * (size_t)M * TN;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * gq + r;
      if (m < M) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          __hip_atomic_store(&part[((size_t)split * M + m) * TN + 16 * nt + c], t.acc[mt][nt][r],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  __threadfence();
  unsigned prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, kWave);
  if (prev != (unsigned)(splits - 1)) return;
  __threadfence();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * gq + r;
      if (m < M) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = n0 + 16 * nt + c;
          float v = 0.0f;
          for (int s = 0; s < splits; ++s)
            v += __hip_atomic_load(&part[((size_t)s * M + m) * TN + 16 * nt + c], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          if (n < N) Y[(size_t)m * N + n] = v * g;
        }
      }
    }
  if (lane == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- lm_head ----------------------------------------------------------------
template <int MT, int NT, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void lmhead_mfma_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    float g, int M, int K, int V, int T, const int32_t* drafts, int32_t* argmax, int32_t* accept_len,
    LmheadWorkspace* ws) {
  __shared__ float best_v[(kBlock / kWave) * 16 * MT];
  __shared__ int best_i[(kBlock / kWave) * 16 * MT];
  __shared__ int lds_am[16 * MT];
  __shared__ int lds_last;
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int wv = threadIdx.x >> 6;
  const int wave = (blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int waves = (gridDim.x * kBlock) >> 6;
  const int ntiles = (V + 16 * NT - 1) / (16 * NT);
  float bv[MT][4];
  int bi[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) { bv[mt][r] = -__builtin_inff(); bi[mt][r] = -1; }

  for (int tile = wave; tile < ntiles; tile += waves) {
    const int n0 = tile * 16 * NT;
    Tile<MT, NT> t;
    mfma_tile<MT, NT, ALIGNED>(X, M, K, Wq, Ws, V, n0, 0, K, t);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + 16 * nt + c;
      if (n < V) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = t.acc[mt][nt][r] * g;
            if (better(v, n, bv[mt][r], bi[mt][r])) { bv[mt][r] = v; bi[mt][r] = n; }
          }
      }
    }
  }
  // reduce across the 16 lanes that share rows (same g, different column)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv[mt][r], off, kWave);
        const int oi = __shfl_xor(bi[mt][r], off, kWave);
        if (oi >= 0 && (bi[mt][r] < 0 || better(ov, oi, bv[mt][r], bi[mt][r]))) {
          bv[mt][r] = ov;
          bi[mt][r] = oi;
        }
      }
      const int m = 16 * mt + 4 * gq + r;
      if (c == 0 && m < M) {
        best_v[wv * M + m] = bv[mt][r];
        best_i[wv * M + m] = bi[mt][r];
      }
    }
  __syncthreads();
  lmhead_finish(best_v, best_i, kBlock / kWave, M, T, drafts, argmax, accept_len, ws, lds_am,
                &lds_last);
}

int num_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
  }
  return cus;
}

template <int MT>
hipError_t gemm_dispatch_mt(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int M,
                            int N, int K, float* Y, void* workspace, const GemmPlan& p,
                            hipStream_t stream) {
  unsigned* counters = nullptr;
  float* partials = nullptr;
  if (p.splits > 1) {
    counters = static_cast<unsigned*>(workspace);
    partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.counter_bytes);
  }
  const int items = p.ntiles * p.splits;
  const int blocks = (items + 3) / 4;
  if ((K & 31) == 0)
    hipLaunchKernelGGL((gemm_mfma_kernel<MT, kNT, true>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq,
                       Ws, g, M, N, K, Y, p.ntiles, p.splits, p.kchunk, counters, partials);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<MT, kNT, false>), dim3(blocks), dim3(kBlock), 0, stream, X,
                       Wq, Ws, g, M, N, K, Y, p.ntiles, p.splits, p.kchunk, counters, partials);
  return hipGetLastError();
}

template <int MT>
hipError_t lmhead_dispatch_mt(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int M,
                              int K, int V, int T, const int32_t* drafts, int32_t* argmax,
                              int32_t* accept_len, LmheadWorkspace* ws, hipStream_t stream) {
  const int ntiles = (V + 16 * kNT - 1) / (16 * kNT);
  int blocks = (ntiles + 3) / 4;
  const int cap = num_cus() * 4;
  if (blocks > cap) blocks = cap;
  if ((K & 31) == 0)
    hipLaunchKernelGGL((lmhead_mfma_kernel<MT, kNT, true>), dim3(blocks), dim3(kBlock), 0, stream, X,
                       Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws);
  else
    hipLaunchKernelGGL((lmhead_mfma_kernel<MT, kNT, false>), dim3(blocks), dim3(kBlock), 0, stream,
                       X, Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan p{};
  p.mt = (M + 15) / 16;
  p.nt = kNT;
  p.ntiles = (N + 16 * kNT - 1) / (16 * kNT);
  const int windows = (K + 127) / 128;
  // Aim for >= ~4 waves per CU; split K only in whole 128-element windows.
  const int target = kMaxSplitTiles;
  int splits = 1;
  if (p.ntiles < target) {
    splits = (target + p.ntiles - 1) / p.ntiles;
    if (splits > windows) splits = windows;
    if (splits < 1) splits = 1;
  }
  int wper = (windows + splits - 1) / splits;  // windows per split
  splits = (windows + wper - 1) / wper;        // drop empty splits
  p.splits = splits;
  p.kchunk = splits > 1 ? wper * 128 : K;
  // The counter region has a fixed size for every shape, so the partials of
  // one shape can never land on the counters of another when a workspace is
  // reused across shapes (counters must stay zero between calls).
  p.counter_bytes = kMaxSplitTiles * sizeof(unsigned);
  p.partial_bytes = (size_t)p.ntiles * splits * (size_t)M * 16 * kNT * sizeof(float);
  return p;
}

hipError_t launch_gemm_mfma(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int M,
                            int N, int K, float* Y, void* workspace, const GemmPlan& p,
                            hipStream_t stream) {
  switch (p.mt) {
    case 1: return gemm_dispatch_mt<1>(X, Wq, Ws, g, M, N, K, Y, workspace, p, stream);
    case 2: return gemm_dispatch_mt<2>(X, Wq, Ws, g, M, N, K, Y, workspace, p, stream);
    case 3: return gemm_dispatch_mt<3>(X, Wq, Ws, g, M, N, K, Y, workspace, p, stream);
    case 4: return gemm_dispatch_mt<4>(X, Wq, Ws, g, M, N, K, Y, workspace, p, stream);
    case 5: return gemm_dispatch_mt<5>(X, Wq, Ws, g, M, N, K, Y, workspace, p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lmhead_mfma(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g,
                              int M, int K, int V, int T, const int32_t* drafts, int32_t* argmax,
                              int32_t* accept_len, LmheadWorkspace* ws, hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return lmhead_dispatch_mt<1>(X, Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws, stream);
    case 2: return lmhead_dispatch_mt<2>(X, Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws, stream);
    case 3: return lmhead_dispatch_mt<3>(X, Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws, stream);
    case 4: return lmhead_dispatch_mt<4>(X, Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws, stream);
    case 5: return lmhead_dispatch_mt<5>(X, Wq, Ws, g, M, K, V, T, drafts, argmax, accept_len, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vg

// M = 1: the plain-decode GEMV y[n] = g * sum_k x[k] * s[n, k/16] * e[n, k]
// and the lm_head pass at M = 1 (argmax over V rows).
//
// A decode step streams every weight once and is bound by memory bandwidth
// (ling-engine README, opening: the bus, not compute, bounds decoding;
// veloGB10 docs, "Engineered to the roofline").  At one row of X there is
// no reuse to exploit, so this path stays on the vector ALU:
//   * each half-wave (32 lanes) owns one weight row at a time; lane L reads
//     16-byte chunks L, L+32, ... of the packed codes (512 contiguous bytes
//     per half-wave and instruction) with nontemporal loads, plus the two
//     E4M3 scale bytes of each chunk;
//   * per 16-block, 8 v_dot2_f32_bf16 against X multiply the unscaled E2M1
//     values (exact in bf16) and one FMA applies the block scale, so the
//     ALU cost is ~1.1 ops per weight element;
//   * each lane carries RH rows (rows 2i + half) for the same chunk, so one
//     X fetch (64 B per chunk, from L1/L2) serves RH weight rows;
//   * the 32 partial sums of a row meet in a shuffle tree; no split-K and
//     no workspace: every output is owned by exactly one half-wave, so the
//     result is bitwise repeatable.
// Shapes with K % 1024 != 0 take a generic path that walks 16-element
// blocks with 8-byte loads (any K % 16 == 0).
#include "launch.h"
#include "lmhead_finish.h"
#include "nvfp4_device.h"

namespace vg {
namespace {

constexpr int kBlock = 256;  // 4 waves

// Row sums of the RH rows this lane carries (valid in every lane of the
// half-wave after the shuffle reduction).  rowbase = first row of the wave.
template <int NJ, int RH>
__device__ __forceinline__ void gemv_rows_fast(const uint16_t* __restrict__ X,
                                               const uint8_t* __restrict__ Wq,
                                               const uint8_t* __restrict__ Ws, int N, int K,
                                               int rowbase, float (&acc)[RH]) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, L = lane & 31;
  const int nj = NJ ? NJ : (K >> 10);
  const size_t rb = (size_t)K >> 1, sb = (size_t)K >> 4;
  const u32x4* __restrict__ xp = reinterpret_cast<const u32x4*>(X);
  const u32x4* wp[RH];
  const unsigned short* sp[RH];
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    int r = rowbase + 2 * i + h;
    r = r < N ? r : N - 1;  // rows past N re-read the last row; never stored
    wp[i] = reinterpret_cast<const u32x4*>(Wq + (size_t)r * rb);
    sp[i] = reinterpret_cast<const unsigned short*>(Ws + (size_t)r * sb);
    acc[i] = 0.0f;
  }
#pragma unroll(NJ ? NJ : 4)
  for (int j = 0; j < nj; ++j) {
    const int c = L + 32 * j;
    u32x4 q[RH];
    unsigned short sc[RH];
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      q[i] = ld_stream(wp[i] + c);
      sc[i] = ld_stream(sp[i] + c);
    }
    const u32x4 x0 = xp[4 * c], x1 = xp[4 * c + 1], x2 = xp[4 * c + 2], x3 = xp[4 * c + 3];
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      const f32x2 s = e4m3x2_lo(sc[i]);
      acc[i] = block16(q[i][0], q[i][1], x0, x1, s[0], acc[i]);
      acc[i] = block16(q[i][2], q[i][3], x2, x3, s[1], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < RH; ++i) acc[i] = sum_lanes<32>(acc[i]);
}

// Generic K: one 16-element block (8 code bytes, 1 scale byte) per lane step;
// the whole wave owns one row.
__device__ __forceinline__ float gemv_row_generic(const uint16_t* __restrict__ X,
                                                  const uint8_t* __restrict__ Wq,
                                                  const uint8_t* __restrict__ Ws, int K, int r) {
  const int lane = threadIdx.x & 63;
  const int nb = K >> 4;
  const uint8_t* wrow = Wq + (size_t)r * (K >> 1);
  const uint8_t* srow = Ws + (size_t)r * nb;
  float acc = 0.0f;
  for (int b = lane; b < nb; b += kWave) {
    const unsigned* cw = reinterpret_cast<const unsigned*>(wrow + 8 * (size_t)b);
    const unsigned c0 = ld_stream(cw), c1 = ld_stream(cw + 1);
    const float s = e4m3x2_lo(ld_stream(srow + b))[0];
    const u32x4* xb = reinterpret_cast<const u32x4*>(X + 16 * (size_t)b);
    acc = block16(c0, c1, xb[0], xb[1], s, acc);
  }
  return sum_lanes<64>(acc);
}

template <int NJ, int RH>
__global__ __launch_bounds__(kBlock) void gemv_m1_fast(const uint16_t* __restrict__ X,
                                                       const uint8_t* __restrict__ Wq,
                                                       const uint8_t* __restrict__ Ws, float g,
                                                       int N, int K, float* __restrict__ Y) {
  const int wave = (blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int rowbase = wave * 2 * RH;
  if (rowbase >= N) return;
  float acc[RH];
  gemv_rows_fast<NJ, RH>(X, Wq, Ws, N, K, rowbase, acc);
  const int lane = threadIdx.x & 63;
  if ((lane & 31) == 0) {
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      const int r = rowbase + 2 * i + (lane >> 5);
      if (r < N) Y[r] = acc[i] * g;
    }
  }
}

__global__ __launch_bounds__(kBlock) void gemv_m1_generic(const uint16_t* __restrict__ X,
                                                          const uint8_t* __restrict__ Wq,
                                                          const uint8_t* __restrict__ Ws, float g,
                                                          int N, int K, float* __restrict__ Y) {
  const int wave = (blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int waves = (gridDim.x * kBlock) >> 6;
  for (int r = wave; r < N; r += waves) {
    const float v = gemv_row_generic(X, Wq, Ws, K, r);
    if ((threadIdx.x & 63) == 0) Y[r] = v * g;
  }
}

// lm_head at M = 1: grid-stride over row groups, running best per lane,
// then the shared finish (argmax; accept_len is 0 for a single row).
template <int NJ, int RH>
__global__ __launch_bounds__(kBlock) void lmhead_m1_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Ws,
    float g, int K, int V, const int32_t* drafts, int32_t* argmax, int32_t* accept_len,
    LmheadWorkspace* ws) {
  __shared__ float best_v[kBlock / kWave];
  __shared__ int best_i[kBlock / kWave];
  __shared__ int lds_am[1];
  __shared__ int lds_last;
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * kBlock + threadIdx.x) >> 6;
  const int waves = (gridDim.x * kBlock) >> 6;
  float bv = -__builtin_inff();
  int bi = -1;
  const bool fast = (K & 1023) == 0;
  if (fast) {
    for (int rowbase = wave * 2 * RH; rowbase < V; rowbase += waves * 2 * RH) {
      float acc[RH];
      gemv_rows_fast<NJ, RH>(X, Wq, Ws, V, K, rowbase, acc);
#pragma unroll
      for (int i = 0; i < RH; ++i) {
        const int r = rowbase + 2 * i + (lane >> 5);
        const float v = acc[i] * g;
        if (r < V && better(v, r, bv, bi)) { bv = v; bi = r; }
      }
    }
  } else {
    for (int r = wave; r < V; r += waves) {
      const float v = gemv_row_generic(X, Wq, Ws, K, r) * g;
      if (better(v, r, bv, bi)) { bv = v; bi = r; }
    }
  }
  // the two half-waves hold different rows
  const float ov = __shfl_xor(bv, 32, kWave);
  const int oi = __shfl_xor(bi, 32, kWave);
  if (oi >= 0 && better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  if (lane == 0) {
    best_v[threadIdx.x >> 6] = bv;
    best_i[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  lmhead_finish(best_v, best_i, kBlock / kWave, 1, 1, drafts, argmax, accept_len, ws, lds_am,
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

}  // namespace

hipError_t launch_gemv_m1(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int N,
                          int K, float* Y, hipStream_t stream) {
  if ((K & 1023) == 0) {
    constexpr int RH = 2;  // rows per half-wave -> 4 rows per wave
    const int waves = (N + 2 * RH - 1) / (2 * RH);
    const int blocks = (waves + 3) / 4;
    const int nj = K >> 10;
    if (nj == 5)
      hipLaunchKernelGGL((gemv_m1_fast<5, RH>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g, N, K, Y);
    else if (nj == 17)
      hipLaunchKernelGGL((gemv_m1_fast<17, RH>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g, N, K, Y);
    else if (nj == 1)
      hipLaunchKernelGGL((gemv_m1_fast<1, RH>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g, N, K, Y);
    else
      hipLaunchKernelGGL((gemv_m1_fast<0, RH>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g, N, K, Y);
  } else {
    const int waves = N;
    int blocks = (waves + 3) / 4;
    const int cap = num_cus() * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(gemv_m1_generic, dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g, N, K, Y);
  }
  return hipGetLastError();
}

hipError_t launch_lmhead_m1(const uint16_t* X, const uint8_t* Wq, const uint8_t* Ws, float g, int K,
                            int V, const int32_t* drafts, int32_t* argmax, int32_t* accept_len,
                            LmheadWorkspace* ws, hipStream_t stream) {
  constexpr int RH = 2;
  const int groups = (V + 2 * RH - 1) / (2 * RH);
  int blocks = (groups + 3) / 4;
  const int cap = num_cus() * 8;
  if (blocks > cap) blocks = cap;
  if ((K >> 10) == 5 && (K & 1023) == 0)
    hipLaunchKernelGGL((lmhead_m1_kernel<5, RH>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g,
                       K, V, drafts, argmax, accept_len, ws);
  else
    hipLaunchKernelGGL((lmhead_m1_kernel<0, RH>), dim3(blocks), dim3(kBlock), 0, stream, X, Wq, Ws, g,
                       K, V, drafts, argmax, accept_len, ws);
  return hipGetLastError();
}

}  // namespace vg

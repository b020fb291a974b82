// The weight-streaming kernels for batches of M >= 2 rows (and M = 1 shapes
// or formats the step kernel does not take): a single GEMM, the lm_head
// verify pass, and a whole decode / verify step as one persistent launch.
//
// A step of the ~27B hybrid reads every weight once and is bound by memory
// bandwidth (ling-engine README, opening paragraph and "Six levers";
// veloGB10 docs, "Engineered to the roofline").  The unit of work is an
// ITEM: a block of 64 weight rows -- or one K slice of such a block -- run
// by one 256-thread workgroup.  Three launch modes:
//
//   * DIRECT: one item per workgroup, dealt by the hardware dispatcher.
//     A single GEMM, or the jobs of one stage of a step -- the step's
//     default M >= 2 schedule (one launch per stage, which measured faster
//     than one persistent launch there).  With a slice workspace, a narrow
//     matrix's blocks are dealt as K slices (below) so that every CU has
//     work;
//   * GRID: resident workgroups walk the lm_head's blocks;
//   * STATIC: the whole step as one persistent launch: items numbered in
//     pass order, dealt round-robin to co-resident workgroups.  An item of
//     stage s (the per-layer order {q,k,v} -> o -> {gate,up} -> down ->
//     ... -> lm_head) consumes its activations only once stage s-1 is done;
//     a workgroup issues the item's weight loads FIRST and only then waits.
//     Completion is signalled once per workgroup and stage, on one of
//     eight counters per stage; waits are bounded and raise an error flag
//     instead of hanging.
//
// M >= 2, K % 128 == 0 (MfmaLdsItem): the four waves split the block's rows
// and walk K together in 256-element windows; the activations are staged
// once per workgroup through an LDS double buffer (with five M-tiles its
// slots sit M rows apart, so two workgroups fit on a CU); weights are dequantised
// exactly to bf16 (E4M3 x E2M1 has <= 6 significant bits; FP8 E4M3 is exact
// too) and multiplied on v_mfma_f32_16x16x32_bf16.  A row's NVFP4 scales
// are fetched once per group of ring windows and passed between the row's
// lanes through LDS.  A block's sum over K is
// taken as up to three K slices, each summed from zero, added in slice
// order -- by the one workgroup that runs them all, or, with the slices
// dealt as separate items, by the workgroup that completes the block: the
// same bits either way, no float atomics, bitwise repeatable, and a row's
// value independent of M.  Other K take the K-split guarded items.  M = 1:
// GEMV items (a half-wave or a wave per row, v_dot2_f32_bf16 on the
// unscaled E2M1 values, one FMA per 16-block applies the E4M3 scale).
//
// Each weight format is a kernel of its own, and a launch whose every K is
// a multiple of 128 takes a kernel without the guarded items: one kind's
// registers do not crowd another's.
//
// The lm_head never writes logits: its running best (logit, lowest index)
// per row -- in a per-wave LDS table with M-tiles -- is published once per
// workgroup as a 64-bit key with an unsigned atomic max into one of 16
// slots per row; the last workgroup to leave reads the slots, writes the
// argmax, runs the accept rule per sequence (TandemLLM README, introduction:
// keep the longest agreeing prefix, the target's own token replaces the
// first wrong guess) and zeroes the control block for the next launch -- no
// host memset, so a step can be replayed from a graph.
#pragma once

#include <type_traits>

#include "launch.h"
#include "nvfp4_device.h"

namespace vg {

namespace {

constexpr int kWG = 256;
constexpr int kWaves = kWG / kWave;
// A stage wait gives up after half a second of wall-clock time (the GPU's
// constant 100 MHz counter, s_memrealtime) and raises the error flag.
constexpr unsigned long long kStageWaitTicks = 50000000ull;
constexpr unsigned kOOB = 0x80000000u;  // buffer offset past every range used here
constexpr int kNT = 2;                  // buffer-load cache policy: nontemporal

// ---------------------------------------------------------------------------
// control block helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Output stores are agent-coherent (they write through the XCD's L2), so
// a consumer on another XCD sees them once the producer's count is visible.
__device__ __forceinline__ void store_out(float* p, float v) {
  __hip_atomic_store((VG_GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The scale of output row n of a job with per-row scales, 1 otherwise.  A
// GEMM job that stacks matrices keeps each member's tensor scale this way
// (its g is 1, so the row sum is exact up to the store, and sum * scale is
// the same single rounding as sum * g of a job with one scale); an FP8
// job's per-row scales multiply its outputs, or its logits before the
// argmax.  Read right after the item's weight loads are issued, so the
// value has long arrived when the result is used.
__device__ __forceinline__ float row_scale(const StreamJob& j, int n) {
  return j.gr && n < j.n ? j.gr[n] : 1.0f;
}

// Thread 0 polls until `target` workgroups have signalled stage `s`.
__device__ bool wait_stage(StageCounter (*sd)[kDoneSlots], StreamCtl* ctl, int s, unsigned target) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    unsigned sum = 0;
#pragma unroll
    for (int k = 0; k < kDoneSlots; ++k) sum += ld_agent(&sd[s][k].v);
    if (sum >= target) {
      // agent-scope acquire: drop stale lines so this workgroup's later
      // activation reads see what the previous stage wrote
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    if (__builtin_amdgcn_s_memrealtime() - t0 > kStageWaitTicks) break;
    __builtin_amdgcn_s_sleep(2);
  }
  st_agent(&ctl->error, 1u);
  return false;
}

// ---------------------------------------------------------------------------
// M = 1 items
// ---------------------------------------------------------------------------
// CPL = K / 1024 chunks per lane (compile time), RH rows per half-wave: a
// wave owns 2*RH rows, an item 8*RH rows.  All weight loads of the item are
// issued by issue(); compute() needs the activations.
template <int CPL, int RH>
struct GemvItem {
  static constexpr int kRows = 2 * RH * kWaves;
  u32x4 q[CPL][RH];
  unsigned short sc[CPL][RH];
  int row0;

  __device__ __forceinline__ void issue(const StreamJob& j, int item) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, L = lane & 31;
    row0 = item * kRows + w * 2 * RH;
    const size_t rb = (size_t)j.k >> 1, sb = (size_t)j.k >> 4;
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      int r = row0 + 2 * i + h;
      r = r < j.n ? r : j.n - 1;  // rows past N re-read the last row; never stored
      const u32x4* wp = reinterpret_cast<const u32x4*>(j.wq + (size_t)r * rb);
      const unsigned short* sp = reinterpret_cast<const unsigned short*>(j.ws + (size_t)r * sb);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        q[c][i] = ld_stream(wp + L + 32 * c);
        sc[c][i] = ld_stream(sp + L + 32 * c);
      }
    }
  }

  // Row sums (identical in every lane of the half-wave) times g.
  __device__ __forceinline__ void compute(const StreamJob& j, float (&acc)[RH]) {
    const int L = threadIdx.x & 31;
    const u32x4* xp = reinterpret_cast<const u32x4*>(j.x);
#pragma unroll
    for (int i = 0; i < RH; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = L + 32 * c;
      const u32x4 x0 = ld_act(xp + 4 * ch), x1 = ld_act(xp + 4 * ch + 1);
      const u32x4 x2 = ld_act(xp + 4 * ch + 2), x3 = ld_act(xp + 4 * ch + 3);
#pragma unroll
      for (int i = 0; i < RH; ++i) {
        const f32x2 s = e4m3x2_lo(sc[c][i]);
        acc[i] = block16(q[c][i][0], q[c][i][1], x0, x1, s[0], acc[i]);
        acc[i] = block16(q[c][i][2], q[c][i][3], x2, x3, s[1], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < RH; ++i) acc[i] = sum_lanes<32>(acc[i]) * j.g;
  }

  __device__ __forceinline__ int row(int i) const { return row0 + 2 * i + ((threadIdx.x & 63) >> 5); }
};

// Any K % 16 == 0: each wave owns one row of a 4-row item and walks it in
// 16-element blocks (8 code bytes, one scale byte).  Loads are issued in
// compute(); this path serves shapes outside the tuned ones.
struct GemvGenericItem {
  static constexpr int kRows = kWaves;
  int r;
  __device__ __forceinline__ void issue(const StreamJob& j, int item) {
    r = item * kRows + (threadIdx.x >> 6);
  }
  __device__ __forceinline__ float compute(const StreamJob& j) {
    const int lane = threadIdx.x & 63;
    const int rr = r < j.n ? r : j.n - 1;
    const int nb = j.k >> 4;
    const uint8_t* wrow = j.wq + (size_t)rr * (j.k >> 1);
    const uint8_t* srow = j.ws + (size_t)rr * nb;
    float acc = 0.0f;
    for (int b = lane; b < nb; b += kWave) {
      const unsigned* cw = reinterpret_cast<const unsigned*>(wrow + 8 * (size_t)b);
      const unsigned c0 = ld_stream(cw), c1 = ld_stream(cw + 1);
      const float s = e4m3x2_lo(ld_stream(srow + b))[0];
      const u32x4* xb = reinterpret_cast<const u32x4*>(j.x + 16 * (size_t)b);
      acc = block16(c0, c1, ld_act(xb), ld_act(xb + 1), s, acc);
    }
    return sum_lanes<64>(acc) * j.g;
  }
};

// ---------------------------------------------------------------------------
// M >= 2 items (MFMA)
// ---------------------------------------------------------------------------
// Lane (c = lane % 16, gq = lane / 16) streams, per 128-element window, the
// 16-byte code chunk [kwin/2 + 16gq, +16) of row n0 + 16*nt + c and the two
// scale bytes of its 32 elements.  Code dword t is the B operand of MFMA
// step t (K positions kwin + 32gq + 8t + j); X is read in the same order (a
// consistent permutation of K leaves the dot product unchanged).
template <int MT, int NT, int P, bool XPF>
struct MfmaItem {
  static_assert(P % 2 == 0, "ring depth must be even");
  static constexpr int kRows = 16 * NT;
  u32x4 q[P][NT];
  unsigned short sc[P][NT];
  f32x4 acc[MT][NT];
  const uint8_t* wrow[NT];
  const uint8_t* srow[NT];
  int n0, w0, nwin;

  __device__ __forceinline__ void load_window(int slot_win, u32x4 (&qq)[NT], unsigned short (&ss)[NT]) {
    const int gq = (threadIdx.x & 63) >> 4;
    const int kwin = slot_win * 128;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      qq[nt] = ld_stream(reinterpret_cast<const u32x4*>(wrow[nt] + (kwin >> 1)) + gq);
      ss[nt] = ld_stream(reinterpret_cast<const unsigned short*>(srow[nt] + (kwin >> 4)) + gq);
    }
  }

  // K must be a multiple of 128 here (whole windows); the wave's quarter of
  // the windows is [w0, w0 + nwin).
  __device__ __forceinline__ void issue(const StreamJob& j, int item) {
    const int lane = threadIdx.x & 63, c = lane & 15, w = threadIdx.x >> 6;
    n0 = item * kRows;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int n = n0 + 16 * nt + c;
      n = n < j.n ? n : j.n - 1;
      wrow[nt] = j.wq + (size_t)n * (size_t)(j.k >> 1);
      srow[nt] = j.ws + (size_t)n * (size_t)(j.k >> 4);
    }
    const int nw = j.k >> 7;
    w0 = (w * nw) / kWaves;
    nwin = ((w + 1) * nw) / kWaves - w0;
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (p < nwin) load_window(w0 + p, q[p], sc[p]);
  }

  __device__ __forceinline__ void load_x(const StreamJob& j, int M, int win, u32x4 (&xa)[MT][4]) {
    const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
    const int e0 = win * 128 + 32 * gq;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + c;
      const u32x4* xr = reinterpret_cast<const u32x4*>(j.x + (size_t)(m < M ? m : 0) * j.k + e0);
#pragma unroll
      for (int st = 0; st < 4; ++st) xa[mt][st] = m < M ? ld_act(xr + st) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  __device__ __forceinline__ void mma_window(const u32x4 (&qq)[NT], const unsigned short (&ss)[NT],
                                             const u32x4 (&xa)[MT][4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x2 s = e4m3x2_lo(ss[nt]);
        b[nt] = dequant8_bf16(qq[nt][st], st < 2 ? s[0] : s[1]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mt][st]), b[nt],
                                                                acc[mt][nt], 0, 0, 0);
    }
  }

  __device__ __forceinline__ void compute(const StreamJob& j, int M) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (XPF) {
      // activations double-buffered: window wi uses buffer wi & 1 (P even,
      // so the parity of wi is the parity of the ring slot p)
      u32x4 xa[2][MT][4];
      if (nwin > 0) load_x(j, M, w0, xa[0]);
      for (int base = 0; base < nwin; base += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int wi = base + p;
          if (wi < nwin) {
            if (wi + 1 < nwin) load_x(j, M, w0 + wi + 1, xa[(p + 1) & 1]);
            mma_window(q[p], sc[p], xa[p & 1]);
            if (wi + P < nwin) load_window(w0 + wi + P, q[p], sc[p]);
          }
        }
      }
    } else {
      u32x4 xa[MT][4];
      for (int base = 0; base < nwin; base += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int wi = base + p;
          if (wi < nwin) {
            load_x(j, M, w0 + wi, xa);
            mma_window(q[p], sc[p], xa);
            if (wi + P < nwin) load_window(w0 + wi + P, q[p], sc[p]);
          }
        }
      }
    }
  }
};

// M >= 2, K % 128 == 0: activations shared through LDS.  The four waves
// split the item's rows -- wave w owns the NT tiles of 16 rows n0 +
// 16*(NT*w + nt) + c -- and walk K together, one 256-element window at a
// time.  Lane (c, gq) holds elements 64*gq .. 64*gq + 63 of the window of
// its row: 32 contiguous code bytes (two 16-byte loads) and their 4 scale
// bytes.  The four lanes of a row so read its whole 128-byte line of codes
// in one window: a CU can keep only so many cache lines in flight, and
// half-used lines halved the rate.  MFMA step st (0..7) takes elements
// 64*gq + 8*st .. + 7 of every lane -- a fixed permutation of the window's
// K positions, which the activations follow, so the sum is still over all
// of K in a fixed order.
//
// Activations: every wave loads, P windows ahead, its share of the window's
// rows (load i of wave w: rows 8i + 2w and 8i + 2w + 1, lanes 32r .. 32r + 31
// reading the 512 bytes of one row) into registers with ordinary loads the
// compiler tracks -- so its waits are exact.  One window before use each
// wave writes them into an LDS double buffer; after a barrier all waves read
// the whole window from there: the activations cross the memory path once
// per workgroup instead of once per wave.  Rows past M, and the upper half
// of a last window when K % 256 == 128, load as zeros.  Only the first
// 8 * kXLoads rows are loaded: with XH the last M-tile is at most half used
// (M <= 16 MT - 8) and its upper eight rows are not loaded at all, and with
// five M-tiles M <= 68 < 72; MFMA rows past what was loaded read whatever
// the slot holds, and their results are never stored.
//
// LDS layout of a slot: activation row m at byte 512*m; its 16-byte piece
// q (elements 8q .. 8q+7 of the window) at position q ^ (m & 15), so that
// the 16 lanes reading rows 16*mt + c, piece q, hit 16 different bank
// groups (and the 32 lanes writing one row hit 32 different ones).
template <int MT, int NT, int P, int FMT = 0, int XH = 0>
struct MfmaLdsItem {
  static constexpr int kRows = 16 * NT * kWaves;
  static constexpr int kSlotBytes = 16 * MT * 512;
  static constexpr int kRing = 2;  // slots: the window being read, the next one being written
  // Five M-tiles hold at most 68 of their 80 rows.  Their two slots are
  // then M rows apart, not 80: only rows below M are written, and the MFMA
  // rows past M (whose results are never stored) read what follows -- the
  // other slot, or a tail that makes the ring VG_MAX_M_DEV + 80 rows.  That
  // keeps the ring at 75.8 KB (80.1 KB with the scale table below), so two
  // workgroups fit on a CU.
  static constexpr bool kCompact = 16 * MT > VG_MAX_M_DEV;
  static constexpr int kRingBytes = kCompact ? (VG_MAX_M_DEV + 16 * MT) * 512 : kRing * kSlotBytes;
  // NVFP4: a row's scales are loaded once per group of P windows (16P
  // contiguous bytes), 4P bytes per lane -- with P = 4 one window's four
  // quarters, with P = 2 half a window -- and passed between the row's four
  // lanes through a per-wave table (16 rows of 17 dwords: the odd stride
  // spreads the reads over the banks).  P times fewer scale requests; every
  // window sees the same bytes.
  static constexpr bool kGroupScales = FMT == 0 && (P == 4 || P == 2);
  using ScaleLoad = std::conditional_t<P == 4, u32x4, u32x2>;
  static constexpr int kScaleTable = 16 * 17;  // dwords per wave and 16-row tile
  static constexpr int kLdsBytes = kRingBytes + (kGroupScales ? kWaves * NT * kScaleTable * 4 : 0);
  // activation loads per lane per window (eight rows each, see above)
  static constexpr int kXLoads = MT == 5 ? (VG_MAX_M_DEV + 7) / 8 : 2 * MT - XH;
  static_assert(8 * kXLoads >= (MT == 5 ? VG_MAX_M_DEV : 16 * MT - 8 * XH), "every row below M is loaded");
  // A lane's 64 weights of a window: NVFP4 32 code bytes + 4 scale bytes;
  // FP8 (E4M3, scales per row in the epilogue) 64 bytes.
  static constexpr int kQ = FMT == 0 ? 2 : 4;        // 16-byte weight loads per lane per window
  static constexpr unsigned kLaneBytes = 16u * kQ;   // a lane's weight bytes per window
  u32x4 q[P][NT][kQ];
  unsigned sc[P][NT];     // per window: this lane's four scale bytes
  ScaleLoad sg[NT];      // grouped scales in flight: 4P bytes of this lane's row
  u32x4 xq[P][kXLoads];  // this wave's rows of the activation window, per ring position
  f32x4 acc[MT][NT];     // the running slice's sum; after compute(), the result (see fold)
  f32x4 tot[MT][NT];     // sum of the finished slices (whole-block items)
  __amdgpu_buffer_rsrc_t rw[NT], rs[NT], rx;
  unsigned cw, cs, ew;  // this lane's code / scale byte offset within its tile, element offset in a window
  int n0, k, nw, ns;    // first row, K, windows of K, K slices
  int v0, vend, cnt;    // the item's windows [v0, vend), cnt of them
  int mrows, slot_bytes;  // M; the distance between the two ring slots
  int fs, fold_at;      // whole-block items: the running slice and the window its sum ends after

  // Weights are loaded with the default cache policy: the scale bytes of
  // eight windows share a line, which the streaming policy would evict
  // before the next window reads it.
  __device__ __forceinline__ void load_w(int p, int v) {
    const bool in = v < vend && 256u * (unsigned)v + ew < (unsigned)k;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const unsigned o = cw + 4u * kLaneBytes * (unsigned)v;
#pragma unroll
      for (int t = 0; t < kQ; ++t)
        q[p][nt][t] = __builtin_amdgcn_raw_buffer_load_b128(rw[nt], in ? o + 16u * t : kOOB, 0, 0);
      if constexpr (kGroupScales) {
        if (p == 0) {  // the group starting at window v: bytes 4P*gq .. of its 16P
          const unsigned gq = (threadIdx.x & 63) >> 4;
          const bool gin = v + (int)(P * gq / 4) < vend;
          const unsigned off = gin ? cs - 4u * gq + 16u * (unsigned)v + 4u * P * gq : kOOB;
          if constexpr (P == 4)
            sg[nt] = __builtin_amdgcn_raw_buffer_load_b128(rs[nt], off, 0, 0);
          else
            sg[nt] = __builtin_amdgcn_raw_buffer_load_b64(rs[nt], off, 0, 0);
        }
      } else if constexpr (FMT == 0) {
        sc[p][nt] = __builtin_amdgcn_raw_buffer_load_b32(rs[nt], in ? cs + 16u * (unsigned)v : kOOB, 0, 0);
      }
    }
  }

  // Block `block` of job j: all of K (slice < 0; the slice sums are folded
  // into tot as they end) or K slice `slice` alone (its sum stays in acc).
  __device__ __forceinline__ void issue(const StreamJob& j, int block, int slice) {
    const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned rb = FMT == 0 ? (unsigned)j.k >> 1 : (unsigned)j.k, sb = (unsigned)j.k >> 4;
    n0 = block * kRows;
    k = j.k;
    nw = lds_windows(j.k);
    ns = lds_slices(j.k);
    if (slice < 0) {
      v0 = 0;
      vend = nw;
      fs = 0;
      fold_at = nw / ns;
    } else {
      v0 = slice * nw / ns;
      vend = (slice + 1) * nw / ns;
      fs = ns;
      fold_at = -1;  // never
    }
    cnt = vend - v0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int t0 = n0 + 16 * (NT * w + nt);
      const int rows = j.n - t0 < 0 ? 0 : (j.n - t0 > 16 ? 16 : j.n - t0);
      rw[nt] = rsrc_uniform(j.wq + (size_t)t0 * rb, (unsigned)rows * rb);
      if constexpr (FMT == 0) rs[nt] = rsrc_uniform(j.ws + (size_t)t0 * sb, (unsigned)rows * sb);
    }
    cw = (unsigned)c * rb + kLaneBytes * (unsigned)gq;
    cs = (unsigned)c * sb + 4u * (unsigned)gq;
    ew = 64u * (unsigned)gq;
#pragma unroll
    for (int p = 0; p < P; ++p) load_w(p, v0 + p);
  }

  // Row of this lane's activation load i (wave w's rows).
  __device__ __forceinline__ int xrow(int i) const {
    return 2 * (4 * i + (int)(threadIdx.x >> 6)) + ((threadIdx.x & 63) >> 5);
  }

  __device__ __forceinline__ void load_x(int p, int v) {
    const unsigned piece = threadIdx.x & 31;
    const unsigned e = 256u * (unsigned)v + 8u * piece;
    const bool in = v < vend && e < (unsigned)k;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const unsigned off = ((unsigned)xrow(i) * (unsigned)k + e) * 2u;
      xq[p][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? off : kOOB, 0, 0);
    }
  }

  // With the compact ring (slots M rows apart) a row m >= M of slot 0
  // would land on slot 1's rows: it goes to row M + m of the ring instead,
  // the tail past slot 1's rows, which only MFMA rows past M read.  (Slot
  // 1's own rows m >= M are that tail already.)  An address select, not a
  // branch: the rows of one write differ between the half-waves.
  __device__ __forceinline__ void store_x(int p, unsigned char* slot, unsigned char* ring) {
    const unsigned piece = threadIdx.x & 31;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int m = xrow(i);
      unsigned char* row = slot + 512 * m;
      if constexpr (kCompact) row = m < mrows ? row : ring + 512 * (mrows + m);
      *reinterpret_cast<u32x4*>(row + 16 * (piece ^ (unsigned)(m & 15))) = xq[p][i];
    }
  }

  // The activation fragments of MFMA step st+1 are read from LDS while
  // step st multiplies (two register sets): with the reads of a step issued
  // only after the previous step's MFMAs, every step waited one LDS round
  // trip, and with one wave per SIMD nothing else hid it.
  // Group start (window v, ring position 0): lane (c, gq) holds bytes
  // 4P*gq .. 4P*gq+4P-1 of row c's 16P scale bytes of windows v .. v+P-1;
  // after the exchange, sc[t] holds window v + t's bytes 4gq .. 4gq+3 --
  // zero where those elements lie past K (a half window's other half may
  // read the next row's scales).
  __device__ __forceinline__ void spread_scales(int v, unsigned* table) {
    const unsigned lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      unsigned* t0 = table + nt * kScaleTable + 17 * c;
#pragma unroll
      for (int d = 0; d < P; ++d) t0[P * gq + d] = sg[nt][d];
      // other lanes' writes are read next: the wave's LDS operations run in
      // order; the fence keeps the compiler from moving the reads up
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
#pragma unroll
      for (int t = 0; t < P; ++t) {
        const unsigned word = t0[4 * t + gq];
        sc[t][nt] = 256u * (unsigned)(v + t) + ew < (unsigned)k ? word : 0u;
      }
    }
  }

  __device__ __forceinline__ void window(int p, const unsigned char* slot) {
    const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
    f32x2 s[NT][2];
    if constexpr (FMT == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        s[nt][0] = e4m3x2_lo((unsigned short)(sc[p][nt] & 0xFFFFu));
        s[nt][1] = e4m3x2_lo((unsigned short)(sc[p][nt] >> 16));
      }
    }
    u32x4 a[2][MT];
    auto read = [&](int st, u32x4 (&dst)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        dst[mt] = *reinterpret_cast<const u32x4*>(slot + 512 * (16 * mt + c) + 16 * ((8 * gq + st) ^ c));
    };
    read(0, a[0]);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      // With three or more M-tiles the compiler otherwise sinks each read
      // next to its MFMA and waits for it there (measured: M = 68 2.8 %
      // faster pinned; with one or two M-tiles pinning costs registers and
      // is slower).
      if constexpr (MT >= 3) __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < 8) read(st + 1, a[(st + 1) & 1]);
      if constexpr (MT >= 3) __builtin_amdgcn_sched_barrier(0);
      bf16x8 b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (FMT == 0)
          b[nt] = dequant8_bf16(q[p][nt][st >> 2][st & 3], s[nt][st >> 2][(st >> 1) & 1]);
        else  // bytes 8st .. 8st+7 of the lane's 64: elements 64gq + 8st .. + 7, exact in bf16
          b[nt] = fp8x8_bf16(q[p][nt][st >> 1][2 * (st & 1)], q[p][nt][st >> 1][2 * (st & 1) + 1]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[st & 1][mt]), b[nt],
                                                                acc[mt][nt], 0, 0, 0);
    }
  }

  // After the stage wait: the activations of the first P windows, then
  // every window in order.  `lds` holds the ring (kRingBytes).
  __device__ __forceinline__ void compute(const StreamJob& j, int M, unsigned char* lds) {
    rx = rsrc_uniform(j.x, (unsigned)M * (unsigned)j.k * 2u);
    mrows = M;
    slot_bytes = kCompact ? 512 * M : kSlotBytes;
#pragma unroll
    for (int p = 0; p < P; ++p) load_x(p, v0 + p);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        tot[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    store_x(0, lds, lds);
    // The loop over whole groups of P windows must be entered in the order
    // its own iterations leave the loads in, and contain no skipped load:
    // a loop header reached with another order (the first P windows' loads
    // went out as all weights before the stage wait, then all activations)
    // or with fewer loads gets the compiler's most conservative wait -- all
    // loads -- in every iteration.  So the first group is peeled off and
    // every group is whole: steps past the item's last window still issue
    // their (out-of-range, zero-traffic) loads and skip only the compute.
    const int groups = (cnt + P - 1) / P;
#pragma unroll
    for (int p = 0; p < P; ++p) step(p, p, lds);
    for (int g = 1; g < groups; ++g) {
#pragma unroll
      for (int p = 0; p < P; ++p) step(p, g * P + p, lds);
    }
    if (fold_at >= 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = tot[mt][nt];
    }
  }

  // A slice ended (whole-block items): tot += its sum, in slice order from
  // +0.0 -- the order in which a spread block's partials are added.
  __device__ __forceinline__ void fold() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[mt][nt][r] = tot[mt][nt][r] + acc[mt][nt][r];
        acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    ++fs;
    fold_at = (fs + 1) * nw / ns;
  }

  // The item's window i (window v0 + i of K; ring position p = i % P):
  // compute it, pass the next window's activations to LDS, and load window
  // v0 + i + P into position p.
  __device__ __forceinline__ void step(int p, int i, unsigned char* lds) {
    __syncthreads();  // window i is in LDS; every wave is done with window i-1
    if constexpr (kGroupScales)
      if (p == 0) spread_scales(v0 + i, reinterpret_cast<unsigned*>(lds + kRingBytes) +
                                            (threadIdx.x >> 6) * NT * kScaleTable);
    if (i < cnt) {    // wave-uniform; nothing in here loads from memory
      window(p, lds + (i & 1) * slot_bytes);
      if (v0 + i + 1 == fold_at) fold();
    }
    store_x(p + 1 < P ? p + 1 : 0, lds + ((i + 1) & 1) * slot_bytes, lds);
    load_x(p, v0 + i + P);
    load_w(p, v0 + i + P);
  }
};

// Any K % 16 == 0, predicated everywhere: each wave takes a quarter of the
// (possibly partial) 128-element windows.
template <int MT, int NT>
struct MfmaGuardedItem {
  static constexpr int kRows = 16 * NT;
  f32x4 acc[MT][NT];
  int n0;
  __device__ __forceinline__ void issue(const StreamJob&, int item) { n0 = item * kRows; }
  __device__ __forceinline__ void compute(const StreamJob& j, int M) {
    const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4, w = threadIdx.x >> 6;
    const uint8_t* wrow[NT];
    const uint8_t* srow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int n = n0 + 16 * nt + c;
      n = n < j.n ? n : j.n - 1;
      wrow[nt] = j.wq + (size_t)n * (size_t)(j.k >> 1);
      srow[nt] = j.ws + (size_t)n * (size_t)(j.k >> 4);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nw = (j.k + 127) >> 7;
    const int wb = (w * nw) / kWaves, we = ((w + 1) * nw) / kWaves;
    for (int win = wb; win < we; ++win) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int e0 = win * 128 + 32 * gq + 8 * st;
        const bool ok = e0 < j.k;  // K % 16 == 0: an 8-element piece is all in or all out
        bf16x8 b[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          unsigned wd = 0;
          float s = 0.0f;
          if (ok) {
            wd = ld_stream(reinterpret_cast<const unsigned*>(wrow[nt] + (e0 >> 1)));
            s = e4m3x2_lo(ld_stream(srow[nt] + (e0 >> 4)))[0];
          }
          b[nt] = dequant8_bf16(wd, s);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + c;
          u32x4 a = {0u, 0u, 0u, 0u};
          if (ok && m < M) a = ld_act(reinterpret_cast<const u32x4*>(j.x + (size_t)m * j.k + e0));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b[nt],
                                                                  acc[mt][nt], 0, 0, 0);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// FP8 (E4M3) weights: one byte per element, W8[N][K]; g and the per-row
// scales multiply a row's sum.  E4M3 converts to bf16 exactly, so the
// arithmetic is that of the NVFP4 items: v_dot2 at M = 1, bf16 MFMA at
// M >= 2.  Any K % 16 == 0 (a 16-byte piece is 16 elements, a multiple of
// the 8 the MFMA steps take, so a piece is all in or all out of K).
// ---------------------------------------------------------------------------
// M = 1: each wave owns one row of a 4-row item; lane L takes the 16-byte
// pieces L, L+64, ... of the row (1 KB per wave instruction), four pieces
// in flight.
struct Fp8GemvItem {
  static constexpr int kRows = kWaves;
  int r;
  __device__ __forceinline__ void issue(const StreamJob& j, int item) {
    r = item * kRows + (threadIdx.x >> 6);
  }
  __device__ __forceinline__ float compute(const StreamJob& j) {
    const int lane = threadIdx.x & 63;
    const int rr = r < j.n ? r : j.n - 1;
    const int np = j.k >> 4;
    const u32x4* wrow = reinterpret_cast<const u32x4*>(j.wq + (size_t)rr * j.k);
    const u32x4* xp = reinterpret_cast<const u32x4*>(j.x);
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll 4
    for (int p = lane; p < np; p += kWave) {
      const u32x4 w = ld_stream(wrow + p);
      a0 = fp8_dot8(w[0], w[1], ld_act(xp + 2 * p), a0);
      a1 = fp8_dot8(w[2], w[3], ld_act(xp + 2 * p + 1), a1);
    }
    return sum_lanes<64>(a0 + a1) * j.g;
  }
};

// M >= 2: as MfmaGuardedItem -- the four waves split the 128-element
// windows, lane (c, gq) holds K positions win*128 + 32*gq + 8*st + 0..7 of
// row n0 + 16*nt + c (weights) and of activation row 16*mt + c.
template <int MT, int NT>
struct Fp8MfmaItem {
  static constexpr int kRows = 16 * NT;
  f32x4 acc[MT][NT];
  int n0;
  __device__ __forceinline__ void issue(const StreamJob&, int item) { n0 = item * kRows; }
  __device__ __forceinline__ void compute(const StreamJob& j, int M) {
    const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4, w = threadIdx.x >> 6;
    const uint8_t* wrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      int n = n0 + 16 * nt + c;
      n = n < j.n ? n : j.n - 1;
      wrow[nt] = j.wq + (size_t)n * (size_t)j.k;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nw = (j.k + 127) >> 7;
    const int wb = (w * nw) / kWaves, we = ((w + 1) * nw) / kWaves;
    for (int win = wb; win < we; ++win) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int e0 = win * 128 + 32 * gq + 8 * st;
        const bool ok = e0 < j.k;
        bf16x8 b[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          unsigned w0 = 0, w1 = 0;
          if (ok) {
            const unsigned* p = reinterpret_cast<const unsigned*>(wrow[nt] + e0);
            w0 = ld_stream(p);
            w1 = ld_stream(p + 1);
          }
          b[nt] = fp8x8_bf16(w0, w1);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + c;
          u32x4 a = {0u, 0u, 0u, 0u};
          if (ok && m < M) a = ld_act(reinterpret_cast<const u32x4*>(j.x + (size_t)m * j.k + e0));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b[nt],
                                                                  acc[mt][nt], 0, 0, 0);
        }
      }
    }
  }
};

// The four waves' partial tiles meet in LDS and are added in wave order
// 0+1+2+3 by wave 0, which then owns the finished tile (times g).
template <int MT, int NT>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[MT][NT], float* red, float g) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int kVals = MT * NT * 4;
  __syncthreads();  // red may still be read by the previous item's wave 0
  if (w > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[((w - 1) * kVals + (mt * NT + nt) * 4 + r) * kWave + lane] = acc[mt][nt][r];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = acc[mt][nt][r];
#pragma unroll
          for (int ow = 0; ow < kWaves - 1; ++ow) v += red[(ow * kVals + (mt * NT + nt) * 4 + r) * kWave + lane];
          acc[mt][nt][r] = v * g;
        }
  }
}

// ---------------------------------------------------------------------------
// per-workgroup running best for the lm_head
// ---------------------------------------------------------------------------
template <int R>
struct Best {
  float v[R];
  int i[R];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int r = 0; r < R; ++r) { v[r] = -__builtin_inff(); i[r] = -1; }
  }
  __device__ __forceinline__ void offer(int r, float val, int idx) {
    if (i[r] < 0 || better(val, idx, v[r], i[r])) { v[r] = val; i[r] = idx; }
  }
  __device__ __forceinline__ void begin_item() {}
  __device__ __forceinline__ void end_item() {}
};

// Items of GEMM jobs keep no running best.
struct NoBest {
  __device__ __forceinline__ void offer(int, float, int) {}
  __device__ __forceinline__ void begin_item() {}
  __device__ __forceinline__ void end_item() {}
};

// The lm_head's running best with M-tiles: kept in LDS, one key per row m
// per wave, so nothing of it is live in registers across an item's window
// loop.  An item's candidates (lane (c, gq) offers rows m = 16*mt + 4*gq + r
// for its columns) collect in registers during the item's epilogue only;
// end_item() reduces them over the 16 lanes that share each m (largest
// logit, then lowest index: the larger packed key) and folds them into the
// wave's table.
template <int MT>
struct WaveBest {
  static constexpr int R = MT * 4;
  unsigned long long* tab;  // this wave's 16 * MT keys (LDS); 0 = no candidate yet
  float v[R];
  int i[R];
  __device__ __forceinline__ void init() {
    for (int m = threadIdx.x & 63; m < 16 * MT; m += kWave) tab[m] = 0ull;  // 80 rows at MT = 5
  }
  __device__ __forceinline__ void begin_item() {
#pragma unroll
    for (int r = 0; r < R; ++r) { v[r] = -__builtin_inff(); i[r] = -1; }
  }
  __device__ __forceinline__ void offer(int r, float val, int idx) {
    if (i[r] < 0 || better(val, idx, v[r], i[r])) { v[r] = val; i[r] = idx; }
  }
  __device__ __forceinline__ void end_item() {
    const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        unsigned long long k = i[mt * 4 + r] >= 0 ? argmax_key(v[mt * 4 + r], (unsigned)i[mt * 4 + r]) : 0ull;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) {
          const unsigned long long o = __shfl_xor(k, off, kWave);
          k = o > k ? o : k;
        }
        const int m = 16 * mt + 4 * gq + r;
        if (c == 0 && k > tab[m]) tab[m] = k;
      }
  }
};

__device__ __forceinline__ void publish_best(StreamCtl* ctl, int m, float v, int idx) {
  if (idx < 0) return;
  const int slot = blockIdx.x % kKeySlots;
  __hip_atomic_fetch_max(&ctl->keys[m][slot], argmax_key(v, (unsigned)idx), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// MODE_DIRECT: grid = items of one job, no control block (GEMM calls).
// MODE_GRID:   one job, each workgroup walks items blockIdx.x + i*gridDim.x
//              (the standalone lm_head pass).
// MODE_STATIC: the job list of a whole step, items dealt round-robin to
//              resident workgroups, with stage waits (the step kernel).
constexpr int MODE_DIRECT = STREAM_DIRECT, MODE_GRID = STREAM_GRID, MODE_STATIC = STREAM_STATIC;

template <int MT>
struct Cfg;  // MT = 0: the M = 1 GEMV path
template <>
struct Cfg<0> {
  static constexpr int NT = 0;
};
template <int MT>
struct Cfg {
  static constexpr int NT = MT <= 2 ? 2 : 4;   // weight rows per item: 32 or 64
  static constexpr int P = MT <= 2 ? 6 : 2;    // 128-element windows in flight per wave (even)
  static constexpr bool XPF = MT <= 2;         // prefetch the next window's activations
  // the LDS-shared item (K % 128 == 0): 16-row tiles per wave, window ring depth
  static constexpr int LNT = 1;
  static constexpr int LP = MT <= 2 ? 4 : 2;
  template <int FMT, int XH>
  using Item = MfmaLdsItem<MT, LNT, LP, FMT, XH>;  // FMT 1: FP8 weights, the same item otherwise
  using Lds = Item<0, 0>;
};

// Processes one item of job j.  `dep` is called by every thread after the
// weight loads are in flight and before any activation is read; it returns
// false if the stage wait failed (then nothing is stored).
template <int CPL, int RH, class Dep, class BestT>
__device__ __forceinline__ void gemv_run(const StreamJob& j, int item, Dep&& dep, BestT& best) {
  GemvItem<CPL, RH> it;
  it.issue(j, item);
  float rsc[RH];
#pragma unroll
  for (int i = 0; i < RH; ++i) rsc[i] = row_scale(j, it.row(i));
  const bool ok = dep();
  float acc[RH];
  it.compute(j, acc);
  if (!ok) return;
  if (j.kind == 0) {
    if ((threadIdx.x & 31) == 0) {
#pragma unroll
      for (int i = 0; i < RH; ++i) {
        const int r = it.row(i);
        if (r < j.n) store_out(&j.y[r], acc[i] * rsc[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < RH; ++i) {
      const int r = it.row(i);
      if (r < j.n) best.offer(0, acc[i] * rsc[i], r);
    }
  }
}

// One row per wave (GemvGenericItem: NVFP4, any K; Fp8GemvItem: FP8).
template <class Item, class Dep, class BestT>
__device__ __forceinline__ void gemv_generic_run(const StreamJob& j, int item, Dep&& dep, BestT& best) {
  Item it;
  it.issue(j, item);
  const float rsc = row_scale(j, it.r);
  const bool ok = dep();
  const float v = it.compute(j);
  if (!ok || it.r >= j.n) return;
  if (j.kind == 0) {
    if ((threadIdx.x & 63) == 0) store_out(&j.y[it.r], v * rsc);
  } else {
    best.offer(0, v * rsc, it.r);
  }
}

template <int MT, int NT, class Item, class Dep, class BestT>
__device__ __forceinline__ void mfma_run(Item& it, const StreamJob& j, int item, int M, Dep&& dep,
                                         float* red, BestT& best) {
  it.issue(j, item);
  float rsc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) rsc[nt] = row_scale(j, it.n0 + 16 * nt + (threadIdx.x & 15));
  const bool ok = dep();
  it.compute(j, M);
  reduce_waves<MT, NT>(it.acc, red, j.g);
  if (!ok || (threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  best.begin_item();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * gq + r;
      if (m < M) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int n = it.n0 + 16 * nt + c;
          if (n < j.n) {
            if (j.kind == 0) store_out(&j.y[(size_t)m * j.n + n], it.acc[mt][nt][r] * rsc[nt]);
            else best.offer(mt * 4 + r, it.acc[mt][nt][r] * rsc[nt], n);
          }
        }
      }
    }
  best.end_item();
}

// Where a spread job's slice sums meet (STATIC launches; null elsewhere).
struct SpreadCtx {
  float* part;
  unsigned* cnt;
  int* flag;  // an LDS word
};

__device__ __forceinline__ float ld_agent_f(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The LDS-shared MFMA item: each wave finishes its own rows (no reduction
// across waves).  A whole-block item stores (or offers) its rows.  A slice
// of a spread job stores its slice sum to its partial slot and counts
// itself in; the workgroup that completes the block adds the slice sums
// from +0.0 in slice order -- as a whole-block item folds them -- and
// finishes the rows, then clears the count for the next launch.
template <int MT, int FMT, int XH, class Dep, class BestT>
__device__ __forceinline__ void mfma_lds_run(const StreamJob& j, int item, int M, Dep&& dep, unsigned char* xring,
                                             const SpreadCtx& sp, BestT& best) {
  using Item = typename Cfg<MT>::template Item<FMT, XH>;
  constexpr int NT = Cfg<MT>::LNT, R = Item::kRows;
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4, w = threadIdx.x >> 6;
  const int S = lds_slices(j.k), first = j.spread - 1;
  const bool sliced = j.spread && item >= first;
  const int t = item - first;  // this slice item's number within the job's slice items
  const int block = sliced ? first + t / S : item, slice = sliced ? t - (t / S) * S : -1;
  Item it;
  it.issue(j, block, slice);
  float rsc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) rsc[nt] = row_scale(j, it.n0 + 16 * (NT * w + nt) + c);
  const bool ok = dep();
  it.compute(j, M, xring);
  if (sliced) {
    float* mine = sp.part + (size_t)(j.part_base + t) * (size_t)M * R;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * gq + r;
        if (m < M)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) store_out(&mine[m * R + 16 * (NT * w + nt) + c], it.acc[mt][nt][r]);
      }
    // The slice sums are agent-coherent stores and the count is taken once
    // they have completed (vmcnt(0)), as a stage is signalled; the
    // completing workgroup reads them with agent-coherent loads.  No cache
    // write-back or invalidation is needed -- a fence here costs every
    // slice item an L2 write-back.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const int slot0 = j.part_base + (block - first) * S;  // the block's slice 0
    unsigned* count = &sp.cnt[slot0];
    if (threadIdx.x == 0)
      *sp.flag = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(S - 1);
    __syncthreads();
    const bool last = *sp.flag != 0;
    __syncthreads();
    if (!last) return;
    const float* p0 = sp.part + (size_t)slot0 * (size_t)M * R;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mt + 4 * gq + r;
        if (m < M)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int col = 16 * (NT * w + nt) + c;
            float sum = 0.0f;
            for (int q = 0; q < S; ++q)
              sum = sum + (q == slice ? it.acc[mt][nt][r] : ld_agent_f(&p0[((size_t)q * M + m) * R + col]));
            it.acc[mt][nt][r] = sum;
          }
      }
    if (threadIdx.x == 0) st_agent(count, 0u);
  }
  if (!ok) return;
  best.begin_item();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * gq + r;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = it.n0 + 16 * (NT * w + nt) + c;
        if (m < M && n < j.n) {
          const float v = it.acc[mt][nt][r] * j.g * rsc[nt];
          if (j.kind == 0) store_out(&j.y[(size_t)m * j.n + n], v);
          else best.offer(mt * 4 + r, v, n);
        }
      }
    }
  best.end_item();
}

// One item of job j, whose weight format is FMT (a launch holds one format:
// each kernel carries only its own items, so one format's registers do not
// crowd the other's).  ANYK = 0: every K of the launch is a multiple of 128,
// so the kernel carries only the LDS-shared item (the K-split guarded items
// are the register-heaviest code of the kernel).
template <int MT, int FMT, int ANYK, int XH, class Dep, class BestT>
__device__ __forceinline__ void run_item(const StreamJob& j, int item, int M, Dep&& dep, float* red,
                                         unsigned char* xring, const SpreadCtx& sp, BestT& best) {
  if constexpr (MT == 0) {
    if constexpr (FMT == 1) {
      gemv_generic_run<Fp8GemvItem>(j, item, dep, best);
    } else {
      if (j.k == 5120) gemv_run<5, 4>(j, item, dep, best);
      else if (j.k == 17408) gemv_run<17, 1>(j, item, dep, best);
      else if (j.k == 1024) gemv_run<1, 8>(j, item, dep, best);
      else gemv_generic_run<GemvGenericItem>(j, item, dep, best);
    }
  } else {
    constexpr int NT = Cfg<MT>::NT;
    if (!ANYK || (j.k & 127) == 0) {
      mfma_lds_run<MT, FMT, XH>(j, item, M, dep, xring, sp, best);
    } else if constexpr (!ANYK) {
    } else if constexpr (FMT == 1) {
      Fp8MfmaItem<MT, NT> it;
      mfma_run<MT, NT>(it, j, item, M, dep, red, best);
    } else {
      MfmaGuardedItem<MT, NT> it;
      mfma_run<MT, NT>(it, j, item, M, dep, red, best);
    }
  }
}

// Publish the workgroup's lm_head bests (M = 1: every wave's best; M >= 2:
// per row, the best of the four waves' tables, which hold each wave's
// per-lane bests reduced over the 16 lanes sharing rows -- rows that no
// wave holds publish nothing).  Every thread calls it (M >= 2: a barrier).
template <int MT, class BestT>
__device__ __forceinline__ void publish(StreamCtl* ctl, int M, BestT& best) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if constexpr (MT == 0) {
    float v = best.v[0];
    int i = best.i[0];
    const float ov = __shfl_xor(v, 32, kWave);
    const int oi = __shfl_xor(i, 32, kWave);
    if (oi >= 0 && (i < 0 || better(ov, oi, v, i))) { v = ov; i = oi; }
    if (lane == 0) publish_best(ctl, 0, v, i);
  } else {
    // the waves' tables (one key per row m, 0: the wave saw none) reduced
    // by wave 0, one atomic per row and workgroup (the four waves' atomics
    // on the same lines took 72 against 77 us for a 65,536-row head at
    // M = 17); more rows than lanes at MT = 5
    __syncthreads();
    if (w == 0)
      for (int m = lane; m < 16 * MT && m < M; m += kWave) {
        unsigned long long k = 0;
        for (int v = 0; v < kWaves; ++v) {
          const unsigned long long t = best.tab[v * 16 * MT + m];
          k = t > k ? t : k;
        }
        if (k != 0ull)
          __hip_atomic_fetch_max(&ctl->keys[m][blockIdx.x % kKeySlots], k, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
  }
}

// One stage signal from this workgroup.  Outputs are stored with
// agent-coherent (write-through) stores; each wave first waits until its
// own stores have completed (vmcnt(0) -- a workgroup-scope fence does not
// wait for global stores), so after the barrier every output of the stage
// is visible at agent scope before the counter moves.  No L2 write-back is
// needed.  Called by the whole workgroup at a point where no weight loads
// are in flight.
__device__ void signal_stage(const StreamArgs& a, int s) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(&a.stage_done[s][blockIdx.x % kDoneSlots].v, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// The last workgroup out: argmax from the key slots (reported as token ids
// through the head's row map when there is one), the accept rule, reset.
//
// Accept (TandemLLM README, flow diagram and "The parts": the drafters'
// guesses form a tree and the target keeps the longest path it agrees
// with): node 0 of a sequence is the committed position; node i >= 1 holds
// drafts[i-1] below parent parents[i-1], or below i-1 when there is no
// parent array (a chain).  Node i is agreed iff its parent p lies in
// [0, i), p is agreed and drafts[i-1] equals the argmax of row p.  Parents
// precede their children, so one pass in node order settles every node.
// The deepest agreed node (lowest index among equals) gives accept_len
// (its depth) and accept_node; for a chain that is the longest agreeing
// prefix.  Parents outside [0, i) are never followed.
__device__ void finish_lmhead(StreamCtl* ctl, const StreamArgs& a, int* lds_am, int* lds_dep) {
  const int tid = threadIdx.x;
  if (a.has_lmhead) {
    for (int m = tid; m < a.M; m += kWG) {
      unsigned long long best = 0;
      for (int s = 0; s < kKeySlots; ++s) {
        const unsigned long long k =
            __hip_atomic_load(&ctl->keys[m][s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        best = k > best ? k : best;
        __hip_atomic_store(&ctl->keys[m][s], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const int row = (int)key_index(best);
      const int am = a.token_map && row >= 0 && row < a.lm_rows ? a.token_map[row] : row;
      lds_am[m] = am;
      a.argmax[m] = am;
    }
    __syncthreads();
    const int S = a.M / a.T;
    for (int q = tid; q < S; q += kWG) {
      const int32_t* d = a.drafts + (size_t)q * (a.T - 1);
      const int32_t* par = a.parents ? a.parents + (size_t)q * (a.T - 1) : nullptr;
      const int* am = lds_am + q * a.T;
      int* dep = lds_dep + q * a.T;  // depth of an agreed node, -1 otherwise
      dep[0] = 0;
      int best_d = 0, best_n = 0;
      for (int i = 1; i < a.T; ++i) {
        const int p = par ? par[i - 1] : i - 1;
        const bool ok = p >= 0 && p < i && dep[p] >= 0 && d[i - 1] == am[p];
        dep[i] = ok ? dep[p] + 1 : -1;
        if (ok && dep[i] > best_d) {
          best_d = dep[i];
          best_n = i;
        }
      }
      a.accept_len[q] = best_d;
      if (a.accept_node) a.accept_node[q] = best_n;
    }
  }
  if (a.waits)
    for (int s = tid; s < a.nstages * kDoneSlots; s += kWG)
      st_agent(&a.stage_done[s / kDoneSlots][s % kDoneSlots].v, 0u);
  if (tid == 0) st_agent(&ctl->exits, 0u);
}

template <int MT, int MODE, int FMT, int ANYK, int XH>
// Two M-tiles: registers capped for two waves per SIMD, so the step can
// keep two workgroups per CU (measured: the M = 17 step 4 % faster; one
// M-tile and three or four gain nothing or lose).  Five M-tiles, one
// launch per GEMM: the compact ring lets two workgroups share a CU, and
// the cap makes their registers fit (M = 68 per-job step 6 % faster).  One
// M-tile, NVFP4, one launch per GEMM: capped at four waves per SIMD, which
// the grouped scales had just pushed it past (M = 4 per-job step 1 % faster;
// the FP8 kernel would spill).
__global__ __launch_bounds__(kWG)
__attribute__((amdgpu_waves_per_eu(MT == 1 && MODE == MODE_DIRECT && FMT == 0 ? 4
                                   : MT == 2 || (MT == 5 && MODE == MODE_DIRECT) ? 2
                                                                                  : 1))) void stream_kernel(
    StreamArgs a) {
  constexpr int NT = MT == 0 ? 1 : Cfg<MT>::NT;
  constexpr int kRed = MT == 0 ? 1 : (kWaves - 1) * MT * NT * 4 * kWave;
  __shared__ float red[kRed];
  constexpr int kXRing = MT == 0 ? 16 : Cfg<(MT > 0 ? MT : 1)>::Lds::kLdsBytes;
  __shared__ __attribute__((aligned(16))) unsigned char xring[kXRing];
  __shared__ int lds_flag;
  __shared__ int lds_am[VG_MAX_M_DEV];
  __shared__ int lds_dep[VG_MAX_M_DEV];
  __shared__ unsigned long long lds_best[kWaves][MT == 0 ? 1 : 16 * MT];  // lm_head keys per wave and row
  if constexpr (MODE == MODE_DIRECT) {
    auto nodep = [] { return true; };
    const SpreadCtx dsp{a.part, a.part_cnt, &lds_flag};
    NoBest nobest;
    if constexpr (MT > 0) {
      if (a.jobs) {
        // the GEMM jobs of one stage of a step (no dependencies among them)
        // in one launch: the grid covers their items in list order
        const int t = a.jobs[0].item_begin + (int)blockIdx.x;
        int q = 0;
        while (q + 1 < a.njobs && a.jobs[q + 1].item_begin <= t) ++q;
        const StreamJob j = a.jobs[q];
        run_item<MT, FMT, ANYK, XH>(j, t - j.item_begin, a.M, nodep, red, xring, dsp, nobest);
        return;
      }
    }
    run_item<MT, FMT, ANYK, XH>(a.job0, blockIdx.x, a.M, nodep, red, xring, dsp, nobest);
    return;
  } else {
    StreamCtl* ctl = a.ctl;
    const int G = gridDim.x;
    const SpreadCtx sp{a.part, a.part_cnt, &lds_flag};
    int cur = 0;          // job cursor (items only grow)
    int done_stage = -1;  // highest stage known complete
    int my_stage = -1;    // stage of the items this workgroup is working on
    // Items of the GEMM jobs, then those of the lm_head (the last job of a
    // step, every job of a GRID launch): the lm_head's running best is live
    // only in the second loop, not across the whole step.
    const int lm_begin = MODE == MODE_GRID ? 0 : (a.has_lmhead ? a.jobs[a.njobs - 1].item_begin : a.total_items);
    int t = blockIdx.x;
    auto body = [&](int ti, auto& best) {
      const StreamJob* jp;
      if constexpr (MODE == MODE_GRID) {
        jp = &a.job0;
      } else {
        while (cur + 1 < a.njobs && a.jobs[cur + 1].item_begin <= ti) ++cur;
        jp = &a.jobs[cur];
      }
      const StreamJob j = *jp;
      const int item = ti - j.item_begin;
      if constexpr (MODE == MODE_STATIC) {
        if (j.stage != my_stage) {
          // leaving a stage: one signal for all of this workgroup's items in it
          if (my_stage >= 0) signal_stage(a, my_stage);
          my_stage = j.stage;
        }
      }
      // the stage dependency: every workgroup holding items of stage s-1 is done
      auto dep = [&]() -> bool {
        if constexpr (MODE == MODE_STATIC) {
          const int need = j.stage - 1;
          if (need > done_stage) {
            if (threadIdx.x == 0) lds_flag = wait_stage(a.stage_done, ctl, need, a.stage_total[need]) ? 1 : 0;
            __syncthreads();
            const bool ok = lds_flag != 0;
            __syncthreads();
            if (!ok) return false;
            done_stage = need;
          }
        }
        return true;
      };
      run_item<MT, FMT, ANYK, XH>(j, item, a.M, dep, red, xring, sp, best);
      // LDS reuse by the next item (M >= 2: its activation copies go into
      // ring slots the slowest wave may still be reading)
      if constexpr (MODE == MODE_STATIC || MT > 0) __syncthreads();
    };
    {
      NoBest nobest;
      for (; t < lm_begin; t += G) body(t, nobest);
    }
    using BestT = std::conditional_t<MT == 0, Best<1>, WaveBest<MT == 0 ? 1 : MT>>;
    BestT best;
    if constexpr (MT > 0) best.tab = &lds_best[threadIdx.x >> 6][0];
    best.init();
    for (; t < a.total_items; t += G) body(t, best);
    if constexpr (MODE == MODE_STATIC) {
      if (my_stage >= 0) signal_stage(a, my_stage);
    }
    if (a.has_lmhead) publish<MT>(ctl, a.M, best);
    // Counting out without cache fences, as the stage signals do: every
    // wave waits until its own memory operations (stores, signals, key
    // atomics) are acknowledged before the workgroup's exit count, and the
    // last workgroup out reads the keys with agent-scope loads.  (Agent-
    // scope fences here, one per workgroup, made the 248,320-row lm_head
    // verify at M = 17 take 297 instead of 240 us.)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned prev = __hip_atomic_fetch_add(&ctl->exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_flag = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!lds_flag) return;
    finish_lmhead(ctl, a, lds_am, lds_dep);
  }
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

template <int MT, int MODE, int FMT = 0, int ANYK = 1, int XH = 0>
int resident_blocks() {
  static int per_cu = 0;
  if (!per_cu) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, stream_kernel<MT, MODE, FMT, ANYK, XH>, kWG, 0) != hipSuccess ||
        n < 1)
      n = 1;
    per_cu = n;
  }
  return per_cu * num_cus();
}

// XH: the last M-tile is at most half used, so the direct and lm_head
// kernels without guarded items load eight activation rows fewer per window
// (measured: the M = 17 step 3 % faster).  The persistent kernels keep one
// form per M-tile class, and so does the one-tile lm_head: its XH form
// needs fewer registers, runs three workgroups per CU instead of two and
// measured 22 % slower (318 against 261 us at M = 4).
template <int MT, int FMT, int ANYK, int XH>
hipError_t launch_fmt_xh(const StreamArgs& a, int mode, int grid, hipStream_t stream) {
  switch (mode) {
    case MODE_DIRECT:
      hipLaunchKernelGGL((stream_kernel<MT, MODE_DIRECT, FMT, ANYK, XH>), dim3(grid), dim3(kWG), 0, stream, a);
      break;
    case MODE_GRID: {
      const int cap = resident_blocks<MT, MODE_GRID, FMT, ANYK, XH>();
      hipLaunchKernelGGL((stream_kernel<MT, MODE_GRID, FMT, ANYK, XH>), dim3(grid < cap ? grid : cap), dim3(kWG), 0,
                         stream, a);
      break;
    }
    default:
      // exactly stream_static_grid(M) workgroups: the stage targets count them
      hipLaunchKernelGGL((stream_kernel<MT, MODE_STATIC, FMT, ANYK, 0>), dim3(grid), dim3(kWG), 0, stream, a);
      break;
  }
  return hipGetLastError();
}
template <int MT, int FMT, int ANYK>
hipError_t launch_fmt(const StreamArgs& a, int mode, int grid, hipStream_t stream) {
  if constexpr (MT >= 1 && MT <= 4 && ANYK == 0)
    if ((mode == MODE_DIRECT || (mode == MODE_GRID && MT >= 2)) && a.M <= 16 * MT - 8)
      return launch_fmt_xh<MT, FMT, ANYK, 1>(a, mode, grid, stream);
  return launch_fmt_xh<MT, FMT, ANYK, 0>(a, mode, grid, stream);
}

// The weight format of a launch is that of its (first) job: a step's jobs
// are all NVFP4; FP8 comes only as single-job launches.  A launch whose
// every K is a multiple of 128 takes the kernel without the guarded items
// (the GEMV kernels of MT = 0 have no such split).
template <int MT, int FMT>
hipError_t launch_mt_fmt(const StreamArgs& a, int mode, int grid, hipStream_t stream) {
  const bool any_k = MT == 0 || (a.jobs ? a.any_k != 0 : (a.job0.k & 127) != 0);
  return any_k ? launch_fmt<MT, FMT, 1>(a, mode, grid, stream) : launch_fmt<MT, FMT, 0>(a, mode, grid, stream);
}

}  // namespace

// The launcher of one M-tile class and weight format, and the resident
// workgroups of its static (persistent-step) kernel.  Each pair is
// explicitly instantiated in a translation unit of its own
// (stream_mt<MT>_f<FMT>.hip), so the kernel variants compile in parallel.
template <int MT, int FMT>
hipError_t launch_stream_mt(const StreamArgs& a, int mode, int grid, hipStream_t stream) {
  return launch_mt_fmt<MT, FMT>(a, mode, grid, stream);
}
template <int MT, int FMT>
int stream_static_resident() {
  return resident_blocks<MT, MODE_STATIC, FMT>();
}

}  // namespace vg

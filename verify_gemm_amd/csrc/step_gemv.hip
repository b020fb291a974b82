// M = 1 (plain decode): the weight stream of a whole step -- or of one GEMM,
// or of the lm_head pass -- as one launch of one resident workgroup per CU.
//
// A decode step reads every weight once and is bound by memory bandwidth
// (ling-engine README, opening paragraph and "Six levers"; veloGB10 docs,
// "Engineered to the roofline").  On gfx950 what decides whether a CU keeps
// its share of HBM bandwidth is how many weight bytes it has in flight at
// every moment, and the hardware counts a wave's outstanding vector-memory
// operations with ONE in-order counter (vmcnt) that loads and stores share.
// A wave that waits for an activation load, or that has a store pending
// when it waits for a weight load, ends up waiting for everything it issued
// before -- including the weights prefetched for later work.  So the
// workgroup is split by role (eight waves, two per SIMD, so that one can
// compute while the other waits):
//
//   * six COMPUTE waves issue nothing but weight loads.  Each walks the
//     workgroup's chunks with two register buffers: the next chunk's loads
//     are issued before the current chunk is computed.  Every chunk issues
//     the same 18 buffer loads per lane in straight-line code; slots a
//     chunk does not use get an offset past the buffer's range, which the
//     hardware answers with zeros without touching memory.  So waiting for a
//     buffer is always exactly "all but the 18 loads issued after it".
//     Activations and scales are read from LDS, results written to LDS;
//   * one I/O wave waits for the stage a chunk depends on and copies the
//     activation row and each chunk's scales into LDS (global-to-LDS DMA,
//     no registers).  It issues no stores, so its waits for those copies
//     never include a store round trip;
//   * one STORE wave stores the results the compute waves left in LDS and
//     signals a stage once its results are stored and complete.
//
// At a stage boundary the compute waves hold back the next stage's first
// chunk until the store wave has signalled the stage: a CU's vector memory
// operations queue in order, and with that chunk's loads issued first the
// result stores and the signal waited behind ~100 KB of weight loads
// (measured: the pass 6 % faster this way).  The loads still have the whole
// stage wait to arrive in.
//
// The roles hand over through LDS counters, not barriers: the I/O wave
// releases chunk k once its activations and scales are in LDS; each
// compute wave counts the chunks it has finished; the store wave counts
// the chunks it has stored, which frees the LDS areas they used.  Scales
// of chunk k+2 go into the area of chunk k-1 (a three-deep ring), results
// alternate between two areas.
// Activation rows are double-buffered by "epoch" (a new epoch starts where
// the stage or the activation pointer changes), so the next stage's row is
// staged while the last chunk of the current one is still being computed.
// The job table is copied into LDS at the start, so reading a job
// descriptor never waits on memory.
//
// Work split: each dependency stage ({q,k,v} -> o -> {gate,up} -> down per
// layer, then the lm_head) is balanced to a row over the G workgroups.  A
// stage of one matrix splits its rows evenly over all of them; the host may
// instead give the matrices of a stage disjoint runs of workgroups in
// proportion to their bytes (q, k, v of 5120 rows: 85, 85 and 86 of 256
// workgroups, 60 or 61 rows each, rather than 20 rows of each matrix on
// every workgroup), which keeps a workgroup's rows in one matrix and its
// chunks large.  A workgroup's rows of one matrix are cut into chunks of
// 12 * rows_per_half(K) rows (36 at K = 5120), the last one smaller.
//
// Arithmetic: half-wave h of a compute wave owns rows 2i + h of the wave's
// rows; lane L reads 16-byte code pieces L, L+32, ... of the row (512
// contiguous bytes per half-wave and instruction, nontemporal) and the two
// E4M3 scales of each piece.  Per 16-element block eight v_dot2_f32_bf16
// multiply the unscaled E2M1 values (exact in bf16) with X and one FMA
// applies the block scale; the 32 lanes of a half-wave are summed by a
// fixed butterfly, so every row is summed in the same order whatever chunk
// or wave it lands in: results do not depend on the launch.
//
// Stage signals: results are stored with agent-coherent stores; the store
// wave waits until its stores have completed (vmcnt(0)), then adds one to
// one of eight padded counters of the stage.  A waiter polls the counters
// and then reads the activations with device-scope copies (no fence).  Waits are
// bounded: on time-out the error flag in the control block is raised and
// the launch runs on to its end (its results are then invalid).  All
// workgroups are resident (one per CU), and the stage a chunk waits for
// only needs chunks that were released before it, so the waits cannot
// deadlock.
//
// lm_head: compute waves keep their best (logit, lowest index); at the end
// the workgroup publishes the best of its waves as one key (an atomic max
// on a packed key); the last workgroup out writes argmax (as a token id
// through the head's row map when there is one), runs the accept rule
// (TandemLLM README, introduction; with one row there are no drafts, so
// accept_len = 0) and zeroes the control block for the next launch.
#include <type_traits>

#include "launch.h"
#include "nvfp4_device.h"

namespace vg {

namespace {

// Stage timestamps, compiled in only for the diagnostic library
// (libvgemm_stamps.so, built beside libvgemm.so with VG_STAGE_STAMPS): per
// stage s and workgroup, the s_memrealtime (100 MHz) time at which
//   kStampDetect  the I/O wave saw stage s - 1 complete,
//   kStampReady   stage s's first activation row and scales were in LDS,
//   kStampDone    the compute waves had finished the stage's last chunk,
//   kStampSignal  its result stores had completed, just before the signal.
// Each stamp is one extra global store of lane 0 of the wave that takes it,
// so the timed pass runs slightly slower than the product build.
#ifdef VG_STAGE_STAMPS
constexpr int kStampStages = 1024, kStampWGs = 256;
enum { kStampDetect, kStampReady, kStampDone, kStampSignal, kStampKinds };
__device__ unsigned long long g_stamps[kStampKinds][kStampStages][kStampWGs];
__device__ __forceinline__ void stamp(int kind, int s) {
  if ((threadIdx.x & 63) == 0 && s >= 0 && s < kStampStages && blockIdx.x < (unsigned)kStampWGs)
    g_stamps[kind][s][blockIdx.x] = __builtin_amdgcn_s_memrealtime();
}
#else
enum { kStampDetect, kStampReady, kStampDone, kStampSignal };
__device__ __forceinline__ void stamp(int, int) {}
#endif

constexpr int kCW = 6;                  // compute waves
constexpr int kIO = kCW;                // index of the I/O wave
constexpr int kST = kCW + 1;            // index of the store wave
constexpr int kWG = (kCW + 2) * kWave;  // 512 threads: two waves per SIMD
constexpr int kSlots = 18;              // 16-byte code pieces per lane per buffer
constexpr int kMaxK = kSlots * 1024;    // a row of one half-wave fits one buffer
// Rows per half-wave per chunk: 18 / cpl, capped at 3 -- more rows would
// need more accumulators than the hot shapes (K = 5120: 3 rows, K = 17408:
// 1 row) can spare registers for; small K (only in tests) uses 3 of its
// slots' worth.
constexpr int kMaxRH = 3;
constexpr int kMaxChunkRows = 2 * kCW * kMaxRH;
// An activation row sits in LDS "transposed": a 16-byte unit u = 4q + t
// (piece q = 32 elements, sub-block t) is stored at t * kXPieces + q, so
// that the 32 lanes of a half-wave, which read pieces L + 32c, read 512
// consecutive bytes -- conflict-free -- instead of 16-byte reads at a
// 64-byte stride, which fall on two of the 32 banks.
constexpr int kXPieces = kMaxK / 32;
constexpr int kXRow = 4 * kXPieces;
// Largest scale bytes of one chunk: rows * K/16 <= 2 * kCW * (18 / cpl) * cpl * 64,
// copied by a fixed number of 1-KB DMA instructions.
constexpr int kMaxChunkScale = 2 * kCW * kSlots * 64;
constexpr int kScaleDma = (kMaxChunkScale + 1023) / 1024;
constexpr int kScaleBufs = 3;  // chunks k, k+1 (ready) and k+2 (in flight)
constexpr unsigned kOOB = 0x80000000u;  // buffer offset past every range used here
constexpr int kNT = 2;                  // buffer-load cache policy: nontemporal
// Bounded waits measure wall-clock time on the GPU's constant 100 MHz
// counter (s_memrealtime).  A stage wait gives up after half a second.  The
// waits between the roles of one workgroup only ever wait for work that is
// at most one stage wait (plus a chunk's compute) away, so their limit is
// eight times longer: they never expire while the I/O wave still waits for
// a stage, and a stage time-out alone raises the error flag.
constexpr unsigned long long kTicksPerSecond = 100000000ull;
constexpr unsigned long long kStageWaitTicks = kTicksPerSecond / 2;
constexpr unsigned long long kLocalWaitTicks = 4 * kTicksPerSecond;
__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// s_waitcnt immediate for vmcnt(0) (gfx9 encoding: vmcnt[3:0]+[15:14],
// expcnt[6:4], lgkmcnt[11:8]; the other two fields at "no wait").
constexpr int kWaitVm0 = 0x0F70;
// vmcnt(kScaleDma): everything but the newest chunk's scale DMAs.
constexpr int kWaitVmScale = 0x0F70 | (kScaleDma & 15) | ((kScaleDma >> 4) << 14);
static_assert(kScaleDma < 64, "vmcnt holds at most 63");

static_assert(sizeof(StreamJob) % 16 == 0, "job descriptors are copied as 16-byte pieces");

__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_out(float* p, float v) {
  __hip_atomic_store((VG_GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned lds_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}


__host__ __device__ __forceinline__ int pieces_per_lane(int k) { return (k + 1023) >> 10; }
// min(kSlots / pieces, kMaxRH) without a division (this runs per job in
// every wave's chunk walk).
__host__ __device__ __forceinline__ int rows_per_half(int k) {
  static_assert(kSlots == 18 && kMaxRH == 3, "the thresholds below are 18 / pieces, capped at 3");
  const int cpl = pieces_per_lane(k);
  return cpl <= 6 ? 3 : (cpl <= 9 ? 2 : 1);
}
__host__ __device__ __forceinline__ int chunk_cap(int k) { return 2 * kCW * rows_per_half(k); }

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time i).
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F& f) {
  static_for_impl<0, N>(f);
}

struct Shared {
  StreamJob jobs[kStepMaxJobs];      // the launch's job table
  u32x4 xs[2][kXRow];                // activation rows of even / odd epochs (transposed, see kXPieces)
  u32x4 sc[kScaleBufs][kScaleDma * 64];  // scale bytes of chunk ordinal k in sc[k % 3]
  float res[2][kMaxChunkRows];       // results of chunks with even / odd ordinal
  unsigned done[2];                  // compute waves finished with the chunk of that parity
  unsigned ready;                    // chunks released to the compute waves
  unsigned flushed;                  // chunks whose results are stored (all areas they used are free)
  unsigned signalled;                // 1 + the last stage this workgroup has signalled
  int flag;
  unsigned long long lm_key[kCW];    // lm_head: each compute wave's best key, reduced by thread 0
};

// Job i from the LDS table, in scalar registers.
__device__ __forceinline__ StreamJob lds_job(const Shared& sh, int i) {
  struct Words {
    unsigned w[sizeof(StreamJob) / 4];
  } v;
  const unsigned* p = reinterpret_cast<const unsigned*>(&sh.jobs[i]);
#pragma unroll
  for (int k = 0; k < (int)(sizeof(StreamJob) / 4); ++k) v.w[k] = __builtin_amdgcn_readfirstlane(p[k]);
  return __builtin_bit_cast(StreamJob, v);
}

// The code pieces of one chunk, per lane (the chunk's scales are in LDS).
struct Buf {
  u32x4 q[kSlots];
};

struct Chunk {
  int job, r0, rows;
};

// Rows [begin, begin + count) of a chunk belong to compute wave w.
__device__ __forceinline__ void wave_rows(int rows, int w, int& begin, int& count) {
  begin = rows * w / kCW;
  count = rows * (w + 1) / kCW - begin;
}

// Rows per half-wave that a wave's slots are laid out for in one chunk:
// enough for its `count` rows, at most what the job's K allows.  A wave
// computes every row slot of its layout (slots past its rows hold zero
// codes), so a wave with 3 or 4 rows of a 20-row chunk lays out 2 per
// half-wave, not the 3 that K = 5120 allows (measured: those chunks
// computed 6 rows per wave for 3 or 4 real ones).
__device__ __forceinline__ int wave_rh(int k, int count) {
  // never below two when K allows two: the one-row layout sums a row in
  // another order (four chains per piece), so it is kept for the K that
  // allow only one row per half-wave, and a row's bits depend on K alone
  const int r = (count + 1) >> 1, m = rows_per_half(k), lo = m < 2 ? m : 2;
  return r < lo ? lo : (r < m ? r : m);
}

// Walks this workgroup's chunks in job order (the same in every wave).
// The chunk walk runs in every wave between chunks, so it avoids runtime
// divisions (software sequences on this GPU): the workgroup's rows come
// from the job's precomputed split (step_rows), a job's chunk count from a
// constant divisor, and the chunk sizes from the cap and one remainder
// per job.
struct Cursor {
  int job = 0, pos = 0, left = 0;  // left: chunks still to cut, from row pos on
  int base = 0, rem = 0;           // rows per chunk, and in the job's last chunk
};

__device__ __forceinline__ bool next_chunk(const Shared& sh, int njobs, Cursor& cu, Chunk& out) {
  static_assert(2 * kCW == 12, "chunk caps below are 12 * rows_per_half");
  while (cu.left == 0) {
    if (cu.job >= njobs) return false;
    const StreamJob j = lds_job(sh, cu.job);
    const int rows = step_rows(j, (int)blockIdx.x, (int)gridDim.x, cu.pos);
    // chunks of chunk_cap(k) rows and a last one with the rest: the
    // compute of a stage's last chunk is exposed, so it is the smallest
    // (measured: the 64-layer step 0.1-0.4 % faster than equal chunks)
    const int rh = rows_per_half(j.k);
    const int cnt = rh == 3 ? (rows + 35) / 36 : rh == 2 ? (rows + 23) / 24 : (rows + 11) / 12;
    cu.left = cnt;
    cu.base = 12 * rh;
    cu.rem = rows - cu.base * (cnt - 1);
    if (cu.left == 0) ++cu.job;
  }
  const int rows = cu.left == 1 ? cu.rem : cu.base;
  out = Chunk{cu.job, cu.pos, rows};
  cu.pos += rows;
  if (--cu.left == 0) ++cu.job;
  return true;
}

// Activation epochs: a new one starts where the stage or the activation
// pointer changes; its row goes to buffer n & 1.  Both roles track them
// with the same rule.
struct Epoch {
  int stage = -1, n = -1;
  const uint16_t* x = nullptr;
  __device__ __forceinline__ bool advance(const StreamJob& j) {
    if (j.stage == stage && j.x == x) return false;
    stage = j.stage;
    x = j.x;
    ++n;
    return true;
  }
};

// ---- compute waves -----------------------------------------------------

// Slot s of the buffer holds piece c = s / rh of local row 2 * (s % rh) + h,
// rh = wave_rh(K, the wave's rows of the chunk).
__device__ __forceinline__ void issue(const StreamJob& j, const Chunk& ch, int w, Buf& b) {
  const int lane = threadIdx.x & 63, h = lane >> 5, L = lane & 31;
  int wb, wc;
  wave_rows(ch.rows, w, wb, wc);
  const unsigned rb = (unsigned)j.k >> 1;
  const int cpl = pieces_per_lane(j.k), rh = wave_rh(j.k, wc);
  const size_t row0 = (size_t)(ch.r0 + wb);
  const __amdgpu_buffer_rsrc_t rw = rsrc(j.wq + row0 * rb, (unsigned)wc * rb);
  int i = 0, c = 0;
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const unsigned piece = (unsigned)(L + 32 * c), l = (unsigned)(2 * i + h);
    const bool ok = c < cpl && (int)l < wc && piece * 16u < rb;
    b.q[s] = __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? l * rb + piece * 16u : kOOB, 0, kNT);
    const bool wrap = i + 1 == rh;
    i = wrap ? 0 : i + 1;
    c = wrap ? c + 1 : c;
  }
}

// The dot products of G slots.  Slot g uses code pieces q[S0 + g * SS] of
// the buffer and activation set x[XI(g)]; words 0/1 of a piece belong to
// its first 16-element block, words 2/3 to its second, and each block's sum
// is scaled once.  The chains are interleaved in program order (for each
// code byte, first the decodes, then the dot2s into different chains), so
// a dependent dot2 comes several instructions after the previous one on
// its chain and the decode and dot2 latencies hide inside one wave; a
// chain-at-a-time order runs at about a third of the issue rate.
//   * BLK (two or three rows per half-wave: every K <= 9216, whatever a
//     wave's own row count): one eight-deep chain per 16-element block,
//     2*G chains, started from zero once per block and applied with one
//     FMA -- the fewest instructions per code;
//   * otherwise (one row per half-wave: K > 9216): 4*G four-deep chains,
//     one per code word, two added per block, so that even one slot keeps
//     four chains in flight.
// The form depends on K alone, so a row's sum does not depend on the
// chunk or wave it lands in.
template <int G, int S0, int SS, int NX, bool BLK>
__device__ __forceinline__ void piece_group(const Buf& b, const u32x4 (&x)[NX][4], const f32x2 (&s)[G],
                                            float (&acc)[G]) {
  if constexpr (BLK) {
    float ch[G][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sel = j & 3, half = j >> 2;  // word 2 * blk + half, byte sel
      bf16x2 e[G][2];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const unsigned word = b.q[S0 + g * SS][2 * blk + half];
          switch (sel) {
            case 0: e[g][blk] = e2m1x2_bf16<0>(word); break;
            case 1: e[g][blk] = e2m1x2_bf16<1>(word); break;
            case 2: e[g][blk] = e2m1x2_bf16<2>(word); break;
            default: e[g][blk] = e2m1x2_bf16<3>(word); break;
          }
        }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const unsigned xv = x[NX == 1 ? 0 : g][2 * blk + half][sel];
          ch[g][blk] = __builtin_amdgcn_fdot2_f32_bf16(e[g][blk], as_bf16x2(xv), j == 0 ? 0.0f : ch[g][blk], false);
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc[g] = __builtin_fmaf(s[g][0], ch[g][0], acc[g]);
      acc[g] = __builtin_fmaf(s[g][1], ch[g][1], acc[g]);
    }
    return;
  }
  float ch[G][4];
#pragma unroll
  for (int sel = 0; sel < 4; ++sel) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x2 e[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const unsigned word = b.q[S0 + g * SS][st];
        switch (sel) {
          case 0: e[g] = e2m1x2_bf16<0>(word); break;
          case 1: e[g] = e2m1x2_bf16<1>(word); break;
          case 2: e[g] = e2m1x2_bf16<2>(word); break;
          default: e[g] = e2m1x2_bf16<3>(word); break;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const unsigned xv = x[NX == 1 ? 0 : g][st][sel];
        ch[g][st] = __builtin_amdgcn_fdot2_f32_bf16(e[g], as_bf16x2(xv), sel == 0 ? 0.0f : ch[g][st], false);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] = __builtin_fmaf(s[g][0], ch[g][0] + ch[g][1], acc[g]);
    acc[g] = __builtin_fmaf(s[g][1], ch[g][2] + ch[g][3], acc[g]);
  }
}

// Row sums times g for the wave's rows of a chunk whose rows take RH slots
// per half-wave (RH = wave_rh: at most 18 / cpl).  Slots of rows the wave does not have hold
// zero codes (their loads were out of range) and their sums are never
// used.  The rows of one piece form one group (one row: the piece alone);
// pieces c >= cpl are skipped (uniformly).  Results go to LDS (GEMM) or
// into this lane's running best (lm_head).
template <int RH>
__device__ __forceinline__ void compute_cls(const StreamJob& j, const Chunk& ch, int w, const Buf& b,
                                            const unsigned short* sc, float* res, const u32x4* xs,
                                            float& best_v, int& best_i) {
  constexpr int CMAX = kSlots / RH;
  const int lane = threadIdx.x & 63, h = lane >> 5, L = lane & 31;
  const int cpl = pieces_per_lane(j.k);
  const int rp = j.k >> 5;  // 16-byte pieces per row = scale pairs per row
  int wb, wc;
  wave_rows(ch.rows, w, wb, wc);
  if (wc == 0) return;
  float acc[RH];
#pragma unroll
  for (int i = 0; i < RH; ++i) acc[i] = 0.0f;
  // one per-lane base each; every read below adds a constant (immediate)
  // or a wave-uniform offset to it
  const u32x4* xl = xs + L;
  const unsigned short* sl = sc + (wb + h) * rp + L;
  auto xpiece = [&](int c, u32x4 (&x)[4]) {
    x[0] = xl[32 * c];
    x[1] = xl[kXPieces + 32 * c];
    x[2] = xl[2 * kXPieces + 32 * c];
    x[3] = xl[3 * kXPieces + 32 * c];
  };
  // the scale pair of piece c of row slot i, read unconditionally (past
  // the row it reads the next row's scales or the area's slack, still in
  // the area) and replaced by 0 there: those pieces hold zero codes, and
  // whatever LDS holds must not meet them
  auto scale = [&](int c, int i) -> f32x2 {
    const unsigned short raw = sl[2 * i * rp + 32 * c];
    return e4m3x2_lo(L + 32 * c < rp ? raw : (unsigned short)0);
  };
  // activations double-buffered across pieces: piece c+1's LDS reads are
  // in flight while piece c is computed
  u32x4 xb[2][1][4];
  xpiece(0, xb[0][0]);
  if constexpr (RH >= 2) {
    // the RH rows of piece c (slots c*RH + i, one activation set)
    auto piece = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      if (c < cpl) {
        if (c + 1 < CMAX && c + 1 < cpl) xpiece(c + 1, xb[(c + 1) & 1][0]);
        f32x2 s[RH];
#pragma unroll
        for (int i = 0; i < RH; ++i) s[i] = scale(c, i);
        piece_group<RH, c * RH, 1, 1, true>(b, xb[c & 1], s, acc);
      }
      // keep later pieces' reads from being hoisted into this one (they
      // would all be hoisted to the top and spilled)
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<CMAX>(piece);
  } else {
    // one row: each piece alone (four chains)
    auto piece = [&](auto cc) {
      constexpr int c = decltype(cc)::value;
      if (c < cpl) {
        if (c + 1 < CMAX && c + 1 < cpl) xpiece(c + 1, xb[(c + 1) & 1][0]);
        const f32x2 s[1] = {scale(c, 0)};
        piece_group<1, c, 1, 1, false>(b, xb[c & 1], s, acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<CMAX>(piece);
  }
#pragma unroll
  for (int i = 0; i < RH; ++i) {
    if (2 * i < wc) {
      const float v = half_wave_sum(acc[i]) * j.g;  // valid in lanes L >= 16
      const int l = 2 * i + h;
      if (L == 31 && l < wc) {
        const int lr = wb + l;
        if (j.kind == 0) {
          res[lr] = v;
        } else if (better(v, ch.r0 + lr, best_v, best_i)) {
          best_v = v;
          best_i = ch.r0 + lr;
        }
      }
    }
  }
}

__device__ __forceinline__ void compute(const StreamJob& j, const Chunk& ch, int w, const Buf& b,
                                        const unsigned short* sc, float* res, const u32x4* xs,
                                        float& best_v, int& best_i) {
  static_assert(kMaxRH == 3, "the classes below are the values of wave_rh");
  int wb, wc;
  wave_rows(ch.rows, w, wb, wc);
  switch (wave_rh(j.k, wc)) {
    case 3: compute_cls<3>(j, ch, w, b, sc, res, xs, best_v, best_i); break;
    case 2: compute_cls<2>(j, ch, w, b, sc, res, xs, best_v, best_i); break;
    default: compute_cls<1>(j, ch, w, b, sc, res, xs, best_v, best_i); break;
  }
}

__device__ __forceinline__ const unsigned short* scales(const Shared& sh, int idx) {
  return reinterpret_cast<const unsigned short*>(sh.sc[idx]);
}

// Waits until chunk ordinal k has been released by the I/O wave (its
// activations and scales are in LDS).  The I/O wave releases every chunk
// unless a stage wait timed out, and then it still releases them all.
__device__ __forceinline__ void wait_ready(const Shared& sh, unsigned k) {
  while (lds_load(&sh.ready) <= k) __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One released chunk of a compute wave: compute, then report.
// `sidx` is the chunk's scale area (ordinal % 3).
__device__ __forceinline__ void work(Shared& sh, const Chunk& ch, int w, const Buf& b, int parity, int& sidx,
                                     Epoch& ep, float& best_v, int& best_i) {
  const StreamJob j = lds_job(sh, ch.job);
  ep.advance(j);
  compute(j, ch, w, b, scales(sh, sidx), sh.res[parity], sh.xs[ep.n & 1], best_v, best_i);
  sidx = sidx == kScaleBufs - 1 ? 0 : sidx + 1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");  // results are in LDS
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(&sh.done[parity], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until the store wave has signalled stage s - 1.  It does once every
// compute wave has finished that stage's chunks, which the caller has.
__device__ __forceinline__ void wait_signalled(const Shared& sh, unsigned s) {
  while (lds_load(&sh.signalled) < s) __builtin_amdgcn_s_sleep(1);
}

__device__ __forceinline__ void compute_loop(const StreamArgs& a, Shared& sh, int njobs, float& best_v,
                                             int& best_i) {
  // the wave index, known to the compiler as wave-uniform (scalar): buffer
  // descriptors built from it stay in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Cursor cu;
  Chunk cur, nxt;
  Buf b0, b1;
  Epoch ep;
  int sidx = 0;
  unsigned k = 0;  // ordinal of cur
  // Chunk ordinals alternate parity, and so do the two result areas; with two register buffers, b0 always holds an even chunk and b1
  // an odd one.  The prefetch is issued even past the last chunk (as an
  // empty chunk, whose loads are all out of range): every path then has
  // the same loads outstanding, so the compiler's wait for a buffer is
  // exactly "all but the 18 loads issued after it".
  bool have = next_chunk(sh, njobs, cu, cur);
  if (!have) return;
  issue(lds_job(sh, cur.job), cur, w, b0);
  for (;;) {
    bool more = next_chunk(sh, njobs, cu, nxt);
    if (!more) nxt = Chunk{cur.job, 0, 0};
    int cst = lds_job(sh, cur.job).stage;
    bool defer = a.waits && more && lds_job(sh, nxt.job).stage != cst;
    if (!defer) issue(lds_job(sh, nxt.job), nxt, w, b1);
    wait_ready(sh, k++);
    work(sh, cur, w, b0, 0, sidx, ep, best_v, best_i);
    if (defer) {
      wait_signalled(sh, (unsigned)cst + 1u);
      issue(lds_job(sh, nxt.job), nxt, w, b1);
    }
    if (!more) break;
    cur = nxt;
    more = next_chunk(sh, njobs, cu, nxt);
    if (!more) nxt = Chunk{cur.job, 0, 0};
    cst = lds_job(sh, cur.job).stage;
    defer = a.waits && more && lds_job(sh, nxt.job).stage != cst;
    if (!defer) issue(lds_job(sh, nxt.job), nxt, w, b0);
    wait_ready(sh, k++);
    work(sh, cur, w, b1, 1, sidx, ep, best_v, best_i);
    if (defer) {
      wait_signalled(sh, (unsigned)cst + 1u);
      issue(lds_job(sh, nxt.job), nxt, w, b0);
    }
    if (!more) break;
    cur = nxt;
  }
}

// ---- I/O wave ----------------------------------------------------------

// A bounded wait gave up: raise the launch's error flag.  A single GEMM
// launch has no control block (it waits on no stage); then the wait just
// ends and the launch runs on.
__device__ __forceinline__ void raise_error(const StreamArgs& a, int lane) {
  if (lane == 0 && a.ctl) st_agent(&a.ctl->error, 1u);
}

// Polls until `target` workgroups have signalled stage `s` (whole wave,
// uniform result), then acquires at agent scope.
__device__ bool wait_stage(const StreamArgs& a, int s, unsigned target) {
  const int lane = threadIdx.x & 63;
  const unsigned long long t0 = now_ticks();
  for (;;) {
    unsigned v = lane < kDoneSlots ? ld_agent(&a.stage_done[s][lane].v) : 0u;
#pragma unroll
    for (int off = kDoneSlots / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    // No acquire fence: what a stage reads that an earlier stage may have
    // written -- its activation row (stage_x) and the output row scales --
    // is read at agent scope, after this poll has returned.  (The fence,
    // which invalidates the caches once per stage and workgroup, made the
    // 64-layer step 2 % slower.)
    if (__shfl(v, 0, kWave) >= target) return true;
    if (now_ticks() - t0 > kStageWaitTicks) break;
    __builtin_amdgcn_s_sleep(2);
  }
  raise_error(a, lane);
  return false;
}

// Waits until every compute wave has finished the chunk of `parity`.  The
// compute waves need nothing more from this wave to finish a released
// chunk, so the wait ends; it is bounded all the same (kLocalWaitTicks).
__device__ bool wait_done(const StreamArgs& a, Shared& sh, int parity) {
  const unsigned long long t0 = now_ticks();
  for (;;) {
    if (__hip_atomic_load(&sh.done[parity], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= (unsigned)kCW) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      return true;
    }
    if (now_ticks() - t0 > kLocalWaitTicks) break;
    __builtin_amdgcn_s_sleep(1);
  }
  raise_error(a, threadIdx.x & 63);
  return false;
}

// Starts copying the K bf16 activations of job j into `xs` (transposed,
// see kXPieces: each copy instruction gathers sub-block t of 64
// consecutive pieces) and zeroes the pieces past K (up to K rounded up to
// 1024), which the compute waves read as padding.  The copies are at
// device scope (dma16_agent): the row may have been written by an earlier
// stage on another XCD.  Completes at this wave's vmcnt(0).
__device__ void stage_x(const StreamJob& j, u32x4* xs) {
  const int lane = threadIdx.x & 63;
  const int pieces = j.k >> 5;
  const u32x4 rs = rsrc_words(j.x, (unsigned)j.k * 2u);
  for (int b = 0; b * kWave < pieces; ++b) {
    const int q = b * kWave + lane;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      dma16_agent(rs, q < pieces ? (unsigned)(4 * q + t) * 16u : kOOB, lds_addr(xs + t * kXPieces + b * kWave));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the zeroing below must land after the copies
  const int pad = pieces_per_lane(j.k) * 32;
  for (int q = pieces + lane; q < pad; q += kWave)
#pragma unroll
    for (int t = 0; t < 4; ++t) xs[t * kXPieces + q] = u32x4{0, 0, 0, 0};
}

// Starts copying the scale bytes of chunk ch into scale area `idx`
// (chunk-local row-major, K/16 bytes per row) with exactly kScaleDma DMA
// instructions (pieces past the chunk are out of range: nothing is read
// or written for them).  K % 64 == 0 keeps every row's scales whole dwords,
// so the buffer's range check (per dword) cuts exactly at the matrix's end.
__device__ void stage_scales(const StreamJob& j, const Chunk& ch, Shared& sh, int idx) {
  const int lane = threadIdx.x & 63;
  const unsigned sb = (unsigned)j.k >> 4;
  const u32x4 rs = rsrc_words(j.ws, (unsigned)j.n * sb);
  const unsigned base = (unsigned)ch.r0 * sb, bytes = (unsigned)ch.rows * sb;
#pragma unroll
  for (int t = 0; t < kScaleDma; ++t) {
    const unsigned off = (unsigned)(t * kWave + lane) * 16u;
    dma16(rs, off < bytes ? base + off : kOOB, lds_addr(sh.sc[idx] + t * kWave));
  }
}

__device__ void signal_stage(const StreamArgs& a, int s) {
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's result stores have completed
  stamp(kStampSignal, s);
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(&a.stage_done[s][blockIdx.x % kDoneSlots].v, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

struct IoState {
  Epoch ep;
  int done_stage = -1;
};

// Everything chunk `c` needs before it is released: the stage it depends
// on, its activation row, and its scales (staged a chunk earlier).  If the
// newest thing this wave issued is the following chunk's scale DMA
// (`ahead`), that is all it may leave in flight; otherwise nothing.
// Loads complete in order, so "at most kScaleDma outstanding" means every
// load issued before that DMA -- this chunk's scales included -- is done.
__device__ void prepare(const StreamArgs& a, Shared& sh, const StreamJob& j, IoState& st, bool ahead) {
  bool waited = false;
  if (j.stage != st.ep.stage && a.waits) {
    const int need = j.stage - 1;
    if (need >= 0 && need > st.done_stage) {
      (void)wait_stage(a, need, a.stage_total[need]);  // a time-out raises the error flag
      st.done_stage = need;
      waited = true;
      stamp(kStampDetect, j.stage);
    }
  }
  if (st.ep.advance(j)) stage_x(j, sh.xs[st.ep.n & 1]);
  if (ahead)
    __builtin_amdgcn_s_waitcnt(kWaitVmScale);
  else
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (waited) stamp(kStampReady, j.stage);
}

// Stores the results of chunk ch (LDS area `parity`; lane t owns row t)
// times this lane's row scale `rsc`, and clears that area's completion
// count for the chunk after next.  With per-row scales the job's g is 1
// and the sum is exact so far, so sum * rsc is the one rounding sum * g
// would be; without them rsc == 1 (exact).
static_assert(kMaxChunkRows <= kWave, "one store lane per chunk row");
__device__ void flush(Shared& sh, const StreamJob& j, const Chunk& ch, int parity, float rsc) {
  const int lane = threadIdx.x & 63;
  if (j.kind == 0 && lane < ch.rows) store_out(&j.y[ch.r0 + lane], sh.res[parity][lane] * rsc);
  if (lane == 0) lds_store(&sh.done[parity], 0u);
}

// Releases chunk ordinals below `n` to the compute waves.
__device__ __forceinline__ void release(Shared& sh, unsigned n) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if ((threadIdx.x & 63) == 0) lds_store(&sh.ready, n);
}

// Waits until the results of chunk ordinals below n are stored.  The store
// wave needs nothing from this wave for chunks already released.
__device__ bool wait_flushed(const StreamArgs& a, const Shared& sh, unsigned n) {
  const unsigned long long t0 = now_ticks();
  for (;;) {
    if (lds_load(&sh.flushed) >= n) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      return true;
    }
    if (now_ticks() - t0 > kLocalWaitTicks) break;
    __builtin_amdgcn_s_sleep(1);
  }
  raise_error(a, threadIdx.x & 63);
  return false;
}

// Per chunk k: once chunk k-1 is stored, the scales of chunk k+2 go into
// the area chunk k-1 used (a three-deep ring), then chunk k+1 is prepared
// -- its stage waited for, its activation row staged -- and released.
// This wave issues nothing but copies into LDS and the stage polls, so its
// waits never include a store round trip.
__device__ __forceinline__ void io_loop(const StreamArgs& a, Shared& sh, int njobs) {
  IoState st;
  Cursor cu;
  Chunk cur, nxt, nx2;
  int sidx = 0;      // scale area of cur
  unsigned k = 0;    // ordinal of cur
  if (!next_chunk(sh, njobs, cu, cur)) return;
  bool more = next_chunk(sh, njobs, cu, nxt);
  StreamJob cj = lds_job(sh, cur.job), nj = lds_job(sh, more ? nxt.job : cur.job);
  stage_scales(cj, cur, sh, 0);
  if (more) stage_scales(nj, nxt, sh, 1);
  prepare(a, sh, cj, st, false);
  release(sh, 1);
  while (more) {
    const bool more2 = next_chunk(sh, njobs, cu, nx2);
    // chunk k-1's scale area, result area and activation epoch are free
    if (k > 0) (void)wait_flushed(a, sh, k);
    if (more2) {
      const int s2 = sidx + 2 >= kScaleBufs ? sidx + 2 - kScaleBufs : sidx + 2;
      stage_scales(lds_job(sh, nx2.job), nx2, sh, s2);
    }
    prepare(a, sh, nj, st, more2);
    release(sh, k + 2);
    ++k;
    cur = nxt;
    cj = nj;
    nxt = nx2;
    more = more2;
    if (more) nj = lds_job(sh, nxt.job);
    sidx = sidx == kScaleBufs - 1 ? 0 : sidx + 1;
  }
}

// ---- store wave --------------------------------------------------------

// Per chunk, once every compute wave has finished it: stores its results
// and reports it stored; after the last chunk of a stage, waits until its
// stores are complete and signals the stage.
__device__ __forceinline__ void store_loop(const StreamArgs& a, Shared& sh, int njobs) {
  Cursor cu;
  Chunk cur, nxt;
  int parity = 0;
  unsigned k = 0;
  if (!next_chunk(sh, njobs, cu, cur)) return;
  for (;;) {
    const bool more = next_chunk(sh, njobs, cu, nxt);
    const StreamJob j = lds_job(sh, cur.job);
    // the chunk's row scales are read before its results are awaited, so
    // that read is not between "results ready" and the stores
    const int lane = threadIdx.x & 63;
    const float rsc = j.kind == 0 && j.gr && lane < cur.rows
                          ? __hip_atomic_load(&j.gr[cur.r0 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 1.0f;
    wait_done(a, sh, parity);
    if (!more || lds_job(sh, nxt.job).stage != j.stage) stamp(kStampDone, j.stage);
    flush(sh, j, cur, parity, rsc);
    // the LDS reads of the flush have completed before the areas are handed back
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if ((threadIdx.x & 63) == 0) lds_store(&sh.flushed, k + 1);
    if (a.waits && (!more || lds_job(sh, nxt.job).stage != j.stage)) {
      signal_stage(a, j.stage);
      if ((threadIdx.x & 63) == 0) lds_store(&sh.signalled, (unsigned)j.stage + 1u);
    }
    if (!more) break;
    cur = nxt;
    parity ^= 1;
    ++k;
  }
}

__global__ __launch_bounds__(kWG) void step_gemv_kernel(StreamArgs a) {
  __shared__ Shared sh;
  StreamCtl* ctl = a.ctl;
  // the job table into LDS
  const int njobs = a.jobs ? a.njobs : 1;
  if (a.jobs) {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.jobs);
    u32x4* dst = reinterpret_cast<u32x4*>(sh.jobs);
    for (int i = threadIdx.x; i < njobs * (int)(sizeof(StreamJob) / 16); i += kWG) dst[i] = ld_act(src + i);
  } else if (threadIdx.x == 0) {
    sh.jobs[0] = a.job0;
  }
  if (threadIdx.x < 2) sh.done[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    sh.ready = 0;
    sh.flushed = 0;
    sh.signalled = 0;
  }
  __syncthreads();

  float best_v = -__builtin_inff();
  int best_i = -1;
  const int role = threadIdx.x >> 6;
  // The I/O and store waves share SIMDs with compute waves; their hand-offs
  // (polls, releases, result stores) are on every chunk's critical path, so
  // they issue first (measured: the pass 1.2 % faster).
  if (role == kIO) {
    __builtin_amdgcn_s_setprio(3);
    io_loop(a, sh, njobs);
    __builtin_amdgcn_s_setprio(0);
  } else if (role == kST) {
    __builtin_amdgcn_s_setprio(3);
    store_loop(a, sh, njobs);
    __builtin_amdgcn_s_setprio(0);
  } else {
    compute_loop(a, sh, njobs, best_v, best_i);
  }

  // A launch that waits on stages or has an lm_head counts its workgroups
  // out; the last one finishes the lm_head and zeroes the control block and
  // the stage counters for the next launch.
  if (!a.waits && !a.has_lmhead) return;
  if (a.has_lmhead && role < kCW) {
    // each compute wave publishes its best (the half-waves hold different rows)
    const float ov = __shfl_xor(best_v, 32, kWave);
    const int oi = __shfl_xor(best_i, 32, kWave);
    if (oi >= 0 && (best_i < 0 || better(ov, oi, best_v, best_i))) { best_v = ov; best_i = oi; }
    // the row sums (and so the running bests) live in lanes 31 and 63
    if ((threadIdx.x & 63) == 31) sh.lm_key[role] = best_i >= 0 ? argmax_key(best_v, (unsigned)best_i) : 0ull;
  }
  // Counting out without cache fences, as the stage signals do: every wave
  // waits until its own memory operations (result stores, stage signals)
  // are acknowledged; the workgroup's one key goes out and is acknowledged
  // before its exit count.  The last workgroup out then reads the keys
  // with agent-scope loads and resets the counters: every other
  // workgroup's atomics were performed before its count.  (Agent-scope
  // fences here, one per workgroup, made a 65,536-row lm_head call 85
  // instead of 50 us and the 64-layer step 60 us slower.)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (a.has_lmhead) {
      unsigned long long k = 0;
      for (int r = 0; r < kCW; ++r) k = sh.lm_key[r] > k ? sh.lm_key[r] : k;
      if (k) __hip_atomic_fetch_max(&ctl->keys[0][blockIdx.x % kKeySlots], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    const unsigned prev = __hip_atomic_fetch_add(&ctl->exits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.flag = prev == gridDim.x - 1;
  }
  __syncthreads();
  if (!sh.flag) return;
  if (threadIdx.x == 0) {
    if (a.has_lmhead) {
      unsigned long long best = 0;
      for (int s = 0; s < kKeySlots; ++s) {
        const unsigned long long k =
            __hip_atomic_load(&ctl->keys[0][s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        best = k > best ? k : best;
        __hip_atomic_store(&ctl->keys[0][s], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // one row (T = 1): no drafts, so only the root is agreed
      const int row = (int)key_index(best);
      a.argmax[0] = a.token_map && row >= 0 && row < a.lm_rows ? a.token_map[row] : row;
      a.accept_len[0] = 0;
      if (a.accept_node) a.accept_node[0] = 0;
    }
    st_agent(&ctl->exits, 0u);
  }
  if (a.waits)
    for (int s = threadIdx.x; s < a.nstages * kDoneSlots; s += kWG)
      st_agent(&a.stage_done[s / kDoneSlots][s % kDoneSlots].v, 0u);
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

bool step_gemv_supports(int K) { return K >= 64 && K % 64 == 0 && K <= kMaxK; }

// One workgroup per CU: the kernel's LDS and registers allow no more, and
// the stage waits need every workgroup resident.
int step_gemv_grid() { return num_cus(); }

hipError_t launch_step_gemv(const StreamArgs& a, hipStream_t stream) {
  const int G = step_gemv_grid();
  StreamArgs b = a;
  if (!b.jobs) set_step_rows(b.job0, 0, G);
  hipLaunchKernelGGL(step_gemv_kernel, dim3(G), dim3(kWG), 0, stream, b);
  return hipGetLastError();
}

}  // namespace vg

#ifdef VG_STAGE_STAMPS
// Diagnostic library only: copies the stamps of the last step launch into
// out[kind][stage][workgroup] (4 x 1024 x 256 values; slots a launch did
// not stamp keep older values).  Returns 0, or 1 on a HIP error.
extern "C" int vg_stage_stamps(unsigned long long* out) {
  return hipMemcpyFromSymbol(out, HIP_SYMBOL(vg::g_stamps), sizeof(vg::g_stamps)) == hipSuccess ? 0 : 1;
}
#endif

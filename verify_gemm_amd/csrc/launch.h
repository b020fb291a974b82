// Internal interface between the C-ABI layer (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vg {

constexpr int VG_MAX_M_DEV = 68;
constexpr int kKeySlots = 16;     // atomic-max slots per lm_head row
constexpr int kMaxStages = 1024;  // dependency stages of one step

// One NVFP4 matrix of a step.  For the stream kernels, items are
// contiguous blocks of rows_per_item weight rows (all of K) -- or, from a
// spread job's first spread block f on, one K slice of such a block (item
// f + (b - f) * S + s is slice s of block b, S = lds_slices(k)); jobs are
// listed in pass order and their items are numbered consecutively from
// item_begin.  The M = 1 step kernel has no items: the same four words hold
// the job's rows per workgroup (step_rows).
struct StreamJob {
  const uint8_t* wq;  // [n][k/2]
  const uint8_t* ws;  // [n][k/16]
  const uint16_t* x;  // [M][k] bf16 bits
  float* y;           // [M][n] (kind 0)
  const float* gr;    // [n] per-row output scale (kind 0; then g == 1), or null
  float g;
  int n;
  int k;
  int stage;          // dependency stage (non-decreasing along the list)
  int kind;           // 0: GEMM, 1: lm_head (argmax, no output matrix)
  int fmt;            // weight format: 0 NVFP4 (wq codes, ws block scales), 1 FP8 E4M3 (wq [n][k] bytes)
  union {
    struct {            // stream kernels
      int item_begin;
      int items;
      int spread;       // 0, or 1 + the first block whose K slices are separate items (a step, M >= 2)
      int part_base;    // spread: partial slot of the job's first slice item (StreamArgs::part / part_cnt)
    };
    struct {            // step kernel: the rows go to wgn workgroups from wg0 on (cyclically);
      int wg0;          // the i-th of them takes rq rows, one more if i < rr, in order
      int wgn;
      int rq;
      int rr;
    };
  };
};
static_assert(sizeof(StreamJob) % 16 == 0, "the job table is copied in 16-byte pieces");

// The step kernel's rows of job j in workgroup w of a grid of G: returns
// the count and sets pos to the first row (0 rows: w is not one of the
// job's workgroups).  Host and kernel use this one rule.
__host__ __device__ __forceinline__ int step_rows(const StreamJob& j, int w, int G, int& pos) {
  int i = w - j.wg0;
  if (i < 0) i += G;
  if (i >= j.wgn) {
    pos = 0;
    return 0;
  }
  pos = i * j.rq + (i < j.rr ? i : j.rr);
  return j.rq + (i < j.rr ? 1 : 0);
}

// Splits job j's rows as equally as rows allow over wgn workgroups from
// wg0 on (wg0 < G, wgn <= G).
inline void set_step_rows(StreamJob& j, int wg0, int wgn) {
  j.wg0 = wg0;
  j.wgn = wgn;
  j.rq = j.n / wgn;
  j.rr = j.n % wgn;
}

// K slices of the M >= 2 MFMA item (K % 128 == 0): a block's sum over K is
// taken slice by slice, each slice summed from zero over its 256-element
// windows in order, and the slice sums added in slice order.  Whether one
// workgroup runs every slice or each slice is its own item, the result is
// the same to the bit.  Slice s covers windows [s*W/S, (s+1)*W/S) of the
// W = ceil(K/256) windows.
__host__ __device__ constexpr int lds_windows(int k) { return (k + 255) >> 8; }
__host__ __device__ constexpr int lds_slices(int k) {
  return lds_windows(k) / 4 < 1 ? 1 : (lds_windows(k) / 4 > 3 ? 3 : lds_windows(k) / 4);
}

// Device-side control block of a launch that has an lm_head (argmax keys)
// or waits on stages.  It must be zero before the first launch; every
// launch leaves it zero again (the last workgroup out resets it), except
// `error`, which stays set once a stage wait timed out so the host can see it.
struct StreamCtl {
  unsigned exits;
  unsigned error;
  unsigned pad[2];
  unsigned long long keys[VG_MAX_M_DEV][kKeySlots];
};

// Stage completion counters of a step: each on its own 128-byte line --
// measured, polling and signalling adjacent counters on one line slows
// the whole step noticeably.  Zero between launches (reset by the last
// workgroup out).
constexpr int kDoneSlots = 8;  // counters per stage, one per XCD
struct alignas(128) StageCounter {
  unsigned v;
  unsigned pad[31];
};

struct StreamArgs {
  StreamJob job0;                // the job of a single-job launch (jobs == nullptr)
  const StreamJob* jobs;         // device array of a step's jobs (DIRECT: the njobs jobs of one stage)
  const unsigned* stage_total;   // device array: workgroups that signal each stage
  StageCounter (*stage_done)[kDoneSlots];  // [nstages][kDoneSlots]
  StreamCtl* ctl;                // control block (lm_head keys, exit count, error)
  int njobs;
  int nstages;
  int waits;                     // 1: honour stage dependencies (a step)
  int total_items;
  int M;                         // rows of every X
  int T;                         // lm_head rows per sequence
  int has_lmhead;
  const int32_t* drafts;         // [M/T][T-1]: tokens of nodes 1..T-1 of each sequence
  int32_t* argmax;               // [M]
  int32_t* accept_len;           // [M/T]
  const int32_t* parents;        // [M/T][T-1] parent of nodes 1..T-1 (a tree), or null (a chain)
  const int32_t* token_map;      // [V] token id of each lm_head row, or null (row index = id)
  int32_t* accept_node;          // [M/T] node whose argmax is the bonus token, or null
  int lm_rows;                   // V of the lm_head job (bounds the token_map lookup)
  int invariant;                 // 1: every M on the MFMA path (row results independent of M)
  int any_k;                     // a job list (jobs != nullptr) with a K that is not a multiple of 128
  float* part;                   // spread jobs: [slot][M][64] slice sums of a block
  unsigned* part_cnt;            // spread jobs: [slot] slices done of the block whose slice 0 is that slot
};

enum StreamMode { STREAM_DIRECT = 0, STREAM_GRID = 1, STREAM_STATIC = 2 };

// 0 for the M = 1 GEMV path, else the number of 16-row M-tiles.  A batch-
// invariant launch never takes the GEMV path (M = 1 runs as one M-tile).
int stream_mt_class(int M, bool invariant);
// Rows of a block of the LDS-shared MFMA item (M >= 2 or batch-invariant).
int stream_lds_rows(int M, bool invariant);
// Weight rows per item for a batch of M rows and a reduction length K.
int stream_rows_per_item(int M, int K, bool invariant, int fmt);
// DIRECT: grid = items of a.job0, or (M >= 2, jobs != nullptr) the items
// of the njobs jobs at a.jobs, one stage of a step.  GRID: a.job0 walked by up to `grid`
// resident workgroups.  STATIC: the job list of a step, items assigned
// round-robin to a grid of co-resident workgroups (at most `grid`).
hipError_t launch_stream(const StreamArgs& a, int mode, int grid, hipStream_t stream);
// The exact grid a STATIC launch of a batch of M rows uses (all resident).
int stream_static_grid(int M, bool invariant);
// An upper bound of stream_static_grid over every M on this device.
int stream_max_grid();
// Compute units of the current device (what several resident workgroups of
// one CU share: its memory bandwidth).
int stream_num_cus();

// M = 1: the whole step (or a single GEMM / lm_head) as one launch of
// step_gemv_grid() resident workgroups.  A multi-job launch (a.jobs) takes
// each job's rows per workgroup from its step fields (set_step_rows); a
// single job (a.job0) is split evenly over the grid here.
// Every job's K must satisfy step_gemv_supports (K % 64 == 0, K <= 18432);
// other M = 1 shapes take the stream kernel.
// A step launch holds at most kStepMaxJobs jobs (its job table lives in LDS).
constexpr int kStepMaxJobs = 512;
hipError_t launch_step_gemv(const StreamArgs& a, hipStream_t stream);
int step_gemv_grid();
bool step_gemv_supports(int K);

hipError_t launch_bwprobe(const void* buf, size_t bytes, float* sink, hipStream_t stream);
size_t bwprobe_sink_floats();

}  // namespace vg

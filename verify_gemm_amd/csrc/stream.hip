// Host side of the weight-streaming kernels for batches of M >= 2 rows:
// item sizes, grids and the dispatch to the kernel variant of a launch.
// The kernels themselves are in stream_kernel.h; each (M-tile class,
// weight format) pair is compiled in a translation unit of its own
// (stream_mt<MT>_f<FMT>.hip), declared here as explicit instantiations.
#include "stream_kernel.h"

namespace vg {

#define VG_EXTERN_MT(MT, FMT)                                                                   \
  extern template hipError_t launch_stream_mt<MT, FMT>(const StreamArgs&, int, int, hipStream_t); \
  extern template int stream_static_resident<MT, FMT>();
VG_EXTERN_MT(0, 0)
VG_EXTERN_MT(0, 1)
VG_EXTERN_MT(1, 0)
VG_EXTERN_MT(1, 1)
VG_EXTERN_MT(2, 0)
VG_EXTERN_MT(2, 1)
VG_EXTERN_MT(3, 0)
VG_EXTERN_MT(3, 1)
VG_EXTERN_MT(4, 0)
VG_EXTERN_MT(4, 1)
VG_EXTERN_MT(5, 0)
VG_EXTERN_MT(5, 1)
#undef VG_EXTERN_MT


int stream_mt_class(int M, bool invariant) { return M == 1 && !invariant ? 0 : (M + 15) / 16; }

int stream_lds_rows(int M, bool invariant) {
  switch (stream_mt_class(M, invariant)) {
    case 1: return Cfg<1>::Lds::kRows;
    case 2: return Cfg<2>::Lds::kRows;
    case 3: return Cfg<3>::Lds::kRows;
    case 4: return Cfg<4>::Lds::kRows;
    default: return Cfg<5>::Lds::kRows;
  }
}

int stream_rows_per_item(int M, int K, bool invariant, int fmt) {
  const int mt = stream_mt_class(M, invariant);
  if (mt == 0 && fmt == 1) return Fp8GemvItem::kRows;
  if (mt == 0) {
    if (K == 5120) return GemvItem<5, 4>::kRows;
    if (K == 17408) return GemvItem<17, 1>::kRows;
    if (K == 1024) return GemvItem<1, 8>::kRows;
    return GemvGenericItem::kRows;
  }
  if ((K & 127) == 0) return stream_lds_rows(M, invariant);  // the LDS-shared item, NVFP4 or FP8
  return 16 * (mt <= 2 ? 2 : 4);
}

int stream_static_grid(int M, bool invariant) {
  // All workgroups must be resident (the static schedule waits on them);
  // one per CU measured best except with two M-tiles, where two per CU
  // (the kernel's registers allow it) keep more items in flight.
  int cap = 0;
  switch (stream_mt_class(M, invariant)) {
    case 0: cap = stream_static_resident<0, 0>(); break;
    case 1: cap = stream_static_resident<1, 0>(); break;
    case 2: cap = stream_static_resident<2, 0>(); break;
    case 3: cap = stream_static_resident<3, 0>(); break;
    case 4: cap = stream_static_resident<4, 0>(); break;
    default: cap = stream_static_resident<5, 0>(); break;
  }
  const int want = (stream_mt_class(M, invariant) == 2 ? 2 : 1) * num_cus();
  return cap < want ? cap : want;
}

int stream_max_grid() { return 2 * num_cus(); }
int stream_num_cus() { return num_cus(); }

template <int MT>
hipError_t launch_mt(const StreamArgs& a, int mode, int grid, hipStream_t stream) {
  // the weight format of a launch is that of its (first) job: a step's jobs
  // are all NVFP4; FP8 comes only as single-job launches
  return a.job0.fmt == 1 ? launch_stream_mt<MT, 1>(a, mode, grid, stream)
                         : launch_stream_mt<MT, 0>(a, mode, grid, stream);
}

hipError_t launch_stream(const StreamArgs& a, int mode, int grid, hipStream_t stream) {
  switch (stream_mt_class(a.M, a.invariant != 0)) {
    case 0: return launch_mt<0>(a, mode, grid, stream);
    case 1: return launch_mt<1>(a, mode, grid, stream);
    case 2: return launch_mt<2>(a, mode, grid, stream);
    case 3: return launch_mt<3>(a, mode, grid, stream);
    case 4: return launch_mt<4>(a, mode, grid, stream);
    case 5: return launch_mt<5>(a, mode, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vg

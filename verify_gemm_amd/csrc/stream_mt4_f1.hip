// Kernel variants of M-tile class 4, weight format 1 (FP8): one
// translation unit per pair so that the variants compile in parallel.
#include "stream_kernel.h"

namespace vg {
template hipError_t launch_stream_mt<4, 1>(const StreamArgs&, int, int, hipStream_t);
template int stream_static_resident<4, 1>();
}  // namespace vg

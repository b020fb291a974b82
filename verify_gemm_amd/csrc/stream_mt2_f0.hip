// Kernel variants of M-tile class 2, weight format 0 (NVFP4): one
// translation unit per pair so that the variants compile in parallel.
#include "stream_kernel.h"

namespace vg {
template hipError_t launch_stream_mt<2, 0>(const StreamArgs&, int, int, hipStream_t);
template int stream_static_resident<2, 0>();
}  // namespace vg

// Streaming kernels for one element type (f32), stored logits as they are.
#include "stream_impl.h"

namespace vsce {
template int stream_dt<VSCE_F32, false>(int, const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

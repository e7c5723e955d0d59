// Streaming kernels for one element type (f32), soft-capped logits.
#include "stream_impl.h"

namespace vsce {
template int stream_dt<VSCE_F32, true>(int, const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

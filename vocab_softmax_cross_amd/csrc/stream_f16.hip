// Streaming kernels for one element type (f16), stored logits as they are.
#include "stream_impl.h"

namespace vsce {
template int stream_dt<VSCE_F16, false>(int, const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

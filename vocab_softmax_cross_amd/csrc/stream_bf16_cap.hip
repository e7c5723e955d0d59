// Streaming kernels for one element type (bf16), soft-capped logits.
#include "stream_impl.h"

namespace vsce {
template int stream_dt<VSCE_BF16, true>(int, const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

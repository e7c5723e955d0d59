// Resident fused kernels for one element type (bf16), stored logits as they are.
#include "fused_impl.h"

namespace vsce {
template int fused_resident_dt<VSCE_BF16, false>(const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

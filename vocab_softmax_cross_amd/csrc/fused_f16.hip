// Resident fused kernels for one element type (f16), stored logits as they are.
#include "fused_impl.h"

namespace vsce {
template int fused_resident_dt<VSCE_F16, false>(const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

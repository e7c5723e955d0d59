// Resident fused kernels for one element type (f32), stored logits as they are.
#include "fused_impl.h"

namespace vsce {
template int fused_resident_dt<VSCE_F32, false>(const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

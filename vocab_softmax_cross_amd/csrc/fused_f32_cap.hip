// Resident fused kernels for one element type (f32), soft-capped logits.
#include "fused_impl.h"

namespace vsce {
template int fused_resident_dt<VSCE_F32, true>(const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

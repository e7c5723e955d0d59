// Resident fused kernels for one element type (bf16).
#include "fused_impl.h"

namespace vsce {
template int fused_resident_dt<VSCE_BF16>(const Prob&, const RowArgs&, hipStream_t);
}  // namespace vsce

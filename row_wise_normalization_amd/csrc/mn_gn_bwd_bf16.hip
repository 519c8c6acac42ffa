// GroupNorm backward launchers for bf16 activations (bf16 or f32 dX).
#include "mn_gn_instances.hpp"

namespace mn {
template hipError_t launch_gn_bwd_t<ST_BF16, ST_BF16>(const GnPlan&, const GnArgs&, hipStream_t);
template hipError_t launch_gn_bwd_t<ST_BF16, ST_F32>(const GnPlan&, const GnArgs&, hipStream_t);
}  // namespace mn

// GroupNorm backward launchers for f16 activations (f16 or f32 dX).
#include "mn_gn_instances.hpp"

namespace mn {
template hipError_t launch_gn_bwd_t<ST_F16, ST_F16>(const GnPlan&, const GnArgs&, hipStream_t);
template hipError_t launch_gn_bwd_t<ST_F16, ST_F32>(const GnPlan&, const GnArgs&, hipStream_t);
}  // namespace mn

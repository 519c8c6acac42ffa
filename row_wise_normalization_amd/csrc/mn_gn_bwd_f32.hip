// GroupNorm backward launchers for f32 activations.
#include "mn_gn_instances.hpp"

namespace mn {
template hipError_t launch_gn_bwd_t<ST_F32, ST_F32>(const GnPlan&, const GnArgs&, hipStream_t);
}  // namespace mn

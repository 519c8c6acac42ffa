// GroupNorm forward launchers for bf16 activations.
#include "mn_gn_instances.hpp"

namespace mn {
template hipError_t launch_gn_fwd_t<ST_BF16>(const GnPlan&, const GnArgs&, hipStream_t);
}  // namespace mn

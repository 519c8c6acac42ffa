// Kernel instances for binary16 activations.
#define MN_INST_ST ST_F16
#define MN_INST_BWD_TYPES MN_BWD_TYPES_F16
#include "mn_instances.hpp"

// Kernel instances for bfloat16 activations.
#define MN_INST_ST ST_BF16
#define MN_INST_BWD_TYPES MN_BWD_TYPES_BF16
#include "mn_instances.hpp"

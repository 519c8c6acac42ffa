// Kernel instances for binary32 activations.
#define MN_INST_ST ST_F32
#define MN_INST_BWD_TYPES MN_BWD_TYPES_F32
#include "mn_instances.hpp"

// Kernel instances of the training pair (RMSNorm, LayerNorm, fused add +
// RMSNorm) for binary32 activations.
#define MN_INST_ST ST_F32
#define MN_INST_KINDS(X) X(RMS) X(LN) X(ADD)
#define MN_INST_KINDS_BWD(X, S, C, O) X(RMS, S, C, O) X(LN, S, C, O) X(ADD, S, C, O)
#define MN_INST_BWD_TYPES MN_BWD_TYPES_F32
#include "mn_instances.hpp"

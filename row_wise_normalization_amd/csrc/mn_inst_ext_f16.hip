// Kernel instances of the other row-wise norms (Dynamic Tanh, PolyNorm,
// Modulated RMSNorm) for binary16 activations.
#define MN_INST_ST ST_F16
#define MN_INST_KINDS(X) X(DYT) X(POLY) X(MOD)
#define MN_INST_KINDS_BWD(X, S, C, O) X(DYT, S, C, O) X(POLY, S, C, O) X(MOD, S, C, O)
#define MN_INST_BWD_TYPES MN_BWD_TYPES_EXT_F16
#include "mn_instances.hpp"

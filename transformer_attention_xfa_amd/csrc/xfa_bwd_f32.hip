// The fp32 backward kernels: the kernels of xfa_bwd.hip instantiated for
// float in a translation unit of their own, compiled with the default
// placement of matrix-core results (see xfa_bwd.hip's launch code).
#define XFA_BWD_F32
#include "xfa_bwd.hip"

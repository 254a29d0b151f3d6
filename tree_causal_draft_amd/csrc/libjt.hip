// All device code of libjt in one translation unit: the fused step (step.hip) runs the
// device functions of every step, and the library is built without relocatable device
// code.  Each included file keeps its own kernels and host launcher.
#include "mask.hip"
#include "topw.hip"
#include "verify.hip"
#include "sample.hip"
#include "attn.hip"
#include "step.hip"
#include "step_static.hip"
#include "tree.hip"
#include "commit.hip"
#include "probe.hip"

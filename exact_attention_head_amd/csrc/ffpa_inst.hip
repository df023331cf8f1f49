// One explicit instantiation of the forward launcher (and with it the kernel).  The build
// compiles this file once per (element type, head dim) with -DFFPA_INST_T=... -DFFPA_INST_D=...
#include "ffpa_kernel.hpp"
#include "ffpa_launch.hpp"

#if !defined(FFPA_INST_T) || !defined(FFPA_INST_D)
#error "compile with -DFFPA_INST_T=Bf16|Fp16 -DFFPA_INST_D=<head dim>"
#endif

namespace ffpa {
template hipError_t launch_fwd<FFPA_INST_T, FFPA_INST_D>(const FwdArgs&, hipStream_t);
}

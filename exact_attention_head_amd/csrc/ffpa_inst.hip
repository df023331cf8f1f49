// Explicit instantiations of the forward launchers (and with them the kernels).  The build compiles
// this file per (element type, head dim, part) with -DFFPA_INST_T=... -DFFPA_INST_D=... -DFFPA_INST_PART=...
#include "ffpa_kernel.hpp"
#include "ffpa_launch.hpp"

#if !defined(FFPA_INST_T) || !defined(FFPA_INST_D)
#error "compile with -DFFPA_INST_T=Bf16|Fp16 -DFFPA_INST_D=<head dim>"
#endif

// FFPA_INST_PART selects the group: 0 the launcher with the plain and runtime-layout variants, 1 the
// dropout variants, 2 the staged-mask variants.
#if !defined(FFPA_INST_PART) || FFPA_INST_PART == 0
namespace ffpa {
template hipError_t launch_fwd<FFPA_INST_T, FFPA_INST_D>(const FwdArgs&, hipStream_t);
}
#elif FFPA_INST_PART == 1
namespace ffpa {
template hipError_t launch_fwd_drop<FFPA_INST_T, FFPA_INST_D>(const FwdArgs&, hipStream_t, long long, bool);
}
#elif FFPA_INST_PART == 2
namespace ffpa {
template hipError_t launch_fwd_staged<FFPA_INST_T, FFPA_INST_D>(const FwdArgs&, hipStream_t, long long, bool);
}
#else
#error "FFPA_INST_PART must be 0, 1 or 2"
#endif

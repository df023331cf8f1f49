// Explicit instantiations of the fp8 forward launchers (and with them the kernels), one translation unit
// per head dim: the build compiles this file with -DFFPA_FP8_D=<128|256|384|512>.
#include "ffpa_kernel.hpp"
#include "ffpa_fp8_kernel.hpp"
#include "ffpa_launch.hpp"

#if !defined(FFPA_FP8_D)
#error "compile with -DFFPA_FP8_D=<head dim>"
#endif

namespace ffpa {
template hipError_t launch_fwd_fp8<Bf16, FFPA_FP8_D>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_fp8<Fp16, FFPA_FP8_D>(const FwdArgs&, hipStream_t);
}  // namespace ffpa

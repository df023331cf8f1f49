// Explicit instantiations of the fused backward's launchers (and with them its kernels), one
// translation unit per kernel head dim: the build compiles this file with -DFFPA_BWD_KD=<head dim>
// and -DFFPA_BWD_PAD=0 (head dim D = KD) or 1 (D < KD, the columns from D on skipped).
#include "ffpa_kernel.hpp"
#include "ffpa_bwd_kernel.hpp"

#if !defined(FFPA_BWD_KD) || !defined(FFPA_BWD_PAD)
#error "compile with -DFFPA_BWD_KD=<kernel head dim> -DFFPA_BWD_PAD=0|1"
#endif

namespace ffpa {
template hipError_t launch_bwd_fused<Bf16, FFPA_BWD_KD, (FFPA_BWD_PAD != 0)>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_fused<Fp16, FFPA_BWD_KD, (FFPA_BWD_PAD != 0)>(const BwdArgs&, hipStream_t);
}  // namespace ffpa

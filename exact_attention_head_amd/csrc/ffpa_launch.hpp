// Launchers of the forward kernels, one per (element type, head dim).  They are explicitly
// instantiated in the ffpa_inst_*.hip files so the kernels compile in parallel.
#pragma once

#include <hip/hip_runtime.h>

namespace ffpa {

struct FwdArgs;
struct Bf16;
struct Fp16;

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
template <typename T, int D>
hipError_t launch_fwd_drop(const FwdArgs& a, hipStream_t stream, long long blocks, bool plain);
template <typename T, int D>
hipError_t launch_fwd_staged(const FwdArgs& a, hipStream_t stream, long long blocks, bool bool_mask);

// Head dims with a compiled kernel (the row kernel's); every other multiple of 8 up to 1024 runs the
// next of these with padding columns.
#define FFPA_FOR_EACH_D(X) \
  X(64) X(128) X(192) X(256) X(320) X(384) X(448) X(512) X(640) X(768) X(896) X(1024)

// fp8 forward: launchers per output element type and head dim (128, 256, 384, 512, 768, 1024; other
// multiples of 16 run the next one up with padding columns).
template <typename T, int D>
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream);
#define FFPA_FP8_FOR_EACH_D(X) X(128) X(256) X(384) X(512) X(768) X(1024)
#define FFPA_FP8_DECLARE(Dv)                                                          \
  extern template hipError_t launch_fwd_fp8<Bf16, Dv>(const FwdArgs&, hipStream_t); \
  extern template hipError_t launch_fwd_fp8<Fp16, Dv>(const FwdArgs&, hipStream_t);
FFPA_FP8_FOR_EACH_D(FFPA_FP8_DECLARE)
#undef FFPA_FP8_DECLARE

#define FFPA_DECLARE(Dv)                                                                                      \
  extern template hipError_t launch_fwd<Bf16, Dv>(const FwdArgs&, hipStream_t);                               \
  extern template hipError_t launch_fwd<Fp16, Dv>(const FwdArgs&, hipStream_t);                               \
  extern template hipError_t launch_fwd_drop<Bf16, Dv>(const FwdArgs&, hipStream_t, long long, bool);         \
  extern template hipError_t launch_fwd_drop<Fp16, Dv>(const FwdArgs&, hipStream_t, long long, bool);         \
  extern template hipError_t launch_fwd_staged<Bf16, Dv>(const FwdArgs&, hipStream_t, long long, bool);       \
  extern template hipError_t launch_fwd_staged<Fp16, Dv>(const FwdArgs&, hipStream_t, long long, bool);
FFPA_FOR_EACH_D(FFPA_DECLARE)
#undef FFPA_DECLARE

}  // namespace ffpa

// Launchers of the fused backward, one per (element type, kernel head dim, padding), explicitly
// instantiated in ffpa_bwd_inst.hip (one translation unit per kernel head dim), and their arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffpa {

struct Bf16;
struct Fp16;

// Arguments of the fused backward (one struct for both passes).
struct BwdArgs {
  const uint16_t* q;     // [B, Hq, Nq, D]
  const uint16_t* k;     // [B, Hkv, Nkv, D]
  const uint16_t* v;     // [B, Hkv, Nkv, D]
  const uint16_t* dout;  // [B, Hq, Nq, D]
  const float* lse;      // [B, Hq, Nq] natural-log LSE of the forward
  const float* delta;    // [B, Hq, Nq] rowsum(dO * O)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const void* mask;  // bias of (b, h, r, k) at b * msb + h * msh + r * msq + k
  int mask_kind;
  long long msb, msh, msq;
  float* dmask;  // null, or the mask's gradient: dense fp32 [Bm, Hm, Nqm, Nkv], zeroed beforehand
  int dm_bb, dm_bh, dm_bq;  // broadcast over batch / heads / rows (index 0 there)
  int dm_hm, dm_nqm;        // Hm, Nqm
  int dm_atomic;            // several (b, h, r) add into one element
  const uint32_t* keep;     // dropout keep words [B, Hq, Nq, keep_w] (null: none)
  int keep_w;
  float drop_scale;  // 1 / (1 - p)
  int B, Hq, Hkv, Nq, Nkv, D;
  float scale;
  int causal;
};

// The kernel head dim serving head dim D (D % 8 == 0): the smallest of 64, 128, ..., 512, 640, 768,
// 896, 1024 that is at least D (a multiple of 64 up to 512 is its own; 576 -> 640, 704 -> 768,
// 832 -> 896, 960 -> 1024).
constexpr int bwd_kernel_dim(int D) {
  return D <= 512 ? (D + 63) / 64 * 64 : (D <= 640 ? 640 : (D <= 768 ? 768 : (D <= 896 ? 896 : 1024)));
}

// PAD: D < KD, the columns from D on skipped.
template <typename T, int KD, bool PAD>
hipError_t launch_bwd_fused(const BwdArgs& a, hipStream_t stream);
#define FFPA_BWD_FOR_EACH_KD(X) X(64) X(128) X(192) X(256) X(320) X(384) X(448) X(512) X(640) X(768) X(896) X(1024)
#define FFPA_BWD_PAD_KD(X) X(64) X(128) X(192) X(256) X(320) X(384) X(448) X(512) X(640) X(768) X(896) X(1024)
#define FFPA_BWD_DECLARE(KDv)                                                             \
  extern template hipError_t launch_bwd_fused<Bf16, KDv, false>(const BwdArgs&, hipStream_t); \
  extern template hipError_t launch_bwd_fused<Fp16, KDv, false>(const BwdArgs&, hipStream_t);
FFPA_BWD_FOR_EACH_KD(FFPA_BWD_DECLARE)
#undef FFPA_BWD_DECLARE
#define FFPA_BWD_DECLARE_PAD(KDv)                                                        \
  extern template hipError_t launch_bwd_fused<Bf16, KDv, true>(const BwdArgs&, hipStream_t); \
  extern template hipError_t launch_bwd_fused<Fp16, KDv, true>(const BwdArgs&, hipStream_t);
FFPA_BWD_PAD_KD(FFPA_BWD_DECLARE_PAD)
#undef FFPA_BWD_DECLARE_PAD

}  // namespace ffpa

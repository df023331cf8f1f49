// Exact large-head-dim attention forward for gfx950 (MI355X, CDNA4): shared definitions (argument
// block, matrix-core wrappers, logit and mask helpers, the staged O store), the launcher, and the
// shared-staging kernel compiled for the head dims the row-owner kernel (ffpa_row_kernel.hpp: 64,
// 128, 192, ..., 512, 640, 768, 896, 1024) does not take: the multiples of 64 above 512 whose half is
// an odd number of 32-column steps (576, 704, 832, 960).  It serves them with dropout only; without
// it the row kernel of the next head dim runs them padded, several times faster.
//
// Shared-staging kernel.  One workgroup = 4 wave64s = one (batch, query head, tile of BR query rows).
// It loops over the keys in tiles of BC = 64 and keeps an online softmax, as
// in the FlashAttention-2 scheme the older FFPA page builds on
// (sourcepulse page, "How It Works").  The large-D design follows the two
// ideas of the ffpa-attn README, section "Split-D and TiledMMA", rebuilt for
// CDNA4:
//
//  * Split-D (LDS footprint independent of D).  K and V, and for D > 512
//    also Q, reach the MFMA units through LDS in 32-column chunks of the
//    head dimension, in a three-slot ring filled by direct-to-LDS
//    global_load_lds_dwordx4 and prefetched two chunks ahead.  For D <= 512
//    the query tile is instead kept in VGPRs for the whole key loop (it is
//    private to each wave, so staging it through LDS on every tile would only
//    cost L2 and LDS bandwidth).
//
//  * Output-D split (the M4N2 / "TiledMMA" idea).  The fp32 O accumulator of
//    BR rows x D columns does not fit one wave at large D, so the 4 waves are
//    arranged as RG row groups x DG column groups: wave (rg, dg) owns rows
//    rg*R .. rg*R+R-1 and output columns dg*DW .. dg*DW+DW-1 (DW = D/DG).
//    The same split is used for S = Q K^T: each wave forms the partial dot
//    products over its own DW columns, and the DG partials of a row group are
//    summed through LDS in a fixed order, so every wave of the group holds a
//    bit-identical S tile and runs the same softmax.
//
// Matrix-core layout.  Both products use v_mfma_f32_32x32x16_{bf16,f16}.
// S is formed transposed, S^T = K Q^T, so lane l holds query row l%32 and 16
// keys of a 32-key block; O is formed transposed too, O^T = V^T P^T, so lane
// l again holds row l%32.  Row statistics are therefore lane-local and only
// need one cross-half exchange (v_permlane32_swap).  The S accumulator,
// rounded to bf16/fp16, is directly the P^T operand of the second product:
// the key order it implies is matched by reading V through ds_read_b64_tr_b16
// with the same key permutation (the sum over keys does not care about
// order).
//
// Softmax.  Logits are kept in the log2 domain, t = s * scale * log2(e) +
// bias * log2(e), and exponentiated with v_exp_f32.  The running row maximum
// is only moved (and O, l rescaled) when it grows by more than 8, so P stays
// below 2^8 and the O rescale, a pass over up to 256 accumulator registers,
// is skipped on almost every tile; the final O/l and LSE use whichever
// maximum was kept, which is exact algebra.  Fully excluded rows keep
// m = -inf, l = 0 and produce O = 0, LSE = -inf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffpa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned char u8x4 __attribute__((ext_vector_type(4)));

#define FFPA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// The running maximum is moved only when a row's maximum grows by more than this (log2 units).
constexpr float kRescaleSlack = 8.0f;

enum MaskKind { kMaskNone = 0, kMaskBoolU8 = 1, kMaskAddF32 = 2, kMaskAddBf16 = 3, kMaskAddFp16 = 4 };

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const void* mask;
  int64_t msb, msh, msq;  // mask strides in elements; the key stride is 1
  int mask_kind;
  int mask_vec;           // 1: strides and base allow 4-wide vector loads
  int B, Hq, Hkv, Nq, Nkv, group;
  float scale_log2;       // scale * log2(e)
  int causal;
  // Packed variable-length batch (null cu_q: the dense [B, H, N, D] layout).  Q/O are [Tq, Hq, D]
  // and K/V [Tk, Hkv, D]; sequence b holds query tokens cu_q[b] .. cu_q[b+1]-1 and key tokens
  // cu_k[b] .. cu_k[b+1]-1; Nq and Nkv above are then the longest lengths (they size the grid);
  // LSE is [Hq, Tq].
  const int32_t* cu_q;
  const int32_t* cu_k;
  int Tq, Tk;
  // Element strides (batch, head, row; the head-dim stride is 1) of Q, of K and V, and of O.  The
  // contiguous dense variants of the row kernel use their compile-time equivalents instead; a
  // packed batch has no batch stride (its sequences start at the offsets above).
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
  int q_sr, kv_sr, o_sr;
  int strided;  // 1: the dense layout is not contiguous (the runtime-layout variants serve it)
  // Head dim of the tensors.  Below the kernel's compile-time D (a multiple of 8 served by the next
  // compiled head dim, runtime-layout variants only) the columns from dcols on are padding: Q reads
  // zeros there, so K's padding columns add nothing to S, and O is stored up to dcols only.
  int dcols;
  // fp8 forward (ffpa_fwd_fp8): per-head dequantisation factors [B, Hq] and [B, Hkv] (null: 1); q, k, v
  // then point at e4m3 bytes, and the row strides count bytes
  const float* q_desc;
  const float* k_desc;
  const float* v_desc;
  // Measurement aid (null: off): the first wave of workgroup 0 records the shader-clock counter and the
  // 100 MHz real-time counter at its start (stamps[0], stamps[1]) and end (stamps[2], stamps[3]).
  unsigned long long* stamps;
  // Attention dropout (null keep: none; dense contiguous layout only).  keep is [B, Hq, Nq, keep_w]
  // 32-bit words: bit i of word w set keeps the weight of key 32 w + i for that query row; kept
  // weights are scaled by drop_scale = 1 / (1 - p) (applied to O with the 1/l normalisation).
  const uint32_t* keep;
  int keep_w;
  float drop_scale;
};

// Tokens of sequence b of a packed batch.  The offsets are clamped to the packed tensors and the
// lengths to the longest lengths, so that malformed offsets can change results but never move an
// access outside the tensors (the C ABI documents the well-formed case).
struct SeqRange {
  int q0, nq, k0, nkv;
};
__device__ inline SeqRange seq_range(const FwdArgs& a, int b) {
  auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
  const int q0 = clampi(a.cu_q[b], 0, a.Tq), q1 = clampi(a.cu_q[b + 1], q0, a.Tq);
  const int k0 = clampi(a.cu_k[b], 0, a.Tk), k1 = clampi(a.cu_k[b + 1], k0, a.Tk);
  const int nq = q1 - q0 < a.Nq ? q1 - q0 : a.Nq;
  const int nkv = k1 - k0 < a.Nkv ? k1 - k0 : a.Nkv;
  return SeqRange{q0, nq, k0, nkv};
}

struct Bf16 {};
struct Fp16 {};

template <typename T>
struct Elem;

// Matrix-core products are written as inline assembly so that each accumulator lives in the
// register file chosen for it: the O accumulators (up to 256 registers at D = 1024) in AGPRs, the
// S tile in VGPRs.  (Through the builtins the compiler puts every MFMA result in one class, and
// O + S do not fit either class alone.)  The compiler does not see into inline assembly, so the
// wait states it would insert are provided here:
//  * an operand written by a VALU instruction needs 2 wait states before an MFMA reads it: the
//    products whose operands come from VALU code (P, rescaled O) start with s_nop 1;
//  * a chain's first product takes srcC = 0 instead of zeroed registers;
//  * an MFMA result needs 12 wait states before a VALU, LDS or memory instruction reads it: every
//    such read is preceded by mma_guard(), which carries a dependency on the accumulators.
// Back-to-back products accumulating into the same registers need none.
#define FFPA_DEFINE_MMA(TAG, INSN)                                                                         \
  template <>                                                                                                 \
  struct Elem<TAG> {                                                                                          \
    /* d = a*b, d in VGPRs; a from VGPRs, b from VGPRs (BA=false) or AGPRs (BA=true) */                     \
    __device__ static inline void mma_first(f32x16& d, const i32x4& a, const i32x4& b) {                     \
      asm volatile(INSN " %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));                                                 \
    }                                                                                                         \
    __device__ static inline void mma_first_ba(f32x16& d, const i32x4& a, const i32x4& b) {                  \
      asm volatile(INSN " %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));                                                 \
    }                                                                                                         \
    __device__ static inline void mma_acc(f32x16& d, const i32x4& a, const i32x4& b) {                       \
      asm volatile(INSN " %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));                                                 \
    }                                                                                                         \
    __device__ static inline void mma_acc_ba(f32x16& d, const i32x4& a, const i32x4& b) {                    \
      asm volatile(INSN " %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));                                                 \
    }                                                                                                         \
    /* d += a*b with d in AGPRs and VALU-written operands */                                                  \
    __device__ static inline void mma_acc_agpr(f32x16& d, const i32x4& a, const i32x4& b) {                  \
      asm volatile("s_nop 1\n\t" INSN " %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));                                 \
    }                                                                                                         \
    /* d += a*b with d in AGPRs, operands not written by VALU instructions in the last 2 wait states */     \
    __device__ static inline void mma_acc_agpr_nonop(f32x16& d, const i32x4& a, const i32x4& b) {            \
      asm volatile(INSN " %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));                                                 \
    }                                                                                                         \
  };
FFPA_DEFINE_MMA(Bf16, "v_mfma_f32_32x32x16_bf16")
FFPA_DEFINE_MMA(Fp16, "v_mfma_f32_32x32x16_f16")
#undef FFPA_DEFINE_MMA

// Conversions of two floats to two round-to-nearest-even 16-bit values in one dword (low first).
template <typename T>
__device__ inline uint32_t pack2(float lo, float hi);
template <>
__device__ inline uint32_t pack2<Bf16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
template <>
__device__ inline uint32_t pack2<Fp16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
__device__ inline float widen_bf16(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }
__device__ inline float widen_fp16(uint16_t bits) { return (float)__builtin_bit_cast(_Float16, bits); }

// 12 wait states between the MFMAs that wrote these accumulators and any later reader: the tied
// operands order the nops after the producers and before the readers.
template <int RB>
__device__ inline void mma_guard_v(f32x16 (&x)[RB][2]) {
  if constexpr (RB == 1) {
    asm volatile("s_nop 7\n\ts_nop 4" : "+v"(x[0][0]), "+v"(x[0][1]));
  } else {
    static_assert(RB == 2, "one or two row blocks");
    asm volatile("s_nop 7\n\ts_nop 4" : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]));
  }
}
__device__ inline void mma_guard_a(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 4" : "+a"(x)); }
// 12+ wait states after the MFMAs that wrote every accumulator of o, in one nop sequence (all
// accumulators are tied operands of the same statement, so no producer can fall after the nops
// and no reader before them).
template <int N>
__device__ inline void mma_guard_all(f32x16* o);
template <>
__device__ inline void mma_guard_all<1>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]));
}
template <>
__device__ inline void mma_guard_all<2>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]));
}
template <>
__device__ inline void mma_guard_all<3>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]));
}
template <>
__device__ inline void mma_guard_all<4>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}
template <>
__device__ inline void mma_guard_all<5>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]));
}
template <>
__device__ inline void mma_guard_all<6>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]));
}
template <>
__device__ inline void mma_guard_all<7>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]));
}
template <>
__device__ inline void mma_guard_all<8>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]));
}
template <>
__device__ inline void mma_guard_all<9>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]));
}
template <>
__device__ inline void mma_guard_all<10>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]));
}
template <>
__device__ inline void mma_guard_all<11>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]));
}
template <>
__device__ inline void mma_guard_all<12>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]));
}
template <>
__device__ inline void mma_guard_all<13>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]));
}
template <>
__device__ inline void mma_guard_all<14>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]));
}
template <>
__device__ inline void mma_guard_all<15>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]));
}
template <>
__device__ inline void mma_guard_all<16>(f32x16* o) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]), "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]), "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]), "+a"(o[15]));
}

// ---------------------------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------------------------

// Clock stamps of the measurement aid (FwdArgs::stamps): first wave of workgroup 0 only.
__device__ inline void clock_stamp(unsigned long long* stamps, int at) {
  if (stamps != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
    const unsigned long long c = __builtin_amdgcn_s_memtime();
    const unsigned long long r = __builtin_amdgcn_s_memrealtime();
    stamps[2 * at] = c;
    stamps[2 * at + 1] = r;
  }
}

// Bytes of one wave's O staging area: 32 rows of DW 16-bit columns, rows padded by 16 bytes.
template <int DW>
constexpr int o_stage_bytes() {
  return 32 * (2 * DW + 16);
}

// Epilogue store of a wave's O block (the "collective stores" of the sourcepulse page, "How It
// Works"): the NB accumulators (32 rows x 32 columns each; lane l holds row l % 32, element i column
// 8 (i / 4) + 4 (l / 32) + i % 4 of its block) are scaled by this lane's inv, rounded, written to the
// wave's LDS area `stage` and read back so that each store instruction writes whole rows, 16
// contiguous bytes per lane.  Rows from nrows on and columns from ncols on are not stored.  The caller
// has made the LDS area free (no wave reads it any more) and waited for the accumulators.
template <typename T, int DW, int NB, bool OPAQUE_LANE = true>
__device__ inline void store_o_staged(const f32x16* o_acc, float inv, char* stage, uint16_t* orow0, int64_t o_rs,
                                      int nrows, int ncols, int lane) {
  static_assert(NB * 32 == DW, "one accumulator per 32 columns");
  constexpr int PITCH = 2 * DW + 16;
  // opaque: keeps the lane's staging addresses from being formed before the key loop (where they
  // would hold registers throughout); which variants need it is read from the build's register figures
  if constexpr (OPAQUE_LANE) asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, hi = lane >> 5;
  FFPA_LDS char* st = (FFPA_LDS char*)stage;
#pragma unroll
  for (int s = 0; s < NB; ++s) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      i32x2 w;
      w[0] = (int)pack2<T>(o_acc[s][q4 * 4 + 0] * inv, o_acc[s][q4 * 4 + 1] * inv);
      w[1] = (int)pack2<T>(o_acc[s][q4 * 4 + 2] * inv, o_acc[s][q4 * 4 + 3] * inv);
      *(FFPA_LDS i32x2*)(st + l32 * PITCH + (s * 32 + q4 * 8 + hi * 4) * 2) = w;
    }
    __builtin_amdgcn_sched_barrier(0);  // one column block at a time: few registers in flight
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int ROWB = 2 * DW;          // bytes of one row
  constexpr int NI = 32 * ROWB / 1024;  // store instructions (1 KiB each)
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int off = i * 1024 + 16 * lane;
    const int r = off / ROWB, cb = off % ROWB;
    const i32x4 x = *(FFPA_LDS const i32x4*)(st + r * PITCH + cb);
    if (r < nrows && cb / 2 < ncols) *(i32x4*)(orow0 + (int64_t)r * o_rs + cb / 2) = x;
    if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // four rows of reads in flight at a time
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding.  Loads retire in
// order, so this also completes every load issued before the last N.
template <int N>
__device__ inline void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that also completes this wave's outstanding LDS operations first.  The
// memory clobbers keep the compiler from moving LDS accesses across it.
__device__ inline void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane t's bytes land at lds_wave_base + 16*t.
__device__ inline void load_lds16(const void* gsrc, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (FFPA_LDS void*)lds_wave_base, 16, 0, 0);
}

__device__ inline i32x4 lds_read16(const char* p) { return *(const FFPA_LDS i32x4*)(FFPA_LDS const char*)p; }

__device__ inline s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FFPA_LDS s16x4*)(FFPA_LDS const char*)p);
}

// The same transposed read as inline assembly.  Through the builtin the compiler cannot tell the
// read from the in-flight direct-to-LDS loads and waits for all of them (vmcnt(0)) first, which
// would drain the prefetch ring on every use.  The result is only valid after lds_frag_wait().
template <int OFF>
__device__ inline i32x2 lds_read_tr_async(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  i32x2 d;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF) : "memory");
  return d;
}
// The byte form: 16 lanes read 8 rows x 16 bytes (two 8-byte halves per row); lane i of the group
// receives column i of the 8 rows, row j in byte j (lane x addresses row x / 2, half x % 2).
template <int OFF>
__device__ inline i32x2 lds_read_tr8_async(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  i32x2 d;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF) : "memory");
  return d;
}
__device__ inline uint32_t lds_addr(const char* p) { return (uint32_t)(uintptr_t)(FFPA_LDS const char*)p; }

// Completes this wave's LDS reads; the tied operands keep every use of the fragments after it.
__device__ inline void lds_frag_wait(i32x4 (&f)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3])::"memory");
}

// value of the lane in the other 32-lane half
__device__ inline float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __builtin_fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// LDS tiles hold rows of 32 elements (64 bytes = four 16-byte chunks).  Chunk c of row r is stored
// at position c ^ ((r >> 2) & 3): the 16 rows read by 16 lanes of one MFMA-operand read (same
// chunk) then hit 16 distinct bank groups, and so do the 4 rows x 4 chunks of a transposed read.
__device__ inline int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }


// ---------------------------------------------------------------------------------------------
// Logits of one 64-key tile: t = s * scale * log2(e) + bias * log2(e), excluded keys -> -inf, and
// the per-row maximum (lane-local, before the cross-half exchange).
// ---------------------------------------------------------------------------------------------

struct LogitCtx {
  const void* mask;
  int64_t mask_bh;  // offset of (b, h) in the mask
  int64_t msq;      // mask row stride
  int Nq, Nkv, key0, rw0, off, causal;
  bool edge;        // tile touches the key tail or the causal diagonal: test every entry
  float scale_log2;
  int l32, hi;
};

template <int KIND>
__device__ inline float mask_bias(const void* m, int64_t i) {
  if constexpr (KIND == kMaskAddF32) return ((const float*)m)[i];
  else if constexpr (KIND == kMaskBoolU8) return ((const unsigned char*)m)[i] ? 0.f : kNegInf;
  else if constexpr (KIND == kMaskAddBf16) return widen_bf16(((const uint16_t*)m)[i]);
  else return widen_fp16(((const uint16_t*)m)[i]);
}

// Four consecutive keys starting at i (i a multiple of 4, aligned storage).
template <int KIND>
__device__ inline f32x4 mask_bias4(const void* m, int64_t i) {
  f32x4 r;
  if constexpr (KIND == kMaskAddF32) {
    r = *(const f32x4*)((const float*)m + i);
  } else if constexpr (KIND == kMaskBoolU8) {
    const u8x4 x = *(const u8x4*)((const unsigned char*)m + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = x[e] ? 0.f : kNegInf;
  } else {
    const i32x2 x = *(const i32x2*)((const uint16_t*)m + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t bits = (uint16_t)((uint32_t)x[e >> 1] >> (16 * (e & 1)));
      r[e] = KIND == kMaskAddBf16 ? widen_bf16(bits) : widen_fp16(bits);
    }
  }
  return r;
}

// Logits of NQ groups of 4 keys per row block.  Group g of this lane covers keys
// kbase + 8g + 4*hi + (0..3) (the S^T accumulator layout); t holds the raw dot products on entry
// and the log2-domain logits on exit; mx receives the lane-local row maxima.
template <int KIND, bool VEC, int RB, int NQ>
__device__ inline void logits(f32x4 (&t)[RB][NQ], float (&mx)[RB], const LogitCtx& c, int kbase) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = c.rw0 + rb * 32 + c.l32;
    int mrow = row < c.Nq ? row : c.Nq - 1;
    // Opaque per tile: keeps the compiler from hoisting one 64-bit mask address per mask variant
    // out of the key loop (they would stay live across it and spill).
    asm volatile("" : "+v"(mrow));
    const int64_t mo = c.mask_bh + (int64_t)mrow * c.msq;
    float m = kNegInf;
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const int kk = kbase + g * 8 + c.hi * 4;  // first of this lane's 4 consecutive keys
      f32x4 x = t[rb][g] * c.scale_log2;
      if constexpr (KIND != kMaskNone) {
        f32x4 bias;
        if constexpr (VEC) {
          bias = mask_bias4<KIND>(c.mask, mo + kk);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) bias[e] = kk + e < c.Nkv ? mask_bias<KIND>(c.mask, mo + kk + e) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(bias[e], kLog2e, x[e]);
      }
      if (c.edge) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool dead = kk + e >= c.Nkv || (c.causal && kk + e > row + c.off);
          x[e] = dead ? kNegInf : x[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) m = __builtin_fmaxf(m, x[e]);
      t[rb][g] = x;
    }
    mx[rb] = m;
  }
}

// Raw mask biases for NQ groups of 4 keys per row block (same lane layout as logits()); excluded
// boolean entries and keys past Nkv give -inf / 0 respectively.
template <int KIND, bool VEC, int RB, int NQ>
__device__ inline void load_bias(f32x4 (&bias)[RB][NQ], const LogitCtx& c, int kbase) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = c.rw0 + rb * 32 + c.l32;
    int mrow = row < c.Nq ? row : c.Nq - 1;
    asm volatile("" : "+v"(mrow));
    const int64_t mo = c.mask_bh + (int64_t)mrow * c.msq;
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const int kk = kbase + g * 8 + c.hi * 4;
      if constexpr (VEC) {
        bias[rb][g] = mask_bias4<KIND>(c.mask, mo + kk);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[rb][g][e] = kk + e < c.Nkv ? mask_bias<KIND>(c.mask, mo + kk + e) : 0.f;
      }
    }
  }
}

template <int RB, int NQ>
__device__ inline void load_bias_dispatch(f32x4 (&bias)[RB][NQ], const LogitCtx& c, int kbase, int kind, bool vec) {
  switch (kind) {
    case kMaskBoolU8:
      if (vec) load_bias<kMaskBoolU8, true, RB, NQ>(bias, c, kbase);
      else load_bias<kMaskBoolU8, false, RB, NQ>(bias, c, kbase);
      break;
    case kMaskAddF32:
      if (vec) load_bias<kMaskAddF32, true, RB, NQ>(bias, c, kbase);
      else load_bias<kMaskAddF32, false, RB, NQ>(bias, c, kbase);
      break;
    case kMaskAddBf16:
      if (vec) load_bias<kMaskAddBf16, true, RB, NQ>(bias, c, kbase);
      else load_bias<kMaskAddBf16, false, RB, NQ>(bias, c, kbase);
      break;
    case kMaskAddFp16:
      if (vec) load_bias<kMaskAddFp16, true, RB, NQ>(bias, c, kbase);
      else load_bias<kMaskAddFp16, false, RB, NQ>(bias, c, kbase);
      break;
    default:
      break;
  }
}

// t = s * scale * log2(e) + bias * log2(e) with excluded keys at -inf; mx = lane-local row maxima.
template <int RB, int NQ>
__device__ inline void apply_logits(f32x4 (&t)[RB][NQ], const f32x4 (&bias)[RB][NQ], bool has_mask, float (&mx)[RB],
                                    const LogitCtx& c, int kbase) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = c.rw0 + rb * 32 + c.l32;
    float m = kNegInf;
#pragma unroll
    for (int g = 0; g < NQ; ++g) {
      const int kk = kbase + g * 8 + c.hi * 4;
      f32x4 x = t[rb][g] * c.scale_log2;
      if (has_mask) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __builtin_fmaf(bias[rb][g][e], kLog2e, x[e]);
      }
      if (c.edge) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool dead = kk + e >= c.Nkv || (c.causal && kk + e > row + c.off);
          x[e] = dead ? kNegInf : x[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) m = __builtin_fmaxf(m, x[e]);
      t[rb][g] = x;
    }
    mx[rb] = m;
  }
}

template <int RB, int NQ>
__device__ inline void logits_dispatch(f32x4 (&t)[RB][NQ], float (&mx)[RB], const LogitCtx& c, int kbase,
                                       int kind, bool vec) {
  switch (kind) {
    case kMaskBoolU8:
      if (vec) logits<kMaskBoolU8, true, RB, NQ>(t, mx, c, kbase);
      else logits<kMaskBoolU8, false, RB, NQ>(t, mx, c, kbase);
      break;
    case kMaskAddF32:
      if (vec) logits<kMaskAddF32, true, RB, NQ>(t, mx, c, kbase);
      else logits<kMaskAddF32, false, RB, NQ>(t, mx, c, kbase);
      break;
    case kMaskAddBf16:
      if (vec) logits<kMaskAddBf16, true, RB, NQ>(t, mx, c, kbase);
      else logits<kMaskAddBf16, false, RB, NQ>(t, mx, c, kbase);
      break;
    case kMaskAddFp16:
      if (vec) logits<kMaskAddFp16, true, RB, NQ>(t, mx, c, kbase);
      else logits<kMaskAddFp16, false, RB, NQ>(t, mx, c, kbase);
      break;
    default:
      logits<kMaskNone, true, RB, NQ>(t, mx, c, kbase);
  }
}

// ---------------------------------------------------------------------------------------------
// Tiling per head dimension
// ---------------------------------------------------------------------------------------------

template <int D>
struct Tiling {
  // Column groups (DG) x row groups (RG) of waves, 32-row blocks per wave (RB), Q kept in VGPRs?
  static constexpr int DG = D <= 128 ? 1 : D <= 256 ? 2 : (D <= 512 ? ((D % 128 == 0) ? 4 : 2) : ((D % 128 == 0) ? 4 : 2));
  static constexpr int RG = 4 / DG;
  static constexpr int RB = (DG == 2 && (D % 128 != 0)) ? 1 : 2;
  static constexpr bool QREG = D <= 512;
};

template <typename T, int D>
struct FwdKernel {
  using TL = Tiling<D>;
  static constexpr int DG = TL::DG, RG = TL::RG, RB = TL::RB;
  static constexpr bool QREG = TL::QREG;
  static constexpr int NW = DG * RG;
  static_assert(NW == 4, "four waves per workgroup");
  static constexpr int R = 32 * RB;   // query rows per wave
  static constexpr int BR = R * RG;   // query rows per workgroup
  static constexpr int DW = D / DG;   // output columns per wave
  static_assert(D % DG == 0 && DW % 32 == 0, "column slices must be whole 32-column blocks");
  static constexpr int NC = DW / 32;  // 32-column chunks per slice (stages per phase per tile)
  static_assert(NC >= 2, "the two-ahead prefetch needs at least two chunks per phase");
  static constexpr int BC = 64;       // keys per tile
  static constexpr int THREADS = 256;

  // LDS map (bytes).  QK ring: [Q part (if streamed)][K part], 3 slots.  V ring: 3 slots.
  static constexpr int K_PART = DG * BC * 64;
  static constexpr int Q_PART = QREG ? 0 : DG * BR * 64;
  static constexpr int QK_SLOT = Q_PART + K_PART;
  static constexpr int V_SLOT = DG * BC * 64;
  static constexpr int NSLOT = 3;
  // Softmax exchange (DG > 1), aliasing the QK ring: partial S tiles [wave][rb][8 groups][64 lanes]
  // (f32x4), row maxima and row sums [wave][rb][32], packed P^T operands [wave][rb][4/DG][64] (i32x4).
  static constexpr int EX_PART = NW * RB * 8 * 64 * 16;
  static constexpr int EX_MAX = EX_PART;
  static constexpr int EX_SUM = EX_MAX + NW * RB * 32 * 4;
  static constexpr int EX_PK = EX_SUM + NW * RB * 32 * 4;
  static constexpr int EXCH = DG > 1 ? EX_PK + NW * RB * (4 / DG) * 64 * 16 : 0;
  static constexpr int Q_PRELOAD = QREG ? DG * BR * 64 : 0;  // one 32-column chunk of the Q tile
  static constexpr int QK_REGION_0 = NSLOT * QK_SLOT > EXCH ? NSLOT * QK_SLOT : EXCH;
  static constexpr int QK_REGION = QK_REGION_0 > Q_PRELOAD ? QK_REGION_0 : Q_PRELOAD;
  static constexpr int LDS_BYTES = QK_REGION + NSLOT * V_SLOT;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  // direct-to-LDS loads per thread for one stage
  static constexpr int K_LOADS = QK_SLOT / (THREADS * 16);
  static constexpr int V_LOADS = V_SLOT / (THREADS * 16);
  static constexpr int QPRE_LOADS = Q_PRELOAD / (THREADS * 16);
  static_assert(QK_SLOT % (THREADS * 16) == 0 && V_SLOT % (THREADS * 16) == 0, "whole loads");
  static_assert(K_LOADS <= 60 && V_LOADS <= 60, "vmcnt range");
};

// Stages one 32-column chunk of a [rows, D] tensor block into LDS as [DG slices][NROWS rows][4
// chunks of 16 bytes] (swizzled), taking columns slice*DW + col .. +31 of every slice, with
// buffer_load_dwordx4 ... lds.  Each lane's byte offset within the chunk does not depend on the
// stage, so it is computed once; the moving part (first row, first column) goes into the scalar
// buffer descriptor, whose size field ends at the tensor block's last row: rows past it read as
// zero through the hardware range check.
template <int DG, int DW, int NROWS>
struct ChunkLoader {
  static constexpr int N = DG * NROWS * 4 / 256;  // 16-byte loads per thread
  static_assert(DG * NROWS * 4 % 256 == 0, "whole loads");
  uint32_t voff[N];

  // D: the tensor's row stride in elements (the head dim, or heads x head dim when packed)
  __device__ inline void init(int D, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < N; ++t) {
      const int s = (t * 4 + wave) * 64 + lane;  // 16-byte slot this lane fills
      const int slice = s / (NROWS * 4);
      const int row = (s >> 2) % NROWS;
      const int chunk = swz(row, s & 3);
      voff[t] = (uint32_t)((row * D + slice * DW + chunk * 8) * 2);
    }
  }

  // head: first element of the [rows, D] block; rows: its row count; chunk origin (row0, col).
  __device__ inline void issue(char* dst, const uint16_t* head, int rows, int row0, int col, int D, int wave) const {
    const int64_t start = (int64_t)row0 * D + col;
    const int64_t left = (int64_t)rows * D - start;  // elements from the chunk origin to the block's end
    const uint32_t bytes = left > 0 ? (uint32_t)(left * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)(head + start), (short)0, (int)bytes, 0x00020000);
#pragma unroll
    for (int t = 0; t < N; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FFPA_LDS void*)(dst + (t * 4 + wave) * 1024), 16, voff[t], 0, 0,
                                               0);
  }
};

// Attention dropout (FwdArgs::keep set; dense contiguous layout): a weight whose keep bit is clear is
// left out of P V, and O is scaled by 1 / (1 - p) at the end; row sums and LSE keep every weight.
// The launch-uniform branches on it cost the other launches one scalar test per tile.
template <typename T, int D>
__global__ __launch_bounds__(256) void ffpa_fwd_kernel(FwdArgs a) {
  using K = FwdKernel<T, D>;
  using E = Elem<T>;
  constexpr int DG = K::DG, RB = K::RB, R = K::R, BR = K::BR, DW = K::DW, NC = K::NC, BC = K::BC;
  constexpr bool QREG = K::QREG;

  __shared__ __attribute__((aligned(1024))) char smem[K::LDS_BYTES];
  char* const qk_ring = smem;
  char* const v_ring = smem + K::QK_REGION;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / DG;
  const int dg = wave % DG;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: (b, hq, q tile); consecutive items go to one XCD so that a head's tiles share L2.
  // A packed batch (cu_q set) sizes the grid by its longest sequence; items past their sequence's
  // query length leave at once (the whole workgroup, before any barrier).
  const bool packed = a.cu_q != nullptr;
  const int nqt = (a.Nq + BR - 1) / BR;
  const int total = a.B * a.Hq * nqt;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  // packed: head-major order, so that each XCD's share holds whole heads over every sequence (the
  // sequences' lengths differ; the heads' work does not)
  // dense: the query heads of a KV group fastest (they then stream the same K/V tiles together)
  int qt, hq, b;
  if (packed) {
    qt = id % nqt;
    const int bh = id / nqt;
    hq = bh / a.B;
    b = bh % a.B;
  } else {
    const int g = id % a.group, rest = id / a.group;
    qt = rest % nqt;
    const int bk = rest / nqt, hkv = a.Hkv;
    b = bk / hkv;
    hq = (bk % hkv) * a.group + g;
  }
  if (a.causal) qt = nqt - 1 - qt;  // longest tiles of a head first
  const int hk = hq / a.group;
  const int r0 = qt * BR;              // first query row of the workgroup
  int Nq = a.Nq, Nkv = a.Nkv;
  // element offsets of this item's first Q/K/V/O row, from the strides (a packed sequence adds its
  // first token's row instead of a batch stride)
  int64_t q_base = b * a.q_sb + hq * a.q_sh, k_base = b * a.k_sb + hk * a.k_sh;
  int64_t v_base = b * a.v_sb + hk * a.v_sh, o_base = b * a.o_sb + hq * a.o_sh;
  int64_t lse_base = (int64_t)(b * a.Hq + hq) * Nq;
  const int q_rs = a.q_sr, kv_rs = a.kv_sr, o_rs = a.o_sr;  // row strides (elements)
  if (packed) {
    const SeqRange sr = seq_range(a, b);
    Nq = sr.nq;
    Nkv = sr.nkv;
    q_base = (int64_t)sr.q0 * q_rs + hq * a.q_sh;
    k_base = (int64_t)sr.k0 * kv_rs + hk * a.k_sh;
    v_base = (int64_t)sr.k0 * kv_rs + hk * a.v_sh;
    o_base = (int64_t)sr.q0 * o_rs + hq * a.o_sh;
    lse_base = (int64_t)hq * a.Tq + sr.q0;
    if (r0 >= Nq) return;
  }
  const int rw0 = r0 + rg * R;         // first query row of this wave
  const int col0 = dg * DW;            // first output column of this wave
  const int off = Nkv - Nq;            // tail alignment of the causal rule

  const uint16_t* qg = a.q + q_base;
  const uint16_t* kg = a.k + k_base;
  const uint16_t* vg = a.v + v_base;

  int kv_end = Nkv;
  if (a.causal) {
    const int lim = r0 + BR + off;
    kv_end = lim < Nkv ? lim : Nkv;
    kv_end = kv_end > 0 ? kv_end : 0;  // a packed sequence may hold fewer keys than queries
  }
  const int ntiles = (kv_end + BC - 1) / BC;

  ChunkLoader<DG, DW, BR> q_loader;
  ChunkLoader<DG, DW, BC> kv_loader;
  q_loader.init(q_rs, wave, lane);
  kv_loader.init(kv_rs, wave, lane);

  // ---- Q fragments kept for the whole key loop (D <= 512): qf[rb][k-step of 16 columns]
  i32x4 qf[QREG ? RB : 1][QREG ? DW / 16 : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      q_loader.issue(qk_ring, qg, Nq, r0, c * 32, q_rs, wave);
      wait_vmem<0>();
      block_sync();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = rg * R + rb * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int chunk = swz(row, ks * 2 + hi);
          qf[rb][c * 2 + ks] = lds_read16(qk_ring + (dg * BR + row) * 64 + chunk * 16);
        }
      }
      block_sync();
    }
  }

  // ---- stage issue: K stage (j, c) -> QK slot (j*NC + c) % 3; V stage (j, c) -> V slot (j*NC + c) % 3
  auto issue_k = [&](int j, int c) {
    char* slot = qk_ring + ((j * NC + c) % 3) * K::QK_SLOT;
    if constexpr (!QREG) q_loader.issue(slot, qg, Nq, r0, c * 32, q_rs, wave);
    kv_loader.issue(slot + K::Q_PART, kg, Nkv, j * BC, c * 32, kv_rs, wave);
  };
  auto issue_v = [&](int j, int c) {
    char* slot = v_ring + ((j * NC + c) % 3) * K::V_SLOT;
    kv_loader.issue(slot, vg, Nkv, j * BC, c * 32, kv_rs, wave);
  };

  // ---- running state
  f32x16 o_acc[RB][NC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NC; ++c) o_acc[rb][c] = f32x16{};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
  }

  // mask base for this (b, hq)
  const int64_t mask_bh = (int64_t)b * a.msb + (int64_t)hq * a.msh;

  if (ntiles > 0) {  // (a packed sequence may have no key to load)
    issue_k(0, 0);
    issue_k(0, 1);
  }

  for (int j = 0; j < ntiles; ++j) {
    // dropout: the keep words of this wave's keys (key0 + 64/DG * dg + 8g + 4hi + e) for each of its
    // row blocks, requested before the products so that they have arrived by the softmax (a row past
    // Nq reads row Nq - 1 and a word past the row's last one reads the last: never used)
    constexpr int NKW = 2 / DG;  // 32-key words owned per row
    const bool drop = a.keep != nullptr;
    uint32_t kw[RB][NKW];
    if (drop) {
      const int w0 = (j * BC + (BC / DG) * dg) >> 5, wl = a.keep_w - 1;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = rw0 + rb * 32 + l32;
        const uint32_t* kr = a.keep + ((int64_t)(b * a.Hq + hq) * Nq + (row < Nq ? row : Nq - 1)) * a.keep_w;
#pragma unroll
        for (int w = 0; w < NKW; ++w) kw[rb][w] = kr[w0 + w < wl ? w0 + w : wl];
      }
    }
    // ================= S^T = K Q^T over this wave's columns (Split-D chunks) =================
    f32x16 s_acc[RB][2];

#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // wait for stage (j, c); the one issued after it (K(j, c+1) or V(j, 0)) may stay in flight
      if (c + 1 < NC) wait_vmem<K::K_LOADS>();
      else wait_vmem<K::V_LOADS>();
      block_sync();
      if (c + 2 < NC) issue_k(j, c + 2);
      else issue_v(j, c + 2 - NC);

      const char* slot = qk_ring + ((j * NC + c) % 3) * K::QK_SLOT;
      const char* kpart = slot + K::Q_PART + dg * BC * 64;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        i32x4 kf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int key = kb * 32 + l32;
          kf[kb] = lds_read16(kpart + key * 64 + swz(key, ks * 2 + hi) * 16);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (QREG) {
            // Q fragment straight from AGPRs
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              if (c == 0 && ks == 0) E::mma_first_ba(s_acc[rb][kb], kf[kb], qf[rb][c * 2 + ks]);
              else E::mma_acc_ba(s_acc[rb][kb], kf[kb], qf[rb][c * 2 + ks]);
            }
          } else {
            const int row = rg * R + rb * 32 + l32;
            const i32x4 qv = lds_read16(slot + (dg * BR + row) * 64 + swz(row, ks * 2 + hi) * 16);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              if (c == 0 && ks == 0) E::mma_first(s_acc[rb][kb], kf[kb], qv);
              else E::mma_acc(s_acc[rb][kb], kf[kb], qv);
            }
          }
        }
      }
    }

    mma_guard_v<RB>(s_acc);

    // ================= softmax of this tile =================
    // Wave dg owns keys key0 + KO*dg .. key0 + KO*dg + KO - 1 (KO = 64/DG): with DG > 1 it sums the
    // DG partial dot products of those keys (in slice order, so every wave of the row group gets
    // bit-identical logits), computes their logits and probabilities, and the row maxima, row sums
    // and packed P^T operands are shared through LDS.
    constexpr int KO = BC / DG;  // keys owned by a wave
    constexpr int NQ = KO / 8;   // groups of 4 keys per lane (lane halves hold alternate 4s)
    const int key0 = j * BC;
    f32x4 t4[RB][NQ];
    if constexpr (DG == 1) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < NQ; ++g)
          t4[rb][g] = f32x4{s_acc[rb][g >> 2][(g & 3) * 4 + 0], s_acc[rb][g >> 2][(g & 3) * 4 + 1],
                            s_acc[rb][g >> 2][(g & 3) * 4 + 2], s_acc[rb][g >> 2][(g & 3) * 4 + 3]};
    } else {
      block_sync();  // every wave is done with the QK ring
      f32x4* ex = (f32x4*)qk_ring;
      // publish this wave's partial sums of the groups other waves own
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) {
          if (gg / NQ == dg) continue;
          const f32x16 sv = s_acc[rb][gg >> 2];
          const int v = (gg & 3) * 4;
          ex[((wave * RB + rb) * 8 + gg) * 64 + lane] = f32x4{sv[v], sv[v + 1], sv[v + 2], sv[v + 3]};
        }
      block_sync();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < NQ; ++g) {
          // this wave's own partial of group dg*NQ + g, selected without a run-time register index
          f32x4 mine = {};
#pragma unroll
          for (int d2 = 0; d2 < DG; ++d2) {
            const int gg = d2 * NQ + g;
            const int v = (gg & 3) * 4;
            if (d2 == dg) mine = f32x4{s_acc[rb][gg >> 2][v], s_acc[rb][gg >> 2][v + 1], s_acc[rb][gg >> 2][v + 2],
                                       s_acc[rb][gg >> 2][v + 3]};
          }
          const int gg = dg * NQ + g;
          f32x4 sum;
#pragma unroll
          for (int d2 = 0; d2 < DG; ++d2) {
            const f32x4 part = d2 == dg ? mine : ex[(((rg * DG + d2) * RB + rb) * 8 + gg) * 64 + lane];
            sum = d2 == 0 ? part : sum + part;
          }
          t4[rb][g] = sum;
        }
    }

    float mx[RB];
    {
      const bool tail = key0 + BC > Nkv;
      const bool diag = a.causal && (key0 + BC - 1 > rw0 + off);
      LogitCtx ctx{a.mask, mask_bh, a.msq, Nq, Nkv, key0, rw0, off, a.causal, tail || diag, a.scale_log2, l32, hi};
      logits_dispatch<RB, NQ>(t4, mx, ctx, key0 + KO * dg, a.mask_kind, a.mask_vec && !tail);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mx[rb] = max_halves(mx[rb]);
    if constexpr (DG > 1) {
      float* exm = (float*)(qk_ring + K::EX_MAX);
      if (hi == 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) exm[(wave * RB + rb) * 32 + l32] = mx[rb];
      block_sync();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float m = exm[((rg * DG) * RB + rb) * 32 + l32];
#pragma unroll
        for (int d2 = 1; d2 < DG; ++d2) m = __builtin_fmaxf(m, exm[((rg * DG + d2) * RB + rb) * 32 + l32]);
        mx[rb] = m;
      }
    }

    bool any_rescale = false;
    float alpha[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_old = m_run[rb];
      const float m_new = __builtin_fmaxf(m_old, mx[rb]);
      const bool need = (m_old != kNegInf) && (m_new > m_old + kRescaleSlack);
      alpha[rb] = need ? __builtin_amdgcn_exp2f(m_old - m_new) : 1.f;
      m_run[rb] = (m_old == kNegInf || need) ? m_new : m_old;
      any_rescale |= need;
    }
    if (__builtin_amdgcn_ballot_w64(any_rescale) != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        l_run[rb] *= alpha[rb];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          mma_guard_a(o_acc[rb][c]);
          o_acc[rb][c] *= alpha[rb];
          asm volatile("" : "+a"(o_acc[rb][c]));
        }
      }
    }

    // probabilities of the owned keys, packed as P^T operands of the owned 16-key steps
    constexpr int OWN_KS = KO / 16;
    i32x4 pk[RB][4];
    float rsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mref = m_run[rb] == kNegInf ? 0.f : m_run[rb];
      float rs = 0.f;
      f32x4 p[NQ];
#pragma unroll
      for (int g = 0; g < NQ; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[g][e] = __builtin_amdgcn_exp2f(t4[rb][g][e] - mref);
          rs += p[g][e];
        }
      if (drop) {
        // key 8g + 4hi + e of the owned keys: bit 8(g % 4) + 4hi + e of word g / 4
#pragma unroll
        for (int g = 0; g < NQ; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (through a scalar: a bit cast of the vector element itself would read element 0)
            const int sel = -(int)((kw[rb][g >> 2] >> (8 * (g & 3) + 4 * hi + e)) & 1u);
            const float pe = p[g][e];
            p[g][e] = __builtin_bit_cast(float, sel & __builtin_bit_cast(int, pe));
          }
      }
#pragma unroll
      for (int k2 = 0; k2 < OWN_KS; ++k2) {
        i32x4 w;
        w[0] = (int)pack2<T>(p[2 * k2][0], p[2 * k2][1]);
        w[1] = (int)pack2<T>(p[2 * k2][2], p[2 * k2][3]);
        w[2] = (int)pack2<T>(p[2 * k2 + 1][0], p[2 * k2 + 1][1]);
        w[3] = (int)pack2<T>(p[2 * k2 + 1][2], p[2 * k2 + 1][3]);
#pragma unroll
        for (int d2 = 0; d2 < DG; ++d2)
          if (d2 == dg) pk[rb][d2 * OWN_KS + k2] = w;
      }
      rsum[rb] = sum_halves(rs);
    }
    if constexpr (DG == 1) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l_run[rb] += rsum[rb];
    } else {
      float* exs = (float*)(qk_ring + K::EX_SUM);
      i32x4* exp_ = (i32x4*)(qk_ring + K::EX_PK);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (hi == 0) exs[(wave * RB + rb) * 32 + l32] = rsum[rb];
#pragma unroll
        for (int k2 = 0; k2 < OWN_KS; ++k2) {
          i32x4 w = {};
#pragma unroll
          for (int d2 = 0; d2 < DG; ++d2)
            if (d2 == dg) w = pk[rb][d2 * OWN_KS + k2];
          exp_[((wave * RB + rb) * OWN_KS + k2) * 64 + lane] = w;
        }
      }
      block_sync();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float tot = 0.f;
#pragma unroll
        for (int d2 = 0; d2 < DG; ++d2) {
          tot += exs[((rg * DG + d2) * RB + rb) * 32 + l32];
          if (d2 != dg)
#pragma unroll
            for (int k2 = 0; k2 < OWN_KS; ++k2)
              pk[rb][d2 * OWN_KS + k2] = exp_[(((rg * DG + d2) * RB + rb) * OWN_KS + k2) * 64 + lane];
        }
        l_run[rb] += tot;
      }
    }

    // ================= O^T += V^T P^T over this wave's columns =================
    const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) wait_vmem<K::V_LOADS>();
      else if (j + 1 < ntiles) wait_vmem<K::K_LOADS>();
      else wait_vmem<0>();
      block_sync();
      if (c + 2 < NC) issue_v(j, c + 2);
      else if (j + 1 < ntiles) issue_k(j + 1, c + 2 - NC);

      const char* vpart = v_ring + ((j * NC + c) % 3) * K::V_SLOT + dg * BC * 64;
      // transposed read: lanes 16g..16g+15 fetch keys kb4..kb4+3, columns 16*(g&1)..+15
      const int chunk = 2 * (g & 1) + ((i16 & 3) >> 1);
      const int within = 8 * (i16 & 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int keyA = ks * 16 + (g >> 1) * 4 + (i16 >> 2);
        const int keyB = keyA + 8;
        const s16x4 lo = lds_read_tr(vpart + keyA * 64 + swz(keyA, chunk) * 16 + within);
        const s16x4 hi4 = lds_read_tr(vpart + keyB * 64 + swz(keyB, chunk) * 16 + within);
        const i32x2 lo2 = __builtin_bit_cast(i32x2, lo), hi2 = __builtin_bit_cast(i32x2, hi4);
        const i32x4 vfrag = {lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) E::mma_acc_agpr(o_acc[rb][c], vfrag, pk[rb][ks]);
      }
    }
    mma_guard_all<RB * NC>(&o_acc[0][0]);  // O is never read within 12 wait states of a product
  }

  // ================= epilogue: O /= l, round, store; LSE =================
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = rw0 + rb * 32 + l32;
    if (row < Nq) {
      const float l = l_run[rb];
      float inv = l > 0.f ? 1.f / l : 0.f;
      if (a.keep != nullptr) inv *= a.drop_scale;
      uint16_t* orow = a.o + o_base + (int64_t)row * o_rs + col0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16 acc = o_acc[rb][c];
          i32x2 w;
          w[0] = (int)pack2<T>(acc[q4 * 4 + 0] * inv, acc[q4 * 4 + 1] * inv);
          w[1] = (int)pack2<T>(acc[q4 * 4 + 2] * inv, acc[q4 * 4 + 3] * inv);
          *(i32x2*)(orow + c * 32 + q4 * 8 + hi * 4) = w;
        }
      }
      if (a.lse != nullptr && dg == 0 && hi == 0) {
        const float lse = l > 0.f ? (m_run[rb] + __builtin_log2f(l)) * kLn2 : kNegInf;
        a.lse[lse_base + row] = lse;
      }
    }
  }
}

}  // namespace ffpa

#include "ffpa_row_kernel.hpp"

namespace ffpa {

// Query rows per workgroup of the kernel that serves head dim D.
template <int D>
constexpr int rows_per_block() {
  if constexpr (use_row_kernel<D>()) return RowTiling<D>::BR;
  else return FwdKernel<Bf16, D>::BR;
}

// Name of the kernel that serves head dim D (for profiles and reports).
template <int D>
constexpr const char* kernel_name() {
  if constexpr (use_row_kernel<D>()) return "ffpa_fwd_row_kernel";
  else return "ffpa_fwd_kernel";
}

// The row kernel's dropout and staged-mask variants, launched from launch_fwd.  Each group is
// instantiated in a translation unit of its own (ffpa_inst.hip, FFPA_INST_PART), so that the
// variants of one head dim compile in parallel.
template <typename T, int D>
hipError_t launch_fwd_drop(const FwdArgs& a, hipStream_t stream, long long blocks, bool plain) {
  if constexpr (use_row_kernel<D>()) {
    if (plain && !a.causal && a.Nkv % 64 == 0)
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowRaw, false, true>), dim3((unsigned)blocks), dim3(256), 0,
                         stream, a);
    else if (plain && split_drop_fits<D>())
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, split_drop_fits<D>() ? kRowSplit : kRowGeneral, false, true>),
                         dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowGeneral, false, true>), dim3((unsigned)blocks), dim3(256), 0,
                         stream, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_fwd_staged(const FwdArgs& a, hipStream_t stream, long long blocks, bool bool_mask) {
  if constexpr (use_row_kernel<D>()) {
    if (bool_mask)
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowMaskU8, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowMaskF32, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                         a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename T, int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  using K = FwdKernel<T, D>;
  // The kernels index K/V heads as hq / group: refuse a grouping that does not tile Hq exactly
  // (the C ABI validates its arguments; this guards every other caller of the launcher).
  const bool packed = a.cu_q != nullptr;
  if (a.group < 1 || a.Hkv < 1 || a.Hq != a.group * a.Hkv || a.B < 1 || a.Nq < 1 || a.Nkv < (packed ? 0 : 1))
    return hipErrorInvalidValue;
  // dropout: the dense contiguous layout, with a keep word for every 32 keys of a row
  const bool drop = a.keep != nullptr;
  if (drop && (packed || a.strided || a.keep_w != (a.Nkv + 31) / 32)) return hipErrorInvalidValue;
  // a packed batch has both offset arrays and no mask
  if (packed && (a.cu_k == nullptr || a.mask_kind != kMaskNone || a.Tq < 0 || a.Tk < 0)) return hipErrorInvalidValue;
  constexpr int BR = rows_per_block<D>();
  const int nqt = (a.Nq + BR - 1) / BR;
  const long long blocks = (long long)a.B * a.Hq * nqt;
  if (!use_row_kernel<D>() && a.dcols != D) return hipErrorInvalidValue;  // padding runs the row kernel only
  if constexpr (use_row_kernel<D>()) {
    const bool plain = a.mask_kind == kMaskNone && a.scale_log2 > 0.f;
    // fp32 additive mask with 16-byte-aligned rows whose 32-key blocks start on 128-byte lines
    // and whose byte range (including the rows of a partial last query tile) stays below 2 GiB
    const bool staged_mask = a.mask_kind == kMaskAddF32 && a.mask_vec && !a.causal && a.Nkv % 64 == 0 &&
                             a.msq % 32 == 0 &&
                             ((int64_t)a.Nq + RowTiling<D>::BR) * a.msq * 4 + (int64_t)a.Nkv * 4 < (1LL << 31);
    // the same for a boolean byte mask (4-byte aligned row starts for the 4-byte loads)
    const bool staged_bool = a.mask_kind == kMaskBoolU8 && a.mask_vec && !a.causal && a.Nkv % 64 == 0 &&
                             a.msq % 32 == 0 &&
                             ((int64_t)a.Nq + RowTiling<D>::BR) * a.msq + (int64_t)a.Nkv < (1LL << 31);
    // packed batches, strided layouts and padded head dims take the runtime-layout variants (for
    // packed batches the lengths live on the device, so whole and partial tiles are told apart in
    // the kernel)
    const bool padded = a.dcols != D;
    if (padded && (drop || a.dcols > D || a.dcols < 8 || a.dcols % 8 != 0)) return hipErrorInvalidValue;
    const bool runtime_layout = packed || a.strided || padded;
    if (drop) return launch_fwd_drop<T, D>(a, stream, blocks, plain);
    if (!runtime_layout && (staged_mask || staged_bool)) return launch_fwd_staged<T, D>(a, stream, blocks, staged_bool);
    if (runtime_layout && plain)
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowSplit, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (runtime_layout)
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowGeneral, true>), dim3((unsigned)blocks), dim3(256), 0, stream,
                         a);
    else if (plain && !a.causal && a.Nkv % 64 == 0)
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowRaw, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (plain)
      // the runtime-layout variant where the contiguous one does not fit its registers (the
      // contiguous strides are set in the arguments either way)
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowSplit, !dense_split_fits<D>()>), dim3((unsigned)blocks),
                         dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowGeneral, false>), dim3((unsigned)blocks), dim3(256), 0, stream,
                         a);
  } else {
    hipLaunchKernelGGL((ffpa_fwd_kernel<T, D>), dim3((unsigned)blocks), dim3(K::THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ffpa

// Exact large-head-dim attention forward for gfx950 (MI355X, CDNA4): the definitions the forward
// kernels share (argument block, matrix-core wrappers, logit and mask helpers, the staged O store)
// and the launchers of the row-owner kernel (ffpa_row_kernel.hpp), which serves every head dim: 64,
// 128, 192, ..., 512, 640, 768, 896 and 1024 as compiled, every other multiple of 8 as the next of
// those with padding columns.
//
// Matrix-core layout.  Both products use v_mfma_f32_32x32x16_{bf16,f16}.  S is formed transposed,
// S^T = K Q^T, so lane l holds query row l%32 and 16 keys of a 32-key block; O is formed transposed
// too, O^T = V^T P^T, so lane l again holds row l%32.  Row statistics are therefore lane-local and
// only need one cross-half exchange (v_permlane32_swap).  The S accumulator, rounded to bf16/fp16, is
// directly the P^T operand of the second product: the key order it implies is matched by reading V
// through ds_read_b64_tr_b16 with the same key permutation (the sum over keys does not care about
// order).
//
// Softmax.  Logits are kept in the log2 domain and exponentiated with v_exp_f32.  The running row
// maximum is only moved (and O, l rescaled) when it grows by more than 8, so P stays below 2^8 and
// the O rescale, a pass over up to 256 accumulator registers, is skipped on almost every tile; the
// final O/l and LSE use whichever maximum was kept, which is exact algebra.  Fully excluded rows keep
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

}  // namespace ffpa

#include "ffpa_row_kernel.hpp"

namespace ffpa {

// Query rows per workgroup of the kernel that serves head dim D.
template <int D>
constexpr int rows_per_block() {
  static_assert(use_row_kernel<D>(), "a compiled head dim runs the row kernel");
  return RowTiling<D>::BR;
}

// Name of the kernel that serves head dim D (for profiles and reports).
template <int D>
constexpr const char* kernel_name() {
  return "ffpa_fwd_row_kernel";
}

// The row kernel's dropout and staged-mask variants, launched from launch_fwd.  Each group is
// instantiated in a translation unit of its own (ffpa_inst.hip, FFPA_INST_PART), so that the
// variants of one head dim compile in parallel.
template <typename T, int D>
hipError_t launch_fwd_drop(const FwdArgs& a, hipStream_t stream, long long blocks, bool plain) {
  if constexpr (use_row_kernel<D>()) {
    if (a.dcols != D)  // a padded head dim: the runtime-layout general variant, row stride dcols
      hipLaunchKernelGGL((ffpa_fwd_row_kernel<T, D, kRowGeneral, true, true>), dim3((unsigned)blocks), dim3(256), 0,
                         stream, a);
    else if (plain && !a.causal && a.Nkv % 64 == 0)
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
  static_assert(use_row_kernel<D>(), "a compiled head dim runs the row kernel");
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
    if (padded && (a.dcols > D || a.dcols < 8 || a.dcols % 8 != 0)) return hipErrorInvalidValue;
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
  }
  return hipGetLastError();
}

}  // namespace ffpa

// C ABI of the attention forward (declared in include/ffpa.h): argument checking, the dispatch
// to the per-head-dim kernels, and status reporting.  Argument rules follow the ffpa-attn "API
// Reference" page, ffpa_attn_func: dtype fp16/bf16 (else TypeError), key/value sharing Nh_kv and
// Nkv with Nh_q a multiple of Nh_kv, causal only with Nkv >= Nq (else ValueError), and a
// NotImplementedError class for valid requests outside what the kernels cover.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <utility>

#include "../../include/ffpa.h"
#include "ffpa_kernel.hpp"
#include "ffpa_launch.hpp"

namespace {

thread_local char g_detail[256];
// measurement aid: clock-stamp buffer of the calling thread's forward launches (null: off)
thread_local unsigned long long* g_stamps = nullptr;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return status;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t mask_elem_size(int kind) {
  switch (kind) {
    case FFPA_MASK_BOOL_U8: return 1;
    case FFPA_MASK_ADD_F32: return 4;
    case FFPA_MASK_ADD_BF16:
    case FFPA_MASK_ADD_FP16: return 2;
    default: return 0;
  }
}

// Rows per workgroup of the kernel for head dim D, 0 if D has no kernel.
int rows_for(int64_t D) {
  switch (D) {
#define FFPA_ROWS_CASE(Dv) \
  case Dv: return ffpa::rows_per_block<Dv>();
    FFPA_FOR_EACH_D(FFPA_ROWS_CASE)
#undef FFPA_ROWS_CASE
    default: return 0;
  }
}

// Head dim of the kernel that serves tensors of head dim D: the smallest compiled head dim at or
// above D (D a multiple of 8), whose columns past D are padding.  0 if none.
int64_t kernel_dim(int64_t D) {
  if (D < 8 || D % 8 != 0) return 0;
  int64_t best = 0;
#define FFPA_PAD_CASE(Dv) \
  if (best == 0 && Dv >= D && ffpa::use_row_kernel<Dv>()) best = Dv;
  FFPA_FOR_EACH_D(FFPA_PAD_CASE)
#undef FFPA_PAD_CASE
  return best;
}

// Elements from a tensor's first element to one past its last: (B-1)*sb + (H-1)*sh + (N-1)*sn + D.
// (in 128-bit arithmetic: caller strides may be as large as int64_t allows)
__int128 extent(const int64_t st[3], int64_t B, int64_t H, int64_t N, int64_t D) {
  return (__int128)(B - 1) * st[0] + (__int128)(H - 1) * st[1] + (__int128)(N - 1) * st[2] + D;
}

// True when no two elements of a [B, H, N, D] tensor with strides st (and unit head-dim stride)
// share an address: the dimensions of size > 1, sorted by stride, each step past the whole span of
// the smaller ones.
bool non_overlapping(const int64_t st[3], int64_t B, int64_t H, int64_t N, int64_t D) {
  int64_t dims[4][2] = {{1, D}, {st[2], N}, {st[1], H}, {st[0], B}};
  for (int i = 1; i < 4; ++i)
    for (int j = i; j > 0 && dims[j][0] < dims[j - 1][0]; --j) {
      std::swap(dims[j][0], dims[j - 1][0]);
      std::swap(dims[j][1], dims[j - 1][1]);
    }
  __int128 span = 0;  // elements covered by the smaller dimensions, minus one
  for (int i = 0; i < 4; ++i) {
    if (dims[i][1] <= 1) continue;
    if (dims[i][0] <= span) return false;
    span += (__int128)(dims[i][1] - 1) * dims[i][0];
  }
  return true;
}

// Layout rules of ffpa_fwd_strided: strides in elements, >= 0, multiples of 8 (16-byte rows for the
// 128-bit loads), K and V sharing their row stride, O not overlapping itself, and the row spans of
// one head within the kernels' 32-bit offsets.
int check_layout(const ffpa_layout_t* lay, int64_t Hq, int64_t Nq, int64_t Nkv, int64_t D, int64_t B) {
  const int64_t* all[4] = {lay->q, lay->k, lay->v, lay->o};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i) {
      if (all[t][i] < 0) return fail(FFPA_ERR_VALUE, "strides must be >= 0");
      if (all[t][i] % 8 != 0) return fail(FFPA_ERR_VALUE, "strides must be multiples of 8 elements (16 bytes)");
    }
  if (lay->k[2] != lay->v[2]) return fail(FFPA_ERR_UNSUPPORTED, "K and V must share their row stride");
  // rows past a head's last one must fall outside its load range (they read as zero)
  if (lay->q[2] < D || lay->k[2] < D || lay->o[2] < D)
    return fail(FFPA_ERR_UNSUPPORTED, "row strides must be at least D (rows may not overlap)");
  if (lay->q[2] >= (1LL << 30) || lay->k[2] >= (1LL << 30) || lay->o[2] >= (1LL << 30))
    return fail(FFPA_ERR_UNSUPPORTED, "row strides beyond the 32-bit indexing of the kernels");
  if ((Nq + 256) * lay->q[2] * 2 >= (1LL << 31) || (Nkv + 256) * lay->k[2] * 2 >= (1LL << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "one head's Q or K/V rows must span below 2 GiB (buffer addressing)");
  if (!non_overlapping(lay->o, B, Hq, Nq, D)) return fail(FFPA_ERR_VALUE, "the strides of o make elements overlap");
  return FFPA_OK;
}

// Head dim of the fp8 kernel that serves D (the next of 128, 256, 384, 512, 768, 1024), 0 if none.
int64_t fp8_kernel_dim(int64_t D) {
  if (D < 16 || D > 1024 || D % 16 != 0) return 0;
  if (D <= 512) return (D + 127) / 128 * 128;
  return D <= 768 ? 768 : 1024;
}

// fp8: q, k and v hold e4m3 bytes (one byte per element) and dtype is the output's element type.
int check(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o, const float* lse,
          int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal,
          int dtype, const ffpa_layout_t* lay = nullptr, bool fp8 = false) {
  g_detail[0] = '\0';
  if (dtype != FFPA_BF16 && dtype != FFPA_FP16)
    return fail(FFPA_ERR_TYPE, "%s %d is neither bf16 nor fp16", fp8 ? "out_dtype" : "dtype", dtype);
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1)
    return fail(FFPA_ERR_VALUE, "every size must be >= 1 (B=%lld Hq=%lld Hkv=%lld Nq=%lld Nkv=%lld D=%lld)",
                (long long)B, (long long)Hq, (long long)Hkv, (long long)Nq, (long long)Nkv, (long long)D);
  if (Hq % Hkv != 0)
    return fail(FFPA_ERR_VALUE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (is_causal != 0 && is_causal != 1) return fail(FFPA_ERR_VALUE, "is_causal must be 0 or 1");
  if (is_causal && Nkv < Nq)
    return fail(FFPA_ERR_VALUE, "causal attention needs Nkv >= Nq (Nq=%lld, Nkv=%lld)", (long long)Nq, (long long)Nkv);
  if (std::isinf(scale)) return fail(FFPA_ERR_VALUE, "scale must be finite (NaN selects 1/sqrt(D))");
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return fail(FFPA_ERR_VALUE, "q, k, v and o must be non-null");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
    return fail(FFPA_ERR_VALUE, "q, k, v and o must be 16-byte aligned");
  if (lse != nullptr && ((uintptr_t)lse & 3)) return fail(FFPA_ERR_VALUE, "lse must be 4-byte aligned");
  if (fp8 && fp8_kernel_dim(D) == 0)
    return fail(FFPA_ERR_UNSUPPORTED, "head dim %lld: the fp8 kernels cover 16 <= D <= 1024 with D %% 16 == 0",
                (long long)D);
  if (!fp8 && (D > 1024 || kernel_dim(D) == 0))
    return fail(FFPA_ERR_UNSUPPORTED, "head dim %lld: kernels cover 8 <= D <= 1024 with D %% 8 == 0", (long long)D);
  // 32-bit in-kernel indexing, then the grid size (each factor bounded first, so that no product
  // below overflows)
  if (Nq > (1LL << 30) || Nkv > (1LL << 30) || B > (1LL << 30) || Hq > (1LL << 30) || B * Hq > (1LL << 30) ||
      B * Hkv > (1LL << 30))
    return fail(FFPA_ERR_UNSUPPORTED, "sizes beyond the 32-bit row indexing of the kernels");
  const int br = fp8 ? (D <= 512 ? 128 : 64) : rows_for(kernel_dim(D));
  const int64_t nqt = (Nq + br - 1) / br;
  if (B * Hq * nqt > 0x7fffffffLL) return fail(FFPA_ERR_UNSUPPORTED, "too many workgroups");
  if (Nq * D * 2 >= (1LL << 31) || Nkv * D * 2 >= (1LL << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "one head of Q or K/V must stay below 2 GiB (buffer addressing)");
  if (lay != nullptr) {
    const int st = check_layout(lay, Hq, Nq, Nkv, D, B);
    if (st != FFPA_OK) return st;
  }
  const size_t esz = fp8 ? 1 : 2;
  // byte extents of the tensors (for a strided layout: from the first to one past the last element)
  size_t qbytes = (size_t)(B * Hq * Nq * D) * esz, kbytes = (size_t)(B * Hkv * Nkv * D) * esz;
  size_t vbytes = kbytes, obytes = (size_t)(B * Hq * Nq * D) * 2;
  if (lay != nullptr) {
    const __int128 eq = extent(lay->q, B, Hq, Nq, D), ek = extent(lay->k, B, Hkv, Nkv, D),
                   ev = extent(lay->v, B, Hkv, Nkv, D), eo = extent(lay->o, B, Hq, Nq, D);
    const __int128 lim = (__int128)1 << 60;  // no tensor spans an exabyte
    if (eq > lim || ek > lim || ev > lim || eo > lim) return fail(FFPA_ERR_UNSUPPORTED, "strides too large");
    qbytes = (size_t)eq * esz;
    kbytes = (size_t)ek * esz;
    vbytes = (size_t)ev * esz;
    obytes = (size_t)eo * esz;
  }
  const size_t lbytes = lse ? (size_t)(B * Hq * Nq) * 4 : 0;
  if (ranges_overlap(o, obytes, q, qbytes) || ranges_overlap(o, obytes, k, kbytes) ||
      ranges_overlap(o, obytes, v, vbytes) || ranges_overlap(o, obytes, lse, lbytes))
    return fail(FFPA_ERR_VALUE, "o must not overlap q, k, v or lse");
  if (lse != nullptr && (ranges_overlap(lse, lbytes, q, qbytes) || ranges_overlap(lse, lbytes, k, kbytes) ||
                         ranges_overlap(lse, lbytes, v, vbytes)))
    return fail(FFPA_ERR_VALUE, "lse must not overlap q, k or v");
  if (mask != nullptr) {
    if (mask->kind == FFPA_MASK_NONE) {
      // a descriptor that says "no mask"
    } else {
      const size_t msz = mask_elem_size(mask->kind);
      if (msz == 0) return fail(FFPA_ERR_TYPE, "unknown mask kind %d", (int)mask->kind);
      if (mask->data == nullptr) return fail(FFPA_ERR_VALUE, "mask data is null");
      if (mask->stride_k != 1) return fail(FFPA_ERR_UNSUPPORTED, "mask stride_k must be 1");
      if (mask->stride_b < 0 || mask->stride_h < 0 || mask->stride_q < 0)
        return fail(FFPA_ERR_VALUE, "mask strides must be >= 0");
      if ((uintptr_t)mask->data % msz) return fail(FFPA_ERR_VALUE, "mask data misaligned for its element type");
      const __int128 last = (__int128)(B - 1) * mask->stride_b + (__int128)(Hq - 1) * mask->stride_h +
                            (__int128)(Nq - 1) * mask->stride_q + Nkv;
      if (last > ((__int128)1 << 62) / (int64_t)msz) return fail(FFPA_ERR_UNSUPPORTED, "mask too large");
      const size_t mbytes = (size_t)last * msz;
      if (ranges_overlap(o, obytes, mask->data, mbytes) || ranges_overlap(lse, lbytes, mask->data, mbytes))
        return fail(FFPA_ERR_VALUE, "o and lse must not overlap the mask");
    }
  }
  return FFPA_OK;
}

// Argument rules of the packed entry (ffpa-attn "API Reference", ffpa_attn_varlen_func): the
// same dtype, head and scale rules as the dense entry, plus the offsets' pointers and the 32-bit
// offsets the kernels form (one sequence's key rows, and token x head indexes).
int check_varlen(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                 const void* o, const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                 int64_t maxq, int64_t maxk, int64_t D, float scale, int is_causal, int dtype) {
  g_detail[0] = '\0';
  if (dtype != FFPA_BF16 && dtype != FFPA_FP16) return fail(FFPA_ERR_TYPE, "dtype %d is neither bf16 nor fp16", dtype);
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1)
    return fail(FFPA_ERR_VALUE, "B, Hq, Hkv and D must be >= 1 (B=%lld Hq=%lld Hkv=%lld D=%lld)", (long long)B,
                (long long)Hq, (long long)Hkv, (long long)D);
  if (Tq < 0 || Tk < 0 || maxq < 0 || maxk < 0)
    return fail(FFPA_ERR_VALUE, "token counts and longest lengths must be >= 0");
  if (Hq % Hkv != 0)
    return fail(FFPA_ERR_VALUE, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (is_causal != 0 && is_causal != 1) return fail(FFPA_ERR_VALUE, "is_causal must be 0 or 1");
  if (std::isinf(scale)) return fail(FFPA_ERR_VALUE, "scale must be finite (NaN selects 1/sqrt(D))");
  if (cu_q == nullptr || cu_k == nullptr) return fail(FFPA_ERR_VALUE, "cu_seqlens_q and cu_seqlens_k must be non-null");
  if (((uintptr_t)cu_q | (uintptr_t)cu_k) & 3) return fail(FFPA_ERR_VALUE, "cu_seqlens must be 4-byte aligned");
  if ((Tq > 0 && (q == nullptr || o == nullptr)) || (Tk > 0 && (k == nullptr || v == nullptr)))
    return fail(FFPA_ERR_VALUE, "q, k, v and o must be non-null when their tensors are not empty");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15)
    return fail(FFPA_ERR_VALUE, "q, k, v and o must be 16-byte aligned");
  if (lse != nullptr && ((uintptr_t)lse & 3)) return fail(FFPA_ERR_VALUE, "lse must be 4-byte aligned");
  if (D > 1024 || kernel_dim(D) == 0)
    return fail(FFPA_ERR_UNSUPPORTED, "head dim %lld: kernels cover 8 <= D <= 1024 with D %% 8 == 0", (long long)D);
  const int br = rows_for(kernel_dim(D));
  if (B > (1LL << 30) || B * Hq * ((maxq + br - 1) / br) > 0x7fffffffLL)
    return fail(FFPA_ERR_UNSUPPORTED, "too many workgroups");
  if (Tq >= (1LL << 31) || Tk >= (1LL << 31) || Tq * Hq >= (1LL << 31) || Tk * Hkv >= (1LL << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "token x head counts beyond the 32-bit indexing of the kernels");
  if ((maxq + 256) * Hq * D * 2 >= (1LL << 31) || (maxk + 256) * Hkv * D * 2 >= (1LL << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "one sequence's Q or K/V rows must span below 2 GiB (buffer addressing)");
  const size_t qbytes = (size_t)(Tq * Hq * D) * 2, kvbytes = (size_t)(Tk * Hkv * D) * 2;
  const size_t lbytes = lse ? (size_t)(Tq * Hq) * 4 : 0, cbytes = (size_t)(B + 1) * 4;
  if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k, kvbytes) ||
      ranges_overlap(o, qbytes, v, kvbytes) || ranges_overlap(o, qbytes, lse, lbytes) ||
      ranges_overlap(o, qbytes, cu_q, cbytes) || ranges_overlap(o, qbytes, cu_k, cbytes))
    return fail(FFPA_ERR_VALUE, "o must not overlap q, k, v, lse or the offsets");
  if (lse != nullptr && (ranges_overlap(lse, lbytes, q, qbytes) || ranges_overlap(lse, lbytes, k, kvbytes) ||
                         ranges_overlap(lse, lbytes, v, kvbytes) || ranges_overlap(lse, lbytes, cu_q, cbytes) ||
                         ranges_overlap(lse, lbytes, cu_k, cbytes)))
    return fail(FFPA_ERR_VALUE, "lse must not overlap q, k, v or the offsets");
  return FFPA_OK;
}

template <typename T>
hipError_t dispatch(int64_t D, const ffpa::FwdArgs& a, hipStream_t s) {
  switch (kernel_dim(D)) {
#define FFPA_DISPATCH_CASE(Dv) \
  case Dv: return ffpa::launch_fwd<T, Dv>(a, s);
    FFPA_FOR_EACH_D(FFPA_DISPATCH_CASE)
#undef FFPA_DISPATCH_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace ffpa {
int report_failure(int status, const char* msg) { return fail(status, "%s", msg); }
void clear_failure() { g_detail[0] = '\0'; }
}  // namespace ffpa

extern "C" {

int ffpa_check_args(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o,
                    const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                    float scale, int is_causal, int dtype) {
  return check(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
}

static int launch_dense(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                        const ffpa_layout_t* lay, float scale, int is_causal, int dtype, void* stream,
                        const uint32_t* keep = nullptr, float dropout_p = 0.f) {
  ffpa::FwdArgs a{};
  if (keep != nullptr) {
    a.keep = keep;
    a.keep_w = (int)((Nkv + 31) / 32);
    a.drop_scale = (float)(1.0 / (1.0 - (double)dropout_p));
  }
  if (lay == nullptr) {  // contiguous [B, H, N, D]
    a.q_sb = a.o_sb = Hq * Nq * D;
    a.q_sh = a.o_sh = Nq * D;
    a.k_sb = a.v_sb = Hkv * Nkv * D;
    a.k_sh = a.v_sh = Nkv * D;
    a.q_sr = a.kv_sr = a.o_sr = (int)D;
    a.strided = 0;
  } else {
    a.q_sb = lay->q[0];
    a.q_sh = lay->q[1];
    a.q_sr = (int)lay->q[2];
    a.k_sb = lay->k[0];
    a.k_sh = lay->k[1];
    a.v_sb = lay->v[0];
    a.v_sh = lay->v[1];
    a.kv_sr = (int)lay->k[2];
    a.o_sb = lay->o[0];
    a.o_sh = lay->o[1];
    a.o_sr = (int)lay->o[2];
    a.strided = 1;
  }
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.mask_kind = ffpa::kMaskNone;
  if (mask != nullptr && mask->kind != FFPA_MASK_NONE) {
    const size_t msz = mask_elem_size(mask->kind);
    a.mask = mask->data;
    a.mask_kind = mask->kind;  // the enum values match ffpa::MaskKind
    a.msb = mask->stride_b;
    a.msh = mask->stride_h;
    a.msq = mask->stride_q;
    // four consecutive keys form one aligned vector load when every row start is 4-element aligned
    const bool aligned = ((uintptr_t)mask->data % (4 * msz)) == 0;
    a.mask_vec = aligned && (a.msb % 4 == 0) && (a.msh % 4 == 0) && (a.msq % 4 == 0);
  }
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Nq = (int)Nq;
  a.Nkv = (int)Nkv;
  a.group = (int)(Hq / Hkv);
  a.dcols = (int)D;
  a.stamps = g_stamps;
  const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)D) : (double)scale;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.causal = is_causal;
  const hipStream_t s = (hipStream_t)stream;
  const hipError_t e = dtype == FFPA_BF16 ? dispatch<ffpa::Bf16>(D, a, s) : dispatch<ffpa::Fp16>(D, a, s);
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FFPA_OK;
}

int ffpa_fwd(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse, int64_t B,
             int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype,
             void* stream) {
  const int st = check(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  return launch_dense(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, nullptr, scale, is_causal, dtype, stream);
}

int ffpa_check_dropout_args(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o,
                            const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                            float scale, int is_causal, int dtype, const uint32_t* keep, float dropout_p) {
  const int st = check(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  if (!(dropout_p >= 0.f && dropout_p < 1.f)) return fail(FFPA_ERR_VALUE, "dropout probability must lie in [0, 1)");
  if (keep == nullptr || ((uintptr_t)keep & 3)) return fail(FFPA_ERR_VALUE, "keep must be non-null and 4-byte aligned");
  if (B * Hq * Nq * ((Nkv + 31) / 32) >= (1LL << 40)) return fail(FFPA_ERR_UNSUPPORTED, "keep mask too large");
  const size_t kbytes = (size_t)(B * Hq * Nq * ((Nkv + 31) / 32)) * 4;
  const size_t obytes = (size_t)(B * Hq * Nq * D) * 2, lbytes = lse ? (size_t)(B * Hq * Nq) * 4 : 0;
  if (ranges_overlap(o, obytes, keep, kbytes) || ranges_overlap(lse, lbytes, keep, kbytes))
    return fail(FFPA_ERR_VALUE, "o and lse must not overlap the keep mask");
  return FFPA_OK;
}

int ffpa_fwd_dropout(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale,
                     int is_causal, int dtype, const uint32_t* keep, float dropout_p, void* stream) {
  const int st = ffpa_check_dropout_args(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype, keep,
                                         dropout_p);
  if (st != FFPA_OK) return st;
  return launch_dense(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, nullptr, scale, is_causal, dtype, stream, keep,
                      dropout_p);
}

int ffpa_check_strided_args(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, const void* o,
                            const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                            const ffpa_layout_t* layout, float scale, int is_causal, int dtype) {
  if (layout == nullptr) return fail(FFPA_ERR_VALUE, "layout must be non-null");
  return check(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype, layout);
}

int ffpa_fwd_strided(const void* q, const void* k, const void* v, const ffpa_mask_t* mask, void* o, float* lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                     const ffpa_layout_t* layout, float scale, int is_causal, int dtype, void* stream) {
  const int st = ffpa_check_strided_args(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, layout, scale, is_causal,
                                         dtype);
  if (st != FFPA_OK) return st;
  return launch_dense(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, layout, scale, is_causal, dtype, stream);
}

int ffpa_check_varlen_args(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, const void* o, const float* lse, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Tq, int64_t Tk, int64_t max_seqlen_q, int64_t max_seqlen_k,
                           int64_t D, float scale, int is_causal, int dtype) {
  return check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, B, Hq, Hkv, Tq, Tk, max_seqlen_q, max_seqlen_k, D,
                      scale, is_causal, dtype);
}

int ffpa_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Tq, int64_t Tk, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, float scale,
                    int is_causal, int dtype, void* stream) {
  const int st = check_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, o, lse, B, Hq, Hkv, Tq, Tk, max_seqlen_q,
                              max_seqlen_k, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  if (Tq == 0 || max_seqlen_q == 0) return FFPA_OK;  // no query row anywhere
  ffpa::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.mask_kind = ffpa::kMaskNone;
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Nq = (int)max_seqlen_q;
  a.Nkv = (int)max_seqlen_k;
  a.group = (int)(Hq / Hkv);
  a.dcols = (int)D;
  a.stamps = g_stamps;
  const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)D) : (double)scale;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.causal = is_causal;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.Tq = (int)Tq;
  a.Tk = (int)Tk;
  a.q_sh = a.k_sh = a.v_sh = a.o_sh = D;  // [T, H, D]: no batch stride
  a.q_sr = a.o_sr = (int)(Hq * D);
  a.kv_sr = (int)(Hkv * D);
  const hipStream_t s = (hipStream_t)stream;
  const hipError_t e = dtype == FFPA_BF16 ? dispatch<ffpa::Bf16>(D, a, s) : dispatch<ffpa::Fp16>(D, a, s);
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FFPA_OK;
}

int ffpa_check_cu_seqlens(const int32_t* cu_host, int64_t B, int64_t T, int64_t max_seqlen) {
  g_detail[0] = '\0';
  if (cu_host == nullptr || B < 1) return fail(FFPA_ERR_VALUE, "need B >= 1 and B+1 offsets");
  if (cu_host[0] != 0) return fail(FFPA_ERR_VALUE, "cu_seqlens[0] is %d, not 0", (int)cu_host[0]);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t len = (int64_t)cu_host[b + 1] - cu_host[b];
    if (len < 0) return fail(FFPA_ERR_VALUE, "cu_seqlens decreases at index %lld", (long long)(b + 1));
    if (len > max_seqlen)
      return fail(FFPA_ERR_VALUE, "sequence %lld has %lld tokens, more than max_seqlen %lld", (long long)b,
                  (long long)len, (long long)max_seqlen);
  }
  if (cu_host[B] != T)
    return fail(FFPA_ERR_VALUE, "cu_seqlens[B] is %d, not the token count %lld", (int)cu_host[B], (long long)T);
  return FFPA_OK;
}

int ffpa_check_fp8_args(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                        const float* v_descale, const ffpa_mask_t* mask, const void* o, const float* lse, int64_t B,
                        int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal,
                        int out_dtype) {
  const int st = check(q, k, v, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, out_dtype, nullptr, true);
  if (st != FFPA_OK) return st;
  const float* f[3] = {q_descale, k_descale, v_descale};
  const int64_t heads[3] = {Hq, Hkv, Hkv};
  const size_t obytes = (size_t)(B * Hq * Nq * D) * 2, lbytes = lse ? (size_t)(B * Hq * Nq) * 4 : 0;
  for (int t = 0; t < 3; ++t) {
    if (f[t] == nullptr) continue;
    if ((uintptr_t)f[t] & 3) return fail(FFPA_ERR_VALUE, "descale factors must be 4-byte aligned");
    const size_t fb = (size_t)(B * heads[t]) * 4;
    if (ranges_overlap(o, obytes, f[t], fb) || ranges_overlap(lse, lbytes, f[t], fb))
      return fail(FFPA_ERR_VALUE, "o and lse must not overlap the descale factors");
  }
  return FFPA_OK;
}

int ffpa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                 const float* v_descale, const ffpa_mask_t* mask, void* o, float* lse, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int out_dtype,
                 void* stream) {
  const int st = ffpa_check_fp8_args(q, k, v, q_descale, k_descale, v_descale, mask, o, lse, B, Hq, Hkv, Nq, Nkv, D,
                                     scale, is_causal, out_dtype);
  if (st != FFPA_OK) return st;
  ffpa::FwdArgs a{};
  a.q = (const uint16_t*)q;  // e4m3 bytes: the kernels read them as such
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.q_desc = q_descale;
  a.k_desc = k_descale;
  a.v_desc = v_descale;
  a.mask_kind = ffpa::kMaskNone;
  if (mask != nullptr && mask->kind != FFPA_MASK_NONE) {
    const size_t msz = mask_elem_size(mask->kind);
    a.mask = mask->data;
    a.mask_kind = mask->kind;
    a.msb = mask->stride_b;
    a.msh = mask->stride_h;
    a.msq = mask->stride_q;
    const bool aligned = ((uintptr_t)mask->data % (4 * msz)) == 0;
    a.mask_vec = aligned && (a.msb % 4 == 0) && (a.msh % 4 == 0) && (a.msq % 4 == 0);
  }
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Nq = (int)Nq;
  a.Nkv = (int)Nkv;
  a.group = (int)(Hq / Hkv);
  a.dcols = (int)D;
  a.q_sr = a.kv_sr = (int)D;  // bytes per Q/K/V row
  a.o_sr = (int)D;            // elements per O row
  a.stamps = g_stamps;
  const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)D) : (double)scale;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.causal = is_causal;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipErrorInvalidValue;
  switch (fp8_kernel_dim(D)) {
#define FFPA_FP8_CASE(Dv)                                                                                         \
  case Dv:                                                                                                        \
    e = out_dtype == FFPA_BF16 ? ffpa::launch_fwd_fp8<ffpa::Bf16, Dv>(a, s) : ffpa::launch_fwd_fp8<ffpa::Fp16, Dv>(a, s); \
    break;
    FFPA_FP8_FOR_EACH_D(FFPA_FP8_CASE)
#undef FFPA_FP8_CASE
    default: break;
  }
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FFPA_OK;
}

int64_t ffpa_fp8_kernel_head_dim(int64_t D) { return fp8_kernel_dim(D); }

int ffpa_clock_stamps(unsigned long long* stamps) {
  g_detail[0] = '\0';
  if (stamps != nullptr && ((uintptr_t)stamps & 7)) return fail(FFPA_ERR_VALUE, "stamps must be 8-byte aligned");
  g_stamps = stamps;
  return FFPA_OK;
}

const char* ffpa_status_string(int status) {
  switch (status) {
    case FFPA_OK: return "ok";
    case FFPA_ERR_TYPE: return "type error";
    case FFPA_ERR_VALUE: return "value error";
    case FFPA_ERR_UNSUPPORTED: return "not supported";
    case FFPA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ffpa_last_error_detail(void) { return g_detail; }

int ffpa_rows_per_block(int64_t D) { return D > 1024 ? 0 : rows_for(kernel_dim(D)); }

int64_t ffpa_kernel_head_dim(int64_t D) { return D > 1024 ? 0 : kernel_dim(D); }

const char* ffpa_kernel_name(int64_t D) {
  switch (D > 1024 ? 0 : kernel_dim(D)) {
#define FFPA_NAME_CASE(Dv) \
  case Dv: return ffpa::kernel_name<Dv>();
    FFPA_FOR_EACH_D(FFPA_NAME_CASE)
#undef FFPA_NAME_CASE
    default: return nullptr;
  }
}

}  // extern "C"

// Backward of the attention forward (ffpa-attn "API Reference": ffpa_attn_func's backward, which
// the pages run as SDPA's backward): dQ, dK, dV from Q, K, V, O, dO and the forward's fp32 LSE.
//
// One chunk of query heads at a time, over a caller-provided workspace: a KV group (a KV head with
// its G query heads), or, without grouping (G = 1), as many consecutive heads as the workspace
// bound allows, so that every product is one strided-batched call over the chunk:
//   Delta = rowsum(dO * O)                         (HIP kernel, once for every row)
//   S  = Q K^T                    [G, Nq, Nkv] f32 (library GEMM)
//   P  = exp(scale S + bias - LSE), 0 where excluded; kept in f32 and as a 16-bit copy (HIP kernel)
//   dV_g = P^T dO                 [G, Nkv, D] f32  (library GEMM)
//   dP = dO V^T                   [G, Nq, Nkv] f32 (library GEMM)
//   dS = scale P (dP - Delta)     16-bit           (HIP kernel)
//   dQ = dS K                     written as the output dtype (library GEMM)
//   dK_g = dS^T Q                 [G, Nkv, D] f32  (library GEMM)
//   dK, dV = sums over the group's G heads        (HIP kernel)
// With attention dropout (ffpa_bwd_dropout: O = (P * M) V with M = keep / (1 - p) a constant), the
// 16-bit copy of P that forms dV holds P * M, and the row term is applied to dP * M:
// dS = scale P (dP M - Delta), with Delta = rowsum(dO * O) of the dropped-out O.
// With the additive mask's gradient (ffpa_bwd_mask_grad): the logits are scale S + bias, so the
// bias's gradient is the logits' gradient P (dP - Delta) itself, summed over the dimensions the mask
// broadcasts; the row-term kernel also keeps it in f32 (over dP, no longer needed), and one more
// kernel adds each chunk's share into the dense f32 result, every element owned by one thread.
// The matrix products are plain dense GEMMs (rocBLAS strided-batched, bf16/fp16 in, fp32
// accumulate); the softmax recompute, the row term and the group sums are the kernels below.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/ffpa.h"

namespace ffpa {
// the thread's error detail (ffpa_last_error_detail), kept by the C-ABI object
int report_failure(int status, const char* msg);
void clear_failure();
}  // namespace ffpa

namespace {

int bfail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int bfail(int status, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return ffpa::report_failure(status, buf);
}

constexpr float kLog2eB = 1.4426950408889634f;

__device__ inline float load16(const uint16_t* p, int64_t i, int is_fp16) {
  const uint16_t b = p[i];
  if (is_fp16) return __half2float(__ushort_as_half(b));
  return __uint_as_float((uint32_t)b << 16);
}

// round to nearest even into bf16 / fp16 bits
__device__ inline uint16_t store16(float x, int is_fp16) {
  if (is_fp16) return __half_as_ushort(__float2half_rn(x));
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));  // inf / NaN
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline float mask_bias(const void* m, int kind, int64_t off) {
  switch (kind) {
    case FFPA_MASK_BOOL_U8: return ((const uint8_t*)m)[off] ? 0.f : -INFINITY;
    case FFPA_MASK_ADD_F32: return ((const float*)m)[off];
    case FFPA_MASK_ADD_BF16: return __uint_as_float((uint32_t)((const uint16_t*)m)[off] << 16);
    case FFPA_MASK_ADD_FP16: return __half2float(__ushort_as_half(((const uint16_t*)m)[off]));
    default: return 0.f;
  }
}

// Delta[row] = sum_d dO[row, d] * O[row, d]: one wave per row, fp32 accumulation.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows, int D, int is_fp16) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) acc += load16(o, row * D + d, is_fp16) * load16(dout, row * D + d, is_fp16);
  for (int s = 32; s > 0; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (lane == 0) delta[row] = acc;
}

// A chunk of nh consecutive query heads (flat index b * Hq + h), the first being fh0.
struct GroupArgs {
  int fh0, nh, Hq, Nq, Nkv;
  float scale;
  int causal, is_fp16;
  const float* lse;    // [B, Hq, Nq]
  const float* delta;  // [B, Hq, Nq]
  const void* mask;
  int mask_kind;
  int64_t msb, msh, msq;
  const uint32_t* keep;  // dropout keep words [B, Hq, Nq, keep_w] (null: no dropout)
  int keep_w;
  float drop_scale;      // 1 / (1 - p)
  int keep_ds;           // also keep the logits' gradient P (dP - Delta) in f32, over dP
};

// The dropout factor M of (row r of query head h, key k): keep bit / (1 - p).
__device__ inline float drop_factor(const GroupArgs& g, int fh, int r, int k) {
  const uint32_t w = g.keep[((int64_t)fh * g.Nq + r) * g.keep_w + (k >> 5)];
  return ((w >> (k & 31)) & 1u) ? g.drop_scale : 0.f;
}

// P = exp(scale S + bias - LSE) over [nh, Nq, Nkv] in place (f32), plus its 16-bit copy.
__global__ __launch_bounds__(256) void bwd_probs_kernel(float* __restrict__ s, uint16_t* __restrict__ p16, GroupArgs g) {
  const int64_t total = (int64_t)g.nh * g.Nq * g.Nkv;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int k = (int)(i % g.Nkv);
  const int64_t gr = i / g.Nkv;
  const int r = (int)(gr % g.Nq);
  const int fh = g.fh0 + (int)(gr / g.Nq);  // flat query head
  const int b = fh / g.Hq, h = fh % g.Hq;
  const float lse = g.lse[(int64_t)fh * g.Nq + r];
  float p = 0.f;
  const bool visible = !g.causal || k <= r + (g.Nkv - g.Nq);
  if (visible && lse != -INFINITY) {
    float x = g.scale * s[i];
    if (g.mask_kind != FFPA_MASK_NONE) x += mask_bias(g.mask, g.mask_kind, b * g.msb + h * g.msh + r * g.msq + k);
    p = exp2f((x - lse) * kLog2eB);
  }
  s[i] = p;
  p16[i] = store16(g.keep != nullptr ? p * drop_factor(g, fh, r, k) : p, g.is_fp16);
}

// dS = scale P (dP - Delta) as 16-bit, over [nh, Nq, Nkv]; with keep_ds, dP[i] becomes P (dP - Delta).
__global__ __launch_bounds__(256) void bwd_ds_kernel(const float* __restrict__ p, float* __restrict__ dp,
                                                     uint16_t* __restrict__ ds16, GroupArgs g) {
  const int64_t total = (int64_t)g.nh * g.Nq * g.Nkv;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t gr = i / g.Nkv;
  const int r = (int)(gr % g.Nq);
  const int fh = g.fh0 + (int)(gr / g.Nq);  // flat query head
  const float dl = g.delta[(int64_t)fh * g.Nq + r];
  const float dpm = g.keep != nullptr ? dp[i] * drop_factor(g, fh, r, (int)(i % g.Nkv)) : dp[i];
  const float dsu = p[i] * (dpm - dl);
  ds16[i] = store16(g.scale * dsu, g.is_fp16);
  if (g.keep_ds) dp[i] = dsu;
}

// The additive mask's gradient, dense f32 [Bm, Hm, Nqm, Nkv] with Bm = 1 where the mask broadcasts
// over the batch (else B), Hm likewise over the heads, Nqm over the query rows.
struct MaskGradArgs {
  float* dmask;
  int bcast_b, bcast_h, bcast_q;
  int Hm, Nqm;
  int npairs;  // mask heads (b', h') that the chunk's query heads reach
  int b0;      // first batch of the chunk (batch broadcast kept, head broadcast)
};

// Mask head j of the chunk [fh0, fh0 + nh): its flat index in the mask's [Bm, Hm] and the query heads
// fh = first, first + step, ... < end that map to it.
__device__ inline void mask_pair(const GroupArgs& g, const MaskGradArgs& a, int j, int64_t& mh, int& first,
                                 int& end, int& step) {
  const int e = g.fh0 + g.nh;
  step = 1;
  if (!a.bcast_b && !a.bcast_h) {  // one query head each
    first = g.fh0 + j;
    end = first + 1;
    mh = first;
  } else if (!a.bcast_b) {  // a batch's heads
    const int b = a.b0 + j;
    first = max(g.fh0, b * g.Hq);
    end = min(e, (b + 1) * g.Hq);
    mh = b;
  } else if (!a.bcast_h) {  // one head index across the chunk's batches
    first = g.fh0 + j;
    end = e;
    step = g.Hq;
    mh = first % g.Hq;
  } else {  // every head of the chunk
    first = g.fh0;
    end = e;
    mh = 0;
  }
}

// dmask[mh, r', k] += sum over the chunk's query heads mapping to mh (and over the rows if the mask
// broadcasts over them) of the logits' gradient kept by bwd_ds_kernel in dsu [nh, Nq, Nkv].
__global__ __launch_bounds__(256) void bwd_mask_grad_kernel(const float* __restrict__ dsu, GroupArgs g, MaskGradArgs a) {
  const int64_t per_pair = (int64_t)a.Nqm * g.Nkv;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.npairs * per_pair) return;
  const int j = (int)(i / per_pair);
  const int rq = (int)((i % per_pair) / g.Nkv);
  const int k = (int)(i % g.Nkv);
  int64_t mh;
  int first, end, step;
  mask_pair(g, a, j, mh, first, end, step);
  const int r0 = a.bcast_q ? 0 : rq, r1 = a.bcast_q ? g.Nq : rq + 1;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int fh = first; fh < end; fh += step) {
    const float* src = dsu + ((int64_t)(fh - g.fh0) * g.Nq) * g.Nkv + k;
    int r = r0;
    for (; r + 4 <= r1; r += 4)
      for (int u = 0; u < 4; ++u) acc[u] += src[(int64_t)(r + u) * g.Nkv];
    for (; r < r1; ++r) acc[0] += src[(int64_t)r * g.Nkv];
  }
  float* dst = a.dmask + (mh * a.Nqm + rq) * g.Nkv + k;
  *dst += (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

// out[j] = 16-bit(sum over the G heads of acc[g * n + j]), j < n.
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ acc, uint16_t* __restrict__ out,
                                                            int64_t n, int G, int is_fp16) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  float s = 0.f;
  for (int g = 0; g < G; ++g) s += acc[g * n + j];
  out[j] = store16(s, is_fp16);
}

// One library handle per device, created on first use and kept for the process (the handle owns
// the library's own workspace); calls are serialised because a handle's stream is shared state.
std::mutex g_handle_mu;
rocblas_handle g_handles[64];

rocblas_handle handle_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (g_handles[dev] == nullptr && rocblas_create_handle(&g_handles[dev]) != rocblas_status_success)
    g_handles[dev] = nullptr;
  return g_handles[dev];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Workspace {
  size_t delta, s, dp, p16, dk, dv, total;
};

// Query heads per chunk: a KV group (G > 1), or without grouping as many heads as keep the chunk's
// score matrices and accumulators within 4 GiB (at least one).
int64_t chunk_heads(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D) {
  const int64_t G = Hq / Hkv;
  if (G > 1) return G;
  const int64_t per_head = Nq * Nkv * 10 + Nkv * D * 8;
  int64_t n = (4LL << 30) / per_head;
  n = n < 1 ? 1 : n;
  return n < B * Hq ? n : B * Hq;
}

Workspace layout(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D) {
  const int64_t G = chunk_heads(B, Hq, Hkv, Nq, Nkv, D);  // heads per chunk
  Workspace w{};
  size_t off = 0;
  w.delta = off;
  off += align256((size_t)(B * Hq * Nq) * 4);
  w.s = off;
  off += align256((size_t)(G * Nq * Nkv) * 4);
  w.dp = off;
  off += align256((size_t)(G * Nq * Nkv) * 4);
  w.p16 = off;
  off += align256((size_t)(G * Nq * Nkv) * 2);
  w.dk = off;
  off += align256((size_t)(G * Nkv * D) * 4);
  w.dv = off;
  off += align256((size_t)(G * Nkv * D) * 4);
  w.total = off;
  return w;
}

int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              const ffpa_mask_t* mask, const void* dq, const void* dk, const void* dv, int64_t B, int64_t Hq,
              int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype) {
  ffpa::clear_failure();
  if (dtype != FFPA_BF16 && dtype != FFPA_FP16) return bfail(FFPA_ERR_TYPE, "dtype %d is neither bf16 nor fp16", dtype);
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1) return bfail(FFPA_ERR_VALUE, "every size must be >= 1");
  if (Hq % Hkv != 0) return bfail(FFPA_ERR_VALUE, "Hq must be a multiple of Hkv");
  if (is_causal != 0 && is_causal != 1) return bfail(FFPA_ERR_VALUE, "is_causal must be 0 or 1");
  if (is_causal && Nkv < Nq) return bfail(FFPA_ERR_VALUE, "causal attention needs Nkv >= Nq");
  if (std::isinf(scale)) return bfail(FFPA_ERR_VALUE, "scale must be finite (NaN selects 1/sqrt(D))");
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return bfail(FFPA_ERR_VALUE, "q, k, v, o, dout, lse, dq, dk and dv must be non-null");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk |
       (uintptr_t)dv) & 15)
    return bfail(FFPA_ERR_VALUE, "tensors must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return bfail(FFPA_ERR_VALUE, "lse must be 4-byte aligned");
  if (D < 64 || D > 1024 || D % 64 != 0)
    return bfail(FFPA_ERR_UNSUPPORTED, "head dim %lld: 64 <= D <= 1024 with D %% 64 == 0", (long long)D);
  // the elementwise kernels take one thread per score of a chunk: at most 2^32 threads per launch
  if (Nq >= (1LL << 30) || Nkv >= (1LL << 30) || (Hq / Hkv) * Nq * Nkv > (1LL << 32) - 256 || Nkv * D >= (1LL << 31))
    return bfail(FFPA_ERR_UNSUPPORTED, "sizes beyond the backward's indexing");
  if (mask != nullptr && mask->kind != FFPA_MASK_NONE) {
    if (mask->kind < FFPA_MASK_BOOL_U8 || mask->kind > FFPA_MASK_ADD_FP16)
      return bfail(FFPA_ERR_TYPE, "unknown mask kind %d", (int)mask->kind);
    if (mask->data == nullptr) return bfail(FFPA_ERR_VALUE, "mask data is null");
    if (mask->stride_k != 1) return bfail(FFPA_ERR_UNSUPPORTED, "mask stride_k must be 1");
    if (mask->stride_b < 0 || mask->stride_h < 0 || mask->stride_q < 0)
      return bfail(FFPA_ERR_VALUE, "mask strides must be >= 0");
  }
  return FFPA_OK;
}

}  // namespace

extern "C" {

size_t ffpa_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1 || Hq % Hkv != 0) return 0;
  return layout(B, Hq, Hkv, Nq, Nkv, D).total;
}

static int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream, const uint32_t* keep, float dropout_p,
                    float* dmask = nullptr) {
  const Workspace w = layout(B, Hq, Hkv, Nq, Nkv, D);
  if (workspace == nullptr || workspace_bytes < w.total || ((uintptr_t)workspace & 255))
    return bfail(FFPA_ERR_VALUE, "workspace must be 256-byte aligned and hold ffpa_bwd_workspace_size() = %zu bytes",
                 w.total);
  const hipStream_t s = (hipStream_t)stream;
  const int is_fp16 = dtype == FFPA_FP16;
  const int G = (int)(Hq / Hkv);
  const int64_t chunk = chunk_heads(B, Hq, Hkv, Nq, Nkv, D);
  const double sc = std::isnan(scale) ? 1.0 / std::sqrt((double)D) : (double)scale;
  char* ws = (char*)workspace;
  float* delta = (float*)(ws + w.delta);
  float* S = (float*)(ws + w.s);
  float* dP = (float*)(ws + w.dp);
  uint16_t* P16 = (uint16_t*)(ws + w.p16);
  float* dKacc = (float*)(ws + w.dk);
  float* dVacc = (float*)(ws + w.dv);

  MaskGradArgs ma{};
  if (dmask != nullptr) {
    ma.dmask = dmask;
    ma.bcast_b = mask->stride_b == 0;
    ma.bcast_h = mask->stride_h == 0;
    ma.bcast_q = mask->stride_q == 0;
    ma.Hm = ma.bcast_h ? 1 : (int)Hq;
    ma.Nqm = ma.bcast_q ? 1 : (int)Nq;
    const int64_t n = (ma.bcast_b ? 1 : B) * ma.Hm * ma.Nqm * Nkv;
    hipLaunchKernelGGL(bwd_fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dmask, n);
  }

  const int64_t rows = B * Hq * Nq;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const uint16_t*)o,
                     (const uint16_t*)dout, delta, rows, (int)D, is_fp16);
  if (hipGetLastError() != hipSuccess) return bfail(FFPA_ERR_HIP, "kernel launch failed");

  std::lock_guard<std::mutex> lock(g_handle_mu);
  rocblas_handle hnd = handle_for_current_device();
  if (hnd == nullptr) return bfail(FFPA_ERR_HIP, "could not create the GEMM library handle");
  if (rocblas_set_stream(hnd, s) != rocblas_status_success) return bfail(FFPA_ERR_HIP, "could not set the stream");
  const rocblas_datatype t16 = is_fp16 ? rocblas_datatype_f16_r : rocblas_datatype_bf16_r;
  const rocblas_datatype f32 = rocblas_datatype_f32_r;
  const float one = 1.f, zero = 0.f;
  const int n = (int)Nq, m = (int)Nkv, d = (int)D;
  const int64_t qh = Nq * D, kh = Nkv * D, sq = Nq * Nkv;
  // Row-major X[r][c] is the column-major X^T: every product below is written for column-major
  // operands (the library's convention) as the transpose of the row-major one.
  auto gemm = [&](rocblas_operation ta, rocblas_operation tb, int M, int N, int K, const void* A, rocblas_datatype at,
                  int lda, int64_t sa, const void* Bm, rocblas_datatype bt, int ldb, int64_t sb, void* C,
                  rocblas_datatype ct, int ldc, int64_t scs, int batch) {
    return rocblas_gemm_strided_batched_ex(hnd, ta, tb, M, N, K, &one, A, at, lda, sa, Bm, bt, ldb, sb, &zero, C, ct, ldc,
                                           scs, C, ct, ldc, scs, batch, f32, rocblas_gemm_algo_standard, 0, 0);
  };
  const rocblas_operation N_ = rocblas_operation_none, T_ = rocblas_operation_transpose;
  // Chunks: one KV group (G > 1; its K/V shared by the group's heads through a zero stride), or,
  // without grouping, `chunk` consecutive heads (head u reads KV head u, stride kh).
  const int64_t units = B * Hq;  // flat query heads b * Hq + h
  const int64_t step = G > 1 ? G : chunk;
  const int64_t kvs = G > 1 ? 0 : kh;
  for (int64_t u0 = 0; u0 < units; u0 += step) {
    const int nh = (int)(units - u0 < step ? units - u0 : step);
    const int64_t fkv = u0 / G;  // flat KV head of the chunk's first query head
    const uint16_t* Qg = (const uint16_t*)q + u0 * qh;
    const uint16_t* dOg = (const uint16_t*)dout + u0 * qh;
    uint16_t* dQg = (uint16_t*)dq + u0 * qh;
    const uint16_t* Kh = (const uint16_t*)k + fkv * kh;
    const uint16_t* Vh = (const uint16_t*)v + fkv * kh;
    GroupArgs ga{};
    ga.fh0 = (int)u0;
    ga.nh = nh;
    ga.Hq = (int)Hq;
    ga.Nq = n;
    ga.Nkv = m;
    ga.scale = (float)sc;
    ga.causal = is_causal;
    ga.is_fp16 = is_fp16;
    ga.lse = lse;
    ga.delta = delta;
    if (keep != nullptr) {
      ga.keep = keep;
      ga.keep_w = (int)((Nkv + 31) / 32);
      ga.drop_scale = (float)(1.0 / (1.0 - (double)dropout_p));
    }
    if (mask != nullptr && mask->kind != FFPA_MASK_NONE) {
      ga.mask = mask->data;
      ga.mask_kind = mask->kind;
      ga.msb = mask->stride_b;
      ga.msh = mask->stride_h;
      ga.msq = mask->stride_q;
    }
    ga.keep_ds = dmask != nullptr;
    const unsigned eblocks = (unsigned)(((int64_t)nh * sq + 255) / 256);
    rocblas_status r;
    // S^T[Nkv x Nq] = K Q^T  (per head of the chunk)
    r = gemm(T_, N_, m, n, d, Kh, t16, d, kvs, Qg, t16, d, qh, S, f32, m, sq, nh);
    if (r != rocblas_status_success) return bfail(FFPA_ERR_HIP, "GEMM S failed (%d)", (int)r);
    hipLaunchKernelGGL(bwd_probs_kernel, dim3(eblocks), dim3(256), 0, s, S, P16, ga);
    // dV_h^T[D x Nkv] = dO^T P
    r = gemm(N_, T_, d, m, n, dOg, t16, d, qh, P16, t16, m, sq, dVacc, f32, d, kh, nh);
    if (r != rocblas_status_success) return bfail(FFPA_ERR_HIP, "GEMM dV failed (%d)", (int)r);
    // dP^T[Nkv x Nq] = V dO^T
    r = gemm(T_, N_, m, n, d, Vh, t16, d, kvs, dOg, t16, d, qh, dP, f32, m, sq, nh);
    if (r != rocblas_status_success) return bfail(FFPA_ERR_HIP, "GEMM dP failed (%d)", (int)r);
    hipLaunchKernelGGL(bwd_ds_kernel, dim3(eblocks), dim3(256), 0, s, S, dP, P16, ga);
    if (dmask != nullptr) {
      const int e = (int)u0 + nh;
      if (!ma.bcast_b && !ma.bcast_h) ma.npairs = nh;
      else if (!ma.bcast_b) ma.b0 = (int)(u0 / Hq), ma.npairs = (int)((e - 1) / Hq) - ma.b0 + 1;
      else if (!ma.bcast_h) ma.npairs = nh < Hq ? nh : (int)Hq;
      else ma.npairs = 1;
      const int64_t nt = (int64_t)ma.npairs * ma.Nqm * Nkv;
      hipLaunchKernelGGL(bwd_mask_grad_kernel, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, dP, ga, ma);
    }
    // dQ^T[D x Nq] = K^T dS^T, written in the output dtype
    r = gemm(N_, N_, d, n, m, Kh, t16, d, kvs, P16, t16, m, sq, dQg, t16, d, qh, nh);
    if (r != rocblas_status_success) return bfail(FFPA_ERR_HIP, "GEMM dQ failed (%d)", (int)r);
    // dK_h^T[D x Nkv] = Q^T dS
    r = gemm(N_, T_, d, m, n, Qg, t16, d, qh, P16, t16, m, sq, dKacc, f32, d, kh, nh);
    if (r != rocblas_status_success) return bfail(FFPA_ERR_HIP, "GEMM dK failed (%d)", (int)r);
    // dK, dV: the group's G partials summed (G > 1), or the chunk's heads converted (G = 1)
    const int64_t nout = G > 1 ? kh : (int64_t)nh * kh;
    const int nsum = G > 1 ? G : 1;
    const unsigned kblocks = (unsigned)((nout + 255) / 256);
    hipLaunchKernelGGL(bwd_group_sum_kernel, dim3(kblocks), dim3(256), 0, s, dKacc, (uint16_t*)dk + fkv * kh, nout,
                       nsum, is_fp16);
    hipLaunchKernelGGL(bwd_group_sum_kernel, dim3(kblocks), dim3(256), 0, s, dVacc, (uint16_t*)dv + fkv * kh, nout,
                       nsum, is_fp16);
    if (hipGetLastError() != hipSuccess) return bfail(FFPA_ERR_HIP, "kernel launch failed");
  }
  return FFPA_OK;
}

int ffpa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
             int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, void* workspace, size_t workspace_bytes,
             void* stream) {
  const int st = bwd_check(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  return bwd_impl(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype, workspace,
                  workspace_bytes, stream, nullptr, 0.f);
}

int ffpa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, const uint32_t* keep,
                     float dropout_p, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = bwd_check(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  if (!(dropout_p >= 0.f && dropout_p < 1.f)) return bfail(FFPA_ERR_VALUE, "dropout probability must lie in [0, 1)");
  if (keep == nullptr || ((uintptr_t)keep & 3)) return bfail(FFPA_ERR_VALUE, "keep must be non-null and 4-byte aligned");
  return bwd_impl(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype, workspace,
                  workspace_bytes, stream, keep, dropout_p);
}

int ffpa_bwd_mask_grad(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                       const ffpa_mask_t* mask, void* dq, void* dk, void* dv, float* dmask, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype,
                       const uint32_t* keep, float dropout_p, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = bwd_check(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  if (mask == nullptr || mask->kind == FFPA_MASK_NONE || mask->kind == FFPA_MASK_BOOL_U8)
    return bfail(FFPA_ERR_VALUE, "the mask's gradient needs an additive (float32, bf16 or fp16) mask");
  if (dmask == nullptr || ((uintptr_t)dmask & 3)) return bfail(FFPA_ERR_VALUE, "dmask must be non-null and 4-byte aligned");
  if (B * Hq >= (1LL << 31)) return bfail(FFPA_ERR_UNSUPPORTED, "B * Hq beyond the mask gradient's indexing");
  if (keep == nullptr) {
    if (dropout_p != 0.f) return bfail(FFPA_ERR_VALUE, "dropout_p must be 0 without keep words");
  } else {
    if (!(dropout_p >= 0.f && dropout_p < 1.f)) return bfail(FFPA_ERR_VALUE, "dropout probability must lie in [0, 1)");
    if ((uintptr_t)keep & 3) return bfail(FFPA_ERR_VALUE, "keep must be 4-byte aligned");
  }
  return bwd_impl(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype, workspace,
                  workspace_bytes, stream, keep, dropout_p, dmask);
}

}  // extern "C"

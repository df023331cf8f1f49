// Backward of the attention forward (ffpa-attn "API Reference": ffpa_attn_func's backward, which
// the pages run as SDPA's backward): dQ, dK, dV (and, on request, the additive mask's gradient)
// from Q, K, V, O, dO and the forward's fp32 LSE.
//
//   Delta = rowsum(dO * O)       one wave per row (below), into the caller's workspace
//   dK, dV                       fused kernel, KV-stationary: P and dS recomputed per tile
//   dQ (and dMask)               fused kernel, Q-stationary
// The fused kernels (ffpa_bwd_kernel.hpp) recompute P = exp(scale S + bias - LSE) from the
// forward's LSE, so no score matrix is ever stored.  With attention dropout (ffpa_bwd_dropout:
// O = (P * M) V with M = keep / (1 - p) a constant) dV takes P * M and dS = P (dP M - Delta), with
// Delta = rowsum(dO * O) of the dropped-out O.  The additive mask's gradient is the logits'
// gradient P (dP - Delta) summed over the dimensions the mask broadcasts.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/ffpa.h"
#include "ffpa_bwd_launch.hpp"

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


__device__ inline float load16(const uint16_t* p, int64_t i, int is_fp16) {
  const uint16_t b = p[i];
  if (is_fp16) return __half2float(__ushort_as_half(b));
  return __uint_as_float((uint32_t)b << 16);
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

__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ffpa_bwd_noalloc's Delta buffer: a device array in the code object (each GPU holds its own copy
// for as long as the library is loaded), 4 Mi rows = 16 MiB.  Host code reaches it only through
// the address hipGetSymbolAddress returns for the current device.
constexpr int64_t kNoAllocRows = 1LL << 22;
static __device__ __align__(256) float scratch[kNoAllocRows];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device, set on the first call there

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
  if (D < 8 || D > 1024 || D % 8 != 0)
    return bfail(FFPA_ERR_UNSUPPORTED, "head dim %lld: 8 <= D <= 1024 with D %% 8 == 0", (long long)D);
  // 32-bit row indexing and buffer offsets of one head (rows up to 64 past its end included); each
  // factor bounded first, so that no product overflows
  if (Nq >= (1LL << 31) || Nkv >= (1LL << 31) || B >= (1LL << 31) || Hq >= (1LL << 31) ||
      (Nq + 64) * D >= (1LL << 31) || (Nkv + 64) * D >= (1LL << 31) || B * Hq >= (1LL << 31))
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
  if (B >= (1LL << 31) || Hq >= (1LL << 31) || Nq >= (1LL << 31) || B * Hq >= (1LL << 31)) return 0;
  return align256((size_t)(B * Hq * Nq) * 4);  // Delta
}

}  // extern "C"

namespace {

template <typename T>
hipError_t launch_fused(int kd, bool pad, const ffpa::BwdArgs& a, hipStream_t s) {
  switch (kd) {
#define FFPA_BWD_CASE_PAD(KDv) \
  case KDv: return pad ? ffpa::launch_bwd_fused<T, KDv, true>(a, s) : ffpa::launch_bwd_fused<T, KDv, false>(a, s);
    FFPA_BWD_CASE_PAD(64) FFPA_BWD_CASE_PAD(128) FFPA_BWD_CASE_PAD(192) FFPA_BWD_CASE_PAD(256)
    FFPA_BWD_CASE_PAD(320) FFPA_BWD_CASE_PAD(384) FFPA_BWD_CASE_PAD(448) FFPA_BWD_CASE_PAD(512)
    FFPA_BWD_CASE_PAD(640) FFPA_BWD_CASE_PAD(768) FFPA_BWD_CASE_PAD(896) FFPA_BWD_CASE_PAD(1024)
#undef FFPA_BWD_CASE_PAD
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

static int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream, const uint32_t* keep, float dropout_p,
                    float* dmask = nullptr) {
  const size_t need = ffpa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return bfail(FFPA_ERR_VALUE, "workspace must be 256-byte aligned and hold ffpa_bwd_workspace_size() = %zu bytes",
                 need);
  const hipStream_t s = (hipStream_t)stream;
  const int is_fp16 = dtype == FFPA_FP16;
  float* delta = (float*)workspace;

  ffpa::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  if (mask != nullptr && mask->kind != FFPA_MASK_NONE) {
    a.mask = mask->data;
    a.mask_kind = mask->kind;
    a.msb = mask->stride_b;
    a.msh = mask->stride_h;
    a.msq = mask->stride_q;
  }
  if (dmask != nullptr) {
    a.dmask = dmask;
    a.dm_bb = mask->stride_b == 0;
    a.dm_bh = mask->stride_h == 0;
    a.dm_bq = mask->stride_q == 0;
    a.dm_hm = a.dm_bh ? 1 : (int)Hq;
    a.dm_nqm = a.dm_bq ? 1 : (int)Nq;
    a.dm_atomic = (a.dm_bb && B > 1) || (a.dm_bh && Hq > 1) || (a.dm_bq && Nq > 1);
    const int64_t n = (a.dm_bb ? 1 : B) * a.dm_hm * a.dm_nqm * Nkv;
    hipLaunchKernelGGL(bwd_fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dmask, n);
  }
  if (keep != nullptr) {
    a.keep = keep;
    a.keep_w = (int)((Nkv + 31) / 32);
    a.drop_scale = (float)(1.0 / (1.0 - (double)dropout_p));
  }
  a.B = (int)B;
  a.Hq = (int)Hq;
  a.Hkv = (int)Hkv;
  a.Nq = (int)Nq;
  a.Nkv = (int)Nkv;
  a.D = (int)D;
  a.scale = (float)(std::isnan(scale) ? 1.0 / std::sqrt((double)D) : (double)scale);
  a.causal = is_causal;

  const int64_t rows = B * Hq * Nq;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const uint16_t*)o,
                     (const uint16_t*)dout, delta, rows, (int)D, is_fp16);
  if (hipGetLastError() != hipSuccess) return bfail(FFPA_ERR_HIP, "kernel launch failed");
  const int kd = ffpa::bwd_kernel_dim((int)D);
  const hipError_t e = is_fp16 ? launch_fused<ffpa::Fp16>(kd, kd != D, a, s) : launch_fused<ffpa::Bf16>(kd, kd != D, a, s);
  if (e != hipSuccess) return bfail(FFPA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
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

int ffpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     const ffpa_mask_t* mask, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nkv, int64_t D, float scale, int is_causal, int dtype, void* stream) {
  const int st = bwd_check(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype);
  if (st != FFPA_OK) return st;
  if (B * Hq * Nq > kNoAllocRows)
    return bfail(FFPA_ERR_UNSUPPORTED, "B * Hq * Nq = %lld query rows exceed the %lld of the built-in buffer",
                 (long long)(B * Hq * Nq), (long long)kNoAllocRows);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return bfail(FFPA_ERR_HIP, "no current device");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return bfail(FFPA_ERR_HIP, "could not find the built-in buffer's address: %s", hipGetErrorString(e));
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  return bwd_impl(q, k, v, o, dout, lse, mask, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, is_causal, dtype, ws,
                  (size_t)kNoAllocRows * 4, stream, nullptr, 0.f);
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

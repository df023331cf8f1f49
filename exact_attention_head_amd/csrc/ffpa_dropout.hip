// Keep decisions of attention dropout (declared in include/ffpa.h as ffpa_dropout_keep).
//
// The ffpa-attn "API Reference" page gives ffpa_attn_func a dropout_p parameter and calls the
// dropout SDPA-style: each attention weight is kept independently with probability 1 - p.  The
// decisions come from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), restated here from that definition:
// ten rounds over a 128-bit counter under a 64-bit key; a round takes the full 64-bit products of
// counter words 0 and 2 with the two round multipliers and mixes their halves with counter words
// 1 and 3 and the key; the key moves by the two Weyl increments between rounds.
//
// Layout and stream assignment (this library's own choice): keep is [B, Hq, Nq, W] 32-bit words,
// W = ceil(Nkv / 32); bit i of word w keeps key 32 w + i.  For row index R = (b Hq + h) Nq + r the
// word draws the eight blocks with counters (8 w + j, R mod 2^32, R div 2^32, offset), j < 8, under
// key (seed mod 2^32, seed div 2^32); output i of block j decides key 32 w + 4 j + i, kept when it
// is at least floor(p 2^32).  Bits of keys at or past Nkv are 0.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/ffpa.h"

namespace ffpa {
int report_failure(int status, const char* msg);
void clear_failure();
}  // namespace ffpa

namespace {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;  // round multipliers
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;  // key increments

struct U4 {
  uint32_t x, y, z, w;
};

__device__ inline U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint32_t lo0 = kPhiloxM0 * c.x, hi0 = __umulhi(kPhiloxM0, c.x);
    const uint32_t lo1 = kPhiloxM1 * c.z, hi1 = __umulhi(kPhiloxM1, c.z);
    c = U4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

// One thread per keep word: words are consecutive in memory across the threads of a wave.
__global__ __launch_bounds__(256) void ffpa_dropout_keep_kernel(uint32_t* keep, int64_t words, int W, int Nkv,
                                                                 uint32_t thr, uint32_t k0, uint32_t k1,
                                                                 uint32_t offset) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= words) return;
  const int64_t R = idx / W;
  const int w = (int)(idx - R * W);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const U4 u = philox4x32_10(U4{(uint32_t)(8 * w + j), (uint32_t)R, (uint32_t)((uint64_t)R >> 32), offset}, k0, k1);
    word |= (uint32_t)(u.x >= thr) << (4 * j);
    word |= (uint32_t)(u.y >= thr) << (4 * j + 1);
    word |= (uint32_t)(u.z >= thr) << (4 * j + 2);
    word |= (uint32_t)(u.w >= thr) << (4 * j + 3);
  }
  const int valid = Nkv - 32 * w;  // keys of this word below Nkv
  if (valid < 32) word &= (1u << valid) - 1u;
  keep[idx] = word;
}

}  // namespace

extern "C" {

int ffpa_dropout_keep(uint32_t* keep, int64_t B, int64_t Hq, int64_t Nq, int64_t Nkv, float p, uint64_t seed,
                      uint32_t offset, void* stream) {
  ffpa::clear_failure();
  if (B < 1 || Hq < 1 || Nq < 1 || Nkv < 1) return ffpa::report_failure(FFPA_ERR_VALUE, "every size must be >= 1");
  if (!(p >= 0.f && p < 1.f)) return ffpa::report_failure(FFPA_ERR_VALUE, "dropout probability must lie in [0, 1)");
  if (keep == nullptr || ((uintptr_t)keep & 3)) return ffpa::report_failure(FFPA_ERR_VALUE, "keep must be non-null and 4-byte aligned");
  if (Nkv > (1LL << 30)) return ffpa::report_failure(FFPA_ERR_UNSUPPORTED, "Nkv beyond 32-bit indexing");
  const int64_t W = (Nkv + 31) / 32;
  const int64_t rows = B * Hq * Nq;
  if (rows > (1LL << 40) || rows * W > (1LL << 40)) return ffpa::report_failure(FFPA_ERR_UNSUPPORTED, "keep mask too large");
  const int64_t words = rows * W;
  const int64_t blocks = (words + 255) / 256;
  if (blocks > 0x7fffffffLL) return ffpa::report_failure(FFPA_ERR_UNSUPPORTED, "keep mask too large");
  // floor(p * 2^32): exact in double for a float p in [0, 1)
  const uint32_t thr = (uint32_t)std::floor((double)p * 4294967296.0);
  hipLaunchKernelGGL(ffpa_dropout_keep_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, keep, words,
                     (int)W, (int)Nkv, thr, (uint32_t)seed, (uint32_t)(seed >> 32), offset);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ffpa::report_failure(FFPA_ERR_HIP, hipGetErrorString(e));
  return FFPA_OK;
}

}  // extern "C"

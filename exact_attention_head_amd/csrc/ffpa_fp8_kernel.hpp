// FP8 (e4m3) attention forward for gfx950: the FP8 attention of the ffpa-attn README ("Latest News",
// "End-to-End Inference"), rebuilt for the CDNA4 fp8 matrix core.
//
// Q, K and V are OCP e4m3 ("e4m3fn") codes with per-head dequantisation factors dq[b, hq], dk[b, hk]
// and dv[b, hk] (the "scale folding" of the skills page: the factors never touch the tensors; dq dk
// joins the softmax scale in the exponent's coefficient and dv joins the final 1/l).  O is written in
// bf16 or fp16, the LSE in fp32, exactly as the 16-bit forward does:
//
//     O = softmax(scale (dq Q)(dk K)^T + mask) (dv V),   LSE = natural log-sum-exp of those logits
//
// Both products run on v_mfma_f32_32x32x64_f8f6f4 (64 cycles, twice the 16-bit rate): S^T = K Q^T with
// K from LDS and Q in VGPRs, and O^T = V^T P^T with the probabilities rounded once to e4m3 (RNE; the
// lazily moved running maximum keeps them at most 2^8, below the format's 448).  Lane l holds query
// row l % 32 in both.  The probabilities of a 64-key tile fill the B operand in the S accumulators'
// own order (byte j of the lane = element j % 16 of 32-key block j / 16), and V^T is read with
// ds_read_b64_tr_b8 in the matching key order, which the sum over keys does not care about (the
// README's reduction-axis permutation invariance).
//
// One workgroup = 4 waves.  Up to D = 512 each wave owns 32 rows and the whole O row block (32 x D
// fp32 = D / 2 AGPRs) and keeps its Q rows in VGPRs (D / 8 registers): 128 rows per workgroup.  Above,
// two waves share 32 rows and split the columns (DW = D / 2 each: the output-D split of the README's
// "Split-D and TiledMMA"), summing their partial S tiles through LDS: 64 rows per workgroup.  K and V
// stream through an LDS ring of 4 KiB groups ([32 keys][128 columns], 128-byte rows, 16-byte chunks
// swizzled as in the 16-bit kernels; one ring per column group) filled by direct-to-LDS buffer loads,
// one barrier per epoch of eight products (four with two column groups).
//
// Software pipeline.  Stage T issues S(T) (the 2 D / 64 products of tile T) and then P V of tile st - 2
// (D / 32 products).  Tile T - 1's exponentials run as small pieces between all the products of stage
// T, and tile T's logits and row maximum between the P V products, after S(T) is complete; the
// rescale of O and l for tile st - 1 closes the stage.  So the quarter-rate exponentials are spread over
// the whole 64-cycle shadow of every product instead of one phase.  S accumulators and packed
// probabilities alternate between two register sets by stage parity; n tiles take n + 2 stages (the
// first two P V phases multiply zero probabilities, the last two S phases are masked out).
#pragma once

#include <utility>

namespace ffpa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// e4m3 x e4m3 products (format fields 0 = fp8 e4m3 for both operands).  Same conventions as the 16-bit
// products above: inline assembly so that O can live in AGPRs; operands written by VALU instructions
// take s_nop 1 first.
struct Mma8 {
  __device__ static inline void first(f32x16& d, const i32x8& a, const i32x8& b) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  }
  __device__ static inline void acc(f32x16& d, const i32x8& a, const i32x8& b) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  }
  __device__ static inline void acc_agpr(f32x16& d, const i32x8& a, const i32x8& b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
  __device__ static inline void acc_agpr_nonop(f32x16& d, const i32x8& a, const i32x8& b) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  }
};
// 20 wait states after the 16-pass products that wrote this VGPR accumulator
__device__ inline void mma8_guard1(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x)); }

// Two e4m3 codes (RNE) of a and b into byte pair HI (0: bytes 0-1, 1: bytes 2-3) of word w.
template <bool HI>
__device__ inline int pack_fp8x2(float a, float b, int w) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, HI);
}

template <int D>
struct Fp8Tiling {
  static constexpr int DG = D > 512 ? 2 : 1;   // column groups: waves sharing 32 rows (O is D/2 AGPRs per wave)
  static constexpr int DW = D / DG;            // output columns per wave
  static constexpr int NS = DW / 64;           // 64-column steps: S products per 32-key block
  static constexpr int PS = 2 * NS;            // S products per stage
  static constexpr int NPV = DW / 32;          // P V products per stage (one per 32 output columns)
  static constexpr int MPT = PS + NPV;         // products per stage
  static constexpr int NCGW = DW / 128;        // 128-column groups of one column group
  static constexpr int GTW = 4 * NCGW;         // 4 KiB groups per stage of one column group: K, then V
  static constexpr int GT = DG * GTW;          // groups per stage
  static constexpr int RS = DG == 2 ? 1 : (GT <= 4 ? 8 : (GT <= 8 ? 4 : 2));  // stages per turn of the ring
  // products per epoch: the longest of 16, 8 and 4 that divides the stage and leaves the ring four
  // epochs, two of them lookahead (16 at D = 256 and 512, 8 at 128, 384 and 1024, 4 at 768); halving
  // the barriers measured 2.5% faster at D = 256, 4.5% at 512 and 7.5% at 1024
  static constexpr int EM = (MPT % 16 == 0 && RS * GT / (DG * 8) >= 4) ? 16 : (RS * GT / (DG * 4) >= 4 ? 8 : 4);
  static constexpr int BIW = EM / 2;           // groups per epoch of one column group
  static constexpr int BI = DG * BIW;          // groups per epoch
  static constexpr int EPT = MPT / EM;         // epochs per stage
  static constexpr int UNR = RS % 2 ? 2 * RS : RS;  // stages per loop iteration (even: the stage parity)
  static constexpr int CGB = RS * GTW * 4096;  // ring bytes of one column group ([column group][slot][4 KiB])
  static constexpr int NG = RS * GT;           // ring groups
  static constexpr int NE = NG / BI;           // epochs held by the ring
  static constexpr int LA = NE - 2;            // epochs of load lookahead
  static constexpr int BR = 128 / DG;          // query rows per workgroup
  static constexpr int EXCH = DG == 2 ? 4 * 8192 : 0;  // partial S exchange: [wave][32-key block][4 KiB]
  static constexpr int LDS_RING = NG * 4096 + EXCH;
  // the epilogue stages each wave's O block (32 rows x DW 16-bit columns) through LDS
  static constexpr int LDS_BYTES = LDS_RING > 4 * o_stage_bytes<DW>() ? LDS_RING : 4 * o_stage_bytes<DW>();
  static constexpr bool OK = D % 128 == 0 && D >= 128 && D <= 1024 && DW % 128 == 0;
};

// Operand fragments are read this many products ahead of their use.
constexpr int kFp8PF = 3;
// LDS instructions of the fragment read of product m (two 16-byte reads for K, four transposed reads
// for V^T).
constexpr int fp8_reads(int m, int MPT, int PS) { return (m % MPT) < PS ? 2 : 4; }

// Tile variants: kFp8Raw (no mask, no causal limit, whole tiles, positive scale: the maximum is taken
// over the raw products and the coefficient folded into the exponent), kFp8Edge (no mask; explicit
// logits with -inf past Nkv or the causal limit) and kFp8Mask (the same plus a mask bias, loaded one
// 32-key block at a time so that its registers are live only around that block's logits).
enum Fp8Mode { kFp8Mask = 0, kFp8Raw = 1, kFp8Edge = 2 };

// Slot of exponential piece k (0..31) of the previous tile within a stage.
constexpr int fp8_exp_slot(int k, int MPT) { return 1 + (k * (MPT - 3)) / 32; }
// First slot at which block kb's logits can be formed.  One column group: the slot after its last S
// product.  Two: the partial S is published in that slot, becomes visible at the next epoch barrier,
// and the partner's partial read right after it is complete PF products later.
constexpr int fp8_block_first(int kb, int DG, int NS, int EM, int PF) {
  const int w = (kb + 1) * NS;
  if (DG == 1) return w + 1;
  int bs = w;
  while ((bs + PF) % EM != 0) ++bs;
  return bs + PF;
}
constexpr int fp8_block_barrier(int kb, int NS, int EM, int PF) {
  int bs = (kb + 1) * NS;
  while ((bs + PF) % EM != 0) ++bs;
  return bs;
}
// Logit pieces of one 32-key block of the current tile (4 raw maxima of 4 products, or 8 explicit
// pieces of 2 logits).  Block 0's run from its first slot up to block 1's; block 1's, then the
// cross-half maximum and the decision, from its first slot to MPT - 2.
constexpr int fp8_block_pieces(bool raw) { return raw ? 4 : 8; }
constexpr int fp8_logit_slot(int kb, int k, int DG, int NS, int MPT, int EM, int PF, bool raw) {
  const int f0 = fp8_block_first(0, DG, NS, EM, PF), f1 = fp8_block_first(1, DG, NS, EM, PF);
  return kb == 0 ? f0 + (k * (f1 - f0)) / fp8_block_pieces(raw)
                 : f1 + (k * (MPT - 1 - f1)) / (fp8_block_pieces(raw) + 2);
}

template <typename T, int D, int MODE, int MK = kMaskNone>
__global__ __launch_bounds__(256) void ffpa_fwd_fp8_kernel(FwdArgs a) {
  using FT = Fp8Tiling<D>;
  static_assert(FT::OK, "fp8 head dims: 128, 256, 384, 512, 768, 1024");
  constexpr int DG = FT::DG, DW = FT::DW, NS = FT::NS, PS = FT::PS, NPV = FT::NPV, MPT = FT::MPT;
  constexpr int NCGW = FT::NCGW, GTW = FT::GTW, CGB = FT::CGB, UNR = FT::UNR;
  constexpr int EM = FT::EM, BIW = FT::BIW, BI = FT::BI, EPT = FT::EPT, RS = FT::RS, LA = FT::LA, BR = FT::BR;
  constexpr int PF = kFp8PF, NFR = 4, BC = 64;
  constexpr bool RAW = MODE == kFp8Raw;
  constexpr bool MASK = MODE == kFp8Mask;  // mask kind MK (a template parameter: one load path per kernel)
  static_assert(!MASK || MK != kMaskNone, "masked variant needs a mask kind");
  static_assert(MPT % EM == 0 && MPT % NFR == 0 && PF < EM && LA >= 2, "stage plan");
  constexpr int NLB = fp8_block_pieces(RAW);
  constexpr int F0 = fp8_block_first(0, DG, NS, EM, PF), F1 = fp8_block_first(1, DG, NS, EM, PF);
  static_assert(NS >= 2 && F0 < F1 && fp8_logit_slot(1, NLB + 1, DG, NS, MPT, EM, PF, RAW) <= MPT - 2,
                "logit pieces fit their windows");
  static_assert(DG == 1 || (CGB <= 65536 && FT::NG * 4096 + FT::EXCH <= 160 * 1024), "LDS windows");
  static_assert(DG == 1 || fp8_block_barrier(1, NS, EM, PF) + PF < MPT, "publishing barriers inside the stage");
  constexpr int NL = BI;  // loads per wave per epoch (one per group): slot bs + 1 + (q (EM - 1)) / NL
  static_assert(1 + ((NL - 1) * (EM - 1)) / NL < EM, "the loads after a barrier end before the next one");

  __shared__ __attribute__((aligned(1024))) char smem[FT::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int dg = DG == 1 ? 0 : (wave & 1);  // column group
  const int rg = DG == 1 ? wave : (wave >> 1);  // row group
  const int col0 = dg * DW;
  clock_stamp(a.stamps, 0);

  // ---- work item (b, KV head, q tile, query head), XCD-contiguous, heaviest causal tiles first
  const int nqt = (a.Nq + BR - 1) / BR;
  const int total = a.B * a.Hq * nqt;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  // the query heads of a KV group fastest: they take the same query tile together and stream the
  // same K/V tiles at the same time
  const int g = id % a.group, rest = id / a.group;
  int qt = rest % nqt;
  const int bk = rest / nqt, hkv = a.Hkv;
  const int b = bk / hkv;
  const int hq = (bk % hkv) * a.group + g;
  if (a.causal) qt = nqt - 1 - qt;
  const int hk = hq / a.group;
  const int r0 = qt * BR;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int q_rs = a.q_sr, kv_rs = a.kv_sr, o_rs = a.o_sr;  // row strides: bytes of Q/K/V rows, O elements
  const int rw0 = r0 + rg * 32;
  const int row = rw0 + l32;
  const int off = Nkv - Nq;
  int kv_end = Nkv;
  if (a.causal) {
    const int lim = r0 + BR + off;
    kv_end = lim < Nkv ? lim : Nkv;
  }
  const int ntiles = (kv_end + BC - 1) / BC;
  const int nstages = ntiles + 2;
  const int total_epochs = nstages * EPT;

  // per-head dequantisation factors (null: 1) folded into the exponent's coefficient and into 1/l
  const float fq = a.q_desc ? a.q_desc[b * a.Hq + hq] : 1.f;
  const float fk = a.k_desc ? a.k_desc[b * a.Hkv + hk] : 1.f;
  const float fv = a.v_desc ? a.v_desc[b * a.Hkv + hk] : 1.f;
  const float coef = a.scale_log2 * fq * fk;  // logit (log2 units) = coef * raw product + bias * log2 e

  const uint8_t* qg = (const uint8_t*)a.q + (int64_t)(b * a.Hq + hq) * Nq * q_rs;
  const uint8_t* kg = (const uint8_t*)a.k + (int64_t)(b * a.Hkv + hk) * Nkv * kv_rs;
  const uint8_t* vg = (const uint8_t*)a.v + (int64_t)(b * a.Hkv + hk) * Nkv * kv_rs;

  // ---- ring loads: wave w fills rows 8w .. 8w+7 of a group (lane t: row 8w + t/8, physical chunk t%8
  // holding logical chunk (t%8) ^ pi((row >> 1) & 7)); the row part of the offset is a scalar
  auto pi7 = [](int x) { return ((x & 1) << 2) | (x >> 1); };
  const int prow = 8 * wave + (lane >> 3);
  const uint32_t voff_lane = (uint32_t)(prow * kv_rs + ((lane & 7) ^ pi7((prow >> 1) & 7)) * 16);
  const int head_bytes = (int)((int64_t)Nkv * kv_rs);
  const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, head_bytes, 0x00020000);
  char* const ring_w = smem + wave * 1024;
  // group gi of column group cg of stage st into that column group's ring slot (u * GTW + gi): K groups
  // (gi < 2 NCGW) hold key block gi / NCGW of tile min(st, n - 1), columns 128 (cg NCGW + gi % NCGW);
  // V groups hold key block gi % 2 of tile clamp(st - 2, 0, n - 1), columns 128 (cg NCGW + (gi - 2 NCGW) / 2)
  auto issue_group = [&](int st, auto u_c, auto cg_c, auto gi_c) {
    constexpr int U = decltype(u_c)::value, CGR = decltype(cg_c)::value, GI = decltype(gi_c)::value;
    constexpr bool ISK = GI < 2 * NCGW;
    constexpr int KB = ISK ? GI / NCGW : (GI - 2 * NCGW) % 2;
    constexpr int CG = CGR * NCGW + (ISK ? GI % NCGW : (GI - 2 * NCGW) / 2);
    int tile = ISK ? st : st - 2;
    tile = tile < ntiles - 1 ? tile : ntiles - 1;
    tile = tile > 0 ? tile : 0;
    const uint32_t so = (uint32_t)(tile * BC + KB * 32) * (uint32_t)kv_rs + (uint32_t)(CG * 128);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ISK ? rsrc_k : rsrc_v,
                                             (FFPA_LDS void*)(ring_w + CGR * CGB + ((U * GTW + GI) % (RS * GTW)) * 4096),
                                             16, voff_lane, so, 0, 0);
  };
  // load q of local epoch E (E >= EPT: of a later stage) of stage st, whose ring position is U: group
  // E * BIW + q % BIW of column group q / BIW
  auto issue_epoch_load = [&](int st, auto u_c, auto e_c, auto q_c) {
    constexpr int U = decltype(u_c)::value, E = decltype(e_c)::value, Q = decltype(q_c)::value;
    constexpr int SD = E / EPT, EL = E % EPT;
    if (st + SD >= nstages) return;
    issue_group(st + SD, std::integral_constant<int, (U + SD) % RS>{}, std::integral_constant<int, Q / BIW>{},
                std::integral_constant<int, EL * BIW + Q % BIW>{});
  };
  auto wait_epoch = [&](int eg) {
    if (eg + LA - 1 < total_epochs) vm_wait<(LA - 1) * NL>();
    else vm_wait<0>();
  };

  // ---- fragment addresses.  K (key block kb, step s): row l32 of group kb NCG + s / 2, logical chunks
  // 4 (s % 2) + 2 hi and + 1.  V^T (output block c, read r): row 16 (r % 2) + 4 hi + m' of group
  // 2 NCG + 2 (c / 4) + r / 2, with m' = m (m < 4) or m + 4 for m = (lane % 16) / 2, logical chunk
  // 2 (c % 4) + (lane / 16) % 2, half (lane % 2).
  const uint32_t ring_addr = lds_addr(smem);
  const uint32_t cgb = ring_addr + dg * CGB;  // this wave's column group's ring
  uint32_t ka[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int j = 0; j < 2; ++j) ka[s2][j] = cgb + l32 * 128 + ((4 * s2 + 2 * hi + j) ^ pi7((l32 >> 1) & 7)) * 16;
  uint32_t vaddr[2][4];
  {
    const int g16 = lane >> 4, i16 = lane & 15, m = i16 >> 1;
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      const int vrow = 16 * r2 + 4 * (g16 >> 1) + (m < 4 ? m : m + 4);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        vaddr[r2][c4] = cgb + vrow * 128 + ((2 * c4 + (g16 & 1)) ^ pi7((vrow >> 1) & 7)) * 16 + 8 * (i16 & 1);
    }
  }
  i32x8 fr[NFR];
  // fragment of product M of a stage at ring position U (M >= MPT: the next stage's, position U + 1)
  auto read_frag = [&](auto u_c, auto mc) {
    constexpr int M = decltype(mc)::value;
    constexpr int U = (decltype(u_c)::value + M / MPT) % RS;
    constexpr int mm = M % MPT;
    constexpr int r = M % NFR;
    if constexpr (mm < PS) {
      constexpr int kb = mm / NS, s = mm % NS;
      constexpr int ofs = ((U * GTW + kb * NCGW + s / 2) % (RS * GTW)) * 4096;
      constexpr uint32_t win = ofs >= 65536 ? 65536u : 0u;
      const i32x4 x0 = lds_read_b128_async<(ofs & 65535)>(ka[s % 2][0] + win);
      const i32x4 x1 = lds_read_b128_async<(ofs & 65535)>(ka[s % 2][1] + win);
      fr[r] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    } else {
      constexpr int c = mm - PS;
      i32x2 y[4];
      static_for<4>([&](auto rr_c) {
        constexpr int rr = decltype(rr_c)::value;
        constexpr int ofs = ((U * GTW + 2 * NCGW + 2 * (c / 4) + rr / 2) % (RS * GTW)) * 4096;
        constexpr uint32_t win = ofs >= 65536 ? 65536u : 0u;
        y[rr] = lds_read_tr8_async<(ofs & 65535)>(vaddr[rr % 2][c % 4] + win);
      });
      fr[r] = i32x8{y[0][0], y[0][1], y[1][0], y[1][1], y[2][0], y[2][1], y[3][0], y[3][1]};
    }
  };

  const int64_t mask_bh = (int64_t)b * a.msb + (int64_t)hq * a.msh;

  // partial S exchange (two column groups): [wave][block][4 x 1 KiB], 16 bytes per lane
  const uint32_t ex_mine = ring_addr + FT::NG * 4096 + wave * 8192 + lane * 16;
  const uint32_t ex_partner = ring_addr + FT::NG * 4096 + (wave ^ 1) * 8192 + lane * 16;
  f32x4 part[4];  // the partner's partial of the block being published

  // ---- prologue: the Q rows in VGPRs (step s holds bytes col0 + 64 s + 32 hi .. +31 of row l32,
  // zero past dcols), then epochs 0 .. LA-1 in flight behind them, so that the Q rows and the ring's
  // first keys are fetched together; then Q and epoch 0 visible, the first PF fragments requested
  i32x8 qf[NS];
  {
    const int qrow = row < Nq ? row : Nq - 1;
    const i32x4* src = (const i32x4*)(qg + (int64_t)qrow * q_rs + col0 + hi * 32);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = col0 + 64 * s + 32 * hi;
      const i32x4 lo = c < a.dcols ? src[4 * s] : i32x4{0, 0, 0, 0};
      const i32x4 up = c + 16 < a.dcols ? src[4 * s + 1] : i32x4{0, 0, 0, 0};
      qf[s] = i32x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    }
  }
  // the first stage's epochs are issued whether or not it exists (their tile index is clamped into
  // the head, and the wait below completes them before anything else uses the LDS): a load on one
  // path only would make the compiler wait for every load before the Q rows' use
  static_for<LA>([&](auto e_c) {
    constexpr int E = decltype(e_c)::value;
    static_for<NL>([&](auto q_c) {
      constexpr int Q = decltype(q_c)::value;
      if constexpr (E < EPT)
        issue_group(0, std::integral_constant<int, 0>{}, std::integral_constant<int, Q / BIW>{},
                    std::integral_constant<int, E * BIW + Q % BIW>{});
      else
        issue_epoch_load(0, std::integral_constant<int, 0>{}, std::integral_constant<int, E>{}, q_c);
    });
  });
  // complete here, and redefine through the assembler: the compiler then has no load of these
  // registers to wait for inside the key loop
#pragma unroll
  for (int s = 0; s < NS; ++s) asm volatile("" : "+v"(qf[s]));
  wait_epoch(0);
  __builtin_amdgcn_s_barrier();
  static_for<NL>([&](auto q_c) {
    issue_epoch_load(0, std::integral_constant<int, 0>{}, std::integral_constant<int, LA>{}, q_c);
  });
  static_for<PF>([&](auto mc) { read_frag(std::integral_constant<int, 0>{}, mc); });

  f32x16 o_acc[NPV];
#pragma unroll
  for (int c = 0; c < NPV; ++c) {
    o_acc[c] = f32x16{};
    asm volatile("" : "+a"(o_acc[c]));
  }
  // S accumulators (overwritten in place by the logits) and packed probabilities, by stage parity
  f32x16 sacc[2][2];
  i32x8 pk[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    pk[p] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[p][kb][e] = kNegInf;
  }
  float m_run = kNegInf;            // running reference maximum of this lane's row (log2 units)
  float l_lane = 0.f;               // sum of this lane's probabilities (the other half-wave holds the rest)
  float mref[2] = {0.f, 0.f};       // reference of the tile whose probabilities are formed, by parity
  float alpha[2] = {1.f, 1.f};      // rescale of O and l that tile brings
  bool need[2] = {false, false};
  float lmax = kNegInf, mt = kNegInf, m_old = kNegInf, psum = 0.f, pv3[3] = {0.f, 0.f, 0.f};
  (void)part;
  int pw = 0;
  f32x4 bias[4];  // mask biases of one 32-key block (keys 8 g + 4 hi + e)

  auto stage = [&](const int st, auto u_c) {
    constexpr int U = decltype(u_c)::value % RS;  // ring position
    constexpr int PAR = decltype(u_c)::value & 1;  // parity of st (UNR is even)
    // this stage's tile for S and logits (tiles past the last are masked out), the tile of the P V phase
    const bool live = st < ntiles;
    const int key0 = st * BC;
    const bool tail = key0 + BC > Nkv;
    const bool diag = a.causal && (key0 + BC - 1 > rw0 + off);
    const bool edge = !live || tail || diag;
    int edge_lim = Nkv - 1;  // last key of tile st this lane's row may see, relative to the tile
    if (a.causal) edge_lim = edge_lim < row + off ? edge_lim : row + off;
    edge_lim -= key0;
    if (!live) edge_lim = -1;
    LogitCtx ctx{a.mask, mask_bh, a.msq, Nq, Nkv, key0, rw0, off, a.causal, edge, a.scale_log2, l32, hi};

    // the biases of the 32 keys from kbase (four aligned vectors when the rows allow it)
    auto load_block_bias = [&](int kbase) {
      if constexpr (MASK) {
        auto& bb = *reinterpret_cast<f32x4(*)[1][4]>(&bias[0]);
        if (a.mask_vec && !tail) load_bias<MK, true, 1, 4>(bb, ctx, kbase);
        else load_bias<MK, false, 1, 4>(bb, ctx, kbase);
      }
    };
    // tile st's logits and row maximum in pieces: piece k of block kb (k < NLB), then (block 1) the
    // cross-half maximum and the decision
    auto logit_piece = [&](int kb, int k) {
      if (k < NLB) {
        if constexpr (RAW) {
          if (k == 0 && !live) {  // a tile past the last (the pipeline's tail): every key excluded
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[PAR][kb][e] = kNegInf;
          }
          float mx = kb == 0 && k == 0 ? kNegInf : lmax;
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = __builtin_fmaxf(mx, sacc[PAR][kb][4 * k + e]);
          lmax = mx;
          asm volatile("" : "+v"(sacc[PAR][kb]), "+v"(lmax));
        } else {
          const int g = k >> 1, e0 = 2 * (k & 1);
          const int lim = edge_lim - 32 * kb - 4 * hi;
          float mx = kb == 0 && k == 0 ? kNegInf : lmax;
#pragma unroll
          for (int e = e0; e < e0 + 2; ++e) {
            float x = sacc[PAR][kb][4 * g + e] * coef;
            if constexpr (MASK) x = __builtin_fmaf(bias[g][e], kLog2e, x);
            if (edge) x = 8 * g + e > lim ? kNegInf : x;
            mx = __builtin_fmaxf(mx, x);
            sacc[PAR][kb][4 * g + e] = x;
          }
          lmax = mx;
          asm volatile("" : "+v"(sacc[PAR][kb]), "+v"(lmax));
        }
      } else if (k == NLB) {
        mt = RAW ? max_halves(lmax) * coef : max_halves(lmax);
        m_old = m_run;
        asm volatile("" : "+v"(mt), "+v"(m_old));
      } else {
        const bool nd = m_old != kNegInf && mt > m_old + kRescaleSlack;
        const float mn = m_old == kNegInf ? mt : (nd ? mt : m_old);
        need[PAR] = nd;
        m_run = mn;
        mref[PAR] = mn == kNegInf ? 0.f : mn;
        alpha[PAR] = nd ? __builtin_amdgcn_exp2f(m_old - mn) : 1.f;
        asm volatile("" : "+v"(mref[PAR]), "+v"(alpha[PAR]), "+v"(m_run));
      }
    };
    // tile st - 1's exponential piece k (element k % 16 of block k / 16), packing four codes per word
    auto exp_piece = [&](int k) {
      const int kb = k >> 4, i = k & 15;
      const float sv = sacc[PAR ^ 1][kb][i];
      const float x = RAW ? __builtin_fmaf(sv, coef, -mref[PAR ^ 1]) : sv - mref[PAR ^ 1];
      const float p = __builtin_amdgcn_exp2f(x);
      psum = k == 0 ? p : psum + p;
      if ((k & 3) < 3) {
        pv3[k & 3] = p;
        if ((k & 3) == 1) {
          pw = pack_fp8x2<false>(pv3[0], pv3[1], 0);
          asm volatile("" : "+v"(pw), "+v"(psum));
        } else {
          asm volatile("" : "+v"(pv3[k & 3]), "+v"(psum));
        }
      } else {
        pk[PAR ^ 1][k >> 2] = pack_fp8x2<true>(pv3[2], p, pw);
        asm volatile("" : "+v"(pk[PAR ^ 1]), "+v"(psum));
      }
    };

    static_for<MPT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int r = m % NFR;
      if constexpr (m % 2 == 0) {
        // fragments m and m + 1 complete: the LDS reads issued after fragment m + 1 are those of m + 2
        constexpr int after = PF > 2 ? fp8_reads(m + 2, MPT, PS) : 0;
        lgkm_wait<after>();
      }
      if constexpr (m < PS) {
        constexpr int kb = m / NS, s = m % NS;
        if constexpr (s == 0) Mma8::first(sacc[PAR][kb], fr[r], qf[s]);
        else Mma8::acc(sacc[PAR][kb], fr[r], qf[s]);
      } else {
        constexpr int c = m - PS;
        // the probabilities of tile st - 2 were packed by VALU instructions in the previous stage
        if constexpr (c == 0) Mma8::acc_agpr(o_acc[c], fr[r], pk[PAR]);
        else Mma8::acc_agpr_nonop(o_acc[c], fr[r], pk[PAR]);
      }
      __builtin_amdgcn_sched_barrier(0);

      // a block of S(st) finished one product ago: 20 wait states before its logits are formed (two
      // column groups: before its partial is published to the partner)
      if constexpr (m == NS) mma8_guard1(sacc[PAR][0]);
      if constexpr (m == PS) mma8_guard1(sacc[PAR][1]);
      if constexpr (DG == 2 && (m == NS || m == PS)) {
        constexpr int kb = m / NS - 1;
        const f32x16& x = sacc[PAR][kb];
        lds_write_b128_async<kb * 4096 + 0>(ex_mine, f32x4{x[0], x[1], x[2], x[3]});
        lds_write_b128_async<kb * 4096 + 1024>(ex_mine, f32x4{x[4], x[5], x[6], x[7]});
        lds_write_b128_async<kb * 4096 + 2048>(ex_mine, f32x4{x[8], x[9], x[10], x[11]});
        lds_write_b128_async<kb * 4096 + 3072>(ex_mine, f32x4{x[12], x[13], x[14], x[15]});
      }
      // mask biases of tile st's block 0, requested at the start of the stage
      if constexpr (MASK && m == 0) load_block_bias(key0);

      // ---- epoch boundary: the next epoch's groups become visible; the slots of the epoch before
      // last are refilled LA epochs ahead
      if constexpr ((m + PF) % EM == 0) {
        const int eg = st * EPT + (m + PF) / EM;
        // the barrier that publishes a partial: the partial's writes have landed before it
        constexpr int pub = DG == 2 ? (m == fp8_block_barrier(0, NS, EM, PF) ? 0
                                       : (m == fp8_block_barrier(1, NS, EM, PF) ? 1 : -1))
                                    : -1;
        if constexpr (pub >= 0) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (eg < total_epochs) {
          wait_epoch(eg);
          __builtin_amdgcn_s_barrier();
        }
        // the partner's partial of that block (complete once a fragment read issued after it is)
        if constexpr (pub >= 0) {
          part[0] = lds_read_f4_async<pub * 4096 + 0>(ex_partner);
          part[1] = lds_read_f4_async<pub * 4096 + 1024>(ex_partner);
          part[2] = lds_read_f4_async<pub * 4096 + 2048>(ex_partner);
          part[3] = lds_read_f4_async<pub * 4096 + 3072>(ex_partner);
        }
      }
      static_for<EPT + 1>([&](auto eb_c) {
        constexpr int eb = decltype(eb_c)::value;
        constexpr int bs = eb * EM - PF;
        if constexpr (bs >= 0 && bs < MPT) {
          static_for<NL>([&](auto q_c) {
            constexpr int Q = decltype(q_c)::value;
            constexpr int ls = bs + 1 + (Q * (EM - 1)) / NL;
            constexpr int slot = ls < MPT ? ls : MPT - 1;
            if constexpr (slot == m)
              issue_epoch_load(st, std::integral_constant<int, U>{}, std::integral_constant<int, eb + LA>{}, q_c);
          });
        }
      });

      // ---- the fragment PF products ahead (the last ones: the next stage's first products)
      read_frag(std::integral_constant<int, U>{}, std::integral_constant<int, m + PF>{});

      // ---- softmax pieces: tile st - 1's exponentials over the stage, tile st's logits after S(st)
#pragma unroll
      for (int k = 0; k < 32; ++k)
        if (fp8_exp_slot(k, MPT) == m) exp_piece(k);
      // (two column groups) the partner's partial joins this wave's before the block's logits
      if constexpr (DG == 2 && (m == F0 || m == F1)) {
        constexpr int kb = m == F0 ? 0 : 1;
        asm volatile("" : "+v"(part[0]), "+v"(part[1]), "+v"(part[2]), "+v"(part[3]));
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[PAR][kb][4 * g + e] += part[g][e];
        asm volatile("" : "+v"(sacc[PAR][kb]));
      }
#pragma unroll
      for (int k = 0; k < NLB; ++k)
        if (fp8_logit_slot(0, k, DG, NS, MPT, EM, PF, RAW) == m) logit_piece(0, k);
      // block 1's biases replace block 0's once its last logit piece has read them
      if constexpr (MASK && m == fp8_logit_slot(0, NLB - 1, DG, NS, MPT, EM, PF, false)) load_block_bias(key0 + 32);
#pragma unroll
      for (int k = 0; k < NLB + 2; ++k)
        if (fp8_logit_slot(1, k, DG, NS, MPT, EM, PF, RAW) == m) logit_piece(1, k);

      // ---- close the stage: l and O take tile st - 1's rescale (O holds exactly the tiles before it)
      if constexpr (m == MPT - 1) {
        l_lane = l_lane * alpha[PAR ^ 1] + psum;
        if (__builtin_amdgcn_ballot_w64(need[PAR ^ 1]) != 0) {
          mma_guard_all<NPV>(o_acc);
          mma_guard_all<NPV>(o_acc);
#pragma unroll
          for (int c = 0; c < NPV; ++c) {
            o_acc[c] *= alpha[PAR ^ 1];
            asm volatile("" : "+a"(o_acc[c]));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  for (int T0 = 0; T0 < nstages; T0 += UNR) {
    static_for<UNR>([&](auto u_c) {
      constexpr int U = decltype(u_c)::value;
      if (T0 + U < nstages) stage(T0 + U, u_c);
    });
  }
  vm_wait<0>();
  // the last stage read the next stage's first fragments (never used): their registers stay reserved
  // until those reads have landed
  static_assert(NFR == 4, "fragment registers tied below");
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fr[0]), "+v"(fr[1]), "+v"(fr[2]), "+v"(fr[3]) : : "memory");

  // ================= epilogue =================
  mma_guard_all<NPV>(o_acc);
  mma_guard_all<NPV>(o_acc);
  const float l = sum_halves(l_lane);
  const float inv = l > 0.f ? fv / l : 0.f;
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring before the staged O overwrites it
  store_o_staged<T, DW, NPV>(o_acc, inv, smem + wave * o_stage_bytes<DW>(),
                             a.o + (int64_t)(b * a.Hq + hq) * Nq * o_rs + (int64_t)rw0 * o_rs + col0, o_rs, Nq - rw0,
                             a.dcols - col0, lane);
  if (row < Nq && a.lse != nullptr && dg == 0 && hi == 0) {
    const float lse = l > 0.f ? (m_run + __builtin_log2f(l)) * kLn2 : kNegInf;
    a.lse[(int64_t)(b * a.Hq + hq) * Nq + row] = lse;
  }
  clock_stamp(a.stamps, 1);
}

template <typename T, int D>
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream) {
  if (a.group < 1 || a.Hkv < 1 || a.Hq != a.group * a.Hkv || a.B < 1 || a.Nq < 1 || a.Nkv < 1 || a.dcols > D ||
      a.dcols < 16 || a.dcols % 16 != 0)
    return hipErrorInvalidValue;
  constexpr int BR = Fp8Tiling<D>::BR;
  const int nqt = (a.Nq + BR - 1) / BR;
  const long long blocks = (long long)a.B * a.Hq * nqt;
  const bool masked = a.mask_kind != kMaskNone;
  const bool raw = !masked && !a.causal && a.Nkv % 64 == 0 && a.scale_log2 > 0.f;
  if (raw)
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, D, kFp8Raw>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else if (!masked)
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, D, kFp8Edge>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else if (a.mask_kind == kMaskAddF32)
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, D, kFp8Mask, kMaskAddF32>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else if (a.mask_kind == kMaskBoolU8)
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, D, kFp8Mask, kMaskBoolU8>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else if (a.mask_kind == kMaskAddBf16)
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, D, kFp8Mask, kMaskAddBf16>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else if (a.mask_kind == kMaskAddFp16)
    hipLaunchKernelGGL((ffpa_fwd_fp8_kernel<T, D, kFp8Mask, kMaskAddFp16>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ffpa

// Fused backward of the attention forward on gfx950 (ffpa-attn "API Reference": the backward of
// ffpa_attn_func, run as SDPA's backward): dQ, dK, dV, and the additive mask's gradient, from Q, K,
// V, dO, the forward's fp32 LSE and Delta = rowsum(dO * O).  No score matrix is kept in memory.
//
// Two passes of one kernel template.  Each wave keeps its own block of 32 indices ("stationary") in
// registers and loops over tiles of 32 indices of the other side, streamed through LDS:
//   dQ pass: a wave owns 32 query rows (its Q and dO rows in VGPRs) and streams the K and V tiles
//     of its KV head:   S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T * (dP^T - Delta),  dQ^T += K^T dS^T.
//   dK/dV pass: a wave owns 32 keys (its K and V rows in VGPRs) and streams the Q and dO tiles of
//     every query head of its KV group:   S = Q K^T,  dP = dO V^T,  dS = P * (dP - Delta),
//     dV^T += dO^T P,  dK^T += Q^T dS.
// P = exp(scale S + bias - LSE) is recomputed from the forward's LSE, so neither pass needs the
// other's results and no row statistic is formed here.  The accumulators (dQ^T, or dK^T and dV^T)
// live in AGPRs; dQ and dK take the softmax scale once, when they are stored.  With attention
// dropout (keep bits M, factor 1/(1-p)): dV^T += dO^T (P M) and dS = P (dP M - Delta).
//
// Wave roles.  Two waves share a stationary block of 32 (four above D = 512): role A holds the
// Q-side operand of the score product (dQ pass: Q; dK/dV pass: K) and forms S, role B the dO side
// (dO; V) and forms dP, each over all columns (above 512: two waves per role, one per column half,
// whose partial tiles are summed).  The finished tiles are exchanged through LDS, so that every
// wave of the block holds S and dP and forms P and dS itself.  Then the dQ pass splits dQ's
// columns among the block's waves; in the dK/dV pass role A accumulates dK and role B dV.  A wave
// thus keeps one stationary operand (at most 128 VGPRs) and at most 256 accumulators.  Other head
// dims (multiples of 8) run the next kernel head dim: the stationary columns past D load as zero, the
// products of 32-column blocks wholly past D are skipped, and outputs past D are not stored.  The
// streamed tiles' last partial block holds the next row's (finite) values past D, which meet only
// zero operands or accumulator columns that are never stored.
//
// Products (v_mfma_f32_32x32x16, inline assembly as in the forward): a score tile is
// (streamed x stationary), so lane l holds stationary index l % 32 and accumulator element i holds
// streamed index 8 (i / 4) + 4 (l / 32) + i % 4.  Packed to 16 bits, element 8 kk + j of a lane is
// the B operand of the accumulation products at contraction slot j of step kk, provided the
// streamed index of slot j is read in that same order on the A side: the transposed LDS reads
// (ds_read_b64_tr_b16) fetch rows 16 kk + 4 (l / 32) + 0..3 and, with a second read, + 8.
//
// LDS tiles: per tensor, 64-column blocks of [32 rows][128 bytes] (4 KiB), 16-byte chunk c of row r
// stored at position c ^ bwd_swz(r) (conflict-free for the operand reads and the transposed reads),
// filled by buffer_load_dwordx4 ... lds with whole 128-byte row segments (rows past the tensor's end
// read as zero); the dK/dV pass stages each tile's LSE, Delta and keep words beside it.  Tiles are
// double-buffered where two fit next to the exchange slots (D <= 512), the next tile's loads spread
// over the current tile's products.  Above that, one buffer: in the dK/dV pass each wave reloads its
// own quarter of the tile block by block as its products release it; the dQ pass streams the next
// tile in during its accumulation products where its waves' dQ columns are whole 64-column blocks
// (768 and 1024 columns), and otherwise loads it once the current one has been consumed.
#pragma once

#include <type_traits>

#include "ffpa_bwd_launch.hpp"

namespace ffpa {

template <int KD>
struct BwdTiling {
  static constexpr int GW = KD <= 512 ? 2 : 4;  // waves per stationary block of 32
  static constexpr int NH = GW / 2;             // column parts of the score products
  static constexpr int SW = KD / NH;            // score columns per wave
  static constexpr int NKS = SW / 16;           // 16-column steps of a score product
  static constexpr int AWQ = KD / GW;           // dQ columns per wave
  static constexpr int AWK = KD / NH;           // dK (or dV) columns per wave
  static constexpr int RG = 4 / GW;             // stationary blocks per workgroup
  static constexpr int NBLK = KD / 32;          // 32-column blocks per tensor tile
  static constexpr int TILE = 2 * NBLK * 2048;  // the two streamed tensors of one 32-index tile
  static constexpr int ROW1 = 768;              // staged per-row data of a tile: LSE, Delta, keep words
  static constexpr int EXCH = 4 * 4096;         // one partial score tile per wave
  static constexpr int NBUF = 2 * (TILE + ROW1) + EXCH <= 160 * 1024 ? 2 : 1;
  // single-buffered, the dK/dV pass has every wave load its own copy of the staged rows
  static constexpr int ROWS = NBUF == 1 ? 4 * ROW1 : ROW1;
  static constexpr int BUF = TILE + ROWS;
  static constexpr int LDS_BYTES = NBUF * BUF + EXCH;
  static constexpr bool OK = KD % 64 == 0 && KD >= 64 && KD <= 1024 && AWQ % 32 == 0 && AWK % 32 == 0;
};

// Position of the 16-byte chunks of LDS tile row r: logical chunk c of a 64-column block's row r
// sits at c ^ bwd_swz(r).  A bijection of bits 1-3 of r, so that the 16 rows a 16-byte operand
// read takes at once fill 16 distinct 16-byte slots of 256 bytes, and rows r and r + 2 of a
// transposed read fall in different halves of their 128-byte rows.
__device__ inline int bwd_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// addr with bit 6 flipped, formed where it is used (opaque to the compiler, which would otherwise
// keep it in a register of its own across the loop)
__device__ inline uint32_t bwd_flip64(uint32_t addr) {
  uint32_t r;
  asm volatile("v_xor_b32 %0, 64, %1" : "=v"(r) : "v"(addr));
  return r;
}

// The bias of one (row, key) of a runtime mask kind: -inf for an excluded boolean entry.
__device__ inline float bwd_bias(const void* m, int kind, int64_t off) {
  switch (kind) {
    case kMaskBoolU8: return ((const unsigned char*)m)[off] ? 0.f : kNegInf;
    case kMaskAddF32: return ((const float*)m)[off];
    case kMaskAddBf16: return widen_bf16(((const uint16_t*)m)[off]);
    case kMaskAddFp16: return widen_fp16(((const uint16_t*)m)[off]);
    default: return 0.f;
  }
}

// Marks the values as written here, after a wait that completed the LDS reads filling them: every
// use of them then stays behind that wait.
__device__ inline void bwd_tie(f32x4 (&x)[4]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}
// Completes this wave's LDS reads; the tied operands keep every use of the values after it.
__device__ inline void bwd_lds_wait3(f32x4& x, f32x4& y, f32x4& z) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x), "+v"(y), "+v"(z)::"memory");
}

// Score products: d = a * b (+ d) into VGPRs.  The leading s_nop 1 gives the 2 wait states a
// product needs after a VALU write of an operand - the compiler may move a stationary fragment
// between register files (v_accvgpr_read) right before its use.
template <typename T>
__device__ inline void bwd_mma_first(f32x16& d, const i32x4& a, const i32x4& b) {
  if constexpr (std::is_same<T, Bf16>::value)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
template <typename T>
__device__ inline void bwd_mma_acc(f32x16& d, const i32x4& a, const i32x4& b) {
  if constexpr (std::is_same<T, Bf16>::value)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// Roles.  The GW waves of a stationary block split the work by tensor: role A holds the Q side of
// the score product (dQ pass: Q; dK/dV pass: K) and forms S, role B the dO side (dO; V) and forms
// dP; above D = 512 each role is split once more by columns (h).  They exchange the finished tiles
// through LDS, so every wave of the block holds S and dP.  Accumulation: dQ pass, wave gw takes
// columns [gw AWQ, (gw + 1) AWQ) of dQ; dK/dV pass, role A takes dK and role B dV, columns
// [h AWK, (h + 1) AWK).
template <typename T, int KD, bool DQ, bool PAD>
__global__ __launch_bounds__(256) void ffpa_bwd_kernel(BwdArgs a) {
  using BT = BwdTiling<KD>;
  using E = Elem<T>;
  static_assert(BT::OK, "unsupported kernel head dim");
  constexpr int GW = BT::GW, NH = BT::NH, SW = BT::SW, NKS = BT::NKS, RG = BT::RG, NBLK = BT::NBLK;
  constexpr int AW = DQ ? BT::AWQ : BT::AWK;
  constexpr int NCB = AW / 32;
  constexpr int BUF = BT::BUF, TILE = BT::TILE, NBUF = BT::NBUF;
  __shared__ __attribute__((aligned(1024))) char smem[BT::LDS_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int l32 = lane & 31, hi = lane >> 5;
  const int rg = wave / GW, gw = wave % GW;
  const int role = gw / NH, h = gw % NH;
  const int sc0 = h * SW;                       // first score column of this wave
  const int ac0 = DQ ? gw * AW : h * AW;        // first accumulated column
  const int D = a.D;                            // columns in memory (the row stride); D <= KD
  const int G = a.Hq / a.Hkv;
  const int NS = DQ ? a.Nq : a.Nkv;  // stationary extent
  const int NT = DQ ? a.Nkv : a.Nq;  // streamed extent
  const int nsb = (NS + 32 * RG - 1) / (32 * RG);
  const int nblk = (DQ ? a.B * a.Hq : a.B * a.Hkv) * nsb;
  // blocks are dealt to the 8 XCDs in turn: give each XCD a contiguous run of blocks (heads), so
  // that the workgroups streaming one head's tiles share that XCD's L2
  int blk = (int)blockIdx.x;
  {
    const int per = nblk / 8;
    if (blk < per * 8) blk = (blk % 8) * per + blk / 8;
  }
  // dQ pass: blocks (b, KV head, row block, query head of the group) with the group's query heads
  // fastest, so that the G heads sharing K/V stream the same K/V tiles together (one L2 copy);
  // dK/dV pass: blocks (b, KV head, key block)
  int b, hq, hkv, sb;
  if constexpr (DQ) {
    const int g = blk % G, rest = blk / G;
    sb = rest % nsb;
    const int bk = rest / nsb;
    b = bk / a.Hkv;
    hkv = bk % a.Hkv;
    hq = hkv * G + g;
  } else {
    const int head = blk / nsb;
    sb = blk % nsb;
    b = head / a.Hkv;
    hq = 0;
    hkv = head % a.Hkv;
  }
  const int s0wg = sb * 32 * RG;
  const int s0 = s0wg + rg * 32;  // this wave's stationary block
  const int coff = a.Nkv - a.Nq;  // causal: key k is visible from row r when k <= r + coff
  const int s = s0 + l32;         // this lane's stationary index
  const int sc = s < NS ? s : NS - 1;
  const int64_t kvh = (int64_t)(b * a.Hkv + hkv) * a.Nkv * D;

  // ---- this wave's stationary rows (its score columns) as B operands: lane -> index s, 8 columns.
  // The dK/dV pass at D = 1024 keeps its last NRL fragments in L2 instead, re-read at every tile
  // (the 256 accumulators and the other 24 fragments leave no room for them).
  constexpr int NRL = (!DQ && KD == 1024) ? 8 : 0;
  constexpr int NKR = NKS - NRL;  // fragments held in registers
  i32x4 xf[NKS];
  const uint16_t* xrow;  // the lane's stationary row, from the wave's first score column
  {
    const uint16_t* xb;
    if constexpr (DQ) xb = (role == 0 ? a.q : a.dout) + (int64_t)(b * a.Hq + hq) * a.Nq * D;
    else xb = (role == 0 ? a.k : a.v) + kvh;
    xrow = xb + (int64_t)sc * D + sc0 + hi * 8;
#pragma unroll
    for (int kk = 0; kk < NKR; ++kk) {
      const bool in = !PAD || sc0 + 16 * kk + 8 * hi < D;
      xf[kk] = in ? *(const i32x4*)(xrow + 16 * kk) : i32x4{0, 0, 0, 0};
    }
    vm_wait<0>();
#pragma unroll
    for (int kk = 0; kk < NKR; ++kk) asm volatile("" : "+v"(xf[kk]));
  }
  // dQ pass: the lane's row statistics
  float lse_s = 0.f, dl_s = 0.f;
  if constexpr (DQ) {
    const int64_t ri = (int64_t)(b * a.Hq + hq) * a.Nq + sc;
    lse_s = a.lse[ri];
    dl_s = a.delta[ri];
  }

  // ---- streamed tiles
  int ntiles, rb0 = 0, nrbh = 1;
  if constexpr (DQ) {
    int kend = a.Nkv;
    if (a.causal) {
      const int rlast = (s0wg + 32 * RG < a.Nq ? s0wg + 32 * RG : a.Nq) - 1;
      kend = rlast + coff + 1 < a.Nkv ? rlast + coff + 1 : a.Nkv;
    }
    ntiles = (kend + 31) / 32;
  } else {
    const int nrb = (a.Nq + 31) / 32;
    if (a.causal) rb0 = (s0wg - coff > 0 ? s0wg - coff : 0) / 32;
    nrbh = nrb - rb0;
    ntiles = G * nrbh;
  }
  // tile t: the streamed index of its row 0, and the query head it belongs to (dK/dV pass)
  auto tile_pos = [&](int t, int& t0, int& qh) {
    if constexpr (DQ) {
      t0 = 32 * t;
      qh = hq;
    } else {
      const int g = t / nrbh;
      t0 = 32 * (rb0 + t % nrbh);
      qh = hkv * G + g;
    }
  };

  // loads: whole 128-byte row segments.  Wave w fills rows 8w .. 8w + 7 of every 64-column block of
  // each tensor's tile, one 1 KiB load per block; lane t takes row 8w + t / 8, physical chunk t % 8,
  // i.e. logical chunk (t % 8) ^ bwd_swz(row).  The lane's byte offset is fixed, the block step
  // 128 c a scalar offset, and the tile's first row the descriptor's base (its record count ends at
  // the tensor's last row, so rows past it read as zero).
  const uint32_t smem_addr = lds_addr(smem);
  const bool has_drop = a.keep != nullptr;
  uint32_t vlane;
  {
    const int lrow = 8 * wave + (lane >> 3);
    const int lchunk = (lane & 7) ^ bwd_swz(lrow);
    vlane = (uint32_t)(lrow * D + lchunk * 8) * 2u;
  }
  // A tile's loads: NLD per wave, load j the U piece (K, or Q) of 64-column block j / 2 for even j,
  // the W piece (V, or dO) for odd j.  prep_tile forms the two descriptors and the LDS destination and
  // issues the staged rows (PARTS: 1 the U tile, 2 the W tile, 4 the staged rows of the dK/dV pass);
  // issue_load then issues one load.  A tile that is not `valid` (past the last) gets descriptors of
  // no records, so that its loads read nothing and write zeros.
  constexpr int NLD = NBLK;
  auto prep_tile = [&](int t, int buf, __amdgpu_buffer_rsrc_t& ru, __amdgpu_buffer_rsrc_t& rw, uint32_t& dst,
                       auto parts_c, bool valid) {
    constexpr int PARTS = decltype(parts_c)::value;
    int t0, qh;
    tile_pos(t, t0, qh);
    const uint16_t* ub;
    const uint16_t* wb;
    if constexpr (DQ) {
      ub = a.k + kvh;
      wb = a.v + kvh;
    } else {
      ub = a.q + (int64_t)(b * a.Hq + qh) * a.Nq * D;
      wb = a.dout + (int64_t)(b * a.Hq + qh) * a.Nq * D;
    }
    ub += (int64_t)t0 * D;
    wb += (int64_t)t0 * D;
    const int bytes = valid ? (int)((int64_t)(NT - t0) * D * 2) : 0;  // the descriptor's 32-bit record count
    ru = __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0, bytes, 0x00020000);
    rw = __builtin_amdgcn_make_buffer_rsrc((void*)wb, (short)0, bytes, 0x00020000);
    // LDS destinations from the 32-bit LDS address (no generic-pointer conversion); made opaque
    // here so that the compiler forms each one before its load instead of keeping them all in
    // SGPRs across the loop
    dst = smem_addr + (uint32_t)(buf * BUF + wave * 1024);
    asm volatile("" : "+s"(dst));
    if constexpr (!DQ && (PARTS & 4) != 0) {
      // the tile's rows: LSE and Delta (lane l -> row l % 32), keep words of the workgroup's keys
      // (lane l -> row l % 32, word s0wg / 32 + l / 32); rows past Nq read as zero
      if (wave == 0 && valid) {
        const int64_t fr = (int64_t)(b * a.Hq + qh) * a.Nq + t0;
        const int nb = (a.Nq - t0) * 4;
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)(a.lse + fr), (short)0, nb, 0x00020000);
        const __amdgpu_buffer_rsrc_t rd =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.delta + fr), (short)0, nb, 0x00020000);
        const uint32_t rows = smem_addr + (uint32_t)(buf * BUF + TILE);
        const uint32_t ro = (uint32_t)l32 * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (FFPA_LDS void*)(uintptr_t)rows, 4, ro, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FFPA_LDS void*)(uintptr_t)(rows + 256), 4, ro, 0, 0, 0);
        if (has_drop) {
          const int kb = (int)((int64_t)(a.Nq - t0) * a.keep_w * 4);
          const __amdgpu_buffer_rsrc_t rk =
              __builtin_amdgcn_make_buffer_rsrc((void*)(a.keep + fr * a.keep_w), (short)0, kb, 0x00020000);
          const uint32_t ko = ((uint32_t)l32 * (uint32_t)a.keep_w + (uint32_t)(s0wg / 32 + hi)) * 4u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FFPA_LDS void*)(uintptr_t)(rows + 512), 4, ko, 0, 0, 0);
        }
      }
    }
  };
  auto issue_load = [&](const __amdgpu_buffer_rsrc_t& ru, const __amdgpu_buffer_rsrc_t& rw, uint32_t dst, auto j_c,
                        auto parts_c) {
    constexpr int j = decltype(j_c)::value, PARTS = decltype(parts_c)::value;
    constexpr int c = j / 2;
    if (!PAD || 64 * c < D) {
      // the block step goes in the scalar offset: the instruction's immediate offset would move the
      // LDS destination as well
      if constexpr (j % 2 == 0 && (PARTS & 1) != 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (FFPA_LDS void*)(uintptr_t)(dst + 4 * c * 1024), 16, vlane,
                                                 128 * c, 0, 0);
      if constexpr (j % 2 == 1 && (PARTS & 2) != 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (FFPA_LDS void*)(uintptr_t)(dst + NBLK * 2048 + 4 * c * 1024),
                                                 16, vlane, 128 * c, 0, 0);
    }
  };
  auto issue_tile = [&](int t, int buf, auto parts_c) {
    __amdgpu_buffer_rsrc_t ru, rw;
    uint32_t dst;
    prep_tile(t, buf, ru, rw, dst, parts_c, true);
    static_for<NLD>([&](auto j_c) { issue_load(ru, rw, dst, j_c, parts_c); });
  };
  // Single-buffered, the dK/dV pass's waves each read only their own quarter of a tile (their
  // role's tensor, their column half), so each loads its quarter itself, as soon as its own
  // products of the tile before are done, with no barrier, and its score products wait block by
  // block for just the blocks they read.  Its stationary fragments kept in L2 (padded head dims: at
  // the tile start, as their registers allow) and its copy of the staged rows are loaded first, so
  // that the quarter's blocks are its youngest loads, four per 64-column block.
  constexpr bool OWN = !DQ && NBUF == 1;
  // Single-buffered, the dQ pass streams the next tile into the buffer during the accumulation
  // products, where each wave's dQ columns are whole 64-column blocks of K: V is free once the
  // exchange is passed (only the dP products read it), and a K block once its owner (the one wave
  // whose dQ columns it holds) has taken its accumulation products; the next tile's barrier then
  // publishes both.
  constexpr bool STREAM = DQ && NBUF == 1 && BT::AWQ % 64 == 0;
  constexpr int NBH = SW / 64;  // 64-column blocks of a column half
  // rows 8 r .. 8 r + 7 (the lane layout of the tile loads above): rows 16 .. 31 take the lane
  // offsets of rows 0 .. 15 (bwd_swz ignores bit 4) and 16 rows more in the scalar offset
  uint32_t vown[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int lrow = 8 * r + (lane >> 3);
    const int lchunk = (lane & 7) ^ bwd_swz(lrow);
    vown[r] = (uint32_t)(lrow * D + lchunk * 8) * 2u;
  }
  // (the quarter's descriptor and LDS destination, between own_head and the block loads)
  __amdgpu_buffer_rsrc_t own_rt;
  uint32_t own_dst = 0;
  auto own_head = [&](int t) {
    if constexpr (OWN) {
      int t0, qh;
      tile_pos(t, t0, qh);
      if constexpr (NRL > 0 && !PAD) {
        // (the address is made opaque so that the loads stay where they are)
        const uint16_t* xr = xrow;
        asm volatile("" : "+v"(xr));
#pragma unroll
        for (int kk = NKR; kk < NKS; ++kk) {
          const bool in = !PAD || sc0 + 16 * kk + 8 * hi < D;
          xf[kk] = in ? *(const i32x4*)(xr + 16 * kk) : i32x4{0, 0, 0, 0};
        }
      }
      const int64_t fr = (int64_t)(b * a.Hq + qh) * a.Nq + t0;
      {
        // this wave's copy of the tile's rows: LSE and Delta (lane l -> row l % 32), keep words of the
        // workgroup's keys (lane l -> row l % 32, word s0wg / 32 + l / 32); rows past Nq read as zero
        const int nb = (a.Nq - t0) * 4;
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)(a.lse + fr), (short)0, nb, 0x00020000);
        const __amdgpu_buffer_rsrc_t rd =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.delta + fr), (short)0, nb, 0x00020000);
        const uint32_t rows = smem_addr + (uint32_t)(TILE + wave * BT::ROW1);
        const uint32_t ro = (uint32_t)l32 * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (FFPA_LDS void*)(uintptr_t)rows, 4, ro, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (FFPA_LDS void*)(uintptr_t)(rows + 256), 4, ro, 0, 0, 0);
        if (has_drop) {
          const int kb = (int)((int64_t)(a.Nq - t0) * a.keep_w * 4);
          const __amdgpu_buffer_rsrc_t rk =
              __builtin_amdgcn_make_buffer_rsrc((void*)(a.keep + fr * a.keep_w), (short)0, kb, 0x00020000);
          const uint32_t ko = ((uint32_t)l32 * (uint32_t)a.keep_w + (uint32_t)(s0wg / 32 + hi)) * 4u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (FFPA_LDS void*)(uintptr_t)(rows + 512), 4, ko, 0, 0, 0);
        }
      }
      const uint16_t* tb = (role == 0 ? a.q : a.dout) + fr * D;
      const int bytes = (int)((int64_t)(NT - t0) * D * 2);  // the descriptor's 32-bit record count
      own_rt = __builtin_amdgcn_make_buffer_rsrc((void*)tb, (short)0, bytes, 0x00020000);
      own_dst = smem_addr + (uint32_t)(role * NBLK * 2048 + (sc0 / 64) * 4096);
      asm volatile("" : "+s"(own_dst));
    }
  };
  // 64-column block c of the quarter: four loads of 8 rows, the column offset in the scalar offset
  // (the instruction's immediate offset would move the LDS destination as well)
  auto own_block = [&](auto c_c) {
    if constexpr (OWN) {
      constexpr int c = decltype(c_c)::value;
      if (!PAD || sc0 + 64 * c < D) {
        const int soff = (sc0 + 64 * c) * 2;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(own_rt, (FFPA_LDS void*)(uintptr_t)(own_dst + c * 4096 + r * 1024), 16,
                                                   vown[r % 2], soff + (r / 2) * 16 * D * 2, 0, 0);
      }
    }
  };

  // ---- per-lane LDS addresses (block offsets are immediates; buffer offsets added at run time)
  // score operand read: row l32 of the role's tensor, 16-column step q of a 64-column block: chunk
  // 2q + hi (the wave's first score column is a multiple of 64)
  const uint32_t sbase = smem_addr + (uint32_t)(role * NBLK * 2048 + (sc0 / 64) * 4096);
  // (steps 2 and 3 differ from steps 0 and 1 in chunk bit 2 only: their addresses are those of
  // steps 0 and 1 with bit 6 flipped.  FLIP variants form them at each read, which costs an
  // instruction in front of the read but the registers the dK/dV pass at 1024 columns, and padded
  // at 512, do not have.)
  constexpr bool FLIP = !DQ && (KD == 1024 || (KD == 512 && PAD));
  uint32_t fa[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) fa[q] = sbase + l32 * 128 + (((2 * q + hi) ^ bwd_swz(l32)) * 16);
  // transposed read (accumulation products): lanes of a 16-lane group read rows 4 (l / 32) + i16 / 4
  // (and + 8), columns 16 ((l / 16) % 2) + 4 (i16 % 4) .. + 3 of a 32-column block; the lane
  // receives column l % 32 of rows 4 (l / 32) + 0..3 (and + 8).  The wave's 32-column block cb is
  // global block a0b + cb: half (a0b + cb) % 2 of 64-column block (a0b + cb) / 2, so even and odd cb
  // take different bases (t?[0], t?[1]) and share the immediate offset (cb / 2) 4096 + kk 2048.
  // In the dK/dV pass a0b is even, and the odd bases are the even ones with bit 6 flipped (formed at
  // each read in FLIP variants).
  const int atens = DQ ? 0 : role;  // dQ: K^T; dK: Q^T; dV: dO^T
  const int a0b = ac0 / 32;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int trow = 4 * (g16 >> 1) + (i16 >> 2);
  const int tchunk = 2 * (g16 & 1) + ((i16 & 3) >> 1);
  uint32_t ta[2], tb[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int g = a0b + par;  // the global 32-column block of local cb = par
    const uint32_t blk = smem_addr + (uint32_t)(atens * NBLK * 2048 + (g >> 1) * 4096) + 8 * (i16 & 1);
    ta[par] = blk + trow * 128 + (((4 * (g & 1) + tchunk) ^ bwd_swz(trow)) * 16);
    tb[par] = blk + (trow + 8) * 128 + (((4 * (g & 1) + tchunk) ^ bwd_swz(trow + 8)) * 16);
  }
  // partial-tile exchange: slot per wave, 16 bytes per lane in four 1 KiB pieces
  const uint32_t ex_base = smem_addr + NBUF * BUF;
  const uint32_t ex_mine = ex_base + wave * 4096 + lane * 16;

  const bool has_mask = a.mask_kind != kMaskNone;
  const float scale = a.scale;
  const int64_t mask_b = (int64_t)b * a.msb;
  // the dQ pass writes the logits' gradient into the mask gradient from one wave per block
  const bool dm_on = DQ && a.dmask != nullptr && gw == 0;

  f32x16 acc[NCB];  // dQ^T, dK^T or dV^T columns of this wave
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc[c] = f32x16{};

  // The tile's products run in NKS + NA slots, the score products first.  Double-buffered, the next
  // tile's NLD loads are spread over the first LSPAN slots (the score products and the first half of
  // the accumulation products), load j after slot j * LSPAN / NLD: issued all at once they hold the
  // wave at the load unit's queue for about as long as the direct-load path needs to move the tile,
  // with no product issued meanwhile.
  constexpr int NA = NCB * 2;
  // fragments read PF products ahead (two where the dK/dV pass's 256 accumulators and a 512-column
  // stationary operand leave no room for more)
  constexpr int PF = (!DQ && KD > 896) ? 2 : 4;
  // (padded head dims: over the score products only; in the accumulation products the padded dK/dV
  // pass at 512 columns has no registers for them)
  constexpr int LSPAN = PAD ? NKS : NKS + NA / 2;
  // the staged rows' LSE and Delta of all four element groups are read at the start of a tile where
  // two tiles are buffered and no column is padded (otherwise, and for the keep words, at their
  // group's first element: the registers they would hold across the score products are not there)
  constexpr bool HOIST = NBUF == 2 && !PAD;

  constexpr std::integral_constant<int, 7> kAll{};
  if (ntiles > 0) {
    if constexpr (OWN) {
      own_head(0);
      static_for<NBH>([&](auto c_c) { own_block(c_c); });
    } else {
      issue_tile(0, 0, kAll);
    }
  }
  for (int t = 0; t < ntiles; ++t) {
    const int buf = NBUF == 2 ? (t & 1) : 0;
    int t0, qh;
    tile_pos(t, t0, qh);
    // tile t visible, every wave done with tile t - 1 (its buffer, the exchange slots); a wave that
    // loads its own quarter waits for it block by block below (padded head dims: all of it here,
    // some of their blocks not being loaded)
    if constexpr (!OWN || PAD) vm_wait<0>();
    block_sync();
    if constexpr (NRL > 0 && PAD) {
      // (the address is made opaque so that the loads stay inside the loop)
      const uint16_t* xr = xrow;
      asm volatile("" : "+v"(xr));
#pragma unroll
      for (int kk = NKR; kk < NKS; ++kk) {
        const bool in = sc0 + 16 * kk + 8 * hi < D;
        xf[kk] = in ? *(const i32x4*)(xr + 16 * kk) : i32x4{0, 0, 0, 0};
      }
    }
    const uint32_t boff = (uint32_t)(buf * BUF);
    uint32_t kw = 0;
    if constexpr (DQ) {
      // one load whether or not there is dropout (LSE's first word stands in): the compiler can then
      // count it exactly, where a conditional load makes it wait for every load in flight
      const uint32_t* kp = has_drop ? a.keep + ((int64_t)(b * a.Hq + hq) * a.Nq + sc) * a.keep_w + t
                                    : (const uint32_t*)a.lse;
      kw = *kp;
    }
    const bool more = t + 1 < ntiles;
    // (after the last tile the loads still run, reading nothing: loads issued on every path let the
    // compiler count exactly what a wait for an earlier load must let pass)
    __amdgpu_buffer_rsrc_t nru, nrw;
    uint32_t ndst = 0;
    if constexpr (NBUF == 2) prep_tile(t + 1, buf ^ 1, nru, nrw, ndst, kAll, more);
    // the next tile's loads that follow slot u
    auto loads_after = [&](auto u_c) {
      if constexpr (NBUF == 2) {
        constexpr int u = decltype(u_c)::value;
        static_for<NLD>([&](auto j_c) {
          constexpr int j = decltype(j_c)::value;
          if constexpr (j * LSPAN / NLD == u) issue_load(nru, nrw, ndst, j_c, kAll);
        });
      }
    };
    f32x4 lse4[4], dl4[4], kw4[4];
    if constexpr (!DQ && HOIST) {
      // (in LDS order, so the products' fragment waits below cover them)
      const uint32_t ra = smem_addr + boff + TILE + (uint32_t)(16 * hi);
      static_for<4>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        lse4[g] = lds_read_f4_async<32 * g>(ra);
        dl4[g] = lds_read_f4_async<256 + 32 * g>(ra);
      });
    }

    // ---- the role's score product over its columns (fragments read PF products ahead)
    f32x16 own;
    i32x4 fr[PF + 1];
    auto read_s = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr uint32_t off = (uint32_t)((m / 4) * 4096);
      static_assert(off < 65536, "ds offset field");
      // own quarter: 64-column block m / 4 is complete once at most the four loads of each later
      // block are outstanding
      if constexpr (OWN && !PAD && m % 4 == 0) vm_wait<4 * (NBH - 1 - m / 4)>();
      if constexpr (FLIP && m % 4 >= 2) fr[m % (PF + 1)] = lds_read_b128_async<off>(bwd_flip64(fa[m % 2]) + boff);
      else fr[m % (PF + 1)] = lds_read_b128_async<off>(fa[m % 4] + boff);
    };
    static_for<PF>([&](auto mc) {
      if constexpr (decltype(mc)::value < NKS) read_s(mc);
    });
    static_for<NKS>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m + PF < NKS) read_s(std::integral_constant<int, m + PF>{});
      constexpr int after = (m + PF < NKS ? m + PF : NKS - 1) - m;
      lgkm_wait<after>();
      if constexpr (m == 0 && !DQ && HOIST) {
        // every LDS read issued before fragment 0 is complete: the staged rows are in registers
        asm volatile("" : "+v"(lse4[0]), "+v"(lse4[1]), "+v"(lse4[2]), "+v"(lse4[3]), "+v"(dl4[0]), "+v"(dl4[1]),
                     "+v"(dl4[2]), "+v"(dl4[3]));
      }
      if (!PAD || sc0 + 16 * m < D) {
        if constexpr (m == 0) bwd_mma_first<T>(own, fr[m % (PF + 1)], xf[m]);
        else bwd_mma_acc<T>(own, fr[m % (PF + 1)], xf[m]);
      }
      if constexpr (NBUF == 2) {
        __builtin_amdgcn_sched_barrier(0);  // (the loads stay between the products)
        loads_after(mc);
      }
    });
    mma_guard_s(own);

    // ---- exchange: S = the sum over h of role A's partial tiles, dP likewise for role B
    static_for<4>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      lds_write_b128_async<j * 1024>(ex_mine, f32x4{own[4 * j], own[4 * j + 1], own[4 * j + 2], own[4 * j + 3]});
    });
    block_sync();
    // single buffer, dQ pass: V has been read for the last time (by the dP products); its next tile
    // can be loaded while K is still needed
    if constexpr (STREAM) {
      if (more) prep_tile(t + 1, 0, nru, nrw, ndst, kAll, true);
    } else if constexpr (NBUF == 1 && DQ) {
      if (more) issue_tile(t + 1, 0, std::integral_constant<int, 2>{});
    }
    // every wave reads the finished tiles back from the slots, in the same order (two terms per sum:
    // their order does not change the rounded result, so every wave of the block holds the same S
    // and dP).  (The dV side of the dK/dV pass needs S only, but reads dP as well: a read on one
    // path only lets the compiler move its registers before the wait.)
    f32x16 sS, sP;
    {
      const uint32_t pa = ex_base + (uint32_t)(rg * GW * 4096) + lane * 16;
      // slot q's tile into x (four 1 KiB pieces)
      auto read_slot = [&](f32x4(&x)[4], auto q_c) {
        constexpr int q = decltype(q_c)::value;
        x[0] = lds_read_f4_async<q * 4096 + 0>(pa);
        x[1] = lds_read_f4_async<q * 4096 + 1024>(pa);
        x[2] = lds_read_f4_async<q * 4096 + 2048>(pa);
        x[3] = lds_read_f4_async<q * 4096 + 3072>(pa);
      };
      f32x4 xs[4], xp[4];
      read_slot(xs, std::integral_constant<int, 0>{});
      read_slot(xp, std::integral_constant<int, NH>{});
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      bwd_tie(xs);
      bwd_tie(xp);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sS[4 * j + e] = xs[j][e];
          sP[4 * j + e] = xp[j][e];
        }
      if constexpr (NH == 2) {
        // the second halves, in a second round (registers)
        read_slot(xs, std::integral_constant<int, 1>{});
        read_slot(xp, std::integral_constant<int, 3>{});
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        bwd_tie(xs);
        bwd_tie(xp);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sS[4 * j + e] += xs[j][e];
            sP[4 * j + e] += xp[j][e];
          }
      }
    }

    // ---- probabilities and the logits' gradient of the lane's 16 elements, in one of two versions
    // picked once per tile: interior tiles without dropout (every element in range and visible, no
    // mask: no row can then have LSE = -inf), in straight-line code, and the general version with the
    // per-element tests.
    // the accumulation product's B operand: dS, or for dV (role B of the dK/dV pass) the dropped-out P
    const bool use_p = !DQ && role == 1;
    const bool inner = !has_mask && t0 + 32 <= NT && s0 + 32 <= NS &&
                       (!a.causal || (DQ ? t0 + 31 <= s0 + coff : s0 + 31 <= t0 + coff));
    const float sl2 = scale * kLog2e;
    // the operand of k-step kk: elements 8 kk .. 8 kk + 7, two per dword (each group packed as soon as
    // it is complete)
    i32x4 gk[2];
    // MODE 0: interior, no dropout; 2: general
    auto elements = [&](auto mode_c) {
      constexpr int MODE = decltype(mode_c)::value;
      constexpr bool INNER = MODE == 0;
      static_for<4>([&](auto g_c) {
        constexpr int g = decltype(g_c)::value;
        float gv[4];
        if constexpr (!DQ) {
          // the group's staged rows not read yet (waits for every LDS read issued before them)
          const uint32_t ra = smem_addr + boff + TILE + (uint32_t)((OWN ? wave * BT::ROW1 : 0) + (8 * g + 4 * hi) * 4);
          if constexpr (!HOIST) {
            lse4[g] = lds_read_f4_async<0>(ra);
            dl4[g] = lds_read_f4_async<256>(ra);
          }
          if (MODE == 2 && has_drop) kw4[g] = lds_read_f4_async<0>(ra + 512 + (uint32_t)(rg * 128));
          if constexpr (!HOIST || MODE != 0) bwd_lds_wait3(lse4[g], dl4[g], kw4[g]);
        }
        // element e: row 8g + 4 (l / 32) + e of the tile (element 4g + e)
        static_for<4>([&](auto e_c) {
          constexpr int e = decltype(e_c)::value;
          constexpr int i = 4 * g + e;  // the element
          const int ti = t0 + 8 * g + 4 * hi + e;
          const int row = DQ ? s : ti, key = DQ ? ti : s;
          const float lse = DQ ? lse_s : lse4[g][e];
          const float dl = DQ ? dl_s : dl4[g][e];
          float p;
          if constexpr (INNER) {
            p = __builtin_amdgcn_exp2f(__builtin_fmaf(sS[i], sl2, -lse * kLog2e));
          } else {
            const bool valid = row < a.Nq && key < a.Nkv && (!a.causal || key <= row + coff) && lse != kNegInf;
            float x = sS[i] * scale;
            if (has_mask) {
              const int64_t off = mask_b + (int64_t)(DQ ? hq : qh) * a.msh +
                                  (int64_t)(row < a.Nq ? row : a.Nq - 1) * a.msq + (key < a.Nkv ? key : a.Nkv - 1);
              x += bwd_bias(a.mask, a.mask_kind, off);
            }
            // exp2 of -inf is 0
            p = valid ? __builtin_amdgcn_exp2f((x - lse) * kLog2e) : 0.f;
          }
          if constexpr (MODE == 0) {
            gv[e] = use_p ? p : p * (sP[i] - dl);
          } else {
            float m = 1.f;
            if (has_drop) {
              const uint32_t w = DQ ? kw : (uint32_t)__float_as_uint(kw4[g][e]);
              const int bit = DQ ? (8 * g + 4 * hi + e) : (key & 31);
              m = ((w >> bit) & 1u) ? a.drop_scale : 0.f;
            }
            gv[e] = use_p ? p * m : p * (sP[i] * m - dl);
          }
        });
        gk[g / 2][2 * (g % 2)] = (int)pack2<T>(gv[0], gv[1]);
        gk[g / 2][2 * (g % 2) + 1] = (int)pack2<T>(gv[2], gv[3]);
        // the dQ pass stores the mask gradient (a requested one implies a mask, so only the general
        // version does)
        if constexpr (DQ && !INNER) {
          if (dm_on) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = t0 + 8 * g + 4 * hi + e;
              if (s < a.Nq && key < a.Nkv) {
                const int64_t di = (((int64_t)(a.dm_bb ? 0 : b) * a.dm_hm + (a.dm_bh ? 0 : hq)) * a.dm_nqm +
                                    (a.dm_bq ? 0 : s)) * a.Nkv + key;
                if (a.dm_atomic) atomicAdd(a.dmask + di, gv[e]);
                else a.dmask[di] = gv[e];
              }
            }
          }
        }
      });
    };
    // (padded head dims take the general version on every tile: the interior one would cost the
    // padded dK/dV pass at 512 columns registers it does not have)
    if (!PAD && inner && !has_drop) elements(std::integral_constant<int, 0>{});
    else elements(std::integral_constant<int, 2>{});

    // ---- accumulation products: acc[cb] += (tensor^T) G over this wave's columns, step 0 (rows
    // 0-15) of every block first.  A wave that loads its own quarter takes the blocks one at a time
    // instead (both steps of block cb, then block cb + 1) and loads the next tile's block cb as soon
    // as its second step is done: the loads then leave one by one between the products, where all
    // at once they would hold the wave at the load unit's queue for the length of the transfer.
    if constexpr (OWN) {
      if (more) own_head(t + 1);  // (this wave has read its staged rows and re-read fragments)
    }
    constexpr bool BM = OWN || STREAM;  // block-major order
    i32x2 tl[PF + 1], th[PF + 1];
    auto read_a = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int cb = BM ? m / 2 : m % NCB, kk = BM ? m % 2 : m / NCB;
      constexpr uint32_t off = (uint32_t)((cb / 2) * 4096 + kk * 2048);
      static_assert(off < 65536, "ds offset field");
      if constexpr (FLIP && cb % 2 == 1) {
        tl[m % (PF + 1)] = lds_read_tr_async<off>(bwd_flip64(ta[0]) + boff);
        th[m % (PF + 1)] = lds_read_tr_async<off>(bwd_flip64(tb[0]) + boff);
      } else {
        tl[m % (PF + 1)] = lds_read_tr_async<off>(ta[cb % 2] + boff);
        th[m % (PF + 1)] = lds_read_tr_async<off>(tb[cb % 2] + boff);
      }
    };
    static_for<PF>([&](auto mc) {
      if constexpr (decltype(mc)::value < NA) read_a(mc);
    });
    static_for<NA>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int cb = BM ? m / 2 : m % NCB, kk = BM ? m % 2 : m / NCB;
      if constexpr (m + PF < NA) read_a(std::integral_constant<int, m + PF>{});
      constexpr int after = 2 * ((m + PF < NA ? m + PF : NA - 1) - m);
      lgkm_wait<after>();
      if (!PAD || ac0 + 32 * cb < D) {
        const i32x4 af = i32x4{tl[m % (PF + 1)][0], tl[m % (PF + 1)][1], th[m % (PF + 1)][0], th[m % (PF + 1)][1]};
        E::mma_acc_agpr(acc[cb], af, gk[kk]);
      }
      if constexpr (NBUF == 2 && LSPAN > NKS) {
        __builtin_amdgcn_sched_barrier(0);
        loads_after(std::integral_constant<int, NKS + m>{});
      }
      if constexpr (OWN && kk == 1 && cb % 2 == 1) {
        // the reads of 64-column block cb / 2 are complete (waited before this product)
        __builtin_amdgcn_sched_barrier(0);
        if (more) own_block(std::integral_constant<int, cb / 2>{});
      }
      if constexpr (STREAM) {
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          // the next V: this wave's row group of 64-column block c after product c * NA / NVB
          static_for<NBLK / 2>([&](auto c_c) {
            constexpr int c = decltype(c_c)::value;
            if constexpr (c * NA / (NBLK / 2) == m) issue_load(nru, nrw, ndst, std::integral_constant<int, 2 * c + 1>{}, kAll);
          });
          // the next K block this wave owns, once its products here are done (its reads waited
          // before this product): all four row groups
          if constexpr (kk == 1 && cb % 2 == 1) {
            const int blk = ac0 / 64 + cb / 2;
            if (!PAD || 64 * blk < D) {
              const uint32_t kd = smem_addr + (uint32_t)(blk * 4096);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(nru, (FFPA_LDS void*)(uintptr_t)(kd + r * 1024), 16, vown[r % 2],
                                                         blk * 128 + (r / 2) * 16 * D * 2, 0, 0);
            }
          }
        }
      }
    });

    // keeps the accumulators in AGPRs across the loop, after the wait states their last products need
    mma_guard_all<NCB>(acc);

    if constexpr (!OWN && !STREAM && NBUF == 1) {
      if (more) {
        block_sync();  // every wave is done with the buffer
        issue_tile(t + 1, 0, std::integral_constant<int, 1>{});
      }
    }
  }
  vm_wait<0>();  // (the loads after the last tile)

  // ---- epilogue: lane -> stationary index s, element i -> column ac0 + 32 cb + 8 (i / 4) + 4 hi + i % 4
  mma_guard_all<NCB>(acc);
  if (s < NS) {
    uint16_t* out;
    if constexpr (DQ) out = a.dq + (int64_t)(b * a.Hq + hq) * a.Nq * D;
    else out = (role == 0 ? a.dk : a.dv) + kvh;
    const float f = (DQ || role == 0) ? scale : 1.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (PAD && ac0 + 32 * cb >= D) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = ac0 + 32 * cb + 8 * g + 4 * hi;
        if (PAD && col >= D) continue;
        const uint32_t w0 = pack2<T>(acc[cb][4 * g] * f, acc[cb][4 * g + 1] * f);
        const uint32_t w1 = pack2<T>(acc[cb][4 * g + 2] * f, acc[cb][4 * g + 3] * f);
        *(i32x2*)(out + (int64_t)s * D + col) = i32x2{(int)w0, (int)w1};
      }
    }
  }
}

// Both passes on one stream: dK/dV first, then dQ.
template <typename T, int KD, bool PAD>
hipError_t launch_bwd_fused(const BwdArgs& a, hipStream_t stream) {
  using BT = BwdTiling<KD>;
  const int nsk = (a.Nkv + 32 * BT::RG - 1) / (32 * BT::RG);
  const int nsq = (a.Nq + 32 * BT::RG - 1) / (32 * BT::RG);
  hipLaunchKernelGGL((ffpa_bwd_kernel<T, KD, false, PAD>), dim3((unsigned)(a.B * a.Hkv * nsk)), dim3(256), 0, stream,
                     a);
  hipLaunchKernelGGL((ffpa_bwd_kernel<T, KD, true, PAD>), dim3((unsigned)(a.B * a.Hq * nsq)), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace ffpa

// Row-owner forward kernel for the large head dims (gfx950).
//
// Each wave owns 32 query rows and DW = D / DG output columns of them: DG = 1 up to D = 512 (the
// wave holds the whole O row block, 32 x D fp32 = D/2 AGPRs, and its Q rows in VGPRs, so S needs
// no cross-wave reduction at all), DG = 2 above (two waves share 32 rows and split the columns;
// their partial S tiles are summed through LDS once per 32-key block).  The workgroup is 4 waves:
// 128 query rows for DG = 1, 64 for DG = 2.  This is the output-D split of the ffpa-attn README
// ("Split-D and TiledMMA") sized for a 512-register CDNA4 lane instead of the pages' 255-register
// NVIDIA thread.
//
// Split-D staging.  K and V reach the matrix cores through a ring of LDS groups; a group holds one
// [32 keys][64 columns] sub-tile per column group (128-byte rows of eight 16-byte chunks, chunk c
// of row r stored at position c ^ pi((r >> 1) & 7) with pi(x) = ((x & 1) << 2) | (x >> 1), which
// keeps both the operand reads and the transposed reads free of bank conflicts).  The groups are
// filled with buffer_load_dwordx4 ... lds, one instruction per wave per sub-tile covering eight
// whole 128-byte rows (whole cache lines; keys past Nkv read as zero through the descriptor's
// range check).  A 64-key tile is consumed in four phases - K of keys 0-31, K of keys 32-63, V of
// keys 0-31, V of keys 32-63 - each streaming the wave's columns in 32-column steps, two products
// per step, two steps per group.  The ring is shared by the four waves and advanced in epochs of
// EM products: one s_barrier per epoch makes the next epoch's groups visible and frees the slots
// of the epoch before last, which are then refilled LA epochs ahead.
//
// Products.  S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16 (lane l <-> query row l % 32,
// so row statistics are lane-local plus one v_permlane32_swap); the operand fragments come from
// LDS PF products ahead of their use (ds_read_b128 for K, two ds_read_b64_tr_b16 for V^T).
//
// Softmax per 32-key block, overlapped with the matrix core: the logits, the row maximum and
// the exponentials of block kb are computed in small pieces between the products of the next
// phase (S of block 1 for block 0, P V of block 0 for block 1).  The running maximum is moved
// only when a block's maximum exceeds it by more than kRescaleSlack (log2 units); then O and l
// are rescaled in a rare wave-uniform branch - for block 1 after the products of block 0 have
// been accumulated, so that O always matches the reference of the probabilities added to it.
#pragma once

#include <utility>

namespace ffpa {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, each call with its index as a constant.
template <typename F, int... Is>
__device__ inline void static_for_impl(F& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Epoch length (products per wave) and ring size (4 KiB groups) for a head-dim configuration.
struct RingPlan {
  int em, ng;
};

// Lookahead first, up to 32 products (beyond that fewer barriers measured faster: 16-product epochs
// at D = 256 against 8-product ones with 48 products ahead, 5.6%), then fewer barriers.  Epochs
// shorter than min_em are taken only where no plan with longer ones fits; none longer than max_em.
constexpr RingPlan choose_ring(int GT, int MPT, int DG, int exch_bytes, int min_em = 0, int max_em = 32) {
  RingPlan best{0, 0};
  int best_score = -1;
  const int ems[4] = {32, 16, 8, 4};
  for (int i = 0; i < 4; ++i) {
    const int em = ems[i];
    if (em > max_em) continue;
    if (em == 4 && best.em != 0) break;  // four-product epochs only where nothing longer fits (D = 64)
    if (em < min_em && best.em != 0) break;
    if (MPT % em != 0) continue;
    const int bi = em / 4;  // groups per epoch (four products per wave per group)
    for (int ng = 40; ng >= bi; --ng) {
      if (ng % bi != 0 || GT % ng != 0) continue;
      if (ng * DG * 4096 + exch_bytes > 160 * 1024) continue;
      if (DG == 2 && ng * 4096 > 65536) continue;  // each column group's sub-tiles in one 64 KiB window
      const int ne = ng / bi;
      if (ne < 4) continue;
      const int ahead = (ne - 2) * em;  // products of lookahead
      const int capped = ahead < 32 ? ahead : 32;
      const int score = capped * 16 - MPT / em;  // enough lookahead first, then fewer barriers
      if (score > best_score) {
        best_score = score;
        best = RingPlan{em, ng};
      }
    }
  }
  return best;
}

// STAGED: the staged-mask variants.  Above D = 512 they take 16-product epochs where a plan has them
// (D = 1024: half the barriers per tile against 32 products of lookahead instead of 48), which
// measured 1.4% faster on the fp32-mask cross-attention workload; the other variants there keep
// 8-product epochs, which fit their registers (16-product ones spill the general variant at
// D = 1024, and measured no faster on the raw one).
template <int D, bool STAGED = false>
struct RowTiling {
  static constexpr int DG = D <= 512 ? 1 : 2;
  static constexpr int DW = D / DG;             // output columns per wave
  static constexpr int NSUB = DW / 32;          // 32-column steps per phase
  static constexpr int RG = 4 / DG;             // row groups
  static constexpr int BR = 32 * RG;            // query rows per workgroup
  static constexpr int GPP = NSUB / 2;          // groups per phase (64 columns each)
  static constexpr int GT = 4 * GPP;            // groups per 64-key tile
  static constexpr int MPT = 8 * NSUB;          // products per wave per tile
  static constexpr int EXCH = DG == 2 ? 4 * 4096 : 0;  // partial-S exchange: [wave][4 KiB]
  static constexpr int MASKB = BR * 128 * 2;            // staged fp32 mask: [block][row][32 keys]
  static constexpr RingPlan PLAN =
      choose_ring(GT, MPT, DG, EXCH + MASKB, STAGED && DG == 2 ? 16 : 0, DG == 2 && !STAGED ? 8 : 32);
  static constexpr int EM = PLAN.em;
  static constexpr int NG = PLAN.ng;
  static constexpr bool OK = PLAN.em != 0 && D % 64 == 0 && NSUB % 2 == 0 && NSUB >= 2;
  static constexpr int BI = OK ? EM / 4 : 1;    // groups per epoch
  static constexpr int NE = OK ? NG / BI : 1;   // epochs held by the ring
  static constexpr int LA = NE - 2;             // epochs of load lookahead
  static constexpr int EPT = OK ? MPT / EM : 1; // epochs per tile
  static constexpr int RING = NG * DG * 4096;   // ring bytes: [column group][slot][4 KiB]
  static constexpr int LDS_BYTES = RING + EXCH;  // + MASKB when the mask is staged
};

// The head dims the row kernel compiles: every D with a ring plan and an even number of 32-column
// steps per wave (576, 704, 832 and 960 run the next of them, padded).
template <int D>
constexpr bool use_row_kernel() {
  return RowTiling<D>::OK;
}

// Variants that do not fit the register file without spilling (from the kernels' resource metadata;
// the build refuses any spill): the contiguous split variant at D = 1024, whose runtime-layout twin
// fits, and the split variant with dropout above D = 448, where the general variant with dropout
// fits.  The launcher takes the variant that fits and never instantiates the others.
template <int D>
constexpr bool dense_split_fits() {
  return D != 1024;
}
template <int D>
constexpr bool split_drop_fits() {
  return D <= 448;
}

// s_waitcnt lgkmcnt(N) before a product whose operand fragments were read by inline assembly.
// It names no registers: volatile assembly statements keep their order, so the product (also
// volatile assembly) stays behind it, and declaring the fragments as outputs would make the
// compiler treat them as freshly VALU-written and pad every product with a nop.  That nothing
// else touches a fragment before its wait is verified on the generated code at build time.
template <int N>
__device__ inline void lgkm_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
template <int OFF>
__device__ inline i32x4 lds_read_b128_async(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  i32x4 d;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF) : "memory");
  return d;
}
template <int OFF>
__device__ inline void lds_write_b128_async(uint32_t addr, const f32x4& v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(OFF) : "memory");
}
template <int OFF>
__device__ inline f32x4 lds_read_f4_async(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  f32x4 d;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF) : "memory");
  return d;
}
template <int N>
__device__ inline void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// 12 wait states after the products that wrote one VGPR accumulator.
__device__ inline void mma_guard_s(f32x16& x) { asm volatile("s_nop 7\n\ts_nop 4" : "+v"(x)); }

// LDS instructions of the fragment reads issued after fragment m's (those of m+1 .. m+PF-1: one
// ds_read_b128 for a K fragment, two transposed reads for a V^T fragment).
constexpr int row_reads_after(int m, int PF, int MPT, int PH) {
  int n = 0;
  for (int k = 1; k < PF; ++k) n += ((m + k) % MPT) / PH < 2 ? 1 : 2;
  return n;
}

// Operand fragments are read this many products ahead of their use.
constexpr int kRowPF = 3;

// Slot (product index within the tile, after whose issue the piece runs) at which the softmax of
// 32-key block kb can start: right after its S block for one column group; for two, PF slots
// after the first epoch barrier that follows the publication of the partial tiles.
constexpr int row_sm_first(int kb, int DG, int PH, int EM, int PF) {
  const int p0 = (kb + 1) * PH;
  if (DG == 1) return p0;
  int bs = ((p0 + PF + EM - 1) / EM) * EM - PF;  // first barrier slot (e*EM - PF) at or after p0
  while (bs < p0) bs += EM;
  return bs + PF;
}
// Softmax micro-pieces of one 32-key block (each a few VALU instructions, so that no gap between
// two products holds more than the matrix core's shadow): logits and row maximum (4 raw pieces,
// one per 4-key group, or 8 when bias, masking and scaling are applied, two keys each), the
// maximum across the half-waves and the reference decision (3), then the exponential, row sum and
// packing of one key each (16).
constexpr int row_sm_logit_pieces(bool raw) { return raw ? 4 : 8; }
constexpr int row_sm_pieces(bool raw) { return row_sm_logit_pieces(raw) + 3 + 16; }
// the window a block's pieces are spread over: first .. last slot (inclusive)
constexpr int row_sm_last(int kb, int PH) { return (kb + 2) * PH - 2; }
// slot of piece k of block kb: evenly spread over the window (several per slot if it is short)
constexpr int row_sm_slot(int kb, int k, bool raw, int DG, int PH, int EM, int PF) {
  const int first = row_sm_first(kb, DG, PH, EM, PF);
  const int w = row_sm_last(kb, PH) - first + 1;
  return first + (k * w) / row_sm_pieces(raw);
}
constexpr bool row_sm_fits(int DG, int PH, int EM, int PF) {
  for (int kb = 0; kb < 2; ++kb)
    if (row_sm_first(kb, DG, PH, EM, PF) > row_sm_last(kb, PH)) return false;
  return true;
}
// Slot at which load i of the epoch refilled after the barrier at slot bs is issued: spread over
// the slots that follow the barrier, within the tile.
// Slot of load q (one sub-tile per wave) of the refill after the barrier at slot bs: the refill's
// loads are spread evenly over the epoch that follows (a burst of loads would fill the
// texture-address queue and stall the issuing wave while the matrix core drains), all within
// the tile and before the next barrier's wait.
constexpr int row_load_step(int EM, int nloads) { return EM / nloads > 1 ? EM / nloads : 1; }
constexpr int row_load_slot(int bs, int q, int step, int MPT) {
  return bs + 1 + q * step < MPT ? bs + 1 + q * step : MPT - 1;
}

// Tile variants.  A raw tile has every key taking part for every row of the workgroup and no mask,
// under a positive scale: the row maximum is taken over the raw dot products (scaling by a
// positive factor keeps the order) and the scale is folded into the exponent,
// p = exp2(s * scale_log2 - m).  Other tiles form the logits explicitly (scale, mask bias, -inf
// for keys past Nkv or past the causal limit).  MODE selects the kernel's tiles: kRowGeneral (every
// tile explicit), kRowRaw (every tile raw: no mask, no causal limit, whole tiles), kRowSplit (no
// mask: the tiles that every row of the workgroup sees whole are raw, the rest (the causal
// diagonal, a partial last tile) explicit, in two successive loops), kRowMaskF32 (every tile
// explicit, with an fp32 additive mask whose rows are
// staged through LDS: whole 128-byte lines per direct-to-LDS load, one tile ahead, instead of
// scattered 16-byte loads per lane), kRowMaskU8 (the same staging for a boolean byte mask: 32-byte
// row blocks, a zero byte excludes the key).  The launcher picks the variant.  Attention dropout is a
// separate flag (DROP) on the raw, split and general variants: each weight whose keep bit is clear is
// left out of P V, and O is scaled by 1 / (1 - p) at the end; the row sums and the LSE keep every
// weight.
enum RowMode { kRowGeneral = 0, kRowRaw = 1, kRowSplit = 2, kRowMaskF32 = 3, kRowMaskU8 = 4 };

// Loads (per wave) issued in slot x of a tile: load q of the refill after the barrier at slot
// e*EM - PF goes to row_load_slot(...).
constexpr int row_loads_at(int x, int MPT, int EM, int PF, int NL) {
  int n = 0;
  for (int e = 1; e * EM - PF < MPT; ++e)
    for (int q = 0; q < NL; ++q)
      if (row_load_slot(e * EM - PF, q, row_load_step(EM, NL), MPT) == x) ++n;
  return n;
}
// Loads issued after the staged mask rows of block kb (sent in slot nb of one tile, after that
// slot's refills) and before the wait of the last barrier at or before the next tile's read slot:
// they must be at least the number the barrier waits leave in flight, so that the in-order
// completion of loads has finished the mask rows by then.
constexpr bool row_mask_covered(int first, int MPT, int EM, int PF, int NL, int LA) {
  int nb = first;
  while ((nb + PF) % EM != 0) ++nb;
  int rd = first - PF, bl = rd;
  while ((bl + PF) % EM != 0) --bl;
  int n = 0;
  for (int x = nb + 1; x < MPT; ++x) n += row_loads_at(x, MPT, EM, PF, NL);
  for (int x = 0; x < bl; ++x) n += row_loads_at(x, MPT, EM, PF, NL);
  return bl >= 0 && n >= (LA - 1) * NL;
}

// Every staged-mask or exchange reuse below relies on an epoch barrier inside [first, last].
constexpr bool row_barrier_within(int first, int last, int EM, int PF) {
  for (int b = first; b <= last; ++b)
    if ((b + PF) % EM == 0) return true;
  return false;
}

// VL: runtime layouts: a packed variable-length batch (FwdArgs::cu_q: per-sequence lengths, offsets
// and LSE layout) or a strided dense one, both with runtime strides; the contiguous dense layout
// keeps them compile-time.
template <typename T, int D, int MODE, bool VL, bool DROP = false>
__global__ __launch_bounds__(256) void ffpa_fwd_row_kernel(FwdArgs a) {
  using RT = RowTiling<D, MODE == kRowMaskF32 || MODE == kRowMaskU8>;
  using E = Elem<T>;
  static_assert(RT::OK, "no ring plan for this head dim");
  constexpr int DG = RT::DG, DW = RT::DW, NSUB = RT::NSUB, BR = RT::BR, GPP = RT::GPP;
  constexpr int MPT = RT::MPT, EM = RT::EM, BI = RT::BI, NG = RT::NG, LA = RT::LA, EPT = RT::EPT;
  constexpr int CGB = NG * 4096;  // bytes of one column group's sub-tiles in the ring
  constexpr int PF = kRowPF;     // operand fragments are read this many products ahead
  constexpr int NFR = PF < 4 ? 4 : 8;  // fragment registers in rotation (at least PF + 1, dividing MPT)
  constexpr int BC = 64;
  constexpr int PH = 2 * NSUB;   // products per phase
  static_assert(MPT % NFR == 0, "the fragment rotation must line up with the tile");
  static_assert(PF < EM && LA >= 2, "ring plan");
  static_assert(RT::RING <= 2 * 65536 && (DG == 1 || CGB <= 65536), "LDS address windows");
  static_assert(row_sm_fits(DG, PH, EM, PF), "softmax schedule does not fit the phases");
  // the second block's mask biases are requested once the first block's logits are formed
  constexpr int BIAS1_SLOT = row_sm_slot(0, row_sm_logit_pieces(false), false, DG, PH, EM, PF);
  static_assert(BIAS1_SLOT < row_sm_first(1, DG, PH, EM, PF), "mask biases before their use");
  constexpr int NL = BI * DG;                        // loads per wave per epoch
  constexpr int LSTEP = row_load_step(EM, NL);
  static_assert(1 + (NL - 1) * LSTEP < EM, "the loads after a barrier end before the next one");

  constexpr bool MASK_LDS = MODE == kRowMaskF32 || MODE == kRowMaskU8;  // staged mask rows
  constexpr bool MASK_U8 = MODE == kRowMaskU8;
  constexpr int MESZ = MASK_U8 ? 1 : 4;  // bytes per staged mask element
  constexpr int MROWB = 32 * MESZ;       // bytes of one row's 32-key block
  static_assert(!DROP || !MASK_LDS, "dropout runs without a staged mask");
  constexpr int LDS_MAIN = RT::LDS_BYTES + (MASK_LDS ? RT::MASKB : 0);
  // the epilogue stages each wave's O block through LDS once the ring is no longer read
  constexpr int LDS_BYTES = LDS_MAIN > 4 * o_stage_bytes<DW>() ? LDS_MAIN : 4 * o_stage_bytes<DW>();
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  // the partner's partial of block 0 is read (after a barrier, complete PF products later) before
  // block 1's partial overwrites the single exchange buffer: a barrier must separate the two
  static_assert(DG == 1 || row_barrier_within(row_sm_first(0, DG, PH, EM, PF), 2 * PH - 1, EM, PF),
                "exchange reuse needs a barrier in between");
  // staged mask of block kb: read at slot row_sm_first(kb) - PF, complete at row_sm_first(kb); the
  // next tile's rows are loaded after the first barrier that follows (all waves done reading)
  static_assert(!MASK_LDS || (row_sm_first(0, DG, PH, EM, PF) >= PF &&
                              row_barrier_within(row_sm_first(0, DG, PH, EM, PF), MPT - 1, EM, PF) &&
                              row_barrier_within(row_sm_first(1, DG, PH, EM, PF), MPT - 1, EM, PF)),
                "mask staging schedule");
  static_assert(!MASK_LDS || (row_mask_covered(row_sm_first(0, DG, PH, EM, PF), MPT, EM, PF, BI * DG, LA) &&
                              row_mask_covered(row_sm_first(1, DG, PH, EM, PF), MPT, EM, PF, BI * DG, LA)),
                "staged mask rows must be complete at the barrier before their reads");

  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (!VL) clock_stamp(a.stamps, 0);  // (the runtime-layout variants have no register to spare)
  const int dg = DG == 1 ? 0 : (wave & 1);
  const int rg = DG == 1 ? wave : (wave >> 1);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item (b, hq, q tile); consecutive items share an XCD's L2.  A packed batch sizes the
  // grid by its longest sequence; items past their sequence's query length leave at once (the
  // whole workgroup, before any barrier).
  const int nqt = (a.Nq + BR - 1) / BR;
  const int total = a.B * a.Hq * nqt;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  // packed: head-major order, so that each XCD's share holds whole heads over every sequence (the
  // sequences' lengths differ; the heads' work does not)
  // dense: items (b, KV head, q tile, query head of the group) with the group's query heads
  // fastest, so that the G heads sharing a KV head take the same query tile together and stream the
  // same K/V tiles at the same time (one copy in L2)
  int qt, hq, b;
  const bool head_major = VL && a.cu_q != nullptr;
  if (head_major) {
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
  if (a.causal) qt = nqt - 1 - qt;  // heaviest tiles first
  // wave-uniform: kept in SGPRs (the divisions above run on the vector unit)
  qt = __builtin_amdgcn_readfirstlane(qt);
  hq = __builtin_amdgcn_readfirstlane(hq);
  b = __builtin_amdgcn_readfirstlane(b);
  const int hk = hq / a.group;
  const int r0 = qt * BR;
  int Nq = a.Nq, Nkv = a.Nkv;
  const int q_rs = VL ? a.q_sr : D;    // row strides (elements)
  const int kv_rs = VL ? a.kv_sr : D;
  const int o_rs = VL ? a.o_sr : D;
  int64_t q_base = (int64_t)(b * a.Hq + hq) * Nq * D, k_base = (int64_t)(b * a.Hkv + hk) * Nkv * D;
  int64_t v_base = k_base, o_base = q_base;
  int64_t lse_base = (int64_t)(b * a.Hq + hq) * Nq;
  if constexpr (VL) {
    if (a.cu_q != nullptr) {
      const SeqRange sr = seq_range(a, b);
      Nq = sr.nq;
      Nkv = sr.nkv;
      q_base = (int64_t)sr.q0 * q_rs + hq * a.q_sh;
      k_base = (int64_t)sr.k0 * kv_rs + hk * a.k_sh;
      v_base = (int64_t)sr.k0 * kv_rs + hk * a.v_sh;
      o_base = (int64_t)sr.q0 * o_rs + hq * a.o_sh;
      lse_base = (int64_t)hq * a.Tq + sr.q0;
      if (r0 >= Nq) return;
    } else {
      q_base = b * a.q_sb + hq * a.q_sh;
      k_base = b * a.k_sb + hk * a.k_sh;
      v_base = b * a.v_sb + hk * a.v_sh;
      o_base = b * a.o_sb + hq * a.o_sh;
    }
  }
  const int rw0 = r0 + rg * 32;  // first row of this wave
  const int row = rw0 + l32;     // this lane's row
  // dropout: this lane's row of keep words (a row past Nq reads row Nq - 1; it is never stored)
  const uint32_t* keep_row = nullptr;
  if constexpr (DROP) keep_row = a.keep + ((int64_t)(b * a.Hq + hq) * Nq + (row < Nq ? row : Nq - 1)) * a.keep_w;
  const int col0 = dg * DW;
  const int off = Nkv - Nq;
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
  const int total_epochs = ntiles * EPT;

  // ---- ring loads: wave w fills rows 8w .. 8w+7 of every sub-tile (its w-th KiB): lane t takes
  // row 8w + t/8 and stores physical chunk t%8, i.e. logical chunk (t%8) ^ pi((row >> 1) & 7).
  // One descriptor per tensor head (its size ends at key Nkv, so rows past it read as zero); the
  // lane's byte offset = fixed lane part + tile part + a constant per group.
  const int prow = 8 * wave + (lane >> 3);
  auto pi7 = [](int x) { return ((x & 1) << 2) | (x >> 1); };
  const uint32_t voff_lane = (uint32_t)((prow * kv_rs + ((lane & 7) ^ pi7((prow >> 1) & 7)) * 8) * 2);
  const int head_bytes = (int)((int64_t)Nkv * kv_rs * 2);
  const uint32_t rows32_bytes = (uint32_t)(32 * kv_rs * 2);  // packed: byte step of 32 key rows
  const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, head_bytes, 0x00020000);
  char* const ring_w = smem + wave * 1024;
  // sub-tile of column group cg of group gi of tile j + TD, with vt = voff_lane + (byte offset of tile j)
  auto issue_sub = [&](uint32_t vt, auto td_c, auto gi_c, auto cg_c) {
    constexpr int TD = decltype(td_c)::value, gi = decltype(gi_c)::value, cg = decltype(cg_c)::value;
    constexpr int ph = gi / GPP, w = gi % GPP;
    if constexpr (!VL) {
      constexpr uint32_t cst = (uint32_t)(((TD * BC + (ph & 1) * 32) * D + cg * DW + 64 * w) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ph < 2 ? rsrc_k : rsrc_v,
                                               (FFPA_LDS void*)(ring_w + cg * CGB + (gi % NG) * 4096), 16, vt + cst,
                                               0, 0, 0);
    } else {
      // the row part of the offset is a runtime multiple of the row stride: a scalar offset
      const uint32_t so = (uint32_t)(2 * TD + (ph & 1)) * rows32_bytes + (uint32_t)((cg * DW + 64 * w) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ph < 2 ? rsrc_k : rsrc_v,
                                               (FFPA_LDS void*)(ring_w + cg * CGB + (gi % NG) * 4096), 16, vt, so,
                                               0, 0);
    }
  };
  auto issue_group = [&](uint32_t vt, auto td_c, auto gi_c) {
    static_for<DG>([&](auto cg_c) { issue_sub(vt, td_c, gi_c, cg_c); });
  };
  // group i of local epoch E (E >= EPT: of a later tile) relative to tile j, if that tile exists
  auto issue_epoch_group = [&](int j, uint32_t vt, auto e_c, auto i_c) {
    constexpr int E = decltype(e_c)::value, I = decltype(i_c)::value;
    constexpr int TD = E / EPT, EL = E % EPT;
    if (j + TD >= ntiles) return;
    issue_group(vt, std::integral_constant<int, TD>{}, std::integral_constant<int, EL * BI + I>{});
  };
  // load q (group q / DG, column group q % DG) of local epoch E relative to tile j
  auto issue_epoch_load = [&](int j, uint32_t vt, auto e_c, auto q_c) {
    constexpr int E = decltype(e_c)::value, Q = decltype(q_c)::value;
    constexpr int TD = E / EPT, EL = E % EPT;
    if (j + TD >= ntiles) return;
    issue_sub(vt, std::integral_constant<int, TD>{}, std::integral_constant<int, EL * BI + Q / DG>{},
              std::integral_constant<int, Q % DG>{});
  };
  auto issue_epoch = [&](int j, uint32_t vt, auto e_c) {
    static_for<BI>([&](auto i_c) { issue_epoch_group(j, vt, e_c, i_c); });
  };
  // this wave's loads of global epoch eg are complete (the LA-1 later epochs may be in flight)
  auto wait_epoch = [&](int eg) {
    if (eg + LA - 1 < total_epochs) vm_wait<(LA - 1) * BI * DG>();
    else vm_wait<0>();
  };

  // ---- operand fragment addresses (per lane; slot and step offsets are immediates)
  const uint32_t ring_addr = lds_addr(smem);
  const uint32_t cgb = ring_addr + dg * CGB;  // this wave's column group's sub-tiles
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_chunk = 2 * (g16 & 1) + ((i16 & 3) >> 1);
  const int tr_within = 8 * (i16 & 1);
  const int vkeyA = (g16 >> 1) * 4 + (i16 >> 2);
  // K fragment (32 keys x 16 columns; 32-column half h of the sub-tile, 16-column step ks): key
  // l32, logical chunk 4h + 2ks + hi.  V^T fragment (half h, 16-key step ks): two transposed reads
  // of keys vkeyA and vkeyA + 8 (+16 per step, an immediate: the swizzle's row term repeats every
  // 16 rows), logical chunk 4h + tr_chunk.
  uint32_t ka[2][2], va[2], vb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) ka[h][ks] = cgb + l32 * 128 + ((4 * h + 2 * ks + hi) ^ pi7((l32 >> 1) & 7)) * 16;
    va[h] = cgb + vkeyA * 128 + ((4 * h + tr_chunk) ^ pi7((vkeyA >> 1) & 7)) * 16 + tr_within;
    vb[h] = cgb + (vkeyA + 8) * 128 + ((4 * h + tr_chunk) ^ pi7(((vkeyA + 8) >> 1) & 7)) * 16 + tr_within;
  }

  i32x4 kfr[NFR];
  i32x2 vlo[NFR], vhi[NFR];
  // fragment of product M of a tile (M >= MPT: the next tile's product M - MPT, same slots); the
  // slot and step offsets are instruction immediates on a few per-lane base addresses
  auto read_frag = [&](auto mc) {
    constexpr int M = decltype(mc)::value;
    constexpr int mm = M % MPT;
    constexpr int ph = mm / PH, s = (mm % PH) / 2, ks = mm % 2;
    constexpr int gi = ph * GPP + s / 2, h = s & 1;
    constexpr int ofs = (gi % NG) * 4096;
    constexpr uint32_t win = ofs >= 65536 ? 65536u : 0u;
    constexpr int r = M % NFR;
    if constexpr (ph < 2) {
      kfr[r] = lds_read_b128_async<(ofs & 65535)>(ka[h][ks] + win);
    } else {
      constexpr int o2 = (ofs & 65535) + ks * 2048;
      static_assert(o2 < 65536, "ds offset field");
      vlo[r] = lds_read_tr_async<o2>(va[h] + win);
      vhi[r] = lds_read_tr_async<o2>(vb[h] + win);
    }
  };

  const int64_t mask_bh = (int64_t)b * a.msb + (int64_t)hq * a.msh;
  // (the staged-mask modes always have one)
  const bool has_mask = MASK_LDS || a.mask_kind != kMaskNone;
  // explicit logits are formed in natural units, scale S + bias in one operation, and enter the
  // log2-domain softmax through its maximum and exponent
  const float scale_nat = a.scale_log2 * kLn2;

  // partial-S exchange (two column groups): [wave][4 x 1 KiB], 16 bytes per lane, one block at a time
  const uint32_t ex_mine = ring_addr + RT::RING + wave * 4096 + lane * 16;
  const uint32_t ex_partner = ring_addr + RT::RING + (wave ^ 1) * 4096 + lane * 16;

  // ---- staged mask: block kb of the workgroup's rows at MASK_OFF + kb * BR * MROWB, row r's 32 keys
  // in MROWB bytes, as eight chunks of four keys (one per lane of a load).  fp32: 16-byte chunks
  // swizzled like the K/V sub-tiles.  Bytes: 4-byte chunks reordered so that chunk position
  // 4 hi + g holds keys 8g + 4hi .. +3, i.e. the 16 keys of one half-wave are one 16-byte read.
  // Wave w loads rows 8(w + 4i) .. +7 (i < BR/32); keys are whole tiles (Nkv % 64 == 0), rows past
  // Nq read as zero through the descriptor (their results are never stored).
  constexpr int MASK_OFF = RT::RING + RT::EXCH;
  constexpr int MLOADS = BR / 32;  // loads per wave per block
  const int mask_bytes = MASK_LDS ? (int)(((int64_t)(Nq - 1) * a.msq + Nkv) * MESZ) : 0;
  const __amdgpu_buffer_rsrc_t rsrc_m =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.mask + (MASK_LDS ? mask_bh * MESZ : 0)), (short)0,
                                        mask_bytes, 0x00020000);
  const int mrow0 = 8 * wave + (lane >> 3);  // row of load i: mrow0 + 32 i (same swizzle phase)
  const int mchunk = MASK_U8 ? 2 * (lane & 3) + ((lane >> 2) & 1) : ((lane & 7) ^ pi7((mrow0 >> 1) & 7));
  const uint32_t mvoff = (uint32_t)(((int64_t)(r0 + mrow0) * a.msq + mchunk * 4) * MESZ);
  const uint32_t mrow_step = (uint32_t)(32 * a.msq * MESZ);
  // rows of tile jt's block kb into the staging buffer
  auto issue_mask = [&](int jt, int kb) {
    const uint32_t kofs = (uint32_t)((jt * BC + 32 * kb) * MESZ);
#pragma unroll
    for (int i = 0; i < MLOADS; ++i) {
      FFPA_LDS void* dst = (FFPA_LDS void*)(smem + MASK_OFF + kb * BR * MROWB + (wave + 4 * i) * 8 * MROWB);
      // bytes per lane: a literal (the builtin checks it before the template is instantiated)
      if constexpr (MASK_U8) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_m, dst, 4, mvoff + i * mrow_step + kofs, 0, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_m, dst, 16, mvoff + i * mrow_step + kofs, 0, 0, 0);
    }
  };
  // this lane's 16 biases of block kb (keys 8g + 4hi + e): 4 reads (bytes: 1), complete once a
  // fragment read issued after them has been waited for
  const int mr = rg * 32 + l32;  // the lane's row within the workgroup
  const uint32_t mrd = ring_addr + MASK_OFF + mr * MROWB;
  const int mswz = pi7((mr >> 1) & 7);

  // ---- prologue: this wave's Q rows (its DW columns, in VGPRs for the whole key loop), then the
  // first tile's mask rows and epochs 0 .. LA-1 in flight behind them, so that the Q rows and the
  // ring's first keys are fetched together; then Q, epoch 0 (and the mask, issued before it)
  // visible, the first PF fragments requested
  i32x4 qf[DW / 16];
  {
    const int qrow = row < Nq ? row : Nq - 1;
    const i32x4* src = (const i32x4*)(qg + (int64_t)qrow * q_rs + col0 + hi * 8);
#pragma unroll
    for (int k = 0; k < DW / 16; ++k) {
      // runtime layouts may carry a padded head dim: columns from dcols on are not read and hold zero
      if constexpr (VL) qf[k] = col0 + hi * 8 + 16 * k < a.dcols ? src[k * 2] : i32x4{0, 0, 0, 0};
      else qf[k] = src[k * 2];
    }
  }
  if constexpr (MASK_LDS) {
    issue_mask(0, 0);
    issue_mask(0, 1);
  }
  // the first tile's epochs are issued whether or not the tile exists (with no key tile their rows
  // land in the ring unread, and the wait below completes them before anything else uses the LDS):
  // a load on one path only would make the compiler wait for every load before the Q rows' use
  static_for<LA>([&](auto e_c) {
    constexpr int E = decltype(e_c)::value;
    if constexpr (E < EPT) {
      static_for<BI>([&](auto i_c) {
        issue_group(voff_lane, std::integral_constant<int, 0>{}, std::integral_constant<int, E * BI + decltype(i_c)::value>{});
      });
    } else {
      issue_epoch(0, voff_lane, e_c);
    }
  });
  // complete here, and redefine through the assembler: the compiler then has no load of these
  // registers to wait for inside the key loop (where it would drain the prefetch ring)
#pragma unroll
  for (int k = 0; k < DW / 16; ++k) asm volatile("" : "+v"(qf[k]));
  wait_epoch(0);
  __builtin_amdgcn_s_barrier();
  issue_epoch(0, voff_lane, std::integral_constant<int, LA>{});
  static_for<PF>([&](auto mc) { read_frag(mc); });

  f32x16 o_acc[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    o_acc[s] = f32x16{};
    asm volatile("" : "+a"(o_acc[s]));
  }
  float m_run = kNegInf;  // running reference maximum of this lane's row (log2 domain)
  float l_lane = 0.f;     // sum of this lane's probabilities (the other half-wave holds the rest)
  // EDGE: the tile may touch the key tail or the causal diagonal (explicit tiles test each entry
  // then); tiles known to be clear of both skip the tests
  auto tile_body = [&](const int j, auto raw_c, auto edge_c) {
    constexpr bool RAW = decltype(raw_c)::value;
    constexpr bool EDGE = decltype(edge_c)::value;
    constexpr int NLP = row_sm_logit_pieces(RAW);
    constexpr int NSP = row_sm_pieces(RAW);
    const int key0 = j * BC;
    const bool tail = key0 + BC > Nkv;
    const bool diag = a.causal && (key0 + BC - 1 > rw0 + off);
    const bool edge = RAW || !EDGE ? false : (tail || diag);
    // last key of the tile this lane's row may see (keys past Nkv and past the causal limit are
    // excluded), relative to the tile's first key
    int edge_lim = Nkv - 1;
    if (a.causal) edge_lim = edge_lim < row + off ? edge_lim : row + off;
    edge_lim -= key0;
    uint32_t vt = voff_lane + (uint32_t)j * 2 * rows32_bytes;
    asm volatile("" : "+v"(vt));  // keeps the per-group constants from being hoisted as 32 live registers
    LogitCtx ctx{a.mask, mask_bh, a.msq, Nq, Nkv, key0, rw0, off, a.causal, edge, a.scale_log2, l32, hi};

    f32x16 s_acc[2];     // S^T of the two 32-key blocks; overwritten in place by the logits
    f32x4 part[2][4];    // the partner's partial S (two column groups)
    f32x4 bias[2][4];    // mask biases
    float lmax[2], m_new[2], alpha[2], psum[2];
    bool need[2];
    i32x4 pk[2][2];      // P^T operands (bf16/fp16 pairs) of block kb, 16-key step ks

    if (!RAW && !MASK_LDS && has_mask)
      load_bias_dispatch<1, 4>(*reinterpret_cast<f32x4(*)[1][4]>(&bias[0][0]), ctx, key0, a.mask_kind,
                               a.mask_vec && !tail);
    // dropout: the keep words of the tile's two 32-key blocks (a block past the row's last word reads
    // the last word; its keys are excluded anyway)
    uint32_t kw[2] = {0u, 0u};
    if constexpr (DROP) {
      const int wl = a.keep_w - 1, w0 = key0 >> 5;
      kw[0] = keep_row[w0 < wl ? w0 : wl];
      kw[1] = keep_row[w0 + 1 < wl ? w0 + 1 : wl];
    }

    float mt[2], m_old[2], mref[2], pv[2][2];
    // softmax micro-piece k of block kb (see row_sm_pieces)
    auto sm_micro = [&](int kb, int k) {
      if (k < NLP) {
        if constexpr (RAW) {
          const int g = k;
          float mx = g == 0 ? kNegInf : lmax[kb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (DG == 2) s_acc[kb][4 * g + e] += part[kb][g][e];
            mx = __builtin_fmaxf(mx, s_acc[kb][4 * g + e]);
          }
          lmax[kb] = mx;
          // Pins: the results of every piece are redefined by an empty volatile statement in its
          // slot, so that no pass sinks the arithmetic past the branches of later slots to its
          // use (which would bunch it up in front of the products and lose the overlap).
          if constexpr (DG == 2) asm volatile("" : "+v"(s_acc[kb]), "+v"(lmax[kb]));
          else asm volatile("" : "+v"(lmax[kb]));
        } else {
          const int g = k >> 1, e0 = 2 * (k & 1);
          // key 8g + e of this lane's block-relative keys (8g + 4hi + e) is excluded past lim
          const int lim = edge_lim - 32 * kb - 4 * hi;
          float mx = k == 0 ? kNegInf : lmax[kb];
#pragma unroll
          for (int e = e0; e < e0 + 2; ++e) {
            float x = s_acc[kb][4 * g + e];
            if constexpr (DG == 2) x += part[kb][g][e];
            if constexpr (MASK_U8) {
              // byte e of word g: nonzero takes part (through a scalar: a bit cast of the vector
              // element itself would read element 0)
              const float wf = bias[kb][0][g];
              x = ((__builtin_bit_cast(uint32_t, wf) >> (8 * e)) & 0xffu) ? x * scale_nat : kNegInf;
            } else if (has_mask) {
              x = __builtin_fmaf(x, scale_nat, bias[kb][g][e]);
            } else {
              x *= scale_nat;
            }
            if (edge) x = 8 * g + e > lim ? kNegInf : x;
            mx = __builtin_fmaxf(mx, x);
            s_acc[kb][4 * g + e] = x;
          }
          lmax[kb] = mx;
          asm volatile("" : "+v"(s_acc[kb]), "+v"(lmax[kb]));
        }
      } else if (k == NLP) {
        mt[kb] = max_halves(lmax[kb]) * (RAW ? a.scale_log2 : kLog2e);
        m_old[kb] = m_run;
        asm volatile("" : "+v"(mt[kb]), "+v"(m_old[kb]));
      } else if (k == NLP + 1) {
        const float mo = m_old[kb];
        const bool nd = mo != kNegInf && mt[kb] > mo + kRescaleSlack;
        const float mn = mo == kNegInf ? mt[kb] : (nd ? mt[kb] : mo);
        need[kb] = nd;
        m_new[kb] = mn;
        m_run = mn;
        mref[kb] = mn == kNegInf ? 0.f : mn;
        asm volatile("" : "+v"(m_new[kb]), "+v"(mref[kb]));
      } else if (k == NLP + 2) {
        alpha[kb] = need[kb] ? __builtin_amdgcn_exp2f(m_old[kb] - m_new[kb]) : 1.f;
        psum[kb] = 0.f;
        asm volatile("" : "+v"(alpha[kb]), "+v"(psum[kb]));
        if constexpr (DROP) {
          kw[kb] >>= 4 * hi;  // this lane's keys 8g + 4hi + e sit at bits 8g + e
          asm volatile("" : "+v"(kw[kb]));
        }
      } else {
        const int i = k - NLP - 3;  // key 0..15 of this lane's 16 in the block
        const int g = i >> 2, e = i & 3;
        const float sv = s_acc[kb][4 * g + e];
        const float x = __builtin_fmaf(sv, RAW ? a.scale_log2 : kLog2e, -mref[kb]);
        const float p = __builtin_amdgcn_exp2f(x);
        psum[kb] += p;
        float pd = p;  // the weight that enters P V
        if constexpr (DROP) {
          // all ones when the key's keep bit is set, zero otherwise
          const int sel = -(int)((kw[kb] >> (8 * g + e)) & 1u);
          pd = __builtin_bit_cast(float, sel & __builtin_bit_cast(int, p));
        }
        if ((e & 1) == 0) {
          pv[kb][0] = pd;
          asm volatile("" : "+v"(pv[kb][0]), "+v"(psum[kb]));
        } else {
          pk[kb][g >> 1][2 * (g & 1) + (e >> 1)] = (int)pack2<T>(pv[kb][0], pd);
          asm volatile("" : "+v"(pk[kb][g >> 1]), "+v"(psum[kb]));
        }
      }
    };
    // l and O follow block kb's new reference (O holds exactly the blocks before kb)
    auto apply_rescale = [&](int kb) {
      l_lane = l_lane * alpha[kb] + psum[kb];
      if (__builtin_amdgcn_ballot_w64(need[kb]) != 0) {
        mma_guard_all<NSUB>(o_acc);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          o_acc[s] *= alpha[kb];
          asm volatile("" : "+a"(o_acc[s]));
        }
      }
    };

    static_for<MPT>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int ph = m / PH, s = (m % PH) / 2, ks = m % 2;
      constexpr int r = m % NFR;
      // ---- product m, once its fragment is complete: the LDS reads issued after fragment x are those
      // of the fragments x+1 .. x+PF-1 (any other LDS instruction issued later only waits longer)
      // (one wait per pair of products: before product m, m even, for fragments m and m + 1; the
      // reads issued after fragment m + 1 by then are those of fragments m + 2 .. m + PF - 1)
      if constexpr (m % 2 == 0) {
        constexpr int after = row_reads_after(m + 1, PF - 1, MPT, PH);
        static_assert(after <= 15, "lgkmcnt range");
        lgkm_wait<after>();
      }
      if (ph < 2) {
        if (s == 0 && ks == 0) E::mma_first(s_acc[ph], kfr[r], qf[2 * s + ks]);
        else E::mma_acc(s_acc[ph], kfr[r], qf[2 * s + ks]);
      } else {
        const i32x4 vf = i32x4{vlo[r][0], vlo[r][1], vhi[r][0], vhi[r][1]};
        // the probabilities were packed by VALU instructions before the phase began
        if constexpr (s == 0 && ks == 0) E::mma_acc_agpr(o_acc[s], vf, pk[ph - 2][ks]);
        else E::mma_acc_agpr_nonop(o_acc[s], vf, pk[ph - 2][ks]);
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- an S block finished one product ago: 12 wait states, then publish the partial
      if (m == PH || m == 2 * PH) {
        const int kb = m / PH - 1;
        mma_guard_s(s_acc[kb]);
        if constexpr (DG == 2) {
          const f32x16& x = s_acc[kb];
          const uint32_t dst = ex_mine;
          lds_write_b128_async<0>(dst, f32x4{x[0], x[1], x[2], x[3]});
          lds_write_b128_async<1024>(dst, f32x4{x[4], x[5], x[6], x[7]});
          lds_write_b128_async<2048>(dst, f32x4{x[8], x[9], x[10], x[11]});
          lds_write_b128_async<3072>(dst, f32x4{x[12], x[13], x[14], x[15]});
        }
      }
      if (!RAW && !MASK_LDS && m == BIAS1_SLOT && has_mask)
        load_bias_dispatch<1, 4>(*reinterpret_cast<f32x4(*)[1][4]>(&bias[1][0]), ctx, key0 + 32, a.mask_kind,
                                 a.mask_vec && !tail);

      // ---- epoch boundary: the next epoch's groups become visible; the slots of the epoch before
      // last are refilled LA epochs ahead
      if ((m + PF) % EM == 0) {
        const int eg = j * EPT + (m + PF) / EM;  // (m + PF) / EM == EPT: the next tile's first epoch
        int pub = -1;  // block whose partial tiles are read after this barrier (two column groups)
        if (DG == 2) {
          if (m + PF == row_sm_first(0, DG, PH, EM, PF)) pub = 0;
          if (m + PF == row_sm_first(1, DG, PH, EM, PF)) pub = 1;
        }
        if (eg < total_epochs) {
          // a partial published fewer than PF products ago may still be in flight
          if (pub >= 0 && m - (pub + 1) * PH < PF) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          wait_epoch(eg);
          __builtin_amdgcn_s_barrier();
        }
        if (pub >= 0) {
          const uint32_t src = ex_partner;
          part[pub][0] = lds_read_f4_async<0>(src);
          part[pub][1] = lds_read_f4_async<1024>(src);
          part[pub][2] = lds_read_f4_async<2048>(src);
          part[pub][3] = lds_read_f4_async<3072>(src);
        }
      }

      // ---- refills of the slots freed by the last barrier, spread over the following slots
      static_for<EPT + 1>([&](auto eb_c) {
        constexpr int eb = decltype(eb_c)::value;  // barrier of local epoch eb sits at slot eb*EM - PF
        constexpr int bs = eb * EM - PF;
        if constexpr (bs >= 0 && bs < MPT) {
          static_for<NL>([&](auto q_c) {
            if constexpr (row_load_slot(bs, decltype(q_c)::value, LSTEP, MPT) == m)
              issue_epoch_load(j, vt, std::integral_constant<int, eb + LA>{}, q_c);
          });
        }
      });

      // ---- staged mask: this tile's reads ahead of the block's logits (before the fragment read of
      // this slot, so that waiting for that fragment completes them), and the next tile's rows
      // after the first barrier that follows the reads' completion
      if constexpr (MASK_LDS) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int first = row_sm_first(kb, DG, PH, EM, PF);
          if (m == first - PF) {
            const uint32_t base = mrd + kb * BR * MROWB;
            if constexpr (MASK_U8) {
              bias[kb][0] = lds_read_f4_async<0>(base + hi * 16);  // key bytes, as four raw words
            } else {
              bias[kb][0] = lds_read_f4_async<0>(base + ((0 + hi) ^ mswz) * 16);
              bias[kb][1] = lds_read_f4_async<0>(base + ((2 + hi) ^ mswz) * 16);
              bias[kb][2] = lds_read_f4_async<0>(base + ((4 + hi) ^ mswz) * 16);
              bias[kb][3] = lds_read_f4_async<0>(base + ((6 + hi) ^ mswz) * 16);
            }
          }
          int nb = first;
          while ((nb + PF) % EM != 0) ++nb;
          if (m == nb && j + 1 < ntiles) issue_mask(j + 1, kb);
        }
      }

      // ---- the fragment PF products ahead (the last ones: the next tile's first products)
      read_frag(std::integral_constant<int, m + PF>{});

      // ---- softmax micro-pieces
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // the staged biases were read before a fragment whose completion was waited for just
        // before this product: they are complete
        if (MASK_LDS && m == row_sm_first(kb, DG, PH, EM, PF))
          asm volatile("" : "+v"(bias[kb][0]), "+v"(bias[kb][1]), "+v"(bias[kb][2]), "+v"(bias[kb][3]));
        // the partner's partial was read before a fragment whose completion was waited for just
        // before this product: it is complete
        if (DG == 2 && m == row_sm_first(kb, DG, PH, EM, PF))
          asm volatile("" : "+v"(part[kb][0]), "+v"(part[kb][1]), "+v"(part[kb][2]), "+v"(part[kb][3]));
#pragma unroll
        for (int k = 0; k < NSP; ++k)
          if (row_sm_slot(kb, k, RAW, DG, PH, EM, PF) == m) sm_micro(kb, k);
      }
      if constexpr (m == 2 * PH - 1) apply_rescale(0);
      if constexpr (m == 3 * PH - 1) apply_rescale(1);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // tiles whose keys all lie below Nkv and (causal) whose last key is visible to the workgroup's
  // first row are whole for all its rows
  int nwhole = (a.causal ? r0 + off + 1 : Nkv) / BC;
  nwhole = nwhole < ntiles ? nwhole : ntiles;
  nwhole = nwhole > 0 ? nwhole : 0;
  if constexpr (MODE == kRowRaw) {
    for (int j = 0; j < ntiles; ++j) tile_body(j, std::true_type{}, std::false_type{});
  } else if constexpr (MODE == kRowGeneral || MODE == kRowMaskF32 || MODE == kRowMaskU8) {
    // (the dropout variant at D = 1024 has no registers for a second tile body: one loop, tested)
    if constexpr (DROP && D == 1024) {
      for (int j = 0; j < ntiles; ++j) tile_body(j, std::false_type{}, std::true_type{});
    } else {
      for (int j = 0; j < nwhole; ++j) tile_body(j, std::false_type{}, std::false_type{});
      for (int j = nwhole; j < ntiles; ++j) tile_body(j, std::false_type{}, std::true_type{});
    }
  } else {
    static_assert(MODE == kRowSplit, "tile mode");
    for (int j = 0; j < nwhole; ++j) tile_body(j, std::true_type{}, std::false_type{});
    for (int j = nwhole; j < ntiles; ++j) tile_body(j, std::false_type{}, std::true_type{});
  }
  vm_wait<0>();
  // the last tile read the next tile's first fragments (never used): their registers stay reserved until
  // those reads have landed, or the epilogue could reuse one that an in-flight read still writes
  static_assert(NFR == 4, "fragment registers tied below");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(kfr[0]), "+v"(kfr[1]), "+v"(kfr[2]), "+v"(kfr[3]), "+v"(vlo[0]), "+v"(vlo[1]), "+v"(vlo[2]),
                 "+v"(vlo[3]), "+v"(vhi[0]), "+v"(vhi[1]), "+v"(vhi[2]), "+v"(vhi[3])
               :
               : "memory");

  // ================= epilogue =================
  mma_guard_all<NSUB>(o_acc);
  const float l = sum_halves(l_lane);
  float inv = l > 0.f ? 1.f / l : 0.f;
  if constexpr (DROP) inv *= a.drop_scale;
  // O leaves through LDS in row-contiguous 16-byte stores; the runtime-layout variants at D = 1024 have
  // no registers to spare for the staging addresses and store straight from the accumulators
  constexpr bool STAGED_O = !(VL && D == 1024);
  if constexpr (STAGED_O) {
    // every wave is done with the ring before any wave's staged O overwrites it
    __builtin_amdgcn_s_barrier();
    // (with a padded head dim, a multiple of 8, the columns from dcols on are not stored)
    store_o_staged<T, DW, NSUB, !VL>(o_acc, inv, smem + wave * o_stage_bytes<DW>(),
                                     a.o + o_base + (int64_t)rw0 * o_rs + col0, o_rs, Nq - rw0,
                                     VL ? a.dcols - col0 : DW, lane);
  } else if (row < Nq) {
    uint16_t* orow = a.o + o_base + (int64_t)row * o_rs + col0;
    static_for<NSUB>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& acc = o_acc[s];
        i32x2 w;
        w[0] = (int)pack2<T>(acc[q4 * 4 + 0] * inv, acc[q4 * 4 + 1] * inv);
        w[1] = (int)pack2<T>(acc[q4 * 4 + 2] * inv, acc[q4 * 4 + 3] * inv);
        // four columns; with a padded head dim (a multiple of 8) either all or none lie below dcols
        if (col0 + s * 32 + q4 * 8 + hi * 4 < a.dcols) *(i32x2*)(orow + s * 32 + q4 * 8 + hi * 4) = w;
      }
      __builtin_amdgcn_sched_barrier(0);  // one column block at a time: few registers in flight
    });
  }
  if (row < Nq && a.lse != nullptr && dg == 0 && hi == 0) {
    const float lse = l > 0.f ? (m_run + __builtin_log2f(l)) * kLn2 : kNegInf;
    a.lse[lse_base + row] = lse;
  }
  if constexpr (!VL) clock_stamp(a.stamps, 1);
}

}  // namespace ffpa

// Chunked causal prefill against the paged KV cache, on MFMA.
//
// What is computed: [P2] "Unlocking long context ..." section 4.1 (exact
// attention, softmax(q K^T / sqrt(d)) V, with the causal flag of its flash
// attention call) and section 5.2 (a long prompt is processed in chunks, each
// chunk attending to the KV already written); [P3] www.mhpn.cn/news/2466452
// section 1.2 (tiles + online softmax: same flops, no n x n matrix in HBM);
// [P1] "Long-context inference engineering truths 2026 ..." section 3.1 (the
// running max / sum / rescaled accumulator per query row).  A call covers the
// keys [kv_begin, kv_end) only, so a prompt's KV can be cut into shards whose
// partial results are merged exactly afterwards (merge.hip).
//
// Prefill is a dense contraction (about 4*d flops per key per query row), so
// both products run on 32x32x16 MFMA:
//   S^T[t][r]  = K[t][:] . Q[r][:]      bf16; A = K tile (LDS), B = Q (registers)
//   O^T[d][r] += V^T[d][t] P^T[t][r]    fp16; A = V tile (LDS), B = P (registers)
// Computing S transposed puts one query row in each lane (plus its partner
// lane l^32), so a row's max and sum need at most one cross-lane step and the
// softmax weights are already laid out as the B operand of the second
// product.  V is converted to fp16 as it is staged (exact for bf16 values
// within fp16's range) so the weights enter P V with 11 significant bits
// instead of bf16's 8.  Over E4M3 pools ([P2] section 3.2) both products run
// in fp16: K is staged as its exact codes with each page's K scale applied
// to the scores, V dequantised while staged, q converted once.
//
// Workgroup = 8 waves = the NH query heads of one kv head that share K/V x NR
// blocks of 32 query rows (NH * NR = 8).  A 64-token K/V tile (4 pages) is
// gathered through the block table once per workgroup into a three-deep LDS
// ring, so one barrier per tile suffices: K pages go straight from memory to
// LDS (their pool order is already the order the score product reads), V
// pages pass through registers to be converted to fp16 and regrouped.  Each wave software-pipelines: the
// K Q^T products of tile j+1 are issued among the softmax instructions of tile
// j, so the matrix cores and the vector ALUs work at the same time.
// Workgroup i serves kv head i % Hkv, so with 8 kv heads every XCD streams one
// head's K/V through its own L2; heavier (later) row blocks are dispatched
// first.
#include "pkv_common.h"

namespace pkv {
namespace {

constexpr int BN = 64;                   // tokens per K/V tile (4 pages)
constexpr int ROWS_W = 32;               // query rows per wave
constexpr int NWAVE = 8;
constexpr int NTHREADS = 64 * NWAVE;
constexpr int NBUF = 3;                  // LDS ring of K/V tiles

// Sizes for head dimension D (64 or 128).
template <int D>
struct Geo {
  static constexpr int TILE = BN * D * 2;        // bytes of a V tile: 16 KiB at D 128
  static constexpr int KTILE = TILE;             // K tile: 4 pages as they are in the pool
  static constexpr int BUF = KTILE + TILE;       // one ring slot: K tile + V tile
  static constexpr int LDS = NBUF * BUF;
  // after the ring, 32 bytes per slot: the tile's four K scales (E4M3 pools)
  // and one byte per page, 1 when its scores may be used (see page_usable)
  static constexpr int META = 32;
  static constexpr int LDS_ALL = LDS + NBUF * META;
  static constexpr int PAGE = kBlock * D * 2;    // bytes of one page
  static constexpr int PAGE8 = kBlock * D;       // bytes of one E4M3 page
  static constexpr int W8 = PAGE8 / 128 / 4;     // 32-bit words of an E4M3 page per staging thread
  static constexpr int SPT = PAGE / 2048;        // 16-byte pieces per staging thread (128 per page)
  static constexpr int QC = D / 16;              // k-steps of the score product
  static constexpr int DT = D / 32;              // 32-dimension blocks of O
};
constexpr float kLazy = 8.0f;            // log2 headroom of the running max

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

struct PrefillParams {
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;                  // E4M3 pools: [num_blocks][hkv]
  const float* v_scale;
  int64_t block_stride_bytes;
  int num_blocks, hkv, hq, G;
  int NH, NR, HGR;                       // heads per workgroup, row blocks, head groups
  const uint16_t* q;
  int T, q_pos0;
  const int32_t* table;
  int maxb;
  int kv_begin, kv_end;
  int causal;
  float scale_log2;
  int row_tiles;                         // row tiles of 32 * NR rows
  uint16_t* out;
  float* out_lse;
  float* part_o;
  float* part_m;
  float* part_l;
};

// LDS K tile: the tile's 4 K pages copied as they are in the pool (fragment
// order): the 8 dimensions 32c + 8g .. +8 of token t of page pg sit at
// pg * PAGE + c * 1024 + (16 g + t) * 16.  The 16 lanes that read one k-step
// chunk of 16 consecutive tokens read 256 contiguous bytes.
template <int D>
__device__ __forceinline__ int k_lds_off(int t, int k8) {    // k8: index of the 8-dim chunk
  return (t >> 4) * Geo<D>::PAGE + (k8 >> 2) * 1024 + (((k8 & 3) << 4) + (t & 15)) * 16;
}

// LDS V tile: [4 pages][128 dims][32 B]; within a dimension the 16 tokens are
// stored as halves {0-3, 8-11} and {4-7, 12-15} (the token sets one 32x32x16
// k-step takes from each lane half), and the halves swap when (d >> 3) is odd.
template <int D>
__device__ __forceinline__ int v_lds_off(int page, int d, int half) {
  return page * (D * 32) + d * 32 + ((half ^ ((d >> 3) & 1)) << 4);
}

// Staging: the two waves of thread group tid / 128 take page tid / 128 of the
// tile.  Thread tid holds bytes [i*2048 + (tid % 128)*16, +16) of that page's
// V (i < SPT); each wave copies half of the page's K into LDS directly.
template <int D>
struct TileRegs {
  u32x4 v[Geo<D>::SPT];
  bool valid;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Table entry of this thread's page (tid / 128) of a tile, read at a clamped
// index (always in bounds; whether the page exists is decided by load_tile).
// Read one step before the page loads that need it, and never under a
// branch, so the page loads never wait on the table.
__device__ __forceinline__ int tile_entry(const PrefillParams& p, int tile, int tid) {
  return p.table[min(tile * 4 + (tid >> 7), p.maxb - 1)];
}

// Whether a page's scores may enter the softmax: its block id is in the pool,
// or none of its tokens lies in [kv_begin, kv_end) (then the position mask
// hides them anyway).  A page inside the range whose id is outside the pool
// has its scores masked like positions outside the range, so its keys are
// skipped as decode skips them.
__device__ __forceinline__ bool page_usable(const PrefillParams& p, int lblk, bool valid) {
  return valid || lblk * kBlock >= p.kv_end || (lblk + 1) * kBlock <= p.kv_begin;
}

// Page loads of a tile.  A page past kv_end or the table, or whose entry is
// outside the pool, is marked invalid (its V is stored as zeros; its K is
// block 0's, and its scores are masked: by position past kv_end, by the
// tile's page flags otherwise); its loads still run, from block 0, so that
// no load sits under a branch.  The page, its validity and its address are
// wave-uniform (scalar).
//
// K is moved by global_load_lds_dwordx4: each lane's 16 bytes land at
// M0 + 16 * lane, so one instruction fills 1 KiB of LDS.  It is issued from
// inline assembly, which keeps M0 as it was, because the compiler treats an
// LDS-DMA load it knows about as pending on the LDS counter and then waits
// for every outstanding LDS read at once; opaque to it, the loads are awaited
// with an explicit vmcnt(0) before the barrier that publishes the tile.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, uint8_t* kdst, const PrefillParams& p,
                                          int tile, int entry, int tid, int kvh) {
  const int t128 = tid & 127, lane = tid & 63;
  const int pg = __builtin_amdgcn_readfirstlane(tid >> 7);
  const int half = __builtin_amdgcn_readfirstlane((tid >> 6) & 1);
  const int lblk = tile * 4 + pg;
  entry = __builtin_amdgcn_readfirstlane(entry);        // one page per wave
  r.valid = lblk < p.maxb && lblk * kBlock < p.kv_end && (unsigned)entry < (unsigned)p.num_blocks;
  const int blk = r.valid ? entry : 0;
  const uint8_t* kp = p.k + (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * kBlock * D * 2;
  const uint8_t* vp = p.v + (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * D * kBlock * 2;
  // K: this wave copies half of its page, 1 KiB per load, straight into LDS
#pragma unroll
  for (int i = 0; i < Geo<D>::PAGE / 2048; ++i) {
    const int o = half * (Geo<D>::PAGE / 2) + i * 1024;
    const uint8_t* src = kp + o + lane * 16;
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)(kdst + pg * Geo<D>::PAGE + o));
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0"
        : "=&s"(saved)
        : "v"(src), "s"(la)
        : "memory");
  }
#pragma unroll
  for (int i = 0; i < Geo<D>::SPT; ++i)
    r.v[i] = *reinterpret_cast<const u32x4*>(vp + i * 2048 + t128 * 16);
}

// put_piece writes V piece i of this thread: words 0-1 are dimension 32c + li
// and words 2-3 dimension 32c + 16 + li, tokens 4g .. 4g+3, which go to half
// g & 1 at byte 8 * (g >> 1).  V is converted bf16 -> fp16 (exact within
// fp16's normal range; beyond 65504 the round-toward-zero conversion
// saturates instead of overflowing).
template <int D>
__device__ __forceinline__ void put_piece(uint8_t* vs, u32x4 vv, int i, int pg, int t128) {
  const int o = i * 2048 + t128 * 16;
  const int c = o >> 10, l = (o >> 4) & 63, g = l >> 4, li = l & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    vv[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                                             __uint_as_float(vv[e] << 16),
                                             __uint_as_float(vv[e] & 0xffff0000u)));
  const int d0 = 32 * c + li;
  const u32x2 a = {vv[0], vv[1]}, b = {vv[2], vv[3]};
  *reinterpret_cast<u32x2*>(vs + v_lds_off<D>(pg, d0, g & 1) + 8 * (g >> 1)) = a;
  *reinterpret_cast<u32x2*>(vs + v_lds_off<D>(pg, d0 + 16, g & 1) + 8 * (g >> 1)) = b;
}

// V of tokens outside [kv_begin, kv_end) and of pages without a valid block
// is stored as zeros, so masked positions contribute exactly nothing to P V
// (their K, whatever it holds, only ever meets the mask).
template <int D>
__device__ __forceinline__ void store_tile(uint8_t* buf, uint8_t* meta, const TileRegs<D>& r,
                                           const PrefillParams& p, int tile, int tid,
                                           bool flags) {
  uint8_t* vs = buf + Geo<D>::KTILE;
  const int pg = tid >> 7, t128 = tid & 127;
  const int tok_base = tile * BN + pg * kBlock;   // first token of this page
  if (flags && t128 == 0) meta[16 + pg] = page_usable(p, tile * 4 + pg, r.valid) ? 1 : 0;
  const bool boundary = tile * BN < p.kv_begin || tile * BN + BN > p.kv_end;
  if (r.valid && !boundary) {                      // uniform over the wave
#pragma unroll
    for (int i = 0; i < Geo<D>::SPT; ++i) put_piece<D>(vs, r.v[i], i, pg, t128);
    return;
  }
#pragma unroll
  for (int i = 0; i < Geo<D>::SPT; ++i) {
    const int o = i * 2048 + t128 * 16;
    const int l = (o >> 4) & 63, g = l >> 4;
    u32x4 vv = r.valid ? r.v[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tv = tok_base + 4 * g + 2 * (e & 1);
      uint32_t keep = 0u;
      if (tv >= p.kv_begin && tv < p.kv_end) keep |= 0x0000ffffu;
      if (tv + 1 >= p.kv_begin && tv + 1 < p.kv_end) keep |= 0xffff0000u;
      vv[e] &= keep;
    }
    put_piece<D>(vs, vv, i, pg, t128);
  }
}

// ---- E4M3 pools [P2 3.2]: pages of 1-byte codes with one fp32 scale per
// (block, kv head) for K and for V.  K codes are staged as fp16 codes (exact:
// every E4M3 value is an fp16 value) and each page's K scale is applied to
// its scores in fp32, so scores are as exact as for bf16 pools; the tile's
// four K scales ride in a 16-byte LDS slot beside the ring.  V is staged
// dequantised, f16(code * scale) (one rounding of the exact product), since
// the scale cannot be folded into P V without also scaling the row sum.  Both
// products then run on fp16 MFMA (q converted bf16 -> fp16 once).  fp16 must
// hold |code * v_scale|, i.e. a V scale group's largest magnitude (<= 65504).
// Thread tid stages words [W8 * (tid % 128), +W8) of K and of V of page
// tid / 128.
template <int D>
struct TileRegs8 {
  uint32_t k[Geo<D>::W8], v[Geo<D>::W8];
  float ks, vs;
  bool valid;
};

template <int D, bool F8> struct RegsOf { using T = TileRegs<D>; };
template <int D> struct RegsOf<D, true> { using T = TileRegs8<D>; };

// Two E4M3 codes (bytes 2*HI, 2*HI+1 of w) -> f16 pair of code * s.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_scaled_f16(uint32_t w, float s) {
  f32x2v a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);   // exact
  a.x *= s;
  a.y *= s;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(a, f16x2));   // round to nearest even
}

// Two E4M3 codes -> their exact fp16 values.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

template <int D>
__device__ __forceinline__ void load_tile(TileRegs8<D>& r, uint8_t*, const PrefillParams& p,
                                          int tile, int entry, int tid, int kvh) {
  const int t128 = tid & 127;
  const int pg = __builtin_amdgcn_readfirstlane(tid >> 7);
  const int lblk = tile * 4 + pg;
  entry = __builtin_amdgcn_readfirstlane(entry);        // one page per wave
  r.valid = lblk < p.maxb && lblk * kBlock < p.kv_end && (unsigned)entry < (unsigned)p.num_blocks;
  const int blk = r.valid ? entry : 0;
  const int64_t pb = (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * Geo<D>::PAGE8;
  const uint8_t* kp = p.k + pb + t128 * (4 * Geo<D>::W8);
  const uint8_t* vp = p.v + pb + t128 * (4 * Geo<D>::W8);
  if constexpr (Geo<D>::W8 == 4) {
    const u32x4 kk = *reinterpret_cast<const u32x4*>(kp);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(vp);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.k[j] = kk[j];
      r.v[j] = vv[j];
    }
  } else {
    const u32x2 kk = *reinterpret_cast<const u32x2*>(kp);
    const u32x2 vv = *reinterpret_cast<const u32x2*>(vp);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      r.k[j] = kk[j];
      r.v[j] = vv[j];
    }
  }
  r.ks = p.k_scale[(int64_t)blk * p.hkv + kvh];
  r.vs = p.v_scale[(int64_t)blk * p.hkv + kvh];
}

// K: the 8 codes of a word pair are dimensions 32c + 8g .. +8 of token t
// (E4M3 fragment order), which become the 16-byte fp16 piece the score
// product reads (k_lds_off); one lane per page records the page's K scale
// (1 for a page that does not exist, whose scores are all masked).  V: a
// word is 4 consecutive tokens of one dimension, 8 bytes of fp16 in the V
// tile's half layout.  V of tokens outside [kv_begin, kv_end) or of an
// invalid page is stored as zeros (selected, not multiplied, so NaN codes or
// scales there do not leak).
template <int D>
__device__ __forceinline__ void store_tile(uint8_t* buf, uint8_t* meta, const TileRegs8<D>& r,
                                           const PrefillParams& p, int tile, int tid,
                                           bool flags) {
  float* ks_slot = reinterpret_cast<float*>(meta);
  constexpr int W8 = Geo<D>::W8;
  uint8_t* vs = buf + Geo<D>::KTILE;
  const int pg = tid >> 7, t128 = tid & 127;
#pragma unroll
  for (int q = 0; q < W8 / 2; ++q) {
    const int o = (t128 * W8 + 2 * q) * 4;
    const int row = (o >> 4) & 63, g = row >> 4, t = row & 15;
    const int c = 2 * (o >> 10) + ((o >> 3) & 1);
    const u32x4 h = {e4m3x2_f16<false>(r.k[2 * q]), e4m3x2_f16<true>(r.k[2 * q]),
                     e4m3x2_f16<false>(r.k[2 * q + 1]), e4m3x2_f16<true>(r.k[2 * q + 1])};
    *reinterpret_cast<u32x4*>(buf + pg * Geo<D>::PAGE + c * 1024 + ((g << 4) + t) * 16) = h;
  }
  if (t128 == 0) {
    ks_slot[pg] = r.valid ? r.ks : 1.0f;
    if (flags) meta[16 + pg] = page_usable(p, tile * 4 + pg, r.valid) ? 1 : 0;
  }
  const int tok_base = tile * BN + pg * kBlock;   // first token of this page
  const bool plain = r.valid && !(tile * BN < p.kv_begin || tile * BN + BN > p.kv_end);
#pragma unroll
  for (int j = 0; j < W8; ++j) {
    const int o = (t128 * W8 + j) * 4;
    const int row = (o >> 4) & 63, tg = row >> 4;
    const int d = 16 * (4 * (o >> 10) + ((o >> 2) & 3)) + (row & 15);
    u32x2 h = {e4m3x2_scaled_f16<false>(r.v[j], r.vs), e4m3x2_scaled_f16<true>(r.v[j], r.vs)};
    if (!plain) {                                  // uniform over the wave
      const int tv = tok_base + 4 * tg;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t keep = 0u;
        if (r.valid && tv + 2 * e >= p.kv_begin && tv + 2 * e < p.kv_end) keep |= 0x0000ffffu;
        if (r.valid && tv + 2 * e + 1 >= p.kv_begin && tv + 2 * e + 1 < p.kv_end)
          keep |= 0xffff0000u;
        h[e] &= keep;
      }
    }
    *reinterpret_cast<u32x2*>(vs + v_lds_off<D>(pg, d, tg & 1) + 8 * (tg >> 1)) = h;
  }
}

// Stores a staged tile into ring slot `slot`, and (when `flags`: some page
// of the workgroup's range is unusable) its page flags, and for E4M3 pools
// its K scales, into the slot's entry after the ring.
template <int D, typename Regs>
__device__ __forceinline__ void stage_store(uint8_t* smem, int slot, const Regs& r,
                                            const PrefillParams& p, int tile, int tid,
                                            bool flags) {
  store_tile(smem + slot * Geo<D>::BUF, smem + Geo<D>::LDS + Geo<D>::META * slot, r, p, tile,
             tid, flags);
}

// The four page flags of the tile in ring slot `slot` (byte i = page i),
// uniform over the workgroup once the barrier publishing the tile is passed.
template <int D>
__device__ __forceinline__ uint32_t page_flags(const uint8_t* smem, int slot) {
  return __builtin_amdgcn_readfirstlane(
      *reinterpret_cast<const uint32_t*>(smem + Geo<D>::LDS + Geo<D>::META * slot + 16));
}

// Score product S^T = K Q^T: bf16 operands for bf16 pools, fp16 for E4M3
// pools (dequantised tile, converted q).
template <bool F8>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (F8)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int D>
struct RowState {
  f32x16 o[Geo<D>::DT];   // O^T[32*dt + 8*(r/4) + 4*(lane/32) + r%4][row]
  float m, l;      // running max (log2 units, lazy) and this lane's share of the sum
  float mtrue;     // this lane's exact max of the scaled scores
};

// S^T for one tile: s[mt][r] = score of key 32*mt + 8*(r/4) + 4*hi + r%4.
template <int D, bool F8>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const uint8_t* ks,
                                        const u32x4 (&qf)[Geo<D>::QC], int qr, int hi) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
#pragma unroll
  for (int c = 0; c < Geo<D>::QC; ++c)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(ks + k_lds_off<D>(32 * mt + qr, 2 * c + hi));
      s[mt] = mfma_qk<F8>(kf, qf[c], s[mt]);
    }
}

// Tiles crossing kv_begin / kv_end or this wave's causal diagonal need the
// per-score visibility test (uniform over the wave).
__device__ __forceinline__ bool tile_needs_mask(const PrefillParams& p, int tb, int w_minpos) {
  return tb < p.kv_begin || tb + BN > p.kv_end || (p.causal && tb + BN - 1 > w_minpos);
}

// Scores of keys this lane's row may not see become the value that scales
// to -inf.
template <bool NEG_SCALE>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], const PrefillParams& p, int tb,
                                          int my_pos, int hi) {
  const float hidden = NEG_SCALE ? INFINITY : -INFINITY;
  const int lo = p.kv_begin - tb - 4 * hi;
  const int hi_ = (p.causal ? min(p.kv_end, my_pos + 1) : p.kv_end) - tb - 4 * hi;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ti = 32 * mt + 8 * (r >> 2) + (r & 3);
      s[mt][r] = (ti >= lo && ti < hi_) ? s[mt][r] : hidden;
    }
}

// Scores of pages flagged unusable (an id outside the pool inside the key
// range) become the value that scales to -inf.  Page i holds s[i / 2][8 * (i
// % 2) .. +8] in every lane.
template <bool NEG_SCALE>
__device__ __forceinline__ void mask_pages(f32x16 (&s)[2], uint32_t flags) {
  const float hidden = NEG_SCALE ? INFINITY : -INFINITY;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg)
    if (((flags >> (8 * pg)) & 0xffu) == 0u)
#pragma unroll
      for (int r = 0; r < 8; ++r) s[pg >> 1][8 * (pg & 1) + r] = hidden;
}
constexpr uint32_t kAllPagesUsable = 0x01010101u;

// Running max for a tile's scores, in log2 units with the scale c folded in
// (the largest scaled score is c * max(s) for c > 0 and c * min(s) for c < 0).
// The max is raised only when a score exceeds it by more than kLazy, which
// keeps every weight below 2^kLazy; then the row's lane pair agrees on the new
// max and O, l are rescaled.  Returns the max to subtract.
template <int D, bool NEG_SCALE>
__device__ __forceinline__ float update_max(RowState<D>& st, const f32x16 (&s)[2], float c) {
  const float hidden = NEG_SCALE ? INFINITY : -INFINITY;
  float ext = hidden;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ext = NEG_SCALE ? fminf(ext, s[mt][r]) : fmaxf(ext, s[mt][r]);
  const float lmx = ext == hidden ? -INFINITY : ext * c;
  st.mtrue = fmaxf(st.mtrue, lmx);
  if (__ballot(lmx > st.m + kLazy) != 0ull) {
    const float pe = __shfl_xor(ext, 32);
    const float e2 = NEG_SCALE ? fminf(ext, pe) : fmaxf(ext, pe);
    const float mx = e2 == hidden ? -INFINITY : e2 * c;
    const float m_new = fmaxf(st.m, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < Geo<D>::DT; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  return st.m == -INFINITY ? 0.f : st.m;
}

// The same for an E4M3 tile, whose page i carries its own K scale: cp[i] =
// c * k_scale (same sign as c, as scales are positive), so each page's
// extreme raw score is scaled by its own multiplier.
template <int D, bool NEG_SCALE>
__device__ __forceinline__ float update_max_paged(RowState<D>& st, const f32x16 (&s)[2],
                                                  const float (&cp)[4]) {
  const float hidden = NEG_SCALE ? INFINITY : -INFINITY;
  float lmx = -INFINITY;
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) {          // page pg holds s[pg / 2][8 * (pg % 2) .. +8]
    float ext = hidden;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float x = s[pg >> 1][8 * (pg & 1) + r];
      ext = NEG_SCALE ? fminf(ext, x) : fmaxf(ext, x);
    }
    lmx = fmaxf(lmx, ext == hidden ? -INFINITY : ext * cp[pg]);
  }
  st.mtrue = fmaxf(st.mtrue, lmx);
  if (__ballot(lmx > st.m + kLazy) != 0ull) {
    const float mx = fmaxf(lmx, __shfl_xor(lmx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < Geo<D>::DT; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  return st.m == -INFINITY ? 0.f : st.m;
}

// One pipelined step of a wave: the scores s_cur of tile j (already masked)
// become fp16 weights while the K Q^T products of tile j+1 (LDS buffer nxt)
// run into s_next, then O^T += V^T P^T for tile j.  The row sum is taken over
// the rounded weights that enter the product, so the result stays an exact
// weighted average of V rows.
template <int D, bool NEG_SCALE, bool F8>
__device__ __forceinline__ void attend_step(RowState<D>& st, const f32x16 (&s_cur)[2],
                                            f32x16 (&s_next)[2], const uint8_t* cur,
                                            const uint8_t* nxt, const u32x4 (&qf)[Geo<D>::QC],
                                            float c, const float* ks_cur, int qr, int hi) {
  constexpr int QC = Geo<D>::QC;
  constexpr int WPC = 32 / QC;          // weights made per k-step of the score product
  // score multiplier of k-step (= page) i: c, times the page's K scale for E4M3
  float cp[4];
  float m_use;
  if constexpr (F8) {
    const f32x4 kv = *reinterpret_cast<const f32x4*>(ks_cur);
#pragma unroll
    for (int i = 0; i < 4; ++i) cp[i] = c * kv[i];
    m_use = update_max_paged<D, NEG_SCALE>(st, s_cur, cp);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) cp[i] = c;
    m_use = update_max<D, NEG_SCALE>(st, s_cur, c);
  }
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  // raised wave priority while the step's matrix instructions are issued (the
  // arbiter then prefers this wave's products; measured +0.5-0.8 %)
  __builtin_amdgcn_s_setprio(1);
  // the scheduler's interleave of matrix products among the other
  // instructions of one wave (measured +1.5-1.7 % on the 32K and 128K
  // prompts, bf16 and E4M3; pattern 0 lost 5 %, the others 0-0.8 %)
  __builtin_amdgcn_iglp_opt(1);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s_next[mt][r] = 0.f;
  f16x8 pb[4];      // k-step ks = 2*mt + rr takes s_cur[mt][8*rr .. 8*rr+7]
  float rs = 0.f;
#pragma unroll
  for (int cc = 0; cc < QC; ++cc) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const u32x4 kf =
          *reinterpret_cast<const u32x4*>(nxt + k_lds_off<D>(32 * mt + qr, 2 * cc + hi));
      s_next[mt] = mfma_qk<F8>(kf, qf[cc], s_next[mt]);
    }
    const int kst = (cc * WPC) >> 3, e0 = (cc * WPC) & 7;
    // weights in pairs: each pair is rounded to fp16 once (round to nearest
    // even) and that packed value feeds both P V and the row sum
#pragma unroll
    for (int e = 0; e < WPC / 2; ++e) {
      const float x0 = __builtin_amdgcn_exp2f(
          __builtin_fmaf(s_cur[kst >> 1][8 * (kst & 1) + e0 + 2 * e], cp[kst], -m_use));
      const float x1 = __builtin_amdgcn_exp2f(
          __builtin_fmaf(s_cur[kst >> 1][8 * (kst & 1) + e0 + 2 * e + 1], cp[kst], -m_use));
      const f16x2 pr = __builtin_convertvector((f32x2v){x0, x1}, f16x2);
      pb[kst][e0 + 2 * e] = pr[0];
      pb[kst][e0 + 2 * e + 1] = pr[1];
      rs = __builtin_amdgcn_fdot2(pr, ones, rs, false);
    }
  }
  st.l += rs;
  const uint8_t* vs = cur + Geo<D>::KTILE;
#pragma unroll
  for (int kst = 0; kst < 4; ++kst)
#pragma unroll
    for (int dt = 0; dt < Geo<D>::DT; ++dt) {
      const u32x4 vf = *reinterpret_cast<const u32x4*>(vs + v_lds_off<D>(kst, 32 * dt + qr, hi));
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vf), pb[kst],
                                                       st.o[dt], 0, 0, 0);
    }
  __builtin_amdgcn_s_setprio(0);
}

template <int D, bool NEG_SCALE, bool F8>
__global__ __launch_bounds__(NTHREADS) void prefill_kernel(PrefillParams p) {
  using G = Geo<D>;
  using Regs = typename RegsOf<D, F8>::T;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;        // lane half
  const int qr = lane & 31;        // query row within the wave

  // workgroup -> (kv head, head group, row tile); heavier (later) rows first
  const int i = blockIdx.x;
  const int kvh = i % p.hkv;
  const int rest = i / p.hkv;
  const int hgrp = rest % p.HGR;
  const int rt = p.row_tiles - 1 - rest / p.HGR;
  const int h = kvh * p.G + hgrp * p.NH + w % p.NH;
  const int row0 = rt * ROWS_W * p.NR;
  const int wrow0 = row0 + (w / p.NH) * ROWS_W;
  const int my_row = wrow0 + qr;
  const bool row_ok = my_row < p.T;
  const int my_pos = p.q_pos0 + my_row;

  // query fragments (B operand): Q[row][16c + 8*hi .. +8]; for E4M3 pools
  // converted to fp16 (exact for bf16 values within fp16's range)
  u32x4 qf[G::QC];
  {
    const uint16_t* qp = p.q + ((int64_t)my_row * p.hq + h) * D;
#pragma unroll
    for (int c = 0; c < G::QC; ++c) {
      qf[c] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * c + 8 * hi)
                     : u32x4{0u, 0u, 0u, 0u};
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qf[c][e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                                                      __uint_as_float(qf[c][e] << 16),
                                                      __uint_as_float(qf[c][e] & 0xffff0000u)));
      }
    }
  }

  // keys this workgroup may see
  const int last_row = min(row0 + ROWS_W * p.NR, p.T) - 1;
  int key_end = p.kv_end;
  if (p.causal) key_end = min(key_end, p.q_pos0 + last_row + 1);
  const int t_lo = p.kv_begin / BN;
  const int t_hi = key_end > p.kv_begin ? (key_end - 1) / BN : t_lo - 1;
  const int w_minpos = p.q_pos0 + wrow0;

  // Does any page this workgroup reads have an id outside the pool inside the
  // key range?  Checked once over the table; only then do the steps read the
  // per-slot page flags (otherwise no step waits on that LDS read).
  bool any_bad = false;
  if (t_lo <= t_hi)
    for (int lb = t_lo * 4 + tid; lb < min((t_hi + 1) * 4, p.maxb); lb += NTHREADS)
      any_bad |= !page_usable(p, lb, (unsigned)p.table[lb] < (unsigned)p.num_blocks);
  any_bad = __syncthreads_or(any_bad);

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[dt][r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
  st.mtrue = -INFINITY;
  const float c = p.scale_log2;

  if (t_lo <= t_hi) {
    Regs regs;
    load_tile(regs, smem, p, t_lo, tile_entry(p, t_lo, tid), tid, kvh);
    stage_store<D>(smem, 0, regs, p, t_lo, tid, any_bad);
    if (t_lo + 1 <= t_hi) {
      load_tile(regs, smem + G::BUF, p, t_lo + 1, tile_entry(p, t_lo + 1, tid), tid, kvh);
      stage_store<D>(smem, 1, regs, p, t_lo + 1, tid, any_bad);
    }
    int entry_next = tile_entry(p, t_lo + 2, tid);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the direct-to-LDS K loads are in
    __syncthreads();

    f32x16 sa[2], sb[2];
    qk_tile<D, F8>(sa, smem, qf, qr, hi);
    if (tile_needs_mask(p, t_lo * BN, w_minpos)) mask_tile<NEG_SCALE>(sa, p, t_lo * BN, my_pos, hi);
    if (any_bad) {
      const uint32_t fl = page_flags<D>(smem, 0);
      if (fl != kAllPagesUsable) mask_pages<NEG_SCALE>(sa, fl);
    }

    // Tile j lives in ring slot (j - t_lo) % 3.  Step j starts the loads of
    // tile j+2 (K straight into the slot tile j-1 left, V into registers),
    // attends to tile j while computing the scores of tile j+1 (past the last
    // tile those products read a stale slot and are dropped), stores V of
    // tile j+2, and ends on the barrier that publishes it.
    int slot = 0;
    auto step = [&](int j, const f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
      const int s1 = slot == 2 ? 0 : slot + 1;
      const int s2 = s1 == 2 ? 0 : s1 + 1;
      const bool prefetch = j + 2 <= t_hi;
      Regs nregs;
      if (prefetch) load_tile(nregs, smem + s2 * G::BUF, p, j + 2, entry_next, tid, kvh);
      entry_next = tile_entry(p, j + 3, tid);
      attend_step<D, NEG_SCALE, F8>(st, s_cur, s_next, smem + slot * G::BUF, smem + s1 * G::BUF,
                                    qf, c, reinterpret_cast<const float*>(smem + G::LDS + G::META * slot),
                                    qr, hi);
      if (prefetch) stage_store<D>(smem, s2, nregs, p, j + 2, tid, any_bad);
      if (j + 1 <= t_hi) {
        if (tile_needs_mask(p, (j + 1) * BN, w_minpos))
          mask_tile<NEG_SCALE>(s_next, p, (j + 1) * BN, my_pos, hi);
        if (any_bad) {                     // tile j+1's flags, published last step
          const uint32_t fl = page_flags<D>(smem, s1);
          if (fl != kAllPagesUsable) mask_pages<NEG_SCALE>(s_next, fl);
        }
      }
      slot = s1;
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the direct-to-LDS K loads are in
      __syncthreads();
    };
    for (int j = t_lo; j <= t_hi; j += 2) {
      step(j, sa, sb);
      if (j + 1 <= t_hi) step(j + 1, sb, sa);
    }
  }

  // ---- epilogue: row sum over the lane pair, then normalise or emit partials
  float l = st.l + __shfl_xor(st.l, 32);
  const float mtrue = fmaxf(st.mtrue, __shfl_xor(st.mtrue, 32));
  float m = st.m;
  if (!row_ok) return;
  const bool empty = !(l > 0.f);
  const int64_t ro = (int64_t)my_row * p.hq + h;
  if (p.out) {
    const float inv = empty ? 0.f : 1.0f / l;
    uint16_t* op = p.out + ro * D;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hi;
        u32x2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(st.o[dt][4 * j] * inv) |
               ((uint32_t)f32_to_bf16_bits(st.o[dt][4 * j + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(st.o[dt][4 * j + 2] * inv) |
               ((uint32_t)f32_to_bf16_bits(st.o[dt][4 * j + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
    if (p.out_lse && hi == 0) p.out_lse[ro] = empty ? -INFINITY : m * kLn2 + logf(l);
  } else {
    // partials are exported relative to the exact row max (m <= mtrue <= m + kLazy)
    const float f = empty ? 0.f : __builtin_amdgcn_exp2f(m - mtrue);
    l *= f;
    m = mtrue;
    float* op = p.part_o + ro * D;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hi;
        const f32x4 val = empty ? f32x4{0.f, 0.f, 0.f, 0.f}
                                : f32x4{st.o[dt][4 * j] * f, st.o[dt][4 * j + 1] * f,
                                        st.o[dt][4 * j + 2] * f, st.o[dt][4 * j + 3] * f};
        *reinterpret_cast<f32x4*>(op + d) = val;
      }
    if (hi == 0) {
      p.part_m[ro] = empty ? -INFINITY : m * kLn2;
      p.part_l[ro] = empty ? 0.f : l;
    }
  }
}

int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }

// More than 64 KiB of dynamic LDS needs an explicit opt-in per kernel (once
// per process and device is enough; repeating it is harmless).
template <int D, bool NEG, bool F8>
hipError_t launch_one(const PrefillParams& p, unsigned wgs, hipStream_t s) {
  constexpr int lds = Geo<D>::LDS_ALL;      // the ring + each slot's flags and K scales
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, NEG, F8>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((prefill_kernel<D, NEG, F8>), dim3(wgs), dim3(NTHREADS), lds, s, p);
  return hipGetLastError();
}

template <int D, bool F8>
hipError_t launch_sign(const PrefillParams& p, unsigned wgs, float scale, hipStream_t s) {
  return scale < 0.f ? launch_one<D, true, F8>(p, wgs, s) : launch_one<D, false, F8>(p, wgs, s);
}

}  // namespace

hipError_t launch_prefill(const CacheView& c, const void* q, int T, int hq, int q_pos0,
                          const int32_t* table, int maxb, int kv_begin, int kv_end, int causal,
                          float scale, void* out, float* out_lse, float* part_o, float* part_m,
                          float* part_l, hipStream_t s) {
  if (T == 0) return hipSuccess;
  PrefillParams p{};
  p.k = static_cast<const uint8_t*>(c.k);
  p.v = static_cast<const uint8_t*>(c.v);
  const bool f8 = c.kv_dtype == PKV_FP8_E4M3;
  p.k_scale = c.k_scale;
  p.v_scale = c.v_scale;
  p.block_stride_bytes = c.block_stride * (f8 ? 1 : 2);
  p.num_blocks = c.num_blocks;
  p.hkv = c.hkv;
  p.hq = hq;
  p.G = hq / c.hkv;
  p.NH = gcd(p.G, NWAVE);
  p.NR = NWAVE / p.NH;
  p.HGR = p.G / p.NH;
  p.q = static_cast<const uint16_t*>(q);
  p.T = T;
  p.q_pos0 = q_pos0;
  p.table = table;
  p.maxb = maxb;
  p.kv_begin = kv_begin;
  p.kv_end = kv_end;
  p.causal = causal;
  p.scale_log2 = scale * kLog2e;
  p.row_tiles = (T + ROWS_W * p.NR - 1) / (ROWS_W * p.NR);
  p.out = static_cast<uint16_t*>(out);
  p.out_lse = out_lse;
  p.part_o = part_o;
  p.part_m = part_m;
  p.part_l = part_l;
  const int64_t wgs = (int64_t)p.row_tiles * c.hkv * p.HGR;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  if (c.head_dim == 128)
    return f8 ? launch_sign<128, true>(p, (unsigned)wgs, scale, s)
              : launch_sign<128, false>(p, (unsigned)wgs, scale, s);
  if (c.head_dim == 64)
    return f8 ? launch_sign<64, true>(p, (unsigned)wgs, scale, s)
              : launch_sign<64, false>(p, (unsigned)wgs, scale, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv

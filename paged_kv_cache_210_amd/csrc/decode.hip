// Split-KV paged decode: one query per sequence against every cached key.
//
// What is computed ([P3] www.mhpn.cn/news/2466452 section 1.1; [P2] "Unlocking
// long context ..." section 4.1): O = softmax(scale * q K^T) V over the
// sequence's keys, read page by page through the block table ([P1]
// "Long-context inference engineering truths 2026 ..." section 2.2; [P2]
// section 3.1), with kv head h / G serving G query heads ([P3] section 3.2).
// Each partition of the sequence's blocks keeps the online-softmax state
// (running max m, running sum l, rescaled accumulator O) of [P1] section 3.1;
// partitions are combined exactly by the max / log-sum-exp correction of [P4]
// "Sequence-parallel engineering ..." section "numerically stable incremental
// softmax" (merge.hip).
//
// Decode reads every K/V byte once and does about 4*G flops per byte: it is
// HBM-bound ([P2] section 5.1).  The MFMA path keeps the arithmetic off the
// vector ALUs so that the waves spend their issue slots on loads:
//   S^T[t][g] = K[t][:] . Q[g][:]     v_mfma_f32_16x16x32 (bf16, or f16 for E4M3)
//   O^T[d][g] += V^T[d][t] P^T[t][g]  v_mfma_f32_16x16x16
// One wave owns one page (16 tokens) per step.  Lane l holds token 4*(l/16)+i
// (i < 4) of the page for query head l%16: that is both the output layout of
// the score product and the B-operand layout of the PV product, so softmax
// weights never leave their lane.  bf16 and E4M3 pages are stored in fragment
// order (each lane's operands for a whole page are contiguous 16-byte pieces,
// and one load instruction reads 1 KiB of contiguous memory).
#include <type_traits>

#include "pkv_common.h"

namespace pkv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Waves per workgroup (= one partition).  Two, at 3 waves per SIMD: six
// workgroups fit a CU, so a 1024-workgroup decode (4 x 131072 tokens in
// 256-block partitions) is resident in one round instead of 1.33 rounds of
// 768 four-wave workgroups (measured +1.6 % there, +1.0-1.3 % at 8K and 1M).
constexpr int kNW = 2;
#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1
#endif
constexpr int kThreads = 64 * kNW;

struct DecodeParams {
  const uint8_t* k;
  const uint8_t* v;
  int64_t block_stride_bytes;
  const float* k_scale;
  const float* v_scale;
  int num_blocks, hkv, hq, G, HG;
  const void* q;
  int q_dtype;
  const int32_t* tables;
  int maxb;
  const int32_t* seq_lens;
  float scale_log2;          // softmax scale * log2(e)
  int P, PB;
  int64_t rows;              // B * hq
  float* part_o;             // [P][B*hq][D], unnormalised, relative to part_m
  float* part_m;             // [P][B*hq], natural-log units
  float* part_l;             // [P][B*hq]
  // Folded append (bf16 pools): token seq_lens[b]-1 of sequence b takes
  // k_new/v_new[b][kv head][:] (bf16); null when the step appends nothing.
  const uint16_t* k_new;
  const uint16_t* v_new;
};

__device__ __forceinline__ int seq_len_clamped(const DecodeParams& p, int b) {
  int n = p.seq_lens[b];
  n = n < 0 ? 0 : n;
  return min(n, p.maxb * kBlock);
}

template <int D>
struct SoftState {
  float m;            // running max, log2 units (shared by the 4 lanes of a head)
  float l;            // this lane's share of the running sum
  f32x4 o[D / 16];    // O^T[16n + 4*(l/16) + i][head l%16]
};

// Online-softmax step over this lane's 4 scores x (log2 units, -inf = masked).
// The running max m is shared by the 4 lanes of a head and is only raised when
// some score exceeds it by more than kLazy: weights then stay below 2^kLazy
// (well inside fp16 / bf16 / fp32 range) and the result is the same, while the
// cross-lane max and the rescale of O run only on the pages that raise m.
constexpr float kLazy = 8.0f;

template <int D>
__device__ __forceinline__ void online_update(SoftState<D>& st, const float (&x)[4],
                                              float (&pw)[4]) {
  const float local = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__ballot(local > st.m + kLazy) != 0ull) {
    float mx = fmaxf(local, __shfl_xor(local, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) st.o[n] *= alpha;
    st.m = m_new;
  }
  const float m_use = st.m == -INFINITY ? 0.f : st.m;
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
  st.l += (pw[0] + pw[1]) + (pw[2] + pw[3]);
}

// Number of this lane's 4 tokens (starting at tok) that are below n, as a mask
// of 16-bit (bf16) or 8-bit (E4M3) lanes.
__device__ __forceinline__ int valid_count(int tok, int n) {
  const int c = n - tok;
  return c < 0 ? 0 : (c > 4 ? 4 : c);
}

// ---- bf16 pages ---------------------------------------------------------------
// Pages are in fragment order (pkv_common.h: frag_k_off / frag_v_off), so each
// of a lane's loads is the 16-byte piece at j*1024 + 16*l.
template <int D>
struct BF16Page {
  u32x4 k[D / 32];     // piece c: K[t = l%16][32c + 8*(l/16) .. +8]
  u32x4 v[D / 32];     // piece j: V^T[16n + l%16][4*(l/16) .. +4] for n = 2j, 2j+1
  __device__ __forceinline__ u32x2 vfrag(int n) const {
    const u32x4& q = v[n >> 1];
    return (n & 1) ? u32x2{q.z, q.w} : u32x2{q.x, q.y};
  }
};

// K/V pages are read once per step: streaming loads (non-temporal when
// PKV_DECODE_NT is set).
template <typename T>
__device__ __forceinline__ T stream_load(const uint8_t* p) {
#if PKV_DECODE_NT
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
#else
  return *reinterpret_cast<const T*>(p);
#endif
}

template <int D>
__device__ __forceinline__ void load_page(BF16Page<D>& pg, const uint8_t* kp, const uint8_t* vp,
                                          int col, int grp) {
  const int lane = grp * 16 + col;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) pg.k[c] = stream_load<u32x4>(kp + c * 1024 + lane * 16);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) pg.v[j] = stream_load<u32x4>(vp + j * 1024 + lane * 16);
}

template <int D>
__device__ __forceinline__ void compute_page(SoftState<D>& st, const BF16Page<D>& pg,
                                             const u32x4 (&qf)[D / 32], int tok, int n,
                                             float sl2) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pg.k[c]),
                                               __builtin_bit_cast(bf16x8, qf[c]), s, 0, 0, 0);
  const int vc = valid_count(tok, n);
  float x[4], pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = i < vc ? s[i] * sl2 : -INFINITY;
  online_update<D>(st, x, pw);
  // The weights enter the PV product as a bf16 pair hi + lo (lo = bf16 of the
  // remainder), so they keep about 16 significant bits: decode has MFMA time
  // to spare, and one bf16 rounding of a weight alone would cost up to 2^-9
  // relative on rows with few keys.
  s16x4 pb_hi, pb_lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t h = f32_to_bf16_bits(pw[i]);
    pb_hi[i] = (short)h;
    pb_lo[i] = (short)f32_to_bf16_bits(pw[i] - bf16_bits_to_f32(h));
  }
  // masked tokens: select the V values away (stale slots may hold anything)
  u32x2 keep = {vc >= 2 ? 0xffffffffu : (vc == 1 ? 0x0000ffffu : 0u),
                vc >= 4 ? 0xffffffffu : (vc == 3 ? 0x0000ffffu : 0u)};
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn) {
    const u32x2 vv = pg.vfrag(nn) & keep;
    st.o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pb_hi,
                                                        st.o[nn], 0, 0, 0);
  }
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn) {
    const u32x2 vv = pg.vfrag(nn) & keep;
    st.o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vv), pb_lo,
                                                        st.o[nn], 0, 0, 0);
  }
}

// Folded append: the newest token (slot `slot` of this page) is taken from
// k_new / v_new instead of the pool, and written into the pool by the same
// lanes.  Lane l holds K of token l%16 (dims 32c + 8*(l/16) .. +8) and V of
// tokens 4*(l/16) .. +4 (dim 16n + l%16), so the token's K sits in the 4 lanes
// with l%16 == slot and its V in the 16 lanes with l/16 == slot/4.  Nothing
// else reads this page in the launch, so the stores race with no load that
// matters (the page's own load of the slot is replaced here).
template <int D>
__device__ __forceinline__ void fold_new_token(BF16Page<D>& pg, const DecodeParams& p, int b,
                                               int kvh, int blk, int slot, int col, int grp) {
  const int lane = grp * 16 + col;
  const int64_t base = (int64_t)blk * p.block_stride_bytes;
  uint8_t* kp = const_cast<uint8_t*>(p.k) + base + (int64_t)kvh * kBlock * D * 2;
  uint8_t* vp = const_cast<uint8_t*>(p.v) + base + (int64_t)kvh * D * kBlock * 2;
  const uint16_t* kn = p.k_new + ((int64_t)b * p.hkv + kvh) * D;
  const uint16_t* vn = p.v_new + ((int64_t)b * p.hkv + kvh) * D;
  // every read of the token before any store: the stores could alias the
  // inputs as far as the compiler knows, and would otherwise serialise them
  const bool has_k = col == slot, has_v = grp == (slot >> 2);
  u32x4 kx[D / 32];
  uint16_t vx[D / 16];
  if (has_k) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) kx[c] = *reinterpret_cast<const u32x4*>(kn + 32 * c + 8 * grp);
  }
  if (has_v) {
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn) vx[nn] = vn[16 * nn + col];
  }
  if (has_k) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      pg.k[c] = kx[c];
      *reinterpret_cast<u32x4*>(kp + c * 1024 + lane * 16) = kx[c];
    }
  }
  if (has_v) {
    const int wi = (slot & 3) >> 1, sh = 16 * (slot & 1);
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn) {
      const int wd = 2 * (nn & 1) + wi;
      pg.v[nn >> 1][wd] = (pg.v[nn >> 1][wd] & ~(0xffffu << sh)) | ((uint32_t)vx[nn] << sh);
      *reinterpret_cast<uint16_t*>(vp + (nn >> 1) * 1024 + lane * 16 + (nn & 1) * 8 +
                                   (slot & 3) * 2) = vx[nn];
    }
  }
}

// ---- E4M3 pages ---------------------------------------------------------------
// Fragment order as for bf16: K piece i holds the score product's fragments
// c = 2i, 2i+1 (8 codes each: K[t = l%16][32c + 8*(l/16) .. +8]); V piece j
// holds the PV fragments nn = 4j .. 4j+3 (4 codes each: V^T[16nn + l%16]
// [4*(l/16) .. +4]).
template <int D>
struct FP8Page {
  u32x4 k[D / 64];
  u32x4 v[D / 64];
  float ks, vs;        // scales of this (block, head)
  __device__ __forceinline__ u32x2 kfrag(int c) const {
    const u32x4& q = k[c >> 1];
    return (c & 1) ? u32x2{q.z, q.w} : u32x2{q.x, q.y};
  }
  __device__ __forceinline__ uint32_t vfrag(int nn) const { return v[nn >> 2][nn & 3]; }
};

template <int D>
__device__ __forceinline__ void load_page(FP8Page<D>& pg, const uint8_t* kp, const uint8_t* vp,
                                          int col, int grp) {
  const int lane = grp * 16 + col;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) pg.k[i] = stream_load<u32x4>(kp + i * 1024 + lane * 16);
#pragma unroll
  for (int i = 0; i < D / 64; ++i) pg.v[i] = stream_load<u32x4>(vp + i * 1024 + lane * 16);
}

// E4M3 -> fp16 with the gfx950 scaled convert at scale 1: every finite E4M3
// value (max 448, subnormals included) is exact in fp16.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <bool HI>
__device__ __forceinline__ uint32_t cvt2(uint32_t codes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(codes, 1.0f, HI));
}
__device__ __forceinline__ f16x8 codes8_to_f16(u32x2 c) {
  u32x4 h = {cvt2<false>(c.x), cvt2<true>(c.x), cvt2<false>(c.y), cvt2<true>(c.y)};
  return __builtin_bit_cast(f16x8, h);
}
__device__ __forceinline__ f16x4 codes4_to_f16(uint32_t c) {
  u32x2 h = {cvt2<false>(c), cvt2<true>(c)};
  return __builtin_bit_cast(f16x4, h);
}

// E4M3 values enter the MFMA as exact fp16; the per-block scales are applied
// in fp32 to the scores and to each page's PV product.
template <int D>
__device__ __forceinline__ void compute_page(SoftState<D>& st, const FP8Page<D>& pg,
                                             const u32x4 (&qf)[D / 32], int tok, int n,
                                             float sl2) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16(pg.kfrag(c)),
                                              __builtin_bit_cast(f16x8, qf[c]), s, 0, 0, 0);
  const int vc = valid_count(tok, n);
  const float kf = sl2 * pg.ks;
  float x[4], pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = i < vc ? s[i] * kf : -INFINITY;
  online_update<D>(st, x, pw);
  f16x4 pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = (_Float16)pw[i];
  const uint32_t keep = vc >= 4 ? 0xffffffffu : ((1u << (8 * vc)) - 1u);
  const float vf = pg.vs;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 t[D / 16];     // one product per tile, so the MFMAs issue back to back
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn)
    t[nn] = __builtin_amdgcn_mfma_f32_16x16x16f16(codes4_to_f16(pg.vfrag(nn) & keep), pb, zero, 0, 0,
                                                 0);
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn) st.o[nn] += t[nn] * vf;
}

// Folded append into an E4M3 page: the token is encoded exactly as
// pkv_kv_append encodes it, E4M3(f32(x) * f32(1 / scale)) with the page's
// scale (set beforehand, as for pkv_kv_append).  Lanes with l%16 == slot
// hold its K codes (piece i: dims 32c + 8*(l/16) .. +8 for c = 2i, 2i+1);
// lanes with l/16 == slot/4 hold its V codes (byte slot%4 of word n%4 of
// piece n/4, dim 16n + l%16).
template <int D>
__device__ __forceinline__ void fold_new_token(FP8Page<D>& pg, const DecodeParams& p, int b,
                                               int kvh, int blk, int slot, int col, int grp) {
  const int lane = grp * 16 + col;
  const int64_t base = (int64_t)blk * p.block_stride_bytes;
  uint8_t* kp = const_cast<uint8_t*>(p.k) + base + (int64_t)kvh * kBlock * D;
  uint8_t* vp = const_cast<uint8_t*>(p.v) + base + (int64_t)kvh * D * kBlock;
  const uint16_t* kn = p.k_new + ((int64_t)b * p.hkv + kvh) * D;
  const uint16_t* vn = p.v_new + ((int64_t)b * p.hkv + kvh) * D;
  // every read of the token before any store (see the bf16 fold)
  const bool has_k = col == slot, has_v = grp == (slot >> 2);
  u32x4 kx[D / 32];                         // bf16 K[32c + 8*grp .. +8], c < D/32
  uint16_t vx[D / 16];
  if (has_k) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) kx[c] = *reinterpret_cast<const u32x4*>(kn + 32 * c + 8 * grp);
  }
  if (has_v) {
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn) vx[nn] = vn[16 * nn + col];
  }
  if (has_k) {
    const float inv_k = __frcp_rn(pg.ks);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      u32x4 codes = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t w = kx[2 * i + (e >> 3)][(e & 7) >> 1];
        const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xffffu);
        codes[e >> 2] |= e4m3_encode(__fmul_rn(bf16_bits_to_f32(h), inv_k)) << (8 * (e & 3));
      }
      pg.k[i] = codes;
      *reinterpret_cast<u32x4*>(kp + i * 1024 + lane * 16) = codes;
    }
  }
  if (has_v) {
    const float inv_v = __frcp_rn(pg.vs);
    const int sh = 8 * (slot & 3);
#pragma unroll
    for (int nn = 0; nn < D / 16; ++nn) {
      const uint32_t c = e4m3_encode(__fmul_rn(bf16_bits_to_f32(vx[nn]), inv_v));
      pg.v[nn >> 2][nn & 3] = (pg.v[nn >> 2][nn & 3] & ~(0xffu << sh)) | (c << sh);
      vp[(nn >> 2) * 1024 + lane * 16 + (nn & 3) * 4 + (slot & 3)] = (uint8_t)c;
    }
  }
}

template <int D, int KVF>
using PageT = typename std::conditional<KVF == PKV_BF16, BF16Page<D>, FP8Page<D>>::type;

template <int D, int KVF>
__device__ __forceinline__ bool issue_page(PageT<D, KVF>& pg, const DecodeParams& p, int blk,
                                           int kvh, int col, int grp) {
  const bool ok = (unsigned)blk < (unsigned)p.num_blocks;
  const int64_t base = (int64_t)(ok ? blk : 0) * p.block_stride_bytes;
  constexpr int esz = KVF == PKV_BF16 ? 2 : 1;
  const uint8_t* kp = p.k + base + (int64_t)kvh * kBlock * D * esz;
  const uint8_t* vp = p.v + base + (int64_t)kvh * D * kBlock * esz;
  load_page<D>(pg, kp, vp, col, grp);
  if constexpr (KVF == PKV_FP8_E4M3) {
    // vector loads (the address is forced into a VGPR), so the scales are
    // ordered with the page loads instead of waiting on the scalar queue;
    // global (not generic) pointers, so they are counted like the page loads
    typedef const __attribute__((address_space(1))) float gfloat_t;
    gfloat_t* ks = (gfloat_t*)(p.k_scale + (int64_t)(ok ? blk : 0) * p.hkv + kvh);
    gfloat_t* vs = (gfloat_t*)(p.v_scale + (int64_t)(ok ? blk : 0) * p.hkv + kvh);
    asm volatile("" : "+v"(ks), "+v"(vs));
    pg.ks = *ks;
    pg.vs = *vs;
  }
  return ok;
}

// grid (P, hkv * HG, B): one workgroup per (partition, kv head, 16-head group,
// sequence); wave w takes a contiguous 1/kNW of the partition's pages.
template <int D, int KVF>
__global__ __launch_bounds__(kThreads, 3) void decode_mfma_kernel(DecodeParams p) {
  __shared__ float sm_o[kNW][16][D];
  __shared__ float sm_m[kNW][16];
  __shared__ float sm_l[kNW][16];

  const int part = blockIdx.x;
  const int kvh = blockIdx.y / p.HG;
  const int hg = blockIdx.y - kvh * p.HG;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int gi = hg * 16 + col;
  const bool head_ok = gi < p.G;
  const int n = seq_len_clamped(p, b);
  const int nblk = (n + kBlock - 1) / kBlock;
  const int j0 = part * p.PB;
  const int j1 = min(j0 + p.PB, nblk);

  // query fragment (B operand of the score product): Q[g = col][32c + 8*grp .. +8]
  u32x4 qf[D / 32];
  {
    const uint16_t* qp =
        reinterpret_cast<const uint16_t*>(p.q) + ((int64_t)b * p.hq + (int64_t)kvh * p.G + gi) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 raw = head_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * grp)
                          : u32x4{0u, 0u, 0u, 0u};
      if constexpr (KVF == PKV_FP8_E4M3) {
        // bf16 -> fp16 (exact for |q| in fp16's normal range)
        u32x4 h;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const _Float16 lo = (_Float16)bf16_bits_to_f32(raw[e] & 0xffffu);
          const _Float16 hi = (_Float16)bf16_bits_to_f32(raw[e] >> 16);
          h[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        raw = h;
      }
      qf[c] = raw;
    }
  }

  SoftState<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn) st.o[nn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's pages: a contiguous 1/kNW of the partition
  const int per_w = (j1 - j0 + kNW - 1) / kNW;
  const int pw0 = j0 + w * per_w;
  const int cnt = max(0, min(per_w, j1 - pw0));
  // table entries through the constant address space: wave-uniform scalar loads
  typedef const __attribute__((address_space(4))) int32_t ctab_t;
  ctab_t* trow = (ctab_t*)(p.tables + (int64_t)b * p.maxb);

  // Two pages in flight: the next page's loads are always issued (clamped to
  // the wave's last page) so the number of loads outstanding at each compute
  // is fixed and only the page being computed is waited for.
  // Two pages in flight per wave: page k+1's loads are issued before page k
  // is computed.  Every path issues exactly the pages the wave owns (the tail
  // is peeled), so the count of loads outstanding at each compute is fixed
  // and only the page being computed is waited for.  Table entries are read
  // one step ahead of the loads that need them.
  // Folded append: this wave's last page is the sequence's last block, which
  // holds the newest token (the partition holding it has only one workgroup
  // per kv head: a single 16-head group).  bf16 and E4M3 pages.
  bool fold = false;
  int fold_blk = 0;
  {
    const int n_raw = p.seq_lens[b];
    fold = p.k_new != nullptr && cnt > 0 && n_raw > 0 && n_raw <= p.maxb * kBlock &&
           pw0 + cnt == nblk;
    if (fold) fold_blk = trow[nblk - 1];
  }
  auto fold_if_last = [&](PageT<D, KVF>& pg, int kk) {
    if (fold && kk == cnt - 1)
      fold_new_token<D>(pg, p, b, kvh, fold_blk, (n - 1) & (kBlock - 1), col, grp);
  };
  if (cnt > 0) {
    PageT<D, KVF> pa, pb;
    const int last = cnt - 1;
    bool ok_a = issue_page<D, KVF>(pa, p, trow[pw0], kvh, col, grp);
    int tb1 = trow[pw0 + min(1, last)];
    int tb2 = trow[pw0 + min(2, last)];
    int k = 0;
    for (; k + 2 <= last; k += 2) {
      const bool ok_b = issue_page<D, KVF>(pb, p, tb1, kvh, col, grp);
      if (ok_a) compute_page<D>(st, pa, qf, (pw0 + k) * kBlock + 4 * grp, n, p.scale_log2);
      ok_a = issue_page<D, KVF>(pa, p, tb2, kvh, col, grp);
      tb1 = trow[pw0 + min(k + 3, last)];
      tb2 = trow[pw0 + min(k + 4, last)];
      if (ok_b) compute_page<D>(st, pb, qf, (pw0 + k + 1) * kBlock + 4 * grp, n, p.scale_log2);
    }
    if (k + 1 <= last) {
      const bool ok_b = issue_page<D, KVF>(pb, p, tb1, kvh, col, grp);
      if (ok_a) compute_page<D>(st, pa, qf, (pw0 + k) * kBlock + 4 * grp, n, p.scale_log2);
      if (ok_b) {
        fold_if_last(pb, k + 1);
        compute_page<D>(st, pb, qf, (pw0 + k + 1) * kBlock + 4 * grp, n, p.scale_log2);
      }
    } else if (ok_a) {
      fold_if_last(pa, k);
      compute_page<D>(st, pa, qf, (pw0 + k) * kBlock + 4 * grp, n, p.scale_log2);
    }
  }

  // wave state -> LDS (sum l over the 4 lanes of each head)
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (grp == 0) {
    sm_m[w][col] = st.m;
    sm_l[w][col] = l;
  }
#pragma unroll
  for (int nn = 0; nn < D / 16; ++nn)
    *reinterpret_cast<f32x4*>(&sm_o[w][col][16 * nn + 4 * grp]) = st.o[nn];
  __syncthreads();

  // combine the waves: thread -> (head g, D/16 dims), kThreads / 16 heads
  // at a time
  const int dc = threadIdx.x & 15;
  constexpr int DPT = D / 16;
  for (int g = threadIdx.x >> 4; g < 16; g += kThreads / 16) {
    if (hg * 16 + g >= p.G) break;
    const int64_t row = (int64_t)b * p.hq + (int64_t)kvh * p.G + hg * 16 + g;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, sm_m[ww][g]);
    float a[kNW];
    float L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      const float mw = sm_m[ww][g];
      a[ww] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += a[ww] * sm_l[ww][g];
    }
    float* po = p.part_o + ((int64_t)part * p.rows + row) * D;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int d = dc * DPT + e;
      float acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < kNW; ++ww) acc += a[ww] * sm_o[ww][g][d];
      po[d] = acc;
    }
    if (dc == 0) {
      p.part_m[(int64_t)part * p.rows + row] = M == -INFINITY ? -INFINITY : M * kLn2;
      p.part_l[(int64_t)part * p.rows + row] = L;
    }
  }
}

// ---- simple path: any supported dtype pair, vector ALU, one wave per
// (partition, kv head, sequence); heads of the group one after another.
// Element (token t, dimension d) of a K page / V page: f32 pages are plain
// ([16][D] and [D][16]); bf16 pages are in fragment order.
template <int KT>
__device__ __forceinline__ float k_value(const uint8_t* page, int t, int d, int D) {
  static_assert(KT == PKV_F32 || KT == PKV_BF16, "E4M3 pools take the MFMA path");
  if constexpr (KT == PKV_F32) return reinterpret_cast<const float*>(page)[t * D + d];
  else return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(page + frag_k_off<2>(t, d)));
}
template <int KT>
__device__ __forceinline__ float v_value(const uint8_t* page, int t, int d) {
  static_assert(KT == PKV_F32 || KT == PKV_BF16, "E4M3 pools take the MFMA path");
  if constexpr (KT == PKV_F32) return reinterpret_cast<const float*>(page)[d * kBlock + t];
  else return bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(page + frag_v_off<2>(t, d)));
}

template <int QT, int KT>
__global__ __launch_bounds__(64) void decode_simple_kernel(DecodeParams p, int D) {
  const int part = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int n = seq_len_clamped(p, b);
  const int nblk = (n + kBlock - 1) / kBlock;
  const int j0 = part * p.PB, j1 = min(j0 + p.PB, nblk);
  constexpr int esz = KT == PKV_F32 ? 4 : (KT == PKV_BF16 ? 2 : 1);
  const int32_t* trow = p.tables + (int64_t)b * p.maxb;
  for (int gi = 0; gi < p.G; ++gi) {
    const int64_t row = (int64_t)b * p.hq + (int64_t)kvh * p.G + gi;
    float q[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      float val = 0.f;
      if (d < D) {
        if constexpr (QT == PKV_F32) val = reinterpret_cast<const float*>(p.q)[row * D + d];
        else val = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p.q)[row * D + d]);
      }
      q[e] = val;
    }
    float m = -INFINITY, l = 0.f, o[2] = {0.f, 0.f};
    for (int j = j0; j < j1; ++j) {
      const int blk = trow[j];
      if ((unsigned)blk >= (unsigned)p.num_blocks) continue;
      const uint8_t* kp = p.k + (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * kBlock * D * esz;
      const uint8_t* vp = p.v + (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * D * kBlock * esz;
      for (int t = 0; t < kBlock && j * kBlock + t < n; ++t) {
        float part_dot = 0.f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = lane + 64 * e;
          if (d < D) part_dot += q[e] * k_value<KT>(kp, t, d, D);
        }
        const float s = wave_sum(part_dot) * p.scale_log2;
        const float m_new = fmaxf(m, s);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        const float pw = __builtin_amdgcn_exp2f(s - m_new);
        l = l * alpha + pw;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = lane + 64 * e;
          const float vv = d < D ? v_value<KT>(vp, t, d) : 0.f;
          o[e] = o[e] * alpha + pw * vv;
        }
        m = m_new;
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d < D) p.part_o[((int64_t)part * p.rows + row) * D + d] = o[e];
    }
    if (lane == 0) {
      p.part_m[(int64_t)part * p.rows + row] = m == -INFINITY ? -INFINITY : m * kLn2;
      p.part_l[(int64_t)part * p.rows + row] = l;
    }
  }
}

}  // namespace

DecodePlan plan_decode(int B, int hq, int hkv, int head_dim, int maxb, int partition_blocks,
                       int q_dtype, int kv_dtype) {
  DecodePlan plan{};
  plan.mfma = q_dtype == PKV_BF16 && (kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3);
  const int G = hq / hkv;
  plan.head_groups = plan.mfma ? (G + 15) / 16 : 1;
  int pb = partition_blocks;
  if (pb <= 0) {
    // enough workgroups to fill 256 CUs several times over
    const int64_t units = (int64_t)B * hkv * plan.head_groups;
    const int64_t target = plan.mfma ? 1024 : 2048;
    int64_t P = units > 0 ? (target + units - 1) / units : 1;
    if (P < 1) P = 1;
    if (P > maxb) P = maxb;
    pb = (int)((maxb + P - 1) / P);
    if (pb < 1) pb = 1;
  }
  plan.partition_blocks = pb;
  plan.partitions = (maxb + pb - 1) / pb;
  if (plan.partitions < 1) plan.partitions = 1;
  // Workspace: [O~][m][l], each 256-byte aligned.
  const size_t rows = (size_t)B * hq * plan.partitions;
  size_t bytes = (rows * head_dim * sizeof(float) + 255) & ~size_t(255);
  bytes += 2 * ((rows * sizeof(float) + 255) & ~size_t(255));
  plan.ws_bytes = bytes;
  return plan;
}

hipError_t launch_decode_partial(const CacheView& c, const void* q, int q_dtype, int B, int hq,
                                 const int32_t* tables, int maxb, const int32_t* seq_lens,
                                 float scale, const DecodePlan& plan, float* part_o,
                                 float* part_m, float* part_l, hipStream_t s,
                                 const void* k_new, const void* v_new) {
  if (B == 0) return hipSuccess;
  const int D = c.head_dim;
  const int esz = c.kv_dtype == PKV_F32 ? 4 : (c.kv_dtype == PKV_BF16 ? 2 : 1);
  DecodeParams p{};
  p.k = static_cast<const uint8_t*>(c.k);
  p.v = static_cast<const uint8_t*>(c.v);
  p.block_stride_bytes = c.block_stride * esz;
  p.k_scale = c.k_scale;
  p.v_scale = c.v_scale;
  p.num_blocks = c.num_blocks;
  p.hkv = c.hkv;
  p.hq = hq;
  p.G = hq / c.hkv;
  p.HG = plan.head_groups;
  p.q = q;
  p.q_dtype = q_dtype;
  p.tables = tables;
  p.maxb = maxb;
  p.seq_lens = seq_lens;
  p.scale_log2 = scale * kLog2e;
  p.P = plan.partitions;
  p.PB = plan.partition_blocks;
  p.rows = (int64_t)B * hq;
  p.part_o = part_o;
  p.part_m = part_m;
  p.part_l = part_l;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  if (k_new && !(plan.mfma && plan.head_groups == 1))
    return hipErrorInvalidValue;            // the fold needs the MFMA path with one head group

  if (plan.mfma) {
    dim3 grid(plan.partitions, c.hkv * plan.head_groups, B), block(kThreads);
    if (c.kv_dtype == PKV_BF16) {
      if (D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, PKV_BF16>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode_mfma_kernel<64, PKV_BF16>), grid, block, 0, s, p);
    } else {
      if (D == 128) hipLaunchKernelGGL((decode_mfma_kernel<128, PKV_FP8_E4M3>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((decode_mfma_kernel<64, PKV_FP8_E4M3>), grid, block, 0, s, p);
    }
  } else {
    dim3 grid(plan.partitions, c.hkv, B), block(64);
    if (q_dtype == PKV_F32) {
      if (c.kv_dtype == PKV_F32) hipLaunchKernelGGL((decode_simple_kernel<PKV_F32, PKV_F32>), grid, block, 0, s, p, D);
      else if (c.kv_dtype == PKV_BF16) hipLaunchKernelGGL((decode_simple_kernel<PKV_F32, PKV_BF16>), grid, block, 0, s, p, D);
      else return hipErrorInvalidValue;
    } else {
      if (c.kv_dtype == PKV_F32) hipLaunchKernelGGL((decode_simple_kernel<PKV_BF16, PKV_F32>), grid, block, 0, s, p, D);
      else return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_decode(const CacheView& c, const void* q, int q_dtype, int B, int hq,
                         const int32_t* tables, int maxb, const int32_t* seq_lens, float scale,
                         const DecodePlan& plan, void* out, float* out_lse, void* ws,
                         hipStream_t s, const void* k_new, const void* v_new) {
  if (B == 0) return hipSuccess;
  const int D = c.head_dim;
  const size_t rows = (size_t)B * hq * plan.partitions;
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* part_o = reinterpret_cast<float*>(w);
  size_t off = (rows * D * sizeof(float) + 255) & ~size_t(255);
  float* part_m = reinterpret_cast<float*>(w + off);
  off += (rows * sizeof(float) + 255) & ~size_t(255);
  float* part_l = reinterpret_cast<float*>(w + off);
  hipError_t e = launch_decode_partial(c, q, q_dtype, B, hq, tables, maxb, seq_lens, scale, plan,
                                       part_o, part_m, part_l, s, k_new, v_new);
  if (e != hipSuccess) return e;
  return launch_merge(partition_merge_args(plan.partitions, (int64_t)B * hq, D, part_o, part_m,
                                           part_l, out, q_dtype, out_lse),
                      s);
}

MergeArgs partition_merge_args(int S, int64_t rows, int D, const float* part_o,
                               const float* part_m, const float* part_l, void* out,
                               int out_dtype, float* out_lse) {
  MergeArgs a{};
  a.S = S;
  a.rows = rows;
  a.D = D;
  a.o = part_o;
  a.o_row = D;
  a.o_part = rows * D;
  a.m = part_m;
  a.l = part_l;
  a.ml_row = 1;
  a.ml_part = rows;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_m = nullptr;
  a.out_l = nullptr;
  a.out_lse = out_lse;
  return a;
}

}  // namespace pkv

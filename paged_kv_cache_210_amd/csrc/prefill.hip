// Chunked causal prefill against the paged KV cache, on bf16 MFMA.
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
// V is converted to fp16 as it is staged (exact for bf16 values within fp16's
// range) so the softmax weights can enter the second product with 11
// significant bits instead of bf16's 8.
// Computing S transposed puts one query row in each lane (plus its partner
// lane l^32), so row max / sum need a single cross-lane step and the softmax
// weights are already laid out as the B operand of the second product.
//
// Workgroup = 4 waves x 32 query rows of one head; K/V tiles of 64 tokens (4
// pages) are gathered through the block table into double-buffered LDS.
// Workgroup i serves kv head i % Hkv, so with 8 kv heads every XCD streams one
// head's K/V through its own L2.
#include "pkv_common.h"

namespace pkv {
namespace {

constexpr int D = 128;
constexpr int BN = 64;                   // tokens per K/V tile (4 pages)
constexpr int ROWS_W = 32;               // query rows per wave
constexpr int NWAVE = 4;
constexpr int BM = ROWS_W * NWAVE;       // query rows per workgroup
constexpr int TILE_BYTES = BN * D * 2;   // 16 KiB for K, same for V
constexpr float kLazy = 8.0f;            // log2 headroom of the running max

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct PrefillParams {
  const uint8_t* k;
  const uint8_t* v;
  int64_t block_stride_bytes;
  int num_blocks, hkv, hq, G;
  const uint16_t* q;
  int T, q_pos0;
  const int32_t* table;
  int maxb;
  int kv_begin, kv_end;
  int causal;
  float scale_log2;
  int row_tiles;
  uint16_t* out;
  float* out_lse;
  float* part_o;
  float* part_m;
  float* part_l;
};

// LDS K tile: [64 tokens][16 chunks of 16 B]; chunk c of token t sits at
// c ^ (t & 15) so 16 lanes reading one chunk column hit 16 distinct chunks.
__device__ __forceinline__ int k_lds_off(int t, int c) { return t * 256 + ((c ^ (t & 15)) << 4); }

// LDS V tile: [4 pages][128 dims][32 B]; within a dimension the 16 tokens are
// stored as halves {0-3, 8-11} and {4-7, 12-15} (the token sets one 32x32x16
// k-step takes from each lane half), and the halves swap when (d >> 3) is odd.
__device__ __forceinline__ int v_lds_off(int page, int d, int half) {
  return page * 4096 + d * 32 + ((half ^ ((d >> 3) & 1)) << 4);
}

struct TileRegs {
  u32x4 k[4];   // this thread's 4 x 16 B of its wave's K page
  u32x4 v[4];   // and of its V page
};

// Wave w fetches page w of the tile: K page bytes [i*1024 + lane*16), same for V.
__device__ __forceinline__ void load_tile(TileRegs& r, const PrefillParams& p, int tile, int w,
                                          int lane, int kvh, bool& valid) {
  const int lblk = tile * 4 + w;
  int blk = -1;
  if (lblk < p.maxb && lblk * kBlock < p.kv_end) blk = p.table[lblk];
  valid = (unsigned)blk < (unsigned)p.num_blocks;
  if (!valid) return;
  const uint8_t* kp = p.k + (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * kBlock * D * 2;
  const uint8_t* vp = p.v + (int64_t)blk * p.block_stride_bytes + (int64_t)kvh * D * kBlock * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.k[i] = *reinterpret_cast<const u32x4*>(kp + i * 1024 + lane * 16);
    r.v[i] = *reinterpret_cast<const u32x4*>(vp + i * 1024 + lane * 16);
  }
}

// Registers -> LDS.  Tokens outside [kv_begin, kv_end) get zero V (and zero K)
// on boundary tiles, and pages without a valid block are all zero, so masked
// positions contribute exactly nothing to P V.
__device__ __forceinline__ void store_tile(uint8_t* ks, uint8_t* vs, const TileRegs& r,
                                           const PrefillParams& p, int tile, int w, int lane,
                                           bool valid, bool boundary) {
  const int tok_base = tile * BN + w * kBlock;     // first token of this wave's page
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = i * 1024 + lane * 16;
    // K: token o / 256 of the page, chunk (o % 256) / 16
    {
      const int tp = o >> 8, c = (o & 255) >> 4;
      u32x4 val = r.k[i];
      if (!valid) val = u32x4{0u, 0u, 0u, 0u};
      else if (boundary) {
        const int ta = tok_base + tp;
        if (ta < p.kv_begin || ta >= p.kv_end) val = u32x4{0u, 0u, 0u, 0u};
      }
      *reinterpret_cast<u32x4*>(ks + k_lds_off(w * kBlock + tp, c)) = val;
    }
    // V: dimension o / 32, tokens 8*th .. 8*th+7 with th = (o % 32) / 16
    {
      const int d = o >> 5, th = (o & 31) >> 4;
      u32x4 val = r.v[i];
      if (!valid) val = u32x4{0u, 0u, 0u, 0u};
      else if (boundary) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ta = tok_base + 8 * th + 2 * e;
          uint32_t keep = 0u;
          if (ta >= p.kv_begin && ta < p.kv_end) keep |= 0x0000ffffu;
          if (ta + 1 >= p.kv_begin && ta + 1 < p.kv_end) keep |= 0xffff0000u;
          val[e] &= keep;
        }
      }
      // bf16 -> fp16 (exact for |v| within fp16's normal range; beyond 65504
      // the round-toward-zero conversion saturates instead of overflowing)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        val[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(
                                                  __uint_as_float(val[e] << 16),
                                                  __uint_as_float(val[e] & 0xffff0000u)));
      // tokens 8th+0..3 -> half 0, tokens 8th+4..7 -> half 1; byte offset 8*th
      const u32x2 lo = {val[0], val[1]}, hi = {val[2], val[3]};
      *reinterpret_cast<u32x2*>(vs + v_lds_off(w, d, 0) + 8 * th) = lo;
      *reinterpret_cast<u32x2*>(vs + v_lds_off(w, d, 1) + 8 * th) = hi;
    }
  }
}

// One 64-token K/V tile for this wave's 32 query rows: S^T = K Q^T, online
// softmax, O^T += V^T P^T.  The per-score visibility test runs only on tiles
// that cross kv_begin / kv_end or the causal diagonal of this wave's rows
// (need_mask, uniform over the wave).
struct RowState {
  f32x16 o[4];
  float m, l, mtrue;
};

template <bool NEG_SCALE>
__device__ __forceinline__ void attend_tile(RowState& st, const uint8_t* ks, const uint8_t* vs,
                                            const u32x4 (&qf)[8], const PrefillParams& p, int tb,
                                            int my_pos, int qr, int hi, bool need_mask) {
  // ---- S^T = K Q^T over two 32-token halves of the tile
  f32x16 s[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
    const int t = 32 * mt + qr;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(ks + k_lds_off(t, 2 * c + hi));
      s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                     __builtin_bit_cast(bf16x8, qf[c]), s[mt], 0,
                                                     0, 0);
    }
  }
  // ---- mask, online softmax in log2 units.  The largest scaled score is
  // c * max(s) for c > 0 and c * min(s) for c < 0, so the scale is folded
  // into one FMA per score: p = exp2(s * c - m).
  const float c = p.scale_log2;
  const float hidden = NEG_SCALE ? INFINITY : -INFINITY;   // s * c == -inf
  if (need_mask) {
    // visible keys of this lane's row: [lo, hi_) relative to the tile
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
  float ext = hidden;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ext = NEG_SCALE ? fminf(ext, s[mt][r]) : fmaxf(ext, s[mt][r]);
  // The running max is raised only when a score exceeds it by more than
  // kLazy (weights stay below 2^kLazy); the row's lane pair then agrees on the
  // new max and O, l are rescaled.  Same result, and the common tile needs no
  // cross-lane step and no rescale.
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
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= alpha;
    st.m = m_new;
  }
  const float m_use = st.m == -INFINITY ? 0.f : st.m;
  // ---- O^T += V^T P^T, four 16-token k-steps, in fp16 (V was converted
  // exactly when staged; fp16 weights carry 11 significant bits).  The row sum
  // is taken over the rounded weights that enter the product, so the result
  // stays an exact weighted average of V rows.
  float rs = 0.f;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      f16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pb[e] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][8 * rr + e], c, -m_use));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 pr = {pb[2 * e], pb[2 * e + 1]};
        rs = __builtin_amdgcn_fdot2(pr, ones, rs, false);
      }
      const int page = 2 * mt + rr;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int d = 32 * dt + qr;
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vs + v_lds_off(page, d, hi));
        st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, vf), pb,
                                                         st.o[dt], 0, 0, 0);
      }
    }
  st.l += rs;
}

template <bool NEG_SCALE>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2 * TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5;        // lane half
  const int qr = lane & 31;        // query row within the wave

  // workgroup -> (kv head, head in group, row tile); heavier (later) row tiles first
  const int i = blockIdx.x;
  const int kvh = i % p.hkv;
  const int rest = i / p.hkv;
  const int gi = rest % p.G;
  const int rt = p.row_tiles - 1 - rest / p.G;
  const int h = kvh * p.G + gi;
  const int row0 = rt * BM;
  const int wrow0 = row0 + w * ROWS_W;
  const int my_row = wrow0 + qr;
  const bool row_ok = my_row < p.T;
  const int my_pos = p.q_pos0 + my_row;

  // query fragments (B operand): Q[row][16c + 8*hi .. +8]
  u32x4 qf[8];
  {
    const uint16_t* qp = p.q + ((int64_t)my_row * p.hq + h) * D;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[c] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 16 * c + 8 * hi)
                     : u32x4{0u, 0u, 0u, 0u};
  }

  // keys this workgroup may see
  const int last_row = min(row0 + BM, p.T) - 1;
  int key_end = p.kv_end;
  if (p.causal) key_end = min(key_end, p.q_pos0 + last_row + 1);
  const int t_lo = p.kv_begin / BN;
  const int t_hi = key_end > p.kv_begin ? (key_end - 1) / BN : t_lo - 1;
  // this wave's rows: position range for masking decisions
  const int w_last = min(wrow0 + ROWS_W, p.T) - 1;
  const int w_minpos = p.q_pos0 + wrow0;
  const int w_maxpos = p.q_pos0 + w_last;
  const bool wave_live = wrow0 < p.T;

  RowState st;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[dt][r] = 0.f;
  st.m = -INFINITY;
  st.l = 0.f;
  st.mtrue = -INFINITY;           // this lane's exact max of the scaled scores

  TileRegs regs;
  bool valid = false;
  if (t_lo <= t_hi) {
    load_tile(regs, p, t_lo, w, lane, kvh, valid);
    const bool bnd = t_lo * BN < p.kv_begin || t_lo * BN + BN > p.kv_end;
    store_tile(smem[0], smem[0] + TILE_BYTES, regs, p, t_lo, w, lane, valid, bnd);
  }
  __syncthreads();

  for (int tile = t_lo; tile <= t_hi; ++tile) {
    const int buf = (tile - t_lo) & 1;
    const bool more = tile < t_hi;
    if (more) load_tile(regs, p, tile + 1, w, lane, kvh, valid);

    const int tb = tile * BN;
    const bool wave_sees = wave_live && (!p.causal || tb <= w_maxpos);
    if (wave_sees) {
      const uint8_t* ks = smem[buf];
      const uint8_t* vs = smem[buf] + TILE_BYTES;
      const bool need_mask = tb < p.kv_begin || tb + BN > p.kv_end ||
                             (p.causal && tb + BN - 1 > w_minpos);
      attend_tile<NEG_SCALE>(st, ks, vs, qf, p, tb, my_pos, qr, hi, need_mask);
    }

    if (more) {
      const int nb = buf ^ 1;
      const int nt = tile + 1;
      const bool bnd = nt * BN < p.kv_begin || nt * BN + BN > p.kv_end;
      store_tile(smem[nb], smem[nb] + TILE_BYTES, regs, p, nt, w, lane, valid, bnd);
    }
    __syncthreads();
  }

  // ---- epilogue: row sum over the lane pair, then normalise or emit partials
  float l = st.l + __shfl_xor(st.l, 32);
  const float mtrue = fmaxf(st.mtrue, __shfl_xor(st.mtrue, 32));
  float m = st.m;
  f32x16 (&o)[4] = st.o;
  if (!row_ok) return;
  const bool empty = !(l > 0.f);
  const int64_t ro = (int64_t)my_row * p.hq + h;
  if (p.out) {
    const float inv = empty ? 0.f : 1.0f / l;
    uint16_t* op = p.out + ro * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hi;
        u32x2 pk;
        pk.x = (uint32_t)f32_to_bf16_bits(o[dt][4 * j] * inv) |
               ((uint32_t)f32_to_bf16_bits(o[dt][4 * j + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16_bits(o[dt][4 * j + 2] * inv) |
               ((uint32_t)f32_to_bf16_bits(o[dt][4 * j + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(op + d) = pk;
      }
    if (p.out_lse && hi == 0) p.out_lse[ro] = empty ? -INFINITY : m * kLn2 + logf(l);
  } else {
    // partials are exported relative to the exact row max (m <= mtrue <= m + kLazy)
    const float f = empty ? 0.f : __builtin_amdgcn_exp2f(m - mtrue);
    l *= f;
    m = mtrue;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= f;
    float* op = p.part_o + ro * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * dt + 8 * j + 4 * hi;
        const f32x4 val = empty ? f32x4{0.f, 0.f, 0.f, 0.f}
                                : f32x4{o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2],
                                        o[dt][4 * j + 3]};
        *reinterpret_cast<f32x4*>(op + d) = val;
      }
    if (hi == 0) {
      p.part_m[ro] = empty ? -INFINITY : m * kLn2;
      p.part_l[ro] = empty ? 0.f : l;
    }
  }
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
  p.block_stride_bytes = c.block_stride * 2;
  p.num_blocks = c.num_blocks;
  p.hkv = c.hkv;
  p.hq = hq;
  p.G = hq / c.hkv;
  p.q = static_cast<const uint16_t*>(q);
  p.T = T;
  p.q_pos0 = q_pos0;
  p.table = table;
  p.maxb = maxb;
  p.kv_begin = kv_begin;
  p.kv_end = kv_end;
  p.causal = causal;
  p.scale_log2 = scale * kLog2e;
  p.row_tiles = (T + BM - 1) / BM;
  p.out = static_cast<uint16_t*>(out);
  p.out_lse = out_lse;
  p.part_o = part_o;
  p.part_m = part_m;
  p.part_l = part_l;
  const int64_t wgs = (int64_t)p.row_tiles * hq;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  if (scale < 0.f)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)wgs), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)wgs), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv

// kv_append (reshape-and-cache) and FP8 block-wise scales.
//
// [P1] "Long-context inference engineering truths 2026 ..." section 2.2: a
// token at position t lands in slot t % 16 of the physical block that the
// sequence's table names for logical block t / 16.
// [P2] "Unlocking long context ..." section 3.2: FP8 (E4M3) KV with one scale
// per group of 64-128 tokens (64 here).
#include "pkv_common.h"

namespace pkv {
namespace {

struct AppendParams {
  uint8_t* k_pool;
  uint8_t* v_pool;
  int64_t block_stride;      // elements
  const float* k_scale;
  const float* v_scale;
  int num_blocks, hkv, D;
  const void* k_new;
  const void* v_new;
  int num_tokens;
  const int32_t* seq_idx;
  const int32_t* pos;
  const int32_t* tables;
  int num_seqs, maxb;
};

template <typename T>
__device__ __forceinline__ T load_elem(const void* p, int64_t i) {
  return reinterpret_cast<const T*>(p)[i];
}

// A chunk is 8 consecutive elements of one token's [Hkv][d] row.  Its 8 K
// elements stay contiguous in the page (one store); its V elements are
// scattered (one store each).  bf16 and E4M3 pages are written in fragment
// order, f32 pages plainly ([16][d] K, [d][16] V).  Same-type caches copy raw
// bits; E4M3 caches quantise f32(x) * f32(1/scale) with the scale of the
// destination (block, head), two at a time (e4m3_encode2).
constexpr int kChunk = 8;      // elements per chunk

template <int SRC>
struct SrcChunk;
template <>
struct SrcChunk<PKV_BF16> {
  u32x4 k, v;                  // 8 bf16
};
template <>
struct SrcChunk<PKV_F32> {
  u32x4 k[2], v[2];            // 8 fp32
};

// Source rows are read exactly once: non-temporal loads (measured +16 % on
// the 4096-token chunks of a 131072-token prompt, whose rows come from HBM).
template <int SRC>
__device__ __forceinline__ void load_chunk(SrcChunk<SRC>& c, const void* k, const void* v,
                                           int64_t e) {
  if constexpr (SRC == PKV_BF16) {
    c.k = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(k) + e));
    c.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(v) + e));
  } else {
    const u32x4* kp = reinterpret_cast<const u32x4*>(static_cast<const float*>(k) + e);
    const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const float*>(v) + e);
    c.k[0] = __builtin_nontemporal_load(kp);
    c.k[1] = __builtin_nontemporal_load(kp + 1);
    c.v[0] = __builtin_nontemporal_load(vp);
    c.v[1] = __builtin_nontemporal_load(vp + 1);
  }
}

// element i (0..7) of a chunk as fp32
template <int SRC>
__device__ __forceinline__ float chunk_f32(const u32x4& x0, const u32x4* x, int i) {
  if constexpr (SRC == PKV_BF16) {
    const uint32_t w = x0[i >> 1];
    return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
  } else {
    return __uint_as_float(x[i >> 2][i & 3]);
  }
}

template <int SRC, int DST>
__device__ __forceinline__ void store_chunk(const AppendParams& p, const SrcChunk<SRC>& c,
                                            int blk, int64_t base, int off, int e) {
  const int h = e / p.D;
  const int d = e - h * p.D;                 // chunk never crosses a head (D % 8 == 0)
  if constexpr (DST == PKV_FP8_E4M3) {
    // bf16 and E4M3 pages are in fragment order (frag_k_off / frag_v_off);
    // the 8 elements of a chunk stay contiguous in the K page (d % 8 == 0)
    const int64_t kq = base + (int64_t)h * kBlock * p.D + frag_k_off<1>(off, d);
    const int64_t vq = base + (int64_t)h * p.D * kBlock;
    const int64_t si = (int64_t)blk * p.hkv + h;
    const float inv_k = __frcp_rn(p.k_scale[si]);
    const float inv_v = __frcp_rn(p.v_scale[si]);
    const u32x4* kx = nullptr;
    const u32x4* vx = nullptr;
    u32x4 k0{}, v0{};
    if constexpr (SRC == PKV_BF16) {
      k0 = c.k;
      v0 = c.v;
    } else {
      kx = c.k;
      vx = c.v;
    }
    u32x2 codes = {0u, 0u};
#pragma unroll
    for (int i = 0; i < kChunk; i += 2) {
      codes[i >> 2] |= e4m3_encode2(__fmul_rn(chunk_f32<SRC>(k0, kx, i), inv_k),
                                    __fmul_rn(chunk_f32<SRC>(k0, kx, i + 1), inv_k))
                       << (8 * (i & 3));
      const uint32_t cv = e4m3_encode2(__fmul_rn(chunk_f32<SRC>(v0, vx, i), inv_v),
                                       __fmul_rn(chunk_f32<SRC>(v0, vx, i + 1), inv_v));
      p.v_pool[vq + frag_v_off<1>(off, d + i)] = (uint8_t)cv;
      p.v_pool[vq + frag_v_off<1>(off, d + i + 1)] = (uint8_t)(cv >> 8);
    }
    *reinterpret_cast<u32x2*>(p.k_pool + kq) = codes;
  } else if constexpr (DST == PKV_BF16) {
    uint8_t* kpg = p.k_pool + 2 * (base + (int64_t)h * kBlock * p.D);
    uint8_t* vpg = p.v_pool + 2 * (base + (int64_t)h * p.D * kBlock);
    *reinterpret_cast<u32x4*>(kpg + frag_k_off<2>(off, d)) = c.k;
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      *reinterpret_cast<uint16_t*>(vpg + frag_v_off<2>(off, d + i)) =
          (uint16_t)((i & 1) ? (c.v[i >> 1] >> 16) : (c.v[i >> 1] & 0xffffu));
  } else {
    const int64_t kd = base + (int64_t)h * kBlock * p.D + (int64_t)off * p.D + d;
    const int64_t vd = base + (int64_t)h * p.D * kBlock + (int64_t)d * kBlock + off;
    float* kp = reinterpret_cast<float*>(p.k_pool) + kd;
    *reinterpret_cast<u32x4*>(kp) = c.k[0];
    *reinterpret_cast<u32x4*>(kp + 4) = c.k[1];
    float* vp = reinterpret_cast<float*>(p.v_pool) + vd;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) vp[(int64_t)i * kBlock] = __uint_as_float(c.v[i >> 2][i & 3]);
  }
}

// A workgroup takes 16 consecutive input tokens and one kv head; thread
// (t, ch) holds chunk ch of token t's row for that head, loaded before the
// block lookups so that their latencies overlap.  When the 16 tokens are
// positions p0 .. p0+15 (p0 % 16 == 0) of one sequence and the page exists,
// the head's K and V pages are written whole: K chunks go straight to their
// fragment slots, V through a [d][16] LDS transpose in 16-byte pieces (bf16
// and E4M3 pools; a prefill chunk takes this path).  Otherwise each thread
// appends its chunk (store_chunk), which covers decode steps, ragged ends and
// f32 pools.
constexpr int kGroup = 16;

// The V transpose in LDS: row d holds the 16 tokens of dimension d (32 bytes
// for bf16, 16 for E4M3) and every 8 rows are followed by an 8-byte (bf16) or
// 4-byte (E4M3) gap, so the 16 chunks of one token, whose rows lie 8 apart,
// fall in different banks; readers take 4 tokens of one row as one word.
__device__ __forceinline__ int vt16_row(int d) { return d * kGroup + (d >> 3) * 4; }   // uint16s
__device__ __forceinline__ int vt8_row(int d) { return d * kGroup + (d >> 3) * 4; }    // bytes
constexpr int kVtElems = 128 * kGroup + 16 * 4;

template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kVtElems];   // V of one head, [d][16]
  const int tid = threadIdx.x;
  const int tok0 = blockIdx.x * kGroup;
  const int h = blockIdx.y;
  const int HD = p.hkv * p.D;
  const int cpt = p.D / kChunk;                 // chunks per token and head
  const int t = tid / cpt, ch = tid - t * cpt;  // this thread's token and chunk
  const int tok = tok0 + t;
  const bool mine = t < kGroup && tok < p.num_tokens;
  // every thread loads a chunk (threads past the group repeat the last token)
  const int tokc = mine ? tok : min(tok0 + kGroup, p.num_tokens) - 1;
  const int e = h * p.D + ch * kChunk;
  SrcChunk<SRC> c1;
  load_chunk<SRC>(c1, p.k_new, p.v_new, (int64_t)tokc * HD + e);
  const int b = p.seq_idx[tokc], pos = p.pos[tokc];
  // whole-page test: every token is (b0, p0 + t) with p0 a page start
  const int b0 = p.seq_idx[tok0], p0 = p.pos[tok0];
  bool page = (DST != PKV_F32) && tok0 + kGroup <= p.num_tokens && b0 >= 0 &&
              b0 < p.num_seqs && p0 >= 0 && (p0 & (kBlock - 1)) == 0 && (p0 >> 4) < p.maxb;
  int pblk = -1;
  if (page) {
    pblk = p.tables[(int64_t)b0 * p.maxb + (p0 >> 4)];
    page = pblk >= 0 && pblk < p.num_blocks;
  }
  page = __syncthreads_and(page && (!mine || (b == b0 && pos == p0 + t))) != 0;

  if constexpr (DST == PKV_BF16) {
    if (page) {
      const int64_t base = (int64_t)pblk * p.block_stride;
      uint8_t* kpg = p.k_pool + 2 * (base + (int64_t)h * kBlock * p.D);
      uint8_t* vpg = p.v_pool + 2 * (base + (int64_t)h * p.D * kBlock);
      if (mine) {
        __builtin_nontemporal_store(c1.k, reinterpret_cast<u32x4*>(kpg + frag_k_off<2>(t, 8 * ch)));
#pragma unroll
        for (int i = 0; i < kChunk; ++i)
          vt[vt16_row(8 * ch + i) + t] =
              (uint16_t)((i & 1) ? (c1.v[i >> 1] >> 16) : (c1.v[i >> 1] & 0xffffu));
      }
      __syncthreads();
      if (tid < 2 * p.D) {
        // V piece q: tokens 4 ((q / 16) % 4) .. +4 of dimensions 32 (q / 64) + q % 16 and +16
        const int q = tid, c = q >> 6, tg = (q >> 4) & 3, i = q & 15;
        const int d0 = 32 * c + i;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&vt[vt16_row(d0) + 4 * tg]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(&vt[vt16_row(d0 + 16) + 4 * tg]);
        __builtin_nontemporal_store(u32x4{lo.x, lo.y, hi.x, hi.y}, reinterpret_cast<u32x4*>(vpg + 16 * q));
      }
      return;
    }
  }
  if constexpr (DST == PKV_FP8_E4M3) {
    if (page) {
      // codes are f32(x) * f32(1 / scale) rounded to E4M3, exactly as store_chunk
      // makes them; the V codes go through a [d][16] byte transpose
      uint8_t* vt8 = reinterpret_cast<uint8_t*>(vt);
      const int64_t si = (int64_t)pblk * p.hkv + h;
      const float inv_k = __frcp_rn(p.k_scale[si]);
      const float inv_v = __frcp_rn(p.v_scale[si]);
      const int64_t base = (int64_t)pblk * p.block_stride;
      uint8_t* kpg = p.k_pool + base + (int64_t)h * kBlock * p.D;
      uint8_t* vpg = p.v_pool + base + (int64_t)h * p.D * kBlock;
      if (mine) {
        const u32x4* kx = nullptr;
        const u32x4* vx = nullptr;
        u32x4 k0{}, v0{};
        if constexpr (SRC == PKV_BF16) {
          k0 = c1.k;
          v0 = c1.v;
        } else {
          kx = c1.k;
          vx = c1.v;
        }
        u32x2 codes = {0u, 0u};
#pragma unroll
        for (int i = 0; i < kChunk; i += 2) {
          codes[i >> 2] |= e4m3_encode2(__fmul_rn(chunk_f32<SRC>(k0, kx, i), inv_k),
                                        __fmul_rn(chunk_f32<SRC>(k0, kx, i + 1), inv_k))
                           << (8 * (i & 3));
          const uint32_t cv = e4m3_encode2(__fmul_rn(chunk_f32<SRC>(v0, vx, i), inv_v),
                                           __fmul_rn(chunk_f32<SRC>(v0, vx, i + 1), inv_v));
          vt8[vt8_row(8 * ch + i) + t] = (uint8_t)cv;
          vt8[vt8_row(8 * ch + i + 1) + t] = (uint8_t)(cv >> 8);
        }
        __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(kpg + frag_k_off<1>(t, 8 * ch)));
      }
      __syncthreads();
      if (tid < p.D) {
        // V piece q: tokens 4 ((q / 16) % 4) .. +4 of dimensions 64 (q / 64) + 16 k + q % 16
        const int q = tid, c2 = q >> 6, tg = (q >> 4) & 3, i = q & 15;
        u32x4 pc;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pc[k] = *reinterpret_cast<const uint32_t*>(&vt8[vt8_row(64 * c2 + 16 * k + i) + 4 * tg]);
        __builtin_nontemporal_store(pc, reinterpret_cast<u32x4*>(vpg + 16 * q));
      }
      return;
    }
  }
  if (!mine || b < 0 || b >= p.num_seqs || pos < 0 || (pos >> 4) >= p.maxb) return;
  const int blk = p.tables[(int64_t)b * p.maxb + (pos >> 4)];
  if (blk < 0 || blk >= p.num_blocks) return;
  store_chunk<SRC, DST>(p, c1, blk, (int64_t)blk * p.block_stride, pos & (kBlock - 1), e);
}

struct ScaleParams {
  float* k_scale;
  float* v_scale;
  int hkv, D, num_blocks;
  const void* k_src;
  const void* v_src;
  int num_tokens, pos0;
  const int32_t* table_row;
  int maxb;
};

template <int SRC>
__device__ __forceinline__ float src_abs(const void* p, int64_t i) {
  if constexpr (SRC == PKV_BF16) return fabsf(bf16_bits_to_f32(load_elem<uint16_t>(p, i)));
  else return fabsf(load_elem<float>(p, i));
}

// Largest magnitude of a 16-byte piece held in registers (fmaxf skips NaN).
template <int SRC>
__device__ __forceinline__ float reg_absmax(const u32x4& x, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (SRC == PKV_BF16) {
      acc = fmaxf(acc, fabsf(__uint_as_float(x[j] << 16)));
      acc = fmaxf(acc, fabsf(__uint_as_float(x[j] & 0xffff0000u)));
    } else {
      acc = fmaxf(acc, fabsf(__uint_as_float(x[j])));
    }
  }
  return acc;
}

// Largest magnitude of the 16-byte piece at byte offset o (fmaxf skips NaN,
// as the element-wise path does).
template <int SRC>
__device__ __forceinline__ float piece_absmax(const void* p, int64_t o, float acc) {
  const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p) + o);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (SRC == PKV_BF16) {
      acc = fmaxf(acc, fabsf(__uint_as_float(x[j] << 16)));
      acc = fmaxf(acc, fabsf(__uint_as_float(x[j] & 0xffff0000u)));
    } else {
      acc = fmaxf(acc, fabsf(__uint_as_float(x[j])));
    }
  }
  return acc;
}

// grid (groups, hkv): largest magnitude over a 64-token group (the given
// tokens of it) for one head, for K and V; scale = f32(amax / 448), 1 if that
// is 0 or subnormal.  VEC:
// both sources 16-byte aligned, read in 16-byte pieces (head_dim is 64 or
// 128, so a (token, head) row is a whole number of pieces).
template <int SRC, bool VEC>
__global__ __launch_bounds__(256) void fp8_scale_kernel(ScaleParams p) {
  __shared__ float red[2][4];
  const int g = blockIdx.x, h = blockIdx.y;
  const int t0 = g * kScaleGroup;
  const int t1 = min(t0 + kScaleGroup, p.num_tokens);
  float ak = 0.f, av = 0.f;
  if constexpr (VEC) {
    constexpr int ES = SRC == PKV_BF16 ? 2 : 4;
    const int sh = __builtin_ctz((unsigned)(p.D * ES / 16));   // pieces per row = 2^sh
    const int n = (t1 - t0) << sh;
    for (int e = threadIdx.x; e < n; e += 256) {
      const int t = t0 + (e >> sh), c = e & ((1 << sh) - 1);
      const int64_t o = (((int64_t)t * p.hkv + h) * p.D) * ES + 16 * c;
      ak = piece_absmax<SRC>(p.k_src, o, ak);
      av = piece_absmax<SRC>(p.v_src, o, av);
    }
  } else {
    const int n = (t1 - t0) * p.D;
    for (int e = threadIdx.x; e < n; e += 256) {
      const int t = t0 + e / p.D, d = e % p.D;
      const int64_t i = ((int64_t)t * p.hkv + h) * p.D + d;
      ak = fmaxf(ak, src_abs<SRC>(p.k_src, i));
      av = fmaxf(av, src_abs<SRC>(p.v_src, i));
    }
  }
  ak = wave_max(ak);
  av = wave_max(av);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = ak; red[1][w] = av; }
  __syncthreads();
  if (threadIdx.x != 0) return;
  ak = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  av = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  float sk = __fdiv_rn(ak, 448.0f);
  float sv = __fdiv_rn(av, 448.0f);
  if (!(sk >= 1.17549435e-38f)) sk = 1.0f;
  if (!(sv >= 1.17549435e-38f)) sv = 1.0f;
  // every block of the group's 64-token span that the table names takes the
  // scale (blocks of a partial group not yet in the table get it from a later
  // call over the group's first tokens)
  const int first = p.pos0 + t0, last = first + kScaleGroup - 1;
  for (int j = first / kBlock; j <= last / kBlock && j < p.maxb; ++j) {
    const int blk = p.table_row[j];
    if (blk < 0 || blk >= p.num_blocks) continue;
    p.k_scale[(int64_t)blk * p.hkv + h] = sk;
    p.v_scale[(int64_t)blk * p.hkv + h] = sv;
  }
}

// pkv_fp8_group_scales and pkv_kv_append of one sequence's tokens in one
// pass: workgroup (g, h) reads the K and V rows of 64-token group g, head h
// once, reduces their largest magnitudes to the group's scales (the same
// rounding as fp8_scale_kernel), stores them into every block of the group's
// span that the table names, and encodes the rows with them (as store_chunk
// does).  Thread u holds 4 consecutive tokens x 8 dimensions, so it packs
// whole V words (4 tokens of one dimension) in registers.  A whole group is
// assembled as the four K and V pages in LDS and written in 16-byte pieces
// (pages whose block id is outside the pool are skipped, as kv_append skips
// their tokens); a partial last group is written token by token.  The block
// ids are read before the rows, so no lookup waits on the data.  Rows are
// read and whole pages written with non-temporal accesses.
struct GroupAppendParams {
  uint8_t* k_pool;
  uint8_t* v_pool;
  int64_t block_stride;      // elements (= bytes for E4M3)
  float* k_scale;
  float* v_scale;
  int num_blocks, hkv, D;
  const void* k_src;
  const void* v_src;
  int num_tokens, pos0;
  const int32_t* table_row;
  int maxb;
};

// element j (0..7) of an 8-element chunk held as NP 16-byte pieces
template <int SRC>
__device__ __forceinline__ float elem8(const u32x4* x, int j) {
  if constexpr (SRC == PKV_BF16)
    return bf16_bits_to_f32((j & 1) ? (x[0][j >> 1] >> 16) : (x[0][j >> 1] & 0xffffu));
  else
    return __uint_as_float(x[j >> 2][j & 3]);
}

// 16-byte piece q of a page sits in slot q ^ ((q >> 4) & 15) of the LDS page
// image: the K and V pieces that one store instruction fills then lie in
// different banks.  Any slot permutation leaves the page itself unchanged.
__device__ __forceinline__ int img_off(int byte) {
  const int q = byte >> 4;
  return ((q ^ ((q >> 4) & 15)) << 4) | (byte & 15);
}

template <int SRC>
__global__ __launch_bounds__(256) void fp8_group_append_kernel(GroupAppendParams p) {
  constexpr int ES = SRC == PKV_BF16 ? 2 : 4;
  constexpr int NP = SRC == PKV_BF16 ? 1 : 2;   // 16-byte pieces per 8-element chunk
  constexpr int kPage = kBlock * 128;           // bytes of one E4M3 page (d <= 128)
  __shared__ __attribute__((aligned(16))) uint8_t img[2][4 * kPage];   // K, V pages
  __shared__ float red[2][4];
  const int g = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int t0 = g * kScaleGroup;
  const int n = min(kScaleGroup, p.num_tokens - t0);
  const int HD = p.hkv * p.D;
  const int cpt = p.D / kChunk;                 // chunks per row
  const int units = (kScaleGroup / 4) * cpt;    // (4 tokens, 1 chunk) units
  const bool active = tid < units;
  const int u = min(tid, units - 1);
  const int k4 = u / cpt, c = u - k4 * cpt;     // tokens 4 k4 .. +3, dimensions 8 c .. +7
  const int page0 = (p.pos0 + t0) / kBlock;
  int ids[4];
#pragma unroll
  for (int pg = 0; pg < 4; ++pg) ids[pg] = page0 + pg < p.maxb ? p.table_row[page0 + pg] : -1;
  u32x4 kx[4][NP], vx[4][NP];
  float ak = 0.f, av = 0.f;
  // every load is issued (a token past the group's end repeats its last
  // token, which leaves the maxima unchanged)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(4 * k4 + i, n - 1);
    const int64_t o = ((int64_t)(t0 + t) * HD + h * p.D + c * kChunk) * ES;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      kx[i][j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.k_src) + o + 16 * j));
      vx[i][j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(p.v_src) + o + 16 * j));
      ak = reg_absmax<SRC>(kx[i][j], ak);
      av = reg_absmax<SRC>(vx[i][j], av);
    }
  }
  ak = wave_max(ak);
  av = wave_max(av);
  const int w = tid >> 6;
  if ((tid & 63) == 0) { red[0][w] = ak; red[1][w] = av; }
  __syncthreads();
  ak = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  av = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  float sk = __fdiv_rn(ak, 448.0f);
  float sv = __fdiv_rn(av, 448.0f);
  if (!(sk >= 1.17549435e-38f)) sk = 1.0f;
  if (!(sv >= 1.17549435e-38f)) sv = 1.0f;
  if (tid < 4) {
    // every block of the group's 64-token span that the table names
    const int blk = ids[0] * (tid == 0) + ids[1] * (tid == 1) + ids[2] * (tid == 2) +
                    ids[3] * (tid == 3);
    if (blk >= 0 && blk < p.num_blocks) {
      p.k_scale[(int64_t)blk * p.hkv + h] = sk;
      p.v_scale[(int64_t)blk * p.hkv + h] = sv;
    }
  }
  const float inv_k = __frcp_rn(sk), inv_v = __frcp_rn(sv);
  const bool whole = n == kScaleGroup;
  const int pg = k4 >> 2, tp0 = (4 * k4) & (kBlock - 1);   // the quad's page and first slot
  const int qblk = pg == 0 ? ids[0] : pg == 1 ? ids[1] : pg == 2 ? ids[2] : ids[3];
  const bool qok = qblk >= 0 && qblk < p.num_blocks;
  uint8_t* kpg = p.k_pool + (int64_t)qblk * p.block_stride + (int64_t)h * kBlock * p.D;
  uint8_t* vpg = p.v_pool + (int64_t)qblk * p.block_stride + (int64_t)h * p.D * kBlock;
  if (active) {
    uint32_t vw[kChunk] = {};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 kc = {0u, 0u};
#pragma unroll
      for (int j = 0; j < kChunk; j += 2) {
        kc[j >> 2] |= e4m3_encode2(__fmul_rn(elem8<SRC>(kx[i], j), inv_k),
                                   __fmul_rn(elem8<SRC>(kx[i], j + 1), inv_k))
                      << (8 * (j & 3));
        const uint32_t cv = e4m3_encode2(__fmul_rn(elem8<SRC>(vx[i], j), inv_v),
                                         __fmul_rn(elem8<SRC>(vx[i], j + 1), inv_v));
        vw[j] |= (cv & 0xffu) << (8 * i);
        vw[j + 1] |= (cv >> 8) << (8 * i);
      }
      const int ko = frag_k_off<1>(tp0 + i, kChunk * c);
      if (whole) *reinterpret_cast<u32x2*>(&img[0][pg * kPage + img_off(ko)]) = kc;
      else if (qok && 4 * k4 + i < n) *reinterpret_cast<u32x2*>(kpg + ko) = kc;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int vo = frag_v_off<1>(tp0, kChunk * c + j);   // 4 consecutive slots: one word
      if (whole) {
        *reinterpret_cast<uint32_t*>(&img[1][pg * kPage + img_off(vo)]) = vw[j];
      } else if (qok) {
        for (int i = 0; i < 4 && 4 * k4 + i < n; ++i) vpg[vo + i] = (uint8_t)(vw[j] >> (8 * i));
      }
    }
  }
  if (!whole) return;
  __syncthreads();
  // the four pages of K and of V, 16-byte pieces (a page is D pieces)
  for (int e = tid; e < 4 * p.D; e += 256) {
    const int ep = e / p.D, q = e - ep * p.D;
    const int blk = ep == 0 ? ids[0] : ep == 1 ? ids[1] : ep == 2 ? ids[2] : ids[3];
    if (blk < 0 || blk >= p.num_blocks) continue;
    const int64_t base = (int64_t)blk * p.block_stride;
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&img[0][ep * kPage + img_off(16 * q)]),
                                reinterpret_cast<u32x4*>(p.k_pool + base + (int64_t)h * kBlock * p.D + 16 * q));
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&img[1][ep * kPage + img_off(16 * q)]),
                                reinterpret_cast<u32x4*>(p.v_pool + base + (int64_t)h * p.D * kBlock + 16 * q));
  }
}

}  // namespace

hipError_t launch_fp8_group_append(const CacheView& c, float* k_scale, float* v_scale,
                                   const void* k_src, const void* v_src, int src_dtype,
                                   int num_tokens, int pos0, const int32_t* table_row, int maxb,
                                   hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  if (c.head_dim > 128 || c.head_dim % kChunk) return hipErrorInvalidValue;
  GroupAppendParams p{static_cast<uint8_t*>(const_cast<void*>(c.k)),
                      static_cast<uint8_t*>(const_cast<void*>(c.v)), c.block_stride, k_scale,
                      v_scale, c.num_blocks, c.hkv, c.head_dim, k_src, v_src, num_tokens, pos0,
                      table_row, maxb};
  dim3 grid((num_tokens + kScaleGroup - 1) / kScaleGroup, c.hkv), block(256);
  if (src_dtype == PKV_BF16)
    hipLaunchKernelGGL((fp8_group_append_kernel<PKV_BF16>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fp8_group_append_kernel<PKV_F32>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_kv_append(const CacheView& c, void* k_pool, void* v_pool, const void* k_new,
                            const void* v_new, int src_dtype, int num_tokens,
                            const int32_t* seq_idx, const int32_t* pos, const int32_t* tables,
                            int num_seqs, int maxb, hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  AppendParams p{static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), c.block_stride,
                 c.k_scale, c.v_scale, c.num_blocks, c.hkv, c.head_dim, k_new, v_new,
                 num_tokens, seq_idx, pos, tables, num_seqs, maxb};
  if (c.head_dim > 128 || c.head_dim % kChunk) return hipErrorInvalidValue;
  dim3 grid((num_tokens + kGroup - 1) / kGroup, c.hkv), block(256);
  if (c.kv_dtype == PKV_FP8_E4M3) {
    if (src_dtype == PKV_BF16)
      hipLaunchKernelGGL((kv_append_kernel<PKV_BF16, PKV_FP8_E4M3>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((kv_append_kernel<PKV_F32, PKV_FP8_E4M3>), grid, block, 0, s, p);
  } else if (c.kv_dtype == PKV_BF16) {
    hipLaunchKernelGGL((kv_append_kernel<PKV_BF16, PKV_BF16>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((kv_append_kernel<PKV_F32, PKV_F32>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_group_scales(const CacheView& c, float* k_scale, float* v_scale,
                                   const void* k_src, const void* v_src, int src_dtype,
                                   int num_tokens, int pos0, const int32_t* table_row,
                                   int maxb, hipStream_t s) {
  if (num_tokens == 0) return hipSuccess;
  ScaleParams p{k_scale, v_scale, c.hkv, c.head_dim, c.num_blocks, k_src, v_src,
                num_tokens, pos0, table_row, maxb};
  dim3 grid((num_tokens + kScaleGroup - 1) / kScaleGroup, c.hkv), block(256);
  const bool vec = ((reinterpret_cast<uintptr_t>(k_src) | reinterpret_cast<uintptr_t>(v_src)) &
                    15u) == 0 && (c.head_dim == 64 || c.head_dim == 128);
  if (src_dtype == PKV_BF16) {
    if (vec) hipLaunchKernelGGL((fp8_scale_kernel<PKV_BF16, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fp8_scale_kernel<PKV_BF16, false>), grid, block, 0, s, p);
  } else {
    if (vec) hipLaunchKernelGGL((fp8_scale_kernel<PKV_F32, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((fp8_scale_kernel<PKV_F32, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pkv

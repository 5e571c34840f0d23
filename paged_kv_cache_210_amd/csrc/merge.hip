// Exact merge of attention partial states over disjoint key sets.
//
// [P4] "Sequence-parallel engineering for long-context LLM inference ..."
// section "numerically stable incremental softmax": per-shard results are
// combined through a max correction, which is exact when each shard carries its
// own (unnormalised O, max m, sum l): with M = max_s m_s and a_s = exp(m_s - M),
//   L = sum_s a_s l_s,   O = (sum_s a_s O_s) / L,   lse = M + ln L.
// [P1] "Long-context inference engineering truths 2026 ..." section 3.1 keeps
// the same (m, l, O) triple per query row.  Parts with l == 0 (no visible key)
// are skipped, so stale values in them never reach the output.
#include "pkv_common.h"

namespace pkv {
namespace {

constexpr int kMaxD = 256;

// Many parts (long decode splits): one workgroup of 512 threads per row.
// The part weights a_s = exp(m_s - M) (0 for parts with no visible key) go to
// LDS once; then groups of D/VEC threads walk every NG-th part with VEC-wide
// loads of O~, and the groups are summed in LDS.  Parts are taken in chunks
// of kChunk so any S fits.
constexpr int kMergeThreads = 512;
constexpr int kChunk = 2048;

template <int VEC>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int NW = kMergeThreads / 64;
  __shared__ float red[NW];
  __shared__ float wts[kChunk];
  __shared__ float osum[kMergeThreads * VEC];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
  const float* mrow = a.m + row * a.ml_row;
  const float* lrow = a.l + row * a.ml_row;
  const float f = kLog2e;               // m in natural units

  float mx = -INFINITY;
  for (int s = tid; s < a.S; s += kMergeThreads) {
    const float ms = mrow[s * a.ml_part], ls = lrow[s * a.ml_part];
    if (ls > 0.f && ms > -INFINITY) mx = fmaxf(mx, ms);
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[i]);
  __syncthreads();                      // red is reused for L below
  const bool any = M > -INFINITY;

  const int lanes = (a.D + VEC - 1) / VEC;          // threads per group
  const int ng = kMergeThreads / lanes;              // groups
  const int gi = tid / lanes, li = tid - gi * lanes;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  float L = 0.f;
  const float* orow = a.o + row * a.o_row + li * VEC;
  for (int s0 = 0; s0 < a.S; s0 += kChunk) {
    const int n = min(kChunk, a.S - s0);
    for (int i = tid; i < n; i += kMergeThreads) {
      const int s = s0 + i;
      const float ms = mrow[s * a.ml_part], ls = lrow[s * a.ml_part];
      const bool live = any && ls > 0.f && ms > -INFINITY;
      const float ws = live ? __builtin_amdgcn_exp2f((ms - M) * f) : 0.f;
      wts[i] = ws;
      if (live) L += ws * ls;
    }
    __syncthreads();
    if (gi < ng && li * VEC < a.D) {
#pragma unroll 4
      for (int i = gi; i < n; i += ng) {
        const float ws = wts[i];
        if (ws != 0.f) {                // parts with no visible key are skipped
          const float* op = orow + (int64_t)(s0 + i) * a.o_part;
          if constexpr (VEC == 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(op);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += ws * v[e];
          } else {
            acc[0] += ws * op[0];
          }
        }
      }
    }
    __syncthreads();                    // wts is rewritten by the next chunk
  }
  L = wave_sum(L);
  if (lane == 0) red[w] = L;
#pragma unroll
  for (int e = 0; e < VEC; ++e) osum[tid * VEC + e] = acc[e];
  __syncthreads();
  float Lt = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) Lt += red[i];
  const bool empty = !any || !(Lt > 0.f);
  for (int d = tid; d < a.D; d += kMergeThreads) {
    float o = 0.f;
    const int l0 = d / VEC, e = d - l0 * VEC;
    for (int g = 0; g < ng; ++g) o += osum[(g * lanes + l0) * VEC + e];
    o = empty ? 0.f : o / Lt;
    if (a.out_dtype == PKV_BF16)
      reinterpret_cast<uint16_t*>(a.out)[row * a.D + d] = f32_to_bf16_bits(o);
    else
      reinterpret_cast<float*>(a.out)[row * a.D + d] = o;
  }
  if (tid == 0) {
    const float Mn = empty ? -INFINITY : M;
    if (a.out_m) a.out_m[row] = Mn;
    if (a.out_l) a.out_l[row] = empty ? 0.f : Lt;
    if (a.out_lse) a.out_lse[row] = empty ? -INFINITY : Mn + logf(Lt);
  }
}

// A moderate number of parts (a decode split into 17 .. 16 * (512 / (D / 4))
// partitions, e.g. 32 at 128K or 256 at 1M tokens): one workgroup of 512
// threads per row, groups of D/4 threads each owning 4 dimensions; thread
// (group g, lane) takes parts g, g + NG, ... (PPT of them) and issues every
// load of m, l and O~ at once, so the row costs one memory round trip, then
// one block-wide max and one block-wide sum.  Parts past S repeat the last
// part's address and are selected away, as are parts with no visible key.
template <int PPT>
__global__ __launch_bounds__(kMergeThreads) void merge_parts_kernel(MergeArgs a) {
  constexpr int NW = kMergeThreads / 64;
  __shared__ float redm[NW];
  __shared__ float redl[NW];
  __shared__ f32x4 osum[kMergeThreads];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lanes = a.D >> 2;                        // threads per group
  const int ng = kMergeThreads / lanes;              // groups
  const int gi = tid / lanes, li = tid - gi * lanes;
  const float* mrow = a.m + row * a.ml_row;
  const float* lrow = a.l + row * a.ml_row;
  const float* orow = a.o + row * a.o_row + 4 * li;
  const float f = kLog2e;               // m in natural units
  float ms[PPT], ls[PPT];
  f32x4 ov[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int sc = min(gi + ng * k, a.S - 1);
    ms[k] = mrow[sc * a.ml_part];
    ls[k] = lrow[sc * a.ml_part];
    ov[k] = *reinterpret_cast<const f32x4*>(orow + (int64_t)sc * a.o_part);
  }
  bool live[PPT];
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    live[k] = gi + ng * k < a.S && ls[k] > 0.f && ms[k] > -INFINITY;
    if (live[k]) mx = fmaxf(mx, ms[k]);
  }
  mx = wave_max(mx);
  if (lane == 0) redm[w] = mx;
  __syncthreads();
  float M = redm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, redm[i]);
  const bool any = M > -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    if (any && live[k]) {
      const float ws = __builtin_amdgcn_exp2f((ms[k] - M) * f);
      if (li == 0) L += ws * ls[k];                  // each part's l once
      if (ws != 0.f) acc += ws * ov[k];
    }
  }
  L = wave_sum(L);
  if (lane == 0) redl[w] = L;
  osum[tid] = acc;
  __syncthreads();
  float Lt = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) Lt += redl[i];
  const bool empty = !any || !(Lt > 0.f);
  if (tid < lanes) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < ng; ++g) o += osum[g * lanes + tid];
    o = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : o / Lt;
    if (a.out_dtype == PKV_BF16) {
      u32x2 pk;
      pk.x = (uint32_t)f32_to_bf16_bits(o.x) | ((uint32_t)f32_to_bf16_bits(o.y) << 16);
      pk.y = (uint32_t)f32_to_bf16_bits(o.z) | ((uint32_t)f32_to_bf16_bits(o.w) << 16);
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + row * a.D + 4 * tid) = pk;
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + row * a.D + 4 * tid) = o;
    }
  }
  if (tid == 0) {
    const float Mn = empty ? -INFINITY : M;
    if (a.out_m) a.out_m[row] = Mn;
    if (a.out_l) a.out_l[row] = empty ? 0.f : Lt;
    if (a.out_lse) a.out_lse[row] = empty ? -INFINITY : Mn + logf(Lt);
  }
}
constexpr int kMaxPartsPerThread = 16;

// Few parts (prefill shards, short decode splits).  Rows are spread over the
// lanes of a wave, D/4 lanes per row, each lane owning 4 consecutive
// dimensions (16-byte loads); every part's m and l are read per lane (lanes
// of a row read the same address).  Needs D % 4 == 0, D <= 256 and 16-byte
// aligned part rows.
constexpr int kFewParts = 16;

template <int NS>     // number of parts (a.S), compile-time so every load is in flight at once
__global__ __launch_bounds__(256) void merge_rows_kernel(MergeArgs a) {
  const int lanes = a.D >> 2;                            // lanes per row
  const int rpw = 64 / lanes;                            // rows per wave (>= 1)
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int li = lane % lanes;
  const int64_t row = (int64_t)wave * rpw + lane / lanes;
  if (lane >= rpw * lanes || row >= a.rows) return;
  const float* mrow = a.m + row * a.ml_row;
  const float* lrow = a.l + row * a.ml_row;
  const float f = kLog2e;               // m in natural units
  const float* orow = a.o + row * a.o_row + 4 * li;
  // every part's m, l and O~ are loaded at once (all parts' rows exist), so
  // the row costs one memory round trip; parts without keys are selected away
  // afterwards, never multiplied (their O~ may hold anything)
  float ms[NS], ls[NS];
  f32x4 ov[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ms[s] = mrow[s * a.ml_part];
    ls[s] = lrow[s * a.ml_part];
    ov[s] = *reinterpret_cast<const f32x4*>(orow + s * a.o_part);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (ls[s] > 0.f && ms[s] > -INFINITY) M = fmaxf(M, ms[s]);
  const bool any = M > -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (any && ls[s] > 0.f && ms[s] > -INFINITY) {
      const float ws = __builtin_amdgcn_exp2f((ms[s] - M) * f);
      L += ws * ls[s];
      acc += ws * ov[s];
    }
  }
  const bool empty = !any || !(L > 0.f);
  const f32x4 o = empty ? f32x4{0.f, 0.f, 0.f, 0.f} : acc / L;
  if (a.out_dtype == PKV_BF16) {
    u32x2 pk;
    pk.x = (uint32_t)f32_to_bf16_bits(o.x) | ((uint32_t)f32_to_bf16_bits(o.y) << 16);
    pk.y = (uint32_t)f32_to_bf16_bits(o.z) | ((uint32_t)f32_to_bf16_bits(o.w) << 16);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + row * a.D + 4 * li) = pk;
  } else {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + row * a.D + 4 * li) = o;
  }
  if (li == 0) {
    const float Mn = empty ? -INFINITY : M;
    if (a.out_m) a.out_m[row] = Mn;
    if (a.out_l) a.out_l[row] = empty ? 0.f : L;
    if (a.out_lse) a.out_lse[row] = empty ? -INFINITY : Mn + logf(L);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.D > kMaxD || a.rows > 0x7fffffff) return hipErrorInvalidValue;
  // 16-byte loads of O~ need 16-byte aligned part rows (and 4 | D); the
  // output rows then are 8-byte (bf16) or 16-byte (fp32) aligned as well
  const bool vec4 = (a.D % 4) == 0 && (a.o_row % 4) == 0 && (a.o_part % 4) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.o) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.out) & (a.out_dtype == PKV_BF16 ? 7u : 15u)) == 0;
  if (a.S <= kFewParts && vec4 && 64 % (a.D / 4) == 0) {
    const int rpw = 64 / (a.D / 4);
    const int64_t waves = (a.rows + rpw - 1) / rpw;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    switch (a.S) {
#define PKV_MERGE_ROWS(n) \
  case n: hipLaunchKernelGGL(merge_rows_kernel<n>, grid, block, 0, s, a); break;
      PKV_MERGE_ROWS(1) PKV_MERGE_ROWS(2) PKV_MERGE_ROWS(3) PKV_MERGE_ROWS(4)
      PKV_MERGE_ROWS(5) PKV_MERGE_ROWS(6) PKV_MERGE_ROWS(7) PKV_MERGE_ROWS(8)
      PKV_MERGE_ROWS(9) PKV_MERGE_ROWS(10) PKV_MERGE_ROWS(11) PKV_MERGE_ROWS(12)
      PKV_MERGE_ROWS(13) PKV_MERGE_ROWS(14) PKV_MERGE_ROWS(15) PKV_MERGE_ROWS(16)
#undef PKV_MERGE_ROWS
      default: return hipErrorInvalidValue;
    }
  } else if (vec4 && kMergeThreads % (a.D / 4) == 0 &&
             a.S <= kMaxPartsPerThread * (kMergeThreads / (a.D / 4))) {
    const int ng = kMergeThreads / (a.D / 4);
    const int ppt = (a.S + ng - 1) / ng;
    const dim3 grid((unsigned)a.rows), block(kMergeThreads);
    if (ppt <= 2) hipLaunchKernelGGL(merge_parts_kernel<2>, grid, block, 0, s, a);
    else if (ppt <= 4) hipLaunchKernelGGL(merge_parts_kernel<4>, grid, block, 0, s, a);
    else if (ppt <= 8) hipLaunchKernelGGL(merge_parts_kernel<8>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(merge_parts_kernel<16>, grid, block, 0, s, a);
  } else if (vec4) {
    hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)a.rows), dim3(kMergeThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)a.rows), dim3(kMergeThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pkv

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

// Many parts (long decode splits): one workgroup per row.  The max and the
// sum of weights are reduced over all threads; for O~ the workgroup is split
// into groups of D/VEC threads, each group walking every NG-th part with
// VEC-wide loads, and the groups are summed in LDS.
template <int VEC>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  __shared__ float red[2][4];
  __shared__ float osum[256 * VEC];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = tid >> 6;
  const float* mrow = a.m + row * a.ml_row;
  const float* lrow = a.l + row * a.ml_row;
  const float f = kLog2e;               // m in natural units

  float mx = -INFINITY;
  for (int s = tid; s < a.S; s += 256) {
    const float ms = mrow[s * a.ml_part], ls = lrow[s * a.ml_part];
    if (ls > 0.f && ms > -INFINITY) mx = fmaxf(mx, ms);
  }
  mx = wave_max(mx);
  if (lane == 0) red[0][w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));

  float L = 0.f;
  if (M > -INFINITY) {
    for (int s = tid; s < a.S; s += 256) {
      const float ms = mrow[s * a.ml_part], ls = lrow[s * a.ml_part];
      if (ls > 0.f && ms > -INFINITY) L += __builtin_amdgcn_exp2f((ms - M) * f) * ls;
    }
  }
  L = wave_sum(L);
  if (lane == 0) red[1][w] = L;

  const int lanes = (a.D + VEC - 1) / VEC;          // threads per group
  const int ng = 256 / lanes;                        // groups
  const int gi = tid / lanes, li = tid - gi * lanes;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  if (M > -INFINITY && gi < ng && li * VEC < a.D) {
    const float* orow = a.o + row * a.o_row + li * VEC;
#pragma unroll 4
    for (int s = gi; s < a.S; s += ng) {
      const float ms = mrow[s * a.ml_part], ls = lrow[s * a.ml_part];
      if (ls > 0.f && ms > -INFINITY) {
        const float ws = __builtin_amdgcn_exp2f((ms - M) * f);
        const float* op = orow + s * a.o_part;
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
#pragma unroll
  for (int e = 0; e < VEC; ++e) osum[tid * VEC + e] = acc[e];
  __syncthreads();
  const float Lt = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const bool empty = !(M > -INFINITY) || !(Lt > 0.f);
  for (int d = tid; d < a.D; d += 256) {
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

// Few parts (prefill shards, short decode splits): one wave per row, four
// rows per workgroup, lanes over the dims; every part's m and l are read with
// scalar loads and all of a row's O~ loads are issued back to back.
constexpr int kFewParts = 16;

__global__ __launch_bounds__(256) void merge_rows_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.rows) return;
  const float* mrow = a.m + row * a.ml_row;
  const float* lrow = a.l + row * a.ml_row;
  const float f = kLog2e;               // m in natural units
  float ms[kFewParts], ls[kFewParts];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kFewParts; ++s) {
    if (s < a.S) {
      ms[s] = mrow[s * a.ml_part];
      ls[s] = lrow[s * a.ml_part];
      if (ls[s] > 0.f && ms[s] > -INFINITY) M = fmaxf(M, ms[s]);
    }
  }
  const bool any = M > -INFINITY;
  constexpr int kPer = kMaxD / 64;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float L = 0.f;
  const float* orow = a.o + row * a.o_row;
#pragma unroll
  for (int s = 0; s < kFewParts; ++s) {
    if (s < a.S && any && ls[s] > 0.f && ms[s] > -INFINITY) {
      const float ws = __builtin_amdgcn_exp2f((ms[s] - M) * f);
      L += ws * ls[s];
      const float* op = orow + s * a.o_part;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int d = lane + 64 * e;
        if (d < a.D) acc[e] += ws * op[d];
      }
    }
  }
  const bool empty = !any || !(L > 0.f);
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int d = lane + 64 * e;
    if (d >= a.D) continue;
    const float o = empty ? 0.f : acc[e] / L;
    if (a.out_dtype == PKV_BF16)
      reinterpret_cast<uint16_t*>(a.out)[row * a.D + d] = f32_to_bf16_bits(o);
    else
      reinterpret_cast<float*>(a.out)[row * a.D + d] = o;
  }
  if (lane == 0) {
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
  if (a.S <= kFewParts) {
    const int64_t wgs = (a.rows + 3) / 4;
    hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)wgs), dim3(256), 0, s, a);
  } else {
    // VEC-wide loads need 16-byte aligned part rows
    const bool vec4 = (a.D % 4) == 0 && (a.o_row % 4) == 0 && (a.o_part % 4) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.o) & 15u) == 0;
    if (vec4)
      hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)a.rows), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pkv

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

// One workgroup per row; the 4 waves split the parts, lanes split the dims.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  __shared__ float red[2][4];
  __shared__ float osum[4][kMaxD];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* mrow = a.m + row * a.ml_row;
  const float* lrow = a.l + row * a.ml_row;
  // exponent factor: partials in log2 units (decode) or natural units
  const float f = a.m_log2 ? 1.0f : kLog2e;

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

  constexpr int kPer = kMaxD / 64;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  if (M > -INFINITY) {
    const float* orow = a.o + row * a.o_row;
#pragma unroll 4
    for (int s = w; s < a.S; s += 4) {
      const float ms = mrow[s * a.ml_part], ls = lrow[s * a.ml_part];
      if (ls > 0.f && ms > -INFINITY) {
        const float ws = __builtin_amdgcn_exp2f((ms - M) * f);
        const float* op = orow + s * a.o_part;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const int d = lane + 64 * e;
          if (d < a.D) acc[e] += ws * op[d];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int d = lane + 64 * e;
    if (d < a.D) osum[w][d] = acc[e];
  }
  __syncthreads();
  const float Lt = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const bool empty = !(M > -INFINITY) || !(Lt > 0.f);
  for (int d = tid; d < a.D; d += 256) {
    float o = (osum[0][d] + osum[1][d]) + (osum[2][d] + osum[3][d]);
    o = empty ? 0.f : o / Lt;
    if (a.out_dtype == PKV_BF16)
      reinterpret_cast<uint16_t*>(a.out)[row * a.D + d] = f32_to_bf16_bits(o);
    else
      reinterpret_cast<float*>(a.out)[row * a.D + d] = o;
  }
  if (tid == 0) {
    const float Mn = empty ? -INFINITY : (a.m_log2 ? M * kLn2 : M);
    if (a.out_m) a.out_m[row] = Mn;
    if (a.out_l) a.out_l[row] = empty ? 0.f : Lt;
    if (a.out_lse) a.out_lse[row] = empty ? -INFINITY : Mn + logf(Lt);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.D > kMaxD || a.rows > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv

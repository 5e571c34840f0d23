// Internal helpers shared by the libpkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;   // tokens per physical block
constexpr int kScaleGroup = PKV_SCALE_GROUP;
constexpr size_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- element conversions ---------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// OCP E4M3FN encode of an fp32 value: round to nearest, ties to the even
// mantissa; magnitudes at or beyond 448 saturate to 448; NaN gives 0x7F.
// Integer arithmetic only, so host and device agree bit for bit.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                  // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;          // >= 448 (incl. inf)
  if (a < 0x3c800000u) {                              // below 2^-6: subnormal grid
    // steps of 2^-9; the scaling by 2^9 is exact, rintf rounds ties to even.
    const float q = rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)q;                        // q == 8 is the smallest normal
  }
  const uint32_t e = (a >> 23) - 127u + 7u;           // biased E4M3 exponent, 1..15
  const uint32_t keep = (a >> 20) & 0x7u;
  const uint32_t rem = a & 0xfffffu;
  uint32_t code = (e << 3) | keep;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) code += 1u;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// e4m3_encode of two values at once, a in bits 0-7 and b in bits 8-15, on the
// hardware pair convert (OCP E4M3, round to nearest even): the inputs are
// clamped to +-448 first, so that larger magnitudes and infinities saturate,
// and NaN becomes 0x7F afterwards.  The result equals e4m3_encode's for every
// fp32 input (compared over all 2^32 bit patterns on gfx950).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
  const float ca = fminf(fmaxf(a, -448.0f), 448.0f);
  const float cb = fminf(fmaxf(b, -448.0f), 448.0f);
  uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xffffu;
  if (a != a) r = (r & 0xff00u) | 0x7fu;
  if (b != b) r = (r & 0x00ffu) | 0x7f00u;
  return r;
}

// Fragment-order pages (bf16 and E4M3 pools): byte offset of the element of
// token t, dimension d inside one (block, kv head) page of ES-byte elements.
// Lane l = 16*g + i of a decode wave finds all of its matrix-instruction
// fragments in the 16-byte pieces at j*1024 + 16*l (j = 0, 1, ...), so every
// 64-lane load of a page reads 1 KiB of contiguous memory.
//   K: the 8 elements K[t][32c + 8g .. +8] (A operand of the score product
//      for token t = i); a 16-byte piece holds 2/ES of these groups.
//   V: the 4 elements V[4g .. 4g+4][16n + i] (A operand of the PV product for
//      dimension 16n + i); a 16-byte piece holds 4/ES of these groups.
template <int ES>
__host__ __device__ __forceinline__ int frag_k_off(int t, int d) {
  constexpr int CPP = 2 / ES;
  const int c = d >> 5, g = (d >> 3) & 3;
  return (c / CPP) * 1024 + ((g << 4) + t) * 16 + (c % CPP) * 8 * ES + (d & 7) * ES;
}
template <int ES>
__host__ __device__ __forceinline__ int frag_v_off(int t, int d) {
  constexpr int NPP = 4 / ES;
  const int n = d >> 4;
  return (n / NPP) * 1024 + (((t >> 2) << 4) + (d & 15)) * 16 + (n % NPP) * 4 * ES + (t & 3) * ES;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace pkv

// Launchers (defined in the .hip files, called by the C ABI in api.cpp).
namespace pkv {
struct CacheView {
  const void* k;
  const void* v;
  int64_t block_stride;   // elements
  const float* k_scale;
  const float* v_scale;
  int num_blocks;
  int hkv;
  int head_dim;
  int kv_dtype;
};

hipError_t launch_kv_append(const CacheView& c, void* k_pool, void* v_pool, const void* k_new,
                            const void* v_new, int src_dtype, int num_tokens,
                            const int32_t* seq_idx, const int32_t* pos, const int32_t* tables,
                            int num_seqs, int maxb, hipStream_t s);
// launch_fp8_group_scales + launch_kv_append of one sequence's tokens
// [pos0, pos0 + num_tokens) in one pass (each source row read once).
hipError_t launch_fp8_group_append(const CacheView& c, float* k_scale, float* v_scale,
                                   const void* k_src, const void* v_src, int src_dtype,
                                   int num_tokens, int pos0, const int32_t* table_row, int maxb,
                                   hipStream_t s);
hipError_t launch_fp8_group_scales(const CacheView& c, float* k_scale, float* v_scale,
                                   const void* k_src, const void* v_src, int src_dtype,
                                   int num_tokens, int pos0, const int32_t* table_row,
                                   int maxb, hipStream_t s);

struct DecodePlan {
  int partitions;        // P
  int partition_blocks;  // PB
  int head_groups;       // ceil(G / 16) for the MFMA path, 1 otherwise
  bool mfma;
  size_t ws_bytes;
};
DecodePlan plan_decode(int B, int hq, int hkv, int head_dim, int maxb, int partition_blocks,
                       int q_dtype, int kv_dtype);
// k_new / v_new (bf16 [B][hkv][D], or null): the folded append of the
// newest token of every sequence (bf16 MFMA path with one head group only).
hipError_t launch_decode_partial(const CacheView& c, const void* q, int q_dtype, int B, int hq,
                                 const int32_t* tables, int maxb, const int32_t* seq_lens,
                                 float scale, const DecodePlan& plan, float* part_o,
                                 float* part_m, float* part_l, hipStream_t s,
                                 const void* k_new = nullptr, const void* v_new = nullptr);
hipError_t launch_decode(const CacheView& c, const void* q, int q_dtype, int B, int hq,
                         const int32_t* tables, int maxb, const int32_t* seq_lens, float scale,
                         const DecodePlan& plan, void* out, float* out_lse, void* ws,
                         hipStream_t s, const void* k_new = nullptr,
                         const void* v_new = nullptr);

// Device address of this device's copy of the library's static scratch
// (kStaticScratchBytes, 256-byte aligned), looked up once per device.
hipError_t static_scratch(void** out);

hipError_t launch_prefill(const CacheView& c, const void* q, int T, int hq, int q_pos0,
                          const int32_t* table, int maxb, int kv_begin, int kv_end, int causal,
                          float scale, void* out, float* out_lse, float* part_o, float* part_m,
                          float* part_l, hipStream_t s);

// Whole-block copies (copy-on-write, offload): K/V regions of `region` bytes
// per block, block strides in bytes; scales copied when src_ks is set.
struct CopyArgs {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* dst_k;
  uint8_t* dst_v;
  int64_t src_stride, dst_stride;
  int64_t region;
  const float* src_ks;
  const float* src_vs;
  float* dst_ks;
  float* dst_vs;
  int hkv;
  int src_blocks, dst_blocks;
  const int32_t* src_ids;
  const int32_t* dst_ids;
};
// host_pool: one of the pools is in host memory (the copy crosses PCIe).
hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t s, bool host_pool);

// Generic strided merge of S partial states per row.
struct MergeArgs {
  int S;
  int64_t rows;
  int D;
  const float* o;      // O~ of part s, row r at o + r*o_row + s*o_part
  int64_t o_row, o_part;
  const float* m;      // m (natural units) of part s, row r at m + r*ml_row + s*ml_part
  const float* l;
  int64_t ml_row, ml_part;
  void* out;
  int out_dtype;
  float* out_m;
  float* out_l;
  float* out_lse;
};
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
// Merge arguments for partials laid out part-major: O~ [S][rows][D], m/l [S][rows].
MergeArgs partition_merge_args(int S, int64_t rows, int D, const float* part_o,
                               const float* part_m, const float* part_l, void* out,
                               int out_dtype, float* out_lse);

}  // namespace pkv

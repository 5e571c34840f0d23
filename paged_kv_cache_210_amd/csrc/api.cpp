// C ABI of libpkv: host-side argument checks, then kernel launches.
// Nothing is launched when a check fails; device entry points never allocate
// and never synchronise (pkv_validate_tables excepted).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "pkv.h"
#include "pkv_common.h"

namespace {

// Sequences per decode call: the batch is the third grid dimension.
constexpr int32_t kMaxBatch = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int dt) {
  switch (dt) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

int32_t check_cache(const pkv_cache_desc* c) {
  if (!c || !c->k_cache || !c->v_cache) return PKV_ERR_INVALID_ARG;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (c->block_size != PKV_BLOCK_SIZE) return PKV_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  const int es = elem_size(c->kv_dtype);
  if (!es) return PKV_ERR_INVALID_ARG;
  const int64_t min_stride = (int64_t)c->num_kv_heads * PKV_BLOCK_SIZE * c->head_dim;
  if (c->block_stride < min_stride) return PKV_ERR_INVALID_ARG;
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache) || ((c->block_stride * es) & 15))
    return PKV_ERR_INVALID_ARG;
  if (c->kv_dtype == PKV_FP8_E4M3 && (!c->k_scale || !c->v_scale)) return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

pkv::CacheView view(const pkv_cache_desc* c) {
  return pkv::CacheView{c->k_cache, c->v_cache, c->block_stride, c->k_scale, c->v_scale,
                        c->num_blocks, c->num_kv_heads, c->head_dim, c->kv_dtype};
}

int32_t from_hip(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_DEVICE; }

hipStream_t stream_of(void* s) { return static_cast<hipStream_t>(s); }

bool resolve_scale(float scale, int d, float* out) {
  if (!std::isfinite(scale)) return false;
  *out = scale == 0.0f ? 1.0f / std::sqrt((float)d) : scale;
  return true;
}

}  // namespace

extern "C" const char* pkv_status_str(int32_t status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported combination";
    case PKV_ERR_NO_BLOCKS: return "not enough free blocks";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_DEVICE: return "HIP runtime error";
    case PKV_ERR_BAD_TABLE: return "block table entry out of range or aliased";
    case PKV_ERR_SHARED: return "write into a block shared with another sequence";
    case PKV_ERR_TOO_LARGE: return "needs more than the library's static scratch";
    case PKV_ERR_OFFLOADED: return "block is in host memory (page it in first)";
    default: return "unknown status";
  }
}

extern "C" int32_t pkv_kv_append(const pkv_cache_desc* cache, const void* k_new,
                                 const void* v_new, int32_t src_dtype, int32_t num_tokens,
                                 const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* block_tables, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, void* stream) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (num_tokens < 0 || num_seqs <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (cache->kv_dtype == PKV_FP8_E4M3) {
    if (src_dtype != PKV_F32 && src_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  } else if (src_dtype != cache->kv_dtype) {
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !seq_idx || !pos || !block_tables) return PKV_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_kv_append(view(cache), cache->k_cache, cache->v_cache, k_new, v_new,
                                        src_dtype, num_tokens, seq_idx, pos, block_tables,
                                        num_seqs, max_blocks_per_seq, stream_of(stream)));
}

extern "C" int32_t pkv_fp8_group_scales(const pkv_cache_desc* cache, const void* k_src,
                                        const void* v_src, int32_t src_dtype, int32_t num_tokens,
                                        int32_t pos0, const int32_t* table_row, int32_t max_blocks,
                                        void* stream) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (cache->kv_dtype != PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;
  if (src_dtype != PKV_F32 && src_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || pos0 < 0 || (pos0 % PKV_SCALE_GROUP) || max_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!k_src || !v_src || !table_row) return PKV_ERR_INVALID_ARG;
  if ((int64_t)pos0 + num_tokens > (int64_t)max_blocks * PKV_BLOCK_SIZE) return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_fp8_group_scales(view(cache), cache->k_scale, cache->v_scale, k_src,
                                               v_src, src_dtype, num_tokens, pos0, table_row,
                                               max_blocks, stream_of(stream)));
}

extern "C" int32_t pkv_kv_append_fp8_groups(const pkv_cache_desc* cache, const void* k_new,
                                            const void* v_new, int32_t src_dtype,
                                            int32_t num_tokens, int32_t pos0,
                                            const int32_t* table_row, int32_t max_blocks,
                                            void* stream) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (cache->kv_dtype != PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;
  if (src_dtype != PKV_F32 && src_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0 || pos0 < 0 || (pos0 % PKV_SCALE_GROUP) || max_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !table_row || !aligned16(k_new) || !aligned16(v_new))
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)pos0 + num_tokens > (int64_t)max_blocks * PKV_BLOCK_SIZE) return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_fp8_group_append(view(cache), cache->k_scale, cache->v_scale, k_new,
                                               v_new, src_dtype, num_tokens, pos0, table_row,
                                               max_blocks, stream_of(stream)));
}

extern "C" int32_t pkv_decode_workspace_bytes(const pkv_cache_desc* cache, int32_t q_dtype,
                                              int32_t B, int32_t num_q_heads,
                                              int32_t max_blocks_per_seq,
                                              int32_t partition_blocks, size_t* bytes) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (!bytes || B < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || partition_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARG;
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  *bytes = pkv::plan_decode(B, num_q_heads, cache->num_kv_heads, cache->head_dim,
                            max_blocks_per_seq, partition_blocks, q_dtype, cache->kv_dtype)
               .ws_bytes;
  return PKV_OK;
}

namespace {

// Checks shared by pkv_paged_attn_decode and its allocation-free variant;
// fills *sc and *plan.  PKV_OK with B == 0 means there is nothing to launch.
int32_t check_decode(const pkv_cache_desc* cache, const void* q, int32_t q_dtype, int32_t B,
                     int32_t num_q_heads, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale,
                     int32_t partition_blocks, const void* out, float* sc,
                     pkv::DecodePlan* plan) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (B < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || partition_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARG;
  if (cache->kv_dtype == PKV_FP8_E4M3 && q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (!resolve_scale(scale, cache->head_dim, sc)) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (B > kMaxBatch) return PKV_ERR_UNSUPPORTED;
  if (!q || !block_tables || !seq_lens || !out) return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out)) return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE > INT32_MAX) return PKV_ERR_INVALID_ARG;
  *plan = pkv::plan_decode(B, num_q_heads, cache->num_kv_heads, cache->head_dim,
                           max_blocks_per_seq, partition_blocks, q_dtype, cache->kv_dtype);
  return PKV_OK;
}

}  // namespace

extern "C" int32_t pkv_paged_attn_decode(const pkv_cache_desc* cache, const void* q,
                                         int32_t q_dtype, int32_t B, int32_t num_q_heads,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, float scale,
                                         int32_t partition_blocks, void* out, float* out_lse,
                                         void* ws, size_t ws_bytes, void* stream) {
  float sc;
  pkv::DecodePlan plan{};
  const int32_t st = check_decode(cache, q, q_dtype, B, num_q_heads, block_tables,
                                  max_blocks_per_seq, seq_lens, scale, partition_blocks, out,
                                  &sc, &plan);
  if (st != PKV_OK || B == 0) return st;
  if (!ws || ws_bytes < plan.ws_bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return PKV_ERR_WORKSPACE;
  return from_hip(pkv::launch_decode(view(cache), q, q_dtype, B, num_q_heads, block_tables,
                                     max_blocks_per_seq, seq_lens, sc, plan, out, out_lse, ws,
                                     stream_of(stream)));
}

// The same decode with its partials in the library's static scratch (the
// current device's copy): no allocation, no workspace argument.
extern "C" int32_t pkv_paged_attn_decode_noalloc(const pkv_cache_desc* cache, const void* q,
                                                 int32_t q_dtype, int32_t B, int32_t num_q_heads,
                                                 const int32_t* block_tables,
                                                 int32_t max_blocks_per_seq,
                                                 const int32_t* seq_lens, float scale,
                                                 int32_t partition_blocks, void* out,
                                                 float* out_lse, void* stream) {
  float sc;
  pkv::DecodePlan plan{};
  const int32_t st = check_decode(cache, q, q_dtype, B, num_q_heads, block_tables,
                                  max_blocks_per_seq, seq_lens, scale, partition_blocks, out,
                                  &sc, &plan);
  if (st != PKV_OK || B == 0) return st;
  if (plan.ws_bytes > pkv::kStaticScratchBytes) return PKV_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (pkv::static_scratch(&ws) != hipSuccess) return PKV_ERR_DEVICE;
  return from_hip(pkv::launch_decode(view(cache), q, q_dtype, B, num_q_heads, block_tables,
                                     max_blocks_per_seq, seq_lens, sc, plan, out, out_lse, ws,
                                     stream_of(stream)));
}

extern "C" int32_t pkv_decode_partitions(const pkv_cache_desc* cache, int32_t q_dtype,
                                         int32_t B, int32_t num_q_heads,
                                         int32_t max_blocks_per_seq, int32_t partition_blocks,
                                         int32_t* partitions) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (!partitions || B < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
      partition_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARG;
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  *partitions = pkv::plan_decode(B, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                 max_blocks_per_seq, partition_blocks, q_dtype, cache->kv_dtype)
                    .partitions;
  return PKV_OK;
}

extern "C" int32_t pkv_paged_attn_decode_partial(
    const pkv_cache_desc* cache, const void* q, int32_t q_dtype, int32_t B, int32_t num_q_heads,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale,
    int32_t partition_blocks, float* part_o, float* part_m, float* part_l, void* stream) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (B < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || partition_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARG;
  if (cache->kv_dtype == PKV_FP8_E4M3 && q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  float sc;
  if (!resolve_scale(scale, cache->head_dim, &sc)) return PKV_ERR_INVALID_ARG;
  if (B == 0) return PKV_OK;
  if (B > kMaxBatch) return PKV_ERR_UNSUPPORTED;
  if (!q || !block_tables || !seq_lens || !part_o || !part_m || !part_l)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(part_o)) return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE > INT32_MAX) return PKV_ERR_INVALID_ARG;
  pkv::DecodePlan plan = pkv::plan_decode(B, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                          max_blocks_per_seq, partition_blocks, q_dtype,
                                          cache->kv_dtype);
  return from_hip(pkv::launch_decode_partial(view(cache), q, q_dtype, B, num_q_heads,
                                             block_tables, max_blocks_per_seq, seq_lens, sc, plan,
                                             part_o, part_m, part_l, stream_of(stream)));
}

namespace {

// Checks shared by the decode-step entry points; fills *plan.
int32_t check_decode_step(const pkv_cache_desc* cache, const void* k_new, const void* v_new,
                          const void* q, int32_t q_dtype, int32_t B, int32_t num_q_heads,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, float scale, int32_t partition_blocks,
                          float* sc, pkv::DecodePlan* plan) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (B < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || partition_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARG;
  if (q_dtype != PKV_BF16 || (cache->kv_dtype != PKV_BF16 && cache->kv_dtype != PKV_FP8_E4M3))
    return PKV_ERR_UNSUPPORTED;
  if (!resolve_scale(scale, cache->head_dim, sc)) return PKV_ERR_INVALID_ARG;
  if (B > kMaxBatch) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE > INT32_MAX) return PKV_ERR_INVALID_ARG;
  *plan = pkv::plan_decode(B, num_q_heads, cache->num_kv_heads, cache->head_dim,
                           max_blocks_per_seq, partition_blocks, q_dtype, cache->kv_dtype);
  if (!plan->mfma || plan->head_groups != 1) return PKV_ERR_UNSUPPORTED;
  if (B == 0) return PKV_OK;
  if (!q || !block_tables || !seq_lens || !k_new || !v_new) return PKV_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

}  // namespace

extern "C" int32_t pkv_paged_attn_decode_step(const pkv_cache_desc* cache, const void* k_new,
                                              const void* v_new, const void* q, int32_t q_dtype,
                                              int32_t B, int32_t num_q_heads,
                                              const int32_t* block_tables,
                                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                              float scale, int32_t partition_blocks, void* out,
                                              float* out_lse, void* ws, size_t ws_bytes,
                                              void* stream) {
  float sc;
  pkv::DecodePlan plan{};
  const int32_t st = check_decode_step(cache, k_new, v_new, q, q_dtype, B, num_q_heads,
                                       block_tables, max_blocks_per_seq, seq_lens, scale,
                                       partition_blocks, &sc, &plan);
  if (st != PKV_OK || B == 0) return st;
  if (!out || !aligned16(out)) return PKV_ERR_INVALID_ARG;
  if (!ws || ws_bytes < plan.ws_bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return PKV_ERR_WORKSPACE;
  return from_hip(pkv::launch_decode(view(cache), q, q_dtype, B, num_q_heads, block_tables,
                                     max_blocks_per_seq, seq_lens, sc, plan, out, out_lse, ws,
                                     stream_of(stream), k_new, v_new));
}

extern "C" int32_t pkv_paged_attn_decode_step_partial(
    const pkv_cache_desc* cache, const void* k_new, const void* v_new, const void* q,
    int32_t q_dtype, int32_t B, int32_t num_q_heads, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale, int32_t partition_blocks,
    float* part_o, float* part_m, float* part_l, void* stream) {
  float sc;
  pkv::DecodePlan plan{};
  const int32_t st = check_decode_step(cache, k_new, v_new, q, q_dtype, B, num_q_heads,
                                       block_tables, max_blocks_per_seq, seq_lens, scale,
                                       partition_blocks, &sc, &plan);
  if (st != PKV_OK || B == 0) return st;
  if (!part_o || !part_m || !part_l || !aligned16(part_o)) return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_decode_partial(view(cache), q, q_dtype, B, num_q_heads,
                                             block_tables, max_blocks_per_seq, seq_lens, sc, plan,
                                             part_o, part_m, part_l, stream_of(stream), k_new,
                                             v_new));
}

extern "C" int32_t pkv_paged_attn_prefill(const pkv_cache_desc* cache, const void* q,
                                          int32_t q_dtype, int32_t T, int32_t num_q_heads,
                                          int32_t q_pos0, const int32_t* block_table,
                                          int32_t max_blocks, int32_t kv_begin, int32_t kv_end,
                                          int32_t causal, float scale, void* out, float* out_lse,
                                          float* part_o, float* part_m, float* part_l,
                                          void* stream) {
  int32_t st = check_cache(cache);
  if (st != PKV_OK) return st;
  if (q_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (cache->kv_dtype != PKV_BF16 && cache->kv_dtype != PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;
  if (T < 0 || num_q_heads <= 0 || q_pos0 < 0 || max_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARG;
  if (kv_begin < 0 || kv_end < kv_begin || (int64_t)kv_end > (int64_t)max_blocks * PKV_BLOCK_SIZE)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)q_pos0 + T > INT32_MAX) return PKV_ERR_INVALID_ARG;
  const bool final_form = out != nullptr;
  const bool part_form = part_o || part_m || part_l;
  if (final_form == part_form) return PKV_ERR_INVALID_ARG;
  if (part_form && (!part_o || !part_m || !part_l)) return PKV_ERR_INVALID_ARG;
  float sc;
  if (!resolve_scale(scale, cache->head_dim, &sc)) return PKV_ERR_INVALID_ARG;
  if (T == 0) return PKV_OK;
  if (!q || !block_table || !aligned16(q)) return PKV_ERR_INVALID_ARG;
  if ((final_form && !aligned16(out)) || (part_form && !aligned16(part_o)))
    return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_prefill(view(cache), q, T, num_q_heads, q_pos0, block_table,
                                      max_blocks, kv_begin, kv_end, causal != 0, sc, out, out_lse,
                                      part_o, part_m, part_l, stream_of(stream)));
}

extern "C" int32_t pkv_attn_lse_merge(int32_t S, int64_t rows, int32_t head_dim,
                                      const float* part_o, const float* part_m,
                                      const float* part_l, void* out, int32_t out_dtype,
                                      float* out_m, float* out_l, float* out_lse, void* stream) {
  if (S <= 0 || rows < 0 || head_dim <= 0 || head_dim > 256) return PKV_ERR_INVALID_ARG;
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (rows == 0) return PKV_OK;
  if (rows > INT32_MAX) return PKV_ERR_INVALID_ARG;
  if (!part_o || !part_m || !part_l || !out) return PKV_ERR_INVALID_ARG;
  pkv::MergeArgs a{};
  a.S = S;
  a.rows = rows;
  a.D = head_dim;
  a.o = part_o;
  a.o_row = head_dim;
  a.o_part = rows * head_dim;
  a.m = part_m;
  a.l = part_l;
  a.ml_row = 1;
  a.ml_part = rows;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_m = out_m;
  a.out_l = out_l;
  a.out_lse = out_lse;
  return from_hip(pkv::launch_merge(a, stream_of(stream)));
}

// Memory a kernel may address: device memory, or host memory pinned and
// mapped for the device.  Pageable host memory is refused before any launch.
// *host tells whether the memory is on the host side of PCIe.
bool device_addressable(const void* p, bool* host) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();          // do not leave the failed query as a sticky error
    return false;
  }
  *host = at.type == hipMemoryTypeHost;
  return at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeHost ||
         at.type == hipMemoryTypeManaged || at.type == hipMemoryTypeUnified;
}

extern "C" int32_t pkv_copy_blocks(const pkv_cache_desc* src, const pkv_cache_desc* dst,
                                   const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                                   void* stream) {
  int32_t st = check_cache(src);
  if (st != PKV_OK) return st;
  st = check_cache(dst);
  if (st != PKV_OK) return st;
  if (src->kv_dtype != dst->kv_dtype || src->num_kv_heads != dst->num_kv_heads ||
      src->head_dim != dst->head_dim || n < 0)
    return PKV_ERR_INVALID_ARG;
  if (n == 0) return PKV_OK;
  if (!src_ids || !dst_ids) return PKV_ERR_INVALID_ARG;
  const bool f8 = src->kv_dtype == PKV_FP8_E4M3;
  const void* need[] = {src->k_cache, src->v_cache, dst->k_cache, dst->v_cache, src_ids, dst_ids,
                        src->k_scale, src->v_scale, dst->k_scale, dst->v_scale};
  bool host_pool = false;
  for (int i = 0; i < (f8 ? 10 : 6); ++i) {
    bool host = false;
    if (!device_addressable(need[i], &host)) return PKV_ERR_INVALID_ARG;
    if (i < 4) host_pool |= host;
  }
  const int es = elem_size(src->kv_dtype);
  pkv::CopyArgs a{};
  a.src_k = static_cast<const uint8_t*>(src->k_cache);
  a.src_v = static_cast<const uint8_t*>(src->v_cache);
  a.dst_k = static_cast<uint8_t*>(dst->k_cache);
  a.dst_v = static_cast<uint8_t*>(dst->v_cache);
  a.src_stride = src->block_stride * es;
  a.dst_stride = dst->block_stride * es;
  a.region = (int64_t)src->num_kv_heads * PKV_BLOCK_SIZE * src->head_dim * es;
  a.src_ks = f8 ? src->k_scale : nullptr;
  a.src_vs = f8 ? src->v_scale : nullptr;
  a.dst_ks = f8 ? dst->k_scale : nullptr;
  a.dst_vs = f8 ? dst->v_scale : nullptr;
  a.hkv = src->num_kv_heads;
  a.src_blocks = src->num_blocks;
  a.dst_blocks = dst->num_blocks;
  a.src_ids = src_ids;
  a.dst_ids = dst_ids;
  return from_hip(pkv::launch_copy_blocks(a, n, stream_of(stream), host_pool));
}

extern "C" int32_t pkv_validate_tables(const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t B, int32_t max_blocks_per_seq, int32_t num_blocks,
                                       int64_t* first_bad, void* stream) {
  if (!first_bad || B < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  *first_bad = -1;
  if (B == 0) return PKV_OK;
  if (!block_tables || !seq_lens) return PKV_ERR_INVALID_ARG;
  std::vector<int32_t> tab((size_t)B * max_blocks_per_seq), lens(B);
  hipStream_t s = stream_of(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return PKV_ERR_DEVICE;
  if (hipMemcpy(tab.data(), block_tables, tab.size() * sizeof(int32_t), hipMemcpyDeviceToHost) !=
          hipSuccess ||
      hipMemcpy(lens.data(), seq_lens, lens.size() * sizeof(int32_t), hipMemcpyDeviceToHost) !=
          hipSuccess)
    return PKV_ERR_DEVICE;
  // seen[id] = the last sequence whose table covered block id: a block may be
  // named by several sequences (prefix sharing), but only once per table
  std::vector<int32_t> seen(num_blocks, -1);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = lens[b];
    if (n < 0 || n > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE) {
      *first_bad = (int64_t)b * max_blocks_per_seq;
      return PKV_ERR_BAD_TABLE;
    }
    const int64_t nb = (n + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t id = tab[(size_t)b * max_blocks_per_seq + j];
      if (id < 0 || id >= num_blocks || seen[id] == b) {
        *first_bad = (int64_t)b * max_blocks_per_seq + j;
        return PKV_ERR_BAD_TABLE;
      }
      seen[id] = b;
    }
  }
  return PKV_OK;
}

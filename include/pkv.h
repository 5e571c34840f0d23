/*
 * pkv.h - exact softmax attention over a paged KV cache, AMD MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Plain pointers and sizes only; no framework types.
 *
 * Pages this interface follows (cited by title and section):
 *  [P1] "Long-context inference engineering truths 2026: PagedAttention, Ring
 *       Attention and KV-cache offload from 128K to 1M context"
 *       (blog.lonae.com): 2.1 block_size 16 and the waste bound; 2.2 the
 *       block table, append_token and allocate_block; 3.1 online softmax.
 *  [P2] "Unlocking long context: engineering practice and optimisation of
 *       million-token LLM inference" (www.ybb.press/ai-applications/14576):
 *       3.1 block pool + logical block table; 3.2 FP8 (E4M3) KV and
 *       block-wise scaling; 4.1 attention definition and causal flash
 *       attention call; 5.1 prefill is compute-bound, decode is
 *       bandwidth-bound; 5.2 chunked prefill.
 *  [P3] article at www.mhpn.cn/news/2466452: 1.1 softmax(QK^T/sqrt(d))V and
 *       the O(n) per-step decode scan; 1.2 tiling + online softmax keeps the
 *       flops and avoids the n x n matrix; 3.2 GQA.
 *  [P4] "Sequence-parallel engineering for long-context LLM inference: Ring
 *       Attention and distributed KV cache" (www.ybb.press/ai-applications/
 *       14023): "numerically stable incremental softmax" (merge of per-shard
 *       results by a max / log-sum-exp correction).
 *
 * Conventions
 *  - Ownership: the caller owns every buffer.  Device entry points never
 *    allocate device memory; split-KV decode takes a caller workspace sized by
 *    pkv_decode_workspace_bytes (pkv_paged_attn_decode_noalloc uses a fixed
 *    static device array of the library instead).  Only allocator objects are
 *    created by the library (host memory).
 *  - Asynchrony: device entry points enqueue work on `stream` (a hipStream_t
 *    passed as void*, NULL = the null stream) and return without waiting.
 *    pkv_validate_tables is the one exception (it copies to the host).
 *  - Errors: every function returns an int32 status, PKV_OK (0) or a negative
 *    code.  Arguments are checked on the host first; when a check fails
 *    nothing is launched.  pkv_status_str() names a code.
 *  - Table contents are the caller's contract: the entries a sequence length
 *    covers must be valid physical ids, distinct within that sequence's table.
 *    Tables of different sequences may name the same blocks (prefix sharing,
 *    [P2 3.1]): attention only reads them, and writes into shared blocks are
 *    the allocator's copy-on-write business (PKV_ERR_SHARED).  Kernels never
 *    dereference an id outside [0, num_blocks): the tokens such a page would
 *    hold are skipped (decode) or masked out of the softmax (prefill), and the
 *    row's result is then that of the remaining keys, which the caller should
 *    treat as unspecified; pkv_validate_tables reports such entries.
 *  - Reentrancy: functions are reentrant; an allocator object is not
 *    thread-safe.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad shape        */
  PKV_ERR_UNSUPPORTED = -2,  /* valid but not implemented combination       */
  PKV_ERR_NO_BLOCKS = -3,    /* allocator has too few free blocks            */
  PKV_ERR_WORKSPACE = -4,    /* workspace missing or too small               */
  PKV_ERR_DEVICE = -5,       /* a HIP runtime call failed                    */
  PKV_ERR_BAD_TABLE = -6,    /* pkv_validate_tables found a bad entry        */
  PKV_ERR_SHARED = -7,       /* a write would land in a block another table
                                holds (use pkv_allocator_reserve_cow)        */
  PKV_ERR_TOO_LARGE = -8,    /* the call needs more than the library's static
                                scratch (PKV_STATIC_SCRATCH_BYTES)           */
  PKV_ERR_OFFLOADED = -9     /* the block is in host memory (page it in first) */
};

/* ---- element types ----------------------------------------------------- */
enum {
  PKV_F32 = 0,       /* IEEE binary32                                          */
  PKV_BF16 = 1,      /* bfloat16 (upper half of binary32), round-to-nearest-even */
  PKV_FP8_E4M3 = 2   /* OCP E4M3FN: bias 7, max 448, 0x7F/0xFF NaN, no inf      */
};

#define PKV_BLOCK_SIZE 16   /* tokens per physical block [P1 2.1, P2 3.1] */
#define PKV_SCALE_GROUP 64  /* tokens per FP8 scale [P2 3.2]              */
#define PKV_STATIC_SCRATCH_BYTES (16u << 20)  /* per-device scratch of
                                                pkv_paged_attn_decode_noalloc */

/* ---- paged KV cache of one attention layer [P1 2.2, P2 3.1] -------------
 * Physical block b, kv head h: the K page starts at
 *   k_cache + b*block_stride + h*16*head_dim elements,
 * and the V page at
 *   v_cache + b*block_stride + h*head_dim*16 elements.
 * Each page holds the 16 tokens x head_dim elements of that (block, head).
 * block_stride >= num_kv_heads*16*head_dim, counted in elements of kv_dtype,
 * lets K and V share one interleaved allocation.  Pools must be 16-byte
 * aligned and block_stride*elem_size a multiple of 16.
 * Order of the elements inside a page:
 *   PKV_F32: K [16 tokens][head_dim], V [head_dim][16 tokens].
 *   PKV_BF16, PKV_FP8_E4M3 ("fragment order"): the order in which the decode
 *   kernel's matrix instructions consume them, so that each 64-lane load
 *   reads 1 KiB of contiguous memory.  With e = element bytes (2 or 1),
 *   byte offsets of token t, dimension d are
 *     K: (c/(2/e))*1024 + ((g<<4) + t)*16 + (c%(2/e))*8*e + (d&7)*e,
 *        c = d>>5, g = (d>>3)&3;
 *     V: (n/(4/e))*1024 + (((t>>2)<<4) + (d&15))*16 + (n%(4/e))*4*e + (t&3)*e,
 *        n = d>>4.
 * pkv_kv_append writes these orders; callers treat pages as opaque.
 * E4M3 caches carry fp32 scales k_scale/v_scale [num_blocks][num_kv_heads]:
 * element value = decode(code) * scale of its (block, head); otherwise NULL. */
typedef struct pkv_cache_desc {
  void* k_cache;
  void* v_cache;
  int64_t block_stride;
  float* k_scale;
  float* v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;   /* must be PKV_BLOCK_SIZE */
  int32_t head_dim;     /* 64 or 128              */
  int32_t kv_dtype;     /* PKV_F32 | PKV_BF16 | PKV_FP8_E4M3 */
} pkv_cache_desc;

const char* pkv_status_str(int32_t status);

/* ---- host block allocator [P1 2.1-2.2] ------------------------------------
 * A free list of physical block ids.  Blocks leave from the front of the free
 * order; released blocks return to the back, in table order.  A sequence's
 * table grows by one block exactly when a token opens a new logical block
 * (token t needs logical block t/16), so a sequence of n tokens owns
 * ceil(n/16) blocks and wastes 16*ceil(n/16) - n <= 15 slots. */
typedef struct pkv_allocator pkv_allocator;

/* free_order: host array of num_blocks distinct ids in [0, num_blocks)
 * (a permutation), or NULL for 0..num_blocks-1.  *out receives the object. */
int32_t pkv_allocator_create(int32_t num_blocks, const int32_t* free_order,
                             pkv_allocator** out);
/* Grow sequence `seq` (>= 0) to new_len tokens.  All-or-nothing: if fewer free
 * blocks remain than needed, returns PKV_ERR_NO_BLOCKS and changes nothing.
 * A sequence never shrinks (new_len below its length: PKV_ERR_INVALID_ARG).
 * If table_row is not NULL the sequence's full table (up to max_blocks
 * entries, host int32) is copied there and *num_blocks_out (nullable) gets
 * its length; a table longer than max_blocks is PKV_ERR_INVALID_ARG (state is
 * then unchanged). */
int32_t pkv_allocator_reserve(pkv_allocator* a, int32_t seq, int64_t new_len,
                              int32_t* table_row, int32_t max_blocks,
                              int32_t* num_blocks_out);
/* Forget the sequence; each of its blocks is released, and returns to the
 * back of the free list (in table order) when no other table holds it. */
int32_t pkv_allocator_release(pkv_allocator* a, int32_t seq);
/* Unused slots in seq's last block (0 for an unknown sequence). */
int32_t pkv_allocator_waste_slots(const pkv_allocator* a, int32_t seq, int64_t* out);
int32_t pkv_allocator_free_count(const pkv_allocator* a, int32_t* out);
void pkv_allocator_destroy(pkv_allocator* a);

/* ---- prefix sharing [P2 3.1 copy-on-write; P1 5 prefix cache] -------------
 * Every block counts the tables that hold it (pkv_allocator_refcount; 0 for a
 * free block).  pkv_allocator_reserve refuses (PKV_ERR_SHARED, nothing
 * changed) a growth that would write into a partly filled last block that
 * another table also holds; pkv_allocator_reserve_cow then first moves this
 * sequence onto a fresh block (taken from the free list before the growth's
 * own blocks; all-or-nothing as well) and reports the pair: *cow_src = the
 * shared block, *cow_dst = the fresh one, whose contents the caller copies
 * with pkv_copy_blocks before appending (-1, -1 when no copy is needed).
 * Kernels read shared blocks like any other: tables may alias blocks that
 * are only read. */
int32_t pkv_allocator_reserve_cow(pkv_allocator* a, int32_t seq, int64_t new_len,
                                  int32_t* table_row, int32_t max_blocks,
                                  int32_t* num_blocks_out, int32_t* cow_src, int32_t* cow_dst);
/* New sequence dst_seq (must not exist) holding every block of src_seq (which
 * must exist), with its length. */
int32_t pkv_allocator_fork(pkv_allocator* a, int32_t src_seq, int32_t dst_seq);
/* Publish seq's first n_full blocks (all full: n_full*16 <= its length) under
 * block_hashes[j], a caller-computed hash of tokens [0, 16(j+1)) of the prompt
 * (chained, so equal hashes mean equal prefixes).  A hash or block already
 * published keeps its first entry.  A block leaves the index when it is
 * freed. */
int32_t pkv_allocator_publish_prefix(pkv_allocator* a, int32_t seq, const uint64_t* block_hashes,
                                     int32_t n_full);
/* For a sequence that does not exist yet (or holds nothing): take the longest
 * run block_hashes[0..] of published blocks, in order; the sequence then holds
 * them and has length 16 * *matched (its prefill starts at that token). */
int32_t pkv_allocator_match_prefix(pkv_allocator* a, int32_t seq, const uint64_t* block_hashes,
                                   int32_t n, int32_t* matched);
int32_t pkv_allocator_refcount(const pkv_allocator* a, int32_t block, int32_t* out);

/* ---- KV offload: a host tier of the page table [P3 4.2, 4.3; P1 4] ---------
 * The allocator's page table records, for every logical block of a sequence,
 * where it lives (a device block id, or PKV_OFFLOADED in the table and a slot
 * of a pinned host pool that the caller owns), and the last step that read it.
 * Offloading and paging in only update that table and return the copy pairs;
 * the caller moves the data with pkv_copy_blocks (device pool <-> host pool of
 * the same format), on a stream of its choice, so a page-in (the prefetch)
 * can run beside the attention of other blocks.  Ordering is the caller's:
 * a page-in must finish before an attention reads the block, and an offload's
 * copy must be ordered before anything writes the device block it frees
 * (that block returns to the free list at once).  Kernels treat PKV_OFFLOADED
 * entries like any id outside the pool (see the table contract above), so
 * blocks must be resident when read.  Which blocks to move is the caller's
 * policy; pkv_allocator_coldest lists the least recently read ones. */
#define PKV_OFFLOADED (-2)   /* table entry of a block held in a host slot */

/* Give the allocator num_host_slots host slots (ids 0 .. num_host_slots-1 of
 * the caller's host pool); once per allocator. */
int32_t pkv_allocator_set_host_slots(pkv_allocator* a, int32_t num_host_slots);
/* Move the resident blocks among logical blocks [first_block, first_block +
 * count) of seq (clamped to its table) to host slots: pair i copies device
 * block dev_ids[i] to host slot host_slots[i] (arrays of at least count
 * entries), *n_pairs pairs in block order; blocks already offloaded are
 * skipped.  All-or-nothing: PKV_ERR_SHARED if one of them is held by another
 * table too, PKV_ERR_NO_BLOCKS if too few host slots are free. */
int32_t pkv_allocator_offload(pkv_allocator* a, int32_t seq, int32_t first_block, int32_t count,
                              int32_t* dev_ids, int32_t* host_slots, int32_t* n_pairs);
/* Bring the offloaded blocks among [first_block, first_block + count) of seq
 * back: each takes a free device block (from the front of the free list);
 * pair i copies host slot host_slots[i] to device block dev_ids[i].  The host
 * slots return to the back of the host free list.  All-or-nothing:
 * PKV_ERR_NO_BLOCKS if too few device blocks are free. */
int32_t pkv_allocator_page_in(pkv_allocator* a, int32_t seq, int32_t first_block, int32_t count,
                              int32_t* host_slots, int32_t* dev_ids, int32_t* n_pairs);
/* Record that step `step` read blocks [first_block, first_block + count). */
int32_t pkv_allocator_touch(pkv_allocator* a, int32_t seq, int32_t first_block, int32_t count,
                            int64_t step);
/* Page-table entry of logical block `block` of seq: device id (PKV_OFFLOADED
 * when in host memory), host slot (-1 when resident), last step that read it
 * (-1 if none). */
int32_t pkv_allocator_block_state(const pkv_allocator* a, int32_t seq, int32_t block,
                                  int32_t* device_id, int32_t* host_slot, int64_t* last_access);
/* The sequence's table as the kernels take it (device ids, PKV_OFFLOADED for
 * host blocks), up to max_blocks entries (more: PKV_ERR_INVALID_ARG). */
int32_t pkv_allocator_table(const pkv_allocator* a, int32_t seq, int32_t* table_row,
                            int32_t max_blocks, int32_t* num_blocks_out);
int32_t pkv_allocator_host_free_count(const pkv_allocator* a, int32_t* out);
/* Up to max_n offload candidates, least recently read first (ties: sequence,
 * then block, ascending): resident full blocks held by one table only. */
int32_t pkv_allocator_coldest(const pkv_allocator* a, int32_t max_n, int32_t* seqs,
                              int32_t* blocks, int32_t* n);
/* Growth that writes into an offloaded last block returns PKV_ERR_OFFLOADED;
 * fork of a sequence with offloaded blocks returns PKV_ERR_OFFLOADED (host
 * slots are not shared); publish_prefix skips offloaded blocks; release
 * returns a sequence's host slots. */

/* ---- kv_append: write new tokens into pool slots [P1 2.2] ----------------
 * For token i < num_tokens: block = block_tables[seq_idx[i]*max_blocks_per_seq
 * + pos[i]/16], slot = pos[i]%16; K page row `slot` <- k_new[i][h][:] and V
 * page column `slot` <- v_new[i][h][:] for every kv head h.
 * k_new, v_new: device [num_tokens][num_kv_heads][head_dim], src_dtype,
 * 16-byte aligned.
 * seq_idx, pos: device int32 [num_tokens]; block_tables: device int32
 * [num_seqs][max_blocks_per_seq].
 * Same-type caches copy bits (src_dtype must equal kv_dtype).  E4M3 caches
 * take PKV_F32 or PKV_BF16 sources and store E4M3(f32(x) * f32(1/scale)) with
 * the scale of the destination (block, head), rounding to nearest-even and
 * saturating at +-448; the scales must already be set (pkv_fp8_group_scales).
 * Tokens whose seq_idx is outside [0, num_seqs), whose pos is negative or
 * beyond the table, or whose block id is outside [0, num_blocks) are skipped.
 * Two tokens naming the same slot race (one of them wins). */
int32_t pkv_kv_append(const pkv_cache_desc* cache, const void* k_new, const void* v_new,
                      int32_t src_dtype, int32_t num_tokens, const int32_t* seq_idx,
                      const int32_t* pos, const int32_t* block_tables, int32_t num_seqs,
                      int32_t max_blocks_per_seq, void* stream);

/* ---- FP8 block-wise scales [P2 3.2] ----------------------------------------
 * For one sequence's tokens [pos0, pos0 + num_tokens) with pos0 % 64 == 0:
 * every 64-token group (aligned to token 0; the last may be partial) and kv
 * head gets scale = f32(amax / 448), amax = largest |x| over the group's
 * given tokens and head_dim (1.0 when that quotient is 0 or subnormal),
 * separately for K (from k_src) and V (from v_src).  The scale is stored into
 * k_scale/v_scale[block][head] of every block of the group's 64-token span
 * that table_row names (entries past max_blocks or outside [0, num_blocks)
 * are skipped), so scales move with blocks.  k_src, v_src: device
 * [num_tokens][num_kv_heads][head_dim] of src_dtype (PKV_F32 | PKV_BF16);
 * table_row: device int32 [max_blocks] covering the tokens. Requires an E4M3
 * cache.
 * Policy: a group's scale is fixed by the tokens given when it is computed;
 * tokens appended to the group later are encoded with it and saturate at
 * +-448 * scale when larger (pkv_kv_append, the folded decode step).  A
 * decode stream computes a group's scale from the token that opens it (pos0
 * = that position, num_tokens = 1), and, when a later token of the group
 * opens another block, calls again with that same first token, which writes
 * the same scale into the newly named block.  A prompt computes its scales
 * from whole groups before appending them. */
int32_t pkv_fp8_group_scales(const pkv_cache_desc* cache, const void* k_src, const void* v_src,
                             int32_t src_dtype, int32_t num_tokens, int32_t pos0,
                             const int32_t* table_row, int32_t max_blocks, void* stream);

/* ---- FP8 group scales and append in one pass [P2 3.2, P1 2.2] -------------
 * pkv_fp8_group_scales over one sequence's tokens [pos0, pos0 + num_tokens)
 * followed by pkv_kv_append of the same tokens (token i at position pos0 + i
 * of the sequence whose table is table_row), reading each source row once:
 * the pool and the scales end bit for bit as after the two calls.  Arguments
 * and requirements as pkv_fp8_group_scales (E4M3 cache, pos0 % 64 == 0, bf16
 * or f32 sources [num_tokens][num_kv_heads][head_dim], 16-byte aligned);
 * tokens whose block id is outside the pool are skipped, as by
 * pkv_kv_append.  The append of a prompt chunk into an E4M3 pool. */
int32_t pkv_kv_append_fp8_groups(const pkv_cache_desc* cache, const void* k_new,
                                 const void* v_new, int32_t src_dtype, int32_t num_tokens,
                                 int32_t pos0, const int32_t* table_row, int32_t max_blocks,
                                 void* stream);

/* ---- split-KV decode [P2 5.1, P3 1.1, P1 3.1, P4 incremental softmax] ----
 * One query per sequence b (the newest token, already appended) attends to
 * every key t < seq_lens[b] of that sequence:
 *   O[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) V_t,
 * K_t, V_t read from kv head h / (num_q_heads / num_kv_heads) [P3 3.2] through
 * the block table.  The sequence's blocks are cut into partitions of
 * partition_blocks blocks (0 = chosen by the library); each partition yields a
 * partial (unnormalised O, max, sum) in the workspace and a second kernel
 * merges them exactly by log-sum-exp.
 * q: device [B][num_q_heads][head_dim], q_dtype (PKV_F32 | PKV_BF16);
 * out: device [B][num_q_heads][head_dim] in q_dtype; out_lse: device fp32
 * [B][num_q_heads] (natural log of the softmax denominator incl. max) or NULL;
 * seq_lens: device int32 [B]; seq_lens[b] == 0 gives O = 0 and lse = -inf.
 * B <= 65535 (larger batches: PKV_ERR_UNSUPPORTED; split the call).
 * scale == 0 means 1/sqrt(head_dim).  Requires num_q_heads % num_kv_heads == 0.
 * E4M3 caches need q_dtype PKV_BF16.  ws: device buffer of at least
 * pkv_decode_workspace_bytes(cache, q_dtype, B, num_q_heads,
 * max_blocks_per_seq, partition_blocks) bytes, 256-byte aligned, holding
 * the fp32 partials only; it needs no initialisation and may be reused by
 * the next call once this one has finished on the stream.  Calls that
 * overlap on one workspace race. */
int32_t pkv_decode_workspace_bytes(const pkv_cache_desc* cache, int32_t q_dtype, int32_t B,
                                   int32_t num_q_heads, int32_t max_blocks_per_seq,
                                   int32_t partition_blocks, size_t* bytes);
int32_t pkv_paged_attn_decode(const pkv_cache_desc* cache, const void* q, int32_t q_dtype,
                              int32_t B, int32_t num_q_heads, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens, float scale,
                              int32_t partition_blocks, void* out, float* out_lse, void* ws,
                              size_t ws_bytes, void* stream);

/* ---- split-KV decode that allocates nothing ---------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that forbid hipMalloc, harnesses that forbid it):
 * pkv_paged_attn_decode with the same arguments, results and kernels, minus
 * the workspace.  The partials live in a static device array of
 * PKV_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call uses the copy of the current device (the
 * stream must belong to it).  A call whose workspace
 * (pkv_decode_workspace_bytes) exceeds that size returns PKV_ERR_TOO_LARGE
 * and launches nothing.  No allocation of any kind is made.  The scratch needs
 * no initialisation (every partial is written before it is read) and keeps
 * the last call's contents; calls that overlap on one GPU (several streams or
 * host threads) share it and race, so they must be ordered by the caller. */
int32_t pkv_paged_attn_decode_noalloc(const pkv_cache_desc* cache, const void* q,
                                      int32_t q_dtype, int32_t B, int32_t num_q_heads,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, float scale,
                                      int32_t partition_blocks, void* out, float* out_lse,
                                      void* stream);

/* ---- split-KV decode, partial form [P4 incremental softmax] -------------------
 * The attention of pkv_paged_attn_decode stopped before the merge, for callers
 * that merge partitions themselves (e.g. partitions held by several devices).
 * Partition p covers logical blocks [p*PB, (p+1)*PB) of every sequence, PB =
 * partition_blocks (0 = the library's choice); the partition count P comes
 * from pkv_decode_partitions with the same arguments.  Outputs, part-major so
 * pkv_attn_lse_merge(S = P, rows = B*num_q_heads, ...) merges them directly:
 *   part_o fp32 [P][B][num_q_heads][head_dim] unnormalised O~,
 *   part_m fp32 [P][B][num_q_heads] max score (natural units, -inf if the
 *          partition holds no key of the sequence), part_l fp32 sum of
 *          exp(score - m) (0 then). */
int32_t pkv_decode_partitions(const pkv_cache_desc* cache, int32_t q_dtype, int32_t B,
                              int32_t num_q_heads, int32_t max_blocks_per_seq,
                              int32_t partition_blocks, int32_t* partitions);
int32_t pkv_paged_attn_decode_partial(const pkv_cache_desc* cache, const void* q, int32_t q_dtype,
                                      int32_t B, int32_t num_q_heads,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* seq_lens, float scale,
                                      int32_t partition_blocks, float* part_o, float* part_m,
                                      float* part_l, void* stream);

/* ---- decode step with the append folded in [P1 2.2, P2 5.1] ----------------
 * pkv_kv_append of one token per sequence followed by pkv_paged_attn_decode
 * (or its partial form), in the launches of the decode alone: token
 * seq_lens[b] - 1 of sequence b takes k_new[b][h][:] and v_new[b][h][:]
 * (device bf16 [B][num_kv_heads][head_dim], 16-byte aligned), which the
 * kernel uses directly and writes into its pool slot, so seq_lens already
 * count the new token.  The pool ends bit for bit as after pkv_kv_append, and
 * the outputs equal those of the two calls.  Sequences with seq_lens[b] == 0
 * (or beyond the table) append nothing; a block id outside the pool skips the
 * token (as pkv_kv_append does).  bf16 q; bf16 or E4M3 cache (E4M3: the
 * token is encoded with its block's scale, which must already be set, as for
 * pkv_kv_append); at most 16 query heads per kv head (otherwise
 * PKV_ERR_UNSUPPORTED: make the two calls).
 * Other arguments, workspace and outputs as pkv_paged_attn_decode /
 * pkv_paged_attn_decode_partial. */
int32_t pkv_paged_attn_decode_step(const pkv_cache_desc* cache, const void* k_new,
                                   const void* v_new, const void* q, int32_t q_dtype, int32_t B,
                                   int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   float scale, int32_t partition_blocks, void* out,
                                   float* out_lse, void* ws, size_t ws_bytes, void* stream);
int32_t pkv_paged_attn_decode_step_partial(const pkv_cache_desc* cache, const void* k_new,
                                           const void* v_new, const void* q, int32_t q_dtype,
                                           int32_t B, int32_t num_q_heads,
                                           const int32_t* block_tables,
                                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                           float scale, int32_t partition_blocks, float* part_o,
                                           float* part_m, float* part_l, void* stream);

/* ---- chunked causal prefill against paged KV [P2 4.1, P2 5.2, P3 1.2] ----
 * Query rows q[r] (r < T) of one sequence sit at absolute positions q_pos0+r.
 * Row r attends to keys t with kv_begin <= t < kv_end and, when causal, t <=
 * q_pos0 + r, read through block_table (device int32 [max_blocks], covering
 * kv_end).  q: device [T][num_q_heads][head_dim] bf16; a bf16 or E4M3 cache
 * with head_dim 64 or 128 (otherwise PKV_ERR_UNSUPPORTED).
 * bf16 pages: scores use q and K exactly (bf16 products, fp32 sums); V enters
 * the P V product converted to fp16 with round-toward-zero.  That is exact
 * for every bf16 value with 2^-14 <= |v| <= 65504 (fp16's normal range);
 * larger magnitudes saturate to +-65504, and smaller ones are truncated toward
 * zero to a multiple of 2^-24 (fp16 subnormals; below 2^-24 they become 0),
 * an absolute change below 6e-8.  So for V outside that range the result is
 * the attention over the converted V (pkv_paged_attn_decode uses V exactly).
 * E4M3 pages [P2
 * 3.2]: K is read as its exact codes with each page's K scale applied to the
 * scores in fp32; V is dequantised to fp16 as it is read (f16(code * scale),
 * one rounding); q is converted bf16 -> fp16 and both products run in fp16,
 * so q and the dequantised V must stay within fp16's range (|x| <= 65504;
 * beyond it q saturates and V overflows).  Scales must be positive.
 * Exactly one output form:
 *  - final:   out (device bf16 [T][num_q_heads][head_dim]) = normalised O,
 *             out_lse (nullable, fp32 [T][num_q_heads]);
 *  - partial: part_o (fp32 [T][num_q_heads][head_dim], unnormalised),
 *             part_m (fp32 [T][num_q_heads], max score in natural units),
 *             part_l (fp32 [T][num_q_heads], sum of exp(score - max)),
 *             for combining KV shards with pkv_attn_lse_merge.
 * A row with no visible key gets O = 0, m = -inf, l = 0 (lse = -inf). */
int32_t pkv_paged_attn_prefill(const pkv_cache_desc* cache, const void* q, int32_t q_dtype,
                               int32_t T, int32_t num_q_heads, int32_t q_pos0,
                               const int32_t* block_table, int32_t max_blocks,
                               int32_t kv_begin, int32_t kv_end, int32_t causal, float scale,
                               void* out, float* out_lse, float* part_o, float* part_m,
                               float* part_l, void* stream);

/* ---- exact merge of KV-shard partials [P4 incremental softmax, P1 3.1] ---
 * S partial states over disjoint key sets, part_o fp32 [S][rows][head_dim],
 * part_m / part_l fp32 [S][rows] (as written by prefill's partial form):
 *   M = max_s m_s,  a_s = exp(m_s - M),  L = sum_s a_s l_s,
 *   O = sum_s a_s O_s / L.
 * Parts with l == 0 or m == -inf contribute nothing; if all do, O = 0,
 * M = -inf, L = 0.  out: device [rows][head_dim] of out_dtype (PKV_F32 |
 * PKV_BF16); out_m, out_l (nullable, fp32 [rows]) receive (M, L) so merges
 * compose; out_lse (nullable, fp32 [rows]) receives M + ln L. */
int32_t pkv_attn_lse_merge(int32_t S, int64_t rows, int32_t head_dim, const float* part_o,
                           const float* part_m, const float* part_l, void* out,
                           int32_t out_dtype, float* out_m, float* out_l, float* out_lse,
                           void* stream);

/* ---- whole-block copies: copy-on-write and offload [P2 3.1; P1 4] --------
 * For i < n: every kv head's K and V page of block src_ids[i] of pool `src` is
 * copied bit for bit to block dst_ids[i] of pool `dst`, with its K and V
 * scales for E4M3 pools.  src and dst have the same kv_dtype, num_kv_heads and
 * head_dim (block_stride may differ; they may be one pool).  Either pool may
 * be device memory or pinned host memory that the device can address
 * (hipHostMalloc): device -> host moves blocks out of HBM (offload), host ->
 * device brings them back, device -> device serves copy-on-write.
 * src_ids, dst_ids: int32 [n] in memory the device can read.  A pair with an
 * id outside its pool is skipped.  Destinations must be distinct and must not
 * be sources of the same call (such copies race). */
int32_t pkv_copy_blocks(const pkv_cache_desc* src, const pkv_cache_desc* dst,
                        const int32_t* src_ids, const int32_t* dst_ids, int32_t n, void* stream);

/* ---- table check (debug) ---------------------------------------------------
 * Copies block_tables / seq_lens (device) to the host after synchronising
 * `stream`, and checks that every entry covered by seq_lens[b] (the first
 * ceil(seq_lens[b]/16)) is in [0, num_blocks) and that no physical block is
 * covered twice by one sequence (different sequences may share blocks: prefix
 * sharing).  *first_bad (host) gets -1 when all is well, else the flat
 * index b*max_blocks_per_seq + j of the first bad entry (status
 * PKV_ERR_BAD_TABLE); a seq_len below 0 or beyond max_blocks_per_seq*16 is
 * reported at index b*max_blocks_per_seq. */
int32_t pkv_validate_tables(const int32_t* block_tables, const int32_t* seq_lens, int32_t B,
                            int32_t max_blocks_per_seq, int32_t num_blocks, int64_t* first_bad,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

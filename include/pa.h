/*
 * pa.h — C ABI of the MI355X (gfx950) paged KV-cache library.
 *
 * What the library implements, from the PagedAttention pages:
 *   - a KV cache stored as a pool of fixed-size physical blocks (16 tokens by
 *     default), each sequence seeing its tokens as consecutive logical blocks
 *     mapped to physical blocks through a block table, with no contiguity
 *     needed (page 1, jisaku.com glossary "PagedAttention", section
 *     「PagedAttentionの解決策」; page 3, abeam.tech paper review, section
 *     「用語解説」);
 *   - a block manager that takes one new block each time 16 tokens fill up,
 *     returns a finished sequence's blocks to the pool, shares blocks between
 *     forked sequences by reference count and copies a shared block only when
 *     a write must land in it (page 2, hubblespacetelescope blog, section
 *     「OSの知恵をGPUへ…」; page 3, sections 「KV キャッシュマネージャ」 and
 *     「並列サンプリングやビームサーチでの共有」);
 *   - the attention kernel that follows the block table to read a sequence's
 *     keys and values in logical order, giving the same result as attention
 *     over a contiguous cache (page 3, sections
 *     「モデル構造ではなくサービング基盤の変更」 and 「よくある質問」).
 *
 * Conventions shared by every device call
 * ---------------------------------------
 * All pointers to device data are device pointers owned by the caller; the
 * library never allocates device memory.  Device calls are asynchronous on the
 * HIP stream passed as `stream` (a hipStream_t; NULL = the default stream) and
 * return after the launch.  Scalar arguments are validated on the host: on a
 * bad value the call returns an error, sets pa_last_error() and launches
 * nothing.  Data-dependent preconditions (slot numbers, table entries, copy
 * pairs) cannot be checked on the host; kernels check them and never access
 * memory outside the pools: an out-of-range slot or copy pair is skipped, and a
 * sequence whose table entry is out of range, or whose length exceeds
 * max_context_len or max_blocks_per_seq*block_size, gets NaN outputs.
 *
 * Pool layout (block_size = bs = 16, x = 16 / element_bytes: 4 for fp32,
 * 8 for fp16/bf16; Hkv = num_kv_heads, D = head_dim):
 *   K pool: [num_blocks][Hkv][D/x][bs][x]   element (b,h,t,d) at
 *           (((b*Hkv + h)*(D/x) + d/x)*bs + t)*x + d%x
 *   V pool: [num_blocks][Hkv][bs/x][D][x]   element (b,h,t,d) at
 *           (((b*Hkv + h)*(bs/x) + t/x)*D + d)*x + t%x
 *           (one 16-byte load gives x consecutive tokens of one dim)
 * A token at logical position p of a sequence lives in physical block
 * table[p / bs] at in-block offset t = p % bs; its slot number is
 * table[p / bs]*bs + p % bs.
 *
 * Activations: q [num_seqs][Hq][D] in the KV dtype; out [num_seqs][Hq][D]
 * float32; new tokens [num_tokens][Hkv][D] in the KV dtype; block tables int32
 * [num_seqs][max_blocks_per_seq]; context lengths int32 [num_seqs].
 * Grouped-query attention: G = Hq / Hkv, query head h reads KV head h / G.
 *
 * Thread safety: the block manager is single-owner (not thread-safe); device
 * calls are reentrant.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,   /* bad scalar argument or null pointer              */
  PA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. head_dim 96)     */
  PA_ERR_OUT_OF_BLOCKS = 3, /* block manager: not enough free blocks; no change */
  PA_ERR_UNKNOWN_SEQ = 4,   /* block manager: sequence id not present           */
  PA_ERR_SEQ_EXISTS = 5,    /* block manager: sequence id already present       */
  PA_ERR_HIP = 6,           /* HIP runtime error while launching                */
  PA_ERR_WORKSPACE = 7      /* decode workspace missing or too small            */
} pa_status;

/* Element dtypes.  PA_FP8_E4M3 and PA_INT8 are the 8-bit codes of a
 * quantized cache (one byte per element; value = code * the pool's scale):
 *   PA_FP8_E4M3: OCP 8-bit float E4M3 (sign, 4 exponent bits with bias 7,
 *     3 mantissa bits; 0x7F/0xFF are NaN; no infinity; largest finite 448);
 *   PA_INT8: two's-complement integer.
 * Page 1 (jisaku.com glossary, section 「他のKVキャッシュ最適化との組み合わせ」)
 * pairs paging with an INT8 cache, half the size per block; E4M3 is the
 * 8-bit float the target GPU converts natively. */
typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3,
  PA_INT8 = 4
} pa_dtype;

/* Message for the last error on the calling thread ("" if none). */
const char* pa_last_error(void);
/* Library version string. */
const char* pa_version(void);

/* ------------------------------------------------------------------------
 * Host block manager (pure CPU).
 *
 * Free list: a LIFO stack; a fresh manager hands blocks out in free_order
 * (a permutation of [0, num_blocks); NULL = ascending).  Released blocks
 * (count reaching zero, in table order) go on top.  A write to position p of a
 * sequence takes a new block when p % block_size == 0; otherwise it lands in
 * the existing block table[p / block_size], which is first copied if its
 * reference count is above one (the copy is reported as a (src, dst) pair and
 * the sequence's table entry is changed to dst; the last remaining holder
 * writes in place).  Every call either succeeds completely or changes nothing.
 * ---------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

typedef struct pa_bm_stats_t {
  int32_t num_blocks;    /* pool size                                        */
  int32_t free_blocks;   /* blocks on the free list                          */
  int32_t used_blocks;   /* blocks with reference count > 0                  */
  int32_t shared_blocks; /* blocks with reference count > 1                  */
  int32_t num_seqs;      /* live sequences                                   */
  int32_t reserved;
  int64_t tokens;        /* sum of sequence lengths                          */
  int64_t slack_slots;   /* sum over sequences of blocks*block_size - length */
} pa_bm_stats_t;

/* Creates a manager for num_blocks blocks of block_size tokens: the pool of
 * same-size physical blocks reserved up front, which the manager hands out
 * to sequences (page 3, abeam.tech review, section 「KV キャッシュマネージャ」;
 * block_size as a parameter, 16 by default: page 1, jisaku.com glossary,
 * section 「PagedAttentionの解決策」).  free_order (host, [num_blocks]) is
 * copied; NULL = ascending.  *out receives the handle.  PA_ERR_INVALID_ARG
 * for num_blocks <= 0, block_size <= 0, or a free_order that is not a
 * permutation of [0, num_blocks); nothing is allocated then. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_bm** out);
void pa_bm_destroy(pa_bm* bm);

/* New sequence with num_tokens tokens: ceil(num_tokens / block_size) blocks
 * are taken from the free list, their ids become the sequence's block table
 * (logical block k -> physical block table[k], page 1, jisaku.com glossary,
 * section 「PagedAttentionの解決策」; page 3, abeam.tech review, section
 * 「用語解説」, ブロックテーブル).  Slot of position p: table[p / block_size]
 * * block_size + p % block_size, written to slots_out (host, [num_tokens],
 * may be NULL).  PA_ERR_SEQ_EXISTS for a live id, PA_ERR_OUT_OF_BLOCKS when
 * the free list is too short, PA_ERR_INVALID_ARG for num_tokens < 0; no
 * change then. */
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id, int32_t num_tokens, int64_t* slots_out);

/* child shares every block of parent: it gets a copy of parent's block
 * table, every block's reference count goes up by one, and no block is
 * taken or copied (page 2, hubblespacetelescope blog, section
 * 「OSの知恵をGPUへ…」, third bullet: sharing by reference count, no memory
 * copy; page 3, abeam.tech review, section 「並列サンプリングやビームサーチでの共有」).
 * PA_ERR_UNKNOWN_SEQ for an unknown parent, PA_ERR_SEQ_EXISTS for a live
 * child id; no change then. */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);

/* Reserves the next num_tokens positions of one sequence (a prompt chunk, or
 * several generated tokens): tokens fill the last block, and a new block is
 * taken each time a position starts one (page 2, hubblespacetelescope blog,
 * section 「OSの知恵をGPUへ…」, first bullet; page 3, abeam.tech review,
 * section 「KV キャッシュマネージャ」).  A shared last block that would be
 * written is first copied (copy-on-write, page 3, section 「用語解説」).
 * slots_out (host, [num_tokens], may be NULL); cow_pairs_out (host, [1][2]
 * at most, may be NULL only if no copy can arise) receives (src, dst) block
 * pairs to copy before writing; *num_cow_out their count (0 or 1).
 * PA_ERR_UNKNOWN_SEQ / PA_ERR_OUT_OF_BLOCKS: no change. */
pa_status pa_bm_extend(pa_bm* bm, int64_t seq_id, int32_t num_tokens, int64_t* slots_out,
                       int32_t* cow_pairs_out, int32_t* num_cow_out);

/* Decode-step reservation: one more position for each of n distinct
 * sequences, in the order given (page 3, abeam.tech review, section
 * 「KV キャッシュマネージャ」: generated tokens go into the last block, and a
 * full block is followed by a newly taken one, with the table updated).
 * Position p = the sequence's length before the call: a new block when
 * p % block_size == 0; otherwise block table[p / block_size], copied first
 * when its reference count is above one (the writer copies, the last holder
 * writes in place: page 3, section 「並列サンプリングやビームサーチでの共有」;
 * page 2, hubblespacetelescope blog, section 「OSの知恵をGPUへ…」, third
 * bullet).  slots_out (host, [n]) receives each position's slot;
 * cow_pairs_out (host, [n][2]) the (src, dst) block pairs the caller copies
 * (pa_copy_blocks) before the writes; *num_cow_out = number of pairs.
 * All-or-nothing: the blocks the whole batch needs (new tail blocks plus
 * copies) are counted first, and PA_ERR_OUT_OF_BLOCKS leaves the manager
 * unchanged; PA_ERR_UNKNOWN_SEQ or PA_ERR_INVALID_ARG (a repeated id) too. */
pa_status pa_bm_append_slots(pa_bm* bm, const int64_t* seq_ids, int32_t n, int64_t* slots_out,
                             int32_t* cow_pairs_out, int32_t* num_cow_out);

/* One decode step's host work in one call: pa_bm_append_slots for the n
 * sequences, then pa_bm_block_tables of the same sequences after the
 * reservation (page 3, abeam.tech review, section 「KV キャッシュマネージャ」:
 * the manager hands the kernel its block tables).  Outputs (host):
 * slots_out [n], cow_pairs_out [n][2] and *num_cow_out as for
 * pa_bm_append_slots; tables_out [n][max_blocks] (padded with -1) and
 * lens_out [n] as for pa_bm_block_tables; *blocks_needed_out = the longest
 * table after the reservation.  When that exceeds max_blocks the call
 * returns PA_ERR_INVALID_ARG with *blocks_needed_out set and changes
 * nothing, so the caller can grow its buffers and call again; the other
 * errors are those of pa_bm_append_slots, also with no change. */
pa_status pa_bm_step(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                     int64_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out,
                     int32_t* tables_out, int32_t* lens_out, int32_t* blocks_needed_out);

/* Releases a finished sequence: each of its blocks' reference counts drops
 * by one, and blocks reaching zero return to the free list, in table order
 * (page 3, abeam.tech review, section 「KV キャッシュマネージャ」: at the end
 * of a request only its blocks are handed back).  PA_ERR_UNKNOWN_SEQ: no
 * change.  The caller orders reuse of a freed block after the last kernel
 * that reads it (same stream). */
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id);

/* Beam search / parallel sampling step (page 3, abeam.tech review, section
 * 「並列サンプリングやビームサーチでの共有」: beams share blocks; a shared block
 * is copied on write).  Sequence new_ids[j] continues old_ids[parents[j]]:
 * the same id keeps that sequence, another id becomes a fork of it (shared
 * blocks, no copy); then every old id not among new_ids is released.  Forks
 * come before releases, so blocks of a dropped parent live on in its
 * children.  The next write into a shared last block is copied by
 * pa_bm_append_slots as usual.  All-or-nothing: PA_ERR_UNKNOWN_SEQ for an
 * unknown old id, PA_ERR_INVALID_ARG for a repeated old or new id or a parent
 * index outside [0, num_old), PA_ERR_SEQ_EXISTS for a new id that is live
 * and not its own parent; nothing changes then.  Host arrays:
 * old_ids [num_old], new_ids and parents [num_new]. */
pa_status pa_bm_reorder(pa_bm* bm, const int64_t* old_ids, int32_t num_old,
                        const int64_t* new_ids, const int32_t* parents, int32_t num_new);

/* Sliding window: drops the blocks of a sequence whose block_size slots all
 * lie before position first_pos (clamped to the sequence's length), i.e.
 * logical blocks k with (k+1)*block_size <= min(first_pos, len).  Their
 * table entries become -1 (placeholders: position p still maps to entry
 * p / block_size, and pa_bm_block_tables exports the -1s); counts -1, blocks
 * reaching zero return to the pool in table order.  Entries already dropped
 * are skipped.  *released_out (may be NULL) = entries dropped by this call.
 * For attention over the last W positions, call it with first_pos = L - W
 * once the step's length L is reserved; the windowed decode calls never read
 * the dropped entries (page 1, jisaku.com glossary, section
 * 「他のKVキャッシュ最適化との組み合わせ」: blocks that left the window are
 * freed).  The caller orders reuse of a freed block after the last kernel
 * that read it, as for pa_bm_free_seq (same stream). */
pa_status pa_bm_release_before(pa_bm* bm, int64_t seq_id, int32_t first_pos,
                               int32_t* released_out);

/* Block tables of n sequences into tables_out (host, [n][max_blocks], padded
 * with -1) and lengths into lens_out (host, [n], may be NULL): the logical ->
 * physical map the attention kernels walk (page 3, abeam.tech review,
 * section 「用語解説」, ブロックテーブル: the kernel reads the KV it needs
 * by following the table).  PA_ERR_INVALID_ARG when a table is longer than
 * max_blocks; PA_ERR_UNKNOWN_SEQ for an unknown id; outputs unspecified
 * then. */
pa_status pa_bm_block_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* Length (tokens) of a live sequence; PA_ERR_UNKNOWN_SEQ otherwise. */
pa_status pa_bm_seq_len(const pa_bm* bm, int64_t seq_id, int32_t* len_out);
/* Reference count of a block: the number of block tables that hold it (page
 * 2, hubblespacetelescope blog, section 「OSの知恵をGPUへ…」, third bullet:
 * shared blocks are tracked by reference count); 0 for a free block.
 * PA_ERR_INVALID_ARG for an id outside [0, num_blocks). */
pa_status pa_bm_refcount(const pa_bm* bm, int32_t block_id, int32_t* count_out);
/* Pool occupancy (pa_bm_stats_t above).  slack_slots is the paging waste:
 * unused slots in the sequences' blocks, at most block_size - 1 per sequence
 * (page 2, hubblespacetelescope blog, section 「OSの知恵をGPUへ…」, second
 * bullet); num_blocks and the counts mirror the block accounting a serving
 * engine reports at start-up (page 1, jisaku.com glossary, section
 * 「vLLMのメモリ管理確認」). */
pa_status pa_bm_stats(const pa_bm* bm, pa_bm_stats_t* out);

/* ------------------------------------------------------------------------
 * Device operations.
 * ---------------------------------------------------------------------- */

/* Writes token i's K and V (all heads, bit for bit, no conversion) into slot
 * slot_mapping[i] of the pools (page 3, section 「KV キャッシュマネージャ」:
 * generated tokens go into the sequence's last block).
 *   k_new, v_new: device [num_tokens][Hkv][D] in the pool dtype (for the
 *   8-bit dtypes: codes, moved as bytes); slot_mapping: device int64
 *   [num_tokens], -1 = skip; slots outside [0, num_blocks*block_size) skipped.
 * Supported: block_size 16, head_dim a multiple of 16 in [16, 256]. */
pa_status pa_cache_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          pa_dtype dtype, void* stream);

/* pa_cache_append for a quantized cache: k_new/v_new ([num_tokens][Hkv][D],
 * device, in src_dtype: PA_F32, PA_F16 or PA_BF16) are encoded into the
 * codes of cache_dtype (PA_FP8_E4M3 or PA_INT8) with one scale per pool
 * (K element = code * k_scale, V element = code * v_scale):
 *   y = fp32(x * r), r = 1/scale rounded to fp32 (computed on the host);
 *   PA_INT8: code = y rounded half to even, clamped to [-127, 127];
 *   PA_FP8_E4M3: code = y clamped to [-448, 448], rounded to the nearest
 *     E4M3 value, ties to the even code; the sign is kept (-0 -> 0x80).
 * Scale granularity and rounding are not fixed by page 1 (jisaku.com
 * glossary, section 「他のKVキャッシュ最適化との組み合わせ」); these are the
 * library's.  Inputs must be finite.  Scales must be positive and finite
 * (PA_ERR_INVALID_ARG otherwise).  Slots as for pa_cache_append. */
pa_status pa_cache_append_quant(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, int32_t num_tokens,
                                int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, pa_dtype cache_dtype, pa_dtype src_dtype,
                                float k_scale, float v_scale, void* stream);

/* Copy-on-write: for each pair (src, dst) of block_pairs (device int32
 * [num_pairs][2]), block dst := block src in both pools, all heads, bit for
 * bit (page 3, section 「用語解説」, Copy-on-Write).  Pairs run concurrently: no
 * dst may equal another pair's src or dst.  Out-of-range pairs are skipped. */
pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, pa_dtype dtype, void* stream);

/* pa_copy_blocks over the pools of several layers in one launch: for each
 * layer l < num_layers and pair (src, dst), block dst := block src in
 * k_pools[l] and v_pools[l] (device arrays of num_layers pool pointers, each
 * pool laid out as for pa_copy_blocks with the same num_blocks, heads,
 * head_dim and dtype).  A model with one cache per layer copies a step's
 * copy-on-write pairs in every layer (page 3, section
 * 「並列サンプリングやビームサーチでの共有」).  Pairs and layers run
 * concurrently: no dst may equal another pair's src or dst.  Out-of-range
 * pairs are skipped; every pool must be 16-byte aligned (not checked: the
 * pointers are on the device). */
pa_status pa_copy_blocks_layers(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                                const int32_t* block_pairs, int32_t num_pairs,
                                int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, pa_dtype dtype, void* stream);

/* Kernel family of the fp16/bf16 decode calls, process wide:
 * PA_KERNEL_AUTO (the default) runs them on the matrix cores,
 * PA_KERNEL_GENERIC on the plain-FMA kernel (fixed partitions of 256
 * tokens by default), so that both can be checked against each other.  The
 * choice also sizes the workspace (pa_decode_workspace_bytes) and the
 * partition size (pa_decode_partition_size): change it only between calls,
 * with no decode call in flight that was sized under the other choice.
 * Returns the previous choice; an unknown value sets PA_ERR_INVALID_ARG in
 * pa_last_error() and changes nothing. */
typedef enum pa_decode_kernel {
  PA_KERNEL_AUTO = 0,
  PA_KERNEL_GENERIC = 1
} pa_decode_kernel;
pa_decode_kernel pa_set_decode_kernel(pa_decode_kernel kernel);

/* How pa_decode splits contexts for these arguments; partition_size is
 *   > 0 (a multiple of 16): fixed partitions of that many tokens;
 *   0: the library's choice: the even split on the matrix-core path
 *      (fp16/bf16 and the 8-bit dtypes); fixed partitions of 256 tokens for
 *      fp32 and for the plain-FMA kernel;
 *   -1: the even split (matrix-core path only; fp32 and the plain-FMA kernel
 *       use 256-token partitions).
 * The even split counts the batch's work in 32 bits: it needs
 *   num_seqs * num_kv_heads * (12 + 8 * ceil(ceil(max_context_len / 16) / 4))
 * below 2^30.  Beyond that, 0 gives 256-token partitions and -1 is refused
 * (this returns -1, pa_decode_workspace_bytes 0, and the decode calls
 * PA_ERR_UNSUPPORTED).
 * Returns the partition size in tokens for fixed partitions, 0 for the even
 * split, -1 for invalid arguments.
 *   Fixed partitions: partition p of a sequence covers tokens
 *     [p*P, (p+1)*P); each is attended by one wave, merged when more than one.
 *   Even split: the batch's work, as (sequence, KV head, run of 4 blocks)
 *     units, is cut into equal contiguous chunks, one per wave of a grid of
 *     4 waves per compute unit; a (sequence, head) cut into several chunks
 *     is merged the same way. */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size, pa_dtype dtype);

/* Device workspace bytes pa_decode needs for these arguments (0 when every
 * sequence fits in one partition).  Returns 0 for invalid arguments.  The
 * workspace holds the partials of split contexts; its contents need no
 * initialisation and it can be reused call after call. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size, pa_dtype dtype);

/* Decode attention over a paged cache (page 3, abeam.tech review, section
 * 「モデル構造ではなくサービング基盤の変更」: the kernel follows the block table
 * to read K/V in logical order, and the result is ordinary attention:
 * section 「よくある質問」; page 4, pro-knowledge-base FAQ).  The attention
 * formula itself is not on the pages: scaled dot-product attention of one
 * query per sequence.  For each sequence b (length L = context_lens[b]) and
 * query head h,
 *   out[b][h] = softmax_t(scale * q[b][h] . K_b[t]) weighted sum of V_b[t],
 * t in [0, L), where K_b/V_b are KV head h/G of the tokens reached through
 * block_tables[b] in logical order; accumulation in fp32.  L = 0 gives zeros.
 * The context is split (fixed partitions, or an even split of the batch's
 * work; see pa_decode_partition_size) and the partial (max, sum, weighted V)
 * of the pieces are merged with a log-sum-exp reduction.
 *   out: device float [num_seqs][Hq][D].
 *   workspace: device, at least pa_decode_workspace_bytes(...) bytes,
 *   exclusively owned by this call until it completes on `stream`.
 *   max_context_len: upper bound of context_lens (sizes the launch).
 *   q, the pools (and k_new/v_new of the step calls) must be 16-byte aligned,
 *   the workspace 256-byte aligned (PA_ERR_INVALID_ARG otherwise).
 * Supported: block_size 16; head_dim 64 or 128; Hq a multiple of Hkv with
 * G = Hq/Hkv <= 16.  fp16/bf16 run on the matrix cores, fp32 on plain FMAs;
 * pa_set_decode_kernel(PA_KERNEL_GENERIC) makes fp16/bf16 use the plain-FMA
 * kernel too.  8-bit pools are attended by pa_decode_quant
 * (PA_ERR_INVALID_ARG here).  Errors: PA_ERR_UNSUPPORTED for block_size,
 * head_dim or G outside the supported set; PA_ERR_INVALID_ARG for other bad
 * scalars, NULL or misaligned pointers; PA_ERR_WORKSPACE for a missing or
 * short workspace; PA_ERR_HIP for a failed launch.  Nothing is launched on
 * an error. */
pa_status pa_decode(float* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_context_len, float scale, int32_t partition_size,
                    pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* The two phases of pa_decode, same arguments and preconditions:
 *   pa_decode_partial: the partition kernel.  Sequences that fit in one
 *     partition get their final out rows; longer ones leave per-partition
 *     partials (running max, running sum, weighted V sum) in the workspace.
 *   pa_decode_merge: the log-sum-exp merge of those partials into out (with
 *     the even split it also writes the rows of empty sequences; with fixed
 *     partitions nothing is launched when every sequence fits in one).
 * pa_decode(...) == pa_decode_partial(...) then pa_decode_merge(...) on the
 * same stream.  Separately, they let a caller time the partition pass or
 * combine partials produced elsewhere (e.g. a context split across devices). */
pa_status pa_decode_partial(float* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream);
pa_status pa_decode_merge(float* out, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                          int32_t partition_size, pa_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/* One decode step: appends each sequence's new token and attends, with the
 * result of pa_cache_append(k_pool, v_pool, k_new, v_new, slot_mapping,
 * num_seqs, ...) followed by pa_decode(...).  Row b of k_new/v_new
 * ([num_seqs][Hkv][D], KV dtype) is sequence b's token at position
 * context_lens[b] - 1, and slot_mapping[b] (device int64) is the slot of
 * that position in block_tables[b], or -1 to skip the write (position
 * context_lens[b] - 1 is then attended with the pool's current content).  A
 * slot elsewhere in the pool gets the token written there, but then out is
 * only defined when that slot is not attended by the step.  On the
 * matrix-core path (fp16/bf16 and the 8-bit dtypes) the append is done
 * inside the attention kernel, one launch fewer; there a sequence whose
 * length fails the bounds checks (NaN out rows) or is 0 gets no pool write.  Otherwise the two kernels run back to
 * back.  Copy-on-write copies of the step must be issued (pa_copy_blocks)
 * before this call on the same stream.
 *   pa_decode_step_partial / pa_decode_step_merge: the two phases of
 *     pa_decode_step (same arguments and workspace, on the same stream):
 *     pa_decode_step(...) == pa_decode_step_partial(...) then
 *     pa_decode_step_merge(...).  When the merge phase launches a kernel
 *     (even split, or sequences longer than one fixed partition) that kernel
 *     writes the new tokens to their slots and the attention kernel only
 *     attends them; otherwise the attention kernel writes them. */
pa_status pa_decode_step(float* out, const void* q, void* k_pool, void* v_pool,
                         const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         const int32_t* block_tables, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                         int32_t partition_size, pa_dtype dtype, void* workspace,
                         size_t workspace_bytes, void* stream);
pa_status pa_decode_step_partial(float* out, const void* q, void* k_pool, void* v_pool,
                                 const void* k_new, const void* v_new,
                                 const int64_t* slot_mapping, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, int32_t partition_size, pa_dtype dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_decode_step_merge(float* out, const void* q, void* k_pool, void* v_pool,
                               const void* k_new, const void* v_new,
                               const int64_t* slot_mapping, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               int32_t partition_size, pa_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/* pa_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and result as pa_decode_step without the workspace: the
 * partials of split contexts go to a fixed device array inside the library
 * (64 MiB, `static __device__`; each device holds its own copy from the
 * library's load until the process ends; its address is looked up on the
 * first call on each device, with that device current).  The call itself
 * allocates nothing and needs no initialised memory.  The current device must
 * be the one `stream` runs on.  Sizes whose partials exceed the array
 * (pa_decode_workspace_bytes(...) > 64 MiB, e.g. 16 contexts of 131072
 * tokens on the even split) return PA_ERR_WORKSPACE before any device call;
 * use pa_decode_step with a workspace for those.  Every call on one device
 * shares that device's array, which keeps the last call's contents: calls
 * that overlap on one device (different streams or threads without ordering)
 * race and give wrong rows; calls on one stream are ordered. */
pa_status pa_decode_step_noalloc(float* out, const void* q, void* k_pool, void* v_pool,
                                 const void* k_new, const void* v_new,
                                 const int64_t* slot_mapping, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                 float scale, int32_t partition_size, pa_dtype dtype,
                                 void* stream);

/* Shared-prefix plan of a decode batch (host): sequences whose block tables
 * begin with the same physical blocks hold the same tokens there (blocks are
 * shared by forks, e.g. the samples of one prompt: page 2,
 * hubblespacetelescope blog, section 「OSの知恵をGPUへ…」, third bullet;
 * page 3, abeam.tech review, section 「並列サンプリングやビームサーチでの共有」),
 * so their queries can attend those blocks together, reading each once.
 * Sequences are grouped by their first physical block, in batch order; a
 * group's shared prefix is the longest run of table entries common to all
 * its members, capped so that each member keeps at least its last position
 * after it; groups of one member or with fewer than min_shared_blocks
 * shared blocks are dropped.  Inputs (host): tables [n][max_blocks] and
 * lens [n] as exported by pa_bm_block_tables for the step (after its
 * reservation).  Outputs (host): prefix_len_out [n] = tokens of the
 * sequence's shared prefix (a multiple of block_size, 0 = none);
 * group_rows_out [n] = the grouped members' batch indices, group g being
 * group_rows_out[group_start_out[g] .. group_start_out[g+1]-1];
 * group_start_out [n+1]; *num_groups_out; *max_group_out = the largest
 * group.  PA_ERR_INVALID_ARG for bad sizes or NULL pointers. */
pa_status pa_shared_prefix_plan(const int32_t* tables, const int32_t* lens, int32_t n,
                                int32_t max_blocks, int32_t block_size,
                                int32_t min_shared_blocks, int32_t* prefix_len_out,
                                int32_t* group_rows_out, int32_t* group_start_out,
                                int32_t* num_groups_out, int32_t* max_group_out);

/* Workspace bytes of pa_decode_step_shared (0 for invalid arguments). */
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len, pa_dtype dtype);

/* pa_decode_step where groups of sequences share a prefix of blocks (a
 * plan from pa_shared_prefix_plan, on the device): the result of
 * pa_decode_step, with each shared block read once per KV head instead of
 * once per sequence (page 2, hubblespacetelescope blog, section
 * 「OSの知恵をGPUへ…」, third bullet: shared blocks are held once by
 * reference count; page 3, abeam.tech review, section
 * 「並列サンプリングやビームサーチでの共有」).  Three passes:
 *   1. per group and KV head, the members' queries (members x query heads
 *      of that KV head) attend the shared prefix [0, prefix_len) through
 *      the first member's table, on the matrix cores, possibly cut into a
 *      few key ranges; each range's unnormalised rows and their softmax
 *      maxima and sums go to the workspace.  This pass runs on a stream the
 *      library keeps per device (default priority), after the work already
 *      queued on `stream` (an event) and beside pass 2; the merge on
 *      `stream` waits for it (another event), so the call is ordered on
 *      `stream` like any other;
 *   2. the even split attends each sequence from its prefix_len (0 for
 *      sequences in no group) to its end, with the step's new tokens fused
 *      in as in pa_decode_step;
 *   3. the log-sum-exp merge folds the prefix rows with the rest.
 *   prefix_len: device int32 [num_seqs], a multiple of 16 below
 *   context_lens[b] for members, 0 otherwise; group_rows: device int32
 *   [num_rows] batch indices; group_start: device int32 [num_groups + 1],
 *   non-decreasing from 0 to num_rows; all members of a group have the same
 *   prefix_len and the same table entries before it (the plan guarantees
 *   it).  These are checked on the device: a sequence with a nonzero
 *   prefix_len gets a NaN row when that length is not a multiple of 16
 *   below its context length, when it is in no group, when its prefix_len
 *   or prefix blocks differ from its group's first member's, or when that
 *   member's length or table is out of bounds.  max_group_size: the largest
 *   group.  workspace: at least pa_decode_shared_workspace_bytes(...)
 *   bytes, 256-byte aligned; needs no initialisation; calls that share it
 *   must not overlap.  The prefix pass stamps each row it writes with a
 *   per-call number and the merge clears the stamps it reads, so rows left
 *   from an earlier call, or an earlier replay of a captured call (whose
 *   number is fixed at capture), are never taken for this call's.
 * Other arguments and the slot rules as for pa_decode_step.  Supported:
 * fp16/bf16 pools on the matrix cores (PA_ERR_UNSUPPORTED for other dtypes
 * or under pa_set_decode_kernel(PA_KERNEL_GENERIC)), block_size 16, head_dim
 * 64 or 128, G <= 16.  With no group it is pa_decode_step on the even
 * split. */
pa_status pa_decode_step_shared(float* out, const void* q, void* k_pool, void* v_pool,
                                const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* prefix_len,
                                const int32_t* group_rows, const int32_t* group_start,
                                int32_t num_groups, int32_t num_rows, int32_t max_group_size,
                                int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Attention of a chunk of query tokens per sequence over the paged cache
 * (prefill of a prompt, chunked prefill on top of a cached prefix, or decode
 * with one token).  Sequence b holds L = context_lens[b] tokens in its blocks
 * (the chunk's own K/V included: append them with pa_cache_append first);
 * its query rows are query_start[b] .. query_start[b+1]-1 of q, and row
 * query_start[b] + i is the token at position L - n_b + i
 * (n_b = query_start[b+1] - query_start[b] <= L).  For each such row and
 * query head h:
 *   out[row][h] = softmax_t(scale * q[row][h] . K_b[t]) weighted sum of
 *                 V_b[t], t in [0, L - n_b + i]
 * (causal), K_b/V_b being KV head h/G reached through block_tables[b] in
 * logical order (page 3, abeam.tech review, sections 「KV キャッシュマネージャ」
 * and 「モデル構造ではなくサービング基盤の変更」; the prompt phase as its own
 * stage: 「今後注目すべき方向性」).  Accumulation in fp32.
 *   q: device [num_tokens][Hq][D], KV dtype; out: device float
 *   [num_tokens][Hq][D]; query_start: device int32 [num_seqs + 1],
 *   non-decreasing from 0 to num_tokens; max_query_len: an upper bound of n_b
 *   (sizes the launch); max_context_len: upper bound of context_lens.
 * Supported: fp16/bf16 KV (matrix cores), block_size 16, head_dim 64 or 128,
 * Hq a multiple of Hkv.  Rows of a sequence whose length or chunk fails the
 * bounds checks (L > max_context_len, n_b > L or > max_query_len), or whose
 * table holds an entry outside the pool, are NaN; a sequence whose
 * query_start entries are out of order or out of [0, num_tokens] gets no
 * rows written.  Asynchronous on `stream`. */
pa_status pa_prefill(float* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                     int32_t max_context_len, int32_t max_query_len, float scale,
                     pa_dtype dtype, void* stream);

/* Decode attention over a quantized cache (pools of PA_FP8_E4M3 or
 * PA_INT8 codes written by pa_cache_append_quant): pa_decode's result with
 * K_b[t] = k_scale * code and V_b[t] = v_scale * code (page 1, jisaku.com
 * glossary, section 「他のKVキャッシュ最適化との組み合わせ」: an INT8 cache
 * halves the bytes per block).  q is bf16 [num_seqs][Hq][D]; the codes are
 * widened exactly to bf16 on the matrix cores; k_scale is folded into the
 * softmax scale (fp32 product scale * k_scale) and v_scale into the output.
 * Other arguments, the workspace and the bounds checks as for pa_decode.
 * Supported: block_size 16, head_dim 64 or 128, G = Hq/Hkv <= 16
 * (PA_ERR_UNSUPPORTED otherwise); pa_set_decode_kernel does not apply
 * (there is no plain-FMA kernel for codes). */
pa_status pa_decode_quant(float* out, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                          int32_t partition_size, pa_dtype cache_dtype, float k_scale,
                          float v_scale, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step over a quantized cache, with the result of
 * pa_cache_append_quant(k_pool, v_pool, k_new, v_new, slot_mapping,
 * num_seqs, ..., cache_dtype, PA_BF16, k_scale, v_scale) followed by
 * pa_decode_quant(...) (k_new/v_new: bf16 [num_seqs][Hkv][D], sequence b's
 * token at position context_lens[b] - 1).  Slots as for pa_decode_step: the
 * table's slot, -1 (no write; the position is attended as stored), or a slot
 * elsewhere in the pool (written; out only defined when it is not attended).
 * The new tokens are encoded inside the kernels, no separate append launch:
 * the attention kernel attends their codes, and the merge kernel writes them
 * when one runs (else the attention kernel does); a sequence whose length
 * fails the bounds checks (NaN out rows) or is 0 gets no pool write.
 * Copy-on-write copies of the step must be issued before this call on the
 * same stream. */
pa_status pa_decode_step_quant(float* out, const void* q, void* k_pool, void* v_pool,
                               const void* k_new, const void* v_new,
                               const int64_t* slot_mapping, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                               int32_t partition_size, pa_dtype cache_dtype, float k_scale,
                               float v_scale, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Sliding-window decode: pa_decode / pa_decode_step with attention over the
 * last `window` positions of each sequence only, t in
 * [max(0, L - window), L) (window = 0: all L positions, the plain calls).
 * Table entries of blocks wholly before L - window are never read, so they
 * may have been dropped by pa_bm_release_before (page 1, jisaku.com
 * glossary, section 「他のKVキャッシュ最適化との組み合わせ」: a sliding window
 * lets blocks that left it be freed).  Fixed partitions count from the
 * partition holding the window's first position; the workspace is sized as
 * for pa_decode.  Other arguments, bounds checks and the step's slot rules
 * as for pa_decode / pa_decode_step.  Supported: fp32/fp16/bf16 pools,
 * G = Hq/Hkv <= 16.  window < 0 is PA_ERR_INVALID_ARG. */
pa_status pa_decode_window(float* out, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                           int32_t window, int32_t partition_size, pa_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_decode_step_window(float* out, const void* q, void* k_pool, void* v_pool,
                                const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, const int32_t* block_tables,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t num_blocks,
                                int32_t max_blocks_per_seq, int32_t max_context_len,
                                float scale, int32_t window, int32_t partition_size,
                                pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Measurement hook: the next attention kernel launched by a decode call
 * (pa_decode, pa_decode_partial, pa_decode_step, pa_decode_step_partial,
 * pa_decode_quant, pa_decode_step_quant, pa_decode_window or
 * pa_decode_step_window)
 * on this host thread records start_event when it starts executing and
 * stop_event when it finishes, attached to the kernel's own dispatch, so
 * hipEventElapsedTime(start, stop) is that kernel's duration.  The events are
 * hipEvent_t handles created by the caller (with timing enabled); they are
 * consumed by the next decode call whether or not it launches an attention
 * kernel.  Both NULL disarms; one NULL is PA_ERR_INVALID_ARG. */
pa_status pa_time_next_attention(void* start_event, void* stop_event);

/* Measurement utility: streams `bytes` bytes of device buffer `buf` (16-byte
 * aligned, a multiple of 16) through the vector memory path with 16-byte
 * non-temporal loads over a grid of 8 x 256-thread workgroups per compute
 * unit, and discards them (device int `sink` is written only for a buffer
 * whose 16-byte words XOR to one specific pattern).  Its time gives the chip's
 * streaming-read bandwidth, the reference the decode kernels are set against.
 * Asynchronous on `stream`. */
pa_status pa_stream_read(const void* buf, size_t bytes, int32_t* sink, void* stream);

/* Reassembles the logically contiguous cache through the block tables:
 * k_out/v_out device [num_seqs][Hkv][max_context_len][D] in the KV dtype
 * (codes for the 8-bit dtypes), positions >= context_lens[b] zero-filled,
 * positions of a bad length or table entry all-ones bits (NaN for the float
 * dtypes).  Uses the same table walk as
 * pa_decode; meant for checks and for handing a sequence to dense code. */
pa_status pa_gather_kv(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_context_len, pa_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

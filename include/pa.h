/*
 * pa.h -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpa.so.  Plain pointers and sizes only; every tensor argument is
 * device memory owned by the caller.  The library allocates nothing, keeps no
 * state besides the thread-local error string (and the static scratch array of
 * pa_decode_noalloc, one per GPU), never synchronises, and puts
 * every kernel on the stream it is given (a hipStream_t passed as void*;
 * NULL is the default stream).  Calls are asynchronous: a fault inside a
 * kernel surfaces as a HIP error at the caller's next synchronisation.
 *
 * Sources (page title, section):
 *  [DRV]  "揭开 NVIDIA 驱动栈的面纱：GPU 显存页表与 vLLM 中的 PagedAttention 是如何在底层协同的"
 *         (kwkd.cn), section 6: logical token -> (physical block, offset) through the
 *         block table; the K pointer is block * block-stride + head * head-stride + offset.
 *  [SRC]  vLLM source walk-through (peacm.com), section 3.2 (append a token into the
 *         last block), section 3.4 (per-block loop, tail mask, online softmax).
 *  [CON]  "PagedAttention：当 KV Cache 遇到操作系统分页" (forceinjection.github.io),
 *         sections 3.1-3.2 (fixed-size blocks, per-sequence block table, gather).
 *  [SOSP] "《Efficient Memory Management for LLM Serving with PagedAttention》深度解读报告"
 *         (zako-mio.github.io), sections 2.3, 3.2-3.4 (K and V blocks kept apart; the
 *         fill count keeps padding out; write the new token, then attend over all valid KV).
 *         [CON] section 6 adds FP8 storage inside the blocks, expanded by the kernel:
 *         the *_fp8 calls below.
 *
 * Layouts (all row-major, contiguous, 16-byte aligned):
 *   k_cache, v_cache  [num_blocks, num_kv_heads, block_size, head_dim]   (one layer)
 *   k, v              [num_tokens, num_kv_heads, head_dim]
 *   q, out            [num_seqs, num_q_heads, head_dim]
 *   block_tables      [num_seqs, max_blocks_per_seq] int32
 *   context_lens      [num_seqs] int32; counts the token written in this step
 *   slot_mapping      [num_tokens] int64; slot = physical_block * block_size + offset
 *
 * Query head h attends with kv head h / (num_q_heads / num_kv_heads).
 * Supported: dtype PA_F32 or PA_F16 (all of q, k, v, caches and out share it;
 * arithmetic is fp32), head_dim 64 or 128, block_size 8, 16 or 32.
 * The *_fp8 calls keep the pools as one byte per element (FP8 E4M3 codes) with q, k,
 * v and out in fp16; same layouts, same head_dim and block_size support.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define PA_F32 0
#define PA_F16 1

/* return codes; on error pa_last_error() describes the cause */
#define PA_OK 0
#define PA_ERR_INVALID_ARG (-1) /* a size, pointer or alignment is not valid             */
#define PA_ERR_UNSUPPORTED (-2) /* valid but not built: dtype, head_dim or block_size     */
#define PA_ERR_WORKSPACE (-3)   /* workspace missing or smaller than the size query says */
#define PA_ERR_HIP (-4)         /* a HIP launch failed                                   */
#define PA_ERR_EXHAUSTED (-5)   /* the block allocator has no free block left             */

/*
 * pa_cache_write -- store each new token's K and V into its slot of the pools.
 *
 * For t < num_tokens and every kv head h:
 *   k_cache[slot / block_size, h, slot % block_size, :] = k[t, h, :]   (same for v),
 * slot = slot_mapping[t].  This is the append of [SRC] section 3.2 and step one of
 * [SOSP] section 3.4: the new token's K/V goes into the next free slot of the
 * sequence's last block (the block itself is chosen on the host).  The copy is
 * bit-exact.  A negative slot is padding and is skipped; so is a slot at or beyond
 * num_blocks * block_size.  Slots must be distinct: two tokens with one slot race.
 *
 * k, v              device, [num_tokens, num_kv_heads, head_dim], dtype
 * slot_mapping      device, [num_tokens] int64
 * k_cache, v_cache  device, [num_blocks, num_kv_heads, block_size, head_dim], dtype; updated in place
 * num_tokens        >= 0 (0 launches nothing); num_tokens * num_kv_heads * head_dim * element
 *                   size / 16 at most 2^31 - 256 per call (one thread per 16-byte chunk; a
 *                   larger write is refused: split the tokens)
 * returns PA_OK, or a negative code with nothing launched.
 */
int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                   void* k_cache, void* v_cache,
                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream);

/*
 * pa_decode_workspace_bytes -- workspace pa_decode needs for these sizes.
 *
 * The workspace holds, per (sequence, kv head, tile of query heads), where that
 * context's piece records are, and the records (fp32 running max, exp-sum and
 * normalised output of each query head): up to two per persistent wave for
 * partition_size == 0, one per partition of each context for partition_size > 0.
 * Its size depends only on the arguments below, never on the device.
 * Returns 0 for num_seqs <= 0 or invalid sizes.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode -- single-query attention of every (sequence, query head) over the
 * sequence's paged K/V.
 *
 * out[s, h, :] = softmax(scale * K_s q[s, h]) V_s, where K_s, V_s are the first
 * context_lens[s] positions of sequence s, position p living at
 * (block_tables[s, p / block_size], p % block_size) of the pools ([DRV] section 6,
 * [CON] section 3.2).  Positions at or past context_lens[s] are neither read nor
 * used ([SOSP] section 2.3; [SRC] section 3.4 masks them), so the unfilled tail of
 * the last block and table entries past ceil(ctx / block_size) may hold anything.
 * The result equals attention over contiguously stored K/V ([SOSP] sections 3.3
 * and 4.4).  A context of 0 gives a zero row.
 *
 * Work split: the batch is cut into tiles of consecutive tokens and as many
 * persistent waves as the GPU holds at once each take a contiguous run of them, so a
 * long context is split over several waves; a second kernel merges the pieces of each
 * context by log-sum-exp, in token order.
 *   partition_size == 0: each wave's run is equal in tiles plus one tile's worth per
 *     context piece, and a piece ends where a wave's run ends.  Where a context is
 *     split then depends on the whole batch, so the same sequence at another batch
 *     position may differ in rounding.
 *   partition_size > 0 (a multiple of block_size and of 16): each context is cut into
 *     fixed partitions of partition_size tokens (a split of this library's own; the
 *     pages fix no split), a partition is never split between waves, and the runs are
 *     balanced over tiles plus one tile's worth per partition.  A row's result then depends only on
 *     its own query, context and partition_size: bitwise identical at any batch
 *     position and in any batch.
 * In both modes results are bitwise identical under any relabelling of physical blocks
 * and any block size.
 * Arithmetic: fp32 scores, softmax and accumulation.  For PA_F16 the probabilities are
 * rounded to fp16 for the P.V product (on the matrix cores), which bounds the output's
 * deviation from exact attention by about 2^-11 * (|out| + max |v|).
 *
 * out                device, [num_seqs, num_q_heads, head_dim], dtype; written
 * q                  device, [num_seqs, num_q_heads, head_dim], dtype
 * k_cache, v_cache   device, [num_blocks, num_kv_heads, block_size, head_dim], dtype
 * block_tables       device, [num_seqs, max_blocks_per_seq] int32
 * context_lens       device, [num_seqs] int32
 * scale              softmax scale (1/sqrt(head_dim) on the pages); positive and finite
 * max_context_len    host bound on every context_lens[s]; at most max_blocks_per_seq * block_size
 * num_seqs, num_q_heads  at most 65535 each (grid dimensions); num_seqs * num_kv_heads at
 *                    most 2^31 - 1 segments, and, counting max_context_len for every
 *                    segment, at most 2^31 - 1 tiles of 8 tokens plus pieces (one per
 *                    segment, or one per partition) in all
 * partition_size     0 (the default split) or a positive multiple of 16 and of block_size
 *                    (fixed partitions); see the work split above
 * workspace          device, >= pa_decode_workspace_bytes(...) bytes, 256-byte aligned;
 *                    contents need no initialisation and are scratch between calls
 *
 * Device-side checks: a sequence whose context length is negative or exceeds
 * max_context_len gets NaN rows and reads nothing; a table entry outside
 * [0, num_blocks) within a context is not dereferenced (block 0 is read instead) and
 * the affected query heads get NaN.  Calls that share a workspace must not overlap.
 * returns PA_OK, or a negative code with nothing launched.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens,
              float scale, int32_t block_size, int32_t num_kv_heads,
              int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
              int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
              int32_t partition_size, int32_t dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments
 * as pa_decode without the workspace; same kernels, work split and results, bit for bit.
 * Its scratch (the segment descriptors and piece records a workspace would hold) is a
 * static device array of PA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; the call itself allocates nothing.  Sizes whose scratch
 * would exceed that (records for every persistent wave of the launch: at the default split
 * this covers every head_dim and group size) return PA_ERR_WORKSPACE with nothing launched.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on two
 * streams, or from two threads) race and must be serialised by the caller.  The array needs
 * no clearing: whatever a call reads of it, the same call wrote first.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      float scale, int32_t block_size, int32_t num_kv_heads,
                      int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                      int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                      int32_t partition_size, int32_t dtype, void* stream);

/*
 * pa_decode_shared -- pa_decode for a batch in which groups of sequences share the physical
 * blocks of a prefix: the samples of one prompt in parallel sampling, or requests over a
 * common cached prefix, whose tables name the same blocks by reference count ([SOSP]
 * section 2.4; [CON] section 4.3).  The result is attention over each sequence's whole
 * context, as pa_decode gives it, but each group's prefix is read from HBM once for all its
 * members: the members' query heads of one kv head (up to 32 rows) are the columns of one
 * pass over the prefix, and each member's own positions L .. ctx - 1 are a pass of its own;
 * the second launch merges the two by log-sum-exp, in token order.  The split of the batch
 * differs from pa_decode's, so the two agree within rounding, not bit for bit.
 *
 * seq_group          device, [num_seqs] int32: the group whose prefix sequence s shares, or -1
 * group_first        device, [num_groups] int32: the group's first member; its members are the
 *                    consecutive sequences group_first .. group_first + group_size - 1
 * group_size         device, [num_groups] int32: members, 1 .. 32 / (num_q_heads / num_kv_heads)
 * group_prefix       device, [num_groups] int32: shared tokens L, a positive multiple of 16 and
 *                    of block_size, at most max_context_len and at most every member's
 *                    context.  Positions 0 .. L - 1 of every member's table must name the
 *                    same physical blocks: the prefix is read through the first member's
 *                    table, the others' entries there are not read.
 * num_groups         0 .. 65535 (0: no sharing; every sequence's seq_group must then be -1)
 * other arguments    as pa_decode, dtype PA_F16 (q, out, pools); at most 16 query heads per kv
 *                    head; no partition size (the default split)
 * workspace          device, >= pa_decode_shared_workspace_bytes(...) bytes, 256-byte aligned;
 *                    contents need no initialisation
 *
 * Device-side checks: as pa_decode; besides, a sequence whose group is invalid (an L not a
 * multiple of 16 and block_size, a size out of range, members outside the batch), that is
 * not one of its group's members, or whose context is shorter than L gets NaN rows.
 * pa_decode_shared_partitions makes the first launch alone (the stream over the virtual
 * sequences) and leaves the pieces in the workspace; it lets a caller time that kernel.
 * returns PA_OK, or a negative code with nothing launched.
 */
size_t pa_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_groups, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim);
int pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* seq_group, const int32_t* group_first, const int32_t* group_size,
                     const int32_t* group_prefix, int32_t num_groups, float scale, int32_t block_size,
                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                     int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                     void* workspace, size_t workspace_bytes, void* stream);
int pa_decode_shared_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* seq_group, const int32_t* group_first,
                                const int32_t* group_size, const int32_t* group_prefix,
                                int32_t num_groups, float scale, int32_t block_size,
                                int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                                int64_t num_blocks, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * pa_decode_partitions / pa_decode_reduce -- the two launches pa_decode makes,
 * callable on their own (to time each kernel, or to merge pieces computed
 * elsewhere).  pa_decode_partitions takes pa_decode's arguments; it writes the rows
 * of contexts held whole by one wave and leaves the pieces of split contexts in the
 * workspace.  pa_decode_reduce writes every other row (merged pieces, zero rows for
 * empty contexts, NaN rows for invalid ones); it must see the same context_lens,
 * sizes and workspace, and run after pa_decode_partitions on the same stream.
 */
int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float scale, int32_t block_size, int32_t num_kv_heads,
                         int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                         int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                         int32_t partition_size, int32_t dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

int pa_decode_reduce(void* out, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t max_context_len, int32_t partition_size, int32_t dtype,
                     const void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_append -- one decode step in one call: store each sequence's new token and
 * attend over its whole context, the token included ([SRC] section 3.2 appends the token
 * into the sequence's last block; [SOSP] section 3.4 writes it, then attends over every
 * valid position).
 *
 * The new token of sequence s is position p = context_lens[s] - 1; its rows k_new[s], v_new[s]
 * are stored at (block_tables[s, p / block_size], p % block_size) of the pools, the slot
 * that position has in the table, and out is what pa_decode gives after that store.  The
 * results equal pa_cache_write (with that slot for each sequence) followed by pa_decode,
 * bit for bit.  Fewer launches: the attention kernel takes the new token from k_new / v_new
 * rather than the pools, and the second launch (which merges split contexts) stores it.
 * fp16 only (q, k_new, v_new, pools and out), with pa_decode's sizes, workspace, checks and
 * results; sequences with an empty or invalid context, or whose table entry for p lies
 * outside the pool, store nothing.  As with pa_cache_write, two sequences whose new tokens
 * share a slot race, and the caller must not store into a block other tables still read
 * (copy it first, see pa_allocator_append_slot).
 *
 * k_new, v_new   device, [num_seqs, num_kv_heads, head_dim] fp16, 16-byte aligned
 * k_cache, v_cache  updated in place at one slot per sequence
 * other arguments as for pa_decode (dtype is PA_F16)
 *
 * pa_decode_append_partitions -- the first of the two launches alone (attention pieces,
 * new tokens read from k_new / v_new; nothing is stored): pa_decode_reduce merges its
 * pieces, but only pa_decode_append stores the new tokens.
 */
int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, float scale, int32_t block_size,
                     int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                     int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

int pa_decode_append_partitions(void* out, const void* q, const void* k_new, const void* v_new,
                                const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                const int32_t* context_lens, float scale, int32_t block_size,
                                int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                                int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                                int64_t num_blocks, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 KV cache ([CON] section 6: blocks store K/V compressed, the kernel expands them).
 *
 * The pages name FP8 but no format or scaling; these calls take the OCP E4M3 format
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite 448; S.1111.111
 * is NaN; no infinities) and one scale for all of K and one for all of V.  A stored code
 * c of the K pool means value(c) * k_scale, likewise for V.
 *
 * pa_cache_write_fp8 -- pa_cache_write for E4M3 pools: element x of k[t, h, :] (fp16)
 * is stored as the code nearest to the exact quotient x / k_scale; ties go to the even
 * code, a quotient beyond 448 in magnitude saturates to +-448 (code 0x7E / 0xFE), +-0
 * gives 0x00 / 0x80 and any NaN gives 0x7F.  Same for v with v_scale.
 * Slot handling, skips and races are those of pa_cache_write; num_tokens * num_kv_heads *
 * head_dim / 16 is at most 2^31 - 256 per call (one thread per 16 codes).
 *
 * k, v              device, [num_tokens, num_kv_heads, head_dim] fp16
 * k_cache, v_cache  device, [num_blocks, num_kv_heads, block_size, head_dim] uint8; updated in place
 * k_scale, v_scale  positive, finite
 * returns PA_OK, or a negative code with nothing launched.
 */
int pa_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, float k_scale, float v_scale,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, void* stream);

/*
 * pa_decode_fp8 -- pa_decode over E4M3 pools: the result is attention over the
 * dequantized K and V (every code times its scale), everything else as pa_decode with
 * dtype PA_F16 (q and out fp16, the same workspace size query and work split).  The
 * codes are expanded to fp16 exactly; k_scale joins the softmax scale (scale * k_scale
 * must be a positive finite fp32 value) and v_scale multiplies the normalised output.
 * The probabilities are rounded to fp16 for the P.V product, as in pa_decode.
 * pa_decode_fp8_partitions is its first launch alone; pa_decode_reduce with dtype PA_F16
 * is the second.  A NaN code inside a context makes the affected rows NaN.
 */
int pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens,
                  float scale, float k_scale, float v_scale, int32_t block_size,
                  int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                  int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                  int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

int pa_decode_fp8_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             float scale, float k_scale, float v_scale, int32_t block_size,
                             int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                             int32_t head_dim, int32_t max_blocks_per_seq, int32_t max_context_len,
                             int64_t num_blocks, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_fp8_append -- pa_decode_append over E4M3 pools: k_new[s], v_new[s] (fp16) are
 * stored as codes at position context_lens[s] - 1 (rounded as pa_cache_write_fp8 rounds,
 * with k_scale / v_scale) and out is attention over the dequantized context, the new token
 * included.  Equal bit for bit to pa_cache_write_fp8 (at the table's slot) followed by
 * pa_decode_fp8; arguments, checks and stores otherwise as pa_decode_append and
 * pa_decode_fp8.  pa_decode_fp8_append_partitions is its first launch alone (stores
 * nothing); pa_decode_reduce with dtype PA_F16 merges its pieces.
 */
int pa_decode_fp8_append(void* out, const void* q, const void* k_new, const void* v_new,
                         void* k_cache, void* v_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, float k_scale, float v_scale,
                         int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
                         int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int64_t num_blocks, int32_t partition_size,
                         void* workspace, size_t workspace_bytes, void* stream);

int pa_decode_fp8_append_partitions(void* out, const void* q, const void* k_new, const void* v_new,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    float scale, float k_scale, float v_scale, int32_t block_size,
                                    int32_t num_kv_heads, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t head_dim, int32_t max_blocks_per_seq,
                                    int32_t max_context_len, int64_t num_blocks,
                                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * pa_prefill -- causal attention of several query tokens per sequence (a prompt chunk)
 * over the paged cache: the prompt phase of [SOSP] section 2.1, taken in chunks as in
 * [SOSP] section 5.1 (item 5); [VATT] "3 分钟速读" point 1 measures such paged prefill
 * kernels.
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1] - 1, n of them.  They are
 * the last n positions of its context_lens[s] = ctx tokens, whose K/V must already be in
 * the pools (pa_cache_write of the chunk first, as a decode step writes its token).  Row
 * i, at position p = ctx - n + i, and query head h (kv head h / G):
 *   out[row, h, :] = softmax(scale * K_s[0..p] q[row, h]) V_s[0..p]
 * so each token sees the cached prefix and the chunk up to itself.  n = 1 is a decode step.
 * Arithmetic: fp16 products on the matrix cores with fp32 accumulation, fp32 softmax;
 * probabilities are rounded to fp16 for P.V as in pa_decode.
 *
 * q, out             device, [total_q, num_q_heads, head_dim] fp16 (total_q = query_start[num_seqs])
 * k_cache, v_cache   device, [num_blocks, num_kv_heads, block_size, head_dim] fp16
 * block_tables       device, [num_seqs, max_blocks_per_seq] int32
 * context_lens       device, [num_seqs] int32, counting the chunk
 * query_start        device, [num_seqs + 1] int32, non-decreasing, query_start[0] = 0
 * max_query_len      host bound on every n; max_context_len: host bound on every ctx
 * num_seqs, num_q_heads  at most 65535 each; max_query_len * (num_q_heads / num_kv_heads) at
 *                    most 2^30 rows per sequence
 * dtype              PA_F16 (PA_F32 is not built for this call)
 * Device-side checks: a sequence with n > ctx, ctx > max_context_len or n > max_query_len
 * gets NaN rows (only rows below max_query_len are ever written); a table entry outside
 * [0, num_blocks) within the keys a work-group reads is not dereferenced and that
 * work-group's rows get NaN.  No workspace; rows of different sequences never interact.
 * returns PA_OK, or a negative code with nothing launched.
 */
int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
               float scale, int32_t block_size, int32_t num_kv_heads, int32_t num_seqs,
               int32_t num_q_heads, int32_t head_dim, int32_t max_blocks_per_seq,
               int32_t max_query_len, int32_t max_context_len, int64_t num_blocks, int32_t dtype,
               void* stream);

/*
 * Block copies and the block allocator: sharing, copy-on-write and swap.
 * [SRC] section 3.2 (a free pool of blocks, allocate on demand, append a token into the
 * last block or a new one), section 3.3 (preempt by swapping a sequence's blocks out to
 * CPU memory); [DRV] section 4 and [SOSP] section 2.4 (several tables point at one block;
 * reference counts and copy-on-write protect writes); [CON] section 4.3.
 *
 * pa_copy_blocks -- for every pair i: dst_k[pairs[2i+1]] = src_k[pairs[2i]] and the same for
 * V, a block being block_bytes bytes (num_kv_heads * block_size * head_dim * element size
 * for the pools of this library).  Each of the four pools may be device memory of the
 * current device or pinned host memory (hipHostMalloc, torch pin_memory): the same call
 * copies within a pool (copy-on-write), between device pools, and to and from host pools
 * (swap).  The pools are resolved with hipPointerGetAttributes before anything is launched;
 * memory of another kind is refused.  A pair naming a block outside its pool is skipped.
 * No destination may also be the source of another pair of the same call, and the source
 * and destination ranges of one pair must not overlap.
 *
 * pairs          [num_pairs, 2] int32 (source, destination), device or pinned host memory
 * src_num_blocks, dst_num_blocks: blocks in the source and destination pools
 * returns PA_OK, or a negative code with nothing launched.
 */
int pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int32_t* pairs, int32_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int64_t block_bytes, void* stream);

/*
 * pa_allocator -- host-side reference-counted allocator of one pool's blocks.
 * Free blocks form a stack over an initial order (order[0] is handed out first; NULL means
 * 0, 1, 2, ...); a released block is the next one handed out.  Each call either completes
 * or changes nothing (a refused call returns an error code and pa_last_error says why).
 * Not thread-safe: one allocator, one thread at a time.  Tables are host int32 arrays.
 *
 * pa_allocator_append_slot -- the slot of the token at position ctx of a sequence whose
 *   table holds *num_table_blocks entries (capacity at most): a position that starts a
 *   block takes a new block (appended to the table); a position inside a last block that
 *   other tables share first moves the table onto a fresh block, returned as the copy
 *   (*cow_src, *cow_dst) the caller must make with pa_copy_blocks before writing (both -1
 *   when none is needed).  Returns PA_ERR_EXHAUSTED with nothing changed when no block is free.
 * pa_allocator_fork -- child = table, every block shared once more (parallel sampling).
 * pa_allocator_free_table -- release every entry of a table.
 * pa_allocator_move -- rewrite num_tables tables (row t: lens[t] entries at tables + t * stride)
 *   onto the pool of dst: each distinct block once (shared blocks stay shared), writing the
 *   (source, destination) copies to pairs and their count to *num_pairs; the blocks are
 *   released in src.  For swap out (device allocator to host allocator) and back.
 */
typedef struct pa_allocator pa_allocator;
pa_allocator* pa_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* order);
void pa_allocator_destroy(pa_allocator* a);
int32_t pa_allocator_num_free(const pa_allocator* a);
int32_t pa_allocator_refcount(const pa_allocator* a, int32_t block);
int pa_allocator_allocate(pa_allocator* a, int32_t* block);
int pa_allocator_share(pa_allocator* a, int32_t block);
int pa_allocator_release(pa_allocator* a, int32_t block);
int pa_allocator_append_slot(pa_allocator* a, int32_t* table, int32_t capacity, int32_t* num_table_blocks,
                             int32_t ctx, int64_t* slot, int32_t* cow_src, int32_t* cow_dst);
int pa_allocator_fork(pa_allocator* a, const int32_t* table, int32_t n, int32_t* child);
int pa_allocator_free_table(pa_allocator* a, const int32_t* table, int32_t n);
int pa_allocator_move(pa_allocator* src, pa_allocator* dst, int32_t* tables, const int32_t* lens,
                      int32_t num_tables, int32_t stride, int32_t* pairs, int32_t pairs_capacity,
                      int32_t* num_pairs);

/*
 * A virtually contiguous K/V cache: the baseline the vAttention page sets against paging
 * ([VATT] "核心机制" 1-3: reserve virtually contiguous space per request up front, back it
 * with physical pages only as the KV grows, make sure every active request is backed before
 * each iteration's kernels; "GPU / 系统数据路径": the kernel addresses the KV as a flat
 * tensor).  HIP virtual memory (hipMemAddressReserve / hipMemCreate / hipMemMap /
 * hipMemSetAccess) does the mapping; there are no block tables.  One layer, fp16.
 *
 * pa_vkv_create -- reserve K and V address ranges for max_seqs sequences of up to
 *   max_context_len tokens, laid out [max_seqs][region][num_kv_heads][head_dim] with each
 *   sequence's region a whole number of pages.  Pages are multiples of the allocation
 *   granularity and of 16 tokens; page_bytes 0 picks the smallest such page of at least
 *   2 MB, otherwise page_bytes must be such a multiple.  Returns NULL on error (see
 *   pa_last_error).  Allocates device memory.
 * pa_vkv_step -- before an iteration: map pages so that tokens [0, context_lens[s]) of every
 *   sequence s < num_seqs are backed (never unmaps), and record the lengths (host array) for
 *   pa_decode_dense.  Synchronises the stream.  PA_ERR_EXHAUSTED when memory runs out; the
 *   call then maps nothing.
 * pa_vkv_free_seq -- a finished sequence: synchronise the device, unmap its pages.
 * pa_vkv_write -- store token t's K/V rows at (seq_ids[t], positions[t]) (device int32
 *   arrays; k, v [num_tokens, num_kv_heads, head_dim] fp16); positions no page backs are
 *   skipped.
 * pa_decode_dense -- pa_decode over the cache for the sequences of the last step, with their
 *   recorded lengths: out, q [num_seqs, num_q_heads, head_dim] fp16; workspace as
 *   pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
 *   max_context_len, partition_size).  Same kernels, work split and arithmetic as pa_decode
 *   for fp16, with each tile's address computed instead of looked up.
 */
typedef struct pa_vkv pa_vkv;
pa_vkv* pa_vkv_create(int32_t max_seqs, int32_t max_context_len, int32_t num_kv_heads, int32_t head_dim,
                      int32_t dtype, int64_t page_bytes);
void pa_vkv_destroy(pa_vkv* kv);
int pa_vkv_step(pa_vkv* kv, const int32_t* context_lens, int32_t num_seqs, void* stream);
int pa_vkv_free_seq(pa_vkv* kv, int32_t seq);
int pa_vkv_write(pa_vkv* kv, const void* k, const void* v, const int32_t* seq_ids, const int32_t* positions,
                 int32_t num_tokens, void* stream);
void* pa_vkv_k(const pa_vkv* kv);
void* pa_vkv_v(const pa_vkv* kv);
int64_t pa_vkv_seq_bytes(const pa_vkv* kv);
int64_t pa_vkv_page_bytes(const pa_vkv* kv);
int64_t pa_vkv_mapped_bytes(const pa_vkv* kv);
int32_t pa_vkv_capacity(const pa_vkv* kv, int32_t seq);
int pa_decode_dense(void* out, const void* q, const pa_vkv* kv, float scale, int32_t num_q_heads,
                    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/* Description of the last error on the calling thread ("" if none); valid until the next call. */
const char* pa_last_error(void);

/* ABI version of this header: (major << 16) | minor. */
int pa_abi_version(void);
#define PA_ABI_VERSION ((2 << 16) | 9)

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

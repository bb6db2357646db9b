/*
 * pa.h -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpa.so.  Plain pointers and sizes only; every tensor argument is
 * device memory owned by the caller.  The library allocates nothing, keeps no
 * state besides the thread-local error string, never synchronises, and puts
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
 * num_tokens        >= 0 (0 launches nothing)
 * returns PA_OK, or a negative code with nothing launched.
 */
int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping,
                   void* k_cache, void* v_cache,
                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream);

/*
 * pa_decode_workspace_bytes -- workspace pa_decode needs for these sizes.
 *
 * With partition_size > 0 a sequence of ctx tokens is split into
 * ceil(ctx / partition_size) partitions; each partition's maximum, exp-sum and
 * normalised output (fp32) are kept here until the reduce merges them.
 * Returns 0 when partition_size == 0 (single pass) or any size is <= 0.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size);

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
 * partition_size > 0 (a multiple of block_size) splits each context into
 * partitions of that many tokens that run as separate work-groups; a second kernel
 * merges them by log-sum-exp in partition order.  partition_size == 0 runs one
 * pass per sequence and needs no workspace.  Results depend only on logical
 * positions, so they are bitwise identical under any relabelling of physical blocks.
 *
 * out                device, [num_seqs, num_q_heads, head_dim], dtype; written
 * q                  device, [num_seqs, num_q_heads, head_dim], dtype
 * k_cache, v_cache   device, [num_blocks, num_kv_heads, block_size, head_dim], dtype
 * block_tables       device, [num_seqs, max_blocks_per_seq] int32
 * context_lens       device, [num_seqs] int32
 * max_context_len    host bound on every context_lens[s]; sizes the grid
 * workspace          device, >= pa_decode_workspace_bytes(...) bytes (may be NULL if 0)
 *
 * Device-side checks: a sequence whose context length is negative or exceeds
 * max_context_len or max_blocks_per_seq * block_size, or whose table names a block
 * outside [0, num_blocks) within its context, reads nothing invalid and gets NaN
 * in every output element of the affected query heads.
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
 * pa_decode_partitions / pa_decode_reduce -- the two launches pa_decode makes,
 * callable on their own (for timing each kernel, or to merge partitions computed
 * elsewhere).  pa_decode_partitions takes pa_decode's arguments; sequences with a
 * single partition are written to out directly, the others leave their partition
 * results in the workspace.  pa_decode_reduce merges those into out; it must see
 * the same context_lens, sizes and workspace.  pa_decode_reduce with
 * partition_size == 0 does nothing.
 */
int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float scale, int32_t block_size, int32_t num_kv_heads,
                         int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                         int32_t max_blocks_per_seq, int32_t max_context_len, int64_t num_blocks,
                         int32_t partition_size, int32_t dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

int pa_decode_reduce(void* out, const int32_t* context_lens,
                     int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                     int32_t max_context_len, int32_t partition_size, int32_t dtype,
                     const void* workspace, size_t workspace_bytes, void* stream);

/* Description of the last error on the calling thread ("" if none); valid until the next call. */
const char* pa_last_error(void);

/* ABI version of this header: (major << 16) | minor. */
int pa_abi_version(void);
#define PA_ABI_VERSION ((1 << 16) | 0)

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

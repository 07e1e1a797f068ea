/*
 * pagedattn.h -- C ABI of libpagedattn.so: paged decode attention, the
 * slot-mapped KV write and the copy-on-write block copy on MI355X (gfx950).
 *
 * Sources (web pages on the SOSP'23 PagedAttention paper):
 *   [notes-zh]  "PagedAttention 论文精读笔记" (pagedattention-sosp23-notes)
 *   [deep-dive] "paged-attention은 도대체 뭘 최적화 하는 것일까" (hrletsgo.me)
 *   [review-en] "PagedAttention paper review" (junupark.xyz)
 *   [review-kr] "Efficient Memory Management for Large Language Model Serving
 *                with PagedAttention Review" (dimensionstp.github.io)
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers named *_cache, q, out, k_new, v_new, slot_mapping, block_tables,
 * context_lens, block_mapping and workspace are DEVICE pointers owned by the
 * caller; every one must be 16-byte aligned. The library allocates no memory
 * and keeps no state between calls apart from a per-device cache of device
 * properties and the fixed per-device array of pa_decode_noalloc. `stream` is a hipStream_t passed as void* (NULL = the default
 * stream); every call only enqueues work on it and returns without
 * synchronising. The status covers host-side argument checks and launch
 * errors; device-side faults surface on a later synchronisation.
 *
 * KV block pool layout (one contiguous chunk cut into fixed-size physical
 * blocks, each holding K and V for block_size tokens, [notes-zh] §5.1-§5.2;
 * the in-block order is this library's choice):
 *   k_cache: [num_blocks][num_kv_heads][block_size][head_dim]  (token rows)
 *   v_cache: [num_blocks][num_kv_heads][block_size/Bs][head_dim][Bs]
 *            (token columns of sub-tiles: Bs = 32 when block_size is a
 *            multiple of 32 above 32, else Bs = block_size, i.e. a plain
 *            [head_dim][block_size] tile). Channel c of in-block token t is
 *            element ((t / Bs) * head_dim + c) * Bs + t % Bs of the
 *            head_dim*block_size elements of (block, KV head); a 32-token
 *            piece of a block's V is then always whole rows.
 * Token t of a sequence lives in physical block block_tables[s][t / block_size]
 * at offset t % block_size ([deep-dive] §14 and §17), i.e. slot
 * physical_block * block_size + offset.
 *
 * Element types: PA_F32 (IEEE binary32), PA_F16 (IEEE binary16) and PA_BF16
 * (bfloat16). All attention arithmetic is fp32.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, negative or inconsistent size */
  PA_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement */
  PA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = -4        /* the HIP runtime reported an error at launch */
} pa_status;

/* Decode kernel family. AUTO picks MFMA for 16-bit elements (at every group
 * size, MHA included: it measured fastest on MI355X) and the vector kernel
 * for fp32 elements. */
typedef enum pa_algo { PA_ALGO_AUTO = 0, PA_ALGO_VECTOR = 1, PA_ALGO_MFMA = 2 } pa_algo;

/* partition_size values for pa_decode besides a positive multiple of 32:
 *  PA_PARTITION_AUTO:   the context of every (sequence, KV head) is cut so
 *                       that every worker wave gets the same number of
 *                       32-token chunks (split points fall anywhere in the
 *                       batch);
 *  PA_PARTITION_NONE:   one wave per (sequence, KV head), no split;
 *  PA_PARTITION_SHARED: as AUTO, and adjacent sequences that map the same
 *                       physical blocks at the same logical positions from
 *                       position 0 on (forks of one prompt: parallel
 *                       samples, beams, requests on a shared prefix,
 *                       [notes-zh] §6.1-§6.3) form families of up to
 *                       2 * (16 / g) sequences (g = num_heads /
 *                       num_kv_heads) whose common prefix, in whole 32-token
 *                       chunks and at least 64 tokens, is read once and
 *                       attended for all members at once. Only the block ids
 *                       decide (the kernels see nothing else, [notes-zh]
 *                       §6.4); the result is the same attention. It adds two
 *                       planning launches and needs a larger workspace.
 *                       16-bit elements, the MFMA engine and at most 1024
 *                       sequences; otherwise the call runs as AUTO. */
#define PA_PARTITION_AUTO (-1)
#define PA_PARTITION_NONE 0
#define PA_PARTITION_SHARED (-2)

/* Bytes at the start of every decode workspace that hold its arrival
 * counters (zero between calls; see pa_decode). */
#define PA_WORKSPACE_COUNTER_BYTES ((size_t)32768)

/*
 * pa_write_kv -- store new K/V rows into their slots ("fused reshape and
 * block write", [review-kr] §3-2(5); new KV goes into its physical block,
 * [notes-zh] §5.3).
 *   k_new, v_new : [num_tokens][num_kv_heads][head_dim] of `dtype`.
 *   slot_mapping : [num_tokens] int32, slot = physical_block*block_size + offset.
 *                  A negative slot or one >= num_blocks*block_size is skipped.
 *   For every written token n and head h:
 *     k_cache[slot/B][h][slot%B][:] = k_new[n][h][:]
 *     V channel c of (slot/B, h) at in-block token slot%B (layout above) = v_new[n][h][c]
 *   Bit-exact data movement (NaN payloads included). Two tokens naming the
 *   same slot in one call is a precondition violation (the winner is
 *   unspecified). num_tokens == 0 is a no-op. Any head_dim >= 1 and
 *   block_size >= 1 are accepted.
 */
pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                      void* stream);

/*
 * pa_decode -- exact single-query attention of every sequence's newest token
 * over its paged context ([notes-zh] §2.1 attention equation and §4.2
 * block-wise form; [deep-dive] §8 and §14):
 *   for sequence s, query head h, KV head j = h / (num_heads/num_kv_heads),
 *   L = context_lens[s] (the new token included, so write first):
 *     a_t = exp(scale*q[s][h].k_t) / sum_{u<L} exp(scale*q[s][h].k_u),
 *     out[s][h][:] = sum_{t<L} a_t * v_t,
 *   with k_t, v_t read through block_tables[s].
 *   out          : [num_seqs][num_heads][head_dim] of out_dtype (F32, F16 or
 *                  BF16; the value is rounded once at the end).
 *   q            : [num_seqs][num_heads][head_dim] of dtype.
 *   block_tables : [num_seqs][max_blocks_per_seq] int32; only entries below
 *                  ceil(L/block_size) are read. Ids outside [0, num_blocks)
 *                  are clamped into range (the result is then unspecified,
 *                  but no memory outside the pools is read).
 *   context_lens : [num_seqs] int32. L is clamped to
 *                  min(max_blocks_per_seq*block_size, max_context_len) in
 *                  every split mode; L <= 0 writes zeros.
 *   max_context_len : host-side upper bound of context_lens (sizes the work;
 *                  a longer context is cut to it).
 *   partition_size  : PA_PARTITION_AUTO, PA_PARTITION_SHARED, PA_PARTITION_NONE, or a positive
 *                  multiple of 32: fixed partitions of that many tokens per
 *                  (sequence, KV head), merged by their max and sum of
 *                  exponentials ([review-en] "How does this work?": compute
 *                  per block, then combine the partial results).
 *   workspace    : device scratch of at least pa_decode_workspace_bytes(...)
 *                  bytes (may be NULL when that is 0). Its first
 *                  PA_WORKSPACE_COUNTER_BYTES hold arrival counters: they
 *                  must be zero before the workspace's first use (e.g. a
 *                  zero fill of the new allocation), and every call leaves
 *                  them zero; the rest needs no initial contents. Split
 *                  sequences leave their partial results there. Under
 *                  PA_PARTITION_AUTO (and calls that run as AUTO) the decode
 *                  kernel combines them itself: the worker whose piece is
 *                  counted last merges the sequence (the counters decide who
 *                  merges, never the arithmetic). Otherwise a second kernel
 *                  on `stream` combines them. Calls that overlap in time
 *                  must not share a workspace.
 *   Requirements: head_dim in {64, 128}; block_size in {8, 16, 32, 64, 128};
 *   num_heads % num_kv_heads == 0 and num_heads/num_kv_heads <= 8;
 *   PA_ALGO_MFMA needs dtype F16 or BF16.
 *   The reduction order depends only on logical token positions (no atomics
 *   in the arithmetic), so the result does not change under any permutation
 *   of the physical blocks.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                    pa_dtype dtype, pa_dtype out_dtype, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and a bit-identical result. Split sequences keep their partial
 * results in a fixed array of PA_NOALLOC_SCRATCH_BYTES per device that the
 * library owns (it is held on each device used until the process ends; its
 * address is looked up on the first call on a device). Calls whose
 * pa_decode_workspace_bytes exceeds that size return PA_ERR_WORKSPACE before
 * touching the device (e.g. 512-token partitions of 16 sequences of 128K
 * tokens with 64 query heads need 136 MB; their balanced split needs 35 MB).
 * The array is zero when the library is loaded (its counter region, as a
 * workspace's, is left zero by every call). Every call on one device shares
 * it, so calls that may overlap in time on one device (several streams,
 * several host threads) race: serialise them. No memory is allocated by this
 * call.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_dtype dtype, pa_dtype out_dtype, void* stream);

/* pa_decode with an explicit kernel family (pa_algo). Same contract. */
pa_status pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_context_len, float scale, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, pa_dtype dtype,
                       pa_dtype out_dtype, pa_algo algo, void* stream);

/*
 * pa_write_decode -- the decode step's write and attention in one call:
 * the same result as pa_write_kv of every sequence's new token (k_new[s],
 * v_new[s], [num_seqs][num_kv_heads][head_dim] of dtype) into the slot of
 * its position L-1 = context_lens[s]-1, found through block_tables[s],
 * followed by pa_decode with the same arguments: output and cache contents
 * are bit-identical to that pair of calls ([notes-zh] §5.3: the new token's
 * KV goes into the last logical block, then attention reads the blocks).
 * The attention kernel takes position L-1 from k_new/v_new and never uses
 * what the slot holds, so the store may overlap it: the decode kernel
 * stores the new tokens itself under PA_PARTITION_SHARED and when the
 * balanced split merges inside it (at least a quarter as many sequences as
 * workers per KV head); otherwise the launch after it (which also merges
 * split sequences) does.
 * The block of position L-1 must not be shared with another sequence of the
 * call (copy-on-write has already made it private, [notes-zh] §6.1). No
 * write is made for a sequence with L <= 0, with L beyond
 * max_blocks_per_seq*block_size or max_context_len, or whose table entry for
 * position L-1 is not a block of the pool (its output is then unspecified,
 * as with any invalid entry).
 * k_new/v_new: device, 16-byte aligned, both given. Workspace as for
 * pa_decode.
 */
pa_status pa_write_decode(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                          int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, pa_dtype dtype, pa_dtype out_dtype, void* stream);

/*
 * pa_prefill -- prompt-phase attention over the paged cache ([notes-zh] §2.2:
 * every prompt token is processed at once; §2.1: token i attends to tokens
 * 1..i, here 0-based positions).
 *   q: [total_q][num_heads][head_dim] of dtype, the queries of all sequences
 *     packed: sequence s owns rows q_start[s] .. q_start[s+1]-1 (q_start:
 *     device int32 [num_seqs + 1], non-decreasing, from 0 to total_q).
 *   With n queries and L = context_lens[s], query j sits at position
 *   L - n + j (the last n tokens of the context, whose K/V the caller has
 *   already stored, e.g. with pa_write_kv; n = L for a whole prompt, fewer
 *   when its first tokens were cached before) and attends to tokens
 *   0 .. L - n + j through block_tables[s]:
 *     out[row][h] = sum_t a_t v_t,  a = softmax_t(scale * q[row][h] . k_t),
 *   grouped heads as in pa_decode, fp32 accumulation.
 *   out: [total_q][num_heads][head_dim] of out_dtype.
 *   16-bit dtype only (fp32 gives PA_ERR_UNSUPPORTED); head_dim 64 or 128;
 *   block_size a power of two in [8, 128]. Sequences with n <= 0, n > L, L
 *   beyond max_blocks_per_seq*block_size or rows outside [0, total_q) are
 *   skipped (their rows untouched).
 *   No workspace.
 */
pa_status pa_prefill(void* out, const void* q, const int32_t* q_start, int32_t total_q,
                     const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                     pa_dtype dtype, pa_dtype out_dtype, void* stream);

/* Workspace bytes pa_decode needs for these sizes (0 when it needs none).
 * Returns 0 as well for arguments pa_decode would reject. Pure host function. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size);

/* Kernel launches a pa_decode (fused = 0) or pa_write_decode (fused = 1)
 * call with these sizes makes on its stream, on the current device: the
 * decode kernel; under PA_PARTITION_SHARED (16-bit, MFMA) two planning
 * launches before it; and a closing launch after it that merges split
 * sequences and stores the new tokens, except where the balanced split
 * (PA_PARTITION_AUTO) merges inside the decode kernel. 0 for num_seqs == 0
 * or arguments pa_decode would reject. Host function (it reads the
 * device's compute-unit count, as the call does). */
int32_t pa_decode_launches(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_context_len, int32_t partition_size, pa_dtype dtype, pa_algo algo,
                           int32_t fused);

/*
 * pa_copy_blocks -- batched whole-block copy for copy-on-write ([notes-zh]
 * §6.1: a write into a shared block first copies it to a new block; the
 * copies of a step are fused into one launch, [review-kr] §3-2(5)).
 *   block_mapping: [num_pairs][2] int32 (src, dst). For every pair:
 *     k_cache[dst][:][:][:] = k_cache[src][:][:][:] and the same for v_cache
 *   (all KV heads, all slots). Bit-exact. Pairs with an id outside
 *   [0, num_blocks) are skipped. Preconditions: destinations are distinct and
 *   no destination is also a source in the same call (otherwise the result
 *   depends on scheduling). num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_swap_out / pa_swap_in -- move whole blocks between the device pool and a
 * swap space in host memory, for preemption by swapping ([notes-zh] §7.4: the
 * blocks of an evicted group go to CPU RAM, a CPU block allocator tracks
 * them, and they are brought back into GPU blocks when the group resumes;
 * [notes-zh] §7.5: small blocks mean many small transfers). One launch moves
 * every pair; the kernel reads and writes host memory directly.
 *   host: pinned host memory from hipHostMalloc (torch pin_memory), mapped for
 *     the device, holding host_slots slots; slot j is the block's K image
 *     (num_kv_heads*block_size*head_dim elements of dtype, the pool's own
 *     per-block layout) followed by its V image. The call checks that host is
 *     such memory and that the allocation holds host_slots slots from host on;
 *     otherwise PA_ERR_INVALID_ARG.
 *   block_mapping: device [num_pairs][2] int32 (device block, host slot).
 *     swap_out: host slot <- device block; swap_in: device block <- host slot.
 *     Bit-exact. Pairs with a block outside [0, num_blocks) or a slot outside
 *     [0, host_slots) are skipped. Preconditions: the written side (slots for
 *     swap_out, blocks for swap_in) is distinct within one call. The host data
 *     is complete when the stream reaches the end of the call.
 */
pa_status pa_swap_out(void* host, int32_t host_slots, const void* k_cache, const void* v_cache,
                      const int32_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                      void* stream);
pa_status pa_swap_in(void* k_cache, void* v_cache, const void* host, int32_t host_slots,
                     const int32_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                     void* stream);

/* Static, human-readable name of a status. */
const char* pa_status_string(pa_status status);

/* ABI version of this header (incremented on incompatible change). */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */

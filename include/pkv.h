/*
 * pkv.h -- C ABI of libpkv: paged-KV decode attention and the paged KV append
 * on AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones the Rust inference backends on the source pages
 * launch as CUDA kernels:
 *   - the paged KV append        [kapsl-backends 0.1.1, src/gguf_native.rs:
 *                                 launch_kv_write / launch_batch_kv_write in
 *                                 one_token_compute and forward_batch_decode_greedy]
 *   - single-token paged decode attention with grouped-query heads
 *                                [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *                                 BackendPagedKv::paged_decode_attention,
 *                                 paged_batched_decode_single_pass;
 *                                 kapsl-backends 0.1.1: launch_paged_attention]
 *   - its split-K ("flash decoding") form: per-split f32 partials, then a
 *     log-sum-exp combine       [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *                                 SplitKScratch, paged_batched_flash_dispatch]
 *   - the step that feeds it: split QKV, q/k RMS norm, RoPE and the
 *     paged-cache write         [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *                                 split_qkv_norm_rope_into_paged_cache(_varlen)]
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers named q, k, v, k_pool, v_pool, out, block_tables, context_lens,
 *    slot_mapping, partial_*, workspace are DEVICE pointers.  The caller owns
 *    them; the library never frees or reallocates caller memory.
 *  - fp16 data is IEEE binary16, passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on that stream: it enqueues kernels and returns; nothing in
 *    the library synchronises the host on the hot path.
 *  - Return value: PKV_OK (0) or a negative PKV_E* code; pkv_last_error()
 *    returns a thread-local message for the last failing call of the thread.
 *    Argument checks happen on the host before anything is enqueued, so a
 *    failing call enqueues nothing.
 *  - Device-resident indices (block_tables, context_lens, slot_mapping) are
 *    NOT validated on the host (that would need a device->host copy).  The
 *    kernels still never touch memory outside the arrays they are given:
 *    a slot outside [0, N*BS) is skipped, a table entry outside [0, N) makes
 *    its block contribute nothing, a length above M*BS is treated as M*BS and
 *    a negative length as 0.  Results for such inputs are unspecified.
 *
 * Layouts
 * -------
 *    q, out        [num_seqs][num_q_heads][head_dim]            fp16
 *    k_pool        [num_blocks][num_kv_heads][block_size/16][head_dim/32][16][32]  fp16
 *    v_pool        [num_blocks][num_kv_heads][block_size/16][4][head_dim][4]     fp16
 *    block_tables  [num_seqs][max_blocks_per_seq]                int32
 *    context_lens  [num_seqs]                                    int32
 *    k, v (append) [num_tokens][num_kv_heads][head_dim]          fp16
 *    slot_mapping  [num_tokens]                                  int32
 *  The pages fix no pool layout.  Each (block, kv head) tile is one contiguous
 *  run of block_size*head_dim values, stored as block_size/16 panels of 16
 *  rows.  A K panel holds the 16 rows' dims in 32-wide pieces, piece-major
 *  (element (row r, dim d) at ((d/32)*16 + r)*32 + d%32); a V panel holds four
 *  quads of 4 rows, and in a quad each dim's 4 rows side by side (element
 *  (r, d) at ((r/4)*head_dim + d)*4 + r%4).  With this layout every operand
 *  the decode kernel feeds to the matrix cores is whole cache lines (one 1 KB
 *  run per K load, four 128-byte runs per V load of a wavefront), and a new
 *  row written into a panel is head_dim/32 runs of 64 bytes in K and touches
 *  head_dim/16 lines (head_dim/4 32-byte sectors) in V.
 *  K/V row t of a tile is in panel t/16, row t%16.
 *
 *  context_lens[s] counts the rows of sequence s including the token being
 *  decoded (the length after the append) [kapsl-backends 0.1.1,
 *  forward_batch_decode_greedy]; the query attends rows 0..L-1, with row t in
 *  physical block block_tables[s][t / block_size] at offset t % block_size.
 *  Every row of block_tables must be max_blocks_per_seq readable entries: the
 *  decode kernels may read entries past ceil(L/block_size) ahead of knowing L,
 *  but their values never affect a result (any value is allowed there).
 *  Query head hq reads kv head hq / (num_q_heads / num_kv_heads)
 *  [cortiq-engine 0.8.80, src/gpu_cuda.rs: heads-per-kv-head grouping].
 *
 * Compiled geometries: head_dim in {64, 128, 256}, block_size in {16, 32, 64},
 * group size G = num_q_heads / num_kv_heads in 1..16.  The append needs
 * head_dim % 32 == 0 and block_size % 16 == 0 (the K panel's 32-dim pieces).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only the entry points below are exported. */
#define PKV_API __attribute__((visibility("default")))

#define PKV_OK 0
#define PKV_EINVAL (-1)       /* a null pointer, a negative size, Hq % Hkv != 0, misaligned buffer, ... */
#define PKV_EUNSUPPORTED (-2) /* head_dim / block_size / group size not compiled in */
#define PKV_EWORKSPACE (-3)   /* caller workspace smaller than the plan needs */
#define PKV_EHIP (-4)         /* a HIP runtime call or kernel launch failed (message names it) */
#define PKV_ENOMEM (-5)       /* the library could not allocate its own workspace */

/* Geometry of a K/V block pool (both pools share it). */
typedef struct {
    int32_t num_kv_heads; /* Hkv */
    int32_t head_dim;     /* D */
    int32_t block_size;   /* BS: token rows per block */
    int32_t num_blocks;   /* N: blocks in each pool */
} pkv_pool_desc;

/* A launch plan for decode attention (see pkv_plan_decode). */
typedef struct {
    int32_t num_splits;      /* splits per (sequence, kv head) in the grid; 1 = single pass */
    int32_t chunk_blocks;    /* > 0: split j covers blocks [j*chunk_blocks, (j+1)*chunk_blocks);
                                0: each sequence's nb = ceil(L/BS) blocks are cut into
                                   num_splits ranges of ceil(nb/num_splits) blocks */
    int32_t waves_per_group; /* wavefronts per workgroup of the attention kernel */
    int32_t reserved;
    size_t workspace_bytes;  /* f32 partial bytes the plan needs (0 for a single pass) */
} pkv_decode_plan;

/* ---------------------------------------------------------------------------
 * pkv_paged_kv_append
 *   For every token i with 0 <= slot_mapping[i] < N*BS, copies k[i][h][:] and
 *   v[i][h][:] for every kv head h into block slot/BS, row slot%BS of k_pool
 *   and v_pool (bit copy, no arithmetic).  Tokens with a slot outside that
 *   range are skipped (a negative slot marks padding).  Two tokens naming one
 *   slot: which write lands is unspecified.
 *   [kapsl-backends 0.1.1, src/gguf_native.rs: launch_kv_write (one token at
 *   physical_block / pos_in_block), launch_batch_kv_write (per-token blocks
 *   and offsets); the slot = physical_block * block_size + pos_in_block form
 *   folds the two per-token arrays into one]
 *   k, v: [num_tokens][Hkv][D] fp16, 16-byte aligned.  num_tokens == 0 is a
 *   no-op.  Errors: PKV_EINVAL, PKV_EUNSUPPORTED (D not a multiple of 32 or BS
 *   not a multiple of 16),
 *   PKV_EHIP.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_kv_append(const uint16_t *k, const uint16_t *v, const int32_t *slot_mapping,
                        int32_t num_tokens, uint16_t *k_pool, uint16_t *v_pool,
                        pkv_pool_desc pool, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_attention
 *   out[s][hq][:] = softmax(scale * q[s][hq] . K_s^T) . V_s over the L_s =
 *   context_lens[s] rows of sequence s, for every s < num_seqs and every query
 *   head hq (L_s == 0 gives zeros).  f32 arithmetic with an online max/sum;
 *   out rounded to fp16 (nearest even).
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *   BackendPagedKv::paged_decode_attention (q_len == 1 path),
 *   paged_batched_flash_dispatch, paged_batched_decode_single_pass]
 *   num_splits: 0 = the library's dispatcher chooses (pkv_plan_decode),
 *     1 = single pass (no partials), > 1 = that many splits per sequence, cut
 *     by equal block ranges, then the combine.
 *   max_context_hint: host-side upper bound of context_lens used only by the
 *     dispatcher; 0 = block_size * max_blocks_per_seq (the table capacity, as
 *     the pages do).
 *   Split-K partials go to a workspace the library owns: one grow-only buffer
 *   per (device, stream), allocated on first need and replaced by a larger one
 *   when a call needs more.  No workspace buffer is freed before process exit,
 *   the replaced ones included, so a graph captured against a smaller buffer
 *   stays valid after a later, larger call on the same stream grows it (the
 *   growth does not synchronise).  Calls on one stream reuse it in stream
 *   order.
 *   Dispatch order: when the grid (num_seqs * Hkv * splits workgroups) is
 *   larger than the device's CU count and num_seqs <= 16384, a small launch
 *   first ranks the sequences by the rows they attend and the attention grid
 *   runs them longest first (the ranks live in the library workspace; calls
 *   with a caller workspace keep id order).  A single pass without a window
 *   also splits each sequence longer than a CU's fair share of the launch
 *   (all rows * Hkv / CUs, at least 1024 rows) into pieces run by separate
 *   workgroups; the last piece of each (sequence, kv head) to finish merges
 *   the pieces' partials in piece order in the same launch [ferrum-kernels
 *   0.7.7, src/backend/cuda/paged.rs: paged_batched_flash_dispatch, splits
 *   even for grids past the CU count].  The library workspace then holds
 *   (num_seqs + CUs/Hkv) * (num_q_heads * (head_dim + 2) * 4 + 128) bytes
 *   plus 4 * num_seqs * Hkv, rounded up.  Results are the same bits on every
 *   call with the same inputs; a split sequence's outputs differ from a
 *   whole-sequence pass (a caller workspace) by rounding only.
 *   Graph capture: every entry point reads lengths, tables and positions on
 *   the device and sizes its launches from host arguments only, so a captured
 *   call replays correctly with new device-resident values.  A workspace that
 *   would have to grow for split-K partials while its stream is being
 *   captured is PKV_EWORKSPACE: make one call with the same shape on that
 *   stream before capturing, or use a _ws variant with a workspace allocated
 *   beforehand.  (Where only the dispatch order would need the growth, the
 *   captured call keeps id order instead.)
 *   q, k_pool, v_pool, out: 16-byte aligned.  num_seqs == 0 is a no-op.
 *   Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOMEM, PKV_EHIP.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                               pkv_pool_desc pool, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               int32_t num_seqs, int32_t num_q_heads, float scale, uint16_t *out,
                               int32_t num_splits, int32_t max_context_hint, void *stream);

/* Same as pkv_paged_decode_attention, with the split-K partials in a caller
 * workspace (device memory, 256-byte aligned) of at least plan.workspace_bytes
 * bytes for the plan pkv_plan_decode returns for the same arguments; a single
 * pass needs none (workspace may then be NULL).  The workspace must not be in
 * use by other queued work.  Errors: as above, plus PKV_EWORKSPACE. */
PKV_API int pkv_paged_decode_attention_ws(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                  pkv_pool_desc pool, const int32_t *block_tables,
                                  int32_t max_blocks_per_seq, const int32_t *context_lens,
                                  int32_t num_seqs, int32_t num_q_heads, float scale, uint16_t *out,
                                  int32_t num_splits, int32_t max_context_hint, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_attention_noalloc -- for callers that cannot allocate
 *   device memory: code under HIP graph capture on a stream no call has
 *   warmed up, serving loops that must not call hipMalloc, harnesses that
 *   forbid allocation.  Same operation, arguments, dispatcher, results and
 *   errors as pkv_paged_decode_attention, but the split-K partials and the
 *   dispatch-order records live in a fixed device array of
 *   PKV_NOALLOC_SCRATCH_BYTES bytes that the library defines; each device
 *   holds its own copy from the first call on it until the process exits.
 *   The call never allocates or frees device memory (no hipMalloc, no
 *   hipFree, no allocating library routine); its first call on a device
 *   looks the array's device address up once (hipGetSymbolAddress).
 *   Limit: a plan whose partials need more than PKV_NOALLOC_SCRATCH_BYTES
 *   fails with PKV_EWORKSPACE before anything is enqueued (the partials take
 *   num_seqs * num_q_heads * splits * (head_dim + 2) * 4 bytes, rounded up;
 *   a single pass takes none); when the pieces of the dispatch order would
 *   not fit the grid runs whole sequences in order, and when the records
 *   would not fit beside the partials it runs in id order.
 *   Every call on one device shares that device's array, which keeps what
 *   the last call left there: calls whose kernels may overlap on one device
 *   (several host threads, or streams not ordered against each other) race
 *   and give unspecified results.  Calls in one stream's order are safe.
 * ------------------------------------------------------------------------- */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
PKV_API int pkv_paged_decode_attention_noalloc(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                       pkv_pool_desc pool, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *context_lens,
                                       int32_t num_seqs, int32_t num_q_heads, float scale, uint16_t *out,
                                       int32_t num_splits, int32_t max_context_hint, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_step -- the decode step (append + attention): for every
 *   sequence s with L_s = context_lens[s] > 0, first writes k_new[s][h][:] and
 *   v_new[s][h][:] (every kv head h) to row L_s - 1 of the sequence -- block
 *   block_tables[s][(L_s-1)/BS], row (L_s-1)%BS, the slot the callers on
 *   [kapsl-backends 0.1.1, src/gguf_native.rs: forward_batch_decode_greedy]
 *   form for launch_batch_kv_write -- then computes exactly what
 *   pkv_paged_decode_attention computes over the updated pools.  A row whose
 *   table entry names no pool block is not written.
 *   Launches: when the attention grid (num_seqs * Hkv * splits workgroups)
 *   fits one round of the device's CUs, a single fused launch whose workgroups
 *   write the new rows themselves (the row's K runs and the 128-byte V lines
 *   of its quad of rows, the quad's other rows unchanged); otherwise the append kernel
 *   (which also ranks the sequences for the dispatch order described under
 *   pkv_paged_decode_attention) then attention, in stream order.  Results are
 *   identical either way.
 *   k_new, v_new: [num_seqs][Hkv][D] fp16, 16-byte aligned.  The block
 *   holding each sequence's newest row must belong to that sequence alone (no
 *   other sequence of the batch may read or write it).  Other arguments,
 *   workspace and errors as pkv_paged_decode_attention.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_step(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                          uint16_t *v_pool, pkv_pool_desc pool, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,
                          int32_t num_q_heads, float scale, uint16_t *out, int32_t num_splits,
                          int32_t max_context_hint, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_step_qkv -- the decode step from the QKV projection rows:
 *   exactly pkv_split_qkv_norm_rope_into_paged_cache_varlen with one new token
 *   per sequence (token s = sequence s, at position L_s - 1 where L_s =
 *   context_lens[s] counts the rows after the append), followed by
 *   pkv_paged_decode_attention over the updated pools with the rotated q.
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *   split_qkv_norm_rope_into_paged_cache_varlen, then paged_decode_attention;
 *   kapsl-backends 0.1.1, src/gguf_native.rs: forward_batch_decode_greedy,
 *   where the new token's row is written before the attention reads it]
 *   qkv: [num_seqs][(num_q_heads + 2*Hkv) * head_dim] fp16; q_norm_w,
 *   k_norm_w, cos_table, sin_table, max_positions, eps, qk_mode as in
 *   pkv_split_qkv_norm_rope_into_paged_cache_varlen.  q_out: [num_seqs]
 *   [num_q_heads][head_dim] fp16, receives the rotated queries.  Other
 *   arguments as pkv_paged_decode_attention.  Sequences with L_s = 0 are
 *   skipped (no row written, q_out row untouched, output zeros); L_s past
 *   max_positions gives unspecified results (never an access outside the
 *   tables).
 *   Launches: when the attention grid fits one round of the device's CUs, one
 *   launch forms q and the new K/V rows in its prologue (and writes them as
 *   pkv_paged_decode_step does);
 *   otherwise the QKV kernel, then attention.  The two routes agree to within
 *   f32 summation order (the RMS sums are reduced in different orders), not
 *   bit for bit.  The block holding each sequence's newest row must belong to
 *   that sequence alone.
 *   Errors: as pkv_paged_decode_attention, plus those of the QKV arguments.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_step_qkv(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w,
                              const float *cos_table, const float *sin_table, int32_t max_positions, float eps,
                              int32_t qk_mode, uint16_t *q_out, uint16_t *k_pool, uint16_t *v_pool,
                              pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                              const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                              uint16_t *out, int32_t num_splits, int32_t max_context_hint, void *stream);

/* Same computation with a caller-chosen launch plan (from pkv_plan_decode, or
 * tuned by the caller: split count, fixed-size block chunks, waves per
 * workgroup).  The plan is checked (PKV_EINVAL / PKV_EUNSUPPORTED): num_splits
 * in [1, 65535], chunk_blocks >= 0 and, for num_splits > 1 with chunk_blocks > 0,
 * num_splits * chunk_blocks >= max_blocks_per_seq; waves_per_group in
 * {1, 2, 4, 8}, and at most 4 for head_dim 256 (PKV_EUNSUPPORTED).  workspace == NULL uses the library-owned workspace, otherwise
 * it must hold plan->workspace_bytes as computed by pkv_decode_workspace_bytes
 * for plan->num_splits (PKV_EWORKSPACE). */
PKV_API int pkv_paged_decode_attention_planned(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                       pkv_pool_desc pool, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *context_lens,
                                       int32_t num_seqs, int32_t num_q_heads, float scale, uint16_t *out,
                                       const pkv_decode_plan *plan, void *workspace, size_t workspace_bytes,
                                       void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_attention_window -- sliding-window decode attention: as
 *   pkv_paged_decode_attention, but with window > 0 the new row of sequence s
 *   attends only rows max(0, L_s - window) .. L_s - 1; blocks wholly before
 *   the window are never read, so their table entries may name anything.
 *   window = 0 is pkv_paged_decode_attention.  Split ranges start at the
 *   window's first block; the dispatcher plans for at most `window` rows.
 *   [cortiq-engine 0.8.80, src/gpu_cuda.rs: the decode attend, first row =
 *   stored - window (saturating), and the KvMirror window]
 *   Errors: as pkv_paged_decode_attention; window < 0 is PKV_EINVAL.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_attention_window(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                      pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                                      float scale, uint16_t *out, int32_t num_splits, int32_t window,
                                      int32_t max_context_hint, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_step_window -- the decode step with a sliding window:
 *   the append of pkv_paged_decode_step (k_new / v_new to row L_s - 1 of each
 *   sequence), then what pkv_paged_decode_attention_window computes over the
 *   updated pools.  Launch routing, the single-owner rule for the newest
 *   block and the results' independence of the route as
 *   pkv_paged_decode_step; window rules and errors as
 *   pkv_paged_decode_attention_window (window = 0 is pkv_paged_decode_step).
 *   [cortiq-engine 0.8.80, src/gpu_cuda.rs: each decode step stores the new
 *   row, then attends rows stored - window .. stored]
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_step_window(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                 uint16_t *k_pool, uint16_t *v_pool, pkv_pool_desc pool,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                                 uint16_t *out, int32_t num_splits, int32_t window, int32_t max_context_hint,
                                 void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_varlen_attention -- attention for several new query rows per
 *   sequence (speculative verification, chunked prefill): sequence s owns the
 *   rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of q and out; its i-th new row
 *   sits at position pos_offsets[s] + i and attends rows 0 .. pos_offsets[s] + i
 *   of the sequence (itself included, nothing after it), gathered through
 *   block_tables[s] as in pkv_paged_decode_attention.  The pools must already
 *   hold the new rows (pkv_paged_kv_append them first).
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_varlen_attention,
 *   paged_varlen_split_k_dispatch, and the q_len > 1 branch of
 *   paged_decode_attention: cu_seqlens_q = [0, q_len],
 *   pos_offsets = [final_kv_len - q_len]]
 *   q, out: [total_q_tokens][num_q_heads][head_dim] fp16, token-major,
 *     16-byte aligned.  cu_seqlens_q: [num_seqs + 1] int32 prefix sums,
 *     cu_seqlens_q[0] = 0, non-decreasing, cu_seqlens_q[num_seqs] =
 *     total_q_tokens.  pos_offsets: [num_seqs] int32, >= 0, with
 *     pos_offsets[s] + (new rows of s) <= block_size * max_blocks_per_seq.
 *     Device-resident and not validated: values outside these rules never
 *     make a kernel touch memory outside the arrays, but results are then
 *     unspecified.
 *   num_splits: 0 = the library chooses from the grid size (a single pass
 *     once the workgroups fill about half the CUs), 1 = single pass, > 1 = that
 *     many splits per tile of new rows, then the combine (partials in the
 *     library-owned workspace, as pkv_paged_decode_attention).
 *   max_q_len: host upper bound of the new rows of any sequence, used only to
 *     size the grid (0 = total_q_tokens); a smaller value stays correct, the
 *     workgroups then loop.  max_context_hint: as pkv_paged_decode_attention.
 *   A grid of more workgroups than the device has CUs runs its sequences
 *   longest first (pos_offsets[s] + new rows), as pkv_paged_decode_attention
 *   does; results are identical either way.
 *   num_seqs == 0 or total_q_tokens == 0 is a no-op.
 *   Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOMEM, PKV_EHIP.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_varlen_attention(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                               pkv_pool_desc pool, const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *cu_seqlens_q, const int32_t *pos_offsets, int32_t num_seqs,
                               int32_t total_q_tokens, int32_t num_q_heads, float scale, uint16_t *out,
                               int32_t num_splits, int32_t max_q_len, int32_t max_context_hint, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_varlen_step -- the varlen step (append + varlen attention): the
 *   i-th new token of sequence s (token cu_seqlens_q[s] + i) has its K and V
 *   rows k_new[token][h][:], v_new[token][h][:] written to row
 *   p = pos_offsets[s] + i of the sequence (block block_tables[s][p / BS],
 *   row p % BS, every kv head h), then every new row attends as in
 *   pkv_paged_varlen_attention over the updated pools.  A row whose table
 *   entry names no pool block is not written.
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: the q_len > 1 branch
 *   of paged_decode_attention, whose new rows are already in the cache, and
 *   split_qkv_norm_rope_into_paged_cache_varlen, which puts them there]
 *   Launches: one pass with max_q_len <= 32 and no more workgroups than the
 *   device's CUs gives one launch whose workgroups write the new rows
 *   themselves (the new rows' K runs and the V lines of their quads of rows,
 *   other rows unchanged); otherwise a launch writes the new rows (the same
 *   runs and quads, and with a grid of more workgroups than CUs it ranks
 *   the sequences for the attention launch's dispatch order), then attention
 *   runs.  Results are identical either way.
 *   k_new, v_new: [total_q_tokens][Hkv][D] fp16, 16-byte aligned.
 *   max_q_len (required, >= 1): no sequence may have more new rows; it picks
 *   the launches and sizes the append (a sequence with more leaves its rows
 *   past the first max_q_len unspecified; memory stays safe).  The blocks that
 *   receive a sequence's new rows must belong to that sequence alone during
 *   the call.  Other arguments and errors as pkv_paged_varlen_attention.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_varlen_step(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                          uint16_t *v_pool, pkv_pool_desc pool, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                          int32_t num_seqs, int32_t total_q_tokens, int32_t num_q_heads, float scale, uint16_t *out,
                          int32_t num_splits, int32_t max_q_len, int32_t max_context_hint, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_split_qkv_norm_rope_into_paged_cache_varlen -- the step that feeds
 *   paged attention: from the fused QKV projection rows, RMS-normalise the
 *   query and key heads (qk_mode 1), rotate them (RoPE), write the queries to
 *   q_out and the new K and V rows into the paged pools.
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *   split_qkv_norm_rope_into_paged_cache_varlen (one launch over
 *   q_heads + 2 * kv_heads heads per token, cu_seqlens_q / pos_offsets /
 *   block_tables); ferrum-kernels 0.7.1, cuda.rs: qk_norm_rope]
 *   The pages give the arguments, not the arithmetic; computed here, for the
 *   i-th new token of sequence s (token cu_seqlens_q[s] + i) at position
 *   p = pos_offsets[s] + i:
 *     - qkv row = [num_q_heads query heads | Hkv key heads | Hkv value heads],
 *       head_dim values each;
 *     - qk_mode 1: each query/key head x <- x / sqrt(mean(x^2) + eps) * w
 *       (w = q_norm_w for query heads, k_norm_w for key heads); qk_mode 0:
 *       no norm (the weights are not read and may be NULL);
 *     - RoPE turns dim j with dim j + head_dim/2 (j < head_dim/2):
 *       (a, b) -> (a*c - b*s, b*c + a*s), c = cos_table[p][j],
 *       s = sin_table[p][j];
 *     - the query heads go to q_out[token][hq][:]; the key head h and value
 *       head h (copied unchanged) go to row p of the sequence in kv head h:
 *       block block_tables[s][p / block_size], row p % block_size.
 *   f32 arithmetic, each output rounded once to fp16 (nearest even).  The
 *   16-row pool panels that receive new rows are rewritten whole, their other
 *   rows with their own values: the blocks receiving a sequence's new rows
 *   must belong to that sequence alone during the call.
 *   qkv: [total_tokens][(num_q_heads + 2*Hkv) * head_dim] fp16.
 *   q_norm_w, k_norm_w: [head_dim] fp16.  cos_table, sin_table:
 *   [max_positions][head_dim/2] float32.  q_out: [total_tokens][num_q_heads]
 *   [head_dim] fp16, token-major (what pkv_paged_varlen_attention and, for one
 *   token per sequence, pkv_paged_decode_attention read).  cu_seqlens_q,
 *   pos_offsets, block_tables: as pkv_paged_varlen_attention.  qkv, q_out,
 *   pools, tables and weights 16-byte aligned.
 *   Device-resident values are not validated: a token whose cache row has no
 *   pool block is not written to the cache (q_out still is); a 16-row unit of
 *   new rows whose positions leave [0, max_positions) is not written at all.
 *   num_seqs == 0 or total_tokens == 0 is a no-op.
 *   Errors: PKV_EINVAL (null pointers, misalignment, qk_mode not 0 or 1,
 *   eps negative or not finite, max_positions <= 0, ...), PKV_EUNSUPPORTED
 *   (head_dim not 64, 128 or 256; block_size not a multiple of 16), PKV_EHIP.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_split_qkv_norm_rope_into_paged_cache_varlen(const uint16_t *qkv, const uint16_t *q_norm_w,
                                                    const uint16_t *k_norm_w, const float *cos_table,
                                                    const float *sin_table, int32_t max_positions, uint16_t *q_out,
                                                    uint16_t *k_pool, uint16_t *v_pool, pkv_pool_desc pool,
                                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                                    const int32_t *cu_seqlens_q, const int32_t *pos_offsets,
                                                    int32_t num_seqs, int32_t total_tokens, int32_t num_q_heads,
                                                    float eps, int32_t qk_mode, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_split_qkv_norm_rope_into_paged_cache -- the one-sequence form: token i
 *   (of num_tokens) takes RoPE position pos_offset + i and goes to cache row
 *   cache_len + i of the sequence whose table is block_table
 *   [max_blocks_per_seq].  Both are host values, checked here:
 *   pos_offset + num_tokens <= max_positions and cache_len + num_tokens <=
 *   block_size * max_blocks_per_seq (PKV_EINVAL otherwise).  Everything else
 *   as pkv_split_qkv_norm_rope_into_paged_cache_varlen.
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 *   split_qkv_norm_rope_into_paged_cache (tokens, pos_offset, cache_len,
 *   block_size, max_blocks_per_seq)]
 * ------------------------------------------------------------------------- */
PKV_API int pkv_split_qkv_norm_rope_into_paged_cache(const uint16_t *qkv, const uint16_t *q_norm_w, const uint16_t *k_norm_w,
                                             const float *cos_table, const float *sin_table, int32_t max_positions,
                                             uint16_t *q_out, uint16_t *k_pool, uint16_t *v_pool,
                                             pkv_pool_desc pool, const int32_t *block_table,
                                             int32_t max_blocks_per_seq, int32_t num_tokens, int32_t num_q_heads,
                                             int32_t pos_offset, int32_t cache_len, float eps, int32_t qk_mode,
                                             void *stream);

/* ---------------------------------------------------------------------------
 * pkv_plan_decode -- the dispatcher, a pure host function (no device call
 * when cu_count > 0; cu_count <= 0 queries the current device).
 *   Picks single pass or a split count from the number of (sequence, kv head)
 *   tiles, the context bound and the compute-unit count, re-derived for a
 *   256-CU MI355X from the occupancy argument of [ferrum-kernels 0.7.7,
 *   src/backend/cuda/paged.rs: paged_batched_flash_dispatch] (which targets
 *   128 SMs).  num_splits > 0 forces that split count (chunk_blocks = 0).
 *   Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP (device query).
 * ------------------------------------------------------------------------- */
PKV_API int pkv_plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_hint,
                    int32_t num_splits, int32_t cu_count, pkv_decode_plan *plan);

/* Bytes of f32 split-K partials for a grid of num_splits splits:
 * partial_out [B][Hq][S][D] then partial_m and partial_l [B][Hq][S], each
 * array starting on a 256-byte boundary.  0 when num_splits <= 1.
 * [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: SplitKScratch, whose three
 * f32 buffers hold rows * q heads * splits * head_dim (partial_out) and
 * rows * q heads * splits (partial_m, partial_l); one workspace here packs the
 * three.]  Pure host function. */
PKV_API size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_splits);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_split_partials -- split-K phase 1 on its own.
 *   For every sequence s, query head hq and split j with a non-empty block
 *   range (see pkv_decode_plan.chunk_blocks), writes
 *     partial_m[s][hq][j]      = m_j = max over the split's rows of z_t,
 *                                z_t = scale * q[s][hq] . k_t  (natural units)
 *     partial_l[s][hq][j]      = sum_t exp(z_t - m_j)
 *     partial_out[s][hq][j][:] = sum_t exp(z_t - m_j) * v_t   (not normalised)
 *   Entries of empty splits (j >= ceil(nb / chunk)) are not written.
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_batched_flash_dispatch
 *   phase 1 and the partial_out / partial_m / partial_l buffers of SplitKScratch]
 *   partial_out: [num_seqs][Hq][num_splits][D] f32; partial_m, partial_l:
 *   [num_seqs][Hq][num_splits] f32; all 16-byte aligned.
 *   With chunk_blocks > 0 the caller must give num_splits >= ceil(M / chunk_blocks).
 *   Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_split_partials(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                                    pkv_pool_desc pool, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    int32_t num_splits, int32_t chunk_blocks, float *partial_out,
                                    float *partial_m, float *partial_l, void *stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_decode_split_combine -- split-K phase 2 (the reduce) on its own.
 *   out[s][hq][:] = sum_j e^(m_j - M) O_j / sum_j e^(m_j - M) l_j with
 *   M = max_j m_j, over the non-empty splits j < ceil(nb / chunk) of sequence
 *   s (nb from context_lens[s], clamped to max_blocks_per_seq blocks); later
 *   entries are never read.  No rows (or a zero denominator) gives zeros.
 *   Rounded to fp16 (nearest even).
 *   [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_batched_flash_dispatch
 *   phase 2, the reduce launch over (num_heads, num_seqs)]
 *   Errors: PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP.
 * ------------------------------------------------------------------------- */
PKV_API int pkv_paged_decode_split_combine(const float *partial_out, const float *partial_m,
                                   const float *partial_l, const int32_t *context_lens,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq,
                                   int32_t num_splits, int32_t chunk_blocks, uint16_t *out,
                                   void *stream);

/* ---------------------------------------------------------------------------
 * Input checks (cold path, for debugging).  The hot-path entry points read
 * device-resident indices without validating them (see the conventions
 * above); these calls check the same arrays on the device and report through
 * `report`, a device array of 4 int32 the call overwrites:
 *   report[0]  lengths (decode), or prefix sums / positions (varlen), that
 *              break the entry point's rules;
 *   report[1]  table entries outside [0, num_blocks) among those a call with
 *              these lengths would read;
 *   report[2]  the first sequence (slot check: token) with a problem, or
 *              INT32_MAX when there is none;
 *   report[3]  slots at or past num_blocks * block_size (slot check only;
 *              negative slots are padding and allowed).
 * Asynchronous on `stream`: synchronise before reading the report.  No host
 * synchronisation and no allocation (the cold-path counterpart of the check
 * in [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs:
 * paged_decode_attention], which copies the final lengths to the host).
 * Errors: PKV_EINVAL (null or misaligned arrays, negative sizes),
 * PKV_EUNSUPPORTED (block_size not a multiple of 16), PKV_EHIP.
 * ------------------------------------------------------------------------- */

/* Decode: 0 <= context_lens[s] <= block_size * max_blocks_per_seq; the table
 * entries of blocks [max(0, L - window) / block_size, ceil(L / block_size))
 * (window = 0: from block 0) must name pool blocks. */
PKV_API int pkv_check_decode_inputs(const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                            int32_t num_seqs, pkv_pool_desc pool, int32_t window, int32_t *report, void *stream);

/* Varlen: cu_seqlens_q[0] = 0, non-decreasing, cu_seqlens_q[num_seqs] =
 * total_q_tokens; pos_offsets[s] >= 0 with pos_offsets[s] + (new rows of s)
 * <= block_size * max_blocks_per_seq; the entries of blocks
 * [0, ceil((pos + new rows) / block_size)) must name pool blocks. */
PKV_API int pkv_check_varlen_inputs(const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q,
                            const int32_t *pos_offsets, int32_t num_seqs, int32_t total_q_tokens, pkv_pool_desc pool,
                            int32_t *report, void *stream);

/* Slot mapping of pkv_paged_kv_append: slots must be < num_blocks *
 * block_size (negative = padding). */
PKV_API int pkv_check_slot_mapping(const int32_t *slot_mapping, int32_t num_tokens, pkv_pool_desc pool, int32_t *report,
                           void *stream);

/* Number of compute units of the current device (hipDeviceProp_t::multiProcessorCount): the count the
 * dispatcher sizes grids against, where the pages assume a fixed 128 SMs
 * [ferrum-kernels 0.7.7, src/backend/cuda/paged.rs: paged_varlen_split_k_dispatch,
 * "total blocks >= 2 x SM count"].  Errors: PKV_EINVAL (NULL), PKV_EHIP. */
PKV_API int pkv_device_cu_count(int32_t *cu_count);

/* Thread-local message for the last non-zero return on this thread ("" if none): the C form of the
 * error values the pages' backend calls return with a message [ferrum-kernels 0.7.1,
 * src/backend/cuda.rs: Result with a FerrumError, e.g. from end_graph_capture].  The
 * string stays valid until the thread's next failing call. */
PKV_API const char *pkv_last_error(void);

/* Library version string (static storage).  A library utility with no counterpart on the pages. */
PKV_API const char *pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

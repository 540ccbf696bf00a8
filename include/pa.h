/*
 * pa.h -- C ABI of libpagedattn: attention over a paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * The operations are the ones the four pages on paged KV caches build their
 * engines around (InferX, infer-lab, llm-infer, RustInfer):
 *
 *   pa_kv_append             write this step's new K/V rows into their pool
 *                            slots (llm-infer, "What It Does": the captured
 *                            per-layer decode graph writes the KV cache next
 *                            to attention; InferX, "The kernels underneath":
 *                            an fp8 e4m3 KV cache whose per-layer scales are
 *                            fixed during warm-up).
 *   pa_decode                grouped-query softmax(scale * q K^T) V for one
 *                            query token per sequence, K/V gathered through
 *                            per-sequence block tables (infer-lab, technique
 *                            table, PagedAttention row: a block allocator,
 *                            block tables and reference counts; llm-infer,
 *                            "What It Does": a paged KV cache addressed by
 *                            block tables).  Blocks may be shared by several
 *                            sequences (infer-lab, RadixAttention row;
 *                            llm-infer, prefix caching).  With
 *                            partition_size > 0 it computes split-K partials
 *                            instead (flash-decoding).
 *   pa_decode_append         pa_kv_append of each sequence's newest token
 *                            and pa_decode in one launch.
 *   pa_decode_splitk_reduce  merge those partials into the output.
 *   pa_prefill_chunk         causal attention of prefill chunks over their
 *                            cached prefix (InferX, "Status": chunked
 *                            prefill; infer-lab, invariants: prefilling in
 *                            chunks gives the one-shot result; llm-infer,
 *                            "What It Does": prefill of ragged batches).
 *
 * Conventions (the pages leave these open; the library fixes them).  The
 * pool layout below departs from the plainest reading, one [bs][D] tile per
 * (block, KV head) for K and for V: K keeps the 16 tokens of each 16-byte run
 * of head dims together, and V is stored token-minor.  Both make the MFMA
 * operand of a tile one contiguous 16-byte load per lane; the price is that
 * appending one token writes 16-byte pieces spread over its tile.
 *
 *   block size   bs = 16 tokens.  Slot s = block * bs + offset.
 *   K pool       [num_blocks][num_kv_heads][head_dim / X][bs][X], X = the
 *                number of elements in 16 bytes (4 fp32, 8 bf16, 16 fp8):
 *                element (token t, dim d) of a block-head sits at
 *                ((d / X) * bs + t) * X + d % X.  Each 16-byte chunk holds X
 *                consecutive dims of one token; the 16 tokens' chunks of one
 *                dim group are contiguous, so one wave-wide 16-byte load
 *                reads 1 KB in a single contiguous run.
 *   V pool       [num_blocks][num_kv_heads][head_dim][bs]   (token-minor)
 *   Q, out       [tokens][num_heads][head_dim], token-major, contiguous
 *   GQA          query head hq reads KV head hq / G, G = num_heads / num_kv_heads
 *   context_lens include the token appended in this step; a decode query
 *                sits at position L - 1 and attends to positions 0 .. L-1.
 *   block_tables [rows][max_blocks_per_seq] int32; only the first
 *                ceil(L / bs) entries of a row are read.
 *   fp8          OCP E4M3 ("e4m3fn", max 448, no inf).  One fp32 scale per KV
 *                head, separate for K and V: real value = code * scale[h].
 *                Encoding divides by the scale in IEEE binary32, rounds to
 *                nearest even, saturates to +-448, keeps the sign of zero and
 *                maps NaN to 0x7F.
 *   L == 0       the output row is all zeros.
 *
 * Supported (q dtype, cache dtype): (F32, F32), (BF16, BF16), (BF16, FP8).
 * head_dim in {64, 128}; block_size == 16; num_heads % num_kv_heads == 0 and
 * 1 <= G <= 16; pa_decode takes batch <= 4096.  Anything else returns
 * PA_ERR_UNSUPPORTED without launching; there is no fallback path.
 *
 * Ownership and errors.  Every pointer is device memory owned by the caller;
 * the library allocates nothing, frees nothing and keeps no state between
 * calls.  Each call validates its host scalars and pointers (NULL, negative
 * or inconsistent sizes -> PA_ERR_ARG), enqueues its kernels on `stream` and
 * returns; launch failures surface as PA_ERR_LAUNCH.  Device-side contents
 * are trusted, not checked: block ids must be < num_blocks, context lengths
 * must fit the block table row, slots in one append must be distinct and
 * < num_blocks * bs.  Calls on one stream run in order (append before the
 * attention that reads the new token).
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_DT_F32 = 0,
    PA_DT_BF16 = 1,
    PA_DT_FP8_E4M3 = 2
} pa_dtype_t;

typedef enum {
    PA_OK = 0,
    PA_ERR_ARG = 1,          /* NULL pointer, negative or inconsistent size */
    PA_ERR_UNSUPPORTED = 2,  /* dtype / head_dim / block_size / G not built */
    PA_ERR_LAUNCH = 3,       /* the HIP runtime refused a launch */
    PA_ERR_TOO_LARGE = 4     /* pa_decode_noalloc: partials beyond its static scratch */
} pa_status_t;

/* The decode entry point a launch plan is made for (pa_decode_plan). */
typedef enum {
    PA_PLAN_DECODE_APPEND = 0,   /* pa_decode_append: sequence rows */
    PA_PLAN_DECODE_CASCADE = 1,  /* pa_decode_cascade: sequence and prefix-group rows */
    PA_PLAN_DECODE_MULTI = 2     /* pa_decode_multi: multi-query rows */
} pa_plan_entry_t;

/*
 * Write num_tokens new K/V rows into the pools.
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim] of in_dtype
 *   slot_mapping   [num_tokens] int32; slot < 0 skips the token
 *   k_scale/v_scale  [num_kv_heads] fp32, required iff cache_dtype == FP8
 * (F32 -> F32) and (BF16 -> BF16) copy bytes; (BF16 -> FP8) encodes.
 * Exactly the addressed elements change.  num_tokens == 0 is a no-op.
 */
pa_status_t pa_kv_append(const void* k_new, const void* v_new, pa_dtype_t in_dtype,
                         void* k_cache, void* v_cache, pa_dtype_t cache_dtype,
                         const float* k_scale, const float* v_scale,
                         const int32_t* slot_mapping, int32_t num_tokens,
                         int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, hipStream_t stream);

/*
 * Decode attention, one query token per sequence.
 *   out            [batch][num_heads][head_dim], dtype = q_dtype (unused and
 *                  may be NULL when partition_size > 0)
 *   q              [batch][num_heads][head_dim]
 *   block_tables   [batch][max_blocks_per_seq]; context_lens [batch]
 *   scale          multiplies q . k (e.g. 1/sqrt(head_dim) rounded to fp32)
 *   partition_size 0: one pass per (sequence, KV head) writes `out`.
 *                  > 0 (a multiple of 16): split-K; partition p covers
 *                  positions [p*PS, min(L, (p+1)*PS)) and writes, for every
 *                  query head, m_p = max of scale*q.k (natural units),
 *                  l_p = sum exp(s - m_p) and o_p = sum exp(s - m_p) v / l_p
 *                  into part_max/part_sum [batch][num_heads][max_partitions]
 *                  and part_out [batch][num_heads][max_partitions][head_dim]
 *                  (fp32).  Partitions at or past ceil(L / PS) are not written.
 *   max_partitions >= ceil(max_b L_b / PS) (host-known bound; sizes the grid)
 * A context length beyond max_blocks_per_seq * 16 (or, split-K, beyond
 * max_partitions * PS) is cut there: nothing past the table row or the
 * partial buffers is read or written.
 */
pa_status_t pa_decode(void* out, const void* q, pa_dtype_t q_dtype,
                      const void* k_cache, const void* v_cache, pa_dtype_t cache_dtype,
                      const float* k_scale, const float* v_scale,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch,
                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, float scale,
                      int32_t partition_size, int32_t max_partitions,
                      float* part_max, float* part_sum, float* part_out,
                      hipStream_t stream);

/*
 * Append and decode in one launch: the same pool bytes and results as
 * pa_kv_append of each sequence's newest token followed by pa_decode, for
 * the layer-step of a decode batch (llm-infer, "What It Does": the captured
 * per-layer decode graph writes the KV cache beside attention).  The
 * wavefront that reads the block of position L_b - 1 for KV head h writes
 * that token there first, so no other launch or synchronisation is needed.
 *   k_new, v_new   [batch][num_kv_heads][head_dim] of q_dtype: sequence b's
 *                  newest token (position L_b - 1)
 *   new_slots      [batch] int32: that token's slot, which must be position
 *                  L_b - 1 of b's block table, or -1 when its K/V are already
 *                  in the pool (e.g. a token inside a prefix-shared block).
 *                  Any other value writes nothing.
 *                  k_new, v_new and new_slots all NULL: no append.
 *   plan           NULL, or a launch plan pa_decode_plan made (entry
 *                  PA_PLAN_DECODE_APPEND) for the same
 *                  block_tables, context_lens, batch, heads, head_dim,
 *                  cache dtype, partition_size and max_partitions on this
 *                  device: the launch then skips its prologue (see
 *                  pa_decode_plan).  A plan whose header does not match
 *                  these arguments makes the launch append and compute
 *                  nothing and write NaN to every element of `out` (single
 *                  pass) or of the three partial buffers (split-K), so the
 *                  mistake shows in the results instead of passing silently.
 *   plan_bytes     the plan buffer's size; less than pa_decode_plan_bytes
 *                  for this batch returns PA_ERR_ARG
 * Other arguments, outputs, layouts and errors as pa_decode; the pools are
 * written (fp8 caches encode as pa_kv_append does).
 */
pa_status_t pa_decode_append(void* out, const void* q, pa_dtype_t q_dtype,
                             const void* k_new, const void* v_new, const int32_t* new_slots,
                             void* k_cache, void* v_cache, pa_dtype_t cache_dtype,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t batch,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale,
                             int32_t partition_size, int32_t max_partitions,
                             float* part_max, float* part_sum, float* part_out,
                             const int32_t* plan, size_t plan_bytes, hipStream_t stream);

/*
 * Launch plans.  Every layer of a decode step runs the same batch: the same
 * context lengths, block tables, prefix groups and query map.  The decode
 * prologue depends only on those and the launch shape: the row table in
 * LDS, the prefix of tiles, each workgroup's and wavefront's tile range, and
 * the block ids of each wavefront's first two tiles.  pa_decode_plan
 * computes it once, with the decode kernel's own prologue, and writes it to
 * `plan`.  The decode entry named by `entry` then reads it when given the
 * plan, which saves the per-launch prologue for every layer.  This is the
 * plan-once, run-per-layer split of the engines the pages build on
 * (llm-infer, "What It Does": the decode step replayed for every layer).
 *   plan        int32 device buffer of at least pa_decode_plan_bytes(rows,
 *               cache_dtype, head_dim) bytes, rows = batch (+ num_groups for
 *               the cascade).  The workgroup count depends on the device's
 *               compute units.
 *   entry       the decode entry point that will use the plan
 *   new_slots   NULL, or the new_slots the launches will append with: the
 *               plan then lists, per wavefront, the tokens it writes (checked
 *               against the tables once; a wavefront with more than 8 finds
 *               them again in the launch), so the launch loads all their
 *               rows at once
 *   group_*, num_groups, max_group_size   the cascade's groups (else NULL, 0)
 *   query_start_loc, max_query_len        pa_decode_multi's query map (else
 *                                         NULL, 0)
 *   other arguments as that entry point (Q, K/V and scales are not read)
 * Plans for prefix-group and multi-query rows also balance cost rather than
 * tiles across workgroups: an item counts one extra tile, for its Q load and
 * its partial write, so many short items weigh like a few long ones, and one
 * more when it ends a (virtual) head whose token the launch appends.
 * The plan stays valid while context_lens, the first ceil(L_b / 16)
 * block-table entries of every row, new_slots, and the groups or query map
 * are unchanged.  It follows the stream: the plan launch must precede its users
 * on that stream, or be otherwise ordered before them.
 */
size_t pa_decode_plan_bytes(int32_t rows, pa_dtype_t cache_dtype, int32_t head_dim);
pa_status_t pa_decode_plan(int32_t* plan, size_t plan_bytes, pa_plan_entry_t entry,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t batch,
                           const int32_t* new_slots,
                           const int32_t* group_start, const int32_t* group_seqs,
                           const int32_t* group_prefix_lens, int32_t num_groups,
                           int32_t max_group_size, const int32_t* query_start_loc,
                           int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, pa_dtype_t cache_dtype, int32_t partition_size,
                           int32_t max_partitions, hipStream_t stream);

/*
 * Shared-prefix ("cascade") split-K decode: the same partials as pa_decode
 * with partition_size > 0, for a batch in which prefix groups of sequences
 * share their first tokens in the same physical blocks (infer-lab, technique
 * table, RadixAttention row: prefix reuse across requests; llm-infer, "What
 * It Does": prefix caching; InferX, "Status": a radix prefix cache;
 * RustInfer, "Architecture": the scheduler's RadixTree prefix cache).  The
 * whole partitions of a group's shared prefix are read once per KV head for
 * up to 16 / G members at a time instead of once per member; every other
 * partition is computed as pa_decode computes it.  Merge with
 * pa_decode_splitk_reduce.
 *   group_start        [num_groups + 1] int32: members of group j are
 *                      group_seqs[group_start[j] .. group_start[j+1])
 *   group_seqs         member sequence indices (< batch); a sequence belongs
 *                      to at most one group
 *   group_prefix_lens  [num_groups] int32: positions 0 .. P_j - 1 of every
 *                      member are the same tokens in the same blocks (the
 *                      members' block-table rows agree on the first
 *                      ceil(P_j / 16) entries) and P_j <= each member's L.
 *                      Only floor(P_j / partition_size) whole partitions are
 *                      taken as shared; the rest is read per member.
 *   max_group_size     host bound on members per group (sizes the grid)
 * Requires partition_size > 0 (PA_ERR_ARG otherwise) and
 * batch + num_groups <= 4096 (PA_ERR_UNSUPPORTED otherwise).  num_groups == 0
 * computes exactly what pa_decode computes.
 */
/* k_new, v_new, new_slots: NULL, or each sequence's newest token appended
 * in the same launch, as pa_decode_append does (a token in a prefix-shared
 * block carries slot -1).
 * plan, plan_bytes: NULL / 0, or a plan made with PA_PLAN_DECODE_CASCADE
 * (see pa_decode_plan). */
pa_status_t pa_decode_cascade(const void* q, pa_dtype_t q_dtype,
                              const void* k_new, const void* v_new, const int32_t* new_slots,
                              void* k_cache, void* v_cache, pa_dtype_t cache_dtype,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t batch,
                              const int32_t* group_start, const int32_t* group_seqs,
                              const int32_t* group_prefix_lens, int32_t num_groups,
                              int32_t max_group_size,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, float scale,
                              int32_t partition_size, int32_t max_partitions,
                              float* part_max, float* part_sum, float* part_out,
                              const int32_t* plan, size_t plan_bytes, hipStream_t stream);

/*
 * Multi-query split-K decode: several new query tokens per sequence, causal
 * among themselves, as when a batch of draft tokens is verified in one step
 * (infer-lab, technique table, speculative decoding row: draft proposal
 * and one verification pass of the target; llm-infer, "What It Does":
 * prompt-lookup speculative decoding; RustInfer, configuration options:
 * multi-token-prediction draft tokens).  Sequence b's q_b = query_start_loc[b+1] - query_start_loc[b]
 * tokens are rows query_start_loc[b] .. +q_b-1 of q, at positions
 * L_b - q_b .. L_b - 1; the token at position P sees positions 0 .. P.
 * Their K/V are appended beforehand or by this launch (below).  Each
 * (K/V tile, KV head) is read once
 * for up to 16 / G of a sequence's query tokens.
 *   q                  [query_start_loc[batch]][num_heads][head_dim]
 *   part_*             [query_start_loc[batch]][num_heads][max_partitions]
 *                      (+ [head_dim]): per query token, as pa_decode writes
 *                      them for a context of P + 1 positions; partitions at or
 *                      past ceil((P + 1) / partition_size) are not written.
 *                      Merge with pa_decode_splitk_reduce over
 *                      batch = query_start_loc[batch] rows whose context
 *                      lengths are the tokens' P + 1.
 *   max_query_len      host bound on q_b, <= 64 (PA_ERR_UNSUPPORTED beyond;
 *                      longer chunks are prefill: pa_prefill_chunk)
 * Requires partition_size > 0 and q_b <= L_b.
 */
/* k_new, v_new, new_slots: NULL, or the query tokens' own K/V appended in
 * the same launch, with the pool bytes and results of pa_kv_append of
 * them followed by this call (all three NULL: no append).
 *   k_new, v_new   [query_start_loc[batch]][num_kv_heads][head_dim] of
 *                  q_dtype, rows as q's
 *   new_slots      [query_start_loc[batch]] int32: the token's slot, which
 *                  must be its position's slot in b's block table, or -1
 *                  when its K/V are already in the pool; any other value
 *                  writes nothing
 * Every wavefront that reads a tile holding one of b's query positions for
 * KV head h writes b's query tokens for h first (the same bytes whichever
 * writes them), so no other launch or synchronisation is needed.
 * plan, plan_bytes: NULL / 0, or a plan made with PA_PLAN_DECODE_MULTI
 * (see pa_decode_plan). */
pa_status_t pa_decode_multi(const void* q, pa_dtype_t q_dtype,
                            const void* k_new, const void* v_new, const int32_t* new_slots,
                            const int32_t* query_start_loc, int32_t max_query_len,
                            void* k_cache, void* v_cache, pa_dtype_t cache_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, float scale,
                            int32_t partition_size, int32_t max_partitions,
                            float* part_max, float* part_sum, float* part_out,
                            const int32_t* plan, size_t plan_bytes, hipStream_t stream);

/*
 * Merge split-K partials (the layout pa_decode writes) into out
 * [batch][num_heads][head_dim] of out_dtype (F32 or BF16):
 *   M = max_p m_p,  w_p = l_p * exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p
 * over p < ceil(L_b / partition_size); L_b == 0 writes zeros.
 * Supports max_partitions <= 4096.
 */
pa_status_t pa_decode_splitk_reduce(void* out, pa_dtype_t out_dtype,
                                    const float* part_max, const float* part_sum,
                                    const float* part_out, const int32_t* context_lens,
                                    int32_t batch, int32_t num_heads, int32_t head_dim,
                                    int32_t partition_size, int32_t max_partitions,
                                    hipStream_t stream);

/*
 * Causal attention of prefill chunks over the paged cache (their own K/V
 * already appended).  Chunk c owns query rows query_start_loc[c] ..
 * query_start_loc[c+1]-1 (C_c rows, C_c <= max_query_len) and has context
 * length context_lens[c] = P_c + C_c; its row i (position P_c + i) attends
 * to positions 0 .. P_c + i.
 *   out, q         [query_start_loc[num_chunks]][num_heads][head_dim]
 *   block_tables   [num_chunks][max_blocks_per_seq]
 * A context length is taken as at most max_blocks_per_seq * block_size, as
 * in pa_decode: positions past the block-table row are never read.  A chunk
 * whose rows then outnumber its context (C_c > context) writes nothing.
 */
pa_status_t pa_prefill_chunk(void* out, const void* q, pa_dtype_t q_dtype,
                             const int32_t* query_start_loc, int32_t num_chunks,
                             int32_t max_query_len,
                             const void* k_cache, const void* v_cache, pa_dtype_t cache_dtype,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, float scale, hipStream_t stream);

/*
 * Split-K decode that allocates nothing, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid it) and so cannot pass pa_decode's partial buffers.  It is
 * pa_decode with partition_size > 0 followed by pa_decode_splitk_reduce,
 * with the partials in a fixed scratch array that the library holds in each
 * GPU's memory until the process ends; `out` gets the same bits those two
 * calls give.
 *   out            [batch][num_heads][head_dim] of q_dtype
 *   partition_size > 0, a multiple of 16 (PA_ERR_ARG otherwise)
 *   other arguments as pa_decode
 * Requires the partials to fit the scratch: 256-aligned part_max and part_sum
 * of batch * num_heads * max_partitions floats each, then part_out of
 * head_dim times that, within pa_decode_noalloc_max_bytes() = 64 MiB (e.g.
 * batch 8, 32 heads, head_dim 128, 256 partitions: 32.5 MiB).  Larger sizes
 * return PA_ERR_TOO_LARGE before anything is launched.  Calls on one GPU
 * share its scratch, so calls that overlap on one GPU (other streams, other
 * threads) race; calls ordered on one stream do not.
 */
pa_status_t pa_decode_noalloc(void* out, const void* q, pa_dtype_t q_dtype,
                              const void* k_cache, const void* v_cache, pa_dtype_t cache_dtype,
                              const float* k_scale, const float* v_scale,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t batch,
                              int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, float scale,
                              int32_t partition_size, int32_t max_partitions,
                              hipStream_t stream);

/* The size of pa_decode_noalloc's scratch on each GPU, in bytes. */
size_t pa_decode_noalloc_max_bytes(void);

/*
 * Measurement aid, not part of the attention path: reads num_chunks 4 KB
 * chunks of buf (chunk i at byte offset chunk_ids[i] * 4096) in that order,
 * one workgroup of four wavefronts per compute unit, each wavefront keeping
 * eight chunks in flight -- the access pattern of the decode's K/V block
 * tiles.  Timing it gives the HBM read bandwidth this pattern can reach, the
 * context for a roofline fraction taken against the published peak.  Every
 * chunk id must be < bytes / 4096 (device contents are trusted).
 *   sink   at least (compute units * 256) words; receives per-thread folds
 *          of the data read (keeps the loads live), no meaning otherwise
 */
pa_status_t pa_read_probe(const void* buf, size_t bytes, const int32_t* chunk_ids,
                          int32_t num_chunks, uint32_t* sink, size_t sink_bytes,
                          hipStream_t stream);

/*
 * Name of a status code: a static string, never NULL.  Every call above
 * reports an argument, shape or launch problem as a status the caller can
 * name, instead of falling back to another path (RustInfer, "Tensor
 * parallelism": unsupported combinations fail with a clear error rather than
 * silently falling back; infer-lab, technique table: a feature that is not
 * available says so, with a reason).
 */
const char* pa_status_string(pa_status_t status);

/*
 * Bytes of part_max + part_sum + part_out for a split-K decode (fp32):
 * batch * num_heads * max_partitions * (head_dim + 2) * 4.  The caller
 * allocates this scratch once and passes it to every layer's launch; the
 * library allocates no temporary device storage per step (RustInfer,
 * "Architecture": attention kernels take caller-owned, graph-safe scratch
 * and allocate nothing themselves).  0 for a negative argument.
 */
size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim,
                                 int32_t max_partitions);

/*
 * Runs a one-wave kernel on the current device and checks its result:
 * PA_ERR_LAUNCH when no gfx950 code object loads.  A build for the wrong
 * target fails here, loudly, rather than at the first attention call or
 * silently (RustInfer, "Tensor parallelism": fail instead of silently falling
 * back).
 */
pa_status_t pa_selftest(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */

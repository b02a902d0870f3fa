/*
 * cpattn.h — C ABI of the MI355X (gfx950) library for one context-parallel
 * rank's exact blockwise attention.
 *
 * The problem these calls solve is the one stated on the FCP page
 * ("从固定环到自由拓扑：FCP到底在解决什么", §3.3): a rank keeps its local query
 * shard, KV blocks of the other ranks arrive one at a time in an order the
 * communication graph decides, and each arriving block is folded into the
 * running softmax state so that the final result equals ordinary attention
 * whatever the order. Masking is causal by GLOBAL token position (PCP page
 * "大模型长序列显存优化：PCP与DCP序列并行实战指南", §3.5: positions stay global
 * after the split; zig-zag page "大模型长上下文训练的挑战与突破", §4.2: a token
 * sees only earlier tokens). Query heads may share KV heads (GQA) without
 * copying them (Halo page "长上下文训练 256k 不难：Halo 上下文并行（CP + Ulysses
 * 注意力）原理与实测", Ulysses section).
 *
 * Conventions shared by every call
 *  - Q and O are [lq][hq][head_dim], K and V are [lk][hkv][head_dim], all
 *    row-major and contiguous; LSE is [hq][lq] float32.
 *  - Query head h reads KV head h / (hq / hkv).
 *  - scores are scale * <q, k>; LSE is the natural log of the softmax
 *    normaliser, LSE = max + ln(sum of exp(score - max)).
 *  - A query row with no visible key in a call has O = 0 and LSE = -inf; a
 *    merge gives such a partial zero weight, so no NaN is ever produced.
 *  - Positions are int32, ascending within each array (the kernels find the
 *    visible key range by binary search and rely on it).
 *
 * Ownership: the caller allocates and owns every buffer. Device pointers are
 * plain HIP device allocations on the current device; host pointers are
 * plain host memory. The library keeps no state between calls and allocates
 * no device memory.
 *
 * Errors: every argument is checked on the host before anything is enqueued.
 * A non-OK status means nothing was enqueued; cpattn_last_error() returns a
 * message for the calling thread. CPATTN_OK means the work is enqueued on
 * `stream` (a hipStream_t; NULL = the default stream); device-side faults
 * surface at the caller's next synchronisation. With the environment variable
 * CPATTN_VALIDATE=1 the calls also copy the position arrays to the host and
 * check that they are ascending (this synchronises the stream).
 *
 * Calls are reentrant; the error text is thread-local.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CPATTN_OK = 0,
    CPATTN_ERR_NULL = 1,      /* a required pointer is NULL */
    CPATTN_ERR_SHAPE = 2,     /* sizes inconsistent, unsupported head_dim, or not divisible */
    CPATTN_ERR_DTYPE = 3,     /* unsupported dtype or dtype combination */
    CPATTN_ERR_UNSORTED = 4,  /* positions or offsets not ascending */
    CPATTN_ERR_RANGE = 5,     /* rank, cp size, layout or flag out of range */
    CPATTN_ERR_HIP = 6,       /* a HIP runtime call failed; the message holds hipGetErrorString */
    CPATTN_ERR_ALIGN = 7,     /* a pointer is misaligned (16 bytes for tensors, 4 for int32/float32 arrays) */
    CPATTN_ERR_ALIAS = 8      /* an output overlaps an input */
} cpattn_status;

typedef enum { CPATTN_BF16 = 0, CPATTN_F32 = 1 } cpattn_dtype;

typedef enum { CPATTN_CONTIGUOUS = 0, CPATTN_ZIGZAG = 1, CPATTN_STRIPED = 2 } cpattn_layout;

/* Library version as major*10000 + minor*100 + patch. */
int cpattn_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *cpattn_last_error(void);

/*
 * Global positions of rank `rank`'s tokens (host memory, no GPU use).
 *
 * Layouts (total_len is S, cp_size is cp):
 *  - CPATTN_CONTIGUOUS: the rank's slice [rank*S/cp, (rank+1)*S/cp) — the
 *    split of the PCP page, §3.5. Needs S % cp == 0.
 *  - CPATTN_ZIGZAG: the sequence is cut into 2*cp equal chunks and the rank
 *    takes chunk `rank` and chunk 2*cp-1-rank, so every rank holds early and
 *    late tokens and the causal work is exactly balanced (zig-zag page, §4.2).
 *    Needs S % (2*cp) == 0.
 *  - CPATTN_STRIPED: tokens t with t % cp == rank, the zig-zag page's literal
 *    example (0, 4, 8, ... on GPU 0 of four). Needs S % cp == 0.
 *
 * cu_seqlens == NULL: one sequence. Otherwise cu_seqlens holds n_seqs+1
 * ascending packed offsets (cu_seqlens[0] == 0, cu_seqlens[n_seqs] == S) and
 * every document is split on its own with `layout`; the rank's tokens of
 * document t follow those of document t-1 (each document length must meet the
 * divisibility rule above).
 *
 * out_pos receives S/cp positions in ascending order. out_seq_start
 * (nullable) receives, per token, the global offset of its document (0
 * without cu_seqlens).
 */
cpattn_status cpattn_zigzag_index(int64_t total_len, int32_t cp_size, int32_t rank, cpattn_layout layout,
                                  const int32_t *cu_seqlens, int32_t n_seqs,
                                  int32_t *out_pos, int32_t *out_seq_start);

/*
 * One arriving KV block folded into a rank's attention state (device memory,
 * enqueued on `stream`). This is the per-block step of the FCP page, §3.3.
 *
 *  q      [lq][hq][head_dim], in_dtype       (bf16 or float32)
 *  k, v   [lk][hkv][head_dim], in_dtype      (this block's keys and values)
 *  q_pos  [lq] int32, k_pos [lk] int32       global positions, ascending;
 *                                            may be NULL only if causal == 0
 *  causal 1: key j is visible to row i iff k_pos[j] <= q_pos[i]; 0: all keys
 *  softmax_scale  <= 0 selects 1/sqrt(head_dim)
 *  o      [lq][hq][head_dim], o_dtype        bf16 input: bf16 or float32 output;
 *                                            float32 input: float32 output
 *  lse    [hq][lq] float32
 *  accumulate 0: write this block's own (O, LSE) (rows with no visible key get
 *             O = 0, LSE = -inf);
 *             1: merge this block into the (O, LSE) already in o/lse, in place:
 *             LSE' = ln(e^LSE + e^LSE_blk), O' = e^(LSE-LSE')·O + e^(LSE_blk-LSE')·O_blk.
 *             Initialise o = 0, lse = -inf (or make the first call with
 *             accumulate = 0) before the first block.
 *
 * head_dim must be 64 or 128; hq % hkv == 0. Fully masked key tiles are never
 * loaded. Outputs must not overlap inputs. With lk == 0 (k, v, k_pos may then
 * be NULL) the block is empty: accumulate = 0 writes O = 0, LSE = -inf and
 * accumulate = 1 leaves the state unchanged. With lq == 0 nothing is done.
 */
cpattn_status cpattn_partial(const void *q, const void *k, const void *v, cpattn_dtype in_dtype,
                             int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim,
                             const int32_t *q_pos, const int32_t *k_pos, int32_t causal, float softmax_scale,
                             void *o, cpattn_dtype o_dtype, float *lse, int32_t accumulate, void *stream);

/*
 * As cpattn_partial with causal == 1, for packed variable-length documents.
 * Ranks whose sequences differ in length (variable-length data) are named by
 * the FCP page ("从固定环到自由拓扑：FCP到底在解决什么", §3.2, the
 * load-balanced graph construction), and packing several documents into one
 * training sequence is the Halo page's packing option ("长上下文训练 256k
 * 不难", its SFT launch commands); a token then attends only within its own
 * document, causally. Here:
 * cu_seqlens (DEVICE memory, n_seqs+1 ascending global packed offsets,
 * cu_seqlens[0] == 0) says where each document starts, and key j is visible to
 * row i iff seq_start(q_pos[i]) <= k_pos[j] <= q_pos[i], where seq_start(p) is
 * the largest offset <= p. Every position must be < cu_seqlens[n_seqs].
 */
cpattn_status cpattn_varlen_partial(const void *q, const void *k, const void *v, cpattn_dtype in_dtype,
                                    int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim,
                                    const int32_t *q_pos, const int32_t *k_pos,
                                    const int32_t *cu_seqlens, int32_t n_seqs, float softmax_scale,
                                    void *o, cpattn_dtype o_dtype, float *lse, int32_t accumulate, void *stream);

/*
 * Workgroups that one cpattn_partial / cpattn_varlen_partial call launches for
 * these sizes (a plan holds one record per workgroup). -1 if the sizes are
 * invalid (lq < 0, hq or hkv < 1, hq % hkv != 0).
 */
int64_t cpattn_partial_workgroups(int64_t lq, int32_t hq, int32_t hkv);

/* int32 entries per workgroup in a document call's plan (cpattn_varlen_plan). */
#define CPATTN_VARLEN_PLAN_RECORD 48

/*
 * HOST memory in and out. The plan of one document call (one KV block) for
 * cpattn_varlen_partial_planned: one record of CPATTN_VARLEN_PLAN_RECORD int32
 * per workgroup, opaque to the caller. A record holds the logical tile the
 * workgroup computes and every range the kernel would otherwise search for at
 * its start (its key range, and per wave the fully visible keys and the
 * document starts of its first and last rows), so a planned workgroup starts
 * with two dependent memory round trips instead of about seven. The order of
 * the records is the dispatch order: with documents a query tile's work
 * follows its place inside its documents, not its global position, so the
 * default heaviest-rows-first order leaves long tiles for the end of a launch;
 * the plan keeps, for each of the 8 XCDs (workgroup id b runs on XCD b % 8),
 * the set of logical tiles the default order gives it (its K/V stays in that
 * XCD's L2) and puts them in decreasing order of the key tiles they load
 * (ties by logical id): longest processing time first. The method is the
 * document masking of cpattn_varlen_partial (FCP page §3.2 and the Halo page's
 * packing option); the plan only schedules it. Positions and cu_seqlens as in
 * cpattn_varlen_partial (ascending; checked here); in_dtype and head_dim as in
 * the call the plan is for (they fix the key-tile size).
 *  plan      receives plan_len int32
 *  plan_len  must be cpattn_partial_workgroups(lq, hq, hkv) x CPATTN_VARLEN_PLAN_RECORD
 * Errors: CPATTN_ERR_SHAPE (sizes, or plan_len), CPATTN_ERR_NULL, CPATTN_ERR_DTYPE,
 * CPATTN_ERR_UNSORTED. Deterministic; positions are fixed for a workload, so a
 * caller plans each block once.
 */
cpattn_status cpattn_varlen_plan(const int32_t *q_pos, int64_t lq, const int32_t *k_pos, int64_t lk,
                                 const int32_t *cu_seqlens, int32_t n_seqs, int32_t hq, int32_t hkv,
                                 int32_t head_dim, cpattn_dtype in_dtype, int32_t *plan, int64_t plan_len);

/*
 * cpattn_varlen_partial with a plan from cpattn_varlen_plan for exactly these
 * positions, document offsets, sizes, in_dtype and head_dim: plan is DEVICE
 * memory, 4-byte aligned, plan_len int32 as above; the caller keeps it alive
 * until the call's work has finished on `stream`. Each logical tile owns its
 * rows and the record's ranges are the ones the kernel's own searches find,
 * so the results are bit-identical to cpattn_varlen_partial's in any record
 * order. A plan made for other positions gives wrong results: every value in
 * it that addresses memory is clamped into range in the kernel, so it never
 * causes an access outside the tensors; with CPATTN_VALIDATE=1 the plan is
 * recomputed on the host and a different one is rejected (CPATTN_ERR_RANGE)
 * before any work.
 */
cpattn_status cpattn_varlen_partial_planned(const void *q, const void *k, const void *v, cpattn_dtype in_dtype,
                                            int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim,
                                            const int32_t *q_pos, const int32_t *k_pos,
                                            const int32_t *cu_seqlens, int32_t n_seqs, float softmax_scale,
                                            void *o, cpattn_dtype o_dtype, float *lse, int32_t accumulate,
                                            const int32_t *plan, int64_t plan_len, void *stream);

/*
 * Several KV blocks that have all arrived, folded into (o, lse) in ONE launch
 * (the FCP page, §3.3: blocks may arrive together and in any order). The
 * result is that of cpattn_partial (cpattn_varlen_partial when cu_seqlens is
 * non-NULL) called on each block in the given order, up to rounding: the
 * running maximum, running sum and the unnormalised O stay in registers
 * between blocks, so O is rounded and written once instead of once per block
 * (and the state of the rows is read once when accumulate = 1).
 *
 *  k_blocks, v_blocks, k_pos_blocks  HOST arrays of n_blocks DEVICE pointers:
 *                     block b is k_blocks[b], v_blocks[b] [lk_blocks[b]][hkv][head_dim]
 *                     and its ascending key positions k_pos_blocks[b] [lk_blocks[b]]
 *  lk_blocks          HOST array of n_blocks lengths (each in [0, 2^31))
 *  n_blocks           1..32
 *  cu_seqlens, n_seqs documents as in cpattn_varlen_partial (causal must be 1), or NULL / 0
 * Every other argument is as in cpattn_partial; each block is checked as a
 * cpattn_partial call would check it. The caller keeps ownership of every
 * buffer; the host arrays are read before the call returns.
 */
cpattn_status cpattn_partial_multi(const void *q, const void *const *k_blocks, const void *const *v_blocks,
                                   cpattn_dtype in_dtype, int64_t lq, const int64_t *lk_blocks, int32_t n_blocks,
                                   int32_t hq, int32_t hkv, int32_t head_dim, const int32_t *q_pos,
                                   const int32_t *const *k_pos_blocks, const int32_t *cu_seqlens, int32_t n_seqs,
                                   int32_t causal, float softmax_scale, void *o, cpattn_dtype o_dtype, float *lse,
                                   int32_t accumulate, void *stream);

/*
 * In place: (o_acc, lse_acc) <- merge((o_acc, lse_acc), (o_part, lse_part)),
 * the exact combination of two partial results over disjoint key sets (the
 * global max / global sum normaliser of the PCP page, §4.2, taken two shards
 * at a time). Commutative, and associative up to rounding, so partials may be
 * merged in any order (FCP page, §3.3). Device memory, enqueued on `stream`.
 *
 *  o_acc, o_part  [lq][hq][head_dim], o_dtype (bf16 or float32)
 *  lse_acc, lse_part [hq][lq] float32
 * head_dim must be 64 or 128. o_part/lse_part must not overlap o_acc/lse_acc.
 */
cpattn_status cpattn_merge_lse(void *o_acc, float *lse_acc, const void *o_part, const float *lse_part,
                               cpattn_dtype o_dtype, int64_t lq, int32_t hq, int32_t head_dim, void *stream);

/*
 * D = <dO, O> of every (row, head), the one per-row quantity the gradients
 * need besides the log-normaliser: the derivative of the softmax
 * normalisation contributes -P·D to every score's gradient. Training with
 * context parallelism runs the backward pass over the same KV blocks as the
 * forward (PCP page, §2.3); D is computed once per step from the final O and
 * its gradient, before the per-block backward calls. Device memory, enqueued
 * on `stream`.
 *
 *  o      [lq][hq][head_dim], o_dtype (bf16 or float32): the merged output
 *  dout   [lq][hq][head_dim], dout_dtype (bf16 or float32): dLoss/dO
 *  delta  [hq][lq] float32 out, summed in float32
 * head_dim must be 64 or 128; delta must not overlap o or dout.
 */
cpattn_status cpattn_bwd_delta(const void *o, cpattn_dtype o_dtype, const void *dout, cpattn_dtype dout_dtype,
                               int64_t lq, int32_t hq, int32_t head_dim, float *delta, void *stream);

/*
 * Gradients of one KV block's part of the attention (device memory, enqueued
 * on `stream`): the backward of cpattn_partial / cpattn_varlen_partial for
 * one block, given the rows' FINAL log-normalisers (after every block was
 * merged) and D from cpattn_bwd_delta. With P = exp(s - LSE) on the visible
 * pairs and dS = P (dO·v - D):
 *     dQ += scale · dS K   (this block's share; summed over blocks),
 *     dK  = scale · dS^T Q,  dV = P^T dO   (complete for this block's keys
 *                                          once every local row is seen).
 * Query heads sharing a KV head add into its dK, dV (GQA).
 *
 *  q, dout  [lq][hq][head_dim], k, v [lk][hkv][head_dim], all in_dtype (bf16 or float32)
 *  q_pos, k_pos, causal, cu_seqlens, n_seqs   masks as in cpattn_partial
 *                (cu_seqlens == NULL: no documents; otherwise DEVICE offsets
 *                as in cpattn_varlen_partial, and causal must be 1)
 *  softmax_scale <= 0 selects 1/sqrt(head_dim)
 *  lse    [hq][lq] float32, the merged LSE of the forward (a row with -inf
 *         sees no key and gets no gradient)
 *  delta  [hq][lq] float32 from cpattn_bwd_delta
 *  dq     [lq][hq][head_dim] float32; accumulate_dq 0: written, 1: added to
 *  dk, dv [lk][hkv][head_dim] float32; accumulate_dkv 0: written, 1: added to
 *
 * bf16 inputs run bf16 matrix products (P and dS rounded to bf16 for them),
 * float32 inputs float32 ones (every step in float32); head_dim 64 or 128;
 * hq % hkv == 0. Outputs must not overlap the inputs or each other. lq == 0:
 * dk, dv get zeros (or are left as they are when accumulating); lk == 0
 * likewise for dq. The two kernels (keys, then queries) write disjoint
 * outputs with no atomics: results are identical from run to run.
 */
cpattn_status cpattn_partial_bwd(const void *q, const void *k, const void *v, const void *dout, cpattn_dtype in_dtype,
                                 int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t head_dim,
                                 const int32_t *q_pos, const int32_t *k_pos, int32_t causal,
                                 const int32_t *cu_seqlens, int32_t n_seqs, float softmax_scale,
                                 const float *lse, const float *delta,
                                 float *dq, int32_t accumulate_dq, float *dk, float *dv, int32_t accumulate_dkv,
                                 void *stream);

/*
 * Workgroups of the query-gradient kernel of a cpattn_partial_bwd call: the
 * length of a plan for cpattn_varlen_partial_bwd_planned (one int32 per
 * workgroup; 128 query rows of one query head each). -1 for invalid sizes.
 */
int64_t cpattn_bwd_query_workgroups(int64_t lq, int32_t hq);

/*
 * Host-side plan of a gradient call with documents (the backward of
 * cpattn_varlen_partial; PCP page, §2.3, and the FCP page's load balance
 * over variable-length sequences, §3.2). With documents, a query tile's work
 * is the keys from its first row's document start to its last row, so the
 * query kernel's position order leaves long tiles for the end of a launch.
 * The plan is the query kernel's dispatch order: plan[b] is the logical tile
 * workgroup b computes. For each XCD (workgroup b runs on XCD b % 8) it keeps
 * the set of tiles the default order gives that XCD, ordered by the key tiles
 * they load, most first (ties by tile id). The plan changes only the order,
 * so planned and unplanned calls give bit-identical results.
 *
 *  q_pos [lq], k_pos [lk], cu_seqlens [n_seqs + 1]  HOST int32 arrays, ascending
 *  plan  HOST int32 [plan_len], written; plan_len = cpattn_bwd_query_workgroups(lq, hq)
 * Errors: CPATTN_ERR_SHAPE (sizes, plan_len), CPATTN_ERR_NULL, CPATTN_ERR_UNSORTED.
 * A plan depends only on the positions, so it is made once per block.
 */
cpattn_status cpattn_varlen_bwd_plan(const int32_t *q_pos, int64_t lq, const int32_t *k_pos, int64_t lk,
                                     const int32_t *cu_seqlens, int32_t n_seqs, int32_t hq, int32_t hkv,
                                     int32_t *plan, int64_t plan_len);

/*
 * cpattn_partial_bwd with documents (causal = 1, cu_seqlens DEVICE, required)
 * and the query kernel dispatched in the order of `plan` (DEVICE int32
 * [plan_len], from cpattn_varlen_bwd_plan for the same positions; caller
 * owns it). Results are those of the unplanned call, bit for bit. Every
 * tile id read from the plan is clamped into range, so a plan for other
 * positions gives wrong results but no access outside the tensors; with
 * CPATTN_VALIDATE=1 the call recomputes the plan on the host and rejects a
 * different one (CPATTN_ERR_RANGE) before any work. float32 inputs run in
 * the default order. Other arguments and errors as in cpattn_partial_bwd.
 */
cpattn_status cpattn_varlen_partial_bwd_planned(const void *q, const void *k, const void *v, const void *dout,
                                                cpattn_dtype in_dtype, int64_t lq, int64_t lk, int32_t hq,
                                                int32_t hkv, int32_t head_dim, const int32_t *q_pos,
                                                const int32_t *k_pos, const int32_t *cu_seqlens, int32_t n_seqs,
                                                float softmax_scale, const float *lse, const float *delta,
                                                float *dq, int32_t accumulate_dq, float *dk, float *dv,
                                                int32_t accumulate_dkv, const int32_t *plan, int64_t plan_len,
                                                void *stream);

/*
 * The gradients of several KV blocks that are all present, in one call: the
 * backward pass runs over the same blocks as the forward (PCP page, §2.3),
 * and, as in cpattn_partial_multi, blocks may be present together (FCP page,
 * §3.3). The result is that of cpattn_partial_bwd called on each block in
 * the given order (the first call with accumulate_dq, the others adding to
 * dq), up to rounding: dk, dv of every block come out bit for bit as from
 * that call; dq is summed over the blocks in float32 registers and written
 * (or added) once, where the per-block calls round and store it after every
 * block. Two launches: one key-gradient grid over all blocks' keys, then one
 * query-gradient grid whose workgroups walk the blocks in order.
 *
 *  k_blocks, v_blocks, k_pos_blocks, lk_blocks, n_blocks   as in cpattn_partial_multi
 *                     (n_blocks 1..32)
 *  dk_blocks, dv_blocks  HOST arrays of n_blocks DEVICE pointers: block b's
 *                     dk, dv [lk_blocks[b]][hkv][head_dim] float32
 * Every other argument is as in cpattn_partial_bwd, and each block is checked
 * as a cpattn_partial_bwd call would check it. A block's dk and dv must not
 * overlap another block's buffers either (CPATTN_ERR_ALIAS). float32 inputs
 * run the single-block kernels block after block. The caller keeps ownership
 * of every buffer; the host arrays are read before the call returns.
 */
cpattn_status cpattn_partial_bwd_multi(const void *q, const void *const *k_blocks, const void *const *v_blocks,
                                       const void *dout, cpattn_dtype in_dtype, int64_t lq, const int64_t *lk_blocks,
                                       int32_t n_blocks, int32_t hq, int32_t hkv, int32_t head_dim,
                                       const int32_t *q_pos, const int32_t *const *k_pos_blocks, int32_t causal,
                                       const int32_t *cu_seqlens, int32_t n_seqs, float softmax_scale,
                                       const float *lse, const float *delta, float *dq, int32_t accumulate_dq,
                                       float *const *dk_blocks, float *const *dv_blocks, int32_t accumulate_dkv,
                                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */

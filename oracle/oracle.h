/*
 * oracle.h — the CPU fp64 reference for one context-parallel rank's exact
 * attention. TEST INFRASTRUCTURE ONLY: nothing on the product path may link,
 * load or call this library. Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark use it.
 *
 * Sources (cited by page title and section):
 *  [FCP]    "从固定环到自由拓扑：FCP到底在解决什么" (lqnn.cn), §3.3 — blockwise
 *           accumulation over KV blocks that arrive in any order, with the
 *           result required to equal ordinary (serial) attention.
 *  [PCP]    "大模型长序列显存优化：PCP与DCP序列并行实战指南" (hmyw.cn), §2.3 and
 *           §4.2 — the cross-shard softmax normaliser (global max, then global
 *           sum); §3.5 — contiguous split and global positions.
 *  [ZIGZAG] "大模型长上下文训练的挑战与突破" (intelliparadigm.com), §4.2 —
 *           causal masking (a token sees only earlier tokens) and the zig-zag
 *           assignment that mixes early and late tokens on each GPU.
 *  [HALO]   "长上下文训练 256k 不难：Halo 上下文并行（CP + Ulysses 注意力）原理与实测"
 *           (sheratonhq.com), Ulysses section — heads are independent, grouped
 *           KV heads are shared without copying.
 *  The gradients (oracle_attention_grad) are those of the same definition:
 *  the backward pass that training with context parallelism runs over the
 *  same KV blocks ([PCP] §2.3).
 *
 * Everything is the plain definition: scores in fp64 from the exact input
 * values, a max pass, a sum pass, a weighted-sum pass. No tiling, no online
 * rescaling, no shared code with the GPU library.
 */
#ifndef CPATTN_ORACLE_H
#define CPATTN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_CONTIGUOUS = 0, ORACLE_ZIGZAG = 1, ORACLE_STRIPED = 2 };
enum { ORACLE_IN_BF16 = 0, ORACLE_IN_F32 = 1 };

/* Global positions of rank `rank`'s tokens, ascending, by closed form.
 * doc_lens == NULL: one sequence of length S. Otherwise n_docs documents whose
 * lengths sum to S; each document is split on its own with `layout` and the
 * rank's tokens of document t follow those of document t-1.
 * out_start (nullable) receives the global start of each token's document.
 * Returns the number of local tokens, or -1 if S (or a document length) is
 * not divisible as the layout requires. */
int64_t oracle_local_positions(int64_t S, int32_t cp, int32_t rank, int32_t layout,
                               const int64_t *doc_lens, int32_t n_docs,
                               int32_t *out_pos, int32_t *out_start);

/* Exact attention for a list of (query row, query head) pairs.
 * q: [lq][hq][d], k, v: [lk][hkv][d] as bf16 bit patterns (in_dtype 0) or
 * float32 (in_dtype 1); values are widened exactly to fp64.
 * A key j is visible to row i iff causal == 0, or k_pos[j] <= q_pos[i] and
 * (q_start == NULL or k_pos[j] >= q_start[i]).
 * Query head h reads KV head h / (hq / hkv).
 * rows/heads == NULL: every (i, h), in order i*hq + h.
 * Outputs per requested pair n: o[n*d + t], lse[n] (natural log),
 * n_visible[n] (nullable). A pair with no visible key gets o = 0, lse = -inf.
 * Returns 0, or -1 on bad arguments. */
int oracle_attention(const void *q, const void *k, const void *v, int32_t in_dtype,
                     int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                     const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                     int32_t causal, double scale,
                     const int64_t *rows, const int32_t *heads, int64_t n_pairs,
                     double *o, double *lse, int64_t *n_visible, int32_t n_threads);

/* Softmax weights of one (row, head) over all lk keys: p[j] (0 where not
 * visible). Returns the number of visible keys. */
int64_t oracle_softmax_row(const void *q, const void *k, int32_t in_dtype,
                           int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                           const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                           int32_t causal, double scale, int64_t row, int32_t head, double *p);

/* Merge of two normalised partial results of the same rows (fp64):
 * L = log(e^La + e^Lb); O = e^(La-L) Oa + e^(Lb-L) Ob. A -inf side has weight
 * zero; both -inf gives (0, -inf). Output may alias either input. */
void oracle_merge(int64_t n_rows, int32_t d,
                  const double *o_a, const double *lse_a,
                  const double *o_b, const double *lse_b,
                  double *o_out, double *lse_out);

/* Gradients of the attention above for a loss whose gradient with respect to
 * O is dout ([lq][hq][d], fp64). Masking, GQA and dtype as oracle_attention.
 * rows/heads == NULL: every (i, h), in order i*hq + h, and dk, dv (nullable,
 * [lk][hkv][d]) receive the key gradients summed over the query heads of each
 * KV head. With a rows/heads list only dq (and delta) of those pairs are
 * computed; dk and dv must then be NULL.
 * dq (nullable): [n_pairs][d]; delta (nullable): [n_pairs], D = <dO, O>.
 * A pair with no visible key gets dq = 0 and delta = 0.
 * Returns 0, or -1 on bad arguments. */
int oracle_attention_grad(const void *q, const void *k, const void *v, int32_t in_dtype,
                          int64_t lq, int64_t lk, int32_t hq, int32_t hkv, int32_t d,
                          const int32_t *q_pos, const int32_t *q_start, const int32_t *k_pos,
                          int32_t causal, double scale, const double *dout,
                          const int64_t *rows, const int32_t *heads, int64_t n_pairs,
                          double *dq, double *dk, double *dv, double *delta, int32_t n_threads);

#ifdef __cplusplus
}
#endif
#endif

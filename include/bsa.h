/*
 * bsa.h - C ABI of the gfx950 (MI355X) block-sparse self-attention library.
 *
 * What is computed (per batch b and head h, sequence of N tokens, head_dim 128):
 *   1. the sequence is cut into blocks of 128 tokens (the last may be short);
 *      Q, K and V are mean-pooled per block;
 *   2. every query block scores every key block with the dot product of the
 *      pooled vectors and keeps its top_k key blocks;
 *   3. each query attends exactly to every token of its kept key blocks;
 *   4. every key block it did not keep enters the same softmax as one summary
 *      row (mean-pooled, or Spark-Reweight weighted with a log-mass bias).
 * Sources: "h3-sparse-attn 0.1.0" (PyPI page), opening paragraph and section
 * "Use" (top-k 128-token key blocks, one summary row per skipped block; bf16,
 * head_dim 128, forward only); "Spark-H3: Block Sparse Attention Speeds Up
 * MiniMax-H3 in ComfyUI", section "What Spark-Attn changes" (exact branch over
 * the top-ranked blocks, compressed branch for the rest, Spark-Reweight).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises, and keeps no state between calls
 *     (apart from the name of the last HIP error, per thread, for
 *     bsa_hip_error_str).
 *   - Tensors are contiguous.  Q, K, V and out are [B, H, N, 128] bfloat16
 *     (raw 16-bit storage), row-major with the feature dimension fastest.
 *   - nb = ceil(N / 128); k = min(top_k, nb) without conditioning sinks, else
 *     k = n_sink + min(top_k, nb - n_sink) (see bsa_problem.sink_rows).
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and no output is touched.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the null stream).  A failed launch returns BSA_ERR_HIP.  Streams and
 *     device memory must come from the HIP runtime the library is bound to:
 *     a process that also loads torch's bundled runtime maps it before
 *     this library, so that the library binds to that one runtime.
 *   - Results are bit-deterministic: no floating-point atomics.
 *   - Calls on one stream are ordered; the caller orders calls on different
 *     streams that share buffers.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_BLOCK 128
#define BSA_HEAD_DIM 128
/* largest supported number of blocks per sequence (N <= 262144 tokens) */
#define BSA_MAX_BLOCKS 2048
/* largest supported number of extra tokens per query block */
#define BSA_MAX_EXTRA 256

enum {
  BSA_OK = 0,
  BSA_ERR_INVALID = 1,      /* bad pointer, size, range or mode */
  BSA_ERR_UNSUPPORTED = 2,  /* head_dim or block size other than 128, or N too large */
  BSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than bsa_workspace_bytes */
  BSA_ERR_HIP = 4,          /* a HIP launch failed */
  BSA_ERR_SCRATCH = 5       /* bsa_forward_noalloc: problem larger than its static scratch */
};

enum { BSA_SUMMARY_MEAN = 0, BSA_SUMMARY_REWEIGHT = 1 };

typedef struct bsa_problem {
  int32_t batch;       /* B >= 1 */
  int32_t heads;       /* H >= 1 */
  int32_t seq_len;     /* N >= 1; any N, the last block may be short */
  int32_t head_dim;    /* must be 128 */
  int32_t block_size;  /* must be 128 */
  int32_t top_k;       /* >= 0, counts key blocks; capped at nb */
  int32_t summary;     /* BSA_SUMMARY_MEAN or BSA_SUMMARY_REWEIGHT */
  int32_t anchor_rows; /* reweight: anchor = mean of query rows [0, anchor_rows);
                          0 means N; must lie in [0, N] */
  float scale;         /* softmax scale; 0 means 1/sqrt(head_dim); else > 0, finite */
  /* Conditioning sinks: the rows [sink_start, sink_start + sink_rows) are
   * conditioning rows (prompt, reference, audio).  The n_sink blocks holding
   * any of them are sink blocks: every query block keeps all of them exactly,
   * on top of the top_k it picks among the other blocks, and a query block
   * that is a sink block attends to every key block exactly.  sink_rows = 0
   * (with sink_start 0) means no sinks: pure top-k.  The range must lie in
   * [0, N].  Sources: "H3 Sparse Attention" (WAS Node Suite node page),
   * section "The inputs that matter" (with sink_conditioning on, the
   * prompt, reference and audio rows are attended exactly and their own
   * queries attend densely); "H3 Sparse
   * Attention" (node page on video budgets), opening section (conditioning
   * and non-video queries, and the tiles on the boundary between contexts,
   * stay dense). */
  int32_t sink_start;
  int32_t sink_rows;
  /* Block selection rule.  BSA_SELECT_TOPK: the top_k blocks of largest
   * score.  BSA_SELECT_THRESHOLD (variable k): the blocks whose score exceeds
   * mean + select_tau * std of their row's nb block scores (population
   * statistics, float64), at most top_k of them (largest first), so rows keep
   * different numbers of blocks and are padded with -1.  Source: "H3 Sparse
   * Attention" (WAS Node Suite node page), section "The inputs that matter"
   * (the share of key blocks kept exact is given as about 16% at tau 1.0,
   * 7% at 1.5 and 3% at 2.0: the normal tail beyond tau standard
   * deviations). */
  int32_t select_mode;
  float select_tau;    /* threshold mode only; finite */
  /* Extra tokens, in [0, BSA_MAX_EXTRA]: besides its kept blocks, each query
   * block attends exactly to the extra_tokens tokens of the blocks it skipped
   * whose keys score highest against its pooled query (q_pool[r] . k_j);
   * those blocks keep their summary rows.  0 turns the option off.  Used by
   * bsa_select_tokens and bsa_forward_tokens; bsa_forward rejects a problem
   * with extra tokens.  Source: "H3 Sparse Attention" (WAS Node Suite node
   * page), section "The inputs that matter" (extra_tokens: per query block,
   * that many individually highest-scoring tokens on top of its selected
   * blocks; 256 by default, 0 the fastest setting). */
  int32_t extra_tokens;
} bsa_problem;

enum { BSA_SELECT_TOPK = 0, BSA_SELECT_THRESHOLD = 1 };

/* Text of a status code (static storage, never NULL). */
const char* bsa_status_str(int status);

/* Name of the HIP runtime error behind the last BSA_ERR_HIP that a call on
 * this thread returned ("none" if there was none).  Static storage, never
 * NULL.  Each launching call first drops a runtime error that earlier code
 * on the thread left pending, so BSA_ERR_HIP always names its own launches. */
const char* bsa_hip_error_str(void);

/* Number of blocks per sequence and the effective k for a problem. */
int bsa_problem_blocks(const bsa_problem* p, int32_t* n_blocks, int32_t* k_eff);

/*
 * Bytes of device scratch memory ("workspace") that covers every entry point
 * below for problem p; 0 when the problem is rejected (bsa_problem_blocks
 * tells why).  The calls share no state through it: each call writes before
 * it reads, so one workspace can serve a sequence of calls on one stream,
 * while calls that may run at the same time need workspaces of their own.
 * What uses it: bsa_pool in reweight mode (the anchor and its per-block
 * partial sums, B*H*(nb+1)*128 float64); bsa_forward and its variants (the
 * order in which query blocks are visited, B*H*nb int32; optional);
 * bsa_select_tokens (16 KB of candidate keys per query block).  Must be
 * 256-byte aligned.
 */
size_t bsa_workspace_bytes(const bsa_problem* p);

/*
 * Stage 1 (and the Spark-Reweight summaries): block pooling.
 * Sources: PyPI page "h3-sparse-attn 0.1.0", opening paragraph (128-token
 * blocks, one summary row per skipped block); Spark-H3 page, section "What
 * Spark-Attn changes" (mean-pooled key/value summary; Spark-Reweight weighted
 * summaries, log-mass bias, per-head mean-video-query anchor).
 *
 *   q, k, v    in   bf16 [B, H, N, 128]
 *   q_pool     out  fp32 [B, H, nb, 128]  block means of Q (summed in float64)
 *   k_pool     out  fp32 [B, H, nb, 128]  block means of K (summed in float64)
 *   sum_k      out  bf16 [B, H, nb, 128]  summary key of each block
 *   sum_v      out  bf16 [B, H, nb, 128]  summary value of each block
 *   sum_bias   out  fp32 [B, H, nb]       additive summary logit bias
 *   workspace  scratch, bsa_workspace_bytes() bytes; used in reweight mode
 *              only (NULL allowed in mean mode)
 *
 * Mean mode: sum_k / sum_v are the block means of K / V and sum_bias is 0.
 * Reweight mode: with a = mean of the query rows [0, anchor_rows) and, for
 * block c, l_j = scale * a . k_j over its rows j and w = softmax_c(l):
 * sum_k = sum_j w_j k_j, sum_v = sum_j w_j v_j and
 * sum_bias = log(mean_j exp(l_j)) - scale * a . kbar_c (kbar_c = block mean).
 */
int bsa_pool(const bsa_problem* p, const void* q, const void* k, const void* v,
             float* q_pool, float* k_pool, void* sum_k, void* sum_v, float* sum_bias,
             void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Stage 2: block scores and top-k selection.
 * Sources: PyPI page "h3-sparse-attn 0.1.0", opening paragraph ("top-k key
 * blocks"); Spark-H3 page, "What Spark-Attn changes" (top-ranked blocks).
 *
 *   q_pool, k_pool  in   fp32 [B, H, nb, 128] (from bsa_pool)
 *   block_idx       out  int32 [B, H, nb, k]
 *
 * The score of query block r against key block c is q_pool[r] . k_pool[c],
 * evaluated in float64 (exact products, float64 sums).  Row r of block_idx
 * holds the k blocks of largest score, equal scores going to the lower block
 * index, in strictly ascending order; with conditioning sinks it holds the
 * sink blocks plus the k - n_sink best of the other blocks.  In threshold
 * mode a row holds its kept blocks (sink blocks, then at most k - n_sink
 * blocks above the row threshold) ascending, followed by -1 in the unused
 * slots.  block_idx may be NULL when k == 0.
 * Requires nb <= BSA_MAX_BLOCKS (else BSA_ERR_UNSUPPORTED).
 */
int bsa_select(const bsa_problem* p, const float* q_pool, const float* k_pool,
               int32_t* block_idx, void* hip_stream);

/*
 * Stages 3 and 4: exact attention over the selected blocks plus one summary
 * row for every other block, in one online softmax.
 * Sources: PyPI page "h3-sparse-attn 0.1.0", opening paragraph (skipped
 * blocks folded back in as one summary row each); Spark-H3 page, "What
 * Spark-Attn changes" (exact and compressed branches of one attention pass).
 *
 *   q, k, v    in   bf16 [B, H, N, 128]
 *   sum_k      in   bf16 [B, H, nb, 128]   summary keys   } any values (bsa_pool's or
 *   sum_v      in   bf16 [B, H, nb, 128]   summary values } the caller's); all three
 *   sum_bias   in   fp32 [B, H, nb]        summary biases } may be NULL only when no
 *                                          row can skip a block (k == nb, top-k mode)
 *   block_idx  in   int32 [B, H, nb, k]    distinct, in [0, nb), ascending,
 *                                          then -1 padding; the kernel trusts
 *                                          this (bsa_select's output); may be
 *                                          NULL iff k == 0
 *   out        out  bf16 [B, H, N, 128]; must not overlap the inputs
 *   workspace  scratch or NULL: with at least bsa_workspace_bytes() bytes
 *              the query blocks of each head are visited sorted by their
 *              first kept blocks (sink query blocks first), so workgroups
 *              running together read the same key blocks; with NULL they
 *              are visited in block order.  The result is the same bits.
 *
 * For query i of block r: logits scale * q_i . k_j for every row j of every
 * block in block_idx[r], and scale * q_i . sum_k[c] + sum_bias[c] for every
 * other block c; out_i = softmax(logits) . [v_j ... ; sum_v[c] ...], with
 * float32 accumulation and one final bf16 rounding.  A query block that is a
 * conditioning sink block attends to every key block exactly and ignores its
 * block_idx row.  A problem with extra tokens is rejected (BSA_ERR_INVALID):
 * use bsa_forward_tokens.
 */
int bsa_forward(const bsa_problem* p, const void* q, const void* k, const void* v, const void* sum_k,
                const void* sum_v, const float* sum_bias, const int32_t* block_idx, void* out,
                void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * bsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and bits as bsa_forward with a workspace, with no
 * workspace argument.  Its scratch (the visiting order, B*H*nb int32) lives
 * in a static device array of the library, 4 MiB on each GPU it runs on
 * (held until the process ends): problems with B*H*nb > 1048576 are rejected
 * with BSA_ERR_SCRATCH.  It allocates and frees nothing.  Every call on one
 * GPU shares that array, so calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller; each call
 * writes the entries it reads before reading them.  Arguments and errors
 * otherwise as for bsa_forward (extra tokens are rejected).
 */
int bsa_forward_noalloc(const bsa_problem* p, const void* q, const void* k, const void* v,
                        const void* sum_k, const void* sum_v, const float* sum_bias,
                        const int32_t* block_idx, void* out, void* hip_stream);

/*
 * Extra tokens, selection.
 * Source: "H3 Sparse Attention" (WAS Node Suite node page), section "The
 * inputs that matter" (extra_tokens: per query block, individually
 * highest-scoring tokens on top of its selected blocks).
 *
 *   q_pool     in   fp32 [B, H, nb, 128] (from bsa_pool)
 *   k          in   bf16 [B, H, N, 128]
 *   block_idx  in   int32 [B, H, nb, k] (from bsa_select; may be NULL iff k == 0)
 *   token_idx  out  int32 [B, H, nb, E], E = p->extra_tokens
 *   workspace  scratch, bsa_workspace_bytes() bytes
 *
 * Candidates of query block r: every token j of the blocks not in
 * block_idx[r].  Score: q_pool[r] . k_j, with q_pool[r] split exactly into
 * three bfloat16 terms so that every product is exact and the sums are
 * float32.  Row r of token_idx holds the E candidates of largest score,
 * equal scores going to the lower token, in strictly ascending order, then
 * -1 in the unused slots (fewer than E candidates).  A conditioning sink
 * query block has no candidates (its row is all -1).  Returns BSA_OK and
 * does nothing when E == 0 (token_idx may then be NULL).
 */
int bsa_select_tokens(const bsa_problem* p, const float* q_pool, const void* k,
                      const int32_t* block_idx, int32_t* token_idx, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/*
 * Stages 3 and 4 with extra tokens: bsa_forward's result where the logits of
 * query i of block r also hold scale * q_i . k_j for every token j of
 * token_idx[r] (value v_j), all in one softmax.
 * Sources: as for bsa_forward and bsa_select_tokens.
 *
 *   q, k, v, sum_k, sum_v, sum_bias, block_idx, out, workspace
 *              as for bsa_forward
 *   token_idx  in   int32 [B, H, nb, E], E = p->extra_tokens (may be NULL iff
 *                   E == 0): tokens in [0, N), distinct, none in a block of
 *                   block_idx[r], valid entries first, then -1 padding; the
 *                   kernels trust this (bsa_select_tokens' output)
 *
 * The attention kernel takes each query block's extra tokens first (their K
 * and V rows gathered on chip) and continues the same online softmax over
 * its blocks and summary rows.  With E == 0 this is bsa_forward (token_idx
 * unused).
 */
int bsa_forward_tokens(const bsa_problem* p, const void* q, const void* k, const void* v,
                       const void* sum_k, const void* sum_v, const float* sum_bias,
                       const int32_t* block_idx, const int32_t* token_idx, void* out, void* workspace,
                       size_t workspace_bytes, void* hip_stream);

/*
 * Spark-Reblock (the q_reuse_k layout): an adaptive order of the N rows of
 * every (batch, head) whose consecutive 128-row blocks group queries with
 * similar attention-score patterns.
 * Sources: "Spark-H3: Block Sparse Attention Speeds Up MiniMax-H3 in
 * ComfyUI", section "What Spark-Attn changes" (similarity is a cosine in the
 * metric of the keys' second moment; a hierarchical partitioner splits groups
 * until each leaf is one block) and section "Workflows" (reblock_layout =
 * q_reuse_k: keys and values take the query layout).
 *
 * Use: bsa_reblock -> perm, then either
 *  - bsa_pool_reordered (-> k', v', the keys and values in the new order),
 *    bsa_select, [bsa_select_tokens on k'], bsa_forward_reordered -> out,
 *    which read q through perm and write out in the original row order, or
 *  - bsa_permute_rows(q, k, v) -> q', k', v'; the block-sparse path
 *    (bsa_pool ... bsa_forward or bsa_forward_tokens) on q', k', v' with the
 *    same problem -> out'; bsa_unpermute_rows(out') -> out.
 * Both give the same bits.  Problems with conditioning sinks, or
 * Spark-Reweight with an anchor over part of the rows, are rejected with
 * BSA_ERR_UNSUPPORTED by all of these calls: those options name rows by
 * position, which the new order changes.  The reblock and row calls read no
 * other field of the problem.
 *
 * What bsa_reblock computes, per (b, h):
 *   M = (1/N) sum_j k_j k_j^T;  L L^T = M + (1e-6 trace(M) / 128 + 1e-30) I;
 *   z_i = L^T q_i / |L^T q_i| (zero rows stay zero).
 *   A group of n rows, m = ceil(n / 128) >= 2 blocks, splits by two pivot
 *   rows: a, the row farthest from the centroid of the group's z rows, and
 *   b, the row farthest from a (squared Euclidean distances; the lowest row
 *   on ties).  Its 128 ceil(m / 2) rows with the smallest z_i . (z_b - z_a)
 *   (ties to the lower row) form the left group, the others the right group,
 *   both in ascending row order; groups of one block are leaves.  perm lists
 *   the leaves left to right, so every 128-row block of the new order but
 *   the last is full, and its rows ascend.  Only distances between z rows
 *   enter, so the order is a function of the metric cosines z_i . z_j alone.
 * Precision: M as float32 sums of exact products over 2048-row chunks, the
 * chunks and the factorisation in float64, z in float32, distances and keys
 * in float64 from that z (keys then rounded to float32).  Where two
 * distances or two keys are within that rounding of each other, the order
 * may differ from an exact evaluation's.
 *
 *   q, k       in   bf16 [B, H, N, 128]
 *   perm       out  int32 [B, H, N]: perm[p] = the row placed at position p
 *   workspace  in/out  bsa_reblock_workspace_bytes() bytes, 256-byte aligned
 *                   (about N * 552 bytes per (b, h)); its contents are
 *                   scratch and need no initialisation
 */
int bsa_reblock_workspace_bytes(const bsa_problem* p, size_t* bytes);
int bsa_reblock(const bsa_problem* p, const void* q, const void* k, int32_t* perm,
                void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * The block-sparse path on a row order without permuted copies of Q and the
 * output.  Sources: as for bsa_pool, bsa_forward and bsa_reblock.
 *
 * bsa_pool_reordered: bsa_pool of q', k', v' where x'[b, h, p, :] =
 * x[b, h, perm[b, h, p], :], every row read through perm, plus
 *   k_out, v_out  out  bf16 [B, H, N, 128]: k' and v', the keys and values
 *               in the new order, which bsa_forward_reordered (and
 *               bsa_select_tokens) read as contiguous tiles; neither may
 *               overlap q, k, v or the other
 * The pooled vectors, summaries and block indices that follow are those of
 * the new order (block c = positions [128 c, 128 c + 128)).
 *
 * bsa_forward_reordered: bsa_forward_tokens of q', k', v' (bsa_forward when
 * p->extra_tokens == 0; token_idx may then be NULL), with its output row p
 * written to out[b, h, perm[b, h, p], :]:
 *   q          in   bf16 [B, H, N, 128], the original row order
 *   k_r, v_r   in   bf16 [B, H, N, 128], k_out and v_out of bsa_pool_reordered
 *   sum_k, sum_v, sum_bias, block_idx, token_idx   in   as for
 *              bsa_forward_tokens, from the calls on the new order
 *   out        out  bf16 [B, H, N, 128], the original row order; not
 *              overlapping any input
 *   workspace  unused (may be NULL): the reblocked order is visited as it is
 *
 *   perm  in  int32 [B, H, N], a permutation of 0..N-1 per (b, h) (as
 *             bsa_reblock writes it; other values are not checked and read
 *             or write out of bounds); 4-byte aligned
 */
int bsa_pool_reordered(const bsa_problem* p, const int32_t* perm, const void* q, const void* k,
                       const void* v, float* q_pool, float* k_pool, void* sum_k, void* sum_v,
                       float* sum_bias, void* k_out, void* v_out, void* workspace,
                       size_t workspace_bytes, void* hip_stream);
int bsa_forward_reordered(const bsa_problem* p, const int32_t* perm, const void* q, const void* k_r,
                          const void* v_r, const void* sum_k, const void* sum_v, const float* sum_bias,
                          const int32_t* block_idx, const int32_t* token_idx, void* out, void* workspace,
                          size_t workspace_bytes, void* hip_stream);

/*
 * Rows of Q, K and V in the new order (the q_reuse_k layout):
 * x_out[b, h, p, :] = x[b, h, perm[b, h, p], :] for x = q, k, v.
 *   perm             in   int32 [B, H, N], a permutation of 0..N-1 per (b, h)
 *                         (as bsa_reblock writes it; other values are not
 *                         checked and read out of bounds)
 *   q, k, v          in   bf16 [B, H, N, 128]
 *   q_out, k_out, v_out  out  bf16 [B, H, N, 128], not overlapping the inputs
 */
int bsa_permute_rows(const bsa_problem* p, const int32_t* perm, const void* q, const void* k,
                     const void* v, void* q_out, void* k_out, void* v_out, void* hip_stream);

/*
 * Output rows back in their original places: out[b, h, perm[b, h, p], :] =
 * x[b, h, p, :].
 *   perm   in   int32 [B, H, N], as for bsa_permute_rows
 *   x      in   bf16 [B, H, N, 128] (the block-sparse output in the new order)
 *   out    out  bf16 [B, H, N, 128], not overlapping x
 */
int bsa_unpermute_rows(const bsa_problem* p, const int32_t* perm, const void* x, void* out,
                       void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */

"""CPU oracle for block-sparse attention with summary rows.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP library
and its Python binding) never imports, calls or falls back to it, and this
module imports nothing from the product path.  It is deliberately plain and
slow: numpy, float64 arithmetic, one query block at a time.

What it computes, per (batch, head), with inputs of shape [N, d] (bfloat16
values widened exactly to float):

Sources (page titles and sections):
  * "h3-sparse-attn 0.1.0" (PyPI page), opening paragraph: each query block
    attends to its top-k key blocks of 128 tokens, and every skipped key block
    is folded back in as one summary row; top_k counts 128-token key blocks
    (section "Use"); bf16, head_dim 128, forward only.
  * "Spark-H3: Block Sparse Attention Speeds Up MiniMax-H3 in ComfyUI",
    section "What Spark-Attn changes": the exact branch computes the
    top-ranked key/value blocks in full, the compressed branch covers the rest
    cheaply; Spark-Reweight replaces the mean-pooled summary with weighted
    summaries plus a log-mass bias, anchored on the mean of the video queries
    of each head, because mean pooling puts exp(E[x]) where the attention mass
    is E[exp(x)]; the caption of that section's figure states that the pooled
    logit plus the bias exponentiates to the expected exponential.

Readings taken where the pages are silent (each is exercised by a test):
  R1 ragged last block: pooled by its real row count; its exact keys are its
     real rows only.
  R2 block score: plain dot product of the pooled query and key vectors (the
     softmax scale does not change a ranking).
  R3 ties: equal scores go to the lower block index; output ascending.
  R4 no forced blocks (no diagonal or sink block is added to the top-k)
     unless a conditioning range is given (R13).
  R5 a top-k ratio budget becomes k = ceil(ratio * n_blocks) computed exactly.
  R6 softmax scale 1/sqrt(d) for exact and summary logits alike; the bias is
     added in scaled-logit units.
  R7 one summary row per skipped block, with no log(row count) mass term.
  R8 reweight: summary key = softmax-weighted key rows, summary value =
     softmax-weighted value rows, with weights softmax over the block of the
     anchor logits a.k_j/sqrt(d); bias = log(mean_j exp(a.k_j/sqrt(d)))
     - a.kbar/sqrt(d) with kbar the plain block mean of the keys.
  R9 anchor = mean of the query rows [0, anchor_rows) (the video rows, which
     lead the sequence); anchor_rows = 0 means all rows.
  R10 selection uses the mean-pooled vectors in both summary modes.
  R11 no causal mask.
  R13 conditioning sinks (the "exact_kv_and_rows" routing): the conditioning
     rows (prompt, reference, audio) form one contiguous row range.  Every
     block holding at least one of its rows is a sink block: it is forced
     into every query block's exact set, on top of the top_k picked among the
     other blocks (so a row holds min(top_k, nb - n_sink) + n_sink blocks),
     and a query block that is itself a sink block attends to every key block
     exactly (no summary rows).  Sources: "H3 Sparse Attention" (WAS Node
     Suite node page), section "The inputs that matter" (with
     sink_conditioning on, the prompt, reference and audio rows are attended
     exactly and their own queries attend densely); "H3 Sparse Attention"
     (the node page on video budgets), opening section (only attention among
     video tokens is made sparse: conditioning and non-video queries, and
     the tiles where two contexts meet, keep dense attention).  The block straddling the boundary counts as a sink block.
  R14 threshold (variable-k) selection with parameter tau: a key block is
     kept when its score exceeds the mean of its row's block scores by more
     than tau population standard deviations, s > mean + tau * std (both over
     all nb blocks of the row, in float64); at most top_k blocks are kept
     (the highest, ties to the lower index), sink blocks always.  Rows are
     padded with -1 after their kept blocks.  Source: "H3 Sparse Attention"
     (WAS Node Suite node page), section "The inputs that matter" (the
     share of key blocks kept exact is given as about 16% at tau 1.0, 7% at
     1.5 and 3% at 2.0): the normal tail beyond tau standard deviations is
     15.9%, 6.7% and 2.3%.
  R15 extra tokens: besides its kept blocks, each query block r reads exactly
     the E tokens j of the blocks it skipped with the largest q_pool[r] . k_j
     (the same pooled-query score as block selection, float64), ties to the
     lower token index; every skipped block keeps its summary row (R7 weighs
     a summary row as one key, so nothing is counted twice).  Sink query
     blocks skip nothing and read no extra tokens.  Source: "H3 Sparse
     Attention" (WAS Node Suite node page), section "The inputs that matter"
     (extra_tokens: per query block, individually highest-scoring tokens on
     top of its selected blocks).

  R17 Spark-Reblock (the "q_reuse_k" layout).  Sources: "Spark-H3: Block
     Sparse Attention Speeds Up MiniMax-H3 in ComfyUI", section "What
     Spark-Attn changes" (queries are grouped by the similarity of their score
     patterns over the keys, a cosine distance in the metric of the keys'
     second moment; a hierarchical partitioner splits groups until each leaf
     is one block, in O(N log N)), and section "Workflows" (every shipped
     workflow sets reblock_layout=q_reuse_k: the query partition is reused for
     the keys).  Per (batch, head): M = (1/N) sum_j k_j k_j^T over all rows;
     L is the Cholesky factor of M + eps (trace(M)/d) I + 1e-30 I with
     eps = 1e-6 (the small ridge keeps L defined for rank-deficient keys);
     each query row becomes the unit vector z_i = L^T q_i / |L^T q_i| (zero
     stays zero), so z_i . z_j is the cosine of q_i and q_j in the metric M.
     A group of n rows (m = ceil(n / 128) blocks, m >= 2) splits by two
     pivot rows: a, the row farthest from the group's centroid (mean of its
     z rows), and b, the row farthest from a (Euclidean distances between
     the z rows, i.e. the chordal form of the metric cosine distance; the
     lowest row index on ties); the 128 * ceil(m / 2) rows with the smallest
     z_i . (z_b - z_a), i.e. nearest to a relative to b (ties to the lower
     row index), form the left group, the rest the right one, each in
     ascending row order.  The leaves, left to right, give the permutation;
     Q, K and V are all permuted by it, the block-sparse path runs on the
     permuted rows, and the output rows are put back in their original
     places.  The pages name neither the split rule nor its direction; this
     two-pivot (farthest-point) bisection uses nothing but the distances
     between the whitened rows, so the partition is a function of the metric
     cosines alone (any orthogonal map of the head features applied to Q and
     K leaves it unchanged, and so does any map q -> A q, k -> A^-T k that
     keeps every score, up to the small ridge), and each level costs O(n d),
     O(N d log N) in all.

Precision: pooled vectors are summed in float64 and stored as float32 (the
precision in which a block ranking is decided); block scores are float64 dot
products of those float32 vectors; everything else is float64.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

BLOCK = 128


# ----------------------------------------------------------------- blocks ---
def n_blocks(N: int, block: int = BLOCK) -> int:
    """Number of key/query blocks: ceil(N / block) (PyPI page, opening
    paragraph: the sequence is cut into 128-token blocks)."""
    return -(-N // block)


def block_rows(N: int, block: int = BLOCK):
    """[(start, end)] row ranges of every block; the last one may be short (R1)."""
    return [(s, min(s + block, N)) for s in range(0, N, block)]


def effective_k(top_k: int, nb: int) -> int:
    """Key blocks kept per query block: top_k, capped at the number of blocks."""
    if top_k < 0:
        raise ValueError("top_k must be >= 0")
    return min(top_k, nb)


def k_from_ratio(ratio, nb: int) -> int:
    """Top-k ratio budget (Spark-H3 page, "Workflows": topk_mode=topk_ratio)
    turned into a block count, k = ceil(ratio * nb), in exact rational
    arithmetic on the decimal string of the ratio (R5)."""
    r = Fraction(str(ratio))
    if r < 0 or r > 1:
        raise ValueError("ratio must lie in [0, 1]")
    return math.ceil(r * nb)


# ------------------------------------------------------------------- pool ---
def pool_mean(x: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Per-block mean of the rows of x [N, d]: one pooled vector per block.

    Summed in float64, divided by the block's real row count (R1), stored as
    float32.  Spark-H3 page, "What Spark-Attn changes" (mean-pooled summary)."""
    x = np.asarray(x, dtype=np.float64)
    out = []
    for s, e in block_rows(x.shape[0], block):
        out.append(x[s:e].sum(axis=0) / (e - s))
    return np.array(out, dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------- select ---
def block_scores(q_pool: np.ndarray, k_pool: np.ndarray) -> np.ndarray:
    """s[r, c] = q_pool[r] . k_pool[c] in float64 (R2).

    Every element is reduced by the same code path, so two identical key
    blocks score bit-identically against any query block."""
    qp = np.asarray(q_pool, dtype=np.float64)
    kp = np.asarray(k_pool, dtype=np.float64)
    s = np.empty((qp.shape[0], kp.shape[0]))
    for r in range(qp.shape[0]):
        s[r] = (qp[r][None, :] * kp).sum(axis=-1)
    return s


def select_topk(scores: np.ndarray, top_k: int, forced=()) -> np.ndarray:
    """For each query block r the k key blocks of largest score, ties to the
    lower index (R3), returned in ascending index order; int32 [nb, k].

    With forced blocks (R13) every row holds all of them plus the top_k of the
    remaining blocks, k = min(top_k, nb - n_forced) + n_forced.

    PyPI page, opening paragraph ("attends to its top-k key blocks")."""
    nq, nk = scores.shape
    F = sorted(set(int(c) for c in forced))
    if any(c < 0 or c >= nk for c in F):
        raise ValueError("forced block out of range")
    rest = [c for c in range(nk) if c not in set(F)]
    k = effective_k(top_k, len(rest))
    idx = np.zeros((nq, len(F) + k), dtype=np.int32)
    for r in range(nq):
        order = sorted(rest, key=lambda c: (-scores[r, c], c))
        idx[r] = sorted(F + order[:k])
    return idx


def select_threshold(scores: np.ndarray, tau: float, top_k: int, forced=()) -> np.ndarray:
    """Variable-k selection (R14): for each row r, the blocks c whose score is
    above mean_r + tau * std_r (population statistics of the row, float64),
    at most top_k of them (largest first, ties to the lower index), plus the
    forced blocks; ascending, padded with -1 to n_forced + min(top_k, nb -
    n_forced) entries."""
    nq, nk = scores.shape
    F = sorted(set(int(c) for c in forced))
    rest = [c for c in range(nk) if c not in set(F)]
    k = effective_k(top_k, len(rest))
    idx = np.full((nq, len(F) + k), -1, dtype=np.int32)
    for r in range(nq):
        row = np.asarray(scores[r], dtype=np.float64)
        mean = row.sum() / nk
        std = math.sqrt(((row - mean) ** 2).sum() / nk)
        thr = mean + tau * std
        above = [c for c in rest if row[c] > thr]
        order = sorted(above, key=lambda c: (-row[c], c))
        kept = sorted(F + order[:k])
        idx[r, :len(kept)] = kept
    return idx


def select_extra_tokens(q_pool, k, idx, extra: int, block: int = BLOCK, dense_blocks=(),
                        query_blocks=None):
    """Extra tokens (R15): for each query block r, the `extra` tokens of the
    blocks not in idx[r] with the largest q_pool[r] . k_j (float64), ties to
    the lower token index; ascending, padded with -1.  int32 [nb, extra].
    query_blocks restricts the work to those rows (the others stay -1)."""
    qp = np.asarray(q_pool, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    rows = block_rows(k.shape[0], block)
    nb = len(rows)
    out = np.full((nb, extra), -1, dtype=np.int32)
    for r in range(nb):
        if r in set(dense_blocks) or extra == 0:
            continue
        if query_blocks is not None and r not in query_blocks:
            continue
        chosen = set(int(c) for c in idx[r] if c >= 0)
        cand = [j for c in range(nb) if c not in chosen for j in range(rows[c][0], rows[c][1])]
        # the float64 dot products of every candidate key with the pooled query
        s = k[cand] @ qp[r] if cand else np.zeros(0)
        order = sorted(range(len(cand)), key=lambda i: (-s[i], cand[i]))[:extra]
        kept = sorted(cand[i] for i in order)
        out[r, :len(kept)] = kept
    return out


def sink_blocks(N: int, sink_start: int, sink_rows: int, block: int = BLOCK):
    """Blocks holding at least one row of the conditioning range
    [sink_start, sink_start + sink_rows) (R13); empty when sink_rows is 0."""
    if sink_start < 0 or sink_rows < 0 or sink_start + sink_rows > N:
        raise ValueError("conditioning range out of bounds")
    if sink_rows == 0:
        return []
    return list(range(sink_start // block, (sink_start + sink_rows - 1) // block + 1))


# -------------------------------------------------------------- summaries ---
def summaries_mean(k: np.ndarray, v: np.ndarray, block: int = BLOCK):
    """Mean mode: summary key/value of block c are the block means; bias 0.

    Returns float64 (sum_k [nb, d], sum_v [nb, d], bias [nb])."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = block_rows(k.shape[0], block)
    sk = np.array([k[s:e].mean(axis=0) for s, e in rows])
    sv = np.array([v[s:e].mean(axis=0) for s, e in rows])
    return sk, sv, np.zeros(len(rows))


def anchor(q: np.ndarray, anchor_rows: int) -> np.ndarray:
    """Per-head anchor: the mean of the query rows [0, anchor_rows) (R9;
    Spark-H3 page, "What Spark-Attn changes": the mean of the video queries is
    one anchor per head).  anchor_rows = 0 means every row."""
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[0] if anchor_rows == 0 else anchor_rows
    if not 0 < n <= q.shape[0]:
        raise ValueError("anchor_rows out of range")
    return q[:n].sum(axis=0) / n


def summaries_reweight(k: np.ndarray, v: np.ndarray, a: np.ndarray, scale: float,
                       block: int = BLOCK, bias_ref: str = "mean"):
    """Spark-Reweight summaries (R8).

    For block c with rows j:  l_j = scale * a . k_j,  w = softmax_c(l),
    sum_k = sum_j w_j k_j,  sum_v = sum_j w_j v_j,
    bias = log(mean_j exp(l_j)) - scale * a . kbar_c  (bias_ref="mean"), or
    bias = log(mean_j exp(l_j)) - scale * a . sum_k   (bias_ref="weighted").

    The log-mean-exp is evaluated as max + log(sum exp(l - max)) - log(n_c).
    Spark-H3 page, "What Spark-Attn changes" (weighted summaries plus a
    log-mass bias; exp(E[x]) versus E[exp(x)])."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    sks, svs, bs = [], [], []
    for s, e in block_rows(k.shape[0], block):
        kb, vb = k[s:e], v[s:e]
        l = scale * (kb @ a)
        m = l.max()
        ex = np.exp(l - m)
        w = ex / ex.sum()
        sk = w @ kb
        sv = w @ vb
        lme = m + math.log(ex.sum()) - math.log(e - s)
        ref = kb.mean(axis=0) if bias_ref == "mean" else sk
        sks.append(sk)
        svs.append(sv)
        bs.append(lme - scale * float(ref @ a))
    return np.array(sks), np.array(svs), np.array(bs)


# -------------------------------------------------------------- attention ---
def attention(q, k, v, idx, sum_k, sum_v, bias, scale: float, block: int = BLOCK,
              query_blocks=None, dense_blocks=(), extra=None):
    """Block-sparse attention with summary rows for one (batch, head).

    For query i in block r, the logits are
      [scale * q_i . k_j  for every row j of every selected block c in idx[r]]
      ++ [scale * q_i . sum_k[c] + bias[c]  for every block c not in idx[r]],
    one softmax runs over that whole list, and the output is the matching
    weighted sum of [v_j ...] ++ [sum_v[c] ...].  PyPI page, opening paragraph
    (top-k blocks plus one summary row per skipped block); Spark-H3 page,
    "What Spark-Attn changes" (exact and compressed branches of one pass).

    idx may be any [nb, k] array of distinct valid block indices per row (the
    output is unique given idx); entries of -1 are padding and ignored.  Query
    blocks listed in dense_blocks attend to every key block exactly, whatever
    idx holds for them (R13).  extra [nb, E] lists tokens each query block
    also reads exactly (R15; -1 is padding).  query_blocks restricts the work
    to those query blocks (other output rows stay zero).
    Returns float64 [N, d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sum_k = np.asarray(sum_k, dtype=np.float64)
    sum_v = np.asarray(sum_v, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    N, d = q.shape
    rows = block_rows(N, block)
    nb = len(rows)
    out = np.zeros((N, d))
    for r, (s, e) in enumerate(rows):
        if query_blocks is not None and r not in query_blocks:
            continue
        sel = list(range(nb)) if r in set(dense_blocks) else [int(c) for c in idx[r] if c >= 0]
        if len(set(sel)) != len(sel) or any(c < 0 or c >= nb for c in sel):
            raise ValueError("idx row %d is not a set of valid blocks" % r)
        chosen = set(sel)
        skipped = [c for c in range(nb) if c not in chosen]
        ext = [] if extra is None else [int(j) for j in extra[r] if j >= 0]
        keys = [k[rows[c][0]:rows[c][1]] for c in sorted(chosen)] + [k[ext]] + [sum_k[skipped]]
        vals = [v[rows[c][0]:rows[c][1]] for c in sorted(chosen)] + [v[ext]] + [sum_v[skipped]]
        add = ([np.zeros(rows[c][1] - rows[c][0]) for c in sorted(chosen)] + [np.zeros(len(ext))] +
               [bias[skipped]])
        K = np.concatenate(keys, axis=0)
        V = np.concatenate(vals, axis=0)
        B = np.concatenate(add)
        logits = scale * (q[s:e] @ K.T) + B[None, :]
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        out[s:e] = p @ V
    return out


# -------------------------------------------------------------- pipeline ---
def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def run_head(q, k, v, top_k: int, summary: str = "mean", anchor_rows: int = 0,
             scale: float | None = None, block: int = BLOCK, bias_ref: str = "mean",
             sink_start: int = 0, sink_rows: int = 0, tau: float | None = None,
             extra_tokens: int = 0):
    """All four stages for one (batch, head).  Returns a dict with the pooled
    vectors, scores, selection, summaries, sink blocks and the float64 output.
    sink_rows > 0 routes the conditioning rows [sink_start, sink_start +
    sink_rows) as sinks (R13); tau selects blocks by threshold (R14) with top_k
    as the cap; extra_tokens adds that many exact tokens per query block (R15)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    sc = default_scale(d) if not scale else float(scale)
    q_pool = pool_mean(q, block)
    k_pool = pool_mean(k, block)
    s = block_scores(q_pool, k_pool)
    sinks = sink_blocks(q.shape[0], sink_start, sink_rows, block)
    idx = select_topk(s, top_k, sinks) if tau is None else select_threshold(s, tau, top_k, sinks)
    if summary == "mean":
        sk, sv, b = summaries_mean(k, v, block)
    elif summary == "reweight":
        a = anchor(q, anchor_rows)
        sk, sv, b = summaries_reweight(k, v, a, sc, block, bias_ref)
    else:
        raise ValueError("summary must be 'mean' or 'reweight'")
    extra = select_extra_tokens(q_pool, k, idx, extra_tokens, block, sinks) if extra_tokens else None
    out = attention(q, k, v, idx, sk, sv, b, sc, block, dense_blocks=sinks, extra=extra)
    return dict(q_pool=q_pool, k_pool=k_pool, scores=s, idx=idx, sum_k=sk,
                sum_v=sv, bias=b, out=out, scale=sc, sinks=sinks, extra=extra)


# ---------------------------------------------------------- Spark-Reblock ---
REBLOCK_EPS = 1e-6


def key_second_moment(k: np.ndarray) -> np.ndarray:
    """M = (1/N) sum_j k_j k_j^T, the second moment of the key rows that
    defines the query metric (R17; "What Spark-Attn changes", the Spark-Reblock
    item: the metric comes from the opposite side's second moment)."""
    k = np.asarray(k, dtype=np.float64)
    return k.T @ k / k.shape[0]


def mahalanobis_embedding(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Unit rows z_i = L^T q_i / |L^T q_i| with L L^T = M + ridge (R17), so
    that z_i . z_j = q_i^T M q_j / (|q_i|_M |q_j|_M) up to the ridge."""
    q = np.asarray(q, dtype=np.float64)
    M = key_second_moment(k)
    d = M.shape[0]
    ridge = REBLOCK_EPS * (np.trace(M) / d) + 1e-30
    L = np.linalg.cholesky(M + ridge * np.eye(d))
    z = q @ L  # row i holds (L^T q_i)^T
    norm = np.sqrt((z * z).sum(axis=1))
    out = np.zeros_like(z)
    nz = norm > 0
    out[nz] = z[nz] / norm[nz, None]
    return out


def reblock_left_rows(n: int, block: int = BLOCK) -> int:
    """Rows of the left group when a group of n rows splits: 128 * ceil(m / 2)
    for its m = ceil(n / 128) blocks, so every leaf but the last is full (R17)."""
    m = n_blocks(n, block)
    return block * (-(-m // 2))


def split_pivots(zg: np.ndarray):
    """The two pivots of a group (R17), as positions among its rows (which
    are in ascending row order): a = the row farthest from the centroid of
    the group's z rows, b = the row farthest from a; squared Euclidean
    distances, the first (lowest) row on ties."""
    zg = np.asarray(zg, dtype=np.float64)
    c = zg.sum(axis=0) / zg.shape[0]
    a = int(np.argmax(((zg - c) ** 2).sum(axis=1)))
    b = int(np.argmax(((zg - zg[a]) ** 2).sum(axis=1)))
    return a, b


def split_keys(zg: np.ndarray, a: int, b: int) -> np.ndarray:
    """Split key of every row of a group: z_i . (z_b - z_a), which orders the
    rows as |z_i - z_a|^2 - |z_i - z_b|^2 does (smallest: nearest to a)."""
    zg = np.asarray(zg, dtype=np.float64)
    return zg @ (zg[b] - zg[a])


def reblock_permutation(q: np.ndarray, k: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Spark-Reblock permutation of one (batch, head) (R17): perm[p] is the
    original row placed at position p; int64 [N]."""
    z = mahalanobis_embedding(q, k)
    N = z.shape[0]
    leaves = []

    def split(rows: np.ndarray):
        n = len(rows)
        if n_blocks(n, block) <= 1:
            leaves.append(rows)
            return
        a, b = split_pivots(z[rows])
        key = split_keys(z[rows], a, b)
        # rows ordered by their key, ties to the lower row index
        order = rows[np.lexsort((rows, key))]
        nl = reblock_left_rows(n, block)
        split(np.sort(order[:nl]))
        split(np.sort(order[nl:]))

    split(np.arange(N, dtype=np.int64))
    return np.concatenate(leaves) if leaves else np.zeros(0, dtype=np.int64)


def run_head_reblocked(q, k, v, perm, **kw):
    """The block-sparse path on rows permuted by perm (Q, K and V alike, the
    q_reuse_k layout), with the output rows put back in place (R17).  kw as
    for run_head; the result's 'out' is in the original row order."""
    perm = np.asarray(perm, dtype=np.int64)
    res = run_head(np.asarray(q)[perm], np.asarray(k)[perm], np.asarray(v)[perm], **kw)
    out = np.empty_like(res["out"])
    out[perm] = res["out"]
    res["out_permuted"] = res["out"]
    res["out"] = out
    return res


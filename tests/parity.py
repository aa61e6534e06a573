"""Shared checks for the GPU parity tests: converting generator output to
device tensors, the index tie-zone rule and the output tolerance."""
import numpy as np

from block_sparse_attention_25_amd.synth import bf16_to_f32

# Output tolerance against the float64 oracle (bf16 output, fp32 accumulation)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# Index rule: exact, except where the k-th and (k+1)-th oracle scores differ
# by less than this relative amount
TIE_REL = 1e-4


def to_device(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def widen(bits):
    """bf16 bit array -> float64 array (exact)."""
    return bf16_to_f32(np.ascontiguousarray(bits)).astype(np.float64)


def tensor_bits(t):
    """bf16 torch tensor -> uint16 numpy bit array."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def check_idx_row(gpu_row, scores_row, k):
    """True when a GPU row of block indices is acceptable against the oracle's
    scores: k distinct ascending valid indices, equal to the oracle's top-k,
    or differing only inside the tie zone.  Returns (ok, in_tie_zone)."""
    nb = len(scores_row)
    g = [int(x) for x in gpu_row]
    if len(g) != k or any(b <= a for a, b in zip(g, g[1:])) or any(c < 0 or c >= nb for c in g):
        return False, False
    order = sorted(range(nb), key=lambda c: (-scores_row[c], c))
    want = set(order[:k])
    if set(g) == want:
        return True, False
    sk = scores_row[order[k - 1]]
    sk1 = scores_row[order[k]]
    tol = TIE_REL * max(abs(sk), abs(sk1))
    if abs(sk - sk1) >= tol:
        return False, False
    diff = set(g) ^ want
    ok = all(abs(scores_row[c] - sk) <= TIE_REL * max(abs(sk), 1e-300) for c in diff)
    return ok, True


def check_idx_rows(gidx, scores, k):
    """check_idx_row over every row of one (b, h): the oracle's top-k of each
    row (descending score, ties to the lower index) taken for all rows at
    once; rows whose set differs are judged by check_idx_row (tie zone).
    Returns (bad_rows, tie_rows)."""
    gidx = np.asarray(gidx)
    s = np.asarray(scores, dtype=np.float64)
    nq, nb = s.shape
    if gidx.shape != (nq, k):
        return list(range(nq)), 0
    if k == 0:
        return [], 0
    cols = np.broadcast_to(np.arange(nb), (nq, nb))
    order = np.lexsort((cols, -s), axis=-1)[:, :k]
    want = np.sort(order, axis=-1)
    bad, ties = [], 0
    for r in np.nonzero(np.any(gidx != want, axis=-1))[0]:
        ok, tie = check_idx_row(gidx[r], s[r], k)
        if not ok:
            bad.append(int(r))
        ties += tie
    # rows equal to the oracle's must still be strictly ascending (they are,
    # being sorted), so only the differing rows needed the full check
    return bad, ties


def check_idx_row_forced(gpu_row, scores_row, k, forced):
    """check_idx_row with conditioning sinks: the row holds every forced block,
    and its other entries are the top-(k - len(forced)) of the remaining
    blocks, under the same tie-zone rule."""
    g = [int(x) for x in gpu_row]
    F = set(int(c) for c in forced)
    nb = len(scores_row)
    if len(g) != k or any(b <= a for a, b in zip(g, g[1:])) or any(c < 0 or c >= nb for c in g):
        return False, False
    if not F <= set(g):
        return False, False
    rest = [c for c in range(nb) if c not in F]
    pos = {c: i for i, c in enumerate(rest)}
    sub = sorted(pos[c] for c in g if c not in F)
    return check_idx_row(sub, np.asarray(scores_row)[rest], k - len(F))


# Threshold selection: a block whose score lies this close (relative to the
# row's |threshold| + deviation) to the threshold may fall on either side,
# since the GPU sums the row statistics in another order
THR_REL = 1e-9


def check_idx_row_threshold(gpu_row, scores_row, want_row, forced, tau):
    """A threshold-selection row: kept blocks ascending then -1 padding, every
    forced block kept, and equal to the oracle's row except for blocks at the
    row threshold (within THR_REL) or inside the cap's tie zone."""
    g = [int(x) for x in gpu_row]
    w = [int(x) for x in want_row]
    nb = len(scores_row)
    nv = sum(1 for c in g if c >= 0)
    valid = g[:nv]
    if any(c != -1 for c in g[nv:]) or any(b <= a for a, b in zip(valid, valid[1:])):
        return False, False
    if any(c < 0 or c >= nb for c in valid) or not set(forced) <= set(valid):
        return False, False
    if g == w:
        return True, False
    row = np.asarray(scores_row, dtype=np.float64)
    mean = row.mean()
    std = row.std()
    thr = mean + tau * std
    scale = abs(thr) + std + 1e-300
    F = set(forced)
    kept_g = set(valid) - F
    kept_w = set(c for c in w if c >= 0) - F
    cap_bound = len(kept_w) > 0 and min(row[c] for c in kept_w)
    cap = len(w) - len(F)
    for c in kept_g ^ kept_w:
        at_thr = abs(row[c] - thr) <= THR_REL * scale
        at_cap = len(kept_w) == cap and abs(row[c] - cap_bound) <= TIE_REL * max(abs(cap_bound), 1e-300)
        if not (at_thr or at_cap):
            return False, False
    return True, True


def check_tokens_row(gpu_row, cand, cand_scores, E):
    """An extra-token row: the E candidate tokens of largest float64 score
    (ties to the lower token), ascending, then -1 padding when there are fewer
    than E candidates; equal to the oracle's choice except inside the tie zone
    at the E-th score (the GPU ranks float32 sums of exact products).
    cand lists the candidate tokens ascending, cand_scores their scores.
    Returns (ok, in_tie_zone)."""
    g = [int(x) for x in gpu_row]
    n = min(E, len(cand))
    if len(g) != E or any(x != -1 for x in g[n:]):
        return False, False
    pos = {t: i for i, t in enumerate(cand)}
    if any(t not in pos for t in g[:n]):
        return False, False
    if n == 0:
        return True, False
    return check_idx_row([pos[t] for t in g[:n]], np.asarray(cand_scores, dtype=np.float64), n)


def check_output(gpu_out, ref_out):
    d = np.abs(np.asarray(gpu_out, dtype=np.float64) - ref_out)
    return float(d.max()), float(d.mean())


# Reblock rule: a GPU split is accepted when some pair of pivots (a, b), each
# within REBLOCK_DIST_ABS of the largest squared distance behind it (from the
# group's centroid, then from a), orders every left row's key
# z_i . (z_b - z_a) at or below every right row's, up to REBLOCK_KEY_ABS.  z
# has unit rows; the GPU's z differs from the float64 one by the float32
# rounding of M, L and z, measured at most 2.1e-7 per coordinate, so a
# distance moves by at most about 2 |z_i - c| |dz| <= 2e-5 and a key by about
# 1e-5 (the GPU forms both in float64 from its float32 z, the key then
# rounded to float32)
REBLOCK_KEY_ABS = 2e-5
REBLOCK_DIST_ABS = 2e-5


def reblock_splits(N, left_rows, block=128):
    """(start, n, n_left) of every split of the bisection tree over N rows;
    the tree's shape depends on N only."""
    out, stack = [], [(0, N)]
    while stack:
        s, n = stack.pop()
        if -(-n // block) <= 1:
            continue
        nl = left_rows(n, block)
        out.append((s, n, nl))
        stack += [(s, nl), (s + nl, n - nl)]
    return out


def _pivot_candidates(zg, max_each=8):
    """Pivot pairs (a, b) within REBLOCK_DIST_ABS of the farthest, as positions
    in zg (its rows ascending), the lowest first."""
    c = zg.sum(axis=0) / zg.shape[0]
    t = ((zg - c) ** 2).sum(axis=1)
    pairs = []
    for a in np.nonzero(t >= t.max() - REBLOCK_DIST_ABS)[0][:max_each]:
        d = ((zg - zg[a]) ** 2).sum(axis=1)
        for b in np.nonzero(d >= d.max() - REBLOCK_DIST_ABS)[0][:max_each]:
            pairs.append((int(a), int(b)))
    return pairs


def check_partition(z, perm, left_rows, block=128):
    """Validate a GPU permutation against the float64 embedding z of the same
    head: a permutation; every 128-row block ascending; every split separated
    by the keys of an admissible pivot pair.  Returns (ok, message)."""
    N = z.shape[0]
    perm = np.asarray(perm, dtype=np.int64)
    if perm.shape != (N,) or not np.array_equal(np.sort(perm), np.arange(N)):
        return False, "not a permutation"
    for b0 in range(0, N, block):
        if np.any(np.diff(perm[b0:b0 + block]) <= 0):
            return False, "block at %d not ascending" % b0
    for s, n, nl in reblock_splits(N, left_rows, block):
        rows = np.sort(perm[s:s + n])
        zg = z[rows]
        pos = np.searchsorted(rows, perm[s:s + n])
        lp, rp = pos[:nl], pos[nl:]
        ok = False
        for a, b in _pivot_candidates(zg):
            key = zg @ (zg[b] - zg[a])
            if key[lp].max() <= key[rp].min() + REBLOCK_KEY_ABS:
                ok = True
                break
        if not ok:
            return False, "split at %d (n %d) not separated by any admissible pivot pair" % (s, n)
    return True, ""


def reblock_margins(z, perm, left_rows, block=128):
    """Smallest margins of the oracle's own splits: the gap between the
    largest and second-largest squared distance behind either pivot, and the
    gap between the left group's largest and the right group's smallest key."""
    dgap, kgap = np.inf, np.inf
    for s, n, nl in reblock_splits(z.shape[0], left_rows, block):
        rows = np.sort(perm[s:s + n])
        zg = z[rows]
        c = zg.sum(axis=0) / n
        t = ((zg - c) ** 2).sum(axis=1)
        a = int(np.argmax(t))
        d = ((zg - zg[a]) ** 2).sum(axis=1)
        b = int(np.argmax(d))
        for x in (t, d):
            top = np.sort(x)[-2:]
            dgap = min(dgap, top[1] - top[0])
        key = zg @ (zg[b] - zg[a])
        pos = np.searchsorted(rows, perm[s:s + n])
        kgap = min(kgap, key[pos[nl:]].min() - key[pos[:nl]].max())
    return dgap, kgap

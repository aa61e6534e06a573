"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small cases compare every output element; the full-size workloads, run in the
same launch configuration as the benchmark, compare every block index of a
few heads and every output element of sampled query blocks (the oracle
computes those one by one).  Pooled vectors must match bit for bit; block
indices exactly, except inside the tie zone; outputs within max-abs 2e-2 and
mean-abs 2e-3 of the float64 oracle.
"""
import math
import sys

import numpy as np
import pytest

import block_sparse_attention_25_amd as bsa
from block_sparse_attention_25_amd.synth import WORKLOADS, custom, generate
from oracle import bsa_oracle as O
from tests.parity import (MAX_ABS, MEAN_ABS, check_idx_row, check_idx_row_forced, check_idx_rows,
                          check_idx_row_threshold, check_output, check_tokens_row, tensor_bits,
                          to_device, widen)

pytestmark = pytest.mark.gpu


def _log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    bsa.lib()
    return torch


def _run_gpu(torch, qb, kb, vb, nan_out=False, **kw):
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    if nan_out:
        # every output element must be written: start from NaN everywhere
        kw["out"] = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=q.device)
    out, aux = bsa.attention(q, k, v, return_aux=True, **kw)
    torch.cuda.synchronize()
    host = {n: aux[n].cpu() for n in ("q_pool", "k_pool", "sum_k", "sum_v", "sum_bias", "block_idx")}
    host["token_idx"] = None if aux["token_idx"] is None else aux["token_idx"].cpu()
    host["out"] = out
    return host


def _check_tokens(host, qp, K, gidx, b, h, E, rows, sinks, label):
    """Extra-token rows of one (b, h) against the oracle's float64 ranking."""
    gtok = host["token_idx"][b, h].numpy()
    nb = gidx.shape[0]
    assert gtok.shape == (nb, E)
    want = O.select_extra_tokens(qp, K, gidx, E, dense_blocks=sinks, query_blocks=rows)
    ties = 0
    for r in rows:
        if r in sinks:
            assert np.all(gtok[r] == -1), "%s sink row %d has extra tokens" % (label, r)
            continue
        chosen = set(int(c) for c in gidx[r] if c >= 0)
        cand = [j for c in range(nb) if c not in chosen
                for j in range(c * 128, min(c * 128 + 128, K.shape[0]))]
        sc = K[cand] @ qp[r] if cand else np.zeros(0)
        ok, tie = check_tokens_row(gtok[r], cand, sc, E)
        assert ok, "%s token row %d: gpu %s want %s" % (label, r, list(gtok[r][:8]), list(want[r][:8]))
        if not tie:
            assert np.array_equal(gtok[r], want[r]), "%s token row %d" % (label, r)
        ties += tie
    return gtok, ties


def _check_head(host, qb, kb, vb, b, h, top_k, summary="mean", anchor_rows=0,
                query_blocks=None, label="", sink_start=0, sink_rows=0, tau=None, extra=0):
    """Compare one (b, h) of a GPU run with the oracle; returns (tie-zone
    rows, max-abs, mean-abs of the checked output rows)."""
    Q, K, V = (widen(x[b, h]) for x in (qb, kb, vb))
    N = Q.shape[0]
    nb = O.n_blocks(N)
    sinks = O.sink_blocks(N, sink_start, sink_rows)
    k = len(sinks) + O.effective_k(top_k, nb - len(sinks))
    sc = O.default_scale(Q.shape[1])
    # stage 1: pooled vectors bit-exact
    qp, kp = O.pool_mean(Q), O.pool_mean(K)
    assert np.array_equal(host["q_pool"][b, h].numpy(), qp), label + " q_pool"
    assert np.array_equal(host["k_pool"][b, h].numpy(), kp), label + " k_pool"
    # summaries
    if summary == "mean":
        sk, sv, bias = O.summaries_mean(K, V)
    else:
        a = O.anchor(Q, anchor_rows)
        sk, sv, bias = O.summaries_reweight(K, V, a, sc)
    gsk = widen(tensor_bits(host["sum_k"][b, h]))
    gsv = widen(tensor_bits(host["sum_v"][b, h]))
    # one bf16 rounding (via float32): within 2^-8 relative
    assert np.all(np.abs(gsk - sk) <= 2.0 ** -8 * np.abs(sk) + 1e-30), label + " sum_k"
    assert np.all(np.abs(gsv - sv) <= 2.0 ** -8 * np.abs(sv) + 1e-30), label + " sum_v"
    gb = host["sum_bias"][b, h].numpy().astype(np.float64)
    assert np.all(np.abs(gb - bias) <= 1e-6 + 1e-6 * np.abs(bias)), label + " sum_bias"
    # stage 2: indices
    s = O.block_scores(qp, kp)
    gidx = host["block_idx"][b, h].numpy()
    assert gidx.shape == (nb, k)
    ties = 0
    if k > 0:
        want = O.select_threshold(s, tau, top_k, sinks) if tau is not None else None
        for r in range(nb):
            if tau is not None:
                ok, tie = check_idx_row_threshold(gidx[r], s[r], want[r], sinks, tau)
            elif sinks:
                ok, tie = check_idx_row_forced(gidx[r], s[r], k, sinks)
            else:
                break
            assert ok, "%s idx row %d: gpu %s" % (label, r, list(gidx[r]))
            ties += tie
        if tau is None and not sinks:
            # plain top-k: every row at once against the oracle's ranking
            bad, ties = check_idx_rows(gidx, s, k)
            assert not bad, "%s idx rows %s: gpu %s" % (label, bad[:4], list(gidx[bad[0]]))
    # extra tokens: the rows checked below, against the float64 ranking
    gtok = None
    if extra:
        rows_t = list(range(nb)) if query_blocks is None else list(query_blocks)
        gtok, tties = _check_tokens(host, qp, K, gidx if k > 0 else np.zeros((nb, 0), np.int32),
                                    b, h, extra, rows_t, sinks, label)
        ties += tties
    # stages 3+4: output with the GPU's (validated) selection
    ref = O.attention(Q, K, V, gidx if k > 0 else np.zeros((nb, 0), np.int32), sk, sv, bias, sc,
                      query_blocks=query_blocks, dense_blocks=sinks, extra=gtok)
    gout = widen(tensor_bits(host["out"][b, h].cpu()))
    if query_blocks is None:
        rows = np.arange(N)
    else:
        rows = np.concatenate([np.arange(r * 128, min(r * 128 + 128, N)) for r in query_blocks])
    mx, mean = check_output(gout[rows], ref[rows])
    _log("  %s b%d h%d: out max %.3g mean %.3g, tie rows %d" % (label, b, h, mx, mean, ties))
    assert mx <= MAX_ABS and mean <= MEAN_ABS, "%s out max %g mean %g" % (label, mx, mean)
    return ties, mx, mean


# --------------------------------------------------------------- small ---
def test_tiny_workload_mean(torch_cuda):
    w = WORKLOADS["tiny"]
    _log("case tiny mean")
    qb, kb, vb = generate(w)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=w.top_k)
    for h in range(w.heads):
        _check_head(host, qb, kb, vb, 0, h, w.top_k, label="tiny")


def test_tiny_workload_reweight(torch_cuda):
    w = WORKLOADS["tiny"]
    _log("case tiny reweight")
    qb, kb, vb = generate(w)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=w.top_k, summary="reweight",
                    anchor_rows=w.anchor_rows)
    for h in range(w.heads):
        _check_head(host, qb, kb, vb, 0, h, w.top_k, "reweight", w.anchor_rows, label="tiny-rw")


@pytest.mark.parametrize("N,top_k", [(1, 1), (1, 0), (100, 0), (128, 1), (129, 1), (129, 0),
                                     (300, 2), (1000, 0), (1000, 3), (1000, 8), (1000, 50),
                                     (4076, 5), (8191, 16)])
def test_ragged_and_edge_sizes(torch_cuda, N, top_k):
    _log("case N=%d top_k=%d" % (N, top_k))
    w = custom(N, heads=2, seed=N + top_k)
    qb, kb, vb = generate(w)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=top_k)
    for h in range(2):
        _check_head(host, qb, kb, vb, 0, h, top_k, label="N%d-k%d" % (N, top_k))


@pytest.mark.parametrize("N,top_k,anchor_rows", [(1000, 3, 0), (1000, 3, 700), (300, 0, 200),
                                                 (4076, 9, 4000)])
def test_reweight_sizes(torch_cuda, N, top_k, anchor_rows):
    _log("case reweight N=%d top_k=%d anchor=%d" % (N, top_k, anchor_rows))
    w = custom(N, heads=2, seed=7 * N + top_k)
    qb, kb, vb = generate(w)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=top_k, summary="reweight", anchor_rows=anchor_rows)
    for h in range(2):
        _check_head(host, qb, kb, vb, 0, h, top_k, "reweight", anchor_rows, label="rw%d" % N)


@pytest.mark.parametrize("N,top_k,start,rows,summary", [
    (4096, 8, 4032, 64, "mean"),      # the tiny shape: conditioning rows in the last block
    (1000, 3, 900, 100, "mean"),      # sinks in the short last block
    (1000, 2, 300, 200, "mean"),      # sinks in the middle, straddling a block boundary
    (1000, 0, 0, 1, "mean"),          # top_k 0: sink block plus summaries
    (300, 5, 0, 300, "mean"),         # every block a sink: dense attention
    (1000, 3, 900, 100, "reweight"),
    (2000, 20, 1900, 100, "mean"),    # top_k above the blocks left after the sinks
])
def test_conditioning_sinks(torch_cuda, N, top_k, start, rows, summary):
    _log("case sinks N=%d top_k=%d sink=[%d,+%d) %s" % (N, top_k, start, rows, summary))
    w = custom(N, heads=2, seed=N + 3 * top_k + start)
    qb, kb, vb = generate(w)
    anchor = start if summary == "reweight" else 0
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=top_k, summary=summary, anchor_rows=anchor,
                    sink_start=start, sink_rows=rows)
    for h in range(2):
        _check_head(host, qb, kb, vb, 0, h, top_k, summary, anchor, label="sink%d" % N,
                    sink_start=start, sink_rows=rows)


@pytest.mark.parametrize("N,top_k,tau,sink,summary", [
    (1000, 8, 0.5, 0, "mean"),
    (4096, 32, 1.0, 0, "mean"),      # the tiny shape, uncapped
    (2000, 5, -0.5, 0, "mean"),      # the cap binds on most rows
    (1000, 8, 3.0, 0, "mean"),       # most rows keep nothing: summary rows only
    (1000, 8, 0.5, 100, "mean"),     # with conditioning sinks in the last block
    (1000, 6, 0.8, 0, "reweight"),
])
def test_threshold_selection(torch_cuda, N, top_k, tau, sink, summary):
    _log("case threshold N=%d cap=%d tau=%g sink=%d %s" % (N, top_k, tau, sink, summary))
    w = custom(N, heads=2, seed=N + int(10 * tau) + sink)
    qb, kb, vb = generate(w)
    anchor = 800 if summary == "reweight" else 0
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=top_k, summary=summary, anchor_rows=anchor,
                    sink_rows=sink, tau=tau)
    for h in range(2):
        _check_head(host, qb, kb, vb, 0, h, top_k, summary, anchor, label="thr%d" % N,
                    sink_start=N - sink if sink else 0, sink_rows=sink, tau=tau)


@pytest.mark.parametrize("N", [140000, 159900, 166000])
@pytest.mark.parametrize("variant", ["plain", "ties", "sinks", "threshold"])
def test_many_blocks_selection(torch_cuda, variant, N):
    """The selection's large-row forms at 1,094 blocks (short last block): the
    float64 matrix scores, with the high key halves in LDS for top-k and the
    float64 rows of one 16-wavefront workgroup for the threshold; at 1,250
    blocks the high-half kernel for top-k and the row-split float64 VALU
    scores for the threshold; at 1,297 blocks the VALU scores for all.  Every
    index of the head against the oracle, and sampled query blocks."""
    _log("case many blocks %s N=%d" % (variant, N))
    nb = O.n_blocks(N)
    w = custom(N, heads=1, seed=17)
    qb, kb, vb = generate(w, threads=16)
    kw = dict(top_k=16)
    check = dict()
    if variant == "ties":
        kb = kb.copy()
        for dst in (1000, 1001):
            kb[0, 0, dst * 128:(dst + 1) * 128] = kb[0, 0, 256:384]
    elif variant == "sinks":
        kw.update(sink_rows=1000)
        check.update(sink_start=N - 1000, sink_rows=1000)
    elif variant == "threshold":
        kw.update(tau=1.5, top_k=40)
        check.update(tau=1.5)
    host = _run_gpu(torch_cuda, qb, kb, vb, **kw)
    _check_head(host, qb, kb, vb, 0, 0, kw["top_k"], query_blocks=[0, 250, nb - 2, nb - 1],
                label="nb%d-%s" % (nb, variant), **check)
    if variant == "ties":
        s = O.block_scores(O.pool_mean(widen(qb[0, 0])), O.pool_mean(widen(kb[0, 0])))
        assert np.array_equal(host["block_idx"][0, 0].numpy(), O.select_topk(s, 16))


@pytest.mark.parametrize("nb", [200, 300, 600, 1094, 1250])
def test_select_near_ties_high_half_keys(torch_cuda, nb):
    """Top-k keeps only the high 32 bits of each score's key in LDS and ranks
    the blocks that tie there by their float64 scores computed again (every
    kernel size up to 1,280 blocks).  Pooled vectors made here, through bsa_select: every key block is
    one vector plus 0..3 float32 ulps on six features, so a row's scores lie
    within about 1e-6 of each other (most share their high bits, some exactly
    equal).  The indices must equal the float64 oracle's, ties to the lower
    index."""
    torch = torch_cuda
    _log("case select near ties nb=%d" % nb)
    rng = np.random.default_rng(nb)
    qp = rng.standard_normal((nb, 128)).astype(np.float32)
    base = rng.standard_normal(128).astype(np.float32) + np.float32(4.0)
    kp = np.repeat(base[None, :], nb, axis=0)
    feats = rng.choice(128, size=6, replace=False)
    steps = rng.integers(0, 4, size=(nb, 6))
    for j, f in enumerate(feats):
        kp[:, f] = base[f] + steps[:, j].astype(np.float32) * np.spacing(base[f])
    top_k = 16
    p = bsa.make_problem(1, 1, nb * 128, top_k=top_k)
    dq = torch.from_numpy(qp).reshape(1, 1, nb, 128).cuda()
    dk = torch.from_numpy(kp).reshape(1, 1, nb, 128).cuda()
    idx = torch.full((1, 1, nb, top_k), -7, dtype=torch.int32, device="cuda")
    bsa.bsa_select(p, dq, dk, idx)
    torch.cuda.synchronize()
    want = O.select_topk(O.block_scores(qp.astype(np.float64), kp.astype(np.float64)), top_k)
    got = idx[0, 0].cpu().numpy()
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, "rows %s: gpu %s want %s" % (bad[:4], list(got[bad[0]]), list(want[bad[0]]))


def test_forward_with_given_indices(torch_cuda):
    """bsa_forward on an index set chosen here (random ascending rows, not the
    GPU's own selection) against the oracle's attention on the same rows."""
    torch = torch_cuda
    _log("case forward with given indices")
    N, H, top_k = 3000, 2, 7
    w = custom(N, heads=H, seed=31)
    qb, kb, vb = generate(w)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    out, aux = bsa.attention(q, k, v, top_k=top_k, return_aux=True)
    nb = O.n_blocks(N)
    rng = np.random.default_rng(5)
    idx = np.stack([np.stack([np.sort(rng.choice(nb, top_k, replace=False)) for _ in range(nb)])
                    for _ in range(H)])[None].astype(np.int32)
    gidx = torch.from_numpy(idx).cuda()
    out2 = torch.empty_like(q)
    bsa.bsa_forward(aux["problem"], q, k, v, aux["sum_k"], aux["sum_v"], aux["sum_bias"], gidx, out2,
                    aux["workspace"])
    torch.cuda.synchronize()
    for h in range(H):
        Q, K, V = (widen(x[0, h]) for x in (qb, kb, vb))
        sk, sv, bias = O.summaries_mean(K, V)
        ref = O.attention(Q, K, V, idx[0, h], sk, sv, bias, O.default_scale(128))
        mx, mean = check_output(widen(tensor_bits(out2[0, h])), ref)
        _log("  given idx h%d: out max %.3g mean %.3g" % (h, mx, mean))
        assert mx <= MAX_ABS and mean <= MEAN_ABS


@pytest.mark.parametrize("tau", [None, 0.5])
def test_forward_with_caller_summaries(torch_cuda, tau):
    """bsa_forward on inputs that no bsa_pool call produced: a V unrelated to
    the pooled one, random summary keys, values and biases, and the GPU's
    block selection; against the oracle's attention on exactly those tensors.
    The same call without a workspace (query blocks in plain order) gives the
    same bits, and a changed sum_v changes the output as the oracle says."""
    torch = torch_cuda
    _log("case forward with caller summaries tau=%s" % tau)
    N, H, top_k = 3000, 2, 7
    w = custom(N, heads=H, seed=37)
    qb, kb, vb = generate(w)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    out, aux = bsa.attention(q, k, v, top_k=top_k, tau=tau, return_aux=True)
    p, idx = aux["problem"], aux["block_idx"]
    nb = O.n_blocks(N)
    rng = np.random.default_rng(9)
    from block_sparse_attention_25_amd.synth import bf16_bits
    v2b = bf16_bits(rng.standard_normal((1, H, N, 128)).astype(np.float32))
    skb = bf16_bits(rng.standard_normal((1, H, nb, 128)).astype(np.float32))
    svb = bf16_bits(rng.standard_normal((1, H, nb, 128)).astype(np.float32))
    bias = rng.uniform(-2.0, 2.0, (1, H, nb)).astype(np.float32)
    v2, sk, sv = to_device(v2b), to_device(skb), to_device(svb)
    sb = torch.from_numpy(bias).cuda()
    out_ws, out_nows = torch.empty_like(q), torch.empty_like(q)
    bsa.bsa_forward(p, q, k, v2, sk, sv, sb, idx, out_ws, aux["workspace"])
    bsa.bsa_forward(p, q, k, v2, sk, sv, sb, idx, out_nows, None)
    # then sum_v doubled in place: the next call must read the new values
    sv2 = sv.float().mul(2.0).to(torch.bfloat16)
    out_sv2 = torch.empty_like(q)
    bsa.bsa_forward(p, q, k, v2, sk, sv2, sb, idx, out_sv2, aux["workspace"])
    torch.cuda.synchronize()
    assert torch.equal(out_ws.view(torch.int16), out_nows.view(torch.int16))
    gidx = idx.cpu().numpy()
    sc = O.default_scale(128)
    for h in range(H):
        Q, K = widen(qb[0, h]), widen(kb[0, h])
        V2, SK, SV = widen(v2b[0, h]), widen(skb[0, h]), widen(svb[0, h])
        B_ = bias[0, h].astype(np.float64)
        for got, sv_used in ((out_ws, SV), (out_sv2, 2.0 * SV)):
            ref = O.attention(Q, K, V2, gidx[0, h], SK, sv_used, B_, sc)
            mx, mean = check_output(widen(tensor_bits(got[0, h])), ref)
            _log("  caller summaries h%d: out max %.3g mean %.3g" % (h, mx, mean))
            assert mx <= MAX_ABS and mean <= MEAN_ABS


@pytest.mark.parametrize("batch,heads,extra", [(1, 3, 0), (2, 1, 0), (1, 1, 64)])
def test_head_synchronous_map_every_block(torch_cuda, batch, heads, extra):
    """Past 384 blocks the attention grid deals each head to the 8 XCDs in
    chunks of ceil(nb / 8) query blocks with padding workgroups at the end
    (391 blocks: chunks of 49, one padding workgroup per head); every query
    block of every head against the oracle (with extra tokens, whose oracle
    is slow, the query blocks on both sides of each chunk boundary and the
    last two)."""
    N = 50000
    _log("case head-synchronous map batch=%d heads=%d extra=%d" % (batch, heads, extra))
    w = custom(N, heads=heads, batch=batch, seed=43 + extra + batch)
    qb, kb, vb = generate(w, threads=16)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=4, extra_tokens=extra)
    rows = None if not extra else sorted({0, 389, 390} | {49 * x + d for x in range(1, 8) for d in (-1, 0)})
    for b in range(batch):
        for h in range(heads):
            _check_head(host, qb, kb, vb, b, h, 4, label="nb391-b%d-h%d" % (b, h), extra=extra,
                        query_blocks=rows)


@pytest.mark.parametrize("N", [262144, 262100])
def test_maximum_size(torch_cuda, N):
    """The largest supported sequence: 2,048 blocks (exact and ragged)."""
    _log("case maximum size N=%d" % N)
    w = custom(N, heads=1, seed=3)
    qb, kb, vb = generate(w, threads=16)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=64)
    _check_head(host, qb, kb, vb, 0, 0, 64, query_blocks=[0, 1024, 2046, 2047], label="max%d" % N)


def test_all_zero_inputs(torch_cuda):
    """Every score ties: the lowest block indices win, and the output (softmax
    over equal logits of zero values) is exactly zero."""
    torch = torch_cuda
    _log("case all-zero inputs")
    N, H = 1000, 2
    z = np.zeros((1, H, N, 128), dtype=np.uint16)
    host = _run_gpu(torch, z, z, z, top_k=3)
    assert np.array_equal(host["block_idx"].numpy(), np.broadcast_to(np.arange(3, dtype=np.int32),
                                                                     (1, H, 8, 3)))
    assert not bool(host["out"].float().abs().gt(0).any())


@pytest.mark.parametrize("summary,extra,tau", [
    ("mean", 0, None),
    ("reweight", 0, None),   # the summary bias on top of large logits
    ("mean", 64, None),      # exact-max extra-token groups, then the lazy running max
    ("mean", 0, 1.0),        # threshold selection: rows of different lengths
])
def test_large_logits(torch_cuda, summary, extra, tau):
    """Q and K scaled up so logits span thousands: the softmax is close to
    one-hot; the online rescaling must match the oracle's max subtraction."""
    _log("case large logits %s E=%d tau=%s" % (summary, extra, tau))
    N = 1500
    w = custom(N, heads=2, seed=13)
    qb, kb, vb = generate(w)
    from block_sparse_attention_25_amd.synth import bf16_bits
    qb = bf16_bits((widen(qb) * 24.0).astype(np.float32))
    kb = bf16_bits((widen(kb) * 24.0).astype(np.float32))
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=4, summary=summary, tau=tau, extra_tokens=extra)
    for h in range(2):
        _check_head(host, qb, kb, vb, 0, h, 4, summary, 0, label="large", tau=tau, extra=extra)


def test_batch_and_heads(torch_cuda):
    _log("case batch 2 x heads 3")
    w = custom(1500, heads=3, batch=2, seed=3)
    qb, kb, vb = generate(w)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=4)
    for b in range(2):
        for h in range(3):
            _check_head(host, qb, kb, vb, b, h, 4, label="bh")


def test_exact_ties_take_lower_index(torch_cuda):
    """Key block 2 copied into blocks 5 and 6: their scores tie bit-exactly, and
    the lower index must win wherever only some of them fit."""
    _log("case exact ties")
    w = custom(1024, heads=1, seed=11)
    qb, kb, vb = generate(w)
    kb = kb.copy()
    vb = vb.copy()
    for dst in (5, 6):
        kb[0, 0, dst * 128:(dst + 1) * 128] = kb[0, 0, 256:384]
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=3)
    Q, K = widen(qb[0, 0]), widen(kb[0, 0])
    s = O.block_scores(O.pool_mean(Q), O.pool_mean(K))
    want = O.select_topk(s, 3)
    assert np.array_equal(host["block_idx"][0, 0].numpy(), want)
    _check_head(host, qb, kb, vb, 0, 0, 3, label="ties")


@pytest.mark.parametrize("extra", [0, 256])
def test_deterministic_repeats(torch_cuda, extra):
    _log("case determinism, extra tokens %d" % extra)
    w = custom(3000, heads=2, seed=5)
    qb, kb, vb = generate(w)
    a = _run_gpu(torch_cuda, qb, kb, vb, top_k=6, summary="reweight", anchor_rows=2500,
                 extra_tokens=extra)
    b = _run_gpu(torch_cuda, qb, kb, vb, top_k=6, summary="reweight", anchor_rows=2500,
                 extra_tokens=extra)
    for n in a:
        x, y = a[n], b[n]
        if x is None:
            assert y is None, n
            continue
        if hasattr(x, "is_cuda") and x.is_cuda:
            x, y = x.cpu(), y.cpu()
        assert torch_cuda.equal(x.view(torch_cuda.uint8) if x.dtype == torch_cuda.bfloat16 else x,
                                y.view(torch_cuda.uint8) if y.dtype == torch_cuda.bfloat16 else y), n


def test_guard_bands_untouched(torch_cuda):
    """Outputs written through the raw entry points into poisoned buffers: every
    element inside is written, and guard regions after each output stay as
    poisoned."""
    torch = torch_cuda
    _log("case guard bands")
    N, H, top_k = 1000, 2, 3
    w = custom(N, heads=H, seed=2)
    qb, kb, vb = generate(w)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    p = bsa.make_problem(1, H, N, top_k)
    nb, kk = bsa.bsa_problem_blocks(p)
    G = 4096

    def poisoned(n, dtype):
        if dtype == torch.int32:
            buf = torch.full((n + G,), -7, dtype=dtype, device="cuda")
        elif dtype == torch.bfloat16:
            buf = torch.full((n + G,), float("nan"), dtype=torch.float32, device="cuda").to(dtype)
        else:
            buf = torch.full((n + G,), float("nan"), dtype=dtype, device="cuda")
        return buf

    f32, bf = torch.float32, torch.bfloat16
    bufs = dict(q_pool=poisoned(H * nb * 128, f32), k_pool=poisoned(H * nb * 128, f32),
                sum_k=poisoned(H * nb * 128, bf), sum_v=poisoned(H * nb * 128, bf),
                sum_bias=poisoned(H * nb, f32), idx=poisoned(H * nb * kk, torch.int32),
                out=poisoned(H * N * 128, bf))
    n_of = dict(q_pool=H * nb * 128, k_pool=H * nb * 128, sum_k=H * nb * 128, sum_v=H * nb * 128,
                sum_bias=H * nb, idx=H * nb * kk, out=H * N * 128)
    ws = torch.empty(bsa.bsa_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    bsa.bsa_pool(p, q, k, v, bufs["q_pool"], bufs["k_pool"], bufs["sum_k"], bufs["sum_v"],
                 bufs["sum_bias"], ws)
    bsa.bsa_select(p, bufs["q_pool"], bufs["k_pool"], bufs["idx"])
    bsa.bsa_forward(p, q, k, v, bufs["sum_k"], bufs["sum_v"], bufs["sum_bias"], bufs["idx"], bufs["out"], ws)
    torch.cuda.synchronize()
    for name, buf in bufs.items():
        n = n_of[name]
        inside, guard = buf[:n].cpu(), buf[n:].cpu()
        if buf.dtype == torch.int32:
            assert bool((inside >= 0).all()), name
            assert bool((guard == -7).all()), name
        else:
            assert not bool(torch.isnan(inside.float()).any()), name
            assert bool(torch.isnan(guard.float()).all()), name


# --------------------------------------------------------- extra tokens ---
@pytest.mark.parametrize("N,top_k,E,sink,summary,tau", [
    (4096, 8, 64, 0, "mean", None),      # the tiny shape
    (4096, 8, 256, 64, "mean", None),    # with its conditioning rows as sinks
    (1000, 3, 100, 0, "mean", None),     # E not a multiple of 64, short last block
    (1000, 7, 256, 0, "mean", None),     # one skipped block: fewer candidates than E
    (1000, 0, 200, 0, "mean", None),     # top_k 0: every token a candidate
    (1000, 8, 50, 0, "mean", None),      # every block kept: no candidates
    (2000, 5, 256, 0, "reweight", None),
    (2000, 10, 128, 0, "mean", 0.5),     # threshold selection (rows keep different counts)
    (300, 1, 1, 0, "mean", None),        # one extra token
    (1, 0, 5, 0, "mean", None),          # one token, a candidate
    (129, 1, 10, 0, "mean", None),       # two blocks, the second of one row
    (9000, 16, 256, 0, "mean", None),    # several row groups of 32 query blocks
])
def test_extra_tokens(torch_cuda, N, top_k, E, sink, summary, tau):
    _log("case extra tokens N=%d top_k=%d E=%d sink=%d %s tau=%s" % (N, top_k, E, sink, summary, tau))
    w = custom(N, heads=2, seed=N + E + top_k)
    qb, kb, vb = generate(w)
    anchor = N // 2 if summary == "reweight" else 0
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=top_k, summary=summary, anchor_rows=anchor,
                    sink_rows=sink, tau=tau, extra_tokens=E)
    for h in range(2):
        _check_head(host, qb, kb, vb, 0, h, top_k, summary, anchor, label="extra%d-%d" % (N, E),
                    sink_start=N - sink if sink else 0, sink_rows=sink, tau=tau, extra=E)


@pytest.mark.parametrize("N,batch,heads,check", [
    (4200, 1, 129, ((0, 0), (0, 127), (0, 128))),  # 258 groups: the last 2 split into 8 parts of 4-5 blocks
    (9000, 1, 90, ((0, 0), (0, 85), (0, 89))),     # 270 groups: the last 14 (from head 85 on) in 8 parts of ~9 blocks
    (4200, 2, 65, ((0, 0), (1, 63), (1, 64))),     # 260 groups over two batch entries: the last 4 (b 1, h 63 and 64) split
])
def test_extra_tokens_split_groups(torch_cuda, N, batch, heads, check):
    """Token selection runs one workgroup per CU; the groups of 32 query
    blocks past the last whole round split their key blocks into parts whose
    best keys a merge kernel combines.  Every row of heads on both sides of
    that line against the oracle."""
    _log("case extra tokens, split groups N=%d batch=%d heads=%d" % (N, batch, heads))
    w = custom(N, heads=heads, batch=batch, seed=N + heads + batch)
    qb, kb, vb = generate(w, threads=16)
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=16, extra_tokens=256)
    for b, h in check:
        _check_head(host, qb, kb, vb, b, h, 16, label="split%d-b%dh%d" % (N, b, h), extra=256)


def test_extra_token_ties_take_lower_index(torch_cuda):
    """300 copies of one strong key row in blocks 20..31 tie bit-exactly: where
    the E-th place falls among the copies, the lowest copies must win."""
    _log("case extra-token ties")
    from block_sparse_attention_25_amd.synth import bf16_bits
    N, E = 4096, 256
    w = custom(N, heads=1, seed=23)
    qb, kb, vb = generate(w)
    K0 = widen(kb[0, 0])
    qm = widen(qb[0, 0])[:128].mean(axis=0)
    src = bf16_bits((3.0 * K0[128 + int(np.argmax(K0[128:256] @ qm))]).astype(np.float32))
    rng = np.random.default_rng(1)
    dst = np.sort(rng.choice(np.arange(20 * 128, 32 * 128), 300, replace=False))
    kb = kb.copy()
    kb[0, 0, dst] = src
    host = _run_gpu(torch_cuda, qb, kb, vb, top_k=2, extra_tokens=E)
    _check_head(host, qb, kb, vb, 0, 0, 2, label="extra-ties", extra=E)
    Q, K = widen(qb[0, 0]), widen(kb[0, 0])
    qp = O.pool_mean(Q)
    gidx = host["block_idx"][0, 0].numpy()
    gtok = host["token_idx"][0, 0].numpy()
    want = O.select_extra_tokens(qp, K, gidx, E)
    copies = set(int(t) for t in dst)
    exact_rows = 0
    for r in range(gidx.shape[0]):
        chosen = set(int(c) for c in gidx[r])
        cand = [j for c in range(32) if c not in chosen for j in range(c * 128, c * 128 + 128)]
        sc = K[cand] @ qp[r]
        order = sorted(range(len(cand)), key=lambda i: (-sc[i], cand[i]))
        if len(cand) > E and cand[order[E - 1]] in copies and cand[order[E]] in copies:
            assert np.array_equal(gtok[r], want[r]), "row %d" % r
            exact_rows += 1
    _log("  rows whose E-th place falls among the copies: %d" % exact_rows)
    assert exact_rows > 0


def test_forward_tokens_matches_forward_without_tokens(torch_cuda):
    """bsa_forward_tokens with every token row empty (-1) gives bsa_forward's
    output bit for bit: the empty softmax state is the plain start."""
    torch = torch_cuda
    _log("case forward_tokens with empty rows")
    N, H = 3000, 2
    w = custom(N, heads=H, seed=41)
    qb, kb, vb = generate(w)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    out, aux = bsa.attention(q, k, v, top_k=5, return_aux=True)
    pe = bsa.make_problem(1, H, N, 5, extra_tokens=64)
    ws = torch.empty(bsa.bsa_workspace_bytes(pe), dtype=torch.uint8, device="cuda")
    nb = O.n_blocks(N)
    q_pool = torch.empty((1, H, nb, 128), dtype=torch.float32, device="cuda")
    k_pool, sum_bias = torch.empty_like(q_pool), torch.empty((1, H, nb), dtype=torch.float32, device="cuda")
    sum_k = torch.empty((1, H, nb, 128), dtype=torch.bfloat16, device="cuda")
    sum_v = torch.empty_like(sum_k)
    bsa.bsa_pool(pe, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, ws)
    tok = torch.full((1, H, nb, 64), -1, dtype=torch.int32, device="cuda")
    out2 = torch.empty_like(q)
    bsa.bsa_forward_tokens(pe, q, k, v, sum_k, sum_v, sum_bias, aux["block_idx"], tok, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ---------------------------------------------------------- full sizes ---
FULL = [("768p_5s", [0, 37]), ("768p_10s", [5]), ("2k_5s", [55]), ("768p_15s_reweight", [0, 21]),
        ("768p_5s_sinks", [9]), ("768p_5s_tau1", [17]), ("768p_5s_extra256", [3, 50])]


@pytest.mark.parametrize("name,heads", FULL)
def test_full_size_workloads(torch_cuda, name, heads):
    """Every head of the workload runs in one launch, as in the benchmark,
    into an output prefilled with NaN.  Then, for EVERY head: pooled vectors
    bit-exact, summaries within one bf16 rounding, every block index against
    the oracle's float64 ranking (tie zone aside), one query block compared
    element-wise (a different one per head, so the launch's whole grid map is
    sampled; with extra tokens its token row too), and no NaN left anywhere.
    The first head listed is compared in every query block (its whole output
    and, with extra tokens, every token row); the others listed also get the
    first, second, middle, last-but-one and short last query blocks.  Prints
    the worst output error of the workload."""
    torch = torch_cuda
    w = WORKLOADS[name]
    _log("case full %s (H=%d N=%d)" % (name, w.heads, w.seq_len))
    qb, kb, vb = generate(w, threads=16)
    nb = O.n_blocks(w.seq_len)
    top_k = w.top_k if w.top_k is not None else O.k_from_ratio(w.top_k_ratio, nb)
    kw = dict(top_k=top_k, summary=w.summary, sink_start=w.sink_start, sink_rows=w.sink_rows,
              tau=w.tau, extra_tokens=w.extra)
    if w.summary == "reweight":
        kw["anchor_rows"] = w.anchor_rows
    host = _run_gpu(torch, qb, kb, vb, nan_out=True, **kw)
    assert not bool(torch.isnan(host["out"].float()).any()), "output elements left unwritten"
    sinks = O.sink_blocks(w.seq_len, w.sink_start, w.sink_rows)
    kk = len(sinks) + min(top_k, nb - len(sinks))
    idx = host["block_idx"].numpy()
    assert idx.shape == (1, w.heads, nb, kk)
    if w.tau is not None:
        nvalid = (idx >= 0).sum(-1)
        _log("  kept blocks per row: min %d mean %.1f max %d of %d"
             % (nvalid.min(), nvalid.mean(), nvalid.max(), nb))
    sampled = [0, 1, nb // 2, nb - 2, nb - 1]
    if sinks:
        sampled = sorted(set(sampled + [sinks[0] - 1, sinks[0]]))  # last video block, first sink block
    worst_max, worst_mean, ties = 0.0, 0.0, 0
    for h in range(w.heads):
        qbs = None if h == heads[0] else sorted(set([(7 * h + 3) % nb] + (sampled if h in heads else [])))
        t, mx, mean = _check_head(host, qb, kb, vb, 0, h, top_k, w.summary,
                                  w.anchor_rows if w.summary == "reweight" else 0, query_blocks=qbs,
                                  label=name, sink_start=w.sink_start, sink_rows=w.sink_rows, tau=w.tau,
                                  extra=w.extra)
        worst_max, worst_mean, ties = max(worst_max, mx), max(worst_mean, mean), ties + t
    _log("  %s all %d heads: worst out max-abs %.4g (bound %g), worst mean-abs %.4g (bound %g), "
         "tie-zone rows %d" % (name, w.heads, worst_max, MAX_ABS, worst_mean, MEAN_ABS, ties))

"""GPU parity of Spark-Reblock: the permutation against the float64 oracle,
then the whole path on the GPU's order against the oracle run on that order.

The permutation must equal the oracle's wherever the oracle's own splits are
decided by more than the float32 rounding of the GPU's embedding; elsewhere
every GPU split is checked for validity against the float64 embedding
(tests/parity.py: check_partition).  Downstream of the permutation the
checks are those of the other parity tests, on the permuted rows.
"""
import sys

import numpy as np
import pytest

import block_sparse_attention_25_amd as bsa
from block_sparse_attention_25_amd.synth import WORKLOADS, custom, generate
from oracle import bsa_oracle as O
from tests.parity import (REBLOCK_DIST_ABS, REBLOCK_KEY_ABS, check_partition, reblock_margins,
                          tensor_bits, to_device, widen)
from tests.test_gpu_parity import _check_head

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


def _gpu_perm(torch, qb, kb):
    q, k = to_device(qb), to_device(kb)
    B, H, N, _ = q.shape
    p = bsa.make_problem(B, H, N, top_k=0)
    perm = torch.empty((B, H, N), dtype=torch.int32, device="cuda")
    ws = torch.empty(bsa.bsa_reblock_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    bsa.bsa_reblock(p, q, k, perm, ws)
    torch.cuda.synchronize()
    return perm.cpu().numpy()


def _check_perm(gperm, Q, K, label):
    """One head: valid against the float64 embedding; equal to the oracle's
    order when its margins exceed the tolerances.  Returns True if equal."""
    z = O.mahalanobis_embedding(Q, K)
    ok, msg = check_partition(z, gperm, O.reblock_left_rows)
    assert ok, "%s: %s" % (label, msg)
    want = O.reblock_permutation(Q, K)
    dgap, kgap = reblock_margins(z, want, O.reblock_left_rows)
    same = np.array_equal(gperm, want)
    _log("  %s: equal %s, oracle margins: pivot distance %.2g, split key %.2g" % (label, same, dgap, kgap))
    if dgap > REBLOCK_DIST_ABS and kgap > REBLOCK_KEY_ABS:
        assert same, label + ": differs from the oracle's order away from near-ties"
    return same


@pytest.mark.parametrize("N", [100, 128, 129, 1000, 4173])
def test_reblock_permutation(torch_cuda, N):
    _log("case reblock perm N=%d" % N)
    qb, kb, _ = generate(custom(N, heads=2, seed=60), threads=2)
    gperm = _gpu_perm(torch_cuda, qb, kb)
    for h in range(2):
        _check_perm(gperm[0, h], widen(qb[0, h]), widen(kb[0, h]), "N=%d h%d" % (N, h))


def test_reblock_hand_partition(torch_cuda):
    # four clusters of unit vectors at 0, 30, 80 and 120 degrees in
    # coordinates 0, 1 (the second and fourth noisier) and isotropic keys:
    # the order is fixed by hand (the oracle's pin), here through bf16 inputs
    N = 512
    rng = np.random.default_rng(61)
    angles, noise = (0.0, 30.0, 80.0, 120.0), (1e-4, 1e-2, 1e-4, 1e-2)
    q = np.zeros((N, 128), dtype=np.float32)
    for i in range(N):
        t = np.radians(angles[i % 4])
        q[i, 0], q[i, 1] = np.cos(t), np.sin(t)
        q[i] += noise[i % 4] * rng.standard_normal(128).astype(np.float32)
    k = np.zeros((N, 128), dtype=np.float32)
    k[np.arange(N), np.arange(N) % 128] = np.sqrt(128.0)
    from block_sparse_attention_25_amd.synth import bf16_bits
    qb, kb = bf16_bits(q)[None, None], bf16_bits(k)[None, None]
    gperm = _gpu_perm(torch_cuda, qb, kb)[0, 0]
    want = np.concatenate([np.arange(N)[np.arange(N) % 4 == c] for c in (3, 2, 1, 0)])
    assert np.array_equal(gperm, want)


def test_reblock_zero_keys_and_rows(torch_cuda):
    # zero keys leave only the ridge (z = q / |q|); a zero query row stays zero
    N = 700
    qb, _, _ = generate(custom(N, heads=1, seed=62), threads=1)
    qb = qb.copy()
    qb[0, 0, 5] = 0
    kb = np.zeros_like(qb)
    gperm = _gpu_perm(torch_cuda, qb, kb)
    _check_perm(gperm[0, 0], widen(qb[0, 0]), widen(kb[0, 0]), "zero keys")


def _permuted(torch, host, perm, qb, kb, vb):
    """The inputs and the un-permuted GPU output in the GPU's order, per head."""
    B, H = qb.shape[:2]
    idx = [[perm[b, h] for h in range(H)] for b in range(B)]
    qp, kp, vp = (np.stack([np.stack([x[b, h][idx[b][h]] for h in range(H)]) for b in range(B)])
                  for x in (qb, kb, vb))
    out = host["out"]
    pt = torch.from_numpy(perm.astype(np.int64)).to(out.device)
    host = dict(host)
    host["out"] = torch.stack([torch.stack([out[b, h][pt[b, h]] for h in range(H)]) for b in range(B)])
    return host, qp, kp, vp


def _run_reblocked(torch, qb, kb, vb, **kw):
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    out, aux = bsa.attention(q, k, v, return_aux=True, reblock=True, **kw)
    torch.cuda.synchronize()
    host = {n: aux[n].cpu() for n in ("q_pool", "k_pool", "sum_k", "sum_v", "sum_bias", "block_idx")}
    host["token_idx"] = None if aux["token_idx"] is None else aux["token_idx"].cpu()
    host["out"] = out
    return host, aux["perm"].cpu().numpy()


@pytest.mark.parametrize("N,top_k,summary,tau,extra", [
    (4173, 8, "mean", None, 0),
    (4173, 6, "reweight", None, 0),
    (4096, 32, "mean", 1.0, 0),
    (2000, 4, "mean", None, 64),
])
def test_reblock_attention(torch_cuda, N, top_k, summary, tau, extra):
    _log("case reblock attention N=%d k=%d %s tau=%s extra=%d" % (N, top_k, summary, tau, extra))
    qb, kb, vb = generate(custom(N, heads=2, seed=63), threads=2)
    host, perm = _run_reblocked(torch_cuda, qb, kb, vb, top_k=top_k, summary=summary, tau=tau,
                                extra_tokens=extra)
    host_p, qp, kp, vp = _permuted(torch_cuda, host, perm, qb, kb, vb)
    for h in range(2):
        _check_perm(perm[0, h], widen(qb[0, h]), widen(kb[0, h]), "N=%d h%d" % (N, h))
        _check_head(host_p, qp, kp, vp, 0, h, top_k, summary, 0, label="reblock", tau=tau,
                    extra=extra)


@pytest.mark.parametrize("N,top_k,summary,tau,extra", [
    (4173, 8, "mean", None, 0),
    (4173, 6, "reweight", None, 0),
    (4096, 32, "mean", 1.0, 0),
    (2000, 4, "mean", None, 64),
    (50000, 4, "mean", None, 0),   # 391 blocks: the head-synchronous attention grid
])
def test_reordered_calls_equal_permuted_copies(torch_cuda, N, top_k, summary, tau, extra):
    """bsa_pool_reordered / bsa_forward_reordered (rows read through perm, the
    output written back through it) against the permuted-copy path
    (bsa_permute_rows, the plain calls, bsa_unpermute_rows): the same bits in
    every output, and k_r, v_r equal to the permuted K and V."""
    torch = torch_cuda
    _log("case reordered calls N=%d k=%d %s tau=%s extra=%d" % (N, top_k, summary, tau, extra))
    qb, kb, vb = generate(custom(N, heads=2, seed=71), threads=2)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    kw = dict(top_k=top_k, summary=summary, tau=tau, extra_tokens=extra)
    out_a, aux_a = bsa.attention(q, k, v, reblock=True, return_aux=True, **kw)
    perm = aux_a["perm"]
    p = aux_a["problem"]
    qr, kr, vr = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bsa.bsa_permute_rows(p, perm, q, k, v, qr, kr, vr)
    out_r, aux_b = bsa.attention(qr, kr, vr, return_aux=True, **kw)
    out_b = torch.empty_like(out_r)
    bsa.bsa_unpermute_rows(p, perm, out_r, out_b)
    torch.cuda.synchronize()
    assert torch.equal(aux_a["k_r"], kr)
    assert torch.equal(aux_a["v_r"], vr)
    for name in ("q_pool", "k_pool", "sum_k", "sum_v", "sum_bias", "block_idx", "token_idx"):
        if aux_a[name] is not None:
            assert torch.equal(aux_a[name], aux_b[name]), name
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    # k_out and v_out are written row by row: every element of them, nothing past them
    G = 4096
    n_el = 2 * N * 128
    k_out, v_out = (torch.full((n_el + G,), float("nan"), dtype=torch.float32, device="cuda").to(torch.bfloat16)
                    for _ in range(2))
    bsa.bsa_pool_reordered(p, perm, q, k, v, aux_a["q_pool"], aux_a["k_pool"], aux_a["sum_k"],
                           aux_a["sum_v"], aux_a["sum_bias"], k_out, v_out, aux_a["workspace"])
    torch.cuda.synchronize()
    assert torch.equal(k_out[:n_el].view(1, 2, N, 128), kr)
    assert torch.equal(v_out[:n_el].view(1, 2, N, 128), vr)
    assert bool(torch.isnan(k_out[n_el:].float()).all())
    assert bool(torch.isnan(v_out[n_el:].float()).all())


def test_reblock_rejects_position_options(torch_cuda):
    qb, kb, vb = generate(custom(1000, heads=1, seed=64), threads=1)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    with pytest.raises(ValueError):
        bsa.attention(q, k, v, top_k=2, sink_rows=100, reblock=True)
    with pytest.raises(ValueError):
        bsa.attention(q, k, v, top_k=2, summary="reweight", anchor_rows=900, reblock=True)
    # an anchor over every row is the same in any order
    bsa.attention(q, k, v, top_k=2, summary="reweight", anchor_rows=1000, reblock=True)


@pytest.mark.parametrize("N", [1500, 5000])
def test_reblock_all_zero_inputs(torch_cuda, N):
    # zero keys leave only the ridge and zero queries embed to zero: every
    # split value ties, so the order is the identity; every logit is 0 (the
    # selection ties too: the three lowest blocks).  Every distance ties as
    # well, so every row of a group lies in the pivot search's band: at 5,000
    # rows more than its list holds, and the whole group is measured exactly
    torch = torch_cuda
    qb = np.zeros((1, 1, N, 128), dtype=np.uint16)
    _, _, vb = generate(custom(N, heads=1, seed=68), threads=1)
    host, perm = _run_reblocked(torch, qb, qb, vb, top_k=3)
    assert np.array_equal(perm[0, 0], np.arange(N))
    Q, V = widen(qb[0, 0]), widen(vb[0, 0])
    want = O.run_head_reblocked(Q, Q, V, perm[0, 0], top_k=3)["out"]
    got = widen(tensor_bits(host["out"][0, 0]))
    assert np.abs(got - want).max() < 1e-2


def test_reblock_guard_bands_untouched(torch_cuda):
    """perm and the permuted and unpermuted rows written into poisoned
    buffers: every element inside written, the guard regions after them
    untouched."""
    torch = torch_cuda
    N, H, G = 1000, 2, 4096
    qb, kb, vb = generate(custom(N, heads=H, seed=69), threads=2)
    q, k, v = (to_device(x) for x in (qb, kb, vb))
    p = bsa.make_problem(1, H, N, top_k=3)
    n_rows = H * N * 128
    perm = torch.full((H * N + G,), -7, dtype=torch.int32, device="cuda")
    outs = [torch.full((n_rows + G,), float("nan"), dtype=torch.float32, device="cuda").to(torch.bfloat16)
            for _ in range(4)]
    ws = torch.empty(bsa.bsa_reblock_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    bsa.bsa_reblock(p, q, k, perm, ws)
    bsa.bsa_permute_rows(p, perm, q, k, v, outs[0], outs[1], outs[2])
    bsa.bsa_unpermute_rows(p, perm, outs[0], outs[3])
    torch.cuda.synchronize()
    pc = perm.cpu()
    assert bool((pc[:H * N] >= 0).all()) and bool((pc[H * N:] == -7).all())
    for i, o in enumerate(outs):
        oc = o.cpu().float()
        assert not bool(torch.isnan(oc[:n_rows]).any()), i
        assert bool(torch.isnan(oc[n_rows:]).all()), i
    # permute then unpermute gives Q back, bit for bit
    assert torch.equal(outs[3][:n_rows].view(1, H, N, 128), q)


def test_reblock_maximum_size(torch_cuda):
    """The largest supported sequence, ragged: 2,048 blocks, 11 levels, the
    top groups through the global key buffer (256 rows a thread)."""
    N = 262100
    _log("case reblock maximum size N=%d" % N)
    qb, kb, vb = generate(custom(N, heads=1, seed=70), threads=16)
    host, perm = _run_reblocked(torch_cuda, qb, kb, vb, top_k=64)
    _check_perm(perm[0, 0], widen(qb[0, 0]), widen(kb[0, 0]), "max N")
    host_p, qp, kp, vp = _permuted(torch_cuda, host, perm, qb, kb, vb)
    _check_head(host_p, qp, kp, vp, 0, 0, 64, query_blocks=[0, 1024, 2046, 2047], label="reblock max")


def test_reblock_deterministic(torch_cuda):
    qb, kb, vb = generate(custom(4173, heads=2, seed=65), threads=2)
    a = _run_reblocked(torch_cuda, qb, kb, vb, top_k=8)
    b = _run_reblocked(torch_cuda, qb, kb, vb, top_k=8)
    assert np.array_equal(a[1], b[1])
    assert torch_cuda.equal(a[0]["out"], b[0]["out"])


def test_reblock_batch_of_two(torch_cuda):
    # rows of batch 1 must be ordered and attended within batch 1
    w = custom(3000, heads=2, seed=66)
    qb, kb, vb = generate(w, threads=2)
    qb2, kb2, vb2 = generate(custom(3000, heads=2, seed=67), threads=2)
    qb, kb, vb = (np.concatenate([a, b]) for a, b in ((qb, qb2), (kb, kb2), (vb, vb2)))
    host, perm = _run_reblocked(torch_cuda, qb, kb, vb, top_k=5)
    host_p, qp, kp, vp = _permuted(torch_cuda, host, perm, qb, kb, vb)
    for b in range(2):
        for h in range(2):
            _check_perm(perm[b, h], widen(qb[b, h]), widen(kb[b, h]), "batch %d h%d" % (b, h))
    _check_head(host_p, qp, kp, vp, 1, 1, 5, label="reblock batch 1")


@pytest.mark.parametrize("name,heads", [("768p_5s_reblock", [0, 29]), ("2k_5s", [7])])
def test_reblock_full_size_sampled(torch_cuda, name, heads):
    """Full-size heads on the Spark-Reblock order, every head in one launch as
    in the benchmark: the permutation of a few heads against the oracle, then
    their indices, every query block of the first and sampled query blocks of
    the others (2K: 11 levels, the largest groups through the global key
    buffer)."""
    w = WORKLOADS[name]
    _log("case full %s reblock (H=%d N=%d)" % (w.name, w.heads, w.seq_len))
    qb, kb, vb = generate(w, threads=16)
    nb = O.n_blocks(w.seq_len)
    ratio = w.top_k_ratio
    top_k = O.k_from_ratio(ratio, nb) if ratio is not None else w.top_k
    kw = dict(top_k_ratio=ratio) if ratio is not None else dict(top_k=top_k)
    host, perm = _run_reblocked(torch_cuda, qb, kb, vb, **kw)
    for h in range(w.heads):
        assert np.array_equal(np.sort(perm[0, h]), np.arange(w.seq_len))
    for h in heads:
        _check_perm(perm[0, h], widen(qb[0, h]), widen(kb[0, h]), "%s h%d" % (name, h))
    # downstream checks on the selected heads, in the GPU's order
    sel = {n: (None if t is None else t[:, heads]) for n, t in host.items()}
    host_p, qp, kp, vp = _permuted(torch_cuda, sel, perm[:, heads], qb[:, heads], kb[:, heads],
                                   vb[:, heads])
    qbs = [0, 1, nb // 2, nb - 2, nb - 1]
    for i, h in enumerate(heads):
        _check_head(host_p, qp, kp, vp, 0, i, top_k, query_blocks=None if i == 0 else qbs,
                    label="%s reblock h%d" % (name, h))

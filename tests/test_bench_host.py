"""Host logic of bench.py on the CPU: the multi-GPU refusal, the counted-FLOP
formula against a brute-force count, and the JSON line's required keys."""
import ast
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _brute_counted(idx, N, nb, dense=(), tok=None):
    rows = [min(128, N - 128 * c) for c in range(nb)]
    exact = summ = 0
    B, H = idx.shape[:2]
    for b in range(B):
        for h in range(H):
            for r in range(nb):
                if r in dense:
                    exact += rows[r] * N
                    continue
                sel = [int(c) for c in idx[b, h, r] if c >= 0]
                keys = sum(rows[c] for c in sel)
                if tok is not None:
                    keys += int((tok[b, h, r] >= 0).sum())
                exact += rows[r] * keys
                summ += rows[r] * (nb - len(sel))
    return 4 * 128 * exact, 4 * 128 * summ


@pytest.mark.parametrize("case", ["topk", "padded", "dense", "tokens"])
def test_counted_flops_brute_force(case):
    rng = np.random.default_rng(5)
    B, H, N = 2, 3, 1000
    nb = -(-N // 128)
    k = 3
    idx = np.stack([np.stack([np.stack([np.sort(rng.choice(nb, k, replace=False)) for _ in range(nb)])
                              for _ in range(H)]) for _ in range(B)]).astype(np.int32)
    dense, tok = (), None
    if case == "padded":
        idx[..., -1][rng.random(idx.shape[:3]) < 0.5] = -1   # threshold rows keep fewer blocks
    if case == "dense":
        dense = (2, nb - 1)
    if case == "tokens":
        tok = rng.integers(-1, N, size=(B, H, nb, 16)).astype(np.int32)
    got = bench.counted_flops(torch, torch.from_numpy(idx), N, nb, H, B, dense,
                              None if tok is None else torch.from_numpy(tok))
    assert got == _brute_counted(idx, N, nb, dense, tok)


def test_json_line_has_the_contract_keys():
    src = open(os.path.join(ROOT, "bench.py")).read()
    keys = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}
    tree = ast.parse(src)
    found = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Dict):
            found |= {k.value for k in node.keys if isinstance(k, ast.Constant)}
        if isinstance(node, ast.Subscript) and isinstance(node.slice, ast.Constant):
            found.add(node.slice.value)
    assert keys <= found, keys - found
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in found

"""Seeded synthetic inputs shaped like the video-DiT attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention method's arithmetic.  The CPU oracle and the GPU path both take the
arrays it returns, so the two sides see the same bits.

Recipe (one independent stream per (batch, head), so any head subset can be
regenerated on its own):

* a video latent grid of T x Hh x W tokens, row-major with x fastest, followed
  by ``n_cond`` conditioning rows (text / reference / audio stand-ins);
* a coarse Gaussian field F of shape [ceil(T/4), ceil(Hh/8), ceil(W/8), 128]
  ~ N(0, 1), one vector per 4 x 8 x 8 (t, y, x) cell, shared by Q, K and V;
* video token n at (t, y, x) gets F[t//4, y//8, x//8] + 0.5 * N(0, 1) noise,
  drawn separately for Q, K and V;
* conditioning rows are plain N(0, 1);
* everything is rounded to bfloat16 (round to nearest, ties to even).

Draw order inside a head: F, then the Q, K, V video noise, then the Q, K, V
conditioning rows.

The workloads follow the sequence lengths of the h3-sparse-attn "Measured"
table (768p 5s / 10s / 15s and 2K 5s at 24 fps, 56 heads, head_dim 128).  The
pages do not print the latent grids; the grids below are the readings used
here (48 x 84 latent rows per frame at 768p, 90 x 160 at 2K), with the rest of
each sequence filled by conditioning rows.  They stand in for real H3
activations, which are not available.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HEAD_DIM = 128
CELL = (4, 8, 8)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    grid: tuple            # (T, Hh, W) video latent grid
    n_video: int           # video tokens used (grid may be truncated to fill)
    n_cond: int            # conditioning rows after the video rows
    top_k: int | None      # key blocks per query block (None: use top_k_ratio)
    top_k_ratio: str | None = None   # exact decimal string, e.g. "0.1"
    summary: str = "mean"  # "mean" or "reweight"
    seed: int = 0
    sinks: bool = False    # route the conditioning rows as sinks
    tau: float | None = None  # threshold selection (top_k is then the cap)
    extra: int = 0         # extra tokens per query block
    reblock: bool = False  # run on the Spark-Reblock row order (q_reuse_k)

    @property
    def sink_start(self) -> int:
        return self.n_video if self.sinks else 0

    @property
    def sink_rows(self) -> int:
        return self.n_cond if self.sinks else 0

    @property
    def seq_len(self) -> int:
        return self.n_video + self.n_cond

    @property
    def anchor_rows(self) -> int:
        """Rows whose queries form the per-head anchor: the video rows."""
        return self.n_video


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, (1, 48, 84), 4032, 64, 8),
    "768p_5s": Workload("768p_5s", 1, 56, (9, 48, 84), 36288, 1452, 64),
    "768p_10s": Workload("768p_10s", 1, 56, (18, 48, 84), 72576, 840, 64),
    "2k_5s": Workload("2k_5s", 1, 56, (10, 90, 160), 132620, 1024, 64),
    "768p_15s_reweight": Workload("768p_15s_reweight", 1, 56, (25, 48, 84), 100800,
                                  3196, None, "0.1", "reweight"),
    # the 768p 5s shape with its 1,452 conditioning rows routed as sinks
    "768p_5s_sinks": Workload("768p_5s_sinks", 1, 56, (9, 48, 84), 36288, 1452, 64, sinks=True),
    # the 768p 5s shape with threshold selection at tau 1.0, uncapped
    "768p_5s_tau1": Workload("768p_5s_tau1", 1, 56, (9, 48, 84), 36288, 1452, 295, tau=1.0),
    # the 768p 5s shape with 256 extra tokens per query block (the node's default)
    "768p_5s_extra256": Workload("768p_5s_extra256", 1, 56, (9, 48, 84), 36288, 1452, 64, extra=256),
    # the 768p 5s shape on the Spark-Reblock order, with the shipped workflows'
    # ratio budget (0.2 of 295 blocks: 59)
    "768p_5s_reblock": Workload("768p_5s_reblock", 1, 56, (9, 48, 84), 36288, 1452, None, "0.2",
                                reblock=True),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite draws from normal distributions, so no NaN handling is
    needed here."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact widening)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _head_qkv_bits(w: Workload, b: int, h: int, n_video: int, n_cond: int):
    rng = np.random.default_rng([w.seed, b, h])
    T, Hh, W = w.grid
    tc, hc, wc = CELL
    field = rng.standard_normal(((T + tc - 1) // tc, (Hh + hc - 1) // hc,
                                 (W + wc - 1) // wc, HEAD_DIM), dtype=np.float32)
    n = np.arange(n_video)
    t, rem = np.divmod(n, Hh * W)
    y, x = np.divmod(rem, W)
    base = field[t // tc, y // hc, x // wc]            # [n_video, 128]
    out = []
    noise = [rng.standard_normal((n_video, HEAD_DIM), dtype=np.float32) for _ in range(3)]
    cond = [rng.standard_normal((n_cond, HEAD_DIM), dtype=np.float32) for _ in range(3)]
    for i in range(3):
        full = np.empty((n_video + n_cond, HEAD_DIM), dtype=np.float32)
        np.multiply(noise[i], np.float32(0.5), out=full[:n_video])
        full[:n_video] += base
        full[n_video:] = cond[i]
        out.append(bf16_bits(full))
    return out


def generate(w: Workload, heads=None, batches=None, threads: int = 8):
    """Return (q, k, v) as uint16 bfloat16 bit arrays of shape [B', H', N, 128].

    ``heads`` / ``batches`` select a subset (default: all); each (b, h) draws
    from its own stream, so a subset equals the matching slice of the whole."""
    T, Hh, W = w.grid
    if w.n_video > T * Hh * W:
        raise ValueError("n_video exceeds the latent grid")
    heads = list(range(w.heads)) if heads is None else list(heads)
    batches = list(range(w.batch)) if batches is None else list(batches)
    N = w.seq_len
    q = np.empty((len(batches), len(heads), N, HEAD_DIM), dtype=np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def one(ij):
        i, j = ij
        qh, kh, vh = _head_qkv_bits(w, batches[i], heads[j], w.n_video, w.n_cond)
        q[i, j], k[i, j], v[i, j] = qh, kh, vh

    jobs = [(i, j) for i in range(len(batches)) for j in range(len(heads))]
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, jobs))
    else:
        for ij in jobs:
            one(ij)
    return q, k, v


def custom(seq_len: int, heads: int = 1, batch: int = 1, seed: int = 0,
           grid=None, n_cond: int | None = None, name: str = "custom") -> Workload:
    """A workload of any length with the same generator: a one-frame-high video
    grid 48 rows x W columns sized to the length, the remainder conditioning."""
    if grid is None:
        W = 84
        rows = max(1, seq_len // W)
        grid = (1, rows, W)
    T, Hh, W = grid
    if n_cond is None:
        n_video = min(seq_len, T * Hh * W)
        n_cond = seq_len - n_video
    else:
        n_video = seq_len - n_cond
    return Workload(name, batch, heads, tuple(grid), n_video, n_cond, None, seed=seed)

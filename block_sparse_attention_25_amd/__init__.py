"""Block-sparse self-attention with summary rows for gfx950 (MI355X).

A thin ctypes binding over the C ABI of ``libbsa.so`` (declared in
``include/bsa.h``).  Every step of the computation runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with
PyTorch and passes pointers and torch's current HIP stream.  There is no CPU
fallback: when the library is missing, every call raises.

Method (PyPI page "h3-sparse-attn 0.1.0", opening paragraph and "Use"):
each query block of 128 tokens attends to its top-k key blocks, and every
skipped key block is folded back in as one summary row.  The Spark-Reweight
summary mode follows "Spark-H3: Block Sparse Attention Speeds Up MiniMax-H3 in
ComfyUI", section "What Spark-Attn changes".
"""
from __future__ import annotations

import ctypes
import math
import os
from fractions import Fraction

__all__ = [
    "BSA_OK", "BSA_ERR_INVALID", "BSA_ERR_UNSUPPORTED", "BSA_ERR_WORKSPACE", "BSA_ERR_HIP",
    "SUMMARY_MEAN", "SUMMARY_REWEIGHT", "BsaError", "Problem", "lib", "library_path",
    "bsa_status_str", "bsa_problem_blocks", "bsa_workspace_bytes", "bsa_pool", "bsa_select",
    "bsa_forward", "bsa_forward_noalloc", "bsa_select_tokens", "bsa_forward_tokens", "k_from_ratio", "make_problem",
    "attention", "MAX_EXTRA",
]

BSA_OK, BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE, BSA_ERR_HIP, BSA_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
SUMMARY_MEAN, SUMMARY_REWEIGHT = 0, 1
SELECT_TOPK, SELECT_THRESHOLD = 0, 1
BLOCK = 128
HEAD_DIM = 128
MAX_EXTRA = 256

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSA_LIBRARY may name another build of the same library (e.g. the host-side
# sanitizer build that the CPU tests exercise)
library_path = os.environ.get("BSA_LIBRARY") or os.path.join(_HERE, "libbsa.so")


class Problem(ctypes.Structure):
    """Mirror of ``bsa_problem`` in include/bsa.h."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("summary", ctypes.c_int32), ("anchor_rows", ctypes.c_int32), ("scale", ctypes.c_float),
        ("sink_start", ctypes.c_int32), ("sink_rows", ctypes.c_int32),
        ("select_mode", ctypes.c_int32), ("select_tau", ctypes.c_float),
        ("extra_tokens", ctypes.c_int32),
    ]


class BsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s: %s (status %d)" % (where, bsa_status_str(status), status)
        if status == 4:
            msg += ": " + lib().bsa_hip_error_str().decode()
        super().__init__(msg)


_lib = None
_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libbsa.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError("libbsa.so is not built (%s); build it with "
                              "python -m block_sparse_attention_25_amd.build" % library_path)
        # torch ships its own HIP runtime under the same soname as the one
        # the library links; loading torch first makes the process use that
        # one runtime whichever module asks for the library first
        import torch  # noqa: F401
        L = ctypes.CDLL(library_path)
        L.bsa_status_str.argtypes = [ctypes.c_int]
        L.bsa_status_str.restype = ctypes.c_char_p
        L.bsa_hip_error_str.argtypes = []
        L.bsa_hip_error_str.restype = ctypes.c_char_p
        L.bsa_problem_blocks.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.bsa_problem_blocks.restype = ctypes.c_int
        L.bsa_workspace_bytes.argtypes = [_P]
        L.bsa_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_pool.argtypes = [_P] + [_vp] * 9 + [ctypes.c_size_t, _vp]
        L.bsa_pool.restype = ctypes.c_int
        L.bsa_select.argtypes = [_P, _vp, _vp, _vp, _vp]
        L.bsa_select.restype = ctypes.c_int
        L.bsa_forward.argtypes = [_P] + [_vp] * 9 + [ctypes.c_size_t, _vp]
        L.bsa_forward.restype = ctypes.c_int
        L.bsa_forward_noalloc.argtypes = [_P] + [_vp] * 9
        L.bsa_forward_noalloc.restype = ctypes.c_int
        L.bsa_select_tokens.argtypes = [_P] + [_vp] * 5 + [ctypes.c_size_t, _vp]
        L.bsa_select_tokens.restype = ctypes.c_int
        L.bsa_forward_tokens.argtypes = [_P] + [_vp] * 10 + [ctypes.c_size_t, _vp]
        L.bsa_forward_tokens.restype = ctypes.c_int
        L.bsa_reblock_workspace_bytes.argtypes = [_P, ctypes.POINTER(ctypes.c_size_t)]
        L.bsa_reblock_workspace_bytes.restype = ctypes.c_int
        L.bsa_reblock.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.bsa_reblock.restype = ctypes.c_int
        L.bsa_permute_rows.argtypes = [_P] + [_vp] * 8
        L.bsa_permute_rows.restype = ctypes.c_int
        L.bsa_unpermute_rows.argtypes = [_P] + [_vp] * 4
        L.bsa_unpermute_rows.restype = ctypes.c_int
        L.bsa_pool_reordered.argtypes = [_P] + [_vp] * 12 + [ctypes.c_size_t, _vp]
        L.bsa_pool_reordered.restype = ctypes.c_int
        L.bsa_forward_reordered.argtypes = [_P] + [_vp] * 11 + [ctypes.c_size_t, _vp]
        L.bsa_forward_reordered.restype = ctypes.c_int
        _lib = L
    return _lib


def _raise(status: int, where: str):
    if status == BSA_OK:
        return
    if status == BSA_ERR_UNSUPPORTED:
        raise NotImplementedError("%s: %s" % (where, bsa_status_str(status)))
    if status in (BSA_ERR_INVALID, BSA_ERR_WORKSPACE, BSA_ERR_SCRATCH):
        raise ValueError("%s: %s" % (where, bsa_status_str(status)))
    raise BsaError(status, where)


# ------------------------------------------------------------ raw C calls ---
def bsa_status_str(status: int) -> str:
    return lib().bsa_status_str(int(status)).decode()


def bsa_problem_blocks(p: Problem):
    nb, k = ctypes.c_int32(), ctypes.c_int32()
    _raise(lib().bsa_problem_blocks(ctypes.byref(p), ctypes.byref(nb), ctypes.byref(k)),
           "bsa_problem_blocks")
    return nb.value, k.value


def bsa_workspace_bytes(p: Problem) -> int:
    """Scratch bytes covering every entry point for problem p (0 for a
    rejected problem: the problem is validated first, so that raises)."""
    bsa_problem_blocks(p)
    return int(lib().bsa_workspace_bytes(ctypes.byref(p)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def bsa_pool(p: Problem, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, workspace=None, stream=None):
    _raise(lib().bsa_pool(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(q_pool), _ptr(k_pool),
                          _ptr(sum_k), _ptr(sum_v), _ptr(sum_bias), _ptr(workspace), _nbytes(workspace),
                          _stream(stream)), "bsa_pool")


def bsa_select(p: Problem, q_pool, k_pool, block_idx, stream=None):
    _raise(lib().bsa_select(ctypes.byref(p), _ptr(q_pool), _ptr(k_pool), _ptr(block_idx),
                            _stream(stream)), "bsa_select")


def bsa_forward(p: Problem, q, k, v, sum_k, sum_v, sum_bias, block_idx, out, workspace=None,
                stream=None):
    _raise(lib().bsa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sum_k), _ptr(sum_v),
                             _ptr(sum_bias), _ptr(block_idx), _ptr(out), _ptr(workspace),
                             _nbytes(workspace), _stream(stream)), "bsa_forward")


def bsa_forward_noalloc(p: Problem, q, k, v, sum_k, sum_v, sum_bias, block_idx, out, stream=None):
    _raise(lib().bsa_forward_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sum_k),
                                     _ptr(sum_v), _ptr(sum_bias), _ptr(block_idx), _ptr(out),
                                     _stream(stream)), "bsa_forward_noalloc")


def bsa_select_tokens(p: Problem, q_pool, k, block_idx, token_idx, workspace, stream=None):
    _raise(lib().bsa_select_tokens(ctypes.byref(p), _ptr(q_pool), _ptr(k), _ptr(block_idx),
                                   _ptr(token_idx), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)), "bsa_select_tokens")


def bsa_forward_tokens(p: Problem, q, k, v, sum_k, sum_v, sum_bias, block_idx, token_idx, out,
                       workspace=None, stream=None):
    _raise(lib().bsa_forward_tokens(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sum_k),
                                    _ptr(sum_v), _ptr(sum_bias), _ptr(block_idx), _ptr(token_idx),
                                    _ptr(out), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "bsa_forward_tokens")


def bsa_reblock_workspace_bytes(p: Problem) -> int:
    n = ctypes.c_size_t()
    _raise(lib().bsa_reblock_workspace_bytes(ctypes.byref(p), ctypes.byref(n)),
           "bsa_reblock_workspace_bytes")
    return n.value


def bsa_reblock(p: Problem, q, k, perm, workspace, stream=None):
    _raise(lib().bsa_reblock(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(perm), _ptr(workspace),
                             _nbytes(workspace), _stream(stream)), "bsa_reblock")


def bsa_permute_rows(p: Problem, perm, q, k, v, q_out, k_out, v_out, stream=None):
    _raise(lib().bsa_permute_rows(ctypes.byref(p), _ptr(perm), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(q_out), _ptr(k_out), _ptr(v_out), _stream(stream)),
           "bsa_permute_rows")


def bsa_unpermute_rows(p: Problem, perm, x, out, stream=None):
    _raise(lib().bsa_unpermute_rows(ctypes.byref(p), _ptr(perm), _ptr(x), _ptr(out),
                                    _stream(stream)), "bsa_unpermute_rows")


def bsa_pool_reordered(p: Problem, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_out, v_out,
                       workspace=None, stream=None):
    _raise(lib().bsa_pool_reordered(ctypes.byref(p), _ptr(perm), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(q_pool), _ptr(k_pool), _ptr(sum_k), _ptr(sum_v),
                                    _ptr(sum_bias), _ptr(k_out), _ptr(v_out), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)), "bsa_pool_reordered")


def bsa_forward_reordered(p: Problem, perm, q, k_r, v_r, sum_k, sum_v, sum_bias, block_idx, token_idx,
                          out, workspace=None, stream=None):
    _raise(lib().bsa_forward_reordered(ctypes.byref(p), _ptr(perm), _ptr(q), _ptr(k_r), _ptr(v_r),
                                       _ptr(sum_k), _ptr(sum_v), _ptr(sum_bias), _ptr(block_idx),
                                       _ptr(token_idx), _ptr(out), _ptr(workspace), _nbytes(workspace),
                                       _stream(stream)), "bsa_forward_reordered")


# ---------------------------------------------------------------- helpers ---
def k_from_ratio(ratio, n_blocks: int) -> int:
    """Top-k ratio budget -> block count, ceil(ratio * n_blocks) computed on the
    exact decimal value of the ratio (so 0.07 * 100 gives 7, not 8)."""
    r = Fraction(str(ratio))
    if not 0 <= r <= 1:
        raise ValueError("top_k_ratio must lie in [0, 1]")
    return math.ceil(r * n_blocks)


def make_problem(batch, heads, seq_len, top_k=None, top_k_ratio=None, summary="mean",
                 anchor_rows=0, scale=None, sink_rows=0, sink_start=None, tau=None,
                 extra_tokens=0) -> Problem:
    """Fill a bsa_problem.  sink_rows > 0 routes the conditioning rows
    [sink_start, sink_start + sink_rows) as sinks; sink_start defaults to
    N - sink_rows (conditioning rows after the video rows).  tau selects
    blocks by threshold (score above mean + tau * std of the row), with
    top_k as the cap.  extra_tokens (0..256) adds, per query block, that
    many exactly-read tokens from the blocks it skipped."""
    nb = -(-int(seq_len) // BLOCK)
    if (top_k is None) == (top_k_ratio is None):
        raise ValueError("give exactly one of top_k and top_k_ratio")
    if top_k is None:
        top_k = k_from_ratio(top_k_ratio, nb)
    if summary not in ("mean", "reweight"):
        raise ValueError("summary must be 'mean' or 'reweight'")
    sink_rows = int(sink_rows)
    if sink_start is None:
        sink_start = int(seq_len) - sink_rows if sink_rows > 0 else 0
    return Problem(int(batch), int(heads), int(seq_len), HEAD_DIM, BLOCK, int(top_k),
                   SUMMARY_MEAN if summary == "mean" else SUMMARY_REWEIGHT, int(anchor_rows),
                   0.0 if scale is None else float(scale), int(sink_start), sink_rows,
                   SELECT_TOPK if tau is None else SELECT_THRESHOLD,
                   0.0 if tau is None else float(tau), int(extra_tokens))


def _check_qkv(q, k, v):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError("%s must be a contiguous bfloat16 CUDA tensor [B, H, N, 128]" % name)
        if t.shape[-1] != HEAD_DIM:
            raise NotImplementedError("head_dim must be 128")
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k and v must have the same shape")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must live on one device")


def attention(q, k, v, top_k=None, top_k_ratio=None, summary="mean", anchor_rows=0, scale=None,
              sink_rows=0, sink_start=None, tau=None, extra_tokens=0, reblock=False,
              return_aux=False, stream=None, out=None):
    """Block-sparse attention of bf16 q, k, v [B, H, N, 128] on the GPU.

    top_k counts 128-token key blocks (or give top_k_ratio, e.g. "0.1");
    summary is "mean" or "reweight" (Spark-Reweight, anchor = mean of query
    rows [0, anchor_rows), 0 meaning all rows).  sink_rows > 0 routes the
    conditioning rows [sink_start, sink_start + sink_rows) (by default the
    last sink_rows rows) as sinks: their blocks are kept exactly by every
    query block, and their query blocks attend densely.  tau switches to
    threshold selection (blocks scoring above mean + tau * std of their row,
    at most top_k; rows of block_idx padded with -1).  extra_tokens > 0 lets
    each query block also read exactly that many tokens of the blocks it
    skipped, those scoring highest against its pooled query (token_idx in the
    aux dict).  reblock=True runs the path on Spark-Reblock's row order (the
    q_reuse_k layout: Q, K and V permuted alike, the output put back in
    place; perm and k_r, v_r, the keys and values in the new order, in the
    aux dict, the other aux tensors in the new order); it rejects sink rows
    and an anchor over part of the rows.  Returns out
    [B, H, N, 128] bf16 (written into `out` when given: a contiguous bf16
    tensor of q's shape on its device, not overlapping q, k or v), plus a
    dict of intermediate tensors when return_aux is set.  The calls run with
    q's device current, on `stream` when given (a torch.cuda.Stream of that
    device), else on the device's current stream; the outputs and scratch
    tensors are allocated on that same stream, so torch's caching allocator
    does not hand them to other work while its kernels still run."""
    import torch
    _check_qkv(q, k, v)
    if stream is not None and stream.device != q.device:
        raise ValueError("stream must belong to q's device")
    with torch.cuda.device(q.device), torch.cuda.stream(stream):
        return _attention(q, k, v, top_k, top_k_ratio, summary, anchor_rows, scale, sink_rows,
                          sink_start, tau, extra_tokens, reblock, return_aux, stream, out)


def _attention(q, k, v, top_k, top_k_ratio, summary, anchor_rows, scale, sink_rows, sink_start, tau,
               extra_tokens, reblock, return_aux, stream, out):
    import torch
    B, H, N, _ = q.shape
    p = make_problem(B, H, N, top_k, top_k_ratio, summary, anchor_rows, scale, sink_rows, sink_start,
                     tau, extra_tokens)
    nb, kk = bsa_problem_blocks(p)
    dev = q.device
    perm = None
    if reblock:
        if p.sink_rows or (summary == "reweight" and p.anchor_rows not in (0, N)):
            raise ValueError("reblock reorders the rows: sink_rows, and an anchor over part of the "
                             "rows, would name other rows")
        perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
        rws = torch.empty(bsa_reblock_workspace_bytes(p), dtype=torch.uint8, device=dev)
        bsa_reblock(p, q, k, perm, rws, stream)
    f32, bf = torch.float32, torch.bfloat16
    q_pool = torch.empty((B, H, nb, HEAD_DIM), dtype=f32, device=dev)
    k_pool = torch.empty_like(q_pool)
    sum_k = torch.empty((B, H, nb, HEAD_DIM), dtype=bf, device=dev)
    sum_v = torch.empty_like(sum_k)
    sum_bias = torch.empty((B, H, nb), dtype=f32, device=dev)
    idx = torch.empty((B, H, nb, kk), dtype=torch.int32, device=dev)
    ws = torch.empty(bsa_workspace_bytes(p), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(q)
    elif (out.dtype != torch.bfloat16 or out.shape != q.shape or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous bfloat16 tensor shaped and placed like q")
    k_r = v_r = None
    if perm is not None:
        # q is read through perm; K and V get one copy each in the new order
        k_r, v_r = torch.empty_like(k), torch.empty_like(v)
        bsa_pool_reordered(p, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, k_r, v_r, ws,
                           stream)
    else:
        bsa_pool(p, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, ws, stream)
    bsa_select(p, q_pool, k_pool, idx if kk > 0 else None, stream)
    tok = None
    if p.extra_tokens > 0:
        tok = torch.empty((B, H, nb, p.extra_tokens), dtype=torch.int32, device=dev)
        bsa_select_tokens(p, q_pool, k if k_r is None else k_r, idx if kk > 0 else None, tok, ws, stream)
    if perm is not None:
        bsa_forward_reordered(p, perm, q, k_r, v_r, sum_k, sum_v, sum_bias, idx if kk > 0 else None,
                              tok, out, ws, stream)
    elif tok is not None:
        bsa_forward_tokens(p, q, k, v, sum_k, sum_v, sum_bias, idx if kk > 0 else None, tok, out, ws,
                           stream)
    else:
        bsa_forward(p, q, k, v, sum_k, sum_v, sum_bias, idx if kk > 0 else None, out, ws, stream)
    if return_aux:
        return out, dict(q_pool=q_pool, k_pool=k_pool, sum_k=sum_k, sum_v=sum_v,
                         sum_bias=sum_bias, block_idx=idx, token_idx=tok, workspace=ws, problem=p,
                         perm=perm, k_r=k_r, v_r=v_r)
    return out

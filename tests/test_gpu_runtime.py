"""GPU: the library's launch status is its own.

hipGetLastError reports the last failure of any runtime call on the thread,
also one that other code made before the library was called.  Each launching
call drops such a pending error first, so an error left by earlier code does
not turn a good call into BSA_ERR_HIP.  The pending error here comes from a
runtime call with an invalid device ordinal (it fails on the host and changes
nothing)."""
import ctypes

import pytest

import block_sparse_attention_25_amd as bsa
from block_sparse_attention_25_amd.synth import custom, generate
from tests.parity import to_device
from tests.test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu


def test_pending_runtime_error_is_not_the_calls(torch_cuda):
    torch = torch_cuda
    maps = open("/proc/self/maps").read().splitlines()
    assert len({l.split()[-1] for l in maps if "libamdhip64" in l}) == 1, "two HIP runtimes mapped"
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already mapped under this soname
    w = custom(1000, heads=2, batch=1, seed=5)
    print("case pending runtime error N=1000 H=2", flush=True)
    q, k, v = (to_device(x) for x in generate(w))
    ref, aux = bsa.attention(q, k, v, top_k=3, return_aux=True)
    # the C-ABI calls on buffers allocated beforehand (torch's own next
    # launch check would report the pending error itself)
    p = aux["problem"]
    bufs = {n: torch.empty_like(aux[n]) for n in ("q_pool", "k_pool", "sum_k", "sum_v", "sum_bias", "block_idx")}
    ws = torch.empty(bsa.bsa_workspace_bytes(p), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    hip.hipGetLastError()  # start from no pending error
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0  # invalid ordinal: fails on the host
    if hip.hipPeekAtLastError() == 0:
        pytest.skip("this runtime keeps no error from a failed hipSetDevice")
    bsa.bsa_pool(p, q, k, v, bufs["q_pool"], bufs["k_pool"], bufs["sum_k"], bufs["sum_v"], bufs["sum_bias"],
                 ws, stream)
    assert hip.hipPeekAtLastError() == 0  # dropped by the call
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    bsa.bsa_select(p, bufs["q_pool"], bufs["k_pool"], bufs["block_idx"], stream)
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    bsa.bsa_forward(p, q, k, v, bufs["sum_k"], bufs["sum_v"], bufs["sum_bias"], bufs["block_idx"], out, ws,
                    stream)
    torch.cuda.synchronize()
    assert torch.equal(bufs["block_idx"], aux["block_idx"])
    assert torch.equal(out, ref)
    assert bsa.lib().bsa_hip_error_str().decode() == "none"

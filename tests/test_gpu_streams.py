"""GPU: attention() on a caller's stream.

The path's kernels are deterministic, so a call on a second stream (passed as
`stream=`, or made current with torch.cuda.stream) must give the bits of the
same call on torch's current stream.  The second stream's calls are queued
back to back without host synchronisation in between, so scratch that torch
handed to other work while a kernel still read it would show as a mismatch.
"""
import pytest

import block_sparse_attention_25_amd as bsa
from block_sparse_attention_25_amd.synth import custom, generate
from tests.parity import to_device
from tests.test_gpu_parity import torch_cuda  # noqa: F401  (fixture)

pytestmark = pytest.mark.gpu

CASES = {
    "topk": dict(top_k=6),
    "tokens": dict(top_k=4, extra_tokens=32),
    "threshold": dict(top_k=7, tau=1.0),
    "reblock": dict(top_k_ratio="0.2", reblock=True),
    "reweight": dict(top_k=5, summary="reweight"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_attention_on_a_side_stream(torch_cuda, name):
    torch = torch_cuda
    kw = CASES[name]
    w = custom(3000, heads=3, batch=2, seed=77)
    print("case side stream %s N=3000 B=2 H=3" % name, flush=True)
    q, k, v = (to_device(x) for x in generate(w))
    ref = bsa.attention(q, k, v, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = [bsa.attention(q, k, v, stream=side, **kw) for _ in range(3)]
    with torch.cuda.stream(side):
        outs += [bsa.attention(q, k, v, **kw) for _ in range(3)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), "%s call %d differs" % (name, i)


def test_stream_of_another_device_is_rejected(torch_cuda):
    torch = torch_cuda
    q = torch.zeros((1, 1, 256, 128), dtype=torch.bfloat16, device="cuda:0")

    class Foreign:
        device = torch.device("cpu")
    with pytest.raises(ValueError):
        bsa.attention(q, q, q, top_k=1, stream=Foreign())

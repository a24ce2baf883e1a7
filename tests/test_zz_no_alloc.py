"""The allocation-free entry point (moe_forward_static_scratch) against
moe_forward with a caller workspace: two calls in a row, the second with
fewer tokens, each bit-identical in outputs, next-layer input and routing;
a token count whose workspace exceeds the library's array is refused."""
import numpy as np
import pytest
import torch

import synth
import quantized_moe_decode_gemv_amd as q
from helpers import layer_source

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


def _buffers(S, T, dev):
    return (torch.full((T, S.hidden), 7.0, dtype=torch.float32, device=dev),
            torch.zeros(T, S.hidden, dtype=torch.int16, device=dev),
            torch.zeros(T, S.top_k, dtype=torch.int32, device=dev),
            torch.zeros(T, S.top_k, dtype=torch.float32, device=dev))


@pytest.mark.parametrize("mx", [False, True], ids=["q4k", "mxfp4"])
def test_static_scratch_forward_matches_caller_workspace(dev, mx):
    S = synth.QWEN3_30B_A3B_MXFP4 if mx else synth.QWEN3_30B_A3B
    Tmax = 140
    plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=1, max_tokens=Tmax,
                  flags=q.FLAG_WEIGHTS_MXFP4 if mx else 0)
    assert plan.scratch_bytes(Tmax) <= q.STATIC_SCRATCH_BYTES
    blob = plan.upload_blob(layer_source(S), device=dev)
    # 96 tokens (MFMA tiles), then 3 (per-token GEMV) and 1 (fused decode path)
    for T in (96, 3, 1):
        xb = synth.x_bf16(S, 80, T, T=T)
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        y0, n0, i0, w0 = _buffers(S, T, dev)
        plan.forward(blob, 0, x, T, y0, x_next=n0, ids=i0, w=w0, scratch=plan.new_scratch(T, device=dev))
        y1, n1, i1, w1 = _buffers(S, T, dev)
        plan.forward_static_scratch(blob, 0, x, T, y1, x_next=n1, ids=i1, w=w1)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(w0, w1), T
        assert torch.equal(y0, y1) and torch.equal(n0, n1), T
        assert bool(torch.isfinite(y1).all())


def test_static_scratch_refuses_oversized_calls(dev):
    S = synth.QWEN3_30B_A3B
    T = 512
    plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=1, max_tokens=T)
    assert plan.scratch_bytes(T) > q.STATIC_SCRATCH_BYTES
    blob = torch.zeros(4096, dtype=torch.uint8, device=dev)     # refused before any launch
    x = torch.zeros(T, S.hidden, dtype=torch.int16, device=dev)
    y = torch.empty(T, S.hidden, dtype=torch.float32, device=dev)
    with pytest.raises(q.MoeError) as e:
        plan.forward_static_scratch(blob, 0, x, T, y)
    assert e.value.status == -4

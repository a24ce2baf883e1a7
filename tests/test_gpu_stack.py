"""GPU parity of the stacked decode step (residual + RMSNorm between layers,
last layer feeding the next step), run as the captured step graph the
benchmark times. The oracle follows its own trajectory from the same seeded
input; per layer it checks routing ids (near-tie rule), y within
max|err| <= 2e-3 * max|ref| and x_next up to adjacent-bf16 flips."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_moe_decode_gemv_amd as q
from helpers import (REL_TOL, TAU, check_bf16_vector, check_outputs, check_routing, layer_source, reference_outputs,
                     rel_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q.load()
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


def _compare_step(S, L, src, x_in, got):
    """Oracle over one step from x_in (bf16 bits [H]), following its own
    trajectory; got: per-layer GPU arrays after the step (xs: layer inputs,
    xs[0] already holding the next step's input; ys; ids).

    While the GPU's layer input is bitwise the oracle's, the layer is held to
    the full bar (ids, y within 2e-3 * max|ref|, x_next within one bf16 step
    or that tolerance). Once rounding the normalised output to bf16 has put
    the two inputs apart (adjacent-bf16 flips), the trajectories are only
    followed while they still agree to that bar, and the comparison stops at
    the first layer where they do not (the method amplifies such flips;
    every layer's arithmetic is held to the full bar on identical inputs by
    test_full_stack_every_layer_on_seeded_inputs). Returns (layers compared,
    layers compared on identical inputs, worst error, flips, why it stopped).
    """
    x = x_in
    worst, flips, compared, exact_inputs = 0.0, 0, 0, 0
    same = True
    for l in range(L):
        ref = oracle.moe_layer(src, l, x[None, :])
        rid = ref["ids"][0]
        if set(got["ids"][l].tolist()) != set(rid.tolist()):
            if ref["gap"][0] <= TAU:
                return compared, exact_inputs, worst, flips, f"near-tie routing at layer {l}"
            assert not same, f"layer {l}: ids {got['ids'][l]} vs {rid} on identical inputs"
            return compared, exact_inputs, worst, flips, f"routing parted at layer {l}"
        err = np.abs(got["ys"][l] - ref["y"][0]).max() / np.abs(ref["y"][0]).max()
        _, xn = oracle.resid_rmsnorm(x, ref["y"][0])
        if same:
            assert err <= REL_TOL, f"layer {l}: {err:.3e}"
            flips += check_bf16_vector(got["xs"][(l + 1) % L], xn)
            exact_inputs += 1
        else:
            if err > REL_TOL:
                return compared, exact_inputs, worst, flips, f"outputs parted at layer {l} ({err:.1e})"
            try:
                flips += check_bf16_vector(got["xs"][(l + 1) % L], xn)
            except AssertionError:
                return compared, exact_inputs, worst, flips, f"inputs parted after layer {l}"
        worst = max(worst, err)
        compared += 1
        same = bool(np.array_equal(got["xs"][(l + 1) % L], xn))
        x = xn
    return compared, exact_inputs, worst, flips, None


def _check_step_properties(S, got):
    """Properties of every layer of a GPU step that hold at any size."""
    L = got["ys"].shape[0]
    for l in range(L):
        ids = got["ids"][l]
        assert len(set(ids.tolist())) == S.top_k and ids.min() >= 0 and ids.max() < S.n_experts
        assert np.isfinite(got["ys"][l]).all()
        xn = oracle.bf16_array(got["xs"][(l + 1) % L])
        # RMSNorm output (weight 1): unit RMS up to the bf16 rounding and eps
        assert abs(np.sqrt(np.mean(xn * xn)) - 1.0) <= 2.0 ** -8


def _run(S, L, dev, steps, graph=True):
    plan = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=L, max_tokens=1)
    def progress(layer):
        if layer % 8 == 7:
            print(f"  [{S.name}] {layer + 1}/{L} layers uploaded", flush=True)
    blob = plan.upload_blob(layer_source(S), device=dev, progress=progress)
    H, k = S.hidden, S.top_k
    xs = torch.zeros(L, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, k, dtype=torch.float32, device=dev)
    scratch = plan.new_scratch(1, device=dev)
    x0 = synth.x_bf16(S, 3, 0)
    xs[0].copy_(torch.from_numpy(x0[0].view(np.int16)))
    stream = torch.cuda.Stream()
    g = plan.capture_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream) if graph else None
    out = []
    for _ in range(steps):
        x_in = xs[0].cpu().numpy().view(np.uint16).copy()
        if graph:
            g.launch(stream)
        else:
            plan.stack_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream)
        torch.cuda.synchronize()
        out.append(dict(x_in=x_in, xs=xs.cpu().numpy().view(np.uint16).copy(), ys=ys.cpu().numpy().copy(),
                        ids=ids.cpu().numpy().copy()))
    return plan, blob, out


def test_small_stack_graph_equals_eager_and_oracle(dev):
    S = synth.Shape("tiny-stack", 1, 256, 8, 2, 512)
    L = 6
    a = _run(S, L, dev, steps=3, graph=True)[2]
    b = _run(S, L, dev, steps=3, graph=False)[2]
    for sa, sb in zip(a, b):
        assert np.array_equal(sa["xs"], sb["xs"]) and np.array_equal(sa["ys"], sb["ys"])
    for st in a:
        _check_step_properties(S, st)
    src = oracle.ExpertSource(S)
    compared, exact, worst, flips, why = _compare_step(S, L, src, a[0]["x_in"], a[0])
    assert exact >= 1 and compared >= 1


@pytest.fixture(scope="module")
def qwen_stack(dev):
    S = synth.QWEN3_30B_A3B
    plan, blob, out = _run(S, 48, dev, steps=2, graph=True)
    return S, plan, blob, out


def test_full_stack_every_layer_on_seeded_inputs(dev, qwen_stack):
    """All 48 distinct layers of the benchmark's blob, each on its own seeded
    bf16 N(0,1) input, through the same per-layer launches the step graph
    records (moe_forward, T = 1, with the RMSNorm epilogue)."""
    S, plan, blob, _ = qwen_stack
    src = oracle.ExpertSource(S, max_cached=16)
    scratch = plan.new_scratch(1, device=dev)
    worst, exempted = 0.0, 0
    for l in range(48):
        xb = synth.x_bf16(S, 10, l)
        x = torch.from_numpy(xb.view(np.int16)).to(dev)
        y = torch.empty(1, S.hidden, dtype=torch.float32, device=dev)
        xn = torch.empty(1, S.hidden, dtype=torch.int16, device=dev)
        ids = torch.empty(1, S.top_k, dtype=torch.int32, device=dev)
        w = torch.empty(1, S.top_k, dtype=torch.float32, device=dev)
        plan.forward(blob, l, x, 1, y, x_next=xn, ids=ids, w=w, scratch=scratch)
        torch.cuda.synchronize()
        ref = oracle.moe_layer(src, l, xb)
        gid = ids.cpu().numpy()
        exempt = check_routing(gid, w.cpu().numpy(), ref, label=f"layer {l}")
        exempted += len(exempt)
        yref = reference_outputs(src, l, xb, ref, gid, exempt)
        err = rel_err(y.cpu().numpy(), yref)
        assert err <= REL_TOL, f"layer {l}: {err:.3e}"
        worst = max(worst, err)
        _, ref_next = oracle.resid_rmsnorm(xb[0], yref[0])
        check_bf16_vector(xn.cpu().numpy().view(np.uint16)[0], ref_next)
    print(f"48 layers on seeded inputs: worst max|err|/max|ref| = {worst:.3e}, near-tie exemptions {exempted}")
    assert exempted <= 2


def test_full_stack_chained_step_in_bench_configuration(qwen_stack):
    """The benchmark's captured step graph at full size: step 0 from the
    seeded input against the oracle's own trajectory (layer 0 always on
    identical inputs), properties of every layer, and the feedback into
    step 1."""
    S, _, _, out = qwen_stack
    for st in out:
        _check_step_properties(S, st)
    src = oracle.ExpertSource(S, max_cached=16)
    compared, exact, worst, flips, why = _compare_step(S, 48, src, out[0]["x_in"], out[0])
    print(f"chained step 0: {compared} layers compared ({exact} on identical inputs), worst {worst:.3e}, "
          f"x_next flips {flips}, stopped: {why}")
    assert exact >= 1
    assert np.array_equal(out[1]["x_in"], out[0]["xs"][0])


def test_full_stack_256_step_loop_properties(qwen_stack):
    """The benchmark's whole greedy loop: 256 replays of the captured step,
    each feeding the next, and at every step and layer the properties that
    hold at any size (distinct ids in range, finite y, unit-RMS next input),
    the routing weights summing to one, and the feedback (the next step's
    layer-0 input is the last layer's output)."""
    S, plan, blob, _ = qwen_stack
    L, H, k = 48, S.hidden, S.top_k
    dev = blob.device
    xs = torch.zeros(L, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, k, dtype=torch.float32, device=dev)
    scratch = plan.new_scratch(1, device=dev)
    xs[0].copy_(torch.from_numpy(synth.x_bf16(S, 3, 0)[0].view(np.int16)))
    stream = torch.cuda.Stream()
    g = plan.capture_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream)
    for step in range(256):
        x_in = xs[0].clone()
        g.launch(stream)
        torch.cuda.synchronize()
        got = dict(xs=xs.cpu().numpy().view(np.uint16), ys=ys.cpu().numpy(), ids=ids.cpu().numpy())
        _check_step_properties(S, got)
        wsum = ws.sum(dim=1).cpu().numpy()
        assert np.abs(wsum - 1.0).max() <= 1e-5, f"step {step}"
        assert not torch.equal(x_in, xs[0]), f"step {step}: the input did not move"


def _chained_forward(plan, blob, L, H, k, x0, dev):
    """The step as L chained moe_forward calls with the RMSNorm epilogue."""
    xs = torch.zeros(L, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, k, dtype=torch.float32, device=dev)
    xs[0].copy_(x0)
    scratch = plan.new_scratch(1, device=dev)
    for l in range(L):
        nxt = xs[(l + 1) % L] if l + 1 < L else torch.zeros(H, dtype=torch.int16, device=dev)
        plan.forward(blob, l, xs[l].view(1, H), 1, ys[l].view(1, H), x_next=nxt.view(1, H), ids=ids[l].view(1, k),
                     w=ws[l].view(1, k), scratch=scratch)
        if l + 1 == L:
            last = nxt
    torch.cuda.synchronize()
    xs[0].copy_(last)
    return xs, ys, ids, ws


def _stack_once(plan, blob, L, H, k, x0, dev, graph, replays=1):
    xs = torch.zeros(L, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, k, dtype=torch.float32, device=dev)
    scratch = plan.new_scratch(1, device=dev)
    stream = torch.cuda.Stream()
    if not graph:
        xs[0].copy_(x0)
        torch.cuda.synchronize()
        plan.stack_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream)
        torch.cuda.synchronize()
        return [(xs.clone(), ys.clone(), ids.clone(), ws.clone())]
    g = plan.capture_step(blob, xs, ys, 1, ids, ws, scratch=scratch, stream=stream)
    outs = []
    for _ in range(replays):
        xs.zero_(), ys.zero_(), ids.zero_(), ws.zero_()
        xs[0].copy_(x0)
        other = torch.randn(1000, device=dev).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.launch(stream)
        torch.cuda.synchronize()
        assert other.isfinite()
        outs.append((xs.clone(), ys.clone(), ids.clone(), ws.clone()))
    return outs


def _assert_same(a, b, what):
    for name, u, v in zip(("xs", "ys", "ids", "w"), a, b):
        assert torch.equal(u, v), f"{what}: {name} differs"


@pytest.mark.parametrize("hidden,E,k,inter,L,seed,fmt", [
    (1024, 64, 4, 256, 5, 21, "q4k"),
    (4096, 32, 4, 512, 4, 22, "q4k"),
    (2048, 256, 8, 256, 3, 23, "q4k"),     # the most experts a plan takes
    (2048, 100, 6, 512, 3, 24, "q4k"),     # expert count not a multiple of 64
    (512, 16, 2, 256, 4, 25, "q4k"),       # router without the norm prologue: epilogue kernel per layer
    (2048, 128, 8, 768, 4, 26, "mxfp4"),   # MXFP4 expert weights
])
def test_stack_step_equals_chained_forward(dev, hidden, E, k, inter, L, seed, fmt):
    """One-token stacked step (each layer's input formed inside the next
    router launch where the kernel has that prologue): eagerly and as graph
    replays it must reproduce, bit for bit, the chained moe_forward calls
    with the RMSNorm epilogue; step 0 is also held against the oracle's
    trajectory."""
    mx = fmt == "mxfp4"
    S = synth.Shape(f"stack-h{hidden}-e{E}", seed, hidden, E, k, inter, synth.FMT_MXFP4 if mx else synth.FMT_Q4K)
    plan = q.Plan(hidden, E, k, inter, n_layers=L, max_tokens=1, flags=q.FLAG_WEIGHTS_MXFP4 if mx else 0)
    blob = plan.upload_blob(layer_source(S), device=dev)
    x0 = torch.from_numpy(synth.x_bf16(S, 3, 0)[0].view(np.int16)).to(dev)
    ref = _chained_forward(plan, blob, L, hidden, k, x0, dev)
    _assert_same(_stack_once(plan, blob, L, hidden, k, x0, dev, graph=False)[0], ref, "eager")
    for i, o in enumerate(_stack_once(plan, blob, L, hidden, k, x0, dev, graph=True, replays=3)):
        _assert_same(o, ref, f"graph replay {i}")
    got = dict(xs=ref[0].cpu().numpy().view(np.uint16), ys=ref[1].cpu().numpy(), ids=ref[2].cpu().numpy())
    _check_step_properties(S, got)
    compared, exact, worst, flips, why = _compare_step(S, L, oracle.ExpertSource(S), x0.cpu().numpy().view(np.uint16),
                                                       got)
    assert exact >= 1 and compared >= 1


def test_full_stack_step_equals_chained_forward(dev, qwen_stack):
    """The 48-layer stack at hidden 2048 (the benchmark's blob): the step,
    eager and as graph replays, equals the chained moe_forward calls bit for
    bit."""
    S, plan, blob, _ = qwen_stack
    H, k = S.hidden, S.top_k
    x0 = torch.from_numpy(synth.x_bf16(S, 4, 0)[0].view(np.int16)).to(dev)
    ref = _chained_forward(plan, blob, 48, H, k, x0, dev)
    _assert_same(_stack_once(plan, blob, 48, H, k, x0, dev, graph=False)[0], ref, "eager")
    for i, o in enumerate(_stack_once(plan, blob, 48, H, k, x0, dev, graph=True, replays=2)):
        _assert_same(o, ref, f"graph replay {i}")


def _chained_forward_T(plan, blob, L, H, k, T, x0, dev):
    """A T-token step as L chained moe_forward calls with the RMSNorm
    epilogue (x_next of the last layer into a separate buffer)."""
    xs = torch.zeros(L, T, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, T, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, T, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, T, k, dtype=torch.float32, device=dev)
    xs[0].copy_(x0)
    last = torch.zeros(T, H, dtype=torch.int16, device=dev)
    scratch = plan.new_scratch(T, device=dev)
    for l in range(L):
        nxt = xs[l + 1] if l + 1 < L else last
        plan.forward(blob, l, xs[l], T, ys[l], x_next=nxt, ids=ids[l], w=ws[l], scratch=scratch)
    torch.cuda.synchronize()
    xs[0].copy_(last)
    return xs, ys, ids, ws


def _stack_once_T(plan, blob, L, H, k, T, x0, dev, graph, replays=1):
    xs = torch.zeros(L, T, H, dtype=torch.int16, device=dev)
    ys = torch.zeros(L, T, H, dtype=torch.float32, device=dev)
    ids = torch.zeros(L, T, k, dtype=torch.int32, device=dev)
    ws = torch.zeros(L, T, k, dtype=torch.float32, device=dev)
    scratch = plan.new_scratch(T, device=dev)
    stream = torch.cuda.Stream()
    if not graph:
        xs[0].copy_(x0)
        torch.cuda.synchronize()
        plan.stack_step(blob, xs, ys, T, ids, ws, scratch=scratch, stream=stream)
        torch.cuda.synchronize()
        return [(xs.clone(), ys.clone(), ids.clone(), ws.clone())]
    g = plan.capture_step(blob, xs, ys, T, ids, ws, scratch=scratch, stream=stream)
    outs = []
    for _ in range(replays):
        xs.zero_(), ys.zero_(), ids.zero_(), ws.zero_()
        xs[0].copy_(x0)
        other = torch.randn(1000, device=dev).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.launch(stream)
        torch.cuda.synchronize()
        assert other.isfinite()
        outs.append((xs.clone(), ys.clone(), ids.clone(), ws.clone()))
    return outs


QWEN = (2048, 128, 8, 768)


@pytest.mark.parametrize("T,L,dims", [(8, 3, QWEN), (128, 3, QWEN), (1, 1, QWEN), (8, 1, QWEN), (128, 1, QWEN),
                                      (1, 2, (3072, 32, 4, 768)), (8, 2, (3072, 32, 4, 768)),
                                      (1, 2, (4096, 128, 8, 1536))])
def test_stack_step_tokens_and_single_layer(dev, T, L, dims):
    """The stacked step at T = 8 and 128 tokens (the batched paths and the
    router's norm prologue over several tokens), with a single layer (whose
    epilogue writes the next step's input over its own input), and on
    hidden 3072 and a Qwen3-235B-A22B-shaped layer (hidden 4096, inter
    1536): eager and graph replays equal the chained moe_forward calls bit
    for bit; layer 0 (seeded input) is held against the oracle token by
    token (ids, y, x_next), later layers for properties."""
    H_, E_, k_, I_ = dims
    S = synth.Shape(f"stack-T{T}-L{L}-h{H_}", 40 + L + (H_ != 2048), H_, E_, k_, I_)
    H, k = S.hidden, S.top_k
    plan = q.Plan(H, S.n_experts, k, S.inter, n_layers=L, max_tokens=T)
    blob = plan.upload_blob(layer_source(S), device=dev)
    xb0 = synth.x_bf16(S, 44, T, T=T)
    x0 = torch.from_numpy(xb0.view(np.int16)).to(dev)
    ref = _chained_forward_T(plan, blob, L, H, k, T, x0, dev)
    _assert_same(_stack_once_T(plan, blob, L, H, k, T, x0, dev, graph=False)[0], ref, "eager")
    for i, o in enumerate(_stack_once_T(plan, blob, L, H, k, T, x0, dev, graph=True, replays=2)):
        _assert_same(o, ref, f"graph replay {i}")
    xs, ys, ids, ws = (t.cpu().numpy() for t in ref)
    xs = xs.view(np.uint16)
    for l in range(L):
        for t in range(T):
            assert len(set(ids[l, t].tolist())) == k and np.isfinite(ys[l, t]).all()
    src = oracle.ExpertSource(S)
    sample = list(range(T)) if T <= 8 else sorted({0, 1, 31, 64, 100, T - 1})
    oref = oracle.moe_layer(src, 0, xb0[sample])
    exempt = check_routing(ids[0][sample], ws[0][sample], oref, label=f"T={T} L={L} layer 0")
    yref = reference_outputs(src, 0, xb0[sample], oref, ids[0][sample], exempt)
    check_outputs(ys[0][sample], yref, label=f"T={T} L={L} layer 0")
    nxt = xs[1] if L > 1 else xs[0]             # L = 1: the step's output is the next step's input
    for i, t in enumerate(sample):
        _, rn = oracle.resid_rmsnorm(xb0[t], yref[i])
        check_bf16_vector(nxt[t], rn)

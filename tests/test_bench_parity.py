"""bench.py's step-0 parity report on the CPU (no GPU), on step records made by
the oracle itself: such a record passes with zero error; one layer's output
off by more than the tolerance on identical inputs is refused; once one-step
bf16 flips have parted the inputs, the comparison follows the trajectories
and stops, without failing, at the first layer that no longer agrees."""
import numpy as np
import pytest

import bench
import oracle
import synth

S = synth.Shape("tiny-stack", 1, 256, 8, 2, 512)
L = 4


def _oracle_step():
    """A step record in the GPU's layout (xs: layer inputs, xs[0] already the
    next step's input; ys; ids) computed by the oracle."""
    src = oracle.ExpertSource(S)
    x0 = synth.x_bf16(S, 3, 0)
    x = x0[0]
    xs = np.zeros((L, S.hidden), np.uint16)
    ys = np.zeros((L, S.hidden), np.float32)
    ids = np.zeros((L, S.top_k), np.int32)
    for l in range(L):
        rid, rw, _ = oracle.route(oracle.router_logits(synth.router(S, l), x), S.top_k)
        bl = [src.blocks(l, e) for e in rid]
        y = oracle.moe_token([b[0] for b in bl], [b[1] for b in bl], [b[2] for b in bl], rw, x)
        _, xn = oracle.resid_rmsnorm(x, y)
        ys[l], ids[l] = y, rid
        xs[(l + 1) % L] = xn
        x = xn
    return x0, dict(xs=xs, ys=ys, ids=ids)


def test_oracle_record_passes_both_ways():
    x0, gpu = _oracle_step()
    cpu, parity = bench.cpu_baseline(S, L, x0, gpu)
    assert cpu["cores"] == 1 and cpu["value"] > 0
    assert parity["layers_compared"] == L and parity["layers_on_identical_inputs"] == L
    assert parity["worst_rel_err"] < 1e-6 and parity["stopped"] is None


def test_a_wrong_layer_is_refused():
    x0, gpu = _oracle_step()
    gpu["ys"][2] *= 1.01                     # 1 % off: five times the tolerance
    with pytest.raises(AssertionError, match="layer 2"):
        bench.cpu_baseline(S, L, x0, gpu)



def _parted_record():
    """A record whose layer-2 next input has a few elements one bf16 step
    away from the oracle's (the rounding flips that part real trajectories),
    with layers 3.. recomputed by the oracle from that input: consistent
    layer by layer, but no longer on the oracle's own trajectory."""
    x0, gpu = _oracle_step()
    src = oracle.ExpertSource(S)
    x = gpu["xs"][3].copy()
    x[:5] += 1                               # one bf16 step away from zero
    gpu["xs"][3] = x
    for l in range(3, L):
        rid, rw, _ = oracle.route(oracle.router_logits(synth.router(S, l), x), S.top_k)
        bl = [src.blocks(l, e) for e in rid]
        y = oracle.moe_token([b[0] for b in bl], [b[1] for b in bl], [b[2] for b in bl], rw, x)
        _, xn = oracle.resid_rmsnorm(x, y)
        gpu["ys"][l], gpu["ids"][l] = y, rid
        gpu["xs"][(l + 1) % L] = xn
        x = xn
    return x0, gpu


def test_parted_trajectories_are_followed_then_left():
    x0, gpu = _parted_record()
    _, parity = bench.cpu_baseline(S, L, x0, gpu)
    assert parity["layers_on_identical_inputs"] == 3 and parity["layers_compared"] == L
    assert parity["stopped"] is None and parity["x_next_bf16_differences"] >= 5
    # past the parting a layer that no longer agrees ends the comparison
    gpu["ys"][3] *= 1.01
    _, parity = bench.cpu_baseline(S, L, x0, gpu)
    assert parity["stopped"] == "trajectories parted at layer 3" and parity["layers_compared"] == 3

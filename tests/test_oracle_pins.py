"""Pins for the CPU oracle: each check ties a piece of it to something other
than itself (a worked example with exact answers, exhaustive sweeps against a
library conversion, library matmul/sort/softmax, brute force, closed forms).
A plausible slip anywhere in the oracle (wrong nibble, swapped scale/min
fields, sign of the min, dropped term, transposed operand, wrong tie rule)
fails at least one of these."""
import itertools
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth

QB = oracle.QBLOCK_BYTES


def _load_worked_example(golden_dir):
    blk = None
    w = None
    with open(os.path.join(golden_dir, "q4k_worked_example.txt")) as f:
        for line in f:
            if line.startswith("block_hex "):
                blk = np.frombuffer(bytes.fromhex(line.split()[1]), dtype=np.uint8)
            elif line.startswith("weights "):
                w = np.array([int(v) for v in line.split()[1:]], dtype=np.float64)
    return blk, w


def _block_from_fields(d_bits, dmin_bits, sc, m, q):
    """Independent encoder for test blocks (big-integer bit packing)."""
    blk = bytearray(QB)
    blk[0:2] = int(d_bits).to_bytes(2, "little")
    blk[2:4] = int(dmin_bits).to_bytes(2, "little")
    bits = 0
    for f, v in enumerate(list(sc) + list(m)):
        assert 0 <= v < 64
        bits |= int(v) << (6 * f)
    blk[4:16] = bits.to_bytes(12, "little")
    for i in range(256):
        j, e = divmod(i, 32)
        byte = 16 + 16 * j + e // 2
        blk[byte] |= (int(q[i]) << 4) if (e & 1) else int(q[i])
    return np.frombuffer(bytes(blk), dtype=np.uint8)


# ------------------------------------------------------------------ codec
def test_worked_example_block(golden_dir):
    blk, w = _load_worked_example(golden_dir)
    assert blk.size == QB and w.size == 256
    got = oracle.dequant_block(blk)
    assert np.array_equal(got, w)
    assert got[0] == 0 and got[33] == 1 and got[255] == 113


def test_six_bit_fields_every_position_every_value():
    """Each of the 16 packed fields at every value 0..63: scales via q=1,
    mins via q=0 (d = dmin = 1)."""
    one = 0x3C00
    for f in range(16):
        for v in range(64):
            sc = [0] * 8
            m = [0] * 8
            if f < 8:
                sc[f] = v
            else:
                m[f - 8] = v
            q = np.ones(256, dtype=np.int64)
            w = oracle.dequant_block(_block_from_fields(one, one, sc, m, q))
            exp = np.array([sc[i // 32] * 1 - m[i // 32] for i in range(256)], dtype=np.float64)
            assert np.array_equal(w, exp), (f, v)


def test_codes_every_nibble_position():
    rng = np.random.default_rng(1)
    for _ in range(20):
        q = rng.integers(0, 16, 256)
        sc = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        w = oracle.dequant_block(_block_from_fields(0x3C00, 0x3800, sc, m, q))
        exp = np.array([sc[i // 32] * q[i] - 0.5 * m[i // 32] for i in range(256)], dtype=np.float64)
        assert np.array_equal(w, exp)


def test_f16_all_finite_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    got = np.array([oracle.f16(int(b)) for b in bits[finite]])
    assert np.array_equal(got, ref[finite])


def test_d_dmin_scaling_and_extremes():
    q = np.arange(256) % 16
    for d_bits in (0x0000, 0x0001, 0x03FF, 0x0400, 0x3555, 0x7BFF):
        for dmin_bits in (0x0000, 0x0001, 0x2E66, 0x7BFF):
            d = float(np.array([d_bits], dtype=np.uint16).view(np.float16)[0])
            dmin = float(np.array([dmin_bits], dtype=np.uint16).view(np.float16)[0])
            sc = [63, 1, 0, 17, 32, 5, 9, 44]
            m = [0, 63, 12, 1, 2, 33, 60, 7]
            w = oracle.dequant_block(_block_from_fields(d_bits, dmin_bits, sc, m, q))
            exp = np.array([d * sc[i // 32] * q[i] - dmin * m[i // 32] for i in range(256)])
            assert np.array_equal(w, exp)


def test_all_zero_block_is_zero():
    assert np.array_equal(oracle.dequant_block(np.zeros(QB, np.uint8)), np.zeros(256))


# ------------------------------------------------------------------ quantizer vs decoder
def test_decoded_synthetic_weights_within_quantizer_bound():
    """The shared generator's encoder and the oracle's decoder agree: every
    decoded weight lies within half a code step (plus the fp16/6-bit scale
    rounding slack) of the Gaussian value it encodes."""
    S = synth.TINY
    w = synth.expert_matrix_f32(S, 0, 3, synth.GATE).astype(np.float64)
    deq = oracle.dequant_matrix(synth.expert_matrix(S, 0, 3, synth.GATE))
    rows, cols = w.shape
    for r in range(0, rows, 37):
        for b in range(cols // 256):
            seg = w[r, 256 * b:256 * (b + 1)].reshape(8, 32)
            err = np.abs(deq[r, 256 * b:256 * (b + 1)].reshape(8, 32) - seg)
            rng_ = seg.max(1) - np.minimum(seg.min(1), 0)
            # step ~ range/15; scale rounding (6-bit sc, fp16 d) adds <= ~1 step at the ends
            assert np.all(err.max(1) <= rng_ / 15 * 1.5 + 1e-6)
    assert np.abs(deq - w).max() < 0.02 and np.abs(deq - w).mean() < 0.004


# ------------------------------------------------------------------ GEMV
@pytest.mark.parametrize("shape,mat", [(synth.TINY, synth.GATE), (synth.TINY, synth.DOWN),
                                       (synth.QWEN3_30B_A3B, synth.UP)])
def test_qgemv_matches_library_matmul(shape, mat):
    blocks = synth.expert_matrix(shape, 0, 1, mat)
    W = oracle.dequant_matrix(blocks)
    x = np.random.default_rng(2).standard_normal(W.shape[1])
    y = oracle.qgemv(blocks, x)
    ref = W @ x
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(W).sum(1).max())


def test_router_logits_match_library_matmul():
    S = synth.TINY
    wr = synth.router(S, 0)
    xb = synth.x_bf16(S, 0, 0)[0]
    got = oracle.router_logits(wr, xb)
    ref = wr.astype(np.float64) @ oracle.bf16_array(xb)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_bf16_decode_matches_float32_upper_half():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(ref)
    got = np.array([oracle.bf16(int(b)) for b in bits[ok]])
    assert np.array_equal(got, ref[ok])


def test_round_bf16_is_nearest_ties_to_even():
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000)))
    # exact midpoints between neighbouring bf16 values, both parities
    for b in (0x3F80, 0x3F81, 0x4000, 0xC123, 0x0081, 0x0001):
        lo = oracle.bf16(b)
        hi = oracle.bf16(b + 1)
        vals.append((lo + hi) / 2)
    for v in vals:
        r = oracle.round_bf16(v)
        rv = oracle.bf16(r)
        nb = [oracle.bf16((r + d) & 0xFFFF) for d in (-1, 1)]
        for n in nb:
            if np.isfinite(n) and np.sign(n) == np.sign(rv):
                assert abs(v - rv) <= abs(v - n)
                if abs(v - rv) == abs(v - n):
                    assert r % 2 == 0


# ------------------------------------------------------------------ top-k
def test_topk_all_orderings_e8():
    base = np.array([0.5, -1.0, 2.0, 3.25, -0.75, 1.5, 0.0, -2.5])
    for perm in itertools.permutations(range(8)):
        lg = base[list(perm)]
        ref = np.argsort(-lg, kind="stable")
        for k in (1, 2, 3, 8):
            assert np.array_equal(oracle.topk(lg, k), ref[:k])


def test_topk_ties_take_lower_id():
    lg = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -1.0])
    assert list(oracle.topk(lg, 2)) == [1, 2]
    assert list(oracle.topk(lg, 4)) == [1, 2, 4, 3]
    assert list(oracle.topk(np.zeros(5), 3)) == [0, 1, 2]


def test_topk_random_large_matches_library_sort():
    rng = np.random.default_rng(4)
    for _ in range(200):
        lg = rng.standard_normal(128)
        assert np.array_equal(oracle.topk(lg, 8), np.argsort(-lg, kind="stable")[:8])


# ------------------------------------------------------------------ softmax-renorm
def test_route_weights_sum_to_one_and_match_library_softmax():
    rng = np.random.default_rng(5)
    for _ in range(100):
        lg = rng.standard_normal(128) * 3
        ids = oracle.topk(lg, 8)
        w = oracle.route_weights(lg, ids)
        assert abs(w.sum() - 1) <= 1e-15 * 8
        full = softmax(lg)
        ref = full[ids] / full[ids].sum()
        assert np.allclose(w, ref, rtol=1e-13, atol=0)
        w2 = oracle.route_weights(lg + 17.5, ids)
        assert np.allclose(w, w2, rtol=1e-13)
        assert np.all(np.diff(w) <= 0)          # descending logits -> descending weights


def test_route_weights_two_expert_closed_form():
    for a, b in [(0.3, -1.2), (5.0, 4.999), (-3.0, -7.0)]:
        w = oracle.route_weights(np.array([a, b]), np.array([0, 1], dtype=np.int32))
        assert np.isclose(w[0], expit(a - b), rtol=1e-14)
        assert np.isclose(w[1], expit(b - a), rtol=1e-14)


# ------------------------------------------------------------------ SiLU
def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for z in np.linspace(-20, 20, 81):
        assert np.isclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-13, atol=1e-13)
        assert np.isclose(oracle.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------ gate activations
def test_act_silu_is_silu_times_up():
    for g, u in [(0.0, 3.0), (1.5, -2.0), (-4.0, 0.25), (12.0, 1.0)]:
        assert oracle.act(g, u, oracle.ACT_SILU) == oracle.silu(g) * u


def test_act_relu2_closed_forms():
    R = oracle.ACT_RELU2
    for g in (-3.5, -1e-9, 0.0):                     # zero for g <= 0, any u
        assert oracle.act(g, 7.0, R) == 0.0
    assert oracle.act(3.0, 2.0, R) == 18.0           # exact small integers
    assert oracle.act(0.5, 4.0, R) == 1.0
    assert oracle.act(-2.0, -5.0, R) == 0.0
    for c in (0.5, 2.0, 3.0):                        # degree 2 in g, degree 1 in u
        assert np.isclose(oracle.act(c * 1.3, 0.7, R), c * c * oracle.act(1.3, 0.7, R), rtol=1e-14)
        assert np.isclose(oracle.act(1.3, c * 0.7, R), c * oracle.act(1.3, 0.7, R), rtol=1e-14)


def test_act_swiglu_oai_closed_forms():
    O = oracle.ACT_SWIGLU_OAI
    assert oracle.act(0.0, 3.0, O) == 0.0
    for g in (-9.0, 0.3, 6.5, 20.0):                 # u' = -1 cancels the gate for any g
        assert oracle.act(g, -1.0, O) == 0.0
    # g' sigmoid(a g') is a swish: its odd part is g'/2, so act(g) - act(-g) = g (u' + 1)
    for g in np.linspace(-6.9, 6.9, 47):
        for u in (-3.0, 0.4, 6.0):
            assert np.isclose(oracle.act(g, u, O) - oracle.act(-g, u, O), g * (u + 1.0), rtol=1e-12, atol=1e-12)
    # clamps: the gate at 7 from above only, the up value at +-7
    assert oracle.act(7.0, 0.5, O) == oracle.act(50.0, 0.5, O)
    assert oracle.act(-30.0, 0.5, O) != oracle.act(-7.0, 0.5, O)
    assert oracle.act(2.0, 7.0, O) == oracle.act(2.0, 100.0, O)
    assert oracle.act(2.0, -7.0, O) == oracle.act(2.0, -40.0, O)
    # sigmoid with slope 1.702 (scipy's logistic, a library routine)
    for g, u in [(1.0, 0.0), (-2.5, 1.5), (4.0, -0.5)]:
        assert np.isclose(oracle.act(g, u, O), g * expit(1.702 * g) * (u + 1.0), rtol=1e-14)
    # far below zero the gate vanishes
    assert abs(oracle.act(-40.0, 0.0, O)) < 1e-25


# ------------------------------------------------------------------ FFN / MoE
def _dense_ffn(src, layer, e, x, act=None):
    g, u, d = [oracle.dequant_matrix(b) for b in src.blocks(layer, e)]
    hg, hu = g @ x, u @ x
    if act is None:
        return d @ (hg * expit(hg) * hu)
    return d @ np.array([oracle.act(a, b, act) for a, b in zip(hg, hu)])


@pytest.mark.parametrize("act", [1, 2])
def test_expert_ffn_activation_matches_dense_numpy(act):
    """FFN with each non-default gate activation against dense numpy matmuls
    (library routines) on the dequantized matrices; x scaled up so that the
    SwiGLU clamps act on part of the rows."""
    src = oracle.ExpertSource(synth.TINY)
    x = 8.0 * oracle.bf16_array(synth.x_bf16(synth.TINY, 0, 0)[0])
    y, h = oracle.expert_ffn(*src.blocks(0, 5), x, return_h=True, act=act)
    assert np.allclose(y, _dense_ffn(src, 0, 5, x, act), rtol=1e-11, atol=1e-12)
    g = oracle.dequant_matrix(src.blocks(0, 5)[0]) @ x
    if act == 2:
        assert (g > 7.0).any() and (g < 7.0).any()


def test_expert_ffn_matches_dense_numpy():
    src = oracle.ExpertSource(synth.TINY)
    x = oracle.bf16_array(synth.x_bf16(synth.TINY, 0, 0)[0])
    y = oracle.expert_ffn(*src.blocks(0, 5), x)
    assert np.allclose(y, _dense_ffn(src, 0, 5, x), rtol=1e-11, atol=1e-12)


def test_one_hot_k1_is_dense_ffn_of_argmax_expert():
    S = synth.Shape("tiny-k1", 1, 256, 8, 1, 512)
    src = oracle.ExpertSource(S)
    xb = synth.x_bf16(S, 7, 0, T=3)
    res = oracle.moe_layer(src, 0, xb)
    for t in range(3):
        x = oracle.bf16_array(xb[t])
        e = int(np.argmax(synth.router(S, 0).astype(np.float64) @ x))
        assert res["ids"][t, 0] == e and res["w"][t, 0] == 1.0
        assert np.allclose(res["y"][t], _dense_ffn(src, 0, e, x), rtol=1e-11, atol=1e-12)


def test_identical_experts_give_dense_ffn_for_any_k():
    S = synth.TINY
    src = oracle.ExpertSource(S)
    g, u, d = src.blocks(0, 2)
    xb = synth.x_bf16(S, 8, 0)[0]
    x = oracle.bf16_array(xb)
    ref = _dense_ffn(src, 0, 2, x)
    for k in (1, 2, 5, 8):
        w = np.random.default_rng(k).dirichlet(np.ones(k))
        y = oracle.moe_token([g] * k, [u] * k, [d] * k, w, xb)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_moe_layer_is_weighted_sum_of_selected_experts():
    S = synth.TINY
    src = oracle.ExpertSource(S)
    xb = synth.x_bf16(S, 9, 0)
    res = oracle.moe_layer(src, 0, xb)
    x = oracle.bf16_array(xb[0])
    lg = synth.router(S, 0).astype(np.float64) @ x
    ids = np.argsort(-lg, kind="stable")[:2]
    w = softmax(lg)[ids] / softmax(lg)[ids].sum()
    ref = sum(w[s] * _dense_ffn(src, 0, ids[s], x) for s in range(2))
    assert np.array_equal(res["ids"][0], ids)
    assert np.allclose(res["y"][0], ref, rtol=1e-11, atol=1e-13)


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(6)
    xb = synth.f32_to_bf16_bits(rng.standard_normal(2048).astype(np.float32))
    y = rng.standard_normal(2048) * 0.3
    r, rb = oracle.resid_rmsnorm(xb, y, eps=0.0)
    assert np.isclose(np.sqrt(np.mean(r * r)), 1.0, rtol=1e-14)
    v = oracle.bf16_array(xb) + y
    assert np.allclose(r, v / np.sqrt(np.mean(v * v)), rtol=1e-14)
    # scale invariance (eps = 0): RMSNorm(c v) = RMSNorm(v)
    xz = np.zeros(2048, dtype=np.uint16)
    r1, _ = oracle.resid_rmsnorm(xz, v, eps=0.0)
    r2, _ = oracle.resid_rmsnorm(xz, 7.0 * v, eps=0.0)
    assert np.allclose(r1, r2, rtol=1e-14)
    # eps shrinks the norm as sqrt(ms / (ms + eps))
    r3, _ = oracle.resid_rmsnorm(xz, v * 1e-3, eps=1e-6)
    ms = np.mean((v * 1e-3) ** 2)
    assert np.isclose(np.sqrt(np.mean(r3 * r3)), np.sqrt(ms / (ms + 1e-6)), rtol=1e-12)
    assert all(rb[i] == oracle.round_bf16(r[i]) for i in range(0, 2048, 97))


# ------------------------------------------------------------------ MXFP4 codec
MXB = oracle.MXBLOCK_BYTES


def _load_mx_worked_example(golden_dir):
    blk = w = None
    with open(os.path.join(golden_dir, "mxfp4_worked_example.txt")) as f:
        for line in f:
            if line.startswith("block_hex "):
                blk = np.frombuffer(bytes.fromhex(line.split()[1]), dtype=np.uint8)
            elif line.startswith("weights_eighths "):
                w = np.array([float(v) for v in line.split()[1:]], dtype=np.float64) / 8.0
    return blk, w


def _mx_block(e, codes):
    """Independent encoder for test blocks: scale byte, then code pairs."""
    blk = bytearray(MXB)
    blk[0] = int(e)
    for i, c in enumerate(codes):
        blk[1 + i // 2] |= (int(c) << 4) if (i & 1) else int(c)
    return np.frombuffer(bytes(blk), dtype=np.uint8)


def test_mx_worked_example_block(golden_dir):
    blk, w = _load_mx_worked_example(golden_dir)
    assert blk.size == MXB and w.size == 32
    got = oracle.dequant_mx_block(blk)
    assert np.array_equal(got, w)
    assert got[7] == 0.75 and got[9] == -1 / 16 and got[31] == -0.75


def test_e8m0_every_code_matches_library_decode():
    """All 256 scale codes against torch's float8_e8m0fnu conversion."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib_vals = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = np.array([oracle.e8m0(e) for e in range(256)])
    assert np.isnan(mine[255]) and np.isnan(lib_vals[255])
    assert np.array_equal(mine[:255], lib_vals[:255])


def test_fp4_every_code_matches_library_e4m3_decode():
    """Each E2M1 code re-encoded as the float8 E4M3 number of the same sign,
    unbiased exponent and mantissa (E2M1 exponent bias 1, one mantissa bit;
    E4M3 bias 7, three mantissa bits; the E2M1 subnormal 1/2 is the normal
    2^-1), decoded by torch's float8_e4m3fn conversion; plus the format's
    invariants: sign symmetry, strictly increasing magnitudes, largest 6."""
    import torch
    bits = []
    for c in range(16):
        s, ex, m = c >> 3, (c >> 1) & 3, c & 1
        if ex == 0 and m == 0:
            e4 = 0                                    # zero
        elif ex == 0:
            e4 = (s << 7) | ((-1 + 7) << 3)           # 2^-1
        else:
            e4 = (s << 7) | ((ex - 1 + 7) << 3) | (m << 2)
        bits.append(e4)
    lib_vals = torch.tensor(bits, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    mine = np.array([oracle.fp4(c) for c in range(16)])
    assert np.array_equal(np.abs(mine), np.abs(lib_vals.numpy()))
    assert np.array_equal(np.sign(mine[9:]), -np.ones(7)) and np.array_equal(mine[8:], -mine[:8])
    assert np.all(np.diff(mine[:8]) > 0) and mine[7] == 6.0 and mine[1] == 0.5


def test_mx_every_nibble_position_and_scale():
    """A single nonzero code at every element position (the nibble order) and
    every usable scale code 1..254 (the power of two applied)."""
    for i in range(32):
        codes = np.zeros(32, np.int64)
        codes[i] = 5                                   # 3.0
        got = oracle.dequant_mx_block(_mx_block(127, codes))
        ref = np.zeros(32)
        ref[i] = 3.0
        assert np.array_equal(got, ref), i
    for e in range(1, 255):
        got = oracle.dequant_mx_block(_mx_block(e, [2] * 32))   # 1.0 each
        assert np.all(got == 2.0 ** (e - 127)), e


@pytest.mark.parametrize("mat", [synth.GATE, synth.DOWN])
def test_mx_qgemv_matches_library_matmul(mat):
    S = synth.Shape("tiny-mx", 1, 256, 8, 2, 512, synth.FMT_MXFP4)
    blocks = synth.expert_matrix(S, 0, 1, mat)
    assert blocks.shape[-1] == MXB
    W = oracle.dequant_matrix(blocks)
    # the matrix decoder is the block decoder applied block by block
    assert np.array_equal(W[3, 64:96], oracle.dequant_mx_block(blocks[3, 2]))
    x = np.random.default_rng(2).standard_normal(W.shape[1])
    y = oracle.qgemv(blocks, x)
    assert np.allclose(y, W @ x, rtol=1e-12, atol=1e-12 * np.abs(W).sum(1).max())


def test_mx_quantizer_bound_and_idempotence():
    """The shared generator's MXFP4 encoder and the oracle's decoder agree:
    each decoded weight is within half a grid step of its Gaussian value
    (values beyond 6 * scale saturate to 6 * scale), and re-encoding the
    decoded weights gives the same blocks."""
    S = synth.Shape("tiny-mx", 1, 256, 8, 2, 512, synth.FMT_MXFP4)
    w = synth.expert_matrix_f32(S, 0, 3, synth.UP).astype(np.float64)
    blocks = synth.expert_matrix(S, 0, 3, synth.UP)
    deq = oracle.dequant_matrix(blocks)
    scale = np.array([[oracle.e8m0(e) for e in row] for row in blocks[:, :, 0]])
    sc = np.repeat(scale, 32, axis=1)
    a = np.abs(w) / sc
    half_step = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * sc
    sat = a > 6
    assert np.all(np.abs(deq - w)[~sat] <= half_step[~sat] * (1 + 1e-12))
    assert np.all(np.abs(deq[sat]) == 6 * sc[sat])
    assert np.array_equal(synth.quantize_rows(deq.astype(np.float32), synth.FMT_MXFP4), blocks)


def test_mx_expert_ffn_matches_dense_numpy():
    S = synth.Shape("tiny-mx", 1, 256, 8, 2, 512, synth.FMT_MXFP4)
    src = oracle.ExpertSource(S)
    x = oracle.bf16_array(synth.x_bf16(S, 0, 0)[0])
    y = oracle.expert_ffn(*src.blocks(0, 5), x)
    assert np.allclose(y, _dense_ffn(src, 0, 5, x), rtol=1e-11, atol=1e-12)
    res = oracle.moe_layer(src, 0, synth.x_bf16(S, 0, 0))
    ids, w = res["ids"][0], res["w"][0]
    ref = sum(w[s] * _dense_ffn(src, 0, ids[s], x) for s in range(S.top_k))
    assert np.allclose(res["y"][0], ref, rtol=1e-11, atol=1e-13)


# ------------------------------------------------------------------ selection margin
def _kth_largest_by_counting(lg, k):
    """The k-th largest value by counting (no sort): v with #{l > v} < k <= #{l >= v}."""
    for v in lg:
        if np.count_nonzero(lg > v) < k <= np.count_nonzero(lg >= v):
            return v
    raise AssertionError("no k-th value")


def test_selection_margin_against_brute_force():
    """route()'s margin l_(k) - l_(k+1) against k-th values found by counting,
    on random logits, on sorted and reversed logits, with constructed ties
    (margin 0 exactly where the tie rule decides) and with k = E (every
    selection is the same set: infinite margin)."""
    rng = np.random.default_rng(21)
    for trial in range(300):
        E = int(rng.integers(2, 40))
        k = int(rng.integers(1, E + 1))
        lg = rng.standard_normal(E)
        if trial % 5 == 1:
            lg = np.sort(lg)
        elif trial % 5 == 2:
            lg = np.sort(lg)[::-1].copy()
        elif trial % 5 == 3:
            lg = np.round(lg * 2) / 2               # many exact ties
        ids, w, gap = oracle.route(lg, k)
        if k == E:
            assert gap == np.inf
            continue
        ref = _kth_largest_by_counting(lg, k) - _kth_largest_by_counting(lg, k + 1)
        assert gap == ref and gap >= 0
        # the margin separates the selection from the rest, and is attained
        sel = set(ids.tolist())
        rest = [e for e in range(E) if e not in sel]
        assert min(lg[list(sel)]) - max(lg[rest]) == gap
    lg = np.array([3.0, 1.0, 2.0, 2.0, 0.5])
    assert oracle.route(lg, 2)[2] == 0.0          # experts 2 and 3 tie for the 2nd place
    assert oracle.route(lg, 3)[2] == 1.0
    assert oracle.route(lg, 1)[2] == 1.0
    assert oracle.route(np.array([1.0, -1.0]), 2)[2] == np.inf


def test_check_routing_rejects_far_swaps_and_bounds_exemptions():
    """The parity tests' routing rule (host logic): a selection that differs
    from the oracle's only by an expert tied with the k-th logit within tau
    is exempted; one that differs by an expert far from it, or too many
    exemptions, fail."""
    from helpers import TAU, check_routing
    lg = np.array([[4.0, 1.0, 1.0 + 0.5 * TAU, -2.0, 0.0]])
    ref = dict(ids=np.array([[0, 2]]), w=oracle.route_weights(lg[0], np.array([0, 2], np.int32))[None],
               gap=np.array([0.5 * TAU]), logits=lg)
    w_alt = oracle.route_weights(lg[0], np.array([0, 1], np.int32))[None]
    assert check_routing(np.array([[0, 1]]), w_alt, ref) == [0]
    with pytest.raises(AssertionError):
        check_routing(np.array([[0, 1]]), w_alt, ref, exact=True)
    with pytest.raises(AssertionError):            # expert 4 is far from the k-th logit
        check_routing(np.array([[0, 4]]), oracle.route_weights(lg[0], np.array([0, 4], np.int32))[None], ref)
    with pytest.raises(AssertionError):
        check_routing(np.array([[0, 1]]), w_alt, ref, max_exempt=0)


# ------------------------------------------------------------------ recipe emulation
def test_emulation_roundings_match_library_conversions():
    """The emulation's fp16 (nearest even, overflow to inf) and bf16 roundings
    against numpy's float16 and torch's bfloat16 conversions, over normals,
    subnormals, exact midpoints and overflow; the toward-zero fp16 rounding
    never increases the magnitude, stays within one fp16 step and saturates
    at 65504."""
    import torch
    rng = np.random.default_rng(22)
    vals = rng.standard_normal(4000) * np.exp(rng.uniform(-25, 12, 4000))
    mids = (np.arange(1, 2000, dtype=np.float64) + 0.5) * 2.0 ** -24       # fp16 subnormal midpoints
    vals = np.concatenate([vals, mids, -mids, [65504.0, 65519.0, 65520.0, 1e6, -7e4, 2.0 ** -25, 3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref16 = vals.astype(np.float16).astype(np.float64)
    got16 = np.array([oracle.emul_fp16(v) for v in vals])
    assert np.array_equal(got16, ref16)
    v32 = vals.astype(np.float32)                   # bf16 rounds the fp32 value the GPU holds
    refb = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    gotb = np.array([oracle.emul_bf16(float(v)) for v in v32])
    assert np.array_equal(gotb, refb)
    for v in vals:
        r = oracle.emul_fp16_rtz(v)
        assert abs(r) <= abs(v) and np.sign(r) in (0, np.sign(v))
        if abs(v) <= 65504:
            with np.errstate(over="ignore"):
                up = np.nextafter(np.float16(abs(r)), np.float16(np.inf)).astype(np.float64)
            assert abs(v) < up
        else:
            assert abs(r) == 65504.0


def test_recipe_emulation_at_full_precision_is_the_oracle():
    """Exact codes with an fp32 sub-block affine and fp32 h differ from the
    fp64 oracle only by fp32 rounding (both encodings)."""
    for S in (synth.TINY, synth.Shape("tiny-mx", 1, 256, 8, 2, 512, synth.FMT_MXFP4)):
        src = oracle.ExpertSource(S)
        xb = synth.x_bf16(S, 61, 0, T=3)
        y, ref = oracle.emulate_moe_layer(src, 0, xb, oracle.W_EXACT_CODES, oracle.H_FP32)
        err = np.abs(y - ref["y"]).max() / np.abs(ref["y"]).max()
        assert 0 < err < 2e-6, err


def test_recipe_emulation_reproduces_precision_table():
    """P13: on the Qwen3-30B-A3B-shaped layer the emulation reproduces the
    recipe-error table worked out when the survey planned the MFMA recipe
    (max|err|/max|ref| of plain bf16 weights with bf16 h about 3.9e-3, bf16
    weights with fp32 h 3.5e-3, exact codes with bf16 h 2.08e-3, exact codes
    with h as bf16 hi + lo 2.7e-6, weights and h both hi + lo 4.6e-6, exact
    codes with fp16 h 2.1e-4), each within a factor of 2.5 on four tokens,
    and in the same order."""
    S = synth.QWEN3_30B_A3B
    src = oracle.ExpertSource(S)
    xb = synth.x_bf16(S, 60, 0, T=4)
    table = [(oracle.W_BF16, oracle.H_BF16, 3.9e-3), (oracle.W_BF16, oracle.H_FP32, 3.5e-3),
             (oracle.W_EXACT_CODES, oracle.H_BF16, 2.08e-3), (oracle.W_EXACT_CODES, oracle.H_BF16_HILO, 2.7e-6),
             (oracle.W_BF16_HILO, oracle.H_BF16_HILO, 4.6e-6), (oracle.W_EXACT_CODES, oracle.H_FP16, 2.1e-4)]
    ref = oracle.moe_layer(src, 0, xb)
    m = np.abs(ref["y"]).max()
    errs = []
    for wm, hm, expected in table:
        y, _ = oracle.emulate_moe_layer(src, 0, xb, wm, hm)
        e = np.abs(y - ref["y"]).max() / m
        errs.append(e)
        assert expected / 2.5 <= e <= expected * 2.5, (wm, hm, e, expected)
    order = np.argsort([t[2] for t in table])
    assert list(np.argsort(errs)) == list(order)


def test_recipe_emulation_predicts_fp16_range_failure():
    """With the squared-ReLU gate and inputs scaled by 2^8 (exact in bf16),
    h exceeds the fp16 range on the tiny layer: the fp16-h recipe (and fp16
    activations toward zero) breaks down while fp32 h and bf16 hi + lo h stay
    at fp32-level error."""
    S = synth.TINY
    src = oracle.ExpertSource(S)
    xb = synth.x_bf16(S, 62, 0, T=2)
    xs = ((xb.astype(np.uint32) + (8 << 7)) & 0xFFFF).astype(np.uint16)   # exponent + 8: x * 256
    assert np.array_equal(oracle.bf16_array(xs), 256.0 * oracle.bf16_array(xb))
    R = oracle.ACT_RELU2
    y16, ref = oracle.emulate_moe_layer(src, 0, xs, oracle.W_EXACT_CODES, oracle.H_FP16, act=R)
    m = np.abs(ref["y"]).max()
    assert not np.isfinite(y16).all() or np.abs(y16 - ref["y"]).max() / m > 1e-2
    for hm in (oracle.H_FP32, oracle.H_BF16_HILO):
        y, _ = oracle.emulate_moe_layer(src, 0, xs, oracle.W_EXACT_CODES, hm, act=R)
        assert np.abs(y - ref["y"]).max() / m < 2e-5, hm


# ---------------------------------------------------------------- FP8 hi + lo operands (block-scaled MFMA recipe)
def test_e4m3_rounding_against_torch():
    """The emulation's FP8 E4M3 rounding equals torch's float8_e4m3fn
    conversion (nearest even) on every E4M3 value, the midpoints between
    neighbours (ties), points a quarter step either side, subnormals and
    values up to 448; above 448 it saturates (torch's conversion does not,
    so only the in-range values are compared)."""
    import torch
    codes = torch.arange(0, 256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    vals = np.sort(np.unique(codes[np.isfinite(codes)]))
    pos = vals[vals >= 0]
    mids = (pos[1:] + pos[:-1]) / 2
    quarter = np.concatenate([pos[:-1] + (pos[1:] - pos[:-1]) / 4, pos[1:] - (pos[1:] - pos[:-1]) / 4])
    probe = np.concatenate([pos, mids, quarter, -pos, -mids, -quarter, [2.0 ** -12, 3.3e-3, 100.5, 447.9]])
    probe = probe[np.abs(probe) <= 448.0]
    want = torch.from_numpy(probe.astype(np.float32)).to(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.emul_e4m3(v) for v in probe])
    assert np.array_equal(got, want.astype(np.float64))
    assert oracle.emul_e4m3(500.0) == 448.0 and oracle.emul_e4m3(-1e9) == -448.0
    assert oracle.emul_e4m3(240.0) == 240.0 and oracle.emul_e4m3(232.0) == 224.0   # tie to the even code


def test_fp8_hilo_operands():
    """Per block of 32: the hi plane's scale is the smallest power of two
    that keeps max|v| / s within 448, so small integers (4 significant bits)
    come back exactly; a scaled block comes back scaled (powers of two
    commute with the split); the error is below 2^-8 of the block's largest
    magnitude; blocks are independent; zeros stay zero."""
    rng = np.random.default_rng(5)
    ints = rng.integers(-15, 16, size=64).astype(np.float32)
    assert np.array_equal(oracle.emul_fp8_hilo(ints), ints)
    v = rng.standard_normal(32 * 40).astype(np.float32) * np.repeat(2.0 ** rng.integers(-20, 20, 40), 32)
    out = oracle.emul_fp8_hilo(v)
    for b in range(40):
        blk, ob = v[32 * b:32 * b + 32].astype(np.float64), out[32 * b:32 * b + 32].astype(np.float64)
        assert np.abs(ob - blk).max() <= 2.0 ** -8 * np.abs(blk).max()
    assert np.array_equal(oracle.emul_fp8_hilo(v * np.float32(2.0 ** 7)), out * np.float32(2.0 ** 7))
    w = v.copy()
    w[32:64] *= np.float32(1e6)                       # a loud neighbour does not change a block
    assert np.array_equal(oracle.emul_fp8_hilo(w)[:32], out[:32])
    assert np.array_equal(oracle.emul_fp8_hilo(np.zeros(32, np.float32)), np.zeros(32, np.float32))
    # the hi plane alone would miss by up to 2^-4 relative: the lo plane is used
    one = np.full(32, 1.0 + 2.0 ** -6, np.float32)
    assert np.array_equal(oracle.emul_fp8_hilo(one), one)


def test_recipe_emulation_block_scaled_fp8():
    """P14: the block-scaled FP8 x FP4 recipe for MXFP4 experts (weights
    exact, activations and h as FP8 hi + lo with per-32 scales) on the
    Qwen3-30B-A3B-shaped MXFP4 layer: FP8 activations alone stay at fp32
    level (< 1e-5 of max|y|: bf16 inputs fit hi + lo almost exactly) while
    FP8 h costs about 7e-4, a third of the 2e-3 tolerance (between 3e-4
    and 1.5e-3 on two tokens); h in bf16 hi + lo stays below 1e-5."""
    S = synth.QWEN3_30B_A3B_MXFP4
    src = oracle.ExpertSource(S)
    xb = synth.x_bf16(S, 50, 4, T=2)
    ref = oracle.moe_layer(src, 0, xb)
    m = np.abs(ref["y"]).max()
    def err(hm, xm):
        y, _ = oracle.emulate_moe_layer(src, 0, xb, oracle.W_EXACT_CODES, hm, xm)
        return np.abs(y - ref["y"]).max() / m
    assert err(oracle.H_FP32, oracle.X_FP8_HILO) < 1e-5
    assert 3e-4 <= err(oracle.H_FP8_HILO, oracle.X_FP8_HILO) <= 1.5e-3
    assert err(oracle.H_BF16_HILO, oracle.X_FP8_HILO) < 1e-5

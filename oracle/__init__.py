"""CPU oracle for the quantized MoE expert FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The GPU library shares no code with it.

The arithmetic lives in ``oracle.c`` (plain scalar C, fp64); this module only
marshals numpy arrays and composes the per-token steps in the pages' order:
router logits -> exact top-k -> softmax over the selected experts -> per
selected expert SiLU(gate)*up -> down -> routing-weighted sum (sparkinfer
README, kernel table and MoE row; sparkinfer CuTe-DSL README, "moe"
paragraph). Expert weights come from the shared seeded generator ``synth``
(encoded blocks only); the oracle decodes them itself.

Two expert weight encodings are decoded: 144-byte 4-bit super-blocks (256
weights) and 17-byte MXFP4 blocks (32 weights: an E8M0 scale byte and 16 bytes
of FP4 E2M1 codes). Functions taking blocks tell them apart by the last
dimension (144 or 17 bytes).

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (worked block examples, exhaustive 6-bit field
sweep, fp16 table, the library's E8M0 and E4M3 decoders for the MXFP4 scale
and codes, library matmul, brute-force top-k, closed forms). One thing stays
parity unpinned: the block encodings are our readings (the pages print no
bit layout for either), so byte compatibility with any external file is not
claimed.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

QK = 256
QBLOCK_BYTES = 144
MXK = 32
MXBLOCK_BYTES = 17
FMT_Q4K, FMT_MXFP4 = 0, 1
RMS_EPS = 1e-6


def build_lib(force=True):
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_lib()
        L = ctypes.CDLL(_LIB)
        vp, i64, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        L.oracle_f16.restype = f64
        L.oracle_f16.argtypes = [ctypes.c_uint16]
        L.oracle_bf16.restype = f64
        L.oracle_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16.argtypes = [f64]
        L.oracle_dequant_block.restype = None
        L.oracle_dequant_block.argtypes = [vp, vp]
        L.oracle_dequant_matrix.restype = None
        L.oracle_dequant_matrix.argtypes = [vp, i64, i64, vp]
        L.oracle_qgemv.restype = None
        L.oracle_qgemv.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_fp4.restype = f64
        L.oracle_fp4.argtypes = [ctypes.c_int32]
        L.oracle_e8m0.restype = f64
        L.oracle_e8m0.argtypes = [ctypes.c_int32]
        L.oracle_dequant_mx_block.restype = None
        L.oracle_dequant_mx_block.argtypes = [vp, vp]
        L.oracle_dequant_mx_matrix.restype = None
        L.oracle_dequant_mx_matrix.argtypes = [vp, i64, i64, vp]
        L.oracle_qgemv_fmt.restype = None
        L.oracle_qgemv_fmt.argtypes = [vp, i64, i64, vp, vp, ctypes.c_int32]
        L.oracle_expert_ffn_fmt.restype = None
        L.oracle_expert_ffn_fmt.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, ctypes.c_int32, ctypes.c_int32]
        L.oracle_moe_token_fmt.restype = None
        L.oracle_moe_token_fmt.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, ctypes.c_int32, ctypes.c_int32]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [vp, i64, i64, vp, vp]
        L.oracle_topk.restype = None
        L.oracle_topk.argtypes = [vp, i64, i64, vp]
        L.oracle_route_weights.restype = None
        L.oracle_route_weights.argtypes = [vp, vp, i64, vp]
        L.oracle_silu.restype = f64
        L.oracle_silu.argtypes = [f64]
        L.oracle_act.restype = f64
        L.oracle_act.argtypes = [f64, f64, ctypes.c_int32]
        L.oracle_expert_ffn.restype = None
        L.oracle_expert_ffn.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp]
        L.oracle_expert_ffn_act.restype = None
        L.oracle_expert_ffn_act.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, ctypes.c_int32]
        L.oracle_moe_token.restype = None
        L.oracle_moe_token.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp]
        L.oracle_moe_token_act.restype = None
        L.oracle_moe_token_act.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, ctypes.c_int32]
        L.oracle_resid_rmsnorm.restype = None
        L.oracle_resid_rmsnorm.argtypes = [vp, vp, i64, f64, vp, vp]
        for fn in (L.oracle_emul_bf16, L.oracle_emul_fp16, L.oracle_emul_fp16_rtz, L.oracle_emul_e4m3):
            fn.restype = f64
            fn.argtypes = [f64]
        L.oracle_emul_fp8_hilo.restype = None
        L.oracle_emul_fp8_hilo.argtypes = [vp, i64]
        L.oracle_emul_moe_token.restype = None
        L.oracle_emul_moe_token.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp] + [ctypes.c_int32] * 5
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- numbers
def f16(h):
    return lib().oracle_f16(int(h))


def bf16(b):
    return lib().oracle_bf16(int(b))


def bf16_array(bits):
    """bf16 bit patterns -> fp64 values (a bf16 is the top half of an fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v):
    return lib().oracle_round_bf16(float(v))


# ---------------------------------------------------------------- dequant / GEMV
def block_format(blocks):
    """(fmt, weights per block) from the block byte count (144 or 17)."""
    nbytes = np.shape(blocks)[-1]
    if nbytes == QBLOCK_BYTES:
        return FMT_Q4K, QK
    if nbytes == MXBLOCK_BYTES:
        return FMT_MXFP4, MXK
    raise ValueError(f"no block encoding of {nbytes} bytes")


def fp4(code):
    """FP4 E2M1 code -> value."""
    return lib().oracle_fp4(int(code))


def e8m0(e):
    """E8M0 scale code -> 2^(e-127) (NaN for 255)."""
    return lib().oracle_e8m0(int(e))


def dequant_mx_block(blk):
    blk = _c(blk, np.uint8).reshape(MXBLOCK_BYTES)
    w = np.empty(MXK, dtype=np.float64)
    lib().oracle_dequant_mx_block(_p(blk), _p(w))
    return w


def dequant_block(blk):
    blk = _c(blk, np.uint8).reshape(QBLOCK_BYTES)
    w = np.empty(QK, dtype=np.float64)
    lib().oracle_dequant_block(_p(blk), _p(w))
    return w


def dequant_matrix(blocks):
    """[rows, cols/K, bytes] uint8 (either encoding) -> fp64 [rows, cols]."""
    blocks = _c(blocks, np.uint8)
    fmt, K = block_format(blocks)
    rows, nb = blocks.shape[0], blocks.shape[1]
    w = np.empty((rows, nb * K), dtype=np.float64)
    fn = lib().oracle_dequant_mx_matrix if fmt == FMT_MXFP4 else lib().oracle_dequant_matrix
    fn(_p(blocks), rows, nb * K, _p(w))
    return w


def qgemv(blocks, x):
    blocks = _c(blocks, np.uint8)
    fmt, K = block_format(blocks)
    rows, nb = blocks.shape[0], blocks.shape[1]
    x = _c(x, np.float64)
    assert x.shape == (nb * K,)
    y = np.empty(rows, dtype=np.float64)
    lib().oracle_qgemv_fmt(_p(blocks), rows, nb * K, _p(x), _p(y), fmt)
    return y


# ---------------------------------------------------------------- routing
def router_logits(wr, x_bf16):
    wr = _c(wr, np.float32)
    x_bf16 = _c(x_bf16, np.uint16)
    E, H = wr.shape
    assert x_bf16.shape == (H,)
    out = np.empty(E, dtype=np.float64)
    lib().oracle_router_logits(_p(wr), E, H, _p(x_bf16), _p(out))
    return out


def topk(logits, k):
    logits = _c(logits, np.float64)
    ids = np.empty(k, dtype=np.int32)
    lib().oracle_topk(_p(logits), logits.size, k, _p(ids))
    return ids


def route_weights(logits, ids):
    logits = _c(logits, np.float64)
    ids = _c(ids, np.int32)
    w = np.empty(ids.size, dtype=np.float64)
    lib().oracle_route_weights(_p(logits), _p(ids), ids.size, _p(w))
    return w


def selection_margin(logits, k):
    """Margin of the top-k selection: the k-th largest logit minus the
    (k+1)-th largest (0 when they are equal, so that the selection depends on
    the tie rule; inf when k equals the number of experts, where every
    selection is the same set)."""
    srt = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    return srt[k - 1] - srt[k] if k < srt.size else np.inf


def route(logits, k):
    """(ids, weights, gap) for one token. ``gap`` = l_(k) - l_(k+1), the
    margin of the selection (inf when k == E)."""
    ids = topk(logits, k)
    w = route_weights(logits, ids)
    return ids, w, selection_margin(logits, k)


def silu(z):
    return lib().oracle_silu(float(z))


# Gate activations h = act(g, u); the pages (sparkinfer CuTe-DSL README, "moe"
# paragraph) name SiLU, ReLU2 and SwiGLU-OAI without formulas: SiLU(g) u,
# max(g, 0)^2 u, and g' sigmoid(1.702 g') (u' + 1) with g' = min(g, 7),
# u' = clamp(u, -7, 7).
ACT_SILU, ACT_RELU2, ACT_SWIGLU_OAI = 0, 1, 2


def act(g, u, kind=ACT_SILU):
    return lib().oracle_act(float(g), float(u), int(kind))


# ---------------------------------------------------------------- FFN
def expert_ffn(gate, up, down, x, return_h=False, act=ACT_SILU):
    gate, up, down = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    fmt, K = block_format(gate)
    I, H = gate.shape[0], gate.shape[1] * K
    assert up.shape == gate.shape and down.shape[0] == H and down.shape[1] * K == I
    assert block_format(down)[0] == fmt
    x = _c(x, np.float64)
    y = np.empty(H, dtype=np.float64)
    h = np.empty(I, dtype=np.float64)
    lib().oracle_expert_ffn_fmt(_p(gate), _p(up), _p(down), H, I, _p(x), _p(y), _p(h), int(act), fmt)
    return (y, h) if return_h else y


def moe_token(gates, ups, downs, w, x_bf16, act=ACT_SILU):
    """y = sum_s w_s * FFN_s(x) for one token; gates[s] etc. are the blocks
    of the expert in slot s."""
    k = len(gates)
    gates = [_c(g, np.uint8) for g in gates]
    ups = [_c(u, np.uint8) for u in ups]
    downs = [_c(d, np.uint8) for d in downs]
    fmt, K = block_format(gates[0])
    I, H = gates[0].shape[0], gates[0].shape[1] * K
    PA = ctypes.c_void_p * k
    ga = PA(*[g.ctypes.data for g in gates])
    ua = PA(*[u.ctypes.data for u in ups])
    da = PA(*[d.ctypes.data for d in downs])
    w = _c(w, np.float64)
    x_bf16 = _c(x_bf16, np.uint16)
    y = np.empty(H, dtype=np.float64)
    lib().oracle_moe_token_fmt(ga, ua, da, _p(w), k, H, I, _p(x_bf16), _p(y), int(act), fmt)
    return y


def resid_rmsnorm(x_bf16, y, eps=RMS_EPS):
    """(r fp64, r rounded to bf16 bits) for r = RMSNorm(x + y), weight 1."""
    x_bf16 = _c(x_bf16, np.uint16)
    y = _c(y, np.float64)
    n = x_bf16.size
    r = np.empty(n, dtype=np.float64)
    rb = np.empty(n, dtype=np.uint16)
    lib().oracle_resid_rmsnorm(_p(x_bf16), _p(y), n, eps, _p(r), _p(rb))
    return r, rb


# ---------------------------------------------------------------- composed
class ExpertSource:
    """Encoded expert blocks of one shape, drawn from the shared generator on
    demand (only the experts a token selects) and cached per layer."""

    def __init__(self, shape, max_cached=512):
        import synth
        self._synth = synth
        self.shape = shape
        self._cache = {}
        self._max = max_cached

    def blocks(self, layer, expert):
        key = (layer, int(expert))
        if key not in self._cache:
            if len(self._cache) >= self._max:
                self._cache.pop(next(iter(self._cache)))
            s = self._synth
            self._cache[key] = tuple(s.expert_matrix(self.shape, layer, int(expert), m) for m in (s.GATE, s.UP, s.DOWN))
        return self._cache[key]

    def router(self, layer):
        return self._synth.router(self.shape, layer)


def moe_layer(src, layer, x_bf16, logits=None, wr=None, act=ACT_SILU):
    """One MoE layer for T tokens. x_bf16: [T, H] bf16 bits. ``logits`` (fp32
    [T, E]) replaces the router GEMV when given; ``act`` is the gate
    activation. Returns dict with ids [T,k], w [T,k], gap [T], logits [T,E]
    (fp64), y [T,H] (fp64)."""
    S = src.shape
    x_bf16 = np.atleast_2d(np.asarray(x_bf16, dtype=np.uint16))
    T = x_bf16.shape[0]
    if logits is None:
        wr = src.router(layer) if wr is None else wr
        lg = np.stack([router_logits(wr, x_bf16[t]) for t in range(T)]) if T else np.zeros((0, S.n_experts))
    else:
        lg = np.asarray(logits, dtype=np.float32).astype(np.float64).reshape(T, S.n_experts)
    ids = np.zeros((T, S.top_k), dtype=np.int32)
    w = np.zeros((T, S.top_k), dtype=np.float64)
    gap = np.zeros(T, dtype=np.float64)
    y = np.zeros((T, S.hidden), dtype=np.float64)
    for t in range(T):
        ids[t], w[t], gap[t] = route(lg[t], S.top_k)
        bl = [src.blocks(layer, e) for e in ids[t]]
        y[t] = moe_token([b[0] for b in bl], [b[1] for b in bl], [b[2] for b in bl], w[t], x_bf16[t], act=act)
    return dict(ids=ids, w=w, gap=gap, logits=lg, y=y)


# ---------------------------------------------------------------- recipe emulation
# Weight, h and activation modes of the recipe emulation (see oracle.c): it
# predicts a GPU arithmetic recipe's error; parity checks never use it.
W_EXACT_CODES, W_BF16, W_FP16, W_BF16_HILO = 0, 1, 2, 3
H_FP32, H_BF16, H_FP16, H_BF16_HILO, H_FP8_HILO = 0, 1, 2, 3, 4
X_BF16, X_FP16_RTZ, X_FP8_HILO = 0, 1, 2


def emul_bf16(v):
    return lib().oracle_emul_bf16(float(v))


def emul_fp16(v):
    return lib().oracle_emul_fp16(float(v))


def emul_fp16_rtz(v):
    return lib().oracle_emul_fp16_rtz(float(v))


def emul_e4m3(v):
    return lib().oracle_emul_e4m3(float(v))


def emul_fp8_hilo(v):
    """v (fp32, length a multiple of 32) as FP8 E4M3 hi + lo operands with
    per-32 power-of-two scales (the recipe emulation's hmode 4 / xmode 2)."""
    out = np.array(v, dtype=np.float32, copy=True)
    assert out.ndim == 1 and out.size % 32 == 0
    lib().oracle_emul_fp8_hilo(_p(out), out.size)
    return out


def emulate_moe_token(gates, ups, downs, w, x_bf16, wmode, hmode, xmode=X_BF16, act=ACT_SILU):
    """One token through its selected experts with a recipe's roundings (fp32
    result as fp64)."""
    k = len(gates)
    gates = [_c(g, np.uint8) for g in gates]
    ups = [_c(u, np.uint8) for u in ups]
    downs = [_c(d, np.uint8) for d in downs]
    fmt, K = block_format(gates[0])
    I, H = gates[0].shape[0], gates[0].shape[1] * K
    PA = ctypes.c_void_p * k
    ga = PA(*[g.ctypes.data for g in gates])
    ua = PA(*[u.ctypes.data for u in ups])
    da = PA(*[d.ctypes.data for d in downs])
    w = _c(w, np.float64)
    x_bf16 = _c(x_bf16, np.uint16)
    y = np.empty(H, dtype=np.float64)
    lib().oracle_emul_moe_token(ga, ua, da, _p(w), k, H, I, _p(x_bf16), _p(y), int(act), fmt, int(wmode), int(hmode),
                                int(xmode))
    return y


def emulate_moe_layer(src, layer, x_bf16, wmode, hmode, xmode=X_BF16, logits=None, act=ACT_SILU):
    """moe_layer with the expert FFNs under a recipe; routing is the exact
    oracle's. Returns (emulated y [T, H], exact oracle result dict)."""
    ref = moe_layer(src, layer, x_bf16, logits=logits, act=act)
    x_bf16 = np.atleast_2d(np.asarray(x_bf16, dtype=np.uint16))
    y = np.zeros_like(ref["y"])
    for t in range(x_bf16.shape[0]):
        bl = [src.blocks(layer, e) for e in ref["ids"][t]]
        y[t] = emulate_moe_token([b[0] for b in bl], [b[1] for b in bl], [b[2] for b in bl], ref["w"][t],
                                 x_bf16[t], wmode, hmode, xmode, act)
    return y, ref

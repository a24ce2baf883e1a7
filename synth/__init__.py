"""Seeded synthetic workloads for the quantized MoE expert FFN.

The only module both the GPU library's callers and the CPU oracle draw inputs
from. It holds no step of the MoE computation: it makes Gaussian weights,
activations and logits from counter-based streams and encodes expert weights
into canonical 144-byte 4-bit super-blocks or 17-byte MXFP4 blocks (see
``synth.c`` for the layouts and the quantizers; a shape's ``fmt`` picks one).
Both sides decode those blocks with their own code.

Shapes follow the pages' model: a Qwen3-30B-A3B-shaped MoE layer (hidden 2048,
128 experts, top-8, expert intermediate 768) kept quantized-resident, and a
tiny layer (hidden 256, 8 experts, top-2, intermediate 512) for fast checks.
Weights are N(0, 0.02), router weights fp32 N(0, 0.02), activations bf16
N(0, 1), router logits (for the batched cases) fp32 N(0, 1), optionally biased
by a Zipf(s=1.1) per-expert offset.
"""
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

QK = 256
QBLOCK_BYTES = 144
MXK = 32
MXBLOCK_BYTES = 17
WEIGHT_SIGMA = 0.02

# expert weight encodings
FMT_Q4K, FMT_MXFP4 = 0, 1

# stream kinds (second key component)
_K_EXPERT, _K_ROUTER, _K_X, _K_LOGITS, _K_PERM = 0, 1, 2, 3, 4
# matrix ids inside an expert
GATE, UP, DOWN = 0, 1, 2


def build_lib(force=True):
    """Compile libsynth.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
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
        u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
        vp = ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [i64] * 5
        L.synth_normal_f32.restype = None
        L.synth_normal_f32.argtypes = [u64, u64, u64, f32, vp]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_f64_to_f16.argtypes = [ctypes.c_double]
        L.synth_f32_to_bf16.restype = None
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        L.synth_quantize_block.restype = None
        L.synth_quantize_block.argtypes = [vp, vp]
        L.synth_quantize_rows.restype = None
        L.synth_quantize_rows.argtypes = [vp, i64, i64, vp]
        L.synth_q4k_matrix.restype = None
        L.synth_q4k_matrix.argtypes = [u64, i64, i64, f32, vp, ctypes.c_int]
        L.synth_q4k_matrices.restype = None
        L.synth_q4k_matrices.argtypes = [vp, i64, i64, i64, f32, vp, ctypes.c_int]
        L.synth_quantize_mx_block.restype = None
        L.synth_quantize_mx_block.argtypes = [vp, vp]
        L.synth_quantize_mx_rows.restype = None
        L.synth_quantize_mx_rows.argtypes = [vp, i64, i64, vp]
        L.synth_mx_matrices.restype = None
        L.synth_mx_matrices.argtypes = [vp, i64, i64, i64, f32, vp, ctypes.c_int]
        L.synth_philox4x32_10.restype = None
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclass(frozen=True)
class Shape:
    """One MoE layer shape. ``model`` seeds the weight streams; ``fmt``
    picks the expert weight encoding (the same Gaussian weights either way)."""
    name: str
    model: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    fmt: int = FMT_Q4K

    @property
    def block(self):
        """(weights per block, bytes per block) of the encoding."""
        return (MXK, MXBLOCK_BYTES) if self.fmt == FMT_MXFP4 else (QK, QBLOCK_BYTES)

    @property
    def expert_bytes(self):
        """Bytes of one expert's three encoded matrices (gate, up, down)."""
        K, B = self.block
        return 3 * self.inter * self.hidden // K * B


TINY = Shape("tiny", 1, 256, 8, 2, 512)
QWEN3_30B_A3B = Shape("qwen3-30b-a3b-moe", 2, 2048, 128, 8, 768)
# the same layer (same Gaussian weights) with MXFP4 expert weights
QWEN3_30B_A3B_MXFP4 = Shape("qwen3-30b-a3b-moe-mxfp4", 2, 2048, 128, 8, 768, FMT_MXFP4)


# ---------------------------------------------------------------- primitives
def key(*ids):
    ids = list(ids) + [0] * (5 - len(ids))
    return lib().synth_key(*[int(v) for v in ids])


def normal_f32(k, n, scale=1.0, start=0):
    out = np.empty(n, dtype=np.float32)
    if n:
        lib().synth_normal_f32(k, start, n, scale, _ptr(out))
    return out


def f32_to_bf16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_rows(w, fmt=FMT_Q4K):
    """Encode float32 [rows, cols] into canonical blocks: [rows, cols/256, 144]
    uint8 super-blocks, or [rows, cols/32, 17] MXFP4 blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    if fmt == FMT_MXFP4:
        assert cols % MXK == 0
        out = np.empty((rows, cols // MXK, MXBLOCK_BYTES), dtype=np.uint8)
        lib().synth_quantize_mx_rows(_ptr(w), rows, cols, _ptr(out))
        return out
    assert cols % QK == 0
    out = np.empty((rows, cols // QK, QBLOCK_BYTES), dtype=np.uint8)
    lib().synth_quantize_rows(_ptr(w), rows, cols, _ptr(out))
    return out


# ---------------------------------------------------------------- weights
def expert_matrix_shape(shape, mat):
    return (shape.inter, shape.hidden) if mat in (GATE, UP) else (shape.hidden, shape.inter)


def expert_matrix(shape, layer, expert, mat, nthreads=0):
    """Canonical blocks of one expert matrix: [rows, cols/K, bytes] uint8 in
    the shape's encoding."""
    if shape.fmt == FMT_MXFP4:
        return layer_experts(shape, layer, mat, [expert], nthreads)[0]
    rows, cols = expert_matrix_shape(shape, mat)
    out = np.empty((rows, cols // QK, QBLOCK_BYTES), dtype=np.uint8)
    k = key(shape.model, _K_EXPERT, layer, expert, mat)
    lib().synth_q4k_matrix(k, rows, cols, WEIGHT_SIGMA, _ptr(out), nthreads)
    return out


def expert_matrix_f32(shape, layer, expert, mat):
    """The unquantized N(0, 0.02) weights behind ``expert_matrix``."""
    rows, cols = expert_matrix_shape(shape, mat)
    k = key(shape.model, _K_EXPERT, layer, expert, mat)
    return normal_f32(k, rows * cols, WEIGHT_SIGMA).reshape(rows, cols)


def layer_experts(shape, layer, mat, experts=None, nthreads=0):
    """Canonical blocks of one matrix kind for many experts of a layer:
    [n, rows, cols/K, bytes] uint8 (all experts when ``experts`` is None)."""
    if experts is None:
        experts = range(shape.n_experts)
    experts = list(experts)
    rows, cols = expert_matrix_shape(shape, mat)
    K, B = shape.block
    keys = np.array([key(shape.model, _K_EXPERT, layer, e, mat) for e in experts], dtype=np.uint64)
    out = np.empty((len(experts), rows, cols // K, B), dtype=np.uint8)
    if len(experts):
        gen = lib().synth_mx_matrices if shape.fmt == FMT_MXFP4 else lib().synth_q4k_matrices
        gen(_ptr(keys), len(experts), rows, cols, WEIGHT_SIGMA, _ptr(out), nthreads)
    return out


def router(shape, layer):
    """Router weights, fp32 [n_experts, hidden], N(0, 0.02)."""
    k = key(shape.model, _K_ROUTER, layer)
    return normal_f32(k, shape.n_experts * shape.hidden, WEIGHT_SIGMA).reshape(shape.n_experts, shape.hidden)


# ---------------------------------------------------------------- activations
def x_bf16(shape, case, step, T=1):
    """Activations, bf16 bits [T, hidden], N(0, 1) rounded to nearest even."""
    k = key(shape.model, _K_X, case, step)
    return f32_to_bf16_bits(normal_f32(k, T * shape.hidden)).reshape(T, shape.hidden)


def logits_f32(shape, case, T, zipf_s=None):
    """Router logits fp32 [T, n_experts], N(0, 1). With ``zipf_s`` each expert
    e gets the offset -s*ln(rank_e), rank_e = perm(e)+1 for a seeded
    permutation (the log of a Zipf pmf up to a constant); the sum is formed in
    fp64 and rounded once to fp32."""
    E = shape.n_experts
    k = key(shape.model, _K_LOGITS, case, T)
    z = normal_f32(k, T * E).reshape(T, E)
    if zipf_s is None:
        return z
    return (z.astype(np.float64) + zipf_offsets(shape, case, zipf_s)[None, :]).astype(np.float32)


def zipf_offsets(shape, case, s):
    E = shape.n_experts
    # seeded permutation: rank experts by Philox draws (ties broken by id)
    kp = key(shape.model, _K_PERM, case)
    draws = np.empty(E, dtype=np.uint64)
    ctr = np.zeros(4, dtype=np.uint32)
    kk = np.array([kp & 0xFFFFFFFF, kp >> 32], dtype=np.uint32)
    outw = np.zeros(4, dtype=np.uint32)
    for e in range(E):
        ctr[0] = e
        lib().synth_philox4x32_10(_ptr(ctr), _ptr(kk), _ptr(outw))
        draws[e] = (int(outw[0]) << 32) | int(outw[1])
    order = np.lexsort((np.arange(E), draws))      # experts sorted by draw
    rank = np.empty(E, dtype=np.int64)
    rank[order] = np.arange(1, E + 1)
    return -float(s) * np.log(rank.astype(np.float64))

"""Python binding of the gfx950 quantized MoE expert FFN library (libqmoe.so).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory and the stream. The functions mirror
the C ABI declared in ``include/moe.h`` (same names without the ``moe_``
prefix) and raise ``MoeError`` on a non-zero status.
"""
import ctypes
import os

import numpy as np

__all__ = [
    "MoeError", "Config", "RouteOut", "Plan", "load", "is_supported", "status_string",
    "FLAG_FORCE_GEMV", "FLAG_FORCE_GROUPED", "FLAG_FORCE_EXPERT_GEMV", "FLAG_ACT_RELU2", "FLAG_ACT_SWIGLU_OAI",
    "FLAG_WEIGHTS_MXFP4",
    "LIB_PATH",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

FLAG_FORCE_GEMV = 0x1
FLAG_FORCE_GROUPED = 0x2
FLAG_FORCE_EXPERT_GEMV = 0x4
FLAG_ACT_RELU2 = 0x8            # gate activation max(g, 0)^2 * u
FLAG_ACT_SWIGLU_OAI = 0x10      # clamped SwiGLU (see include/moe.h)
FLAG_WEIGHTS_MXFP4 = 0x20       # MXFP4 expert blocks (17 bytes per 32 weights) instead of 4-bit super-blocks

# Every symbol include/moe.h declares.
EXPORTS = [
    "moe_is_supported", "moe_plan_create", "moe_plan_destroy", "moe_blob_bytes", "moe_header_bytes",
    "moe_layer_bytes", "moe_layer_offset", "moe_scratch_bytes", "moe_pack_header", "moe_pack_layer",
    "moe_unpack_layer", "moe_blob_check", "moe_route", "moe_expert_ffn", "moe_forward", "moe_stack_step",
    "moe_graph_capture_step", "moe_graph_launch", "moe_graph_destroy", "moe_profile_gate_up", "moe_status_string",
    "moe_forward_static_scratch",
]
STATIC_SCRATCH_BYTES = 16 << 20   # MOE_STATIC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("rms_eps", ctypes.c_float),
    ]


class RouteOut(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("pairs", ctypes.c_void_p)]


_lib = None


def load():
    """Load libqmoe.so into the process. torch is imported first so the
    library binds to the same HIP runtime as torch's tensors and streams."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (HIP runtime of the process)
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run quantized_moe_decode_gemv_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, u8p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    P = ctypes.c_void_p
    L.moe_is_supported.restype = ctypes.c_int
    L.moe_is_supported.argtypes = [ctypes.POINTER(Config)]
    L.moe_plan_create.restype = ctypes.c_int
    L.moe_plan_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P)]
    L.moe_plan_destroy.restype = None
    L.moe_plan_destroy.argtypes = [P]
    for f in ("moe_blob_bytes", "moe_header_bytes", "moe_layer_bytes"):
        getattr(L, f).restype = sz
        getattr(L, f).argtypes = [P]
    L.moe_layer_offset.restype = sz
    L.moe_layer_offset.argtypes = [P, i32]
    L.moe_scratch_bytes.restype = sz
    L.moe_scratch_bytes.argtypes = [P, i32]
    L.moe_pack_header.restype = ctypes.c_int
    L.moe_pack_header.argtypes = [P, vp]
    L.moe_pack_layer.restype = ctypes.c_int
    L.moe_pack_layer.argtypes = [P, u8p, u8p, u8p, vp, vp]
    L.moe_unpack_layer.restype = ctypes.c_int
    L.moe_unpack_layer.argtypes = [P, vp, u8p, u8p, u8p, vp]
    L.moe_blob_check.restype = ctypes.c_int
    L.moe_blob_check.argtypes = [P, vp]
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [P, vp, i32, vp, vp, i32, ctypes.POINTER(RouteOut), vp, sz, vp]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_expert_ffn.argtypes = [P, vp, i32, vp, i32, ctypes.POINTER(RouteOut), vp, vp, sz, vp]
    L.moe_forward.restype = ctypes.c_int
    L.moe_forward.argtypes = [P, vp, i32, vp, i32, vp, vp, ctypes.POINTER(RouteOut), vp, sz, vp]
    L.moe_forward_static_scratch.restype = ctypes.c_int
    L.moe_forward_static_scratch.argtypes = [P, vp, i32, vp, i32, vp, vp, ctypes.POINTER(RouteOut), vp]
    L.moe_stack_step.restype = ctypes.c_int
    L.moe_stack_step.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.moe_graph_capture_step.restype = ctypes.c_int
    L.moe_graph_capture_step.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, sz, vp, ctypes.POINTER(P)]
    L.moe_graph_launch.restype = ctypes.c_int
    L.moe_graph_launch.argtypes = [P, vp]
    L.moe_graph_destroy.restype = None
    L.moe_graph_destroy.argtypes = [P]
    L.moe_profile_gate_up.restype = ctypes.c_int
    L.moe_profile_gate_up.argtypes = [P, vp, i32, vp, i32, vp, sz, vp, vp, vp]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [ctypes.c_int]
    _lib = L
    return L


def status_string(status):
    return load().moe_status_string(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise MoeError(status, where)


def is_supported(cfg):
    return bool(load().moe_is_supported(ctypes.byref(cfg)))


def _np_ptr(a):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _dptr(t):
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Plan:
    """Immutable plan for one configuration (host object)."""

    def __init__(self, hidden, n_experts, top_k, inter, n_layers=1, max_tokens=1, flags=0, rms_eps=1e-6):
        self.cfg = Config(hidden, n_experts, top_k, inter, n_layers, max_tokens, flags, rms_eps)
        L = load()
        h = ctypes.c_void_p()
        _check(L.moe_plan_create(ctypes.byref(self.cfg), ctypes.byref(h)), "moe_plan_create")
        self._h = h
        self.hidden, self.n_experts, self.top_k, self.inter = hidden, n_experts, top_k, inter
        self.n_layers, self.max_tokens = n_layers, max_tokens
        # canonical block of the expert weights: (weights, bytes)
        self.block = (32, 17) if flags & FLAG_WEIGHTS_MXFP4 else (256, 144)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.moe_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    # ---- sizes
    def blob_bytes(self):
        return load().moe_blob_bytes(self._h)

    def header_bytes(self):
        return load().moe_header_bytes(self._h)

    def layer_bytes(self):
        return load().moe_layer_bytes(self._h)

    def layer_offset(self, layer):
        return load().moe_layer_offset(self._h, layer)

    def scratch_bytes(self, T):
        return load().moe_scratch_bytes(self._h, T)

    # ---- host packing
    def pack_header(self):
        out = np.zeros(self.header_bytes(), dtype=np.uint8)
        _check(load().moe_pack_header(self._h, _np_ptr(out)), "moe_pack_header")
        return out

    def pack_layer(self, gate, up, down, router, out=None):
        E, H, I = self.n_experts, self.hidden, self.inter
        gate = np.ascontiguousarray(gate, dtype=np.uint8)
        up = np.ascontiguousarray(up, dtype=np.uint8)
        down = np.ascontiguousarray(down, dtype=np.uint8)
        router = np.ascontiguousarray(router, dtype=np.float32)
        K, B = self.block
        assert gate.size == E * I * H // K * B and up.size == gate.size and down.size == gate.size
        assert router.shape == (E, H)
        if out is None:
            out = np.empty(self.layer_bytes(), dtype=np.uint8)
        assert out.size >= self.layer_bytes()
        _check(load().moe_pack_layer(self._h, _np_ptr(gate), _np_ptr(up), _np_ptr(down), _np_ptr(router),
                                     _np_ptr(out)), "moe_pack_layer")
        return out

    def unpack_layer(self, packed):
        E, H, I = self.n_experts, self.hidden, self.inter
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        K, B = self.block
        gate = np.empty((E, I, H // K, B), dtype=np.uint8)
        up = np.empty_like(gate)
        down = np.empty((E, H, I // K, B), dtype=np.uint8)
        router = np.empty((E, H), dtype=np.float32)
        _check(load().moe_unpack_layer(self._h, _np_ptr(packed), _np_ptr(gate), _np_ptr(up), _np_ptr(down),
                                       _np_ptr(router)), "moe_unpack_layer")
        return gate, up, down, router

    def blob_check(self, header):
        header = np.ascontiguousarray(header, dtype=np.uint8)
        return load().moe_blob_check(self._h, _np_ptr(header))

    # ---- device calls
    def route(self, blob, layer, x, logits, T, ids, w, counts=None, offsets=None, pairs=None, scratch=None,
              stream=None):
        ro = RouteOut(_dptr(ids), _dptr(w), _dptr(counts), _dptr(offsets), _dptr(pairs))
        sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
        _check(load().moe_route(self._h, _dptr(blob), layer, _dptr(x), _dptr(logits), T, ctypes.byref(ro),
                                _dptr(scratch), sb, _stream(stream)), "moe_route")

    def expert_ffn(self, blob, layer, x, T, ids, w, out, counts=None, offsets=None, pairs=None, scratch=None,
                   stream=None):
        ro = RouteOut(_dptr(ids), _dptr(w), _dptr(counts), _dptr(offsets), _dptr(pairs))
        sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
        _check(load().moe_expert_ffn(self._h, _dptr(blob), layer, _dptr(x), T, ctypes.byref(ro), _dptr(out),
                                     _dptr(scratch), sb, _stream(stream)), "moe_expert_ffn")

    def forward(self, blob, layer, x, T, out, x_next=None, ids=None, w=None, scratch=None, stream=None,
                counts=None, offsets=None, pairs=None):
        ro = None
        if ids is not None or w is not None:
            ro = ctypes.byref(RouteOut(_dptr(ids), _dptr(w), _dptr(counts), _dptr(offsets), _dptr(pairs)))
        sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
        _check(load().moe_forward(self._h, _dptr(blob), layer, _dptr(x), T, _dptr(out), _dptr(x_next), ro,
                                  _dptr(scratch), sb, _stream(stream)), "moe_forward")

    def forward_static_scratch(self, blob, layer, x, T, out, x_next=None, ids=None, w=None, stream=None,
                               counts=None, offsets=None, pairs=None):
        """moe_forward on the library's own device workspace (no scratch
        argument; see moe_forward_static_scratch)."""
        ro = None
        if ids is not None or w is not None:
            ro = ctypes.byref(RouteOut(_dptr(ids), _dptr(w), _dptr(counts), _dptr(offsets), _dptr(pairs)))
        _check(load().moe_forward_static_scratch(self._h, _dptr(blob), layer, _dptr(x), T, _dptr(out), _dptr(x_next),
                                                 ro, _stream(stream)), "moe_forward_static_scratch")

    def profile_gate_up(self, blob, layer, x, T, start, stop, scratch=None, stream=None):
        """moe_forward's launches up to the gate/up GEMV kernel, whose
        execution is bracketed by torch.cuda.Event objects start/stop
        (created with enable_timing=True)."""
        sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
        _check(load().moe_profile_gate_up(self._h, _dptr(blob), layer, _dptr(x), T, _dptr(scratch), sb,
                                          ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event),
                                          _stream(stream)), "moe_profile_gate_up")

    def stack_step(self, blob, xs, ys, T=1, ids=None, w=None, scratch=None, stream=None):
        """One decode step through every layer (see moe_stack_step)."""
        sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
        _check(load().moe_stack_step(self._h, _dptr(blob), _dptr(xs), _dptr(ys), _dptr(ids), _dptr(w), T,
                                     _dptr(scratch), sb, _stream(stream)), "moe_stack_step")

    def capture_step(self, blob, xs, ys, T=1, ids=None, w=None, scratch=None, stream=None):
        """Capture one decode step as a hipGraph (returns a StepGraph)."""
        return StepGraph(self, blob, xs, ys, T, ids, w, scratch, stream)

    # ---- convenience
    def new_scratch(self, T=None, device="cuda"):
        import torch
        n = self.scratch_bytes(self.max_tokens if T is None else T)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def upload_blob(self, layer_source, device="cuda", blob=None, progress=None):
        """Pack every layer on the host and copy it into a device blob.
        ``layer_source(layer)`` returns canonical (gate, up, down, router);
        ``progress(layer)`` is called after each layer when given."""
        import torch
        if blob is None:
            blob = torch.empty(self.blob_bytes(), dtype=torch.uint8, device=device)
        blob[: self.header_bytes()].copy_(torch.from_numpy(self.pack_header()))
        staging = torch.empty(self.layer_bytes(), dtype=torch.uint8, pin_memory=True)
        host = staging.numpy()
        for layer in range(self.n_layers):
            self.pack_layer(*layer_source(layer), out=host)
            off = self.layer_offset(layer)
            blob[off:off + self.layer_bytes()].copy_(staging, non_blocking=False)
            if progress is not None:
                progress(layer)
        return blob


class StepGraph:
    """A captured decode step (moe_graph_capture_step); keeps its buffers alive."""

    def __init__(self, plan, blob, xs, ys, T, ids, w, scratch, stream):
        import torch
        if stream is None:
            raise ValueError("capture needs an explicit non-default stream")
        self._keep = (plan, blob, xs, ys, ids, w, scratch)
        sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
        h = ctypes.c_void_p()
        torch.cuda.synchronize()
        _check(load().moe_graph_capture_step(plan.handle, _dptr(blob), _dptr(xs), _dptr(ys), _dptr(ids), _dptr(w), T,
                                             _dptr(scratch), sb, _stream(stream), ctypes.byref(h)),
               "moe_graph_capture_step")
        self._h = h

    def launch(self, stream=None):
        _check(load().moe_graph_launch(self._h, _stream(stream)), "moe_graph_launch")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.moe_graph_destroy(h)
            self._h = None

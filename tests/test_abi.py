"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every symbol include/moe.h declares, configuration validation, size
queries, the packer's inverse, blob header checks and argument errors that
are caught before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
import quantized_moe_decode_gemv_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = q.load()
    declared = _declared_symbols()
    assert len(declared) >= 16
    assert sorted(q.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    assert q.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert q.status_string(s) != "unknown status"
    assert q.status_string(-99) == "unknown status"


@pytest.mark.parametrize("cfg,ok", [
    ((256, 8, 2, 512, 1, 1, 0, 1e-6), True),
    ((2048, 128, 8, 768, 48, 1, 0, 1e-6), True),
    ((4096, 64, 4, 1024, 1, 4096, 0, 1e-6), True),
    ((2048, 128, 8, 768, 1, 1, 3, 1e-6), False),    # two force flags
    ((2048, 128, 8, 768, 1, 1, 5, 1e-6), False),    # two force flags
    ((2048, 128, 8, 768, 1, 1, 6, 1e-6), False),    # two force flags
    ((2048, 128, 8, 768, 1, 1, 4, 1e-6), True),     # expert-major GEMV forced
    ((256, 8, 2, 2048, 1, 1, 4, 1e-6), True),       # expert-major GEMV: inter up to 2048
    ((256, 8, 2, 2304, 1, 1, 4, 1e-6), False),      # expert-major GEMV: inter above 2048
    ((256, 8, 2, 2304, 1, 1, 0, 1e-6), True),       # same shape without the flag
    ((2048, 128, 8, 768, 1, 1, 0x8, 1e-6), True),   # ReLU2 gate activation
    ((2048, 128, 8, 768, 1, 1, 0x10, 1e-6), True),  # SwiGLU-OAI gate activation
    ((2048, 128, 8, 768, 1, 1, 0x12, 1e-6), True),  # an activation and a forced path
    ((2048, 128, 8, 768, 1, 1, 0x18, 1e-6), False), # two activations
    ((2048, 128, 8, 768, 1, 1, 0x20, 1e-6), True),  # MXFP4 expert weights
    ((2048, 128, 8, 768, 1, 1, 0x29, 1e-6), True),  # MXFP4 with an activation and the per-token path forced
    ((2048, 128, 8, 768, 1, 1, 0x22, 1e-6), True),  # MXFP4 with the 16-pair MFMA tiles forced
    ((4096, 32, 4, 512, 1, 1, 0x22, 1e-6), False),  # ... which hidden 4096 does not have
    ((2048, 128, 8, 768, 1, 1, 0x24, 1e-6), True),  # MXFP4 with the expert-major GEMV forced
    ((256, 8, 2, 2304, 1, 1, 0x24, 1e-6), False),   # ... which needs inter <= 2048
    ((2048, 128, 8, 768, 1, 1, 0x40, 1e-6), False), # unknown flag
    ((2048, 128, 8, 768, 1, 1, 0x2, 1e-6), True),   # MFMA tiles forced
    ((4096, 32, 4, 512, 1, 1, 0x2, 1e-6), False),   # ... which hidden 4096 does not have
    ((2048, 128, 8, 768, 1, 131071, 0, 1e-6), True),   # T*k*max(H, I) just below 2^31
    ((2048, 128, 8, 768, 1, 131072, 0, 1e-6), False),  # ... and at 2^31 (32-bit device indexing)
    ((300, 8, 2, 512, 1, 1, 0, 1e-6), False),       # hidden not a multiple of 256
    ((768, 8, 2, 512, 1, 1, 0, 1e-6), False),       # hidden lane mapping unsupported
    ((256, 8, 9, 512, 1, 1, 0, 1e-6), False),       # k > E
    ((256, 8, 0, 512, 1, 1, 0, 1e-6), False),       # k = 0
    ((256, 300, 2, 512, 1, 1, 0, 1e-6), False),     # E > 256
    ((256, 8, 2, 500, 1, 1, 0, 1e-6), False),       # inter not a multiple of 256
    ((2048, 128, 16, 1024, 1, 1, 0, 1e-6), True),   # k*inter/32 = 512: eight waves per down row
    ((2048, 128, 16, 1280, 1, 1, 0, 1e-6), False),  # k*inter/32 > 512
    ((4096, 128, 8, 1536, 48, 1, 0, 1e-6), True),   # a Qwen3-235B-A22B-shaped stack
    ((4096, 128, 8, 1536, 1, 64, 0x4, 1e-6), True), # ... with the expert-major GEMV forced
    ((4096, 128, 8, 1536, 1, 64, 0x2, 1e-6), False),# ... but no MFMA tiles
    ((3072, 32, 4, 768, 2, 8, 0, 1e-6), True),      # hidden 3072 (32-lane groups, three sub-blocks each)
    ((3072, 32, 4, 768, 1, 8, 0x24, 1e-6), True),   # ... MXFP4 on the expert-major GEMV
    ((5120, 32, 4, 768, 1, 1, 0, 1e-6), False),     # hidden 5120: no lane mapping
    ((256, 8, 2, 512, 0, 1, 0, 1e-6), False),       # no layers
    ((256, 8, 2, 512, 1, 0, 0, 1e-6), False),       # max_tokens 0
    ((256, 8, 2, 512, 1, 1, 0, -1.0), False),       # negative eps
])
def test_is_supported(cfg, ok):
    assert q.is_supported(q.Config(*cfg)) == ok
    if not ok:
        with pytest.raises(q.MoeError) as e:
            q.Plan(*cfg[:4], n_layers=cfg[4], max_tokens=cfg[5], flags=cfg[6], rms_eps=cfg[7])
        assert e.value.status == -2


def test_sizes_qwen_stack():
    S = synth.QWEN3_30B_A3B
    p = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, n_layers=48, max_tokens=1)
    expert_bytes = 128 * S.expert_bytes
    router = 128 * 2048 * 4
    assert p.layer_bytes() == expert_bytes + router
    assert p.blob_bytes() == p.header_bytes() + 48 * p.layer_bytes()
    assert p.layer_offset(47) == p.header_bytes() + 47 * p.layer_bytes()
    assert p.layer_offset(48) == 0 and p.layer_offset(-1) == 0
    # 48 layers: 16,307,453,952 expert bytes resident
    assert 48 * expert_bytes == 16_307_453_952
    assert p.scratch_bytes(1) > 0 and p.scratch_bytes(2) == 0


def test_pack_unpack_identity():
    S = synth.Shape("pack", 20, 512, 4, 2, 256)
    p = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter)
    g = synth.layer_experts(S, 0, synth.GATE)
    u = synth.layer_experts(S, 0, synth.UP)
    d = synth.layer_experts(S, 0, synth.DOWN)
    r = synth.router(S, 0)
    packed = p.pack_layer(g, u, d, r)
    assert packed.size == p.layer_bytes()
    g2, u2, d2, r2 = p.unpack_layer(packed)
    assert np.array_equal(g2, g) and np.array_equal(u2, u) and np.array_equal(d2, d) and np.array_equal(r2, r)
    # the device layout is not the canonical one: codes are split from headers
    assert not np.array_equal(packed[p.layer_bytes() - d.size:], d.reshape(-1))


def test_sizes_qwen_mxfp4():
    """MXFP4 records: codes plus one scale byte per 32 weights, padded to 16
    bytes (gate/up row pair 2048 + 128 = 2176 B, down row 384 + 24 -> 416 B)."""
    S = synth.QWEN3_30B_A3B_MXFP4
    p = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, flags=q.FLAG_WEIGHTS_MXFP4)
    assert p.block == (32, 17)
    per_expert = 768 * 2176 + 2048 * 416
    assert p.layer_bytes() == 128 * per_expert + 128 * 2048 * 4
    # algorithmic bytes of one expert: 3 matrices x 1,572,864 weights x 4.25 bits
    assert S.expert_bytes == 3 * 768 * 2048 // 32 * 17 == 2_506_752


def test_pack_unpack_identity_mxfp4():
    S = synth.Shape("pack-mx", 20, 512, 4, 2, 256, synth.FMT_MXFP4)
    p = q.Plan(S.hidden, S.n_experts, S.top_k, S.inter, flags=q.FLAG_WEIGHTS_MXFP4)
    g = synth.layer_experts(S, 0, synth.GATE)
    u = synth.layer_experts(S, 0, synth.UP)
    d = synth.layer_experts(S, 0, synth.DOWN)
    r = synth.router(S, 0)
    assert g.shape == (4, 256, 16, 17) and d.shape == (4, 512, 8, 17)
    packed = p.pack_layer(g, u, d, r)
    g2, u2, d2, r2 = p.unpack_layer(packed)
    assert np.array_equal(g2, g) and np.array_equal(u2, u) and np.array_equal(d2, d) and np.array_equal(r2, r)
    # scale codes outside 2..252 are refused (2^-127 and 2^-126 would make
    # subnormal or flushed products, 2^126 and up overflow bf16, 255 is NaN)
    for bad in (0, 1, 253, 254, 255):
        d_bad = d.copy()
        d_bad[1, 7, 3, 0] = bad
        with pytest.raises(q.MoeError):
            p.pack_layer(g, u, d_bad, r)
        g_bad = g.copy()
        g_bad[2, 5, 0, 0] = bad
        with pytest.raises(q.MoeError):
            p.pack_layer(g_bad, u, d, r)


def test_blob_header_check():
    p = q.Plan(256, 8, 2, 512, n_layers=3)
    hdr = p.pack_header()
    assert p.blob_check(hdr) == 0
    bad = hdr.copy()
    bad[0] ^= 1
    assert p.blob_check(bad) == -3
    other = q.Plan(256, 8, 2, 512, n_layers=2)
    assert other.blob_check(hdr) == -3
    # a blob of the other weight encoding does not match
    mx = q.Plan(256, 8, 2, 512, n_layers=3, flags=q.FLAG_WEIGHTS_MXFP4)
    assert mx.blob_check(mx.pack_header()) == 0
    assert mx.blob_check(hdr) == -3 and p.blob_check(mx.pack_header()) == -3


def test_argument_errors_before_launch():
    """Invalid arguments are rejected on the host; nothing is launched, so
    these run without a GPU (fake non-null device pointers are never touched)."""
    L = q.load()
    p = q.Plan(256, 8, 2, 512, n_layers=1, max_tokens=4)
    fake = ctypes.c_void_p(1 << 20)          # 256-aligned, never dereferenced
    ro = q.RouteOut(fake, fake, None, None, None)
    out = fake
    # NULL plan / blob
    assert L.moe_forward(None, fake, 0, fake, 1, out, None, None, fake, 1 << 20, None) == -1
    assert L.moe_forward(p.handle, None, 0, fake, 1, out, None, None, fake, 1 << 20, None) == -1
    # layer / T out of range
    assert L.moe_forward(p.handle, fake, 1, fake, 1, out, None, None, fake, 1 << 20, None) == -1
    assert L.moe_forward(p.handle, fake, 0, fake, 5, out, None, None, fake, 1 << 20, None) == -1
    assert L.moe_forward(p.handle, fake, 0, fake, -1, out, None, None, fake, 1 << 20, None) == -1
    # scratch too small
    assert L.moe_forward(p.handle, fake, 0, fake, 1, out, None, None, fake, 16, None) == -4
    # misaligned blob
    assert L.moe_forward(p.handle, ctypes.c_void_p((1 << 20) + 16), 0, fake, 1, out, None, None, fake, 1 << 20,
                         None) == -1
    # route: incomplete dispatch list set
    ro2 = q.RouteOut(fake, fake, fake, None, None)
    assert L.moe_route(p.handle, fake, 0, fake, None, 1, ctypes.byref(ro2), fake, 1 << 20, None) == -1
    # expert_ffn without routing buffers
    assert L.moe_expert_ffn(p.handle, fake, 0, fake, 1, None, out, fake, 1 << 20, None) == -1
    # T == 0 is a no-op (scratch may be NULL)
    assert L.moe_forward(p.handle, fake, 0, fake, 0, out, None, None, None, 0, None) == 0
    assert L.moe_route(p.handle, fake, 0, fake, None, 0, ctypes.byref(ro), None, 0, None) == 0

"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355moe.h")
LIB = os.path.join(ROOT, "mxfp8_mxfp4_experts_amd", "libmi355moe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmi355moe.so not built")


def _header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+\**)+(moe_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    from mxfp8_mxfp4_experts_amd import _binding
    return _binding.load_library(LIB)


def test_header_declares_expected_calls():
    syms = _header_symbols()
    for name in ("moe_route", "moe_quant_mxfp8", "moe_permute", "moe_fc1_situ",
                 "moe_fc2_combine", "moe_workspace_size", "moe_strerror", "moe_abi_version"):
        assert name in syms


def test_library_exports_every_header_symbol(lib):
    from mxfp8_mxfp4_experts_amd._binding import EXPORTS
    raw = ctypes.CDLL(LIB)
    for name in _header_symbols():
        assert hasattr(raw, name), name
    assert set(_header_symbols()) == set(EXPORTS)


def test_version_and_strerror(lib):
    assert lib.moe_abi_version() == 3
    for code in (0, 1, 2, 3, 4, 5, 6, 7, 8):
        assert lib.moe_strerror(code)
    assert lib.moe_strerror(99) == b"unknown status"


def test_workspace_size(lib):
    n = lib.moe_workspace_size(8, 16, 896, 7168, 3584, 0)
    # tile prefix + restaged scale dwords [T*K, max(H, I)/32] + y rows [T*K, H] fp16
    # + their scale exponents [T*K, H/64]
    R = 8 * 16
    assert n >= R * (7168 // 32) + R * 7168 * 2 + R * (7168 // 64) and n % 256 == 0
    # atomic combine: the float [T, H] sums instead of the per-route rows
    na = lib.moe_workspace_size(8, 16, 896, 7168, 3584, 1)
    assert na >= R * (7168 // 32) + 8 * 7168 * 4 and na % 256 == 0 and na < n
    assert lib.moe_workspace_size(8, 16, 896, 7168, 3584, 2) == 0   # unknown mode
    assert lib.moe_workspace_size(8, 16, 896, 7000, 3584, 0) == 0   # H % 128
    assert lib.moe_workspace_size(8, 0, 896, 7168, 3584, 0) == 0    # top_k
    assert lib.moe_workspace_size(8, 16, 5000, 7168, 3584, 0) == 0  # E_local


FAKE = 1 << 20          # 16-byte aligned, never dereferenced by a failing call
MIS = FAKE + 2          # misaligned


def test_route_validation(lib):
    st = lib.moe_route
    assert st(FAKE, 4, FAKE, 5, 4, 0, 1.0, FAKE, FAKE, None) == 2          # top_k 0
    assert st(FAKE, 4, FAKE, 5, 4, 5, 1.0, FAKE, FAKE, None) == 2          # top_k > E
    assert st(FAKE, 3, FAKE, 5, 4, 2, 1.0, FAKE, FAKE, None) == 2          # ld < E
    assert st(FAKE, 5000, None, 5, 5000, 2, 1.0, FAKE, FAKE, None) == 2    # E > 4096
    assert st(None, 4, FAKE, 5, 4, 2, 1.0, FAKE, FAKE, None) == 1          # null logits
    assert st(FAKE, 4, FAKE, 5, 4, 2, 1.0, None, FAKE, None) == 1
    assert st(MIS, 4, FAKE, 5, 4, 2, 1.0, FAKE, FAKE, None) == 3
    assert st(None, 4, None, 0, 4, 2, 1.0, None, None, None) == 0          # T = 0: nothing


def test_quant_validation(lib):
    q = lib.moe_quant_mxfp8
    assert q(FAKE, 128, 4, 100, FAKE, FAKE, None) == 2                     # H % 32
    assert q(FAKE, 64, 4, 128, FAKE, FAKE, None) == 2                      # ld < H
    assert q(None, 128, 4, 128, FAKE, FAKE, None) == 1
    assert q(FAKE + 8, 128, 4, 128, FAKE, FAKE, None) == 3                 # x not 16-aligned
    assert q(FAKE, 132, 4, 128, FAKE, FAKE, None) == 3                     # ld % 8


def test_permute_validation(lib):
    p = lib.moe_permute
    assert p(FAKE, 4, 0, 0, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2   # top_k
    assert p(FAKE, 4, 2, -1, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2  # offset
    assert p(FAKE, 4, 2, 0, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2   # E_local
    assert p(FAKE, 4, 2, 0, 8, None, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert p(FAKE, 4, 2, 0, 8, FAKE, FAKE, FAKE, FAKE + 16, 1 << 20, None) == 3  # ws align
    assert p(FAKE, 4, 2, 0, 8, FAKE, FAKE, FAKE, FAKE, 8, None) == 5          # ws too small


def test_route_quant_permute_validation(lib):
    f = lib.moe_route_quant_permute

    def call(**kw):
        a = dict(logits=FAKE, ld=8, bias=None, T=4, E=8, k=2, sc=1.0, x=FAKE, ld_x=128, H=128,
                 off=0, el=8, idx=FAKE, w=FAKE, xq=FAKE, xs=FAKE, offs=FAKE, sr=FAKE, rr=FAKE,
                 ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return f(a["logits"], a["ld"], a["bias"], a["T"], a["E"], a["k"], a["sc"], a["x"],
                 a["ld_x"], a["H"], a["off"], a["el"], a["idx"], a["w"], a["xq"], a["xs"],
                 a["offs"], a["sr"], a["rr"], a["ws"], a["wsb"], None)

    assert call(k=0) == 2                 # top_k
    assert call(k=9) == 2                 # top_k > E
    assert call(ld=7) == 2                # ld_logits < E
    assert call(H=100, ld_x=128) == 2     # H % 32
    assert call(ld_x=64) == 2             # ld_x < H
    assert call(off=-1) == 2              # expert offset
    assert call(el=0) == 2                # E_local
    assert call(x=None) == 1
    assert call(offs=None) == 1
    assert call(x=FAKE + 8) == 3          # x not 16-aligned
    assert call(ld_x=132) == 3            # ld_x % 8
    assert call(ws=FAKE + 16) == 3        # workspace alignment
    assert call(wsb=8) == 5               # workspace too small


def test_quant_permute_validation(lib):
    f = lib.moe_quant_permute

    def call(**kw):
        a = dict(x=FAKE, ld_x=128, T=4, H=128, idx=FAKE, k=2, off=0, el=8, xq=FAKE, xs=FAKE,
                 offs=FAKE, sr=FAKE, rr=FAKE, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return f(a["x"], a["ld_x"], a["T"], a["H"], a["idx"], a["k"], a["off"], a["el"], a["xq"],
                 a["xs"], a["offs"], a["sr"], a["rr"], a["ws"], a["wsb"], None)

    assert call(k=0) == 2                 # top_k
    assert call(H=100, ld_x=128) == 2     # H % 32
    assert call(ld_x=64) == 2             # ld_x < H
    assert call(off=-1) == 2              # expert offset
    assert call(el=0) == 2                # E_local
    assert call(T=-1) == 2
    assert call(x=None) == 1
    assert call(idx=None) == 1
    assert call(offs=None) == 1
    assert call(ws=None) == 1
    assert call(x=FAKE + 8) == 3          # x not 16-aligned
    assert call(ld_x=132) == 3            # ld_x % 8
    assert call(idx=FAKE + 2) == 3        # topk_idx not 4-aligned
    assert call(ws=FAKE + 16) == 3        # workspace alignment
    assert call(wsb=8) == 5               # workspace too small


def test_prepack_layout_validation(lib):
    f = lib.moe_prepack_w13_layout
    assert f(FAKE, FAKE, 2, 256, 256, 3, FAKE, FAKE, None) == 4       # unknown layout
    assert f(FAKE, FAKE, 2, 256, 256, -1, FAKE, FAKE, None) == 4
    assert f(FAKE, FAKE, 2, 256, 128, 2, FAKE, FAKE, None) == 2       # I % 256
    assert f(None, FAKE, 2, 256, 256, 2, FAKE, FAKE, None) == 1
    assert f(FAKE + 8, FAKE, 2, 256, 256, 1, FAKE, FAKE, None) == 3


def test_fc_validation(lib):
    f1 = lib.moe_fc1_situ
    args = [FAKE, FAKE, 4, 256, 128, 2, 4, FAKE, FAKE, FAKE, FAKE, 4.0, 25.0, FAKE, FAKE, FAKE,
            1 << 30, None]
    bad = list(args); bad[3] = 200
    assert f1(*bad) == 2                                                    # H % 128
    bad = list(args); bad[11] = 0.0
    assert f1(*bad) == 2                                                    # alpha
    bad = list(args); bad[9] = None
    assert f1(*bad) == 1                                                    # w13 null
    bad = list(args); bad[9] = MIS
    assert f1(*bad) == 3
    bad = list(args); bad[16] = 16
    assert f1(*bad) == 5
    f2 = lib.moe_fc2_combine
    # hq hs T H I top_k E_local offs sroute rrow w w2 w2_s mode out ld_out ws ws_bytes stream
    args2 = [FAKE, FAKE, 4, 256, 128, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 256,
             FAKE, 1 << 30, None]
    bad = list(args2); bad[15] = 128
    assert f2(*bad) == 2                                                    # ld_out < H
    bad = list(args2); bad[15] = 260
    assert f2(*bad) == 3                                                    # ld_out % 8
    bad = list(args2); bad[17] = 1024
    assert f2(*bad) == 5
    bad = list(args2); bad[12] = None
    assert f2(*bad) == 1
    for mode in (2, -1, 99):                                                # unknown mode
        bad = list(args2); bad[13] = mode
        assert f2(*bad) == 4
        tiled = list(bad); tiled[3] = 512; tiled[15] = 512                 # H % 512 for tiled
        assert lib.moe_fc2_combine_tiled(*tiled) == 4
    bad = list(args2); bad[13] = 1; bad[8] = None
    assert f2(*bad) == 1                                                    # atomic needs routes


def test_binding_rejects_cpu_tensors():
    import torch
    from mxfp8_mxfp4_experts_amd import _binding as B
    with pytest.raises(ValueError):
        B.moe_route(torch.zeros(4, 8), None, 2)
    with pytest.raises(ValueError):
        B.moe_quant_mxfp8(torch.zeros(4, 128, dtype=torch.bfloat16))


class _FakeCuda:
    """Stands in for a device tensor in the binding's checks (they read only
    dtype, is_cuda, device, shape and contiguity), so the shape checks that
    guard the prepack launches can be exercised without a GPU."""

    def __init__(self, shape, dtype):
        import torch
        self.t = torch.empty(shape, dtype=dtype)
        self.shape, self.dtype, self.is_cuda, self.device = self.t.shape, dtype, True, "cuda:0"

    def dim(self):
        return self.t.dim()

    def is_contiguous(self):
        return True


def test_binding_checks_prepack_scale_shapes(monkeypatch):
    import torch
    from mxfp8_mxfp4_experts_amd import _binding as B
    monkeypatch.setattr(B, "_need", _need_fake(B._need))
    w = _FakeCuda((2, 512, 128), torch.uint8)                 # E=2, N=512, K=256
    for name in ("moe_prepack_w13", "moe_prepack_w2"):
        fn = getattr(B, name)
        for bad in ((2, 512, 4), (2, 256, 8), (1, 512, 8)):   # K/32 = 8 expected
            with pytest.raises(ValueError):
                fn(w, _FakeCuda(bad, torch.uint8))
    with pytest.raises(ValueError):
        B.moe_prepack_w13_layout(w, _FakeCuda((2, 512, 7), torch.uint8), B.W13_UP_GATE)
    with pytest.raises(ValueError):                            # K/2 not a multiple of 16
        B.moe_prepack_w2(_FakeCuda((2, 512, 100), torch.uint8), _FakeCuda((2, 512, 6), torch.uint8))


def _need_fake(orig):
    def need(t, name, dtype, shape=None, contiguous=True, device=None):
        if isinstance(t, _FakeCuda):
            if t.dtype != dtype:
                raise ValueError(name)
            if shape is not None and tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} must have shape {tuple(shape)}")
            return
        return orig(t, name, dtype, shape, contiguous, device)
    return need


def test_layer_checks_weight_shapes(monkeypatch):
    import torch
    from mxfp8_mxfp4_experts_amd import _binding as B
    from mxfp8_mxfp4_experts_amd.layer import MoELayer
    monkeypatch.setattr(B, "_need", _need_fake(B._need))
    E, H, I = 2, 512, 256
    good = dict(w13=((E, 2 * I, H // 2)), w13_s=((E, 2 * I, H // 32)), w2=((E, H, I // 2)),
                w2_s=((E, H, I // 32)))
    for key, shape in (("w13_s", (E, 2 * I, H // 64)), ("w2", (E, H, I)), ("w2", (E, I, H // 2)),
                       ("w2_s", (E, H, I // 16))):
        args = {k: _FakeCuda(v, torch.uint8) for k, v in good.items()}
        args[key] = _FakeCuda(shape, torch.uint8)
        with pytest.raises(ValueError):
            MoELayer(args["w13"], args["w13_s"], args["w2"], args["w2_s"], top_k=2, E=E)
    args = {k: _FakeCuda(v, torch.uint8) for k, v in good.items()}
    with pytest.raises(ValueError):
        MoELayer(args["w13"], args["w13_s"], args["w2"], args["w2_s"], top_k=2, E=E,
                 combine="fused")


def test_permute_noalloc_validation(lib):
    p = lib.moe_permute_noalloc
    assert p(FAKE, 4, 0, 0, 8, FAKE, FAKE, FAKE, None) == 2                # top_k 0
    assert p(FAKE, 4, 2, -1, 8, FAKE, FAKE, FAKE, None) == 2               # offset < 0
    assert p(FAKE, 4, 2, 0, 5000, FAKE, FAKE, FAKE, None) == 2             # E_local > 4096
    assert p(None, 4, 2, 0, 8, FAKE, FAKE, FAKE, None) == 1                # null ids
    assert p(FAKE, 4, 2, 0, 8, None, FAKE, FAKE, None) == 1                # null offsets
    assert p(FAKE, 4, 2, 0, 8, MIS, FAKE, FAKE, None) == 3
    # 2^18 routes over 4096 local experts need an 8 MiB schedule: past the
    # 4 MiB static scratch, refused before any HIP call.
    assert p(FAKE, 16384, 16, 0, 4096, FAKE, FAKE, FAKE, None) == 8

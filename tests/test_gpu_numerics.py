"""Hardware arithmetic under the FC kernels, measured against exact float64.

The test-only probe library (``tests/probe/numerics_probe.hip``, built by
``build()``) runs single device functions of the FC kernels on inputs chosen
here:

* the FC1 epilogue's hardware scaled E4M3 conversion, swept over every E4M3
  code, every rounding midpoint and its float neighbours, and random values,
  at scales across the whole normal range, against the oracle's encoder;
* the FC1 epilogue's float32 SiTU against the float64 SiTU of the same
  float32 inputs;
* the block-scaled MFMA (E2M1 x E4M3, E8M0 per 32 K) accumulated over the
  full hidden width as the FC kernels do, against the exact float64 sum.

The last two also report how many requantised bytes each error source alone
flips (the FC1 output is requantised to E4M3 right after SiTU), which is what
the requantisation bar of the parity tests has to allow for.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.codecs import mxfp4_dequantize, mxfp8_dequantize, mxfp8_quantize

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libnumprobe.so")
_P, _I, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        raise FileNotFoundError(f"{PROBE} missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE)
    lib.probe_mfma_w4a8.restype = _I
    lib.probe_mfma_w4a8.argtypes = [_P, _P, _P, _P, _I, _I, _P, _P]
    lib.probe_situ.restype = _I
    lib.probe_situ.argtypes = [_P, _P, _I, _F, _F, _P, _P]
    lib.probe_e4m3_scaled.restype = _I
    lib.probe_e4m3_scaled.argtypes = [_P, _P, _I, _P, _P, _P]
    return lib


def _stream():
    return torch.cuda.current_stream().cuda_stream


def test_e4m3_scaled_conversion_sweep(probe):
    """Every E4M3 magnitude, every midpoint between neighbours and the float32
    neighbours of both, plus 2^20 random values in [-448, 448], each times
    2^e for e across the normal scale range: the hardware conversion gives
    the oracle's nearest-even code of x / 2^e, and so does the integer
    encoder."""
    from oracle.codecs import E4M3_TABLE, e4m3_encode

    mags = E4M3_TABLE[:0x7F].astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    base = np.concatenate([mags, mids]).astype(np.float32)
    near = np.concatenate([base, np.nextafter(base, np.float32(np.inf)),
                           np.nextafter(base, np.float32(0))])
    near = np.concatenate([near, -near])
    rng = np.random.default_rng(7)
    rand = rng.uniform(-448.0, 448.0, 1 << 20).astype(np.float32)
    vals = np.concatenate([near, rand])
    vals = np.concatenate([vals, np.zeros((-len(vals)) % 4, np.float32)])
    for e in (-126, -100, -40, -9, -7, -1, 0, 3, 40, 100, 127):
        x = (vals.astype(np.float64) * 2.0 ** e).astype(np.float32)
        exact = x.astype(np.float64) * 2.0 ** -e
        keep = np.abs(exact) <= 448.0          # the scale rule keeps |x / 2^e| <= 448
        xs = np.where(keep, x, np.float32(0))
        n4 = len(xs) // 4
        xd = torch.from_numpy(xs).to(DEV)
        ed = torch.full((n4,), e, dtype=torch.int32, device=DEV)
        hw = torch.empty(n4, dtype=torch.int32, device=DEV)
        ref = torch.empty(n4, dtype=torch.int32, device=DEV)
        assert probe.probe_e4m3_scaled(xd.data_ptr(), ed.data_ptr(), n4, hw.data_ptr(),
                                       ref.data_ptr(), _stream()) == 0
        torch.cuda.synchronize()
        hw_b = hw.cpu().numpy().view(np.uint8)
        ref_b = ref.cpu().numpy().view(np.uint8)
        want = e4m3_encode(xs.astype(np.float64) * 2.0 ** -e)
        bad = np.nonzero(hw_b != want)[0]
        assert bad.size == 0, (e, xs[bad[:4]], hw_b[bad[:4]], want[bad[:4]])
        assert np.array_equal(ref_b, want), e


def _situ_inputs():
    rng = np.random.default_rng(11)
    g = rng.normal(0.0, 1.7, 1 << 20)
    u = rng.normal(0.0, 1.7, 1 << 20)
    # near zero, where tanh's 1 - e^(-2x) form cancels, and far out, where
    # the exponentials are capped
    small = np.geomspace(1e-8, 1.0, 4096)
    big = np.geomspace(1.0, 200.0, 1024)
    grid = np.concatenate([small, -small, big, -big])
    g = np.concatenate([g, grid, np.full(grid.size, 1.3), np.zeros(8)])
    u = np.concatenate([u, np.full(grid.size, 1.1), grid, np.linspace(-3, 3, 8)])
    return g.astype(np.float32), u.astype(np.float32)


def situ_float32_bound(g, u, alpha=4.0, beta=25.0):
    """What the kernel's float32 SiTU may be off by: a few float32 ulps
    relative plus the rounding of the exponent g log2(e) (|g| 2^-24), plus,
    where 1 - e^(-2y) cancels for small |g| / alpha or |u| / beta, a few ulps
    of each tanh factor's scale times the other factor."""
    from tests.gpu_util import situ_f32_error

    return situ_f32_error(g, u, alpha, beta)


@pytest.mark.parametrize("alpha,beta", [(4.0, 25.0), (2.0, 10.0)])
def test_situ_float32_against_float64(probe, alpha, beta):
    g, u = _situ_inputs()
    n = g.size
    gd, ud = torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV)
    out = torch.empty(n, dtype=torch.float32, device=DEV)
    assert probe.probe_situ(gd.data_ptr(), ud.data_ptr(), n, alpha, beta, out.data_ptr(),
                            _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.situ(g.astype(np.float64), u.astype(np.float64), alpha, beta)
    err = np.abs(got - ref)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    n_rand = 1 << 20
    print(f"[situ alpha={alpha}] float32 vs float64: max rel {rel.max():.3g}, median rel "
          f"{np.median(rel[:n_rand]):.3g}, p99.9 {np.quantile(rel[:n_rand], 0.999):.3g}",
          flush=True)
    # requantised bytes this error alone flips (rows of 3584 = 112 groups of 32)
    rows = n_rand // 3584
    a_ref = ref[:rows * 3584].reshape(rows, 3584)
    a_got = got[:rows * 3584].reshape(rows, 3584)
    q_ref, _ = mxfp8_quantize(a_ref)
    q_got, _ = mxfp8_quantize(a_got)
    flips = float(np.mean(q_ref != q_got))
    print(f"[situ] requantised bytes flipped by the float32 SiTU alone: {flips:.3g}", flush=True)
    assert np.all(np.isfinite(got))
    bound = situ_float32_bound(g.astype(np.float64), u.astype(np.float64), alpha, beta)
    worst = int(np.argmax(err / bound))
    print(f"[situ] worst error / bound: {err[worst] / bound[worst]:.3g}", flush=True)
    assert np.all(err <= bound), (g[worst], u[worst], got[worst], ref[worst])


def _mfma_case(n_tiles, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((16, K)).astype(np.float32)
    aq, asc = oracle.quant_x(synth.f32_to_bf16_bits(x))
    w = torch.from_numpy((0.02 * rng.standard_normal((16 * n_tiles, K))).astype(np.float32))
    w = w.to(torch.bfloat16).to(torch.float32)
    wq, wsc = synth._mxfp4_encode_torch(w)
    return aq, asc, wq.numpy(), wsc.numpy()


@pytest.mark.parametrize("K,n_tiles", [(128, 224), (256, 224), (7168, 224)])
def test_mfma_accumulation_against_exact(probe, K, n_tiles):
    """Raw float32 accumulators of the block-scaled MFMA over K (one MFMA
    step; two; one FC1 row of the full-size layer) against the exact float64
    dot products.  The error is reported relative to the sum of |products|
    (the natural scale of a summation error), and held to the bound the
    requantisation check of the parity tests assumes (2^-15 of that sum); the
    bytes it flips after SiTU and requantisation are reported too."""
    from tests.gpu_util import ACC_EPS

    aq, asc, wq, wsc = _mfma_case(n_tiles, K, 3 + K)
    A = mxfp8_dequantize(aq, asc)
    W = mxfp4_dequantize(wq, wsc)
    exact = W @ A.T                                  # [rows, 16]
    absum = np.abs(W) @ np.abs(A).T
    d = [torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for v in (wq, wsc, aq, asc)]
    out = torch.empty((16 * n_tiles, 16), dtype=torch.float32, device=DEV)
    assert probe.probe_mfma_w4a8(d[0].data_ptr(), d[1].data_ptr(), d[2].data_ptr(),
                                 d[3].data_ptr(), n_tiles, K, out.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - exact) / absum
    rel = np.abs(got - exact) / np.maximum(np.abs(exact), 1e-30)
    print(f"[mfma K={K}] |err| / sum|products|: max {err.max():.3g}, median {np.median(err):.3g}; "
          f"|err| / |exact|: median {np.median(rel):.3g}, p99 {np.quantile(rel, 0.99):.3g}; "
          f"exact in float32: {np.mean(got == exact.astype(np.float32)):.3f}", flush=True)
    # Bytes flipped when these accumulators feed SiTU and the requantisation
    # (gate = the first half of the rows, up = the second, per token).
    h = 8 * n_tiles
    q_ref, _ = mxfp8_quantize(oracle.situ(exact[:h].T, exact[h:].T))
    q_got, _ = mxfp8_quantize(oracle.situ(got[:h].T, got[h:].T))
    print(f"[mfma K={K}] requantised bytes flipped by the accumulation alone: "
          f"{np.mean(q_ref != q_got):.3g}", flush=True)
    assert err.max() <= ACC_EPS

"""Pins of the oracle's layer steps (CPU only).

The oracle is checked against the independent brute force, against special
cases that reduce to a library routine or to integer arithmetic, against
one-hot probes that fix the layouts, and against invariants of the method.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import codecs as C
from oracle.brute import brute_force_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kimi_k3_facts.json")


def _np_weights(case):
    return {k: case[k].numpy() for k in ("w13", "w13_s", "w2", "w2_s")}


def _run_both(cfg, case, **kw):
    w = _np_weights(case)
    args = (case["x_bf16"], case["logits"], case["bias"], w["w13"], w["w13_s"], w["w2"], w["w2_s"])
    o = oracle.oracle_layer(*args, top_k=cfg.K, expert_offset=cfg.expert_offset,
                            routed_scaling=cfg.routed_scaling, **kw)
    b = brute_force_layer(*args, top_k=cfg.K, expert_offset=cfg.expert_offset,
                          routed_scaling=cfg.routed_scaling, **kw)
    return o, b


def _assert_agree(o, b):
    assert np.array_equal(o["topk_idx"], b["topk_idx"])
    assert np.array_equal(o["topk_w"], b["topk_w"])
    scale = max(np.abs(o["out"]).max(), 1e-300)
    assert np.abs(o["out"] - b["out"]).max() <= 1e-12 * scale
    T, K = o["topk_idx"].shape
    for (t, k), (hc, hsc) in b["h"].items():
        row = o["route_row"][t * K + k]
        assert row >= 0
        assert np.array_equal(o["hq"][row], np.array(hc, np.uint8))
        assert np.array_equal(o["hs"][row], np.array(hsc, np.uint8))
    assert len(b["h"]) == int(o["expert_offsets"][-1])


def test_oracle_equals_bruteforce_tiny_config():
    cfg = synth.WORKLOADS["tiny"]
    case = synth.make_case(cfg)
    o, b = _run_both(cfg, case)
    _assert_agree(o, b)


@pytest.mark.parametrize("shape", [
    dict(T=5, H=64, I=32, E=6, K=3, E_local=6),
    dict(T=7, H=96, I=64, E=8, K=2, E_local=3, expert_offset=2),
    dict(T=4, H=32, I=32, E=3, K=3, E_local=3, bias_kind="zero"),
])
def test_oracle_equals_bruteforce_random_tiny(shape):
    cfg = synth.custom_config("t", 50 + shape["T"], **shape)
    case = synth.make_case(cfg)
    o, b = _run_both(cfg, case)
    _assert_agree(o, b)


def test_oracle_equals_bruteforce_with_masked_slots():
    cfg = synth.custom_config("m", 61, T=6, H=64, I=32, E=5, K=3, E_local=5)
    case = synth.make_case(cfg)
    ids, w = oracle.route(case["logits"], case["bias"], cfg.K)
    ids = ids.copy()
    ids[0, 1] = -1
    ids[2, :] = -1            # a token with no kept slot
    ids[4, 2] = -1
    o, b = _run_both(cfg, case, topk_idx=ids, topk_w=w)
    _assert_agree(o, b)
    assert np.all(o["out"][2] == 0)


# ---------------------------------------------------------------- routing
def test_route_bias_free_is_topk_of_logits():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((64, 40)).astype(np.float32)
    ids, w = oracle.route(logits, None, 6)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :6]
    assert np.array_equal(ids, ref)


def test_route_tie_goes_to_lower_index_and_invariants():
    logits = np.zeros((1, 6), np.float32)
    logits[0, 3] = logits[0, 1] = 2.0
    logits[0, 5] = 1.0
    ids, w = oracle.route(logits, np.zeros(6, np.float32), 3)
    assert list(ids[0]) == [1, 3, 5]
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((100, 896)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(896)).astype(np.float32)
    ids, w = oracle.route(lg, bias, 16, routed_scaling=2.5)
    assert all(len(set(r)) == 16 for r in ids)
    assert np.all((ids >= 0) & (ids < 896))
    s = 1 / (1 + np.exp(-lg.astype(np.float64)))
    sel = np.take_along_axis(s, ids, 1)
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=4 * 2.0 ** -23)
    np.testing.assert_allclose(w / w.sum(1, keepdims=True), sel / sel.sum(1, keepdims=True), rtol=1e-6)
    # Selection used s + bias, ordered by the key
    key = s.astype(np.float32) + bias[None]
    ks = np.take_along_axis(key, ids, 1)
    assert np.all(np.diff(ks, axis=1) <= 0)
    assert np.all(ks[:, -1:] >= np.sort(key, 1)[:, -16:-15])


def test_route_bias_changes_selection_not_weights():
    # A huge bias on expert 0 forces it in; its weight still uses the
    # bias-free score (page 1, Key sources table, routing row).
    logits = np.array([[-3.0, 1.0, 2.0, 0.5]], np.float32)
    bias = np.array([10.0, 0, 0, 0], np.float32)
    ids, w = oracle.route(logits, bias, 2)
    assert list(ids[0]) == [0, 2]
    s0, s2 = 1 / (1 + math.exp(3.0)), 1 / (1 + math.exp(-2.0))
    np.testing.assert_allclose(w[0], [s0 / (s0 + s2), s2 / (s0 + s2)], rtol=1e-6)


# ---------------------------------------------------------------- permute
def test_permute_bruteforce_and_window():
    rng = np.random.default_rng(5)
    ids = rng.integers(-1, 20, (50, 4)).astype(np.int32)
    offs, sr, rr = oracle.permute(ids, 5, 10)
    flat = ids.reshape(-1)
    kept = [r for r in range(flat.size) if 5 <= flat[r] < 15]
    assert offs[-1] == len(kept)
    for e in range(10):
        rows = [r for r in kept if flat[r] - 5 == e]
        assert list(sr[offs[e]:offs[e + 1]]) == rows       # stable, ascending
    for r in range(flat.size):
        if r in kept:
            assert sr[rr[r]] == r
        else:
            assert rr[r] == -1


# ---------------------------------------------------------------- layouts
def _one_hot_case(H=128, I=64, seed=7):
    rng = np.random.default_rng(seed)
    w13 = rng.integers(0, 256, (1, 2 * I, H // 2)).astype(np.uint8)
    w13_s = rng.integers(120, 134, (1, 2 * I, H // 32)).astype(np.uint8)
    return w13, w13_s


@pytest.mark.parametrize("j", [0, 1, 33, 126, 127])
def test_fc1_one_hot_probe_pins_nibbles_halves_and_scales(j):
    H, I = 128, 64
    w13, w13_s = _one_hot_case(H, I)
    x = np.zeros((1, H), np.uint16)
    x[0, j] = 0x3F80                 # bf16 1.0 -> scale 2^-8, payload 256 (exact)
    xq, xs = oracle.quant_x(x)
    assert xq[0, j] == 0x78 and xs[0, j // 32] == 127 - 8
    offs = np.array([0, 1], np.int32)
    hq, hs, acc = oracle.fc1_situ_requant(xq, xs, offs, np.array([0], np.int32), 1,
                                          w13, w13_s, return_acc=True)
    byte = w13[0, :, j // 2]
    nib = (byte & 0xF) if j % 2 == 0 else (byte >> 4)
    expect = C.E2M1_TABLE[nib] * np.ldexp(1.0, w13_s[0, :, j // 32].astype(np.int64) - 127)
    assert np.array_equal(acc[0], expect)
    # gate = first half, up = second half (accumulators start from +0.0, so an
    # all-zero column is +0.0 whatever the sign of the zero weight code)
    expect = expect + 0.0
    a = oracle.situ(expect[:I], expect[I:])
    eq, es = C.mxfp8_quantize(a[None])
    assert np.array_equal(hq, eq) and np.array_equal(hs, es)


def test_fc1_gate_up_halves_not_swapped():
    # up half all zero -> SiTU output zero; a [up; gate] swap would not be.
    H, I = 64, 32
    w13 = np.zeros((1, 2 * I, H // 2), np.uint8)
    w13[0, :I] = 0x22                 # gate rows: every element 1.0
    w13_s = np.full((1, 2 * I, H // 32), 127, np.uint8)
    x = np.full((1, H), 0x3F80, np.uint16)
    xq, xs = oracle.quant_x(x)
    hq, hs, acc = oracle.fc1_situ_requant(xq, xs, np.array([0, 1], np.int32),
                                          np.array([0], np.int32), 1, w13, w13_s, return_acc=True)
    assert np.all(acc[0, :I] == H) and np.all(acc[0, I:] == 0)
    assert np.all((hq & 0x7F) == 0)


def test_fc_integer_special_case():
    # all scales 2^0, weight codes +-1 and activations of small integers:
    # FC1 reduces to an integer matrix product.
    rng = np.random.default_rng(8)
    H, I, n = 128, 64, 5
    signs = rng.integers(0, 2, (1, 2 * I, H))
    codes = (2 | (signs << 3)).astype(np.uint8)            # +-1.0
    w13 = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    w13_s = np.full((1, 2 * I, H // 32), 127, np.uint8)
    xi = rng.integers(-7, 8, (n, H))
    xi[:, ::32] = 7                                         # same group scale everywhere
    xf = xi.astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)        # exact in bf16
    xq, xs = oracle.quant_x(x)
    offs = np.array([0, n], np.int32)
    _, _, acc = oracle.fc1_situ_requant(xq, xs, offs, np.arange(n, dtype=np.int32), 1,
                                        w13, w13_s, return_acc=True)
    wint = np.where(signs[0] == 1, -1, 1)
    assert np.array_equal(acc, (xi @ wint.T).astype(np.float64))


def test_fc2_one_hot_probe():
    H, I = 64, 64
    rng = np.random.default_rng(9)
    w2 = rng.integers(0, 256, (1, H, I // 2)).astype(np.uint8)
    w2_s = rng.integers(122, 132, (1, H, I // 32)).astype(np.uint8)
    j = 45
    hq = np.zeros((1, I), np.uint8)
    hq[0, j] = 0x38                  # E4M3 1.0
    hs = np.full((1, I // 32), 127, np.uint8)
    y = oracle.fc2(hq, hs, np.array([0, 1], np.int32), w2, w2_s)
    nib = (w2[0, :, j // 2] >> 4) if j % 2 else (w2[0, :, j // 2] & 0xF)
    expect = C.E2M1_TABLE[nib] * np.ldexp(1.0, w2_s[0, :, j // 32].astype(np.int64) - 127)
    assert np.array_equal(y[0], expect)


# ---------------------------------------------------------------- SiTU
def test_situ_limits_and_identities():
    assert oracle.situ(0.0, 3.0) == 0.0
    assert oracle.situ(2.0, 0.0) == 0.0
    np.testing.assert_allclose(oracle.situ(60.0, 1000.0), 4.0 * 25.0, rtol=1e-12)
    assert abs(oracle.situ(-60.0, 1.0)) < 1e-20
    np.testing.assert_allclose(oracle.situ(60.0, -1000.0), -100.0, rtol=1e-12)
    # |g| << 4 and |u| << 25: SiLU(g) * u
    g, u = 1e-3, 2e-3
    np.testing.assert_allclose(oracle.situ(g, u), g / (1 + math.exp(-g)) * u, rtol=1e-6)
    facts = json.load(open(GOLDEN))["model_config"]
    g, u = 1.7, -3.2
    ref = (facts["situ_gate_beta"] * math.tanh(g / facts["situ_gate_beta"]) / (1 + math.exp(-g))
           * facts["situ_linear_beta"] * math.tanh(u / facts["situ_linear_beta"]))
    np.testing.assert_allclose(oracle.situ(g, u), ref, rtol=1e-15)


# ---------------------------------------------------------------- combine / EP
def test_combine_k1_and_linearity():
    rng = np.random.default_rng(10)
    y = rng.standard_normal((6, 8))
    rr = np.arange(6, dtype=np.int32)
    out = oracle.combine(y, rr, np.ones(6, np.float32), 6, 1)
    assert np.array_equal(out, y)
    w = rng.random((3, 2)).astype(np.float32)
    out2 = oracle.combine(y, rr, w, 3, 2)
    ref = w[:, :1].astype(np.float64) * y[0::2] + w[:, 1:].astype(np.float64) * y[1::2]
    np.testing.assert_allclose(out2, ref, rtol=1e-15)


def test_expert_parallel_shards_sum_to_full_layer():
    cfg = synth.custom_config("ep", 70, T=9, H=64, I=32, E=8, K=3, E_local=8)
    case = synth.make_case(cfg)
    w = _np_weights(case)
    full = oracle.oracle_layer(case["x_bf16"], case["logits"], case["bias"], w["w13"], w["w13_s"],
                               w["w2"], w["w2_s"], top_k=3)
    total = np.zeros_like(full["out"])
    for off in (0, 2, 4, 6):
        sl = slice(off, off + 2)
        part = oracle.oracle_layer(case["x_bf16"], case["logits"], case["bias"], w["w13"][sl],
                                   w["w13_s"][sl], w["w2"][sl], w["w2_s"][sl], top_k=3,
                                   expert_offset=off)
        total += part["out"]
    np.testing.assert_allclose(total, full["out"], rtol=1e-12, atol=1e-15)


def test_oracle_tokens_matches_full_layer_rows():
    cfg = synth.custom_config("s", 71, T=10, H=64, I=64, E=6, K=2, E_local=4, expert_offset=1)
    case = synth.make_case(cfg)
    w = _np_weights(case)
    full = oracle.oracle_layer(case["x_bf16"], case["logits"], case["bias"], w["w13"], w["w13_s"],
                               w["w2"], w["w2_s"], top_k=2, expert_offset=1)
    sub = oracle.oracle_tokens([7, 2, 9], case["x_bf16"], full["topk_idx"], full["topk_w"],
                               lambda e: (w["w13"][e], w["w13_s"][e], w["w2"][e], w["w2_s"][e]),
                               top_k=2, expert_offset=1, E_local=4)
    np.testing.assert_allclose(sub["out"], full["out"][[7, 2, 9]], rtol=1e-13, atol=1e-300)


def test_generator_weights_are_mxfp4_of_bf16_normals():
    # The input generator's bytes decode to values whose per-group absmax
    # sits in (3, 6] after scaling (smallest-scale rule), as the recipe says.
    cfg = synth.WORKLOADS["tiny"]
    wt = synth.make_expert_weights(cfg, experts=[0])
    v = C.mxfp4_dequantize(wt["w13"][0].numpy(), wt["w13_s"][0].numpy())
    sc = C.e8m0_decode(wt["w13_s"][0].numpy())
    r = np.abs(v).reshape(v.shape[0], -1, 32).max(-1) / sc
    assert np.all(r <= 6.0) and np.all(r >= 3.0)
    assert 0.01 < v.std() < 0.03


def test_report_accumulators_agree_and_bound_the_sums():
    """The report-only FC1 outputs: oracle_tokens' per-route accumulators and
    |product| sums equal oracle_layer's rows, and every |accumulator| is at
    most its sum of |products| (triangle inequality), with equality where
    all products share a sign (a one-hot activation row)."""
    cfg = synth.custom_config("s", 72, T=10, H=64, I=64, E=6, K=2, E_local=4, expert_offset=1)
    case = synth.make_case(cfg)
    w = _np_weights(case)
    full = oracle.oracle_layer(case["x_bf16"], case["logits"], case["bias"], w["w13"], w["w13_s"],
                               w["w2"], w["w2_s"], top_k=2, expert_offset=1, report=True)
    assert np.all(np.abs(full["acc"]) <= full["absum"] * (1 + 1e-15))
    sub = oracle.oracle_tokens([7, 2, 9], case["x_bf16"], full["topk_idx"], full["topk_w"],
                               lambda e: (w["w13"][e], w["w13_s"][e], w["w2"][e], w["w2_s"][e]),
                               top_k=2, expert_offset=1, E_local=4)
    toks = [7, 2, 9]
    for (j, k), (hq, hs, a, acc, absum) in sub["h"].items():
        row = int(full["route_row"][toks[j] * 2 + k])
        assert np.array_equal(hq, full["hq"][row]) and np.array_equal(hs, full["hs"][row])
        np.testing.assert_allclose(acc, full["acc"][row], rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(absum, full["absum"][row], rtol=1e-13, atol=1e-300)
    # one-hot activation: x = 1.0 at column 5 only, so acc = deq(w[:, 5]) and
    # absum = |acc| exactly
    xb = np.zeros((1, 64), np.uint16)
    xb[0, 5] = 0x3F80
    one = oracle.oracle_layer(xb, None, None, w["w13"], w["w13_s"], w["w2"], w["w2_s"], top_k=1,
                              topk_idx=np.array([[1]], np.int32),
                              topk_w=np.array([[1.0]], np.float32), report=True)
    assert np.array_equal(np.abs(one["acc"]), one["absum"])

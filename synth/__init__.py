"""Seeded synthetic inputs for the Kimi-K3-style MoE expert layer.

This module is shared by the CPU oracle and by the GPU path's tests and
benchmark.  It only *draws* inputs; it holds none of the layer's arithmetic
(routing, activation quantisation, GEMMs, SiTU, combine).  The one encoder it
contains turns the drawn bf16 expert weights into MXFP4 bytes, because the
layer receives its expert weights already in that checkpoint format (page 1,
"real checkpoint contract": packed E2M1 weights with one E8M0 scale per 32
elements along K; page 5: w13 ``[E, 2I, H/2]`` with scales ``[E, 2I, H/32]``).

Recipe (one seeded scheme for every workload):

* root ``SeedSequence(20261202)``; workload ``c`` uses child ``spawn_key=(c,)``
  split into four streams in the order logits, bias, x, perm;
* ``x``: ``standard_normal(float32)`` rounded to bf16 (nearest-even), ``[T, H]``;
* router logits: ``standard_normal(float32)`` ``[T, E]``;
* correction bias: ``0.1 * standard_normal(float32)`` ``[E]``, or for the
  skewed expert-parallel share ``0.04 * ln(r ** -1.2)`` with ``r`` a seeded
  permutation of ``1..E`` (a Zipf(1.2) popularity folded into the bias);
* "ep_mixed" workloads (the checkpoint-true expert shape of page 1, "真实
  checkpoint 契约": routed latent 3584, expert intermediate 3072, 28 local
  experts of 896 on rank 7 of 32, and its benchmark, where 8 of each token's
  16 slots name local experts and 8 remote ones) take their top-k ids and
  weights from the generator instead of the router: per token, 8 distinct
  local ids and 8 distinct remote ids (uniform, without replacement, from
  the ``bias`` stream), the 16 slots in a seeded random order (``perm``
  stream), weights ``sigmoid(z)`` with ``z ~ N(0, 1)`` (``logits`` stream)
  normalised to sum 1 over the token's slots;
* expert weights: per-expert torch generator seeded from
  ``spawn_key=(99, e)``; ``0.02 * randn`` rounded to bf16, then MXFP4 with the
  smallest power-of-two scale that keeps the group's absmax within 6 and
  nearest-even E2M1 rounding.  w13 rows are ``[gate (I); up (I)]``.

The weight set depends on the device that draws it (torch's CPU and GPU
generators differ); every consumer receives the same bytes, so both sides of a
comparison always see identical inputs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

ROOT_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape of one MoE-layer workload."""

    name: str
    key: int          # spawn key of the workload's activation streams
    T: int            # tokens
    H: int            # hidden width (FC1 K, FC2 N)
    I: int            # expert intermediate width (FC1 N = 2I, FC2 K)
    E: int            # global experts (routing width)
    K: int            # top-k
    E_local: int      # experts held by this GPU
    expert_offset: int = 0
    bias_kind: str = "normal"   # "normal" | "zipf" | "zero"
    routing: str = "router"     # "router" (a1 on the logits) | "ep_mixed" (given top-k)
    routed_scaling: float = 1.0
    situ_alpha: float = 4.0
    situ_beta: float = 25.0

    @property
    def R(self) -> int:
        return self.T * self.K


# The workloads by name (the second field is each one's seed-stream key):
# tiny, decode, batched decode, 8K prefill chunk, and one GPU's
# expert-parallel share with Zipf-skewed load ...
_ALL = [
    LayerConfig("tiny", 0, T=16, H=128, I=128, E=4, K=2, E_local=4),
    LayerConfig("decode_T8", 1, T=8, H=7168, I=3584, E=896, K=16, E_local=896),
    LayerConfig("batched_decode_T256", 2, T=256, H=7168, I=3584, E=896, K=16, E_local=896),
    LayerConfig("prefill_T8192", 3, T=8192, H=7168, I=3584, E=896, K=16, E_local=896),
    LayerConfig("ep_share_T4096", 4, T=4096, H=7168, I=3584, E=896, K=16, E_local=224,
                expert_offset=0, bias_kind="zipf"),
]
# ... and the checkpoint-true expert shape with the pages' own benchmark
# routing (one GPU of 32 holding experts [196, 224), 8 local + 8 remote slots
# per token), at the four local batch sizes the pages measure.
for _i, _m in enumerate((128, 512, 2048, 8192)):
    _ALL.append(LayerConfig(f"ckpt_ep32r7_M{_m}", 5 + _i, T=_m, H=3584, I=3072, E=896,
                            K=16, E_local=28, expert_offset=196, routing="ep_mixed"))
# ... and the same shape at one token, the real-size decode case of the
# pages' coverage matrix (page 1, "对称性约束").
_ALL.append(LayerConfig("ckpt_ep32r7_M1", 9, T=1, H=3584, I=3072, E=896, K=16, E_local=28,
                        expert_offset=196, routing="ep_mixed"))
WORKLOADS = {c.name: c for c in _ALL}


def custom_config(name: str, key: int, **kw) -> LayerConfig:
    """A test workload with its own activation seed stream ``key``."""
    kw.setdefault("E_local", kw.get("E"))
    return LayerConfig(name, key, **kw)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.ascontiguousarray(a, dtype=np.float32))
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _streams(cfg: LayerConfig, seed: int):
    ss = np.random.SeedSequence(seed, spawn_key=(cfg.key,))
    return [np.random.default_rng(s) for s in ss.spawn(4)]


def make_topk_ep_mixed(cfg: LayerConfig, T: int, r_w, r_ids, r_order):
    """Top-k ids and weights of an "ep_mixed" workload: 8 local and 8 remote
    distinct experts per token (K = 16), slots shuffled, positive weights
    summing to 1 per token."""
    assert cfg.K == 16 and cfg.E_local >= 8 and cfg.E - cfg.E_local >= 8
    n_loc = cfg.K // 2
    loc = np.argsort(r_ids.random((T, cfg.E_local)), axis=1)[:, :n_loc] + cfg.expert_offset
    rem = np.argsort(r_ids.random((T, cfg.E - cfg.E_local)), axis=1)[:, :cfg.K - n_loc]
    rem = np.where(rem < cfg.expert_offset, rem, rem + cfg.E_local)
    ids = np.concatenate([loc, rem], axis=1)
    order = np.argsort(r_order.random((T, cfg.K)), axis=1)
    ids = np.take_along_axis(ids, order, axis=1).astype(np.int32)
    s = 1.0 / (1.0 + np.exp(-r_w.standard_normal((T, cfg.K))))
    w = (s / s.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def make_activations(cfg: LayerConfig, seed: int = ROOT_SEED, T: Optional[int] = None):
    """Return dict(x_bf16 uint16[T,H], logits f32[T,E], bias f32[E]); for
    "ep_mixed" workloads dict(x_bf16, topk_idx int32[T,K], topk_w f32[T,K])
    instead of the router inputs.

    ``T`` may shorten the token count (the first rows of the same streams are
    NOT reproduced; a shorter draw is its own case)."""
    T = cfg.T if T is None else T
    r_logits, r_bias, r_x, r_perm = _streams(cfg, seed)
    if cfg.routing == "ep_mixed":
        ids, w = make_topk_ep_mixed(cfg, T, r_logits, r_bias, r_perm)
        x = f32_to_bf16_bits(r_x.standard_normal((T, cfg.H), dtype=np.float32))
        return {"x_bf16": x, "topk_idx": ids, "topk_w": w}
    logits = r_logits.standard_normal((T, cfg.E), dtype=np.float32)
    if cfg.bias_kind == "normal":
        bias = (np.float32(0.1) * r_bias.standard_normal(cfg.E, dtype=np.float32)).astype(np.float32)
    elif cfg.bias_kind == "zipf":
        rank = r_perm.permutation(cfg.E).astype(np.float64) + 1.0
        bias = (0.04 * np.log(rank ** -1.2)).astype(np.float32)
    elif cfg.bias_kind == "zero":
        bias = np.zeros(cfg.E, np.float32)
    else:
        raise ValueError(cfg.bias_kind)
    x = f32_to_bf16_bits(r_x.standard_normal((T, cfg.H), dtype=np.float32))
    return {"x_bf16": x, "logits": logits, "bias": bias}


def expert_seed(e: int, seed: int = ROOT_SEED) -> int:
    st = np.random.SeedSequence(seed, spawn_key=(99, int(e))).generate_state(2, np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


# E2M1 rounding thresholds between consecutive magnitudes 0,.5,1,1.5,2,3,4,6.
# A value exactly on threshold i goes to the even code of {i, i+1}.
_E2M1_THRESH = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _mxfp4_encode_torch(w):
    """bf16-valued float32 weights ``[rows, K]`` -> (packed uint8 [rows,K/2], scale uint8 [rows,K/32])."""
    import torch

    rows, K = w.shape
    g = w.reshape(rows, K // 32, 32).double()
    amax = g.abs().amax(-1)
    m, p = torch.frexp(amax)                       # amax = m * 2**p, m in [0.5, 1)
    e = torch.where(m <= 0.75, p - 3, p - 2)       # smallest e with amax <= 6 * 2**e
    e = torch.where(amax == 0, torch.full_like(e, -127), e).clamp(-127, 127).to(torch.int64)
    inv = ((1023 - e) << 52).view(torch.float64)   # exactly 2**-e
    a = g.abs() * inv[..., None]
    code = torch.zeros_like(a, dtype=torch.uint8)
    for i, t in enumerate(_E2M1_THRESH):
        code += (a > t).to(torch.uint8) if i % 2 == 0 else (a >= t).to(torch.uint8)
    code |= torch.signbit(g).to(torch.uint8) << 3
    code = code.reshape(rows, K)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def make_expert_weights(cfg: LayerConfig, experts: Optional[Sequence[int]] = None,
                        device="cpu", seed: int = ROOT_SEED, out=None):
    """Draw MXFP4 expert weights.

    Returns dict of torch uint8 tensors on ``device``:
    ``w13 [n, 2I, H/2]``, ``w13_s [n, 2I, H/32]``, ``w2 [n, H, I/2]``,
    ``w2_s [n, H, I/32]`` for the global expert ids ``experts`` (default: the
    local window ``[expert_offset, expert_offset + E_local)``).  ``out`` may
    hold preallocated tensors of those shapes to fill in place.
    """
    import torch

    if experts is None:
        experts = range(cfg.expert_offset, cfg.expert_offset + cfg.E_local)
    experts = list(experts)
    H, I = cfg.H, cfg.I
    n = len(experts)
    if out is None:
        out = {
            "w13": torch.empty((n, 2 * I, H // 2), dtype=torch.uint8, device=device),
            "w13_s": torch.empty((n, 2 * I, H // 32), dtype=torch.uint8, device=device),
            "w2": torch.empty((n, H, I // 2), dtype=torch.uint8, device=device),
            "w2_s": torch.empty((n, H, I // 32), dtype=torch.uint8, device=device),
        }
    gen = torch.Generator(device=device)
    for j, e in enumerate(experts):
        gen.manual_seed(expert_seed(e, seed))
        w13 = (torch.randn((2 * I, H), generator=gen, dtype=torch.float32, device=device) * 0.02)
        w13 = w13.to(torch.bfloat16).to(torch.float32)
        p, s = _mxfp4_encode_torch(w13)
        out["w13"][j].copy_(p)
        out["w13_s"][j].copy_(s)
        del w13, p, s
        w2 = (torch.randn((H, I), generator=gen, dtype=torch.float32, device=device) * 0.02)
        w2 = w2.to(torch.bfloat16).to(torch.float32)
        p, s = _mxfp4_encode_torch(w2)
        out["w2"][j].copy_(p)
        out["w2_s"][j].copy_(s)
        del w2, p, s
    return out


def make_case(cfg: LayerConfig, seed: int = ROOT_SEED, device="cpu"):
    """Activations (numpy) + local-window weights (torch on ``device``)."""
    case = make_activations(cfg, seed)
    case.update(make_expert_weights(cfg, device=device, seed=seed))
    case["cfg"] = cfg
    return case

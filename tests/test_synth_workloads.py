"""The seeded workloads reproduce the shapes and routing structure the pages
state for their own benchmark (facts in tests/golden/kimi_k3_facts.json)."""
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kimi_k3_facts.json")


def _facts():
    return json.load(open(GOLDEN))


def test_ep_mixed_configs_match_the_pages_benchmark():
    f = _facts()["ep_mixed_benchmark"]
    ck = _facts()["ep_mapping"]
    cfgs = [c for c in synth.WORKLOADS.values() if c.routing == "ep_mixed"]
    assert [c.T for c in cfgs if c.T in f["M"]] == f["M"]
    for c in cfgs:
        assert (c.H, c.I, c.E, c.E_local, c.K) == (f["H"], f["I"], f["E"], f["E_local"], f["top_k"])
        assert c.E_local == ck["num_global"] // ck["ep"]
        assert c.expert_offset == f["ep_rank"] * c.E_local


def test_ep_mixed_configs_cover_the_real_size_decode_and_prefill():
    """The pages' coverage matrix runs the real-size shape at decode M = 1 and
    prefill M = 128; both are workloads here, and the rest of the ep_mixed
    workloads are the benchmark's batch sizes."""
    cov = _facts()["coverage_matrix"]
    bench = _facts()["ep_mixed_benchmark"]["M"]
    cfgs = [c for c in synth.WORKLOADS.values() if c.routing == "ep_mixed"]
    Ts = [c.T for c in cfgs]
    assert cov["decode_M"] in Ts and cov["prefill_M"] in Ts
    assert set(Ts) == set(bench) | {cov["decode_M"], cov["prefill_M"]}
    for c in cfgs:
        assert (c.H, c.I, c.E_local, c.K) == (cov["H"], cov["I"], cov["E_local"], cov["top_k"])


def test_ep_mixed_routing_structure():
    f = _facts()["ep_mixed_benchmark"]
    for c, avg in zip([c for c in synth.WORKLOADS.values() if c.routing == "ep_mixed"][:2],
                      f["avg_local_routes_per_expert"]):
        a = synth.make_activations(c)
        ids, w = a["topk_idx"], a["topk_w"]
        assert ids.shape == (c.T, c.K) and ids.dtype == np.int32 and w.dtype == np.float32
        local = (ids >= c.expert_offset) & (ids < c.expert_offset + c.E_local)
        assert np.all(local.sum(1) == f["local_slots"])
        assert all(len(set(row)) == c.K for row in ids)           # distinct experts per token
        assert ids.min() >= 0 and ids.max() < c.E
        assert np.all(w > 0) and np.allclose(w.sum(1), 1.0, atol=1e-6)
        per_expert = np.bincount(ids[local] - c.expert_offset, minlength=c.E_local)
        assert abs(per_expert.mean() - avg) < 0.05                # M * 8 / 28, as printed


def test_checkpoint_true_weight_shapes():
    """w13 = [w1; w3] and w2 of the local window have the checkpoint's shapes."""
    t = _facts()["checkpoint_expert_tensors"]
    c = synth.WORKLOADS["ckpt_ep32r7_M128"]
    small = synth.custom_config("shape", 0, T=1, H=c.H, I=c.I, E=c.E, K=1, E_local=1)
    w = synth.make_expert_weights(small, experts=[c.expert_offset])
    assert tuple(w["w13"].shape[1:]) == (2 * t["w1.weight_packed"][0], t["w1.weight_packed"][1])
    assert tuple(w["w13_s"].shape[1:]) == (2 * t["w1.weight_scale"][0], t["w1.weight_scale"][1])
    assert tuple(w["w2"].shape[1:]) == tuple(t["w2.weight_packed"])
    assert tuple(w["w2_s"].shape[1:]) == tuple(t["w2.weight_scale"])


def test_workload_table_names_keys_and_shapes():
    """Each workload keeps its seed-stream key and its shape, so every drawn
    input (and every stored figure measured on it) stays the same."""
    want = {
        "tiny": (0, 16, 128, 128, 4, 2, 4, 0),
        "decode_T8": (1, 8, 7168, 3584, 896, 16, 896, 0),
        "batched_decode_T256": (2, 256, 7168, 3584, 896, 16, 896, 0),
        "prefill_T8192": (3, 8192, 7168, 3584, 896, 16, 896, 0),
        "ep_share_T4096": (4, 4096, 7168, 3584, 896, 16, 224, 0),
        "ckpt_ep32r7_M128": (5, 128, 3584, 3072, 896, 16, 28, 196),
        "ckpt_ep32r7_M512": (6, 512, 3584, 3072, 896, 16, 28, 196),
        "ckpt_ep32r7_M2048": (7, 2048, 3584, 3072, 896, 16, 28, 196),
        "ckpt_ep32r7_M8192": (8, 8192, 3584, 3072, 896, 16, 28, 196),
        "ckpt_ep32r7_M1": (9, 1, 3584, 3072, 896, 16, 28, 196),
    }
    assert list(synth.WORKLOADS) == list(want)
    for name, c in synth.WORKLOADS.items():
        assert c.name == name
        assert (c.key, c.T, c.H, c.I, c.E, c.K, c.E_local, c.expert_offset) == want[name]

"""The seeded input generators: determinism, bf16 rounding, gap enforcement and the
capped-Zipf load of the prefill workload."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    a = a.astype(np.float32)
    ours = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_layer_is_deterministic_and_expert_streams_independent():
    sp = synth.spec("qwen", d=128, n_expert=16, ff=64, shared_ff=32)
    a = synth.make_layer(sp, seed=3)
    b = synth.make_layer(sp, seed=3)
    only = synth.make_layer(sp, seed=3, experts=[5, 9])
    for n in ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_gate_inp"):
        assert np.array_equal(a[n], b[n])
    for n in ("w_gate", "w_up", "w_down"):
        assert np.array_equal(only[n][[5, 9]], a[n][[5, 9]])
        assert not only[n][0].any()
    c = synth.make_layer(sp, seed=4)
    assert not np.array_equal(a["w_gate"], c["w_gate"])


@pytest.mark.parametrize("name,kw", [("qwen", dict(d=256)), ("gptoss", dict(d=192, ff=64)),
                                     ("tiny_f32", {})])
def test_gap_enforcement(name, kw):
    sp = synth.spec(name, **kw)
    L = synth.make_layer(sp, seed=0, experts=[])
    x = synth.make_tokens(L, 300, seed=0)
    z = synth.storage_to_f32(x).astype(np.float64) @ synth.storage_to_f32(L["w_router"]).astype(np.float64).T
    if L["b_router"] is not None:
        z += L["b_router"]
    top = -np.sort(-z, axis=1)[:, :sp.k + 1]
    assert np.all(top[:, :-1] - top[:, 1:] > 1e-3)
    assert np.array_equal(x, synth.make_tokens(L, 300, seed=0))


def test_zipf_targets_sum_to_k():
    q = synth.zipf_targets(256, 8, 1.1)
    assert abs(q.sum() - 8) < 1e-9 and q[0] == 1.0 and np.all(np.diff(q) <= 0)


def test_zipf_bias_realises_target_load():
    # Noise rows ~N(0,1) plus the bias: realised share per rank within sampling error.
    E, k = 256, 8
    b = synth.zipf_router_bias(E, k, 1.1).astype(np.float64)
    rank = synth.zipf_rank_of_expert(E)
    q = synth.zipf_targets(E, k, 1.1)
    rows = 20000
    z = np.random.default_rng(123).standard_normal((rows, E)) + b
    kth = -np.partition(-z, k - 1, axis=1)[:, k - 1:k]
    share = (z >= kth).sum(axis=0) / rows
    got = np.empty(E)
    got[rank] = share
    err = np.abs(got - q)
    # sampling error of the calibration (32768 noise rows) and of this check
    sigma = np.sqrt(q / 32768 + q / rows)
    assert np.all(err <= 0.03 * q + 5 * sigma), np.max(err / q)
    assert np.all(err[:16] <= 0.03 * q[:16] + 3 * sigma[:16])
    assert np.all(share > 0)


def test_q4k_layer_inputs():
    L = synth.make_layer(synth.spec("qwen_q4k", d=512, n_expert=4, ff=256, shared_ff=256), seed=0)
    assert L["w_gate"].shape == (4, 256, 2, 144) and L["w_gate"].dtype == np.uint8
    assert L["w_down"].shape == (4, 512, 1, 144)
    assert L["ws_gate"].dtype == np.uint16          # the shared expert stays bf16
    d = L["w_gate"][..., 0:2].copy().view("<f2").astype(np.float64)
    assert np.all(np.isfinite(d)) and np.all(d > 0)
    import oracle
    w = oracle.q4k_dequant(L["w_up"])
    assert 0.01 < w.std() < 0.04
    # The same seed gives the same bytes.
    L2 = synth.make_layer(synth.spec("qwen_q4k", d=512, n_expert=4, ff=256, shared_ff=256), seed=0)
    assert np.array_equal(L["w_down"], L2["w_down"])

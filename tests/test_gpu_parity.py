"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Small shapes span several blocks/tiles with ragged tails; the full workload shapes are
covered further down (routing on every token, outputs on every token or on a seeded
sample when the oracle would take too long).
"""
import numpy as np
import pytest

import oracle
from sparse_mixture_experts_amd import synth

from gpu_common import (SG_ATOL, W_ATOL, assert_close, assert_shell_close, case, layer_arrays, rel_err,
                        say, to_numpy_y)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mixture_experts_amd import moe
    moe.lib()


def moe_mod():
    from sparse_mixture_experts_amd import moe
    return moe


_DEV = {}


def dev_layer(name, seed=0, path="auto", **ov):
    key = (name, seed, tuple(sorted(ov.items())))
    if key not in _DEV:
        if len(_DEV) > 2:
            _DEV.clear()
            torch.cuda.empty_cache()
        _DEV[key] = moe_mod().Layer.from_arrays(layer_arrays(name, seed, **ov))
    lay = _DEV[key]
    return lay if path == "auto" else lay.with_path(path)


def xdev(x):
    return moe_mod().to_device(x)


# Small shapes: several blocks per kernel and ragged tails (T not a multiple of 4/64).
SMALL = [
    ("tiny_f32", {}, [1, 16, 77]),
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), [1, 5, 64, 150]),
    # Shared expert as wide as the routed ones, whole 256-column N-tiles.
    ("qwen", dict(d=512, n_expert=64, ff=256, shared_ff=256), [1, 5, 150, 300]),
    ("qwen_zipf", dict(d=512, ff=128, shared_ff=192), [300]),
    ("gptoss", dict(d=320, n_expert=16, ff=192), [1, 7, 100]),
    # K of 5.5 16-byte chunks per lane (a 6-chunk batch with a masked tail), on the up
    # projection (d) and on the down projection (ff).
    ("gptoss", dict(d=2816, n_expert=8, ff=192), [1, 5]),
    ("gptoss", dict(d=320, n_expert=8, ff=2816), [1, 5]),
    ("mixtral", dict(d=256, ff=448), [1, 3, 130]),
]
SMALL_CASES = [(n, ov, T) for n, ov, Ts in SMALL for T in Ts]


def _id(c):
    n, ov, T = c
    dims = "".join(f"-{key}{ov[key]}" for key in ("d", "ff") if key in ov)
    return f"{n}{dims}-T{T}"


@pytest.mark.parametrize("c", SMALL_CASES, ids=_id)
def test_route(c):
    name, ov, T = c
    say("route", name, ov, T)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, **ov)
    idx, w, sg = moe_mod().route(lay, xdev(x))
    torch.cuda.synchronize()
    ridx, rw, rsg = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= W_ATOL
    if rsg is not None:
        assert np.max(np.abs(sg.cpu().numpy() - rsg)) <= SG_ATOL


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (64, 8, 256), (65, 8, 256), (1000, 4, 32),
                                   (4097, 2, 8), (300, 8, 8), (200, 3, 500)])
def test_permute(T, k, E):
    say("permute", T, k, E)
    rng = np.random.default_rng(T * 7 + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, pt, pi = moe_mod().permute(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    counts, roff, rpt, rpi = oracle.permute(idx.astype(np.int64), E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(pt.cpu().numpy(), rpt)
    assert np.array_equal(pi.cpu().numpy(), rpi.reshape(-1))


def test_permute_ignores_out_of_range_ids():
    E, k, T = 16, 2, 70
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[5, 1] = -3
    idx[66, 0] = E + 4
    off, pt, pi = moe_mod().permute(torch.from_numpy(idx).cuda(), E)
    pi = pi.cpu().numpy()
    assert pi[5 * k + 1] == -1 and pi[66 * k] == -1
    assert off.cpu().numpy()[-1] == T * k - 2
    valid = np.ones(T * k, bool)
    valid[[5 * k + 1, 66 * k]] = False
    ref_counts = np.bincount(idx.reshape(-1)[valid], minlength=E)
    assert np.array_equal(np.diff(off.cpu().numpy()), ref_counts)
    assert np.array_equal(pt.cpu().numpy()[pi[valid]], np.repeat(np.arange(T), k)[valid])


@pytest.mark.parametrize("path", ["decode", "grouped"])
@pytest.mark.parametrize("c", SMALL_CASES, ids=_id)
def test_expert_ffn(c, path):
    name, ov, T = c
    if path == "grouped" and name == "tiny_f32":
        pytest.skip("grouped path is bf16-only")
    say("expert_ffn", name, ov, T, path)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, path=path, **ov)
    ridx, _, _ = oracle.route(L, x)
    _, roff, rpt, _ = oracle.permute(ridx, L["n_expert"])
    y = moe_mod().expert_ffn(lay, xdev(x), torch.from_numpy(roff.astype(np.int32)).cuda(),
                            torch.from_numpy(rpt.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    ref = oracle.expert_rows(L, x, roff, rpt)
    assert_close(y.cpu().numpy(), ref, L["dtype"], "y_perm")


@pytest.mark.parametrize("E,T", [(100, 1), (512, 1), (512, 40)])
def test_expert_ffn_expert_counts(E, T):
    # At one token the decode up GEMV finds each group from the expert offsets itself, one
    # wave scanning ceil(E / 64) experts per lane: a partial last lane (E = 100) and eight
    # experts per lane (the largest E), with most experts empty.  T = 40 takes the list
    # from the planning kernel.
    ov = dict(d=256, n_expert=E, ff=64, shared_ff=64)
    say("expert_ffn expert counts", ov, T)
    L, x = case("qwen", T, **ov)
    lay = dev_layer("qwen", path="decode", **ov)
    ridx, _, _ = oracle.route(L, x)
    _, roff, rpt, _ = oracle.permute(ridx, L["n_expert"])
    y = moe_mod().expert_ffn(lay, xdev(x), torch.from_numpy(roff.astype(np.int32)).cuda(),
                             torch.from_numpy(rpt.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert_close(y.cpu().numpy(), oracle.expert_rows(L, x, roff, rpt), L["dtype"], "y_perm")


@pytest.mark.parametrize("c", SMALL_CASES, ids=_id)
def test_combine_fed_oracle_rows(c):
    name, ov, T = c
    say("combine", name, ov, T)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, **ov)
    ridx, rw, rsg = oracle.route(L, x)
    _, roff, rpt, rpi = oracle.permute(ridx, L["n_expert"])
    yp = oracle.expert_rows(L, x, roff, rpt)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    y = moe_mod().combine(lay, f32(yp), torch.from_numpy(rpi.reshape(-1).astype(np.int32)).cuda(),
                         f32(rw), None if rsg is None else f32(rsg))
    torch.cuda.synchronize()
    # inputs rounded to fp32: compare against the oracle's combine of the same rounded rows
    ref = oracle.combine(yp.astype(np.float32).astype(np.float64), rpi, rw.astype(np.float32),
                         None if rsg is None else rsg.astype(np.float32))
    assert_close(to_numpy_y(y), ref, L["dtype"], "combine")


@pytest.mark.parametrize("path", ["auto", "decode", "grouped"])
@pytest.mark.parametrize("c", SMALL_CASES, ids=_id)
def test_forward(c, path):
    name, ov, T = c
    if path == "grouped" and name == "tiny_f32":
        pytest.skip("grouped path is bf16-only")
    say("forward", name, ov, T, path)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, path=path, **ov)
    y = moe_mod().forward(lay, xdev(x))
    torch.cuda.synchronize()
    ref = oracle.moe_forward(L, x)
    e = assert_close(to_numpy_y(y), ref, L["dtype"], "y")
    say(f"  rel err {e:.2e}")


# ----------------------------------------------------------------------------- edge cases

def test_zero_tokens():
    lay = dev_layer("tiny_f32")
    x = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    y = moe_mod().forward(lay, x, ws=torch.empty(1, dtype=torch.uint8, device="cuda"))
    assert y.shape == (0, 256)


def _custom(L):
    return moe_mod().Layer.from_arrays(L)


def test_k_equals_E_dense_case():
    L = dict(layer_arrays("tiny_f32", k=8))
    x = synth.make_tokens(L, 33, seed=4)
    y = moe_mod().forward(_custom(L), xdev(x))
    assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "f32", "k=E")


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_k_equals_E_bf16(path):
    # Every expert selected by every token (k = E): each group holds all T rows, several
    # M-tiles per expert on the grouped path; the shared expert on top.
    L = dict(layer_arrays("qwen", d=256, n_expert=16, k=16, ff=128, shared_ff=64))
    x = synth.make_tokens(L, 150, seed=14)
    lay = _custom(L).with_path(path)
    idx, _, _ = moe_mod().route(lay, xdev(x))
    ridx, _, _ = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    y = moe_mod().forward(lay, xdev(x))
    assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", f"k=E {path}")


def test_one_expert_takes_every_token():
    L = dict(layer_arrays("qwen", d=256, n_expert=32, ff=128, shared_ff=64))
    L["w_router"] = np.zeros_like(L["w_router"])
    b = np.zeros(32, np.float32)
    b[13] = 100.0
    L["b_router"] = b
    L["k"] = 1
    x = synth.make_tokens(L, 200, seed=5, gap=0)
    for path in ("decode", "grouped"):
        lay = _custom(L).with_path(path)
        idx, w, _ = moe_mod().route(lay, xdev(x))
        assert (idx.cpu().numpy() == 13).all() and (w.cpu().numpy() == 1.0).all()
        y = moe_mod().forward(lay, xdev(x))
        assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", path)


@pytest.mark.parametrize("T", [9, 40, 200])
def test_all_tie_router_bit_exact(T):
    # T = 9: top-k inside the decode routing block; 40: its own launch; 200: MFMA router.
    L = dict(layer_arrays("qwen", d=256, n_expert=32, ff=128, shared_ff=64))
    L["w_router"] = np.zeros_like(L["w_router"])
    x = synth.make_tokens(L, T, seed=6, gap=0)
    idx, w, _ = moe_mod().route(_custom(L), xdev(x))
    assert (idx.cpu().numpy() == np.arange(8)).all()
    assert (w.cpu().numpy() == np.float32(1.0 / 8)).all()


@pytest.mark.parametrize("T", [5, 40, 300])
def test_masked_experts(T):
    # A router bias of -inf masks all experts but two: top-4 takes those two, then the
    # two lowest-index masked experts with weight exactly 0.
    L = dict(layer_arrays("gptoss", d=320, n_expert=16, ff=192))
    b = np.full(16, -np.inf, np.float32)
    b[[3, 11]] = 0.0
    L["b_router"] = b
    # Keep tokens whose two live logits differ by more than 1e-3 (the usual gap rule).
    x = synth.make_tokens(L, 2 * T + 8, seed=9, gap=0)
    z = oracle.router_logits(L, x)
    x = x[np.abs(z[:, 3] - z[:, 11]) > 1e-3][:T]
    assert x.shape[0] == T
    lay = _custom(L)
    idx, w, _ = moe_mod().route(lay, xdev(x))
    ridx, rw, _ = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert (np.sort(ridx[:, 2:], axis=1) == [0, 1]).all()
    assert (w.cpu().numpy()[:, 2:] == 0).all()
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= W_ATOL
    y = moe_mod().forward(lay, xdev(x))
    assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "masked experts")


@pytest.mark.parametrize("T", [3, 40, 300])
def test_nan_logits_rank_last(T):
    # A token whose input holds a NaN has NaN logits only; NaN ranks below every number
    # and ties go to the lower index, so its picks are experts 0..k-1 (the oracle's
    # stable sort puts NaN last as well).  Other tokens are unaffected.
    L = dict(layer_arrays("qwen", d=256, n_expert=32, ff=128, shared_ff=64))
    x = synth.make_tokens(L, T, seed=10).copy()
    x[1, 17] = 0x7FC0  # bf16 quiet NaN
    idx, _, _ = moe_mod().route(_custom(L), xdev(x))
    ridx, _, _ = oracle.route(L, x)
    got = idx.cpu().numpy()
    assert (ridx[1] == np.arange(8)).all()
    assert np.array_equal(got, ridx)


def test_identical_experts():
    L = dict(layer_arrays("qwen", d=256, n_expert=16, ff=128, shared_ff=64))
    for n in ("w_gate", "w_up", "w_down"):
        L[n] = np.broadcast_to(L[n][:1], L[n].shape).copy()
    x = synth.make_tokens(L, 40, seed=7)
    y = moe_mod().forward(_custom(L), xdev(x))
    assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "identical experts")


def test_oai_clamp_coverage():
    # Larger gate_up weights (std 0.4 at d=320: pre-activations ~N(0, 7.2^2)) so that
    # |gate| and |up| exceed the limit often.
    sp = synth.spec("gptoss", d=320, n_expert=16, ff=192, weight_std=0.4)
    L = synth.make_layer(sp, seed=3)
    x = synth.make_tokens(L, 50, seed=8)
    xf = synth.storage_to_f32(x).astype(np.float64)
    v = xf @ synth.storage_to_f32(L["w_gate_up"][0]).astype(np.float64).T
    assert (v[:, 0::2] > 7).mean() > 0.05 and (np.abs(v[:, 1::2]) > 7).mean() > 0.05
    for path in ("decode", "grouped"):
        y = moe_mod().forward(_custom(L).with_path(path), xdev(x))
        assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "clamp " + path)


def test_deterministic():
    L, x = case("qwen", 64, d=512, n_expert=64, ff=192, shared_ff=128)
    lay = dev_layer("qwen", d=512, n_expert=64, ff=192, shared_ff=128)
    for path in ("decode", "grouped"):
        a = moe_mod().forward(lay.with_path(path), xdev(x))
        b = moe_mod().forward(lay.with_path(path), xdev(x))
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,expect", [(4, "decode"), (12, "decode"), (16, "grouped"), (40, "grouped")])
def test_auto_path_rows_per_expert(T, expect):
    # AUTO takes the grouped MFMA path at or below 64 tokens once the expected rows per
    # active expert, T*k / (E * (1 - (1 - k/E)^T)), reach 4 (E = 8, k = 2: from T = 16 on);
    # the paths round differently, so the output matches the forced path bit for bit.
    ov = dict(d=256, ff=448)
    say("auto path", T, expect)
    L, x = case("mixtral", T, **ov)
    lay = dev_layer("mixtral", **ov)
    auto = moe_mod().forward(lay, xdev(x))
    forced = moe_mod().forward(lay.with_path(expect), xdev(x))
    other = moe_mod().forward(lay.with_path("grouped" if expect == "decode" else "decode"), xdev(x))
    assert torch.equal(auto, forced)
    assert not torch.equal(auto, other)
    assert_close(to_numpy_y(auto), oracle.moe_forward(L, x), "bf16", "y")


def test_batch_invariance():
    # Rows of a batch equal the same tokens run alone (the batched-decode check of the
    # "Llama Forward Pass" page, applied to the MoE layer).
    ov = dict(d=512, n_expert=64, ff=192, shared_ff=128)
    L, x = case("qwen", 100, **ov)
    lay = dev_layer("qwen", **ov)
    full = moe_mod().forward(lay, xdev(x))
    idx_full, _, _ = moe_mod().route(lay, xdev(x))
    for t in (0, 37, 99):
        one = moe_mod().forward(lay, xdev(x[t:t + 1]))
        idx_one, _, _ = moe_mod().route(lay, xdev(x[t:t + 1]))
        assert torch.equal(idx_one[0], idx_full[t])
        assert rel_err(to_numpy_y(one)[0], to_numpy_y(full)[t]) <= 2e-2


# Token independence, bit for bit: on the grouped path every output element's sums run in
# a fixed order whatever the other tokens of the batch and the row's place in its expert's
# tile, so permuting the batch permutes the output rows exactly (routing included).  (The
# page's batched-versus-sequential pattern crosses paths here -- one token takes the GEMV
# kernels -- and is checked within tolerance by test_batch_invariance above.)
@pytest.mark.parametrize("name,ov,T", [
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), 150),
    ("gptoss", dict(d=320, n_expert=16, ff=192), 100),
    ("gptoss_mx", dict(d=320, n_expert=16, ff=192), 100),
    ("qwen_q4k", dict(d=512, n_expert=16, ff=256, shared_ff=256), 300),
], ids=lambda v: v if isinstance(v, str) else (str(v) if isinstance(v, int) else ""))
def test_grouped_token_permutation_bitwise(name, ov, T):
    say("permutation", name, ov, T)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, path="grouped", **ov)
    perm = np.random.default_rng(5).permutation(T)
    y = moe_mod().forward(lay, xdev(x))
    yp = moe_mod().forward(lay, xdev(np.ascontiguousarray(x[perm])))
    idx, _, _ = moe_mod().route(lay, xdev(x))
    idxp, _, _ = moe_mod().route(lay, xdev(np.ascontiguousarray(x[perm])))
    torch.cuda.synchronize()
    pt = torch.as_tensor(perm, device=y.device)
    assert torch.equal(idxp, idx[pt])
    assert torch.equal(yp, y[pt])


# The same on the decode path: each hidden and output row is a fixed-order sum over its
# own token's activations (rows of a group are served one by one from the same decoded
# weights, and the cross-lane reductions pair lanes the same way for every row), so a
# permuted batch of the same size gives the permuted output, bit for bit.
@pytest.mark.parametrize("name,ov,T", [
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), 8),
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), 50),
    ("gptoss_mx", dict(d=320, n_expert=16, ff=192), 8),
    ("gptoss_mx", dict(d=320, n_expert=16, ff=192), 50),
    ("qwen_q4k", dict(d=512, n_expert=16, ff=256, shared_ff=256), 8),
    ("qwen_q4k", dict(d=512, n_expert=16, ff=256, shared_ff=256), 50),
], ids=lambda v: v if isinstance(v, str) else (str(v) if isinstance(v, int) else ""))
def test_decode_token_permutation_bitwise(name, ov, T):
    say("decode permutation", name, ov, T)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, path="decode", **ov)
    perm = np.random.default_rng(6).permutation(T)
    y = moe_mod().forward(lay, xdev(x))
    yp = moe_mod().forward(lay, xdev(np.ascontiguousarray(x[perm])))
    torch.cuda.synchronize()
    assert torch.equal(yp, y[torch.as_tensor(perm, device=y.device)])


# ----------------------------------------------------------------------------- full sizes

@pytest.mark.parametrize("T", [1, 8, 64])
def test_full_qwen_decode(T):
    say("full qwen decode", T)
    L, x = case("qwen", T)
    lay = dev_layer("qwen")
    idx, w, sg = moe_mod().route(lay, xdev(x))
    y = moe_mod().forward(lay, xdev(x))
    torch.cuda.synchronize()
    ridx, rw, rsg = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= W_ATOL
    assert np.max(np.abs(sg.cpu().numpy() - rsg)) <= SG_ATOL
    e = assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "y")
    say(f"  rel err {e:.2e}")


def test_full_qwen_prefill_zipf():
    T = 8192
    say("full qwen prefill", T)
    L, x = case("qwen_zipf", T)
    lay = dev_layer("qwen_zipf")
    idx, w, sg = moe_mod().route(lay, xdev(x))
    y = moe_mod().forward(lay, xdev(x))
    torch.cuda.synchronize()
    ridx, rw, rsg = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= W_ATOL
    counts = np.bincount(ridx.reshape(-1), minlength=256)
    say("  counts min/median/max", counts.min(), int(np.median(counts)), counts.max())
    e = assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "y")
    say(f"  rel err {e:.2e}")
    # As benchmarked: with the grouped copy of the down weights, bit for bit the same.
    y_pack = moe_mod().forward(lay.with_grouped_pack(), xdev(x))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_pack.view(torch.int16))


@pytest.mark.parametrize("name,T,sample", [("gptoss", 1, None), ("gptoss", 4096, 256),
                                           ("mixtral", 16, None), ("mixtral", 16384, 512),
                                           ("gptoss_mx", 1, None), ("gptoss_mx", 64, None),
                                           ("gptoss_mx", 1000, 128), ("qwen_q4k", 1, None),
                                           ("qwen_q4k", 8, None), ("qwen_q4k", 64, None), ("qwen_q4k", 2048, 128)])
def test_full_other_layers(name, T, sample):
    say("full", name, T)
    L, x = case(name, T)
    lay = dev_layer(name)
    idx, w, _ = moe_mod().route(lay, xdev(x))
    y = moe_mod().forward(lay, xdev(x))
    torch.cuda.synchronize()
    ridx, rw, _ = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= W_ATOL
    yn = to_numpy_y(y)
    if sample is None:
        ref, got = oracle.moe_forward(L, x), yn
    else:
        tok = np.sort(np.random.default_rng(11).choice(T, sample, replace=False))
        ref, got = oracle.moe_forward(L, x[tok]), yn[tok]
    e = assert_close(got, ref, "bf16", "y")
    say(f"  rel err {e:.2e}")


def test_grouped_many_tiles():
    # 4096 tokens, 64 experts of 256 units, shared expert: ~290 M-tiles x 2 N-tiles, more
    # tiles than blocks in flight and several M-tiles per expert.  Rows of the expert stage
    # (fp32) and the layer output are compared on a seeded sample of tokens.
    ov = dict(d=512, n_expert=64, ff=256, shared_ff=256)
    T = 4096
    say("grouped many tiles", ov, T)
    L, x = case("qwen", T, **ov)
    lay = dev_layer("qwen", **ov)
    ridx, rw, rsg = oracle.route(L, x)
    idx, _, _ = moe_mod().route(lay, xdev(x))
    assert np.array_equal(idx.cpu().numpy(), ridx)
    _, roff, rpt, rinv = oracle.permute(ridx, L["n_expert"])
    yp = moe_mod().expert_ffn(lay, xdev(x), torch.from_numpy(roff.astype(np.int32)).cuda(),
                             torch.from_numpy(rpt.astype(np.int32)).cuda()).cpu().numpy()
    y = to_numpy_y(moe_mod().forward(lay, xdev(x)))
    tok = np.sort(np.random.default_rng(12).choice(T, 192, replace=False))
    # Expert rows of the sampled tokens: their k routed rows and their shared row.
    rows = np.concatenate([rinv[tok].reshape(-1), T * L["k"] + tok])
    ref_rows = np.concatenate([
        np.stack([oracle.expert_apply(L, int(ridx[t, j]), oracle.widen(x[t:t + 1]))[0]
                  for t in tok for j in range(L["k"])]),
        oracle.swiglu_ffn(oracle.widen(x[tok]), oracle.widen(L["ws_gate"]), oracle.widen(L["ws_up"]),
                          oracle.widen(L["ws_down"]))])
    assert_close(yp[rows], ref_rows, "bf16", "expert rows")
    assert_close(y[tok], oracle.moe_forward(L, x[tok]), "bf16", "y")


def test_max_tokens():
    # The largest batch the library accepts, 2^22 tokens, on a small layer: 8M routed rows
    # and 4M shared rows, so the grouping, the offsets, the M-tile map and every row index
    # are at their largest.  Routing and grouping are compared on every token (bit-exact),
    # the output on a seeded sample that includes the last token.  The same layer at 300
    # tokens first.
    ov = dict(d=64, n_expert=8, k=2, ff=64, shared_ff=64)
    T = 1 << 22
    L = layer_arrays("qwen", 0, **ov)
    lay = dev_layer("qwen", **ov)
    xs = synth.make_tokens(L, 300, seed=101)
    assert_close(to_numpy_y(moe_mod().forward(lay, xdev(xs))), oracle.moe_forward(L, xs), "bf16", "y (300)")
    say("max tokens", ov, T)
    x = synth.make_tokens(L, T, seed=100)
    xd = xdev(x)
    idx, _, _ = moe_mod().route(lay, xd)
    off, pt, pinv = moe_mod().permute(idx, L["n_expert"])
    y = moe_mod().forward(lay, xd)
    torch.cuda.synchronize()
    ridx, _, _ = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    counts, roff, rpt, rinv = oracle.permute(ridx, L["n_expert"])
    say("  counts", counts.tolist())
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(pt.cpu().numpy(), rpt) and np.array_equal(pinv.cpu().numpy(), rinv.reshape(-1))
    tok = np.concatenate([np.sort(np.random.default_rng(13).choice(T - 1, 255, replace=False)), [T - 1]])
    got = to_numpy_y(y[torch.from_numpy(tok).to(y.device)])
    e = assert_close(got, oracle.moe_forward(L, x[tok]), "bf16", "y (sample)")
    say(f"  rel err {e:.2e}")


# ----------------------------------------------------------------------------- layer shell

EPS = 1e-5
SHELL = [
    ("tiny_f32", {}, [1, 16, 77]),
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), [1, 5, 64, 150]),
    ("gptoss", dict(d=320, n_expert=16, ff=192), [1, 7, 100]),
    # K of 5.5 16-byte chunks per lane (a 6-chunk batch with a masked tail), on the up
    # projection (d) and on the down projection (ff).
    ("gptoss", dict(d=2816, n_expert=8, ff=192), [1, 5]),
    ("gptoss", dict(d=320, n_expert=8, ff=2816), [1, 5]),
]
SHELL_CASES = [(n, ov, T) for n, ov, Ts in SHELL for T in Ts]


def shell_case(name, T, **ov):
    L = layer_arrays(name, 0, **ov)
    w = synth.make_norm_weight(L, seed=7)

    def view(rows):
        return oracle.store_activation(oracle.rmsnorm(rows, w, EPS), L["dtype"])

    # bf16: small residual magnitudes keep the block's part visible after the rounding of
    # the sum; the rows still span a factor 16 for the norm.
    scale = 2.0 ** -4 if L["dtype"] == "bf16" else 1.0
    h = synth.make_hidden(L, T, seed=8, router_view=view, scale=scale)
    return L, w, h


@pytest.mark.parametrize("path", ["auto", "grouped"])
@pytest.mark.parametrize("c", SHELL_CASES, ids=_id)
def test_forward_shell(c, path):
    name, ov, T = c
    if path == "grouped" and name == "tiny_f32":
        pytest.skip("grouped path is bf16-only")
    say("shell", name, ov, T, path)
    L, w, h = shell_case(name, T, **ov)
    lay = dev_layer(name, path=path, **ov)
    out = moe_mod().forward_shell(lay, xdev(h), xdev(w), EPS)
    torch.cuda.synchronize()
    ref = oracle.moe_shell(L, h, w, EPS)
    e = assert_shell_close(to_numpy_y(out), ref, oracle.widen(h), L["dtype"], "shell")
    say(f"  block part rel err {e:.2e}")


@pytest.mark.parametrize("T", [1, 5, 64, 150])
def test_forward_shell_in_place(T):
    ov = dict(d=512, n_expert=64, ff=192, shared_ff=128)
    say("shell in place", T)
    L, w, h = shell_case("qwen", T, **ov)
    lay = dev_layer("qwen", **ov)
    wd = xdev(w)
    apart = moe_mod().forward_shell(lay, xdev(h), wd, EPS)
    hd = xdev(h)
    same = moe_mod().forward_shell(lay, hd, wd, EPS, out=hd)
    torch.cuda.synchronize()
    assert same.data_ptr() == hd.data_ptr()
    assert torch.equal(same, apart)


@pytest.mark.parametrize("T", [1, 64])
def test_full_qwen_shell(T):
    say("full qwen shell", T)
    L, w, h = shell_case("qwen", T)
    lay = dev_layer("qwen")
    out = moe_mod().forward_shell(lay, xdev(h), xdev(w), EPS)
    torch.cuda.synchronize()
    ref = oracle.moe_shell(L, h, w, EPS)
    e = assert_shell_close(to_numpy_y(out), ref, oracle.widen(h), "bf16", "shell")
    say(f"  block part rel err {e:.2e}")


# ----------------------------------------------------------------------------- grouped copy, dense

def dense_pack_expected(L):
    """The grouped copy of a dense bf16 layer (its down weights), built with numpy: routed
    W_d as [E][NTd][ff/32][256][32] (NTd = ceil(d/256); tile row r of N-tile nt is output
    row min(nt * 256 + r, d - 1); slice s holds inputs 32s .. 32s+31), then, 256-byte
    aligned, the shared expert's W_d as [NTd][shared_ff/32][256][32]."""
    d = L["d"]
    ntd = -(-d // 256)
    n = np.minimum(np.arange(ntd)[:, None] * 256 + np.arange(256)[None, :], d - 1)   # [NTd, 256]

    def part(w):  # w [E, d, K] -> [E, NTd, K/32, 256, 32]
        E, _, K = w.shape
        return w.reshape(E, d, K // 32, 32)[:, n].transpose(0, 1, 3, 2, 4)

    routed = np.ascontiguousarray(part(L["w_down"])).reshape(-1)
    out = [(0, routed)]
    if L["shared_ff"]:
        out.append((-(-routed.size * 2 // 256) * 256 // 2, np.ascontiguousarray(part(L["ws_down"][None])).reshape(-1)))
    total = out[-1][0] + out[-1][1].size
    return out, total


DENSE_PACK = [("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128)),
              ("gptoss", dict(d=320, n_expert=16, ff=192)),
              ("mixtral", dict(d=512, ff=1024))]


@pytest.mark.parametrize("name,ov", DENSE_PACK, ids=["qwen", "gptoss_d320", "mixtral"])
def test_dense_grouped_pack_layout(name, ov):
    # Byte for byte the layout above (d = 320 leaves a partial N-tile).
    say("dense grouped pack layout", name, ov)
    L, _ = case(name, 1, **ov)
    lay = dev_layer(name, **ov).with_grouped_pack()
    torch.cuda.synchronize()
    got = lay.tensors["grouped_pack"].view(torch.int16).cpu().numpy().view(np.uint16)
    regions, total = dense_pack_expected(L)
    assert got.size == total
    for off, want in regions:
        assert np.array_equal(got[off:off + want.size], want), off


@pytest.mark.parametrize("T", [7, 100, 300])
@pytest.mark.parametrize("name,ov", DENSE_PACK, ids=["qwen", "gptoss_d320", "mixtral"])
def test_dense_grouped_pack_forward(name, ov, T):
    # The grouped path (forced; T = 7 takes split-K down tiles) on the grouped copy: bit for
    # bit the output of the weights in place, and within tolerance of the oracle; and the
    # expert stage's fp32 rows (the other down-kernel instance) bit for bit too.
    say("dense grouped forward, grouped copy", name, ov, T)
    L, x = case(name, T, **ov)
    lay = dev_layer(name, **ov).with_path("grouped")
    pk = lay.with_grouped_pack()
    y0 = moe_mod().forward(lay, xdev(x))
    y1 = moe_mod().forward(pk, xdev(x))
    idx, _, _ = moe_mod().route(lay, xdev(x))
    off, pt, _ = moe_mod().permute(idx, L["n_expert"])
    r0 = moe_mod().expert_ffn(lay, xdev(x), off, pt)
    r1 = moe_mod().expert_ffn(pk, xdev(x), off, pt)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(r0, r1)
    assert_close(to_numpy_y(y1), oracle.moe_forward(L, x), "bf16", "y")


@pytest.mark.parametrize("name,T", [("gptoss", 4096), ("mixtral", 16384)])
def test_full_dense_grouped_pack(name, T):
    # The full layers as benchmarked: with the grouped copy, bit for bit the output of the
    # weights in place (which test_full_other_layers checks against the oracle).
    say("full dense grouped copy", name, T)
    L, x = case(name, T)
    lay = dev_layer(name)
    y0 = moe_mod().forward(lay, xdev(x))
    y1 = moe_mod().forward(lay.with_grouped_pack(), xdev(x))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


# ----------------------------------------------------------------------------- MXFP4 experts

MX_SMALL = [dict(d=320, n_expert=16, ff=192), dict(d=4096, n_expert=8, ff=128, k=2)]


@pytest.mark.parametrize("T", [1, 7, 100])
@pytest.mark.parametrize("ov", MX_SMALL, ids=["d320", "d4096"])
def test_mxfp4_forward(ov, T):
    say("mxfp4 forward", ov, T)
    L, x = case("gptoss_mx", T, **ov)
    lay = dev_layer("gptoss_mx", **ov)
    y = moe_mod().forward(lay, xdev(x))
    torch.cuda.synchronize()
    e = assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "y")
    say(f"  rel err {e:.2e}")


def test_mxfp4_expert_ffn_rows():
    # The expert stage alone through the ABI: unweighted rows of every (token, pick) pair.
    ov = MX_SMALL[0]
    L, x = case("gptoss_mx", 37, **ov)
    lay = dev_layer("gptoss_mx", **ov)
    idx, _, _ = moe_mod().route(lay, xdev(x))
    off, pt, pi = moe_mod().permute(idx, L["n_expert"])
    yp = moe_mod().expert_ffn(lay, xdev(x), off, pt)
    torch.cuda.synchronize()
    ridx, _, _ = oracle.route(L, x)
    _, roff, rpt, _ = oracle.permute(ridx, L["n_expert"])
    assert np.array_equal(off.cpu().numpy(), roff) and np.array_equal(pt.cpu().numpy(), rpt)
    ref = oracle.expert_rows(L, x, roff, rpt)
    assert_close(to_numpy_y(yp), ref, "bf16", "rows")


def test_mxfp4_shell():
    ov = MX_SMALL[0]
    for T in (1, 64, 100):
        L, w, h = shell_case("gptoss_mx", T, **ov)
        lay = dev_layer("gptoss_mx", **ov)
        out = moe_mod().forward_shell(lay, xdev(h), xdev(w), EPS)
        torch.cuda.synchronize()
        ref = oracle.moe_shell(L, h, w, EPS)
        assert_shell_close(to_numpy_y(out), ref, oracle.widen(h), "bf16", f"mx shell T={T}")


@pytest.mark.parametrize("T", [1, 7, 100, 300])
@pytest.mark.parametrize("ov", MX_SMALL, ids=["d320", "d4096"])
def test_mxfp4_grouped_forward(ov, T):
    # The grouped MFMA path with the FP4 blocks expanded into LDS (forced at every T; T=7
    # takes split-K down tiles), against the oracle on the dequantised weights.
    say("mxfp4 grouped forward", ov, T)
    L, x = case("gptoss_mx", T, **ov)
    lay = dev_layer("gptoss_mx", **ov)
    y = moe_mod().forward(lay.with_path("grouped"), xdev(x))
    torch.cuda.synchronize()
    e = assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "y")
    say(f"  rel err {e:.2e}")


def test_mxfp4_grouped_expert_ffn_rows():
    # Unweighted expert rows of the grouped path (fp32 output tiles), several M-tiles per
    # expert and a ragged last tile.
    ov = MX_SMALL[0]
    L, x = case("gptoss_mx", 333, **ov)
    lay = dev_layer("gptoss_mx", **ov).with_path("grouped")
    idx, _, _ = moe_mod().route(lay, xdev(x))
    off, pt, _ = moe_mod().permute(idx, L["n_expert"])
    yp = moe_mod().expert_ffn(lay, xdev(x), off, pt)
    torch.cuda.synchronize()
    ridx, _, _ = oracle.route(L, x)
    _, roff, rpt, _ = oracle.permute(ridx, L["n_expert"])
    assert np.array_equal(off.cpu().numpy(), roff) and np.array_equal(pt.cpu().numpy(), rpt)
    assert_close(to_numpy_y(yp), oracle.expert_rows(L, x, roff, rpt), "bf16", "rows")


def mx_pack_expected(L):
    """The grouped copy of an MXFP4 layer's expert weights, built with numpy from the
    checkpoint arrays: regions [up codes | up scales | down codes | down scales], each
    256-byte aligned.  Up piece ((e * NTu + nt) * Su + s) * 512 + t is block 2s + t % 2 of
    gate_up row 2f (t / 2 < 128) or 2f + 1 (else), f = min(nt * 128 + (t / 2) % 128, ff - 1);
    down piece ((e * NTd + nt) * Sd + s) * 256 + r is block s of W_d row min(nt * 256 + r,
    d - 1).  Returns [(offset, bytes)] per region."""
    E, d, ff = L["n_expert"], L["d"], L["ff"]
    ntu, su, ntd, sdn = -(-ff // 128), d // 64, -(-d // 256), ff // 32
    t = np.arange(512)
    r = t // 2
    f = np.minimum(np.arange(ntu)[:, None] * 128 + (r % 128)[None, :], ff - 1)
    R = 2 * f + (r >= 128)[None, :]                                   # [ntu, 512]
    blk = 2 * np.arange(su)[:, None] + (t % 2)[None, :]               # [su, 512]
    up_c = L["w_gate_up"][:, R[:, None, :], blk[None, :, :]]          # [E, ntu, su, 512, 16]
    up_s = L["w_gate_up_scales"][:, R[:, None, :], blk[None, :, :]]   # [E, ntu, su, 512]
    n = np.minimum(np.arange(ntd)[:, None] * 256 + np.arange(256)[None, :], d - 1)  # [ntd, 256]
    sl = np.arange(sdn)
    dn_c = L["w_down"][:, n[:, None, :], sl[None, :, None]]           # [E, ntd, sdn, 256, 16]
    dn_s = L["w_down_scales"][:, n[:, None, :], sl[None, :, None]]    # [E, ntd, sdn, 256]
    out, off = [], 0
    for a in (up_c, up_s, dn_c, dn_s):
        b = np.ascontiguousarray(a, dtype=np.uint8).reshape(-1)
        out.append((off, b))
        off += -(-b.size // 256) * 256
    assert up_c.shape == (E, ntu, su, 512, 16) and dn_c.shape == (E, ntd, sdn, 256, 16)
    return out, off


@pytest.mark.parametrize("ov", MX_SMALL, ids=["d320", "d4096"])
def test_mxfp4_grouped_pack_layout(ov):
    # moe_grouped_pack writes, byte for byte, the layout described above (partial N-tiles
    # of both GEMMs included: ff = 192 leaves half an up tile, d = 320 a partial down tile).
    say("mxfp4 grouped pack layout", ov)
    L, _ = case("gptoss_mx", 1, **ov)
    lay = dev_layer("gptoss_mx", **ov).with_grouped_pack()
    torch.cuda.synchronize()
    got = lay.tensors["grouped_pack"].cpu().numpy()
    regions, total = mx_pack_expected(L)
    assert got.size == total
    for off, want in regions:
        assert np.array_equal(got[off:off + want.size], want), off


@pytest.mark.parametrize("T", [7, 100, 300])
@pytest.mark.parametrize("ov", MX_SMALL, ids=["d320", "d4096"])
def test_mxfp4_grouped_pack_forward(ov, T):
    # The grouped path on the grouped copy: bit for bit the output of the checkpoint layout
    # (same codes, scales and sums; T = 7 takes split-K down tiles), and within tolerance of
    # the oracle.
    say("mxfp4 grouped forward, grouped copy", ov, T)
    L, x = case("gptoss_mx", T, **ov)
    lay = dev_layer("gptoss_mx", **ov).with_path("grouped")
    y0 = moe_mod().forward(lay, xdev(x))
    y1 = moe_mod().forward(lay.with_grouped_pack(), xdev(x))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert_close(to_numpy_y(y1), oracle.moe_forward(L, x), "bf16", "y")


def test_mxfp4_full_grouped_pack():
    # The full gpt-oss-shaped MXFP4 layer at 4096 tokens as the benchmark runs it (grouped
    # copy), on a seeded sample of tokens.
    T, sample = 4096, 128
    say("full gptoss_mx grouped copy", T)
    L, x = case("gptoss_mx", T)
    lay = dev_layer("gptoss_mx").with_grouped_pack()
    y = to_numpy_y(moe_mod().forward(lay, xdev(x)))
    tok = np.sort(np.random.default_rng(11).choice(T, sample, replace=False))
    e = assert_close(y[tok], oracle.moe_forward(L, x[tok]), "bf16", "y")
    say(f"  rel err {e:.2e}")


# ----------------------------------------------------------------------------- Q4_K experts

# Rows of 8, 12 (a ragged lane group of 16) and 64 quant runs per lane group on the up
# projection; 4 and 8 on the down projection; a bf16 shared expert as wide as the routed
# experts (served by the Q4_K GEMVs), one twice as wide (dense GEMVs), and none.
Q4K_SMALL = [dict(d=512, n_expert=16, ff=256, shared_ff=256),
             dict(d=768, n_expert=8, ff=512, k=2, shared_ff=0),
             dict(d=4096, n_expert=4, ff=256, k=2, shared_ff=256),
             dict(d=512, n_expert=16, ff=256, shared_ff=512)]
Q4K_IDS = ["d512", "d768", "d4096", "d512_sh512"]


@pytest.mark.parametrize("T", [1, 7, 100])
@pytest.mark.parametrize("ov", Q4K_SMALL, ids=Q4K_IDS)
def test_q4k_forward(ov, T):
    say("q4k forward", ov, T)
    L, x = case("qwen_q4k", T, **ov)
    lay = dev_layer("qwen_q4k", **ov)
    idx, _, _ = moe_mod().route(lay, xdev(x))
    y = moe_mod().forward(lay, xdev(x))
    torch.cuda.synchronize()
    ridx, _, _ = oracle.route(L, x)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    e = assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "y")
    say(f"  rel err {e:.2e}")


@pytest.mark.parametrize("path", ["decode", "grouped"])
@pytest.mark.parametrize("T", [1, 7, 100, 300])
@pytest.mark.parametrize("ov", Q4K_SMALL, ids=Q4K_IDS)
def test_q4k_forced_path(ov, T, path):
    # Both kernel families at every batch size: the GEMVs with several rows per group, the
    # grouped MFMA path with the super-blocks expanded into LDS (T=7: split-K down tiles).
    say("q4k", path, ov, T)
    L, x = case("qwen_q4k", T, **ov)
    lay = dev_layer("qwen_q4k", **ov)
    y = moe_mod().forward(lay.with_path(path), xdev(x))
    torch.cuda.synchronize()
    e = assert_close(to_numpy_y(y), oracle.moe_forward(L, x), "bf16", "y")
    say(f"  rel err {e:.2e}")


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_q4k_expert_ffn_rows(path):
    # Unweighted expert rows (fp32) through the ABI, including the shared expert's rows.
    ov = Q4K_SMALL[0]
    L, x = case("qwen_q4k", 133, **ov)
    lay = dev_layer("qwen_q4k", **ov).with_path(path)
    idx, _, _ = moe_mod().route(lay, xdev(x))
    off, pt, _ = moe_mod().permute(idx, L["n_expert"])
    yp = moe_mod().expert_ffn(lay, xdev(x), off, pt)
    torch.cuda.synchronize()
    ridx, _, _ = oracle.route(L, x)
    _, roff, rpt, _ = oracle.permute(ridx, L["n_expert"])
    assert np.array_equal(off.cpu().numpy(), roff) and np.array_equal(pt.cpu().numpy(), rpt)
    assert_close(to_numpy_y(yp), oracle.expert_rows(L, x, roff, rpt), "bf16", "rows")


def test_q4k_shell():
    ov = Q4K_SMALL[0]
    for T in (1, 64, 100):
        L, w, h = shell_case("qwen_q4k", T, **ov)
        lay = dev_layer("qwen_q4k", **ov)
        out = moe_mod().forward_shell(lay, xdev(h), xdev(w), EPS)
        torch.cuda.synchronize()
        ref = oracle.moe_shell(L, h, w, EPS)
        assert_shell_close(to_numpy_y(out), ref, oracle.widen(h), "bf16", f"q4k shell T={T}")


def q4k_pack_expected(L):
    """The grouped copy of a Q4_K layer's routed experts, built with numpy from the
    checkpoint super-blocks: up region then down region (256-byte aligned).  Group
    (e, nt, sb) of 256 tile rows: the rows' 16-byte headers, then quant run c = 0..3 of each
    row as 32 bytes.  Up tile row r: gate unit min(nt * 128 + r, ff - 1) for r < 128, else
    the up unit min(nt * 128 + r - 128, ff - 1); down tile row r: W_d row min(nt * 256 + r,
    d - 1).  Returns [(offset, bytes)] and the total size."""
    E, d, ff = L["n_expert"], L["d"], L["ff"]

    def groups(mats, tile_rows, n_rows, n_tiles):
        r = np.arange(256)
        half = len(mats) == 2
        local = r % 128 if half else r
        n = np.minimum(np.arange(n_tiles)[:, None] * tile_rows + local[None, :], n_rows - 1)  # [nt, 256]
        blocks = [m.reshape(E, n_rows, -1, 144) for m in mats]
        out = np.empty((E, n_tiles, blocks[0].shape[2], 256, 144), np.uint8)
        for t in range(n_tiles):
            for rr in range(256):
                src = blocks[1] if half and rr >= 128 else blocks[0]
                out[:, t, :, rr, :] = src[:, n[t, rr], :, :]
        head = out[..., :16].reshape(out.shape[:3] + (-1,))                        # 256 x 16 B
        runs = out[..., 16:].reshape(out.shape[:4] + (4, 32)).transpose(0, 1, 2, 4, 3, 5)
        return np.concatenate([head, runs.reshape(out.shape[:3] + (-1,))], axis=3).reshape(-1)

    up = groups([L["w_gate"], L["w_up"]], 128, ff, -(-ff // 128))
    dn = groups([L["w_down"]], 256, d, -(-d // 256))
    off_dn = -(-up.size // 256) * 256
    return [(0, up), (off_dn, dn)], off_dn + dn.size


@pytest.mark.parametrize("ov", Q4K_SMALL[:3], ids=Q4K_IDS[:3])
def test_q4k_grouped_pack_layout(ov):
    say("q4k grouped pack layout", ov)
    L, _ = case("qwen_q4k", 1, **ov)
    lay = dev_layer("qwen_q4k", **ov).with_grouped_pack()
    torch.cuda.synchronize()
    got = lay.tensors["grouped_pack"].cpu().numpy()
    regions, total = q4k_pack_expected(L)
    assert got.size == total
    for off, want in regions:
        assert np.array_equal(got[off:off + want.size], want), off


@pytest.mark.parametrize("T", [7, 100, 300])
@pytest.mark.parametrize("ov", Q4K_SMALL, ids=Q4K_IDS)
def test_q4k_grouped_pack_forward(ov, T):
    # The grouped path on the grouped copy: bit for bit the output of the checkpoint layout
    # (T = 7 takes split-K down tiles), and within tolerance of the oracle.
    say("q4k grouped forward, grouped copy", ov, T)
    L, x = case("qwen_q4k", T, **ov)
    lay = dev_layer("qwen_q4k", **ov).with_path("grouped")
    y0 = moe_mod().forward(lay, xdev(x))
    y1 = moe_mod().forward(lay.with_grouped_pack(), xdev(x))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert_close(to_numpy_y(y1), oracle.moe_forward(L, x), "bf16", "y")


def test_q4k_full_grouped_pack():
    # The full Qwen-shaped Q4_K layer at 2048 tokens with the grouped copy, on a seeded
    # sample of tokens.
    T, sample = 2048, 128
    say("full qwen_q4k grouped copy", T)
    L, x = case("qwen_q4k", T)
    lay = dev_layer("qwen_q4k").with_grouped_pack()
    y = to_numpy_y(moe_mod().forward(lay, xdev(x)))
    tok = np.sort(np.random.default_rng(11).choice(T, sample, replace=False))
    e = assert_close(y[tok], oracle.moe_forward(L, x[tok]), "bf16", "y")
    say(f"  rel err {e:.2e}")

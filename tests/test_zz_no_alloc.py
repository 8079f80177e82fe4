"""moe_forward_noalloc (the library's fixed scratch array as the workspace) against
moe_forward with a caller workspace, through the C ABI: two calls in a row on each
layer, the second with a smaller batch, each bit-identical to moe_forward (same kernels,
same order of arithmetic) and within the oracle tolerance."""
import ctypes

import numpy as np
import pytest

import oracle

from gpu_common import assert_close, case, layer_arrays, say, to_numpy_y

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mixture_experts_amd import moe
    moe.lib()


# (layer, overrides, path, [first T, second smaller T]): the decode GEMVs with the
# one-token and few-token fused kernels, the grouped MFMA path with split-K, the grouped
# path above 64 tokens, fp32, the clamped variant, and the full Qwen-shaped decode layer.
CASES = [
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), "auto", [64, 5]),
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), "auto", [8, 1]),
    ("qwen", dict(d=512, n_expert=64, ff=256, shared_ff=256), "grouped", [300, 7]),
    ("tiny_f32", {}, "auto", [77, 16]),
    ("gptoss", dict(d=320, n_expert=16, ff=192), "auto", [100, 1]),
    ("mixtral", dict(d=256, ff=448), "auto", [130, 3]),
    ("qwen", {}, "auto", [64, 8]),
]


def _id(c):
    n, ov, path, Ts = c
    return f"{n}{'-small' if ov else ''}-{path}-T{Ts[0]}-T{Ts[1]}"


@pytest.mark.parametrize("c", CASES, ids=_id)
def test_noalloc_matches_forward(c):
    from sparse_mixture_experts_amd import moe
    name, ov, path, Ts = c
    lay = moe.Layer.from_arrays(layer_arrays(name, 0, **ov))
    lay = lay if path == "auto" else lay.with_path(path)
    for T in Ts:
        say("noalloc", name, ov, path, T)
        L, x = case(name, T, **ov)
        assert moe.workspace_size(lay, T) <= moe.NOALLOC_SCRATCH_BYTES
        xd = moe.to_device(x)
        ref_y = moe.forward(lay, xd)
        got = moe.forward_noalloc(lay, xd)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                           ref_y.view(torch.int16) if ref_y.dtype == torch.bfloat16 else ref_y), \
            "moe_forward_noalloc differs from moe_forward"
        e = assert_close(to_numpy_y(got), oracle.moe_forward(L, x), L["dtype"], "y")
        say(f"  identical to moe_forward, rel err {e:.2e}")


def test_noalloc_refuses_oversized_batch():
    from sparse_mixture_experts_amd import moe
    lay = moe.Layer.from_arrays(layer_arrays("qwen", 0, d=512, n_expert=64, ff=192, shared_ff=128))
    T = 1
    while moe.workspace_size(lay, T) <= moe.NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros((T, 512), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    st = moe.lib().moe_forward_noalloc(lay.ref(), x.data_ptr(), T, y.data_ptr(), moe._stream())
    assert st == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a refused call wrote its output"

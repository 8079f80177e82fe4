"""The layer forward captured into a HIP graph: every replay equals the eager forward.

The library allocates nothing and enqueues no memset inside moe_forward, so a caller may
capture it.  Each case captures one forward, then replays it three times with other eager
forwards (on another workspace and output) and synchronisations between the replays, and
compares every replay with the eager result bit for bit (same kernels, same inputs).
Cases cover the one-token, few-token and decode GEMV paths, the grouped path, and the
MXFP4 and Q4_K expert formats.
"""
import pytest

from gpu_common import case, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    ("qwen", dict(d=512, n_expert=64, ff=192, shared_ff=128), [1, 5, 64, 150]),
    ("gptoss", dict(d=320, n_expert=16, ff=192), [1, 7, 100]),
    ("gptoss_mx", dict(d=320, n_expert=16, ff=192), [1, 7, 100]),
    ("qwen_q4k", dict(d=512, n_expert=16, ff=256, shared_ff=256), [1, 7, 300]),
]
GRAPH_CASES = [(n, ov, T) for n, ov, Ts in CASES for T in Ts]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("c", GRAPH_CASES, ids=lambda c: f"{c[0]}-T{c[2]}")
def test_graph_replay_matches_eager(c):
    from sparse_mixture_experts_amd import moe
    name, ov, T = c
    say("graph", name, ov, T)
    L, x = case(name, T, **ov)
    _, x2 = case(name, T, seed=7, **ov)
    lay = moe.Layer.from_arrays(L)
    xd, x2d = moe.to_device(x), moe.to_device(x2)
    ref = moe.forward(lay, xd)
    torch.cuda.synchronize()

    ws, ws2 = moe.workspace(lay, T), moe.workspace(lay, T)
    y = torch.empty_like(ref)
    y2 = torch.empty_like(ref)
    moe.forward(lay, xd, ws, out=y)  # warm-up on the eager stream before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.forward(lay, xd, ws, out=y)
    torch.cuda.synchronize()
    y.zero_()
    for r in range(3):
        moe.forward(lay, x2d, ws2, out=y2)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {r} differs from the eager forward"
        y.zero_()

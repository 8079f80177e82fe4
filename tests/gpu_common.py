"""Shared helpers of the GPU parity tests: seeded cases, uploads and the tolerance rule.

Tolerance (whole-tensor rule): max |got - ref| <= rtol * max |ref| with rtol = 2e-2 for
bf16 weights (fp32 accumulation) and 1e-4 for fp32.  Routing indices and grouping are
compared bit-exactly.  Routing weights within 4e-6 absolute: the fp32 logits carry an
accumulation error of order sqrt(d) * 2^-24 * sum_i |x_i w_i| (a few 1e-6 at d = 4096),
and a weight moves by at most half of the error of a logit difference.  The shared-gate
input within 1e-4 absolute.
"""
import functools
import sys

import numpy as np

import oracle
from sparse_mixture_experts_amd import synth

RTOL = {"bf16": 2e-2, "f32": 1e-4}
W_ATOL = 4e-6
SG_ATOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / (scale if scale > 0 else 1.0))


def assert_close(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    assert e <= RTOL[dtype], f"{what}: max|err|/max|ref| = {e:.3e} > {RTOL[dtype]}"
    return e


@functools.lru_cache(maxsize=4)
def layer_arrays(name: str, seed: int = 0, **overrides):
    return synth.make_layer(synth.spec(name, **dict(overrides)), seed=seed)


def case(name, T, seed=0, **overrides):
    L = layer_arrays(name, seed, **overrides)
    x = synth.make_tokens(L, T, seed=seed + 100)
    return L, x


def to_numpy_y(y):
    """A device output tensor as fp64 numpy (bf16 widened exactly)."""
    import torch
    return y.detach().to("cpu", torch.float64).numpy()


# Half an ulp of the output, relative to the value: bf16 keeps 8 significant bits, fp32 24.
OUT_ULP = {"bf16": 2.0 ** -8, "f32": 2.0 ** -23}


def assert_shell_close(got, ref, h, dtype, what=""):
    """Layer-shell outputs: the block's part (ref - h) is held to the usual rule, relative
    to its own largest magnitude, and each element may also carry the rounding of the
    residual sum to the output dtype (half an ulp of the value)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    part = ref - np.asarray(h, dtype=np.float64)
    scale = np.max(np.abs(part)) if part.size else 0.0
    allow = RTOL[dtype] * scale + OUT_ULP[dtype] * np.abs(ref)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(allow, 1e-300))) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error reaches {worst:.3f} of the allowance"
    return float(np.max(err) / scale) if scale > 0 else 0.0

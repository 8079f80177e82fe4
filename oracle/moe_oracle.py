"""CPU fp64 oracle of the sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and the
bench's ``cpu_baseline`` leg may import or call this module.  The HIP library never
reaches it, and it imports nothing from the HIP path.

Every input is widened exactly to fp64 (bf16 -> fp64 and fp32 -> fp64 are exact) and all
arithmetic is fp64.  GPU rounding is not emulated; parity tolerances absorb it.

The passages followed:

* "Qwen3.5-MoE Model Implementation", section "MoE routing": router logits, softmax,
  top-8, renormalisation, ``expert_weights_scale``; SwiGLU experts
  ``silu(gate.x) * (up.x) -> down``; ``moe_out = sum_e weight_e * SwiGLU_e(x)``; the
  always-on shared expert scaled by ``sigmoid(gate_inp_shexp . x)``; combine
  ``out = moe_out + shexp_out`` with the residual left to the caller.
* "Llama Forward Pass", section "Mixture of Experts (Mixtral)": the same
  softmax -> top-k -> renormalise order ("weights sum to 1"), and section "SwiGLU FFN".
* "Phase 19: MoE - gpt-oss-20b", section 2 (router and experts of the reference math):
  logits with a bias, top-k first, softmax over the k selected; fused interleaved
  ``gate_up`` with bias, gate clamped from above, up clamped on both sides,
  ``glu = gate * sigmoid(alpha * gate)``, ``h = (up + 1) * glu``, down projection with
  bias, weighted sum with the routing scores.
* "Phase 19: MoE - gpt-oss-20b", section 3 and the tensor layout: MXFP4 expert weights
  (32 FP4 codes and one E8M0 scale per block), dequantised before use.
* "Qwen3.5-MoE Model Implementation", numeric status (K-quant Q3_K experts) and "Engine",
  Prefill (Q4 / Q2 / Q3 GEMMs): K-quant expert weights; the Q4_K block layout is not on
  the pages and follows the GGUF definition (``q4k_dequant``).
* "Llama Forward Pass", section "Key Operations", RMSNorm, and "Qwen3.5-MoE Model
  Implementation", section "Architecture" (post-attention norm -> MoE FFN -> residual):
  the layer shell around the block (``moe_shell``).
* "Engine" (Cherenkov), section "Prefill": each expert evaluated once over the rows
  routed to it, the results returned to their tokens -- the grouped evaluation below;
  section "Address tables": the union of the experts a batch selects, with a zero weight
  where a row did not select an expert.

Readings where the pages are silent (top-k tie-break and output order, router bias
placement, permutation order inside an expert, ...) are listed with the design notes of
the repository; each is restated at the function that depends on it.

Parity pins: every public function here is pinned by a CPU test against closed forms,
special cases, brute force or independent library routines (see ``tests/test_oracle_*``).
"""
from __future__ import annotations

import itertools

import numpy as np

# ----------------------------------------------------------------------------- inputs


def widen(a) -> np.ndarray | None:
    """Stored tensor -> fp64.  uint16 arrays are bf16 bit patterns: the bf16 value is the
    fp32 number whose upper 16 bits are those bits and lower 16 bits are zero."""
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# FP4 (E2M1) code table of the OCP Microscaling formats: sign bit 3, two exponent bits
# (bias 1), one mantissa bit; exponent 0 holds 0 and the subnormal 0.5.  The gpt-oss page
# names the table (fp4_lut) without printing it.
FP4_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def mxfp4_dequant(blocks, scales) -> np.ndarray:
    """MXFP4 weights ("Phase 19: MoE - gpt-oss-20b", section 3, MXFP4 dequantisation, and
    the measured tensor layout): ``blocks[..., nblk, 16]`` uint8 hold 32 FP4 codes per 16
    bytes, the low nibble of byte i being element 2i and the high nibble element 2i+1;
    ``scales[..., nblk]`` uint8 are E8M0 exponents shared by the block's 32 elements;
    value = fp4(code) * 2^(scale - 127) (scale 255 is NaN).  Returns fp64
    ``[..., nblk * 32]``."""
    b = np.asarray(blocks, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.int64)
    codes = np.stack([b & 0x0F, b >> 4], axis=-1).reshape(b.shape[:-1] + (32,))
    mult = np.where(sc == 255, np.nan, np.ldexp(1.0, sc - 127))
    vals = FP4_E2M1[codes] * mult[..., None]
    return vals.reshape(b.shape[:-2] + (b.shape[-2] * 32,))


# GGUF "K-quant" Q4_K super-block: 256 weights in 144 bytes.  The pages name K-quant
# experts (Q3_K on "Qwen3.5-MoE Model Implementation", numeric status; Q4 / Q2 / Q3 GEMMs
# on "Engine", Prefill) but print no block layout; the layout below is the GGUF Q4_K
# definition, taken as a reading:
#   bytes 0-1   d     fp16, multiplier of the sub-block scales
#   bytes 2-3   dmin  fp16, multiplier of the sub-block mins
#   bytes 4-15  eight 6-bit scales sc_j and eight 6-bit mins m_j of the 32-weight
#               sub-blocks j = 0..7: for j < 4, sc_j and m_j are the low 6 bits of bytes
#               4+j and 8+j; for j >= 4, the low 4 bits of sc_j / m_j are the low / high
#               nibble of byte 12+(j-4), and their top 2 bits are the top 2 bits of byte
#               4+(j-4) (for sc_j) and byte 8+(j-4) (for m_j)
#   bytes 16-143  128 bytes of 4-bit quants in 4 runs of 32: byte l of run c holds the
#               quant of weight 64c + l in its low nibble (sub-block 2c) and of weight
#               64c + 32 + l in its high nibble (sub-block 2c + 1)
#   weight = d * sc_j * q - dmin * m_j
Q4K_BLOCK = 144
Q4K_WEIGHTS = 256


def q4k_dequant(blocks) -> np.ndarray:
    """Q4_K weights (layout above): ``blocks[..., nsb, 144]`` uint8 -> fp64
    ``[..., nsb * 256]`` (fp16 d and dmin widen exactly; every product is exact in fp64)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    lead = b.shape[:-1]
    d = b[..., 0:2].copy().view("<f2").astype(np.float64)[..., 0]
    dmin = b[..., 2:4].copy().view("<f2").astype(np.float64)[..., 0]
    lo6 = b[..., 4:12].astype(np.int64) & 63            # sc_0..3 then m_0..3
    top2 = b[..., 4:12].astype(np.int64) >> 6           # upper bits of sc_4..7 then m_4..7
    nib = b[..., 12:16].astype(np.int64)
    sc = np.concatenate([lo6[..., 0:4], (nib & 15) | (top2[..., 0:4] << 4)], axis=-1)
    mn = np.concatenate([lo6[..., 4:8], (nib >> 4) | (top2[..., 4:8] << 4)], axis=-1)
    runs = b[..., 16:144].astype(np.int64).reshape(lead + (4, 32))
    q = np.stack([runs & 15, runs >> 4], axis=-2).reshape(lead + (8, 32))  # sub-block 2c, 2c+1
    vals = d[..., None, None] * sc[..., :, None] * q - dmin[..., None, None] * mn[..., :, None]
    return vals.reshape(b.shape[:-2] + (b.shape[-2] * Q4K_WEIGHTS,))


def _expert(L: dict, name: str, e: int) -> np.ndarray | None:
    t = L.get(name)
    if t is None:
        return None
    if L.get("expert_format") == "mxfp4" and name in ("w_gate_up", "w_down"):
        return mxfp4_dequant(t[e], L[name + "_scales"][e])
    if L.get("expert_format") == "q4k" and name in ("w_gate", "w_up", "w_down"):
        return q4k_dequant(t[e])
    return widen(t[e])


# ----------------------------------------------------------------------------- router

def router_logits(L: dict, x) -> np.ndarray:
    """z[t,e] = sum_i x[t,i] W_r[e,i] (+ b[e]).

    "Qwen3.5-MoE Model Implementation", MoE routing: ``ffn_gate_inp [n_expert, n_embd]``
    maps x to logits.  "Phase 19: MoE - gpt-oss-20b", Router: ``x @ W^T + b``.
    Reading: where a router bias is present it is added to the logits before any
    selection or softmax, in both routing modes.
    """
    z = widen(x) @ widen(L["w_router"]).T
    if L.get("b_router") is not None:
        z = z + widen(L["b_router"])[None, :]
    return z


def topk_select(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits of each row, ordered by descending logit.

    Reading (pages silent): ties go to the lower expert index.  A stable sort of -z
    orders experts by (-z_e, e), which fixes both the selected set and its order.
    """
    order = np.argsort(-z, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax exp(z - max) / sum exp(z - max)."""
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def weights_softmax_topk_renorm(z: np.ndarray, idx: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """Mode A ("Qwen3.5-MoE Model Implementation", MoE routing; "Llama Forward Pass",
    Mixture of Experts): p = softmax over all experts, take the selected p, renormalise
    so they sum to 1, multiply by ``expert_weights_scale`` (default 1.0)."""
    p = softmax(z)
    sel = np.take_along_axis(p, idx, axis=1)
    return scale * sel / sel.sum(axis=1, keepdims=True)


def weights_topk_softmax(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Mode B ("Phase 19: MoE - gpt-oss-20b", Router): softmax over the k selected
    logits only."""
    return softmax(np.take_along_axis(z, idx, axis=1))


def shared_gate_input(L: dict, x) -> np.ndarray | None:
    """a[t] = gate_inp_shexp . x[t], the input of the shared expert's sigmoid gate
    ("Qwen3.5-MoE Model Implementation", MoE routing, shared expert)."""
    if L.get("ws_gate_inp") is None:
        return None
    return widen(x) @ widen(L["ws_gate_inp"])


def route(L: dict, x):
    """(topk_idx[T,k], topk_w[T,k], shared_gate_input[T] or None) for the layer's mode."""
    z = router_logits(L, x)
    idx = topk_select(z, L["k"])
    if L["route"] == "softmax_topk_renorm":
        w = weights_softmax_topk_renorm(z, idx, L.get("route_scale", 1.0))
    elif L["route"] == "topk_softmax":
        w = weights_topk_softmax(z, idx)
    else:
        raise ValueError(L["route"])
    return idx, w, shared_gate_input(L, x)


# ----------------------------------------------------------------------------- experts

def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a / (1 + exp(-a)) ("Llama Forward Pass", SwiGLU FFN)."""
    return a / (1.0 + np.exp(-a))


def sigmoid(a: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-a))


def swiglu_ffn(xr: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Rows of x through one SwiGLU expert: W_d (silu(W_g x) * (W_u x)).
    "Llama Forward Pass", SwiGLU FFN and Mixture of Experts."""
    h = silu(xr @ wg.T) * (xr @ wu.T)
    return h @ wd.T


def swiglu_oai_hidden(v: np.ndarray, alpha: float, limit: float) -> np.ndarray:
    """Clamped interleaved activation of "Phase 19: MoE - gpt-oss-20b", Experts:
    gate = even columns, up = odd columns; gate clamped from above at ``limit``; up
    clamped to [-limit, limit]; h = (up + 1) * gate * sigmoid(alpha * gate)."""
    gate = np.minimum(v[:, 0::2], limit)
    up = np.clip(v[:, 1::2], -limit, limit)
    return (up + 1.0) * (gate * sigmoid(alpha * gate))


def swiglu_oai_ffn(xr, wgu, bgu, wd, bd, alpha, limit) -> np.ndarray:
    """Rows of x through one expert of the clamped variant, biases included
    ("Phase 19: MoE - gpt-oss-20b", Experts).  Reading: the down bias is part of the
    expert output, so the routing weight scales it too."""
    v = xr @ wgu.T + bgu[None, :]
    return swiglu_oai_hidden(v, alpha, limit) @ wd.T + bd[None, :]


def expert_apply(L: dict, e: int, xr: np.ndarray) -> np.ndarray:
    """FFN_e applied to fp64 rows xr[n, d]."""
    if L["act"] == "swiglu":
        return swiglu_ffn(xr, _expert(L, "w_gate", e), _expert(L, "w_up", e), _expert(L, "w_down", e))
    return swiglu_oai_ffn(xr, _expert(L, "w_gate_up", e), _expert(L, "b_gate_up", e),
                          _expert(L, "w_down", e), _expert(L, "b_down", e),
                          L["oai_alpha"], L["oai_limit"])


def shared_expert(L: dict, x) -> np.ndarray | None:
    """sigmoid(gate_inp_shexp . x) * W_sd (silu(W_sg x) * (W_su x)), or None without a
    shared expert ("Qwen3.5-MoE Model Implementation", MoE routing)."""
    if L.get("ws_gate") is None or L.get("shared_ff", 0) == 0:
        return None
    xf = widen(x)
    y = swiglu_ffn(xf, widen(L["ws_gate"]), widen(L["ws_up"]), widen(L["ws_down"]))
    return sigmoid(shared_gate_input(L, x))[:, None] * y


# ----------------------------------------------------------------------------- grouping

def permute(idx: np.ndarray, E: int):
    """Expert grouping ("Engine", section "Prefill": the rows of each expert made
    contiguous so that the expert is evaluated once over them).

    Returns counts[E], offsets[E+1] (exclusive prefix sum of counts), perm_token[T*k]
    (token of each grouped row) and perm_inv[T,k] (grouped row of (t, j)).
    Reading (pages silent): rows are expert-major and, within an expert, in ascending
    token order; a token selects an expert at most once.
    """
    T, k = idx.shape
    counts = np.zeros(E, dtype=np.int64)
    for e in idx.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm_token = np.empty(T * k, dtype=np.int64)
    perm_inv = np.empty((T, k), dtype=np.int64)
    for t in range(T):                       # ascending token order inside every expert
        for j in range(k):
            e = idx[t, j]
            perm_token[fill[e]] = t
            perm_inv[t, j] = fill[e]
            fill[e] += 1
    return counts, offsets, perm_token, perm_inv


def expert_rows(L: dict, x, offsets: np.ndarray, perm_token: np.ndarray) -> np.ndarray:
    """Y_perm[T*k (+T), d]: row r holds FFN_e(x[perm_token[r]]) for the expert e whose
    group contains r; when the layer has a shared expert, rows T*k + t hold the
    shared expert's output for token t *without* its sigmoid gate."""
    xf = widen(x)
    T, d = xf.shape
    n = int(offsets[-1])
    shared = L.get("ws_gate") is not None and L.get("shared_ff", 0) > 0
    y = np.zeros((n + (T if shared else 0), d))
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = expert_apply(L, e, xf[perm_token[a:b]])
    if shared:
        y[n:] = swiglu_ffn(xf, widen(L["ws_gate"]), widen(L["ws_up"]), widen(L["ws_down"]))
    return y


def combine(y_perm: np.ndarray, perm_inv: np.ndarray, w: np.ndarray, shared_a) -> np.ndarray:
    """out[t] = sum_j w[t,j] Y_perm[perm_inv[t,j]] (+ sigmoid(a[t]) Y_perm[T*k + t]).
    "Qwen3.5-MoE Model Implementation", MoE routing (combine; no residual add)."""
    T, k = perm_inv.shape
    out = np.zeros((T, y_perm.shape[1]))
    for j in range(k):
        out += w[:, j:j + 1] * y_perm[perm_inv[:, j]]
    if shared_a is not None:
        out += sigmoid(shared_a)[:, None] * y_perm[T * k:T * k + T]
    return out


def moe_forward(L: dict, x) -> np.ndarray:
    """The whole layer, grouped by expert: route -> group -> per-expert FFN -> combine."""
    xf = widen(x)
    if xf.shape[0] == 0:
        return np.zeros((0, L["d"]))
    idx, w, a = route(L, x)
    _, offsets, perm_token, perm_inv = permute(idx, L["n_expert"])
    y_perm = expert_rows(L, x, offsets, perm_token)
    return combine(y_perm, perm_inv, w, a)


def moe_forward_tokens(L: dict, x, tokens=None) -> np.ndarray:
    """The layer's definition token by token, with no grouping: for each token,
    ``sum_j w_j FFN_{s_j}(x) + shared``.  ``tokens`` restricts the rows evaluated
    (for sampled checks of large batches)."""
    xf = widen(x)
    tok = np.arange(xf.shape[0]) if tokens is None else np.asarray(tokens)
    xs = xf[tok]
    idx, w, a = route(L, xs)
    sh = shared_expert(L, xs)
    out = np.zeros((len(tok), L["d"]))
    for i in range(len(tok)):
        for j in range(L["k"]):
            out[i] += w[i, j] * expert_apply(L, int(idx[i, j]), xs[i:i + 1])[0]
        if sh is not None:
            out[i] += sh[i]
    return out


# ----------------------------------------------------------------------------- layer shell

def rmsnorm(x, weight, eps: float) -> np.ndarray:
    """RMSNorm ("Llama Forward Pass", Key Operations, RMSNorm; "Phase 19: MoE -
    gpt-oss-20b", section 2, RMSNorm, eps 1e-5): every row divided by the square root of
    the mean of its squares plus eps, then multiplied elementwise by the weight."""
    xf = widen(x)
    wf = widen(weight)
    mean_sq = np.mean(xf * xf, axis=1, keepdims=True)
    return xf / np.sqrt(mean_sq + eps) * wf[None, :]


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value (8 significant bits, ties to even),
    returned as fp64.  Finite values in the normal bf16 range only (the normalised
    activations this is used on are far from under- and overflow)."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                   # a = m * 2**e, 0.5 <= |m| < 1
    ulp = np.ldexp(1.0, e - 8)           # spacing of 8-bit significands at that exponent
    return np.round(a / ulp) * ulp       # np.round: half to even


def store_activation(a: np.ndarray, dtype: str):
    """The normalised activation in the layer's storage form: bf16 bit patterns (uint16)
    for a bf16 layer, float32 otherwise.  Reading taken: the norm's output is stored in
    the dtype of the layer's activations before the MoE block reads it, as a separate
    norm kernel would store it."""
    if dtype == "bf16":
        r = round_to_bf16(a).astype(np.float32)          # exact: 8-bit significands fit fp32
        return (r.view(np.uint32) >> 16).astype(np.uint16)
    return np.asarray(a, dtype=np.float32)


def moe_shell(L: dict, h, norm_w, eps: float) -> np.ndarray:
    """The FFN half of a decoder layer around the MoE block ("Qwen3.5-MoE Model
    Implementation", Architecture: post-attention norm, then the shared-MoE FFN, then the
    residual add): out = h + MoE(RMSNorm(h)), the normalised rows stored in the layer's
    dtype first."""
    hf = widen(h)
    if hf.shape[0] == 0:
        return np.zeros((0, L["d"]))
    xn = store_activation(rmsnorm(h, norm_w, eps), L["dtype"])
    return hf + moe_forward(L, xn)


# ----------------------------------------------------------------------------- decode view

def active_union(idx: np.ndarray, w: np.ndarray, E: int):
    """Union of experts selected by any row of a small batch, with the per-row weight
    map that holds zero where a row did not select the expert ("Engine", Address
    tables).  Returns (experts ascending, wmap[n_active, T]).  The page orders its table
    by residency and then by largest weight; here the experts are in ascending id (a
    reading: no output depends on the order of the union)."""
    active = np.unique(idx.reshape(-1))
    wmap = np.zeros((active.size, idx.shape[0]))
    pos = {int(e): i for i, e in enumerate(active)}
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            wmap[pos[int(idx[t, j])], t] = w[t, j]
    return active, wmap


# ----------------------------------------------------------------------------- brute force

def brute_topk(zrow, k):
    """Top-k by enumerating every k-subset: the subset with the largest logit sum wins,
    ties broken by the lexicographically smallest sorted index tuple; its members are
    then ordered by (-z, e).  Tiny E only."""
    E = len(zrow)
    best, best_s = None, None
    for S in itertools.combinations(range(E), k):
        s = sum(float(zrow[e]) for e in S)
        if best is None or s > best_s:
            best, best_s = S, s
    return sorted(best, key=lambda e: (-float(zrow[e]), e))


def brute_forward(L: dict, x) -> np.ndarray:
    """Scalar Python loops over the whole layer for tiny shapes (d, ff <= 16, E <= 6), dense
    expert weights only."""
    import math
    if L.get("expert_format", "dense") != "dense":
        raise ValueError("brute_forward takes dense expert weights")
    xf = widen(x)
    T, d = xf.shape
    E, k, ff = L["n_expert"], L["k"], L["ff"]
    wr = widen(L["w_router"])
    br = widen(L["b_router"]) if L.get("b_router") is not None else [0.0] * E
    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        z = [sum(xf[t][i] * wr[e][i] for i in range(d)) + br[e] for e in range(E)]
        S = brute_topk(z, k)
        if L["route"] == "softmax_topk_renorm":
            m = max(z)
            den = sum(math.exp(v - m) for v in z)
            p = [math.exp(z[e] - m) / den for e in S]
            w = [L.get("route_scale", 1.0) * pi / sum(p) for pi in p]
        else:
            m = z[S[0]]
            ex = [math.exp(z[e] - m) for e in S]
            w = [v / sum(ex) for v in ex]
        for j, e in enumerate(S):
            if L["act"] == "swiglu":
                wg, wu, wd = (widen(L[n][e]) for n in ("w_gate", "w_up", "w_down"))
                h = []
                for f in range(ff):
                    g = sum(wg[f][i] * xf[t][i] for i in range(d))
                    u = sum(wu[f][i] * xf[t][i] for i in range(d))
                    h.append(g / (1.0 + math.exp(-g)) * u)
                y = [sum(wd[i][f] * h[f] for f in range(ff)) for i in range(d)]
            else:
                wgu, bgu = widen(L["w_gate_up"][e]), widen(L["b_gate_up"][e])
                wd, bd = widen(L["w_down"][e]), widen(L["b_down"][e])
                al, lim = L["oai_alpha"], L["oai_limit"]
                h = []
                for f in range(ff):
                    g = sum(wgu[2 * f][i] * xf[t][i] for i in range(d)) + bgu[2 * f]
                    u = sum(wgu[2 * f + 1][i] * xf[t][i] for i in range(d)) + bgu[2 * f + 1]
                    g = min(g, lim)
                    u = min(max(u, -lim), lim)
                    h.append((u + 1.0) * g / (1.0 + math.exp(-al * g)))
                y = [sum(wd[i][f] * h[f] for f in range(ff)) + bd[i] for i in range(d)]
            for i in range(d):
                out[t][i] += w[j] * y[i]
        if L.get("ws_gate") is not None and L.get("shared_ff", 0) > 0:
            sg, su, sd = widen(L["ws_gate"]), widen(L["ws_up"]), widen(L["ws_down"])
            gi = widen(L["ws_gate_inp"])
            a = sum(gi[i] * xf[t][i] for i in range(d))
            h = []
            for f in range(L["shared_ff"]):
                g = sum(sg[f][i] * xf[t][i] for i in range(d))
                u = sum(su[f][i] * xf[t][i] for i in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for i in range(d):
                out[t][i] += (1.0 / (1.0 + math.exp(-a))) * sum(sd[i][f] * h[f] for f in range(L["shared_ff"]))
    return np.array(out)

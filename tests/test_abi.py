"""The C ABI without a GPU: the library loads, exports every function include/moe.h
declares, the struct layout matches, and every argument error is reported before any
HIP call (fake, never-dereferenced pointers are enough)."""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 64 KiB-aligned address; the library must never touch it in these tests

# These tests call real entry points with fake device addresses, which every check must
# reject before any launch.  On a machine where a GPU can be reached (/dev/kfd exists)
# the module runs in a child process that sees no GPU (tests/conftest.py deselects the
# tests here and keeps test_in_child_without_gpu), so a regressed check returns
# MOE_ERR_DEVICE there instead of launching a kernel on a fake address.
CHILD_ENV = "SMOE_ABI_CHILD"


def test_in_child_without_gpu():
    import subprocess
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    env[CHILD_ENV] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", __file__],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail("libsmoe.so is not built")
    return moe.lib()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) == 13, names
    assert sorted(moe.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout(lib):
    assert moe.MoeLayer.route_scale.offset == 36
    assert moe.MoeLayer.w_router.offset == 48
    assert moe.MoeLayer.ws_gate_inp.offset == 48 + 11 * 8
    assert moe.MoeLayer.expert_format.offset == 144
    assert moe.MoeLayer.w_gate_up_scales.offset == 152
    assert moe.MoeLayer.w_down_scales.offset == 160
    assert moe.MoeLayer.grouped_pack.offset == 168
    assert ctypes.sizeof(moe.MoeLayer) == 176


def fake_layer(**kw):
    s = moe.MoeLayer()
    s.d, s.n_expert, s.ff, s.k, s.shared_ff = 256, 8, 512, 2, 0
    s.dtype, s.route, s.act, s.path = moe.MOE_BF16, 0, 0, 0
    s.route_scale, s.oai_alpha, s.oai_limit = 1.0, 1.702, 7.0
    s.w_router = s.w_gate = s.w_up = s.w_down = FAKE
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def ws_size(lib, s, T):
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(s), T, ctypes.byref(n))
    return st, n.value


def fwd(lib, s, T=4, x=FAKE, y=FAKE * 2, ws=FAKE * 3, nbytes=1 << 40):
    return lib.moe_forward(ctypes.byref(s), x, T, y, ws, nbytes, None)


def test_status_strings(lib):
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(3)
    assert moe.status_string(99) == "unknown status"


def test_workspace_size_grows_with_T(lib):
    s = fake_layer()
    st0, n0 = ws_size(lib, s, 1)
    st1, n1 = ws_size(lib, s, 1000)
    assert st0 == st1 == 0 and 0 < n0 < n1


def test_token_count_limit(lib):
    # At most 2^22 tokens per call; negative counts are argument errors.
    s = fake_layer()
    assert ws_size(lib, s, 1 << 22)[0] == moe.MOE_OK
    assert ws_size(lib, s, (1 << 22) + 1)[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(lib, s, -1)[0] == moe.MOE_ERR_ARG


@pytest.mark.parametrize("field,value,status", [
    ("k", 0, moe.MOE_ERR_ARG), ("k", 9, moe.MOE_ERR_ARG), ("d", 0, moe.MOE_ERR_ARG),
    ("n_expert", -1, moe.MOE_ERR_ARG), ("shared_ff", -64, moe.MOE_ERR_ARG),
    ("dtype", 5, moe.MOE_ERR_ARG), ("route", 2, moe.MOE_ERR_ARG), ("act", 7, moe.MOE_ERR_ARG),
    ("path", 3, moe.MOE_ERR_ARG), ("w_router", None, moe.MOE_ERR_ARG),
    ("w_gate", None, moe.MOE_ERR_ARG), ("w_down", None, moe.MOE_ERR_ARG),
    ("route_scale", float("nan"), moe.MOE_ERR_ARG),
    ("shared_ff", 512, moe.MOE_ERR_ARG),            # shared expert without its pointers
    ("d", 200, moe.MOE_ERR_UNSUPPORTED), ("ff", 100, moe.MOE_ERR_UNSUPPORTED),
    ("w_up", FAKE + 2, moe.MOE_ERR_UNSUPPORTED),    # misaligned weights
    ("b_router", FAKE + 2, moe.MOE_ERR_UNSUPPORTED),
])
def test_layer_errors(lib, field, value, status):
    s = fake_layer(**{field: value})
    assert fwd(lib, s) == status
    assert ws_size(lib, s, 4)[0] == status


def test_too_many_experts_or_k(lib):
    assert fwd(lib, fake_layer(n_expert=1024, k=2)) == moe.MOE_ERR_UNSUPPORTED
    assert fwd(lib, fake_layer(n_expert=64, k=33)) == moe.MOE_ERR_UNSUPPORTED


def test_oai_needs_fused_weights(lib):
    s = fake_layer(act=moe.MOE_ACT_SWIGLU_OAI)
    assert fwd(lib, s) == moe.MOE_ERR_ARG
    s = fake_layer(act=moe.MOE_ACT_SWIGLU_OAI, w_gate_up=FAKE, b_gate_up=FAKE)
    assert ws_size(lib, s, 4)[0] == 0


def test_grouped_path_needs_bf16(lib):
    assert fwd(lib, fake_layer(dtype=moe.MOE_F32, path=moe.MOE_PATH_GROUPED)) == moe.MOE_ERR_UNSUPPORTED


def test_forward_argument_errors(lib):
    s = fake_layer()
    assert fwd(lib, s, T=-1) == moe.MOE_ERR_ARG
    assert fwd(lib, s, T=0) == moe.MOE_OK                     # no-op, nothing launched
    assert fwd(lib, s, T=0, x=None, y=None, ws=None) == moe.MOE_OK
    assert fwd(lib, s, x=None) == moe.MOE_ERR_ARG
    assert fwd(lib, s, y=None) == moe.MOE_ERR_ARG
    assert fwd(lib, s, ws=None) == moe.MOE_ERR_ARG
    assert fwd(lib, s, x=FAKE, y=FAKE) == moe.MOE_ERR_ARG      # y aliases x
    assert fwd(lib, s, x=FAKE + 8) == moe.MOE_ERR_UNSUPPORTED  # misaligned x
    assert fwd(lib, s, T=1 << 23) == moe.MOE_ERR_UNSUPPORTED
    _, need = ws_size(lib, s, 4)
    assert fwd(lib, s, nbytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_forward(None, FAKE, 4, FAKE * 2, FAKE * 3, 1 << 40, None) == moe.MOE_ERR_ARG


def test_route_permute_ffn_combine_argument_errors(lib):
    s = fake_layer()
    L = ctypes.byref(s)
    # shared_gate output for a layer without a shared expert
    assert lib.moe_route(L, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_ARG
    assert lib.moe_route(L, FAKE, 4, None, FAKE, None, FAKE, 1 << 40, None) == moe.MOE_ERR_ARG
    assert lib.moe_route(L, FAKE, 4, FAKE, FAKE, None, FAKE, 10, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_route(L, FAKE, 0, None, None, None, None, 0, None) == moe.MOE_OK
    n = ctypes.c_size_t(0)
    assert lib.moe_permute_workspace_size(4, 3, 2, ctypes.byref(n)) == moe.MOE_ERR_ARG    # k > E
    assert lib.moe_permute_workspace_size(4, 2, 8, ctypes.byref(n)) == moe.MOE_OK
    assert lib.moe_permute(FAKE, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, n.value - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_permute(None, 4, 2, 8, FAKE, FAKE, FAKE, FAKE, n.value, None) == moe.MOE_ERR_ARG
    assert lib.moe_permute(FAKE, -2, 2, 8, FAKE, FAKE, FAKE, FAKE, n.value, None) == moe.MOE_ERR_ARG
    assert lib.moe_expert_ffn(L, FAKE, 4, None, FAKE, FAKE, FAKE, 1 << 40, None) == moe.MOE_ERR_ARG
    assert lib.moe_expert_ffn(L, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 10, None) == moe.MOE_ERR_WORKSPACE
    # combine: shared_gate must be given exactly when the layer has a shared expert
    assert lib.moe_combine(L, FAKE, FAKE, FAKE, FAKE, 4, FAKE, None) == moe.MOE_ERR_ARG
    assert lib.moe_combine(L, FAKE, FAKE, None, None, 4, FAKE, None) == moe.MOE_ERR_ARG
    sh = fake_layer(shared_ff=512, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE, ws_gate_inp=FAKE)
    assert lib.moe_combine(ctypes.byref(sh), FAKE, FAKE, FAKE, None, 4, FAKE, None) == moe.MOE_ERR_ARG


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        moe.lib()


def shell(lib, s, T=4, h=FAKE, w=FAKE * 4, eps=1e-5, out=FAKE * 2, ws=FAKE * 3, nbytes=1 << 40):
    return lib.moe_forward_shell(ctypes.byref(s), h, T, w, eps, out, ws, nbytes, None)


def test_shell_argument_errors(lib):
    s = fake_layer()
    assert shell(lib, s, T=0) == moe.MOE_OK
    assert shell(lib, s, T=-1) == moe.MOE_ERR_ARG
    assert shell(lib, s, eps=-1.0) == moe.MOE_ERR_ARG
    assert shell(lib, s, eps=float("nan")) == moe.MOE_ERR_ARG
    assert shell(lib, s, eps=float("inf")) == moe.MOE_ERR_ARG
    for name in ("h", "w", "out", "ws"):
        assert shell(lib, s, **{name: None}) == moe.MOE_ERR_ARG, name
    assert shell(lib, s, out=FAKE + 256) == moe.MOE_ERR_ARG        # overlaps h partially
    assert shell(lib, s, w=FAKE * 4 + 8) == moe.MOE_ERR_UNSUPPORTED  # misaligned norm weight
    assert shell(lib, s, h=FAKE + 8, out=FAKE * 2 + 8) == moe.MOE_ERR_UNSUPPORTED
    _, need = ws_size(lib, s, 4)
    assert shell(lib, s, nbytes=need - 1) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_forward_shell(None, FAKE, 4, FAKE, 1e-5, FAKE * 2, FAKE * 3, 1 << 40, None) == moe.MOE_ERR_ARG


def test_mxfp4_layer_checks(lib):
    mx = dict(expert_format=moe.MOE_EXPERTS_MXFP4, act=moe.MOE_ACT_SWIGLU_OAI, w_gate_up=FAKE,
              b_gate_up=FAKE, w_gate_up_scales=FAKE * 5, w_down_scales=FAKE * 6)
    assert ws_size(lib, fake_layer(**mx), 4)[0] == moe.MOE_OK
    assert ws_size(lib, fake_layer(**dict(mx, w_down_scales=None)), 4)[0] == moe.MOE_ERR_ARG
    assert ws_size(lib, fake_layer(**dict(mx, expert_format=7)), 4)[0] == moe.MOE_ERR_ARG
    assert ws_size(lib, fake_layer(**dict(mx, reserved0=1)), 4)[0] == moe.MOE_ERR_ARG
    assert ws_size(lib, fake_layer(**dict(mx, dtype=moe.MOE_F32)), 4)[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(lib, fake_layer(**dict(mx, act=moe.MOE_ACT_SWIGLU, w_gate=FAKE, w_up=FAKE, b_gate_up=None)),
                   4)[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(lib, fake_layer(**dict(mx, path=moe.MOE_PATH_GROUPED)), 4)[0] == moe.MOE_OK
    assert ws_size(lib, fake_layer(**dict(mx, d=8192)), 4)[0] == moe.MOE_ERR_UNSUPPORTED  # K > 4096
    sh = dict(mx, shared_ff=64, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE, ws_gate_inp=FAKE)
    assert ws_size(lib, fake_layer(**sh), 4)[0] == moe.MOE_ERR_UNSUPPORTED


def pack_size(lib, s):
    n = ctypes.c_size_t(0)
    return lib.moe_grouped_pack_size(ctypes.byref(s), ctypes.byref(n)), n.value


def test_grouped_pack_checks(lib):
    # The grouped copy exists for MXFP4, Q4_K and dense bf16 layers; its size follows the tile counts
    # (up: ceil(ff/128) N-tiles x d/64 slices x 512 blocks of 17 bytes; down: ceil(d/256)
    # x ff/32 x 256), each region rounded up to 256 bytes.
    mx = dict(expert_format=moe.MOE_EXPERTS_MXFP4, act=moe.MOE_ACT_SWIGLU_OAI, w_gate_up=FAKE,
              b_gate_up=FAKE, w_gate_up_scales=FAKE * 5, w_down_scales=FAKE * 6)
    s = fake_layer(**mx)
    st, n = pack_size(lib, s)
    E, d, ff = 8, 256, 512
    up = E * ((ff + 127) // 128) * (d // 64) * 512
    dn = E * ((d + 255) // 256) * (ff // 32) * 256
    r256 = lambda b: (b + 255) // 256 * 256
    assert st == moe.MOE_OK and n == r256(16 * up) + r256(up) + r256(16 * dn) + r256(dn)
    f32 = fake_layer(dtype=moe.MOE_F32)                                # no grouped path in fp32
    assert pack_size(lib, f32)[0] == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_pack(ctypes.byref(f32), FAKE * 7, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_pack(ctypes.byref(s), None, 1 << 40, None) == moe.MOE_ERR_ARG
    assert lib.moe_grouped_pack(ctypes.byref(s), FAKE * 7 + 4, 1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_grouped_pack(ctypes.byref(s), FAKE * 7, n - 1, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_grouped_pack(None, FAKE * 7, n, None) == moe.MOE_ERR_ARG
    # The field: MXFP4 only, 16-byte aligned.
    assert ws_size(lib, fake_layer(**dict(mx, grouped_pack=FAKE * 7)), 4)[0] == moe.MOE_OK
    assert ws_size(lib, fake_layer(**dict(mx, grouped_pack=FAKE * 7 + 8)), 4)[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(lib, fake_layer(dtype=moe.MOE_F32, grouped_pack=FAKE * 7), 4)[0] == moe.MOE_ERR_UNSUPPORTED
    assert fwd(lib, fake_layer(dtype=moe.MOE_F32, grouped_pack=FAKE * 7)) == moe.MOE_ERR_UNSUPPORTED
    # Dense bf16: the down weights only, routed [E][ceil(d/256)][ff/32][256][32] bf16, then the
    # shared expert's [ceil(d/256)][shared_ff/32][256][32].
    assert pack_size(lib, fake_layer()) == (moe.MOE_OK, 8 * 1 * 256 * 512 * 2)
    sh = fake_layer(d=320, shared_ff=128, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE, ws_gate_inp=FAKE)
    assert pack_size(lib, sh) == (moe.MOE_OK, r256(8 * 2 * 256 * 512 * 2) + 2 * 256 * 128 * 2)
    assert ws_size(lib, fake_layer(grouped_pack=FAKE * 7), 4)[0] == moe.MOE_OK
    # Q4_K: per (expert, N-tile, super-block) 256 rows of 144 bytes; up tiles of 128 units
    # over d/256 super-blocks, down tiles of 256 rows over ff/256.
    q4 = fake_layer(expert_format=moe.MOE_EXPERTS_Q4K, d=512, ff=256)
    st, n = pack_size(lib, q4)
    up = 8 * 2 * 2 * 256 * 144
    assert st == moe.MOE_OK and n == r256(up) + 8 * 2 * 1 * 256 * 144
    assert ws_size(lib, fake_layer(expert_format=moe.MOE_EXPERTS_Q4K, d=512, ff=256, grouped_pack=FAKE * 7),
                   4)[0] == moe.MOE_OK


def test_swiglu_rejects_expert_biases(lib):
    # Expert biases belong to the clamped variant; a plain SwiGLU layer carrying one is an
    # argument error, whichever kernel path the batch would take.
    for field in ("b_down", "b_gate_up"):
        s = fake_layer(**{field: FAKE})
        assert fwd(lib, s) == moe.MOE_ERR_ARG, field
        assert ws_size(lib, s, 4)[0] == moe.MOE_ERR_ARG, field
        assert fwd(lib, fake_layer(path=moe.MOE_PATH_GROUPED, **{field: FAKE}), T=1000) == moe.MOE_ERR_ARG


def test_noalloc_argument_errors(lib):
    # Every check of moe_forward_noalloc runs before the scratch array's address is looked
    # up or anything is enqueued.
    s = fake_layer()
    L = ctypes.byref(s)
    assert lib.moe_forward_noalloc(L, FAKE, 0, FAKE * 2, None) == moe.MOE_OK
    assert lib.moe_forward_noalloc(L, FAKE, -1, FAKE * 2, None) == moe.MOE_ERR_ARG
    assert lib.moe_forward_noalloc(L, None, 4, FAKE * 2, None) == moe.MOE_ERR_ARG
    assert lib.moe_forward_noalloc(L, FAKE, 4, None, None) == moe.MOE_ERR_ARG
    assert lib.moe_forward_noalloc(L, FAKE, 4, FAKE, None) == moe.MOE_ERR_ARG       # y aliases x
    assert lib.moe_forward_noalloc(L, FAKE + 8, 4, FAKE * 2, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_forward_noalloc(None, FAKE, 4, FAKE * 2, None) == moe.MOE_ERR_ARG
    assert lib.moe_forward_noalloc(ctypes.byref(fake_layer(k=0)), FAKE, 4, FAKE * 2, None) == moe.MOE_ERR_ARG
    # A batch whose workspace exceeds the scratch array is refused.
    big = 1 << 16
    assert ws_size(lib, s, big)[1] > moe.NOALLOC_SCRATCH_BYTES
    assert lib.moe_forward_noalloc(L, FAKE, big, FAKE * 2, None) == moe.MOE_ERR_WORKSPACE


def test_workspace_size_covers_smaller_batches(lib):
    # One size query covers every batch of at most T tokens (the decode-only split-K
    # planes make some small batches' layouts larger than a slightly bigger batch's).
    s = fake_layer(d=2048, n_expert=256, k=8)
    sizes = [ws_size(lib, s, T)[1] for T in range(1, 200)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m, "MOE_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) << int(m.group(2)) == moe.NOALLOC_SCRATCH_BYTES


def test_q4k_layer_checks(lib):
    q4 = dict(expert_format=moe.MOE_EXPERTS_Q4K, d=512, ff=256)
    assert ws_size(lib, fake_layer(**q4), 4)[0] == moe.MOE_OK
    assert ws_size(lib, fake_layer(**dict(q4, path=moe.MOE_PATH_GROUPED)), 4)[0] == moe.MOE_OK
    assert ws_size(lib, fake_layer(**dict(q4, d=320)), 4)[0] == moe.MOE_ERR_UNSUPPORTED      # not a multiple of 256
    assert ws_size(lib, fake_layer(**dict(q4, ff=192)), 4)[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(lib, fake_layer(**dict(q4, d=8192)), 4)[0] == moe.MOE_ERR_UNSUPPORTED     # K > 4096
    assert ws_size(lib, fake_layer(**dict(q4, dtype=moe.MOE_F32)), 4)[0] == moe.MOE_ERR_UNSUPPORTED
    oai = dict(q4, act=moe.MOE_ACT_SWIGLU_OAI, w_gate_up=FAKE, b_gate_up=FAKE)
    assert ws_size(lib, fake_layer(**oai), 4)[0] == moe.MOE_ERR_UNSUPPORTED
    assert ws_size(lib, fake_layer(**dict(q4, w_down_scales=FAKE)), 4)[0] == moe.MOE_ERR_ARG
    sh = dict(q4, shared_ff=256, ws_gate=FAKE, ws_up=FAKE, ws_down=FAKE, ws_gate_inp=FAKE)
    assert ws_size(lib, fake_layer(**sh), 4)[0] == moe.MOE_OK                                # bf16 shared expert

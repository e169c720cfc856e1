"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and its host-only argument checks return the documented
status codes.  No compute call is made here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmoe.h")

lmoe = pytest.importorskip("sparse_moe_transformer_gemm_amd.lmoe")

if not os.path.exists(lmoe.LIB_PATH):
    pytest.skip("liblmoe.so not built", allow_module_level=True)

from synth import get_config  # noqa: E402


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lmoe_[a-z0-9_]+)\s*\(", src)))


def fake_weights(sh, **override):
    """Non-null host addresses: validation never dereferences them (no packed
    expert weights unless asked for)."""
    vals = {n: 0x1000 + 0x100 * i for i, n in enumerate(lmoe._WEIGHT_FIELDS)}
    vals["packed"] = None
    vals.update(override)
    return lmoe.Weights(**vals)


@pytest.fixture(scope="module")
def lib():
    return lmoe.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(lmoe.EXPORTS) <= set(names)
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lmoe.h but not exported"


def test_status_strings(lib):
    for code, name in lmoe.STATUS.items():
        assert lib.lmoe_status_str(code).decode() == name


def k3(**kw):
    d = dict(T=8192, H=7168, L=3584, E=896, k=16, I=1024, S=2, Is=1024, act="bf16", w_expert="bf16")
    d.update(kw)
    return lmoe.make_shape(**d)


def test_valid_layers_pass(lib):
    for name in ("tiny_f32", "small_bf16", "small_fp8", "small_w8a8", "small_identity_bf16", "k3_t8192",
                 "k3_fp8_t8192", "k3_w8a8_t8192", "fp8_448x8_l7168_t8192", "k3_zipf_t16384", "k3_decode_t64"):
        cfg = get_config(name)
        sh = lmoe.shape_of(cfg)
        over = {"w_down": None, "w_up": None} if cfg.identity_proj else {}
        w = fake_weights(sh, **over)
        need = lmoe.workspace_bytes(sh)
        assert need > 0
        assert lmoe.validate(sh, w, need) == 0, lmoe.last_error()
        assert lmoe.validate(sh, w, need - 1) == 3  # LMOE_EWORKSPACE


def test_workspace_grows_with_tokens(lib):
    a, b = lmoe.workspace_bytes(k3(T=64)), lmoe.workspace_bytes(k3(T=8192))
    assert 0 < a < b
    assert lmoe.workspace_bytes(k3(T=0)) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), 1),
    (dict(H=0), 1),
    (dict(k=0), 1),
    (dict(k=897), 1),
    (dict(S=-1), 1),
    (dict(cap=0.0), 1),
    (dict(cap=-5.0), 1),
    (dict(cap=float("nan")), 1),
    (dict(eps=-1e-6), 1),
    (dict(eps=float("inf")), 1),
    (dict(H=7160), 2),                       # not a multiple of 64
    (dict(L=8192 + 64, H=8256), 2),          # L above 8192
    (dict(E=1100, k=16), 2),
    (dict(k=65, E=128), 2),
    (dict(S=9), 2),
    (dict(w_expert="f8", L=3584 + 64), 2),   # fp8 needs multiples of 128
    (dict(act="f32"), 2),                    # f32 layer with bf16 experts
    (dict(act="bf16", w_expert="f32"), 2),
    (dict(T=(1 << 31) // 16), 2),            # T*k reaches 2^31
    (dict(a8=True), 2),                      # W8A8 with bf16 expert weights
    (dict(a8=True, w_expert="f32", act="f32"), 2),
])
def test_shape_errors(lib, kw, code):
    sh = k3(**kw)
    assert lmoe.validate(sh, fake_weights(sh), 1 << 40) == code
    assert lmoe.last_error()
    assert lmoe.workspace_bytes(sh) == 0


def test_act_fp8_is_unsupported(lib):
    sh = k3()
    sh.act = lmoe.F8E4M3
    assert lmoe.validate(sh, fake_weights(sh), 1 << 40) == 2


@pytest.mark.parametrize("field", ["w_router", "b_router", "w_gate", "w_value", "w_out", "gamma", "ws_gate",
                                   "ws_value", "ws_out"])
def test_missing_weight(lib, field):
    sh = k3()
    assert lmoe.validate(sh, fake_weights(sh, **{field: None}), 1 << 40) == 1
    assert field.split("_")[0] in lmoe.last_error() or "required" in lmoe.last_error()


def test_fp8_needs_scales(lib):
    sh = k3(w_expert="f8")
    assert lmoe.validate(sh, fake_weights(sh), 1 << 40) == 0
    for f in ("s_gate", "s_value", "s_out", "ss_gate", "ss_value", "ss_out"):
        assert lmoe.validate(sh, fake_weights(sh, **{f: None}), 1 << 40) == 1


def test_identity_projection_needs_square_latent(lib):
    sh = k3()
    assert lmoe.validate(sh, fake_weights(sh, w_down=None), 1 << 40) == 1
    assert lmoe.validate(sh, fake_weights(sh, w_up=None), 1 << 40) == 1
    sq = k3(L=7168, E=448, k=8)
    assert lmoe.validate(sq, fake_weights(sq, w_down=None, w_up=None), 1 << 40) == 0


def test_no_shared_experts_need_no_shared_weights(lib):
    sh = k3(S=0)
    assert lmoe.validate(sh, fake_weights(sh, ws_gate=None, ws_value=None, ws_out=None), 1 << 40) == 0


def test_null_shape_and_weights(lib):
    assert lib.lmoe_validate(None, None, 0) == 1
    sh = k3()
    assert lib.lmoe_validate(ctypes.byref(sh), None, 1 << 40) == 1


def test_misaligned_tensors_are_rejected(lib):
    """Matrices and activations move in 16-byte vectors: a base address that
    is not 16-byte aligned is EINVAL, named in the message, before any GPU
    call (weights through lmoe_validate, activations and gradients at the
    entry points)."""
    sh = k3(T=4)
    need = lmoe.workspace_bytes(sh)
    ws = ctypes.c_void_p(0x10000)
    assert lmoe.validate(sh, fake_weights(sh, w_gate=0x1008), 1 << 40) == 1
    assert "w_gate must be 16-byte aligned" in lmoe.last_error()
    assert lmoe.validate(sh, fake_weights(sh, ws_out=0x1004), 1 << 40) == 1
    w = fake_weights(sh)
    s = lib.lmoe_forward(ctypes.byref(sh), ctypes.byref(w), 0x2008, 0x3000, None, None, ws, need, None, None)
    assert s == 1 and "x must be 16-byte aligned" in lmoe.last_error()
    s = lib.lmoe_forward(ctypes.byref(sh), ctypes.byref(w), 0x2000, 0x3002, None, None, ws, need, None, None)
    assert s == 1 and "y must be 16-byte aligned" in lmoe.last_error()
    bneed = lib.lmoe_backward_workspace_bytes(ctypes.byref(sh))
    g = lmoe.Grads(**{n: 0x2000 + 0x100 * i for i, n in enumerate(lmoe.GRAD_FIELDS)})
    g.dw_value = 0x5008
    s = lib.lmoe_backward(ctypes.byref(sh), ctypes.byref(w), ctypes.c_void_p(0x8000), ctypes.c_void_p(0x9000), None,
                          ctypes.byref(g), ctypes.c_void_p(0x200000), bneed, None, None)
    assert s == 1 and "dw_value must be 16-byte aligned" in lmoe.last_error()


def test_entry_points_reject_before_any_gpu_call(lib):
    """Argument errors return before anything touches the device, so they are
    testable here: a short workspace, a misaligned one, null outputs."""
    sh = k3(T=4)
    w = fake_weights(sh)
    need = lmoe.workspace_bytes(sh)
    ws = ctypes.c_void_p(0x10000)
    s = lib.lmoe_forward(ctypes.byref(sh), ctypes.byref(w), 0x2000, 0x3000, None, None, ws, need - 1, None, None)
    assert s == 3
    s = lib.lmoe_forward(ctypes.byref(sh), ctypes.byref(w), 0x2000, 0x3000, None, None, ctypes.c_void_p(0x10010),
                         need, None, None)
    assert s == 1 and "aligned" in lmoe.last_error()
    s = lib.lmoe_route(ctypes.byref(sh), ctypes.byref(w), None, None, None, None, ws, need, None)
    assert s == 1
    s = lib.lmoe_permute(ctypes.byref(sh), None, None, None, None, ws, need, None)
    assert s == 1
    s = lib.lmoe_expert_gemm(ctypes.byref(sh), ctypes.byref(w), None, None, None, None, ws, need, None)
    assert s == 1
    s = lib.lmoe_combine_norm(ctypes.byref(sh), None, None, None, None, None, None)
    assert s == 1
    s = lib.lmoe_up(ctypes.byref(sh), ctypes.byref(w), None, None, None, ws, need, None)
    assert s == 1
    # an empty batch is a valid no-op that launches nothing
    sh0 = k3(T=0)
    need0 = lmoe.workspace_bytes(sh0)
    assert lib.lmoe_forward(ctypes.byref(sh0), ctypes.byref(w), None, None, None, None, ws, need0, None, None) == 0


def test_binding_refuses_host_tensors(lib):
    import torch
    cfg = get_config("small_bf16")
    sh = lmoe.shape_of(cfg)
    with pytest.raises(ValueError):
        lmoe.make_weights(sh, {"w_router": torch.zeros(cfg.E, cfg.H, dtype=torch.bfloat16)})


def test_packed_bytes(lib):
    sh = k3()
    blocks = 896 * (1024 // 128) * (3584 // 64) + 896 * (3584 // 256) * (1024 // 64)
    assert lmoe.packed_bytes(sh) == blocks * 32768
    # padding: gate/value tiles of 128 units, out tiles of 256 rows
    odd = k3(I=192, L=320)
    assert lmoe.packed_bytes(odd) == 896 * (2 * 5 + 2 * 3) * 32768
    assert lmoe.packed_bytes(k3(w_expert="f8")) == 0
    assert lmoe.packed_bytes(k3(act="f32", w_expert="f32")) == 0
    assert lmoe.packed_bytes(k3(T=-1)) == 0


def test_packed_weights_validation(lib):
    sh = k3()
    # packed expert weights replace the row-major stacks
    w = fake_weights(sh, packed=0x100000, w_gate=None, w_value=None, w_out=None)
    assert lmoe.validate(sh, w, 1 << 40) == 0
    assert lmoe.validate(sh, fake_weights(sh, packed=0x100010), 1 << 40) == 1
    assert "aligned" in lmoe.last_error()
    f8 = k3(w_expert="f8")
    assert lmoe.validate(f8, fake_weights(f8, packed=0x100000), 1 << 40) == 2


def test_pack_experts_rejects_before_any_gpu_call(lib):
    sh = k3()
    n = lmoe.packed_bytes(sh)
    w = fake_weights(sh)
    buf = ctypes.c_void_p(0x100000)
    assert lib.lmoe_pack_experts(ctypes.byref(sh), None, buf, n, None) == 1
    assert lib.lmoe_pack_experts(ctypes.byref(sh), ctypes.byref(fake_weights(sh, w_out=None)), buf, n, None) == 1
    assert lib.lmoe_pack_experts(ctypes.byref(sh), ctypes.byref(w), None, n, None) == 1
    assert lib.lmoe_pack_experts(ctypes.byref(sh), ctypes.byref(w), ctypes.c_void_p(0x100080), n, None) == 1
    assert lib.lmoe_pack_experts(ctypes.byref(sh), ctypes.byref(w), buf, n - 1, None) == 1
    assert "needed" in lmoe.last_error()
    f8 = k3(w_expert="f8")
    assert lib.lmoe_pack_experts(ctypes.byref(f8), ctypes.byref(fake_weights(f8)), buf, n, None) == 2


def test_router_logits_and_quantile_bias_reject_before_any_gpu_call(lib):
    sh = k3(T=64)
    w = fake_weights(sh)
    buf = ctypes.c_void_p(0x100000)
    assert lib.lmoe_router_logits(ctypes.byref(sh), None, buf, buf, None) == 1
    assert lib.lmoe_router_logits(ctypes.byref(sh), ctypes.byref(fake_weights(sh, w_router=None)), buf, buf, None) == 1
    assert lib.lmoe_router_logits(ctypes.byref(sh), ctypes.byref(w), None, buf, None) == 1
    sh0 = k3(T=0)
    assert lib.lmoe_router_logits(ctypes.byref(sh0), ctypes.byref(w), None, None, None) == 0  # empty batch: no-op
    need = lmoe.workspace_bytes(sh)
    assert lib.lmoe_quantile_bias(ctypes.byref(sh0), buf, buf, buf, need, None) == 1  # needs a token
    assert "at least one token" in lmoe.last_error()
    assert lib.lmoe_quantile_bias(ctypes.byref(sh), None, buf, buf, need, None) == 1
    assert lib.lmoe_quantile_bias(ctypes.byref(sh), buf, None, buf, need, None) == 1
    assert lib.lmoe_quantile_bias(ctypes.byref(sh), buf, buf, buf, need - 1, None) == 3


def test_a8_flag_values(lib):
    sh = k3(w_expert="f8", a8=True)
    assert lmoe.validate(sh, fake_weights(sh), lmoe.workspace_bytes(sh)) == 0, lmoe.last_error()
    # W8A8 needs the e4m3 copies of z and of the SiTU-GLU output
    assert lmoe.workspace_bytes(sh) > lmoe.workspace_bytes(k3(w_expert="f8"))
    sh.a8 = 2
    assert lmoe.validate(sh, fake_weights(sh), 1 << 40) == 1
    assert "a8" in lmoe.last_error()


def test_quantize_1x128_rejects_before_any_gpu_call(lib):
    buf = ctypes.c_void_p(0x100000)
    q = lib.lmoe_quantize_1x128
    assert q(buf, -1, 128, buf, buf, None) == 1
    assert q(buf, 4, 100, buf, buf, None) == 1
    assert q(buf, 4, 0, buf, buf, None) == 1
    assert q(buf, 0, 128, None, None, None) == 0  # empty: no-op
    assert q(None, 4, 128, buf, buf, None) == 1
    assert q(buf, 4, 128, None, buf, None) == 1
    assert q(buf, 4, 128, buf, None, None) == 1
    assert q(ctypes.c_void_p(0x100008), 4, 128, buf, buf, None) == 1  # x not 16-byte aligned
    assert "aligned" in lmoe.last_error()


def test_backward_rejects_before_any_gpu_call(lib):
    sh = k3(T=64)
    w = fake_weights(sh)
    need = lmoe.backward_workspace_bytes(sh)
    assert need > 0 and lmoe.backward_workspace_bytes(k3(T=8192)) > need
    buf = ctypes.c_void_p(0x100000)
    g = lmoe.Grads(**{n: 0x2000 + 0x100 * i for i, n in enumerate(lmoe.GRAD_FIELDS)})
    ws = ctypes.c_void_p(0x200000)
    bw = lib.lmoe_backward
    assert bw(ctypes.byref(sh), ctypes.byref(w), buf, buf, None, ctypes.byref(g), ws, need - 1, None, None) == 3
    assert bw(ctypes.byref(sh), ctypes.byref(w), buf, buf, None, None, ws, need, None, None) == 1
    g2 = lmoe.Grads(**{n: 0x2000 + 0x100 * i for i, n in enumerate(lmoe.GRAD_FIELDS)})
    g2.dw_out = None
    assert bw(ctypes.byref(sh), ctypes.byref(w), buf, buf, None, ctypes.byref(g2), ws, need, None, None) == 1
    assert bw(ctypes.byref(sh), ctypes.byref(w), None, buf, None, ctypes.byref(g), ws, need, None, None) == 1
    f8 = k3(T=64, w_expert="f8")
    assert bw(ctypes.byref(f8), ctypes.byref(fake_weights(f8)), buf, buf, None, ctypes.byref(g), ws, 1 << 40,
              None, None) == 2
    big = k3(T=70000)
    assert bw(ctypes.byref(big), ctypes.byref(fake_weights(big)), buf, buf, None, ctypes.byref(g), ws, 1 << 45,
              None, None) == 2
    packed_only = fake_weights(sh, w_gate=None, w_value=None, w_out=None, packed=0x9000)
    assert bw(ctypes.byref(sh), ctypes.byref(packed_only), buf, buf, None, ctypes.byref(g), ws, need, None, None) == 1


def test_forward_noalloc_rejects_before_any_gpu_call(lib):
    """The no-allocation entry point checks the shape, its scratch limit and
    the weights on the host first (EWORKSPACE names the limit), and an empty
    call returns before touching a device."""
    vp = ctypes.c_void_p
    big = k3()  # T = 8192: far more scratch than the fixed array holds
    assert lmoe.workspace_bytes(big) > lmoe.NOALLOC_SCRATCH_BYTES
    st = lib.lmoe_forward_noalloc(ctypes.byref(big), ctypes.byref(fake_weights(big)), vp(0x10), vp(0x20), None,
                                  None, None)
    assert st == 3 and "lmoe_forward_noalloc holds" in lmoe.last_error()
    small = k3(T=64)
    assert lmoe.workspace_bytes(small) <= lmoe.NOALLOC_SCRATCH_BYTES
    st = lib.lmoe_forward_noalloc(ctypes.byref(small), ctypes.byref(fake_weights(small, gamma=None)), vp(0x10),
                                  vp(0x20), None, None, None)
    assert st == 1 and "gamma" in lmoe.last_error()
    assert lib.lmoe_forward_noalloc(None, ctypes.byref(fake_weights(small)), vp(0x10), vp(0x20), None, None,
                                    None) == 1
    empty = k3(T=0)
    assert lib.lmoe_forward_noalloc(ctypes.byref(empty), ctypes.byref(fake_weights(empty)), None, None, None, None,
                                    None) == 0

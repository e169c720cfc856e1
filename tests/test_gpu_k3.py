"""GPU parity at the K3 layer shape (hidden 7168, latent 3584, 896 experts,
top-16, 2 shared experts, intermediate 1024): the whole batch runs on the GPU
in the launch configuration the benchmark times; the oracle checks the
selection of every token and the outputs of a seeded sample of rows (each
output row depends only on its own token)."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import lmoe_oracle as O
from synth import get_config, make_inputs, raw_numpy
from synth.inputs import make_router_bias, make_x

from gpu_common import check_selection, lazy_inputs, note, pick_rows, rowwise_rel_err, spec_of, to_f64, tol_of

pytestmark = pytest.mark.gpu

lmoe = pytest.importorskip("sparse_moe_transformer_gemm_amd.lmoe")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    lmoe.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def k3w(dev):
    """K3 bf16 weights (seed 1), generated on the device once for the module."""
    note("[k3] generating bf16 weights on the device")
    g = make_inputs(get_config("k3_t8192"), device=dev, with_x=False)
    torch.cuda.synchronize()
    yield g
    g.clear()
    torch.cuda.empty_cache()


def _route_all(g, x, cfg):
    """Oracle routing of every token (cheap next to the experts)."""
    x64 = O.decode(raw_numpy(x), cfg.act)
    return O.route(x64, O.decode(raw_numpy(g["w_router"]), cfg.act),
                   raw_numpy(g["b_router"]).astype(np.float64), cfg.k)


def _run(cfg, g, dev, sample=64, x=None):
    note(f"[k3] {cfg.name}: T={cfg.T} E={cfg.E} k={cfg.k} L={cfg.L} {cfg.act}/{cfg.w_expert} bias={cfg.bias}")
    x = make_x(cfg, dev) if x is None else x
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    y, idx, tw = lmoe.forward(sh, w, x)
    torch.cuda.synchronize()
    r = _route_all(g, x, cfg)
    idx_h = idx.cpu().numpy()
    sel = check_selection(idx_h, tw.cpu().numpy(), r)
    note(f"    selection: {sel['mismatch']}/{sel['tokens']} token sets differ from the oracle, all with gap < 1e-3 "
         f"(largest {sel['max_gap_mismatch']:.2e}); near-tie tokens {sel['near_tie_frac']:.3f}; "
         f"order compared on {sel['order_checked']} tokens")
    rows = pick_rows(idx_h, cfg.E, min(sample, cfg.T), bt=256, seed=cfg.T)  # 256-row expert token tiles
    inp = lazy_inputs(g, None)
    inp["x"] = raw_numpy(x[torch.as_tensor(rows, device=dev)])
    ref = O.forward(inp, spec_of(cfg), forced_idx=idx_h[rows].astype(np.int64), forced_tol=1e-5)
    err = rowwise_rel_err(to_f64(y[torch.as_tensor(rows, device=dev)]), ref["y"])
    note(f"    {len(rows)} sampled rows (first {rows[:6].tolist()} ... last {rows[-3:].tolist()}): "
         f"max row rel err {err:.3e} (tol {tol_of(cfg)})")
    assert err <= tol_of(cfg)
    return y, idx


def test_k3_t8192(dev, k3w):
    _run(get_config("k3_t8192"), k3w, dev, sample=256)


def test_k3_packed_matches_row_major(dev, k3w):
    """The benchmark's configuration: expert weights packed once, then the
    layer at T=8192 (256-row token tiles) and T=64 (32-row tiles); every output
    is bitwise equal to the row-major path, which the oracle checks above."""
    for name in ("k3_t8192", "k3_decode_t64"):
        cfg = get_config(name)
        note(f"[k3 packed] {name}")
        x = make_x(cfg, dev)
        sh = lmoe.shape_of(cfg)
        w = lmoe.make_weights(sh, k3w)
        y0, i0, _ = lmoe.forward(sh, w, x)
        pk = lmoe.pack_experts(sh, w)
        y1, i1, _ = lmoe.forward(sh, lmoe.with_packed(sh, w, pk), x)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1)
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        del pk, y0, y1
        torch.cuda.empty_cache()


def test_k3_prefill_and_decode_batch_invariant(dev, k3w):
    cfg = get_config("k3_prefill_t2048")
    y, idx = _run(cfg, k3w, dev)
    dcfg = get_config("k3_decode_t64")
    xd = make_x(dcfg, dev)
    assert torch.equal(xd, make_x(cfg, dev)[:64])  # the decode batch is the first 64 prefill tokens
    yd, idd = _run(dcfg, k3w, dev, x=xd)
    assert torch.equal(idd, idx[:64])
    assert torch.equal(yd, y[:64])


def test_k3_t2100_recut_router_tiles(dev, k3w):
    """T = 2100: the route GEMM's 9 x 34 tiles leave a last round of 50,
    re-cut into 128 x 128 sub-tiles, and it holds the last token tile's
    router tiles; the second half of the last one (features 896 .. 1023)
    lies wholly past E, so its DMAs must read inside W_router.  Oracle on
    every token's selection and on sampled rows, and the first 2048 rows
    bitwise equal to the T = 2048 batch (whose router tiles all run as
    256 x 256 tiles)."""
    base = get_config("k3_prefill_t2048")
    cfg = replace(base, name="k3_prefill_t2100", T=2100)
    x = make_x(cfg, dev)
    assert torch.equal(x[:2048], make_x(base, dev))  # the T = 2048 batch is a prefix
    y, idx = _run(cfg, k3w, dev, x=x)
    y0, idx0 = _run(base, k3w, dev, sample=16, x=x[:2048].contiguous())
    assert torch.equal(idx[:2048], idx0)
    assert torch.equal(y[:2048], y0)


def test_k3_zipf_t16384(dev, k3w):
    cfg = get_config("k3_zipf_t16384")
    g = dict(k3w)
    g["b_router"] = make_router_bias(cfg, dev)
    y, idx = _run(cfg, g, dev)
    counts = torch.bincount(idx.flatten().long(), minlength=cfg.E)
    note(f"    tokens per expert: max {int(counts.max())}, min {int(counts.min())}")
    assert int(counts.max()) == cfg.T  # the most favoured expert is in every token's top-16


@pytest.mark.parametrize("name", ["k3_fp8_t8192", "k3_w8a8_t8192", "fp8_448x8_l7168_t8192",
                                  "k3_448x8_identity_t8192"])
def test_comparison_layers(dev, k3w, name):
    """fp8 expert weights at the K3 shape, and the 448/8 layer at latent 7168:
    with a real square projection (fp8) and with none (bf16)."""
    cfg = get_config(name)
    note(f"[k3] generating {name} weights on the device")
    g = make_inputs(cfg, device=dev, with_x=False)
    try:
        _run(cfg, g, dev)
    finally:
        g.clear()
        torch.cuda.empty_cache()


def test_k3_backward_t2048(dev, k3w):
    """The K3 layer's backward at T = 2048: sampled dx rows against the
    oracle (a token's dx depends on that token alone), and at full size the
    property that the weight gradients of the batch are the sums of those of
    its two halves (each token's selection is its own)."""
    cfg = get_config("k3_prefill_t2048")
    note(f"[k3 backward] {cfg.name}")
    x = make_x(cfg, dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, k3w)
    gen = torch.Generator(device=dev).manual_seed(78)
    dy = torch.randn((cfg.T, cfg.H), generator=gen, device=dev).to(torch.bfloat16)
    slices = {"dw_router": lambda t: t, "dw_down": lambda t: t, "dw_up": lambda t: t, "dgamma": lambda t: t,
              "dws_gate": lambda t: t[:, :64], "dws_out": lambda t: t[:, :, :64],
              "dw_gate": lambda t: t[:64:9], "dw_value": lambda t: t[5:200:13], "dw_out": lambda t: t[::97]}

    def run(lo, hi):
        s2 = lmoe.shape_of(cfg, T=hi - lo)
        grads, idx = lmoe.backward(s2, w, x[lo:hi].contiguous(), dy[lo:hi].contiguous())
        torch.cuda.synchronize()
        out = {n: f(grads[n]).double().cpu() for n, f in slices.items()}
        dx = grads["dx"].double().cpu()
        del grads
        torch.cuda.empty_cache()
        return out, dx, idx

    full, dx_full, idx = run(0, cfg.T)
    a, dx_a, _ = run(0, cfg.T // 2)
    b, dx_b, _ = run(cfg.T // 2, cfg.T)
    for n in slices:
        ref = full[n]
        err = float((a[n] + b[n] - ref).abs().max() / ref.abs().max())
        note(f"    {n:10s} halves vs whole: rel {err:.2e}")
        assert err <= 1e-4, n
    assert torch.equal(torch.cat([dx_a, dx_b]), dx_full)  # a token's dx is its own, bit for bit

    rows = np.sort(np.random.default_rng(79).choice(cfg.T, size=4, replace=False))
    rt = torch.as_tensor(rows, device=dev)
    inp = lazy_inputs(k3w, None)
    inp["x"] = raw_numpy(x[rt])
    ref = O.backward(inp, spec_of(cfg), O.bf16_bits_to_f64(raw_numpy(dy[rt])),
                     forced_idx=idx[rt].cpu().numpy().astype(np.int64), forced_tol=1e-5)
    err = rowwise_rel_err(dx_full[torch.from_numpy(rows)].numpy(), ref["dx"])
    note(f"    dx rows {rows.tolist()}: max row rel err {err:.3e}")
    assert err <= 2e-2

"""GPU parity of Quantile Balancing (the per-expert threshold solve that
produces the router's selection bias) and of the router-logits entry point,
against the fp64 oracle; and the balancing it brings to a skewed router."""

import numpy as np
import pytest
import torch

from oracle import lmoe_oracle as O
from synth import get_config, make_inputs, raw_numpy
from synth.inputs import make_router_logits

from gpu_common import check_selection, make_case, note

pytestmark = pytest.mark.gpu

lmoe = pytest.importorskip("sparse_moe_transformer_gemm_amd.lmoe")

# |tau_gpu - tau_oracle| <= max_t |s_gpu - s_oracle| (an order statistic is
# 1-Lipschitz in the sup norm, and so is the interpolation between two); the
# fp32 sigmoid is within a few units in the last place of 1 (2^-23).
TAU_TOL = 1e-6


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    lmoe.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("T,E,k,spread", [(1, 8, 2, 0.0), (2, 8, 3, 0.0), (37, 16, 2, 1.0), (1000, 24, 4, 3.0),
                                          (8192, 896, 16, 0.0), (8192, 896, 16, 4.0), (333, 48, 48, 0.0)])
def test_quantile_bias_matches_oracle(dev, T, E, k, spread):
    note(f"[quantile] T={T} E={E} k={k} spread={spread}")
    lg = make_router_logits(T, E, seed=11, spread=spread)
    sh = lmoe.make_shape(T=T, H=256, L=128, E=E, k=k, I=128, S=0, Is=0, act="bf16", w_expert="bf16")
    b = lmoe.quantile_bias(sh, torch.from_numpy(lg).to(dev))
    torch.cuda.synchronize()
    ref = O.quantile_bias(lg.astype(np.float64), k)
    err = float(np.abs(b.cpu().numpy().astype(np.float64) - ref).max())
    note(f"    max |bias - oracle| = {err:.3e}")
    assert err <= TAU_TOL


def test_quantile_bias_balances_skewed_logits(dev):
    """Selection on s + b with the GPU's bias: every expert lands near its fair
    share T k / E, where the plain selection piles tokens on a few."""
    T, E, k = 8192, 896, 16
    lg = make_router_logits(T, E, seed=12, spread=4.0)
    sh = lmoe.make_shape(T=T, H=256, L=128, E=E, k=k, I=128, S=0, Is=0, act="bf16", w_expert="bf16")
    b = lmoe.quantile_bias(sh, torch.from_numpy(lg).to(dev)).cpu().numpy().astype(np.float64)
    s = O.sigmoid(lg.astype(np.float64))
    plain = np.bincount(O.select_topk(s, k)[0].ravel(), minlength=E)
    qb = np.bincount(O.select_topk(s + b[None, :], k)[0].ravel(), minlength=E)
    fair = T * k / E
    note(f"    max load: plain {plain.max()}, balanced {qb.max()} (fair {fair:.1f})")
    assert plain.max() > 5 * fair
    assert qb.max() < 2 * fair and qb.min() > 0.5 * fair


@pytest.mark.parametrize("name", ["small_bf16", "tiny_f32"])
def test_router_logits_and_balanced_layer(dev, name):
    """lmoe_router_logits against the oracle's x W_r^T, then the layer run
    with the Quantile Balancing bias of its own batch: the selection agrees
    with the oracle's under that bias (near-tie rule)."""
    cfg = get_config(name)
    note(f"[router logits + balanced layer] {name}")
    t, g = make_case(cfg, dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    lg = lmoe.router_logits(sh, w, g["x"])
    torch.cuda.synchronize()
    x64 = O.decode(raw_numpy(g["x"]), cfg.act)
    wr64 = O.decode(raw_numpy(g["w_router"]), cfg.act)
    ref = x64 @ wr64.T
    scale = np.abs(x64).max() * np.abs(wr64).max() * cfg.H
    lerr = float(np.abs(lg.cpu().numpy().astype(np.float64) - ref).max())
    note(f"    logits max err {lerr:.3e} (scale {scale:.3e})")
    assert lerr <= 1e-5 * scale
    bias = lmoe.quantile_bias(sh, lg)
    gb = dict(g)
    gb["b_router"] = bias
    y, idx, tw = lmoe.forward(sh, lmoe.make_weights(sh, gb), g["x"])
    torch.cuda.synchronize()
    r = O.route(x64, wr64, bias.cpu().numpy().astype(np.float64), cfg.k)
    check_selection(idx.cpu().numpy(), tw.cpu().numpy(), r)

"""GPU parity of the layer backward (lmoe_backward) against the fp64 oracle's
gradients on the same input bytes: every gradient tensor, on layers with and
without projections and shared experts, with k == E, with several 128-row
tiles per expert, and on an empty batch."""

from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import lmoe_oracle as O
from synth import get_config

from gpu_common import host_inputs, make_case, note, spec_of

pytestmark = pytest.mark.gpu

lmoe = pytest.importorskip("sparse_moe_transformer_gemm_amd.lmoe")

# bf16 operands (rounded once on their way into each GEMM) with fp32
# accumulation: the same budget as the bf16 forward, per gradient tensor.
TOL = 2e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    lmoe.load_library()
    return torch.device("cuda:0")


def _dy(cfg, dev):
    gen = torch.Generator().manual_seed(1000 + cfg.T)
    return torch.randn((cfg.T, cfg.H), generator=gen).to(torch.bfloat16)


def _rel(got, want):
    """Largest error over the tensor relative to its largest reference value."""
    scale = np.abs(want).max() if want.size else 0.0
    if scale == 0.0:
        return float(np.abs(got).max()) if got.size else 0.0
    return float(np.abs(got - want).max() / scale)


def _run(cfg, dev):
    note(f"[backward] {cfg.name} T={cfg.T} H={cfg.H} L={cfg.L} E={cfg.E} k={cfg.k} S={cfg.S} I={cfg.I}")
    t, g = make_case(cfg, dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    dy = _dy(cfg, dev)
    grads, idx = lmoe.backward(sh, w, g["x"], dy.to(dev))
    torch.cuda.synchronize()
    inp = host_inputs(t)
    ref = O.backward(inp, spec_of(cfg), O.bf16_bits_to_f64(dy.view(torch.int16).numpy().astype(np.uint16)),
                     forced_idx=idx.cpu().numpy().astype(np.int64), forced_tol=1e-5)
    worst = 0.0
    for name, tns in grads.items():
        got = tns.cpu().numpy().astype(np.float64)
        err = _rel(got, ref[name])
        note(f"    {name:10s} {tuple(tns.shape)}: rel err {err:.3e}")
        worst = max(worst, err)
        assert err <= TOL, name
    return grads, ref, worst


@pytest.mark.parametrize("name,T,E", [("small_bf16", None, None), ("small_identity_bf16", None, None),
                                      ("small_full_k", None, None), ("small_bf16", 40, None), ("small_bf16", 700, None),
                                      ("small_wide_bf16", None, None), ("small_wide_bf16", 700, 8),
                                      ("small_bf16", 700, 64), ("small_identity_bf16", 700, 64)])
def test_backward_matches_oracle(dev, name, T, E):
    """small_wide_bf16 runs the persistent expert-gradient kernels: at its own
    size some of the 160 experts get no rows (their weight gradients must be
    exact zeros), and at T = 700 over 8 experts each expert spans several
    64-row k-tiles with a partial last one.  E = 64 at T = 700 routes the
    router's dx through the persistent data-gradient engine (with the latent
    segment, or alone onto dx when there is no latent projection)."""
    cfg = get_config(name)
    if T is not None:
        cfg = replace(cfg, T=T, name=f"{name}_T{T}")
    if E is not None:
        cfg = replace(cfg, E=E, name=f"{cfg.name}_E{E}")
    grads, ref, _ = _run(cfg, dev)
    # experts no token chose get exact zeros
    counts = np.bincount(ref["idx"].ravel(), minlength=cfg.E)
    if name == "small_wide_bf16" and E is None:
        assert (counts == 0).any(), "the case is meant to hold experts without rows"
    for e in np.nonzero(counts == 0)[0]:
        for n in ("dw_gate", "dw_value", "dw_out"):
            assert not grads[n][int(e)].any()


def test_backward_ragged_dense_tiles(dev):
    """H = 576 and S * Is = 2 * 192 leave the dense data gradients (dx, dh)
    with a partial last 256-feature tile, and one tile of dh spans both
    shared experts' out matrices."""
    cfg = replace(get_config("small_bf16"), T=700, H=576, Is=192, name="small_bf16_T700_H576_Is192")
    _run(cfg, dev)


def test_backward_empty_batch(dev):
    cfg = replace(get_config("small_bf16"), T=0, name="small_bf16_T0")
    t, g = make_case(cfg, dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    grads = {n: torch.full(s, 7.0, device=dev) for n, s in lmoe.grad_shapes(sh, w).items()}
    lmoe.backward(sh, w, g["x"], torch.empty((0, cfg.H), dtype=torch.bfloat16, device=dev), grads=grads)
    torch.cuda.synchronize()
    for n, tns in grads.items():
        assert not tns.any(), n


def test_backward_deterministic(dev):
    cfg = get_config("small_bf16")
    t, g = make_case(cfg, dev)
    sh = lmoe.shape_of(cfg)
    w = lmoe.make_weights(sh, g)
    dy = _dy(cfg, dev).to(dev)
    a, ia = lmoe.backward(sh, w, g["x"], dy)
    b, ib = lmoe.backward(sh, w, g["x"], dy)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib)
    for n in a:
        assert torch.equal(a[n], b[n]), n

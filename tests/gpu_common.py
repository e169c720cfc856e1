"""Helpers shared by the GPU parity tests: upload seeded inputs, run the
oracle on the same bytes, and compare."""

import sys

import numpy as np
import torch

from oracle import lmoe_oracle as O
from synth import make_inputs, raw_numpy
from synth.inputs import LazyExperts

# Output tolerances: max over tokens of |y_t - r_t|_inf / |r_t|_inf.  bf16 and
# fp8 bars are the layer's stated targets; fp32 is derived from fp32
# accumulation over K <= 8192 terms (about 1e-6 relative) with margin.
TOL = {"f32": 1e-4, "bf16": 2e-2, "f8": 6e-2}
# Selection: expert sets must agree where the oracle's k-th and (k+1)-th biased
# scores differ by at least this much.
GAP = 1e-3
# The GPU's selection must be a valid top-k of the oracle's fp64 scores within
# this margin (fp32 sigmoid of fp32-accumulated logits).
SEL_TOL = 1e-5


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def tol_of(cfg):
    return TOL["f8"] if cfg.w_expert == "f8" else TOL[cfg.act]


def spec_of(cfg):
    return dict(act=cfg.act, w_expert=cfg.w_expert, k=cfg.k, cap=cfg.cap, eps=cfg.eps, a8=cfg.a8)


def upload(t, dev):
    return {k: (v.to(dev) if v is not None else None) for k, v in t.items()}


def host_inputs(t):
    return {k: raw_numpy(v) for k, v in t.items()}


def lazy_inputs(g, x_rows=None):
    """Oracle inputs straight from device tensors: dense tensors copied, expert
    stacks fetched expert by expert; x restricted to `x_rows`."""
    out = {}
    for k, v in g.items():
        if v is None:
            out[k] = None
        elif k in ("w_gate", "w_value", "w_out", "s_gate", "s_value", "s_out"):
            out[k] = LazyExperts(v)
        elif k == "x" and x_rows is not None:
            out[k] = raw_numpy(v[torch.as_tensor(x_rows, device=v.device)])
        else:
            out[k] = raw_numpy(v)
    return out


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(raw_numpy(t))
    return t.detach().double().cpu().numpy()


def rowwise_rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.shape[0] == 0:
        return 0.0
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float((num / np.maximum(den, 1e-300)).max())


def check_selection(idx_gpu, w_gpu, ref, gap=GAP):
    """Expert sets equal where the oracle's gap >= `gap`; everywhere a valid
    top-k within SEL_TOL; weights equal to the oracle's renormalised scores of
    the GPU's selection.  Returns (strict mismatches, tokens compared)."""
    idx = np.asarray(idx_gpu, np.int64)
    T = idx.shape[0]
    if T == 0:
        return 0, 0
    O.check_forced(ref["biased"], idx, SEL_TOL)
    sure = ref["gap"] >= gap
    mism = [t for t in range(T) if set(idx[t]) != set(ref["idx"][t].tolist())]
    bad = [t for t in mism if sure[t]]
    assert not bad, f"{len(bad)} tokens with gap >= {gap} select other experts, e.g. token {bad[0]}"
    wref = O.combine_weights(ref["scores"], idx)
    np.testing.assert_allclose(np.asarray(w_gpu, np.float64), wref, rtol=1e-4, atol=1e-6)
    return len(mism), T


def make_case(cfg, dev):
    """Seeded inputs generated on the host (so the oracle reads them as they
    are) and uploaded."""
    t = make_inputs(cfg, device="cpu")
    return t, upload(t, dev)

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


# Order: on tokens whose oracle biased scores around the top k (the k+1
# largest, sorted) all differ by at least this much, the GPU's list must equal
# the oracle's in order (descending biased score).
ORDER_GAP = 1e-5


def adjacent_gaps(biased, k):
    """Smallest difference between consecutive scores among each token's k+1
    largest biased scores (inf when k == E)."""
    b = np.asarray(biased, np.float64)
    E = b.shape[1]
    if k >= E:
        top = -np.sort(-b, axis=1)
    else:
        top = -np.sort(-np.partition(b, E - k - 1, axis=1)[:, E - k - 1:], axis=1)
    if top.shape[1] < 2:
        return np.full(b.shape[0], np.inf)
    return (top[:, :-1] - top[:, 1:]).min(axis=1)


def check_selection(idx_gpu, w_gpu, ref, gap=GAP):
    """Expert sets equal where the oracle's gap >= `gap`; everywhere a valid
    top-k within SEL_TOL; the order equal to the oracle's wherever the k+1
    leading scores are ORDER_GAP apart; weights equal to the oracle's
    renormalised scores of the GPU's selection.  Returns a summary: strict
    set mismatches over all tokens, tokens compared, the near-tie fraction
    (oracle gap < `gap`), the largest oracle gap among mismatches and the
    number of tokens whose order was compared."""
    idx = np.asarray(idx_gpu, np.int64)
    T = idx.shape[0]
    if T == 0:
        return dict(mismatch=0, tokens=0, near_tie_frac=0.0, max_gap_mismatch=0.0, order_checked=0)
    k = idx.shape[1]
    O.check_forced(ref["biased"], idx, SEL_TOL)
    sure = ref["gap"] >= gap
    ridx = np.asarray(ref["idx"], np.int64)
    mism = np.array([set(idx[t]) != set(ridx[t].tolist()) for t in range(T)])
    bad = np.nonzero(mism & sure)[0]
    assert bad.size == 0, f"{bad.size} tokens with gap >= {gap} select other experts, e.g. token {bad[0]}"
    ordered = adjacent_gaps(ref["biased"], k) >= ORDER_GAP
    wrong = np.nonzero(ordered & (idx != ridx).any(axis=1))[0]
    assert wrong.size == 0, (f"{wrong.size} tokens with well-separated scores list their experts in another "
                             f"order, e.g. token {wrong[0]}: {idx[wrong[0]].tolist()} vs {ridx[wrong[0]].tolist()}")
    wref = O.combine_weights(ref["scores"], idx)
    np.testing.assert_allclose(np.asarray(w_gpu, np.float64), wref, rtol=1e-4, atol=1e-6)
    return dict(mismatch=int(mism.sum()), tokens=T, near_tie_frac=float((~sure).mean()),
                max_gap_mismatch=float(np.asarray(ref["gap"])[mism].max()) if mism.any() else 0.0,
                order_checked=int(ordered.sum()))


def pick_rows(idx, E, n, bt=256, seed=0):
    """Up to `n` token rows for sampled output checks at large T: the first
    and last tokens; the tokens in the final (partial) token tile of the
    busiest expert; tokens of the highest-numbered experts that hold rows
    (their tiles come last in the expert tile list, so the persistent GEMMs
    reach them at the end of a work-group's walk); the rest seeded at random."""
    idx = np.asarray(idx, np.int64)
    T = idx.shape[0]
    rows = [0, T - 1]
    counts = np.bincount(idx.ravel(), minlength=E)
    hot = int(counts.argmax())
    toks = np.nonzero((idx == hot).any(axis=1))[0]
    rows += toks[(len(toks) - 1) // bt * bt:][-16:].tolist()
    for e in np.nonzero(counts)[0][::-1][:4]:
        rows += np.nonzero((idx == e).any(axis=1))[0][-4:].tolist()
    rows = list(dict.fromkeys(rows))[:n]
    rest = np.setdiff1d(np.arange(T), rows)
    if n > len(rows) and rest.size:
        rows += np.random.default_rng(seed).choice(rest, size=min(n - len(rows), rest.size), replace=False).tolist()
    return np.sort(np.array(rows, np.int64))


def make_case(cfg, dev):
    """Seeded inputs generated on the host (so the oracle reads them as they
    are) and uploaded."""
    t = make_inputs(cfg, device="cpu")
    return t, upload(t, dev)

"""Pins of the fp64 oracle against things other than itself.

The pages print no worked example, so the oracle is pinned by library
routines (torch / scipy in float64), closed forms, invariants the layer's
definition fixes, and brute force on tiny inputs.  The last test plants a
set of plausible mistakes in the oracle and checks that each one breaks at
least one pin.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import lmoe_oracle as O
from synth import get_config, make_inputs, raw_numpy
from synth.inputs import quantize_e4m3_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def rand_layer(seed, T=9, H=12, L=10, E=6, k=2, S=1, I=5, Is=4, identity=False,
               wstd=0.35, cap=100.0, eps=1e-6):
    rng = np.random.default_rng(seed)
    if identity:
        L = H
    inp = dict(
        x=rng.standard_normal((T, H)),
        w_router=rng.standard_normal((E, H)) * wstd,
        b_router=np.zeros(E, np.float32),
        w_down=None if identity else rng.standard_normal((L, H)) * wstd,
        w_gate=rng.standard_normal((E, I, L)) * wstd,
        w_value=rng.standard_normal((E, I, L)) * wstd,
        w_out=rng.standard_normal((E, L, I)) * wstd,
        gamma=rng.uniform(0.5, 1.5, L).astype(np.float32),
        w_up=None if identity else rng.standard_normal((H, L)) * wstd,
        ws_gate=rng.standard_normal((S, Is, H)) * wstd if S else None,
        ws_value=rng.standard_normal((S, Is, H)) * wstd if S else None,
        ws_out=rng.standard_normal((S, H, Is)) * wstd if S else None,
    )
    spec = dict(act="f64", w_expert="f64", k=k, cap=cap, eps=eps)
    return inp, spec


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def torch_shared(inp, c):
    """Shared experts written with torch's own linear / silu / tanh."""
    x = t64(inp["x"])
    y = torch.zeros_like(x)
    if inp.get("ws_gate") is None:
        return y.numpy()
    for s in range(len(inp["ws_gate"])):
        g = F.linear(x, t64(inp["ws_gate"][s]))
        v = F.linear(x, t64(inp["ws_value"][s]))
        if math.isfinite(c):
            g, v = c * torch.tanh(g / c), c * torch.tanh(v / c)
        y += F.linear(F.silu(g) * v, t64(inp["ws_out"][s]))
    return y.numpy()


def close(a, b, rtol=1e-11, atol=1e-12):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


# ----------------------------------------------------------------------------
# pins (plain functions so the mutant test below can rerun them)
# ----------------------------------------------------------------------------

def pin_bf16_decode():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.bf16_bits_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def pin_e4m3fn_decode():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3fn_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def pin_dequant_blocks():
    rng = np.random.default_rng(7)
    w = torch.from_numpy(rng.standard_normal((256, 384)).astype(np.float32) * 0.02)
    q, s = quantize_e4m3_blocks(w)
    q8 = q.view(torch.uint8).numpy()
    deq = O.dequant_blocks(q8, s.numpy())
    # element by element from the block definition
    for r in range(0, 256, 37):
        for c in range(0, 384, 29):
            assert deq[r, c] == O.E4M3FN[q8[r, c]] * float(s.numpy()[r // 128, c // 128])
    # e4m3 keeps 3 mantissa bits: round-to-nearest error <= 2^-4 relative for
    # normal codes (|q| >= 2^-6), <= half the subnormal step 2^-10 below that.
    wf = w.double().numpy()
    sc = np.repeat(np.repeat(s.double().numpy(), 128, 0), 128, 1)
    qa = np.abs(wf / sc)
    err = np.abs(deq - wf)
    normal = qa >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(wf[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * sc[~normal] * (1 + 1e-6))


def pin_sigmoid_silu_vs_libraries():
    u = np.linspace(-40, 40, 2001)
    close(O.sigmoid(u), scipy.special.expit(u), rtol=1e-14, atol=1e-300)
    close(O.silu(u), F.silu(t64(u)).numpy(), rtol=1e-13, atol=1e-300)


def pin_situ_near_zero_is_swiglu():
    g, v = np.meshgrid(np.linspace(-1, 1, 201), np.linspace(-1, 1, 201))
    swiglu = (F.silu(t64(g)) * t64(v)).numpy()
    d = np.abs(O.situ_glu(g, v, 100.0) - swiglu)
    assert d.max() < 1e-4
    assert d.max() > 0  # the cap really is applied


def pin_situ_bounded():
    u = np.array([-1e12, -1e6, -3e3, -150.0, 150.0, 3e3, 1e6, 1e12])
    cu = O.cap(u, 100.0)
    assert np.all(np.abs(cu) <= 100.0)
    close(O.cap(np.array([-1e9, 1e9]), 100.0), [-100.0, 100.0], rtol=0, atol=1e-12)
    g, v = np.meshgrid(u, u)
    s = O.situ_glu(g, v, 100.0)
    assert np.all(np.isfinite(s)) and np.abs(s).max() <= 1e4
    # at saturation the unit behaves like silu(100) * (+-100) = +-1e4
    assert abs(O.situ_glu(np.array(1e9), np.array(1e9), 100.0) - 1e4) < 1e-6


def pin_cap_closed_forms():
    u = np.linspace(-300, 300, 1201)
    close(O.cap(-u, 100.0), -O.cap(u, 100.0), rtol=0, atol=0)
    close(O.silu(u) - O.silu(-u), u, rtol=1e-12, atol=1e-12)
    # tanh series: c*tanh(u/c) = u - u^3/(3c^2) + 2u^5/(15c^4) - ...
    s = np.linspace(-2, 2, 41)
    assert np.all(np.abs(O.cap(s, 100.0) - (s - s ** 3 / 3e4)) <= 2 * np.abs(s) ** 5 / 15e8 + 1e-15)
    # no cap: exactly SwiGLU
    g, v = np.meshgrid(np.linspace(-50, 50, 101), np.linspace(-50, 50, 101))
    close(O.situ_glu(g, v, math.inf), (F.silu(t64(g)) * t64(v)).numpy(), rtol=1e-14, atol=0)


def pin_topk_bruteforce():
    rng = np.random.default_rng(11)
    for trial in range(20):
        T, E = 7, 1 + trial % 12
        k = 1 + trial % E
        # few distinct values so ties are frequent
        biased = rng.integers(0, 4, size=(T, E)).astype(np.float64) / 4
        idx, gap = O.select_topk(biased, k)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-biased[t, e], e))
            assert list(idx[t]) == order[:k]
            want = biased[t, order[k - 1]] - biased[t, order[k]] if k < E else math.inf
            assert gap[t] == want


def pin_topk_k_equals_E():
    rng = np.random.default_rng(12)
    b = rng.standard_normal((5, 9))
    idx, gap = O.select_topk(b, 9)
    assert all(sorted(r) == list(range(9)) for r in idx.tolist())
    assert np.all(np.isinf(gap))


def pin_route_library_and_invariants():
    inp, spec = rand_layer(21, T=11, E=9, k=3)
    x, wr = inp["x"], inp["w_router"]
    r = O.route(x, wr, np.zeros(9), 3)
    close(r["logits"], F.linear(t64(x), t64(wr)).numpy())
    close(r["scores"], scipy.special.expit(r["logits"]), rtol=1e-14, atol=0)
    # combine weights sum to 1 and are proportional to the chosen scores
    close(r["w"].sum(1), np.ones(11))
    sel = np.take_along_axis(r["scores"], r["idx"], 1)
    close(r["w"][:, 0:1] * sel, sel[:, 0:1] * r["w"])
    # a constant bias shift leaves the selection unchanged
    r2 = O.route(x, wr, np.full(9, 0.37), 3)
    assert np.array_equal(r["idx"], r2["idx"])
    # x = 0: every score is 1/2, selection follows the bias, weights uniform
    b = np.array([0.1, 0.5, 0.5, -0.2, 0.9, 0.0, 0.3, 0.5, 0.2])
    r0 = O.route(np.zeros((2, x.shape[1])), wr, b, 3)
    assert r0["idx"].tolist() == [[4, 1, 2]] * 2
    close(r0["w"], np.full((2, 3), 1 / 3))


def pin_permute_bruteforce():
    rng = np.random.default_rng(31)
    E, T, k = 7, 13, 3
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    offsets, srt, pos = O.permute(idx, E)
    want = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    want.append(t * k + j)
    assert srt.tolist() == want
    assert offsets.tolist() == [0] + list(np.cumsum([np.sum(idx == e) for e in range(E)]))
    assert np.array_equal(srt[pos], np.arange(T * k))


def pin_rmsnorm_vs_torch():
    rng = np.random.default_rng(41)
    c = rng.standard_normal((6, 33)) * 3
    g = rng.uniform(0.5, 1.5, 33)
    close(O.rmsnorm(c, g, 1e-6), F.rms_norm(t64(c), (33,), weight=t64(g), eps=1e-6).numpy())
    n = O.rmsnorm(c, g, 0.0)
    close(np.sqrt(np.mean((n / g) ** 2, axis=1)), np.ones(6))
    assert np.all(O.rmsnorm(np.zeros((2, 33)), g, 1e-6) == 0)


def pin_layer_dense_reduction():
    """E=1, k=1, L=H, identity projections, no shared expert: the layer is
    RMSNorm of one gated FFN.  With no cap that is RMSNorm(SwiGLU FFN)."""
    for c in (math.inf, 100.0):
        inp, spec = rand_layer(51, T=8, H=10, E=1, k=1, S=0, I=7, identity=True, cap=c)
        eye = np.eye(10)
        inp["w_down"], inp["w_up"] = eye, eye
        scale = 1.0 if math.isinf(c) else 300.0  # push the gate past the cap
        inp["x"] = inp["x"] * scale
        y = O.forward(inp, spec)["y"]
        x = t64(inp["x"])
        g = F.linear(x, t64(inp["w_gate"][0]))
        v = F.linear(x, t64(inp["w_value"][0]))
        if math.isfinite(c):
            assert g.abs().max() > 150
            g, v = c * torch.tanh(g / c), c * torch.tanh(v / c)
        h = F.linear(F.silu(g) * v, t64(inp["w_out"][0]))
        ref = F.rms_norm(h, (10,), weight=t64(inp["gamma"]), eps=1e-6)
        close(y, ref.numpy())


def pin_layer_shared_only():
    inp, spec = rand_layer(52, S=2, Is=3)
    inp["w_out"] = np.zeros_like(inp["w_out"])
    out = O.forward(inp, spec)
    assert np.all(out["n"] == 0)
    close(out["y"], torch_shared(inp, spec["cap"]))
    inp["x"] = inp["x"] * 500  # saturate the shared experts' caps too
    close(O.forward(inp, spec)["y"], torch_shared(inp, spec["cap"]), rtol=1e-10)


def pin_layer_token_permutation():
    inp, spec = rand_layer(53, T=12)
    a = O.forward(inp, spec)
    perm = np.random.default_rng(0).permutation(12)
    inp2 = dict(inp, x=inp["x"][perm])
    b = O.forward(inp2, spec)
    close(b["y"], a["y"][perm])
    assert np.array_equal(b["idx"], a["idx"][perm])


def pin_layer_row_independence():
    inp, spec = rand_layer(54, T=15)
    a = O.forward(inp, spec)
    rows = np.array([3, 0, 14, 7])
    b = O.forward(dict(inp, x=inp["x"][rows]), spec)
    close(b["y"], a["y"][rows])


def pin_layer_expert_relabel():
    inp, spec = rand_layer(55, E=7, k=3)
    inp["b_router"] = np.linspace(0, 0.3, 7).astype(np.float32)
    a = O.forward(inp, spec)
    perm = np.random.default_rng(1).permutation(7)  # new expert p holds old expert perm[p]
    inp2 = dict(inp)
    for key in ("w_router", "b_router", "w_gate", "w_value", "w_out"):
        inp2[key] = inp[key][perm]
    b = O.forward(inp2, spec)
    close(b["y"], a["y"])
    assert np.array_equal(perm[b["idx"]], a["idx"])


def pin_layer_norm_after_combine():
    """With eps = 0, scaling every expert's output (W_o) leaves y unchanged:
    the norm sits after the weighted combine."""
    inp, spec = rand_layer(56)
    spec = dict(spec, eps=0.0)
    a = O.forward(inp, spec)
    b = O.forward(dict(inp, w_out=inp["w_out"] * 3.5), spec)
    close(b["y"], a["y"], rtol=1e-10)


def pin_layer_linearity():
    inp, spec = rand_layer(57, S=1)
    a = O.forward(inp, spec)
    b = O.forward(dict(inp, w_up=inp["w_up"] * 2.0), spec)
    close(b["y"] - b["shared"], 2.0 * (a["y"] - a["shared"]))
    c = O.forward(dict(inp, gamma=(inp["gamma"] * 2).astype(np.float32)), spec)
    close(c["y"] - c["shared"], 2.0 * (a["y"] - a["shared"]))


def pin_layer_two_shared_is_one_concat():
    inp, spec = rand_layer(58, S=2, Is=3)
    a = O.forward(inp, spec)
    cat = dict(inp,
               ws_gate=np.concatenate([inp["ws_gate"][0], inp["ws_gate"][1]], 0)[None],
               ws_value=np.concatenate([inp["ws_value"][0], inp["ws_value"][1]], 0)[None],
               ws_out=np.concatenate([inp["ws_out"][0], inp["ws_out"][1]], 1)[None])
    close(O.forward(cat, spec)["y"], a["y"])


def pin_layer_identity_projection():
    inp, spec = rand_layer(59, identity=True)
    a = O.forward(inp, spec)
    eye = np.eye(inp["x"].shape[1])
    close(O.forward(dict(inp, w_down=eye, w_up=eye), spec)["y"], a["y"])


def pin_layer_bruteforce_per_token():
    """The whole layer token by token in pure Python (no permutation, no
    vectorised gathers), against the vectorised oracle."""
    inp, spec = rand_layer(60, T=5, H=8, L=6, E=5, k=2, S=1, I=4, Is=3)
    inp["b_router"] = np.array([0.0, 0.2, -0.1, 0.05, 0.0], np.float32)
    c, eps, k = spec["cap"], spec["eps"], spec["k"]
    inp["x"] = inp["x"] * 60  # some pre-activations beyond the cap's knee
    X = inp["x"].tolist()
    Wr, b = inp["w_router"].tolist(), [float(v) for v in inp["b_router"]]
    Wd, Wu = inp["w_down"].tolist(), inp["w_up"].tolist()
    G, V, Wo = inp["w_gate"].tolist(), inp["w_value"].tolist(), inp["w_out"].tolist()
    gam = [float(v) for v in inp["gamma"]]
    SG, SV, SO = inp["ws_gate"].tolist(), inp["ws_value"].tolist(), inp["ws_out"].tolist()
    H, L, E, I = 8, 6, 5, 4

    def capf(u):
        return c * math.tanh(u / c)

    def siluf(u):
        return u / (1.0 + math.exp(-u))

    def dot(a, bb):
        return sum(p * q for p, q in zip(a, bb))

    y = []
    for t in range(5):
        s = [1.0 / (1.0 + math.exp(-dot(X[t], Wr[e]))) for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-(s[e] + b[e]), e))[:k]
        tot = sum(s[e] for e in sel)
        z = [dot(X[t], Wd[l]) for l in range(L)]
        acc = [0.0] * L
        for e in sel:
            a = [siluf(capf(dot(z, G[e][i]))) * capf(dot(z, V[e][i])) for i in range(I)]
            for l in range(L):
                acc[l] += (s[e] / tot) * dot(a, Wo[e][l])
        rms = math.sqrt(sum(v * v for v in acc) / L + eps)
        n = [gam[l] * acc[l] / rms for l in range(L)]
        row = [dot(n, Wu[h]) for h in range(H)]
        for si in range(len(SG)):
            a = [siluf(capf(dot(X[t], SG[si][i]))) * capf(dot(X[t], SV[si][i])) for i in range(len(SG[si]))]
            for h in range(H):
                row[h] += dot(a, SO[si][h])
        y.append(row)
    close(O.forward(inp, spec)["y"], np.array(y), rtol=1e-10, atol=1e-12)


def pin_fp8_forward_is_dequantised_forward():
    cfg = get_config("small_fp8")
    from dataclasses import replace
    cfg = replace(cfg, T=17)
    t = make_inputs(cfg)
    inp = {k: raw_numpy(v) for k, v in t.items()}
    spec = dict(act=cfg.act, w_expert="f8", k=cfg.k, cap=cfg.cap, eps=cfg.eps)
    a = O.forward(inp, spec)
    deq = dict(inp)
    for w, s in (("w_gate", "s_gate"), ("w_value", "s_value"), ("w_out", "s_out"),
                 ("ws_gate", "ss_gate"), ("ws_value", "ss_value"), ("ws_out", "ss_out")):
        deq[w] = np.stack([O.E4M3FN[inp[w][i]] * np.kron(inp[s][i].astype(np.float64), np.ones((128, 128)))
                           for i in range(len(inp[w]))])
    deq["x"] = O.bf16_bits_to_f64(inp["x"])
    deq["w_router"] = O.bf16_bits_to_f64(inp["w_router"])
    deq["w_down"] = O.bf16_bits_to_f64(inp["w_down"])
    deq["w_up"] = O.bf16_bits_to_f64(inp["w_up"])
    b = O.forward(deq, dict(spec, act="f64", w_expert="f64"))
    close(b["y"], a["y"], rtol=0, atol=0)


def pin_forced_routing():
    inp, spec = rand_layer(61, T=10, E=8, k=3)
    a = O.forward(inp, spec)
    b = O.forward(inp, spec, forced_idx=a["idx"][:, ::-1].copy())  # same sets, other order
    close(b["y"], a["y"])
    bad = a["idx"].copy()
    full = O.route(O.decode(inp["x"], "f64"), inp["w_router"], np.zeros(8), 8)["idx"]
    bad[:, 0] = full[:, -1]  # the lowest-scored expert instead of the best one
    with pytest.raises(ValueError):
        O.forward(inp, spec, forced_idx=bad, forced_tol=1e-9)


def pin_empty_batch():
    inp, spec = rand_layer(62, T=0)
    out = O.forward(inp, spec)
    assert out["y"].shape == (0, inp["w_up"].shape[0])
    assert out["idx"].shape == (0, spec["k"])


def pin_quantile_thresholds_library_and_brute_force():
    """tau_e against numpy's own quantile (method 'linear') and against the
    definition written out with a pure-Python sort of one column."""
    rng = np.random.default_rng(71)
    for T, E, k in ((1, 4, 2), (2, 5, 1), (37, 16, 2), (100, 7, 3), (64, 8, 8)):
        s = rng.random((T, E))
        tau = O.quantile_thresholds(s, k)
        assert tau.shape == (E,)
        close(tau, np.quantile(s, 1.0 - k / E, axis=0, method="linear"), rtol=0, atol=1e-15)
        for e in range(E):
            col = sorted(float(v) for v in s[:, e])
            h = (T - 1) * (1.0 - k / E)
            lo = math.floor(h)
            hi = min(lo + 1, T - 1)
            want = col[lo] + (h - lo) * (col[hi] - col[lo])
            assert abs(tau[e] - want) <= 1e-15


def pin_quantile_fair_share():
    """About T k / E tokens score at or above each threshold: the count is
    T - floor(h) (or one less where tau falls strictly between two order
    statistics), with h = (T - 1)(1 - k/E), so it is within one of T k / E."""
    rng = np.random.default_rng(72)
    for T, E, k in ((500, 12, 3), (999, 9, 2), (64, 16, 4)):
        s = rng.random((T, E))
        tau = O.quantile_thresholds(s, k)
        above = (s >= tau[None, :]).sum(axis=0)
        h = (T - 1) * (1.0 - k / E)
        assert np.all((above == T - math.floor(h)) | (above == T - math.floor(h) - 1))
        assert np.all(np.abs(above - T * k / E) <= 1.0 + 1e-9)


def pin_quantile_special_cases():
    rng = np.random.default_rng(73)
    s = rng.random((40, 6))
    close(O.quantile_thresholds(s, 6), s.min(axis=0), rtol=0, atol=0)  # k = E: every token qualifies
    close(O.quantile_thresholds(s[:1], 2), s[0], rtol=0, atol=0)       # one token
    const = np.full((25, 5), 0.375)
    close(O.quantile_thresholds(const, 2), np.full(5, 0.375), rtol=0, atol=0)
    perm = rng.permutation(40)
    close(O.quantile_thresholds(s[perm], 2), O.quantile_thresholds(s, 2), rtol=0, atol=0)
    close(O.quantile_thresholds(s + 0.25, 2), O.quantile_thresholds(s, 2) + 0.25, rtol=0, atol=1e-15)
    # the bias is minus the threshold of the sigmoid scores
    lg = rng.standard_normal((30, 5)) * 2
    close(O.quantile_bias(lg, 2), -np.quantile(scipy.special.expit(lg), 1 - 2 / 5, axis=0), rtol=0, atol=1e-15)


def pin_quantile_bias_balances_a_skewed_router():
    """With per-expert score offsets (a router that favours some experts), the
    plain top-k piles tokens on the favoured experts; the quantile bias,
    applied through the same selection, brings every expert within a factor
    of 2 of T k / E (here the plain maximum is over 5 times that)."""
    rng = np.random.default_rng(74)
    T, E, k = 4000, 16, 2
    logits = rng.standard_normal((T, E)) + np.linspace(-3, 3, E)[None, :]
    s = O.sigmoid(logits)
    plain = np.bincount(O.select_topk(s, k)[0].ravel(), minlength=E)
    qb = np.bincount(O.select_topk(s + O.quantile_bias(logits, k)[None, :], k)[0].ravel(), minlength=E)
    fair = T * k / E
    assert plain.max() > 3 * fair
    assert qb.max() < 2 * fair and qb.min() > 0.5 * fair


def pin_e4m3fn_encode():
    """Rounding to e4m3fn against torch's own conversion, plus what the format
    fixes: every finite value encodes to its own code, midpoints go to the
    even code, magnitudes past 448 saturate, the sign survives rounding to 0."""
    rng = np.random.default_rng(81)
    v = rng.standard_normal(50000) * np.exp(rng.uniform(-14, 7, 50000))
    want = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3fn_encode(v), want)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(O.e4m3fn_encode(O.E4M3FN[codes]), codes)
    pos = O.E4M3FN[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    got = O.e4m3fn_encode(mid).astype(np.int64)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert np.array_equal(O.e4m3fn_encode(np.nextafter(mid, 0)), lo.astype(np.uint8))
    assert np.array_equal(O.e4m3fn_encode(np.nextafter(mid, 1e9)), (lo + 1).astype(np.uint8))
    assert list(O.e4m3fn_encode([500.0, -1e9, -1e-9, np.nan])) == [0x7E, 0xFE, 0x80, 0x7F]


def pin_quantize_1x128_round_trip():
    """Values built as code * 2^m with a 448 in every block come back as the
    same codes and scale 2^m exactly; an all-zero block gets scale 1; scaling
    one block by a power of two scales only that block's scale."""
    rng = np.random.default_rng(82)
    R, nb = 6, 3
    codes = rng.integers(0, 256, (R, nb * 128)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x11  # no NaN codes
    codes[:, ::128] = np.where(rng.random((R, nb)) < 0.5, 0x7E, 0xFE)  # +-448 in each block
    m = rng.integers(-20, 6, (R, nb))
    v = O.E4M3FN[codes] * np.repeat(2.0 ** m, 128, axis=1)
    q, sc = O.quantize_1x128(v)
    assert sc.dtype == np.float32 and sc.shape == (R, nb)
    assert np.array_equal(q, codes) and np.array_equal(sc, (2.0 ** m).astype(np.float32))
    v2 = v.copy()
    v2[2, 128:256] *= 2.0 ** -7
    v2[4, :128] = 0.0
    q2, sc2 = O.quantize_1x128(v2)
    assert sc2[2, 1] == sc[2, 1] * 2.0 ** -7 and np.array_equal(q2[2], q[2])
    assert sc2[4, 0] == 1.0 and not q2[4, :128].any()
    keep = np.ones((R, nb), bool)
    keep[2, 1] = keep[4, 0] = False
    assert np.array_equal(sc2[keep], sc[keep])


def pin_quantize_1x128_error_bound():
    """Each block's largest magnitude maps to +-448, scale = fp32(amax / 448),
    and the decoded error is at most half an e4m3 step (2^-4 relative for
    normal codes, 2^-10 scale below them)."""
    rng = np.random.default_rng(83)
    v = rng.standard_normal((5, 384)) * np.exp(rng.uniform(-6, 6, (5, 384)))
    q, sc = O.quantize_1x128(v)
    v32 = v.astype(np.float32).astype(np.float64)
    blocks = np.abs(v32).reshape(5, 3, 128)
    amax = blocks.max(axis=2)
    assert np.array_equal(sc, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    arg = blocks.argmax(axis=2)
    for r in range(5):
        for b in range(3):
            assert q[r, b * 128 + arg[r, b]] & 0x7F == 0x7E
    deq = O.dequant_rows(q, sc)
    scale = np.repeat(sc.astype(np.float64), 128, axis=1)
    err = np.abs(deq - v32)
    normal = np.abs(v32) / scale >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(v32[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * scale[~normal] * (1 + 1e-6))


def pin_bf16_round():
    """Against torch's float32 -> bf16 conversion (one rounding of an exact
    float32), and at ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and
    goes to 1 (even), 1 + 3 * 2^-8 goes to 1 + 2^-6; a hair past a tie goes up."""
    rng = np.random.default_rng(86)
    v = (rng.standard_normal(40000) * np.exp(rng.uniform(-30, 30, 40000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.bf16_round(v.astype(np.float64)), want)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -40])
    assert list(O.bf16_round(ties)) == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]


def pin_a8_quantises_the_exact_activation():
    """W8A8 quantises the routed experts' inputs as the layer computes them:
    z = x W_dn^T and the SiTU-GLU output, unrounded.  One expert, W_o = I,
    identity up-projection, no shared expert: the layer is RMSNorm of the
    quantised SiTU-GLU output of the quantised z, written here with numpy and
    the pinned quantiser.  A copy rounded to bf16 before quantising takes
    other codes on this layer, so that reading would fail here."""
    inp, spec = _a8_layer(87, T=6, E=1, k=1, S=0)
    inp["w_up"] = None
    inp["w_out"] = np.eye(128)[None]
    gamma = inp["gamma"].astype(np.float64)
    z = inp["x"] @ inp["w_down"].T
    zq = O.dequant_rows(*O.quantize_1x128(z))
    g = zq @ inp["w_gate"][0].T
    vv = zq @ inp["w_value"][0].T
    capg, capv = 100 * np.tanh(g / 100), 100 * np.tanh(vv / 100)
    a = capg / (1 + np.exp(-capg)) * capv
    aq = O.dequant_rows(*O.quantize_1x128(a))
    want = gamma * aq / np.sqrt(np.mean(aq * aq, axis=1, keepdims=True) + spec["eps"])
    close(O.forward(inp, spec)["y"], want, rtol=1e-10, atol=1e-12)
    assert not np.array_equal(zq, O.dequant_rows(*O.quantize_1x128(O.bf16_round(z))))
    assert not np.array_equal(aq, O.dequant_rows(*O.quantize_1x128(O.bf16_round(a))))


def _a8_layer(seed, T=7, **kw):
    base = dict(H=128, L=128, E=4, k=2, S=1, I=128, Is=128)
    base.update(kw)
    inp, spec = rand_layer(seed, T=T, wstd=0.1, **base)
    return inp, dict(spec, a8=True)


def pin_a8_single_expert_written_out():
    """E = k = 1, identity projections, no shared expert, W_o = identity: the
    layer is RMSNorm of the quantised SiTU-GLU output of the quantised input,
    written here with numpy and the pinned quantiser only."""
    inp, spec = _a8_layer(84, T=5, E=1, k=1, S=0)
    inp["w_down"] = inp["w_up"] = None
    inp["w_out"] = np.eye(128)[None]
    gamma = inp["gamma"].astype(np.float64)
    xq = O.dequant_rows(*O.quantize_1x128(inp["x"]))
    g = xq @ inp["w_gate"][0].T
    vv = xq @ inp["w_value"][0].T
    capg, capv = 100 * np.tanh(g / 100), 100 * np.tanh(vv / 100)
    a = capg / (1 + np.exp(-capg)) * capv
    aq = O.dequant_rows(*O.quantize_1x128(a))
    want = gamma * aq / np.sqrt(np.mean(aq * aq, axis=1, keepdims=True) + spec["eps"])
    close(O.forward(inp, spec)["y"], want, rtol=1e-10, atol=1e-12)


def pin_a8_row_independence_and_bounded_change():
    """W8A8 quantises each token on its own, so rows stay independent; the
    output moves from the unquantised layer's by a few percent, not zero."""
    inp, spec = _a8_layer(85, T=9)
    full = O.forward(inp, spec)
    sub = dict(inp, x=inp["x"][[6, 1, 3]])
    close(O.forward(sub, spec)["y"], full["y"][[6, 1, 3]], rtol=1e-10, atol=1e-12)
    ref = O.forward(inp, dict(spec, a8=False))
    assert np.array_equal(full["idx"], ref["idx"])
    rel = np.abs(full["y"] - ref["y"]).max(axis=1) / np.abs(ref["y"]).max(axis=1)
    assert rel.max() < 0.1 and rel.min() > 1e-4


_GRADS = ("dx", "dw_router", "dw_down", "dw_gate", "dw_value", "dw_out", "dgamma", "dw_up", "dws_gate",
          "dws_value", "dws_out")
_PARAM = {"dx": "x", "dw_router": "w_router", "dw_down": "w_down", "dw_gate": "w_gate", "dw_value": "w_value",
          "dw_out": "w_out", "dgamma": "gamma", "dw_up": "w_up", "dws_gate": "ws_gate", "dws_value": "ws_value",
          "dws_out": "ws_out"}


def _torch_layer_grads(inp, spec, idx, dy):
    """The layer written again with torch ops on float64 leaves, one token
    and slot at a time, differentiated by torch.autograd."""
    c = float(spec["cap"])
    capf = (lambda u: c * torch.tanh(u / c)) if math.isfinite(c) else (lambda u: u)
    leaves = {}
    for name in ("x", "w_router", "w_down", "w_gate", "w_value", "w_out", "gamma", "w_up", "ws_gate", "ws_value",
                 "ws_out"):
        if inp.get(name) is not None:
            leaves[name] = t64(inp[name]).clone().requires_grad_(True)
    x = leaves["x"]
    T = x.shape[0]
    k = idx.shape[1]
    s = torch.sigmoid(x @ leaves["w_router"].T)
    ti = torch.from_numpy(np.asarray(idx, dtype=np.int64))
    sel = s.gather(1, ti)
    w = sel / sel.sum(1, keepdim=True)
    z = x @ leaves["w_down"].T if "w_down" in leaves else x
    rows = []
    for t in range(T):
        acc = 0
        for j in range(k):
            e = int(idx[t, j])
            a = F.silu(capf(leaves["w_gate"][e] @ z[t])) * capf(leaves["w_value"][e] @ z[t])
            acc = acc + w[t, j] * (leaves["w_out"][e] @ a)
        rows.append(acc)
    comb = torch.stack(rows)
    n = leaves["gamma"] * comb / torch.sqrt((comb * comb).mean(1, keepdim=True) + spec["eps"])
    y = n @ leaves["w_up"].T if "w_up" in leaves else n
    if "ws_gate" in leaves:
        for si in range(leaves["ws_gate"].shape[0]):
            h = F.silu(capf(x @ leaves["ws_gate"][si].T)) * capf(x @ leaves["ws_value"][si].T)
            y = y + h @ leaves["ws_out"][si].T
    (y * t64(dy)).sum().backward()
    return {g: leaves[p].grad.numpy() for g, p in _PARAM.items() if p in leaves}


def _bwd_cases():
    yield rand_layer(91, T=7, E=5, k=2, S=2, I=6, Is=5, L=8, H=10)
    yield rand_layer(92, T=6, E=4, k=3, S=0, identity=True, H=9, I=4)
    yield rand_layer(93, T=5, E=6, k=2, S=1, I=5, Is=3, cap=float("inf"))
    inp, spec = rand_layer(94, T=5, E=3, k=1, S=1, I=4, Is=4, cap=1.5)  # a small cap, well inside the tanh
    yield inp, spec


def pin_backward_vs_torch_autograd():
    """Every gradient against torch.autograd of an independent torch forward
    (same selection), on layers with and without projections, shared experts
    and the cap."""
    for inp, spec in _bwd_cases():
        f = O.forward(inp, spec)
        dy = np.random.default_rng(95).standard_normal(f["y"].shape)
        b = O.backward(inp, spec, dy)
        ref = _torch_layer_grads(inp, spec, f["idx"], dy)
        for gname, want in ref.items():
            close(b[gname], want, rtol=1e-9, atol=1e-11)
        assert set(ref) == {gname for gname in _GRADS if gname in b}


def pin_backward_finite_differences():
    """Central differences of <y, dy> along a random direction of each input
    and weight, with the selection held fixed (the oracle's own forward)."""
    for inp, spec in _bwd_cases():
        f = O.forward(inp, spec)
        rng = np.random.default_rng(96)
        dy = rng.standard_normal(f["y"].shape)
        b = O.backward(inp, spec, dy)
        h = 1e-6
        for gname, pname in _PARAM.items():
            if inp.get(pname) is None:
                continue
            base = np.asarray(inp[pname], dtype=np.float64)
            d = rng.standard_normal(base.shape)
            fx = []
            for sign in (1, -1):
                pert = dict(inp)
                pert[pname] = base + sign * h * d  # float64 (gamma too: taken as it is)
                fx.append(np.sum(O.forward(pert, spec, forced_idx=f["idx"])["y"] * dy))
            fd = (fx[0] - fx[1]) / (2 * h)
            an = float(np.sum(b[gname] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gname, fd, an)


PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[4:] for p in PINS])
def test_pin(pin):
    pin()


def test_golden_page_figures():
    """Config shapes agree with the figures the pages state."""
    with open(os.path.join(GOLDEN, "k3_layer_figures.json")) as f:
        g = json.load(f)
    for name in ("k3_prefill_t2048", "k3_t8192", "k3_decode_t64", "k3_zipf_t16384", "k3_fp8_t8192"):
        c = get_config(name)
        assert (c.H, c.L, c.E, c.k, c.S) == (g["hidden"]["value"], g["latent"]["value"],
                                             g["routed_experts"]["value"], g["active_experts"]["value"],
                                             g["shared_experts"]["value"])
        assert c.cap == g["situ_cap"]["value"]
    assert g["latent"]["value"] * 2 == g["hidden"]["value"]
    assert round(100 * 16 / 896, 1) == g["routed_active_percent"]["value"]
    alt = get_config("fp8_448x8_l7168_t8192")
    assert [alt.E, alt.k] == g["alternative_pool"]["value"]


# ----------------------------------------------------------------------------
# planted mistakes: every mutant must break at least one pin
# ----------------------------------------------------------------------------

_ORIG = {n: getattr(O, n) for n in ("combine", "route", "permute")}


def _mut_value_uncapped(g, v, c):
    return O.silu(O.cap(g, c)) * v


def _mut_gate_value_swapped(g, v, c):
    return O.silu(O.cap(v, c)) * O.cap(g, c)


def _mut_silu_sign(u):
    return u * O.sigmoid(-u)


def _mut_norm_no_gamma(c, gamma, eps):
    return c / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)


def _mut_norm_sum_not_mean(c, gamma, eps):
    return gamma[None, :] * c / np.sqrt(np.sum(c * c, axis=1, keepdims=True) + eps)


def _mut_combine_drops_last(Ov, pos, w):
    T, k = w.shape
    out = np.zeros((T, Ov.shape[1]))
    for j in range(k - 1):
        out += w[:, j:j + 1] * Ov[pos.reshape(T, k)[:, j]]
    return out


def _mut_combine_unweighted(Ov, pos, w):
    return _ORIG["combine"](Ov, pos, np.ones_like(w))


def _mut_topk_ties_high(biased, k):
    T, E = biased.shape
    order = np.lexsort((np.broadcast_to(-np.arange(E), (T, E)), -biased), axis=-1)
    idx = order[:, :k]
    rows = np.arange(T)
    gap = biased[rows, order[:, k - 1]] - biased[rows, order[:, k]] if k < E else np.full(T, np.inf)
    return idx, gap


def _mut_route_weights_from_logits(x, w_router, b_router, k):
    r = _ORIG["route"](x, w_router, b_router, k)
    sel = np.take_along_axis(r["logits"], r["idx"], 1)
    r["w"] = sel / sel.sum(1, keepdims=True)
    return r


def _mut_permute_unstable(idx, E):
    offsets, srt, pos = _ORIG["permute"](idx, E)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        srt[lo:hi] = srt[lo:hi][::-1]
    pos[srt] = np.arange(srt.size)
    return offsets, srt, pos


def _mut_down_uses_router_input_scaled(x, w_down):
    return x * 0.5 if w_down is None else (x @ w_down.T) * 0.5


def _mut_no_shared(x, ws_gate, ws_value, ws_out, ss, tag, S, c):
    return np.zeros((x.shape[0], x.shape[1]))


def _mut_bf16_truncates_low_byte(bits):
    b = np.asarray(bits, dtype=np.uint16) & np.uint16(0xFF00)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _mut_sigmoid_tanh(u):
    return np.tanh(u)


def _mut_quantile_of_k_over_e(scores, k):
    T, E = scores.shape
    return np.quantile(scores, k / E, axis=0)


def _mut_quantile_nearest_lower(scores, k):
    T, E = scores.shape
    h = (T - 1) * (1.0 - k / E)
    return np.sort(scores, axis=0)[int(np.floor(h))]


def _mut_quantile_bias_plus(logits, k):
    return O.quantile_thresholds(O.sigmoid(logits), k)


def _mut_encode_truncates(v):
    v = np.asarray(v, dtype=np.float64)
    pos = O.E4M3FN[:0x7F]
    a = np.minimum(np.abs(v), pos[-1])
    code = (np.searchsorted(pos, a, side="right") - 1).astype(np.uint8)
    return np.where(np.isnan(v), 0x7F, code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _mut_quantize_per_row(v):
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    R, C = v32.shape
    amax = np.abs(v32).max(axis=1, keepdims=True)
    scale = np.where(amax > 0, amax / np.float32(448), np.float32(1)).astype(np.float32)
    return O.e4m3fn_encode(v32 / scale), np.repeat(scale, C // 128, axis=1)


def _mut_quantize_e4m3_max_240(v):
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    R, C = v32.shape
    b = v32.reshape(R, C // 128, 128)
    amax = np.abs(b).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(240), np.float32(1)).astype(np.float32)
    return O.e4m3fn_encode(b / scale[:, :, None]).reshape(R, C), scale


def _mut_fp8_activations_skipped(v):
    return np.asarray(v, dtype=np.float64)


def _mut_fp8_activations_rounded_bf16(v):
    return O.dequant_rows(*O.quantize_1x128(O.bf16_round(v)))


def _mut_expert_ffn_a_not_quantised(zrows, wg, wv, wo, c, a8=False):
    a = O.situ_glu(zrows @ wg.T, zrows @ wv.T, c)
    return a, a @ wo.T


def _mut_bf16_round_truncates(v):
    m, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)


def _mut_situ_grad_no_cap_slope(g, v, c, da):
    cg, cv = O.cap(g, c), O.cap(v, c)
    sg = O.sigmoid(cg)
    return da * cv * sg * (1.0 + cg * (1.0 - sg)), da * cg * sg


def _mut_rmsnorm_grad_no_mean_term(c, gamma, eps, dn):
    r = 1.0 / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)
    return r * gamma[None, :] * dn, np.sum(dn * c * r, axis=0)


def _mut_combine_grad_unweighted(O_, pos, w, dc):
    T, k = w.shape
    p = pos.reshape(T, k)
    dO = np.zeros_like(O_)
    dw = np.zeros((T, k))
    for j in range(k):
        dO[p[:, j]] = dc
        dw[:, j] = np.sum(dc * O_[p[:, j]], axis=1)
    return dO, dw


def _mut_route_grad_unrenormalised(scores, idx, dw):
    sel = np.take_along_axis(scores, idx, axis=1)
    S = sel.sum(axis=1, keepdims=True)
    out = np.zeros_like(scores)
    np.put_along_axis(out, idx, dw / S * sel * (1 - sel), axis=1)
    return out


MUTANTS = {
    "situ_glu_grad": [_mut_situ_grad_no_cap_slope],
    "rmsnorm_grad": [_mut_rmsnorm_grad_no_mean_term],
    "combine_grad": [_mut_combine_grad_unweighted],
    "route_grad": [_mut_route_grad_unrenormalised],
    "e4m3fn_encode": [_mut_encode_truncates],
    "quantize_1x128": [_mut_quantize_per_row, _mut_quantize_e4m3_max_240],
    "fp8_activations": [_mut_fp8_activations_skipped, _mut_fp8_activations_rounded_bf16],
    "bf16_round": [_mut_bf16_round_truncates],
    "expert_ffn": [_mut_expert_ffn_a_not_quantised],
    "situ_glu": [_mut_value_uncapped, _mut_gate_value_swapped],
    "silu": [_mut_silu_sign],
    "rmsnorm": [_mut_norm_no_gamma, _mut_norm_sum_not_mean],
    "combine": [_mut_combine_drops_last, _mut_combine_unweighted],
    "select_topk": [_mut_topk_ties_high],
    "route": [_mut_route_weights_from_logits],
    "permute": [_mut_permute_unstable],
    "latent_down": [_mut_down_uses_router_input_scaled],
    "shared_experts": [_mut_no_shared],
    "bf16_bits_to_f64": [_mut_bf16_truncates_low_byte],
    "sigmoid": [_mut_sigmoid_tanh],
    "quantile_thresholds": [_mut_quantile_of_k_over_e, _mut_quantile_nearest_lower],
    "quantile_bias": [_mut_quantile_bias_plus],
}


@pytest.mark.parametrize("target,mutant",
                         [(t, m) for t, ms in MUTANTS.items() for m in ms],
                         ids=[m.__name__[5:] for ms in MUTANTS.values() for m in ms])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(O, target, mutant)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant.__name__} of {target} passed every pin"

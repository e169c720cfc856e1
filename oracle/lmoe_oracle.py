"""CPU fp64 oracle of one Stable Latent MoE layer: the forward pass (bf16,
fp32, e4m3 expert weights, W8A8 routed experts), the Quantile Balancing
thresholds and the backward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module: only tests/, the smoke check in __graft_entry__ and the
benchmark's cpu_baseline leg use it.  It shares no code with the HIP
library; it reads the same storage bytes (fp32, bf16 bit patterns, e4m3fn
codes with fp32 block scales), decodes them exactly and computes every step
in float64 with numpy, one plain step after another.

Sources (the pages describe the layer only in prose; no formula is printed):
  P1  aitrending.vip, "The 2.8-Trillion-Parameter Problem: Why Bigger Models
      Break the Old Playbook" -- TL;DR and Technical Details bullets.
  P2  wpnews.pro, same title, Part 1 of "Inside Kimi K3" -- the MoE passage
      ("From a dense feed-forward layer to 896 experts"), the Stable
      LatentMoE passage and the stabilizer passage that follows it.
  P3  daily-ai-frontier, "苏神复盘 Kimi K3：896 个专家背后，藏着哪些关键技术取舍？"
      -- Merged summary, LatentMoE and Stable LatentMoE bullets.

Readings taken where the pages are silent (each is a documented choice):
  * router scores are sigmoid(x . W_r^T); a per-expert bias is added for
    selection only; the k selected scores, renormalised to sum to 1, are the
    combine weights; ties in the biased score go to the lower expert index;
  * SiTU-GLU(g, v) = silu(cap(g)) * cap(v) with cap(u) = c * tanh(u / c),
    c = 100 by default;
  * RMSNorm n = gamma * c / sqrt(mean(c^2) + eps) with eps = 1e-6;
  * shared experts run at full width on x, use the same SiTU-GLU, have
    weight 1 and are added after the up-projection;
  * no capacity limit (no token is dropped), no biases in the linears, and
    the residual add is outside the layer;
  * W8A8: the routed experts' activations (z, and each expert's SiTU-GLU
    output), as the layer computes them, are quantised per row per 128
    columns to e4m3fn (scale amax / 448, the decisions taken in fp32);
  * Quantile Balancing: expert e's threshold is the (1 - k/E) quantile of its
    batch scores (linear interpolation), and its bias is minus that;
  * backward: the gradient of sum(y * dy); the selection and its bias carry
    none, the router's flows through the renormalised combine weights.

Parity pins: every function here is pinned by tests/test_oracle.py against
library routines (torch/scipy, torch.autograd for the gradients), closed
forms, invariants, finite differences or brute force; the chosen readings
above are conventions and are pinned only through those properties.
"""

import numpy as np

F8_BLOCK = 128


# ----------------------------------------------------------------------------
# Storage decoding (exact)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> float64.  A bf16 value is the upper half
    of the fp32 with the same bits, so widening is exact."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3fn_table():
    """Value of every OCP e4m3fn code: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
    there are no infinities, so the largest finite magnitude is 448."""
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3FN = _e4m3fn_table()


def e4m3fn_to_f64(codes):
    return E4M3FN[np.asarray(codes, dtype=np.uint8)]


def decode(raw, tag):
    """Raw storage -> float64.  tag: "f32" (float32 array), "bf16" (uint16
    bits), "f8" (uint8 e4m3fn codes, unscaled), "f64" (already float)."""
    if raw is None:
        return None
    if tag == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if tag == "bf16":
        return bf16_bits_to_f64(raw)
    if tag == "f8":
        return e4m3fn_to_f64(raw)
    if tag == "f64":
        return np.asarray(raw, dtype=np.float64)
    raise ValueError(f"unknown storage tag {tag!r}")


def dequant_blocks(codes, scales):
    """fp8 matrix [R, C] with one fp32 scale per 128x128 block: value = q*s."""
    q = e4m3fn_to_f64(codes)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return q * np.repeat(np.repeat(s, F8_BLOCK, axis=0), F8_BLOCK, axis=1)


def e4m3fn_encode(v):
    """float -> OCP e4m3fn code: the nearest finite value, a tie going to the
    code with an even mantissa (round to nearest even), magnitudes beyond 448
    saturated to 448.  The sign bit is the sign of v, so a negative value
    that rounds to zero gives the negative zero 0x80.  NaN -> 0x7F."""
    v = np.asarray(v, dtype=np.float64)
    pos = E4M3FN[:0x7F]  # codes 0 .. 126: every positive finite value, ascending
    a = np.minimum(np.abs(v), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 1, 0x7E)
    lo = hi - 1
    dlo, dhi = a - pos[lo], pos[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == pos[hi], hi, code)
    code = code.astype(np.uint8) | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quantize_1x128(v):
    """Activation quantisation of the W8A8 expert GEMMs (per-token 1x128
    blocks; the pages name the BF16/FP8 dynamic-range problem, P3 merged
    summary, and fix no format).  Each row is cut into blocks of 128
    consecutive columns; a block's scale is amax / 448 (1 for an all-zero
    block) and its codes are e4m3fn(v / scale).  The value enters as fp32 and
    the scale and quotient are fp32 operations, the precision the kernel
    decides the codes in.  Returns codes [R, C] uint8, scales [R, C/128]
    float32; value = code * scale."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    R, C = v32.shape
    if C % F8_BLOCK:
        raise ValueError("the quantised width must be a multiple of 128")
    blocks = v32.reshape(R, C // F8_BLOCK, F8_BLOCK)
    amax = np.abs(blocks).max(axis=2, initial=np.float32(0))
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (blocks / scale[:, :, None]).astype(np.float32)
    return e4m3fn_encode(q).reshape(R, C), scale


def dequant_rows(codes, scales):
    """e4m3fn codes [R, C] with one fp32 scale per row per 128 columns -> float64."""
    q = e4m3fn_to_f64(codes)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return q * np.repeat(s, F8_BLOCK, axis=1)


def bf16_round(v):
    """float64 -> the nearest bf16 value (8 significant bits), ties to the even
    one, computed directly (no intermediate fp32 rounding); for the normal
    range, which is all the activations here reach."""
    m, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def fp8_activations(v):
    """The values a W8A8 expert GEMM multiplies: the activation as the layer
    computes it, quantised 1x128 (code decisions in fp32, quantize_1x128),
    decoded.  No intermediate storage rounding is modelled: the pages name
    only the BF16/FP8 dynamic-range problem (P3 merged summary), so the
    quantiser reads the exact activation."""
    return dequant_rows(*quantize_1x128(v))


def matrix(stack, scales, idx, tag):
    """Decoded fp64 matrix idx of a stacked weight tensor (experts or shared
    experts).  `stack` may be any indexable whose items are raw arrays."""
    raw = stack[idx]
    if tag == "f8":
        return dequant_blocks(raw, scales[idx])
    return decode(raw, tag)


# ----------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------

def sigmoid(u):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-u))


def silu(u):
    """SiLU / swish: u * sigmoid(u)."""
    return u * sigmoid(u)


def cap(u, c):
    """Smooth cap to about +-c (P2 stabilizer passage: gate and value are
    bounded to roughly +-100 yet behave like SwiGLU near zero; P3 Stable
    LatentMoE bullet: soft cap of SwiGLU outliers).  c = inf means no cap."""
    if not np.isfinite(c):
        return u
    return c * np.tanh(u / c)


def situ_glu(g, v, c):
    """SiTU-GLU: SwiGLU applied to capped gate and value branches."""
    return silu(cap(g, c)) * cap(v, c)


# ----------------------------------------------------------------------------
# Layer steps
# ----------------------------------------------------------------------------

def select_topk(biased, k):
    """Per token, the k experts with the largest biased score, in descending
    score order, equal scores ordered by ascending expert index (a library
    sort on the key (-score, index)).  Also returns gap = k-th minus
    (k+1)-th biased score (inf when k == E)."""
    T, E = biased.shape
    if T == 0:
        return np.zeros((0, k), np.int64), np.zeros((0,), np.float64)
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -biased), axis=-1)
    idx = order[:, :k]
    rows = np.arange(T)
    if k < E:
        gap = biased[rows, order[:, k - 1]] - biased[rows, order[:, k]]
    else:
        gap = np.full(T, np.inf)
    return idx, gap


def route(x, w_router, b_router, k):
    """Router (P1 Technical Details: a lightweight router picks 16 of 896 per
    token; P2 MoE passage).  Scores s = sigmoid(x W_r^T); selection on s + b;
    combine weights = selected s renormalised to sum 1."""
    logits = x @ w_router.T
    scores = sigmoid(logits)
    biased = scores + b_router[None, :]
    idx, gap = select_topk(biased, k)
    w = combine_weights(scores, idx)
    return dict(logits=logits, scores=scores, biased=biased, idx=idx, gap=gap, w=w)


def quantile_thresholds(scores, k):
    """Quantile Balancing (P3, Stable LatentMoE bullet: per-expert top-k
    thresholds are solved for directly instead of nudging biases by fixed
    steps; P2, the balancing passage: the thresholds come from the batch's
    score distribution, as the score an expert needs to keep its fair share
    of tokens).  Reading taken: expert e's threshold is the (1 - k/E)
    quantile of its scores over the T tokens of the batch, interpolated
    linearly between order statistics: with the column sorted ascending,
    h = (T - 1)(1 - k/E) and tau = s_(floor h) + frac(h) (s_(floor h + 1) -
    s_(floor h)).  About T k / E tokens then score at or above tau_e."""
    T, E = scores.shape
    if T == 0:
        raise ValueError("quantile thresholds need at least one token")
    h = (T - 1) * (1.0 - k / E)
    lo = int(np.floor(h))
    hi = min(lo + 1, T - 1)
    frac = h - lo
    col = np.sort(scores, axis=0)  # each expert's scores, ascending
    return col[lo] + frac * (col[hi] - col[lo])


def quantile_bias(logits, k):
    """Selection bias of Quantile Balancing: b_e = -tau_e, so that the a1
    selection on s + b ranks each expert's scores against its own threshold."""
    return -quantile_thresholds(sigmoid(logits), k)


def combine_weights(scores, idx):
    sel = np.take_along_axis(scores, idx, axis=1)
    if sel.shape[0] == 0:
        return sel
    return sel / sel.sum(axis=1, keepdims=True)


def check_forced(biased, forced_idx, tol):
    """A given selection is accepted if its k experts are distinct, in range,
    and each has a biased score within tol of the k-th largest score."""
    T, E = biased.shape
    f = np.asarray(forced_idx, dtype=np.int64)
    k = f.shape[1]
    if f.shape[0] != T:
        raise ValueError("forced_idx has the wrong number of tokens")
    if T == 0:
        return f
    if f.min() < 0 or f.max() >= E:
        raise ValueError("forced_idx holds an expert index out of range")
    if any(len(set(r.tolist())) != k for r in f):
        raise ValueError("forced_idx repeats an expert within a token")
    kth = -np.sort(-biased, axis=1)[:, k - 1]
    chosen = np.take_along_axis(biased, f, axis=1)
    worst = (kth[:, None] - chosen).max()
    if worst > tol:
        raise ValueError(f"forced_idx is not a top-k selection: an expert lies {worst:.3g} below the k-th score")
    return f


def latent_down(x, w_down):
    """Routed path only: x (hidden) -> z (latent), P2 Stable LatentMoE
    passage; with no projection the latent is x itself."""
    return x if w_down is None else x @ w_down.T


def permute(idx, E):
    """Group the T*k (token, slot) assignments a = t*k + j by expert with a
    stable library sort on the expert id: within an expert, assignments keep
    ascending a, i.e. ascending token.  offsets[e]..offsets[e+1] is expert
    e's range of `sorted`; pos is the inverse permutation."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    sorted_ = np.argsort(flat, kind="stable").astype(np.int64)
    pos = np.empty_like(sorted_)
    pos[sorted_] = np.arange(flat.size)
    return offsets, sorted_, pos


def expert_ffn(zrows, wg, wv, wo, c, a8=False):
    """One routed expert on its latent rows: gated FFN with gate and value
    branches (P2 stabilizer passage) and the SiTU-GLU activation.  With a8
    (W8A8) the SiTU-GLU output is quantised 1x128 before the down GEMM; the
    caller passes rows already quantised for the gate/value GEMM."""
    a = situ_glu(zrows @ wg.T, zrows @ wv.T, c)
    return a, (fp8_activations(a) if a8 else a) @ wo.T


def combine(O, pos, w):
    """Weighted sum of each token's k expert outputs, slot j ascending (P2
    Stable LatentMoE passage: the selected experts' outputs are combined)."""
    T, k = w.shape
    out = np.zeros((T, O.shape[1]))
    for j in range(k):
        out += w[:, j:j + 1] * O[pos.reshape(T, k)[:, j]]
    return out


def rmsnorm(c, gamma, eps):
    """RMSNorm after aggregation, before the up-projection (P2 stabilizer
    passage; P3 Stable LatentMoE bullet)."""
    return gamma[None, :] * c / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)


def shared_experts(x, ws_gate, ws_value, ws_out, ss, tag, S, c):
    """Always-on shared experts (P1 Technical Details; P3 LatentMoE bullet)
    at full width on x, weight 1, summed."""
    y = np.zeros((x.shape[0], x.shape[1]))
    for s in range(S):
        wg = matrix(ws_gate, ss[0], s, tag)
        wv = matrix(ws_value, ss[1], s, tag)
        wo = matrix(ws_out, ss[2], s, tag)
        y += situ_glu(x @ wg.T, x @ wv.T, c) @ wo.T
    return y


def _vector(v):
    """A per-feature vector (gamma, b_router): stored fp32 values widen
    exactly; a float64 array (test inputs only) is taken as it is."""
    a = np.asarray(v)
    return a.astype(np.float64) if a.dtype == np.float64 else a.astype(np.float32).astype(np.float64)


def forward(inp, spec, forced_idx=None, forced_tol=1e-3):
    """Whole layer.  `inp` holds raw storage arrays under the keys x,
    w_router, b_router, w_down, w_gate, w_value, w_out, s_gate, s_value,
    s_out, gamma, w_up, ws_gate, ws_value, ws_out, ss_gate, ss_value, ss_out
    (expert stacks may be any indexable over experts).  `spec` gives act,
    w_expert, k, cap, eps and optionally a8 (W8A8 routed experts: their
    activations quantised 1x128 to e4m3fn, see fp8_activations).  Returns
    every intermediate as float64/int64 (A before any quantisation).

    Steps: route on x; z = latent down-projection of x; tokens grouped by
    expert; each expert's SiTU-GLU FFN on its latent rows; weighted combine;
    RMSNorm; up-projection to full width; plus the shared experts (P2 Stable
    LatentMoE passage and stabilizer passage; P3 LatentMoE bullets)."""
    act, wt = spec["act"], spec["w_expert"]
    k, c, eps = int(spec["k"]), float(spec["cap"]), float(spec["eps"])
    a8 = bool(spec.get("a8", False))
    x = decode(inp["x"], act)
    w_router = decode(inp["w_router"], act)
    b = np.asarray(inp["b_router"], dtype=np.float32).astype(np.float64)
    w_down = decode(inp.get("w_down"), act)
    w_up = decode(inp.get("w_up"), act)
    gamma = _vector(inp["gamma"])
    T, H = x.shape
    E = w_router.shape[0]

    r = route(x, w_router, b, k)
    if forced_idx is not None:
        r["idx"] = check_forced(r["biased"], forced_idx, forced_tol)
        r["w"] = combine_weights(r["scores"], r["idx"])
    idx, w = r["idx"], r["w"]

    z = latent_down(x, w_down)
    L = z.shape[1]
    # W8A8: each token's latent row is quantised once, whatever expert reads it
    zx = fp8_activations(z) if a8 else z
    offsets, sorted_, pos = permute(idx, E)
    I = None
    A = None
    O = np.zeros((T * k, L))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = sorted_[lo:hi] // k
        wg = matrix(inp["w_gate"], inp.get("s_gate"), e, wt)
        wv = matrix(inp["w_value"], inp.get("s_value"), e, wt)
        wo = matrix(inp["w_out"], inp.get("s_out"), e, wt)
        a, o = expert_ffn(zx[toks], wg, wv, wo, c, a8)
        if A is None:
            I = a.shape[1]
            A = np.zeros((T * k, I))
        A[lo:hi] = a
        O[lo:hi] = o
    if A is None:
        A = np.zeros((T * k, 0))

    comb = combine(O, pos, w)
    n = rmsnorm(comb, gamma, eps)
    up = n if w_up is None else n @ w_up.T
    S = 0 if inp.get("ws_gate") is None else len(inp["ws_gate"])
    sh = shared_experts(x, inp.get("ws_gate"), inp.get("ws_value"), inp.get("ws_out"),
                        (inp.get("ss_gate"), inp.get("ss_value"), inp.get("ss_out")), wt, S, c)
    y = up + sh
    out = dict(r)
    out.update(z=z, offsets=offsets, sorted=sorted_, pos=pos, A=A, O=O, c=comb, n=n,
               shared=sh, y=y)
    return out


# ----------------------------------------------------------------------------
# Backward pass (gradients of <y, dy> with respect to x and every weight)
# ----------------------------------------------------------------------------
# The pages motivate the layer's stabilisers by training (P2 stabilizer
# passage); the gradients below are the chain rule of the forward above,
# written step by step in reverse.  The top-k selection is piecewise constant,
# so no gradient flows through the choice of experts or the selection bias;
# the combine weights carry the router's gradient.

def situ_glu_grad(g, v, c, da):
    """d/dg and d/dv of a = silu(cap g) * cap v, times da.  cap'(u) =
    1 - tanh(u / c)^2 (1 for c = inf); silu'(u) = sigma(u) (1 + u (1 -
    sigma(u)))."""
    if np.isfinite(c):
        tg, tv = np.tanh(g / c), np.tanh(v / c)
        cg, cv = c * tg, c * tv
        dcg, dcv = 1.0 - tg * tg, 1.0 - tv * tv
    else:
        cg, cv, dcg, dcv = g, v, 1.0, 1.0
    sg = sigmoid(cg)
    dsilu = sg * (1.0 + cg * (1.0 - sg))
    return da * cv * dsilu * dcg, da * cg * sg * dcv


def rmsnorm_grad(c, gamma, eps, dn):
    """n = gamma * c * r with r = (mean(c^2) + eps)^-1/2 per row.  Returns
    dc = r u - r^3 c (u . c) / L with u = gamma * dn, and dgamma = sum over
    rows of dn * c * r."""
    L = c.shape[1]
    r = 1.0 / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + eps)
    u = gamma[None, :] * dn
    dc = r * u - r ** 3 * c * np.sum(u * c, axis=1, keepdims=True) / L
    return dc, np.sum(dn * c * r, axis=0)


def combine_grad(O, pos, w, dc):
    """c_t = sum_j w_tj O[pos(t, j)]: dO[pos(t, j)] = w_tj dc_t and dw_tj =
    dc_t . O[pos(t, j)]."""
    T, k = w.shape
    p = pos.reshape(T, k)
    dO = np.zeros_like(O)
    dw = np.zeros((T, k))
    for j in range(k):
        dO[p[:, j]] = w[:, j:j + 1] * dc
        dw[:, j] = np.sum(dc * O[p[:, j]], axis=1)
    return dO, dw


def route_grad(scores, idx, dw):
    """w_tj = s_tj / S_t over the selected scores (S_t their sum), s =
    sigmoid(logit): ds_tj = (dw_tj - sum_j' dw_tj' w_tj') / S_t, and
    dlogit = ds * s (1 - s) at the selected experts, 0 elsewhere."""
    T, E = scores.shape
    sel = np.take_along_axis(scores, idx, axis=1)
    S = sel.sum(axis=1, keepdims=True)
    w = sel / S
    ds = (dw - np.sum(dw * w, axis=1, keepdims=True)) / S
    dlogits = np.zeros((T, E))
    np.put_along_axis(dlogits, idx, ds * sel * (1.0 - sel), axis=1)
    return dlogits


def backward(inp, spec, dy, forced_idx=None, forced_tol=1e-3):
    """Gradients of sum(y * dy) for one layer (the forward's inputs and spec;
    dy [T, H] float64).  Returns the forward's intermediates plus dx and
    d<weight> for every weight present (dw_router, dw_down, dw_gate,
    dw_value, dw_out, dgamma, dw_up, dws_gate, dws_value, dws_out).  Expert
    weights are decoded exactly as in the forward; W8A8 is not covered."""
    act, wt = spec["act"], spec["w_expert"]
    k, c, eps = int(spec["k"]), float(spec["cap"]), float(spec["eps"])
    if spec.get("a8"):
        raise ValueError("the backward covers the unquantised layer")
    f = forward(inp, spec, forced_idx=forced_idx, forced_tol=forced_tol)
    x = decode(inp["x"], act)
    w_router = decode(inp["w_router"], act)
    w_down = decode(inp.get("w_down"), act)
    w_up = decode(inp.get("w_up"), act)
    gamma = _vector(inp["gamma"])
    dy = np.asarray(dy, dtype=np.float64)
    T, H = x.shape
    E = w_router.shape[0]
    idx, wts, z = f["idx"], f["w"], f["z"]
    L = z.shape[1]
    g = {}

    # up-projection: y = n W_up^T + shared
    dn = dy if w_up is None else dy @ w_up
    if w_up is not None:
        g["dw_up"] = dy.T @ f["n"]
    # shared experts
    dx = np.zeros((T, H))
    S = 0 if inp.get("ws_gate") is None else len(inp["ws_gate"])
    ss = (inp.get("ss_gate"), inp.get("ss_value"), inp.get("ss_out"))
    if S:
        dsg, dsv, dso = [], [], []
        for s in range(S):
            wg = matrix(inp["ws_gate"], ss[0], s, wt)
            wv = matrix(inp["ws_value"], ss[1], s, wt)
            wo = matrix(inp["ws_out"], ss[2], s, wt)
            gs, vs = x @ wg.T, x @ wv.T
            hs = situ_glu(gs, vs, c)
            dso.append(dy.T @ hs)
            dgs, dvs = situ_glu_grad(gs, vs, c, dy @ wo)
            dsg.append(dgs.T @ x)
            dsv.append(dvs.T @ x)
            dx += dgs @ wg + dvs @ wv
        g["dws_gate"], g["dws_value"], g["dws_out"] = np.stack(dsg), np.stack(dsv), np.stack(dso)
    # RMSNorm and combine
    dcomb, g["dgamma"] = rmsnorm_grad(f["c"], gamma, eps, dn)
    dO, dwts = combine_grad(f["O"], f["pos"], wts, dcomb)
    # routed experts (sorted order)
    offsets, sorted_ = f["offsets"], f["sorted"]
    I = f["A"].shape[1]
    dgate = np.zeros((E, I, L))
    dvalue = np.zeros((E, I, L))
    dout = np.zeros((E, L, I))
    dzrows = np.zeros((T * k, L))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        zr = z[sorted_[lo:hi] // k]
        wg = matrix(inp["w_gate"], inp.get("s_gate"), e, wt)
        wv = matrix(inp["w_value"], inp.get("s_value"), e, wt)
        wo = matrix(inp["w_out"], inp.get("s_out"), e, wt)
        ge, ve = zr @ wg.T, zr @ wv.T
        ae = situ_glu(ge, ve, c)
        dout[e] = dO[lo:hi].T @ ae
        dge, dve = situ_glu_grad(ge, ve, c, dO[lo:hi] @ wo)
        dgate[e] = dge.T @ zr
        dvalue[e] = dve.T @ zr
        dzrows[lo:hi] = dge @ wg + dve @ wv
    g["dw_gate"], g["dw_value"], g["dw_out"] = dgate, dvalue, dout
    # each token's latent gradient: sum over its k assignments
    dz = np.zeros((T, L))
    p = f["pos"].reshape(T, k)
    for j in range(k):
        dz += dzrows[p[:, j]]
    if w_down is None:
        dx += dz
    else:
        g["dw_down"] = dz.T @ x
        dx += dz @ w_down
    # router, through the combine weights
    dlogits = route_grad(f["scores"], idx, dwts)
    g["dw_router"] = dlogits.T @ x
    dx += dlogits @ w_router
    g["dx"] = dx
    out = dict(f)
    out.update(g, dn=dn, dc=dcomb, dO=dO, dwts=dwts, dz=dz, dlogits=dlogits)
    return out

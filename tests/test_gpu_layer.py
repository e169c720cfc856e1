"""GPU parity: every C-ABI entry point and the whole layer against the fp64
oracle on the same input bytes, at small sizes that span several tiles with
ragged tails, plus edge cases (empty batch, k == E, no shared expert,
identity projections, saturated SiTU-GLU caps)."""

import ctypes
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import lmoe_oracle as O
from synth import get_config, make_inputs, raw_numpy

from gpu_common import (GAP, check_selection, host_inputs, make_case, note, rowwise_rel_err, spec_of, to_f64,
                        tol_of)

pytestmark = pytest.mark.gpu

lmoe = pytest.importorskip("sparse_moe_transformer_gemm_amd.lmoe")

SMALL = ["tiny_f32", "tiny_situ_stress", "small_bf16", "small_situ_stress_bf16", "small_fp8", "small_w8a8",
         "small_identity_bf16", "small_full_k"]


def _saturates(inp, cfg, z64=None):
    """The largest |gate| pre-activation of the routed experts (on z64, or on
    the layer's own z) and of the shared experts, in fp64."""
    x = O.decode(inp["x"], cfg.act)
    z = z64 if z64 is not None else (x if inp["w_down"] is None else x @ O.decode(inp["w_down"], cfg.act).T)
    routed = np.abs(z @ O.decode(inp["w_gate"][0], cfg.w_expert).T).max()
    shared = np.abs(x @ O.decode(inp["ws_gate"][0], cfg.act).T).max() if inp.get("ws_gate") is not None else 0.0
    return routed, shared


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    lmoe.load_library()
    return torch.device("cuda:0")


def _weights(cfg, g):
    sh = lmoe.shape_of(cfg)
    return sh, lmoe.make_weights(sh, g)


@pytest.mark.parametrize("name", SMALL)
def test_forward_small(dev, name):
    cfg = get_config(name)
    note(f"[forward] {name} T={cfg.T} H={cfg.H} L={cfg.L} E={cfg.E} k={cfg.k} {cfg.act}/{cfg.w_expert}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    y, idx, tw = lmoe.forward(sh, w, g["x"])
    torch.cuda.synchronize()
    inp = host_inputs(t)
    ref = O.forward(inp, spec_of(cfg))
    check_selection(idx.cpu().numpy(), tw.cpu().numpy(), ref)
    forced = O.forward(inp, spec_of(cfg), forced_idx=idx.cpu().numpy().astype(np.int64), forced_tol=1e-5)
    err = rowwise_rel_err(to_f64(y), forced["y"])
    note(f"    max row rel err {err:.3e} (tol {tol_of(cfg)})")
    assert err <= tol_of(cfg)
    if cfg.x_scale > 1:
        # the stress input really drives the gate pre-activations past the cap
        routed, shared = _saturates(inp, cfg)
        note(f"    max |gate| pre-activation: routed {routed:.0f}, shared {shared:.0f} (cap {cfg.cap})")
        assert routed > 3 * cfg.cap and shared > 3 * cfg.cap


@pytest.mark.parametrize("name,T", [("small_bf16", 20), ("small_bf16", 256), ("small_bf16", 257),
                                    ("small_bf16", 300), ("small_bf16", 700),
                                    ("small_bf16", 2000), ("small_situ_stress_bf16", 20),
                                    ("small_situ_stress_bf16", 2000), ("small_fp8", 700), ("small_fp8", 2000),
                                    ("small_w8a8", 20), ("small_w8a8", 2000)])
def test_forward_tile_variants(dev, name, T):
    """Token counts that select each kernel tile: thin / dense x- and up-GEMMs
    (and the one-group / multi-group permute) on either side of T = 256,
    small / mid / big expert token tiles (experts with 1-3, ~50, ~330 rows);
    with e4m3 expert weights, the register-staged tiles at T=300 and the
    LDS-DMA tiles that widen codes at the fragment load from T=700 on; W8A8
    with nearly empty and with full token tiles."""
    cfg = replace(get_config(name), T=T, name=f"{name}_T{T}")
    note(f"[forward] {cfg.name}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    y, idx, tw = lmoe.forward(sh, w, g["x"])
    torch.cuda.synchronize()
    inp = host_inputs(t)
    ref = O.forward(inp, spec_of(cfg))
    check_selection(idx.cpu().numpy(), tw.cpu().numpy(), ref)
    forced = O.forward(inp, spec_of(cfg), forced_idx=idx.cpu().numpy().astype(np.int64), forced_tol=1e-5)
    err = rowwise_rel_err(to_f64(y), forced["y"])
    note(f"    max row rel err {err:.3e}")
    assert err <= tol_of(cfg)


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "small_fp8", "small_identity_bf16"])
def test_route(dev, name):
    cfg = get_config(name)
    note(f"[route] {name}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    idx, tw, z = lmoe.route(sh, w, g["x"])
    torch.cuda.synchronize()
    inp = host_inputs(t)
    x = O.decode(inp["x"], cfg.act)
    r = O.route(x, O.decode(inp["w_router"], cfg.act), inp["b_router"].astype(np.float64), cfg.k)
    check_selection(idx.cpu().numpy(), tw.cpu().numpy(), r)
    if cfg.identity_proj:
        assert z is None
    else:
        zr = O.latent_down(x, O.decode(inp["w_down"], cfg.act))
        zt = 1e-5 if cfg.act == "f32" else 8e-3
        assert rowwise_rel_err(to_f64(z), zr) <= zt


@pytest.mark.parametrize("T,E,k,ident", [(16484, 896, 16, True), (2049, 896, 16, False), (700, 200, 8, True)])
def test_route_ragged_router_tiles(dev, T, E, k, ident):
    """Router tiles at the edges of the route GEMM's tile walk.  At T = 16484
    with identity projections and no shared expert the GEMM has 4 x 65 router
    tiles; the last token tile's four run in the re-cut tail launch as
    128 x 128 sub-tiles, and the second half of the last router tile
    (features 896 .. 1023) lies wholly past E: its DMAs must stay inside
    W_router while nothing of it is stored.  T = 2049 leaves one token in the
    last token tile; E = 200 is one partial router tile.  Every token's
    selection is checked against the oracle."""
    base = get_config("small_identity_bf16" if ident else "small_bf16")
    cfg = replace(base, name=f"route_t{T}_e{E}", T=T, E=E, k=k, S=0, Is=0, I=128)
    note(f"[route ragged router tiles] T={T} E={E} k={k} identity={ident}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    idx, tw, _ = lmoe.route(sh, w, g["x"])
    torch.cuda.synchronize()
    inp = host_inputs(t)
    x = O.decode(inp["x"], cfg.act)
    r = O.route(x, O.decode(inp["w_router"], cfg.act), inp["b_router"].astype(np.float64), cfg.k)
    res = check_selection(idx.cpu().numpy(), tw.cpu().numpy(), r)
    assert res["tokens"] == T


def test_forward_recut_tails_past_segments(dev):
    """Re-cut tail launches in which sub-tiles lie wholly past their segment.
    H = 384, L = 128, E = 200, S*Is = 192 at T = 32800 (129 token tiles):
    the route GEMM's 516 tiles leave a tail of 4 (the last token tile's
    router, z and two shared-GLU tiles), re-cut into 128 x 128 sub-tiles, so
    the second halves of the z tile (rows 128..255 of 128) and of the last
    GLU tile (units 192..255 of 192) hold no rows; the up GEMM's 258 tiles
    leave 2, and the second half of its last feature tile (384..511 of 384)
    holds none.  Every row against the oracle, and the first 32768 rows
    bitwise equal to the T = 32768 batch (no tail launch there)."""
    base = get_config("small_bf16")
    cfg = replace(base, name="recut_tails_t32800", T=32800, H=384, L=128, E=200, k=4, S=3, I=128, Is=64)
    note(f"[forward re-cut tails] {cfg.name}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    y, idx, tw = lmoe.forward(sh, w, g["x"])
    torch.cuda.synchronize()
    inp = host_inputs(t)
    ref = O.forward(inp, spec_of(cfg))
    check_selection(idx.cpu().numpy(), tw.cpu().numpy(), ref)
    forced = O.forward(inp, spec_of(cfg), forced_idx=idx.cpu().numpy().astype(np.int64), forced_tol=1e-5)
    err = rowwise_rel_err(to_f64(y), forced["y"])
    note(f"    max row rel err {err:.3e}")
    assert err <= tol_of(cfg)
    sh0 = lmoe.shape_of(cfg, T=32768)
    y0, idx0, _ = lmoe.forward(sh0, w, g["x"][:32768].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(idx0, idx[:32768])
    assert torch.equal(y0, y[:32768])


def _bruteforce_permute(idx, E):
    """Expected result including the dropping rule for ids out of range and
    repeats within a token."""
    T, k = idx.shape
    keep = np.zeros((T, k), bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if 0 <= e < E and e not in seen:
                keep[t, j] = True
                seen.add(e)
    offsets, srt = [0], []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if keep[t, j] and idx[t, j] == e:
                    srt.append(t * k + j)
        offsets.append(len(srt))
    pos = np.full(T * k, -1, np.int64)
    pos[np.array(srt, np.int64)] = np.arange(len(srt))
    return np.array(offsets), np.array(srt), pos


@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (300, 24, 4), (513, 896, 16), (1000, 7, 7)])
def test_permute_matches_oracle(dev, T, E, k):
    note(f"[permute] T={T} E={E} k={k}")
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    sh = lmoe.make_shape(T=T, H=64, L=64, E=E, k=k, I=64, S=0, Is=0)
    off, srt, pos = lmoe.permute(sh, torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    o_off, o_srt, o_pos = O.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(srt.cpu().numpy(), o_srt)
    assert np.array_equal(pos.cpu().numpy(), o_pos)


def test_permute_drops_bad_ids(dev):
    note("[permute] invalid and repeated ids")
    rng = np.random.default_rng(5)
    T, E, k = 300, 10, 4
    idx = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)  # out-of-range ids and repeats
    sh = lmoe.make_shape(T=T, H=64, L=64, E=E, k=k, I=64, S=0, Is=0)
    off, srt, pos = lmoe.permute(sh, torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    b_off, b_srt, b_pos = _bruteforce_permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), b_off)
    assert np.array_equal(srt.cpu().numpy()[: b_off[-1]], b_srt)
    assert np.array_equal(pos.cpu().numpy(), b_pos)


def _oracle_experts(inp, cfg, z64, idx):
    """Oracle expert outputs (sorted order) for latent rows z64 and selection idx."""
    off, srt, _ = O.permute(idx, cfg.E)
    out = np.zeros((idx.size, z64.shape[1]))
    for e in range(cfg.E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        wg = O.matrix(inp["w_gate"], inp.get("s_gate"), e, cfg.w_expert)
        wv = O.matrix(inp["w_value"], inp.get("s_value"), e, cfg.w_expert)
        wo = O.matrix(inp["w_out"], inp.get("s_out"), e, cfg.w_expert)
        zx = O.fp8_activations(z64) if cfg.a8 else z64
        out[lo:hi] = O.expert_ffn(zx[srt[lo:hi] // cfg.k], wg, wv, wo, cfg.cap, cfg.a8)[1]
    return out, off, srt


@pytest.mark.parametrize("name,T", [("tiny_f32", None), ("tiny_situ_stress", None), ("small_bf16", None),
                                    ("small_situ_stress_bf16", None), ("small_situ_stress_bf16", 2000),
                                    ("small_fp8", None), ("small_w8a8", None), ("small_full_k", None)])
def test_expert_gemm(dev, name, T):
    """Latent rows scaled by 1000 where the config is a stress case: |gate| and
    |value| then run far past the cap in the SiTU-GLU epilogue (T = 2000
    reaches the 256-row persistent tiles)."""
    cfg = get_config(name) if T is None else replace(get_config(name), T=T, name=f"{name}_T{T}")
    note(f"[expert_gemm] {cfg.name}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    inp = host_inputs(t)
    # latent rows: seeded, scaled like the stress case when it applies
    gen = torch.Generator().manual_seed(123)
    z = torch.randn((cfg.T, cfg.L), generator=gen) * (1000.0 if cfg.x_scale > 1 else 1.0)
    z = z.to(g["x"].dtype)
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(cfg.E, cfg.k, replace=False) for _ in range(cfg.T)]).astype(np.int64)
    ref, off, srt = _oracle_experts(inp, cfg, to_f64(z), idx)
    if cfg.x_scale > 1:
        routed, _ = _saturates(inp, cfg, to_f64(z))
        note(f"    max |gate| pre-activation {routed:.0f} (cap {cfg.cap})")
        assert routed > 3 * cfg.cap
    out = lmoe.expert_gemm(sh, w, z.to(dev), torch.from_numpy(off.astype(np.int32)).to(dev),
                           torch.from_numpy(srt.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    err = rowwise_rel_err(to_f64(out), ref)
    note(f"    max row rel err {err:.3e}")
    assert err <= tol_of(cfg)


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16"])
def test_combine_norm(dev, name):
    cfg = get_config(name)
    note(f"[combine_norm] {name}")
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    gen = torch.Generator().manual_seed(7)
    T, k, L = cfg.T, cfg.k, cfg.L
    O_rows = (torch.randn((T * k, L), generator=gen) * 3).to(dt)
    perm = torch.randperm(T * k, generator=gen)
    pos = perm.to(torch.int32)
    pos[5] = -1  # a dropped assignment is skipped
    wts = torch.rand((T, k), generator=gen)
    wts = wts / wts.sum(1, keepdim=True)
    gamma = torch.rand(L, generator=gen) + 0.5
    n = lmoe.combine_norm(lmoe.shape_of(cfg), O_rows.to(dev), pos.to(dev), wts.to(dev), gamma.to(dev))
    torch.cuda.synchronize()
    p = pos.numpy().astype(np.int64)
    O64 = to_f64(O_rows)
    c = np.zeros((T, L))
    for j in range(k):
        pj = p.reshape(T, k)[:, j]
        c += np.where(pj[:, None] >= 0, wts.numpy()[:, j:j + 1].astype(np.float64) * O64[np.maximum(pj, 0)], 0)
    ref = O.rmsnorm(c, gamma.numpy().astype(np.float64), cfg.eps)
    err = rowwise_rel_err(to_f64(n), ref)
    assert err <= (1e-5 if cfg.act == "f32" else 8e-3)


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "small_fp8", "small_identity_bf16", "small_full_k"])
def test_up(dev, name):
    cfg = get_config(name)
    note(f"[up] {name}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    inp = host_inputs(t)
    gen = torch.Generator().manual_seed(11)
    n = torch.randn((cfg.T, cfg.L), generator=gen).to(g["x"].dtype)
    y = lmoe.up(sh, w, n.to(dev), g["x"])
    torch.cuda.synchronize()
    x = O.decode(inp["x"], cfg.act)
    n64 = to_f64(n)
    up = n64 if inp["w_up"] is None else n64 @ O.decode(inp["w_up"], cfg.act).T
    S = 0 if inp["ws_gate"] is None else len(inp["ws_gate"])
    sh_ref = O.shared_experts(x, inp["ws_gate"], inp["ws_value"], inp["ws_out"],
                              (inp["ss_gate"], inp["ss_value"], inp["ss_out"]), cfg.w_expert, S, cfg.cap)
    err = rowwise_rel_err(to_f64(y), up + sh_ref)
    note(f"    max row rel err {err:.3e}")
    assert err <= tol_of(cfg)


def test_forward_empty_and_single_token(dev):
    cfg = get_config("small_bf16")
    note("[forward] T=0 and T=1")
    t, g = make_case(replace(cfg, T=1), dev)
    sh, w = _weights(replace(cfg, T=1), g)
    y, idx, tw = lmoe.forward(sh, w, g["x"])
    torch.cuda.synchronize()
    inp = host_inputs(t)
    ref = O.forward(inp, spec_of(cfg), forced_idx=idx.cpu().numpy().astype(np.int64), forced_tol=1e-5)
    assert rowwise_rel_err(to_f64(y), ref["y"]) <= tol_of(cfg)
    sh0 = lmoe.shape_of(cfg, T=0)
    y0, i0, w0 = lmoe.forward(sh0, w, g["x"][:0])
    torch.cuda.synchronize()
    assert y0.shape == (0, cfg.H) and i0.shape == (0, cfg.k)


def test_forward_null_selection_outputs_and_events(dev):
    """lmoe_forward with topk_idx/topk_w NULL (kept in the workspace) gives
    the same y; stage events are recorded in order."""
    cfg = get_config("small_bf16")
    note("[forward] NULL selection outputs, stage events")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(lmoe.NUM_STAGES + 1)]
    y1, _, _ = lmoe.forward(sh, w, g["x"], events=ev)
    lib = lmoe.load_library()
    y2 = torch.empty_like(y1)
    ws = lmoe.alloc_workspace(sh, dev)
    s = lib.lmoe_forward(ctypes.byref(sh), ctypes.byref(w), g["x"].data_ptr(), y2.data_ptr(), None, None,
                         ws.data_ptr(), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), None)
    assert s == 0, lmoe.last_error()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(lmoe.NUM_STAGES)]
    assert all(m >= 0 for m in ms)


def test_forward_deterministic_and_batch_invariant(dev):
    """Two calls agree bit for bit, and the first rows of a batch do not
    depend on the rows after them (each output element is reduced in the same
    order whatever the batch size or tile)."""
    cfg = get_config("small_bf16")
    note("[forward] determinism / batch invariance")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    y1, i1, _ = lmoe.forward(sh, w, g["x"])
    y2, i2, _ = lmoe.forward(sh, w, g["x"])
    shp = lmoe.shape_of(cfg, T=40)
    yp, ip, _ = lmoe.forward(shp, w, g["x"][:40].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(i1, i2)
    assert torch.equal(i1[:40], ip)
    assert torch.equal(y1[:40], yp)


# ----------------------------------------------------------------------------
# Packed expert weights: the layout (bit-exact, against an index-only
# re-arrangement written here) and the layer reading them (bitwise equal to
# the row-major path: same products, same order).
# ----------------------------------------------------------------------------

def _packed_reference(g, cfg):
    """The packed layout of include/lmoe.h built with plain tensor indexing
    on the host (uint16 bit patterns)."""
    E, I, L = cfg.E, cfg.I, cfg.L
    wg, wv, wo = (g[n].cpu().view(torch.int16) for n in ("w_gate", "w_value", "w_out"))
    r = torch.arange(256)
    p = torch.arange(8)
    ch = p[None, :] ^ ((r[:, None] >> 1) & 7)                       # [256, 8] source chunk per position
    cols = (ch[:, :, None] * 8 + torch.arange(8)).reshape(256, 64)  # [256, 64] column within the k-tile
    blocks = []
    nft = -(-I // 128)
    m = r % 64
    u_all = (r // 64) * 32 + (m % 32)
    val = m >= 32
    for e in range(E):
        for f in range(nft):
            u = 128 * f + u_all
            ok = u < I
            uc = torch.where(ok, u, torch.zeros_like(u))
            rows = torch.where(val[:, None], wv[e][uc], wg[e][uc])     # [256, L]
            rows = torch.where(ok[:, None], rows, torch.zeros_like(rows))
            for kt in range(L // 64):
                blocks.append(torch.gather(rows[:, kt * 64:(kt + 1) * 64], 1, cols))
    nfd = -(-L // 256)
    for e in range(E):
        for f in range(nfd):
            fr = 256 * f + r
            ok = fr < L
            rows = wo[e][torch.where(ok, fr, torch.zeros_like(fr))]
            rows = torch.where(ok[:, None], rows, torch.zeros_like(rows))
            for kt in range(I // 64):
                blocks.append(torch.gather(rows[:, kt * 64:(kt + 1) * 64], 1, cols))
    return torch.stack(blocks).reshape(-1)


@pytest.mark.parametrize("name", ["small_bf16", "small_full_k"])
def test_pack_layout(dev, name):
    """small_bf16 pads gate/value tiles (I = 192), small_full_k pads out tiles (L = 128)."""
    cfg = get_config(name)
    note(f"[pack] {name} E={cfg.E} I={cfg.I} L={cfg.L}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    pk = lmoe.pack_experts(sh, w)
    torch.cuda.synchronize()
    assert pk.numel() == lmoe.packed_bytes(sh)
    ref = _packed_reference(g, cfg)
    got = pk.cpu().view(torch.int16)
    assert got.shape == ref.shape
    assert torch.equal(got, ref)


@pytest.mark.parametrize("name,T", [("small_bf16", None), ("small_full_k", None), ("small_identity_bf16", None),
                                    ("small_bf16", 20), ("small_bf16", 700), ("small_bf16", 2000)])
def test_forward_packed_matches_row_major(dev, name, T):
    """Same products in the same order: the packed layer is bitwise equal to
    the row-major one, also with the row-major stacks withheld."""
    cfg = get_config(name) if T is None else replace(get_config(name), T=T, name=f"{name}_T{T}")
    note(f"[packed forward] {cfg.name}")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    y0, i0, w0 = lmoe.forward(sh, w, g["x"])
    pk = lmoe.pack_experts(sh, w)
    wp = lmoe.with_packed(sh, w, pk)
    y1, i1, w1 = lmoe.forward(sh, wp, g["x"])
    only = {k: v for k, v in g.items() if k not in ("w_gate", "w_value", "w_out")}
    wpo = lmoe.with_packed(sh, lmoe.make_weights(sh, only), pk)
    y2, _, _ = lmoe.forward(sh, wpo, g["x"])
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(w0, w1)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal(y0.view(torch.int16), y2.view(torch.int16))


def test_expert_gemm_packed(dev):
    cfg = get_config("small_bf16")
    note("[packed expert_gemm] small_bf16")
    t, g = make_case(cfg, dev)
    sh, w = _weights(cfg, g)
    idx, tw, z = lmoe.route(sh, w, g["x"])
    offsets, sorted_, pos = lmoe.permute(sh, idx)
    o0 = lmoe.expert_gemm(sh, w, z, offsets, sorted_)
    wp = lmoe.with_packed(sh, w, lmoe.pack_experts(sh, w))
    o1 = lmoe.expert_gemm(sh, wp, z, offsets, sorted_)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


def _quant_input(R, C, seed):
    """bf16 rows whose 128-column blocks span 1e-30 .. 1e4 in magnitude, with
    all-zero blocks, lone nonzeros, negative zeros and values far below their
    block's maximum (codes in the e4m3 subnormal range and rounded to zero)."""
    rng = np.random.default_rng(seed)
    nb = C // 128
    mag = np.exp(rng.uniform(np.log(1e-30), np.log(1e4), (R, nb)))
    v = rng.standard_normal((R, C)) * np.repeat(mag, 128, axis=1)
    v[:, ::7] *= 1e-4  # far below the block max
    v[3, C - 128:] = 0.0
    v[4, :] = -0.0
    v[5, :128] = 0.0
    v[5, 17] = -2.5
    v[6, C - 56] = 1e30  # one huge value, the rest of its block rounds to zero
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("R,C", [(1, 128), (333, 384), (1000, 1024)])
def test_quantize_1x128_bit_exact(dev, R, C):
    """Codes and scales bit for bit against the oracle's quantiser, which takes
    the same fp32 decisions (scale = amax / 448, code = e4m3fn(x / scale))."""
    note(f"[quantize_1x128] R={R} C={C}")
    x = _quant_input(max(R, 8), C, seed=R + C)[:R].contiguous()
    q, sc = lmoe.quantize_1x128(x.to(dev))
    torch.cuda.synchronize()
    rq, rs = O.quantize_1x128(to_f64(x))
    got_q = q.cpu().view(torch.uint8).numpy()
    got_s = sc.cpu().numpy()
    assert got_s.shape == (C // 128, R)
    bad = np.argwhere(got_q != rq)
    if bad.size:
        r, c = bad[0]
        note(f"    first code mismatch at ({r}, {c}): x={float(x[r, c])!r} got {got_q[r, c]:#04x} want {rq[r, c]:#04x}")
    assert bad.size == 0
    assert np.array_equal(got_s.T.view(np.uint32), rs.view(np.uint32))


def test_quantize_1x128_expert_rows_at_k3_size(dev):
    """The down GEMM's input at the 8192-token K3 layer: 131072 rows of 1024,
    sampled rows checked bit for bit."""
    R, C = 8192 * 16, 1024
    note(f"[quantize_1x128] R={R} C={C}")
    gen = torch.Generator().manual_seed(31)
    x = (torch.randn((R, C), generator=gen) * 0.3).to(torch.bfloat16)
    q, sc = lmoe.quantize_1x128(x.to(dev))
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(R, 300, replace=False)
    rows[0], rows[1] = 0, R - 1
    rq, rs = O.quantize_1x128(to_f64(x[torch.from_numpy(rows)]))
    assert np.array_equal(q[torch.from_numpy(rows).to(dev)].cpu().view(torch.uint8).numpy(), rq)
    assert np.array_equal(sc[:, torch.from_numpy(rows).to(dev)].cpu().numpy().T, rs)


def test_quantize_1x128_rejects(dev):
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(lmoe.LmoeError):
        lmoe.quantize_1x128(x[:, :200].contiguous())
    q, sc = lmoe.quantize_1x128(x[:0])
    assert q.shape == (0, 256) and sc.shape == (2, 0)


@pytest.mark.gpu
def test_topk_exact_ties_and_infinite_bias(dev):
    """Identical router rows give every expert the same logit, so the biased
    scores tie exactly wherever the bias does: the selection must run by bias
    descending, then expert index ascending, with -inf biases last, and every
    selected weight is 1/k.  Checked against the oracle's selection rule
    (a library sort on (-score, index)) applied to the biases alone."""
    cfg = get_config("small_bf16")
    note(f"[top-k ties] {cfg.name}")
    t, g = make_case(cfg, dev)
    E, k = cfg.E, cfg.k
    g = dict(g)
    g["w_router"] = g["w_router"][:1].expand(E, -1).contiguous()
    # two experts at the top level, four tied at the next, the rest lower or -inf
    levels = np.full(E, -0.5)
    levels[[7, 3]] = 0.25
    levels[[20, 9, 1, 5]] = 0.0
    levels[[0, 2, 4, 6, 11]] = -np.inf
    g["b_router"] = torch.tensor(levels, dtype=torch.float32, device=dev)
    sh, w = _weights(cfg, g)
    logits = lmoe.router_logits(sh, w, g["x"])
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    assert (lg == lg[:, :1]).all(), "identical router rows give identical logits"
    idx, tw, _ = lmoe.route(sh, w, g["x"])
    torch.cuda.synchronize()
    want, _ = O.select_topk(np.broadcast_to(levels, (cfg.T, E)).astype(np.float64), k)
    assert k == 4 and list(want[0]) == [3, 7, 1, 5]
    np.testing.assert_array_equal(idx.cpu().numpy(), want)
    np.testing.assert_allclose(tw.cpu().numpy(), 1.0 / k, rtol=1e-6)

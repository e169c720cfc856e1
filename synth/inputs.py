"""Deterministic synthetic tensors for a LayerConfig.

Distributions: x ~ N(0,1) (times cfg.x_scale); every projection and expert
weight ~ N(0, 0.02); RMSNorm gain ~ U(0.5, 1.5); router bias 0, or for the
skewed-routing config b_e = r_e^-1.1 with r a seeded permutation of 1..E.

Each tensor (and each expert slice, and each 64-row block of x) has its own
seed derived from (config seed, tensor name, index), so any expert can be
regenerated alone and the first rows of x agree between token counts.  Draws
are fp32 and are rounded to the storage dtype by torch's own conversion.
fp8 storage is OCP e4m3fn with one fp32 scale per 128x128 block: scale =
amax/448 (1 where the block is all zero), code = e4m3fn(clamp(w/scale)).
That quantisation is input preparation: both sides decode the same codes.
"""

import zlib

import numpy as np
import torch

from .configs import LayerConfig

STD_W = 0.02
X_BLOCK = 64
F8_BLOCK = 128
F8_MAX = 448.0

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f8": torch.float8_e4m3fn}


def derive_seed(seed: int, name: str, index: int = 0) -> int:
    ss = np.random.SeedSequence([int(seed), zlib.crc32(name.encode()), int(index)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, seed, device, std=1.0):
    t = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def quantize_e4m3_blocks(w: torch.Tensor):
    """fp32 [R, C] (R, C multiples of 128) -> (e4m3fn codes [R, C], fp32 scales [R/128, C/128])."""
    R, C = w.shape
    blk = w.reshape(R // F8_BLOCK, F8_BLOCK, C // F8_BLOCK, F8_BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / F8_MAX, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp_(-F8_MAX, F8_MAX)
    return q.reshape(R, C).to(torch.float8_e4m3fn), scale.contiguous()


def _expert_stack(cfg, name, n, rows, cols, dtype, device):
    """n independent [rows, cols] matrices, one seed per slice."""
    if dtype == "f8":
        if rows % F8_BLOCK or cols % F8_BLOCK:
            raise ValueError(f"{name}: fp8 block scaling needs dims divisible by 128, got {rows}x{cols}")
        out = torch.empty((n, rows, cols), dtype=torch.float8_e4m3fn, device=device)
        sc = torch.empty((n, rows // F8_BLOCK, cols // F8_BLOCK), dtype=torch.float32, device=device)
        for e in range(n):
            q, s = quantize_e4m3_blocks(_randn((rows, cols), derive_seed(cfg.seed, name, e), device, STD_W))
            out[e].copy_(q)
            sc[e].copy_(s)
        return out, sc
    out = torch.empty((n, rows, cols), dtype=_TORCH_DT[dtype], device=device)
    for e in range(n):
        out[e].copy_(_randn((rows, cols), derive_seed(cfg.seed, name, e), device, STD_W))
    return out, None


def make_x(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    seed = cfg.x_seed if cfg.x_seed >= 0 else cfg.seed
    x = torch.empty((cfg.T, cfg.H), dtype=_TORCH_DT[cfg.act], device=device)
    for b in range(0, cfg.T, X_BLOCK):
        rows = min(X_BLOCK, cfg.T - b)
        blk = _randn((X_BLOCK, cfg.H), derive_seed(seed, "x", b // X_BLOCK), device)
        if cfg.x_scale != 1.0:
            blk.mul_(cfg.x_scale)
        x[b:b + rows].copy_(blk[:rows])
    return x


def make_router_bias(cfg: LayerConfig, device="cpu") -> torch.Tensor:
    if cfg.bias == "zero":
        return torch.zeros(cfg.E, dtype=torch.float32, device=device)
    if cfg.bias == "zipf1.1":
        rng = np.random.Generator(np.random.PCG64(derive_seed(cfg.seed, "router_bias", 0)))
        rank = rng.permutation(cfg.E).astype(np.float64) + 1.0
        return torch.from_numpy((rank ** -1.1).astype(np.float32)).to(device)
    raise ValueError(f"unknown bias kind {cfg.bias!r}")


def make_inputs(cfg: LayerConfig, device="cpu", with_x: bool = True) -> dict:
    """All tensors of one layer call, as torch tensors on `device`.

    Keys: x, w_router, b_router, w_down, w_gate, w_value, w_out, s_gate,
    s_value, s_out, gamma, w_up, ws_gate, ws_value, ws_out, ss_gate,
    ss_value, ss_out.  Absent tensors (identity projections, fp8 scales of
    non-fp8 storage, shared weights when S == 0) are None.
    """
    if cfg.identity_proj and cfg.L != cfg.H:
        raise ValueError("identity projections need L == H")
    act = cfg.act
    t = {}
    t["x"] = make_x(cfg, device) if with_x else None
    t["w_router"] = _randn((cfg.E, cfg.H), derive_seed(cfg.seed, "w_router"), device, STD_W).to(_TORCH_DT[act])
    t["b_router"] = make_router_bias(cfg, device)
    if cfg.identity_proj:
        t["w_down"] = None
        t["w_up"] = None
    else:
        t["w_down"] = _randn((cfg.L, cfg.H), derive_seed(cfg.seed, "w_down"), device, STD_W).to(_TORCH_DT[act])
        t["w_up"] = _randn((cfg.H, cfg.L), derive_seed(cfg.seed, "w_up"), device, STD_W).to(_TORCH_DT[act])
    t["w_gate"], t["s_gate"] = _expert_stack(cfg, "w_gate", cfg.E, cfg.I, cfg.L, cfg.w_expert, device)
    t["w_value"], t["s_value"] = _expert_stack(cfg, "w_value", cfg.E, cfg.I, cfg.L, cfg.w_expert, device)
    t["w_out"], t["s_out"] = _expert_stack(cfg, "w_out", cfg.E, cfg.L, cfg.I, cfg.w_expert, device)
    g = torch.rand((cfg.L,), generator=_gen(derive_seed(cfg.seed, "gamma"), device), device=device,
                   dtype=torch.float32)
    t["gamma"] = g.add_(0.5)
    if cfg.S > 0:
        t["ws_gate"], t["ss_gate"] = _expert_stack(cfg, "ws_gate", cfg.S, cfg.Is, cfg.H, cfg.w_expert, device)
        t["ws_value"], t["ss_value"] = _expert_stack(cfg, "ws_value", cfg.S, cfg.Is, cfg.H, cfg.w_expert, device)
        t["ws_out"], t["ss_out"] = _expert_stack(cfg, "ws_out", cfg.S, cfg.H, cfg.Is, cfg.w_expert, device)
    else:
        for n in ("ws_gate", "ws_value", "ws_out", "ss_gate", "ss_value", "ss_out"):
            t[n] = None
    return t


def raw_numpy(t):
    """Storage bytes of a tensor as numpy: f32 -> float32, bf16 -> uint16 bit
    patterns, e4m3fn -> uint8 codes, int32 -> int32.  Copies to host."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype in (torch.float32, torch.int32, torch.int64, torch.float64):
        return t.cpu().numpy()
    raise TypeError(f"no raw view for {t.dtype}")


class LazyExperts:
    """Indexable over experts: item e is raw_numpy(t[e]), fetched on demand.

    Lets a host consumer touch only the experts it needs from a large device
    tensor without copying the whole stack."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __len__(self):
        return self.shape[0]

    def __getitem__(self, e):
        return raw_numpy(self.t[int(e)])


def make_router_logits(T: int, E: int, seed: int, spread: float = 0.0, std: float = 1.7) -> np.ndarray:
    """Seeded fp32 router logits [T, E]: N(0, std^2) (std 1.7 is the logit
    spread of the K3-shape router on N(0,1) inputs), plus a per-expert offset
    growing linearly from -spread to +spread (a router that favours some
    experts; 0: none)."""
    rng = np.random.default_rng(derive_seed(seed, "router_logits", T * 4096 + E))
    lg = rng.standard_normal((T, E)) * std
    if spread:
        lg = lg + np.linspace(-spread, spread, E)[None, :]
    return lg.astype(np.float32)

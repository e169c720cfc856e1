"""ctypes binding of liblmoe.so: the Stable Latent MoE layer forward pass.

Argument marshalling only: torch tensors become device pointers, the current
HIP stream is passed through, and a non-zero status raises LmoeError with the
library's message.  Every step of the layer runs in the library's kernels;
there is no fallback path, and using the binding without the built library
raises immediately.
"""

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblmoe.so")

F32, BF16, F8E4M3 = 0, 1, 2
NUM_STAGES = 7
NOALLOC_SCRATCH_BYTES = 64 << 20  # LMOE_NOALLOC_SCRATCH_BYTES
STAGES = ("route_gemm", "topk", "permute", "expert_gate_value", "expert_down", "combine_norm", "up")
BWD_STAGES = ("forward_recompute", "up_norm_grads", "expert_grads", "latent_router_grads", "shared_grads")
STATUS = {0: "LMOE_OK", 1: "LMOE_EINVAL", 2: "LMOE_EUNSUPPORTED", 3: "LMOE_EWORKSPACE", 4: "LMOE_EHIP"}
DTYPE_CODE = {"f32": F32, "bf16": BF16, "f8": F8E4M3}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16, F8E4M3: torch.float8_e4m3fn}

EXPORTS = ("lmoe_validate", "lmoe_workspace_bytes", "lmoe_forward", "lmoe_forward_noalloc", "lmoe_route",
           "lmoe_permute",
           "lmoe_expert_gemm", "lmoe_combine_norm", "lmoe_up", "lmoe_router_logits", "lmoe_quantile_bias",
           "lmoe_packed_bytes", "lmoe_pack_experts", "lmoe_quantize_1x128", "lmoe_backward",
           "lmoe_backward_workspace_bytes",
           "lmoe_status_str", "lmoe_last_error")


class LmoeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("S", ctypes.c_int32), ("Is", ctypes.c_int32),
                ("act", ctypes.c_int32), ("w_expert", ctypes.c_int32), ("cap", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("a8", ctypes.c_int32)]


_WEIGHT_FIELDS = ("w_router", "b_router", "w_down", "w_gate", "w_value", "w_out", "s_gate", "s_value", "s_out",
                  "gamma", "w_up", "ws_gate", "ws_value", "ws_out", "ss_gate", "ss_value", "ss_out", "packed")


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


GRAD_FIELDS = ("dx", "dw_router", "dw_down", "dw_gate", "dw_value", "dw_out", "dgamma", "dw_up", "dws_gate",
               "dws_value", "dws_out")


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load liblmoe.so (torch's HIP runtime must be the one it binds to, so
    torch is imported first).  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_moe_transformer_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32p, f32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    sp, wp = ctypes.POINTER(Shape), ctypes.POINTER(Weights)
    sig = {
        "lmoe_validate": (ctypes.c_int, [sp, wp, sz]),
        "lmoe_workspace_bytes": (sz, [sp]),
        "lmoe_forward": (ctypes.c_int, [sp, wp, vp, vp, i32p, f32p, vp, sz, vp, vp]),
        "lmoe_forward_noalloc": (ctypes.c_int, [sp, wp, vp, vp, i32p, f32p, vp]),
        "lmoe_route": (ctypes.c_int, [sp, wp, vp, i32p, f32p, vp, vp, sz, vp]),
        "lmoe_permute": (ctypes.c_int, [sp, i32p, i32p, i32p, i32p, vp, sz, vp]),
        "lmoe_expert_gemm": (ctypes.c_int, [sp, wp, vp, i32p, i32p, vp, vp, sz, vp]),
        "lmoe_combine_norm": (ctypes.c_int, [sp, vp, i32p, f32p, f32p, vp, vp]),
        "lmoe_up": (ctypes.c_int, [sp, wp, vp, vp, vp, vp, sz, vp]),
        "lmoe_router_logits": (ctypes.c_int, [sp, wp, vp, f32p, vp]),
        "lmoe_quantile_bias": (ctypes.c_int, [sp, f32p, f32p, vp, sz, vp]),
        "lmoe_packed_bytes": (sz, [sp]),
        "lmoe_pack_experts": (ctypes.c_int, [sp, wp, vp, sz, vp]),
        "lmoe_quantize_1x128": (ctypes.c_int, [vp, ctypes.c_int64, ctypes.c_int32, vp, f32p, vp]),
        "lmoe_backward_workspace_bytes": (sz, [sp]),
        "lmoe_backward": (ctypes.c_int, [sp, wp, vp, vp, i32p, ctypes.POINTER(Grads), vp, sz, vp, vp]),
        "lmoe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "lmoe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise LmoeError(status, _lib.lmoe_last_error().decode())


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def make_shape(T, H, L, E, k, I, S, Is, act="bf16", w_expert="bf16", cap=100.0, eps=1e-6, a8=False) -> Shape:
    return Shape(int(T), int(H), int(L), int(E), int(k), int(I), int(S), int(Is), DTYPE_CODE[act],
                 DTYPE_CODE[w_expert], float(cap), float(eps), int(bool(a8)))


def shape_of(cfg, T=None) -> Shape:
    """Shape from any object with the fields T, H, L, E, k, I, S, Is, act,
    w_expert, cap, eps and optionally a8 (e.g. synth.LayerConfig)."""
    return make_shape(cfg.T if T is None else T, cfg.H, cfg.L, cfg.E, cfg.k, cfg.I, cfg.S, cfg.Is, cfg.act,
                      cfg.w_expert, cfg.cap, cfg.eps, getattr(cfg, "a8", False))


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def make_weights(sh: Shape, t: dict) -> Weights:
    """Weights struct from a dict of tensors (keys as in include/lmoe.h;
    "packed" is the uint8 buffer filled by pack_experts, or absent)."""
    act, wexp = _TORCH[sh.act], _TORCH[sh.w_expert]
    want = {"w_router": act, "b_router": torch.float32, "w_down": act, "w_gate": wexp, "w_value": wexp,
            "w_out": wexp, "s_gate": torch.float32, "s_value": torch.float32, "s_out": torch.float32,
            "gamma": torch.float32, "w_up": act, "ws_gate": wexp, "ws_value": wexp, "ws_out": wexp,
            "ss_gate": torch.float32, "ss_value": torch.float32, "ss_out": torch.float32, "packed": torch.uint8}
    vals = {}
    for n in _WEIGHT_FIELDS:
        vals[n] = _ptr(t.get(n), want[n], n)
    w = Weights(**vals)
    w._keep = [t.get(n) for n in _WEIGHT_FIELDS]  # keep the tensors alive with the struct
    return w


def router_logits(sh: Shape, w: Weights, x, out=None, stream=None):
    """logits [T, E] fp32 = x . W_r^T."""
    lib = load_library()
    out = torch.empty((sh.T, sh.E), dtype=torch.float32, device=x.device) if out is None else out
    _check(lib.lmoe_router_logits(ctypes.byref(sh), ctypes.byref(w), _ptr(x, _act_dtype(sh), "x"),
                                  _ptr(out, torch.float32, "logits"), _stream(stream)))
    return out


def quantile_bias(sh: Shape, logits, out=None, ws=None, stream=None):
    """Quantile Balancing selection bias [E] fp32 of a batch's router logits."""
    lib = load_library()
    out = torch.empty((sh.E,), dtype=torch.float32, device=logits.device) if out is None else out
    ws = alloc_workspace(sh, logits.device) if ws is None else ws
    _check(lib.lmoe_quantile_bias(ctypes.byref(sh), _ptr(logits, torch.float32, "logits"), _ptr(out, torch.float32, "bias"),
                                  _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
    return out


def quantize_1x128(x, q=None, scales=None, stream=None):
    """Per-row 1x128 e4m3fn quantisation of a bf16 [R, C] device tensor:
    returns (codes [R, C] float8_e4m3fn, scales [C/128, R] fp32, block-major);
    see lmoe_quantize_1x128 in include/lmoe.h."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [R, C]")
    R, C = x.shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.float8_e4m3fn, device=x.device)
    if scales is None:
        scales = torch.empty((C // 128 if C % 128 == 0 else 0, R), dtype=torch.float32, device=x.device)
    _check(lib.lmoe_quantize_1x128(_ptr(x, torch.bfloat16, "x"), ctypes.c_int64(R), ctypes.c_int32(C),
                                   _ptr(q, torch.float8_e4m3fn, "q"), _ptr(scales, torch.float32, "scales"),
                                   _stream(stream)))
    return q, scales


def backward_workspace_bytes(sh: Shape) -> int:
    load_library()
    return int(_lib.lmoe_backward_workspace_bytes(ctypes.byref(sh)))


def grad_shapes(sh: Shape, w: Weights) -> dict:
    """Shapes of the fp32 gradients lmoe_backward writes for this layer."""
    T, H, L, E, I, S, Is = sh.T, sh.H, sh.L, sh.E, sh.I, sh.S, sh.Is
    out = {"dx": (T, H), "dw_router": (E, H), "dw_gate": (E, I, L), "dw_value": (E, I, L), "dw_out": (E, L, I),
           "dgamma": (L,)}
    if w.w_down:
        out["dw_down"] = (L, H)
    if w.w_up:
        out["dw_up"] = (H, L)
    if S > 0:
        out.update(dws_gate=(S, Is, H), dws_value=(S, Is, H), dws_out=(S, H, Is))
    return out


def backward(sh: Shape, w: Weights, x, dy, grads=None, ws=None, stream=None, events=None):
    """Gradients of sum(y * dy) for x and every weight (fp32 device tensors,
    allocated when `grads` is None) and the selection the recomputed forward
    took; see lmoe_backward in include/lmoe.h.  Returns (grads dict, idx).
    events: optional list of len(BWD_STAGES) + 1 torch.cuda.Event recorded
    around the stages."""
    lib = load_library()
    dev = x.device
    if grads is None:
        grads = {n: torch.empty(shp, dtype=torch.float32, device=dev) for n, shp in grad_shapes(sh, w).items()}
    g = Grads(**{n: _ptr(grads.get(n), torch.float32, n) for n in GRAD_FIELDS})
    idx = torch.empty((sh.T, sh.k), dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(max(backward_workspace_bytes(sh), 256), dtype=torch.uint8, device=dev)
    ev = None
    if events is not None:
        if len(events) != len(BWD_STAGES) + 1:
            raise ValueError(f"events must hold {len(BWD_STAGES) + 1} torch.cuda.Event objects")
        for e in events:
            if not e.cuda_event:
                e.record()  # creates the underlying event
        ev = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(lib.lmoe_backward(ctypes.byref(sh), ctypes.byref(w), _ptr(x, _TORCH[sh.act], "x"),
                             _ptr(dy, _TORCH[sh.act], "dy"), _ptr(idx, torch.int32, "topk_idx"), ctypes.byref(g),
                             _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream), ev))
    return grads, idx


def packed_bytes(sh: Shape) -> int:
    """Bytes of the packed expert weights (0: the shape has no packed form)."""
    load_library()
    return int(_lib.lmoe_packed_bytes(ctypes.byref(sh)))


def pack_experts(sh: Shape, w: Weights, out=None, stream=None):
    """Packed copy of the routed expert weights (uint8 device tensor) for
    Weights.packed; see lmoe_pack_experts in include/lmoe.h."""
    n = packed_bytes(sh)
    if n == 0:
        raise LmoeError(2, "this shape has no packed expert layout")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
    if out.dtype != torch.uint8 or out.numel() < n:
        raise ValueError(f"out must be a uint8 tensor of at least {n} bytes")
    _check(_lib.lmoe_pack_experts(ctypes.byref(sh), ctypes.byref(w), _ptr(out, torch.uint8, "out"), n,
                                  _stream(stream)))
    return out


def with_packed(sh: Shape, w: Weights, packed) -> Weights:
    """Copy of `w` whose expert GEMMs read `packed` (from pack_experts)."""
    vals = {n: getattr(w, n) for n in _WEIGHT_FIELDS}
    vals["packed"] = _ptr(packed, torch.uint8, "packed")
    w2 = Weights(**vals)
    w2._keep = list(getattr(w, "_keep", [])) + [packed]
    return w2


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_bytes(sh: Shape) -> int:
    return int(load_library().lmoe_workspace_bytes(ctypes.byref(sh)))


def validate(sh: Shape, w: Weights, ws_bytes: int) -> int:
    """Host-only check; returns the status code (no exception)."""
    return int(load_library().lmoe_validate(ctypes.byref(sh), ctypes.byref(w) if w is not None else None, ws_bytes))


def last_error() -> str:
    return load_library().lmoe_last_error().decode()


def alloc_workspace(sh: Shape, device="cuda"):
    n = workspace_bytes(sh)
    if n == 0:
        raise LmoeError(1, "invalid shape: " + last_error())
    return torch.empty(n, dtype=torch.uint8, device=device)


def _act_dtype(sh):
    return _TORCH[sh.act]


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def forward(sh: Shape, w: Weights, x, y=None, topk_idx=None, topk_w=None, ws=None, stream=None, events=None):
    """Whole layer; returns (y, topk_idx, topk_w)."""
    lib = load_library()
    T = sh.T
    y = torch.empty((T, sh.H), dtype=_act_dtype(sh), device=x.device) if y is None else y
    topk_idx = torch.empty((T, sh.k), dtype=torch.int32, device=x.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, sh.k), dtype=torch.float32, device=x.device) if topk_w is None else topk_w
    ws = alloc_workspace(sh, x.device) if ws is None else ws
    ev = None
    if events is not None:
        if len(events) != NUM_STAGES + 1:
            raise ValueError(f"events must hold {NUM_STAGES + 1} torch.cuda.Event objects")
        for e in events:
            if not e.cuda_event:
                e.record()  # torch creates the HIP event on first use
        ev = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check(lib.lmoe_forward(ctypes.byref(sh), ctypes.byref(w), _ptr(x, _act_dtype(sh), "x"),
                            _ptr(y, _act_dtype(sh), "y"), _ptr(topk_idx, torch.int32, "topk_idx"),
                            _ptr(topk_w, torch.float32, "topk_w"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
                            _stream(stream), ev))
    return y, topk_idx, topk_w


def forward_noalloc(sh: Shape, w: Weights, x, y, topk_idx=None, topk_w=None, stream=None):
    """Whole layer through lmoe_forward_noalloc (the library's own per-device
    scratch, no workspace); y, and topk_idx / topk_w when given, are written
    in place.  Returns (y, topk_idx, topk_w)."""
    lib = load_library()
    _check(lib.lmoe_forward_noalloc(ctypes.byref(sh), ctypes.byref(w), _ptr(x, _act_dtype(sh), "x"),
                                    _ptr(y, _act_dtype(sh), "y"),
                                    None if topk_idx is None else _ptr(topk_idx, torch.int32, "topk_idx"),
                                    None if topk_w is None else _ptr(topk_w, torch.float32, "topk_w"),
                                    _stream(stream)))
    return y, topk_idx, topk_w


def route(sh: Shape, w: Weights, x, topk_idx=None, topk_w=None, z=None, ws=None, stream=None):
    """Router + latent down-projection; returns (topk_idx, topk_w, z).  z is
    None when the layer has no down-projection."""
    lib = load_library()
    T = sh.T
    topk_idx = torch.empty((T, sh.k), dtype=torch.int32, device=x.device) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, sh.k), dtype=torch.float32, device=x.device) if topk_w is None else topk_w
    if z is None and w.w_down is not None:
        z = torch.empty((T, sh.L), dtype=_act_dtype(sh), device=x.device)
    ws = alloc_workspace(sh, x.device) if ws is None else ws
    _check(lib.lmoe_route(ctypes.byref(sh), ctypes.byref(w), _ptr(x, _act_dtype(sh), "x"),
                          _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(topk_w, torch.float32, "topk_w"),
                          _ptr(z, _act_dtype(sh), "z"), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
    return topk_idx, topk_w, z


def permute(sh: Shape, topk_idx, ws=None, stream=None):
    """Counting sort by expert; returns (offsets [E+1], sorted [T*k], pos [T*k])."""
    lib = load_library()
    dev = topk_idx.device
    offsets = torch.empty(sh.E + 1, dtype=torch.int32, device=dev)
    sorted_ = torch.empty(sh.T * sh.k, dtype=torch.int32, device=dev)
    pos = torch.empty(sh.T * sh.k, dtype=torch.int32, device=dev)
    ws = alloc_workspace(sh, dev) if ws is None else ws
    _check(lib.lmoe_permute(ctypes.byref(sh), _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(offsets),
                            _ptr(sorted_), _ptr(pos), _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
    return offsets, sorted_, pos


def expert_gemm(sh: Shape, w: Weights, z, offsets, sorted_, out=None, ws=None, stream=None):
    """Routed experts; returns expert_out [T*k, L] in sorted order."""
    lib = load_library()
    out = torch.empty((sh.T * sh.k, sh.L), dtype=_act_dtype(sh), device=z.device) if out is None else out
    ws = alloc_workspace(sh, z.device) if ws is None else ws
    _check(lib.lmoe_expert_gemm(ctypes.byref(sh), ctypes.byref(w), _ptr(z, _act_dtype(sh), "z"),
                                _ptr(offsets, torch.int32, "offsets"), _ptr(sorted_, torch.int32, "sorted"),
                                _ptr(out, _act_dtype(sh), "expert_out"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
                                _stream(stream)))
    return out


def combine_norm(sh: Shape, expert_out, pos, topk_w, gamma, n=None, stream=None):
    """Weighted combine + RMSNorm; returns n [T, L]."""
    lib = load_library()
    n = torch.empty((sh.T, sh.L), dtype=_act_dtype(sh), device=expert_out.device) if n is None else n
    _check(lib.lmoe_combine_norm(ctypes.byref(sh), _ptr(expert_out, _act_dtype(sh), "expert_out"),
                                 _ptr(pos, torch.int32, "pos"), _ptr(topk_w, torch.float32, "topk_w"),
                                 _ptr(gamma, torch.float32, "gamma"), _ptr(n, _act_dtype(sh), "n"),
                                 _stream(stream)))
    return n


def up(sh: Shape, w: Weights, n, x, y=None, ws=None, stream=None):
    """Up-projection + shared experts; returns y [T, H]."""
    lib = load_library()
    y = torch.empty((sh.T, sh.H), dtype=_act_dtype(sh), device=n.device) if y is None else y
    ws = alloc_workspace(sh, n.device) if ws is None else ws
    _check(lib.lmoe_up(ctypes.byref(sh), ctypes.byref(w), _ptr(n, _act_dtype(sh), "n"),
                       _ptr(x, _act_dtype(sh), "x"), _ptr(y, _act_dtype(sh), "y"), _ptr(ws, torch.uint8, "ws"),
                       ws.numel(), _stream(stream)))
    return y


# ----------------------------------------------------------------------------
# work accounting (used by the benchmark)
# ----------------------------------------------------------------------------

def layer_flops(sh: Shape, tokens=None, projections=True) -> float:
    """Algorithmic FLOPs of one layer call (2 per multiply-add): router, down,
    k experts per token (gate, value, out), up, shared experts.  projections
    False: identity down/up projections (no latent) cost nothing."""
    T = sh.T if tokens is None else tokens
    H, L, E, k, I, S, Is = sh.H, sh.L, sh.E, sh.k, sh.I, sh.S, sh.Is
    proj = 2 * L * H if projections else 0
    per_tok = 2 * (E * H + k * 3 * L * I + S * 3 * H * Is) + 2 * proj
    return float(T) * per_tok


def backward_flops(sh: Shape, projections=True, up=True) -> dict:
    """Algorithmic FLOPs of one lmoe_backward call by stage (2 per
    multiply-add): the forward recompute (router, down, expert gate/value/out),
    dn and dW_up, the routed expert dgrads and wgrads (dA, dW_out, dz rows,
    dW_gate, dW_value), the latent and router gradients, and the shared
    experts (recompute, dgrads, wgrads)."""
    T, H, L, E, k, I, S, Is = sh.T, sh.H, sh.L, sh.E, sh.k, sh.I, sh.S, sh.Is
    p = 1 if projections else 0
    u = 1 if up else 0
    st = {
        "forward_recompute": T * (2 * E * H + 2 * L * H * p + 2 * k * 3 * L * I),
        "up_norm_grads": T * 4 * H * L * u,
        "expert_grads": T * 12 * k * L * I,
        "latent_router_grads": T * (4 * L * H * p + 4 * E * H),
        "shared_grads": T * 16 * S * Is * H,
    }
    return {n: float(v) for n, v in st.items()}


def backward_expert_bytes(sh: Shape) -> float:
    """Algorithmic HBM bytes of lmoe_backward's routed-expert gradient stage:
    the bf16 gate, value and out weights of every expert read once (the
    dgrads), the fp32 gate, value and out gradients of every expert written
    once (experts no token chose get zeros), and each activation written or
    read once: dO (bf16), A (bf16), dA (fp32), G and V (fp32), dG and dV
    (bf16), the latent gradient rows (fp32) and z (bf16)."""
    T, L, E, k, I = sh.T, sh.L, sh.E, sh.k, sh.I
    tk = T * k
    weights = 3 * E * I * L * 2
    grads = 3 * E * I * L * 4
    acts = tk * (L * 2 + I * 2 + I * 4 + 2 * I * 4 + 2 * I * 2 + L * 4) + T * L * 2
    return float(weights + grads + acts)


def expert_bytes(sh: Shape, touched: int, which="all") -> float:
    """Weight bytes of `touched` routed experts: gate+value, down, or all."""
    wb = {F32: 4, BF16: 2, F8E4M3: 1}[sh.w_expert]
    gv = 2 * sh.I * sh.L * wb
    dn = sh.L * sh.I * wb
    if sh.w_expert == F8E4M3:  # fp32 block scales
        gv += 2 * (sh.I // 128) * (sh.L // 128) * 4
        dn += (sh.I // 128) * (sh.L // 128) * 4
    per = {"gv": gv, "down": dn, "all": gv + dn}[which]
    return float(touched) * per


def dense_bytes(sh: Shape, projections=True) -> float:
    """Router, down, up and shared-expert weight bytes (plus the bias and gamma)."""
    ab = {F32: 4, BF16: 2}[sh.act]
    wb = {F32: 4, BF16: 2, F8E4M3: 1}[sh.w_expert]
    b = sh.E * sh.H * ab + 4 * sh.E + (2 * sh.L * sh.H * ab if projections else 0) + 4 * sh.L
    b += sh.S * 3 * sh.H * sh.Is * wb
    if sh.w_expert == F8E4M3:
        b += sh.S * 3 * (sh.H // 128) * (sh.Is // 128) * 4
    return float(b)


def isfinite_cap(sh: Shape) -> bool:
    return math.isfinite(sh.cap)

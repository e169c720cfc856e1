"""Layer configurations for the Stable Latent MoE forward pass.

The K3 shape (hidden 7168, latent 3584 = half of it, 896 routed experts with
16 active per token, 2 always-on shared experts, SiTU-GLU cap about 100) is
the one the Kimi K3 write-ups give: P1 = aitrending.vip, "The 2.8-Trillion-
Parameter Problem: Why Bigger Models Break the Old Playbook", Technical
Details; P2 = wpnews.pro, same title (Part 1 of "Inside Kimi K3"), the
Stable LatentMoE passage; P3 = daily-ai-frontier, "苏神复盘 Kimi K3：896 个专家
背后，藏着哪些关键技术取舍？", Merged summary.  The pages leave the expert
intermediate width open; 1024 is used for every K3-shape config here.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens
    H: int            # hidden width (residual stream)
    L: int            # latent width of the routed path
    E: int            # routed experts
    k: int            # experts selected per token
    S: int            # shared experts (always on, full width)
    I: int            # routed expert intermediate width
    Is: int           # shared expert intermediate width
    act: str          # activation / dense-weight storage: "f32" | "bf16"
    w_expert: str     # expert FFN weight storage: "f32" | "bf16" | "f8"
    seed: int
    bias: str = "zero"        # router selection bias: "zero" | "zipf1.1"
    cap: float = 100.0        # SiTU-GLU soft cap
    eps: float = 1e-6         # RMSNorm epsilon
    x_scale: float = 1.0      # multiplies x ~ N(0,1) (stress inputs)
    identity_proj: bool = False   # no latent projections (L == H)
    x_seed: int = -1          # seed of x if it differs from the weights' seed
    a8: bool = False          # W8A8 routed experts (e4m3 activations, 1x128 scales)

    @property
    def tk(self) -> int:
        return self.T * self.k

    def with_T(self, T: int, name: str = None) -> "LayerConfig":
        return replace(self, T=T, name=name or f"{self.name}_T{T}")


K3 = dict(H=7168, L=3584, E=896, k=16, S=2, I=1024, Is=1024)

_LIST = [
    # Tiny fp32 layer: parity only.
    LayerConfig("tiny_f32", T=64, H=256, L=128, E=16, k=2, S=1, I=128, Is=128,
                act="f32", w_expert="f32", seed=0),
    # Same shape, x scaled so that gate/value pre-activations exceed the cap.
    LayerConfig("tiny_situ_stress", T=64, H=256, L=128, E=16, k=2, S=1, I=128,
                Is=128, act="f32", w_expert="f32", seed=2, x_scale=4000.0),
    # Small bf16 / fp8 layers that span several tiles with ragged tails.
    LayerConfig("small_bf16", T=333, H=512, L=256, E=24, k=4, S=2, I=192, Is=128,
                act="bf16", w_expert="bf16", seed=3),
    # small_bf16 with x scaled so that the routed and the shared experts' gate
    # and value pre-activations run far past the cap in the bf16 kernels.
    LayerConfig("small_situ_stress_bf16", T=333, H=512, L=256, E=24, k=4, S=2, I=192, Is=128,
                act="bf16", w_expert="bf16", seed=8, x_scale=4000.0),
    LayerConfig("small_fp8", T=301, H=512, L=256, E=20, k=4, S=2, I=256, Is=128,
                act="bf16", w_expert="f8", seed=4),
    LayerConfig("small_w8a8", T=301, H=512, L=256, E=20, k=4, S=2, I=256, Is=128,
                act="bf16", w_expert="f8", seed=4, a8=True),
    # Whole 256-wide expert matrices (I, L multiples of 256) above 256 tokens,
    # with more experts than the batch fills: the backward's persistent
    # expert-gradient kernels, experts without rows included.
    LayerConfig("small_wide_bf16", T=300, H=512, L=512, E=160, k=2, S=1, I=256, Is=128,
                act="bf16", w_expert="bf16", seed=9),
    LayerConfig("small_identity_bf16", T=130, H=256, L=256, E=12, k=3, S=1, I=128,
                Is=128, act="bf16", w_expert="bf16", seed=5, identity_proj=True),
    # Every expert selected (k == E) and no shared expert.
    LayerConfig("small_full_k", T=77, H=256, L=128, E=8, k=8, S=0, I=128, Is=0,
                act="bf16", w_expert="bf16", seed=6),
    # K3-shape layers.
    LayerConfig("k3_prefill_t2048", T=2048, act="bf16", w_expert="bf16", seed=1, **K3),
    LayerConfig("k3_t8192", T=8192, act="bf16", w_expert="bf16", seed=1, **K3),
    LayerConfig("k3_decode_t64", T=64, act="bf16", w_expert="bf16", seed=1, **K3),
    LayerConfig("k3_zipf_t16384", T=16384, act="bf16", w_expert="bf16", seed=1,
                bias="zipf1.1", **K3),
    LayerConfig("k3_fp8_t8192", T=8192, act="bf16", w_expert="f8", seed=1, **K3),
    LayerConfig("k3_w8a8_t8192", T=8192, act="bf16", w_expert="f8", seed=1, a8=True, **K3),
    LayerConfig("fp8_448x8_l7168_t8192", T=8192, H=7168, L=7168, E=448, k=8, S=2,
                I=1024, Is=1024, act="bf16", w_expert="f8", seed=1),
    # The pages' 448/8 comparison read as a classic MoE with no latent (identity
    # projections): experts on the full 7168-wide hidden state.
    LayerConfig("k3_448x8_identity_t8192", T=8192, H=7168, L=7168, E=448, k=8, S=2,
                I=1024, Is=1024, act="bf16", w_expert="bf16", seed=1, identity_proj=True),
]

CONFIGS = {c.name: c for c in _LIST}


def get_config(name: str) -> LayerConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown layer config {name!r}; known: {sorted(CONFIGS)}")

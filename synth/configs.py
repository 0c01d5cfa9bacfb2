"""Workload shapes of the DiT denoise step.

Five workloads, from a one-block fp32 unit fixture to a Wan-14B-shaped video
DiT.  The video shapes stand in for the Wan2.1 text-to-video models that the
SGLang-Diffusion "Disaggregated Diffusion Pipeline" page runs (section
"Single-Machine Example (Verified)", 832x480, 81 frames); the large image DiT
stands in for the GLM-Image 7B DiT of that page's GLM-Image deployment.

Latents are [C, F, H, W] (batch 1); a patch is (pf, ph, pw); tokens are laid
out over the patch grid (F/pf, H/ph, W/pw) in row-major order.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class DiTConfig:
    name: str
    num_blocks: int
    hidden: int
    heads: int
    head_dim: int
    mlp_hidden: int
    in_channels: int
    patch: tuple          # (pf, ph, pw)
    latent: tuple         # (F, H, W)
    rope: tuple           # (d_f, d_h, d_w), even, summing to head_dim
    ctx_len: int
    text_dim: int
    steps: int
    shift: float
    dtype: str            # "f32" or "bf16"
    freq_dim: int = 256
    rope_theta: float = 10000.0
    ln_eps: float = 1e-6

    # ---- derived sizes -------------------------------------------------
    @property
    def grid(self) -> tuple:
        pf, ph, pw = self.patch
        f, h, w = self.latent
        return (f // pf, h // ph, w // pw)

    @property
    def tokens(self) -> int:
        g = self.grid
        return g[0] * g[1] * g[2]

    @property
    def patch_dim(self) -> int:
        pf, ph, pw = self.patch
        return self.in_channels * pf * ph * pw

    @property
    def latent_shape(self) -> tuple:
        return (self.in_channels,) + tuple(self.latent)

    @property
    def latent_numel(self) -> int:
        c, f, h, w = self.latent_shape
        return c * f * h * w

    @property
    def has_text_proj(self) -> bool:
        return self.text_dim != self.hidden

    def with_(self, **kw) -> "DiTConfig":
        return replace(self, **kw)

    def flops_per_step(self) -> dict:
        """Algorithmic FLOPs of one denoise step (dense, nothing skipped)."""
        S, D, F, L, B, P = (self.tokens, self.hidden, self.mlp_hidden,
                            self.ctx_len, self.num_blocks, self.patch_dim)
        gemm_blk = 2 * S * D * 3 * D + 2 * S * D * D + 2 * S * D * D \
            + 2 * L * D * 2 * D + 2 * S * D * D + 2 * S * D * F * 2
        attn_blk = 4 * S * S * D + 4 * S * L * D
        extra = 2 * S * P * D + 2 * S * D * P
        if self.has_text_proj:
            extra += 2 * L * self.text_dim * D
        tmlp = 2 * (self.freq_dim * D + D * D + D * 6 * D)
        return {"gemm": B * gemm_blk + extra, "attention": B * attn_blk,
                "time": tmlp, "total": B * (gemm_blk + attn_blk) + extra + tmlp}


CONFIGS = {
    "tiny_f32": DiTConfig(
        name="tiny_f32", num_blocks=1, hidden=64, heads=2, head_dim=32, mlp_hidden=256,
        in_channels=4, patch=(1, 2, 2), latent=(1, 8, 8), rope=(0, 16, 16),
        ctx_len=8, text_dim=64, steps=4, shift=1.0, dtype="f32"),
    "image_s_bf16": DiTConfig(
        name="image_s_bf16", num_blocks=12, hidden=768, heads=12, head_dim=64, mlp_hidden=3072,
        in_channels=16, patch=(1, 2, 2), latent=(1, 64, 64), rope=(0, 32, 32),
        ctx_len=256, text_dim=768, steps=20, shift=1.0, dtype="bf16"),
    "wan1p3b_bf16": DiTConfig(
        name="wan1p3b_bf16", num_blocks=30, hidden=1536, heads=12, head_dim=128, mlp_hidden=8960,
        in_channels=16, patch=(1, 2, 2), latent=(21, 60, 104), rope=(44, 42, 42),
        ctx_len=512, text_dim=4096, steps=50, shift=5.0, dtype="bf16"),
    "image_l_bf16": DiTConfig(
        name="image_l_bf16", num_blocks=30, hidden=3584, heads=28, head_dim=128, mlp_hidden=14336,
        in_channels=16, patch=(1, 2, 2), latent=(1, 128, 128), rope=(0, 64, 64),
        ctx_len=1024, text_dim=3584, steps=50, shift=1.0, dtype="bf16"),
    "wan14b_bf16": DiTConfig(
        name="wan14b_bf16", num_blocks=40, hidden=5120, heads=40, head_dim=128, mlp_hidden=13824,
        in_channels=16, patch=(1, 2, 2), latent=(21, 60, 104), rope=(44, 42, 42),
        ctx_len=512, text_dim=4096, steps=50, shift=1.0, dtype="bf16"),
}

# Short aliases in workload order.
ALIASES = {"C1": "tiny_f32", "C2": "image_s_bf16", "C3": "wan1p3b_bf16",
           "C4": "image_l_bf16", "C5": "wan14b_bf16"}


def get_config(name: str) -> DiTConfig:
    name = ALIASES.get(name, name)
    return CONFIGS[name]

"""Seeded parameters and inputs of a DiT workload.

Every tensor is drawn from its own Philox stream (see ``synth.philox``):
weights, biases and modulation tables are N(0, 0.02^2) from seed 0, the
initial latents are N(0, 1) from seed 1, the conditioning tokens are N(0, 1)
from seed 2.  A draw is scaled in float64, rounded to float32 and, for bf16
workloads, rounded again to bfloat16 (round-to-nearest-even) - except the
latents, which stay float32 in every workload.  Values are returned as float32
arrays holding exactly the stored numbers; ``to_device_bits`` gives the
bfloat16 bit patterns for upload.

Weight matrices are row-major [out_features, in_features].  Row blocks:
  qkv_w  rows [0, D) = q, [D, 2D) = k, [2D, 3D) = v; head h of each is rows
         [h*d, (h+1)*d) of that block;
  ckv_w  rows [0, D) = cross k, [D, 2D) = cross v;
  mod_w  rows [j*D, (j+1)*D) give modulation vector j of
         (shift_a, scale_a, gate_a, shift_f, scale_f, gate_f);
  table  [6, D] per-block learned offsets of those six vectors;
  head_table [2, D] = (shift_o, scale_o) offsets of the final layer.
"""
from __future__ import annotations

import numpy as np

from .bf16 import f32_to_bf16_bits, round_to_bf16
from .configs import DiTConfig
from .philox import normals_f32

WEIGHT_SEED = 0
LATENT_SEED = 1
CTX_SEED = 2
WEIGHT_STD = 0.02

GLOBAL_TENSORS = ("t1_w", "t1_b", "t2_w", "t2_b", "mod_w", "mod_b", "txt_w", "txt_b",
                  "pe_w", "pe_b", "head_table", "out_w", "out_b")
BLOCK_TENSORS = ("table", "qkv_w", "qkv_b", "o_w", "o_b", "cq_w", "cq_b", "ckv_w", "ckv_b",
                 "co_w", "co_b", "w1", "b1", "w2", "b2")
_BLOCK_ID_BASE = 256
_BLOCK_ID_STRIDE = 16


def global_shapes(cfg: DiTConfig) -> dict:
    D, P, Z = cfg.hidden, cfg.patch_dim, cfg.freq_dim
    shapes = {
        "t1_w": (D, Z), "t1_b": (D,), "t2_w": (D, D), "t2_b": (D,),
        "mod_w": (6 * D, D), "mod_b": (6 * D,),
        "pe_w": (D, P), "pe_b": (D,), "head_table": (2, D), "out_w": (P, D), "out_b": (P,),
    }
    if cfg.has_text_proj:
        shapes["txt_w"] = (D, cfg.text_dim)
        shapes["txt_b"] = (D,)
    return shapes


def block_shapes(cfg: DiTConfig) -> dict:
    D, F = cfg.hidden, cfg.mlp_hidden
    return {
        "table": (6, D), "qkv_w": (3 * D, D), "qkv_b": (3 * D,), "o_w": (D, D), "o_b": (D,),
        "cq_w": (D, D), "cq_b": (D,), "ckv_w": (2 * D, D), "ckv_b": (2 * D,),
        "co_w": (D, D), "co_b": (D,), "w1": (F, D), "b1": (F,), "w2": (D, F), "b2": (D,),
    }


def tensor_id(name: str, block: int | None = None) -> int:
    if block is None:
        return GLOBAL_TENSORS.index(name)
    return _BLOCK_ID_BASE + _BLOCK_ID_STRIDE * int(block) + BLOCK_TENSORS.index(name)


def _draw(seed: int, tid: int, shape, std: float, dtype: str) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    v = normals_f32(seed, tid, n, std).reshape(shape)
    if dtype == "bf16":
        v = round_to_bf16(v).reshape(shape)
    return v


def make_global_params(cfg: DiTConfig) -> dict:
    return {k: _draw(WEIGHT_SEED, tensor_id(k), s, WEIGHT_STD, cfg.dtype)
            for k, s in global_shapes(cfg).items()}


def make_block_params(cfg: DiTConfig, block: int) -> dict:
    return {k: _draw(WEIGHT_SEED, tensor_id(k, block), s, WEIGHT_STD, cfg.dtype)
            for k, s in block_shapes(cfg).items()}


def make_params(cfg: DiTConfig, blocks=None) -> dict:
    """All parameters: {"global": {...}, "blocks": [ {...}, ... ]}.  ``blocks``
    limits generation to the listed block indices (others are None)."""
    want = range(cfg.num_blocks) if blocks is None else set(blocks)
    return {"global": make_global_params(cfg),
            "blocks": [make_block_params(cfg, b) if b in want else None
                       for b in range(cfg.num_blocks)]}


def make_latents(cfg: DiTConfig, seed: int = LATENT_SEED) -> np.ndarray:
    """Initial latents X0 ~ N(0, 1), float32 [C, F, H, W] in every workload."""
    return _draw(seed, 0, cfg.latent_shape, 1.0, "f32")


def make_ctx(cfg: DiTConfig, seed: int = CTX_SEED, length: int | None = None) -> np.ndarray:
    """Conditioning tokens E ~ N(0, 1), [L, text_dim], in the workload's dtype."""
    L = cfg.ctx_len if length is None else int(length)
    return _draw(seed, 0, (L, cfg.text_dim), 1.0, cfg.dtype)


def to_device_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage representation: float32 as is, or bfloat16 bit patterns (uint16)."""
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    return np.ascontiguousarray(a, dtype=np.float32)

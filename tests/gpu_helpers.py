"""Helpers shared by the GPU parity tests: workload setup through the C ABI
and the oracle side fed the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

from synth import params as SP
from synth.configs import get_config


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (run them with -m gpu)"


def announce(*what):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *what, flush=True, file=sys.stderr)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dev_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def storage_round(a: np.ndarray, dtype: str) -> np.ndarray:
    """The value the device stores for float input a (bf16 RNE or fp32)."""
    a32 = np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        from synth.bf16 import round_to_bf16
        return round_to_bf16(a32).astype(np.float64)
    return a32.astype(np.float64)


def workload(name: str, **over):
    cfg = get_config(name)
    return cfg.with_(**over) if over else cfg


def tolerances(cfg) -> dict:
    """Relative-L2 bars: fp32 workloads 1e-4 everywhere; bf16 workloads 2e-2
    per block (also on the block's update x_out - x_in), 3e-2 on velocity and
    final latents."""
    if cfg.dtype == "f32":
        return {"block": 1e-4, "delta": 1e-4, "velocity": 1e-4, "latents": 1e-4}
    return {"block": 2e-2, "delta": 2e-2, "velocity": 3e-2, "latents": 3e-2}

"""Seeded synthetic inputs for the DiT denoise step.

This package is the only code that both the CPU oracle (``oracle/``) and the
HIP path's harness consume.  It holds no arithmetic of the method itself: it
draws Gaussian numbers from a counter-based generator (Philox-4x32-10 with a
Box-Muller transform), rounds them to the storage precision, and describes the
tensor shapes of each workload.

Modules:
  philox   -- Philox-4x32-10 (Salmon et al., "Parallel random numbers: as easy
              as 1, 2, 3", SC'11) and the Box-Muller normal stream built on it.
  bf16     -- fp32 <-> bfloat16 conversion with round-to-nearest-even.
  configs  -- the workload shapes (tiny fp32 DiT ... Wan-14B-shaped video DiT).
  params   -- per-tensor parameter and input generation for a workload.
"""
from .configs import DiTConfig, CONFIGS, get_config  # noqa: F401

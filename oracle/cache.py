"""Block caching across denoise steps, Cache-DiT style (TEST INFRASTRUCTURE ONLY).

Source.  Page "Disaggregated Diffusion Pipeline", section "GLM-Image
distributed mode": each of its batch-1 denoisers runs with Cache-DiT enabled
and seven knobs, FN = 2, BN = 1, WARMUP = 4, RDT = 0.4, MC = 4,
TAYLORSEER = true, TS_ORDER = 2.  The page gives the knob names and values and
nothing else, so every rule below is a reading of those names (the dual block
cache of the Cache-DiT project, with TaylorSeer extrapolation):

* FN: the first FN blocks run on every step.  Their residual
  P = h_FN - h_0 (the stream after them minus the embedded tokens) is the
  probe that decides whether the step may reuse the cache.
* BN: the last BN blocks run on every step, after the middle ones or after
  the cached stand-in for them.
* The middle blocks [FN, B - BN) are the ones skipped.  A cached step uses
  h = h_FN + M~, where M~ stands in for the middle blocks' residual
  M = h_{B-BN} - h_FN.
* RDT: a step may reuse the cache only while the relative L1 difference
  sum|P - P_ref| / sum|P_ref| is below RDT, where P_ref is the probe of the
  last step that ran every block.
* WARMUP: steps 0 .. WARMUP-1 (counted from the first step of a sampling run)
  always run every block.
* MC: at most MC cached steps in a row; the next one runs every block.
* TAYLORSEER, TS_ORDER: the cached residual is extrapolated in the step
  index by a Taylor series of order TS_ORDER whose derivatives are finite
  differences over the full steps: after a full step at index i whose
  previous full step was at j (gap N = i - j), the factors become
  T_0 = M, T_q = (T_{q-1}(new) - T_{q-1}(old)) / N for q = 1 .. TS_ORDER
  (each only once the older factor exists), and a cached step k steps after
  the last full one uses M~ = sum_q T_q k^q / q!.  Without TaylorSeer,
  M~ = T_0, the last middle residual.
* With classifier-free guidance both branches share one decision: the probe
  difference sums over both sequences; each keeps its own residual cache.

Everything here is float64 numpy built from the block, embedding and head
functions of ``oracle.dit``; a caller may force the per-step decisions (to
follow another implementation's choice when the probe difference lies within
rounding of RDT) and gets back the differences this oracle measured.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import dit as O

F64 = np.float64


@dataclass(frozen=True)
class CacheKnobs:
    fn: int = 2
    bn: int = 1
    warmup: int = 4
    rdt: float = 0.4
    max_consecutive: int = 4
    taylorseer: bool = True
    ts_order: int = 2

    @property
    def order(self) -> int:
        return int(self.ts_order) if self.taylorseer else 0


class CachePolicy:
    """The decision rule, on the step counters alone."""

    def __init__(self, knobs: CacheKnobs):
        self.k = knobs
        self.step = 0          # steps taken
        self.consecutive = 0   # cached steps since the last full one
        self.last_full = -1    # index of the last full step
        self.factors = 0       # Taylor factors in hand (0: nothing cached yet)

    def eligible(self) -> bool:
        """May the current step reuse the cache (its probe then decides)?"""
        return (self.step >= self.k.warmup and self.factors >= 1
                and self.consecutive < self.k.max_consecutive)

    def decide(self, diff: float) -> bool:
        return self.eligible() and diff < self.k.rdt

    def advance(self, hit: bool):
        if hit:
            self.consecutive += 1
        else:
            self.consecutive = 0
            self.last_full = self.step
            self.factors = min(self.factors + 1, self.k.order + 1)
        self.step += 1


def relative_l1(cur, ref) -> float:
    """sum|cur - ref| / sum|ref| (0 when both sums are zero, inf when only the
    reference is)."""
    num = float(np.abs(np.asarray(cur, F64) - np.asarray(ref, F64)).sum())
    den = float(np.abs(np.asarray(ref, F64)).sum())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def taylor_update(factors: list, M, gap: int, order: int) -> list:
    """New factors after a full step with middle residual M, ``gap`` steps
    after the previous full one (``factors`` holds that step's factors; empty
    before the first full step)."""
    new = [np.asarray(M, F64)]
    for q in range(1, order + 1):
        if q - 1 >= len(factors):
            break
        new.append((new[q - 1] - factors[q - 1]) / F64(gap))
    return new


def taylor_predict(factors: list, k: int):
    """sum_q T_q k^q / q! over the factors in hand."""
    out = np.zeros_like(factors[0])
    fact = 1.0
    for q, T in enumerate(factors):
        if q > 0:
            fact *= q
        out = out + T * (F64(k) ** q / fact)
    return out


class CachedDenoiser:
    """The cached sampling loop on the oracle's DiT (one or two sequences)."""

    def __init__(self, params: dict, cfg, knobs: CacheKnobs):
        if not (1 <= knobs.fn and 0 <= knobs.bn and knobs.fn + knobs.bn <= cfg.num_blocks):
            raise ValueError("need 1 <= FN and FN + BN <= number of blocks")
        self.p, self.cfg, self.k = params, cfg, knobs
        self.policy = CachePolicy(knobs)
        self.p_ref = None      # probe of the last full step (stacked sequences)
        self.factors = []      # per sequence: list of Taylor factors

    def _blocks(self, x, c, e, lo, hi):
        pos = O.token_positions(O._grid(self.cfg))
        for b in range(lo, hi):
            p = self.p["blocks"][b]
            x = O.dit_block(x, c, O.block_modulation(e, p["table"]), p, self.cfg, pos)
        return x

    def step(self, X, Es, t: float, sigma: float, sigma_next: float, guidance: float = 1.0,
             force: bool | None = None):
        """One step with the contexts Es (one, or positive then negative).
        Returns (X_next, V, hit, diff); diff is None when the step could not
        reuse the cache (no probe comparison needed)."""
        cfg, g = self.cfg, self.p["global"]
        B, fn, bn = cfg.num_blocks, self.k.fn, self.k.bn
        temb, e = O.time_embedding(t, g, cfg.freq_dim)
        h0 = O.linear(O.patchify(X, cfg.patch), g["pe_w"], g["pe_b"])
        cs = [O.context_projection(E, g, cfg) for E in Es]
        hF = [self._blocks(h0, c, e, 0, fn) for c in cs]
        probe = np.concatenate([h - h0 for h in hF])
        diff = None
        if self.policy.eligible():
            diff = relative_l1(probe, self.p_ref)
        hit = self.policy.decide(diff) if diff is not None else False
        if force is not None:
            if force and not self.policy.eligible():
                raise ValueError("forced a cached step where none is allowed")
            hit = bool(force)
        k = self.policy.step - self.policy.last_full   # steps since the last full one
        hs, new_factors = [], []
        for n, c in enumerate(cs):
            if hit:
                h = hF[n] + taylor_predict(self.factors[n], k)
            else:
                h = self._blocks(hF[n], c, e, fn, B - bn)
                old = self.factors[n] if self.factors else []
                new_factors.append(taylor_update(old, h - hF[n], k, self.k.order))
            hs.append(self._blocks(h, c, e, B - bn, B))
        if not hit:
            self.factors = new_factors
            self.p_ref = probe
        self.policy.advance(hit)
        Vs = [O.unpatchify(O.final_layer(h, temb, g, cfg), cfg.patch,
                           (cfg.in_channels,) + tuple(cfg.latent)) for h in hs]
        V = Vs[0] if len(Vs) == 1 else Vs[1] + float(guidance) * (Vs[0] - Vs[1])
        return O.euler_step(X, V, sigma, sigma_next), V, hit, diff


def sample_cached(X0, Es, params: dict, cfg, knobs: CacheKnobs, sched, guidance: float = 1.0,
                  force=None):
    """Run the cached loop over ``sched`` [(t, sigma, sigma_next), ...].
    Returns a list of (X_after, V, hit, diff) per step; ``force`` optionally
    fixes each step's decision."""
    den = CachedDenoiser(params, cfg, knobs)
    X = np.asarray(X0, F64)
    out = []
    for i, (t, s0, s1) in enumerate(sched):
        X, V, hit, diff = den.step(X, Es, t, s0, s1, guidance,
                                   None if force is None else force[i])
        out.append((X, V, hit, diff))
    return out

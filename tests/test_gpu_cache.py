"""Block caching across denoise steps (dit_denoise_step_cached) against the
oracle's cached loop (oracle/cache.py).  The decision to reuse the cache is
taken on the probe difference, a float computed on both sides in their own
precision; so the oracle follows the GPU's decisions (force=...) and the test
checks (a) every step's velocity and latents against the oracle's, (b) the
measured differences against the oracle's, and (c) that wherever the oracle's
difference is clear of the threshold, its own decision is the GPU's.
Properties that hold at any size are checked at full size: a zero threshold
gives the plain steps bit for bit, and a frozen step (same input every time)
gives the full step's velocity from the cache."""
import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_denoising_amd import binding as B
from diffusion_transformer_denoising_amd.model import DeviceDiT
from oracle.cache import CacheKnobs, CachePolicy, sample_cached
from synth import params as SP
from tests.gpu_helpers import announce, dev_tensor, rel_l2, require_gpu, storage_round, to_np, \
    tolerances, workload

pytestmark = pytest.mark.gpu

PAGES = dict(fn=2, bn=1, warmup=4, rdt=0.4, max_consecutive=4, taylorseer=True, ts_order=2)


def _sched(cfg, n):
    sig = oracle.flow_sigmas(n, cfg.shift)
    return [(float(np.float32(1000.0 * sig[i])), float(np.float32(sig[i])),
             float(np.float32(sig[i + 1]))) for i in range(n)]


def _gpu_run(m, X0, ctx, sched, knobs, ctx_neg=None, g=1.0):
    m.cache_begin(**knobs)
    X = torch.from_numpy(X0).cuda()
    v = torch.empty_like(X)
    out = []
    for t, s0, s1 in sched:
        m.denoise_step_cached(X, ctx, t, s0, s1, ctx_neg=ctx_neg, guidance_scale=g, v_out=v)
        torch.cuda.synchronize()
        st = m.cache_state()
        out.append((to_np(X), to_np(v), bool(st["hit"]), st["diff"]))
    return out


CASES = [
    ("tiny_f32", dict(num_blocks=4), 10,
     dict(fn=1, bn=1, warmup=2, rdt=float("inf"), max_consecutive=2, taylorseer=True, ts_order=2)),
    ("tiny_f32", dict(num_blocks=5), 10,
     dict(fn=2, bn=1, warmup=1, rdt=0.05, max_consecutive=3, taylorseer=False, ts_order=0)),
    ("tiny_f32", dict(num_blocks=5), 14, dict(PAGES, rdt=float("inf"))),
    ("image_s_bf16", dict(latent=(1, 8, 12), num_blocks=5), 12, PAGES),
    ("image_s_bf16", dict(latent=(1, 8, 12), num_blocks=5), 12,
     dict(PAGES, rdt=float("inf"), max_consecutive=3, ts_order=1)),
]


@pytest.mark.parametrize("guided", [False, True])
@pytest.mark.parametrize("name,over,nsteps,knobs", CASES)
def test_cached_loop_matches_oracle(name, over, nsteps, knobs, guided):
    require_gpu()
    cfg = workload(name, **over)
    if guided and cfg.tokens % 8:
        pytest.skip("guided steps need a token count that is a multiple of 8")
    if guided and cfg.dtype == "bf16":
        # The order-2 stand-in k steps after a full step combines the last
        # three middle residuals with weights (1 + k + k^2/2, -(k + k^2), k^2/2),
        # so their bf16 rounding reaches it amplified by the root sum of squares
        # of those weights (3.2 at k = 1, 15 at k = 3, 25 at k = 4), and the
        # guided combination scales branch differences by g = 4 on top.  At
        # k = 4 that exceeds the velocity bar on its own; the guided bf16 runs
        # stop at three cached steps in a row (the fp32 runs take the full
        # four, at fp32 precision).
        knobs = dict(knobs, max_consecutive=min(knobs["max_consecutive"], 3))
    announce("cached loop", name, cfg.tokens, cfg.num_blocks, knobs, "guided" if guided else "")
    prm = SP.make_params(cfg)
    if guided:
        for p in prm["blocks"]:
            p["co_w"] = storage_round(p["co_w"] * 25.0, cfg.dtype)
    X0 = SP.make_latents(cfg)
    E = SP.make_ctx(cfg)
    En = SP.make_ctx(cfg, seed=3) if guided else None
    sched = _sched(cfg, nsteps)
    m = DeviceDiT(cfg, prm, guidance=guided, cache=True)
    got = _gpu_run(m, X0, dev_tensor(E, cfg.dtype), sched, knobs,
                   dev_tensor(En, cfg.dtype) if guided else None, 4.0)
    m.close()
    hits = [h for _, _, h, _ in got]
    ok = CacheKnobs(**knobs)
    ref = sample_cached(X0, [E, En] if guided else [E], prm, cfg, ok, sched, 4.0, force=hits)
    tol = tolerances(cfg)
    # differences: measured on the same steps; decisions: the oracle's own
    # wherever its difference is clear of the threshold
    dtol = (lambda d: 1e-3 * max(d, 1e-2)) if cfg.dtype == "f32" else (lambda d: 0.05 * max(d, 0.1))
    pol = CachePolicy(ok)
    ev, ex = [], []
    for i, ((Xg, Vg, hg, dg), (Xo, Vo, ho, do)) in enumerate(zip(got, ref)):
        assert (dg < 0) == (do is None), i
        if do is not None:
            assert abs(dg - do) <= dtol(do), (i, dg, do)
            if abs(do - ok.rdt) > dtol(do):
                assert pol.decide(do) == hg, (i, do, hg)
        pol.advance(hg)
        ev.append(rel_l2(Vg, Vo))
        ex.append(rel_l2(Xg, Xo))
    print("[cache] hits", hits, "diffs", [round(d, 4) for _, _, _, d in got], flush=True)
    print("[cache] err v", [f"{e:.2e}" for e in ev], "x", [f"{e:.2e}" for e in ex], flush=True)
    assert max(ev) < tol["velocity"] and max(ex) < tol["latents"]
    if knobs["rdt"] == float("inf"):
        assert sum(hits) >= 3


def test_zero_threshold_is_the_plain_step_full_size():
    require_gpu()
    cfg = workload("image_s_bf16")
    announce("cached loop, zero threshold", cfg.name)
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    ctx = dev_tensor(SP.make_ctx(cfg), cfg.dtype)
    sched = _sched(cfg, 6)
    m = DeviceDiT(cfg, prm, cache=True)
    got = _gpu_run(m, X0, ctx, sched, dict(PAGES, warmup=1, rdt=0.0))
    X = torch.from_numpy(X0).cuda()
    v = torch.empty_like(X)
    for i, (t, s0, s1) in enumerate(sched):
        m.denoise_step(X, ctx, t, s0, s1, v_out=v)
        torch.cuda.synchronize()
        assert not got[i][2]
        assert np.array_equal(to_np(X), got[i][0]) and np.array_equal(to_np(v), got[i][1])


@pytest.mark.parametrize("name,over", [("image_s_bf16", {}),
                                       ("wan1p3b_bf16", dict(num_blocks=4))])
def test_frozen_step_reuses_the_full_velocity_full_size(name, over):
    # every step sees the same latents and timestep: the full steps are
    # identical, so every Taylor factor beyond the first is exactly zero and a
    # cached step must give the full step's velocity up to the rounding of
    # h_fn + (h_mid - h_fn) carried through the last block and the head
    require_gpu()
    cfg = workload(name, **over)
    announce("cached loop, frozen step", cfg.name, cfg.num_blocks)
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    ctx = dev_tensor(SP.make_ctx(cfg), cfg.dtype)
    t, s0, _ = _sched(cfg, 10)[3]
    m = DeviceDiT(cfg, prm, cache=True)
    got = _gpu_run(m, X0, ctx, [(t, s0, s0)] * 6, dict(fn=1, bn=1, warmup=2, rdt=0.4,
                                                        max_consecutive=3, taylorseer=True,
                                                        ts_order=2))
    assert [h for _, _, h, _ in got] == [False, False, True, True, True, False]
    V0 = got[0][1]
    for i, (X, V, h, d) in enumerate(got):
        assert np.array_equal(X, X0.astype(np.float64))
        if d >= 0:
            assert d == 0.0
        if h:
            assert rel_l2(V, V0) < 2e-3, i
        else:
            assert np.array_equal(V, V0), i


def test_cached_offload_matches_resident():
    require_gpu()
    cfg = workload("image_s_bf16", latent=(1, 8, 12), num_blocks=5)
    announce("cached loop, offload", cfg.tokens)
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    ctx = dev_tensor(SP.make_ctx(cfg), cfg.dtype)
    sched = _sched(cfg, 10)
    knobs = dict(PAGES, warmup=2, rdt=float("inf"), max_consecutive=2)
    runs = []
    for off in (False, True):
        m = DeviceDiT(cfg, prm, offload=off, cache=True)
        runs.append(_gpu_run(m, X0, ctx, sched, knobs))
        m.close()
    for a, b in zip(*runs):
        assert a[2] == b[2]
        assert rel_l2(b[1], a[1]) < 1e-3 and rel_l2(b[0], a[0]) < 1e-3


def test_cache_call_validation():
    require_gpu()
    cfg = workload("tiny_f32", num_blocks=3)
    announce("cache validation")
    prm = SP.make_params(cfg)
    X = torch.from_numpy(SP.make_latents(cfg)).cuda()
    ctx = dev_tensor(SP.make_ctx(cfg), cfg.dtype)
    plain = DeviceDiT(cfg, prm)
    with pytest.raises(B.DitError) as e:
        plain.cache_begin()
    assert e.value.status == B.DIT_ERR_WORKSPACE
    m = DeviceDiT(cfg, prm, cache=True)
    with pytest.raises(B.DitError) as e:       # no run begun
        m.denoise_step_cached(X, ctx, 500.0, 0.5, 0.45)
    assert e.value.status == B.DIT_ERR_INVALID_ARG
    for bad, status in ((dict(fn=0, bn=1), B.DIT_ERR_SHAPE), (dict(fn=2, bn=2), B.DIT_ERR_SHAPE),
                        (dict(fn=1, bn=0, rdt=-1.0), B.DIT_ERR_INVALID_ARG),
                        (dict(fn=1, bn=0, rdt=float("nan")), B.DIT_ERR_INVALID_ARG),
                        (dict(fn=1, bn=0, warmup=-1), B.DIT_ERR_INVALID_ARG),
                        (dict(fn=1, bn=0, ts_order=3), B.DIT_ERR_UNSUPPORTED)):
        with pytest.raises(B.DitError) as e:
            m.cache_begin(**bad)
        assert e.value.status == status, bad
    m.cache_begin(fn=1, bn=1)
    with pytest.raises(B.DitError) as e:       # guided step on an unguided workspace
        m.denoise_step_cached(X, ctx, 500.0, 0.5, 0.45, ctx_neg=ctx, guidance_scale=4.0)
    assert e.value.status == B.DIT_ERR_WORKSPACE
    m.denoise_step_cached(X, ctx, 500.0, 0.5, 0.45)
    torch.cuda.synchronize()
    assert m.cache_state()["step"] == 1


def test_cached_guided_offloaded_run_matches_oracle():
    # all three options at once: guided steps, block weights streamed from
    # host memory, block caching with the pages' knobs (three cached in a row)
    require_gpu()
    cfg = workload("image_s_bf16", latent=(1, 8, 12), num_blocks=5)
    announce("cached guided offloaded loop", cfg.tokens)
    prm = SP.make_params(cfg)
    for p in prm["blocks"]:
        p["co_w"] = storage_round(p["co_w"] * 25.0, cfg.dtype)
    X0 = SP.make_latents(cfg)
    E, En = SP.make_ctx(cfg), SP.make_ctx(cfg, seed=3)
    knobs = dict(PAGES, rdt=float("inf"), max_consecutive=3)
    sched = _sched(cfg, 10)
    m = DeviceDiT(cfg, prm, guidance=True, offload=True, cache=True)
    got = _gpu_run(m, X0, dev_tensor(E, cfg.dtype), sched, knobs, dev_tensor(En, cfg.dtype), 4.0)
    m.close()
    hits = [h for _, _, h, _ in got]
    assert sum(hits) >= 3
    ref = sample_cached(X0, [E, En], prm, cfg, CacheKnobs(**knobs), sched, 4.0, force=hits)
    tol = tolerances(cfg)
    for (Xg, Vg, _, _), (Xo, Vo, _, _) in zip(got, ref):
        assert rel_l2(Vg, Vo) < tol["velocity"]
        assert rel_l2(Xg, Xo) < tol["latents"]


def test_plain_steps_between_cached_steps_leave_the_run_alone():
    # the cached residuals live in their own part of the workspace: plain and
    # guided-free steps on the same handle between the steps of a cached run
    # must not change the run (bitwise, same launches on the same values)
    require_gpu()
    cfg = workload("image_s_bf16", latent=(1, 8, 12), num_blocks=4)
    announce("cached run with plain steps interleaved", cfg.tokens)
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    ctx = dev_tensor(SP.make_ctx(cfg), cfg.dtype)
    other = dev_tensor(SP.make_ctx(cfg, seed=7), cfg.dtype)
    sched = _sched(cfg, 8)
    knobs = dict(PAGES, warmup=2, rdt=float("inf"), max_consecutive=2)
    m = DeviceDiT(cfg, prm, cache=True)
    ref = _gpu_run(m, X0, ctx, sched, knobs)
    m.cache_begin(**knobs)
    X = torch.from_numpy(X0).cuda()
    Y = torch.from_numpy(X0[::-1].copy()).cuda()
    v = torch.empty_like(X)
    for i, (t, s0, s1) in enumerate(sched):
        m.denoise_step(Y, other, 300.0, 0.3, 0.25)          # unrelated plain step
        m.denoise_step_cached(X, ctx, t, s0, s1, v_out=v)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(X), ref[i][0]) and np.array_equal(to_np(v), ref[i][1]), i
        assert bool(m.cache_state()["hit"]) == ref[i][2]

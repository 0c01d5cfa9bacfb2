"""Pins of the oracle's block cache (oracle/cache.py) against what the knob
definitions and plain arithmetic fix, without reference to the code itself:
decision patterns in closed form, Taylor extrapolation exact on linear data and
off by a known amount on quadratic data, and whole cached loops that must equal
the plain loop bit for bit where the cache can change nothing."""
import numpy as np
import pytest

import oracle
from oracle.cache import CacheKnobs, CachePolicy, relative_l1, sample_cached, taylor_predict, \
    taylor_update
from synth import params as SP
from synth.configs import get_config


def _pattern(knobs, n, diffs=None):
    pol = CachePolicy(knobs)
    out = []
    for i in range(n):
        hit = pol.decide(0.0 if diffs is None else diffs[i])
        pol.advance(hit)
        out.append(hit)
    return out


def test_policy_patterns_closed_form():
    # a probe that never changes: warm-up steps full, then runs of MC cached
    # steps, each followed by one full step
    k = CacheKnobs(warmup=4, max_consecutive=4)
    assert _pattern(k, 20) == [i >= 4 and (i - 4) % 5 != 4 for i in range(20)]
    k = CacheKnobs(warmup=0, max_consecutive=2)
    # step 0 has nothing cached yet
    assert _pattern(k, 10) == [i >= 1 and (i - 1) % 3 != 2 for i in range(10)]
    assert not any(_pattern(CacheKnobs(warmup=0, max_consecutive=0), 10))
    # the threshold is strict, and a large difference forces a full step
    k = CacheKnobs(warmup=1, rdt=0.4, max_consecutive=10)
    assert _pattern(k, 5, [0.0, 0.4, 0.39, 0.5, 0.1]) == [False, False, True, False, True]


def test_relative_l1_by_hand():
    ref = np.array([1.0, -2.0, 3.0])
    cur = np.array([1.5, -2.0, 2.0])
    assert relative_l1(cur, ref) == pytest.approx(1.5 / 6.0, rel=1e-15)
    assert relative_l1(np.zeros(3), np.zeros(3)) == 0.0
    assert relative_l1(np.ones(3), np.zeros(3)) == float("inf")


def test_taylor_linear_is_exact_and_gap_divides():
    # M(s) = a + b s observed at full steps s = 0, 2, 4 (gap 2): order >= 1
    # predicts every later step exactly; order 0 holds the last value
    a, b = np.array([0.5, -1.0]), np.array([0.25, 2.0])
    for order in (1, 2):
        f = []
        for s, gap in ((0, 1), (2, 2), (4, 2)):
            f = taylor_update(f, a + b * s, gap, order)
        assert len(f) == order + 1
        for kk in range(1, 5):
            np.testing.assert_allclose(taylor_predict(f, kk), a + b * (4 + kk), rtol=0, atol=1e-14)
    f = []
    for s in (0, 2):
        f = taylor_update(f, a + b * s, 2, 0)
    np.testing.assert_array_equal(taylor_predict(f, 3), a + b * 2)


def test_taylor_quadratic_error_closed_form():
    # M(s) = c s^2 at full steps 0, 1, 2: the factors are backward differences
    # (3c and 2c), so order 2 predicts 4c + 3c j + c j^2 against the true
    # c (2 + j)^2, an error of -c j; order 1 predicts 4c + 3c j
    c = np.array([1.0, -0.5, 3.0])
    f2, f1 = [], []
    for s in (0, 1, 2):
        f2 = taylor_update(f2, c * s * s, 1, 2)
        f1 = taylor_update(f1, c * s * s, 1, 1)
    for j in (1, 2, 3):
        np.testing.assert_allclose(taylor_predict(f2, j) - c * (2 + j) ** 2, -c * j, atol=1e-13)
        np.testing.assert_allclose(taylor_predict(f1, j), 4 * c + 3 * c * j, atol=1e-13)


# ------------------------------------------------------------------ whole loops
def _setup(num_blocks=4, **over):
    cfg = get_config("tiny_f32").with_(num_blocks=num_blocks, **over)
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg).astype(np.float64)
    E = SP.make_ctx(cfg).astype(np.float64)
    sig = oracle.flow_sigmas(cfg.steps * 2, cfg.shift)
    sched = [(1000.0 * sig[i], sig[i], sig[i + 1]) for i in range(cfg.steps * 2)]
    return cfg, prm, X0, E, sched


def _plain(X0, Es, prm, cfg, sched, g=None):
    X, out = X0, []
    for t, s0, s1 in sched:
        if g is None:
            X, V = oracle.denoise_step(X, Es[0], t, s0, s1, prm, cfg)
        else:
            X, V = oracle.denoise_step_cfg(X, Es[0], Es[1], t, s0, s1, g, prm, cfg)
        out.append((X, V))
    return out


def test_zero_threshold_is_the_plain_loop():
    cfg, prm, X0, E, sched = _setup()
    got = sample_cached(X0, [E], prm, cfg, CacheKnobs(warmup=1, rdt=0.0), sched)
    ref = _plain(X0, [E], prm, cfg, sched)
    assert not any(h for _, _, h, _ in got)
    for (X, V, _, _), (Xr, Vr) in zip(got, ref):
        np.testing.assert_array_equal(X, Xr)
        np.testing.assert_array_equal(V, Vr)


def test_zero_threshold_guided_is_the_plain_guided_loop():
    cfg, prm, X0, E, sched = _setup()
    En = SP.make_ctx(cfg, seed=3).astype(np.float64)
    got = sample_cached(X0, [E, En], prm, cfg, CacheKnobs(warmup=1, rdt=0.0), sched[:4], 4.0)
    ref = _plain(X0, [E, En], prm, cfg, sched[:4], 4.0)
    for (X, V, _, _), (Xr, Vr) in zip(got, ref):
        np.testing.assert_array_equal(X, Xr)
        np.testing.assert_array_equal(V, Vr)


@pytest.mark.parametrize("mode", ["empty-middle", "identity-middle"])
def test_cache_that_cannot_change_anything(mode):
    # no middle blocks, or middle blocks that are the identity (zero gates and
    # zero cross-attention output): the middle residual is exactly zero, so
    # every cached step must equal the full step bit for bit, whatever the
    # threshold lets through
    cfg, prm, X0, E, sched = _setup()
    if mode == "empty-middle":
        knobs = CacheKnobs(fn=2, bn=2, warmup=1, rdt=float("inf"), max_consecutive=3)
    else:
        knobs = CacheKnobs(fn=1, bn=1, warmup=1, rdt=float("inf"), max_consecutive=3)
        # every gate exactly zero for every t (the shared projection's gate rows
        # and every table's gate rows zeroed), and the middle blocks 1 and 2
        # without cross-attention output: those two are exact identities, while
        # blocks 0 and 3 still add their cross-attention
        D = cfg.hidden
        g = prm["global"]
        g["mod_w"], g["mod_b"] = g["mod_w"].copy(), g["mod_b"].copy()
        for r in (2, 5):
            g["mod_w"][r * D:(r + 1) * D] = 0
            g["mod_b"][r * D:(r + 1) * D] = 0
        for b, p in enumerate(prm["blocks"]):
            p["table"] = p["table"].copy()
            p["table"][[2, 5]] = 0
            if b in (1, 2):
                p["co_w"], p["co_b"] = np.zeros_like(p["co_w"]), np.zeros_like(p["co_b"])
    got = sample_cached(X0, [E], prm, cfg, knobs, sched)
    ref = _plain(X0, [E], prm, cfg, sched)
    assert sum(h for _, _, h, _ in got) >= 3
    for (X, V, _, _), (Xr, Vr) in zip(got, ref):
        np.testing.assert_array_equal(X, Xr)
        np.testing.assert_array_equal(V, Vr)


def test_frozen_step_cached_equals_full():
    # the same timestep, sigma_next = sigma (X never moves): every step sees
    # the same input, the probe difference is 0, the middle residual never
    # changes so every derivative factor is 0, and a cached step must give the
    # full step's velocity up to the rounding of h_F + (h_M - h_F)
    cfg, prm, X0, E, sched = _setup()
    t, s0, _ = sched[3]
    frozen = [(t, s0, s0)] * 8
    knobs = CacheKnobs(fn=1, bn=1, warmup=2, rdt=0.4, max_consecutive=3)
    got = sample_cached(X0, [E], prm, cfg, knobs, frozen)
    hits = [h for _, _, h, _ in got]
    assert hits == [False, False, True, True, True, False, True, True]
    assert all(d == 0.0 for _, _, h, d in got if d is not None)
    Vfull = got[0][1]
    for X, V, _, _ in got:
        np.testing.assert_array_equal(X, X0)
        np.testing.assert_allclose(V, Vfull, rtol=0, atol=1e-12 * np.abs(Vfull).max())
    # and a step that reuses a wrong residual would not: a cache built at
    # another timestep is visibly off
    t2 = sched[0][0]
    mixed = [(t2, s0, s0)] * 2 + [(t, s0, s0)]
    got2 = sample_cached(X0, [E], prm, cfg, knobs, mixed, force=[False, False, True])
    assert np.abs(got2[2][1] - Vfull).max() > 1e-6 * np.abs(Vfull).max()


def test_probe_reference_is_the_last_full_step():
    # every eligible step is cached (infinite threshold), at most two in a
    # row: full, full, cached, cached, full, cached, cached, full.  Each
    # measured difference must be that of the step's probe h_FN - h_0 against
    # the probe of the last full step, recomputed here from the step's input
    cfg, prm, X0, E, sched = _setup()
    knobs = CacheKnobs(fn=2, bn=1, warmup=2, rdt=float("inf"), max_consecutive=2)
    got = sample_cached(X0, [E], prm, cfg, knobs, sched[:8])
    assert [h for _, _, h, _ in got] == [False, False, True, True, False, True, True, False]
    g = prm["global"]
    pos = oracle.token_positions(oracle.dit._grid(cfg))
    c = oracle.context_projection(E, g, cfg)

    def probe(X, t):
        _, e = oracle.time_embedding(t, g, cfg.freq_dim)
        h0 = oracle.linear(oracle.patchify(X, cfg.patch), g["pe_w"], g["pe_b"])
        h = h0
        for b in range(2):
            p = prm["blocks"][b]
            h = oracle.dit_block(h, c, oracle.block_modulation(e, p["table"]), p, cfg, pos)
        return h - h0

    inputs = [X0] + [X for X, _, _, _ in got[:-1]]
    probes = [probe(X, sched[i][0]) for i, X in enumerate(inputs)]
    last_full = None
    for i, (_, _, hit, diff) in enumerate(got):
        if hit:
            assert diff == pytest.approx(relative_l1(probes[i], probes[last_full]), rel=1e-12)
            assert diff != pytest.approx(relative_l1(probes[i], probes[0]), rel=1e-6) or last_full == 0
        else:
            last_full = i

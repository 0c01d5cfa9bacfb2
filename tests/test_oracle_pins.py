"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, invariants, special cases that reduce to textbook results, and
brute force on tiny inputs.  Each test names the mistake it is meant to catch.
CPU only."""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


def tiny_cfg(**kw):
    base = dict(hidden=8, heads=2, head_dim=4, mlp_hidden=16, in_channels=2, patch=(1, 2, 2),
                latent=(2, 4, 4), rope=(0, 2, 2), rope_theta=10000.0, ln_eps=1e-6,
                freq_dim=16, text_dim=8)
    base.update(kw)
    return SimpleNamespace(**base)


def rand_block(cfg, std=0.3):
    D, F = cfg.hidden, cfg.mlp_hidden
    shp = {"table": (6, D), "qkv_w": (3 * D, D), "qkv_b": (3 * D,), "o_w": (D, D), "o_b": (D,),
           "cq_w": (D, D), "cq_b": (D,), "ckv_w": (2 * D, D), "ckv_b": (2 * D,),
           "co_w": (D, D), "co_b": (D,), "w1": (F, D), "b1": (F,), "w2": (D, F), "b2": (D,)}
    return {k: RNG.normal(0, std, s) for k, s in shp.items()}


# ----------------------------------------------------------------- schedule
def test_schedule_linear_points():
    # 4 steps with no shift: sigma linear 1 -> 0.
    np.testing.assert_array_equal(oracle.flow_sigmas(4, 1.0), [1.0, 0.75, 0.5, 0.25, 0.0])


def test_schedule_shift_closed_form():
    # shift 5 at s = 1/2: 5 * 0.5 / (1 + 4 * 0.5) = 5/6; endpoints fixed.
    s = oracle.flow_sigmas(2, 5.0)
    assert s[0] == 1.0 and s[2] == 0.0
    assert abs(s[1] - 5.0 / 6.0) < 1e-15
    s50 = oracle.flow_sigmas(50, 5.0)
    assert np.all(np.diff(s50) < 0)          # strictly decreasing
    assert np.all(s50[1:-1] > 1 - np.arange(1, 50) / 50)   # shift > 1 keeps sigma high
    np.testing.assert_allclose(oracle.flow_timesteps(s), 1000 * s)


# ----------------------------------------------------------------- sinusoid
def test_sinusoid_zero_time():
    s = oracle.sinusoid(0.0, 256)
    np.testing.assert_array_equal(s, np.r_[np.ones(128), np.zeros(128)])


def test_sinusoid_frequencies():
    # Frequency j is 10000^(-j/128): at t = (pi/2) * 10000^(j/128) its sine is 1
    # and its cosine 0 (catches a wrong base, exponent or half order).
    for j in (0, 1, 37, 127):
        t = 0.5 * math.pi * 10000.0 ** (j / 128)
        s = oracle.sinusoid(t, 256)
        assert abs(s[128 + j] - 1.0) < 1e-9 and abs(s[j]) < 1e-9


# ----------------------------------------------------------------- softmax / attention
def brute_attention(q, k, v):
    Sq, H, d = q.shape
    Sk = k.shape[0]
    out = np.zeros((Sq, H, d))
    for h in range(H):
        for i in range(Sq):
            sc = [sum(q[i, h, c] * k[j, h, c] for c in range(d)) / math.sqrt(d) for j in range(Sk)]
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            z = sum(w)
            for c in range(d):
                out[i, h, c] = sum(w[j] * v[j, h, c] for j in range(Sk)) / z
    return out


def test_softmax_rows_sum_to_one():
    s = RNG.normal(0, 5, (37, 53))
    p = oracle.softmax_rows(s)
    assert np.all(p > 0)
    assert np.max(np.abs(p.sum(-1) - 1.0)) <= 1e-12


@pytest.mark.parametrize("Sq,Sk,H,d", [(5, 7, 2, 4), (16, 16, 1, 32), (3, 1, 3, 8), (9, 13, 2, 16)])
def test_attention_brute_force(Sq, Sk, H, d):
    q = RNG.normal(0, 1, (Sq, H, d))
    k = RNG.normal(0, 1, (Sk, H, d))
    v = RNG.normal(0, 1, (Sk, H, d))
    np.testing.assert_allclose(oracle.attention(q, k, v), brute_attention(q, k, v),
                               rtol=0, atol=1e-12)


def test_attention_special_cases():
    q = RNG.normal(0, 1, (6, 2, 8))
    k = RNG.normal(0, 1, (1, 2, 8))
    v = RNG.normal(0, 1, (1, 2, 8))
    # one key: output is that key's value
    np.testing.assert_allclose(oracle.attention(q, k, v), np.broadcast_to(v, (6, 2, 8)), atol=1e-15)
    # q = 0: uniform weights, output is the mean value
    k = RNG.normal(0, 1, (11, 2, 8))
    v = RNG.normal(0, 1, (11, 2, 8))
    o = oracle.attention(np.zeros((4, 2, 8)), k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), (4, 2, 8)), atol=1e-14)
    # V == 1: output is 1
    o = oracle.attention(q, k, np.ones_like(v))
    np.testing.assert_allclose(o, 1.0, atol=1e-14)
    # permuting keys together with values changes nothing
    perm = RNG.permutation(11)
    np.testing.assert_allclose(oracle.attention(q, k[perm], v[perm]), oracle.attention(q, k, v),
                               atol=1e-14)


# ----------------------------------------------------------------- layer norm
def test_layer_norm_moments_and_affine_invariance():
    x = RNG.normal(3, 2, (20, 64))
    eps = 1e-6
    y = oracle.layer_norm(x, eps)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(1), 0, atol=1e-13)
    np.testing.assert_allclose(y.var(1), var / (var + eps), rtol=1e-12)
    # per-row affine map x -> a x + b leaves the output unchanged up to eps
    a = RNG.uniform(0.5, 4, (20, 1))
    b = RNG.normal(0, 10, (20, 1))
    np.testing.assert_allclose(oracle.layer_norm(a * x + b, 0.0), oracle.layer_norm(x, 0.0),
                               atol=1e-12)


# ----------------------------------------------------------------- GELU
def test_gelu_tanh():
    z = np.linspace(-8, 8, 4001)
    g = oracle.gelu_tanh(z)
    # odd part: GELU(z) - GELU(-z) = z, GELU(0) = 0
    np.testing.assert_allclose(g - oracle.gelu_tanh(-z), z, atol=1e-14)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    # the tanh form stays within its known 5e-4 of the exact z * Phi(z)
    exact = np.array([0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in z])
    assert np.max(np.abs(g - exact)) < 5e-4


def test_silu_closed_values():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.silu(np.array([1.0])), [1 / (1 + math.exp(-1))], rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.array([-40.0, 40.0])), [0.0, 40.0], atol=1e-15)


# ----------------------------------------------------------------- RoPE
def test_rope_invariants():
    cfg = tiny_cfg(head_dim=12, rope=(4, 4, 4))
    q = RNG.normal(0, 1, (30, 3, 12))
    pos = RNG.integers(0, 50, (30, 3))
    r = oracle.rope_rotate(q, pos, cfg.rope)
    # each channel pair keeps its norm
    np.testing.assert_allclose(np.hypot(r[..., 0::2], r[..., 1::2]),
                               np.hypot(q[..., 0::2], q[..., 1::2]), rtol=1e-13)
    # position 0 is the identity
    np.testing.assert_allclose(oracle.rope_rotate(q, np.zeros_like(pos), cfg.rope), q, atol=0)
    # relative position: shifting every position by a constant keeps q . k
    k = RNG.normal(0, 1, (30, 3, 12))
    shift = np.array([3, 11, 7])
    a = np.einsum("shd,thd->hst", oracle.rope_rotate(q, pos, cfg.rope),
                  oracle.rope_rotate(k, pos, cfg.rope))
    b = np.einsum("shd,thd->hst", oracle.rope_rotate(q, pos + shift, cfg.rope),
                  oracle.rope_rotate(k, pos + shift, cfg.rope))
    np.testing.assert_allclose(a, b, atol=1e-11)


def test_rope_pair_layout_and_frequency():
    # Split (0, 4, 4): channels 0-3 belong to axis h, 4-7 to axis w, pairs are
    # interleaved (2j, 2j+1).  Pair j=1 of a 4-wide segment turns at
    # pos * 10000^(-2/4) = pos / 100 radians; pair 0 at pos radians.
    q = np.zeros((1, 1, 8))
    q[0, 0, 2] = 1.0          # axis h, pair 1, first channel
    q[0, 0, 4] = 1.0          # axis w, pair 0, first channel
    r = oracle.rope_rotate(q, np.array([[9, 100, 2]]), (0, 4, 4))
    assert abs(r[0, 0, 2] - math.cos(1.0)) < 1e-15 and abs(r[0, 0, 3] - math.sin(1.0)) < 1e-15
    assert abs(r[0, 0, 4] - math.cos(2.0)) < 1e-15 and abs(r[0, 0, 5] - math.sin(2.0)) < 1e-15
    assert np.all(r[0, 0, [0, 1, 6, 7]] == 0)
    # f axis is first when present: split (2, 2, 2), position f = pi/2 turns (1, 0) to (0, 1)
    q = np.zeros((1, 1, 6))
    q[0, 0, 0] = 1.0
    r = oracle.rope_rotate(q, np.array([[math.pi / 2, 0, 0]]), (2, 2, 2))
    np.testing.assert_allclose(r[0, 0, :2], [0.0, 1.0], atol=1e-15)


# ----------------------------------------------------------------- patchify
def test_patchify_round_trip_and_indexing():
    X = RNG.normal(0, 1, (3, 4, 6, 8))
    patch = (2, 2, 4)
    u = oracle.patchify(X, patch)
    G = (2, 3, 2)
    assert u.shape == (12, 3 * 16)
    np.testing.assert_array_equal(oracle.unpatchify(u, patch, X.shape), X)
    for _ in range(50):
        c, i, j, k = RNG.integers(0, 3), RNG.integers(0, 2), RNG.integers(0, 2), RNG.integers(0, 4)
        f_, h_, w_ = RNG.integers(0, G[0]), RNG.integers(0, G[1]), RNG.integers(0, G[2])
        n = (f_ * G[1] + h_) * G[2] + w_
        e = ((c * 2 + i) * 2 + j) * 4 + k
        assert u[n, e] == X[c, f_ * 2 + i, h_ * 2 + j, w_ * 4 + k]
    pos = oracle.token_positions(G)
    assert pos.shape == (12, 3) and tuple(pos[7]) == (1, 0, 1)


# ----------------------------------------------------------------- block special cases
def _block_inputs(cfg, S=8, L=3):
    x = RNG.normal(0, 1, (S, cfg.hidden))
    c = RNG.normal(0, 1, (L, cfg.hidden))
    pos = oracle.token_positions((1, 2, 4))[:S]
    return x, c, pos


def test_block_zero_gates_identity():
    cfg = tiny_cfg()
    p = rand_block(cfg)
    p["co_w"][:] = 0
    p["co_b"][:] = 0
    x, c, pos = _block_inputs(cfg)
    mod = RNG.normal(0, 1, (6, cfg.hidden))
    mod[2] = 0
    mod[5] = 0
    out = oracle.dit_block(x, c, mod, p, cfg, pos)
    assert np.array_equal(out, x)           # bitwise


def test_block_cross_attention_single_key():
    # Gates zero, one context token: softmax over one key is 1, so the block
    # adds W_co (W_cv c0 + b_cv) + b_co to every token.
    cfg = tiny_cfg()
    p = rand_block(cfg)
    x, c, pos = _block_inputs(cfg, L=1)
    mod = RNG.normal(0, 1, (6, cfg.hidden))
    mod[2] = 0
    mod[5] = 0
    D = cfg.hidden
    vc = p["ckv_w"][D:] @ c[0] + p["ckv_b"][D:]
    expect = x + (p["co_w"] @ vc + p["co_b"])
    np.testing.assert_allclose(oracle.dit_block(x, c, mod, p, cfg, pos), expect, atol=1e-13)


def test_block_self_attention_constant_values():
    # Value projection zero with bias beta: every attention output is beta, so
    # the self-attention branch adds gate_a * (W_o beta + b_o) whatever q, k,
    # RoPE and the softmax do.
    cfg = tiny_cfg()
    p = rand_block(cfg)
    D = cfg.hidden
    p["qkv_w"][2 * D:] = 0
    beta = RNG.normal(0, 1, D)
    p["qkv_b"][2 * D:] = beta
    p["co_w"][:] = 0
    p["co_b"][:] = 0
    x, c, pos = _block_inputs(cfg)
    mod = RNG.normal(0, 1, (6, D))
    mod[5] = 0
    expect = x + mod[2] * (p["o_w"] @ beta + p["o_b"])
    np.testing.assert_allclose(oracle.dit_block(x, c, mod, p, cfg, pos), expect, atol=1e-13)


def test_block_mlp_closed_form():
    # Attention branches off; W1 = W2 = I, zero biases, scale_f = -1 so the
    # modulated input is shift_f: the block adds gate_f * GELU(shift_f).
    cfg = tiny_cfg(mlp_hidden=8)
    p = rand_block(cfg)
    D = cfg.hidden
    p["co_w"][:] = 0
    p["co_b"][:] = 0
    p["w1"] = np.eye(D)
    p["w2"] = np.eye(D)
    p["b1"][:] = 0
    p["b2"][:] = 0
    x, c, pos = _block_inputs(cfg)
    mod = RNG.normal(0, 1, (6, D))
    mod[2] = 0
    mod[4] = -1.0
    z = mod[3]
    gelu = np.array([0.5 * t * (1 + math.tanh(math.sqrt(2 / math.pi) * (t + 0.044715 * t ** 3)))
                     for t in z])
    np.testing.assert_allclose(oracle.dit_block(x, c, mod, p, cfg, pos), x + mod[5] * gelu,
                               atol=1e-13)


def test_block_token_permutation_equivariance():
    # With every position equal (RoPE the identity) the block is equivariant
    # under token permutations; attention must not depend on token order.
    cfg = tiny_cfg()
    p = rand_block(cfg)
    x, c, _ = _block_inputs(cfg)
    pos = np.zeros((x.shape[0], 3), dtype=int)
    mod = RNG.normal(0, 0.5, (6, cfg.hidden))
    perm = RNG.permutation(x.shape[0])
    a = oracle.dit_block(x, c, mod, p, cfg, pos)[perm]
    b = oracle.dit_block(x[perm], c, mod, p, cfg, pos)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_block_rows_subset_matches_full():
    cfg = tiny_cfg()
    p = rand_block(cfg)
    x, c, pos = _block_inputs(cfg)
    mod = RNG.normal(0, 0.5, (6, cfg.hidden))
    full = oracle.dit_block(x, c, mod, p, cfg, pos)
    rows = np.array([5, 0, 3])
    np.testing.assert_allclose(oracle.dit_block(x, c, mod, p, cfg, pos, rows=rows), full[rows],
                               atol=1e-13)


# ----------------------------------------------------------------- Euler / chain
def test_euler_constant_velocity_chain():
    X0 = RNG.normal(0, 1, (2, 1, 4, 4))
    v = RNG.normal(0, 1, X0.shape)
    sig = oracle.flow_sigmas(7, 3.0)
    X = X0.copy()
    for k in range(7):
        X = oracle.euler_step(X, v, sig[k], sig[k + 1])
        np.testing.assert_allclose(X, X0 + (sig[k + 1] - sig[0]) * v, atol=1e-14)
    np.testing.assert_allclose(X, X0 - v, atol=1e-14)


def test_euler_linear_velocity_product():
    X0 = RNG.normal(0, 1, (5,))
    a = -0.7
    sig = oracle.flow_sigmas(10, 1.0)
    X = X0.copy()
    for k in range(10):
        X = oracle.euler_step(X, a * X, sig[k], sig[k + 1])
    np.testing.assert_allclose(X, X0 * np.prod(1 + a * np.diff(sig)), rtol=1e-14)


def _tiny_params(cfg, blocks=1):
    D, P, Z = cfg.hidden, cfg.in_channels * int(np.prod(cfg.patch)), cfg.freq_dim
    g = {"t1_w": RNG.normal(0, .1, (D, Z)), "t1_b": RNG.normal(0, .1, D),
         "t2_w": RNG.normal(0, .1, (D, D)), "t2_b": RNG.normal(0, .1, D),
         "mod_w": RNG.normal(0, .1, (6 * D, D)), "mod_b": RNG.normal(0, .1, 6 * D),
         "pe_w": RNG.normal(0, .1, (D, P)), "pe_b": RNG.normal(0, .1, D),
         "head_table": RNG.normal(0, .1, (2, D)), "out_w": RNG.normal(0, .1, (P, D)),
         "out_b": RNG.normal(0, .1, P)}
    return {"global": g, "blocks": [rand_block(cfg, 0.1) for _ in range(blocks)]}


def test_forward_constant_head_gives_closed_form_chain():
    # Output projection zero: the velocity is the output bias scattered back to
    # latent layout, constant across steps, so N steps give X0 - V exactly.
    cfg = tiny_cfg()
    params = _tiny_params(cfg, blocks=2)
    params["global"]["out_w"][:] = 0
    X0 = RNG.normal(0, 1, (cfg.in_channels,) + cfg.latent)
    E = RNG.normal(0, 1, (3, cfg.text_dim))
    V = oracle.dit_forward(X0, E, 500.0, params, cfg)
    P = params["global"]["out_b"]
    expect = oracle.unpatchify(np.broadcast_to(P, (8, P.size)), cfg.patch, X0.shape)
    np.testing.assert_allclose(V, expect, atol=1e-15)
    XN = oracle.sample(X0, E, params, cfg, 4, 1.0)
    np.testing.assert_allclose(XN, X0 - expect, atol=1e-14)


def test_forward_identity_blocks_reduce_to_embed_and_head():
    # All block gates and cross outputs zero: the blocks are identities and the
    # velocity tokens are the final layer applied to the patch embedding.
    cfg = tiny_cfg()
    params = _tiny_params(cfg, blocks=3)
    for p in params["blocks"]:
        p["co_w"][:] = 0
        p["co_b"][:] = 0
    # every block's gates exactly zero: the table cancels e on the gate rows
    X0 = RNG.normal(0, 1, (cfg.in_channels,) + cfg.latent)
    E = RNG.normal(0, 1, (3, cfg.text_dim))
    t = 321.0
    _, e = oracle.time_embedding(t, params["global"], cfg.freq_dim)
    for p in params["blocks"]:
        p["table"][2] = -e[2]
        p["table"][5] = -e[5]
    V, u = oracle.dit_forward(X0, E, t, params, cfg, return_tokens=True)
    g = params["global"]
    x = oracle.patchify(X0, cfg.patch) @ g["pe_w"].T + g["pe_b"]
    temb, _ = oracle.time_embedding(t, g, cfg.freq_dim)
    np.testing.assert_allclose(u, oracle.final_layer(x, temb, g, cfg), atol=1e-13)


# ----------------------------------------------------------------- guidance
def _cfg_case(blocks=2):
    cfg = tiny_cfg()
    params = _tiny_params(cfg, blocks=blocks)
    X0 = RNG.normal(0, 1, (cfg.in_channels,) + cfg.latent)
    E = RNG.normal(0, 1, (3, cfg.text_dim))
    En = RNG.normal(0, 1, (3, cfg.text_dim))
    return cfg, params, X0, E, En


def test_cfg_equal_embeddings_is_the_unguided_step():
    # Same embeddings on both sides: the guidance term vanishes for every scale
    # (catches a scale applied to X or to one branch only, or branches that
    # see each other's context).
    cfg, params, X0, E, _ = _cfg_case()
    X1, V1 = oracle.denoise_step(X0, E, 700.0, 0.7, 0.6, params, cfg)
    for g in (0.0, 1.0, 4.0, -2.5):
        X2, V2 = oracle.denoise_step_cfg(X0, E, E, 700.0, 0.7, 0.6, g, params, cfg)
        np.testing.assert_array_equal(V2, V1)
        np.testing.assert_array_equal(X2, X1)


def test_cfg_scales_zero_and_one_select_a_branch():
    # g = 0 is the negative branch exactly, g = 1 the positive one (catches the
    # two embeddings swapped or the difference taken the wrong way round).
    cfg, params, X0, E, En = _cfg_case()
    _, Vp = oracle.denoise_step(X0, E, 400.0, 0.4, 0.3, params, cfg)
    _, Vn = oracle.denoise_step(X0, En, 400.0, 0.4, 0.3, params, cfg)
    assert np.max(np.abs(Vp - Vn)) > 1e-3  # the two contexts do differ
    _, V0 = oracle.denoise_step_cfg(X0, E, En, 400.0, 0.4, 0.3, 0.0, params, cfg)
    np.testing.assert_array_equal(V0, Vn)
    _, V1 = oracle.denoise_step_cfg(X0, E, En, 400.0, 0.4, 0.3, 1.0, params, cfg)
    np.testing.assert_allclose(V1, Vp, rtol=0, atol=1e-14)


def test_cfg_affine_in_the_scale():
    # The guided velocity is affine in g with slope V_pos - V_neg (catches a
    # scale applied twice, squared, or folded into the Euler step size).
    cfg, params, X0, E, En = _cfg_case()
    Vs = {g: oracle.denoise_step_cfg(X0, E, En, 250.0, 0.25, 0.2, g, params, cfg)[1]
          for g in (1.0, 2.0, 3.0)}
    _, Vp = oracle.denoise_step(X0, E, 250.0, 0.25, 0.2, params, cfg)
    _, Vn = oracle.denoise_step(X0, En, 250.0, 0.25, 0.2, params, cfg)
    np.testing.assert_allclose(Vs[3.0] - Vs[2.0], Vs[2.0] - Vs[1.0], atol=1e-13)
    np.testing.assert_allclose(Vs[2.0] - Vs[1.0], Vp - Vn, atol=1e-13)
    X4, V4 = oracle.denoise_step_cfg(X0, E, En, 250.0, 0.25, 0.2, 4.0, params, cfg)
    np.testing.assert_allclose(X4, X0 + (0.2 - 0.25) * V4, atol=1e-15)


# ----------------------------------------------------------------- closed forms through
# the time path, the final layer, the pre-cross-attention LayerNorm, the cross keys,
# the self-attention modulation and the rotary on keys.  Each builds selection or
# identity weights so the expected value is a scalar formula evaluated here with
# ``math``, not by calling the oracle piece under test.
def _silu(z):
    return z / (1.0 + math.exp(-z))


def _alt(n):
    """The +1, -1, +1, ... pattern: mean 0 over an even width, so LayerNorm of
    alpha * alt + beta is alt * alpha / sqrt(alpha^2 + eps) exactly."""
    return np.array([1.0 if e % 2 == 0 else -1.0 for e in range(n)])


def _time_weights(D, Z, gate_rows_zero=False):
    """Selection weights for the time path at t = 0, where the sinusoid is
    ones on its cosine half and zeros on its sine half."""
    half = Z // 2
    t1_w = np.zeros((D, Z))
    for i in range(D):
        t1_w[i, i] = -2.0              # cosine half: contributes -2 at t = 0
        t1_w[i, half + i] = 7.0        # sine half: contributes nothing at t = 0
    t1_b = np.linspace(-1.0, 0.5, D)
    t2_w = 3.0 * np.eye(D)
    t2_b = np.full(D, 0.1)
    mod_w = np.vstack([(k + 1) * np.eye(D) for k in range(6)])
    mod_b = np.concatenate([np.full(D, 0.05 * k) for k in range(6)])
    if gate_rows_zero:
        for k in (2, 5):
            mod_w[k * D:(k + 1) * D] = 0
            mod_b[k * D:(k + 1) * D] = 0
    g = {"t1_w": t1_w, "t1_b": t1_b, "t2_w": t2_w, "t2_b": t2_b, "mod_w": mod_w, "mod_b": mod_b}
    temb = np.array([3.0 * _silu(-2.0 + t1_b[i]) + 0.1 for i in range(D)])
    e = np.array([[(k + 1) * _silu(temb[i]) + 0.05 * k for i in range(D)] for k in range(6)])
    if gate_rows_zero:
        e[2] = 0
        e[5] = 0
    return g, temb, e


def test_time_embedding_closed_form():
    # Catches: SiLU dropped between the two time layers or before the shared
    # modulation projection; bias added after the activation; the sine half
    # first; the six modulation vectors reshaped in the wrong order.
    D, Z = 6, 16
    g, temb, e = _time_weights(D, Z)
    t_o, e_o = oracle.time_embedding(0.0, g, Z)
    np.testing.assert_allclose(t_o, temb, rtol=0, atol=1e-15)
    np.testing.assert_allclose(e_o, e, rtol=0, atol=1e-15)


def test_context_projection_selection():
    # A selection text projection (text width 12 -> hidden 8) copies the
    # chosen columns and adds the bias; equal widths leave the context alone.
    cfg = tiny_cfg(text_dim=12)
    sel = np.array([11, 0, 5, 3, 9, 1, 7, 2])
    w = np.zeros((8, 12))
    w[np.arange(8), sel] = 1.0
    b = np.arange(8) * 0.25
    E = RNG.normal(0, 1, (5, 12))
    c = oracle.context_projection(E, {"txt_w": w, "txt_b": b}, cfg)
    np.testing.assert_array_equal(c, E[:, sel] + b)
    same = tiny_cfg()
    E8 = RNG.normal(0, 1, (5, 8))
    np.testing.assert_array_equal(oracle.context_projection(E8, {"txt_w": None}, same), E8)


def _structured_latents(cfg, alpha, beta):
    """Latents whose every patch vector is alpha_n * alt + beta_n (patch
    (1, 2, 2): patch element e = 4c + 2j + k, and alt flips with k)."""
    C = cfg.in_channels
    F, H, W = cfg.latent
    G = (F, H // 2, W // 2)
    X = np.zeros((C, F, H, W))
    for c in range(C):
        for f in range(F):
            for h in range(H):
                for w in range(W):
                    n = (f * G[1] + h // 2) * G[2] + w // 2
                    X[c, f, h, w] = alpha[n] * (1.0 if w % 2 == 0 else -1.0) + beta[n]
    return X


def test_forward_closed_form_text_projection_cross_value_and_final_layer():
    # One block with both gates zero, so only its ungated cross-attention
    # branch changes the residual.  One context token: the softmax weight is 1
    # and that branch adds W_co (W_cv c0 + b_cv) + b_co = c0 to every token
    # (identity value and output weights).  c0 comes from a selection text
    # projection with a bias, arranged so that c0 = gam * alt + kap.  Patch
    # embedding is the identity, so every token stays of the form
    # a * alt + b and each LayerNorm is a closed form.  The final layer's
    # shift and scale are the head table plus temb from the closed-form time
    # path.  Catches: the text projection skipped or its bias dropped; the
    # final layer's shift and scale swapped, its LayerNorm dropped, the head
    # table or temb ignored; SiLU dropped anywhere in the time path.
    cfg = tiny_cfg(text_dim=12, freq_dim=16)
    D, eps = cfg.hidden, cfg.ln_eps
    alt = _alt(D)
    g, temb, e = _time_weights(D, cfg.freq_dim, gate_rows_zero=True)
    sel = np.array([2, 7, 0, 11, 4, 9, 1, 5])
    txt_w = np.zeros((D, 12))
    txt_w[np.arange(D), sel] = 1.0
    gam1, kap1, gam2, kap2 = 0.4, -0.3, 0.25, 0.6
    E = RNG.normal(0, 1, (1, 12))
    E[0, sel] = gam1 * alt + kap1
    T = np.stack([np.linspace(-0.5, 0.5, D), np.linspace(0.3, -0.2, D)])
    out_b = RNG.normal(0, 0.5, D)
    g.update({"txt_w": txt_w, "txt_b": gam2 * alt + kap2, "pe_w": np.eye(D), "pe_b": np.zeros(D),
              "head_table": T, "out_w": np.eye(D), "out_b": out_b})
    blk = rand_block(cfg)
    blk["table"][:] = 0
    blk["ckv_w"] = np.vstack([RNG.normal(0, 1, (D, D)), np.eye(D)])
    blk["ckv_b"] = np.concatenate([RNG.normal(0, 1, D), np.zeros(D)])
    blk["co_w"] = np.eye(D)
    blk["co_b"] = np.zeros(D)
    params = {"global": g, "blocks": [blk]}
    S = 8
    alpha = np.array([0.5, 1.5, -0.7, 2.0, 0.9, -1.2, 0.3, 1.1])
    beta = np.array([0.2, -1.0, 3.0, 0.0, -0.4, 1.7, 0.8, -2.2])
    X = _structured_latents(cfg, alpha, beta)
    V = oracle.dit_forward(X, E, 0.0, params, cfg)
    gam = gam1 + gam2
    expect = np.zeros_like(X)
    C = cfg.in_channels
    for c in range(C):
        for f in range(cfg.latent[0]):
            for h in range(cfg.latent[1]):
                for w in range(cfg.latent[2]):
                    n = (f * 2 + h // 2) * 2 + w // 2
                    el = 4 * c + 2 * (h % 2) + (w % 2)
                    a = alpha[n] + gam
                    r = a / math.sqrt(a * a + eps)
                    expect[c, f, h, w] = (r * alt[el] * (1.0 + T[1, el] + temb[el])
                                          + T[0, el] + temb[el] + out_b[el])
    assert S == 8
    np.testing.assert_allclose(V, expect, rtol=0, atol=1e-12)


def test_block_two_key_cross_attention_closed_form():
    # Gates zero, so the block adds only its cross branch.  Tokens are
    # alpha_n * alt + beta_n, so the LayerNorm in front of the cross query is
    # r_n * alt.  With identity query, key, value and output weights and the two
    # context rows +a * alt and -a * alt, each head's scores are +-2 r_n a
    # (head width 4, scaled by 1/2), the first key's weight is sigma(4 r_n a),
    # and the block adds tanh(2 r_n a) * a * alt.  Catches: the LayerNorm before
    # cross-attention dropped (the scores would follow alpha_n, not r_n); keys
    # or values built from one context row; the softmax scale missing.
    cfg = tiny_cfg()
    D, eps, a = cfg.hidden, cfg.ln_eps, 0.25
    alt = _alt(D)
    p = rand_block(cfg)
    p["cq_w"], p["cq_b"] = np.eye(D), np.zeros(D)
    p["ckv_w"], p["ckv_b"] = np.vstack([np.eye(D), np.eye(D)]), np.zeros(2 * D)
    p["co_w"], p["co_b"] = np.eye(D), np.zeros(D)
    alpha = np.array([0.3, 2.5, -1.5, 0.8, 4.0, -0.2, 1.3, -3.0])
    beta = RNG.normal(0, 2, 8)
    x = alpha[:, None] * alt + beta[:, None]
    c = np.stack([a * alt, -a * alt])
    mod = RNG.normal(0, 1, (6, D))
    mod[2] = 0
    mod[5] = 0
    pos = oracle.token_positions((1, 2, 4))
    out = oracle.dit_block(x, c, mod, p, cfg, pos)
    expect = np.array([x[n] + math.tanh(2 * (alpha[n] / math.sqrt(alpha[n] ** 2 + eps)) * a)
                       * a * alt for n in range(8)])
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-13)


def test_block_self_attention_modulation_order():
    # scale_a = -1 turns the modulated self-attention input into shift_a for
    # every token, so all values are W_v shift_a + b_v and every attention row
    # returns that vector whatever the queries, keys and RoPE are.  The block
    # then adds gate_a * (W_o (W_v shift_a + b_v) + b_o).  Catches: shift and
    # scale of the self-attention modulation swapped (the input would then
    # follow each token's LayerNorm), or modulation by (scale) instead of
    # (1 + scale).
    cfg = tiny_cfg()
    D = cfg.hidden
    p = rand_block(cfg)
    p["co_w"][:] = 0
    p["co_b"][:] = 0
    x, c, pos = _block_inputs(cfg)
    mod = RNG.normal(0, 1, (6, D))
    mod[1] = -1.0
    mod[5] = 0
    v = p["qkv_w"][2 * D:] @ mod[0] + p["qkv_b"][2 * D:]
    expect = x + mod[2] * (p["o_w"] @ v + p["o_b"])
    np.testing.assert_allclose(oracle.dit_block(x, c, mod, p, cfg, pos), expect, atol=1e-13)


def test_block_rotary_relative_positions():
    # Rotary on both queries and keys makes self-attention scores depend only
    # on position differences, so a common shift of every token's grid position
    # leaves the block output unchanged, while moving tokens relative to each
    # other changes it.  Catches: rotary applied to the queries only or to the
    # keys only, or to neither.
    cfg = tiny_cfg(head_dim=8, heads=1, rope=(2, 2, 4))
    D = cfg.hidden
    p = rand_block(cfg, std=0.8)
    x, c, _ = _block_inputs(cfg)
    pos = oracle.token_positions((2, 2, 2))
    mod = RNG.normal(0, 0.5, (6, D))
    mod[2] = 1.0
    base = oracle.dit_block(x, c, mod, p, cfg, pos)
    shifted = oracle.dit_block(x, c, mod, p, cfg, pos + np.array([3, 5, 11]))
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-12)
    moved = pos.copy()
    moved[:, 2] *= 3
    assert np.max(np.abs(oracle.dit_block(x, c, mod, p, cfg, moved) - base)) > 1e-4

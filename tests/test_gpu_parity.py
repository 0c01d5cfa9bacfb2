"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same
seeded inputs.  Small workloads are compared element by element over every
output; bars are relative L2 (fp32: 1e-4; bf16: 2e-2 per block and on the
block update, 3e-2 on velocity and latents)."""
import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_denoising_amd.model import DeviceDiT, attention, layernorm_modulate
from synth import params as SP
from tests.gpu_helpers import (announce, dev_tensor, rel_l2, require_gpu, storage_round, to_np,
                               tolerances, workload)

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(7)


# ----------------------------------------------------------------- Euler
def test_euler_constant_velocity_chain():
    require_gpu()
    from diffusion_transformer_denoising_amd import binding as B
    announce("euler chain n=1000003")
    n = 1_000_003                              # odd length: vector body + scalar tail
    X0 = RNG.standard_normal(n).astype(np.float32)
    v = RNG.standard_normal(n).astype(np.float32)
    X = torch.from_numpy(X0).cuda()
    vd = torch.from_numpy(v).cuda()
    sig = oracle.flow_sigmas(50, 5.0)
    Xo = X0.astype(np.float64)
    for k in range(50):
        B.dit_euler_step(X.data_ptr(), vd.data_ptr(), n, float(sig[k]), float(sig[k + 1]))
        Xo = oracle.euler_step(Xo, v, sig[k], sig[k + 1])
    torch.cuda.synchronize()
    got = to_np(X)
    # closed form X_N = X_0 - v, and the oracle's step-by-step chain
    assert np.max(np.abs(got - (X0.astype(np.float64) - v))) < 1e-5
    assert rel_l2(got, Xo) < 1e-6


# ----------------------------------------------------------------- time path
@pytest.mark.parametrize("name,over", [
    ("tiny_f32", {}), ("image_s_bf16", {}), ("wan1p3b_bf16", {}),
    # more than 64 blocks: modulation rows past the first 64 per wave
    ("tiny_f32", dict(num_blocks=70)),
    # width 2560 in bf16: weight pieces past the ones read before the input
    ("image_s_bf16", dict(hidden=2560, heads=20, head_dim=128, rope=(0, 64, 64),
                          mlp_hidden=512, text_dim=2560)),
])
def test_time_embedding(name, over):
    require_gpu()
    cfg = workload(name, **{"num_blocks": 2, "latent": (1, 8, 8), **over})
    announce("time_embedding", name, over)
    prm = SP.make_params(cfg)
    m = DeviceDiT(cfg, prm)
    for t in (1000.0, 617.25, 0.0):
        bmod, hmod, temb = m.time_embedding(t)
        torch.cuda.synchronize()
        temb_o, e_o = oracle.time_embedding(t, prm["global"], cfg.freq_dim)
        tol = 1e-5 if cfg.dtype == "f32" else 1e-4
        assert rel_l2(to_np(temb), temb_o) < tol
        for b in range(cfg.num_blocks):
            assert rel_l2(to_np(bmod[b]), oracle.block_modulation(e_o, prm["blocks"][b]["table"])) < tol
        assert rel_l2(to_np(hmod), prm["global"]["head_table"] + temb_o) < tol


# ----------------------------------------------------------------- LayerNorm + modulate
@pytest.mark.parametrize("name", ["tiny_f32", "image_s_bf16", "wan14b_bf16"])
def test_layernorm_modulate(name):
    require_gpu()
    cfg = workload(name)
    announce("layernorm_modulate", name)
    D = cfg.hidden
    rows = 37
    x = (RNG.standard_normal((rows, D)) * 3 + 1).astype(np.float32)
    sh = RNG.standard_normal(D).astype(np.float32)
    sc = RNG.standard_normal(D).astype(np.float32)
    y = torch.empty((rows, D), dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                    device="cuda")
    xd = torch.from_numpy(x).cuda()
    layernorm_modulate(cfg.dtype, cfg.ln_eps, xd, torch.from_numpy(sh).cuda(),
                       torch.from_numpy(sc).cuda(), y)
    y_plain = torch.empty_like(y)
    layernorm_modulate(cfg.dtype, cfg.ln_eps, xd, None, None, y_plain)
    torch.cuda.synchronize()
    tol = 1e-5 if cfg.dtype == "f32" else 5e-3
    assert rel_l2(to_np(y), oracle.modulate(oracle.layer_norm(x, cfg.ln_eps), sh, sc)) < tol
    assert rel_l2(to_np(y_plain), oracle.layer_norm(x, cfg.ln_eps)) < tol


@pytest.mark.parametrize("D", [1000, 1536, 3584])
def test_layernorm_modulate_widths(D):
    # the other row widths of the workloads (1536, 3584) and one whose last
    # 16-byte group per lane is partial (1000 = 250 groups of 4), so the
    # masked reads of x, shift and scale all run
    require_gpu()
    announce("layernorm_modulate width", D)
    rows, eps = 45, 1e-6
    x = (RNG.standard_normal((rows, D)) * 2 - 0.5).astype(np.float32)
    sh = RNG.standard_normal(D).astype(np.float32)
    sc = RNG.standard_normal(D).astype(np.float32)
    y = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    layernorm_modulate("bf16", eps, torch.from_numpy(x).cuda(), torch.from_numpy(sh).cuda(),
                       torch.from_numpy(sc).cuda(), y)
    torch.cuda.synchronize()
    assert rel_l2(to_np(y), oracle.modulate(oracle.layer_norm(x, eps), sh, sc)) < 5e-3


# ----------------------------------------------------------------- attention
def _attention_case(cfg, sq, sk, v_const=None, rng=RNG, pad=0.0):
    H, d, D = cfg.heads, cfg.head_dim, cfg.hidden
    q = storage_round(rng.standard_normal((sq, D)), cfg.dtype)
    k = storage_round(rng.standard_normal((sk, D)), cfg.dtype)
    v = storage_round(rng.standard_normal((sk, D)), cfg.dtype) if v_const is None \
        else np.full((sk, D), v_const)
    ldv = (sk + 63) // 64 * 64
    vt = np.full((D, ldv), pad)
    vt[:, :sk] = v.T
    qd, kd, vtd = dev_tensor(q, cfg.dtype), dev_tensor(k, cfg.dtype), dev_tensor(vt, cfg.dtype)
    od = torch.empty_like(qd)
    attention(cfg.dtype, H, d, qd, kd, vtd, od, sq, sk)
    torch.cuda.synchronize()
    return to_np(od), q, k, v


@pytest.mark.parametrize("name,sq,sk", [
    ("tiny_f32", 16, 16), ("tiny_f32", 16, 8), ("tiny_f32", 130, 77),
    ("image_s_bf16", 1024, 1024), ("image_s_bf16", 1024, 256), ("image_s_bf16", 300, 1000),
    ("image_s_bf16", 1, 1), ("image_s_bf16", 129, 65),
    # small grids split the keys in two ranges: even tile counts, ragged last tile
    ("image_s_bf16", 200, 250), ("image_s_bf16", 100, 2000),
    ("wan1p3b_bf16", 777, 1500), ("wan1p3b_bf16", 256, 512), ("wan1p3b_bf16", 64, 3),
    # head_dim 128 at 40 and 28 heads, key counts under the eight-wave threshold
    ("wan14b_bf16", 1700, 1000), ("wan14b_bf16", 1537, 64), ("image_l_bf16", 2400, 777),
])
def test_attention_parity(name, sq, sk):
    require_gpu()
    cfg = workload(name)
    announce("attention", name, sq, sk)
    o, q, k, v = _attention_case(cfg, sq, sk)
    H, d = cfg.heads, cfg.head_dim
    ref = oracle.attention(q.reshape(sq, H, d), k.reshape(sk, H, d), v.reshape(sk, H, d))
    tol = 1e-5 if cfg.dtype == "f32" else 1e-2
    assert rel_l2(o, ref.reshape(sq, -1)) < tol


@pytest.mark.parametrize("name,sq,sk", [
    ("tiny_f32", 130, 77), ("image_s_bf16", 300, 1000), ("image_s_bf16", 200, 250),
    ("image_s_bf16", 2600, 4100), ("wan1p3b_bf16", 777, 1500), ("wan14b_bf16", 800, 4100),
])
def test_attention_nan_value_padding(name, sq, sk):
    # the caller's V^T columns past the last key (up to the 64-key padded
    # stride) hold NaN: the kernels clear them in the ragged last tile instead
    # of multiplying them by a zero P, so the result is the oracle's
    require_gpu()
    cfg = workload(name)
    announce("attention NaN padding", name, sq, sk)
    o, q, k, v = _attention_case(cfg, sq, sk, pad=np.nan)
    H, d = cfg.heads, cfg.head_dim
    ref = oracle.attention(q.reshape(sq, H, d), k.reshape(sk, H, d), v.reshape(sk, H, d))
    tol = 1e-5 if cfg.dtype == "f32" else 1e-2
    assert np.isfinite(o).all() and rel_l2(o, ref.reshape(sq, -1)) < tol


@pytest.mark.parametrize("name,sk", [("image_s_bf16", 333), ("image_s_bf16", 1000),
                                     ("wan1p3b_bf16", 333)])
def test_attention_constant_values(name, sk):
    # V = 1: every output is exactly a normalised sum of ones, whatever the
    # split of the keys (an odd tile count at 333 keys, an even one at 1000)
    require_gpu()
    cfg = workload(name)
    announce("attention V=1", name, sk)
    o, *_ = _attention_case(cfg, 200, sk, v_const=1.0)
    assert np.max(np.abs(o - 1.0)) <= 2 ** -7


@pytest.mark.parametrize("name,sq,sk", [
    ("image_s_bf16", 200, 2000),     # head_dim 64, two key ranges
    ("image_s_bf16", 2600, 4100),    # head_dim 64, eight waves, one key range
    ("wan1p3b_bf16", 777, 1500),     # head_dim 128, two key ranges
    ("image_l_bf16", 600, 4150),     # head_dim 128, two key ranges
    ("wan14b_bf16", 800, 4100),      # head_dim 128, eight waves, one key range
])
def test_attention_running_max_moves(name, sq, sk):
    # Scores that rise along the keys: a ramp of 40 (natural-log units) on
    # the first channel of every head, so a later key's score exceeds the
    # first tile's maximum by far more than 2^16 in p.  The running maximum
    # then has to move several times, in every key range, with the largest
    # scores in the ragged last tile (its masked keys included).
    require_gpu()
    cfg = workload(name)
    H, d, D = cfg.heads, cfg.head_dim, cfg.hidden
    announce("attention running max", name, sq, sk)
    rng = np.random.default_rng(31)
    q = rng.standard_normal((sq, H, d)) * 0.5
    k = rng.standard_normal((sk, H, d)) * 0.5
    a = 8.0
    q[:, :, 0] += a
    k[:, :, 0] += (40.0 * np.sqrt(d) / a) * np.arange(sk)[:, None] / sk
    q = storage_round(q.reshape(sq, D), cfg.dtype)
    k = storage_round(k.reshape(sk, D), cfg.dtype)
    v = storage_round(rng.standard_normal((sk, D)), cfg.dtype)
    # the inputs do take the rare path: in log2 units, for every query and
    # head, some key beats the first 64 keys' maximum by more than 16
    lg = np.einsum("qhd,khd->qhk", q.reshape(sq, H, d)[:64], k.reshape(sk, H, d)) \
        / np.sqrt(d) / np.log(2.0)
    assert np.all(lg.max(-1) - lg[:, :, :64].max(-1) > 16.0)
    ldv = (sk + 63) // 64 * 64
    vt = np.zeros((D, ldv))
    vt[:, :sk] = v.T
    qd, kd, vtd = dev_tensor(q, cfg.dtype), dev_tensor(k, cfg.dtype), dev_tensor(vt, cfg.dtype)
    od = torch.empty_like(qd)
    attention(cfg.dtype, H, d, qd, kd, vtd, od, sq, sk)
    torch.cuda.synchronize()
    ref = oracle.attention(q.reshape(sq, H, d), k.reshape(sk, H, d), v.reshape(sk, H, d))
    err = rel_l2(to_np(od), ref.reshape(sq, -1))
    print(f"[attention running max] {name} {sq}x{sk}: {err:.2e}", flush=True)
    assert np.isfinite(to_np(od)).all() and err < 1e-2


# ----------------------------------------------------------------- one block, teacher-forced
def _block_case(cfg, stress=False, seed=0, sharp=False):
    rng = np.random.default_rng(100 + seed)
    cfg1 = cfg.with_(num_blocks=1)
    prm = SP.make_params(cfg1)
    if sharp:
        # q and k projection weights scaled to std 1.2/sqrt(D): q, k entries
        # of std ~1.2 and logits of std ~1.5-2, so the softmax is far from
        # uniform and an error in q, k or RoPE shows in the output
        D = cfg.hidden
        for key in ("qkv_w", "cq_w", "ckv_w"):
            w = prm["blocks"][0][key]
            rows = slice(0, 2 * D) if key == "qkv_w" else slice(0, D)
            w[rows] = storage_round(w[rows] * (60.0 / np.sqrt(D)), cfg.dtype)
    m = DeviceDiT(cfg1, prm)
    S, D, L = cfg.tokens, cfg.hidden, cfg.ctx_len
    x = rng.standard_normal((S, D)).astype(np.float32)
    c = storage_round(rng.standard_normal((L, D)), cfg.dtype)
    if stress:
        mod = rng.standard_normal((6, D)).astype(np.float32)
        mod[2] = 1.0
        mod[5] = 1.0
    else:
        _, e = oracle.time_embedding(1000.0 * 0.7, prm["global"], cfg.freq_dim)
        mod = oracle.block_modulation(e, prm["blocks"][0]["table"]).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    m.block_forward(0, xd, dev_tensor(c, cfg.dtype), torch.from_numpy(mod).cuda())
    torch.cuda.synchronize()
    out = to_np(xd)
    pos = oracle.token_positions(cfg.grid)
    ref = oracle.dit_block(x, c, mod, prm["blocks"][0], cfg, pos)
    return out, ref, x.astype(np.float64)


@pytest.mark.parametrize("name", ["tiny_f32", "image_s_bf16"])
@pytest.mark.parametrize("mode", ["time-mod", "stress", "sharp"])
def test_block_parity(name, mode):
    require_gpu()
    cfg = workload(name)
    announce("block", name, mode)
    out, ref, x = _block_case(cfg, stress=mode != "time-mod", sharp=mode == "sharp")
    tol = tolerances(cfg)
    assert rel_l2(out, ref) < tol["block"]
    assert rel_l2(out - x, ref - x) < tol["delta"]


def test_block_zero_gates_identity():
    require_gpu()
    cfg = workload("image_s_bf16", num_blocks=1)
    announce("block zero gates")
    prm = SP.make_params(cfg)
    prm["blocks"][0]["co_w"][:] = 0
    prm["blocks"][0]["co_b"][:] = 0
    m = DeviceDiT(cfg, prm)
    x = RNG.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)
    mod = RNG.standard_normal((6, cfg.hidden)).astype(np.float32)
    mod[2] = 0
    mod[5] = 0
    c = storage_round(RNG.standard_normal((cfg.ctx_len, cfg.hidden)), cfg.dtype)
    xd = torch.from_numpy(x).cuda()
    m.block_forward(0, xd, dev_tensor(c, cfg.dtype), torch.from_numpy(mod).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(xd.cpu().numpy(), x)      # bitwise identity


# ----------------------------------------------------------------- denoise steps and chains
def _chain(cfg, n_steps, check_steps):
    prm = SP.make_params(cfg)
    m = DeviceDiT(cfg, prm)
    X0 = SP.make_latents(cfg)
    E = SP.make_ctx(cfg)
    sig = oracle.flow_sigmas(cfg.steps, cfg.shift)
    X = torch.from_numpy(X0).cuda()
    Ed = dev_tensor(E, cfg.dtype)
    v = torch.empty_like(X)
    Xo = X0.astype(np.float64)
    tol = tolerances(cfg)
    worst = {"velocity": 0.0, "latents": 0.0}
    for k in range(n_steps):
        t = np.float32(1000.0 * sig[k])
        s0, s1 = np.float32(sig[k]), np.float32(sig[k + 1])
        X_before = to_np(X) if k in check_steps else None
        m.denoise_step(X, Ed, float(t), float(s0), float(s1), v_out=v)
        torch.cuda.synchronize()
        if k in check_steps:
            # velocity teacher-forced on the GPU's own latents before the update
            Vo = oracle.dit_forward(X_before, E, float(t), prm, cfg)
            worst["velocity"] = max(worst["velocity"], rel_l2(to_np(v), Vo))
        Xo, _ = oracle.denoise_step(Xo, E, float(t), sig[k], sig[k + 1], prm, cfg)
    worst["latents"] = rel_l2(to_np(X), Xo)
    return worst, tol


def test_denoise_chain_tiny_f32():
    require_gpu()
    cfg = workload("tiny_f32")
    announce("chain tiny_f32 4 steps")
    worst, tol = _chain(cfg, cfg.steps, check_steps=range(cfg.steps))
    assert worst["velocity"] < tol["velocity"], worst
    assert worst["latents"] < tol["latents"], worst


def test_denoise_chain_image_s_bf16():
    require_gpu()
    cfg = workload("image_s_bf16")
    announce("chain image_s_bf16 20 steps")
    worst, tol = _chain(cfg, cfg.steps, check_steps={0, 10, 19})
    assert worst["velocity"] < tol["velocity"], worst
    assert worst["latents"] < tol["latents"], worst


def test_denoise_step_deterministic():
    require_gpu()
    cfg = workload("image_s_bf16")
    announce("determinism image_s_bf16")
    prm = SP.make_params(cfg)
    m = DeviceDiT(cfg, prm)
    X0 = torch.from_numpy(SP.make_latents(cfg)).cuda()
    E = dev_tensor(SP.make_ctx(cfg), cfg.dtype)
    outs = []
    for _ in range(2):
        X = X0.clone()
        m.denoise_step(X, E, 1000.0, 1.0, 0.95)
        torch.cuda.synchronize()
        outs.append(X.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])

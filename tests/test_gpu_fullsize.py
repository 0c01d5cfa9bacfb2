"""Parity at the full workload sizes, in the launch configurations the step
uses, on sampled outputs the float64 oracle computes one by one (every key and
every token still enters the sampled outputs).  Sampled rows always include
the last token, which sits in the ragged last tile."""
import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_denoising_amd.model import DeviceDiT, attention
from synth import params as SP
from tests.gpu_helpers import (announce, dev_tensor, rel_l2, require_gpu, storage_round, to_np,
                               tolerances, workload)

pytestmark = pytest.mark.gpu


def _rows(n, k, seed):
    rng = np.random.default_rng(seed)
    r = np.sort(rng.choice(n - 1, k - 1, replace=False))
    return np.append(r, n - 1)


@pytest.mark.parametrize("name,cross", [("wan1p3b_bf16", False), ("wan1p3b_bf16", True),
                                        ("image_l_bf16", False), ("wan14b_bf16", False)])
def test_attention_full_size(name, cross):
    require_gpu()
    cfg = workload(name)
    S, H, d, D = cfg.tokens, cfg.heads, cfg.head_dim, cfg.hidden
    sk = cfg.ctx_len if cross else S
    announce("attention full", name, "cross" if cross else "self", S, sk)
    g = torch.Generator(device="cuda").manual_seed(11)
    q = torch.randn((S, D), device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn((sk, D), device="cuda", generator=g).to(torch.bfloat16)
    ldv = (sk + 63) // 64 * 64
    vt = torch.zeros((D, ldv), device="cuda", dtype=torch.bfloat16)
    vt[:, :sk] = torch.randn((D, sk), device="cuda", generator=g).to(torch.bfloat16)
    o = torch.empty_like(q)
    attention("bf16", H, d, q, k, vt, o, S, sk)
    torch.cuda.synchronize()
    rows = _rows(S, 48, 5)
    qr = to_np(q[torch.from_numpy(rows).cuda()]).reshape(len(rows), H, d)
    kk = to_np(k).reshape(sk, H, d)
    vv = to_np(vt[:, :sk].t()).reshape(sk, H, d)
    ref = oracle.attention(qr, kk, vv).reshape(len(rows), D)
    got = to_np(o[torch.from_numpy(rows).cuda()])
    assert rel_l2(got, ref) < 1e-2


def _block_full(cfg, rows, mode):
    cfg1 = cfg.with_(num_blocks=1)
    prm = SP.make_params(cfg1)
    rng = np.random.default_rng(21)
    S, D, L = cfg.tokens, cfg.hidden, cfg.ctx_len
    if mode == "sharp":
        for key in ("qkv_w", "cq_w", "ckv_w"):
            w = prm["blocks"][0][key]
            sl = slice(0, 2 * D) if key == "qkv_w" else slice(0, D)
            w[sl] = storage_round(w[sl] * (60.0 / np.sqrt(D)), cfg.dtype)
    m = DeviceDiT(cfg1, prm)
    x = rng.standard_normal((S, D)).astype(np.float32)
    c = storage_round(rng.standard_normal((L, D)), cfg.dtype)
    _, e = oracle.time_embedding(1000.0 * 0.6, prm["global"], cfg.freq_dim)
    mod = oracle.block_modulation(e, prm["blocks"][0]["table"]).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    m.block_forward(0, xd, dev_tensor(c, cfg.dtype), torch.from_numpy(mod).cuda())
    torch.cuda.synchronize()
    got = to_np(xd)[rows]
    ref = oracle.dit_block(x, c, mod, prm["blocks"][0], cfg, oracle.token_positions(cfg.grid),
                           rows=rows)
    return got, ref, x[rows].astype(np.float64)


@pytest.mark.parametrize("name,mode", [("wan1p3b_bf16", "time-mod"), ("wan1p3b_bf16", "sharp"),
                                       ("image_l_bf16", "time-mod"), ("wan14b_bf16", "time-mod"),
                                       ("wan14b_bf16", "sharp")])
def test_block_full_size(name, mode):
    require_gpu()
    cfg = workload(name)
    announce("block full", name, mode)
    rows = _rows(cfg.tokens, 24, 9)
    got, ref, x = _block_full(cfg, rows, mode)
    tol = tolerances(cfg)
    assert rel_l2(got, ref) < tol["block"]
    assert rel_l2(got - x, ref - x) < tol["delta"]


def test_block_zero_gates_identity_wan14b():
    """Wan-14B width at its full 32760 tokens: gates and the cross output
    projection zero make the block the identity, bitwise."""
    require_gpu()
    cfg = workload("wan14b_bf16", num_blocks=1)
    announce("block identity wan14b full")
    prm = SP.make_params(cfg)
    prm["blocks"][0]["co_w"][:] = 0
    prm["blocks"][0]["co_b"][:] = 0
    m = DeviceDiT(cfg, prm)
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((cfg.tokens, cfg.hidden), device="cuda", generator=g)
    x0 = x.clone()
    mod = torch.randn((6, cfg.hidden), device="cuda", generator=g)
    mod[2] = 0
    mod[5] = 0
    c = torch.randn((cfg.ctx_len, cfg.hidden), device="cuda", generator=g).to(torch.bfloat16)
    m.block_forward(0, x, c, mod)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)


@pytest.mark.parametrize("name", ["wan1p3b_bf16", "image_l_bf16"])
def test_denoise_step_one_block_full_size(name):
    """One denoise step with one block at full size (Wan-1.3B: text
    projection 4096 -> 1536; large image DiT: 4096 tokens of width 3584, 1024
    context tokens, no projection), patch embed, block, head, unpatchify +
    Euler; velocity and latents compared at every latent element of sampled
    tokens."""
    require_gpu()
    cfg = workload(name, num_blocks=1)
    announce("step full 1 block", name)
    prm = SP.make_params(cfg)
    m = DeviceDiT(cfg, prm)
    X0 = SP.make_latents(cfg)
    E = SP.make_ctx(cfg)
    sig = oracle.flow_sigmas(cfg.steps, cfg.shift)
    t = float(np.float32(1000.0 * sig[3]))
    X = torch.from_numpy(X0).cuda()
    v = torch.empty_like(X)
    m.denoise_step(X, dev_tensor(E, cfg.dtype), t, float(sig[3]), float(sig[4]), v_out=v)
    torch.cuda.synchronize()
    # oracle at sampled tokens: the block needs every token for K and V
    g = prm["global"]
    temb, e = oracle.time_embedding(t, g, cfg.freq_dim)
    c = oracle.context_projection(E, g, cfg)
    x = oracle.linear(oracle.patchify(X0, cfg.patch), g["pe_w"], g["pe_b"])
    rows = _rows(cfg.tokens, 24, 13)
    xr = oracle.dit_block(x, c, oracle.block_modulation(e, prm["blocks"][0]["table"]),
                          prm["blocks"][0], cfg, oracle.token_positions(cfg.grid), rows=rows)
    u = oracle.final_layer(xr, temb, g, cfg)                # velocity tokens [rows, P]
    vtok = oracle.patchify(to_np(v), cfg.patch)[rows]       # GPU velocity, same tokens
    assert rel_l2(vtok, u) < tolerances(cfg)["velocity"]
    Xtok = oracle.patchify(to_np(X), cfg.patch)[rows]
    X0tok = oracle.patchify(X0, cfg.patch)[rows]
    ref = oracle.euler_step(X0tok, u, sig[3], sig[4])
    assert rel_l2(Xtok, ref) < tolerances(cfg)["latents"]


def test_guided_step_one_block_full_size():
    """The guided step at the Wan-1.3B shape with one block (32760 tokens: the
    transposed values of the two stacked sequences at a padded column stride):
    the guided velocity and latents at sampled tokens against the oracle's two
    branches combined with g = 4.  The cross-attention output projection is
    scaled up so that the branches differ visibly."""
    require_gpu()
    cfg = workload("wan1p3b_bf16", num_blocks=1)
    announce("guided step full wan1p3b 1 block")
    prm = SP.make_params(cfg)
    prm["blocks"][0]["co_w"] = storage_round(prm["blocks"][0]["co_w"] * 25.0, cfg.dtype)
    m = DeviceDiT(cfg, prm, guidance=True)
    X0 = SP.make_latents(cfg)
    E = SP.make_ctx(cfg)
    En = SP.make_ctx(cfg, seed=3)
    sig = oracle.flow_sigmas(cfg.steps, cfg.shift)
    t = float(np.float32(1000.0 * sig[3]))
    X = torch.from_numpy(X0).cuda()
    v = torch.empty_like(X)
    m.denoise_step_cfg(X, dev_tensor(E, cfg.dtype), dev_tensor(En, cfg.dtype), t, float(sig[3]),
                       float(sig[4]), 4.0, v_out=v)
    torch.cuda.synchronize()
    g = prm["global"]
    temb, e = oracle.time_embedding(t, g, cfg.freq_dim)
    x = oracle.linear(oracle.patchify(X0, cfg.patch), g["pe_w"], g["pe_b"])
    rows = _rows(cfg.tokens, 16, 29)
    mod = oracle.block_modulation(e, prm["blocks"][0]["table"])
    pos = oracle.token_positions(cfg.grid)
    u = {}
    for name, ctx in (("pos", E), ("neg", En)):
        c = oracle.context_projection(ctx, g, cfg)
        xr = oracle.dit_block(x, c, mod, prm["blocks"][0], cfg, pos, rows=rows)
        u[name] = oracle.final_layer(xr, temb, g, cfg)
    assert rel_l2(u["pos"] - u["neg"], u["neg"]) > 0.05
    ug = u["neg"] + 4.0 * (u["pos"] - u["neg"])
    vtok = oracle.patchify(to_np(v), cfg.patch)[rows]
    assert rel_l2(vtok, ug) < tolerances(cfg)["velocity"]
    Xtok = oracle.patchify(to_np(X), cfg.patch)[rows]
    ref = oracle.euler_step(oracle.patchify(X0, cfg.patch)[rows], ug, sig[3], sig[4])
    assert rel_l2(Xtok, ref) < tolerances(cfg)["latents"]

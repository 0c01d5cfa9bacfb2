"""Layerwise weight offload (dit_config.offload = 1): the block weights stay in
page-locked host memory and stream block by block through two device slots on
the library's own copy stream.  An offloaded model must give the resident
model's step (the same kernels on the same values; the cross K/V of each block
is computed by that block instead of in one grouped launch) and the oracle's.
Block counts 1, 2 and 5 cover fewer blocks than slots, exactly two, and slots
refilled while the other one runs; two steps in a row check that the second
step's first copies wait for the first step's last blocks.  The weights sit
either in one page-locked buffer per block, in the layout the library moves in
one transfer, or in one buffer per field."""
import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_denoising_amd.model import DeviceDiT
from synth import params as SP
from tests.gpu_helpers import announce, dev_tensor, rel_l2, require_gpu, storage_round, to_np, \
    tolerances, workload

pytestmark = pytest.mark.gpu

CASES = [("tiny_f32", dict(num_blocks=5)), ("image_s_bf16", dict(latent=(1, 8, 12), num_blocks=1)),
         ("image_s_bf16", dict(latent=(1, 8, 12), num_blocks=2)),
         ("image_s_bf16", dict(num_blocks=5))]


def _same(cfg) -> float:
    # resident and offloaded runs of the same kernels on the same values; the
    # only difference is the launch shape of the cross K/V projection
    return 1e-6 if cfg.dtype == "f32" else 1e-3


def _times(cfg):
    sig = oracle.flow_sigmas(cfg.steps, cfg.shift)
    return [(float(np.float32(1000.0 * sig[i])), float(np.float32(sig[i])),
             float(np.float32(sig[i + 1])), sig[i], sig[i + 1]) for i in (1, 2)]


@pytest.mark.parametrize("name,over,packed", [c + (True,) for c in CASES] + [CASES[-1] + (False,)])
def test_offloaded_steps_match_resident_and_oracle(name, over, packed):
    require_gpu()
    cfg = workload(name, **over)
    announce("offload steps", name, cfg.tokens, cfg.num_blocks, "packed" if packed else "fields")
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    E = SP.make_ctx(cfg)
    Ed = dev_tensor(E, cfg.dtype)
    res = {}
    for off in (False, True):
        m = DeviceDiT(cfg, prm, offload=off, pack_offload=packed)
        X = torch.from_numpy(X0).cuda()
        v = torch.empty_like(X)
        vs = []
        for t, s0, s1, _, _ in _times(cfg):       # two steps back to back
            m.denoise_step(X, Ed, t, s0, s1, v_out=v)
            vs.append(v.clone())
        torch.cuda.synchronize()
        res[off] = (to_np(X), [to_np(u) for u in vs])
        m.close()
    bar = _same(cfg)
    assert rel_l2(res[True][0], res[False][0]) < bar
    for a, b in zip(res[True][1], res[False][1]):
        assert rel_l2(a, b) < bar
    # the first step against the oracle
    t, _, _, s0, s1 = _times(cfg)[0]
    tol = tolerances(cfg)
    Vo = oracle.dit_forward(X0, E, t, prm, cfg)
    assert rel_l2(res[True][1][0], Vo) < tol["velocity"]


def test_offloaded_guided_step_matches_resident():
    require_gpu()
    cfg = workload("image_s_bf16", latent=(1, 8, 12), num_blocks=3)
    announce("offload guided step", cfg.tokens, cfg.num_blocks)
    prm = SP.make_params(cfg)
    for p in prm["blocks"]:
        p["co_w"] = storage_round(p["co_w"] * 25.0, cfg.dtype)
    X0 = SP.make_latents(cfg)
    E, En = SP.make_ctx(cfg), SP.make_ctx(cfg, seed=3)
    Ed, End = dev_tensor(E, cfg.dtype), dev_tensor(En, cfg.dtype)
    t, s0, s1, S0, S1 = _times(cfg)[0]
    res = {}
    for off in (False, True):
        m = DeviceDiT(cfg, prm, guidance=True, offload=off)
        X = torch.from_numpy(X0).cuda()
        v = torch.empty_like(X)
        m.denoise_step_cfg(X, Ed, End, t, s0, s1, 4.0, v_out=v)
        torch.cuda.synchronize()
        res[off] = (to_np(X), to_np(v))
        m.close()
    assert rel_l2(res[True][1], res[False][1]) < _same(cfg)
    assert rel_l2(res[True][0], res[False][0]) < _same(cfg)
    Xo, Vo = oracle.denoise_step_cfg(X0, E, En, t, S0, S1, 4.0, prm, cfg)
    tol = tolerances(cfg)
    assert rel_l2(res[True][1], Vo) < tol["velocity"]
    assert rel_l2(res[True][0], Xo) < tol["latents"]


def test_offloaded_block_forward_matches_resident():
    require_gpu()
    cfg = workload("image_s_bf16", latent=(1, 8, 12), num_blocks=3)
    announce("offload block forward", cfg.tokens)
    prm = SP.make_params(cfg)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)
    c = dev_tensor(storage_round(rng.standard_normal((cfg.ctx_len, cfg.hidden)), cfg.dtype),
                   cfg.dtype)
    mod = torch.from_numpy(rng.standard_normal((6, cfg.hidden)).astype(np.float32)).cuda()
    outs = {}
    for off in (False, True):
        m = DeviceDiT(cfg, prm, offload=off)
        xd = torch.from_numpy(x).cuda()
        m.block_forward(2, xd, c, mod)
        bm, hm, te = m.time_embedding(500.0)
        torch.cuda.synchronize()
        outs[off] = (xd.cpu().numpy(), bm.cpu().numpy(), hm.cpu().numpy())
        m.close()
    # same launches on the same values: bitwise equal
    for a, b in zip(outs[True], outs[False]):
        assert np.array_equal(a, b)

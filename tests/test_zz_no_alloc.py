"""dit_block_forward_static, the block call that allocates nothing (its
intermediates live in the library's static device scratch), against
dit_block_forward on a handle with a caller-provided workspace: the same
kernels on the same inputs must give the same block output.  Calls run back to
back on one device, each on a smaller input than the one before, so every call
finds the previous call's contents in the scratch.  The size and flag checks
run on the CPU."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_denoising_amd import binding as B
from diffusion_transformer_denoising_amd.model import DeviceDiT
from synth import params as SP
from synth.configs import CONFIGS
from tests.gpu_helpers import announce, dev_tensor, rel_l2, require_gpu, storage_round, to_np, \
    tolerances, workload


def _fake_block(ptr=4096):
    w = B.dit_block_weights()
    for n in B.BLOCK_FIELDS:
        setattr(w, n, ptr)
    return w


def test_static_block_rejects_before_device_work():
    L = B.lib()
    w = _fake_block()
    # the Wan-14B block needs gigabytes of intermediates: refused by size
    big = B.make_config(CONFIGS["wan14b_bf16"])
    assert L.dit_block_forward_static(ctypes.byref(big), ctypes.byref(w), 4096, 4096, 1, 4096,
                                      None) == B.DIT_ERR_WORKSPACE
    # guided, offloaded or cached configurations are not served by this call
    for flag in ("guidance", "offload", "cache"):
        c = B.make_config(CONFIGS["image_s_bf16"])
        setattr(c, flag, 1)
        assert L.dit_block_forward_static(ctypes.byref(c), ctypes.byref(w), 4096, 4096, 1, 4096,
                                          None) == B.DIT_ERR_UNSUPPORTED, flag
    c = B.make_config(CONFIGS["image_s_bf16"])
    assert L.dit_block_forward_static(ctypes.byref(c), ctypes.byref(w), 4096, 4096, 0, 4096,
                                      None) == B.DIT_ERR_SHAPE
    assert L.dit_block_forward_static(ctypes.byref(c), None, 4096, 4096, 1, 4096,
                                      None) == B.DIT_ERR_INVALID_ARG
    w.w2 = 4098
    assert L.dit_block_forward_static(ctypes.byref(c), ctypes.byref(w), 4096, 4096, 1, 4096,
                                      None) == B.DIT_ERR_INVALID_ARG


# largest first: each call runs on what the previous one left in the scratch
CASES = [("image_s_bf16", {}), ("image_s_bf16", dict(latent=(1, 8, 12))),
         ("tiny_f32", {})]


@pytest.mark.gpu
def test_static_block_matches_the_handle_call():
    require_gpu()
    for name, over in CASES:
        cfg = workload(name, num_blocks=1, **over)
        announce("static block", name, cfg.tokens)
        prm = SP.make_params(cfg)
        m = DeviceDiT(cfg, prm)
        rng = np.random.default_rng(cfg.tokens)
        x = rng.standard_normal((cfg.tokens, cfg.hidden)).astype(np.float32)
        c = storage_round(rng.standard_normal((cfg.ctx_len, cfg.hidden)), cfg.dtype)
        _, e = oracle.time_embedding(600.0, prm["global"], cfg.freq_dim)
        mod = torch.from_numpy(
            oracle.block_modulation(e, prm["blocks"][0]["table"]).astype(np.float32)).cuda()
        cd = dev_tensor(c, cfg.dtype)
        xa = torch.from_numpy(x).cuda()
        m.block_forward(0, xa, cd, mod)
        xb = torch.from_numpy(x).cuda()
        B.dit_block_forward_static(m.c, m._blocks[0], xb.data_ptr(), cd.data_ptr(), cfg.ctx_len,
                                   mod.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        err = rel_l2(to_np(xb), to_np(xa))
        print(f"[static] {name} {cfg.tokens} tokens: rel_l2 to the handle call {err:.2e}, "
              f"bitwise {torch.equal(xa, xb)}", flush=True)
        assert err < tolerances(cfg)["block"]
        assert torch.equal(xa, xb)
        m.close()

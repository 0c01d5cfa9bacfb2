"""Host logic of bench.py, without a GPU: the per-kind work figures the
roofline uses agree with the step's FLOP total written separately in the
workload definitions; the traffic lookup honours the kernel-source hash; and
the one-GPU contract refuses other GPU counts."""
import importlib.util
import json
import os

import pytest

from synth.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


BLOCK_GEMMS = ("gemm_qkv_rope", "gemm_o", "gemm_cross_q", "gemm_cross_o", "gemm_mlp1_gelu",
               "gemm_mlp2")


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_kind_work_sums_to_step_flops(name):
    # one step launches every block kind once per block, the grouped cross K/V
    # once, patch embed and head once, and the text projection when present
    b = _bench()
    cfg = CONFIGS[name]
    w = b.kind_work(cfg)
    assert all(w[k][0] == "flop" for k in BLOCK_GEMMS + b.ATTN_KINDS)
    gemm = cfg.num_blocks * sum(w[k][1] for k in BLOCK_GEMMS) + w["gemm_cross_kv"][1] \
        + w["gemm_patch_embed"][1] + w["gemm_head"][1]
    if cfg.has_text_proj:
        gemm += w["gemm_text_proj"][1]
    attn = cfg.num_blocks * sum(w[k][1] for k in b.ATTN_KINDS)
    ref = cfg.flops_per_step()
    assert gemm == ref["gemm"]
    assert attn == ref["attention"]


def test_kind_work_guided_and_offloaded():
    # the guided step doubles the rows of every block kernel and the head but
    # projects each context once; with offload every block projects its own
    # cross K / V, so one launch carries one block's share
    b = _bench()
    cfg = CONFIGS["image_s_bf16"]
    w1, w2, wo = b.kind_work(cfg), b.kind_work(cfg, nb=2), b.kind_work(cfg, offload=True)
    for k in BLOCK_GEMMS + b.ATTN_KINDS + ("gemm_head", "layernorm_modulate"):
        assert w2[k][1] == 2 * w1[k][1], k
    assert w2["gemm_cross_kv"] == w1["gemm_cross_kv"]
    assert w2["gemm_patch_embed"] == w1["gemm_patch_embed"]
    assert wo["gemm_cross_kv"][1] * cfg.num_blocks == w1["gemm_cross_kv"][1]


def test_measured_traffic_follows_source_hash(tmp_path, monkeypatch):
    b = _bench()
    csrc = tmp_path / "diffusion_transformer_denoising_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = csrc / "k.hip"
    src.write_text("// kernel v1\n")
    rec = {"k@w": {"source": "k.hip", "source_sha256_16": b.source_hash(str(src)),
                   "bytes_per_launch": 1234}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("k", "w") == 1234
    assert b.measured_traffic("k", "other") is None
    src.write_text("// kernel v2\n")  # the kernel changed after the counters were taken
    assert b.measured_traffic("k", "w") is None


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n, capsys):
    b = _bench()
    assert b.main(["--gpus", str(n)]) == 2
    assert "exactly one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name,unit", [("tiny_f32", "steps"), ("image_s_bf16", "steps"),
                                       ("wan1p3b_bf16", "block_prefix"),
                                       ("image_l_bf16", "block"),
                                       ("wan14b_bf16", "block_prefix")])
def test_cpu_sample_plan(name, unit):
    # At 100 GFLOP/s and a 20 s budget: whole steps of the two small
    # workloads fit, one block of the large image DiT fits, and the video
    # shapes (a step is hours, a block minutes) get one block on a prefix of
    # whole grid rows that is the largest one inside the budget.
    b = _bench()
    cfg = CONFIGS[name]
    rate, budget = 1e11, 20.0
    got, n = b.plan_cpu_sample(cfg, budget, rate)
    assert got == unit
    if unit == "block":
        assert n == cfg.tokens
    if unit == "block_prefix":
        row = cfg.grid[2]
        assert n % row == 0 and row <= n < cfg.tokens
        assert b.block_flops(cfg, n) / rate <= budget
        assert b.block_flops(cfg, n + row) / rate > budget


def test_block_flops_sum_to_step():
    # B blocks at the full token count plus the patch, head, text and time
    # terms make the step's FLOP total
    b = _bench()
    for cfg in CONFIGS.values():
        f = cfg.flops_per_step()
        extra = 2 * cfg.tokens * cfg.patch_dim * cfg.hidden * 2 + f["time"]
        if cfg.has_text_proj:
            extra += 2 * cfg.ctx_len * cfg.text_dim * cfg.hidden
        assert cfg.num_blocks * b.block_flops(cfg, cfg.tokens) + extra == f["total"]


def test_cpu_baseline_block_unit():
    # A zero budget forces the smallest sample: one block on one grid row.
    b = _bench()
    from synth import params as SP
    cfg = CONFIGS["tiny_f32"]
    prm = SP.make_params(cfg)
    r = b.cpu_baseline(cfg, prm, SP.make_latents(cfg), SP.make_ctx(cfg), budget_s=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s" and r["value"] > 0
    assert r["sample_unit"] == "block_prefix" and r["sample_tokens"] == cfg.grid[2]
    assert f"the first {cfg.grid[2]}" in r["sample"] and r["cores"] >= 1

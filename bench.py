"""Benchmark: denoise steps per second of one DiT denoising step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--guidance G] [--offload] [--cache] [--no-cpu-baseline]
                    [--no-other-configs] [--calibrate-copy]

The default workload is the Wan-14B-shaped video DiT (40 blocks, hidden 5120,
40 heads x 128, MLP 13824, 32760 tokens, text 512 x 4096 projected to 5120),
the largest of the five workloads and the one that fills one GPU.

A step is one call of dit_denoise_step: time embedding, context projection,
patch embedding, every DiT block (LayerNorm+adaLN, QKV projection, RoPE,
self-attention, gated output projection, cross-attention, GELU MLP) and the
head, then the fused unpatchify + Euler update.  Inputs and weights are seeded
synthetic data already resident in HBM when timing starts; the timestep and
sigmas cycle through the workload's flow schedule.  With --guidance G a step is
one call of dit_denoise_step_cfg instead: both branches (positive context and
a second, negative one) as one batch of two sequences, guidance scale G.  With
--offload the block weights live in page-locked host memory and every step
streams them block by block into two HBM slots (layerwise offload); the line
then also reports the streamed bytes per step and their rate.  With --cache the
steps go through dit_denoise_step_cached with the Cache-DiT knobs of the pages'
deployment (FN 2, BN 1, WARMUP 4, RDT 0.4, MC 4, TaylorSeer order 2): the timed
steps are whole sampling runs of the workload's schedule, each begun afresh,
and the line reports how many steps reused the cache.

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value          whole-job steps/s (K timed steps, bracketed by
                 torch.cuda.synchronize(), HIP events on the launch stream)
  roofline       the kernel kind with the largest share of step time: its
                 algorithmic FLOPs (or bytes) per launch over its average launch
                 duration, from HIP events attached to every launch (recorded at
                 the kernel's own dispatch and completion) during a second pass
                 over the same K steps, against the MI355X peak;
                 traffic = HBM bytes per launch from committed rocprofv3
                 FETCH_SIZE / WRITE_SIZE runs (profiles/traffic.json), or null
  attention / gemm   TFLOP/s and fraction of the bf16 MFMA peak, same events
  cpu_baseline   the CPU oracle timed on a bounded sample of the same workload:
                 whole steps where one fits the budget, else one block, else one
                 block on a prefix of the token sequence (whole grid rows) at the
                 full widths; a block sample is converted to steps/s through its
                 FLOP rate over the step's FLOPs
  per_config     seconds per step of every other workload, timed after the main
                 one in the same process (the two smallest: median over five
                 whole sampling runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "denoise steps/sec per config + attention/GEMM TFLOP/s as % bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
# v_exp_f32 issues once per ~8.5 cycles per wave64 per SIMD (measured), i.e.
# 64 / 8.5 results per clock per SIMD; 4 SIMDs x 256 CUs at 2.4 GHz
PEAK_EXP_PER_S = 64 / 8.5 * 4 * 256 * 2.4e9
DEFAULT_WORKLOAD = "wan14b_bf16"
# Cache-DiT knobs of the pages' GLM-Image denoisers (page "Disaggregated
# Diffusion Pipeline", section "GLM-Image distributed mode")
CACHE_KNOBS = dict(fn=2, bn=1, warmup=4, rdt=0.4, max_consecutive=4, taylorseer=True, ts_order=2)

GEMM_KINDS = ("gemm_qkv_rope", "gemm_o", "gemm_cross_q", "gemm_cross_kv", "gemm_cross_o",
              "gemm_mlp1_gelu", "gemm_mlp2", "gemm_text_proj", "gemm_patch_embed", "gemm_head")
ATTN_KINDS = ("attention_self", "attention_cross")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kind_work(cfg, nb: int = 1, offload: bool = False) -> dict:
    """Algorithmic work per launch of each kernel kind: ("flop", n) for matrix-core
    kernels, ("byte", n) for bandwidth-bound ones (minimum HBM traffic).  nb = 2
    is the guided step: the block kernels and the head process two stacked
    sequences per launch, the context kernels run once per context.  With
    offload each block projects its own cross K / V."""
    S, D, F, L, P = cfg.tokens, cfg.hidden, cfg.mlp_hidden, cfg.ctx_len, cfg.patch_dim
    R = nb * S
    es = 2 if cfg.dtype == "bf16" else 4
    n_lat = cfg.latent_numel
    return {
        "gemm_qkv_rope": ("flop", 2 * R * D * 3 * D),
        "gemm_o": ("flop", 2 * R * D * D),
        "gemm_cross_q": ("flop", 2 * R * D * D),
        # one grouped launch per context computes every block's cross K / V^T
        "gemm_cross_kv": ("flop", (1 if offload else cfg.num_blocks) * 2 * L * D * 2 * D),
        "gemm_cross_o": ("flop", 2 * R * D * D),
        "gemm_mlp1_gelu": ("flop", 2 * R * D * F),
        "gemm_mlp2": ("flop", 2 * R * F * D),
        "gemm_text_proj": ("flop", 2 * L * cfg.text_dim * D),
        "gemm_patch_embed": ("flop", 2 * S * P * D),
        "gemm_head": ("flop", 2 * R * D * P),
        "attention_self": ("flop", nb * 4 * S * S * D),
        "attention_cross": ("flop", nb * 4 * S * L * D),
        # read the fp32 row, write the normalised row
        "layernorm_modulate": ("byte", R * D * (4 + es)),
        "patchify": ("byte", n_lat * (4 + es)),
        # read the velocity tokens (of each branch), read-modify-write the latents
        "unpatchify_euler": ("byte", n_lat * 4 * (nb + 2)),
        # three GEMV launches per step; the per-launch figure is their mean
        "time_embedding": ("byte", es * (cfg.freq_dim * D + D * D + 6 * D * D) // 3),
        # block caching, float buffers of R * D elements: the probe reads x, h_0
        # and the reference and writes the probe and h_fn; with three Taylor
        # factors in hand the stand-in reads x and the factors and writes x, and
        # the update reads x, h_fn and the factors and writes the factors
        "cache_probe": ("byte", 20 * R * D),
        "cache_apply": ("byte", 20 * R * D),
        "cache_update": ("byte", 32 * R * D),
    }


def exp_work(cfg, nb: int = 1) -> dict:
    """Exponentials per launch of the attention kinds: one per (query, key,
    head) score of the softmax."""
    S, L, H = cfg.tokens, cfg.ctx_len, cfg.heads
    return {"attention_self": nb * H * S * S, "attention_cross": nb * H * S * L}


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel_kind}@{workload}")
    if not rec:
        return None
    src = os.path.join(ROOT, "diffusion_transformer_denoising_amd", "csrc", rec["source"])
    if not os.path.exists(src) or source_hash(src) != rec["source_sha256_16"]:
        return None
    return rec["bytes_per_launch"]


def block_flops(cfg, S: int) -> int:
    """Algorithmic FLOPs of one DiT block over S tokens at the workload's widths
    (projections, the cross K / V of the context, both attentions)."""
    D, F, L = cfg.hidden, cfg.mlp_hidden, cfg.ctx_len
    return 12 * S * D * D + 4 * L * D * D + 4 * S * D * F + 4 * S * S * D + 4 * S * L * D


def plan_cpu_sample(cfg, budget_s: float, rate_flops: float):
    """Which oracle unit fits the budget at an assumed host FLOP rate:
    ("steps", None) when one whole step does, else ("block", S) when one whole
    block does, else ("block_prefix", n): one block on the first n tokens, n a
    whole number of grid rows (at least one)."""
    if cfg.flops_per_step()["total"] / rate_flops <= budget_s:
        return ("steps", None)
    S = cfg.tokens
    if block_flops(cfg, S) / rate_flops <= budget_s:
        return ("block", S)
    row = cfg.grid[2]
    n = row
    while n + row < S and block_flops(cfg, n + row) / rate_flops <= budget_s:
        n += row
    return ("block_prefix", n)


def host_matmul_rate() -> float:
    """float64 matmul FLOP/s of the host (numpy's BLAS), for sizing the sample."""
    a = np.random.default_rng(0).standard_normal((2048, 2048))
    a @ a
    t0 = time.perf_counter()
    for _ in range(3):
        a @ a
    return 3 * 2 * 2048 ** 3 / (time.perf_counter() - t0)


def _host_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, prm, X0, E, budget_s: float = 20.0, E_neg=None, g=None) -> dict:
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload (see plan_cpu_sample); with E_neg and g, the oracle's
    guided step."""
    import oracle
    cores = _host_threads()
    step_flops = cfg.flops_per_step()["total"] * (2 if E_neg is not None else 1)
    rate = host_matmul_rate()
    # the oracle's block reaches ~18 % of the host's large-matmul rate at the
    # Wan-14B width (its attention is elementwise numpy over S x S scores), so
    # the sample is sized at 15 % of it
    unit, n = plan_cpu_sample(cfg, budget_s, 0.15 * rate / (2 if E_neg is not None else 1))
    sig = oracle.flow_sigmas(cfg.steps, cfg.shift)
    if unit == "steps":
        X = X0.astype(np.float64)
        done = 0
        t0 = time.perf_counter()
        while done < cfg.steps:
            t = float(np.float32(1000.0 * sig[done]))
            if E_neg is None:
                X, _ = oracle.denoise_step(X, E, t, sig[done], sig[done + 1], prm, cfg)
            else:
                X, _ = oracle.denoise_step_cfg(X, E, E_neg, t, sig[done], sig[done + 1], g, prm,
                                               cfg)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": done / dt, "unit": "steps/s", "cores": cores, "kind": "oracle",
                "sample": f"first {done} of the {cfg.steps} "
                          f"{'guided ' if E_neg is not None else ''}denoise steps of {cfg.name}, "
                          f"float64 numpy oracle, {dt:.1f} s"}
    # one block (block 0, its own weights) on the first n tokens of the step's
    # embedded latents, with the step's first modulation and projected context;
    # the guided step runs it for both contexts
    g_ = prm["global"]
    t = float(np.float32(1000.0 * sig[0]))
    _, e = oracle.time_embedding(t, g_, cfg.freq_dim)
    p0 = prm["blocks"][0]
    mod = oracle.block_modulation(e, p0["table"])
    x = oracle.linear(oracle.patchify(X0, cfg.patch)[:n], g_["pe_w"], g_["pe_b"])
    pos = oracle.token_positions(cfg.grid)[:n]
    ctxs = [E] if E_neg is None else [E, E_neg]
    cs = [oracle.context_projection(c, g_, cfg) for c in ctxs]
    t0 = time.perf_counter()
    for c in cs:
        oracle.dit_block(x, c, mod, p0, cfg, pos)
    dt = time.perf_counter() - t0
    flops = len(cs) * block_flops(cfg, n)
    what = "all" if n == cfg.tokens else f"the first {n} (whole grid rows)"
    return {"value": flops / dt / step_flops, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"one DiT block of {cfg.name} (block 0, hidden {cfg.hidden}, "
                      f"{cfg.heads} heads, MLP {cfg.mlp_hidden}, context {cfg.ctx_len}) on {what} "
                      f"of its {cfg.tokens} tokens{' for both contexts' if len(cs) > 1 else ''}, "
                      f"float64 numpy oracle: {flops / 1e12:.3f} TFLOP in {dt:.1f} s = "
                      f"{flops / dt / 1e9:.1f} GFLOP/s; steps/s = that rate over the "
                      f"{step_flops / 1e12:.2f} TFLOP of one step",
            "sample_unit": unit, "sample_tokens": n, "block_seconds": dt,
            "host_matmul_gflops": round(rate / 1e9, 1)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--guidance", type=float, default=None,
                    help="time the guided step (classifier-free guidance) at this scale")
    ap.add_argument("--offload", action="store_true",
                    help="layerwise offload: block weights streamed from pinned host memory")
    ap.add_argument("--cache", action="store_true",
                    help="block caching across steps with the pages' Cache-DiT knobs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the seconds-per-step lines of the other workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (the known-size kernel "
                         "that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "the denoise step is sized for one GPU's share and nothing here uses a second.",
              file=sys.stderr)
        return 2

    import torch
    if args.calibrate_copy:
        n = 1 << 28  # float32 elements: 1 GiB read + 1 GiB written per copy
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 5}))
        return 0
    from diffusion_transformer_denoising_amd import binding as B
    from diffusion_transformer_denoising_amd.model import DeviceDiT, torch_dtype
    from synth import params as SP
    from synth.configs import get_config

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    cfg = get_config(args.workload)
    log(f"[bench] workload {cfg.name}: S={cfg.tokens} D={cfg.hidden} B={cfg.num_blocks} "
        f"H={cfg.heads}x{cfg.head_dim} F={cfg.mlp_hidden} L={cfg.ctx_len}")
    t0 = time.perf_counter()
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    E = SP.make_ctx(cfg)
    guided = args.guidance is not None
    nb = 2 if guided else 1
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")
    m = DeviceDiT(cfg, prm, guidance=guided, offload=args.offload, cache=args.cache)
    X = torch.from_numpy(X0).cuda()
    Ed = torch.from_numpy(E).cuda().to(torch_dtype(cfg))
    # the negative context of a guided step: its own seed (3)
    End = torch.from_numpy(SP.make_ctx(cfg, seed=3)).cuda().to(torch_dtype(cfg)) if guided else None
    sig = B.dit_flow_sigmas(cfg.steps, cfg.shift)
    sched = [(float(np.float32(1000.0 * sig[k])), float(sig[k]), float(sig[k + 1]))
             for k in range(cfg.steps)]

    hits = [0]

    def run(n, k0=0):
        for i in range(n):
            k = (k0 + i) % cfg.steps
            t, s0, s1 = sched[k]
            if args.cache:
                if k == 0:
                    m.cache_begin(**CACHE_KNOBS)
                m.denoise_step_cached(X, Ed, t, s0, s1, ctx_neg=End,
                                      guidance_scale=args.guidance if guided else 1.0)
                hits[0] += m.cache_state()["hit"]
            elif guided:
                m.denoise_step_cfg(X, Ed, End, t, s0, s1, args.guidance)
            else:
                m.denoise_step(X, Ed, t, s0, s1)

    run(args.warmup)
    torch.cuda.synchronize()
    hits[0] = 0
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    run(args.steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / args.steps
    timed_hits = hits[0]
    log(f"[bench] {args.steps} steps: {ms:.2f} ms (events), {wall * 1e3:.2f} ms (wall)")

    # second pass over the same K steps with events attached to every launch
    B.dit_profile_enable(m.handle, True)
    run(args.steps)
    torch.cuda.synchronize()
    B.dit_profile_enable(m.handle, False)
    prof = B.profile_summary(m.handle)
    work = kind_work(cfg, nb, args.offload)
    kernels = {}
    for name, (n, tms) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        unit, amount = work.get(name, ("flop", 0))
        avg_s = tms / n / 1e3
        rate = amount / avg_s if avg_s > 0 else 0.0
        kernels[name] = {"launches": n, "avg_us": round(avg_s * 1e6, 3),
                         "share": round(tms / sum(v[1] for v in prof.values()), 4),
                         ("tflops" if unit == "flop" else "gbs"):
                             round(rate / (1e12 if unit == "flop" else 1e9), 2)}
        if name in ATTN_KINDS and avg_s > 0:
            ex = exp_work(cfg, nb)[name] / avg_s
            kernels[name]["exp_per_s"] = round(ex / 1e12, 3)   # 10^12 exponentials / s
            kernels[name]["exp_frac"] = round(ex / PEAK_EXP_PER_S, 4)
        log(f"[bench]   {name:20s} {n:6d} x {avg_s * 1e6:9.2f} us  "
            f"{rate / (1e12 if unit == 'flop' else 1e9):9.2f} {'TFLOP/s' if unit == 'flop' else 'GB/s'}")

    def group_rate(kinds):
        fl = sum(work[k][1] * prof[k][0] for k in kinds if k in prof)
        tm = sum(prof[k][1] for k in kinds if k in prof) / 1e3
        return (fl / tm / 1e12) if tm > 0 else 0.0

    peak = PEAK_TFLOPS[cfg.dtype]
    att_tf, gemm_tf = group_rate(ATTN_KINDS), group_rate(GEMM_KINDS)
    ew = exp_work(cfg, nb)
    att_ms = sum(prof[k][1] for k in ATTN_KINDS if k in prof)
    att_exp = (sum(ew[k] * prof[k][0] for k in ATTN_KINDS if k in prof) / (att_ms / 1e3)
               if att_ms > 0 else 0.0)

    dom = max(prof.items(), key=lambda kv: kv[1][1])[0]
    unit, amount = work[dom]
    n_dom, ms_dom = prof[dom]
    avg = ms_dom / n_dom / 1e3
    src = "attention.hip" if dom.startswith("attention") else (
        "gemm.hip" if dom.startswith("gemm") else "pointwise.hip")
    if unit == "flop":
        roof = {"bound": "mfma", "achieved": round(amount / avg / 1e12, 2), "peak": peak,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(amount / avg / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, cfg.name)
    roof["kernel"] = dom
    roof["per_launch"] = {"work": amount, "work_unit": "FLOP" if unit == "flop" else "byte",
                          "avg_us": round(avg * 1e6, 3), "launches": n_dom,
                          "timing": "start/stop events attached to each launch "
                                    "(hipExtLaunchKernelGGL), launch stream",
                          "source": src}

    fl = cfg.flops_per_step()
    if guided:
        # both branches, except the patch embedding and the time path (shared)
        shared = 2 * cfg.tokens * cfg.patch_dim * cfg.hidden + fl["time"]
        fl = {k: (2 * v if k != "time" else v) for k, v in fl.items()}
        fl["total"] -= shared
    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_per_step, 4),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded Philox N(0,1) latents/context, N(0,0.02^2) random-init weights)",
        "config": {"workload": cfg.name, "tokens": cfg.tokens, "hidden": cfg.hidden,
                   "blocks": cfg.num_blocks, "heads": cfg.heads, "head_dim": cfg.head_dim,
                   "mlp_hidden": cfg.mlp_hidden, "ctx_len": cfg.ctx_len,
                   "text_dim": cfg.text_dim, "latent": list(cfg.latent_shape),
                   "schedule_steps": cfg.steps, "shift": cfg.shift, "batch": 1,
                   "parallelism": "single GPU",
                   **({"guidance_scale": args.guidance, "sequences": 2} if guided else {}),
                   **({"weights": "layerwise offload from pinned host memory"}
                      if args.offload else {}),
                   **({"cache": dict(CACHE_KNOBS, runs_of=cfg.steps)} if args.cache else {})},
        "step_tflops": round(fl["total"] / (ms_per_step / 1e3) / 1e12, 2),
        "step_frac_of_peak": round(fl["total"] / (ms_per_step / 1e3) / 1e12 / peak, 4),
        "attention": {"tflops": round(att_tf, 2), "frac_of_peak": round(att_tf / peak, 4),
                      "exp_per_s": round(att_exp / 1e12, 3),
                      "exp_frac_of_peak": round(att_exp / PEAK_EXP_PER_S, 4)},
        "gemm": {"tflops": round(gemm_tf, 2), "frac_of_peak": round(gemm_tf / peak, 4)},
        "roofline": roof,
        "kernels": kernels,
    }
    if args.cache:
        out["cache"] = {"cached_steps": timed_hits, "steps": args.steps}
        log(f"[bench] cache: {timed_hits} of {args.steps} timed steps reused the cache")
    if args.offload:
        es = 2 if cfg.dtype == "bf16" else 4
        D, F = cfg.hidden, cfg.mlp_hidden
        streamed = es * cfg.num_blocks * (8 * D * D + 2 * F * D + 9 * D + F)
        out["offload"] = {"bytes_per_step": streamed,
                          "host_to_device_gbs": round(streamed / (ms_per_step / 1e3) / 1e9, 2)}
        log(f"[bench] offload: {streamed / 1e9:.3f} GB streamed per step, "
            f"{out['offload']['host_to_device_gbs']} GB/s")
    plain = not (guided or args.offload or args.cache)
    if plain and cfg.name in CHAIN_MEDIAN:
        out["chain_median_ms_per_step"] = round(time_chains(m, X0, Ed, sched, 5), 4)
    m.close()
    del m, X, Ed, End
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample of the same workload")
        out["cpu_baseline"] = (cpu_baseline(cfg, prm, X0, E, E_neg=SP.make_ctx(cfg, seed=3),
                                            g=args.guidance) if guided else
                               cpu_baseline(cfg, prm, X0, E))
        log(f"[bench] cpu_baseline: {out['cpu_baseline']['sample']}")
    else:
        out["cpu_baseline"] = None
    del prm
    if plain and not args.no_other_configs:
        per = {cfg.name: {"ms_per_step": out["ms_per_step"], "steps_timed": args.steps,
                          "step_frac_of_peak": out["step_frac_of_peak"]}}
        if "chain_median_ms_per_step" in out:
            per[cfg.name]["chain_median_ms_per_step"] = out["chain_median_ms_per_step"]
        for name in OTHER_CONFIG_STEPS:
            if name != cfg.name:
                per[name] = time_other_config(name)
        out["per_config"] = per
    print(json.dumps(out), flush=True)
    return 0


# the two smallest workloads: median over five whole sampling runs
CHAIN_MEDIAN = ("tiny_f32", "image_s_bf16")
# steps timed for each workload's seconds-per-step line (after one warm-up
# step); the two smallest time whole runs instead
OTHER_CONFIG_STEPS = {"tiny_f32": None, "image_s_bf16": None, "wan1p3b_bf16": 4,
                      "image_l_bf16": 10, "wan14b_bf16": 3}


def time_chains(m, X0, Ed, sched, runs: int) -> float:
    """Median over ``runs`` whole sampling runs (every step of the schedule,
    begun afresh from X0) of the run time divided by its steps, in ms."""
    import torch
    stream = torch.cuda.current_stream()
    X = torch.from_numpy(X0).cuda()
    per = []
    for _ in range(runs + 1):          # the first run warms up
        X.copy_(torch.from_numpy(X0))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t, s0, s1 in sched:
            m.denoise_step(X, Ed, t, s0, s1)
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / len(sched))
    return float(np.median(per[1:]))


def time_other_config(name: str) -> dict:
    """Seconds per plain denoise step of another workload (fresh inputs and
    model, freed afterwards)."""
    import torch
    from diffusion_transformer_denoising_amd import binding as B
    from diffusion_transformer_denoising_amd.model import DeviceDiT, torch_dtype
    from synth import params as SP
    from synth.configs import get_config
    cfg = get_config(name)
    t0 = time.perf_counter()
    prm = SP.make_params(cfg)
    X0 = SP.make_latents(cfg)
    m = DeviceDiT(cfg, prm)
    del prm
    Ed = torch.from_numpy(SP.make_ctx(cfg)).cuda().to(torch_dtype(cfg))
    sig = B.dit_flow_sigmas(cfg.steps, cfg.shift)
    sched = [(float(np.float32(1000.0 * sig[k])), float(sig[k]), float(sig[k + 1]))
             for k in range(cfg.steps)]
    k = OTHER_CONFIG_STEPS[name]
    if k is None:
        ms = time_chains(m, X0, Ed, sched, 5)
        rec = {"ms_per_step": round(ms, 4), "chain_median_ms_per_step": round(ms, 4),
               "runs": 5, "steps_per_run": cfg.steps}
    else:
        X = torch.from_numpy(X0).cuda()
        stream = torch.cuda.current_stream()
        m.denoise_step(X, Ed, *sched[0])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(k):
            m.denoise_step(X, Ed, *sched[(1 + i) % cfg.steps])
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / k
        rec = {"ms_per_step": round(ms, 4), "steps_timed": k}
    peak = PEAK_TFLOPS[cfg.dtype]
    rec["step_frac_of_peak"] = round(cfg.flops_per_step()["total"] / (ms / 1e3) / 1e12 / peak, 4)
    m.close()
    del m
    torch.cuda.empty_cache()
    log(f"[bench] {name}: {rec['ms_per_step']:.4f} ms/step ({time.perf_counter() - t0:.1f} s "
        f"with inputs)")
    return rec


if __name__ == "__main__":
    sys.exit(main())

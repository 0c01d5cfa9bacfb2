"""ctypes binding of libdit.so: the C ABI of include/dit.h under the same names.

Argument marshalling only.  Device pointers are plain integers (e.g.
``tensor.data_ptr()``), streams are integers (``torch.cuda.current_stream()
.cuda_stream``) or 0 for the default stream.  Every function raises
``DitError`` when the library returns a non-OK status.  There is no fallback:
if libdit.so is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdit.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "include", "dit.h")

DIT_OK = 0
DIT_ERR_INVALID_ARG = -1
DIT_ERR_SHAPE = -2
DIT_ERR_UNSUPPORTED = -3
DIT_ERR_WORKSPACE = -4
DIT_ERR_HIP = -5
DIT_F32 = 0
DIT_BF16 = 1

c_i32, c_i64, c_f32, c_f64, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_double, ctypes.c_void_p)


class dit_config(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in (
        "num_blocks", "hidden", "heads", "head_dim", "mlp_hidden", "freq_dim", "in_channels",
        "patch_f", "patch_h", "patch_w", "lat_f", "lat_h", "lat_w", "rope_f", "rope_h", "rope_w",
        "ctx_len_max", "text_dim")] + [("rope_theta", c_f32), ("ln_eps", c_f32), ("dtype", c_i32),
                                       ("guidance", c_i32), ("offload", c_i32), ("cache", c_i32)]


class dit_cache_params(ctypes.Structure):
    _fields_ = [("fn", c_i32), ("bn", c_i32), ("warmup", c_i32), ("rdt", c_f32),
                ("max_consecutive", c_i32), ("taylorseer", c_i32), ("ts_order", c_i32)]


class dit_cache_state(ctypes.Structure):
    _fields_ = [("step", c_i32), ("consecutive", c_i32), ("last_full", c_i32), ("factors", c_i32),
                ("hit", c_i32), ("cached_total", c_i32), ("diff", c_f64)]


GLOBAL_FIELDS = ("t1_w", "t1_b", "t2_w", "t2_b", "mod_w", "mod_b", "txt_w", "txt_b",
                 "pe_w", "pe_b", "head_table", "out_w", "out_b")
BLOCK_FIELDS = ("table", "qkv_w", "qkv_b", "o_w", "o_b", "cq_w", "cq_b", "ckv_w", "ckv_b",
                "co_w", "co_b", "w1", "b1", "w2", "b2")


class dit_global_weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in GLOBAL_FIELDS]


class dit_block_weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in BLOCK_FIELDS]


class dit_weights(ctypes.Structure):
    _fields_ = [("global_", dit_global_weights), ("blocks", ctypes.POINTER(dit_block_weights))]


class DitError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_LIB = None

_SIGS = {
    "dit_workspace_size": ([ctypes.POINTER(dit_config), ctypes.POINTER(ctypes.c_size_t)], c_i32),
    "dit_create": ([ctypes.POINTER(dit_config), ctypes.POINTER(dit_weights), c_vp, ctypes.c_size_t,
                    c_vp, ctypes.POINTER(c_vp)], c_i32),
    "dit_destroy": ([c_vp], c_i32),
    "dit_block_forward": ([c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp], c_i32),
    "dit_block_forward_static": ([ctypes.POINTER(dit_config), ctypes.POINTER(dit_block_weights),
                                  c_vp, c_vp, c_i32, c_vp, c_vp], c_i32),
    "dit_denoise_step": ([c_vp, c_vp, c_vp, c_i32, c_f32, c_f32, c_f32, c_vp, c_vp], c_i32),
    "dit_denoise_step_cfg": ([c_vp, c_vp, c_vp, c_vp, c_i32, c_f32, c_f32, c_f32, c_f32, c_vp,
                              c_vp], c_i32),
    "dit_cache_begin": ([c_vp, ctypes.POINTER(dit_cache_params)], c_i32),
    "dit_cache_state_get": ([c_vp, ctypes.POINTER(dit_cache_state)], c_i32),
    "dit_denoise_step_cached": ([c_vp, c_vp, c_vp, c_vp, c_i32, c_f32, c_f32, c_f32, c_f32, c_vp,
                                 c_vp], c_i32),
    "dit_cache_factor_get": ([c_vp, c_i32, c_vp, c_vp], c_i32),
    "dit_euler_step": ([c_vp, c_vp, c_i64, c_f32, c_f32, c_vp], c_i32),
    "dit_flow_sigmas": ([c_i32, c_f64, ctypes.POINTER(c_f64)], c_i32),
    "dit_attention": ([c_i32, c_i32, c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64,
                       c_i32, c_i32, c_vp], c_i32),
    "dit_layernorm_modulate": ([c_i32, c_i32, c_f32, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp], c_i32),
    "dit_gemm": ([c_i32, c_i32, c_vp, c_i64, c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp, c_i64,
                  c_vp, c_i32, c_vp], c_i32),
    "dit_time_embedding": ([c_vp, c_f32, c_vp, c_vp, c_vp, c_vp], c_i32),
    "dit_status_string": ([c_i32], ctypes.c_char_p),
    "dit_profile_enable": ([c_vp, c_i32], c_i32),
    "dit_profile_read": ([c_vp, c_i32, ctypes.POINTER(c_i64), ctypes.POINTER(c_f64)], c_i32),
    "dit_profile_kind_count": ([], c_i32),
    "dit_profile_kind_name": ([c_i32], ctypes.c_char_p),
}


def lib() -> ctypes.CDLL:
    """Load libdit.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m diffusion_transformer_denoising_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def header_functions() -> list:
    """Names of the functions include/dit.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dit_[a-z_]+)\s*\(", text)))


def _check(status: int, where: str):
    if status != DIT_OK:
        raise DitError(status, where)


def status_string(status: int) -> str:
    return lib().dit_status_string(int(status)).decode()


def dit_status_string(status: int) -> str:
    return status_string(status)


def make_config(cfg, guidance: bool = False, offload: bool = False,
                cache: bool = False) -> dit_config:
    """dit_config from any object with the workload attributes (hidden, heads,
    head_dim, mlp_hidden, num_blocks, in_channels, patch, latent, rope,
    ctx_len, text_dim, freq_dim, rope_theta, ln_eps, dtype); guidance sizes
    the workspace for guided steps; offload streams the block weights from
    page-locked host memory; cache sizes the workspace for cached steps."""
    c = dit_config()
    c.guidance = 1 if guidance else 0
    c.offload = 1 if offload else 0
    c.cache = 1 if cache else 0
    c.num_blocks, c.hidden, c.heads, c.head_dim = cfg.num_blocks, cfg.hidden, cfg.heads, cfg.head_dim
    c.mlp_hidden, c.freq_dim, c.in_channels = cfg.mlp_hidden, cfg.freq_dim, cfg.in_channels
    c.patch_f, c.patch_h, c.patch_w = cfg.patch
    c.lat_f, c.lat_h, c.lat_w = cfg.latent
    c.rope_f, c.rope_h, c.rope_w = cfg.rope
    c.ctx_len_max, c.text_dim = cfg.ctx_len, cfg.text_dim
    c.rope_theta, c.ln_eps = cfg.rope_theta, cfg.ln_eps
    c.dtype = DIT_BF16 if cfg.dtype == "bf16" else DIT_F32
    return c


def dit_workspace_size(cfg: dit_config) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dit_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), "dit_workspace_size")
    return n.value


def dit_create(cfg: dit_config, weights: dit_weights, workspace: int, workspace_bytes: int,
               stream: int = 0) -> int:
    h = c_vp()
    _check(lib().dit_create(ctypes.byref(cfg), ctypes.byref(weights), workspace, workspace_bytes,
                            stream, ctypes.byref(h)), "dit_create")
    return h.value


def dit_destroy(handle: int) -> None:
    _check(lib().dit_destroy(handle), "dit_destroy")


def dit_block_forward(handle: int, block: int, x: int, ctx: int, ctx_len: int, mod: int,
                      stream: int = 0) -> None:
    _check(lib().dit_block_forward(handle, block, x, ctx, ctx_len, mod, stream), "dit_block_forward")


def dit_denoise_step(handle: int, X: int, ctx: int, ctx_len: int, t: float, sigma: float,
                     sigma_next: float, v_out: int | None = None, stream: int = 0) -> None:
    _check(lib().dit_denoise_step(handle, X, ctx, ctx_len, t, sigma, sigma_next, v_out, stream),
           "dit_denoise_step")


def dit_denoise_step_cfg(handle: int, X: int, ctx: int, ctx_neg: int, ctx_len: int, t: float,
                         sigma: float, sigma_next: float, guidance_scale: float,
                         v_out: int | None = None, stream: int = 0) -> None:
    _check(lib().dit_denoise_step_cfg(handle, X, ctx, ctx_neg, ctx_len, t, sigma, sigma_next,
                                      guidance_scale, v_out, stream), "dit_denoise_step_cfg")


def make_cache_params(fn: int = 2, bn: int = 1, warmup: int = 4, rdt: float = 0.4,
                      max_consecutive: int = 4, taylorseer: bool = True,
                      ts_order: int = 2) -> dit_cache_params:
    """dit_cache_params; the defaults are the knob values of the pages'
    Cache-DiT deployment."""
    p = dit_cache_params()
    p.fn, p.bn, p.warmup, p.rdt = fn, bn, warmup, rdt
    p.max_consecutive, p.taylorseer, p.ts_order = max_consecutive, 1 if taylorseer else 0, ts_order
    return p


def dit_cache_begin(handle: int, params: dit_cache_params) -> None:
    _check(lib().dit_cache_begin(handle, ctypes.byref(params)), "dit_cache_begin")


def dit_cache_state_get(handle: int) -> dit_cache_state:
    st = dit_cache_state()
    _check(lib().dit_cache_state_get(handle, ctypes.byref(st)), "dit_cache_state_get")
    return st


def dit_block_forward_static(cfg: dit_config, weights: dit_block_weights, x: int, ctx: int,
                             ctx_len: int, mod: int, stream: int = 0) -> None:
    _check(lib().dit_block_forward_static(ctypes.byref(cfg), ctypes.byref(weights), x, ctx,
                                          ctx_len, mod, stream), "dit_block_forward_static")


def dit_cache_factor_get(handle: int, q: int, dst: int, stream: int = 0) -> None:
    _check(lib().dit_cache_factor_get(handle, q, dst, stream), "dit_cache_factor_get")


def dit_denoise_step_cached(handle: int, X: int, ctx: int, ctx_neg: int | None, ctx_len: int,
                            t: float, sigma: float, sigma_next: float, guidance_scale: float = 1.0,
                            v_out: int | None = None, stream: int = 0) -> None:
    _check(lib().dit_denoise_step_cached(handle, X, ctx, ctx_neg, ctx_len, t, sigma, sigma_next,
                                         guidance_scale, v_out, stream), "dit_denoise_step_cached")


def dit_euler_step(X: int, v: int, n: int, sigma: float, sigma_next: float, stream: int = 0) -> None:
    _check(lib().dit_euler_step(X, v, n, sigma, sigma_next, stream), "dit_euler_step")


def dit_flow_sigmas(n_steps: int, shift: float) -> list:
    out = (c_f64 * (max(int(n_steps), 0) + 1))()
    _check(lib().dit_flow_sigmas(n_steps, shift, out), "dit_flow_sigmas")
    return list(out)


def dit_attention(dtype: int, heads: int, head_dim: int, q: int, ldq: int, k: int, ldk: int,
                  vt: int, ldv: int, o: int, ldo: int, sq: int, sk: int, stream: int = 0) -> None:
    _check(lib().dit_attention(dtype, heads, head_dim, q, ldq, k, ldk, vt, ldv, o, ldo, sq, sk,
                               stream), "dit_attention")


DIT_EPI_STORE, DIT_EPI_GELU, DIT_EPI_RESIDUAL, DIT_EPI_STORE_F32 = 0, 1, 2, 3


def dit_gemm(dtype: int, epilogue: int, A: int, lda: int, W: int, ldw: int, M: int, N: int, K: int,
             bias: int | None, out: int, ldo: int, gate: int | None = None, tile: int = 0,
             stream: int = 0) -> None:
    _check(lib().dit_gemm(dtype, epilogue, A, lda, W, ldw, M, N, K, bias, out, ldo, gate, tile,
                          stream), "dit_gemm")


def dit_layernorm_modulate(dtype: int, D: int, eps: float, x: int, rows: int, shift: int | None,
                           scale: int | None, y: int, stream: int = 0) -> None:
    _check(lib().dit_layernorm_modulate(dtype, D, eps, x, rows, shift, scale, y, stream),
           "dit_layernorm_modulate")


def dit_time_embedding(handle: int, t: float, block_mod: int, head_mod: int, temb: int,
                       stream: int = 0) -> None:
    _check(lib().dit_time_embedding(handle, t, block_mod, head_mod, temb, stream),
           "dit_time_embedding")


def dit_profile_enable(handle: int, enable: bool) -> None:
    _check(lib().dit_profile_enable(handle, 1 if enable else 0), "dit_profile_enable")


def dit_profile_read(handle: int, kind: int):
    n = c_i64(0)
    ms = c_f64(0.0)
    _check(lib().dit_profile_read(handle, kind, ctypes.byref(n), ctypes.byref(ms)),
           "dit_profile_read")
    return n.value, ms.value


def dit_profile_kind_count() -> int:
    return lib().dit_profile_kind_count()


def dit_profile_kind_name(kind: int) -> str | None:
    r = lib().dit_profile_kind_name(kind)
    return r.decode() if r is not None else None


def profile_summary(handle: int) -> dict:
    """{kind name: (launches, total ms)} for every kind with launches."""
    out = {}
    for k in range(dit_profile_kind_count()):
        n, ms = dit_profile_read(handle, k)
        if n:
            out[dit_profile_kind_name(k)] = (n, ms)
    return out

"""Device-resident DiT model for the C ABI: torch provides the device memory
(weights, workspace) and the stream; every step of the computation runs in
libdit.so.

    m = DeviceDiT(cfg, params)            # params: {"global": {...}, "blocks": [...]}
    m.denoise_step(X, ctx, t, sigma, sigma_next, v_out=None)
    m.block_forward(b, x, ctx_proj, mod)

Tensors passed in must already be on the device, contiguous and of the right
dtype (float32 latents / residual / modulation, model dtype for context).
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import binding as B


def torch_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload float32 values as the storage type ("bf16": rounded to nearest
    even, exact for values that are already bfloat16 numbers)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _stream_of(device, stream=None) -> int:
    if stream is not None:
        return int(stream)
    return torch.cuda.current_stream(device).cuda_stream


def attention(dtype: str, heads: int, head_dim: int, q, k, vt, o, sq: int, sk: int, stream=None):
    """dit_attention on torch tensors (row strides taken from the tensors)."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for t in (q, k, vt, o):
        if t.dtype != dt or t.stride(1) != 1:
            raise ValueError("attention operands must be row-major tensors of the model dtype")
    B.dit_attention(B.DIT_BF16 if dtype == "bf16" else B.DIT_F32, heads, head_dim,
                    q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), vt.data_ptr(),
                    vt.stride(0), o.data_ptr(), o.stride(0), sq, sk, _stream_of(q.device, stream))


def layernorm_modulate(dtype: str, eps: float, x, shift, scale, y, stream=None):
    """dit_layernorm_modulate on torch tensors: x float [rows, D] -> y [rows, D]."""
    B.dit_layernorm_modulate(B.DIT_BF16 if dtype == "bf16" else B.DIT_F32, x.shape[1], eps,
                             x.data_ptr(), x.shape[0],
                             shift.data_ptr() if shift is not None else None,
                             scale.data_ptr() if scale is not None else None,
                             y.data_ptr(), _stream_of(x.device, stream))


def gemm(dtype: str, epilogue: int, A, W, bias, out, gate=None, tile: int = 0, stream=None):
    """dit_gemm on torch tensors: out (+)= epilogue(A @ W^T + bias)."""
    B.dit_gemm(B.DIT_BF16 if dtype == "bf16" else B.DIT_F32, epilogue, A.data_ptr(), A.stride(0),
               W.data_ptr(), W.stride(0), A.shape[0], W.shape[0], A.shape[1],
               bias.data_ptr() if bias is not None else None, out.data_ptr(), out.stride(0),
               gate.data_ptr() if gate is not None else None, tile, _stream_of(A.device, stream))


class DeviceDiT:
    def __init__(self, cfg, params: dict, device: str = "cuda", stream: int | None = None,
                 guidance: bool = False, offload: bool = False, pack_offload: bool = True,
                 cache: bool = False, workspace: torch.Tensor | None = None):
        """`workspace`: an optional caller-owned uint8 device tensor of at least
        dit_workspace_size bytes, 256-byte aligned, that the handle uses instead
        of allocating its own; its contents on entry do not matter."""
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = B.make_config(cfg, guidance, offload, cache)
        g = params["global"]
        self._keep = []

        def up(a):
            t = to_device(a, cfg.dtype, self.device)
            self._keep.append(t)
            return t.data_ptr()

        def pinned(a):
            t = to_device(a, cfg.dtype, torch.device("cpu")).pin_memory()
            self._keep.append(t)
            return t.data_ptr()

        def pinned_block(p):
            # the weights of one offloaded block in one page-locked buffer, each
            # field after the table at the first 256-byte boundary past the
            # previous one (the layout the library copies in one transfer)
            host = {n: to_device(p[n], cfg.dtype, torch.device("cpu")).reshape(-1).view(torch.uint8)
                    for n in B.BLOCK_FIELDS}
            offs, end = {}, 0
            for n in B.BLOCK_FIELDS[1:]:
                offs[n] = end
                end = (end + host[n].numel() + 255) // 256 * 256
            buf = torch.empty(end, dtype=torch.uint8, pin_memory=True)
            for n in B.BLOCK_FIELDS[1:]:
                buf[offs[n]:offs[n] + host[n].numel()].copy_(host[n])
            table = host[B.BLOCK_FIELDS[0]].clone().pin_memory()
            self._keep += [buf, table]
            return {B.BLOCK_FIELDS[0]: table.data_ptr(),
                    **{n: buf.data_ptr() + offs[n] for n in B.BLOCK_FIELDS[1:]}}

        gw = B.dit_global_weights()
        for name in B.GLOBAL_FIELDS:
            a = g.get(name)
            setattr(gw, name, up(a) if a is not None else None)
        self._blocks = (B.dit_block_weights * cfg.num_blocks)()
        for i, p in enumerate(params["blocks"]):
            if p is None:
                raise ValueError(f"block {i} parameters missing")
            if offload and pack_offload:
                ptrs = pinned_block(p)
            elif offload:   # one page-locked buffer per field: copied field by field
                ptrs = {n: pinned(p[n]) for n in B.BLOCK_FIELDS}
            else:
                ptrs = {n: up(p[n]) for n in B.BLOCK_FIELDS}
            for name in B.BLOCK_FIELDS:
                setattr(self._blocks[i], name, ptrs[name])
        self._w = B.dit_weights()
        self._w.global_ = gw
        self._w.blocks = ctypes.cast(self._blocks, ctypes.POINTER(B.dit_block_weights))
        self.ws_bytes = B.dit_workspace_size(self.c)
        if workspace is None:
            workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        elif (workspace.dtype != torch.uint8 or workspace.device.type != self.device.type
              or (self.device.index is not None and workspace.device.index != self.device.index)
              or not workspace.is_contiguous() or workspace.numel() < self.ws_bytes):
            raise ValueError(f"workspace must be a contiguous uint8 tensor of at least "
                             f"{self.ws_bytes} bytes on {self.device}")
        self.workspace = workspace
        self.handle = B.dit_create(self.c, self._w, self.workspace.data_ptr(), self.ws_bytes,
                                   self._stream(stream))

    def _stream(self, stream=None) -> int:
        if stream is not None:
            return int(stream)
        return torch.cuda.current_stream(self.device).cuda_stream

    def close(self):
        if getattr(self, "handle", None):
            B.dit_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- calls -----------------------------------------------------------
    def denoise_step(self, X: torch.Tensor, ctx: torch.Tensor, t: float, sigma: float,
                     sigma_next: float, v_out: torch.Tensor | None = None, stream=None):
        self._check(X, torch.float32)
        self._check(ctx, torch_dtype(self.cfg))
        if v_out is not None:
            self._check(v_out, torch.float32)
        B.dit_denoise_step(self.handle, X.data_ptr(), ctx.data_ptr(), ctx.shape[0], t, sigma,
                           sigma_next, v_out.data_ptr() if v_out is not None else None,
                           self._stream(stream))

    def denoise_step_cfg(self, X: torch.Tensor, ctx: torch.Tensor, ctx_neg: torch.Tensor,
                         t: float, sigma: float, sigma_next: float, guidance_scale: float,
                         v_out: torch.Tensor | None = None, stream=None):
        """Guided step (the model must be built with guidance=True)."""
        self._check(X, torch.float32)
        self._check(ctx, torch_dtype(self.cfg))
        self._check(ctx_neg, torch_dtype(self.cfg))
        if ctx_neg.shape != ctx.shape:
            raise ValueError("positive and negative contexts must have the same shape")
        if v_out is not None:
            self._check(v_out, torch.float32)
        B.dit_denoise_step_cfg(self.handle, X.data_ptr(), ctx.data_ptr(), ctx_neg.data_ptr(),
                               ctx.shape[0], t, sigma, sigma_next, guidance_scale,
                               v_out.data_ptr() if v_out is not None else None,
                               self._stream(stream))

    def cache_begin(self, **knobs):
        """Start a cached sampling run (model built with cache=True); knobs as
        binding.make_cache_params."""
        B.dit_cache_begin(self.handle, B.make_cache_params(**knobs))

    def cache_state(self) -> dict:
        st = B.dit_cache_state_get(self.handle)
        return {n: getattr(st, n) for n, _ in B.dit_cache_state._fields_}

    def cache_factor(self, q: int, nb: int = 1, stream=None) -> torch.Tensor:
        """Taylor factor q of the current cached run, float [nb, S, D] (a copy)."""
        out = torch.empty((nb, self.cfg.tokens, self.cfg.hidden), dtype=torch.float32,
                          device=self.device)
        B.dit_cache_factor_get(self.handle, q, out.data_ptr(), self._stream(stream))
        return out

    def denoise_step_cached(self, X: torch.Tensor, ctx: torch.Tensor, t: float, sigma: float,
                            sigma_next: float, ctx_neg: torch.Tensor | None = None,
                            guidance_scale: float = 1.0, v_out: torch.Tensor | None = None,
                            stream=None):
        """One step of the cached run (guided when ctx_neg is given)."""
        self._check(X, torch.float32)
        self._check(ctx, torch_dtype(self.cfg))
        if ctx_neg is not None:
            self._check(ctx_neg, torch_dtype(self.cfg))
            if ctx_neg.shape != ctx.shape:
                raise ValueError("positive and negative contexts must have the same shape")
        if v_out is not None:
            self._check(v_out, torch.float32)
        B.dit_denoise_step_cached(self.handle, X.data_ptr(), ctx.data_ptr(),
                                  ctx_neg.data_ptr() if ctx_neg is not None else None,
                                  ctx.shape[0], t, sigma, sigma_next, guidance_scale,
                                  v_out.data_ptr() if v_out is not None else None,
                                  self._stream(stream))

    def block_forward(self, block: int, x: torch.Tensor, ctx: torch.Tensor, mod: torch.Tensor,
                      stream=None):
        self._check(x, torch.float32)
        self._check(mod, torch.float32)
        self._check(ctx, torch_dtype(self.cfg))
        B.dit_block_forward(self.handle, block, x.data_ptr(), ctx.data_ptr(), ctx.shape[0],
                            mod.data_ptr(), self._stream(stream))

    def time_embedding(self, t: float, stream=None):
        D = self.cfg.hidden
        bmod = torch.empty((self.cfg.num_blocks, 6, D), dtype=torch.float32, device=self.device)
        hmod = torch.empty((2, D), dtype=torch.float32, device=self.device)
        temb = torch.empty((D,), dtype=torch.float32, device=self.device)
        B.dit_time_embedding(self.handle, t, bmod.data_ptr(), hmod.data_ptr(), temb.data_ptr(),
                             self._stream(stream))
        return bmod, hmod, temb

    def _check(self, t: torch.Tensor, dtype):
        if t.device.type != self.device.type or not t.is_contiguous() or t.dtype != dtype:
            raise ValueError(f"expected a contiguous {dtype} tensor on {self.device}, got "
                             f"{t.dtype} on {t.device} (contiguous={t.is_contiguous()})")

"""Plain float64 CPU oracle of one DiT denoising step (TEST INFRASTRUCTURE ONLY).

What is computed.  The SGLang-Diffusion page "Disaggregated Diffusion Pipeline"
(section "Quick Start", the role table) defines the denoiser as the DiT forward
loop plus the scheduler stepping it drives.  The page "Support New Diffusion
Models" fixes the interface: the DiT forward takes ``hidden_states`` (latents),
``encoder_hidden_states`` (prompt embeddings) and ``timestep`` (section
"2. Pipeline Config"), and the denoising stage consumes latents, timesteps in
the reference order and a separate list of sigmas (section "4. Last-Resort
Before-Denoising Stage", the table of fields required by DenoisingStage).  The
stable-diffusion.cpp page "Model Configuration Conventions" (section "Sampling
And Geometry") names the flow-prediction denoisers and the flow-shift default.
The pages print no formula for the block itself; every form below is the
plainest standard reading (an adaLN DiT block with self-attention, cross-
attention and a GELU MLP, a shifted linear flow schedule and an Euler update),
each one called out where it is chosen.

How.  Everything is float64 numpy, written as the definitions read: no
blocking, fusion or reordering.  Inputs are the exact stored values (bf16
workloads pass their bf16-rounded weights as float32/float64 arrays).  A
library matmul is the only composite primitive used.  ``rows`` arguments only
evaluate the same definition at a subset of output tokens.

Shape arguments come from any object with the attributes used here (hidden,
heads, head_dim, patch, latent, in_channels, rope, rope_theta, ln_eps,
freq_dim); this module imports nothing from the GPU side or the input
generator.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f(a):
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Schedule  ("Support New Diffusion Models", section "Read the Reference First":
# timestep and sigma schedule; section "4. Last-Resort Before-Denoising Stage":
# timesteps and sigmas are separate fields; "Model Configuration Conventions",
# section "Sampling And Geometry": default flow shift.)
# Reading: sigma runs linearly from 1 to 0 over N steps (N + 1 points) and is
# then shifted by s -> shift*s / (1 + (shift - 1)*s); the timestep fed to the
# network is 1000*sigma.
# ---------------------------------------------------------------------------
def flow_sigmas(n_steps: int, shift: float = 1.0) -> np.ndarray:
    n = int(n_steps)
    if n < 1:
        raise ValueError("n_steps must be >= 1")
    s = 1.0 - np.arange(n + 1, dtype=F64) / n
    return shift * s / (1.0 + (shift - 1.0) * s)


def flow_timesteps(sigmas) -> np.ndarray:
    return 1000.0 * _f(sigmas)


# ---------------------------------------------------------------------------
# Elementwise pieces (standard definitions; readings listed in the header).
# ---------------------------------------------------------------------------
def silu(z):
    z = _f(z)
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z):
    """GELU, tanh approximation: z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3)))."""
    z = _f(z)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def linear(x, w, b=None):
    """x @ w^T (+ b), w stored [out_features, in_features]."""
    y = _f(x) @ _f(w).T
    if b is not None:
        y = y + _f(b)
    return y


def layer_norm(x, eps: float):
    """Per-row normalisation over the last axis: (x - mean) / sqrt(var + eps),
    biased variance, no affine parameters."""
    x = _f(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(y, shift, scale):
    """adaLN modulation y * (1 + scale) + shift (scale, shift broadcast over rows)."""
    return _f(y) * (1.0 + _f(scale)) + _f(shift)


def softmax_rows(s):
    """Row softmax over the last axis (max-subtracted for range only)."""
    s = _f(s)
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Timestep embedding.  Reading: a 256-wide sinusoid of t (cosine half first,
# frequencies 10000^(-j/128)), a two-layer SiLU MLP giving temb [D], and one
# shared projection of SiLU(temb) to the six modulation vectors [6, D].
# ---------------------------------------------------------------------------
def sinusoid(t: float, dim: int = 256) -> np.ndarray:
    half = dim // 2
    omega = 10000.0 ** (-np.arange(half, dtype=F64) / half)
    a = F64(t) * omega
    return np.concatenate([np.cos(a), np.sin(a)])


def time_embedding(t: float, g: dict, dim: int = 256):
    """Returns (temb [D], e [6, D])."""
    s = sinusoid(t, dim)
    temb = linear(silu(linear(s, g["t1_w"], g["t1_b"])), g["t2_w"], g["t2_b"])
    e = linear(silu(temb), g["mod_w"], g["mod_b"])
    return temb, e.reshape(6, -1)


# ---------------------------------------------------------------------------
# Latent packing ("Support New Diffusion Models", section "Read the Reference
# First": latent shape and packing; "Verify the Port": decode needs the raw
# latent shape).  Token n = (f'*H' + h')*W' + w'; within a token the patch
# element (c, i, j, k) sits at ((c*pf + i)*ph + j)*pw + k and holds
# X[c, f'*pf + i, h'*ph + j, w'*pw + k].
# ---------------------------------------------------------------------------
def patchify(X, patch) -> np.ndarray:
    X = _f(X)
    C, F, H, W = X.shape
    pf, ph, pw = patch
    g = (F // pf, H // ph, W // pw)
    Y = X.reshape(C, g[0], pf, g[1], ph, g[2], pw).transpose(1, 3, 5, 0, 2, 4, 6)
    return Y.reshape(g[0] * g[1] * g[2], C * pf * ph * pw)


def unpatchify(u, patch, latent_shape) -> np.ndarray:
    u = _f(u)
    C, F, H, W = latent_shape
    pf, ph, pw = patch
    g = (F // pf, H // ph, W // pw)
    Y = u.reshape(g[0], g[1], g[2], C, pf, ph, pw).transpose(3, 0, 4, 1, 5, 2, 6)
    return Y.reshape(C, F, H, W)


def token_positions(grid) -> np.ndarray:
    """Integer (f', h', w') grid coordinates of every token, [S, 3]."""
    f, h, w = np.meshgrid(np.arange(grid[0]), np.arange(grid[1]), np.arange(grid[2]),
                          indexing="ij")
    return np.stack([f.ravel(), h.ravel(), w.ravel()], axis=1)


# ---------------------------------------------------------------------------
# Rotary embedding ("Support New Diffusion Models", section "Verify the Port",
# which lists a rotary shape or style mismatch among the failure points).
# Reading: interleaved pairs.  Each head's channels are split into consecutive
# segments of widths (d_f, d_h, d_w) for the three grid axes; pair j of the
# segment of axis a is the channel pair (off_a + 2j, off_a + 2j + 1), rotated
# by the angle pos_a * theta^(-2j / d_a).
# ---------------------------------------------------------------------------
def rope_rotate(q, pos, split, theta: float = 10000.0) -> np.ndarray:
    """q [S, H, d] rotated by token positions pos [S, 3]."""
    q = _f(q)
    out = q.copy()
    off = 0
    for axis in range(3):
        da = int(split[axis])
        for j in range(da // 2):
            phi = _f(pos[:, axis]) * theta ** (-2.0 * j / da)
            c = np.cos(phi)[:, None]
            s = np.sin(phi)[:, None]
            u0 = q[:, :, off + 2 * j]
            u1 = q[:, :, off + 2 * j + 1]
            out[:, :, off + 2 * j] = u0 * c - u1 * s
            out[:, :, off + 2 * j + 1] = u0 * s + u1 * c
        off += da
    return out


# ---------------------------------------------------------------------------
# Attention: per head, softmax(q k^T / sqrt(d)) v; non-causal, no mask.
# ---------------------------------------------------------------------------
def attention(q, k, v) -> np.ndarray:
    """q [Sq, H, d], k and v [Sk, H, d] -> [Sq, H, d]."""
    q, k, v = _f(q), _f(k), _f(v)
    d = q.shape[-1]
    out = np.empty_like(q)
    for h in range(q.shape[1]):
        p = softmax_rows(q[:, h, :] @ k[:, h, :].T / np.sqrt(d))
        out[:, h, :] = p @ v[:, h, :]
    return out


# ---------------------------------------------------------------------------
# One DiT block.  Readings: modulation vectors are ordered (shift_a, scale_a,
# gate_a, shift_f, scale_f, gate_f); LayerNorm has no affine; cross-attention
# is preceded by a plain LayerNorm and is not gated; RoPE applies to self-
# attention q and k only.
# ---------------------------------------------------------------------------
def dit_block(x, c, mod, p: dict, cfg, pos, rows=None) -> np.ndarray:
    """x [S, D] residual stream, c [L, D] projected context, mod [6, D].
    Returns the block output at ``rows`` (all tokens when None)."""
    x = _f(x)
    c = _f(c)
    mod = _f(mod)
    S, D = x.shape
    H, d = cfg.heads, cfg.head_dim
    eps = cfg.ln_eps
    rows = np.arange(S) if rows is None else np.asarray(rows)
    shift_a, scale_a, gate_a, shift_f, scale_f, gate_f = mod

    # self-attention branch
    y = modulate(layer_norm(x, eps), shift_a, scale_a)
    wq, wk, wv = np.split(_f(p["qkv_w"]), 3, axis=0)
    bq, bk, bv = np.split(_f(p["qkv_b"]), 3)
    q = linear(y[rows], wq, bq).reshape(len(rows), H, d)
    k = linear(y, wk, bk).reshape(S, H, d)
    v = linear(y, wv, bv).reshape(S, H, d)
    q = rope_rotate(q, pos[rows], cfg.rope, cfg.rope_theta)
    k = rope_rotate(k, pos, cfg.rope, cfg.rope_theta)
    o = attention(q, k, v).reshape(len(rows), D)
    xr = x[rows] + gate_a * linear(o, p["o_w"], p["o_b"])

    # cross-attention branch
    y = layer_norm(xr, eps)
    qc = linear(y, p["cq_w"], p["cq_b"]).reshape(len(rows), H, d)
    wck, wcv = np.split(_f(p["ckv_w"]), 2, axis=0)
    bck, bcv = np.split(_f(p["ckv_b"]), 2)
    kc = linear(c, wck, bck).reshape(c.shape[0], H, d)
    vc = linear(c, wcv, bcv).reshape(c.shape[0], H, d)
    oc = attention(qc, kc, vc).reshape(len(rows), D)
    xr = xr + linear(oc, p["co_w"], p["co_b"])

    # MLP branch
    y = modulate(layer_norm(xr, eps), shift_f, scale_f)
    h = gelu_tanh(linear(y, p["w1"], p["b1"]))
    return xr + gate_f * linear(h, p["w2"], p["b2"])


def block_modulation(e, table) -> np.ndarray:
    """Reading: each block's six vectors are the shared projection e plus the
    block's own learned table."""
    return _f(e) + _f(table)


def context_projection(E, g: dict, cfg) -> np.ndarray:
    """Reading: one Linear text_dim -> D when the widths differ, else identity."""
    if "txt_w" in g and g["txt_w"] is not None and cfg.text_dim != cfg.hidden:
        return linear(E, g["txt_w"], g["txt_b"])
    return _f(E)


def final_layer(x, temb, g: dict, cfg) -> np.ndarray:
    """Reading: (shift_o, scale_o) = head_table + temb; LayerNorm, modulate and
    a Linear D -> patch_dim give velocity tokens [S, P]."""
    shift_o, scale_o = _f(g["head_table"]) + _f(temb)
    return linear(modulate(layer_norm(x, cfg.ln_eps), shift_o, scale_o), g["out_w"], g["out_b"])


def dit_forward(X, E, t: float, params: dict, cfg, return_tokens: bool = False):
    """Velocity V [C, F, H, W] of latents X [C, F, H, W] at timestep t under
    conditioning E [L, text_dim]."""
    g = params["global"]
    temb, e = time_embedding(t, g, cfg.freq_dim)
    c = context_projection(E, g, cfg)
    x = linear(patchify(X, cfg.patch), g["pe_w"], g["pe_b"])
    pos = token_positions(_grid(cfg))
    for b, p in enumerate(params["blocks"]):
        x = dit_block(x, c, block_modulation(e, p["table"]), p, cfg, pos)
    u = final_layer(x, temb, g, cfg)
    V = unpatchify(u, cfg.patch, (cfg.in_channels,) + tuple(cfg.latent))
    return (V, u) if return_tokens else V


# ---------------------------------------------------------------------------
# Euler update ("Model Configuration Conventions", section "Sampling And
# Geometry": flow-prediction denoisers).  Reading: the network predicts a
# velocity and one step moves X by (sigma_next - sigma) * V.
# ---------------------------------------------------------------------------
def euler_step(X, V, sigma: float, sigma_next: float) -> np.ndarray:
    return _f(X) + (F64(sigma_next) - F64(sigma)) * _f(V)


def denoise_step(X, E, t: float, sigma: float, sigma_next: float, params: dict, cfg):
    """One denoise step: (X_next, V)."""
    V = dit_forward(X, E, t, params, cfg)
    return euler_step(X, V, sigma, sigma_next), V


def denoise_step_cfg(X, E, E_neg, t: float, sigma: float, sigma_next: float, guidance: float,
                     params: dict, cfg):
    """One denoise step with classifier-free guidance: (X_next, V).

    The network runs twice on the same latents and timestep, once with the
    positive embeddings E and once with the negative ones E_neg (page "Support
    New Diffusion Models - SGLang Documentation": section 2 "Pipeline Config",
    the positive and negative condition kwargs; section 1 "Sampling Params",
    guidance_scale; section 4, the DenoisingStage field table,
    negative_prompt_embeds when CFG is used).  Reading (the pages print no
    formula): the guided velocity is V_neg + g (V_pos - V_neg), followed by the
    same Euler update as the unguided step."""
    V_pos = dit_forward(X, E, t, params, cfg)
    V_neg = dit_forward(X, E_neg, t, params, cfg)
    V = V_neg + float(guidance) * (V_pos - V_neg)
    return euler_step(X, V, sigma, sigma_next), V


def sample(X0, E, params: dict, cfg, n_steps: int, shift: float, first_steps=None):
    """Run the schedule from X0; returns X after ``first_steps`` steps (all
    when None)."""
    sig = flow_sigmas(n_steps, shift)
    ts = flow_timesteps(sig)
    X = _f(X0)
    last = n_steps if first_steps is None else int(first_steps)
    for k in range(last):
        X, _ = denoise_step(X, E, ts[k], sig[k], sig[k + 1], params, cfg)
    return X


def _grid(cfg):
    pf, ph, pw = cfg.patch
    f, h, w = cfg.latent
    return (f // pf, h // ph, w // pw)

"""Seeded synthetic inputs for latent-condensed MLA.

This module is shared by the oracle tests, the GPU tests and bench.py. It holds
no step of the method: only random draws, the rotary rotation used to
synthesise the decoupled position keys (the method reads k_R as stored data),
and the round-to-nearest-even conversion of stored values to bfloat16.

Recipe (one generator per tensor, numpy PCG64 seeded with 1000*cfg + id):
  id 1  latent c_KV rows            N(0, 1)             [B, L, 512]
  id 2  position keys before RoPE   N(0, 1)             [B, L, 64], then RoPE
        (base 10000, rotate-half pairs (i, i+32), position = token index)
  id 3  absorbed queries            N(0, 1/576)         [B, T, H, 576]
        optionally with a per-sequence shared direction u ~ N(0, rho/576)
        plus independent noise N(0, (1-rho)/576): the marginal stays
        N(0, 1/576) while the summary query becomes informative.
  id 4  W_UV                        N(0, 1/512)         [H, 512, 128]
  id 5  W_UK                        N(0, 1/512)         [H, 512, 128]
  id 6  needle rows (planted rows aligned with u, for unit-scale outputs)
  id 7  one pre-rotation position vector per sequence, N(0, 1) [B, 64], for
        inputs where position carries signal: every token's k_R is that
        vector rotated to the token's position, and a query's RoPE part is
        it rotated to the query's position (so the RoPE logit depends on the
        distance only).
  id 8  hidden states x             N(0, 1)             [T, d_model]
  id 9  projection weights          N(0, 1/d_model)     [576 + 192 H, d_model]
        (one row per output: c, the RoPE key, then per head 128 no-RoPE
        and 64 RoPE query outputs), so every projected value is ~N(0, 1)
Values are drawn in float32 and, for bf16 runs, rounded once on the host, so
the oracle and the GPU read identical numbers.
"""
from __future__ import annotations

import numpy as np

D_C = 512   # latent c_KV width
D_R = 64    # decoupled RoPE key width
D_ROW = D_C + D_R
D_V = 128   # per-head value width after the up-projection

ID_C, ID_K, ID_Q, ID_WUV, ID_WUK, ID_NEEDLE, ID_POS, ID_X, ID_WPROJ = 1, 2, 3, 4, 5, 6, 7, 8, 9


def rng(cfg: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg + tensor_id))


def bf16_round(x) -> np.ndarray:
    """float32 array holding the bfloat16 nearest to x (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16_round(x)."""
    return (bf16_round(x).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rope(k: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis (64 wide) by position pos (rotate-half pairing)."""
    half = k.shape[-1] // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / k.shape[-1])
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang).astype(np.float32)
    sin = np.sin(ang).astype(np.float32)
    k1, k2 = k[..., :half], k[..., half:]
    return np.concatenate([k1 * cos - k2 * sin, k1 * sin + k2 * cos], axis=-1).astype(np.float32)


def latent_cache(cfg: int, B: int, L: int, bf16: bool = True, pos0: int = 0):
    """(c [B,L,512], kr [B,L,64]) float32; bf16-representable when bf16=True."""
    c = rng(cfg, ID_C).standard_normal((B, L, D_C), dtype=np.float32)
    k = rng(cfg, ID_K).standard_normal((B, L, D_R), dtype=np.float32)
    k = rope(k, np.arange(pos0, pos0 + L))
    if bf16:
        c, k = bf16_round(c), bf16_round(k)
    return c, k


def positional_keys(cfg: int, B: int, L: int, bf16: bool = True) -> np.ndarray:
    """k_R [B, L, 64]: the sequence's position vector rotated to each token position."""
    v = rng(cfg, ID_POS).standard_normal((B, D_R), dtype=np.float32)
    pos = np.arange(L)
    k = np.stack([rope(np.broadcast_to(v[b], (L, D_R)), pos) for b in range(B)])
    return bf16_round(k) if bf16 else k


def positional_query_rope(cfg: int, B: int, pos: int, gain: float, bf16: bool = True) -> np.ndarray:
    """[B, 64]: gain times the sequence's position vector rotated to position pos."""
    v = rng(cfg, ID_POS).standard_normal((B, D_R), dtype=np.float32) * np.float32(gain)
    q = np.stack([rope(v[b][None], np.array([pos]))[0] for b in range(B)])
    return bf16_round(q) if bf16 else q


def shared_direction(cfg: int, B: int) -> np.ndarray:
    """Per-sequence unit direction u/|u| used by correlated queries and needles."""
    u = rng(cfg, ID_Q + 100).standard_normal((B, D_ROW))
    return (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)


def queries(cfg: int, B: int, T: int, H: int, rho: float = 0.0, bf16: bool = True,
            stream: int = 0) -> np.ndarray:
    """Absorbed queries [B, T, H, 576] with marginal N(0, 1/576).

    rho > 0 mixes in a per-sequence shared direction (see module doc). `stream`
    selects an independent draw (e.g. one per decode step) from the same cfg.
    """
    g = rng(cfg, ID_Q + 1000 * stream)
    eps = g.standard_normal((B, T, H, D_ROW), dtype=np.float32)
    q = eps * np.float32(np.sqrt((1.0 - rho) / D_ROW))
    if rho > 0.0:
        u = shared_direction(cfg, B) * np.float32(np.sqrt(rho))  # |u|^2 = rho ~ 576 * rho/576
        q += u[:, None, None, :]
    if bf16:
        q = bf16_round(q)
    return q


def plant_needles(cfg: int, c: np.ndarray, kr: np.ndarray, n_per_seq: int, logit: float,
                  lo: int, hi: int, bf16: bool = True):
    """Overwrite n_per_seq rows per sequence in [lo, hi) with rows beta*u.

    beta is chosen so that a query equal to the shared direction scaled by
    sqrt(rho)=1 would see a logit of about `logit`; returns the positions.
    """
    B = c.shape[0]
    u = shared_direction(cfg, B)
    g = rng(cfg, ID_NEEDLE)
    pos = np.stack([np.sort(g.choice(np.arange(lo, hi), size=n_per_seq, replace=False))
                    for _ in range(B)])
    for b in range(B):
        row = (u[b] * np.float32(logit)).astype(np.float32)
        if bf16:
            row = bf16_round(row)
        c[b, pos[b]] = row[:D_C]
        kr[b, pos[b]] = row[D_C:]
    return pos


def w_uv(cfg: int, H: int, bf16: bool = True) -> np.ndarray:
    w = rng(cfg, ID_WUV).standard_normal((H, D_C, D_V), dtype=np.float32) * np.float32(1.0 / np.sqrt(D_C))
    return bf16_round(w) if bf16 else w


def w_uk(cfg: int, H: int, bf16: bool = True) -> np.ndarray:
    w = rng(cfg, ID_WUK).standard_normal((H, D_C, D_V), dtype=np.float32) * np.float32(1.0 / np.sqrt(D_C))
    return bf16_round(w) if bf16 else w


def hidden_states(cfg: int, T: int, d_model: int, bf16: bool = True) -> np.ndarray:
    x = rng(cfg, ID_X).standard_normal((T, d_model), dtype=np.float32)
    return bf16_round(x) if bf16 else x


def w_proj(cfg: int, H: int, d_model: int, bf16: bool = True) -> np.ndarray:
    w = (rng(cfg, ID_WPROJ).standard_normal((D_ROW + 192 * H, d_model), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(d_model)))
    return bf16_round(w) if bf16 else w


# ------------------------------------------------------------------------
# Device-side generation for the benchmark's large workloads (same recipe,
# torch's Philox generator instead of PCG64, so values differ from the numpy
# draws but follow the same distributions). The benchmark's CPU baseline
# copies the sequences it samples back to the host.
def latent_cache_torch(seed: int, B: int, L: int, device="cuda", dtype=None):
    """Packed [B, L, 576] cache: N(0,1) c_KV and RoPE-rotated N(0,1) k_R."""
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((B, L, D_ROW), dtype=dtype, device=device)
    step = max(1, (1 << 24) // max(1, L * D_ROW))  # bound the fp32 temporaries
    half = D_R // 2
    inv = 10000.0 ** (-torch.arange(half, device=device, dtype=torch.float64) * 2.0 / D_R)
    ang = torch.arange(L, device=device, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    for b0 in range(0, B, step):
        b1 = min(B, b0 + step)
        x = torch.randn((b1 - b0, L, D_ROW), generator=g, device=device, dtype=torch.float32)
        k1, k2 = x[..., D_C:D_C + half].clone(), x[..., D_C + half:].clone()
        x[..., D_C:D_C + half] = k1 * cos - k2 * sin
        x[..., D_C + half:] = k1 * sin + k2 * cos
        out[b0:b1] = x.to(dtype)
    return out


def queries_torch(seed: int, shape, device="cuda", dtype=None):
    """Absorbed queries N(0, 1/576) of the given shape (last axis 576)."""
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            * (1.0 / np.sqrt(D_ROW))).to(dtype)


def w_uv_torch(seed: int, H: int, device="cuda", dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn((H, D_C, D_V), generator=g, device=device, dtype=torch.float32)
            * (1.0 / np.sqrt(D_C))).to(dtype)


def projection_torch(seed: int, T: int, d_model: int, H: int, device="cuda", dtype=None):
    """Hidden states x [T, d] ~ N(0, 1), projection weights [576 + 192 H, d]
    ~ N(0, 1/d) and W_UK [H, 512, 128] ~ N(0, 1/512)."""
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((T, d_model), generator=g, device=device, dtype=torch.float32).to(dtype)
    w = (torch.randn((D_ROW + 192 * H, d_model), generator=g, device=device, dtype=torch.float32)
         * (1.0 / np.sqrt(d_model))).to(dtype)
    wuk = (torch.randn((H, D_C, D_V), generator=g, device=device, dtype=torch.float32)
           * (1.0 / np.sqrt(D_C))).to(dtype)
    return x, w, wuk

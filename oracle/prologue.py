"""Plain CPU oracle for the attention-layer prologue: q/k RMSNorm, RoPE, store.

TEST INFRASTRUCTURE ONLY — see ``oracle/__init__.py``.  Nothing in the
library imports this module; it imports nothing from the library.

Source: "Mini-SGLang complete analysis" (blog.rzhang-lab.cn):
  - §4.6.7, the attention layer's forward: the merged qkv projection output
    is split into q, k, v; for models with q/k norms (Qwen3) q and k are
    RMS-normalised per head in place; RoPE is applied in place to q and k at
    the batch's positions; the attention backend then stores k and v into
    the paged pool at ``out_loc`` before attending;
  - §4.5.6, one RoPE instance (one cos/sin cache of max_position x
    rotary_dim) is shared by every layer.

Readings where the pages are silent:
  * RMSNorm of a head vector x (length D) with weight w:
    ``x / sqrt(mean(x^2) + eps) * w`` (eps = 1e-6 in the workloads);
  * RoPE rotates the pairs (x[i], x[i + D/2]) ("rotate half") by the angle
    ``pos * theta_i``, theta_i = base^(-2i/D), over the whole head dim; the
    cache row of position p holds cos(p theta_i) in columns [0, D/2) and
    sin(p theta_i) in [D/2, D) (fp32, built by the input generator);
  * the result is computed exactly (float64 here) and rounded to bf16 once.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64


def rope_cache(max_position: int, rotary_dim: int, base: float) -> np.ndarray:
    """cos/sin table [max_position, rotary_dim] float64: row p holds
    cos(p theta_i) then sin(p theta_i), theta_i = base^(-2i/rotary_dim),
    i < rotary_dim/2.  [MSCA §4.5.6]"""
    half = rotary_dim // 2
    theta = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def rms_norm(x: np.ndarray, weight: np.ndarray | None, eps: float) -> np.ndarray:
    """x [..., D] float64; weight [D] float64 or None (no norm)."""
    if weight is None:
        return x
    rms = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / rms * weight


def rope(x: np.ndarray, positions: np.ndarray, cos_sin_cache: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE.  x [T, H, D] float64, positions [T], cache [P, D]."""
    D = x.shape[-1]
    half = D // 2
    c = cos_sin_cache[np.asarray(positions, np.int64)].astype(np.float64)
    cos = c[:, None, :half]
    sin = c[:, None, half:]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def qk_norm_rope_store(qkv_bits: np.ndarray, num_q_heads: int, num_kv_heads: int,
                       q_norm_w_bits, k_norm_w_bits, eps: float, positions: np.ndarray,
                       cos_sin_cache: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                       out_loc: np.ndarray):
    """The prologue of one attention layer for T tokens.

    qkv_bits: [T, (Hq + 2 Hkv) * D] bf16 bits (q heads, then k heads, then v
    heads, as the merged projection lays them out); norm weights: [D] bf16
    bits or None; k_pool / v_pool: [slots, Hkv, D] bf16 bits (not modified).
    Returns (q [T, Hq, D] float64, k [T, Hkv, D] float64, new K pool bits,
    new V pool bits): the new pools hold k rounded to bf16 (RNE) and v
    copied, at out_loc.  [MSCA §4.6.7, §4.5.6]
    """
    from .attention import f64_to_bf16_rne, store_kv
    T = qkv_bits.shape[0]
    Hq, Hkv = num_q_heads, num_kv_heads
    D = qkv_bits.shape[1] // (Hq + 2 * Hkv)
    x = bf16_to_f64(qkv_bits).reshape(T, Hq + 2 * Hkv, D)
    q, k = x[:, :Hq], x[:, Hq:Hq + Hkv]
    v_bits = qkv_bits.reshape(T, Hq + 2 * Hkv, D)[:, Hq + Hkv:]
    qw = None if q_norm_w_bits is None else bf16_to_f64(q_norm_w_bits)
    kw = None if k_norm_w_bits is None else bf16_to_f64(k_norm_w_bits)
    q = rope(rms_norm(q, qw, eps), positions, cos_sin_cache)
    k = rope(rms_norm(k, kw, eps), positions, cos_sin_cache)
    kp, vp = store_kv(k_pool, v_pool, f64_to_bf16_rne(k), np.ascontiguousarray(v_bits), out_loc)
    return q, k, kp, vp

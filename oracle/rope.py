"""Rotary position embedding, rotate-half form, float64 (test infrastructure).

Source: neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2) and the
ruixiangma.github.io blog, 方法 › 文档级RoPE: positions are reset to 0 at the
start of every document (document-wise / parallel RoPE); the active context
is shifted by k (global RoPE).  The pages do not print the RoPE formula.
Reading taken: the rotate-half pairing used by the Qwen3 backbone the pages
name -- element i pairs with i + d/2, inv_freq_i = theta^(-2i/d) for
i < d/2, angle = pos * inv_freq_i (computed in float64),

    x'_i       = x_i       cos(angle) - x_{i+d/2} sin(angle)
    x'_{i+d/2} = x_{i+d/2} cos(angle) + x_i       sin(angle)

Pinned by tests/test_oracle_rope.py: identity at position 0 (bit-exact),
the complex-multiplication form (x_i + j x_{i+d/2}) * exp(j angle), norm
preservation, the relative-position identity of dot products, and closed
forms of inv_freq.
"""

import numpy as np


def inv_freq(d, theta):
    if d % 2:
        raise ValueError("head dim must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def rope_angles(pos, d, theta):
    """angles[..., i] = pos * inv_freq_i in float64; pos any integer array."""
    p = np.asarray(pos, dtype=np.float64)
    return p[..., None] * inv_freq(d, theta)


def rope(x, pos, theta):
    """Rotate x[..., d] by positions pos, broadcastable to x.shape[:-1]
    (e.g. x of shape [T, H, d] with pos of shape [T, 1])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)

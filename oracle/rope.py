"""Rotary position embedding, float64.

AstrAI docs/developer/internals.md, "Rotary Position Embedding (RoPE)":
q_i = R_i W_q x_i and k_j = R_j W_k x_j, so that q_i^T k_j depends only on i - j;
the rotation is a complex multiplication by a cos/sin table ``freqs_cis`` of
shape [max_len, dim/2, 2] holding [cos, sin] pairs, indexed by position.
docs/guides/inference.md, "Rotary Embedding Backend": the fallback views the
input as complex numbers, multiplies and views back as real, which makes the
complex number of pair i the adjacent elements (x[2i], x[2i+1]).
AstrAI paper, "Model Architecture" table: theta = 10 000, citing RoFormer,
whose frequencies are theta^(-2i/d) for i = 0 .. d/2 - 1 over the whole head.

Readings where the pages are silent: the rotation covers the whole head_dim,
with no scaling; the table's angles and cos/sin are computed in float64 and
rounded to float32 (the pages fix the stored table as float32), and the
method rotates with those stored float32 entries: ``rotate`` is the exact
rotation (pinned by the invariants), ``rotate_with_table`` the method's
table lookup plus complex multiply.
"""

import numpy as np


def inv_freq(head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """theta^(-2i/head_dim), i = 0 .. head_dim/2 - 1 (float64)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def angles(positions, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Rotation angle of every (position, pair): positions[..., None] * inv_freq."""
    pos = np.asarray(positions, dtype=np.float64)
    return pos[..., None] * inv_freq(head_dim, theta)


def freqs_cis(max_pos: int, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """The [max_pos, head_dim/2, 2] table of [cos, sin], float64."""
    a = angles(np.arange(max_pos), head_dim, theta)
    return np.stack([np.cos(a), np.sin(a)], axis=-1)


def freqs_cis_f32(max_pos: int, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """The table as the method stores it: float32 [cos, sin] (float64 values
    rounded to nearest float32), returned as float64 holding those values."""
    return freqs_cis(max_pos, head_dim, theta).astype(np.float32).astype(np.float64)


def rotate_with_table(x, positions, table) -> np.ndarray:
    """The method's rotation: look up [cos, sin] = table[pos, i] and multiply the
    complex number (x[2i], x[2i+1]) by cos + i sin, in float64.

    With float32 table entries and inputs of at most float32 precision every
    product is exact in float64, so the result is the exact rotation by the
    stored table up to one float64 rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    t = np.asarray(table, dtype=np.float64)[np.asarray(positions)]     # [..., D/2, 2]
    c, s = t[..., 0], t[..., 1]
    re, im = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (x.shape[-1],)), dtype=np.float64)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def rotate(x, positions, theta: float = 10000.0) -> np.ndarray:
    """Rotate each adjacent pair (x[2i], x[2i+1]) of the last axis by the angle
    positions * theta^(-2i/D): (a, b) -> (a cos - b sin, a sin + b cos).

    ``x`` is [..., D]; ``positions`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = angles(positions, d, theta)
    c, s = np.cos(a), np.sin(a)
    re, im = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, c.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def rotate_backward_with_table(g, positions, table) -> np.ndarray:
    """Gradient of ``rotate_with_table`` with respect to its input, given the
    gradient ``g`` of its output (the backward pass autograd forms for the
    complex-multiply path the pages keep for training; internals.md, "Rotary
    Position Embedding (RoPE)").  The forward map of one pair is the matrix
    [[c, -s], [s, c]]; its gradient is the transpose [[c, s], [-s, c]]
    applied to g: (ga, gb) -> (ga c + gb s, gb c - ga s), i.e. multiplication
    by the complex conjugate of the same table entry.
    """
    g = np.asarray(g, dtype=np.float64)
    t = np.asarray(table, dtype=np.float64)[np.asarray(positions)]
    c, s = t[..., 0], t[..., 1]
    ga, gb = g[..., 0::2], g[..., 1::2]
    out = np.empty(np.broadcast_shapes(g.shape, c.shape[:-1] + (g.shape[-1],)), dtype=np.float64)
    out[..., 0::2] = ga * c + gb * s
    out[..., 1::2] = gb * c - ga * s
    return out

"""fp64 CPU oracle for rotary position embedding around attention (test infrastructure;
see the package header).

Page "A transformer in PTX", section "The model": after the fused QKV matmul the queries
and keys are rotated with RoPE, in place in the bf16 QKV buffer, before causal attention.
The pages give no formula; the reading taken here is the usual one: the head dimension
splits into pairs (x[2i], x[2i+1]), pair i of token t turns by the angle whose cosine and
sine are cos[t][i] and sin[t][i] (tables the caller supplies):

    y[2i]   = x[2i] cos - x[2i+1] sin
    y[2i+1] = x[2i] sin + x[2i+1] cos

and the rotated values are stored as bf16, as the pages' in-place pass stores them. The
pages fix no precision for the rotation itself, so the oracle's rotated tensor is the exact
rotation (float64 from the bf16 inputs and the fp32 tables: each product is exact, and
their sum rounds at 53 bits, far below bf16's 8) rounded to bf16, to nearest even. The
gradient with respect to the unrotated input is the transposed rotation of the gradient
with respect to the rotated one (the bf16 rounding passes gradients through unchanged):

    g_x[2i]   =  g_y[2i] cos + g_y[2i+1] sin
    g_x[2i+1] = -g_y[2i] sin + g_y[2i+1] cos
"""
import numpy as np

from . import bf16_to_f64
from .gemm import round_to_bf16


def _pairs(x):
    x = np.asarray(x, dtype=np.float64)
    return x[..., 0::2], x[..., 1::2]


def _tables(cos, sin, shape):
    """Broadcast [T][d/2] tables over x of shape [B][T][H][d]."""
    c = np.asarray(cos, dtype=np.float64)[None, :, None, :]
    s = np.asarray(sin, dtype=np.float64)[None, :, None, :]
    assert c.shape[1] == shape[1] and c.shape[3] * 2 == shape[3], (c.shape, shape)
    return c, s


def rotate(x, cos, sin):
    """y = R(t) x for float64 x [B][T][H][d]."""
    x0, x1 = _pairs(x)
    c, s = _tables(cos, sin, np.shape(x))
    y = np.empty(np.shape(x), dtype=np.float64)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def rotate_back(g, cos, sin):
    """g_x = R(t)^T g_y for float64 g [B][T][H][d]."""
    g0, g1 = _pairs(g)
    c, s = _tables(cos, sin, np.shape(g))
    y = np.empty(np.shape(g), dtype=np.float64)
    y[..., 0::2] = g0 * c + g1 * s
    y[..., 1::2] = -g0 * s + g1 * c
    return y


def rotate_bf16(x_bits, cos, sin):
    """The rotated bf16 tensor (as float64 values) of a bf16 input given as bit patterns."""
    return round_to_bf16(rotate(bf16_to_f64(np.ascontiguousarray(x_bits, dtype=np.uint16)), cos, sin))

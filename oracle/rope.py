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
rounding to bf16 is a quantisation, so the oracle takes it in the precision the kernels
compute the rotation in (the pages fix none): y[2i] = fma(x[2i], cos, -fl(x[2i+1] sin)) and
y[2i+1] = fma(x[2i], sin, fl(x[2i+1] cos)) in float32, then bf16 (round to nearest even). The
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


def fma32(a, b, c):
    """fl32(a*b + c) for float32 arrays: the exact value rounded once to float32 (nearest,
    ties to even), as a fused multiply-add computes it. a*b is exact in float64 (24 + 24
    significant bits); TwoSum gives s + err == a*b + c exactly; s rounded to float32 is
    the answer unless s sits exactly halfway between two float32 numbers while err != 0,
    in which case the exact value lies on err's side of it."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bb = s - p
    err = (p - (s - bb)) + (c - bb)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    other = np.where(r64 > s, np.nextafter(r, np.float32(-np.inf)), np.nextafter(r, np.float32(np.inf)))
    o64 = other.astype(np.float64)
    halfway = (r64 + o64) / 2.0 == s
    fix = halfway & (err != 0)
    up = np.maximum(r, other)
    down = np.minimum(r, other)
    return np.where(fix, np.where(err > 0, up, down), r)


def rotate_bf16_fp32(x_bits, cos, sin):
    """The rotated bf16 tensor as the kernels compute it (float32 rotation, see the module
    docstring), as float64 values, from bf16 bit patterns [B][T][H][d]."""
    x = bf16_to_f64(np.ascontiguousarray(x_bits, dtype=np.uint16)).astype(np.float32)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    c = np.asarray(cos, dtype=np.float32)[None, :, None, :]
    s = np.asarray(sin, dtype=np.float32)[None, :, None, :]
    y = np.empty(x.shape, dtype=np.float32)
    y[..., 0::2] = fma32(x0, c, -(x1 * s))
    y[..., 1::2] = fma32(x0, s, x1 * c)
    return round_to_bf16(y.astype(np.float64))

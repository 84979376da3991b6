"""Row samples that cover every tile, and per-element error bounds, for the
GPU parity tests.

Rows.  The grouped GEMM cuts each segment (the rows of one (source block,
expert) pair, offsets[g] .. offsets[g+1]) into row tiles of 256 rows, and a
tile of the grid's last round may run as two 128-row halves.  covering_rows
picks, from the ORACLE's offsets (routing is compared bit for bit
separately, so they are the GPU's too, but no oracle input is taken from the
GPU), one seeded row in every 128-row half of every row tile, plus each
segment's last row; comparing whole rows (every column) then covers every
(row tile, column tile) of both layers, including the last round's half
tiles and its k-split tiles.

Bounds.  u = 2^-24 (f32 unit roundoff).  Products of two bf16 values (and
of two e4m3 values with their power-of-two scales) are exact in f32, so a
GPU sum of K products differs from the exact sum only by the accumulation.
For the bf16 matrix cores and f32 FMAs it is bounded by ACC_ULPS * u *
(sum of |terms|) (measured on MI355X: at most 4.4 u, median 0.12 u, over
2.2M Layer1 elements of three layers):  under
the standard model of independent rounding errors (each addition rounds by
a uniform fraction of u times the partial sum, and the partial sums of
zero-mean terms grow like a random walk) the error's standard deviation is
about u/4 of the sum of |terms|, so 8 u is a 30-sigma allowance, whatever
the summation order (the matrix cores' blocks, a split of the k range).
Through SwiGLU h = silu(g) u with |silu'| <= 1.1 everywhere:
    |h_gpu_f32 - h| <= 1.1 eg (|u| + eu) + |silu(g)| eu + 8 u |h| = D
(eg, eu the gate and up allowances; 8 u |h| the f32 exponential, reciprocal
and products of the epilogue), and both sides then round to bf16 (unit
roundoff 2^-8), so
    |bf16(h_gpu) - bf16(h)| <= 2^-8 (2 |h| + D) + D.
Layer1 on the GPU's own Hact:
    |Y_gpu - Y_ref| <= sum_f |Hact_gpu - Hact_ref| |W| + 8 u sum_f |Hact_gpu W|,
and the combine (k fused multiply-adds from zero, in order; the f32
weights may differ from the oracle's by their rounding):
    |out_gpu - out_ref| <= sum_j (|w_j| bound_Y_j + |w_j - w_ref_j| |Y_ref_j|)
                           + k u sum_j |w_j Y_gpu_j|.
The exact gate/up sums and the sums of |terms| are recomputed here in f64
(torch on the GPU) for the compared rows only; they feed the bound, never
the expected value, which is the oracle's.
"""
from __future__ import annotations

import numpy as np
import torch

U32 = 2.0 ** -24
ACC_ULPS = 8.0
# The fp8 (MXFP8) matrix cores sum each block of 64 scaled products with less
# than f32 precision; how is not documented.  Measured on MI355X (the GPU's
# own Hact and W_down codes against the exact f64 sum of their dequantised
# products; 12 layers, K = 256 .. 14336, 2M elements): at most about 820 f32
# ulps of the sum of |terms| (median 8 to 30, shrinking with K as the blocks'
# errors average out), whether or not e4m3 subnormal codes are counted.  The
# allowance is 2^-13 of the sum of |terms| (2048 ulps): a model taken from
# measurement, not from a specification.  A wrong block scale moves a Y
# element by at least the block's 32 terms, 2^-9 of the sum or more for
# F <= 16384, so it is still caught.
ACC_ULPS_FP8 = 2048.0
BF16_U = 2.0 ** -8
TILE = 256
HALF = 128


def covering_rows(offsets, seed):
    """Seeded sorted rows covering every 128-row half of every 256-row tile
    of every segment, and each segment's last row.  Returns (rows, number of
    row tiles, number of halves covered)."""
    rng = np.random.default_rng(seed)
    offsets = np.asarray(offsets, np.int64)
    rows, tiles, halves = [], 0, 0
    for g in range(len(offsets) - 1):
        a, n = int(offsets[g]), int(offsets[g + 1] - offsets[g])
        for m0 in range(0, n, TILE):
            tiles += 1
            for h0 in (m0, m0 + HALF):
                h1 = min(h0 + HALF, n)
                if h0 < h1:
                    rows.append(a + int(rng.integers(h0, h1)))
                    halves += 1
        if n:
            rows.append(a + n - 1)
    return np.unique(np.asarray(rows, np.int64)), tiles, halves


def experts_of(offsets, rows, EL):
    """Weight slot of each sorted row (segment g uses slot g % EL)."""
    g = np.searchsorted(np.asarray(offsets, np.int64), rows, side="right") - 1
    return (g % EL).astype(np.int64)


def _groups(experts):
    for e in np.unique(experts):
        yield int(e), torch.from_numpy(np.nonzero(experts == e)[0]).cuda()


def gate_up_sums(x_rows, w_gate, w_up, experts):
    """Exact (f64) gate and up sums of the given token rows [n, H] (device
    tensor) with their experts' weights [EL, F, H], and the sums of |terms|."""
    n, F = x_rows.shape[0], w_gate.shape[1]
    out = {k: torch.zeros((n, F), dtype=torch.float64, device="cuda") for k in ("g", "u", "sg", "su")}
    for e, sel in _groups(experts):
        X = x_rows[sel].double()
        for key, W in (("g", w_gate[e]), ("u", w_up[e])):
            Wd = W.double()
            out[key][sel] = X @ Wd.t()
            out["s" + key][sel] = X.abs() @ Wd.abs().t()
            del Wd
    return out


def silu64(z):
    return z / (1.0 + torch.exp(-z))


def hact_allowance(sums, bf16):
    """Per-element bound on |Hact_gpu - Hact_oracle| (see the module doc);
    bf16: both sides round the activation to bf16."""
    g, u, sg, su = sums["g"], sums["u"], sums["sg"], sums["su"]
    eg, eu = ACC_ULPS * U32 * sg, ACC_ULPS * U32 * su
    h = silu64(g) * u
    D = 1.1 * eg * (u.abs() + eu) + silu64(g).abs() * eu + 8 * U32 * h.abs()
    allow = D + 1e-12 * h.abs() + 1e-30
    if bf16:
        allow = allow + BF16_U * (2 * h.abs() + D)
    return allow


def y_allowance(h_gpu, h_ref, experts, w_of, H, acc_ulps=ACC_ULPS):
    """Per-element bound on |Y_gpu - Y_oracle| for rows whose activations
    are h_gpu (the GPU's) and h_ref (the oracle's), both f64 [n, F] device
    tensors; w_of(e) gives expert e's down weights as f64 [H, F]; acc_ulps
    the accumulation allowance (ACC_ULPS_FP8 for the fp8 matrix cores)."""
    n = h_gpu.shape[0]
    out = torch.zeros((n, H), dtype=torch.float64, device="cuda")
    for e, sel in _groups(experts):
        W = w_of(e).abs()
        b = (h_gpu[sel] - h_ref[sel]).abs() @ W.t() + acc_ulps * U32 * (h_gpu[sel].abs() @ W.t())
        out[sel] = b + 1e-12 * (h_ref[sel].abs() @ W.t()) + 1e-30
        del W
    return out


def out_allowance(w_gpu, w_ref, y_gpu, y_ref, y_bound, kept):
    """Per-element bound on |out_gpu - out_oracle| for n tokens: w_* [n, k]
    (numpy), y_* and y_bound [n * k, H] (numpy, pair (i, j) at row i*k + j),
    kept [n, k] the pairs held here."""
    n, k = w_gpu.shape
    H = y_gpu.shape[1]
    yg, yr, yb = (a.reshape(n, k, H) for a in (y_gpu, y_ref, y_bound))
    m = kept[:, :, None].astype(np.float64)
    wg, dw = np.abs(w_gpu)[:, :, None], np.abs(w_gpu.astype(np.float64) - w_ref.astype(np.float64))[:, :, None]
    b = (m * (wg * yb + dw * np.abs(yr))).sum(axis=1) + k * U32 * (m * wg * np.abs(yg)).sum(axis=1)
    return b + 1e-30


def check_within(name, got, ref, allow):
    """Assert |got - ref| <= allow element-wise; print the tightest ratio."""
    got, ref, allow = (np.asarray(a, np.float64) for a in (got, ref, allow))
    d = np.abs(got - ref)
    ratio = float(np.max(d / allow)) if d.size else 0.0
    print(f"[bound] {name}: {d.size} elements, max |d| {d.max() if d.size else 0:.3e}, "
          f"max |d|/bound {ratio:.3f}", flush=True)
    bad = np.argwhere(d > allow)
    assert bad.size == 0, (name, bad[:5].tolist(), d[tuple(bad[0])], allow[tuple(bad[0])])

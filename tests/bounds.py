"""Derived tolerances shared by the GPU parity tests.

End to end, the decode scores the cache against q_abs as the absorption kernel stored it:
its latent part (columns < d_c) rounded once to bf16, the RoPE part copied exactly.  bf16
keeps 8 significant bits, so each rounded component is within u = 2^-8 of its exact value
(relative), and the scaled logit of row j moves by at most

    u * scale * sum_c |q_abs[n, i, c]| * |c_j[c]|        (c < d_c).

A log-sum-exp is 1-Lipschitz in the largest-entry norm of its arguments, so the same maximum
over the visible rows bounds the shift of lse[n, i].  The decode's own rounding (fp32 sums of
exact bf16 products, exp2, the merge) is held to the per-call 1e-3 on top.
"""

import numpy as np

BF16_UNIT_ROUNDOFF = 2.0 ** -8


def lse_bound(q_abs, c_kv, offsets, q_per_seq: int, scale: float, floor: float = 1e-3) -> np.ndarray:
    """Per-(query, head) bound on |lse_gpu - lse_oracle| for a decode fed a bf16-rounded q_abs.

    q_abs: [n_q, n_h, d_c + d_r] (exact values; only the first d_c columns are rounded);
    c_kv: [rows, d_c] cache latents; offsets: [B+1].  Returns [n_q, n_h].
    """
    d_c = c_kv.shape[1]
    q = np.abs(np.asarray(q_abs, np.float64)[..., :d_c])
    out = np.zeros(q.shape[:2])
    for b in range(len(offsets) - 1):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        C = np.abs(np.asarray(c_kv[lo:hi], np.float64))
        for r in range(q_per_seq):
            n = b * q_per_seq + r
            vis = (hi - lo) - q_per_seq + r + 1
            if vis <= 0:
                continue
            out[n] = (q[n] @ C[:vis].T).max(axis=1)
    return BF16_UNIT_ROUNDOFF * scale * out + floor


def check_lse(what, got, ref, bound, say=print):
    """Element-wise |got - ref| <= bound where both are finite; -inf patterns must agree."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape == bound.shape, (what, got.shape, ref.shape, bound.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), what
    d = np.abs(got[fin] - ref[fin])
    err = float(d.max()) if fin.any() else 0.0
    ratio = float((d / bound[fin]).max()) if fin.any() else 0.0
    say(f"    {what}: max|d| = {err:.3e}, max |d|/bound = {ratio:.3f} (bound {float(bound.min()):.2e}.."
        f"{float(bound.max()):.2e})")
    assert ratio <= 1.0, f"{what}: |d| exceeds the derived bound (ratio {ratio})"
    return err, ratio

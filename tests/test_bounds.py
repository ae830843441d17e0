"""CPU checks of the derived end-to-end lse tolerance (tests/bounds.py).

The bound says: rounding the latent part of q_abs to bf16 moves lse[n, i] by at most
2^-8 * scale * max_j sum_c |q_abs[n, i, c]| |c_j[c]|.  Here the oracle itself decodes with the
exact and with the rounded q_abs (fp64 throughout), so the bound is checked against the
very perturbation it claims to cover, with no GPU arithmetic on either side.
"""

import numpy as np
import pytest

import oracle as O
from bounds import lse_bound
from mla_latent_kv_20_amd import workloads as W


@pytest.mark.parametrize("name", ["dsv2_small", "dsv2_small_mtp", "dsv2_ragged_small"])
def test_rounded_query_shift_within_bound(name):
    w = W.make_config(name)
    scale = O.default_scale(w.d_h, w.d_r)
    q_exact = O.absorb_q(w.f64("q_c"), w.f64("q_r"), w.f64("w_uk"))
    q_round = q_exact.copy()
    q_round[..., :w.d_c] = W.to_f64(W.round_to_storage(q_exact[..., :w.d_c], W.BF16), W.BF16)
    _, l_exact = O.attend_latent(q_exact, w.f64("c_kv"), w.f64("k_r"), w.offsets, w.q_per_seq, scale)
    _, l_round = O.attend_latent(q_round, w.f64("c_kv"), w.f64("k_r"), w.offsets, w.q_per_seq, scale)
    shift = np.abs(l_round - l_exact)
    bound = lse_bound(q_exact, w.f64("c_kv"), w.offsets, w.q_per_seq, scale, floor=0.0)
    assert np.all(shift <= bound)
    # not vacuous: the worst observed shift is a visible fraction of the worst case (about
    # a tenth on these inputs: the rounding errors of 512 components have mixed signs)
    assert float(np.max(shift / bound)) > 1e-2


def test_rounding_unit_is_reached():
    # bf16 keeps 8 significant bits: round-to-nearest errors reach (almost) 2^-8 relative,
    # so a 2^-9 unit would under-cover single components
    w = W.make_config("dsv2_small")
    q = O.absorb_q(w.f64("q_c"), w.f64("q_r"), w.f64("w_uk"))[..., :w.d_c]
    qr = W.to_f64(W.round_to_storage(q, W.BF16), W.BF16)
    rel = np.abs(qr - q)[q != 0] / np.abs(q[q != 0])
    assert rel.max() <= 2.0 ** -8 and rel.max() > 2.0 ** -9


def test_bound_tracks_the_rounding_unit():
    # doubling every row doubles the bound; a zero query gives a zero bound
    w = W.make_config("dsv2_small")
    scale = O.default_scale(w.d_h, w.d_r)
    q = O.absorb_q(w.f64("q_c"), w.f64("q_r"), w.f64("w_uk"))
    b1 = lse_bound(q, w.f64("c_kv"), w.offsets, w.q_per_seq, scale, floor=0.0)
    b2 = lse_bound(q, 2.0 * w.f64("c_kv"), w.offsets, w.q_per_seq, scale, floor=0.0)
    assert np.allclose(b2, 2.0 * b1)
    assert np.all(lse_bound(0.0 * q, w.f64("c_kv"), w.offsets, w.q_per_seq, scale, floor=0.0) == 0.0)

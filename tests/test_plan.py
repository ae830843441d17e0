"""mla_plan_splits on the host (no GPU): the plans it picks for the measured workloads, the
rules every plan keeps, and its argument checks.

The expected plans are the ones measured fastest on MI355X for those workloads (graph-replayed
decode steps, one box per comparison): 8 x 512 rows at 32 x 4096, 64 x 2048 at 4 x 131072,
one split with 4 queries per sequence and for the prefill, and 4 x 4544 on the ragged batch,
where it took 453.9 us per step against 466.1 us at 7 x 2560 and 531.1 us at 5 x 3648.
"""

import ctypes
import os

import numpy as np
import pytest

from mla_latent_kv_20_amd import binding as B
from mla_latent_kv_20_amd import workloads as W


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mla_latent_kv_20_amd import build
        build.build()
    return B.load()


DSV2_DIMS = dict(n_h=128, d_h=128, d_c=512, d_r=64)


def dims():
    return B.dims(DSV2_DIMS["n_h"], DSV2_DIMS["d_h"], DSV2_DIMS["d_c"], DSV2_DIMS["d_r"], B.MLA_BF16)


def offsets(lengths):
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int64)


def lengths_of(name):
    """The sequence lengths (rows, new tokens included) a named workload draws."""
    kw = W.CONFIGS[name][1]
    if "ragged_range" in kw:
        lo, hi = kw["ragged_range"]
        lens = np.random.default_rng(0).integers(lo, hi + 1, size=kw["ragged_batch"])
    else:
        lens = np.asarray(kw["lengths"], np.int64)
    q = kw.get("q_per_seq", 1)
    return (lens + q if kw.get("appended_rows") else lens), q


@pytest.mark.parametrize("name,plan", [("dsv2_b32_t4096", (8, 512)), ("dsv2_b4_t131072", (64, 2048)),
                                       ("dsv2_ragged_b128", (4, 4544)), ("dsv2_mtp4_b64_t8192", (1, 0)),
                                       ("dsv2_prefill_b1_t4096", (1, 0))])
def test_plans_of_the_measured_workloads(lib, name, plan):
    lens, q = lengths_of(name)
    w = W.make_config(name) if name == "dsv2_b32_t4096" else None
    if w is not None:                                  # the drawn workload has these lengths
        assert np.array_equal(np.diff(w.offsets), lens)
    assert B.plan_splits(dims(), offsets(lens), len(lens), q) == plan
    kw = W.CONFIGS[name][1]
    assert (kw["num_splits"], kw["split_rows"]) == plan      # the workloads run the planned split


@pytest.mark.parametrize("seed", range(6))
def test_every_plan_keeps_the_rules(lib, seed):
    rng = np.random.default_rng(seed)
    batch = int(rng.choice([1, 3, 8, 17, 40, 130]))
    q = int(rng.choice([1, 1, 2, 4]))
    lens = rng.integers(q, int(rng.choice([64, 3000, 40000])), size=batch)
    max_splits = int(rng.choice([1, 4, 16, 64]))
    S, R = B.plan_splits(dims(), offsets(lens), batch, q, max_splits)
    assert 1 <= S <= max_splits
    if S == 1:
        assert R == 0
    else:
        assert R > 0 and R % 32 == 0
        if S < max_splits:                            # every split holds rows of the longest
            assert (S - 1) * R < lens.max() <= S * R
    assert B.plan_splits(dims(), offsets(lens), batch, q, max_splits) == (S, R)     # deterministic


def test_the_split_cap_is_kept(lib):
    lens = [4096] * 32
    assert B.plan_splits(dims(), offsets(lens), 32, 1, 1) == (1, 0)
    S, R = B.plan_splits(dims(), offsets(lens), 32, 1, 4)
    assert S <= 4 and (S == 1 or R % 32 == 0)


def test_argument_checks(lib):
    f = lib.mla_plan_splits
    d = dims()
    ns, sr = ctypes.c_int32(-1), ctypes.c_int32(-1)
    offs = offsets([100, 50])
    p = offs.ctypes.data
    assert f(None, p, 2, 1, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_NULL
    assert f(ctypes.byref(d), p, 2, 1, 8, None, ctypes.byref(sr)) == B.MLA_ERR_NULL
    assert f(ctypes.byref(d), None, 2, 1, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_NULL
    assert f(ctypes.byref(d), p, -1, 1, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_SHAPE
    assert f(ctypes.byref(d), p, 2, 0, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_SHAPE
    assert f(ctypes.byref(d), p, 2, 1, 0, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_SHAPE
    assert f(ctypes.byref(d), p, 2, 51, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_SHAPE  # len 50 < 51
    bad = np.array([0, 10, 5], np.int64)                                # a negative length
    assert f(ctypes.byref(d), bad.ctypes.data, 2, 1, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_ERR_SHAPE
    assert f(ctypes.byref(d), None, 0, 1, 8, ctypes.byref(ns), ctypes.byref(sr)) == B.MLA_OK
    assert (ns.value, sr.value) == (1, 0)

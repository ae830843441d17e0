"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Tolerances (on outputs o; m = max|o_ref|):
  fp32 workloads  max|o - o_ref| <= 1e-5 * m
  bf16 workloads  max|o - o_ref| <= 1e-2 * m + 1e-3
log-sum-exp values of mla_decode on a given q_abs are checked in absolute terms
(|d lse| <= 1e-3 bf16, 1e-5 fp32): the scores are then exact fp32 sums of exact bf16
products, so only summation order and exp2 rounding separate them from the fp64 values.
End to end, q_abs itself is rounded to bf16 (2^-8 relative per element), which moves each
logit by up to 2^-8 * scale * sum_c |q_c||row_c|; there every lse[n, i] is held to that
shift, maxed over its visible rows, plus 1e-3 (tests/bounds.py).

Every GPU step first prints the case it runs (test, workload, split plan).
"""

import numpy as np
import pytest

import oracle as O
from bounds import check_lse, lse_bound
from mla_latent_kv_20_amd import binding as B
from mla_latent_kv_20_amd import device as D
from mla_latent_kv_20_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("needs a GPU")
    B.load()
    return t


_cache = {}


def workload(name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _cache:
        _cache[key] = W.make_config(name, **kw)
    return _cache[key]


def dims_of(w):
    return B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_BF16 if w.dtype == W.BF16 else B.MLA_F32)


def bound(w, ref):
    m = float(np.max(np.abs(ref)))
    return 1e-5 * m if w.dtype == W.F32 else 1e-2 * m + 1e-3


def assert_close(what, got, ref, w, lse=False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite pattern differs"
    if lse:
        assert np.array_equal(got[~fin], ref[~fin]), what
        tol = 1e-5 if w.dtype == W.F32 else 1e-3
        err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    else:
        tol = bound(w, ref[fin])
        err = float(np.max(np.abs(got[fin] - ref[fin])))
    say(f"    {what}: max|d| = {err:.3e} (bound {tol:.3e})")
    assert err <= tol, f"{what}: max|d| {err} > {tol}"


def oracle_args(w):
    return dict(c_kv=w.f64("c_kv"), k_r=w.f64("k_r"), offsets=w.offsets, q_c=w.f64("q_c"),
                q_r=w.f64("q_r"), w_uk=w.f64("w_uk"), w_uv=w.f64("w_uv"), q_per_seq=w.q_per_seq)


def step_lse_bound(a, w):
    """The derived end-to-end lse bound for oracle arguments `a` (see tests/bounds.py); the
    fp32 workloads keep their exact q_abs, so only the per-call bound applies."""
    if w.dtype == W.F32:
        return np.full((len(a["q_c"]), w.n_h), 1e-5)
    q_abs = O.absorb_q(a["q_c"], a["q_r"], a["w_uk"])
    return lse_bound(q_abs, a["c_kv"], a["offsets"], a["q_per_seq"], O.default_scale(w.d_h, w.d_r))


SMALL = ["tiny_f32", "toy_p3", "dsv2_small", "dsv2_small_mtp", "dsv2_ragged_small"]
PLANS = {"tiny_f32": [(1, 0), (3, 20)], "toy_p3": [(1, 0), (2, 4)],
         "dsv2_small": [(1, 0), (3, 256), (5, 33)], "dsv2_small_mtp": [(1, 0), (2, 128), (9, 32)],
         "dsv2_ragged_small": [(1, 0), (4, 96), (7, 40)]}


# ----------------------------------------------------------------------------
# One call at a time, on drawn inputs
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", SMALL)
def test_absorb_q(torch, name):
    w = workload(name)
    say(f"[absorb_q] {name}")
    t = D.to_device(w)
    qa = B.absorb_q(dims_of(w), t["q_c"], t["q_r"], t["w_uk"])
    torch.cuda.synchronize()
    ref = O.absorb_q(w.f64("q_c"), w.f64("q_r"), w.f64("w_uk"))
    got = D.to_numpy_f64(qa)
    assert_close("q_abs", got, ref, w)
    if w.dtype == W.BF16:          # one rounding of an fp32 sum: within 2^-8 of each value
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4 * np.std(ref))
        assert np.array_equal(got[..., w.d_c:], ref[..., w.d_c:])


@pytest.mark.parametrize("d_h,d_c,n_q", [(48, 128, 5), (64, 256, 40), (256, 128, 33)])
def test_absorb_q_other_head_dims(torch, d_h, d_c, n_q):
    """bf16 absorb_q at head dimensions other than 128 (the kernel's general form): a weight
    slice that does not fill the last load round (d_h = 48), two 32-row query blocks, a
    head count that is not a multiple of 8; with and without RoPE positions."""
    n_h, d_r = 12, 16
    rng = np.random.default_rng(d_h + n_q)
    bf = lambda a: W.round_to_storage(a, W.BF16)
    q_c, q_r = bf(rng.standard_normal((n_q, n_h, d_h))), bf(rng.standard_normal((n_q, n_h, d_r)))
    w_uk = bf(rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_h))
    pos = rng.integers(0, 163840, size=n_q).astype(np.int64)
    d = B.dims(n_h, d_h, d_c, d_r, B.MLA_BF16)
    dev = lambda a: D._tensor(a, W.BF16, "cuda")
    say(f"[absorb_q] d_h={d_h} d_c={d_c} n_q={n_q} n_h={n_h}")
    qa = B.absorb_q(d, dev(q_c), dev(q_r), dev(w_uk))
    qa_r = B.absorb_q_rope(d, dev(q_c), dev(q_r), dev(w_uk), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    f = lambda a: W.to_f64(a, W.BF16)
    for what, got, ref in [("q_abs", qa, O.absorb_q(f(q_c), f(q_r), f(w_uk))),
                           ("q_abs with positions", qa_r, O.absorb_q_rope(f(q_c), f(q_r), f(w_uk), pos))]:
        got = D.to_numpy_f64(got)
        lim = 2.0 ** -8 * np.abs(ref[..., :d_c]) + 1e-4 * np.std(ref[..., :d_c])   # one rounding of an fp32 sum
        assert np.all(np.abs(got[..., :d_c] - ref[..., :d_c]) <= lim), what
        if what == "q_abs":
            assert np.array_equal(got[..., d_c:], ref[..., d_c:])
        else:                              # the rotation's one bf16 rounding
            assert np.all(np.abs(got[..., d_c:] - ref[..., d_c:]) <= 2.0 ** -8 * np.abs(ref[..., d_c:]) + 1e-6), what


@pytest.mark.parametrize("name", SMALL)
def test_decode(torch, name):
    w = workload(name)
    d = dims_of(w)
    qa = W.draw_q_abs(w)
    t = D.to_device(w)
    qa_t = D._tensor(qa, w.dtype, "cuda")
    partials = [B.MLA_F32, B.MLA_F16] if w.dtype == W.BF16 else [B.MLA_F32]
    for (S, R), pd in [(plan, pd) for plan in PLANS[name] for pd in partials]:
        say(f"[decode] {name} splits={S} split_rows={R} partials={'f16' if pd == B.MLA_F16 else 'f32'}")
        # NaN-filled: every non-empty split's row must be written; empty ones are left alone
        op0 = torch.full((S, w.n_q, w.n_h, w.d_c), float("nan"), dtype=B._torch_dtype(pd), device="cuda")
        op, lp = B.decode(d, qa_t, t["c_kv"], t["k_r"], t["offsets"], w.batch, w.q_per_seq, S, R,
                          o_part=op0)
        torch.cuda.synchronize()
        ro, rl = O.split_partials(W.to_f64(qa, w.dtype), w.f64("c_kv"), w.f64("k_r"), w.offsets,
                                  w.q_per_seq, S, R, O.default_scale(w.d_h, w.d_r))
        live = ~np.isneginf(rl)
        got_o = D.to_numpy_f64(op)
        assert np.all(np.isnan(got_o[~live]))
        assert_close("o_part", got_o[live], ro[live], w)
        assert_close("lse_part", D.to_numpy_f64(lp), rl, w, lse=True)


@pytest.mark.parametrize("S,f16", [(1, False), (2, False), (7, False), (64, False), (3, True), (64, True)])
def test_merge(torch, S, f16):
    n_q, n_h, d_c = 5, 128, 512
    say(f"[merge] splits={S} partials={'f16' if f16 else 'f32'}")
    o, l = W.draw_partials(S, n_q, n_h, d_c, seed=S)
    if f16:
        o = o.astype(np.float16)       # the partials the GPU consumes; the oracle widens the same values
    d = B.dims(n_h, 128, d_c, 64, B.MLA_BF16)
    ol, ll = B.merge_splits(d, torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda())
    torch.cuda.synchronize()
    ro, rl = O.merge_splits(o.astype(np.float64), l.astype(np.float64))
    w32 = W.make_config("tiny_f32")          # fp32 tolerance: the merge is fp32 end to end
    assert_close("o_lat", D.to_numpy_f64(ol), ro, w32)
    assert_close("lse", D.to_numpy_f64(ll), rl, w32, lse=True)


def test_merge_all_empty_and_odd_width(torch):
    say("[merge] all splits empty, d_c = 30")
    o, l = W.draw_partials(3, 2, 4, 30, seed=9, empty_frac=0.0)
    l[:, 1, 2] = -np.inf
    o[:, 1, 2] = 0.0
    d = B.dims(4, 16, 30, 8, B.MLA_F32)
    ol, ll = B.merge_splits(d, torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda())
    torch.cuda.synchronize()
    got_o, got_l = D.to_numpy_f64(ol), D.to_numpy_f64(ll)
    assert np.all(got_o[1, 2] == 0.0) and got_l[1, 2] == -np.inf
    keep = np.ones((2, 4), bool)
    keep[1, 2] = False
    ro, rl = O.merge_splits(o[:, keep].astype(np.float64)[:, None], l[:, keep].astype(np.float64)[:, None])
    w32 = W.make_config("tiny_f32")
    assert_close("o_lat", got_o[keep][None], ro, w32)
    assert_close("lse", got_l[keep][None], rl, w32, lse=True)


@pytest.mark.parametrize("n_q", [64, 100, 128, 300, 700])
def test_absorb_and_out_proj_many_rows(torch, n_q):
    """Many query rows (a prefill's worth, the many-row kernels): runs of whole 32-row blocks,
    the last one ragged; every row against the oracle, with and without RoPE positions, and
    absorb_q bitwise against the decode-size kernel called on 60 rows at a time."""
    n_h, d_h, d_c, d_r = 128, 128, 512, 64
    rng = np.random.default_rng(n_q)
    bf = lambda a: W.round_to_storage(a, W.BF16)
    q_c, q_r = bf(rng.standard_normal((n_q, n_h, d_h))), bf(rng.standard_normal((n_q, n_h, d_r)))
    w_uk = bf(rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c))
    w_uv = bf(rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c))
    o_lat = rng.standard_normal((n_q, n_h, d_c)).astype(np.float32)
    pos = rng.integers(0, 163840, size=n_q).astype(np.int64)
    d = B.dims(n_h, d_h, d_c, d_r, B.MLA_BF16)
    dev = lambda a: D._tensor(a, W.BF16, "cuda")
    say(f"[many rows] n_q={n_q}: absorb_q, absorb_q_rope, out_proj")
    qa = B.absorb_q(d, dev(q_c), dev(q_r), dev(w_uk))
    qa_r = B.absorb_q_rope(d, dev(q_c), dev(q_r), dev(w_uk), torch.from_numpy(pos).cuda())
    oc = B.out_proj(d, torch.from_numpy(o_lat).cuda(), dev(w_uv))
    # the same rows in calls of 60 (the decode-size kernels): bitwise equal
    qc_t, qr_t, wk_t, pos_t = dev(q_c), dev(q_r), dev(w_uk), torch.from_numpy(pos).cuda()
    parts = [(B.absorb_q(d, qc_t[a:a + 60], qr_t[a:a + 60], wk_t),
              B.absorb_q_rope(d, qc_t[a:a + 60], qr_t[a:a + 60], wk_t, pos_t[a:a + 60])) for a in range(0, n_q, 60)]
    torch.cuda.synchronize()
    assert torch.equal(qa.view(torch.int16), torch.cat([p[0] for p in parts]).view(torch.int16))
    assert torch.equal(qa_r.view(torch.int16), torch.cat([p[1] for p in parts]).view(torch.int16))
    f = lambda a: W.to_f64(a, W.BF16)
    for what, got, ref in [("q_abs", qa, O.absorb_q(f(q_c), f(q_r), f(w_uk))),
                           ("q_abs with positions", qa_r, O.absorb_q_rope(f(q_c), f(q_r), f(w_uk), pos))]:
        got = D.to_numpy_f64(got)
        lim = 2.0 ** -8 * np.abs(ref) + 1e-4 * np.std(ref)     # one rounding of an fp32 sum
        say(f"    {what}: worst |d|/limit {float(np.max(np.abs(got - ref) / lim)):.3f}")
        assert np.all(np.abs(got - ref) <= lim), what
    assert np.array_equal(D.to_numpy_f64(qa)[..., d_c:], f(q_r))
    ref = O.out_proj(W.to_f64(bf(o_lat), W.BF16), f(w_uv))   # the kernel's operand rounding
    got = D.to_numpy_f64(oc)
    lim = 2.0 ** -8 * np.abs(ref) + 1e-4 * np.std(ref)
    say(f"    o_c: worst |d|/limit {float(np.max(np.abs(got - ref) / lim)):.3f}")
    assert np.all(np.abs(got - ref) <= lim)


@pytest.mark.parametrize("n_q", [129, 257])
def test_out_proj_many_rows_off_the_head_group(torch, n_q):
    """160 heads (the last XCD group half empty) and row runs of 96 rows with a ragged last
    block: mla_out_proj against the oracle, and the fused call bitwise against the two calls."""
    n_h, d_h, d_c = 160, 128, 512
    rng = np.random.default_rng(40 + n_q)
    w_uv = W.round_to_storage(rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c), W.BF16)
    o, l = W.draw_partials(2, n_q, n_h, d_c, seed=41 + n_q)
    o = o.astype(np.float16)
    d = B.dims(n_h, d_h, d_c, 64, B.MLA_BF16)
    say(f"[out_proj many rows] n_h=160 n_q={n_q}")
    ot, lt, wt = torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(), D._tensor(w_uv, W.BF16, "cuda")
    ol, _ = B.merge_splits(d, ot, lt)
    oc = B.out_proj(d, ol, wt)
    oc2, _, _ = B.merge_out_proj(d, ot, lt, wt)
    torch.cuda.synchronize()
    assert torch.equal(oc.view(torch.int16), oc2.view(torch.int16))
    o_lat = ol.cpu().numpy().astype(np.float64)
    ref = O.out_proj(W.to_f64(W.round_to_storage(o_lat, W.BF16), W.BF16), W.to_f64(w_uv, W.BF16))
    got = D.to_numpy_f64(oc)
    lim = 2.0 ** -8 * np.abs(ref) + 1e-4 * np.std(ref)
    say(f"    o_c: worst |d|/limit {float(np.max(np.abs(got - ref) / lim)):.3f}")
    assert np.all(np.abs(got - ref) <= lim)


@pytest.mark.parametrize("name", SMALL)
def test_out_proj(torch, name):
    w = workload(name)
    say(f"[out_proj] {name}")
    o_lat = W.draw_o_lat(w.n_q, w.n_h, w.d_c)
    t = D.to_device(w)
    oc = B.out_proj(dims_of(w), torch.from_numpy(o_lat).cuda(), t["w_uv"])
    torch.cuda.synchronize()
    assert_close("o_c", D.to_numpy_f64(oc), O.out_proj(o_lat.astype(np.float64), w.f64("w_uv")), w)


@pytest.mark.parametrize("S,f16,n_q", [(1, True, 1), (3, True, 33), (8, True, 32), (8, False, 64),
                                        (13, False, 40), (12, True, 48), (16, True, 17), (17, True, 9),
                                        (64, True, 7), (70, True, 3), (3, True, 160),
                                        (1, False, 300)])
def test_merge_out_proj_equals_the_two_calls(torch, S, f16, n_q):
    """The fused call writes exactly what mla_merge_splits + mla_out_proj write."""
    n_h, d_h, d_c = 128, 128, 512
    say(f"[merge_out_proj] splits={S} partials={'f16' if f16 else 'f32'} n_q={n_q}")
    o, l = W.draw_partials(S, n_q, n_h, d_c, seed=100 + S + n_q)
    l[:, 0, 5] = -np.inf                  # one query head that no split saw
    o[:, 0, 5] = 0.0
    if f16:
        o = o.astype(np.float16)
    rng = np.random.default_rng(S)
    w_uv = W.round_to_storage(rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c), W.BF16)
    d = B.dims(n_h, d_h, d_c, 64, B.MLA_BF16)
    ot, lt = torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda()
    wt = D._tensor(w_uv, W.BF16, "cuda")
    ol, ll = B.merge_splits(d, ot, lt)
    oc = B.out_proj(d, ol, wt)
    oc2, ll2, ol2 = B.merge_out_proj(d, ot, lt, wt, want_o_lat=True)
    oc3, _, _ = B.merge_out_proj(d, ot, lt, wt, want_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(oc, oc2) and torch.equal(oc, oc3)
    assert torch.equal(ll, ll2) and torch.equal(ol, ol2)
    ro, rl = O.merge_splits(o.astype(np.float64), l.astype(np.float64))
    ref = O.out_proj(ro, W.to_f64(w_uv, W.BF16))
    assert_close("o_c", D.to_numpy_f64(oc2), ref, workload("dsv2_small"))
    assert np.all(D.to_numpy_f64(oc2)[0, 5] == 0.0) and np.isneginf(D.to_numpy_f64(ll2)[0, 5])


def test_merge_out_proj_fp32(torch):
    say("[merge_out_proj] fp32 dims n_h=4 d_h=16 d_c=32, splits=3")
    o, l = W.draw_partials(3, 6, 4, 32, seed=12)
    rng = np.random.default_rng(13)
    w_uv = (rng.standard_normal((4, 16, 32)) / np.sqrt(32)).astype(np.float32)
    d = B.dims(4, 16, 32, 8, B.MLA_F32)
    oc, ll, ol = B.merge_out_proj(d, torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda(),
                                  torch.from_numpy(w_uv).cuda())
    torch.cuda.synchronize()
    ro, rl = O.merge_splits(o.astype(np.float64), l.astype(np.float64))
    w32 = W.make_config("tiny_f32")
    assert_close("o_c", D.to_numpy_f64(oc), O.out_proj(ro, w_uv.astype(np.float64)), w32)
    assert_close("o_lat", D.to_numpy_f64(ol), ro, w32)
    assert_close("lse", D.to_numpy_f64(ll), rl, w32, lse=True)


# ----------------------------------------------------------------------------
# The four calls end to end, from raw inputs
# ----------------------------------------------------------------------------

def run_step(w, S, R, fused=False):
    t = D.to_device(w)
    bufs = None
    if fused:
        import torch
        bufs = dict(o_lat=torch.empty((w.n_q, w.n_h, w.d_c), dtype=torch.float32, device="cuda"))
    out = B.decode_step(dims_of(w), t["q_c"], t["q_r"], t["w_uk"], t["w_uv"], t["cache"],
                        t["offsets"], w.batch, w.q_per_seq, S, R, bufs=bufs, fused=fused)
    import torch
    torch.cuda.synchronize()
    return {k: D.to_numpy_f64(v) for k, v in out.items() if k in ("o_c", "o_lat", "lse")}


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", SMALL)
def test_end_to_end(torch, name, fused):
    w = workload(name)
    a = oracle_args(w)
    naive = O.naive_decode(**a, seqs=[0, w.batch - 1] if w.d_c == 512 else None)
    for S, R in PLANS[name]:
        say(f"[end_to_end] {name} splits={S} split_rows={R} fused={fused}")
        got = run_step(w, S, R, fused)
        ref = O.absorbed_decode(**a, num_splits=S, split_rows=R)
        assert_close("o_c", got["o_c"], ref["o_c"], w)
        assert_close("o_lat", got["o_lat"], ref["o_lat"], w)
        check_lse("lse", got["lse"], ref["lse"], step_lse_bound(a, w), say)
        sel = ~np.isnan(naive["o_c"][:, 0, 0])
        assert_close("o_c vs naive", got["o_c"][sel], naive["o_c"][sel], w)


# ----------------------------------------------------------------------------
# Edge cases
# ----------------------------------------------------------------------------

def test_single_row_gives_the_row_exactly(torch):
    w = W.make_workload("t1", **W.DSV2, dtype=W.BF16, lengths=[1, 1, 1, 1], seed=4)
    say("[edge] single cached row per sequence")
    got = run_step(w, 1, 0)
    c = w.f64("c_kv")
    for b in range(4):
        assert np.array_equal(got["o_lat"][b], np.broadcast_to(c[b], (w.n_h, w.d_c)))


def test_decode_rows_inside_wider_rows(torch):
    """Cache rows inside 640-element rows (row stride 1280 bytes): every tile takes the
    general-stride loads, lengths straddle tile edges and splits; against the oracle, and
    equal bit for bit to the same call on the packed cache."""
    w = W.make_workload("wide", **W.DSV2, dtype=W.BF16, lengths=[1, 33, 64, 95, 130], seed=21)
    d = dims_of(w)
    qa = W.draw_q_abs(w, seed=22)
    t = D.to_device(w)
    say("[edge] row stride 640 elements, splits=3 split_rows=64")
    wide = torch.zeros((w.rows, 640), dtype=torch.bfloat16, device="cuda")
    wide[:, :w.d_c + w.d_r] = t["cache"]
    qa_t = D._tensor(qa, w.dtype, "cuda")
    op, lp = B.decode(d, qa_t, wide[:, :w.d_c], wide[:, w.d_c:w.d_c + w.d_r], t["offsets"], w.batch, 1, 3, 64)
    op2, lp2 = B.decode(d, qa_t, t["c_kv"], t["k_r"], t["offsets"], w.batch, 1, 3, 64)
    torch.cuda.synchronize()
    ro, rl = O.split_partials(W.to_f64(qa, w.dtype), w.f64("c_kv"), w.f64("k_r"), w.offsets, 1, 3, 64,
                              O.default_scale(w.d_h, w.d_r))
    live = ~np.isneginf(rl)
    assert not live.all()
    assert_close("o_part", D.to_numpy_f64(op)[live], ro[live], w)
    assert_close("lse_part", D.to_numpy_f64(lp), rl, w, lse=True)
    assert torch.equal(lp, lp2)
    assert torch.equal(op[torch.from_numpy(live).cuda()], op2[torch.from_numpy(live).cuda()])


def test_empty_splits_and_ragged_tails(torch):
    # lengths straddle tile edges; 6 splits of 40 rows leave trailing splits empty
    w = W.make_workload("tails", **W.DSV2, dtype=W.BF16, lengths=[1, 31, 32, 33, 95, 200], seed=6)
    d = dims_of(w)
    qa = W.draw_q_abs(w, seed=7)
    t = D.to_device(w)
    say("[edge] empty splits and ragged tails, splits=6 split_rows=40")
    op0 = torch.full((6, w.n_q, w.n_h, w.d_c), float("nan"), dtype=torch.float16, device="cuda")
    op, lp = B.decode(d, D._tensor(qa, w.dtype, "cuda"), t["c_kv"], t["k_r"], t["offsets"], w.batch,
                      1, 6, 40, o_part=op0)
    torch.cuda.synchronize()
    ro, rl = O.split_partials(W.to_f64(qa, w.dtype), w.f64("c_kv"), w.f64("k_r"), w.offsets, 1, 6, 40,
                              O.default_scale(w.d_h, w.d_r))
    got_o, got_l = D.to_numpy_f64(op), D.to_numpy_f64(lp)
    empty = np.isneginf(rl)
    assert empty.any()
    # empty splits: lse = -inf, o_part untouched (still NaN)
    assert np.all(np.isnan(got_o[empty])) and np.all(np.isneginf(got_l[empty]))
    assert_close("o_part", got_o[~empty], ro[~empty], w)
    assert_close("lse_part", got_l, rl, w, lse=True)
    # the merges never read an empty split's o_part: NaN there must not reach their outputs
    mo, ml = O.merge_splits(ro, rl)
    ol, ll = B.merge_splits(d, op, lp)
    rng = np.random.default_rng(3)
    w_uv = W.round_to_storage(rng.standard_normal((w.n_h, w.d_h, w.d_c)) / np.sqrt(w.d_c), W.BF16)
    oc, ll2, ol2 = B.merge_out_proj(d, op, lp, D._tensor(w_uv, W.BF16, "cuda"), want_o_lat=True)
    torch.cuda.synchronize()
    assert_close("o_lat (merge)", D.to_numpy_f64(ol), mo, w)
    assert_close("lse (merge)", D.to_numpy_f64(ll), ml, w, lse=True)
    assert torch.equal(ol, ol2) and torch.equal(ll, ll2)
    assert_close("o_c (merge_out_proj)", D.to_numpy_f64(oc), O.out_proj(mo, W.to_f64(w_uv, W.BF16)), w)


@pytest.mark.parametrize("n_h", [96, 160])
def test_head_counts_off_the_group_size(torch, n_h):
    w = W.make_workload("heads", n_h=n_h, d_h=128, d_c=512, d_r=64, dtype=W.BF16,
                        lengths=[70, 5], seed=8)
    say(f"[edge] n_h={n_h}")
    got = run_step(w, 2, 64)
    ref = O.absorbed_decode(**oracle_args(w), num_splits=2, split_rows=64)
    assert_close("o_c", got["o_c"], ref["o_c"], w)
    check_lse("lse", got["lse"], ref["lse"], step_lse_bound(oracle_args(w), w), say)


@pytest.mark.parametrize("lengths", [[70] * 24, [70] * 11 + [71] + [70] * 12])
def test_sixteen_or_more_sequences_equal_and_unequal(torch, lengths):
    """At 16 or more sequences the decode deals them to XCDs by length; with every length
    equal it takes the ranks as the indices without ranking.  Both, with the last of 4 splits
    of 32 rows left empty (70 rows need 3), so the split-0 workgroup marks it."""
    w = W.make_workload("uni", **W.DSV2, dtype=W.BF16, lengths=lengths, seed=11)
    a = oracle_args(w)
    say(f"[edge] {len(lengths)} sequences, {'equal' if len(set(lengths)) == 1 else 'unequal'} lengths, 4 x 32")
    got = run_step(w, 4, 32)
    ref = O.absorbed_decode(**a, num_splits=4, split_rows=32)
    assert_close("o_c", got["o_c"], ref["o_c"], w)
    assert_close("o_lat", got["o_lat"], ref["o_lat"], w)
    check_lse("lse", got["lse"], ref["lse"], step_lse_bound(a, w), say)


@pytest.mark.parametrize("count,equal", [(300, False), (300, True), (600, False)])
def test_more_sequences_than_threads(torch, count, equal):
    """300 sequences: more than the workgroup's 256 threads, so each loop of the length
    ranking (offsets read, equal-length vote, ranks) takes several passes; ragged lengths of
    1..40 rows (several splits empty) or all equal.  600 ragged sequences put more than 64
    on an XCD, where its items go sequence by sequence instead of longest first."""
    rng = np.random.default_rng(23)
    lengths = [17] * count if equal else [int(x) for x in rng.integers(1, 41, size=count)]
    w = W.make_workload("many", **W.DSV2, dtype=W.BF16, lengths=lengths, seed=12)
    a = oracle_args(w)
    say(f"[edge] {count} sequences, {'equal' if equal else 'ragged'} lengths, 3 x 16")
    got = run_step(w, 3, 16)
    ref = O.absorbed_decode(**a, num_splits=3, split_rows=16)
    assert_close("o_c", got["o_c"], ref["o_c"], w)
    assert_close("o_lat", got["o_lat"], ref["o_lat"], w)
    check_lse("lse", got["lse"], ref["lse"], step_lse_bound(a, w), say)


def test_ragged_sequences_with_several_queries(torch):
    """20 sequences of unequal lengths (the longest-first dealing of an XCD's items), each
    with 3 new tokens that attend causally among themselves."""
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(0, 200, size=20)]
    w = W.make_workload("rq", **W.DSV2, dtype=W.BF16, lengths=lengths, q_per_seq=3, appended_rows=True,
                        seed=13)
    a = oracle_args(w)
    say("[edge] 20 ragged sequences, 3 queries each, 4 x 48")
    got = run_step(w, 4, 48)
    ref = O.absorbed_decode(**a, num_splits=4, split_rows=48)
    assert_close("o_c", got["o_c"], ref["o_c"], w)
    assert_close("o_lat", got["o_lat"], ref["o_lat"], w)
    check_lse("lse", got["lse"], ref["lse"], step_lse_bound(a, w), say)


def test_split_plans_agree_and_runs_repeat_bitwise(torch):
    w = workload("dsv2_small")
    say("[edge] split plans 1/7/64 and repeatability")
    outs = [run_step(w, S, R) for S, R in [(1, 0), (7, 160), (64, 32)]]
    for o in outs[1:]:
        assert_close("o_c across plans", o["o_c"], outs[0]["o_c"], w)
    again = run_step(w, 7, 160)
    assert np.array_equal(again["o_c"], outs[1]["o_c"]) and np.array_equal(again["lse"], outs[1]["lse"])


@pytest.mark.parametrize("f16", [False, True])
def test_outputs_stay_inside_their_buffers(torch, f16):
    """Guard bands of NaN around every output are untouched after a step."""
    w = workload("dsv2_small_mtp")
    d = dims_of(w)
    t = D.to_device(w)
    G = 4096
    S, R = 3, 64

    def guarded(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * G,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[G:G + n].view(*shape)

    bufs = {}
    raw = {}
    for k, shape, dt in [("q_abs", (w.n_q, w.n_h, 576), torch.bfloat16),
                         ("o_part", (S, w.n_q, w.n_h, 512), torch.float16 if f16 else torch.float32),
                         ("lse_part", (S, w.n_q, w.n_h), torch.float32),
                         ("o_lat", (w.n_q, w.n_h, 512), torch.float32),
                         ("lse", (w.n_q, w.n_h), torch.float32),
                         ("o_c", (w.n_q, w.n_h, 128), torch.bfloat16)]:
        raw[k], bufs[k] = guarded(shape, dt)
    say(f"[edge] guard bands, partials={'f16' if f16 else 'f32'}")
    B.decode_step(d, t["q_c"], t["q_r"], t["w_uk"], t["w_uv"], t["cache"], t["offsets"], w.batch,
                  w.q_per_seq, S, R, bufs=bufs)
    torch.cuda.synchronize()
    empty = torch.isneginf(bufs["lse_part"])
    assert empty.any()                    # sequence 0 (7 rows) leaves its later splits empty
    for k, buf in raw.items():
        assert torch.isnan(buf[:G].float()).all() and torch.isnan(buf[-G:].float()).all(), k
        if k == "o_part":                 # an empty split's row is never written
            assert torch.isnan(bufs[k][empty].float()).all(), k
            assert not torch.isnan(bufs[k][~empty].float()).any(), k
        else:
            assert not torch.isnan(bufs[k].float()).any(), k


# ----------------------------------------------------------------------------
# Full-size workloads, in the split plans the benchmark uses; every sequence and query
# against the absorbed oracle, one sequence at a time (bounded host memory)
# ----------------------------------------------------------------------------

def subset(w, seqs):
    """The sub-workload of some sequences (rows, queries; same weights)."""
    rows = np.concatenate([np.arange(w.offsets[b], w.offsets[b + 1]) for b in seqs])
    qs = np.concatenate([np.arange(b * w.q_per_seq, (b + 1) * w.q_per_seq) for b in seqs])
    lens = w.lengths[seqs]
    return dict(c_kv=W.to_f64(w.c_kv[rows], w.dtype),
                k_r=W.to_f64(w.k_r[rows], w.dtype),
                offsets=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64),
                q_c=W.to_f64(w.q_c[qs], w.dtype), q_r=W.to_f64(w.q_r[qs], w.dtype),
                w_uk=w.f64("w_uk"), w_uv=w.f64("w_uv"), q_per_seq=w.q_per_seq), qs


FULL = ["dsv2_b32_t4096", "dsv2_b4_t131072", "dsv2_ragged_b128", "dsv2_mtp4_b64_t8192"]


def compare_every_sequence(w, got, ref_of, label):
    """got: the step's outputs for the whole batch; ref_of(b) -> (oracle outputs, query rows,
    lse bound) for sequence b.  Each output is held to its bound over the whole batch
    (o_c, o_lat: 1e-2 max|ref| + 1e-3; lse: the derived per-element bound)."""
    worst = {"o_c": 0.0, "o_lat": 0.0}
    peak = {"o_c": 0.0, "o_lat": 0.0}
    lse_err, lse_ratio = 0.0, 0.0
    for b in range(w.batch):
        ref, qs, lb = ref_of(b)
        for k in worst:
            g, r = got[k][qs], ref[k]
            worst[k] = max(worst[k], float(np.max(np.abs(g - r))))
            peak[k] = max(peak[k], float(np.max(np.abs(r))))
        gl, rl = got["lse"][qs], ref["lse"]
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(gl), fin) and np.array_equal(gl[~fin], rl[~fin]), f"{label} seq {b}"
        d = np.abs(gl[fin] - rl[fin])
        lse_err = max(lse_err, float(d.max()))
        lse_ratio = max(lse_ratio, float((d / lb[fin]).max()))
    for k in worst:
        tol = 1e-2 * peak[k] + 1e-3
        say(f"    {label} {k}: max|d| = {worst[k]:.3e} over all {w.batch} sequences (bound {tol:.3e})")
        assert worst[k] <= tol, f"{label} {k}: {worst[k]} > {tol}"
    say(f"    {label} lse: max|d| = {lse_err:.3e}, max |d|/bound = {lse_ratio:.3f}")
    assert lse_ratio <= 1.0, f"{label} lse exceeds its derived bound ({lse_ratio})"


@pytest.mark.parametrize("name", FULL)
def test_full_size(torch, name):
    w = workload(name)
    say(f"[full] {name} rows={w.rows} splits={w.num_splits} split_rows={w.split_rows} "
        f"oracle on every sequence")
    got = run_step(w, w.num_splits, w.split_rows)

    def ref_of(b):
        a, qs = subset(w, [b])
        ref = O.absorbed_decode(**a, num_splits=w.num_splits, split_rows=w.split_rows)
        return ref, qs, step_lse_bound(a, w)

    compare_every_sequence(w, got, ref_of, name)
    seqs = [0]
    if name in ("dsv2_b32_t4096", "dsv2_mtp4_b64_t8192"):   # the pages' definition, sampled heads
        heads = [5, 100]
        b0 = seqs[0]
        a1, qs1 = subset(w, [b0])
        a1 = dict(a1, q_c=a1["q_c"][:, heads], q_r=a1["q_r"][:, heads], w_uk=a1["w_uk"][heads],
                  w_uv=a1["w_uv"][heads])
        nv = O.naive_decode(**a1)
        assert_close("o_c vs naive", got["o_c"][qs1][:, heads], nv["o_c"], w)

"""mla_kv_append_noalloc (partial sums in the library's fixed device array) against
mla_kv_append (partial sums in a caller's workspace): the same kernels, so every cache row
must come back bit for bit equal.

Two calls in a row on one GPU, the second with fewer tokens, so the second call runs over
the partial sums the first one left in the array: the largest call the array allows (455
new tokens at the DeepSeek-V2 width), then 40 (not a multiple of the 32-token block).  The
first call's rows are also held to the oracle (one bf16 rounding of the fp64 value plus the
fp32 summation error, as for mla_kv_append).  Every GPU step first prints its case.
"""

import numpy as np
import pytest

import oracle as O
from mla_latent_kv_20_amd import binding as B
from mla_latent_kv_20_amd import device as D
from mla_latent_kv_20_amd import workloads as W

pytestmark = pytest.mark.gpu

D_MODEL = 5120


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("needs a GPU")
    B.load()
    return t


def _bits(t):
    import torch
    return t.view(torch.int16)


def test_noalloc_matches_workspace_entry_point(torch):
    w = W.make_config("dsv2_small")
    d = B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_BF16)
    most = B.NOALLOC_SCRATCH_BYTES // B.kv_append_workspace_bytes(d, 1)
    assert most == 455
    rope = B.rope(theta=10000.0)
    for call, n in enumerate((most, 40)):
        pos = (np.arange(n, dtype=np.int64) * 977 + 4096) % 131072
        dst = np.random.default_rng(call).permutation(8 * n)[:n].astype(np.int64)   # distinct rows, any order
        p = W.draw_prologue(w, D_MODEL, pos, dst, seed=40 + call)
        say(f"[kv_append_noalloc] call {call}: n_new={n} d_model={D_MODEL} rows={8 * n}")
        h = D._tensor(p.h, W.BF16, "cuda")
        w_dkv = D._tensor(p.w_dkv, W.BF16, "cuda")
        w_kr = D._tensor(p.w_kr, W.BF16, "cuda")
        positions = torch.from_numpy(p.positions).cuda()
        dst_rows = torch.from_numpy(p.dst_rows).cuda()
        base = D._tensor(W.round_to_storage(np.full((8 * n, w.d_c + w.d_r), 3.0), W.BF16), W.BF16, "cuda")
        ref = base.clone()
        got = base.clone()
        B.kv_append(d, h, w_dkv, w_kr, positions, dst_rows, ref, rope=rope)
        B.kv_append_noalloc(d, h, w_dkv, w_kr, positions, dst_rows, got, rope=rope)
        torch.cuda.synchronize()
        same = torch.equal(_bits(got), _bits(ref))
        say(f"    rows equal bit for bit: {same}")
        assert same
        if call == 0:
            c, k = O.kv_prologue(W.to_f64(p.h, W.BF16), W.to_f64(p.w_dkv, W.BF16), W.to_f64(p.w_kr, W.BF16), pos)
            g = D.to_numpy_f64(got)
            for what, a, b in (("c_kv", g[dst, :w.d_c], c), ("k_r", g[dst, w.d_c:], k)):
                err = np.abs(a - b)
                lim = 2.0 ** -8 * np.abs(b) + 1e-4
                say(f"    {what}: worst |d|/limit {float((err / lim).max()):.3f}")
                assert np.all(err <= lim), what
            untouched = np.setdiff1d(np.arange(8 * n), dst)
            assert torch.equal(_bits(got[torch.from_numpy(untouched).cuda()]),
                               _bits(base[torch.from_numpy(untouched).cuda()]))


def test_noalloc_fp32_needs_no_array(torch):
    """fp32 rows use no partial sums: the call takes no scratch and still equals mla_kv_append."""
    w = W.make_config("tiny_f32")
    d = B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_F32)
    n, d_model = 6, 24
    pos = np.arange(n, dtype=np.int64) * 5 + 3
    dst = np.array([4, 0, 9, 2, 7, 5], dtype=np.int64)
    p = W.draw_prologue(w, d_model, pos, dst, seed=5)
    say(f"[kv_append_noalloc] fp32: n_new={n} d_model={d_model}")
    args = [D._tensor(p.h, W.F32, "cuda"), D._tensor(p.w_dkv, W.F32, "cuda"), D._tensor(p.w_kr, W.F32, "cuda"),
            torch.from_numpy(p.positions).cuda(), torch.from_numpy(p.dst_rows).cuda()]
    base = torch.full((10, w.d_c + w.d_r), 2.0, dtype=torch.float32, device="cuda")
    ref, got = base.clone(), base.clone()
    B.kv_append(d, *args, ref)
    B.kv_append_noalloc(d, *args, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_noalloc_rejects_more_than_the_array_holds(torch):
    w = W.make_config("dsv2_small")
    d = B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_BF16)
    n = 456
    say(f"[kv_append_noalloc] over the limit: n_new={n} (checked on the host, nothing launched)")
    h = torch.zeros((n, D_MODEL), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((w.d_c, D_MODEL), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((w.d_r, D_MODEL), dtype=torch.bfloat16, device="cuda")
    idx = torch.arange(n, dtype=torch.int64, device="cuda")
    rows = torch.zeros((n, w.d_c + w.d_r), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MlaError) as e:
        B.kv_append_noalloc(d, h, wd, wr, idx, idx, rows)
    assert e.value.status == B.MLA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert not torch.any(rows)

"""The decode step captured as a HIP graph: every replay equals the eager step bit for bit.

The benchmark times the step (mla_absorb_q, mla_decode, mla_merge_out_proj; and the
quantized-cache, prologue and projection calls beside it) as graph replays.  None of these
calls records a memset, the empty-split marks are written by the decode kernel itself and
every workspace is written before it is read within one call, so replays must reproduce the
eager outputs exactly.  Each graph is replayed several times with eager
work and synchronizations between replays, and every replay is checked.

Every GPU step first prints the case it runs.
"""

import pytest

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


@pytest.mark.parametrize("name,S,R", [("dsv2_ragged_small", 4, 96), ("dsv2_small_mtp", 2, 128)])
def test_step_graph_replays_equal_eager(torch, name, S, R):
    w = W.make_config(name)
    d = B.dims(w.n_h, w.d_h, w.d_c, w.d_r, B.MLA_BF16)
    t = D.to_device(w)
    n_q = w.n_q
    bufs = dict(q_abs=torch.empty((n_q, w.n_h, w.d_c + w.d_r), dtype=torch.bfloat16, device="cuda"),
                o_part=torch.empty((S, n_q, w.n_h, w.d_c), dtype=torch.float16, device="cuda"),
                lse_part=torch.empty((S, n_q, w.n_h), dtype=torch.float32, device="cuda"),
                o_c=torch.empty((n_q, w.n_h, w.d_h), dtype=torch.bfloat16, device="cuda"),
                lse=torch.empty((n_q, w.n_h), dtype=torch.float32, device="cuda"))
    codes, scales = B.quantize_rows_fp8(d, t["cache"])
    o8 = torch.empty_like(bufs["o_c"])
    stream = torch.cuda.Stream()

    def step():
        qa = B.absorb_q(d, t["q_c"], t["q_r"], t["w_uk"], bufs["q_abs"])
        op, lp = B.decode(d, qa, t["c_kv"], t["k_r"], t["offsets"], w.batch, w.q_per_seq, S, R,
                          bufs["o_part"], bufs["lse_part"])
        B.merge_out_proj(d, op, lp, t["w_uv"], bufs["o_c"], bufs["lse"], None)
        op8, lp8 = B.decode_fp8(d, qa, codes, scales, t["offsets"], w.batch, w.q_per_seq, S, R,
                                bufs["o_part"], bufs["lse_part"])
        B.merge_out_proj(d, op8, lp8, t["w_uv"], o8, None, None)

    say(f"[graph] {name} splits={S} split_rows={R}: eager")
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = {k: bufs[k].clone() for k in ("o_c", "lse")}
    ref8 = o8.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for k in ("o_c", "lse"):                       # clobber the outputs between replays
            bufs[k].fill_(float("nan"))
        o8.fill_(float("nan"))
        bufs["o_part"].normal_()
        torch.cuda.synchronize()
        say(f"[graph] {name} replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["o_c"].view(torch.int16), ref["o_c"].view(torch.int16)), rep
        assert torch.equal(bufs["lse"], ref["lse"]), rep
        assert torch.equal(o8.view(torch.int16), ref8.view(torch.int16)), rep
        with torch.cuda.stream(stream):                # eager work between replays
            step()
        torch.cuda.synchronize()
        assert torch.equal(bufs["o_c"].view(torch.int16), ref["o_c"].view(torch.int16)), rep


def test_prologue_and_projections_graph_replays_equal_eager(torch):
    """mla_kv_append (split-K workspace) and mla_absorb_q_rope under YaRN, then the skinny
    GEMMs mla_q_up and mla_o_proj (split-K partials in a caller workspace), at DeepSeek-V2
    widths."""
    n_h, d_h, d_c, d_r, d_model, d_cq, n = 128, 128, 512, 64, 5120, 1536, 8
    d = B.dims(n_h, d_h, d_c, d_r, B.MLA_BF16)
    rope = B.rope(yarn_factor=40.0)
    gen = torch.Generator(device="cuda").manual_seed(5)

    def rnd(*shape, scale=1.0):
        return (torch.randn(shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)

    h = rnd(n, d_model)
    w_dkv, w_kr = rnd(d_c, d_model, scale=d_model ** -0.5), rnd(d_r, d_model, scale=d_model ** -0.5)
    pos = torch.tensor([0, 1, 7, 4095, 4096, 20000, 163839, 3], dtype=torch.int64, device="cuda")
    dst = torch.tensor([9, 2, 0, 15, 4, 11, 6, 13], dtype=torch.int64, device="cuda")
    rows = torch.zeros((16, d_c + d_r), dtype=torch.bfloat16, device="cuda")
    ws_kv = torch.empty(max(1, B.kv_append_workspace_bytes(d, n)), dtype=torch.uint8, device="cuda")
    q_c, q_r, w_uk = rnd(n, n_h, d_h), rnd(n, n_h, d_r), rnd(n_h, d_h, d_c, scale=d_c ** -0.5)
    q_abs = torch.empty((n, n_h, d_c + d_r), dtype=torch.bfloat16, device="cuda")
    c_q, w_uq = rnd(n, d_cq), rnd(n_h, d_h, d_cq, scale=d_cq ** -0.5)
    o_c, w_o = rnd(n, n_h, d_h), rnd(d_model, n_h * d_h, scale=(n_h * d_h) ** -0.5)
    q_up_out = torch.empty((n, n_h, d_h), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((n, d_model), dtype=torch.bfloat16, device="cuda")
    wsb = B.proj_workspace_bytes(d, n, d_model, d_cq)
    ws_p = torch.empty(max(1, wsb), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    outs = (rows, q_abs, q_up_out, u)

    def step():
        B.kv_append(d, h, w_dkv, w_kr, pos, dst, rows, rope=rope, workspace=ws_kv)
        B.absorb_q_rope(d, q_c, q_r, w_uk, pos, q_abs, rope=rope)
        B.q_up(d, c_q, w_uq, q_up_out, ws_p)
        B.o_proj(d, o_c, w_o, u, ws_p)

    say(f"[graph] prologue and projections n={n} workspace {wsb} B: eager")
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    assert torch.isfinite(u.float()).all() and torch.isfinite(rows.float()).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for x in outs:
            x.fill_(float("nan"))
        ws_p.random_(0, 256)
        ws_kv.random_(0, 256)
        torch.cuda.synchronize()
        say(f"[graph] prologue and projections replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for x, r in zip((rows[dst],) + outs[1:], (ref[0][dst],) + tuple(ref[1:])):    # rows: written ones
            assert torch.equal(x.view(torch.int16), r.view(torch.int16)), rep
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        assert torch.equal(u.view(torch.int16), ref[3].view(torch.int16)), rep


def test_many_row_kernels_graph_replays_equal_eager(torch):
    """The many-row forms of mla_absorb_q, mla_absorb_q_rope and mla_out_proj (300 query
    rows) captured once: every replay equals the eager run bit for bit."""
    n_h, d_h, d_c, d_r, n = 128, 128, 512, 64, 300
    d = B.dims(n_h, d_h, d_c, d_r, B.MLA_BF16)
    gen = torch.Generator(device="cuda").manual_seed(9)
    rnd = lambda *shape, scale=1.0: (torch.randn(shape, generator=gen, device="cuda") * scale).to(torch.bfloat16)
    q_c, q_r = rnd(n, n_h, d_h), rnd(n, n_h, d_r)
    w_uk, w_uv = rnd(n_h, d_h, d_c, scale=d_c ** -0.5), rnd(n_h, d_h, d_c, scale=d_c ** -0.5)
    o_lat = torch.randn((n, n_h, d_c), generator=gen, device="cuda")
    pos = torch.randint(0, 163840, (n,), generator=gen, device="cuda", dtype=torch.int64)
    qa = torch.empty((n, n_h, d_c + d_r), dtype=torch.bfloat16, device="cuda")
    qa_r, oc = torch.empty_like(qa), torch.empty((n, n_h, d_h), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        B.absorb_q(d, q_c, q_r, w_uk, qa)
        B.absorb_q_rope(d, q_c, q_r, w_uk, pos, qa_r, rope=B.rope(yarn_factor=40.0))
        B.out_proj(d, o_lat, w_uv, oc)

    say(f"[graph] many-row kernels n_q={n}: eager")
    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (qa, qa_r, oc)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for x in (qa, qa_r, oc):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"[graph] many-row kernels replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for x, r in zip((qa, qa_r, oc), ref):
            assert torch.equal(x.view(torch.int16), r.view(torch.int16)), rep

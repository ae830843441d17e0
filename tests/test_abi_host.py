"""The C-ABI library on the host: it loads without a GPU, exports every declared
entry point, and rejects bad arguments with the documented status before launching.

No call here passes arguments that would reach a kernel launch.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from mla_latent_kv_20_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mla_kv.h", "mla_calib.h")]

FAKE = 0x100000          # 1 MiB-aligned fake device address: never dereferenced in these tests


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from mla_latent_kv_20_amd import build
        build.build()
    return B.load()


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(mla_[a-z_0-9]+)\s*\(", text, re.M)))


def test_every_declared_entry_point_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)
    assert lib.mla_abi_version() == 10


def test_calibration_argument_checks(lib):
    assert lib.mla_calib_mfma_grid() == 1024
    assert lib.mla_calib_mfma(0, FAKE, None) == B.MLA_ERR_SHAPE
    assert lib.mla_calib_mfma(10, None, None) == B.MLA_ERR_NULL
    assert lib.mla_calib_mfma_flop(10) == 1024 * 4 * 10 * 4 * 32768.0
    assert lib.mla_calib_mfma_flop(0) == 0.0
    assert lib.mla_calib_read(None, 1 << 30, 256, FAKE, None) == B.MLA_ERR_NULL
    assert lib.mla_calib_read(FAKE, 1 << 30, 0, FAKE, None) == B.MLA_ERR_SHAPE
    assert lib.mla_calib_read(FAKE, 1000, 256, FAKE, None) == B.MLA_ERR_SHAPE      # under one tile each
    assert lib.mla_calib_read(FAKE + 8, 1 << 30, 256, FAKE, None) == B.MLA_ERR_ALIGN
    assert lib.mla_calib_read_bytes(1 << 30, 256) == (1 << 30) // (256 * 36864) * 256 * 36864


def test_status_strings(lib):
    for code in range(9):
        assert lib.mla_status_string(code)
    assert lib.mla_status_string(99) == b"unknown status"


DSV2_BF16 = dict(n_h=128, d_h=128, d_c=512, d_r=64, dtype=B.MLA_BF16)


def dims(**kw):
    a = dict(DSV2_BF16)
    a.update(kw)
    return B.dims(**a)


def decode(lib, d, batch=2, q_per_seq=1, q_abs=FAKE, c_kv=FAKE, c_stride=576, k_r=FAKE + 1024,
           r_stride=576, offsets=FAKE, num_splits=1, split_rows=0, o_part=FAKE, lse_part=FAKE,
           partial=B.MLA_F32):
    return lib.mla_decode(ctypes.byref(d), batch, q_per_seq, q_abs, c_kv, c_stride, k_r, r_stride,
                          offsets, num_splits, split_rows, partial, o_part, lse_part, None)


def test_decode_argument_checks(lib):
    d = dims()
    assert lib.mla_decode(None, 2, 1, FAKE, FAKE, 576, FAKE, 576, FAKE, 1, 0, 0, FAKE, FAKE, None) == B.MLA_ERR_NULL
    assert decode(lib, d, partial=B.MLA_BF16) == B.MLA_ERR_DTYPE      # partials: fp32 or fp16
    assert decode(lib, dims(dtype=B.MLA_F32), partial=B.MLA_F16) == B.MLA_ERR_UNSUPPORTED
    assert decode(lib, d, batch=0) == B.MLA_OK                      # empty batch: no-op
    assert decode(lib, d, batch=-1) == B.MLA_ERR_SHAPE
    assert decode(lib, d, q_per_seq=0) == B.MLA_ERR_SHAPE
    assert decode(lib, d, num_splits=0) == B.MLA_ERR_SHAPE
    assert decode(lib, d, num_splits=4, split_rows=0) == B.MLA_ERR_SHAPE
    assert decode(lib, d, q_abs=None) == B.MLA_ERR_NULL
    assert decode(lib, d, offsets=None) == B.MLA_ERR_NULL
    assert decode(lib, d, o_part=None) == B.MLA_ERR_NULL
    assert decode(lib, d, c_stride=100) == B.MLA_ERR_SHAPE          # stride shorter than a latent
    assert decode(lib, dims(dtype=7)) == B.MLA_ERR_DTYPE
    assert decode(lib, dims(n_h=0)) == B.MLA_ERR_SHAPE
    assert decode(lib, dims(d_r=63)) == B.MLA_ERR_SHAPE             # RoPE works on pairs
    assert decode(lib, dims(softmax_scale=float("nan"))) == B.MLA_ERR_SHAPE
    assert decode(lib, dims(d_c=256)) == B.MLA_ERR_UNSUPPORTED      # bf16 kernel is 512 + 64
    assert decode(lib, dims(n_h=48)) == B.MLA_ERR_UNSUPPORTED       # heads go 32 per wave
    assert decode(lib, d, k_r=FAKE + 4096) == B.MLA_ERR_UNSUPPORTED  # bf16 needs packed rows
    assert decode(lib, d, c_kv=FAKE + 2, k_r=FAKE + 2 + 1024) == B.MLA_ERR_ALIGN
    assert decode(lib, d, c_stride=580, r_stride=580) == B.MLA_ERR_ALIGN
    assert decode(lib, d, offsets=FAKE + 4) == B.MLA_ERR_ALIGN
    assert decode(lib, d, q_abs=FAKE + 8) == B.MLA_ERR_ALIGN


def test_absorb_merge_out_proj_argument_checks(lib):
    d = dims()
    byref = ctypes.byref
    assert lib.mla_absorb_q(byref(d), 0, None, None, None, None, None) == B.MLA_OK
    assert lib.mla_absorb_q(byref(d), -3, FAKE, FAKE, FAKE, FAKE, None) == B.MLA_ERR_SHAPE
    assert lib.mla_absorb_q(byref(d), 4, FAKE, None, FAKE, FAKE, None) == B.MLA_ERR_NULL
    assert lib.mla_absorb_q(byref(d), 4, FAKE + 1, FAKE, FAKE, FAKE, None) == B.MLA_ERR_ALIGN
    # bf16: every operand moves in 16-byte pieces, q_r and q_abs included
    assert lib.mla_absorb_q(byref(d), 4, FAKE, FAKE + 8, FAKE, FAKE, None) == B.MLA_ERR_ALIGN
    assert lib.mla_absorb_q(byref(d), 4, FAKE, FAKE, FAKE, FAKE + 8, None) == B.MLA_ERR_ALIGN
    assert lib.mla_absorb_q_rope(byref(d), 4, FAKE, FAKE + 2, FAKE, FAKE, None, FAKE + 8, None) == B.MLA_ERR_ALIGN
    # fp32 keeps element alignment
    assert lib.mla_absorb_q(byref(dims(dtype=B.MLA_F32)), 4, FAKE, FAKE + 2, FAKE, FAKE, None) == B.MLA_ERR_ALIGN
    assert lib.mla_absorb_q(byref(dims(d_c=200)), 4, FAKE, FAKE, FAKE, FAKE, None) == B.MLA_ERR_UNSUPPORTED
    assert lib.mla_merge_splits(byref(d), 4, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == B.MLA_ERR_SHAPE
    assert lib.mla_merge_splits(byref(d), 4, 2, 0, FAKE, FAKE, None, FAKE, None) == B.MLA_ERR_NULL
    assert lib.mla_merge_splits(byref(d), 4, 2, 0, FAKE + 4, FAKE, FAKE, FAKE, None) == B.MLA_ERR_ALIGN
    assert lib.mla_merge_splits(byref(d), 4, 2, 5, FAKE, FAKE, FAKE, FAKE, None) == B.MLA_ERR_DTYPE
    assert lib.mla_merge_splits(byref(d), 0, 2, 0, None, None, None, None, None) == B.MLA_OK
    assert lib.mla_out_proj(byref(d), 4, FAKE, FAKE, None, None) == B.MLA_ERR_NULL
    assert lib.mla_out_proj(byref(d), 4, FAKE + 2, FAKE, FAKE, None) == B.MLA_ERR_ALIGN
    assert lib.mla_out_proj(byref(dims(d_h=100)), 4, FAKE, FAKE, FAKE, None) == B.MLA_ERR_UNSUPPORTED
    assert lib.mla_out_proj(byref(dims(dtype=3)), 4, FAKE, FAKE, FAKE, None) == B.MLA_ERR_DTYPE


def test_merge_out_proj_argument_checks(lib):
    d = dims()
    f = lambda d, n_q=4, S=2, part=B.MLA_F16, o_part=FAKE, lse_part=FAKE, w=FAKE, o_c=FAKE, lse=FAKE, o_lat=None: \
        lib.mla_merge_out_proj(ctypes.byref(d), n_q, S, part, o_part, lse_part, w, o_c, lse, o_lat, None)
    assert f(d, n_q=0, o_part=None, lse_part=None, w=None, o_c=None, lse=None) == B.MLA_OK
    assert f(d, n_q=-1) == B.MLA_ERR_SHAPE
    assert f(d, S=0) == B.MLA_ERR_SHAPE
    assert f(d, part=B.MLA_BF16) == B.MLA_ERR_DTYPE
    assert f(d, o_part=None) == B.MLA_ERR_NULL
    assert f(d, w=None) == B.MLA_ERR_NULL
    assert f(d, o_c=None) == B.MLA_ERR_NULL
    assert f(dims(dtype=B.MLA_F32), lse=None, o_lat=FAKE) == B.MLA_ERR_NULL   # fp32 needs both
    assert f(dims(dtype=B.MLA_F32), lse=FAKE, o_lat=None) == B.MLA_ERR_NULL
    assert f(dims(d_h=96)) == B.MLA_ERR_UNSUPPORTED                         # d_h = 128 only
    assert f(dims(d_c=256)) == B.MLA_ERR_UNSUPPORTED
    assert f(d, o_part=FAKE + 8) == B.MLA_ERR_ALIGN
    assert f(d, o_lat=FAKE + 4) == B.MLA_ERR_ALIGN
    assert f(d, lse=FAKE + 2) == B.MLA_ERR_ALIGN
    assert f(dims(dtype=9)) == B.MLA_ERR_DTYPE


def test_prologue_argument_checks(lib):
    """mla_kv_append and mla_absorb_q_rope reject bad arguments before any launch."""
    d = dims()
    app = lambda d, n=4, dm=5120, h=FAKE, wd=FAKE, wr=FAKE, pos=FAKE, dst=FAKE, rows=FAKE, stride=576, \
        ws=FAKE, wsb=1 << 30, rope=None: \
        lib.mla_kv_append(ctypes.byref(d), n, dm, h, wd, wr, pos, dst, rows, stride,
                          ctypes.byref(rope) if rope is not None else None, ws, wsb, None)
    assert app(d, n=0, h=None, wd=None, wr=None, pos=None, dst=None, rows=None, ws=None, wsb=0) == B.MLA_OK
    assert app(d, n=-1) == B.MLA_ERR_SHAPE
    assert app(d, dm=0) == B.MLA_ERR_SHAPE
    assert app(d, stride=575) == B.MLA_ERR_SHAPE                  # a row must hold d_c + d_r
    for k in ("h", "wd", "wr", "pos", "dst", "rows", "ws"):
        assert app(d, **{k: None}) == B.MLA_ERR_NULL
    need = lib.mla_kv_append_workspace_bytes(ctypes.byref(d), 4)
    assert need == 8 * 4 * 576 * 4                               # fp32 partial sums of 8 slices
    assert app(d, wsb=need - 1) == B.MLA_ERR_SHAPE
    assert app(d, pos=FAKE + 4) == B.MLA_ERR_ALIGN
    assert app(d, dst=FAKE + 2) == B.MLA_ERR_ALIGN
    assert app(d, h=FAKE + 8) == B.MLA_ERR_ALIGN                   # bf16 operands: 16-byte rows
    assert app(d, rows=FAKE + 1) == B.MLA_ERR_ALIGN
    assert app(d, ws=FAKE + 2) == B.MLA_ERR_ALIGN
    assert app(d, dm=5000) == B.MLA_ERR_UNSUPPORTED                # bf16: d_model % 512 == 0
    assert app(d, dm=9216) == B.MLA_ERR_UNSUPPORTED                # bf16: d_model <= 8192
    assert app(dims(d_r=63)) == B.MLA_ERR_SHAPE                    # RoPE pairs need an even d_r
    f32 = dims(dtype=B.MLA_F32)
    assert lib.mla_kv_append_workspace_bytes(ctypes.byref(f32), 4) == 0
    # the no-allocation form: the same checks, then the fixed array's limit, all before any
    # HIP call (so they run here, with no GPU)
    nal = lambda d, n=4, dm=5120, h=FAKE, wd=FAKE, wr=FAKE, pos=FAKE, dst=FAKE, rows=FAKE, stride=576: \
        lib.mla_kv_append_noalloc(ctypes.byref(d), n, dm, h, wd, wr, pos, dst, rows, stride, None, None)
    assert nal(d, n=0, h=None, wd=None, wr=None, pos=None, dst=None, rows=None) == B.MLA_OK
    assert nal(d, n=-1) == B.MLA_ERR_SHAPE
    for k in ("h", "wd", "wr", "pos", "dst", "rows"):
        assert nal(d, **{k: None}) == B.MLA_ERR_NULL
    assert nal(d, h=FAKE + 8) == B.MLA_ERR_ALIGN
    assert nal(d, dm=5000) == B.MLA_ERR_UNSUPPORTED
    most = B.NOALLOC_SCRATCH_BYTES // (8 * 576 * 4)
    assert most == 455
    assert lib.mla_kv_append_workspace_bytes(ctypes.byref(d), most) <= B.NOALLOC_SCRATCH_BYTES
    assert lib.mla_kv_append_workspace_bytes(ctypes.byref(d), most + 1) > B.NOALLOC_SCRATCH_BYTES
    assert nal(d, n=most + 1) == B.MLA_ERR_SCRATCH
    assert nal(d, n=4096) == B.MLA_ERR_SCRATCH
    assert b"scratch" in lib.mla_status_string(B.MLA_ERR_SCRATCH)
    rope = lambda d, n=4, qc=FAKE, qr=FAKE, w=FAKE, pos=FAKE, out=FAKE, rp=None: \
        lib.mla_absorb_q_rope(ctypes.byref(d), n, qc, qr, w, pos, ctypes.byref(rp) if rp is not None else None,
                              out, None)
    assert rope(d, n=0, qc=None, qr=None, w=None, pos=None, out=None) == B.MLA_OK
    assert rope(d, n=-2) == B.MLA_ERR_SHAPE
    assert rope(d, pos=None) == B.MLA_ERR_NULL
    assert rope(d, qr=None) == B.MLA_ERR_NULL
    assert rope(d, pos=FAKE + 4) == B.MLA_ERR_ALIGN
    assert rope(d, qr=FAKE + 1) == B.MLA_ERR_ALIGN
    assert rope(dims(d_r=1024)) == B.MLA_ERR_UNSUPPORTED           # bf16: d_r <= 512
    assert rope(dims(dtype=7)) == B.MLA_ERR_DTYPE
    # YaRN parameters: checked only when the factor turns YaRN on
    for bad in (B.rope(yarn_factor=40.0, yarn_original_len=0), B.rope(yarn_factor=40.0, yarn_beta=1.0),
                B.rope(theta=float("nan")), B.rope(yarn_factor=float("inf"))):
        assert rope(d, rp=bad) == B.MLA_ERR_SHAPE
        assert app(d, rope=bad) == B.MLA_ERR_SHAPE
    assert rope(d, rp=B.rope(yarn_factor=1.0, yarn_original_len=0), pos=FAKE + 4) == B.MLA_ERR_ALIGN   # s <= 1: plain


def test_rope_softmax_scale(lib):
    d = dims()
    base = 1.0 / np.sqrt(192.0)
    assert np.isclose(lib.mla_rope_softmax_scale(ctypes.byref(d), None), base, rtol=1e-6)
    assert np.isclose(lib.mla_rope_softmax_scale(ctypes.byref(d), ctypes.byref(B.rope())), base, rtol=1e-6)
    y = B.rope(yarn_factor=40.0)
    t = (0.0707 * np.log(40.0) + 1.0) ** 2                          # sqrt(t) = 0.0707 ln s + 1
    assert np.isclose(lib.mla_rope_softmax_scale(ctypes.byref(d), ctypes.byref(y)), base * t, rtol=1e-6)
    assert np.isclose(lib.mla_rope_softmax_scale(ctypes.byref(dims(softmax_scale=0.5)), ctypes.byref(y)),
                      0.5 * t, rtol=1e-6)
    assert lib.mla_rope_softmax_scale(None, None) == 0.0


def test_quantized_cache_argument_checks(lib):
    """mla_quantize_rows_fp8 and mla_decode_fp8 reject bad arguments before any launch."""
    d = dims()
    q = lambda d, n=4, rows=FAKE, rs=576, dst=None, codes=FAKE, cs=576, sc=FAKE: \
        lib.mla_quantize_rows_fp8(ctypes.byref(d), n, rows, rs, dst, codes, cs, sc, None)
    assert q(d, n=0, rows=None, codes=None, sc=None) == B.MLA_OK
    assert q(d, n=-1) == B.MLA_ERR_SHAPE
    assert q(d, rs=575) == B.MLA_ERR_SHAPE                         # a row holds d_c + d_r
    assert q(d, cs=575) == B.MLA_ERR_SHAPE
    for k in ("rows", "codes", "sc"):
        assert q(d, **{k: None}) == B.MLA_ERR_NULL
    assert q(d, rows=FAKE + 1) == B.MLA_ERR_ALIGN                  # bf16 elements
    assert q(d, sc=FAKE + 2) == B.MLA_ERR_ALIGN
    assert q(d, dst=FAKE + 4) == B.MLA_ERR_ALIGN
    assert q(dims(d_c=1000, d_r=64), rs=2048, cs=2048) == B.MLA_ERR_UNSUPPORTED   # width <= 1024
    assert q(dims(dtype=B.MLA_F16)) == B.MLA_ERR_DTYPE
    dec = lambda d, batch=2, qps=1, qa=FAKE, codes=FAKE, cs=576, sc=FAKE, off=FAKE, S=1, R=0, \
        part=B.MLA_F32, op=FAKE, lp=FAKE: \
        lib.mla_decode_fp8(ctypes.byref(d), batch, qps, qa, codes, cs, sc, off, S, R, part, op, lp, None)
    assert dec(d, batch=0) == B.MLA_OK
    assert dec(d, batch=-1) == B.MLA_ERR_SHAPE
    assert dec(d, qps=0) == B.MLA_ERR_SHAPE
    assert dec(d, S=3, R=0) == B.MLA_ERR_SHAPE
    assert dec(d, cs=575) == B.MLA_ERR_SHAPE
    assert dec(d, part=B.MLA_BF16) == B.MLA_ERR_DTYPE
    for k in ("qa", "codes", "sc", "off", "op", "lp"):
        assert dec(d, **{k: None}) == B.MLA_ERR_NULL
    assert dec(dims(dtype=B.MLA_F32)) == B.MLA_ERR_UNSUPPORTED      # queries are bf16
    assert dec(dims(d_c=256)) == B.MLA_ERR_UNSUPPORTED
    assert dec(dims(n_h=48)) == B.MLA_ERR_UNSUPPORTED
    assert dec(d, codes=FAKE + 8) == B.MLA_ERR_ALIGN
    assert dec(d, cs=584) == B.MLA_ERR_ALIGN                       # code rows: 16-byte multiples
    assert dec(d, sc=FAKE + 2) == B.MLA_ERR_ALIGN
    assert dec(d, qa=FAKE + 8) == B.MLA_ERR_ALIGN
    assert dec(d, off=FAKE + 4) == B.MLA_ERR_ALIGN


def test_folding_argument_checks(lib):
    d = dims()
    by = ctypes.byref
    ws = lib.mla_proj_workspace_bytes(by(d), 32, 5120, 1536)
    assert ws > 0 and ws % 4 == 0
    assert lib.mla_proj_workspace_bytes(by(dims(dtype=B.MLA_F32)), 32, 5120, 1536) == 0
    qup = lambda d, n=32, dcq=1536, cq=FAKE, w=FAKE, out=FAKE, w_s=FAKE, nb=1 << 30: \
        lib.mla_q_up(by(d), n, dcq, cq, w, out, w_s, nb, None)
    assert qup(d, n=0, cq=None, w=None, out=None, w_s=None, nb=0) == B.MLA_OK
    assert qup(d, n=-1) == B.MLA_ERR_SHAPE
    assert qup(d, dcq=1500) == B.MLA_ERR_UNSUPPORTED                 # multiples of 128
    assert qup(dims(dtype=B.MLA_F32)) == B.MLA_ERR_UNSUPPORTED
    assert qup(d, cq=None) == B.MLA_ERR_NULL
    assert qup(d, w_s=None, nb=0) == B.MLA_ERR_NULL                 # the split needs a workspace
    assert qup(d, nb=8) == B.MLA_ERR_SHAPE
    assert qup(d, cq=FAKE + 8) == B.MLA_ERR_ALIGN
    fq = lambda d, dcq=1536, a=FAKE, b=FAKE, g=FAKE: lib.mla_fold_q(by(d), dcq, a, b, g, None)
    assert fq(d, dcq=0) == B.MLA_ERR_SHAPE and fq(d, g=None) == B.MLA_ERR_NULL and fq(d, a=FAKE + 1) == B.MLA_ERR_ALIGN
    aqf = lambda d, n=32, dcq=1536, cq=FAKE, g=FAKE, qr=FAKE, out=FAKE: \
        lib.mla_absorb_q_folded(by(d), n, dcq, cq, g, qr, out, None)
    assert aqf(d, n=0, cq=None, g=None, qr=None, out=None) == B.MLA_OK
    assert aqf(d, qr=None) == B.MLA_ERR_NULL and aqf(d, g=FAKE + 4) == B.MLA_ERR_ALIGN
    assert aqf(dims(d_c=200)) == B.MLA_ERR_UNSUPPORTED
    op = lambda d, n=32, dm=5120, oc=FAKE, w=FAKE, u=FAKE, w_s=FAKE, nb=1 << 30: \
        lib.mla_o_proj(by(d), n, dm, oc, w, u, w_s, nb, None)
    assert op(d, dm=5000) == B.MLA_ERR_UNSUPPORTED and op(d, u=None) == B.MLA_ERR_NULL
    assert op(d, oc=FAKE + 2) == B.MLA_ERR_ALIGN and op(d, dm=0) == B.MLA_ERR_SHAPE
    fo = lambda d, dm=5120, a=FAKE, b=FAKE, wf=FAKE: lib.mla_fold_o(by(d), dm, a, b, wf, None)
    assert fo(d, dm=0) == B.MLA_ERR_SHAPE and fo(d, wf=None) == B.MLA_ERR_NULL
    of = lambda d, n=32, dm=5120, ol=FAKE, wf=FAKE, u=FAKE, w_s=FAKE, nb=1 << 30: \
        lib.mla_out_folded(by(d), n, dm, ol, wf, u, w_s, nb, None)
    assert of(d, ol=FAKE + 4) == B.MLA_ERR_ALIGN and of(d, wf=None) == B.MLA_ERR_NULL
    assert of(d, w_s=FAKE + 2) == B.MLA_ERR_ALIGN and of(dims(dtype=B.MLA_F32)) == B.MLA_ERR_UNSUPPORTED


def test_partial_bytes(lib):
    d = dims()
    assert lib.mla_partial_bytes(ctypes.byref(d), 32, 8, B.MLA_F32) == 8 * 32 * 128 * 512 * 4
    assert lib.mla_partial_bytes(ctypes.byref(d), 32, 8, B.MLA_F16) == 8 * 32 * 128 * 512 * 2
    assert lib.mla_partial_bytes(ctypes.byref(d), 32, 8, B.MLA_BF16) == 0
    assert lib.mla_partial_bytes(ctypes.byref(d), 32, 0, B.MLA_F32) == 0
    assert lib.mla_partial_bytes(None, 32, 1, B.MLA_F32) == 0
    # decode workspace: fp32 split results plus the split lse values
    assert lib.mla_decode_workspace_bytes(ctypes.byref(d), 32, 8) == 8 * 32 * 128 * (512 * 4 + 4)
    assert lib.mla_decode_workspace_bytes(ctypes.byref(d), 0, 8) == 0
    assert lib.mla_decode_workspace_bytes(ctypes.byref(d), 32, 0) == 0
    assert lib.mla_decode_workspace_bytes(ctypes.byref(d), -1, 8) == 0
    assert lib.mla_decode_workspace_bytes(None, 32, 8) == 0


def test_check_offsets(lib):
    ok = np.array([0, 64, 101], np.int64)
    assert B.check_offsets(ok, 2, 1, 101) == B.MLA_OK
    assert B.check_offsets(ok, 2, 1, 100) == B.MLA_ERR_SHAPE          # beyond the cache
    assert B.check_offsets(np.array([0, 64, 60], np.int64), 2, 1, 101) == B.MLA_ERR_SHAPE
    assert B.check_offsets(np.array([0, 3, 9], np.int64), 2, 4, 9) == B.MLA_ERR_SHAPE   # len < q_per_seq
    assert B.check_offsets(np.array([0, 4, 9], np.int64), 2, 4, 9) == B.MLA_OK
    assert B.check_offsets(np.array([-1, 4], np.int64), 1, 1, 9) == B.MLA_ERR_SHAPE
    assert B.check_offsets(np.zeros(1, np.int64), 0, 1, 0) == B.MLA_OK


def test_no_kernel_spills_to_scratch():
    """The build records the compiler's per-kernel resource figures; no kernel may spill (a
    spill in the decode's tile loop would cost a memory round trip per tile)."""
    import csv
    import os
    path = os.path.join(os.path.dirname(B.LIB_PATH), "kernel_resources.txt")
    if not os.path.exists(path):
        pytest.skip("library not built")
    rows = list(csv.DictReader(open(path), delimiter="\t"))
    assert any("mla_decode_bf16_kernel" in r["kernel"] for r in rows)
    for r in rows:
        assert r["ScratchSize [bytes/lane]"] == "0", r["kernel"]
        assert r["VGPRs Spill"] == "0", r["kernel"]
    # the bf16 decode holds a 128-head group per workgroup: one wave per SIMD, every register
    dec = [r for r in rows if "mla_decode_bf16_kernel" in r["kernel"]]
    assert all(int(r["VGPRs"]) + int(r["AGPRs"]) <= 512 for r in dec)

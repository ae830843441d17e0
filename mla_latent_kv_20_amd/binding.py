"""Thin ctypes binding of the MLA decode C ABI (include/mla_kv.h).

Argument marshalling only: every step runs in the HIP library ``libmla_kv.so``.
Tensors are torch tensors on the GPU (torch supplies device memory and streams);
each wrapper passes their device pointers and the current HIP stream through.
Nothing here computes a result: a missing library raises instead of falling back.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_kv.so")

MLA_OK = 0
MLA_ERR_NULL = 1
MLA_ERR_SHAPE = 2
MLA_ERR_ALIGN = 3
MLA_ERR_DTYPE = 4
MLA_ERR_UNSUPPORTED = 5
MLA_ERR_LAUNCH = 6
MLA_ERR_SCRATCH = 7
MLA_ERR_DEVICE = 8
NOALLOC_SCRATCH_BYTES = 8 << 20
MLA_F32 = 0
MLA_BF16 = 1
MLA_F16 = 2

# Every entry point the header declares, with its ctypes signature.
_I32, _I64, _F32, _P, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MlaDims(ctypes.Structure):
    _fields_ = [("n_h", _I32), ("d_h", _I32), ("d_c", _I32), ("d_r", _I32), ("dtype", _I32),
                ("softmax_scale", _F32)]


class MlaRope(ctypes.Structure):
    _fields_ = [("theta", _F32), ("yarn_factor", _F32), ("yarn_original_len", _I32), ("yarn_alpha", _F32),
                ("yarn_beta", _F32), ("yarn_mscale", _F32)]


def rope(theta: float = 10000.0, yarn_factor: float = 0.0, yarn_original_len: int = 4096,
         yarn_alpha: float = 1.0, yarn_beta: float = 32.0, yarn_mscale: float = 0.0707) -> MlaRope:
    """RoPE parameters; the YaRN defaults are DeepSeek-V2's (yarn_factor 40 turns them on)."""
    return MlaRope(theta, yarn_factor, yarn_original_len, yarn_alpha, yarn_beta, yarn_mscale)


_DIMS_P = ctypes.POINTER(MlaDims)
_ROPE_P = ctypes.POINTER(MlaRope)
SIGNATURES = {
    "mla_abi_version": (_I32, []),
    "mla_status_string": (ctypes.c_char_p, [_I32]),
    "mla_partial_bytes": (_SZ, [_DIMS_P, _I32, _I32, _I32]),
    "mla_decode_workspace_bytes": (_SZ, [_DIMS_P, _I32, _I32]),
    "mla_check_offsets": (_I32, [_P, _I32, _I32, _I64]),
    "mla_plan_splits": (_I32, [_DIMS_P, _P, _I32, _I32, _I32, _P, _P]),
    "mla_absorb_q": (_I32, [_DIMS_P, _I32, _P, _P, _P, _P, _P]),
    "mla_decode": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _I64, _P, _I64, _P, _I32, _I32, _I32, _P, _P, _P]),
    "mla_merge_splits": (_I32, [_DIMS_P, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "mla_out_proj": (_I32, [_DIMS_P, _I32, _P, _P, _P, _P]),
    "mla_merge_out_proj": (_I32, [_DIMS_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "mla_absorb_q_rope": (_I32, [_DIMS_P, _I32, _P, _P, _P, _P, _ROPE_P, _P, _P]),
    "mla_kv_append": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _I64, _ROPE_P, _P, _SZ, _P]),
    "mla_rope_softmax_scale": (_F32, [_DIMS_P, _ROPE_P]),
    "mla_proj_workspace_bytes": (_SZ, [_DIMS_P, _I32, _I32, _I32]),
    "mla_q_up": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "mla_fold_q": (_I32, [_DIMS_P, _I32, _P, _P, _P, _P]),
    "mla_absorb_q_folded": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _P, _P, _P]),
    "mla_o_proj": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "mla_fold_o": (_I32, [_DIMS_P, _I32, _P, _P, _P, _P]),
    "mla_out_folded": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "mla_kv_append_workspace_bytes": (_SZ, [_DIMS_P, _I32]),
    "mla_kv_append_noalloc": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _I64, _ROPE_P, _P]),
    "mla_quantize_rows_fp8": (_I32, [_DIMS_P, _I64, _P, _I64, _P, _P, _I64, _P, _P]),
    "mla_decode_fp8": (_I32, [_DIMS_P, _I32, _I32, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _P]),
    # device calibration (include/mla_calib.h)
    "mla_calib_mfma_grid": (_I32, []),
    "mla_calib_mfma": (_I32, [_I32, _P, _P]),
    "mla_calib_mfma_flop": (ctypes.c_double, [_I32]),
    "mla_calib_read": (_I32, [_P, _I64, _I32, _P, _P]),
    "mla_calib_read_bytes": (_I64, [_I64, _I32]),
}

_lib = None


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmla_kv.so (once).  Raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing: build it with `python -m mla_latent_kv_20_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


def dims(n_h: int, d_h: int, d_c: int, d_r: int, dtype: int, softmax_scale: float = 0.0) -> MlaDims:
    return MlaDims(n_h, d_h, d_c, d_r, dtype, softmax_scale)


def _check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MlaError(fn, status)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.float16:
        return MLA_F16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _torch_dtype(code: int):
    import torch
    return {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16, MLA_F16: torch.float16}[code]


def dims_for(q_c, q_r, w_uk, softmax_scale: float = 0.0) -> MlaDims:
    """Dimensions read off the query and weight tensors ([n_q, n_h, d_h], [n_q, n_h, d_r], [n_h, d_h, d_c])."""
    n_h, d_h, d_c = w_uk.shape
    return dims(n_h, d_h, d_c, q_r.shape[-1], _dtype_code(q_c), softmax_scale)


# ---------------------------------------------------------------------------
# The four calls
# ---------------------------------------------------------------------------

def absorb_q(d: MlaDims, q_c, q_r, w_uk, q_abs=None, stream=None):
    """q_abs[n, i] = [W^UK_i^T q_c[n, i] ; q_r[n, i]]  -> [n_q, n_h, d_c + d_r]."""
    import torch
    n_q = q_c.shape[0]
    if q_abs is None:
        q_abs = torch.empty((n_q, d.n_h, d.d_c + d.d_r), dtype=q_c.dtype, device=q_c.device)
    _check("mla_absorb_q", load().mla_absorb_q(ctypes.byref(d), n_q, _ptr(q_c), _ptr(q_r), _ptr(w_uk),
                                                _ptr(q_abs), _stream(stream)))
    return q_abs


def absorb_q_rope(d: MlaDims, q_c, q_r_raw, w_uk, positions, q_abs=None, rope: Optional[MlaRope] = None,
                  stream=None):
    """q_abs[n, i] = [W^UK_i^T q_c[n, i] ; RoPE(q_r_raw[n, i], positions[n])] (rope: MlaRope or
    None for theta 10000 without YaRN)."""
    import torch
    n_q = q_c.shape[0]
    if q_abs is None:
        q_abs = torch.empty((n_q, d.n_h, d.d_c + d.d_r), dtype=q_c.dtype, device=q_c.device)
    _check("mla_absorb_q_rope", load().mla_absorb_q_rope(ctypes.byref(d), n_q, _ptr(q_c), _ptr(q_r_raw),
                                                          _ptr(w_uk), _ptr(positions),
                                                          ctypes.byref(rope) if rope is not None else None,
                                                          _ptr(q_abs), _stream(stream)))
    return q_abs


def kv_append_workspace_bytes(d: MlaDims, n_new: int) -> int:
    return int(load().mla_kv_append_workspace_bytes(ctypes.byref(d), n_new))


def kv_append(d: MlaDims, h, w_dkv, w_kr, positions, dst_rows, rows, rope: Optional[MlaRope] = None,
              workspace=None, stream=None):
    """Write [W^DKV h_t ; RoPE(W^KR h_t, positions[t])] into cache row dst_rows[t] of `rows`
    ([*, stride] tensor, stride = rows.stride(0)); returns rows.  The workspace (bytes from
    kv_append_workspace_bytes) is allocated here when not given."""
    import torch
    n_new, d_model = h.shape
    need = kv_append_workspace_bytes(d, n_new)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("mla_kv_append", load().mla_kv_append(ctypes.byref(d), n_new, d_model, _ptr(h), _ptr(w_dkv),
                                                  _ptr(w_kr), _ptr(positions), _ptr(dst_rows), _ptr(rows),
                                                  rows.stride(0), ctypes.byref(rope) if rope is not None else None,
                                                  _ptr(workspace) if workspace is not None else None,
                                                  ws_bytes, _stream(stream)))
    return rows


def kv_append_noalloc(d: MlaDims, h, w_dkv, w_kr, positions, dst_rows, rows, rope: Optional[MlaRope] = None,
                      stream=None):
    """kv_append with the partial sums in the library's fixed device array: no workspace,
    nothing allocated here or in the call; returns rows."""
    n_new, d_model = h.shape
    _check("mla_kv_append_noalloc",
           load().mla_kv_append_noalloc(ctypes.byref(d), n_new, d_model, _ptr(h), _ptr(w_dkv), _ptr(w_kr),
                                        _ptr(positions), _ptr(dst_rows), _ptr(rows), rows.stride(0),
                                        ctypes.byref(rope) if rope is not None else None, _stream(stream)))
    return rows


def decode(d: MlaDims, q_abs, c_kv, k_r, offsets, batch: int, q_per_seq: int = 1,
           num_splits: int = 1, split_rows: int = 0, o_part=None, lse_part=None, stream=None,
           partial_dtype: int = MLA_F32):
    """Split-KV attention in latent space -> (o_part [S, n_q, n_h, d_c], lse_part [S, n_q, n_h]).

    ``c_kv`` and ``k_r`` are 2-D row views (their row strides are passed through); for the
    bf16 path they must be the two column ranges of one packed [rows, d_c + d_r] cache.
    ``offsets`` is an int64 device tensor [batch + 1].  o_part is stored in ``partial_dtype``
    (MLA_F32 or MLA_F16); a given ``o_part`` tensor decides it.
    """
    import torch
    n_q = batch * q_per_seq
    if o_part is None:
        o_part = torch.empty((num_splits, n_q, d.n_h, d.d_c), dtype=_torch_dtype(partial_dtype),
                             device=q_abs.device)
    partial_dtype = _dtype_code(o_part)
    if lse_part is None:
        lse_part = torch.empty((num_splits, n_q, d.n_h), dtype=torch.float32, device=q_abs.device)
    _check("mla_decode", load().mla_decode(
        ctypes.byref(d), batch, q_per_seq, _ptr(q_abs), _ptr(c_kv), int(c_kv.stride(0)), _ptr(k_r),
        int(k_r.stride(0)), _ptr(offsets), num_splits, split_rows, partial_dtype, _ptr(o_part),
        _ptr(lse_part), _stream(stream)))
    return o_part, lse_part


def quantize_rows_fp8(d: MlaDims, rows, dst_rows=None, codes=None, scales=None, stream=None):
    """E4M3 codes and one fp32 scale per row of ``rows`` [n, >= d_c + d_r] -> (codes, scales).

    Without ``dst_rows`` row i goes to code row i and new [n, d_c + d_r] uint8 / [n] fp32
    tensors are returned; with it, ``codes`` and ``scales`` must be given.
    """
    import torch
    n = int(rows.shape[0])
    width = d.d_c + d.d_r
    if codes is None:
        codes = torch.empty((n, width), dtype=torch.uint8, device=rows.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=rows.device)
    _check("mla_quantize_rows_fp8", load().mla_quantize_rows_fp8(
        ctypes.byref(d), n, _ptr(rows), int(rows.stride(0)), _ptr(dst_rows), _ptr(codes),
        int(codes.stride(0)), _ptr(scales), _stream(stream)))
    return codes, scales


def decode_fp8(d: MlaDims, q_abs, codes, scales, offsets, batch: int, q_per_seq: int = 1,
               num_splits: int = 1, split_rows: int = 0, o_part=None, lse_part=None, stream=None,
               partial_dtype: int = MLA_F32):
    """mla_decode over a quantized cache (uint8 code rows ``codes``, fp32 ``scales``)."""
    import torch
    n_q = batch * q_per_seq
    if o_part is None:
        o_part = torch.empty((num_splits, n_q, d.n_h, d.d_c), dtype=_torch_dtype(partial_dtype),
                             device=q_abs.device)
    partial_dtype = _dtype_code(o_part)
    if lse_part is None:
        lse_part = torch.empty((num_splits, n_q, d.n_h), dtype=torch.float32, device=q_abs.device)
    _check("mla_decode_fp8", load().mla_decode_fp8(
        ctypes.byref(d), batch, q_per_seq, _ptr(q_abs), _ptr(codes), int(codes.stride(0)), _ptr(scales),
        _ptr(offsets), num_splits, split_rows, partial_dtype, _ptr(o_part), _ptr(lse_part), _stream(stream)))
    return o_part, lse_part


def merge_splits(d: MlaDims, o_part, lse_part, o_lat=None, lse=None, stream=None):
    """Log-sum-exp merge of split results -> (o_lat [n_q, n_h, d_c], lse [n_q, n_h])."""
    import torch
    S, n_q = o_part.shape[0], o_part.shape[1]
    if o_lat is None:
        o_lat = torch.empty((n_q, d.n_h, d.d_c), dtype=torch.float32, device=o_part.device)
    if lse is None:
        lse = torch.empty((n_q, d.n_h), dtype=torch.float32, device=o_part.device)
    _check("mla_merge_splits", load().mla_merge_splits(ctypes.byref(d), n_q, S, _dtype_code(o_part),
                                                        _ptr(o_part), _ptr(lse_part), _ptr(o_lat),
                                                        _ptr(lse), _stream(stream)))
    return o_lat, lse


def out_proj(d: MlaDims, o_lat, w_uv, o_c=None, out_dtype=None, stream=None):
    """o_c[n, i] = W^UV_i o_lat[n, i]  -> [n_q, n_h, d_h] in the weights' dtype."""
    import torch
    n_q = o_lat.shape[0]
    if o_c is None:
        o_c = torch.empty((n_q, d.n_h, d.d_h), dtype=out_dtype or w_uv.dtype, device=o_lat.device)
    _check("mla_out_proj", load().mla_out_proj(ctypes.byref(d), n_q, _ptr(o_lat), _ptr(w_uv), _ptr(o_c),
                                                _stream(stream)))
    return o_c


def merge_out_proj(d: MlaDims, o_part, lse_part, w_uv, o_c=None, lse=None, o_lat=None,
                   want_lse: bool = True, want_o_lat: bool = False, stream=None):
    """mla_merge_splits then mla_out_proj in one call -> (o_c, lse or None, o_lat or None)."""
    import torch
    S, n_q = o_part.shape[0], o_part.shape[1]
    dev = o_part.device
    if o_c is None:
        o_c = torch.empty((n_q, d.n_h, d.d_h), dtype=w_uv.dtype, device=dev)
    if lse is None and (want_lse or d.dtype == MLA_F32):
        lse = torch.empty((n_q, d.n_h), dtype=torch.float32, device=dev)
    if o_lat is None and (want_o_lat or d.dtype == MLA_F32):
        o_lat = torch.empty((n_q, d.n_h, d.d_c), dtype=torch.float32, device=dev)
    _check("mla_merge_out_proj", load().mla_merge_out_proj(
        ctypes.byref(d), n_q, S, _dtype_code(o_part), _ptr(o_part), _ptr(lse_part), _ptr(w_uv), _ptr(o_c),
        _ptr(lse), _ptr(o_lat), _stream(stream)))
    return o_c, lse, o_lat


def check_offsets(host_offsets, batch: int, q_per_seq: int, total_rows: int) -> int:
    """mla_check_offsets on a host int64 numpy array; returns the status code."""
    import numpy as np
    a = np.ascontiguousarray(host_offsets, dtype=np.int64)
    return int(load().mla_check_offsets(a.ctypes.data if a.size else None, batch, q_per_seq, total_rows))


def plan_splits(d: MlaDims, host_offsets, batch: int, q_per_seq: int, max_splits: int = 64):
    """mla_plan_splits on a host int64 numpy array: (num_splits, split_rows)."""
    import numpy as np
    a = np.ascontiguousarray(host_offsets, dtype=np.int64)
    ns, sr = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("mla_plan_splits", load().mla_plan_splits(ctypes.byref(d), a.ctypes.data if a.size else None, batch,
                                                     q_per_seq, max_splits, ctypes.byref(ns), ctypes.byref(sr)))
    return ns.value, sr.value


def default_partial_dtype(d: MlaDims, num_splits: int) -> int:
    """fp16 split results for the bf16 path when there is a merge to do, else fp32."""
    return MLA_F16 if d.dtype == MLA_BF16 and num_splits > 1 else MLA_F32


def decode_step(d: MlaDims, q_c, q_r, w_uk, w_uv, cache, offsets, batch: int, q_per_seq: int = 1,
                num_splits: int = 1, split_rows: int = 0, bufs: Optional[dict] = None, stream=None,
                partial_dtype: Optional[int] = None, fused: bool = False):
    """One decode step on a packed cache [rows, d_c + d_r]; returns the output buffers.

    ``bufs`` may hold preallocated q_abs / o_part / lse_part / o_lat / lse / o_c tensors.
    Unfused: the four calls; with one fp32 split the decode's results already are o_lat
    and lse.  Fused: mla_absorb_q, mla_decode, mla_merge_out_proj (o_lat is written only
    when ``bufs`` holds it).
    """
    if partial_dtype is None:
        partial_dtype = default_partial_dtype(d, num_splits)
    b = {} if bufs is None else bufs
    q_abs = absorb_q(d, q_c, q_r, w_uk, b.get("q_abs"), stream)
    c_kv = cache[:, :d.d_c]
    k_r = cache[:, d.d_c:d.d_c + d.d_r]
    o_part, lse_part = decode(d, q_abs, c_kv, k_r, offsets, batch, q_per_seq, num_splits, split_rows,
                              b.get("o_part"), b.get("lse_part"), stream, partial_dtype)
    if fused:
        o_c, lse, o_lat = merge_out_proj(d, o_part, lse_part, w_uv, b.get("o_c"), b.get("lse"),
                                         b.get("o_lat"), stream=stream)
        return dict(q_abs=q_abs, o_part=o_part, lse_part=lse_part, o_lat=o_lat, lse=lse, o_c=o_c)
    if num_splits == 1 and _dtype_code(o_part) == MLA_F32:
        o_lat, lse = o_part[0], lse_part[0]
    else:
        o_lat, lse = merge_splits(d, o_part, lse_part, b.get("o_lat"), b.get("lse"), stream)
    o_c = out_proj(d, o_lat, w_uv, b.get("o_c"), stream=stream)
    return dict(q_abs=q_abs, o_part=o_part, lse_part=lse_part, o_lat=o_lat, lse=lse, o_c=o_c)


def proj_workspace_bytes(d: MlaDims, n_q: int, d_model: int, d_cq: int) -> int:
    return int(load().mla_proj_workspace_bytes(ctypes.byref(d), n_q, d_model, d_cq))


def _ws(workspace, need, device):
    import torch
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return workspace, nbytes


def q_up(d: MlaDims, c_q, w_uq, q_c=None, workspace=None, stream=None):
    """q^C = W^UQ c^Q: c_q [n_q, d_cq], w_uq [n_h, d_h, d_cq] -> [n_q, n_h, d_h] bf16."""
    import torch
    n_q, d_cq = c_q.shape
    if q_c is None:
        q_c = torch.empty((n_q, d.n_h, d.d_h), dtype=torch.bfloat16, device=c_q.device)
    ws, nb = _ws(workspace, proj_workspace_bytes(d, n_q, d.d_c, d_cq), c_q.device)
    _check("mla_q_up", load().mla_q_up(ctypes.byref(d), n_q, d_cq, _ptr(c_q), _ptr(w_uq), _ptr(q_c), _ptr(ws), nb,
                                       _stream(stream)))
    return q_c


def fold_q(d: MlaDims, w_uq, w_uk, g=None, stream=None):
    """G_i = (W^UK_i)^T W^UQ_i -> [n_h, d_c, d_cq] bf16."""
    import torch
    d_cq = w_uq.shape[2]
    if g is None:
        g = torch.empty((d.n_h, d.d_c, d_cq), dtype=torch.bfloat16, device=w_uq.device)
    _check("mla_fold_q", load().mla_fold_q(ctypes.byref(d), d_cq, _ptr(w_uq), _ptr(w_uk), _ptr(g), _stream(stream)))
    return g


def absorb_q_folded(d: MlaDims, c_q, g, q_r, q_abs=None, stream=None):
    """q_abs[n, i] = [G_i c^Q[n] ; q_r[n, i]] -> [n_q, n_h, d_c + d_r] bf16."""
    import torch
    n_q, d_cq = c_q.shape
    if q_abs is None:
        q_abs = torch.empty((n_q, d.n_h, d.d_c + d.d_r), dtype=torch.bfloat16, device=c_q.device)
    _check("mla_absorb_q_folded", load().mla_absorb_q_folded(ctypes.byref(d), n_q, d_cq, _ptr(c_q), _ptr(g),
                                                              _ptr(q_r), _ptr(q_abs), _stream(stream)))
    return q_abs


def o_proj(d: MlaDims, o_c, w_o, u=None, workspace=None, stream=None):
    """u = W^O [o^C_1; ...; o^C_nh]: o_c [n_q, n_h, d_h], w_o [d_model, n_h d_h] -> [n_q, d_model]."""
    import torch
    n_q = o_c.shape[0]
    d_model = w_o.shape[0]
    if u is None:
        u = torch.empty((n_q, d_model), dtype=torch.bfloat16, device=o_c.device)
    ws, nb = _ws(workspace, proj_workspace_bytes(d, n_q, d_model, 128), o_c.device)
    _check("mla_o_proj", load().mla_o_proj(ctypes.byref(d), n_q, d_model, _ptr(o_c), _ptr(w_o), _ptr(u), _ptr(ws),
                                           nb, _stream(stream)))
    return u


def fold_o(d: MlaDims, w_o, w_uv, w_fold=None, stream=None):
    """W'^O_i = W^O_i W^UV_i side by side -> [d_model, n_h d_c] bf16."""
    import torch
    d_model = w_o.shape[0]
    if w_fold is None:
        w_fold = torch.empty((d_model, d.n_h * d.d_c), dtype=torch.bfloat16, device=w_o.device)
    _check("mla_fold_o", load().mla_fold_o(ctypes.byref(d), d_model, _ptr(w_o), _ptr(w_uv), _ptr(w_fold),
                                           _stream(stream)))
    return w_fold


def out_folded(d: MlaDims, o_lat, w_fold, u=None, workspace=None, stream=None):
    """u = W'^O [o_lat_1; ...]: o_lat [n_q, n_h, d_c] fp32 -> [n_q, d_model] bf16."""
    import torch
    n_q = o_lat.shape[0]
    d_model = w_fold.shape[0]
    if u is None:
        u = torch.empty((n_q, d_model), dtype=torch.bfloat16, device=o_lat.device)
    ws, nb = _ws(workspace, proj_workspace_bytes(d, n_q, d_model, 128), o_lat.device)
    _check("mla_out_folded", load().mla_out_folded(ctypes.byref(d), n_q, d_model, _ptr(o_lat), _ptr(w_fold), _ptr(u),
                                                   _ptr(ws), nb, _stream(stream)))
    return u


def rope_softmax_scale(d: MlaDims, rope: Optional[MlaRope] = None) -> float:
    """The softmax scale with YaRN's length factor (mla_rope_softmax_scale)."""
    return float(load().mla_rope_softmax_scale(ctypes.byref(d), ctypes.byref(rope) if rope is not None else None))



# ---------------------------------------------------------------------------
# Device calibration (include/mla_calib.h): the benchmark brackets these with events.
# ---------------------------------------------------------------------------

def calib_mfma(iters: int, out=None):
    """Back-to-back bf16 MFMAs on every SIMD; returns (out buffer, FLOPs of the launch)."""
    import torch
    lib = load()
    n = int(lib.mla_calib_mfma_grid()) * 256
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    _check("mla_calib_mfma", lib.mla_calib_mfma(int(iters), _ptr(out), _stream(None)))
    return out, float(lib.mla_calib_mfma_flop(int(iters)))


def calib_read(src, workgroups: int = 256, out=None):
    """Streaming read of (most of) the device tensor src; returns (out buffer, bytes read)."""
    import torch
    lib = load()
    if out is None:
        out = torch.empty(int(workgroups), dtype=torch.float32, device=src.device)
    nbytes = src.numel() * src.element_size()
    _check("mla_calib_read", lib.mla_calib_read(_ptr(src), int(nbytes), int(workgroups), _ptr(out), _stream(None)))
    return out, int(lib.mla_calib_read_bytes(int(nbytes), int(workgroups)))

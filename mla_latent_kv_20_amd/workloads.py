"""Seeded synthetic workloads for MLA absorbed decode over a latent KV cache.

These are the inputs both sides consume: the oracle (fp64, on the CPU) and the
HIP path (bf16 or fp32, on the GPU).  The module uses numpy only and holds no
step of the decode itself.  It draws Gaussian tensors, rotates the decoupled
RoPE parts at their token positions, and rounds to the storage precision.  The
rotation belongs here because the pages cache the shared key k^R already
rotated and feed the query's q^R rotated at its own position ("Техотчёт
DeepSeek-V2 (2024): MLA и экономика инференса", section "Идея 2";
"MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리", section "Decoupled
Rotary Position Embedding"); the decode consumes both as plain vectors.

Shapes follow the DeepSeek-V2 attention dimensions (n_h=128, d_h=128, d_c=512,
d_h^R=64; "DeepSeek-V2 review" section 4.1; DeepSeek-V3 Technical Report notes,
"Multi-Head Latent Attention" dimension list).  Every array is a numpy array:

  c_kv   [rows, d_c]          latent rows of all sequences, back to back
  k_r    [rows, d_r]          shared RoPE key of each row, already rotated
  offsets[batch+1] int64      sequence b owns rows offsets[b] .. offsets[b+1]-1
  q_c    [n_q, n_h, d_h]      n_q = batch * q_per_seq, query-major per sequence
  q_r    [n_q, n_h, d_r]      rotated at the query's own position
  w_uk   [n_h, d_h, d_c]      up-projection for keys (k^C_i = W^UK_i c)
  w_uv   [n_h, d_h, d_c]      up-projection for values (v^C_i = W^UV_i c)

bf16 arrays are held as their raw 16-bit patterns (uint16); fp32 arrays as
float32.  ``to_f64`` widens either exactly.

Draw order (fixed, one numpy PCG64 generator seeded per workload): sequence
lengths (ragged workloads only), c_kv, raw k_r, q_c, raw q_r, w_uk, w_uv, then
the appended new rows (c_kv, raw k_r) of multi-token workloads.  Normals are
drawn in fp64 and rounded once, with round-to-nearest-even, to the storage type.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Rows drawn per generator call for the big caches; consecutive calls on one
# PCG64 generator continue the same normal stream, so chunking does not change
# any value (a CPU test checks this).
_DRAW_CHUNK_ROWS = 1 << 16


# ----------------------------------------------------------------------------
# bf16 rounding (exact, numpy only)
# ----------------------------------------------------------------------------

def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, nearest-even); return bit patterns.

    Rounds once, directly from fp64, so no double rounding through fp32.
    Magnitudes below the smallest normal fp32 (2^-126) flush to signed zero;
    a N(0, sigma) draw with sigma near 1 never reaches them in practice.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0) * (1.0 / 256.0)   # keep 8 significant bits, ties to even
    r = np.ldexp(q, e)
    r = np.where(np.abs(r) < 2.0 ** -126, np.copysign(0.0, x), r)
    f32 = r.astype(np.float32)               # exact: r has 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp64 exactly."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_from_f64(x)
    if dtype == F32:
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f64_from_bf16_bits(a)
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# RoPE, rotate-half form (input preparation only)
# ----------------------------------------------------------------------------

def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of ``x`` by RoPE at ``positions`` (fp64 angles).

    Rotate-half convention of the RoPE helpers in "MLA(Multi-head Latent
    Attention): DeepSeek-V2 논문정리", section "MLA 코드 구현": frequency
    k (0 <= k < d/2) is theta^(-2k/d), the angle table repeats the d/2
    frequencies over both halves, and RoPE(x) = x*cos + rotate_half(x)*sin with
    rotate_half([x1, x2]) = [-x2, x1].  ``positions`` broadcasts against
    x[..., 0].  Angles are formed in fp64 so that positions past 10^5 keep full
    resolution.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE width must be even")
    half = d // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq    # [..., d/2]
    cos = np.cos(ang)
    sin = np.sin(ang)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# ----------------------------------------------------------------------------
# Workload container
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    n_h: int
    d_h: int
    d_c: int
    d_r: int
    dtype: str                      # BF16 or F32: storage of every tensor input and of q_abs / o_c
    q_per_seq: int
    lengths: np.ndarray             # int64 [batch], rows per sequence (new rows included)
    offsets: np.ndarray             # int64 [batch+1]
    c_kv: np.ndarray
    k_r: np.ndarray
    q_c: np.ndarray
    q_r: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    num_splits: int = 1             # default split plan for this workload
    split_rows: int = 0
    seed: int = 0
    note: str = ""

    @property
    def batch(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def n_q(self) -> int:
        return self.batch * self.q_per_seq

    @property
    def rows(self) -> int:
        return int(self.offsets[-1])

    @property
    def d_qk(self) -> int:
        return self.d_c + self.d_r

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h + self.d_r)

    def f64(self, field: str) -> np.ndarray:
        return to_f64(getattr(self, field), self.dtype)

    def cached_rows(self) -> int:
        """Rows that were in the cache before this step's new tokens (the metric's unit)."""
        return self.rows - (self.batch * self.q_per_seq if self.note == "appended" else 0)


def _draw_rows(rng: np.random.Generator, n_rows: int, width: int, scale: float,
               dtype: str, post=None) -> np.ndarray:
    """Draw an [n_rows, width] N(0, scale^2) matrix in row chunks, rounded to storage.

    ``post(chunk_f64, row0)`` may transform each fp64 chunk before rounding.
    """
    out = np.empty((n_rows, width), dtype=np.uint16 if dtype == BF16 else np.float32)
    r0 = 0
    while r0 < n_rows:
        r1 = min(n_rows, r0 + _DRAW_CHUNK_ROWS)
        v = rng.standard_normal((r1 - r0, width))
        if scale != 1.0:
            v *= scale
        if post is not None:
            v = post(v, r0)
        out[r0:r1] = round_to_storage(v, dtype)
        r0 = r1
    return out


def make_workload(name: str, *, n_h: int, d_h: int, d_c: int, d_r: int, dtype: str,
                  lengths: Optional[Sequence[int]] = None,
                  ragged_range: Optional[tuple] = None, ragged_batch: int = 0,
                  q_per_seq: int = 1, appended_rows: bool = False,
                  q_mult: float = 1.0, padded_draw: bool = False,
                  num_splits: int = 1, split_rows: int = 0,
                  theta: float = 10000.0, seed: int = 0) -> Workload:
    """Draw one workload.

    lengths       cached rows per sequence (before any appended rows); or
    ragged_range  (lo, hi) inclusive: lengths drawn first, uniformly, for ragged_batch sequences.
    q_per_seq     query tokens per sequence; query r sits at position T_b + r.
    appended_rows the q_per_seq new tokens' own rows (positions T_b..T_b+q_per_seq-1) are drawn
                  after the weights and appended to each sequence, so query r attends rows
                  0..T_b+r (the generalized causal mask).  Without it q_per_seq must be 1 and
                  the single query at position T_b attends all T_b cached rows.
    q_mult        multiplies q_c and q_r (logit std scales by the same factor).
    padded_draw   draw the cache as a padded [batch, max T, .] block and keep each sequence's
                  first T_b rows (the tiny config's literal [B, T, .] shapes).
    """
    rng = np.random.default_rng(seed)
    if ragged_range is not None:
        lo, hi = ragged_range
        lens = rng.integers(lo, hi + 1, size=ragged_batch).astype(np.int64)
    else:
        lens = np.asarray(lengths, dtype=np.int64)
    if q_per_seq > 1 and not appended_rows:
        raise ValueError("several queries per sequence need their own appended rows")
    B = int(lens.shape[0])
    n_q = B * q_per_seq
    cached_offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n_cached = int(cached_offsets[-1])
    # position of every cached row within its sequence
    seq_of_row = np.repeat(np.arange(B), lens)
    pos_of_row = np.arange(n_cached, dtype=np.int64) - cached_offsets[seq_of_row]

    if padded_draw:
        tmax = int(lens.max())
        pad_c = rng.standard_normal((B, tmax, d_c))
        pad_r = rng.standard_normal((B, tmax, d_r))
        pad_r = rope_rotate(pad_r, np.arange(tmax)[None, :])
        keep = np.arange(tmax)[None, :] < lens[:, None]
        c_kv = round_to_storage(pad_c[keep], dtype)
        k_r = round_to_storage(pad_r[keep], dtype)
    else:
        c_kv = _draw_rows(rng, n_cached, d_c, 1.0, dtype)
        k_r = _draw_rows(rng, n_cached, d_r, 1.0, dtype,
                         post=lambda v, r0: rope_rotate(v, pos_of_row[r0:r0 + v.shape[0]], theta))

    q_pos = (lens[:, None] + np.arange(q_per_seq)[None, :]).reshape(n_q)      # [n_q]
    q_c = rng.standard_normal((n_q, n_h, d_h)) * q_mult
    q_r = rng.standard_normal((n_q, n_h, d_r)) * q_mult
    q_r = rope_rotate(q_r, q_pos[:, None], theta)
    w_std = 1.0 / math.sqrt(d_c)
    w_uk = rng.standard_normal((n_h, d_h, d_c)) * w_std
    w_uv = rng.standard_normal((n_h, d_h, d_c)) * w_std
    q_c = round_to_storage(q_c, dtype)
    q_r = round_to_storage(q_r, dtype)
    w_uk = round_to_storage(w_uk, dtype)
    w_uv = round_to_storage(w_uv, dtype)

    note = ""
    if appended_rows:
        new_c = rng.standard_normal((B, q_per_seq, d_c))
        new_r = rope_rotate(rng.standard_normal((B, q_per_seq, d_r)), q_pos.reshape(B, q_per_seq))
        new_c = round_to_storage(new_c, dtype)
        new_r = round_to_storage(new_r, dtype)
        total = lens + q_per_seq
        offsets = np.concatenate([[0], np.cumsum(total)]).astype(np.int64)
        c_all = np.empty((int(offsets[-1]), d_c), dtype=c_kv.dtype)
        r_all = np.empty((int(offsets[-1]), d_r), dtype=k_r.dtype)
        for b in range(B):
            o, t, s = int(offsets[b]), int(lens[b]), int(cached_offsets[b])
            c_all[o:o + t] = c_kv[s:s + t]
            r_all[o:o + t] = k_r[s:s + t]
            c_all[o + t:o + t + q_per_seq] = new_c[b]
            r_all[o + t:o + t + q_per_seq] = new_r[b]
        c_kv, k_r, lens = c_all, r_all, total
        note = "appended"
    else:
        offsets = cached_offsets

    return Workload(name=name, n_h=n_h, d_h=d_h, d_c=d_c, d_r=d_r, dtype=dtype,
                    q_per_seq=q_per_seq, lengths=lens, offsets=offsets,
                    c_kv=c_kv, k_r=k_r, q_c=q_c, q_r=q_r, w_uk=w_uk, w_uv=w_uv,
                    num_splits=num_splits, split_rows=split_rows, seed=seed, note=note)


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------

DSV2 = dict(n_h=128, d_h=128, d_c=512, d_r=64)

# name -> (description, keyword arguments of make_workload)
CONFIGS: Dict[str, tuple] = {
    "tiny_f32": (
        "B=2, T=(64,37), n_h=4, d_h=16, d_c=32, d_h^R=8, fp32",
        dict(n_h=4, d_h=16, d_c=32, d_r=8, dtype=F32, lengths=[64, 37], padded_draw=True)),
    "dsv2_b32_t4096": (
        "DeepSeek-V2 dims, B=32, T=4096, bf16",
        dict(**DSV2, dtype=BF16, lengths=[4096] * 32, num_splits=8, split_rows=512)),
    "dsv2_b4_t131072": (
        "DeepSeek-V2 dims, B=4, T=131072, bf16, 64 KV splits",
        dict(**DSV2, dtype=BF16, lengths=[131072] * 4, num_splits=64, split_rows=2048)),
    "dsv2_ragged_b128": (
        "DeepSeek-V2 dims, B=128, T~U{512..16384}, queries x3 (logit std ~3), bf16",
        dict(**DSV2, dtype=BF16, ragged_range=(512, 16384), ragged_batch=128, q_mult=3.0,
             num_splits=4, split_rows=4544)),
    "dsv2_mtp4_b64_t8192": (
        "DeepSeek-V2 dims, B=64, T=8192 cached + 4 new rows, 4 queries/seq, causal among new, bf16",
        dict(**DSV2, dtype=BF16, lengths=[8192] * 64, q_per_seq=4, appended_rows=True,
             num_splits=1, split_rows=0)),
    # prefill (T_q = T_k, causal): every row is a new token's own row and query r sees rows
    # 0..r, the generalized mask with no cached rows
    "dsv2_prefill_b1_t4096": (
        "DeepSeek-V2 dims, prefill of one 4096-token sequence (causal), bf16",
        dict(**DSV2, dtype=BF16, lengths=[0], q_per_seq=4096, appended_rows=True,
             num_splits=1, split_rows=0)),
    "dsv2_prefill_small": (
        "DeepSeek-V2 dims, prefill of two 83-token sequences (causal), bf16",
        dict(**DSV2, dtype=BF16, lengths=[0, 0], q_per_seq=83, appended_rows=True,
             num_splits=2, split_rows=48)),
    # extra shapes (not measured): the toy module dims of "MLA(Multi-head Latent Attention):
    # DeepSeek-V2 논문정리" section "MLA 코드 구현", and small DeepSeek-V2-shaped caches
    "toy_p3": (
        "toy dims n_h=96, d_h=8, d_c=64, d_h^R=16 (d_h^R > d_h), fp32",
        dict(n_h=96, d_h=8, d_c=64, d_r=16, dtype=F32, lengths=[10, 11, 3])),
    "dsv2_small": (
        "DeepSeek-V2 dims, B=3, T=(1, 77, 1000), bf16",
        dict(**DSV2, dtype=BF16, lengths=[1, 77, 1000], num_splits=3, split_rows=256)),
    "dsv2_ragged_small": (
        "DeepSeek-V2 dims, B=19, T~U{1..400}, queries x3, bf16 (sequences dealt to XCDs by length)",
        dict(**DSV2, dtype=BF16, ragged_range=(1, 400), ragged_batch=19, q_mult=3.0,
             num_splits=4, split_rows=96)),
    "dsv2_small_mtp": (
        "DeepSeek-V2 dims, B=2, T=(3, 250) + 4 new rows, 4 queries/seq, bf16",
        dict(**DSV2, dtype=BF16, lengths=[3, 250], q_per_seq=4, appended_rows=True,
             num_splits=2, split_rows=128)),
}


def make_config(name: str, seed: int = 0, **overrides) -> Workload:
    """Draw the named workload (all named workloads use seed 0 unless told otherwise)."""
    _, kw = CONFIGS[name]
    kw = dict(kw)
    kw.update(overrides)
    return make_workload(name, seed=seed, **kw)


# ----------------------------------------------------------------------------
# Inputs for testing one call on its own (drawn, never computed from another call)
# ----------------------------------------------------------------------------

def draw_q_abs(w: Workload, seed: int = 1, q_mult: float = 1.0) -> np.ndarray:
    """Absorbed queries [n_q, n_h, d_c + d_r] in storage type, drawn directly.

    The latent part has the variance of W^UK^T q^C for unit queries and weights of
    variance 1/d_c (that is d_h/d_c); the RoPE part is unit variance.
    """
    rng = np.random.default_rng(seed)
    lat = rng.standard_normal((w.n_q, w.n_h, w.d_c)) * math.sqrt(w.d_h / w.d_c) * q_mult
    rope = rng.standard_normal((w.n_q, w.n_h, w.d_r)) * q_mult
    return round_to_storage(np.concatenate([lat, rope], axis=2), w.dtype)


def draw_partials(num_splits: int, n_q: int, n_h: int, d_c: int, seed: int = 2,
                  empty_frac: float = 0.2):
    """Split results (o_part fp32 [S, n_q, n_h, d_c], lse_part fp32 [S, n_q, n_h]).

    A fraction of the (split, query, head) entries are empty splits (lse = -inf, o = 0);
    the first split of every query head is never empty.
    """
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((num_splits, n_q, n_h, d_c)).astype(np.float32)
    lse = (rng.standard_normal((num_splits, n_q, n_h)) * 3.0 + 5.0).astype(np.float32)
    empty = rng.random((num_splits, n_q, n_h)) < empty_frac
    empty[0] = False
    lse[empty] = -np.inf
    o[empty] = 0.0
    return o, lse


def draw_o_lat(n_q: int, n_h: int, d_c: int, seed: int = 3) -> np.ndarray:
    """Latent attention outputs [n_q, n_h, d_c] fp32 (scale of a softmax-weighted mean)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n_q, n_h, d_c)) * 0.05).astype(np.float32)


@dataclasses.dataclass
class Prologue:
    """Inputs of the decode prologue for n_new new tokens (storage type, drawn directly).

    h [n_new, d_model] hidden states ~ N(0, 1); w_dkv [d_c, d_model] and w_kr [d_r, d_model]
    ~ N(0, 1/d_model) (unit-variance outputs, as for the other weights); q_r_raw
    [n_new, n_h, d_r] ~ N(0, 1), the query's RoPE part before rotation; positions [n_new]
    and dst_rows [n_new] int64.
    """
    dtype: str
    d_model: int
    h: np.ndarray
    w_dkv: np.ndarray
    w_kr: np.ndarray
    q_r_raw: np.ndarray
    positions: np.ndarray
    dst_rows: np.ndarray


def draw_prologue(w: Workload, d_model: int, positions, dst_rows, seed: int = 4) -> Prologue:
    """Prologue inputs for len(positions) new tokens with the dimensions of workload w."""
    rng = np.random.default_rng(seed)
    n = len(positions)
    h = rng.standard_normal((n, d_model))
    w_dkv = rng.standard_normal((w.d_c, d_model)) * math.sqrt(1.0 / d_model)
    w_kr = rng.standard_normal((w.d_r, d_model)) * math.sqrt(1.0 / d_model)
    q_r_raw = rng.standard_normal((n, w.n_h, w.d_r))
    pos = np.asarray(positions, np.int64).reshape(n)
    dst = np.asarray(dst_rows, np.int64).reshape(n)
    return Prologue(w.dtype, d_model, round_to_storage(h, w.dtype), round_to_storage(w_dkv, w.dtype),
                    round_to_storage(w_kr, w.dtype), round_to_storage(q_r_raw, w.dtype), pos, dst)

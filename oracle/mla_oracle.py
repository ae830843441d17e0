"""CPU oracle for MLA decode over a latent KV cache (fp64, numpy).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline use this module.  The library in ``mla_latent_kv_20_amd`` never
imports it, and it imports nothing from there: inputs reach it as plain numpy
arrays (fp64, widened exactly from the storage type).

Pages cited (title, then section / equation):
  [review]  "DeepSeek-V2 review" (velog.io/@jmsong62)
  [obsidian] "DeepSeek-V2: A Strong, Economical, and Efficient Mixture-of-Experts Language Model"
  [notes]   "MLA(Multi-head Latent Attention): DeepSeek-V2 논문정리"
  [report]  "Техотчёт DeepSeek-V2 (2024): MLA и экономика инференса"
  [v3]      DeepSeek-V3 Technical Report notes (xuxeong.tistory.com), "Multi-Head Latent Attention"

Notation follows the pages:
  c^KV_j  latent row j, width d_c                          ([notes] eq. 9)
  k^C_{j,i} = W^UK_i c^KV_j, v^C_{j,i} = W^UV_i c^KV_j      ([notes] eq. 10, 11); W^UK_i is [d_h, d_c]
  k^R_j   decoupled RoPE key, width d_h^R, one per row shared by all heads
          ([notes] "Decoupled Rotary Position Embedding", item 3; [review] 2.3; [report] "Идея 2")
  q_{t,i} = [q^C_{t,i}; q^R_{t,i}],  k_{j,i} = [k^C_{j,i}; k^R_j]
  o_{t,i} = sum_j softmax_j(q_{t,i}^T k_{j,i} / sqrt(d_h + d_h^R)) v^C_{j,i}
          ([v3] eq. 10; [report] "Идея 2"; [obsidian] "Multi-head Latent Attention (MLA)" prints the
           same sum with the square root lost in extraction)
  mask    query r of T_q new queries against T_k rows sees rows j <= T_k - T_q + r
          ([notes] "MLA 코드 구현": triu of -inf with diagonal T_k - T_q + 1)

Two formulations are computed independently:
  naive_decode     materializes k^C and v^C for every row and head, then runs textbook
                   softmax attention: the pages' definition.
  absorbed_decode  folds W^UK into the query and applies W^UV after the weighted sum of
                   latents ([notes] "Key에 대한 수식 전개" and "Value에 대한 수식 전개";
                   [report] "Идея 1"): the form the GPU path computes.
and the per-call pieces of the absorbed form (absorb_q, split_partials, merge_splits,
out_proj) that the C-ABI entry points are compared against one by one.  The decode
prologue (kv_prologue, append_rows, absorb_q_rope) gives the new tokens' cache rows and
the rotated queries from the hidden states.  A quantized cache (e4m3_value, e4m3_encode,
quantize_rows, dequantize_rows) stores each row as FP8 E4M3 codes with one scale per row;
its decode is the decode above over the dequantized rows.  Offline weight folding (q_up,
fold_q, absorb_q_folded, o_proj, fold_o, out_folded) gives the path from the compressed
query c^Q to the attention block's output u in the unfolded and the folded forms.

Readings where the pages are silent or garbled (each is listed in the design notes):
  * scale 1/sqrt(d_h + d_h^R) (three pages agree; one prints it without the root);
  * k^R is one vector per row shared by every head (three pages; one page's code
    gives each head its own and never uses it);
  * log-sum-exp is the natural log of sum_j exp(scaled logit);
  * a split (a contiguous range of rows) that holds no visible row has lse = -inf
    and a zero output; the merge gives it weight zero.
"""

from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np


def default_scale(d_h: int, d_r: int) -> float:
    """1/sqrt(d_h + d_h^R): the attention normalisation of decoupled-RoPE MLA."""
    return 1.0 / math.sqrt(d_h + d_r)


def visible_rows(length: int, q_per_seq: int, r: int) -> int:
    """Rows query r (0-based, of q_per_seq new queries) may attend in a length-row sequence."""
    return int(length) - int(q_per_seq) + int(r) + 1


def _softmax_stats(s: np.ndarray):
    """Textbook softmax along axis 0 of s (masked entries are -inf).

    Returns p, the row maximum m and the log-sum-exp m + ln(sum exp(s - m)).
    """
    m = np.max(s, axis=0)
    e = np.exp(s - m)
    z = np.sum(e, axis=0)
    return e / z, m, m + np.log(z)


# ----------------------------------------------------------------------------
# The definition: materialized keys and values
# ----------------------------------------------------------------------------

def naive_decode(c_kv, k_r, offsets, q_c, q_r, w_uk, w_uv, q_per_seq: int,
                 scale: Optional[float] = None, seqs: Optional[Iterable[int]] = None,
                 return_weights: bool = False) -> Dict[str, np.ndarray]:
    """Multi-head attention over keys and values rebuilt from the latent cache (fp64).

    For each sequence b and head i: K^C = C_b W^UK_i^T and V^C = C_b W^UV_i^T over all
    rows of b ([notes] eq. 10, 11); keys are [K^C ; k^R] with k^R broadcast to every head; the
    query is [q^C ; q^R]; scores are scaled by ``scale`` (default 1/sqrt(d_h + d_h^R)),
    masked by the generalized causal rule, normalised by a textbook softmax, and o^C is
    the weighted sum of V^C.  Also returns the log-sum-exp of the scaled scores and
    o_lat = sum_j p_j c^KV_j (the latent-space output the absorbed form produces).

    ``seqs`` restricts the work to some sequences (other outputs stay NaN).
    """
    c_kv = np.asarray(c_kv, np.float64)
    k_r = np.asarray(k_r, np.float64)
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    n_q, n_h, d_h = q_c.shape
    d_r = q_r.shape[2]
    d_c = c_kv.shape[1]
    B = len(offsets) - 1
    if scale is None:
        scale = default_scale(d_h, d_r)
    o_c = np.full((n_q, n_h, d_h), np.nan)
    o_lat = np.full((n_q, n_h, d_c), np.nan)
    lse = np.full((n_q, n_h), np.nan)
    weights = {}
    for b in (range(B) if seqs is None else seqs):
        lo, hi = int(offsets[b]), int(offsets[b + 1])
        C = c_kv[lo:hi]
        R = k_r[lo:hi]
        L = hi - lo
        for i in range(n_h):
            K = np.concatenate([C @ w_uk[i].T, R], axis=1)     # [L, d_h + d_h^R]
            V = C @ w_uv[i].T                                  # [L, d_h]
            for r in range(q_per_seq):
                n = b * q_per_seq + r
                q = np.concatenate([q_c[n, i], q_r[n, i]])
                s = (K @ q) * scale
                s[visible_rows(L, q_per_seq, r):] = -np.inf
                p, _, l = _softmax_stats(s)
                o_c[n, i] = p @ V
                o_lat[n, i] = p @ C
                lse[n, i] = l
                if return_weights:
                    weights[(n, i)] = p
    out = dict(o_c=o_c, o_lat=o_lat, lse=lse)
    if return_weights:
        out["weights"] = weights
    return out


# ----------------------------------------------------------------------------
# The absorbed form, one function per C-ABI call
# ----------------------------------------------------------------------------

def absorb_q(q_c, q_r, w_uk) -> np.ndarray:
    """q_abs[n, i] = [ W^UK_i^T q^C_{n,i} ; q^R_{n,i} ].

    Key absorption ([notes] "Key에 대한 수식 전개"; [report] "Идея 1") and the concat
    identity ([notes] "Decoupled Rotary Position Embedding", item 4).

    The content score q^C . (W^UK c) equals (W^UK^T q^C) . c, so the query moves into
    latent space once and keys are never rebuilt; the RoPE part is carried unchanged
    because [a;b].[c;d] = a.c + b.d.
    """
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    lat = np.einsum("nid,idc->nic", q_c, w_uk)
    return np.concatenate([lat, q_r], axis=2)


def split_bounds(visible: int, s: int, num_splits: int, split_rows: int):
    """Row range [lo, hi) of split s among ``visible`` rows.

    Split s < num_splits-1 covers rows [s*split_rows, (s+1)*split_rows); the last split
    covers everything from (num_splits-1)*split_rows on; each range is clipped to the
    visible rows, so it may be empty.  With one split the range is all visible rows.
    """
    if num_splits == 1:
        return 0, visible
    lo = s * split_rows
    hi = visible if s == num_splits - 1 else (s + 1) * split_rows
    return min(lo, visible), min(hi, visible)


def split_partials(q_abs, c_kv, k_r, offsets, q_per_seq: int, num_splits: int,
                   split_rows: int, scale: float):
    """Softmax attention of every query head over each split's rows, in latent space.

    Row j's key is the whole latent row [c^KV_j ; k^R_j]; its value is c^KV_j.  For each
    split: o_s = sum_j p_j c_j with p the softmax over the split's rows only, and
    lse_s = log-sum-exp of the split's scaled scores.  Empty splits: o_s = 0, lse_s = -inf.
    Returns o_part [S, n_q, n_h, d_c] and lse_part [S, n_q, n_h].
    """
    q_abs = np.asarray(q_abs, np.float64)
    c_kv = np.asarray(c_kv, np.float64)
    k_r = np.asarray(k_r, np.float64)
    n_q, n_h, _ = q_abs.shape
    d_c = c_kv.shape[1]
    B = len(offsets) - 1
    o_part = np.zeros((num_splits, n_q, n_h, d_c))
    lse_part = np.full((num_splits, n_q, n_h), -np.inf)
    for b in range(B):
        lo_b, hi_b = int(offsets[b]), int(offsets[b + 1])
        X = np.concatenate([c_kv[lo_b:hi_b], k_r[lo_b:hi_b]], axis=1)   # [L, d_c + d_r]
        for r in range(q_per_seq):
            n = b * q_per_seq + r
            vis = visible_rows(hi_b - lo_b, q_per_seq, r)
            for s in range(num_splits):
                lo, hi = split_bounds(vis, s, num_splits, split_rows)
                if hi <= lo:
                    continue
                S = (X[lo:hi] @ q_abs[n].T) * scale        # [rows, n_h]
                p, _, l = _softmax_stats(S)
                o_part[s, n] = p.T @ X[lo:hi, :d_c]
                lse_part[s, n] = l
    return o_part, lse_part


def merge_splits(o_part, lse_part):
    """Combine split results: softmax over a disjoint union of row sets.

    With M = max_s lse_s and w_s = exp(lse_s - M): o = sum_s w_s o_s / sum_s w_s and
    lse = M + ln sum_s w_s.  Splits with lse_s = -inf get w_s = 0; a query head that
    no split saw (every lse_s = -inf) gets o = 0 and lse = -inf.
    """
    o_part = np.asarray(o_part, np.float64)
    lse_part = np.asarray(lse_part, np.float64)
    M = np.max(lse_part, axis=0)
    none = np.isneginf(M)                         # no split saw a row: o = 0, lse = -inf
    Ms = np.where(none, 0.0, M)
    w = np.exp(lse_part - Ms)                     # [S, n_q, n_h]; exp(-inf) = 0
    z = np.sum(w, axis=0)
    zs = np.where(none, 1.0, z)
    o = np.einsum("snh,snhc->nhc", w, o_part) / zs[..., None]
    return o, np.where(none, -np.inf, M + np.log(zs))


def attend_latent(q_abs, c_kv, k_r, offsets, q_per_seq: int, scale: float):
    """Unsplit latent attention: o_lat [n_q, n_h, d_c] and lse [n_q, n_h]."""
    o, l = split_partials(q_abs, c_kv, k_r, offsets, q_per_seq, 1, 0, scale)
    return o[0], l[0]


def out_proj(o_lat, w_uv) -> np.ndarray:
    """o^C[n, i] = W^UV_i o_lat[n, i].

    Value absorption ([notes] "Value에 대한 수식 전개"): the weighted sum of latents is
    projected once instead of projecting every row."""
    return np.einsum("idc,nic->nid", np.asarray(w_uv, np.float64), np.asarray(o_lat, np.float64))


def absorbed_decode(c_kv, k_r, offsets, q_c, q_r, w_uk, w_uv, q_per_seq: int,
                    scale: Optional[float] = None, num_splits: int = 1,
                    split_rows: int = 0) -> Dict[str, np.ndarray]:
    """The four calls end to end: absorb_q -> split_partials -> merge_splits -> out_proj."""
    d_h = np.asarray(q_c).shape[2]
    d_r = np.asarray(q_r).shape[2]
    if scale is None:
        scale = default_scale(d_h, d_r)
    qa = absorb_q(q_c, q_r, w_uk)
    op, lp = split_partials(qa, c_kv, k_r, offsets, q_per_seq, num_splits, split_rows, scale)
    o_lat, lse = merge_splits(op, lp)
    return dict(q_abs=qa, o_part=op, lse_part=lp, o_lat=o_lat, lse=lse, o_c=out_proj(o_lat, w_uv))


# ----------------------------------------------------------------------------
# Helpers for the pages' side claims
# ----------------------------------------------------------------------------

def rope_frequencies(d: int, theta: float = 10000.0, yarn: Optional[dict] = None) -> np.ndarray:
    """Per-position angle of each rotate-half pair k < d/2: theta^(-2k/d) ([notes] "MLA 코드
    구현"), or with yarn = dict(factor=s, original_len=L, alpha=a, beta=b) YaRN's NTK-by-parts
    ([report] training and infrastructure section: each frequency pair is scaled by the number
    of turns it makes over the training length; DeepSeek-V2: s = 40, a = 1, b = 32).  Reading
    taken where the page is brief: a pair making r = L f / (2 pi) turns over L keeps f when
    r >= b, is interpolated to f / s when r <= a, and between the two the frequency is the
    linear blend of f / s and f with weight (r - a) / (b - a) on f."""
    k = np.arange(d // 2, dtype=np.float64)
    f = np.power(float(theta), -2.0 * k / d)
    if yarn is None or yarn["factor"] <= 1.0:
        return f
    turns = yarn["original_len"] * f / (2.0 * math.pi)
    g = np.clip((turns - yarn["alpha"]) / (yarn["beta"] - yarn["alpha"]), 0.0, 1.0)
    return (1.0 - g) * f / yarn["factor"] + g * f


def yarn_softmax_scale(d_h: int, d_r: int, yarn: Optional[dict] = None) -> float:
    """1/sqrt(d_h + d_h^R) times YaRN's length factor t, sqrt(t) = mscale * ln s + 1 ([report]
    training and infrastructure section: DeepSeek-V2 takes mscale = 0.0707).  Reading: t
    multiplies every logit."""
    base = default_scale(d_h, d_r)
    if yarn is None or yarn["factor"] <= 1.0:
        return base
    return base * (yarn["mscale"] * math.log(yarn["factor"]) + 1.0) ** 2


def rope_pairs(x, positions, theta: float = 10000.0, yarn: Optional[dict] = None) -> np.ndarray:
    """RoPE as a complex rotation of the pairs (x_k, x_{k+d/2}) by angle pos * f_k
    (rope_frequencies).

    Same rotate-half convention as the helpers in [notes] "MLA 코드 구현", written as complex
    multiplication so that it shares no arithmetic with any other implementation.
    """
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    ang = np.asarray(positions, np.float64)[..., None] * rope_frequencies(d, theta, yarn)
    z = z * np.exp(1j * ang)
    return np.concatenate([z.real, z.imag], axis=-1)


# ----------------------------------------------------------------------------
# Decode prologue: the new tokens' latent rows and the rotated query part
# ----------------------------------------------------------------------------

def kv_prologue(h, w_dkv, w_kr, positions, theta: float = 10000.0, yarn: Optional[dict] = None):
    """Latent row of each new token: c^KV = W^DKV h ([notes] eq. 9) and the decoupled RoPE
    key k^R = RoPE(W^KR h) at the token's position ([notes] "Decoupled Rotary Position
    Embedding", items 2-3; "MLA 코드 구현": the down-projections and the rotation apply to the
    new tokens only, and the cache keeps k^R after rotation).

    h [n, d_model]; w_dkv [d_c, d_model]; w_kr [d_r, d_model]; positions [n].
    Returns (c_kv [n, d_c], k_r [n, d_r]) in fp64.
    """
    h = np.asarray(h, np.float64)
    c_kv = h @ np.asarray(w_dkv, np.float64).T
    k_r = rope_pairs(h @ np.asarray(w_kr, np.float64).T, np.asarray(positions), theta, yarn)
    return c_kv, k_r


def append_rows(rows, dst_rows, c_kv, k_r) -> np.ndarray:
    """The cache after the new tokens' rows [c^KV ; k^R] are written at dst_rows; every other
    row is unchanged ([notes] "MLA 코드 구현": the new latent rows are concatenated after the
    cached ones)."""
    out = np.array(rows, np.float64, copy=True)
    c_kv = np.asarray(c_kv, np.float64)
    k_r = np.asarray(k_r, np.float64)
    d_c, d_r = c_kv.shape[1], k_r.shape[1]
    for t, r in enumerate(np.asarray(dst_rows)):
        out[int(r), :d_c] = c_kv[t]
        out[int(r), d_c:d_c + d_r] = k_r[t]
    return out


def absorb_q_rope(q_c, q_r_raw, w_uk, positions, theta: float = 10000.0,
                  yarn: Optional[dict] = None) -> np.ndarray:
    """absorb_q with every head's RoPE part rotated at its token's position first ([notes]
    "MLA 코드 구현": q^R is rotated head by head at the new tokens' positions; "Decoupled
    Rotary Position Embedding", item 1).  positions [n_q]."""
    q_r = rope_pairs(np.asarray(q_r_raw, np.float64), np.asarray(positions)[:, None], theta, yarn)
    return absorb_q(q_c, q_r, w_uk)


def cache_elems_per_token(kind: str, layers: int, n_h: int = 0, d_h: int = 0, n_g: int = 0,
                          d_c: int = 0, d_r: int = 0) -> int:
    """KV-cache elements per token ([report] "Сколько получилось" table; [review] 2.4)."""
    if kind == "mha":
        return 2 * n_h * d_h * layers
    if kind == "gqa":
        return 2 * n_g * d_h * layers
    if kind == "mqa":
        return 2 * d_h * layers
    if kind == "mla":
        return (d_c + d_r) * layers
    raise ValueError(kind)


# ----------------------------------------------------------------------------
# Quantized latent cache: FP8 E4M3 codes with one fp32 scale per row
# ----------------------------------------------------------------------------
# The pages say the served DeepSeek-V2 quantizes its KV cache to about 6 bits per element
# ([review] section 4, "Inference efficiency"; [report] the 93.3% derivation and the
# economics section) and name no format.  The first concrete format taken here is the
# OCP FP8 E4M3 ("fn") encoding of every element of the row [c^KV ; k^R], with one scale
# per row that maps the row's largest magnitude to the format's largest value, 448.
#
# E4M3: bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m.
#   e > 0: (-1)^sign * 2^(e-7) * (1 + m/8);   e == 0: (-1)^sign * 2^-6 * m/8;
#   codes 0x7F and 0xFF are NaN; there is no infinity; the largest finite value is 448.
#
# Quantization decides integer codes, so it is written in the precision the kernel uses,
# float32: amax = max |x| over the row, s = fp32(amax / 448), code = E4M3 nearest to
# fp32(x / s), ties to even, magnitudes above 448 saturated to 448.  A row of zeros gets
# s = 0 and all codes 0.  Dequantization: x^ = value(code) * s.

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of every E4M3 code (uint8 array); NaN for 0x7F and 0xFF."""
    c = np.asarray(code).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of every value of y (exact binary values, e.g. float32), ties to
    even, magnitudes above 448 saturated; the sign bit follows y's sign bit (so -0.0 and
    negative values that round to zero give 0x80)."""
    y = np.asarray(y, np.float64)                 # exact: float32 widens without rounding
    neg = np.signbit(y)
    a = np.abs(y)
    # normal range: a = f * 2^k with 0.5 <= f < 1 (frexp is exact), so a = 2^(k-1) (1 + t)
    f, k = np.frexp(a)
    e = k - 1                                    # a in [2^e, 2^(e+1))
    step = np.exp2(e - 3.0)                      # spacing of E4M3 values in that binade
    q_norm = np.rint(a / step)                   # exact division by a power of two; rint: ties to even
    # q_norm in [8, 16]; 16 is the next binade's 8 (code arithmetic carries it over)
    code_norm = (e + 7) * 8 + (q_norm - 8)
    # subnormal range a < 2^-6: spacing 2^-9, codes 0..8 (8 is the smallest normal)
    code_sub = np.rint(a / 2.0 ** -9)
    mag = np.where(a < 2.0 ** -6, code_sub, code_norm)
    mag = np.minimum(mag, 0x7E)                  # saturate (also the carry past 448)
    return (mag.astype(np.int64) | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(rows):
    """Per-row E4M3 quantization of rows [R, W] (values exact in float32).  Returns
    (codes uint8 [R, W], scales float32 [R]); decisions in float32 as stated above."""
    x = np.asarray(rows, np.float32)
    amax = np.max(np.abs(x), axis=1)
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)      # float32 division
    safe = np.where(scales > 0, scales, np.float32(1.0)).astype(np.float32)
    y = (x / safe[:, None]).astype(np.float32)                     # float32 division
    codes = e4m3_encode(y)
    codes[scales == 0] = 0
    return codes, scales


def dequantize_rows(codes, scales) -> np.ndarray:
    """x^ = value(code) * scale, fp64 [R, W]."""
    return e4m3_value(codes) * np.asarray(scales, np.float64)[:, None]


# ----------------------------------------------------------------------------
# Offline weight folding: from c^Q to the block output u
# ----------------------------------------------------------------------------
# q^C = W^UQ c^Q ([notes] eq. 13).  The score's content term is
# (W^UQ c^Q)^T (W^UK c^KV) = (c^Q)^T ((W^UQ)^T W^UK) c^KV ([notes] "Decoupled Rotary Position
# Embedding", the expansion of the score; [report] "Идея 1"), so the token-independent product
# can be formed once: per head, G_i = (W^UK_i)^T W^UQ_i [d_c x d_cq] maps c^Q straight to the
# absorbed query.  On the output side u = W^O [o^C_1; ...; o^C_nh] with o^C_i = W^UV_i o_lat_i
# ([notes] "Value에 대한 수식 전개": W'^O = W^O W^UV), so W'^O_i = W^O_i W^UV_i [d_model x d_c]
# and u = sum_i W'^O_i o_lat_i.
# Layouts: c^Q [n, d_cq]; W^UQ [n_h, d_h, d_cq] (head i's rows of W^UQ); W^O [d_model, n_h d_h]
# (columns i d_h .. i d_h + d_h - 1 act on head i); G [n_h, d_c, d_cq]; W'^O [d_model, n_h d_c].

def q_up(c_q, w_uq) -> np.ndarray:
    """q^C[n, i] = W^UQ_i c^Q[n] ([notes] eq. 13) -> [n, n_h, d_h]."""
    return np.einsum("idk,nk->nid", np.asarray(w_uq, np.float64), np.asarray(c_q, np.float64))


def fold_q(w_uq, w_uk) -> np.ndarray:
    """G_i = (W^UK_i)^T W^UQ_i -> [n_h, d_c, d_cq]."""
    return np.einsum("idc,idk->ick", np.asarray(w_uk, np.float64), np.asarray(w_uq, np.float64))


def absorb_q_folded(c_q, g, q_r) -> np.ndarray:
    """q_abs[n, i] = [G_i c^Q[n] ; q_r[n, i]] -> [n, n_h, d_c + d_r]."""
    lat = np.einsum("ick,nk->nic", np.asarray(g, np.float64), np.asarray(c_q, np.float64))
    return np.concatenate([lat, np.asarray(q_r, np.float64)], axis=2)


def o_proj(o_c, w_o) -> np.ndarray:
    """u[n] = W^O [o^C[n, 0]; ...; o^C[n, n_h-1]] -> [n, d_model]."""
    o_c = np.asarray(o_c, np.float64)
    return o_c.reshape(o_c.shape[0], -1) @ np.asarray(w_o, np.float64).T


def fold_o(w_o, w_uv) -> np.ndarray:
    """W'^O_i = W^O_i W^UV_i, side by side -> [d_model, n_h d_c]."""
    w_o = np.asarray(w_o, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    n_h, d_h, d_c = w_uv.shape
    blocks = [w_o[:, i * d_h:(i + 1) * d_h] @ w_uv[i] for i in range(n_h)]
    return np.concatenate(blocks, axis=1)


def out_folded(o_lat, w_fold) -> np.ndarray:
    """u[n] = W'^O [o_lat[n, 0]; ...; o_lat[n, n_h-1]] -> [n, d_model]."""
    o_lat = np.asarray(o_lat, np.float64)
    return o_lat.reshape(o_lat.shape[0], -1) @ np.asarray(w_fold, np.float64).T

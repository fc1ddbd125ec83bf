"""CPU oracle for the latent down-projection that fills the cache, its append, and rollback.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the tests, the smoke check in __graft_entry__ and the cpu_baseline leg of bench.py
use it.  It shares no code with the HIP library.  Inputs are plain numpy arrays (bf16 values as
uint16 bit patterns, int32 lengths).

What the pages fix:
* "Module 05 -- MLA: Compressing Per-Token History", section 1: every token is projected DOWN
  to one shared latent c_t of width 512, and c_t is what the cache keeps (the formula after the
  colon is missing from the extracted text);
* "Module 08 -- Vision, MTP, and Hybrid Serving State", section 1: the language model's hidden
  width is 4096; section 3: the MLA latent cache is truncatable by position, and the state after
  a rollback must equal the state of a run that never generated the rejected tokens.

Readings taken where the pages are silent:
* c_t = W h_t, a plain linear map from the hidden state h_t (width 4096) to the latent (width
  512), W stored as [512][4096] (row r holds the weights of latent channel r); no bias and no
  normalisation of the latent, since the pages name none;
* the cache stores bf16, so the stored row is c_t rounded to the nearest bf16, ties to even;
* a pass over Q new tokens of sequence b whose cache length, after the pass, is cache_len[b]
  writes token i's latent at position cache_len[b] - Q + i, the position its query sits at in
  the attention call;
* rollback is a smaller cache_len: rows past it are never read, so nothing is erased.
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import bf16_bits_to_f64


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to the nearest bf16, ties to even; returns uint16 bit patterns.

    bf16 keeps 8 significant bits and float32's exponent range.  For |x| in [2^e, 2^(e+1)) the
    bf16 spacing is 2^(e-7) (2^-133 below the smallest normal 2^-126); x divided by the spacing
    is exact in float64, np.rint rounds it half to even, and the result is exactly a float32,
    whose top 16 bits are the bf16 pattern.  Values past the largest bf16 become +-inf."""
    x = np.asarray(x, np.float64)
    out = np.zeros(x.shape, np.float64)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])                      # x = m * 2^e, 0.5 <= |m| < 1, so |x| in [2^(e-1), 2^e)
    spacing = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    out[fin] = np.rint(x[fin] / spacing) * spacing
    out[~fin] = x[~fin]
    big = np.abs(out) > float.fromhex("0x1.fep127")
    out[big] = np.copysign(np.inf, out[big])
    f32 = out.astype(np.float32)                  # exact: at most 8 significant bits, float32 range
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def down_project(h_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """c = W h for every token (Module 05, section 1).  h_bits [..., hidden], w_bits
    [R, hidden] (bf16 bits) -> [..., R] float64: c[r] = sum_k W[r, k] h[k]."""
    return bf16_bits_to_f64(h_bits) @ bf16_bits_to_f64(w_bits).T


def latent_rows(h_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """The rows the cache stores: c = W h rounded to bf16 (bits)."""
    return f64_to_bf16_bits(down_project(h_bits, w_bits))


def append_reference(cache_bits: np.ndarray, cache_len: np.ndarray, h_bits: np.ndarray,
                     w_bits: np.ndarray) -> np.ndarray:
    """A copy of the cache after a pass of Q new tokens per sequence.

    cache_bits [B, L_max, R], cache_len [B] (the length AFTER the pass), h_bits [B, Q, hidden].
    Token i of sequence b goes to position cache_len[b] - Q + i; every other row is unchanged."""
    out = np.array(cache_bits, copy=True)
    B, Q = h_bits.shape[:2]
    rows = latent_rows(h_bits, w_bits)            # [B, Q, R]
    for b in range(B):
        for i in range(Q):
            t = int(cache_len[b]) - Q + i
            if t < 0 or t >= out.shape[1]:
                raise ValueError(f"position {t} of sequence {b} is outside the cache")
            out[b, t] = rows[b, i]
    return out


def rounding_interval(h_bits: np.ndarray, w_bits: np.ndarray, rel: float):
    """For a kernel that sums the products in a lower precision and then rounds to bf16: the bf16
    values (bits) that an accumulation error of at most rel * sum_k |W[r,k] h[k]| can produce.
    Rounding is monotone, so they are exactly the values between the roundings of the two ends.
    Returns (low_bits, high_bits) as float64 values of those bf16 patterns."""
    c = down_project(h_bits, w_bits)
    mag = np.abs(bf16_bits_to_f64(h_bits)) @ np.abs(bf16_bits_to_f64(w_bits)).T
    lo = bf16_bits_to_f64(f64_to_bf16_bits(c - rel * mag))
    hi = bf16_bits_to_f64(f64_to_bf16_bits(c + rel * mag))
    return lo, hi

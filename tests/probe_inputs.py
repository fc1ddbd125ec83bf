"""Selection probes: inputs whose output reveals, as exact integers, which cache positions a
query attended to.  Tolerance-based parity cannot see a causal off-by-one (one extra position
out of 32,768 moves the output far below any float tolerance), so these probes make the
selected set itself observable.

Count/bit-sum probe: with a zero query every score is 0 and every softmax weight is exactly
1/n, so o_lat[r] = (1/n) * sum_{j selected} c_j[r].  Latent channels hold exact 0/1 values:
  channel r < 17          : bit r of the position j
  channels 17 .. 33       : bit (r-17) of a hash of j
  channel 34              : 1 (so o_lat[34] * n == n)
  channels 35 .. R-1      : 0
Then round(o_lat[r] * n) = number of selected positions with that bit set, and
n = round(exp(lse)) because lse = ln(sum_j exp(0)) = ln(n).  Comparing these integers with
the ones computed from the expected set checks the set (up to collisions of all 35 bit sums,
which a shifted or widened causal bound cannot produce).
"""
from __future__ import annotations

import numpy as np

N_POS_BITS = 17
N_HASH_BITS = 17
ONE_CHANNEL = N_POS_BITS + N_HASH_BITS
BF16_ONE = 0x3F80


def position_hash(j: np.ndarray) -> np.ndarray:
    j = np.asarray(j, dtype=np.uint64)
    h = (j * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(15)
    return (h * np.uint64(0x9E3779B1)) & np.uint64(0x1FFFF)


def coded_cache(B: int, L_max: int, R: int, cache_len) -> np.ndarray:
    """[B, L_max, R] bf16 bits with the position code in every valid row; rows at or past
    cache_len[b] are NaN so any read of them poisons the output."""
    assert R >= ONE_CHANNEL + 1
    j = np.arange(L_max, dtype=np.int64)
    bits = np.zeros((L_max, R), np.uint16)
    for r in range(N_POS_BITS):
        bits[:, r] = np.where((j >> r) & 1, BF16_ONE, 0)
    hj = position_hash(j).astype(np.int64)
    for r in range(N_HASH_BITS):
        bits[:, N_POS_BITS + r] = np.where((hj >> r) & 1, BF16_ONE, 0)
    bits[:, ONE_CHANNEL] = BF16_ONE
    out = np.repeat(bits[None], B, axis=0)
    for b in range(B):
        out[b, int(cache_len[b]):] = 0x7FC0
    return out


# ------------------------------------------------------------------ read through the log-sum-exp
# The count probe above reads the counts out of o_lat, which needs the accumulated latents exact
# to the last unit; a library that keeps its split partials in fp16 rounds them.  This form reads
# the same 35 integers out of lse instead, which the attention computes from the fp32 running
# maxima and sums only.  Head 0 has a zero query: every score is 0, every weight exactly 1, so
# lse = ln(n).  Head 1 + c (c < 34) scores K * (c_j[c] - c_j[34]): 0 for a position whose code
# bit c is set and -K otherwise, so with K = 512 (exact in bf16; scale * K = 32) the clear
# positions weigh exp(-32) and lse = ln(number of positions with bit c set) up to 1e-9 relative.
# Heads 35..63 repeat head 0.  Every product and sum that reaches lse is then exact (scores 0 or
# -K, weights 1, sums of ones below 2^24); only the final logarithm rounds, by a few parts in 1e7,
# so the counts are recovered exactly while they stay below about 2^19.
PROBE_K = 512.0


def lse_probe_query(R: int = 512, heads: int = 64) -> np.ndarray:
    """[heads, R] bf16 bits of the absorbed query for the log-sum-exp form of the probe."""
    assert heads >= ONE_CHANNEL + 1 and R >= ONE_CHANNEL + 1
    q = np.zeros((heads, R), np.float32)
    for c in range(ONE_CHANNEL):
        q[1 + c, c] = PROBE_K
        q[1 + c, ONE_CHANNEL] = -PROBE_K
    b = (q.view(np.uint32) >> 16).astype(np.uint16)  # the values are exact in bf16
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), q)
    return b


def expected_lse_counts(positions: np.ndarray, heads: int = 64) -> np.ndarray:
    """The integers the log-sum-exp probe must recover per head for a selected set."""
    c = expected_counts(positions)  # 34 bit counts, then n
    n = c[-1]
    out = np.full(heads, n, np.int64)
    out[1:1 + ONE_CHANNEL] = c[:ONE_CHANNEL]
    return out


LN2_F32 = float(np.float32(0.69314718055994531))  # the fp32 constant a library multiplies by


def decoded_lse_counts(lse_row: np.ndarray) -> tuple[np.ndarray, float]:
    """Per head: round(exp(lse)), and the largest distance of exp(lse) from an integer.  lse is
    divided by the fp32 value of ln 2 so that a base-2 logarithm times that constant inverts
    exactly but for the logarithm's own rounding."""
    v = np.exp2(np.asarray(lse_row, np.float64) / LN2_F32)
    n = np.rint(v)
    return n.astype(np.int64), float(np.max(np.abs(v - n)))


def expected_counts(positions: np.ndarray) -> np.ndarray:
    """The 35 integers the probe must recover for a selected set."""
    p = np.asarray(positions, dtype=np.int64)
    hj = position_hash(p).astype(np.int64)
    cnt = [int(((p >> r) & 1).sum()) for r in range(N_POS_BITS)]
    cnt += [int(((hj >> r) & 1).sum()) for r in range(N_HASH_BITS)]
    cnt.append(int(p.size))
    return np.array(cnt, np.int64)


def decoded_counts(o_lat_row: np.ndarray, lse: float) -> tuple[np.ndarray, int]:
    """Integers recovered from one (query, head) output row of the probe."""
    n = int(np.rint(np.exp(float(lse))))
    vals = np.asarray(o_lat_row[: ONE_CHANNEL + 1], np.float64) * n
    return np.rint(vals).astype(np.int64), n


def decode_error(o_lat_row: np.ndarray, n: int) -> float:
    """Largest distance of o_lat*n from the nearest integer (should be << 0.5)."""
    vals = np.asarray(o_lat_row[: ONE_CHANNEL + 1], np.float64) * n
    return float(np.max(np.abs(vals - np.rint(vals))))

"""Seeded synthetic inputs for absorbed MLA attention over a latent KV cache.

This module is the ONLY code shared by the CPU oracle side (tests) and the
GPU side (tests, bench).  It draws random numbers and lays them out; it holds
none of the attention arithmetic.  Everything it returns is a plain numpy
array: bf16 values as uint16 bit patterns, lengths and positions as int32.

Workload shapes follow the checkpoint dimensions stated on the page
"Module 05 -- MLA: Compressing Per-Token History" (section 1, "The latent
representation"): latent width 512, 64 heads, 256-dim NoPE query/key and value
heads.  The verification pass of speculative decoding (page "Module 08 --
Vision, MTP, and Hybrid Serving State", section 2, target verification) runs
1 + k query positions in one pass; the GLM-5.3-Flash MTP explainer page gives
the serving recipe of five speculative tokens, hence 6 query positions.

Distributions: q and the cached latents c ~ N(0, 1); W_k and W_v ~ N(0, 1/512);
all rounded to bf16 with round-to-nearest-even from float32 draws.

Seeding: numpy SeedSequence([0x4D4C41, workload_id, set_index]) spawned into
independent streams, in this order: lengths, q, c, W_k, W_v, spikes, index
sets.  Large arrays are drawn in fixed 4 Mi-element chunks, each from its own
spawned child sequence, so the values do not depend on the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SEED_ROOT = 0x4D4C41
CHUNK = 1 << 22

HEADS = 64
HEAD_DIM = 256
LATENT = 512
SCALE = 1.0 / 16.0
W_STD = float(np.sqrt(1.0 / 512.0))

BF16_NAN = 0x7FC0


@dataclass(frozen=True)
class WorkloadSpec:
    """Shape and structure of one synthetic workload."""
    name: str
    batch: int
    q_len: int
    cache_len: int                   # uniform length, or the upper bound when ragged
    min_cache_len: Optional[int] = None  # ragged lengths: integer-uniform in [min, cache_len]
    spike_frac: float = 0.0          # fraction of positions per sequence whose latent is scaled
    spike_scale: float = 1.0
    n_index: int = 0                 # indexed variant: positions drawn per query (plus causal tail)
    workload_id: int = 0
    scale: float = SCALE             # softmax scale applied to q.k (1/16 for 256-dim heads)
    heads: int = HEADS
    head_dim: int = HEAD_DIM
    latent: int = LATENT

    @property
    def indexed(self) -> bool:
        return self.n_index > 0

    @property
    def k_max(self) -> int:
        """Slots per query in the index array: drawn positions plus the longest causal tail."""
        return self.n_index + self.q_len


# The five workloads: single-token decode (small and HBM-sized), the 6-position
# verification pass, long-context decode with 1% of latents scaled x8, and the
# ragged indexed verification pass.
WORKLOADS = {
    "decode_b1_l256": WorkloadSpec("decode_b1_l256", 1, 1, 256, workload_id=0),
    "decode_b32_l8192": WorkloadSpec("decode_b32_l8192", 32, 1, 8192, workload_id=1),
    "verify_b16_q6_l32768": WorkloadSpec("verify_b16_q6_l32768", 16, 6, 32768, workload_id=2),
    "decode_b4_l131072_spiked": WorkloadSpec("decode_b4_l131072_spiked", 4, 1, 131072,
                                             spike_frac=0.01, spike_scale=8.0, workload_id=3),
    "indexed_verify_b32_q4_ragged": WorkloadSpec("indexed_verify_b32_q4_ragged", 32, 4, 65536,
                                                 min_cache_len=4096, n_index=2048, workload_id=4),
}


@dataclass
class Workload:
    """One batch of inputs.  Shapes:
    q        [B, Q, H, D]  uint16 (bf16 bits)
    cache    [B, L_max, R] uint16 (bf16 bits); rows at or past cache_len[b] hold pad_bits
    w_k, w_v [H, D, R]     uint16 (bf16 bits); k_{j,h} = w_k[h] @ c_j, v_{j,h} = w_v[h] @ c_j
    cache_len [B] int32
    idx      [B, Q, K_max] int32 sorted positions (indexed variant), slots past idx_len hold pad_index
    idx_len  [B, Q] int32
    """
    spec: WorkloadSpec
    q: np.ndarray
    cache: np.ndarray
    w_k: np.ndarray
    w_v: np.ndarray
    cache_len: np.ndarray
    idx: Optional[np.ndarray] = None
    idx_len: Optional[np.ndarray] = None
    spikes: list = field(default_factory=list)

    @property
    def scale(self) -> float:
        return self.spec.scale


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.
    Inputs here are finite draws, so no NaN special case is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: np.random.SeedSequence, n: int, std: float = 1.0) -> np.ndarray:
    """n draws of N(0, std^2) rounded to bf16 bits, chunked and threaded but thread-count independent."""
    out = np.empty(n, np.uint16)
    nchunks = (n + CHUNK - 1) // CHUNK
    kids = seed.spawn(nchunks)

    def work(k):
        lo, hi = k * CHUNK, min(n, (k + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[k]))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(x)

    if nchunks <= 1:
        for k in range(nchunks):
            work(k)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def make_spec(batch, q_len, cache_len, *, heads=HEADS, head_dim=HEAD_DIM, latent=LATENT,
              min_cache_len=None, spike_frac=0.0, spike_scale=1.0, n_index=0, workload_id=100,
              scale=SCALE, name=None) -> WorkloadSpec:
    """A custom workload with the same distributions (used for small parity cases)."""
    return WorkloadSpec(name or f"custom_b{batch}_q{q_len}_l{cache_len}", batch, q_len, cache_len,
                        min_cache_len=min_cache_len, spike_frac=spike_frac, spike_scale=spike_scale,
                        n_index=n_index, workload_id=workload_id, scale=scale, heads=heads,
                        head_dim=head_dim, latent=latent)


def _draw_lengths(spec: WorkloadSpec, s_len: np.random.SeedSequence) -> np.ndarray:
    if spec.min_cache_len is not None:
        g = np.random.Generator(np.random.PCG64(s_len))
        return g.integers(spec.min_cache_len, spec.cache_len, size=spec.batch, endpoint=True).astype(np.int32)
    return np.full(spec.batch, spec.cache_len, np.int32)


def cache_lengths(spec, set_index: int = 0) -> np.ndarray:
    """The cache_len array make_workload(spec, set_index) draws, without drawing the rest."""
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    return _draw_lengths(spec, np.random.SeedSequence([SEED_ROOT, spec.workload_id, set_index]).spawn(7)[0])


def make_workload(spec, set_index: int = 0, *, pad_bits: int = BF16_NAN, pad_index: int = -1,
                  l_max: Optional[int] = None) -> Workload:
    """Draw one batch of inputs for `spec` (a WorkloadSpec or a key of WORKLOADS).

    pad_bits: bf16 pattern written into cache rows at or past cache_len[b] (NaN by default, so a
              kernel that reads them poisons its output).
    pad_index: value written into index slots past idx_len[b, i].
    l_max: allocated rows per sequence (>= the longest cache_len); default cache_len bound.
    """
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    B, Q, H, D, R = spec.batch, spec.q_len, spec.heads, spec.head_dim, spec.latent
    streams = np.random.SeedSequence([SEED_ROOT, spec.workload_id, set_index]).spawn(7)
    s_len, s_q, s_c, s_wk, s_wv, s_spk, s_idx = streams

    cache_len = _draw_lengths(spec, s_len)
    L_max = int(l_max if l_max is not None else spec.cache_len)
    if L_max < int(cache_len.max()):
        raise ValueError("l_max smaller than the longest cache")
    if int(cache_len.min()) < Q:
        raise ValueError("every cache must hold the q_len new positions")

    q = normal_bf16(s_q, B * Q * H * D).reshape(B, Q, H, D)
    w_k = normal_bf16(s_wk, H * D * R, W_STD).reshape(H, D, R)
    w_v = normal_bf16(s_wv, H * D * R, W_STD).reshape(H, D, R)

    cache = np.empty((B, L_max, R), np.uint16)
    c_kids = s_c.spawn(B)
    for b in range(B):
        n = int(cache_len[b])
        cache[b, :n] = normal_bf16(c_kids[b], n * R).reshape(n, R)
        cache[b, n:] = pad_bits

    spikes = []
    if spec.spike_frac > 0.0:
        g = np.random.Generator(np.random.PCG64(s_spk))
        for b in range(B):
            n = int(cache_len[b])
            cnt = int(round(spec.spike_frac * n))
            pos = np.sort(g.choice(n, size=cnt, replace=False)).astype(np.int64)
            # scaling by a power of two is exact in bf16 for these magnitudes
            vals = (cache[b, pos].astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(spec.spike_scale)
            cache[b, pos] = f32_to_bf16_bits(vals)
            spikes.append(pos)

    idx = idx_len = None
    if spec.indexed:
        g = np.random.Generator(np.random.PCG64(s_idx))
        K = spec.k_max
        idx = np.full((B, Q, K), pad_index, np.int32)
        idx_len = np.zeros((B, Q), np.int32)
        for b in range(B):
            first_new = int(cache_len[b]) - Q       # committed prefix is [0, first_new)
            if first_new < spec.n_index:
                raise ValueError("committed prefix shorter than the index count")
            for i in range(Q):
                drawn = np.sort(g.choice(first_new, size=spec.n_index, replace=False))
                tail = np.arange(first_new, first_new + i + 1)
                sel = np.concatenate([drawn, tail]).astype(np.int32)
                idx[b, i, :sel.size] = sel
                idx_len[b, i] = sel.size
    return Workload(spec, q, cache, w_k, w_v, cache_len, idx, idx_len, spikes)


def latent_query_bits(spec, set_index: int = 0) -> np.ndarray:
    """A stand-in absorbed query [B, Q, H, R] (bf16 bits) for testing the latent-attention stage
    on its own: N(0, 1/2), the variance of W_k^T q under the distributions above (256 * 1/512)."""
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    s = np.random.SeedSequence([SEED_ROOT, spec.workload_id, set_index, 0x51]).spawn(1)[0]
    n = spec.batch * spec.q_len * spec.heads * spec.latent
    return normal_bf16(s, n, float(np.sqrt(0.5))).reshape(spec.batch, spec.q_len, spec.heads, spec.latent)


# ---------------------------------------------------------------- k-pooled indexer inputs
INDEXER_DIM = 128   # indexer key / query width (a reading: the pages give none)
INDEXER_POOL = 4    # positions per pool (`index_kpool`; a reading: the pages give no value)
INDEXER_TOPK = 2048  # positions selected per query (a multiple of the pool)


@dataclass
class IndexerInputs:
    """Inputs of the k-pooled indexer for one batch.  Shapes:
    q [B, Q, d], k and g [B, L_max, d]  uint16 (bf16 bits): indexer queries, keys, gate logits;
    rows at or past cache_len[b] hold pad_bits.  cache_len [B] int32 (the same lengths as the
    attention workload's)."""
    q: np.ndarray
    k: np.ndarray
    g: np.ndarray
    cache_len: np.ndarray
    pool: int
    topk: int


def make_indexer_inputs(spec, cache_len: np.ndarray, set_index: int = 0, *, d: int = INDEXER_DIM,
                        pool: int = INDEXER_POOL, topk: int = INDEXER_TOPK, pad_bits: int = BF16_NAN,
                        l_max: Optional[int] = None) -> IndexerInputs:
    """N(0, 1) indexer queries, keys and gate logits (bf16) for the sequences of `spec`, seeded
    from SeedSequence([SEED_ROOT, workload_id, set_index, 0x1D]) spawned into q, k, g."""
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    B, Q = spec.batch, spec.q_len
    L_max = int(l_max if l_max is not None else spec.cache_len)
    s_q, s_k, s_g = np.random.SeedSequence([SEED_ROOT, spec.workload_id, set_index, 0x1D]).spawn(3)
    q = normal_bf16(s_q, B * Q * d).reshape(B, Q, d)
    k = np.empty((B, L_max, d), np.uint16)
    g = np.empty((B, L_max, d), np.uint16)
    k_kids, g_kids = s_k.spawn(B), s_g.spawn(B)
    for b in range(B):
        n = int(cache_len[b])
        k[b, :n] = normal_bf16(k_kids[b], n * d).reshape(n, d)
        g[b, :n] = normal_bf16(g_kids[b], n * d).reshape(n, d)
        k[b, n:] = pad_bits
        g[b, n:] = pad_bits
    return IndexerInputs(q, k, g, np.asarray(cache_len, np.int32), pool, topk)


# --------------------------------------------------------------------------
# down-projection inputs: hidden states of the new tokens and the latent projection
# --------------------------------------------------------------------------
HIDDEN = 4096                        # the language model's hidden width
W_DKV_STD = float(np.sqrt(1.0 / HIDDEN))  # keeps the projected latents near N(0, 1), like the caches


@dataclass
class AppendInputs:
    """Inputs of the latent down-projection for one pass: h [B, Q, hidden] (bf16 bits), the new
    tokens' hidden states; w_dkv [R, hidden] (bf16 bits), row r = the weights of latent channel r."""
    h: np.ndarray
    w_dkv: np.ndarray


def make_append_inputs(spec, set_index: int = 0, *, hidden: int = HIDDEN, rows: Optional[int] = None,
                       w_seed: int = 0) -> AppendInputs:
    """N(0, 1) hidden states for the spec's B x Q new tokens (or `rows` x 1) and an N(0, 1/hidden)
    projection, bf16, seeded from SeedSequence([SEED_ROOT, workload_id, set_index, 0xD0]) (h) and
    SeedSequence([SEED_ROOT, 0xD1, w_seed]) (the projection, shared by every workload)."""
    if isinstance(spec, str):
        spec = WORKLOADS[spec]
    B, Q = (spec.batch, spec.q_len) if rows is None else (rows, 1)
    s_h = np.random.SeedSequence([SEED_ROOT, spec.workload_id, set_index, 0xD0])
    s_w = np.random.SeedSequence([SEED_ROOT, 0xD1, w_seed])
    h = normal_bf16(s_h, B * Q * hidden).reshape(B, Q, hidden)
    w = normal_bf16(s_w, spec.latent * hidden, W_DKV_STD if hidden == HIDDEN else float(np.sqrt(1.0 / hidden)))
    return AppendInputs(h, w.reshape(spec.latent, hidden))

"""Helpers for the GPU tests: move workload arrays to the device and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def bf16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> bf16 tensor on the GPU (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bits on the host."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_parity(got, ref, what="", ref_max=None):
    """max|got - ref| <= 1e-2 * max|ref| + 1e-3, max|ref| taken over `ref` or, when a sample of a
    larger output is checked, given as `ref_max`: the largest |value| of the whole reference output
    (of whole_output_reference), which the bar is stated against."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = float(np.abs(got - ref).max())
    m = float(np.abs(ref).max())
    if ref_max is not None:
        assert ref_max >= m * (1 - 1e-9), f"{what}: the whole output's maximum is below the sample's"
        m = ref_max
    bar = 1e-2 * m + 1e-3
    print(f"{what}: max|err| = {err:.3e}, bar {bar:.3e}, max|ref| = {m:.3e}", flush=True)
    assert err <= bar, f"{what}: max|err| {err:.3e} > {bar:.3e}"
    return err


def whole_output_reference(w) -> np.ndarray:
    """Reference output of workload w at every (sequence, query, head) row, computed by the oracle in
    its absorbed form in fp64 (unrounded absorbed queries, attention over the cached latents, then
    the up-projection), which equals the expanded form up to fp64 rounding (the absorption identity
    the oracle is pinned to).  Cheap where the expanded form at full size is not.  [B, Q, H, D]."""
    import oracle
    q_abs = oracle.absorbed_query(w.q, w.w_k)
    o_lat, _ = oracle.latent_attention(q_abs, w.cache, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len)
    return oracle.up_project(o_lat, w.w_v)


def lse_bound(w, batches, queries, heads):
    """Largest lse error the whole path can show, from its arithmetic: the absorbed query is
    rounded to bf16 (relative error <= 2^-8 per element), which moves every score by at most
    scale * 2^-8 * sum_r |q~_r c_jr|; lse moves by at most the largest score change.  Plus 1e-3
    for fp32 exponentials, logarithms and sums.  Returns [nb, nq, nh]."""
    import oracle
    qt = np.abs(oracle.absorbed_query(w.q[np.ix_(batches)], w.w_k))  # [nb, Q, H, R]
    out = np.zeros((len(batches), len(queries), len(heads)))
    for ib, b in enumerate(batches):
        L = int(w.cache_len[b])
        for iq, i in enumerate(queries):
            if w.idx is None:
                pos = np.arange(L - w.q.shape[1] + i + 1)
            else:
                pos = w.idx[b, i, : w.idx_len[b, i]]
            c = np.abs(oracle.bf16_bits_to_f64(w.cache[b, pos]))
            m = c @ qt[ib, i][list(heads)].T                      # [T, nh]
            out[ib, iq] = w.scale * 2.0 ** -8 * m.max(axis=0) + 1e-3
    return out

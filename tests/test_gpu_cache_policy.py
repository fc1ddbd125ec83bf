"""The split kernels' two cache policies give the same bits (GPU).

A call whose cache rows have one reader each (one query unit and one head group per sequence)
runs the kernel instance whose tile copies are non-temporal; a call whose workgroups share rows
runs the instance with the default policy.  Only where the rows are kept differs, not what is
computed, so the two must agree bit for bit.  A call with 64 heads (one head group: the
non-temporal instance) is compared with the same call on 128 heads whose two head groups hold
the same queries (two groups share the rows: the default instance), at the same split count, for
the dense single-query kernel, the query-pair kernel, the indexed kernel and the two-term query.
The attention itself is checked against the oracle elsewhere (the latent attention of page
"Module 05 -- MLA: Compressing Per-Token History", section 3).
"""
import pytest
import torch

from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import DEV, bf16, i32

pytestmark = pytest.mark.gpu

CASES = [
    # (B, Q, L, n_index, splits, two_term)
    (3, 1, 1500, 0, 3, False),   # dense, single-query kernel, ragged lengths
    (2, 2, 900, 0, 2, False),    # dense, query-pair kernel
    (2, 1, 1200, 300, 2, False),  # indexed
    (2, 1, 1000, 0, 4, True),    # two-term absorbed query
    (1, 1, 700, 0, 1, False),    # one split: the split kernel writes the latents itself
]


@pytest.mark.parametrize("B,Q,L,n_index,splits,two_term", CASES)
def test_policies_give_the_same_bits(B, Q, L, n_index, splits, two_term):
    spec = wl.make_spec(B, Q, L, min_cache_len=L // 2, n_index=n_index, heads=64, workload_id=3100 + B + Q + splits)
    w = wl.make_workload(spec)
    print(f"B={B} Q={Q} L={L} indexed={n_index > 0} splits={splits} two_term={two_term}", flush=True)
    q64 = bf16(wl.latent_query_bits(spec))
    lo64 = None
    if two_term:
        g = torch.Generator(device=DEV)
        g.manual_seed(3100 + B)
        lo64 = (torch.randn(q64.shape, generator=g, device=DEV) * 2.0 ** -10).to(torch.bfloat16)
    q128 = torch.cat([q64, q64], dim=2).contiguous()
    lo128 = None if lo64 is None else torch.cat([lo64, lo64], dim=2).contiguous()
    c, cl = bf16(w.cache), i32(w.cache_len)

    def run(q, lo):
        if n_index:
            return binding.mla_latent_attn_indexed(q, c, cl, i32(w.idx), i32(w.idx_len), L, w.scale, splits,
                                                   q_abs_lo=lo)
        return binding.mla_latent_attn(q, c, cl, L, w.scale, splits, q_abs_lo=lo)

    o1, l1 = run(q64, lo64)
    o2, l2 = run(q128, lo128)
    torch.cuda.synchronize()
    assert torch.isfinite(o1).all()
    for half in (slice(0, 64), slice(64, 128)):
        assert torch.equal(o1.view(torch.int32), o2[:, :, half].contiguous().view(torch.int32)), "o_lat bits differ"
        assert torch.equal(l1.view(torch.int32), l2[:, :, half].contiguous().view(torch.int32)), "lse bits differ"

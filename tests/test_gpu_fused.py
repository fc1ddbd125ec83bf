"""GPU parity of the fused call mla_latent_attn_up_v (latent attention, then the split merge fused
into the value up-projection), called through the C ABI.

Checked against the fp64 oracle (page "Module 05 -- MLA: Compressing Per-Token History",
sections 3 and 4: out_h = U_h^V sum_j a_j c_j), and against the separate calls mla_latent_attn +
mla_up_v on the same inputs.  Those do the same arithmetic in the same order (the same merge, the
same hi / lo split of the merged latents, the same matrix products), so the two must agree bit
for bit.  The cases cover every row-group size the launcher picks (16, 8 and 4 rows, with a
ragged last group), one split (no merge: the plain up-projection), dense and indexed attention,
two head groups, and more than eight splits (the wide merge kernel, one and two rounds of
eight groups).
"""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import assert_parity, bf16, i32, whole_output_reference

pytestmark = pytest.mark.gpu


def both_paths(w, splits, two_term=False):
    q, c, wk, wv = bf16(w.q), bf16(w.cache), bf16(w.w_k), bf16(w.w_v)
    cl = i32(w.cache_len)
    Lmax = int(w.cache.shape[1])
    q_abs, q_lo = binding.mla_absorb_q(q, wk, lo=True) if two_term else (binding.mla_absorb_q(q, wk), None)
    idx = idx_len = None
    if w.idx is not None:
        idx, idx_len = i32(w.idx), i32(w.idx_len)
        o_lat, lse_s = binding.mla_latent_attn_indexed(q_abs, c, cl, idx, idx_len, Lmax, w.scale, splits,
                                                       q_abs_lo=q_lo)
    else:
        o_lat, lse_s = binding.mla_latent_attn(q_abs, c, cl, Lmax, w.scale, splits, q_abs_lo=q_lo)
    out_s = binding.mla_up_v(o_lat, wv)
    out_f, lse_f = binding.mla_latent_attn_up_v(q_abs, c, cl, Lmax, w.scale, wv, idx, idx_len, splits,
                                                q_abs_lo=q_lo)
    torch.cuda.synchronize()
    return out_f, lse_f, out_s, lse_s


def assert_same_bits(a, b, what):
    ea, eb = a.view(torch.int32), b.view(torch.int32)
    n = int((ea != eb).sum())
    assert n == 0, f"{what}: {n} of {a.numel()} values differ from the separate calls"


CASES = [
    # (B, Q, L, min_len, n_index, heads, splits)  rows = B*Q; the merge takes rows in passes of 16,
    # spread over just enough row groups to fill the CUs, or in single passes of 8 where one pass
    # of 16 would already leave CUs idle (64 heads: 16 rows or fewer)
    (10, 5, 300, 120, 0, 64, 4),    # 50 rows: two groups of two passes, the last pass holds 2
    (32, 1, 500, 200, 0, 64, 0),    # 32 rows: two groups of one pass, automatic split count
    (5, 1, 900, 300, 0, 64, 7),     # 5 rows: one pass of 8 holding 5
    (3, 6, 700, 200, 0, 64, 1),     # one split: no merge
    (2, 4, 600, 300, 100, 64, 3),   # indexed
    (2, 3, 400, 150, 0, 128, 2),    # two head groups
    (2, 2, 333, 100, 0, 192, 0),    # three head groups, a length bound that is not a whole tile
    (3, 2, 1500, 600, 0, 64, 12),   # more than eight splits: the wide merge, one round of groups
    (9, 2, 1500, 600, 0, 64, 10),   # 18 rows in passes of 16, more than eight splits
    (16, 4, 1500, 600, 0, 64, 9),   # 64 rows: two passes a group with the general merge
    (2, 1, 5000, 4000, 0, 64, 70),  # nine groups of splits: two rounds of the wide merge
    (64, 4, 300, 100, 0, 16, 3),    # 16 heads, 256 rows: eight groups of two passes
    (9, 2, 700, 300, 0, 64, 2),     # two splits (two merge slots loaded), passes of 16 with loads ahead
    (3, 1, 500, 200, 0, 64, 2),     # two splits, one pass of 8 rows: the general merge
    (16, 5, 400, 150, 0, 48, 5),    # 48 heads, 80 rows: three groups of two passes, the last group one
]


@pytest.mark.parametrize("B,Q,L,min_len,n_index,heads,splits", CASES)
def test_fused_matches_oracle_and_separate_calls(B, Q, L, min_len, n_index, heads, splits):
    spec = wl.make_spec(B, Q, L, min_cache_len=min_len, n_index=n_index, heads=heads,
                        workload_id=1100 + B * 7 + Q + heads)
    w = wl.make_workload(spec)
    print(f"fused B={B} Q={Q} L={L} H={heads} splits={splits}", flush=True)
    out_f, lse_f, out_s, lse_s = both_paths(w, splits)
    assert_same_bits(out_f, out_s, "out")
    assert_same_bits(lse_f, lse_s, "lse")
    hs = list(range(0, heads, 7))
    ref, lse_ref = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, idx=w.idx,
                                        idx_len=w.idx_len, heads=hs)
    assert_parity(out_f.cpu().numpy()[:, :, hs], ref, "fused out")
    np.testing.assert_allclose(lse_f.cpu().numpy()[:, :, hs], lse_ref, rtol=0, atol=1e-2)


# (workload, absorbed query in two bf16 terms).  With one term the spiked workload is checked against
# the oracle given the absorbed query rounded to bf16 (the oracle's own q~, rounded on the CPU),
# which is what the calls compute from a one-term query: the rounding of q~ alone moves that
# workload's worst row past the bar of the unrounded reference, and the two-term query brings it
# back within.
FULL_FUSED = [("decode_b32_l8192", False), ("decode_b32_l8192", True), ("verify_b16_q6_l32768", False),
              ("decode_b4_l131072_spiked", False), ("decode_b4_l131072_spiked", True),
              ("indexed_verify_b32_q4_ragged", False)]


@pytest.mark.parametrize("name,two_term", FULL_FUSED)
def test_fused_full_size(name, two_term):
    # the full sizes, in the launch configuration the benchmark times: bit-equal to the separate
    # calls everywhere, and every row against the oracle
    print(f"fused full size {name}{' (two-term query)' if two_term else ''}", flush=True)
    w = wl.make_workload(name)
    out_f, lse_f, out_s, lse_s = both_paths(w, 0, two_term)
    assert_same_bits(out_f, out_s, f"{name} out")
    assert_same_bits(lse_f, lse_s, f"{name} lse")
    out = out_f.cpu().numpy()
    if w.spikes and not two_term:
        qr = oracle.bf16_bits_to_f64(oracle.latent_append.f64_to_bf16_bits(oracle.absorbed_query(w.q, w.w_k)))
        o_lat, _ = oracle.latent_attention(qr, w.cache, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len)
        assert_parity(out, oracle.up_project(o_lat, w.w_v), f"{name} fused, every row (same rounded q~)")
        return
    # every row against the oracle's absorbed fp64 form; sampled rows also against its expanded form
    # (the bar relative to the largest value of the whole output)
    ref_all = whole_output_reference(w)
    assert_parity(out, ref_all, f"{name} fused, every row")
    bs, hs = [0, w.q.shape[0] - 1], [3, 62]
    ref, _ = oracle.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len,
                                  batches=bs, heads=hs)
    got = out[np.ix_(bs, range(w.q.shape[1]), hs)]
    assert_parity(got, ref, f"{name} fused sampled", ref_max=float(np.abs(ref_all).max()))


def test_fused_in_a_graph_and_workspace_checks():
    # the fused call only enqueues kernels: captured once, every replay gives the eager bits;
    # a workspace one byte short is refused before anything runs
    spec = wl.make_spec(4, 2, 1200, min_cache_len=500, workload_id=1190)
    w = wl.make_workload(spec)
    q_abs = binding.mla_absorb_q(bf16(w.q), bf16(w.w_k))
    c, cl, wv = bf16(w.cache), i32(w.cache_len), bf16(w.w_v)
    need = binding.mla_latent_attn_up_v_workspace_size(4, 2, 64, 512, 1200, 0)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=c.device)
    out = torch.empty((4, 2, 64, 256), dtype=torch.float32, device=c.device)
    lse = torch.empty((4, 2, 64), dtype=torch.float32, device=c.device)

    def step():
        binding.mla_latent_attn_up_v(q_abs, c, cl, 1200, w.scale, wv, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l)
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o)
    short = torch.empty(need - 1, dtype=torch.uint8, device=c.device)
    out.fill_(7.0)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_latent_attn_up_v(q_abs, c, cl, 1200, w.scale, wv, out=out, lse=lse, workspace=short)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

"""The C ABI's calls captured in a HIP graph and replayed (GPU): a serving loop captures its
decode step once and replays it.  Every call only enqueues kernels on the given stream, with no
allocation, memset or synchronisation inside, so each replay must give the eager results bit for
bit (the kernels are deterministic for fixed inputs).  Replays are interleaved with eager work
and host synchronisation, and every replay is checked."""
import numpy as np
import pytest
import torch

from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import bf16, i32

pytestmark = pytest.mark.gpu


def replay_and_check(fn, outputs, reps=3):
    """Run fn eagerly, capture it, replay `reps` times; each replay must reproduce the eager
    outputs exactly.  `outputs` are the tensors fn writes."""
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for r in range(reps):
        for o in outputs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w), f"replay {r} differs from the eager call"
        # eager work between replays
        fn()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w)


def test_decode_step_in_a_graph():
    spec = wl.make_spec(4, 1, 3000, min_cache_len=1000, workload_id=900)
    w = wl.make_workload(spec)
    q, wk, wv, cache, cl = bf16(w.q), bf16(w.w_k), bf16(w.w_v), bf16(w.cache), i32(w.cache_len)
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    q_abs = torch.empty((B, Q, H, R), dtype=torch.bfloat16, device=q.device)
    o_lat = torch.empty((B, Q, H, R), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(binding.mla_latent_attn_workspace_size(B, Q, H, R, 3000), 1), dtype=torch.uint8,
                     device=q.device)

    def step():
        binding.mla_absorb_q(q, wk, q_abs=q_abs)
        binding.mla_latent_attn(q_abs, cache, cl, 3000, spec.scale, 0, o_lat=o_lat, lse=lse, workspace=ws)
        binding.mla_up_v(o_lat, wv, out=out)

    replay_and_check(step, [q_abs, o_lat, lse, out])


def test_two_term_fused_decode_step_in_a_graph():
    # the absorbed query in two bf16 terms, then the fused attention and up-projection
    spec = wl.make_spec(4, 1, 3000, min_cache_len=1000, spike_frac=0.01, spike_scale=8.0, workload_id=902)
    w = wl.make_workload(spec)
    q, wk, wv, cache, cl = bf16(w.q), bf16(w.w_k), bf16(w.w_v), bf16(w.cache), i32(w.cache_len)
    B, Q, H, D = w.q.shape
    R = w.cache.shape[2]
    q_abs = torch.empty((B, Q, H, R), dtype=torch.bfloat16, device=q.device)
    q_lo = torch.empty_like(q_abs)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(binding.mla_latent_attn_up_v_workspace_size(B, Q, H, R, 3000), 1), dtype=torch.uint8,
                     device=q.device)

    def step():
        binding.mla_absorb_q(q, wk, q_abs=q_abs, q_abs_lo=q_lo)
        binding.mla_latent_attn_up_v(q_abs, cache, cl, 3000, spec.scale, wv, out=out, lse=lse, workspace=ws,
                                     q_abs_lo=q_lo)

    replay_and_check(step, [q_abs, q_lo, lse, out])


def test_verify_step_with_indexer_and_append_in_a_graph():
    spec = wl.make_spec(2, 4, 2500, min_cache_len=1500, workload_id=901)
    w = wl.make_workload(spec)
    ix = wl.make_indexer_inputs(spec, w.cache_len, d=128, pool=4, topk=256)
    inp = wl.make_append_inputs(spec)
    B, Q = 2, 4
    cache, cl = bf16(w.cache), i32(w.cache_len)
    h, wd = bf16(inp.h), bf16(inp.w_dkv)
    kq, kk, kg = bf16(ix.q), bf16(ix.k), bf16(ix.g)
    max_pools = 2500 // 4
    pooled = torch.empty((B, max_pools, 128), dtype=torch.float32, device=cache.device)
    scores = torch.empty((B, Q, max_pools), dtype=torch.float32, device=cache.device)
    idx = torch.empty((B, Q, 256 + 3), dtype=torch.int32, device=cache.device)
    idx_len = torch.empty((B, Q), dtype=torch.int32, device=cache.device)
    qa = bf16(wl.latent_query_bits(spec))
    o_lat = torch.empty((B, Q, 64, 512), dtype=torch.float32, device=cache.device)
    lse = torch.empty((B, Q, 64), dtype=torch.float32, device=cache.device)
    ws = torch.empty(max(binding.mla_latent_attn_workspace_size(B, Q, 64, 512, 256 + 3, indexed=True), 1),
                     dtype=torch.uint8, device=cache.device)

    def step():
        binding.mla_latent_append(h, wd, cache, cl, 2500)
        binding.mla_kpool_keys(kk, kg, cl, 2500, 4, pooled=pooled)
        binding.mla_indexer_scores(kq, pooled, cl, 2500, 4, scores=scores)
        binding.mla_indexer_select(scores, cl, 2500, 4, 256, True, idx=idx, idx_len=idx_len)
        binding.mla_latent_attn_indexed(qa, cache, cl, idx, idx_len, 2500, spec.scale, 0, o_lat=o_lat, lse=lse,
                                        workspace=ws)

    replay_and_check(step, [idx, idx_len, o_lat, lse])
    # the appended rows are the same after every replay
    rows = cache[torch.arange(B, device=cache.device)[:, None],
                 (cl[:, None] - Q + torch.arange(Q, device=cache.device)[None, :]).long()]
    assert torch.isfinite(rows.float()).all()

"""The no-allocation entry point (mla_latent_attn_up_v_noalloc): the fused attention and
up-projection with its split partials in the library's fixed device scratch.  It must give the bits
of mla_latent_attn_up_v (same kernels, same split count), call after call: the scratch keeps the
previous call's partials, so two calls in a row, the second smaller, are compared; and it must
refuse a call whose partials would not fit, before writing anything."""
import numpy as np
import pytest
import torch

import oracle
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import DEV, assert_parity, bf16, i32

pytestmark = pytest.mark.gpu

F = oracle.bf16_bits_to_f64


def inputs(B, Q, L, wid, **kw):
    spec = wl.make_spec(B, Q, L, workload_id=wid, **kw)
    w = wl.make_workload(spec)
    return w, wl.latent_query_bits(spec)


def both_calls(w, qa, splits=0):
    q, c, cl, wv = bf16(qa), bf16(w.cache), i32(w.cache_len), bf16(w.w_v)
    idx = None if w.idx is None else i32(w.idx)
    idx_len = None if w.idx is None else i32(w.idx_len)
    L = int(w.cache.shape[1])
    ref, lse_ref = binding.mla_latent_attn_up_v(q, c, cl, L, w.scale, wv, idx, idx_len, splits)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    binding.mla_latent_attn_up_v_noalloc(q, c, cl, L, w.scale, wv, out, lse, idx, idx_len, splits)
    torch.cuda.synchronize()
    return out, lse, ref, lse_ref


def check(w, qa, what, splits=0):
    B, Q = w.q.shape[:2]
    Kp = int(w.cache.shape[1]) if w.idx is None else int(w.idx.shape[2])
    s = binding.mla_latent_attn_num_splits(B, Q, 64, Kp, splits, indexed=w.idx is not None)
    print(f"{what}: B{B} Q{Q} L{w.cache.shape[1]}, {s} splits", flush=True)
    out, lse, ref, lse_ref = both_calls(w, qa, splits)
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), what
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), what
    # and against the oracle (latent attention, then the one expansion by U^V)
    o_lat, _ = oracle.latent_attention(F(qa), w.cache, w.cache_len, w.scale, idx=w.idx, idx_len=w.idx_len)
    assert_parity(out.cpu().numpy(), oracle.up_project(o_lat, w.w_v), f"{what} against the oracle")
    return s


def test_noalloc_equals_fused_call_two_calls_in_a_row():
    # first a larger call (several splits, ragged), then a smaller one: the second must not see
    # anything the first left in the scratch
    w1, q1 = inputs(6, 1, 3000, 900, min_cache_len=1000)
    s1 = check(w1, q1, "first call (decode, ragged)")
    w2, q2 = inputs(2, 3, 400, 901)
    s2 = check(w2, q2, "second call (smaller, three queries)")
    assert s1 > 1 and s2 >= 1
    # the smaller call again with a forced split count, then a one-split call (the accumulated
    # latents in the scratch instead of partials)
    check(w2, q2, "second call, 5 splits", splits=5)
    check(w2, q2, "second call, 1 split", splits=1)


def test_noalloc_indexed_equals_fused_call():
    w, qa = inputs(3, 4, 2500, 902, min_cache_len=1500, n_index=300)
    check(w, qa, "indexed")
    w2, q2 = inputs(2, 2, 900, 903, min_cache_len=600, n_index=100)
    check(w2, q2, "indexed, smaller")


def test_noalloc_refuses_more_than_its_scratch():
    # 32 x 8 queries x 16 splits: 16 * 256 * 64 rows of 2,056 bytes = 539 MB of partials
    B, Q, L = 32, 8, 512
    need = binding.mla_latent_attn_up_v_workspace_size(B, Q, 64, 512, L, 16)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Q, 64, 512), dtype=torch.bfloat16, device=DEV)
    c = torch.zeros((B, L, 512), dtype=torch.bfloat16, device=DEV)
    cl = torch.full((B,), L, dtype=torch.int32, device=DEV)
    wv = torch.zeros((64, 256, 512), dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, Q, 64, 256), 7.0, device=DEV)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_latent_attn_up_v_noalloc(q, c, cl, L, 1.0 / 16, wv, out, None, num_splits=16)
    assert e.value.status == binding.MLA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # the largest split count that fits still runs and matches the fused call
    w, qa = inputs(2, 1, 8192, 904)
    check(w, qa, "after a refused call")

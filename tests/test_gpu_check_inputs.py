"""GPU tests of the debug check of the attention calls' device-side preconditions
(mla_check_attn_inputs) and of the MLA_CHECK_INPUTS environment flag that runs it before every
attention call.  Page "Module 05 -- MLA: Compressing Per-Token History", section 4 (query t
sees j <= t); page "Module 08 -- Vision, MTP, and Hybrid Serving State", section 2 (the Q new
positions are the cache's last Q); colibri "DSA with k-pooling" (sorted selections of the
prefix)."""
import numpy as np
import pytest
import torch

from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import bf16, i32

pytestmark = pytest.mark.gpu


def check(lens, Q, Lmax, idx=None, idx_len=None):
    return binding.mla_check_attn_inputs(i32(np.array(lens)), Q, Lmax,
                                         None if idx is None else i32(np.array(idx)),
                                         None if idx_len is None else i32(np.array(idx_len)))


def test_valid_workloads_pass():
    w = wl.make_workload(wl.make_spec(5, 4, 900, min_cache_len=4, workload_id=1300))
    assert check(w.cache_len, 4, 900) == 0
    wi = wl.make_workload(wl.make_spec(3, 4, 700, min_cache_len=200, n_index=60, workload_id=1301))
    # slots past idx_len hold -1 and are not examined
    assert check(wi.cache_len, 4, 700, wi.idx, wi.idx_len) == 0
    assert check(wi.cache_len, 4, 700) == 0


def test_cache_length_bounds():
    assert check([5, 2], 3, 10) == 1           # 2 < Q
    assert check([5, 11], 3, 10) == 2          # past max_cache_len
    assert check([2, 11], 3, 10) == 3
    assert check([3, 10], 3, 10) == 0          # both bounds inclusive


def test_index_rows():
    # one sequence of 10 positions, Q = 2: query 0 at position 8, query 1 at position 9
    lens, Q, K = [10], 2, 4
    good = [[[0, 3, 5, 8], [1, 2, 9, -1]]]
    assert check(lens, Q, 10, good, [[4, 3]]) == 0
    assert check(lens, Q, 10, good, [[0, 3]]) == 4                     # empty row
    assert check(lens, Q, 10, good, [[5, 3]]) == 4                     # longer than K_max
    assert check(lens, Q, 10, [[[0, 3, 5, 9], [1, 2, 9, -1]]], [[4, 3]]) == 32   # query 0 sees 9
    assert check(lens, Q, 10, [[[0, 5, 3, 8], [1, 2, 9, -1]]], [[4, 3]]) == 16   # not ascending
    assert check(lens, Q, 10, [[[0, 3, 3, 8], [1, 2, 9, -1]]], [[4, 3]]) == 16   # repeated
    assert check(lens, Q, 10, [[[-1, 3, 5, 8], [1, 2, 9, -1]]], [[4, 3]]) == 8                 # negative
    assert check(lens, Q, 10, [[[0, 3, 5, 8], [1, 2, 10, -1]]], [[4, 3]]) == 8 | 32  # past the cache
    # max_cache_len below cache_len: positions past it are out of range too
    assert check(lens, Q, 9, good, [[4, 3]]) == 2 | 8


def test_environment_flag_checks_before_every_attention_call(monkeypatch):
    spec = wl.make_spec(2, 2, 300, min_cache_len=100, workload_id=1302)
    w = wl.make_workload(spec)
    q_abs = bf16(wl.latent_query_bits(spec))
    cache, wv = bf16(w.cache), bf16(w.w_v)
    good = i32(w.cache_len)
    bad = i32(np.array([1, 200]))  # 1 < Q
    want, _ = binding.mla_latent_attn(q_abs, cache, good, 300, spec.scale)
    monkeypatch.setenv("MLA_CHECK_INPUTS", "1")
    got, _ = binding.mla_latent_attn(q_abs, cache, good, 300, spec.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    o = torch.full_like(want, 7.0)
    out = torch.full((2, 2, 64, 256), 7.0, dtype=torch.float32, device=cache.device)
    for call in (lambda: binding.mla_latent_attn(q_abs, cache, bad, 300, spec.scale, o_lat=o),
                 lambda: binding.mla_latent_attn_up_v(q_abs, cache, bad, 300, spec.scale, wv, out=out),
                 lambda: binding.mla_latent_attn_indexed(q_abs, cache, bad, i32(np.zeros((2, 2, 1))),
                                                         i32(np.ones((2, 2))), 300, spec.scale, o_lat=o)):
        with pytest.raises(binding.MlaError) as e:
            call()
        assert e.value.status == binding.MLA_ERR_ARG and "cache_len < Q" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((out == 7.0).all())

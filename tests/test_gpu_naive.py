"""GPU parity of the naive (expanded) form, called through the C ABI, against the fp64 oracle.

The expansion's bf16 keys and values are held to the rounding of the exact value moved by the
largest fp32 summation error (a bound from the arithmetic); the attention is checked on the
kernel's own expanded keys and values, end to end against the reference, and against the absorbed
form on the same inputs (page "Module 05 -- MLA: Compressing Per-Token History", section 5 and its
equivalence laboratory: both forms must give the same attention).
"""
import numpy as np
import pytest
import torch

from oracle import latent_append as la
from oracle import mla_oracle as mo
from oracle import naive_form as nf
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import DEV, assert_parity, bf16, bits, i32

pytestmark = pytest.mark.gpu

F = mo.bf16_bits_to_f64
# each expanded value sums 512 products in fp32 with at most 512 additions one after another
# (32 matrix instructions of 16 products each): |fl(x) - x| <= 512 * 2^-24 * sum |U c|
REL = 512 * 2.0 ** -24
SENTINEL = 0x7FC1


def interval(c_bits_b, w_bits, n):
    """bf16 values an expansion of positions 0..n-1 may take: [n, H, D] low / high."""
    c = F(c_bits_b[:n])
    H, D, R = w_bits.shape
    w = F(w_bits).reshape(H * D, R)
    x = (c @ w.T).reshape(n, H, D)
    mag = (np.abs(c) @ np.abs(w).T).reshape(n, H, D)
    lo = F(la.f64_to_bf16_bits(x - REL * mag))
    hi = F(la.f64_to_bf16_bits(x + REL * mag))
    return lo, hi, la.f64_to_bf16_bits(x)


def expand(w, lens, Lmax):
    k = torch.full((w.cache.shape[0], Lmax, 64, 256), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vt = torch.full((w.cache.shape[0], 64, 256, binding.vt_length(Lmax)), SENTINEL, dtype=torch.int16,
                    device=DEV).view(torch.bfloat16)
    binding.mla_expand_kv(bf16(w.cache), i32(lens), bf16(w.w_k), bf16(w.w_v), Lmax, k_out=k, vt_out=vt)
    torch.cuda.synchronize()
    return k, vt


@pytest.mark.parametrize("lens,Lmax", [([200, 77], 256), ([64, 1], 130), ([384], 384), ([700, 513], 720)])
def test_expansion_rounded_and_padded(lens, Lmax):
    spec = wl.make_spec(len(lens), 1, Lmax, workload_id=720 + Lmax)
    w = wl.make_workload(spec)
    lens = np.array(lens, np.int32)
    print(f"expand lens={lens.tolist()} Lmax={Lmax}", flush=True)
    k, vt = expand(w, lens, Lmax)
    kb, vtb = bits(k), bits(vt)
    for b, L in enumerate(lens):
        L = int(L)
        for name, got, wts in (("k", kb[b, :L], w.w_k), ("v", vtb[b].transpose(2, 0, 1)[:L], w.w_v)):
            lo, hi, exact = interval(w.cache[b], wts, L)
            v = F(got)
            assert np.all((lo <= v) & (v <= hi)), name
            frac = float(np.mean(got == exact))
            print(f"  {name}[{b}]: {frac:.5f} equal to the rounded exact value", flush=True)
            assert frac > 0.99
        # untouched rows of k; zeros up to the next multiple of 64 in V^T, untouched after
        assert np.all(kb[b, L:] == SENTINEL)
        pad = min((L + 63) // 64 * 64, vtb.shape[3])
        assert np.all(vtb[b, :, :, L:pad] == 0)
        assert np.all(vtb[b, :, :, pad:] == SENTINEL)


@pytest.mark.parametrize("B,Q,lens,Lmax", [(2, 1, [300, 129], 320), (1, 6, [1000], 1000), (2, 200, [333, 260], 333),
                                           (1, 130, [130], 192)])
def test_attention_on_the_kernels_expansion(B, Q, lens, Lmax):
    # the attention kernel alone: the oracle attends over the very keys and values the expansion
    # kernel wrote (widened exactly from bf16)
    spec = wl.make_spec(B, Q, Lmax, workload_id=740 + Q)
    w = wl.make_workload(spec)
    lens = np.array(lens, np.int32)
    print(f"naive attention B={B} Q={Q} lens={lens.tolist()}", flush=True)
    k, vt = expand(w, lens, Lmax)
    out, lse = binding.mla_naive_attn(bf16(w.q), k, vt, i32(lens), Lmax, spec.scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    kb, vtb = bits(k), bits(vt)
    heads = [0, 17, 63]
    qs = sorted(set([0, Q // 2, Q - 1]))
    for b in range(B):
        L = int(lens[b])
        kk = F(kb[b, :L])
        vv = F(vtb[b, :, :, :L]).transpose(2, 0, 1)
        ref, ref_lse = nf.attention_on_expanded(w.q[b], kk, vv, L, spec.scale, queries=qs, heads=heads)
        assert_parity(out[b][np.ix_(qs, heads)], ref, f"naive attention b={b}")
        np.testing.assert_allclose(lse[b][np.ix_(qs, heads)], ref_lse, rtol=0, atol=1e-3)


def test_naive_equals_absorbed_and_reference():
    # the equivalence half of the laboratory: both GPU forms on identical inputs, and the oracle
    spec = wl.make_spec(2, 6, 700, min_cache_len=300, workload_id=760)
    w = wl.make_workload(spec)
    cl = i32(w.cache_len)
    args = (bf16(w.q), bf16(w.w_k), bf16(w.w_v), bf16(w.cache), cl, 700, spec.scale)
    out_n, lse_n = binding.mla_naive_forward(*args)
    out_a, lse_a = binding.mla_forward(*args)
    torch.cuda.synchronize()
    out_n, out_a = out_n.cpu().numpy(), out_a.cpu().numpy()
    ref, ref_lse = mo.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, spec.scale, heads=range(0, 64, 9))
    assert_parity(out_n[:, :, ::9], ref, "naive vs reference")
    assert_parity(out_a[:, :, ::9], ref, "absorbed vs reference")
    assert_parity(out_n, out_a, "naive vs absorbed")
    np.testing.assert_allclose(lse_n.cpu().numpy(), lse_a.cpu().numpy(), rtol=0, atol=2e-3)


def test_prefill_shape_sampled():
    # a 4096-token causal prefill of one sequence (every query sees its own prefix): sampled
    # queries and heads against the reference
    spec = wl.make_spec(1, 4096, 4096, workload_id=780)
    w = wl.make_workload(spec)
    print("naive prefill 4096", flush=True)
    out, lse = binding.mla_naive_forward(bf16(w.q), bf16(w.w_k), bf16(w.w_v), bf16(w.cache), i32(w.cache_len),
                                         4096, spec.scale)
    torch.cuda.synchronize()
    qs, hs = [0, 1, 1000, 2047, 4095], [0, 41]
    ref, ref_lse = mo.mla_reference(w.q, w.cache, w.w_k, w.w_v, w.cache_len, spec.scale, queries=qs, heads=hs)
    assert_parity(out.cpu().numpy()[0][np.ix_(qs, hs)], ref[0], "naive prefill 4096")
    np.testing.assert_allclose(lse.cpu().numpy()[0][np.ix_(qs, hs)], ref_lse[0], rtol=0, atol=2e-3)

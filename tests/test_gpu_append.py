"""GPU parity of the latent down-projection with cache append (called through the C ABI)
against the fp64 CPU oracle, and the rollback invariant on the GPU.

The stored rows are bf16 roundings of fp32 sums.  On inputs whose sums are exact in fp32 they
are checked bit for bit; otherwise each row must lie between the roundings of the exact value
moved by the largest error fp32 summation can make (a bound from the arithmetic, below), and
rows the pass must not write are checked bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import latent_append as la
from oracle import mla_oracle as mo
from mla_latent_cache_absorb_amd import binding, workloads as wl
from tests.gpu_util import DEV, bf16, bits, i32

pytestmark = pytest.mark.gpu

HIDDEN, R = wl.HIDDEN, wl.LATENT
# each output is summed in fp32 with at most 8 * 32 products accumulated one after another
# inside the matrix instructions and then 16 partial sums added in order: 272 additions, so
# |fl(c) - c| <= 272 * 2^-24 * sum_k |W[r,k] h[k]| (first order; any order of the additions)
REL = 272 * 2.0 ** -24


def small_int_bits(rng, shape, lo=-3, hi=3):
    return wl.f32_to_bf16_bits(rng.integers(lo, hi + 1, shape).astype(np.float32))


def run_append(cache_bits, lens, h_bits, w_bits, max_cache_len=None):
    cache = bf16(cache_bits)
    binding.mla_latent_append(bf16(h_bits), bf16(w_bits), cache, i32(lens),
                              int(max_cache_len or cache_bits.shape[1]))
    torch.cuda.synchronize()
    return bits(cache)


def check_rows(got, cache_before, lens, h_bits, w_bits):
    """Appended rows within the rounding bound, every other row unchanged (bitwise)."""
    B, Q = h_bits.shape[:2]
    lo, hi = la.rounding_interval(h_bits, w_bits, REL)      # [B, Q, R]
    exact = la.latent_rows(h_bits, w_bits)
    expect_other = np.array(cache_before, copy=True)
    n_exact = n_all = 0
    for b in range(B):
        for i in range(Q):
            t = int(lens[b]) - Q + i
            if t < 0:
                continue
            row = mo.bf16_bits_to_f64(got[b, t])
            assert np.all((lo[b, i] <= row) & (row <= hi[b, i])), (b, i, t)
            n_exact += int(np.sum(got[b, t] == exact[b, i]))
            n_all += R
            expect_other[b, t] = got[b, t]
    np.testing.assert_array_equal(got, expect_other)
    print(f"rows within bound; {n_exact}/{n_all} equal to the rounded exact value", flush=True)
    return n_exact / max(n_all, 1)


@pytest.mark.parametrize("B,Q,L", [(1, 1, 4), (3, 5, 40), (2, 17, 64), (33, 16, 20), (4, 520, 600)])
def test_exact_inputs_bit_exact(B, Q, L):
    # small integers: every partial sum is an integer below 2^24, exact in fp32 in any order, so
    # the stored rows equal the oracle's bit for bit (ragged lengths, a ragged last tile of 16
    # tokens, more tiles than row groups for B*Q = 528; B*Q = 2080 takes the tiled product for
    # long passes, with a ragged last tile of 32)
    rng = np.random.default_rng(100 + B * Q)
    h = small_int_bits(rng, (B, Q, HIDDEN))
    w = small_int_bits(rng, (R, HIDDEN))
    lens = rng.integers(Q, L + 1, B).astype(np.int32)
    lens[0] = L
    cache = wl.normal_bf16(np.random.SeedSequence([7, B, Q]), B * L * R).reshape(B, L, R)
    print(f"append exact B={B} Q={Q} L={L}", flush=True)
    got = run_append(cache, lens, h, w)
    np.testing.assert_array_equal(got, la.append_reference(cache, lens, h, w))


def test_positions_outside_the_cache_are_skipped():
    # a length below Q breaks the precondition: tokens whose position would be negative are not
    # written, the others land at 0 .. cache_len - 1, nothing else changes
    rng = np.random.default_rng(5)
    h = small_int_bits(rng, (2, 4, HIDDEN))
    w = small_int_bits(rng, (R, HIDDEN))
    lens = np.array([2, 4], np.int32)
    cache = np.full((2, 8, R), wl.BF16_NAN, np.uint16)
    got = run_append(cache, lens, h, w)
    rows = la.latent_rows(h, w)
    want = cache.copy()
    want[0, 0:2] = rows[0, 2:4]
    want[1, 0:4] = rows[1]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("name", ["decode_b32_l8192", "verify_b16_q6_l32768"])
def test_workload_shapes(name):
    # the pass's new tokens at the workload's batch shape, N(0, 1) hidden states and an
    # N(0, 1/4096) projection; a small cache per sequence (the rows written depend only on h, W
    # and the lengths)
    spec = wl.WORKLOADS[name]
    inp = wl.make_append_inputs(spec)
    B, Q = spec.batch, spec.q_len
    L = 64
    lens = np.random.default_rng(3).integers(Q, L + 1, B).astype(np.int32)
    cache = wl.normal_bf16(np.random.SeedSequence([8, B]), B * L * R).reshape(B, L, R)
    print(f"append {name}: B={B} Q={Q}", flush=True)
    got = run_append(cache, lens, inp.h, inp.w_dkv)
    frac = check_rows(got, cache, lens, inp.h, inp.w_dkv)
    assert frac > 0.99


def test_prefill_chunk_rows():
    # many tokens in one pass (a prefill chunk of 1000 tokens for one sequence): every row group
    # loops over several tiles, and the last tile is ragged
    spec = wl.WORKLOADS["decode_b32_l8192"]
    inp = wl.make_append_inputs(spec, rows=1000)
    h = inp.h.reshape(1, 1000, HIDDEN)
    cache = np.full((1, 1024, R), wl.BF16_NAN, np.uint16)
    lens = np.array([1010], np.int32)
    print("append prefill chunk 1000 tokens", flush=True)
    got = run_append(cache, lens, h, inp.w_dkv)
    assert check_rows(got, cache, lens, h, inp.w_dkv) > 0.99


def test_full_size_cache_append():
    # the decode workload's full cache (32 x 8192 rows): the last row of each sequence is
    # written, the other 256 MiB stay as they were
    spec = wl.WORKLOADS["decode_b32_l8192"]
    inp = wl.make_append_inputs(spec)
    B, L = spec.batch, spec.cache_len
    cache = torch.randint(-32768, 32767, (B, L, R), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    before = cache.clone()
    lens = np.full(B, L, np.int32)
    lens[1::2] = L - 5
    print("append full-size decode cache", flush=True)
    binding.mla_latent_append(bf16(inp.h), bf16(inp.w_dkv), cache, i32(lens), L)
    torch.cuda.synchronize()
    pos = torch.from_numpy(lens - 1).long().to(DEV)
    ar = torch.arange(B, device=DEV)
    got_rows = bits(cache[ar, pos]).reshape(B, 1, R)
    lo, hi = la.rounding_interval(inp.h, inp.w_dkv, REL)
    v = mo.bf16_bits_to_f64(got_rows)
    assert np.all((lo <= v) & (v <= hi))
    cache[ar, pos] = before[ar, pos]
    assert torch.equal(cache.view(torch.int16), before.view(torch.int16))


@pytest.mark.parametrize("B,Q", [(1, 2100), (3, 700)])
def test_long_pass_matches_short_passes(B, Q):
    # a pass of 2048 tokens or more takes the tiled product; the same tokens appended 100 at a
    # time take the batch kernel.  Same sum in the same order: identical bits, and rows within
    # the bound (2100 tokens = 32 tiles of 64 and a ragged one; three sequences of ragged lengths)
    spec = wl.WORKLOADS["decode_b32_l8192"]
    inp = wl.make_append_inputs(spec, rows=B * Q)
    h = inp.h.reshape(B, Q, HIDDEN)
    L = 2200
    lens = np.array([2150, 1500, 733][:B], np.int32) if B == 3 else np.array([2120], np.int32)
    cache0 = np.full((B, L, R), wl.BF16_NAN, np.uint16)
    print(f"append long pass B={B} Q={Q}", flush=True)
    long = run_append(cache0, lens, h, inp.w_dkv)
    assert check_rows(long, cache0, lens, h, inp.w_dkv) > 0.99
    short = cache0.copy()
    for k in range(Q // 100):
        part = np.ascontiguousarray(h[:, 100 * k:100 * (k + 1)])
        short = run_append(short, lens - Q + 100 * (k + 1), part, inp.w_dkv)
    np.testing.assert_array_equal(long, short)


def test_same_token_same_bits_in_any_batch():
    # a token's row depends only on its hidden state: projected inside a 6-token verification
    # pass or alone, it gets identical bits
    spec = wl.WORKLOADS["verify_b16_q6_l32768"]
    inp = wl.make_append_inputs(spec)
    h = inp.h[:2]                                   # [2, 6, hidden]
    cache6 = run_append(np.zeros((2, 16, R), np.uint16), np.array([10, 16], np.int32), h, inp.w_dkv)
    for i in range(6):
        one = run_append(np.zeros((2, 16, R), np.uint16), np.array([5 + i, 11 + i], np.int32),
                         np.ascontiguousarray(h[:, i:i + 1]), inp.w_dkv)
        np.testing.assert_array_equal(one[0, 4 + i], cache6[0, 4 + i])
        np.testing.assert_array_equal(one[1, 10 + i], cache6[1, 10 + i])


def test_rollback_equals_never_generated():
    # page "Module 08", section 3: a verification pass appends the current token and five
    # drafts, two drafts are accepted and the cache is rolled back to them, then the next token
    # is appended and decoded.  A run that only ever saw the accepted tokens must reach the same
    # cache prefix and the same attention output, bit for bit (same split count in both runs).
    rng = np.random.default_rng(11)
    spec = wl.make_spec(1, 6, 512, workload_id=211)
    w = wl.make_workload(spec)
    inp = wl.make_append_inputs(spec)
    L0, L_max = 300, 512
    base = np.full((1, L_max, R), wl.BF16_NAN, np.uint16)
    base[0, :L0] = w.cache[0, :L0]
    h_pass = inp.h                                     # [1, 6, hidden]: current token + 5 drafts
    h_next = wl.normal_bf16(np.random.SeedSequence([12]), HIDDEN).reshape(1, 1, HIDDEN)
    q_next = w.q[:, :1]                                # [1, 1, H, D]
    wk, wv = bf16(w.w_k), bf16(w.w_v)
    wd = bf16(inp.w_dkv)
    splits = 4

    def attend(cache_t, L, q):
        out, lse = binding.mla_forward(bf16(q), wk, wv, cache_t, i32([L]), L_max, spec.scale,
                                       num_splits=splits)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    # run A: verify pass of 6, accept 1 + 2, roll back, append and decode the next token
    ca = bf16(base)
    binding.mla_latent_append(bf16(h_pass), wd, ca, i32([L0 + 6]), L_max)
    out_a6, _ = attend(ca, L0 + 6, w.q)
    binding.mla_latent_append(bf16(h_next), wd, ca, i32([L0 + 4]), L_max)
    out_a, lse_a = attend(ca, L0 + 4, q_next)
    # run B: only the accepted tokens, then the same next token
    cb = bf16(base)
    binding.mla_latent_append(bf16(np.ascontiguousarray(h_pass[:, :3])), wd, cb, i32([L0 + 3]), L_max)
    out_b3, _ = attend(cb, L0 + 3, np.ascontiguousarray(w.q[:, :3]))
    binding.mla_latent_append(bf16(h_next), wd, cb, i32([L0 + 4]), L_max)
    out_b, lse_b = attend(cb, L0 + 4, q_next)
    a_bits, b_bits = bits(ca), bits(cb)
    print("rollback: comparing caches and outputs", flush=True)
    np.testing.assert_array_equal(a_bits[0, :L0 + 4], b_bits[0, :L0 + 4])
    assert not np.array_equal(a_bits[0, L0 + 4], b_bits[0, L0 + 4])   # stale rejected draft
    np.testing.assert_array_equal(out_a, out_b)
    np.testing.assert_array_equal(lse_a, lse_b)
    # the verification pass's accepted queries saw exactly what the accepted-only pass saw
    np.testing.assert_array_equal(out_a6[:, :3], out_b3)
    # and the decoded output matches the oracle on the rolled-back state
    ref, ref_lse = mo.mla_reference(q_next, b_bits, w.w_k, w.w_v, np.array([L0 + 4]), spec.scale)
    err = float(np.abs(out_a - ref).max())
    assert err <= 1e-2 * float(np.abs(ref).max()) + 1e-3, err

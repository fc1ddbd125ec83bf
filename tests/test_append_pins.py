"""Pins of the down-projection / append / rollback oracle to facts the pages and mathematics fix
(CPU only).

Page "Module 05 -- MLA: Compressing Per-Token History", section 1: each token is projected down
to one shared 512-wide latent, which is what the cache keeps.  Page "Module 08 -- Vision, MTP,
and Hybrid Serving State", section 3: the latent cache is truncatable by position, and the state
after a rollback must equal that of a run that never generated the rejected tokens.
"""
import numpy as np
import pytest
import torch

from mla_latent_cache_absorb_amd import workloads as wl
from oracle import latent_append as la
from oracle import mla_oracle as mo


def bits(x):
    return wl.f32_to_bf16_bits(np.asarray(x, np.float32))


# ---- rounding to bf16 ------------------------------------------------------------------------
def test_rounding_matches_torch_on_float32_values():
    # a library routine: torch rounds float32 to bfloat16 to nearest, ties to even
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([u, (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)])  # exact ties
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = la.f64_to_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_rounding_worked_cases():
    # hand-checked: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes to the even one (1);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 and goes to 1 + 2^-6 (even);
    # a hair above the halfway point rounds up; half the smallest subnormal rounds to zero (even);
    # 3.4e38 lies past the halfway point above the largest bf16 and overflows to infinity
    cases = {1 + 2 ** -8: 0x3F80, 1 + 3 * 2 ** -8: 0x3F82, -(1 + 2 ** -8 + 2 ** -30): 0xBF81,
             2.0 ** -134: 0x0000, 3 * 2.0 ** -134: 0x0002, 255.5: 0x4380, 3.0e38: 0x7F62, 3.4e38: 0x7F80}
    for x, want in cases.items():
        assert int(la.f64_to_bf16_bits(np.array([x]))[0]) == want, (x, hex(want))


def test_rounding_is_not_truncation():
    # values just below a bf16 neighbour must round up, which truncating the bits would miss
    x = np.array([1.0 + 2 ** -7 - 2 ** -12])
    assert int(la.f64_to_bf16_bits(x)[0]) == 0x3F81


# ---- the projection ------------------------------------------------------------------------
def test_one_hot_hidden_state_picks_a_column():
    # c = W h with h = e_k is column k of W; the transposed operand would give row k instead
    rng = np.random.default_rng(3)
    w = bits(rng.standard_normal((6, 6)))
    for k in range(6):
        h = np.zeros(6, np.float32)
        h[k] = 1.0
        c = la.down_project(bits(h), w)
        np.testing.assert_array_equal(c, mo.bf16_bits_to_f64(w)[:, k])
        assert not np.array_equal(c, mo.bf16_bits_to_f64(w)[k, :])


def test_projection_by_scalar_loops():
    # brute force on a tiny case, with Python floats summed in order
    rng = np.random.default_rng(4)
    h = bits(rng.standard_normal((3, 5)))
    w = bits(rng.standard_normal((4, 5)))
    hf, wf = mo.bf16_bits_to_f64(h), mo.bf16_bits_to_f64(w)
    want = np.zeros((3, 4))
    for n in range(3):
        for r in range(4):
            s = 0.0
            for k in range(5):
                s += float(wf[r, k]) * float(hf[n, k])
            want[n, r] = s
    np.testing.assert_allclose(la.down_project(h, w), want, rtol=1e-15, atol=0)


def test_small_integers_project_exactly():
    # integer inputs give integer latents, so the stored rows are known exactly
    h = bits([[1, -2, 0, 3]])
    w = bits([[1, 1, 1, 1], [2, 0, -1, 0], [0, 0, 0, 4]])
    np.testing.assert_array_equal(la.down_project(h, w), [[2.0, 2.0, 12.0]])
    np.testing.assert_array_equal(la.latent_rows(h, w), bits([[2.0, 2.0, 12.0]]))


def test_rounding_interval_brackets_the_rounded_value():
    rng = np.random.default_rng(5)
    h = bits(rng.standard_normal((4, 64)))
    w = bits(rng.standard_normal((8, 64)) / 8)
    lo, hi = la.rounding_interval(h, w, 0.0)
    exact = mo.bf16_bits_to_f64(la.latent_rows(h, w))
    np.testing.assert_array_equal(lo, exact)
    np.testing.assert_array_equal(hi, exact)
    lo, hi = la.rounding_interval(h, w, 1e-3)
    assert np.all(lo <= exact) and np.all(exact <= hi) and np.any(lo < hi)


# ---- append position and rollback ------------------------------------------------------------
def _tiny_model(rng, H=2, D=3, R=4, hidden=5):
    w_k = bits(rng.standard_normal((H, D, R)) / 2)
    w_v = bits(rng.standard_normal((H, D, R)) / 2)
    w_dkv = bits(rng.standard_normal((R, hidden)) / 2)
    return w_k, w_v, w_dkv


def test_first_token_attends_to_its_own_projected_latent():
    # cache_len = Q = 1: the only visible position is the token's own, so the output is
    # U^V (W h) computed from the rounded row -- ties the append position to the attention's
    rng = np.random.default_rng(6)
    w_k, w_v, w_dkv = _tiny_model(rng)
    h = bits(rng.standard_normal((1, 1, 5)))
    cache = np.full((1, 3, 4), wl.BF16_NAN, np.uint16)
    cache = la.append_reference(cache, np.array([1]), h, w_dkv)
    q = bits(rng.standard_normal((1, 1, 2, 3)))
    out, _ = mo.mla_reference(q, cache, w_k, w_v, np.array([1]), 0.5)
    c = mo.bf16_bits_to_f64(la.latent_rows(h, w_dkv))[0, 0]
    for hh in range(2):
        np.testing.assert_allclose(out[0, 0, hh], mo.bf16_bits_to_f64(w_v[hh]) @ c, rtol=1e-13)


def test_append_writes_only_the_last_q_rows():
    rng = np.random.default_rng(8)
    _, _, w_dkv = _tiny_model(rng)
    cache = bits(rng.standard_normal((2, 9, 4)))
    h = bits(rng.standard_normal((2, 3, 5)))
    new = la.append_reference(cache, np.array([5, 9]), h, w_dkv)
    rows = la.latent_rows(h, w_dkv)
    np.testing.assert_array_equal(new[0, 2:5], rows[0])
    np.testing.assert_array_equal(new[1, 6:9], rows[1])
    np.testing.assert_array_equal(new[0, :2], cache[0, :2])
    np.testing.assert_array_equal(new[0, 5:], cache[0, 5:])
    np.testing.assert_array_equal(new[1, :6], cache[1, :6])
    with pytest.raises(ValueError):
        la.append_reference(cache, np.array([2, 9]), h, w_dkv)   # 2 - 3 < 0


def _rollback_runs(rng, history=6, drafts=4, accepted=2):
    w_k, w_v, w_dkv = _tiny_model(rng)
    L_max = history + drafts + 2
    base = np.full((1, L_max, 4), wl.BF16_NAN, np.uint16)
    base[0, :history] = bits(rng.standard_normal((history, 4)))
    h_drafts = bits(rng.standard_normal((1, drafts, 5)))
    h_next = bits(rng.standard_normal((1, 1, 5)))
    q = bits(rng.standard_normal((1, 1, 2, 3)))
    # run A: verify pass appends every draft, rollback keeps `accepted`, then the next token
    a = la.append_reference(base, np.array([history + drafts]), h_drafts, w_dkv)
    len_a = history + accepted + 1
    a = la.append_reference(a, np.array([len_a]), h_next, w_dkv)
    # run B: never generated the rejected drafts
    b = la.append_reference(base, np.array([history + accepted]), h_drafts[:, :accepted], w_dkv)
    b = la.append_reference(b, np.array([history + accepted + 1]), h_next, w_dkv)
    return (w_k, w_v, q), a, b, len_a


def test_rollback_state_equals_never_generated():
    # Module 08 section 3: after rollback the cache's visible prefix and the attention output
    # equal those of a run that only generated the accepted tokens
    (w_k, w_v, q), a, b, L = _rollback_runs(np.random.default_rng(9))
    np.testing.assert_array_equal(a[0, :L], b[0, :L])
    assert not np.array_equal(a[0, L], b[0, L])  # a stale rejected draft remains past the length
    out_a, lse_a = mo.mla_reference(q, a, w_k, w_v, np.array([L]), 0.5)
    out_b, lse_b = mo.mla_reference(q, b, w_k, w_v, np.array([L]), 0.5)
    np.testing.assert_array_equal(out_a, out_b)
    np.testing.assert_array_equal(lse_a, lse_b)


def test_planted_mistake_rollback_without_truncation_is_caught():
    # a rollback that forgets to lower the length still sees the rejected draft: the check above
    # must tell the two apart
    (w_k, w_v, q), a, b, L = _rollback_runs(np.random.default_rng(9))
    out_a, _ = mo.mla_reference(q, a, w_k, w_v, np.array([L + 1]), 0.5)
    out_b, _ = mo.mla_reference(q, b, w_k, w_v, np.array([L]), 0.5)
    assert not np.allclose(out_a, out_b)

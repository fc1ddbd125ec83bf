"""The C ABI: the library builds, loads, exports every entry point include/mla_absorb.h
declares, and its host-side validation answers without touching a GPU."""
import ctypes
import os
import re

import pytest

from mla_latent_cache_absorb_amd import binding, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mla_absorb.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert "mla_latent_attn" in names and "mla_latent_attn_indexed" in names
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), f"missing export {n}"
    # exported with C linkage (no mangling)
    out = os.popen(f"nm -D --defined-only {binding.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert binding.status_string(s) and binding.status_string(s) != "unknown status"
    assert "workspace" in binding.status_string(binding.MLA_ERR_WORKSPACE)


def test_host_validation_without_device(L):
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    # null pointers and shapes are rejected before any device call
    assert L.mla_absorb_q(None, fake, fake, None, 1, 64, 256, 512, 1.0, None) == binding.MLA_ERR_NULL
    assert L.mla_absorb_q(fake, fake, fake, None, 1, 64, 128, 512, 1.0, None) == binding.MLA_ERR_SHAPE
    assert L.mla_absorb_q(fake, fake, fake, None, 1, 40, 256, 512, 1.0, None) == binding.MLA_ERR_SHAPE  # H % 16 != 0
    assert L.mla_absorb_q(fake, fake, fake, None, 0, 64, 256, 512, 1.0, None) == binding.MLA_ERR_SHAPE
    assert L.mla_absorb_q(fake, fake, fake, None, 1, 64, 256, 512, float("nan"), None) == binding.MLA_ERR_ARG
    assert L.mla_up_v(fake, None, fake, 1, 64, 256, 512, None) == binding.MLA_ERR_NULL
    assert L.mla_up_v(fake, fake, fake, 1, 64, 256, 256, None) == binding.MLA_ERR_SHAPE
    a = dict(q=fake, c=fake, st=512 * 100, cl=fake)
    assert L.mla_latent_attn(fake, None, fake, 51200, None, 1, 1, 64, 512, 100, 0.0625, 0, fake, None, None, 0, None) \
        == binding.MLA_ERR_NULL
    assert L.mla_latent_attn(fake, None, fake, 51200, fake, 1, 1, 64, 512, 100, 0.0625, -1, fake, None, None, 0, None) \
        == binding.MLA_ERR_ARG
    # batch stride shorter than max_cache_len rows
    assert L.mla_latent_attn(fake, None, fake, 512 * 99, fake,
                             1, 1, 64, 512, 100, 0.0625, 0, fake, None, None, 0, None) \
        == binding.MLA_ERR_ARG
    assert L.mla_latent_attn(fake, None, fake, 51200, fake, 1, 1, 64, 512, 100, -1.0, 0, fake, None, None, 0, None) \
        == binding.MLA_ERR_ARG
    assert L.mla_latent_attn(fake, None, fake, 51200, fake, 1, 4, 64, 512, 3, 0.0625, 0, fake, None, None, 0, None) \
        == binding.MLA_ERR_ARG
    assert L.mla_latent_attn_indexed(fake, None, fake, 51200, fake, None, fake, 8, 1, 1, 64, 512, 100, 0.0625, 0, fake,
                                     None, None, 0, None) == binding.MLA_ERR_NULL
    assert L.mla_latent_attn_indexed(fake, None, fake, 51200, fake, fake, fake, 0, 1, 1, 64, 512, 100, 0.0625, 0, fake,
                                     None, None, 0, None) == binding.MLA_ERR_ARG


def test_split_sizing(L):
    # at least one split; never more than one per 32-position tile; workspace matches the count
    for B, Q, Lmax in ((1, 1, 1), (1, 1, 256), (32, 1, 8192), (16, 6, 32768), (4, 1, 131072), (32, 4, 2052)):
        s = binding.mla_latent_attn_num_splits(B, Q, 64, Lmax, 0)
        assert 1 <= s <= max(1, (Lmax + 31) // 32)
        ws = binding.mla_latent_attn_workspace_size(B, Q, 64, 512, Lmax, 0)
        # fp16 normalised partials, then fp32 (m, l) per row
        assert ws == (0 if s == 1 else s * B * Q * 64 * (512 * 2 + 2 * 4))
    # splits hold whole 32-position tiles and none is left empty
    assert binding.mla_latent_attn_num_splits(1, 1, 64, 256, 8) == 8
    assert binding.mla_latent_attn_num_splits(1, 1, 64, 256, 5) == 4   # 8 tiles as 2+2+2+2
    assert binding.mla_latent_attn_num_splits(1, 1, 64, 64, 5) == 2    # two tiles at most
    assert binding.mla_latent_attn_num_splits(1, 1, 64, 100, 3) == 2   # 4 tiles as 2+2
    assert binding.mla_latent_attn_workspace_size(1, 1, 64, 512, 256, 1) == 0


def test_split_choice_without_device(L):
    # with no GPU visible the choice assumes 256 CUs, one workgroup per CU: whole rounds of
    # workgroups, as few splits (partials) as that allows
    assert binding.mla_latent_attn_num_splits(32, 1, 64, 8192, 0) == 8          # 256 workgroups
    assert binding.mla_latent_attn_num_splits(4, 1, 64, 131072, 0) == 64        # 256 workgroups
    # dense calls with an even number of queries take them in pairs: 16 x 3 pairs x 5 splits = 240
    assert binding.mla_latent_attn_num_splits(16, 6, 64, 32768, 0) == 5
    assert binding.mla_latent_attn_num_splits(16, 6, 64, 32768, 0, indexed=True) == 8  # 768 = 3 rounds


def test_split_choice_counts_query_pairs(L):
    # the work units the choice prices: pairs of queries for dense calls with an even Q, single
    # queries otherwise, so a dense call with 2P queries chooses as an indexed call with P
    for B, Lmax in ((16, 32768), (32, 8192), (4, 131072), (3, 1000)):
        for Q in (2, 4, 6, 8):
            assert (binding.mla_latent_attn_num_splits(B, Q, 64, Lmax, 0)
                    == binding.mla_latent_attn_num_splits(B, Q // 2, 64, Lmax, 0, indexed=True)), (B, Q)
        for Q in (1, 3, 5, 7):
            assert (binding.mla_latent_attn_num_splits(B, Q, 64, Lmax, 0)
                    == binding.mla_latent_attn_num_splits(B, Q, 64, Lmax, 0, indexed=True)), (B, Q)
    # 16 sequences of 32,768 positions: one round of 256 (Q = 2: 16 pairs x 16; Q = 8: 64 x 4)
    assert binding.mla_latent_attn_num_splits(16, 2, 64, 32768, 0) == 16
    assert binding.mla_latent_attn_num_splits(16, 8, 64, 32768, 0) == 4
    assert binding.mla_latent_attn_num_splits(32, 4, 64, 2052, 0, indexed=True) == 2
    assert binding.mla_latent_attn_workspace_size(32, 4, 64, 512, 2052, 0, indexed=True) == 2 * 128 * 64 * 1032


def test_indexer_host_validation(L):
    fake = ctypes.c_void_p(0x1000)
    # null pointers, bad widths, and sizes the kernels cannot hold are refused before any launch
    assert L.mla_kpool_keys(None, fake, 128 * 64, fake, None, 1, 64, 128, 4, fake, 16, None) == binding.MLA_ERR_NULL
    assert L.mla_kpool_keys(fake, fake, 96 * 64, fake, None, 1, 64, 96, 4, fake, 16, None) == binding.MLA_ERR_SHAPE
    assert L.mla_kpool_keys(fake, fake, 128 * 63, fake, None, 1, 64, 128, 4, fake, 16, None) == binding.MLA_ERR_ARG
    assert L.mla_kpool_keys(fake, fake, 128 * 64 + 4, fake, None, 1, 64, 128, 4, fake, 16, None) == binding.MLA_ERR_ARG
    assert L.mla_kpool_keys(fake, fake, 128 * 64, fake, None, 1, 64, 128, 4, fake, 15, None) == binding.MLA_ERR_ARG
    assert L.mla_indexer_scores(fake, fake, fake, 1, 9, 128, 4, 16, 64, fake, None) == binding.MLA_ERR_SHAPE
    assert L.mla_indexer_scores(fake, None, fake, 1, 4, 128, 4, 16, 64, fake, None) == binding.MLA_ERR_NULL
    # topk must be a multiple of the pool, rows must hold topk + pool - 1 with the tail
    assert L.mla_indexer_select(fake, fake, 1, 1, 4, 16, 64, 6, 1, fake, fake, 9, None) == binding.MLA_ERR_ARG
    assert L.mla_indexer_select(fake, fake, 1, 1, 4, 16, 64, 8, 1, fake, fake, 10, None) == binding.MLA_ERR_ARG
    assert L.mla_indexer_select(fake, fake, 1, 1, 4, 16384 * 2, 65536 * 2, 8, 1, fake, fake, 11, None) \
        == binding.MLA_ERR_ARG


def test_append_host_validation(L):
    fake = ctypes.c_void_p(0x1000)
    # null pointers, widths other than 4096 -> 512, and a stride or cache too small for the pass
    assert L.mla_latent_append(None, fake, fake, 512 * 64, fake, 1, 1, 4096, 512, 64, None) == binding.MLA_ERR_NULL
    assert L.mla_latent_append(fake, fake, fake, 512 * 64, None, 1, 1, 4096, 512, 64, None) == binding.MLA_ERR_NULL
    assert L.mla_latent_append(fake, fake, fake, 512 * 64, fake, 1, 1, 2048, 512, 64, None) == binding.MLA_ERR_SHAPE
    assert L.mla_latent_append(fake, fake, fake, 512 * 64, fake, 1, 1, 4096, 256, 64, None) == binding.MLA_ERR_SHAPE
    assert L.mla_latent_append(fake, fake, fake, 512 * 64, fake, 0, 1, 4096, 512, 64, None) == binding.MLA_ERR_SHAPE
    assert L.mla_latent_append(fake, fake, fake, 512 * 63, fake, 1, 1, 4096, 512, 64, None) == binding.MLA_ERR_ARG
    assert L.mla_latent_append(fake, fake, fake, 512 * 64, fake, 1, 6, 4096, 512, 5, None) == binding.MLA_ERR_ARG


def test_fused_up_projection_host_validation(L):
    fake = ctypes.c_void_p(0x1000)
    f = L.mla_latent_attn_up_v
    # args: q_abs q_abs_lo cache stride cache_len idx idx_len K_max B Q H R max_len scale splits w_v D out lse ws
    # bytes stream
    ok = [fake, None, fake, 51200, fake, None, None, 0, 1, 1, 64, 512, 100, 0.0625, 0, fake, 256, fake, None, fake,
          1 << 30, None]

    def call(**kw):
        a = list(ok)
        names = ["q", "q_lo", "c", "st", "cl", "idx", "idx_len", "K", "B", "Q", "H", "R", "L", "scale", "s", "w_v", "D",
                 "out", "lse", "ws", "wsb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(w_v=None) == binding.MLA_ERR_NULL
    assert call(out=None) == binding.MLA_ERR_NULL
    assert call(idx=fake) == binding.MLA_ERR_NULL          # idx without idx_len
    assert call(idx_len=fake) == binding.MLA_ERR_NULL      # idx_len without idx
    assert call(D=128) == binding.MLA_ERR_SHAPE
    assert call(H=40) == binding.MLA_ERR_SHAPE  # not a multiple of 16
    assert call(scale=0.0) == binding.MLA_ERR_ARG
    assert call(st=512 * 99) == binding.MLA_ERR_ARG
    assert call(idx=fake, idx_len=fake, K=0) == binding.MLA_ERR_ARG
    # workspace: the split partials, or the accumulated latents when there is one split
    s = binding.mla_latent_attn_num_splits(32, 1, 64, 8192, 0)
    assert binding.mla_latent_attn_up_v_workspace_size(32, 1, 64, 512, 8192, 0) == \
        binding.mla_latent_attn_workspace_size(32, 1, 64, 512, 8192, 0) == s * 32 * 64 * 1032
    assert binding.mla_latent_attn_up_v_workspace_size(2, 3, 64, 512, 256, 1) == 2 * 3 * 64 * 512 * 4
    assert binding.mla_latent_attn_up_v_workspace_size(2, 3, 64, 256, 256, 1) == 0


def test_noalloc_host_validation(L):
    fake = ctypes.c_void_p(0x1000)
    f = L.mla_latent_attn_up_v_noalloc
    # args: q_abs q_abs_lo cache stride cache_len idx idx_len K_max B Q H R max_len scale splits w_v D out lse stream
    ok = [fake, None, fake, 51200, fake, None, None, 0, 1, 1, 64, 512, 100, 0.0625, 0, fake, 256, fake, None, None]
    names = ["q", "q_lo", "c", "st", "cl", "idx", "idx_len", "K", "B", "Q", "H", "R", "L", "scale", "s", "w_v", "D",
             "out", "lse", "stream"]

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    # every host-side error comes before the device is touched (no GPU here)
    assert call(w_v=None) == binding.MLA_ERR_NULL
    assert call(out=None) == binding.MLA_ERR_NULL
    assert call(q=None) == binding.MLA_ERR_NULL
    assert call(idx=fake) == binding.MLA_ERR_NULL
    assert call(D=128) == binding.MLA_ERR_SHAPE
    assert call(R=256) == binding.MLA_ERR_SHAPE
    assert call(scale=float("inf")) == binding.MLA_ERR_ARG
    assert call(st=512 * 99) == binding.MLA_ERR_ARG
    assert call(s=-1) == binding.MLA_ERR_ARG
    # the four full-size workloads fit the fixed scratch
    for B, Q, Lmax, ind in ((32, 1, 8192, False), (16, 6, 32768, False), (4, 1, 131072, False),
                            (32, 4, 2052, True)):
        assert binding.mla_latent_attn_up_v_workspace_size(B, Q, 64, 512, Lmax, 0, ind) <= \
            binding.NOALLOC_SCRATCH_BYTES
    # the binding allocates nothing for it: out is required
    import torch
    with pytest.raises(ValueError):
        binding.mla_latent_attn_up_v_noalloc(_bf(1, 1, 64, 512), _bf(1, 40, 512), _i32(1), 40, 0.0625,
                                             _bf(64, 256, 512), None)


def test_second_query_term_host_validation(L):
    # a second query term must match the first's dtype and shape; checked before any device use
    import torch
    qa, c, cl, wv = _bf(1, 1, 64, 512), _bf(1, 40, 512), _i32(1), _bf(64, 256, 512)
    with pytest.raises(ValueError):
        binding.mla_latent_attn(qa, c, cl, 40, 0.0625, q_abs_lo=_bf(1, 1, 64, 256))
    with pytest.raises(TypeError):
        binding.mla_latent_attn(qa, c, cl, 40, 0.0625, q_abs_lo=torch.zeros(1, 1, 64, 512))
    with pytest.raises(ValueError):
        binding.mla_latent_attn_up_v(qa, c, cl, 40, 0.0625, wv, q_abs_lo=_bf(2, 1, 64, 512))
    with pytest.raises(ValueError):
        binding.mla_latent_attn_indexed(qa, c, cl, _i32(1, 1, 8), _i32(1, 1), 40, 0.0625, q_abs_lo=_bf(1, 1, 48, 512))
    with pytest.raises(ValueError):
        binding.mla_absorb_q(_bf(1, 64, 256), _bf(64, 256, 512), q_abs_lo=_bf(1, 64, 256))
    # the C ABI takes NULL for the second term and validates the rest as before
    fake = ctypes.c_void_p(0x1000)
    assert L.mla_latent_attn_up_v(None, fake, fake, 51200, fake, None, None, 0, 1, 1, 64, 512, 100, 0.0625, 0, fake,
                                  256, fake, None, fake, 1 << 30, None) == binding.MLA_ERR_NULL


def test_stream_read_host_validation(L):
    fake = ctypes.c_void_p(0x1000)
    f = L.mla_stream_read
    assert f(None, 32768, 0, fake, None) == binding.MLA_ERR_NULL
    assert f(fake, 32768, 0, None, None) == binding.MLA_ERR_NULL
    assert f(fake, 0, 0, fake, None) == binding.MLA_ERR_SHAPE
    assert f(fake, 32768 + 16, 0, fake, None) == binding.MLA_ERR_SHAPE
    with pytest.raises(ValueError):
        binding.mla_stream_read(_bf(100), _i32(1))


def test_input_check_host_validation(L):
    fake = ctypes.c_void_p(0x1000)
    f = L.mla_check_attn_inputs
    # args: cache_len idx idx_len B Q K_max max_cache_len flags stream
    assert f(None, None, None, 1, 1, 0, 10, fake, None) == binding.MLA_ERR_NULL
    assert f(fake, None, None, 1, 1, 0, 10, None, None) == binding.MLA_ERR_NULL
    assert f(fake, fake, None, 1, 1, 4, 10, fake, None) == binding.MLA_ERR_NULL
    assert f(fake, None, fake, 1, 1, 4, 10, fake, None) == binding.MLA_ERR_NULL
    assert f(fake, None, None, 0, 1, 0, 10, fake, None) == binding.MLA_ERR_SHAPE
    assert f(fake, None, None, 1, 0, 0, 10, fake, None) == binding.MLA_ERR_SHAPE
    assert f(fake, None, None, 1, 1, 0, 0, fake, None) == binding.MLA_ERR_SHAPE
    assert f(fake, fake, fake, 1, 1, 0, 10, fake, None) == binding.MLA_ERR_ARG
    # the flag bits the header names
    assert set(binding.BAD_INPUT_BITS) == {1, 2, 4, 8, 16, 32}


# --------------------------------------------------------------------------------------------
# The binding checks every tensor's extent against the call's sizes before anything is launched:
# on tensors in host memory a mismatch raises ValueError and matching shapes get as far as the
# device check (TypeError), so none of these calls reaches the library's compute entry points.
def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def _i32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.int32)


def _f32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


def _attn_args(B=2, Q=3, H=64, R=512, L=40):
    return dict(q_abs=_bf(B, Q, H, R), cache=_bf(B, L, R), cache_len=_i32(B), max_cache_len=L, scale=0.0625)


def _expect(exc, fn, **kw):
    with pytest.raises(exc):
        fn(**kw)


def test_attention_wrappers_check_every_extent(L):
    ok = _attn_args()
    _expect(TypeError, binding.mla_latent_attn, **ok)      # shapes fine: stopped by the device check
    bad = [
        dict(cache=_bf(3, 40, 512)),                        # more sequences than q_abs
        dict(cache=_bf(1, 40, 512)),                        # fewer
        dict(cache=_bf(2, 40, 256)),                        # another latent width
        dict(max_cache_len=41),                             # longer than the cache rows
        dict(max_cache_len=0),
        dict(cache_len=_i32(3)),
        dict(cache_len=_i32(2, 1)),
        dict(o_lat=_f32(2, 3, 64, 256)),
        dict(lse=_f32(2, 3, 63)),
        dict(q_abs=_bf(2, 3, 64 * 512)),                    # not [B, Q, H, R]
    ]
    for b in bad:
        _expect(ValueError, binding.mla_latent_attn, **{**ok, **b})
    idx_ok = dict(idx=_i32(2, 3, 7), idx_len=_i32(2, 3))
    _expect(TypeError, binding.mla_latent_attn_indexed, **ok, **idx_ok)
    for b in (dict(idx=_i32(2, 2, 7)), dict(idx=_i32(3, 3, 7)), dict(idx=_i32(2, 3, 0)), dict(idx=_i32(2, 3)),
              dict(idx_len=_i32(2, 2)), dict(idx_len=_i32(3, 3)), dict(idx_len=None)):
        _expect(ValueError, binding.mla_latent_attn_indexed, **ok, **{**idx_ok, **b})
        _expect(ValueError, binding.mla_latent_attn_up_v, **ok, w_v=_bf(64, 256, 512), **{**idx_ok, **b})
    _expect(TypeError, binding.mla_latent_attn_up_v, **ok, w_v=_bf(64, 256, 512))
    for b in (dict(w_v=_bf(32, 256, 512)), dict(w_v=_bf(64, 256, 256)), dict(out=_f32(2, 3, 64, 512)),
              dict(lse=_f32(2, 3)), dict(cache=_bf(2, 39, 512))):
        _expect(ValueError, binding.mla_latent_attn_up_v, **{**ok, "w_v": _bf(64, 256, 512), **b})
    # the debug precondition check
    _expect(TypeError, binding.mla_check_attn_inputs, cache_len=_i32(2), Q=3, max_cache_len=40, **idx_ok)
    _expect(ValueError, binding.mla_check_attn_inputs, cache_len=_i32(2), Q=4, max_cache_len=40, **idx_ok)
    _expect(ValueError, binding.mla_check_attn_inputs, cache_len=_i32(2), Q=3, max_cache_len=40,
            idx=_i32(2, 3, 7), idx_len=_i32(2, 4))


def test_projection_wrappers_check_every_extent(L):
    _expect(TypeError, binding.mla_absorb_q, q=_bf(4, 64, 256), w_k=_bf(64, 256, 512))
    _expect(ValueError, binding.mla_absorb_q, q=_bf(4, 64, 128), w_k=_bf(64, 256, 512))
    _expect(ValueError, binding.mla_absorb_q, q=_bf(4, 64, 256), w_k=_bf(64, 256, 512), q_abs=_bf(4, 64, 256))
    _expect(ValueError, binding.mla_absorb_q, q=_bf(4, 64, 256), w_k=_bf(64, 256, 512), q_abs=_bf(3, 64, 512))
    _expect(TypeError, binding.mla_up_v, o_lat=_f32(4, 64, 512), w_v=_bf(64, 256, 512))
    _expect(ValueError, binding.mla_up_v, o_lat=_f32(4, 32, 512), w_v=_bf(64, 256, 512))
    _expect(ValueError, binding.mla_up_v, o_lat=_f32(4, 64, 512), w_v=_bf(64, 256, 512), out=_f32(4, 64, 512))
    # down-projection with cache append
    ap = dict(h=_bf(2, 3, 4096), w_dkv=_bf(512, 4096), cache=_bf(2, 40, 512), cache_len=_i32(2), max_cache_len=40)
    _expect(TypeError, binding.mla_latent_append, **ap)
    for b in (dict(cache=_bf(3, 40, 512)), dict(cache_len=_i32(1)), dict(max_cache_len=41),
              dict(w_dkv=_bf(512, 2048)), dict(cache=_bf(2, 40, 256))):
        _expect(ValueError, binding.mla_latent_append, **{**ap, **b})


def test_naive_and_indexer_wrappers_check_every_extent(L):
    ex = dict(cache=_bf(2, 40, 512), cache_len=_i32(2), w_k=_bf(64, 256, 512), w_v=_bf(64, 256, 512),
              max_cache_len=40)
    _expect(TypeError, binding.mla_expand_kv, **ex)
    for b in (dict(cache_len=_i32(3)), dict(w_v=_bf(64, 128, 512)), dict(max_cache_len=41),
              dict(k_out=_bf(2, 40, 64, 128)), dict(vt_out=_bf(2, 64, 256, 40))):
        _expect(ValueError, binding.mla_expand_kv, **{**ex, **b})
    na = dict(q=_bf(2, 3, 64, 256), k=_bf(2, 40, 64, 256), vt=_bf(2, 64, 256, 64), cache_len=_i32(2),
              max_cache_len=40, scale=0.0625)
    _expect(TypeError, binding.mla_naive_attn, **na)
    for b in (dict(k=_bf(2, 39, 64, 256)), dict(vt=_bf(2, 64, 256, 32)), dict(cache_len=_i32(1)),
              dict(out=_f32(2, 3, 64, 512)), dict(lse=_f32(2, 3, 32))):
        _expect(ValueError, binding.mla_naive_attn, **{**na, **b})
    kp = dict(k=_bf(2, 40, 128), g=_bf(2, 40, 128), cache_len=_i32(2), max_cache_len=40, pool=4)
    _expect(TypeError, binding.mla_kpool_keys, **kp)
    for b in (dict(g=_bf(2, 40, 64)), dict(cache_len=_i32(3)), dict(max_cache_len=41),
              dict(pooled=_f32(2, 9, 128)), dict(pool_begin=_i32(1))):
        _expect(ValueError, binding.mla_kpool_keys, **{**kp, **b})
    sc = dict(q=_bf(2, 4, 128), pooled=_f32(2, 10, 128), cache_len=_i32(2), max_cache_len=40, pool=4)
    _expect(TypeError, binding.mla_indexer_scores, **sc)
    for b in (dict(pooled=_f32(3, 10, 128)), dict(pooled=_f32(2, 10, 64)), dict(cache_len=_i32(1)),
              dict(scores=_f32(2, 4, 9))):
        _expect(ValueError, binding.mla_indexer_scores, **{**sc, **b})
    se = dict(scores=_f32(2, 4, 10), cache_len=_i32(2), max_cache_len=40, pool=4, topk=8)
    _expect(TypeError, binding.mla_indexer_select, **se)
    for b in (dict(cache_len=_i32(3)), dict(idx=_i32(2, 3, 11)), dict(idx_len=_i32(2, 3))):
        _expect(ValueError, binding.mla_indexer_select, **{**se, **b})


def test_head_counts_multiple_of_16(L):
    # H a multiple of 16: the attention kernels take heads in groups of 64, the last partial
    for H in (16, 48, 80, 112):
        s = binding.mla_latent_attn_num_splits(2, 1, H, 4096, 0)
        assert s >= 1
        assert binding.mla_latent_attn_workspace_size(2, 1, H, 512, 4096, 0) == (0 if s == 1 else s * 2 * H * 1032)
    for H in (8, 24, 40, 72):
        assert L.mla_latent_attn_num_splits(2, 1, H, 4096, 0, 0) == binding.MLA_ERR_SHAPE
        assert L.mla_latent_attn_workspace_size(2, 1, H, 512, 4096, 0, 0) == 0

"""Python binding of libmla_absorb.so: the C ABI of include/mla_absorb.h with the same names.

Argument marshalling only: tensors are torch tensors on the current HIP device (PyTorch is
used for device memory and streams); every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is missing, `lib()` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_absorb.so")

# status codes (enum mla_status)
MLA_OK = 0
MLA_ERR_NULL = -1
MLA_ERR_SHAPE = -2
MLA_ERR_ARG = -3
MLA_ERR_WORKSPACE = -4
MLA_ERR_HIP = -5
MLA_ERR_DEVICE = -6
MLA_ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 64 << 20   # MLA_NOALLOC_SCRATCH_BYTES

EXPORTS = ("mla_status_string", "mla_absorb_q", "mla_latent_attn_num_splits", "mla_latent_attn_workspace_size",
           "mla_latent_attn", "mla_latent_attn_indexed", "mla_up_v", "mla_kpool_keys", "mla_indexer_scores",
           "mla_indexer_select", "mla_latent_append", "mla_expand_kv", "mla_naive_attn",
           "mla_latent_attn_up_v_workspace_size", "mla_latent_attn_up_v", "mla_check_attn_inputs",
           "mla_latent_attn_up_v_noalloc", "mla_stream_read")


class MlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_cache_absorb_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_absorb_q.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
        L.mla_absorb_q.restype = ctypes.c_int
        L.mla_latent_attn_num_splits.argtypes = [i32, i32, i32, i32, i32, i32]
        L.mla_latent_attn_num_splits.restype = i32
        L.mla_latent_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.mla_latent_attn_workspace_size.restype = sz
        L.mla_latent_attn.argtypes = [vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, sz, vp]
        L.mla_latent_attn.restype = ctypes.c_int
        L.mla_latent_attn_indexed.argtypes = [vp, vp, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                              vp, vp, vp, sz, vp]
        L.mla_latent_attn_indexed.restype = ctypes.c_int
        L.mla_latent_attn_up_v_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.mla_latent_attn_up_v_workspace_size.restype = sz
        L.mla_latent_attn_up_v.argtypes = [vp, vp, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, vp,
                                           i32, vp, vp, vp, sz, vp]
        L.mla_latent_attn_up_v.restype = ctypes.c_int
        L.mla_latent_attn_up_v_noalloc.argtypes = [vp, vp, vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                                   i32, vp, i32, vp, vp, vp]
        L.mla_latent_attn_up_v_noalloc.restype = ctypes.c_int
        L.mla_stream_read.argtypes = [vp, sz, ctypes.c_uint32, vp, vp]
        L.mla_stream_read.restype = ctypes.c_int
        L.mla_check_attn_inputs.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
        L.mla_check_attn_inputs.restype = ctypes.c_int
        L.mla_up_v.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
        L.mla_up_v.restype = ctypes.c_int
        L.mla_kpool_keys.argtypes = [vp, vp, i64, vp, vp, i32, i32, i32, i32, vp, i32, vp]
        L.mla_kpool_keys.restype = ctypes.c_int
        L.mla_indexer_scores.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
        L.mla_indexer_scores.restype = ctypes.c_int
        L.mla_indexer_select.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, i32, vp]
        L.mla_expand_kv.restype = ctypes.c_int
        L.mla_expand_kv.argtypes = [vp, i64, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp]
        L.mla_naive_attn.restype = ctypes.c_int
        L.mla_naive_attn.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp]
        L.mla_latent_append.restype = ctypes.c_int
        L.mla_latent_append.argtypes = [vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, vp]
        L.mla_indexer_select.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MLA_OK:
        raise MlaError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# Every wrapper checks, in this order and before anything is launched: each tensor's dtype and
# layout (_need), every extent against the sizes the call is given (_shape and the wrapper's own
# checks, ValueError), then that every tensor lives on the GPU of the first one (_gpu).  The C ABI
# receives raw pointers and cannot see a tensor's extent, so a mismatch caught here would
# otherwise become an out-of-bounds device access.
def _need(t: torch.Tensor, dtype, name: str, contiguous: bool = True):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype:
        raise TypeError(f"{name} must be a {dtype} tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: Optional[torch.Tensor], want, name: str):
    if t is not None and tuple(t.shape) != tuple(int(x) for x in want):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in want)}, got {tuple(t.shape)}")


def _gpu(*tensors):
    """Every given tensor (None skipped) is on the GPU, the same one as the first."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or t.device != dev:
            raise TypeError(f"every tensor must be on the same GPU ({dev}); got one on {t.device}")


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# ----------------------------------------------------------------------------------------
def mla_absorb_q(q: torch.Tensor, w_k: torch.Tensor, q_abs: Optional[torch.Tensor] = None,
                 prescale: float = 1.0, stream=None, lo: bool = False, q_abs_lo: Optional[torch.Tensor] = None):
    """q [..., H, D] bf16, w_k [H, D, R] bf16 -> q_abs [..., H, R] bf16 = prescale * W_k^T q.
    With lo=True (or q_abs_lo given) the second bf16 term is written too and (q_abs, q_abs_lo) is
    returned."""
    _need(q, torch.bfloat16, "q")
    _need(w_k, torch.bfloat16, "w_k")
    if w_k.dim() != 3:
        raise ValueError("w_k must be [H, D, R]")
    H, D, R = w_k.shape
    if q.dim() < 2 or tuple(q.shape[-2:]) != (H, D):
        raise ValueError("q must end in [H, D]")
    rows = q.numel() // (H * D)
    lo = lo or q_abs_lo is not None
    for t, nm in ((q_abs, "q_abs"), (q_abs_lo, "q_abs_lo")):
        if t is not None:
            _need(t, torch.bfloat16, nm)
            _shape(t, tuple(q.shape[:-1]) + (R,), nm)
    _gpu(q, w_k, q_abs, q_abs_lo)
    if q_abs is None:
        q_abs = torch.empty(q.shape[:-1] + (R,), dtype=torch.bfloat16, device=q.device)
    if lo and q_abs_lo is None:
        q_abs_lo = torch.empty(q.shape[:-1] + (R,), dtype=torch.bfloat16, device=q.device)
    _check(lib().mla_absorb_q(_ptr(q), _ptr(w_k), _ptr(q_abs), _ptr(q_abs_lo), rows, H, D, R, float(prescale),
                              _stream(stream)), "mla_absorb_q")
    return (q_abs, q_abs_lo) if lo else q_abs


def mla_latent_attn_num_splits(B: int, Q: int, H: int, max_positions: int, num_splits: int = 0,
                               indexed: bool = False) -> int:
    s = lib().mla_latent_attn_num_splits(B, Q, H, max_positions, num_splits, int(bool(indexed)))
    _check(min(int(s), 0), "mla_latent_attn_num_splits")
    return int(s)


def mla_latent_attn_workspace_size(B: int, Q: int, H: int, R: int, max_positions: int, num_splits: int = 0,
                                   indexed: bool = False) -> int:
    return int(lib().mla_latent_attn_workspace_size(B, Q, H, R, max_positions, num_splits, int(bool(indexed))))


def _cache_stride(cache: torch.Tensor) -> int:
    if cache.dim() != 3 or cache.stride(2) != 1 or cache.stride(1) != cache.shape[2]:
        raise ValueError("cache must be [B, L, R] with contiguous rows")
    return int(cache.stride(0))


def _attn_inputs(q_abs, cache, cache_len, max_cache_len, idx=None, idx_len=None, q_abs_lo=None):
    """dtype and extent checks shared by the attention calls; returns (B, Q, H, R, K_max)."""
    _need(q_abs, torch.bfloat16, "q_abs")
    if q_abs_lo is not None:
        _need(q_abs_lo, torch.bfloat16, "q_abs_lo")
        _shape(q_abs_lo, tuple(q_abs.shape), "q_abs_lo")
    _need(cache, torch.bfloat16, "cache", contiguous=False)
    _need(cache_len, torch.int32, "cache_len")
    if q_abs.dim() != 4:
        raise ValueError("q_abs must be [B, Q, H, R]")
    B, Q, H, R = q_abs.shape
    _cache_stride(cache)
    if cache.shape[0] != B or cache.shape[2] != R:
        raise ValueError(f"cache must be [B={B}, L, R={R}], got {tuple(cache.shape)}")
    if int(max_cache_len) < 1 or cache.shape[1] < int(max_cache_len):
        raise ValueError(f"max_cache_len ({max_cache_len}) must be in [1, cache.shape[1] = {cache.shape[1]}]")
    _shape(cache_len, (B,), "cache_len")
    K_max = 0
    if (idx is None) != (idx_len is None):
        raise ValueError("idx and idx_len go together")
    if idx is not None:
        _need(idx, torch.int32, "idx")
        _need(idx_len, torch.int32, "idx_len")
        if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, Q) or idx.shape[2] < 1:
            raise ValueError(f"idx must be [B={B}, Q={Q}, K_max >= 1], got {tuple(idx.shape)}")
        K_max = int(idx.shape[2])
        _shape(idx_len, (B, Q), "idx_len")
    return B, Q, H, R, K_max


def _attn_outputs(q_abs, o_lat, lse, want_lse):
    B, Q, H, R = q_abs.shape
    if o_lat is not None:
        _need(o_lat, torch.float32, "o_lat")
        _shape(o_lat, (B, Q, H, R), "o_lat")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        _shape(lse, (B, Q, H), "lse")
    return o_lat, lse


def _alloc_outputs(q_abs, o_lat, lse, want_lse):
    B, Q, H, R = q_abs.shape
    if o_lat is None:
        o_lat = torch.empty((B, Q, H, R), dtype=torch.float32, device=q_abs.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q_abs.device)
    return o_lat, lse


def _workspace_arg(workspace):
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor")
    return workspace


def _workspace(workspace, need, device):
    if need == 0:
        return workspace
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace


BAD_INPUT_BITS = {1: "cache_len < Q", 2: "cache_len > max_cache_len", 4: "idx_len outside [1, K_max]",
                  8: "a listed position outside the cache", 16: "listed positions not strictly ascending",
                  32: "a listed position past the query's own"}


def mla_check_attn_inputs(cache_len: torch.Tensor, Q: int, max_cache_len: int, idx: Optional[torch.Tensor] = None,
                          idx_len: Optional[torch.Tensor] = None, stream=None) -> int:
    """Check the attention calls' device-side preconditions on the GPU; returns the flag word
    (0 = all hold; else an OR of the keys of BAD_INPUT_BITS).  Synchronises the stream."""
    _need(cache_len, torch.int32, "cache_len")
    if cache_len.dim() != 1:
        raise ValueError("cache_len must be [B]")
    B = cache_len.numel()
    K_max = 0
    if (idx is None) != (idx_len is None):
        raise ValueError("idx and idx_len go together")
    if idx is not None:
        _need(idx, torch.int32, "idx")
        _need(idx_len, torch.int32, "idx_len")
        if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, int(Q)) or idx.shape[2] < 1:
            raise ValueError(f"idx must be [B={B}, Q={Q}, K_max >= 1], got {tuple(idx.shape)}")
        _shape(idx_len, (B, Q), "idx_len")
        K_max = idx.shape[-1]
    _gpu(cache_len, idx, idx_len)
    flags = torch.empty(1, dtype=torch.int32, device=cache_len.device)
    _check(lib().mla_check_attn_inputs(_ptr(cache_len), _ptr(idx), _ptr(idx_len), B, int(Q), K_max,
                                       int(max_cache_len), _ptr(flags), _stream(stream)), "mla_check_attn_inputs")
    (torch.cuda.current_stream() if stream is None else stream).synchronize()
    return int(flags.item())


def _debug_check(cache_len, Q, max_cache_len, idx=None, idx_len=None, stream=None):
    """With MLA_CHECK_INPUTS=1 in the environment, every attention call first checks its
    device-side preconditions and raises MlaError(MLA_ERR_ARG) naming the ones that fail."""
    if os.environ.get("MLA_CHECK_INPUTS", "0") in ("", "0"):
        return
    f = mla_check_attn_inputs(cache_len, Q, max_cache_len, idx, idx_len, stream)
    if f:
        what = ", ".join(v for k, v in BAD_INPUT_BITS.items() if f & k)
        raise MlaError(MLA_ERR_ARG, f"device-side preconditions fail ({what})")


def mla_latent_attn(q_abs: torch.Tensor, cache: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int,
                    scale: float, num_splits: int = 0, o_lat=None, lse=None, workspace=None, want_lse=True,
                    stream=None, q_abs_lo=None):
    """Dense latent attention.  q_abs [B, Q, H, R] bf16 (and optionally its second term q_abs_lo);
    cache [B, L_max, R] bf16 (a view with any batch stride); cache_len [B] int32 on the GPU.
    Returns (o_lat [B, Q, H, R] fp32, lse [B, Q, H])."""
    B, Q, H, R, _ = _attn_inputs(q_abs, cache, cache_len, max_cache_len, q_abs_lo=q_abs_lo)
    o_lat, lse = _attn_outputs(q_abs, o_lat, lse, want_lse)
    _gpu(q_abs, q_abs_lo, cache, cache_len, o_lat, lse, _workspace_arg(workspace))
    o_lat, lse = _alloc_outputs(q_abs, o_lat, lse, want_lse)
    _debug_check(cache_len, Q, max_cache_len, stream=stream)
    need = mla_latent_attn_workspace_size(B, Q, H, R, max_cache_len, num_splits)
    workspace = _workspace(workspace, need, q_abs.device)
    _check(lib().mla_latent_attn(_ptr(q_abs), _ptr(q_abs_lo), _ptr(cache), _cache_stride(cache), _ptr(cache_len), B, Q, H, R,
                                 int(max_cache_len), float(scale), int(num_splits), _ptr(o_lat), _ptr(lse),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "mla_latent_attn")
    return o_lat, lse


def mla_latent_attn_indexed(q_abs: torch.Tensor, cache: torch.Tensor, cache_len: torch.Tensor, idx: torch.Tensor,
                            idx_len: torch.Tensor, max_cache_len: int, scale: float, num_splits: int = 0,
                            o_lat=None, lse=None, workspace=None, want_lse=True, stream=None, q_abs_lo=None):
    """Indexed latent attention: idx [B, Q, K_max] int32 (sorted positions), idx_len [B, Q] int32."""
    if idx is None or idx_len is None:
        raise ValueError("the indexed call needs idx and idx_len")
    B, Q, H, R, K_max = _attn_inputs(q_abs, cache, cache_len, max_cache_len, idx, idx_len, q_abs_lo)
    o_lat, lse = _attn_outputs(q_abs, o_lat, lse, want_lse)
    _gpu(q_abs, q_abs_lo, cache, cache_len, idx, idx_len, o_lat, lse, _workspace_arg(workspace))
    o_lat, lse = _alloc_outputs(q_abs, o_lat, lse, want_lse)
    _debug_check(cache_len, Q, max_cache_len, idx, idx_len, stream=stream)
    need = mla_latent_attn_workspace_size(B, Q, H, R, K_max, num_splits, indexed=True)
    workspace = _workspace(workspace, need, q_abs.device)
    _check(lib().mla_latent_attn_indexed(_ptr(q_abs), _ptr(q_abs_lo), _ptr(cache), _cache_stride(cache), _ptr(cache_len), _ptr(idx),
                                         _ptr(idx_len), K_max, B, Q, H, R, int(max_cache_len), float(scale),
                                         int(num_splits), _ptr(o_lat), _ptr(lse), _ptr(workspace),
                                         _nbytes(workspace), _stream(stream)),
           "mla_latent_attn_indexed")
    return o_lat, lse


def mla_up_v(o_lat: torch.Tensor, w_v: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """o_lat [..., H, R] fp32, w_v [H, D, R] bf16 -> out [..., H, D] fp32 = W_v o_lat."""
    _need(o_lat, torch.float32, "o_lat")
    _need(w_v, torch.bfloat16, "w_v")
    if w_v.dim() != 3:
        raise ValueError("w_v must be [H, D, R]")
    H, D, R = w_v.shape
    if o_lat.dim() < 2 or tuple(o_lat.shape[-2:]) != (H, R):
        raise ValueError("o_lat must end in [H, R]")
    rows = o_lat.numel() // (H * R)
    if out is not None:
        _need(out, torch.float32, "out")
        _shape(out, tuple(o_lat.shape[:-1]) + (D,), "out")
    _gpu(o_lat, w_v, out)
    if out is None:
        out = torch.empty(o_lat.shape[:-1] + (D,), dtype=torch.float32, device=o_lat.device)
    _check(lib().mla_up_v(_ptr(o_lat), _ptr(w_v), _ptr(out), rows, H, D, R, _stream(stream)), "mla_up_v")
    return out


def mla_latent_attn_up_v_workspace_size(B: int, Q: int, H: int, R: int, max_positions: int, num_splits: int = 0,
                                        indexed: bool = False) -> int:
    return int(lib().mla_latent_attn_up_v_workspace_size(B, Q, H, R, max_positions, num_splits, int(bool(indexed))))


def mla_latent_attn_up_v(q_abs: torch.Tensor, cache: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int,
                         scale: float, w_v: torch.Tensor, idx: Optional[torch.Tensor] = None,
                         idx_len: Optional[torch.Tensor] = None, num_splits: int = 0, out=None, lse=None,
                         workspace=None, want_lse=True, stream=None, q_abs_lo=None):
    """Latent attention (dense, or indexed when idx / idx_len are given) followed by the value
    up-projection, the split merge fused into the latter.  Returns (out [B, Q, H, D] fp32,
    lse [B, Q, H] fp32)."""
    B, Q, H, R, K_max = _attn_inputs(q_abs, cache, cache_len, max_cache_len, idx, idx_len, q_abs_lo)
    _need(w_v, torch.bfloat16, "w_v")
    if w_v.dim() != 3 or w_v.shape[0] != H or w_v.shape[2] != R:
        raise ValueError(f"w_v must be [H={H}, D, R={R}], got {tuple(w_v.shape)}")
    D = w_v.shape[1]
    indexed = idx is not None
    if out is not None:
        _need(out, torch.float32, "out")
        _shape(out, (B, Q, H, D), "out")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        _shape(lse, (B, Q, H), "lse")
    _gpu(q_abs, q_abs_lo, cache, cache_len, w_v, idx, idx_len, out, lse, _workspace_arg(workspace))
    if out is None:
        out = torch.empty((B, Q, H, D), dtype=torch.float32, device=q_abs.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q_abs.device)
    _debug_check(cache_len, Q, max_cache_len, idx, idx_len, stream=stream)
    need = mla_latent_attn_up_v_workspace_size(B, Q, H, R, K_max if indexed else max_cache_len, num_splits, indexed)
    workspace = _workspace(workspace, need, q_abs.device)
    _check(lib().mla_latent_attn_up_v(_ptr(q_abs), _ptr(q_abs_lo), _ptr(cache), _cache_stride(cache), _ptr(cache_len), _ptr(idx),
                                      _ptr(idx_len), K_max, B, Q, H, R, int(max_cache_len), float(scale),
                                      int(num_splits), _ptr(w_v), D, _ptr(out), _ptr(lse), _ptr(workspace),
                                      _nbytes(workspace), _stream(stream)),
           "mla_latent_attn_up_v")
    return out, lse


def mla_latent_attn_up_v_noalloc(q_abs: torch.Tensor, cache: torch.Tensor, cache_len: torch.Tensor,
                                 max_cache_len: int, scale: float, w_v: torch.Tensor, out: torch.Tensor,
                                 lse: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                                 idx_len: Optional[torch.Tensor] = None, num_splits: int = 0, stream=None,
                                 q_abs_lo: Optional[torch.Tensor] = None):
    """mla_latent_attn_up_v with the split partials in the library's fixed device scratch: neither
    the library nor this wrapper allocates (the caller passes out, and lse or None).  Calls that
    overlap on one GPU race on that scratch.  Returns (out, lse)."""
    B, Q, H, R, K_max = _attn_inputs(q_abs, cache, cache_len, max_cache_len, idx, idx_len, q_abs_lo)
    _need(w_v, torch.bfloat16, "w_v")
    if w_v.dim() != 3 or w_v.shape[0] != H or w_v.shape[2] != R:
        raise ValueError(f"w_v must be [H={H}, D, R={R}], got {tuple(w_v.shape)}")
    D = w_v.shape[1]
    if out is None:
        raise ValueError("out must be given: this call allocates nothing")
    _need(out, torch.float32, "out")
    _shape(out, (B, Q, H, D), "out")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        _shape(lse, (B, Q, H), "lse")
    _gpu(q_abs, q_abs_lo, cache, cache_len, w_v, idx, idx_len, out, lse)
    _check(lib().mla_latent_attn_up_v_noalloc(_ptr(q_abs), _ptr(q_abs_lo), _ptr(cache), _cache_stride(cache), _ptr(cache_len),
                                              _ptr(idx), _ptr(idx_len), K_max, B, Q, H, R, int(max_cache_len),
                                              float(scale), int(num_splits), _ptr(w_v), D, _ptr(out), _ptr(lse),
                                              _stream(stream)), "mla_latent_attn_up_v_noalloc")
    return out, lse


def mla_stream_read(src: torch.Tensor, sink: torch.Tensor, never: int = 0x7BADF00D, stream=None) -> None:
    """Measurement helper: read every byte of src (contiguous, a multiple of 32 KiB) once as a plain
    streaming read; sink is one int32 on the same GPU, practically never written."""
    if not isinstance(src, torch.Tensor) or not src.is_contiguous():
        raise ValueError("src must be a contiguous tensor")
    if not isinstance(sink, torch.Tensor) or sink.dtype != torch.int32 or sink.numel() < 1:
        raise TypeError("sink must be an int32 tensor")
    nbytes = _nbytes(src)
    if nbytes < 32768 or nbytes % 32768:
        raise ValueError("src must hold a positive multiple of 32 KiB")
    _gpu(src, sink)
    _check(lib().mla_stream_read(_ptr(src), nbytes, int(never) & 0xFFFFFFFF, _ptr(sink), _stream(stream)),
           "mla_stream_read")


# ------------------------------------------------------------------ down-projection and append
def mla_latent_append(h: torch.Tensor, w_dkv: torch.Tensor, cache: torch.Tensor, cache_len: torch.Tensor,
                      max_cache_len: int, stream=None) -> torch.Tensor:
    """h [B, Q, hidden] bf16, w_dkv [R, hidden] bf16: writes bf16(W h) of token i of sequence b
    into cache[b, cache_len[b] - Q + i] (cache_len: lengths after the pass).  Returns cache."""
    _need(h, torch.bfloat16, "h")
    _need(w_dkv, torch.bfloat16, "w_dkv")
    _need(cache_len, torch.int32, "cache_len")
    _need(cache, torch.bfloat16, "cache", contiguous=False)
    if h.dim() != 3 or w_dkv.dim() != 2:
        raise ValueError("h must be [B, Q, hidden] and w_dkv [R, hidden]")
    B, Q, hidden = h.shape
    R = w_dkv.shape[0]
    _cache_stride(cache)
    if w_dkv.shape != (R, hidden) or cache.shape[0] != B or cache.shape[2] != R:
        raise ValueError("shape mismatch between h, w_dkv and cache")
    if int(max_cache_len) < 1 or cache.shape[1] < int(max_cache_len):
        raise ValueError(f"max_cache_len ({max_cache_len}) must be in [1, cache.shape[1] = {cache.shape[1]}]")
    _shape(cache_len, (B,), "cache_len")
    _gpu(h, w_dkv, cache, cache_len)
    _check(lib().mla_latent_append(_ptr(h), _ptr(w_dkv), _ptr(cache), _cache_stride(cache), _ptr(cache_len), B, Q,
                                   hidden, R, int(max_cache_len), _stream(stream)), "mla_latent_append")
    return cache


# ------------------------------------------------------------------------------ the naive form
def vt_length(max_cache_len: int) -> int:
    """Positions per row of the transposed value buffer: max_cache_len rounded up to 64."""
    return (int(max_cache_len) + 63) // 64 * 64


def mla_expand_kv(cache: torch.Tensor, cache_len: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                  max_cache_len: int, k_out: Optional[torch.Tensor] = None, vt_out: Optional[torch.Tensor] = None,
                  stream=None):
    """The naive form's expansion.  cache [B, L, R] bf16, w_k / w_v [H, D, R] bf16 ->
    (k [B, max_cache_len, H, D] bf16, vt [B, H, D, vt_len] bf16, values transposed)."""
    _need(cache, torch.bfloat16, "cache", contiguous=False)
    _need(cache_len, torch.int32, "cache_len")
    _need(w_k, torch.bfloat16, "w_k")
    _need(w_v, torch.bfloat16, "w_v")
    if w_k.dim() != 3 or w_v.shape != w_k.shape:
        raise ValueError("w_k and w_v must both be [H, D, R]")
    H, D, R = w_k.shape
    _cache_stride(cache)
    B = cache.shape[0]
    L = int(max_cache_len)
    if cache.shape[2] != R or L < 1 or cache.shape[1] < L:
        raise ValueError(f"cache must be [B, L >= max_cache_len, R={R}], got {tuple(cache.shape)}")
    _shape(cache_len, (B,), "cache_len")
    vt_len = vt_length(L)
    for t, name in ((k_out, "k_out"), (vt_out, "vt_out")):
        if t is not None:
            _need(t, torch.bfloat16, name)
    _shape(k_out, (B, L, H, D), "k_out")
    _shape(vt_out, (B, H, D, vt_len), "vt_out")
    _gpu(cache, cache_len, w_k, w_v, k_out, vt_out)
    if k_out is None:
        k_out = torch.empty((B, L, H, D), dtype=torch.bfloat16, device=cache.device)
    if vt_out is None:
        vt_out = torch.empty((B, H, D, vt_len), dtype=torch.bfloat16, device=cache.device)
    _check(lib().mla_expand_kv(_ptr(cache), _cache_stride(cache), _ptr(cache_len), _ptr(w_k), _ptr(w_v), B, H, D, R,
                               L, _ptr(k_out), _ptr(vt_out), vt_len, _stream(stream)), "mla_expand_kv")
    return k_out, vt_out


def mla_naive_attn(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int,
                   scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   want_lse: bool = True, stream=None):
    """Causal multi-head attention on expanded keys and values.  q [B, Q, H, D] bf16; k, vt from
    mla_expand_kv.  Returns (out [B, Q, H, D] fp32, lse [B, Q, H] fp32 or None)."""
    _need(q, torch.bfloat16, "q")
    _need(k, torch.bfloat16, "k")
    _need(vt, torch.bfloat16, "vt")
    _need(cache_len, torch.int32, "cache_len")
    if q.dim() != 4:
        raise ValueError("q must be [B, Q, H, D]")
    B, Q, H, D = q.shape
    _shape(k, (B, int(max_cache_len), H, D), "k")
    if vt.dim() != 4 or tuple(vt.shape[:3]) != (B, H, D) or vt.shape[3] < int(max_cache_len):
        raise ValueError(f"vt must be [B={B}, H={H}, D={D}, >= max_cache_len], got {tuple(vt.shape)}")
    _shape(cache_len, (B,), "cache_len")
    if out is not None:
        _need(out, torch.float32, "out")
        _shape(out, (B, Q, H, D), "out")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        _shape(lse, (B, Q, H), "lse")
    _gpu(q, k, vt, cache_len, out, lse)
    if out is None:
        out = torch.empty((B, Q, H, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device)
    _check(lib().mla_naive_attn(_ptr(q), _ptr(k), _ptr(vt), vt.shape[3], _ptr(cache_len), B, Q, H, D,
                                int(max_cache_len), float(scale), _ptr(out), _ptr(lse), _stream(stream)),
           "mla_naive_attn")
    return out, lse


def mla_naive_forward(q, w_k, w_v, cache, cache_len, max_cache_len, scale, stream=None):
    """The whole naive path: expand keys and values, then attention.  Returns (out, lse)."""
    k, vt = mla_expand_kv(cache, cache_len, w_k, w_v, max_cache_len, stream=stream)
    return mla_naive_attn(q, k, vt, cache_len, max_cache_len, scale, stream=stream)


# ---------------------------------------------------------------------------- k-pooled indexer
def _rows(t: torch.Tensor, name: str):
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [B, L, d] with contiguous rows")
    return int(t.stride(0))


def mla_kpool_keys(k: torch.Tensor, g: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int, pool: int,
                   pooled: Optional[torch.Tensor] = None, max_pools: Optional[int] = None, pool_begin=None,
                   stream=None) -> torch.Tensor:
    """k, g [B, L, d] bf16 (indexer keys, gate logits) -> pooled [B, max_pools, d] fp32."""
    _need(k, torch.bfloat16, "k", contiguous=False)
    _need(g, torch.bfloat16, "g", contiguous=False)
    _need(cache_len, torch.int32, "cache_len")
    stride = _rows(k, "k")
    B, Lk, d = k.shape
    if _rows(g, "g") != stride or g.shape != k.shape:
        raise ValueError("g must have the layout of k")
    if int(max_cache_len) < 1 or Lk < int(max_cache_len):
        raise ValueError(f"max_cache_len ({max_cache_len}) must be in [1, k.shape[1] = {Lk}]")
    _shape(cache_len, (B,), "cache_len")
    if max_pools is None:
        max_pools = max(1, max_cache_len // pool)
    if pooled is not None:
        _need(pooled, torch.float32, "pooled")
        _shape(pooled, (B, max_pools, d), "pooled")
    if pool_begin is not None:
        _need(pool_begin, torch.int32, "pool_begin")
        _shape(pool_begin, (B,), "pool_begin")
    _gpu(k, g, cache_len, pooled, pool_begin)
    if pooled is None:
        pooled = torch.empty((B, max_pools, d), dtype=torch.float32, device=k.device)
    _check(lib().mla_kpool_keys(_ptr(k), _ptr(g), stride, _ptr(cache_len), _ptr(pool_begin), B, int(max_cache_len),
                                d, int(pool), _ptr(pooled), int(max_pools), _stream(stream)), "mla_kpool_keys")
    return pooled


def mla_indexer_scores(q: torch.Tensor, pooled: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int,
                       pool: int, scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q [B, Q, d] bf16, pooled [B, max_pools, d] fp32 -> scores [B, Q, max_pools] fp32."""
    _need(q, torch.bfloat16, "q")
    _need(pooled, torch.float32, "pooled")
    _need(cache_len, torch.int32, "cache_len")
    if q.dim() != 3 or pooled.dim() != 3:
        raise ValueError("q must be [B, Q, d] and pooled [B, max_pools, d]")
    B, Q, d = q.shape
    max_pools = pooled.shape[1]
    if pooled.shape[0] != B or pooled.shape[2] != d:
        raise ValueError(f"pooled must be [B={B}, max_pools, d={d}], got {tuple(pooled.shape)}")
    _shape(cache_len, (B,), "cache_len")
    if scores is not None:
        _need(scores, torch.float32, "scores")
        _shape(scores, (B, Q, max_pools), "scores")
    _gpu(q, pooled, cache_len, scores)
    if scores is None:
        scores = torch.empty((B, Q, max_pools), dtype=torch.float32, device=q.device)
    _check(lib().mla_indexer_scores(_ptr(q), _ptr(pooled), _ptr(cache_len), B, Q, d, int(pool), max_pools,
                                    int(max_cache_len), _ptr(scores), _stream(stream)), "mla_indexer_scores")
    return scores


def mla_indexer_select(scores: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int, pool: int, topk: int,
                       tail: bool = True, idx: Optional[torch.Tensor] = None, idx_len: Optional[torch.Tensor] = None,
                       stream=None):
    """scores [B, Q, max_pools] fp32 -> (idx [B, Q, topk + pool - 1] int32, idx_len [B, Q] int32)."""
    _need(scores, torch.float32, "scores")
    _need(cache_len, torch.int32, "cache_len")
    if scores.dim() != 3:
        raise ValueError("scores must be [B, Q, max_pools]")
    B, Q, max_pools = scores.shape
    _shape(cache_len, (B,), "cache_len")
    K_max = topk + (pool - 1 if tail else 0)
    if idx is not None:
        _need(idx, torch.int32, "idx")
        if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, Q):
            raise ValueError(f"idx must be [B={B}, Q={Q}, K_max], got {tuple(idx.shape)}")
    if idx_len is not None:
        _need(idx_len, torch.int32, "idx_len")
        _shape(idx_len, (B, Q), "idx_len")
    _gpu(scores, cache_len, idx, idx_len)
    if idx is None:
        idx = torch.empty((B, Q, K_max), dtype=torch.int32, device=scores.device)
    if idx_len is None:
        idx_len = torch.empty((B, Q), dtype=torch.int32, device=scores.device)
    _check(lib().mla_indexer_select(_ptr(scores), _ptr(cache_len), B, Q, int(pool), max_pools, int(max_cache_len),
                                    int(topk), int(bool(tail)), _ptr(idx), _ptr(idx_len), idx.shape[2],
                                    _stream(stream)), "mla_indexer_select")
    return idx, idx_len


def mla_indexer(q: torch.Tensor, k: torch.Tensor, g: torch.Tensor, cache_len: torch.Tensor, max_cache_len: int,
                pool: int, topk: int, tail: bool = True, stream=None):
    """The three indexer steps: pooled keys -> pool scores -> position lists (idx, idx_len)."""
    pooled = mla_kpool_keys(k, g, cache_len, max_cache_len, pool, stream=stream)
    scores = mla_indexer_scores(q, pooled, cache_len, max_cache_len, pool, stream=stream)
    return mla_indexer_select(scores, cache_len, max_cache_len, pool, topk, tail, stream=stream)


def mla_forward(q, w_k, w_v, cache, cache_len, max_cache_len, scale, idx=None, idx_len=None, num_splits=0,
                stream=None, two_term=False):
    """The whole absorbed path: absorb_q -> latent attention (dense or indexed) with the
    up-projection fused into the split merge (mla_latent_attn_up_v); two_term carries the
    absorbed query as two bf16 terms into the scores.
    Returns (out [B, Q, H, D] fp32, lse [B, Q, H] fp32)."""
    if two_term:
        q_abs, q_abs_lo = mla_absorb_q(q, w_k, stream=stream, lo=True)
    else:
        q_abs, q_abs_lo = mla_absorb_q(q, w_k, stream=stream), None
    return mla_latent_attn_up_v(q_abs, cache, cache_len, max_cache_len, scale, w_v, idx, idx_len, num_splits,
                                stream=stream, q_abs_lo=q_abs_lo)

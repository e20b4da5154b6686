"""Thin ctypes binding of libne_rope_attn.so (include/ne_rope_attn.h).

Argument marshalling only: torch supplies device memory and the current HIP stream; every
step of the computation runs in the library's kernels.  There is no fallback: if the HIP
library is missing or the tensors are not on a GPU, the calls raise.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libne_rope_attn.so")

NE_F32, NE_BF16, NE_F16 = 0, 1, 2
_DT = {torch.float32: NE_F32, torch.bfloat16: NE_BF16, torch.float16: NE_F16}
STATUS = {0: "NE_OK", 1: "NE_ERR_NULL", 2: "NE_ERR_SHAPE", 3: "NE_ERR_UNSUPPORTED",
          4: "NE_ERR_ALIGN", 5: "NE_ERR_WORKSPACE", 6: "NE_ERR_NO_ROPE_TABLE", 7: "NE_ERR_HIP"}
NE_FLAG_NONDETERMINISTIC = 0x1
NE_FLAG_BF16_OPERANDS = 0x2
NE_FLAG_ROPE_HALF_SPLIT = 0x4
NE_FLAG_STORE_DS = 0x8

# Every symbol include/ne_rope_attn.h declares.
EXPORTS = ("ne_rope_attn_workspace_bytes", "ne_rope_table_init", "ne_rope_table_check",
           "ne_rope_attn_fwd", "ne_rope_attn_bwd", "ne_rope_attn_fwd_ex", "ne_rope_attn_bwd_ex",
           "ne_kv_cache_bytes", "ne_kv_cache_append", "ne_rope_attn_decode_workspace_bytes",
           "ne_rope_attn_decode", "ne_rope_attn_decode_noalloc", "ne_qkv_rope_workspace_bytes", "ne_qkv_rope_proj",
           "ne_status_str", "ne_last_error", "ne_abi_version")


class AttnOpts(ctypes.Structure):
    """ne_attn_opts_t: window (<= 0: causal prefix), QK norm (on, gain, eps)."""
    _fields_ = [("window", ctypes.c_int), ("qk_norm", ctypes.c_int), ("qk_gain", ctypes.c_float),
                ("qk_eps", ctypes.c_float), ("rope_half_split", ctypes.c_int)]


def make_opts(window=0, qk_norm=None, rope_half_split=False):
    """qk_norm: None or (gain, eps); rope_half_split: RoPE pairs (i, i + D/2)."""
    if qk_norm is None:
        return AttnOpts(int(window), 0, 1.0, 0.0, int(bool(rope_half_split)))
    gain, eps = qk_norm
    return AttnOpts(int(window), 1, float(gain), float(eps), int(bool(rope_half_split)))


class NeError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library with ctypes signatures (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m causal_gqa_flashattention_rope_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz, d, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_double, ctypes.c_uint
    op = ctypes.POINTER(AttnOpts)
    evp = ctypes.POINTER(vp)
    L.ne_rope_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, d, i, u]
    L.ne_rope_attn_workspace_bytes.restype = sz
    L.ne_rope_table_init.argtypes = [vp, sz, i, i, d, vp]
    L.ne_rope_table_init.restype = i
    L.ne_rope_table_check.argtypes = [vp, sz, i, i, d, vp]
    L.ne_rope_table_check.restype = i
    L.ne_rope_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, d, i, i, u, vp, sz, vp]
    L.ne_rope_attn_fwd.restype = i
    L.ne_rope_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, d, i, i, u, vp, sz, vp]
    L.ne_rope_attn_bwd.restype = i
    L.ne_rope_attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, d, op, i, i, u, vp, sz, vp, evp]
    L.ne_rope_attn_fwd_ex.restype = i
    L.ne_rope_attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, d, op, i, i, u, vp, sz, vp, evp]
    L.ne_rope_attn_bwd_ex.restype = i
    L.ne_kv_cache_bytes.argtypes = [i, i, i, i, i]
    L.ne_kv_cache_bytes.restype = sz
    L.ne_kv_cache_append.argtypes = [vp, sz, vp, vp, vp, i, i, i, i, i, d, op, i, vp]
    L.ne_kv_cache_append.restype = i
    L.ne_rope_attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.ne_rope_attn_decode_workspace_bytes.restype = sz
    L.ne_rope_attn_decode.argtypes = [vp, vp, sz, vp, vp, vp, i, i, i, i, i, i, d, op, i, i, vp, sz, vp, evp]
    L.ne_rope_attn_decode.restype = i
    L.ne_rope_attn_decode_noalloc.argtypes = [vp, vp, sz, vp, vp, vp, i, i, i, i, i, i, d, op, i, i, vp]
    L.ne_rope_attn_decode_noalloc.restype = i
    L.ne_qkv_rope_workspace_bytes.argtypes = [i, i]
    L.ne_qkv_rope_workspace_bytes.restype = sz
    L.ne_qkv_rope_proj.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, d, op, i, i, vp, sz, vp, evp]
    L.ne_qkv_rope_proj.restype = i
    L.ne_status_str.argtypes = [i]
    L.ne_status_str.restype = ctypes.c_char_p
    L.ne_last_error.argtypes = []
    L.ne_last_error.restype = ctypes.c_char_p
    L.ne_abi_version.argtypes = []
    L.ne_abi_version.restype = i
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise NeError(status, lib().ne_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k must be [B, T, H, D]")
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    return B, T, Hq, Hkv, D


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise RuntimeError("ne_rope_attn runs on the GPU only: tensors must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, T, H, D]")


def _nbytes(t):
    return t.numel() * t.element_size()


def workspace_bytes(is_bwd, B, T, Hq, Hkv, D, rope_base, in_dtype, flags=0):
    return int(lib().ne_rope_attn_workspace_bytes(int(bool(is_bwd)), B, T, Hq, Hkv, D, float(rope_base),
                                                  _DT[in_dtype], int(flags)))


def alloc_workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def ne_rope_table_init(workspace, T, D, rope_base):
    """Build the RoPE table of T positions in the workspace (once per workspace and arguments)."""
    _require_gpu(workspace)
    _check(lib().ne_rope_table_init(_ptr(workspace), _nbytes(workspace), T, D, float(rope_base), _stream()))
    return workspace


def ne_rope_table_check(workspace, T, D, rope_base):
    """The status of the workspace's table for (T, D, rope_base): 0 (NE_OK) or 6 (NE_ERR_NO_ROPE_TABLE).
    Synchronises the current stream."""
    _require_gpu(workspace)
    return int(lib().ne_rope_table_check(_ptr(workspace), _nbytes(workspace), T, D, float(rope_base), _stream()))


def new_workspace(is_bwd, q, k, rope_base, flags=0):
    """A workspace for these tensors with its RoPE table built."""
    B, T, Hq, Hkv, D = _dims(q, k)
    ws = alloc_workspace(workspace_bytes(is_bwd, B, T, Hq, Hkv, D, rope_base, q.dtype, flags), q.device)
    return ne_rope_table_init(ws, T, D, rope_base)


def _events_arg(events, n):
    """List of torch.cuda.Event or raw hipEvent_t handles (int) -> void*[n] (None -> untimed call;
    a None entry -> that record is skipped)."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"need {n} events")
    handles = []
    for e in events:
        if e is None or isinstance(e, int):
            handles.append(e)
            continue
        if e.cuda_event == 0:   # torch creates the HIP event lazily on first record
            e.record()
        handles.append(e.cuda_event)
    return (ctypes.c_void_p * n)(*handles)


def ne_rope_attn_fwd(q, k, v, rope_base, out_dtype=torch.float32, o=None, lse=None, workspace=None, flags=0,
                     window=0, qk_norm=None, events=None):
    """o, lse = attention forward.  q [B,T,Hq,D], k/v [B,T,Hkv,D] of one dtype.

    workspace: None (a new one, its table built here) or one whose table ne_rope_table_init built.
    window / qk_norm / events select ne_rope_attn_fwd_ex (events: 4 torch.cuda.Event or None)."""
    _require_gpu(q, k, v)
    B, T, Hq, Hkv, D = _dims(q, k)
    if o is None:
        o = torch.empty((B, T, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(False, q, k, rope_base, flags)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D, float(rope_base))
    tail = (_DT[q.dtype], _DT[o.dtype], int(flags), _ptr(workspace), _nbytes(workspace), _stream())
    if window or qk_norm is not None or events is not None:
        opts = make_opts(window, qk_norm)
        _check(lib().ne_rope_attn_fwd_ex(*head, ctypes.byref(opts), *tail, _events_arg(events, 4)))
    else:
        _check(lib().ne_rope_attn_fwd(*head, *tail))
    return o, lse


def ne_rope_attn_fwd_ex(q, k, v, rope_base, window=0, qk_norm=None, **kw):
    """Forward with every option: window (<= 0: causal prefix), qk_norm None or (gain, eps)."""
    return ne_rope_attn_fwd(q, k, v, rope_base, window=window, qk_norm=qk_norm, **kw)


def ne_rope_attn_bwd(q, k, v, o, lse, dO, rope_base, dq=None, dk=None, dv=None, workspace=None, flags=0,
                     window=0, qk_norm=None, events=None):
    """dq, dk, dv = attention backward (out dtype = o's dtype); window / qk_norm must be the forward's.

    workspace: None (a new one sized for `flags`, its table built here) or one sized with the same flags
    whose table ne_rope_table_init built.  events: 6 torch.cuda.Event or None."""
    _require_gpu(q, k, v, o, lse, dO)
    B, T, Hq, Hkv, D = _dims(q, k)
    if dq is None:
        dq = torch.empty((B, T, Hq, D), dtype=o.dtype, device=q.device)
    if dk is None:
        dk = torch.empty((B, T, Hkv, D), dtype=o.dtype, device=q.device)
    if dv is None:
        dv = torch.empty((B, T, Hkv, D), dtype=o.dtype, device=q.device)
    if workspace is None:
        workspace = new_workspace(True, q, k, rope_base, flags)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
            B, T, Hq, Hkv, D, float(rope_base))
    tail = (_DT[q.dtype], _DT[o.dtype], int(flags), _ptr(workspace), _nbytes(workspace), _stream())
    if window or qk_norm is not None or events is not None:
        opts = make_opts(window, qk_norm)
        _check(lib().ne_rope_attn_bwd_ex(*head, ctypes.byref(opts), *tail, _events_arg(events, 6)))
    else:
        _check(lib().ne_rope_attn_bwd(*head, *tail))
    return dq, dk, dv


def ne_rope_attn_bwd_ex(q, k, v, o, lse, dO, rope_base, window=0, qk_norm=None, **kw):
    """Backward with every option; the options must be the forward's."""
    return ne_rope_attn_bwd(q, k, v, o, lse, dO, rope_base, window=window, qk_norm=qk_norm, **kw)


# ---------------------------------------------------------------------------------------------
# Key/value cache: decode and chunked prefill.
# ---------------------------------------------------------------------------------------------
def kv_cache_bytes(B, Tcap, Hkv, D, in_dtype):
    return int(lib().ne_kv_cache_bytes(B, Tcap, Hkv, D, _DT[in_dtype]))


def new_kv_cache(B, Tcap, Hkv, D, in_dtype, device):
    """A zeroed cache buffer (uint8) in the library's layout."""
    n = kv_cache_bytes(B, Tcap, Hkv, D, in_dtype)
    if n == 0:
        raise ValueError("invalid cache shape")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _lens_arg(lens, B, device):
    if isinstance(lens, torch.Tensor):
        if lens.dtype != torch.int32 or not lens.is_cuda or lens.numel() != B:
            raise ValueError("cache_lens must be a device int32 tensor of B entries")
        return lens
    return torch.tensor(list(lens), dtype=torch.int32, device=device)


def ne_kv_cache_append(cache, cache_lens, k_new, v_new, Tcap, rope_base, qk_norm=None, rope_half_split=False):
    """Write k_new, v_new [B, Tn, Hkv, D] at positions cache_lens[b] .. of the cache."""
    _require_gpu(cache, k_new, v_new)
    B, Tn, Hkv, D = k_new.shape
    lens = _lens_arg(cache_lens, B, k_new.device)
    opts = make_opts(0, qk_norm, rope_half_split)
    _check(lib().ne_kv_cache_append(_ptr(cache), cache.numel() * cache.element_size(), _ptr(lens), _ptr(k_new),
                                    _ptr(v_new), B, Tn, Tcap, Hkv, D, float(rope_base), ctypes.byref(opts),
                                    _DT[k_new.dtype], _stream()))
    return lens


def decode_workspace_bytes(B, Tq, Tcap, Hq, Hkv, D, in_dtype):
    return int(lib().ne_rope_attn_decode_workspace_bytes(B, Tq, Tcap, Hq, Hkv, D, _DT[in_dtype]))


def ne_rope_attn_decode(q, cache, cache_lens, Tcap, Hkv, rope_base, window=0, out_dtype=torch.float32,
                        o=None, lse=None, workspace=None, events=None, qk_norm=None, rope_half_split=False):
    """o, lse for the queries q [B, Tq, Hq, D] at positions cache_lens[b] + t against the cache.

    events: optional 4 events (or None entries) around the two launches."""
    _require_gpu(q, cache)
    B, Tq, Hq, D = q.shape
    lens = _lens_arg(cache_lens, B, q.device)
    if o is None:
        o = torch.empty((B, Tq, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(decode_workspace_bytes(B, Tq, Tcap, Hq, Hkv, D, q.dtype), q.device)
    opts = make_opts(window, qk_norm, rope_half_split)
    _check(lib().ne_rope_attn_decode(_ptr(q), _ptr(cache), cache.numel() * cache.element_size(), _ptr(lens),
                                     _ptr(o), _ptr(lse), B, Tq, Tcap, Hq, Hkv, D, float(rope_base), ctypes.byref(opts),
                                     _DT[q.dtype], _DT[o.dtype], _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(),
                                     _events_arg(events, 4)))
    return o, lse


DECODE_SCRATCH_BYTES = 64 << 20


def ne_rope_attn_decode_noalloc(q, cache, cache_lens, Tcap, Hkv, rope_base, window=0, out_dtype=torch.float32,
                                o=None, lse=None, qk_norm=None, rope_half_split=False):
    """ne_rope_attn_decode without a workspace: the split partials go to the library's own scratch
    (DECODE_SCRATCH_BYTES per GPU); shapes that need more are rejected.  Pass o and lse to make the
    call allocate nothing at all."""
    _require_gpu(q, cache)
    B, Tq, Hq, D = q.shape
    lens = _lens_arg(cache_lens, B, q.device)
    if o is None:
        o = torch.empty((B, Tq, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    opts = make_opts(window, qk_norm, rope_half_split)
    _check(lib().ne_rope_attn_decode_noalloc(_ptr(q), _ptr(cache), _nbytes(cache), _ptr(lens), _ptr(o), _ptr(lse),
                                             B, Tq, Tcap, Hq, Hkv, D, float(rope_base), ctypes.byref(opts),
                                             _DT[q.dtype], _DT[o.dtype], _stream()))
    return o, lse


# ---------------------------------------------------------------------------------------------
# QKV projection with the RoPE epilogue.
# ---------------------------------------------------------------------------------------------
def ne_qkv_rope_proj(x, w, Hq, Hkv, rope_base, qk_norm=None, out_dtype=torch.float32, q=None, k=None, v=None,
                     workspace=None, events=None, rope_half_split=False):
    """q', k', v from x [B, T, C] and w [(Hq + 2 Hkv) D, C]: y = x w^T, RoPE (after the optional QK norm)
    applied to the query and key heads in the product's epilogue."""
    _require_gpu(x, w)
    B, T, C = x.shape
    N = w.shape[0]
    D = N // (Hq + 2 * Hkv)
    if w.shape[1] != C or D * (Hq + 2 * Hkv) != N:
        raise ValueError("weight shape does not match C, Hq, Hkv")
    if q is None:
        q = torch.empty((B, T, Hq, D), dtype=out_dtype, device=x.device)
    if k is None:
        k = torch.empty((B, T, Hkv, D), dtype=out_dtype, device=x.device)
    if v is None:
        v = torch.empty((B, T, Hkv, D), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(int(lib().ne_qkv_rope_workspace_bytes(T, D)), x.device)
    opts = make_opts(0, qk_norm, rope_half_split)
    _check(lib().ne_qkv_rope_proj(_ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), B, T, C, Hq, Hkv, D, float(rope_base),
                                  ctypes.byref(opts), _DT[x.dtype], _DT[q.dtype], _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(), _events_arg(events, 4)))
    return q, k, v

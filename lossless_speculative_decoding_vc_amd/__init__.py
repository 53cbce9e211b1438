"""Python binding of libvc, the MI355X (gfx950) VeriCache hot path.

Argument marshalling only: every computation runs in the HIP kernels of
``libvc.so`` (built in-tree by :mod:`lossless_speculative_decoding_vc_amd.build`).
torch supplies device memory and the current HIP stream.  There is no CPU
fallback: if the library is missing or fails to load, every call raises.

Tensor layouts follow ``include/vc.h``: K token-major ``[..][tokens][D]``,
V channel-major ``[..][D][tokens]``.
"""
import ctypes
import os

import torch

__all__ = [
    "VcError", "lib", "library_path", "draft_attn", "verify_attn", "accept",
    "draft_workspace_size", "verify_workspace_size", "declared_symbols",
    "argmax", "commit_rows", "quantize_int4", "csm_round", "Stagger", "new_workspace",
    "draft_args", "verify_args", "ROUND_STAGGERED", "ROUND_BULK",
    "VC_BF16", "VC_FP32", "VC_KV_DENSE", "VC_KV_INT4", "VC_KV_INT4_PACKED",
]

VC_OK, VC_EINVAL, VC_ENOTSUP, VC_EHIP = 0, 1, 2, 3
VC_BF16, VC_FP32 = 0, 1
VC_KV_DENSE, VC_KV_INT4, VC_KV_INT4_PACKED = 0, 1, 2
INT4_PACKED_BLOCK = 5120   # bytes per 32-token block of a packed int4 cache (head_dim 128)

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libvc.so")
_INCLUDE = os.path.join(os.path.dirname(_HERE), "include")
_HEADERS = sorted(os.path.join(_INCLUDE, f) for f in os.listdir(_INCLUDE) if f.endswith(".h"))


class VcError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {VC_OK: "VC_OK", VC_EINVAL: "VC_EINVAL", VC_ENOTSUP: "VC_ENOTSUP", VC_EHIP: "VC_EHIP"}

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class DraftArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("D", _i32),
                ("dtype", _i32), ("fmt", _i32), ("scale", ctypes.c_float), ("num_splits", _i32),
                ("cap", _i64), ("tcap", _i64),
                ("q", _p), ("main_len", _p), ("k", _p), ("v", _p),
                ("k_scale", _p), ("k_zero", _p), ("v_scale", _p), ("v_zero", _p),
                ("degree", _p), ("degree_h_stride", _i64),
                ("tail_k", _p), ("tail_v", _p), ("tail_len", _p),
                ("out", _p), ("out_lse", _p), ("workspace", _p), ("workspace_bytes", ctypes.c_size_t)]


class VerifyArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("D", _i32), ("M", _i32),
                ("dtype", _i32), ("scale", ctypes.c_float), ("num_splits", _i32),
                ("ccap", _i64),
                ("q", _p), ("ctx_k", _p), ("ctx_v", _p), ("ctx_len", _p),
                ("blk_k", _p), ("blk_v", _p), ("out", _p), ("out_lse", _p),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t)]


class AcceptArgs(ctypes.Structure):
    _fields_ = [("B", _i32), ("M", _i32), ("V", _i32), ("logit_dtype", _i32),
                ("logits", _p), ("draft", _p), ("argmax", _p), ("accept_len", _p),
                ("out_tokens", _p), ("n_out", _p)]


class RoundCommit(ctypes.Structure):
    _fields_ = [("kind", _i32), ("dst_k", _p), ("dst_v", _p), ("len", _p), ("degree", _p), ("degree_h_stride", _i64),
                ("cap", _i64), ("dst_v_blocked", _i32), ("tail_k", _p), ("tail_v", _p), ("tcap", _i64),
                ("tail_len", _p), ("packed", _p), ("main_len", _p), ("host_k", _p), ("host_v", _p)]


ROUND_HOOK = ctypes.CFUNCTYPE(None, _p, _i32, _p)


class RoundFetch(ctypes.Structure):
    _fields_ = [("host_src", _p), ("dev_dst", _p), ("bytes", ctypes.c_size_t), ("layer", _i32)]


class RoundDesc(ctypes.Structure):
    _fields_ = [("layers", _i32), ("steps", _i32), ("mode", _i32),
                ("lm_w", _p), ("Dm", _i32), ("V", _i32),
                ("draft", ctypes.POINTER(DraftArgs)), ("step_tail_len", ctypes.POINTER(_p)),
                ("draft_hidden", ctypes.POINTER(_p)), ("drafts", _p), ("draft_lm_ws", _p),
                ("draft_lm_ws_bytes", ctypes.c_size_t),
                ("verify", ctypes.POINTER(VerifyArgs)), ("host_kv", ctypes.POINTER(_p)),
                ("kv_bytes", ctypes.c_size_t), ("v_offset", ctypes.c_size_t),
                ("verify_hidden", _p), ("verify_drafts", _p), ("argmax", _p), ("accept_len", _p),
                ("out_tokens", _p), ("n_out", _p), ("verify_lm_ws", _p), ("verify_lm_ws_bytes", ctypes.c_size_t),
                ("commit", ctypes.POINTER(RoundCommit)), ("before_verify", ROUND_HOOK), ("hook_ctx", _p),
                ("time_kernels", _i32), ("fetch", ctypes.POINTER(RoundFetch)), ("n_fetch", _i32)]


ROUND_STAGGERED, ROUND_BULK, ROUND_CHAINED = 0, 1, 2
TIME_NONE, TIME_DRAFT_STEPS, TIME_ATTENTION_KERNELS = 0, 1, 2   # vc_round_timing
COMMIT_ROWS, COMMIT_INT4_TAIL = 0, 1

_lib = None


def lib():
    """The loaded ``libvc.so`` (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"libvc.so not built at {library_path}; run "
                              "python -m lossless_speculative_decoding_vc_amd.build")
        L = ctypes.CDLL(library_path)
        for name, argt in (("vc_draft_attn", [ctypes.POINTER(DraftArgs), _p]),
                           ("vc_verify_attn", [ctypes.POINTER(VerifyArgs), _p]),
                           ("vc_accept", [ctypes.POINTER(AcceptArgs), _p])):
            fn = getattr(L, name)
            fn.argtypes = argt
            fn.restype = ctypes.c_int
        L.vc_draft_attn_noalloc.argtypes = [ctypes.POINTER(DraftArgs), _p]
        L.vc_draft_attn_noalloc.restype = ctypes.c_int
        L.vc_draft_noalloc_max_scratch.restype = ctypes.c_size_t
        L.vc_draft_workspace_size.argtypes = [ctypes.POINTER(DraftArgs)]
        L.vc_draft_workspace_size.restype = ctypes.c_size_t
        L.vc_verify_workspace_size.argtypes = [ctypes.POINTER(VerifyArgs)]
        L.vc_verify_workspace_size.restype = ctypes.c_size_t
        L.vc_argmax.argtypes = [_i32, _i32, _i32, _p, _p, _i32, _p]
        L.vc_argmax.restype = ctypes.c_int
        L.vc_next_input.argtypes = [_i32, _i32, _p, _p, _p, _i64, _p]
        L.vc_next_input.restype = ctypes.c_int
        L.vc_lm_head_argmax_workspace_size.argtypes = [_i32, _i32]
        L.vc_lm_head_argmax_workspace_size.restype = ctypes.c_size_t
        L.vc_lm_head_argmax.argtypes = [_i32, _i32, _i32, _p, _p, _p, _i32, _p, ctypes.c_size_t, _p]
        L.vc_lm_head_argmax.restype = ctypes.c_int
        L.vc_lm_head_accept.argtypes = [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
        L.vc_lm_head_accept.restype = ctypes.c_int
        L.vc_commit_rows.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _i64, _p]
        L.vc_commit_rows.restype = ctypes.c_int
        L.vc_quantize_int4.argtypes = [_i32, _i32, _i32, _p, _p, _i64, _p, _i32, _i64, _p, _p, _p, _p, _p, _p, _p, _p]
        L.vc_quantize_int4.restype = ctypes.c_int
        L.vc_compact_kv.argtypes = [_i32, _i32, _i32, _i32, _p, _p, _i64, _p, _i64, _p, _p, _p, _i64, _p, _p]
        L.vc_compact_kv.restype = ctypes.c_int
        L.vc_quantize_int4_packed.argtypes = [_i32, _i32, _i32, _p, _p, _i64, _p, _i32, _i64, _p, _p, _p]
        L.vc_int4_commit.argtypes = [_i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _i64, _p, _p, _i64, _p, _p]
        L.vc_int4_commit.restype = ctypes.c_int
        L.vc_quantize_int4_packed.restype = ctypes.c_int
        L.vc_csm_round.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_double, _p, _p, _p, _i64,
                                   _p, _p, _p, _i64, ctypes.POINTER(_i32), _p, _p]
        L.vc_csm_round_due.argtypes = [_i64, _i64, _i32, _i32]
        L.vc_csm_round_due.restype = _i32
        L.vc_csm_schedule_ratio.argtypes = [ctypes.c_double, ctypes.c_double, _i32]
        L.vc_csm_schedule_ratio.restype = ctypes.c_double
        L.vc_csm_round.restype = ctypes.c_int
        L.vc_stagger_create.argtypes = [ctypes.POINTER(_p), ctypes.POINTER(_p), _i32, ctypes.c_size_t, _i32]
        L.vc_stagger_stream_layer.argtypes = [_p, _i32, _p, ctypes.c_size_t]
        L.vc_stagger_acquire.argtypes = [_p, _i32, _p, ctypes.POINTER(_p)]
        L.vc_stagger_release.argtypes = [_p, _i32, _p]
        L.vc_stagger_writeback.argtypes = [_p, _p, _p, ctypes.c_size_t, _p]
        L.vc_stagger_after.argtypes = [_p, _p]
        L.vc_stagger_sync.argtypes = [_p]
        L.vc_stagger_copy_ms.argtypes = [_p, _i32, ctypes.POINTER(ctypes.c_float)]
        L.vc_stagger_destroy.argtypes = [_p]
        L.vc_stagger_round.argtypes = [_p, ctypes.POINTER(RoundDesc), _p, _p]
        L.vc_stagger_round_times.argtypes = [_p, _p, ctypes.POINTER(_i32), _p, ctypes.POINTER(_i32)]
        for n in ("vc_stagger_create", "vc_stagger_stream_layer", "vc_stagger_acquire", "vc_stagger_release",
                  "vc_stagger_writeback", "vc_stagger_after", "vc_stagger_sync", "vc_stagger_copy_ms",
                  "vc_stagger_destroy", "vc_stagger_round", "vc_stagger_round_times"):
            getattr(L, n).restype = ctypes.c_int
        L.vc_last_error.restype = ctypes.c_char_p
        L.vc_status_string.restype = ctypes.c_char_p
        L.vc_status_string.argtypes = [ctypes.c_int]
        L.vc_build_info.restype = ctypes.c_char_p
        _lib = L
    return _lib


def declared_symbols():
    """Function names declared by the public headers."""
    import re
    names = []
    for h in _HEADERS:
        with open(h) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(vc_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def _check(status):
    if status != VC_OK:
        raise VcError(status, lib().vc_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_out(out, rows, stride):
    """The kernels write out[r * stride] for r < rows: the tensor must reach that far."""
    if rows > 0 and out.numel() < (rows - 1) * stride + 1:
        raise ValueError(f"out holds {out.numel()} entries; {rows} rows at stride {stride} need "
                         f"{(rows - 1) * stride + 1}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _want(t, name, shape, dtypes):
    """Shape and dtype of a tensor against the layout the C ABI reads: the
    kernels see raw pointers, so a short or mistyped buffer must be refused
    here, before anything is enqueued."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must be {list(int(x) for x in shape)}, got {list(t.shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


_HALF = None   # binary16 carriers (float16 or int16), filled on first use


def _half():
    global _HALF
    if _HALF is None:
        _HALF = (torch.float16, torch.int16)
    return _HALF


def new_workspace(nbytes, device):
    """A workspace for the split / tiled entry points (uint8, at least
    ``nbytes`` bytes; its contents need no initialisation)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _vc_dtype(t):
    if t.dtype == torch.bfloat16:
        return VC_BF16
    if t.dtype == torch.float32:
        return VC_FP32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _draft_struct(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse,
                  scale, num_splits, fmt, k_scale, k_zero, v_scale, v_zero, Hkv, cap):
    B, Hq, D = q.shape
    a = DraftArgs()
    a.B, a.Hq, a.Hkv, a.D = B, Hq, Hkv, D
    a.dtype = _vc_dtype(q)
    a.fmt = fmt
    a.scale = D ** -0.5 if scale is None else scale
    a.num_splits = num_splits
    a.cap = cap
    a.tcap = 0 if tail_k is None else tail_k.shape[2]
    a.q, a.main_len, a.k, a.v = _ptr(q), _ptr(main_len), _ptr(k), _ptr(v)
    a.k_scale, a.k_zero, a.v_scale, a.v_zero = map(_ptr, (k_scale, k_zero, v_scale, v_zero))
    a.degree = _ptr(degree)
    a.degree_h_stride = 0 if degree is None or degree.shape[1] == 1 else cap
    a.tail_k, a.tail_v, a.tail_len = _ptr(tail_k), _ptr(tail_v), _ptr(tail_len)
    a.out, a.out_lse = _ptr(out), _ptr(out_lse)
    return a


def draft_attn(q, k, v, main_len, degree=None, tail_k=None, tail_v=None, tail_len=None,
               out=None, out_lse=None, scale=None, num_splits=0, workspace=None,
               fmt=VC_KV_DENSE, k_scale=None, k_zero=None, v_scale=None, v_zero=None,
               stream=None):
    """Draft decode attention (``vc_draft_attn``).

    ``q [B][Hq][D]``; dense ``k [B][Hkv][cap][D]``, ``v [B][Hkv][cap/32][D][32]``
    (32-token blocks, channel-major inside a block);
    ``main_len`` int32 ``[B][Hkv]``; ``degree`` fp32 ``[B][1 or Hkv][cap]``;
    ``tail_k [B][Hkv][tcap][D]``, ``tail_v [B][Hkv][D][tcap]``, ``tail_len``
    int32 ``[B]``.  Returns ``out [B][Hq][D]`` (and fills ``out_lse``).
    """
    if out is None:
        out = torch.empty_like(q)
    a = draft_args(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse, scale, num_splits,
                   workspace, fmt, k_scale, k_zero, v_scale, v_zero)
    _check(lib().vc_draft_attn(ctypes.byref(a), _stream(stream)))
    return out


def draft_attn_noalloc(q, k, v, main_len, degree=None, tail_k=None, tail_v=None, tail_len=None, out=None,
                       out_lse=None, scale=None, num_splits=0, fmt=VC_KV_DENSE, k_scale=None, k_zero=None,
                       v_scale=None, v_zero=None, stream=None):
    """:func:`draft_attn` through ``vc_draft_attn_noalloc``: the split
    partials live in the library's static per-GPU array, so the library
    allocates nothing (``out`` is required: this wrapper allocates nothing
    either)."""
    if out is None:
        raise ValueError("out is required")
    _check_draft_shapes(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse, fmt,
                        k_scale, k_zero, v_scale, v_zero)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (tail_k, "tail_k"), (tail_v, "tail_v"),
                 (out, "out"), (degree, "degree"), (out_lse, "out_lse"), (k_scale, "k_scale"),
                 (k_zero, "k_zero"), (v_scale, "v_scale"), (v_zero, "v_zero")):
        _dev(t, n)
    _dev(main_len, "main_len", torch.int32)
    _dev(tail_len, "tail_len", torch.int32)
    cap = k.shape[2] * 32 if fmt == VC_KV_INT4_PACKED else k.shape[2]
    a = _draft_struct(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse,
                      scale, num_splits, fmt, k_scale, k_zero, v_scale, v_zero, k.shape[1], cap)
    _check(lib().vc_draft_attn_noalloc(ctypes.byref(a), _stream(stream)))
    return out


def draft_args(q, k, v, main_len, degree=None, tail_k=None, tail_v=None, tail_len=None, out=None, out_lse=None,
               scale=None, num_splits=0, workspace=None, fmt=VC_KV_DENSE, k_scale=None, k_zero=None, v_scale=None,
               v_zero=None):
    """The checked ``vc_draft_args`` of one draft call (the arguments of
    :func:`draft_attn`; ``out`` is required), with a workspace attached when
    the call is split (a new zeroed one unless ``workspace`` is big enough).
    The struct holds raw pointers: keep the tensors alive while it is used."""
    if out is None:
        raise ValueError("out is required")
    _check_draft_shapes(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse, fmt,
                        k_scale, k_zero, v_scale, v_zero)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (tail_k, "tail_k"), (tail_v, "tail_v"),
                 (out, "out"), (degree, "degree"), (out_lse, "out_lse"), (k_scale, "k_scale"),
                 (k_zero, "k_zero"), (v_scale, "v_scale"), (v_zero, "v_zero")):
        _dev(t, n)
    _dev(main_len, "main_len", torch.int32)
    _dev(tail_len, "tail_len", torch.int32)
    Hkv = k.shape[1]
    cap = k.shape[2] * 32 if fmt == VC_KV_INT4_PACKED else k.shape[2]
    a = _draft_struct(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse,
                      scale, num_splits, fmt, k_scale, k_zero, v_scale, v_zero, Hkv, cap)
    need = lib().vc_draft_workspace_size(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = new_workspace(need, q.device)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    a._keep = workspace
    return a


def _check_draft_shapes(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse, fmt,
                        k_scale, k_zero, v_scale, v_zero):
    """Every tensor of a draft call against the layouts of ``vc_draft_args``."""
    if q.dim() != 3:
        raise ValueError(f"q must be [B][Hq][D], got {list(q.shape)}")
    B, Hq, D = q.shape
    act = (torch.bfloat16, torch.float32)
    _want(q, "q", (B, Hq, D), act)
    if k.dim() < 2 or k.shape[0] != B:
        raise ValueError(f"k must start with [B={B}][Hkv], got {list(k.shape)}")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of the KV heads of k ({Hkv})")
    u8 = (torch.uint8,)
    if fmt == VC_KV_INT4_PACKED:
        if k.dim() != 4:
            raise ValueError("a packed int4 cache is [B][Hkv][cap/32][5120] uint8")
        cap = k.shape[2] * 32
        _want(k, "k", (B, Hkv, cap // 32, INT4_PACKED_BLOCK), u8)
        if any(t is not None for t in (v, k_scale, k_zero, v_scale, v_zero)):
            raise ValueError("a packed int4 cache lives in k alone: v and the scales/zeros must be None")
    elif fmt == VC_KV_INT4:
        if k.dim() != 4:
            raise ValueError("int4 k codes are [B][Hkv][cap][D/2] uint8")
        cap = k.shape[2]
        _want(k, "k", (B, Hkv, cap, D // 2), u8)
        _want(v, "v", (B, Hkv, cap // 32, D, 16), u8)
        for t, n in ((k_scale, "k_scale"), (k_zero, "k_zero")):
            if t is None:
                raise ValueError(f"{n} is required for an int4 cache")
            _want(t, n, (B, Hkv, cap // 32, D), _half())
        for t, n in ((v_scale, "v_scale"), (v_zero, "v_zero")):
            if t is None:
                raise ValueError(f"{n} is required for an int4 cache")
            _want(t, n, (B, Hkv, cap // 32, D // 32, 32), _half())
    elif fmt == VC_KV_DENSE:
        if k.dim() != 4:
            raise ValueError("k must be [B][Hkv][cap][D]")
        cap = k.shape[2]
        _want(k, "k", (B, Hkv, cap, D), (q.dtype,))
        if v is None:
            raise ValueError("v is required for a dense cache")
        _want(v, "v", (B, Hkv, cap // 32, D, 32), (q.dtype,))
        if any(t is not None for t in (k_scale, k_zero, v_scale, v_zero)):
            raise ValueError("scales/zeros belong to an int4 cache only")
    else:
        raise ValueError(f"unknown kv format {fmt}")
    if main_len is None:
        raise ValueError("main_len is required")
    _want(main_len, "main_len", (B, Hkv), (torch.int32,))
    if degree is not None:
        if degree.dim() != 3 or degree.shape[1] not in (1, Hkv):
            raise ValueError(f"degree must be [B][1 or Hkv][cap], got {list(degree.shape)}")
        _want(degree, "degree", (B, degree.shape[1], cap), (torch.float32,))
    if (tail_k is None) != (tail_v is None) or (tail_len is not None and tail_k is None):
        raise ValueError("tail_k, tail_v (and tail_len) go together")
    if tail_k is not None:
        if tail_k.dim() != 4:
            raise ValueError("tail_k must be [B][Hkv][tcap][D]")
        tcap = tail_k.shape[2]
        _want(tail_k, "tail_k", (B, Hkv, tcap, D), (q.dtype,))
        _want(tail_v, "tail_v", (B, Hkv, D, tcap), (q.dtype,))
        _want(tail_len, "tail_len", (B,), (torch.int32,))
    _want(out, "out", (B, Hq, D), (q.dtype,))
    _want(out_lse, "out_lse", (B, Hq), (torch.float32,))


def draft_workspace_size(**kw):
    a = DraftArgs()
    for key, val in kw.items():
        setattr(a, key, val)
    return lib().vc_draft_workspace_size(ctypes.byref(a))


def verify_attn(q, ctx_k, ctx_v, ctx_len, blk_k, blk_v, out=None, out_lse=None, scale=None,
                num_splits=0, workspace=None, stream=None):
    """Verify block attention (``vc_verify_attn``).

    ``q [B][M][Hq][D]``; ``ctx_k [B][Hkv][ccap][D]``, ``ctx_v [B][Hkv][D][ccap]``;
    ``ctx_len`` int32 ``[B]``; ``blk_k [B][Hkv][M][D]``, ``blk_v [B][Hkv][D][M]``.
    Returns ``out [B][M][Hq][D]``.
    """
    if out is None:
        out = torch.empty_like(q)
    a = verify_args(q, ctx_k, ctx_v, ctx_len, blk_k, blk_v, out, out_lse, scale, num_splits, workspace)
    _check(lib().vc_verify_attn(ctypes.byref(a), _stream(stream)))
    return out


def verify_args(q, ctx_k, ctx_v, ctx_len, blk_k, blk_v, out, out_lse=None, scale=None, num_splits=0,
                workspace=None, ccap=None):
    """The checked ``vc_verify_args`` of one verify call (the arguments of
    :func:`verify_attn`; ``out`` is required).  With ``ctx_k = ctx_v = None``
    and ``ccap`` given, the context comes from elsewhere (the staging slot of
    :meth:`Stagger.round`).  The struct holds raw pointers: keep the tensors
    alive while it is used."""
    if out is None:
        raise ValueError("out is required")
    _check_verify_shapes(q, ctx_k, ctx_v, ctx_len, blk_k, blk_v, out, out_lse)
    for t, n in ((q, "q"), (ctx_k, "ctx_k"), (ctx_v, "ctx_v"), (blk_k, "blk_k"),
                 (blk_v, "blk_v"), (out, "out"), (out_lse, "out_lse")):
        _dev(t, n)
    _dev(ctx_len, "ctx_len", torch.int32)
    B, M, Hq, D = q.shape
    Hkv = blk_k.shape[1]
    a = VerifyArgs()
    a.B, a.Hq, a.Hkv, a.D, a.M = B, Hq, Hkv, D, M
    a.dtype = _vc_dtype(q)
    a.scale = D ** -0.5 if scale is None else scale
    a.num_splits = num_splits
    if ctx_k is not None:
        a.ccap = ctx_k.shape[2]
    else:
        a.ccap = 0 if ccap is None else int(ccap)
    a.q, a.ctx_k, a.ctx_v, a.ctx_len = _ptr(q), _ptr(ctx_k), _ptr(ctx_v), _ptr(ctx_len)
    a.blk_k, a.blk_v, a.out, a.out_lse = _ptr(blk_k), _ptr(blk_v), _ptr(out), _ptr(out_lse)
    need = lib().vc_verify_workspace_size(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = new_workspace(need, q.device)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    a._keep = workspace
    return a


def _check_verify_shapes(q, ctx_k, ctx_v, ctx_len, blk_k, blk_v, out, out_lse):
    """Every tensor of a verify call against the layouts of ``vc_verify_args``."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B][M][Hq][D], got {list(q.shape)}")
    B, M, Hq, D = q.shape
    _want(q, "q", (B, M, Hq, D), (torch.bfloat16, torch.float32))
    if blk_k is None or blk_v is None or ctx_len is None:
        raise ValueError("blk_k, blk_v and ctx_len are required")
    if blk_k.dim() != 4:
        raise ValueError("blk_k must be [B][Hkv][M][D]")
    Hkv = blk_k.shape[1]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError(f"Hq ({Hq}) must be a multiple of the KV heads of blk_k ({Hkv})")
    _want(blk_k, "blk_k", (B, Hkv, M, D), (q.dtype,))
    _want(blk_v, "blk_v", (B, Hkv, D, M), (q.dtype,))
    _want(ctx_len, "ctx_len", (B,), (torch.int32,))
    if (ctx_k is None) != (ctx_v is None):
        raise ValueError("ctx_k and ctx_v go together")
    if ctx_k is not None:
        if ctx_k.dim() != 4:
            raise ValueError("ctx_k must be [B][Hkv][ccap][D]")
        ccap = ctx_k.shape[2]
        _want(ctx_k, "ctx_k", (B, Hkv, ccap, D), (q.dtype,))
        _want(ctx_v, "ctx_v", (B, Hkv, D, ccap), (q.dtype,))
    _want(out, "out", (B, M, Hq, D), (q.dtype,))
    _want(out_lse, "out_lse", (B, M, Hq), (torch.float32,))


def verify_workspace_size(**kw):
    a = VerifyArgs()
    for key, val in kw.items():
        setattr(a, key, val)
    return lib().vc_verify_workspace_size(ctypes.byref(a))


def accept(logits, draft, argmax=None, accept_len=None, out_tokens=None, n_out=None, stream=None):
    """Greedy argmax + accept-until-first-mismatch (``vc_accept``).

    ``logits [B][M][V]`` (bf16 or fp32); ``draft`` int32 ``[B][M-1]``.
    Returns ``(argmax [B][M], accept_len [B], out_tokens [B][M], n_out [B])``.
    """
    _dev(logits, "logits")
    _dev(draft, "draft", torch.int32)
    B, M, V = logits.shape
    dev = logits.device
    argmax = torch.empty((B, M), dtype=torch.int32, device=dev) if argmax is None else argmax
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    out_tokens = torch.empty((B, M), dtype=torch.int32, device=dev) if out_tokens is None else out_tokens
    n_out = torch.empty(B, dtype=torch.int32, device=dev) if n_out is None else n_out
    for t, n, numel in ((argmax, "argmax", B * M), (accept_len, "accept_len", B), (out_tokens, "out_tokens", B * M),
                        (n_out, "n_out", B)):
        _dev(t, n, torch.int32)
        if t.numel() < numel:
            raise ValueError(f"{n} holds {t.numel()} entries, {numel} needed")
    if draft.numel() < B * (M - 1):
        raise ValueError(f"draft must be [B][M-1] = [{B}][{M - 1}]")
    a = AcceptArgs()
    a.B, a.M, a.V = B, M, V
    a.logit_dtype = _vc_dtype(logits)
    a.logits, a.draft = _ptr(logits), _ptr(draft)
    a.argmax, a.accept_len, a.out_tokens, a.n_out = map(_ptr, (argmax, accept_len, out_tokens, n_out))
    _check(lib().vc_accept(ctypes.byref(a), _stream(stream)))
    return argmax, accept_len, out_tokens, n_out


def argmax(logits, out=None, out_stride=1, stream=None):
    """Drafter token choice (``vc_argmax``): row argmax of ``logits [R][V]``,
    lowest index on ties, written to ``out[r * out_stride]`` (int32)."""
    _dev(logits, "logits")
    R, V = logits.shape[0], logits.shape[-1]
    R = logits.numel() // V
    if out is None:
        out = torch.empty(R * out_stride, dtype=torch.int32, device=logits.device)
    _dev(out, "out", torch.int32)
    _check_out(out, R, out_stride)
    _check(lib().vc_argmax(R, V, _vc_dtype(logits), _ptr(logits), _ptr(out), out_stride, _stream(stream)))
    return out


def next_input(out_tokens, n_out, out, out_stride=1, stream=None):
    """The next round's first input token of each request (``vc_next_input``):
    ``out[b * out_stride] = out_tokens[b][n_out[b] - 1]`` for ``out_tokens
    [B][M]`` and ``n_out [B]`` as :func:`accept` writes them."""
    _dev(out_tokens, "out_tokens", torch.int32)
    _dev(n_out, "n_out", torch.int32)
    _dev(out, "out", torch.int32)
    if out_tokens.dim() != 2:
        raise ValueError("out_tokens must be [B][M]")
    B, M = out_tokens.shape
    _want(n_out, "n_out", (B,), (torch.int32,))
    _check_out(out, B, out_stride)
    _check(lib().vc_next_input(B, M, _ptr(out_tokens), _ptr(n_out), _ptr(out), out_stride, _stream(stream)))
    return out


def lm_head_argmax_workspace(R, V, device):
    """Workspace tensor (uint8) for :func:`lm_head_argmax` over R rows."""
    return new_workspace(lib().vc_lm_head_argmax_workspace_size(R, V), device)


def lm_head_argmax(h, w, out=None, out_stride=1, workspace=None, stream=None):
    """Greedy token of each hidden row without writing logits
    (``vc_lm_head_argmax``): ``out[r * out_stride] = argmax_v h[r] . w[v]``
    for ``h [R][Dm]`` and vocab-major ``w [V][Dm]`` (bf16)."""
    _dev(h, "h", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    Dm = h.shape[-1]
    R = h.numel() // Dm
    V = w.shape[0]
    if w.shape[1] != Dm:
        raise ValueError("w must be [V][Dm]")
    if out is None:
        out = torch.empty(R * out_stride, dtype=torch.int32, device=h.device)
    _dev(out, "out", torch.int32)
    _check_out(out, R, out_stride)
    if workspace is None:
        workspace = lm_head_argmax_workspace(R, V, h.device)
    _check(lib().vc_lm_head_argmax(R, Dm, V, _ptr(h), _ptr(w), _ptr(out), out_stride, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def lm_head_accept(h, w, draft, argmax=None, accept_len=None, out_tokens=None, n_out=None, workspace=None,
                   stream=None):
    """Verify logits, greedy acceptance and emitted tokens in one call
    (``vc_lm_head_accept``): ``h [B][M][Dm]``, vocab-major ``w [V][Dm]``
    (bf16), ``draft`` int32 ``[B][M-1]``.  Returns
    ``(argmax [B][M], accept_len [B], out_tokens [B][M], n_out [B])``."""
    _dev(h, "h", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    _dev(draft, "draft", torch.int32)
    B, M, Dm = h.shape
    V = w.shape[0]
    if w.shape[1] != Dm:
        raise ValueError("w must be [V][Dm]")
    dev = h.device
    argmax = torch.empty((B, M), dtype=torch.int32, device=dev) if argmax is None else argmax
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    out_tokens = torch.empty((B, M), dtype=torch.int32, device=dev) if out_tokens is None else out_tokens
    n_out = torch.empty(B, dtype=torch.int32, device=dev) if n_out is None else n_out
    for t, n, numel in ((argmax, "argmax", B * M), (accept_len, "accept_len", B), (out_tokens, "out_tokens", B * M),
                        (n_out, "n_out", B)):
        _dev(t, n, torch.int32)
        if t.numel() < numel:
            raise ValueError(f"{n} holds {t.numel()} entries, {numel} needed")
    if draft.numel() < B * (M - 1):
        raise ValueError(f"draft must be [B][M-1] = [{B}][{M - 1}]")
    if workspace is None:
        workspace = lm_head_argmax_workspace(B * M, V, dev)
    _check(lib().vc_lm_head_accept(B, M, Dm, V, _ptr(h), _ptr(w), _ptr(draft), _ptr(argmax), _ptr(accept_len),
                                   _ptr(out_tokens), _ptr(n_out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))
    return argmax, accept_len, out_tokens, n_out


def commit_rows(blk_k, blk_v, n_out, dst_k, dst_v, length, degree=None, v_blocked=False, stream=None):
    """Append the first ``n_out[b]`` block rows to a cache (``vc_commit_rows``).

    ``blk_k [B][Hkv][M][D]``, ``blk_v [B][Hkv][D][M]``, ``dst_k [B][Hkv][cap][D]``,
    ``dst_v [B][Hkv][D][cap]`` (a full cache) or, with ``v_blocked``,
    ``[B][Hkv][cap/32][D][32]`` (a compressed main segment), ``length`` int32
    ``[B][Hkv]`` (updated in place).
    """
    if blk_k.dim() != 4 or dst_k.dim() != 4:
        raise ValueError("blk_k must be [B][Hkv][M][D] and dst_k [B][Hkv][cap][D]")
    B, Hkv, M, D = blk_k.shape
    cap = dst_k.shape[2]
    act = (torch.bfloat16, torch.float32)
    _want(blk_k, "blk_k", (B, Hkv, M, D), act)
    _want(blk_v, "blk_v", (B, Hkv, D, M), (blk_k.dtype,))
    _want(dst_k, "dst_k", (B, Hkv, cap, D), (blk_k.dtype,))
    if v_blocked:
        if cap % 32:
            raise ValueError("a blocked V cache needs cap % 32 == 0")
        _want(dst_v, "dst_v", (B, Hkv, cap // 32, D, 32), (blk_k.dtype,))
    else:
        _want(dst_v, "dst_v", (B, Hkv, D, cap), (blk_k.dtype,))
    _want(n_out, "n_out", (B,), (torch.int32,))
    _want(length, "length", (B, Hkv), (torch.int32,))
    if degree is not None:
        if degree.dim() != 3 or degree.shape[1] not in (1, Hkv):
            raise ValueError(f"degree must be [B][1 or Hkv][cap], got {list(degree.shape)}")
        _want(degree, "degree", (B, degree.shape[1], cap), (torch.float32,))
    for t, n in ((blk_k, "blk_k"), (blk_v, "blk_v"), (dst_k, "dst_k"), (dst_v, "dst_v"), (degree, "degree")):
        _dev(t, n)
    _dev(n_out, "n_out", torch.int32)
    _dev(length, "length", torch.int32)
    hstride = 0 if degree is None or degree.shape[1] == 1 else cap
    _check(lib().vc_commit_rows(B, Hkv, D, M, _vc_dtype(blk_k), cap, 1 if v_blocked else 0, _ptr(blk_k), _ptr(blk_v), _ptr(n_out),
                                _ptr(dst_k), _ptr(dst_v), _ptr(length), _ptr(degree), hstride, _stream(stream)))


def quantize_int4(src_k, src_v, src_start, n_groups, dst_start, k_codes, k_scale, k_zero, v_codes, v_scale,
                  v_zero, stream=None):
    """Quantize 32-token groups of bf16 rows into an int4 cache (``vc_quantize_int4``).

    ``src_k [B][Hkv][src_cap][D]``, ``src_v [B][Hkv][D][src_cap]`` bf16;
    ``src_start``/``dst_start`` int32 ``[B][Hkv]``; the cache tensors have the
    int4 layouts :func:`draft_attn` takes (``k_codes [B][Hkv][cap][D/2]`` uint8,
    ``k_scale/k_zero [B][Hkv][cap/32][D]``, ``v_codes [B][Hkv][cap/32][D][16]``,
    ``v_scale/v_zero [B][Hkv][cap/32][D/32][32]``, binary16 as float16 or int16).
    """
    _dev(src_k, "src_k", torch.bfloat16)
    _dev(src_v, "src_v", torch.bfloat16)
    _dev(src_start, "src_start", torch.int32)
    _dev(dst_start, "dst_start", torch.int32)
    for t, n in ((k_codes, "k_codes"), (v_codes, "v_codes")):
        _dev(t, n, torch.uint8)
    for t, n in ((k_scale, "k_scale"), (k_zero, "k_zero"), (v_scale, "v_scale"), (v_zero, "v_zero")):
        _dev(t, n)
        if t.element_size() != 2:
            raise ValueError(f"{n} must hold binary16 values (float16 or int16)")
    B, Hkv, src_cap, D = src_k.shape
    cap = k_codes.shape[2]
    _check(lib().vc_quantize_int4(B, Hkv, D, _ptr(src_k), _ptr(src_v), src_cap, _ptr(src_start), int(n_groups), cap,
                                  _ptr(dst_start), _ptr(k_codes), _ptr(k_scale), _ptr(k_zero), _ptr(v_codes),
                                  _ptr(v_scale), _ptr(v_zero), _stream(stream)))


def compact_kv(src_k, src_v, idx, n_kept, dst_k, dst_v, dst_len=None, stream=None):
    """Eviction compaction (``vc_compact_kv``): row j < n_kept[b] of the
    compacted cache is row ``idx[b][j]`` of the full cache, for every KV head.

    ``src_k [B][Hkv][src_cap][D]``, ``src_v [B][Hkv][D][src_cap]`` (a full
    cache); ``idx`` int32 ``[B][stride]``, ``n_kept`` int32 ``[B]``;
    ``dst_k [B][Hkv][cap][D]``, ``dst_v [B][Hkv][cap/32][D][32]`` (the draft
    main segment); ``dst_len`` int32 ``[B][Hkv]`` or None.
    """
    for t, n in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        _dev(t, n, src_k.dtype)
    _dev(idx, "idx", torch.int32)
    _dev(n_kept, "n_kept", torch.int32)
    _dev(dst_len, "dst_len", torch.int32)
    B, Hkv, src_cap, D = src_k.shape
    cap = dst_k.shape[2]
    if tuple(src_v.shape) != (B, Hkv, D, src_cap) or tuple(dst_v.shape) != (B, Hkv, cap // 32, D, 32):
        raise ValueError("src_v must be [B][Hkv][D][src_cap] and dst_v [B][Hkv][cap/32][D][32]")
    if idx.dim() != 2 or idx.shape[0] != B or n_kept.numel() < B:
        raise ValueError("idx must be [B][stride] and n_kept [B]")
    if dst_len is not None and dst_len.numel() < B * Hkv:
        raise ValueError("dst_len must hold B * Hkv entries")
    _check(lib().vc_compact_kv(B, Hkv, D, _vc_dtype(src_k), _ptr(src_k), _ptr(src_v), src_cap, _ptr(idx),
                               idx.shape[1], _ptr(n_kept), _ptr(dst_k), _ptr(dst_v), cap, _ptr(dst_len),
                               _stream(stream)))


def quantize_int4_packed(src_k, src_v, src_start, n_groups, dst_start, packed, stream=None):
    """:func:`quantize_int4` into a packed int4 cache (``vc_quantize_int4_packed``):
    ``packed [B][Hkv][cap/32][5120]`` uint8, one interleaved block per 32 tokens
    (K codes, V codes, K scales, K zeros, V scales, V zeros)."""
    _dev(src_k, "src_k", torch.bfloat16)
    _dev(src_v, "src_v", torch.bfloat16)
    _dev(src_start, "src_start", torch.int32)
    _dev(dst_start, "dst_start", torch.int32)
    _dev(packed, "packed", torch.uint8)
    if packed.dim() != 4 or packed.shape[3] != INT4_PACKED_BLOCK:
        raise ValueError("a packed int4 cache is [B][Hkv][cap/32][5120] uint8")
    B, Hkv, src_cap, D = src_k.shape
    cap = packed.shape[2] * 32
    _check(lib().vc_quantize_int4_packed(B, Hkv, D, _ptr(src_k), _ptr(src_v), src_cap, _ptr(src_start),
                                         int(n_groups), cap, _ptr(dst_start), _ptr(packed), _stream(stream)))


def int4_commit(blk_k, blk_v, n_out, tail_k, tail_v, tail_len, packed, main_len, stream=None):
    """Commit verified rows into a packed int4 cache through its bf16 tail
    (``vc_int4_commit``): ``blk_k [B][Hkv][M][D]``, ``blk_v [B][Hkv][D][M]``,
    ``n_out`` int32 ``[B]``, ``tail_k [B][Hkv][tcap][D]``, ``tail_v
    [B][Hkv][D][tcap]`` (bf16), ``tail_len`` int32 ``[B]`` (in/out),
    ``packed [B][Hkv][cap/32][5120]`` uint8, ``main_len`` int32 ``[B][Hkv]``
    (in/out)."""
    if blk_k.dim() != 4 or tail_k.dim() != 4 or packed.dim() != 4:
        raise ValueError("blk_k, tail_k and packed are 4-dimensional")
    B, Hkv, M, D = blk_k.shape
    tcap = tail_k.shape[2]
    bf = (torch.bfloat16,)
    _want(blk_k, "blk_k", (B, Hkv, M, D), bf)
    _want(blk_v, "blk_v", (B, Hkv, D, M), bf)
    _want(n_out, "n_out", (B,), (torch.int32,))
    _want(tail_k, "tail_k", (B, Hkv, tcap, D), bf)
    _want(tail_v, "tail_v", (B, Hkv, D, tcap), bf)
    _want(tail_len, "tail_len", (B,), (torch.int32,))
    _want(packed, "packed", (B, Hkv, packed.shape[2], INT4_PACKED_BLOCK), (torch.uint8,))
    _want(main_len, "main_len", (B, Hkv), (torch.int32,))
    for t, n in ((blk_k, "blk_k"), (blk_v, "blk_v"), (n_out, "n_out"), (tail_k, "tail_k"), (tail_v, "tail_v"),
                 (tail_len, "tail_len"), (packed, "packed"), (main_len, "main_len")):
        _dev(t, n)
    _check(lib().vc_int4_commit(B, Hkv, D, M, _ptr(blk_k), _ptr(blk_v), _ptr(n_out), _ptr(tail_k), _ptr(tail_v), tcap,
                                _ptr(tail_len), _ptr(packed), packed.shape[2] * 32, _ptr(main_len), _stream(stream)))


def csm_round(in_k, in_v, n_in, n_sink, n_recent, chunk, r, out_k, out_v, out_deg, in_deg=None, out_len=None,
              stream=None):
    """One Chunked Soft Matching round (``vc_csm_round``); returns the survivor count.

    ``in_k [B][Hkv][cap_in][D]``, ``in_v [B][Hkv][cap_in/32][D][32]`` bf16,
    ``in_deg [B][Hkv][cap_in]`` float32 or None; outputs in the same layouts with
    ``cap_out``; ``out_deg [B][Hkv][cap_out]`` float32; ``out_len`` int32
    ``[B][Hkv]`` (optional) receives the survivor count on the device.
    """
    _dev(in_k, "in_k", torch.bfloat16)
    _dev(in_v, "in_v", torch.bfloat16)
    _dev(out_k, "out_k", torch.bfloat16)
    _dev(out_v, "out_v", torch.bfloat16)
    _dev(out_deg, "out_deg", torch.float32)
    _dev(in_deg, "in_deg", torch.float32)
    _dev(out_len, "out_len", torch.int32)
    B, Hkv, cap_in, D = in_k.shape
    cap_out = out_k.shape[2]
    _want(in_v, "in_v", (B, Hkv, cap_in // 32, D, 32), (torch.bfloat16,))
    _want(in_deg, "in_deg", (B, Hkv, cap_in), (torch.float32,))
    _want(out_k, "out_k", (B, Hkv, cap_out, D), (torch.bfloat16,))
    _want(out_v, "out_v", (B, Hkv, cap_out // 32, D, 32), (torch.bfloat16,))
    _want(out_deg, "out_deg", (B, Hkv, cap_out), (torch.float32,))
    _want(out_len, "out_len", (B, Hkv), (torch.int32,))
    n_out = _i32()
    _check(lib().vc_csm_round(B, Hkv, D, int(n_in), int(n_sink), int(n_recent), int(chunk), float(r), _ptr(in_k),
                              _ptr(in_v), _ptr(in_deg), cap_in, _ptr(out_k), _ptr(out_v), _ptr(out_deg),
                              cap_out, ctypes.byref(n_out), _ptr(out_len), _stream(stream)))
    return n_out.value


def csm_round_due(n_tokens, budget, decode_step, every):
    """Whether the CentroidKV schedule runs a round now (``vc_csm_round_due``)."""
    d = lib().vc_csm_round_due(int(n_tokens), int(budget), int(decode_step), int(every))
    if d < 0:
        raise ValueError("every must be >= 1 and decode_step >= 0")
    return bool(d)


def csm_schedule_ratio(r_init, delta_r, round_index):
    """Ratio of clustering round ``round_index`` (``vc_csm_schedule_ratio``)."""
    return lib().vc_csm_schedule_ratio(float(r_init), float(delta_r), int(round_index))


class Stagger:
    """Owner of the ``vc_stagger`` runtime object (copy streams, slot ring, events)."""

    def __init__(self, slots, slot_bytes, max_layers):
        arr = (_p * len(slots))(*[t.data_ptr() for t in slots])
        self._slots = slots
        h = _p()
        _check(lib().vc_stagger_create(ctypes.byref(h), arr, len(slots), slot_bytes, max_layers))
        self.h = h

    def stream_layer(self, layer, host_src, nbytes):
        _check(lib().vc_stagger_stream_layer(self.h, layer, _ptr(host_src), nbytes))

    def acquire(self, layer, stream):
        out = _p()
        _check(lib().vc_stagger_acquire(self.h, layer, _stream(stream), ctypes.byref(out)))
        return out.value

    def release(self, layer, stream):
        _check(lib().vc_stagger_release(self.h, layer, _stream(stream)))

    def writeback(self, host_dst, dev_src, nbytes, after):
        _check(lib().vc_stagger_writeback(self.h, _ptr(host_dst), _ptr(dev_src), nbytes, _stream(after)))

    def after(self, stream):
        _check(lib().vc_stagger_after(self.h, _stream(stream)))

    def sync(self):
        _check(lib().vc_stagger_sync(self.h))

    def round(self, layers, mode, lm_w, draft=None, step_tail_len=None, draft_hidden=None, drafts=None,
              draft_lm_ws=None, verify=None, host_kv=None, kv_bytes=0, v_offset=0, verify_hidden=None,
              verify_drafts=None, argmax=None, accept_len=None, out_tokens=None, n_out=None, verify_lm_ws=None,
              commit=None, before_verify=None, time_kernels=False, draft_stream=None, verify_stream=None,
              fetch=None):
        """One round of the staggered schedule (``vc_stagger_round``), enqueued
        natively on ``draft_stream`` / ``verify_stream`` and the copy streams.

        ``draft``: list over layers of :func:`draft_args` structs (the drafting
        cohort; None for none), ``step_tail_len``: list over the draft steps of
        int32 ``[Bd]`` tail lengths, ``draft_hidden``: list over the steps of
        bf16 ``[Bd][Dm]`` rows, ``drafts`` int32 ``[Bd][steps]``.  ``verify``:
        list over layers of :func:`verify_args` structs built with ``ccap``
        (the context comes from the slot), ``host_kv``: list of pinned uint8
        tensors (the layer's full K then V; V at ``v_offset``),
        ``verify_hidden`` bf16 ``[Bv][M][Dm]``, ``verify_drafts`` int32
        ``[Bv][M-1]`` and the acceptance outputs of :func:`lm_head_accept`.
        ``commit``: list over layers of dicts, either rows into a dense cache
        (``dst_k, dst_v, length, degree, v_blocked``) or, with ``int4=True``,
        rows into a packed int4 cache through its bf16 tail (``tail_k, tail_v,
        tail_len, packed, main_len``, as :func:`int4_commit`); both may add
        ``host_k, host_v`` (pinned write-back of the block rows).  ``before_verify(layer, stream_ptr)`` is
        called on the host before each verify is enqueued.  ``time_kernels``
        (:data:`TIME_DRAFT_STEPS` or True: each draft step's run of draft
        attention calls and every verify call; :data:`TIME_ATTENTION_KERNELS`:
        every draft and verify attention kernel alone, split merges excluded)
        records events read by :meth:`round_times`.  ``lm_w`` is the
        vocab-major ``[V][Dm]`` LM head.  ``fetch`` (chained mode): list of
        ``(host_src, dev_dst, layer)`` -- pinned host tensor, device tensor of
        the same byte size (a layer's compressed cache) -- copied over the link
        ahead of everything else, each layer's first draft call waiting for its
        copies (remote prefix caching).  Returns without synchronizing."""
        d = RoundDesc()
        keep = []
        if time_kernels is True or time_kernels is False:
            time_kernels = TIME_DRAFT_STEPS if time_kernels else TIME_NONE
        if time_kernels not in (TIME_NONE, TIME_DRAFT_STEPS, TIME_ATTENTION_KERNELS):
            raise ValueError(f"unknown timing mode {time_kernels!r}")
        d.layers, d.mode, d.time_kernels = int(layers), int(mode), int(time_kernels)
        _dev(lm_w, "lm_w", torch.bfloat16)
        d.lm_w, d.V, d.Dm = _ptr(lm_w), lm_w.shape[0], lm_w.shape[1]
        steps = 0
        if draft is not None:
            if len(draft) != layers or draft_hidden is None or drafts is None:
                raise ValueError("draft needs one struct per layer, draft_hidden and drafts")
            steps = len(draft_hidden)
            arr = (DraftArgs * layers)(*draft)
            keep.append(arr)
            d.draft = ctypes.cast(arr, ctypes.POINTER(DraftArgs))
            Bd = draft[0].B
            _dev(drafts, "drafts", torch.int32)
            _want(drafts, "drafts", (Bd, steps), (torch.int32,))
            for i, h in enumerate(draft_hidden):
                _dev(h, f"draft_hidden[{i}]", torch.bfloat16)
                _want(h, f"draft_hidden[{i}]", (Bd, d.Dm), (torch.bfloat16,))
            hid = (_p * steps)(*[h.data_ptr() for h in draft_hidden])
            keep.append(hid)
            d.draft_hidden = ctypes.cast(hid, ctypes.POINTER(_p))
            if step_tail_len is not None:
                if len(step_tail_len) != steps:
                    raise ValueError("step_tail_len needs one tensor per draft step")
                for i, t in enumerate(step_tail_len):
                    _dev(t, f"step_tail_len[{i}]", torch.int32)
                    _want(t, f"step_tail_len[{i}]", (Bd,), (torch.int32,))
                tl = (_p * steps)(*[t.data_ptr() for t in step_tail_len])
                keep.append(tl)
                d.step_tail_len = ctypes.cast(tl, ctypes.POINTER(_p))
            d.drafts = _ptr(drafts)
            if draft_lm_ws is None:
                draft_lm_ws = lm_head_argmax_workspace(Bd, d.V, drafts.device)
            keep.append(draft_lm_ws)
            d.draft_lm_ws, d.draft_lm_ws_bytes = _ptr(draft_lm_ws), draft_lm_ws.numel()
        d.steps = steps
        if verify is not None:
            if len(verify) != layers or host_kv is None or len(host_kv) != layers:
                raise ValueError("verify and host_kv need one entry per layer")
            arr = (VerifyArgs * layers)(*verify)
            keep.append(arr)
            d.verify = ctypes.cast(arr, ctypes.POINTER(VerifyArgs))
            for i, t in enumerate(host_kv):
                if t.is_cuda or not t.is_pinned():
                    raise ValueError(f"host_kv[{i}] must be pinned host memory")
                if t.numel() * t.element_size() < kv_bytes:
                    raise ValueError(f"host_kv[{i}] holds fewer than kv_bytes bytes")
            hk = (_p * layers)(*[t.data_ptr() for t in host_kv])
            keep.append(hk)
            d.host_kv = ctypes.cast(hk, ctypes.POINTER(_p))
            d.kv_bytes, d.v_offset = int(kv_bytes), int(v_offset)
            Bv, M = verify[0].B, verify[0].M
            _dev(verify_hidden, "verify_hidden", torch.bfloat16)
            _want(verify_hidden, "verify_hidden", (Bv, M, d.Dm), (torch.bfloat16,))
            _dev(verify_drafts, "verify_drafts", torch.int32)
            _want(verify_drafts, "verify_drafts", (Bv, M - 1), (torch.int32,))
            for t, n, shape in ((argmax, "argmax", (Bv, M)), (accept_len, "accept_len", (Bv,)),
                                (out_tokens, "out_tokens", (Bv, M)), (n_out, "n_out", (Bv,))):
                if t is None:
                    raise ValueError(f"{n} is required")
                _dev(t, n, torch.int32)
                _want(t, n, shape, (torch.int32,))
            d.verify_hidden, d.verify_drafts = _ptr(verify_hidden), _ptr(verify_drafts)
            d.argmax, d.accept_len, d.out_tokens, d.n_out = map(_ptr, (argmax, accept_len, out_tokens, n_out))
            if verify_lm_ws is None:
                verify_lm_ws = lm_head_argmax_workspace(Bv * M, d.V, verify_hidden.device)
            keep.append(verify_lm_ws)
            d.verify_lm_ws, d.verify_lm_ws_bytes = _ptr(verify_lm_ws), verify_lm_ws.numel()
            if commit is not None:
                if len(commit) != layers:
                    raise ValueError("commit needs one entry per layer")
                cs = (RoundCommit * layers)()
                for l, c in enumerate(commit):
                    vb = verify[l]
                    Bc, Hkv, D = vb.B, vb.Hkv, vb.D
                    blk_bytes = Bc * Hkv * vb.M * D * (2 if vb.dtype == VC_BF16 else 4)
                    for n in ("host_k", "host_v"):
                        t = c.get(n)
                        if t is not None and (t.is_cuda or not t.is_pinned()
                                              or t.numel() * t.element_size() < blk_bytes):
                            raise ValueError(f"commit[{l}].{n} must be pinned host memory of >= {blk_bytes} bytes")
                    cs[l].host_k, cs[l].host_v = _ptr(c.get("host_k")), _ptr(c.get("host_v"))
                    if c.get("int4"):
                        tk, tv, tl, pk, ml = c["tail_k"], c["tail_v"], c["tail_len"], c["packed"], c["main_len"]
                        tcap = tk.shape[2]
                        bf = (torch.bfloat16,)
                        _want(tk, f"commit[{l}].tail_k", (Bc, Hkv, tcap, D), bf)
                        _want(tv, f"commit[{l}].tail_v", (Bc, Hkv, D, tcap), bf)
                        _want(tl, f"commit[{l}].tail_len", (Bc,), (torch.int32,))
                        _want(pk, f"commit[{l}].packed", (Bc, Hkv, pk.shape[2], INT4_PACKED_BLOCK), (torch.uint8,))
                        _want(ml, f"commit[{l}].main_len", (Bc, Hkv), (torch.int32,))
                        for t, n in ((tk, "tail_k"), (tv, "tail_v"), (tl, "tail_len"), (pk, "packed"), (ml, "main_len")):
                            _dev(t, f"commit[{l}].{n}")
                        cs[l].kind = COMMIT_INT4_TAIL
                        cs[l].tail_k, cs[l].tail_v, cs[l].tcap = _ptr(tk), _ptr(tv), tcap
                        cs[l].tail_len, cs[l].packed, cs[l].main_len = _ptr(tl), _ptr(pk), _ptr(ml)
                        cs[l].cap = pk.shape[2] * 32
                        continue
                    dk, dv, ln, deg = c["dst_k"], c["dst_v"], c["length"], c.get("degree")
                    blocked = bool(c.get("v_blocked", False))
                    cap = dk.shape[2]
                    want_dt = torch.bfloat16 if vb.dtype == VC_BF16 else torch.float32
                    _want(dk, f"commit[{l}].dst_k", (Bc, Hkv, cap, D), (want_dt,))
                    _want(dv, f"commit[{l}].dst_v", (Bc, Hkv, cap // 32, D, 32) if blocked else (Bc, Hkv, D, cap),
                          (want_dt,))
                    _want(ln, f"commit[{l}].length", (Bc, Hkv), (torch.int32,))
                    if deg is not None:
                        if deg.dim() != 3 or deg.shape[1] not in (1, Hkv):
                            raise ValueError(f"commit[{l}].degree must be [B][1 or Hkv][cap]")
                        _want(deg, f"commit[{l}].degree", (Bc, deg.shape[1], cap), (torch.float32,))
                    for t, n in ((dk, "dst_k"), (dv, "dst_v"), (ln, "length"), (deg, "degree")):
                        _dev(t, f"commit[{l}].{n}")
                    cs[l].kind = COMMIT_ROWS
                    cs[l].dst_k, cs[l].dst_v, cs[l].len = _ptr(dk), _ptr(dv), _ptr(ln)
                    cs[l].degree = _ptr(deg)
                    cs[l].degree_h_stride = 0 if deg is None or deg.shape[1] == 1 else cap
                    cs[l].cap, cs[l].dst_v_blocked = cap, 1 if blocked else 0
                keep.append(cs)
                d.commit = ctypes.cast(cs, ctypes.POINTER(RoundCommit))
        if fetch:
            fs = (RoundFetch * len(fetch))()
            for j, (hsrc, ddst, layer) in enumerate(fetch):
                if hsrc.is_cuda or not hsrc.is_pinned():
                    raise ValueError(f"fetch[{j}] source must be pinned host memory")
                _dev(ddst, f"fetch[{j}] destination")
                nb = hsrc.numel() * hsrc.element_size()
                if ddst.numel() * ddst.element_size() != nb:
                    raise ValueError(f"fetch[{j}]: source and destination sizes differ")
                fs[j].host_src, fs[j].dev_dst, fs[j].bytes, fs[j].layer = hsrc.data_ptr(), ddst.data_ptr(), nb, int(layer)
            keep.append(fs)
            d.fetch, d.n_fetch = ctypes.cast(fs, ctypes.POINTER(RoundFetch)), len(fetch)
        if before_verify is not None:
            hook = ROUND_HOOK(lambda ctx, layer, stream: before_verify(int(layer), stream))
            keep.append(hook)
            d.before_verify = hook
        _check(lib().vc_stagger_round(self.h, ctypes.byref(d), _stream(draft_stream), _stream(verify_stream)))
        return keep

    def round_times(self):
        """(draft_ms, verify_ms) of the last timed round, once it completed:
        per draft step and per verify layer (TIME_DRAFT_STEPS), or per draft
        kernel, step-major, and per verify kernel (TIME_ATTENTION_KERNELS)."""
        nd, nv = _i32(), _i32()
        _check(lib().vc_stagger_round_times(self.h, None, ctypes.byref(nd), None, ctypes.byref(nv)))
        dm = (ctypes.c_float * max(nd.value, 1))()
        vm = (ctypes.c_float * max(nv.value, 1))()
        _check(lib().vc_stagger_round_times(self.h, dm, ctypes.byref(nd), vm, ctypes.byref(nv)))
        return list(dm)[:nd.value], list(vm)[:nv.value]

    def copy_ms(self, layer):
        ms = ctypes.c_float()
        _check(lib().vc_stagger_copy_ms(self.h, layer, ctypes.byref(ms)))
        return ms.value

    def close(self):
        if self.h:
            lib().vc_stagger_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

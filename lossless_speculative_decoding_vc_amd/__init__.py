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
    "argmax", "lm_head", "commit_rows", "quantize_int4", "csm_round", "Stagger",
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
        L.vc_draft_workspace_size.argtypes = [ctypes.POINTER(DraftArgs)]
        L.vc_draft_workspace_size.restype = ctypes.c_size_t
        L.vc_verify_workspace_size.argtypes = [ctypes.POINTER(VerifyArgs)]
        L.vc_verify_workspace_size.restype = ctypes.c_size_t
        L.vc_argmax.argtypes = [_i32, _i32, _i32, _p, _p, _i32, _p]
        L.vc_argmax.restype = ctypes.c_int
        L.vc_lm_head.argtypes = [_i32, _i32, _i32, _p, _p, _p, _p]
        L.vc_lm_head.restype = ctypes.c_int
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
        L.vc_quantize_int4_packed.restype = ctypes.c_int
        L.vc_csm_round.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _p, _p, _i64,
                                   _p, _p, _p, _i64, ctypes.POINTER(_i32), _p]
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
        for n in ("vc_stagger_create", "vc_stagger_stream_layer", "vc_stagger_acquire", "vc_stagger_release",
                  "vc_stagger_writeback", "vc_stagger_after", "vc_stagger_sync", "vc_stagger_copy_ms",
                  "vc_stagger_destroy"):
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
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (tail_k, "tail_k"), (tail_v, "tail_v"),
                 (out, "out"), (degree, "degree"), (out_lse, "out_lse"), (k_scale, "k_scale"),
                 (k_zero, "k_zero"), (v_scale, "v_scale"), (v_zero, "v_zero")):
        _dev(t, n)
    _dev(main_len, "main_len", torch.int32)
    _dev(tail_len, "tail_len", torch.int32)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    cap = k.shape[2]
    if fmt == VC_KV_INT4_PACKED:   # k is [B][Hkv][cap/32][5120] uint8
        if k.dim() != 4 or k.shape[3] != INT4_PACKED_BLOCK:
            raise ValueError("a packed int4 cache is [B][Hkv][cap/32][5120] uint8")
        cap = k.shape[2] * 32
    if out is None:
        out = torch.empty_like(q)
    a = _draft_struct(q, k, v, main_len, degree, tail_k, tail_v, tail_len, out, out_lse,
                      scale, num_splits, fmt, k_scale, k_zero, v_scale, v_zero, Hkv, cap)
    need = lib().vc_draft_workspace_size(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib().vc_draft_attn(ctypes.byref(a), _stream(stream)))
    return out


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
    for t, n in ((q, "q"), (ctx_k, "ctx_k"), (ctx_v, "ctx_v"), (blk_k, "blk_k"),
                 (blk_v, "blk_v"), (out, "out"), (out_lse, "out_lse")):
        _dev(t, n)
    _dev(ctx_len, "ctx_len", torch.int32)
    B, M, Hq, D = q.shape
    Hkv = blk_k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    a = VerifyArgs()
    a.B, a.Hq, a.Hkv, a.D, a.M = B, Hq, Hkv, D, M
    a.dtype = _vc_dtype(q)
    a.scale = D ** -0.5 if scale is None else scale
    a.num_splits = num_splits
    a.ccap = 0 if ctx_k is None else ctx_k.shape[2]
    a.q, a.ctx_k, a.ctx_v, a.ctx_len = _ptr(q), _ptr(ctx_k), _ptr(ctx_v), _ptr(ctx_len)
    a.blk_k, a.blk_v, a.out, a.out_lse = _ptr(blk_k), _ptr(blk_v), _ptr(out), _ptr(out_lse)
    need = lib().vc_verify_workspace_size(ctypes.byref(a))
    if need:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check(lib().vc_verify_attn(ctypes.byref(a), _stream(stream)))
    return out


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


def lm_head(h, w, logits=None, stream=None):
    """``logits [R][V] (fp32) = h [R][Dm] (bf16) @ w [Dm][V] (bf16)`` (``vc_lm_head``)."""
    _dev(h, "h", torch.bfloat16)
    _dev(w, "w", torch.bfloat16)
    R, Dm = h.shape
    V = w.shape[1]
    if logits is None:
        logits = torch.empty((R, V), dtype=torch.float32, device=h.device)
    _dev(logits, "logits", torch.float32)
    _check(lib().vc_lm_head(R, Dm, V, _ptr(h), _ptr(w), _ptr(logits), _stream(stream)))
    return logits


def lm_head_argmax_workspace(R, V, device):
    """Workspace tensor (uint8) for :func:`lm_head_argmax` over R rows."""
    n = lib().vc_lm_head_argmax_workspace_size(R, V)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


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
    for t, n in ((blk_k, "blk_k"), (blk_v, "blk_v"), (dst_k, "dst_k"), (dst_v, "dst_v"), (degree, "degree")):
        _dev(t, n)
    _dev(n_out, "n_out", torch.int32)
    _dev(length, "length", torch.int32)
    B, Hkv, M, D = blk_k.shape
    cap = dst_k.shape[2]
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


def csm_round(in_k, in_v, n_in, n_sink, n_recent, chunk, r, out_k, out_v, out_deg, in_deg=None, stream=None):
    """One Chunked Soft Matching round (``vc_csm_round``); returns the survivor count.

    ``in_k [B][Hkv][cap_in][D]``, ``in_v [B][Hkv][cap_in/32][D][32]`` bf16,
    ``in_deg [B][Hkv][cap_in]`` float32 or None; outputs in the same layouts with
    ``cap_out``; ``out_deg [B][Hkv][cap_out]`` float32.
    """
    _dev(in_k, "in_k", torch.bfloat16)
    _dev(in_v, "in_v", torch.bfloat16)
    _dev(out_k, "out_k", torch.bfloat16)
    _dev(out_v, "out_v", torch.bfloat16)
    _dev(out_deg, "out_deg", torch.float32)
    _dev(in_deg, "in_deg", torch.float32)
    B, Hkv, cap_in, D = in_k.shape
    n_out = _i32()
    _check(lib().vc_csm_round(B, Hkv, D, int(n_in), int(n_sink), int(n_recent), int(chunk), float(r), _ptr(in_k),
                              _ptr(in_v), _ptr(in_deg), cap_in, _ptr(out_k), _ptr(out_v), _ptr(out_deg),
                              out_k.shape[2], ctypes.byref(n_out), _stream(stream)))
    return n_out.value


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

"""Python binding of libfa.so, the gfx950 fused exact-attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/fa.h.  PyTorch supplies device memory and
the current HIP stream.  There is no fallback: if libfa.so is missing or the
tensors are not on the GPU, the calls raise.

Low-level functions carry the C names (``fa_fwd``, ``fa_bwd``, ...) and take
torch tensors; ``forward`` / ``backward`` allocate their outputs (on the
stream they launch on, so that the caching allocator does not hand their
memory to other work while the kernels still use it).  Tuning options go
with each call as an ``Options`` value (None = the library defaults).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 16 << 20  # FA_NOALLOC_SCRATCH_BYTES of include/fa.h
# backward(): most bytes of stored dS it allocates (8 GiB: four heads at S = 32768, which keeps
# the speed of the single launch); beyond that the heads run in groups
STORED_DS_WORKSPACE_CAP = 8 << 30

_lib = None


class Options(ctypes.Structure):
    """Per-call tuning options (struct fa_options of include/fa.h)."""
    _fields_ = [("rescale_tau", ctypes.c_float), ("poly_eighths", ctypes.c_int),
                ("poly_degree", ctypes.c_int), ("longest_first", ctypes.c_int), ("fused_backward", ctypes.c_int),
                ("stored_ds", ctypes.c_int)]

    def __init__(self, rescale_tau: float = 8.0, poly_eighths: int = 0, poly_degree: int = 3,
                 longest_first: bool = True, fused_backward: bool = False, stored_ds: bool = False):
        super().__init__(float(rescale_tau), int(poly_eighths), int(poly_degree), int(bool(longest_first)),
                         int(bool(fused_backward)), int(bool(stored_ds)))

    def __repr__(self):
        return (f"Options(rescale_tau={self.rescale_tau}, poly_eighths={self.poly_eighths}, "
                f"poly_degree={self.poly_degree}, longest_first={bool(self.longest_first)}, "
                f"fused_backward={bool(self.fused_backward)}, stored_ds={bool(self.stored_ds)})")


class FaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


def load_library():
    """Load libfa.so (built by exact_attention_39_amd.build).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_39_amd.build` "
                           "(the attention path has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    op = ctypes.POINTER(Options)
    lib.fa_default_options.argtypes = []
    lib.fa_default_options.restype = Options
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_opt.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, op, vp]
    lib.fa_fwd_opt.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, op, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes_opt.argtypes = [i, i, i, i, i, op]
    lib.fa_bwd_workspace_bytes_opt.restype = sz
    lib.fa_bwd_workspace_bytes_min.argtypes = [i, i, i, i, i, op]
    lib.fa_bwd_workspace_bytes_min.restype = sz
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_opt.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, op, vp, sz, vp]
    lib.fa_bwd_opt.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, op, vp, sz, vp]
    lib.fa_bwd_dkdv.restype = i
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, op, vp, sz, vp]
    lib.fa_bwd_dq.restype = i
    lib.fa_bwd_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_fused.restype = i
    lib.fa_exp2_poly.argtypes = [vp, vp, ctypes.c_int64, i, vp]
    lib.fa_exp2_poly.restype = i
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != FA_OK:
        raise FaError(code, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _opts(opts):
    """Options -> pointer argument (None -> NULL, the library defaults)."""
    if opts is None:
        return None
    if not isinstance(opts, Options):
        raise TypeError("opts must be an exact_attention_39_amd.Options or None")
    return ctypes.byref(opts)


def default_options() -> Options:
    return load_library().fa_default_options()


def _check_tensor(t, name, dtype, shape):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (the attention path has no CPU fallback)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(q):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, S, d]")
    return tuple(int(x) for x in q.shape)


# ------------------------------------------------------------------ C names
def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None, opts=None):
    import torch
    B, H, S, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_tensor(t, nm, torch.bfloat16, (B, H, S, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, S))
    _check(load_library().fa_fwd_opt(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, S, d,
                                     float(scale), int(bool(causal)), _opts(opts), _stream(stream)),
           "fa_fwd")


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen: int, scale: float, causal: bool, stream=None,
                  opts=None):
    """Packed variable-length forward: q, k, v, o bf16 [total, H, d]; lse fp32
    [H, total]; cu_seqlens int32 [nseq + 1] on the GPU."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [total, H, d]")
    total, H, d = (int(x) for x in q.shape)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_tensor(t, nm, torch.bfloat16, (total, H, d))
    _check_tensor(lse, "lse", torch.float32, (H, total))
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 offsets")
    _check_tensor(cu_seqlens, "cu_seqlens", torch.int32, tuple(cu_seqlens.shape))
    nseq = cu_seqlens.numel() - 1
    _check(load_library().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens),
                                        nseq, H, total, int(max_seqlen), d, float(scale),
                                        int(bool(causal)), _opts(opts), _stream(stream)), "fa_fwd_varlen")


def fa_bwd_workspace_bytes(B: int, H: int, S: int, d: int, causal: bool = False, opts=None) -> int:
    """Workspace bytes of a backward with these options (None = defaults)."""
    if opts is None:
        return int(load_library().fa_bwd_workspace_bytes(B, H, S, d))
    return int(load_library().fa_bwd_workspace_bytes_opt(B, H, S, d, int(bool(causal)), _opts(opts)))


def fa_bwd_workspace_bytes_min(B: int, H: int, S: int, d: int, causal: bool = False, opts=None) -> int:
    """The least workspace fa_bwd accepts with these options (stored dS: one
    head's dS; fa_bwd then takes the heads in groups)."""
    return int(load_library().fa_bwd_workspace_bytes_min(B, H, S, d, int(bool(causal)), _opts(opts)))


def _bwd_checks(q, k, v, o, lse, do, dq, dk, dv):
    import torch
    B, H, S, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (do, "do"), (dk, "dk"), (dv, "dv")):
        _check_tensor(t, nm, torch.bfloat16, (B, H, S, d))
    if o is not None:
        _check_tensor(o, "o", torch.bfloat16, (B, H, S, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, S))
    _check_tensor(dq, "dq", torch.float32, (B, H, S, d))
    return B, H, S, d


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool, workspace, stream=None, opts=None):
    B, H, S, d = _bwd_checks(q, k, v, o, lse, do, dq, dk, dv)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd_opt(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                     _ptr(dk), _ptr(dv), B, H, S, d, float(scale), int(bool(causal)),
                                     _opts(opts), _ptr(workspace), ws_bytes, _stream(stream)), "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool, stream=None):
    """fa_bwd with the library's static device workspace: allocates nothing.
    Calls that overlap on one GPU race on that workspace."""
    B, H, S, d = _bwd_checks(q, k, v, o, lse, do, dq, dk, dv)
    _check(load_library().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                         _ptr(dk), _ptr(dv), B, H, S, d, float(scale), int(bool(causal)),
                                         _stream(stream)), "fa_bwd_noalloc")


def fa_bwd_preprocess(o, do, lse, workspace, stream=None):
    import torch
    B, H, S, d = _dims(o)
    _check_tensor(o, "o", torch.bfloat16, (B, H, S, d))
    _check_tensor(do, "do", torch.bfloat16, (B, H, S, d))
    _check_tensor(lse, "lse", torch.float32, (B, H, S))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), B, H, S, d, _ptr(workspace),
                                            ws_bytes, _stream(stream)), "fa_bwd_preprocess")


def _grad_checks(q, k, v, do):
    import torch
    B, H, S, d = _dims(q)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
        _check_tensor(t, nm, torch.bfloat16, (B, H, S, d))
    return B, H, S, d


def fa_bwd_dkdv(q, k, v, do, dk, dv, scale: float, causal: bool, workspace, stream=None, opts=None):
    """dK, dV from the workspace that fa_bwd_preprocess filled on the same stream."""
    import torch
    B, H, S, d = _grad_checks(q, k, v, do)
    _check_tensor(dk, "dk", torch.bfloat16, (B, H, S, d))
    _check_tensor(dv, "dv", torch.bfloat16, (B, H, S, d))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
                                      B, H, S, d, float(scale), int(bool(causal)), _opts(opts), _ptr(workspace),
                                      ws_bytes, _stream(stream)), "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, do, dq, scale: float, causal: bool, workspace, stream=None, opts=None):
    """dQ from the workspace that fa_bwd_preprocess filled on the same stream."""
    import torch
    B, H, S, d = _grad_checks(q, k, v, do)
    _check_tensor(dq, "dq", torch.float32, (B, H, S, d))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), B, H, S, d,
                                    float(scale), int(bool(causal)), _opts(opts), _ptr(workspace), ws_bytes,
                                    _stream(stream)), "fa_bwd_dq")


def fa_bwd_fused(q, k, v, do, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    """dQ, dK, dV in one pass (the single-pass backward) from the workspace
    that fa_bwd_preprocess filled on the same stream."""
    import torch
    B, H, S, d = _grad_checks(q, k, v, do)
    _check_tensor(dq, "dq", torch.float32, (B, H, S, d))
    _check_tensor(dk, "dk", torch.bfloat16, (B, H, S, d))
    _check_tensor(dv, "dv", torch.bfloat16, (B, H, S, d))
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().fa_bwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                                       B, H, S, d, float(scale), int(bool(causal)), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "fa_bwd_fused")


def fa_exp2_poly(x, y, degree: int = 3, stream=None):
    import torch
    _check_tensor(x, "x", torch.float32, tuple(x.shape))
    _check_tensor(y, "y", torch.float32, tuple(x.shape))
    _check(load_library().fa_exp2_poly(_ptr(x), _ptr(y), x.numel(), int(degree), _stream(stream)),
           "fa_exp2_poly")


# ------------------------------------------------------------------ allocating wrappers
def _launch_stream(stream, *tensors):
    """The stream the kernels go on; the tensors are checked to be on the GPU
    first, so that a CPU tensor gets the clear error rather than a stream
    lookup failure."""
    import torch
    for t in tensors:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError("inputs must be torch tensors on the GPU (the attention path has no CPU fallback)")
    return torch.cuda.current_stream() if stream is None else stream


def forward(q, k, v, causal: bool = False, scale: float | None = None, stream=None, opts=None):
    """(O bf16 [B,H,S,d], LSE fp32 [B,H,S]) for bf16 q, k, v on the GPU.
    The outputs are allocated on the launch stream."""
    import torch
    B, H, S, d = _dims(q)
    scale = d ** -0.5 if scale is None else scale
    s = _launch_stream(stream, q, k, v)
    with torch.cuda.stream(s):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, causal, s, opts)
    return o, lse


def forward_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
                   stream=None, opts=None):
    """(O bf16 [total, H, d], LSE fp32 [H, total]) for a packed batch of
    sequences delimited by cu_seqlens (int32 [nseq + 1] on the GPU)."""
    import torch
    total, H, d = (int(x) for x in q.shape)
    scale = d ** -0.5 if scale is None else scale
    s = _launch_stream(stream, q, k, v, cu_seqlens)
    with torch.cuda.stream(s):
        o = torch.empty_like(q)
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, causal, s, opts)
    return o, lse


def backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, stream=None, opts=None):
    """(dQ fp32, dK bf16, dV bf16) for the O, LSE that ``forward`` returned.
    Outputs and the workspace are allocated on the launch stream: the
    workspace returns to that stream's pool when this function returns, so
    later allocations on it are ordered after the kernels that read it.
    With ``Options(stored_ds=True)`` the workspace also holds dS: about
    2*B*H*S*S bytes (half that causal), capped at STORED_DS_WORKSPACE_CAP
    bytes (but at least one head's dS), beyond which the heads run in groups."""
    import torch
    B, H, S, d = _dims(q)
    scale = d ** -0.5 if scale is None else scale
    s = _launch_stream(stream, q, k, v, o, lse, do)
    with torch.cuda.stream(s):
        dq = torch.empty((B, H, S, d), dtype=torch.float32, device=q.device)
        dk = torch.empty_like(q)
        dv = torch.empty_like(q)
        ws_bytes = fa_bwd_workspace_bytes(B, H, S, d, causal, opts)
        if opts is not None and opts.stored_ds:
            ws_bytes = min(ws_bytes, max(fa_bwd_workspace_bytes_min(B, H, S, d, causal, opts),
                                         fa_bwd_workspace_bytes(B, H, S, d) + STORED_DS_WORKSPACE_CAP))
        ws = torch.empty(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device=q.device)
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, scale, causal, ws, s, opts)
    return dq, dk, dv

"""ctypes binding over the C-ABI library (``include/fa.h``).

Argument marshalling only: each function checks the torch tensors it is
given, allocates outputs with torch on the inputs' device, and passes raw
device pointers plus the current HIP stream to the entry point of the same
name.  Every step of the computation runs in the library's HIP kernels.  If
the library has not been built, every call raises; there is no fallback.
"""

import ctypes
import math
import os

import torch

from . import _build

__all__ = [
    "FAError", "fa_fwd", "fa_fwd_blocksparse", "fa_fwd_splitkv",
    "fa_fwd_splitkv_chunks", "fa_fwd_splitkv_workspace_bytes", "fa_bwd",
    "fa_bwd_blocksparse", "fa_bwd_noalloc", "fa_bwd_preprocess",
    "fa_bwd_dkdv", "fa_bwd_dq", "fa_bwd_dq_stats", "fa_bwd_workspace_bytes",
    "fa_status_str",
    "fa_tile_grid", "fa_fwd_tile_visits", "fa_bwd_tile_visits",
    "fa_version", "library", "LIB_PATH",
]

LIB_PATH = _build.LIB_PATH
FA_F32, FA_BF16 = 0, 1
FA_ERR_HIP = 6

_lib = None


class FAError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def library():
    """The loaded ctypes library (loaded once; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP attention library not built ({LIB_PATH} missing); run "
            "__graft_entry__.build() first. There is no fallback path.")
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declare(lib):
    """Set the argument and result types of every entry point of a loaded
    library (the signatures of include/fa.h); returns it."""
    P, I64, F, I, SZ, U64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64)
    sigs = {
        "fa_fwd": [P, P, P, P, P, I64, I64, I64, I64, I, F, I, P],
        "fa_fwd_blocksparse": [P, P, P, P, P, I64, I64, I64, I64, I, F, I, P,
                               I64, I64, P],
        "fa_fwd_splitkv": [P, P, P, P, P, P, SZ, I64, I64, I64, I64, I64, I,
                           F, I, I64, P],
        "fa_bwd": [P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I64, I64, I, F,
                   I, P],
        "fa_bwd_blocksparse": [P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I64,
                               I64, I, F, I, P, I64, I64, P],
        "fa_bwd_preprocess": [P, P, P, P, SZ, I64, I64, I64, I64, I, P],
        "fa_bwd_dkdv": [P, P, P, P, P, P, P, SZ, I64, I64, I64, I64, I, F, I,
                        P],
        "fa_bwd_dq": [P, P, P, P, P, P, SZ, I64, I64, I64, I64, I, F, I, P],
        "fa_bwd_dq_stats": [P, P, P, P, P, P, P, P, SZ, I64, I64, I64, I64, I,
                            F, I, P],
        "fa_fwd_dropout": [P, P, P, P, P, I64, I64, I64, I64, I, F, I, F, U64,
                           P],
        "fa_bwd_dropout": [P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I64,
                           I64, I, F, I, F, U64, P],
        "fa_bwd_noalloc": [P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I,
                           F, I, P],
        "fa_fwd_general": [P, P, P, P, P, I64, I64, I64, I64, I64, I, F, I,
                           P, I64, I64, F, U64, P],
        "fa_bwd_general": [P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I64,
                           I64, I64, I, F, I, P, I64, I64, F, U64, P],
        "fa_tile_grid": [I, I64, I, P, P],
        "fa_fwd_tile_visits": [P, P, P, P, P, I64, I64, I64, I64, I, F, I, P,
                               I64, I64, P, SZ, P],
        "fa_bwd_tile_visits": [P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I64,
                               I64, I, F, I, P, I64, I64, P, SZ, P, SZ, P],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.fa_bwd_workspace_bytes.argtypes = [I64, I64, I64, I64]
    lib.fa_bwd_workspace_bytes.restype = SZ
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [I64] * 6
    lib.fa_fwd_splitkv_workspace_bytes.restype = SZ
    lib.fa_fwd_splitkv_chunks.argtypes = [I64] * 6
    lib.fa_fwd_splitkv_chunks.restype = I64
    lib.fa_status_str.argtypes = [I]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    return lib


def fa_status_str(status):
    return library().fa_status_str(int(status)).decode()


def fa_version():
    return library().fa_version().decode()


def _check(status):
    if status != 0:
        raise FAError(status, fa_status_str(status))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _shape4(*ts):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("tensors must be B x H x N x d")
    for t in ts:
        if t.shape != ref.shape:
            raise ValueError(f"shape mismatch {tuple(t.shape)} vs {tuple(ref.shape)}")
        if t.dtype != ref.dtype:
            raise ValueError("all of Q, K, V (, O, dO) must share one dtype")
        if t.device != ref.device or t.device.type != "cuda":
            raise ValueError("tensors must be on the same GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (d fastest)")
    return tuple(ref.shape)


def _arg(t, name, shape, dtype, device):
    """Check a caller-supplied tensor that the kernels read or write: exact
    shape, dtype, device and contiguity (the library trusts its sizes)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got "
                         f"{tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ws_arg(ws, device):
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the "
                         "inputs' device")
    return ws, ws.numel() * ws.element_size()


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fa_fwd(q, k, v, scale=None, causal=False, out=None, lse=None):
    """O, LSE = attention(q, k, v); q, k, v are B x H x N x d bf16 or fp32."""
    B, H, N, d = _shape4(q, k, v)
    lib = library()
    o, lse_t = _fwd_outputs(q, (B, H, N, d), out, lse)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B,
                          H, N, d, _dtype_code(q), _scale(scale, d),
                          int(bool(causal)), _stream(q.device)))
    return o, lse_t


def _fwd_outputs(q, shape, out, lse):
    """O (shape, q's dtype) and LSE (shape[:-1], float32): allocated, or the
    caller's tensors after checking them."""
    if out is None:
        out = torch.empty(shape, dtype=q.dtype, device=q.device)
    else:
        _arg(out, "out", shape, q.dtype, q.device)
    if lse is None:
        lse = torch.empty(shape[:-1], dtype=torch.float32, device=q.device)
    else:
        _arg(lse, "lse", shape[:-1], torch.float32, q.device)
    return out, lse


def _grads(q, dq, dk, dv):
    """dQ, dK, dV (float32, q's shape): allocated, or checked."""
    res = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        else:
            _arg(t, name, q.shape, torch.float32, q.device)
        res.append(t)
    return res


def _mask_arg(block_mask, N, block_m, block_n, device, Nk=None):
    """The block mask as a contiguous uint8 device tensor (or None); its
    shape is ceil(N / block_m) x ceil(Nk / block_n), Nk = N by default."""
    if block_mask is None:
        return None
    rows = -(-N // int(block_m))
    cols = -(-(N if Nk is None else Nk) // int(block_n))
    if tuple(block_mask.shape) != (rows, cols):
        raise ValueError(f"block mask must be {rows} x {cols}, got "
                         f"{tuple(block_mask.shape)}")
    if block_mask.device != device:
        raise ValueError("block mask must be on the inputs' device")
    return block_mask.to(torch.uint8).contiguous()


def fa_fwd_blocksparse(q, k, v, block_mask, block_m=128, block_n=128,
                       scale=None, causal=False, out=None, lse=None):
    """Forward over the nonzero blocks of ``block_mask`` only.

    ``block_mask`` is a uint8 (or bool) tensor of shape
    (ceil(N / block_m), ceil(N / block_n)) on the inputs' device, or None for
    a dense mask.
    """
    B, H, N, d = _shape4(q, k, v)
    lib = library()
    mask_t = _mask_arg(block_mask, N, block_m, block_n, q.device)
    o, lse_t = _fwd_outputs(q, (B, H, N, d), out, lse)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_blocksparse(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
            _dtype_code(q), _scale(scale, d), int(bool(causal)),
            _ptr(mask_t), int(block_m), int(block_n), _stream(q.device)))
    return o, lse_t


def fa_fwd_splitkv_chunks(B, H, Nq, Nk, d, n_splits=0):
    """Number of key chunks fa_fwd_splitkv uses (0 for empty/invalid)."""
    return int(library().fa_fwd_splitkv_chunks(B, H, Nq, Nk, d, n_splits))


def fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits=0):
    return int(library().fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d,
                                                        n_splits))


def fa_fwd_splitkv(q, k, v, scale=None, causal=False, n_splits=0,
                   workspace=None, out=None, lse=None):
    """Split-KV forward: q is B x H x Nq x d, k and v B x H x Nk x d (bf16).

    The queries are the last Nq positions of the key sequence (causal: query
    i sees keys j <= Nk - Nq + i).  ``n_splits`` caps the number of key
    chunks (0 = automatic).  Returns O (B x H x Nq x d) and LSE (B x H x Nq).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("tensors must be B x H x N x d")
    B, H, Nq, d = q.shape
    Bk, Hk, Nk, dk = k.shape
    if (Bk, Hk, dk) != (B, H, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k "
                         f"{tuple(k.shape)} v {tuple(v.shape)}")
    for t in (q, k, v):
        if t.dtype != q.dtype:
            raise ValueError("all of Q, K, V must share one dtype")
        if t.device != q.device or t.device.type != "cuda":
            raise ValueError("tensors must be on the same GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (d fastest)")
    lib = library()
    need = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8,
                                device=q.device)
    workspace, ws_bytes = _ws_arg(workspace, q.device)
    o, lse_t = _fwd_outputs(q, (B, H, Nq, d), out, lse)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_splitkv(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), _ptr(workspace),
            ws_bytes, B, H, Nq, Nk, d, _dtype_code(q), _scale(scale, d),
            int(bool(causal)), int(n_splits), _stream(q.device)))
    return o, lse_t


def fa_bwd_workspace_bytes(B, H, N, d):
    return int(library().fa_bwd_workspace_bytes(B, H, N, d))


def _workspace(B, H, N, d, device, workspace):
    need = fa_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    return _ws_arg(workspace, device)


def fa_bwd(q, k, v, o, do, lse, scale=None, causal=False, workspace=None,
           dq=None, dk=None, dv=None):
    """dQ, dK, dV (float32) of L = sum(O * dO), recomputing P from lse."""
    B, H, N, d = _shape4(q, k, v, o, do)
    lib = library()
    _arg(lse, "lse", (B, H, N), torch.float32, q.device)
    dq, dk, dv = _grads(q, dq, dk, dv)
    ws, ws_bytes = _workspace(B, H, N, d, q.device, workspace)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                          _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                          ws_bytes, B, H, N, d, _dtype_code(q),
                          _scale(scale, d), int(bool(causal)),
                          _stream(q.device)))
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale=None,
                   causal=False):
    """fa_bwd without a workspace: the library's own scratch holds the
    per-row values (B*H*N <= 2^20).  The caller passes the output tensors
    dq, dk, dv (float32, q's shape); nothing is allocated."""
    B, H, N, d = _shape4(q, k, v, o, do)
    lib = library()
    _arg(lse, "lse", (B, H, N), torch.float32, q.device)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _arg(t, name, q.shape, torch.float32, q.device)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                  _ptr(dv), B, H, N, d, _dtype_code(q),
                                  _scale(scale, d), int(bool(causal)),
                                  _stream(q.device)))
    return dq, dk, dv


def fa_fwd_dropout(q, k, v, p_drop, seed, scale=None, causal=False, out=None,
                   lse=None):
    """O, LSE of attention with dropout on P (bf16 q, k, v): elements are
    dropped with probability round(256 p_drop) / 256 by the Philox mask of
    ``seed`` (a 64-bit integer) and survivors scaled by 1/(1-p); LSE is that
    of the undropped softmax."""
    B, H, N, d = _shape4(q, k, v)
    lib = library()
    o, lse_t = _fwd_outputs(q, (B, H, N, d), out, lse)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(lse_t), B, H, N, d, _dtype_code(q),
                                  _scale(scale, d), int(bool(causal)),
                                  float(p_drop), int(seed) & (2**64 - 1),
                                  _stream(q.device)))
    return o, lse_t


def fa_bwd_dropout(q, k, v, o, do, lse, p_drop, seed, scale=None,
                   causal=False, workspace=None, dq=None, dk=None, dv=None):
    """dQ, dK, dV (float32) of fa_fwd_dropout with the same p_drop and seed."""
    B, H, N, d = _shape4(q, k, v, o, do)
    lib = library()
    _arg(lse, "lse", (B, H, N), torch.float32, q.device)
    dq, dk, dv = _grads(q, dq, dk, dv)
    ws, ws_bytes = _workspace(B, H, N, d, q.device, workspace)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(ws), ws_bytes, B, H, N, d,
                                  _dtype_code(q), _scale(scale, d),
                                  int(bool(causal)), float(p_drop),
                                  int(seed) & (2**64 - 1), _stream(q.device)))
    return dq, dk, dv


def fa_bwd_blocksparse(q, k, v, o, do, lse, block_mask, block_m=128,
                       block_n=128, scale=None, causal=False, workspace=None,
                       dq=None, dk=None, dv=None):
    """Gradients of ``fa_fwd_blocksparse`` (same mask; o, lse from it)."""
    B, H, N, d = _shape4(q, k, v, o, do)
    lib = library()
    mask_t = _mask_arg(block_mask, N, block_m, block_n, q.device)
    _arg(lse, "lse", (B, H, N), torch.float32, q.device)
    dq, dk, dv = _grads(q, dq, dk, dv)
    ws, ws_bytes = _workspace(B, H, N, d, q.device, workspace)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_blocksparse(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes, B, H, N, d, _dtype_code(q),
            _scale(scale, d), int(bool(causal)), _ptr(mask_t), int(block_m),
            int(block_n), _stream(q.device)))
    return dq, dk, dv


def _qk_shapes(q, k, v, o=None, do=None):
    """(B, H, Nq, Nk, d) of a call with Nq query rows and Nk key rows:
    q (and o, do) B x H x Nq x d, k and v B x H x Nk x d, one dtype and
    device, contiguous."""
    B, H, Nk, d = _shape4(k, v)
    for name, t in (("q", q), ("o", o), ("do", do)):
        if t is None:
            continue
        if t.dim() != 4 or tuple(t.shape[:2]) != (B, H) or t.shape[3] != d:
            raise ValueError(f"{name} must be B x H x Nq x d with B, H, d of "
                             f"k; got {tuple(t.shape)}")
        if t.dtype != k.dtype or t.device != k.device:
            raise ValueError(f"{name} must share k's dtype and device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    Nq = q.shape[2]
    for name, t in (("o", o), ("do", do)):
        if t is not None and t.shape[2] != Nq:
            raise ValueError(f"{name} must have q's {Nq} rows")
    return B, H, Nq, Nk, d


def fa_fwd_general(q, k, v, scale=None, causal=False, block_mask=None,
                   block_m=128, block_n=128, p_drop=0.0, seed=0, out=None,
                   lse=None):
    """The forward with every option together: q is B x H x Nq x d, k and v
    B x H x Nk x d; under the causal rule the queries are the last Nq of the
    Nk tokens (query i sees key j iff j <= Nk - Nq + i); an optional block
    mask of shape (ceil(Nq / block_m), ceil(Nk / block_n)); dropout with
    probability round(256 p_drop) / 256 (bf16 only)."""
    B, H, Nq, Nk, d = _qk_shapes(q, k, v)
    lib = library()
    mask_t = _mask_arg(block_mask, Nq, block_m, block_n, q.device, Nk)
    o, lse_t = _fwd_outputs(q, (B, H, Nq, d), out, lse)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_general(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Nq, Nk, d,
            _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(mask_t),
            int(block_m), int(block_n), float(p_drop),
            int(seed) & (2**64 - 1), _stream(q.device)))
    return o, lse_t


def fa_bwd_general(q, k, v, o, do, lse, scale=None, causal=False,
                   block_mask=None, block_m=128, block_n=128, p_drop=0.0,
                   seed=0, workspace=None, dq=None, dk=None, dv=None):
    """dQ (B x H x Nq x d), dK and dV (B x H x Nk x d), float32, of
    ``fa_fwd_general`` with the same arguments (o, lse from it)."""
    B, H, Nq, Nk, d = _qk_shapes(q, k, v, o, do)
    lib = library()
    mask_t = _mask_arg(block_mask, Nq, block_m, block_n, q.device, Nk)
    _arg(lse, "lse", (B, H, Nq), torch.float32, q.device)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    else:
        _arg(dq, "dq", q.shape, torch.float32, q.device)
    dk, dv = (torch.empty(k.shape, dtype=torch.float32, device=q.device)
              if t is None else _arg(t, name, k.shape, torch.float32, q.device)
              for name, t in (("dk", dk), ("dv", dv)))
    ws, ws_bytes = _workspace(B, H, Nq, d, q.device, workspace)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_general(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes, B, H, Nq, Nk, d,
            _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(mask_t),
            int(block_m), int(block_n), float(p_drop),
            int(seed) & (2**64 - 1), _stream(q.device)))
    return dq, dk, dv


def fa_bwd_preprocess(o, do, lse, workspace):
    B, H, N, d = _shape4(o, do)
    _arg(lse, "lse", (B, H, N), torch.float32, o.device)
    workspace, ws_bytes = _ws_arg(workspace, o.device)
    with torch.cuda.device(o.device):
        _check(library().fa_bwd_preprocess(
            _ptr(o), _ptr(do), _ptr(lse), _ptr(workspace), ws_bytes, B, H, N,
            d, _dtype_code(o), _stream(o.device)))


def fa_bwd_dkdv(q, k, v, do, workspace, dk, dv, scale=None, causal=False):
    B, H, N, d = _shape4(q, k, v, do)
    _arg(dk, "dk", q.shape, torch.float32, q.device)
    _arg(dv, "dv", q.shape, torch.float32, q.device)
    workspace, ws_bytes = _ws_arg(workspace, q.device)
    with torch.cuda.device(q.device):
        _check(library().fa_bwd_dkdv(
            _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dk), _ptr(dv),
            _ptr(workspace), ws_bytes, B, H, N, d, _dtype_code(q),
            _scale(scale, d), int(bool(causal)), _stream(q.device)))


def fa_bwd_dq(q, k, v, do, workspace, dq, scale=None, causal=False):
    B, H, N, d = _shape4(q, k, v, do)
    _arg(dq, "dq", q.shape, torch.float32, q.device)
    workspace, ws_bytes = _ws_arg(workspace, q.device)
    with torch.cuda.device(q.device):
        _check(library().fa_bwd_dq(
            _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(workspace),
            ws_bytes, B, H, N, d, _dtype_code(q), _scale(scale, d),
            int(bool(causal)), _stream(q.device)))


def fa_bwd_dq_stats(q, k, v, o, do, lse, workspace, dq, scale=None,
                    causal=False):
    """The preprocess and the dQ pass in one call: writes dq and the row
    statistics into `workspace`, ready for fa_bwd_dkdv."""
    B, H, N, d = _shape4(q, k, v, o, do)
    _arg(lse, "lse", (B, H, N), torch.float32, q.device)
    _arg(dq, "dq", q.shape, torch.float32, q.device)
    workspace, ws_bytes = _ws_arg(workspace, q.device)
    with torch.cuda.device(q.device):
        _check(library().fa_bwd_dq_stats(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
            _ptr(workspace), ws_bytes, B, H, N, d, _dtype_code(q),
            _scale(scale, d), int(bool(causal)), _stream(q.device)))


def fa_tile_grid(pass_, d, sparse=False):
    """(rows, cols) of one pass's tiles in the bf16 kernels: pass 0 forward
    (query tile x key tile), 1 dK/dV pass (query stage x key tile), 2 dQ
    pass (query tile x key tile)."""
    rows, cols = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(library().fa_tile_grid(int(pass_), int(d), int(bool(sparse)),
                                  ctypes.byref(rows), ctypes.byref(cols)))
    return rows.value, cols.value


def fa_fwd_tile_visits(q, k, v, block_mask=None, block_m=128, block_n=128,
                       scale=None, causal=False):
    """fa_fwd_blocksparse (block_mask None: fa_fwd) through the counting
    kernel instances: returns O, LSE and an int32 tensor B x H x Tq of the
    key tiles each query tile visited."""
    B, H, N, d = _shape4(q, k, v)
    lib = library()
    mask_t = _mask_arg(block_mask, N, block_m, block_n, q.device)
    rows, _ = fa_tile_grid(0, d, mask_t is not None)
    visits = torch.full((B, H, -(-N // rows)), -1, dtype=torch.int32,
                        device=q.device)
    o, lse_t = _fwd_outputs(q, (B, H, N, d), None, None)
    with torch.cuda.device(q.device):
        _check(lib.fa_fwd_tile_visits(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, N, d,
            _dtype_code(q), _scale(scale, d), int(bool(causal)),
            _ptr(mask_t), int(block_m), int(block_n), _ptr(visits),
            visits.numel(), _stream(q.device)))
    return o, lse_t, visits


def fa_bwd_tile_visits(q, k, v, o, do, lse, block_mask=None, block_m=128,
                       block_n=128, scale=None, causal=False):
    """fa_bwd_blocksparse (block_mask None: fa_bwd) through the counting
    kernel instances: returns dQ, dK, dV, the query stages each key tile of
    the dK/dV pass visited (B x H x Tk) and the key tiles each query tile of
    the dQ pass visited (B x H x Tq)."""
    B, H, N, d = _shape4(q, k, v, o, do)
    lib = library()
    mask_t = _mask_arg(block_mask, N, block_m, block_n, q.device)
    _arg(lse, "lse", (B, H, N), torch.float32, q.device)
    _, kv_cols = fa_tile_grid(1, d, mask_t is not None)
    q_rows, _ = fa_tile_grid(2, d, mask_t is not None)
    v_kv = torch.full((B, H, -(-N // kv_cols)), -1, dtype=torch.int32,
                      device=q.device)
    v_q = torch.full((B, H, -(-N // q_rows)), -1, dtype=torch.int32,
                     device=q.device)
    dq, dk, dv = _grads(q, None, None, None)
    ws, ws_bytes = _workspace(B, H, N, d, q.device, None)
    with torch.cuda.device(q.device):
        _check(lib.fa_bwd_tile_visits(
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes, B, H, N, d, _dtype_code(q),
            _scale(scale, d), int(bool(causal)), _ptr(mask_t), int(block_m),
            int(block_n), _ptr(v_kv), v_kv.numel(), _ptr(v_q), v_q.numel(),
            _stream(q.device)))
    return dq, dk, dv, v_kv, v_q


# Short names for the common calls (the same functions).
fwd = fa_fwd
bwd = fa_bwd


def fwd_blocksparse(q, k, v, mask, block=128, scale=None, causal=False):
    """fa_fwd_blocksparse with square mask blocks of ``block`` rows/keys."""
    return fa_fwd_blocksparse(q, k, v, mask, block, block, scale=scale,
                              causal=causal)

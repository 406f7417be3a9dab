"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects every invalid argument with the documented status before any HIP
call (no GPU is touched; pointers below are never dereferenced)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_DTYPE = 0, 1, 2, 3
FA_ERR_UNSUPPORTED, FA_ERR_MASK, FA_ERR_HIP, FA_ERR_ALIGN, FA_ERR_ARG = (
    4, 5, 6, 7, 8)
FA_ERR_SCRATCH = 9
F32, BF16 = 0, 1

# Fake, aligned, never-dereferenced device addresses.
P = 0x10000
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    from exact_io_aware_amd import _build, fa
    alt = os.environ.get("FA_ABI_TEST_LIB")
    if alt:  # the host-only sanitizer build (tests/test_abi_sanitized.py)
        return fa.declare(ctypes.CDLL(alt))
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    return fa.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_fwd_blocksparse"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in fa.h but not exported"


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.fa_version()
    for code in range(10):
        assert lib.fa_status_str(code).startswith(b"FA_")
    assert lib.fa_status_str(99) == b"unknown fa_status"


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, dt=BF16,
        scale=0.125, causal=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, dt, scale, causal, None)


def test_fwd_validation(lib):
    assert fwd(lib, B=-1) == FA_ERR_SHAPE
    assert fwd(lib, N=-5) == FA_ERR_SHAPE
    assert fwd(lib, dt=7) == FA_ERR_DTYPE
    assert fwd(lib, d=32) == FA_ERR_UNSUPPORTED
    assert fwd(lib, d=96) == FA_ERR_UNSUPPORTED
    assert fwd(lib, scale=float("nan")) == FA_ERR_ARG
    assert fwd(lib, scale=float("inf")) == FA_ERR_ARG
    assert fwd(lib, scale=0.0) == FA_ERR_ARG
    assert fwd(lib, scale=-1.0) == FA_ERR_ARG
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{name: None}) == FA_ERR_NULL, name
    for name in ("q", "k", "v", "o"):
        assert fwd(lib, **{name: MISALIGNED}) == FA_ERR_ALIGN, name
    assert fwd(lib, lse=P + 2) == FA_ERR_ALIGN
    # sizes whose element count overflows
    assert fwd(lib, B=1 << 40, H=1 << 20) == FA_ERR_SHAPE
    assert fwd(lib, N=(1 << 30) + 1) == FA_ERR_SHAPE


def test_empty_problems_are_noops(lib):
    # Nothing to compute: FA_OK without looking at the (NULL) pointers.
    for B, H, N in ((0, 4, 128), (2, 0, 128), (2, 4, 0)):
        assert fwd(lib, q=None, k=None, v=None, o=None, lse=None, B=B, H=H,
                   N=N) == FA_OK
        assert lib.fa_bwd(None, None, None, None, None, None, None, None,
                          None, None, 0, B, H, N, 64, BF16, 0.125, 1,
                          None) == FA_OK
        assert lib.fa_bwd_workspace_bytes(B, H, N, 64) == 0


def sparse(lib, mask=P, bm=128, bn=128, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=256, d=64, dt=BF16,
             scale=0.125, causal=0)
    a.update(kw)
    return lib.fa_fwd_blocksparse(a["q"], a["k"], a["v"], a["o"], a["lse"],
                                  a["B"], a["H"], a["N"], a["d"], a["dt"],
                                  a["scale"], a["causal"], mask, bm, bn, None)


def test_blocksparse_validation(lib):
    assert sparse(lib, bm=64) == FA_ERR_MASK
    assert sparse(lib, bn=100) == FA_ERR_MASK
    assert sparse(lib, bm=0) == FA_ERR_MASK
    assert sparse(lib, bn=-128) == FA_ERR_MASK
    assert sparse(lib, d=48) == FA_ERR_UNSUPPORTED
    assert sparse(lib, q=None) == FA_ERR_NULL
    assert sparse(lib, N=0) == FA_OK


def bwd(lib, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, B=2,
             H=3, N=256, d=128, dt=BF16, scale=0.088, causal=1)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
    return lib.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                      a["dq"], a["dk"], a["dv"], a["ws"], ws_bytes, a["B"],
                      a["H"], a["N"], a["d"], a["dt"], a["scale"],
                      a["causal"], None)


def test_bwd_validation(lib):
    need = lib.fa_bwd_workspace_bytes(2, 3, 256, 128)
    assert need >= 2 * 2 * 3 * 256 * 4
    assert bwd(lib, dt=9) == FA_ERR_DTYPE
    # float32 runs the same checks (only failures are exercised here: a
    # valid call would launch kernels)
    assert bwd(lib, dt=F32, d=96) == FA_ERR_UNSUPPORTED
    assert bwd(lib, dt=F32, ws_bytes=need - 4) == FA_ERR_ARG
    assert bwd(lib, dt=F32, scale=0.0) == FA_ERR_ARG
    for name in ("q", "dq", "ws"):
        assert bwd(lib, dt=F32, **{name: None}) == FA_ERR_NULL, name
        assert bwd(lib, dt=F32, **{name: MISALIGNED}) == FA_ERR_ALIGN, name
    assert bwd(lib, d=256) == FA_ERR_UNSUPPORTED
    assert bwd(lib, ws_bytes=need - 4) == FA_ERR_ARG
    assert bwd(lib, scale=float("nan")) == FA_ERR_ARG
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert bwd(lib, **{name: None}) == FA_ERR_NULL, name
    for name in ("q", "k", "v", "o", "do", "dq", "dk", "dv", "ws"):
        assert bwd(lib, **{name: MISALIGNED}) == FA_ERR_ALIGN, name
    assert bwd(lib, B=-2) == FA_ERR_SHAPE


def test_bwd_pass_validation(lib):
    ws = lib.fa_bwd_workspace_bytes(1, 1, 128, 64)
    # preprocess needs o, dout, lse, workspace
    assert lib.fa_bwd_preprocess(None, P, P, P, ws, 1, 1, 128, 64, BF16,
                                 None) == FA_ERR_NULL
    assert lib.fa_bwd_preprocess(P, P, P, P, ws - 1, 1, 1, 128, 64, BF16,
                                 None) == FA_ERR_ARG
    # dkdv needs q, k, v, dout, dk, dv; dq needs q, k, v, dout, dq
    assert lib.fa_bwd_dkdv(P, P, P, P, None, P, P, ws, 1, 1, 128, 64, BF16,
                           0.125, 0, None) == FA_ERR_NULL
    assert lib.fa_bwd_dq(P, P, P, P, None, P, ws, 1, 1, 128, 64, BF16, 0.125,
                         0, None) == FA_ERR_NULL
    assert lib.fa_bwd_dq(P, P, P, P, P, P, ws, 1, 1, 128, 64, BF16, -0.1, 0,
                         None) == FA_ERR_ARG
    # dq_stats needs q, k, v, o, dout, lse, dq and the workspace
    args = [P, P, P, P, P, P, P, P]
    for i in range(8):
        a = list(args)
        a[i] = None
        assert lib.fa_bwd_dq_stats(*a, ws, 1, 1, 128, 64, BF16, 0.125, 1,
                                   None) == FA_ERR_NULL, i
        assert lib.fa_bwd_dq_stats(*a, ws, 1, 1, 128, 64, F32, 0.125, 1,
                                   None) == FA_ERR_NULL, i
    assert lib.fa_bwd_dq_stats(*args, ws - 1, 1, 1, 128, 64, BF16, 0.125, 0,
                               None) == FA_ERR_ARG
    assert lib.fa_bwd_dq_stats(*args, ws, 1, 1, 128, 96, BF16, 0.125, 0,
                               None) == FA_ERR_UNSUPPORTED
    assert lib.fa_bwd_dq_stats(*args, ws, 1, 1, 128, 64, BF16, 0.0, 0,
                               None) == FA_ERR_ARG


def test_workspace_bytes(lib):
    assert lib.fa_bwd_workspace_bytes(1, 1, 1, 64) == 2 * 64 * 4
    assert lib.fa_bwd_workspace_bytes(4, 16, 4096, 128) == 2 * 4 * 16 * 4096 * 4
    assert lib.fa_bwd_workspace_bytes(1, 1, 128, 32) == 0  # unsupported d
    assert lib.fa_bwd_workspace_bytes(-1, 1, 128, 64) == 0


def test_binding_fails_loudly_without_gpu_tensors(lib):
    import torch

    from exact_io_aware_amd import fa
    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)  # CPU tensors are rejected, never computed on CPU


def bwd_sparse(lib, mask=P, bm=128, bn=128, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, B=1,
             H=2, N=384, d=64, dt=BF16, scale=0.125, causal=0)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(a["B"], a["H"], a["N"], a["d"])
    return lib.fa_bwd_blocksparse(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
        a["dv"], a["ws"], ws_bytes, a["B"], a["H"], a["N"], a["d"], a["dt"],
        a["scale"], a["causal"], mask, bm, bn, None)


def test_bwd_blocksparse_validation(lib):
    assert bwd_sparse(lib, bm=64) == FA_ERR_MASK
    assert bwd_sparse(lib, bn=200) == FA_ERR_MASK
    assert bwd_sparse(lib, bm=-128) == FA_ERR_MASK
    assert bwd_sparse(lib, dt=F32, bm=64) == FA_ERR_MASK
    assert bwd_sparse(lib, dt=F32, dv=None) == FA_ERR_NULL
    assert bwd_sparse(lib, scale=0.0) == FA_ERR_ARG
    assert bwd_sparse(lib, ws_bytes=16) == FA_ERR_ARG
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws"):
        assert bwd_sparse(lib, **{name: None}) == FA_ERR_NULL, name
    assert bwd_sparse(lib, dk=MISALIGNED) == FA_ERR_ALIGN
    assert bwd_sparse(lib, N=0, q=None, ws=None) == FA_OK


def splitkv(lib, q=P, k=P, v=P, o=P, lse=P, ws=P, ws_bytes=None, B=2, H=3,
            Nq=1, Nk=1000, d=128, dt=BF16, scale=0.09, causal=0, splits=0):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, splits)
    return lib.fa_fwd_splitkv(q, k, v, o, lse, ws, ws_bytes, B, H, Nq, Nk, d,
                              dt, scale, causal, splits, None)


def test_splitkv_validation(lib):
    assert splitkv(lib, B=-1) == FA_ERR_SHAPE
    assert splitkv(lib, Nk=-1) == FA_ERR_SHAPE
    assert splitkv(lib, Nq=5, Nk=4) == FA_ERR_SHAPE        # more queries than keys
    assert splitkv(lib, Nk=(1 << 30) + 1) == FA_ERR_SHAPE
    assert splitkv(lib, B=1 << 40, H=1 << 20) == FA_ERR_SHAPE
    assert splitkv(lib, dt=9) == FA_ERR_DTYPE
    assert splitkv(lib, dt=F32) == FA_ERR_UNSUPPORTED
    assert splitkv(lib, d=96) == FA_ERR_UNSUPPORTED
    assert splitkv(lib, splits=-1) == FA_ERR_ARG
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert splitkv(lib, scale=bad) == FA_ERR_ARG
    for name in ("q", "k", "v", "o", "lse", "ws"):
        assert splitkv(lib, **{name: None}) == FA_ERR_NULL, name
    for name in ("q", "k", "v", "o", "ws"):
        assert splitkv(lib, **{name: MISALIGNED}) == FA_ERR_ALIGN, name
    assert splitkv(lib, lse=P + 2) == FA_ERR_ALIGN
    need = lib.fa_fwd_splitkv_workspace_bytes(2, 3, 1, 1000, 128, 0)
    assert splitkv(lib, ws_bytes=need - 1) == FA_ERR_ARG
    # empty problems: no pointer is looked at
    for B, H, Nq in ((0, 3, 1), (2, 0, 1), (2, 3, 0)):
        assert splitkv(lib, q=None, k=None, v=None, o=None, lse=None, ws=None,
                       ws_bytes=0, B=B, H=H, Nq=Nq) == FA_OK


def test_splitkv_chunk_plan(lib):
    chunks = lib.fa_fwd_splitkv_chunks
    wsb = lib.fa_fwd_splitkv_workspace_bytes
    # 1000 keys = 32 tiles of 32 keys; a cap is honoured, and the tiles are
    # spread evenly with no empty chunk: 32 tiles over at most 5 chunks is
    # 7 tiles per chunk, hence 5 chunks; over at most 6 it is 6 tiles per
    # chunk, hence 6; a cap above the tile count gives one tile per chunk.
    assert chunks(1, 1, 1, 1000, 128, 5) == 5
    assert chunks(1, 1, 1, 1000, 128, 6) == 6
    assert chunks(1, 1, 1, 1000, 128, 7) == 7     # 5 tiles each, 7 chunks
    assert chunks(1, 1, 1, 1000, 128, 1000) == 32
    assert chunks(1, 1, 1, 1000, 128, 1) == 1
    # Automatic, several queries: at least 8 tiles per chunk, and no more
    # chunks than needed for about 2048 workgroups.
    assert chunks(8, 32, 4, 16384, 128, 0) == 8
    assert chunks(1, 1, 40, 1000, 64, 0) == 4
    # Automatic, one query (one wave per chunk): about 2048 chunks in all
    # (2048 // (B*H) per head) with at least 8 tiles per chunk (24 heads of
    # 200 tiles: 85 per head wanted, 25 allowed).
    assert chunks(1, 1, 1, 1000, 128, 0) == 4
    assert chunks(8, 32, 1, 16384, 128, 0) == 8
    assert chunks(16, 32, 1, 16384, 128, 0) == 4
    assert chunks(3, 8, 1, 6400, 64, 0) == 25
    assert chunks(64, 64, 1, 16384, 128, 0) == 1
    assert chunks(1, 1, 1, 16, 64, 0) == 1
    # workspace: chunks * rows * (d floats) + the logsumexps, 16-B rounded
    s = chunks(2, 3, 5, 1000, 64, 3)
    rows = s * 2 * 3 * 5
    assert wsb(2, 3, 5, 1000, 64, 3) == rows * 64 * 4 + (rows * 4 + 15) // 16 * 16
    assert wsb(0, 3, 5, 1000, 64, 3) == 0
    assert wsb(2, 3, 5, 4, 64, 3) == 0              # invalid: Nq > Nk
    assert chunks(2, 3, 5, 4, 64, 3) == 0


def test_row_count_limits(lib):
    # 2^35 rows (2^30 heads of 32): every other size check passes, but the
    # row passes and the split-KV merge would need more than 2^31
    # workgroups; rejected up front.
    assert fwd(lib, B=1 << 20, H=1 << 10, N=32) == FA_ERR_SHAPE
    assert bwd(lib, B=1 << 20, H=1 << 10, N=32, d=64, ws_bytes=0) == FA_ERR_SHAPE
    assert splitkv(lib, B=1 << 25, H=1 << 5, Nq=32, Nk=32, ws_bytes=0) == FA_ERR_SHAPE
    assert lib.fa_fwd_splitkv_chunks(1 << 25, 1 << 5, 32, 32, 128, 0) == 0


def fwd_drop(lib, p=0.1, seed=1, dt=BF16, N=128, d=64, q=P, scale=0.125):
    return lib.fa_fwd_dropout(q, P, P, P, P, 1, 1, N, d, dt, scale, 0, p,
                              seed, None)


def bwd_drop(lib, p=0.1, seed=1, dt=BF16, N=128, d=64, ws_bytes=1 << 20,
             ws=P):
    return lib.fa_bwd_dropout(P, P, P, P, P, P, P, P, P, ws, ws_bytes, 1, 1,
                              N, d, dt, 0.125, 1, p, seed, None)


def test_dropout_validation(lib):
    # drop probability: round(256 p) must lie in [0, 255]
    for bad in (-0.01, 255.6 / 256, 1.0, 2.0, float("nan"), float("inf")):
        assert fwd_drop(lib, p=bad) == FA_ERR_ARG, bad
        assert bwd_drop(lib, p=bad) == FA_ERR_ARG, bad
    # bf16 only
    assert fwd_drop(lib, dt=F32) == FA_ERR_UNSUPPORTED
    assert bwd_drop(lib, dt=F32) == FA_ERR_UNSUPPORTED
    # shared checks come first and keep their codes
    assert fwd_drop(lib, d=96) == FA_ERR_UNSUPPORTED
    assert fwd_drop(lib, N=-1) == FA_ERR_SHAPE
    assert fwd_drop(lib, scale=0.0) == FA_ERR_ARG
    assert fwd_drop(lib, q=None) == FA_ERR_NULL
    assert fwd_drop(lib, q=MISALIGNED) == FA_ERR_ALIGN
    assert bwd_drop(lib, ws=None) == FA_ERR_NULL
    assert bwd_drop(lib, ws_bytes=16) == FA_ERR_ARG
    # empty problems do nothing, whatever the seed
    assert fwd_drop(lib, N=0, seed=2**64 - 1) == FA_OK
    assert bwd_drop(lib, N=0, seed=0) == FA_OK


def test_binding_short_names():
    from exact_io_aware_amd import fa
    assert fa.fwd is fa.fa_fwd and fa.bwd is fa.fa_bwd
    assert callable(fa.fwd_blocksparse)


def test_bwd_noalloc_validation(lib):
    """fa_bwd_noalloc checks as fa_bwd does, and rejects problems larger
    than its fixed scratch (B*H*N > 2^20 rows) with FA_ERR_SCRATCH, all
    before any HIP call."""
    def call(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, H=2,
             N=128, d=64, dt=BF16, scale=0.125, causal=1):
        return lib.fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N,
                                  d, dt, scale, causal, None)
    assert call(B=1, H=1, N=(1 << 20) + 1) == FA_ERR_SCRATCH
    assert call(B=2, H=32, N=16384 + 1) == FA_ERR_SCRATCH
    assert call(B=1, H=64, N=(1 << 14) + 64, q=None) == FA_ERR_SCRATCH
    assert call(B=-1) == FA_ERR_SHAPE
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(dt=5) == FA_ERR_DTYPE
    assert call(scale=float("nan")) == FA_ERR_ARG
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert call(**{name: None}) == FA_ERR_NULL, name
    assert call(dk=MISALIGNED) == FA_ERR_ALIGN
    for B, H, N in ((0, 4, 128), (2, 0, 128), (2, 4, 0)):
        assert call(q=None, k=None, v=None, o=None, do=None, lse=None,
                    dq=None, dk=None, dv=None, B=B, H=H, N=N) == FA_OK


def test_tile_grid(lib):
    """The tile grids of the bf16 kernels (a host-side query, no GPU)."""
    from exact_io_aware_amd import fa
    assert fa.fa_tile_grid(0, 128) == (256, 64)
    assert fa.fa_tile_grid(0, 64) == (128, 128)
    assert fa.fa_tile_grid(0, 128, sparse=True) == (128, 64)
    assert fa.fa_tile_grid(1, 128) == (32, 256)
    assert fa.fa_tile_grid(1, 128, sparse=True) == (64, 128)
    assert fa.fa_tile_grid(1, 64) == (128, 128)
    assert fa.fa_tile_grid(2, 128) == (256, 64)
    assert fa.fa_tile_grid(2, 128, sparse=True) == (128, 64)
    assert fa.fa_tile_grid(2, 64) == (128, 128)
    r, c = ctypes.c_int64(0), ctypes.c_int64(0)
    assert lib.fa_tile_grid(3, 128, 0, ctypes.byref(r), ctypes.byref(c)) == FA_ERR_ARG
    assert lib.fa_tile_grid(0, 96, 0, ctypes.byref(r), ctypes.byref(c)) == FA_ERR_UNSUPPORTED
    assert lib.fa_tile_grid(0, 128, 0, None, ctypes.byref(c)) == FA_ERR_NULL


def test_tile_visits_validation(lib):
    """The counting calls validate as the plain calls, plus their count
    buffers (NULL, alignment, length) and the dtype (bf16 only)."""
    def fwdv(visits=P, n_vis=1 << 20, dt=BF16, B=1, H=2, N=1000, d=128,
             mask=None, q=P):
        return lib.fa_fwd_tile_visits(q, P, P, P, P, B, H, N, d, dt, 0.1, 1,
                                      mask, 128, 128, visits, n_vis, None)
    assert fwdv(dt=F32) == FA_ERR_UNSUPPORTED
    assert fwdv(visits=None) == FA_ERR_NULL
    assert fwdv(visits=P + 2) == FA_ERR_ALIGN
    assert fwdv(n_vis=2 * 4 - 1) == FA_ERR_ARG       # 2 heads x 4 tiles of 256
    assert fwdv(q=None) == FA_ERR_NULL
    assert fwdv(B=0, visits=None) == FA_OK

    def bwdv(vkv=P, nkv=1 << 20, vq=P, nq=1 << 20, dt=BF16, ws=1 << 20):
        return lib.fa_bwd_tile_visits(P, P, P, P, P, P, P, P, P, P, ws, 1, 2,
                                      1000, 128, dt, 0.1, 1, None, 128, 128,
                                      vkv, nkv, vq, nq, None)
    assert bwdv(dt=F32) == FA_ERR_UNSUPPORTED
    assert bwdv(vkv=None) == FA_ERR_NULL
    assert bwdv(vq=P + 1) == FA_ERR_ALIGN
    assert bwdv(nkv=2 * 4 - 1) == FA_ERR_ARG        # 2 heads x 4 key tiles of 256
    assert bwdv(nq=2 * 4 - 1) == FA_ERR_ARG         # 2 heads x 4 query tiles
    assert bwdv(ws=16) == FA_ERR_ARG


def fwd_gen(lib, q=P, B=1, H=2, Nq=100, Nk=300, d=128, dt=BF16, scale=0.1,
            causal=1, mask=None, bm=128, bn=128, p=0.0, seed=3):
    return lib.fa_fwd_general(q, P, P, P, P, B, H, Nq, Nk, d, dt, scale,
                              causal, mask, bm, bn, p, seed, None)


def bwd_gen(lib, ws=P, ws_bytes=1 << 20, B=1, H=2, Nq=100, Nk=300, d=128,
            dt=BF16, causal=1, mask=None, bm=128, bn=128, p=0.0, dq=P):
    return lib.fa_bwd_general(P, P, P, P, P, P, dq, P, P, ws, ws_bytes, B, H,
                              Nq, Nk, d, dt, 0.1, causal, mask, bm, bn, p, 7,
                              None)


def test_general_validation(lib):
    """fa_fwd_general / fa_bwd_general: key length 1..2^30, Nq <= Nk under
    the causal rule (any lengths otherwise), block sizes checked only with a
    mask, dropout bf16 only and in range, the workspace sized by query
    rows; the shared checks keep their codes."""
    # Non-causal calls take any lengths: the shape passes, the NULL pointer
    # checked after it is what fails.
    assert fwd_gen(lib, Nq=301, Nk=300, causal=0, q=None) == FA_ERR_NULL
    assert bwd_gen(lib, Nq=301, Nk=300, causal=0, ws=None) == FA_ERR_NULL
    for f in (fwd_gen, bwd_gen):
        assert f(lib, Nq=301, Nk=300) == FA_ERR_SHAPE      # causal: Nq <= Nk
        assert f(lib, Nk=0) == FA_ERR_SHAPE
        assert f(lib, Nk=-1) == FA_ERR_SHAPE
        assert f(lib, Nk=(1 << 30) + 1) == FA_ERR_SHAPE
        assert f(lib, Nq=-1) == FA_ERR_SHAPE
        assert f(lib, d=96) == FA_ERR_UNSUPPORTED
        assert f(lib, mask=P, bm=64) == FA_ERR_MASK
        assert f(lib, mask=P, bn=100) == FA_ERR_MASK
        assert f(lib, p=-0.5) == FA_ERR_ARG
        assert f(lib, p=1.0) == FA_ERR_ARG
        assert f(lib, p=0.2, dt=F32) == FA_ERR_UNSUPPORTED
        assert f(lib, B=0) == FA_OK                         # empty: no-op
        assert f(lib, Nq=0, Nk=0) == FA_OK
    assert fwd_gen(lib, q=None) == FA_ERR_NULL
    assert fwd_gen(lib, q=MISALIGNED) == FA_ERR_ALIGN
    assert fwd_gen(lib, scale=0.0) == FA_ERR_ARG
    assert bwd_gen(lib, ws=None) == FA_ERR_NULL
    assert bwd_gen(lib, dq=None) == FA_ERR_NULL
    # The workspace is per query row: enough for Nq rows, too small for Nk.
    need = lib.fa_bwd_workspace_bytes(1, 2, 100, 128)
    assert need < lib.fa_bwd_workspace_bytes(1, 2, 300, 128)
    assert bwd_gen(lib, ws_bytes=need - 1) == FA_ERR_ARG

"""The Python binding checks every caller-supplied tensor the kernels read or
write (shape, dtype, device, contiguity) and raises before any launch, so a
wrong output buffer can never be written out of bounds; and the entry
points take the caller's buffers when they are right."""

import sys

import pytest
import torch

from exact_io_aware_amd import fa
from tests.test_gpu_parity import dev, gen  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    sys.stdout.flush()
    yield


def test_forward_outputs_checked(dev):
    x = gen(1, 2, 128, 64, seed=1, dev=dev)
    q, k, v = x["q"], x["k"], x["v"]
    bad_out = [torch.empty(1, 2, 127, 64, dtype=q.dtype, device=dev),
               torch.empty(1, 2, 128, 64, dtype=torch.float32, device=dev),
               torch.empty(1, 2, 64, 128, dtype=q.dtype, device=dev).transpose(2, 3)]
    for o in bad_out:
        with pytest.raises(ValueError):
            fa.fa_fwd(q, k, v, out=o)
    for lse in (torch.empty(1, 2, 129, device=dev),
                torch.empty(1, 2, 128, dtype=torch.float64, device=dev)):
        with pytest.raises(ValueError):
            fa.fa_fwd(q, k, v, lse=lse)
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 128, device=dev)
    o2, lse2 = fa.fa_fwd(q, k, v, out=o, lse=lse)
    assert o2.data_ptr() == o.data_ptr() and lse2.data_ptr() == lse.data_ptr()
    ref, lref = fa.fa_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, ref) and torch.equal(lse, lref)


def test_backward_buffers_checked(dev):
    x = gen(1, 2, 128, 64, seed=2, with_do=True, dev=dev)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse[:, :, :64].contiguous(), causal=True)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse, causal=True,
                  dq=torch.empty_like(q))          # bf16, not float32
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse, causal=True,
                  dk=torch.empty(1, 2, 128, 32, device=dev))
    ws = torch.empty(2 * fa.fa_bwd_workspace_bytes(1, 2, 128, 64),
                     dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse, causal=True, workspace=ws[::2])
    with pytest.raises(ValueError):
        fa.fa_bwd_dq(q, k, v, do, ws, torch.empty(1, 2, 128, 63, device=dev))
    with pytest.raises(fa.FAError):                # too small: the library
        fa.fa_bwd(q, k, v, o, do, lse, causal=True, workspace=ws[:16])


def test_splitkv_outputs_checked(dev):
    q = torch.randn(1, 2, 3, 64, device=dev).bfloat16()
    k = torch.randn(1, 2, 200, 64, device=dev).bfloat16()
    with pytest.raises(ValueError):
        fa.fa_fwd_splitkv(q, k, k, out=torch.empty_like(k))
    with pytest.raises(ValueError):
        fa.fa_fwd_splitkv(q, k, k, lse=torch.empty(1, 2, 200, device=dev))
    o, lse = fa.fa_fwd_splitkv(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (1, 2, 3, 64) and tuple(lse.shape) == (1, 2, 3)

"""The Python binding refuses tensors the library could not use safely.

The library takes raw addresses and trusts them, so the binding must stop
anything that is not a contiguous tensor of the right dtype and shape on the
caller's GPU before a pointer is taken.  On the CPU: host tensors are refused
by every wrapper (no HIP call is made).  On the GPU: wrong dtypes, shapes,
contiguity of caller-given outputs and planes are refused.
"""
import pytest

from test_abi import sattn  # noqa: F401  (module fixture: builds and loads the library)

T, HQ, HKV = 64, 4, 2


def host_inputs(torch):
    q = torch.zeros((HQ, T, 64), dtype=torch.float16)
    k = torch.zeros((HKV, T, 64), dtype=torch.float16)
    vt = torch.zeros((HKV, 64, T), dtype=torch.float16)
    return q, k, vt


def test_host_tensors_are_refused(sattn):
    import torch
    q, k, vt = host_inputs(torch)
    v = vt.transpose(1, 2).contiguous()
    with pytest.raises(ValueError):
        sattn.fwd(q, k, vt, 0.18)
    with pytest.raises(ValueError):
        sattn.fwd_vrows(q, k, v, 0.18)
    with pytest.raises(ValueError):
        sattn.mat_fwd(q, k, vt, 0.18)
    o = torch.zeros((T, HQ * 64), dtype=torch.float16)
    lse = torch.zeros((HQ, T), dtype=torch.float32)
    with pytest.raises(ValueError):
        sattn.bwd(q, k, vt, o, o, lse, 0.18, 0.125)


def test_non_tensors_are_refused(sattn):
    with pytest.raises(ValueError):
        sattn.fwd(None, None, None, 0.18)
    with pytest.raises(ValueError):
        sattn.mat_fwd([1.0], [1.0], [1.0], 0.18)


@pytest.mark.gpu
def test_bad_outputs_and_planes_are_refused(sattn, dev):
    import torch
    q, k, vt = (t.to(dev) for t in host_inputs(torch))
    f16, f32 = torch.float16, torch.float32
    bad_mat = [
        dict(scores=torch.empty((HQ, T, T), dtype=f16, device=dev)),          # dtype
        dict(scores=torch.empty((HQ, T, T - 1), dtype=f32, device=dev)),      # shape
        dict(scores=torch.empty((HQ, T, T), dtype=f32)),                      # host memory
        dict(probs=torch.empty((HQ, T, T), dtype=f32, device=dev)),           # dtype
        dict(probs=torch.empty((HQ, T, 2 * T), dtype=f16, device=dev)[:, :, :T]),  # strided
        dict(out=torch.empty((T, HQ * 64), dtype=f32, device=dev)),
        dict(lse=torch.empty((HQ, T + 1), dtype=f32, device=dev)),
    ]
    for kw in bad_mat:
        with pytest.raises(ValueError):
            sattn.mat_fwd(q, k, vt, 0.18, **kw)
    with pytest.raises(ValueError):
        sattn.fwd(q, k, vt, 0.18, out=torch.empty((T, HQ * 64), dtype=f16))
    with pytest.raises(ValueError):
        sattn.fwd(q, k, vt.transpose(1, 2), 0.18)
    with pytest.raises(ValueError):
        sattn.fwd(q.to(f32), k, vt, 0.18)
    torch.cuda.synchronize()

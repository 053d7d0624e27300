"""tri_dyn_plan_noalloc (the dynamic plan with its workspace in the library's
own device array, for callers that cannot allocate) against tri_dyn_plan with
a caller workspace, through the C ABI: the lists are index data, so they must
agree bit for bit.  Two calls in a row, the second on a smaller layer, so the
second runs over the first one's leftovers in the shared array."""
import ctypes

import numpy as np
import pytest
import torch

import static_triangle_sparse_amd as tsa
from static_triangle_sparse_amd import _abi
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gu.require_gpu()


def _inputs(seed, Hq, Hkv, N, d, qscale, dev):
    qb, kb, vb = synth.qkv_bf16_bits(seed, 1, Hq, Hkv, N, d)
    qb = synth.f32_to_bf16_bits((gu.as_f64(qb) * qscale).astype(np.float32))
    return gu.bits_to_device(qb, dev), gu.bits_to_device(kb, dev)


def _lists(rp, kt, fl):
    rp = rp.cpu().numpy()
    n = int(rp[-1])
    return rp, kt[:n].cpu().numpy(), fl[:n].cpu().numpy()


def _noalloc(q, k, alpha, dev):
    o = torch.empty((1, 1, 1, 8), dtype=torch.bfloat16, device=dev)   # not written
    t = tsa.make_tensors(q, k, k, o, None)
    _, rows, max_nnz = tsa.tri_dyn_plan_sizes(t)
    rp = torch.full((rows + 1,), -7, dtype=torch.int32, device=dev)
    kt = torch.full((max_nnz,), -7, dtype=torch.int32, device=dev)
    fl = torch.full((max_nnz,), 0xAB, dtype=torch.uint8, device=dev)
    dp = tsa.DynParams(float(alpha), tsa.TRI_DYN_PROBES)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = _abi.load().tri_dyn_plan_noalloc(ctypes.byref(t), ctypes.byref(dp), rp.data_ptr(), kt.data_ptr(),
                                          fl.data_ptr(), max_nnz, stream)
    assert st == tsa.TRI_OK, tsa.last_error()
    torch.cuda.synchronize()
    return _lists(rp, kt, fl)


def test_noalloc_lists_equal_the_caller_workspace_lists_on_two_calls(dev):
    calls = [  # (seed, Hq, Hkv, N, d, alpha, qscale): the second is smaller
        (5, 8, 2, 5000, 128, 0.5, 4.0),
        (6, 4, 1, 1300, 64, 0.3, 6.0),
    ]
    for seed, Hq, Hkv, N, d, alpha, qscale in calls:
        gu.note(f"no-alloc dynamic plan: Hq={Hq} Hkv={Hkv} N={N} d={d} alpha={alpha}")
        q, k = _inputs(seed, Hq, Hkv, N, d, qscale, dev)
        ref = tsa.dyn_plan(q, k, alpha)
        torch.cuda.synchronize()
        want = _lists(ref.d_row_ptr, ref.d_k_tile, ref.d_flags)
        got = _noalloc(q, k, alpha, dev)
        assert 0 < want[0][-1] < ref.max_nnz        # the threshold dropped tiles
        for g, w in zip(got, want):
            assert g.shape == w.shape and np.array_equal(g, w)

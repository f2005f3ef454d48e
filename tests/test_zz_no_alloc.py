"""The no-allocation int8-activation entry point against the entry point
with a caller workspace, through the C ABI: the same kernels, so the same
bits, on two calls in a row (the second smaller, so the first call's codes
are still in the scratch array), and within the oracle's bound.  Also the
requests it refuses before any HIP call."""
import numpy as np
import pytest

from block_wise_int4_amd import synth
from oracle import oracle as o
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mnb():
    from block_wise_int4_amd import mnb as m
    return m


def _case(mnb, M, N, K, g, zp, seed):
    t = G.torch()
    w = synth.weight(N, K, g, "f32", (0.005, 0.02), zp, (400, N, K, g, seed))
    q = G.upload(w)
    A = synth.activation(M, K, "f32", 1.0, (401, M, K, seed))
    bias = synth.activation(1, N, "f32", 1.0, (402, N, seed)).reshape(N)
    a, b = G.to_dev(A), G.to_dev(bias)
    n = mnb.mnb_gemm_accuracy4_workspace_bytes(q.desc, M)
    ws = t.zeros(max(n, 256), dtype=t.uint8, device="cuda")
    y_ref = t.empty((M, N), dtype=t.float32, device="cuda")
    y_na = t.full((M, N), 12345.0, dtype=t.float32, device="cuda")
    mnb.mnb_gemm_accuracy4(q.desc, q.repacked, a, M, b, y_ref, ws, n)
    mnb.mnb_gemm_accuracy4_noalloc(q.desc, q.repacked, a, M, b, y_na)
    t.cuda.synchronize()
    assert t.equal(y_ref, y_na), "M=%d N=%d K=%d g=%d" % (M, N, K, g)
    Y, B, _, _ = o.acc4_matmul(A, w.packed, w.scales, w.zero_points, N, K, g, bias)
    G.assert_within(G.host(y_na), Y, B, "no-alloc M=%d N=%d K=%d g=%d" % (M, N, K, g), bound=o.acc4_bound(B, K, g))


def test_no_alloc_matches_the_workspace_form_on_two_calls(mnb):
    # prefill-size call, then a smaller one (the scratch keeps the first
    # call's codes past the second's end), then small M and decode
    _case(mnb, 200, 300, 1024, 32, True, 1)
    _case(mnb, 40, 96, 512, 128, False, 2)
    _case(mnb, 9, 130, 384, 64, True, 3)
    _case(mnb, 1, 200, 512, 32, True, 4)


def test_no_alloc_refuses_requests_beyond_its_scratch(mnb):
    t = G.torch()
    w = synth.weight(64, 4096, 128, "f16", (0.005, 0.02), False, (403,))
    q = G.upload(w)
    limit = mnb.MNB_NOALLOC_SCRATCH_BYTES
    M = 4100   # 4100 x 4096 fp16 codes: beyond 32 MiB
    assert mnb.mnb_gemm_accuracy4_workspace_bytes(q.desc, M) > limit
    a = t.zeros((M, 4096), dtype=t.float32, device="cuda")
    y = t.full((M, 64), 7.0, dtype=t.float32, device="cuda")
    with pytest.raises(mnb.MnbError) as e:
        mnb.mnb_gemm_accuracy4_noalloc(q.desc, q.repacked, a, M, None, y)
    assert e.value.status == mnb.MNB_ERR_UNSUPPORTED
    t.cuda.synchronize()
    assert (G.host(y) == 7.0).all()

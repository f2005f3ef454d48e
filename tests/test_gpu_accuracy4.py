"""GPU parity of the int8-activation product (accuracy_level 4): the HIP path
through the C ABI against the fp64 CPU oracle on the same seeded inputs.

Bars: the activation codes and their scales bit-exact (both sides take every
rounding decision in binary32, in the pages' steps); outputs within
oracle.acc4_bound (the binary32 roundings of the evaluation; every block dot
is an exact integer), NaN agreeing with NaN.
"""
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


def _weight(N, K, g, sdt, zp, seed):
    return synth.weight(N, K, g, sdt, (0.005, 0.02), zp, (300, N, K, g, seed))


def _run(mnb, w, A, bias, with_ws=True):
    """(y [M,N] fp32, codes [M,K] or None, scales [M] or None) from the GPU."""
    t = G.torch()
    M, K = A.shape
    q = G.upload(w)
    n_ws = mnb.mnb_gemm_accuracy4_workspace_bytes(q.desc, M)
    ws = t.full((n_ws,), 0xA5, dtype=t.uint8, device="cuda") if with_ws else None
    y = t.full((M, w.N), float("nan"), dtype=t.float32, device="cuda")
    b = None if bias is None else G.to_dev(bias)
    mnb.mnb_gemm_accuracy4(q.desc, q.repacked, G.to_dev(A), M, b, y, ws, n_ws if with_ws else 0)
    t.cuda.synchronize()
    if not with_ws:
        return y.cpu().numpy(), None, None, mnb.mnb_last_variant()
    raw = ws.cpu().numpy()
    off = (4 * M + 255) // 256 * 256
    scales = raw[:4 * M].view(np.float32).copy()
    codes = raw[off:off + 2 * M * K].view(np.float16).reshape(M, K).copy()
    return y.cpu().numpy(), codes, scales, mnb.mnb_last_variant()


def _check(mnb, w, A, bias, what):
    M, K = A.shape
    y, codes, scales, variant = _run(mnb, w, A, bias)
    Y, B, q, sc = o.acc4_matmul(A, w.packed, w.scales, w.zero_points, w.N, K, w.group, bias)
    # the codes are integers in [-127, 127] written as fp16: exact
    assert (codes.astype(np.float64) == q.astype(np.float64)).all(), \
        "%s: %d codes differ" % (what, int((codes.astype(np.float64) != q).sum()))
    assert (scales.view(np.uint32) == sc.view(np.uint32)).all(), (what, scales, sc)
    G.assert_within(y, Y, B, what, bound=o.acc4_bound(B, K, w.group))
    return y, variant


ACC4_CASES = [
    # M, N, K, g, scale dtype, zero points, bias: the decode GEMV (every
    # group size), the small-M GEMM and the prefill GEMM
    (1, 300, 512, 32, "f32", False, True), (1, 200, 640, 64, "f16", True, False),
    (1, 257, 896, 16, "f32", True, True), (1, 64, 4096, 128, "f32", False, False),
    (1, 40, 11008, 128, "f32", True, True),
    (2, 300, 512, 32, "f32", True, True), (5, 257, 896, 64, "f16", False, False),
    (16, 100, 1024, 16, "f32", True, True),
    (40, 300, 512, 64, "f32", True, True), (130, 70, 384, 128, "f16", False, False),
    (200, 513, 1024, 32, "f32", True, True), (260, 300, 512, 128, "f32", True, True),
    # 16 < M <= 48: the small-M kernel on 16-row slices (the last ragged)
    (48, 96, 640, 32, "f16", True, True), (17, 130, 384, 128, "f32", False, True),
    # the prefill's 64-row tiles (groups of 32 or 16 k, fp32 scales with zero
    # points at 64 k) with 16-byte fp32 row stores (N % 4 == 0), ragged M
    (150, 256, 1024, 32, "f32", True, True), (97, 260, 512, 16, "f16", False, False),
    (70, 128, 768, 64, "f32", True, True),
    # K not a multiple of the 128-k chunk: the last chunk's padding
    (1, 70, 400, 16, "f32", True, True), (3, 70, 352, 32, "f16", True, False),
    (33, 70, 400, 16, "f32", True, True), (1, 90, 1088, 64, "f16", False, True),
]


@pytest.mark.parametrize("M,N,K,g,sdt,zp,with_bias", ACC4_CASES)
def test_accuracy4_parity(mnb, prefill_rows, M, N, K, g, sdt, zp, with_bias):
    G.needs_forced_height(prefill_rows, g, M)
    w = _weight(N, K, g, sdt, zp, seed=M)
    A = synth.activation(M, K, "f32", 1.0, (310, M, K))
    bias = synth.activation(1, N, "f32", 1.0, (311, N)).reshape(N) if with_bias else None
    y, variant = _check(mnb, w, A, bias, "accuracy4 M=%d N=%d K=%d g=%d %s zp=%s" % (M, N, K, g, sdt, zp))
    expect = "gemv_accuracy4_i8" if M == 1 else ("gemm_small_m_accuracy4" if M <= 48
                                                 else "gemm_mfma_32x32x16_accuracy4")
    assert variant == expect


def test_accuracy4_decode_grid_with_eight_waves(mnb):
    """N above 8192 columns gives the decode kernel 8-wave workgroups, and
    K = 12288 then exceeds what its threads hold in registers, so the
    activation is read again in the tail loops."""
    N, K, g = 8208, 12288, 64
    w = _weight(N, K, g, "f16", True, seed=7)
    A = synth.activation(1, K, "f32", 2.0, (312, K))
    _check(mnb, w, A, None, "accuracy4 decode N=%d K=%d" % (N, K))


def test_accuracy4_special_rows(mnb):
    """Rows the quantization treats specially, through the GEMV (one row at a
    time) and the GEMMs (all rows at once): a row of zeros gives the bias; a
    NaN is skipped by the maximum and its code is -127 (the row stays
    finite); ties of a*(1/scale) round away from zero (max 127 gives scale 1);
    a row whose 1/scale overflows gives codes +-127 and -127 for its zeros;
    an infinite activation makes the row's result an infinity."""
    N, K, g = 96, 256, 32
    w = _weight(N, K, g, "f32", True, seed=9)
    rng = np.random.default_rng(313)
    rows = []
    rows.append(np.zeros(K, np.float32))
    r = rng.standard_normal(K).astype(np.float32)
    r[[3, 100]] = np.nan
    rows.append(r)
    r = (rng.integers(-120, 121, K) + 0.5).astype(np.float32)
    r[0] = 127.0
    rows.append(r)
    r = np.zeros(K, np.float32)
    r[:40] = (rng.standard_normal(40) * 1e-40).astype(np.float32)
    r[5] = 1e-40
    rows.append(r)
    r = rng.standard_normal(K).astype(np.float32)
    r[7] = np.inf
    rows.append(r)
    A = np.stack(rows)
    bias = rng.standard_normal(N).astype(np.float32)
    for m in range(A.shape[0]):
        _check(mnb, w, A[m:m + 1], bias, "accuracy4 special row %d (GEMV)" % m)
    _check(mnb, w, A, bias, "accuracy4 special rows (small-M GEMM)")
    _check(mnb, w, np.tile(A, (13, 1))[:64], bias, "accuracy4 special rows (prefill GEMM)")
    big = np.concatenate([A] * 5)
    _check(mnb, w, big, bias, "accuracy4 special rows (prefill GEMM)")


def test_accuracy4_decode_at_maximum_k(mnb):
    """The decode kernel's largest K (32768 codes in LDS) with 16-wide blocks
    (the most zero-point sums), then one chunk more is refused."""
    N, K, g = 40, 32768, 16
    w = _weight(N, K, g, "f32", True, seed=13)
    A = synth.activation(1, K, "f32", 1.0, (315, K))
    _check(mnb, w, A, None, "accuracy4 decode at K=%d" % K)
    t = G.torch()
    big = synth.weight(N, K + 128, 128, "f32", (0.005, 0.02), False, (316,))
    q = G.upload(big)
    y = t.empty((1, N), dtype=t.float32, device="cuda")
    with pytest.raises(mnb.MnbError, match="decode limit"):
        mnb.mnb_gemm_accuracy4(q.desc, q.repacked, G.to_dev(np.zeros((1, K + 128), np.float32)), 1, None, y)


def test_accuracy4_decode_without_workspace(mnb):
    """M = 1 needs no workspace; the result is the same bits as with one."""
    N, K, g = 300, 1024, 32
    w = _weight(N, K, g, "f32", False, seed=11)
    A = synth.activation(1, K, "f32", 1.0, (314, K))
    y1, _, _, _ = _run(mnb, w, A, None, with_ws=True)
    y2, _, _, _ = _run(mnb, w, A, None, with_ws=False)
    assert (y1.view(np.uint32) == y2.view(np.uint32)).all()


def test_accuracy4_workload_sizes_sampled(mnb):
    """The bench's shapes (decode K=4096 N=4096 g=32 fp32 scales without zero
    points; prefill M=2048 K=4096 N=14336 g=128), every code and scale
    bit-exact, outputs sampled against the oracle row by row."""
    t = G.torch()
    for (M, K, N, g, zp, rows) in ((1, 4096, 4096, 32, False, [0]), (2048, 4096, 14336, 128, True, [0, 777, 2047])):
        w = synth.weight(N, K, g, "f32", (0.002, 0.01), zp, (320, M))
        A = synth.activation(M, K, "f32", 1.0, (321, M))
        bias = synth.activation(1, N, "f32", 1.0, (322, N)).reshape(N)
        y, codes, scales, _ = _run(mnb, w, A, bias)
        q_all, sc_all = o.acc4_quantize(A)
        assert (codes.astype(np.float64) == q_all).all()
        assert (scales.view(np.uint32) == sc_all.view(np.uint32)).all()
        for m in rows:
            Y, B, _, _ = o.acc4_matmul(A[m:m + 1], w.packed, w.scales, w.zero_points, N, K, g, bias)
            G.assert_within(y[m:m + 1], Y, B, "accuracy4 M=%d row %d" % (M, m), bound=o.acc4_bound(B, K, g))
        del y
        t.cuda.empty_cache()


def test_accuracy4_prefill_workload_every_output(mnb):
    """The int8-activation prefill workload (M=2048, K=4096, N=14336, g=128,
    fp32 scales, zero points, fp32 bias): all 2048 rows, every output, against
    the oracle's int8 rows and dequantized weights through a library fp64
    matrix product (oracle.acc4_matmul_lib, pinned against acc4_matmul)."""
    t = G.torch()
    M, K, N, g = 2048, 4096, 14336, 128
    w = synth.weight(N, K, g, "f32", (0.002, 0.01), True, (320, M))
    A = synth.activation(M, K, "f32", 1.0, (321, M))
    bias = synth.activation(1, N, "f32", 1.0, (322, N)).reshape(N)
    y, _, _, _ = _run(mnb, w, A, bias)
    t.cuda.empty_cache()
    Y, B, _, _ = o.acc4_matmul_lib(A, w.packed, w.scales, w.zero_points, N, K, g, bias)
    G.assert_within(y, Y, B, "accuracy4 prefill, every output", bound=o.acc4_bound(B, K, g))


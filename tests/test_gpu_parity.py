"""GPU parity: the HIP path, called through the C ABI, against the fp64 CPU
oracle on the same seeded inputs.

Bars: repacked bytes, unpacked codes and dequantized weights bit-exact;
outputs within |gpu - oracle| <= 1e-3 * sum_k |a_k w_nk| + 1e-5 per element
(NaN == NaN agrees); the fused SwiGLU output within the bound propagated from
that one (oracle.swiglu_bound).
"""
import json
import os

import numpy as np
import pytest

from block_wise_int4_amd import synth
from oracle import oracle as o
from tests import gpu_util as G
from tests import layout_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mnb():
    from block_wise_int4_amd import mnb as m
    return m


def _weight(N, K, g, sdt="f16", zp=True, seed=0, lo=0.005, hi=0.02):
    return synth.weight(N, K, g, sdt, (lo, hi), zp, (100, N, K, g, seed))


def _act(M, K, dtype="f16", sigma=1.0, seed=0):
    return synth.activation(M, K, dtype, sigma, (200, M, K, seed))


# ---------------------------------------------------------------- repack ----

REPACK_CASES = [
    (1, 16, 16, "f32", False), (5, 48, 16, "f16", True), (70, 384, 128, "f16", True),
    (130, 160, 32, "f32", True), (33, 4096, 64, "f16", False), (200, 640, 64, "f16", True),
    (17, 96, 32, "f16", True), (256, 256, 32, "f32", False)]


@pytest.mark.parametrize("N,K,g,sdt,zp", REPACK_CASES)
def test_repack_bytes_match_the_documented_layout(mnb, N, K, g, sdt, zp):
    w = _weight(N, K, g, sdt, zp)
    q = G.upload(w)
    got = q.repacked.cpu().numpy()
    codes = o.unpack_codes(w.packed, N, K, g)
    z = o.unpack_zero_points(w.zero_points, N, K, g)
    want = layout_ref.repack_ref(codes, z, w.scales, g, zp)
    assert got.size == want.size
    assert (got == want).all(), np.argwhere(got != want)[:10]


@pytest.mark.parametrize("N,K,g,sdt,zp", REPACK_CASES)
def test_unpacked_codes_and_weights_are_bit_exact(mnb, N, K, g, sdt, zp):
    t = G.torch()
    w = _weight(N, K, g, sdt, zp)
    q = G.upload(w)
    codes = t.empty((N, K), dtype=t.uint8, device="cuda")
    wf = t.empty((N, K), dtype=t.float32, device="cuda")
    mnb.mnb_unpack_debug(q.desc, q.repacked, codes, wf)
    t.cuda.synchronize()
    assert (codes.cpu().numpy() == o.unpack_codes(w.packed, N, K, g)).all()
    want = o.dequant(w.packed, w.scales, w.zero_points, N, K, g).astype(np.float32)
    got = wf.cpu().numpy()
    assert (got.view(np.uint32) == want.view(np.uint32)).all()


# --------------------------------------------------------- worked examples --

def _golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
    return json.load(open(path))["examples"]


def test_worked_examples_through_the_f32_gemv(mnb):
    """Hand-derived values (tests/golden) are exactly representable, so the
    fp32 GEMV must reproduce them bit for bit."""
    t = G.torch()
    from tests.test_oracle import _example_operands, _case_A
    for ex in _golden():
        N, K, g, packed, zp, scales = _example_operands(ex)
        if K % g:
            d = mnb.desc(N, K, g, zp is not None, mnb.MNB_F32)
            with pytest.raises(mnb.MnbError) as e:
                mnb.mnb_repacked_layout(d)
            assert e.value.status == mnb.MNB_ERR_UNSUPPORTED
            continue
        q = mnb.repack(G.to_dev(packed), G.to_dev(scales.reshape(-1)),
                       None if zp is None else G.to_dev(zp), N, K, g)
        for case in ex["cases"]:
            a = G.to_dev(_case_A(case["A"], K).reshape(-1))
            y = t.empty(N, dtype=t.float32, device="cuda")
            mnb.mnb_gemv(q.desc, q.repacked, a, y)
            assert G.host(y).tolist() == case["Y"], (ex["name"], case["A"])


# ------------------------------------------------------------------ GEMV ----

GEMV_CASES = [
    # N, K, g, act, scale dtype, zp
    (256, 256, 32, "f32", "f32", False),      # tiny GEMV workload
    (4096, 4096, 32, "f16", "f16", True),     # decode GEMV workload
    (70, 4096, 32, "f16", "f16", False),
    (130, 384, 128, "f16", "f32", True),
    (5, 48, 16, "f16", "f16", True),
    (200, 640, 64, "f32", "f16", True),
    (1, 16, 16, "f32", "f32", True),
    (333, 2176, 16, "f16", "f16", True),
    (4864, 896, 32, "f16", "f16", False),
    (96, 11008, 128, "f16", "f16", True),
]


@pytest.mark.parametrize("N,K,g,adt,sdt,zp", GEMV_CASES)
def test_gemv_parity(mnb, N, K, g, adt, sdt, zp):
    t = G.torch()
    w = _weight(N, K, g, sdt, zp)
    A = _act(1, K, adt)
    q = G.upload(w)
    y = t.empty(N, dtype=t.float16 if adt == "f16" else t.float32, device="cuda")
    mnb.mnb_gemv(q.desc, q.repacked, G.to_dev(A.reshape(-1)), y)
    assert mnb.mnb_last_variant() == ("gemv_" + adt)
    Y, B, _ = G.oracle_dense(A, w)
    G.assert_within(G.host(y)[None, :], Y, B, "gemv N=%d K=%d g=%d %s" % (N, K, g, adt))
    # mnb_gemm with M = 1 is the same kernel and the same bits
    y2 = t.empty_like(y)
    G.gemm(q, G.to_dev(A), 1, y2)
    assert t.equal(y, y2)


def test_down_projection_workload_parity(mnb):
    """The down projection at M=1 (K=11008 > N=4096, g=128, default zero
    point): the workload's own operands, every output against the oracle."""
    t = G.torch()
    wl = synth.DOWN_PROJ_GEMV
    w = synth.workload_weights(wl)
    A = synth.workload_activation(wl)
    q = G.upload(w)
    y = t.empty(wl.N, dtype=t.float16, device="cuda")
    mnb.mnb_gemv(q.desc, q.repacked, G.to_dev(A.reshape(-1)), y)
    Y, B, _ = G.oracle_dense(A, w)
    G.assert_within(G.host(y)[None, :], Y, B, "down projection")


def test_tiny_gemv_workload_exact_match_with_one_hot_rows(mnb):
    """One-hot activations pull single dequantized weights through the f32
    GEMV: the result is the exact product (code - zp) * scale rounded once to
    fp32."""
    t = G.torch()
    wl = synth.TINY_GEMV
    w = synth.workload_weights(wl)
    q = G.upload(w)
    W = o.dequant(w.packed, w.scales, w.zero_points, w.N, w.K, w.group)
    for k in (0, 1, 31, 32, 127, 255):
        a = np.zeros(wl.K, np.float32)
        a[k] = 1.0
        y = t.empty(wl.N, dtype=t.float32, device="cuda")
        mnb.mnb_gemv(q.desc, q.repacked, G.to_dev(a), y)
        got = y.cpu().numpy()
        assert (got.view(np.uint32) == W[:, k].astype(np.float32).view(np.uint32)).all(), k


MAX_K_CASES = [
    # the largest K the decode GEMV stages in LDS (fp16 and fp32 activations),
    # at every group size's register path: many chunks per wave, the batch loop
    (40, 31744, 128, "f16", False), (37, 31744, 16, "f16", True), (24, 15872, 32, "f32", True),
]


@pytest.mark.parametrize("N,K,g,adt,zp", MAX_K_CASES)
def test_gemv_at_maximum_k(mnb, N, K, g, adt, zp):
    t = G.torch()
    limit = 31744 if adt == "f16" else 15872
    assert K == limit
    w = _weight(N, K, g, "f16", zp, seed=5)
    A = _act(1, K, adt, seed=5)
    q = G.upload(w)
    y = t.empty(N, dtype=t.float16 if adt == "f16" else t.float32, device="cuda")
    mnb.mnb_gemv(q.desc, q.repacked, G.to_dev(A.reshape(-1)), y)
    Y, B, _ = G.oracle_dense(A, w)
    G.assert_within(G.host(y)[None, :], Y, B, "GEMV at K=%d g=%d %s" % (K, g, adt))
    # one chunk more is refused, not computed some other way
    big = mnb.desc(N, K + 128, 128, False, mnb.MNB_F16)
    assert mnb.lib.mnb_gemv(ctypes_byref(big), None, None, 1 if adt == "f16" else 0, None, None) == \
        mnb.MNB_ERR_UNSUPPORTED


def test_gate_up_and_act_order_at_maximum_k(mnb):
    """The fused gate/up pair at the GEMV's largest K, and act order at the
    largest K whose two staged copies fit in LDS (its in-LDS gather)."""
    t = G.torch()
    N, K, g = 48, 31744, 64
    wg = _weight(N, K, g, "f16", False, seed=8, lo=0.002, hi=0.01)
    wu = _weight(N, K, g, "f16", False, seed=9, lo=0.002, hi=0.01)
    A = _act(1, K, "f16", seed=8)
    qg, qu = G.upload(wg), G.upload(wu)
    y = t.empty(N, dtype=t.float16, device="cuda")
    mnb.mnb_gemv_gate_up_swiglu(qg.desc, qg.repacked, qu.repacked, G.to_dev(A.reshape(-1)), y)
    Yg, Bg, _ = G.oracle_dense(A, wg)
    Yu, Bu, _ = G.oracle_dense(A, wu)
    G.assert_within(G.host(y)[None, :], o.swiglu(Yg, Yu), None, "gate/up at K=%d" % K,
                    bound=o.swiglu_bound(Yg, Bg, Yu, Bu))
    K = 15872
    w = _weight(N, K, 128, "f16", True, seed=10)
    rng = np.random.default_rng(11)
    g_idx = np.empty(K, np.int32)
    g_idx[rng.permutation(K)] = np.arange(K) // 128
    d = mnb.desc(N, K, 128, True, mnb.MNB_F16)
    perm_dev = G.to_dev(mnb.mnb_act_order_permutation(d, g_idx))
    rep = t.empty(mnb.mnb_repacked_bytes(d), dtype=t.uint8, device="cuda")
    mnb.mnb_repack_act_order(d, G.to_dev(w.packed.reshape(-1)), G.to_dev(w.scales.reshape(-1)),
                             G.to_dev(w.zero_points.reshape(-1)), perm_dev, rep)
    A = _act(1, K, "f16", seed=12)
    n_ws = mnb.mnb_gemm_act_order_workspace_bytes(d, 1, mnb.MNB_F16)
    ws = t.zeros(n_ws, dtype=t.uint8, device="cuda")
    y = t.empty((1, N), dtype=t.float16, device="cuda")
    mnb.mnb_gemm_act_order(d, rep, G.to_dev(A), 1, perm_dev, y, ws, n_ws)
    assert mnb.mnb_last_variant() == "gemv_act_order_f16"
    W = o.dequant_gidx(w.packed, w.scales, w.zero_points, g_idx, N, K, 128)
    Y, B = o.matmul(o.decode(A.reshape(-1, K)), W)
    G.assert_within(G.host(y), Y, B, "act order at K=%d" % K)


def ctypes_byref(x):
    import ctypes
    return ctypes.byref(x)


# ------------------------------------------------------- gate/up SwiGLU ----

GATE_UP_CASES = [(11008, 4096, 128, "f16"), (4864, 896, 32, "f16"), (70, 384, 64, "f16"),
                 (133, 512, 16, "f32"),
                 # more than 512 tiles (8-wave workgroups) and more than 4
                 # chunks per wave: the two-set loop of the fused pair
                 (13824, 5120, 128, "f16"), (9000, 4608, 64, "f32")]


@pytest.mark.parametrize("N,K,g,adt", GATE_UP_CASES)
def test_gate_up_swiglu_parity(mnb, N, K, g, adt):
    t = G.torch()
    if (N, K, g) == (11008, 4096, 128):
        wg, wu = synth.workload_weights(synth.GATE_UP_SWIGLU)
        A = synth.workload_activation(synth.GATE_UP_SWIGLU)
    else:
        wg = _weight(N, K, g, "f16", False, seed=1, lo=0.002, hi=0.01)
        wu = _weight(N, K, g, "f16", False, seed=2, lo=0.002, hi=0.01)
        A = _act(1, K, adt)
    qg, qu = G.upload(wg), G.upload(wu)
    odt = t.float16 if adt == "f16" else t.float32
    a = G.to_dev(A.reshape(-1))
    y = t.empty(N, dtype=odt, device="cuda")
    mnb.mnb_gemv_gate_up_swiglu(qg.desc, qg.repacked, qu.repacked, a, y)
    assert mnb.mnb_last_variant().startswith("gemv_gate_up_swiglu")
    Yg, Bg, _ = G.oracle_dense(A, wg)
    Yu, Bu, _ = G.oracle_dense(A, wu)
    S = o.swiglu(Yg, Yu)
    G.assert_within(G.host(y)[None, :], S, None, "gate/up N=%d K=%d" % (N, K),
                    bound=o.swiglu_bound(Yg, Bg, Yu, Bu))
    # each projection alone through mnb_gemv, under the base bound
    for q_, Y_, B_ in ((qg, Yg, Bg), (qu, Yu, Bu)):
        yy = t.empty(N, dtype=odt, device="cuda")
        mnb.mnb_gemv(q_.desc, q_.repacked, a, yy)
        G.assert_within(G.host(yy)[None, :], Y_, B_, "projection")


# --------------------------------------------------------------- small M ----

@pytest.fixture(scope="module")
def small_m_workload():
    w = synth.workload_weights(synth.SMALL_M_GEMM)
    W64 = o.dequant(w.packed, w.scales, w.zero_points, w.N, w.K, w.group)
    return w, W64


@pytest.mark.parametrize("M", synth.SMALL_M_VALUES)
def test_small_m_workload_parity(mnb, small_m_workload, M):
    t = G.torch()
    w, W64 = small_m_workload
    A = synth.workload_activation(synth.SMALL_M_GEMM, M)
    q = G.upload(w)
    y = t.empty((M, w.N), dtype=t.float16, device="cuda")
    ws_n = mnb.mnb_gemm_workspace_bytes(q.desc, M)
    ws = t.empty(max(ws_n, 16), dtype=t.uint8, device="cuda")
    mnb.mnb_gemm(q.desc, q.repacked, G.to_dev(A), M, y, ws, ws_n)
    assert mnb.mnb_last_variant() == "gemm_small_m"
    Y, B, _ = G.oracle_dense(A, w, W64)
    G.assert_within(G.host(y), Y, B, "small-M M=%d" % M)


SMALL_CASES = [(2, 70, 384, 128, True), (3, 130, 160, 32, True), (7, 33, 4096, 64, False),
               (16, 5, 48, 16, True), (9, 300, 640, 16, False), (5, 257, 896, 32, True),
               # K not a multiple of 128 with two-chunk batches (groups of 64),
               # M ending inside a row quad
               (6, 100, 192, 64, True), (13, 40, 320, 64, False),
               # several batches per wave (65 chunks) and a ragged last chunk
               (4, 48, 8256, 64, True),
               # 16 < M <= 48 (fp16 A): one launch per 16-row slice, the last
               # ragged; every group size
               (17, 70, 384, 128, True), (32, 257, 512, 64, False), (33, 40, 160, 16, True),
               (48, 300, 640, 32, True), (41, 16, 8256, 64, False)]


@pytest.mark.parametrize("M,N,K,g,zp", SMALL_CASES)
def test_small_m_ragged_parity(mnb, M, N, K, g, zp):
    t = G.torch()
    w = _weight(N, K, g, "f16", zp)
    A = _act(M, K)
    q = G.upload(w)
    y = t.empty((M, N), dtype=t.float16, device="cuda")
    ws_n = mnb.mnb_gemm_workspace_bytes(q.desc, M)
    ws = t.empty(max(ws_n, 16), dtype=t.uint8, device="cuda")
    mnb.mnb_gemm(q.desc, q.repacked, G.to_dev(A), M, y, ws, ws_n)
    assert mnb.mnb_last_variant() == "gemm_small_m"
    Y, B, _ = G.oracle_dense(A, w)
    G.assert_within(G.host(y), Y, B, "small-M M=%d N=%d K=%d g=%d" % (M, N, K, g))


# --------------------------------------------------------------- prefill ----

PREFILL_CASES = [(49, 70, 384, 128, True, "f16"), (130, 300, 512, 64, True, "f16"),
                 (64, 257, 256, 32, False, "f32"), (57, 40, 160, 16, True, "f16"),
                 (300, 512, 1024, 128, False, "f16"), (129, 16, 4096, 128, True, "f16"),
                 # 64-row tiles: groups of 32 or 16 k, and fp32 scales with
                 # zero points at 64 k; several row blocks and a ragged one
                 (200, 300, 1024, 32, True, "f16"), (65, 64, 256, 32, False, "f16"),
                 (150, 130, 640, 64, True, "f32"), (130, 96, 512, 16, True, "f32"),
                 # one chunk (every later DMA of the pipeline is for a chunk past K)
                 (70, 48, 64, 32, True, "f16"), (88, 80, 128, 128, False, "f32"),
                 # groups of 128 k with ragged row blocks of either height and a
                 # ragged column block
                 (200, 300, 512, 128, True, "f16"), (129, 48, 256, 128, False, "f32"),
                 (260, 40, 384, 128, True, "f32")]


@pytest.mark.parametrize("M,N,K,g,zp,sdt", PREFILL_CASES)
def test_prefill_ragged_parity(mnb, prefill_rows, M, N, K, g, zp, sdt):
    G.needs_forced_height(prefill_rows, g)
    t = G.torch()
    w = _weight(N, K, g, sdt, zp, lo=0.002, hi=0.01)
    A = _act(M, K, sigma=0.5)
    q = G.upload(w)
    y = t.empty((M, N), dtype=t.float16, device="cuda")
    G.gemm(q, G.to_dev(A), M, y)
    assert mnb.mnb_last_variant().startswith("gemm_mfma")
    Y, B, _ = G.oracle_dense(A, w)
    G.assert_within(G.host(y), Y, B, "prefill M=%d N=%d K=%d g=%d" % (M, N, K, g))


def test_prefill_workload_sampled_parity(mnb):
    """The full prefill workload (M=2048, K=4096, N=14336, g=128) in the
    launch bench.py times; 6000 outputs checked one by one against the
    oracle: random ones plus every tile-boundary row/column pattern."""
    t = G.torch()
    wl = synth.PREFILL_GEMM
    w = synth.workload_weights(wl)
    A = synth.workload_activation(wl)
    q = G.upload(w)
    y = t.empty((wl.M, wl.N), dtype=t.float16, device="cuda")
    G.gemm(q, G.to_dev(A), wl.M, y)
    yh = G.host(y)
    rng = np.random.default_rng(5)
    ms = list(rng.integers(0, wl.M, 4000))
    ns = list(rng.integers(0, wl.N, 4000))
    for m in (0, 1, 15, 16, 127, 128, 2047):
        for n in (0, 15, 16, 63, 64, 255, 256, 14335):
            ms.append(m)
            ns.append(n)
    ms += list(range(0, wl.M, 1))[:1000]
    ns += list(rng.integers(0, wl.N, 1000))
    ms, ns = np.array(ms), np.array(ns)
    Y, B = o.matmul_nbits_at(A, w.packed, w.scales, w.zero_points, wl.N, wl.K, wl.group, ms, ns)
    G.assert_within(yh[ms, ns], Y, B, "prefill workload (sampled)")
    assert np.isfinite(yh).all()


def test_prefill_workload_every_output(mnb):
    """The full prefill workload (M=2048, K=4096, N=14336, g=128) in the
    launch bench.py times: all 29,360,128 outputs against the oracle's
    dequantized weights and a library fp64 matrix product (oracle.matmul_lib,
    pinned against the naive loops)."""
    t = G.torch()
    wl = synth.PREFILL_GEMM
    w = synth.workload_weights(wl)
    A = synth.workload_activation(wl)
    q = G.upload(w)
    y = t.empty((wl.M, wl.N), dtype=t.float16, device="cuda")
    G.gemm(q, G.to_dev(A), wl.M, y)
    yh = G.host(y)
    del y, q
    t.cuda.empty_cache()
    W64 = o.dequant(w.packed, w.scales, w.zero_points, wl.N, wl.K, wl.group)
    Y, B = o.matmul_lib(o.decode(A), W64)
    del W64
    G.assert_within(yh, Y, B, "prefill workload, every output")


def test_prefill_mid_size_sampled_parity(mnb):
    """Mid-size prefill shapes: between one and two rounds of output tiles
    (M=1000, N=14336: 11 x 56 tiles of 96 x 256) and fewer tiles than the
    chip holds (M=300, N=1000), asymmetric zero points, g = 64 and 128.
    Sampled outputs (every row at least once) against the oracle, then the
    same call again must give identical bits."""
    t = G.torch()
    for (M, N, K, g, seed) in ((1000, 14336, 1024, 64, 3), (300, 1000, 2048, 128, 4)):
        w = _weight(N, K, g, "f16", True, seed=seed, lo=0.002, hi=0.01)
        A = _act(M, K, sigma=0.5, seed=seed)
        q = G.upload(w)
        a = G.to_dev(A)
        y = t.empty((M, N), dtype=t.float16, device="cuda")
        G.gemm(q, a, M, y)
        yh = G.host(y)
        rng = np.random.default_rng(seed)
        ms = np.concatenate([rng.integers(0, M, 3000), np.arange(M)])
        ns = np.concatenate([rng.integers(0, N, 3000), rng.integers(0, N, M)])
        Y, B = o.matmul_nbits_at(A, w.packed, w.scales, w.zero_points, N, K, g, ms, ns)
        G.assert_within(yh[ms, ns], Y, B, "mid-size prefill M=%d N=%d K=%d (sampled)" % (M, N, K))
        assert np.isfinite(yh).all()
        y2 = t.empty_like(y)
        G.gemm(q, a, M, y2)
        t.cuda.synchronize()
        assert t.equal(y, y2)


@pytest.mark.parametrize("g", [64, 128])
def test_prefill_output_alignment_paths_agree(mnb, prefill_rows, g):
    """The prefill GEMM stores whole 16-byte row segments when N % 8 == 0 and
    Y is 16-byte aligned, and element by element otherwise: the same product
    into a Y shifted by one element (2-byte aligned only) gives the same bits,
    with and without a bias, and for the fp32 output of the int8-activation
    path (4-byte shift)."""
    G.needs_forced_height(prefill_rows, g)
    t = G.torch()
    M, N, K = 200, 520, 512
    w = _weight(N, K, g, "f16", True, seed=31)
    q = G.upload(w)
    a = G.to_dev(_act(M, K, seed=31))
    bias = G.to_dev(_act(1, N, seed=32).reshape(N))
    for b in (None, bias):
        outs = []
        for shift in (0, 1):
            buf = t.full((M * N + 8,), float("nan"), dtype=t.float16, device="cuda")
            y = buf[shift:shift + M * N].view(M, N)
            if b is None:
                G.gemm(q, a, M, y)
            else:
                mnb.mnb_gemm_bias(q.desc, q.repacked, a, M, b, 0, mnb.MNB_BIAS_FUSED, y, None, 0)
            outs.append(G.host(y))
        assert (outs[0] == outs[1]).all()
    w32 = _weight(N, K, g, "f32", True, seed=33)
    q32 = G.upload(w32)
    a32 = G.to_dev(_act(M, K, "f32", seed=33))
    n_ws = mnb.mnb_gemm_accuracy4_workspace_bytes(q32.desc, M)
    ws = t.zeros(n_ws, dtype=t.uint8, device="cuda")
    outs = []
    for shift in (0, 1):
        buf = t.full((M * N + 8,), float("nan"), dtype=t.float32, device="cuda")
        y = buf[shift:shift + M * N].view(M, N)
        mnb.mnb_gemm_accuracy4(q32.desc, q32.repacked, a32, M, None, y, ws, n_ws)
        outs.append(y.cpu().numpy().copy())
    assert (outs[0].view(np.uint32) == outs[1].view(np.uint32)).all()


def _sparse_row(K, seed):
    """An fp16 row that is zero except its first and last 128-k chunks and 8
    random chunks between them (~N(0,1) there): the tolerance stays tight at
    any K, so a chunk read wrongly at the far end cannot hide in it."""
    rng = np.random.default_rng(seed)
    C = K // 128
    r = np.zeros(K, np.float16)
    for c in np.concatenate([[0, C - 1], rng.choice(np.arange(1, C - 1), 8, replace=False)]):
        r[c * 128:(c + 1) * 128] = rng.standard_normal(128).astype(np.float16)
    return r


def test_prefill_at_maximum_k(mnb):
    """The prefill GEMM at its largest K (16777088 = 131071 chunks): the 16
    code tiles of a 256-column workgroup span 2^31 bytes less 16 KiB, so the
    last tile's code offsets come within 0.001% of the 32-bit limit, and the
    64 rows of A behind one buffer resource of the plain per-group path just
    as close.  M = 128 in each tile height (64: two blocks; 96: a full block
    and a partial one; 128: one block), each on one column block (N = 256).  Rows are
    sparse (_sparse_row, the memory traffic is that of a dense row); rows 0,
    1, 95, 96 and 127 are checked against the oracle on the columns of the
    first and the last tile, and the two heights give the same bits
    everywhere."""
    t = G.torch()
    M, N, g = 128, 256, 128
    K = 16777088
    w = _weight(N, K, g, "f16", True, seed=21, lo=0.002, hi=0.01)
    q = G.upload(w)
    a = t.empty((M, K), dtype=t.float16, device="cuda")
    rows = [0, 1, 95, 96, 127]
    kept = {}
    for m in range(M):
        r = _sparse_row(K, (210, m))
        a[m].copy_(t.from_numpy(r))
        if m in rows:
            kept[m] = r
    outs = {}
    try:
        for bm in (64, 96, 128):
            mnb.mnb_debug_prefill_rows(bm)
            y = t.empty((M, N), dtype=t.float16, device="cuda")
            G.gemm(q, a, M, y)
            assert mnb.mnb_last_variant() == "gemm_mfma_32x32x16"
            outs[bm] = G.host(y)
            del y
    finally:
        mnb.mnb_debug_prefill_rows(0)
    del a
    t.cuda.empty_cache()
    assert np.array_equal(outs[96].view(np.uint16), outs[128].view(np.uint16))
    assert np.array_equal(outs[96].view(np.uint16), outs[64].view(np.uint16))
    cols = np.r_[0:16, N - 16:N]
    A = np.stack([kept[m] for m in rows])
    ms = np.repeat(np.arange(len(rows)), len(cols))
    ns = np.tile(cols, len(rows))
    Y, B = o.matmul_nbits_at(A, w.packed, w.scales, w.zero_points, N, K, g, ms, ns)
    for bm in (64, 96, 128):
        G.assert_within(outs[bm][np.array(rows)[ms], ns], Y, B, "prefill (%d rows) at K=%d" % (bm, K))


@pytest.mark.parametrize("M", [16, 20])
def test_small_m_at_maximum_k(mnb, M):
    """The small-M kernel at its largest K (2^25 = 262144 chunks): 16 rows of
    fp16 A are 2^30 bytes, so the activation offsets reach 2^30; at M = 20 the
    second 16-row slice starts 2^30 bytes into A.  One workgroup (N = 16) runs
    every chunk.  Rows are sparse (_sparse_row); rows 0, 1, 7 and 15 (and 16
    and 19 at M = 20) are checked against the oracle on every column."""
    t = G.torch()
    N, g = 16, 128
    K = 1 << 25
    w = _weight(N, K, g, "f16", True, seed=22, lo=0.002, hi=0.01)
    q = G.upload(w)
    a = t.empty((M, K), dtype=t.float16, device="cuda")
    rows = [0, 1, 7, 15] + ([16, M - 1] if M > 16 else [])
    kept = {}
    for m in range(M):
        r = _sparse_row(K, (220, m))
        a[m].copy_(t.from_numpy(r))
        if m in rows:
            kept[m] = r
    y = t.empty((M, N), dtype=t.float16, device="cuda")
    G.gemm(q, a, M, y)
    assert mnb.mnb_last_variant() == "gemm_small_m"
    yh = G.host(y)
    del a
    t.cuda.empty_cache()
    A = np.stack([kept[m] for m in rows])
    ms = np.repeat(np.arange(len(rows)), N)
    ns = np.tile(np.arange(N), len(rows))
    Y, B = o.matmul_nbits_at(A, w.packed, w.scales, w.zero_points, N, K, g, ms, ns)
    G.assert_within(yh[np.array(rows)[ms], ns], Y, B, "small M at K=%d" % K)


BIAS_CASES = [
    # M, N, K, g, activation dtype, zp: every path (GEMV fp16/fp32, small M, prefill)
    (1, 300, 512, 32, "f16", True), (1, 200, 640, 64, "f32", False),
    (4, 257, 896, 32, "f16", True), (40, 300, 512, 64, "f16", True),
    (130, 70, 384, 128, "f16", False),
    # the prefill with N % 8 == 0: outputs staged in LDS and stored 16 bytes
    # per lane, the bias read per output element (ragged M)
    (130, 264, 384, 128, "f16", True), (75, 512, 640, 64, "f16", False),
]


@pytest.mark.parametrize("M,N,K,g,adt,zp", BIAS_CASES)
def test_bias_epilogue_parity(mnb, prefill_rows, M, N, K, g, adt, zp):
    """The bias epilogue on every path, one bias vector for all rows (stride
    0) and a per-row residual (stride N + 5).  After-round mode must equal,
    bit for bit, the oracle's epilogue applied to the unbiased output (the
    two-operator path); fused mode is checked against Y + b (fp64) under the
    accumulator's bound plus one fp32 add and one fp16 rounding; a zero bias
    changes nothing.  fp32 outputs add once in both modes."""
    G.needs_forced_height(prefill_rows, g, M)
    t = G.torch()
    w = _weight(N, K, g, "f16", zp, seed=M)
    A = _act(M, K, adt, seed=M + 1)
    q = G.upload(w)
    odt = t.float16 if adt == "f16" else t.float32
    ndt = np.float16 if adt == "f16" else np.float32
    a = G.to_dev(A)
    y0 = t.empty((M, N), dtype=odt, device="cuda")
    G.gemm(q, a, M, y0)
    y0h = y0.cpu().numpy()
    Y, B, _ = G.oracle_dense(A, w)
    rng = np.random.default_rng(M * 7 + N)
    for stride in (0, N + 5):
        rows = M if stride else 1
        bias = np.zeros((rows, max(stride, N)), dtype=ndt)
        bias[:, :N] = (rng.standard_normal((rows, N)) * 2.0).astype(ndt)
        bias_dev = G.to_dev(bias.reshape(-1))
        b_mn = np.broadcast_to(bias[:, :N], (M, N)) if stride == 0 else bias[:, :N]
        ws, n_ws = G.workspace(q, M)
        outs = {}
        for mode in (mnb.MNB_BIAS_FUSED, mnb.MNB_BIAS_AFTER_ROUND):
            y = t.empty((M, N), dtype=odt, device="cuda")
            mnb.mnb_gemm_bias(q.desc, q.repacked, a, M, bias_dev, stride, mode, y, ws, n_ws)
            outs[mode] = y.cpu().numpy()
        yf, ya = outs[mnb.MNB_BIAS_FUSED], outs[mnb.MNB_BIAS_AFTER_ROUND]
        what = "bias M=%d N=%d K=%d g=%d %s stride=%d" % (M, N, K, g, adt, stride)
        if adt == "f16":
            want = o.bias_epilogue_f16(y0h.astype(np.float32), b_mn, True)
            assert (ya.view(np.uint16) == want.view(np.uint16)).all(), what + " (after-round)"
        else:
            assert (yf.view(np.uint32) == ya.view(np.uint32)).all(), what
            assert (yf == (y0h + b_mn)).all(), what
        b64 = b_mn.astype(np.float64)
        ok = np.abs(yf.astype(np.float64) - (Y + b64)) <= o.bias_bound(Y, B, b64)
        assert ok.all(), "%s (fused): %d of %d outside" % (what, (~ok).sum(), ok.size)
    # a zero bias is the plain GEMM
    zb = G.to_dev(np.zeros(N, dtype=ndt))
    for mode in (mnb.MNB_BIAS_FUSED, mnb.MNB_BIAS_AFTER_ROUND):
        y = t.empty((M, N), dtype=odt, device="cuda")
        ws, n_ws = G.workspace(q, M)
        mnb.mnb_gemm_bias(q.desc, q.repacked, a, M, zb, 0, mode, y, ws, n_ws)
        assert (y.cpu().numpy() == y0h).all()


ACT_ORDER_CASES = [
    # M, N, K, g, activation dtype, zp: every path after the column permutation
    (1, 300, 512, 32, "f16", True), (1, 200, 640, 64, "f32", False),
    (4, 257, 896, 32, "f16", True), (40, 300, 512, 64, "f16", True),
    (130, 70, 384, 128, "f16", False),
    # decode beyond the K at which the GEMV holds both copies of A in LDS:
    # the separate column permutation, then the plain GEMV
    (1, 48, 16384, 128, "f16", True), (1, 40, 8192, 64, "f32", False),
    # K not a multiple of the 128-k chunk (the gather's padding) on every path
    (1, 60, 400, 16, "f16", True), (1, 50, 352, 32, "f32", False), (6, 60, 400, 16, "f16", True),
    (70, 60, 352, 32, "f16", False),
    # rows longer than the LDS a workgroup gets (64 KiB): the gathering
    # permutation instead of the row-staged one
    (2, 24, 33280, 128, "f16", True),
]


@pytest.mark.parametrize("M,N,K,g,adt,zp", ACT_ORDER_CASES)
def test_act_order_parity(mnb, prefill_rows, M, N, K, g, adt, zp):
    """Act-order weights (random g_idx, every group of exactly g positions):
    the repack in permuted order and the GEMM on permuted activation columns,
    against the oracle's act-order dequant (scale and zero point of group
    g_idx[k]) and fp64 matmul, on every path."""
    G.needs_forced_height(prefill_rows, g, M)
    t = G.torch()
    w = _weight(N, K, g, "f16", zp, seed=M + 3)
    rng = np.random.default_rng(M * 31 + K)
    g_idx = np.empty(K, np.int32)
    g_idx[rng.permutation(K)] = np.arange(K) // g
    A = _act(M, K, adt, seed=M + 5)
    d = mnb.desc(N, K, g, zp, mnb.MNB_F16)
    perm = mnb.mnb_act_order_permutation(d, g_idx)
    perm_dev = G.to_dev(perm)
    rep = t.empty(mnb.mnb_repacked_bytes(d), dtype=t.uint8, device="cuda")
    mnb.mnb_repack_act_order(d, G.to_dev(w.packed.reshape(-1)), G.to_dev(w.scales.reshape(-1)),
                             None if w.zero_points is None else G.to_dev(w.zero_points.reshape(-1)),
                             perm_dev, rep)
    n_ws = mnb.mnb_gemm_act_order_workspace_bytes(d, M, mnb.MNB_F16 if adt == "f16" else mnb.MNB_F32)
    ws = t.zeros(n_ws, dtype=t.uint8, device="cuda")
    y = t.empty((M, N), dtype=t.float16 if adt == "f16" else t.float32, device="cuda")
    mnb.mnb_gemm_act_order(d, rep, G.to_dev(A), M, perm_dev, y, ws, n_ws)
    W = o.dequant_gidx(w.packed, w.scales, w.zero_points, g_idx, N, K, g)
    Y, B = o.matmul(o.decode(A.reshape(-1, K)), W)
    G.assert_within(G.host(y), Y, B, "act order M=%d N=%d K=%d g=%d %s" % (M, N, K, g, adt))
    # the plain repack of the same operands is a different weight unless the
    # order is the identity
    assert not (perm == np.arange(K)).all()
    if M == 1:
        f16 = adt == "f16"
        gathered = K <= (15872 if f16 else 7936)
        suffix = "f16" if f16 else "f32"
        assert mnb.mnb_last_variant() == ("gemv_act_order_" if gathered else "gemv_") + suffix
        # a perm that is not 16-byte aligned takes the separate permutation;
        # both paths feed the GEMV the same values, so the results agree bit
        # for bit
        shifted = t.zeros(K + 1, dtype=t.int32, device="cuda")
        shifted[1:] = perm_dev
        y2 = t.empty_like(y)
        mnb.mnb_gemm_act_order(d, rep, G.to_dev(A), M, shifted[1:], y2, ws, n_ws)
        assert mnb.mnb_last_variant() == "gemv_" + suffix
        t.cuda.synchronize()
        assert t.equal(y, y2)


GIDX_CASES = [
    # M, N, K, g, activation dtype, scale dtype, zp, how g_idx is drawn
    (1, 300, 512, 32, "f32", "f32", True, "random"),    # the fp32 operator's decode
    (1, 257, 400, 16, "f16", "f16", True, "random"),    # K not a multiple of the 128-k chunk
    (5, 1000, 1024, 64, "f32", "f16", False, "random"),
    (40, 70, 384, 128, "f16", "f32", True, "skewed"),   # sizes far from g, some groups empty
    (130, 60, 896, 32, "f32", "f32", False, "one"),     # every k in one group
    (17, 48, 512, 32, "f16", "f16", True, "whole"),     # whole groups: the sorted route's input
    (3, 40, 640, 64, "f32", "f16", True, "range"),      # values outside 0..k_blocks-1 weigh 0
    (16, 33, 512, 32, "f16", "f16", True, "random"),    # the largest M of the streaming kernel
    (6, 60, 400, 16, "f16", "f16", True, "skewed"),     # its matrix-core products over a K tail
    (17, 200, 1024, 16, "f32", "f32", True, "random"),  # the smallest of the matrix-core kernel
    (300, 130, 768, 128, "f16", "f16", False, "range"),
    # a table of 688 groups (88 KiB of LDS); metadata too large for LDS (2048
    # groups; 512 groups of fp32 scales and zero points for the four tiles of
    # the matrix-core kernel): read from L2
    (1, 40, 11008, 16, "f16", "f32", True, "random"),
    (2, 40, 32768, 16, "f16", "f32", True, "random"),
    (70, 48, 8192, 16, "f32", "f32", True, "random"),
    (20, 40, 11008, 16, "f32", "f16", True, "random"),   # 64-row blocks, table too large (88 KiB)
]


def _g_idx(kind, K, kb, rng):
    if kind == "random":
        return rng.integers(0, kb, K).astype(np.int32)
    if kind == "skewed":
        # group b drawn with weight 2^-b: a few large groups, many empty
        p = 0.5 ** np.arange(kb)
        return rng.choice(kb, K, p=p / p.sum()).astype(np.int32)
    if kind == "one":
        return np.full(K, kb // 2, np.int32)
    if kind == "whole":
        g = np.empty(K, np.int32)
        g[rng.permutation(K)] = np.arange(K) // (K // kb)
        return g
    g = rng.integers(0, kb, K).astype(np.int32)
    g[rng.choice(K, K // 8, replace=False)] = rng.choice(np.array([-1, kb, -(1 << 30), 1 << 30], np.int32), K // 8)
    return g


@pytest.mark.parametrize("M,N,K,g,adt,sdt,zp,kind", GIDX_CASES)
def test_group_indices_parity(mnb, M, N, K, g, adt, sdt, zp, kind):
    """Any g_idx through the general route (plain repack, scale and zero
    point of group g_idx[k] looked up per k): against the oracle's act-order
    dequant and fp64 matmul, without a bias, with a bias vector and with a
    per-row bias (fused mode under its bound, after-round mode bit for bit
    against the oracle's epilogue on the unbiased output); two calls agree
    bit for bit; the host check's answer for this g_idx."""
    t = G.torch()
    kb = K // g
    w = _weight(N, K, g, sdt, zp, seed=M + 11)
    rng = np.random.default_rng(M * 131 + K + kb)
    g_idx = _g_idx(kind, K, kb, rng)
    A = _act(M, K, adt, seed=M + 12)
    q = G.upload(w)
    gi = G.to_dev(g_idx)
    a = G.to_dev(A)
    odt = t.float16 if adt == "f16" else t.float32
    ndt = np.float16 if adt == "f16" else np.float32
    y = t.empty((M, N), dtype=odt, device="cuda")
    mnb.mnb_gemm_group_indices(q.desc, q.repacked, a, M, gi, y)
    assert mnb.mnb_last_variant() == "gemm_gidx_stream_" + adt
    y2 = t.empty_like(y)
    mnb.mnb_gemm_group_indices(q.desc, q.repacked, a, M, gi, y2)
    W = o.dequant_gidx(w.packed, w.scales, w.zero_points, g_idx, N, K, g)
    Y, B = o.matmul(o.decode(A.reshape(-1, K)), W)
    what = "group indices %s M=%d N=%d K=%d g=%d %s/%s" % (kind, M, N, K, g, adt, sdt)
    G.assert_within(G.host(y), Y, B, what)
    assert t.equal(y, y2), what + " (two calls)"
    y0h = y.cpu().numpy()
    for stride in (0, N):
        rows = M if stride else 1
        bias = (rng.standard_normal((rows, N)) * 2.0).astype(ndt)
        bias_dev = G.to_dev(bias.reshape(-1))
        b64 = np.broadcast_to(bias.astype(np.float64), (M, N))
        outs = {}
        for mode in (mnb.MNB_BIAS_FUSED, mnb.MNB_BIAS_AFTER_ROUND):
            yb = t.empty((M, N), dtype=odt, device="cuda")
            mnb.mnb_gemm_group_indices(q.desc, q.repacked, a, M, gi, yb, bias_dev, stride, mode)
            outs[mode] = yb.cpu().numpy()
        yf, ya = outs[mnb.MNB_BIAS_FUSED], outs[mnb.MNB_BIAS_AFTER_ROUND]
        b_mn = np.broadcast_to(bias, (M, N))
        if adt == "f16":
            want = o.bias_epilogue_f16(y0h.astype(np.float32), b_mn, True)
            assert (ya.view(np.uint16) == want.view(np.uint16)).all(), what + " (after-round)"
            tol = o.bias_bound(Y, B, b64)
        else:
            assert (yf.view(np.uint32) == ya.view(np.uint32)).all(), what
            assert (yf == (y0h + b_mn)).all(), what
            tol = o.REL_TOL * B + o.ABS_TOL + 2.0 ** -23 * np.abs(Y + b64)
        G.assert_within(yf.astype(np.float64), Y + b64, B, what + " bias stride %d" % stride, bound=tol)
    # the host check: whole groups are the sorted route's, others this one's
    d = mnb.desc(N, K, g, zp, mnb.MNB_F16 if sdt == "f16" else mnb.MNB_F32)
    if kind == "whole":
        mnb.mnb_act_order_permutation(d, g_idx)
    else:
        with pytest.raises(mnb.MnbError) as e:
            mnb.mnb_act_order_permutation(d, g_idx)
        want = mnb.MNB_ERR_INVALID_ARGUMENT if kind == "range" else mnb.MNB_ERR_UNSUPPORTED
        assert e.value.status == want


# ------------------------------------------------------------ properties ----

def test_results_are_deterministic(mnb):
    t = G.torch()
    for (M, N, K, g) in ((1, 4096, 4096, 32), (8, 1000, 4096, 64), (200, 512, 1024, 128)):
        w = _weight(N, K, g)
        q = G.upload(w)
        a = G.to_dev(_act(M, K))
        y1 = t.empty((M, N), dtype=t.float16, device="cuda")
        y2 = t.empty_like(y1)
        G.gemm(q, a, M, y1)
        G.gemm(q, a, M, y2)
        t.cuda.synchronize()
        assert t.equal(y1, y2)


def test_absent_zero_points_equal_explicit_eights(mnb):
    t = G.torch()
    for (M, N, K, g) in ((1, 200, 512, 32), (4, 96, 1024, 64), (40, 64, 256, 128), (64, 64, 256, 128)):
        w = _weight(N, K, g, zp=False)
        kb = K // g
        w8 = synth.Weight(N, K, g, w.packed, w.scales, np.full((N, (kb + 1) // 2), 0x88, np.uint8))
        q, q8 = G.upload(w), G.upload(w8)
        a = G.to_dev(_act(M, K))
        y, y8 = (t.empty((M, N), dtype=t.float16, device="cuda") for _ in range(2))
        G.gemm(q, a, M, y)
        G.gemm(q8, a, M, y8)
        t.cuda.synchronize()
        assert t.equal(y, y8)


def test_code_equal_to_zero_point_gives_zero(mnb):
    t = G.torch()
    for (M, N, K, g) in ((1, 48, 256, 32), (5, 48, 256, 16), (64, 48, 256, 128)):
        kb = K // g
        rng = np.random.default_rng(M)
        z = rng.integers(0, 16, (N, kb), dtype=np.uint8)
        packed = o.pack_codes(np.repeat(z, g, axis=1), g)
        w = synth.Weight(N, K, g, packed, rng.uniform(1, 2, (N, kb)).astype(np.float16),
                         o.pack_zero_points(z))
        q = G.upload(w)
        y = t.full((M, N), 7.0, dtype=t.float16, device="cuda")
        G.gemm(q, G.to_dev(_act(M, K)), M, y)
        assert (G.host(y) == 0.0).all()


def test_nan_and_inf_propagate(mnb):
    """A NaN and an infinite activation on every path (GEMV, small M, its
    16-row slices, prefill), also with groups of 16 k, where one 32-k MFMA
    step holds two groups: the infinity reaches only its own group's weight."""
    t = G.torch()
    for (M, N, K, g) in ((1, 40, 256, 32), (3, 40, 256, 32), (20, 40, 256, 32), (1, 40, 256, 16),
                         (3, 40, 256, 16), (20, 40, 256, 16), (60, 40, 256, 16)):
        w = _weight(N, K, g)
        A = _act(M, K)
        A[0, 7] = np.nan
        if M > 1:
            A[M - 1, 100] = np.inf
        q = G.upload(w)
        y = t.empty((M, N), dtype=t.float16, device="cuda")
        G.gemm(q, G.to_dev(A), M, y)
        Y, B, _ = G.oracle_dense(A, w)
        G.assert_within(G.host(y), Y, B, "nan/inf M=%d" % M)


def test_zero_and_non_finite_scales(mnb, prefill_rows):
    """Groups whose scale is 0 add exactly nothing, and a NaN scale makes
    its column NaN, on every path: GEMV, small M, MFMA.  The same weights are
    checked at several group sizes and both scale dtypes (the dequantized
    weight (c - z) * s is exact in fp64).  Infinite scales are left out: the
    oracle dequantizes first, (c - z) * inf, which is NaN wherever a code
    equals its zero point, while scaling a group's sum gives +-inf; the
    stored format carries finite scales."""
    t = G.torch()
    for (N, K, g, sdt) in ((64, 512, 128, "f16"), (48, 384, 32, "f16"), (40, 256, 64, "f32")):
        w = _weight(N, K, g, sdt, seed=7)
        kb = K // g
        rng = np.random.default_rng(N + K)
        s = w.scales.copy()
        # a third of all groups, at random, have scale 0; column 3 has every
        # scale 0; column 9 one NaN scale
        s[rng.random((N, kb)) < 0.33] = 0
        s[3, :] = 0
        s[9, 0] = np.nan
        w2 = synth.Weight(N, K, g, w.packed, s.astype(w.scales.dtype), w.zero_points)
        q = G.upload(w2)
        for M in (1, 4, 40, 64):
            A = _act(M, K, seed=M)
            y = t.empty((M, N), dtype=t.float16, device="cuda")
            G.gemm(q, G.to_dev(A), M, y)
            Y, B, _ = G.oracle_dense(A, w2)
            yh = G.host(y)
            G.assert_within(yh, Y, B, "special scales M=%d N=%d K=%d g=%d %s" % (M, N, K, g, sdt))
            assert (yh[:, 3] == 0).all()


F32_CASES = [
    # M, N, K, g, scale dtype, zero points: the small-M kernel on 2M <= 16
    # rows, the prefill kernel beyond, K tails, every group size
    (2, 200, 512, 32, "f16", True), (5, 257, 896, 64, "f32", False), (8, 130, 384, 128, "f16", True),
    (9, 96, 1024, 16, "f16", True), (16, 300, 512, 64, "f32", True), (40, 513, 1024, 32, "f16", True),
    (200, 300, 384, 128, "f16", False), (33, 70, 400, 16, "f32", True), (3, 70, 352, 32, "f16", True),
    (70, 256, 512, 32, "f16", True),
    # 2M <= 48: the small-M kernel on slices of 8 rows (16 fp16 rows), the last ragged
    (24, 130, 384, 128, "f16", False), (13, 257, 640, 64, "f32", True)]


def _f32_rows(M, K, seed):
    """fp32 activations N(0,1) with special rows: huge, tiny, mixed
    magnitudes, a NaN, an infinity, zeros, a subnormal-only row."""
    A = synth.activation(M, K, "f32", 1.0, (230, M, K, seed))
    rng = np.random.default_rng(M + K)
    specials = [lambda r: r * np.float32(1e30), lambda r: r * np.float32(1e-30),
                lambda r: np.where(rng.random(K) < 0.5, r * 1e6, r * 1e-6).astype(np.float32),
                lambda r: np.where(np.arange(K) == 3, np.float32(np.nan), r),
                lambda r: np.where(np.arange(K) == 7, np.float32(np.inf), r),
                lambda r: np.zeros_like(r), lambda r: (r * np.float32(1e-40)).astype(np.float32)]
    for j, f in enumerate(specials):
        if j < M:
            A[(j * 7) % M] = f(A[(j * 7) % M])
    return A


@pytest.mark.parametrize("M,N,K,g,sdt,zp", F32_CASES)
def test_f32_activations_gemm_parity(mnb, prefill_rows, M, N, K, g, sdt, zp):
    """fp32 activations with M > 1: rows split into fp16 (hi, lo) pairs under
    a power-of-two row scale, the fp16 GEMM on the 2M rows, the pairs summed
    and scaled back in fp32.  Against the oracle on the fp32 values (exact in
    fp64), with huge, tiny, subnormal, NaN and infinite rows, and with an fp32
    bias vector and a per-row bias."""
    G.needs_forced_height(prefill_rows, g, 2 * M)
    t = G.torch()
    w = _weight(N, K, g, sdt, zp, seed=M + 21)
    q = G.upload(w)
    A = _f32_rows(M, K, 1)
    a = G.to_dev(A)
    y = t.empty((M, N), dtype=t.float32, device="cuda")
    G.gemm(q, a, M, y)
    expect = "gemm_small_m_f32act" if 2 * M <= 48 else "gemm_mfma_32x32x16_f32act"
    assert mnb.mnb_last_variant() == expect
    Y, B, W64 = G.oracle_dense(A, w)
    G.assert_within(G.host(y), Y, B, "fp32 activations M=%d N=%d K=%d g=%d" % (M, N, K, g))
    # bias: a vector, then a per-row residual [M, N + 3]; the fp32 add is
    # covered by the rule applied to sum |a w| + |b|
    ws, n = G.workspace(q, M, mnb.MNB_F32)
    rows_ok = np.isfinite(A).all(axis=1)
    for stride in (0, N + 3):
        rows = 1 if stride == 0 else M
        b = synth.activation(rows, max(stride, N), "f32", 2.0, (231, M, stride))
        mnb.mnb_gemm_bias(q.desc, q.repacked, a, M, G.to_dev(b), stride, mnb.MNB_BIAS_FUSED, y, ws, n)
        b64 = (b[0, :N][None, :] if stride == 0 else b[:, :N]).astype(np.float64)
        yh = G.host(y)
        G.assert_within(yh[rows_ok], (Y + b64)[rows_ok], (B + np.abs(b64))[rows_ok],
                        "fp32 activations + bias stride %d" % stride)


def test_f32_activations_act_order(mnb):
    """Act-order weights with fp32 activations and M > 1: the columns of A
    permuted in fp32, then the row-pair GEMM."""
    t = G.torch()
    for (M, N, K, g) in ((4, 96, 512, 32), (40, 130, 1024, 128)):
        w = _weight(N, K, g, "f16", True, seed=M + 9)
        rng = np.random.default_rng(M * 7 + K)
        g_idx = np.empty(K, np.int32)
        g_idx[rng.permutation(K)] = np.arange(K) // g
        A = _act(M, K, "f32", seed=M + 11)
        d = mnb.desc(N, K, g, True, mnb.MNB_F16)
        perm = G.to_dev(mnb.mnb_act_order_permutation(d, g_idx))
        rep = t.empty(mnb.mnb_repacked_bytes(d), dtype=t.uint8, device="cuda")
        mnb.mnb_repack_act_order(d, G.to_dev(w.packed.reshape(-1)), G.to_dev(w.scales.reshape(-1)),
                                 G.to_dev(w.zero_points.reshape(-1)), perm, rep)
        n_ws = mnb.mnb_gemm_act_order_workspace_bytes(d, M, mnb.MNB_F32)
        ws = t.zeros(n_ws, dtype=t.uint8, device="cuda")
        y = t.empty((M, N), dtype=t.float32, device="cuda")
        mnb.mnb_gemm_act_order(d, rep, G.to_dev(A), M, perm, y, ws, n_ws)
        W = o.dequant_gidx(w.packed, w.scales, w.zero_points, g_idx, N, K, g)
        Y, B = o.matmul(o.decode(A), W)
        G.assert_within(G.host(y), Y, B, "act order fp32 M=%d N=%d K=%d g=%d" % (M, N, K, g))


def _extreme_scales(N, kb, base, big=False):
    """fp32 scales [N, kb] from `base` with columns whose groups span extreme
    ranges: a tiny scale beside ordinary ones (ratio about 2^90), a
    subnormal one, one at the smallest normal binary32 value beside 0.02, a
    spread of exactly 2^64 and one of 2^60 (inside the prefill's range
    class), and with big=True a 1e30 scale beside 1e-30."""
    s = base.astype(np.float64).copy()
    s[17, 0] = 1e-30                      # tile 1: ratio ~2^90
    s[33, 1 % kb] = 1e-39                 # tile 2: subnormal
    s[66, 0] = 1.1754944e-38              # tile 4: smallest normal beside 0.02
    s[66, kb - 1] = 0.02
    s[80, :] = 0.01                       # tile 5: spread exactly 2^64
    s[80, 0] = 0.01 * 2.0 ** -64
    s[50, ::2] = 0.01 * 2.0 ** -60        # tile 3: spread 2^60, alternating
    if big:
        s[90, 0], s[90, kb - 1] = 1e30, 1e-30
    return s.astype(np.float32)


@pytest.mark.parametrize("K,g", [(512, 128), (512, 32), (400, 16)])
def test_extreme_scale_ranges(mnb, prefill_rows, K, g):
    """fp32 scales whose magnitudes within a column differ by up to 2^121, or
    are subnormal, on every path: the GEMV and small-M kernels apply each
    group's scale to a fresh partial; the prefill GEMM keeps one rescaled
    accumulator for tiles in its range class (recorded by the repack, checked
    here against the host model) and computes the other tiles with fresh
    partials.  Outputs within the bound everywhere."""
    G.needs_forced_height(prefill_rows, g)
    t = G.torch()
    N = 96
    kb = K // g
    w = _weight(N, K, g, "f32", seed=11)
    s = _extreme_scales(N, kb, w.scales)
    w2 = synth.Weight(N, K, g, w.packed, s, w.zero_points)
    q = G.upload(w2)
    flags = layout_ref.range_flags(s, N)
    assert flags.tolist() == [1, 0, 0, 1, 0, 1]
    Gm = layout_ref.geometry(N, K, g, True, False)
    assert (q.repacked.cpu().numpy()[Gm["F0"]:Gm["F0"] + Gm["T"]] == flags).all()
    for M in (1, 8, 40, 200):
        A = _act(M, K, seed=M + 5)
        y = t.empty((M, N), dtype=t.float16, device="cuda")
        G.gemm(q, G.to_dev(A), M, y)
        Y, B, _ = G.oracle_dense(A, w2)
        G.assert_within(G.host(y), Y, B, "extreme scales M=%d K=%d g=%d (%s)" % (M, K, g, mnb.mnb_last_variant()))


@pytest.mark.parametrize("K,g", [(512, 128), (400, 16)])
def test_extreme_scale_ranges_int8_activations(mnb, prefill_rows, K, g):
    """The same extreme scales, plus a 1e30 scale beside a 1e-30 one, through
    the int8-activation product (fp32 outputs hold the large values)."""
    G.needs_forced_height(prefill_rows, g)
    t = G.torch()
    N = 96
    kb = K // g
    w = _weight(N, K, g, "f32", seed=12)
    w2 = synth.Weight(N, K, g, w.packed, _extreme_scales(N, kb, w.scales, big=True), w.zero_points)
    q = G.upload(w2)
    for M in (1, 8, 40, 200):
        A = synth.activation(M, K, "f32", 1.0, (205, M, K))
        ws = t.zeros(max(mnb.mnb_gemm_accuracy4_workspace_bytes(q.desc, M), 256), dtype=t.uint8, device="cuda")
        y = t.empty((M, N), dtype=t.float32, device="cuda")
        mnb.mnb_gemm_accuracy4(q.desc, q.repacked, G.to_dev(A), M, None, y, ws, ws.numel())
        Y, B, _, _ = o.acc4_matmul(A, w2.packed, w2.scales, w2.zero_points, N, K, g)
        G.assert_within(G.host(y), Y, B, "int8 activations, extreme scales M=%d K=%d g=%d" % (M, K, g),
                        bound=o.acc4_bound(B, K, g))


def test_empty_and_unsupported_requests(mnb):
    t = G.torch()
    w = _weight(64, 256, 32)
    q = G.upload(w)
    y = t.full((1, 64), 3.0, dtype=t.float16, device="cuda")
    mnb.mnb_gemm(q.desc, q.repacked, G.to_dev(_act(1, 256)), 0, y)
    assert (G.host(y) == 3.0).all()
    with pytest.raises(mnb.MnbError) as e:
        # fp32 activations with M > 1 need their workspace
        mnb.mnb_gemm(q.desc, q.repacked, G.to_dev(_act(4, 256, "f32")), 4,
                     t.empty((4, 64), dtype=t.float32, device="cuda"))
    assert e.value.status == mnb.MNB_ERR_INVALID_ARGUMENT

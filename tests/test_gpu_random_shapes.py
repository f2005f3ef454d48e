"""Seeded random shapes through every path, against the oracle.

Each case draws M (decode, small-M and prefill sizes), N and K (ragged against
the 16-column tile and the 128-k chunk), the group size, the scale dtype and
zero points, then runs one of the calls: the plain product, the bias epilogue
(either rounding), act order, or int8 activations.  The bars are those of the
other parity tests.
"""
import numpy as np
import pytest

from block_wise_int4_amd import synth
from oracle import oracle as o
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

N_CASES = 48


def _draw(i):
    rng = np.random.default_rng((500, i))
    g = int(rng.choice([16, 32, 64, 128]))
    K = g * int(rng.integers(1, max(2, 1536 // g) + 1))
    N = int(rng.integers(1, 400))
    M = int(rng.choice([1, 1, int(rng.integers(2, 17)), int(rng.integers(17, 200))]))
    sdt = str(rng.choice(["f16", "f32"]))
    zp = bool(rng.integers(0, 2))
    kind = str(rng.choice(["plain", "bias", "act_order", "accuracy4"]))
    return M, N, K, g, sdt, zp, kind, rng


N_PREFILL_CASES = 16


def _draw_prefill(i):
    """Prefill shapes with groups of 128 or 64 k, the ones with several tile
    heights."""
    rng = np.random.default_rng((510, i))
    g = int(rng.choice([64, 128]))
    K = g * int(rng.integers(1, 13))
    N = int(rng.integers(1, 400))
    M = int(rng.integers(49, 300))
    sdt = str(rng.choice(["f16", "f32"]))
    zp = bool(rng.integers(0, 2))
    kind = str(rng.choice(["plain", "bias", "act_order", "accuracy4"]))
    return M, N, K, g, sdt, zp, kind, rng


@pytest.fixture(scope="module")
def mnb():
    from block_wise_int4_amd import mnb as m
    return m


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(mnb, i):
    _run_case(mnb, i, *_draw(i), seed=500)


@pytest.mark.parametrize("i", range(N_PREFILL_CASES))
def test_random_prefill_shape_in_every_tile_height(mnb, i):
    """The prefill GEMM's tile heights (64, 96 and 128 rows, forced; 128 only
    for groups of 128 k) on seeded shapes with groups of 128 or 64 k: each
    within the bound against the oracle, and all bit for bit the same."""
    outs = []
    try:
        for rows in (64, 96, 128):
            assert mnb.mnb_debug_prefill_rows(rows) in (0, 64, 96, 128)
            outs.append(_run_case(mnb, i, *_draw_prefill(i), seed=510))
    finally:
        mnb.mnb_debug_prefill_rows(0)
    for o_ in outs[1:]:
        assert o_.dtype == outs[0].dtype
        assert np.array_equal(outs[0].view(np.uint8), o_.view(np.uint8)), "case %d: the heights differ" % i


def _run_case(mnb, i, M, N, K, g, sdt, zp, kind, rng, seed):
    """One drawn case through its call, checked against the oracle; returns
    the output on the host."""
    t = G.torch()
    what = "case %d/%d: %s M=%d N=%d K=%d g=%d %s zp=%s" % (seed, i, kind, M, N, K, g, sdt, zp)
    print(what, flush=True)
    w = synth.weight(N, K, g, sdt, (0.005, 0.02), zp, (seed + 1, i))
    if kind == "accuracy4":
        A = synth.activation(M, K, "f32", 1.0, (seed + 2, i))
        bias = synth.activation(1, N, "f32", 1.0, (seed + 3, i)).reshape(N) if rng.integers(0, 2) else None
        q = G.upload(w)
        n_ws = mnb.mnb_gemm_accuracy4_workspace_bytes(q.desc, M)
        ws = t.zeros(n_ws, dtype=t.uint8, device="cuda")
        y = t.empty((M, N), dtype=t.float32, device="cuda")
        mnb.mnb_gemm_accuracy4(q.desc, q.repacked, G.to_dev(A), M, None if bias is None else G.to_dev(bias),
                               y, ws, n_ws)
        Y, B, qc, sc = o.acc4_matmul(A, w.packed, w.scales, w.zero_points, N, K, g, bias)
        raw = ws.cpu().numpy()
        off = (4 * M + 255) // 256 * 256
        codes = raw[off:off + 2 * M * K].view(np.float16).reshape(M, K).astype(np.float64)
        assert (codes == qc).all(), what
        assert (raw[:4 * M].view(np.uint32) == sc.view(np.uint32)).all(), what
        yh = G.host(y)
        G.assert_within(yh, Y, B, what, bound=o.acc4_bound(B, K, g))
        return yh
    # fp16 activations for every GEMM; fp32 only at M = 1
    adt = "f32" if (M == 1 and rng.integers(0, 3) == 0) else "f16"
    A = synth.activation(M, K, adt, 1.0, (seed + 4, i))
    odt = t.float16 if adt == "f16" else t.float32
    y = t.empty((M, N), dtype=odt, device="cuda")
    if kind == "act_order":
        g_idx = np.empty(K, np.int32)
        g_idx[rng.permutation(K)] = np.arange(K) // g
        d = mnb.desc(N, K, g, zp, mnb.MNB_F16 if sdt == "f16" else mnb.MNB_F32)
        perm = G.to_dev(mnb.mnb_act_order_permutation(d, g_idx))
        rep = t.empty(mnb.mnb_repacked_bytes(d), dtype=t.uint8, device="cuda")
        mnb.mnb_repack_act_order(d, G.to_dev(w.packed.reshape(-1)), G.to_dev(w.scales.reshape(-1)),
                                 None if w.zero_points is None else G.to_dev(w.zero_points.reshape(-1)),
                                 perm, rep)
        n_ws = mnb.mnb_gemm_act_order_workspace_bytes(d, M, mnb.MNB_F16 if adt == "f16" else mnb.MNB_F32)
        ws = t.zeros(n_ws, dtype=t.uint8, device="cuda")
        mnb.mnb_gemm_act_order(d, rep, G.to_dev(A), M, perm, y, ws, n_ws)
        W = o.dequant_gidx(w.packed, w.scales, w.zero_points, g_idx, N, K, g)
        Y, B = o.matmul(o.decode(A.reshape(-1, K)), W)
        yh = G.host(y)
        G.assert_within(yh, Y, B, what)
        return yh
    q = G.upload(w)
    ws, n = G.workspace(q, M)
    if kind == "bias":
        after = bool(rng.integers(0, 2))
        bias = synth.activation(1, N, adt, 1.0, (seed + 5, i)).reshape(N)
        mnb.mnb_gemm_bias(q.desc, q.repacked, G.to_dev(A), M, G.to_dev(bias), 0,
                          mnb.MNB_BIAS_AFTER_ROUND if after else mnb.MNB_BIAS_FUSED, y, ws, n)
        Y, B = o.matmul_nbits(A, w.packed, w.scales, w.zero_points, N, K, g)
        b64 = o.decode(bias).reshape(1, N)
        if adt == "f16":
            bound = o.bias_bound(Y, B, b64)
        else:
            bound = o.REL_TOL * B + o.ABS_TOL + 2.0 ** -24 * np.abs(Y + b64)
        yh = G.host(y)
        G.assert_within(yh, Y + b64, B, what, bound=bound)
        return yh
    mnb.mnb_gemm(q.desc, q.repacked, G.to_dev(A), M, y, ws, n)
    Y, B = o.matmul_nbits(A, w.packed, w.scales, w.zero_points, N, K, g)
    yh = G.host(y)
    G.assert_within(yh, Y, B, what)
    return yh

"""Helpers shared by the GPU tests: upload seeded operands, run the C ABI,
compare with the oracle under the per-element bound."""
import numpy as np
import pytest

from block_wise_int4_amd import synth
from oracle import oracle as o


def torch():
    import torch as _t
    return _t


def to_dev(x: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x)).cuda()


def upload(w: synth.Weight):
    from block_wise_int4_amd import mnb
    packed = to_dev(w.packed.reshape(-1))
    scales = to_dev(w.scales.reshape(-1))
    zp = to_dev(w.zero_points.reshape(-1)) if w.zero_points is not None else None
    q = mnb.repack(packed, scales, zp, w.N, w.K, w.group)
    torch().cuda.synchronize()
    return q


_WS = {}


def workspace(q, M, a_dtype=None):
    """A GEMM workspace for (q, M) and the activation dtype (zero-filled),
    shared by every call that fits in it."""
    from block_wise_int4_amd import mnb
    n = mnb.mnb_gemm_workspace_bytes_for(q.desc, M, mnb.MNB_F16 if a_dtype is None else a_dtype)
    buf = _WS.get("buf")
    if buf is None or buf.numel() < n:
        buf = torch().zeros(max(n, 256), dtype=torch().uint8, device="cuda")
        _WS["buf"] = buf
    return buf, n


def gemm(q, a, M, y, stream=None):
    from block_wise_int4_amd import mnb
    ws, n = workspace(q, M, mnb._dtype_code(a))
    mnb.mnb_gemm(q.desc, q.repacked, a, M, y, ws, n, stream=stream)


def host(y) -> np.ndarray:
    torch().cuda.synchronize()
    return y.detach().cpu().numpy().astype(np.float64)


def oracle_dense(A: np.ndarray, w: synth.Weight, W64=None):
    """(Y, Bnd, W64) over all outputs, via the oracle's dequant + matmul."""
    if W64 is None:
        W64 = o.dequant(w.packed, w.scales, w.zero_points, w.N, w.K, w.group)
    Y, B = o.matmul(o.decode(A.reshape(-1, w.K)), W64)
    return Y, B, W64


def assert_within(y: np.ndarray, Y: np.ndarray, B: np.ndarray, what: str, bound=None):
    y = np.asarray(y, np.float64).reshape(Y.shape)
    # one verdict for both forms: a finite expected value within the
    # tolerance, NaN against NaN, or the same infinity (an infinite Y is never
    # matched by a distance, whatever its bound)
    tol = o.REL_TOL * B + o.ABS_TOL if bound is None else np.asarray(bound, np.float64)
    tol = np.broadcast_to(tol, Y.shape)
    ok = o.within_bound(y, Y, None, tol=tol)
    if not ok.all():
        bad = np.argwhere(~ok)
        lines = []
        for idx in bad[:8]:
            idx = tuple(idx)
            lines.append("  at %s: gpu=%r oracle=%r tol=%r" % (idx, y[idx], Y[idx], tol[idx]))
        raise AssertionError("%s: %d of %d outputs outside the bound\n%s"
                             % (what, len(bad), y.size, "\n".join(lines)))
    # the worst error as a fraction of its tolerance, over finite expected
    # values (the others matched exactly)
    fin = np.isfinite(Y) & (tol > 0)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = float(np.max(np.abs(y[fin] - Y[fin]) / tol[fin])) if fin.any() else 0.0
    print("%s: max |err|/bound = %.3g over %d outputs" % (what, r, y.size))
    return r


def needs_forced_height(rows, g, M=None):
    """Skip a forced tile height the case would not reach: forced heights
    serve the prefill GEMM (M > 16), 64 rows with groups of 128 or 64 k, 128
    rows with groups of 128 k."""
    if not rows:
        return
    if M is not None and M <= 16:
        pytest.skip("forced tile heights serve the prefill GEMM (M > 16)")
    if (rows == 128 and g != 128) or (rows == 64 and g not in (64, 128)):
        pytest.skip("the group size offers no %d-row form" % rows)

"""Helpers shared by the GPU tests: upload seeded operands, run the C ABI,
compare with the oracle under the per-element bound."""
import numpy as np

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


def workspace(q, M):
    """A GEMM workspace for (q, M) (zero-filled), shared by every call that
    fits in it."""
    from block_wise_int4_amd import mnb
    n = mnb.mnb_gemm_workspace_bytes(q.desc, M)
    buf = _WS.get("buf")
    if buf is None or buf.numel() < n:
        buf = torch().zeros(max(n, 256), dtype=torch().uint8, device="cuda")
        _WS["buf"] = buf
    return buf, n


def gemm(q, a, M, y, stream=None):
    from block_wise_int4_amd import mnb
    ws, n = workspace(q, M)
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
    if bound is None:
        ok = o.within_bound(y, Y, B)
        tol = o.REL_TOL * B + o.ABS_TOL
    else:
        tol = bound
        with np.errstate(invalid="ignore"):
            ok = ((np.abs(y - Y) <= tol) | (np.isnan(y) & np.isnan(Y)) |
                  (np.isinf(y) & np.isinf(Y) & (np.sign(y) == np.sign(Y))))
    if not ok.all():
        bad = np.argwhere(~ok)
        lines = []
        for idx in bad[:8]:
            idx = tuple(idx)
            lines.append("  at %s: gpu=%r oracle=%r tol=%r" % (idx, y[idx], Y[idx], tol[idx]))
        raise AssertionError("%s: %d of %d outputs outside the bound\n%s"
                             % (what, len(bad), y.size, "\n".join(lines)))
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.nanmax(np.where(tol > 0, np.abs(y - Y) / tol, 0.0)) if y.size else 0.0
    print("%s: max |err|/bound = %.3g over %d outputs" % (what, r, y.size))
    return r

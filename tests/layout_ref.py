"""Host model of the repacked layout, written from the "Repacked layout"
section of include/mnb.h (not from the library's sources).  Used to check the
device repack byte for byte and to invert repacked bytes on the host.

The codes it consumes come from the oracle (``oracle.unpack_codes``), so the
ONNX side is decoded by the oracle and only the gfx950 layout is modelled here.
"""
import numpy as np


def _align(x, a=256):
    return (x + a - 1) // a * a


def geometry(N, K, g, has_zp, f16_scales):
    T = -(-N // 16)
    C = -(-K // 128)
    Q = 128 // g
    ss = 2 if f16_scales else 4
    S0 = _align(T * C * 1024)
    Z0 = _align(S0 + T * C * 16 * Q * ss)
    end = (Z0 + T * C * 8 * Q) if has_zp else (S0 + T * C * 16 * Q * ss)
    F0 = _align(end)
    return dict(T=T, C=C, Q=Q, ss=ss, S0=S0, Z0=Z0 if has_zp else 0, F0=F0, total=_align(F0 + T))


def range_flags(scales, N):
    """Byte per 16-column tile: 1 when every scale of its columns that is
    neither zero nor NaN has magnitude in [2^-100, 2^100] and each column's
    largest such magnitude is at most 2^64 times its smallest (the range class
    stated in the header), else 0."""
    T = -(-N // 16)
    a = np.abs(np.asarray(scales, np.float64)).reshape(N, -1)
    live = (a != 0) & ~np.isnan(a)
    out = np.ones(T, dtype=np.uint8)
    for n in range(N):
        v = a[n][live[n]]
        if v.size == 0:
            continue
        if (v < 2.0 ** -100).any() or (v > 2.0 ** 100).any() or v.max() > v.min() * 2.0 ** 64:
            out[n // 16] = 0
    return out


# nibble slot p(i) of k-offset i
SLOT = np.array([0, 4, 1, 5, 2, 6, 3, 7])


def slot(i, q, Q):
    return i * Q + q if Q <= 4 else ((q % 2) * 16 + i) * 4 + q // 2


def repack_ref(codes, z, scales, g, has_zp):
    """codes u8[N,K] (0..15), z u8[N,K/g] zero points, scales [N,K/g] (fp16 or
    fp32 numpy) -> repacked bytes (np.uint8) per the documented layout."""
    N, K = codes.shape
    f16 = scales.dtype == np.float16
    G = geometry(N, K, g, has_zp, f16)
    T, C, Q = G["T"], G["C"], G["Q"]
    out = np.zeros(G["total"], dtype=np.uint8)
    # codes: pad to whole tiles / chunks with 0
    cp = np.zeros((T * 16, C * 128), dtype=np.uint32)
    cp[:N, :K] = codes
    # [t, i, c, j, h, e] with n = 16t+i, k = 128c + 32j + 8h + e
    v = cp.reshape(T, 16, C, 4, 4, 8)
    words = np.zeros((T, C, 4, 16, 4), dtype=np.uint32)  # [t, c, h, i, j] -> lane = 16h + i
    for e in range(8):
        words |= (v[:, :, :, :, :, e].transpose(0, 2, 4, 1, 3) << np.uint32(4 * SLOT[e]))
    out[:T * C * 1024] = words.astype("<u4").view(np.uint8).reshape(-1)
    # scales
    kb = K // g
    sdt = np.float16 if f16 else np.float32
    srec = np.zeros((T, C, 16 * Q), dtype=sdt)
    zrec = np.zeros((T, C, 16 * Q), dtype=np.uint8)
    for t in range(T):
        for i in range(16):
            n = 16 * t + i
            if n >= N:
                continue
            for c in range(C):
                for q in range(Q):
                    G_ = c * Q + q
                    if G_ < kb:
                        srec[t, c, slot(i, q, Q)] = scales[n, G_]
                        zrec[t, c, slot(i, q, Q)] = z[n, G_]
    sb = srec.reshape(-1).view(np.uint8)
    out[G["S0"]:G["S0"] + sb.size] = sb
    if has_zp:
        zr = zrec.reshape(-1)
        zb = (zr[0::2] | (zr[1::2] << 4)).astype(np.uint8)
        out[G["Z0"]:G["Z0"] + zb.size] = zb
    out[G["F0"]:G["F0"] + T] = range_flags(scales, N)
    return out


def unrepack_codes(buf, N, K, g, has_zp, f16_scales):
    """Inverse for the code section: repacked bytes -> codes u8[N,K]."""
    G = geometry(N, K, g, has_zp, f16_scales)
    T, C = G["T"], G["C"]
    words = np.frombuffer(buf[:T * C * 1024].tobytes(), dtype="<u4").reshape(T, C, 4, 16, 4)
    cp = np.zeros((T, 16, C, 4, 4, 8), dtype=np.uint8)
    for e in range(8):
        cp[:, :, :, :, :, e] = ((words >> np.uint32(4 * SLOT[e])) & 15).transpose(0, 3, 1, 4, 2)
    return cp.reshape(T * 16, C * 128)[:N, :K]

"""The calls on the caller's stream and inside a captured HIP graph.

Every entry point enqueues its kernels on the stream it is given and
allocates, frees and synchronises nothing, so a sequence of calls can be
captured into a graph and replayed.  These tests capture one call of every
path on a side stream, replay the graph several times with the program's own
eager work and synchronisations between the replays, and check every replay
bit for bit against the same calls run eagerly (the kernels are
deterministic).  A second test runs every path on a non-default stream.
"""
import numpy as np
import pytest

from block_wise_int4_amd import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mnb():
    from block_wise_int4_amd import mnb as m
    return m


def _setup(mnb):
    """Operands of every path, resident on the device, and a function that
    issues one call of each on a given stream into preallocated outputs."""
    t = G.torch()
    K, N = 512, 300
    w = synth.weight(N, K, 32, "f16", (0.005, 0.02), True, (400,))
    wg = synth.weight(N, K, 128, "f16", (0.002, 0.01), False, (401,))
    wu = synth.weight(N, K, 128, "f16", (0.002, 0.01), False, (402,))
    w32 = synth.weight(N, K, 64, "f32", (0.005, 0.02), True, (403,))
    q, qg, qu, q32 = G.upload(w), G.upload(wg), G.upload(wu), G.upload(w32)
    a1 = G.to_dev(synth.activation(1, K, "f16", 1.0, (404,)).reshape(-1))
    a8 = G.to_dev(synth.activation(8, K, "f16", 1.0, (405,)))
    a40 = G.to_dev(synth.activation(40, K, "f16", 1.0, (406,)))
    f1 = G.to_dev(synth.activation(1, K, "f32", 1.0, (407,)))
    f40 = G.to_dev(synth.activation(40, K, "f32", 1.0, (408,)))
    bias16 = G.to_dev(synth.activation(1, N, "f16", 1.0, (409,)).reshape(-1))
    bias32 = G.to_dev(synth.activation(1, N, "f32", 1.0, (410,)).reshape(-1))
    rng = np.random.default_rng(411)
    g_idx = np.empty(K, np.int32)
    g_idx[rng.permutation(K)] = np.arange(K) // 32
    perm = G.to_dev(mnb.mnb_act_order_permutation(q.desc, g_idx))
    rep_ao = t.empty(mnb.mnb_repacked_bytes(q.desc), dtype=t.uint8, device="cuda")
    mnb.mnb_repack_act_order(q.desc, G.to_dev(w.packed.reshape(-1)), G.to_dev(w.scales.reshape(-1)),
                             G.to_dev(w.zero_points.reshape(-1)), perm, rep_ao)
    # a g_idx of uneven groups for the general route
    gi_any = G.to_dev(rng.integers(0, K // 32, K).astype(np.int32))
    n_ao = mnb.mnb_gemm_act_order_workspace_bytes(q.desc, 40, mnb.MNB_F16)
    n_a4 = mnb.mnb_gemm_accuracy4_workspace_bytes(q32.desc, 40)
    n_g = max(mnb.mnb_gemm_workspace_bytes(q.desc, 8), 16)
    ws = {k: t.zeros(n, dtype=t.uint8, device="cuda") for k, n in (("ao", n_ao), ("a4", n_a4), ("g", n_g))}
    outs = {
        "gemv": t.empty(N, dtype=t.float16, device="cuda"),
        "gate_up": t.empty(N, dtype=t.float16, device="cuda"),
        "small_m": t.empty((8, N), dtype=t.float16, device="cuda"),
        "prefill_bias": t.empty((40, N), dtype=t.float16, device="cuda"),
        "act_order": t.empty((40, N), dtype=t.float16, device="cuda"),
        "acc4_decode": t.empty((1, N), dtype=t.float32, device="cuda"),
        "acc4_prefill": t.empty((40, N), dtype=t.float32, device="cuda"),
        "gidx_stream": t.empty((8, N), dtype=t.float16, device="cuda"),
        "gidx_mfma": t.empty((40, N), dtype=t.float32, device="cuda"),
    }
    t.cuda.synchronize()

    def issue(stream):
        mnb.mnb_gemv(q.desc, q.repacked, a1, outs["gemv"], stream=stream)
        mnb.mnb_gemv_gate_up_swiglu(qg.desc, qg.repacked, qu.repacked, a1, outs["gate_up"], stream=stream)
        mnb.mnb_gemm(q.desc, q.repacked, a8, 8, outs["small_m"], ws["g"], n_g, stream=stream)
        mnb.mnb_gemm_bias(q.desc, q.repacked, a40, 40, bias16, 0, mnb.MNB_BIAS_FUSED, outs["prefill_bias"],
                          None, 0, stream=stream)
        mnb.mnb_gemm_act_order(q.desc, rep_ao, a40, 40, perm, outs["act_order"], ws["ao"], n_ao,
                               stream=stream)
        mnb.mnb_gemm_accuracy4(q32.desc, q32.repacked, f1, 1, bias32, outs["acc4_decode"], stream=stream)
        mnb.mnb_gemm_accuracy4(q32.desc, q32.repacked, f40, 40, bias32, outs["acc4_prefill"], ws["a4"], n_a4,
                               stream=stream)
        mnb.mnb_gemm_group_indices(q.desc, q.repacked, a8, 8, gi_any, outs["gidx_stream"], stream=stream)
        mnb.mnb_gemm_group_indices(q.desc, q.repacked, f40, 40, gi_any, outs["gidx_mfma"], bias32, 0,
                                   stream=stream)

    return issue, outs


def _snapshot(outs):
    return {k: v.detach().cpu().numpy().copy() for k, v in outs.items()}


def _same_bits(a, b, what):
    for k in a:
        assert a[k].tobytes() == b[k].tobytes(), "%s: %s differs" % (what, k)


def test_calls_replay_from_a_captured_graph(mnb):
    t = G.torch()
    issue, outs = _setup(mnb)
    issue(t.cuda.current_stream())
    t.cuda.synchronize()
    eager = _snapshot(outs)
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    graph = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(graph, stream=s):
            issue(s)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    for r in range(3):
        for v in outs.values():
            v.fill_(float("nan"))       # eager work between the replays
        t.cuda.synchronize()
        graph.replay()
        t.cuda.synchronize()
        _same_bits(eager, _snapshot(outs), "replay %d" % r)


def test_calls_run_on_the_callers_stream(mnb):
    t = G.torch()
    issue, outs = _setup(mnb)
    issue(t.cuda.current_stream())
    t.cuda.synchronize()
    eager = _snapshot(outs)
    for v in outs.values():
        v.fill_(float("nan"))
    t.cuda.synchronize()
    s = t.cuda.Stream()
    issue(s)
    s.synchronize()
    _same_bits(eager, _snapshot(outs), "side stream")

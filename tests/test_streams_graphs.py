"""The C ABI is asynchronous and stateless: calls on several streams at once,
and calls recorded into a HIP graph and replayed, must give the same bits as
plain calls on one stream (the kernels' arithmetic order does not depend on
what else runs).  Parity with the oracle is checked once per product."""
import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import seeded_inputs as si
from tests.gpu_util import assert_within_tolerance, upload

pytestmark = pytest.mark.gpu


def _bits(C):
    import torch
    return C.cpu().view(torch.int16).numpy().view(np.uint16)


def _gemm(A, B, C, M, N, K, trans_b, stream, schedule=mcs.GEMM_SCHED_AUTO):
    st = mcs.gemm_ex(mcs.GEMM_DTYPE_F16, M, N, K, A.data_ptr(), K, B.data_ptr(), K if trans_b else N, trans_b,
                     C.data_ptr(), N, mcs.GEMM_OUT_SAME, schedule, stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)


def test_two_streams_at_once_match_one_stream():
    torch = pytest.importorskip("torch")
    shapes = [(1024, 768, 2048, 1), (520, 1032, 1000, 0)]
    ops, ref = [], []
    for i, (M, N, K, tb) in enumerate(shapes):
        print(f"[gpu] streams {M}x{N}x{K} tb={tb}", flush=True)
        a = si.matrix_bits("f16", "uniform", M, K, seed=8100 + i, stream=0)
        b = si.matrix_bits("f16", "uniform", N, K, seed=8100 + i, stream=1) if tb else \
            si.matrix_bits("f16", "uniform", K, N, seed=8100 + i, stream=1)
        A, _ = upload(a, "f16")
        B, _ = upload(b, "f16")
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        _gemm(A, B, C, M, N, K, tb, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        cref, sabs = oracle.gemm(a, b, "f16", tb, K=K, N=N)
        assert_within_tolerance(oracle.decode(_bits(C), "f16"), cref, sabs, f"stream shape {i}", out="f16")
        ops.append((A, B, M, N, K, tb))
        ref.append(_bits(C))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.full((M, N), 9.0, dtype=torch.float16, device="cuda") for _ in range(4)]
            for (_, _, M, N, _, _) in ops]
    torch.cuda.synchronize()
    for r in range(4):                       # interleave the enqueues of both streams
        for s, (A, B, M, N, K, tb), o in zip(streams, ops, outs):
            _gemm(A, B, o[r], M, N, K, tb, s.cuda_stream)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        for r in range(4):
            assert np.array_equal(_bits(o[r]), ref[i]), f"shape {i} launch {r} differs on its own stream"


@pytest.mark.parametrize("schedule", [mcs.GEMM_SCHED_AUTO, mcs.GEMM_SCHED_PIPELINED, mcs.GEMM_SCHED_TILE128])
def test_graph_replays_match_eager(schedule):
    """gemm_ex recorded into a graph (one kernel, no memset, no allocation) and
    replayed with new operand values copied in between replays: every replay
    equals an eager call on the same values, bit for bit."""
    torch = pytest.importorskip("torch")
    M, N, K = 768, 1024, 1536
    print(f"[gpu] graph {M}x{N}x{K} schedule={schedule}", flush=True)
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    B = torch.empty((N, K), dtype=torch.float16, device="cuda")
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    Ce = torch.empty_like(C)

    def fill(seed):
        a = si.matrix_bits("f16", "uniform", M, K, seed=seed, stream=0)
        b = si.matrix_bits("f16", "uniform", N, K, seed=seed, stream=1)
        A.copy_(torch.from_numpy(a.view(np.int16)).view(torch.float16))
        B.copy_(torch.from_numpy(b.view(np.int16)).view(torch.float16))
        return a, b

    fill(8200)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up on the capture stream, outside the graph
        _gemm(A, B, C, M, N, K, 1, side.cuda_stream, schedule)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _gemm(A, B, C, M, N, K, 1, torch.cuda.current_stream().cuda_stream, schedule)
    for rep in range(3):
        a, b = fill(8201 + rep)
        C.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _gemm(A, B, Ce, M, N, K, 1, torch.cuda.current_stream().cuda_stream, schedule)   # eager, same values
        torch.cuda.synchronize()
        got, want = _bits(C), _bits(Ce)
        assert np.array_equal(got, want), f"replay {rep}: {(got != want).sum()} elements differ from eager"
        if rep == 0:
            cref, sabs = oracle.gemm(a, b, "f16", 1, K=K, N=N)
            assert_within_tolerance(oracle.decode(got, "f16"), cref, sabs, "graph replay", out="f16")


def _attention(Q, K, V, O, L, B, H, S, causal, stream):
    import math
    st = mcs.attention_fwd(mcs.GEMM_DTYPE_F16, B, H, S, S, 128, Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                           O.data_ptr(), L.data_ptr(), 1 / math.sqrt(128), causal, stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)


@pytest.mark.parametrize("causal", [0, 1])
def test_attention_graph_replays_match_eager(causal):
    """attention_fwd (the persistent kernel: one workgroup per CU, its tiles in
    a fixed order) recorded into a graph and replayed with new Q, K, V in
    between: O and lse of every replay equal an eager call, bit for bit; two
    launches on two streams at once give the same bits as well."""
    torch = pytest.importorskip("torch")
    import oracle.attention as at
    B, H, S = 2, 5, 700                     # ragged last tile and last key block; 30 tiles
    print(f"[gpu] attention graph B={B} H={H} S={S} causal={causal}", flush=True)
    Q, K, V = (torch.empty((B * H * S, 128), dtype=torch.float16, device="cuda") for _ in range(3))
    O, Oe = torch.empty_like(Q), torch.empty_like(Q)
    L, Le = (torch.empty(B * H * S, dtype=torch.float32, device="cuda") for _ in range(2))

    def fill(seed):
        out = []
        for i, T in enumerate((Q, K, V)):
            x = si.matrix_bits("f16", "normal", B * H * S, 128, seed=seed, stream=i)
            T.copy_(torch.from_numpy(x.view(np.int16)).view(torch.float16))
            out.append(x.reshape(B, H, S, 128))
        return out

    fill(8300)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _attention(Q, K, V, O, L, B, H, S, causal, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _attention(Q, K, V, O, L, B, H, S, causal, torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        q, k, v = fill(8301 + rep)
        O.fill_(5.0)
        L.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _attention(Q, K, V, Oe, Le, B, H, S, causal, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(O.view(torch.int16), Oe.view(torch.int16)), f"replay {rep}: O differs from eager"
        assert torch.equal(L.view(torch.int32), Le.view(torch.int32)), f"replay {rep}: lse differs from eager"
        if rep == 0:
            oref, lref, a, sabs = at.attention(q, k, v, "f16", 1 / np.sqrt(128), bool(causal))
            got = oracle.decode(_bits(O).reshape(B, H, S, 128), "f16")
            assert at.within_tolerance(got, oref, a, sabs, 128, S, "f16").all(), "graph replay vs the oracle"
    # two launches at once on two streams, same inputs: the eager bits
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [(torch.full_like(Q, 3.0), torch.full_like(L, 7.0)) for _ in streams]
    torch.cuda.synchronize()
    for s, (o, l) in zip(streams, outs):
        _attention(Q, K, V, o, l, B, H, S, causal, s.cuda_stream)
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o.view(torch.int16), Oe.view(torch.int16)), "O on a second stream differs"
        assert torch.equal(l.view(torch.int32), Le.view(torch.int32)), "lse on a second stream differs"

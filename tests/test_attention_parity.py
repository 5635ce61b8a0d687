"""GPU parity of the attention forward pass: attention_fwd (through the C ABI)
against the float64 oracle, every element of O and every lse at small and
ragged sizes, sampled rows at the full 4 x 32 x 4096 x 128 size.

Bar (oracle.attention.within_tolerance): |O - Oref| <= (u + e) A + u |Oref|
with A = sum_j P_ij |V_jd|, u the operand type's rounding unit (the kernel
rounds P to it) and e the FP32 score / sum error bound; lse within its FP32
bound; rows with no visible key give O = 0 and lse = -inf exactly."""
import math

import numpy as np
import pytest

import matrix_core_scheduling_amd as mcs
import oracle
import oracle.attention as at
import seeded_inputs as si
from tests.gpu_util import TORCH_DT, _torch, upload

pytestmark = pytest.mark.gpu

DT = {"f16": mcs.GEMM_DTYPE_F16, "bf16": mcs.GEMM_DTYPE_BF16}


def qkv(elem, B, H, Sq, Sk, D, seed, dist="normal"):
    q = si.matrix_bits(elem, dist, B * H * Sq, D, seed=seed, stream=0).reshape(B, H, Sq, D)
    k = si.matrix_bits(elem, dist, B * H * max(Sk, 1), D, seed=seed, stream=1).reshape(B, H, max(Sk, 1), D)
    v = si.matrix_bits(elem, dist, B * H * max(Sk, 1), D, seed=seed, stream=2).reshape(B, H, max(Sk, 1), D)
    return q, k[:, :, :Sk].copy(), v[:, :, :Sk].copy()


SCHED = {"auto": mcs.GEMM_SCHED_AUTO, "pipelined": mcs.GEMM_SCHED_PIPELINED, "in_phase": mcs.GEMM_SCHED_IN_PHASE,
         "interleaved": mcs.GEMM_SCHED_INTERLEAVED}


def run_attention(elem, q, k, v, scale, causal, o_fill=-5.0, sched="auto"):
    """O (float64), lse (float64) and raw O bits from attention_fwd (sched "auto")
    or attention_fwd_ex with the named schedule."""
    torch = _torch()
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    print(f"[gpu] attention elem={elem} B={B} H={H} Sq={Sq} Sk={Sk} D={D} causal={causal} sched={sched}",
          flush=True)
    Q, _ = upload(q.reshape(-1, D), elem)
    K, _ = upload(k.reshape(-1, D) if Sk else np.zeros((1, D), np.uint16), elem)
    V, _ = upload(v.reshape(-1, D) if Sk else np.zeros((1, D), np.uint16), elem)
    O = torch.full((B * H * Sq * D,), o_fill, dtype=TORCH_DT[elem], device="cuda")
    L = torch.full((B * H * Sq,), 7.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    if sched == "auto":
        st = mcs.attention_fwd(DT[elem], B, H, Sq, Sk, D, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                               L.data_ptr(), scale, int(causal), stream)
    else:
        st = mcs.attention_fwd_ex(DT[elem], B, H, Sq, Sk, D, Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                                  O.data_ptr(), L.data_ptr(), scale, int(causal), SCHED[sched], stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    bits = O.cpu().view(torch.int16).numpy().view(np.uint16).reshape(B, H, Sq, D)
    return oracle.decode(bits, elem), L.cpu().double().numpy().reshape(B, H, Sq), bits


def check(elem, q, k, v, scale, causal, rows=None, what="", sched="auto"):
    o, lse, _ = run_attention(elem, q, k, v, scale, causal, sched=sched)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    oref, lref, a, sabs = at.attention(q, k, v, elem, scale, causal, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    ok = at.within_tolerance(o, oref, a, sabs, D, Sk, elem)
    bad = np.argwhere(~ok)
    assert ok.all(), (f"{what}: {bad.shape[0]} of {ok.size} outside; first {bad[:3].tolist()} "
                      f"got {o[tuple(bad[0])]} want {oref[tuple(bad[0])]}")
    okl = at.lse_within_tolerance(lse, lref, sabs, D, Sk)
    bad = np.argwhere(~okl)
    assert okl.all(), f"{what}: lse {bad[:3].tolist()} got {lse[tuple(bad[0])]} want {lref[tuple(bad[0])]}"
    return o, lse


SHAPES = [  # (B, H, Sq, Sk)
    (1, 1, 1, 1), (1, 2, 17, 33), (1, 1, 64, 64), (2, 3, 300, 200), (1, 2, 256, 256), (1, 1, 512, 64),
    (1, 2, 100, 700), (1, 1, 257, 513), (2, 1, 96, 1000),
]


@pytest.mark.parametrize("sched", ["pipelined", "interleaved"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes_every_element(shape, elem, causal, sched):
    B, H, Sq, Sk = shape
    q, k, v = qkv(elem, B, H, Sq, Sk, 128, seed=Sq * 7 + Sk)
    check(elem, q, k, v, 1 / math.sqrt(128), causal, what=f"{shape} {elem} causal={causal} {sched}", sched=sched)


# 2 .. 8 blocks of 64 keys, full and ragged last blocks: the K and V rings of
# four slots wrap, and the trips near the end copy blocks past the last one
BLOCK_COUNTS = [(nb, 64 * nb - (23 if nb % 2 else 0)) for nb in range(2, 9)]


@pytest.mark.parametrize("sched", ["pipelined", "interleaved"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nb,sk", BLOCK_COUNTS, ids=lambda x: str(x))
def test_every_block_count(nb, sk, causal, sched):
    assert (sk + 63) // 64 == nb
    q, k, v = qkv("f16", 1, 2, sk, sk, 128, seed=900 + nb)
    check("f16", q, k, v, 1 / math.sqrt(128), causal, what=f"blocks={nb} Sk={sk}", sched=sched)


# More tiles than CUs, so that each persistent workgroup of the 8-wave kernel
# runs several tiles in a row: (B, H, Sq, Sk, causal) and the tile-to-tile
# path each exercises (blocks per tile in brackets)
TRANSITIONS = [
    (2, 300, 256, 200, False),   # [4] -> [4]: the next tile's first blocks and Q fetched ahead
    (2, 300, 256, 130, False),   # [3] -> [3]: not fetched ahead (the next tile's block 3 would be
                                 # the first block of the tile after it); zero windows settle first
    (2, 300, 256, 100, False),   # [2] -> [2]: likewise
    (1, 120, 600, 150, True),    # [0], [1], [3] mixed: tiles without blocks, one block, three
    (1, 120, 600, 460, True),    # [2], [6], [8] mixed: fetched ahead into the longer tiles only
    (1, 123, 768, 300, False),   # [5] -> [5], 369 tiles: the XCDs' ranges differ by one tile
    (1, 123, 768, 700, True),    # causal [3], [7], [11] with a ragged last block, 369 tiles
]


@pytest.mark.parametrize("B,H,Sq,Sk,causal", TRANSITIONS, ids=lambda x: str(x))
def test_persistent_tile_transitions(B, H, Sq, Sk, causal):
    assert B * H * ((Sq + 255) // 256) > 256
    q, k, v = qkv("f16", B, H, Sq, Sk, 128, seed=7000 + Sk + Sq)
    check("f16", q, k, v, 1 / math.sqrt(128), causal, what=f"{B}x{H}x{Sq}x{Sk} causal={causal}")


@pytest.mark.parametrize("sched", ["pipelined", "interleaved"])
def test_uniform_values_and_other_scales(sched):
    # scale 4: scores span hundreds in log2 units, so a running max that is not
    # the true row max overflows the exponentials
    for dist, scale in (("uniform", 0.3), ("normal", 0.02), ("normal", 0.25), ("normal", 4.0)):
        q, k, v = qkv("f16", 1, 2, 192, 320, 128, seed=3, dist=dist)
        check("f16", q, k, v, scale, False, what=f"{dist} scale={scale}", sched=sched)


def test_rows_without_keys_and_no_keys():
    """Causal with more queries than keys: the first Sq - Sk rows see no key
    (O = 0, lse = -inf); Sk = 0: every row."""
    q, k, v = qkv("f16", 1, 2, 300, 40, 128, seed=8)
    o, lse = check("f16", q, k, v, 0.1, True, what="Sq > Sk causal")
    assert np.array_equal(o[:, :, :260], np.zeros_like(o[:, :, :260]))
    assert np.isneginf(lse[:, :, :260]).all() and np.isfinite(lse[:, :, 260:]).all()
    q, k, v = qkv("bf16", 2, 1, 70, 0, 128, seed=9)
    o, lse, _ = run_attention("bf16", q, k, v, 0.1, False)
    assert np.array_equal(o, np.zeros_like(o)) and np.isneginf(lse).all()


def test_identical_keys_give_the_mean_of_v():
    """A closed form on the GPU: equal keys weigh every visible V row alike."""
    q, k, v = qkv("f16", 1, 1, 128, 192, 128, seed=10)
    k[:] = k[:, :, :1]
    o, _ = check("f16", q, k, v, 0.125, False, what="identical keys")
    mean = oracle.decode(v, "f16").mean(axis=2)
    assert np.allclose(o[0, 0], np.broadcast_to(mean[0, 0], o[0, 0].shape), rtol=2 ** -9, atol=2e-3)


def test_deterministic():
    q, k, v = qkv("bf16", 1, 4, 512, 512, 128, seed=12)
    b1 = run_attention("bf16", q, k, v, 0.09, True)[2]
    b2 = run_attention("bf16", q, k, v, 0.09, True)[2]
    assert np.array_equal(b1, b2)


@pytest.mark.parametrize("causal", [False, True])
def test_in_phase_schedule_is_bitwise_identical(causal):
    """Same stages and arithmetic with the groups in step: the offset changes
    only timing."""
    torch = _torch()
    q, k, v = qkv("f16", 1, 3, 520, 777, 128, seed=15)
    _, lse0, b0 = run_attention("f16", q, k, v, 0.08, causal)
    Q, K, V = (upload(x.reshape(-1, 128), "f16")[0] for x in (q, k, v))
    O = torch.empty_like(Q)
    L = torch.empty(3 * 520, dtype=torch.float32, device="cuda")
    st = mcs.attention_fwd_ex(mcs.GEMM_DTYPE_F16, 1, 3, 520, 777, 128, Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                              O.data_ptr(), L.data_ptr(), 0.08, int(causal), mcs.GEMM_SCHED_IN_PHASE,
                              torch.cuda.current_stream().cuda_stream)
    assert st == mcs.GEMM_OK
    torch.cuda.synchronize()
    assert np.array_equal(O.cpu().view(torch.int16).numpy().view(np.uint16).reshape(b0.shape), b0)
    assert np.array_equal(L.cpu().double().numpy().reshape(lse0.shape), lse0)


@pytest.mark.parametrize("elem", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_four_wave_form_is_bitwise_identical(elem, causal):
    """The 4-wave form (one wave per SIMD, 64 query rows each) runs the same
    MFMA sequence per output element and the same softmax arithmetic as the
    8-wave form: the same bits of O and lse, on ragged sizes with masked
    blocks, rows past the end and several key-block counts."""
    for (B, H, Sq, Sk) in [(1, 3, 520, 777), (2, 2, 256, 64), (1, 1, 300, 129), (1, 2, 1000, 1100)]:
        q, k, v = qkv(elem, B, H, Sq, Sk, 128, seed=Sq + Sk)
        _, l8, b8 = run_attention(elem, q, k, v, 0.08, causal, sched="pipelined")
        _, l4, b4 = run_attention(elem, q, k, v, 0.08, causal, sched="interleaved")
        assert np.array_equal(b4, b8), (B, H, Sq, Sk, int((b4 != b8).sum()))
        assert np.array_equal(l4, l8), (B, H, Sq, Sk)


def test_torch_binding_matches_abi():
    torch = _torch()
    q, k, v = qkv("f16", 2, 2, 200, 330, 128, seed=14)
    o_abi, lse_abi, _ = run_attention("f16", q, k, v, 1 / math.sqrt(128), True)
    t = [upload(x.reshape(-1, 128), "f16")[0].view(x.shape) for x in (q, k, v)]
    o, lse = mcs.attention(*t, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(oracle.decode(o.cpu().view(torch.int16).numpy().view(np.uint16), "f16"), o_abi)
    assert np.array_equal(lse.cpu().double().numpy(), lse_abi)


@pytest.mark.parametrize("name", [n for n in si.ATTN_WORKLOADS])
def test_attention_workload(name):
    """The workloads in the configuration bench.py runs: every element for the
    small one, 24 sampled query rows (block edges included) of every head for
    the full-size ones."""
    w = si.ATTN_WORKLOADS[name]
    q, k, v = w.operands(0)
    if w.B * w.H * w.Sq * w.Sk <= 2 ** 22:
        check(w.dtype, q, k, v, w.scale, w.causal, what=name)
        return
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([rng.integers(0, w.Sq, 16), [0, 63, 64, 255, 256, w.Sq - 257, w.Sq - 1]]))
    o, lse = check(w.dtype, q, k, v, w.scale, w.causal, rows=rows, what=name)
    assert np.isfinite(o).all()


@pytest.mark.parametrize("name", [n for n in si.ATTN_WORKLOADS if n != "attn_f16_b1h4s512d128"])
def test_four_wave_form_full_size(name):
    """The bench.py workloads at full size: the 4-wave form gives the 8-wave
    form's bits for every element of O and lse (the 8-wave form is checked
    against the oracle on sampled rows by test_attention_workload)."""
    w = si.ATTN_WORKLOADS[name]
    q, k, v = w.operands(0)
    _, l8, b8 = run_attention(w.dtype, q, k, v, w.scale, w.causal, sched="pipelined")
    _, l4, b4 = run_attention(w.dtype, q, k, v, w.scale, w.causal, sched="interleaved")
    assert np.array_equal(b4, b8), (name, int((b4 != b8).sum()))
    assert np.array_equal(l4, l8), name


@pytest.mark.parametrize("B,H,Sq,Sk,causal", [(2, 300, 256, 200, False), (1, 120, 600, 460, True)],
                         ids=lambda x: str(x))
def test_without_lse_same_output(B, H, Sq, Sk, causal):
    """lse = NULL (no lse stores: the waits between tiles count fewer stores)
    gives O bit for bit as with lse, over more tiles than CUs."""
    torch = _torch()
    q, k, v = qkv("f16", B, H, Sq, Sk, 128, seed=7300 + Sk)
    _, _, bits = run_attention("f16", q, k, v, 1 / math.sqrt(128), causal)
    Q, _ = upload(q.reshape(-1, 128), "f16")
    K, _ = upload(k.reshape(-1, 128), "f16")
    V, _ = upload(v.reshape(-1, 128), "f16")
    O = torch.full((B * H * Sq * 128,), -5.0, dtype=torch.float16, device="cuda")
    print(f"[gpu] attention without lse B={B} H={H} Sq={Sq} Sk={Sk} causal={causal}", flush=True)
    st = mcs.attention_fwd(DT["f16"], B, H, Sq, Sk, 128, Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(),
                           None, 1 / math.sqrt(128), int(causal), torch.cuda.current_stream().cuda_stream)
    assert st == mcs.GEMM_OK, mcs.gemm_status_string(st)
    torch.cuda.synchronize()
    got = O.cpu().view(torch.int16).numpy().view(np.uint16).reshape(B, H, Sq, 128)
    assert np.array_equal(got, bits), f"{(got != bits).sum()} O elements differ without lse"

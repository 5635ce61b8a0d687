"""Pins of the attention oracle: each check takes the oracle module (the real
one, or a copy with a planted mistake) and raises AssertionError if it does
not hold.  None of them re-types the oracle's own formula: they compare with
a pure-Python loop brute force, with torch's scaled-dot-product attention in
float64, and with closed forms and invariances of softmax attention."""
import math

import numpy as np

import seeded_inputs as si


def _f64(bits, elem):
    """Widen bit patterns with numpy (FP16) or torch (BF16), not the oracle's decoder."""
    if elem == "f16":
        return np.asarray(bits).view(np.float16).astype(np.float64)
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def qkv(elem, B, H, Sq, Sk, D, seed, dist="normal"):
    q = si.matrix_bits(elem, dist, B * H * Sq, D, seed=seed, stream=0).reshape(B, H, Sq, D)
    k = si.matrix_bits(elem, dist, B * H * Sk, D, seed=seed, stream=1).reshape(B, H, Sk, D)
    v = si.matrix_bits(elem, dist, B * H * Sk, D, seed=seed, stream=2).reshape(B, H, Sk, D)
    return q, k, v


def brute_force(q, k, v, elem, scale, causal):
    """Attention with Python loops and math.fsum, one row at a time."""
    qf, kf, vf = _f64(q, elem), _f64(k, elem), _f64(v, elem)
    B, H, Sq, D = qf.shape
    Sk = kf.shape[2]
    O = np.zeros((B, H, Sq, D))
    L = np.full((B, H, Sq), -math.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                keys = [j for j in range(Sk) if not causal or j - (Sk - Sq) <= i]
                if not keys:
                    continue
                s = {j: scale * math.fsum(qf[b, h, i, d] * kf[b, h, j, d] for d in range(D)) for j in keys}
                top = max(s.values())
                w = {j: math.exp(s[j] - top) for j in keys}
                tot = math.fsum(w.values())
                L[b, h, i] = top + math.log(tot)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(w[j] * vf[b, h, j, d] for j in keys) / tot
    return O, L


def check_brute_force(at):
    for elem in ("f16", "bf16"):
        for (B, H, Sq, Sk, D, causal) in [(1, 2, 5, 7, 8, False), (2, 1, 6, 6, 4, True), (1, 1, 7, 4, 8, True),
                                          (1, 2, 3, 9, 16, True), (1, 1, 1, 1, 4, False)]:
            q, k, v = qkv(elem, B, H, Sq, Sk, D, seed=Sq * 31 + Sk)
            scale = 1.0 / math.sqrt(D)
            O, L, A, S = at.attention(q, k, v, elem, scale, causal)
            Ob, Lb = brute_force(q, k, v, elem, scale, causal)
            assert np.allclose(O, Ob, rtol=1e-12, atol=1e-13), (elem, B, H, Sq, Sk, D, causal)
            fin = np.isfinite(Lb)
            assert np.array_equal(np.isfinite(L), fin)
            assert np.allclose(L[fin], Lb[fin], rtol=1e-12, atol=1e-13)


def check_torch_sdpa(at):
    import torch

    for elem in ("f16", "bf16"):
        for (B, H, Sq, Sk, D, causal) in [(2, 3, 64, 80, 32, False), (1, 2, 96, 96, 64, True),
                                          (1, 1, 40, 72, 128, True)]:
            q, k, v = qkv(elem, B, H, Sq, Sk, D, seed=7 + D)
            scale = 0.7 / math.sqrt(D)
            O, L, _, _ = at.attention(q, k, v, elem, scale, causal)
            t = [torch.from_numpy(_f64(x, elem)) for x in (q, k, v)]
            mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq) if causal else None
            ref = torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=mask, scale=scale).numpy()
            assert np.allclose(O, ref, rtol=1e-10, atol=1e-12), (elem, Sq, Sk, D, causal)
            # lse from torch's own log-sum-exp of the masked scores
            s = torch.einsum("bhid,bhjd->bhij", t[0], t[1]) * scale
            if mask is not None:
                s = s.masked_fill(~mask, float("-inf"))
            assert np.allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def check_one_key(at):
    """Sk = 1: the softmax is 1, O = V exactly, lse = the score."""
    q, k, v = qkv("f16", 2, 2, 5, 1, 16, seed=3)
    O, L, A, _ = at.attention(q, k, v, "f16", 0.25, False)
    vf, qf, kf = _f64(v, "f16"), _f64(q, "f16"), _f64(k, "f16")
    assert np.array_equal(O, np.broadcast_to(vf, O.shape))
    assert np.array_equal(A, np.abs(O))
    assert np.allclose(L, 0.25 * np.einsum("bhid,bhd->bhi", qf, kf[:, :, 0]), rtol=1e-14, atol=1e-15)


def check_identical_keys(at):
    """Every key the same: uniform weights over the allowed keys, so O is the
    mean of the allowed V rows and lse = score + log(count)."""
    B, H, Sq, Sk, D = 1, 2, 6, 9, 8
    q, k, v = qkv("f16", B, H, Sq, Sk, D, seed=11)
    k[:] = k[:, :, :1, :]
    for causal in (False, True):
        O, L, _, _ = at.attention(q, k, v, "f16", 0.5, causal)
        vf, qf, kf = _f64(v, "f16"), _f64(q, "f16"), _f64(k, "f16")
        for i in range(Sq):
            n = Sk if not causal else i + 1 + (Sk - Sq)
            assert np.allclose(O[:, :, i], vf[:, :, :n].mean(axis=2), rtol=1e-12, atol=1e-13), (causal, i)
            s = 0.5 * np.einsum("bhd,bhd->bh", qf[:, :, i], kf[:, :, 0])
            assert np.allclose(L[:, :, i], s + math.log(n), rtol=1e-13, atol=1e-13)


def check_dominant_key(at):
    """One key aligned with the query and far larger: O is that key's V row
    (the others weigh less than e^-40 each)."""
    D, Sk = 16, 12
    q, k, v = qkv("f16", 1, 1, 1, Sk, D, seed=5)
    qv = np.zeros(D, dtype=np.float16)
    qv[:] = 1.0
    q[0, 0, 0] = qv.view(np.uint16)
    k[0, 0] = (np.zeros((Sk, D), dtype=np.float16)).view(np.uint16)
    kd = np.zeros(D, dtype=np.float16)
    kd[:] = 4.0
    k[0, 0, 7] = kd.view(np.uint16)                       # score 64 * scale against 0 for the rest
    O, L, _, _ = at.attention(q, k, v, "f16", 1.0, False)
    assert np.allclose(O[0, 0, 0], _f64(v, "f16")[0, 0, 7], rtol=1e-15, atol=Sk * math.exp(-60))
    assert abs(L[0, 0, 0] - 64.0) < 1e-20 + Sk * math.exp(-60)


def check_key_permutation(at):
    """Non-causal attention does not depend on the order of the keys (K and V
    rows permuted together), but does depend on K and V staying paired."""
    q, k, v = qkv("bf16", 1, 2, 8, 16, 32, seed=21)
    O, L, _, _ = at.attention(q, k, v, "bf16", 0.2, False)
    perm = np.random.default_rng(0).permutation(16)
    O2, L2, _, _ = at.attention(q, k[:, :, perm], v[:, :, perm], "bf16", 0.2, False)
    assert np.allclose(O, O2, rtol=1e-12, atol=1e-13) and np.allclose(L, L2, rtol=1e-13, atol=1e-13)
    O3, _, _, _ = at.attention(q, k, v[:, :, perm], "bf16", 0.2, False)
    assert not np.allclose(O, O3, rtol=1e-6, atol=1e-6)


def check_causal_masked_keys_ignored(at):
    """A causal row does not change when keys it may not see change."""
    Sq, Sk = 8, 11
    q, k, v = qkv("f16", 1, 1, Sq, Sk, 8, seed=9)
    O, L, _, _ = at.attention(q, k, v, "f16", 0.3, True)
    k2, v2 = k.copy(), v.copy()
    i = 4
    last = i + (Sk - Sq)                    # last key row i may see
    k2[0, 0, last + 1:] ^= 0x1234
    v2[0, 0, last + 1:] ^= 0x0F0F
    O2, L2, _, _ = at.attention(q, k2, v2, "f16", 0.3, True)
    assert np.array_equal(O[0, 0, :i + 1], O2[0, 0, :i + 1]) and np.array_equal(L[0, 0, :i + 1], L2[0, 0, :i + 1])
    assert not np.allclose(O[0, 0, -1], O2[0, 0, -1])      # the last row sees them all
    # a query row with no visible key (Sq > Sk): O = 0, lse = -inf
    q, k, v = qkv("f16", 1, 1, 6, 3, 8, seed=2)
    O, L, _, _ = at.attention(q, k, v, "f16", 0.3, True)
    assert np.array_equal(O[0, 0, :3], np.zeros((3, 8))) and np.isneginf(L[0, 0, :3]).all()
    assert np.isfinite(L[0, 0, 3:]).all()


def check_probabilities(at):
    """P is a probability distribution over each row's allowed keys."""
    q, k, v = qkv("f16", 1, 2, 7, 10, 16, seed=4)
    for causal in (False, True):
        P = at.probabilities(q, k, "f16", 0.25, causal)
        mask = np.ones((7, 10), dtype=bool) if not causal else (
            np.arange(10)[None, :] <= np.arange(7)[:, None] + 3)
        assert (P >= 0).all() and np.array_equal(P[..., ~mask], np.zeros_like(P[..., ~mask]))
        assert np.allclose(P.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
        # and it is the matrix the output is made of
        O, _, _, _ = at.attention(q, k, v, "f16", 0.25, causal)
        assert np.allclose(O, P @ _f64(v, "f16"), rtol=1e-12, atol=1e-13)


def check_tolerance(at):
    """The acceptance bound takes the correctly rounded output and refuses an
    error of several units of A."""
    import oracle

    q, k, v = qkv("f16", 1, 2, 32, 48, 64, seed=13)
    O, L, A, S = at.attention(q, k, v, "f16", 0.125, False)
    r = oracle.decode(oracle.round_to(O, "f16"), "f16")
    assert at.within_tolerance(r, O, A, S, 64, 48, "f16").all()
    assert not at.within_tolerance(O + 4 * at.UNIT["f16"] * A + 1e-3, O, A, S, 64, 48, "f16").any()
    rb = oracle.decode(oracle.round_to(O, "bf16"), "bf16")
    assert at.within_tolerance(rb, O, A, S, 64, 48, "bf16").all()
    assert at.lse_within_tolerance(L.astype(np.float32), L, S, 64, 48).all()
    assert not at.lse_within_tolerance(L + 1e-3, L, S, 64, 48).any()


ALL = [check_brute_force, check_torch_sdpa, check_one_key, check_identical_keys, check_dominant_key,
       check_key_permutation, check_causal_masked_keys_ignored, check_probabilities, check_tolerance]

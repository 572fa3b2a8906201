"""Pins of the oracle's indexer scores (closed forms, special cases, invariants)."""
import numpy as np

import oracle
import synth


def _bf16(x):
    return synth.encode_bf16(np.asarray(x, np.float32))


def test_one_hot_weight_reduces_to_relu_dot():
    # small integers: every product and sum is exact in fp32 and fp64
    rng = np.random.default_rng(2)
    q = rng.integers(-3, 4, (1, 32, 128)).astype(np.float32)
    k = rng.integers(-3, 4, (50, 128)).astype(np.float64)
    for h in (0, 7, 31):
        w = np.zeros((1, 32), np.float32)
        w[0, h] = 1.0
        s = oracle.indexer_scores(_bf16(q), w, k)[0]
        expect = [max(0.0, float(np.dot(q[0, h].astype(np.float64), k[t]))) for t in range(50)]
        assert np.array_equal(s, np.array(expect))


def test_closed_form_relu_per_head_before_weighting():
    # keys c_t * u, queries a_h * u with u = (+-1)^128: q_h . k_t = 128 a_h c_t,
    # so s(t) = sum_h w_h * max(0, 128 a_h c_t).  Mixed-sign a_h makes "ReLU after
    # the weighted sum" give a different number.
    rng = np.random.default_rng(3)
    u = rng.choice([-1.0, 1.0], 128)
    a = np.array([(h % 5) - 2 for h in range(32)], np.float64)
    c = np.array([-2.0, -1.0, 0.0, 1.0, 3.0])
    w = (np.arange(32, dtype=np.float32) + 1) / 32
    q = (a[:, None] * u[None, :])[None].astype(np.float32)
    k = c[:, None] * u[None, :]
    s = oracle.indexer_scores(_bf16(q), w[None], k)[0]
    expect = np.array([sum(float(w[h]) * max(0.0, 128.0 * a[h] * ct) for h in range(32)) for ct in c])
    assert np.array_equal(s, expect)
    assert s[2] == 0.0 and not np.signbit(s[2])


def test_visibility_of_draft_queries():
    # query j of S sees L - S + 1 + j rows: its own row and earlier ones
    rng = np.random.default_rng(4)
    S, L = 4, 37
    q = _bf16(rng.integers(-2, 3, (S, 32, 128)))
    w = (rng.integers(1, 9, (S, 32)) / 8).astype(np.float32)
    k = rng.integers(-2, 3, (L, 128)).astype(np.float64)
    out = oracle.indexer_scores(q, w, k)
    assert [o.shape[0] for o in out] == [34, 35, 36, 37]
    # a row's score depends only on its own key: dropping the last row keeps the rest
    out2 = oracle.indexer_scores(q, w, k[:36].copy())
    for j in range(S):
        assert np.array_equal(out2[j], out[j][:33 + j])


def test_weight_scaling_and_nonnegativity():
    rng = np.random.default_rng(5)
    q = _bf16(rng.standard_normal((2, 32, 128)))
    w = rng.random((2, 32)).astype(np.float32)
    k = rng.standard_normal((300, 128))
    s1 = oracle.indexer_scores(q, w, k)
    s2 = oracle.indexer_scores(q, (w * 4).astype(np.float32), k)
    for a, b in zip(s1, s2):
        assert np.array_equal(b, 4 * a)
        assert np.all(a >= 0)


def test_all_negative_dots_give_zero():
    q = _bf16(np.ones((1, 32, 128)))
    k = -np.ones((10, 128))
    s = oracle.indexer_scores(q, np.ones((1, 32), np.float32), k)[0]
    assert np.all(s == 0.0) and not np.any(np.signbit(s))


def test_fp8_scale_factors_out():
    # ReLU(s x) = s ReLU(x) for s > 0: a shared power-of-two scale scales every score
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, (64, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10                       # no NaN codes
    q = _bf16(rng.standard_normal((1, 32, 128)))
    w = rng.random((1, 32)).astype(np.float32)
    k1 = oracle.dequant_idx_keys(codes, np.ones(64, np.float32))
    k8 = oracle.dequant_idx_keys(codes, np.full(64, 0.125, np.float32))
    assert np.array_equal(oracle.indexer_scores(q, w, k8)[0], 0.125 * oracle.indexer_scores(q, w, k1)[0])


def test_generated_workload_keys_roundtrip():
    # the generator's token-ordered keys, dequantised, stay within e4m3 rounding of N(0,1)+shift
    wl = synth.toy(seed=11, batch=1, ctx=(300,))
    codes, scale = synth.idx_tokens(wl, 0, 0, 300)
    k = oracle.dequant_idx_keys(codes, scale)
    sal = synth.salient_mask(wl, 0, 0, 300)
    assert abs(k[~sal].mean()) < 0.05 and abs(k[sal].mean() - 3.0) < 0.5
    assert np.allclose(np.abs(k).max(axis=1), 448 * scale.astype(np.float64), rtol=1e-6)

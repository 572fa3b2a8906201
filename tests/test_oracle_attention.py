"""Pins of the oracle's sparse MLA attention (dense SDPA special case, closed forms)."""
import math

import numpy as np
import torch

import oracle
import synth


def _q(rng, scale=1.0):
    return synth.encode_bf16(rng.standard_normal((64, 576)).astype(np.float32) * scale)


def test_selecting_every_row_equals_torch_sdpa_mqa():
    # K >= L: sparse attention over all rows is dense attention; one latent row
    # serves all 64 heads as key (576 dims) and value (first 512 dims)
    rng = np.random.default_rng(0)
    n = 77
    lat = rng.standard_normal((n, 576))
    qb = _q(rng)
    q = oracle.bf16_decode(qb)
    scale = 1.0 / math.sqrt(576)
    out, lse = oracle.attention(qb, lat, scale)
    qt = torch.from_numpy(q).view(1, 64, 1, 576)
    k = torch.from_numpy(lat).view(1, 1, n, 576).expand(1, 64, n, 576)
    v = torch.from_numpy(lat[:, :512].copy()).view(1, 1, n, 512).expand(1, 64, n, 512)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=scale)
    assert np.allclose(out, ref.view(64, 512).numpy(), rtol=1e-12, atol=1e-13)
    logits = scale * (qt.view(64, 576) @ torch.from_numpy(lat).T)
    assert np.allclose(lse, torch.logsumexp(logits, dim=1).numpy(), rtol=1e-13)


def test_identical_rows_return_that_row():
    rng = np.random.default_rng(1)
    row = rng.standard_normal(576)
    lat = np.tile(row, (9, 1))
    qb = _q(rng)
    out, lse = oracle.attention(qb, lat, 0.1)
    assert np.allclose(out, np.tile(row[:512], (64, 1)), rtol=1e-14, atol=1e-14)
    logit = 0.1 * oracle.bf16_decode(qb) @ row
    assert np.allclose(lse, logit + math.log(9), rtol=1e-13)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    lat = rng.standard_normal((31, 576))
    out, lse = oracle.attention(np.zeros((64, 576), np.uint16), lat, 0.5)
    assert np.allclose(out, np.tile(lat[:, :512].mean(axis=0), (64, 1)), rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, math.log(31))


def test_row_permutation_invariance():
    rng = np.random.default_rng(3)
    lat = rng.standard_normal((200, 576))
    qb = _q(rng, 2.0)
    out1, lse1 = oracle.attention(qb, lat, 1 / 24)
    perm = rng.permutation(200)
    out2, lse2 = oracle.attention(qb, lat[perm], 1 / 24)
    assert np.allclose(out1, out2, rtol=1e-12, atol=1e-14) and np.allclose(lse1, lse2, rtol=1e-13)


def test_two_rows_closed_form():
    # two rows: out = sigmoid(d) v0 + sigmoid(-d) v1 with d = logit0 - logit1
    rng = np.random.default_rng(4)
    lat = rng.standard_normal((2, 576))
    qb = _q(rng)
    q = oracle.bf16_decode(qb)
    out, _ = oracle.attention(qb, lat, 0.05)
    d = 0.05 * (q @ lat[0] - q @ lat[1])
    a = 1 / (1 + np.exp(-d))
    expect = a[:, None] * lat[0, :512] + (1 - a)[:, None] * lat[1, :512]
    assert np.allclose(out, expect, rtol=1e-12, atol=1e-14)

"""Pins of oracle.attention: textbook identities of softmax attention, the
eq. (4) online recurrence against the dense definition (memory-budget page),
extreme logits, and independent library implementations (SciPy softmax,
PyTorch scaled_dot_product_attention in float64 on the CPU)."""

import numpy as np
import pytest
import scipy.special
import torch

from oracle.attention import dense_attention, kv_head_of, online_attention, softmax_weights
from tests.conftest import load_golden

EPS = np.finfo(np.float64).eps


def _rand(rng, n, Hq, Hkv, d, s=1.0):
    return (rng.standard_normal((Hq, d)) * s, rng.standard_normal((n, Hkv, d)),
            rng.standard_normal((n, Hkv, d)))


def test_softmax_matches_scipy_and_sums_to_one():
    rng = np.random.default_rng(1)
    for n in (1, 2, 17, 1000):
        s = rng.standard_normal(n) * 5
        p = softmax_weights(s)
        assert np.allclose(p, scipy.special.softmax(s), rtol=1e-14, atol=1e-300)
        assert abs(p.sum() - 1.0) <= n * EPS
        assert np.all(p >= 0)
    # shift invariance
    s = rng.standard_normal(50)
    assert np.allclose(softmax_weights(s), softmax_weights(s + 123.0), rtol=1e-13)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(2)
    q, K, V = _rand(rng, 1, 8, 2, 128)
    out = dense_attention(q, K, V, 0.1)
    for h in range(8):
        assert np.array_equal(out[h], V[0, h // 4])


def test_zero_query_or_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    q, K, V = _rand(rng, 37, 4, 4, 16)
    out = dense_attention(np.zeros_like(q), K, V, 0.3)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)
    K_eq = np.broadcast_to(K[:1], K.shape).copy()
    out = dense_attention(q, K_eq, V, 0.3)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(4)
    n, d = 50, 32
    q, K, V = _rand(rng, n, 1, 1, d)
    K[17, 0] = q[0] * 1e3       # score ~ 1e3 * |q|^2 dominates everything
    out = dense_attention(q, K, V, 1.0)
    assert np.allclose(out[0], V[17, 0], rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(5)
    n, Hq, Hkv, d = 29, 8, 2, 16
    q, K, V = _rand(rng, n, Hq, Hkv, d)
    out = dense_attention(q, K, V, 0.25)
    K_rep = np.repeat(K, Hq // Hkv, axis=1)   # query head h -> copy of kv head h // G
    V_rep = np.repeat(V, Hq // Hkv, axis=1)
    assert np.array_equal(out, dense_attention(q, K_rep, V_rep, 0.25))
    assert [kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(6)
    for (n, Hq, Hkv, d) in ((1, 4, 4, 8), (37, 8, 2, 128), (300, 4, 1, 64), (5, 6, 3, 16)):
        q, K, V = _rand(rng, n, Hq, Hkv, d)
        scale = 1.0 / np.sqrt(d)
        ours = dense_attention(q, K, V, scale)
        tq = torch.from_numpy(q)[None, :, None, :]                      # [1, Hq, 1, d]
        tk = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]  # [1, Hkv, n, d]
        tv = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, scale=scale, enable_gqa=True)[0, :, 0, :].numpy()
        assert np.allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_permuting_keys_and_values_together_leaves_output_unchanged():
    rng = np.random.default_rng(8)
    q, K, V = _rand(rng, 64, 4, 2, 32)
    perm = rng.permutation(64)
    a = dense_attention(q, K, V, 0.2)
    b = dense_attention(q, K[perm], V[perm], 0.2)
    assert np.allclose(a, b, rtol=0, atol=1e-14)
    # but permuting values alone does change it (keys and values stay paired)
    c = dense_attention(q, K, V[perm], 0.2)
    assert not np.allclose(a, c, atol=1e-6)


def test_empty_context_gives_zero():
    q = np.ones((4, 8))
    out = dense_attention(q, np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 1.0)
    assert np.array_equal(out, np.zeros((4, 8)))


def test_online_equals_dense_several_block_sizes():
    g = load_golden("memory_budget_witness.json")["online_vs_dense"]
    rng = np.random.default_rng(9)
    worst = 0.0
    cases = 0
    for (n, Hq, Hkv, d) in ((7, 2, 1, 8), (16, 4, 4, 16), (33, 8, 2, 32), (511, 4, 1, 128)):
        q, K, V = _rand(rng, n, Hq, Hkv, d)
        dense = dense_attention(q, K, V, 1 / np.sqrt(d))
        for blk in (1, 4, 16, 32):
            on = online_attention(q, K, V, 1 / np.sqrt(d), blk)
            worst = max(worst, float(np.max(np.abs(on - dense))))
            cases += 1
    # the page's 8 small cases reached 2.2e-16; our larger n may reach a few eps
    assert cases >= g["attention_cases"]
    assert worst <= 1e-14
    assert worst >= 0.0 and g["largest_absolute_error"] == EPS


def test_online_with_block_equal_to_n_is_dense_up_to_rounding():
    rng = np.random.default_rng(10)
    q, K, V = _rand(rng, 40, 2, 2, 8)
    assert np.allclose(online_attention(q, K, V, 0.5, 40), dense_attention(q, K, V, 0.5),
                       rtol=0, atol=4 * EPS)


@pytest.mark.parametrize("mag", [1e2, 1e4])
def test_extreme_logits_no_overflow(mag):
    rng = np.random.default_rng(11)
    n, d = 200, 16
    q, K, V = _rand(rng, n, 2, 1, d)
    q = q / np.linalg.norm(q, axis=1, keepdims=True) * np.sqrt(mag)
    K = K / np.linalg.norm(K, axis=2, keepdims=True) * np.sqrt(mag)   # scores in [-mag, mag]
    dense = dense_attention(q, K, V, 1.0)
    assert np.all(np.isfinite(dense))
    for blk in (1, 8, 64):
        on = online_attention(q, K, V, 1.0, blk)
        assert np.all(np.isfinite(on))
        assert np.allclose(on, dense, rtol=0, atol=1e-12)
    # naive exp without the maximum shift overflows at these scores
    with np.errstate(over="ignore", invalid="ignore"):
        s = 1.0 * (K[:, 0, :] @ q[0])
        naive = np.exp(s) / np.sum(np.exp(s))
    if mag >= 1e4:
        assert not np.all(np.isfinite(naive))

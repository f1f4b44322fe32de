"""Pins for the oracle's causal prefill attention (no GPU).

The oracle writes out ordinary causal softmax attention over the prompt's
fp16 tensors ("Makale Bülteni -- KIVI", section "Kod ve Entegrasyon
Haritası": the prefill phase attends over full-precision keys and values).
Each pin fixes its result by something other than the formula: the single
visible token, closed forms (uniform weights give prefix means; logits
ln 1 and ln 3 give weights 1/4 and 3/4), a limit (a large logit gap selects
one value row), and invariants (causality, order of the past, GQA as MHA
with repeated KV heads), so that a dropped term, a wrong mask or index, or a
transposed operand fails one of them.
"""
import math

import numpy as np
import pytest


def f16(a):
    return np.asarray(a, np.float16).view(np.uint16)


def gauss(rng, *shape):
    return f16(rng.standard_normal(shape))


def test_first_row_is_first_value(orc):
    rng = np.random.default_rng(1)
    q, k, v = gauss(rng, 2, 4, 9, 16), gauss(rng, 2, 2, 9, 16), gauss(rng, 2, 2, 9, 16)
    out = orc.prefill_attention(q, k, v, 0.7)
    vf = v.view(np.float16).astype(np.float64)
    for h in range(4):
        assert np.array_equal(out[:, h, 0], vf[:, h // 2, 0])


@pytest.mark.parametrize("kind", ["zero_scale", "equal_keys"])
def test_uniform_weights_give_prefix_means(orc, kind):
    rng = np.random.default_rng(2)
    T = 23
    q, v = gauss(rng, 1, 2, T, 8), gauss(rng, 1, 1, T, 8)
    if kind == "zero_scale":
        k, sigma = gauss(rng, 1, 1, T, 8), 0.0
    else:
        k, sigma = np.repeat(gauss(rng, 1, 1, 1, 8), T, axis=2), 0.9
    out = orc.prefill_attention(q, k, v, sigma)
    vf = v.view(np.float16).astype(np.float64)[0, 0]
    want = np.cumsum(vf, axis=0) / np.arange(1, T + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(out[0, h], want, rtol=0, atol=1e-13)


def test_weights_one_quarter_three_quarters(orc):
    # q = e0, k0 = 0, k1 = e0, sigma = ln 3: logits 0 and ln 3, weights 1/4, 3/4
    d = 8
    q = np.zeros((1, 1, 2, d), np.float16)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, 2, d), np.float16)
    k[0, 0, 1, 0] = 1.0
    v = np.zeros((1, 1, 2, d), np.float16)
    v[0, 0, 0] = np.arange(d)
    v[0, 0, 1] = -2.0 * np.arange(d) + 1.0
    out = orc.prefill_attention(f16(q), f16(k), f16(v), math.log(3.0))
    want = 0.25 * np.arange(d) + 0.75 * (-2.0 * np.arange(d) + 1.0)
    np.testing.assert_allclose(out[0, 0, 1], want, rtol=0, atol=1e-14)


def test_large_gap_selects_the_maximum(orc):
    # q = e0 and k_j[0] integer, so logits are sigma * k_j[0]; with gaps >= 1
    # and sigma = 60 every other weight is below e^-60
    rng = np.random.default_rng(3)
    T, d = 17, 8
    keys0 = rng.permutation(T).astype(np.float64)
    q = np.zeros((1, 1, T, d), np.float16)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, T, d), np.float16)
    k[0, 0, :, 0] = keys0
    v = gauss(rng, 1, 1, T, d)
    out = orc.prefill_attention(f16(q), f16(k), v, 60.0)
    vf = v.view(np.float16).astype(np.float64)[0, 0]
    for i in range(T):
        j = int(np.argmax(keys0[:i + 1]))
        np.testing.assert_allclose(out[0, 0, i], vf[j], rtol=0, atol=1e-20 + 1e-12 * np.abs(vf[j]).max())


def test_causal_rows_ignore_later_tokens(orc):
    rng = np.random.default_rng(4)
    T = 12
    q, k, v = gauss(rng, 1, 2, T, 8), gauss(rng, 1, 1, T, 8), gauss(rng, 1, 1, T, 8)
    base = orc.prefill_attention(q, k, v, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, 7:] = gauss(rng, T - 7, 8)
    v2[0, 0, 7:] = gauss(rng, T - 7, 8)
    moved = orc.prefill_attention(q, k2, v2, 0.5)
    assert np.array_equal(base[:, :, :7], moved[:, :, :7])
    assert not np.allclose(base[:, :, 7:], moved[:, :, 7:])


def test_last_row_ignores_order_of_the_past(orc):
    rng = np.random.default_rng(5)
    T = 15
    q, k, v = gauss(rng, 1, 1, T, 8), gauss(rng, 1, 1, T, 8), gauss(rng, 1, 1, T, 8)
    perm = rng.permutation(T)
    rows = np.array([[0, 0, T - 1]])
    a = orc.prefill_attention(q, k, v, 0.6, rows=rows)
    b = orc.prefill_attention(q, k[:, :, perm], v[:, :, perm], 0.6, rows=rows)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads(orc):
    rng = np.random.default_rng(6)
    T = 10
    q, k, v = gauss(rng, 2, 4, T, 8), gauss(rng, 2, 2, T, 8), gauss(rng, 2, 2, T, 8)
    gqa = orc.prefill_attention(q, k, v, 0.4)
    mha = orc.prefill_attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), 0.4)
    assert np.array_equal(gqa, mha)


def test_row_selection_matches_full_output(orc):
    rng = np.random.default_rng(7)
    q, k, v = gauss(rng, 2, 2, 11, 8), gauss(rng, 2, 1, 11, 8), gauss(rng, 2, 1, 11, 8)
    full = orc.prefill_attention(q, k, v, 0.3)
    rows = np.array([[1, 0, 10], [0, 1, 3], [1, 1, 0]])
    part = orc.prefill_attention(q, k, v, 0.3, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(part[r], full[b, h, i])

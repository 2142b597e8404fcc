"""Pins of the low-rank latent decode oracle (CPU only).

Each check ties oracle/latent.py to something other than itself: the
textbook attention of a library routine when the up-projections are the
identity, the invariance of the factorisation under a change of latent
basis, closed forms (uniform scores, a single position), the query-head to
KV-head mapping of grouped-query attention, and the layout's own
properties (distinct, in-bounds offsets; the tile and row shapes).
"""
import numpy as np
import pytest
import torch

from oracle import latent


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_identity_up_projection_is_textbook_attention():
    """r = D, B_K = B_V = I: plain attention over the latents themselves,
    checked against torch's scaled_dot_product_attention in float64."""
    rng = np.random.default_rng(1)
    T, D = 37, 16
    ck, cv, q = _rand(rng, T, D), _rand(rng, T, D), _rand(rng, D)
    eye = np.eye(D)
    for length in (1, 5, 37):
        got = latent.decode_one(ck, cv, eye, eye, q, length, 0.3)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[None, None, None]), torch.tensor(ck[None, None, :length]),
            torch.tensor(cv[None, None, :length]), scale=0.3)[0, 0, 0].numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_latent_basis_change_leaves_output_unchanged():
    """c -> c M, B -> M^-1 B reconstructs the same K and V, so the output
    must not move (a transposed or swapped factor breaks this)."""
    rng = np.random.default_rng(2)
    T, r, D = 50, 8, 24
    ck, cv, q = _rand(rng, T, r), _rand(rng, T, r), _rand(rng, D)
    bk, bv = _rand(rng, r, D) / 3, _rand(rng, r, D) / 3
    Qm, _ = np.linalg.qr(_rand(rng, r, r))
    M = Qm @ np.diag(rng.uniform(0.5, 2.0, r))
    Mi = np.linalg.inv(M)
    a = latent.decode_one(ck, cv, bk, bv, q, 41, 0.25)
    b = latent.decode_one(ck @ M, cv @ M, Mi @ bk, Mi @ bv, q, 41, 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    # K and V factors are independent: changing only V's basis is also exact
    c = latent.decode_one(ck, cv @ M, bk, Mi @ bv, q, 41, 0.25)
    np.testing.assert_allclose(a, c, rtol=1e-10, atol=1e-12)


def test_zero_key_latents_average_the_values():
    """Zero K latents give equal scores: the output is the mean V row,
    mean(c^V) B_V, over the attended prefix only."""
    rng = np.random.default_rng(3)
    T, r, D = 40, 6, 10
    cv, q, bk, bv = _rand(rng, T, r), _rand(rng, D), _rand(rng, r, D), _rand(rng, r, D)
    for length in (1, 7, 40):
        got = latent.decode_one(np.zeros((T, r)), cv, bk, bv, q, length, 1.0)
        np.testing.assert_allclose(got, cv[:length].mean(0) @ bv, rtol=1e-12, atol=1e-13)


def test_single_position_returns_its_value_row():
    rng = np.random.default_rng(4)
    r, D = 5, 7
    ck, cv, bk, bv, q = _rand(rng, 3, r), _rand(rng, 3, r), _rand(rng, r, D), \
        _rand(rng, r, D), _rand(rng, D)
    np.testing.assert_allclose(latent.decode_one(ck, cv, bk, bv, q, 1, 0.7), cv[0] @ bv,
                               rtol=1e-12, atol=1e-13)
    assert not latent.decode_one(ck, cv, bk, bv, q, 0, 0.7).any()


def test_two_positions_closed_form():
    """Two positions: weight of the second = sigmoid(score difference)."""
    rng = np.random.default_rng(5)
    r, D = 4, 6
    ck, cv, bk, bv, q = _rand(rng, 2, r), _rand(rng, 2, r), _rand(rng, r, D), \
        _rand(rng, r, D), _rand(rng, D)
    s = np.array([sum(q[d] * sum(ck[t, j] * bk[j, d] for j in range(r)) for d in range(D))
                  for t in range(2)]) * 0.5
    w1 = 1.0 / (1.0 + np.exp(s[0] - s[1]))
    V = np.array([[sum(cv[t, j] * bv[j, d] for j in range(r)) for d in range(D)]
                  for t in range(2)])
    np.testing.assert_allclose(latent.decode_one(ck, cv, bk, bv, q, 2, 0.5),
                               (1 - w1) * V[0] + w1 * V[1], rtol=1e-12, atol=1e-13)


def test_query_heads_read_their_group_kv_head():
    """With every V row of KV head h equal to e_h B_V (one-hot latent), each
    query head's output is exactly the row of its own KV head i // G."""
    rng = np.random.default_rng(6)
    L, B, Hkv, G, T, r, D = 2, 2, 3, 4, 9, 4, 8
    ck = _rand(rng, L, B, Hkv, T, r)
    cv = np.zeros((L, B, Hkv, T, r))
    for h in range(Hkv):
        cv[:, :, h, :, h] = 1.0
    bk, bv = _rand(rng, L, Hkv, r, D), _rand(rng, L, Hkv, r, D)
    q = _rand(rng, L, B, Hkv * G, D)
    out = latent.decode(ck, cv, bk, bv, q, [9, 4], 0.4)
    for l in range(L):
        for i in range(Hkv * G):
            for s in range(B):
                np.testing.assert_allclose(out[l, s, i], bv[l, i // G, i // G], rtol=1e-12)


def test_layout_is_a_bijection_onto_disjoint_tiles():
    cap, Hkv, r, L = [5, 33, 64, 1], 2, 8, 2
    seen = set()
    total = latent.cache_bytes(L, Hkv, cap, r)
    assert latent.row_bases(cap) == [0, 32, 96, 160, 192]
    assert total == L * Hkv * 2 * (-(-(192 * r * 2) // 256) * 256)
    for l in range(L):
        for h in range(Hkv):
            for X in (0, 1):
                for s, c in enumerate(cap):
                    for t in range(c):
                        for j in range(r):
                            o = latent.latent_offset(Hkv, cap, r, l, h, X, s, t, j)
                            assert o % 2 == 0 and 0 <= o and o + 2 <= total
                            assert o not in seen
                            seen.add(o)
    # rows are r contiguous bf16 values, consecutive positions consecutive
    # rows, and a sequence starts on a 32-row boundary of its plane
    plane = total // (L * Hkv * 2)
    for X in (0, 1):
        o0 = latent.latent_offset(Hkv, cap, r, 1, 1, X, 1, 3, 0)
        assert latent.latent_offset(Hkv, cap, r, 1, 1, X, 1, 3, 7) == o0 + 14
        assert latent.latent_offset(Hkv, cap, r, 1, 1, X, 1, 4, 0) == o0 + 2 * r
        assert latent.latent_offset(Hkv, cap, r, 1, 1, X, 2, 0, 0) == \
            ((1 * Hkv + 1) * 2 + X) * plane + 96 * r * 2


@pytest.mark.parametrize("bits,value", [(0x3F80, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -133),
                                        (0x7F7F, 3.3895313892515355e38)])
def test_bf16_bits(bits, value):
    assert latent.bf16_bits_to_f64(np.array([bits], np.uint16))[0] == value


def test_huge_scores_pick_the_best_position():
    """Scores near 1e4 apart: the softmax is one-hot on the largest score
    (finite, no overflow), so the output is that position's V row."""
    rng = np.random.default_rng(7)
    T, r, D = 12, 3, 5
    ck, cv, bk, bv, q = _rand(rng, T, r), _rand(rng, T, r), _rand(rng, r, D), \
        _rand(rng, r, D), _rand(rng, D)
    s = (ck @ bk) @ q
    got = latent.decode_one(ck, cv, bk, bv, q, T, 1e4 / np.ptp(s))
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, cv[int(np.argmax(s))] @ bv, rtol=1e-9, atol=1e-12)

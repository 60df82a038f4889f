"""Pins of the attention / decode / merge oracle against what the pages and the
mathematics fix (no GPU). Each pin is chosen so that a plausible slip in the
oracle -- a dropped correction factor, a wrong sign in exp(m_old - m_new), a
transposed operand, a wrong GQA mapping, an off-by-one causal mask -- fails."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import merge_pair, segment_bounds
from online_softmax_attention_cascaded_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _worked():
    with open(GOLDEN) as f:
        return json.load(f)


def _score_embedding(scores, values):
    """q = e0, k_j = s_j e0, v_j = value_j e0 (d = 1), so scale-1 scores are s_j."""
    n = len(scores)
    q = np.ones((1, 1, 1, 1))
    k = np.asarray(scores, np.float64).reshape(1, 1, n, 1)
    v = np.asarray(values, np.float64).reshape(1, 1, n, 1)
    return q, k, v


# ---------------------------------------------------------------- worked example


def test_worked_example_printed_values():
    """Transcript cue 15: tile A = {1, 3}, tile B = {5}; the page prints the
    running values to two decimals and states the from-scratch sum in words."""
    g = _worked()
    tile_a, tile_b = g["tiles"]
    scores = tile_a + tile_b
    q, k, v = _score_embedding(scores, g["value_vector"])
    _, lse, trace = oracle.attention_online(q, k, v, 1.0, tile=len(tile_a))
    (m_a, l_a, _), (m_b, l_b, _) = trace
    pr = g["printed_rounded"]
    st = g["stated"]
    assert m_a == st["running_max_after_tile_A"]
    assert m_b == st["running_max_after_tile_B"]
    assert round(math.exp(m_a - m_b), pr["decimals"]) == pr["correction_after_tile_A_exp_minus_2"]
    assert round(l_a, pr["decimals"]) == pr["denominator_after_tile_A"]
    assert round(l_b, pr["decimals"]) == pr["denominator_after_tile_B"]
    # The from-scratch denominator relative to the final max, stated in words.
    from_scratch = math.exp(-4) + math.exp(-2) + 1
    assert abs(l_b - from_scratch) < 1e-15
    # And the unfused oracle gives the same log-sum-exp.
    _, lse_unfused = oracle.attention(q, k, v, 1.0)
    assert abs(lse_unfused[0, 0, 0] - (5 + math.log(from_scratch))) < 1e-14
    assert abs(lse[0, 0, 0] - lse_unfused[0, 0, 0]) < 1e-14


def test_worked_example_accumulator():
    """Visual explainer 'Rescale the output accumulator too': the accumulator of
    sum exp(x - m) v is rescaled by the same factor; divided once by l at the
    end it equals the from-scratch weighted average of v = [2, -1, 4]."""
    g = _worked()
    scores = g["tiles"][0] + g["tiles"][1]
    vals = g["value_vector"]
    q, k, v = _score_embedding(scores, vals)
    o_online, _, trace = oracle.attention_online(q, k, v, 1.0, tile=2)
    o_unfused, _ = oracle.attention(q, k, v, 1.0)
    # After tile A the accumulator is relative to max 3.
    acc_a = trace[0][2]
    assert abs(acc_a - (2 * math.exp(1 - 3) + (-1) * math.exp(3 - 3))) < 1e-15
    w = [math.exp(s - 5) for s in scores]
    expect = sum(wi * vi for wi, vi in zip(w, vals)) / sum(w)
    assert abs(o_online[0, 0, 0, 0] - expect) < 1e-14
    assert abs(o_unfused[0, 0, 0, 0] - expect) < 1e-14


@pytest.mark.parametrize("x3", _worked()["slider_variants"]["third_scores"])
def test_worked_example_slider(x3):
    """The slider of 'Online softmax, step by step' varies the third score: the
    online denominator relative to the final max equals the from-scratch one."""
    scores = [1.0, 3.0, x3]
    q, k, v = _score_embedding(scores, [2.0, -1.0, 4.0])
    _, lse_on, trace = oracle.attention_online(q, k, v, 1.0, tile=2)
    m = max(scores)
    assert trace[-1][0] == m
    assert abs(trace[-1][1] - sum(math.exp(s - m) for s in scores)) < 1e-14
    if x3 <= 3.0:  # no change of max: the correction factor is exactly 1
        assert trace[0][0] == trace[1][0] == 3.0


def test_worked_example_as_two_segments():
    """The same three keys split into ceil(3/2)=2 segments give tiles {1,3} | {5};
    the partial states and their merge reproduce the worked example."""
    q, k, v = inputs.worked_example_decode(d=8)
    m, l, acc = oracle.decode_partials(q, k, v, 1.0, 2)
    assert segment_bounds(3, 2) == [(0, 2), (2, 3)]
    assert m[0, 0].tolist() == [3.0, 5.0]
    assert abs(l[0, 0, 0] - (math.exp(-2) + 1)) < 1e-15
    assert l[0, 0, 1] == 1.0
    assert acc[0, 0, 1, 0] == 4.0
    o, lse = oracle.merge_states(m, l, acc)
    den = math.exp(-4) + math.exp(-2) + 1
    assert abs(lse[0, 0] - (5 + math.log(den))) < 1e-14
    assert abs(o[0, 0, 0] - (2 * math.exp(-4) - math.exp(-2) + 4) / den) < 1e-14
    assert np.all(o[0, 0, 1:] == 0)


# ---------------------------------------------------------------- closed forms


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_causal_first_row_is_first_value():
    q, k, v = _rand(1, 2, 3, 5, 8), _rand(2, 2, 3, 5, 8), _rand(3, 2, 3, 5, 8)
    o, lse = oracle.attention(q, k, v, 0.7, causal=True)
    assert np.allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    assert np.allclose(lse[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)


def test_zero_queries_average_values():
    """With q = 0 every visible score is 0: O is the mean of the visible V rows
    and lse = ln(number of visible keys)."""
    Lk = 7
    q = np.zeros((1, 2, Lk, 4))
    k, v = _rand(4, 1, 2, Lk, 4), _rand(5, 1, 2, Lk, 4)
    o, lse = oracle.attention(q, k, v, 1.3)
    assert np.allclose(o, v.mean(axis=2, keepdims=True).repeat(Lk, axis=2), atol=1e-15)
    assert np.allclose(lse, math.log(Lk), atol=1e-15)
    o, lse = oracle.attention(q, k, v, 1.3, causal=True)
    for i in range(Lk):
        assert np.allclose(o[:, :, i], v[:, :, : i + 1].mean(axis=2), atol=1e-15)
        assert np.allclose(lse[:, :, i], math.log(i + 1), atol=1e-15)


def test_single_key_returns_its_value():
    q, k, v = _rand(6, 1, 1, 3, 4), _rand(7, 1, 1, 1, 4), _rand(8, 1, 1, 1, 4)
    o, _ = oracle.attention(q, k, v, 0.5)
    assert np.allclose(o, np.broadcast_to(v, o.shape), atol=1e-15)


def test_gqa_groups_are_contiguous():
    """Query head h reads KV head h // group: a head remapped any other way gives
    a different answer, so this pins the mapping."""
    q = _rand(9, 1, 4, 3, 4)
    k, v = _rand(10, 1, 2, 5, 4), _rand(11, 1, 2, 5, 4)
    o, _ = oracle.attention(q, k, v, 0.5)
    for h in range(4):
        oh, _ = oracle.attention(q[:, h : h + 1], k[:, h // 2 : h // 2 + 1], v[:, h // 2 : h // 2 + 1], 0.5)
        assert np.allclose(o[:, h : h + 1], oh, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    """Library pin: torch's scaled_dot_product_attention in float64 on the CPU."""
    B, Hq, Hkv, L, d = 2, 4, 2, 19, 16
    q, k, v = _rand(12, B, Hq, L, d), _rand(13, B, Hkv, L, d), _rand(14, B, Hkv, L, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, scale, causal=causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    tk = tk.repeat_interleave(Hq // Hkv, dim=1)
    tv = tv.repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    # lse pin: logsumexp of the masked scaled scores.
    s = scale * torch.einsum("bhid,bhjd->bhij", tq, tk)
    if causal:
        s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), -math.inf)
    assert np.allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-13)


def test_latent_values_narrower_than_keys():
    """Multi-latent form: one shared latent row per key serves as the key (all
    dk columns) and as the value (its first dv columns). Pinned by torch's
    float64 attention with a narrower value width, and by linearity in V: the
    output equals the first dv columns of the output with v = k."""
    B, H, L, dk, dv = 2, 8, 37, 24, 16
    q = _rand(31, B, H, 1, dk)
    lat = _rand(32, B, 1, L, dk)
    scale = 1 / math.sqrt(dk)
    o, lse = oracle.attention(q, lat, lat[..., :dv], scale)
    tq, tk = torch.from_numpy(q), torch.from_numpy(lat).expand(B, H, L, dk)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tk[..., :dv], scale=scale)
    assert o.shape == (B, H, 1, dv)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    o_full, lse_full = oracle.attention(q, lat, lat, scale)
    assert np.allclose(o, o_full[..., :dv], rtol=0, atol=1e-15)
    assert np.array_equal(lse, lse_full)
    # decode partials with the narrower values merge to the same result
    m, l, acc = oracle.decode_partials(q[:, :, 0], lat, lat[..., :dv], scale, 3)
    assert acc.shape == (B, H, 3, dv)
    om, lm = oracle.merge_states(m, l, acc)
    assert np.allclose(om, o[:, :, 0], rtol=0, atol=1e-14) and np.allclose(lm, lse[:, :, 0], rtol=0, atol=1e-14)
    oo, lo, _ = oracle.attention_online(q, lat, lat[..., :dv], scale, tile=5)
    assert np.allclose(oo, o, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 3, 16, 64])
def test_online_equals_unfused(causal, tile):
    q, k, v = _rand(15, 1, 2, 21, 8), _rand(16, 1, 2, 21, 8), _rand(17, 1, 2, 21, 8)
    o1, l1 = oracle.attention(q, k, v, 0.4, causal=causal)
    o2, l2, _ = oracle.attention_online(q, k, v, 0.4, causal=causal, tile=tile)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14)
    assert np.allclose(l1, l2, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- segmentation and merge


def _compositions(n):
    """Every way to write n as an ordered sum of positive parts."""
    for cuts in range(1 << (n - 1)):
        parts, last = [], 0
        for i in range(1, n):
            if cuts >> (i - 1) & 1:
                parts.append(i - last)
                last = i
        parts.append(n - last)
        yield parts


@pytest.mark.parametrize("Lk", [1, 2, 3, 5, 8])
def test_every_segmentation_merges_to_unsplit(Lk):
    """Brute force over all 2^(Lk-1) segmentations (plus empty segments spliced in)."""
    d = 3
    q = _rand(20 + Lk, 2, 4, d)
    k, v = _rand(30 + Lk, 2, 2, Lk, d), _rand(40 + Lk, 2, 2, Lk, d)
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, 0.9)
    o_ref, lse_ref = o_ref[:, :, 0], lse_ref[:, :, 0]
    for parts in _compositions(Lk):
        bounds, t = [], 0
        for p in parts:
            bounds.append((t, t + p))
            t += p
        for with_empty in (False, True):
            bb = bounds + [(Lk, Lk)] if with_empty else bounds
            if with_empty:
                bb = [(0, 0)] + bb
            m, l, acc = oracle.decode_partials(q, k, v, 0.9, len(bb), bounds=bb)
            o, lse = oracle.merge_states(m, l, acc)
            assert np.allclose(o, o_ref, rtol=0, atol=1e-14), parts
            assert np.allclose(lse, lse_ref, rtol=0, atol=1e-14), parts


@pytest.mark.parametrize("S", [1, 4, 16, 64, 100])
def test_ceil_div_segments_merge_to_unsplit(S):
    d, Lk = 8, 1000
    q = _rand(50, 1, 4, d)
    k, v = _rand(51, 1, 1, Lk, d), _rand(52, 1, 1, Lk, d)
    o_ref, lse_ref = oracle.attention(q[:, :, None], k, v, 0.35)
    m, l, acc = oracle.decode_partials(q, k, v, 0.35, S)
    o, lse = oracle.merge_states(m, l, acc)
    assert np.allclose(o, o_ref[:, :, 0], rtol=0, atol=1e-13)
    assert np.allclose(lse, lse_ref[:, :, 0], rtol=0, atol=1e-13)


def test_trailing_empty_segments_are_identity():
    """Lk = 5, S = 4 gives lengths 2, 2, 1, 0: the last state is the identity."""
    assert segment_bounds(5, 4) == [(0, 2), (2, 4), (4, 5), (5, 5)]
    q = _rand(60, 1, 1, 4)
    k, v = _rand(61, 1, 1, 5, 4), _rand(62, 1, 1, 5, 4)
    m, l, acc = oracle.decode_partials(q, k, v, 1.0, 4)
    assert m[0, 0, 3] == -math.inf and l[0, 0, 3] == 0 and np.all(acc[0, 0, 3] == 0)


def test_merge_is_a_commutative_monoid():
    rng = np.random.default_rng(70)
    states = [(float(rng.normal() * 3), float(rng.uniform(0.5, 4)), rng.normal(size=5)) for _ in range(4)]
    ident = (-math.inf, 0.0, np.zeros(5))

    def close(a, b):
        return a[0] == b[0] and abs(a[1] - b[1]) < 1e-12 * abs(a[1]) and np.allclose(a[2], b[2], atol=1e-12)

    a, b, c, _ = states
    assert close(merge_pair(merge_pair(a, b), c), merge_pair(a, merge_pair(b, c)))
    assert close(merge_pair(a, b), merge_pair(b, a))
    assert close(merge_pair(a, ident), a) and close(merge_pair(ident, a), a)
    # The array merge is order independent too.
    m = np.array([s[0] for s in states])
    l = np.array([s[1] for s in states])
    acc = np.stack([s[2] for s in states])
    o0, lse0 = oracle.merge_states(m, l, acc)
    for perm in itertools.permutations(range(4)):
        o1, lse1 = oracle.merge_states(m[list(perm)], l[list(perm)], acc[list(perm)])
        assert np.allclose(o0, o1, atol=1e-14) and abs(lse0 - lse1) < 1e-14


def test_merge_of_identities_only():
    m = np.full((2, 3), -math.inf)
    l = np.zeros((2, 3))
    acc = np.zeros((2, 3, 4))
    o, lse = oracle.merge_states(m, l, acc)
    assert np.all(o == 0) and np.all(lse == -math.inf)


def test_merge_with_identity_is_noop():
    m = np.array([[1.5, -math.inf, -0.5]])
    l = np.array([[2.0, 0.0, 3.0]])
    acc = _rand(71, 1, 3, 6)
    acc[0, 1] = 0
    o, lse = oracle.merge_states(m, l, acc)
    o2, lse2 = oracle.merge_states(m[:, [0, 2]], l[:, [0, 2]], acc[:, [0, 2]])
    assert np.allclose(o, o2, atol=1e-15) and np.allclose(lse, lse2, atol=1e-15)

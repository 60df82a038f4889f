"""Pins of the softmax -> top-k oracle (no GPU)."""

import numpy as np
import pytest
import torch

import oracle
from online_softmax_attention_cascaded_amd import inputs


def _brute(row, k):
    return sorted(range(len(row)), key=lambda j: (-float(row[j]), j))[:k]


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("E,k", [(1, 1), (5, 2), (8, 8), (16, 4), (33, 7)])
def test_indices_match_brute_force(seed, E, k):
    x = np.random.default_rng(seed).standard_normal((6, E)).astype(np.float32)
    _, idx = oracle.softmax_topk(x, k)
    for r in range(x.shape[0]):
        assert idx[r].tolist() == _brute(x[r], k)


@pytest.mark.parametrize("seed", range(3))
def test_ties_go_to_the_lower_index(seed):
    x = inputs.tie_heavy_logits(seed, 50, 24).numpy()
    _, idx = oracle.softmax_topk(x, 8)
    for r in range(x.shape[0]):
        assert idx[r].tolist() == _brute(x[r], 8)


def test_all_equal_row_selects_first_k():
    x = np.zeros((2, 16), np.float32)
    w, idx = oracle.softmax_topk(x, 5)
    assert idx.tolist() == [[0, 1, 2, 3, 4]] * 2
    assert np.allclose(w, 0.2, atol=1e-15)


def test_softmax_matches_torch_float64():
    x = np.random.default_rng(9).standard_normal((7, 40)) * 5
    p = oracle.softmax_rows(x)
    assert np.allclose(p, torch.softmax(torch.from_numpy(x), dim=-1).numpy(), rtol=0, atol=1e-15)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)


def test_softmax_closed_form_and_safety():
    """exp(ln j) = j: the row [0, ln 2, ln 3, ln 4] has softmax [1, 2, 3, 4] / 10,
    whatever constant is added (even +-1000, where exp alone over- or
    underflows); a constant row is uniform; -inf entries get weight 0."""
    base = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    want = np.array([1.0, 2.0, 3.0, 4.0]) / 10.0
    for c in (0.0, 1000.0, -1000.0, 37.5):
        assert np.allclose(oracle.softmax_rows((base + c)[None]), want, rtol=1e-12, atol=0)
    assert np.all(oracle.softmax_rows(np.full((2, 7), -3.25)) == 1.0 / 7)
    p = oracle.softmax_rows(np.array([[0.0, -np.inf, np.log(3.0), -np.inf]]))
    assert np.allclose(p, [[0.25, 0.0, 0.75, 0.0]], rtol=1e-15, atol=0)


def test_weights_invariants_and_modes():
    x = inputs.routing_inputs(3, 64, 256).numpy()
    w, idx = oracle.softmax_topk(x, 8, renormalize=True)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)
    w0, idx0 = oracle.softmax_topk(x, 8, renormalize=False)
    assert np.array_equal(idx, idx0)
    p = oracle.softmax_rows(x)
    assert np.allclose(w0, np.take_along_axis(p, idx0, axis=1), atol=0)
    # Renormalised weights depend only on the selected logits.
    sel = np.take_along_axis(x.astype(np.float64), idx, axis=1)
    e = np.exp(sel - sel[:, :1])
    assert np.allclose(w, e / e.sum(axis=1, keepdims=True), atol=1e-15)


def test_unique_spike_is_first():
    x = np.random.default_rng(4).standard_normal((10, 32)).astype(np.float32)
    cols = np.arange(10) * 3
    x[np.arange(10), cols] = 100.0
    w, idx = oracle.softmax_topk(x, 3)
    assert idx[:, 0].tolist() == cols.tolist()
    assert np.all(w[:, 0] > 0.999)


def test_spiked_rows_in_generator():
    """The generator adds +6 to one expert in exactly round(1 % T) rows."""
    T, E = 2000, 64
    x = inputs.routing_inputs(11, T, E).numpy()
    base = np.random.default_rng(11).standard_normal(size=(T, E), dtype=np.float32)
    changed = np.argwhere(x != base)
    assert len(changed) == 20 and len(set(changed[:, 0].tolist())) == 20
    assert np.allclose(x[tuple(changed.T)] - base[tuple(changed.T)], 6.0, atol=1e-5)

"""GPU parity of rf_softmax_topk (through the C ABI) against the fp64 oracle:
indices bit-exact (ties to the lower index), weights within 1e-5 relative."""

import numpy as np
import pytest

import oracle
import online_softmax_attention_cascaded_amd as rf
from online_softmax_attention_cascaded_amd import inputs
from gpu_util import DEV, needs_gpu, np32, print_case

pytestmark = [pytest.mark.gpu, needs_gpu]


def _check(x, k, renormalize):
    w, idx = rf.softmax_topk(x.to(DEV), k, renormalize)
    w_ref, idx_ref = oracle.softmax_topk(x.numpy(), k, renormalize)
    got = idx.cpu().numpy()
    bad = np.argwhere(got != idx_ref)
    assert len(bad) == 0, f"first index mismatch at {bad[:3].tolist()}"
    rel = np.abs(np32(w) - w_ref) / w_ref
    assert rel.max() <= 1e-5, rel.max()


@pytest.mark.parametrize("renormalize", [True, False])
def test_routing_config(renormalize):
    """16384 tokens x 256 experts, 1 % spiked rows, top-8."""
    print_case(test="routing_full", renormalize=renormalize)
    _check(inputs.routing_inputs(3, 16384, 256), 8, renormalize)


@pytest.mark.parametrize("E,k", [(4, 1), (4, 4), (64, 2), (128, 8), (256, 1), (256, 2), (256, 5), (256, 7), (256, 8), (256, 9), (256, 16), (256, 32), (512, 8), (1024, 16), (1000, 5)])
def test_routing_shapes(E, k):
    print_case(test="routing_shapes", E=E, k=k)
    _check(inputs.routing_inputs(9, 37, E), k, True)


@pytest.mark.parametrize("seed", [0, 1])
def test_routing_ties(seed):
    """Logits drawn from four values: almost every selection is a tie."""
    _check(inputs.tie_heavy_logits(seed, 300, 256), 8, True)
    _check(inputs.tie_heavy_logits(seed, 300, 64), 8, False)
    _check(inputs.tie_heavy_logits(seed, 300, 256), 8, False)
    _check(inputs.tie_heavy_logits(seed, 300, 256), 3, True)


@pytest.mark.parametrize("renormalize", [True, False])
def test_routing_winners_in_one_slice(renormalize):
    """256 experts: the kernel gives each of 16 lanes the experts 4 j + 64 c + e
    (c, e < 4). Rows whose whole top-8 lies in one such set of 16, with equal
    values among them, so one lane supplies every winner."""
    import torch

    g = torch.Generator().manual_seed(4)
    x = torch.randn((48, 256), generator=g)
    for r in range(48):
        j = r % 16
        own = [4 * j + 64 * c + e for c in range(4) for e in range(4)]
        vals = torch.tensor([9.0, 9.0, 8.5, 8.0, 8.0, 8.0, 7.5, 7.0, 6.5, 6.5, 6.0, 5.5, 5.0, 5.0, 4.5, 4.0])
        perm = torch.randperm(16, generator=g)
        x[r, own] = vals[perm]
    _check(x, 8, renormalize)
    _check(x, 5, renormalize)
    # distinct values: the same rows without equal keys
    for r in range(48):
        j = r % 16
        own = [4 * j + 64 * c + e for c in range(4) for e in range(4)]
        x[r, own] = 4.0 + 0.25 * torch.randperm(16, generator=g).float()
    _check(x, 8, renormalize)


@pytest.mark.parametrize("renormalize", [True, False])
def test_routing_one_ulp_neighbours(renormalize):
    """256 experts: the leading logits are consecutive fp32 values (keys that
    differ only in their lowest bits), placed at random experts, so some rows
    hold such neighbours inside one lane's set of experts and others only
    across lanes."""
    import torch

    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    ladder = [np.float32(5.0)]
    for _ in range(11):
        ladder.append(np.nextafter(ladder[-1], np.float32(np.inf)))
    for r in range(64):
        cols = rng.choice(256, size=12, replace=False)
        x[r, cols] = np.array(ladder, np.float32)[rng.permutation(12)]
    _check(torch.from_numpy(x), 8, renormalize)
    _check(torch.from_numpy(x), 3, renormalize)


def test_routing_signed_zero_ties():
    """-0.0 and +0.0 are equal logits: the lower index goes first."""
    import torch

    for E in (64, 256):
        x = torch.zeros((8, E))
        x[:, ::2] = -0.0
        x[:, 5] = 1.0
        _check(x, 8, True)
        _check(x, 8, False)


def test_routing_empty():
    import torch

    x = torch.zeros((0, 256), device=DEV)
    w, idx = rf.softmax_topk(x, 8)
    assert w.shape == (0, 8) and idx.shape == (0, 8)

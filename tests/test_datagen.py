"""Seeded input generators: determinism and mask recipes (CPU only)."""
import numpy as np
import torch

from group_sparse_ffn_amd import datagen as dg


def test_inputs_are_deterministic():
    a = dg.make_inputs(dg.TINY)
    b = dg.make_inputs(dg.TINY)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["X"].dtype == torch.float32 and a["mask"].dtype == torch.uint8
    assert a["mask"].shape == (64, 16)


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], dtype=np.float32)
    y = dg.to_dtype(x, "bf16").float().numpy()
    # ties go to even mantissa; below half rounds down
    assert y.tolist() == [1.0, 1.0 + 2 ** -6, 1.0]


def test_topk_mask_has_exactly_k_per_token():
    m = dg.mask_topk(500, 112, 56, seed=9)
    assert np.all(m.sum(axis=1) == 56)


def test_waterfill_hits_target_mean():
    rng = np.random.default_rng(0)
    b = rng.beta(2, 2, size=512)
    for target in (0.3, 0.5, 0.75, 0.9):
        p = dg.waterfill(b, target)
        assert abs(p.mean() - target) < 1e-9 and p.max() <= 1.0


def test_zipf_profile_saturates_and_averages_half():
    p = dg.zipf_profile(136, 0.5, seed=5004)
    assert abs(p.mean() - 0.5) < 1e-9
    assert np.sum(p >= 1.0 - 1e-12) > 10 and p.min() > 0.05


def test_sweep_cells_cover_the_grid():
    cells = dg.llama3b_sweep_cells()
    assert len(cells) == 72 and len({c.cell for c in cells}) == 72
    assert all(c.d_ff % c.G == 0 for c in cells)

"""The seeded input generators: determinism and the stated distributions (CPU)."""
import numpy as np
import torch

import synth


def test_deterministic_and_independent_per_expert():
    a = synth.gen_expert(3, 5, synth.PROJ_UP)
    b = synth.gen_expert(3, 5, synth.PROJ_UP)
    c = synth.gen_expert(3, 6, synth.PROJ_UP)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (1856, 2688 // 2) and a[1].shape == (1856, 2688 // 16)
    d = synth.gen_expert(3, 5, synth.PROJ_DOWN)
    assert d[0].shape == (2688, 1856 // 2) and d[1].shape == (2688, 1856 // 16)


def test_value_distributions():
    pk, sc = synth.gen_expert(2, 0, synth.PROJ_GATE)
    lo, hi = pk & 0xF, pk >> 4
    for nib in (lo, hi):
        counts = np.bincount(nib.reshape(-1), minlength=16)
        assert counts.min() > 0.9 * nib.size / 16 and counts.max() < 1.1 * nib.size / 16
    vals = torch.from_numpy(sc).view(torch.float8_e4m3fn).double().numpy()
    assert vals.min() >= 2.0 ** -4 and vals.max() <= 4.0
    assert 1.8 < vals.mean() < 2.2          # uniform on [1/16, 4] has mean ~2.03
    x = synth.gen_x(4).astype(np.uint32) << 16
    xf = x.view(np.float32)
    assert abs(xf.mean()) < 0.01 and abs(xf.std() - 1.0) < 0.01


def test_routing_uniform_and_zipf():
    ids, w = synth.gen_routing(4)
    assert ids.shape == (64, 8) and w.dtype == np.float32
    assert all(len(set(r)) == 8 for r in ids.tolist())
    assert np.allclose(w.sum(1), 1.0, atol=1e-6) and np.all(np.diff(w, axis=1) <= 0)
    ids3, _ = synth.gen_routing(3)
    counts = np.sort(np.bincount(ids3.reshape(-1), minlength=128))[::-1]
    assert counts[0] >= 15 and (counts > 0).sum() < 60      # skewed, uneven rows per expert
    ids5, _ = synth.gen_routing(5)
    c5 = np.bincount(ids5.reshape(-1), minlength=64)
    assert c5.min() > 80 and c5.max() < 180 and c5.sum() == 8192


def test_expert_bytes():
    assert synth.expert_bytes(synth.config(2)) == 2654208
    assert synth.expert_bytes(synth.config(4)) == 24772608

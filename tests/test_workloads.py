"""The seeded input generator: determinism, rounding and the recipe."""
import numpy as np
import pytest
import torch

from vision_mamba_selective_amd import workloads as wlm


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-30, 65504.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8],
                                 np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(wlm.round_bf16(x), ref)


def test_bf16_bits_roundtrip():
    x = wlm.round_bf16(np.linspace(-3, 3, 1001, dtype=np.float32))
    bits = wlm.to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, x)
    with pytest.raises(ValueError):
        wlm.to_bf16_bits(np.array([1.0 + 2 ** -12], np.float32))


def test_inputs_are_deterministic_and_shaped():
    wl = wlm.WORKLOADS[0].with_(dim=8)
    a = wlm.make_inputs(wl)
    b = wlm.make_inputs(wl)
    for name in ("u", "delta", "z", "B", "C", "A", "D", "dt_bias"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert a.u.shape == (1, 8, 197) and a.B.shape == (1, 16, 197)
    assert a.A.shape == (2, 8, 16) and a.D.shape == (2, 8) and a.dt_bias.shape == (2, 8)
    c = wlm.make_inputs(wl, seed=5)
    assert not np.array_equal(a.u, c.u)


def test_recipe_values():
    wl = wlm.WORKLOADS[1].with_(batch=2, dim=64)
    inp = wlm.make_inputs(wl)
    # A[d, n] = -(n+1), D = 1
    assert np.array_equal(inp.A[1, 5], -(np.arange(16, dtype=np.float32) + 1))
    assert np.all(inp.D == 1.0)
    # softplus(dt_bias) lands in [dt_min, dt_max]
    dt = np.logaddexp(0.0, inp.dt_bias.astype(np.float64))
    assert dt.min() >= wl.dt_min * (1 - 1e-5) and dt.max() <= wl.dt_max * (1 + 1e-5)
    # bf16 activations are bf16-exact
    for a in (inp.u, inp.delta, inp.z, inp.B, inp.C):
        wlm.to_bf16_bits(a)
    # delta_raw is 0.5 * N(0,1)
    assert 0.45 < inp.delta.std() < 0.55


def test_cross4_workload_layout():
    wl = wlm.WORKLOADS[3].with_(batch=1, dim=4)
    inp = wlm.make_inputs(wl)
    assert inp.B.shape == (1, 4, 16, 64 * 64)
    assert inp.z is None and wl.H * wl.W == wl.seqlen


def test_algorithmic_bytes_of_headline():
    wl = wlm.WORKLOADS[wlm.HEADLINE]
    # u, delta, z, y in bf16 + B, C in bf16 + A, D, dt_bias in fp32
    tc = 8 * 768 * 4097
    exp = 4 * tc * 2 + 2 * 8 * 16 * 4097 * 2 + 2 * 768 * 18 * 4
    assert wl.algorithmic_bytes() == exp == 203_584_000


def test_channel_subset_matches_slices():
    wl = wlm.WORKLOADS[0].with_(dim=10)
    inp = wlm.make_inputs(wl)
    sub = wlm.channel_subset(inp, [0], [3, 7])
    assert np.array_equal(sub.u, inp.u[:, [3, 7]])
    assert np.array_equal(sub.A, inp.A[:, [3, 7]])
    assert sub.wl.dim == 2


def test_high_resolution_workload_shape():
    """1248 x 1248 pixels at 16 x 16 patches plus the class token."""
    wl = wlm.WORKLOADS[5]
    assert (wl.kind, wl.seqlen, wl.dim, wl.dstate, wl.dtype) == ("vim", 6085, 768, 16, wlm.BF16)

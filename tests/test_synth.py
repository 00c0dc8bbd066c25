"""The seeded input generator: determinism, layouts and bf16 rounding."""
import numpy as np
import torch

from sparse_prefix_kv_amd import synth


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, 1e-40],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = synth.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    bits = synth.bf16_bits(got)
    assert np.array_equal(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy(),
                          got)


def test_layouts_and_determinism():
    for name, wl in synth.WORKLOADS.items():
        if wl.ragged is None:
            lay = synth.layout_from_runs(wl.segments)
            assert lay.total_L == sum(n for r in wl.segments for _, n in r)
    lay = synth.layout_from_runs(synth.WORKLOADS["interleaved32k"].segments)
    assert lay.total_L == 32768 and lay.n_text[0] == 8192 and lay.n_img[0] == 24576
    assert lay.modality[1023] == 0 and lay.modality[1024] == 1 and lay.modality[4096] == 0
    wl = synth.Workload("x", "bf16", 4, 2, 8, 4, 32, segments=(((0, 5), (1, 6)),))
    a = synth.make_inputs(wl, 3)
    b = synth.make_inputs(wl, 3)
    assert np.array_equal(a.K, b.K) and np.array_equal(a.W, b.W)
    assert np.array_equal(synth.bf16_round(a.K), a.K)


def test_ragged_layout_draw():
    wl = synth.WORKLOADS["ragged8"]
    x = synth.make_inputs(wl, 0, with_lmhead=False)
    lay = x.layout
    assert lay.nseq == 8
    assert np.all((lay.lens >= 2048) & (lay.lens <= 16384))
    f = lay.n_img / lay.lens
    assert np.all((f > 0.25 - 1e-3) & (f < 0.9 + 1e-3))

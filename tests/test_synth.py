"""Host-side checks of the seeded input generators (no GPU)."""

import numpy as np

import synth
from synth import workloads as wl_mod


def test_workload_shapes():
    g = synth.workload("gpt2s")
    assert len(g.tensors) == 72
    assert sum(t.rows * t.cols for t in g.tensors) == 12 * (4 * 768 * 768 + 2 * 3072 * 768)
    x = synth.workload("gpt2xl")
    assert len(x.tensors) == 288
    assert sum(t.rows * t.cols for t in x.tensors) == 48 * (4 * 1600 ** 2 + 2 * 6400 * 1600)
    n = synth.workload("nmuon")
    assert [(t.rows, t.cols, t.split_rows, t.precond) for t in n.tensors] == [
        (2304, 768, 768, 0), (768, 768, 0, 0), (3072, 768, 0, 0), (768, 3072, 0, 1)]


def test_generators_deterministic_and_dtyped():
    w = synth.workload("gpt2s", layers=1)
    t = w.tensors[4]
    a = synth.gradient(w, t)
    b = synth.gradient(w, t)
    assert a.dtype == np.uint16 and a.shape == (3072, 768)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, synth.gradient(w, w.tensors[5].__class__(**{**t.__dict__, "index": 99})))
    tiny = synth.workload("tiny")
    g = synth.gradient(tiny, tiny.tensors[0])
    assert g.dtype == np.float32 and abs(g.std() - 1.0) < 0.01
    assert np.all(synth.momentum0(tiny, tiny.tensors[0]) == 0)
    wt = synth.weight(tiny, tiny.tensors[0])
    assert abs(wt.std() - 0.02) < 5e-4


def test_bf16_encoder_round_trip():
    x = np.array([1.0, -2.5, 0.0, 3.140625, 65536.0, -0.0078125], np.float32)
    assert np.array_equal(synth.bf16_bits_to_f32(synth.to_bf16_bits(x)), x)
    # ties to even at 1 + 2^-8
    assert synth.bf16_bits_to_f32(synth.to_bf16_bits(np.float32([1 + 2 ** -8])))[0] == 1.0


def test_lowrank_spectrum_decays():
    w = synth.workload("square")
    t = wl_mod.TensorSpec("w", 0, 0, 256, 256, "bf16")
    g = synth.bf16_bits_to_f32(synth.gradient(w, t)).astype(np.float64)
    s = np.linalg.svd(g, compute_uv=False)
    assert s[0] > 5 * s[8] and s[40] < 0.1   # rank-32 decaying part, then the 1e-3 noise bulk


def test_every_workload_generates():
    # one tensor of each workload draws its inputs (seed ids cover every name)
    for name in wl_mod.WORKLOADS:
        w = synth.workload(name, layers=1) if name in ("gpt2s", "gpt2xl") else synth.workload(name)
        t = min(w.tensors, key=lambda s: s.rows * s.cols)
        g = synth.gradient(w, t)
        assert g.shape == (t.rows, t.cols)
        assert synth.weight(w, t).shape == (t.rows, t.cols)
        assert synth.momentum0(w, t).shape == (t.rows, t.cols)
    c = synth.workload("conv")
    assert [(t.rows, t.cols) for t in c.tensors] == [(64, 288), (64, 576), (256, 576), (256, 2304),
                                                      (256, 2304), (256, 2304)]

"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
identical seeded inputs.

Bars (rel_F = ||x - ref||_F / ||ref||_F in float64, max over matrices):
  momentum buffer                        <= 1e-6
  orthogonalised update O, bf16 path     <= 2e-2
  orthogonalised update O, fp32 path     <= 1e-5
  new weight, fp32                       rel_F(W' - W) <= 1e-5
  new weight, bf16                       ||W' - W'_oracle||_F <= half a bf16 ulp
                                         of W' per element plus lr * scale *
                                         2e-2 ||O|| (the rounding of W' and the
                                         O bar); with ns_steps = 0, where O is
                                         exact to float32, every element within
                                         one ulp of RNE(oracle W')
  fused update, bf16, element by element every element of W' one of the two
                                         bf16 neighbours of W - lr*wd*W -
                                         lr*s*O_gpu (float64, from the GPU's
                                         own O), up to 8 float32 ulps of |W| +
                                         lr*s*|O| where the terms cancel
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_muon_amd as mm
from matrix_aware_optimizer_muon_amd import binding as B
import synth
from synth.workloads import TensorSpec, Workload
from tests.parity_common import (bf16_ulp_distance, check_w_bf16, check_w_update_elementwise, from_device,
                                 oracle_step, rel_f, say, to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_O = {"bf16": 2e-2, "f32": 1e-5}
TOL_M = 1e-6


class Case:
    """Device tensors + oracle inputs for one list of matrices."""

    def __init__(self, wl, specs, step=0, M0=None, W0=None):
        self.wl, self.specs = wl, specs
        self.G = [synth.gradient(wl, s, step) for s in specs]
        self.M = M0 if M0 is not None else [synth.momentum0(wl, s) for s in specs]
        self.W = W0 if W0 is not None else [synth.weight(wl, s) for s in specs]
        self.dW = [to_device(torch, w, s.dtype) for w, s in zip(self.W, specs)]
        self.dG = [to_device(torch, g, s.dtype) for g, s in zip(self.G, specs)]
        self.dM = [torch.from_numpy(m.copy()).cuda() for m in self.M]
        self.dO = [torch.empty(s.rows, s.cols, dtype=torch.float32, device="cuda") for s in specs]

    def descs(self, lr_mults=None, filters=False):
        out = []
        for k, s in enumerate(self.specs):
            ts = (self.dW[k], self.dG[k], self.dM[k], self.dO[k])
            if filters:
                # the same storage as 4-D 3x3 convolution filters (out, in, 3, 3)
                ts = tuple(t.view(s.rows, s.cols // 9, 3, 3) for t in ts)
            out.append(mm.tensor_desc(ts[0], ts[1], ts[2], split_rows=s.split_rows,
                                      lr_mult=1.0 if lr_mults is None else lr_mults[k],
                                      update_out=ts[3]))
        return out

    def run(self, hp, lr=-1.0, lr_mults=None, filters=False):
        st = mm.MuonStep(self.descs(lr_mults, filters), hp)
        st.step(lr)
        torch.cuda.synchronize()
        flags = st.flags()
        st.close()
        return flags

    def results(self, k):
        s = self.specs[k]
        return (from_device(torch, self.dW[k], s.dtype), self.dM[k].cpu().numpy(),
                self.dO[k].cpu().numpy())


def check(case, hp, idx=None, lr=None, lr_mults=None, label=""):
    worst = {"M": 0.0, "O": 0.0, "W": 0.0, "Woff": 0.0, "Wulp": 0, "Wupd_off": 0.0}
    for k in (range(len(case.specs)) if idx is None else idx):
        s = case.specs[k]
        ref = oracle_step(case.W[k], case.G[k], case.M[k], s.dtype, hp, split_rows=s.split_rows,
                          lr=lr, lr_mult=1.0 if lr_mults is None else lr_mults[k])
        W1, M1, O1 = case.results(k)
        eM, eO = rel_f(M1, ref["M"]), rel_f(O1, ref["O"])
        assert eM <= TOL_M, f"{label} matrix {k} {s.rows}x{s.cols}: momentum rel_F {eM:.3e}"
        assert eO <= TOL_O[s.dtype], f"{label} matrix {k} {s.rows}x{s.cols}: O rel_F {eO:.3e}"
        if s.dtype == "bf16":
            lr_used = float(hp.lr) if lr is None else lr
            err, bound, frac = check_w_bf16(W1, ref, lr_used, ref["scale"])
            assert err <= bound, f"{label} matrix {k}: ||W'-W'_ref|| {err:.3e} > bound {bound:.3e}"
            if hp.ns_steps == 0:
                # O is exact to float32 here: W' must be the correctly rounded value
                assert bf16_ulp_distance(W1, ref["W_bits"]).max() <= 1, f"{label} matrix {k}: W ulp"
            # the update the kernel fused, per element, from its own O
            wd = float(hp.weight_decay)
            ulp, off = check_w_update_elementwise(W1, case.W[k], O1, lr_used, wd, ref["scale"])
            assert ulp <= 1.0, f"{label} matrix {k} {s.rows}x{s.cols}: fused update off by {ulp:.2f} of its bound"
            worst["Woff"] = max(worst["Woff"], 1.0 - frac)
            worst["Wulp"] = max(worst["Wulp"], ulp)
            worst["Wupd_off"] = max(worst["Wupd_off"], off)
        else:
            W0 = np.asarray(case.W[k], np.float64)
            eW = rel_f(np.asarray(W1, np.float64) - W0, ref["W"] - W0)
            assert eW <= 1e-5, f"{label} matrix {k}: rel_F(dW) {eW:.3e}"
            worst["W"] = max(worst["W"], eW)
        worst["M"] = max(worst["M"], eM)
        worst["O"] = max(worst["O"], eO)
    say(f"  {label}: max rel_F M {worst['M']:.2e}  O {worst['O']:.2e}  dW {worst['W']:.2e}  "
        f"W not bitwise {worst['Woff']:.1%}  fused update: max {worst['Wulp']:.2f} of bound, "
        f"{worst['Wupd_off']:.2%} not bitwise")
    return worst


def adhoc(name, shapes, dtype, law="gauss", mom0=1e-2, split=None, std=1.0, **kw):
    specs = [TensorSpec(f"m{k}", 0, 1000 + k, r, c, dtype, split_rows=(split or {}).get(k, 0))
             for k, (r, c) in enumerate(shapes)]
    return Workload("tiny", specs, grad_law=law, grad_std=std, mom0_std=mom0, **kw)


# ---------------------------------------------------------------------------

def test_tiny_fp32_workload():
    say("case: tiny 256x512 fp32, one step")
    wl = synth.workload("tiny")
    c = Case(wl, wl.tensors)
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    check(c, hp, label="tiny")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_shapes(dtype):
    shapes = [(300, 520), (520, 300), (17, 33), (33, 17), (1, 7), (7, 1), (1, 1),
              (257, 1000), (1000, 257), (64, 64), (3 * 96, 96), (129, 129),
              (128, 200), (200, 128)]   # bf16 m = 128: two K steps in the square and B X
    say(f"case: ragged shapes {dtype}")
    wl = adhoc("ragged", shapes, dtype, split={10: 96})
    c = Case(wl, wl.tensors)
    hp = mm.default_hparams()
    c.run(hp)
    check(c, hp, label=f"ragged/{dtype}")


class StridedCase(Case):
    """Case whose W, G and M are column slices of wider buffers (leading
    dimension ld = cols + pad); the padding columns hold a sentinel that the
    step must leave alone."""

    SENTINEL = 3.0

    def __init__(self, wl, specs, pads):
        super().__init__(wl, specs)
        self.bufs = []
        for k, pad in enumerate(pads):
            for name in ("dW", "dG", "dM"):
                t = getattr(self, name)[k]
                r, c = t.shape
                buf = torch.full((r, c + pad), self.SENTINEL, dtype=t.dtype, device="cuda")
                buf[:, :c] = t
                getattr(self, name)[k] = buf[:, :c]
                self.bufs.append((name, k, buf, c))

    def padding_untouched(self):
        return all(bool((buf[:, c:] == self.SENTINEL).all()) for _, _, buf, c in self.bufs)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_rows(dtype):
    # ld > cols for weights, gradients and momenta: pads of 8 keep bf16 rows
    # 16-byte aligned where cols allows, pads of 3 make every row unaligned
    # (the kernels' element-wise paths); left, right, odd and split shapes
    shapes = [(300, 520), (520, 300), (129, 129), (64, 200), (3 * 96, 96)]
    pads = [8, 3, 3, 8, 5]
    say(f"case: strided rows {dtype}, pads {pads}")
    wl = adhoc("strided", shapes, dtype, split={4: 96})
    c = StridedCase(wl, wl.tensors, pads)
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    check(c, hp, label=f"strided/{dtype}")
    assert c.padding_untouched()


@pytest.mark.parametrize("variant", ["sgd", "no_nesterov", "ns0", "ns1", "ns3", "scale_none",
                                     "scale_rms", "scale_spectral", "lr_mult", "wd0", "lr0", "lr_override"])
def test_hyperparameter_variants(variant):
    shapes = [(200, 136), (136, 200), (3 * 64, 64)]
    say(f"case: variant {variant}")
    wl = adhoc("var", shapes, "bf16", split={2: 64})
    c = Case(wl, wl.tensors)
    kw, lr, mults = {}, -1.0, None
    if variant == "sgd": kw = dict(momentum_form=B.MOM_SGD)
    if variant == "no_nesterov": kw = dict(nesterov=0)
    if variant == "ns0": kw = dict(ns_steps=0)
    if variant == "ns1": kw = dict(ns_steps=1)
    if variant == "ns3": kw = dict(ns_steps=3)
    if variant == "scale_none": kw = dict(scale_mode=B.SCALE_NONE)
    if variant == "scale_rms": kw = dict(scale_mode=B.SCALE_MATCH_RMS_ADAMW)
    if variant == "scale_spectral": kw = dict(scale_mode=B.SCALE_SPECTRAL)
    if variant == "wd0": kw = dict(weight_decay=0.0)
    if variant == "lr0": lr = 0.0
    if variant == "lr_override": lr = 0.05
    if variant == "lr_mult": mults = [0.5, 2.0, 1.5]
    hp = mm.default_hparams(**kw)
    c.run(hp, lr=lr, lr_mults=mults)
    check(c, hp, lr=None if lr < 0 else float(np.float32(lr)),
          lr_mults=None if mults is None else [float(np.float32(x)) for x in mults], label=variant)
    if variant == "lr0":
        for k, s in enumerate(c.specs):
            assert np.array_equal(c.results(k)[0], c.W[k])


@pytest.mark.parametrize("rank", [8, 32])
def test_low_rank_plus_noise_mid_sizes(rank):
    # the failure mode of an X kept only in bf16: a rank-r gradient with a
    # decaying spectrum plus 1e-3 noise; the noise directions must grow by
    # a^5 through the iteration without being swamped by the rounding of
    # the large ones.  Short sides 128 .. 768, left and right.
    shapes = [(128, 384), (129, 300), (200, 200), (300, 520), (768, 768), (520, 300), (1536, 768)]
    say(f"case: low rank {rank} + 1e-3 noise, bf16, m in 128..768")
    wl = adhoc("lowrank", shapes, "bf16", law="lowrank", mom0=0.0, grad_rank=rank, noise_std=1e-3)
    c = Case(wl, wl.tensors)
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    w = check(c, hp, label=f"lowrank{rank}")
    assert w["O"] < 2e-2


def test_large_ragged_256_tiles():
    # a short side of 2048 or more takes 256 x 256 tiles in every phase: the
    # units are padded to 128 (2100 -> 2176) and the strip past the last
    # whole 256-tile is covered by 128-tiles (a row and a column strip for
    # the Gram and square, mirror-stored; a row strip for B X); a tall
    # matrix (the last B X writes weight rows from tile columns) and an exact
    # multiple of the tile; enough units that no phase counts as small (the
    # planner gives a phase that fits one round of 128-tiles 128-tiles)
    shapes = [(2100, 2300), (2300, 2100), (2048, 2048), (2100, 2500)]
    say("case: large ragged bf16 (256 x 256 tiles)")
    wl = adhoc("large", shapes, "bf16")
    c = Case(wl, wl.tensors)
    plan = mm.plan_describe(c.descs(), mm.default_hparams())
    assert [u["tiles"] for u in plan["units"]] == [[256] * 3] * 4
    assert all(v > 0 for v in plan["groups"][0]["tiles_by_edge"]["128"])   # the strips past 2048
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    w = check(c, hp, label="large/256")
    assert w["O"] < 2e-2


def test_mid_ragged_mixed_tiles():
    # mid-sized short sides: B X at 256 x 256 with 128-tile strips past the
    # last whole 256-tile (1000 x 1100: a column strip; 1100 x 1000 tall: the
    # column strip holds weight rows), the Gram and square at 128; the
    # 1600-row units: the Gram at 256 with its 128-strip too, the square at
    # 128.  Seven units (one lane), so that no phase counts as small.
    shapes = [(1000, 1100), (1100, 1000), (1600, 1700), (1700, 1600), (1600, 3000), (1600, 1700), (1700, 1600)]
    say("case: mid ragged bf16 (256- and 128-tiles in one phase)")
    wl = adhoc("mid", shapes, "bf16")
    c = Case(wl, wl.tensors)
    plan = mm.plan_describe(c.descs(), mm.default_hparams())
    assert [u["tiles"] for u in plan["units"]] == [[128, 128, 256]] * 2 + [[256, 128, 256]] * 5
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    w = check(c, hp, label="mid/mixed")
    assert w["O"] < 2e-2


def test_zero_gradient_and_nonfinite_flag():
    say("case: zero gradient / non-finite flag")
    wl = adhoc("zero", [(64, 96)], "bf16", mom0=0.0)
    c = Case(wl, wl.tensors)
    c.dG[0].zero_()
    c.G[0] = np.zeros_like(c.G[0])
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    W1, M1, O1 = c.results(0)
    assert np.all(O1 == 0) and np.all(M1 == 0)
    ref = oracle_step(c.W[0], c.G[0], c.M[0], "bf16", hp)
    assert bf16_ulp_distance(W1, ref["W_bits"]).max() <= 1     # O = 0: pure decay
    c2 = Case(wl, wl.tensors)
    c2.dG[0][3, 5] = float("nan")
    assert c2.run(hp) & 1


def test_gpt2_small_full_grouped_step():
    say("case: gpt2s full 72-matrix grouped step")
    wl = synth.workload("gpt2s")
    c = Case(wl, wl.tensors)
    hp = mm.default_hparams()
    assert c.run(hp) == 0
    # every one of the 72 matrices: momentum, O, the new weight (aggregate
    # and per element); the maximum over matrices is reported
    w = check(c, hp, label="gpt2s all 72 matrices")
    assert w["O"] < 2e-2


def test_conv_filters_as_4d_tensors():
    # convolution filters handed over as (out, in, 3, 3) tensors: Muon works
    # on their out x (in*9) views; m = 64 filters run the float32 path, m =
    # 256 the bf16 path
    say("case: conv filter set, 4-D tensors")
    wl = synth.workload("conv")
    c = Case(wl, wl.tensors)
    hp = mm.default_hparams()
    assert c.run(hp, filters=True) == 0
    w = check(c, hp, label="conv filters")
    assert w["O"] < 2e-2


def test_square_4096_ten_steps():
    say("case: square 4096x4096 bf16, 10 consecutive steps")
    wl = synth.workload("square")
    spec = wl.tensors[0]
    c = Case(wl, [spec], step=0)
    hp = mm.default_hparams()
    st = mm.MuonStep(c.descs(), hp)
    from oracle import muon_oracle as orc
    M_ref = np.asarray(c.M[0], np.float64)
    W_first = None
    for step in range(10):
        G = synth.gradient(wl, spec, step)
        c.dG[0].copy_(to_device(torch, G, "bf16"))
        if step == 0:
            W_first = c.W[0]
        st.step()
        torch.cuda.synchronize()
        M_prev = M_ref
        M_ref, U = orc.momentum_update(M_ref, orc.bf16_bits_to_f64(G), float(hp.momentum))
        eM = rel_f(c.dM[0].cpu().numpy(), M_ref)
        assert eM <= TOL_M, f"step {step}: momentum rel_F {eM:.3e}"
        if step in (0, 9):
            O_ref = orc.orthogonalise(U, hp.ns_steps, float(hp.eps), float(hp.ns_a), float(hp.ns_b), float(hp.ns_c))
            eO = rel_f(c.dO[0].cpu().numpy(), O_ref)
            say(f"  step {step + 1}: momentum {eM:.2e}  O {eO:.2e}")
            assert eO <= TOL_O["bf16"]
            if step == 0:
                Wref = orc.apply_update(orc.bf16_bits_to_f64(W_first), O_ref, float(hp.lr),
                                        float(hp.weight_decay), 1.0)
                ref = {"W": Wref, "O": O_ref, "W_bits": orc.f64_to_bf16_bits(Wref)}
                W1 = from_device(torch, c.dW[0], "bf16")
                err, bound, frac = check_w_bf16(W1, ref, float(hp.lr), [1.0] * spec.rows)
                ulp, off = check_w_update_elementwise(W1, W_first, c.dO[0].cpu().numpy(), float(hp.lr),
                                                      float(hp.weight_decay), [1.0] * spec.rows)
                say(f"  step 1: ||dW err|| {err:.3e} <= {bound:.3e}; bitwise {frac:.1%}; "
                    f"fused update max {ulp:.2f} of bound ({off:.2%} off)")
                assert err <= bound and ulp <= 1.0
    assert st.flags() == 0
    st.close()


def test_gpt2_xl_full_grouped_step_sampled():
    say("case: gpt2xl full 288-matrix grouped step (sampled check)")
    wl = synth.workload("gpt2xl")
    specs = wl.tensors
    checked = [k for k, s in enumerate(specs) if s.layer == 0 or (s.layer == 47 and s.name in ("mlp_up", "mlp_down"))]
    gen = torch.Generator(device="cuda").manual_seed(4747)
    dW, dG, dM, dO, G, W, M = [], [], [], [], {}, {}, {}
    for k, s in enumerate(specs):
        if k in checked:
            G[k], W[k], M[k] = synth.gradient(wl, s), synth.weight(wl, s), synth.momentum0(wl, s)
            dG.append(to_device(torch, G[k], "bf16"))
            dW.append(to_device(torch, W[k], "bf16"))
        else:
            L = torch.randn(s.rows, 64, device="cuda", generator=gen) / torch.arange(1, 65, device="cuda")
            R = torch.randn(s.cols, 64, device="cuda", generator=gen)
            g = L @ R.T / 8.0 + 1e-3 * torch.randn(s.rows, s.cols, device="cuda", generator=gen)
            dG.append(g.to(torch.bfloat16))
            dW.append((0.02 * torch.randn(s.rows, s.cols, device="cuda", generator=gen)).to(torch.bfloat16))
        dM.append(torch.zeros(s.rows, s.cols, device="cuda"))
        dO.append(torch.empty(s.rows, s.cols, device="cuda") if k in checked else None)
    descs = [mm.tensor_desc(dW[k], dG[k], dM[k], update_out=dO[k]) for k in range(len(specs))]
    hp = mm.default_hparams()
    st = mm.MuonStep(descs, hp)
    st.step()
    torch.cuda.synchronize()
    assert st.flags() == 0
    st.close()
    worst = 0.0
    for k in checked:
        s = specs[k]
        ref = oracle_step(W[k], G[k], M[k], "bf16", hp)
        eO = rel_f(dO[k].cpu().numpy(), ref["O"])
        eM = rel_f(dM[k].cpu().numpy(), ref["M"])
        W1 = from_device(torch, dW[k], "bf16")
        err, bound, frac = check_w_bf16(W1, ref, float(hp.lr), ref["scale"])
        ulp, off = check_w_update_elementwise(W1, W[k], dO[k].cpu().numpy(), float(hp.lr),
                                              float(hp.weight_decay), ref["scale"])
        say(f"  {s.name} layer {s.layer} {s.rows}x{s.cols}: O {eO:.2e}  M {eM:.2e}  "
            f"W err/bound {err / bound:.2f} bitwise {frac:.1%}  fused update max {ulp:.2f} of bound")
        assert eO <= TOL_O["bf16"] and eM <= TOL_M and err <= bound and ulp <= 1.0
        worst = max(worst, eO)


def test_determinism_and_resume():
    say("case: determinism and resume")
    wl = adhoc("det", [(384, 640), (640, 384)], "bf16")
    hp = mm.default_hparams()

    def run(steps_a, steps_b):
        c = Case(wl, wl.tensors)
        st = mm.MuonStep(c.descs(), hp)
        for _ in range(steps_a):
            st.step()
        torch.cuda.synchronize()
        st.close()
        # save and reload the optimizer state (momentum) and weights
        saved = [(w.clone(), m.clone()) for w, m in zip(c.dW, c.dM)]
        for k, (w, m) in enumerate(saved):
            c.dW[k] = w
            c.dM[k] = m
        st = mm.MuonStep(c.descs(), hp)
        for _ in range(steps_b):
            st.step()
        torch.cuda.synchronize()
        st.close()
        return [from_device(torch, w, "bf16") for w in c.dW] + [m.cpu().numpy() for m in c.dM]

    a = run(3, 0)
    b = run(3, 0)
    r = run(2, 1)
    for x, y, z in zip(a, b, r):
        assert np.array_equal(x, y)
        assert np.array_equal(x, z)


def test_step_timed_reports_every_launch():
    wl = adhoc("timed", [(256, 512)], "bf16")
    c = Case(wl, wl.tensors)
    st = mm.MuonStep(c.descs(), mm.default_hparams())
    ph = st.step_timed()
    st.close()
    names = [n for n, _ in ph]
    assert names[0] == "momentum/bf16" and names[-1] == "bx/bf16#5" and len(names) == 16
    assert all(ms >= 0 for _, ms in ph)


def test_degenerate_handles_step_cleanly():
    """Handles with nothing for some phases: no tensors at all; only AdamW
    tensors (no Newton-Schulz group); a preconditioner slot that no tensor
    uses, refreshed anyway.  Each steps without error or flag, and leaves
    what it does not own untouched."""
    say("case: degenerate handles (empty, AdamW only, unused slot)")
    hp = mm.default_hparams()
    st = mm.MuonStep([], hp)
    st.step()
    torch.cuda.synchronize()
    assert st.flags() == 0
    st.close()

    w = torch.full((4, 6), 0.5, device="cuda")
    g = torch.full((4, 6), 0.25, device="cuda")
    m, v = torch.zeros_like(w), torch.zeros_like(w)
    st = mm.MuonStep([mm.adam_tensor_desc(w, g, m, v)], hp)
    st.step()
    torch.cuda.synchronize()
    assert st.flags() == 0 and bool(torch.isfinite(w).all()) and not bool((w == 0.5).all())
    st.close()

    p = B.MuonPrecond()
    p.d, p.nblocks = 64, 1
    W = torch.zeros(8, 16, device="cuda")
    G = torch.randn(8, 16, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    M = torch.zeros_like(W)
    st = mm.MuonStep([mm.tensor_desc(W, G, M)], hp, preconds=[p])
    acts = torch.randn(100, 64, device="cuda", generator=torch.Generator("cuda").manual_seed(6))
    st.precond_refresh(0, 0, acts, damping=1e-2)
    st.step()
    torch.cuda.synchronize()
    assert st.flags() == 0
    st.close()
    # the matrix ignored the slot: its momentum is the plain (1 - mu) G
    assert torch.allclose(M, (1.0 - hp.momentum) * G, rtol=1e-6, atol=0)

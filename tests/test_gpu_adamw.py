"""GPU parity of the AdamW part of the step (the parameters Muon does not
take: embeddings, heads, gains, biases) against the float64 oracle.

Each case runs several steps from the same seeded start on both sides.  The
oracle keeps its own state (float64 moments; the weight rounded to the
stored dtype after every step, which is what a bf16 or float32 parameter
is) and never sees a GPU value.

Bars: both moments rel_F <= 1e-6 at every step.  bf16 weights: within one
bf16 ulp per step taken (rounding-boundary differences can carry over) and
at most 2% of elements off at all.  float32 weights: per step taken, one
float32 ulp plus 1e-6 * lr (the float32 arithmetic of the update term, whose
size is about lr, shows against the ulp of small weights).
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_muon_amd as mm
from oracle import muon_oracle as orc
from tests.parity_common import (bf16_ulp_distance, from_device, oracle_step, rel_f, say, to_device)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_MOM = 1e-6


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([7000, *key])))


def _store(x, dtype):
    return orc.f64_to_bf16_bits(x) if dtype == "bf16" else np.asarray(x, np.float32)


def _decode(a, dtype):
    return orc.bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, np.float64)


class AdamCase:
    """AdamW tensors of several shapes, dtypes and layouts: a bias vector, a
    contiguous matrix, a 3-D tensor and a float32 matrix stored with a
    leading dimension larger than its width."""

    SPECS = [("bias", (768,), "bf16", None), ("embed", (300, 64), "bf16", None),
             ("gain3d", (4, 5, 6), "bf16", None), ("head32", (37, 50), "f32", 56)]

    def __init__(self):
        self.W, self.M, self.V, self.dW, self.dG, self.dM, self.dV, self.store = [], [], [], [], [], [], [], []
        for k, (name, shape, dtype, ld) in enumerate(self.SPECS):
            w = _store(_rng(k, 1).normal(0.0, 0.02, shape), dtype)
            self.W.append(w)
            self.M.append(np.zeros(shape))
            self.V.append(np.zeros(shape))
            if ld is None:
                self.dW.append(to_device(torch, w, dtype))
                self.dM.append(torch.zeros(shape, dtype=torch.float32, device="cuda"))
                self.dV.append(torch.zeros(shape, dtype=torch.float32, device="cuda"))
                self.dG.append(torch.empty_like(self.dW[-1]))
            else:   # row-major with leading dimension ld > cols: slices of wider buffers
                r, c = shape
                buf = lambda dt: torch.zeros(r, ld, dtype=dt, device="cuda")
                wb = buf(torch.float32)
                wb[:, :c] = torch.from_numpy(np.asarray(w, np.float32)).cuda()
                self.dW.append(wb[:, :c])
                self.dM.append(buf(torch.float32)[:, :c])
                self.dV.append(buf(torch.float32)[:, :c])
                self.dG.append(buf(torch.float32)[:, :c])

    def descs(self):
        return [mm.adam_tensor_desc(self.dW[k], self.dG[k], self.dM[k], self.dV[k]) for k in range(len(self.SPECS))]

    def set_grads(self, step):
        self.G = []
        for k, (name, shape, dtype, ld) in enumerate(self.SPECS):
            g = _store(_rng(k, 2, step).normal(0.0, 1e-2, shape) * (10.0 ** _rng(k, 3, step).uniform(-2, 2)), dtype)
            self.G.append(g)
            self.dG[k].copy_(to_device(torch, g, dtype))

    def oracle(self, t, hp):
        """Advance the oracle's own state by step t."""
        for k, (name, shape, dtype, ld) in enumerate(self.SPECS):
            W1, self.M[k], self.V[k] = orc.adamw_update(
                _decode(self.W[k], dtype), _decode(self.G[k], dtype), self.M[k], self.V[k], t,
                lr=float(np.float32(hp.adam_lr)), betas=(float(np.float32(hp.adam_beta1)),
                                                         float(np.float32(hp.adam_beta2))),
                eps=float(np.float32(hp.adam_eps)), weight_decay=float(np.float32(hp.adam_weight_decay)))
            self.W[k] = _store(W1, dtype)

    def compare(self, steps_taken, label, lr):
        for k, (name, shape, dtype, ld) in enumerate(self.SPECS):
            eM = rel_f(self.dM[k].cpu().numpy(), self.M[k])
            eV = rel_f(self.dV[k].cpu().numpy(), self.V[k])
            assert eM <= TOL_MOM and eV <= TOL_MOM, f"{label} {name}: moments rel_F {eM:.2e} {eV:.2e}"
            got = from_device(torch, self.dW[k].contiguous(), dtype)
            if dtype == "bf16":
                d = bf16_ulp_distance(got.reshape(-1), self.W[k].reshape(-1))
                assert d.max() <= steps_taken, f"{label} {name}: {d.max()} bf16 ulps off"
                assert (d > 0).mean() <= 0.02, f"{label} {name}: {(d > 0).mean():.1%} of elements off"
            else:
                ref = self.W[k].astype(np.float32)
                ulp = np.spacing(np.maximum(np.abs(ref), np.abs(got))).astype(np.float64)
                err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
                bound = steps_taken * (ulp + 1e-6 * lr)
                assert (err <= bound).all(), f"{label} {name}: float32 weight off by {(err / bound).max():.2f} x bound"
        say(f"  {label}: AdamW moments and weights match")


def test_adamw_three_steps_then_resume():
    say("case: AdamW tensors (vector, matrix, 3-D, strided float32), 3 steps, then resume at t = 4")
    hp = mm.default_hparams()
    c = AdamCase()
    st = mm.MuonStep(c.descs(), hp)
    for t in (1, 2, 3):
        c.set_grads(t)
        st.step()
        c.oracle(t, hp)
        c.compare(t, f"step {t}", hp.adam_lr)
    assert st.adam_step() == 3
    st.close()
    # a fresh handle over the same tensors resumes the count
    st2 = mm.MuonStep(c.descs(), hp)
    assert st2.adam_step() == 0
    st2.set_adam_step(3)
    c.set_grads(4)
    st2.step()
    c.oracle(4, hp)
    c.compare(4, "resumed step 4", hp.adam_lr)
    assert st2.adam_step() == 4
    assert st2.flags() == 0
    st2.close()


def test_adamw_beside_muon_and_nonfinite_flag():
    say("case: AdamW and Muon tensors in one step; a NaN AdamW gradient sets the flag")
    hp = mm.default_hparams()
    c = AdamCase()
    # one Muon matrix in the same handle
    rng = _rng(99, 1)
    Wm = orc.f64_to_bf16_bits(rng.normal(0.0, 0.02, (256, 512)))
    Gm = orc.f64_to_bf16_bits(rng.normal(0.0, 1e-2, (256, 512)))
    dWm, dGm = to_device(torch, Wm, "bf16"), to_device(torch, Gm, "bf16")
    dMm = torch.zeros(256, 512, dtype=torch.float32, device="cuda")
    dOm = torch.empty(256, 512, dtype=torch.float32, device="cuda")
    descs = c.descs() + [mm.tensor_desc(dWm, dGm, dMm, update_out=dOm)]
    st = mm.MuonStep(descs, hp)
    c.set_grads(1)
    st.step()
    c.oracle(1, hp)
    c.compare(1, "mixed step", hp.adam_lr)
    ref = oracle_step(Wm, Gm, np.zeros((256, 512)), "bf16", hp)
    assert rel_f(dOm.cpu().numpy(), ref["O"]) < 2e-2
    assert rel_f(dMm.cpu().numpy(), ref["M"]) <= TOL_MOM
    assert st.flags() == 0
    c.dG[0][5] = float("nan")
    st.step()
    assert st.flags(reset=True) & 1
    st.close()

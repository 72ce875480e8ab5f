"""Graph capture of the whole step.

One muon_step is captured into a HIP graph (stream capture, through
torch.cuda.CUDAGraph) on a handle whose plan splits its matrices into two
lanes and runs AdamW beside them, so the capture includes the fork onto the
handle's own streams and the join back.  The graph is replayed with new
gradients copied in before each replay, eager work and synchronisations in
between, and one ordinary (eager) step of the same handle among the replays;
after every step the weights, momenta and AdamW moments must equal, bit for
bit, those of a second handle stepped eagerly on the same inputs (the step is
deterministic: every reduction has a fixed order).  The first step is also
compared with the float64 oracle.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_muon_amd as mm
from tests.parity_common import from_device, oracle_step, rel_f, say, to_device
from oracle import muon_oracle as orc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SHAPES = [(256, 512)] * 8 + [(512, 256)] * 2 + [(384, 768)] * 2
ADAM_SHAPES = [(768,), (300, 64)]
STEPS = 4


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([8100, *key])))


class State:
    """One copy of every parameter and optimizer buffer, on the GPU."""

    def __init__(self):
        self.W, self.G, self.M, self.aW, self.aG, self.aM, self.aV = [], [], [], [], [], [], []
        for k, (r, c) in enumerate(SHAPES):
            self.W.append(to_device(torch, orc.f64_to_bf16_bits(_rng(k, 1).normal(0, 0.02, (r, c))), "bf16"))
            self.G.append(torch.empty(r, c, dtype=torch.bfloat16, device="cuda"))
            self.M.append(torch.zeros(r, c, dtype=torch.float32, device="cuda"))
        for k, shp in enumerate(ADAM_SHAPES):
            self.aW.append(to_device(torch, orc.f64_to_bf16_bits(_rng(50 + k, 1).normal(0, 0.02, shp)), "bf16"))
            self.aG.append(torch.empty(shp, dtype=torch.bfloat16, device="cuda"))
            self.aM.append(torch.zeros(shp, dtype=torch.float32, device="cuda"))
            self.aV.append(torch.zeros(shp, dtype=torch.float32, device="cuda"))

    def descs(self):
        d = [mm.tensor_desc(w, g, m) for w, g, m in zip(self.W, self.G, self.M)]
        return d + [mm.adam_tensor_desc(w, g, m, v) for w, g, m, v in zip(self.aW, self.aG, self.aM, self.aV)]

    def handle(self, hp):
        return mm.MuonStep(self.descs(), hp)

    def load_grads(self, grads):
        for dst, src in zip(self.G + self.aG, grads):
            dst.copy_(src)

    def snapshot(self):
        return [t.clone() for t in self.W + self.M + self.aW + self.aM + self.aV]


def _grads(step):
    out = []
    for k, shp in enumerate(SHAPES + ADAM_SHAPES):
        g = _rng(k, 2, step).normal(0, 1e-2, shp) * (10.0 ** _rng(k, 3, step).uniform(-1, 1))
        out.append(to_device(torch, orc.f64_to_bf16_bits(g), "bf16"))
    return out


def test_graph_capture_replays_match_eager():
    say("case: one step captured in a HIP graph (two lanes + AdamW stream), 4 steps vs eager")
    hp = mm.default_hparams()
    grads = [_grads(t) for t in range(STEPS)]
    # reference: eager steps
    ref = State()
    plan = mm.plan_describe(ref.descs(), hp)
    assert [g["lane"] for g in plan["groups"]] == [0, 1], "the case must exercise two lanes"
    W0 = [from_device(torch, w, "bf16") for w in ref.W]
    st_ref = ref.handle(hp)
    expect = []
    for t in range(STEPS):
        ref.load_grads(grads[t])
        st_ref.step()
        torch.cuda.synchronize()
        expect.append(ref.snapshot())
    assert st_ref.flags() == 0
    st_ref.close()

    # the first eager step against the oracle (first matrix, first AdamW tensor)
    o = oracle_step(W0[0], from_device(torch, grads[0][0], "bf16"), np.zeros(SHAPES[0]), "bf16", hp)
    assert rel_f(expect[0][len(SHAPES)].cpu().numpy(), o["M"]) <= 1e-6

    # captured step, replayed
    gs = State()
    st = gs.handle(hp)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        st.step()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for t in range(STEPS):
        gs.load_grads(grads[t])
        torch.cuda.synchronize()
        how = "eager" if t == 2 else "replay"
        if how == "eager":
            st.step()
        else:
            graph.replay()
        scratch.mul_(1.0001).add_(1.0)      # unrelated eager work between replays
        torch.cuda.synchronize()
        got = gs.snapshot()
        for k, (a, b) in enumerate(zip(got, expect[t])):
            assert torch.equal(a, b), f"step {t + 1} ({how}): buffer {k} differs from the eager run"
        say(f"  step {t + 1} ({how}): every buffer equals the eager run")
    assert st.adam_step() == STEPS
    assert st.flags() == 0
    del graph
    st.close()

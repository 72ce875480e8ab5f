"""The no-allocation entry point (muon_init_static: the workspace is the
library's static device array) against the ordinary one (muon_init with a
caller workspace), through the C ABI: two static inits in a row, the second
on a smaller request, each compared with the ordinary path on identical
inputs.  The kernels and the per-matrix arithmetic are the same, so every
output (new weights, momentum, orthogonalised update) must be bitwise equal.
The file is collected last: each static init zero-fills and takes over the
array that earlier calls in the process may have left behind."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_muon_amd as mm
from matrix_aware_optimizer_muon_amd import binding as B
import synth
from synth.workloads import TensorSpec, Workload
from tests.parity_common import say, to_device

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _inputs(shapes, dtypes, seed):
    specs = [TensorSpec(f"m{k}", 0, seed + k, r, c, dt, split_rows=sp)
             for k, ((r, c, sp), dt) in enumerate(zip(shapes, dtypes))]
    wl = Workload("tiny", specs, grad_law="gauss", grad_std=1.0, mom0_std=1e-2)
    return wl, [(synth.gradient(wl, s), synth.momentum0(wl, s), synth.weight(wl, s)) for s in specs]


def _run(wl, host, static):
    tens = []
    for s, (G, M, W) in zip(wl.tensors, host):
        tens.append((to_device(torch, W, s.dtype), to_device(torch, G, s.dtype), torch.from_numpy(M.copy()).cuda(),
                     torch.zeros(s.rows, s.cols, device="cuda")))
    # an AdamW vector beside the matrices (its state also lives in the workspace)
    aw = torch.linspace(-1, 1, 300, device="cuda")
    ag = torch.linspace(0.5, -0.5, 300, device="cuda")
    am, av = torch.zeros_like(aw), torch.zeros_like(aw)
    descs = [mm.tensor_desc(w, g, m, split_rows=s.split_rows, update_out=o) for s, (w, g, m, o) in zip(wl.tensors, tens)]
    descs.append(mm.adam_tensor_desc(aw, ag, am, av))
    hp = mm.default_hparams()
    before = torch.cuda.memory_allocated()
    st = mm.MuonStep(descs, hp, static_scratch=static)
    if static:
        assert st.workspace is None and torch.cuda.memory_allocated() == before
    for _ in range(2):
        st.step()
    torch.cuda.synchronize()
    flags = st.flags()
    return st, flags, [t.cpu() for ts in tens for t in ts] + [aw.cpu(), am.cpu(), av.cpu()]


def _compare(label, shapes, dtypes, seed):
    wl, host = _inputs(shapes, dtypes, seed)
    st_ref, f_ref, ref = _run(wl, host, static=False)
    st_ref.close()
    st, f, got = _run(wl, host, static=True)
    assert f == 0 and f_ref == 0
    for a, b in zip(ref, got):
        assert torch.equal(a, b), label
    say(f"  {label}: {len(shapes)} matrices + 1 AdamW vector, two steps, bitwise equal to muon_init "
        f"({st.workspace_bytes / 2**20:.1f} MiB of static scratch)")
    return st


def test_static_scratch_matches_caller_workspace_twice():
    say("case: muon_init_static vs muon_init, a larger then a smaller request")
    first = _compare("first", [(384, 640, 0), (640, 384, 0), (3 * 128, 128, 128), (96, 160, 0), (64, 200, 0)],
                     ["bf16", "bf16", "bf16", "bf16", "f32"], 6100)
    second = _compare("second (smaller)", [(256, 300, 0), (130, 129, 0)], ["bf16", "f32"], 6200)
    # the second static init took the array over: the first handle refuses to run
    with pytest.raises(B.MuonError):
        first.step()
    first.close()
    second.close()


def test_static_scratch_rejects_oversized_requests():
    big = torch.zeros(4096, 4096, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(4096, 4096, device="cuda")
    with pytest.raises(B.MuonError) as ei:
        mm.MuonStep([mm.tensor_desc(big, big.clone(), m)], mm.default_hparams(), static_scratch=True)
    assert "MUON_ERR_WORKSPACE_TOO_SMALL" in str(ei.value)

"""The bounds-checking debug build (lib/libmuon_debug.so, built with
MUON_DEBUG_BOUNDS=1): every GEMM and elementwise task checks its tile and K
extent against the unit's padded sizes and, instead of reading or writing
out of bounds, skips the tile and sets flag bit 2.  Over shapes that reach
every tile shape of the planner (float32 tiles, 128- and 256-tiles, the
128-strips past the last whole 256-tile, tall and wide units, the
stand-alone update) the debug build must set no flag and give results
bit-identical to the release build's: the checks add no arithmetic."""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import matrix_aware_optimizer_muon_amd as mm
from matrix_aware_optimizer_muon_amd import build as BLD
from tests.parity_common import say
from tests.test_gpu_parity import Case, adhoc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SHAPES = [(300, 520), (520, 300), (17, 33), (96, 160), (1000, 1100), (1100, 1000), (1600, 1700),
          (768, 3072), (3072, 768), (2100, 2300)]
BOUNDS_FLAG = 4


def _step(case, hp, library):
    st = mm.MuonStep(case.descs(), hp, library=library)
    st.step()
    torch.cuda.synchronize()
    flags = st.flags()
    st.close()
    return flags


@pytest.mark.parametrize("ns_steps", [5, 0])
def test_debug_build_sets_no_bounds_flag_and_matches_release(ns_steps):
    assert os.path.exists(BLD.DEBUG_LIB), "the debug library is built with the release one"
    say(f"case: debug bounds build against release, ns_steps={ns_steps}")
    wl = adhoc("dbg", SHAPES, "bf16")
    hp = mm.default_hparams(ns_steps=ns_steps)
    rel, dbg = Case(wl, wl.tensors), Case(wl, wl.tensors)     # identical seeded inputs
    assert _step(rel, hp, None) == 0
    flags = _step(dbg, hp, BLD.DEBUG_LIB)
    assert flags & BOUNDS_FLAG == 0, f"bounds check fired (flags {flags:#x})"
    assert flags == 0
    for k, s in enumerate(wl.tensors):
        for name in ("dW", "dM", "dO"):
            a, b = getattr(rel, name)[k], getattr(dbg, name)[k]
            assert torch.equal(a, b), f"{s.rows}x{s.cols} {name} differs between builds"

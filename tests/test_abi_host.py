"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function include/muon.h declares, validates arguments with the documented
status codes, and plans the workloads as designed.  Pointers here are fake
addresses that the library only compares and never dereferences."""

import ctypes
import math
import subprocess

import pytest

import matrix_aware_optimizer_muon_amd as mm
from matrix_aware_optimizer_muon_amd import binding as B
import synth

lib = pytest.importorskip("matrix_aware_optimizer_muon_amd.binding").load_library()

BASE = 1 << 36


def fake(rows, cols, dtype=B.MUON_BF16, base=BASE, split=0, precond=-1, ld=None, out=False):
    es = 4 if dtype == B.MUON_F32 else 2
    ld = ld or cols
    span = ((rows * ld * es + 4095) // 4096 + 1) * 4096
    mspan = ((rows * ld * 4 + 4095) // 4096 + 1) * 4096
    t = B.MuonTensor()
    t.param, t.grad, t.momentum = base, base + span, base + 2 * span
    t.rows, t.cols = rows, cols
    t.ld_param = t.ld_grad = t.ld_momentum = ld
    t.dtype, t.split_rows, t.precond, t.lr_mult = dtype, split, precond, 1.0
    t.update_out = base + 2 * span + mspan if out else None
    return t, 3 * span + 2 * mspan


def fakes(shapes, dtype=B.MUON_BF16):
    out, base = [], BASE
    for r, c in shapes:
        t, span = fake(r, c, dtype, base)
        out.append(t)
        base += span
    return out


def ws_status(tensors, hp=None, preconds=()):
    hp = hp or mm.default_hparams()
    ta, n = B._array(tensors, B.MuonTensor)
    pa, npc = B._array(list(preconds), B.MuonPrecond)
    out = ctypes.c_size_t(0)
    st = lib.muon_workspace_size(ta, n, pa, npc, ctypes.byref(hp), ctypes.byref(out))
    return B.STATUS_NAMES[st], out.value


def test_exports_every_declared_symbol():
    names = mm.header_functions()
    assert len(names) >= 10
    dyn = subprocess.run(["nm", "-D", "--defined-only", mm.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = {l.split()[-1] for l in dyn.splitlines() if l.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def test_default_hparams_are_the_pages_values():
    hp = mm.default_hparams()
    assert math.isclose(hp.lr, 0.02, rel_tol=1e-7)
    assert math.isclose(hp.momentum, 0.95, rel_tol=1e-7)
    assert math.isclose(hp.weight_decay, 0.01, rel_tol=1e-7)
    assert hp.nesterov == 1 and hp.ns_steps == 5
    assert (hp.ns_a, hp.ns_b, hp.ns_c) == tuple(float(ctypes.c_float(x).value) for x in (3.4445, -4.7750, 2.0315))
    assert hp.scale_mode == B.SCALE_ORIGINAL and hp.momentum_form == B.MOM_EMA


def test_status_strings():
    for code, name in B.STATUS_NAMES.items():
        assert lib.muon_status_str(code).decode() == name


def test_validation_errors():
    ok = fakes([(64, 128)])
    assert ws_status(ok)[0] == "MUON_OK"
    # empty list is a valid no-op
    assert ws_status([])[0] == "MUON_OK"
    t = fakes([(64, 128)])[0]; t.rows = 0
    assert ws_status([t])[0] == "MUON_ERR_BAD_SHAPE"
    t = fakes([(64, 128)])[0]; t.ld_grad = 100
    assert ws_status([t])[0] == "MUON_ERR_BAD_SHAPE"
    t = fakes([(64, 128)])[0]; t.dtype = 7
    assert ws_status([t])[0] == "MUON_ERR_BAD_DTYPE"
    t = fakes([(64, 128)])[0]; t.param = BASE + 1
    assert ws_status([t])[0] == "MUON_ERR_ALIGNMENT"
    t = fakes([(64, 128)])[0]; t.momentum = t.momentum + 2
    assert ws_status([t])[0] == "MUON_ERR_ALIGNMENT"
    t = fakes([(64, 128)])[0]; t.grad = None
    assert ws_status([t])[0] == "MUON_ERR_NULL_ARG"
    t = fakes([(96, 128)])[0]; t.split_rows = 40
    assert ws_status([t])[0] == "MUON_ERR_BAD_SHAPE"
    t = fakes([(64, 128)])[0]; t.grad = t.param + 64
    assert ws_status([t])[0] == "MUON_ERR_ALIASING"
    a, b = fakes([(64, 128), (64, 128)])
    b.momentum = a.momentum + 128
    assert ws_status([a, b])[0] == "MUON_ERR_ALIASING"
    t = fakes([(64, 128)])[0]; t.precond = 0
    assert ws_status([t])[0] == "MUON_ERR_BAD_ARG"          # no such slot
    t = fakes([(64, 128)])[0]; t.lr_mult = float("nan")
    assert ws_status([t])[0] == "MUON_ERR_BAD_ARG"
    hp = mm.default_hparams(ns_steps=65)
    assert ws_status(ok, hp)[0] == "MUON_ERR_BAD_ARG"
    hp = mm.default_hparams(scale_mode=9)
    assert ws_status(ok, hp)[0] == "MUON_ERR_BAD_ARG"
    hp = mm.default_hparams(momentum_form=5)
    assert ws_status(ok, hp)[0] == "MUON_ERR_BAD_ARG"
    # the square phase computes c (A A + (b/c) A): c = 0 is refused unless no
    # iteration runs
    assert ws_status(ok, mm.default_hparams(ns_c=0.0))[0] == "MUON_ERR_BAD_ARG"
    assert "ns_c" in lib.muon_last_error().decode()
    assert ws_status(ok, mm.default_hparams(ns_c=0.0, ns_steps=0))[0] == "MUON_OK"
    # the message names the offending tensor
    t = fakes([(64, 128)])[0]; t.ld_param = 3
    ws_status([t])
    assert "tensor 0" in lib.muon_last_error().decode()


def test_init_rejects_bad_workspace_without_touching_the_gpu():
    ts = fakes([(64, 128)])
    ta, n = B._array(ts, B.MuonTensor)
    pa, npc = B._array([], B.MuonPrecond)
    hp = mm.default_hparams()
    need = ws_status(ts)[1]
    h = ctypes.c_void_p()
    st = lib.muon_init(ctypes.byref(h), ta, n, pa, npc, ctypes.byref(hp), ctypes.c_void_p(1 << 40), need - 1, None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_WORKSPACE_TOO_SMALL"
    st = lib.muon_init(ctypes.byref(h), ta, n, pa, npc, ctypes.byref(hp), ctypes.c_void_p((1 << 40) + 16), need, None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_ALIGNMENT"
    st = lib.muon_init(ctypes.byref(h), ta, n, pa, npc, ctypes.byref(hp), None, need, None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_NULL_ARG"
    st = lib.muon_init(ctypes.byref(h), ta, n, pa, npc, ctypes.byref(hp), ctypes.c_void_p(ts[0].param), need, None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_ALIASING"
    assert B.STATUS_NAMES[lib.muon_step(None, 0.02, None)] == "MUON_ERR_NULL_ARG"


def test_init_static_rejects_oversized_requests_without_touching_the_gpu():
    # the static scratch holds 64 MiB: a 4096 x 4096 bf16 matrix needs more
    # (two bf16 X buffers, the int8 corrections, A and B: 160 MiB), and the
    # call fails before any GPU call; invalid requests fail as for muon_init
    pa, npc = B._array([], B.MuonPrecond)
    hp = mm.default_hparams()
    h = ctypes.c_void_p()
    big = fakes([(4096, 4096)])
    assert ws_status(big)[1] > 64 << 20
    ta, n = B._array(big, B.MuonTensor)
    st = lib.muon_init_static(ctypes.byref(h), ta, n, pa, npc, ctypes.byref(hp), None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_WORKSPACE_TOO_SMALL" and not h.value
    assert b"static scratch" in lib.muon_last_error()
    bad = fakes([(64, 128)])
    bad[0].ld_param = 100
    ta, n = B._array(bad, B.MuonTensor)
    st = lib.muon_init_static(ctypes.byref(h), ta, n, pa, npc, ctypes.byref(hp), None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_BAD_SHAPE"
    st = lib.muon_init_static(None, ta, n, pa, npc, ctypes.byref(hp), None)
    assert B.STATUS_NAMES[st] == "MUON_ERR_NULL_ARG"


def _workload_fakes(name, layers=None):
    w = synth.workload(name, layers)
    ts, base = [], BASE
    for s in w.tensors:
        dt = B.MUON_F32 if s.dtype == "f32" else B.MUON_BF16
        t, span = fake(s.rows, s.cols, dt, base, split=s.split_rows)
        ts.append(t)
        base += span
    return ts


def test_plan_gpt2_small():
    plan = mm.plan_describe(_workload_fakes("gpt2s"), mm.default_hparams())
    units = plan["units"]
    assert len(units) == 72
    assert all(u["m"] == 768 for u in units)
    right = [u for u in units if u["side"] == "right"]
    assert len(right) == 12 and all((u["rows"], u["cols"], u["n"]) == (3072, 768, 3072) for u in right)
    assert sum(u["n"] == 3072 for u in units) == 24
    assert all(abs(u["lr_scale"] - (2.0 if u["side"] == "right" else 1.0)) < 1e-7 for u in units)
    # two lanes (run on two streams) of equal Newton-Schulz work: 12 MLP and
    # 24 attention matrices each
    g0, g1 = plan["groups"]
    assert (g0["lane"], g1["lane"]) == (0, 1) and g0["units"] == g1["units"] == 36
    # m = 768: 128 x 128 Gram tiles, 256 x 256 square and B X tiles (768 and
    # 3072 are multiples of 256, so no extra padding)
    assert all(u["tiles"] == [128, 256, 256] and u["mp"] == 768 for u in units)
    for k, total in (("gram", 72 * 21), ("square", 72 * 6), ("bx", 48 * 9 + 24 * 36),
                     ("momentum", 12 * (4 * 72 + 2 * 288))):
        assert g0[f"{k}_tiles"] + g1[f"{k}_tiles"] == total
    assert g0["tiles_by_edge"] == {"256": [0, g0["square_tiles"], g0["bx_tiles"]],
                                   "128": [g0["gram_tiles"], 0, 0]}
    assert g0["bx_tiles"] == g1["bx_tiles"]
    # the XCD interleave pads the shorter per-XCD sequences with empty blocks
    # (the Gram's tiles differ 4x in cost, so its sequences differ in length)
    for g in (g0, g1):
        assert g["bx_blocks"] <= g["bx_tiles"] * 1.05 + 8
        for k in ("gram", "square"):
            assert g[f"{k}_tiles"] <= g[f"{k}_blocks"] <= g[f"{k}_tiles"] * 1.4 + 8
    order = plan["launch_order"]
    assert order[0] == "momentum/bf16" and order[-1] == "bx/bf16x256" and len(order) == 32
    assert order[1:4] == ["gram/bf16", "square/bf16x256", "bx/bf16x256"]


def test_plan_gpt2_xl_and_padding():
    plan = mm.plan_describe(_workload_fakes("gpt2xl", layers=2), mm.default_hparams())
    units = plan["units"]
    # 1600 = 6 x 256 + 64: units padded to 1664 only; the Gram and B X cover
    # 1536 x 1536 (1536 x 6400) with 256-tiles and the rest with 128-tiles,
    # the square stays at 128
    assert all(u["m"] == 1600 and u["mp"] == 1664 and u["tiles"] == [256, 128, 256] for u in units)
    assert {u["np"] for u in units} == {1664, 6400}
    assert sum(u["side"] == "right" for u in units) == 2
    # the full 48-layer set has far more B X tiles per phase than two lanes
    # help with: one group on one stream
    full = mm.plan_describe(_workload_fakes("gpt2xl"), mm.default_hparams())
    assert [g["lane"] for g in full["groups"]] == [0] and full["groups"][0]["units"] == 288


def test_plan_large_units_take_256_tiles():
    # Tile shape per phase: the Gram at 256 from m = 1536, the square where m
    # is a multiple of 256 (from 768) or from 2048, B X from 768.  Units are
    # padded to 128; a 256-tile phase covers the largest multiple of 256 and
    # the remaining 128-strips with 128-tiles.  One group holding both shapes
    # runs two launches per phase, the 256 one first.
    ts = fakes([(4096, 4096), (2100, 3000), (1024, 4096), (1000, 1100), (640, 2048)])
    plan = mm.plan_describe(ts, mm.default_hparams())
    u = plan["units"]
    assert [(x["tiles"], x["mp"], x["np"]) for x in u] == [
        ([256] * 3, 4096, 4096), ([256] * 3, 2176, 3072), ([128, 256, 256], 1024, 4096),
        ([128, 128, 256], 1024, 1152), ([128] * 3, 640, 2048)]
    g = plan["groups"][0]
    sym = lambda k: k * (k + 1) // 2          # upper tiles of a k x k tile grid
    # 2100 x 3000: 256-tiles over 2048 x 3072, then the 128-row strip 2048..2175
    # (17 upper tiles in its column for the square products, 24 in its row for B X);
    # 1000 x 1100 B X: 256-tiles over 1024 x 1024, the 128-column strip 1024..1151
    assert g["tiles_by_edge"]["256"] == [sym(16) + sym(8), sym(16) + sym(8) + sym(4), 16 * 16 + 8 * 12 + 4 * 16 + 4 * 4]
    assert g["tiles_by_edge"]["128"] == [17 + sym(8) + sym(8) + sym(5), 17 + sym(8) + sym(5), 24 + 8 + 5 * 16]
    assert plan["launch_order"][1:7] == ["gram/bf16x256", "gram/bf16", "square/bf16x256", "square/bf16",
                                          "bx/bf16x256", "bx/bf16"]


def test_plan_split_rows_and_fp32():
    t = fakes([(3 * 128, 128)])[0]
    t.split_rows = 128   # three 128 x 128 units (a QKV-style row split)
    f = fake(256, 512, B.MUON_F32, base=BASE + (1 << 30))[0]
    small = fake(17, 33, B.MUON_BF16, base=BASE + (1 << 31))[0]
    plan = mm.plan_describe([t, f, small], mm.default_hparams())
    u = plan["units"]
    assert [x["row0"] for x in u[:3]] == [0, 128, 256]
    assert all(x["lr_scale"] == 1.0 and x["side"] == "left" and x["ns"] == "bf16" for x in u[:3])
    assert u[3]["ns"] == "f32" and u[3]["mp"] == 256 and u[3]["np"] == 512
    # a bf16 matrix with a short side below 128 runs its iteration in float32
    assert u[4]["ns"] == "f32" and (u[4]["mp"], u[4]["np"]) == (64, 64)
    assert [g["ns"] for g in plan["groups"]] == ["bf16", "f32"]
    assert [g["units"] for g in plan["groups"]] == [3, 2]
    assert [g["lane"] for g in plan["groups"]] == [0, 1]
    assert len(plan["launch_order"]) == 32
    p0 = mm.plan_describe([t], mm.default_hparams(ns_steps=0))
    assert p0["launch_order"] == ["momentum/bf16", "update/bf16"]


def test_plan_small_phases_take_128_tiles():
    # A group's phase with fewer 256-tiles than CUs whose 128-tiles fit in
    # one round of the 512 block slots takes 128-tiles: the Newton-Muon
    # layer's six 768-row units (36 square and 108 B X 256-tiles) run on
    # 128-tiles in every phase; GPT-2-small's lanes (216 square 256-tiles
    # each, 756 as 128-tiles) and the 4096^2 matrix (136 / 544) keep 256
    plan = mm.plan_describe(_workload_fakes("nmuon"), mm.default_hparams())
    assert all(u["tiles"] == [128] * 3 for u in plan["units"] if u["ns"] == "bf16")
    assert plan["groups"][0]["tiles_by_edge"] == {"128": [6 * 21, 6 * 21, 4 * 36 + 2 * 144]}
    assert all(u["tiles"] == [128, 256, 256] for u in mm.plan_describe(_workload_fakes("gpt2s"),
                                                                       mm.default_hparams())["units"])
    assert mm.plan_describe(fakes([(4096, 4096)]), mm.default_hparams())["units"][0]["tiles"] == [256] * 3


def test_plan_tiles_cover_every_output_exactly_once():
    """The planner checks its own GEMM task lists on every plan (every
    128 x 128 block of a unit's B X output covered exactly once, every block
    on or above the diagonal of its Gram and square exactly once) and fails
    the plan otherwise; so planning many seeded random shapes -- ragged,
    tall and wide, both precisions, row splits, the 256-tile thresholds and
    the strips past the last whole 256-tile -- must succeed, with the tile
    counts of each plan consistent with its units."""
    import random
    rng = random.Random(7)
    sizes = [1, 7, 64, 127, 128, 129, 255, 256, 300, 640, 767, 768, 769, 1000, 1024, 1100, 1535, 1536,
             1600, 2047, 2048, 2100, 2304, 3000, 4096]
    for case in range(60):
        shapes, base, ts = [], BASE, []
        for _ in range(rng.randint(1, 4)):
            r, c = rng.choice(sizes), rng.choice(sizes)
            dt = B.MUON_F32 if rng.random() < 0.25 else B.MUON_BF16
            split = 0
            if r % 2 == 0 and r >= 256 and rng.random() < 0.3:
                split = r // 2
            t, span = fake(r, c, dt, base, split=split)
            ts.append(t)
            base += span
            shapes.append((r, c, dt, split))
        plan = mm.plan_describe(ts, mm.default_hparams())
        assert len(plan["units"]) == sum(2 if s else 1 for _, _, _, s in shapes), (case, shapes)
        for g in plan["groups"]:
            for k in ("gram", "square", "bx"):
                assert g[f"{k}_tiles"] == sum(v[("gram", "square", "bx").index(k)]
                                              for v in g["tiles_by_edge"].values()), (case, shapes)


def test_workspace_size_formula():
    # bf16 unit: two X hi buffers (m_p x n_p bf16 each), the int8 master
    # corrections (m_p x n_p bytes) + A, B (m_p^2 bf16)
    ts = fakes([(768, 3072)])
    need = ws_status(ts)[1]
    plan = mm.plan_describe(ts, mm.default_hparams())
    per_unit = 2 * 768 * 3072 * 2 + 768 * 3072 + 2 * 768 * 768 * 2
    assert need - plan["meta_bytes"] == per_unit
    # ns_steps does not change the footprint
    assert ws_status(ts, mm.default_hparams(ns_steps=1))[1] == need


def test_plan_newton_muon_layer():
    w = synth.workload("nmuon")
    ts, base = [], BASE
    for s in w.tensors:
        t, span = fake(s.rows, s.cols, B.MUON_BF16, base, split=s.split_rows, precond=s.precond)
        ts.append(t)
        base += span
    pcs = []
    for d, nb in ((768, 1), (768, 4)):
        p = B.MuonPrecond()
        p.d, p.nblocks = d, nb
        pcs.append(p)
    plan = mm.plan_describe(ts, mm.default_hparams(), pcs)
    assert [{k: pc[k] for k in ("d", "nblocks", "dp")} for pc in plan["preconds"]] == \
        [{"d": 768, "nblocks": 1, "dp": 768}, {"d": 768, "nblocks": 4, "dp": 768}]
    # the slots' S and S^-1 lie inside the workspace, apart, 256-byte aligned
    spans = []
    for pc in plan["preconds"]:
        blk = pc["dp"] * pc["dp"] * pc["nblocks"]
        spans += [(pc["s_offset"], pc["s_offset"] + 4 * blk), (pc["sinv_offset"], pc["sinv_offset"] + 6 * blk)]
    spans.sort()
    assert all(a % 256 == 0 for a, _ in spans) and spans[-1][1] <= plan["workspace_bytes"]
    assert all(spans[i][1] <= spans[i + 1][0] for i in range(len(spans) - 1))
    # tiles of P, 128 rows x 64 columns: QKV 2304, O 768, up 3072 rows against one
    # 768-wide S^-1 (12 column tiles); down 768 rows against four
    assert plan["apply_tiles"] == (18 + 6 + 24) * 12 + 4 * 6 * 12
    assert plan["launch_order"][0] == "precond_apply"
    assert len(plan["units"]) == 3 + 1 + 1 + 1          # packed QKV split into three blocks
    # a preconditioned tensor must match d * nblocks of its slot
    bad = ts[3]
    bad.precond = 0
    assert ws_status([bad], preconds=pcs)[0] == "MUON_ERR_BAD_SHAPE"


def test_filter_tensors_become_matrices():
    # a (out, in, kh, kw) convolution filter is described as out x (in*kh*kw)
    torch = pytest.importorskip("torch")
    w = torch.zeros(8, 4, 3, 3, dtype=torch.bfloat16)
    g = torch.zeros_like(w)
    m = torch.zeros(8, 4, 3, 3, dtype=torch.float32)
    d = mm.tensor_desc(w, g, m)
    assert (d.rows, d.cols, d.ld_param, d.ld_momentum) == (8, 36, 36, 36)
    # a filter whose trailing dimensions are not contiguous is refused
    wt = w.permute(0, 2, 3, 1)
    with pytest.raises(ValueError):
        mm.tensor_desc(wt, wt, m.permute(0, 2, 3, 1))
    with pytest.raises(ValueError):
        mm.tensor_desc(w[:, :, 0, 0].reshape(-1), g[:, :, 0, 0].reshape(-1), m[:, :, 0, 0].reshape(-1))
    # the conv workload plans one float32 group (m = 64) and one bf16 group (m = 256)
    wl = synth.workload("conv")
    ts = fakes([(s.rows, s.cols) for s in wl.tensors])
    plan = mm.plan_describe(ts, mm.default_hparams())
    assert sorted(u["m"] for u in plan["units"]) == [64, 64, 256, 256, 256, 256]
    assert [g["units"] for g in plan["groups"]] == [4, 2]
    # two single-lane groups of different precision take lanes 0 and 1 (their
    # launch-bound chains run side by side on two streams)
    assert [g["lane"] for g in plan["groups"]] == [0, 1]


def fake_adam(rows, cols, base, dtype=B.MUON_BF16, ld=None):
    """An AdamW descriptor with fake pointers: param, grad, exp_avg, exp_avg_sq
    laid out one after the other from `base`; returns (desc, bytes used)."""
    t, span = fake(rows, cols, dtype, base, ld=ld)
    mspan = ((rows * (ld or cols) * 4 + 4095) // 4096 + 1) * 4096
    t.kind = B.KIND_ADAMW
    t.exp_avg_sq = base + span
    return t, span + mspan


def test_adamw_descriptors_validate_and_plan():
    muon = fakes([(64, 128), (128, 64)])
    base = BASE + (1 << 32)
    vec, n1 = fake_adam(1, 768, base)
    mat, n2 = fake_adam(100, 50, base + n1, dtype=B.MUON_F32)           # contiguous: one flat row
    strided, n3 = fake_adam(10, 30, base + n1 + n2, ld=40)               # ld > cols: ten rows
    ts = muon + [vec, mat, strided]
    assert ws_status(ts)[0] == "MUON_OK"
    plan = mm.plan_describe(ts, mm.default_hparams())
    assert plan["adamw_tensors"] == 3
    assert plan["adamw_tasks"] == 1 + 3 + 10        # 768 / 2048, 5000 / 2048, 10 rows of 30
    assert plan["launch_order"][:3] == ["adam_tick", "adamw", "momentum/f32"]   # m = 64: float32 NS
    assert len(plan["units"]) == 2                   # AdamW tensors are not orthogonalised
    # AdamW-only requests are valid
    assert mm.plan_describe([vec], mm.default_hparams())["launch_order"] == ["adam_tick", "adamw"]
    # descriptor errors
    t, _ = fake_adam(4, 8, base); t.exp_avg_sq = None
    assert ws_status([t])[0] == "MUON_ERR_NULL_ARG"
    t, _ = fake_adam(4, 8, base); t.split_rows = 2
    assert ws_status([t])[0] == "MUON_ERR_BAD_ARG"
    t, _ = fake_adam(4, 8, base); t.kind = 3
    assert ws_status([t])[0] == "MUON_ERR_BAD_ARG"
    t = fakes([(64, 128)])[0]; t.exp_avg_sq = base
    assert ws_status([t])[0] == "MUON_ERR_BAD_ARG"       # only AdamW tensors carry a second moment
    t, _ = fake_adam(4, 8, base); t.exp_avg_sq = t.momentum + 16
    assert ws_status([t])[0] == "MUON_ERR_ALIASING"
    for bad in (dict(adam_beta1=1.0), dict(adam_beta2=-0.1), dict(adam_eps=-1.0), dict(adam_lr=float("inf"))):
        assert ws_status([vec], mm.default_hparams(**bad))[0] == "MUON_ERR_BAD_ARG"


def test_adam_default_hparams_are_the_pages_values():
    hp = mm.default_hparams()
    assert math.isclose(hp.adam_lr, 3e-4, rel_tol=1e-6)
    assert math.isclose(hp.adam_beta1, 0.9, rel_tol=1e-6) and math.isclose(hp.adam_beta2, 0.95, rel_tol=1e-6)
    assert math.isclose(hp.adam_weight_decay, 0.01, rel_tol=1e-6)
    assert math.isclose(hp.adam_eps, 1e-8, rel_tol=1e-6)


def test_precond_calls_reject_a_null_handle():
    # argument checks that need no GPU: a NULL handle is refused up front
    assert B.STATUS_NAMES[lib.muon_precond_accumulate(None, 0, 0, None, 1, 1, 1, ctypes.c_float(1.0), None)] == \
        "MUON_ERR_NULL_ARG"
    assert B.STATUS_NAMES[lib.muon_precond_refresh_accumulated(None, 0, 0, ctypes.c_float(1e-4), 1, None)] == \
        "MUON_ERR_NULL_ARG"
    assert B.STATUS_NAMES[lib.muon_set_adam_step(None, 1, None)] == "MUON_ERR_NULL_ARG"

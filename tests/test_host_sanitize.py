"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  `muon_host.cpp` (validation, planning, XCD ordering, the
workspace carve-up and the plan's JSON) is compiled with its host code
instrumented, together with stub kernel launchers and a small driver
(`tests/host_sanitize/`), into an executable.  The driver runs the pure-host
entry points over every synthetic workload, ragged, split, float32, strided,
AdamW, preconditioned and invalid requests; it must finish without a
sanitizer report, and its statuses, workspace sizes and plans must equal the
shipped library's.  Pointers are fake addresses the planner only compares."""

import ctypes
import json
import os
import shutil
import struct
import subprocess

import pytest

import matrix_aware_optimizer_muon_amd as mm
from matrix_aware_optimizer_muon_amd import binding as B
from matrix_aware_optimizer_muon_amd import build as BLD
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# sanitizers on the host side only (the device pass of a HIP compile takes none)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
BASE = 1 << 36

lib = B.load_library()


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-4000:]}"
    return r


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("needs hipcc")
    d = tmp_path_factory.mktemp("sanitize")
    common = [f"--offload-arch={BLD.ARCH}", "-O1", "-g", "-fPIC", "-std=c++17",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              f"-I{BLD.INCLUDE}", f"-I{BLD.CSRC}"]
    objs = []
    for src, lang in ((os.path.join(BLD.CSRC, "muon_host.cpp"), "hip"),
                      (os.path.join(HERE, "host_sanitize", "launch_stubs.cpp"), "hip"),
                      (os.path.join(HERE, "host_sanitize", "driver.cpp"), "c++")):
        obj = str(d / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        _run([HIPCC, *common, "-x", lang, *SAN, "-c", src, "-o", obj])
        objs.append(obj)
    # the planner's own object is instrumented: it calls the sanitizers'
    # checks (undefined symbols their runtimes provide)
    nm = _run(["nm", "-u", objs[0]]).stdout
    assert "__asan_report_load" in nm and "__ubsan_handle_" in nm
    exe = str(d / "planner_san")
    _run([HIPCC, f"--offload-arch={BLD.ARCH}", *SAN, *objs, *BLD.LINK_FLAGS, "-o", exe])
    return exe


def fake(rows, cols, base, dtype=B.MUON_BF16, split=0, precond=-1, ld=None, out=False, adam=False):
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
    if adam:
        t.kind = B.KIND_ADAMW
        t.exp_avg_sq = base + 2 * span + 2 * mspan
    return t, 3 * span + 3 * mspan


def workload_request(name):
    w = synth.workload(name)
    ts, base = [], BASE
    for s in w.tensors:
        dt = B.MUON_F32 if s.dtype == "f32" else B.MUON_BF16
        t, span = fake(s.rows, s.cols, base, dt, split=s.split_rows, precond=s.precond,
                       adam=s.kind == "adamw")
        ts.append(t)
        base += span
    pcs = []
    if name == "nmuon":
        for d, nb in ((768, 1), (768, 4)):
            p = B.MuonPrecond()
            p.d, p.nblocks = d, nb
            pcs.append(p)
    return ts, pcs, mm.default_hparams()


def shapes_request(shapes, hp=None, **kw):
    ts, base = [], BASE
    for r, c in shapes:
        t, span = fake(r, c, base, **kw)
        ts.append(t)
        base += span
    return ts, [], hp or mm.default_hparams()


def requests():
    out = [(f"workload {n}", workload_request(n)) for n in synth.WORKLOADS]
    ragged = [(300, 520), (520, 300), (17, 33), (33, 17), (1, 7), (7, 1), (1, 1), (257, 1000),
              (1000, 257), (64, 64), (129, 129), (128, 200), (200, 128), (2100, 2300), (2300, 2100),
              (4096, 128), (128, 4096)]
    out.append(("ragged bf16", shapes_request(ragged)))
    out.append(("ragged f32", shapes_request(ragged, dtype=B.MUON_F32)))
    out.append(("strided", shapes_request([(300, 520), (129, 129), (64, 200)], ld=523)))
    out.append(("update_out", shapes_request([(300, 520), (520, 300)], out=True)))
    ts, pcs, hp = shapes_request([(3 * 96, 96), (4 * 128, 256)])
    ts[0].split_rows, ts[1].split_rows = 96, 128
    out.append(("split rows", (ts, pcs, hp)))
    out.append(("no iterations", shapes_request([(300, 520)], hp=mm.default_hparams(ns_steps=0))))
    out.append(("empty", ([], [], mm.default_hparams())))
    # invalid requests: the planner must refuse them cleanly
    bad = shapes_request([(64, 128), (64, 128)])
    bad[0][1].momentum = bad[0][0].momentum + 128
    out.append(("aliasing", bad))
    bad = shapes_request([(64, 128)])
    bad[0][0].ld_param = 100
    out.append(("ld < cols", bad))
    bad = shapes_request([(96, 128)])
    bad[0][0].split_rows = 64
    out.append(("split does not divide", bad))
    bad = shapes_request([(64, 128)])
    bad[0][0].precond = 3
    out.append(("no such slot", bad))
    out.append(("ns_c = 0", shapes_request([(64, 128)], hp=mm.default_hparams(ns_c=0.0))))
    out.append(("too many steps", shapes_request([(64, 128)], hp=mm.default_hparams(ns_steps=65))))
    return out


def _serialise(ts, pcs, hp):
    ta = (B.MuonTensor * len(ts))(*ts)
    pa = (B.MuonPrecond * len(pcs))(*pcs)
    return struct.pack("<ii", len(ts), len(pcs)) + bytes(ta) + bytes(pa) + bytes(hp)


def _library_result(ts, pcs, hp):
    ta, n = B._array(ts, B.MuonTensor)
    pa, npc = B._array(pcs, B.MuonPrecond)
    nbytes = ctypes.c_size_t(0)
    st = B.STATUS_NAMES[lib.muon_workspace_size(ta, n, pa, npc, ctypes.byref(hp), ctypes.byref(nbytes))]
    plan = mm.plan_describe(ts, hp, pcs) if st == "MUON_OK" else None
    return st, nbytes.value, plan


def test_planner_under_address_and_undefined_behaviour_sanitizers(driver, tmp_path):
    reqs = requests()
    path = tmp_path / "requests.bin"
    path.write_bytes(b"".join(_serialise(*r) for _, r in reqs))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver, str(path)], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-6000:]
    lines = r.stdout.splitlines()
    got, i = [], 0
    while i < len(lines):
        head = lines[i].split()
        assert head[0] == "request", lines[i]
        st, nbytes = head[3], int(head[5])
        nxt = lines[i + 1]
        plan = json.loads(nxt[len("plan "):]) if nxt.startswith("plan ") else None
        got.append((st, nbytes, plan))
        i += 2
    assert len(got) == len(reqs)
    refused = 0
    for (label, req), (st, nbytes, plan) in zip(reqs, got):
        ref = _library_result(*req)
        assert (st, nbytes) == ref[:2], label
        assert plan == ref[2], label
        refused += st != "MUON_OK"
    assert refused == 6

"""ctypes binding of libmuon.so (include/muon.h).  Argument marshalling only:
every step of the Muon update runs in the library's HIP kernels.

The library is loaded from this package's lib/ directory.  If it is missing
or cannot be loaded, every entry point raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import json
import os
import re
from typing import List, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libmuon.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "muon.h")

MUON_OK = 0
STATUS_NAMES = {
    0: "MUON_OK", 1: "MUON_ERR_NULL_ARG", 2: "MUON_ERR_BAD_SHAPE", 3: "MUON_ERR_BAD_DTYPE",
    4: "MUON_ERR_ALIGNMENT", 5: "MUON_ERR_ALIASING", 6: "MUON_ERR_WORKSPACE_TOO_SMALL",
    7: "MUON_ERR_UNSUPPORTED", 8: "MUON_ERR_HIP", 9: "MUON_ERR_BAD_ARG",
}
MUON_F32, MUON_BF16 = 0, 1
SCALE_NONE, SCALE_ORIGINAL, SCALE_MATCH_RMS_ADAMW, SCALE_SPECTRAL = 0, 1, 2, 3
MOM_EMA, MOM_SGD = 0, 1
KIND_MUON, KIND_ADAMW = 0, 1


class MuonTensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("ld_param", ctypes.c_int64), ("ld_grad", ctypes.c_int64), ("ld_momentum", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("split_rows", ctypes.c_int32), ("precond", ctypes.c_int32),
        ("lr_mult", ctypes.c_float), ("update_out", ctypes.c_void_p),
        ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32), ("exp_avg_sq", ctypes.c_void_p),
    ]


class MuonPrecond(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("nblocks", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class MuonHparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("momentum", ctypes.c_float), ("weight_decay", ctypes.c_float),
        ("eps", ctypes.c_float), ("nesterov", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
        ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
        ("scale_mode", ctypes.c_int32), ("momentum_form", ctypes.c_int32),
        ("adam_lr", ctypes.c_float), ("adam_beta1", ctypes.c_float), ("adam_beta2", ctypes.c_float),
        ("adam_eps", ctypes.c_float), ("adam_weight_decay", ctypes.c_float),
    ]


class MuonError(RuntimeError):
    def __init__(self, status, detail=""):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmuon.so (this package's build, or the file named by the
    MUON_LIBRARY environment variable) and declare its signatures.  Raises if
    it is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("MUON_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libmuon.so not built: {p} is missing (run __graft_entry__.build())")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7.  If
    # torch is importable, load it first so the library's libamdhip64.so.7
    # dependency resolves to the runtime that owns torch's memory and streams.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    PT = ctypes.POINTER(MuonTensor)
    PP = ctypes.POINTER(MuonPrecond)
    PH = ctypes.POINTER(MuonHparams)
    sigs = {
        "muon_default_hparams": (None, [PH]),
        "muon_workspace_size": (i32, [PT, i32, PP, i32, PH, ctypes.POINTER(sz)]),
        "muon_init": (i32, [ctypes.POINTER(vp), PT, i32, PP, i32, PH, vp, sz, vp]),
        "muon_init_static": (i32, [ctypes.POINTER(vp), PT, i32, PP, i32, PH, vp]),
        "muon_precond_refresh": (i32, [vp, i32, i32, vp, i64, i64, i32, f32, vp]),
        "muon_precond_accumulate": (i32, [vp, i32, i32, vp, i64, i64, i32, f32, vp]),
        "muon_precond_refresh_accumulated": (i32, [vp, i32, i32, f32, i32, vp]),
        "muon_step": (i32, [vp, f32, vp]),
        "muon_step_timed": (i32, [vp, f32, vp, ctypes.POINTER(f32), i32, ctypes.POINTER(i32)]),
        "muon_phase_name": (ctypes.c_char_p, [vp, i32]),
        "muon_get_flags": (i32, [vp, vp, i32, ctypes.POINTER(ctypes.c_uint32)]),
        "muon_set_adam_step": (i32, [vp, i64, vp]),
        "muon_get_adam_step": (i32, [vp, vp, ctypes.POINTER(i64)]),
        "muon_destroy": (i32, [vp]),
        "muon_plan_describe": (i32, [PT, i32, PP, i32, PH, ctypes.c_char_p, sz, ctypes.POINTER(sz)]),
        "muon_status_str": (ctypes.c_char_p, [i32]),
        "muon_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def header_functions() -> List[str]:
    """Names of the functions declared in include/muon.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


def _check(status, lib=None):
    if status != MUON_OK:
        lib = lib or load_library()
        raise MuonError(status, lib.muon_last_error().decode())


def default_hparams(**overrides) -> MuonHparams:
    hp = MuonHparams()
    load_library().muon_default_hparams(ctypes.byref(hp))
    for k, v in overrides.items():
        if not hasattr(hp, k):
            raise KeyError(k)
        setattr(hp, k, v)
    return hp


def _array(items, cls):
    n = len(items)
    arr = (cls * max(n, 1))()
    for i, it in enumerate(items):
        arr[i] = it
    return arr, n


def workspace_size(tensors: Sequence[MuonTensor], hp: MuonHparams,
                   preconds: Sequence[MuonPrecond] = (), lib: Optional[ctypes.CDLL] = None) -> int:
    """Workspace bytes a handle over these tensors needs (with `lib`, as
    that build of the library plans them)."""
    lib = lib or load_library()
    ta, n = _array(tensors, MuonTensor)
    pa, npc = _array(preconds, MuonPrecond)
    out = ctypes.c_size_t(0)
    _check(lib.muon_workspace_size(ta, n, pa, npc, ctypes.byref(hp), ctypes.byref(out)))
    return out.value


def plan_describe(tensors: Sequence[MuonTensor], hp: MuonHparams,
                  preconds: Sequence[MuonPrecond] = ()) -> dict:
    lib = load_library()
    ta, n = _array(tensors, MuonTensor)
    pa, npc = _array(preconds, MuonPrecond)
    need = ctypes.c_size_t(0)
    _check(lib.muon_plan_describe(ta, n, pa, npc, ctypes.byref(hp), None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check(lib.muon_plan_describe(ta, n, pa, npc, ctypes.byref(hp), buf, need.value, ctypes.byref(need)))
    return json.loads(buf.value.decode())


def status_of(fn_result) -> str:
    return STATUS_NAMES.get(fn_result, str(fn_result))


# ---------------------------------------------------------------------------
# torch-facing wrapper (torch supplies device memory and the stream)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _as_matrix(t):
    """A >= 2-D tensor as the row-major matrix (shape[0], prod(shape[1:])):
    a convolution filter (out, in, kh, kw) becomes out x (in*kh*kw), the 2-D
    view Muon orthogonalises.  The trailing dimensions must be contiguous."""
    if t.dim() == 2:
        return t
    if t.dim() < 2:
        raise ValueError("Muon tensors must have at least 2 dimensions")
    inner = t[0].numel() if t.shape[0] > 0 else 0
    if not t[0].is_contiguous() or (t.shape[0] > 1 and t.stride(0) < inner):
        raise ValueError("the trailing dimensions of a filter must be contiguous")
    return t.as_strided((t.shape[0], inner), (t.stride(0), 1))


def tensor_desc(param, grad, momentum, *, split_rows=0, precond=-1, lr_mult=1.0,
                update_out=None) -> MuonTensor:
    torch = _torch()
    if grad.shape != param.shape or momentum.shape != param.shape:
        raise ValueError("param, grad and momentum must share one shape")
    param, grad, momentum = _as_matrix(param), _as_matrix(grad), _as_matrix(momentum)
    if update_out is not None:
        update_out = _as_matrix(update_out)
    for t in (param, grad, momentum):
        if t.stride(1) != 1:
            raise ValueError("tensors must be row-major (unit column stride)")
    if param.dtype != grad.dtype:
        raise ValueError("param and grad must share a dtype")
    if momentum.dtype != torch.float32:
        raise ValueError("momentum must be float32")
    dt = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}.get(param.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {param.dtype}")
    d = MuonTensor()
    d.param, d.grad, d.momentum = param.data_ptr(), grad.data_ptr(), momentum.data_ptr()
    d.rows, d.cols = param.shape
    d.ld_param, d.ld_grad, d.ld_momentum = param.stride(0), grad.stride(0), momentum.stride(0)
    d.dtype, d.split_rows, d.precond, d.lr_mult = dt, split_rows, precond, lr_mult
    if update_out is not None:
        if update_out.dtype != torch.float32 or not update_out.is_contiguous() or update_out.shape != param.shape:
            raise ValueError("update_out must be a contiguous float32 tensor of the param's shape")
        d.update_out = update_out.data_ptr()
    else:
        d.update_out = None
    return d


def adam_tensor_desc(param, grad, exp_avg, exp_avg_sq, *, lr_mult=1.0) -> MuonTensor:
    """A parameter stepped with AdamW (embedding, head, gain, bias): any
    shape, viewed as rows x cols (a vector as 1 x n, a >= 2-D tensor as
    shape[0] x rest); exp_avg and exp_avg_sq are its float32 moments."""
    torch = _torch()
    if not (grad.shape == param.shape == exp_avg.shape == exp_avg_sq.shape):
        raise ValueError("param, grad and both moments must share one shape")
    if exp_avg.stride() != exp_avg_sq.stride():
        raise ValueError("the two moments must share one layout")
    if param.dim() == 1:
        param, grad, exp_avg, exp_avg_sq = (t.view(1, -1) if t.is_contiguous() else t.unsqueeze(0)
                                            for t in (param, grad, exp_avg, exp_avg_sq))
    else:
        param, grad, exp_avg, exp_avg_sq = (_as_matrix(t) for t in (param, grad, exp_avg, exp_avg_sq))
    for t in (param, grad, exp_avg, exp_avg_sq):
        if t.stride(1) != 1:
            raise ValueError("tensors must be row-major (unit column stride)")
    if param.dtype != grad.dtype:
        raise ValueError("param and grad must share a dtype")
    if exp_avg.dtype != torch.float32 or exp_avg_sq.dtype != torch.float32:
        raise ValueError("the moments must be float32")
    dt = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}.get(param.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {param.dtype}")
    d = MuonTensor()
    d.param, d.grad, d.momentum = param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr()
    d.exp_avg_sq = exp_avg_sq.data_ptr()
    d.rows, d.cols = param.shape
    d.ld_param, d.ld_grad, d.ld_momentum = param.stride(0), grad.stride(0), exp_avg.stride(0)
    d.dtype, d.split_rows, d.precond, d.lr_mult = dt, 0, -1, lr_mult
    d.kind = KIND_ADAMW
    d.update_out = None
    return d


class MuonStep:
    """One handle over a list of (param, grad, momentum) device tensors.

    The workspace is a torch uint8 tensor owned by this object; the tensors
    registered must stay alive and unmoved while the object is used.
    """

    def __init__(self, descs: Sequence[MuonTensor], hp: Optional[MuonHparams] = None,
                 preconds: Sequence[MuonPrecond] = (), device=None, keepalive=(), static_scratch=False,
                 library: Optional[str] = None):
        """static_scratch=True binds the handle to the library's static
        device scratch (muon_init_static): no workspace is allocated, the
        request must fit in it, and a later static handle on the same GPU
        supersedes this one.  `library`: path of another build of the
        library to run this handle on (e.g. the bounds-checking debug build,
        build.DEBUG_LIB); default the one load_library() returns."""
        torch = _torch()
        self._lib = load_library(library)
        self.hp = hp if hp is not None else default_hparams()
        self._descs, self._n = _array(list(descs), MuonTensor)
        self._pcs, self._npc = _array(list(preconds), MuonPrecond)
        self.workspace_bytes = workspace_size(descs, self.hp, preconds, lib=self._lib)
        self.device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        self._keep = list(keepalive)
        h = ctypes.c_void_p()
        if static_scratch:
            self.workspace = None
            with torch.cuda.device(self.device):
                self._check(self._lib.muon_init_static(ctypes.byref(h), self._descs, self._n, self._pcs, self._npc,
                                                  ctypes.byref(self.hp), self._stream(None)))
        else:
            self.workspace = torch.empty(max(self.workspace_bytes, 256), dtype=torch.uint8, device=self.device)
            self._check(self._lib.muon_init(ctypes.byref(h), self._descs, self._n, self._pcs, self._npc,
                                       ctypes.byref(self.hp), ctypes.c_void_p(self.workspace.data_ptr()),
                                       self.workspace.numel(), self._stream(None)))
        self._h = h

    def _torch_stream(self, stream):
        torch = _torch()
        return stream if stream is not None else torch.cuda.current_stream(self.device)

    def _stream(self, stream):
        return ctypes.c_void_p(self._torch_stream(stream).cuda_stream)

    @staticmethod
    def _guard(acts, stream):
        """The activations are read asynchronously on `stream`.  Instead of
        holding a reference (which would pin every micro-batch until a
        synchronising call), tell torch's caching allocator that `stream`
        uses the memory: once the caller drops the tensor, its block is not
        handed out again before the work queued on `stream` so far is done."""
        acts.record_stream(stream)

    def plan(self) -> dict:
        """The plan of this handle (muon_plan_describe of its tensors)."""
        descs = [self._descs[i] for i in range(self._n)]
        pcs = [self._pcs[i] for i in range(self._npc)]
        return plan_describe(descs, self.hp, pcs)

    def _check(self, status):
        """Raise on a non-zero status with the error text of this handle's own library."""
        _check(status, self._lib)

    def step(self, lr: float = -1.0, stream=None):
        self._check(self._lib.muon_step(self._h, ctypes.c_float(lr), self._stream(stream)))

    def step_timed(self, lr: float = -1.0, stream=None):
        """Run one step with HIP events between launches; returns
        [(phase_name, ms), ...] (synchronises the stream)."""
        cap = 4096
        ms = (ctypes.c_float * cap)()
        n = ctypes.c_int32(0)
        self._check(self._lib.muon_step_timed(self._h, ctypes.c_float(lr), self._stream(stream), ms, cap,
                                         ctypes.byref(n)))
        return [(self._lib.muon_phase_name(self._h, i).decode(), ms[i]) for i in range(min(n.value, cap))]

    def precond_refresh(self, slot: int, block: int, acts, damping: float = 1e-4, stream=None):
        torch = _torch()
        if acts.dim() != 2 or acts.stride(1) != 1:
            raise ValueError("activations must be 2-D row-major")
        dt = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}.get(acts.dtype)
        if dt is None:
            raise ValueError(f"unsupported activation dtype {acts.dtype}")
        s = self._torch_stream(stream)
        self._check(self._lib.muon_precond_refresh(self._h, slot, block, ctypes.c_void_p(acts.data_ptr()),
                                              acts.shape[0], acts.stride(0), dt, ctypes.c_float(damping),
                                              ctypes.c_void_p(s.cuda_stream)))
        self._guard(acts, s)

    def precond_accumulate(self, slot: int, block: int, acts, beta: float = 1.0, stream=None):
        """Add one micro-batch of layer-input activations to the running
        second moment of (slot, block): Sigma <- beta Sigma + X^T X."""
        torch = _torch()
        if acts.dim() != 2 or acts.stride(1) != 1:
            raise ValueError("activations must be 2-D row-major")
        dt = {torch.float32: MUON_F32, torch.bfloat16: MUON_BF16}.get(acts.dtype)
        if dt is None:
            raise ValueError(f"unsupported activation dtype {acts.dtype}")
        s = self._torch_stream(stream)
        self._check(self._lib.muon_precond_accumulate(self._h, slot, block, ctypes.c_void_p(acts.data_ptr()),
                                                 acts.shape[0], acts.stride(0), dt, ctypes.c_float(beta),
                                                 ctypes.c_void_p(s.cuda_stream)))
        self._guard(acts, s)

    def precond_refresh_accumulated(self, slot: int, block: int, damping: float = 1e-4, reset: bool = True,
                                    stream=None):
        """Rebuild S^-1 of (slot, block) from its running second moment."""
        self._check(self._lib.muon_precond_refresh_accumulated(self._h, slot, block, ctypes.c_float(damping),
                                                          int(reset), self._stream(stream)))

    def set_adam_step(self, steps_taken: int, stream=None):
        """Resume the AdamW step count (steps already taken)."""
        self._check(self._lib.muon_set_adam_step(self._h, int(steps_taken), self._stream(stream)))

    def adam_step(self, stream=None) -> int:
        """AdamW steps taken so far (synchronises the stream)."""
        v = ctypes.c_int64(0)
        self._check(self._lib.muon_get_adam_step(self._h, self._stream(stream), ctypes.byref(v)))
        return v.value

    def flags(self, reset: bool = False, stream=None) -> int:
        v = ctypes.c_uint32(0)
        self._check(self._lib.muon_get_flags(self._h, self._stream(stream), int(reset), ctypes.byref(v)))
        return v.value

    def close(self):
        if getattr(self, "_h", None):
            self._check(self._lib.muon_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

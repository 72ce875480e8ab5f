"""Host-only checks of the Python binding's argument marshalling (no GPU):
asynchronous calls that read caller activations keep no reference to them
(the memory is guarded through the caching allocator's stream tracking
instead), so repeated micro-batch calls do not pin device memory."""

import ctypes

import pytest

torch = pytest.importorskip("torch")

from matrix_aware_optimizer_muon_amd import binding as B


class _FakeLib:
    """Stands in for libmuon.so: records the calls, returns MUON_OK."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return B.MUON_OK
        return fn


class _FakeStream:
    cuda_stream = 0


class _FakeActs:
    """A 2-D bf16 device tensor as far as the binding looks at it."""

    def __init__(self, recorded):
        self.dtype = torch.bfloat16
        self.shape = (256, 64)
        self._recorded = recorded

    def dim(self):
        return 2

    def stride(self, i=None):
        return (64, 1) if i is None else (64, 1)[i]

    def data_ptr(self):
        return 1 << 40

    def record_stream(self, s):
        self._recorded.append(s)


def _step_object():
    st = object.__new__(B.MuonStep)
    st._lib = _FakeLib()
    st._h = ctypes.c_void_p(1)
    st._keep = []
    st.device = torch.device("cpu")
    return st


def test_activation_calls_keep_no_reference():
    st = _step_object()
    recorded = []
    s = _FakeStream()
    for _ in range(1000):
        st.precond_accumulate(0, 0, _FakeActs(recorded), beta=1.0, stream=s)
        st.precond_refresh(0, 0, _FakeActs(recorded), damping=1e-4, stream=s)
    assert st._lib.calls.count("muon_precond_accumulate") == 1000
    assert st._lib.calls.count("muon_precond_refresh") == 1000
    assert len(st._keep) == 0
    # every call told the allocator which stream reads the activations
    assert len(recorded) == 2000 and all(r is s for r in recorded)
    st._h = None

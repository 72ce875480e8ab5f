"""MI355X-native Muon optimizer step: a C-ABI library (libmuon.so, HIP for
gfx950) and its thin ctypes binding.  See include/muon.h for the ABI."""

from matrix_aware_optimizer_muon_amd.binding import (  # noqa: F401
    LIB_PATH, MuonError, MuonHparams, MuonPrecond, MuonStep, MuonTensor,
    adam_tensor_desc, default_hparams, header_functions, load_library, plan_describe,
    tensor_desc, workspace_size,
)

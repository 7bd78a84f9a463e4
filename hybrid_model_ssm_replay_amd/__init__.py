"""ReplaySSM decode path for AMD Instinct MI355X: Python binding of libreplayssm.so.

The compute lives in the HIP library (``csrc/``, C ABI in ``include/replayssm.h``).
This package only marshals arguments: ``binding`` mirrors the C calls one for one
(``replay_init``, ``replay_step``, ``replay_flush``, ``replay_verify``,
``replay_commit`` and the baselines), and ``layer.ReplayLayer`` allocates the
device buffers with PyTorch and passes their addresses and the current stream.

Importing the package does not load the library; the first call does, and it
raises if ``libreplayssm.so`` has not been built -- there is no fallback path.
"""
from .binding import (KIND_GDN, KIND_MAMBA2, FMT_F32, FMT_F16_SR, FMT_F8E4M3, FMT_F4E2M1_B16, FMT_F4E2M1_CS,
                      STATUS_ACCEPT_CLAMPED, STATUS_BAD_POINTERS, ReplayError, lib_path, load_library)

__all__ = ["KIND_GDN", "KIND_MAMBA2", "FMT_F32", "FMT_F16_SR", "FMT_F8E4M3", "FMT_F4E2M1_B16", "FMT_F4E2M1_CS",
           "STATUS_ACCEPT_CLAMPED", "STATUS_BAD_POINTERS", "ReplayError", "lib_path", "load_library"]

"""ctypes mirror of include/replayssm.h.  Argument marshalling only.

Every function here takes plain integers (device addresses, sizes, a
hipStream_t handle) and calls the C function of the same name; a negative
return code raises ``ReplayError``.
"""
from __future__ import annotations

import ctypes
import os

KIND_MAMBA2, KIND_GDN = 0, 1
FMT_F32, FMT_F16_SR, FMT_F8E4M3, FMT_F4E2M1_B16, FMT_F4E2M1_CS = 0, 1, 2, 3, 4
STATUS_ACCEPT_CLAMPED, STATUS_BAD_POINTERS = 0x1, 0x2
FLAG_DECAY_SKIP = 0x1
FLAG_BF16_RECORDS = 0x2
FLAG_RECORDS_IN_RING = 0x4
OK, EINVAL, EHIP, ENOTSUP = 0, -1, -2, -3

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libreplayssm.so")


class ReplayError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {code} ({_strerror(code)})")
        self.code = code


class replay_config(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("state_dim", ctypes.c_int32),
                ("window", ctypes.c_int32), ("max_draft", ctypes.c_int32), ("ckpt_fmt", ctypes.c_int32),
                ("read_fmt", ctypes.c_int32), ("seed", ctypes.c_uint64), ("flags", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class replay_buffers(ctypes.Structure):
    _fields_ = [("ckpt", ctypes.c_void_p), ("read_copy", ctypes.c_void_p), ("ring", ctypes.c_void_p),
                ("pointers", ctypes.c_void_p), ("status", ctypes.c_void_p), ("A", ctypes.c_void_p),
                ("D", ctypes.c_void_p)]


class replay_record(ctypes.Structure):
    _fields_ = [("f0", ctypes.c_void_p), ("f1", ctypes.c_void_p), ("f2", ctypes.c_void_p),
                ("f3", ctypes.c_void_p), ("f4", ctypes.c_void_p)]


class replay_ring_view(ctypes.Structure):
    _fields_ = [("f", ctypes.c_void_p * 5), ("slots", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class replay_ctx(ctypes.Structure):
    _fields_ = [("cfg", replay_config), ("buf", replay_buffers), ("parity", ctypes.c_int32),
                ("t_pending", ctypes.c_int32), ("magic", ctypes.c_uint32), ("reserved", ctypes.c_int32)]


_lib = None

_P = ctypes.c_void_p
_SIG = {
    "replay_validate_config": (ctypes.c_int, [ctypes.POINTER(replay_config)]),
    "replay_ckpt_bytes": (ctypes.c_size_t, [ctypes.POINTER(replay_config)]),
    "replay_read_copy_bytes": (ctypes.c_size_t, [ctypes.POINTER(replay_config)]),
    "replay_ring_bytes": (ctypes.c_size_t, [ctypes.POINTER(replay_config)]),
    "replay_pointer_words": (ctypes.c_size_t, [ctypes.POINTER(replay_config)]),
    "replay_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "replay_abi_sizeof": (ctypes.c_size_t, [ctypes.c_int]),
    "replay_init": (ctypes.c_int, [ctypes.POINTER(replay_ctx), ctypes.POINTER(replay_config),
                                   ctypes.POINTER(replay_buffers), _P]),
    "replay_set_state": (ctypes.c_int, [ctypes.POINTER(replay_ctx), _P, _P]),
    "replay_step": (ctypes.c_int, [ctypes.POINTER(replay_ctx), ctypes.POINTER(replay_record), _P, _P]),
    "replay_flush": (ctypes.c_int, [ctypes.POINTER(replay_ctx), _P, _P]),
    "replay_verify": (ctypes.c_int, [ctypes.POINTER(replay_ctx), ctypes.c_int32, ctypes.POINTER(replay_record),
                                     _P, _P]),
    "replay_commit": (ctypes.c_int, [ctypes.POINTER(replay_ctx), _P, _P]),
    "replay_current_pointers": (ctypes.c_int, [ctypes.POINTER(replay_ctx), ctypes.POINTER(ctypes.c_void_p),
                                               ctypes.POINTER(ctypes.c_void_p)]),
    "replay_ring_fields": (ctypes.c_int, [ctypes.POINTER(replay_ctx), ctypes.POINTER(replay_ring_view)]),
    "replay_record_slots": (ctypes.c_int, [ctypes.POINTER(replay_ctx), _P, _P]),
    "replay_conv_step": (ctypes.c_int, [ctypes.POINTER(replay_config), _P, _P, _P, ctypes.POINTER(replay_record),
                                        _P, _P]),
    "replay_snapshot_verify": (ctypes.c_int, [ctypes.POINTER(replay_config), _P, _P, ctypes.c_int32, _P, _P,
                                              ctypes.POINTER(replay_record), _P, _P]),
    "replay_snapshot_commit": (ctypes.c_int, [ctypes.POINTER(replay_config), _P, _P, ctypes.c_int32, _P]),
    "replay_hbm_probe": (ctypes.c_int, [_P, _P, ctypes.c_size_t, ctypes.c_int, _P]),
}
EXPORTS = tuple(_SIG)


def load_library(path: str | None = None):
    """Load libreplayssm.so (once) and check that the struct sizes agree."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or lib_path()
    # The library must bind to the HIP runtime that PyTorch (which owns the
    # device memory and streams) has loaded; load torch first if it is present.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -m hybrid_model_ssm_replay_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIG.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    for i, st in enumerate((replay_config, replay_buffers, replay_record, replay_ctx)):
        if lib.replay_abi_sizeof(i) != ctypes.sizeof(st):
            raise ImportError(f"ABI mismatch for {st.__name__}: C {lib.replay_abi_sizeof(i)} "
                              f"vs ctypes {ctypes.sizeof(st)}")
    _lib = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load_library().replay_strerror(code).decode()
    except Exception:
        return "?"


def _check(fn: str, rc: int) -> None:
    if rc != OK:
        raise ReplayError(fn, rc)


def make_config(kind, batch, heads, groups, head_dim, state_dim, window, max_draft=0,
                ckpt_fmt=FMT_F32, read_fmt=FMT_F32, seed=0, flags=0) -> replay_config:
    return replay_config(kind, batch, heads, groups, head_dim, state_dim, window, max_draft, ckpt_fmt,
                         read_fmt, seed, flags, 0)


def make_record(*fields) -> replay_record:
    vals = list(fields) + [0] * (5 - len(fields))
    return replay_record(*[ctypes.c_void_p(v or None) for v in vals])


# ---- one wrapper per C call -------------------------------------------------
def replay_validate_config(cfg: replay_config) -> int:
    return load_library().replay_validate_config(ctypes.byref(cfg))


def replay_ckpt_bytes(cfg) -> int:
    return load_library().replay_ckpt_bytes(ctypes.byref(cfg))


def replay_read_copy_bytes(cfg) -> int:
    return load_library().replay_read_copy_bytes(ctypes.byref(cfg))


def replay_ring_bytes(cfg) -> int:
    return load_library().replay_ring_bytes(ctypes.byref(cfg))


def replay_pointer_words(cfg) -> int:
    return load_library().replay_pointer_words(ctypes.byref(cfg))


def replay_init(ctx: replay_ctx, cfg: replay_config, buf: replay_buffers, stream: int) -> None:
    _check("replay_init", load_library().replay_init(ctypes.byref(ctx), ctypes.byref(cfg), ctypes.byref(buf),
                                                     stream or None))


def replay_set_state(ctx, state: int, stream: int) -> None:
    _check("replay_set_state", load_library().replay_set_state(ctypes.byref(ctx), state, stream or None))


def replay_step(ctx, rec: replay_record, y: int, stream: int) -> None:
    _check("replay_step", load_library().replay_step(ctypes.byref(ctx), ctypes.byref(rec), y, stream or None))


def replay_flush(ctx, seq_mask: int, stream: int) -> None:
    _check("replay_flush", load_library().replay_flush(ctypes.byref(ctx), seq_mask or None, stream or None))


def replay_verify(ctx, T: int, drafts: replay_record, y: int, stream: int) -> None:
    _check("replay_verify", load_library().replay_verify(ctypes.byref(ctx), T, ctypes.byref(drafts), y,
                                                         stream or None))


def replay_commit(ctx, accepted: int, stream: int) -> None:
    _check("replay_commit", load_library().replay_commit(ctypes.byref(ctx), accepted, stream or None))


def replay_current_pointers(ctx) -> tuple[int, int]:
    pos, ck = ctypes.c_void_p(), ctypes.c_void_p()
    _check("replay_current_pointers",
           load_library().replay_current_pointers(ctypes.byref(ctx), ctypes.byref(pos), ctypes.byref(ck)))
    return pos.value, ck.value


def replay_ring_fields(ctx) -> replay_ring_view:
    view = replay_ring_view()
    _check("replay_ring_fields", load_library().replay_ring_fields(ctypes.byref(ctx), ctypes.byref(view)))
    return view


def replay_record_slots(ctx, slots: int, stream: int) -> None:
    _check("replay_record_slots", load_library().replay_record_slots(ctypes.byref(ctx), slots, stream))


def replay_conv_step(cfg, state: int, A: int, D: int, rec: replay_record, y: int, stream: int) -> None:
    _check("replay_conv_step", load_library().replay_conv_step(ctypes.byref(cfg), state, A or None, D or None,
                                                               ctypes.byref(rec), y, stream or None))


def replay_snapshot_verify(cfg, slots: int, cur: int, T: int, A: int, D: int, drafts: replay_record, y: int,
                           stream: int) -> None:
    _check("replay_snapshot_verify",
           load_library().replay_snapshot_verify(ctypes.byref(cfg), slots, cur, T, A or None, D or None,
                                                 ctypes.byref(drafts), y, stream or None))


def replay_snapshot_commit(cfg, cur: int, accepted: int, T: int, stream: int) -> None:
    _check("replay_snapshot_commit",
           load_library().replay_snapshot_commit(ctypes.byref(cfg), cur, accepted, T, stream or None))


def replay_hbm_probe(src: int, dst: int, nbytes: int, mode: int, stream: int) -> None:
    _check("replay_hbm_probe", load_library().replay_hbm_probe(src, dst, nbytes, mode, stream or None))

"""ctypes loader for ``libsd_amd.so`` and the raw C-ABI signatures.

This module only marshals arguments; every step of the computation runs in
the HIP kernels behind ``include/sd.h``.  Importing it never falls back to
anything: if the library has not been built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# SD_LIB_PATH selects another build of the same library (the host-sanitized
# one of the checking build); there is no fallback of any kind.
LIB_PATH = os.environ.get("SD_LIB_PATH") or os.path.join(PKG, "libsd_amd.so")

SD_OK = 0
STATUS_NAMES = {0: "SD_OK", 1: "SD_ERR_NULL", 2: "SD_ERR_SHAPE",
                3: "SD_ERR_WORKSPACE", 4: "SD_ERR_LAUNCH", 5: "SD_ERR_DEVICE",
                6: "SD_ERR_SCRATCH"}

_vp, _i32, _i64, _sz, _f32, _u64 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float, C.c_uint64

SIGNATURES = {
    "sd_status_str": (C.c_char_p, [_i32]),
    "sd_version": (C.c_char_p, []),
    "sd_probe_read": (_i32, [_vp, _sz, _vp, _vp]),
    "sd_probe_mfma_flops": (_i64, [_i32]),
    "sd_probe_mfma": (_i32, [_i32, _vp, _vp]),
    "sd_draft_attn_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i64, _i32]),
    "sd_draft_attn": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                             _i64, _i32, _f32, _i32, _i32, _vp, _vp, _i32,
                             _vp, _vp, _sz, _vp]),
    "sd_draft_attn_noalloc_max_scratch": (_sz, []),
    "sd_draft_attn_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                     _i64, _i32, _f32, _i32, _i32, _vp, _vp, _i32,
                                     _vp, _vp]),
    "sd_summary_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "sd_summary_update": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]),
    "sd_schedule_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "sd_schedule_draft": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sd_schedule_verify": (_i32, [_vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp,
                                  _i32, _i32, _i32, _i32, _i32, _i32,
                                  _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sd_lm_head_workspace_size": (_sz, [_i32, _i32]),
    "sd_lm_head_probs": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _u64,
                                _vp, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sd_markov_workspace_size": (_sz, [_i32, _i32, _i32]),
    "sd_markov_sample": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _i32, _vp, _i32, _i32, _i32,
                                _i32, _i32, _vp, _u64, _vp, _sz, _vp]),
    "sd_log_prior_bias": (_i32, [_vp, _i32, C.c_double, _f32, _vp, _vp]),
    "sd_verify_workspace_size": (_sz, [_i32, _i32, _i32, _i32]),
    "sd_verify": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                         _vp, _i32, _i32, _vp, _u64, _vp, _vp, _vp, _vp, _sz, _vp]),
}

_LIB = None


class SdError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the built library (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m block_drafting_sd_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != SD_OK:
        msg = load().sd_status_str(status).decode()
        raise SdError(fn, status, msg)

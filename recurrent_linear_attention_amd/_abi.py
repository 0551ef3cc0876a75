"""ctypes mirror of ``include/kda.h``: structs, prototypes and the loaded library.

Marshalling only. Every computation runs in ``lib/libkda.so``; if it is missing this module
raises at import -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_size_t, c_uint32, c_void_p

# torch must load its HIP runtime before libkda.so does: both carry the soname
# libamdhip64.so.7, so libkda.so then binds to torch's copy and the process holds a single
# HIP/HSA runtime (two runtimes in one process do not share devices, streams or memory).
import torch  # noqa: F401

# KDA_LIB_PATH names another build of the same library (the tests load a host-only build under
# the address and undefined-behaviour sanitizers through it).
LIB_PATH = os.environ.get("KDA_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libkda.so")

KDA_OK, KDA_EINVAL, KDA_ENOSLOT, KDA_ESTATE, KDA_EUNSUPPORTED, KDA_EWORKSPACE, KDA_EHIP = \
    0, -1, -2, -3, -4, -5, -6
KDA_DEVERR_NACC_RANGE = 1
KDA_DEVERR_SLOT_RANGE = 2
KDA_DEVERR_DECAY_RANGE = 4


class kda_pool_desc(ctypes.Structure):
    _fields_ = [("num_slots", c_int32), ("num_heads", c_int32), ("dk", c_int32),
                ("dv", c_int32), ("ring_cap", c_int32)]


class kda_slot_meta(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_int64), ("ring_head", c_int32), ("pending", c_int32),
                ("v_base", c_int32), ("v_npos", c_int32)]


class kda_prefill_args(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("a", c_void_p),
                ("b", c_void_p), ("o", c_void_p),
                ("n_seq", c_int32), ("n_tok", c_int32), ("chunk", c_int32),
                ("ckpt_interval", c_int32),
                ("h_cu_seqlens", c_void_p), ("d_cu_seqlens", c_void_p),
                ("h_init_slot", c_void_p), ("d_init_slot", c_void_p),
                ("h_out_slot", c_void_p), ("d_out_slot", c_void_p),
                ("h_ckpt_slot", c_void_p), ("d_ckpt_slot", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


class kda_step_args(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("a", c_void_p),
                ("b", c_void_p), ("o", c_void_p), ("B", c_int32),
                ("h_slots", c_void_p), ("d_slots", c_void_p)]


class kda_mixed_args(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("a", c_void_p),
                ("b", c_void_p), ("o", c_void_p), ("prefill", kda_prefill_args),
                ("n_decode", c_int32), ("h_decode_slots", c_void_p),
                ("d_decode_slots", c_void_p), ("n_verify", c_int32), ("n_pos", c_int32),
                ("h_verify_slots", c_void_p), ("d_verify_slots", c_void_p),
                ("n_commit", c_int32), ("h_commit_slots", c_void_p), ("d_commit_slots", c_void_p),
                ("d_n_accepted", c_void_p), ("side_stream", c_void_p), ("fork_event", c_void_p),
                ("join_event", c_void_p)]


# name -> (restype, argtypes); every symbol include/kda.h declares.
PROTOTYPES = {
    "kda_state_bytes": (c_size_t, [POINTER(kda_pool_desc)]),
    "kda_ring_bytes": (c_size_t, [POINTER(kda_pool_desc)]),
    "kda_ring_layout": (c_int32, [POINTER(kda_pool_desc), POINTER(c_size_t)]),
    "kda_meta_bytes": (c_size_t, [POINTER(kda_pool_desc)]),
    "kda_meta_error_offset": (c_size_t, [POINTER(kda_pool_desc)]),
    "kda_pool_create": (c_int32, [POINTER(kda_pool_desc), c_void_p, c_void_p, c_void_p,
                                  POINTER(c_void_p)]),
    "kda_pool_destroy": (c_int32, [c_void_p]),
    "kda_slot_alloc": (c_int32, [c_void_p, POINTER(c_int32)]),
    "kda_slot_free": (c_int32, [c_void_p, c_int32]),
    "kda_slot_reset": (c_int32, [c_void_p, c_int32, c_void_p]),
    "kda_slot_checkpoint": (c_int32, [c_void_p, c_int32, c_int32, c_void_p]),
    "kda_prefill_workspace_bytes": (c_size_t, [c_void_p, c_int32, c_int32, c_int32, c_int32]),
    "kda_prefill": (c_int32, [c_void_p, POINTER(kda_prefill_args), c_void_p]),
    "kda_prefill_noalloc": (c_int32, [c_void_p, POINTER(kda_prefill_args), c_void_p]),
    "kda_prefill_plan": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "kda_decode": (c_int32, [c_void_p, POINTER(kda_step_args), c_void_p]),
    "kda_verify": (c_int32, [c_void_p, POINTER(kda_step_args), c_int32, c_void_p]),
    "kda_commit": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "kda_rollback": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "kda_draft_state_bytes": (c_size_t, [POINTER(kda_pool_desc), c_int32, c_int32]),
    "kda_verify_direct": (c_int32, [c_void_p, POINTER(kda_step_args), c_int32, c_void_p, c_void_p]),
    "kda_commit_direct": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_int32, c_void_p]),
    "kda_mixed_batch": (c_int32, [c_void_p, POINTER(kda_mixed_args), c_void_p]),
    "kda_read_device_error": (c_int32, [c_void_p, POINTER(c_uint32), c_void_p]),
    "kda_status_string": (c_char_p, [c_int32]),
    "kda_last_error": (c_char_p, []),
    "kda_slot_host_state": (c_int32, [c_void_p, c_int32]),
}


def _mapped_hip_runtimes() -> set[str]:
    try:
        maps = open("/proc/self/maps").read().splitlines()
    except OSError:
        return set()
    return {ln.split()[-1] for ln in maps if "libamdhip64" in ln}


def _check_single_runtime() -> None:
    hip = _mapped_hip_runtimes()
    if len(hip) > 1:
        raise ImportError("two HIP runtimes are loaded in this process (" + ", ".join(sorted(hip))
                          + "); import torch before loading libkda.so")


def hip_runtime() -> ctypes.CDLL:
    """The HIP runtime this process already holds (the one torch loaded and libkda.so binds
    to), opened by its mapped path, so that events created through it belong to the same
    runtime as torch's streams."""
    hip = _mapped_hip_runtimes()
    if len(hip) != 1:
        raise RuntimeError(f"expected one mapped HIP runtime, found {sorted(hip)}")
    return ctypes.CDLL(next(iter(hip)))


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"KDA HIP library not found at {path}; build it with "
            "`python recurrent_linear_attention_amd/build.py` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    _check_single_runtime()
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = load()


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.kda_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.kda_status_string(status).decode()} ({status}): {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != KDA_OK:
        raise KDAError(status, where)

"""Thin Python binding of the C ABI in include/moe_verify.h (argument marshalling only).

Every step of the verify path runs in the HIP library; this module turns torch device
tensors into pointers, the current torch stream into a hipStream_t, and status codes
into exceptions. It raises if the library is not built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from .build import LIB_PATH

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EDEVICE, MOE_EUNSUPPORTED = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1

EXPORTS = ("moe_verify_check_config", "moe_verify_check_step", "moe_verify_init", "moe_verify_step",
           "accept_greedy", "moe_verify_destroy", "moe_verify_last_error", "moe_verify_debug_layer",
           "moe_verify_profile", "moe_verify_profile_read", "moe_verify_expert_counts", "moe_draft_init",
           "moe_draft_step", "moe_verify_step_mixed", "moe_verify_debug_head", "moe_verify_debug_plan",
           "moe_verify_step_static")
PROF_KINDS = ("norm_route", "plan", "gemm_up", "gemm_down", "lm_head", "argmax")


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_routed", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("wdtype", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("max_positions", ctypes.c_int32)]


class WeightPtrs(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p), ("lm_head", ctypes.c_void_p)]


class DraftWeightPtrs(ctypes.Structure):
    _fields_ = [("inter", ctypes.c_int32), ("proj", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class MoeVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe_verify.so (once) and declare the C signatures.

    The path defaults to the in-tree build.
    """
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m lossless_speculative_verification_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    L.moe_verify_check_config.argtypes = [ctypes.POINTER(Config)]
    L.moe_verify_check_step.argtypes = [ctypes.POINTER(Config), i32, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.moe_verify_init.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(WeightPtrs), vp, ctypes.POINTER(vp)]
    L.moe_verify_step.argtypes = [vp, vp, i32, i32, vp, f32p, f32p, vp]
    L.accept_greedy.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    L.moe_verify_destroy.argtypes = [vp]
    L.moe_verify_destroy.restype = None
    L.moe_verify_last_error.argtypes = []
    L.moe_verify_last_error.restype = ctypes.c_char_p
    L.moe_verify_debug_layer.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp]
    L.moe_verify_profile.argtypes = [vp, ctypes.c_int]
    L.moe_verify_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.moe_verify_expert_counts.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    L.moe_draft_init.argtypes = [vp, ctypes.POINTER(DraftWeightPtrs), vp]
    L.moe_verify_step_mixed.argtypes = [vp, vp, i32, i32, i32, vp, f32p, f32p, vp]
    L.moe_draft_step.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp]
    L.moe_verify_debug_head.argtypes = [vp, vp, i32, vp, f32p, vp]
    L.moe_verify_debug_plan.argtypes = [vp, vp, vp, vp]
    L.moe_verify_step_static.argtypes = [vp, vp, i32, i32, vp, f32p, f32p, vp]
    for name in EXPORTS:
        if name not in ("moe_verify_destroy", "moe_verify_last_error"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return load_library().moe_verify_last_error().decode()


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeVerifyError(rc, f"{what} failed with status {rc}: {last_error()}")


def make_config(wl, max_positions: Optional[int] = None) -> Config:
    """C config from a workload-like object (hidden, n_routed, top_k, ... attributes)."""
    return Config(wl.hidden, wl.n_routed, wl.top_k, wl.n_shared, wl.inter, wl.n_layers, wl.vocab,
                  MOE_BF16 if wl.wdtype == "bf16" else MOE_F32, wl.rms_eps,
                  int(max_positions if max_positions is not None else wl.positions))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def upload_weights(weights, device="cuda") -> dict:
    """Copy host weights (numpy; bf16 as uint16 bit patterns) to device tensors."""
    import torch

    def dev(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    return {"router_w": dev(weights.router), "router_bias": dev(weights.router_bias), "w_gate": dev(weights.w_gate),
            "w_up": dev(weights.w_up), "w_down": dev(weights.w_down), "lm_head": dev(weights.lm_head)}


def upload_draft_weights(dweights, device="cuda") -> dict:
    """Copy host draft-block weights (workload.DraftWeights) to device tensors."""
    import torch

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    return {"inter": int(dweights.inter), "proj": dev(dweights.proj), "w_gate": dev(dweights.w_gate),
            "w_up": dev(dweights.w_up), "w_down": dev(dweights.w_down)}


class MoeVerify:
    """A library context: repacked weights plus workspace for up to max_positions positions."""

    def __init__(self, wl, dev_weights: dict, max_positions: Optional[int] = None, stream=None):
        L = load_library()
        self.wl = wl
        self.cfg = make_config(wl, max_positions)
        w = WeightPtrs(*(_ptr(dev_weights.get(k)) for k in ("router_w", "router_bias", "w_gate", "w_up", "w_down",
                                                            "lm_head")))
        h = ctypes.c_void_p()
        _check(L.moe_verify_init(ctypes.byref(self.cfg), ctypes.byref(w), _stream(stream), ctypes.byref(h)),
               "moe_verify_init")
        self._h = h

    def step(self, hidden_in, B: int, K: int, argmax_out=None, margin_out=None, hidden_out=None, stream=None):
        _check(load_library().moe_verify_step(self._h, _ptr(hidden_in), B, K, _ptr(argmax_out), _ptr(margin_out),
                                              _ptr(hidden_out), _stream(stream)), "moe_verify_step")

    def step_static(self, hidden_in, B: int, K: int, argmax_out=None, margin_out=None, hidden_out=None,
                    stream=None):
        _check(load_library().moe_verify_step_static(self._h, _ptr(hidden_in), B, K, _ptr(argmax_out),
                                                     _ptr(margin_out), _ptr(hidden_out), _stream(stream)),
               "moe_verify_step_static")

    def step_mixed(self, hidden_in, n_prefill: int, B: int, K: int, argmax_out=None, margin_out=None,
                   hidden_out=None, stream=None):
        _check(load_library().moe_verify_step_mixed(self._h, _ptr(hidden_in), n_prefill, B, K, _ptr(argmax_out),
                                                    _ptr(margin_out), _ptr(hidden_out), _stream(stream)),
               "moe_verify_step_mixed")

    def debug_layer(self, layer: int, x_in, T: int, moe_out=None, topk_id=None, topk_w=None, stream=None):
        _check(load_library().moe_verify_debug_layer(self._h, layer, _ptr(x_in), T, _ptr(moe_out), _ptr(topk_id),
                                                     _ptr(topk_w), _stream(stream)), "moe_verify_debug_layer")

    def debug_head(self, x_in, T: int, argmax_out, margin_out=None, stream=None):
        _check(load_library().moe_verify_debug_head(self._h, _ptr(x_in), T, _ptr(argmax_out), _ptr(margin_out),
                                                    _stream(stream)), "moe_verify_debug_head")

    def debug_plan(self, row_slot, counts=None, stream=None):
        _check(load_library().moe_verify_debug_plan(self._h, _ptr(row_slot), _ptr(counts), _stream(stream)),
               "moe_verify_debug_plan")

    def draft_init(self, dev_draft_weights: dict, stream=None):
        w = DraftWeightPtrs(dev_draft_weights["inter"], *(_ptr(dev_draft_weights[k])
                                                          for k in ("proj", "w_gate", "w_up", "w_down")))
        _check(load_library().moe_draft_init(self._h, ctypes.byref(w), _stream(stream)), "moe_draft_init")

    def draft_step(self, hidden, accepted_len, committed, B: int, Kv: int, K: int, drafts, stream=None):
        _check(load_library().moe_draft_step(self._h, _ptr(hidden), _ptr(accepted_len), _ptr(committed), B, Kv, K,
                                              _ptr(drafts), _stream(stream)), "moe_draft_step")

    def profile(self, enable: bool):
        _check(load_library().moe_verify_profile(self._h, int(enable)), "moe_verify_profile")

    def profile_read(self) -> dict:
        """Totals since profiling was enabled: {kind: (milliseconds, launches)}."""
        n = len(PROF_KINDS)
        ms, cnt = (ctypes.c_double * n)(), (ctypes.c_int64 * n)()
        _check(load_library().moe_verify_profile_read(self._h, ms, cnt), "moe_verify_profile_read")
        return {k: (ms[i], cnt[i]) for i, k in enumerate(PROF_KINDS)}

    def expert_counts(self) -> np.ndarray:
        """Routed-slot count per (block, routed expert) of the last step."""
        out = np.zeros((self.wl.n_layers, self.wl.n_routed), np.int32)
        _check(load_library().moe_verify_expert_counts(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))),
               "moe_verify_expert_counts")
        return out

    def close(self):
        if getattr(self, "_h", None):
            load_library().moe_verify_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def accept_greedy(draft_ids, argmax_ids, B: int, K: int, accepted_len, committed, stream=None):
    _check(load_library().accept_greedy(_ptr(draft_ids) if K > 0 else None, _ptr(argmax_ids), B, K,
                                        _ptr(accepted_len), _ptr(committed), _stream(stream)), "accept_greedy")

"""ctypes binding of libmoe_ffn.so (the C ABI in include/moe_ffn.h, and the
timing call of include/moe_ffn_profile.h).

Argument marshalling only: torch tensors in, device pointers and sizes out.
Every step of the layer runs in the HIP library; if the library is missing
this module raises instead of computing anything another way.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_FFN_LIB selects another build of the same library (same ABI)
LIB_PATH = os.environ.get("MOE_FFN_LIB") or os.path.join(_PKG, "libmoe_ffn.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_PKG), "include")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_ALIGNMENT",
                4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP"}


class MoeConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("route_scale", ctypes.c_float), ("swiglu_limit", ctypes.c_float), ("score_func", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("expert_format", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p), ("gu_q", ctypes.c_void_p),
                ("gu_s", ctypes.c_void_p), ("dn_q", ctypes.c_void_p), ("dn_s", ctypes.c_void_p),
                ("sh_gu", ctypes.c_void_p), ("sh_dn", ctypes.c_void_p), ("norm_gamma", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                          " or `python mixture_experts_ffn_07_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    cfgp, wp = ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeWeights)
    sig = {
        "moe_workspace_bytes": (sz, [cfgp, i64]),
        "moe_rmsnorm": (ctypes.c_int, [cfgp, vp, vp, i64, vp, vp]),
        "moe_route": (ctypes.c_int, [cfgp, wp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "moe_permute": (ctypes.c_int, [cfgp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "moe_expert_ffn": (ctypes.c_int, [cfgp, wp, vp, i64, vp, vp, vp, vp, vp, sz, vp]),
        "moe_combine": (ctypes.c_int, [cfgp, vp, vp, vp, vp, i64, vp, vp]),
        "moe_layer_forward": (ctypes.c_int, [cfgp, wp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "moe_layer_forward_noalloc": (ctypes.c_int, [cfgp, wp, vp, i64, vp, vp, vp, vp]),
        "moe_layer_forward_timed": (ctypes.c_int, [cfgp, wp, vp, i64, vp, vp, sz, vp,
                                                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p),
                                                   ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
        "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_abi_version": (ctypes.c_int32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions declared in the headers under include/."""
    names = []
    for path in sorted(os.path.join(INCLUDE_DIR, h) for h in os.listdir(INCLUDE_DIR) if h.endswith(".h")):
        with open(path) as f:
            text = f.read()
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", text, flags=re.M)
    return names


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status, load().moe_last_error().decode())


def make_config(hidden, n_experts, top_k, inter, n_shared=1, shared_inter=None, route_scale=1.5,
                swiglu_limit=10.0, score_func=0, norm_eps=1e-20, expert_format=0) -> MoeConfig:
    """expert_format: 0 or "mxfp4" (E2M1), 1 or "mxfp8" (E4M3)."""
    fmt = {"mxfp4": 0, "mxfp8": 1}.get(expert_format, expert_format)
    return MoeConfig(hidden, n_experts, top_k, inter, n_shared, inter if shared_inter is None else shared_inter,
                     route_scale, swiglu_limit, score_func, norm_eps, fmt)


def config_from(cfg) -> MoeConfig:
    """MoeConfig from any object with the layer-shape attributes (e.g. moe_synth.LayerConfig)."""
    return make_config(cfg.hidden, cfg.n_experts, cfg.top_k, cfg.inter, cfg.n_shared,
                       cfg.shared_inter if cfg.n_shared else 0, cfg.route_scale, cfg.swiglu_limit,
                       norm_eps=getattr(cfg, "norm_eps", 1e-20),
                       expert_format=getattr(cfg, "expert_format", "mxfp4"))


def make_weights(router_w, router_bias, gu_q, gu_s, dn_q, dn_s, sh_gu=None, sh_dn=None,
                 norm_gamma=None) -> MoeWeights:
    return MoeWeights(_ptr(router_w), _ptr(router_bias), _ptr(gu_q), _ptr(gu_s), _ptr(dn_q), _ptr(dn_s),
                      _ptr(sh_gu), _ptr(sh_dn), _ptr(norm_gamma))


def weights_from(inp) -> MoeWeights:
    """MoeWeights from an object with the weight tensors as attributes (e.g. moe_synth.LayerInputs)."""
    return make_weights(inp.router_w, inp.router_bias, inp.gu_q, inp.gu_s, inp.dn_q, inp.dn_s, inp.sh_gu, inp.sh_dn,
                        getattr(inp, "norm_gamma", None))


# ------------------------------------------------------------------ entry points (same names as the C ABI)

def moe_workspace_bytes(cfg: MoeConfig, tokens: int) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(cfg), tokens))


def workspace(cfg: MoeConfig, tokens: int, device="cuda") -> torch.Tensor:
    nbytes = moe_workspace_bytes(cfg, tokens)
    if nbytes == 0:
        raise MoeError("moe_workspace_bytes", 1, load().moe_last_error().decode())
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def moe_rmsnorm(cfg, gamma, x, tokens, x_norm, stream=None):
    _check("moe_rmsnorm", load().moe_rmsnorm(ctypes.byref(cfg), _ptr(gamma), _ptr(x), tokens, _ptr(x_norm),
                                             _stream(stream)))


def moe_route(cfg, w, x, tokens, topk_idx, topk_w, tie_gap, ws, stream=None):
    _check("moe_route", load().moe_route(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), tokens, _ptr(topk_idx),
                                         _ptr(topk_w), _ptr(tie_gap), _ptr(ws), ws.numel() if ws is not None else 0,
                                         _stream(stream)))


def moe_permute(cfg, topk_idx, tokens, expert_offsets, sorted_slots, slot_pos, ws, stream=None):
    _check("moe_permute", load().moe_permute(ctypes.byref(cfg), _ptr(topk_idx), tokens, _ptr(expert_offsets),
                                             _ptr(sorted_slots), _ptr(slot_pos), _ptr(ws),
                                             ws.numel() if ws is not None else 0, _stream(stream)))


def moe_expert_ffn(cfg, w, x, tokens, expert_offsets, sorted_slots, y_slot, y_shared, ws, stream=None):
    _check("moe_expert_ffn", load().moe_expert_ffn(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), tokens,
                                                   _ptr(expert_offsets), _ptr(sorted_slots), _ptr(y_slot),
                                                   _ptr(y_shared), _ptr(ws), ws.numel() if ws is not None else 0,
                                                   _stream(stream)))


def moe_combine(cfg, y_slot, slot_pos, topk_w, y_shared, tokens, y, stream=None):
    _check("moe_combine", load().moe_combine(ctypes.byref(cfg), _ptr(y_slot), _ptr(slot_pos), _ptr(topk_w),
                                             _ptr(y_shared), tokens, _ptr(y), _stream(stream)))


def moe_layer_forward(cfg, w, x, tokens, y, topk_idx_out, topk_w_out, ws, stream=None):
    _check("moe_layer_forward", load().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), tokens,
                                                         _ptr(y), _ptr(topk_idx_out), _ptr(topk_w_out), _ptr(ws),
                                                         ws.numel() if ws is not None else 0, _stream(stream)))


def moe_layer_forward_noalloc(cfg, w, x, tokens, y, topk_idx_out, topk_w_out, stream=None):
    _check("moe_layer_forward_noalloc",
           load().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), tokens, _ptr(y),
                                            _ptr(topk_idx_out), _ptr(topk_w_out), _stream(stream)))


def moe_layer_forward_timed(cfg, w, x, tokens, y, ws, stream=None, max_kernels: int = 32):
    """Per-kernel milliseconds of one layer forward, as a list of (kernel name, ms)."""
    ms = (ctypes.c_float * max_kernels)()
    names = (ctypes.c_char_p * max_kernels)()
    n = ctypes.c_int32(0)
    _check("moe_layer_forward_timed",
           load().moe_layer_forward_timed(ctypes.byref(cfg), ctypes.byref(w), _ptr(x), tokens, _ptr(y), _ptr(ws),
                                          ws.numel() if ws is not None else 0, _stream(stream), ms, names,
                                          max_kernels, ctypes.byref(n)))
    return [(names[i].decode(), float(ms[i])) for i in range(min(n.value, max_kernels))]

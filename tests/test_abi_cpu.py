"""The C ABI on a host without a GPU: exported symbols and argument checks.

Every call here either fails an argument check or has tokens == 0, so the
library returns before it touches the HIP runtime; pointers are placeholders
that are never dereferenced.
"""

import ctypes
import subprocess

import pytest

import mixture_experts_ffn_07_amd as moe
from mixture_experts_ffn_07_amd import _lib

OK, INVALID, UNSUPPORTED, ALIGN, WS = 0, 1, 2, 3, 4
P = 0x10000  # aligned placeholder address (never dereferenced)


def test_library_loads_and_exports_every_header_function():
    lib = moe.load()
    names = moe.header_functions()
    assert set(names) == {"moe_workspace_bytes", "moe_rmsnorm", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
                          "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_timed",
                          "moe_status_str", "moe_last_error", "moe_abi_version"}
    for n in names:
        assert hasattr(lib, n)
    dyn = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if " T " in line}
    assert set(names) <= exported
    assert lib.moe_abi_version() == 2


@pytest.mark.parametrize("tokens,code", [(77672, OK), (77673, UNSUPPORTED), (1 << 22, UNSUPPORTED)])
def test_buffer_extent_limit(tokens, code):
    """Matrices read through 32-bit buffer descriptors must stay below 2^31 - 16 bytes: at the full layer shape
    the routed activations [T*k][I] bf16 reach that at 77,673 tokens."""
    lib = moe.load()
    c, w, r, big = moe.make_config(5120, 384, 6, 2304), _weights(), ctypes.byref, 1 << 44
    assert (moe.moe_workspace_bytes(c, tokens) > 0) == (code == OK)
    if code != OK:
        assert lib.moe_layer_forward(r(c), r(w), P, tokens, P, None, None, P, big, None) == code
        assert "split the tokens" in lib.moe_last_error().decode()
        assert lib.moe_route(r(c), r(w), P, tokens, P, P, None, P, big, None) == code
        assert lib.moe_expert_ffn(r(c), r(w), P, tokens, P, P, P, P, P, big, None) == code
    # one MXFP8 expert's gate/up codes at H = I = 65536 would take 8 GiB
    c8 = moe.make_config(65536, 8, 2, 65536, n_shared=0, expert_format=1)
    assert moe.moe_workspace_bytes(c8, 1) == 0
    assert lib.moe_layer_forward(r(c8), r(_weights(sh_gu=None, sh_dn=None)), P, 1, P, None, None, P, big, None) \
        == UNSUPPORTED


def test_status_strings():
    lib = moe.load()
    for code in range(6):
        assert lib.moe_status_str(code)
    assert lib.moe_status_str(0) == b"ok"


def _cfg(**kw):
    base = dict(hidden=512, n_experts=32, top_k=6, inter=256, n_shared=1, shared_inter=256)
    base.update(kw)
    return moe.make_config(**base)


def _weights(**kw):
    w = moe.MoeWeights(P, 0, P, P, P, P, P, P)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def test_workspace_bytes():
    lib = moe.load()
    assert moe.moe_workspace_bytes(_cfg(), 8) > 0
    assert moe.moe_workspace_bytes(_cfg(), 64) >= moe.moe_workspace_bytes(_cfg(), 8)
    assert moe.moe_workspace_bytes(_cfg(hidden=100), 8) == 0
    assert moe.moe_workspace_bytes(_cfg(), -1) == 0
    assert lib.moe_workspace_bytes(None, 8) == 0
    # full-size decode and prefill shapes
    big = moe.make_config(5120, 384, 6, 2304)
    assert moe.moe_workspace_bytes(big, 4096) > 4096 * 6 * (5120 + 2304) * 2


BAD_CONFIGS = [
    (dict(hidden=0), INVALID), (dict(hidden=48), INVALID), (dict(hidden=65568), INVALID),
    (dict(inter=16), INVALID), (dict(n_experts=0), INVALID), (dict(n_experts=1025), INVALID),
    (dict(top_k=0), INVALID), (dict(top_k=17, n_experts=64), INVALID), (dict(top_k=7, n_experts=6), INVALID),
    (dict(n_shared=2), INVALID), (dict(shared_inter=40), INVALID), (dict(score_func=1), UNSUPPORTED),
    (dict(route_scale=float("inf")), INVALID), (dict(swiglu_limit=0.0), INVALID),
    (dict(swiglu_limit=float("nan")), INVALID), (dict(expert_format=2), INVALID), (dict(expert_format=-1), INVALID),
]


@pytest.mark.parametrize("mut,code", BAD_CONFIGS)
def test_bad_config_rejected_by_every_entry_point(mut, code):
    lib = moe.load()
    c = _cfg(**mut)
    w = _weights()
    r = ctypes.byref
    assert lib.moe_route(r(c), r(w), P, 8, P, P, None, P, 1 << 40, None) == code
    assert lib.moe_permute(r(c), P, 8, P, P, P, P, 1 << 40, None) == code
    assert lib.moe_expert_ffn(r(c), r(w), P, 8, P, P, P, P, P, 1 << 40, None) == code
    assert lib.moe_combine(r(c), P, P, P, P, 8, P, None) == code
    assert lib.moe_layer_forward(r(c), r(w), P, 8, P, None, None, P, 1 << 40, None) == code
    assert lib.moe_rmsnorm(r(c), P, P, 8, P, None) == code
    assert lib.moe_last_error()


def test_null_config_and_weights():
    lib = moe.load()
    c, w, r = _cfg(), _weights(), ctypes.byref
    assert lib.moe_route(None, r(w), P, 8, P, P, None, P, 1 << 40, None) == INVALID
    assert lib.moe_route(r(c), None, P, 8, P, P, None, P, 1 << 40, None) == INVALID
    assert lib.moe_layer_forward(r(c), None, P, 8, P, None, None, P, 1 << 40, None) == INVALID


@pytest.mark.parametrize("tokens", [-1, (1 << 22) + 1])
def test_bad_token_counts(tokens):
    lib = moe.load()
    c, w, r = _cfg(), _weights(), ctypes.byref
    assert lib.moe_layer_forward(r(c), r(w), P, tokens, P, None, None, P, 1 << 40, None) == INVALID
    assert lib.moe_combine(r(c), P, P, P, P, tokens, P, None) == INVALID


def test_pointer_checks_layer_forward():
    lib = moe.load()
    c, r = _cfg(), ctypes.byref
    big = 1 << 40
    assert lib.moe_layer_forward(r(c), r(_weights()), None, 8, P, None, None, P, big, None) == INVALID
    assert lib.moe_layer_forward(r(c), r(_weights()), P + 2, 8, P, None, None, P, big, None) == ALIGN
    assert lib.moe_layer_forward(r(c), r(_weights()), P, 8, None, None, None, P, big, None) == INVALID
    assert lib.moe_layer_forward(r(c), r(_weights()), P, 8, P, P + 2, None, P, big, None) == ALIGN
    for field in ("router_w", "gu_q", "gu_s", "dn_q", "dn_s", "sh_gu", "sh_dn"):
        assert lib.moe_layer_forward(r(c), r(_weights(**{field: None})), P, 8, P, None, None, P, big, None) \
            == INVALID, field
        assert lib.moe_layer_forward(r(c), r(_weights(**{field: P + 8})), P, 8, P, None, None, P, big, None) \
            == ALIGN, field
    assert lib.moe_layer_forward(r(c), r(_weights(router_bias=P + 2)), P, 8, P, None, None, P, big, None) == ALIGN
    # shared weights must be absent without a shared expert
    c0 = _cfg(n_shared=0)
    assert lib.moe_layer_forward(r(c0), r(_weights()), P, 8, P, None, None, P, big, None) == INVALID


def test_workspace_checks():
    lib = moe.load()
    c, w, r = _cfg(), _weights(), ctypes.byref
    need = moe.moe_workspace_bytes(c, 8)
    assert lib.moe_layer_forward(r(c), r(w), P, 8, P, None, None, None, big := 1 << 40, None) == WS
    assert lib.moe_layer_forward(r(c), r(w), P, 8, P, None, None, P, need - 1, None) == WS
    assert lib.moe_layer_forward(r(c), r(w), P, 8, P, None, None, P + 16, big, None) == ALIGN
    assert lib.moe_route(r(c), r(w), P, 8, P, P, None, P, need - 1, None) == WS
    assert lib.moe_permute(r(c), P, 8, P, P, P, P, need - 1, None) == WS
    assert lib.moe_expert_ffn(r(c), r(w), P, 8, P, P, P, P, P, need - 1, None) == WS


def test_other_entry_point_pointer_checks():
    lib = moe.load()
    c, w, r, big = _cfg(), _weights(), ctypes.byref, 1 << 40
    assert lib.moe_route(r(c), r(w), P, 8, None, P, None, P, big, None) == INVALID
    assert lib.moe_route(r(c), r(w), P, 8, P, None, None, P, big, None) == INVALID
    assert lib.moe_route(r(c), r(w), P, 8, P, P, P + 1, P, big, None) == ALIGN
    assert lib.moe_permute(r(c), None, 8, P, P, P, P, big, None) == INVALID
    assert lib.moe_permute(r(c), P, 8, P, None, P, P, big, None) == INVALID
    assert lib.moe_expert_ffn(r(c), r(w), P, 8, P, P, P, None, P, big, None) == INVALID  # shared output missing
    c0 = _cfg(n_shared=0)
    w0 = _weights(sh_gu=None, sh_dn=None)
    assert lib.moe_expert_ffn(r(c0), r(w0), P, 8, P, P, P, P, P, big, None) == INVALID  # shared output given
    assert lib.moe_combine(r(c), None, P, P, P, 8, P, None) == INVALID
    assert lib.moe_combine(r(c), P, P, P, P + 4, 8, P, None) == ALIGN


def test_zero_tokens_is_a_no_op():
    lib = moe.load()
    c, w, r, big = _cfg(), _weights(), ctypes.byref, 1 << 40
    assert lib.moe_route(r(c), r(w), P, 0, P, P, None, P, big, None) == OK
    assert lib.moe_permute(r(c), P, 0, P, P, P, P, big, None) == OK
    assert lib.moe_expert_ffn(r(c), r(w), P, 0, P, P, P, P, P, big, None) == OK
    assert lib.moe_combine(r(c), P, P, P, P, 0, P, None) == OK
    assert lib.moe_layer_forward(r(c), r(w), P, 0, P, None, None, P, big, None) == OK


def test_timed_forward_argument_checks():
    lib = moe.load()
    c, w, r, big = _cfg(), _weights(), ctypes.byref, 1 << 40
    ms = (ctypes.c_float * 4)()
    names = (ctypes.c_char_p * 4)()
    n = ctypes.c_int32(-1)
    assert lib.moe_layer_forward_timed(r(c), r(w), P, 8, P, P, big, None, None, names, 4, r(n)) == INVALID
    assert lib.moe_layer_forward_timed(r(c), r(w), P, 8, P, P, big, None, ms, None, 4, r(n)) == INVALID
    assert lib.moe_layer_forward_timed(r(c), r(w), P, 8, P, P, big, None, ms, names, -1, r(n)) == INVALID


def test_binding_raises_with_status_and_message():
    c = _cfg(hidden=48)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_combine(c, None, None, None, None, 8, None)
    assert ei.value.status == INVALID
    assert "hidden" in str(ei.value)


def test_norm_checks():
    """moe_rmsnorm and the norm fields of moe_layer_forward are checked before anything is enqueued."""
    lib = moe.load()
    r, big = ctypes.byref, 1 << 40
    c = _cfg()
    assert lib.moe_rmsnorm(r(c), None, P, 8, P, None) == INVALID
    assert lib.moe_rmsnorm(r(c), P + 2, P, 8, P, None) == ALIGN
    assert lib.moe_rmsnorm(r(c), P, None, 8, P, None) == INVALID
    assert lib.moe_rmsnorm(r(c), P, P + 8, 8, P, None) == ALIGN
    assert lib.moe_rmsnorm(r(c), P, P, 8, None, None) == INVALID
    assert lib.moe_rmsnorm(r(c), P, P, -1, P, None) == INVALID
    assert lib.moe_rmsnorm(r(c), P, P, 0, P, None) == OK  # nothing to do, nothing enqueued
    for eps in (0.0, -1e-20, float("inf"), float("nan")):
        ce = _cfg(norm_eps=eps)
        assert lib.moe_rmsnorm(r(ce), P, P, 8, P, None) == INVALID, eps
        assert lib.moe_layer_forward(r(ce), r(_weights(norm_gamma=P)), P, 8, P, None, None, P, big, None) \
            == INVALID, eps
        # without a gain the eps is not read
        assert lib.moe_layer_forward(r(ce), r(_weights()), P, 0, P, None, None, P, big, None) == OK, eps
    assert lib.moe_layer_forward(r(c), r(_weights(norm_gamma=P + 2)), P, 8, P, None, None, P, big, None) == ALIGN
    assert "norm" in lib.moe_last_error().decode()


def test_noalloc_argument_checks():
    """moe_layer_forward_noalloc checks its arguments (and its scratch limit) before it touches the HIP runtime."""
    lib = moe.load()
    c, w, r = _cfg(), _weights(), ctypes.byref
    assert lib.moe_layer_forward_noalloc(r(c), r(w), P, 0, P, None, None, None) == OK
    assert lib.moe_layer_forward_noalloc(r(_cfg(hidden=48)), r(w), P, 8, P, None, None, None) == INVALID
    assert lib.moe_layer_forward_noalloc(r(c), r(w), None, 8, P, None, None, None) == INVALID
    assert lib.moe_layer_forward_noalloc(r(c), r(w), P + 2, 8, P, None, None, None) == ALIGN
    assert lib.moe_layer_forward_noalloc(r(c), r(_weights(gu_q=None)), P, 8, P, None, None, None) == INVALID
    assert lib.moe_layer_forward_noalloc(r(c), r(w), P, -1, P, None, None, None) == INVALID
    # the full-size layer at 128 tokens needs more than the 16 MiB of scratch the library holds
    big = moe.make_config(5120, 384, 6, 2304)
    assert moe.moe_workspace_bytes(big, 128) > (16 << 20) >= moe.moe_workspace_bytes(big, 64)
    assert lib.moe_layer_forward_noalloc(r(big), r(w), P, 128, P, None, None, None) == UNSUPPORTED
    assert "scratch" in lib.moe_last_error().decode()

"""The C ABI loads, exports what include/moe.h declares, and validates on the
host (no GPU needed: every call here fails validation before any launch)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

L = pytest.importorskip("sparse_mixture_experts_04_amd._lib")
lib = L.lib


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.SYMBOLS) == names


def test_version_and_status_strings():
    assert lib.moe_abi_version() == L.ABI_VERSION == 4
    for code in range(7):
        s = lib.moe_status_string(code)
        assert s and isinstance(s, bytes)
    assert lib.moe_status_string(99) == b"unknown status"


def desc(**kw):
    base = dict(T=128, d=512, F=128, E=256, S=2, k=6, act=L.F32, weight=L.F32,
                gate_norm=L.GATE_RATIO, gate_scale=1.0, capacity_factor=0.0)
    base.update(kw)
    return L.Desc(**base)


def ws_size(d, call):
    n = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(ctypes.byref(d) if d is not None else None, call,
                                ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), 2), (dict(d=0), 2), (dict(k=0), 2),
    (dict(act=L.BF16), 3), (dict(act=7, weight=7), 3),
    (dict(E=128), 0), (dict(E=64, S=0), 0), (dict(S=1), 0),
    (dict(E=96), 5), (dict(E=512), 5), (dict(S=3), 5), (dict(k=8), 5),
    (dict(d=384), 5), (dict(F=96), 5), (dict(d=48), 5),
    (dict(T=1 << 29), 5),
    (dict(gate_norm=2), 2), (dict(gate_norm=-1), 2), (dict(gate_scale=0.0), 2),
    (dict(gate_scale=-8.0), 2), (dict(gate_scale=float("inf")), 2),
    (dict(gate_scale=float("nan")), 2),
    (dict(gate_norm=L.GATE_LOGSUMEXP, gate_scale=6.5), 0),
    (dict(capacity_factor=-1.0), 2), (dict(capacity_factor=float("inf")), 2),
    (dict(capacity_factor=float("nan")), 2), (dict(capacity_factor=1.25), 0),
    # FP4 routed weights: bf16 activations, decode batches only
    (dict(act=L.BF16, weight=L.MXFP4, T=64), 0), (dict(act=L.BF16, weight=L.MXFP4, T=2047), 0),
    (dict(act=L.BF16, weight=L.MXFP4, T=2048), 5), (dict(act=L.F32, weight=L.MXFP4), 3),
])
def test_desc_validation(kw, code):
    st, _ = ws_size(desc(**kw), L.CALL_FORWARD)
    assert st == code


def test_routing_calls_accept_narrow_embeddings():
    """The router, dispatch, combine and bias update need d % 32 == 0; the
    expert GEMMs d % 256 == 0 and F % 128 == 0."""
    d = desc(E=64, S=0, d=32, F=96, T=2048, capacity_factor=1.25)
    for call in (L.CALL_ROUTER, L.CALL_DISPATCH, L.CALL_COMBINE, L.CALL_BIAS_UPDATE):
        assert ws_size(d, call)[0] == 0
    for call in (L.CALL_GATE_UP, L.CALL_DOWN, L.CALL_EXPERT_FFN, L.CALL_FORWARD):
        assert ws_size(d, call)[0] == 5
    # no shared experts: y_shared may be NULL; a NULL routed output still fails
    P = ctypes.c_void_p(0x1000)
    assert lib.moe_combine(ctypes.byref(d), P, None, P, P, None, None) == 1
    assert lib.moe_combine(ctypes.byref(d), None, None, P, P, P, None) == 1


def test_null_desc_and_null_out():
    st, _ = ws_size(None, L.CALL_FORWARD)
    assert st == 1
    assert lib.moe_workspace_size(ctypes.byref(desc()), L.CALL_FORWARD, None) == 1


def test_workspace_sizes_are_consistent():
    for act in (L.F32, L.BF16):
        d = desc(act=act, weight=act, T=4096, d=2048, F=768)
        sizes = {c: ws_size(d, c)[1] for c in range(8)}
        assert ws_size(d, 8)[0] == 2
        assert sizes[L.CALL_COMBINE] == 0 and sizes[L.CALL_BIAS_UPDATE] == 0
        assert sizes[L.CALL_EXPERT_FFN] > sizes[L.CALL_GATE_UP] > 0
        assert sizes[L.CALL_FORWARD] >= max(sizes[c] for c in range(7))
        # h alone: (k+S) * T * F elements of the act dtype
        esz = 4 if act == L.F32 else 2
        assert sizes[L.CALL_EXPERT_FFN] >= 8 * 4096 * 768 * esz
    # T = 0 is valid
    assert ws_size(desc(T=0), L.CALL_FORWARD)[0] == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_calls_reject_bad_arguments_before_launch():
    d = desc()
    P = FAKE
    # missing pointers
    assert lib.moe_router(ctypes.byref(d), None, P, P, P, P, None, P, 1 << 30, None) == 1
    assert lib.moe_dispatch(ctypes.byref(d), P, None, P, P, P, P, 1 << 30, None) == 1
    w = L.Weights(w_router=0x1000, w_gate=0x1000, w_up=0x1000, w_down=None,
                  ws_gate=0x1000, ws_up=0x1000, ws_down=0x1000)
    assert lib.moe_expert_ffn(ctypes.byref(d), P, ctypes.byref(w), P, P, P, P, P, 1 << 30,
                              None) == 1
    assert lib.moe_combine(ctypes.byref(d), P, P, None, P, P, None) == 1
    assert lib.moe_bias_update(ctypes.byref(d), None, 1e-3, P, None) == 1
    # workspace too small
    _, need = ws_size(d, L.CALL_ROUTER)
    assert lib.moe_router(ctypes.byref(d), P, P, P, P, P, None, P, need - 1, None) == 4
    assert lib.moe_router(ctypes.byref(d), P, P, P, P, P, None, None, need, None) == 4
    _, need = ws_size(d, L.CALL_DISPATCH)
    assert lib.moe_dispatch(ctypes.byref(d), P, P, P, P, P, P, need - 1, None) == 4
    # non-finite gamma
    assert lib.moe_bias_update(ctypes.byref(d), P, math.inf, P, None) == 2
    assert lib.moe_bias_update(ctypes.byref(d), P, math.nan, P, None) == 2
    wf = L.Weights(*([0x1000] * 7))
    _, need = ws_size(d, L.CALL_FORWARD)
    assert lib.moe_forward(ctypes.byref(d), P, ctypes.byref(wf), P, math.nan, P, None, P,
                           need, None) == 2
    # unsupported dtype combination
    bad = desc(act=L.BF16, weight=L.F32)
    assert lib.moe_forward(ctypes.byref(bad), P, ctypes.byref(wf), P, 1e-3, P, None, P,
                           need, None) == 3
    # forward without the router weights
    wf2 = L.Weights(None, *([0x1000] * 6))
    assert lib.moe_forward(ctypes.byref(d), P, ctypes.byref(wf2), P, 1e-3, P, None, P,
                           need, None) == 1
    # the marked forward needs all seven events
    assert lib.moe_forward_marked(ctypes.byref(d), P, ctypes.byref(wf), P, 1e-3, P, None, P,
                                  need, None, None) == 1
    marks = (ctypes.c_void_p * 7)(*([0x1000] * 6 + [0]))
    assert lib.moe_forward_marked(ctypes.byref(d), P, ctypes.byref(wf), P, 1e-3, P, None, P,
                                  need, marks, None) == 1


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    d = L.make_desc(4, 512, 128, torch.float32)
    x = torch.zeros(4, 512)
    with pytest.raises(ValueError):
        L._ptr(x, torch.float32, (4, 512), "x")
    with pytest.raises(TypeError):
        L.make_desc(4, 512, 128, torch.float16)
    assert d.T == 4


def test_quantize_argument_checks():
    P = ctypes.c_void_p(0x1000)
    assert lib.moe_quantize_mxfp4(2, 8, 48, P, P, P, None) == 2       # K % 128
    assert lib.moe_quantize_mxfp4(2, 8, 64, P, P, P, None) == 2
    assert lib.moe_quantize_mxfp4(-1, 8, 128, P, P, P, None) == 2
    assert lib.moe_quantize_mxfp4(2, 0, 128, P, P, P, None) == 2
    assert lib.moe_quantize_mxfp4(2, 8, 128, None, P, P, None) == 1
    assert lib.moe_quantize_mxfp4(2, 8, 128, ctypes.c_void_p(0x1004), P, P, None) == 5
    assert lib.moe_quantize_mxfp4(0, 8, 128, None, None, None, None) == 0  # nothing to do


def test_quantize_binding_needs_whole_k_tiles():
    # the codes are stored by 128-value K tiles; the binding refuses other K
    # before it touches any device memory
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError, match="multiple of 128"):
        L.quantize_mxfp4(torch.zeros((2, 8, 96), dtype=torch.bfloat16))


def test_dispatch_noalloc_validates_before_launch():
    """moe_dispatch_noalloc checks its arguments, then that the batch fits its
    1 MiB scratch (523776 pairs at E=256), before it touches a device."""
    P = FAKE
    d = desc(T=1023 * 512 // 6 + 1)                      # 1024 segments of 512 pairs
    assert lib.moe_dispatch_noalloc(ctypes.byref(d), P, P, P, P, P, None) == 5
    d64 = desc(T=4095 * 512 // 6 + 1, E=64, S=0)         # 4096 segments at E=64
    assert lib.moe_dispatch_noalloc(ctypes.byref(d64), P, P, P, P, P, None) == 5
    ok = desc(T=1000)
    assert lib.moe_dispatch_noalloc(ctypes.byref(ok), P, None, P, P, P, None) == 1
    assert lib.moe_dispatch_noalloc(ctypes.byref(ok), None, P, P, P, P, None) == 1
    assert lib.moe_dispatch_noalloc(None, P, P, P, P, P, None) == 1
    assert lib.moe_dispatch_noalloc(ctypes.byref(desc(k=8)), P, P, P, P, P, None) == 5


def test_router_prepare_validates_before_launch():
    d = desc(d=7168, F=2048, act=L.BF16, weight=L.BF16)
    n = ctypes.c_size_t(0)
    assert lib.moe_router_planes_size(ctypes.byref(d), ctypes.byref(n)) == 0
    # three bf16 planes of the 258 router rows padded to 320
    assert n.value == 3 * 320 * 7168 * 2
    assert lib.moe_router_planes_size(ctypes.byref(d), None) == 1
    assert lib.moe_router_planes_size(None, ctypes.byref(n)) == 1
    e64 = desc(E=64, S=0)
    assert lib.moe_router_planes_size(ctypes.byref(e64), ctypes.byref(n)) == 0
    assert n.value == 3 * 64 * 512 * 4 // 2
    P = FAKE
    assert lib.moe_router_prepare(ctypes.byref(d), None, P, None) == 1
    assert lib.moe_router_prepare(ctypes.byref(d), P, None, None) == 1
    assert lib.moe_router_prepare(ctypes.byref(desc(E=100)), P, P, None) == 5
    assert lib.moe_router_prepare(ctypes.byref(desc(d=-1)), P, P, None) == 2
    # the binding's Weights carries the prepared planes as its last field
    assert L.Weights._fields_[-1][0] == "w_router_planes"
    assert ctypes.sizeof(L.Weights) == 11 * ctypes.sizeof(ctypes.c_void_p)

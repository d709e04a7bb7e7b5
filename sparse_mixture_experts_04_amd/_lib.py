"""ctypes binding of libmoe.so (argument marshalling only).

Every function here checks dtypes, devices, shapes and contiguity of torch
tensors, then calls the C entry point of the same name on torch's current
stream.  All arithmetic runs in the library's HIP kernels; there is no
fallback: if libmoe.so is missing the import fails with an error that says
how to build it.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

# MOE_ABI_VERSION of include/moe.h that the structures below follow
ABI_VERSION = 4

F32, BF16, MXFP4 = 0, 1, 2
CALL_ROUTER, CALL_DISPATCH, CALL_GATE_UP, CALL_DOWN = 0, 1, 2, 3
CALL_EXPERT_FFN, CALL_COMBINE, CALL_BIAS_UPDATE, CALL_FORWARD = 4, 5, 6, 7

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE",
          4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_UNSUPPORTED", 6: "MOE_ERR_HIP"}

SYMBOLS = ("moe_abi_version", "moe_status_string", "moe_workspace_size", "moe_router",
           "moe_dispatch", "moe_expert_gate_up", "moe_expert_down", "moe_expert_ffn",
           "moe_combine", "moe_bias_update", "moe_forward", "moe_expert_gate_up_marked",
           "moe_expert_down_marked", "moe_quantize_mxfp4", "moe_forward_marked",
           "moe_dispatch_noalloc", "moe_router_planes_size", "moe_router_prepare")


class MoEError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("F", ctypes.c_int32),
                ("E", ctypes.c_int32), ("S", ctypes.c_int32), ("k", ctypes.c_int32),
                ("act", ctypes.c_int), ("weight", ctypes.c_int),
                ("gate_norm", ctypes.c_int32), ("gate_scale", ctypes.c_float),
                ("capacity_factor", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down",
                 "sc_gate", "sc_up", "sc_down", "w_router_planes")]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "gates", "margin", "counts", "offsets", "sorted_pair",
                 "pair_pos")]


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run "
                          "`python -m sparse_mixture_experts_04_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(Desc)
    W = ctypes.POINTER(Weights)
    sig = {
        "moe_abi_version": (I, []),
        "moe_status_string": (ctypes.c_char_p, [I]),
        "moe_workspace_size": (I, [D, I, ctypes.POINTER(Z)]),
        "moe_router": (I, [D, P, P, P, P, P, P, P, Z, P]),
        "moe_dispatch": (I, [D, P, P, P, P, P, P, Z, P]),
        "moe_dispatch_noalloc": (I, [D, P, P, P, P, P, P]),
        "moe_expert_gate_up": (I, [D, P, W, P, P, P, P, Z, P]),
        "moe_expert_down": (I, [D, W, P, P, P, P, P, Z, P]),
        "moe_expert_gate_up_marked": (I, [D, P, W, P, P, P, P, Z, P, P]),
        "moe_expert_down_marked": (I, [D, W, P, P, P, P, P, Z, P, P]),
        "moe_expert_ffn": (I, [D, P, W, P, P, P, P, P, Z, P]),
        "moe_combine": (I, [D, P, P, P, P, P, P]),
        "moe_bias_update": (I, [D, P, ctypes.c_float, P, P]),
        "moe_forward": (I, [D, P, W, P, ctypes.c_float, P, ctypes.POINTER(Routing), P, Z, P]),
        "moe_forward_marked": (I, [D, P, W, P, ctypes.c_float, P, ctypes.POINTER(Routing), P, Z,
                                   P, P]),
        "moe_quantize_mxfp4": (I, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P]),
        "moe_router_planes_size": (I, [D, ctypes.POINTER(Z)]),
        "moe_router_prepare": (I, [D, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.moe_abi_version()}, the binding expects "
                          f"{ABI_VERSION}; rebuild with `python -m sparse_mixture_experts_04_amd.build`")
    return lib


lib = _load()


def _check(fn, status):
    if status != 0:
        raise MoEError(fn, status, lib.moe_status_string(status).decode())


def act_code(dtype):
    if dtype == torch.float32:
        return F32
    if dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported activation dtype {dtype}")


GATE_RATIO, GATE_LOGSUMEXP = 0, 1


def make_desc(T, d, F, act_dtype, E=256, S=2, k=6, gate_norm="ratio", gate_scale=1.0,
              capacity_factor=0.0, fp4_weights=False):
    """Layer descriptor; ``fp4_weights`` marks the routed experts' weights as
    MXFP4 (quantize_mxfp4 outputs, bf16 activations only)."""
    a = act_code(act_dtype)
    norm = {"ratio": GATE_RATIO, "logsumexp": GATE_LOGSUMEXP}[gate_norm]
    return Desc(T, d, F, E, S, k, a, MXFP4 if fp4_weights else a, norm, gate_scale,
                capacity_factor)


def _act(desc):
    return torch.float32 if desc.act == F32 else torch.bfloat16


def _ptr(t, dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(desc, call):
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", lib.moe_workspace_size(ctypes.byref(desc), call, ctypes.byref(n)))
    return n.value


def alloc_workspace(desc, call, device):
    n = workspace_size(desc, call)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def router_planes(desc, w_router):
    """moe_router_prepare: the router's bf16 planes of w_router [E+S, d]
    fp32, once per weights.  Returns a bfloat16 tensor [3, P, d] (P = E+S
    rounded up to 64) to pass as ``w_router_planes``."""
    n = ctypes.c_size_t(0)
    _check("moe_router_planes_size",
           lib.moe_router_planes_size(ctypes.byref(desc), ctypes.byref(n)))
    E, S, d = desc.E, desc.S, desc.d
    planes = torch.empty((3, n.value // (6 * d), d), dtype=torch.bfloat16,
                         device=w_router.device)
    st = lib.moe_router_prepare(ctypes.byref(desc),
                                _ptr(w_router, torch.float32, (E + S, d), "w_router"),
                                planes.data_ptr(), _stream(w_router.device))
    _check("moe_router_prepare", st)
    return planes


def with_router_planes(weights, planes):
    """The same Weights with w_router_planes set (planes from router_planes,
    which must stay alive while the Weights are used)."""
    if planes is not None and (planes.dtype != torch.bfloat16 or not planes.is_contiguous()):
        raise ValueError("planes must be a contiguous bfloat16 tensor from router_planes")
    wt = Weights.from_buffer_copy(weights)
    wt.w_router_planes = planes.data_ptr() if planes is not None else None
    return wt


def make_weights(w_router, w_gate, w_up, w_down, ws_gate, ws_up, ws_down):
    wt = Weights()
    dt = w_gate.dtype
    E, F, d = w_gate.shape
    S = ws_gate.shape[0]
    wt.w_router = _ptr(w_router, torch.float32, (E + S, d), "w_router") if w_router is not None else None
    wt.w_gate = _ptr(w_gate, dt, (E, F, d), "w_gate")
    wt.w_up = _ptr(w_up, dt, (E, F, d), "w_up")
    wt.w_down = _ptr(w_down, dt, (E, d, F), "w_down")
    wt.ws_gate = _ptr(ws_gate, dt, (S, F, d), "ws_gate")
    wt.ws_up = _ptr(ws_up, dt, (S, F, d), "ws_up")
    wt.ws_down = _ptr(ws_down, dt, (S, d, F), "ws_down")
    return wt


def weights_from(inp):
    return make_weights(inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                        inp["ws_gate"], inp["ws_up"], inp["ws_down"])


def quantize_mxfp4(w):
    """moe_quantize_mxfp4 of a bf16 stack w [E, N, K]: returns (codes
    uint8 [E, K/128, N, 64], scales uint8 [E, K/128, N, 4]) on w's device."""
    E, N, K = w.shape
    if K % 128:
        raise ValueError(f"quantize_mxfp4: K = {K} is not a multiple of 128")
    codes = torch.empty((E, K // 128, N, 64), dtype=torch.uint8, device=w.device)
    scales = torch.empty((E, K // 128, N, 4), dtype=torch.uint8, device=w.device)
    st = lib.moe_quantize_mxfp4(E, N, K, _ptr(w, torch.bfloat16, (E, N, K), "w"),
                                codes.data_ptr(), scales.data_ptr(), _stream(w.device))
    _check("moe_quantize_mxfp4", st)
    return codes, scales


def fp4_weights(inp):
    """Weights with the routed experts quantized to MXFP4 (the shared experts
    and the router as given).  Returns (Weights, dict of the new tensors,
    which must stay alive while the Weights are used)."""
    q = {}
    for n in ("w_gate", "w_up", "w_down"):
        q[n], q["sc_" + n[2:]] = quantize_mxfp4(inp[n])
    E, F, d = inp["w_gate"].shape
    S = inp["ws_gate"].shape[0]
    wt = Weights()
    wt.w_router = _ptr(inp["w_router"], torch.float32, (E + S, d), "w_router")
    wt.w_gate = _ptr(q["w_gate"], torch.uint8, (E, d // 128, F, 64), "w_gate")
    wt.w_up = _ptr(q["w_up"], torch.uint8, (E, d // 128, F, 64), "w_up")
    wt.w_down = _ptr(q["w_down"], torch.uint8, (E, F // 128, d, 64), "w_down")
    wt.sc_gate = _ptr(q["sc_gate"], torch.uint8, (E, d // 128, F, 4), "sc_gate")
    wt.sc_up = _ptr(q["sc_up"], torch.uint8, (E, d // 128, F, 4), "sc_up")
    wt.sc_down = _ptr(q["sc_down"], torch.uint8, (E, F // 128, d, 4), "sc_down")
    dt = torch.bfloat16
    wt.ws_gate = _ptr(inp["ws_gate"], dt, (S, F, d), "ws_gate")
    wt.ws_up = _ptr(inp["ws_up"], dt, (S, F, d), "ws_up")
    wt.ws_down = _ptr(inp["ws_down"], dt, (S, d, F), "ws_down")
    return wt, q


# ------------------------------------------------------------------ calls

def router(desc, x, w_router, bias, topk_idx, gates, margin=None, ws=None):
    T, d, E, S, k = desc.T, desc.d, desc.E, desc.S, desc.k
    ws = alloc_workspace(desc, CALL_ROUTER, x.device) if ws is None else ws
    st = lib.moe_router(ctypes.byref(desc), _ptr(x, _act(desc), (T, d), "x"),
                        _ptr(w_router, torch.float32, (E + S, d), "w_router"),
                        _ptr(bias, torch.float32, (E,), "bias"),
                        _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
                        _ptr(gates, torch.float32, (T, k + S), "gates"),
                        _ptr(margin, torch.float32, (T,), "margin"),
                        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(x.device))
    _check("moe_router", st)


def dispatch(desc, topk_idx, counts, offsets, sorted_pair, pair_pos, ws=None):
    T, E, k = desc.T, desc.E, desc.k
    ws = alloc_workspace(desc, CALL_DISPATCH, counts.device) if ws is None else ws
    st = lib.moe_dispatch(ctypes.byref(desc), _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
                          _ptr(counts, torch.int32, (E,), "counts"),
                          _ptr(offsets, torch.int32, (E + 1,), "offsets"),
                          _ptr(sorted_pair, torch.int32, (T * k,), "sorted_pair"),
                          _ptr(pair_pos, torch.int32, (T * k,), "pair_pos"),
                          _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(counts.device))
    _check("moe_dispatch", st)


def dispatch_noalloc(desc, topk_idx, counts, offsets, sorted_pair, pair_pos):
    """moe_dispatch_noalloc: the dispatch with its scratch in the library's
    own device array (no workspace, nothing allocated)."""
    T, E, k = desc.T, desc.E, desc.k
    st = lib.moe_dispatch_noalloc(ctypes.byref(desc),
                                  _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
                                  _ptr(counts, torch.int32, (E,), "counts"),
                                  _ptr(offsets, torch.int32, (E + 1,), "offsets"),
                                  _ptr(sorted_pair, torch.int32, (T * k,), "sorted_pair"),
                                  _ptr(pair_pos, torch.int32, (T * k,), "pair_pos"),
                                  _stream(counts.device))
    _check("moe_dispatch_noalloc", st)


def expert_gate_up(desc, x, weights, offsets, sorted_pair, h, ws=None):
    ws = alloc_workspace(desc, CALL_GATE_UP, offsets.device) if ws is None else ws
    st = lib.moe_expert_gate_up(ctypes.byref(desc), _ptr(x, _act(desc), (desc.T, desc.d), "x"),
                                ctypes.byref(weights),
                                _ptr(offsets, torch.int32, (desc.E + 1,), "offsets"),
                                _ptr(sorted_pair, torch.int32, (desc.T * desc.k,), "sorted_pair"),
                                _ptr(h, _act(desc), ((desc.k + desc.S) * desc.T, desc.F), "h"),
                                _ptr(ws, torch.uint8, None, "ws"), ws.numel(),
                                _stream(offsets.device))
    _check("moe_expert_gate_up", st)


def expert_down(desc, weights, offsets, h, y_routed, y_shared, ws=None):
    ws = alloc_workspace(desc, CALL_DOWN, offsets.device) if ws is None else ws
    T, d, k, S = desc.T, desc.d, desc.k, desc.S
    st = lib.moe_expert_down(ctypes.byref(desc), ctypes.byref(weights),
                             _ptr(offsets, torch.int32, (desc.E + 1,), "offsets"),
                             _ptr(h, _act(desc), ((k + S) * T, desc.F), "h"),
                             _ptr(y_routed, _act(desc), (T * k, d), "y_routed"),
                             _ptr(y_shared, _act(desc), (S, T, d), "y_shared"),
                             _ptr(ws, torch.uint8, None, "ws"), ws.numel(),
                             _stream(offsets.device))
    _check("moe_expert_down", st)


def _marks(events, n=2):
    if len(events) != n:
        raise ValueError(f"{n} events are needed")
    arr = (ctypes.c_void_p * n)(*[e.cuda_event for e in events])
    return arr


def expert_gate_up_marked(desc, x, weights, offsets, sorted_pair, h, events, ws=None):
    """moe_expert_gate_up recording events[0..1] (torch.cuda.Event, created
    with enable_timing=True and recorded once beforehand) after the tile
    plan and after the GEMM kernel."""
    ws = alloc_workspace(desc, CALL_GATE_UP, offsets.device) if ws is None else ws
    st = lib.moe_expert_gate_up_marked(
        ctypes.byref(desc), _ptr(x, _act(desc), (desc.T, desc.d), "x"), ctypes.byref(weights),
        _ptr(offsets, torch.int32, (desc.E + 1,), "offsets"),
        _ptr(sorted_pair, torch.int32, (desc.T * desc.k,), "sorted_pair"),
        _ptr(h, _act(desc), ((desc.k + desc.S) * desc.T, desc.F), "h"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _marks(events), _stream(offsets.device))
    _check("moe_expert_gate_up_marked", st)


def expert_down_marked(desc, weights, offsets, h, y_routed, y_shared, events, ws=None):
    """moe_expert_down with the same two marks as expert_gate_up_marked."""
    ws = alloc_workspace(desc, CALL_DOWN, offsets.device) if ws is None else ws
    T, d, k, S = desc.T, desc.d, desc.k, desc.S
    st = lib.moe_expert_down_marked(
        ctypes.byref(desc), ctypes.byref(weights),
        _ptr(offsets, torch.int32, (desc.E + 1,), "offsets"),
        _ptr(h, _act(desc), ((k + S) * T, desc.F), "h"),
        _ptr(y_routed, _act(desc), (T * k, d), "y_routed"),
        _ptr(y_shared, _act(desc), (S, T, d), "y_shared"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _marks(events), _stream(offsets.device))
    _check("moe_expert_down_marked", st)


def expert_ffn(desc, x, weights, offsets, sorted_pair, y_routed, y_shared, ws=None):
    ws = alloc_workspace(desc, CALL_EXPERT_FFN, offsets.device) if ws is None else ws
    T, d, k, S = desc.T, desc.d, desc.k, desc.S
    st = lib.moe_expert_ffn(ctypes.byref(desc), _ptr(x, _act(desc), (T, d), "x"), ctypes.byref(weights),
                            _ptr(offsets, torch.int32, (desc.E + 1,), "offsets"),
                            _ptr(sorted_pair, torch.int32, (desc.T * desc.k,), "sorted_pair"),
                            _ptr(y_routed, _act(desc), (T * k, d), "y_routed"),
                            _ptr(y_shared, _act(desc), (S, T, d), "y_shared"),
                            _ptr(ws, torch.uint8, None, "ws"), ws.numel(),
                            _stream(offsets.device))
    _check("moe_expert_ffn", st)


def combine(desc, y_routed, y_shared, gates, pair_pos, y):
    T, d, k, S = desc.T, desc.d, desc.k, desc.S
    st = lib.moe_combine(ctypes.byref(desc), _ptr(y_routed, _act(desc), (T * k, d), "y_routed"),
                         _ptr(y_shared, _act(desc), (S, T, d), "y_shared"),
                         _ptr(gates, torch.float32, (T, k + S), "gates"),
                         _ptr(pair_pos, torch.int32, (T * k,), "pair_pos"),
                         _ptr(y, _act(desc), (T, d), "y"), _stream(y.device))
    _check("moe_combine", st)


def bias_update(desc, counts, gamma, bias):
    st = lib.moe_bias_update(ctypes.byref(desc), _ptr(counts, torch.int32, (desc.E,), "counts"),
                             ctypes.c_float(gamma), _ptr(bias, torch.float32, (desc.E,), "bias"),
                             _stream(bias.device))
    _check("moe_bias_update", st)


def forward(desc, x, weights, bias, gamma, y, routing=None, ws=None, events=None):
    """moe_forward.  ``routing`` is an optional dict of output tensors with
    keys topk_idx, gates, margin, counts, offsets, sorted_pair, pair_pos.
    With ``events`` (7 torch.cuda.Event, enable_timing=True, each recorded
    once beforehand) it calls moe_forward_marked, which records them after
    the router, dispatch, tile plan, gate/up GEMM, down GEMM, combine and
    bias update."""
    ws = alloc_workspace(desc, CALL_FORWARD, bias.device) if ws is None else ws
    T, d, k, S, E = desc.T, desc.d, desc.k, desc.S, desc.E
    r = None
    if routing is not None:
        shapes = {"topk_idx": ((T, k), torch.int32), "gates": ((T, k + S), torch.float32),
                  "margin": ((T,), torch.float32), "counts": ((E,), torch.int32),
                  "offsets": ((E + 1,), torch.int32), "sorted_pair": ((T * k,), torch.int32),
                  "pair_pos": ((T * k,), torch.int32)}
        r = Routing()
        for key, (shp, dt) in shapes.items():
            setattr(r, key, _ptr(routing.get(key), dt, shp, key))
    args = (ctypes.byref(desc), _ptr(x, _act(desc), (T, d), "x"), ctypes.byref(weights),
            _ptr(bias, torch.float32, (E,), "bias"), ctypes.c_float(gamma),
            _ptr(y, _act(desc), (T, d), "y"), ctypes.byref(r) if r is not None else None,
            _ptr(ws, torch.uint8, None, "ws"), ws.numel())
    if events is None:
        st = lib.moe_forward(*args, _stream(bias.device))
        _check("moe_forward", st)
    else:
        st = lib.moe_forward_marked(*args, _marks(events, 7), _stream(bias.device))
        _check("moe_forward_marked", st)

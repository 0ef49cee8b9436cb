"""Python binding of libmoe_ffn (the routed low-bit expert FFN for MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/moe_ffn.h.  PyTorch provides device memory
(tensors' data pointers) and the current stream.  There is no fallback: if the
library is not built, or a call fails, an exception is raised.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ffn.so")

Q2_64 = 1
Q4_32 = 2
F32 = 0
BF16 = 1
QK = {Q2_64: 64, Q4_32: 32}

# Functions the header declares (the CPU test checks that each is exported).
EXPORTS = ["moe_expert_blob_bytes", "moe_expert_workspace_bytes", "moe_layer_workspace_bytes", "moe_route_topk",
           "moe_expert_ffn", "moe_layer_forward", "moe_layer_forward_ex", "moe_router_logits", "moe_layer_forward_timed", "moe_dequant_matrix", "moe_validate_table",
           "moe_layer_forward_noalloc", "moe_max_tokens", "moe_workspace_check", "moe_debug_set_wait_limit", "moe_status_str", "moe_last_error"]


class MoeError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{status_str(status)}: {detail}")
        self.status = status


class ExpertDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ff", ctypes.c_int32), ("qtype", ctypes.c_int32),
                ("zero_point", ctypes.c_float), ("act", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("expert", ExpertDesc), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("shared_ff", ctypes.c_int32)]


class Router(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("in_scale", ctypes.c_void_p), ("norm", ctypes.c_int32),
                ("eps", ctypes.c_float)]


class LayerOpts(ctypes.Structure):
    _fields_ = [("router", ctypes.POINTER(Router)), ("logits_out", ctypes.c_void_p), ("down_scale", ctypes.c_void_p),
                ("ids_in", ctypes.c_void_p), ("w_in", ctypes.c_void_p)]


ACT_SWIGLU = 0
ACT_GEGLU_TANH = 1


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.moe_expert_blob_bytes.restype = sz
        L.moe_expert_blob_bytes.argtypes = [ctypes.POINTER(ExpertDesc)]
        L.moe_expert_workspace_bytes.restype = sz
        L.moe_expert_workspace_bytes.argtypes = [ctypes.POINTER(ExpertDesc), i32]
        L.moe_layer_workspace_bytes.restype = sz
        L.moe_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), i32]
        L.moe_route_topk.restype = ctypes.c_int
        L.moe_route_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [ctypes.POINTER(ExpertDesc), vp, vp, i32, i32, vp, vp, sz, vp]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, sz,
                                        vp]
        L.moe_layer_forward_ex.restype = ctypes.c_int
        L.moe_layer_forward_ex.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerOpts), vp, vp, vp, i32, vp,
                                           i32, vp, vp, vp, vp, sz, vp]
        L.moe_router_logits.restype = ctypes.c_int
        L.moe_router_logits.argtypes = [ctypes.POINTER(Router), i32, i32, vp, i32, i32, vp, vp]
        L.moe_layer_forward_timed.restype = ctypes.c_int
        L.moe_layer_forward_timed.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp, i32, vp, i32, vp, vp, vp, vp,
                                              sz, vp, vp, i32, ctypes.POINTER(i32)]
        L.moe_dequant_matrix.restype = ctypes.c_int
        L.moe_dequant_matrix.argtypes = [ctypes.POINTER(ExpertDesc), vp, i32, vp, vp]
        L.moe_validate_table.restype = ctypes.c_int
        L.moe_validate_table.argtypes = [vp, i32, vp]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, vp, i32, vp, i32, vp, vp, vp, vp]
        L.moe_max_tokens.restype = ctypes.c_int64
        L.moe_max_tokens.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_workspace_check.restype = ctypes.c_int
        L.moe_workspace_check.argtypes = [ctypes.POINTER(LayerDesc), vp, sz, vp]
        L.moe_debug_set_wait_limit.restype = None
        L.moe_debug_set_wait_limit.argtypes = [ctypes.c_int64]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        _lib = L
    return _lib


def status_str(s):
    return lib().moe_status_str(s).decode()


def _check(status):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def expert_desc(hidden, ff, qtype, zero_point, act=ACT_SWIGLU):
    return ExpertDesc(hidden, ff, qtype, float(zero_point), act)


def layer_desc(hidden, ff, qtype, zero_point, n_experts, top_k, renormalize=True, shared_ff=0, act=ACT_SWIGLU):
    return LayerDesc(expert_desc(hidden, ff, qtype, zero_point, act), n_experts, top_k, int(bool(renormalize)),
                     shared_ff)


def router(weight, in_scale=None, norm=False, eps=1e-6):
    """weight: bf16 CUDA tensor [E][H]; in_scale: fp32 CUDA tensor [H] or None.
    The returned struct holds references to both tensors, so their memory
    stays allocated while it is in use."""
    _need_cuda(weight, in_scale)
    rt = Router(weight.data_ptr(), in_scale.data_ptr() if in_scale is not None else None, int(bool(norm)), float(eps))
    rt._tensors = (weight, in_scale)
    return rt


def expert_blob_bytes(desc):
    return int(lib().moe_expert_blob_bytes(ctypes.byref(desc)))


def layer_workspace_bytes(desc, T):
    return int(lib().moe_layer_workspace_bytes(ctypes.byref(desc), T))


def expert_workspace_bytes(desc, T):
    return int(lib().moe_expert_workspace_bytes(ctypes.byref(desc), T))


def workspace(nbytes, device):
    """A workspace buffer, zeroed once as the library requires."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which temporaries are allocated (and zeroed) on the launch
    stream, so that the kernels see them ready and the caching allocator does
    not hand them out while the call runs."""
    import contextlib
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _xdtype(x):
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float32:
        return F32
    raise TypeError("activations must be torch.bfloat16 or torch.float32")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


def route_topk(logits, k, renormalize=True, ids=None, weights=None, stream=None):
    _need_cuda(logits)
    T, E = logits.shape
    with _on(stream):
        if ids is None:
            ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        if weights is None:
            weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(ids), _ptr(weights),
                                _stream(stream)))
    return ids, weights


def expert_ffn(desc, blob, x, y=None, ws=None, stream=None):
    _need_cuda(blob, x)
    T = x.shape[0]
    need = expert_workspace_bytes(desc, T)
    with _on(stream):
        if y is None:
            y = torch.empty((T, desc.hidden), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = workspace(need, x.device)
    _check(lib().moe_expert_ffn(ctypes.byref(desc), _ptr(blob), _ptr(x), _xdtype(x), T, _ptr(y), _ptr(ws),
                                ws.numel(), _stream(stream)))
    return y


def layer_forward(desc, table, x, logits, shared=None, y=None, ids=None, weights=None, ws=None, stream=None):
    """table: int64 CUDA tensor of E blob addresses (blob.data_ptr())."""
    _need_cuda(table, x, logits, shared, y, ids, weights, ws)
    T = x.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((T, desc.expert.hidden), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = workspace(layer_workspace_bytes(desc, T), x.device)
    _check(lib().moe_layer_forward(ctypes.byref(desc), _ptr(table), _ptr(shared), _ptr(x), _xdtype(x),
                                   _ptr(logits), T, _ptr(y), _ptr(ids), _ptr(weights), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return y


def router_logits(rt, E, x, logits=None, stream=None):
    """rt: a Router (see router()); x [T][H]; returns logits [T][E] fp32."""
    _need_cuda(x, logits)
    T, H = x.shape
    with _on(stream):
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_logits(ctypes.byref(rt), E, H, _ptr(x), _xdtype(x), T, _ptr(logits), _stream(stream)))
    return logits


def layer_forward_ex(desc, table, x, logits=None, shared=None, rt=None, logits_out=None, down_scale=None,
                     ids_in=None, w_in=None, y=None, ids=None, weights=None, ws=None, stream=None):
    """The layer with options: rt (a Router: logits computed inside the call),
    down_scale [E], or caller-supplied routing ids_in / w_in [T][k]."""
    _need_cuda(table, x, logits, shared, logits_out, down_scale, ids_in, w_in, y, ids, weights, ws)
    T = x.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((T, desc.expert.hidden), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = workspace(layer_workspace_bytes(desc, T), x.device)
    opts = LayerOpts(ctypes.pointer(rt) if rt is not None else None, logits_out.data_ptr() if logits_out is not None
                     else None, down_scale.data_ptr() if down_scale is not None else None,
                     ids_in.data_ptr() if ids_in is not None else None, w_in.data_ptr() if w_in is not None else None)
    _check(lib().moe_layer_forward_ex(ctypes.byref(desc), ctypes.byref(opts), _ptr(table), _ptr(shared), _ptr(x),
                                      _xdtype(x), _ptr(logits), T, _ptr(y), _ptr(ids), _ptr(weights), _ptr(ws),
                                      ws.numel(), _stream(stream)))
    return y


def layer_forward_timed(desc, table, x, logits, events, shared=None, y=None, ids=None, weights=None, ws=None,
                        stream=None):
    """layer_forward that also records `events` (torch.cuda.Event objects with
    timing, each already recorded once so that its HIP event exists) at the
    kernel boundaries on the launch stream.  Returns (y, number of kernels)."""
    _need_cuda(table, x, logits, shared, y, ids, weights, ws)
    T = x.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((T, desc.expert.hidden), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = workspace(layer_workspace_bytes(desc, T), x.device)
    handles = [e.cuda_event for e in events]
    if any(h == 0 for h in handles):
        raise ValueError("record every event once before passing it (torch creates HIP events lazily)")
    arr = (ctypes.c_void_p * max(1, len(handles)))(*handles)
    nk = ctypes.c_int32(0)
    _check(lib().moe_layer_forward_timed(ctypes.byref(desc), _ptr(table), _ptr(shared), _ptr(x), _xdtype(x),
                                         _ptr(logits), T, _ptr(y), _ptr(ids), _ptr(weights), _ptr(ws), ws.numel(),
                                         _stream(stream), arr, len(handles), ctypes.byref(nk)))
    return y, nk.value


def dequant_matrix(desc, blob, m, stream=None):
    _need_cuda(blob)
    rows, cols = [(desc.ff, desc.hidden), (desc.ff, desc.hidden), (desc.hidden, desc.ff)][m]
    with _on(stream):
        out = torch.empty((rows, cols), dtype=torch.float32, device=blob.device)
    _check(lib().moe_dequant_matrix(ctypes.byref(desc), _ptr(blob), m, _ptr(out), _stream(stream)))
    return out


def layer_forward_noalloc(desc, table, x, logits, shared=None, y=None, ids=None, weights=None, stream=None):
    """layer_forward (T <= 8) with the library's own device array as workspace."""
    _need_cuda(table, x, logits, shared, y, ids, weights)
    T = x.shape[0]
    with _on(stream):
        if y is None:
            y = torch.empty((T, desc.expert.hidden), dtype=torch.float32, device=x.device)
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(desc), _ptr(table), _ptr(shared), _ptr(x), _xdtype(x),
                                           _ptr(logits), T, _ptr(y), _ptr(ids), _ptr(weights), _stream(stream)))
    return y


def max_tokens(desc):
    return int(lib().moe_max_tokens(ctypes.byref(desc)))


def workspace_check(desc, ws, stream=None):
    """Raises MoeError (MOE_ERR_DEVICE) if a call on `ws` failed; the library
    then has zero-filled the workspace's shared region."""
    _need_cuda(ws)
    _check(lib().moe_workspace_check(ctypes.byref(desc), _ptr(ws), ws.numel(), _stream(stream)))


def debug_set_wait_limit(polls):
    """Bound of every kernel wait in polls; 0 forces every wait to give up; < 0 restores the default."""
    lib().moe_debug_set_wait_limit(int(polls))


def validate_table(table, stream=None):
    _need_cuda(table)
    _check(lib().moe_validate_table(_ptr(table), table.numel(), _stream(stream)))

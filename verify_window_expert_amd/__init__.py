"""Python binding of libstrata_window.so, the verify-window MoE layer for gfx950.

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream. The entry points keep the C
names (strata_window_route / strata_window_moe / strata_window_head); their contracts
are in include/strata_window.h. If the library has not been built, every call raises.
"""
import ctypes
import os

import torch

from .build import LIB_PATH, build  # noqa: F401  (build() compiles the library)

STRATA_OK, STRATA_EINVAL, STRATA_EUNSUPPORTED, STRATA_EHIP = 0, -1, -2, -3
STRATA_F32, STRATA_BF16 = 0, 1
STRATA_ROUTE_RENORM = 1
MAX_ROWS, MAX_TOPK, MAX_EXPERTS = 8, 8, 256
NOALLOC_SCRATCH_BYTES = 2 << 20
WS_COUNTER_BYTES = 4096


class StrataError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"strata_window status {status}: {message}")
        self.status = status


class CQMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("n_mat", ctypes.c_int32),
                ("mat_stride_codes", ctypes.c_int64), ("mat_stride_meta", ctypes.c_int64)]


class CRouteOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_idx", "topk_w", "n_active", "active", "offsets", "entry_row", "entry_w", "row_mask",
                 "entry_pos", "row_w")]


class CLayer(ctypes.Structure):
    _fields_ = [("gate_w", ctypes.c_void_p), ("logit_bias", ctypes.c_void_p)] + \
        [(n, CQMat) for n in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down")] + [("route", CRouteOut)]


_lib = None


def library():
    """The loaded library (ctypes.CDLL). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: call verify_window_expert_amd.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.strata_window_route.argtypes = [P, P, I, I, I, P, P, I, I, I, ctypes.POINTER(CRouteOut), P, S, P]
        L.strata_window_route.restype = I
        L.strata_window_moe.argtypes = [P, P, I, I, I, I] + [ctypes.POINTER(CQMat)] * 6 + \
            [ctypes.POINTER(CRouteOut), I, I, P, P, P, P, S, P]
        L.strata_window_moe.restype = I
        L.strata_window_head.argtypes = [P, P, I, I, I, ctypes.POINTER(CQMat), I, P, P, P, S, P]
        L.strata_window_head.restype = I
        L.strata_window_layer.argtypes = [P, P, I, I, I, I, P, P, I] + [ctypes.POINTER(CQMat)] * 6 + \
            [I, I, ctypes.POINTER(CRouteOut), P, P, P, P, S, P]
        L.strata_window_layer.restype = I
        L.strata_window_layer_noalloc.argtypes = [P, P, I, I, I, I, P, P, I] + [ctypes.POINTER(CQMat)] * 6 + \
            [I, I, ctypes.POINTER(CRouteOut), P, P, P, P]
        L.strata_window_layer_noalloc.restype = I
        L.strata_window_accept.argtypes = [P, P, I, I, I, P, P, P, P, P]
        L.strata_window_accept.restype = I
        L.strata_window_sample.argtypes = [P, P, I, I, P, P, P, P, S, P]
        L.strata_window_sample.restype = I
        L.strata_window_tier.argtypes = [P, P, I, P, ctypes.c_float, P, I, ctypes.c_float, P, P, P]
        L.strata_window_tier.restype = I
        L.strata_window_stack.argtypes = [P, P, I, I, I, I, I, I, I, I, ctypes.POINTER(CLayer),
                                          ctypes.POINTER(CQMat), I, P, P, P, P, P, S, P]
        L.strata_window_stack.restype = I
        L.strata_window_stream_read.argtypes = [P, P, S, P, ctypes.c_uint32, P]
        L.strata_window_stream_read.restype = I
        L.strata_window_workspace.argtypes = [I, I, I, I, I, I, I]
        L.strata_window_workspace.restype = S
        L.strata_window_last_error.argtypes = []
        L.strata_window_last_error.restype = ctypes.c_char_p
        L.strata_window_abi_version.argtypes = []
        L.strata_window_abi_version.restype = I
        _lib = L
    return _lib


def _check(status):
    if status != STRATA_OK:
        raise StrataError(status, library().strata_window_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _events(prof):
    """ctypes array of hipEvent_t handles (ints) for the prof_events argument, or None."""
    if prof is None:
        return None
    arr = (ctypes.c_void_p * len(prof))(*[p or None for p in prof])
    return arr


def _x_dtype(x):
    if x.dtype == torch.float32:
        return STRATA_F32
    if x.dtype == torch.bfloat16:
        return STRATA_BF16
    raise TypeError("activations must be float32 or bfloat16")


def _need(t, name, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _need_buf(t, name, dtype, numel):
    """A caller-supplied device tensor the kernels read or write: contiguous, of dtype, with
    at least numel elements. The library sees only its pointer, so a short buffer would be
    accessed past its end; it is refused here, before anything is enqueued."""
    _need(t, name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    return t


def _need_x(x):
    _need(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [rows, hidden]")
    _x_dtype(x)
    return x.shape


def _need_router(gate_w, bias, hidden):
    _need(gate_w, "gate_w")
    if gate_w.dtype != torch.float32 or gate_w.dim() != 2 or gate_w.shape[1] != hidden:
        raise ValueError(f"gate_w must be float32 [n_experts, {hidden}]")
    if bias is not None:
        _need_buf(bias, "bias", torch.float32, gate_w.shape[0])
    return gate_w.shape[0]


def _need_route(route, rows, n_experts, top_k, name="route"):
    if not isinstance(route, RouteOut):
        raise TypeError(f"{name} must be a RouteOut")
    if (route.rows, route.n_experts, route.top_k) != (rows, n_experts, top_k):
        raise ValueError(f"{name} was made for rows {route.rows}, experts {route.n_experts}, top_k {route.top_k}; "
                         f"the call has {rows}, {n_experts}, {top_k}")
    return route


def _ws_bytes(ws):
    _need(ws, "ws")
    return ws.numel() * ws.element_size()


def _need_outs(x, rows, hidden, residual, out, x_next):
    n = rows * hidden
    if residual is not None:
        _need_buf(residual, "residual", x.dtype, n)
    if out is not None:
        _need_buf(out, "out", torch.float32, n)
    if x_next is not None:
        _need_buf(x_next, "x_next", torch.bfloat16, n)


class QMat:
    """Device view of one block-quantized matrix, or n_mat stacked ones.

    codes: uint8 tensor [n_mat, rows*cols*bits/8] in the documented chunk layout;
    meta: int32 (scale | min << 16) or int16 (8-bit scale) tensor [n_mat, rows*cols/32].
    """

    def __init__(self, codes, meta, rows, cols, bits):
        self.codes = _need(codes, "codes")
        self.meta = _need(meta, "meta")
        self.rows, self.cols, self.bits = int(rows), int(cols), int(bits)
        self.n_mat = codes.shape[0] if codes.dim() == 2 else 1
        # every matrix's codes and per-block meta words must be there in full
        need_c = self.rows * self.cols * self.bits // 8
        need_m = self.rows * (self.cols // 32) * (2 if self.bits == 8 else 4)
        if codes.numel() * codes.element_size() < self.n_mat * need_c or \
                meta.numel() * meta.element_size() < self.n_mat * need_m:
            raise ValueError(f"codes/meta hold less than {self.n_mat} matrices of {self.rows} x {self.cols} "
                             f"at {self.bits} bits")

    def c(self):
        per_c = self.codes.numel() // self.n_mat
        per_m = self.meta.numel() // self.n_mat
        return CQMat(self.codes.data_ptr(), self.meta.data_ptr(), self.rows, self.cols, self.bits,
                     self.n_mat, per_c, per_m)


def upload_qmat(codes, meta, rows, cols, bits, device="cuda"):
    """QMat from NumPy arrays (codes uint8, meta uint32/uint16) copied to the device."""
    import numpy as np
    c = torch.from_numpy(np.ascontiguousarray(codes)).to(device)
    m = np.ascontiguousarray(meta)
    m = torch.from_numpy(m.view(np.int32) if m.dtype == np.uint32 else m.view(np.int16)).to(device)
    if c.dim() == 1:
        c, m = c.unsqueeze(0), m.unsqueeze(0)
    return QMat(c, m, rows, cols, bits)


class RouteOut:
    """Device tensors of one window's routing (see strata_route_out)."""

    def __init__(self, rows, n_experts, top_k, device="cuda"):
        i32 = dict(dtype=torch.int32, device=device)
        A = min(n_experts, rows * top_k) + 1
        ent = rows * top_k + rows
        self.rows, self.n_experts, self.top_k = rows, n_experts, top_k
        self.topk_idx = torch.empty(rows * top_k, **i32)
        self.topk_w = torch.empty(rows * top_k, dtype=torch.float32, device=device)
        self.n_active = torch.empty(4, **i32)
        self.active = torch.empty(A, **i32)
        self.offsets = torch.empty(A + 1, **i32)
        self.entry_row = torch.empty(ent, **i32)
        self.entry_w = torch.empty(ent, dtype=torch.float32, device=device)
        self.row_mask = torch.empty(n_experts + 1, dtype=torch.uint8, device=device)
        self.entry_pos = torch.empty(ent, **i32)
        self.row_w = torch.empty(rows * (top_k + 1), dtype=torch.float32, device=device)

    def c(self):
        return CRouteOut(*(t.data_ptr() for t in (self.topk_idx, self.topk_w, self.n_active, self.active,
                                                   self.offsets, self.entry_row, self.entry_w, self.row_mask,
                                                   self.entry_pos, self.row_w)))

    def host(self):
        """Copy to the host as NumPy arrays, cut to the active length."""
        n = int(self.n_active[0].item())
        off = self.offsets[:n + 1].cpu().numpy()
        e = int(off[-1])
        R, K = self.rows, self.top_k
        return dict(topk_idx=self.topk_idx[:R * K].reshape(R, K).cpu().numpy(),
                    topk_w=self.topk_w[:R * K].reshape(R, K).cpu().numpy(),
                    n_active=n, active=self.active[:n].cpu().numpy(), offsets=off,
                    entry_row=self.entry_row[:e].cpu().numpy(), entry_w=self.entry_w[:e].cpu().numpy(),
                    row_mask=self.row_mask[:self.n_experts + 1].cpu().numpy(),
                    entry_pos=self.entry_pos[:e].cpu().numpy(),
                    row_w=self.row_w[:R * (K + 1)].reshape(R, K + 1).cpu().numpy())


def workspace_bytes(which, rows, hidden, ffn=0, n_experts=0, top_k=0, vocab=0):
    return library().strata_window_workspace(which, rows, hidden, ffn, n_experts, top_k, vocab)


def workspace(nbytes, device="cuda"):
    """A device workspace of at least nbytes (the library needs its contents in no
    particular state; it is zero-filled here only so that runs start alike)."""
    return torch.zeros(max(int(nbytes), WS_COUNTER_BYTES), dtype=torch.uint8, device=device)


def strata_window_route(x, gate_w, bias, top_k, renorm=False, out=None, ws=None, stream=None, prof=None):
    """Router, softmax, top-k and grouping of one window. Returns a RouteOut.
    prof: None or [start, end] hipEvent_t handles recorded around the kernel."""
    rows, hidden = _need_x(x)
    E = _need_router(gate_w, bias, hidden)
    out = RouteOut(rows, E, top_k, x.device) if out is None else _need_route(out, rows, E, top_k, "out")
    if ws is None:
        ws = workspace(workspace_bytes(0, rows, hidden, n_experts=E), x.device)
    ro = out.c()
    _check(library().strata_window_route(_stream(stream), _ptr(x), _x_dtype(x), rows, hidden, _ptr(gate_w),
                                         _ptr(bias), E, top_k, STRATA_ROUTE_RENORM if renorm else 0,
                                         ctypes.byref(ro), _ptr(ws), _ws_bytes(ws), _events(prof)))
    return out


def strata_window_moe(x, gate, up, down, sh_gate, sh_up, sh_down, route, residual=None, out=None,
                      x_next=None, ws=None, stream=None, prof=None):
    """Experts of one window. Returns out [rows, hidden] float32 (x_next filled if given).
    prof: None or [gate/up start, gate/up end, down start, down end] hipEvent_t handles."""
    rows, hidden = _need_x(x)
    ffn = gate.rows
    _need_route(route, rows, route.n_experts, route.top_k)
    _need_outs(x, rows, hidden, residual, out, x_next)
    if out is None:
        out = torch.empty(rows, hidden, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(workspace_bytes(1, rows, hidden, ffn, route.n_experts, route.top_k), x.device)
    qs = [q.c() for q in (gate, up, down, sh_gate, sh_up, sh_down)]
    ro = route.c()
    _check(library().strata_window_moe(_stream(stream), _ptr(x), _x_dtype(x), rows, hidden, ffn,
                                       *[ctypes.byref(q) for q in qs], ctypes.byref(ro), route.n_experts,
                                       route.top_k, _ptr(residual), _ptr(out), _ptr(x_next), _ptr(ws),
                                       _ws_bytes(ws), _events(prof)))
    return out


def strata_window_layer(x, gate_w, bias, top_k, gate, up, down, sh_gate, sh_up, sh_down, renorm=False,
                        route=None, residual=None, out=None, x_next=None, ws=None, stream=None, prof=None):
    """The whole layer of one window in one call (router, then experts). Returns
    (out [rows, hidden] float32, the window's RouteOut); x_next filled if given.
    prof: None or [router start, end, gate/up start, end, down start, end] handles."""
    rows, hidden = _need_x(x)
    E = _need_router(gate_w, bias, hidden)
    ffn = gate.rows
    route = RouteOut(rows, E, top_k, x.device) if route is None else _need_route(route, rows, E, top_k)
    _need_outs(x, rows, hidden, residual, out, x_next)
    if out is None:
        out = torch.empty(rows, hidden, dtype=torch.float32, device=x.device)
    if ws is None:
        ws = workspace(workspace_bytes(3, rows, hidden, ffn, E, top_k), x.device)
    qs = [q.c() for q in (gate, up, down, sh_gate, sh_up, sh_down)]
    ro = route.c()
    _check(library().strata_window_layer(_stream(stream), _ptr(x), _x_dtype(x), rows, hidden, ffn, _ptr(gate_w),
                                         _ptr(bias), STRATA_ROUTE_RENORM if renorm else 0,
                                         *[ctypes.byref(q) for q in qs], E, top_k, ctypes.byref(ro),
                                         _ptr(residual), _ptr(out), _ptr(x_next), _ptr(ws), _ws_bytes(ws),
                                         _events(prof)))
    return out, route


def strata_window_layer_noalloc(x, gate_w, bias, top_k, gate, up, down, sh_gate, sh_up, sh_down, renorm=False,
                                route=None, residual=None, out=None, x_next=None, stream=None, prof=None):
    """strata_window_layer with the library's fixed per-GPU scratch array as its workspace
    (the C call allocates nothing; pass route and out to allocate nothing here either).
    Returns (out, route) as strata_window_layer."""
    rows, hidden = _need_x(x)
    E = _need_router(gate_w, bias, hidden)
    route = RouteOut(rows, E, top_k, x.device) if route is None else _need_route(route, rows, E, top_k)
    _need_outs(x, rows, hidden, residual, out, x_next)
    if out is None:
        out = torch.empty(rows, hidden, dtype=torch.float32, device=x.device)
    qs = [q.c() for q in (gate, up, down, sh_gate, sh_up, sh_down)]
    ro = route.c()
    _check(library().strata_window_layer_noalloc(_stream(stream), _ptr(x), _x_dtype(x), rows, hidden, gate.rows,
                                                 _ptr(gate_w), _ptr(bias), STRATA_ROUTE_RENORM if renorm else 0,
                                                 *[ctypes.byref(q) for q in qs], E, top_k, ctypes.byref(ro),
                                                 _ptr(residual), _ptr(out), _ptr(x_next), _events(prof)))
    return out, route


def strata_window_stack(x, layers, top_k, head=None, renorm=False, routes=None, logits=True, argmax=None,
                        out=None, x_final=None, ws=None, stream=None, prof=None):
    """One window through a stack of MoE layers (residual between layers) and, with head,
    the 8-bit head (see strata_window_stack). layers: a sequence of
    (gate_w, bias or None, gate, up, down, sh_gate, sh_up, sh_down) with QMat matrices;
    routes: None (one RouteOut shared by all layers) or one RouteOut per layer.
    Returns (x_final bf16 [rows, hidden], the routes list, logits or None, argmax or None);
    out (the last layer's float output) is filled if given."""
    rows, hidden = _need_x(x)
    n = len(layers)
    if n < 1:
        raise ValueError("at least one layer")
    E = layers[0][0].shape[0]
    ffn = layers[0][2].rows
    if routes is None:
        shared = RouteOut(rows, E, top_k, x.device)
        routes = [shared] * n
    if len(routes) != n:
        raise ValueError("one RouteOut per layer, or None")
    cl = (CLayer * n)()
    for i, (gw, bias, *mats) in enumerate(layers):
        if _need_router(gw, bias, hidden) != E:
            raise ValueError(f"layer {i} has {gw.shape[0]} experts, layer 0 {E}")
        _need_route(routes[i], rows, E, top_k, f"routes[{i}]")
        cl[i] = CLayer(gw.data_ptr(), None if bias is None else bias.data_ptr(), *[q.c() for q in mats],
                       routes[i].c())
    if x_final is None:
        x_final = torch.empty(rows, hidden, dtype=torch.bfloat16, device=x.device)
    _need_buf(x_final, "x_final", torch.bfloat16, rows * hidden)
    if out is not None:
        _need_buf(out, "out", torch.float32, rows * hidden)
    lg = am = None
    V = 0
    if head is not None:
        V = head.rows
        lg = torch.empty(rows, V, dtype=torch.float32, device=x.device) if logits is True else logits
        if lg is False:
            lg = None
        am = torch.empty(max(rows, 4), dtype=torch.int32, device=x.device) if argmax is None else argmax
        if lg is not None:
            _need_buf(lg, "logits", torch.float32, rows * V)
        _need_buf(am, "argmax", torch.int32, rows)
    if ws is None:
        ws = workspace(workspace_bytes(4, rows, hidden, ffn, E, top_k, V), x.device)
    hq = head.c() if head is not None else None
    _check(library().strata_window_stack(_stream(stream), _ptr(x), _x_dtype(x), rows, hidden, ffn, E, top_k,
                                         STRATA_ROUTE_RENORM if renorm else 0, n, cl,
                                         None if hq is None else ctypes.byref(hq), V, _ptr(lg), _ptr(am),
                                         _ptr(out), _ptr(x_final), _ptr(ws), _ws_bytes(ws), _events(prof)))
    return x_final, routes, lg, (None if am is None else am[:rows])


def strata_window_head(x, head, logits=True, argmax=None, ws=None, stream=None, prof=None):
    """Head GEMV and argmax of one window. Returns (logits or None, argmax int32 [rows])."""
    rows, hidden = _need_x(x)
    V = head.rows
    lg = torch.empty(rows, V, dtype=torch.float32, device=x.device) if logits is True else logits
    if lg is False:
        lg = None
    am = torch.empty(max(rows, 4), dtype=torch.int32, device=x.device) if argmax is None else argmax
    if lg is not None:
        _need_buf(lg, "logits", torch.float32, rows * V)
    _need_buf(am, "argmax", torch.int32, rows)
    if ws is None:
        ws = workspace(workspace_bytes(2, rows, hidden, vocab=V), x.device)
    q = head.c()
    _check(library().strata_window_head(_stream(stream), _ptr(x), _x_dtype(x), rows, hidden, ctypes.byref(q),
                                        V, _ptr(lg), _ptr(am), _ptr(ws), _ws_bytes(ws), _events(prof)))
    return lg, am[:rows]


def strata_window_accept(argmax, proposal=None, mtp=True, tokens=None, n_tokens=None, n_accepted=None,
                         stream=None, prof=None):
    """Greedy verification of the window's MTP proposals (see strata_window_accept).
    argmax: int32 [rows]; proposal: int32 [rows // 2] with mtp. Returns (tokens [n_slots, 2],
    n_tokens [n_slots], n_accepted [1]) int32 device tensors."""
    _need(argmax, "argmax")
    if argmax.dtype != torch.int32:
        raise TypeError("argmax must be int32")
    rows = argmax.numel()
    n_slots = rows // 2 if mtp else rows
    if mtp:
        _need(proposal, "proposal")
        if proposal.dtype != torch.int32:
            raise TypeError("proposal must be int32")
    if mtp:
        _need_buf(proposal, "proposal", torch.int32, n_slots)
    i32 = dict(dtype=torch.int32, device=argmax.device)
    tokens = torch.empty(n_slots, 2, **i32) if tokens is None else tokens
    n_tokens = torch.empty(n_slots, **i32) if n_tokens is None else n_tokens
    n_accepted = torch.empty(4, **i32) if n_accepted is None else n_accepted
    _need_buf(tokens, "tokens", torch.int32, 2 * n_slots)
    _need_buf(n_tokens, "n_tokens", torch.int32, n_slots)
    _need_buf(n_accepted, "n_accepted", torch.int32, 1)
    _check(library().strata_window_accept(_stream(stream), _ptr(argmax), rows, n_slots, int(bool(mtp)),
                                          _ptr(proposal) if mtp else None, _ptr(tokens), _ptr(n_tokens),
                                          _ptr(n_accepted), _events(prof)))
    return tokens, n_tokens, n_accepted


SAMPLE_PARAMS_BYTES = 24


def sample_params(rows, device="cuda"):
    """Device array of per-row sampling parameters (strata_sample_params) from a list of
    (temperature, top_k, top_p, min_p, seed) tuples, one per row."""
    import numpy as np
    dt = np.dtype([("temperature", "<f4"), ("top_k", "<i4"), ("top_p", "<f4"), ("min_p", "<f4"),
                   ("seed", "<u8")])
    assert dt.itemsize == SAMPLE_PARAMS_BYTES
    a = np.array([tuple(r) for r in rows], dtype=dt)
    return torch.from_numpy(a.view(np.uint8).copy()).to(device)


def strata_window_sample(logits, params, position, tokens=None, ws=None, stream=None, prof=None):
    """Sampled token per row (see strata_window_sample). logits: float32 [rows, vocab];
    params: sample_params(...) of the rows; position: int64 [rows]. Returns int32 [rows]."""
    _need(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be float32 [rows, vocab]")
    rows, vocab = logits.shape
    _need_buf(params, "params", torch.uint8, rows * SAMPLE_PARAMS_BYTES)
    _need_buf(position, "position", torch.int64, rows)
    tokens = torch.empty(max(rows, 4), dtype=torch.int32, device=logits.device) if tokens is None else tokens
    _need_buf(tokens, "tokens", torch.int32, rows)
    if ws is None:
        ws = workspace(workspace_bytes(5, rows, 0, vocab=vocab), logits.device)
    _check(library().strata_window_sample(_stream(stream), _ptr(logits), rows, vocab, _ptr(params), _ptr(position),
                                          _ptr(tokens), _ptr(ws), _ws_bytes(ws), _events(prof)))
    return tokens[:rows]


def strata_window_stream_read(src, sink, magic=0x9E3779B9, stream=None, prof=None):
    """A plain streaming read of the device tensor src (all its bytes; a nonzero multiple of
    16): the bandwidth yardstick. sink: a device tensor of at least 4 bytes, written only if
    the xor of the 16-byte words that one lane reads equals magic."""
    _need(src, "src"); _need(sink, "sink")
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _check(library().strata_window_stream_read(_stream(stream), _ptr(src), src.numel() * src.element_size(),
                                               _ptr(sink), int(magic) & 0xFFFFFFFF, _events(prof)))


def strata_window_tier(row_mask, counts, decay=1.0, resident=None, max_swaps=0, min_gain=1.5, swaps=None,
                       n_swaps=None, stream=None, prof=None):
    """Routing counts of a window (row_mask: uint8 [E + 1], e.g. RouteOut.row_mask; counts:
    float32 [E], updated in place) and, when resident (uint8 [E], updated in place) is
    given, one round of the adaptive tier. Returns (swaps [max_swaps, 2], n_swaps [1])
    int32 device tensors, or None when only counting."""
    _need(row_mask, "row_mask"); _need(counts, "counts")
    E = counts.numel()
    if counts.dtype != torch.float32 or row_mask.dtype != torch.uint8 or row_mask.numel() < E:
        raise TypeError("counts must be float32 [E] and row_mask uint8 [E + 1]")
    if resident is not None:
        _need_buf(resident, "resident", torch.uint8, E)
        i32 = dict(dtype=torch.int32, device=counts.device)
        swaps = torch.empty(max(max_swaps, 1), 2, **i32) if swaps is None else swaps
        n_swaps = torch.empty(4, **i32) if n_swaps is None else n_swaps
        _need_buf(swaps, "swaps", torch.int32, 2 * max_swaps)
        _need_buf(n_swaps, "n_swaps", torch.int32, 1)
    _check(library().strata_window_tier(_stream(stream), _ptr(row_mask), E, _ptr(counts), float(decay),
                                        _ptr(resident), int(max_swaps), float(min_gain), _ptr(swaps),
                                        _ptr(n_swaps), _events(prof)))
    return None if resident is None else (swaps, n_swaps)

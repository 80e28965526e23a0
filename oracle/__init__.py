"""TEST INFRASTRUCTURE ONLY: the CPU oracle of the batched verify-window MoE layer.

`oracle.c` is a plain scalar double-precision C implementation of the layer's
definition (Strata docs/BATCHING.md, "Several requests at once (batch slots)": the
opening paragraph and "Exactness"). This module builds it with gcc and wraps it with
ctypes over NumPy arrays. Only the tests, the smoke check and the benchmark's CPU
baseline may import it; it imports nothing from the HIP library's package.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OR_F32, OR_BF16 = 0, 1


def build(force=True):
    """Compile oracle.c into liboracle.so (gcc, -O2, no FMA contraction, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


class QMat(ctypes.Structure):
    """The oracle's own view of one (stacked) quantized matrix."""
    _fields_ = [("codes", ctypes.c_void_p), ("meta", ctypes.c_void_p),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("n_mat", ctypes.c_int32),
                ("mat_stride_codes", ctypes.c_int64), ("mat_stride_meta", ctypes.c_int64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        QP = ctypes.POINTER(QMat)
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]; L.oracle_bf16_to_double.restype = D
        L.oracle_f16_to_double.argtypes = [ctypes.c_uint16]; L.oracle_f16_to_double.restype = D
        L.oracle_double_to_bf16.argtypes = [D]; L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_code.argtypes = [QP, I, I, I]; L.oracle_code.restype = I
        L.oracle_weight.argtypes = [QP, I, I, I]; L.oracle_weight.restype = D
        L.oracle_dequant.argtypes = [QP, I, P]; L.oracle_dequant.restype = None
        L.oracle_route.argtypes = [P, I, I, I, P, P, I, I, I, P, P, P, P]; L.oracle_route.restype = None
        L.oracle_group.argtypes = [I, I, I, P, P, P, P, P, P, P]; L.oracle_group.restype = I
        L.oracle_expert.argtypes = [QP, QP, QP, I, P, I, I, P]; L.oracle_expert.restype = None
        L.oracle_moe.argtypes = [P, I, I, I, I, QP, QP, QP, QP, QP, QP, I, P, P, P, P, P]
        L.oracle_moe.restype = None
        L.oracle_head.argtypes = [P, I, I, I, QP, I, I, P, P]; L.oracle_head.restype = None
        L.oracle_accept.argtypes = [I, I, P, P, P, P]; L.oracle_accept.restype = I
        L.oracle_tier_count.argtypes = [I, P, P, ctypes.c_float]; L.oracle_tier_count.restype = None
        L.oracle_tier_select.argtypes = [I, P, P, I, ctypes.c_float, P]; L.oracle_tier_select.restype = I
        L.oracle_philox4x32_10.argtypes = [P, P, P]; L.oracle_philox4x32_10.restype = None
        L.oracle_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]; L.oracle_uniform.restype = D
        L.oracle_sample.argtypes = [P, I, D, I, D, D, ctypes.c_uint64, ctypes.c_uint64, P]
        L.oracle_sample.restype = I
        L.oracle_threads.argtypes = []; L.oracle_threads.restype = I
        L.oracle_set_threads.argtypes = [I]; L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def qmat(codes, meta, rows, cols, bits, n_mat=1):
    """Describe NumPy code/meta arrays (kept alive by the returned object's `_keep`)."""
    codes = _c(codes, np.uint8)
    meta = _c(meta, np.uint16 if bits == 8 else np.uint32)
    q = QMat(codes.ctypes.data, meta.ctypes.data, rows, cols, bits, n_mat,
             codes.size // n_mat, meta.size // n_mat)
    q._keep = (codes, meta)
    return q


def _xdt(x):
    if x.dtype == np.float32:
        return OR_F32
    if x.dtype == np.uint16:  # bf16 bit patterns
        return OR_BF16
    raise TypeError("activations must be float32 or uint16 (bf16 bits)")


def f16_to_double(h):
    return lib().oracle_f16_to_double(int(h))


def bf16_to_double(h):
    return lib().oracle_bf16_to_double(int(h))


def double_to_bf16(v):
    return lib().oracle_double_to_bf16(float(v))


def code(q, mat, n, k):
    return lib().oracle_code(ctypes.byref(q), mat, n, k)


def dequant(q, mat=0):
    out = np.empty((q.rows, q.cols), np.float64)
    lib().oracle_dequant(ctypes.byref(q), mat, _p(out))
    return out


def route(x, G, bias, top_k, renorm=False):
    """Returns (logits [R,E], probs [R,E], topk_idx [R,k] int32, topk_w [R,k])."""
    x = np.ascontiguousarray(x)
    R, H = x.shape
    G = _c(G, np.float32)
    E = G.shape[0]
    assert E <= 1024
    bias = None if bias is None else _c(bias, np.float32)
    logits = np.empty((R, E)); probs = np.empty((R, E))
    idx = np.empty((R, top_k), np.int32); w = np.empty((R, top_k))
    lib().oracle_route(_p(x), _xdt(x), R, H, _p(G), _p(bias), E, top_k, int(bool(renorm)),
                       _p(logits), _p(probs), _p(idx), _p(w))
    return logits, probs, idx, w


def group(topk_idx, topk_w, n_experts):
    """Returns dict(n_active, active, offsets, entry_row, entry_w, row_mask)."""
    idx = _c(topk_idx, np.int32); w = _c(topk_w, np.float64)
    R, K = idx.shape
    A = min(n_experts, R * K) + 1
    active = np.full(A, -1, np.int32); offsets = np.full(A + 1, -1, np.int32)
    entry_row = np.full(R * K + R, -1, np.int32); entry_w = np.full(R * K + R, np.nan)
    row_mask = np.zeros(n_experts + 1, np.uint8)
    n = lib().oracle_group(R, n_experts, K, _p(idx), _p(w), _p(active), _p(offsets),
                           _p(entry_row), _p(entry_w), _p(row_mask))
    return dict(n_active=n, active=active[:n], offsets=offsets[:n + 1],
                entry_row=entry_row[:offsets[n]], entry_w=entry_w[:offsets[n]],
                row_mask=row_mask)


def expert(gate, up, down, mat, x_row):
    xr = _c(x_row, np.float64)
    H = gate.cols; F = gate.rows
    y = np.empty(H)
    lib().oracle_expert(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), mat,
                        _p(xr), H, F, _p(y))
    return y


def moe(x, gate, up, down, sh_gate, sh_up, sh_down, topk_idx, topk_w, residual=None,
        want_x_next=False):
    """Returns out [R,H] float64 (and x_next bf16 bits [R,H] uint16 when asked)."""
    x = np.ascontiguousarray(x)
    R, H = x.shape
    F = gate.rows
    idx = _c(topk_idx, np.int32); w = _c(topk_w, np.float64)
    K = idx.shape[1]
    if residual is not None:
        residual = np.ascontiguousarray(residual)
        assert residual.dtype == x.dtype and residual.shape == x.shape
    out = np.empty((R, H))
    xn = np.empty((R, H), np.uint16) if want_x_next else None
    lib().oracle_moe(_p(x), _xdt(x), R, H, F, ctypes.byref(gate), ctypes.byref(up),
                     ctypes.byref(down), ctypes.byref(sh_gate), ctypes.byref(sh_up),
                     ctypes.byref(sh_down), K, _p(idx), _p(w), _p(residual), _p(out), _p(xn))
    return (out, xn) if want_x_next else out


def head(x, q, v0=0, v1=None):
    """Returns (logits [R, v1-v0] float64, argmax [R] int32 over [v0, v1))."""
    x = np.ascontiguousarray(x)
    R, H = x.shape
    v1 = q.rows if v1 is None else v1
    logits = np.empty((R, v1 - v0)); am = np.empty(R, np.int32)
    lib().oracle_head(_p(x), _xdt(x), R, H, ctypes.byref(q), v0, v1, _p(logits), _p(am))
    return logits, am


def accept(argmax, proposal, mtp=True):
    """Greedy verification of a window's proposals. argmax [rows] (the head's argmax per
    row), proposal [n_slots] (ignored without mtp). Returns (tokens [n_slots, 2] int32
    with -1 where unused, n_tokens [n_slots] int32, number of kept proposals)."""
    am = _c(argmax, np.int32)
    n_slots = am.size // 2 if mtp else am.size
    assert am.size == (2 * n_slots if mtp else n_slots)
    prop = _c(proposal if proposal is not None else np.zeros(n_slots), np.int32)
    tokens = np.empty((n_slots, 2), np.int32)
    n_tok = np.empty(n_slots, np.int32)
    kept = lib().oracle_accept(n_slots, int(bool(mtp)), _p(am), _p(prop), _p(tokens), _p(n_tok))
    return tokens, n_tok, kept


def tier_count(row_mask, counts, decay):
    """One window's routing counts: counts[e] = fmaf(counts[e], decay, rows routed to e)
    for the routed experts (row_mask [E+1] uint8; the shared expert's entry is not
    counted). Returns the new float32 counts [E]."""
    rm = _c(row_mask, np.uint8)
    c = np.array(counts, np.float32, copy=True)
    lib().oracle_tier_count(c.size, _p(rm), _p(c), float(decay))
    return c


def tier_select(counts, resident, max_swaps, min_gain=1.5):
    """One round of the adaptive tier. Returns (new resident [E] uint8, swaps [n, 2] int32
    as (in, out) pairs)."""
    c = _c(counts, np.float32)
    res = np.array(resident, np.uint8, copy=True)
    sw = np.empty(2 * max(max_swaps, 1), np.int32)
    n = lib().oracle_tier_select(c.size, _p(c), _p(res), int(max_swaps), float(min_gain), _p(sw))
    return res, sw[:2 * n].reshape(n, 2)


def philox4x32_10(ctr, key):
    """The four output words of Philox4x32-10 for counter ctr (4 words) and key (2 words)."""
    c = _c(ctr, np.uint32); k = _c(key, np.uint32)
    o = np.empty(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(o))
    return o


def uniform(seed, position):
    """The draw's uniform in [0, 1) for (seed, position)."""
    return lib().oracle_uniform(int(seed) & (2**64 - 1), int(position) & (2**64 - 1))


def sample(logits, temperature, top_k, top_p=1.0, min_p=0.0, seed=0, position=0):
    """A sampled token from one row's logits [V] (see oracle_sample). Returns (token,
    margin: the smallest relative distance of a decision to its boundary)."""
    lg = _c(logits, np.float32)
    m = ctypes.c_double(0.0)
    t = lib().oracle_sample(_p(lg), lg.size, float(temperature), int(top_k), float(top_p), float(min_p),
                            int(seed) & (2**64 - 1), int(position) & (2**64 - 1), ctypes.byref(m))
    return t, m.value


def threads():
    return lib().oracle_threads()


def set_threads(n):
    """Threads for the oracle's parallel loops from now on."""
    lib().oracle_set_threads(int(n))

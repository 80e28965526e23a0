"""CPU checks of the C-ABI library: it loads, exports what include/strata_window.h
declares, and rejects invalid arguments before any device work (no GPU needed)."""
import ctypes
import json
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sw():
    import verify_window_expert_amd as m
    if not os.path.exists(m.LIB_PATH):
        m.build()
    return m


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(strata_window_\w+)\s*\(", text, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(sw):
    names = declared_functions()
    assert {"strata_window_route", "strata_window_moe", "strata_window_head",
            "strata_window_workspace", "strata_window_last_error", "strata_window_abi_version"} <= set(names)
    lib = ctypes.CDLL(sw.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(sw):
    """The built library reports the version its header declares."""
    text = open(os.path.join(ROOT, "include", "strata_window.h")).read()
    declared = int(re.search(r"#define STRATA_WINDOW_ABI_VERSION (\d+)", text).group(1))
    assert declared == 6
    assert sw.library().strata_window_abi_version() == declared


def test_workspace_sizes(sw):
    L = sw.library()
    for name in ("small_f32", "two_slots_mtp", "four_slots_mtp_zipf", "e256_2bit"):
        c = synth.config(name)
        r = L.strata_window_workspace(0, c.rows, c.hidden, c.ffn, c.experts, c.top_k, 0)
        m = L.strata_window_workspace(1, c.rows, c.hidden, c.ffn, c.experts, c.top_k, 0)
        assert r >= sw.WS_COUNTER_BYTES + 8 * c.rows * c.experts
        ent = c.rows * c.top_k + c.rows
        # h as bf16 hi and lo per entry and ffn input
        assert m >= sw.WS_COUNTER_BYTES + 4 * ent * c.ffn
        assert r % 256 == 0 and m % 256 == 0
    assert L.strata_window_workspace(2, 8, 2048, 0, 0, 0, 151936) > 0
    assert L.strata_window_workspace(0, 0, 2048, 768, 128, 8, 0) == 0      # rows 0
    assert L.strata_window_workspace(0, 9, 2048, 768, 128, 8, 0) == 0      # rows 9
    assert L.strata_window_workspace(7, 8, 2048, 768, 128, 8, 0) == 0      # unknown
    # the sampled draw: each 4096-logit chunk's 128 candidate keys and indices per row
    s = L.strata_window_workspace(5, 8, 0, 0, 0, 0, 151936)
    assert s >= sw.WS_COUNTER_BYTES + 8 * 8 * 38 * 128 and s % 256 == 0
    assert L.strata_window_workspace(5, 8, 0, 0, 0, 0, 0) == 0             # vocab 0
    assert L.strata_window_workspace(5, 9, 0, 0, 0, 0, 100) == 0           # rows 9


# fake, aligned device addresses: the checks reject the call before anything uses them
A = 0x10000000


def route_out(sw, bad=None, misalign=None):
    vals = [A + 0x1000 * i for i in range(len(sw.CRouteOut._fields_))]
    names = [f[0] for f in sw.CRouteOut._fields_]
    if bad:
        vals[names.index(bad)] = 0
    if misalign:
        vals[names.index(misalign)] += 4
    return sw.CRouteOut(*vals)


def call_route(sw, rows=8, hidden=2048, E=128, k=8, flags=0, x=A, ws=A, ws_bytes=1 << 30, dtype=1, ro=None,
               gate=A, bias=None):
    ro = route_out(sw) if ro is None else ro
    return sw.library().strata_window_route(None, x, dtype, rows, hidden, gate, bias, E, k, flags,
                                            ctypes.byref(ro), ws, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(rows=0), dict(rows=9), dict(k=0), dict(k=9), dict(E=4, k=8),
                                dict(E=257), dict(flags=2), dict(x=0), dict(x=A + 8), dict(ws=0),
                                dict(ws=A + 16), dict(ws_bytes=100), dict(dtype=2), dict(gate=0),
                                dict(bias=A + 4), dict(hidden=0), dict(hidden=2040)])
def test_route_rejects(sw, kw):
    assert call_route(sw, **kw) == sw.STRATA_EINVAL
    assert sw.library().strata_window_last_error().decode() != ""


@pytest.mark.parametrize("field", ["topk_idx", "active", "row_mask", "entry_pos", "row_w"])
def test_route_rejects_bad_outputs(sw, field):
    assert call_route(sw, ro=route_out(sw, bad=field)) == sw.STRATA_EINVAL
    assert call_route(sw, ro=route_out(sw, misalign=field)) == sw.STRATA_EINVAL


def qm(sw, rows, cols, bits, n_mat, codes=A, meta=A):
    per_c = rows * cols * bits // 8
    per_m = rows * cols // 32
    return sw.CQMat(codes, meta, rows, cols, bits, n_mat, per_c if n_mat > 1 else 0, per_m if n_mat > 1 else 0)


def call_moe(sw, rows=8, H=2048, F=768, E=128, k=8, bits=4, mats=None, out=A, ws_bytes=1 << 30, residual=None):
    m = mats or {}
    g = m.get("gate", qm(sw, F, H, bits, E)); u = m.get("up", qm(sw, F, H, bits, E))
    d = m.get("down", qm(sw, H, F, bits, E))
    sg = m.get("sh_gate", qm(sw, F, H, bits, 1)); su = m.get("sh_up", qm(sw, F, H, bits, 1))
    sd = m.get("sh_down", qm(sw, H, F, bits, 1))
    ro = route_out(sw)
    return sw.library().strata_window_moe(None, A, 1, rows, H, F, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                          ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), ctypes.byref(ro),
                                          E, k, residual, out, None, A, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(rows=9), dict(rows=0), dict(out=0), dict(out=A + 4), dict(ws_bytes=4096),
                                dict(residual=A + 2), dict(F=760), dict(H=2000)])
def test_moe_rejects(sw, kw):
    assert call_moe(sw, **kw) == sw.STRATA_EINVAL


def test_moe_rejects_mismatched_matrices(sw):
    assert call_moe(sw, mats=dict(up=qm(sw, 768, 2048, 4, 127))) == sw.STRATA_EINVAL      # wrong n_mat
    assert call_moe(sw, mats=dict(down=qm(sw, 768, 2048, 4, 128))) == sw.STRATA_EINVAL    # transposed
    assert call_moe(sw, mats=dict(sh_up=qm(sw, 768, 2048, 2, 1))) == sw.STRATA_EINVAL     # bits differ
    assert call_moe(sw, mats=dict(gate=qm(sw, 768, 2048, 4, 128, codes=A + 8))) == sw.STRATA_EINVAL
    bad = qm(sw, 768, 2048, 4, 128)
    bad.mat_stride_codes = 100
    assert call_moe(sw, mats=dict(gate=bad)) == sw.STRATA_EINVAL


def test_moe_8bit_experts_unsupported(sw):
    mats = dict(gate=qm(sw, 768, 2048, 8, 128), up=qm(sw, 768, 2048, 8, 128), down=qm(sw, 2048, 768, 8, 128),
                sh_gate=qm(sw, 768, 2048, 8, 1), sh_up=qm(sw, 768, 2048, 8, 1), sh_down=qm(sw, 2048, 768, 8, 1))
    assert call_moe(sw, mats=mats) == sw.STRATA_EUNSUPPORTED


def test_head_rejects(sw):
    L = sw.library()
    h = qm(sw, 151936, 2048, 8, 1)
    ok = dict(rows=8, H=2048, V=151936, am=A, lg=A, ws=1 << 30)
    def call(**kw):
        a = dict(ok, **kw)
        return L.strata_window_head(None, A, 1, a["rows"], a["H"], ctypes.byref(kw.get("q", h)), a["V"], a["lg"],
                                    a["am"], A, a["ws"], None)
    assert call(rows=9) == sw.STRATA_EINVAL
    assert call(am=0) == sw.STRATA_EINVAL
    assert call(lg=A + 4) == sw.STRATA_EINVAL
    assert call(V=151920) == sw.STRATA_EINVAL                    # rows != vocab
    assert call(q=qm(sw, 151936, 2048, 4, 1)) == sw.STRATA_EINVAL
    assert call(ws=64) == sw.STRATA_EINVAL


def test_window_limits_from_pages(sw):
    """The row limit of the ABI is the window size the pages state."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "window_limits.json")))
    assert sw.MAX_ROWS == g["max_rows_per_window"]
    assert g["rows_per_slot_with_batch_mtp"] * g["max_slots_per_window_with_batch_mtp"] == sw.MAX_ROWS
    assert call_route(sw, rows=g["max_rows_per_window"] + 1) == sw.STRATA_EINVAL
    # the synthetic workloads: two MTP slots = 4 rows, four MTP slots = 8 rows
    assert synth.config("two_slots_mtp").rows == 2 * g["rows_per_slot_with_batch_mtp"] == g["workloads"]["two_slots_mtp"]
    assert synth.config("four_slots_mtp_zipf").rows == 4 * g["rows_per_slot_with_batch_mtp"] == g["workloads"]["four_slots_mtp"]


def test_accept_rejects(sw):
    L = sw.library()
    def call(rows=8, n_slots=4, mtp=1, am=A, prop=A, tok=A, ntok=A, nacc=A):
        return L.strata_window_accept(None, am, rows, n_slots, mtp, prop, tok, ntok, nacc, None)
    assert call(mtp=2) == sw.STRATA_EINVAL
    assert call(n_slots=5, rows=10) == sw.STRATA_EINVAL          # more than 8 rows with MTP
    assert call(n_slots=0, rows=0) == sw.STRATA_EINVAL
    assert call(rows=7) == sw.STRATA_EINVAL                      # not two rows per slot
    assert call(mtp=0, n_slots=4, rows=8) == sw.STRATA_EINVAL   # one row per slot without MTP
    assert call(mtp=0, n_slots=9, rows=9) == sw.STRATA_EINVAL
    assert call(prop=None) == sw.STRATA_EINVAL                   # MTP needs the proposals
    assert call(am=None) == sw.STRATA_EINVAL
    assert call(tok=A + 4) == sw.STRATA_EINVAL
    assert call(nacc=0) == sw.STRATA_EINVAL


def test_sample_rejects(sw):
    """strata_window_sample refuses bad shapes, pointers and a short workspace before it
    enqueues anything (the fake device addresses are never touched)."""
    L = sw.library()
    need = L.strata_window_workspace(5, 8, 0, 0, 0, 0, 151936)

    def call(rows=8, vocab=151936, lg=A, prm=A, pos=A, tok=A, ws=A, wsb=need):
        return L.strata_window_sample(None, lg, rows, vocab, prm, pos, tok, ws, wsb, None)
    assert call(rows=0) == sw.STRATA_EINVAL
    assert call(rows=9) == sw.STRATA_EINVAL
    assert call(vocab=0) == sw.STRATA_EINVAL
    assert call(lg=None) == sw.STRATA_EINVAL
    assert call(prm=A + 8) == sw.STRATA_EINVAL
    assert call(pos=None) == sw.STRATA_EINVAL
    assert call(tok=A + 4) == sw.STRATA_EINVAL
    assert call(ws=None) == sw.STRATA_EINVAL
    assert call(wsb=need - 1) == sw.STRATA_EINVAL
    assert "workspace" in L.strata_window_last_error().decode()


def test_tier_rejects(sw):
    L = sw.library()
    def call(E=128, rm=A, c=A, decay=1.0, res=A, ms=4, gain=1.5, swp=A, ns=A):
        return L.strata_window_tier(None, rm, E, c, decay, res, ms, gain, swp, ns, None)
    assert call(E=0) == sw.STRATA_EINVAL
    assert call(E=257) == sw.STRATA_EINVAL
    assert call(rm=None) == sw.STRATA_EINVAL
    assert call(c=A + 4) == sw.STRATA_EINVAL
    assert call(decay=1.5) == sw.STRATA_EINVAL
    assert call(decay=float("nan")) == sw.STRATA_EINVAL
    assert call(ms=-1) == sw.STRATA_EINVAL
    assert call(ms=129) == sw.STRATA_EINVAL
    assert call(gain=-1.0) == sw.STRATA_EINVAL
    assert call(gain=float("inf")) == sw.STRATA_EINVAL
    assert call(swp=None) == sw.STRATA_EINVAL
    assert call(ns=None) == sw.STRATA_EINVAL


def test_layer_rejects_and_workspace(sw):
    L = sw.library()
    assert L.strata_window_workspace(3, 8, 2048, 768, 128, 8, 0) >= \
        L.strata_window_workspace(1, 8, 2048, 768, 128, 8, 0) + 8 * 8 * 128 * 4
    assert L.strata_window_workspace(3, 8, 2048, 768, 0, 8, 0) == 0
    ro = route_out(sw)
    m = dict(gate=qm(sw, 768, 2048, 4, 128), up=qm(sw, 768, 2048, 4, 128), down=qm(sw, 2048, 768, 4, 128),
             sh_gate=qm(sw, 768, 2048, 4, 1), sh_up=qm(sw, 768, 2048, 4, 1), sh_down=qm(sw, 2048, 768, 4, 1))

    def call(rows=8, H=2048, F=768, E=128, k=8, flags=0, gw=A, ws_bytes=1 << 30, mats=m, out=A):
        return L.strata_window_layer(None, A, 1, rows, H, F, gw, None, flags,
                                     *[ctypes.byref(mats[n]) for n in ("gate", "up", "down", "sh_gate", "sh_up",
                                                                      "sh_down")],
                                     E, k, ctypes.byref(ro), None, out, None, A, ws_bytes, None)
    assert call(rows=9) == sw.STRATA_EINVAL
    assert call(gw=0) == sw.STRATA_EINVAL                # router weights
    assert call(flags=2) == sw.STRATA_EINVAL             # route flags
    assert call(out=A + 4) == sw.STRATA_EINVAL           # moe output
    assert call(F=640) == sw.STRATA_EINVAL               # matrices of another shape
    assert call(ws_bytes=L.strata_window_workspace(1, 8, 2048, 768, 128, 8, 0)) == sw.STRATA_EINVAL


def test_stream_read_rejects(sw):
    L = sw.library()
    def call(src=A, nbytes=1 << 20, sink=A):
        return L.strata_window_stream_read(None, src, nbytes, sink, 0x9E3779B9, None)
    assert call(src=None) == sw.STRATA_EINVAL
    assert call(src=A + 8) == sw.STRATA_EINVAL
    assert call(nbytes=0) == sw.STRATA_EINVAL
    assert call(nbytes=1000) == sw.STRATA_EINVAL
    assert call(sink=None) == sw.STRATA_EINVAL
    assert call(sink=A + 2) == sw.STRATA_EINVAL


def test_stack_rejects_and_workspace(sw):
    L = sw.library()
    layers = (sw.CLayer * 2)()
    def call(n=2, lay=layers, xf=A, ws=A, wsb=1 << 30, rows=8, out=None):
        return L.strata_window_stack(None, A, sw.STRATA_BF16, rows, 2048, 768, 128, 8, 0, n, lay, None, 0, None,
                                     None, out, xf, ws, wsb, None)
    assert call(n=0) == sw.STRATA_EINVAL
    assert call(n=1025) == sw.STRATA_EINVAL
    assert call(lay=None) == sw.STRATA_EINVAL
    assert call(xf=None) == sw.STRATA_EINVAL
    assert call(xf=A + 8) == sw.STRATA_EINVAL
    assert call(out=A + 4) == sw.STRATA_EINVAL
    assert call(ws=A + 16) == sw.STRATA_EINVAL
    assert call(wsb=1024) == sw.STRATA_EINVAL
    assert call(rows=9) == sw.STRATA_EINVAL
    assert call() == sw.STRATA_EINVAL            # the layers' descriptors are empty
    assert "layer 0" in L.strata_window_last_error().decode()
    # the stack's workspace holds a layer's, two bf16 inputs and the head's
    w3 = sw.workspace_bytes(3, 8, 2048, 768, 128, 8)
    w4 = sw.workspace_bytes(4, 8, 2048, 768, 128, 8, 0)
    w4h = sw.workspace_bytes(4, 8, 2048, 768, 128, 8, 151936)
    assert w4 >= w3 + 2 * 2 * 8 * 2048
    assert w4h >= w4 + sw.workspace_bytes(2, 8, 2048, vocab=151936) - 4096


def test_noalloc_rejects_before_any_device_call(sw):
    """strata_window_layer_noalloc refuses a shape whose workspace exceeds its fixed scratch
    array, and an out-of-range shape, before it looks at the device (no GPU here)."""
    L = sw.library()
    assert L.strata_window_workspace(3, 8, 7936, 4096, 256, 8, 0) > sw.NOALLOC_SCRATCH_BYTES
    assert L.strata_window_workspace(3, 8, 2048, 768, 128, 8, 0) <= sw.NOALLOC_SCRATCH_BYTES

    def call(rows, hidden, ffn, E, k):
        qs = [qm(sw, ffn, hidden, 4, E), qm(sw, ffn, hidden, 4, E), qm(sw, hidden, ffn, 4, E),
              qm(sw, ffn, hidden, 4, 1), qm(sw, ffn, hidden, 4, 1), qm(sw, hidden, ffn, 4, 1)]
        ro = route_out(sw)
        return L.strata_window_layer_noalloc(None, A, 1, rows, hidden, ffn, A, None, 0,
                                             *[ctypes.byref(q) for q in qs], E, k, ctypes.byref(ro), None, A, None,
                                             None)
    assert call(8, 7936, 4096, 256, 8) == sw.STRATA_EINVAL
    assert b"scratch" in L.strata_window_last_error()
    assert call(9, 2048, 768, 128, 8) == sw.STRATA_EINVAL
    assert call(8, 2048, 768, 128, 0) == sw.STRATA_EINVAL

"""GPU parity of the fused layer entry point (strata_window_layer: the router's GEMV,
then gate/up with the routing taken in every workgroup, then down and the combine)
against the CPU oracle, through the C ABI; and its agreement with the two-call path."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import (REL_TOL, DevLayer, assert_route_equal, gpu_window, oracle_mats,  # noqa: E402
                         oracle_window, row_rel_err, to_dev_x, topk_gap, assert_close)

_layers = {}


def layer_for(cfg):
    if cfg not in _layers:
        if len(_layers) > 4:
            _layers.clear()
        L = synth.make_layer(cfg, 0)
        _layers[cfg] = (L, DevLayer(L, cfg), oracle_mats(L, cfg))
    return _layers[cfg]


def check(cfg, window=0, renorm=False, residual=False, x_next=False, layer=True):
    L, dl, mats = layer_for(cfg)
    x = synth.make_window(cfg, window)
    print(f"[layer] {cfg.name} H={cfg.hidden} E={cfg.experts} bits={cfg.bits} R={x.shape[0]} "
          f"window={window} renorm={renorm} residual={residual} layer={layer}", flush=True)
    gr, gout, gxn = gpu_window(dl, to_dev_x(x), cfg.top_k, renorm, residual, x_next, layer=layer)
    orc, oout, oxn = oracle_window(L, mats, x, cfg, renorm, residual, x_next)
    assert topk_gap(orc["logits"], cfg.top_k) > 1e-9, "near-tie in the routing of this seed"
    assert_route_equal(gr, orc, cfg)
    err, eerr = assert_close(gout, oout)
    print(f"[parity] row err {err:.2e}, element err {eerr:.2e}", flush=True)
    return dl, x, gr, gout, gxn, oxn


@pytest.mark.parametrize("window", [0, 1])
def test_layer_small_f32(window):
    check(synth.config("small_f32"), window)


def test_layer_small_f32_renorm_residual_x_next():
    _, _, _, gout, gxn, oxn = check(synth.config("small_f32"), 2, renorm=True, residual=True, x_next=True)
    # x_next is the bf16 rounding of the GPU's own output
    want = (np.frombuffer(np.ascontiguousarray(gout, np.float32).tobytes(), np.uint32))
    rne = ((want + 0x7FFF + ((want >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(gxn.ravel(), rne)


def test_layer_two_slots_mtp():
    check(synth.config("two_slots_mtp"), 0)


@pytest.mark.parametrize("window", [0, 1, 2])
def test_layer_four_slots_mtp_zipf(window):
    check(synth.config("four_slots_mtp_zipf"), window)


@pytest.mark.parametrize("rows", synth.E256_ROWS)
def test_layer_e256_2bit_rows(rows):
    check(synth.config("e256_2bit", rows=rows), 0)


def test_layer_row_equals_row_alone_bitwise():
    cfg = synth.config("four_slots_mtp_zipf")
    dl, x, _, gout, _, _ = check(cfg, 3)
    for r in range(x.shape[0]):
        print(f"[layer] row {r} alone", flush=True)
        _, g1, _ = gpu_window(dl, to_dev_x(x[r:r + 1]), cfg.top_k, layer=True)
        assert np.array_equal(g1[0].view(np.uint32), gout[r].view(np.uint32)), r


@pytest.mark.parametrize("hidden,bits,layer", [(5632, 4, True), (5632, 2, True), (6144, 4, True), (6656, 4, False)])
def test_row_equals_row_alone_where_the_waves_depend_on_rows(hidden, bits, layer):
    """bf16 rows at hiddens where the gate/up wave count depends on the window's rows: at
    5632 a lone row runs 16-wave workgroups and an 8-row window 8-wave ones; at 6144 (fused
    layer call) and 6656 (two-call path) a lone row would want 16 waves, whose partial sums
    do not fit next to the activation image. The k-split of a row's sums is fixed by the
    shapes alone, so each row of the window is bit-identical to the row computed alone."""
    cfg = synth.config("two_slots_mtp", hidden=hidden, ffn=256, experts=16, top_k=4, rows=8, bits=bits)
    dl, x, _, gout, _, _ = check(cfg, 0, layer=layer)
    for r in range(x.shape[0]):
        print(f"[layer] H={hidden} bits={bits} row {r} alone", flush=True)
        _, g1, _ = gpu_window(dl, to_dev_x(x[r:r + 1]), cfg.top_k, layer=layer)
        assert np.array_equal(g1[0].view(np.uint32), gout[r].view(np.uint32)), r


def test_layer_matches_two_call_path():
    cfg = synth.config("four_slots_mtp_zipf")
    L, dl, _ = layer_for(cfg)
    xd = to_dev_x(synth.make_window(cfg, 5))
    print("[layer] against route + moe", flush=True)
    gr1, o1, _ = gpu_window(dl, xd, cfg.top_k, layer=True)
    gr2, o2, _ = gpu_window(dl, xd, cfg.top_k, layer=False)
    for k in ("topk_idx", "active", "offsets", "entry_row", "entry_pos", "row_mask"):
        assert np.array_equal(gr1[k], gr2[k]), k
    np.testing.assert_allclose(gr1["topk_w"], gr2["topk_w"], rtol=1e-6)
    assert row_rel_err(o1, o2) <= 1e-5


def test_layer_hidden_beyond_the_fused_lds():
    """hidden 7936 (bf16): the activation image and the routing core's tables do not fit
    one compute unit's LDS together, so the layer call runs the routing as a kernel of its
    own and the plain gate/up; the same results."""
    check(synth.config("two_slots_mtp", hidden=7936, ffn=256, experts=16, top_k=4, rows=3), 0)


def test_binding_refuses_short_or_mismatched_buffers():
    """The library sees only pointers, so the binding refuses, before anything is enqueued,
    caller buffers that the kernels would access past their end (or read with the wrong
    type), and routing outputs made for another window shape; the call then still works."""
    cfg = synth.config("small_f32")
    L, dl, mats = layer_for(cfg)
    x = to_dev_x(synth.make_window(cfg, 0))
    R, H, E, k = cfg.rows, cfg.hidden, cfg.experts, cfg.top_k
    f32 = dict(dtype=torch.float32, device="cuda")
    layer = lambda **kw: sw.strata_window_layer(x, dl.gate_w, dl.bias, k, dl.gate, dl.up, dl.down, *dl.sh, **kw)
    with pytest.raises(ValueError):
        layer(out=torch.empty(R, H - 32, **f32))
    with pytest.raises(TypeError):
        layer(x_next=torch.empty(R, H, **f32))
    with pytest.raises(ValueError):
        layer(route=sw.RouteOut(R + 1, E, k))
    with pytest.raises(ValueError):
        sw.strata_window_route(x, dl.gate_w[:, : H - 32].contiguous(), dl.bias, k)
    with pytest.raises(ValueError):
        sw.strata_window_moe(x, dl.gate, dl.up, dl.down, *dl.sh, sw.RouteOut(R, E, k), residual=x[:1])
    with pytest.raises(ValueError):
        sw.QMat(dl.gate.codes[:, :-16].contiguous(), dl.gate.meta, dl.gate.rows, dl.gate.cols, dl.gate.bits)
    with pytest.raises(ValueError):
        sw.strata_window_accept(torch.zeros(4, dtype=torch.int32, device="cuda"),
                                torch.zeros(1, dtype=torch.int32, device="cuda"))
    out, ro = layer()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()

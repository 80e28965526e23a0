"""GPU parity of the verify-window MoE layer against the CPU oracle, through the C ABI.

Routing indices and per-expert row lists must match bit for bit; outputs must be within
a per-row relative error of 2e-3 (float32 accumulation against the double-precision
definition). A window's row must equal the same row computed alone, bit for bit (Strata
docs/BATCHING.md, "Exactness").
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import (REL_TOL, DevLayer, assert_route_equal, gpu_window, oracle_mats,  # noqa: E402
                         oracle_window, row_rel_err, to_dev_x, topk_gap, assert_close)

_layers = {}


def layer_for(cfg, layer=0):
    key = (cfg, layer)
    if key not in _layers:
        if len(_layers) > 6:
            _layers.clear()
        L = synth.make_layer(cfg, layer)
        _layers[key] = (L, DevLayer(L, cfg), oracle_mats(L, cfg))
    return _layers[key]


def check_window(cfg, window=0, renorm=False, residual=False, x=None, x_next=False, ties=False, layer=False):
    L, dl, mats = layer_for(cfg)
    x = synth.make_window(cfg, window) if x is None else x
    print(f"[parity] {cfg.name} H={cfg.hidden} F={cfg.ffn} E={cfg.experts} k={cfg.top_k} bits={cfg.bits} "
          f"R={x.shape[0]} window={window} renorm={renorm} residual={residual} layer={layer}", flush=True)
    gr, gout, gxn = gpu_window(dl, to_dev_x(x), cfg.top_k, renorm, residual, x_next, layer=layer)
    orc, oout, oxn = oracle_window(L, mats, x, cfg, renorm, residual, x_next)
    # exact ties (equal logits) are decided identically by index; near-ties are not
    # well-posed across summation orders, so a seed must not produce them
    if not ties:
        assert topk_gap(orc["logits"], cfg.top_k) > 1e-9, "near-tie in the routing of this seed"
    assert_route_equal(gr, orc, cfg)
    err, eerr = assert_close(gout, oout)
    print(f"[parity] row err {err:.2e}, element err {eerr:.2e}", flush=True)
    return gr, gout, oout, err, gxn, oxn


# --------------------------------------------------------------------- the five configs

@pytest.mark.parametrize("window", [0, 1])
def test_small_f32(window):
    check_window(synth.config("small_f32"), window)


def test_small_f32_renorm_residual():
    check_window(synth.config("small_f32"), 2, renorm=True, residual=True)


@pytest.mark.parametrize("window", [0, 1])
def test_two_slots_mtp(window):
    _, _, _, err, _, _ = check_window(synth.config("two_slots_mtp"), window)
    print("two_slots_mtp rel err", err)


@pytest.mark.parametrize("window", [0, 1, 2])
def test_four_slots_mtp_zipf(window):
    _, _, _, err, _, _ = check_window(synth.config("four_slots_mtp_zipf"), window)
    print("four_slots_mtp_zipf rel err", err)


@pytest.mark.parametrize("rows", synth.E256_ROWS)
def test_e256_2bit_row_sweep(rows):
    cfg = synth.config("e256_2bit", rows=rows)
    check_window(cfg, 0)


def test_x_next_is_bf16_of_output():
    cfg = synth.config("two_slots_mtp")
    _, gout, oout, _, gxn, oxn = check_window(cfg, 3, residual=True, x_next=True)
    gx = synth.bf16_bits_to_f32(gxn)
    # x_next is the bf16 rounding of the GPU's own output
    assert np.array_equal(gxn, synth.f32_to_bf16_bits(gout))
    ox = synth.bf16_bits_to_f32(oxn)
    # each side rounds its own output to bf16 (half an ulp: at most 2^-8 of the value),
    # so the two may differ by those roundings plus the outputs' own difference
    bound = 2.0 ** -8 * (np.abs(gout) + np.abs(oout)) + np.abs(gout - oout) + 1e-30
    assert np.all(np.abs(gx.astype(np.float64) - ox) <= bound)


# --------------------------------------------------------------------- shapes and edges

@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("layer", [False, True])
def test_every_row_count(rows, layer):
    cfg = synth.config("small_f32", rows=rows, top_k=3, experts=13)
    check_window(cfg, 5, layer=layer)


@pytest.mark.parametrize("layer", [False, True])
def test_ragged_shapes(layer):
    """Expert count not a multiple of the router's 4 experts per workgroup, hidden not a
    multiple of its 512-input chunk, several output ranges, 2-bit."""
    check_window(synth.config("small_f32", hidden=640, ffn=384, experts=13, top_k=5, rows=7), 0, layer=layer)
    check_window(synth.config("small_f32", hidden=768, ffn=512, experts=10, top_k=4, rows=5, bits=2, x_dtype="bf16"), 1, layer=layer)


@pytest.mark.parametrize("layer", [False, True])
def test_two_bit_float_input(layer):
    """2-bit weights with float activations (the staged image's bf16 hi and lo columns, each
    input divided by its code position's power of two), rows of very different magnitudes
    (2^-20 .. 2^20): against the oracle, and each row of the window equal to that row alone,
    bit for bit."""
    cfg = synth.config("small_f32", hidden=1024, ffn=512, experts=16, top_k=4, rows=6, bits=2)
    x = synth.make_window(cfg, 2)
    x *= (2.0 ** np.array([-20, -7, 0, 3, 11, 20]))[:, None].astype(np.float32)
    check_window(cfg, x=x, layer=layer)
    L, dl, mats = layer_for(cfg)
    gr, gout, _ = gpu_window(dl, to_dev_x(x), cfg.top_k, layer=layer)
    for r in range(cfg.rows):
        g1, o1, _ = gpu_window(dl, to_dev_x(x[r:r + 1]), cfg.top_k, layer=layer)
        assert np.array_equal(g1["topk_idx"][0], gr["topk_idx"][r])
        assert np.array_equal(o1[0], gout[r]), (r, np.max(np.abs(o1[0] - gout[r])))


@pytest.mark.parametrize("layer", [False, True])
def test_all_rows_share_experts(layer):
    cfg = synth.config("small_f32", rows=8, top_k=4)
    x = np.repeat(synth.make_window(cfg, 0)[:1], 8, axis=0)
    gr, gout, _, _, _, _ = check_window(cfg, x=x, layer=layer)
    assert gr["n_active"] == 4 + 1
    assert np.all(gout == gout[0])


@pytest.mark.parametrize("layer", [False, True])
def test_disjoint_rows(layer):
    cfg = synth.config("small_f32", rows=8, top_k=2, experts=16)
    L, dl, mats = layer_for(cfg)
    x = np.zeros((8, cfg.hidden), np.float32)
    # rows aligned with pairs of router rows so every row picks its own pair of experts
    G = L.gate_w.astype(np.float64)
    for r in range(8):
        x[r] = (40.0 * (G[2 * r] + G[2 * r + 1]) / np.linalg.norm(G[2 * r] + G[2 * r + 1]) ** 2).astype(np.float32)
    gr, _, _, _, _, _ = check_window(cfg, x=x, layer=layer)
    assert gr["n_active"] == 16 + 1
    assert sorted(gr["topk_idx"].ravel().tolist()) == list(range(16))


@pytest.mark.parametrize("layer", [False, True])
def test_k_equals_e_full_mixture(layer):
    check_window(synth.config("small_f32", experts=8, top_k=8, rows=3), 0, renorm=True, layer=layer)


@pytest.mark.parametrize("layer", [False, True])
def test_zero_rows(layer):
    cfg = synth.config("small_f32", rows=3)
    x = synth.make_window(cfg, 0)
    x[1] = 0.0
    gr, gout, oout, _, _, _ = check_window(cfg, x=x, ties=True, layer=layer)
    assert list(gr["topk_idx"][1]) == list(range(cfg.top_k))   # equal logits: lowest indices
    assert np.all(gout[1] == 0.0)


@pytest.mark.parametrize("layer", [False, True])
def test_max_limits(layer):
    """rows 8, k 8, 256 experts (the ABI's maxima), reduced width."""
    check_window(synth.config("e256_2bit", hidden=1024, ffn=256, rows=8), 0, layer=layer)


@pytest.mark.parametrize("rows", [4, 8])
def test_large_ffn(rows):
    """ffn 4096: the down kernel stages the most h per thread (4 groups of 8 inputs), in
    8-wave workgroups at 4 rows and 16-wave ones at 8; each row also equals the row alone."""
    cfg = synth.config("two_slots_mtp", hidden=512, ffn=4096, experts=8, top_k=2, rows=rows)
    _, gout = check_window(cfg, 0, layer=True)[:2]
    _, dl, _ = layer_for(cfg)
    x = synth.make_window(cfg, 0)
    for r in range(rows):
        _, g1, _ = gpu_window(dl, to_dev_x(x[r:r + 1]), cfg.top_k, layer=True)
        assert np.array_equal(g1[0].view(np.uint32), gout[r].view(np.uint32)), r


@pytest.mark.parametrize("layer", [False, True])
def test_hidden_beyond_eight_router_chunks(layer):
    """hidden 4608: nine 512-input router chunks, more than the routing core keeps in
    registers (the rest are read where they are added)."""
    check_window(synth.config("two_slots_mtp", hidden=4608, ffn=256, experts=16, top_k=4, rows=6), 0, layer=layer)


# --------------------------------------------------------------------- invariance

@pytest.mark.parametrize("name", ["four_slots_mtp_zipf", "e256_2bit"])
def test_window_row_equals_row_alone_bitwise(name):
    """Strata docs/BATCHING.md, "Exactness": batching leaves a row's arithmetic that of the
    window's. Each row of a full window equals that row run as a 1-row window, bit for bit."""
    cfg = synth.config(name)
    L, dl, mats = layer_for(cfg)
    x = synth.make_window(cfg, 7)
    gr, gout, _ = gpu_window(dl, to_dev_x(x), cfg.top_k)
    for r in range(cfg.rows):
        g1, o1, _ = gpu_window(dl, to_dev_x(x[r:r + 1]), cfg.top_k)
        assert np.array_equal(g1["topk_idx"][0], gr["topk_idx"][r])
        assert np.array_equal(o1[0], gout[r]), (r, np.max(np.abs(o1[0] - gout[r])))


def test_window_row_equals_row_alone_bitwise_f32():
    """float32 input (bf16 hi and lo columns) at hidden 1024, whose 8 k-groups split over
    two waves per gate/up item: each row of a full window (~40 experts) equals that row run
    as a 1-row window, bit for bit, through both entry paths."""
    cfg = synth.config("small_f32", hidden=1024, ffn=768, experts=64, top_k=8, rows=8)
    check_window(cfg, 0)
    L, dl, mats = layer_for(cfg)
    x = synth.make_window(cfg, 3)
    gr, gout, _ = gpu_window(dl, to_dev_x(x), cfg.top_k)
    for layer in (False, True):
        for r in range(cfg.rows):
            g1, o1, _ = gpu_window(dl, to_dev_x(x[r:r + 1]), cfg.top_k, layer=layer)
            assert np.array_equal(g1["topk_idx"][0], gr["topk_idx"][r])
            assert np.array_equal(o1[0], gout[r]), (layer, r, np.max(np.abs(o1[0] - gout[r])))


def test_run_to_run_deterministic():
    cfg = synth.config("four_slots_mtp_zipf")
    L, dl, mats = layer_for(cfg)
    xd = to_dev_x(synth.make_window(cfg, 4))
    ref = gpu_window(dl, xd, cfg.top_k)[1]
    for _ in range(20):
        assert np.array_equal(gpu_window(dl, xd, cfg.top_k)[1], ref)


def test_workspace_reuse_across_shapes():
    """One workspace, filled with garbage first (it needs no initialisation), serves
    windows of different row counts back to back."""
    cfg = synth.config("four_slots_mtp_zipf")
    L, dl, mats = layer_for(cfg)
    ws_r = sw.workspace(sw.workspace_bytes(0, 8, cfg.hidden, n_experts=cfg.experts)).fill_(0xA5)
    ws_m = sw.workspace(sw.workspace_bytes(1, 8, cfg.hidden, cfg.ffn, cfg.experts, cfg.top_k)).fill_(0xFF)
    for rows in (8, 3, 8, 1):
        x = synth.make_window(cfg, 9)[:rows]
        xd = to_dev_x(x)
        ro = sw.strata_window_route(xd, dl.gate_w, dl.bias, cfg.top_k, ws=ws_r)
        out = sw.strata_window_moe(xd, dl.gate, dl.up, dl.down, *dl.sh, ro, ws=ws_m)
        torch.cuda.synchronize()
        _, o2, _ = gpu_window(dl, xd, cfg.top_k)
        assert np.array_equal(out.cpu().numpy(), o2)

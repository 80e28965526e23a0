"""GPU parity of the path the benchmark times: the layer call captured into one HIP graph
of 64 windows of the 8-row Zipf workload over 8 layer instances (bench.py's own Steps and
capture_steps), replayed.

Every window's routing must equal the oracle's bit for bit and its output be within the
row tolerance of the oracle's; the graph's results must equal the same steps run eagerly,
bit for bit; 100 further replays must reproduce the first one bit for bit.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import bench  # noqa: E402
import oracle  # noqa: E402
import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import (REL_TOL, assert_close, assert_route_equal, oracle_mats, oracle_window,  # noqa: E402
                         topk_gap)

STEPS, LAYERS = 64, 8


def bits(t):
    """The tensor's bytes as integers: equal bit patterns compare equal, NaN included (the
    routing arrays' padding past the written entries holds whatever the memory held)."""
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.fixture(scope="module")
def replayed():
    cfg = synth.config("four_slots_mtp_zipf")
    DevLayer, to_dev_x = bench.device_layer_types(torch, sw)
    print(f"[graph] {cfg.name}: {STEPS} windows over {LAYERS} layer instances", flush=True)
    st = bench.Steps(cfg, LAYERS, STEPS, STEPS, sw, torch, synth, DevLayer, to_dev_x, 1, "layer",
                     out_per_step=True, keep_host_layers=True)
    g = bench.capture_steps(torch, st, STEPS, 1)
    g.replay()
    torch.cuda.synchronize()
    outs = torch.stack(st.out).clone()
    routes = {n: t[:STEPS].clone() for n, t in st.big.items()}
    yield cfg, st, g, outs, routes
    del g
    torch.cuda.synchronize()


def _check_windows(cfg, st, outs, lo, hi):
    mats = {}
    for i in range(lo, hi):
        L = st.host_layers[i % LAYERS]
        if i % LAYERS not in mats:
            mats[i % LAYERS] = oracle_mats(L, cfg)
        x = synth.make_window(cfg, i, rows=cfg.rows)
        orc, oout, _ = oracle_window(L, mats[i % LAYERS], x, cfg)
        assert topk_gap(orc["logits"], cfg.top_k) > 1e-9
        assert_route_equal(st.routes[i].host(), orc, cfg)
        err, eerr = assert_close(outs[i].cpu().numpy(), oout)
        print(f"[graph] window {i} (layer {i % LAYERS}): row err {err:.2e}, element err {eerr:.2e}", flush=True)


def test_graph_windows_0_31_against_oracle(replayed):
    cfg, st, g, outs, routes = replayed
    _check_windows(cfg, st, outs, 0, STEPS // 2)


def test_graph_windows_32_63_against_oracle(replayed):
    cfg, st, g, outs, routes = replayed
    _check_windows(cfg, st, outs, STEPS // 2, STEPS)


def test_graph_equals_eager(replayed):
    """The same steps launched one call at a time give the graph's results bit for bit."""
    cfg, st, g, outs, routes = replayed
    for i in range(STEPS):
        st.out[i].fill_(float("nan"))
        st.step(i)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch.stack(st.out)), bits(outs))
    for n, t in st.big.items():
        assert torch.equal(bits(t[:STEPS]), bits(routes[n])), n


def test_graph_replays_bitwise(replayed):
    """100 replays of the captured graph reproduce the first replay bit for bit."""
    cfg, st, g, outs, routes = replayed
    for rep in range(100):
        for o in st.out:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(torch.stack(st.out)), bits(outs)), rep
        for n, t in st.big.items():
            assert torch.equal(bits(t[:STEPS]), bits(routes[n])), (rep, n)
    print("[graph] 100 replays bitwise equal", flush=True)

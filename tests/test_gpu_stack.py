"""GPU parity of strata_window_stack, the whole stack of MoE layers (residual between
layers) and the head in one call, where layer l's combine and layer l + 1's router GEMV
share a launch. Its routing, every layer's x_next and the head's logits must equal, bit
for bit, the same layers run one strata_window_layer call at a time; every layer is also
checked against the CPU oracle given that layer's own input."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import (REL_TOL, DevLayer, assert_route_equal, oracle_mats, oracle_window,  # noqa: E402
                         row_rel_err, to_dev_x, topk_gap)


def bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def chain(dls, xd, top_k, renorm):
    """The same layers, one strata_window_layer call at a time: every layer's input, the
    routes, the last layer's float output and the last x_next."""
    x, xs, routes, out = xd, [], [], None
    for dl in dls:
        xs.append(x)
        xn = torch.empty(x.shape, dtype=torch.bfloat16, device="cuda")
        out, ro = sw.strata_window_layer(x, dl.gate_w, dl.bias, top_k, dl.gate, dl.up, dl.down, *dl.sh,
                                         renorm=renorm, residual=x, x_next=xn)
        routes.append(ro.host())
        x = xn
    torch.cuda.synchronize()
    return xs, routes, out, x


def check_stack(cfg, n_layers, renorm=False, head=False, shared_route=False, oracle_layers=()):
    R, H, E, k = cfg.rows, cfg.hidden, cfg.experts, cfg.top_k
    print(f"[stack] {cfg.name} H={H} F={cfg.ffn} E={E} k={k} bits={cfg.bits} R={R} layers={n_layers} "
          f"renorm={renorm} head={head} shared_route={shared_route}", flush=True)
    Ls = [synth.make_layer(cfg, l) for l in range(n_layers)]
    dls = [DevLayer(L, cfg) for L in Ls]
    x = synth.make_window(cfg, 3)
    xd = to_dev_x(x)
    hq = None
    if head:
        codes, meta = synth.make_head(cfg)
        hq = sw.upload_qmat(codes, meta, cfg.vocab, H, 8)

    layers = [(dl.gate_w, dl.bias, dl.gate, dl.up, dl.down, *dl.sh) for dl in dls]
    routes = None if shared_route else [sw.RouteOut(R, E, k) for _ in dls]
    out = torch.empty(R, H, dtype=torch.float32, device="cuda")
    xf, routes, lg, am = sw.strata_window_stack(xd, layers, k, head=hq, renorm=renorm, routes=routes, out=out)
    torch.cuda.synchronize()
    s_routes = [ro.host() for ro in routes]
    xf_s, out_s = bits16(xf), out.cpu().numpy()
    lg_s = None if lg is None else lg.cpu().numpy()
    am_s = None if am is None else am.cpu().numpy()

    xs, c_routes, c_out, c_xf = chain(dls, xd, k, renorm)
    # the stack against the chain: bit for bit
    if not shared_route:
        for l in range(n_layers):
            for key in ("topk_idx", "topk_w", "active", "offsets", "entry_row", "entry_w", "row_mask", "entry_pos",
                        "row_w"):
                assert np.array_equal(s_routes[l][key], c_routes[l][key]), (l, key)
    else:
        for key in ("topk_idx", "active", "offsets", "entry_row", "row_w"):
            assert np.array_equal(s_routes[-1][key], c_routes[-1][key]), key
    assert np.array_equal(xf_s, bits16(c_xf))
    assert np.array_equal(out_s.view(np.uint32), c_out.cpu().numpy().view(np.uint32))
    if head:
        c_lg, c_am = sw.strata_window_head(c_xf, hq)
        torch.cuda.synchronize()
        assert np.array_equal(lg_s.view(np.uint32), c_lg.cpu().numpy().view(np.uint32))
        assert np.array_equal(am_s, c_am.cpu().numpy())

    # chosen layers against the oracle, given the layer's own input
    for l in oracle_layers:
        x_in = xs[l]
        x_np = x_in.cpu().numpy() if x_in.dtype == torch.float32 else bits16(x_in).view(np.uint16)
        orc, oout, _ = oracle_window(Ls[l], oracle_mats(Ls[l], cfg), x_np, cfg, renorm=renorm, residual=True)
        assert topk_gap(orc["logits"], k) > 1e-9
        assert_route_equal(s_routes[l], orc, cfg)
        if l == n_layers - 1:
            err = row_rel_err(out_s, oout)
            print(f"[stack] layer {l} vs oracle: rel err {err:.3e}", flush=True)
            assert err <= REL_TOL, err
    return s_routes


@pytest.mark.parametrize("renorm", [False, True])
def test_stack_float_input_two_chunks(renorm):
    """Layer 0 takes float activations (the fused hand-over reads a float residual), later
    layers bf16; hidden 1024 = two router chunks; 5 rows."""
    cfg = synth.config("small_f32", hidden=1024, ffn=256, experts=16, top_k=2, rows=5)
    check_stack(cfg, 3, renorm=renorm, oracle_layers=(0, 1, 2))


def test_stack_one_layer_is_the_layer_call():
    cfg = synth.config("small_f32", rows=3)
    check_stack(cfg, 1, oracle_layers=(0,))


def test_stack_zipf_bias_head_ragged_hidden():
    """The Zipf prior's bias in every layer, hidden 640 (a ragged last router chunk), a
    head, one routing buffer shared by the layers."""
    cfg = synth.config("four_slots_mtp_zipf", hidden=640, ffn=256, experts=24, top_k=4, vocab=1024)
    check_stack(cfg, 4, head=True, shared_route=True)


def test_stack_two_bit_256_experts():
    cfg = synth.config("e256_2bit", hidden=1024, ffn=256, rows=4)
    check_stack(cfg, 3, oracle_layers=(2,))


def test_stack24_head_full():
    """The layer-stack workload at its full size: 24 layers and the vocab-151936 head."""
    cfg = synth.config("stack24_head")
    check_stack(cfg, cfg.layers, head=True, oracle_layers=(0, 23))


def test_stack_hidden_beyond_the_fused_lds():
    """hidden 7936 (bf16): every layer takes the routing as a kernel of its own and the
    plain gate/up after the fused hand-over; still bit-identical to the layer calls."""
    cfg = synth.config("two_slots_mtp", hidden=7936, ffn=256, experts=16, top_k=4, rows=3)
    check_stack(cfg, 2, oracle_layers=(0, 1))

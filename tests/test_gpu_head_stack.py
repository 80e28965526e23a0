"""GPU parity of the 8-bit head and of the 24-layer stack (the layer-stack workload:
24 MoE layers of the 2048/768/128/top-8 shape with a residual add between layers, then a
head of vocab 151936), through the C ABI, against the CPU oracle."""
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
                         oracle_window, row_rel_err, to_dev_x, topk_gap)


def head_check(cfg, x, window_label):
    codes, meta = synth.make_head(cfg)
    print(f"[head] V={cfg.vocab} H={cfg.hidden} R={x.shape[0]} dtype={x.dtype} {window_label}", flush=True)
    hq = sw.upload_qmat(codes, meta, cfg.vocab, cfg.hidden, 8)
    lg, am = sw.strata_window_head(to_dev_x(x), hq)
    torch.cuda.synchronize()
    lg = lg.cpu().numpy(); am = am.cpu().numpy()
    q = oracle.qmat(codes[0], meta[0], cfg.vocab, cfg.hidden, 8)
    ol, oam = oracle.head(x, q)
    err = row_rel_err(lg, ol)
    assert err <= REL_TOL, err
    # the argmax is the first index of the GPU logits' maximum
    assert np.array_equal(am, np.argmax(lg, axis=1))
    # and the oracle's wherever the oracle's top two are apart by more than the tolerance
    for r in range(x.shape[0]):
        s = np.sort(ol[r])[::-1]
        if s[0] - s[1] > 1e-4 * np.max(np.abs(ol[r])):
            assert am[r] == oam[r], (r, am[r], oam[r])
    return err


def test_head_small_bf16():
    cfg = synth.config("stack24_head", vocab=4096)
    print("head rel err", head_check(cfg, synth.make_window(cfg, 0), "small"))


def test_head_small_f32_ragged_rows():
    cfg = synth.config("small_f32", vocab=1040, hidden=256, rows=5)
    head_check(cfg, synth.make_window(cfg, 1), "f32")


def test_head_f32_hidden_1920_lds_boundary():
    """Float rows at hidden 1920: the activation image takes exactly 64 KiB of dynamic LDS,
    which with the kernel's static LDS needs the raised limit."""
    cfg = synth.config("small_f32", vocab=1024, hidden=1920, rows=8)
    head_check(cfg, synth.make_window(cfg, 3), "f32 hidden 1920")


def test_head_large_magnitudes():
    """Rows scaled by 2^20 and 2^-20 stay exact through the per-row power-of-two scaling."""
    cfg = synth.config("stack24_head", vocab=2048, rows=3)
    x = synth.bf16_bits_to_f32(synth.make_window(cfg, 2))
    x[0] *= 2.0 ** 20
    x[2] *= 2.0 ** -20
    head_check(cfg, synth.f32_to_bf16_bits(x), "scaled")


def test_head_full_vocab():
    cfg = synth.config("stack24_head")
    print("head full rel err", head_check(cfg, synth.make_window(cfg, 0), "full"))


def test_layer_stack_teacher_forced():
    """24 layers back to back on the GPU (route, experts with residual, bf16 x_next feeds
    the next layer); every layer is checked against the oracle given the GPU's own input
    to that layer; then the head runs on the last layer's output."""
    cfg = synth.config("stack24_head")
    x = synth.make_window(cfg, 0)
    xd = to_dev_x(x)
    worst = 0.0
    for l in range(cfg.layers):
        L = synth.make_layer(cfg, l)
        dl = DevLayer(L, cfg)
        x_in = xd.view(torch.int16).cpu().numpy().view(np.uint16)
        gr, gout, gxn = gpu_window(dl, xd, cfg.top_k, residual=True, x_next=True)
        orc, oout, _ = oracle_window(L, oracle_mats(L, cfg), x_in, cfg, residual=True)
        assert topk_gap(orc["logits"], cfg.top_k) > 1e-9
        assert_route_equal(gr, orc, cfg)
        err = row_rel_err(gout, oout)
        worst = max(worst, err)
        print(f"[stack] layer {l}: rel err {err:.3e}", flush=True)
        assert err <= REL_TOL, (l, err)
        assert np.array_equal(gxn, synth.f32_to_bf16_bits(gout))
        xd = to_dev_x(gxn)
        del dl, L
    x_last = xd.view(torch.int16).cpu().numpy().view(np.uint16)
    print("stack worst layer rel err", worst, "final |x| max", float(np.abs(synth.bf16_bits_to_f32(x_last)).max()))
    head_check(cfg, x_last, "after 24 layers")

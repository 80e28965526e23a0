"""GPU parity of the per-window routing counts and the adaptive tier's swap choice,
through the C ABI, against the CPU oracle: counts bit-exact (float fmaf on both sides),
resident flags and swap pairs exact."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import DevLayer, to_dev_x  # noqa: E402


def random_mask(rng, E, R, k, zipf=False):
    p = None
    if zipf:
        w = 1.0 / np.arange(1, E + 1) ** 1.1
        p = w / w.sum()
    m = np.zeros(E + 1, np.uint8)
    for r in range(R):
        for e in rng.choice(E, k, replace=False, p=p):
            m[e] |= 1 << r
    m[E] = (1 << R) - 1
    return m


@pytest.mark.parametrize("E,decay,every,max_swaps,gain", [(128, 0.875, 4, 8, 1.5), (256, 1.0, 2, 16, 1.5),
                                                        (16, 0.5, 1, 4, 1.0), (64, 0.0, 3, 64, 2.0)])
def test_tier_sequence_matches_oracle(E, decay, every, max_swaps, gain):
    rng = np.random.default_rng(E + every)
    counts_h = np.zeros(E, np.float32)
    res_h = (rng.random(E) < 0.4).astype(np.uint8)
    counts_d = torch.zeros(E, dtype=torch.float32, device="cuda")
    res_d = torch.from_numpy(res_h.copy()).cuda()
    for w in range(12):
        mask = random_mask(rng, E, 8, min(8, E), zipf=True)
        mask_d = torch.from_numpy(mask).cuda()
        select = (w + 1) % every == 0
        print(f"[tier] E={E} window={w} select={select}", flush=True)
        counts_h = oracle.tier_count(mask, counts_h, decay)
        if select:
            res_h, sw_h = oracle.tier_select(counts_h, res_h, max_swaps, gain)
            swaps, n = sw.strata_window_tier(mask_d, counts_d, decay, res_d, max_swaps, gain)
        else:
            sw.strata_window_tier(mask_d, counts_d, decay)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(counts_d.cpu().numpy().view(np.uint32), counts_h.view(np.uint32))
        if select:
            nn = int(n[0].item())
            assert nn == len(sw_h)
            np.testing.assert_array_equal(swaps[:nn].cpu().numpy(), sw_h)
            np.testing.assert_array_equal(res_d.cpu().numpy(), res_h)


def test_tier_counts_from_gpu_routing():
    """The routing output of a config-2 window (Zipf prior, 8 rows) feeds the counts."""
    cfg = synth.config("four_slots_mtp_zipf")
    L = synth.make_layer(cfg, 0)
    dl = DevLayer(L, cfg)
    counts_d = torch.zeros(cfg.experts, dtype=torch.float32, device="cuda")
    counts_h = np.zeros(cfg.experts, np.float32)
    for w in range(4):
        print(f"[tier] routed window {w}", flush=True)
        ro = sw.strata_window_route(to_dev_x(synth.make_window(cfg, w)), dl.gate_w, dl.bias, cfg.top_k)
        sw.strata_window_tier(ro.row_mask, counts_d, 0.875)
        torch.cuda.synchronize()
        counts_h = oracle.tier_count(ro.row_mask.cpu().numpy(), counts_h, 0.875)
    np.testing.assert_array_equal(counts_d.cpu().numpy().view(np.uint32), counts_h.view(np.uint32))
    assert counts_h.sum() > 0

"""GPU check of strata_window_layer_noalloc (the layer call whose workspace is the
library's fixed per-GPU scratch array): two calls in a row, the second on a smaller
window, each equal bit for bit to strata_window_layer with a caller workspace, and each
checked against the oracle."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import (DevLayer, assert_close, assert_route_equal, oracle_mats, oracle_window,  # noqa: E402
                         to_dev_x, topk_gap)


def test_noalloc_equals_layer_call_twice():
    cfg = synth.config("four_slots_mtp_zipf")
    L = synth.make_layer(cfg, 0)
    dl = DevLayer(L, cfg)
    mats = oracle_mats(L, cfg)
    for rows, window in ((8, 3), (3, 4)):
        print(f"[noalloc] {cfg.name} rows={rows} window={window}", flush=True)
        x = synth.make_window(cfg, window)[:rows]
        xd = to_dev_x(x)
        ref, rref = sw.strata_window_layer(xd, dl.gate_w, dl.bias, cfg.top_k, dl.gate, dl.up, dl.down, *dl.sh)
        got, rgot = sw.strata_window_layer_noalloc(xd, dl.gate_w, dl.bias, cfg.top_k, dl.gate, dl.up, dl.down,
                                                   *dl.sh)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        hg, hr = rgot.host(), rref.host()
        for k in hr:
            assert np.array_equal(np.asarray(hg[k]), np.asarray(hr[k])), k
        orc, oout, _ = oracle_window(L, mats, x, cfg)
        assert topk_gap(orc["logits"], cfg.top_k) > 1e-9
        assert_route_equal(hg, orc, cfg)
        err, eerr = assert_close(got.cpu().numpy(), oout)
        print(f"[noalloc] rows={rows}: equal to the layer call; oracle row err {err:.2e}", flush=True)


def test_noalloc_rejects_shape_beyond_scratch():
    """A valid shape whose workspace exceeds the fixed array is refused before any launch."""
    need = sw.workspace_bytes(3, 8, 7936, 4096, 256, 8)
    assert need > sw.NOALLOC_SCRATCH_BYTES
    cfg = synth.config("four_slots_mtp_zipf")
    L = synth.make_layer(cfg, 0)
    dl = DevLayer(L, cfg)
    x = to_dev_x(synth.make_window(cfg, 0))
    # the shape check comes first: a hidden of 7936 against this layer's matrices is refused
    # for its size before the matrices are looked at
    lib = sw.library()
    qs = [q.c() for q in (dl.gate, dl.up, dl.down, *dl.sh)]
    ro = sw.RouteOut(8, cfg.experts, cfg.top_k)
    import ctypes
    rc = lib.strata_window_layer_noalloc(None, x.data_ptr(), 1, 8, 7936, 4096, dl.gate_w.data_ptr(), None, 0,
                                         *[ctypes.byref(q) for q in qs], 256, 8, ctypes.byref(ro.c()), None,
                                         x.data_ptr(), None, None)
    assert rc == sw.STRATA_EINVAL
    assert b"scratch" in lib.strata_window_last_error()

"""Shared pieces of the GPU parity tests: upload synthetic layers, run windows through the
C ABI (via the binding), run the same windows through the CPU oracle, compare."""
import numpy as np
import torch

import oracle
import synth
import verify_window_expert_amd as sw


def to_dev_x(x):
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


class DevLayer:
    """One MoE layer's weights on the device."""

    def __init__(self, layer, cfg):
        H, F, b = cfg.hidden, cfg.ffn, cfg.bits
        self.cfg = cfg
        self.gate_w = torch.from_numpy(layer.gate_w).cuda()
        self.bias = None if layer.bias is None else torch.from_numpy(layer.bias).cuda()
        up = lambda m, r, c: sw.upload_qmat(m[0], m[1], r, c, b)
        self.gate, self.up, self.down = up(layer.gate, F, H), up(layer.up, F, H), up(layer.down, H, F)
        self.sh = (up(layer.sh_gate, F, H), up(layer.sh_up, F, H), up(layer.sh_down, H, F))


def oracle_mats(layer, cfg):
    H, F, b, E = cfg.hidden, cfg.ffn, cfg.bits, cfg.experts
    q = lambda m, n, r, c: oracle.qmat(m[0], m[1], r, c, b, n)
    return (q(layer.gate, E, F, H), q(layer.up, E, F, H), q(layer.down, E, H, F),
            q(layer.sh_gate, 1, F, H), q(layer.sh_up, 1, F, H), q(layer.sh_down, 1, H, F))


def gpu_window(dl, x_dev, top_k, renorm=False, residual=False, x_next=False, layer=False):
    """Route + experts of one window on the GPU, by strata_window_route and then
    strata_window_moe, or (layer) by strata_window_layer. Returns (route host dict, out np,
    x_next np)."""
    xn = torch.empty(x_dev.shape, dtype=torch.bfloat16, device="cuda") if x_next else None
    if layer:
        out, ro = sw.strata_window_layer(x_dev, dl.gate_w, dl.bias, top_k, dl.gate, dl.up, dl.down, *dl.sh,
                                         renorm=renorm, residual=x_dev if residual else None, x_next=xn)
    else:
        ro = sw.strata_window_route(x_dev, dl.gate_w, dl.bias, top_k, renorm=renorm)
        out = sw.strata_window_moe(x_dev, dl.gate, dl.up, dl.down, *dl.sh, ro,
                                   residual=x_dev if residual else None, x_next=xn)
    torch.cuda.synchronize()
    xnn = None if xn is None else xn.view(torch.int16).cpu().numpy().view(np.uint16)
    return ro.host(), out.cpu().numpy(), xnn


def oracle_window(layer, mats, x, cfg, renorm=False, residual=False, x_next=False):
    logits, probs, idx, w = oracle.route(x, layer.gate_w, layer.bias, cfg.top_k, renorm)
    grp = oracle.group(idx, w, cfg.experts)
    res = oracle.moe(x, *mats, idx, w, residual=x if residual else None, want_x_next=x_next)
    out, xn = res if x_next else (res, None)
    return dict(logits=logits, idx=idx, w=w, group=grp), out, xn


def topk_gap(logits, k):
    """Smallest gap between each row's k-th and (k+1)-th largest logit."""
    s = -np.sort(-logits, axis=1)
    if s.shape[1] <= k:
        return np.inf
    return float(np.min(s[:, k - 1] - s[:, k]))


def assert_route_equal(gr, orc, cfg):
    """Bit-exact routing indices and per-expert row lists; weights to float rounding."""
    assert np.array_equal(gr["topk_idx"], orc["idx"]), (gr["topk_idx"], orc["idx"])
    g = orc["group"]
    assert gr["n_active"] == g["n_active"]
    assert np.array_equal(gr["active"], g["active"])
    assert np.array_equal(gr["offsets"], g["offsets"])
    assert np.array_equal(gr["entry_row"], g["entry_row"])
    assert np.array_equal(gr["row_mask"], g["row_mask"])
    # the GPU rounds each double-precision weight to float (tiny ones to 0 or subnormal)
    np.testing.assert_allclose(gr["topk_w"], orc["w"].astype(np.float32), rtol=1e-6, atol=1e-44)
    np.testing.assert_allclose(gr["entry_w"], g["entry_w"].astype(np.float32), rtol=1e-6, atol=1e-44)
    # each row's list of experts in ascending id order (shared last): every entry's place
    # in it, and the row's weights in that order, derived here from the oracle's top-k
    idx, w = orc["idx"], orc["w"]
    R, K = idx.shape
    place, row_w = {}, np.zeros((R, K + 1))
    for r in range(R):
        for p, j in enumerate(np.argsort(idx[r], kind="stable")):
            place[(r, int(idx[r][j]))] = p
            row_w[r, p] = w[r, j]
        row_w[r, K] = 1.0
    E = cfg.experts
    want_pos = []
    for a, e in enumerate(g["active"]):
        for n in range(g["offsets"][a], g["offsets"][a + 1]):
            r = int(g["entry_row"][n])
            want_pos.append(K if e == E else place[(r, int(e))])
    assert np.array_equal(gr["entry_pos"], np.array(want_pos)), (gr["entry_pos"], want_pos)
    np.testing.assert_allclose(gr["row_w"], row_w.astype(np.float32), rtol=1e-6, atol=1e-44)


# The tolerance the layer's outputs are held to: per row, max |gpu - oracle| over
# max |oracle| (float32 accumulation against the double-precision definition).
REL_TOL = 2e-3


def row_rel_err(g, o):
    """Per row max |g - o| / max |o|; a row whose reference is all zero counts its
    absolute error instead."""
    g = np.atleast_2d(g); o = np.atleast_2d(o)
    num = np.max(np.abs(g - o), axis=1)
    den = np.max(np.abs(o), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


# The element-wise error: |gpu - oracle| over max(|oracle|, 1e-3 * the row's max |oracle|),
# reported beside the row metric. Near zero it is 1000 times the error relative to the
# row's max: float32 accumulation of a row (every product exact, sums of up to 4096 terms)
# has measured 1.7e-5 of the row's max at worst (1.3e-2 in this metric), so 5e-2 bounds the
# error of the smallest elements 40 times tighter than the row tolerance does.
ELEM_FLOOR = 1e-3
ELEM_TOL = 5e-2


def elem_rel_err(g, o):
    """Max over elements of |g - o| / max(|o|, ELEM_FLOOR * max |o| of the element's row)."""
    g = np.atleast_2d(g); o = np.atleast_2d(o)
    floor = ELEM_FLOOR * np.max(np.abs(o), axis=1, keepdims=True)
    den = np.maximum(np.abs(o), floor)
    num = np.abs(g - o)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def assert_close(g, o):
    """Row metric within REL_TOL (and the floored element metric within ELEM_TOL when set);
    returns both."""
    err, eerr = row_rel_err(g, o), elem_rel_err(g, o)
    assert err <= REL_TOL, (err, eerr)
    if ELEM_TOL is not None:
        assert eerr <= ELEM_TOL, (err, eerr)
    return err, eerr

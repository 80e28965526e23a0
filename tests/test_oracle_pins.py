"""Pins of the CPU oracle against what the definition and the mathematics fix.

Each test checks the oracle against something other than itself: library routines
(NumPy float16/float64, np.lexsort, np.argmax, scipy's softmax/expit), closed forms,
invariants, special cases that reduce to a dense SwiGLU FFN, and the dense brute force
of all experts masked to the routing (tests/npref.py, an independent NumPy decoding).
The layer's definition is Strata docs/BATCHING.md, "Several requests at once (batch
slots)", opening paragraph and "Exactness".
"""
import math

import numpy as np
import pytest

import npref
import synth


# ------------------------------------------------------------------ number formats

def test_f16_decode_matches_numpy(oracle_lib):
    # every binary16 bit pattern that is finite
    for h in list(range(0, 0x7C00, 37)) + [0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001, 0xBC00, 0xFBFF]:
        want = float(np.array([h], np.uint16).view(np.float16)[0])
        assert oracle_lib.f16_to_double(h) == want, hex(h)


def test_bf16_decode_matches_bitcast(oracle_lib):
    for h in [0x0000, 0x0001, 0x3F80, 0x4049, 0xC2F7, 0x7F7F, 0x0080, 0x807F]:
        want = float(np.array([h << 16], np.uint32).view(np.float32)[0])
        assert oracle_lib.bf16_to_double(h) == want


def _bf16_val(h):
    return float(np.array([h << 16], np.uint32).view(np.float32)[0])


def test_bf16_rounding_is_nearest_even(oracle_lib):
    """Brute force: the result is the nearest bf16 value; on an exact tie, the even one."""
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(400) * 10.0 ** rng.integers(-30, 30, 400))
    # exact ties between two bf16 neighbours, both parities
    for h in [0x3F80, 0x3F81, 0x4000, 0x4001, 0xC123, 0xC124]:
        vals.append((_bf16_val(h) + _bf16_val(h + 1)) / 2)
    for v in vals:
        h = oracle_lib.double_to_bf16(v)
        got = _bf16_val(h)
        base = np.array([v], np.float32).view(np.uint32)[0] >> 16
        cands = [int(base) + d for d in (-2, -1, 0, 1, 2)]
        dist = {c: abs(_bf16_val(c) - v) for c in cands}
        best = min(dist.values())
        assert abs(got - v) == best, (v, hex(h))
        ties = [c for c in cands if dist[c] == best]
        if len(ties) > 1:
            assert h % 2 == 0, (v, hex(h))


# ------------------------------------------------------------------ layout + dequant

@pytest.mark.parametrize("bits", [2, 4, 8])
def test_layout_roundtrip_known_codes(oracle_lib, bits):
    """Codes placed by the NumPy packer read back at the same (n, k) through the oracle."""
    rows, cols = 32, 2 * (512 // bits)
    rng = np.random.default_rng(bits)
    lo, hi = (-127, 128) if bits == 8 else (0, 1 << bits)
    dense = rng.integers(lo, hi, size=(rows, cols))
    codes = npref.pack_codes(dense, bits)
    nblk = rows * cols // 32
    meta = np.zeros(nblk, np.uint16 if bits == 8 else np.uint32)
    q = oracle_lib.qmat(codes, meta, rows, cols, bits)
    for n in range(rows):
        for k in range(cols):
            assert oracle_lib.code(q, 0, n, k) == dense[n, k]
    assert np.array_equal(npref.unpack_codes(codes, rows, cols, bits), dense)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_dequant_closed_form_every_code(oracle_lib, bits):
    """W = scale*q + min (affine) / scale*q (8-bit), exactly, over every code value."""
    rows, cols = 16, 512 // bits
    ncode = 1 << bits
    k = np.arange(cols)
    dense = np.tile((k % ncode) - (128 if bits == 8 else 0), (rows, 1)) + np.arange(rows)[:, None] % 3
    dense = np.clip(dense, -127 if bits == 8 else 0, 127 if bits == 8 else ncode - 1)
    rng = np.random.default_rng(7)
    scale = rng.uniform(0.01, 2.0, size=(rows, cols // 32)).astype(np.float16)
    mn = rng.uniform(-3.0, 3.0, size=(rows, cols // 32)).astype(np.float16)
    codes = npref.pack_codes(dense, bits)
    meta = npref.pack_meta(scale, mn, bits)
    q = oracle_lib.qmat(codes, meta, rows, cols, bits)
    W = oracle_lib.dequant(q)
    s = np.repeat(scale.astype(np.float64), 32, axis=1)
    m = np.repeat(mn.astype(np.float64), 32, axis=1) if bits != 8 else 0.0
    assert np.array_equal(W, s * dense + m)


def test_generated_weights_are_exact_in_float32(oracle_lib):
    """The generator's (scale, min) keep every dequantised weight exact in float32."""
    cfg = synth.config("two_slots_mtp")
    codes, meta = synth.qmatrix(np.random.default_rng(3), 1, 32, cfg.hidden, 4)
    q = oracle_lib.qmat(codes[0], meta[0], 32, cfg.hidden, 4)
    W = oracle_lib.dequant(q)
    assert np.array_equal(W.astype(np.float32).astype(np.float64), W)


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_logits_match_float64_matmul(oracle_lib, dtype):
    cfg = synth.config("two_slots_mtp", x_dtype=dtype)
    gate_w, _ = synth.make_router(cfg)
    x = synth.make_window(cfg, 5)
    logits, probs, idx, w = oracle_lib.route(x, gate_w, None, cfg.top_k)
    ref = npref.act(x) @ gate_w.astype(np.float64).T
    assert np.allclose(logits, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_router_one_hot_returns_gate_column(oracle_lib):
    E, H = 16, 256
    G = np.random.default_rng(1).normal(0, 0.02, (E, H)).astype(np.float32)
    x = np.zeros((3, H), np.float32)
    for r, h in enumerate([0, 77, 255]):
        x[r, h] = 1.0
    logits, *_ = oracle_lib.route(x, G, None, 2)
    for r, h in enumerate([0, 77, 255]):
        assert np.array_equal(logits[r], G[:, h].astype(np.float64))


def test_router_bias_is_added(oracle_lib):
    E, H = 16, 256
    rng = np.random.default_rng(2)
    G = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    b = rng.normal(0, 1, E).astype(np.float32)
    x = rng.standard_normal((2, H)).astype(np.float32)
    l0, *_ = oracle_lib.route(x, G, None, 2)
    l1, *_ = oracle_lib.route(x, G, b, 2)
    assert np.allclose(l1 - l0, b.astype(np.float64)[None, :], rtol=0, atol=1e-14)


def test_softmax_properties(oracle_lib):
    from scipy.special import softmax
    E, H = 16, 256
    rng = np.random.default_rng(4)
    G = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    x = rng.standard_normal((4, H)).astype(np.float32)
    logits, probs, _, _ = oracle_lib.route(x, G, None, 3)
    assert np.allclose(probs.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.allclose(probs, softmax(logits, axis=1), rtol=1e-12, atol=0)
    # shift invariance: a constant bias on every expert changes no probability
    _, p2, i2, _ = oracle_lib.route(x, G, np.full(E, 3.25, np.float32), 3)
    assert np.allclose(p2, probs, rtol=1e-12, atol=0)
    # equal logits -> uniform
    _, pu, _, _ = oracle_lib.route(np.zeros((1, H), np.float32), G, None, 3)
    assert np.allclose(pu, 1.0 / E, rtol=1e-15, atol=0)


@pytest.mark.parametrize("renorm", [False, True])
def test_topk_matches_lexsort(oracle_lib, renorm):
    cfg = synth.config("four_slots_mtp_zipf")
    gate_w, bias = synth.make_router(cfg)
    x = synth.make_window(cfg, 1)
    logits, probs, idx, w = oracle_lib.route(x, gate_w, bias, cfg.top_k, renorm)
    _, _, ridx, rw = npref.route_bruteforce(npref.act(x), gate_w, bias, cfg.top_k, renorm)
    assert np.array_equal(idx, ridx)
    assert np.allclose(w, rw, rtol=1e-12, atol=0)
    if renorm:
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)


def test_topk_forced_ties_take_lower_index(oracle_lib):
    E, H = 16, 256
    # all-zero router: every logit equal -> experts 0..k-1
    _, _, idx, _ = oracle_lib.route(np.ones((2, H), np.float32), np.zeros((E, H), np.float32), None, 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (2, 1)))
    # duplicated router rows: identical logits, the lower index first
    rng = np.random.default_rng(9)
    G = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    G[11] = G[3] = G[5] * 4.0      # strongly preferred by x = G[5]-like rows
    x = (G[5:6] * 100).astype(np.float32)
    _, _, idx, _ = oracle_lib.route(x, G, None, 3)
    assert list(idx[0]) == [3, 11, 5]


# ------------------------------------------------------------------ grouping

def test_grouping_bruteforce(oracle_lib):
    cfg = synth.config("four_slots_mtp_zipf")
    gate_w, bias = synth.make_router(cfg)
    for win in range(3):
        x = synth.make_window(cfg, win)
        _, _, idx, w = oracle_lib.route(x, gate_w, bias, cfg.top_k)
        g = oracle_lib.group(idx, w, cfg.experts)
        R, K, E = cfg.rows, cfg.top_k, cfg.experts
        used = sorted(set(idx.ravel().tolist()))
        assert list(g["active"]) == used + [E]
        assert g["n_active"] == len(used) + 1
        assert g["offsets"][-1] == R * K + R
        seen = set()
        for a, e in enumerate(g["active"]):
            rows = list(g["entry_row"][g["offsets"][a]:g["offsets"][a + 1]])
            want = list(range(R)) if e == E else [r for r in range(R) if e in idx[r]]
            assert rows == want
            for t, r in enumerate(rows):
                ww = g["entry_w"][g["offsets"][a] + t]
                if e == E:
                    assert ww == 1.0
                else:
                    assert ww == w[r][list(idx[r]).index(e)]
                seen.add((r, e))
            assert g["row_mask"][e] == sum(1 << r for r in rows)
        assert len(seen) == R * K + R
        unused = [e for e in range(E) if e not in used]
        assert all(g["row_mask"][e] == 0 for e in unused)


# ------------------------------------------------------------------ experts

def _single_expert_cfg():
    return synth.config("small_f32", experts=1, top_k=1)


def test_single_expert_reduces_to_dense_swiglu(oracle_lib):
    """E = 1, k = 1, renormalised: out = FFN_0(x) + FFN_shared(x), a dense SwiGLU pair."""
    cfg = _single_expert_cfg()
    layer = synth.make_layer(cfg)
    x = synth.make_window(cfg, 0)
    H, F, b = cfg.hidden, cfg.ffn, cfg.bits
    q = lambda m, i, r, c: oracle_lib.qmat(m[0][i], m[1][i], r, c, b)
    _, _, idx, w = oracle_lib.route(x, layer.gate_w, None, 1, renorm=True)
    assert np.all(idx == 0) and np.all(w == 1.0)
    out = oracle_lib.moe(x, q(layer.gate, 0, F, H), q(layer.up, 0, F, H), q(layer.down, 0, H, F),
                         q(layer.sh_gate, 0, F, H), q(layer.sh_up, 0, F, H), q(layer.sh_down, 0, H, F), idx, w)
    X = npref.act(x)
    D = lambda m, r, c: npref.dequant(m[0][0], m[1][0], r, c, b)
    ref = (npref.dense_ffn(D(layer.gate, F, H), D(layer.up, F, H), D(layer.down, H, F), X)
           + npref.dense_ffn(D(layer.sh_gate, F, H), D(layer.sh_up, F, H), D(layer.sh_down, H, F), X))
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_constant_blocks_closed_form(oracle_lib):
    """scale = 0, min = c everywhere: g = cg*sum(x), u = cu*sum(x), y[n] = cd*F*silu(g)*u."""
    H, F, bits = 256, 128, 4
    x = np.random.default_rng(5).standard_normal((1, H)).astype(np.float32)
    def const(rows, cols, c):
        codes = np.random.default_rng(rows + cols).integers(0, 256, rows * cols // 2, dtype=np.uint8)
        scale = np.zeros((rows, cols // 32), np.float16)
        mn = np.full((rows, cols // 32), c, np.float16)
        return oracle_lib.qmat(codes, npref.pack_meta(scale, mn, bits), rows, cols, bits)
    cg, cu, cd = 0.0625, -0.125, 0.5
    y = oracle_lib.expert(const(F, H, cg), const(F, H, cu), const(H, F, cd), 0, x[0].astype(np.float64))
    sx = math.fsum(x[0].astype(np.float64))
    g, u = cg * sx, cu * sx
    h = g / (1.0 + math.exp(-g)) * u
    assert np.allclose(y, cd * F * h, rtol=1e-13, atol=0)


def test_zero_up_projection_gives_zero(oracle_lib):
    H, F, bits = 256, 128, 4
    rng = np.random.default_rng(6)
    x = rng.standard_normal(H)
    cfg = synth.config("small_f32")
    g = synth.qmatrix(rng, 1, F, H, bits)
    d = synth.qmatrix(rng, 1, H, F, bits)
    zero_meta = np.zeros(F * H // 32, np.uint32)
    up = oracle_lib.qmat(g[0][0], zero_meta, F, H, bits)
    y = oracle_lib.expert(oracle_lib.qmat(g[0][0], g[1][0], F, H, bits), up,
                          oracle_lib.qmat(d[0][0], d[1][0], H, F, bits), 0, x)
    assert np.all(y == 0.0)


def _layer_qmats(oracle_lib, layer, cfg):
    H, F, b, E = cfg.hidden, cfg.ffn, cfg.bits, cfg.experts
    qm = lambda m, n, r, c: oracle_lib.qmat(m[0], m[1], r, c, b, n)
    return (qm(layer.gate, E, F, H), qm(layer.up, E, F, H), qm(layer.down, E, H, F),
            qm(layer.sh_gate, 1, F, H), qm(layer.sh_up, 1, F, H), qm(layer.sh_down, 1, H, F))


@pytest.mark.parametrize("renorm,residual", [(False, False), (True, True)])
def test_layer_matches_dense_bruteforce_masked(oracle_lib, renorm, residual):
    cfg = synth.config("small_f32")
    layer = synth.make_layer(cfg)
    mats = _layer_qmats(oracle_lib, layer, cfg)
    for win in range(2):
        x = synth.make_window(cfg, win)
        _, _, idx, w = oracle_lib.route(x, layer.gate_w, layer.bias, cfg.top_k, renorm)
        out = oracle_lib.moe(x, *mats, idx, w, residual=x if residual else None)
        ref, ridx, rw = npref.layer_dense(x, layer, cfg, renorm=renorm, residual=residual)
        assert np.array_equal(idx, ridx)
        assert np.allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_reduced_shape_bf16_pairs_zipf_bruteforce(oracle_lib):
    """A reduced four_slots_mtp_zipf-like window: bf16 pairs, Zipf prior, 8 rows, 2-bit weights."""
    cfg = synth.config("four_slots_mtp_zipf", hidden=256, ffn=256, experts=12, top_k=3, bits=2)
    layer = synth.make_layer(cfg)
    mats = _layer_qmats(oracle_lib, layer, cfg)
    x = synth.make_window(cfg, 3)
    _, _, idx, w = oracle_lib.route(x, layer.gate_w, layer.bias, cfg.top_k)
    out = oracle_lib.moe(x, *mats, idx, w)
    ref, ridx, _ = npref.layer_dense(x, layer, cfg)
    assert np.array_equal(idx, ridx)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_full_mixture_when_k_equals_e(oracle_lib):
    """k = E with renormalisation: the output is the full softmax mixture of all experts."""
    cfg = synth.config("small_f32", experts=4, top_k=4)
    layer = synth.make_layer(cfg)
    mats = _layer_qmats(oracle_lib, layer, cfg)
    x = synth.make_window(cfg, 2)
    _, probs, idx, w = oracle_lib.route(x, layer.gate_w, None, 4, renorm=True)
    out = oracle_lib.moe(x, *mats, idx, w)
    X = npref.act(x)
    H, F, b = cfg.hidden, cfg.ffn, cfg.bits
    ref = np.zeros_like(X)
    for e in range(4):
        D = lambda m, r, c: npref.dequant(m[0][e], m[1][e], r, c, b)
        ref += probs[:, e:e + 1] * npref.dense_ffn(D(layer.gate, F, H), D(layer.up, F, H), D(layer.down, H, F), X)
    Ds = lambda m, r, c: npref.dequant(m[0][0], m[1][0], r, c, b)
    ref += npref.dense_ffn(Ds(layer.sh_gate, F, H), Ds(layer.sh_up, F, H), Ds(layer.sh_down, H, F), X)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


def test_window_row_equals_row_alone(oracle_lib):
    """Batching invariance (Strata docs/BATCHING.md, "Exactness"): bitwise in the oracle."""
    cfg = synth.config("small_f32", rows=2)
    layer = synth.make_layer(cfg)
    mats = _layer_qmats(oracle_lib, layer, cfg)
    x = synth.make_window(cfg, 4)
    _, _, idx, w = oracle_lib.route(x, layer.gate_w, None, cfg.top_k)
    out = oracle_lib.moe(x, *mats, idx, w)
    for r in range(cfg.rows):
        _, _, i1, w1 = oracle_lib.route(x[r:r + 1], layer.gate_w, None, cfg.top_k)
        o1 = oracle_lib.moe(x[r:r + 1], *mats, i1, w1)
        assert np.array_equal(i1[0], idx[r])
        assert np.array_equal(o1[0], out[r])


def test_x_next_is_bf16_of_output(oracle_lib):
    cfg = synth.config("two_slots_mtp", hidden=256, ffn=128, experts=8, top_k=2)
    layer = synth.make_layer(cfg)
    mats = _layer_qmats(oracle_lib, layer, cfg)
    x = synth.make_window(cfg, 0)
    _, _, idx, w = oracle_lib.route(x, layer.gate_w, None, cfg.top_k)
    out, xn = oracle_lib.moe(x, *mats, idx, w, residual=x, want_x_next=True)
    # nearest bf16 of each value: within half a bf16 ulp
    xv = npref.act(xn)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(out))) - 7)
    assert np.all(np.abs(xv - out) <= ulp / 2)


# ------------------------------------------------------------------ head

def test_head_matches_dense_and_argmax(oracle_lib):
    cfg = synth.config("stack24_head", vocab=512, hidden=256)
    codes, meta = synth.make_head(cfg)
    q = oracle_lib.qmat(codes[0], meta[0], cfg.vocab, cfg.hidden, 8)
    x = synth.make_window(cfg, 0)
    logits, am = oracle_lib.head(x, q)
    W = npref.dequant(codes[0], meta[0], cfg.vocab, cfg.hidden, 8)
    ref = npref.act(x) @ W.T
    assert np.allclose(logits, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(am, np.argmax(ref, axis=1))
    # a sub-range returns the same logits and an argmax within it
    l2, am2 = oracle_lib.head(x, q, 100, 300)
    assert np.array_equal(l2, logits[:, 100:300])
    assert np.array_equal(am2, 100 + np.argmax(ref[:, 100:300], axis=1))


def test_head_argmax_ties_take_lower_index(oracle_lib):
    V, H = 64, 64
    dense = np.zeros((V, H), np.int64)
    dense[[9, 40, 41], :] = 5          # three identical best rows
    dense[3, :] = 4
    codes = npref.pack_codes(dense, 8)
    scale = np.full((V, H // 32), 0.5, np.float16)
    q = oracle_lib.qmat(codes, npref.pack_meta(scale, None, 8), V, H, 8)
    x = np.ones((2, H), np.float32)
    _, am = oracle_lib.head(x, q)
    assert list(am) == [9, 9]


# ---------------------------------------------------------------- verify / accept
# Greedy verification of one MTP proposal per slot (Strata docs/BATCHING.md, --batch-mtp
# paragraph; docs/MULTI_GPU.md, --pipeline-windows paragraph: an accepted window yields a
# bonus token).

def test_accept_hand_cases(oracle_lib):
    # slot 0: proposal 7 == argmax of its token row -> kept, bonus 9
    # slot 1: proposal 4 != 5 -> rejected, emits the correction 5
    # slot 2: proposal 0 == 0 -> kept, bonus 0
    argmax = np.array([7, 9, 5, 6, 0, 0], np.int32)
    tokens, n_tok, kept = oracle_lib.accept(argmax, np.array([7, 4, 0], np.int32))
    np.testing.assert_array_equal(tokens, [[7, 9], [5, -1], [0, 0]])
    np.testing.assert_array_equal(n_tok, [2, 1, 2])
    assert kept == 2


def test_accept_without_mtp_emits_one_token_per_row(oracle_lib):
    argmax = np.array([3, 1, 4, 1, 5, 9, 2, 6], np.int32)
    tokens, n_tok, kept = oracle_lib.accept(argmax, None, mtp=False)
    np.testing.assert_array_equal(tokens[:, 0], argmax)
    assert (tokens[:, 1] == -1).all() and (n_tok == 1).all() and kept == 0


def test_accept_reproduces_serial_greedy_decoding(oracle_lib):
    """Speculative windows give the serial loop's tokens: a toy greedy model whose next
    token is a fixed function of the current one, four slots decoding in windows with a
    drafter that is right about two times in three, against plain one-token-at-a-time
    greedy decoding of the same model."""
    rng = np.random.default_rng(5)
    V = 50
    nxt = rng.integers(0, V, size=V)            # the model: next token after t

    def serial(t0, n):
        out, t = [], t0
        for _ in range(n):
            t = int(nxt[t])
            out.append(t)
        return out

    slots = 4
    starts = rng.integers(0, V, size=slots)
    gen = [[] for _ in range(slots)]
    cur = [int(s) for s in starts]
    total_kept = total_windows = 0
    while min(len(g) for g in gen) < 40:
        # drafter: right with probability 2/3, otherwise a wrong token
        prop = np.array([int(nxt[c]) if rng.random() < 2 / 3 else int((nxt[c] + 1 + rng.integers(V - 1)) % V)
                         for c in cur], np.int32)
        # the window's rows: (token, proposal) per slot; the model's argmax per row
        argmax = np.array([int(nxt[v]) for c, p in zip(cur, prop) for v in (c, p)], np.int32)
        tokens, n_tok, kept = oracle_lib.accept(argmax, prop)
        total_kept += kept
        total_windows += slots
        for s in range(slots):
            emitted = [int(t) for t in tokens[s, :n_tok[s]]]
            gen[s].extend(emitted)
            cur[s] = emitted[-1]
    for s in range(slots):
        assert gen[s] == serial(int(starts[s]), len(gen[s]))
    assert 0.5 < total_kept / total_windows < 0.8


# ------------------------------------------------------- routing counts and the tier
# Strata docs/BATCHING.md, the paragraph on batch windows counting the experts they route
# to (--adapt-every, --adapt-decay, --adapt-min-gain, whose default is 1.5): per-expert
# counts accumulate over windows; a periodic round exchanges well-used experts outside
# the fast tier for little-used resident ones while the count ratio clears the bar.

def test_tier_count_matches_bruteforce_and_decay_closed_form(oracle_lib):
    rng = np.random.default_rng(3)
    E, R = 64, 8
    c = np.zeros(E, np.float32)
    hist = np.zeros(E)
    for w in range(6):
        idx = np.stack([rng.choice(E, 8, replace=False) for _ in range(R)])
        mask = np.zeros(E + 1, np.uint8)
        for r in range(R):
            for e in idx[r]:
                mask[e] |= 1 << r
        mask[E] = 0xFF                                   # the shared expert: not counted
        c = oracle_lib.tier_count(mask, c, 0.5)
        hist = hist * 0.5 + np.bincount(idx.ravel(), minlength=E)   # closed form, exact in binary
    np.testing.assert_array_equal(c, hist.astype(np.float32))


def test_tier_select_hand_case(oracle_lib):
    counts = np.array([9, 0, 4, 6, 1, 3, 2, 5], np.float32)
    resident = np.array([0, 1, 0, 1, 1, 0, 1, 0], np.uint8)
    # outside, by count: 0 (9), 7 (5), 2 (4), 5 (3); resident, ascending: 1 (0), 4 (1), 6 (2), 3 (6)
    # pairs: 9 vs 0 ok, 5 vs 1 ok, 4 vs 2 ok (4 >= 3), 3 vs 6 fails
    res, sw = oracle_lib.tier_select(counts, resident, max_swaps=8, min_gain=1.5)
    np.testing.assert_array_equal(sw, [[0, 1], [7, 4], [2, 6]])
    np.testing.assert_array_equal(res, [1, 0, 1, 1, 0, 0, 0, 1])
    _, sw2 = oracle_lib.tier_select(counts, resident, max_swaps=2, min_gain=1.5)
    np.testing.assert_array_equal(sw2, [[0, 1], [7, 4]])
    _, sw3 = oracle_lib.tier_select(counts, resident, max_swaps=8, min_gain=2.5)   # 4 < 2.5 * 2
    np.testing.assert_array_equal(sw3, [[0, 1], [7, 4]])


def test_tier_select_bruteforce_properties(oracle_lib):
    """Against an exhaustive definition: the swaps are the longest prefix of the paired
    orderings that clears the bar, and no expert moves twice."""
    rng = np.random.default_rng(11)
    for trial in range(50):
        E = int(rng.integers(4, 40))
        counts = rng.integers(0, 6, size=E).astype(np.float32) * np.float32(0.75)
        resident = (rng.random(E) < 0.5).astype(np.uint8)
        gain = np.float32(rng.choice([1.0, 1.5, 2.0]))
        ms = int(rng.integers(1, 10))
        res, sw = oracle_lib.tier_select(counts, resident, max_swaps=ms, min_gain=gain)
        ins = sorted([e for e in range(E) if not resident[e]], key=lambda e: (-counts[e], e))
        outs = sorted([e for e in range(E) if resident[e]], key=lambda e: (counts[e], e))
        for i, (a, b) in enumerate(sw):
            assert a == ins[i] and b == outs[i]
            assert counts[a] > 0 and counts[a] >= np.float32(gain * counts[b])
        n = len(sw)
        if n < min(ms, len(ins), len(outs)):   # the next pair fails the bar
            a, b = ins[n], outs[n]
            assert not (counts[a] > 0 and counts[a] >= np.float32(gain * counts[b]))
        assert res.sum() == resident.sum()
        assert len(set(sw.ravel())) == 2 * n

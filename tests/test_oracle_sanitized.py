"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/oracle_sanitize_main.c links oracle/oracle.c with both sanitizers (any finding ends
the run with an error) and runs the whole oracle once on the small float window: routing,
grouping, the layer with residual and x_next, the head, the accept step and a tier round.
Its results must equal those of the normal build (loaded through ctypes) bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    d = tmp_path_factory.mktemp("oracle_sanitize")
    exe = str(d / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_main.c"),
           "-o", exe, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.skip("the sanitizers are not available to gcc here: " + res.stderr[-400:])
    return d, exe


def test_oracle_clean_under_sanitizers_and_equal_to_normal_build(sanitized, oracle_lib):
    d, exe = sanitized
    oracle = oracle_lib
    cfg = synth.config("small_f32", vocab=1040)
    R, H, F, E, K, V = cfg.rows, cfg.hidden, cfg.ffn, cfg.experts, cfg.top_k, cfg.vocab
    L = synth.make_layer(cfg)
    x = synth.make_window(cfg, 0)
    hc, hm = synth.make_head(cfg)
    rng = np.random.default_rng(11)
    S = R // 2
    am_in = rng.integers(0, V, size=R, dtype=np.int32)
    prop = am_in[0::2].copy()
    row_mask = rng.integers(0, 1 << R, size=E + 1, dtype=np.uint8)
    counts = rng.uniform(0, 8, size=E).astype(np.float32)
    resident = (np.arange(E) % 3 == 0).astype(np.uint8)
    with open(d / "in.bin", "wb") as f:
        for a in (x, L.gate_w, *L.gate, *L.up, *L.down, *L.sh_gate, *L.sh_up, *L.sh_down, hc, hm, am_in, prop,
                  row_mask, counts, resident):
            np.ascontiguousarray(a).tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe, str(d), str(R), str(H), str(F), str(E), str(K), str(V)], capture_output=True,
                         text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]

    # the normal build on the same inputs
    q = lambda m, n, r, c, b=4: oracle.qmat(m[0], m[1], r, c, b, n)
    mats = (q(L.gate, E, F, H), q(L.up, E, F, H), q(L.down, E, H, F), q(L.sh_gate, 1, F, H), q(L.sh_up, 1, F, H),
            q(L.sh_down, 1, H, F))
    logits, probs, idx, w = oracle.route(x, L.gate_w, None, K)
    grp = oracle.group(idx, w, E)
    out, xn = oracle.moe(x, *mats, idx, w, residual=x, want_x_next=True)
    hq = oracle.qmat(hc[0], hm[0], V, H, 8)
    hl, am = oracle.head(x, hq)
    tokens, ntok, kept = oracle.accept(am_in, prop, mtp=True)
    c2 = oracle.tier_count(row_mask, counts, 0.875)
    res2, swaps = oracle.tier_select(c2, resident, E // 4, 1.5)

    buf = open(d / "out.bin", "rb").read()
    pos = 0

    def nxt(dtype, n):
        nonlocal pos
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a
    A, NE = min(E, R * K) + 1, R * K + R
    assert np.array_equal(nxt(np.float64, R * E), logits.ravel())
    assert np.array_equal(nxt(np.float64, R * E), probs.ravel())
    assert np.array_equal(nxt(np.int32, R * K), idx.ravel())
    assert np.array_equal(nxt(np.float64, R * K), w.ravel())
    n = int(nxt(np.int32, 1)[0])
    assert n == grp["n_active"]
    assert np.array_equal(nxt(np.int32, A)[:n], grp["active"])
    assert np.array_equal(nxt(np.int32, A + 1)[:n + 1], grp["offsets"])
    ne = int(grp["offsets"][-1])
    assert np.array_equal(nxt(np.int32, NE)[:ne], grp["entry_row"])
    assert np.array_equal(nxt(np.float64, NE)[:ne], grp["entry_w"])
    assert np.array_equal(nxt(np.float64, R * H), out.ravel())
    assert np.array_equal(nxt(np.uint16, R * H), xn.ravel())
    assert np.array_equal(nxt(np.float64, R * V), hl.ravel())
    assert np.array_equal(nxt(np.int32, R), am)
    assert np.array_equal(nxt(np.int32, 2 * S), tokens.ravel())
    assert np.array_equal(nxt(np.int32, S), ntok)
    assert int(nxt(np.int32, 1)[0]) == kept
    assert np.array_equal(nxt(np.float32, E), c2)
    assert np.array_equal(nxt(np.uint8, E), res2)
    ns = len(swaps)
    assert np.array_equal(nxt(np.int32, 2 * ns), swaps.ravel())
    assert int(nxt(np.int32, 1)[0]) == ns
    assert pos == len(buf)

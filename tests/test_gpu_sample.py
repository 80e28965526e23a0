"""GPU parity of the sampled draw (strata_window_sample) and of the sampled verify
(strata_window_sample, then strata_window_accept) against the oracle, through the C ABI.

Tokens are integers decided in double on both sides (Strata docs/BATCHING.md,
"Exactness": sampled rows are drawn row by row with Philox(seed, position)); exp and the
summation order may differ in the last bits, so every case checks that the oracle's
decisions lie more than 1e-9 (relative) from their boundaries, and then the tokens must be
equal."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import oracle  # noqa: E402
import verify_window_expert_amd as sw  # noqa: E402
from gpu_helpers import to_dev_x  # noqa: E402

MARGIN = 1e-9


def gpu_sample(logits, params, positions):
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    tok = sw.strata_window_sample(lg, sw.sample_params(params), torch.tensor(positions, dtype=torch.int64).cuda())
    torch.cuda.synchronize()
    return tok.cpu().numpy()


def oracle_sample(logits, params, positions):
    """The oracle's draws with the parameters as the kernel reads them (float32)."""
    f32 = lambda v: float(np.float32(v))
    out, margins = [], []
    for r, (T, k, tp, mp, seed) in enumerate(params):
        t, m = oracle.sample(logits[r], f32(T), k, f32(tp), f32(mp), seed=seed, position=positions[r])
        out.append(t)
        margins.append(m)
    return np.array(out, np.int32), np.array(margins)


def check(logits, params, positions, label):
    print(f"[sample] {label}: rows {len(params)}, vocab {logits.shape[1]}", flush=True)
    g = gpu_sample(logits, params, positions)
    o, m = oracle_sample(logits, params, positions)
    assert (m > MARGIN).all(), ("a decision of this seed lies on its boundary", m)
    assert np.array_equal(g, o), (g, o)
    return g


PARAMS = [(0.0, 40, 0.95, 0.05, 1), (1.0, 40, 0.95, 0.05, 2), (0.7, 128, 1.0, 0.0, 3), (1.5, 5, 1.0, 0.0, 4),
          (1.0, 1, 1.0, 0.0, 5), (0.8, 64, 0.5, 0.0, 6), (2.0, 100, 0.9, 0.1, 7), (1.0, 128, 0.99, 0.01, 2**40 + 3)]


def test_sample_full_vocab_random_logits():
    rng = np.random.default_rng(21)
    V = 151936
    for rep in range(3):
        logits = (rng.standard_normal((8, V)) * 3).astype(np.float32)
        check(logits, PARAMS, [1000 * rep + r for r in range(8)], f"random logits, pass {rep}")


def test_sample_many_positions_small_vocab():
    rng = np.random.default_rng(22)
    logits = np.repeat((rng.standard_normal((1, 96)) * 2).astype(np.float32), 8, axis=0)
    draws = []
    for call in range(32):
        pos = [8 * call + r for r in range(8)]
        draws.append(check(logits, [(1.0, 96, 1.0, 0.0, 99)] * 8, pos, f"positions {pos[0]}.."))
    assert len(set(np.concatenate(draws).tolist())) > 10   # the draws vary with the position


def test_sample_ties():
    # an all-equal row: the candidates are the lowest indices
    z = np.zeros((4, 1000), np.float32)
    g = check(z, [(1.0, 5, 1.0, 0.0, 7), (0.0, 5, 1.0, 0.0, 7), (1.0, 128, 1.0, 0.0, 8), (1.0, 1, 1.0, 0.0, 9)],
              [3, 4, 5, 6], "all-equal rows")
    assert g[0] < 5 and g[1] == 0 and g[2] < 128 and g[3] == 0
    # many equal maxima around the top_k boundary, and equal values straddling it
    rng = np.random.default_rng(23)
    l = rng.standard_normal((4, 5000)).astype(np.float32)
    l[0, rng.choice(5000, 300, replace=False)] = 9.0
    l[1, rng.choice(5000, 30, replace=False)] = 9.0
    l[1, rng.choice(5000, 30, replace=False)] = 8.0
    l[2, :] = np.round(l[2, :] * 4) / 4          # coarse values: many exact ties everywhere
    l[3, ::2] = 1.0
    check(l, [(1.0, 40, 1.0, 0.0, 11), (1.0, 45, 1.0, 0.0, 12), (0.5, 100, 0.9, 0.0, 13), (1.0, 17, 1.0, 0.0, 14)],
          [10, 11, 12, 13], "tied logits")


def test_sample_special_values_and_sizes():
    """Signed zeros (equal, so the lower index first), -inf logits, a vocabulary smaller
    than top_k, one entry, ragged chunk tails, and a vocabulary long enough that each
    reducing wave takes a second round of chunks (more than 8 x 7 chunks of 4096)."""
    rng = np.random.default_rng(25)
    l = -np.abs(rng.standard_normal((4, 9000))).astype(np.float32)
    l[0, 100], l[0, 200] = -0.0, 0.0          # the largest two, equal
    l[1, 7], l[1, 8000] = 0.0, -0.0
    l[2, :] = -np.inf
    l[2, rng.choice(9000, 50, replace=False)] = rng.standard_normal(50).astype(np.float32)
    l[3, 4095:4098] = 5.0                      # equal maxima across a chunk boundary
    g = check(l, [(0.0, 1, 1.0, 0.0, 1), (0.0, 1, 1.0, 0.0, 2), (1.0, 40, 1.0, 0.0, 3), (0.5, 2, 1.0, 0.0, 4)],
              [1, 2, 3, 4], "signed zeros, -inf, chunk boundary")
    assert g[0] == 100 and g[1] == 7 and g[3] in (4095, 4096)
    for V, params in ((5, [(1.0, 40, 1.0, 0.0, 5), (0.7, 128, 0.9, 0.0, 6)]), (1, [(1.0, 40, 0.5, 0.2, 7)]),
                      (4097, [(1.3, 128, 0.99, 0.0, 8), (0.9, 3, 1.0, 0.0, 9)])):
        lg = (rng.standard_normal((len(params), V)) * 2).astype(np.float32)
        check(lg, params, list(range(10, 10 + len(params))), f"vocab {V}")
    lg = (rng.standard_normal((2, 300000)) * 3).astype(np.float32)
    check(lg, [(1.0, 128, 0.95, 0.01, 10), (0.6, 64, 1.0, 0.05, 11)], [20, 21], "vocab 300000")


def test_sample_window_equals_alone():
    rng = np.random.default_rng(24)
    logits = (rng.standard_normal((8, 20000)) * 2).astype(np.float32)
    pos = list(range(500, 508))
    g = gpu_sample(logits, PARAMS, pos)
    for r in range(8):
        assert gpu_sample(logits[r:r + 1], PARAMS[r:r + 1], pos[r:r + 1])[0] == g[r]


def test_greedy_equals_head_argmax_and_sampled_verify():
    """The head's logits of a window (vocab 151936): temperature 0 gives the head's argmax;
    then a sampled verify of four MTP slots (rows 2s, 2s + 1 at positions p_s, p_s + 1) on
    the GPU against the oracle's draws from the same logits and the oracle's accept."""
    cfg = synth.config("stack24_head")
    codes, meta = synth.make_head(cfg)
    hq = sw.upload_qmat(codes, meta, cfg.vocab, cfg.hidden, 8)
    x = to_dev_x(synth.make_window(cfg, 5))
    lg, am = sw.strata_window_head(x, hq)
    torch.cuda.synchronize()
    L = lg.cpu().numpy()
    greedy = gpu_sample(L, [(0.0, 40, 0.9, 0.05, s) for s in range(8)], list(range(8)))
    assert np.array_equal(greedy, am.cpu().numpy())
    params = [(0.9, 64, 0.95, 0.02, 1000 + r // 2) for r in range(8)]
    pos = [p for s in range(4) for p in (200 + 17 * s, 201 + 17 * s)]
    draws = check(L, params, pos, "head logits")
    o_draws, _ = oracle_sample(L, params, pos)
    proposal = draws[0::2].copy()
    proposal[[1, 3]] += 1                     # two slots' proposals miss their draw
    tok, ntok, nacc = sw.strata_window_accept(torch.from_numpy(draws).cuda(),
                                              torch.from_numpy(proposal.astype(np.int32)).cuda(), mtp=True)
    torch.cuda.synchronize()
    ot, on, ok = oracle.accept(o_draws, proposal, mtp=True)
    assert np.array_equal(tok.cpu().numpy(), ot) and np.array_equal(ntok.cpu().numpy(), on)
    assert int(nacc[0].item()) == ok == 2

"""GPU parity of the greedy verify/accept step (one MTP proposal per slot), through the C
ABI, against the CPU oracle: bit-exact tokens, token counts and kept-proposal counts."""
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


def check(argmax, proposal, mtp):
    am_d = torch.from_numpy(argmax).cuda()
    pr_d = torch.from_numpy(proposal).cuda() if mtp else None
    tok, ntok, nacc = sw.strata_window_accept(am_d, pr_d, mtp=mtp)
    torch.cuda.synchronize()
    ot, on, ok = oracle.accept(argmax, proposal if mtp else None, mtp=mtp)
    np.testing.assert_array_equal(tok.cpu().numpy(), ot)
    np.testing.assert_array_equal(ntok.cpu().numpy(), on)
    assert int(nacc[0].item()) == ok
    return ok


@pytest.mark.parametrize("mtp,n_slots", [(1, 1), (1, 2), (1, 3), (1, 4), (0, 1), (0, 5), (0, 8)])
def test_accept_matches_oracle(mtp, n_slots):
    rng = np.random.default_rng(100 + 10 * mtp + n_slots)
    V = 151936
    for trial in range(20):
        rows = n_slots * (2 if mtp else 1)
        argmax = rng.integers(0, V, size=rows).astype(np.int32)
        proposal = np.zeros(n_slots, np.int32)
        if mtp:
            keep = rng.random(n_slots) < 2 / 3
            proposal = np.where(keep, argmax[0::2], (argmax[0::2] + 1) % V).astype(np.int32)
        print(f"[accept] mtp={mtp} slots={n_slots} trial={trial}", flush=True)
        check(argmax, proposal, mtp)


def test_accept_after_gpu_head():
    """The head's argmax on the GPU feeds the accept step: slots 0 and 2 propose the token
    row's argmax (kept, with the proposal row's argmax as bonus), slots 1 and 3 a wrong
    token (one token each)."""
    cfg = synth.config("stack24_head", vocab=4096)
    x = synth.make_window(cfg, 3)
    codes, meta = synth.make_head(cfg)
    hq = sw.upload_qmat(codes, meta, cfg.vocab, cfg.hidden, 8)
    print(f"[accept] head V={cfg.vocab} then accept, 4 slots", flush=True)
    _, am = sw.strata_window_head(to_dev_x(x), hq)
    torch.cuda.synchronize()
    amh = am.cpu().numpy()
    prop = np.array([amh[0], (amh[2] + 7) % cfg.vocab, amh[4], (amh[6] + 1) % cfg.vocab], np.int32)
    assert check(amh, prop, 1) == 2
    tok, ntok, nacc = sw.strata_window_accept(am, torch.from_numpy(prop).cuda())
    torch.cuda.synchronize()
    t = tok.cpu().numpy()
    assert list(ntok.cpu().numpy()) == [2, 1, 2, 1]
    assert t[0, 1] == amh[1] and t[2, 1] == amh[5] and t[1, 0] == amh[2] and t[3, 0] == amh[6]

"""(eps, delta) at the full sizes of the long-context workloads, on the GPU
against the oracle's dense fp64 attention.

The contract (edgentiq blog post "vAttention: a new approach to sparse
attention with guaranteed accuracy", section "Introducing vAttention"): the
user's (eps, delta) bounds the probability that the denominator estimate is
off by more than eps, relative, at delta.  Over 1000 seeds of every head the
empirical rate of |D_hat / D - 1| > eps (D_hat / D = exp(lse - lse_dense)) must
not exceed delta; the two-sided 95% Clopper-Pearson interval is printed.
"""
import numpy as np
import pytest

import oracle
import synthetic

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

SEEDS = 1000

FULL = {
    "llama8b_32k": lambda: synthetic.llama8b_32k(),
    "flat_128k": lambda: synthetic.flat_128k(),
    "ragged_b64": lambda: synthetic.ragged_b64(),
    "wide_gqa_64k": lambda: synthetic.wide_gqa_64k(),
}


def _interval(k, n):
    from scipy.stats import beta
    lo = 0.0 if k == 0 else float(beta.ppf(0.025, k, n - k + 1))
    hi = 1.0 if k == n else float(beta.ppf(0.975, k + 1, n - k))
    return lo, hi


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_eps_delta_rate(name):
    import torch
    from tests.gpu_run import GpuCase, log
    w = FULL[name]()
    log("[rate] %s full size: B=%d Hq=%d L<=%d, base %d ppm, %d seeds"
        % (name, w.B, w.Hq, w.max_seq_len, w.cfg["base_ppm"], SEEDS))
    dense = oracle.dense(**w.oracle_arrays(), nthreads=8, want_out=False)["lse_dense"]
    case = GpuCase(w, want_idx=False)
    eps_list = (0.01, 0.02, 0.05, 0.1) if name == "wide_gqa_64k" else (w.cfg["eps"],)
    for eps in eps_list:
        case.dec.cfg.eps = eps
        case.dec._ccfg.eps = eps
        lse = torch.empty((SEEDS,) + tuple(case.dec.lse.shape), dtype=torch.float32, device=case.dec.lse.device)
        for s in range(SEEDS):
            case.dec.set_seed(s)
            case.dec()
            lse[s].copy_(case.dec.lse)
        torch.cuda.synchronize()
        rel = np.abs(np.exp(lse.cpu().numpy().astype(np.float64) - dense[None]) - 1.0)
        viol, trials = int((rel > eps).sum()), rel.size
        lo, hi = _interval(viol, trials)
        log("[rate] %s eps=%g: %d / %d = %.4f (95%% CI %.4f-%.4f), delta %g"
            % (name, eps, viol, trials, viol / trials, lo, hi, w.cfg["delta"]))
        assert viol / trials <= w.cfg["delta"], (name, eps, viol, trials)

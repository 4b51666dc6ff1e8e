"""Statistical pins of the GPU estimator itself, over Philox offsets.

Per-call parity (test_gpu_parity) shows each GPU call equals the oracle's
estimate for the same draws. These tests check the estimator's defining
properties on the GPU's own outputs across many independent draw sets
(offsets 0 .. R-1; the counter includes the offset, so each call draws
afresh, as at every decode step):

  - the Horvitz-Thompson denominator and numerator are unbiased: the mean of
    D_hat / D = exp(lse - lse_dense) is 1 and the mean of
    N_hat / D = out * exp(lse - lse_dense) is the dense output, each within
    five standard errors ("SANTA++", abstract: with the 1/pi weights the
    drawn teams give an unbiased stand-in for the whole cache's sums);
  - the mean size of a head's drawn set is sum_t pi_t and the mean union of a
    KV head's sets is sum_t (1 - prod_h (1 - p_ht)^M), the closed forms of
    draws with replacement.

Dense targets and team probabilities come from the float64 oracle. The
offsets are fixed, so the outcome is deterministic.
"""
import numpy as np
import pytest
import torch

from oracle import numerics, santa as osanta
from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu

R = 3000            # decode calls (offsets) per case
Z_MAX = 5.0         # standard errors


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()


CASES = {
    # the tiny single-head float32 configuration (32 teams, M = 8)
    "tiny_f32": lambda: W.tiny_planted(),
    # bfloat16, grouped query heads, a ragged last team, two sequences
    "bf16_gqa_ragged": lambda: W.qwen_planted(batch=2, seq_len=4000 + 37, T=64, M=12, hq=8, hkv=2, d=128,
                                              plants=3),
}


def _zscore(samples, target):
    """|mean - target| in standard errors of the mean (per element)."""
    mean = samples.mean(axis=0)
    se = samples.std(axis=0, ddof=1) / np.sqrt(samples.shape[0])
    return np.abs(mean - target) / np.maximum(se, 1e-300)


@pytest.mark.parametrize("name", list(CASES))
def test_gpu_estimator_unbiased_and_set_sizes(name):
    w = CASES[name]()
    B, Hq, d, G = w.batch, w.num_q_heads, w.head_dim, w.group
    print(f"[estimator] {name} B={B} Hq={Hq} d={d} T={w.page_size} M={w.M} calls={R}", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    ws = S.make_workspace(kv, w.M)
    out = torch.empty((R, B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((R, B, Hq), dtype=torch.float32, device="cuda")
    sampled = torch.empty((R, B, Hq, w.M), dtype=torch.int32, device="cuda")
    inv_pi = torch.empty((R, B, Hq, w.M), dtype=torch.float32, device="cuda")
    for i in range(R):
        S.santa_select_teams(kv, q, reps, w.M, w.seed, i, ws, sampled[i], inv_pi[i])
        S.santa_attend_selected(kv, q, w.M, ws, out[i], lse[i])
    torch.cuda.synchronize()
    out, lse, sampled = out.cpu().numpy(), lse.cpu().numpy(), sampled.cpu().numpy()

    okv = parity.oracle_kv(w)
    oreps = osanta.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    for b in range(B):
        K = osanta.num_teams(int(w.seq_lens[b]), w.page_size)
        assert K > w.M, "the case must sample (M < K), not cover every team"
        p_heads = []
        for h in range(Hq):
            g = h // G
            qh = numerics.decode(w.q[b, h], w.dtype)
            dout, dlse = osanta.dense_head(okv, qh, b, h, Hq)
            ratio = np.exp(lse[:, b, h].astype(np.float64) - dlse)            # D_hat / D per call
            z_den = _zscore(ratio[:, None], np.array([1.0]))
            z_num = _zscore(out[:, b, h].astype(np.float64) * ratio[:, None], dout)
            assert z_den.max() < Z_MAX, f"b={b} h={h}: denominator mean off by {z_den.max():.2f} s.e."
            assert z_num.max() < Z_MAX, f"b={b} h={h}: numerator mean off by {z_num.max():.2f} s.e."

            rows = np.stack([oreps[b, t, g] for t in range(K)])
            p = osanta.select_teams(qh, rows, w.M, w.seed, 0, b, h).p
            p_heads.append(p)
            sizes = (sampled[:, b, h] >= 0).sum(axis=1).astype(np.float64)
            z_set = _zscore(sizes[:, None], np.array([osanta.expected_set_size(p, w.M)]))
            assert z_set.max() < Z_MAX, f"b={b} h={h}: mean set size off by {z_set.max():.2f} s.e."
        for g in range(w.num_kv_heads):
            heads = range(g * G, (g + 1) * G)
            unions = np.array([len(set(sampled[i, b, list(heads)].ravel()) - {-1}) for i in range(R)], np.float64)
            expect = osanta.expected_union_size([p_heads[h] for h in heads], w.M)
            z_u = _zscore(unions[:, None], np.array([expect]))
            assert z_u.max() < Z_MAX, f"b={b} g={g}: mean union size off by {z_u.max():.2f} s.e."

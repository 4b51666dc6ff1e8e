"""Systematic and stratified team draws (santa_decode_attention_ex): the HIP
sets, weights 1/pi, outputs and lse match the oracle head by head, the
independent scheme through the _ex entry equals the plain call bit for bit,
and select + attend equals one decode call."""
import numpy as np
import pytest
import torch

from oracle import numerics
from oracle import santa as O
from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()


CASES = {
    "tiny_f32": lambda: W.tiny_planted(),
    "qwen_bf16_ragged": lambda: W.qwen_planted(batch=1, seq_len=4096 + 77, M=31),
    "qwen_mixq_b2": lambda: W.qwen_mixed_query(batch=2, seq_len=8192, M=32),
    "mixture_t256": lambda: W.gaussian_mixture(batch=2, seq_len=8192 + 100, T=256, M=16),
    "paged_ragged": lambda: W.paged_ragged(num_seqs=4, len_min=300, len_max=9000, M=20),
    "f32_d128_t64_g2": lambda: W.qwen_planted(batch=2, seq_len=3000, T=64, M=9, hq=4, hkv=2, d=128,
                                              plants=3, dtype="f32"),
    "bf16_b3_g16_p2048": lambda: W.qwen_planted(batch=3, seq_len=32768, T=16, M=24, hq=48, hkv=3, d=64,
                                                plants=2),
    # M >= K for the short sequences: full coverage under every scheme
    "bf16_full_cover": lambda: W.paged_ragged(num_seqs=3, len_min=100, len_max=700, T=32, M=12, hq=4, hkv=2,
                                              d=64),
}
SCHEMES = {"systematic": O.DRAW_SYSTEMATIC, "stratified": O.DRAW_STRATIFIED}


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", list(CASES))
def test_scheme_parity(name, scheme):
    w = CASES[name]()
    print(f"[scheme] {scheme} {name} B={w.batch} Hq={w.num_q_heads} T={w.page_size} M={w.M} {w.dtype}",
          flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention_ex(kv, q, reps, w.M, scheme, seed=w.seed, offset=w.offset,
                                                          return_sets=True)
    torch.cuda.synchronize()
    out, lse, teams, inv_pi = (x.cpu().numpy() for x in (out, lse, teams, inv_pi))
    okv = parity.oracle_kv(w)
    ref_reps = parity.oracle_reps(w)
    flips = 0
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            _, flip = parity.check_santa_head(w, okv, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h],
                                              inv_pi[b, h], scheme=SCHEMES[scheme])
            flips += flip
    assert flips <= max(1, w.batch * w.num_q_heads // 50)


def test_iid_ex_equals_plain_and_select_attend_equals_decode():
    w = CASES["qwen_mixq_b2"]()
    print("[scheme] iid through _ex; select_ex + attend", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    a = S.santa_decode_attention(kv, q, reps, w.M, seed=3, offset=4, return_sets=True)
    b = S.santa_decode_attention_ex(kv, q, reps, w.M, "iid", seed=3, offset=4, return_sets=True)
    ws = S.make_workspace(kv, w.M)
    c = S.santa_decode_attention_ex(kv, q, reps, w.M, "stratified", seed=3, offset=4, workspace=ws,
                                    return_sets=True)
    sampled = torch.empty_like(c[2])
    inv_pi = torch.empty_like(c[3])
    S.santa_select_teams_ex(kv, q, reps, w.M, "stratified", 3, 4, ws, sampled, inv_pi)
    out = torch.empty_like(c[0])
    lse = torch.empty_like(c[1])
    S.santa_attend_selected(kv, q, w.M, ws, out, lse)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip(c, (out, lse, sampled, inv_pi)):
        assert torch.equal(x, y)


def test_systematic_draws_m_distinct_teams_on_flat_scores():
    # Identical representatives: p = 1/K < 1/M for every team, so the M
    # systematic points are one unit apart and land in M distinct teams.
    T, d, K, M = 16, 64, 200, 24
    keys = np.zeros((1, 2, K * T, d), np.float32)
    vals = np.random.default_rng(3).standard_normal((1, 2, K * T, d)).astype(np.float32)
    q = np.random.default_rng(4).standard_normal((1, 8, d)).astype(np.float32)
    w = W._contiguous("flat", "bf16", keys, vals, q, T, M)
    print("[scheme] systematic on flat scores", flush=True)
    kv, qd = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention_ex(kv, qd, reps, M, "systematic", seed=9,
                                                          return_sets=True)
    torch.cuda.synchronize()
    teams = teams.cpu().numpy()
    assert np.all(teams >= 0)                                   # M distinct teams in every head
    assert np.allclose(inv_pi.cpu().numpy(), K / M, rtol=1e-6)


FULL = {
    "qwen7b_32k_b1_m31": [(0, 0), (0, 13), (0, 27)],
    "qwen7b_32k_b8_m32": [(0, 1), (7, 27)],
    "mixture_128k_b4_t256_m64": [(2, 11)],
}


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", list(FULL))
def test_scheme_full_size_sampled_heads(name, scheme):
    # Full-size configurations in the launch configuration the benchmark
    # times; the oracle evaluates a sample of heads one by one.
    w = W.FULL_SIZE[name]()
    pairs = FULL[name]
    print(f"[scheme full] {scheme} {name} B={w.batch} P={w.num_pages} heads={pairs}", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention_ex(kv, q, reps, w.M, scheme, seed=w.seed, offset=w.offset,
                                                          return_sets=True)
    torch.cuda.synchronize()
    out, lse, teams, inv_pi = (x.cpu().numpy() for x in (out, lse, teams, inv_pi))
    ref_reps = parity.check_reps(w, reps, pairs)
    okv = parity.oracle_kv(w)
    for b, h in pairs:
        parity.check_santa_head(w, okv, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h],
                                scheme=SCHEMES[scheme])
        if scheme == "systematic":       # every team with M p >= 1 holds a point
            K = O.num_teams(int(w.seq_lens[b]), w.page_size)
            g = h // w.group
            qh = numerics.decode(w.q[b, h], w.dtype)
            sel = O.select_teams(qh, np.stack([ref_reps[b, t, g] for t in range(K)]), w.M, w.seed, w.offset, b, h,
                                 O.DRAW_SYSTEMATIC)
            sure = {t for t in range(K) if w.M * sel.p[t] >= 1.0 + 1e-3}    # clear of near-ties
            assert sure <= set(int(x) for x in teams[b, h] if x >= 0)
    # Every head: sets ascending, unique, in range, at most min(M, K) teams.
    for b in range(w.batch):
        K = O.num_teams(int(w.seq_lens[b]), w.page_size)
        for h in range(w.num_q_heads):
            t = teams[b, h][teams[b, h] >= 0]
            assert np.all(np.diff(t) > 0) and (len(t) == 0 or (t[0] >= 0 and t[-1] < K))
            assert len(t) <= min(K, w.M)
    assert np.all(np.isfinite(out))

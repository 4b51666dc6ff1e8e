"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints what it runs (workload, shape, entry point) before its
first GPU call. Small cases compare every head; the full-size workloads
compare a sample of heads that the oracle evaluates one by one, in the same
launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

from oracle import santa as osanta
from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()          # a missing library fails here, loudly


def say(*a):
    print(*a, flush=True)


def _with_lens(w, lens):
    """Workload w with its sequence lengths replaced (each at most its capacity)."""
    return W.dataclasses.replace(w, seq_lens=np.asarray(lens, dtype=w.seq_lens.dtype))


SMALL = {
    "tiny_f32": lambda: W.tiny_planted(),
    "qwen_bf16_ragged": lambda: W.qwen_planted(batch=1, seq_len=4096 + 77, M=31),
    "qwen_mixq_b2": lambda: W.qwen_mixed_query(batch=2, seq_len=8192, M=32),
    "mixture_t256": lambda: W.gaussian_mixture(batch=2, seq_len=8192 + 100, T=256, M=16),
    "paged_ragged": lambda: W.paged_ragged(num_seqs=4, len_min=300, len_max=9000, M=20),
    "bf16_d64_t16_g16": lambda: W.qwen_planted(batch=2, seq_len=1000, T=16, M=12, hq=16, hkv=1, d=64,
                                               plants=2),
    "f32_d128_t64_g2": lambda: W.qwen_planted(batch=2, seq_len=3000, T=64, M=9, hq=4, hkv=2, d=128,
                                              plants=3, dtype="f32"),
    "f32_d64_t256_g8": lambda: W.gaussian_mixture(batch=1, seq_len=5000, T=256, M=6, hq=8, hkv=1, d=64,
                                                  run_min=32, run_max=600, dtype="f32"),
    # many (sequence, KV head) groups: multi-team split blocks in union-rank order
    "bf16_b16_t16_union_rank": lambda: W.qwen_planted(batch=16, seq_len=4800, T=16, M=64, hq=8, hkv=2,
                                                      d=64, plants=4),
    "bf16_ragged12_t16_union_rank": lambda: W.paged_ragged(num_seqs=12, len_min=300, len_max=9000, T=16,
                                                           M=40, hq=8, hkv=2, d=64),
    "f32_b16_t16_union_rank": lambda: W.qwen_planted(batch=16, seq_len=4500, T=16, M=50, hq=8, hkv=2, d=64,
                                                     plants=4, dtype="f32"),
    # the longest page table (2048 teams of 16 tokens), 16-head groups
    "bf16_b3_g16_p2048": lambda: W.qwen_planted(batch=3, seq_len=32768, T=16, M=24, hq=48, hkv=3,
                                                            d=64, plants=2),
    # ragged batches: dense decode then splits all groups' chunks evenly over
    # the grid — a dominant group whose slot count exceeds the combine's
    # first read, empty groups, and 256 small groups whose blocks each span
    # several groups
    "bf16_b2_hkv1_skewed": lambda: _with_lens(W.qwen_planted(batch=2, seq_len=12000, T=32, M=20, hq=4, hkv=1,
                                                             d=64, plants=3), [150, 12000]),
    "bf16_b4_empty_groups": lambda: _with_lens(W.qwen_mixed_query(batch=4, seq_len=9000, T=64, M=24, hq=8,
                                                                  hkv=2, d=128), [0, 3000, 50, 9000]),
    "bf16_b64_256_groups": lambda: W.paged_ragged(num_seqs=64, len_min=1, len_max=400, T=16, M=6, hq=8, hkv=4,
                                                  d=64),
    # a full 16-head group over 300 small teams
    "bf16_g16_p300": lambda: W.qwen_planted(batch=1, seq_len=4800, T=16, M=40, hq=16, hkv=1, d=64,
                                                        plants=3),
    # the largest call the per-head blocks take: 64 (sequence, query head)
    # pairs over 512-team page tables (one split per head), ragged lengths
    "bf16_perhead_64heads_p512": lambda: _with_lens(W.qwen_planted(batch=4, seq_len=8192, T=16, M=40, hq=16,
                                                                   hkv=2, d=64, plants=2), [8192, 8191, 17, 5000]),
    # per-head blocks under full coverage (M >= K: every team, pi = 1)
    "bf16_perhead_full_coverage": lambda: W.qwen_planted(batch=2, seq_len=300, T=64, M=8, hq=8, hkv=2, d=128,
                                                         plants=1),
}


def run_santa(w, kv, q, reps, M=None, seed=None, offset=None):
    out, lse, teams, inv_pi = S.santa_decode_attention(
        kv, q, reps, w.M if M is None else M, w.seed if seed is None else seed,
        w.offset if offset is None else offset, return_sets=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), teams.cpu().numpy(), inv_pi.cpu().numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_build_reps_bit_exact(name):
    w = SMALL[name]()
    say(f"[build_reps] {name} B={w.batch} P={w.num_pages} T={w.page_size} d={w.head_dim} {w.dtype}")
    kv, _ = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    torch.cuda.synchronize()
    parity.check_reps(w, reps)


@pytest.mark.parametrize("name", list(SMALL))
def test_dense_parity(name):
    w = SMALL[name]()
    say(f"[dense] {name} B={w.batch} Hq={w.num_q_heads} L={list(w.seq_lens)} {w.dtype}")
    kv, q = S.kv_from_workload(w)
    out, lse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    okv = parity.oracle_kv(w)
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            parity.check_dense_head(w, okv, b, h, out[b, h], lse[b, h])


@pytest.mark.parametrize("name", list(SMALL))
def test_given_teams_parity(name):
    """The estimator (gather + combine) alone, on the oracle's own team sets."""
    w = SMALL[name]()
    say(f"[given_teams] {name}")
    okv = parity.oracle_kv(w)
    reps = parity.oracle_reps(w)
    from oracle import numerics
    B, Hq, M = w.batch, w.num_q_heads, w.M
    teams = np.full((B, Hq, M), -1, dtype=np.int32)
    wts = np.zeros((B, Hq, M), dtype=np.float32)
    refs = {}
    for b in range(B):
        for h in range(Hq):
            qh = numerics.decode(w.q[b, h], w.dtype)
            r = osanta.santa_head(okv, qh, reps, b, h, Hq, M, w.seed, w.offset)
            n = len(r.selection.teams)
            teams[b, h, :n] = r.selection.teams
            wts[b, h, :n] = np.float32(r.selection.inv_pi)
            # the oracle re-evaluated with the float32 weights the kernel receives
            refs[(b, h)] = osanta.evaluate_given_set(okv, qh, b, h, Hq, r.selection.teams,
                                                     [float(x) for x in wts[b, h, :n]])
    kv, q = S.kv_from_workload(w)
    out, lse = S.santa_attention_given_teams(kv, q, torch.from_numpy(teams).cuda(), torch.from_numpy(wts).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for (b, h), (ro, rl) in refs.items():
        err = float(np.max(np.abs(out[b, h] - ro)))
        assert err <= parity.OUT_TOL[w.dtype], f"(b={b}, h={h}) max-abs {err}"
        parity._check_lse(w, lse[b, h], rl, b, h)


@pytest.mark.parametrize("name", list(SMALL))
def test_santa_parity(name):
    w = SMALL[name]()
    say(f"[santa] {name} B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} M={w.M} T={w.page_size} {w.dtype}")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = run_santa(w, kv, q, reps_gpu)
    reps = parity.check_reps(w, reps_gpu)
    okv = parity.oracle_kv(w)
    flips = 0
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            _, f = parity.check_santa_head(w, okv, reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h])
            flips += f
    say(f"  near-tie flips: {flips}")
    assert flips <= parity.MAX_FLIPS, f"{flips} near-tie flips in one workload"


@pytest.mark.parametrize("name", ["qwen_bf16_ragged", "mixture_t256", "bf16_g16_p300",
                                  "f32_d128_t64_g2", "bf16_perhead_64heads_p512", "bf16_perhead_full_coverage",
                                  "qwen_mixq_b2", "bf16_b16_t16_union_rank"])
def test_decode_equals_select_then_attend(name):
    """santa_decode_attention and santa_select_teams + santa_attend_selected on
    one workspace give bit-identical results (sets, weights, outputs)."""
    w = SMALL[name]()
    say(f"[decode == select + attend] {name}")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    a = run_santa(w, kv, q, reps)
    ws = S.make_workspace(kv, w.M)
    B, Hq = w.batch, w.num_q_heads
    teams = torch.empty((B, Hq, w.M), dtype=torch.int32, device="cuda")
    inv_pi = torch.empty((B, Hq, w.M), dtype=torch.float32, device="cuda")
    S.santa_select_teams(kv, q, reps, w.M, w.seed, w.offset, ws, teams, inv_pi)
    out = torch.empty((B, Hq, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    S.santa_attend_selected(kv, q, w.M, ws, out, lse)
    torch.cuda.synchronize()
    for x, y in zip(a, (out.cpu().numpy(), lse.cpu().numpy(), teams.cpu().numpy(), inv_pi.cpu().numpy())):
        assert np.array_equal(x, y)


def test_santa_deterministic_and_seeded():
    w = SMALL["qwen_mixq_b2"]()
    say("[determinism] qwen_mixq_b2")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    a = run_santa(w, kv, q, reps)
    b = run_santa(w, kv, q, reps)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = run_santa(w, kv, q, reps, offset=1)
    assert not np.array_equal(a[2], c[2])
    d1, _ = S.dense_decode_attention(kv, q)
    d2, _ = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)


def test_paged_permutation_invariance():
    w = SMALL["paged_ragged"]()
    say("[permutation] paged_ragged")
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_pages)
    k2, v2 = np.empty_like(w.k_pages), np.empty_like(w.v_pages)
    k2[perm], v2[perm] = w.k_pages, w.v_pages
    kv1, q = S.kv_from_workload(w)
    w.k_pages, w.v_pages, w.page_table = k2, v2, perm[w.page_table].astype(np.int32)
    kv2, _ = S.kv_from_workload(w)
    a = run_santa(w, kv1, q, S.santa_build_reps(kv1))
    b = run_santa(w, kv2, q, S.santa_build_reps(kv2))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_edge_cases_empty_short_full_and_single_draw():
    w = W.paged_ragged(num_seqs=5, len_min=200, len_max=3000, M=4, hq=8, hkv=2, T=64)
    w.seq_lens[0] = 0          # empty sequence
    w.seq_lens[1] = 1          # one token
    w.seq_lens[2] = 64 * 3     # exactly K = 3 <= M: full coverage
    say(f"[edge] lens={list(w.seq_lens)} M in (1, 4)")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    reps = parity.check_reps(w, reps_gpu)
    okv = parity.oracle_kv(w)
    for M in (1, 4):
        out, lse, teams, inv_pi = run_santa(w, kv, q, reps_gpu, M=M)
        for b in range(w.batch):
            for h in range(w.num_q_heads):
                parity.check_santa_head(w, okv, reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h], M=M)
        assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
        assert np.all(teams[0] == -1)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    dout, dlse = dout.cpu().numpy(), dlse.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            parity.check_dense_head(w, okv, b, h, dout[b, h], dlse[b, h])


def test_all_sequences_empty():
    # Every group empty: the split has no chunk at all; outputs are zeros
    # with log-sum-exp -inf for both paths.
    w = _with_lens(W.paged_ragged(num_seqs=3, len_min=100, len_max=900, T=32, M=5, hq=4, hkv=2, d=64), [0, 0, 0])
    say("[edge] all sequences empty, B=3")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, _ = run_santa(w, kv, q, reps)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and np.all(teams == -1)
    assert torch.all(dout == 0) and torch.all(torch.isneginf(dlse))


def _groups(pairs_bg, group=7):
    """Every query head of the (sequence, KV head) groups listed."""
    return [(b, h) for b, g in pairs_bg for h in range(g * group, (g + 1) * group)]


# Heads compared with the oracle at full size: every head of the headline
# layer, and elsewhere one whole (sequence, KV head) group per KV head, each
# from a different sequence.
FULL = {
    "tiny_f32_n1024_m8": None,                                   # every head
    "qwen7b_32k_b1_m31": None,                                   # every head
    "qwen7b_32k_b8_m32": _groups([(0, 0), (3, 1), (5, 2), (7, 3)]),
    "qwen7b_32k_b8_m64": _groups([(1, 0), (2, 1), (4, 2), (6, 3)]),
    "mixture_128k_b4_t256_m64": _groups([(0, 0), (1, 1), (2, 2), (3, 3)]),
    "paged_ragged_16seq_m48": _groups([(0, 0), (5, 1), (11, 2), (15, 3)]),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_heads(name):
    w = W.FULL_SIZE[name]()
    pairs = FULL[name] or [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]
    say(f"[full] {name} B={w.batch} P={w.num_pages} T={w.page_size} M={w.M} heads={pairs}")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = run_santa(w, kv, q, reps_gpu)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    dout, dlse = dout.cpu().numpy(), dlse.cpu().numpy()
    reps = parity.check_reps(w, reps_gpu, pairs)
    okv = parity.oracle_kv(w)
    flips = 0
    for b, h in pairs:
        _, f = parity.check_santa_head(w, okv, reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h])
        flips += f
        parity.check_dense_head(w, okv, b, h, dout[b, h], dlse[b, h])
    say(f"  compared {len(pairs)} heads, near-tie flips: {flips}")
    assert flips <= parity.MAX_FLIPS, f"{flips} near-tie flips in one workload"
    # Structural checks on every head: sets ascending, unique, in range; finite outputs.
    for b in range(w.batch):
        K = osanta.num_teams(int(w.seq_lens[b]), w.page_size)
        for h in range(w.num_q_heads):
            t = teams[b, h][teams[b, h] >= 0]
            assert np.all(np.diff(t) > 0) and (len(t) == 0 or (t[0] >= 0 and t[-1] < K))
            assert len(t) == (K if w.M >= K else len(t)) and len(t) <= min(K, w.M)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(dout))

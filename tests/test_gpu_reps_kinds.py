"""Medoid and random-member representatives (santa_build_reps_ex): every row
equals the oracle's choice bit for bit, the update mode equals a rebuild, and
one SANTA++ decode on medoid representatives matches the oracle head by head."""
import numpy as np
import pytest
import torch

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


KINDS = {"medoid": O.REP_MEDOID, "random": O.REP_RANDOM}


def _check_kind(w, gpu_reps, kind, seed):
    ref = O.build_reps_kind(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype, KINDS[kind], seed)
    got = parity.decoded_reps(gpu_reps, w.dtype)
    for b in range(w.batch):
        K = O.num_teams(int(w.seq_lens[b]), w.page_size)
        bad = np.argwhere(np.any(got[b, :K] != ref[b, :K], axis=-1))
        assert bad.size == 0, f"{kind}: sequence {b}, (team, head) rows {bad[:5].tolist()} differ from the oracle"


@pytest.mark.parametrize("kind", ["medoid", "random"])
@pytest.mark.parametrize("dtype,T,d", [("bf16", 16, 128), ("f32", 32, 64), ("bf16", 64, 64),
                                       ("bf16", 128, 128), ("f32", 256, 128)])
def test_reps_kind_matches_oracle(kind, dtype, T, d):
    w = W.paged_ragged(num_seqs=3, len_min=T + 1, len_max=6 * T - 3, T=T, M=4, hq=4, hkv=2, d=d, dtype=dtype)
    print(f"[reps_kind] {kind} {dtype} T={T} d={d} lens={list(w.seq_lens)}", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = S.santa_build_reps_ex(kv, kind, seed=11)
    torch.cuda.synchronize()
    _check_kind(w, reps, kind, 11)


def test_medoid_ties_take_the_lowest_member():
    # Every key of a team repeated: all sums tie, member 0 is taken. Then
    # points x * (1, ..., 1) of a line with 16 members: every member with x
    # between the 8th and 9th smallest (1, 1, 4: members 3, 9, 6) has the
    # same, exactly computed, smallest sum; the lowest member wins.
    T, d = 16, 64
    rng = np.random.default_rng(8)
    keys = np.repeat(rng.standard_normal((1, 1, 1, d)), 2 * T, axis=2).astype(np.float32)   # [1][1][2T][d]
    x = np.array([5, -3, 7, 1, 9, -7, 4, 12, -2, 1, 30, -9, 6, 0, 8, -5], dtype=np.float32)
    keys[0, 0, T:] = x[:, None] * np.ones((1, d), np.float32)
    w = W._contiguous("medoid_ties", "f32", keys, keys, np.zeros((1, 1, d), np.float32), T, 2)
    print("[reps_kind] medoid ties", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = S.santa_build_reps_ex(kv, "medoid")
    torch.cuda.synchronize()
    got = reps.cpu().numpy()
    assert np.array_equal(got[0, 0, 0], keys[0, 0, 0])
    assert np.array_equal(got[0, 1, 0], keys[0, 0, T + 3])
    _check_kind(w, reps, "medoid", 0)


@pytest.mark.parametrize("kind", ["medoid", "random"])
def test_reps_kind_update_equals_rebuild(kind):
    T = 32
    w = W.paged_ragged(num_seqs=4, len_min=300, len_max=900, T=T, M=8, hq=4, hkv=2, d=64, dtype="bf16")
    new_lens = w.seq_lens.copy()
    appended = np.array([1, T, 2 * T + 5, 7])[: w.batch]
    old_lens = np.maximum(new_lens - appended, 0).astype(np.int32)
    print(f"[reps_kind] update {kind} old={list(old_lens)} new={list(new_lens)}", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = torch.full((kv.batch, kv.max_pages_per_seq, kv.num_kv_heads, kv.head_dim), -7.0,
                      dtype=kv.dtype, device=kv.device)
    kv.seq_lens.copy_(torch.from_numpy(old_lens))
    S.santa_build_reps_ex(kv, kind, reps=reps, seed=5)
    kv.seq_lens.copy_(torch.from_numpy(new_lens))
    S.santa_build_reps_ex(kv, kind, reps=reps, seed=5, prev_seq_lens=torch.from_numpy(old_lens).cuda(),
                          max_new_tokens=int(appended.max()))
    torch.cuda.synchronize()
    _check_kind(w, reps, kind, 5)
    got = reps.float().cpu().numpy()
    for b in range(w.batch):
        K = -(-int(new_lens[b]) // T)
        assert np.all(got[b, K:] == -7.0), f"sequence {b}: rows past its last team were written"


def test_mean_kind_is_build_reps():
    w = W.paged_ragged(num_seqs=3, len_min=100, len_max=700, T=32, M=8, hq=4, hkv=2, d=64, dtype="bf16")
    kv, _ = S.kv_from_workload(w)
    a = S.santa_build_reps(kv)
    b = S.santa_build_reps_ex(kv, "mean")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_santa_decode_on_medoid_reps_matches_oracle(dtype):
    w = W.qwen_planted(batch=2, seq_len=3000, T=64, M=8, hq=8, hkv=2, d=128, plants=2, dtype=dtype)
    print(f"[reps_kind] decode on medoid reps {dtype}", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps_ex(kv, "medoid")
    out, lse, sampled, inv_pi = S.santa_decode_attention(kv, q, reps, w.M, seed=w.seed, offset=w.offset,
                                                         return_sets=True)
    torch.cuda.synchronize()
    ref_reps = O.build_reps_kind(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype, O.REP_MEDOID)
    okv = parity.oracle_kv(w)
    out, lse, sampled, inv_pi = (x.cpu().numpy() for x in (out, lse, sampled, inv_pi))
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            parity.check_santa_head(w, okv, ref_reps, b, h, out[b, h], lse[b, h], sampled[b, h], inv_pi[b, h])


@pytest.mark.parametrize("kind", ["medoid", "random"])
def test_reps_kind_full_size_sampled_teams(kind):
    # The 128K configuration (T = 256, d = 128): every representative row is
    # a member of its team, and a sample of (sequence, team, KV head) rows
    # equals the oracle's choice.
    w = W.FULL_SIZE["mixture_128k_b4_t256_m64"]()
    print(f"[reps_kind full] {kind}", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = S.santa_build_reps_ex(kv, kind, seed=21)
    torch.cuda.synchronize()
    got = parity.decoded_reps(reps, w.dtype)
    rng = np.random.default_rng(4)
    T = w.page_size
    for _ in range(12):
        b = int(rng.integers(0, w.batch))
        K = O.num_teams(int(w.seq_lens[b]), T)
        t = int(rng.integers(0, K))
        g = int(rng.integers(0, w.num_kv_heads))
        n = O.team_size(int(w.seq_lens[b]), T, t)
        keys = O.decode(w.k_pages[int(w.page_table[b][t]), g, :n, :], w.dtype)
        i = O.team_medoid_index(keys) if kind == "medoid" else O.team_random_index(n, 21, b, t, g)
        assert np.array_equal(got[b, t, g], keys[i]), f"{kind}: (b={b}, t={t}, g={g}) differs from the oracle"

"""k-means-partitioned teams (santa_pack_pages_kmeans): cluster ids, the
stable sort and the packed pages are bit-exact against the oracle's Lloyd
iterations; SANTA++ on the k-means cache matches the oracle on the permuted
cache head by head, and dense attention is unchanged by the permutation."""
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


def _zero_len(w, b):
    lens = w.seq_lens.copy()
    lens[b] = 0
    return W.dataclasses.replace(w, seq_lens=lens)


# name -> (workload, clusters, iters)
CASES = {
    "bf16_d64_t32_b4_per_team": (lambda: W.paged_ragged(num_seqs=4, len_min=300, len_max=5000, T=32, M=12, hq=8,
                                                        hkv=2, d=64), 0, 5),
    "f32_d128_t16_c40": (lambda: W.qwen_planted(batch=2, seq_len=3000, T=16, M=20, hq=4, hkv=2, d=128, plants=4,
                                                dtype="f32"), 40, 4),
    "bf16_t256_mixture": (lambda: W.gaussian_mixture(batch=2, seq_len=5000, T=256, M=6, hq=4, hkv=2, d=64,
                                                     run_min=1, run_max=16), 0, 8),
    "bf16_clusters_over_len": (lambda: W.paged_ragged(num_seqs=5, len_min=3, len_max=200, T=16, M=4, hq=4, hkv=2,
                                                      d=64), 150, 3),
    "bf16_one_cluster": (lambda: W.qwen_planted(batch=1, seq_len=700, T=32, M=4, hq=4, hkv=2, d=64, plants=2), 1, 2),
    "bf16_1024_clusters": (lambda: W.qwen_planted(batch=1, seq_len=4096 + 5, T=16, M=8, hq=2, hkv=1, d=64,
                                                  plants=4), 1024, 2),
    "bf16_empty_seq": (lambda: _zero_len(W.paged_ragged(num_seqs=3, len_min=100, len_max=2000, T=32, M=8, hq=4,
                                                        hkv=2, d=64), 1), 7, 3),
}


def _used_pages(w):
    pages = []
    for b in range(w.batch):
        pages += [int(p) for p in w.page_table[b][:O.num_teams(int(w.seq_lens[b]), w.page_size)]]
    return torch.tensor(sorted(pages), dtype=torch.long)


def _oracle(w, clusters, iters):
    return O.cluster_pages_kmeans(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size, w.dtype,
                                  None if clusters == 0 else clusters, iters)


@pytest.mark.parametrize("name", list(CASES))
def test_kmeans_pack_matches_oracle(name):
    make, clusters, iters = CASES[name]
    w = make()
    print(f"[kmeans] {name} B={w.batch} T={w.page_size} d={w.head_dim} clusters={clusters} iters={iters} "
          f"{w.dtype}", flush=True)
    kv, q, codes, token_of = S.kv_from_workload_kmeans(w, clusters, iters)
    k2, v2, codes_ref, tok_ref = _oracle(w, clusters, iters)
    assert np.array_equal(codes.cpu().numpy(), codes_ref), "cluster ids differ from the oracle"
    assert np.array_equal(token_of.cpu().numpy(), tok_ref), "token order differs from the oracle"
    wp = W.permuted_workload(w, k2, v2, "kmeans")
    kvp, _ = S.kv_from_workload(wp)
    used = _used_pages(w).to(kv.device)
    assert torch.equal(kv.k_pages[used], kvp.k_pages[used]) and torch.equal(kv.v_pages[used], kvp.v_pages[used])


def test_kmeans_repeat_call_and_workspace_reuse():
    # A second call on the same buffers (the workspace keeps the first call's
    # centroids) gives the same result: nothing carries over.
    make, clusters, iters = CASES["bf16_d64_t32_b4_per_team"]
    w = make()
    kv, _, codes, token_of = S.kv_from_workload_kmeans(w, clusters, iters)
    k_src = S.storage_tensor(w.k_pages, w.dtype, "cuda")
    v_src = S.storage_tensor(w.v_pages, w.dtype, "cuda")
    ws = torch.full((S.santa_kmeans_workspace_size(kv, clusters),), 0x7f, dtype=torch.uint8, device="cuda")
    c2 = torch.full_like(codes, 123)
    t2 = torch.full_like(token_of, 456)
    for _ in range(2):
        S.santa_pack_pages_kmeans(kv, k_src, v_src, clusters, iters, codes=c2, token_of=t2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(c2, codes) and torch.equal(t2, token_of)


@pytest.mark.parametrize("name", ["bf16_d64_t32_b4_per_team", "f32_d128_t16_c40", "bf16_empty_seq"])
def test_santa_and_dense_on_kmeans_cache(name):
    make, clusters, iters = CASES[name]
    w = make()
    print(f"[kmeans] decode {name}", flush=True)
    kv, q, _, _ = S.kv_from_workload_kmeans(w, clusters, iters)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention(kv, q, reps, w.M, seed=w.seed, offset=w.offset,
                                                       return_sets=True)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    k2, v2, _, _ = _oracle(w, clusters, iters)
    wp = W.permuted_workload(w, k2, v2, "kmeans")
    parity.check_reps(wp, reps)
    okv_p, okv = parity.oracle_kv(wp), parity.oracle_kv(w)
    ref_reps = parity.oracle_reps(wp)
    out, lse, teams, inv_pi, dout, dlse = (x.cpu().numpy() for x in (out, lse, teams, inv_pi, dout, dlse))
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            parity.check_santa_head(wp, okv_p, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h])
            parity.check_dense_head(w, okv, b, h, dout[b, h], dlse[b, h])


def test_kmeans_full_size():
    # The 32K-token Qwen2.5-7B-shaped layer with one cluster per team (256
    # per sequence): the GPU runs every KV head; the oracle checks KV head 2
    # (ids, order and its pages bit for bit). Two assignments keep the oracle
    # to seconds.
    w = W.FULL_SIZE["qwen7b_32k_b1_m31"]()
    g, iters = 2, 2
    print(f"[kmeans full] qwen7b_32k_b1_m31 kv head {g} iters={iters}", flush=True)
    kv, q, codes, token_of = S.kv_from_workload_kmeans(w, 0, iters)
    torch.cuda.synchronize()
    w1 = W.kv_head_slice(w, g)
    k2, v2, codes_ref, tok_ref = _oracle(w1, 0, iters)
    assert np.array_equal(codes[:, g].cpu().numpy(), codes_ref[:, 0])
    assert np.array_equal(token_of[:, g].cpu().numpy(), tok_ref[:, 0])
    wp = W.permuted_workload(w1, k2, v2, "kmeans")
    kvp, _ = S.kv_from_workload(wp)
    used = _used_pages(w).to(kv.device)
    assert torch.equal(kv.k_pages[used][:, g], kvp.k_pages[used][:, 0])
    assert torch.equal(kv.v_pages[used][:, g], kvp.v_pages[used][:, 0])

"""Hash-partitioned teams (santa_pack_pages_hashed): codes, the stable sort
and the packed pages are bit-exact against the oracle; SANTA++ on the hashed
cache matches the oracle on the permuted cache head by head, and dense
attention is unchanged by the permutation."""
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


CASES = {
    "bf16_d64_t32_b4": (lambda: W.paged_ragged(num_seqs=4, len_min=300, len_max=5000, T=32, M=12, hq=8, hkv=2,
                                               d=64), 6),
    "f32_d128_t16": (lambda: W.qwen_planted(batch=2, seq_len=3000, T=16, M=20, hq=4, hkv=2, d=128, plants=4,
                                            dtype="f32"), 7),
    "bf16_d128_t128_bits1": (lambda: W.qwen_planted(batch=1, seq_len=4096 + 77, T=128, M=8, hq=8, hkv=2,
                                                    plants=4), 1),
    "bf16_t256_mixture_bits10": (lambda: W.gaussian_mixture(batch=2, seq_len=5000, T=256, M=6, hq=4, hkv=2,
                                                            d=64, run_min=1, run_max=16), 10),
    "bf16_t16_p2048_bits10": (lambda: W.qwen_planted(batch=1, seq_len=32768, T=16, M=24, hq=4, hkv=1, d=64,
                                                     plants=4), 10),
    "bf16_empty_seq": (lambda: _zero_len(W.paged_ragged(num_seqs=3, len_min=100, len_max=2000, T=32, M=8, hq=4,
                                                        hkv=2, d=64), 1), 5),
}


def _used_pages(w):
    pages = []
    for b in range(w.batch):
        pages += [int(p) for p in w.page_table[b][:O.num_teams(int(w.seq_lens[b]), w.page_size)]]
    return torch.tensor(sorted(pages), dtype=torch.long)


@pytest.mark.parametrize("name", list(CASES))
def test_hashed_pack_matches_oracle(name):
    make, bits = CASES[name]
    w = make()
    dirs = W.hash_directions(hkv=w.num_kv_heads, bits=bits, d=w.head_dim)
    print(f"[hashed] {name} B={w.batch} T={w.page_size} d={w.head_dim} bits={bits} {w.dtype}", flush=True)
    kv, q, codes, token_of = S.kv_from_workload_hashed(w, dirs)
    k2, v2, codes_ref, tok_ref = O.cluster_pages(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size,
                                                 w.dtype, dirs)
    assert np.array_equal(codes.cpu().numpy(), codes_ref), "hash codes differ from the oracle"
    assert np.array_equal(token_of.cpu().numpy(), tok_ref), "token order differs from the oracle"
    # The pages of every sequence equal the plain pack of the oracle's permuted pages.
    wp = W.permuted_workload(w, k2, v2)
    kvp, _ = S.kv_from_workload(wp)
    used = _used_pages(w).to(kv.device)
    assert torch.equal(kv.k_pages[used], kvp.k_pages[used]) and torch.equal(kv.v_pages[used], kvp.v_pages[used])


@pytest.mark.parametrize("name", ["bf16_d64_t32_b4", "f32_d128_t16", "bf16_t256_mixture_bits10", "bf16_empty_seq"])
def test_santa_and_dense_on_hashed_cache(name):
    make, bits = CASES[name]
    w = make()
    dirs = W.hash_directions(hkv=w.num_kv_heads, bits=bits, d=w.head_dim)
    print(f"[hashed] decode {name}", flush=True)
    kv, q, _, _ = S.kv_from_workload_hashed(w, dirs)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention(kv, q, reps, w.M, seed=w.seed, offset=w.offset,
                                                       return_sets=True)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    k2, v2, _, _ = O.cluster_pages(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size, w.dtype, dirs)
    wp = W.permuted_workload(w, k2, v2)
    parity.check_reps(wp, reps)
    okv_p, okv = parity.oracle_kv(wp), parity.oracle_kv(w)
    ref_reps = parity.oracle_reps(wp)
    out, lse, teams, inv_pi, dout, dlse = (x.cpu().numpy() for x in (out, lse, teams, inv_pi, dout, dlse))
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            parity.check_santa_head(wp, okv_p, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h])
            parity.check_dense_head(w, okv, b, h, dout[b, h], dlse[b, h])   # the original order


@pytest.mark.parametrize("name,pairs", [("qwen7b_32k_b1_m31", [(0, 0), (0, 20)]),
                                        ("mixture_128k_b4_t256_m64", [(1, 5), (3, 26)])])
def test_hashed_full_size(name, pairs):
    # Full-size configurations: codes, order and pages of every sequence bit
    # for bit; SANTA++ on the hashed cache for a sample of heads.
    w = W.FULL_SIZE[name]()
    K = max(1, -(-int(w.seq_lens.max()) // w.page_size))
    bits = min(10, max(1, int(np.ceil(np.log2(K)))))
    dirs = W.hash_directions(hkv=w.num_kv_heads, bits=bits, d=w.head_dim)
    print(f"[hashed full] {name} bits={bits} heads={pairs}", flush=True)
    kv, q, codes, token_of = S.kv_from_workload_hashed(w, dirs)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention(kv, q, reps, w.M, seed=w.seed, offset=w.offset,
                                                       return_sets=True)
    torch.cuda.synchronize()
    k2, v2, codes_ref, tok_ref = O.cluster_pages(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size,
                                                 w.dtype, dirs)
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert np.array_equal(token_of.cpu().numpy(), tok_ref)
    wp = W.permuted_workload(w, k2, v2)
    kvp, _ = S.kv_from_workload(wp)
    used = _used_pages(w).to(kv.device)
    assert torch.equal(kv.k_pages[used], kvp.k_pages[used]) and torch.equal(kv.v_pages[used], kvp.v_pages[used])
    del kvp
    ref_reps = parity.check_reps(wp, reps, pairs)
    okv = parity.oracle_kv(wp)
    out, lse, teams, inv_pi = (x.cpu().numpy() for x in (out, lse, teams, inv_pi))
    for b, h in pairs:
        parity.check_santa_head(wp, okv, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h])

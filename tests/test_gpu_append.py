"""GPU: a serving loop that grows the cache with santa_append_kv.

Each step appends a few tokens per sequence (none for some, across a page
boundary for others, one sequence starting empty), refreshes the
representatives with santa_update_reps and decodes; every head is compared
with the CPU oracle at the new lengths. After the loop the cache tiles must
equal, byte for byte, the tiles santa_pack_pages writes from the whole
sequences. Every case prints what it runs before its first GPU call.
"""
import numpy as np
import pytest
import torch

from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()


def say(*a):
    print(*a, flush=True)


def _shuffled(w, seed=11):
    """w with its physical pages permuted (the page table follows)."""
    perm = np.random.default_rng(seed).permutation(w.num_pages).astype(np.int32)
    k = np.empty_like(w.k_pages)
    v = np.empty_like(w.v_pages)
    k[perm] = w.k_pages
    v[perm] = w.v_pages
    return W.dataclasses.replace(w, k_pages=k, v_pages=v, page_table=perm[w.page_table])


def _truncated(w, lens):
    """Plain pages of w with every position at or beyond lens[b] zeroed."""
    k, v = w.k_pages.copy(), w.v_pages.copy()
    T = w.page_size
    for b in range(w.batch):
        for t in range(w.max_pages_per_seq):
            lo = int(lens[b]) - t * T
            if lo < T:
                pg = w.page_table[b, t]
                k[pg, :, max(lo, 0):] = 0
                v[pg, :, max(lo, 0):] = 0
    return k, v


def _rows(w, pages, lo, hi, width):
    """[B][width][Hkv][d] rows of positions lo[b] .. hi[b] - 1 (zero after)."""
    out = np.zeros((w.batch, width, w.num_kv_heads, w.head_dim), dtype=pages.dtype)
    T = w.page_size
    for b in range(w.batch):
        for i, pos in enumerate(range(int(lo[b]), int(hi[b]))):
            out[b, i] = pages[w.page_table[b, pos // T], :, pos % T]
    return out


def _bits(t):
    """A tensor's bit patterns on the host (so -0.0 and 0.0 differ)."""
    t = t.cpu()
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _cache(w, k_plain, v_plain, lens, dev):
    k_pages, v_pages = S.pack_pages(S.storage_tensor(k_plain, w.dtype, dev), S.storage_tensor(v_plain, w.dtype, dev))
    return S.KVCache(k_pages, v_pages, torch.from_numpy(w.page_table.astype(np.int32)).to(dev),
                     torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev), w.num_q_heads, w.page_size)


CASES = {
    # bf16, 32-token pages, 4 sequences (one starts empty), GQA group 4
    "bf16_t32": dict(make=lambda: W.qwen_planted(batch=4, seq_len=1500, T=32, M=12, hq=8, hkv=2, d=128, plants=3),
                     steps=[[1, 1, 1, 1], [0, 3, 40, 1], [5, 0, 1, 33], [1, 1, 0, 64]], start_empty=2),
    # float32, 16-token pages, head_dim 64
    "f32_t16_d64": dict(make=lambda: W.qwen_planted(batch=3, seq_len=700, T=16, M=9, hq=4, hkv=1, d=64, plants=2,
                                                    dtype="f32"),
                        steps=[[1, 2, 17], [16, 0, 1], [3, 1, 0]], start_empty=1),
}


@pytest.mark.parametrize("name", list(CASES))
def test_serving_loop_append_update_decode(name):
    case = CASES[name]
    w = _shuffled(case["make"]())
    dev = torch.device("cuda:0")
    full = w.seq_lens.astype(np.int64).copy()
    grow = np.asarray(case["steps"], dtype=np.int64)              # [steps][B]
    start = full - grow.sum(0)
    start[case["start_empty"]] = 0                                  # this sequence is empty before the loop
    full[case["start_empty"]] = grow[:, case["start_empty"]].sum()
    assert (start >= 0).all()
    k0, v0 = _truncated(w, start)
    say(f"[append] {name} B={w.batch} T={w.page_size} d={w.head_dim} {w.dtype} start={start.tolist()} "
        f"steps={grow.tolist()}")
    kv = _cache(w, k0, v0, start, dev)
    q = S.storage_tensor(w.q, w.dtype, dev)
    reps = S.santa_build_reps(kv)
    lens = start.copy()
    flips = 0
    for s, n in enumerate(grow):
        new = lens + n
        width = max(1, int(n.max()))
        k_new = S.storage_tensor(_rows(w, w.k_pages, lens, new, width), w.dtype, dev)
        v_new = S.storage_tensor(_rows(w, w.v_pages, lens, new, width), w.dtype, dev)
        prev = torch.from_numpy(lens.astype(np.int32)).to(dev)
        kv.seq_lens.copy_(torch.from_numpy(new.astype(np.int32)).to(dev))
        say(f"  step {s}: lengths {lens.tolist()} -> {new.tolist()}")
        S.santa_append_kv(kv, prev, k_new, v_new)
        S.santa_update_reps(kv, reps, prev, width)
        out, lse, teams, inv_pi = S.santa_decode_attention(kv, q, reps, w.M, w.seed, w.offset + s, return_sets=True)
        torch.cuda.synchronize()
        lens = new
        ws = W.dataclasses.replace(w, seq_lens=lens.astype(np.int32))
        oreps = parity.check_reps(ws, reps)
        okv = parity.oracle_kv(ws)
        out, lse, teams, inv_pi = (x.cpu().numpy() for x in (out, lse, teams, inv_pi))
        for b in range(w.batch):
            for h in range(w.num_q_heads):
                _, f = parity.check_santa_head(ws, okv, oreps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h],
                                               offset=w.offset + s)
                flips += f
    say(f"  near-tie flips: {flips}")
    assert flips <= parity.MAX_FLIPS
    # The grown cache holds exactly the tiles a fresh pack of the whole sequences gives.
    kf, vf = _truncated(w, lens)
    ref = _cache(w, kf, vf, lens, dev)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kv.k_pages), _bits(ref.k_pages))
    assert torch.equal(_bits(kv.v_pages), _bits(ref.v_pages))


def test_append_skips_positions_past_the_table():
    """Lengths past the page table's capacity: only positions inside it are
    written; nothing else in the cache changes."""
    w = _shuffled(W.qwen_planted(batch=2, seq_len=256, T=32, M=4, hq=4, hkv=2, d=64, plants=1))
    dev = torch.device("cuda:0")
    cap = w.max_pages_per_seq * w.page_size
    say(f"[append] capacity {cap}: prev [cap - 1, 10], new [cap + 2, 10]")
    k0, v0 = _truncated(w, [cap - 1, 10])
    kv = _cache(w, k0, v0, [cap - 1, 10], dev)
    before_k = _bits(kv.k_pages)
    rows_k = _rows(w, w.k_pages, [cap - 1, 10], [cap, 10], 3)
    rows_v = _rows(w, w.v_pages, [cap - 1, 10], [cap, 10], 3)
    rows_k[0, 1:] = 0x3f80 if w.dtype == "bf16" else 1.0          # rows past the table: must not land anywhere
    rows_v[0, 1:] = 0x3f80 if w.dtype == "bf16" else 1.0
    prev = torch.tensor([cap - 1, 10], dtype=torch.int32, device=dev)
    kv.seq_lens.copy_(torch.tensor([cap + 2, 10], dtype=torch.int32, device=dev))
    S.santa_append_kv(kv, prev, S.storage_tensor(rows_k, w.dtype, dev), S.storage_tensor(rows_v, w.dtype, dev))
    torch.cuda.synchronize()
    kf, vf = _truncated(w, [cap, 10])
    ref = _cache(w, kf, vf, [cap, 10], dev)
    torch.cuda.synchronize()
    assert torch.equal(_bits(kv.k_pages), _bits(ref.k_pages))
    assert torch.equal(_bits(kv.v_pages), _bits(ref.v_pages))
    assert not torch.equal(before_k, _bits(ref.k_pages))          # the one valid position was written

"""HIP-graph capture of the decode entry points (the benchmark times graph
replays): every replay, with eager work and synchronisations between the
replays, must reproduce the eager results bit for bit."""
import numpy as np
import pytest
import torch

from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()


def test_graph_replays_match_eager():
    w = W.qwen_planted(batch=2, seq_len=4096 + 77, M=31)
    print(f"[graph] {w.name}", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    ws_s, ws_d = S.make_workspace(kv, w.M), S.make_workspace(kv, w.M)
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    dout = torch.empty_like(out)
    dlse = torch.empty_like(lse)

    def step():
        S.santa_decode_attention(kv, q, reps, w.M, w.seed, 5, ws_s, out, lse)
        S.dense_decode_attention(kv, q, ws_d, dout, dlse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, dout, dlse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t in (out, lse, dout, dlse):
            t.fill_(float("nan"))
        # eager work of the program between replays
        S.santa_decode_attention(kv, q, reps, w.M, w.seed, 6 + r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, lse, dout, dlse), ref):
            assert torch.equal(got, want), f"replay {r} differs from the eager result"


@pytest.mark.parametrize("scheme", ["iid", "stratified"])
def test_graph_captured_decode_loop(scheme):
    # One serving step captured once and replayed: every sequence gets its
    # next token's key and value (gathered on the device from the plain
    # pages at the current length) written by santa_append_kv, the lengths
    # advance, the touched teams' representatives are refreshed, and the
    # layer is decoded. The cache starts with every position past the start
    # lengths zeroed. After each replay the representatives equal a fresh
    # full build and the outputs an eager decode at the new lengths, bit for
    # bit; at the end the grown tiles equal a fresh pack of the sequences.
    w = W.paged_ragged(num_seqs=3, len_min=500, len_max=1500, T=32, M=16, hq=8, hkv=2, d=128)
    print(f"[graph loop] {scheme}", flush=True)
    steps = 6
    final = w.seq_lens.astype(np.int64)
    start = final - (steps + 2)                      # start a few tokens back
    T = w.page_size

    def truncated(lens):
        k, v = w.k_pages.copy(), w.v_pages.copy()
        for b in range(w.batch):
            for t in range(w.max_pages_per_seq):
                lo = int(lens[b]) - t * T
                if lo < T:
                    k[w.page_table[b, t], :, max(lo, 0):] = 0
                    v[w.page_table[b, t], :, max(lo, 0):] = 0
        return k, v

    def cache(k_plain, v_plain, lens):
        kp, vp = S.pack_pages(S.storage_tensor(k_plain, w.dtype, "cuda"), S.storage_tensor(v_plain, w.dtype, "cuda"))
        return S.KVCache(kp, vp, torch.from_numpy(w.page_table.astype(np.int32)).cuda(),
                         torch.from_numpy(lens.astype(np.int32)).cuda(), w.num_q_heads, T)

    kv = cache(*truncated(start), start)
    q = S.storage_tensor(w.q, w.dtype, "cuda")
    k_src = S.storage_tensor(w.k_pages, w.dtype, "cuda")         # [pages][Hkv][T][d], every token
    v_src = S.storage_tensor(w.v_pages, w.dtype, "cuda")
    table = kv.page_table.long()
    rows = torch.arange(w.batch, device="cuda")
    reps = S.santa_build_reps(kv)
    prev = kv.seq_lens.clone()
    ws = S.make_workspace(kv, w.M)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")

    def step():
        prev.copy_(kv.seq_lens)
        pos = prev.long()
        page = table[rows, pos // T]
        k_new = k_src[page, :, pos % T, :].unsqueeze(1).contiguous()   # [B][1][Hkv][d]
        v_new = v_src[page, :, pos % T, :].unsqueeze(1).contiguous()
        kv.seq_lens.add_(1)
        S.santa_append_kv(kv, prev, k_new, v_new)
        S.santa_update_reps(kv, reps, prev, 1)
        S.santa_decode_attention_ex(kv, q, reps, w.M, scheme, 3, 11, ws, out, lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                       # warm-up step (one token)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()                                       # capture only: lengths do not move
    torch.cuda.synchronize()
    for r in range(steps):
        g.replay()
        torch.cuda.synchronize()
        fresh = S.santa_build_reps(kv)
        o2, l2 = S.santa_decode_attention_ex(kv, q, fresh, w.M, scheme, 3, 11)
        torch.cuda.synchronize()
        assert torch.equal(reps, fresh), f"replay {r}: representatives differ from a full build"
        assert torch.equal(out, o2) and torch.equal(lse, l2), f"replay {r}: outputs differ from eager"
    lens = kv.seq_lens.cpu().numpy().astype(np.int64)
    assert np.array_equal(lens, final - 1)
    ref = cache(*truncated(lens), lens)
    torch.cuda.synchronize()
    assert torch.equal(kv.k_pages.view(torch.int16), ref.k_pages.view(torch.int16)), "grown keys differ from a fresh pack"
    assert torch.equal(kv.v_pages.view(torch.int16), ref.v_pages.view(torch.int16)), "grown values differ from a fresh pack"

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
    # One serving step captured once and replayed: advance every sequence by
    # one token (its key and value already in the pages), refresh the
    # representatives of the touched teams, decode. After each replay the
    # representatives equal a fresh full build and the outputs equal an
    # eager decode at the new lengths, bit for bit.
    w = W.paged_ragged(num_seqs=3, len_min=500, len_max=1500, T=32, M=16, hq=8, hkv=2, d=128)
    print(f"[graph loop] {scheme}", flush=True)
    kv, q = S.kv_from_workload(w)
    final = kv.seq_lens.clone()
    steps = 6
    kv.seq_lens.sub_(steps + 2)                      # start a few tokens back
    reps = S.santa_build_reps(kv)
    prev = kv.seq_lens.clone()
    ws = S.make_workspace(kv, w.M)
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device="cuda")

    def step():
        prev.copy_(kv.seq_lens)
        kv.seq_lens.add_(1)
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
    assert torch.equal(kv.seq_lens, final - 1)

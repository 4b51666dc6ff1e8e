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

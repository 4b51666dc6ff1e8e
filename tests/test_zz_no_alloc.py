"""santa_decode_attention_noalloc (the workspace-free entry point) through
the C ABI against santa_decode_attention on the same inputs: team sets,
weights, outputs and log-sum-exp bit for bit, over calls in a row whose
sizes shrink (the device scratch keeps the previous call's contents)."""
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


def say(*a):
    print(*a, flush=True)


CASES = [
    ("bf16 32K-shaped, batch 2", lambda: W.qwen_mixed_query(batch=2, seq_len=8192, M=32)),
    ("bf16 ragged, 3 sequences (smaller)", lambda: W.paged_ragged(num_seqs=3, len_min=200, len_max=3000, M=12,
                                                                 hq=8, hkv=2, T=64)),
    ("fp32 tiny (smaller)", lambda: W.tiny_planted()),
]


def _run(kv, q, reps, w, noalloc):
    B, Hq, M = w.batch, w.num_q_heads, w.M
    sampled = torch.full((B, Hq, M), 7, dtype=torch.int32, device="cuda")
    inv_pi = torch.full((B, Hq, M), 7.0, dtype=torch.float32, device="cuda")
    out = torch.full((B, Hq, w.head_dim), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), 7.0, dtype=torch.float32, device="cuda")
    if noalloc:
        S.santa_decode_attention_noalloc(kv, q, reps, M, w.seed, w.offset, out, lse, sampled, inv_pi)
    else:
        ws = S.make_workspace(kv, M)
        S.santa_decode_attention(kv, q, reps, M, w.seed, w.offset, ws, out, lse)
        S.santa_select_teams(kv, q, reps, M, w.seed, w.offset, ws, sampled, inv_pi)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (out, lse, sampled, inv_pi)]


def test_noalloc_equals_decode_on_shrinking_calls():
    for name, make in CASES:
        w = make()
        say(f"[noalloc] {name}: B={w.batch} Hq={w.num_q_heads} P={w.max_pages_per_seq} M={w.M} {w.dtype}")
        kv, q = S.kv_from_workload(w)
        reps = S.santa_build_reps(kv)
        ref = _run(kv, q, reps, w, noalloc=False)
        got = _run(kv, q, reps, w, noalloc=True)
        for label, a, b in zip(("out", "lse", "sampled", "inv_pi"), ref, got):
            assert np.array_equal(a, b), f"{name}: {label} differs from santa_decode_attention"
        assert np.all(np.isfinite(got[0]))

"""santa_update_reps: after tokens are appended, refreshing only the teams
that received them gives the oracle's representatives of the new lengths bit
for bit, and leaves every other row untouched."""
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


def _sentinel_reps(kv):
    reps = torch.empty((kv.batch, kv.max_pages_per_seq, kv.num_kv_heads, kv.head_dim), dtype=kv.dtype,
                       device=kv.device)
    reps.fill_(-7.0)                     # a value no team mean of these inputs takes
    return reps


@pytest.mark.parametrize("dtype,T", [("bf16", 32), ("f32", 16), ("bf16", 128)])
def test_update_after_append_matches_rebuild(dtype, T):
    w = W.paged_ragged(num_seqs=5, len_min=400, len_max=3000, T=T, M=8, hq=8, hkv=2, d=64, dtype=dtype)
    new_lens = w.seq_lens.copy()
    appended = np.array([1, 5, T, 3 * T + 7, 2 * T - 1])[: w.batch]
    old_lens = np.maximum(new_lens - appended, 0).astype(np.int32)
    print(f"[update_reps] {dtype} T={T} old={list(old_lens)} new={list(new_lens)}", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = _sentinel_reps(kv)
    kv.seq_lens.copy_(torch.from_numpy(old_lens))
    S.santa_build_reps(kv, reps)                       # representatives before the append
    kv.seq_lens.copy_(torch.from_numpy(new_lens))
    prev = torch.from_numpy(old_lens).cuda()
    S.santa_update_reps(kv, reps, prev, int(appended.max()))
    torch.cuda.synchronize()
    parity.check_reps(w, reps)                         # every team of the new lengths
    got = reps.float().cpu().numpy()
    for b in range(w.batch):
        K = -(-int(new_lens[b]) // T)
        assert np.all(got[b, K:] == -7.0), f"sequence {b}: rows past its last team were written"


def test_token_by_token_decode_keeps_reps_exact():
    w = W.qwen_planted(batch=2, seq_len=2000, T=32, M=8, hq=8, hkv=2, d=64, plants=2)
    final = w.seq_lens.copy()
    start = final - 70
    print(f"[update_reps] decode from {list(start)} to {list(final)}", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = _sentinel_reps(kv)
    lens = torch.from_numpy(start.astype(np.int32)).cuda()
    kv.seq_lens.copy_(lens)
    S.santa_build_reps(kv, reps)
    for step in range(70):
        prev = kv.seq_lens.clone()
        kv.seq_lens.add_(1)
        S.santa_update_reps(kv, reps, prev, 1)
    torch.cuda.synchronize()
    assert np.array_equal(kv.seq_lens.cpu().numpy(), final)
    parity.check_reps(w, reps)


def test_update_with_no_growth_writes_nothing():
    # prev >= new length for every sequence (equal, or a rolled-back
    # sequence): no team received tokens, so no row may change.
    w = W.paged_ragged(num_seqs=3, len_min=300, len_max=900, T=32, M=8, hq=4, hkv=2, d=64)
    print("[update_reps] no growth", flush=True)
    kv, _ = S.kv_from_workload(w)
    reps = _sentinel_reps(kv)
    prev = torch.from_numpy((w.seq_lens + np.array([0, 5, 40])).astype(np.int32)).cuda()
    S.santa_update_reps(kv, reps, prev, 64)
    torch.cuda.synchronize()
    assert np.all(reps.float().cpu().numpy() == -7.0)

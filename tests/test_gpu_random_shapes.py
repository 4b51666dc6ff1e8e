"""Randomised shapes against the oracle: a fixed list of configurations
drawn from one seed covers cache type, head dim, team size, group size,
batch, ragged lengths (from one token up), draw count and draw scheme.
Every head of every configuration is compared (sets, weights, outputs,
lse), together with the representatives and the dense baseline.

A second, wider list (up to 100 sequences and 8 KV heads, so more than 256
(sequence, KV head) groups; sequences up to 60K tokens and 2047 teams)
compares a sample of heads per configuration, which the oracle evaluates
one by one."""
import numpy as np
import pytest
import torch

from oracle import santa as O
from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu

SCHEMES = {"iid": O.DRAW_IID, "systematic": O.DRAW_SYSTEMATIC, "stratified": O.DRAW_STRATIFIED}


def _configs(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([16, 32, 64, 128, 256]))
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 5, 7, 8, 16]))
        seqs = int(rng.integers(1, 6))
        if rng.random() < 0.3:                       # short sequences: one team, ragged, single tokens
            len_max = int(rng.integers(1, 2 * T + 1))
            len_min = 1
        else:
            cap = max(1, 6000 // T)                  # at most ~6000 tokens per sequence
            len_max = int(rng.integers(1, cap + 1)) * T + int(rng.integers(0, T))
            len_min = int(rng.integers(1, len_max + 1))
        out.append(dict(name=f"r{i:02d}", dtype=str(rng.choice(["bf16", "f32"])), T=T, d=d, hkv=hkv, hq=G * hkv,
                        seqs=seqs, len_min=len_min, len_max=len_max, M=int(rng.integers(1, 81)),
                        scheme=str(rng.choice(list(SCHEMES))), data_seed=int(rng.integers(0, 2 ** 31)),
                        philox_seed=int(rng.integers(0, 2 ** 63)), offset=int(rng.integers(0, 2 ** 32))))
    return out


CONFIGS = _configs()


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c["name"] for c in CONFIGS])
def test_random_shape(cfg):
    w = W.paged_ragged(data_seed=cfg["data_seed"], num_seqs=cfg["seqs"], len_min=cfg["len_min"],
                       len_max=cfg["len_max"], T=cfg["T"], M=cfg["M"], hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                       dtype=cfg["dtype"], philox_seed=cfg["philox_seed"])
    w = W.dataclasses.replace(w, offset=cfg["offset"])
    print(f"[random] {cfg}", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention_ex(kv, q, reps, w.M, cfg["scheme"], seed=w.seed,
                                                          offset=w.offset, return_sets=True)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    ref_reps = parity.check_reps(w, reps)
    okv = parity.oracle_kv(w)
    out, lse, teams, inv_pi, dout, dlse = (x.cpu().numpy() for x in (out, lse, teams, inv_pi, dout, dlse))
    flips = 0
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            _, flip = parity.check_santa_head(w, okv, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h],
                                              inv_pi[b, h], scheme=SCHEMES[cfg["scheme"]])
            flips += flip
            parity.check_dense_head(w, okv, b, h, dout[b, h], dlse[b, h])
    assert flips <= max(1, w.batch * w.num_q_heads // 50)


def _wide_configs(n=64, seed=777):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        T = int(rng.choice([16, 32, 64, 128, 256]))
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 7, 8, 16]))
        seqs = int(rng.choice([1, 2, 3, 8, 16, 33, 70, 100]))
        if rng.random() < 0.25:
            len_min, len_max = 1, int(rng.integers(1, 3 * T + 1))
        else:
            cap = min(max(1, int(rng.choice([2000, 20000, 60000])) // T), 2047)
            len_max = int(rng.integers(1, cap + 1)) * T + int(rng.integers(0, T))
            len_min = int(rng.integers(1, len_max + 1)) if rng.random() < 0.7 else len_max
        if seqs * len_max * hkv * d > 3e8:            # cache of at most ~1.2 GB
            continue
        M = int(rng.choice([1, 2, 7, 16, 31, 48, 64, 200]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        out.append(dict(name=f"w{len(out):02d}", T=T, d=d, hkv=hkv, hq=G * hkv, seqs=seqs, len_min=len_min,
                        len_max=len_max, M=M, dtype=dtype, scheme=str(rng.choice(list(SCHEMES))),
                        data_seed=int(rng.integers(0, 2 ** 31)), philox_seed=int(rng.integers(0, 2 ** 63)),
                        offset=int(rng.integers(0, 2 ** 32))))
    return out


# Page tables of 1250-2047 teams (the random draw above rarely reaches them).
LONG_TABLES = [
    dict(name="long_t16_bf16", T=16, d=64, hkv=2, hq=14, seqs=3, len_min=20000, len_max=32750, M=48, dtype="bf16",
         scheme="iid", data_seed=91, philox_seed=17, offset=3),
    dict(name="long_t32_f32", T=32, d=64, hkv=1, hq=4, seqs=2, len_min=40000, len_max=65500, M=31, dtype="f32",
         scheme="stratified", data_seed=92, philox_seed=18, offset=4),
    dict(name="long_t16_g64", T=16, d=128, hkv=4, hq=28, seqs=16, len_min=1, len_max=20000, M=64, dtype="bf16",
         scheme="systematic", data_seed=93, philox_seed=19, offset=5),
]
WIDE = _wide_configs() + LONG_TABLES


@pytest.mark.parametrize("cfg", WIDE, ids=[c["name"] for c in WIDE])
def test_random_wide_shape(cfg):
    w = W.paged_ragged(data_seed=cfg["data_seed"], num_seqs=cfg["seqs"], len_min=cfg["len_min"],
                       len_max=cfg["len_max"], T=cfg["T"], M=cfg["M"], hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                       dtype=cfg["dtype"], philox_seed=cfg["philox_seed"])
    w = W.dataclasses.replace(w, offset=cfg["offset"])
    rng = np.random.default_rng(cfg["data_seed"])
    pairs = sorted(set([(int(rng.integers(0, w.batch)), int(rng.integers(0, w.num_q_heads))) for _ in range(6)]
                       + [(0, 0), (w.batch - 1, w.num_q_heads - 1)]))
    print(f"[wide] {cfg} heads={pairs}", flush=True)
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, inv_pi = S.santa_decode_attention_ex(kv, q, reps, w.M, cfg["scheme"], seed=w.seed,
                                                          offset=w.offset, return_sets=True)
    dout, dlse = S.dense_decode_attention(kv, q)
    torch.cuda.synchronize()
    ref_reps = parity.check_reps(w, reps, pairs)
    okv = parity.oracle_kv(w)
    out, lse, teams, inv_pi, dout, dlse = (x.cpu().numpy() for x in (out, lse, teams, inv_pi, dout, dlse))
    for b, h in pairs:
        parity.check_santa_head(w, okv, ref_reps, b, h, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h],
                                scheme=SCHEMES[cfg["scheme"]])
        parity.check_dense_head(w, okv, b, h, dout[b, h], dlse[b, h])
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(dout))

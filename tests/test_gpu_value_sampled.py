"""GPU: SANTA++ team draws followed by value samples inside the drawn teams
(santa_decode_attention_value_sampled) against the CPU oracle.

The teams, weights and log-sum-exp are SANTA++'s; each of the S samples must
land on the oracle's token (a near-tie sample may take a neighbour it can
reach), and the output must be the mean of the sampled tokens' values. Every
case prints what it runs before its first GPU call.
"""
import numpy as np
import pytest
import torch

from sampled_sparse_decode_amd import santa as S
from sampled_sparse_decode_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu

MAX_SAMPLE_FLIPS = 2      # near-tie samples per workload (float64 cumulative sums: expected ~0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()


def say(*a):
    print(*a, flush=True)


def _with_lens(w, lens):
    return W.dataclasses.replace(w, seq_lens=np.asarray(lens, dtype=w.seq_lens.dtype))


def run_vs(w, kv, q, reps, S_, scheme="iid", value_scheme="iid", M=None, offset=None):
    out, lse, teams, inv_pi, pos = S.santa_decode_attention_value_sampled(
        kv, q, reps, w.M if M is None else M, S_, scheme, value_scheme, w.seed,
        w.offset if offset is None else offset, return_sets=True, return_positions=True)
    torch.cuda.synchronize()
    return tuple(x.cpu().numpy() for x in (out, lse, teams, inv_pi, pos))


def compare(w, res, S_, pairs=None, scheme="iid", value_scheme="iid", M=None, offset=None, okv=None, reps=None):
    out, lse, teams, inv_pi, pos = res
    okv = parity.oracle_kv(w) if okv is None else okv
    reps = parity.oracle_reps(w, pairs) if reps is None else reps
    pairs = pairs or [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]
    flips = 0
    for b, h in pairs:
        _, f = parity.check_value_sampled_head(
            w, okv, reps, b, h, S_, out[b, h], lse[b, h], teams[b, h], inv_pi[b, h], pos[b, h], M=M, offset=offset,
            scheme=S._SCHEMES[scheme], value_scheme=S._SCHEMES[value_scheme])
        flips += f
    return flips


SMALL = {
    "tiny_f32": (lambda: W.tiny_planted(), 64),
    "qwen_bf16_ragged": (lambda: W.qwen_planted(batch=1, seq_len=4096 + 77, M=31), 128),
    "mixture_t256": (lambda: W.gaussian_mixture(batch=2, seq_len=8192 + 100, T=256, M=16), 256),
    "f32_d128_t64_g2": (lambda: W.qwen_planted(batch=2, seq_len=3000, T=64, M=9, hq=4, hkv=2, d=128, plants=3,
                                               dtype="f32"), 33),
    "bf16_d64_t16_g16": (lambda: W.qwen_planted(batch=2, seq_len=1000, T=16, M=12, hq=16, hkv=1, d=64,
                                                plants=2), 1),
    "paged_ragged": (lambda: W.paged_ragged(num_seqs=4, len_min=300, len_max=9000, M=20), 17),
    "bf16_full_coverage": (lambda: W.qwen_planted(batch=2, seq_len=300, T=64, M=8, hq=8, hkv=2, d=128,
                                                  plants=1), 200),
    "bf16_empty_and_short": (lambda: _with_lens(W.qwen_mixed_query(batch=4, seq_len=9000, T=64, M=24, hq=8, hkv=2,
                                                                   d=128), [0, 1, 50, 9000]), 40),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_value_sampled_parity(name):
    make, S_ = SMALL[name]
    w = make()
    say(f"[value_sampled] {name} B={w.batch} Hq={w.num_q_heads} T={w.page_size} M={w.M} S={S_} {w.dtype}")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    res = run_vs(w, kv, q, reps_gpu, S_)
    reps = parity.check_reps(w, reps_gpu)
    flips = compare(w, res, S_, reps=reps)
    say(f"  near-tie flips: {flips}")
    assert flips <= MAX_SAMPLE_FLIPS


@pytest.mark.parametrize("scheme,value_scheme", [("systematic", "systematic"), ("stratified", "stratified"),
                                                 ("iid", "systematic"), ("stratified", "iid")])
def test_value_sampled_schemes(scheme, value_scheme):
    w = W.qwen_mixed_query(batch=2, seq_len=8192, M=32)
    S_ = 96
    say(f"[value_sampled schemes] teams {scheme}, values {value_scheme}, S={S_}")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    res = run_vs(w, kv, q, reps_gpu, S_, scheme, value_scheme)
    flips = compare(w, res, S_, scheme=scheme, value_scheme=value_scheme)
    assert flips <= MAX_SAMPLE_FLIPS
    if value_scheme == "systematic":
        # one shared offset: the sampled positions are non-decreasing in sample order
        pos = res[4]
        assert np.all(np.diff(pos.astype(np.int64), axis=-1) >= 0)


def test_value_sampled_teams_equal_select_and_deterministic():
    """The team lists and weights are santa_select_teams'; two calls agree bit
    for bit; another offset moves the samples."""
    w = W.qwen_mixed_query(batch=2, seq_len=8192, M=32)
    say("[value_sampled] teams == select, determinism")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    a = run_vs(w, kv, q, reps, 64)
    b = run_vs(w, kv, q, reps, 64)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    ws = S.make_workspace(kv, w.M)
    teams = torch.empty((w.batch, w.num_q_heads, w.M), dtype=torch.int32, device="cuda")
    inv_pi = torch.empty((w.batch, w.num_q_heads, w.M), dtype=torch.float32, device="cuda")
    S.santa_select_teams(kv, q, reps, w.M, w.seed, w.offset, ws, teams, inv_pi)
    torch.cuda.synchronize()
    assert np.array_equal(a[2], teams.cpu().numpy()) and np.array_equal(a[3], inv_pi.cpu().numpy())
    c = run_vs(w, kv, q, reps, 64, offset=w.offset + 1)
    assert not np.array_equal(a[4], c[4])


def test_value_sampled_all_empty_and_limits():
    w = _with_lens(W.paged_ragged(num_seqs=3, len_min=100, len_max=900, T=32, M=5, hq=4, hkv=2, d=64), [0, 0, 0])
    say("[value_sampled] all sequences empty; S = 256; token limit")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    out, lse, teams, _, pos = run_vs(w, kv, q, reps, 256)
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and np.all(teams == -1) and np.all(pos == -1)
    # more drawn tokens than one block holds on chip: refused on the host
    w2 = W.qwen_planted(batch=1, seq_len=32768, T=256, M=8, hq=4, hkv=1, d=64, plants=1)
    kv2, q2 = S.kv_from_workload(w2)
    reps2 = S.santa_build_reps(kv2)
    with pytest.raises(RuntimeError):
        S.santa_decode_attention_value_sampled(kv2, q2, reps2, 65, 8)    # 65 x 256 > 16384
    with pytest.raises(RuntimeError):
        S.santa_decode_attention_value_sampled(kv2, q2, reps2, 8, 257)


# Full-size workloads in the benchmark's shapes: one whole (sequence, KV head)
# group per KV head is compared with the oracle; every head is checked for
# positions inside its drawn teams.
FULL = {
    "qwen7b_32k_b1_m31": [(0, h) for h in range(28)],
    "qwen7b_32k_b8_m32": [(b, h) for b, g in [(0, 0), (3, 1), (5, 2), (7, 3)] for h in range(7 * g, 7 * g + 7)],
    "mixture_128k_b4_t256_m64": [(b, h) for b, g in [(0, 0), (1, 1), (2, 2), (3, 3)]
                                 for h in range(7 * g, 7 * g + 7)],
}


@pytest.mark.parametrize("name", list(FULL))
def test_value_sampled_full_size(name):
    w = W.FULL_SIZE[name]()
    S_ = 64
    pairs = FULL[name]
    say(f"[value_sampled full] {name} B={w.batch} T={w.page_size} M={w.M} S={S_} heads={len(pairs)}")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    res = run_vs(w, kv, q, reps_gpu, S_)
    reps = parity.check_reps(w, reps_gpu, pairs)
    flips = compare(w, res, S_, pairs=pairs, reps=reps)
    say(f"  near-tie flips: {flips}")
    assert flips <= MAX_SAMPLE_FLIPS
    out, lse, teams, _, pos = res
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for h in range(w.num_q_heads):
            t = set(int(x) for x in teams[b, h] if x >= 0)
            assert all(0 <= x < L and x // w.page_size in t for x in pos[b, h])
    # The same draws, teams and log-sum-exp as the SANTA++ decode.
    o2, l2, t2, i2 = S.santa_decode_attention(kv, q, reps_gpu, w.M, w.seed, w.offset, return_sets=True)
    torch.cuda.synchronize()
    assert np.array_equal(teams, t2.cpu().numpy())
    assert np.allclose(lse, l2.cpu().numpy(), rtol=0, atol=parity.LSE_TOL[w.dtype] + 1e-6 * np.abs(lse).max())


def _random_configs(n=16, seed=4242):
    """Shapes drawn from one seed: cache type, head dim, team size, group
    size, batch, ragged lengths from one token, M (kept to at most 16384 drawn
    tokens per head), S from 1 to 256, both schemes."""
    rng = np.random.default_rng(seed)
    schemes = ["iid", "systematic", "stratified"]
    out = []
    for i in range(n):
        T = int(rng.choice([16, 32, 64, 128, 256]))
        hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 5, 7, 8, 16]))
        if rng.random() < 0.3:
            len_max, len_min = int(rng.integers(1, 2 * T + 1)), 1
        else:
            len_max = int(rng.integers(1, max(1, 5000 // T) + 1)) * T + int(rng.integers(0, T))
            len_min = int(rng.integers(1, len_max + 1))
        out.append(dict(name=f"v{i:02d}", dtype=str(rng.choice(["bf16", "f32"])), T=T, d=int(rng.choice([64, 128])),
                        hkv=hkv, hq=G * hkv, seqs=int(rng.integers(1, 6)), len_min=len_min, len_max=len_max,
                        M=int(rng.integers(1, min(80, 16384 // T) + 1)), S=int(rng.integers(1, 257)),
                        scheme=str(rng.choice(schemes)), value_scheme=str(rng.choice(schemes)),
                        data_seed=int(rng.integers(0, 2 ** 31)), philox_seed=int(rng.integers(0, 2 ** 63)),
                        offset=int(rng.integers(0, 2 ** 32))))
    return out


RANDOM = _random_configs()


@pytest.mark.parametrize("cfg", RANDOM, ids=[c["name"] for c in RANDOM])
def test_value_sampled_random_shapes(cfg):
    w = W.paged_ragged(data_seed=cfg["data_seed"], num_seqs=cfg["seqs"], len_min=cfg["len_min"],
                       len_max=cfg["len_max"], T=cfg["T"], M=cfg["M"], hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"],
                       dtype=cfg["dtype"], philox_seed=cfg["philox_seed"])
    w = W.dataclasses.replace(w, offset=cfg["offset"])
    say(f"[value_sampled random] {cfg}")
    kv, q = S.kv_from_workload(w)
    reps_gpu = S.santa_build_reps(kv)
    res = run_vs(w, kv, q, reps_gpu, cfg["S"], cfg["scheme"], cfg["value_scheme"])
    reps = parity.check_reps(w, reps_gpu)
    flips = compare(w, res, cfg["S"], scheme=cfg["scheme"], value_scheme=cfg["value_scheme"], reps=reps)
    assert flips <= max(MAX_SAMPLE_FLIPS, w.batch * w.num_q_heads // 50)


def test_value_samples_unbiased_given_the_teams():
    """Over many offsets (each call draws its teams and its value samples
    afresh), the value-sampled output minus SANTA++'s output for the same
    offset (the same teams: the team stream is shared) averages to zero
    within five standard errors, per element: given the teams, the value
    samples are unbiased for SANTA++'s estimate (the oracle pins show that
    the same check catches value samples drawn without the team weights)."""
    w = W.qwen_planted(batch=2, seq_len=4000 + 37, T=64, M=12, hq=8, hkv=2, d=128, plants=3)
    R, S_ = 2000, 16
    say(f"[value_sampled unbiased] {w.name} calls={R} S={S_}")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    vws, ws = S.make_value_sampled_workspace(kv, w.M), S.make_workspace(kv, w.M)
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    vout = torch.empty((R, B, Hq, d), dtype=torch.float32, device="cuda")
    sout = torch.empty((R, B, Hq, d), dtype=torch.float32, device="cuda")
    vteams = torch.empty((R, B, Hq, w.M), dtype=torch.int32, device="cuda")
    steams = torch.empty((R, B, Hq, w.M), dtype=torch.int32, device="cuda")
    vinv = torch.empty((B, Hq, w.M), dtype=torch.float32, device="cuda")
    sinv = torch.empty((B, Hq, w.M), dtype=torch.float32, device="cuda")
    for i in range(R):
        out, _, t, _ = S.santa_decode_attention_value_sampled(kv, q, reps, w.M, S_, seed=w.seed, offset=i,
                                                              workspace=vws, out=vout[i], return_sets=True)
        vteams[i].copy_(t)
        S.santa_select_teams(kv, q, reps, w.M, w.seed, i, ws, steams[i], sinv)
        S.santa_attend_selected(kv, q, w.M, ws, sout[i])
    torch.cuda.synchronize()
    assert torch.equal(vteams, steams)
    v, s = vout.double().cpu().numpy(), sout.double().cpu().numpy()

    def zmax(diff):
        se = diff.std(axis=0, ddof=1) / np.sqrt(diff.shape[0])
        return float(np.max(np.abs(diff.mean(axis=0)) / np.maximum(se, 1e-300)))

    z = zmax(v - s)
    say(f"  max |z| over {B * Hq * d} elements: {z:.2f}")
    assert z < 5.0


def test_value_sampled_graph_replays_match_eager():
    """The three launches captured in a HIP graph: every replay, with eager
    work between replays, reproduces the eager outputs and positions bit for
    bit."""
    w = W.qwen_mixed_query(batch=2, seq_len=8192, M=32)
    say(f"[value_sampled graph] {w.name}")
    kv, q = S.kv_from_workload(w)
    reps = S.santa_build_reps(kv)
    vws = S.make_value_sampled_workspace(kv, w.M)
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    teams = torch.empty((B, Hq, w.M), dtype=torch.int32, device="cuda")
    inv_pi = torch.empty((B, Hq, w.M), dtype=torch.float32, device="cuda")
    pos = torch.empty((B, Hq, 64), dtype=torch.int32, device="cuda")
    lib = S.load()

    def step():
        desc = kv.desc()
        st = lib.santa_decode_attention_value_sampled(
            S.ctypes.byref(desc), S._ptr(q), S._ptr(reps), w.M, 0, 64, 1, w.seed, 7, S._ptr(out), S._ptr(lse),
            S._ptr(teams), S._ptr(inv_pi), S._ptr(pos), S._ptr(vws), vws.numel(), S._stream())
        assert st == 0

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, teams, inv_pi, pos)]
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
        for t in (out, lse, inv_pi):
            t.fill_(float("nan"))
        teams.fill_(-7)
        pos.fill_(-7)
        S.santa_decode_attention_value_sampled(kv, q, reps, w.M, 64, offset=8 + r)     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, lse, teams, inv_pi, pos), ref):
            assert torch.equal(got, want), f"replay {r} differs from the eager result"

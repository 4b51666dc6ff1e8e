"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a published value, a library routine
that is not the one the oracle calls, a closed form, an exact enumeration or
an invariant, chosen so that a dropped term, a wrong sign, a wrong index or a
transposed operand in the oracle fails at least one of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import numerics, philox, santa
from sampled_sparse_decode_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# Philox4x32-10: published known-answer vectors
# --------------------------------------------------------------------------

def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((tuple(w[0:4]), tuple(w[4:6]), tuple(w[6:10])))
    return rows


@pytest.mark.parametrize("ctr,key,expected", _kat_rows())
def test_philox_known_answers(ctr, key, expected):
    assert philox.philox4x32_10(ctr, key) == expected


def test_philox_draw_layout_streams_differ():
    # Different heads, sequences and offsets read different counters.
    a = philox.draw_words(8, 0, 0, 0, 0)
    assert a != philox.draw_words(8, 0, 0, 0, 1)
    assert a != philox.draw_words(8, 0, 0, 1, 0)
    assert a != philox.draw_words(8, 0, 1, 0, 0)
    assert a != philox.draw_words(8, 1, 0, 0, 0)
    # Draw j is word j mod 4 of block j div 4.
    blk = philox.philox4x32_10((1, 3, 2, 5), (7, 0))
    assert philox.draw_words(8, 7, 5, 2, 3)[4:8] == list(blk)


def test_uniform_mapping_open_interval():
    assert philox.word_to_uniform(0) == 2.0 ** -33
    assert philox.word_to_uniform(0xFFFFFFFF) == 1.0 - 2.0 ** -33


# --------------------------------------------------------------------------
# bfloat16 decode and rounding against torch's conversions
# --------------------------------------------------------------------------

def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                 # no inf / nan
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(numerics.decode_bf16(bits), ref)


def test_bf16_round_matches_torch_on_binary32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # binary32 subnormals
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = numerics.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_round_is_one_step():
    # 1 + 2^-8 + 2^-40 is above the tie between 1 and 1 + 2^-7, so it rounds up;
    # rounding first to binary32 would land on the tie and go down to 1.
    assert numerics.round_to_bf16(1.0 + 2 ** -8 + 2 ** -40) == 1.0 + 2 ** -7
    assert numerics.round_to_bf16(1.0 + 2 ** -8) == 1.0                  # tie -> even
    assert numerics.round_to_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6     # tie -> even
    assert numerics.round_to_bf16(2.0 ** 128) == math.inf
    big = float.fromhex("0x1.fep127")
    assert numerics.round_to_bf16(big) == big


def _fraction_round_bf16(fr):
    """Independent exact rounding of a rational to bfloat16 (normal range)."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 128                      # 8 significant bits
    r = round(scaled)                     # Python rounds Fractions half to even
    return sign * float(Fraction(r, 128) * Fraction(2) ** e)


def test_reps_are_exact_rounded_means():
    rng = np.random.default_rng(2)
    T, d = 8, 16
    lens = [8 * 3 + 3]                    # a ragged last team of 3 tokens
    keys = rng.standard_normal((1, 1, lens[0], d)).astype(np.float32)
    w = wl._contiguous("t", "bf16", keys, keys, np.zeros((1, 1, d), np.float32), T, 4)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, T, "bf16")
    kd = numerics.decode_bf16(w.k_pages)
    for t in range(4):
        n = santa.team_size(lens[0], T, t)
        for c in range(d):
            exact = sum(Fraction(float(v)) for v in kd[t, 0, :n, c]) / n
            assert reps[0, t, 0, c] == _fraction_round_bf16(exact)


# --------------------------------------------------------------------------
# Dense attention and team scores against torch's attention routine
# --------------------------------------------------------------------------

def test_dense_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    for L, d in [(1, 8), (37, 64), (300, 128)]:
        q = rng.standard_normal(d)
        k = rng.standard_normal((L, d)) * 2
        v = rng.standard_normal((L, d))
        out, _ = santa.dense_attention(q, k, v)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None],
            torch.from_numpy(v)[None, None])[0, 0, 0].numpy()
        assert np.max(np.abs(out - ref)) < 1e-12


def test_dense_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(32)
    k = rng.standard_normal((50, 32)) * 3
    _, lse = santa.dense_attention(q, k, k)
    ref = torch.logsumexp(torch.from_numpy(k) @ torch.from_numpy(q) / math.sqrt(32), 0).item()
    assert abs(lse - ref) < 1e-12


def test_one_token_teams_give_attention_weights():
    # With one token per team the representative is the key itself, so the
    # team probabilities are the attention weights of the dense softmax.
    rng = np.random.default_rng(5)
    L, d = 40, 16
    keys = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    w = wl._contiguous("t", "f32", keys, keys, q, 1, 4)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, 1, "f32")
    qh = q[0, 0].astype(np.float64)
    s = santa.rep_scores(qh, np.stack([reps[0, t, 0] for t in range(L)]))
    _, _, _, p = santa.team_softmax(s)
    eye = torch.eye(L, dtype=torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qh)[None, None, None], torch.from_numpy(keys[0, 0].astype(np.float64))[None, None],
        eye[None, None])[0, 0, 0].numpy()
    assert np.max(np.abs(p - ref)) < 1e-14


# --------------------------------------------------------------------------
# Whole-pipeline special cases
# --------------------------------------------------------------------------

def _kv(w):
    return santa.PagedKV(w.dtype, w.k_pages, w.v_pages, w.page_table, w.seq_lens)


def test_full_coverage_equals_dense():
    w = wl.tiny_planted(n=200, d=32, T=16, M=13)    # 13 teams, M >= K
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    qh = numerics.decode(w.q[0, 0], w.dtype)
    r = santa.santa_head(kv, qh, reps, 0, 0, 1, w.M, 0, 0)
    assert r.selection.full and r.selection.teams == list(range(13))
    out, lse = santa.dense_head(kv, qh, 0, 0, 1)
    assert np.max(np.abs(r.out - out)) < 1e-12 and abs(r.lse - lse) < 1e-12


def test_constant_values_give_constant_output():
    w = wl.qwen_planted(batch=1, seq_len=1000, T=64, hq=4, hkv=2, d=64, plants=2, M=5, dtype="bf16")
    w.v_pages[:] = numerics.bf16_bits_of(np.array([1.5]))[0]
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    for h in range(4):
        r = santa.santa_head(kv, numerics.decode(w.q[0, h], "bf16"), reps, 0, h, 4, w.M, 7, 3)
        assert np.max(np.abs(r.out - 1.5)) < 1e-12


def test_permuted_page_table_same_result():
    w = wl.paged_ragged(num_seqs=3, len_min=500, len_max=2000, T=64, M=6, hq=4, hkv=2, d=64)
    rng = np.random.default_rng(9)
    perm = rng.permutation(w.num_pages)            # new physical position of each page
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    k2[perm] = w.k_pages
    v2[perm] = w.v_pages
    pt2 = perm[w.page_table].astype(np.int32)
    kv1, kv2 = _kv(w), santa.PagedKV(w.dtype, k2, v2, pt2, w.seq_lens)
    r1 = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    r2 = santa.build_reps(k2, pt2, w.seq_lens, w.page_size, w.dtype)
    for b in range(3):
        for h in range(4):
            qh = numerics.decode(w.q[b, h], w.dtype)
            a = santa.santa_head(kv1, qh, r1, b, h, 4, w.M, 1, 0)
            c = santa.santa_head(kv2, qh, r2, b, h, 4, w.M, 1, 0)
            assert a.selection.teams == c.selection.teams
            assert np.array_equal(a.out, c.out) and a.lse == c.lse


def test_empty_sequence():
    w = wl.paged_ragged(num_seqs=2, len_min=100, len_max=300, T=32, M=4, hq=2, hkv=1, d=64)
    w.seq_lens[1] = 0
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    r = santa.santa_head(kv, numerics.decode(w.q[1, 0], w.dtype), reps, 1, 0, 2, w.M, 0, 0)
    assert r.lse == -math.inf and np.all(r.out == 0)


# --------------------------------------------------------------------------
# Inverse CDF
# --------------------------------------------------------------------------

def test_inverse_cdf_uniform_mass_closed_form():
    K = 10
    e = np.ones(K)
    C = np.cumsum(e)
    for x in range(1, 1000):
        u = x / 1000 + 1e-7
        assert santa.inverse_cdf(u, e, C, C[-1]) == int(math.floor(u * K))


def test_inverse_cdf_never_picks_zero_mass():
    e = np.array([0.0, 1.0, 0.0, 0.0, 2.0, 0.0])
    C = np.cumsum(e)
    for u in np.linspace(1e-9, 1 - 1e-9, 997):
        assert santa.inverse_cdf(u, e, C, C[-1]) in (1, 4)


# Near-tie record. A draw whose point lies within 1e-6 of a boundary C_t / Z
# may land on another team in an implementation whose probabilities differ
# by less than that; the GPU parity tests accept set differences only inside
# the oracle's record, so the record is pinned here on cumulative sums whose
# boundaries are exact binary fractions.

def _near_tie_pin_failures(fn):
    """Failures of a near-tie detector fn(u, e, C, Z) -> set on hand-built
    cumulative sums (an empty list when it passes every pin)."""
    bad = []

    def check(name, u, e, want):
        e = np.asarray(e, dtype=np.float64)
        C = np.cumsum(e)
        got = set(fn(u, e, C, C[-1]))
        if got != set(want):
            bad.append((name, u, sorted(got), sorted(want)))

    e = [1.0, 2.0, 3.0, 2.0]                       # boundaries 1/8, 3/8, 3/4 (exact)
    for t, b in enumerate((0.125, 0.375, 0.75)):
        for du in (-5e-7, 5e-7, -9.5e-7, 9.5e-7):
            check(f"inside band at boundary {t}", b + du, e, {t, t + 1})
        for du in (-2e-6, 2e-6, -1.05e-6, 1.05e-6):
            check(f"outside band at boundary {t}", b + du, e, set())
    check("mid-team", 0.25, e, set())
    check("near 0", 5e-7, e, set())
    check("C_last / Z = 1 is not a boundary", 1.0 - 5e-7, e, set())
    check("C_last / Z = 1 is not a boundary (closer)", 1.0 - 2.0 ** -33, e, set())
    # zero-mass teams between two teams with mass: the boundary at 1/2 is
    # shared by teams 0, 1 and 2; the reachable teams are 0 and 3
    for du in (-5e-7, 5e-7):
        check("zero-mass neighbours", 0.5 + du, [1.0, 0.0, 0.0, 1.0], {0, 3})
    check("zero-mass neighbours, outside band", 0.5 + 3e-6, [1.0, 0.0, 0.0, 1.0], set())
    # a team narrower than the band: all three teams reachable
    check("narrow middle team", 0.5 + 2.0 ** -22, [2.0 ** 20, 1.0, 2.0 ** 20 - 1], {0, 1, 2})
    return bad


def test_near_tie_record_pins():
    assert _near_tie_pin_failures(santa.near_tie_teams_of_draw) == []


def _old_argmin_detector(u, e, C, Z):
    # the earlier record: nearest interior boundary k by argmin, teams (k, k + 1)
    if santa.draw_distance_to_boundary(u, C, Z) < santa.NEAR_TIE:
        k = int(np.argmin(np.abs(u - C[:-1] / Z)))
        return {k, k + 1}
    return set()


def _with_last_boundary(u, e, C, Z):
    # treats C_last / Z = 1 as a boundary a draw could cross
    r = set(santa.near_tie_teams_of_draw(u, e, C, Z))
    if abs(u - 1.0) < santa.NEAR_TIE:
        r |= {len(C) - 1, len(C)}
    return r


@pytest.mark.parametrize("mutant", [
    lambda u, e, C, Z: santa.near_tie_teams_of_draw(u, e, C, Z, band=santa.NEAR_TIE * 1000),   # threshold x 1000
    lambda u, e, C, Z: santa.near_tie_teams_of_draw(u, e, C, Z, band=santa.NEAR_TIE / 1000),   # threshold / 1000
    lambda u, e, C, Z: {t + 1 for t in santa.near_tie_teams_of_draw(u, e, C, Z)},            # teams off by one
    lambda u, e, C, Z: {t - 1 for t in santa.near_tie_teams_of_draw(u, e, C, Z)},
    _old_argmin_detector,
    _with_last_boundary,
], ids=["band_x1000", "band_div1000", "plus_one", "minus_one", "argmin_pair", "last_boundary"])
def test_near_tie_pins_catch_planted_mistakes(mutant):
    assert _near_tie_pin_failures(mutant) != []


def test_select_teams_records_near_tie_draws(monkeypatch):
    # Scores chosen so the team softmax has boundaries near 1/8, 3/8, 3/4; the
    # draw points are placed by hand beside the second boundary.
    s = np.log(np.array([1.0, 2.0, 3.0, 2.0]))
    rep_rows = np.diag(np.ones(4)) * 0.0
    e, C, Z, p = santa.team_softmax(s)
    b1 = C[1] / Z
    pts = [b1 - 4e-7, 0.9, b1 + 3e-6]
    monkeypatch.setattr(santa, "draw_uniforms", lambda scheme, M, seed, offset, b, h: pts)
    monkeypatch.setattr(santa, "rep_scores", lambda q_h, rows: s)
    sel = santa.select_teams(np.zeros(4), rep_rows, 3, 0, 0, 0, 0)
    assert sel.draws == [1, 3, 2]
    assert sel.near_tie_teams == {1, 2}


def test_draw_frequencies_chi_square():
    from scipy.stats import chisquare
    rng = np.random.default_rng(11)
    s = rng.standard_normal(24)
    e, C, Z, p = santa.team_softmax(s)
    counts = np.zeros(24)
    for seed in range(300):
        for x in philox.draw_words(64, seed, 0, 0, 0):
            counts[santa.inverse_cdf(philox.word_to_uniform(x), e, C, Z)] += 1
    assert chisquare(counts, p * counts.sum()).pvalue > 1e-3


# --------------------------------------------------------------------------
# Horvitz-Thompson sums: exact enumeration on tiny inputs
# --------------------------------------------------------------------------

def _tiny_five_teams(seed):
    rng = np.random.default_rng(seed)
    d, T, L = 8, 4, 19                       # teams of 4,4,4,4,3 tokens
    keys = (rng.standard_normal((1, 1, L, d)) * 1.5).astype(np.float32)
    vals = rng.standard_normal((1, 1, L, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    return wl._contiguous("five", "f32", keys, vals, q, T, 1)


@pytest.mark.parametrize("M", [1, 2, 3])
def test_ht_sums_unbiased_by_enumeration(M):
    w = _tiny_five_teams(12 + M)
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    qh = numerics.decode(w.q[0, 0], "f32")
    K = 5
    s = santa.rep_scores(qh, np.stack([reps[0, t, 0] for t in range(K)]))
    _, _, _, p = santa.team_softmax(s)
    teams = [kv.team(0, 0, t) for t in range(K)]
    keys, vals = kv.all_tokens(0, 0)
    a = np.exp(santa.token_scores(qh, keys))
    N_exact, D_exact = a @ vals, a.sum()
    EN, ED = np.zeros(w.head_dim), 0.0
    incl = np.zeros(K)
    for seq in itertools.product(range(K), repeat=M):
        prob = float(np.prod([p[t] for t in seq]))
        S = sorted(set(seq))
        wts = [1.0 / santa.inclusion_probability(p[t], M) for t in S]
        n, dd = santa.ht_sums(qh, [teams[t] for t in S], wts, 0.0)
        EN += prob * n
        ED += prob * dd
        for t in S:
            incl[t] += prob
    assert abs(ED - D_exact) < 1e-12 * abs(D_exact)
    assert np.max(np.abs(EN - N_exact)) < 1e-12 * np.max(np.abs(N_exact))
    for t in range(K):
        assert abs(incl[t] - santa.inclusion_probability(p[t], M)) < 1e-14


# --------------------------------------------------------------------------
# Monte Carlo over Philox seeds: convergence and closed-form set size
# --------------------------------------------------------------------------

def test_monte_carlo_converges_and_set_size_closed_form():
    w = wl.tiny_planted(n=512, d=32, T=32, M=6)
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    qh = numerics.decode(w.q[0, 0], "f32")
    keys, vals = kv.all_tokens(0, 0)
    out_d, lse_d = santa.dense_attention(qh, keys, vals)
    R = 3000
    Dr = np.empty(R)
    Nr = np.empty((R, w.head_dim))
    sizes = np.empty(R)
    for seed in range(R):
        r = santa.santa_head(kv, qh, reps, 0, 0, 1, w.M, seed, 0)
        Dr[seed] = math.exp(r.lse - lse_d)           # estimated D / exact D
        Nr[seed] = r.out * Dr[seed]                  # estimated N / exact D
        sizes[seed] = len(r.selection.teams)
    se = Dr.std() / math.sqrt(R)
    assert abs(Dr.mean() - 1.0) < 5 * se + 1e-12
    seN = Nr.std(axis=0) / math.sqrt(R)
    assert np.all(np.abs(Nr.mean(axis=0) - out_d) < 5 * seN + 1e-12)
    # The ratio of the means converges to the dense output.
    assert np.max(np.abs(Nr.mean(axis=0) / Dr.mean() - out_d)) < 10 * np.max(seN) / Dr.mean()
    # Expected number of distinct teams: sum of inclusion probabilities.
    K = santa.num_teams(int(w.seq_lens[0]), w.page_size)
    s = santa.rep_scores(qh, np.stack([reps[0, t, 0] for t in range(K)]))
    _, _, _, p = santa.team_softmax(s)
    assert abs(sizes.mean() - santa.expected_set_size(p, w.M)) < 5 * sizes.std() / math.sqrt(R)


def test_union_size_closed_form():
    rng = np.random.default_rng(21)
    K, M, G = 40, 5, 3
    ps = [santa.team_softmax(rng.standard_normal(K))[3] for _ in range(G)]
    R = 4000
    sizes = np.empty(R)
    for r in range(R):
        u = set()
        for h in range(G):
            e, C, Z = ps[h], np.cumsum(ps[h]), np.cumsum(ps[h])[-1]
            for x in philox.draw_words(M, r, 0, 0, h):
                u.add(santa.inverse_cdf(philox.word_to_uniform(x), e, C, Z))
        sizes[r] = len(u)
    assert abs(sizes.mean() - santa.expected_union_size(ps, M)) < 5 * sizes.std() / math.sqrt(R)


# --------------------------------------------------------------------------
# Alternative representatives: medoid and random member (reading R9)
# --------------------------------------------------------------------------

def test_medoid_of_collinear_keys_is_the_median():
    # Points x_i * u on one line: the sum of distances |x_i - x_j| ||u|| is
    # smallest at the median of the x_i (odd count: unique).
    rng = np.random.default_rng(40)
    u = np.zeros(32)
    u[[0, 5, 17]] = [1.0, -2.0, 0.5]
    for n in (3, 5, 9, 31):
        x = rng.permutation(np.arange(n) * 3 - 20).astype(np.float64)
        x[:] = x + rng.integers(0, 2, n)                     # uneven gaps, still distinct
        keys = x[:, None] * u[None, :]
        assert santa.team_medoid_index(keys) == int(np.argsort(x)[n // 2])
    # Skewed: the median (member 4, x = 2) is not the point nearest the mean
    # (member 0, x = 50), which summed squared distances would pick.
    x = np.array([50.0, 100.0, 0.0, 1.0, 2.0])
    assert santa.team_medoid_index(x[:, None] * u[None, :]) == 4


def test_medoid_matches_scipy_distance_sums():
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(41)
    for n, d in ((16, 64), (37, 128), (128, 64)):
        keys = numerics.round_to_dtype(rng.standard_normal((n, d)) * 2.0, "bf16")
        sums = cdist(keys, keys).sum(axis=1)
        order = np.argsort(sums)
        assert sums[order[1]] - sums[order[0]] > 1e-9 * sums[order[0]]   # no near tie in this sample
        assert santa.team_medoid_index(keys) == int(order[0])


def test_medoid_ties_go_to_the_lowest_index():
    rng = np.random.default_rng(42)
    k = rng.standard_normal((1, 16))
    assert santa.team_medoid_index(np.repeat(k, 6, axis=0)) == 0             # all equal
    assert santa.team_medoid_index(rng.standard_normal((2, 16))) == 0       # two keys: equal sums
    assert santa.team_medoid_index(k) == 0                                  # a team of one
    # The median point of a line, present twice (members 2 and 4): both have
    # the smallest sum, member 2 is taken.
    x = np.array([5.0, -3.0, 1.0, 9.0, 1.0, -7.0, 4.0])
    assert santa.team_medoid_index(x[:, None] * np.ones((1, 8))) == 2


def test_medoid_ignores_translation_and_never_takes_an_outlier():
    rng = np.random.default_rng(43)
    keys = np.round(rng.standard_normal((12, 16)) * 8)                       # small integers: exact
    i = santa.team_medoid_index(keys)
    assert santa.team_medoid_index(keys + 64.0) == i
    far = keys.copy()
    far[5] += 1e4
    assert santa.team_medoid_index(far) != 5


def test_random_member_is_uniform_and_in_range():
    # Over many teams the chosen member of a team of n is uniform on 0..n-1.
    from scipy.stats import chisquare
    for n in (16, 5, 1):
        idx = np.array([santa.team_random_index(n, 99, b, t, g)
                        for b in range(4) for t in range(256) for g in range(4)])
        assert idx.min() >= 0 and idx.max() < n
        if n > 1:
            counts = np.bincount(idx, minlength=n)
            assert chisquare(counts).pvalue > 1e-4
    # Its stream is not the draws': for one (b, team = draw block) the words differ.
    assert [santa.team_random_index(2 ** 16, 7, 0, t, 0) for t in range(4)] != \
        [(philox.philox4x32_10((t, 0, 0, 0), (7, 0))[0] * 2 ** 16) >> 32 for t in range(4)]


def test_build_reps_kind_rows_are_team_members():
    w = wl.paged_ragged(num_seqs=3, len_min=40, len_max=150, T=16, M=4, hq=4, hkv=2, d=32, dtype="bf16")
    mean = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    assert np.array_equal(santa.build_reps_kind(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype,
                                                santa.REP_MEAN), mean, equal_nan=True)
    kd = numerics.decode(w.k_pages, w.dtype)
    for kind in (santa.REP_MEDOID, santa.REP_RANDOM):
        reps = santa.build_reps_kind(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype, kind, seed=3)
        for b in range(w.batch):
            L = int(w.seq_lens[b])
            for t in range(santa.num_teams(L, w.page_size)):
                n = santa.team_size(L, w.page_size, t)
                tile = kd[int(w.page_table[b][t])]
                for g in range(w.num_kv_heads):
                    hits = np.all(tile[g, :n] == reps[b, t, g][None, :], axis=1)
                    assert hits.any(), (kind, b, t, g)
            assert np.all(np.isnan(reps[b, santa.num_teams(L, w.page_size):]))


# --------------------------------------------------------------------------
# Variance-reduced team draws: systematic and stratified (reading R10)
# --------------------------------------------------------------------------

def _team_probs(K, seed, spread=1.5):
    s = list(np.random.default_rng(seed).standard_normal(K) * spread)
    return santa.team_softmax(s)


def test_scheme_points_layout():
    for M in (1, 5, 31):
        iid = santa.draw_uniforms(santa.DRAW_IID, M, 7, 3, 1, 2)
        sys_ = santa.draw_uniforms(santa.DRAW_SYSTEMATIC, M, 7, 3, 1, 2)
        strat = santa.draw_uniforms(santa.DRAW_STRATIFIED, M, 7, 3, 1, 2)
        assert 0 < sys_[0] < 1 / M
        assert np.allclose(np.diff(sys_), 1 / M, rtol=0, atol=1e-15)     # one unit apart
        assert abs(sys_[0] * M - iid[0]) < 1e-15
        for j in range(M):
            assert j / M < strat[j] < (j + 1) / M                      # one point per unit
            assert abs(strat[j] * M - j - iid[j]) < 1e-13


def _pieces(breaks):
    b = sorted(set([0.0, 1.0] + [x for x in breaks if 0.0 < x < 1.0]))
    return zip(b[:-1], b[1:])


def test_systematic_inclusion_by_exact_integration():
    # With one uniform u0 the drawn set is piecewise constant in u0, changing
    # only where a point (j + u0)/M crosses a boundary C_t/Z. Integrating the
    # selection rule itself over the pieces gives P(t in S) exactly; it must
    # equal min(1, M p_t), and the weighted team sums must be unbiased.
    for K, M, seed in ((40, 8, 1), (17, 5, 2), (64, 31, 3)):
        e, C, Z, p = _team_probs(K, seed)
        X = np.random.default_rng(seed + 10).standard_normal(K)
        pi = np.array([santa.inclusion_probability_scheme(santa.DRAW_SYSTEMATIC, t, C, Z, p, M)
                       for t in range(K)])
        incl = np.zeros(K)
        ht = 0.0
        for lo, hi in _pieces([(M * c / Z) % 1.0 for c in C]):
            S = {santa.inverse_cdf((j + (lo + hi) / 2) / M, e, C, Z) for j in range(M)}
            for t in S:
                incl[t] += hi - lo
                ht += (hi - lo) * X[t] / pi[t]
        assert np.max(np.abs(incl - pi)) < 1e-12
        assert abs(ht - X.sum()) < 1e-10 * np.abs(X).sum()
        assert np.any((pi > 0.3) & (pi < 1.0)) and np.any(pi == 1.0)  # both regimes occur


def test_stratified_inclusion_by_exact_integration():
    # Stratum j's point is uniform on [j/M, (j+1)/M) and independent of the
    # others: P(point j in t) is the measure of the piece of the stratum the
    # selection rule sends to t, and P(t in S) = 1 - prod_j (1 - that).
    for K, M, seed in ((40, 8, 4), (17, 5, 5), (64, 31, 6), (6, 4, 7)):
        e, C, Z, p = _team_probs(K, seed)
        hit = np.zeros((M, K))
        for j in range(M):
            for lo, hi in _pieces([M * c / Z - j for c in C]):
                hit[j, santa.inverse_cdf((j + (lo + hi) / 2) / M, e, C, Z)] += hi - lo
        brute = 1.0 - np.prod(1.0 - hit, axis=0)
        pi = np.array([santa.inclusion_probability_scheme(santa.DRAW_STRATIFIED, t, C, Z, p, M)
                       for t in range(K)])
        assert np.max(np.abs(brute - pi)) < 1e-12
        # It is neither the independent nor the systematic probability.
        iid = np.array([santa.inclusion_probability(x, M) for x in p])
        assert np.max(np.abs(pi - iid)) > 1e-3 and np.max(np.abs(pi - np.minimum(1, M * p))) > 1e-3


def test_stratified_inclusion_of_tiny_teams_is_accurate():
    # A team far narrower than a unit: pi = M p to full relative precision.
    s = [0.0] * 10 + [-40.0] + [0.0] * 10
    e, C, Z, p = santa.team_softmax(s)
    for scheme in (santa.DRAW_SYSTEMATIC, santa.DRAW_STRATIFIED):
        pi = santa.inclusion_probability_scheme(scheme, 10, C, Z, p, 7)
        assert abs(pi / (7 * p[10]) - 1.0) < 1e-9


def test_systematic_uniform_teams_draw_exactly_m():
    # Equal team probabilities 1/K < 1/M: the points are one unit apart and
    # every team is narrower than a unit, so M distinct teams every time.
    K, M = 50, 12
    e, C, Z, p = santa.team_softmax([0.0] * K)
    for seed in range(50):
        u = santa.draw_uniforms(santa.DRAW_SYSTEMATIC, M, seed, 0, 0, 0)
        assert len({santa.inverse_cdf(x, e, C, Z) for x in u}) == M


def test_variance_reduced_schemes_lower_the_error():
    # Teams of keys around their own centre (so the representatives are
    # informative, p close to each team's share of the softmax mass); many
    # seeds: every scheme is unbiased in the denominator, and the systematic
    # and stratified ones spread it, and the output error, clearly less than
    # independent draws.
    K, d, T, M = 32, 32, 16, 8
    rng = np.random.default_rng(9)
    mu = rng.standard_normal((K, d))
    keys = (np.repeat(mu, T, axis=0) + 0.3 * rng.standard_normal((K * T, d))).astype(np.float32)[None, None]
    vals = rng.standard_normal((1, 1, K * T, d)).astype(np.float32)
    q = (2.0 * rng.standard_normal((1, 1, d))).astype(np.float32)
    w = wl._contiguous("coherent_teams", "f32", keys, vals, q, T, M)
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    qh = numerics.decode(w.q[0, 0], "f32")
    out_d, lse_d = santa.dense_attention(qh, *kv.all_tokens(0, 0))
    R = 600
    sd, mse = {}, {}
    for scheme in (santa.DRAW_IID, santa.DRAW_SYSTEMATIC, santa.DRAW_STRATIFIED):
        Dr = np.empty(R)
        err = np.empty(R)
        for seed in range(R):
            r = santa.santa_head(kv, qh, reps, 0, 0, 1, M, seed, 0, scheme)
            Dr[seed] = math.exp(r.lse - lse_d)
            err[seed] = np.sum((r.out - out_d) ** 2)
        assert abs(Dr.mean() - 1.0) < 5 * Dr.std() / math.sqrt(R) + 1e-12
        sd[scheme], mse[scheme] = Dr.std(), err.mean()
    for scheme in (santa.DRAW_SYSTEMATIC, santa.DRAW_STRATIFIED):
        assert sd[scheme] < 0.6 * sd[santa.DRAW_IID]
        assert mse[scheme] < 0.75 * mse[santa.DRAW_IID]


# --------------------------------------------------------------------------
# Hash-partitioned teams (reading R11)
# --------------------------------------------------------------------------

def test_hash_code_bits_follow_the_direction_order():
    # Directions = the first basis vectors: bit j (most significant first) is
    # the sign of channel j.
    rng = np.random.default_rng(50)
    bits, d = 5, 16
    dirs = np.eye(d)[:bits]
    keys = rng.standard_normal((200, d))
    expect = np.zeros(200, dtype=np.int64)
    for j in range(bits):
        expect += (keys[:, j] > 0).astype(np.int64) << (bits - 1 - j)
    assert np.array_equal(santa.hash_codes(keys, dirs), expect)
    assert np.array_equal(santa.hash_codes(-keys, dirs), (2 ** bits - 1) - expect)   # no exact zeros here


def test_hash_codes_match_exact_rational_signs():
    rng = np.random.default_rng(51)
    keys = numerics.round_to_dtype(rng.standard_normal((60, 24)), "bf16")
    dirs = rng.standard_normal((6, 24)).astype(np.float32).astype(np.float64)
    codes = santa.hash_codes(keys, dirs)
    for i in range(60):
        c = 0
        for j in range(6):
            exact = sum(Fraction(float(a)) * Fraction(float(r)) for a, r in zip(keys[i], dirs[j]))
            c = 2 * c + (1 if exact > 0 else 0)
        assert codes[i] == c


def test_hash_order_is_a_stable_sort_that_groups_clusters():
    rng = np.random.default_rng(54)
    d, bits = 32, 6
    dirs = rng.standard_normal((bits, d))
    centres = rng.standard_normal((4, d)) * 4.0
    label = rng.integers(0, 4, 400)
    keys = centres[label] + 0.05 * rng.standard_normal((400, d))
    order = santa.hash_partition_order(keys, dirs)
    codes = santa.hash_codes(keys, dirs)
    assert sorted(order.tolist()) == list(range(400))
    assert np.all(np.diff(codes[order]) >= 0)
    for c in set(codes.tolist()):                       # equal codes keep token order
        pos = order[codes[order] == c]
        assert np.all(np.diff(pos) > 0)
    # With these inputs every cluster has one code of its own (no direction
    # cuts a cluster), so each cluster is one run of the order.
    per = [set(codes[label == c].tolist()) for c in range(4)]
    assert all(len(x) == 1 for x in per) and len(set.union(*per)) == 4
    assert 1 + np.count_nonzero(np.diff(label[order])) == 4


def test_cluster_pages_is_a_per_head_permutation_that_keeps_dense_attention():
    w = wl.paged_ragged(num_seqs=3, len_min=200, len_max=900, T=32, M=8, hq=4, hkv=2, d=32, dtype="bf16")
    dirs = wl.hash_directions(hkv=2, bits=5, d=32)
    k2, v2, codes, tok = santa.cluster_pages(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size,
                                             w.dtype, dirs)
    kv0, kv1 = _kv(w), santa.PagedKV(w.dtype, k2, v2, w.page_table, w.seq_lens)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for g in range(2):
            k0, v0 = kv0.all_tokens(b, g)
            k1, v1 = kv1.all_tokens(b, g)
            order = tok[b, g, :L]
            assert np.array_equal(k1, k0[order]) and np.array_equal(v1, v0[order])
            assert np.all(tok[b, g, L:] == -1) and np.all(codes[b, g, L:] == -1)
            assert np.array_equal(codes[b, g, :L], santa.hash_codes(k0, dirs[g]))
        for h in range(4):
            qh = numerics.decode(w.q[b, h], w.dtype)
            o0, l0 = santa.dense_head(kv0, qh, b, h, 4)
            o1, l1 = santa.dense_head(kv1, qh, b, h, 4)
            assert np.max(np.abs(o0 - o1)) < 1e-12 and abs(l0 - l1) < 1e-12


def test_hash_teams_lower_the_error_on_planted_tokens():
    # A few keys aligned with each query hide among random keys: contiguous
    # teams dilute them, hash teams gather them, so their representatives
    # carry the signal and the estimate is far closer to dense attention.
    w = wl.qwen_planted(batch=1, seq_len=4096, T=32, M=16, hq=4, hkv=1, d=64, plants=8)
    dirs = wl.hash_directions(hkv=1, bits=7, d=64)
    k2, v2, _, _ = santa.cluster_pages(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size, w.dtype,
                                       dirs)
    mse = {}
    for name, ww in (("contiguous", w), ("hashed", wl.permuted_workload(w, k2, v2))):
        kv = _kv(ww)
        reps = santa.build_reps(ww.k_pages, ww.page_table, ww.seq_lens, ww.page_size, ww.dtype)
        err = []
        for h in range(4):
            qh = numerics.decode(ww.q[0, h], ww.dtype)
            out_d, _ = santa.dense_attention(qh, *kv.all_tokens(0, 0))
            for seed in range(60):
                r = santa.santa_head(kv, qh, reps, 0, h, 4, ww.M, seed, 0)
                err.append(np.sum((r.out - out_d) ** 2))
        mse[name] = np.mean(err)
    assert mse["hashed"] < 0.5 * mse["contiguous"]


# --------------------------------------------------------------------------
# k-means-partitioned teams (reading R12)
# --------------------------------------------------------------------------

def test_kmeans_matches_scikit_learn_lloyd():
    # Same start (the keys of tokens floor(c L / C)), iters assignments with
    # iters - 1 centroid moves in between: scikit-learn's Lloyd k-means with
    # max_iter = iters - 1 ends with the same labels (its final E-step makes
    # them consistent with the last centres). Data without near ties.
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(60)
    for L, d, C, iters in ((600, 16, 6, 4), (900, 32, 12, 3), (256, 8, 4, 6)):
        centres = rng.standard_normal((C, d)) * 3.0
        x = centres[rng.integers(0, C, L)] + rng.standard_normal((L, d))
        init = x[[(c * L) // C for c in range(C)]]
        km = KMeans(n_clusters=C, init=init, n_init=1, max_iter=iters - 1, algorithm="lloyd", tol=0.0).fit(x)
        assert np.array_equal(santa.kmeans_codes(x, C, iters), km.labels_)


def test_kmeans_recovers_separated_runs():
    # C runs of equal length, far apart: the evenly spaced start puts one
    # centroid in each run, and every token keeps its run's label.
    rng = np.random.default_rng(61)
    C, n, d = 5, 40, 16
    centres = rng.standard_normal((C, d)) * 20.0
    x = np.repeat(centres, n, axis=0) + 0.1 * rng.standard_normal((C * n, d))
    assert np.array_equal(santa.kmeans_codes(x, C, 3), np.repeat(np.arange(C), n))


def test_kmeans_objective_never_rises_and_ties_go_low():
    rng = np.random.default_rng(62)
    x = rng.standard_normal((500, 12))
    C = 7
    costs = []
    for iters in range(1, 7):
        a = santa.kmeans_codes(x, C, iters)
        mu = np.array([x[a == c].mean(axis=0) if np.any(a == c) else np.zeros(12) for c in range(C)])
        costs.append(float(np.sum((x - mu[a]) ** 2)))
    assert all(costs[i + 1] <= costs[i] + 1e-9 for i in range(len(costs) - 1))
    # Two identical starting centroids (centroids come from tokens 0, 2, 4,
    # 6, 8; tokens 0 and 2 are made equal): cluster 1 always ties with
    # cluster 0 and is never chosen.
    y = x[:10].copy()
    y[2] = y[0]
    a = santa.kmeans_codes(y, 5, 1)
    assert not np.any(a == 1) and a[2] == 0


def test_cluster_pages_kmeans_is_a_permutation_that_keeps_dense_attention():
    w = wl.gaussian_mixture(batch=2, seq_len=700, T=32, M=8, hq=4, hkv=2, d=32, components=6, run_min=1,
                            run_max=12)
    k2, v2, codes, tok = santa.cluster_pages_kmeans(w.k_pages, w.v_pages, w.page_table, w.seq_lens, w.page_size,
                                                    w.dtype, None, 3)
    kv0, kv1 = _kv(w), santa.PagedKV(w.dtype, k2, v2, w.page_table, w.seq_lens)
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        for g in range(2):
            k0, v0 = kv0.all_tokens(b, g)
            k1, v1 = kv1.all_tokens(b, g)
            order = tok[b, g, :L]
            assert np.array_equal(k1, k0[order]) and np.array_equal(v1, v0[order])
            assert np.all(np.diff(codes[b, g, order]) >= 0)
        for h in range(4):
            qh = numerics.decode(w.q[b, h], w.dtype)
            o0, l0 = santa.dense_head(kv0, qh, b, h, 4)
            o1, l1 = santa.dense_head(kv1, qh, b, h, 4)
            assert np.max(np.abs(o0 - o1)) < 1e-12 and abs(l0 - l1) < 1e-12


# --------------------------------------------------------------------------
# Value samples inside the drawn teams (readings R13-R14)
# --------------------------------------------------------------------------

def _value_case(M=5, n=700, T=32):
    w = wl.tiny_planted(n=n, d=32, T=T, M=M)
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    return w, kv, reps, numerics.decode(w.q[0, 0], "f32")


def _conditional_means(fn, R=3000, S=8):
    """Mean over R independent value-point sets of fn's output with the team
    draws held fixed (seed 5, offset 3): the points come from numpy, not
    Philox, through the oracle's own inverse CDF."""
    w, kv, reps, qh = _value_case()
    rng = np.random.default_rng(17)
    orig = santa.value_uniforms
    outs = np.empty((R, w.head_dim))
    try:
        for r in range(R):
            pts = list(rng.random(S))
            santa.value_uniforms = lambda *a, **k: pts
            outs[r] = fn(kv, qh, reps, 0, 0, 1, w.M, S, 5, 3).out
    finally:
        santa.value_uniforms = orig
    ref = santa.santa_head(kv, qh, reps, 0, 0, 1, w.M, 5, 3)
    return outs, ref


def test_value_samples_average_to_the_santa_estimate_of_the_same_teams():
    # Given the drawn teams, the mean of the sampled values is unbiased for
    # the weighted value sum: averaging over many independent point sets
    # lands on santa_head's estimate (a separate code path: weights multiply
    # exp(s - shift) there, they shift the logits here).
    outs, ref = _conditional_means(santa.value_sampled_head)
    se = outs.std(axis=0) / math.sqrt(len(outs))
    assert np.all(np.abs(outs.mean(axis=0) - ref.out) < 5 * se + 1e-12)
    # and the log-sum-exp is that of the drawn tokens
    w, kv, reps, qh = _value_case()
    r = santa.value_sampled_head(kv, qh, reps, 0, 0, 1, w.M, 8, 5, 3)
    assert abs(r.lse - ref.lse) < 1e-12 * max(1.0, abs(ref.lse))
    assert r.selection.teams == ref.selection.teams


def _without_weights(kv, q_h, reps, b, h, Hq, M, S, seed, offset):
    # planted mistake: the logits without log w
    r = santa.value_sampled_head(kv, q_h, reps, b, h, Hq, M, S, seed, offset)
    g = 0
    logits, vals = [], []
    for t in r.selection.teams:
        keys, v = kv.team(b, g, t)
        logits.append(santa.token_scores(q_h, keys))
        vals.append(v)
    logits, vals = np.concatenate(logits), np.concatenate(vals)
    e, C, Z, _ = santa.team_softmax(logits)
    picks = [santa.inverse_cdf(u, e, C, Z) for u in santa.value_uniforms(0, S, seed, offset, b, h)]
    r.out = np.mean(vals[picks], axis=0)
    return r


def test_value_sample_pin_catches_dropped_weights():
    outs, ref = _conditional_means(_without_weights)
    se = outs.std(axis=0) / math.sqrt(len(outs))
    assert np.any(np.abs(outs.mean(axis=0) - ref.out) >= 5 * se + 1e-12)


def test_value_samples_under_full_coverage_average_to_dense_attention():
    # Every team read (M >= K, w = 1): the samples come from the exact
    # attention weights, so their mean over many offsets is dense attention.
    w, kv, reps, qh = _value_case(M=64, n=300, T=32)
    keys, vals = kv.all_tokens(0, 0)
    out_d, lse_d = santa.dense_attention(qh, keys, vals)
    R, S = 3000, 4
    outs = np.stack([santa.value_sampled_head(kv, qh, reps, 0, 0, 1, w.M, S, 9, off).out for off in range(R)])
    se = outs.std(axis=0) / math.sqrt(R)
    assert np.all(np.abs(outs.mean(axis=0) - out_d) < 5 * se + 1e-12)
    r = santa.value_sampled_head(kv, qh, reps, 0, 0, 1, w.M, S, 9, 0)
    assert abs(r.lse - lse_d) < 1e-12 * max(1.0, abs(lse_d))


def test_systematic_value_samples_follow_the_token_probabilities():
    # One point per unit of width 1/S: token j is sampled floor(S p_j) or
    # ceil(S p_j) times.
    w, kv, reps, qh = _value_case()
    S = 64
    r = santa.value_sampled_head(kv, qh, reps, 0, 0, 1, w.M, S, 5, 3, value_scheme=santa.DRAW_SYSTEMATIC)
    p = np.exp(r.logits - r.logits.max())
    p /= p.sum()
    pos = []
    for t in r.selection.teams:
        n = santa.team_size(int(w.seq_lens[0]), w.page_size, t)
        pos.extend(t * w.page_size + j for j in range(n))
    counts = np.array([r.positions.count(x) for x in pos])
    assert counts.sum() == S
    assert np.all(counts >= np.floor(S * p - 1e-9)) and np.all(counts <= np.ceil(S * p + 1e-9))


def test_value_samples_of_a_one_token_sequence():
    import dataclasses
    w = dataclasses.replace(wl.tiny_planted(n=64, d=32, T=32, M=4), seq_lens=np.array([1], dtype=np.int32))
    kv = _kv(w)
    reps = santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
    qh = numerics.decode(w.q[0, 0], "f32")
    r = santa.value_sampled_head(kv, qh, reps, 0, 0, 1, w.M, 5, 1, 0)
    keys, vals = kv.all_tokens(0, 0)
    assert r.positions == [0] * 5
    assert np.array_equal(r.out, vals[0])
    assert r.lse == pytest.approx(float(santa.token_scores(qh, keys)[0]), abs=1e-12)


def test_value_stream_differs_from_the_team_stream():
    for scheme in (santa.DRAW_IID, santa.DRAW_SYSTEMATIC, santa.DRAW_STRATIFIED):
        a = santa.value_uniforms(scheme, 16, 7, 2, 1, 3)
        b = santa.draw_uniforms(scheme, 16, 7, 2, 1, 3)
        assert all(0.0 < x < 1.0 for x in a) and len(set(a) & set(b)) == 0

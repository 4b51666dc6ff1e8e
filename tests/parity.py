"""Shared comparison logic of the GPU parity tests: run the CPU oracle on the
same seeded inputs and compare the HIP results with it, head by head.

Tolerances (max-abs over every output element): 4e-3 for a bfloat16 cache
with float32 accumulation, 1e-5 for a float32 cache. Team sets must match
exactly, except that a draw whose uniform lies within 1e-6 of a CDF boundary
(a near-tie, flagged by the oracle) may land on another team it can reach;
then the HIP output is compared with the oracle's estimate on the HIP set.

The log-sum-exp is a float32 output with no tolerance of its own in the
method's statement: it is held to the output tolerance plus four float32
roundings of its own magnitude (the shift, the sum of exponentials, the
logarithm and the final add each round once), i.e. OUT_TOL + 4 * 2^-24 * |lse|.
"""
import math

import numpy as np

from oracle import numerics, santa

OUT_TOL = {"bf16": 4e-3, "f32": 1e-5}
LSE_TOL = {"bf16": 4e-3, "f32": 1e-5}
LSE_RTOL = 4 * 2.0 ** -24
INV_PI_RTOL = 1e-6
MAX_FLIPS = 1          # near-tie flips allowed per workload (selection is float64: expected ~0)


def oracle_kv(w):
    return santa.PagedKV(w.dtype, w.k_pages, w.v_pages, w.page_table, w.seq_lens)


def oracle_reps(w, pairs=None):
    seqs = None if pairs is None else set(b for b, _ in pairs)
    return santa.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype, seqs=seqs)


def decoded_reps(gpu_reps, dtype):
    arr = gpu_reps.cpu()
    if dtype == "bf16":
        import torch
        return numerics.decode_bf16(arr.view(torch.int16).numpy().view(np.uint16))
    return arr.numpy().astype(np.float64)


def check_reps(w, gpu_reps, pairs=None):
    """Representatives of every team of the sequences in ``pairs`` (all when None) are bit exact."""
    ref = oracle_reps(w, pairs)
    got = decoded_reps(gpu_reps, w.dtype)
    seqs = sorted(set(b for b, _ in pairs)) if pairs is not None else range(w.batch)
    for b in seqs:
        K = santa.num_teams(int(w.seq_lens[b]), w.page_size)
        assert np.array_equal(got[b, :K], ref[b, :K]), f"representatives of sequence {b} differ from the oracle"
    return ref


def check_dense_head(w, kv, b, h, out, lse):
    qh = numerics.decode(w.q[b, h], w.dtype)
    ref_out, ref_lse = santa.dense_head(kv, qh, b, h, w.num_q_heads)
    err = float(np.max(np.abs(out - ref_out)))
    assert err <= OUT_TOL[w.dtype], f"dense (b={b}, h={h}) max-abs {err}"
    _check_lse(w, lse, ref_lse, b, h)
    return err


def _check_lse(w, got, ref, b, h):
    if ref == -math.inf:
        assert got == -math.inf, f"(b={b}, h={h}) lse {got}, expected -inf"
    else:
        tol = LSE_TOL[w.dtype] + LSE_RTOL * abs(ref)
        assert abs(got - ref) <= tol, f"(b={b}, h={h}) lse {got} vs {ref} (tolerance {tol:.3g})"


def check_santa_head(w, kv, reps, b, h, out, lse, teams, inv_pi, M=None, seed=None, offset=None,
                     scheme=santa.DRAW_IID):
    """Compare one head's HIP sets, weights, output and lse with the oracle.

    Returns (max-abs error, near_tie_flip: bool).
    """
    M = w.M if M is None else M
    seed = w.seed if seed is None else seed
    offset = w.offset if offset is None else offset
    qh = numerics.decode(w.q[b, h], w.dtype)
    res = santa.santa_head(kv, qh, reps, b, h, w.num_q_heads, M, seed, offset, scheme)
    got_teams, ref_w, flip = _check_sets(res.selection, b, h, teams, inv_pi, M, scheme)
    if flip:
        ref_out, ref_lse = santa.evaluate_given_set(kv, qh, b, h, w.num_q_heads, got_teams, ref_w)
    else:
        ref_out, ref_lse = res.out, res.lse
    err = float(np.max(np.abs(out - ref_out))) if len(ref_out) else 0.0
    assert err <= OUT_TOL[w.dtype], f"santa (b={b}, h={h}) max-abs {err}"
    _check_lse(w, lse, ref_lse, b, h)
    return err, flip


def _check_sets(sel, b, h, teams, inv_pi, M, scheme):
    """The HIP team list (ascending, -1 padded) against the oracle's selection:
    equal, or different only in near-tie teams; the weights 1/pi of the HIP
    teams within INV_PI_RTOL. Returns (HIP teams, their exact weights, flip)."""
    got_teams = [int(t) for t in teams if t >= 0]
    assert all(t < 0 for t in teams[len(got_teams):]), "sampled list not -1 padded"
    assert got_teams == sorted(set(got_teams)), "sampled list not ascending and unique"
    flip = got_teams != sel.teams
    if flip:
        diff = set(got_teams) ^ set(sel.teams)
        assert diff <= sel.near_tie_teams, (
            f"(b={b}, h={h}) team sets differ outside near-ties: gpu-only "
            f"{sorted(set(got_teams) - set(sel.teams))}, oracle-only {sorted(set(sel.teams) - set(got_teams))}")
    if sel.full:
        ref_w = [1.0] * len(got_teams)
    else:
        ref_w = [1.0 / santa.inclusion_probability_scheme(scheme, t, sel.C, sel.Z, sel.p, M) for t in got_teams]
    w_got = np.asarray(inv_pi[:len(got_teams)], dtype=np.float64)
    assert np.all(np.abs(w_got - ref_w) <= INV_PI_RTOL * np.abs(ref_w) + 1e-30), f"(b={b}, h={h}) 1/pi differs"
    assert np.all(np.asarray(inv_pi[len(got_teams):]) == 0.0)
    return got_teams, ref_w, flip


def check_value_sampled_head(w, kv, reps, b, h, S, out, lse, teams, inv_pi, positions, M=None, seed=None,
                             offset=None, scheme=santa.DRAW_IID, value_scheme=santa.DRAW_IID):
    """One head of santa_decode_attention_value_sampled against the oracle.

    Teams and weights as for SANTA++; the S sample positions must equal the
    oracle's, except that a sample within NEAR_TIE of a token boundary may
    take another token it can reach (both listed as near-tie positions). On a
    near-tie team flip the logits differ, so each position is only checked to
    lie in a HIP team. The output is compared with the mean of the values at
    the HIP positions (the oracle's own when they agree); the log-sum-exp
    with the oracle's on the HIP team set. Returns (max-abs error, flips).
    """
    M = w.M if M is None else M
    seed = w.seed if seed is None else seed
    offset = w.offset if offset is None else offset
    qh = numerics.decode(w.q[b, h], w.dtype)
    res = santa.value_sampled_head(kv, qh, reps, b, h, w.num_q_heads, M, S, seed, offset, scheme, value_scheme)
    L = int(w.seq_lens[b])
    got = [int(x) for x in positions[:S]]
    if L == 0:
        assert got == [-1] * S, f"(b={b}, h={h}) positions of an empty sequence {got}"
        assert np.all(out == 0.0) and lse == -math.inf
        return 0.0, 0
    got_teams, ref_w, flip = _check_sets(res.selection, b, h, teams, inv_pi, M, scheme)
    assert all(0 <= x < L and x // w.page_size in got_teams for x in got), f"(b={b}, h={h}) positions {got}"
    flips = int(flip)
    if flip:
        ref_lse = santa.evaluate_given_set(kv, qh, b, h, w.num_q_heads, got_teams, ref_w)[1]
    else:
        ref_lse = res.lse
        bad = [(x, y) for x, y in zip(got, res.positions) if x != y]
        assert all(x in res.near_tie_positions and y in res.near_tie_positions for x, y in bad), (
            f"(b={b}, h={h}) sample positions differ outside near-ties: {bad[:4]}")
        flips += len(bad)
    ref_out = res.out if got == res.positions else santa.value_sampled_given(kv, qh, b, h, w.num_q_heads, got)
    err = float(np.max(np.abs(out - ref_out)))
    assert err <= OUT_TOL[w.dtype], f"value-sampled (b={b}, h={h}) max-abs {err}"
    _check_lse(w, lse, ref_lse, b, h)
    return err, flips

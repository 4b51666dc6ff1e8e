"""SANTA++ sampled-team decode attention, step by step, in float64 on the CPU.

TEST INFRASTRUCTURE (see the package docstring): the plain, slow reference the
HIP path is compared with. It shares no code with that path.

What the method computes ([ABS]; [EXP] section 三 "核心方法"): the cache is
partitioned into teams, each summarised by one key; the query's dot products
with those keys, through a softmax, give each team a probability p; M teams
are drawn from p; only the drawn teams' tokens get exact scores; a drawn
team's terms count 1/pi times, pi the chance the team was drawn at all, so
the sums over drawn teams are unbiased for the sums over every token.

Readings taken where the pages leave a step open (each repeated where used):
  R1  teams are contiguous runs of T tokens, one team per KV page; the last
      team of a sequence may be shorter ([EXP] 3.2 says the partition is open).
  R2  the representative is the mean key of the team, stored in the KV type
      (one round-to-nearest-even of the exact mean), unscaled ([EXP] section 三
      lists mean / medoid / random).
  R3  team scores and token scores carry the usual 1/sqrt(d) factor.
  R4  "sample M teams" = M independent draws with replacement by inverse CDF,
      then duplicates removed; inclusion probability pi = 1 - (1 - p)^M and the
      weight is 1/pi ([ABS] weights a drawn team by 1/pi; [EXP] step 5
      writes 1/p_i, which the abstract overrides).
  R5  the estimate of the attention output is the ratio of the weighted
      numerator sum to the weighted denominator sum (both sums are
      unbiased; the ratio is consistent).
  R6  if M >= number of teams, every team is read and pi = 1 (full coverage).
  R7  draws are independent per query head; a KV head's G query heads share
      nothing but the cache.
  R8  an empty sequence (length 0) gives out = 0 and lse = -inf.
  R9  alternative representatives ([EXP] section 三 step 2 lists mean,
      medoid and random; the mean is the default). The medoid is the member
      key with the smallest sum of Euclidean distances to all members of its
      team; each distance is the correctly rounded square root of the
      channel-ordered float64 sum of squared float64 differences, the n
      distances of a member are added in member order, and ties go to the
      lowest member index. The random representative is member
      floor(x n / 2^32), x = word 0 of Philox4x32-10 with counter
      (t, g, b, 0) and key (seed lo ^ 0x52455053, seed hi) (a key of its own,
      so its stream is disjoint from the team draws'). Both are copies of a
      cached key, so no rounding is involved.
  R10 variance-reduced team draws (the SANTA page, "Stochastic Sparse
      Attention for Memory-Bound Inference", abstract: stratified and
      systematic sampling lower the estimator's variance; here applied to the
      team draw). The M points u_j that pick teams through the same inverse
      CDF are, for the systematic scheme, (j + u0) / M with one uniform u0
      (word 0 of the block with counter (0, h, b, offset)), and for the
      stratified scheme (j + U_j) / M with U_j the uniform of draw j of the
      independent scheme. In units of 1/M team t covers [a, a + w) with
      a = M C_(t-1) / Z and w = M p_t; its inclusion probability is
      min(1, w) (systematic: the points are one unit apart) and
      1 - prod_j (1 - |[a, a + w) n [j, j + 1)|) (stratified: one
      independent point per unit). Full coverage (R6) is unchanged.
  R11 hash-partitioned teams ([EXP] section 三 step 1 clusters the keys into
      teams; section 八 pitfall 3 names sequential, hash and cluster
      partitions and asks for a configurable one). Per (sequence, KV head),
      token i gets the code whose bit j (most significant first) is
      [k_i . r_j > 0] for caller-supplied directions r_j, the dot product a
      float64 sum in channel order of exact products; the tokens are stably
      sorted by code and cut into runs of T, so team t holds sorted
      positions tT .. tT + T - 1 (the last team may be short). The cache
      is rewritten in that order, so every other step is unchanged.
  R12 k-means-partitioned teams (the "cluster" partition of the same
      passages). Per (sequence, KV head) with L tokens and C clusters:
      centroids start at the keys of tokens floor(c L / C); each iteration
      assigns every token to argmax_c (k . mu_c - |mu_c|^2 / 2) (the nearest
      centroid; lowest c on ties), both terms float64 sums in channel order
      of separately rounded products, then moves each non-empty cluster's
      centroid to the float64 mean of its members (sums in token order, one
      divide); after `iters` assignments (no move after the last) the
      assignment is the code, and the tokens are stably sorted by code and
      cut into runs of T as in R11.
  R13 value samples (optional, [SANTA] abstract): S points per head from
      their own Philox stream (key word 0 xored with VALUE_KEY_XOR), pushed
      through the inverse CDF of the drawn tokens' weighted logits in team
      order, then token order; independent, systematic or stratified points
      as for the team draws.
  R14 the value-sampled output is the plain mean of the sampled values; the
      log-sum-exp stays that of the drawn tokens (the denominator is exact).

Parity pins (tests/test_oracle_pins.py): dense attention against torch's
scaled_dot_product_attention; full coverage against dense; brute-force
enumeration of all draw sequences on tiny inputs for unbiasedness of both
sums and for P(t in S) = pi_t; Monte Carlo convergence over seeds; the
expected set size against its closed form; chi-square of draw frequencies
against p; invariants (constant values, permuted page tables); team scores
with one-token teams against the attention weights of the library routine;
the near-tie record on cumulative sums with exact binary boundaries (points
just inside and just outside the band at each interior boundary, the last
sum never a boundary, zero-mass neighbours, a team narrower than the band),
with planted detector mistakes (band x1000 or /1000, teams off by one, the
last sum taken as a boundary) each failing a pin.
R9: the medoid of collinear keys is the median member (a skewed set
separates it from the squared-distance choice), scipy's distance sums
agree, ties go to the lowest index, translation invariance, outliers are
never chosen; the random member is uniform (chi-square). R10: both
inclusion probabilities equal an exact integration of the selection rule
over its piecewise-constant pieces, the team sums stay unbiased, tiny teams
keep full precision, equal teams give M distinct systematic draws, and on
team-coherent keys both schemes lower the error. R11: code bits against
basis directions, signs against exact rational dot products, a stable
order that keeps separated clusters in one run, a per-head permutation
that leaves dense attention unchanged, lower error on planted keys.
R13-R14: given the teams, the mean over many offsets converges to the
SANTA++ estimate of the same teams (and a planted oracle without the team
weights does not), full coverage converges to dense attention, systematic
points sample every drawn token floor(S p) or ceil(S p) times, a one-token
head returns its value, and the value stream differs from the team stream.
"""
import math
from fractions import Fraction

import numpy as np

from .numerics import decode, round_to_dtype
from .philox import draw_words, word_to_uniform

NEAR_TIE = 1e-6   # a draw closer than this to a CDF boundary may differ between implementations


# ----------------------------------------------------------------------------
# Teams and the paged cache (reading R1)
# ----------------------------------------------------------------------------

def num_teams(L, T):
    """Number of teams of a sequence of L tokens with team size T (R1)."""
    return (int(L) + T - 1) // T


def team_size(L, T, t):
    """Valid tokens in team t of a sequence of L tokens (the last may be short, R1)."""
    return min(T, int(L) - t * T)


# ----------------------------------------------------------------------------
# Representatives (reading R2)
# ----------------------------------------------------------------------------

def build_reps(k_pages, page_table, seq_lens, page_size, dtype, seqs=None):
    """Mean key of every team, rounded once to the KV type.

    [EXP] section 三 step 2: one representative key per team (mean, medoid or
    random are listed); [ABS]: team selection looks only at these summary
    keys. Reading R2: the mean, as math.fsum(column) / n (exact sum, one
    correctly rounded divide), then one round-to-nearest-even into the KV type.

    Returns a float64 array [B][max_pages][Hkv][d] indexed by logical team;
    rows of teams past a sequence's end (or of sequences not in ``seqs`` when
    given) are NaN.
    """
    _, hkv, T, d = k_pages.shape
    B, P = np.asarray(page_table).shape
    reps = np.full((B, P, hkv, d), np.nan)
    for b in range(B):
        if seqs is not None and b not in seqs:
            continue
        L = int(seq_lens[b])
        for t in range(num_teams(L, T)):
            p = int(page_table[b][t])
            n = team_size(L, T, t)
            keys = decode(k_pages[p, :, :n, :], dtype)          # [Hkv][n][d]
            for g in range(hkv):
                for c in range(d):
                    reps[b, t, g, c] = math.fsum(keys[g, :, c]) / n
            reps[b, t] = round_to_dtype(reps[b, t], dtype)
    return reps


REP_MEAN, REP_MEDOID, REP_RANDOM = 0, 1, 2
REP_KEY_XOR = 0x52455053     # separates the random-representative stream from the draws (R9)


def team_medoid_index(keys):
    """Medoid of a team's keys [n][d] (float64 values of cached keys), reading R9.

    [EXP] section 三 step 2 names the medoid as a representative choice: the
    member whose distances to all members have the smallest sum. The loops
    fix R9's orders (channels inside a distance, members across distances)
    and run over all (i, j) pairs at once; np.sqrt is correctly rounded;
    np.argmin takes the first (lowest) index among equal sums.
    """
    keys = np.asarray(keys, dtype=np.float64)
    n, d = keys.shape
    s2 = np.zeros((n, n))
    for c in range(d):
        diff = keys[:, None, c] - keys[None, :, c]              # [i][j]
        s2 = s2 + diff * diff
    dist = np.sqrt(s2)
    total = np.zeros(n)
    for j in range(n):
        total = total + dist[:, j]
    return int(np.argmin(total))


def team_random_index(n, seed, b, t, g):
    """Random member of a team of n keys (reading R9): floor(x n / 2^32)."""
    from .philox import philox4x32_10, MASK32
    seed = int(seed)
    x = philox4x32_10((t, g, b, 0), ((seed & MASK32) ^ REP_KEY_XOR, (seed >> 32) & MASK32))[0]
    return (x * n) >> 32


def build_reps_kind(k_pages, page_table, seq_lens, page_size, dtype, kind, seed=0, seqs=None):
    """Representatives of every team for kind REP_MEAN (build_reps), REP_MEDOID
    or REP_RANDOM (R9); same layout and NaN convention as build_reps."""
    if kind == REP_MEAN:
        return build_reps(k_pages, page_table, seq_lens, page_size, dtype, seqs)
    _, hkv, T, d = k_pages.shape
    B, P = np.asarray(page_table).shape
    reps = np.full((B, P, hkv, d), np.nan)
    for b in range(B):
        if seqs is not None and b not in seqs:
            continue
        L = int(seq_lens[b])
        for t in range(num_teams(L, T)):
            p = int(page_table[b][t])
            n = team_size(L, T, t)
            keys = decode(k_pages[p, :, :n, :], dtype)          # [Hkv][n][d]
            for g in range(hkv):
                i = team_medoid_index(keys[g]) if kind == REP_MEDOID else team_random_index(n, seed, b, t, g)
                reps[b, t, g] = keys[g, i]
    return reps


# ----------------------------------------------------------------------------
# Hash-partitioned teams (reading R11)
# ----------------------------------------------------------------------------

def hash_codes(keys, directions):
    """Code of each key [L][d] for directions [bits][d] (R11): bit j, most
    significant first, is 1 when the channel-ordered float64 dot product with
    direction j is > 0. The products (of a bfloat16 or float32 key and a
    float32 direction) are exact in float64."""
    keys = np.asarray(keys, dtype=np.float64)
    dirs = np.asarray(directions, dtype=np.float64)
    L, d = keys.shape
    code = np.zeros(L, dtype=np.int64)
    for j in range(dirs.shape[0]):
        dot = np.zeros(L)
        for c in range(d):
            dot = dot + keys[:, c] * dirs[j, c]
        code = 2 * code + (dot > 0)
    return code


def hash_partition_order(keys, directions):
    """Token order of the hash partition (R11): a stable sort by code."""
    return np.argsort(hash_codes(keys, directions), kind="stable")


def cluster_pages(k_pages, v_pages, page_table, seq_lens, page_size, dtype, directions):
    """The cache rewritten in hash-partition order (R11).

    k_pages, v_pages: stored pages [num_pages][Hkv][T][d]; directions:
    float32 [Hkv][bits][d]. Returns (k, v, codes, token_of): the rewritten
    pages (slots past a sequence's end are zero), the code of every original
    token and the original token at every new position, both [B][Hkv][P*T]
    with -1 past the sequence's end. Pages outside the sequences' teams are
    copied unchanged.
    """
    _, hkv, T, d = k_pages.shape
    B, P = np.asarray(page_table).shape
    k2, v2 = k_pages.copy(), v_pages.copy()
    codes = np.full((B, hkv, P * T), -1, dtype=np.int64)
    token_of = np.full((B, hkv, P * T), -1, dtype=np.int64)
    for b in range(B):
        L = int(seq_lens[b])
        K = num_teams(L, T)
        pages = np.asarray(page_table[b][:K], dtype=np.int64)
        for g in range(hkv):
            keys = k_pages[pages, g].reshape(K * T, d)[:L]
            vals = v_pages[pages, g].reshape(K * T, d)[:L]
            c = hash_codes(decode(keys, dtype), directions[g])
            order = np.argsort(c, kind="stable")
            codes[b, g, :L] = c
            token_of[b, g, :L] = order
            nk = np.zeros((K * T, d), dtype=k_pages.dtype)
            nv = np.zeros((K * T, d), dtype=v_pages.dtype)
            nk[:L] = keys[order]
            nv[:L] = vals[order]
            k2[pages, g] = nk.reshape(K, T, d)
            v2[pages, g] = nv.reshape(K, T, d)
    return k2, v2, codes, token_of


def kmeans_codes(keys, clusters, iters):
    """Cluster of each key [L][d] after `iters` k-means assignments (R12).

    Plain loops in the orders R12 fixes, vectorised over tokens and
    clusters only: every product is rounded before it is added.
    """
    x = np.asarray(keys, dtype=np.float64)
    L, d = x.shape
    C = int(clusters)
    mu = x[[(c * L) // C for c in range(C)]].copy()          # [C][d]
    assign = np.zeros(L, dtype=np.int64)
    for it in range(int(iters)):
        half = np.zeros(C)
        for ch in range(d):
            half = half + mu[:, ch] * mu[:, ch]
        for i0 in range(0, L, 1024):                          # token blocks (same arithmetic per element)
            xb = x[i0:i0 + 1024]
            dot = np.zeros((len(xb), C))
            for ch in range(d):
                dot = dot + xb[:, ch:ch + 1] * mu[None, :, ch]
            assign[i0:i0 + 1024] = np.argmax(dot - half[None, :] / 2.0, axis=1)   # lowest c on ties
        if it + 1 < int(iters):
            for c in range(C):
                members = np.nonzero(assign == c)[0]          # token order
                if len(members) == 0:
                    continue
                # running sum from +0.0, one row at a time, in token order
                acc = np.add.accumulate(np.vstack([np.zeros((1, d)), x[members]]), axis=0)[-1]
                mu[c] = acc / len(members)
    return assign


def cluster_pages_kmeans(k_pages, v_pages, page_table, seq_lens, page_size, dtype, clusters, iters):
    """The cache rewritten in k-means order (R12); same outputs as
    cluster_pages. `clusters` is per sequence: a number, or None for one
    cluster per team (K_b)."""
    _, hkv, T, d = k_pages.shape
    B, P = np.asarray(page_table).shape
    k2, v2 = k_pages.copy(), v_pages.copy()
    codes = np.full((B, hkv, P * T), -1, dtype=np.int64)
    token_of = np.full((B, hkv, P * T), -1, dtype=np.int64)
    for b in range(B):
        L = int(seq_lens[b])
        K = num_teams(L, T)
        if L == 0:
            continue
        C = min(L, K if clusters is None else int(clusters))
        pages = np.asarray(page_table[b][:K], dtype=np.int64)
        for g in range(hkv):
            keys = k_pages[pages, g].reshape(K * T, d)[:L]
            vals = v_pages[pages, g].reshape(K * T, d)[:L]
            c = kmeans_codes(decode(keys, dtype), C, iters)
            order = np.argsort(c, kind="stable")
            codes[b, g, :L] = c
            token_of[b, g, :L] = order
            nk = np.zeros((K * T, d), dtype=k_pages.dtype)
            nv = np.zeros((K * T, d), dtype=v_pages.dtype)
            nk[:L] = keys[order]
            nv[:L] = vals[order]
            k2[pages, g] = nk.reshape(K, T, d)
            v2[pages, g] = nv.reshape(K, T, d)
    return k2, v2, codes, token_of


# ----------------------------------------------------------------------------
# Selection: scores, team softmax, draws, inclusion probabilities
# ----------------------------------------------------------------------------

def rep_scores(q_h, rep_rows):
    """s_t = (1/sqrt(d)) * q . rep_t for every team ([EXP] section 三 step 2; R3).

    The products of two bfloat16 or two binary32 values are exact in float64;
    math.fsum makes each dot product correctly rounded.
    """
    d = q_h.shape[0]
    inv_sqrt_d = 1.0 / math.sqrt(d)
    return np.array([math.fsum(q_h * r) * inv_sqrt_d for r in rep_rows])


def team_softmax(s):
    """Team-level softmax and its cumulative sums ([EXP] section 三 step 2).

    Returns (e, C, Z, p): e_t = exp(s_t - max s); C_t = e_0 + ... + e_t summed
    left to right; Z = C_last; p_t = e_t / Z.
    """
    m = max(s)
    e = np.array([math.exp(x - m) for x in s])
    C = np.empty_like(e)
    acc = 0.0
    for t, x in enumerate(e):
        acc += x
        C[t] = acc
    Z = C[-1]
    return e, C, Z, e / Z


def inverse_cdf(u, e, C, Z):
    """Team drawn by uniform u: the first t with u * Z < C_t.

    Strict '<' on the unnormalised cumulative sums never selects a team with
    zero mass. If rounding leaves no such t, the last team with positive mass
    is taken (this cannot happen for u < 1, kept as a guard).
    """
    x = u * Z
    for t in range(len(C)):
        if x < C[t]:
            return t
    return int(np.nonzero(e > 0)[0][-1])


def draw_distance_to_boundary(u, C, Z):
    """Distance from u to the nearest interior CDF boundary C_t / Z (t < K-1).

    C_(K-1) / Z = 1 lies above every point a draw can take, so it is never a
    boundary a draw can cross."""
    if len(C) < 2:
        return math.inf
    return float(np.min(np.abs(u - C[:-1] / Z)))


def near_tie_teams_of_draw(u, e, C, Z, band=None):
    """Teams a draw at point u can land on when the normalised cumulative
    sums C_t / Z move by less than `band` (NEAR_TIE by default).

    Reading of the near-tie rule: an implementation whose team
    probabilities differ by less than the band may send such a draw to any
    team with positive mass whose interval [C_(t-1) / Z, C_t / Z) meets
    (u - band, u + band). Teams with zero mass have empty intervals and are
    never listed, so a boundary shared by several empty teams names the
    teams on both sides that have mass. Returns that set when it holds two
    or more teams (the draw is a near-tie), else the empty set.
    """
    band = NEAR_TIE if band is None else band
    lo, hi = u - band, u + band
    reach = set()
    prev = 0.0
    for t in range(len(C)):
        right = C[t] / Z
        if e[t] > 0 and prev < hi and right > lo:
            reach.add(t)
        prev = right
    return reach if len(reach) >= 2 else set()


DRAW_IID, DRAW_SYSTEMATIC, DRAW_STRATIFIED = 0, 1, 2


def draw_uniforms(scheme, M, seed, offset, b, h):
    """The M points in (0, 1) that pick one head's teams (R4; R10).

    Independent: u_j from draw j's Philox word. Systematic: (j + u0) / M,
    u0 the first of those uniforms. Stratified: (j + u_j) / M. The sums
    j + u are exact in float64 (u has 33 significant bits) and the division
    is correctly rounded.
    """
    u = [word_to_uniform(x) for x in draw_words(M, seed, offset, b, h)]
    if scheme == DRAW_IID:
        return u
    if scheme == DRAW_SYSTEMATIC:
        return [(j + u[0]) / M for j in range(M)]
    if scheme == DRAW_STRATIFIED:
        return [(j + u[j]) / M for j in range(M)]
    raise ValueError(f"unknown draw scheme {scheme!r}")


def inclusion_probability_scheme(scheme, t, C, Z, p, M):
    """Inclusion probability of team t under a draw scheme (R4; R10).

    For the stratified scheme the product over units is evaluated exactly in
    rational arithmetic on the float64 values a = M C_(t-1) / Z and
    w = M p_t, then rounded once.
    """
    if scheme == DRAW_IID:
        return inclusion_probability(p[t], M)
    if scheme == DRAW_SYSTEMATIC:
        return min(1.0, M * p[t])
    if scheme != DRAW_STRATIFIED:
        raise ValueError(f"unknown draw scheme {scheme!r}")
    a = Fraction(M * C[t - 1] / Z) if t > 0 else Fraction(0)
    end = a + Fraction(M) * Fraction(p[t])
    miss = Fraction(1)
    for j in range(max(0, math.floor(a)), min(M, math.ceil(end))):
        overlap = min(end, Fraction(j + 1)) - max(a, Fraction(j))
        if overlap > 0:
            miss *= 1 - overlap
    return float(1 - miss)


def inclusion_probability(p, M):
    """pi = 1 - (1 - p)^M, computed as -expm1(M * log1p(-p)) (R4).

    [ABS]: a drawn team's terms carry the weight 1/pi; with M independent
    draws, team t misses every draw with chance (1 - p_t)^M, so it is drawn
    at least once with chance 1 - (1 - p_t)^M.
    """
    return -math.expm1(M * math.log1p(-p))


class Selection:
    """Result of sampling teams for one query head."""

    def __init__(self, teams, pi, p, near_tie_teams, draws, full):
        self.teams = teams                  # ascending unique team indices
        self.pi = pi                        # inclusion probability of each, same order
        self.p = p                          # team probabilities, all teams
        self.near_tie_teams = near_tie_teams  # teams reached or missed via a near-tie draw
        self.draws = draws                  # raw draw results t_j (empty if full)
        self.full = full                    # True when every team is read (R6)

    @property
    def inv_pi(self):
        return [1.0 / x for x in self.pi]


def select_teams(q_h, rep_rows, M, seed, offset, b, h, scheme=DRAW_IID):
    """Sample teams for one query head (steps 2-3 of [EXP] section 三; [ABS]; R4, R6, R7, R10).

    Draw j uses point u_j of draw_uniforms (Philox4x32-10; see oracle/philox.py
    for the counter layout) and takes team inverse_cdf(u_j). Draws whose
    point lies within NEAR_TIE of a CDF boundary are recorded: every team
    with mass the draw could reach under such a shift is listed in
    near_tie_teams (near_tie_teams_of_draw).
    """
    K = len(rep_rows)
    s = rep_scores(q_h, rep_rows)
    e, C, Z, p = team_softmax(s)
    if M >= K:
        teams = list(range(K))
        return Selection(teams, [1.0] * K, p, set(), [], True)
    near = set()
    draws = []
    for u in draw_uniforms(scheme, M, seed, offset, b, h):
        t = inverse_cdf(u, e, C, Z)
        draws.append(t)
        near.update(near_tie_teams_of_draw(u, e, C, Z))
    teams = sorted(set(draws))
    pi = [inclusion_probability_scheme(scheme, t, C, Z, p, M) for t in teams]
    sel = Selection(teams, pi, p, near, draws, False)
    sel.C, sel.Z = C, Z
    return sel


# ----------------------------------------------------------------------------
# Estimation inside the sampled teams
# ----------------------------------------------------------------------------

def token_scores(q_h, keys):
    """s_j = (1/sqrt(d)) * q . k_j for the rows of ``keys`` (R3)."""
    d = q_h.shape[0]
    return (keys @ q_h) * (1.0 / math.sqrt(d))


def ht_sums(q_h, team_kv, weights, shift):
    """Weighted sums over the sampled teams ([EXP] steps 4-5; [ABS]; R5).

    team_kv: list of (keys [n][d], values [n][d]) for the sampled teams;
    weights: w_t for each (1/pi_t). Returns (numerator [d], denominator):
      N = sum_t w_t sum_{j in t} exp(s_j - shift) v_j
      D = sum_t w_t sum_{j in t} exp(s_j - shift)
    """
    d = q_h.shape[0]
    num = np.zeros(d)
    den = 0.0
    for (keys, vals), w in zip(team_kv, weights):
        a = np.exp(token_scores(q_h, keys) - shift)
        num += w * (a @ vals)
        den += w * a.sum()
    return num, den


def estimate(q_h, team_kv, weights):
    """Estimated attention output and log-sum-exp from sampled teams (R5).

    out = N / D; lse = shift + log(D), where shift is the largest token score
    among the sampled teams (it cancels in out). An empty team list (an empty
    sequence) gives out = 0 and lse = -inf (R8).
    """
    d = q_h.shape[0]
    if not team_kv:
        return np.zeros(d), -math.inf
    shift = max(float(np.max(token_scores(q_h, k))) for k, _ in team_kv)
    num, den = ht_sums(q_h, team_kv, weights, shift)
    return num / den, shift + math.log(den)


def dense_attention(q_h, keys, vals):
    """Exact softmax attention of one query over all L cached tokens.

    The dense baseline SANTA++ is measured against ([ABS] compares with
    exact attention over every token). Returns (out [d], lse).
    """
    if keys.shape[0] == 0:
        return np.zeros(q_h.shape[0]), -math.inf
    s = token_scores(q_h, keys)
    m = float(np.max(s))
    a = np.exp(s - m)
    return (a @ vals) / a.sum(), m + math.log(a.sum())


# ----------------------------------------------------------------------------
# Whole decode step over a paged batch
# ----------------------------------------------------------------------------

class PagedKV:
    """Float64 view of a paged KV cache (pages in plain token-major order).

    k_pages, v_pages: stored arrays [num_pages][Hkv][T][d] (uint16 bf16 bits
    or float32); page_table [B][max_pages]; seq_lens [B]. Pages are decoded
    to float64 on first use.
    """

    def __init__(self, dtype, k_pages, v_pages, page_table, seq_lens):
        self.dtype = dtype
        self.k_raw, self.v_raw = k_pages, v_pages
        self.page_table = np.asarray(page_table)
        self.seq_lens = np.asarray(seq_lens)
        self.num_pages, self.hkv, self.T, self.d = k_pages.shape
        self._k, self._v = {}, {}

    def _page(self, cache, raw, p):
        if p not in cache:
            cache[p] = decode(raw[p], self.dtype)
        return cache[p]

    def team(self, b, g, t):
        """(keys [n][d], values [n][d]) of team t of sequence b, KV head g."""
        L = int(self.seq_lens[b])
        p = int(self.page_table[b][t])
        n = team_size(L, self.T, t)
        return (self._page(self._k, self.k_raw, p)[g, :n, :],
                self._page(self._v, self.v_raw, p)[g, :n, :])

    def all_tokens(self, b, g):
        L = int(self.seq_lens[b])
        K = num_teams(L, self.T)
        if K == 0:
            return np.zeros((0, self.d)), np.zeros((0, self.d))
        parts = [self.team(b, g, t) for t in range(K)]
        return np.concatenate([k for k, _ in parts]), np.concatenate([v for _, v in parts])


class HeadResult:
    def __init__(self, out, lse, selection):
        self.out, self.lse, self.selection = out, lse, selection


def santa_head(kv, q_h, reps, b, h, num_q_heads, M, seed, offset, scheme=DRAW_IID):
    """SANTA++ for one (sequence b, query head h): select teams, then estimate.

    q_h: float64 query [d]; reps: float64 [B][max_pages][Hkv][d] (from build_reps).
    KV head of query head h is h // (Hq / Hkv) (grouped-query attention).
    """
    g = h // (num_q_heads // kv.hkv)
    L = int(kv.seq_lens[b])
    K = num_teams(L, kv.T)
    if K == 0:
        return HeadResult(np.zeros(kv.d), -math.inf, Selection([], [], np.zeros(0), set(), [], True))
    rep_rows = np.stack([reps[b, t, g] for t in range(K)])
    sel = select_teams(q_h, rep_rows, M, seed, offset, b, h, scheme)
    out, lse = estimate(q_h, [kv.team(b, g, t) for t in sel.teams], sel.inv_pi)
    return HeadResult(out, lse, sel)


# ----------------------------------------------------------------------------
# Value samples inside the drawn teams (the optional half of the
# variance-reduced row; [SANTA] abstract; readings R13-R14)
# ----------------------------------------------------------------------------

VALUE_KEY_XOR = 0x56414C55   # separates the value-sample stream from the team draws (R13)


def value_uniforms(scheme, S, seed, offset, b, h):
    """The S points in (0, 1) that pick one head's value samples (R13).

    Sample k takes word k mod 4 of Philox4x32-10 with counter
    (k div 4, h, b, offset) and key (seed lo xor VALUE_KEY_XOR, seed hi);
    u = (x + 1/2) 2^-32. Independent points u_k; systematic (k + u_0) / S;
    stratified (k + u_k) / S, as for the team draws.
    """
    from .philox import philox4x32_10, MASK32, word_to_uniform
    seed = int(seed)
    key = ((seed & MASK32) ^ VALUE_KEY_XOR, (seed >> 32) & MASK32)
    u = [word_to_uniform(philox4x32_10((k // 4, h, b, offset), key)[k % 4]) for k in range(S)]
    if scheme == DRAW_IID:
        return u
    if scheme == DRAW_SYSTEMATIC:
        return [(k + u[0]) / S for k in range(S)]
    if scheme == DRAW_STRATIFIED:
        return [(k + u[k]) / S for k in range(S)]
    raise ValueError(f"unknown draw scheme {scheme!r}")


class ValueSampled:
    """SANTA++ teams with value samples: the estimate and what decided it."""

    def __init__(self, out, lse, selection, positions, near_tie_positions, logits):
        self.out, self.lse, self.selection = out, lse, selection
        self.positions = positions                    # sampled token positions (t * T + j), in sample order
        self.near_tie_positions = near_tie_positions  # positions a near-tie sample may land on instead
        self.logits = logits                          # weighted logits of the drawn tokens, team then token order


def value_sampled_head(kv, q_h, reps, b, h, num_q_heads, M, S, seed, offset, scheme=DRAW_IID,
                       value_scheme=DRAW_IID):
    """SANTA++ team draws, then S value samples inside the drawn teams (R13,
    R14; [SANTA] abstract: positions picked with probability equal to their
    attention weight, then the mean of their values, stand in for the
    attention output without bias).

    The drawn teams and weights are select_teams'. Over the drawn tokens in
    team order, then token order, the weighted logits are
    l_j = s_j + log w_t (s_j = q . k_j / sqrt(d), w_t = 1 / pi_t); with
    m = max l, e_j = exp(l_j - m) and C the running sums (Z = C_last), sample k
    takes the first token j with u_k Z < C_j (the team rule, one level down).
    out = (1/S) sum_k v_(j_k), which given the drawn teams averages to the
    SANTA++ estimate sum_j (e_j / Z) v_j; lse = m + log Z, the SANTA++ log-sum-exp.
    Samples within NEAR_TIE of a boundary record the positions they can reach.
    """
    g = h // (num_q_heads // kv.hkv)
    L = int(kv.seq_lens[b])
    K = num_teams(L, kv.T)
    if K == 0:
        return ValueSampled(np.zeros(kv.d), -math.inf, Selection([], [], np.zeros(0), set(), [], True), [], set(),
                            np.zeros(0))
    rep_rows = np.stack([reps[b, t, g] for t in range(K)])
    sel = select_teams(q_h, rep_rows, M, seed, offset, b, h, scheme)
    logits, vals, pos = [], [], []
    for t, w in zip(sel.teams, sel.inv_pi):
        keys, v = kv.team(b, g, t)
        logits.append(token_scores(q_h, keys) + math.log(w))
        vals.append(v)
        pos.extend(t * kv.T + j for j in range(keys.shape[0]))
    logits = np.concatenate(logits)
    vals = np.concatenate(vals)
    e, C, Z, _ = team_softmax(logits)
    m = float(np.max(logits))
    picks, near = [], set()
    for u in value_uniforms(value_scheme, S, seed, offset, b, h):
        j = inverse_cdf(u, e, C, Z)
        picks.append(j)
        near.update(pos[i] for i in near_tie_teams_of_draw(u, e, C, Z))
    out = np.mean(vals[picks], axis=0)
    return ValueSampled(out, m + math.log(Z), sel, [pos[j] for j in picks], near, logits)


def value_sampled_given(kv, q_h, b, h, num_q_heads, positions):
    """The value-sampled output for supplied sample positions (a near-tie
    made the HIP path pick another valid position): their values' mean."""
    g = h // (num_q_heads // kv.hkv)
    rows = []
    for p in positions:
        _, v = kv.team(b, g, p // kv.T)
        rows.append(v[p % kv.T])
    return np.mean(np.stack(rows), axis=0)


def evaluate_given_set(kv, q_h, b, h, num_q_heads, teams, inv_pi):
    """Estimate for a supplied team set and weights (used when a near-tie draw
    made the HIP path pick a different but equally valid set)."""
    g = h // (num_q_heads // kv.hkv)
    return estimate(q_h, [kv.team(b, g, t) for t in teams], list(inv_pi))


def dense_head(kv, q_h, b, h, num_q_heads):
    g = h // (num_q_heads // kv.hkv)
    k, v = kv.all_tokens(b, g)
    return dense_attention(q_h, k, v)


# ----------------------------------------------------------------------------
# Read accounting and closed forms
# ----------------------------------------------------------------------------

def expected_set_size(p, M):
    """E|S| = sum_t pi_t for M draws with replacement (closed form of R4)."""
    if M >= len(p):
        return float(len(p))
    return math.fsum(inclusion_probability(x, M) for x in p)


def expected_union_size(p_heads, M):
    """E|union over heads of S_h| = sum_t (1 - prod_h (1 - p_ht)^M), independent heads (R7)."""
    K = len(p_heads[0])
    if M >= K:
        return float(K)
    total = []
    for t in range(K):
        miss = 1.0
        for p in p_heads:
            miss *= math.exp(M * math.log1p(-p[t]))
        total.append(1.0 - miss)
    return math.fsum(total)

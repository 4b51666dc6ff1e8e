"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE (see the package docstring).

[PHX] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2,
3" (SC'11), Philox family: a 4-word counter and a 2-word key; each round
multiplies counter words 0 and 2 by two fixed 32-bit multipliers, keeps the
high and low halves of the 64-bit products, xors the high halves with the
other two counter words and the key, and permutes; the key is bumped by two
fixed Weyl constants between rounds. Ten rounds.

Pinned by the published known-answer vectors in tests/golden/.

How SANTA++ draws are laid out over the generator is this library's own
convention (the pages say only that teams are sampled at random with
probability p_i): draw j of query head h of sequence b at step ``offset``
takes word (j mod 4) of Philox4x32-10 with counter (j div 4, h, b, offset)
and key (seed low 32 bits, seed high 32 bits).
"""
MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10


def _mulhilo(a, b):
    """Full 64-bit product of two 32-bit words, split into (high, low)."""
    p = (a & MASK32) * (b & MASK32)
    return (p >> 32) & MASK32, p & MASK32


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words.

    [PHX] Philox round: (hi0, lo0) = mulhilo(M0, c0); (hi1, lo1) =
    mulhilo(M1, c2); new counter = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).
    Key schedule: k0 += W0, k1 += W1 (mod 2^32) before every round after the
    first.
    """
    c0, c1, c2, c3 = (int(x) & MASK32 for x in ctr)
    k0, k1 = (int(x) & MASK32 for x in key)
    for r in range(ROUNDS):
        if r > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & MASK32, lo1, (hi0 ^ c3 ^ k1) & MASK32, lo0
    return c0, c1, c2, c3


def draw_words(num_draws, seed, offset, b, h):
    """The 32-bit words for draws 0..num_draws-1 of query head h of sequence b.

    Convention (this library's; see the module docstring): draw j takes word
    j mod 4 of the block with counter (j div 4, h, b, offset), key = (seed lo, seed hi).
    """
    seed = int(seed)
    key = (seed & MASK32, (seed >> 32) & MASK32)
    words = []
    for j in range(num_draws):
        block = philox4x32_10((j // 4, h, b, offset), key)
        words.append(block[j % 4])
    return words


def word_to_uniform(x):
    """Map a 32-bit word x to u = (x + 1/2) * 2^-32, strictly inside (0, 1).

    This library's convention: the half-offset keeps u away from 0 and 1, and
    the value is exact in float64 (33 significant bits at most).
    """
    return (float(x) + 0.5) * (2.0 ** -32)

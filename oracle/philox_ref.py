"""Counter-based dropout bits for the CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library.

What the pages fix and what is read into them
---------------------------------------------
The PyTorch PR "REDO of dropout support for mem eff" (pytorch#103704, Summary)
states two facts about dropout inside a fused attention kernel:

* the forward hands its RNG state to the backward, which regenerates the same
  mask instead of storing it;
* the random stream is indexed by the *absolute* position of a score element,
  not by its position inside a tile (the bug it fixes gave wrong gradients for
  more than 64 keys with dropout and causal masking).

The nvFuser PR "DID loop split for SDPA" (test ``test_sdpa_loop_split``) shows
the forward returning ``seed`` and ``offset`` and the backward taking them.

The pages name no generator and no index formula.  The reading used here:

* generator: Philox-4x32 with 10 rounds, as defined by Salmon, Moraes, Dror and
  Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  The round
  multiplies counter words 0 and 2 by two fixed odd constants, keeps both halves
  of each 64-bit product, and mixes the high halves with the other two counter
  words and the key; the two key words are bumped by two Weyl constants between
  rounds;
* key = (low 32 bits of seed, high 32 bits of seed);
* one Philox call covers four consecutive keys of one query row:
  ``g = ((b*H + h)*Sq + i) * ceil(Sk/4) + j // 4``, counter =
  ``offset + g`` (mod 2**64) split into (low word, high word, 0, 0), and key
  ``j`` uses output word ``j % 4``;
* element (b, h, i, j) is kept iff that word is >= ``floor(p * 2**32)``.

The mask is therefore a pure function of (seed, offset, p, B, H, Sq, Sk, b, h,
i, j), independent of any tiling, which is the property the PR asks for.
"""

from __future__ import annotations

import math

import numpy as np

# Philox-4x32 constants (Salmon et al., SC'11): round multipliers and the key
# schedule's Weyl increments (golden ratio and sqrt(3) - 1, scaled by 2**32).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10

_MASK32 = np.uint64(0xFFFFFFFF)
_SHIFT32 = np.uint64(32)


def philox4x32(c0, c1, c2, c3, k0, k1, rounds: int = PHILOX_ROUNDS):
    """Philox-4x32-R on broadcastable arrays of 32-bit words.

    Arguments are integer scalars or arrays holding values in [0, 2**32).
    Returns the four output words as ``np.uint64`` arrays (values < 2**32).
    The products of two 32-bit words are formed exactly in uint64.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) for c in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64)
    k1 = np.asarray(k1, dtype=np.uint64)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    w0 = np.uint64(PHILOX_W0)
    w1 = np.uint64(PHILOX_W1)
    for rnd in range(rounds):
        if rnd > 0:  # key schedule: bump between rounds
            k0 = (k0 + w0) & _MASK32
            k1 = (k1 + w1) & _MASK32
        prod0 = m0 * c0
        prod1 = m1 * c2
        hi0, lo0 = prod0 >> _SHIFT32, prod0 & _MASK32
        hi1, lo1 = prod1 >> _SHIFT32, prod1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def drop_threshold(p: float) -> int:
    """floor(p * 2**32): a word below it drops its element (exact in double)."""
    if not (0.0 <= p < 1.0):
        raise ValueError(f"dropout probability must lie in [0, 1), got {p}")
    return int(math.floor(p * 4294967296.0))


def group_index(B: int, H: int, Sq: int, Sk: int, b, h, i, j):
    """Absolute Philox group ``g`` of element (b, h, i, j); integer math, uint64."""
    sk4 = (Sk + 3) // 4
    b = np.asarray(b, dtype=np.uint64)
    h = np.asarray(h, dtype=np.uint64)
    i = np.asarray(i, dtype=np.uint64)
    j = np.asarray(j, dtype=np.uint64)
    return ((b * np.uint64(H) + h) * np.uint64(Sq) + i) * np.uint64(sk4) + j // np.uint64(4)


def element_words(seed: int, offset: int, B: int, H: int, Sq: int, Sk: int, b, h, i, j):
    """The 32-bit Philox word that decides element (b, h, i, j)."""
    g = group_index(B, H, Sq, Sk, b, h, i, j)
    with np.errstate(over="ignore"):
        ctr = np.uint64(offset % 2**64) + g  # wraps modulo 2**64
    seed = int(seed) % 2**64
    words = philox4x32(ctr & _MASK32, ctr >> _SHIFT32, 0, 0, seed & 0xFFFFFFFF, seed >> 32)
    stacked = np.stack(np.broadcast_arrays(*words), axis=0)  # [4, ...]
    sel = np.broadcast_to(np.asarray(j, dtype=np.int64) % 4, stacked.shape[1:])
    return np.take_along_axis(stacked, sel[None, ...], axis=0)[0]


def keep_mask_head(seed: int, offset: int, p: float, B: int, H: int, Sq: int, Sk: int,
                   b: int, h: int, rows=None) -> np.ndarray:
    """Boolean keep mask [len(rows), Sk] of head (b, h); ``rows`` defaults to all queries."""
    t = drop_threshold(p)
    i = np.arange(Sq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(Sk, dtype=np.int64)
    words = element_words(seed, offset, B, H, Sq, Sk, b, h, i[:, None], j[None, :])
    return words >= np.uint64(t)


def keep_mask(seed: int, offset: int, p: float, B: int, H: int, Sq: int, Sk: int) -> np.ndarray:
    """Boolean keep mask [B, H, Sq, Sk] for the whole problem."""
    out = np.empty((B, H, Sq, Sk), dtype=bool)
    for b in range(B):
        for h in range(H):
            out[b, h] = keep_mask_head(seed, offset, p, B, H, Sq, Sk, b, h)
    return out


def offset_advance(B: int, H: int, Sq: int, Sk: int) -> int:
    """Counter values one forward with dropout consumes: one per four keys of each row."""
    return B * H * Sq * ((Sk + 3) // 4)

"""Pins for the oracle's Philox generator and dropout keep mask (CPU only).

* Known-answer vectors of Philox-4x32-10 (Random123, the SC'11 authors'
  reference implementation) -- ``tests/golden/philox4x32_10_kat.txt``.
* rocRAND's own Philox-4x32-10 (a library in this image), driven from the host
  through ``tests/rocrand_philox_words.cpp``, on random keys and counters.
* The index convention (a reading) against hand-worked examples in
  ``tests/golden/dropout_group_index.txt``.
* Statistics of the keep mask and its dependence on seed and offset.
"""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import philox_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_known_answer_vectors():
    for row in _golden_rows("philox4x32_10_kat.txt"):
        w = [int(x, 16) for x in row]
        out = philox_ref.philox4x32(w[0], w[1], w[2], w[3], w[4], w[5])
        assert [int(x) for x in out] == w[6:10]


@pytest.fixture(scope="module")
def rocrand_words(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc or rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("rocrand") / "philox_words")
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox_words.cpp")
    subprocess.run([hipcc, "-O1", src, "-o", exe], check=True, timeout=300,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)

    def run(pairs):
        text = "".join(f"{s} {c}\n" for s, c in pairs)
        res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True,
                             timeout=60)
        return [[int(x, 16) for x in ln.split()] for ln in res.stdout.strip().splitlines()]

    return run


def test_matches_rocrand(rocrand_words):
    rng = np.random.default_rng(7)
    seeds = [0, 1, 1234, 2**64 - 1] + [int(x) for x in rng.integers(0, 2**63, 60)]
    ctrs = [0, 1, 2**32 - 1, 2**32, 2**62 - 1] + [int(x) for x in rng.integers(0, 2**62, 59)]
    pairs = list(zip(seeds, ctrs))
    expect = rocrand_words(pairs)
    s = np.array([p[0] for p in pairs], dtype=np.uint64)
    c = np.array([p[1] for p in pairs], dtype=np.uint64)
    m = np.uint64(0xFFFFFFFF)
    got = philox_ref.philox4x32(c & m, c >> np.uint64(32), 0, 0, s & m, s >> np.uint64(32))
    got = np.stack(got, axis=1).astype(np.int64).tolist()
    assert got == expect


def test_group_index_examples():
    for row in _golden_rows("dropout_group_index.txt"):
        B, H, Sq, Sk, b, h, i, j, g, word = (int(x) for x in row)
        assert int(philox_ref.group_index(B, H, Sq, Sk, b, h, i, j)) == g
        assert j % 4 == word


def test_element_words_use_counter_offset_plus_group(rocrand_words):
    # Each worked example, at two offsets, against rocRAND's output at counter offset+g.
    pairs, cases = [], []
    for row in _golden_rows("dropout_group_index.txt"):
        B, H, Sq, Sk, b, h, i, j, g, word = (int(x) for x in row)
        for seed, offset in ((1234, 0), (987654321987, 5 * 2**33 + 17)):
            pairs.append((seed, offset + g))
            cases.append((seed, offset, B, H, Sq, Sk, b, h, i, j, word))
    expect = rocrand_words(pairs)
    for (seed, offset, B, H, Sq, Sk, b, h, i, j, word), words in zip(cases, expect):
        got = int(philox_ref.element_words(seed, offset, B, H, Sq, Sk, b, h, i, j))
        assert got == words[word]


def test_counter_wraps_modulo_2_64():
    # offset + g past 2**64 wraps; the carry into the high word is exact.
    seed, B, H, Sq, Sk = 99, 1, 1, 2, 8
    off = 2**64 - 1
    w_wrap = philox_ref.element_words(seed, off, B, H, Sq, Sk, 0, 0, 0, 4)  # g = 1 -> ctr 0
    w_zero = philox_ref.element_words(seed, 0, B, H, Sq, Sk, 0, 0, 0, 0)    # g = 0 -> ctr 0
    assert int(w_wrap) == int(w_zero)


def test_threshold():
    assert philox_ref.drop_threshold(0.0) == 0
    assert philox_ref.drop_threshold(0.1) == 429496729
    assert philox_ref.drop_threshold(0.5) == 2**31
    for bad in (-0.1, 1.0, 1.5, float("nan")):
        with pytest.raises(ValueError):
            philox_ref.drop_threshold(bad)


def test_keep_fraction_is_binomial():
    p = 0.1
    mask = philox_ref.keep_mask(1234, 0, p, 2, 3, 200, 333)
    n = mask.size
    keep_prob = 1.0 - philox_ref.drop_threshold(p) / 2**32
    mean, sd = n * keep_prob, math.sqrt(n * keep_prob * (1 - keep_prob))
    assert abs(mask.sum() - mean) < 5 * sd
    # Keys inside one Philox call (same group, different word) are not correlated
    # in an obvious way: each word position keeps about the same fraction.
    for w in range(4):
        frac = mask[..., w::4].mean()
        assert abs(frac - keep_prob) < 0.01


def test_zero_p_keeps_everything():
    assert philox_ref.keep_mask(5, 6, 0.0, 1, 2, 17, 19).all()


def test_seed_and_offset_change_the_mask():
    base = philox_ref.keep_mask(1234, 0, 0.3, 1, 2, 64, 70)
    assert not np.array_equal(base, philox_ref.keep_mask(1235, 0, 0.3, 1, 2, 64, 70))
    assert not np.array_equal(base, philox_ref.keep_mask(1234, 1, 0.3, 1, 2, 64, 70))
    assert np.array_equal(base, philox_ref.keep_mask(1234, 0, 0.3, 1, 2, 64, 70))


def test_offset_shift_equals_group_shift():
    # Advancing the offset by one group slides the counter stream by one group:
    # row i, key group c at offset o+1 equals key group c+1 at offset o.
    B, H, Sq, Sk = 1, 1, 4, 16
    a = philox_ref.element_words(77, 1, B, H, Sq, Sk, 0, 0, 2, np.arange(0, 12))
    b = philox_ref.element_words(77, 0, B, H, Sq, Sk, 0, 0, 2, np.arange(4, 16))
    assert np.array_equal(a, b)


def test_offset_advance():
    assert philox_ref.offset_advance(4, 16, 1000, 1000) == 16_000_000
    assert philox_ref.offset_advance(1, 1, 3, 5) == 6

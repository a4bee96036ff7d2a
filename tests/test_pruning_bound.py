"""CPU checks of the arithmetic behind the Gumbel pruning bound of the verify kernel.

The kernel skips scoring a 16-byte chunk when max(x)/T plus an upper bound of the
chunk's noise cannot reach the best score seen. In a full noise group of 8 indices
the bound is the group's maximum, which its group word gives directly; in a partial
last group, whose indices draw on their own, it is taken from the largest index
hash word of the chunk, computed without the finalizer's last step
(x ^= x >> 16): the step keeps the top 16 bits, so the largest word before it, with
its low 16 bits set, is at least every final word of the chunk, and the uniform
u = (2 (h >> 9) + 1) 2^-24, hence the noise, grows with the word. These tests
restate the published MurmurHash3 finalizer (Appleby) in numpy, check the oracle's
mix32 against it, and check the bound on many chunks and on its worst cases. They
run no GPU code.
"""

import numpy as np

from oracle import noise

M32 = np.uint64(0xFFFFFFFF)


def _head(x):
    """The finalizer without its last step, on uint64 arrays holding 32-bit words."""
    x = x ^ (x >> np.uint64(16))
    x = (x * np.uint64(0x85EBCA6B)) & M32
    x = x ^ (x >> np.uint64(13))
    x = (x * np.uint64(0xC2B2AE35)) & M32
    return x


def _full(x):
    h = _head(x)
    return h ^ (h >> np.uint64(16))


def _uniform(h):
    return (2.0 * (h >> np.uint64(9)).astype(np.float64) + 1.0) * 2.0 ** -24


def test_head_is_the_finalizer_without_its_last_step():
    rng = np.random.default_rng(11)
    x = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64)
    want = np.array([int(noise.mix32(int(v))) for v in x[:2000]], dtype=np.uint64)
    np.testing.assert_array_equal(_full(x[:2000]), want)
    # the last step keeps the top 16 bits
    np.testing.assert_array_equal(_full(x) >> np.uint64(16), _head(x) >> np.uint64(16))


def test_chunk_bound_covers_every_word_and_its_noise():
    """For chunks of 8 (bf16) and 4 (fp32) consecutive vocabulary indices under random keys,
    the bound word is at least every final word, so its uniform (and noise) is too."""
    rng = np.random.default_rng(12)
    step = np.uint64(0x9E3779B9)
    for n in (8, 4):
        keys = rng.integers(0, 1 << 32, size=4096, dtype=np.uint64)
        chunks = rng.integers(0, (1 << 31) // n, size=4096, dtype=np.uint64)
        idx = chunks[:, None] * np.uint64(n) + np.arange(n, dtype=np.uint64)[None, :]
        words = keys[:, None] ^ ((idx * step) & M32)
        full = _full(words)
        bound = _head(words).max(axis=1) | np.uint64(0xFFFF)
        assert (bound[:, None] >= full).all()
        assert (_uniform(bound)[:, None] >= _uniform(full)).all()
        # the chunk's largest final word shares the bound's top half, so the bound exceeds it by at
        # most 0xFFFF: u by at most 2 * (0xFFFF >> 9) * 2^-24 < 2^-16
        assert (_uniform(bound) - _uniform(full.max(axis=1)) < 2.0 ** -16).all()


def test_bound_at_the_edges_of_the_word_range():
    """Words whose top half is all ones or all zeros, and chunks whose largest word after the
    last step differs from the largest word before it."""
    xs = np.array([0, 1, 0xFFFF, 0x10000, 0xFFFF0000, 0xFFFFFFFF, 0x7FFFFFFF, 0x80000000], dtype=np.uint64)
    for x in xs:
        h, f = _head(np.array([x]))[0], _full(np.array([x]))[0]
        assert (h | np.uint64(0xFFFF)) >= f
    # two pre-final words with equal top halves: the larger one before the last step may be the
    # smaller one after it; the bound covers both
    rng = np.random.default_rng(13)
    words = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64)
    h = _head(words)
    top = h >> np.uint64(16)
    order = np.argsort(top, kind="stable")
    same = np.nonzero(top[order][1:] == top[order][:-1])[0]
    assert same.size > 0
    a, b = words[order][same], words[order][same + 1]
    pair_head = np.maximum(_head(a), _head(b)) | np.uint64(0xFFFF)
    assert (pair_head >= np.maximum(_full(a), _full(b))).all()

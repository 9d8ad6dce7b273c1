"""The uniform layout stated in include/dflash.h, evaluated from the header's
own text with numpy's independent Philox4x64-10, equals oracle.uniforms: a
caller reproducing verification or draft draws from the header gets the
same uniforms as the oracle (and the kernels, which the GPU tests tie to
the oracle)."""

import os
import re

import numpy as np

import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dflash.h")


def _layout_text():
    text = open(HEADER).read()
    start = text.index("Uniforms: U(s, b, k, i)")
    return text[start:text.index("Stream 0 holds", start)]


def _numpy_block(counter, key):
    """Block at `counter` from numpy.random.Philox, which increments its
    256-bit counter before producing a block (so it starts one below)."""
    v = sum(int(x) << (64 * j) for j, x in enumerate(counter)) - 1
    prev = np.array([(v >> (64 * j)) & ((1 << 64) - 1) for j in range(4)], dtype=np.uint64)
    return np.random.Philox(key=np.array(key, dtype=np.uint64), counter=prev).random_raw(4)


def test_header_states_the_layout():
    t = " ".join(re.sub(r"(?m)^\s*\*", " ", _layout_text()).split())
    for phrase in ("key (seed, 0)", "counter (floor(i / 8), 8b + k, s, offset)",
                   "word floor(i / 2) mod 4", "(w >> 41) & 0x7FFFFF when i is even",
                   "(w >> 9) & 0x7FFFFF when i is odd", "U = (bits + 0.5) * 2^-23"):
        assert phrase in t, phrase
    consts = {int(c, 16) for c in re.findall(r"0x[0-9A-F]{16}", t)}
    assert consts == {0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B}


def _header_uniform(seed, offset, s, b, k, i):
    """U(s, b, k, i) as the header defines it."""
    blk = _numpy_block([i // 8, 8 * b + k, s, offset], [seed, 0])
    w = int(blk[(i // 2) % 4])
    bits = ((w >> 41) if i % 2 == 0 else (w >> 9)) & 0x7FFFFF
    return (bits + 0.5) * 2.0 ** -23


def test_header_formula_equals_oracle_uniforms():
    rng = np.random.default_rng(8)
    for _ in range(40):
        seed = int(rng.integers(0, 2 ** 63))
        offset = int(rng.integers(0, 2 ** 20))
        s = int(rng.integers(0, 3))
        b = int(rng.integers(0, 256))
        k = int(rng.integers(1, 9))
        i = int(rng.integers(0, 262144))
        assert _header_uniform(seed, offset, s, b, k, i) == float(oracle.uniforms(seed, offset, s, b, k, i)), \
            (seed, offset, s, b, k, i)
    # all eight entries of one block, both halves of every word
    for i in range(16):
        assert _header_uniform(3, 1, 1, 2, 5, i) == float(oracle.uniforms(3, 1, 1, 2, 5, i))

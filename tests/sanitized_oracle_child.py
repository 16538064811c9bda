"""Child process of test_oracle_sanitizers.py: the pin battery and exhaustive
tiny cases against an oracle library built with AddressSanitizer and
UndefinedBehaviorSanitizer (path in argv[1]).  Started with the ASan runtime
preloaded; any sanitizer report aborts the process with a non-zero status.
Runs on the CPU only."""
import itertools
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import numpy as np  # noqa: E402

import bruteforce  # noqa: E402
import oracle  # noqa: E402
import pins  # noqa: E402


def main(path):
    orc = oracle.Oracle(path)
    for check in pins.ALL_CHECKS:
        check(orc)
    n = 0
    for Lq, Lk in [(1, 1), (1, 4), (3, 2), (4, 4), (6, 5), (2, 6)]:
        rng = np.random.default_rng(100 * Lq + Lk)
        q = rng.standard_normal((2, 2, Lq, 3))
        k = rng.standard_normal((2, 2, Lk, 3))
        v = rng.standard_normal((2, 2, Lk, 2))
        lengths = list(range(-1, Lk + 2))
        for causal, (l0, l1) in itertools.product((False, True), zip(lengths, reversed(lengths))):
            for radius in (None, 0, 1, Lk):
                got = orc.attention(q, k, v, key_lengths=[l0, l1], causal=causal, radius=radius)
                ref = np.array(bruteforce.attention(q, k, v, [l0, l1], causal, radius))
                assert np.max(np.abs(got - ref)) <= 1e-12, (Lq, Lk, causal, l0, l1, radius)
                rows = np.array([(b, h, i) for b in range(2) for h in range(2) for i in range(Lq)])
                got_r, _ = orc.attention_rows(q, k, v, rows, key_lengths=[l0, l1], causal=causal,
                                              radius=radius)
                assert np.max(np.abs(got_r - got.reshape(-1, 2))) == 0.0
                n += 1
    xq = np.random.default_rng(5).standard_normal((2, 4, 6))
    ws = [np.random.default_rng(6 + i).standard_normal(s)
          for i, s in enumerate(((6, 4), (6, 4), (6, 4), (4, 6)))]
    for causal in (False, True):
        got = orc.multihead(xq, xq, *ws, 2, key_lengths=[4, 1], causal=causal)
        ref = np.array(bruteforce.multihead(xq, xq, *ws, 2, [4, 1], causal))
        assert np.max(np.abs(got - ref)) <= 1e-10 * max(1.0, np.abs(ref).max())
        rows = np.array([(b, i) for b in range(2) for i in range(4)])
        got_r = orc.multihead_rows(xq, xq, *ws, 2, rows, key_lengths=[4, 1], causal=causal)
        assert np.max(np.abs(got_r - got.reshape(-1, 6))) == 0.0
    print("sanitized oracle: %d pins, %d tiny cases ok" % (len(pins.ALL_CHECKS), n), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])

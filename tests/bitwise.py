"""Bit-for-bit comparison of arrays with a short failure message.

pytest's own explanation of a failed ``a.tobytes() == b.tobytes()`` diffs the
two byte strings line by line; for arrays of a megabyte or more that runs for
minutes without printing anything, so tests compare through this instead.
"""
import numpy as np


def _raw(x):
    return np.frombuffer(np.ascontiguousarray(x).tobytes(), np.uint8)


def assert_same_bytes(first, *others, what=""):
    """Every array in ``others`` holds exactly the bytes of ``first``."""
    a = _raw(first)
    for i, other in enumerate(others):
        b = _raw(other)
        label = "%s[%d]" % (what or "arrays", i + 1)
        if a.size != b.size:
            raise AssertionError("%s: %d bytes against %d" % (label, b.size, a.size))
        bad = np.flatnonzero(a != b)
        if bad.size:
            raise AssertionError("%s: %d of %d bytes differ, the first at byte %d"
                                 % (label, bad.size, a.size, bad[0]))

"""Helpers for the CPU tests of the C ABI: fake address layouts and a checker
of the kernels' replayed address walk."""
import numpy as np

TAG = np.uint64(1) << np.uint64(63)
ESIZE = {0: 4, 1: 2, 2: 2}


def fake_layout(rng, numels, esize, misalign=True, base=1 << 20):
    """Non-overlapping device-like addresses; starts at random multiples of
    the element size (or 256-byte aligned when misalign is False)."""
    addrs = []
    a = base
    for n in numels:
        a = (a + 255) // 256 * 256
        if misalign:
            a += int(rng.integers(0, 16 // esize)) * esize
        addrs.append(a)
        a += n * esize + int(rng.integers(0, 4)) * 256
    return addrs


def check_walk(trace_addrs, addrs, numels, esize):
    """Every access lies inside a tensor, no two overlap, and together they
    cover every byte of every tensor exactly once."""
    tagged = (trace_addrs & TAG) != 0
    start = (trace_addrs & ~TAG).astype(np.uint64)
    length = np.where(tagged, esize, 16).astype(np.uint64)
    assert np.all(start[~tagged] % 16 == 0), "vector access not 16-byte aligned"
    order = np.argsort(start, kind="stable")
    s, l = start[order], length[order]
    if len(s) > 1:
        assert np.all(s[1:] >= s[:-1] + l[:-1]), "two accesses overlap"
    t_start = np.array([a for a, n in zip(addrs, numels) if n > 0], dtype=np.uint64)
    t_end = np.array([a + n * esize for a, n in zip(addrs, numels) if n > 0], dtype=np.uint64)
    o = np.argsort(t_start)
    t_start, t_end = t_start[o], t_end[o]
    if len(s):
        idx = np.searchsorted(t_start, s, side="right") - 1
        assert np.all(idx >= 0), "access below every tensor"
        assert np.all(s >= t_start[idx]) and np.all(s + l <= t_end[idx]), "access outside its tensor"
    assert int(l.sum()) == int(sum(n * esize for n in numels)), "bytes covered != bytes in the list"

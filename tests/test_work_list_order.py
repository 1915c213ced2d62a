"""The split kernels' in-kernel work list (dispatch order 4), written out on
the host step for step as the device derives it, one sequence per lane: an
inclusive scan of the full-split counts places the full units; the partial
last splits are ranked by the key ((tokens - 1) / 16 + 1) * 64 + (63 - b)
and the j-th largest is selected bit by bit.  Pinned against what the list
must be: every (sequence, split) unit that holds a token exactly once, full
units first in sequence order, then the partial ones longest 16-token bucket
first, ties by sequence.  (The GPU test compares the device's order 4 with
the order-3 list built by its own kernel, bit for bit.)"""
import numpy as np


def derive(lengths, chunk, max_len, n_slots):
    B = len(lengths)
    assert B <= 64
    L = np.zeros(64, np.int64)
    L[:B] = np.clip(lengths, 0, max_len)
    n = (L + chunk - 1) // chunk
    full = np.where((n > 0) & (L - (n - 1) * chunk == chunk), n, np.maximum(n - 1, 0))
    part = np.where(n > full, L - (n - 1) * chunk, 0)
    incl = np.cumsum(full)
    n_full = int(incl[63])
    lane = np.arange(64)
    key = np.where(part > 0, ((((part - 1) >> 4) + 1) << 6) | (63 - lane), 0)
    units = []
    for k in range(n_slots):
        if k < n_full:
            hit = np.flatnonzero((incl - full <= k) & (k < incl))
            assert hit.size == 1
            b = int(hit[0])
            units.append((b, int(k - (incl[b] - full[b]))))
            continue
        cand = part > 0
        j = k - n_full
        if j >= cand.sum():
            continue                        # past the list: the workgroup exits
        for bit in range(15, -1, -1):
            ones = cand & (((key >> bit) & 1) == 1)
            c1 = int(ones.sum())
            if j < c1:
                cand = ones
            else:
                j -= c1
                cand = cand & ~ones
        assert cand.sum() == 1
        b = int(np.flatnonzero(cand)[0])
        units.append((b, int(full[b])))
    return units


def expected(lengths, chunk, max_len):
    L = np.clip(lengths, 0, max_len)
    full = [(b, s) for b in range(len(L)) for s in range(int(L[b]) // chunk)]
    part = [(b, int(L[b]) // chunk) for b in range(len(L)) if L[b] % chunk]
    part.sort(key=lambda u: (-((int(L[u[0]]) - u[1] * chunk - 1) >> 4), u[0]))
    return full + part


def test_random_batches_give_the_list():
    rng = np.random.default_rng(7)
    for _ in range(300):
        B = int(rng.integers(2, 65))
        chunk = int(rng.choice([16, 64, 128, 1024, 2048, 8192]))
        max_len = int(rng.integers(1, 20000))
        lengths = rng.integers(0, max_len + 1, B)
        n_splits = (max_len + chunk - 1) // chunk
        got = derive(lengths, chunk, max_len, B * n_splits)
        assert got == expected(lengths, chunk, max_len)


def test_ties_empty_and_exact_multiples():
    lengths = np.array([0, 1, 16, 17, 1024, 2048, 1040, 1041, 1056, 17, 16, 0, 2047], np.int64)
    got = derive(lengths, 1024, 2048, len(lengths) * 2)
    assert got == expected(lengths, 1024, 2048)
    # sequences 1 and 10 (1 and 16 tokens) share a bucket: sequence order decides
    tail = [u for u in got if u[0] in (1, 10)]
    assert tail == [(1, 0), (10, 0)]

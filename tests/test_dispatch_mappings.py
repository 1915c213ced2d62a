"""Two device-side index mappings written out on the host step for step, and
pinned against what they must be.

1. The prefill's balanced XCD runs (order 8 with up to 64 sequences, a
   multiple of the XCD count): each lane ranks its sequence's clamped length
   (longer first, ties by index), and slot s of run x = s / (B / n_xcd),
   position j, takes the sequence of rank j * n_xcd + x (j even) or
   j * n_xcd + n_xcd - 1 - x (j odd).  It must be a permutation of the
   sequences, and it must even out the runs' summed lengths: never worse
   than the longest single sequence above the mean, and on the ragged c3
   batch within a few percent.

2. The append's vector kernel: item i of a token is four rotation pairs of
   a q or k head row or eight v elements.  Its two runs of four elements
   must cover every element of every row exactly once, and pair k of item
   c must be the scalar kernel's pair 4c + k (elements 2f, 2f + 1 when
   interleaved; f, f + D/2 for half pairs), which uses factor f.  The
   slices must hand every item to exactly one thread.  (The GPU test holds
   both kernels to the same bits.)
"""
import itertools

import numpy as np
import pytest

from kv_cache_gqa_decode_amd import workloads as W


def balanced_order(lengths, max_len, n_xcd):
    B = len(lengths)
    assert B <= 64 and B % n_xcd == 0
    L = np.clip(np.asarray(lengths, np.int64), 0, max_len)
    lane = np.arange(B)
    rank = np.array([np.sum((L > L[l]) | ((L == L[l]) & (lane < l))) for l in range(B)])
    per = B // n_xcd
    order = []
    for slot in range(B):
        x, j = divmod(slot, per)
        r = j * n_xcd + ((n_xcd - 1 - x) if j & 1 else x)
        hit = np.flatnonzero(rank == r)
        assert hit.size == 1
        order.append(int(hit[0]))
    return order


def run_sums(lengths, order, n_xcd):
    per = len(order) // n_xcd
    L = np.asarray(lengths, np.int64)
    return np.array([L[order[x * per:(x + 1) * per]].sum() for x in range(n_xcd)])


@pytest.mark.parametrize("B,n_xcd", [(8, 8), (16, 8), (64, 8), (64, 4), (24, 8), (6, 2)])
def test_balanced_runs_are_a_permutation(B, n_xcd):
    rng = np.random.default_rng(B * 10 + n_xcd)
    for trial in range(20):
        lengths = rng.integers(-3, 50, B)       # ties, negatives (clamped to 0)
        order = balanced_order(lengths, 40, n_xcd)
        assert sorted(order) == list(range(B))


def test_balanced_runs_even_out_the_c3_batch():
    s = W.spec("c3")
    L = np.clip(W.draw_lengths(s), 512, s.max_seq_len) - 512 + 272   # work per sequence
    ident = run_sums(L, list(range(64)), 8)
    bal = run_sums(L, balanced_order(L, 1 << 30, 8), 8)
    assert ident.max() / ident.mean() > 1.15     # batch order: one XCD a fifth over the mean
    assert bal.max() / bal.mean() < 1.03


def test_balanced_runs_bound():
    """Dealing back and forth by rank keeps every run within the longest
    length of the mean (a bound of the snake order), on random batches."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        B = 8 * int(rng.integers(1, 9))
        L = rng.integers(0, 10000, B)
        sums = run_sums(L, balanced_order(L, 1 << 30, 8), 8)
        assert sums.max() - sums.mean() <= L.max()


def vec_items(H, G, D, inter, with_q=True):
    """(kind, head, [8 element indices], [4 (ia, ib, factor)]) per item."""
    N8, HALF = D // 8, D // 2
    nq = H * N8 if with_q else 0
    nrot = nq + G * N8
    items = []
    for i in range(nrot + G * N8):
        j = i if i < nq else (i - nq if i < nrot else i - nrot)
        head, c = divmod(j, N8)
        rot = i < nrot
        o1 = 4 * c if (rot and not inter) else 8 * c
        o2 = 4 * c + HALF if (rot and not inter) else 8 * c + 4
        xs = [o1 + t for t in range(4)] + [o2 + t for t in range(4)]
        pairs = []
        if rot:
            for k in range(4):
                ia, ib = (2 * k, 2 * k + 1) if inter else (k, 4 + k)
                pairs.append((xs[ia], xs[ib], 4 * c + k))
        kind = "q" if i < nq else ("k" if rot else "v")
        items.append((kind, head, xs, pairs))
    return items


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("inter", [True, False])
@pytest.mark.parametrize("H,G", [(1, 1), (8, 2), (12, 4), (32, 8), (32, 32)])
def test_vector_append_items(D, inter, H, G):
    seen = set()
    for kind, head, xs, pairs in vec_items(H, G, D, inter):
        for e in xs:
            assert 0 <= e < D and (kind, head, e) not in seen
            seen.add((kind, head, e))
        for ea, eb, f in pairs:
            assert (ea, eb) == ((2 * f, 2 * f + 1) if inter else (f, f + D // 2))
    counts = {"q": H, "k": G, "v": G}
    assert len(seen) == D * sum(counts.values())


def slices(tokens, nrot, nv, rot_workgroups=1024):
    if tokens >= 4096:
        return 1, 1
    rmax = (nrot + 255) // 256
    want = (rot_workgroups + tokens - 1) // tokens
    R = max(1, min(want, rmax))
    return R, R + (nv + 255) // 256


@pytest.mark.parametrize("D,H,G", [(64, 8, 2), (128, 32, 8), (128, 64, 8), (128, 32, 32)])
@pytest.mark.parametrize("with_q", [True, False])
def test_append_slices_cover_every_item_once(D, H, G, with_q):
    N8 = D // 8
    nq = H * N8 if with_q else 0
    for unit, nv in ((N8, G * N8), (N8, G * D)):      # v per token, or by 16-token groups
        nrot = nq + G * N8
        nall = nrot + nv
        for tokens in (1, 64, 320, 512, 1000, 4096):
            R, ny = slices(tokens, nrot, nv)
            cnt = np.zeros(nall, np.int64)
            for ys in range(ny):
                split = R < ny
                first = nrot + (ys - R) * 256 if split and ys >= R else ys * 256
                stride = 256 * ((R if ys < R else ny - R) if split else ny)
                end = nrot if split and ys < R else nall
                for tid in range(256):
                    cnt[first + tid:end:stride] += 1
            assert (cnt == 1).all(), (tokens, R, ny)


def test_group_runs_partition_a_chunk():
    """INT8 v by 16-token groups: the tokens that start a run (the chunk's
    first, or one at a multiple of 16) and their run lengths cover the
    chunk's tokens exactly once, each run inside one group."""
    for P, T in itertools.product((0, 7, 15, 16, 100, 248), (16, 17, 40, 512)):
        covered = []
        for t in range(T):
            pos = P + t
            if t == 0 or pos % 16 == 0:
                cnt = min(16 - pos % 16, T - t)
                assert (pos // 16) == ((pos + cnt - 1) // 16)
                covered.extend(range(t, t + cnt))
        assert covered == list(range(T))

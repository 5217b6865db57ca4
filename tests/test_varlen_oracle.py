"""Pins of the chunk-metadata definition (oracle/varlen.py).

The definition (_packed_metadata on the hyper-parallel Diff Coverage page) is
checked against a brute-force enumeration that labels every token with its
(sequence, token // 64) pair and keeps the distinct labels in order."""
import random

import pytest

from oracle import varlen


def brute(offsets, chunk=64):
    seen = []
    for seq, (a, b) in enumerate(zip(offsets, offsets[1:])):
        for t in range(a, b):
            lab = (seq, (t - a) // chunk)
            if not seen or seen[-1] != lab:
                seen.append(lab)
    return seen


@pytest.mark.parametrize("lens", [[1], [63], [64], [65], [1, 1, 1], [128, 1, 64, 65, 200],
                                  [4000] * 3 + [100]])
def test_chunk_indices_match_brute_force(lens):
    offs = [0]
    for x in lens:
        offs.append(offs[-1] + x)
    assert varlen.chunk_indices(offs) == brute(offs)
    co = varlen.chunk_offsets(offs)
    assert co[-1] == len(brute(offs))
    assert all(co[i + 1] - co[i] == -(-lens[i] // 64) for i in range(len(lens)))


def test_random_offsets():
    rnd = random.Random(5)
    for _ in range(50):
        lens = [rnd.randint(1, 300) for _ in range(rnd.randint(1, 20))]
        offs = [0]
        for x in lens:
            offs.append(offs[-1] + x)
        assert varlen.chunk_indices(offs) == brute(offs)


def test_offset_rules():
    assert varlen.valid_offsets([0, 5, 9], 9)
    assert not varlen.valid_offsets([0], 0)            # fewer than two entries
    assert not varlen.valid_offsets([1, 5, 9], 9)      # does not start at 0
    assert not varlen.valid_offsets([0, 5, 8], 9)      # does not end at the token count
    assert not varlen.valid_offsets([0, 5, 5, 9], 9)   # empty sequence
    assert not varlen.valid_offsets([0, 6, 5, 9], 9)   # decreasing
    assert not varlen.valid_offsets([0, True, 9], 9)   # bools are not offsets
    assert not varlen.valid_offsets([0, 4.0, 9], 9)    # floats are not offsets


def brute_pieces(docs, segs):
    """Label every token with (document, segment) and keep the runs."""
    offs, pdoc, pseg = [], [], []
    total = docs[-1]
    for t in range(total):
        lab = (sum(1 for o in docs[1:] if o <= t), sum(1 for o in segs[1:] if o <= t))
        if not pdoc or (pdoc[-1], pseg[-1]) != lab:
            offs.append(t)
            pdoc.append(lab[0])
            pseg.append(lab[1])
    return offs + [total], pdoc, pseg


@pytest.mark.parametrize("docs,segs", [([0, 10], [0, 10]), ([0, 10], [0, 3, 7, 10]), ([0, 3, 7, 10], [0, 10]),
                                       ([0, 4, 10], [0, 4, 10]), ([0, 5, 10], [0, 4, 6, 10]),
                                       ([0, 1, 2, 3], [0, 2, 3])])
def test_split_pieces_small(docs, segs):
    assert varlen.split_pieces(docs, segs) == brute_pieces(docs, segs)


def test_split_pieces_random():
    rnd = random.Random(9)
    for _ in range(200):
        total = rnd.randint(1, 400)
        cut = lambda n: [0] + sorted(rnd.sample(range(1, total), min(n, total - 1))) + [total]
        docs, segs = cut(rnd.randint(0, 12)), cut(rnd.randint(0, 6))
        po, pd, ps = varlen.split_pieces(docs, segs)
        assert (po, pd, ps) == brute_pieces(docs, segs)
        # a piece continues its predecessor exactly when it does not start a document
        for p in range(1, len(pd)):
            assert (pd[p] == pd[p - 1]) == (po[p] not in docs)

"""Chunk metadata for packed variable-length input (test infrastructure only).

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU baseline leg
of the benchmark may import this module. It shares no code with the HIP
library.

Definition followed: ``_packed_metadata`` / ``_packed_offsets`` on the
hyper-parallel "Diff Coverage" page. Offsets must be integers that start at 0,
end at the packed token count and strictly increase; every sequence of length
``L`` contributes ``ceil(L / 64)`` chunks, listed in sequence order as
``(sequence index, chunk index within the sequence)`` pairs.
"""
from __future__ import annotations


def valid_offsets(offsets, total_tokens: int) -> bool:
    """The offset rules of ``_packed_offsets``: ints only (no bools), at least
    two entries, first 0, last ``total_tokens``, strictly increasing."""
    offs = list(offsets)
    if len(offs) < 2:
        return False
    if any(isinstance(x, bool) or not isinstance(x, int) for x in offs):
        return False
    if offs[0] != 0 or offs[-1] != total_tokens:
        return False
    return all(a < b for a, b in zip(offs, offs[1:]))


def chunk_indices(offsets, chunk_size: int = 64) -> list[tuple[int, int]]:
    """(sequence, chunk-in-sequence) pairs, sequence-major."""
    out = []
    for seq, (start, end) in enumerate(zip(offsets, offsets[1:])):
        n = (end - start + chunk_size - 1) // chunk_size
        for c in range(n):
            out.append((seq, c))
    return out


def chunk_offsets(offsets, chunk_size: int = 64) -> list[int]:
    """Index of the first chunk of every sequence, plus the total chunk count."""
    out = [0]
    for start, end in zip(offsets, offsets[1:]):
        out.append(out[-1] + (end - start + chunk_size - 1) // chunk_size)
    return out


def split_pieces(doc_offsets, seg_offsets):
    """Pieces of packed documents cut into segments.

    The packed context-parallel plan on the Diff Coverage page gives every
    rank's share of the token axis a head window (the end of a document begun
    on an earlier rank), whole documents, and a tail window (the start of a
    document that goes on to a later rank). Over the whole axis this is the
    list of token ranges between consecutive cuts, where the cuts are all
    document boundaries and all segment boundaries. Returns
    ``(piece_offsets, piece_doc, piece_seg)``; a piece continues its
    predecessor exactly when both have the same document."""
    total = doc_offsets[-1]
    if not valid_offsets(doc_offsets, total) or not valid_offsets(seg_offsets, total):
        raise ValueError("bad offsets")
    cuts = sorted(set(doc_offsets) | set(seg_offsets))
    docs, segs = [], []
    for start in cuts[:-1]:
        # the document / segment holding the piece's first token
        docs.append(max(i for i, o in enumerate(doc_offsets[:-1]) if o <= start))
        segs.append(max(i for i, o in enumerate(seg_offsets[:-1]) if o <= start))
    return cuts, docs, segs

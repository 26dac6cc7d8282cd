"""Host-side model of the append kernels' stage ownership (CPU, no GPU).

The value and MLA latent append kernels keep one open block per sequence in the stage.
Inside one call only the workgroup of a sequence's first block in the batch touches that
sequence's stage rows: it reads the rows earlier calls left and then writes the rows of the
chunk's last block when that block stays incomplete, also when it is a later block (the case
where a chunk starts inside a block and ends inside a later one: chunked prefill or a
multi-token append that crosses a block boundary).  This model restates the kernels' rules
(block leaders, chunk_first / continues, the probing search for the chunk's end) and checks,
for random batches of such chunks, that no stage row is read by one workgroup and written by
another, and that the rows left in the stage are those of each sequence's open block.
"""
import numpy as np
import pytest


def chunk_end(seq_ids, i0, nthr):
    """The kernels' search: probes nthr evenly spaced indices of the open range per round."""
    s = seq_ids[i0]
    lo, hi, rounds = i0, len(seq_ids), 0
    while hi - lo > 1:
        step = (hi - lo - 1 + nthr - 1) // nthr
        cnt = sum(1 for t in range(nthr) if lo + step * (t + 1) < hi and seq_ids[lo + step * (t + 1)] == s)
        lo = lo + step * cnt
        hi = min(hi, lo + step)
        rounds += 1
    return hi, rounds


def simulate(seq_ids, positions, B, nthr):
    """Per workgroup (leading token): the stage rows it reads and writes, per sequence."""
    n = len(seq_ids)
    reads, writes = {}, {}
    for i in range(n):
        s, pos = seq_ids[i], positions[i]
        if not (i == 0 or seq_ids[i - 1] != s or pos % B == 0):
            continue
        bstart = pos - pos % B
        first = pos - bstart
        k = 1
        while i + k < n and seq_ids[i + k] == s and positions[i + k] < bstart + B:
            k += 1
        chunk_first = i == 0 or seq_ids[i - 1] != s
        continues = i + k < n and seq_ids[i + k] == s
        r = {(s, row) for row in range(first)}
        w = set()
        if chunk_first and not continues and first + k < B:
            w = {(s, row) for row in range(first, first + k)}
        if chunk_first and continues:
            i1, _ = chunk_end(seq_ids, i, nthr)
            pos_last = positions[i1 - 1]
            tn = pos_last % B + 1
            ti = i1 - tn
            if tn < B and ti > i and positions[ti] == pos_last - (tn - 1):
                w = {(s, row) for row in range(tn)}
        reads[i], writes[i] = r, w
    return reads, writes


@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("nthr", [128, 512, 7])
def test_stage_rows_have_one_owner_per_call(B, nthr):
    rng = np.random.default_rng(40 + B + nthr)
    for trial in range(60):
        nseq = int(rng.integers(1, 6))
        held = rng.integers(0, 3 * B, size=nseq)        # tokens already in the cache
        new = rng.integers(0, 4 * B, size=nseq)         # tokens appended by this call
        seq_ids, positions = [], []
        for s in range(nseq):
            seq_ids += [s] * int(new[s])
            positions += list(range(int(held[s]), int(held[s] + new[s])))
        if not seq_ids:
            continue
        reads, writes = simulate(seq_ids, positions, B, nthr)
        owner = {}
        for i in reads:
            for row in reads[i] | writes[i]:
                assert owner.setdefault(row, i) == i, (trial, row, owner[row], i)
        # the rows written are exactly the open block of every sequence that ends incomplete
        written = set().union(*writes.values()) if writes else set()
        for s in range(nseq):
            if new[s] == 0:
                continue
            end = int(held[s] + new[s])
            open_rows = {(s, r) for r in range(end % B)} if end % B else set()
            start_block = int(held[s]) - int(held[s]) % B
            if end - end % B == start_block:    # single-block chunk: only its new rows
                open_rows = {(s, r) for r in range(int(held[s]) % B, end % B)}
            assert {x for x in written if x[0] == s} == open_rows, (trial, s)


def test_chunk_end_search_matches_a_scan():
    rng = np.random.default_rng(41)
    for nthr in (1, 2, 7, 128, 512):
        for trial in range(200):
            lens = rng.integers(1, 3000 if nthr > 2 else 300, size=int(rng.integers(1, 5)))
            seq_ids = np.repeat(np.arange(len(lens)), lens)
            i0 = int(rng.integers(0, len(seq_ids)))
            i0 = int(np.searchsorted(seq_ids, seq_ids[i0]))       # a chunk's first token
            want = int(np.searchsorted(seq_ids, seq_ids[i0], side="right"))
            got, rounds = chunk_end(list(seq_ids), i0, nthr)
            assert got == want
            if nthr >= 128:
                assert rounds <= 3

"""Host-side model of the staged epilogues (the forward's `epilogue` and the backward's
`store_rows_staged`): each lane writes its accumulator pieces into the wave's LDS rows, then
the wave reads whole rows back and stores them. The model checks, for head dimensions 64 and
128 and for the query-position order of the dQ-from-dS kernel (position p holds query p with
bits 2 and 3 swapped), that every (row, column) of the wave's 32 rows is written to LDS once
and stored to its global row once, from the value the lane holds for that row and column,
that the staging stays inside the wave's area, and that rows past the sequence end are not
stored. Planted index mistakes fail it.
"""
import pytest

WAVE_ROWS = 32


def swap23(i):
    return (i & ~0b1100) | ((i >> 1) & 0b0100) | ((i << 1) & 0b1000)


def staged_store(D, lrow_of, nvalid, pitch=None, mutate=None):
    """{(global row, column): (lane, value id)} stored by one wave, and the LDS bytes used."""
    pitch = pitch if pitch is not None else 2 * D + 16
    chunks, rows_per = D // 8, 64 // (D // 8)
    lds = {}
    for lane in range(64):
        i, hf = lane & 31, lane >> 5
        lrow = lrow_of(i)
        for cb in range(D // 32):
            for j in range(4):
                for e in range(4):
                    col = 32 * cb + 8 * j + 4 * hf + e
                    if mutate == "hf":
                        col = 32 * cb + 8 * j + e
                    addr = lrow * pitch + 2 * col
                    assert addr not in lds, "an LDS element written twice"
                    lds[addr] = (lrow, col)      # the value of (local row, column) this lane holds
    stored = {}
    for lane in range(64):
        ch = lane % chunks
        for k in range(WAVE_ROWS // rows_per):
            r = k * rows_per + lane // chunks
            if mutate == "rowstep":
                r = k + lane // chunks
            if r >= nvalid:
                continue
            for e in range(8):
                addr = r * pitch + 16 * ch + 2 * e
                key = (r, 8 * ch + e)
                assert key not in stored, "an output element stored twice"
                stored[key] = lds.get(addr)
    return stored, max(lds) + 2


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("order", ["rows", "swap23"])
@pytest.mark.parametrize("nvalid", [32, 17, 1])
def test_every_element_is_stored_once_from_its_own_value(D, order, nvalid):
    lrow_of = (lambda i: i) if order == "rows" else swap23
    stored, used = staged_store(D, lrow_of, nvalid)
    assert used <= WAVE_ROWS * (2 * D + 16)
    assert set(stored) == {(r, c) for r in range(nvalid) for c in range(D)}
    for (r, c), src in stored.items():
        assert src == (r, c), f"row {r} column {c} stored from {src}"


def test_swap23_is_a_permutation_of_the_rows():
    assert sorted(swap23(i) for i in range(32)) == list(range(32))
    assert swap23(4) == 8 and swap23(8) == 4 and swap23(12) == 12 and swap23(3) == 3


@pytest.mark.parametrize("mutate", ["hf", "rowstep"])
def test_planted_mistakes_fail(mutate):
    with pytest.raises(AssertionError):
        stored, _ = staged_store(128, lambda i: i, 32, mutate=mutate)
        assert set(stored) == {(r, c) for r in range(32) for c in range(128)}
        for (r, c), src in stored.items():
            assert src == (r, c)


@pytest.mark.parametrize("D", [64, 128])
def test_padded_row_writes_hit_every_bank_equally(D):
    # one write instruction (block cb, group j): 64 lanes x 8 bytes = 512 bytes, at best two
    # passes over the 64 four-byte banks; the 16-byte row pad gives exactly that
    pitch = 2 * D + 16
    for cb in range(D // 32):
        for j in range(4):
            hits = [0] * 64
            for lane in range(64):
                i, hf = lane & 31, lane >> 5
                word = (i * pitch + 2 * (32 * cb + 8 * j + 4 * hf)) // 4
                hits[word % 64] += 1
                hits[(word + 1) % 64] += 1
            assert hits == [2] * 64
    # without the pad the 32 rows of a half land on one bank (two at D = 64)
    hits = [0] * 64
    for lane in range(64):
        i, hf = lane & 31, lane >> 5
        word = (i * 2 * D + 8 * hf) // 4
        hits[word % 64] += 1
    assert max(hits) == (32 if D == 128 else 16)

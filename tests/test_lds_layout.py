"""Host-side checks of the LDS row-block layout used by the attention backward
kernels (`csrc/attn_bwd.hip`): the byte offset each lane's transposing read
(ds_read_b64_tr_b16) takes, written out directly, against the short form the
kernels use (one per-lane offset XOR an immediate, plus the k-chunk); and a
model of the LDS banks for both kinds of read of a row block.

Row blocks hold 32 token rows of D bf16 values; 16-byte chunk c of row r sits
at chunk position c ^ rsw(r) (rsw below, as in the kernels). Within each
16-lane group of a transposing read, lane j addresses row kb + j / 4 and
columns n0 + 4·(j mod 4) .. +3; a fragment for column block nb and k-chunk c
reads row bases 16c + 4g and 16c + 8 + 4g (g = lane / 32). A fragment read
(16 bytes per lane) gives lane (l32, g) row l32, chunk 2k + g.

Bank model: 64 banks of 4 bytes (256 bytes per cycle). A 16-byte read is
served 16 lanes per cycle, an 8-byte read 32 lanes per cycle; a cycle's lanes
are conflict-free when the 4-byte words they touch fall in 64 distinct banks.
The model reproduces what the counters measured on the GPU with the earlier
swizzle (rsw(r) = r mod 16 at D = 128): conflicts in the two kernels with
transposing reads (dK, dQ), none in dV (fragment reads only)."""
import pytest


def rsw(D, r):
    q = r // (128 // D)
    return (q ^ (q << 2)) & (D // 8 - 1)


def rsw_before(D, r):
    """The earlier swizzle, which left the transposing reads in conflict."""
    return (r // (128 // D)) & (D // 8 - 1)


def direct(D, lane, nb, c, half, sw=rsw):
    j, g = lane & 15, lane >> 5
    col = nb * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)
    r = 16 * c + 4 * g + (j >> 2) + 8 * half
    return (r * D + (((col >> 3) ^ sw(D, r)) << 3) + (col & 7)) * 2


def short_form(D, lane, nb, c, half):
    o0 = direct(D, lane, 0, 0, 0)
    flip = (((D // 16) << 4) | 16 * D) if half else 0
    return c * 32 * D + (o0 ^ (nb << 6) ^ flip)


def fragment_offset(D, lane, k, sw=rsw):
    row, chunk = lane & 31, 2 * k + (lane >> 5)
    return row * 2 * D + ((chunk ^ sw(D, row)) << 4)


def conflict_free(offsets, nbytes):
    banks = [((o + 4 * w) // 4) % 64 for o in offsets for w in range(nbytes // 4)]
    return len(set(banks)) == len(banks)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_swizzle_keeps_rows_and_bit_fields(D):
    for r in range(32):
        assert 0 <= rsw(D, r) < D // 8
    for r in range(8):  # the identities the short form relies on
        assert rsw(D, r + 8) == rsw(D, r) ^ (D // 16)
        assert rsw(D, r + 16) == rsw(D, r)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_transposing_read_offsets_short_form(D):
    for lane in range(64):
        for nb in range(D // 32):
            for c in range(2):
                for half in range(2):
                    assert short_form(D, lane, nb, c, half) == direct(D, lane, nb, c, half)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_transposing_reads_cover_each_row_block_once(D):
    # the 8-byte pieces read for one 32-token block (all nb, c, halves, lanes)
    # tile the block exactly: every byte once, nothing outside it
    seen = set()
    for lane in range(64):
        for nb in range(D // 32):
            for c in range(2):
                for half in range(2):
                    o = direct(D, lane, nb, c, half)
                    assert 0 <= o and o + 8 <= 32 * D * 2
                    seen.add(o)
    assert len(seen) == 32 * D * 2 // 8


@pytest.mark.parametrize("D", [32, 64, 128])
def test_fragment_reads_cover_rows_and_are_conflict_free(D):
    for k in range(D // 16):
        offs = [fragment_offset(D, lane, k) for lane in range(64)]
        # lane (l32, g) gets exactly row l32, logical chunk 2k + g
        for lane, o in enumerate(offs):
            row, pos = divmod(o, 2 * D)
            assert row == lane & 31 and (pos >> 4) ^ rsw(D, row) == 2 * k + (lane >> 5)
        for p in range(4):
            assert conflict_free(offs[16 * p:16 * p + 16], 16), (D, k, p)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_transposing_reads_are_conflict_free(D):
    for nb in range(D // 32):
        for c in range(2):
            for half in range(2):
                offs = [direct(D, lane, nb, c, half) for lane in range(64)]
                for p in range(2):
                    assert conflict_free(offs[32 * p:32 * p + 32], 8), (D, nb, c, half, p)


@pytest.mark.parametrize("D", [64, 128])
def test_the_bank_model_sees_the_earlier_conflicts(D):
    # the earlier swizzle: fragment reads conflict-free, transposing reads not
    for k in range(D // 16):
        offs = [fragment_offset(D, lane, k, rsw_before) for lane in range(64)]
        assert all(conflict_free(offs[16 * p:16 * p + 16], 16) for p in range(4))
    offs = [direct(D, lane, 0, 0, 0, rsw_before) for lane in range(64)]
    assert not conflict_free(offs[:32], 8)

"""Host-side checks of the LDS row-block layout used by the attention backward
kernels (`csrc/attn_bwd.hip`): the byte offset each lane's transposing read
(ds_read_b64_tr_b16) takes, written out directly, against the short form the
kernels use (one per-lane offset XOR an immediate, plus the k-chunk).

Row blocks hold 32 token rows of D bf16 values; 16-byte chunk c of row r sits
at chunk position c ^ rsw(r), rsw(r) = (r / (128 / D)) mod (D / 8). Within
each 16-lane group of a read, lane j addresses row kb + j / 4 and columns
n0 + 4·(j mod 4) .. +3; a fragment for column block nb and k-chunk c reads row
bases 16c + 4g and 16c + 8 + 4g (g = lane / 32)."""
import pytest


def rsw(D, r):
    return (r // (128 // D)) & (D // 8 - 1)


def direct(D, lane, nb, c, half):
    j, g = lane & 15, lane >> 5
    col = nb * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)
    r = 16 * c + 4 * g + (j >> 2) + 8 * half
    return (r * D + (((col >> 3) ^ rsw(D, r)) << 3) + (col & 7)) * 2


def short_form(D, lane, nb, c, half):
    o0 = direct(D, lane, 0, 0, 0)
    flip = (((D // 16) << 4) | 16 * D) if half else 0
    return c * 32 * D + (o0 ^ (nb << 6) ^ flip)


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

"""Host model of the LDS tile layout shared by the 128-head decode kernel
(decode_wide.hip) and the absorbed prefill kernel (prefill_mfma.hip).

A tile holds 32 cache rows; the 16-byte chunks of row r sit XOR-swizzled within
groups of eight by row_key(r) = 2·((r/2) mod 4).  This model restates the
kernels' index arithmetic (the copy offsets, the score's fragment addresses and
the transposed PV reads) and checks that

- the copies put every global chunk of the tile in exactly one LDS slot;
- every fragment read finds the (row, chunk) the MFMA operand needs;
- no two lanes served in the same LDS cycle share a bank.

The bank model is the one rocprofv3's SQ_LDS_BANK_CONFLICT counter showed on
gfx950 for probes of both read kinds: 64 banks of 4 bytes; a ds_read_b128
serves 16 lanes a cycle, lane groups of eight paired as (0-7, 24-31),
(8-15, 16-23), (32-39, 56-63), (40-47, 48-55); a ds_read_b64_tr_b16 serves
lanes 0-31, then 32-63.
"""
import pytest

B128_PASSES = [[l for l in range(64) if (l >> 3) in pair] for pair in ((0, 3), (1, 2), (4, 7), (5, 6))]
B64_PASSES = [list(range(32)), list(range(32, 64))]


def ways(addrs, passes, width):
    """Largest number of lanes of one pass that touch the same bank group of `width` bytes."""
    worst = 1
    for lanes in passes:
        slots = [(addrs[l] % 256) // width for l in lanes]
        worst = max(worst, max(slots.count(s) for s in slots))
    return worst


def row_key(r):
    return ((r >> 1) & 3) << 1


def old_key(r):
    return (r >> 1) & 7


def swz(c, r, key=row_key):
    return (c & ~7) | ((c ^ key(r)) & 7)


def score_addrs(row_bytes, ks, rb, key=row_key):
    """Byte addresses of the score's A fragments (tile row 16rb + l16, chunk 4ks + lg)."""
    out = []
    for lane in range(64):
        l16, lg = lane & 15, lane >> 4
        x_even, x_odd = (lg ^ key(l16)) & 7, ((4 + lg) ^ key(l16)) & 7
        coff = (ks >> 1) * 128 + (x_odd if ks & 1 else x_even) * 16
        out.append((16 * rb + l16) * row_bytes + coff)
    return out


def tr_addrs(row_bytes, nb, hi, key=row_key):
    """Byte addresses of the transposed C reads of column block nb (rows 4lg + l16/4, +16 for hi)."""
    out = []
    for lane in range(64):
        l16, lg = lane & 15, lane >> 4
        r = lg * 4 + (l16 >> 2) + 16 * hi
        chunk = nb * 2 + ((l16 & 3) >> 1)
        out.append(r * row_bytes + swz(chunk, r, key) * 16 + (l16 & 1) * 8)
    return out


# (row bytes, latent columns read by the PV): the 128-head decode, the absorbed
# prefill at r = 256 and the V4 prefill (one 512-wide row as key and value)
SHAPES = [(1152, 512), (640, 256), (1024, 512)]


@pytest.mark.parametrize("row_bytes,r", SHAPES)
def test_copies_and_reads_agree(row_bytes, r):
    rc = row_bytes // 16
    # LDS chunk L of the tile image holds global chunk L ^ row_key(L // rc)
    held = {}
    for L in range(32 * rc):
        g = L ^ row_key(L // rc)
        assert g // rc == L // rc  # the key stays inside the row
        held[L] = g
    assert sorted(held.values()) == list(range(32 * rc))
    # the 128-head decode's whole-tile copies: lane offset 16·lane ^ (key << 4) within each kilobyte
    if row_bytes == 1152:
        for j in range(32 * rc // 64):
            r0 = (j * 64) // rc
            bnd = (r0 + 1) * rc - j * 64
            for ln in range(64):
                voff = (ln * 16) ^ ((row_key(r0) if ln < bnd else row_key(r0 + 1)) << 4)
                assert (j * 1024 + voff) // 16 == held[j * 64 + ln]
    for ks in range(rc // 4):
        for rb in range(2):
            for lane, a in enumerate(score_addrs(row_bytes, ks, rb)):
                row = 16 * rb + (lane & 15)
                assert held[a // 16] == row * rc + 4 * ks + (lane >> 4)
    for nb in range(r // 16):
        for hi in range(2):
            for lane, a in enumerate(tr_addrs(row_bytes, nb, hi)):
                l16, lg = lane & 15, lane >> 4
                row = lg * 4 + (l16 >> 2) + 16 * hi
                assert held[a // 16] == row * rc + nb * 2 + ((l16 & 3) >> 1)


@pytest.mark.parametrize("row_bytes,r", SHAPES)
def test_bank_conflicts(row_bytes, r):
    rc = row_bytes // 16
    score = max(ways(score_addrs(row_bytes, ks, rb), B128_PASSES, 16) for ks in range(rc // 4) for rb in range(2))
    tr = max(ways(tr_addrs(row_bytes, nb, hi), B64_PASSES, 8) for nb in range(r // 16) for hi in range(2))
    if row_bytes % 256 == 128:
        # rows 128 bytes past a multiple of 256: both read kinds conflict-free
        assert (score, tr) == (1, 1)
        # the earlier key (row/2) mod 8 left every transposed read two-way conflicted
        old_tr = max(ways(tr_addrs(row_bytes, nb, 0, old_key), B64_PASSES, 8) for nb in range(r // 16))
        assert old_tr == 2
    else:
        # rows of 1024 bytes all start on the same bank: two-way is the least an
        # unpadded tile allows, and the earlier key made the transposed reads four-way
        assert (score, tr) == (2, 2)
        old_tr = max(ways(tr_addrs(row_bytes, nb, 0, old_key), B64_PASSES, 8) for nb in range(r // 16))
        assert old_tr == 4

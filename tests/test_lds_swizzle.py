"""Bank-conflict freedom of the LDS layouts the kernels use (host-side check of
the layout arithmetic; no GPU).

gfx950's LDS has 64 four-byte banks and serves 256 bytes per cycle: 16 lanes
of a 16-byte read (ds_read_b128) or 32 lanes of an 8-byte read
(ds_read_b64_tr_b16).  K/V tiles are row-major with the 16-byte chunk index
XOR-swizzled by the row: physical chunk = logical chunk ^ swz(row).  This
restates that swizzle and the per-lane addresses of every LDS read pattern
and checks that each cycle's lanes hit distinct banks.
"""
import pytest


def swz(D, row):
    if D == 128:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    if D == 64:
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)
    return (row >> 2) & 3


def addr(D, row, col):
    """Byte address of element (row, col) of a swizzled row-major tile."""
    return row * D * 2 + (((col // 8) ^ swz(D, row)) << 4) + (col % 8) * 2


def banks_b128(addrs):
    return [((a // 4) + i) % 64 for a in addrs for i in range(4)]


def banks_b64(addrs):
    return [((a // 4) + i) % 64 for a in addrs for i in range(2)]


def assert_conflict_free(addrs, width):
    per_cycle = 16 if width == 16 else 32
    for c0 in range(0, len(addrs), per_cycle):
        group = addrs[c0:c0 + per_cycle]
        b = banks_b128(group) if width == 16 else banks_b64(group)
        assert len(set(b)) == len(b), (width, c0, sorted(b))


@pytest.mark.parametrize("D", [32, 64, 128])
def test_swizzle_is_a_permutation_of_chunks(D):
    for row in range(64):
        assert sorted((c ^ swz(D, row)) for c in range(D // 8)) == list(range(D // 8))


@pytest.mark.parametrize("D", [32, 64, 128])
def test_prefill_k_operand_reads(D):
    # 32x32x16 MFMA A operand: lane l reads row 32kb + l%32, logical chunk 2t + l/32
    for kb in range(2):
        for t in range(D // 16):
            addrs = [addr(D, 32 * kb + l % 32, 8 * (2 * t + l // 32)) for l in range(64)]
            assert_conflict_free(addrs, 16)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_prefill_v_transposed_reads(D):
    # ds_read_b64_tr_b16: lane s of 16-lane group G addresses row 4(G/2) + s/4 (+8 for
    # the second half), column 32db + 16(G%2) + 4(s%4)
    for kb in range(2):
        for st in range(2):
            for hh in range(2):
                for db in range(D // 32):
                    addrs = []
                    for l in range(64):
                        G, s = l // 16, l % 16
                        row = 32 * kb + 16 * st + 4 * (G // 2) + s // 4 + 8 * hh
                        col = 32 * db + 16 * (G % 2) + 4 * (s % 4)
                        addrs.append(addr(D, row, col))
                    assert_conflict_free(addrs, 8)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_decode_k_and_q_operand_reads(D):
    # 16x16x32 MFMA: lane (j = l%16, g = l/16) reads row 32w + 16kb + j, logical chunk 4s + g
    for w in range(4):
        for kb in range(2):
            for s in range(D // 32):
                addrs = [addr(D, 32 * w + 16 * kb + l % 16, 8 * (4 * s + l // 16)) for l in range(64)]
                assert_conflict_free(addrs, 16)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_decode_v_transposed_reads(D):
    # lane s of group g addresses row 32ks + 8g + 4hh + s/4, column 16*blk + 4(s%4)
    for ks in range(4):
        for hh in range(2):
            for blk in range(D // 16):
                addrs = [addr(D, 32 * ks + 8 * (l // 16) + 4 * hh + (l % 16) // 4, 16 * blk + 4 * (l % 4))
                         for l in range(64)]
                assert_conflict_free(addrs, 8)


def test_decode_p_operand_reads():
    # P^T rows of 128 keys padded to 136 elements: lane (j, g) reads P[j][32ks + 8g ..]
    row = 136
    for ks in range(4):
        addrs = [(l % 16 * row + 8 * (l // 16)) * 2 + 64 * ks for l in range(64)]
        assert_conflict_free(addrs, 16)

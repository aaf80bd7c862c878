"""Bank-conflict freedom of the LDS access patterns the kernels use (host-side
check of the layout arithmetic; no GPU).

The service model of gfx950's LDS below was measured on MI355X with
single-wave probes (one 64-lane workgroup repeating one LDS instruction at
per-lane byte offsets, rocprofv3 --pmc SQ_LDS_BANK_CONFLICT
SQ_LDS_IDX_ACTIVE, one dispatch per pattern; pairs of lanes sent to the same
bank at different addresses, every other lane reading one broadcast address,
tell which lanes share a cycle):

  * reads serve 256 bytes a cycle over 64 four-byte banks.  ds_read_b128
    serves 16 lanes a cycle: within each 32-lane half of the wave, the 4-lane
    quads whose index (lane bits 2..4) has even bit parity form one group and
    those with odd parity the other.  ds_read_b64 and ds_read_b64_tr_b16
    serve the two 32-lane halves.
  * writes serve 128 bytes a cycle over 32 banks: ds_write_b128 in groups of
    8 consecutive lanes, ds_write_b64 in groups of 16 consecutive lanes.
  * lanes of one group that touch the same bank at different addresses cost
    one extra cycle per extra address; the same address is free (broadcast).

`test_model_reproduces_measurements` pins the model to the measured extra
cycles of a set of probe patterns; the other tests restate each kernel's
per-lane LDS addresses and require zero extra cycles.
"""
import pytest


def swz(D, row):
    """16-byte chunk swizzle of the K/V tiles (d = 256 uses the d = 128 one)."""
    if D in (128, 256):
        return ((row & 3) << 2) | ((row >> 2) & 3)
    if D == 64:
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)
    return (row >> 2) & 3


def addr(D, row, col):
    """Byte address of element (row, col) of a swizzled row-major tile."""
    return row * D * 2 + (((col // 8) ^ swz(D, row)) << 4) + (col % 8) * 2


def _parity(x):
    return bin(x).count("1") & 1


GROUPS = {
    "read_b128": [[l for l in range(64) if l >> 5 == h and _parity((l >> 2) & 7) == p]
                  for h in (0, 1) for p in (0, 1)],
    "read_b64": [list(range(0, 32)), list(range(32, 64))],
    "read_tr_b16": [list(range(0, 32)), list(range(32, 64))],
    "write_b128": [list(range(i, i + 8)) for i in range(0, 64, 8)],
    "write_b64": [list(range(i, i + 16)) for i in range(0, 64, 16)],
}
BYTES = {"read_b128": 16, "read_b64": 8, "read_tr_b16": 8, "write_b128": 16, "write_b64": 8}
BANKS = {"read_b128": 64, "read_b64": 64, "read_tr_b16": 64, "write_b128": 32, "write_b64": 32}


def extra_cycles(kind, addrs):
    """Extra LDS cycles of one wave-wide instruction under the model."""
    assert len(addrs) == 64
    extra = 0
    for group in GROUPS[kind]:
        words = {}
        for l in group:
            for i in range(BYTES[kind] // 4):
                w = addrs[l] // 4 + i
                words.setdefault(w % BANKS[kind], set()).add(w)
        extra += max(len(s) for s in words.values()) - 1
    return extra


def assert_conflict_free(kind, addrs):
    assert extra_cycles(kind, addrs) == 0, (kind, addrs)


# Measured extra cycles per instruction (SQ_LDS_BANK_CONFLICT over 256
# repetitions of one instruction by one wave).
MEASURED = [
    ("read_b128", "1 KB contiguous", [16 * l for l in range(64)], 0),
    ("read_b128", "16 rows of 256 B x 4 chunks, unswizzled", [(l % 16) * 256 + 16 * (l // 16) for l in range(64)], 28),
    ("read_b128", "rows l%32, chunk (l/32)^swz", [(l % 32) * 256 + (((l // 32) ^ swz(128, l % 32)) << 4)
                                                   for l in range(64)], 0),
    ("read_b128", "rows l%16, chunk (l/16)^swz", [(l % 16) * 256 + (((l // 16) ^ swz(128, l % 16)) << 4)
                                                   for l in range(64)], 4),
    ("read_b128", "rows of 272 B, chunk l/16", [(l % 16) * 272 + 16 * (l // 16) for l in range(64)], 4),
    ("read_b64", "512 B contiguous", [8 * l for l in range(64)], 0),
    ("write_b64", "512 B contiguous", [8 * l for l in range(64)], 0),
    ("write_b64", "rows of 272 B, 8 B at 8*(l/16)", [(l % 16) * 272 + 8 * (l // 16) for l in range(64)], 4),
]


@pytest.mark.parametrize("kind,what,addrs,extra", MEASURED, ids=[m[1] for m in MEASURED])
def test_model_reproduces_measurements(kind, what, addrs, extra):
    assert extra_cycles(kind, addrs) == extra


def test_model_groups_match_pair_probes():
    # lanes found to share a cycle by the pair probes
    assert GROUPS["read_b128"][0] == [0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27]
    assert GROUPS["read_b128"][1] == [4, 5, 6, 7, 8, 9, 10, 11, 16, 17, 18, 19, 28, 29, 30, 31]
    assert GROUPS["write_b64"][1] == list(range(16, 32))
    assert GROUPS["write_b128"][1] == list(range(8, 16))


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_swizzle_is_a_permutation_of_chunks(D):
    for row in range(64):
        assert sorted((c ^ swz(D, row)) for c in range(D // 8)) == list(range(D // 8))


# ---- prefill kernel ----

@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_prefill_k_operand_reads(D):
    # 32x32x16 MFMA A operand: lane l reads row 32kb + l%32, logical chunk 2t + l/32
    # (the FP8 Q/K kernel reads chunks 2t and 2t + 1 of 16-bit steps t = 2u, 2u + 1)
    for kb in range(2):
        for t in range(D // 16):
            assert_conflict_free("read_b128", [addr(D, 32 * kb + l % 32, 8 * (2 * t + l // 32)) for l in range(64)])


@pytest.mark.parametrize("D", [32, 64, 128, 256])
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
                    assert_conflict_free("read_tr_b16", addrs)


# ---- decode matrix-core kernel ----

def perm4(g):
    return ((g & 1) << 1) | (g >> 1)


def qk_chunk(D, s, g):
    kS, kX = D // 32, {32: 2, 64: 1, 128: 0, 256: 0}[D]
    return (kS * g + s) ^ (kX if g & 1 else 0)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_decode_qk_chunk_map_is_a_bijection(D):
    assert sorted(qk_chunk(D, s, g) for s in range(D // 32) for g in range(4)) == list(range(D // 8))


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_decode_k_and_q_operand_reads(D):
    # 16x16x32 MFMA: lane (j = l%16, g = l/16) reads row 32w + 16kb + j (Q: row j),
    # logical chunk qk_chunk(s, g)
    for w in range(4):
        for kb in range(2):
            for s in range(D // 32):
                assert_conflict_free("read_b128", [addr(D, 32 * w + 16 * kb + l % 16, 8 * qk_chunk(D, s, l // 16))
                                                   for l in range(64)])


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_decode_v_transposed_reads(D):
    # lane s of group g addresses row 32ks + 4 perm4(g) + 16hh + s/4, column 16*blk + 4(s%4)
    for ks in range(4):
        for hh in range(2):
            for blk in range(D // 16):
                addrs = [addr(D, 32 * ks + 4 * perm4(l // 16) + 16 * hh + (l % 16) // 4, 16 * blk + 4 * (l % 4))
                         for l in range(64)]
                assert_conflict_free("read_tr_b16", addrs)


def test_decode_p_slot_order_matches_v_rows():
    # slot 8 perm4(g) + 4 kb + r of a k-step holds key 16 kb + 4 g + r (P^T write);
    # the V^T read of group G supplies keys 4 perm4(G) + 16 hh + 0..3 for slots 8G + 4hh + 0..3
    for g in range(4):
        for kb in range(2):
            for r in range(4):
                slot = 8 * perm4(g) + 4 * kb + r
                G, hh, rr = slot // 8, (slot % 8) // 4, slot % 4
                assert 4 * perm4(G) + 16 * hh + rr == 16 * kb + 4 * g + r


def test_decode_p_writes_and_reads():
    # P^T rows of 256 bytes, 16-byte unit u of row j at unit u ^ j; lane (j, g) of
    # wave w writes unit 4w + perm4(g), the P.V lane (j, g) reads unit 4ks + g
    for w in range(4):
        assert_conflict_free("write_b128", [(l % 16) * 256 + (((4 * w + perm4(l // 16)) ^ (l % 16)) << 4)
                                            for l in range(64)])
    for ks in range(4):
        assert_conflict_free("read_b128", [(l % 16) * 256 + (((4 * ks + l // 16) ^ (l % 16)) << 4)
                                           for l in range(64)])


@pytest.mark.parametrize("D", [32, 64, 128])
def test_decode_fp8_row_writes(D):
    # FP8 KV: piece u (16 codes) of a 128-key sub-chunk becomes logical chunks
    # 2(u % kPR8) + half of row (u / kPR8) ^ (4 if bit 2 of u is set)
    kPR8 = D // 16
    row_of = lambda u: (u // kPR8) ^ (((u >> 2) & 1) << 2)
    assert sorted((row_of(u), u % kPR8) for u in range(128 * kPR8)) == [(r, c) for r in range(128) for c in range(kPR8)]
    for p in range(128 * kPR8 // 256):
        for half in range(2):
            for w in range(4):
                addrs = []
                for l in range(64):
                    u = p * 256 + 64 * w + l
                    row, pc8 = row_of(u), u % kPR8
                    addrs.append(row * D * 2 + (((2 * pc8 + half) ^ swz(D, row)) << 4))
                assert_conflict_free("write_b128", addrs)
                # one wave's pieces cover whole consecutive rows (coalesced loads)
                rows = sorted({row_of(p * 256 + 64 * w + l) for l in range(64)})
                assert rows == list(range(rows[0], rows[0] + 64 // kPR8))

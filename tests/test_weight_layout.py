"""The native weight-code order (include/moe_mxfp4.h, "Native code order"),
as the tests' numpy definition (tests/helpers.native_order) writes it,
against entries worked out by hand from the header's rule: block
((s*C + c)*NQ + q) holds at byte 16*l (l = 16*g + n) the row-major bytes of
row 32*(s/2) + 8*(n/4) + 4*(s%2) + n%4 starting at NQ*(64*c + 16*g) + 16*q.
Likewise the blocked row order of MXFP4 activations
(tests/helpers.blocked_order against the rule of moe_mxfp4_quantize_blocked:
row p's chunk c at ((p/16)*C + c)*1024 + (p%16)*64 for the codes,
((p/16)*C + c)*64 + (p%16)*4 for the scales)."""
import numpy as np

from tests.helpers import blocked_order, native_order


def _labelled(rows, row_bytes):
    """Each byte's value encodes where it sat: (row, byte) -> distinct ids."""
    r, b = np.meshgrid(np.arange(rows), np.arange(row_bytes), indexing="ij")
    return r * row_bytes + b


def _piece(nat, rb, k):
    """The k-th 16-byte piece of the native array, as (row, first byte) of its source."""
    flat = nat.reshape(-1)[16 * k:16 * k + 16]
    assert np.array_equal(np.diff(flat), np.ones(15))     # one contiguous run of a row
    return divmod(int(flat[0]), rb)


def test_mxfp4_one_strip_pair_one_chunk():
    rb = 64                                    # 128 MXFP4 codes per row: C = 1
    nat = native_order(_labelled(32, rb), 1)
    assert _piece(nat, rb, 0) == (0, 0)        # block 0 = strip 0; lane 0: n 0, g 0
    assert _piece(nat, rb, 1) == (1, 0)        # lane 1: n 1 -> row 1
    assert _piece(nat, rb, 3) == (3, 0)
    assert _piece(nat, rb, 4) == (8, 0)        # lane 4: n 4 -> 8*1 + 0
    assert _piece(nat, rb, 15) == (27, 0)      # n 15 -> 8*3 + 3
    assert _piece(nat, rb, 16) == (0, 16)      # lane 16: n 0, g 1
    assert _piece(nat, rb, 63) == (27, 48)     # lane 63: n 15, g 3
    assert _piece(nat, rb, 64) == (4, 0)       # block 1 = strip 1; lane 0 -> 4*1
    assert _piece(nat, rb, 64 + 5) == (13, 0)  # strip 1, n 5 -> 8 + 4 + 1
    assert _piece(nat, rb, 64 + 63) == (31, 48)


def test_mxfp4_two_strips_two_chunks():
    rb = 128                                   # 256 codes per row: C = 2
    nat = native_order(_labelled(32, rb), 1)
    assert _piece(nat, rb, 64) == (0, 64)      # block 1 = (s 0, c 1), lane 0
    assert _piece(nat, rb, 64 + 17) == (1, 80)  # block 1, lane 17: n 1, g 1
    assert _piece(nat, rb, 128) == (4, 0)      # block 2 = (s 1, c 0), lane 0
    assert _piece(nat, rb, 3 * 64 + 63) == (31, 112)   # block 3 = (s 1, c 1), lane 63


def test_mxfp4_second_strip_pair():
    rb = 64
    nat = native_order(_labelled(64, rb), 1)
    assert _piece(nat, rb, 2 * 64) == (32, 0)           # block 2 = strip 2, lane 0
    assert _piece(nat, rb, 2 * 64 + 6) == (42, 0)       # n 6 -> 32 + 8 + 2
    assert _piece(nat, rb, 3 * 64 + 32 + 12) == (60, 32)   # strip 3, lane 44: n 12, g 2


def test_mxfp8_parts():
    rb = 256                                   # 256 E4M3 codes per row: C = 2, NQ = 2
    nat = native_order(_labelled(32, rb), 2)
    assert _piece(nat, rb, 0) == (0, 0)        # block 0 = (s 0, c 0, q 0), lane 0
    assert _piece(nat, rb, 64) == (0, 16)      # block 1 = (c 0, q 1), lane 0
    assert _piece(nat, rb, 16) == (0, 32)      # block 0, lane 16: g 1 -> byte 2*16
    assert _piece(nat, rb, 2 * 64 + 5) == (9, 128)     # block 2 = (c 1, q 0), lane 5: n 5
    assert _piece(nat, rb, 3 * 64 + 50) == (2, 128 + 96 + 16)   # block 3 (c 1, q 1), lane 50: n 2, g 3
    assert _piece(nat, rb, 4 * 64) == (4, 0)   # block 4 = (s 1, c 0, q 0), lane 0


def test_is_a_permutation_of_pieces_and_keeps_experts_in_place():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(3 * 32, 192), dtype=np.uint8)   # 3 experts x 32 rows
    nat = native_order(codes, 1)
    assert nat.shape == codes.shape
    assert sorted(map(bytes, codes.reshape(-1, 16))) == sorted(map(bytes, nat.reshape(-1, 16)))
    for e in range(3):          # converting the stack = converting each expert on its own
        assert np.array_equal(nat[32 * e:32 * e + 32], native_order(codes[32 * e:32 * e + 32], 1))


def test_blocked_activation_rows():
    R, C = 32, 2                               # 32 rows of 256 codes: 128 code bytes, 8 scale bytes
    codes, scales = _labelled(R, 64 * C), _labelled(R, 4 * C)
    bc, bs = blocked_order(codes, scales)
    fc, fs = bc.reshape(-1), bs.reshape(-1)
    # row 0, chunk 0: code bytes 0..63 first, its scale bytes 0..3 first
    assert list(fc[:64]) == list(range(64)) and list(fs[:4]) == [0, 1, 2, 3]
    # row 1, chunk 0 right after row 0's: codes at 64, scales at 4
    assert fc[64] == 1 * 128 and fs[4] == 1 * 8
    # row 0, chunk 1 (code bytes 64..127, scale bytes 4..7): block (0, 1) at 1024 / 64
    assert fc[1024] == 64 and fs[64] == 4
    # row 17 = block 1, row 1; chunk 1: ((1*2 + 1)*1024 + 64), ((1*2 + 1)*64 + 4)
    assert fc[3 * 1024 + 64] == 17 * 128 + 64 and fs[3 * 64 + 4] == 17 * 8 + 4
    # row 31, chunk 1, last code byte / last scale byte: the arrays' last bytes
    assert fc[-1] == 31 * 128 + 127 and fs[-1] == 31 * 8 + 7
    # a permutation: every byte once
    assert sorted(fc) == sorted(codes.reshape(-1)) and sorted(fs) == sorted(scales.reshape(-1))

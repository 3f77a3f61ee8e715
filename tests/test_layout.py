"""Host-side checks of the tiled MX layout helpers used by the GPU parity tests
(no GPU needed)."""

import numpy as np

from oracle import mx_oracle as O
from tests.parity import tiled_chunk_offsets, tiled_to_rows


def test_chunk_offsets_are_a_permutation():
    off = tiled_chunk_offsets()
    assert off.shape == (32, 96)
    assert np.array_equal(np.sort(off.ravel()), np.arange(3072))


def test_chunk_offsets_planes():
    """Each 24-byte block of a row is one 16-byte run plus one 8-byte run, in
    planes whose rows are 16 or 8 bytes apart."""
    off = tiled_chunk_offsets()
    for j in (0, 7, 31):
        for q in range(4):
            blk = off[j, 24 * q:24 * q + 24]
            h = q >> 1
            if q % 2 == 0:
                assert np.array_equal(blk[:16], h * 1536 + j * 16 + np.arange(16))
                assert np.array_equal(blk[16:], h * 1536 + 512 + j * 8 + np.arange(8))
            else:
                assert np.array_equal(blk[:8], h * 1536 + 768 + j * 8 + np.arange(8))
                assert np.array_equal(blk[8:], h * 1536 + 1024 + j * 16 + np.arange(16))


def test_tiled_round_trip_with_padding():
    """Scatter row-major packed codes into the tiled layout by the offsets, pad,
    and read them back with tiled_to_rows."""
    rng = np.random.default_rng(0)
    rows, k = 45, 288  # 2 groups (ragged), 3 stages (ragged: 9 blocks of 12)
    codes = rng.integers(0, 64, size=(rows, k))
    packed = O.pack(codes)
    scales = rng.integers(0, 255, size=(rows, k // 32)).astype(np.uint8)
    stages, groups = 3, 2
    ct = np.zeros((stages, groups, 3072), dtype=np.uint8)
    st = np.full((stages, groups, 32, 4), 127, dtype=np.uint8)
    off = tiled_chunk_offsets()
    for r in range(rows):
        g, j = divmod(r, 32)
        for s in range(stages):
            sl = packed[r, 96 * s:96 * s + 96]
            ct[s, g, off[j, :len(sl)]] = sl
            nb = min(4, k // 32 - 4 * s)
            st[s, g, j, :nb] = scales[r, 4 * s:4 * s + nb]
    c, sc, pad_c, pad_s = tiled_to_rows(ct.ravel(), st.ravel(), rows, k)
    assert np.array_equal(c, packed) and np.array_equal(sc, scales)
    assert not pad_c.any() and np.all(pad_s == 127)
    assert np.array_equal(O.unpack(c, k), codes)

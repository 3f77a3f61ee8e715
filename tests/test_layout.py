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


def test_chunk_offsets_fp4_fp8_planes():
    """4- and 8-bit chunks: a permutation of 512 * bits bytes, each block of a
    row split into 16-byte runs in planes whose rows are 16 bytes apart."""
    for bits in (4, 8):
        off = tiled_chunk_offsets(bits)
        eb = 4 * bits
        assert off.shape == (32, 4 * eb)
        assert np.array_equal(np.sort(off.ravel()), np.arange(512 * bits))
        for j in (0, 9, 31):
            for q in range(4):
                for t in range(0, eb, 16):
                    run = off[j, eb * q + t:eb * q + t + 16]
                    assert np.array_equal(run, run[0] + np.arange(16))
                    assert run[0] % 512 == j * 16
        if bits == 8:  # block q's bytes 0..15 in half 0, 16..31 in half 1, plane 2 (q % 2) + q // 2
            for q in range(4):
                assert off[5, 32 * q] == (2 * (q % 2) + q // 2) * 512 + 5 * 16
                assert off[5, 32 * q + 16] == 2048 + (2 * (q % 2) + q // 2) * 512 + 5 * 16


def test_tiled_round_trip_fp4_fp8():
    rng = np.random.default_rng(1)
    rows, k = 45, 288
    for fmt in ("e2m1", "e4m3"):
        bits = O.element_bits(fmt)
        codes = rng.integers(0, 1 << bits, size=(rows, k))
        packed = O.pack(codes, fmt)
        stages, groups, rb = 3, 2, 16 * bits
        ct = np.zeros((stages, groups, 512 * bits), dtype=np.uint8)
        st = np.full((stages, groups, 32, 4), 127, dtype=np.uint8)
        off = tiled_chunk_offsets(bits)
        for r in range(rows):
            g, j = divmod(r, 32)
            for s_ in range(stages):
                sl = packed[r, rb * s_:rb * s_ + rb]
                ct[s_, g, off[j, :len(sl)]] = sl
        c, sc, pad_c, pad_s = tiled_to_rows(ct.ravel(), st.ravel(), rows, k, bits)
        assert np.array_equal(c, packed) and not pad_c.any()
        assert np.array_equal(O.unpack(c, k, fmt), codes)


def test_rows_gather_matches_the_whole_view():
    """mx_rows_gather (the large-size tests' device-side row pick) returns the
    same bytes as tiled_to_rows over the whole tensor, for every element width,
    ragged rows and K, rows in any order and repeated."""
    import types

    import torch

    from tests.parity import mx_rows_gather

    rng = np.random.default_rng(5)
    for fmt, bits in (("e2m3", 6), ("e2m1", 4), ("e4m3", 8)):
        rows, k = 77, 416  # 3 groups (ragged), 4 stages (ragged)
        stages, groups = 4, 3
        codes = rng.integers(0, 256, size=stages * groups * 512 * bits, dtype=np.uint8)
        scales = rng.integers(0, 256, size=stages * groups * 128, dtype=np.uint8)
        t = types.SimpleNamespace(codes=torch.from_numpy(codes), scales=torch.from_numpy(scales), fmt=fmt,
                                  rows=rows, k=k, layout="tiled")
        c, s, _, _ = tiled_to_rows(codes, scales, rows, k, bits)
        pick = np.array([76, 0, 31, 32, 33, 64, 5, 5])
        gc, gs = mx_rows_gather(t, pick)
        assert np.array_equal(gc, c[pick]) and np.array_equal(gs, s[pick])

"""Host side of the offline repack into the GPU-tiled 4-bit layout
(qmoe_repack_tiled4; devtrends.cc "Come eseguire un modello da 26 miliardi…",
section "Senza dipendenze da llama.cpp e MLX": the weights are converted once
into the engine's own layout).  The layout is checked against its definition
in include/qmoe.h element by element, and by undoing it."""
import numpy as np
import pytest

import synth


@pytest.fixture(scope="module")
def q():
    import bit_quantized_gemv_amd as q

    return q


def _expected(m):
    """The tiled bytes, written out from the definition: codes [RB][CH][8][16 B],
    then (scale | bias << 16) [RB][8][G]; rows past the matrix are zero."""
    rows, cols = m.rows, m.cols
    CH, G, RB = cols // 32, cols // 64, -(-rows // 8)
    qb = m.q.view(np.uint8).reshape(rows, cols // 2)
    codes = np.zeros((RB, CH, 8, 16), dtype=np.uint8)
    pairs = np.zeros((RB, 8, G), dtype=np.uint32)
    for row in range(rows):
        rb, r = divmod(row, 8)
        for c in range(CH):
            codes[rb, c, r] = qb[row, 16 * c:16 * c + 16]
        pairs[rb, r] = m.s[row].astype(np.uint32) | (m.b[row].astype(np.uint32) << 16)
    return np.concatenate([codes.reshape(-1), pairs.reshape(-1).view(np.uint8)])


@pytest.mark.parametrize("rows,cols", [(13, 128), (8, 64), (40, 704), (3, 2816)])
def test_repack_matches_layout_definition(q, rows, cols):
    m = synth.random_qmat(rows, cols, 4, rows * 31 + cols)
    got = q.qmoe_repack_tiled4(m.q.view(np.uint8), m.s, m.b, rows, cols)
    assert got.size == q.qmoe_tiled4_bytes(rows, cols)
    assert np.array_equal(got, _expected(m))


def test_repack_round_trip_and_padding(q):
    """Undo the tiling: every code byte and scale/bias pair comes back, and
    the padded rows of the last row-block are zero."""
    rows, cols = 21, 256
    m = synth.random_qmat(rows, cols, 4, 5)
    t = q.qmoe_repack_tiled4(m.q.view(np.uint8), m.s, m.b, rows, cols)
    CH, G, RB = cols // 32, cols // 64, 3
    codes = t[:RB * CH * 8 * 16].reshape(RB, CH, 8, 16)
    pairs = t[RB * CH * 8 * 16:].view(np.uint32).reshape(RB, 8, G)
    back = codes.transpose(0, 2, 1, 3).reshape(RB * 8, CH * 16)
    assert np.array_equal(back[:rows], m.q.view(np.uint8).reshape(rows, cols // 2))
    assert not back[rows:].any()
    pr = pairs.reshape(RB * 8, G)
    assert np.array_equal((pr[:rows] & 0xFFFF).astype(np.uint16), m.s)
    assert np.array_equal((pr[:rows] >> 16).astype(np.uint16), m.b)
    assert not pr[rows:].any()


def test_repack_one_element_placement(q):
    """A single non-zero code byte lands where the definition puts it: row
    10 (row-block 1, row 2 of it), byte 37 (chunk 2, byte 5 of the chunk)."""
    rows, cols = 16, 128
    m = synth.random_qmat(rows, cols, 4, 9)
    qb = np.zeros((rows, cols // 2), dtype=np.uint8)
    qb[10, 37] = 0xA5
    t = q.qmoe_repack_tiled4(qb, m.s, m.b, rows, cols)
    CH = cols // 32
    off = ((1 * CH + 2) * 8 + 2) * 16 + 5
    assert t[off] == 0xA5
    assert np.count_nonzero(t[:2 * CH * 8 * 16]) == 1


def test_repack_sizes_and_errors(q):
    assert q.qmoe_tiled4_bytes(13, 128) == 2 * 4 * 8 * 16 + 2 * 8 * 2 * 4
    assert q.qmoe_tiled4_bytes(0, 128) == 0
    assert q.qmoe_tiled4_bytes(8, 100) == 0
    m = synth.random_qmat(8, 128, 4, 1)
    with pytest.raises(q.QmoeError):
        q.qmoe_repack_tiled4(m.q.view(np.uint8), m.s, m.b, 8, 100)
    import ctypes as C

    out = np.empty(q.qmoe_tiled4_bytes(8, 128) - 1, dtype=np.uint8)
    rc = q.lib().qmoe_repack_tiled4(m.q.ctypes.data, m.s.ctypes.data, m.b.ctypes.data, 8, 128,
                                    out.ctypes.data, C.c_size_t(out.size))
    assert rc == 4  # QMOE_ERR_WORKSPACE: the output is too small

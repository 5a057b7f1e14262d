"""Shape bookkeeping and seeded input generation (no GPU)."""
import json
import os

import numpy as np
import pytest

from rank_decomposed_linear_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_table1_communication_counts():
    g = json.load(open(os.path.join(GOLDEN, "table1_llama3_70b.json")))
    got = W.table1_comm_elements(**g["inputs"])
    for key, val in g["printed"].items():
        assert got[key] == val, key


def test_rank_formula_examples():
    s8 = W.LLAMA3_8B_C40_DECODE.shape
    assert (s8.rank("q"), s8.rank("k"), s8.rank("v"), s8.rank("o")) == (1216, 448, 448, 1216)
    assert (s8.rank("gate"), s8.rank("up"), s8.rank("down")) == (1856, 1856, 1856)
    s70 = W.LLAMA3_70B_C50_DECODE.shape
    assert (s70.rank("q"), s70.rank("k"), s70.rank("o")) == (2048, 448, 2048)
    assert (s70.rank("gate"), s70.rank("down")) == (3136, 3136)
    sweep = {w.compression_pct: (w.shape.rank("q"), w.shape.rank("k"), w.shape.rank("gate"))
             for w in W.LLAMA3_8B_SWEEP}
    assert sweep == {20: (1600, 640, 2496), 30: (1408, 512, 2176), 40: (1216, 448, 1856),
                     50: (1024, 384, 1536), 60: (768, 320, 1216)}
    # every rank is a multiple of 64 and removes at least the requested share
    for w in W.ALL_WORKLOADS[1:]:
        for p, (m, n) in w.shape.shapes().items():
            k = w.shape.rank(p)
            assert k % 64 == 0
            assert (m + n) * k <= (100 - w.compression_pct) * m * n / 100


def test_tiny_parameter_count():
    assert W.TINY.shape.weight_elements() == 312320


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, np.pi, -2.5, 0.0], np.float32)
    bits = W.f32_to_bf16_bits(vals)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0x4049, 0xC020, 0x0000]
    assert np.array_equal(W.bf16_bits_to_f32(bits)[[0, 4]], np.array([1.0, -2.5], np.float32))


def test_draws_are_seeded_and_shaped():
    w = W.TINY
    a_w, a_in = W.draw(w)
    b_w, b_in = W.draw(w)
    assert np.array_equal(a_in.x, b_in.x)
    for p in W.PROJECTIONS:
        assert np.array_equal(a_w.factors[p][0], b_w.factors[p][0])
    A, B = a_w.factors["gate"]
    assert A.shape == (256, 64) and B.shape == (64, 688) and A.dtype == np.float32
    assert a_in.x.shape == (2, 32, 256) and a_in.decode_x.shape == (8, 2, 1, 256)
    # 32 prefill + 8 decode rows, rounded up to a 64-row page
    assert a_in.ck.shape == (2, 64, 64) and W.TINY.l_max == 64
    assert W.LLAMA3_8B_C40_DECODE.l_max == 1088
    assert abs(float(np.std(A)) - 0.02) < 0.002


def test_library_storage_order():
    """f32 factors are stored transposed, the value cache rank-major; pure
    data movement, invertible."""
    a = np.arange(6 * 4, dtype=np.float32).reshape(6, 4)     # A [m=6, k=4]
    t = W.to_library_factor(a)
    assert t.shape == (4, 6) and t.flags["C_CONTIGUOUS"]
    assert t[3, 5] == a[5, 3]
    cv = np.arange(2 * 5 * 3, dtype=np.float32).reshape(2, 5, 3)  # [Bsz, L, r_v]
    c = W.to_library_value_cache(cv)
    assert c.shape == (2, 3, 5) and c.flags["C_CONTIGUOUS"]
    assert c[1, 2, 4] == cv[1, 4, 2]
    assert np.array_equal(W.from_library_value_cache(c, False), cv)


def test_operand_tile_order():
    """bf16 storage is the transposed matrix in 16 x 32 operand tiles: element
    (r, c) of an [R, C] matrix at tile (r // 16) * (C // 32) + c // 32, offset
    ((c % 32) // 8 * 16 + r % 16) * 8 + c % 8 -- MFMA lane l = r % 16 +
    16 * ((c % 32) // 8) holding 8 consecutive columns."""
    R, C = 32, 96
    a = (np.arange(R * C, dtype=np.uint32) % 65521).astype(np.uint16).reshape(R, C)
    flat = W.tile_operands(a).reshape(-1)
    for r, c in ((0, 0), (5, 7), (15, 8), (16, 31), (31, 95), (17, 40)):
        off = ((r // 16) * (C // 32) + c // 32) * 512 + (((c % 32) // 8) * 16 + r % 16) * 8 + c % 8
        assert flat[off] == a[r, c], (r, c)
    assert np.array_equal(W.untile_operands(W.tile_operands(a)), a)
    # a bf16 factor: transpose, then tiles
    A = a.T.copy()                                            # A [m=96, k=32]
    assert np.array_equal(W.to_library_factor(A), W.tile_operands(a))
    # bf16 caches round-trip
    ck = (np.arange(2 * 64 * 32, dtype=np.uint32) % 60000).astype(np.uint16).reshape(2, 64, 32)
    assert np.array_equal(W.from_library_key_cache(W.to_library_key_cache(ck), True), ck)
    cv = (np.arange(2 * 64 * 48, dtype=np.uint32) % 60000).astype(np.uint16).reshape(2, 64, 48)
    assert np.array_equal(W.from_library_value_cache(W.to_library_value_cache(cv), True), cv)
    import pytest
    with pytest.raises(ValueError):
        W.tile_operands(np.zeros((8, 32), np.uint16))


def test_b_row_decay_scaling():
    w = W.Workload("t", W.make_shape(64, 2, 1, 32, 96, "f32", 0.0, fixed_rank=64), batch=1,
                   phase="decode", context=4, seed=5, b_row_decay=True)
    ws, _ = W.draw(w)
    B = ws.factors["up"][1]
    s = np.std(B, axis=1)
    # row i scaled by i^-1/2: the std ratio of rows 1 and 64 is about 8
    assert 5.0 < s[:4].mean() / s[-4:].mean() < 12.0

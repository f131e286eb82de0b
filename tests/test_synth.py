"""The seeded generator: determinism, ranges and the byte layout of its packers.

The packers are checked against byte patterns assembled by hand (not against
the oracle), so the generator and the oracle pin each other's layout from two
independent writings of it.
"""
import numpy as np

import synth


def test_determinism_per_tensor_stream():
    a = synth.gen_tensor(synth.CFG1, 0)
    b = synth.gen_tensor(synth.CFG1, 0)
    c = synth.gen_tensor(synth.CFG1, 1)
    assert np.array_equal(a.raw, b.raw) and not np.array_equal(a.raw, c.raw)


def test_q4_0_pack_layout_by_hand():
    d = np.array([[1.0, -2.0]], np.float16)
    q = np.arange(64, dtype=np.uint8).reshape(1, 64) % 16
    raw = synth.pack_q4_0(d, q)
    assert raw.shape == (1, 36)
    assert list(raw[0, 0:2]) == [0x00, 0x3C] and list(raw[0, 18:20]) == [0x00, 0xC0]
    for l in range(16):
        assert raw[0, 2 + l] == (q[0, l] | (q[0, 16 + l] << 4))


def test_q8_0_pack_layout_by_hand():
    d = np.array([[0.5]], np.float16)
    q = np.arange(-16, 16, dtype=np.int8).reshape(1, 32)
    raw = synth.pack_q8_0(d, q)
    assert list(raw[0, :2]) == [0x00, 0x38]
    assert raw[0, 2] == 0xF0 and raw[0, 33] == 15


def test_q4_k_pack_layout_by_hand():
    d = np.array([[1.0]], np.float16)
    dmin = np.array([[0.5]], np.float16)
    sc = np.array([[[1, 2, 3, 4, 26, 44, 62, 1]]], np.uint8)
    m = np.array([[[5, 6, 7, 8, 25, 43, 61, 15]]], np.uint8)
    q = np.zeros((1, 256), np.uint8)
    q[0, 0], q[0, 32], q[0, 65], q[0, 97] = 1, 2, 15, 3
    raw = synth.pack_q4_k(d, dmin, sc, m, q)
    # the same twelve bytes worked out by hand in tests/golden/q4_k_block.json
    assert bytes(raw[0, 4:16]).hex() == "4182c30445 86c7089abcdef1".replace(" ", "")
    assert raw[0, 16] == 0x21 and raw[0, 16 + 33] == 0x3F
    assert int(np.count_nonzero(raw[0, 16:])) == 2


def test_q6_k_pack_layout_by_hand():
    # the columns of the hand-worked super-block in tests/golden/q6_k_block.json
    d = np.array([[0.5]], np.float16)
    sc = np.array([[[-128, -8, -6, 1, -4, 7, -2, 127, 5, 3, 16, -1, 9, 2, -64, 11]]], np.int8)
    q = np.zeros((1, 256), np.uint8)                           # every unlisted code is 0
    for col, v in {0: 1, 32: 19, 64: 34, 96: 52, 31: 16, 63: 58, 95: 0, 127: 41,
                   128: 63, 160: 39, 192: 21, 224: 0, 159: 32, 191: 12, 223: 32, 255: 19}.items():
        q[0, col] = v
    raw = synth.pack_q6_k(d, sc, q)
    assert raw.shape == (1, 210)
    want = {0: 0x21, 32: 0x43, 63: 0x9A, 64: 0x5F, 96: 0x07, 127: 0x3C,
            128: 0xE4, 159: 0x8D, 160: 0x1B, 191: 0x62}
    for off in range(192):
        assert raw[0, off] == want.get(off, 0), off
    assert bytes(raw[0, 192:208]).hex() == "80f8fa01fc07fe7f050310ff0902c00b"
    assert list(raw[0, 208:210]) == [0x00, 0x38]


def test_distributions_in_range():
    t = synth.make_tensor("q4_0", 64, 256, np.random.default_rng(0), keep_logical=True)
    d = t.logical["d"].astype(np.float64)
    assert d.min() >= 0.0049 and d.max() <= 0.0501
    t = synth.make_tensor("i8row", 64, 256, np.random.default_rng(0), keep_logical=True)
    assert t.logical["q"].min() >= -127 and t.logical["q"].max() <= 127
    assert 1e-4 <= t.row_scale.min() and t.row_scale.max() <= 1e-3
    t = synth.make_tensor("q4_k", 8, 512, np.random.default_rng(0), keep_logical=True)
    assert t.logical["sc"].max() < 64 and t.logical["q"].max() < 16
    t = synth.make_tensor("q6_k", 8, 512, np.random.default_rng(0), keep_logical=True)
    assert t.logical["sc"].min() >= -128 and t.logical["q"].max() < 64


def test_algorithmic_bytes_match_block_sizes():
    assert synth.algorithmic_bytes("q4_0", 17408, 5120) == 50_135_040
    assert synth.algorithmic_bytes("q8_0", 49152, 576) == 30_081_024
    assert synth.algorithmic_bytes("q4_k", 2048, 2048) == 2_359_296
    assert synth.algorithmic_bytes("i8row", 49152, 2048) == 100_859_904
    assert synth.algorithmic_bytes("q6_k", 32000, 2048) == 53_760_000

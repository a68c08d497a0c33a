"""The interleaved wire layout of the oracle (TACO paper, section 4.4.2):
pinned to a hand-written byte image and to its own inverse."""
import numpy as np

from conftest import read_golden


def golden_records():
    rows = read_golden("packed_layout_b32.txt")
    recs, cur = [], None
    for r in rows:
        if r[0] == "record":
            cur = []
            recs.append(cur)
        else:
            cur.extend(int(v, 16) for v in r)
    return np.array(recs, dtype=np.uint8)


def test_pack_matches_handwritten_bytes(oracle_mod):
    codes = np.zeros(64, np.uint8)
    codes[:32] = np.arange(32)
    codes[32] = 0x7E
    codes[63] = 0xFE
    alpha = np.array([1.0, -2.0], np.float32)
    scale = np.array([0.5, 3.0], np.float32)
    got = oracle_mod.pack(codes, alpha, scale, 32)
    want = golden_records()
    assert got.shape == (2, 40)
    assert np.array_equal(got, want)


def test_unpack_inverts_pack(oracle_mod, synth_mod):
    x = synth_mod.generate(synth_mod.WORKLOADS["laplace_2048x1024"].with_shape(4))
    for B in (32, 128, 512):
        c, a, s = oracle_mod.compress(x, B)
        p = oracle_mod.pack(c, a, s, B)
        assert p.shape == (x.size // B, B + 8)
        c2, a2, s2 = oracle_mod.unpack(p, B)
        assert np.array_equal(c2, c.reshape(-1))
        assert np.array_equal(a2, a) and np.array_equal(s2, s)

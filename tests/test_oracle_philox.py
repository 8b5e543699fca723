"""Pins of oracle/philox.py: the published Random123 known-answer vectors for
Philox4x32-10, the same round/key-schedule code instantiated as Philox4x64-10
against numpy's Philox bit generator (a library routine), and the vectorised
form against the scalar one."""

import numpy as np

from oracle import philox as P


# Known-answer vectors distributed with the Random123 library (kat_vectors):
# counter words, key words -> output words.
KAT_4x32_10 = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF), (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def test_philox4x32_known_answers():
    for ctr, key, out in KAT_4x32_10:
        assert tuple(P.philox_block(ctr, key)) == out


def test_generic_rounds_match_numpy_philox4x64():
    # numpy's Philox is the 4x64-10 member of the family; its raw stream for
    # key k and initial counter 0 is the blocks for counters 1, 2, ... (the
    # counter is advanced before each block).
    for key in ((0, 0), (12345, 0), (2 ** 63 + 17, 5)):
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=0)
        raw = [int(x) for x in bg.random_raw(12)]
        ours = []
        for n in range(1, 4):
            ours += P.philox_block((n, 0, 0, 0), key, params=P.PHILOX4x64)
        assert raw == ours


def test_vectorised_matches_scalar():
    rs = np.random.default_rng(0)
    c = rs.integers(0, 2 ** 32, (4, 200), dtype=np.uint64).astype(np.uint32)
    k0, k1 = 0x1234ABCD, 0x0BADF00D
    vec = P.philox4x32_np(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(200):
        ref = P.philox_block([int(c[j, i]) for j in range(4)], (k0, k1))
        assert [int(vec[j][i]) for j in range(4)] == ref


def test_element_draw_mapping():
    seed = (7 << 32) | 99
    idx = np.arange(0, 40)
    r16 = P.element_r16(idx, seed, stream_id=1, tensor_tag=5)
    for i in idx:
        n = int(i) // 8
        words = P.philox_block((n & 0xFFFFFFFF, n >> 32, 1, 5), (99, 7))
        w = words[(int(i) % 8) // 2]
        want = (w & 0xFFFF) if i % 2 == 0 else (w >> 16)
        assert r16[i] == want
    big = np.array([2 ** 40 + 3])
    n = (2 ** 40 + 3) // 8
    w = P.philox_block((n & 0xFFFFFFFF, n >> 32, 0, 0), (0, 0))[1]
    assert P.element_r16(big, 0, 0)[0] == (w >> 16)

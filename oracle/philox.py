"""Philox counter-based generator (Salmon, Moraes, Dror, Shaw: "Parallel random
numbers: as easy as 1, 2, 3", SC'11), written from its published definition.

The pages ask only that gradient rounding be stochastic and unbiased ("Train
models faster ... NVFP4", section "NVFP4 pretraining recipe"; "NVFP4 RL
training", baseline-recipe section).  Reproducible draws need a counter-based
generator; Philox4x32-10 is the published one chosen here.

One Philox-N x W round on counter words (c0, c1, c2, c3) with key (k0, k1):
    (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2      (full 2W-bit products)
    c' = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)
and between rounds the key is bumped by the Weyl constants (k0 += W0,
k1 += W1) modulo 2^W.  Ten rounds.

Mapping onto the quantizer (a reading; the pages are silent): key = (seed lo,
seed hi); counter = (n lo, n hi, stream_id, tensor_tag) with n = idx // 8 and
idx = row * cols + col the element's index in the logical input.  Element idx
takes output word (idx % 8) // 2, its low 16 bits when idx is even and its high
16 bits when idx is odd.

Test infrastructure only (see the package docstring).
"""

import numpy as np

PHILOX4x32 = dict(width=32, M=(0xD2511F53, 0xCD9E8D57), W=(0x9E3779B9, 0xBB67AE85))
PHILOX4x64 = dict(width=64, M=(0xD2E7470EE14C6C93, 0xCA5A826395121157),
                  W=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B))


def philox_block(ctr, key, params=PHILOX4x32, rounds=10):
    """Philox on Python integers: ctr is 4 words, key is 2 words."""
    w = params["width"]
    mask = (1 << w) - 1
    M0, M1 = params["M"]
    W0, W1 = params["W"]
    c = [int(x) & mask for x in ctr]
    k = [int(x) & mask for x in key]
    for r in range(rounds):
        if r > 0:
            k = [(k[0] + W0) & mask, (k[1] + W1) & mask]
        p0 = M0 * c[0]
        p1 = M1 * c[2]
        hi0, lo0 = p0 >> w, p0 & mask
        hi1, lo1 = p1 >> w, p1 & mask
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return c


def philox4x32_np(c0, c1, c2, c3, k0, k1, rounds=10):
    """Vectorised Philox4x32 over numpy arrays of counters (uint32 words)."""
    M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
    W0, W1 = np.uint32(0x9E3779B9), np.uint32(0xBB67AE85)
    m32 = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint32) for x in (c0, c1, c2, c3)]
    shape = np.broadcast(*c).shape
    c = [np.broadcast_to(x, shape).astype(np.uint32) for x in c]
    k0 = np.uint32(k0)
    k1 = np.uint32(k1)
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r > 0:
                k0 = np.uint32((int(k0) + int(W0)) & 0xFFFFFFFF)
                k1 = np.uint32((int(k1) + int(W1)) & 0xFFFFFFFF)
            p0 = c[0].astype(np.uint64) * M0
            p1 = c[2].astype(np.uint64) * M1
            hi0 = (p0 >> np.uint64(32)).astype(np.uint32)
            lo0 = (p0 & m32).astype(np.uint32)
            hi1 = (p1 >> np.uint64(32)).astype(np.uint32)
            lo1 = (p1 & m32).astype(np.uint32)
            c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def element_r16(idx, seed, stream_id, tensor_tag=0):
    """16-bit random draw of each logical element index (numpy int64 array)."""
    idx = np.asarray(idx, dtype=np.int64)
    n = (idx // 8).astype(np.uint64)
    lo = (n & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = (n >> np.uint64(32)).astype(np.uint32)
    seed = int(seed)
    words = philox4x32_np(lo, hi, np.uint32(stream_id), np.uint32(tensor_tag),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    which = (idx % 8) // 2
    w = np.choose(which, words)
    return np.where(idx % 2 == 0, w & 0xFFFF, w >> 16).astype(np.int64)

"""Oracle: sampled drafting by Gumbel-top-k (test infrastructure only: imported
by tests/ and the smoke check, never by the product path).

Follows
  * "Speculative Decoding Deep Dive III", section "EAGLE-1", "Inference": the
    drafter samples its next token from its own distribution, t ~ p-hat;
  * for k children per node, k tokens are drawn without replacement from
    softmax(s * logits): the k largest of s * logits + G, with G independent
    standard Gumbel variables (the Gumbel-top-k trick; for k = 1 it is the
    Gumbel-max identity).

Random numbers come from one counter-based generator, Philox4x32-10 (Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11),
written here from its published definition:
  * ten rounds; each multiplies words 0 and 2 of the counter by 0xD2511F53 and
    0xCD9E8D57 (64-bit products split into high and low halves) and permutes:
    (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is bumped by the Weyl
    constants 0x9E3779B9 and 0xBB67AE85 after every round.
Readings (the pages name no generator; listed in the design notes):
  * key = the 64-bit round seed (low word, high word); counter = (id // 4,
    row key, 0, 0), the four outputs serving ids 4q .. 4q + 3; the row key of
    a draft row is b * pool_cap + node (unique within a round);
  * u = ((bits >> 9) + 0.5) * 2^-23 (23 bits, so the sum is exact in fp32
    and 2^-24 <= u <= 1 - 2^-24);
    G = -log(-log(u)) and the key s * logit + G are formed in fp32.
"""
from __future__ import annotations

import numpy as np

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 on uint32 arrays: counter = (c0, c1, c2, c3), key =
    (k0, k1) (broadcast together).  Returns the four output words."""
    c = [np.asarray(x, np.uint64) & _LO for x in counter]
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _LO
        hi1, lo1 = p1 >> np.uint64(32), p1 & _LO
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return [x.astype(np.uint32) for x in c]


def uniforms(seed, row_key, V):
    """u in (0, 1), float32 [V], for one draft row."""
    ids = np.arange(V, dtype=np.uint64)
    q = ids >> np.uint64(2)
    z = np.zeros_like(q)
    words = philox4x32_10((q, np.full_like(q, row_key & 0xFFFFFFFF), z, z),
                          (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    w = np.stack(words)[(ids & np.uint64(3)).astype(np.int64), np.arange(V)]
    return ((w >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def gumbel(seed, row_key, V):
    """Standard Gumbel variables -log(-log(u)) in fp32, [V]."""
    u = uniforms(seed, row_key, V)
    return -np.log(-np.log(u))


def gumbel_keys(logits, inv_temp, seed, row_key):
    """s * logits + G in fp32 for one row."""
    l32 = np.asarray(logits, np.float32)
    return (np.float32(inv_temp) * l32) + gumbel(seed, row_key, l32.shape[-1])


def gumbel_topk(logits, k, inv_temp, seed, row_key):
    """k token ids drawn without replacement from softmax(s * logits): the k
    largest keys, ties by lowest id.  Returns (ids [k], keys [V])."""
    key = gumbel_keys(logits, inv_temp, seed, row_key)
    order = np.lexsort((np.arange(key.size), -key.astype(np.float64)))
    return order[:k], key

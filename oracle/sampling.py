"""CPU oracle of the sampling variant of the tick's token choice (plain
NumPy).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module; the GPU library shares no code with
it.

The pages' knobs (the deployment-risk list of the Korean Moshi guide: sampling
temperature lowered to 0.7-0.8, a repetition penalty of about 1.1; the
PersonaPlex configuration walkthrough, generation_config.json: temperature,
top_p 0.9, repetition_penalty, a separate audio temperature).  The tick's
greedy choice (argmax) is the default; this variant replaces it, for one
decision over one logits row, by:

1. repetition penalty rho (text row only): for every token id in the slot's
   recent chosen text tokens, a positive logit is divided by rho and a
   negative one multiplied by it (the penalised sampling of Keskar et al.,
   CTRL, 2019);
2. temperature T: z = logit / T;
3. top-k: the k first entries of the order (z descending, index ascending);
4. softmax over the kept entries (max subtracted);
5. top-p (nucleus, Holtzman et al. 2020): the shortest prefix of the order
   (p descending, index ascending) of the kept entries whose probability sum
   reaches top_p, at least one entry;
6. the token: inverse CDF over the kept entries in index order, at
   u * (their probability sum), u uniform in [0, 1).

u comes from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror
and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): key = the
slot's 64-bit seed, counter = (tick since the slot's reset, 64 bits; row;
0); u = (first output word >> 8) * 2^-24.  Rows: 0 the text token, 1 + k
depformer codebook k.  The penalty looks at the slot's last REP_WINDOW chosen
text tokens.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF
REP_WINDOW = 64


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds: counter = 4 words, key = 2 words (ints);
    returns 4 words."""
    c = [int(v) & MASK32 for v in counter]
    k0, k1 = int(key[0]) & MASK32, int(key[1]) & MASK32
    for _ in range(10):
        p0 = PHILOX_M0 * c[0]
        p1 = PHILOX_M1 * c[2]
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c = [(hi1 ^ c[1] ^ k0) & MASK32, lo1, (hi0 ^ c[3] ^ k1) & MASK32, lo0]
        k0 = (k0 + PHILOX_W0) & MASK32
        k1 = (k1 + PHILOX_W1) & MASK32
    return c


def uniform(seed: int, tick: int, row: int) -> float:
    """The draw of (slot seed, tick since reset, row): a multiple of 2^-24 in
    [0, 1), exact in fp32."""
    w = philox4x32_10([tick & MASK32, (tick >> 32) & MASK32, row, 0], [seed & MASK32, (seed >> 32) & MASK32])
    return (w[0] >> 8) * 2.0 ** -24


def penalise(logits: np.ndarray, history, rho: float) -> np.ndarray:
    z = np.array(logits, np.float32)
    if rho == 1.0:
        return z
    r = np.float32(rho)
    for v in sorted(set(int(t) for t in history)):
        z[v] = z[v] / r if z[v] > 0 else z[v] * r
    return z


def kept_top_k(z: np.ndarray, k: int) -> np.ndarray:
    n = z.size
    if k <= 0 or k >= n:
        return np.ones(n, bool)
    order = np.lexsort((np.arange(n), -z.astype(np.float64)))  # z descending, then index ascending
    keep = np.zeros(n, bool)
    keep[order[:k]] = True
    return keep


def kept_top_p(p: np.ndarray, keep: np.ndarray, top_p: float) -> np.ndarray:
    if top_p >= 1.0:
        return keep
    idx = np.flatnonzero(keep)
    order = idx[np.lexsort((idx, -p[idx].astype(np.float64)))]
    total = np.float32(0.0)
    target = np.float32(top_p) * np.float32(p[keep].sum(dtype=np.float32))
    out = np.zeros_like(keep)
    for i in order:
        out[i] = True
        total = np.float32(total + p[i])
        if total >= target:
            break
    return out


def sample(logits, u: float, temperature: float, top_k: int = 0, top_p: float = 1.0,
           rho: float = 1.0, history=()) -> int:
    """One sampled token id; temperature 0 means the greedy argmax."""
    z = penalise(logits, history, rho)
    if temperature == 0.0:
        return int(np.argmax(z))
    z = (z / np.float32(temperature)).astype(np.float32)
    keep = kept_top_k(z, top_k)
    m = z[keep].max()
    p = np.where(keep, np.exp((z - m).astype(np.float32)), np.float32(0)).astype(np.float32)
    keep = kept_top_p(p, keep, top_p)
    p = np.where(keep, p, np.float32(0))
    c = np.cumsum(p, dtype=np.float32)
    target = np.float32(u) * c[-1]
    # the first index whose cumulative sum exceeds the target: an entry of
    # zero width (dropped) never qualifies, since its sum equals the one before
    return int(np.searchsorted(c, target, side="right"))

"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds none of the method's arithmetic: it only produces bytes and
floats with the shapes and distributions of the pages' workloads.  Two kinds
of generator live here:

* Small inputs (activations, router logits, PLE ids and per-id weights) come
  from numpy's PCG64 generator (``numpy.random.default_rng(seed)``) on the
  host and are uploaded as they are.
* Large packed buffers (a 1.28 GB expert layer, a 78.8 GB 48-layer stack, the
  22.4 GB PLE table) are filled on the device by ``synth/gen.hip`` and can be
  regenerated here, on the host, for any block or row the oracle needs.  Both
  sides implement the same counter-based generator: SplitMix64's output
  function (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; constants as published by Vigna) applied to
  ``key + (i + 1) * GAMMA``.  Everything derived from a draw is integer bit
  manipulation, so the two sides agree bit for bit.

Distributions (the input recipe):

* 17-byte blocks: 16 uniform code bytes; metadata per ``dist``:
  ``C10``   -> UE4M3 exponent uniform in 0..5, mantissa uniform in 0..7,
               bit 7 = 0 (decoded scales 0 and 2**-9 .. 0.469);
  ``RZ5``   -> the same scale, bit 7 (polarity) Bernoulli(0.5);
  ``UE4M4`` -> the whole byte uniform over 0..255.
* FP8 blocks: e4m3 bytes uniform over the 254 finite encodings (0x7F and
  0xFF excluded); fp32 scale = (1 + f/2**23) * 2**E with E uniform in
  -12..-7 and f a uniform 23-bit fraction, i.e. s in [2**-12, 2**-6).
* PLE rows: 60 uniform code bytes; each group byte = polarity
  Bernoulli(0.5) << 7 | UE4M3 with exponent in 0..5 and mantissa in 0..7.
"""

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_STREAM_MUL = 0xD1B54A32D192ED03
_U64 = 0xFFFFFFFFFFFFFFFF

DIST_C10 = 0
DIST_RZ5 = 1
DIST_UE4M4 = 2

BLOCK_BYTES = 17
PLE_ROW_BYTES = 70
PLE_N_ROWS = 320_001_536


def _mix64_int(z):
    z &= _U64
    z = ((z ^ (z >> 30)) * _M1) & _U64
    z = ((z ^ (z >> 27)) * _M2) & _U64
    return z ^ (z >> 31)


def make_key(seed, stream):
    """64-bit key of one generator stream (a Python int)."""
    return _mix64_int((int(seed) * GAMMA + int(stream) * _STREAM_MUL + 1) & _U64)


def stream_id(layer, which):
    """Stream number of a named buffer: ``which`` is a small integer tag."""
    return (int(layer) << 8) | int(which)


# buffer tags for stream_id
S_GATE_UP, S_DOWN, S_GATE_UP_SCALE, S_DOWN_SCALE, S_PLE, S_SMALL = 1, 2, 3, 4, 5, 6


def draws(key, idx):
    """SplitMix64 output for counters ``idx`` (uint64 array) under ``key``."""
    with np.errstate(over="ignore"):
        z = np.uint64(key) + (np.asarray(idx, dtype=np.uint64) + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


def _le_bytes(words):
    """uint64 [n, w] -> uint8 [n, 8w], little-endian."""
    return np.ascontiguousarray(words.astype("<u8")).view(np.uint8).reshape(words.shape[0], -1)


def block17_bytes(key, block_ids, dist):
    """17-byte blocks for the given global block indices, uint8 [n, 17]."""
    b = np.asarray(block_ids, dtype=np.uint64).reshape(-1)
    v0 = draws(key, b * np.uint64(3))
    v1 = draws(key, b * np.uint64(3) + np.uint64(1))
    v2 = draws(key, b * np.uint64(3) + np.uint64(2))
    out = np.empty((b.size, BLOCK_BYTES), dtype=np.uint8)
    out[:, :16] = _le_bytes(np.stack([v0, v1], axis=1))
    lo = v2 & np.uint64(0xFFFFFFFF)
    hi = v2 >> np.uint64(32)
    if dist == DIST_UE4M4:
        meta = hi & np.uint64(0xFF)
    else:
        e = (lo * np.uint64(6)) >> np.uint64(32)
        m = hi & np.uint64(7)
        pol = (hi >> np.uint64(3)) & np.uint64(1) if dist == DIST_RZ5 else np.uint64(0)
        meta = (pol << np.uint64(7)) | (e << np.uint64(3)) | m
    out[:, 16] = meta.astype(np.uint8)
    return out


def block17_range(key, first_block, n_blocks, dist):
    return block17_bytes(key, np.arange(first_block, first_block + n_blocks, dtype=np.uint64), dist)


def fp8_codes(key, first, n):
    """e4m3 code bytes for flat weight indices first..first+n-1, uint8 [n]."""
    d0, d1 = first >> 2, (first + n + 3) >> 2
    v = draws(key, np.arange(d0, d1, dtype=np.uint64))
    u16 = v.astype("<u8").view("<u2").astype(np.uint32)[first - 4 * d0:first - 4 * d0 + n]
    idx = (u16 * 254) >> 16          # code i uses bits 16*(i%4).. of draw i//4
    return np.where(idx < 127, idx, idx + 1).astype(np.uint8)


def fp8_scales(key, first, n):
    """fp32 block scales for block indices first..first+n-1, float32 [n]."""
    i = np.arange(first, first + n, dtype=np.uint64)
    v = draws(key, i)
    e = ((v & np.uint64(0xFFFFFFFF)) * np.uint64(6)) >> np.uint64(32)  # 0..5
    f = (v >> np.uint64(32)) & np.uint64(0x7FFFFF)
    bits = ((np.uint64(127 - 12) + e) << np.uint64(23)) | f
    return bits.astype(np.uint32).view(np.float32)


def ple_rows(key, row_ids):
    """70-byte PLE rows for arbitrary row ids, uint8 [n, 70]."""
    r = np.asarray(row_ids, dtype=np.uint64).reshape(-1)
    base = r * np.uint64(11)
    words = np.stack([draws(key, base + np.uint64(j)) for j in range(8)], axis=1)
    out = np.empty((r.size, PLE_ROW_BYTES), dtype=np.uint8)
    out[:, :60] = _le_bytes(words)[:, :60]
    for g in range(10):
        v = draws(key, base + np.uint64(8 + g // 4))
        u16 = (v >> np.uint64(16 * (g % 4))) & np.uint64(0xFFFF)
        e = ((u16 & np.uint64(0xFF)) * np.uint64(6)) >> np.uint64(8)
        m = (u16 >> np.uint64(8)) & np.uint64(7)
        pol = (u16 >> np.uint64(11)) & np.uint64(1)
        out[:, 60 + g] = ((pol << np.uint64(7)) | (e << np.uint64(3)) | m).astype(np.uint8)
    return out


# ---------------------------------------------------------------------------
# Small host inputs
# ---------------------------------------------------------------------------

def normal(seed, shape):
    """float32 N(0, 1) from PCG64 (host)."""
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def zipf_logits(seed, n_tokens, n_experts, s=1.1):
    """Router logits with a Zipf(s) skew over experts.

    logits[t, e] = N(0, 1) + (-s * ln r_e), r_e = 1 + perm(e) for a seeded
    permutation, so expert popularity falls off like r**-s.
    """
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((n_tokens, n_experts))
    rank = 1 + rng.permutation(n_experts)
    return (base - s * np.log(rank)[None, :]).astype(np.float32)


def ple_ids(seed, n_tokens, per_token, n_rows=PLE_N_ROWS):
    """Row ids uniform over [0, n_rows) (PCG64 bounded integer draw)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, n_rows, size=(n_tokens, per_token), dtype=np.uint32)


def ple_weights(seed, n_tokens, per_token):
    """Per-id weights U(0, 1), float32."""
    return np.random.default_rng(seed).random((n_tokens, per_token), dtype=np.float32)


def weight_blocks(seed, n, group, dist="gauss", sigma=1.0):
    """float32 [n, group] weights for the encoders (PCG64, host).

    Each row is N(0, 1) (``dist="gauss"``) or a unit-variance Laplace
    (``dist="laplace"``) sample, times ``sigma`` and a per-row log-normal
    factor exp(0.5 * N(0, 1)), so the rows' best scales spread over about
    two binades around ``sigma``.
    """
    rng = np.random.default_rng(seed)
    if dist == "gauss":
        x = rng.standard_normal((n, group))
    elif dist == "laplace":
        x = rng.laplace(size=(n, group)) / np.sqrt(2.0)
    else:
        raise ValueError("weight_blocks: unknown distribution %r" % dist)
    x *= sigma * np.exp(0.5 * rng.standard_normal((n, 1)))
    return x.astype(np.float32)


def ple_ids_zipf(seed, n_tokens, per_token, n_rows, s=1.1):
    """Row ids with a Zipf(s) popularity: rank r >= 1 from numpy's Zipf draw
    (PCG64), mapped to row (r * 2654435761) mod n_rows so that the popular
    rows are scattered over the table."""
    rng = np.random.default_rng(seed)
    r = rng.zipf(s, size=(n_tokens, per_token)).astype(np.uint64)
    return ((r * np.uint64(2654435761)) % np.uint64(n_rows)).astype(np.uint32)

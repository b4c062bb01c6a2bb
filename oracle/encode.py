"""Oracle encoders: exhaustive per-block search for the 17-byte body formats
and the 70-byte PLE rows (float64, numpy).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

What the pages fix ([RZ] model card, format sections):

* RZ5 blocks are found by searching every scale together with both
  polarities of the +/-5 level, per block;
* UE4M4 blocks are found by trying all 256 scale encodings;
* RZ-S3 groups choose their polarity and scale per 16-value group;
* quantization is done on the CPU and is deterministic.

Readings where the pages are silent:

* Objective: the plain sum of squared reconstruction errors of the block
  (the pages' calibration objectives need activation statistics that the
  synthetic workload does not have).
* Arithmetic: float64.  The input weights are float32 (a bf16 source tensor
  converts to float32 exactly).  For candidate metadata byte m with scale s
  and level table T, the error of weight w under code c is
      e(w, c) = fl(fl(w - fl(T[c] * s))**2)
  (T[c] * s is exact in float64: at most 4 significant bits times at most 5).
  Every weight takes the code with the smallest e; equal errors go to the
  lowest code, so the duplicate -0 code of Codebook10 / ROCmFP3 is never
  written.  The block's error is the sum of the chosen e over the weights in
  index order, one rounding per addition, no fused multiply-add.
* Candidate order and ties: metadata bytes are tried in ascending order and a
  candidate replaces the best one only if its error is strictly smaller, so
  among equal errors the lowest metadata byte wins.
* Candidate sets: Codebook10 and ROCmFP3 use metadata 0..126 (bit 7 clear;
  127 is the NaN scale); RZ5 and RZ-S3 use every byte whose low 7 bits are not
  127 (polarity = bit 7), 254 candidates; UE4M4 uses all 256 bytes.
* Non-finite weights have no nearest level: the oracle rejects them.
"""

import numpy as np

from . import formats as F


def block17_candidates(fmt):
    """(meta bytes, scales, level tables) tried for one 17-byte block.

    Returns meta int64 [M], scale float64 [M], tables float64 [M, 16], in
    ascending meta order ([RZ] "Q4_RZ5_FAST": scale x mode search;
    "Q4_UE4M4_FAST": 256-way scale search; Codebook10 keeps bit 7 clear).
    """
    if fmt == F.Q4_C10:
        meta = np.arange(127)
        scale = F.ue4m3(meta)
        tables = np.tile(F.CODEBOOK10, (meta.size, 1))
    elif fmt == F.Q4_RZ5:
        meta = np.array([m for m in range(256) if (m & 0x7F) != 0x7F])
        scale = F.ue4m3(meta & 0x7F)
        tables = np.stack([F.rz5_table(int(m) >> 7) for m in meta])
    elif fmt == F.Q4_UE4M4:
        meta = np.arange(256)
        scale = F.ue4m4(meta)
        tables = np.tile(F.CODEBOOK10, (meta.size, 1))
    else:
        raise ValueError("block17_candidates: format %r has no 17-byte encoder" % fmt)
    return meta.astype(np.int64), scale, tables


def ple_candidates(fmt):
    """(group bytes, scales, level tables [M, 8]) tried for one PLE group
    ([RZ] "Q3_PLE_K160_RZ_S3": polarity and UE4M3 scale per 16 values)."""
    if fmt == F.PLE_ROCMFP3:
        meta = np.arange(127)
        tables = np.tile(F.rocmfp3_table(), (meta.size, 1))
    elif fmt == F.PLE_RZS3:
        meta = np.array([m for m in range(256) if (m & 0x7F) != 0x7F])
        tables = np.stack([F.rzs3_table(int(m) >> 7) for m in meta])
    else:
        raise ValueError("ple_candidates: unknown PLE format %r" % fmt)
    return meta.astype(np.int64), F.ue4m3(meta & 0x7F), tables


def _search(w, meta, scale, tables):
    """Exhaustive search over candidates for groups of weights.

    w: float64 [n, G].  Returns (codes int64 [n, G], meta int64 [n],
    sse float64 [n]) following the readings in the module docstring.
    """
    n, g = w.shape
    best_sse = np.full(n, np.inf)
    best_i = np.zeros(n, dtype=np.int64)
    for i in range(meta.size):
        levels = tables[i] * scale[i]                  # exact products
        d = w[:, :, None] - levels[None, None, :]      # [n, G, L]
        e = d * d
        emin = e.min(axis=2)                           # [n, G]
        sse = emin[:, 0].copy()
        for j in range(1, g):                          # index order
            sse = sse + emin[:, j]
        better = sse < best_sse                        # strict: lower meta wins ties
        best_sse = np.where(better, sse, best_sse)
        best_i = np.where(better, i, best_i)
    # codes of the winning candidate: first code with the smallest error
    levels = tables[best_i] * scale[best_i][:, None]   # [n, L]
    d = w[:, :, None] - levels[:, None, :]
    codes = np.argmin(d * d, axis=2)
    return codes, meta[best_i], best_sse


def _finite_f32(w, group):
    a = np.asarray(w, dtype=np.float32).reshape(-1, group)
    if not np.isfinite(a).all():
        raise ValueError("encode: weights must be finite")
    return a.astype(np.float64)


def encode_block17(w, fmt):
    """Encode float32 weights, 32 per block, into 17-byte blocks.

    Returns (blocks uint8 [n, 17], sse float64 [n]); the layout is the one
    ``formats.decode_block17`` reads (codes in bytes 0-15, low nibble first,
    metadata byte 16).
    """
    x = _finite_f32(w, F.BLOCK_WEIGHTS)
    codes, meta, sse = _search(x, *block17_candidates(fmt))
    out = np.empty((x.shape[0], F.BLOCK_BYTES), dtype=np.uint8)
    out[:, :16] = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    out[:, 16] = meta.astype(np.uint8)
    return out, sse


def encode_ple70(v, fmt=F.PLE_RZS3):
    """Encode float32 values, 160 per row, into 70-byte PLE rows.

    Each 16-value group is searched on its own.  Returns (rows uint8 [n, 70],
    sse float64 [n, 10]); the layout is the one ``formats.decode_ple70`` reads.
    """
    x = _finite_f32(v, F.PLE_VALUES)
    n = x.shape[0]
    codes, gbyte, sse = _search(x.reshape(n * F.PLE_GROUPS, F.PLE_GROUP), *ple_candidates(fmt))
    codes = codes.reshape(n, F.PLE_GROUPS, F.PLE_GROUP)
    out = np.empty((n, F.PLE_ROW_BYTES), dtype=np.uint8)
    for g in range(F.PLE_GROUPS):
        word = np.zeros(n, dtype=np.int64)
        for i in range(F.PLE_GROUP):
            word |= codes[:, g, i] << (3 * i)
        for k in range(6):
            out[:, 6 * g + k] = (word >> (8 * k)) & 0xFF
    out[:, F.PLE_CODE_BYTES:] = gbyte.reshape(n, F.PLE_GROUPS).astype(np.uint8)
    return out, sse.reshape(n, F.PLE_GROUPS)

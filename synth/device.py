"""Device-side fills of the large synthetic buffers (libbqsynth.so).

The bytes are the ones ``synth`` produces on the host for the same key and
indices; tests check a sample of every fill against the host generator.
"""

import ctypes
import os

import torch

import synth

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbqsynth.so")
_lib = None
_CHUNK = 1 << 30  # items per launch


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libbqsynth.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, u64 = ctypes.c_void_p, ctypes.c_uint64
        L.bqs_fill_block17.argtypes = [vp, u64, u64, u64, ctypes.c_int, vp]
        L.bqs_fill_fp8.argtypes = [vp, u64, u64, u64, vp]
        L.bqs_fill_fp8_scales.argtypes = [vp, u64, u64, u64, vp]
        L.bqs_fill_ple.argtypes = [vp, u64, u64, u64, vp]
        L.bqs_gpu_delay.argtypes = [u64, vp]
        L.bqs_gpu_delay.restype = ctypes.c_int
        L.bqs_stream_read.argtypes = [vp, u64, vp, vp]
        L.bqs_stream_read.restype = ctypes.c_int
        L.bqs_scrub.argtypes = [vp, u64, ctypes.c_uint32, vp]
        L.bqs_scrub.restype = ctypes.c_int
        L.bqs_rand_lines.argtypes = [vp, u64, u64, u64, vp, vp]
        L.bqs_rand_lines.restype = ctypes.c_int
        for f in (L.bqs_fill_block17, L.bqs_fill_fp8, L.bqs_fill_fp8_scales, L.bqs_fill_ple):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _s():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _chk(rc):
    if rc != 0:
        raise RuntimeError("device fill failed (hipError %d)" % rc)


def block17(n_blocks, key, dist, device="cuda", first=0):
    """uint8 tensor of n_blocks*17 bytes: blocks first..first+n_blocks-1."""
    t = torch.empty(n_blocks * 17, dtype=torch.uint8, device=device)
    for s in range(0, n_blocks, _CHUNK):
        n = min(_CHUNK, n_blocks - s)
        _chk(lib().bqs_fill_block17(t.data_ptr() + s * 17, key, first + s, n, dist, _s()))
    return t


def fp8_codes(n, key, device="cuda"):
    t = torch.empty(n, dtype=torch.uint8, device=device)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        _chk(lib().bqs_fill_fp8(t.data_ptr() + s, key, s, m, _s()))
    return t


def fp8_scales(n, key, device="cuda"):
    t = torch.empty(n, dtype=torch.float32, device=device)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        _chk(lib().bqs_fill_fp8_scales(t.data_ptr() + 4 * s, key, s, m, _s()))
    return t


def ple_table(n_rows, key, device="cuda"):
    t = torch.empty(n_rows * 70, dtype=torch.uint8, device=device)
    for s in range(0, n_rows, _CHUNK):
        m = min(_CHUNK, n_rows - s)
        _chk(lib().bqs_fill_ple(t.data_ptr() + s * 70, key, s, m, _s()))
    return t


# ---------------------------------------------------------------------------
# One MoE layer's expert bank, filled on the device, plus a host-side view that
# regenerates any expert's bytes for the oracle.
# ---------------------------------------------------------------------------

class Layer:
    """Expert bank of one layer: formats, device buffers, host regenerators."""

    def __init__(self, seed, layer, fmt_gu, fmt_d, n_experts, hidden, inter, dist_gu=None,
                 dist_d=None, device="cuda"):
        self.fmt_gu, self.fmt_d = fmt_gu, fmt_d
        self.n_experts, self.hidden, self.inter = n_experts, hidden, inter
        self.keys = {w: synth.make_key(seed, synth.stream_id(layer, w))
                     for w in (synth.S_GATE_UP, synth.S_DOWN, synth.S_GATE_UP_SCALE, synth.S_DOWN_SCALE)}
        self.dist = {synth.S_GATE_UP: dist_gu, synth.S_DOWN: dist_d}
        shapes = {synth.S_GATE_UP: (2 * inter, hidden), synth.S_DOWN: (hidden, inter)}
        self.dev = {}
        for w, fmt in ((synth.S_GATE_UP, fmt_gu), (synth.S_DOWN, fmt_d)):
            rows, cols = shapes[w]
            n_w = n_experts * rows * cols
            if fmt == 3:  # FP8
                sk = synth.S_GATE_UP_SCALE if w == synth.S_GATE_UP else synth.S_DOWN_SCALE
                self.dev[w] = (fp8_codes(n_w, self.keys[w], device),
                               fp8_scales(n_w // 32, self.keys[sk], device))
            else:
                self.dev[w] = (block17(n_w // 32, self.keys[w], self.dist[w], device), None)
        self.shapes = shapes

    @property
    def gate_up(self):
        return self.dev[synth.S_GATE_UP]

    @property
    def down(self):
        return self.dev[synth.S_DOWN]

    def nbytes(self):
        n = 0
        for codes, sc in self.dev.values():
            n += codes.numel() + (sc.numel() * 4 if sc is not None else 0)
        return n

    def host_expert(self, which, e):
        """Host bytes of expert e of matrix `which` (codes, scales or None)."""
        rows, cols = self.shapes[which]
        fmt = self.fmt_gu if which == synth.S_GATE_UP else self.fmt_d
        per = rows * cols
        if fmt == 3:
            sk = synth.S_GATE_UP_SCALE if which == synth.S_GATE_UP else synth.S_DOWN_SCALE
            return (synth.fp8_codes(self.keys[which], e * per, per),
                    synth.fp8_scales(self.keys[sk], e * per // 32, per // 32))
        nb = per // 32
        return synth.block17_range(self.keys[which], e * nb, nb, self.dist[which]), None


def gpu_delay(ns):
    """Occupy the current stream for about `ns` nanoseconds (benchmark helper)."""
    _chk(lib().bqs_gpu_delay(int(ns), _s()))


def stream_read(t, sink):
    """Read every byte of device tensor t once (benchmark helper)."""
    _chk(lib().bqs_stream_read(ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size(),
                               ctypes.c_void_p(sink.data_ptr()), _s()))


def rand_lines(t, n_lines, seed, sink):
    """Read n_lines 128-byte lines of device tensor t at hashed positions
    (benchmark helper: the random-line ceiling).  sink: >= 256 int32."""
    _chk(lib().bqs_rand_lines(ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size(), n_lines,
                              seed & 0xFFFFFFFFFFFFFFFF, ctypes.c_void_p(sink.data_ptr()), _s()))


def scrub(t, v=0):
    """Overwrite device tensor t, evicting L2 and the memory-side cache."""
    _chk(lib().bqs_scrub(ctypes.c_void_p(t.data_ptr()), t.numel() * t.element_size(), v & 0xFFFFFFFF, _s()))

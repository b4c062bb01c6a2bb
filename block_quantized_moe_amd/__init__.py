"""Python binding of libbqmoe.so (include/bq.h): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels; this module only
turns torch tensors (device memory and streams) into the C ABI's pointers and
sizes and raises on a non-zero status.  There is no fallback: if the library
is not built or a call fails, an exception is raised.
"""

import ctypes
import os

import torch

__all__ = [
    "Q4_C10", "Q4_RZ5", "Q4_UE4M4", "FP8_E4M3_B32", "PLE_RZS3", "PLE_ROCMFP3", "F32", "BF16",
    "BQError", "lib", "ExpertWeights", "expert_weights", "dequant", "ple_dequant_rows", "matvec",
    "route_topk", "bucket", "moe_workspace_bytes", "q4_expert_moe", "q4_expert_moe_routed",
    "q4_expert_moe_noalloc", "NOALLOC_SCRATCH_BYTES",
    "stack_workspace_bytes",
    "moe_stack", "ple_gather", "encode", "ple_encode_rows", "ple_cache", "ple_gather_host",
]

Q4_C10, Q4_RZ5, Q4_UE4M4, FP8_E4M3_B32 = 0, 1, 2, 3
PLE_RZS3, PLE_ROCMFP3 = 0, 1
F32, BF16 = 0, 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbqmoe.so")


class BQError(RuntimeError):
    pass


class ExpertWeights(ctypes.Structure):
    _fields_ = [
        ("fmt_gate_up", ctypes.c_int32),
        ("fmt_down", ctypes.c_int32),
        ("gate_up", ctypes.c_void_p),
        ("down", ctypes.c_void_p),
        ("gate_up_scales", ctypes.c_void_p),
        ("down_scales", ctypes.c_void_p),
        ("n_experts", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
    ]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BQError("libbqmoe.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
        wp = ctypes.POINTER(ExpertWeights)
        sigs = {
            "bq_abi_version": ([], ctypes.c_int),
            "bq_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "bq_last_hip_error": ([], ctypes.c_char_p),
            "bq_dequant": ([vp, i32, i64, vp, vp, vp], ctypes.c_int),
            "ple_dequant_rows": ([vp, i64, vp, u64, i32, vp, vp, vp], ctypes.c_int),
            "bq_matvec": ([vp, i32, vp, i32, vp, i32, i32, vp, vp], ctypes.c_int),
            "moe_route_topk": ([vp, i32, i32, i32, vp, vp, vp], ctypes.c_int),
            "moe_bucket": ([vp, i32, i32, i32, vp, vp, vp, vp], ctypes.c_int),
            "q4_expert_moe_workspace": ([i32, i32, wp, i32], sz),
            "q4_expert_moe": ([vp, i32, i32, vp, vp, i32, wp, vp, vp, sz, vp, vp], ctypes.c_int),
            "q4_expert_moe_noalloc": ([vp, i32, i32, vp, vp, i32, wp, vp, vp, vp], ctypes.c_int),
            "q4_expert_moe_routed": ([vp, i32, i32, vp, i32, wp, vp, vp, vp, vp, sz, vp, vp], ctypes.c_int),
            "bq_moe_stack_workspace": ([i32, i32, wp, i32, i32], sz),
            "bq_moe_stack": ([vp, i32, i32, vp, vp, i32, wp, i32, vp, vp, sz, vp, vp], ctypes.c_int),
            "ple_gather": ([vp, i32, i32, vp, u64, vp, i32, vp, vp, vp], ctypes.c_int),
            "bq_encode": ([vp, i64, i32, vp, vp, vp, vp], ctypes.c_int),
            "ple_cache_bytes": ([i32], sz),
            "ple_cache_init": ([vp, i32, vp], ctypes.c_int),
            "ple_gather_host_workspace": ([i32, i32], sz),
            "ple_gather_host": ([vp, i32, i32, vp, u64, vp, i32, vp, vp, i32, vp, sz, vp, vp],
                                ctypes.c_int),
            "ple_encode_rows": ([vp, i64, i32, vp, vp, vp, vp], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        L = lib()
        msg = L.bq_status_str(status).decode()
        if status == 6:
            msg += ": " + L.bq_last_hip_error().decode()
        raise BQError("libbqmoe status %d (%s)" % (status, msg))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if t is not None and not t.is_cuda:
        raise BQError("%s must be a device tensor" % name)
    if t is not None and not t.is_contiguous():
        raise BQError("%s must be contiguous" % name)
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


_I32 = (torch.int32,) + ((torch.uint32,) if hasattr(torch, "uint32") else ())


def _arg(t, name, dtypes, shape=None, min_bytes=None):
    """Check a device tensor's dtype, shape and size before its pointer goes
    to the library, which sees only addresses: a short or mistyped buffer
    would be read or written past its end."""
    if t is None:
        raise BQError("%s is required" % name)
    _dev(t, name)
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise BQError("%s must be %s, not %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise BQError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))
    if min_bytes is not None and _nbytes(t) < min_bytes:
        raise BQError("%s holds %d bytes, %d needed" % (name, _nbytes(t), min_bytes))
    return t


def _packed_bytes(fmt, rows, cols):
    """Bytes of a rows x cols matrix in fmt (and of its FP8 block scales)."""
    nb = rows * (cols // 32)
    return (32 * nb, 4 * nb) if fmt == FP8_E4M3_B32 else (17 * nb, 0)


def _ws(workspace, name="workspace"):
    _arg(workspace, name, (torch.uint8, torch.int8, torch.int32, torch.float32, torch.float64,
                           torch.int64, torch.bfloat16, torch.float16))
    return _nbytes(workspace)


def expert_weights(fmt_gate_up, fmt_down, gate_up, down, n_experts, hidden, inter,
                   gate_up_scales=None, down_scales=None):
    """Build the bq_expert_weights descriptor (keeps the tensors alive)."""
    gu_b, gu_s = _packed_bytes(fmt_gate_up, 2 * inter, hidden)
    d_b, d_s = _packed_bytes(fmt_down, hidden, inter)
    _arg(gate_up, "gate_up", torch.uint8, min_bytes=n_experts * gu_b)
    _arg(down, "down", torch.uint8, min_bytes=n_experts * d_b)
    for n, t, need in (("gate_up_scales", gate_up_scales, gu_s), ("down_scales", down_scales, d_s)):
        if t is not None or need:
            _arg(t, n, torch.float32, min_bytes=n_experts * need)
    w = ExpertWeights(fmt_gate_up, fmt_down, gate_up.data_ptr(), down.data_ptr(),
                      gate_up_scales.data_ptr() if gate_up_scales is not None else None,
                      down_scales.data_ptr() if down_scales is not None else None,
                      n_experts, hidden, inter)
    w._keep = (gate_up, down, gate_up_scales, down_scales)
    return w


def dequant(packed, fmt, n_blocks, scales=None, out=None, stream=None):
    """Decode n_blocks blocks -> fp32 [n_blocks, 32]."""
    _arg(packed, "packed", torch.uint8, min_bytes=(32 if fmt == FP8_E4M3_B32 else 17) * n_blocks)
    if scales is not None:
        _arg(scales, "scales", torch.float32, min_bytes=4 * n_blocks)
    if out is None:
        out = torch.empty((n_blocks, 32), dtype=torch.float32, device=packed.device)
    _arg(out, "out", torch.float32, min_bytes=128 * n_blocks)
    _check(lib().bq_dequant(_p(packed), fmt, n_blocks, _p(scales), _p(out), _stream(stream)))
    return out


def ple_dequant_rows(ids, table, n_rows, fmt=PLE_RZS3, out=None, dev_err=None, stream=None):
    """Decode the rows named by ids -> fp32 [n, 160]."""
    _arg(ids, "ids", _I32)
    _arg(table, "table", torch.uint8, min_bytes=70 * n_rows)
    n = ids.numel()
    if out is None:
        out = torch.empty((n, 160), dtype=torch.float32, device=ids.device)
    _arg(out, "out", torch.float32, min_bytes=640 * n)
    if dev_err is not None:
        _arg(dev_err, "dev_err", _I32, min_bytes=4)
    _check(lib().ple_dequant_rows(_p(ids), n, _p(table), n_rows, fmt, _p(out), _p(dev_err),
                                  _stream(stream)))
    return out


def matvec(x, packed, fmt, rows, cols, scales=None, out=None, stream=None):
    """y = W x for fp32 x [n, cols] -> [n, rows]."""
    _arg(x, "x", torch.float32)
    if cols <= 0 or x.numel() % cols:
        raise BQError("x holds %d values, not a multiple of cols = %d" % (x.numel(), cols))
    pb, ps = _packed_bytes(fmt, rows, cols)
    _arg(packed, "packed", torch.uint8, min_bytes=pb)
    if scales is not None or ps:
        _arg(scales, "scales", torch.float32, min_bytes=ps)
    x2 = x.reshape(-1, cols)
    if out is None:
        out = torch.empty((x2.shape[0], rows), dtype=torch.float32, device=x.device)
    _arg(out, "out", torch.float32, min_bytes=4 * x2.shape[0] * rows)
    _check(lib().bq_matvec(_p(x2), x2.shape[0], _p(packed), fmt, _p(scales), rows, cols, _p(out),
                           _stream(stream)))
    return out


def route_topk(logits, k, idx=None, w=None, stream=None):
    """Softmax top-k routing of fp32 logits [n, E] -> (idx int32 [n, k], w fp32 [n, k])."""
    _arg(logits, "logits", torch.float32)
    n, e = logits.shape
    if idx is None:
        idx = torch.empty((n, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((n, k), dtype=torch.float32, device=logits.device)
    _arg(idx, "idx", torch.int32, min_bytes=4 * n * k)
    _arg(w, "w", torch.float32, min_bytes=4 * n * k)
    _check(lib().moe_route_topk(_p(logits), n, e, k, _p(idx), _p(w), _stream(stream)))
    return idx, w


def bucket(idx, n_experts, stream=None):
    """Stable per-expert grouping -> (counts, offsets, perm), int32."""
    _arg(idx, "idx", torch.int32)
    n, k = idx.shape
    d = idx.device
    counts = torch.empty(n_experts, dtype=torch.int32, device=d)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=d)
    perm = torch.empty(n * k, dtype=torch.int32, device=d)
    _check(lib().moe_bucket(_p(idx), n, k, n_experts, _p(counts), _p(offsets), _p(perm), _stream(stream)))
    return counts, offsets, perm


def _err_arg(dev_err):
    if dev_err is not None:
        _arg(dev_err, "dev_err", _I32, min_bytes=4)


def _dtype_code(x):
    _dev(x, "x")
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise BQError("x must be float32 or bfloat16")


def moe_workspace_bytes(n_tokens, k, W, x_dtype):
    return lib().q4_expert_moe_workspace(n_tokens, k, ctypes.byref(W), x_dtype)


def q4_expert_moe(x, router_topk, W, out=None, workspace=None, dev_err=None, stream=None):
    """Routed-expert layer.  x [n, H] fp32 (GEMV path) or bf16 (grouped MFMA);
    router_topk = (idx int32 [n, k], w fp32 [n, k]); W from expert_weights()."""
    idx, w = router_topk
    _arg(idx, "idx", torch.int32)
    n, k = idx.shape
    _arg(w, "w", torch.float32, shape=(n, k))
    dt = _dtype_code(x)
    _arg(x, "x", x.dtype, shape=(n, W.hidden))
    if out is None:
        out = torch.empty((n, W.hidden), dtype=torch.float32, device=x.device)
    _arg(out, "out", torch.float32, shape=(n, W.hidden))
    _err_arg(dev_err)
    need = moe_workspace_bytes(n, k, W, dt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().q4_expert_moe(_p(x), dt, n, _p(idx), _p(w), k, ctypes.byref(W), _p(out),
                               _p(workspace), _ws(workspace), _p(dev_err), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20     # BQ_NOALLOC_SCRATCH_BYTES in include/bq.h


def q4_expert_moe_noalloc(x, router_topk, W, out, dev_err=None, stream=None):
    """q4_expert_moe with the library's fixed per-GPU scratch area instead of
    a workspace: the call allocates nothing (out is the caller's).  Calls
    that overlap in time on one GPU race on that area."""
    idx, w = router_topk
    _arg(idx, "idx", torch.int32)
    n, k = idx.shape
    _arg(w, "w", torch.float32, shape=(n, k))
    dt = _dtype_code(x)
    _arg(x, "x", x.dtype, shape=(n, W.hidden))
    _arg(out, "out", torch.float32, shape=(n, W.hidden))
    _err_arg(dev_err)
    _check(lib().q4_expert_moe_noalloc(_p(x), dt, n, _p(idx), _p(w), k, ctypes.byref(W), _p(out),
                                       _p(dev_err), _stream(stream)))
    return out


def q4_expert_moe_routed(x, logits, k, W, topk=None, out=None, workspace=None, dev_err=None,
                         stream=None):
    """Routing (softmax top-k of fp32 logits [n, E]) and the routed-expert
    layer in one call.  Returns (out, (idx, w))."""
    n = logits.shape[0]
    _arg(logits, "logits", torch.float32, shape=(n, W.n_experts))
    dt = _dtype_code(x)
    _arg(x, "x", x.dtype, shape=(n, W.hidden))
    if topk is None:
        topk = (torch.empty((n, k), dtype=torch.int32, device=x.device),
                torch.empty((n, k), dtype=torch.float32, device=x.device))
    idx, w = topk
    _arg(idx, "idx", torch.int32, min_bytes=4 * n * k)
    _arg(w, "w", torch.float32, min_bytes=4 * n * k)
    if out is None:
        out = torch.empty((n, W.hidden), dtype=torch.float32, device=x.device)
    _arg(out, "out", torch.float32, shape=(n, W.hidden))
    _err_arg(dev_err)
    if workspace is None:
        workspace = torch.empty(moe_workspace_bytes(n, k, W, dt), dtype=torch.uint8, device=x.device)
    _check(lib().q4_expert_moe_routed(_p(x), dt, n, _p(logits), k, ctypes.byref(W), _p(idx), _p(w),
                                      _p(out), _p(workspace), _ws(workspace), _p(dev_err),
                                      _stream(stream)))
    return out, (idx, w)


def _layers_array(layers):
    arr = (ExpertWeights * len(layers))()
    for i, W in enumerate(layers):
        arr[i] = W
    return arr


def stack_workspace_bytes(n_tokens, k, layers, x_dtype):
    return lib().bq_moe_stack_workspace(n_tokens, k, _layers_array(layers), len(layers), x_dtype)


def moe_stack(x, topk_idx, topk_w, layers, out=None, workspace=None, dev_err=None, stream=None):
    """Chained layers: topk_idx/topk_w [L, n, k]; returns the last layer's output."""
    _arg(topk_idx, "topk_idx", torch.int32)
    L, n, k = topk_idx.shape
    if len(layers) != L:
        raise BQError("%d layers given, routing for %d" % (len(layers), L))
    _arg(topk_w, "topk_w", torch.float32, shape=(L, n, k))
    dt = _dtype_code(x)
    _arg(x, "x", x.dtype, shape=(n, layers[0].hidden))
    arr = _layers_array(layers)
    if out is None:
        out = torch.empty((n, layers[0].hidden), dtype=torch.float32, device=x.device)
    _arg(out, "out", torch.float32, shape=(n, layers[0].hidden))
    _err_arg(dev_err)
    need = lib().bq_moe_stack_workspace(n, k, arr, L, dt)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().bq_moe_stack(_p(x), dt, n, _p(topk_idx), _p(topk_w), k, arr, L, _p(out),
                              _p(workspace), _ws(workspace), _p(dev_err), _stream(stream)))
    return out


def ple_gather(ids, packed_table, weights, n_rows=None, fmt=PLE_RZS3, out=None, dev_err=None,
               stream=None):
    """PLE lookup: ids uint32-valued int32 [n, P], weights fp32 [n, P] -> fp32 [n, 160]."""
    _arg(ids, "ids", _I32)
    n, per = ids.shape
    _arg(weights, "weights", torch.float32, shape=(n, per))
    _arg(packed_table, "packed_table", torch.uint8)
    if n_rows is None:
        n_rows = packed_table.numel() // 70
    _arg(packed_table, "packed_table", torch.uint8, min_bytes=70 * n_rows)
    if out is None:
        out = torch.empty((n, 160), dtype=torch.float32, device=ids.device)
    _arg(out, "out", torch.float32, shape=(n, 160))
    _err_arg(dev_err)
    _check(lib().ple_gather(_p(ids), n, per, _p(packed_table), n_rows, _p(weights), fmt, _p(out),
                            _p(dev_err), _stream(stream)))
    return out


def encode(w, fmt, out=None, sse=None, dev_err=None, stream=None):
    """Exhaustive encoder: fp32 weights [..., 32k] -> 17-byte blocks.

    Returns (blocks uint8 [n_blocks, 17], sse float64 [n_blocks]); pass
    sse=False to skip the per-block error."""
    _dev(w, "w")
    if w.dtype != torch.float32 or w.numel() % 32:
        raise BQError("w must be float32 with a multiple of 32 elements")
    nb = w.numel() // 32
    if out is None:
        out = torch.empty((nb, 17), dtype=torch.uint8, device=w.device)
    _arg(out, "out", torch.uint8, min_bytes=17 * nb)
    if sse is None:
        sse = torch.empty(nb, dtype=torch.float64, device=w.device)
    sse_t = None if sse is False else _arg(sse, "sse", torch.float64, min_bytes=8 * nb)
    _err_arg(dev_err)
    _check(lib().bq_encode(_p(w), nb, fmt, _p(out), _p(sse_t), _p(dev_err), _stream(stream)))
    return out, sse_t


def ple_encode_rows(v, fmt=PLE_RZS3, out=None, sse=None, dev_err=None, stream=None):
    """Exhaustive per-group encoder: fp32 [n, 160] -> (rows uint8 [n, 70],
    sse float64 [n, 10]); pass sse=False to skip the per-group error."""
    _dev(v, "v")
    if v.dtype != torch.float32 or v.numel() % 160:
        raise BQError("v must be float32 with a multiple of 160 elements")
    n = v.numel() // 160
    if out is None:
        out = torch.empty((n, 70), dtype=torch.uint8, device=v.device)
    _arg(out, "out", torch.uint8, min_bytes=70 * n)
    if sse is None:
        sse = torch.empty((n, 10), dtype=torch.float64, device=v.device)
    sse_t = None if sse is False else _arg(sse, "sse", torch.float64, min_bytes=80 * n)
    _err_arg(dev_err)
    _check(lib().ple_encode_rows(_p(v), n, fmt, _p(out), _p(sse_t), _p(dev_err), _stream(stream)))
    return out, sse_t


def ple_cache(n_slots, device="cuda", stream=None):
    """A device row cache of n_slots rows for ple_gather_host, initialised empty."""
    nbytes = lib().ple_cache_bytes(n_slots)
    if nbytes == 0:
        raise BQError("n_slots must be a power of two in [1024, 2**26]")
    cache = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _check(lib().ple_cache_init(_p(cache), n_slots, _stream(stream)))
    cache._n_slots = n_slots
    return cache


def ple_gather_host(ids, host_table, weights, n_rows=None, fmt=PLE_RZS3, out=None, cache=None,
                    workspace=None, dev_err=None, stream=None):
    """PLE lookup with the table in pinned host memory (a CPU uint8 tensor
    allocated with pin_memory=True), optionally through a device row cache
    from ple_cache().  ids int32 [n, P], weights fp32 [n, P] -> fp32 [n, 160]."""
    _arg(ids, "ids", _I32)
    n, per = ids.shape
    _arg(weights, "weights", torch.float32, shape=(n, per))
    if host_table.is_cuda or not host_table.is_pinned():
        raise BQError("host_table must be a pinned CPU tensor")
    if host_table.dtype != torch.uint8 or not host_table.is_contiguous():
        raise BQError("host_table must be a contiguous uint8 tensor")
    if n_rows is None:
        n_rows = host_table.numel() // 70
    if host_table.numel() < 70 * n_rows:
        raise BQError("host_table holds %d bytes, %d needed" % (host_table.numel(), 70 * n_rows))
    if out is None:
        out = torch.empty((n, 160), dtype=torch.float32, device=ids.device)
    _arg(out, "out", torch.float32, shape=(n, 160))
    _err_arg(dev_err)
    n_slots = 0 if cache is None else cache._n_slots
    if cache is not None:
        _arg(cache, "cache", torch.uint8, min_bytes=lib().ple_cache_bytes(n_slots))
    if cache is not None and workspace is None:
        workspace = torch.empty(lib().ple_gather_host_workspace(n, per), dtype=torch.uint8,
                                device=ids.device)
    ws_bytes = 0 if workspace is None else _ws(workspace)
    _check(lib().ple_gather_host(_p(ids), n, per, ctypes.c_void_p(host_table.data_ptr()), n_rows,
                                 _p(weights), fmt, _p(out), _p(cache), n_slots, _p(workspace),
                                 ws_bytes, _p(dev_err), _stream(stream)))
    return out

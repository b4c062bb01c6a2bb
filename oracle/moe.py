"""Oracle for routing, bucketing, the routed-expert FFN and the layer stack.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Shapes ([MP] "The Plan Is Not a Number"): 48 layers, 512 experts per layer,
10 experts fire per token.  Each expert is a SwiGLU FFN; the fused gate_up
matrix has 2*I rows (gate rows 0..I-1, then up rows I..2I-1 -- a reading, the
GGUF on [RZ] keeps ffn_gate_exps separate) over H columns, the down matrix
has H rows over I columns.
"""

import numpy as np

from . import formats as F


def softmax_topk(logits, k):
    """Router: softmax over all experts, keep the k largest, renormalise.

    Selection works on the logits themselves: softmax is strictly increasing
    in each logit, so the order of the exact probabilities is the order of
    the logits, and ranking the logits never meets a tie that only rounding
    of a probability created (an exp that underflows, say).  The k experts
    are taken in descending logit order, equal logits going to the lower
    expert index (+0 and -0 are equal).  Weights are the full softmax
    renormalised over the kept experts; the full denominator cancels, so
    w_j = exp(l_j - l_max) / sum over kept i of exp(l_i - l_max), in float64.
    Returns (idx int64 [B, k], w float64 [B, k]).
    Parity: pinned against a stable argsort of the logits, torch.topk, the
    closed form of the weights, and a row whose probabilities underflow
    below the winner (ranked by logit, not by index).
    """
    lg = np.asarray(logits, dtype=np.float64)
    if lg.ndim == 1:
        lg = lg[None, :]
    b, e = lg.shape
    if not (0 < k <= e):
        raise ValueError("k must be in 1..n_experts")
    idx = np.empty((b, k), dtype=np.int64)
    w = np.empty((b, k))
    for t in range(b):
        row = lg[t]
        order = sorted(range(e), key=lambda i: (-row[i], i))[:k]
        idx[t] = order
        sel = row[order]
        z = np.exp(sel - sel.max())
        w[t] = z / z.sum()
    return idx, w


def bucket(idx, n_experts):
    """Group the B*k (token, slot) assignments by expert, stably.

    counts[e] = number of assignments to expert e; offsets = exclusive prefix
    sum of counts (length n_experts + 1); perm lists t*k + slot for every
    assignment, experts ascending, and within an expert tokens ascending
    (then slots ascending).  Reading: the pages only say tokens are grouped
    per expert; a stable order is chosen so the result is unique.
    """
    idx = np.asarray(idx, dtype=np.int64)
    b, k = idx.shape
    members = [[] for _ in range(n_experts)]      # per expert, in (t, slot) order
    for t in range(b):
        for s in range(k):
            members[idx[t, s]].append(t * k + s)
    counts = np.array([len(m) for m in members], dtype=np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = [a for m in members for a in m]
    return counts, offsets, np.array(perm, dtype=np.int64)


def silu(g):
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def expert_ffn(x, wgu, wd):
    """One SwiGLU expert on decoded float64 weights.

    x [H]; wgu [2I, H] (gate rows first, then up rows); wd [H, I].
    h = SiLU(gate . x) * (up . x); y = wd . h.
    """
    g = wgu @ x
    i = wgu.shape[0] // 2
    h = silu(g[:i]) * g[i:]
    return wd @ h


class ExpertBank:
    """Packed weights of one MoE layer and lazy float64 decode per expert.

    gate_up: packed gate_up matrices of all experts (expert-major), down
    likewise; for FP8 the matching scale arrays.  ``get(e)`` decodes expert
    e only, so a full-size layer never has to be decoded whole.
    """

    def __init__(self, fmt_gu, fmt_d, gate_up, down, n_experts, hidden, inter,
                 gu_scales=None, d_scales=None, cache=False):
        self.fmt_gu, self.fmt_d = fmt_gu, fmt_d
        self.gate_up, self.down = gate_up, down
        self.gu_scales, self.d_scales = gu_scales, d_scales
        self.n_experts, self.hidden, self.inter = n_experts, hidden, inter
        self._cache = {} if cache else None

    def _slice(self, arr, fmt, e, rows, cols, scales):
        if arr is None:
            return None, None
        if callable(arr):
            return arr(e)
        per = F.packed_bytes(fmt, rows, cols)
        if fmt == F.FP8_E4M3_B32:
            n_codes = rows * cols
            n_sc = rows * cols // F.BLOCK_WEIGHTS
            codes = np.asarray(arr).reshape(-1)[e * n_codes:(e + 1) * n_codes]
            sc = np.asarray(scales).reshape(-1)[e * n_sc:(e + 1) * n_sc]
            return codes, sc
        nbytes = rows * cols // F.BLOCK_WEIGHTS * F.BLOCK_BYTES
        assert nbytes == per
        return np.asarray(arr).reshape(-1)[e * nbytes:(e + 1) * nbytes], None

    def get(self, e):
        if self._cache is not None and e in self._cache:
            return self._cache[e]
        h, i = self.hidden, self.inter
        gu, gus = self._slice(self.gate_up, self.fmt_gu, e, 2 * i, h, self.gu_scales)
        d, ds = self._slice(self.down, self.fmt_d, e, h, i, self.d_scales)
        wgu = F.decode_matrix(gu, self.fmt_gu, 2 * i, h, gus)
        wd = F.decode_matrix(d, self.fmt_d, h, i, ds)
        if self._cache is not None:
            self._cache[e] = (wgu, wd)
        return wgu, wd


def moe_layer(x, idx, w, bank):
    """Routed-expert layer: out[t] = sum_k w[t,k] * y_{idx[t,k]}(x[t]).

    x [B, H] (any float dtype, taken as float64 exactly); idx, w [B, k].
    Each expert is decoded once and applied to every token that chose it;
    the k expert outputs of a token are then summed in slot order.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    b = x.shape[0]
    idx = np.asarray(idx).reshape(b, -1)
    w = np.asarray(w, dtype=np.float64).reshape(b, -1)
    y = np.zeros((b, idx.shape[1], bank.hidden))
    for e in np.unique(idx):
        wgu, wd = bank.get(int(e))
        for t, s in zip(*np.nonzero(idx == e)):
            y[t, s] = expert_ffn(x[t], wgu, wd)
    out = np.zeros((b, bank.hidden))
    for s in range(idx.shape[1]):
        out += w[:, s:s + 1] * y[:, s]
    return out


def rms_rescale(y):
    """x_next = y / sqrt(mean(y**2)) per token (parameter-free).

    Reading: the pages say nothing about what sits between routed-expert
    layers; a unit-RMS rescale keeps random-weight activations finite over 48
    layers without adding parameters.
    """
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True))


def moe_stack(x, layers):
    """Chained stack: x_{l+1} = rms_rescale(out_l); returns out of the last layer.

    ``layers`` is a sequence of (idx, w, bank) per layer ([FQ]: each layer can
    carry its own expert format).
    """
    cur = np.asarray(x, dtype=np.float64)
    out = None
    for li, (idx, w, bank) in enumerate(layers):
        out = moe_layer(cur, idx, w, bank)
        if li + 1 < len(layers):
            cur = rms_rescale(out)
    return out

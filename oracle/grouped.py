"""Grouped fp64 evaluation of the expert outputs and of Refill-RMS (test infrastructure).

Only the tests may import this module.  It computes the same quantities as
``moe_oracle.c``'s per-pair expert outputs and its Refill-RMS re-evaluation,
from the same definitions:

* expert output o = W_down ( silu(W_gate x) * (W_up x) ), silu(a) = a / (1 + e^-a),
  all in fp64 with no intermediate rounding (Qwen3.8-Flash-Next architecture
  sheet, FFN / MoE entries: SwiGLU experts, no bias, no clamp); AWQ weights
  decoded exactly as (q - z) * s (Qwen3.8-Flash-Next-AWQ-g32 card,
  "Checkpoint"; nibble order as in include/moe.h);
* Refill-RMS (RAZOR E256of512 card, "Selection and calibration"): for each
  valid token and each selected expert j, the layer output re-evaluated with
  j dropped and the highest-ranked unselected expert promoted, gates
  renormalised over the new set; ||y' - y||^2 added to sum[j], 1 to count[j].

The difference from ``moe_oracle.c`` is only in how independent work is
grouped: each expert's weights are decoded once to fp64 and applied to all
tokens routed to it with one fp64 matrix product (numpy), instead of one
token at a time, so that batches of thousands of tokens finish in seconds.
Rounding order inside a dot product differs (fp64 either way), so the two
agree to fp64 rounding; ``tests/test_oracle_grouped.py`` pins this module to
the C oracle on small banks of every supported format.
"""
from __future__ import annotations

import numpy as np

from . import AWQ, AWQ_OM, BF16, Bank, Proj, rank

# Nibble j of an AWQ word holds column 8c + _AWQ_COL[j] (include/moe.h, AWQ layout).
_AWQ_COL = (0, 2, 4, 6, 1, 3, 5, 7)


def _bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def proj_matrix(p: Proj, e: int) -> np.ndarray:
    """Dequantised weight matrix [out, in] (fp64, exact) of expert e of projection p."""
    if p.fmt == BF16:
        return _bf16_f64(p.w[e])
    if p.fmt in (AWQ, AWQ_OM):
        I, O = p.in_dim, p.out_dim
        zwords = p.qzeros[e].view(np.uint32)           # [I/32][O/8]
        q = np.empty((I, O), np.int64)
        z = np.empty((I // 32, O), np.int64)
        if p.fmt == AWQ:
            words = p.qweight[e].view(np.uint32)       # [I][O/8]
            for j, col in enumerate(_AWQ_COL):
                q[:, col::8] = (words >> np.uint32(4 * j)) & np.uint32(15)
        else:
            words = p.qweight[e].view(np.uint32)       # [O][I/8]: nibble j = input 8w + j
            for j in range(8):
                q[j::8, :] = ((words >> np.uint32(4 * j)) & np.uint32(15)).T
        for j, col in enumerate(_AWQ_COL):
            z[:, col::8] = (zwords >> np.uint32(4 * j)) & np.uint32(15)
        s = p.scales[e].view(np.float16).astype(np.float64)  # [I/32][O]
        g = np.arange(I) // 32
        w = (q - z[g]).astype(np.float64) * s[g]           # [I][O]
        return np.ascontiguousarray(w.T)
    raise NotImplementedError("grouped evaluation covers bf16 and AWQ banks (both code layouts)")


def _silu(a):
    return a / (1.0 + np.exp(-a))


def expert_outputs(x_bits: np.ndarray, idx: np.ndarray, bank: Bank, pairs=None) -> np.ndarray:
    """Expert outputs [n, H] fp64 of the pairs (t, slot) listed in `pairs`
    (an [n, 2] array; default: every pair of idx in pair order t*kk + slot):
    output of expert idx[t, slot] on token t."""
    idx = np.asarray(idx)
    T, kk = idx.shape
    if pairs is None:
        pairs = np.stack(np.divmod(np.arange(T * kk), kk), axis=1)
    pairs = np.asarray(pairs, np.int64)
    ex = idx[pairs[:, 0], pairs[:, 1]]
    out = np.empty((len(pairs), bank.hidden), np.float64)
    x = np.asarray(x_bits, np.uint16)
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        xe = _bf16_f64(x[pairs[sel, 0]])                    # [m, H]
        wg, wu, wd = (proj_matrix(bank.gate, e), proj_matrix(bank.up, e), proj_matrix(bank.down, e))
        h = _silu(xe @ wg.T) * (xe @ wu.T)                  # [m, F]
        out[sel] = h @ wd.T                                 # [m, H]
    return out


def refill_accumulate(x_bits, logits, k: int, bank: Bank, stat_sum: np.ndarray,
                      stat_count: np.ndarray, valid=None, tokens=None, chunk: int = 256):
    """Adds Refill-RMS statistics of the listed tokens (default: all) into
    stat_sum (fp64 [E]) and stat_count (int64 [E]), by full re-evaluation of
    the routed output (the shared expert cancels in the difference).
    logits are the exact router logits [T, E]."""
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    if valid is not None:
        tokens = tokens[np.asarray(valid)[tokens] != 0]
    if tokens.size == 0:
        return
    K1 = k + 1
    l = logits[tokens].astype(np.float64)
    idx = rank(logits[tokens], K1)                              # [n, k+1]
    # softmax over all E experts, then the listed experts' probabilities
    m = l.max(axis=1, keepdims=True)
    p_all = np.exp(l - m)
    p_all /= p_all.sum(axis=1, keepdims=True)
    p = np.take_along_axis(p_all, idx.astype(np.int64), axis=1)  # [n, k+1]
    xs = np.asarray(x_bits, np.uint16)[tokens]
    n = len(tokens)
    # every listed expert's output, each expert decoded once
    o_all = expert_outputs(xs, idx, bank).reshape(n, K1, bank.hidden)
    dsq = np.empty((n, k), np.float64)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        o = o_all[c0:c1]
        pc = p[c0:c1]
        g = pc[:, :k] / pc[:, :k].sum(axis=1, keepdims=True)          # gates of S
        y = np.einsum("tj,tjh->th", g, o[:, :k])
        # S' = S - {j} + {r}: weights over the k+1 listed experts with slot j removed
        wts = np.repeat(pc[:, None, :], k, axis=1)                   # [n, k, k+1]
        wts[:, np.arange(k), np.arange(k)] = 0.0
        wts /= wts.sum(axis=2, keepdims=True)
        y2 = np.matmul(wts, o)                                        # [n, k, H]
        d = y2 - y[:, None, :]
        dsq[c0:c1] = (d * d).sum(axis=2)
    # token order, as the C oracle adds them
    for t in range(n):
        for j in range(k):
            stat_sum[idx[t, j]] += dsq[t, j]
            stat_count[idx[t, j]] += 1

"""Independent float64 dense brute force of the MoE forward path (test-only).

Every expert is evaluated for every token with whole-matrix numpy/scipy
operations, and the result is masked by the routing: this formulation shares
nothing with the oracle's per-token loop, so a dropped term, a wrong sign or
index, or a transposed operand in either one shows up as a mismatch.

Definitions: [R] = the Pith review of "Cross-Platform Fused MoE Dispatch in
Triton"; "The reading" and "What carries the argument" (score, top-k,
SwiGLU expert FFN, weighted combination), Eq. (1)-(4) named in
"Assumptions & free parameters".
"""
import numpy as np
from scipy.special import expit, softmax


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def topk_lexsort(logits, k):
    """Top-k by a library sort: descending logit, ties to the lower index."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -logits), axis=-1)
    return order[:, :k].astype(np.int32)


def routing_weights_f64(logits, ids, score, renormalize):
    l = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    if score == 0:
        if renormalize:
            return softmax(sel, axis=1)
        return np.take_along_axis(softmax(l, axis=1), ids.astype(np.int64), axis=1)
    s = expit(sel)
    if renormalize:
        s = s / s.sum(axis=1, keepdims=True)
    return s


def dense_moe_f64(x_bits, logits, wgu_bits, wd_bits, k, score, renormalize, weights=None):
    """out[t] = sum_e M[t,e] * (silu(x Wg_e^T) * (x Wu_e^T)) Wd_e^T, where
    M[t,e] is the routing weight of e for t if e is among t's top-k, else 0."""
    x = bf16_bits_to_f64(x_bits)
    wgu = bf16_bits_to_f64(wgu_bits)
    wd = bf16_bits_to_f64(wd_bits)
    T, E = np.asarray(logits).shape
    F = wgu.shape[1] // 2
    ids = topk_lexsort(logits, k)
    w = routing_weights_f64(logits, ids, score, renormalize) if weights is None else weights
    M = np.zeros((T, E))
    np.put_along_axis(M, ids.astype(np.int64), w, axis=1)
    out = np.zeros((T, x.shape[1]))
    for e in range(E):
        G = x @ wgu[e, :F].T
        U = x @ wgu[e, F:].T
        H = G * expit(G) * U
        out += M[:, e:e + 1] * (H @ wd[e].T)
    return out

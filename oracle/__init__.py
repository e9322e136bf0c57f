"""CPU oracle of the single-GPU MoE forward path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp32 accumulation -- fp64
for the router scores -- one token at a time, OpenMP over tokens only).  This module compiles it with gcc
and marshals numpy arrays to it; it holds no arithmetic of its own except the
composition of the steps in their documented order.

bf16 tensors are passed as ``numpy.uint16`` bit patterns.

Steps (named after the page they follow, [R] = the Pith review of
"Cross-Platform Fused MoE Dispatch in Triton: Portable Expert Routing Without
CUDA"):
  router_logits   O0 router scores x.W_r^T   [R] "The reading", Eq. (1)-(4)
  route           O1 top-k + O2 weights      [R] "The reading", Eq. (1)-(4)
  counts_offsets  O3 histogram + scan        [R] "What carries the argument"
  permute         O4 stable reorder          [R] "The reading"; abstract
  block_table     O5 (expert, offset) blocks [R] "What carries the argument"
  block_order     O5b blocks longest first   [R] "Assumptions & free parameters"
  ffn             O6 SwiGLU FFN + combine    [R] "What carries the argument"
  round_bf16      O7 RNE to bf16
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

_lock = threading.Lock()
_lib = None


# ORACLE_SANITIZE=1: build and load liboracle_san.so instead, compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer (the process must preload
# gcc's libasan; oracle/sanitize_check.sh runs the CPU tests that way).
_SANITIZE = os.environ.get("ORACLE_SANITIZE", "") not in ("", "0")
if _SANITIZE:
    _SO = os.path.join(_HERE, "liboracle_san.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (host only, no GPU headers)."""
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(_SRC):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", *(_SAN_FLAGS if _SANITIZE else []), "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.orc_abi_version.restype = I
        lib.orc_max_threads.restype = I
        lib.orc_set_threads.argtypes = [I]
        lib.orc_set_threads.restype = None
        lib.orc_select_topk.argtypes = [P, I, I, I, P]
        lib.orc_weights.argtypes = [P, P, I, I, I, I, I, P]
        lib.orc_counts_offsets.argtypes = [P, I, I, P, P]
        lib.orc_permute.argtypes = [P, I, I, P, P, P]
        lib.orc_block_table.argtypes = [P, P, I, I, P, I, P]
        lib.orc_block_order.argtypes = [P, I, P, I, P]
        lib.orc_var_block_table.argtypes = [P, P, I, I, I, I, I, P, I, P]
        lib.orc_ffn_tokens.argtypes = [P, P, P, P, P, I, I, I, I, I, P, I, P]
        lib.orc_round_bf16.argtypes = [P, P, ctypes.c_long]
        lib.orc_router_logits.argtypes = [P, P, I, I, I, P]
        for f in ("orc_select_topk", "orc_weights", "orc_counts_offsets", "orc_permute",
                  "orc_block_table", "orc_var_block_table", "orc_ffn_tokens", "orc_round_bf16",
                  "orc_router_logits"):
            getattr(lib, f).restype = I
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's later calls (results do not depend on it)."""
    _load().orc_set_threads(int(n))


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    _check(_load().orc_select_topk(_ptr(logits), T, E, k, _ptr(ids)), "select_topk")
    return ids


def weights(logits: np.ndarray, ids: np.ndarray, score: int, renormalize: bool) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, E = logits.shape
    k = ids.shape[1]
    w = np.empty((T, k), dtype=np.float32)
    _check(_load().orc_weights(_ptr(logits), _ptr(ids), T, E, k, int(score), int(bool(renormalize)),
                               _ptr(w)), "weights")
    return w


def route(logits: np.ndarray, k: int, score: int, renormalize: bool):
    """O1 + O2: returns (ids int32 [T,k], w float32 [T,k])."""
    ids = select_topk(logits, k)
    return ids, weights(logits, ids, score, renormalize)


def counts_offsets(ids: np.ndarray, E: int):
    flat = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    _check(_load().orc_counts_offsets(_ptr(flat), flat.size, E, _ptr(counts), _ptr(offsets)),
           "counts_offsets")
    return counts, offsets


def permute(ids: np.ndarray, E: int, offsets: np.ndarray):
    flat = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    perm = np.empty(flat.size, dtype=np.int32)
    inv = np.empty(flat.size, dtype=np.int32)
    _check(_load().orc_permute(_ptr(flat), flat.size, E, _ptr(offsets), _ptr(perm), _ptr(inv)),
           "permute")
    return perm, inv


def block_table(counts: np.ndarray, offsets: np.ndarray, BM: int):
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = counts.size
    max_blocks = int(sum((int(c) + BM - 1) // BM for c in counts)) + 1
    blocks = np.zeros((max_blocks, 2), dtype=np.int32)
    nb = np.zeros(1, dtype=np.int32)
    _check(_load().orc_block_table(_ptr(counts), _ptr(offsets), E, BM, _ptr(blocks), max_blocks,
                                   _ptr(nb)), "block_table")
    return blocks[: int(nb[0])].copy(), int(nb[0])


def block_order(blocks: np.ndarray, offsets: np.ndarray, BM: int):
    """O5b: the blocks longest first (stable by block index)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.int32).reshape(-1, 2)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    nb = blocks.shape[0]
    order = np.zeros(max(nb, 1), dtype=np.int32)
    _check(_load().orc_block_order(_ptr(blocks), nb, _ptr(offsets), BM, _ptr(order)),
           "block_order")
    return order[:nb].copy()


def var_block_table(counts: np.ndarray, offsets: np.ndarray, BM: int, tiles: int, mode: int,
                    round_wgs: int = 256):
    """O5c: the gate/up GEMM's table with a variable block size per expert
    (experts past BM rows in blocks of 2 BM when the table merges).  Returns
    (table [n, 3] of (expert, first row, rows), n), or (None, -1) when the
    rule keeps the fixed table."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = counts.size
    max_blocks = int(sum((int(c) + BM - 1) // BM for c in counts)) + 1
    vb = np.zeros((max_blocks, 3), dtype=np.int32)
    vnb = np.zeros(1, dtype=np.int32)
    _check(_load().orc_var_block_table(_ptr(counts), _ptr(offsets), E, BM, tiles, mode, round_wgs,
                                       _ptr(vb), max_blocks, _ptr(vnb)), "var_block_table")
    n = int(vnb[0])
    return (None, -1) if n < 0 else (vb[:n].copy(), n)


def _expert_ptrs(w, E: int):
    """Accepts one [E, R, C] uint16 array or a list of E arrays (None allowed)."""
    arr = (ctypes.c_void_p * E)()
    keep = []
    for e in range(E):
        we = w[e]
        if we is None:
            arr[e] = None
            continue
        we = np.ascontiguousarray(we, dtype=np.uint16)
        keep.append(we)
        arr[e] = we.ctypes.data
    return arr, keep


def ffn(x: np.ndarray, ids: np.ndarray, w: np.ndarray, w_gate_up, w_down, ffn_dim: int,
        tokens=None) -> np.ndarray:
    """O6: fp32 [ntok, d] = sum_j w[t,j] * expert_j(x_t) for the listed tokens."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, d = x.shape
    k = ids.shape[1]
    E = len(w_gate_up)
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    gu, keep1 = _expert_ptrs(w_gate_up, E)
    dn, keep2 = _expert_ptrs(w_down, E)
    out = np.empty((tokens.size, d), dtype=np.float32)
    _check(_load().orc_ffn_tokens(_ptr(x), _ptr(ids), _ptr(w), gu, dn, T, d, int(ffn_dim), E, k,
                                  _ptr(tokens), tokens.size, _ptr(out)), "ffn")
    del keep1, keep2
    return out


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """O0: fp32 [T, E] router scores x . W_r^T of bf16 bits x [T, d] and
    W_r [E, d] (fp64 sums, one rounding to fp32)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wr = np.ascontiguousarray(w_router, dtype=np.uint16)
    T, d = x.shape
    E, d2 = wr.shape
    if d2 != d:
        raise ValueError("x and W_r disagree on d")
    out = np.empty((T, E), dtype=np.float32)
    _check(_load().orc_router_logits(_ptr(x), _ptr(wr), T, d, E, _ptr(out)), "router_logits")
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _check(_load().orc_round_bf16(_ptr(a), _ptr(out), a.size), "round_bf16")
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (bits << 16)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def forward(x, logits, w_gate_up, w_down, top_k: int, renormalize: bool, score: int,
            ffn_dim: int, BM: int = 16, tokens=None) -> dict:
    """All steps O1..O7 in order.  Returns a dict of every routing artefact,
    ``ref32`` (fp32 [ntok,d]) and ``ref16`` (bf16 bits [ntok,d])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    E = logits.shape[1]
    ids, w = route(logits, top_k, score, renormalize)
    counts, offsets = counts_offsets(ids, E)
    perm, inv = permute(ids, E, offsets)
    blocks, nb = block_table(counts, offsets, BM)
    ref32 = ffn(x, ids, w, w_gate_up, w_down, ffn_dim, tokens)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv,
                blocks=blocks, nb=nb, ref32=ref32, ref16=round_bf16(ref32))

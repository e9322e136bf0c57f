"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before any HIP
call (so these calls never reach a kernel launch).

Every call below is built to fail a host check; none of them passes a set of
arguments that validation would accept, so nothing is ever launched.
"""
import ctypes
import os
import re

import pytest

import expert_dispatch_router_amd as moe
from expert_dispatch_router_amd import _lib
from expert_dispatch_router_amd.synth import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")

OK, NULL, SHAPE, TOPK, ALIGN, WS, UNSUP = 0, -1, -2, -3, -4, -5, -6


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 12
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, n
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "moe.h")).read()
    assert moe.moe_abi_version() == int(re.search(r"#define\s+MOE_ABI_VERSION\s+(\d+)",
                                                  hdr).group(1))


def test_status_strings():
    for s in (OK, NULL, SHAPE, TOPK, ALIGN, WS, UNSUP, -7, 99):
        assert isinstance(moe.status_string(s), str) and moe.status_string(s)


def _ws(T, d, F, E, k, opt=None):
    n = ctypes.c_size_t(0)
    rc = moe.lib().moe_workspace_size_ex(T, d, F, E, k, opt, ctypes.byref(n))
    return rc, n.value


def test_workspace_size_checks():
    assert _ws(-1, 64, 64, 4, 2)[0] == SHAPE
    assert _ws(4, 0, 64, 4, 2)[0] == SHAPE
    assert _ws(4, 64, 64, 0, 1)[0] == SHAPE
    assert _ws(4, 64, 64, 4, 0)[0] == TOPK
    assert _ws(4, 64, 64, 4, 5)[0] == TOPK
    assert _ws(4, 64, 64, 513, 2)[0] == UNSUP
    assert _ws(4, 64, 64, 64, 17)[0] == UNSUP
    assert _ws(4, 96, 64, 4, 2)[0] == ALIGN
    assert _ws(4, 64, 100, 4, 2)[0] == ALIGN
    assert _ws(1 << 20, 64, 64, 8, 2)[0] == UNSUP
    assert _ws(0, 64, 64, 4, 2) == (OK, 0)
    rc, n = _ws(64, 256, 512, 8, 2)
    assert rc == OK and n > 0 and n % 256 == 0
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_workspace_size(4, 64, 64, 4, 2, None) == NULL


def _o(bm=0, split=0, variant=0, rotate=0, routing=0, gather=0, unfused=0, xcd=0, dvar=0,
       fold=0, fuse=0, sched=0):
    return ctypes.byref(_lib.MoeOptions(bm, split, variant, dvar, rotate, routing, gather, unfused,
                                        xcd, fold, fuse, sched, None))


def test_options_checks():
    for bad in (_o(8), _o(0, 9), _o(0, -1), _o(0, 0, 1), _o(32, 0, 2), _o(64, 0, 3), _o(192, 0, 4), _o(0, 0, 0, 5),
                _o(0, 0, -1), _o(0, 0, 0, -1)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    for bm in (16, 32, 64, 128, 192):
        rc, n = _ws(64, 256, 512, 8, 2, _o(bm))
        assert rc == OK and n > 0
        assert _ws(64, 256, 512, 8, 2, _o(bm, 0, 1))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(64, 0, 2))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(192, 0, 2))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(128, 0, 2))[0] == OK
    # the LDS-staged tiles (variant 2 of BM = 128 and 192, option value 3):
    # gate/up at any ffn (a partial last tile), not with K-step-tiled
    # activations; down at d a multiple of 256, not with the folded
    # combination
    assert _ws(64, 256, 512, 8, 2, _o(128, 0, 3))[0] == OK
    assert _ws(64, 256, 384, 8, 2, _o(128, 0, 3))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(192, 0, 3))[0] == OK
    assert _ws(64, 256, 448, 8, 2, _o(192, 0, 3))[0] == OK
    assert _ws(64, 256, 448, 8, 2, _o(192, 0, 3, gather=3))[0] == UNSUP
    # the narrow LDS-staged gate/up tile (variant 3 of BM = 128, option value 4)
    assert _ws(64, 256, 512, 8, 2, _o(128, 0, 4))[0] == OK
    assert _ws(64, 256, 448, 8, 2, _o(128, 0, 4, gather=3))[0] == UNSUP
    assert _ws(64, 256, 512, 8, 2, _o(128, 0, 5))[0] == UNSUP
    for bm in (128, 192):
        assert _ws(64, 256, 512, 8, 2, _o(bm, dvar=3))[0] == OK
        assert _ws(64, 320, 512, 8, 2, _o(bm, dvar=3))[0] == UNSUP
        assert _ws(64, 256, 512, 8, 2, _o(bm, dvar=3, fold=2))[0] == UNSUP
        # the wide LDS-staged down tile (variant 3, option value 4): any d (a
        # partial last tile), not with the folded combination
        assert _ws(64, 256, 512, 8, 2, _o(bm, dvar=4))[0] == OK
        assert _ws(64, 320, 512, 8, 2, _o(bm, dvar=4))[0] == OK
        assert _ws(64, 256, 512, 8, 2, _o(bm, dvar=4, fold=2))[0] == UNSUP
    assert _ws(64, 256, 512, 8, 2, _o(64, dvar=4))[0] == UNSUP
    # its 7-wave form (variant 4, option value 5): BM = 128 only
    assert _ws(64, 320, 512, 8, 2, _o(128, dvar=5))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(128, dvar=5, fold=2))[0] == UNSUP
    assert _ws(64, 256, 512, 8, 2, _o(192, dvar=5))[0] == UNSUP
    assert _ws(64, 256, 512, 8, 2, _o(128, dvar=6))[0] == UNSUP
    # automatic: the 7-wave tile where its whole tiles fill the rounds better
    assert moe.moe_plan_ex(512, 3584, 2560, 64, 8)["down_variant"] == 4     # Qwen2 T=512
    assert moe.moe_plan_ex(512, 7168, 2048, 256, 8)["down_variant"] == 3    # DeepSeek-V3 T=512
    for r in (1, 2, 3):
        assert _ws(64, 256, 512, 8, 2, _o(0, 0, 0, r))[0] == OK


def test_routing_and_gather_options():
    for bad in (_o(routing=4), _o(routing=-1), _o(gather=4), _o(gather=-1)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    # two launches: the histogram kernel keeps every 64-row group's counts in LDS
    assert _ws(4096, 256, 512, 256, 1, _o(routing=3))[0] == OK          # 64 groups x 256
    assert _ws(4097, 256, 512, 256, 1, _o(routing=3))[0] == UNSUP       # 65 groups x 256
    assert _ws(512, 256, 512, 64, 4, _o(routing=3))[0] == OK
    for r in (0, 1, 2, 3):
        for g in (0, 1, 2, 3):
            assert _ws(64, 256, 512, 8, 2, _o(routing=r, gather=g))[0] == OK
    # the one-workgroup routing kernel: one token per thread, at most 64 experts
    assert _ws(1024, 256, 512, 32, 16, _o(routing=1))[0] == OK
    assert _ws(1024, 256, 512, 64, 16, _o(routing=1))[0] == OK
    assert _ws(1025, 256, 512, 8, 2, _o(routing=1))[0] == UNSUP
    assert _ws(512, 256, 512, 65, 2, _o(routing=1))[0] == UNSUP
    assert _ws(1025, 256, 512, 8, 2, _o(routing=2))[0] == OK
    r = ctypes.c_size_t(0)
    assert moe.lib().moe_route_workspace_size(1025, 8, 2, _o(routing=1), ctypes.byref(r)) == UNSUP
    # gather inside the GEMM addresses x with 32-bit byte offsets
    assert _ws(65536, 16384, 512, 8, 1, _o(gather=1))[0] == UNSUP
    assert _ws(65536, 16384, 512, 8, 1, _o(gather=2))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(192, dvar=2))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(64, dvar=1))[0] == OK
    # the unfused SwiGLU ablation keeps gate and up products: 2 * A*ffn*2 bytes more
    for x in (0, 1, 2, 3):
        assert _ws(64, 256, 512, 8, 2, _o(xcd=x))[0] == OK
    for bad in (_o(unfused=2), _o(unfused=-1), _o(xcd=4), _o(xcd=-1), _o(dvar=1), _o(dvar=-1),
                _o(64, dvar=2), _o(192, dvar=5)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    u0 = moe.moe_workspace_size(512, 4096, 14336, 8, 2)
    u1 = moe.moe_workspace_size(512, 4096, 14336, 8, 2, unfused_swiglu=1)
    assert u1 - u0 == 2 * 1024 * 14336 * 2
    # no x_perm buffer when the GEMM gathers: the workspace shrinks by A*d*2 (256-aligned)
    g1 = moe.moe_workspace_size(512, 4096, 14336, 8, 2, gather_mode=1)
    g2 = moe.moe_workspace_size(512, 4096, 14336, 8, 2, gather_mode=2)
    assert g2 - g1 == 1024 * 4096 * 2
    assert moe.moe_workspace_size(512, 4096, 14336, 8, 2) == g1


def test_fold_combine_option():
    for bad in (_o(fold=3), _o(fold=-1)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    for f in (0, 1, 2):
        assert _ws(64, 256, 512, 8, 2, _o(fold=f))[0] == OK
    # folded: one int32 arrival counter per (token, down-GEMM column tile);
    # Mixtral T=512 at BM=192 has 256-column down tiles -> 512 * 16 counters
    f1 = moe.moe_workspace_size(512, 4096, 14336, 8, 2, fold_combine=1)
    f2 = moe.moe_workspace_size(512, 4096, 14336, 8, 2, fold_combine=2)
    assert f2 - f1 == 512 * 16 * 4
    # the 16-row tiles of the down GEMM are 512 columns wide
    g1 = moe.moe_workspace_size(64, 1024, 512, 8, 2, block_rows=16, fold_combine=1)
    g2 = moe.moe_workspace_size(64, 1024, 512, 8, 2, block_rows=16, fold_combine=2)
    assert g2 - g1 == 64 * 2 * 4


def test_fuse_down_option():
    for bad in (_o(fuse=3), _o(fuse=-1)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    # compiled for BM 64 (variant 1), 128 (variant 1, the automatic choice
    # with fusion), 192 (variant 0); option values are variant + 1
    for bm, v in ((128, 0), (128, 2), (64, 2), (192, 1)):
        assert _ws(64, 256, 512, 8, 2, _o(bm, variant=v, fuse=2))[0] == OK, (bm, v)
    for bm, v in ((16, 0), (32, 0), (64, 1), (128, 1), (192, 2)):
        assert _ws(64, 256, 512, 8, 2, _o(bm, variant=v, fuse=2))[0] == UNSUP, (bm, v)
    assert _ws(64, 256, 512, 8, 2, _o(128, fuse=2, unfused=1))[0] == UNSUP
    # automatic: only launches below one round with small partials fuse
    assert moe.moe_plan(64, 256, 512, 8, 2, with_fusion=True) == (128, 8, True)
    assert moe.moe_plan(64, 256, 512, 8, 2, fuse_down=1, with_fusion=True)[2] is False
    assert moe.moe_plan(512, 4096, 14336, 8, 2, with_fusion=True)[2] is False
    assert moe.moe_plan(512, 7168, 2048, 256, 8, with_fusion=True)[2] is False
    # fused: no h buffer [A, ffn] bf16; one fp32 part [A, d] per 64-column tile
    a = moe.moe_workspace_size(64, 256, 512, 8, 2, block_rows=128, tile_variant=2, fuse_down=1,
                               split_k=1)
    b = moe.moe_workspace_size(64, 256, 512, 8, 2, block_rows=128, tile_variant=2, fuse_down=2)
    assert b - a == 8 * 128 * 256 * 4 - 128 * 256 * 4 - 128 * 512 * 2


def test_plan_choices_for_the_workloads():
    # near-uniform routing: one block per expert in the common case; never
    # fewer than 128 rows per block (robust to skewed routing)
    assert moe.moe_plan(512, 4096, 14336, 8, 2)[0] == 192
    assert moe.moe_plan(512, 7168, 2048, 256, 8)[0] == 128
    assert moe.moe_plan(64, 256, 512, 8, 2)[0] == 128
    assert moe.moe_plan(4096, 7168, 2048, 256, 8)[0] == 192
    for name, c in CONFIGS.items():
        bm, split = moe.moe_plan(c.T, c.d, c.ffn, c.E, c.top_k)
        assert bm in (16, 32, 64, 128, 192) and 1 <= split <= 8, name
        assert moe.moe_plan(c.T, c.d, c.ffn, c.E, c.top_k, block_rows=16, split_k=3) == (16, 3)


def test_workspace_grows_with_split_and_small_blocks():
    a = moe.moe_workspace_size(512, 4096, 14336, 8, 2, block_rows=192, split_k=1)
    b = moe.moe_workspace_size(512, 4096, 14336, 8, 2, block_rows=192, split_k=4)
    c = moe.moe_workspace_size(512, 4096, 14336, 8, 2, block_rows=16, split_k=4)
    assert a < b < c
    # the fp32 split partials dominate: 3 more parts of [A, d] fp32
    assert b - a == 3 * 1024 * 4096 * 4


FAKE = 1 << 20  # a 256-aligned non-null address that is never dereferenced


def _fwd(**kw):
    a = dict(x=FAKE, logits=FAKE, wgu=FAKE, wd=FAKE, k=2, renorm=1, out=FAKE, T=4, d=64, F=64, E=4,
             score=0, opt=None, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return moe.lib().moe_forward_ex(a["x"], a["logits"], a["wgu"], a["wd"], a["k"], a["renorm"],
                                    a["out"], a["T"], a["d"], a["F"], a["E"], a["score"], a["opt"],
                                    a["ws"], a["wsb"], a["stream"])


def test_forward_rejects_before_any_launch():
    # wsb=0 makes every otherwise-valid combination fail with MOE_ERR_WORKSPACE
    assert _fwd() == WS
    for name in ("x", "logits", "wgu", "wd", "out", "ws"):
        assert _fwd(**{name: None}) == NULL, name
    for name in ("x", "logits", "wgu", "wd", "out"):
        assert _fwd(**{name: FAKE + 8}) == ALIGN, name
    assert _fwd(ws=FAKE + 16) == ALIGN
    assert _fwd(T=-1) == SHAPE
    assert _fwd(k=0) == TOPK
    assert _fwd(k=5) == TOPK
    assert _fwd(d=100) == ALIGN
    assert _fwd(F=32) == ALIGN
    assert _fwd(score=2) == UNSUP
    assert _fwd(E=600, k=2) == UNSUP
    assert _fwd(opt=_o(48)) == UNSUP
    rc, need = _ws(4, 64, 64, 4, 2)
    assert _fwd(wsb=need - 1) == WS
    # T = 0 is a no-op that succeeds even with NULL buffers
    assert _fwd(T=0, x=None, logits=None, wgu=None, wd=None, out=None, ws=None) == OK


def test_plain_forward_entry_validates_the_same_way():
    L = moe.lib()
    assert L.moe_forward(FAKE, FAKE, FAKE, FAKE, 2, 1, FAKE, 4, 64, 64, 4, 0, FAKE, 0, None) == WS
    assert L.moe_forward(None, FAKE, FAKE, FAKE, 2, 1, FAKE, 4, 64, 64, 4, 0, FAKE, 0, None) == NULL


def _route(**kw):
    a = dict(logits=FAKE, T=4, E=4, k=2, renorm=1, score=0, opt=None, x=None, d=0, xp=None,
             ws=FAKE, wsb=0)
    a.update(kw)
    bm = ctypes.c_int(-1)
    rc = moe.lib().moe_route(a["logits"], a["T"], a["E"], a["k"], a["renorm"], a["score"], a["opt"],
                             FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["x"], a["d"],
                             a["xp"],
                             ctypes.byref(bm), a["ws"], a["wsb"], None)
    return rc, bm.value


def test_route_rejects_before_any_launch():
    assert _route()[0] == WS
    assert _route(logits=None)[0] == NULL
    assert _route(ws=None)[0] == NULL
    assert _route(logits=FAKE + 4)[0] == ALIGN
    assert _route(k=7)[0] == TOPK
    assert _route(score=5)[0] == UNSUP
    assert _route(x=FAKE, xp=FAKE, d=96)[0] == ALIGN
    assert _route(x=FAKE, xp=FAKE, d=0)[0] == SHAPE
    assert _route(x=FAKE + 8, xp=FAKE, d=64)[0] == ALIGN
    rc, bm = _route(T=0, logits=None, ws=None)
    assert rc == OK and bm in (16, 32, 64, 128, 192)
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_route_workspace_size(4, 4, 2, None, ctypes.byref(n)) == OK and n.value > 0


def _rl(**kw):
    a = dict(x=FAKE, w=FAKE, out=FAKE, T=4, d=64, E=4, ws=None, wsb=0)
    a.update(kw)
    return moe.lib().moe_router_logits(a["x"], a["w"], a["out"], a["T"], a["d"], a["E"], a["ws"],
                                       a["wsb"], None)


def test_router_logits_rejects_before_any_launch():
    # every call below fails a host check (a valid one would launch)
    assert _rl(T=-1) == SHAPE
    assert _rl(E=0) == SHAPE
    assert _rl(d=0) == SHAPE
    assert _rl(E=513) == UNSUP
    assert _rl(T=(1 << 20) + 1) == UNSUP
    assert _rl(d=100) == ALIGN
    assert _rl(d=1 << 25) == UNSUP
    for name in ("x", "w", "out"):
        assert _rl(**{name: None}) == NULL, name
        assert _rl(**{name: FAKE + 4}) == ALIGN, name
    assert _rl(T=0, x=None, w=None, out=None) == OK
    # sizes that split the reduction need the workspace for partial sums
    need = moe.moe_router_workspace_size(512, 4096, 8)
    assert need >= 2 * 512 * 8 * 4 and need % 256 == 0
    assert _rl(T=512, d=4096, E=8) == NULL
    assert _rl(T=512, d=4096, E=8, ws=FAKE, wsb=need - 1) == WS
    assert _rl(T=512, d=4096, E=8, ws=FAKE + 16, wsb=need) == ALIGN
    assert moe.moe_router_workspace_size(8192, 64, 512) == 0  # one part: no workspace
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_router_workspace_size(4, 100, 4, ctypes.byref(n)) == ALIGN


def _fr(**kw):
    a = dict(x=FAKE, wr=FAKE, wgu=FAKE, wd=FAKE, k=2, renorm=1, out=FAKE, lo=None, T=4, d=64, F=64,
             E=4, score=0, opt=None, ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return moe.lib().moe_forward_router(a["x"], a["wr"], a["wgu"], a["wd"], a["k"], a["renorm"],
                                        a["out"], a["lo"], a["T"], a["d"], a["F"], a["E"],
                                        a["score"], a["opt"], a["ws"], a["wsb"], a["stream"])


def test_forward_router_rejects_before_any_launch():
    assert _fr() == WS  # wsb = 0
    for name in ("x", "wr", "wgu", "wd", "out", "ws"):
        assert _fr(**{name: None}) == NULL, name
    assert _fr(lo=FAKE + 4) == ALIGN
    assert _fr(wr=FAKE + 8) == ALIGN
    assert _fr(k=0) == TOPK
    assert _fr(d=96) == ALIGN
    assert _fr(E=513) == UNSUP
    assert _fr(score=2, wsb=1 << 30) == UNSUP
    assert _fr(T=0, x=None, wr=None) == OK


def test_timer_argument_checks():
    L = moe.lib()
    assert L.moe_timer_create(None) == NULL
    assert L.moe_timer_destroy(None) == NULL
    assert L.moe_timer_elapsed_ms(None, None, None) == NULL
    assert L.moe_timer_record(None, None) == NULL


def test_product_path_never_imports_the_oracle():
    pkg = os.path.dirname(moe.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "moe_oracle" not in text and "liboracle" not in text, f


def test_binding_rejects_wrong_output_shapes_before_any_call():
    """The binding raises before it reaches the library when a caller's
    output buffer does not have the shape the kernels write ([T, d] for the
    forward pass, [T, E] for the scores) or when moe_route's x does not have
    one row per token.  Host tensors suffice: the shape checks come first."""
    import torch

    T, d, F, E, k = 8, 64, 64, 4, 2
    x = torch.zeros(T, d, dtype=torch.bfloat16)
    lg = torch.zeros(T, E)
    wgu = torch.zeros(E, 2 * F, d, dtype=torch.bfloat16)
    wd = torch.zeros(E, d, F, dtype=torch.bfloat16)
    wr = torch.zeros(E, d, dtype=torch.bfloat16)
    for bad in (torch.empty(T - 1, d, dtype=torch.bfloat16), torch.empty(T, d // 2, dtype=torch.bfloat16),
                torch.empty(T * d, dtype=torch.bfloat16)):
        with pytest.raises(ValueError, match="out must be"):
            moe.moe_forward(x, lg, wgu, wd, k, True, out=bad)
        with pytest.raises(ValueError, match="out must be"):
            moe.moe_forward_router(x, wr, wgu, wd, k, True, out=bad)
    with pytest.raises(ValueError, match="logits_out must be"):
        moe.moe_forward_router(x, wr, wgu, wd, k, True, logits_out=torch.empty(T, E + 1))
    with pytest.raises(ValueError, match="out must be"):
        moe.moe_router_logits(x, wr, out=torch.empty(T - 1, E))
    with pytest.raises(ValueError, match="one row per token"):
        moe.moe_route(lg, k, True, x=torch.zeros(T + 1, d, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="x must be"):
        moe.moe_route(lg, k, True, x=torch.zeros(T * d, dtype=torch.bfloat16))


def test_binding_rejects_tensors_on_different_devices():
    """Tensors on two devices are refused before any launch (checked by
    device identity, so a host tensor beside a meta tensor is enough)."""
    import torch

    T, d, F, E, k = 8, 64, 64, 4, 2
    x = torch.zeros(T, d, dtype=torch.bfloat16)
    lg = torch.zeros(T, E)
    wgu = torch.zeros(E, 2 * F, d, dtype=torch.bfloat16, device="meta")
    wd = torch.zeros(E, d, F, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="different devices"):
        moe.moe_forward(x, lg, wgu, wd, k, True)


def test_plan_ex_reports_the_launches():
    """moe_plan_ex (host only) agrees with moe_plan and counts the kernels
    of each path: one-workgroup routing + gate/up + down + combination at
    Mixtral T=512 (4 launches), the down projection fused at tiny (3), the
    unfused ablation's three kernels, a separate gather, the folded
    combination."""
    mix = CONFIGS["mixtral_512"]
    info = moe.moe_plan_ex(mix.T, mix.d, mix.ffn, mix.E, mix.top_k)
    bm, split, fd = moe.moe_plan(mix.T, mix.d, mix.ffn, mix.E, mix.top_k, with_fusion=True)
    assert (info["block_rows"], info["split_k"], info["fused_down"]) == (bm, split, int(fd))
    assert info["routing_launches"] == 1 and info["launches"] == 4
    tiny = CONFIGS["tiny"]
    t = moe.moe_plan_ex(tiny.T, tiny.d, tiny.ffn, tiny.E, tiny.top_k)
    assert t["fused_down"] == 1 and t["down_variant"] == -1 and t["launches"] == 3
    dsv = CONFIGS["dsv3_4096"]
    dv = moe.moe_plan_ex(dsv.T, dsv.d, dsv.ffn, dsv.E, dsv.top_k)
    assert dv["routing_launches"] == 3 and dv["xcd_grouped"] == 1 and dv["launches"] == 6
    u = moe.moe_plan_ex(mix.T, mix.d, mix.ffn, mix.E, mix.top_k, unfused_swiglu=1)
    assert u["unfused_swiglu"] == 1 and u["launches"] == 6
    g = moe.moe_plan_ex(mix.T, mix.d, mix.ffn, mix.E, mix.top_k, gather_mode=2, routing_kernels=2)
    assert g["gather_launch"] == 1 and g["routing_launches"] == 3 and g["launches"] == 7
    f = moe.moe_plan_ex(mix.T, mix.d, mix.ffn, mix.E, mix.top_k, block_rows=192, down_variant=1,
                        fold_combine=2)
    assert f["fold_combine"] == 1 and f["launches"] == 3
    assert moe.moe_plan_ex(0, 64, 64, 4, 2)["launches"] == 0
    assert moe.lib().moe_plan_ex(4, 64, 64, 4, 2, None, None) == NULL
    with pytest.raises(moe.MoeError):
        moe.moe_plan_ex(4, 96, 64, 4, 2)


def test_forward_static_host_checks():
    """moe_forward_static rejects, before any HIP call, problems whose
    workspace exceeds the static array (MOE_ERR_STATIC_LIMIT) and the same
    bad arguments as moe_forward; the binding's constant is the header's."""
    hdr = open(HEADER).read()
    want = int(re.search(r"#define\s+MOE_STATIC_WORKSPACE_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)",
                         hdr).group(1))
    shift = int(re.search(r"#define\s+MOE_STATIC_WORKSPACE_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)",
                          hdr).group(2))
    assert _lib.MOE_STATIC_WORKSPACE_BYTES == want << shift
    L = moe.lib()
    P = 4096  # aligned stand-ins: every call below fails a host check first
    big = CONFIGS["dsv3_4096"]
    assert moe.moe_workspace_size(big.T, big.d, big.ffn, big.E, big.top_k) > \
        _lib.MOE_STATIC_WORKSPACE_BYTES
    assert L.moe_forward_static(P, P, P, P, big.top_k, 1, P, big.T, big.d, big.ffn, big.E, 1,
                                None) == -8
    assert "static" in moe.status_string(-8)
    mix = CONFIGS["mixtral_512"]
    assert moe.moe_workspace_size(mix.T, mix.d, mix.ffn, mix.E, mix.top_k) <= \
        _lib.MOE_STATIC_WORKSPACE_BYTES
    dsv = CONFIGS["dsv3_512"]
    assert moe.moe_workspace_size(dsv.T, dsv.d, dsv.ffn, dsv.E, dsv.top_k) <= \
        _lib.MOE_STATIC_WORKSPACE_BYTES
    assert L.moe_forward_static(None, P, P, P, 2, 1, P, 64, 256, 512, 8, 0, None) == NULL
    assert L.moe_forward_static(P, P, P, P, 2, 1, None, 64, 256, 512, 8, 0, None) == NULL
    assert L.moe_forward_static(P + 8, P, P, P, 2, 1, P, 64, 256, 512, 8, 0, None) == ALIGN
    assert L.moe_forward_static(P, P, P, P, 9, 1, P, 64, 256, 512, 8, 0, None) == TOPK
    assert L.moe_forward_static(P, P, P, P, 2, 1, P, 64, 96, 512, 8, 0, None) == ALIGN
    assert L.moe_forward_static(P, P, P, P, 2, 1, P, 64, 256, 512, 8, 7, None) == UNSUP
    assert L.moe_forward_static(None, None, None, None, 2, 1, None, 0, 256, 512, 8, 0, None) == OK
    import torch
    with pytest.raises(ValueError, match="out is required"):
        moe.moe_forward_static(torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(4, 4),
                               torch.zeros(4, 128, 64, dtype=torch.bfloat16),
                               torch.zeros(4, 64, 64, dtype=torch.bfloat16), 2, True, None)


def test_plan_ex_split_on_device():
    """An automatic split above one is an upper bound the kernels refine on
    the device; a forced split, a single part, the folded combination and
    the fused down projection are used as planned."""
    sk = CONFIGS["skewed_512"]
    info = moe.moe_plan_ex(sk.T, sk.d, sk.ffn, sk.E, sk.top_k)
    assert info["split_k"] == 2 and info["split_on_device"] == 1
    assert moe.moe_plan_ex(sk.T, sk.d, sk.ffn, sk.E, sk.top_k, split_k=2)["split_on_device"] == 0
    q = CONFIGS["qwen2_512"]
    assert moe.moe_plan_ex(q.T, q.d, q.ffn, q.E, q.top_k)["split_on_device"] == 0  # one part
    mix = CONFIGS["mixtral_512"]
    assert moe.moe_plan_ex(mix.T, mix.d, mix.ffn, mix.E, mix.top_k)["split_on_device"] == 1
    assert moe.moe_plan_ex(mix.T, mix.d, mix.ffn, mix.E, mix.top_k, block_rows=192,
                           down_variant=1, fold_combine=2)["split_on_device"] == 0
    tiny = CONFIGS["tiny"]
    assert moe.moe_plan_ex(tiny.T, tiny.d, tiny.ffn, tiny.E, tiny.top_k)["split_on_device"] == 0


def test_stream_k_schedule_options():
    """schedule = 2 (stream-K gate/up GEMM): runs the narrow 128-row LDS tile
    (automatic block rows become 128), adds 2 x 256 partial slots of 128 KiB
    and one counter per (block, column tile) unit to the workspace, and is
    refused where that tile cannot run."""
    sk = CONFIGS["skewed_128"]
    args = (sk.T, sk.d, sk.ffn, sk.E, sk.top_k)
    info = moe.moe_plan_ex(*args, schedule=2)
    assert info["stream_k"] == 1 and info["block_rows"] == 128 and info["gate_up_variant"] == 3
    assert moe.moe_plan_ex(*args, schedule=1)["stream_k"] == 0
    assert moe.moe_plan_ex(*args, schedule=2, block_rows=128, tile_variant=4)["stream_k"] == 1
    plain = moe.moe_workspace_size(*args, block_rows=128, tile_variant=4, schedule=1)
    streamed = moe.moe_workspace_size(*args, schedule=2)
    units = (-(-sk.T * sk.top_k // 128) + min(sk.E, sk.T * sk.top_k)) * (sk.ffn // 128)
    assert streamed - plain >= 2 * 256 * 128 * 1024 + 4 * units
    assert streamed - plain <= 2 * 256 * 128 * 1024 + 4 * units + 512
    for bad in (_o(0, sched=4), _o(0, sched=-1), _o(192, sched=2), _o(128, 0, 1, sched=2),
                _o(128, 0, 3, sched=2), _o(0, unfused=1, sched=2), _o(0, gather=3, sched=2),
                _o(0, fuse=2, sched=2)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    assert _ws(64, 256, 512, 8, 2, _o(0, sched=2))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(128, 0, 4, sched=2))[0] == OK


def test_variable_rows_schedule_options():
    """schedule = 3 (the gate/up GEMM over the variable-size block table,
    merged always) and its automatic form (merged on the device when one
    round needs it): the narrow 128-row tile, 12 bytes per block more
    workspace, refused where the tile or the table cannot run."""
    sk = CONFIGS["skewed_512"]
    args = (sk.T, sk.d, sk.ffn, sk.E, sk.top_k)
    info = moe.moe_plan_ex(*args, schedule=3)
    assert info["variable_rows"] == 2 and info["block_rows"] == 128
    assert info["gate_up_variant"] == 3 and info["fused_down"] == 0 and info["stream_k"] == 0
    assert moe.moe_plan_ex(*args)["variable_rows"] == 1          # automatic
    assert 0 <= info["var_table_offset"] < info["var_count_offset"]
    assert info["var_count_offset"] + 4 <= moe.moe_workspace_size(*args, schedule=3)
    assert moe.moe_plan_ex(*args, schedule=1)["var_table_offset"] == -1
    assert moe.moe_plan_ex(*args, schedule=1)["variable_rows"] == 0
    assert moe.moe_plan_ex(*args, schedule=2)["variable_rows"] == 0
    nb_max = -(-sk.T * sk.top_k // 128) + min(sk.E, sk.T * sk.top_k)
    fixed = moe.moe_workspace_size(*args, schedule=1)
    var = moe.moe_workspace_size(*args, schedule=3)
    assert 12 * nb_max <= var - fixed <= 12 * nb_max + 512
    # where the automatic plan takes another tile or order, or no routing can
    # make the table merge (Qwen2 T=512: even 256-row blocks holding every row
    # need 16 x 20 > 256 workgroups), the table is not built
    for name in ("mixtral_512", "dsv3_512", "qwen2_512"):
        c = CONFIGS[name]
        assert moe.moe_plan_ex(c.T, c.d, c.ffn, c.E, c.top_k)["variable_rows"] == 0
    for bad in (_o(192, sched=3), _o(128, 0, 1, sched=3), _o(128, 0, 3, sched=3),
                _o(0, unfused=1, sched=3), _o(0, gather=3, sched=3), _o(0, fuse=2, sched=3),
                _o(0, xcd=2, sched=3), _o(0, xcd=3, sched=3)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    assert _ws(64, 256, 512, 8, 2, _o(0, sched=3))[0] == OK
    assert _ws(64, 256, 512, 8, 2, _o(128, 0, 4, sched=3))[0] == OK


def test_256_row_block_options():
    """block_rows = 256 (asked for only): the narrow gate/up tile and the
    256-column down tile, so d must be a multiple of 256; refused with the
    other tiles, the unfused ablation, gather mode 3, the folded combination
    and the fused down projection."""
    info = moe.moe_plan_ex(512, 2048, 1408, 64, 4, block_rows=256)
    assert info["block_rows"] == 256 and info["gate_up_variant"] == 3 and info["down_variant"] == 2
    assert _ws(64, 256, 512, 8, 2, _o(256))[0] == OK
    for bad in (_o(256, 0, 1), _o(256, 0, 3), _o(256, dvar=1), _o(256, dvar=4),
                _o(256, unfused=1), _o(256, gather=3), _o(256, fold=2), _o(256, fuse=2)):
        assert _ws(64, 256, 512, 8, 2, bad)[0] == UNSUP
    assert _ws(64, 128, 512, 8, 2, _o(256))[0] == UNSUP   # d = 128

"""The C-ABI library without a GPU: it loads, it exports every entry point the
header declares, and every argument check returns its status before any
HIP call (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from mxfp4_routed_expert_top_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = (ops.MOE_OK, ops.MOE_ERR_INVALID_ARGUMENT,
                                      ops.MOE_ERR_UNSUPPORTED, ops.MOE_ERR_WORKSPACE_TOO_SMALL)
FAKE = ctypes.c_void_p(0x100000)        # never dereferenced: every call below fails validation
MIS = ctypes.c_void_p(0x100004)          # not 16-byte aligned
FAKE2 = ctypes.c_void_p(0x200000)       # a second, distinct fake buffer


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = ops.lib()
    names = declared_functions()
    assert len(names) == 29
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ops.EXPORTS)


def test_debug_build_exports_the_same_symbols():
    # the MOE_DEBUG build (built beside the release one) has the same interface
    dbg = ctypes.CDLL(ops.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(dbg, n), n


def test_release_build_debug_flags_are_zero():
    # release builds compile the checks away and answer without touching a device
    assert ops.lib().moe_debug_flags(1) == 0 and ops.debug_flags() == 0


def test_status_strings():
    assert ops.status_string(0) == "MOE_OK"
    assert ops.status_string(4) == "MOE_ERR_DEVICE"
    assert ops.status_string(99) == "MOE_ERR_UNKNOWN"


def test_route_topk_argument_errors():
    f = ops.lib().moe_route_topk
    assert f(None, None, 4, 8, 2, 0, 1, FAKE, FAKE, None) == INVALID        # null logits
    assert f(FAKE, None, 4, 8, 2, 1, 1, FAKE, FAKE, None) == INVALID        # shared without gate
    assert f(FAKE, None, -1, 8, 2, 0, 1, FAKE, FAKE, None) == INVALID       # T < 0
    assert f(FAKE, None, 4, 8, 0, 0, 1, FAKE, FAKE, None) == INVALID        # K < 1
    assert f(FAKE, None, 4, 8, 9, 0, 1, FAKE, FAKE, None) == INVALID        # K > E
    assert f(FAKE, None, 4, 8, 2, 2, 1, FAKE, FAKE, None) == INVALID        # shared flag
    assert f(FAKE, None, 4, 8, 2, 0, 3, FAKE, FAKE, None) == INVALID        # renormalize flag
    assert f(FAKE, None, 4, 8, 2, 0, 1, None, FAKE, None) == INVALID        # null output
    assert f(FAKE, None, 4, 2048, 2, 0, 1, FAKE, FAKE, None) == UNSUPPORTED  # E > 1024
    assert f(FAKE, FAKE, 4, 64, 32, 1, 1, FAKE, FAKE, None) == UNSUPPORTED   # K' > 32
    assert f(None, None, 0, 8, 2, 0, 1, None, None, None) == OK             # T = 0: nothing to do


def test_route_topk_gemm_argument_errors():
    f = ops.lib().moe_route_topk_gemm
    ws = ops.route_gemm_workspace_size(64, 4096, 512, 1)
    assert ws >= 64 * 513 * 4 and ops.route_gemm_workspace_size(0, 4096, 512, 1) == 0
    assert ops.route_gemm_workspace_size(64, 4000, 512, 1) == 0
    def call(**kw):
        a = dict(x=FAKE, w=FAKE, T=64, H=4096, E=512, K=10, s=1, r=1, ids=FAKE, wt=FAKE, lo=None,
                 ws=FAKE, wsb=ws)
        a.update(kw)
        return f(a["x"], a["w"], a["T"], a["H"], a["E"], a["K"], a["s"], a["r"], a["ids"], a["wt"],
                 a["lo"], a["ws"], a["wsb"], None)
    assert call(x=None) == INVALID
    assert call(w=None) == INVALID
    assert call(ids=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(x=MIS) == INVALID
    assert call(K=0) == INVALID
    assert call(K=513) == INVALID
    assert call(s=2) == INVALID
    assert call(r=2) == INVALID
    assert call(T=-1) == INVALID
    assert call(H=4000) == UNSUPPORTED
    assert call(E=2048, K=4) == UNSUPPORTED
    assert call(K=32) == UNSUPPORTED                     # K' = 33
    assert call(T=1 << 20) == UNSUPPORTED                # x beyond 2^31 bytes
    assert call(wsb=ws - 1) == WS_SMALL
    assert call(T=0, x=None, w=None, ids=None, wt=None, ws=None) == OK


def test_align_sort_argument_errors():
    f = ops.lib().moe_align_sort
    ws = ops.align_workspace_size(10, 3, 7)
    assert ws > 0
    args = lambda **kw: [kw.get("ids", FAKE), kw.get("T", 10), kw.get("Kp", 3), kw.get("Ep", 7),
                         kw.get("tm", 32), kw.get("cnt", FAKE), kw.get("off", FAKE),
                         kw.get("srt", FAKE), None, None, kw.get("nt", FAKE), kw.get("ws", FAKE),
                         kw.get("wsb", ws), None]
    assert f(*args(ids=None)) == INVALID
    assert f(*args(T=-1)) == INVALID
    assert f(*args(Kp=0)) == INVALID
    assert f(*args(Ep=0)) == INVALID
    assert f(*args(tm=0)) == INVALID
    assert f(*args(cnt=None)) == INVALID
    assert f(*args(nt=None)) == INVALID
    assert f(*args(Ep=4096)) == UNSUPPORTED
    assert f(*args(wsb=ws - 1)) == WS_SMALL
    assert f(*args(ws=None)) == INVALID


def test_route_align_argument_errors():
    f = ops.lib().moe_route_align
    ws = ops.align_workspace_size(10, 3, 9)
    def call(**kw):
        a = dict(lg=FAKE, g=FAKE, T=10, E=8, K=2, s=1, r=1, tm=32, ids=FAKE, wt=FAKE, cnt=FAKE,
                 off=FAKE, srt=FAKE, inv=None, tiles=None, nt=FAKE, ws=FAKE, wsb=ws)
        a.update(kw)
        return f(a["lg"], a["g"], a["T"], a["E"], a["K"], a["s"], a["r"], a["tm"], a["ids"],
                 a["wt"], a["cnt"], a["off"], a["srt"], a["inv"], a["tiles"], a["nt"], a["ws"],
                 a["wsb"], None)
    assert call(lg=None) == INVALID
    assert call(g=None) == INVALID                       # shared without gate
    assert call(T=-1) == INVALID
    assert call(K=0) == INVALID
    assert call(K=9) == INVALID                          # K > E
    assert call(r=2) == INVALID
    assert call(tm=0) == INVALID
    assert call(ids=None) == INVALID
    assert call(wt=None) == INVALID
    assert call(cnt=None) == INVALID
    assert call(off=None) == INVALID
    assert call(srt=None) == INVALID
    assert call(nt=None) == INVALID
    assert call(ws=None) == INVALID
    assert call(E=2048, K=4) == UNSUPPORTED              # E > 1024
    assert call(E=64, K=32) == UNSUPPORTED               # K' = 33
    assert call(wsb=ws - 1) == WS_SMALL


def test_residual_rmsnorm_argument_errors():
    f = ops.lib().moe_residual_rmsnorm
    two = (ctypes.c_void_p * 2)(FAKE, FAKE)
    def call(**kw):
        a = dict(p=two, G=2, r=FAKE, gm=FAKE, eps=1e-6, T=4, H=4096, ro=FAKE, o=FAKE)
        a.update(kw)
        return f(a["p"], a["G"], a["r"], a["gm"], a["eps"], a["T"], a["H"], a["ro"], a["o"], None)
    assert call(p=None) == INVALID
    assert call(G=0) == INVALID
    assert call(G=9) == INVALID                                       # above MOE_NORM_MAX_RANKS
    assert call(p=(ctypes.c_void_p * 2)(FAKE, None)) == INVALID       # a null partial
    assert call(p=(ctypes.c_void_p * 2)(FAKE, MIS)) == INVALID        # a misaligned partial
    assert call(gm=None) == INVALID
    assert call(o=None) == INVALID
    assert call(r=MIS) == INVALID
    assert call(ro=MIS) == INVALID
    assert call(T=-1) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(eps=float("inf")) == INVALID
    assert call(H=4100) == UNSUPPORTED                                # not a multiple of 8
    assert call(H=16392) == UNSUPPORTED                               # above 16384
    assert call(T=0) == OK                                            # nothing to do
    assert call(T=0, r=None, ro=None, gm=None, o=None) == OK          # no data pointer read
    assert call(T=0, H=4100) == UNSUPPORTED                           # the shape still checked


def test_forward_layers_norm_argument_errors():
    f = ops.lib().moe_mxfp4_forward_layers_norm
    lay = (ops._Layer * 2)(ops._Layer(FAKE, FAKE, FAKE, FAKE, FAKE),
                           ops._Layer(FAKE, FAKE, FAKE, FAKE, FAKE))
    gam = (ctypes.c_void_p * 2)(FAKE, FAKE)
    def call(**kw):
        a = dict(x=FAKE, L=2, lay=ctypes.cast(lay, ctypes.c_void_p), g=gam, eps=1e-6, r=FAKE,
                 T=4, H=512, I=256, E=8, K=2, s=1, act=0, pf=0, o=FAKE2, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return f(a["x"], a["L"], a["lay"], a["g"], a["eps"], a["r"], a["T"], a["H"], a["I"],
                 a["E"], a["K"], a["s"], a["act"], a["pf"], a["o"], a["ws"], a["wsb"], None)
    assert call(g=None) == INVALID
    assert call(L=0) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(r=None) == INVALID
    assert call(r=MIS) == INVALID
    assert call(r=FAKE, o=FAKE) == INVALID                            # residual is out
    assert call(g=(ctypes.c_void_p * 2)(FAKE, None)) == INVALID       # a null gamma
    assert call(g=(ctypes.c_void_p * 2)(FAKE, MIS)) == INVALID        # a misaligned gamma
    assert call(H=32768) == UNSUPPORTED                               # beyond the norm's rows
    assert call(pf=2) == INVALID                                      # checks of the layers pass
    assert call(lay=None) == INVALID
    assert call(I=100) == UNSUPPORTED                                 # the layer's own checks


def test_quantize_argument_errors():
    f = ops.lib().moe_mxfp4_quantize
    assert f(FAKE, 0, 4, 48, FAKE, FAKE, None) == UNSUPPORTED      # cols % 32
    assert f(FAKE, 2, 4, 64, FAKE, FAKE, None) == INVALID          # dtype
    assert f(FAKE, 0, -1, 64, FAKE, FAKE, None) == INVALID
    assert f(None, 0, 4, 64, FAKE, FAKE, None) == INVALID
    assert f(MIS, 0, 4, 64, FAKE, FAKE, None) == INVALID           # misaligned source
    assert f(FAKE, 0, 0, 64, FAKE, FAKE, None) == OK               # empty


def test_quantize_blocked_argument_errors():
    f = ops.lib().moe_mxfp4_quantize_blocked
    assert f(FAKE, 0, 4, 96, None, 1, 4, FAKE, FAKE, None) == UNSUPPORTED    # cols % 128
    assert f(FAKE, 2, 4, 128, None, 1, 4, FAKE, FAKE, None) == INVALID       # dtype
    assert f(FAKE, 0, 4, 128, None, 1, 3, FAKE, FAKE, None) == INVALID       # out_rows < rows
    assert f(FAKE, 0, 4, 128, FAKE, 0, 12, FAKE, FAKE, None) == INVALID      # map with Kp < 1
    assert f(FAKE, 0, -1, 128, None, 1, 4, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 0, 4, 128, None, 1, 4, FAKE, MIS, None) == INVALID        # misaligned scales
    assert f(None, 0, 4, 128, None, 1, 4, FAKE, FAKE, None) == INVALID
    assert f(FAKE, 0, 4, 128, None, 1, 1 << 25, FAKE, FAKE, None) == UNSUPPORTED  # >= 2 GiB out
    assert f(FAKE, 0, 1, 1 << 31, FAKE, 1, 0, FAKE, FAKE, None) == UNSUPPORTED    # cols > 2^30
    assert f(FAKE, 0, 1 << 33, 128, FAKE, 1, 16, FAKE, FAKE, None) == UNSUPPORTED  # rows * Kp
    assert f(FAKE, 0, 0, 128, None, 1, 0, FAKE, FAKE, None) == OK            # empty


def test_weights_to_native_argument_errors():
    f = ops.lib().moe_weights_to_native
    B = ctypes.c_void_p(0x200000)                                  # FAKE + 1 MiB
    assert f(FAKE, 0, 24, 256, B, None) == UNSUPPORTED             # rows % 32
    assert f(FAKE, 0, 48, 256, B, None) == UNSUPPORTED             # whole strips, not pairs
    assert f(FAKE, 0, 32, 192, B, None) == UNSUPPORTED             # cols % 128
    assert f(FAKE, 2, 32, 256, B, None) == INVALID                 # weight format
    assert f(FAKE, 0, -16, 256, B, None) == INVALID
    assert f(None, 0, 32, 256, B, None) == INVALID
    assert f(FAKE, 1, 32, 256, None, None) == INVALID
    assert f(MIS, 0, 32, 256, B, None) == INVALID                  # misaligned source
    assert f(FAKE, 0, 32, 256, ctypes.c_void_p(0x100800), None) == INVALID   # overlap (4 KiB)
    assert f(FAKE, 1, 32, 256, ctypes.c_void_p(0x101000), None) == INVALID   # overlap (8 KiB)
    assert f(FAKE, 0, 0, 256, B, None) == OK                       # empty


def test_gemm_and_combine_argument_errors():
    gu = ops.lib().moe_expert_gate_up
    base = [FAKE, None, 0, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, 8, 256, 128, 16, 2, FAKE, None]
    def call(f, a, **over):
        a = list(a)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(gu, base, a0=None) == INVALID
    assert call(gu, base, a2=1) == INVALID                 # MXFP4 activations need scales
    assert call(gu, base, a2=7) == INVALID
    assert call(gu, base, a11=200) == UNSUPPORTED          # H % 128
    assert call(gu, base, a12=96) == UNSUPPORTED           # I % 128
    assert call(gu, base, a7=48) == UNSUPPORTED            # no kernel for 48-row tiles
    assert call(gu, base, a7=128, a11=384) == UNSUPPORTED  # tiled kernels need H % 256
    assert call(gu, base, a7=128, a11=6144, a10=0) == UNSUPPORTED  # bf16 tiled: H <= 4096
    # buffers addressed with 32-bit offsets stay below 2 GiB (checked before the pointers)
    assert call(gu, base, a10=300000, a11=4096) == UNSUPPORTED    # x: T*H*2 bytes
    assert call(gu, base, a11=65536, a12=32768) == UNSUPPORTED    # one expert's W13 codes
    assert call(gu, base, a7=128, a11=6144, a2=1, a1=FAKE, a10=0) == OK   # MXFP4: H <= 8192
    assert call(gu, base, a0=MIS) == INVALID
    assert call(gu, base, a10=0) == OK
    # blocked MXFP4 rows: tiled kernels only, scales needed and 16-byte aligned
    assert call(gu, base, a2=2, a1=FAKE) == UNSUPPORTED                     # 32-row tiles
    assert call(gu, base, a2=2, a7=128, a11=512) == INVALID                 # no scales
    assert call(gu, base, a2=2, a7=128, a11=512, a1=MIS) == INVALID         # misaligned scales
    assert call(gu, base, a2=3, a1=FAKE) == INVALID                         # no such format
    # blocked rows of T*K' sorted rows (rounded up to 16), not T tokens
    assert call(gu, base, a2=2, a7=128, a1=FAKE, a10=120000, a11=512, a14=80) == UNSUPPORTED
    assert call(gu, base, a2=1, a7=128, a1=FAKE, a10=120000, a11=512, a14=80, a15=None) == INVALID
    # gate/up with h quantised in the epilogue: blocked MXFP4 activations, tiled kernels
    gq = ops.lib().moe_expert_gate_up_quant
    baseq = [FAKE, FAKE, 2, FAKE, FAKE, FAKE, FAKE, 128, FAKE, FAKE, 8, 512, 128, 16, 2, FAKE,
             FAKE, None]
    assert call(gq, baseq, a7=32) == UNSUPPORTED                             # 32-row tiles
    assert call(gq, baseq, a7=32, a2=1) == UNSUPPORTED
    assert call(gq, baseq, a2=0) == INVALID and call(gq, baseq, a2=3) == INVALID   # bf16 / none
    assert call(gq, baseq, a11=384) == UNSUPPORTED                           # H % 256
    assert call(gq, baseq, a1=None) == INVALID                               # no scales
    assert call(gq, baseq, a15=None) == INVALID and call(gq, baseq, a16=None) == INVALID
    assert call(gq, baseq, a15=None, a16=None) == INVALID
    assert call(gq, baseq, a15=MIS) == INVALID and call(gq, baseq, a16=MIS) == INVALID
    assert call(gq, baseq, a10=0) == OK and call(gq, baseq, a10=0, a2=1) == OK
    dn = ops.lib().moe_expert_down
    based = [FAKE, None, 0, FAKE, FAKE, FAKE, 32, FAKE, FAKE, 8, 256, 128, 16, 2, FAKE, None]
    assert call(dn, based, a14=None) == INVALID
    assert call(dn, based, a10=100) == UNSUPPORTED
    assert call(dn, based, a6=64, a10=384) == UNSUPPORTED
    assert call(dn, based, a9=300000, a11=4096) == UNSUPPORTED   # h: T*K'*I*2 bytes >= 2 GiB
    assert call(dn, based, a9=0) == OK
    assert call(dn, based, a2=2, a1=FAKE) == UNSUPPORTED                    # 32-row tiles
    assert call(dn, based, a2=2, a6=128, a1=MIS) == INVALID                 # misaligned scales
    cb = ops.lib().moe_combine
    assert cb(None, FAKE, FAKE, 4, 256, 3, FAKE, None) == INVALID
    assert cb(FAKE, FAKE, FAKE, 4, 200, 3, FAKE, None) == UNSUPPORTED
    assert cb(FAKE, FAKE, FAKE, 0, 256, 3, FAKE, None) == OK


def test_gemm_tile_choice():
    # decode-like groups stream weights; larger groups use the LDS-tiled kernels
    assert ops.gemm_tile_m(64, 11, 513, 4096, 1024) == 32
    assert ops.gemm_tile_m(160, 11, 513, 4096, 1024) == 32     # 3 rows per expert
    assert ops.gemm_tile_m(192, 11, 513, 4096, 1024) == 64     # 4: the tiled kernels
    assert ops.gemm_tile_m(372, 11, 513, 4096, 1024, ops.ACT_MXFP4) == 32   # W4A4: 7
    assert ops.gemm_tile_m(450, 11, 513, 4096, 1024, ops.ACT_MXFP4) == 64   # W4A4: 9
    assert ops.gemm_tile_m(1536, 11, 513, 4096, 1024) == 64
    assert ops.gemm_tile_m(8192, 11, 513, 4096, 1024) == 64     # bf16: two workgroups per CU
    assert ops.gemm_tile_m(8192, 11, 513, 384, 1024) == 32      # H % 256 != 0
    # the tiled kernels keep a workgroup's weight scales for the whole K in LDS
    # MXFP4 activations: 128-row tiles above 48 rows (256-row tiles only on request)
    assert ops.gemm_tile_m(4096, 9, 257, 6144, 1536, ops.ACT_MXFP4) == 128
    assert ops.gemm_tile_m(2048, 9, 257, 6144, 1536, ops.ACT_MXFP4) == 128
    assert ops.gemm_tile_m(914, 9, 257, 6144, 1536, ops.ACT_MXFP4) == 64     # 32 rows per expert
    assert ops.gemm_tile_m(945, 9, 257, 6144, 1536, ops.ACT_MXFP4) == 128    # 33
    assert ops.gemm_tile_m(4096, 9, 257, 8192, 1536, ops.ACT_MXFP4) == 128
    assert ops.gemm_tile_m(4096, 9, 257, 6144, 1536, ops.ACT_BF16) == 32
    assert ops.gemm_tile_m(8192, 11, 513, 4096, 4608, ops.ACT_BF16) == 32


def test_forward_argument_errors_and_workspace():
    f = ops.lib().moe_mxfp4_forward
    need = ops.workspace_size(8, 256, 128, 16, 2, 0, 0)
    assert need > 0 and ops.workspace_size(0, 256, 128, 16, 2, 0, 0) == 0
    assert ops.workspace_size(8, 256, 128, 16, 2, 0, 1) > need      # W4A4 adds the quantised copies
    base = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 8, 256, 128, 16, 2, 0, 0, FAKE, None, None,
            FAKE, need, None]
    def call(**over):
        a = list(base)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a18=need - 1) == WS_SMALL
    assert call(a17=None) == INVALID
    assert call(a0=None) == INVALID
    assert call(a14=None) == INVALID
    assert call(a12=1) == INVALID                          # shared without gate logits
    assert call(a13=5) == INVALID
    assert call(a11=17) == INVALID                         # K > E
    assert call(a8=96) == UNSUPPORTED
    assert call(a10=2048) == UNSUPPORTED
    assert call(a7=300000, a8=4096) == UNSUPPORTED          # x: T*H*2 bytes >= 2 GiB
    assert call(a3=MIS) == INVALID
    assert call(a7=0, a0=None, a17=None, a18=0) == OK      # T = 0
    fr = ops.lib().moe_mxfp4_forward_router
    based = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 256, 128, 16, 2, 1, 0, FAKE, None, None, None,
             FAKE, ops.workspace_size(8, 256, 128, 16, 2, 1, 0), None]
    def callr(**over):
        a = list(based)
        for i, v in over.items():
            a[int(i[1:])] = v
        return fr(*a)
    assert callr(a1=None) == INVALID                        # no router rows
    assert callr(a1=MIS) == INVALID
    assert callr(a0=None) == INVALID
    assert callr(a10=17) == INVALID                         # K > E
    assert callr(a7=200) == UNSUPPORTED                     # H % 128
    assert callr(a18=1) == WS_SMALL
    assert callr(a6=0, a0=None, a1=None, a17=None, a18=0) == OK


def test_mxfp8_argument_errors():
    L = ops.lib()
    q = L.moe_mxfp8_quantize
    assert q(FAKE, 2, 4, 64, FAKE, FAKE, None) == INVALID       # bad dtype
    assert q(FAKE, 0, 4, 48, FAKE, FAKE, None) == UNSUPPORTED   # cols not a multiple of 32
    assert q(MIS, 0, 4, 64, FAKE, FAKE, None) == INVALID        # misaligned source
    assert q(None, 0, 0, 64, None, None, None) == OK            # nothing to do
    gu = L.moe_mxfp8_expert_gate_up
    # x, sorted, offsets, tiles, num_tiles, tile_m, w13, w13s, T, H, I, Ep, Kp, h, stream
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, 4, 256, 128, 9, 3, FAKE, None]
    def call(f, args, **kw):
        a = list(args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)
    assert call(gu, base, a5=256) == UNSUPPORTED                # no 256-row MXFP8 tiles
    assert call(gu, base, a5=64, a9=384) == UNSUPPORTED         # tiled: H a multiple of 256
    assert call(gu, base, a9=200) == UNSUPPORTED                # H not a multiple of 128
    assert call(gu, base, a0=None) == INVALID
    assert call(gu, base, a0=MIS) == INVALID
    assert call(gu, base, a8=0, a0=None) == OK                  # T = 0
    dn = L.moe_mxfp8_expert_down
    # h, offsets, tiles, num_tiles, tile_m, w2, w2s, T, H, I, Ep, Kp, y, stream
    based = [FAKE, FAKE, FAKE, FAKE, 32, FAKE, FAKE, 4, 256, 128, 9, 3, FAKE, None]
    assert call(dn, based, a4=256) == UNSUPPORTED
    assert ops.mxfp8_gemm_tile_m(64, 11, 513, 4096, 1024) == 32
    assert ops.mxfp8_gemm_tile_m(192, 11, 513, 4096, 1024) == 32   # 4 rows per expert
    assert ops.mxfp8_gemm_tile_m(256, 11, 513, 4096, 1024) == 64   # 5
    assert ops.mxfp8_gemm_tile_m(1536, 11, 513, 4096, 1024) == 64
    assert ops.mxfp8_gemm_tile_m(8192, 11, 513, 4096, 1024) == 64
    assert ops.mxfp8_gemm_tile_m(8192, 11, 513, 4096, 4608) == 32   # I above the tiled limit
    assert call(dn, based, a12=None) == INVALID
    assert call(dn, based, a5=MIS) == INVALID
    # an expert's 2I x H code bytes must fit a 32-bit buffer range
    assert call(gu, base, a9=65536, a10=65536) == UNSUPPORTED
    ws = ops.mxfp8_workspace_size(64, 4096, 1024, 512, 10, 1)
    assert ws == ops.workspace_size(64, 4096, 1024, 512, 10, 1, ops.ACT_BF16) and ws > 0
    assert ops.mxfp8_workspace_size(0, 4096, 1024, 512, 10, 1) == 0
    fw = L.moe_mxfp8_forward
    # x, logits, gate, w13, w13s, w2, w2s, T, H, I, E, K, shared, out, ids, w, ws, bytes, stream
    fb = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 256, 128, 8, 2, 1, FAKE, None, None, FAKE,
          1 << 30, None]
    assert call(fw, fb, a17=16) == WS_SMALL
    assert call(fw, fb, a2=None) == INVALID                     # shared without gate logits
    assert call(fw, fb, a8=300) == UNSUPPORTED
    assert call(fw, fb, a7=0) == OK


def test_forward_layers_argument_errors():
    f = ops.lib().moe_mxfp4_forward_layers
    arr = (ops._Layer * 2)(ops._Layer(FAKE, FAKE, FAKE, FAKE, FAKE),
                           ops._Layer(FAKE, FAKE, FAKE, FAKE, FAKE))
    p = ctypes.cast(arr, ctypes.c_void_p)
    # x, L, layers, T, H, I, E, K, shared, act, prefetch, out, ws, bytes, stream
    base = [FAKE, 2, p, 4, 256, 128, 8, 2, 1, 0, 1, FAKE, FAKE, 1 << 30, None]
    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return f(*a)
    assert call(a1=0) == INVALID                       # L < 1
    assert call(a2=None) == INVALID                    # no layer array
    assert call(a10=2) == INVALID                      # prefetch flag
    assert call(a13=16) == WS_SMALL
    assert call(a4=200) == UNSUPPORTED                 # H not a multiple of 128
    assert call(a3=0) == OK                            # T = 0: nothing to do
    arr[1] = ops._Layer(FAKE, None, FAKE, FAKE, FAKE)  # a later layer's null pointer
    assert call() == INVALID
    arr[1] = ops._Layer(FAKE, FAKE, FAKE, MIS, FAKE)   # a later layer's misaligned W2
    assert call() == INVALID


def test_forward_noalloc_argument_errors():
    """Every check of the no-allocation forward returns before any HIP call,
    including the limit of its scratch."""
    f = ops.lib().moe_mxfp4_forward_noalloc
    a = [FAKE] * 7
    assert f(None, *a[1:], 4, 256, 128, 16, 2, 0, 0, FAKE, None, None, None) == INVALID   # null x
    assert f(*a, 4, 200, 128, 16, 2, 0, 0, FAKE, None, None, None) == UNSUPPORTED         # H % 128
    assert f(*a, 4, 256, 128, 16, 2, 0, 5, FAKE, None, None, None) == INVALID             # act_fmt
    assert f(*a, 0, 256, 128, 16, 2, 0, 0, FAKE, None, None, None) == OK                  # T = 0
    # 588 decode tokens need more than the 64 MiB scratch; 587 fit
    assert ops.lib().moe_mxfp4_workspace_size(588, 4096, 1024, 512, 10, 1, 0) > ops.NOALLOC_SCRATCH_BYTES
    assert f(*a, 588, 4096, 1024, 512, 10, 1, 0, FAKE, None, None, None) == WS_SMALL
    assert ops.lib().moe_mxfp4_workspace_size(587, 4096, 1024, 512, 10, 1, 0) <= ops.NOALLOC_SCRATCH_BYTES

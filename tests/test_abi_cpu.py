"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every symbol include/moe_wq.h declares, reject invalid
arguments with the documented status codes before touching a device, and pack weights into
the documented layout (checked with a test-local unpacker written from that description).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import quantized_expert_layer_amd as q
from tests.conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "moe_wq.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert set(declared) == set(q.EXPORTED_SYMBOLS), declared
    L = q.lib()
    for name in declared:
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", q.lib_path], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", nm))
    assert set(declared) <= exported


def test_version_and_status_strings():
    assert q.version() >= 100
    for s in (0, -1, -2, -3, -4, -5):
        assert q.status_str(s).startswith("MOE_")
    assert q.status_str(123) == "unknown status"


def test_packed_bytes():
    assert q.moe_packed_bytes("int4", 3, 256, 32) == 3 * 256 * 32 // 2
    assert q.moe_packed_bytes("int8", 3, 256, 32) == 3 * 256 * 32
    assert q.moe_packed_bytes("fp16", 3, 256, 32) == 3 * 256 * 32 * 2
    assert q.moe_packed_bytes("int4", 3, 100, 32) == 0        # K % 128
    assert q.moe_packed_bytes("int4", 3, 128, 24) == 0        # N % 16


# ---------------------------------------------------------------- packer vs documented layout
def _unpack(packed, wtype, E, K, N):
    """Inverse of the documented layout, written independently of the C packer."""
    ncb = N // 16
    if wtype == "int4":
        ksb = 128
        words = packed.view(np.uint32).reshape(E, ncb, K // ksb, 64, 4)
        out = np.empty((E, K, N), np.int64)
        order = [0, 2, 4, 6, 1, 3, 5, 7]
        for l in range(64):
            n = np.arange(ncb)[:, None] * 16 + (l & 15)                      # [ncb, 1]
            for j in range(4):
                w = words[:, :, :, l, j].astype(np.int64)                      # [E, ncb, nSB]
                for p in range(8):
                    k = np.arange(K // ksb)[None, :] * ksb + j * 32 + 8 * (l >> 4) + order[p]
                    out[:, k, n] = ((w >> (4 * p)) & 0xF) - 8
        return out
    if wtype == "int8":
        ksb = 64
        words = packed.view(np.uint32).reshape(E, ncb, K // ksb, 64, 4)
        out = np.empty((E, K, N), np.int64)
        for l in range(64):
            n = np.arange(ncb)[:, None] * 16 + (l & 15)
            for wi in range(4):
                w = words[:, :, :, l, wi].astype(np.int64)
                for b in range(4):
                    k = (np.arange(K // ksb)[None, :] * ksb + (wi >> 1) * 32 + 8 * (l >> 4)
                         + 4 * (wi & 1) + b)
                    out[:, k, n] = ((w >> (8 * b)) & 0xFF) - 128
        return out
    ksb = 32
    halves = packed.view(np.uint16).reshape(E, ncb, K // ksb, 64, 8)
    out = np.empty((E, K, N), np.uint16)
    for l in range(64):
        n = np.arange(ncb)[:, None] * 16 + (l & 15)
        for i in range(8):
            k = np.arange(K // ksb)[None, :] * ksb + 8 * (l >> 4) + i
            out[:, k, n] = halves[:, :, :, l, i]
    return out


@pytest.mark.parametrize("wtype,E,K,N", [("int4", 2, 256, 48), ("int8", 3, 128, 32),
                                         ("int4", 1, 384, 16)])
def test_pack_roundtrip_integer_codes(wtype, E, K, N):
    rng = np.random.default_rng(1)
    lo, hi = (-8, 8) if wtype == "int4" else (-128, 128)
    codes = rng.integers(lo, hi, size=(E, K, N)).astype(np.int8)
    packed = q.moe_pack_wq(codes, wtype)
    assert packed.size == q.moe_packed_bytes(wtype, E, K, N)
    assert np.array_equal(_unpack(packed, wtype, E, K, N), codes)


def test_pack_roundtrip_fp16():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((2, 128, 32)).astype(np.float16)
    packed = q.moe_pack_wq(w, "fp16")
    assert np.array_equal(_unpack(packed, "fp16", 2, 128, 32), w.view(np.uint16))


def test_pack_int4_nibble_order_matches_page():
    # K-step 0 of lane 0 holds rows 0..7 of column 0; nibble p holds row order[p] (+8).
    codes = np.zeros((1, 128, 16), np.int8)
    codes[0, :8, 0] = np.arange(8) - 4                       # rows 0..7 -> -4..3
    word = q.moe_pack_wq(codes, "int4").view(np.uint32)[0]
    nibbles = [(int(word) >> (4 * p)) & 0xF for p in range(8)]
    assert nibbles == [r - 4 + 8 for r in (0, 2, 4, 6, 1, 3, 5, 7)]


def test_pack_rejects_out_of_range_int4():
    codes = np.zeros((1, 128, 16), np.int8)
    codes[0, 5, 3] = 8
    with pytest.raises(q.MoEError) as ei:
        q.moe_pack_wq(codes, "int4")
    assert ei.value.status == q.MOE_ERR_INVALID


# ---------------------------------------------------------------- validation before launch
FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced on these paths
MIS = ctypes.c_void_p(0x10002)        # misaligned


def test_route_topk_active_validation():
    L = q.lib()
    f = L.moe_route_topk_active
    assert f(FAKE, FAKE, 4, 8, 9, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID     # k > E
    assert f(FAKE, FAKE, 4, 8, 2, 7, FAKE, FAKE, None) == q.MOE_ERR_INVALID     # gate mode
    assert f(None, FAKE, 4, 8, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID
    assert f(None, None, 0, 8, 2, 0, None, None, None) == q.MOE_OK              # T = 0
    if not gpu_available():
        assert f(FAKE, None, 4, 8, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_NO_DEVICE
        assert f(FAKE, MIS, 4, 8, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_NO_DEVICE   # bytes


def test_route_topk_validation():
    L = q.lib()
    assert L.moe_route_topk(FAKE, 4, 8, 9, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID   # k > E
    assert L.moe_route_topk(FAKE, 4, 8, 0, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID   # k = 0
    assert L.moe_route_topk(FAKE, 4, 300, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID  # E > 256
    assert L.moe_route_topk(FAKE, 4, 8, 2, 7, FAKE, FAKE, None) == q.MOE_ERR_INVALID   # gate mode
    assert L.moe_route_topk(None, 4, 8, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID
    assert L.moe_route_topk(None, 0, 8, 2, 0, None, None, None) == q.MOE_OK            # T = 0
    assert L.moe_route_topk(FAKE, -1, 8, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_INVALID


def test_permute_workspace_size():
    L = q.lib()
    assert L.moe_permute_workspace_size(512, 2, 8) == 0               # one workgroup sorts
    assert L.moe_permute_workspace_size(513, 2, 8) == 0                # 2 blocks, one launch
    assert L.moe_permute_workspace_size(4096, 2, 16) == 0              # 8 blocks, one launch
    assert L.moe_permute_workspace_size(4097, 2, 16) == 9 * 16 * 4     # 9 blocks: two launches
    assert L.moe_permute_workspace_size(0, 2, 8) == 0


def test_permute_validation():
    L = q.lib()
    args = lambda **kw: [kw.get(n, v) for n, v in (
        ("ids", FAKE), ("w", FAKE), ("x", FAKE), ("T", 4), ("k", 2), ("E", 8), ("d", 64),
        ("perm", FAKE), ("inv", FAKE), ("off", FAKE), ("xp", FAKE), ("wp", FAKE),
        ("ws", None), ("wsb", 0), ("s", None))]
    assert L.moe_permute(*args(d=60)) == q.MOE_ERR_UNSUPPORTED
    assert L.moe_permute(*args(k=9)) == q.MOE_ERR_INVALID
    assert L.moe_permute(*args(x=MIS)) == q.MOE_ERR_INVALID
    assert L.moe_permute(*args(w=None)) == q.MOE_ERR_INVALID          # w_perm needs topk_w
    assert L.moe_permute(*args(perm=None)) == q.MOE_ERR_INVALID
    assert L.moe_permute(*args(T=0, ids=None, x=None)) == q.MOE_OK
    assert L.moe_permute(*args(x=None)) == q.MOE_ERR_INVALID          # x_perm needs x
    assert L.moe_permute(*args(x=None, xp=None, T=0)) == q.MOE_OK      # x may go with x_perm
    # more than 8192 slots need the workspace of the two-launch sort (k = 2: 9 blocks)
    assert L.moe_permute(*args(T=4097, ws=None, wsb=0)) == q.MOE_ERR_WORKSPACE
    assert L.moe_permute(*args(T=4097, ws=FAKE, wsb=9 * 8 * 4 - 1)) == q.MOE_ERR_WORKSPACE


def _gemm_args(**kw):
    d = dict(a=FAKE, off=FAKE, R=64, E=8, K=256, N=64, w=FAKE, s=FAKE, wt=0, g=128, act=1,
             rs=None, out=FAKE, opts=None, ws=None, wsb=0, stream=None)
    d.update(kw)
    return [d[n] for n in ("a", "off", "R", "E", "K", "N", "w", "s", "wt", "g", "act", "rs",
                           "out", "opts", "ws", "wsb", "stream")]


def test_gemm_validation():
    L = q.lib()
    g = L.moe_grouped_gemm_wq
    assert g(*_gemm_args(K=200)) == q.MOE_ERR_UNSUPPORTED
    assert g(*_gemm_args(N=40)) == q.MOE_ERR_UNSUPPORTED
    assert g(*_gemm_args(N=48, act=2)) == q.MOE_ERR_UNSUPPORTED        # SwiGLU needs N % 32
    assert g(*_gemm_args(g=64)) == q.MOE_ERR_UNSUPPORTED
    assert g(*_gemm_args(wt=2, g=128)) == q.MOE_ERR_UNSUPPORTED        # fp16 has no groups
    assert g(*_gemm_args(wt=5)) == q.MOE_ERR_INVALID
    assert g(*_gemm_args(act=3)) == q.MOE_ERR_INVALID
    assert g(*_gemm_args(E=0)) == q.MOE_ERR_INVALID
    assert g(*_gemm_args(E=257)) == q.MOE_ERR_INVALID
    assert g(*_gemm_args(s=None)) == q.MOE_ERR_INVALID                 # int codes need scales
    assert g(*_gemm_args(a=MIS)) == q.MOE_ERR_INVALID
    assert g(*_gemm_args(R=0, a=None, out=None)) == q.MOE_OK
    o = q.GemmOpts()
    o.path = 9
    assert g(*_gemm_args(opts=ctypes.byref(o))) == q.MOE_ERR_INVALID
    o.path, o.split_k = q.PATH_STREAM, q.MOE_MAX_SPLIT_K + 1            # beyond the limit
    assert g(*_gemm_args(opts=ctypes.byref(o))) == q.MOE_ERR_INVALID
    o.split_k = -1
    assert g(*_gemm_args(opts=ctypes.byref(o))) == q.MOE_ERR_INVALID
    # the int-to-float choice: 0 or 1; the conversion-instruction kernels exist for the tile
    # path with per-channel scales, ReLU or no activation and the 48-row / 64x128 tiles
    o.path, o.split_k, o.i2f = q.PATH_TILE, 0, 2
    assert g(*_gemm_args(opts=ctypes.byref(o))) == q.MOE_ERR_INVALID
    o.i2f = -1
    assert g(*_gemm_args(opts=ctypes.byref(o))) == q.MOE_ERR_INVALID
    o.i2f, o.tile = q.I2F_NATIVE, q.TILE_48x256
    for kw in (dict(g=128), dict(act=2), dict(wt=2, g=0, s=None)):
        assert g(*_gemm_args(opts=ctypes.byref(o), **kw)) == q.MOE_ERR_UNSUPPORTED, kw
    for t in (q.TILE_128x128,):
        o.tile = t
        assert g(*_gemm_args(g=0, opts=ctypes.byref(o))) == q.MOE_ERR_UNSUPPORTED, t
    o.path, o.tile = q.PATH_STREAM, q.TILE_AUTO
    assert g(*_gemm_args(g=0, opts=ctypes.byref(o))) == q.MOE_ERR_UNSUPPORTED
    o.path, o.tile = q.PATH_TILE, q.TILE_48x128
    assert g(*_gemm_args(g=0, R=0, a=None, out=None, opts=ctypes.byref(o))) == q.MOE_OK
    o.i2f, o.tile = q.I2F_TRICK, q.TILE_AUTO
    # the K split happens inside a block: no path needs a workspace
    for path in (q.PATH_AUTO, q.PATH_STREAM, q.PATH_TILE):
        for split in (0, 1, q.MOE_MAX_SPLIT_K):
            o.path, o.split_k = path, split
            assert L.moe_gemm_workspace_size(64, 8, 256, 64, 0, 1, ctypes.byref(o)) == 0


def test_combine_and_dequant_validation():
    L = q.lib()
    assert L.moe_unpermute_combine(FAKE, FAKE, None, None, 4, 9, 64, FAKE, None) == q.MOE_ERR_INVALID
    assert L.moe_unpermute_combine(FAKE, FAKE, None, None, 4, 2, 12, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    assert L.moe_unpermute_combine(FAKE, FAKE, None, MIS, 4, 2, 64, FAKE, None) == q.MOE_ERR_INVALID
    assert L.moe_dequant(FAKE, FAKE, 2, 0, 2, 128, 16, FAKE, None) == q.MOE_ERR_INVALID  # fp16
    assert L.moe_dequant(FAKE, FAKE, 0, 0, 2, 100, 16, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    assert L.moe_dequant(None, FAKE, 0, 0, 2, 128, 16, FAKE, None) == q.MOE_ERR_INVALID
    # every pointer follows the header's 16-byte convention
    assert L.moe_dequant(MIS, FAKE, 0, 0, 2, 128, 16, FAKE, None) == q.MOE_ERR_INVALID
    assert L.moe_dequant(FAKE, MIS, 0, 0, 2, 128, 16, FAKE, None) == q.MOE_ERR_INVALID
    assert L.moe_dequant(FAKE, FAKE, 0, 0, 2, 128, 16, MIS, None) == q.MOE_ERR_INVALID


@pytest.mark.skipif(gpu_available(), reason="valid calls would launch on a real GPU")
def test_valid_calls_report_no_device_without_gpu():
    L = q.lib()
    assert L.moe_route_topk(FAKE, 4, 8, 2, 0, FAKE, FAKE, None) == q.MOE_ERR_NO_DEVICE
    assert L.moe_grouped_gemm_wq(*_gemm_args()) == q.MOE_ERR_NO_DEVICE
    assert L.moe_dequant(FAKE, FAKE, 0, 0, 2, 128, 16, FAKE, None) == q.MOE_ERR_NO_DEVICE


def test_binding_limits_match_header():
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "include", "moe_wq.h")).read()
    for name in ("MOE_MAX_EXPERTS", "MOE_MAX_TOPK", "MOE_MAX_SPLIT_K", "MOE_DECODE_MAX_TOKENS",
                 "MOE_DECODE_MAX_ROWS"):
        m = re.search(r"#define\s+" + name + r"\s+(\d+)", text)
        assert m and int(m.group(1)) == getattr(q, name), name


def test_gemm_rows_validation():
    L = q.lib()
    g = L.moe_grouped_gemm_wq_rows

    def args(**kw):
        d = dict(a=FAKE, an=64, ar=FAKE, div=2, off=FAKE, R=64, E=8, K=256, N=64, w=FAKE, s=FAKE,
                 wt=0, g=128, act=1, rs=None, out=FAKE, on=64, orows=None, opts=None, ws=None,
                 wsb=0, stream=None)
        d.update(kw)
        return [d[n] for n in ("a", "an", "ar", "div", "off", "R", "E", "K", "N", "w", "s", "wt",
                               "g", "act", "rs", "out", "on", "orows", "opts", "ws", "wsb",
                               "stream")]

    assert g(*args(div=0)) == q.MOE_ERR_INVALID
    assert g(*args(an=-1)) == q.MOE_ERR_INVALID
    assert g(*args(on=-1)) == q.MOE_ERR_INVALID
    assert g(*args(ar=MIS)) == q.MOE_ERR_INVALID
    assert g(*args(ar=None, orows=MIS)) == q.MOE_ERR_INVALID
    assert g(*args(an=0)) == q.MOE_ERR_INVALID                          # a_rows needs rows of a
    assert g(*args(K=200)) == q.MOE_ERR_UNSUPPORTED                    # the plain checks apply
    assert g(*args(R=0, a=None, out=None, ar=None)) == q.MOE_OK
    if not gpu_available():
        assert g(*args()) == q.MOE_ERR_NO_DEVICE
        assert g(*args(ar=None, div=0, orows=FAKE)) == q.MOE_ERR_NO_DEVICE   # div unused


def test_probe_validation():
    L = q.lib()
    assert L.moe_probe_read(FAKE, 64, FAKE, 0, None) == q.MOE_ERR_INVALID       # no blocks
    assert L.moe_probe_read(FAKE, 60, FAKE, 8, None) == q.MOE_ERR_INVALID       # bytes % 16
    assert L.moe_probe_read(MIS, 64, FAKE, 8, None) == q.MOE_ERR_INVALID
    assert L.moe_probe_read(None, 0, None, 8, None) == q.MOE_OK                 # nothing to read
    assert L.moe_probe_mfma(-1, FAKE, 8, None) == q.MOE_ERR_INVALID
    assert L.moe_probe_mfma(1 << 15, FAKE, 8, None) == q.MOE_ERR_INVALID
    assert L.moe_probe_mfma(4, FAKE, 0, None) == q.MOE_ERR_INVALID
    if not gpu_available():
        assert L.moe_probe_mfma(4, FAKE, 8, None) == q.MOE_ERR_NO_DEVICE


def test_decode_layer_validation():
    L = q.lib()
    f = L.moe_decode_layer
    ws_need = L.moe_decode_workspace_size(4, 2, 8, 256, 512, 0)
    assert ws_need > 0

    def args(**kw):
        d = dict(logits=FAKE, active=None, x=FAKE, T=4, E=8, k=2, gate=0, d=256, inter=512,
                 act=2, w1=FAKE, s1=FAKE, w2=FAKE, s2=FAKE, wt=0, g=128, add=None, ready=None,
                 ids=FAKE, w=FAKE, out=FAKE, ws=FAKE, wsb=ws_need, stream=None)
        d.update(kw)
        return [d[n] for n in ("logits", "active", "x", "T", "E", "k", "gate", "d", "inter",
                               "act", "w1", "s1", "w2", "s2", "wt", "g", "add", "ready", "ids",
                               "w", "out", "ws", "wsb", "stream")]

    assert f(*args(k=9)) == q.MOE_ERR_INVALID
    assert f(*args(k=9, E=8)) == q.MOE_ERR_INVALID
    assert f(*args(gate=3)) == q.MOE_ERR_INVALID
    assert f(*args(act=3)) == q.MOE_ERR_INVALID
    assert f(*args(T=-1)) == q.MOE_ERR_INVALID
    assert f(*args(T=q.MOE_DECODE_MAX_TOKENS + 1)) == q.MOE_ERR_UNSUPPORTED
    assert f(*args(T=64, k=8, E=16, wsb=0)) == q.MOE_ERR_WORKSPACE
    assert f(*args(d=200)) == q.MOE_ERR_UNSUPPORTED
    assert f(*args(inter=1400)) == q.MOE_ERR_UNSUPPORTED
    assert f(*args(g=64)) == q.MOE_ERR_UNSUPPORTED
    assert f(*args(wt=2, g=128)) == q.MOE_ERR_UNSUPPORTED                # fp16 has no groups
    assert f(*args(s1=None)) == q.MOE_ERR_INVALID                        # int codes need scales
    assert f(*args(ids=None)) == q.MOE_ERR_INVALID
    assert f(*args(x=MIS)) == q.MOE_ERR_INVALID
    assert f(*args(add=MIS)) == q.MOE_ERR_INVALID
    assert f(*args(ws=None)) == q.MOE_ERR_WORKSPACE
    assert f(*args(wsb=ws_need - 1)) == q.MOE_ERR_WORKSPACE
    assert f(*args(T=0, logits=None, x=None, ids=None, w=None, out=None, ws=None)) == q.MOE_OK
    if not gpu_available():
        assert f(*args()) == q.MOE_ERR_NO_DEVICE
        # fp16 weights take no scales; the most rows a call takes (T * k = 512) is accepted
        fp16_ws = L.moe_decode_workspace_size(4, 2, 8, 256, 512, 2)
        assert f(*args(wt=2, g=0, s1=None, s2=None, wsb=fp16_ws)) == q.MOE_ERR_NO_DEVICE
        big = L.moe_decode_workspace_size(64, 8, 16, 256, 512, 0)
        assert f(*args(T=64, k=8, E=16, wsb=big)) == q.MOE_ERR_NO_DEVICE


def test_decode_shared_validation():
    """moe_decode_layer_shared validates as moe_decode_layer, plus its shared-expert arguments:
    a positive shared_inter that is a multiple of 128, both shared weights, 16-byte aligned, and
    integer-coded routed weights."""
    L = q.lib()
    f = L.moe_decode_layer_shared
    ws_need = L.moe_decode_shared_workspace_size(4, 2, 8, 256, 512, 0, 384)
    # the shared experts' hidden rows and output rows on top of the routed step's workspace
    assert ws_need >= L.moe_decode_workspace_size(4, 2, 8, 256, 512, 0) + 2 * 4 * (384 + 256)

    def args(**kw):
        d = dict(logits=FAKE, active=None, x=FAKE, T=4, E=8, k=2, gate=0, d=256, inter=512,
                 act=2, w1=FAKE, s1=FAKE, w2=FAKE, s2=FAKE, wt=0, g=128, sw1=FAKE, sw2=FAKE,
                 si=384, ids=FAKE, w=FAKE, out=FAKE, ws=FAKE, wsb=ws_need, stream=None)
        d.update(kw)
        return [d[n] for n in ("logits", "active", "x", "T", "E", "k", "gate", "d", "inter",
                               "act", "w1", "s1", "w2", "s2", "wt", "g", "sw1", "sw2", "si",
                               "ids", "w", "out", "ws", "wsb", "stream")]

    assert f(*args(k=9)) == q.MOE_ERR_INVALID
    assert f(*args(si=0)) == q.MOE_ERR_INVALID
    assert f(*args(si=-128)) == q.MOE_ERR_INVALID
    assert f(*args(si=200)) == q.MOE_ERR_UNSUPPORTED                     # shared_inter % 128
    assert f(*args(sw1=None)) == q.MOE_ERR_INVALID
    assert f(*args(sw2=None)) == q.MOE_ERR_INVALID
    assert f(*args(sw1=MIS)) == q.MOE_ERR_INVALID
    assert f(*args(sw2=MIS)) == q.MOE_ERR_INVALID
    assert f(*args(wt=2, g=0, s1=None, s2=None)) == q.MOE_ERR_UNSUPPORTED  # fp16 routed weights
    assert f(*args(d=200)) == q.MOE_ERR_UNSUPPORTED
    assert f(*args(ws=None)) == q.MOE_ERR_WORKSPACE
    assert f(*args(wsb=ws_need - 1)) == q.MOE_ERR_WORKSPACE
    # the routed step's workspace is not enough
    assert f(*args(wsb=L.moe_decode_workspace_size(4, 2, 8, 256, 512, 0))) == q.MOE_ERR_WORKSPACE
    assert f(*args(T=0, logits=None, x=None, ids=None, w=None, out=None, ws=None)) == q.MOE_OK
    if not gpu_available():
        assert f(*args()) == q.MOE_ERR_NO_DEVICE
        # more routed rows than the side launch takes (T * k > 128) is accepted too
        big = L.moe_decode_shared_workspace_size(64, 8, 16, 256, 512, 0, 384)
        assert f(*args(T=64, k=8, E=16, wsb=big)) == q.MOE_ERR_NO_DEVICE
    assert L.moe_decode_shared_workspace_size(4, 2, 8, 256, 512, 0, 0) == 0
    assert L.moe_decode_shared_workspace_size(4, 2, 8, 256, 512, 0, 200) == 0
    assert L.moe_decode_shared_workspace_size(4, 2, 8, 256, 512, 2, 384) == 0    # fp16 routed
    assert L.moe_decode_shared_workspace_size(65, 2, 8, 256, 512, 0, 384) == 0


def test_decode_noalloc_rejects_a_step_beyond_its_scratch():
    """moe_decode_layer_noalloc validates as moe_decode_layer, then refuses a step whose workspace
    exceeds its scratch array, before touching a device."""
    L = q.lib()
    f = L.moe_decode_layer_noalloc
    # 64 tokens x 8 experts x 6400 intermediate columns: 6.5 MB of hidden rows alone, plus the
    # second GEMM's partial sums, over the array's 8 MiB
    assert L.moe_decode_workspace_size(64, 8, 16, 4096, 6400, 0) > q.MOE_DECODE_SCRATCH_BYTES
    args = [FAKE, None, FAKE, 64, 16, 8, 0, 4096, 6400, 2, FAKE, FAKE, FAKE, FAKE, 0, 128, None,
            None, FAKE, FAKE, FAKE, None]
    assert f(*args) == q.MOE_ERR_UNSUPPORTED
    bad = list(args)
    bad[5] = 9                                             # k > MOE_MAX_TOPK
    assert f(*bad) == q.MOE_ERR_INVALID
    small = list(args)
    small[3], small[8] = 4, 512                            # fits the array
    assert L.moe_decode_workspace_size(4, 8, 16, 4096, 512, 0) <= q.MOE_DECODE_SCRATCH_BYTES
    if not gpu_available():
        assert f(*small) == q.MOE_ERR_NO_DEVICE


def test_decode_workspace_size():
    L = q.lib()
    assert L.moe_decode_workspace_size(65, 1, 8, 256, 512, 0) == 0          # T too large
    assert L.moe_decode_workspace_size(64, 9, 16, 256, 512, 0) == 0         # k too large
    assert L.moe_decode_workspace_size(4, 2, 8, 200, 512, 0) == 0           # d % 128
    T, k, E, d, inter = 17, 4, 60, 2048, 1408 // 128 * 128
    need = L.moe_decode_workspace_size(T, k, E, d, inter, 0)
    R = T * k
    # perm, inv_perm, offsets, w_perm, counters and the fp16 hidden rows at least
    assert need >= 4 * (3 * R + E + 1) + 4 * (d // 16) + 2 * R * inter
    # and it grows with the tokens
    assert L.moe_decode_workspace_size(T + 1, k, E, d, inter, 0) > need


def test_elb_validation():
    L = q.lib()
    acc, top = L.moe_elb_accumulate, L.moe_elb_top_m
    assert acc(FAKE, 2, 1, 0, 8, FAKE, None) == q.MOE_ERR_INVALID          # k = 0
    assert acc(FAKE, 2, 1, 2, 257, FAKE, None) == q.MOE_ERR_INVALID        # E > 256
    assert acc(FAKE, -1, 1, 2, 8, FAKE, None) == q.MOE_ERR_INVALID
    assert acc(FAKE, 2, 1, 2, 8, None, None) == q.MOE_ERR_INVALID          # no counts
    assert acc(MIS, 2, 1, 2, 8, FAKE, None) == q.MOE_ERR_INVALID
    assert acc(None, 0, 1, 2, 8, None, None) == q.MOE_OK                   # L = 0
    assert top(FAKE, 2, 8, 0, FAKE, None, None) == q.MOE_ERR_INVALID       # M = 0
    assert top(FAKE, 2, 8, 9, FAKE, None, None) == q.MOE_ERR_INVALID       # M > E
    assert top(FAKE, 2, 8, 3, None, None, None) == q.MOE_ERR_INVALID
    assert top(FAKE, 2, 8, 3, FAKE, MIS, None) == q.MOE_ERR_INVALID
    assert top(None, 0, 8, 3, None, None, None) == q.MOE_OK
    if not gpu_available():
        assert acc(FAKE, 2, 1, 2, 8, FAKE, None) == q.MOE_ERR_NO_DEVICE
        assert acc(None, 2, 0, 2, 8, FAKE, None) == q.MOE_ERR_NO_DEVICE    # T = 0: no ids needed
        assert top(FAKE, 2, 8, 3, FAKE, None, None) == q.MOE_ERR_NO_DEVICE


def test_bf16_recombine_validation():
    L = q.lib()
    f = L.moe_bf16_recombine
    assert f(None, None, 0, None, None) == q.MOE_OK                        # nothing to do
    assert f(None, FAKE, 16, FAKE, None) == q.MOE_ERR_INVALID
    assert f(FAKE, FAKE, 16, None, None) == q.MOE_ERR_INVALID
    assert f(MIS, FAKE, 16, FAKE, None) == q.MOE_ERR_INVALID               # 16-byte aligned
    assert f(FAKE, FAKE, 1 << 41, FAKE, None) == q.MOE_ERR_UNSUPPORTED
    if not gpu_available():
        assert f(FAKE, FAKE, 17, FAKE, None) == q.MOE_ERR_NO_DEVICE

"""Python binding of libmoe_wq.so, the MI355X (gfx950) weight-only-quantized MoE expert layer.

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and the stream; nothing here computes.  The
functions carry the names of the C entry points declared in include/moe_wq.h.

The library is loaded on first use and a missing or unloadable library raises
`MoELibraryError`: there is no fallback implementation.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "MOE_OK", "MOE_ERR_INVALID", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
    "MOE_ERR_NO_DEVICE", "MOE_ERR_HIP",
    "GATE_TOPK", "GATE_ALL", "W_INT4", "W_INT8", "W_FP16", "ACT_NONE", "ACT_RELU",
    "ACT_SWIGLU", "PATH_AUTO", "PATH_STREAM", "PATH_TILE", "TILE_AUTO", "TILE_64x256",
    "TILE_64x128", "TILE_128x128", "TILE_48x256", "TILE_48x128", "I2F_TRICK", "I2F_NATIVE",
    "MOE_MAX_EXPERTS", "MOE_MAX_TOPK", "MOE_MAX_SPLIT_K",
    "MoEError", "MoELibraryError", "lib", "lib_path", "status_str", "version",
    "moe_route_topk", "moe_route_topk_active", "moe_permute", "moe_grouped_gemm_wq",
    "moe_grouped_gemm_wq_rows",
    "moe_unpermute_combine",
    "moe_dequant", "moe_pack_wq", "moe_packed_bytes", "moe_gemm_workspace_size",
    "moe_permute_workspace_size", "GemmOpts", "EXPORTED_SYMBOLS", "new_output",
    "moe_probe_read", "moe_probe_mfma", "moe_decode_layer", "moe_decode_workspace_size",
    "moe_decode_layer_noalloc", "MOE_DECODE_SCRATCH_BYTES", "moe_decode_layer_shared",
    "moe_decode_shared_workspace_size",
    "MOE_DECODE_MAX_TOKENS", "MOE_DECODE_MAX_ROWS", "moe_elb_accumulate", "moe_elb_top_m",
    "moe_bf16_recombine",
]

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE = 0, -1, -2, -3
MOE_ERR_NO_DEVICE, MOE_ERR_HIP = -4, -5
GATE_TOPK, GATE_ALL = 0, 1
W_INT4, W_INT8, W_FP16 = 0, 1, 2
ACT_NONE, ACT_RELU, ACT_SWIGLU = 0, 1, 2
PATH_AUTO, PATH_STREAM, PATH_TILE = 0, 1, 2
TILE_AUTO, TILE_64x256, TILE_64x128, TILE_128x128, TILE_48x256, TILE_48x128 = 0, 1, 2, 3, 4, 5
I2F_TRICK, I2F_NATIVE = 0, 1
I2FS = {"trick": I2F_TRICK, "native": I2F_NATIVE}
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_SPLIT_K = 256, 8, 8
MOE_DECODE_MAX_TOKENS, MOE_DECODE_MAX_ROWS = 64, 512
MOE_DECODE_SCRATCH_BYTES = 8 << 20

WTYPES = {"int4": W_INT4, "int8": W_INT8, "fp16": W_FP16}
ACTS = {"none": ACT_NONE, "relu": ACT_RELU, "swiglu": ACT_SWIGLU}
GATES = {"topk": GATE_TOPK, "all": GATE_ALL}

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_wq.so")

# Every symbol include/moe_wq.h declares.
EXPORTED_SYMBOLS = (
    "moe_route_topk", "moe_permute", "moe_permute_workspace_size", "moe_grouped_gemm_wq",
    "moe_grouped_gemm_wq_rows", "moe_gemm_workspace_size", "moe_unpermute_combine", "moe_dequant", "moe_packed_bytes",
    "moe_pack_wq", "moe_status_str", "moe_version", "moe_probe_read", "moe_probe_mfma",
    "moe_decode_layer", "moe_decode_workspace_size", "moe_route_topk_active",
    "moe_decode_layer_noalloc", "moe_decode_layer_shared", "moe_decode_shared_workspace_size",
    "moe_elb_accumulate", "moe_elb_top_m", "moe_bf16_recombine",
)


class MoEError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} ({status})")


class MoELibraryError(ImportError):
    pass


class GemmOpts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("i2f", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 4)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t


def lib():
    """The loaded library (loaded once; raises MoELibraryError when unavailable)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise MoELibraryError(f"{lib_path} is missing: build it with "
                              "`python -m quantized_expert_layer_amd.build`")
    # torch ships its own HIP runtime under the same soname.  Load it first so that the
    # library binds to that copy: two HIP runtimes in one process do not share devices,
    # and the library would then find no usable device for torch's tensors.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    try:
        L = ctypes.CDLL(lib_path)
    except OSError as e:
        raise MoELibraryError(f"cannot load {lib_path}: {e}") from e
    sig = {
        "moe_route_topk": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
        "moe_permute": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "moe_permute_workspace_size": (_SZ, [_I, _I, _I]),
        "moe_grouped_gemm_wq": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P,
                                     _P, _SZ, _P]),
        "moe_grouped_gemm_wq_rows": (_I, [_P, _I, _P, _I, _P, _I, _I, _I, _I, _P, _P, _I, _I,
                                          _I, _P, _P, _I, _P, _P, _P, _SZ, _P]),
        "moe_gemm_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _P]),
        "moe_unpermute_combine": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _P]),
        "moe_dequant": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P]),
        "moe_packed_bytes": (_SZ, [_I, _I, _I, _I]),
        "moe_pack_wq": (_I, [_P, _I, _I, _I, _I, _P]),
        "moe_status_str": (ctypes.c_char_p, [_I]),
        "moe_version": (_I, []),
        "moe_probe_read": (_I, [_P, _SZ, _P, _I, _P]),
        "moe_probe_mfma": (_I, [_I, _P, _I, _P]),
        "moe_decode_layer": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I,
                                  _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        "moe_decode_layer_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                          _I, _I, _P, _P, _P, _P, _P, _P]),
        "moe_route_topk_active": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
        "moe_elb_accumulate": (_I, [_P, _I, _I, _I, _I, _P, _P]),
        "moe_elb_top_m": (_I, [_P, _I, _I, _I, _P, _P, _P]),
        "moe_bf16_recombine": (_I, [_P, _P, _SZ, _P, _P]),
        "moe_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
        "moe_decode_layer_shared": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                         _I, _I, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]),
        "moe_decode_shared_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def version() -> int:
    return lib().moe_version()


def _check(fn, status):
    if status != MOE_OK:
        raise MoEError(fn, status)


# ---------------------------------------------------------------- tensor marshalling
# MOE_WQ_POISON=1: outputs (and layer workspaces) the binding allocates start as NaN (floating
# point) or 0 (integer) instead of whatever the allocator hands back, so an element a kernel
# failed to write cannot pass a test by holding a previous call's correct value.
_POISON = os.environ.get("MOE_WQ_POISON", "") not in ("", "0")


def new_output(shape, dtype, device):
    """torch.empty, pre-filled with the poison pattern when MOE_WQ_POISON is set."""
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if _POISON:
        t.fill_(float("nan") if t.is_floating_point() else 0)
    return t


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t, dtype, name, numel=None):
    torch = _torch()
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements, has {t.numel()}")


def _opts(path=PATH_AUTO, split_k=0, tile=TILE_AUTO, i2f=I2F_TRICK):
    if path == PATH_AUTO and split_k == 0 and tile == TILE_AUTO and i2f == I2F_TRICK:
        return None
    o = GemmOpts()
    o.path, o.split_k, o.tile, o.i2f = int(path), int(split_k), int(tile), int(i2f)
    return o


# ---------------------------------------------------------------- the five calls
def moe_route_topk(logits, k, gate_mode, topk_ids=None, topk_w=None, stream=None, active=None):
    """active (uint8 [T] device tensor or None): batch pruning, moe_route_topk_active."""
    torch = _torch()
    T, E = logits.shape
    gm = GATES.get(gate_mode, gate_mode)
    if topk_ids is None:
        topk_ids = new_output((T, k), torch.int32, logits.device)
    if topk_w is None:
        topk_w = new_output((T, k), torch.float32, logits.device)
    _need(logits, torch.float32, "logits")
    _need(topk_ids, torch.int32, "topk_ids", T * k)
    _need(topk_w, torch.float32, "topk_w", T * k)
    if active is None:
        _check("moe_route_topk", lib().moe_route_topk(_ptr(logits), T, E, k, gm, _ptr(topk_ids),
                                                      _ptr(topk_w), _stream(stream)))
    else:
        _need(active, torch.uint8, "active", T)
        _check("moe_route_topk_active", lib().moe_route_topk_active(
            _ptr(logits), _ptr(active), T, E, k, gm, _ptr(topk_ids), _ptr(topk_w),
            _stream(stream)))
    return topk_ids, topk_w


def moe_permute(topk_ids, topk_w, x, E, want_w_perm=True, out=None, stream=None,
                want_x_perm=True, ws=None):
    """Returns (perm, inv_perm, expert_offsets, x_perm or None, w_perm or None).
    want_x_perm=False skips the row copy (the first GEMM then reads x through perm).
    ws: uint8 device workspace of moe_permute_workspace_size bytes (allocated if None)."""
    torch = _torch()
    T, k = topk_ids.shape
    d = x.shape[1]
    R = T * k
    dev = x.device
    if out is None:
        out = (new_output(R, torch.int32, dev),
               new_output(R, torch.int32, dev),
               new_output(E + 1, torch.int32, dev),
               new_output((R, d), torch.float16, dev) if want_x_perm else None,
               new_output(R, torch.float32, dev)
               if (want_w_perm and topk_w is not None) else None)
    perm, inv_perm, offsets, x_perm, w_perm = out
    _need(topk_ids, torch.int32, "topk_ids")
    _need(topk_w, torch.float32, "topk_w")
    _need(x, torch.float16, "x")
    _need(perm, torch.int32, "perm", R)
    _need(inv_perm, torch.int32, "inv_perm", R)
    _need(offsets, torch.int32, "expert_offsets", E + 1)
    _need(x_perm, torch.float16, "x_perm", R * d)
    _need(w_perm, torch.float32, "w_perm", R)
    need = lib().moe_permute_workspace_size(T, k, E)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(ws, torch.uint8, "ws")
    _check("moe_permute", lib().moe_permute(
        _ptr(topk_ids), _ptr(topk_w), _ptr(x), T, k, E, d, _ptr(perm), _ptr(inv_perm),
        _ptr(offsets), _ptr(x_perm), _ptr(w_perm), _ptr(ws), 0 if ws is None else ws.numel(),
        _stream(stream)))
    return perm, inv_perm, offsets, x_perm, w_perm


def moe_gemm_workspace_size(R, E, K, N, wtype, act, path=PATH_AUTO, split_k=0):
    o = _opts(path, split_k)
    return lib().moe_gemm_workspace_size(R, E, K, N, WTYPES.get(wtype, wtype),
                                         ACTS.get(act, act), ctypes.byref(o) if o else None)


def moe_permute_workspace_size(T, k, E):
    return lib().moe_permute_workspace_size(T, k, E)


def moe_grouped_gemm_wq(a, expert_offsets, E, K, N, w_packed, scales, wtype, group_size, act,
                        row_scale=None, out=None, path=PATH_AUTO, split_k=0, ws=None,
                        stream=None, tile=TILE_AUTO, i2f=I2F_TRICK):
    torch = _torch()
    R = a.shape[0]
    wt = WTYPES.get(wtype, wtype)
    ac = ACTS.get(act, act)
    n_out = N // 2 if ac == ACT_SWIGLU else N
    if out is None:
        out = new_output((R, n_out), torch.float16, a.device)
    o = _opts(path, split_k, tile, I2FS.get(i2f, i2f))
    need_ws = lib().moe_gemm_workspace_size(R, E, K, N, wt, ac, ctypes.byref(o) if o else None)
    if need_ws and ws is None:
        ws = torch.empty(need_ws, dtype=torch.uint8, device=a.device)
    _need(a, torch.float16, "a", R * K)
    _need(expert_offsets, torch.int32, "expert_offsets", E + 1)
    _need(w_packed, torch.uint8, "w_packed")
    _need(scales, torch.float16, "scales")
    _need(row_scale, torch.float32, "row_scale", R)
    _need(out, torch.float16, "out", R * n_out)
    _need(ws, torch.uint8, "ws")
    _check("moe_grouped_gemm_wq", lib().moe_grouped_gemm_wq(
        _ptr(a), _ptr(expert_offsets), R, E, K, N, _ptr(w_packed), _ptr(scales), wt,
        int(group_size), ac, _ptr(row_scale), _ptr(out), ctypes.byref(o) if o else None,
        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out


def moe_grouped_gemm_wq_rows(a, a_rows, a_row_div, expert_offsets, R, E, K, N, w_packed, scales,
                             wtype, group_size, act, row_scale=None, out=None, out_rows=None,
                             path=PATH_AUTO, split_k=0, stream=None, tile=TILE_AUTO,
                             i2f=I2F_TRICK):
    """GEMM row p reads a[a_rows[p] // a_row_div] (a[p] if a_rows is None) and writes
    out[out_rows[p]] (out[p] if out_rows is None); R = number of GEMM rows."""
    torch = _torch()
    wt = WTYPES.get(wtype, wtype)
    ac = ACTS.get(act, act)
    n_out = N // 2 if ac == ACT_SWIGLU else N
    if out is None:
        out = new_output((R, n_out), torch.float16, a.device)
    o = _opts(path, split_k, tile, I2FS.get(i2f, i2f))
    a_nrows = a.shape[0]
    out_nrows = out.shape[0]
    _need(a, torch.float16, "a", a_nrows * K)
    _need(a_rows, torch.int32, "a_rows", R)
    _need(expert_offsets, torch.int32, "expert_offsets", E + 1)
    _need(w_packed, torch.uint8, "w_packed")
    _need(scales, torch.float16, "scales")
    _need(row_scale, torch.float32, "row_scale", R)
    _need(out, torch.float16, "out", out_nrows * n_out)
    _need(out_rows, torch.int32, "out_rows", R)
    _check("moe_grouped_gemm_wq_rows", lib().moe_grouped_gemm_wq_rows(
        _ptr(a), a_nrows, _ptr(a_rows), int(a_row_div), _ptr(expert_offsets), R, E, K, N,
        _ptr(w_packed), _ptr(scales), wt, int(group_size), ac, _ptr(row_scale), _ptr(out),
        out_nrows, _ptr(out_rows), ctypes.byref(o) if o else None, None, 0, _stream(stream)))
    return out


def moe_probe_read(src, blocks, sink=None, stream=None):
    """Attainable-read probe: reads all of `src` (a device tensor, bytes % 16 == 0) once;
    returns the per-block XOR sink (uint32 as int32 [blocks])."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(blocks, dtype=torch.int32, device=src.device)
    _need(sink, torch.int32, "sink", blocks)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _check("moe_probe_read", lib().moe_probe_read(_ptr(src), src.numel() * src.element_size(),
                                                  _ptr(sink), int(blocks), _stream(stream)))
    return sink


def moe_probe_mfma(iters, blocks, out=None, device="cuda", stream=None):
    """Attainable-MFMA probe: blocks x 4 waves x iters x 16 MFMA 16x16x32 fp16; returns the
    fp32 [blocks * 256] result (every element 512 * iters)."""
    torch = _torch()
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    _need(out, torch.float32, "out", blocks * 256)
    _check("moe_probe_mfma", lib().moe_probe_mfma(int(iters), _ptr(out), int(blocks),
                                                  _stream(stream)))
    return out


def moe_decode_workspace_size(T, k, E, d, inter, wtype):
    return lib().moe_decode_workspace_size(T, k, E, d, inter, WTYPES.get(wtype, wtype))


def moe_decode_layer(logits, x, k, gate_mode, inter, act, w1, s1, w2, s2, wtype, group_size,
                     addend=None, topk_ids=None, topk_w=None, out=None, ws=None, stream=None,
                     active=None, addend_ready=None):
    """The routed layer for a decode / verify step (T <= MOE_DECODE_MAX_TOKENS tokens).
    Returns (out fp16 [T, d], topk_ids int32 [T, k], topk_w fp32 [T, k]).  addend_ready: a
    recorded torch.cuda.Event the call waits for before it first reads addend."""
    torch = _torch()
    T, E = logits.shape
    d = x.shape[1]
    wt = WTYPES.get(wtype, wtype)
    dev = x.device
    if out is None:
        out = new_output((T, d), torch.float16, dev)
    if topk_ids is None:
        topk_ids = new_output((T, k), torch.int32, dev)
    if topk_w is None:
        topk_w = new_output((T, k), torch.float32, dev)
    if ws is None:
        need = lib().moe_decode_workspace_size(T, k, E, d, inter, wt)
        ws = new_output(max(need, 16), torch.uint8, dev)
    _need(logits, torch.float32, "logits", T * E)
    _need(x, torch.float16, "x", T * d)
    _need(w1, torch.uint8, "w1")
    _need(s1, torch.float16, "s1")
    _need(w2, torch.uint8, "w2")
    _need(s2, torch.float16, "s2")
    _need(addend, torch.float16, "addend", T * d)
    _need(topk_ids, torch.int32, "topk_ids", T * k)
    _need(topk_w, torch.float32, "topk_w", T * k)
    _need(out, torch.float16, "out", T * d)
    _need(ws, torch.uint8, "ws")
    _need(active, torch.uint8, "active", T)
    _check("moe_decode_layer", lib().moe_decode_layer(
        _ptr(logits), _ptr(active), _ptr(x), T, E, k, GATES.get(gate_mode, gate_mode), d, int(inter),
        ACTS.get(act, act), _ptr(w1), _ptr(s1), _ptr(w2), _ptr(s2), wt, int(group_size),
        _ptr(addend), None if addend_ready is None else addend_ready.cuda_event,
        _ptr(topk_ids), _ptr(topk_w), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))
    return out, topk_ids, topk_w


def moe_decode_shared_workspace_size(T, k, E, d, inter, wtype, shared_inter):
    return lib().moe_decode_shared_workspace_size(T, k, E, d, inter, WTYPES.get(wtype, wtype),
                                                  shared_inter)


def moe_decode_layer_shared(logits, x, k, gate_mode, inter, act, w1, s1, w2, s2, wtype,
                            group_size, shared_w1, shared_w2, shared_inter, topk_ids=None,
                            topk_w=None, out=None, ws=None, stream=None, active=None):
    """moe_decode_layer with the shared experts (fp16, SwiGLU, packed for E = 1) computed in
    the same launches.  Returns (out fp16 [T, d], topk_ids int32 [T, k], topk_w fp32 [T, k])."""
    torch = _torch()
    T, E = logits.shape
    d = x.shape[1]
    wt = WTYPES.get(wtype, wtype)
    dev = x.device
    if out is None:
        out = new_output((T, d), torch.float16, dev)
    if topk_ids is None:
        topk_ids = new_output((T, k), torch.int32, dev)
    if topk_w is None:
        topk_w = new_output((T, k), torch.float32, dev)
    if ws is None:
        need = lib().moe_decode_shared_workspace_size(T, k, E, d, inter, wt, int(shared_inter))
        ws = new_output(max(need, 16), torch.uint8, dev)
    _need(logits, torch.float32, "logits", T * E)
    _need(x, torch.float16, "x", T * d)
    _need(w1, torch.uint8, "w1")
    _need(s1, torch.float16, "s1")
    _need(w2, torch.uint8, "w2")
    _need(s2, torch.float16, "s2")
    _need(shared_w1, torch.uint8, "shared_w1")
    _need(shared_w2, torch.uint8, "shared_w2")
    _need(topk_ids, torch.int32, "topk_ids", T * k)
    _need(topk_w, torch.float32, "topk_w", T * k)
    _need(out, torch.float16, "out", T * d)
    _need(ws, torch.uint8, "ws")
    _need(active, torch.uint8, "active", T)
    _check("moe_decode_layer_shared", lib().moe_decode_layer_shared(
        _ptr(logits), _ptr(active), _ptr(x), T, E, k, GATES.get(gate_mode, gate_mode), d,
        int(inter), ACTS.get(act, act), _ptr(w1), _ptr(s1), _ptr(w2), _ptr(s2), wt,
        int(group_size), _ptr(shared_w1), _ptr(shared_w2), int(shared_inter), _ptr(topk_ids),
        _ptr(topk_w), _ptr(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out, topk_ids, topk_w


def moe_decode_layer_noalloc(logits, x, k, gate_mode, inter, act, w1, s1, w2, s2, wtype,
                             group_size, addend=None, topk_ids=None, topk_w=None, out=None,
                             stream=None, active=None, addend_ready=None):
    """moe_decode_layer on the library's own scratch array (no workspace argument; calls that
    overlap on one device race).  Returns (out, topk_ids, topk_w)."""
    torch = _torch()
    T, E = logits.shape
    d = x.shape[1]
    wt = WTYPES.get(wtype, wtype)
    dev = x.device
    if out is None:
        out = new_output((T, d), torch.float16, dev)
    if topk_ids is None:
        topk_ids = new_output((T, k), torch.int32, dev)
    if topk_w is None:
        topk_w = new_output((T, k), torch.float32, dev)
    _need(logits, torch.float32, "logits", T * E)
    _need(x, torch.float16, "x", T * d)
    _need(w1, torch.uint8, "w1")
    _need(s1, torch.float16, "s1")
    _need(w2, torch.uint8, "w2")
    _need(s2, torch.float16, "s2")
    _need(addend, torch.float16, "addend", T * d)
    _need(topk_ids, torch.int32, "topk_ids", T * k)
    _need(topk_w, torch.float32, "topk_w", T * k)
    _need(out, torch.float16, "out", T * d)
    _need(active, torch.uint8, "active", T)
    _check("moe_decode_layer_noalloc", lib().moe_decode_layer_noalloc(
        _ptr(logits), _ptr(active), _ptr(x), T, E, k, GATES.get(gate_mode, gate_mode), d,
        int(inter), ACTS.get(act, act), _ptr(w1), _ptr(s1), _ptr(w2), _ptr(s2), wt,
        int(group_size), _ptr(addend), None if addend_ready is None else addend_ready.cuda_event,
        _ptr(topk_ids), _ptr(topk_w), _ptr(out), _stream(stream)))
    return out, topk_ids, topk_w


def moe_elb_accumulate(ids, E, counts, stream=None):
    """One draft step: ids int32 [L, T, k] (device), counts int32 [L, E] updated in place."""
    torch = _torch()
    L, T, k = ids.shape
    _need(ids, torch.int32, "ids")
    _need(counts, torch.int32, "counts", L * E)
    _check("moe_elb_accumulate", lib().moe_elb_accumulate(_ptr(ids), L, T, k, E, _ptr(counts),
                                                          _stream(stream)))
    return counts


def moe_elb_top_m(counts, M, experts=None, top_counts=None, stream=None):
    """Per layer the M most-counted experts: returns (experts int32 [L, M], counts [L, M])."""
    torch = _torch()
    L, E = counts.shape
    if experts is None:
        experts = new_output((L, M), torch.int32, counts.device)
    if top_counts is None:
        top_counts = new_output((L, M), torch.int32, counts.device)
    _need(counts, torch.int32, "counts", L * E)
    _need(experts, torch.int32, "experts", L * M)
    _need(top_counts, torch.int32, "top_counts", L * M)
    _check("moe_elb_top_m", lib().moe_elb_top_m(_ptr(counts), L, E, int(M), _ptr(experts),
                                                _ptr(top_counts), _stream(stream)))
    return experts, top_counts


def moe_bf16_recombine(exponents, sign_mantissa, out=None, stream=None):
    """BF16 tensor [n] from uint8 exponent bytes [n] and sign-mantissa bytes [n] (device)."""
    torch = _torch()
    n = exponents.numel()
    if out is None:
        out = new_output(n, torch.bfloat16, exponents.device)
    _need(exponents, torch.uint8, "exponents", n)
    _need(sign_mantissa, torch.uint8, "sign_mantissa", n)
    _need(out, torch.bfloat16, "out", n)
    _check("moe_bf16_recombine", lib().moe_bf16_recombine(_ptr(exponents), _ptr(sign_mantissa),
                                                          n, _ptr(out), _stream(stream)))
    return out


def moe_unpermute_combine(y_perm, inv_perm, topk_w, addend, T, k, out=None, stream=None):
    torch = _torch()
    d = y_perm.shape[1]
    if out is None:
        out = new_output((T, d), torch.float16, y_perm.device)
    _need(y_perm, torch.float16, "y_perm")
    _need(inv_perm, torch.int32, "inv_perm", T * k)
    _need(topk_w, torch.float32, "topk_w", T * k)
    _need(addend, torch.float16, "addend", T * d)
    _need(out, torch.float16, "out", T * d)
    _check("moe_unpermute_combine", lib().moe_unpermute_combine(
        _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(addend), T, k, d, _ptr(out),
        _stream(stream)))
    return out


def moe_dequant(w_packed, scales, wtype, group_size, E, K, N, out=None, stream=None):
    torch = _torch()
    if out is None:
        out = new_output((E, K, N), torch.float16, w_packed.device)
    _need(w_packed, torch.uint8, "w_packed")
    _need(scales, torch.float16, "scales")
    _need(out, torch.float16, "w_out", E * K * N)
    _check("moe_dequant", lib().moe_dequant(_ptr(w_packed), _ptr(scales), WTYPES.get(wtype, wtype),
                                            int(group_size), E, K, N, _ptr(out), _stream(stream)))
    return out


# ---------------------------------------------------------------- host helpers
def moe_packed_bytes(wtype, E, K, N):
    return lib().moe_packed_bytes(WTYPES.get(wtype, wtype), E, K, N)


def moe_pack_wq(codes: np.ndarray, wtype) -> np.ndarray:
    """Pack host codes [E, K, N] (int8 codes, or float16 weights for "fp16") -> uint8 array."""
    wt = WTYPES.get(wtype, wtype)
    codes = np.ascontiguousarray(codes)
    if wt == W_FP16:
        if codes.dtype != np.float16:
            raise TypeError("fp16 weights must be float16")
    elif codes.dtype != np.int8:
        raise TypeError("integer codes must be int8")
    E, K, N = codes.shape
    nbytes = lib().moe_packed_bytes(wt, E, K, N)
    if nbytes == 0:
        raise MoEError("moe_pack_wq", MOE_ERR_UNSUPPORTED)
    out = np.empty(nbytes, dtype=np.uint8)
    _check("moe_pack_wq", lib().moe_pack_wq(codes.ctypes.data_as(_P), wt, E, K, N,
                                            out.ctypes.data_as(_P)))
    return out


from .layer import DeviceLayer, Workspace  # noqa: E402,F401

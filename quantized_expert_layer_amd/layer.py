"""A whole MoE expert layer on the device: the C entry points called in order.

DeviceLayer owns the packed expert weights in device memory; forward() enqueues
  moe_route_topk -> moe_permute -> moe_grouped_gemm_wq (gate/up or W1, activation)
  -> moe_grouped_gemm_wq (down or W2, gate weight as row scale)
  [-> shared fp16 experts through the same GEMM entry, E = 1]
  -> moe_unpermute_combine
on one stream, with no host synchronisation.  A step of at most MOE_DECODE_MAX_TOKENS tokens
(decode / verify) instead makes one moe_decode_layer call, or one moe_decode_layer_shared call
for a layer with shared experts (fp16 routed weights: the shared experts on a side stream, and
moe_decode_layer adds their output).  Nothing here computes: torch only allocates.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

import ctypes

from . import (ACTS, GATES, MOE_DECODE_MAX_ROWS, MOE_DECODE_MAX_TOKENS, WTYPES, MoEError, _ptr,
               _stream, lib, moe_decode_layer, moe_decode_layer_shared,
               moe_decode_shared_workspace_size, moe_decode_workspace_size,
               moe_gemm_workspace_size, moe_grouped_gemm_wq, moe_grouped_gemm_wq_rows,
               moe_pack_wq, moe_permute, moe_permute_workspace_size, moe_route_topk,
               moe_unpermute_combine, new_output)


def _dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


@dataclass
class Workspace:
    """Per-(T) device buffers reused across forward() calls."""
    T: int
    bufs: Dict[str, object] = field(default_factory=dict)


class DeviceLayer:
    def __init__(self, *, E: int, k: int, d: int, inter: int, act: str, wtype: str, group: int,
                 gate_mode: str, codes1: np.ndarray, scales1: np.ndarray, codes2: np.ndarray,
                 scales2: np.ndarray, shared: Optional[List[Tuple[np.ndarray, np.ndarray]]] = None,
                 device: str = "cuda", gemm_path: int = 0, gemm_tile: int = 0,
                 fuse_rows: bool = True, decode: Optional[bool] = None, gemm_i2f: int = 0):
        import torch
        self.E, self.k, self.d, self.inter = E, k, d, inter
        self.act, self.wtype, self.group, self.gate_mode = act, wtype, group, gate_mode
        self.n1 = 2 * inter if act == "swiglu" else inter
        self.device = torch.device(device)
        self.gemm_path = gemm_path
        self.gemm_tile = gemm_tile
        # int-to-float conversion of the routed GEMMs (0: exponent-of-1024 construction,
        # 1: conversion instructions, the baseline it is measured against)
        self.gemm_i2f = gemm_i2f
        # fuse_rows: the first GEMM reads x through perm (no x_perm copy), and with k = 1 the
        # second GEMM writes the output rows through perm (no combine launch)
        self.fuse_rows = fuse_rows
        # decode: None = moe_decode_layer for every step it accepts (and default GEMM
        # settings); False = always the five calls; True = require it
        self.decode = decode
        self.w1 = _dev(moe_pack_wq(codes1, wtype), self.device)
        self.w2 = _dev(moe_pack_wq(codes2, wtype), self.device)
        # fp16 experts (wtype "fp16") carry no scales
        self.s1 = None if scales1 is None else _dev(scales1.astype(np.float16), self.device)
        self.s2 = None if scales2 is None else _dev(scales2.astype(np.float16), self.device)
        self.weight_bytes_per_expert = (self.w1.numel() + self.w2.numel()) // E + \
            (0 if scales1 is None else 2 * (scales1[0].size + scales2[0].size))
        self.shared = None
        if shared:
            # n always-on SwiGLU experts summed = one expert whose intermediate columns are
            # concatenated: W1 = [gate_1 .. gate_n | up_1 .. up_n], W2 = [W2_1; ..; W2_n].
            gates = [w1[:, : w1.shape[1] // 2] for w1, _ in shared]
            ups = [w1[:, w1.shape[1] // 2:] for w1, _ in shared]
            sw1 = np.concatenate(gates + ups, axis=1)[None]
            sw2 = np.concatenate([w2 for _, w2 in shared], axis=0)[None]
            self.shared_inter = sw2.shape[1]
            self.shared = (_dev(moe_pack_wq(sw1.astype(np.float16), "fp16"), self.device),
                           _dev(moe_pack_wq(sw2.astype(np.float16), "fp16"), self.device))

    @classmethod
    def from_inputs(cls, inp, device="cuda", gemm_path=0, gemm_tile=0, fuse_rows=True,
                    decode=None, gemm_i2f=0):
        c = inp.cfg
        return cls(E=c.E, k=c.k, d=c.d, inter=c.inter, act=c.act, wtype=inp.wtype,
                   group=c.group, gate_mode=c.gate_mode, codes1=inp.codes1,
                   scales1=inp.scales1, codes2=inp.codes2, scales2=inp.scales2,
                   shared=inp.shared or None, device=device, gemm_path=gemm_path,
                   gemm_tile=gemm_tile, fuse_rows=fuse_rows, decode=decode, gemm_i2f=gemm_i2f)

    def uses_decode(self, T: int, gate_in_gemm: bool = True) -> bool:
        """Whether a step of T tokens runs as one moe_decode_layer call."""
        fits = (0 < T <= MOE_DECODE_MAX_TOKENS and T * self.k <= MOE_DECODE_MAX_ROWS
                and self.d % 128 == 0 and self.inter % 128 == 0)
        if self.decode is True:
            if not fits:
                raise ValueError(f"moe_decode_layer does not take T={T}, k={self.k}")
            return True
        return (self.decode is None and fits and self.gemm_path == 0 and self.gemm_tile == 0
                and self.gemm_i2f == 0 and self.fuse_rows and gate_in_gemm)

    def _scatter_out(self, gate_in_gemm: bool, pruned: bool = False) -> bool:
        """Whether the second GEMM writes the layer output itself: one expert per token, the
        gate weight applied in the GEMM and nothing to add.  Not with batch pruning: a finished
        token has no row in the GEMM, and the combine writes its output row."""
        return (self.fuse_rows and self.k == 1 and gate_in_gemm and self.shared is None
                and not pruned)

    def workspace(self, T: int) -> Workspace:
        import torch
        dev, R, d = self.device, T * self.k, self.d
        n_h = self.inter
        b = {
            "ids": new_output((T, self.k), torch.int32, dev),
            "w": new_output((T, self.k), torch.float32, dev),
            "perm": new_output(R, torch.int32, dev),
            "inv": new_output(R, torch.int32, dev),
            "off": new_output(self.E + 1, torch.int32, dev),
            "xp": new_output((R, d), torch.float16, dev),
            "wp": new_output(R, torch.float32, dev),
            "h": new_output((R, n_h), torch.float16, dev),
            "y": new_output((R, d), torch.float16, dev),
            "out": new_output((T, d), torch.float16, dev),
        }
        ws1 = moe_gemm_workspace_size(R, self.E, d, self.n1, self.wtype, self.act, self.gemm_path)
        ws2 = moe_gemm_workspace_size(R, self.E, self.inter, d, self.wtype, "none", self.gemm_path)
        wsz = max(ws1, ws2)
        if self.shared is not None:
            b["sh_off"] = torch.tensor([0, T], dtype=torch.int32, device=dev)
            b["sh_h"] = new_output((T, self.shared_inter), torch.float16, dev)
            b["sh_y"] = new_output((T, d), torch.float16, dev)
            wsz = max(wsz, moe_gemm_workspace_size(T, 1, d, 2 * self.shared_inter, "fp16",
                                                   "swiglu", self.gemm_path),
                      moe_gemm_workspace_size(T, 1, self.shared_inter, d, "fp16", "none",
                                              self.gemm_path))
        b["ws"] = new_output(max(wsz, 16), torch.uint8, dev)
        b["pws"] = new_output(max(moe_permute_workspace_size(T, self.k, self.E), 16),
                              torch.uint8, dev)
        if self._shared_in_decode():
            dws = moe_decode_shared_workspace_size(T, self.k, self.E, d, self.inter, self.wtype,
                                                   self.shared_inter)
        else:
            dws = moe_decode_workspace_size(T, self.k, self.E, d, self.inter, self.wtype)
        if dws:
            b["dws"] = new_output(dws, torch.uint8, dev)
        return Workspace(T=T, bufs=b)

    def _shared_in_decode(self) -> bool:
        """Whether a decode step computes the shared experts inside its own launches
        (moe_decode_layer_shared: integer-coded routed weights)."""
        return self.shared is not None and self.wtype != "fp16"

    def _side_stream(self):
        """The stream the shared experts of a decode step run on (one per layer)."""
        import torch
        if getattr(self, "_side", None) is None:
            self._side = torch.cuda.Stream(device=self.device)
        return self._side

    def _shared_calls(self, b, x, T, shared=None):
        """(name, C function, args) of the shared experts (fp16, E = 1) into b["sh_y"]."""
        L, st = lib(), None
        sw1, sw2 = shared if shared is not None else self.shared
        return [
            ("shared1", L.moe_grouped_gemm_wq, (_ptr(x), _ptr(b["sh_off"]), T, 1, self.d,
                                                2 * self.shared_inter, _ptr(sw1),
                                                None, 2, 0, 2, None, _ptr(b["sh_h"]), None,
                                                _ptr(b["ws"]), b["ws"].numel(), st)),
            ("shared2", L.moe_grouped_gemm_wq, (_ptr(b["sh_h"]), _ptr(b["sh_off"]), T, 1,
                                                self.shared_inter, self.d,
                                                _ptr(sw2), None, 2, 0, 0, None,
                                                _ptr(b["sh_y"]), None, _ptr(b["ws"]),
                                                b["ws"].numel(), st)),
        ]

    def forward(self, x, logits, ws: Optional[Workspace] = None, gate_in_gemm: bool = True,
                stream=None, active=None):
        """Layer output fp16 [T, d] for x fp16 [T, d] and router logits fp32 [T, E].
        active: uint8 [T] device tensor or None; batch pruning (a token with 0 is finished,
        takes no expert, and its output row is the shared experts' output, or 0)."""
        T = x.shape[0]
        if ws is None or ws.T != T:
            ws = self.workspace(T)
        b = ws.bufs
        path = self.gemm_path
        if self.uses_decode(T, gate_in_gemm):
            if self._shared_in_decode():
                moe_decode_layer_shared(logits, x, self.k, self.gate_mode, self.inter, self.act,
                                        self.w1, self.s1, self.w2, self.s2, self.wtype,
                                        self.group, self.shared[0], self.shared[1],
                                        self.shared_inter, topk_ids=b["ids"], topk_w=b["w"],
                                        out=b["out"], ws=b["dws"], stream=stream,
                                        active=active)
                return b["out"]
            addend, ready = None, None
            if self.shared is not None:
                # the shared experts run on a side stream beside the routed step; the decode
                # call waits for them only before its last launch, which adds their output
                import torch
                main = stream if stream is not None else torch.cuda.current_stream(self.device)
                side, fork, ready = self._side_stream(), torch.cuda.Event(), torch.cuda.Event()
                fork.record(main)
                side.wait_event(fork)
                for name, fn, args in self._shared_calls(b, x, T):
                    st = fn(*(args[:-1] + (_stream(side),)))
                    if st != 0:
                        raise MoEError(name, st)
                ready.record(side)
                addend = b["sh_y"]
            moe_decode_layer(logits, x, self.k, self.gate_mode, self.inter, self.act, self.w1,
                             self.s1, self.w2, self.s2, self.wtype, self.group, addend=addend,
                             topk_ids=b["ids"], topk_w=b["w"], out=b["out"], ws=b["dws"],
                             stream=stream, active=active, addend_ready=ready)
            return b["out"]
        moe_route_topk(logits, self.k, self.gate_mode, b["ids"], b["w"], stream=stream,
                       active=active)
        fused = self.fuse_rows
        scatter = self._scatter_out(gate_in_gemm, active is not None)
        R = T * self.k
        moe_permute(b["ids"], b["w"], x, self.E,
                    out=(b["perm"], b["inv"], b["off"], None if fused else b["xp"], b["wp"]),
                    stream=stream, ws=b["pws"])
        if fused:
            moe_grouped_gemm_wq_rows(x, b["perm"], self.k, b["off"], R, self.E, self.d, self.n1,
                                     self.w1, self.s1, self.wtype, self.group, self.act,
                                     out=b["h"], path=path, stream=stream, tile=self.gemm_tile,
                                     i2f=self.gemm_i2f)
        else:
            moe_grouped_gemm_wq(b["xp"], b["off"], self.E, self.d, self.n1, self.w1, self.s1,
                                self.wtype, self.group, self.act, out=b["h"], path=path,
                                ws=b["ws"], stream=stream, tile=self.gemm_tile, i2f=self.gemm_i2f)
        rs = b["wp"] if gate_in_gemm else None
        if scatter:
            moe_grouped_gemm_wq_rows(b["h"], None, 1, b["off"], R, self.E, self.inter, self.d,
                                     self.w2, self.s2, self.wtype, self.group, "none",
                                     row_scale=rs, out=b["out"], out_rows=b["perm"], path=path,
                                     stream=stream, tile=self.gemm_tile, i2f=self.gemm_i2f)
            return b["out"]
        moe_grouped_gemm_wq(b["h"], b["off"], self.E, self.inter, self.d, self.w2, self.s2,
                            self.wtype, self.group, "none", row_scale=rs, out=b["y"],
                            path=path, ws=b["ws"], stream=stream, tile=self.gemm_tile,
                            i2f=self.gemm_i2f)
        addend = None
        if self.shared is not None:
            moe_grouped_gemm_wq(x, b["sh_off"], 1, self.d, 2 * self.shared_inter,
                                self.shared[0], None, "fp16", 0, "swiglu", out=b["sh_h"],
                                path=path, ws=b["ws"], stream=stream)
            moe_grouped_gemm_wq(b["sh_h"], b["sh_off"], 1, self.shared_inter, self.d,
                                self.shared[1], None, "fp16", 0, "none", out=b["sh_y"],
                                path=path, ws=b["ws"], stream=stream)
            addend = b["sh_y"]
        moe_unpermute_combine(b["y"], b["inv"], None if gate_in_gemm else b["w"], addend, T,
                              self.k, out=b["out"], stream=stream)
        return b["out"]

    # ------------------------------------------------------------------ cached launch plan
    def plan(self, ws: Workspace, x, logits, weights=None, gate_in_gemm: bool = True,
             stream=None, active=None, overlap_shared: bool = False) -> "LayerPlan":
        """Pre-marshal every C call of one forward() for fixed buffers, so that a step is
        just the C calls (no per-call Python argument checks).  `weights` = (w1, w2) or, for a
        layer with shared experts, (w1, w2, shared w1, shared w2): device tensors in the packed
        layout (defaults to this layer's own).  overlap_shared (for a plan captured into a HIP
        graph): the five-call step runs the shared experts on a side stream forked before the
        gating and joined before the combine, so the graph runs them beside the routed
        launches (the fork and join cost host time when the plan runs eagerly)."""
        w1, w2 = weights[:2] if weights is not None else (self.w1, self.w2)
        shw = tuple(weights[2:4]) if weights is not None and len(weights) == 4 else self.shared
        b, L, T = ws.bufs, lib(), ws.T
        st = _stream(stream)
        path = self.gemm_path
        opts = None
        if path or self.gemm_tile or self.gemm_i2f:
            from . import GemmOpts
            opts = GemmOpts()
            opts.path = path
            opts.tile = self.gemm_tile
            opts.i2f = self.gemm_i2f
        ob = ctypes.byref(opts) if opts is not None else None
        wsp, wsn = _ptr(b["ws"]), b["ws"].numel()
        wt, ac = WTYPES[self.wtype], ACTS[self.act]
        fused = self.fuse_rows
        scatter = self._scatter_out(gate_in_gemm, active is not None)
        R = T * self.k
        rs = _ptr(b["wp"]) if gate_in_gemm else None
        keep = (opts, x, logits, w1, w2, self.s1, self.s2, self.shared, shw, ws, active)
        if self.uses_decode(T, gate_in_gemm):
            if self._shared_in_decode():
                calls = [("decode", L.moe_decode_layer_shared,
                          (_ptr(logits), _ptr(active), _ptr(x), T, self.E, self.k,
                           GATES[self.gate_mode], self.d, self.inter, ac, _ptr(w1),
                           _ptr(self.s1), _ptr(w2), _ptr(self.s2), wt, self.group,
                           _ptr(shw[0]), _ptr(shw[1]), self.shared_inter,
                           _ptr(b["ids"]), _ptr(b["w"]), _ptr(b["out"]), _ptr(b["dws"]),
                           b["dws"].numel(), st))]
                return LayerPlan(calls, b["out"], keep=keep)
            calls = []
            addend, ready = None, None
            if self.shared is not None:
                # shared experts on a side stream, joined by the decode call before the launch
                # that adds their output (fork and join are event records and waits, which a
                # captured graph keeps as dependencies)
                import torch
                addend = b["sh_y"]
                main = stream if stream is not None else torch.cuda.current_stream(self.device)
                side = torch.cuda.Stream(device=self.device)
                fork, join = torch.cuda.Event(), torch.cuda.Event()
                join.record(side)                  # creates the event whose handle is passed

                def do_fork():
                    fork.record(main)
                    side.wait_event(fork)
                    return 0

                def do_join():
                    join.record(side)
                    return 0

                ss = _stream(side)
                calls = [("fork", do_fork, ())]
                calls += [(n, fn, args[:-1] + (ss,))
                          for n, fn, args in self._shared_calls(b, x, T, shw)]
                calls.append(("join", do_join, ()))
                ready = join.cuda_event
                keep = keep + (side, fork, join)
            calls.append(("decode", L.moe_decode_layer,
                          (_ptr(logits), _ptr(active), _ptr(x), T, self.E, self.k,
                           GATES[self.gate_mode], self.d, self.inter, ac, _ptr(w1),
                           _ptr(self.s1), _ptr(w2), _ptr(self.s2), wt, self.group, _ptr(addend),
                           ready, _ptr(b["ids"]), _ptr(b["w"]), _ptr(b["out"]), _ptr(b["dws"]),
                           b["dws"].numel(), st)))
            return LayerPlan(calls, b["out"], keep=keep)
        calls = [
            ("route", L.moe_route_topk_active, (_ptr(logits), _ptr(active), T, self.E, self.k,
                                                GATES[self.gate_mode], _ptr(b["ids"]),
                                                _ptr(b["w"]), st)),
            ("permute", L.moe_permute, (_ptr(b["ids"]), _ptr(b["w"]), _ptr(x), T, self.k, self.E,
                                        self.d, _ptr(b["perm"]), _ptr(b["inv"]), _ptr(b["off"]),
                                        None if fused else _ptr(b["xp"]), _ptr(b["wp"]),
                                        _ptr(b["pws"]), b["pws"].numel(), st)),
        ]
        if fused:
            calls.append(("gemm1", L.moe_grouped_gemm_wq_rows,
                          (_ptr(x), T, _ptr(b["perm"]), self.k, _ptr(b["off"]), R, self.E, self.d,
                           self.n1, _ptr(w1), _ptr(self.s1), wt, self.group, ac, None,
                           _ptr(b["h"]), R, None, ob, wsp, wsn, st)))
        else:
            calls.append(("gemm1", L.moe_grouped_gemm_wq,
                          (_ptr(b["xp"]), _ptr(b["off"]), R, self.E, self.d, self.n1, _ptr(w1),
                           _ptr(self.s1), wt, self.group, ac, None, _ptr(b["h"]), ob, wsp, wsn,
                           st)))
        if scatter:
            calls.append(("gemm2", L.moe_grouped_gemm_wq_rows,
                          (_ptr(b["h"]), R, None, 1, _ptr(b["off"]), R, self.E, self.inter, self.d,
                           _ptr(w2), _ptr(self.s2), wt, self.group, 0, rs, _ptr(b["out"]), T,
                           _ptr(b["perm"]), ob, wsp, wsn, st)))
            return LayerPlan(calls, b["out"], keep=keep)
        calls.append(("gemm2", L.moe_grouped_gemm_wq,
                      (_ptr(b["h"]), _ptr(b["off"]), R, self.E, self.inter, self.d, _ptr(w2),
                       _ptr(self.s2), wt, self.group, 0, rs, _ptr(b["y"]), ob, wsp, wsn, st)))
        addend = None
        if self.shared is not None:
            overlap = overlap_shared
            ss = st
            if overlap:
                # the shared experts on a side stream forked before the gating, joined before
                # the combine (event records and waits, which a captured graph keeps as edges)
                import torch
                main = stream if stream is not None else torch.cuda.current_stream(self.device)
                side = torch.cuda.Stream(device=self.device)
                fork, join = torch.cuda.Event(), torch.cuda.Event()

                def do_fork():
                    fork.record(main)
                    side.wait_event(fork)
                    return 0

                def do_join():
                    join.record(side)
                    main.wait_event(join)
                    return 0

                ss = _stream(side)
                keep = keep + (side, fork, join)
            shared_calls = [
                ("shared1", L.moe_grouped_gemm_wq, (_ptr(x), _ptr(b["sh_off"]), T, 1, self.d,
                                                    2 * self.shared_inter, _ptr(shw[0]),
                                                    None, 2, 0, 2, None, _ptr(b["sh_h"]), ob,
                                                    wsp, wsn, ss)),
                ("shared2", L.moe_grouped_gemm_wq, (_ptr(b["sh_h"]), _ptr(b["sh_off"]), T, 1,
                                                    self.shared_inter, self.d,
                                                    _ptr(shw[1]), None, 2, 0, 0, None,
                                                    _ptr(b["sh_y"]), ob, wsp, wsn, ss)),
            ]
            if overlap:
                calls = [("fork", do_fork, ())] + shared_calls + calls + [("join", do_join, ())]
            else:
                calls += shared_calls
            addend = b["sh_y"]
        calls.append(("combine", L.moe_unpermute_combine,
                      (_ptr(b["y"]), _ptr(b["inv"]), None if gate_in_gemm else _ptr(b["w"]),
                       _ptr(addend), T, self.k, self.d, _ptr(b["out"]), st)))
        # the plan holds raw device pointers: keep every tensor they point into alive for as
        # long as the plan exists (the layer itself may be dropped by the caller)
        return LayerPlan(calls, b["out"], keep=keep)


class LayerPlan:
    """The C calls of one layer forward with their arguments fixed."""

    def __init__(self, calls, out, keep):
        self.calls = calls
        self.out = out
        self._keep = keep                     # keeps referenced tensors / opts alive
        self.names = [c[0] for c in calls]

    def run(self, marker=None):
        for i, (name, fn, args) in enumerate(self.calls):
            if marker is not None:
                marker(i)
            st = fn(*args)
            if st != 0:
                raise MoEError(fn.__name__, st)
        if marker is not None:
            marker(len(self.calls))
        return self.out

"""Thin torch-facing binding of the C ABI (same names as the entry points).

PyTorch provides device memory and streams; every step of the layer runs in the
HIP library.  Functions check dtypes, devices and shapes, marshal pointers and
raise MoeError on a non-zero status.  The ``*_into`` forms write into
caller-provided buffers and allocate nothing, for use in timed loops and graphs.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import check, lib

MODE_AUTO, MODE_DECODE, MODE_PREFILL = 0, 1, 2
GROUP = 128


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def expert_layout(d: int, I: int) -> dict:
    lay = _lib.ExpertLayout()
    check("moe_expert_layout_get", lib().moe_expert_layout_get(d, I, ctypes.byref(lay)))
    return {f: getattr(lay, f) for f, _ in _lib.ExpertLayout._fields_}


# ---------------------------------------------------------------- pack

def pack_w4_g128(w: torch.Tensor, gateup_interleave: bool, codes: torch.Tensor, codes_stride: int,
                 scales: torch.Tensor, scales_stride: int, codes_offset: int = 0, scales_offset: int = 0,
                 stream=None):
    """Quantise + pack bf16 w [E, N, K] into codes/scales (uint8 device buffers, byte strides/offsets)."""
    _need(w, torch.bfloat16, "w")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    E, N, K = w.shape
    check("pack_w4_g128", lib().pack_w4_g128(
        _ptr(w), E, N, K, int(bool(gateup_interleave)),
        ctypes.c_void_p(codes.data_ptr() + codes_offset), codes_stride,
        ctypes.c_void_p(scales.data_ptr() + scales_offset), scales_stride, _stream(stream)))


def pack_experts(w13: torch.Tensor, w2: torch.Tensor, bank: Optional[torch.Tensor] = None, stream=None):
    """Quantise + pack experts into a bank of blobs: w13 [E, 2I, d], w2 [E, d, I] (bf16, GPU).

    Returns (bank uint8 [E, blob_bytes], layout dict).  Packing may be split over
    calls by passing slices of the expert axis and the matching bank rows.
    """
    E, twoI, d = w13.shape
    I = twoI // 2
    lay = expert_layout(d, I)
    if bank is None:
        bank = torch.empty((E, lay["blob_bytes"]), dtype=torch.uint8, device=w13.device)
    stride = bank.stride(0)
    pack_w4_g128(w13, True, bank, stride, bank, stride, lay["w13_codes"], lay["w13_scales"], stream)
    pack_w4_g128(w2, False, bank, stride, bank, stride, lay["w2_codes"], lay["w2_scales"], stream)
    return bank, lay


# ---------------------------------------------------------------- route

@dataclass
class RouteOut:
    logits: torch.Tensor   # [T, E] fp32
    ids: torch.Tensor      # [T, k] int32
    weights: torch.Tensor  # [T, k] fp32


def alloc_route(T: int, E: int, k: int, device) -> RouteOut:
    return RouteOut(torch.empty((T, E), dtype=torch.float32, device=device),
                    torch.empty((T, k), dtype=torch.int32, device=device),
                    torch.empty((T, k), dtype=torch.float32, device=device))


def moe_route_into(x, w_router, k, out: RouteOut, renormalize=True, stream=None) -> RouteOut:
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router")
    T, d = x.shape
    E = w_router.shape[0]
    check("moe_route", lib().moe_route(_ptr(x), _ptr(w_router), T, d, E, k, int(bool(renormalize)),
                                       _ptr(out.logits), _ptr(out.ids), _ptr(out.weights), _stream(stream)))
    return out


def moe_route(x, w_router, k, renormalize=True, stream=None) -> RouteOut:
    return moe_route_into(x, w_router, k, alloc_route(x.shape[0], w_router.shape[0], k, x.device),
                          renormalize, stream)


# ---------------------------------------------------------------- align

@dataclass
class AlignOut:
    offsets: torch.Tensor        # [E+1]
    sorted_pairs: torch.Tensor   # [T*k]
    pair_pos: torch.Tensor       # [T*k]
    active: torch.Tensor         # [4 + 4E] work list: U, then {expert, first position, count, 0}
    tile_offsets: Optional[torch.Tensor]  # [E+1] or None
    block_m: int = 0


def alloc_align(T: int, k: int, E: int, device, block_m: int = 0) -> AlignOut:
    i32 = dict(dtype=torch.int32, device=device)
    return AlignOut(torch.empty(E + 1, **i32), torch.empty(max(T * k, 1), **i32), torch.empty(max(T * k, 1), **i32),
                    torch.empty(4 + 4 * E, **i32), torch.empty(E + 1, **i32) if block_m > 0 else None, block_m)


def active_experts(al: AlignOut):
    """Host copy of the active-expert work list: list of (expert, first position, count)."""
    w = al.active.cpu()
    U = int(w[0])
    return [tuple(int(v) for v in w[4 + 4 * u: 7 + 4 * u]) for u in range(U)]


def moe_align_into(ids, E, out: AlignOut, stream=None) -> AlignOut:
    _need(ids, torch.int32, "topk_ids")
    T, k = ids.shape
    check("moe_align", lib().moe_align(_ptr(ids), T, k, E, out.block_m, _ptr(out.offsets), _ptr(out.sorted_pairs),
                                       _ptr(out.pair_pos), _ptr(out.active), _ptr(out.tile_offsets),
                                       _stream(stream)))
    return out


def moe_align(ids, E, block_m=0, stream=None) -> AlignOut:
    T, k = ids.shape
    return moe_align_into(ids, E, alloc_align(T, k, E, ids.device, block_m), stream)


ROUTE_ALIGN_COUNTERS = 256  # MOE_ROUTE_ALIGN_COUNTERS in w4a16_moe.h


def alloc_counter(device) -> torch.Tensor:
    """Zeroed device counters for moe_route_align (each call leaves them zero)."""
    return torch.zeros(ROUTE_ALIGN_COUNTERS, dtype=torch.int32, device=device)


def moe_route_align_into(x, w_router, k, route: RouteOut, al: AlignOut, counter: torch.Tensor, renormalize=True,
                         stream=None):
    """moe_route + moe_align in one launch for T <= 128 (bit-identical outputs)."""
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router")
    _need(counter, torch.int32, "counter")
    if counter.numel() < ROUTE_ALIGN_COUNTERS:
        raise ValueError(f"moe_route_align needs {ROUTE_ALIGN_COUNTERS} counters, got {counter.numel()}")
    T, d = x.shape
    E = w_router.shape[0]
    check("moe_route_align", lib().moe_route_align(
        _ptr(x), _ptr(w_router), T, d, E, k, int(bool(renormalize)), al.block_m, _ptr(route.logits),
        _ptr(route.ids), _ptr(route.weights), _ptr(al.offsets), _ptr(al.sorted_pairs), _ptr(al.pair_pos),
        _ptr(al.active), _ptr(al.tile_offsets), _ptr(counter), _stream(stream)))
    return route, al


# ---------------------------------------------------------------- grouped FFN

def ffn_workspace_bytes(T, d, I, E, k, mode=MODE_AUTO) -> int:
    return int(lib().moe_ffn_workspace_bytes(T, d, I, E, k, mode))


def alloc_workspace(T, d, I, E, k, mode=MODE_AUTO, device="cuda") -> torch.Tensor:
    return torch.empty(max(ffn_workspace_bytes(T, d, I, E, k, mode), 256), dtype=torch.uint8, device=device)


def _ffn_args(x, route: RouteOut, al: AlignOut, bank: torch.Tensor, I: int, out, workspace, mode, combine,
              slot_of_expert, bank_stride):
    _need(x, torch.bfloat16, "x")
    _need(bank, torch.uint8, "bank")
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
    if combine:
        _need(out, torch.bfloat16, "out")
    if slot_of_expert is not None:
        _need(slot_of_expert, torch.int32, "slot_of_expert")
    T, d = x.shape
    E = route.logits.shape[1]
    k = route.ids.shape[1]
    a = _lib.FfnArgs()
    a.x, a.T, a.d, a.I, a.E, a.k = x.data_ptr(), T, d, I, E, k
    a.topk_ids, a.topk_weights = route.ids.data_ptr(), route.weights.data_ptr()
    a.expert_offsets, a.sorted_pairs = al.offsets.data_ptr(), al.sorted_pairs.data_ptr()
    a.pair_pos, a.active_experts = al.pair_pos.data_ptr(), al.active.data_ptr()
    a.tile_offsets = al.tile_offsets.data_ptr() if al.tile_offsets is not None else None
    a.bank = bank.data_ptr()
    a.bank_stride = bank.stride(0) if bank_stride is None else bank_stride
    a.slot_of_expert = slot_of_expert.data_ptr() if slot_of_expert is not None else None
    a.mode, a.combine = mode, int(bool(combine))
    a.out = out.data_ptr() if out is not None else None
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() if workspace is not None else 0
    return a


def moe_w4a16_grouped_ffn_into(x, route: RouteOut, al: AlignOut, bank: torch.Tensor, I: int, out: torch.Tensor,
                               workspace: torch.Tensor, mode=MODE_AUTO, combine=True,
                               slot_of_expert: Optional[torch.Tensor] = None, bank_stride: Optional[int] = None,
                               stream=None):
    if workspace is None:
        raise ValueError("workspace is required (moe_w4a16_grouped_ffn_noalloc_into uses the library's scratch)")
    a = _ffn_args(x, route, al, bank, I, out, workspace, mode, combine, slot_of_expert, bank_stride)
    check("moe_w4a16_grouped_ffn", lib().moe_w4a16_grouped_ffn(ctypes.byref(a), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES in w4a16_moe.h


def moe_w4a16_grouped_ffn_noalloc_into(x, route: RouteOut, al: AlignOut, bank: torch.Tensor, I: int,
                                       out: torch.Tensor, mode=MODE_AUTO, combine=True,
                                       slot_of_expert: Optional[torch.Tensor] = None,
                                       bank_stride: Optional[int] = None, stream=None):
    """moe_w4a16_grouped_ffn with the library's per-GPU scratch as its workspace
    (no workspace argument, no allocation); calls on one GPU must not overlap."""
    a = _ffn_args(x, route, al, bank, I, out, None, mode, combine, slot_of_expert, bank_stride)
    check("moe_w4a16_grouped_ffn_noalloc", lib().moe_w4a16_grouped_ffn_noalloc(ctypes.byref(a), _stream(stream)))
    return out


# ---------------------------------------------------------------- whole decode layer

DECODE_LAYER_COUNTERS = 1024  # MOE_DECODE_LAYER_COUNTERS in w4a16_moe.h


def alloc_layer_counters(device) -> torch.Tensor:
    """Zeroed device counters for moe_decode_layer (each call leaves them zero,
    the last one excepted: a timeout flag)."""
    return torch.zeros(DECODE_LAYER_COUNTERS, dtype=torch.int32, device=device)


def decode_layer_workspace_bytes(T, d, I, E, k) -> int:
    return int(lib().moe_decode_layer_workspace_bytes(T, d, I, E, k))


def _layer_args(x, w_router, bank, I, k, route, out, workspace, counters, renormalize, bank_stride, name):
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router")
    _need(bank, torch.uint8, "bank")
    _need(out, torch.bfloat16, "out")
    _need(workspace, torch.uint8, "workspace")
    _need(counters, torch.int32, "counters")
    if counters.numel() < DECODE_LAYER_COUNTERS:
        raise ValueError(f"{name} needs {DECODE_LAYER_COUNTERS} counters, got {counters.numel()}")
    T, d = x.shape
    E = w_router.shape[0]
    a = _lib.LayerArgs()
    a.x, a.w_router, a.T, a.d, a.I, a.E, a.k = x.data_ptr(), w_router.data_ptr(), T, d, I, E, k
    a.renormalize = int(bool(renormalize))
    a.bank = bank.data_ptr()
    a.bank_stride = bank.stride(0) if bank_stride is None else bank_stride
    a.logits, a.topk_ids, a.topk_weights = route.logits.data_ptr(), route.ids.data_ptr(), route.weights.data_ptr()
    a.out = out.data_ptr()
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    a.counters = counters.data_ptr()
    return a


def moe_decode_layer_into(x, w_router, bank: torch.Tensor, I: int, k: int, route: RouteOut, out: torch.Tensor,
                          workspace: torch.Tensor, counters: torch.Tensor, renormalize=True,
                          bank_stride: Optional[int] = None, stream=None):
    """Router, top-k, grouped gate/up, down and combine of one decode step (T <= 16)
    in two launches; outputs bit-identical to moe_route_align + moe_w4a16_grouped_ffn."""
    a = _layer_args(x, w_router, bank, I, k, route, out, workspace, counters, renormalize, bank_stride,
                    "moe_decode_layer")
    check("moe_decode_layer", lib().moe_decode_layer(ctypes.byref(a), _stream(stream)))
    return out


def moe_mat_decode_layer_into(x, w_router, bank: torch.Tensor, I: int, k: int, route: RouteOut, out: torch.Tensor,
                              workspace: torch.Tensor, counters: torch.Tensor, tau: float, renormalize=True,
                              bank_stride: Optional[int] = None, stream=None):
    """moe_decode_layer_into on nested two/four-bit blobs (layout m1, from mat_from_w4):
    each expert at four bits when the largest routing weight of its pairs reaches tau."""
    a = _layer_args(x, w_router, bank, I, k, route, out, workspace, counters, renormalize, bank_stride,
                    "moe_mat_decode_layer")
    check("moe_mat_decode_layer", lib().moe_mat_decode_layer(ctypes.byref(a), float(tau), _stream(stream)))
    return out


def layer_routing_timed_out(counters: torch.Tensor) -> bool:
    """Whether a moe_decode_layer call on these counters gave up its bounded wait
    for the routing (the last counter; the outputs of that call are invalid).
    Synchronises the device (every stream) before reading the flag."""
    torch.cuda.synchronize(counters.device)
    return bool(int(counters[DECODE_LAYER_COUNTERS - 1].item()))


def moe_decode_layer(x, w_router, bank: torch.Tensor, I: int, k: int, renormalize=True, stream=None):
    """Allocating convenience form of moe_decode_layer_into: returns (out, route).
    It reads the routing-wait flag after the call (a device round trip) and raises
    MoeError if the wait timed out."""
    T, d = x.shape
    E = w_router.shape[0]
    route = alloc_route(T, E, k, x.device)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    ws = torch.empty(max(decode_layer_workspace_bytes(T, d, I, E, k), 256), dtype=torch.uint8, device=x.device)
    ctr = alloc_layer_counters(x.device)
    moe_decode_layer_into(x, w_router, bank, I, k, route, out, ws, ctr, renormalize, stream=stream)
    if layer_routing_timed_out(ctr):
        raise _lib.MoeError("moe_decode_layer", 5, "the bounded wait for the routing timed out; outputs are invalid")
    return out, route


def bf16_expert_bytes(d: int, I: int) -> int:
    return int(lib().moe_bf16_expert_bytes(d, I))


def pack_bf16_experts(w13: torch.Tensor, w2: torch.Tensor, bank: Optional[torch.Tensor] = None, stream=None):
    """BF16 expert bank: w13 [E, 2I, d], w2 [E, d, I] (bf16, GPU) copied into blobs
    (uint8 [E, stride], stride = bf16 blob bytes rounded up to 256)."""
    _need(w13, torch.bfloat16, "w13")
    _need(w2, torch.bfloat16, "w2")
    E, twoI, d = w13.shape
    I = twoI // 2
    stride = (bf16_expert_bytes(d, I) + 255) // 256 * 256
    if bank is None:
        bank = torch.empty((E, stride), dtype=torch.uint8, device=w13.device)
    check("moe_bf16_pack", lib().moe_bf16_pack(_ptr(w13.contiguous()), _ptr(w2.contiguous()), E, d, I, _ptr(bank),
                                               bank.stride(0), _stream(stream)))
    return bank


def moe_bf16_grouped_ffn_into(x, route: RouteOut, al: AlignOut, bank: torch.Tensor, I: int, out: torch.Tensor,
                              workspace: torch.Tensor, combine=True, slot_of_expert: Optional[torch.Tensor] = None,
                              stream=None):
    """The grouped pass over BF16 expert blobs (pack_bf16_experts); workspace sized
    with mode=MODE_DECODE."""
    _need(x, torch.bfloat16, "x")
    _need(bank, torch.uint8, "bank")
    _need(workspace, torch.uint8, "workspace")
    if combine:
        _need(out, torch.bfloat16, "out")
    if slot_of_expert is not None:
        _need(slot_of_expert, torch.int32, "slot_of_expert")
    T, d = x.shape
    a = _lib.FfnArgs()
    a.x, a.T, a.d, a.I, a.E, a.k = x.data_ptr(), T, d, I, route.logits.shape[1], route.ids.shape[1]
    a.topk_ids, a.topk_weights = route.ids.data_ptr(), route.weights.data_ptr()
    a.expert_offsets, a.sorted_pairs = al.offsets.data_ptr(), al.sorted_pairs.data_ptr()
    a.pair_pos, a.active_experts = al.pair_pos.data_ptr(), al.active.data_ptr()
    a.tile_offsets = al.tile_offsets.data_ptr() if al.tile_offsets is not None else None
    a.bank, a.bank_stride = bank.data_ptr(), bank.stride(0)
    a.slot_of_expert = slot_of_expert.data_ptr() if slot_of_expert is not None else None
    a.mode, a.combine = MODE_DECODE, int(bool(combine))
    a.out = out.data_ptr() if out is not None else None
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    check("moe_bf16_grouped_ffn", lib().moe_bf16_grouped_ffn(ctypes.byref(a), _stream(stream)))
    return out


def moe_bf16_grouped_ffn(x, route, al, bank, I, stream=None):
    T, d = x.shape
    E, k = route.logits.shape[1], route.ids.shape[1]
    out = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    ws = alloc_workspace(T, d, I, E, k, MODE_DECODE, x.device)
    return moe_bf16_grouped_ffn_into(x, route, al, bank, I, out, ws, True, stream=stream)


def mat_layout(d: int, I: int) -> dict:
    lay = _lib.MatLayout()
    check("moe_mat_layout_get", lib().moe_mat_layout_get(d, I, ctypes.byref(lay)))
    return {f: getattr(lay, f) for f, _ in _lib.MatLayout._fields_}


def mat_from_w4(w4_bank: torch.Tensor, d: int, I: int, stream=None) -> torch.Tensor:
    """Nested two/four-bit bank (layout m1) from a four-bit bank (pack_experts)."""
    _need(w4_bank, torch.uint8, "w4_bank")
    E = w4_bank.shape[0]
    stride = mat_layout(d, I)["blob_bytes"]
    bank = torch.empty((E, stride), dtype=torch.uint8, device=w4_bank.device)
    check("moe_mat_from_w4", lib().moe_mat_from_w4(_ptr(w4_bank), w4_bank.stride(0), E, d, I, _ptr(bank), stride,
                                                   _stream(stream)))
    return bank


def moe_mat_grouped_ffn_into(x, route: RouteOut, al: AlignOut, bank: torch.Tensor, I: int, out: torch.Tensor,
                             workspace: torch.Tensor, tau: float, combine=True,
                             slot_of_expert: Optional[torch.Tensor] = None, stream=None):
    """The grouped pass over nested two/four-bit blobs (mat_from_w4): an expert runs
    at four bits when its largest routing weight in the step is >= tau, else at two."""
    _need(x, torch.bfloat16, "x")
    _need(bank, torch.uint8, "bank")
    _need(workspace, torch.uint8, "workspace")
    if combine:
        _need(out, torch.bfloat16, "out")
    T, d = x.shape
    a = _lib.FfnArgs()
    a.x, a.T, a.d, a.I, a.E, a.k = x.data_ptr(), T, d, I, route.logits.shape[1], route.ids.shape[1]
    a.topk_ids, a.topk_weights = route.ids.data_ptr(), route.weights.data_ptr()
    a.expert_offsets, a.sorted_pairs = al.offsets.data_ptr(), al.sorted_pairs.data_ptr()
    a.pair_pos, a.active_experts = al.pair_pos.data_ptr(), al.active.data_ptr()
    a.tile_offsets = al.tile_offsets.data_ptr() if al.tile_offsets is not None else None
    a.bank, a.bank_stride = bank.data_ptr(), bank.stride(0)
    a.slot_of_expert = slot_of_expert.data_ptr() if slot_of_expert is not None else None
    a.mode, a.combine = MODE_DECODE, int(bool(combine))
    a.out = out.data_ptr() if out is not None else None
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    check("moe_mat_grouped_ffn", lib().moe_mat_grouped_ffn(ctypes.byref(a), float(tau), _stream(stream)))
    return out


def moe_w4a16_grouped_ffn(x, route, al, bank, I, mode=MODE_AUTO, slot_of_expert=None, stream=None):
    T, d = x.shape
    E, k = route.logits.shape[1], route.ids.shape[1]
    out = torch.empty((T, d), dtype=torch.bfloat16, device=x.device)
    ws = alloc_workspace(T, d, I, E, k, mode, x.device)
    return moe_w4a16_grouped_ffn_into(x, route, al, bank, I, out, ws, mode, True, slot_of_expert, stream=stream)


class MoELayer:
    """One W4A16 MoE layer step with preallocated buffers (no allocation per call).

    forward(x) = moe_route -> moe_align -> moe_w4a16_grouped_ffn on the current stream.
    """

    def __init__(self, w_router: torch.Tensor, bank: torch.Tensor, I: int, k: int, T_max: int,
                 mode=MODE_AUTO, renormalize=True):
        self.w_router, self.bank, self.I, self.k, self.mode = w_router, bank, I, k, mode
        self.renormalize = renormalize
        self.E, self.d = w_router.shape
        dev = w_router.device
        self.T_max = T_max
        self.route = alloc_route(T_max, self.E, k, dev)
        self.align = alloc_align(T_max, k, self.E, dev)
        self.counter = alloc_counter(dev)
        self.out = torch.empty((T_max, self.d), dtype=torch.bfloat16, device=dev)
        need = max(ffn_workspace_bytes(t, self.d, I, self.E, k, mode) for t in range(1, T_max + 1))
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def views(self, T):
        r = RouteOut(self.route.logits[:T], self.route.ids[:T], self.route.weights[:T])
        a = AlignOut(self.align.offsets, self.align.sorted_pairs[:max(T * self.k, 1)],
                     self.align.pair_pos[:max(T * self.k, 1)], self.align.active, None, 0)
        return r, a

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        if T > self.T_max:
            raise ValueError(f"T={T} exceeds T_max={self.T_max}")
        r, a = self.views(T)
        moe_route_align_into(x, self.w_router, self.k, r, a, self.counter, self.renormalize, stream)
        o = self.out[:T] if out is None else out
        ws_need = ffn_workspace_bytes(T, self.d, self.I, self.E, self.k, self.mode)
        moe_w4a16_grouped_ffn_into(x, r, a, self.bank, self.I, o, self.ws[:max(ws_need, 256)], self.mode, True,
                                   stream=stream)
        return o


# ---------------------------------------------------------------- slot cache

class SlotCache:
    """Host LRU bookkeeping for S device slots over a pinned host expert store."""

    def __init__(self, E: int, S: int, blob_bytes: int, host_store: torch.Tensor, device_slots: torch.Tensor):
        _need(host_store, torch.uint8, "host_store", device=False)
        _need(device_slots, torch.uint8, "device_slots")
        if not host_store.is_pinned():
            raise ValueError("host_store must be pinned host memory")
        self.E, self.S, self.blob_bytes = E, S, blob_bytes
        self.host_store, self.device_slots = host_store, device_slots
        h = ctypes.c_void_p()
        check("moe_slot_cache_create", lib().moe_slot_cache_create(E, S, blob_bytes, _ptr(host_store),
                                                                   _ptr(device_slots), ctypes.byref(h)))
        self._h = h
        self.words = (E + 63) // 64

    def close(self):
        if getattr(self, "_h", None):
            lib().moe_slot_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load(self, pending: set, slot_table_dev: torch.Tensor, copy_stream, wait_event, done_event):
        """One round: returns (round experts set, hits, misses)."""
        # torch creates an event's HIP handle on its first record; make sure both exist
        if done_event.cuda_event == 0:
            done_event.record(copy_stream)
        if wait_event is not None and wait_event.cuda_event == 0:
            wait_event.record(torch.cuda.current_stream())
        pm = (ctypes.c_uint64 * self.words)()
        for e in pending:
            pm[e >> 6] |= 1 << (e & 63)
        rm = (ctypes.c_uint64 * self.words)()
        nh, nm = ctypes.c_int32(), ctypes.c_int32()
        check("slot_cache_load", lib().slot_cache_load(
            self._h, pm, rm, _ptr(slot_table_dev), ctypes.byref(nh), ctypes.byref(nm),
            ctypes.c_void_p(copy_stream.cuda_stream),
            ctypes.c_void_p(wait_event.cuda_event) if wait_event is not None else None,
            ctypes.c_void_p(done_event.cuda_event)))
        got = {e for e in range(self.E) if (rm[e >> 6] >> (e & 63)) & 1}
        return got, nh.value, nm.value

    POLICY_LRU, POLICY_COST = 0, 1

    def configure(self, policy: int = 0, decay: float = 0.9, copy_streams: int = 1):
        """Replacement policy (POLICY_LRU / POLICY_COST), usage decay and 1 or 2 copy streams."""
        check("moe_slot_cache_configure", lib().moe_slot_cache_configure(self._h, int(policy), float(decay),
                                                                         int(copy_streams)))

    def _mask(self, experts):
        m = (ctypes.c_uint64 * self.words)()
        for e in experts:
            m[e >> 6] |= 1 << (e & 63)
        return m

    def begin_step(self, needed: set):
        """The needed experts of a new step (usage averages of the cost-aware policy)."""
        check("slot_cache_begin_step", lib().slot_cache_begin_step(self._h, self._mask(needed)))

    def set_prefix(self, prefix_bytes: int):
        """Precision-aware loads: the blobs' first prefix_bytes are their two-bit part."""
        check("moe_slot_cache_set_prefix", lib().moe_slot_cache_set_prefix(self._h, int(prefix_bytes)))

    def load_precision(self, pending: set, full: set, slot_table_dev: torch.Tensor, copy_stream, wait_event,
                       done_event):
        """One round with per-expert precision (full: experts needed at four bits):
        returns (round experts set, hits, misses, bytes copied)."""
        if done_event.cuda_event == 0:
            done_event.record(copy_stream)
        if wait_event is not None and wait_event.cuda_event == 0:
            wait_event.record(torch.cuda.current_stream())
        rm = (ctypes.c_uint64 * self.words)()
        nh, nm, nb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
        check("slot_cache_load_precision", lib().slot_cache_load_precision(
            self._h, self._mask(pending), self._mask(full), rm, _ptr(slot_table_dev), ctypes.byref(nh),
            ctypes.byref(nm), ctypes.byref(nb), ctypes.c_void_p(copy_stream.cuda_stream),
            ctypes.c_void_p(wait_event.cuda_event) if wait_event is not None else None,
            ctypes.c_void_p(done_event.cuda_event)))
        got = {e for e in range(self.E) if (rm[e >> 6] >> (e & 63)) & 1}
        return got, nh.value, nm.value, nb.value

    def planes(self):
        """([S] 1 where the slot holds the whole blob, low-plane completions, bytes copied so far)."""
        sf = (ctypes.c_int32 * self.S)()
        up, nb = ctypes.c_int64(), ctypes.c_int64()
        check("moe_slot_cache_planes", lib().moe_slot_cache_planes(self._h, sf, ctypes.byref(up), ctypes.byref(nb)))
        return list(sf), up.value, nb.value

    def prefetch(self, predicted: set, max_copies: int, copy_stream, wait_event=None) -> int:
        """Copy predicted experts ahead of their round; returns the number of copies."""
        if wait_event is not None and wait_event.cuda_event == 0:
            wait_event.record(torch.cuda.current_stream())
        pm = (ctypes.c_uint64 * self.words)()
        for e in predicted:
            pm[e >> 6] |= 1 << (e & 63)
        n = ctypes.c_int32()
        check("slot_cache_prefetch", lib().slot_cache_prefetch(
            self._h, pm, int(max_copies), ctypes.byref(n), ctypes.c_void_p(copy_stream.cuda_stream),
            ctypes.c_void_p(wait_event.cuda_event) if wait_event is not None else None))
        return n.value

    def state(self):
        se = (ctypes.c_int32 * self.S)()
        h, m = ctypes.c_int64(), ctypes.c_int64()
        check("moe_slot_cache_state", lib().moe_slot_cache_state(self._h, se, ctypes.byref(h), ctypes.byref(m)))
        return list(se), h.value, m.value


# ---------------------------------------------------------------- timing

KERNELS = {"gateup_decode": 0, "down_decode": 1, "gateup_prefill": 2, "down_prefill": 3, "combine": 4,
           "gateup_bf16": 7, "down_bf16": 8, "gateup_mat": 9, "down_mat": 10,
           "route": 5, "align": 6}


def timing_enable(on: bool):
    check("moe_timing_enable", lib().moe_timing_enable(int(on)))


def timing_reset():
    check("moe_timing_reset", lib().moe_timing_reset())


def timing_read(kernel: str):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    check("moe_timing_read", lib().moe_timing_read(KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value

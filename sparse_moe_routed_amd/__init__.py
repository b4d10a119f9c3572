"""Python binding of libmoe.so, the MI355X routed mixture-of-experts layer.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so (include/moe.h).  PyTorch supplies device memory and the current
HIP stream.  There is no fallback: if the library is missing or no GPU is
visible, the compute calls raise.

    import sparse_moe_routed_amd as moe
    router = moe.pack_router(w_r, b)                  # once per router matrix
    ids, gates = moe.route(x, router)                 # top-6 routing
    y = moe.forward(x, ids, gates, experts)           # routed experts
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_PKG, "libmoe.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
WFMT = {"bf16": 0, "fp8": 1, "nvfp4": 2}
Y_BF16, Y_F32 = 0, 1


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class Router(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("up_bs", ctypes.c_void_p), ("down_bs", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class Cache(ctypes.Structure):
    _fields_ = [("n_slots", ctypes.c_int32), ("host", Experts), ("up_s", ctypes.c_void_p),
                ("down_s", ctypes.c_void_p), ("slot_up", ctypes.c_void_p),
                ("slot_down", ctypes.c_void_p), ("slot_up_bs", ctypes.c_void_p),
                ("slot_down_bs", ctypes.c_void_p), ("slot_of", ctypes.c_void_p)]


class CacheStats(ctypes.Structure):
    _fields_ = [("touched", ctypes.c_int32), ("hits", ctypes.c_int32), ("misses", ctypes.c_int32),
                ("bytes_uploaded", ctypes.c_int64)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("counts", "offsets", "sorted_src", "inv", "act", "out_rows", "x_q", "act_q",
                 "scales", "total")]


# symbol name -> (restype, argtypes); must match include/moe.h
_SIGS = {
    "moe_abi_version": (ctypes.c_int32, []),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "moe_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32]),
    "moe_workspace_layout": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(WsLayout)]),
    "moe_router_pack": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    "moe_route_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Dims), ctypes.c_int32]),
    "moe_route": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.POINTER(Router), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_forward": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Experts),
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]),
    "moe_forward_timed": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Experts),
                                           ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]),
    "moe_shared_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Dims), ctypes.c_int32,
                                                    ctypes.c_int32]),
    "moe_shared_forward": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.POINTER(Experts), ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_void_p]),
    "moe_forward_noalloc": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Experts),
                                             ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "moe_cache_state_size": (ctypes.c_size_t, [ctypes.POINTER(Dims), ctypes.c_int32]),
    "moe_cache_init": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.POINTER(Cache), ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]),
    "moe_forward_cached": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Cache),
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.POINTER(CacheStats)]),
    "moe_quantize_experts": (ctypes.c_int32, [ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]),
    "moe_quantize_activation": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                                 ctypes.c_void_p]),
    "moe_prenorm": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]),
    "moe_residual_add": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "moe_residual_prenorm": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
}

_lib = None
ABI_VERSION = 7  # MOE_ABI_VERSION of include/moe.h this binding describes


def lib():
    """Load libmoe.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m sparse_moe_routed_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        l.moe_abi_version.restype = ctypes.c_int32
        if l.moe_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI version {l.moe_abi_version()}, this binding "
                              f"expects {ABI_VERSION}: rebuild with `python -m sparse_moe_routed_amd.build`")
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise MoeError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


@dataclass
class LayerDims:
    hidden: int = 2688
    ffn: int = 1856
    n_experts: int = 128
    top_k: int = 6

    def c(self) -> Dims:
        return Dims(self.hidden, self.ffn, self.n_experts, self.top_k)


@dataclass
class ExpertBank:
    """Device expert bank in one of the three formats (see moe_experts in moe.h)."""
    fmt: str
    up: torch.Tensor
    down: torch.Tensor
    up_bs: Optional[torch.Tensor] = None
    down_bs: Optional[torch.Tensor] = None
    up_s: Optional[torch.Tensor] = None
    down_s: Optional[torch.Tensor] = None

    def c(self) -> Experts:
        return Experts(WFMT[self.fmt], self.up.data_ptr(), self.down.data_ptr(),
                       self.up_bs.data_ptr() if self.up_bs is not None else None,
                       self.down_bs.data_ptr() if self.down_bs is not None else None,
                       self.up_s.data_ptr() if self.up_s is not None else None,
                       self.down_s.data_ptr() if self.down_s is not None else None)


def abi_version() -> int:
    return lib().moe_abi_version()


def workspace_size(dims: LayerDims, fmt: str, max_tokens: int) -> int:
    d = dims.c()
    return int(lib().moe_workspace_size(ctypes.byref(d), WFMT[fmt], int(max_tokens)))


def workspace_layout(dims: LayerDims, fmt: str, T: int) -> dict:
    d = dims.c()
    out = WsLayout()
    _check("moe_workspace_layout", lib().moe_workspace_layout(ctypes.byref(d), WFMT[fmt], int(T),
                                                              ctypes.byref(out)))
    return {n: getattr(out, n) for n, _ in WsLayout._fields_}


def workspace(dims: LayerDims, fmt: str, max_tokens: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(256, workspace_size(dims, fmt, max_tokens)), dtype=torch.uint8, device=device)


@dataclass
class PackedRouter:
    """Router matrix packed by moe_router_pack (bf16 [3, E, H]) and its bias."""
    w_packed: torch.Tensor
    bias: Optional[torch.Tensor] = None


def pack_router(w_r: torch.Tensor, bias: Optional[torch.Tensor] = None,
                dims: LayerDims = LayerDims()) -> PackedRouter:
    """moe_router_pack: fp32 [E, H] -> exact bf16 (hi, mid, lo) split."""
    _dev(w_r, torch.float32, "w_r", (dims.n_experts, dims.hidden))
    if bias is not None:
        _dev(bias, torch.float32, "bias", (dims.n_experts,))
    packed = torch.empty((3, dims.n_experts, dims.hidden), dtype=torch.bfloat16, device=w_r.device)
    d = dims.c()
    _check("moe_router_pack", lib().moe_router_pack(ctypes.byref(d), _ptr(w_r), _ptr(packed), _stream()))
    return PackedRouter(packed, bias)


def route_workspace(dims: LayerDims, max_tokens: int, device="cuda") -> torch.Tensor:
    d = dims.c()
    n = int(lib().moe_route_workspace_size(ctypes.byref(d), int(max_tokens)))
    return torch.empty(max(256, n), dtype=torch.uint8, device=device)


def route(x: torch.Tensor, router: PackedRouter, dims: LayerDims = LayerDims(),
          ids: Optional[torch.Tensor] = None, gates: Optional[torch.Tensor] = None,
          ws: Optional[torch.Tensor] = None):
    """moe_route: ids int32 [T, k], gates fp32 [T, k]."""
    T = x.shape[0]
    _dev(x, torch.bfloat16, "x", (T, dims.hidden))
    _dev(router.w_packed, torch.bfloat16, "w_packed", (3, dims.n_experts, dims.hidden))
    if ids is None:
        ids = torch.empty((T, dims.top_k), dtype=torch.int32, device=x.device)
    if gates is None:
        gates = torch.empty((T, dims.top_k), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = route_workspace(dims, T, x.device)
    _dev(ids, torch.int32, "ids", (T, dims.top_k))
    _dev(gates, torch.float32, "gates", (T, dims.top_k))
    _dev(ws, torch.uint8, "ws")
    d = dims.c()
    r = Router(router.w_packed.data_ptr(),
               router.bias.data_ptr() if router.bias is not None else None)
    _check("moe_route", lib().moe_route(ctypes.byref(d), T, _ptr(x), ctypes.byref(r), _ptr(ids),
                                        _ptr(gates), _ptr(ws), ws.numel(), _stream()))
    return ids, gates


def forward(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, experts: ExpertBank,
            dims: LayerDims = LayerDims(), y_dtype: torch.dtype = torch.float32,
            ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_forward: y [T, H] in fp32 or bf16."""
    T = x.shape[0]
    _dev(x, torch.bfloat16, "x", (T, dims.hidden))
    _dev(ids, torch.int32, "ids", (T, dims.top_k))
    _dev(gates, torch.float32, "gates", (T, dims.top_k))
    if ws is None:
        ws = workspace(dims, experts.fmt, T, x.device)
    _dev(ws, torch.uint8, "ws")
    if y is None:
        y = torch.empty((T, dims.hidden), dtype=y_dtype, device=x.device)
    _dev(y, y_dtype, "y", (T, dims.hidden))
    yd = {torch.float32: Y_F32, torch.bfloat16: Y_BF16}[y_dtype]
    d = dims.c()
    e = experts.c()
    _check("moe_forward", lib().moe_forward(ctypes.byref(d), T, _ptr(x), _ptr(ids), _ptr(gates),
                                            ctypes.byref(e), _ptr(y), yd, _ptr(ws),
                                            ws.numel(), _stream()))
    return y


def shared_dims(hidden: int = 2688, ffn: int = 3712) -> LayerDims:
    """Dims of a shared expert: one expert that every token takes."""
    return LayerDims(hidden, ffn, 1, 1)


def shared_workspace(dims: LayerDims, fmt: str, max_tokens: int, device="cuda") -> torch.Tensor:
    d = dims.c()
    n = int(lib().moe_shared_workspace_size(ctypes.byref(d), WFMT[fmt], int(max_tokens)))
    if n == 0:
        raise ValueError(f"moe_shared_workspace_size: invalid dims {dims} or format {fmt}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def shared_forward(x: torch.Tensor, expert: ExpertBank, dims: LayerDims,
                   y: Optional[torch.Tensor] = None, y_dtype: torch.dtype = torch.float32,
                   accumulate: bool = False, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_shared_forward: the shared expert on every token; with accumulate,
    added to the fp32 y given (the routed output, for the MoE block)."""
    T = x.shape[0]
    _dev(x, torch.bfloat16, "x", (T, dims.hidden))
    if y is None:
        if accumulate:
            raise ValueError("accumulate needs the y to add to")
        y = torch.empty((T, dims.hidden), dtype=y_dtype, device=x.device)
    _dev(y, y_dtype, "y", (T, dims.hidden))
    if ws is None:
        ws = shared_workspace(dims, expert.fmt, T, x.device)
    _dev(ws, torch.uint8, "ws")
    yd = {torch.float32: Y_F32, torch.bfloat16: Y_BF16}[y_dtype]
    d = dims.c()
    e = expert.c()
    _check("moe_shared_forward", lib().moe_shared_forward(
        ctypes.byref(d), T, _ptr(x), ctypes.byref(e), _ptr(y), yd, int(bool(accumulate)),
        _ptr(ws), ws.numel(), _stream()))
    return y


NOALLOC_SCRATCH_BYTES = 8 << 20  # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h


def forward_noalloc(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, experts: ExpertBank,
                    dims: LayerDims = LayerDims(), y_dtype: torch.dtype = torch.float32,
                    y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_forward_noalloc: moe_forward with the library's fixed device
    scratch instead of a workspace (y is allocated here unless passed)."""
    T = x.shape[0]
    _dev(x, torch.bfloat16, "x", (T, dims.hidden))
    _dev(ids, torch.int32, "ids", (T, dims.top_k))
    _dev(gates, torch.float32, "gates", (T, dims.top_k))
    if y is None:
        y = torch.empty((T, dims.hidden), dtype=y_dtype, device=x.device)
    _dev(y, y_dtype, "y", (T, dims.hidden))
    yd = {torch.float32: Y_F32, torch.bfloat16: Y_BF16}[y_dtype]
    d = dims.c()
    e = experts.c()
    _check("moe_forward_noalloc", lib().moe_forward_noalloc(
        ctypes.byref(d), T, _ptr(x), _ptr(ids), _ptr(gates), ctypes.byref(e), _ptr(y), yd,
        _stream()))
    return y


N_STAGES = 6
STAGES = ("permute", "quant_x", "up", "quant_act", "down", "combine")
N_TIMED_EVENTS = N_STAGES + 5


def forward_timed(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, experts: ExpertBank,
                  events, dims: LayerDims = LayerDims(), y_dtype: torch.dtype = torch.float32,
                  ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_forward_timed: like forward, recording the caller's hipEvent_t handles
    (a sequence of N_STAGES + 1 ints) before each stage and after the last;
    N_TIMED_EVENTS handles add the up and down GEMM kernels' own start and end."""
    T = x.shape[0]
    if ws is None:
        ws = workspace(dims, experts.fmt, T, x.device)
    if y is None:
        y = torch.empty((T, dims.hidden), dtype=y_dtype, device=x.device)
    _dev(x, torch.bfloat16, "x", (T, dims.hidden))
    _dev(ids, torch.int32, "ids", (T, dims.top_k))
    _dev(gates, torch.float32, "gates", (T, dims.top_k))
    _dev(ws, torch.uint8, "ws")
    _dev(y, y_dtype, "y", (T, dims.hidden))
    yd = {torch.float32: Y_F32, torch.bfloat16: Y_BF16}[y_dtype]
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e) for e in events])
    d = dims.c()
    e = experts.c()
    _check("moe_forward_timed", lib().moe_forward_timed(
        ctypes.byref(d), T, _ptr(x), _ptr(ids), _ptr(gates), ctypes.byref(e), _ptr(y), yd,
        _ptr(ws), ws.numel(), _stream(), arr, len(events)))
    return y


class ExpertCache:
    """moe_cache: the bank's codes in pinned host memory and n_slots device
    slots that hold the experts batches select (least recently used replaced).
    Per-expert scales stay on the device."""

    def __init__(self, bank: ExpertBank, n_slots: int, dims: LayerDims = LayerDims()):
        dev = bank.up.device

        def host(t):
            if t is None:
                return None
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t)
            return h

        def slots(t):
            return None if t is None else torch.empty((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype,
                                                       device=dev)

        self.fmt, self.n_slots, self.dims = bank.fmt, int(n_slots), dims
        self.host_up, self.host_down = host(bank.up), host(bank.down)
        self.host_up_bs, self.host_down_bs = host(bank.up_bs), host(bank.down_bs)
        self.up_s, self.down_s = bank.up_s, bank.down_s
        self.slot_up, self.slot_down = slots(bank.up), slots(bank.down)
        self.slot_up_bs, self.slot_down_bs = slots(bank.up_bs), slots(bank.down_bs)
        self.slot_of = torch.empty(dims.n_experts, dtype=torch.int32, device=dev)
        d = dims.c()
        self.state_bytes = int(lib().moe_cache_state_size(ctypes.byref(d), self.n_slots))
        if self.state_bytes == 0:
            raise ValueError(f"n_slots {n_slots} outside [top_k, n_experts]")
        self.state = (ctypes.c_uint64 * ((self.state_bytes + 7) // 8))()  # 8-byte aligned
        c = self.c()
        _check("moe_cache_init", lib().moe_cache_init(ctypes.byref(d), ctypes.byref(c), self.state,
                                                      self.state_bytes, _stream()))

    def c(self) -> Cache:
        p = lambda t: t.data_ptr() if t is not None else None
        h = Experts(WFMT[self.fmt], p(self.host_up), p(self.host_down), p(self.host_up_bs),
                    p(self.host_down_bs), None, None)
        return Cache(self.n_slots, h, p(self.up_s), p(self.down_s), p(self.slot_up),
                     p(self.slot_down), p(self.slot_up_bs), p(self.slot_down_bs), p(self.slot_of))


def forward_cached(x: torch.Tensor, ids: torch.Tensor, gates: torch.Tensor, cache: ExpertCache,
                   dims: LayerDims = LayerDims(), y_dtype: torch.dtype = torch.float32,
                   ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None):
    """moe_forward_cached: (y [T, H], stats dict); y equals forward() on the
    bank the cache was built from."""
    T = x.shape[0]
    _dev(x, torch.bfloat16, "x", (T, dims.hidden))
    _dev(ids, torch.int32, "ids", (T, dims.top_k))
    _dev(gates, torch.float32, "gates", (T, dims.top_k))
    if ws is None:
        ws = workspace(dims, cache.fmt, T, x.device)
    _dev(ws, torch.uint8, "ws")
    if y is None:
        y = torch.empty((T, dims.hidden), dtype=y_dtype, device=x.device)
    _dev(y, y_dtype, "y", (T, dims.hidden))
    yd = {torch.float32: Y_F32, torch.bfloat16: Y_BF16}[y_dtype]
    d = dims.c()
    c = cache.c()
    st = CacheStats()
    _check("moe_forward_cached", lib().moe_forward_cached(
        ctypes.byref(d), T, _ptr(x), _ptr(ids), _ptr(gates), ctypes.byref(c), cache.state, _ptr(y),
        yd, _ptr(ws), ws.numel(), _stream(), ctypes.byref(st)))
    return y, {"touched": st.touched, "hits": st.hits, "misses": st.misses,
               "bytes_uploaded": st.bytes_uploaded}


def quantize_experts(up: torch.Tensor, down: torch.Tensor, fmt: str,
                     dims: LayerDims = LayerDims()) -> ExpertBank:
    """moe_quantize_experts: pack a bf16 bank [E,F,H] / [E,H,F] into fp8 or nvfp4."""
    if fmt == "bf16":
        return ExpertBank("bf16", up, down)
    E, F, H = dims.n_experts, dims.ffn, dims.hidden
    _dev(up, torch.bfloat16, "up", (E, F, H))
    _dev(down, torch.bfloat16, "down", (E, H, F))
    dev = up.device
    if fmt == "fp8":
        up_q = torch.empty((E, F, H), dtype=torch.uint8, device=dev)
        # down codes: per-expert byte arrays in the panel layout (moe.h)
        down_q = torch.empty((E, H * F), dtype=torch.uint8, device=dev)
        up_bs = down_bs = None
    elif fmt == "nvfp4":
        # per-expert byte arrays in the panel layout of moe_experts (moe.h)
        up_q = torch.empty((E, F * H // 2), dtype=torch.uint8, device=dev)
        down_q = torch.empty((E, H * F // 2), dtype=torch.uint8, device=dev)
        up_bs = torch.empty((E, F * H // 16), dtype=torch.uint8, device=dev)
        down_bs = torch.empty((E, H * F // 16), dtype=torch.uint8, device=dev)
    else:
        raise ValueError(fmt)
    up_s = torch.empty(E, dtype=torch.float32, device=dev)
    down_s = torch.empty(E, dtype=torch.float32, device=dev)
    d = dims.c()
    _check("moe_quantize_experts", lib().moe_quantize_experts(
        ctypes.byref(d), WFMT[fmt], _ptr(up), _ptr(down), _ptr(up_q), _ptr(down_q),
        _ptr(up_bs), _ptr(down_bs), _ptr(up_s), _ptr(down_s), _stream()))
    return ExpertBank(fmt, up_q, down_q, up_bs, down_bs, up_s, down_s)


def quantize_activation(x: torch.Tensor, fmt: str):
    """moe_quantize_activation: (codes, block scales or None, scale fp32[1])."""
    rows, cols = x.shape
    _dev(x, torch.bfloat16, "x")
    dev = x.device
    if fmt == "fp8":
        codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        bs = None
    elif fmt == "nvfp4":
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        bs = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    else:
        raise ValueError(fmt)
    scale = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    _check("moe_quantize_activation", lib().moe_quantize_activation(
        WFMT[fmt], rows, cols, _ptr(x), _ptr(codes), _ptr(bs), _ptr(scale), _ptr(ws), 256, _stream()))
    return codes, bs, scale


def prenorm(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    T, H = x.shape
    _dev(x, torch.bfloat16, "x")
    if out is None:
        out = torch.empty_like(x)
    _check("moe_prenorm", lib().moe_prenorm(T, H, _ptr(x), _ptr(out), _stream()))
    return out


def residual_add(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    T, H = x.shape
    _dev(x, torch.bfloat16, "x")
    _dev(y, torch.float32, "y", (T, H))
    _check("moe_residual_add", lib().moe_residual_add(T, H, _ptr(x), _ptr(y), _stream()))
    return x


def residual_prenorm(x: torch.Tensor, y: torch.Tensor,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_residual_prenorm: x <- bf16(x + y) in place, returns prenorm(x) in out."""
    T, H = x.shape
    _dev(x, torch.bfloat16, "x")
    _dev(y, torch.float32, "y", (T, H))
    if out is None:
        out = torch.empty_like(x)
    _dev(out, torch.bfloat16, "out", (T, H))
    _check("moe_residual_prenorm",
           lib().moe_residual_prenorm(T, H, _ptr(x), _ptr(y), _ptr(out), _stream()))
    return out

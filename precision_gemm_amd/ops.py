"""Python binding of the C ABI in include/lora_lowp.h, on torch device tensors.

Argument marshalling only: every step of the layer runs in the HIP library.  torch is
used for device memory and for the current HIP stream.  Names follow the C ABI.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass, field

import torch

from ._lib import check, lib

LORA_W_FP8_E4M3 = 0
LORA_W_MXFP4_E2M1 = 1
LORA_FUSE_SHRINK = 1
LORA_BUILD_SEGMENTS = 2
LORA_ACT_BF16 = 4

_FMT = {"fp8": LORA_W_FP8_E4M3, "mxfp4": LORA_W_MXFP4_E2M1}


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    return t


@dataclass
class LowpWeight:
    """Base weight on the device: fmt "fp8" (q uint8 [N,K], scale float32 [N]) or
    "mxfp4" (q uint8 [N,K/2], scale uint8 [N,K/32]).  ``packed`` says whether q (and the
    MXFP4 scales) are in the packed form the GEMM reads (see :func:`pack_weight`); the
    tensors keep their [N, ...] shapes either way."""

    fmt: str
    q: torch.Tensor
    scale: torch.Tensor
    packed: bool = False

    @property
    def N(self) -> int:
        return self.q.shape[0]

    @property
    def K(self) -> int:
        return self.q.shape[1] * (1 if self.fmt == "fp8" else 2)


def pack_weight(w: LowpWeight) -> LowpWeight:
    """Reorder a row-major weight into the packed form (lora_pack_weight), once, offline."""
    if w.packed:
        return w
    _dev(w.q, "q", torch.uint8)
    qp = torch.empty_like(w.q)
    if w.fmt == "mxfp4":
        sp = torch.empty_like(w.scale)
        sc_in, sc_out = _ptr(w.scale), _ptr(sp)
    else:
        sp = w.scale
        sc_in = sc_out = _ptr(None)
    check("lora_pack_weight", lib().lora_pack_weight(_FMT[w.fmt], _ptr(w.q), sc_in, w.N, w.K, _ptr(qp), sc_out,
                                                     _stream()))
    return LowpWeight(w.fmt, qp, sp, packed=True)


@dataclass
class Adapters:
    """A set of LoRA adapters resident on the device.

    ``At[a]`` is A_a^T (bf16 [r_a, K]) and ``Bt[a]`` is B_a^T (bf16 [N, r_a]); the
    pointer tables, ranks and scales are device arrays built once here.
    """

    At: list
    Bt: list
    scales: torch.Tensor            # float32 [n]
    ranks: torch.Tensor = field(init=False)
    A_ptrs: torch.Tensor = field(init=False)
    B_ptrs: torch.Tensor = field(init=False)
    r_max: int = field(init=False)

    def __post_init__(self):
        dev = self.scales.device
        for a, b in zip(self.At, self.Bt):
            _dev(a, "A^T", torch.bfloat16)
            _dev(b, "B^T", torch.bfloat16)
        rk = [int(a.shape[0]) for a in self.At]
        self.ranks = torch.tensor(rk, dtype=torch.int32, device=dev)
        self.r_max = max(rk)
        self.A_ptrs = torch.tensor([a.data_ptr() for a in self.At], dtype=torch.int64, device=dev)
        self.B_ptrs = torch.tensor([b.data_ptr() for b in self.Bt], dtype=torch.int64, device=dev)
        self.scales = self.scales.to(torch.float32).contiguous()

    @property
    def n(self) -> int:
        return len(self.At)


@dataclass
class Segments:
    adapter_id: torch.Tensor   # int32 [T]
    seg_indptr: torch.Tensor   # int32 [n+1]
    sorted_tok: torch.Tensor   # int32 [T]
    err: torch.Tensor          # int32 [1]


def version() -> str:
    return lib().lora_version().decode()


def workspace_bytes(T: int, K: int, N: int, n_adapters: int, r_max: int) -> int:
    return int(lib().lora_workspace_bytes(T, K, N, n_adapters, r_max))


def alloc_workspace(T, K, N, n_adapters, r_max, device="cuda") -> torch.Tensor:
    nbytes = workspace_bytes(T, K, N, n_adapters, r_max)
    if nbytes == 0:
        raise ValueError("sizes outside the library's limits")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    check("lora_workspace_init", lib().lora_workspace_init(_ptr(ws), nbytes, _stream()))
    return ws


def workspace_status(ws: torch.Tensor) -> int:
    out = torch.zeros(1, dtype=torch.int32, device=ws.device)
    check("lora_workspace_status", lib().lora_workspace_status(_ptr(ws), _ptr(out), _stream()))
    return int(out.item())


def workspace_segment_error(ws: torch.Tensor) -> int:
    """Error word of the last segment build inside the layer call on ``ws``."""
    out = torch.zeros(1, dtype=torch.int32, device=ws.device)
    check("lora_workspace_segment_error", lib().lora_workspace_segment_error(_ptr(ws), _ptr(out), _stream()))
    return int(out.item())


def plan_info(T, K, N, n_adapters, r_max, fmt="fp8") -> dict:
    buf = (ctypes.c_int32 * 16)()
    n = lib().lora_plan_info(T, K, N, n_adapters, r_max, _FMT[fmt], buf, 16)
    if n < 0:
        raise ValueError("sizes outside the library's limits")
    keys = ["TT", "CT", "WC", "WK", "XQ", "KC", "ksplit", "krange", "n_cb", "n_tb", "n_gemm_wg",
            "s_tblk", "s_njg", "s_kparts", "n_shrink_wg"]
    return dict(zip(keys, list(buf)[:n]))


def empty_segments(adapter_id: torch.Tensor, n_adapters: int) -> Segments:
    """Buffers for the segments of a batch (filled by build_segments, or by the layer
    call with ``build_segments=True``)."""
    _dev(adapter_id, "adapter_id", torch.int32)
    T = adapter_id.numel()
    dev = adapter_id.device
    return Segments(adapter_id, torch.empty(n_adapters + 1, dtype=torch.int32, device=dev),
                    torch.empty(max(T, 1), dtype=torch.int32, device=dev)[:T],
                    torch.empty(1, dtype=torch.int32, device=dev))


def build_segments(adapter_id: torch.Tensor, n_adapters: int, out: Segments | None = None) -> Segments:
    """Group tokens by adapter; with ``out`` the result goes into its buffers."""
    _dev(adapter_id, "adapter_id", torch.int32)
    T = adapter_id.numel()
    if out is None:
        out = empty_segments(adapter_id, n_adapters)
    check("lora_build_segments", lib().lora_build_segments(_ptr(adapter_id), T, n_adapters, _ptr(out.seg_indptr),
                                                           _ptr(out.sorted_tok), _ptr(out.err), _stream()))
    return out


def quant_act_mxfp8(x: torch.Tensor):
    _dev(x, "x", torch.bfloat16)
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.uint8, device=x.device)
    xsc = torch.empty((T, K // 32), dtype=torch.uint8, device=x.device)
    check("lora_quant_act_mxfp8", lib().lora_quant_act_mxfp8(_ptr(x), T, K, _ptr(xq), _ptr(xsc), _stream()))
    return xq, xsc


def shrink(x: torch.Tensor, seg: Segments, ad: Adapters, ws: torch.Tensor, t: torch.Tensor | None = None):
    _dev(x, "x", torch.bfloat16)
    T, K = x.shape
    if t is None:
        t = torch.empty((T, ad.r_max), dtype=torch.float32, device=x.device)
    check("lora_shrink", lib().lora_shrink(_ptr(x), T, K, _ptr(seg.seg_indptr), _ptr(seg.sorted_tok),
                                           _ptr(ad.A_ptrs), _ptr(ad.ranks), ad.n, ad.r_max, _ptr(t), _ptr(ws),
                                           ws.numel(), _stream()))
    return t


def expand(t: torch.Tensor, seg: Segments, ad: Adapters, y: torch.Tensor) -> torch.Tensor:
    _dev(y, "y", torch.bfloat16)
    T, N = y.shape
    check("lora_expand", lib().lora_expand(_ptr(t), T, N, _ptr(seg.adapter_id), _ptr(ad.B_ptrs), _ptr(ad.ranks),
                                           _ptr(ad.scales), ad.n, ad.r_max, _ptr(y), _stream()))
    return y


def gemm_lowp_lora_epilogue(x: torch.Tensor, w: LowpWeight, seg: Segments | None, ad: Adapters | None,
                            ws: torch.Tensor, *, t: torch.Tensor | None = None, fuse_shrink: bool = True,
                            y: torch.Tensor | None = None, n_adapters: int | None = None,
                            r_max: int | None = None, build_segments: bool = False,
                            act_bf16: bool = False) -> torch.Tensor:
    """The fused layer.  With ``fuse_shrink`` the down-projection runs in the same
    launch (``t``, if given, receives it); otherwise ``t`` is an input and ``t=None``
    computes the base GEMM only.  With ``build_segments`` the same launch also fills
    ``seg`` (from ``seg.adapter_id``; see ``empty_segments``).  With ``act_bf16`` the
    base product reads x in bf16 as it is (16-bit activations)."""
    _dev(x, "x", torch.bfloat16)
    if not w.packed:
        raise ValueError("the GEMM reads W in the packed form: call pack_weight(w) once first")
    T, K = x.shape
    N = w.N
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    n = ad.n if ad is not None else (n_adapters or 1)
    rm = ad.r_max if ad is not None else (r_max or 8)
    flags = ((LORA_FUSE_SHRINK if fuse_shrink else 0) | (LORA_BUILD_SEGMENTS if build_segments else 0)
             | (LORA_ACT_BF16 if act_bf16 else 0))
    g = lambda o, name: _ptr(getattr(o, name)) if o is not None else _ptr(None)  # noqa: E731
    check("gemm_lowp_lora_epilogue", lib().gemm_lowp_lora_epilogue(
        _ptr(x), T, K, N, _FMT[w.fmt], _ptr(w.q), _ptr(w.scale), _ptr(t),
        g(seg, "adapter_id"), g(seg, "seg_indptr"), g(seg, "sorted_tok"),
        g(ad, "A_ptrs"), g(ad, "B_ptrs"), g(ad, "ranks"), g(ad, "scales"), n, rm,
        _ptr(y), flags, _ptr(ws), ws.numel(), _stream()))
    return y

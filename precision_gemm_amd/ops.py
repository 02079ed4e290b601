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


def rank_pad(r: int) -> int:
    """Stored rank of B_a^T for an adapter of rank r: r rounded up to a multiple of 8."""
    return (int(r) + 7) // 8 * 8


def a_rows(r: int) -> int:
    """Rank rows of the packed A_a (whole rank tiles of 16)."""
    return (int(r) + 15) // 16 * 16


def pack_adapter(A: torch.Tensor, B: torch.Tensor):
    """Pack one adapter, A bf16 [K, r] and B bf16 [r, N], into the form the layer reads
    (lora_pack_adapter): returns ``(At, Bt)``: At bf16 [a_rows(r), K] holding A in the
    MFMA operand order of lora_lowp.h, Bt bf16 [N, rank_pad(r)] = B^T with zero padding."""
    _dev(A, "A", torch.bfloat16)
    _dev(B, "B", torch.bfloat16)
    K, r = A.shape
    r2, N = B.shape
    if r2 != r:
        raise ValueError(f"A is [K, {r}] but B is [{r2}, N]")
    rp = rank_pad(r)
    At = torch.empty((a_rows(r), K), dtype=torch.bfloat16, device=A.device)
    Bt = torch.empty((N, rp), dtype=torch.bfloat16, device=A.device)
    check("lora_pack_adapter", lib().lora_pack_adapter(_ptr(A), _ptr(B), K, N, r, _ptr(At), _ptr(Bt), _stream()))
    return At, Bt


@dataclass
class Adapters:
    """A set of LoRA adapters resident on the device.

    ``A[a]`` is bf16 [K, r_a] and ``B[a]`` bf16 [r_a, N] (the layouts of the problem
    statement); they are packed once here by lora_pack_adapter into ``At[a]`` (bf16
    [rank_pad(r_a), K]) and ``Bt[a]`` (bf16 [N, rank_pad(r_a)]), which the kernels read.
    The pointer tables, ranks and scales are device arrays built once here.
    """

    A: list
    B: list
    scales: torch.Tensor            # float32 [n]
    At: list = field(init=False)
    Bt: list = field(init=False)
    ranks: torch.Tensor = field(init=False)
    A_ptrs: torch.Tensor = field(init=False)
    B_ptrs: torch.Tensor = field(init=False)
    r_max: int = field(init=False)

    def __post_init__(self):
        dev = self.scales.device
        packed = [pack_adapter(a, b) for a, b in zip(self.A, self.B)]
        self.At = [p[0] for p in packed]
        self.Bt = [p[1] for p in packed]
        rk = [int(a.shape[1]) for a in self.A]
        self.ranks = torch.tensor(rk, dtype=torch.int32, device=dev)
        self.r_max = max(rk)
        self.A_ptrs = torch.tensor([a.data_ptr() for a in self.At], dtype=torch.int64, device=dev)
        self.B_ptrs = torch.tensor([b.data_ptr() for b in self.Bt], dtype=torch.int64, device=dev)
        self.scales = self.scales.to(torch.float32).contiguous()

    @property
    def n(self) -> int:
        return len(self.A)


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


def shrink(x: torch.Tensor, seg: Segments, ad: Adapters, ws: torch.Tensor | None = None,
           t: torch.Tensor | None = None):
    _dev(x, "x", torch.bfloat16)
    T, K = x.shape
    if t is None:
        t = torch.empty((T, ad.r_max), dtype=torch.float32, device=x.device)
    check("lora_shrink", lib().lora_shrink(_ptr(x), T, K, _ptr(seg.seg_indptr), _ptr(seg.sorted_tok),
                                           _ptr(ad.A_ptrs), _ptr(ad.ranks), ad.n, ad.r_max, _ptr(t), _ptr(ws),
                                           0 if ws is None else ws.numel(), _stream()))
    return t


def shrink_configured(x: torch.Tensor, seg: Segments, ad: Adapters, config, t: torch.Tensor | None = None):
    """The standalone down-projection with an explicit configuration (TG, JP, U, TBLK, ORDER);
    see lora_shrink_configured."""
    _dev(x, "x", torch.bfloat16)
    T, K = x.shape
    if t is None:
        t = torch.empty((T, ad.r_max), dtype=torch.float32, device=x.device)
    cfg = (ctypes.c_int32 * 5)(*[int(v) for v in config])
    check("lora_shrink_configured", lib().lora_shrink_configured(
        _ptr(x), T, K, _ptr(seg.seg_indptr), _ptr(seg.sorted_tok), _ptr(ad.A_ptrs), _ptr(ad.ranks), ad.n, ad.r_max,
        _ptr(t), cfg, _stream()))
    return t


def shrink_config_info(tg: int, jp: int, u: int, nt: int = 1) -> dict:
    """Registers, spill bytes and LDS bytes of a compiled down-projection instance (tg = 0:
    the wave-reduction kernel with nt positions per item)."""
    out = (ctypes.c_int32 * 3)()
    if tg == 0:
        check("lora_shrink_bgmv_info", lib().lora_shrink_bgmv_info(nt, jp, u, out))
    else:
        check("lora_shrink_config_info", lib().lora_shrink_config_info(tg, jp, u, out))
    return {"regs": out[0], "spill": out[1], "lds": out[2]}


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


def gemm_lowp_lora_epilogue_noalloc(x: torch.Tensor, w: LowpWeight, seg: Segments | None, ad: Adapters | None, *,
                                    t: torch.Tensor | None = None, fuse_shrink: bool = True,
                                    y: torch.Tensor | None = None, n_adapters: int | None = None,
                                    r_max: int | None = None, build_segments: bool = False,
                                    act_bf16: bool = False) -> torch.Tensor:
    """:func:`gemm_lowp_lora_epilogue` without a workspace: the library's per-GPU scratch
    array serves instead (gemm_lowp_lora_epilogue_noalloc).  ``y`` (and ``t``) may be
    passed in, so that the call itself allocates nothing."""
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
    check("gemm_lowp_lora_epilogue_noalloc", lib().gemm_lowp_lora_epilogue_noalloc(
        _ptr(x), T, K, N, _FMT[w.fmt], _ptr(w.q), _ptr(w.scale), _ptr(t),
        g(seg, "adapter_id"), g(seg, "seg_indptr"), g(seg, "sorted_tok"),
        g(ad, "A_ptrs"), g(ad, "B_ptrs"), g(ad, "ranks"), g(ad, "scales"), n, rm,
        _ptr(y), flags, _stream()))
    return y


def adapter_rows(ad: Adapters) -> tuple:
    """A_a as bf16 [K, rank_pad(r_a)] row-major per adapter (zero columns past r_a) and the
    device array of their addresses: the A operand of lora_merged_layer.  A layout copy."""
    rows = []
    for a in ad.A:
        K, r = a.shape
        t = torch.zeros((K, rank_pad(r)), dtype=torch.bfloat16, device=a.device)
        t[:, :r].copy_(a)
        rows.append(t)
    ptrs = torch.tensor([t.data_ptr() for t in rows], dtype=torch.int64, device=ad.scales.device)
    return rows, ptrs


def merged_layer(x: torch.Tensor, w_rowmajor: LowpWeight, adapter_id: torch.Tensor, ad: Adapters, a_rows_ptrs,
                 y: torch.Tensor | None = None) -> torch.Tensor:
    """The per-token merged-weight layer (lora_merged_layer): W in its row-major form, A rows
    from :func:`adapter_rows`, B_a^T from the adapter set."""
    _dev(x, "x", torch.bfloat16)
    if w_rowmajor.packed:
        raise ValueError("the merged-weight layer reads W in its row-major form")
    T, K = x.shape
    N = w_rowmajor.N
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    check("lora_merged_layer", lib().lora_merged_layer(
        _ptr(x), T, K, N, _FMT[w_rowmajor.fmt], _ptr(w_rowmajor.q), _ptr(w_rowmajor.scale), _ptr(adapter_id),
        _ptr(a_rows_ptrs), _ptr(ad.B_ptrs), _ptr(ad.ranks), _ptr(ad.scales), ad.n, ad.r_max, _ptr(y), _stream()))
    return y


# ---- backward: the adapters train on the frozen FP8 base (see lora_backward) ----

def pack_weight_t(w: LowpWeight) -> torch.Tensor:
    """W^T in the packed form lora_backward reads (lora_pack_weight_t), from the row-major
    FP8 codes of ``w``; returns uint8 [N*K].  An 8-bit copy made once; the channel scales of
    ``w`` serve as they are."""
    if w.packed:
        raise ValueError("lora_pack_weight_t reads W in its row-major form")
    _dev(w.q, "q", torch.uint8)
    qt = torch.empty(w.N * w.K, dtype=torch.uint8, device=w.q.device)
    check("lora_pack_weight_t", lib().lora_pack_weight_t(_FMT[w.fmt], _ptr(w.q), w.N, w.K, _ptr(qt), _stream()))
    return qt


@dataclass
class BackwardAdapters:
    """The backward forms of an adapter set (lora_pack_adapter_bwd): ``Bop[a]`` bf16
    [a_rows(r_a), N] (B_a in operand order over N) and ``Ar[a]`` bf16 [K, rank_pad(r_a)], and
    the device arrays of their addresses.  Re-pack after the adapters change."""

    Bop: list
    Ar: list
    Bop_ptrs: torch.Tensor
    Ar_ptrs: torch.Tensor


def pack_adapters_bwd(ad: Adapters) -> BackwardAdapters:
    Bop, Ar = [], []
    for A, B in zip(ad.A, ad.B):
        K, r = A.shape
        N = B.shape[1]
        bo = torch.empty((a_rows(r), N), dtype=torch.bfloat16, device=A.device)
        ar = torch.empty((K, rank_pad(r)), dtype=torch.bfloat16, device=A.device)
        check("lora_pack_adapter_bwd", lib().lora_pack_adapter_bwd(_ptr(A), _ptr(B), K, N, r, _ptr(bo), _ptr(ar),
                                                                   _stream()))
        Bop.append(bo)
        Ar.append(ar)
    dev = ad.scales.device
    return BackwardAdapters(Bop, Ar, torch.tensor([b.data_ptr() for b in Bop], dtype=torch.int64, device=dev),
                            torch.tensor([a.data_ptr() for a in Ar], dtype=torch.int64, device=dev))


@dataclass
class Grads:
    """Gradient buffers of an adapter set: ``dA[a]`` float32 [K, r_a], ``dB[a]`` float32
    [r_a, N], and the device arrays of their addresses (built once, so that a call can be
    captured in a HIP graph)."""

    dA: list
    dB: list
    dA_ptrs: torch.Tensor
    dB_ptrs: torch.Tensor


def grads_from(dA: list, dB: list) -> Grads:
    dev = dA[0].device
    for m in dA + dB:
        _dev(m, "gradient buffer", torch.float32)
    return Grads(dA, dB, torch.tensor([m.data_ptr() for m in dA], dtype=torch.int64, device=dev),
                 torch.tensor([m.data_ptr() for m in dB], dtype=torch.int64, device=dev))


def alloc_grads(ad: Adapters, K: int, N: int) -> Grads:
    dev = ad.scales.device
    rk = [int(a.shape[1]) for a in ad.A]
    return grads_from([torch.empty((K, r), dtype=torch.float32, device=dev) for r in rk],
                      [torch.empty((r, N), dtype=torch.float32, device=dev) for r in rk])


def backward_workspace_bytes(T: int, K: int, N: int, n_adapters: int, r_max: int) -> int:
    """Bytes of the workspace lora_backward needs (0: none)."""
    return int(lib().lora_backward_workspace_bytes(T, K, N, n_adapters, r_max))


def lora_backward(x: torch.Tensor, dy: torch.Tensor, t: torch.Tensor, wt: torch.Tensor, w_scale: torch.Tensor,
                  seg: Segments, ad: Adapters, bw: BackwardAdapters, *, dx=None, u=None, grads: Grads | None = None,
                  status: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Gradients of the 16-bit-activation layer (lora_backward): returns ``(dx, u, grads)``
    with dx bf16 [T, K], u float32 [T, r_max] and ``grads`` (:class:`Grads`: dA[a] float32
    [K, r_a], dB[a] float32 [r_a, N]).  ``wt`` from :func:`pack_weight_t`, ``w_scale`` the FP8
    channel scales, ``t`` the forward's down-projection.  Output buffers and the workspace
    (:func:`backward_workspace_bytes` bytes) may be passed in (then the call allocates nothing
    and can be captured in a HIP graph)."""
    _dev(x, "x", torch.bfloat16)
    _dev(dy, "dy", torch.bfloat16)
    T, K = x.shape
    N = dy.shape[1]
    dev = x.device
    if dx is None:
        dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    if u is None:
        u = torch.empty((T, ad.r_max), dtype=torch.float32, device=dev)
    if grads is None:
        grads = alloc_grads(ad, K, N)
    nws = backward_workspace_bytes(T, K, N, ad.n, ad.r_max)
    if workspace is None and nws > 0:
        workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
    check("lora_backward", lib().lora_backward(
        _ptr(x), _ptr(dy), _ptr(t), T, K, N, LORA_W_FP8_E4M3, _ptr(wt), _ptr(w_scale), _ptr(seg.adapter_id),
        _ptr(seg.seg_indptr), _ptr(seg.sorted_tok), _ptr(bw.Bop_ptrs), _ptr(bw.Ar_ptrs), _ptr(ad.ranks),
        _ptr(ad.scales), ad.n, ad.r_max, _ptr(dx), _ptr(u), _ptr(grads.dA_ptrs), _ptr(grads.dB_ptrs), _ptr(status),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(), _stream()))
    return dx, u, grads

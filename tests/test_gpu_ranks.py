"""GPU parity for every adapter rank 1..64 ("Punica" README, Overview: A [H1, r] and
B [r, H2] for any r; ranks differ per adapter), and for the error paths around ranks
and the launch epoch.

* Mixed ranks {1, 4, 12, 20, 60} (and all-small ranks {1, 3, 5}) in one batch, on every
  tile plan the host picks -- the 16-token stream, 64-row tiles, 128-row tiles with their
  register B operands, the prefill plan with 64-token down-projection items -- fused and
  unfused, in both activation forms, against the oracle (y and t).
* lora_pack_adapter writes A^T / B^T with zero padding, byte for byte.
* A rank outside [1, r_max] in device memory: the adapter's term is left out (those
  tokens get the base term) and bit 1 of the workspace status word is set.
* Zero W on the stream, 64-row, 128-row and prefill plans: y is the adapter term alone.
* The launch epoch near the top of its range: parity and a clean status across the wrap,
  on a K-split shape (partial sums handed between workgroups) and a down-projection shape.
"""

import numpy as np
import pytest

import workloads
from gpu_util import assert_t_close, assert_y_close, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MIXED = [1, 4, 12, 20, 60]
SMALL = [1, 3, 5]

PLANS = [
    # T, K, N, fmt: which plan (see lora_plan_info)
    (16, 1024, 512, "fp8"),      # 16-token stream, K-parts of t
    (11, 640, 192, "mxfp4"),     # stream, MXFP4, ragged T
    (48, 1024, 512, "fp8"),      # 64-row tiles, pre-quantised x
    (40, 1024, 320, "mxfp4"),    # 64-row tiles, 64-channel columns, x quantised in the loader
    (100, 2048, 512, "fp8"),     # 128-row tiles, register B operands, K-split
    (128, 4096, 256, "mxfp4"),   # 128-row tiles, K-split
    (300, 1024, 512, "fp8"),     # prefill plan: 128 x 256 tiles, 64-token down-projection items
    (1000, 512, 8192, "fp8"),    # 128 x 512 eight-wave tiles (k_gemm_pf), a 104-row last row block
    (200, 768, 384, "mxfp4"),    # 64-token tiles, two workgroups per CU
]


def _wl(T, K, N, fmt, ranks, seed, **kw):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, len(ranks), T)
    ids[: len(ranks)] = np.arange(len(ranks))[: T]          # every adapter present where T allows
    ids = rng.permutation(ids)
    scale = kw.pop("scale", [1.5 + 0.25 * i for i in range(len(ranks))])
    return workloads.make_custom(T, K, N, fmt, ranks, ids, scale, seed, a_std=kw.pop("a_std", 0.1),
                                 b_std=kw.pop("b_std", 0.05), **kw)


@pytest.mark.parametrize("plan", PLANS, ids=[f"T{p[0]}_K{p[1]}_N{p[2]}_{p[3]}" for p in PLANS])
@pytest.mark.parametrize("ranks", [MIXED, SMALL], ids=["r1-4-12-20-60", "r1-3-5"])
@pytest.mark.parametrize("mode", ["fused", "unfused", "fused_bf16"])
def test_any_rank_matches_oracle(plan, ranks, mode):
    T, K, N, fmt = plan
    print(f"[case] ranks {ranks} plan {plan} {mode}", flush=True)
    wl = _wl(T, K, N, fmt, ranks, 100 + T + len(ranks))
    act = "bf16" if mode.endswith("bf16") else "mxfp8"
    g = run_gpu(wl, fused=mode != "unfused", act_bf16=act == "bf16")
    assert g["status"] == 0
    ref = run_oracle(wl, act=act)
    m, f = assert_y_close(g["y"], ref["y"], f"{plan} {ranks} {mode}")
    tf = assert_t_close(g["t"].astype(np.float64), ref["t"], f"{plan} {ranks} {mode}")
    # the adapter term itself (the base dominates y): y - y_base against the oracle's y_lora
    d = g["y"] - ref["y_base"]
    lora_err = np.linalg.norm(d - ref["y_lora"]) / np.linalg.norm(ref["y_lora"])
    assert lora_err < 0.05, lora_err
    print(f"  y max_rel={m:.2e} frob={f:.2e} t frob={tf:.2e} lora term rel={lora_err:.2e}", flush=True)


@pytest.mark.parametrize("T", [16, 100, 300], ids=["stream", "rows128", "prefill"])
def test_any_rank_segments_built_in_launch(T):
    print(f"[case] ranks {MIXED} T={T} segments in the launch", flush=True)
    wl = _wl(T, 1024, 512, "fp8", MIXED, 300 + T)
    g = run_gpu(wl, fused=True, build=True)
    assert g["status"] == 0 and g["err"] == 0
    ref = run_oracle(wl)
    assert np.array_equal(g["seg_indptr"], ref["seg_indptr"]) and np.array_equal(g["sorted_tok"], ref["sorted_tok"])
    assert_y_close(g["y"], ref["y"], f"T={T}")
    assert_t_close(g["t"].astype(np.float64), ref["t"], f"T={T}")


def test_pack_adapter_layout():
    """lora_pack_adapter against its definition in lora_lowp.h, padding included: A in
    operand order (rank tile jt, k-step ks, half h, lane l = 16 g + i, element e holds
    A[64 ks + 16 g + 8 h + e][16 jt + i]), B as B^T with zero columns past r."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import bf16_tensor
    rng = np.random.default_rng(8)
    for K, N, r in [(256, 128, 1), (512, 192, 12), (128, 64, 60), (384, 320, 64), (256, 64, 8), (192, 64, 17)]:
        A = rng.integers(0, 1 << 16, (K, r), dtype=np.uint16)
        B = rng.integers(0, 1 << 16, (r, N), dtype=np.uint16)
        At, Bt = P.pack_adapter(bf16_tensor(A), bf16_tensor(B))
        torch.cuda.synchronize()
        rp, ra = P.rank_pad(r), P.a_rows(r)
        at = At.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        bt = Bt.view(torch.int16).cpu().numpy().view(np.uint16)
        assert at.size == ra * K and bt.shape == (N, rp)
        Apad = np.zeros((K, ra), np.uint16)
        Apad[:, :r] = A
        # [jt][ks][h][g][i][e] <- A[64 ks + 16 g + 8 h + e][16 jt + i]
        ref = Apad.reshape(K // 64, 4, 2, 8, ra // 16, 16).transpose(4, 0, 2, 1, 5, 3).reshape(-1)
        assert np.array_equal(at, ref)
        assert np.array_equal(bt[:, :r], B.T) and not bt[:, r:].any()


@pytest.mark.parametrize("bad", [0, 61, -5], ids=["rank0", "rank_above_rmax", "negative"])
@pytest.mark.parametrize("shape", [(16, 1024, 512), (100, 1024, 512), (300, 1024, 512), (1000, 512, 8192)],
                         ids=["stream", "rows128", "prefill", "tiles128x512"])
@pytest.mark.parametrize("act", ["mxfp8", "bf16"])
def test_rank_outside_limits_is_reported(bad, shape, act):
    """An adapter whose rank (in device memory) is outside [1, r_max]: its tokens get the
    base term only, the other tokens are unaffected, and the status word says so (at 300
    tokens: the pre-pass down-projection, then the 128 x 256 or, with 16-bit activations,
    the 64 x 256 tiles)."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    from gpu_util import bf16_to_f64
    T, K, N = shape
    print(f"[case] bad rank {bad} shape={shape} act={act}", flush=True)
    wl = _wl(T, K, N, "fp8", MIXED, 400 + T)
    x, w, ad, ids = upload(wl)
    ad.ranks[2] = bad                                         # adapter 2 (rank 12) made invalid
    ws = P.alloc_workspace(wl.T, wl.K, wl.N, ad.n, ad.r_max)
    seg = P.build_segments(ids, ad.n)
    y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, fuse_shrink=True, act_bf16=(act == "bf16"))
    torch.cuda.synchronize()
    assert P.workspace_status(ws) == 2
    ref = run_oracle(wl, act=act)
    yg = bf16_to_f64(y)
    on2 = np.flatnonzero(wl.ids == 2)
    rest = np.flatnonzero(wl.ids != 2)
    assert on2.size > 0 and rest.size > 0
    assert_y_close(yg[rest], ref["y"][rest], "other adapters")
    assert_y_close(yg[on2], ref["y_base"][on2], "invalid rank: base term only")


@pytest.mark.parametrize("plan", [(16, 2048, 512, "fp8"), (48, 1024, 512, "fp8"), (100, 2048, 512, "mxfp4"),
                                  (300, 1024, 512, "fp8"), (1000, 512, 8192, "fp8")],
                         ids=["stream", "rows64", "rows128_ksplit", "prefill", "tiles128x512"])
def test_zero_w_gives_the_adapter_term(plan):
    """With W = 0 the output is bf16(s_a t B_a) alone: the epilogue's adapter term on its own,
    on every plan (the base term cannot hide an error in it)."""
    T, K, N, fmt = plan
    print(f"[case] zero W {plan}", flush=True)
    wl = _wl(T, K, N, fmt, [16, 64, 8, 32], 500 + T, zero_w=True)
    ref = run_oracle(wl)
    assert not ref["y_base"].any()
    for fused in (True, False):
        for a16 in (False, True):  # the adapter term does not depend on the activation form
            g = run_gpu(wl, fused=fused, act_bf16=a16)
            assert g["status"] == 0
            assert_y_close(g["y"], ref["y_lora"], f"zero W {plan} fused={fused} act_bf16={a16}")


@pytest.mark.parametrize("start", [0x7FFFFFFF - 2, 0x3FFFFFFF - 1], ids=["int_max-2", "mask_top-1"])
def test_epoch_wrap(start):
    """Workspace epoch set near the top of its range from the host; several fused calls in
    a row (a K-split shape and a many-adapter down-projection shape) must stay correct and
    leave a clean status while the epoch wraps to 0."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    from gpu_util import bf16_to_f64
    print(f"[case] epoch wrap from {start:#x}", flush=True)
    for T, K, N, fmt, ranks in [(100, 4096, 512, "mxfp4", [16, 64, 8]), (64, 2048, 512, "fp8", [16] * 8),
                                (16, 2048, 256, "fp8", [4, 20])]:
        wl = _wl(T, K, N, fmt, ranks, 600 + T)
        p = P.plan_info(T, K, N, len(ranks), max(ranks), fmt)
        x, w, ad, ids = upload(wl)
        ws = P.alloc_workspace(T, K, N, ad.n, ad.r_max)
        ws[:4].view(torch.int32)[0] = start
        seg = P.build_segments(ids, ad.n)
        ref = run_oracle(wl)
        epochs = []
        for i in range(5):
            y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, fuse_shrink=True, build_segments=(i % 2 == 0))
            torch.cuda.synchronize()
            epochs.append(int(ws[:4].view(torch.int32)[0].item()))
            assert P.workspace_status(ws) == 0, (T, i)
            assert_y_close(bf16_to_f64(y), ref["y"], f"T={T} call {i}")
        assert all(0 <= e < (1 << 30) for e in epochs), epochs
        assert 0 in epochs or start < (1 << 30) - 8, epochs
        print(f"  T={T} ksplit={p['ksplit']} epochs {epochs}", flush=True)

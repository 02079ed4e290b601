"""The allocation-free layer call (gemm_lowp_lora_epilogue_noalloc) through the C ABI
against the workspace call (gemm_lowp_lora_epilogue) on the same inputs: bitwise equal
y and t, and the oracle's bounds, on several calls in a row whose sizes shrink and grow
again (each change of layout re-clears the scratch array's hand-over tags)."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_y_close, bf16_to_f64, run_oracle

pytestmark = pytest.mark.gpu

CALLS = [
    # T, K, N, fmt, ranks, flags: (build segments in the call, 16-bit activations)
    (1000, 512, 8192, "fp8", [16, 64, 4, 12], (True, False)),    # 128 x 512 tiles, x in operand order in the scratch
    (300, 1024, 512, "fp8", [16, 64, 4, 12], (True, False)),     # prefill plan, pre-pass in the scratch
    (16, 2048, 256, "fp8", [1, 20, 60], (True, False)),          # smaller: the one-tile stream
    (100, 4096, 512, "mxfp4", [8, 16, 64], (False, False)),      # larger again: K-split partials
    (100, 4096, 512, "mxfp4", [8, 16, 64], (False, False)),      # same layout twice (no re-clear)
    (200, 512, 512, "fp8", [8, 32], (True, True)),               # 16-bit activations, t in the scratch
    (48, 1024, 512, "fp8", [16] * 6, (True, True)),              # 16-bit activations, smaller
]


def test_noalloc_matches_the_workspace_call():
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    for i, (T, K, N, fmt, ranks, (build, a16)) in enumerate(CALLS):
        print(f"[case] noalloc call {i}: T={T} K={K} N={N} {fmt} ranks={ranks} build={build} a16={a16}", flush=True)
        rng = np.random.default_rng(700 + i)
        ids = rng.integers(0, len(ranks), T)
        wl = workloads.make_custom(T, K, N, fmt, ranks, ids, [1.0 + 0.5 * a for a in range(len(ranks))], 700 + i,
                                   a_std=0.1, b_std=0.05)
        x, w, ad, idt = upload(wl)
        ws = P.alloc_workspace(T, K, N, ad.n, ad.r_max)
        seg_w = P.empty_segments(idt, ad.n) if build else P.build_segments(idt, ad.n)
        seg_n = P.empty_segments(idt, ad.n) if build else seg_w
        t_w = torch.zeros((T, ad.r_max), dtype=torch.float32, device="cuda")
        t_n = torch.full((T, ad.r_max), -1.0, dtype=torch.float32, device="cuda")
        y_n = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        y_w = P.gemm_lowp_lora_epilogue(x, w, seg_w, ad, ws, t=t_w, fuse_shrink=True, build_segments=build,
                                        act_bf16=a16)
        P.gemm_lowp_lora_epilogue_noalloc(x, w, seg_n, ad, t=t_n, y=y_n, fuse_shrink=True, build_segments=build,
                                          act_bf16=a16)
        torch.cuda.synchronize()
        assert P.workspace_status(ws) == 0
        assert torch.equal(y_n.view(torch.int16), y_w.view(torch.int16)), f"call {i}: y differs"
        assert torch.equal(t_n, t_w), f"call {i}: t differs"
        if build:
            assert torch.equal(seg_n.seg_indptr, seg_w.seg_indptr) and torch.equal(seg_n.sorted_tok, seg_w.sorted_tok)
        ref = run_oracle(wl, act="bf16" if a16 else "mxfp8")
        assert_y_close(bf16_to_f64(y_n), ref["y"], f"noalloc call {i}")

"""Long-batch calls captured in a HIP graph and replayed: the fused layer call past 128
tokens (MXFP8: the pre-pass with the down-projection, then the GEMM launch, on 128 x 256
and on 128 x 512 tiles; 16-bit
activations: the rows down-projection, then the 64 x 256-tile GEMM), with t left in the
workspace and the segments built by the call, and one lora_backward call with every output
buffer passed in.  Each graph is replayed three times with eager work and synchronisations
in between (the outputs and the segment buffers overwritten with junk before each replay);
every replay must equal the eager call bit for bit, rebuild the segments exactly and leave
a clean status."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_y_close, bf16_to_f64, run_oracle

pytestmark = pytest.mark.gpu

RANKS = [8, 64, 24, 1, 16]


@pytest.mark.parametrize("shape,act_bf16", [((300, 1024, 512), False), ((300, 1024, 512), True),
                                            ((1000, 512, 8192), False)],
                         ids=["mxfp8", "bf16", "mxfp8_tiles128x512"])
def test_long_batch_layer_call_in_graph(shape, act_bf16):
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    from oracle.segments import build_segments as oracle_segments
    T, K, N = shape
    print(f"[case] graph replay, layer call T={T} K={K} N={N} act_bf16={act_bf16}", flush=True)
    ids = np.random.default_rng(90).integers(0, len(RANKS), T)
    wl = workloads.make_custom(T, K, N, "fp8", RANKS, ids, [1.5] * len(RANKS), 91, a_std=0.1, b_std=0.05)
    x, w, ad, ids_d = upload(wl)
    ws = P.alloc_workspace(T, K, N, ad.n, ad.r_max)
    seg = P.empty_segments(ids_d, ad.n)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")

    def call():
        P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, t=None, y=y, fuse_shrink=True, build_segments=True,
                                  act_bf16=act_bf16)

    call()
    torch.cuda.synchronize()
    eager = y.view(torch.int16).clone()
    assert P.workspace_status(ws) == 0 and P.workspace_segment_error(ws) == 0
    ref = run_oracle(wl, act="bf16" if act_bf16 else "mxfp8")
    assert_y_close(bf16_to_f64(y), ref["y"], "eager")
    seg_ref, srt_ref = oracle_segments(ids, ad.n)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        y.fill_(0.0)                   # eager work between the replays
        seg.seg_indptr.fill_(-7)
        seg.sorted_tok.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager), f"replay {rep}"
        assert P.workspace_status(ws) == 0
        assert np.array_equal(seg.seg_indptr.cpu().numpy(), seg_ref)
        assert np.array_equal(seg.sorted_tok.cpu().numpy(), srt_ref)


def test_backward_call_in_graph():
    import torch
    import precision_gemm_amd as P
    from workloads.device import bf16_tensor, upload
    T, K, N = 300, 512, 512
    print(f"[case] graph replay, backward T={T} K={K} N={N}", flush=True)
    ids = np.random.default_rng(92).integers(0, len(RANKS), T).astype(np.int32)
    wl = workloads.make_custom(T, K, N, "fp8", RANKS, ids, [2.0] * len(RANKS), 93, a_std=1.0 / 16, b_std=0.05)
    dy = bf16_tensor(workloads.grad_output(T, N, 94))
    x, w, ad, ids_d = upload(wl)
    q = torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda()
    sc = torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda()
    wt = P.pack_weight_t(P.LowpWeight("fp8", q, sc))
    bw = P.pack_adapters_bwd(ad)
    seg = P.build_segments(ids_d, ad.n)
    t = P.shrink(x, seg, ad)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    u = torch.empty((T, ad.r_max), dtype=torch.float32, device="cuda")
    dA = [torch.empty((K, r), device="cuda") for r in RANKS]
    dB = [torch.empty((r, N), device="cuda") for r in RANKS]
    grads = P.grads_from(dA, dB)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        P.lora_backward(x, dy, t, wt, sc, seg, ad, bw, dx=dx, u=u, grads=grads, status=st)

    call()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    eager = [dx.view(torch.int16).clone(), u.clone()] + [m.clone() for m in dA + dB]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        dx.fill_(0.0)                  # eager work between the replays
        u.fill_(float("nan"))
        for m in dA + dB:
            m.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [dx.view(torch.int16), u] + dA + dB
        for k, (a, b) in enumerate(zip(got, eager)):
            assert torch.equal(a, b), f"replay {rep}, output {k}"
        assert int(st.item()) == 0

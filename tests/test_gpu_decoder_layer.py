"""The four LoRA projections of one decoder layer (Llama-3-8B shapes, 8 adapters of mixed
ranks shared by all projections) as a caller chains them: the first call builds the
batch's segments in its own launch, the other three read them.  The chain is captured in
one HIP graph and replayed three times with eager work and synchronisations in between
(the segment buffers are overwritten with junk before each replay); every replay must
equal the eager chain bit for bit and rebuild the segments exactly, and the eager chain
must match the oracle per projection (both activation forms).  At 16 tokens the
down-projection takes its rows by adapter id; at 64 tokens it reads the segments built
by the first call, so the chain's hand-over of the segments is exercised."""

import numpy as np
import pytest

import workloads
from gpu_util import assert_t_close, assert_y_close, bf16_to_f64, run_oracle

pytestmark = pytest.mark.gpu

PROJ = [  # name, K, N, W format
    ("qkv", 4096, 6144, "fp8"),
    ("o", 4096, 4096, "fp8"),
    ("gate_up", 4096, 28672, "fp8"),
    ("down", 14336, 4096, "mxfp4"),
]
RANKS = [8, 16, 16, 32, 64, 8, 16, 32]


@pytest.mark.parametrize("T", [16, 64])
@pytest.mark.parametrize("act_bf16", [False, True], ids=["mxfp8", "bf16"])
def test_decoder_layer_chain_in_one_graph(act_bf16, T):
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    from oracle.segments import build_segments as oracle_segments
    print(f"[case] decoder layer chain act_bf16={act_bf16} T={T}", flush=True)
    ids = np.random.default_rng(60).integers(0, len(RANKS), T)
    wls, dev = [], []
    for i, (name, K, N, fmt) in enumerate(PROJ):
        wl = workloads.make_custom(T, K, N, fmt, RANKS, ids, [1.0 + 0.25 * a for a in range(len(RANKS))], 61 + i,
                                   name=name, b_std=0.02)
        x, w, ad, idt = upload(wl)
        ws = P.alloc_workspace(T, K, N, ad.n, ad.r_max)
        t = torch.empty((T, ad.r_max), dtype=torch.float32, device="cuda")
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        wls.append(wl)
        dev.append(dict(x=x, w=w, ad=ad, ws=ws, t=t, y=y))
    ids_d = torch.from_numpy(np.asarray(ids, np.int32)).cuda()
    seg = P.empty_segments(ids_d, len(RANKS))
    seg_ref, srt_ref = oracle_segments(ids, len(RANKS))

    def chain():
        for i, d in enumerate(dev):
            P.gemm_lowp_lora_epilogue(d["x"], d["w"], seg, d["ad"], d["ws"], t=d["t"], y=d["y"], fuse_shrink=True,
                                      build_segments=(i == 0), act_bf16=act_bf16)

    chain()
    torch.cuda.synchronize()
    eager = [d["y"].view(torch.int16).clone() for d in dev]
    act = "bf16" if act_bf16 else "mxfp8"
    for wl, d in zip(wls, dev):
        ref = run_oracle(wl, act=act)
        m, f = assert_y_close(bf16_to_f64(d["y"]), ref["y"], wl.name)
        assert_t_close(d["t"].cpu().numpy().astype(np.float64), ref["t"], wl.name)
        print(f"  {wl.name}: y max_rel={m:.2e} frob={f:.2e}", flush=True)
    assert P.workspace_segment_error(dev[0]["ws"]) == 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for rep in range(3):
        for d in dev:
            d["y"].fill_(0.0)          # eager work between the replays
        seg.seg_indptr.fill_(-7)
        seg.sorted_tok.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, d in enumerate(dev):
            assert torch.equal(d["y"].view(torch.int16), eager[i]), f"replay {rep}, projection {PROJ[i][0]}"
        assert all(P.workspace_status(d["ws"]) == 0 for d in dev)
        assert np.array_equal(seg.seg_indptr.cpu().numpy(), seg_ref)
        assert np.array_equal(seg.sorted_tok.cpu().numpy(), srt_ref)

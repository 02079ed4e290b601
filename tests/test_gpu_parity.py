"""GPU parity: the HIP path through the C ABI against the oracle.

Bars: segment metadata and MXFP8 codes bit-exact; t within 1e-4 relative Frobenius;
y within max|y - y_ref| <= 1e-2 max|y_ref| and relative Frobenius <= 5e-3.
Cases: the five named workloads at full size (fused and unfused schedules), ragged
and tiny shapes, long batches of many tiles (ragged, N / 256 odd, every schedule), mixed ranks, empty adapters, zero B / zero W, a LoRA-heavy input,
bad adapter ids, bitwise determinism."""

import numpy as np
import pytest

import workloads
from gpu_util import (assert_t_close, assert_y_close, errors, named, named_oracle, run_gpu, run_oracle,
                      sample_rows)
from oracle.mxquant import quantize_mxfp8
from oracle.segments import build_segments as oracle_segments

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "decode_qkv", "decode_gateup", "prefill", "downproj_fp4"]


def _rows_for(name):
    if name == "prefill":  # oracle on 192 random rows plus the first and last row of every segment
        return sample_rows(named(name), 192, 7)
    return None


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_layer_matches_oracle(name, fused):
    print(f"[case] layer {name} fused={fused}", flush=True)
    wl = named(name)
    rows = _rows_for(name)
    ref = named_oracle(name, rows)
    g = run_gpu(wl, fused=fused)
    assert g["status"] == 0 and g["err"] == 0
    seg_ref, srt_ref = oracle_segments(wl.ids, wl.n_adapters)
    assert np.array_equal(g["seg_indptr"], seg_ref) and np.array_equal(g["sorted_tok"], srt_ref)
    sel = slice(None) if rows is None else np.asarray(rows)
    if rows is not None:  # the sample holds both ends of every segment (adapter 0's rows 0 .. 3 among them)
        for a in range(wl.n_adapters):
            where = np.flatnonzero(np.asarray(wl.ids) == a)
            assert where[0] in rows and where[-1] in rows
    m, f = assert_y_close(g["y"][sel], ref["y"], name)
    tf = assert_t_close(g["t"][sel].astype(np.float64), ref["t"], name)
    print(f"  y max_rel={m:.2e} frob={f:.2e} t frob={tf:.2e}", flush=True)


BUILD = [
    # T, K, N, fmt, ranks, seed: segments built inside the layer launch
    (4, 256, 256, "fp8", [8, 8], 21),
    (16, 1024, 384, "fp8", [16], 22),
    (16, 512, 256, "mxfp4", [16, 8, 32], 23),
    (64, 1024, 512, "fp8", [16] * 32, 24),
    (128, 2048, 256, "mxfp4", [8, 16, 32, 64] * 16, 25),
    (300, 768, 256, "fp8", [48, 8, 16, 64], 26),
]


@pytest.mark.parametrize("case", BUILD, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}_{c[3]}_a{len(c[4])}" for c in BUILD])
def test_segments_built_in_layer_launch(case):
    T, K, N, fmt, ranks, seed = case
    print(f"[case] in-launch segments {case}", flush=True)
    rng = np.random.default_rng(seed)
    n = len(ranks)
    ids = rng.integers(0, n, T)
    wl = _custom(T, K, N, fmt, ranks, ids, seed, a_std=0.1, b_std=0.05)
    g = run_gpu(wl, fused=True, build=True)
    assert g["status"] == 0 and g["err"] == 0
    seg_ref, srt_ref = oracle_segments(wl.ids, wl.n_adapters)
    assert np.array_equal(g["seg_indptr"], seg_ref) and np.array_equal(g["sorted_tok"], srt_ref)
    ref = run_oracle(wl)
    assert_y_close(g["y"], ref["y"], str(case))
    assert_t_close(g["t"].astype(np.float64), ref["t"], str(case))
    # the same kernels with the segments from their own launch: bitwise the same y
    g2 = run_gpu(wl, fused=True)
    assert np.array_equal(g["y_bits"], g2["y_bits"])


@pytest.mark.parametrize("reps", [5, 20], ids=["T40_in_launch", "T160_own_launch"])
def test_segments_built_in_layer_launch_bad_ids(reps):
    ids = np.array([0, 1, 7, 1, 0, -1, 1, 0] * reps, np.int32)  # > 16 tokens: the down-projection reads the segments
    T = ids.size
    wl = _custom(T, 512, 256, "fp8", [16, 16], np.where((ids >= 0) & (ids < 2), ids, 0), 27)
    wl.ids = ids
    g = run_gpu(wl, fused=True, build=True)
    assert g["status"] == 0 and g["err"] == 3
    good = np.flatnonzero((ids >= 0) & (ids < 2))
    seg_ref, srt_ref = oracle_segments(ids[good], 2)
    assert np.array_equal(g["seg_indptr"], seg_ref)
    assert np.array_equal(g["sorted_tok"][:good.size], good[srt_ref])
    ref = run_oracle(wl, rows=tuple(good.tolist()))
    assert_y_close(g["y"][good], ref["y"], "valid tokens")


def test_quant_all_bf16_patterns():
    import torch
    import precision_gemm_amd as P
    from workloads.device import bf16_tensor
    bits = np.arange(65536, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(4)
    bits = rng.permutation(bits)
    n = (bits.size // 256) * 256
    x = bits[:n].reshape(-1, 256)
    xq, xsc = P.quant_act_mxfp8(bf16_tensor(x))
    q_ref, s_ref = quantize_mxfp8(x)
    assert np.array_equal(xsc.cpu().numpy(), s_ref)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    # the same patterns confined to exponent windows placed across the range, so that the
    # blocks' scale codes cover 0 .. 246 (not only the top codes of the above)
    rows = []
    windows = [(24, e0) for e0 in (0, 1, 12, 40, 77, 100, 115, 126, 140, 170, 200, 231)] + [(4, 0), (8, 1), (6, 3)]
    for width, e0 in windows:
        e = (bits.astype(np.uint32) >> 7) & 0xFF
        b = (bits.astype(np.uint32) & 0x807F) | (((e % width) + e0) << 7)
        b = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)
        m = (b.size // 256) * 256
        rows.append(b[:m].reshape(-1, 256))
    x = np.concatenate(rows)
    xq, xsc = P.quant_act_mxfp8(bf16_tensor(x))
    q_ref, s_ref = quantize_mxfp8(x)
    assert np.array_equal(xsc.cpu().numpy(), s_ref)
    assert s_ref.min() == 0 and s_ref.max() >= 240
    assert np.array_equal(xq.cpu().numpy(), q_ref)


def test_segments_random_and_bad_ids():
    import torch
    import precision_gemm_amd as P
    rng = np.random.default_rng(5)
    cases = [(1, 1), (7, 3), (64, 32), (1000, 257), (4096, 8), (5000, 2048), (300, 8192),
             (4000, 5), (2000, 64), (2048, 65), (4096, 8, "sorted"), (3000, 3, "sorted")]
    for case in cases:
        T, n = case[0], case[1]
        ids = rng.integers(0, n, T).astype(np.int32)
        if len(case) > 2:  # contiguous segments, as in a prefill batch
            ids = np.sort(ids)
        seg = P.build_segments(torch.from_numpy(ids).cuda(), n)
        s_ref, o_ref = oracle_segments(ids, n)
        assert np.array_equal(seg.seg_indptr.cpu().numpy(), s_ref)
        assert np.array_equal(seg.sorted_tok.cpu().numpy(), o_ref)
        assert int(seg.err.item()) == 0
    # bad ids among few adapters in a long batch: skipped, the first one reported
    ids = rng.integers(0, 4, 3000).astype(np.int32)
    ids[[700, 1500, 2999]] = [7, -1, 4]
    seg = P.build_segments(torch.from_numpy(ids).cuda(), 4)
    assert int(seg.err.item()) == 701
    keep = np.flatnonzero((ids >= 0) & (ids < 4))
    s_ref, o_ref = oracle_segments(ids[keep], 4)
    assert np.array_equal(seg.seg_indptr.cpu().numpy(), s_ref)
    assert np.array_equal(seg.sorted_tok.cpu().numpy()[:keep.size], keep[o_ref])
    ids = np.array([0, 1, 5, 1, -2, 0], np.int32)
    seg = P.build_segments(torch.from_numpy(ids).cuda(), 2)
    assert int(seg.err.item()) == 3                      # 1 + first bad token index
    s_ref, o_ref = oracle_segments(ids[[0, 1, 3, 5]], 2)
    assert seg.seg_indptr.cpu().numpy().tolist() == [0, 2, 4]
    assert seg.sorted_tok.cpu().numpy()[:4].tolist() == [0, 5, 1, 3]


def _custom(T, K, N, fmt, ranks, ids, seed, **kw):
    scale = kw.pop("scale", [2.0] * len(ranks))
    return workloads.make_custom(T, K, N, fmt, ranks, ids, scale, seed, **kw)


EDGE = [
    # T, K, N, fmt, ranks, seed
    (1, 128, 64, "fp8", [8], 1),
    (5, 256, 128, "mxfp4", [16, 8], 2),
    (17, 512, 192, "fp8", [8, 16, 24, 32], 3),
    (37, 384, 256, "mxfp4", [64, 40, 8], 4),
    (65, 1024, 320, "fp8", [16] * 9, 5),
    (100, 640, 256, "mxfp4", [8, 16, 32, 64, 56], 6),
    (129, 256, 512, "fp8", [32, 16], 7),
    (200, 512, 384, "mxfp4", [8, 64, 16], 8),
    (300, 768, 256, "fp8", [48, 8, 16, 64], 9),
    (150, 640, 192, "fp8", [16, 32], 10),  # pre-quantised x with a partial last K-chunk
    # many adapters with a few tokens each: up-projection by the down-projection workgroups
    (96, 8192, 192, "fp8", [8, 16, 32, 64] * 20, 11),
    (200, 4096, 256, "mxfp4", [64, 8, 32, 16, 48] * 14, 12),
    (130, 1024, 320, "fp8", [16, 64] * 32, 13),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}_{c[3]}_a{len(c[4])}" for c in EDGE])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "unfused"])
def test_edge_shapes(case, fused):
    T, K, N, fmt, ranks, seed = case
    print(f"[case] edge {case} fused={fused}", flush=True)
    rng = np.random.default_rng(seed)
    n = len(ranks)
    ids = rng.integers(0, n, T)
    if n > 2:
        ids[ids == n - 1] = 0                 # leave the last adapter empty
    wl = _custom(T, K, N, fmt, ranks, ids, seed, a_std=0.1, b_std=0.05)
    ref = run_oracle(wl)
    g = run_gpu(wl, fused=fused)
    assert g["status"] == 0
    assert_y_close(g["y"], ref["y"], str(case))
    assert_t_close(g["t"].astype(np.float64), ref["t"], str(case))


LONG = [
    # T, K, N, ranks, seed: long batches of many tiles (128 x 256 tiles, pre-pass down-projection)
    (4100, 256, 4096, [1, 4, 12, 20, 60, 64], 31),  # 33 x 16 tiles, XCD-grouped order; a 4-row last token tile
    (3100, 384, 5376, [16, 64, 8], 32),              # 25 x 21 = 525 tiles: plain order
    # 128 x 512 eight-wave tiles (k_gemm_pf): 33 x 8 tiles in the XCD-grouped order, a
    # 4-row last token tile; 25 x 6 = 150 tiles (an odd number of row blocks), plain order
    (4100, 1024, 4096, [1, 4, 12, 20, 60, 64], 33),
    (3100, 512, 3072, [16, 64, 8], 34),
]


@pytest.mark.parametrize("case", LONG, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}_a{len(c[3])}" for c in LONG])
@pytest.mark.parametrize("mode", ["fused", "fused_t_in_workspace", "unfused", "base_only", "build"])
def test_long_batch_shapes(case, mode):
    T, K, N, ranks, seed = case
    print(f"[case] long batch {case} {mode}", flush=True)
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, len(ranks), T)
    wl = _custom(T, K, N, "fp8", ranks, ids, seed, a_std=0.1, b_std=0.05)
    # sampled rows, both ends of every segment, and every row of the last (partial) token tiles
    rows = tuple(sorted(set(sample_rows(wl, 256, seed)) | set(range(256 * (T // 256), T))))
    ref = run_oracle(wl, rows)
    g = run_gpu(wl, fused=(mode != "unfused"), want_t=(mode != "fused_t_in_workspace"),
                base_only=(mode == "base_only"), build=(mode == "build"))
    assert g["status"] == 0 and g["err"] == 0
    sel = np.asarray(rows)
    key = "y_base" if mode == "base_only" else "y"
    m, f = assert_y_close(g["y"][sel], ref[key], f"{case} {mode}")
    if "t" in g:
        assert_t_close(g["t"][sel].astype(np.float64), ref["t"], f"{case} {mode}")
    print(f"  y max_rel={m:.2e} frob={f:.2e}", flush=True)


# Long MXFP8 batches on the 128 x 512 tiles whose tokens come in runs of one adapter (the
# prefill form: positions are tokens), with run lengths that are not multiples of 16: waves
# of the pre-pass whose 16 positions hold two adapters, 64-position blocks split over several,
# a last block of 4 positions, and (second case) a tail of tokens without an adapter.
PF_RUNS = [
    (4100, 1024, 4096, [1, 4, 12, 20, 60, 64], [7, 300, 1, 513, 29, 1000, 250, 2000], 41),
    (1000, 512, 8192, [64, 16, 33], [100, 3, 17, 700], 42),
]


@pytest.mark.parametrize("case", PF_RUNS, ids=[f"T{c[0]}_K{c[1]}_N{c[2]}" for c in PF_RUNS])
@pytest.mark.parametrize("mode", ["fused", "build"])
def test_long_batch_adapter_runs(case, mode):
    T, K, N, ranks, runs, seed = case
    print(f"[case] long batch in adapter runs {case[:3]} {mode}", flush=True)
    ids = np.concatenate([np.full(n, i % len(ranks)) for i, n in enumerate(runs)] +
                         [np.full(T - sum(runs), -1)]).astype(np.int32)
    wl = _custom(T, K, N, "fp8", ranks, np.maximum(ids, 0), seed, a_std=0.1, b_std=0.05)
    wl.ids = ids
    rows = np.asarray(sorted(set(sample_rows(wl, 256, seed)) | set(range(256 * (T // 256), T))))
    good, bad = rows[ids[rows] >= 0], rows[ids[rows] < 0]
    g = run_gpu(wl, fused=True, want_t=True, build=(mode == "build"))
    assert g["status"] == 0 and (g["err"] != 0) == bool((ids < 0).any())
    ref = run_oracle(wl, tuple(good.tolist()))
    m, f = assert_y_close(g["y"][good], ref["y"], f"{case[:3]} {mode}")
    assert_t_close(g["t"][good].astype(np.float64), ref["t"], f"{case[:3]} {mode}")
    if len(bad):
        from oracle.layer import LowpWeight as OW, base_gemm
        xq, xs = quantize_mxfp8(wl.x[bad])
        assert_y_close(g["y"][bad], base_gemm(xq, xs, OW(wl.fmt, wl.w_q, wl.w_scale)), "tokens without an adapter")
    print(f"  y max_rel={m:.2e} frob={f:.2e}", flush=True)


def test_zero_b_equals_base_only_and_zero_w_gives_lora():
    wl = _custom(48, 1024, 512, "fp8", [16, 32, 8], np.arange(48) % 3, 11, zero_b=True)
    fused = run_gpu(wl, fused=True)
    base = run_gpu(wl, base_only=True)
    assert np.array_equal(fused["y"], base["y"])           # numerically equal (+0 / -0 may differ)
    ref = run_oracle(wl)
    assert_y_close(base["y"], ref["y_base"], "base only")
    wl = _custom(48, 1024, 512, "mxfp4", [16, 32, 8], np.arange(48) % 3, 12, zero_w=True, b_std=0.05)
    g = run_gpu(wl, fused=True)
    ref = run_oracle(wl)
    assert not ref["y_base"].any()
    assert_y_close(g["y"], ref["y_lora"], "zero W")


def test_lora_heavy_input():
    # B std raised so that the adapter term is as large as the base term
    wl = _custom(64, 2048, 1024, "fp8", [16, 64], np.arange(64) % 2, 13, b_std=0.07, a_std=1 / 45)
    ref = run_oracle(wl)
    ratio = np.linalg.norm(ref["y_lora"]) / np.linalg.norm(ref["y_base"])
    assert 0.3 < ratio < 3
    for fused in (True, False):
        g = run_gpu(wl, fused=fused)
        assert_y_close(g["y"], ref["y"], f"lora-heavy fused={fused}")


def test_bad_ids_skip_adapter_term():
    ids = np.array([0, 1, 7, 1, 0, -1, 1, 0], np.int32)
    wl = _custom(8, 512, 256, "fp8", [16, 16], np.where((ids >= 0) & (ids < 2), ids, 0), 14)
    wl.ids = ids
    g = run_gpu(wl, fused=True)
    assert g["err"] == 3
    good = np.array([0, 1, 3, 4, 6, 7])
    ref = run_oracle(wl, rows=good)
    assert_y_close(g["y"][good], ref["y"], "valid tokens")
    from oracle.layer import LowpWeight as OW, base_gemm
    xq, xs = quantize_mxfp8(wl.x[[2, 5]])
    y_base = base_gemm(xq, xs, OW(wl.fmt, wl.w_q, wl.w_scale))
    assert np.isfinite(g["y"][[2, 5]]).all()
    assert_y_close(g["y"][[2, 5]], y_base, "bad-id tokens get the base term only")


@pytest.mark.parametrize("name", ["decode_gateup", "downproj_fp4"])
def test_bitwise_determinism(name):
    wl = named(name)
    outs = [run_gpu(wl, fused=True) for _ in range(3)]
    for o in outs[1:]:
        assert np.array_equal(o["y_bits"], outs[0]["y_bits"])
        assert np.array_equal(o["t"], outs[0]["t"])


def test_expand_standalone_matches_oracle():
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    wl = named("decode_gateup")
    ref = named_oracle("decode_gateup", None)
    x, w, ad, ids = upload(wl)
    seg = P.build_segments(ids, ad.n)
    ws = P.alloc_workspace(wl.T, wl.K, wl.N, ad.n, ad.r_max)
    y = P.gemm_lowp_lora_epilogue(x, w, seg, ad, ws, t=None, fuse_shrink=False)
    t = P.shrink(x, seg, ad, ws)
    P.expand(t, seg, ad, y)
    torch.cuda.synchronize()
    from gpu_util import bf16_to_f64
    assert_y_close(bf16_to_f64(y), ref["y"], "unfused expand")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_pack_weight_layout(fmt):
    """The packed W layout, checked byte for byte against its definition in lora_lowp.h."""
    import torch
    import precision_gemm_amd as P
    rng = np.random.default_rng(6)
    N, K = 128, 512
    kb = K if fmt == "fp8" else K // 2
    q = rng.integers(0, 256, (N, kb), dtype=np.uint8)
    sc = rng.integers(0, 256, (N, K // 32), dtype=np.uint8) if fmt == "mxfp4" else rng.random(N).astype(np.float32)
    w = P.pack_weight(P.LowpWeight(fmt, torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda()))
    got = w.q.cpu().numpy().reshape(-1)
    lanes = np.arange(64)
    j, g = lanes % 16, lanes // 16
    ref = []
    for nt in range(N // 16):
        for ks in range(K // 128):
            if fmt == "fp8":
                for h in range(2):
                    for l in range(64):
                        k0 = ks * 128 + h * 64 + g[l] * 16
                        ref.append(q[nt * 16 + j[l], k0:k0 + 16])
            else:
                for l in range(64):
                    b0 = ks * 64 + g[l] * 16
                    ref.append(q[nt * 16 + j[l], b0:b0 + 16])
    assert np.array_equal(got, np.concatenate(ref))
    if fmt == "mxfp4":
        sref = np.array([sc[nt * 16 + j[l], ks * 4 + g[l]] for nt in range(N // 16) for ks in range(K // 128)
                         for l in range(64)], np.uint8)
        assert np.array_equal(w.scale.cpu().numpy().reshape(-1), sref)

"""GPU parity of the backward (lora_backward, with lora_pack_weight_t and
lora_pack_adapter_bwd) against the backward oracle, oracle/backward.py.

Tolerances, from the arithmetic the header states:
* dX: W enters as bf16(code x channel scale) (relative error <= 2^-9 per element), the
  fp32 factor s_a u as two bf16 terms (<= 2^-18), sums in fp32, the result rounded to bf16
  (<= 2^-9).  Element by element |dX - ref| <= 2^-8 (|dY| |W_d|^T + s_a |u| |A_a|^T + |ref|),
  and the layer's own bounds: max error <= 1e-2 max |ref|, relative Frobenius <= 5e-3.
* dA, dB: exact bf16 products of M and the two bf16 terms of the fp32 factor (<= 2^-18),
  fp32 sums over at most a few thousand tokens: element by element
  |g - ref| <= 2^-14 s_a (|M|^T |V|), and relative Frobenius <= 1e-5.
* u: the forward's down-projection kernel (exact products, fp32 sums): relative Frobenius
  <= 1e-5 against dY B_a^T.
Cases: the tiny and the 4096-token prefill shapes of the layer, a ragged batch (T not a
multiple of 128, K not a multiple of 256) with mixed ranks 1..60 in random order, several
row blocks with contiguous segments, an adapter without tokens, largest ranks 62, 21, 40
and 30 (two to four rank tiles in the gradient kernel), short batches whose dX contraction is
split over N (16, 8 and 4 ranges, a partial column block, a shorter last range), t from the
GPU's own forward, T = 0, an invalid rank, and bitwise repeatability (whole and split).
"""

import functools

import numpy as np
import pytest

import workloads
from oracle import backward as BW
from oracle.layer import LowpWeight as OracleWeight

pytestmark = pytest.mark.gpu

DX_MAX_REL, DX_FROB_REL = 1e-2, 5e-3
G_FROB_REL = 1e-5
U_FROB_REL = 1e-5


def _contig(T, n, rng):
    cuts = np.sort(rng.choice(np.arange(1, T), n - 1, replace=False))
    return np.repeat(np.arange(n), np.diff(np.concatenate([[0], cuts, [T]]))).astype(np.int32)


CASES = {
    # name: (T, K, N, ranks, ids kind)
    "tiny": (4, 256, 256, [8, 8], "tiny"),
    "ragged_mixed": (77, 640, 384, [1, 12, 20, 60], "random"),
    "contig_rows": (300, 1024, 512, [16, 64, 8, 32], "contig"),
    "empty_adapter": (130, 512, 256, [16, 24, 8], "skip1"),
    # the gradient kernel's rank tiles: largest ranks 62 (four tiles, the last partial), 21
    # (two, the second holding one rank), 40 (three), 30 (two, with a rank-1 adapter)
    "rmax62": (150, 512, 256, [62, 5, 33], "random"),
    "rmax21": (100, 384, 256, [21, 3], "random"),
    "rmax40": (90, 256, 384, [40, 17], "random"),
    "rmax30": (100, 384, 256, [30, 7, 1], "contig"),
    # short batches: dX's contraction over N split into ranges (workspace partial sums)
    "split16": (40, 1024, 4096, [16, 64, 8], "random"),       # 4 tiles x 16 ranges of 4 steps
    "split8_raggedK": (70, 640, 2048, [32, 5], "contig"),     # a half column block; 8 ranges
    "split4_tail": (20, 512, 1408, [24, 1, 64], "random"),    # 4 ranges, the last shorter
}


@functools.lru_cache(maxsize=4)
def _case(name):
    if name == "prefill":
        wl = workloads.make("prefill")
        return wl, workloads.grad_output(wl.T, wl.N, 2004)
    T, K, N, ranks, kind = CASES[name]
    rng = np.random.default_rng(sum(map(ord, name)))
    if kind == "tiny":
        ids = np.array([0, 1, 1, 0], np.int32)
    elif kind == "random":
        ids = rng.integers(0, len(ranks), T).astype(np.int32)
    elif kind == "contig":
        ids = _contig(T, len(ranks), rng)
    else:  # adapter 1 has no tokens
        ids = rng.choice(np.array([0, 2]), T).astype(np.int32)
    scale = [2.0, 0.5, 1.25, 16.0 / 60][: len(ranks)]
    wl = workloads.make_custom(T, K, N, "fp8", ranks, ids, scale, 700 + T, a_std=1.0 / 16, b_std=0.05)
    return wl, workloads.grad_output(T, N, 800 + T)


@functools.lru_cache(maxsize=4)
def _oracle(name):
    wl, dy = _case(name)
    return BW.lora_backward(wl.x, OracleWeight(wl.fmt, wl.w_q, wl.w_scale), wl.A, wl.B, wl.scale, wl.ids, dy)


def _f64(bits):
    return workloads.bf16_to_f32(bits).astype(np.float64)


def run_backward(wl, dy_bits, t=None, nan_fill=True, repeat=1):
    """lora_backward on the GPU.  t: float32 [T, r_max] input, or None for the GPU's own
    forward down-projection (lora_shrink).  Returns numpy results."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import bf16_tensor, upload
    x, w, ad, ids = upload(wl)
    q = torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda()
    sc = torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda()
    wt = P.pack_weight_t(P.LowpWeight("fp8", q, sc))
    bw = P.pack_adapters_bwd(ad)
    seg = P.build_segments(ids, ad.n)
    dy = bf16_tensor(dy_bits)
    tt = P.shrink(x, seg, ad) if t is None else torch.from_numpy(np.ascontiguousarray(t, np.float32)).cuda()
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(repeat):
        dA = [torch.full((wl.K, int(r)), float("nan") if nan_fill else 0.0, device="cuda") for r in wl.ranks]
        dB = [torch.full((int(r), wl.N), float("nan") if nan_fill else 0.0, device="cuda") for r in wl.ranks]
        dx, u, gr = P.lora_backward(x, dy, tt, wt, sc, seg, ad, bw, grads=P.grads_from(dA, dB), status=st)
        torch.cuda.synchronize()
        outs.append({"dx_bits": dx.view(torch.int16).cpu().numpy().view(np.uint16),
                     "dx": dx.float().cpu().numpy().astype(np.float64), "u": u.cpu().numpy().astype(np.float64),
                     "dA": [m.cpu().numpy().astype(np.float64) for m in dA],
                     "dB": [m.cpu().numpy().astype(np.float64) for m in dB], "status": int(st.item())})
    return outs if repeat > 1 else outs[0]


def check_against_oracle(wl, dy, g, ref, what):
    Wd = BW.base_weight(OracleWeight(wl.fmt, wl.w_q, wl.w_scale))
    x, d = _f64(wl.x), _f64(dy)
    seg, srt = ref["seg_indptr"], ref["sorted_tok"]
    # u
    uf = np.linalg.norm(g["u"] - ref["u"]) / max(np.linalg.norm(ref["u"]), 1e-300)
    assert uf <= U_FROB_REL, f"{what}: u frob {uf:.2e}"
    # dX
    assert np.isfinite(g["dx"]).all(), what
    bound = np.abs(d) @ np.abs(Wd) + np.abs(ref["dx"])
    for a in range(wl.n_adapters):
        R = srt[seg[a]:seg[a + 1]]
        if R.size:
            r = int(wl.ranks[a])
            bound[R] += float(np.float32(wl.scale[a])) * (np.abs(ref["u"][R, :r]) @ np.abs(_f64(wl.A[a])).T)
    err = np.abs(g["dx"] - ref["dx"])
    worst = float((err / (2.0 ** -8 * bound + 1e-30)).max())
    assert worst <= 1.0, f"{what}: dx element bound exceeded x{worst:.2f}"
    m = err.max() / np.abs(ref["dx"]).max()
    f = np.linalg.norm(g["dx"] - ref["dx"]) / np.linalg.norm(ref["dx"])
    assert m <= DX_MAX_REL and f <= DX_FROB_REL, f"{what}: dx max_rel {m:.2e} frob {f:.2e}"
    # dA, dB
    gworst, gfrob = 0.0, 0.0
    for a in range(wl.n_adapters):
        R = srt[seg[a]:seg[a + 1]]
        s = abs(float(np.float32(wl.scale[a])))
        r = int(wl.ranks[a])
        for key, M, V in (("dA", x, ref["u"]), ("dB", d, ref["t"])):
            gg, rr = g[key][a], ref[key][a]
            assert np.isfinite(gg).all(), f"{what}: {key}[{a}] not fully written"
            absb = s * (np.abs(M[R]).T @ np.abs(V[R, :r]))           # [C, r]
            if key == "dB":
                absb = absb.T
            e = np.abs(gg - rr)
            if R.size == 0:
                assert not gg.any(), f"{what}: {key}[{a}] of an adapter without tokens is not zero"
                continue
            gworst = max(gworst, float((e / (2.0 ** -14 * absb + 1e-30)).max()))
            gfrob = max(gfrob, float(np.linalg.norm(e) / max(np.linalg.norm(rr), 1e-300)))
    assert gworst <= 1.0, f"{what}: dA/dB element bound exceeded x{gworst:.2f}"
    assert gfrob <= G_FROB_REL, f"{what}: dA/dB frob {gfrob:.2e}"
    return m, f, gfrob


@pytest.mark.parametrize("name", ["tiny", "ragged_mixed", "contig_rows", "empty_adapter", "rmax62", "rmax21", "rmax40",
                                  "rmax30", "split16", "split8_raggedK", "split4_tail", "prefill"])
def test_backward_matches_oracle(name):
    print(f"[case] backward {name}", flush=True)
    wl, dy = _case(name)
    ref = _oracle(name)
    g = run_backward(wl, dy, t=ref["t"].astype(np.float32))
    assert g["status"] == 0
    m, f, gf = check_against_oracle(wl, dy, g, ref, name)
    print(f"  dx max_rel={m:.2e} frob={f:.2e}  dA/dB frob={gf:.2e}", flush=True)


@pytest.mark.parametrize("name", ["ragged_mixed", "prefill"])
def test_backward_on_the_gpu_forward_t(name):
    """t from the GPU's own down-projection (the forward a trainer saved), not the oracle's."""
    print(f"[case] backward {name}, t from lora_shrink", flush=True)
    wl, dy = _case(name)
    g = run_backward(wl, dy, t=None)
    assert g["status"] == 0
    check_against_oracle(wl, dy, g, _oracle(name), name + " gpu t")


@pytest.mark.parametrize("name", ["contig_rows", "split16"])
def test_backward_is_bitwise_repeatable(name):
    wl, dy = _case(name)
    a, b = run_backward(wl, dy, t=_oracle(name)["t"].astype(np.float32), repeat=2)
    assert np.array_equal(a["dx_bits"], b["dx_bits"]) and np.array_equal(a["u"], b["u"])
    for k in ("dA", "dB"):
        for x, y in zip(a[k], b[k]):
            assert np.array_equal(x, y)


def test_backward_without_tokens_zero_fills():
    """T = 0: every dA_a and dB_a is zero (written), nothing else is touched."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import upload
    print("[case] backward T=0", flush=True)
    wl, _ = _case("tiny")
    x, w, ad, ids = upload(wl)
    q = torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda()
    sc = torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda()
    wt = P.pack_weight_t(P.LowpWeight("fp8", q, sc))
    bw = P.pack_adapters_bwd(ad)
    seg = P.build_segments(ids[:0], ad.n)
    dA = [torch.full((wl.K, int(r)), float("nan"), device="cuda") for r in wl.ranks]
    dB = [torch.full((int(r), wl.N), float("nan"), device="cuda") for r in wl.ranks]
    z = torch.empty((0, wl.K), dtype=torch.bfloat16, device="cuda")
    P.lora_backward(z, torch.empty((0, wl.N), dtype=torch.bfloat16, device="cuda"),
                    torch.empty((0, ad.r_max), device="cuda"), wt, sc, seg, ad, bw, grads=P.grads_from(dA, dB))
    torch.cuda.synchronize()
    assert all(not m.cpu().numpy().any() for m in dA + dB)


def test_backward_reports_an_invalid_rank():
    """An adapter with tokens whose rank (in device memory) is outside [1, r_max]: status bit
    1, its gradients untouched, its tokens get dY W_d^T only, the others are unaffected."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import bf16_tensor, upload
    print("[case] backward invalid rank", flush=True)
    wl, dy_bits = _case("contig_rows")
    ref = _oracle("contig_rows")
    x, w, ad, ids = upload(wl)
    q = torch.from_numpy(np.ascontiguousarray(wl.w_q)).cuda()
    sc = torch.from_numpy(np.ascontiguousarray(wl.w_scale)).cuda()
    wt = P.pack_weight_t(P.LowpWeight("fp8", q, sc))
    bw = P.pack_adapters_bwd(ad)
    seg = P.build_segments(ids, ad.n)
    ad.ranks[2] = 65
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dA = [torch.full((wl.K, int(r)), 7.0, device="cuda") for r in wl.ranks]
    dB = [torch.full((int(r), wl.N), 7.0, device="cuda") for r in wl.ranks]
    t = torch.from_numpy(ref["t"].astype(np.float32)).cuda()
    dx, u, _ = P.lora_backward(x, bf16_tensor(dy_bits), t, wt, sc, seg, ad, bw, grads=P.grads_from(dA, dB), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 2
    assert (dA[2].cpu().numpy() == 7.0).all() and (dB[2].cpu().numpy() == 7.0).all()
    dxg = dx.float().cpu().numpy().astype(np.float64)
    on2 = np.flatnonzero(wl.ids == 2)
    rest = np.flatnonzero(wl.ids != 2)
    base = _f64(dy_bits) @ BW.base_weight(OracleWeight(wl.fmt, wl.w_q, wl.w_scale))
    for rows, want in ((on2, base[on2]), (rest, ref["dx"][rest])):
        f = np.linalg.norm(dxg[rows] - want) / np.linalg.norm(want)
        assert f <= DX_FROB_REL, f
    for a in (0, 1, 3):
        gg, rr = dA[a].cpu().numpy(), ref["dA"][a]
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= G_FROB_REL


def test_pack_layouts():
    """lora_pack_weight_t and lora_pack_adapter_bwd against their definitions in lora_lowp.h,
    byte for byte."""
    import torch
    import precision_gemm_amd as P
    from workloads.device import bf16_tensor
    rng = np.random.default_rng(5)
    N, K = 384, 256
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)
    qt = P.pack_weight_t(P.LowpWeight("fp8", torch.from_numpy(q).cuda(), torch.ones(N, device="cuda")))
    got = qt.cpu().numpy()
    # [kt][ns][g][i][e] <- W[64 ns + 16 g + e][16 kt + i]
    ref = q.reshape(N // 64, 4, 16, K // 16, 16).transpose(3, 0, 1, 4, 2).reshape(-1)
    assert np.array_equal(got, ref)
    for K, N, r in [(256, 128, 1), (128, 192, 12), (64, 256, 60), (192, 64, 64), (128, 320, 17)]:
        A = rng.integers(0, 1 << 16, (K, r), dtype=np.uint16)
        B = rng.integers(0, 1 << 16, (r, N), dtype=np.uint16)
        import precision_gemm_amd.ops as O
        ad = O.Adapters([bf16_tensor(A)], [bf16_tensor(B)], torch.ones(1, device="cuda"))
        bw = P.pack_adapters_bwd(ad)
        torch.cuda.synchronize()
        ra, rp = P.a_rows(r), P.rank_pad(r)
        bop = bw.Bop[0].view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        ar = bw.Ar[0].view(torch.int16).cpu().numpy().view(np.uint16)
        Bp = np.zeros((ra, N), np.uint16)
        Bp[:r] = B
        # [jt][ns][h][g][i][e] <- B[16 jt + i][64 ns + 16 g + 8 h + e]
        refb = Bp.reshape(ra // 16, 16, N // 64, 4, 2, 8).transpose(0, 2, 4, 3, 1, 5).reshape(-1)
        assert np.array_equal(bop, refb), (K, N, r)
        assert ar.shape == (K, rp) and np.array_equal(ar[:, :r], A) and not ar[:, r:].any()

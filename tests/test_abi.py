"""The C-ABI library loads, exports every function include/lora_lowp.h declares, and
rejects bad arguments on the host with the documented status codes (no GPU needed:
every call here fails validation before anything touches the device)."""

import ctypes

import pytest

from precision_gemm_amd import _lib

LORA_OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_header_function(L):
    names = _lib.header_functions()
    assert {"lora_build_segments", "lora_shrink", "lora_expand", "gemm_lowp_lora_epilogue"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib._SIGNATURES)


def test_status_strings_and_version(L):
    for s in (0, 1, 2, 3, 5, 99):
        assert L.lora_status_string(s)
    assert b"gfx950" in L.lora_version()


def test_workspace_bytes(L):
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 16) > 0
    assert L.lora_workspace_bytes(16, 4000, 6144, 1, 16) == 0      # K % 128
    assert L.lora_workspace_bytes(16, 4096, 6100, 1, 16) == 0      # N % 64
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 12) > 0       # any r_max in [1, 64]
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 1) > 0
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 65) == 0      # r_max > 64
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 0) == 0
    assert L.lora_workspace_bytes(16, 4096, 6144, 0, 16) == 0
    assert L.lora_workspace_bytes(-1, 4096, 6144, 1, 16) == 0


def test_plan_info(L):
    buf = (ctypes.c_int32 * 16)()
    assert L.lora_plan_info(16, 4096, 6144, 1, 16, 0, buf, 16) == 15
    assert buf[0] == 1 and buf[10] > 0
    assert L.lora_plan_info(4096, 4096, 4096, 8, 64, 0, buf, 16) == 15 and buf[4] == 1
    assert L.lora_plan_info(16, 100, 6144, 1, 16, 0, buf, 16) == -1


NULL = None
FAKE = ctypes.c_void_p(0x1000)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x1004)


def _gemm(L, **kw):
    a = dict(x=FAKE, T=16, K=4096, N=6144, fmt=0, wq=FAKE, ws=FAKE, t=NULL, ids=FAKE, seg=FAKE, srt=FAKE,
             A=FAKE, B=FAKE, rk=FAKE, sc=FAKE, n=1, r=16, y=FAKE, flags=1, wsp=NULL, wsb=0, stream=NULL)
    a.update(kw)
    return L.gemm_lowp_lora_epilogue(a["x"], a["T"], a["K"], a["N"], a["fmt"], a["wq"], a["ws"], a["t"], a["ids"],
                                     a["seg"], a["srt"], a["A"], a["B"], a["rk"], a["sc"], a["n"], a["r"], a["y"],
                                     a["flags"], a["wsp"], a["wsb"], a["stream"])


def test_gemm_validation(L):
    assert _gemm(L, T=-1) == INVALID
    assert _gemm(L, T=0) == LORA_OK                      # no-op
    assert _gemm(L, K=4000) == UNSUPPORTED
    assert _gemm(L, N=100) == UNSUPPORTED
    assert _gemm(L, T=70000) == UNSUPPORTED
    assert _gemm(L, fmt=7) == INVALID
    assert _gemm(L, flags=8) == INVALID                  # unknown flag
    assert _gemm(L, flags=2) == INVALID                  # segment build without the fused down-projection
    assert _gemm(L, flags=5) == WORKSPACE                # 16-bit activations: valid (fails at the workspace)
    assert _gemm(L, flags=5, T=4096) == WORKSPACE
    assert _gemm(L, x=NULL) == INVALID
    assert _gemm(L, x=MISALIGNED) == INVALID
    assert _gemm(L, A=NULL) == INVALID                   # fused needs A
    assert _gemm(L, flags=0, t=NULL, A=NULL, B=NULL, ids=NULL, rk=NULL, sc=NULL) == WORKSPACE  # base only: adapters optional
    assert _gemm(L, r=12) == WORKSPACE                   # any r_max in [1, 64] is valid
    assert _gemm(L, r=1) == WORKSPACE
    assert _gemm(L, r=65) == UNSUPPORTED
    assert _gemm(L, r=0) == INVALID
    assert _gemm(L, n=0) == INVALID
    assert _gemm(L) == WORKSPACE                         # no workspace
    assert _gemm(L, wsp=FAKE, wsb=16) == WORKSPACE       # too small


def test_other_entry_points_validation(L):
    assert L.lora_build_segments(FAKE, -1, 4, FAKE, FAKE, FAKE, NULL) == INVALID
    assert L.lora_build_segments(FAKE, 4, 0, FAKE, FAKE, FAKE, NULL) == INVALID
    assert L.lora_build_segments(FAKE, 4, 9000, FAKE, FAKE, FAKE, NULL) == UNSUPPORTED
    assert L.lora_build_segments(NULL, 4, 4, FAKE, FAKE, FAKE, NULL) == INVALID
    assert L.lora_quant_act_mxfp8(FAKE, 4, 48, FAKE, FAKE, NULL) == UNSUPPORTED
    assert L.lora_quant_act_mxfp8(NULL, 4, 64, FAKE, FAKE, NULL) == INVALID
    assert L.lora_quant_act_mxfp8(FAKE, 0, 64, FAKE, FAKE, NULL) == LORA_OK
    assert L.lora_shrink(FAKE, 4, 250, FAKE, FAKE, FAKE, FAKE, 2, 8, FAKE, NULL, 0, NULL) == UNSUPPORTED
    assert L.lora_shrink(NULL, 4, 256, FAKE, FAKE, FAKE, FAKE, 2, 8, FAKE, NULL, 0, NULL) == INVALID
    assert L.lora_expand(FAKE, 4, 256, FAKE, FAKE, FAKE, FAKE, 2, 8, NULL, NULL) == INVALID
    assert L.lora_expand(FAKE, 4, 250, FAKE, FAKE, FAKE, FAKE, 2, 8, FAKE, NULL) == UNSUPPORTED
    assert L.lora_workspace_init(NULL, 16, NULL) == INVALID
    assert L.lora_pack_weight(0, FAKE, NULL, 100, 256, FAKE, NULL, NULL) == UNSUPPORTED
    assert L.lora_pack_weight(1, FAKE, NULL, 128, 256, FAKE, NULL, NULL) == INVALID   # MXFP4 needs scales
    assert L.lora_pack_weight(0, FAKE, NULL, 128, 256, FAKE, NULL, NULL) == INVALID   # in place
    assert L.lora_pack_weight(3, FAKE, NULL, 128, 256, MISALIGNED, NULL, NULL) == INVALID
    assert L.lora_workspace_status(NULL, FAKE, NULL) == INVALID


def test_plan_long_batch_tiles():
    """Host plan (no GPU): MXFP8 batches past 128 tokens with FP8 W, K and N multiples of 512
    and at least 128 tiles of 128 tokens x 512 channels take the eight-wave tiles (8 token
    tiles x 8 column tiles x 4 waves of columns, no K-split); MXFP4 W, fewer tiles or other
    K and N keep the 128 x 256 tiles."""
    from precision_gemm_amd.ops import plan_info
    for T, K, N, fmt, pf in [(4096, 4096, 4096, "fp8", True), (1000, 512, 8192, "fp8", True),
                             (4100, 1024, 4096, "fp8", True), (4100, 256, 4096, "fp8", False),
                             (3100, 384, 5376, "fp8", False), (300, 1024, 512, "fp8", False),
                             (4096, 4096, 4096, "mxfp4", False), (4096, 1024, 4352, "fp8", False),
                             (128, 4096, 8192, "fp8", False), (1000, 512, 4096, "fp8", False)]:
        p = plan_info(T, K, N, 8, 64, fmt)
        assert ((p["TT"], p["CT"], p["WC"]) == (8, 8, 4)) == pf, (T, K, N, fmt, p)
        if pf:
            assert p["ksplit"] == 1 and p["n_tb"] == -(-T // 128) and p["n_cb"] == N // 512 and p["XQ"] == 1


def test_plan_down_projection_grid_and_k_split():
    """Host plan (no GPU): past 128 tokens the fused launch's down-projection grid holds
    every item that has work for any segment structure of T tokens (each adapter adds at
    most one partial token block); from 17 to 128 tokens it holds at most one workgroup per
    CU (the workgroups loop over the rest); K-splits keep the GEMM grid within 224
    workgroups once a shape has fewer than 128 tiles."""
    import numpy as np
    from precision_gemm_amd.ops import plan_info
    rng = np.random.default_rng(3)
    for T, n_ad, r_max, K, N in [(129, 2, 64, 4096, 4096), (300, 40, 64, 1024, 256), (4096, 8, 64, 4096, 4096),
                                 (1000, 257, 32, 2048, 512), (4096, 1, 16, 4096, 8192), (2048, 4096, 64, 1024, 1024)]:
        p = plan_info(T, K, N, n_ad, r_max)
        tblk, njg, kparts, jper = p["s_tblk"], p["s_njg"], p["s_kparts"], 2
        for _ in range(20):
            n_used = int(rng.integers(1, min(n_ad, T) + 1))
            cuts = np.sort(rng.choice(np.arange(1, T), n_used - 1, replace=False)) if n_used > 1 else np.array([], int)
            lens = np.diff(np.concatenate([[0], cuts, [T]]))
            ranks = rng.choice(np.arange(8, r_max + 1, 8), n_used)
            items = sum(-(-int(L) // tblk) * min(njg, -(-int(r) // (16 * jper))) * kparts for L, r in zip(lens, ranks))
            assert items <= p["n_shrink_wg"], (T, n_ad, items, p)
    for T, n_ad in [(17, 4), (64, 32), (128, 128), (100, 5)]:
        p = plan_info(T, 4096, 4096, n_ad, 64)
        assert 1 <= p["n_shrink_wg"] <= 256
    for T, K, N in [(128, 21504, 5376), (64, 4096, 1024), (100, 2048, 2048), (4096, 4096, 4096)]:
        p = plan_info(T, K, N, 8, 64)
        tiles = p["n_cb"] * p["n_tb"]
        assert p["n_gemm_wg"] == tiles * p["ksplit"]
        assert tiles >= 128 or p["n_gemm_wg"] <= max(224, tiles), p


def test_flag_values_match_header():
    import re
    import precision_gemm_amd as P
    text = open(_lib.HEADER).read()
    vals = {m.group(1): 1 << int(m.group(2)) for m in re.finditer(r"(LORA_[A-Z0-9_]+) = 1u << (\d+)", text)}
    assert vals == {"LORA_FUSE_SHRINK": P.LORA_FUSE_SHRINK, "LORA_BUILD_SEGMENTS": P.LORA_BUILD_SEGMENTS,
                    "LORA_ACT_BF16": P.LORA_ACT_BF16}


def test_status_of_every_unsupported_shape_and_rank(L):
    """Each limit of the header, on each call that takes it: the documented status, and
    nothing enqueued (every pointer here is fake, so a launch would fault)."""
    # shapes: K % 128, N % 64, T above 65536, ranks above 64, adapters above 8192
    for kw, want in [(dict(K=4096 + 32), UNSUPPORTED), (dict(K=4096 + 96), UNSUPPORTED), (dict(K=0), INVALID),
                     (dict(N=6144 + 32), UNSUPPORTED), (dict(N=0), INVALID), (dict(T=65537), UNSUPPORTED),
                     (dict(r=65), UNSUPPORTED), (dict(r=-3), INVALID), (dict(n=8193), UNSUPPORTED),
                     (dict(n=-1), INVALID)]:
        for flags in (0, 1, 3, 5):
            got = _gemm(L, flags=flags, **kw) if flags != 0 else _gemm(L, flags=0, t=FAKE, **kw)
            assert got == want, (kw, flags, got)
    assert L.lora_workspace_bytes(16, 4096 + 32, 6144, 1, 16) == 0
    assert L.lora_workspace_bytes(70000, 4096, 6144, 1, 16) == 0
    assert L.lora_workspace_bytes(16, 4096, 6144, 8193, 16) == 0
    assert L.lora_shrink(FAKE, 4, 4096 + 32, FAKE, FAKE, FAKE, FAKE, 2, 8, FAKE, NULL, 0, NULL) == UNSUPPORTED
    assert L.lora_shrink(FAKE, 4, 256, FAKE, FAKE, FAKE, FAKE, 2, 65, FAKE, NULL, 0, NULL) == UNSUPPORTED
    assert L.lora_shrink(FAKE, 4, 256, FAKE, FAKE, FAKE, FAKE, 2, 0, FAKE, NULL, 0, NULL) == INVALID
    assert L.lora_expand(FAKE, 4, 256, FAKE, FAKE, FAKE, FAKE, 2, 65, FAKE, NULL) == UNSUPPORTED
    assert L.lora_expand(FAKE, 4, 256 + 32, FAKE, FAKE, FAKE, FAKE, 2, 8, FAKE, NULL) == UNSUPPORTED
    assert L.lora_pack_weight(0, FAKE, NULL, 128, 256 + 32, MISALIGNED, NULL, NULL) == UNSUPPORTED
    # adapters: any rank 1..64 packs; 65 and up are unsupported, 0 and below invalid
    A, B, At, Bt = (ctypes.c_void_p(0x10000 * i) for i in (1, 2, 3, 4))
    assert L.lora_pack_adapter(A, B, 4096, 6144, 65, At, Bt, NULL) == UNSUPPORTED
    assert L.lora_pack_adapter(A, B, 4096, 6144, 0, At, Bt, NULL) == INVALID
    assert L.lora_pack_adapter(A, B, 0, 6144, 4, At, Bt, NULL) == INVALID
    assert L.lora_pack_adapter(NULL, B, 4096, 6144, 4, At, Bt, NULL) == INVALID
    assert L.lora_pack_adapter(A, B, 4096, 6144, 4, MISALIGNED, Bt, NULL) == INVALID
    assert L.lora_pack_adapter(A, B, 4096, 6144, 4, A, Bt, NULL) == INVALID      # not in place
    big = ctypes.c_void_p(0x10000 + 4096 * 4 * 2 - 16)                          # overlaps the end of A
    assert L.lora_pack_adapter(A, B, 4096, 6144, 4, big, ctypes.c_void_p(0x4000000), NULL) == INVALID


def test_rank_pad_matches_header():
    import precision_gemm_amd as P
    assert [P.rank_pad(r) for r in (1, 4, 7, 8, 9, 12, 20, 60, 64)] == [8, 8, 8, 8, 16, 16, 24, 64, 64]


def _noalloc(L, **kw):
    a = dict(x=FAKE, T=16, K=4096, N=6144, fmt=0, wq=FAKE, ws=FAKE, t=NULL, ids=FAKE, seg=FAKE, srt=FAKE,
             A=FAKE, B=FAKE, rk=FAKE, sc=FAKE, n=1, r=16, y=FAKE, flags=1, stream=NULL)
    a.update(kw)
    return L.gemm_lowp_lora_epilogue_noalloc(a["x"], a["T"], a["K"], a["N"], a["fmt"], a["wq"], a["ws"], a["t"],
                                             a["ids"], a["seg"], a["srt"], a["A"], a["B"], a["rk"], a["sc"], a["n"],
                                             a["r"], a["y"], a["flags"], a["stream"])


def test_noalloc_checks_before_touching_the_device(L):
    """The allocation-free call rejects sizes whose workspace exceeds its 32 MiB scratch, and
    every bad argument, on the host before its scratch is looked up."""
    SCRATCH_LIMIT = 6
    assert L.lora_workspace_bytes(8192, 8192, 8192, 8, 64) > (32 << 20)
    assert _noalloc(L, T=8192, K=8192, N=8192, n=8, r=64) == SCRATCH_LIMIT
    assert _noalloc(L, T=8192, K=8192, N=8192, n=8, r=64, flags=3) == SCRATCH_LIMIT
    assert L.lora_workspace_bytes(4096, 4096, 4096, 8, 64) <= (32 << 20)     # the prefill workload fits
    assert _noalloc(L, T=-1) == INVALID
    assert _noalloc(L, K=4000) == UNSUPPORTED
    assert _noalloc(L, r=65) == UNSUPPORTED
    assert _noalloc(L, flags=8) == INVALID
    assert _noalloc(L, flags=2) == INVALID
    assert _noalloc(L, T=0) == LORA_OK
    assert _noalloc(L, x=NULL) == INVALID
    assert _noalloc(L, y=MISALIGNED) == INVALID
    assert _noalloc(L, A=NULL) == INVALID
    assert L.lora_status_string(SCRATCH_LIMIT).startswith(b"sizes need more")


def test_shrink_configured_validation(L):
    cfg = lambda *v: (ctypes.c_int32 * 5)(*v)  # noqa: E731
    args = lambda c, **kw: (kw.get("x", FAKE), kw.get("T", 64), kw.get("K", 1024), FAKE, FAKE, FAKE, FAKE,  # noqa: E731
                            kw.get("n", 4), kw.get("r", 16), FAKE, c, NULL)
    assert L.lora_shrink_configured(*args(cfg(3, 1, 1, 16, 0))) == UNSUPPORTED     # TG
    assert L.lora_shrink_configured(*args(cfg(1, 8, 1, 16, 0))) == UNSUPPORTED     # JP
    assert L.lora_shrink_configured(*args(cfg(1, 1, 3, 16, 0))) == UNSUPPORTED     # U
    assert L.lora_shrink_configured(*args(cfg(1, 1, 1, 24, 0))) == UNSUPPORTED     # TBLK % 16
    assert L.lora_shrink_configured(*args(cfg(1, 1, 1, 16, 2))) == UNSUPPORTED     # ORDER
    assert L.lora_shrink_configured(*args(None)) == INVALID
    assert L.lora_shrink_configured(*args(cfg(1, 1, 1, 16, 0), x=NULL)) == INVALID
    assert L.lora_shrink_configured(*args(cfg(1, 1, 1, 16, 0), K=1000)) == UNSUPPORTED
    assert L.lora_shrink_configured(*args(cfg(1, 1, 1, 16, 0), r=65)) == UNSUPPORTED
    assert L.lora_shrink_configured(*args(cfg(1, 1, 1, 16, 0), T=0)) == LORA_OK
    out = (ctypes.c_int32 * 3)()
    assert L.lora_shrink_config_info(3, 1, 1, out) == UNSUPPORTED
    assert L.lora_shrink_config_info(1, 1, 1, None) == INVALID


def _bwd(L, **kw):
    a = dict(x=FAKE, dy=FAKE, t=FAKE, T=64, K=4096, N=4096, fmt=0, wt=FAKE, ws=FAKE, ids=FAKE, seg=FAKE, srt=FAKE,
             Bop=FAKE, Ar=FAKE, rk=FAKE, sc=FAKE, n=8, r=64, dx=FAKE, u=FAKE, dA=FAKE, dB=FAKE, status=NULL,
             work=NULL, work_bytes=0)
    a.update(kw)
    return L.lora_backward(a["x"], a["dy"], a["t"], a["T"], a["K"], a["N"], a["fmt"], a["wt"], a["ws"], a["ids"],
                           a["seg"], a["srt"], a["Bop"], a["Ar"], a["rk"], a["sc"], a["n"], a["r"], a["dx"], a["u"],
                           a["dA"], a["dB"], a["status"], a["work"], a["work_bytes"], NULL)


def test_backward_validation(L):
    """lora_backward and its packs: every limit of the header returns its status before
    anything is enqueued (the pointers here are fake)."""
    assert _bwd(L, fmt=1) == UNSUPPORTED          # MXFP4 base: not in the backward
    assert _bwd(L, fmt=2) == INVALID
    assert _bwd(L, K=4096 + 64) == UNSUPPORTED
    assert _bwd(L, N=4096 + 64) == UNSUPPORTED    # the contraction of dX runs in 128-channel pairs of steps
    assert _bwd(L, T=65537) == UNSUPPORTED
    assert _bwd(L, T=-1) == INVALID
    assert _bwd(L, r=65) == UNSUPPORTED
    assert _bwd(L, n=0) == INVALID
    assert _bwd(L, dA=NULL) == INVALID
    for name in ("x", "dy", "t", "wt", "ws", "ids", "seg", "srt", "Bop", "Ar", "dx", "u"):
        assert _bwd(L, **{name: NULL}) == INVALID, name
    for name in ("x", "dy", "wt", "ws", "dx", "u"):
        assert _bwd(L, **{name: MISALIGNED}) == INVALID, name
    # short batches split dX's contraction: the partial sums need the workspace the query names
    need = L.lora_backward_workspace_bytes(64, 4096, 4096, 8, 64)
    # 16 tiles: 16 ranges of 4 steps; u: 8 adapters at most, 16 parts of 256 channels
    assert need == 16 * 64 * 4096 * 4 + 16 * 64 * 64 * 4
    assert L.lora_backward_workspace_bytes(8192, 4096, 4096, 8, 64) == 0     # 2048 tiles fill the GPU, T > 128
    assert L.lora_backward_workspace_bytes(64, 4096, 4096 + 64, 8, 64) == 0  # sizes the call does not accept
    assert L.lora_backward_workspace_bytes(64, 4096, 4096, 8, 65) == 0
    assert _bwd(L) == WORKSPACE
    assert _bwd(L, work=FAKE, work_bytes=need - 1) == WORKSPACE
    assert _bwd(L, work=MISALIGNED, work_bytes=need) == WORKSPACE
    assert L.lora_pack_weight_t(1, FAKE, 4096, 4096, ctypes.c_void_p(0x4000000), NULL) == UNSUPPORTED
    assert L.lora_pack_weight_t(0, FAKE, 4096 + 64, 4096, ctypes.c_void_p(0x4000000), NULL) == UNSUPPORTED
    assert L.lora_pack_weight_t(0, FAKE, 4096, 4096, FAKE, NULL) == INVALID           # in place
    assert L.lora_pack_weight_t(0, FAKE, 4096, 4096, MISALIGNED, NULL) == INVALID
    A, B, O, R = (ctypes.c_void_p(0x1000000 * i) for i in (1, 2, 3, 4))
    assert L.lora_pack_adapter_bwd(A, B, 4096, 4096, 65, O, R, NULL) == UNSUPPORTED
    assert L.lora_pack_adapter_bwd(A, B, 4096, 4096 + 32, 8, O, R, NULL) == UNSUPPORTED
    assert L.lora_pack_adapter_bwd(A, B, 4096, 4096, 0, O, R, NULL) == INVALID
    assert L.lora_pack_adapter_bwd(A, B, 4096, 4096, 8, A, R, NULL) == INVALID         # not in place
    assert L.lora_pack_adapter_bwd(A, B, 4096, 4096, 8, MISALIGNED, R, NULL) == INVALID

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
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 12) == 0      # r_max % 8
    assert L.lora_workspace_bytes(16, 4096, 6144, 1, 128) == 0     # r_max > 64
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
    assert _gemm(L, r=12) == UNSUPPORTED
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

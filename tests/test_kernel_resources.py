"""Register and scratch use of the built layer kernels (from the compiler's
kernel-resource-usage remarks recorded by the build).

A scratch spill in a kernel stalls its loop on memory round trips (one spill of the t
gather once cost the prefill workload 15% of its time), so none may spill; the GEMM
kernels built for two workgroups per CU (16-bit-activation long batches, the backward's
dX) must fit two.  Skipped when the library was built without the record."""

import pytest

from precision_gemm_amd import build as B


def _layer_kernels():
    res = B.resources()
    if not res:
        pytest.skip("no resource record (run precision_gemm_amd.build first)")
    return {k: v for k, v in res.items() if "k_layer" in k}


def test_layer_kernels_do_not_spill():
    ks = _layer_kernels()
    assert ks, "no layer kernel in the resource record"
    bad = {k: v.get("ScratchSize [bytes/lane]") for k, v in ks.items() if v.get("ScratchSize [bytes/lane]", 0) != 0}
    assert not bad, f"layer kernels using scratch: {bad}"


def test_layer_kernels_fit_their_occupancy():
    # 64-token prefill tiles are compiled for two workgroups per CU, the others for one
    for name, v in _layer_kernels().items():
        assert v.get("Occupancy [waves/SIMD]", 0) >= 1, name
        assert v.get("VGPRs", 0) <= 256 and v.get("AGPRs", 0) <= 256, name


def test_no_kernel_spills():
    res = B.resources()
    if not res:
        pytest.skip("no resource record (run precision_gemm_amd.build first)")
    bad = {k: v.get("ScratchSize [bytes/lane]") for k, v in res.items() if v.get("ScratchSize [bytes/lane]", 0) != 0}
    assert not bad, f"kernels using scratch: {bad}"


@pytest.mark.parametrize("name", ["k_gemm_a16", "k_bwd_dx"])
def test_two_workgroups_per_cu(name):
    res = B.resources()
    if not res:
        pytest.skip("no resource record (run precision_gemm_amd.build first)")
    ks = {k: v for k, v in res.items() if name in k}
    assert ks, f"{name} not in the resource record"
    for k, v in ks.items():
        # 256 threads = four waves, one per SIMD: two workgroups need two waves per SIMD
        assert v.get("Occupancy [waves/SIMD]", 0) >= 2, (k, v)

// Internal interface between the C-ABI host layer (lora_api.cpp) and the gfx950
// kernels (lora_kernels.hip).  Not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/lora_lowp.h"

namespace lora {

constexpr int SEG_THREADS = 1024;
constexpr int MAX_ADAPTERS = 8192;
constexpr int MAX_RANK = 64;

struct ShrinkParams {
  const uint16_t* x;
  int T, K;
  const int* seg_indptr;
  const int* sorted_tok;
  const uint64_t* A_ptrs;  // A_a^T, bf16 [r_a][K]
  const int* ranks;
  int n_ad, r_max;
  float* t;     // [T][r_max], original token order
  float* part;  // [nchunks][T][r_max], rows in sorted order (split-K partial sums)
  int* ad_ctr;  // [n_ad] arrival counters, zero between calls
  int KC, nchunks;
};

struct GemmParams {
  const uint16_t* x;   // bf16 [T][K]
  const uint8_t* xq;   // pre-quantised MXFP8 codes (XQ kernels)
  const uint8_t* xsc;  // and scales
  int T, K, N;
  const uint8_t* wq;
  const float* ws_fp8;   // FP8 channel scales [N]
  const uint8_t* ws_fp4; // MXFP4 block scales [N][K/32]
  const float* t;        // [T][r_max]
  int r_max;
  const int* ids;
  const uint64_t* B_ptrs;  // B_a^T, bf16 [N][r_a]
  const int* ranks;
  const float* scales;
  int n_ad;
  uint16_t* y;
  int ksplit, krange, n_cb, n_tb;
  float* gpart;   // K-split partial accumulators
  int* tile_ctr;  // [tiles] arrival counters
  int lora;       // add the adapter term
  int n_shrink;   // down-projection workgroups in the same launch (0: none)
  int* shrink_done;
  int* wait_done;
  int* status;
  int spin_limit;
};

struct ExpandParams {
  const float* t;
  int T, N, r_max, n_ad;
  const int* ids;
  const uint64_t* B_ptrs;
  const int* ranks;
  const float* scales;
  uint16_t* y;
};

// Tile plan for one (T, K, N, n_adapters, r_max, format); a pure function of these.
struct LayerPlan {
  int fmt;
  int TT, CT;       // token tiles of 16 per workgroup, column tiles of 16 per wave
  bool XQ;          // x is quantised by a separate pass into the workspace
  int KC;           // K-chunk staged in LDS
  int ksplit, krange, n_cb, n_tb, n_gemm_wg;
  int shrink_KC, shrink_nchunks, shrink_tg, n_shrink_wg;
  // workspace layout (byte offsets)
  size_t off_ctrl, off_adctr, off_tilectr, off_spart, off_t, off_gpart, off_xq, off_xsc, total;
};

hipError_t launch_build_segments(const int* ids, int T, int n_ad, int* seg, int* sorted, int* err, hipStream_t s);
hipError_t launch_quant(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s);
hipError_t launch_shrink(int tg, int grid, hipStream_t stream, const ShrinkParams& sp);
hipError_t launch_expand(const ExpandParams& p, hipStream_t s);
hipError_t launch_layer(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp, const GemmParams& gp);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace lora

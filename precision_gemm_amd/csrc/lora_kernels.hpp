// Internal interface between the C-ABI host layer (lora_api.cpp) and the gfx950
// kernels (lora_kernels.hip).  Not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/lora_lowp.h"

namespace lora {

constexpr int MAX_ADAPTERS = 8192;
constexpr int MAX_RANK = 64;

// Workspace control block (int32 words at the start of every workspace)
enum : int {
  CTRL_EPOCH = 0,    // number of fused launches completed on this workspace (tag = epoch + 1)
  CTRL_STARTED = 1,  // workgroups of the current launch that have read the epoch
  CTRL_STATUS = 2,   // non-zero: a bounded wait gave up
  CTRL_SEGREADY = 3, // tag of the launch whose segment builder has finished
  CTRL_SEGERR = 4,   // error word of the last in-launch segment build
};

struct ShrinkParams {
  const uint16_t* x;
  int T, K;
  const int* seg_indptr;
  const int* sorted_tok;
  const int* ids;          // fused launch with T <= 16: tokens found by id (may be null)
  const uint64_t* A_ptrs;  // A_a^T, bf16 [r_a][K]
  const int* ranks;
  int n_ad, r_max;
  float* t_out;        // plain fp32 [T][r_max] (may be null in the fused launch)
  uint64_t* t_tag;     // tagged [kparts][T][r_max] (fused launch only, else null)
  int t_pack;          // t_tag holds [T][r_max / 2] tagged bf16 pairs of s_a t (one K-part)
  const float* scales; // adapter scales (for the pairs)
  int tblk;            // tokens of one segment per workgroup item (multiple of 16)
  int n_tblk;          // token blocks per adapter
  int n_jg;            // rank groups per adapter (16 * jper ranks each)
  int jper;            // 16-rank tiles per group (1..4)
  int kparts, kpart_len;
  int seg_wait;        // the segments are built in the same launch: wait for them, read them coherently
  int compact;         // fused launch: workgroups loop over the items with tokens (long batches)
  int compact_off;     // LDS byte offset of the block prefix (after the down-projection's area)
  int spin_limit;
};

struct GemmParams {
  const uint16_t* x;   // bf16 [T][K]
  const uint8_t* xq;   // pre-quantised MXFP8 codes (XQ kernels)
  const uint8_t* xsc;  // and scales
  int T, K, N;
  const uint8_t* wq;
  const float* ws_fp8;    // FP8 channel scales [N]
  const uint8_t* ws_fp4;  // MXFP4 block scales [N][K/32]
  const float* t;         // plain t (unfused), or null
  float* t_out;           // fused launch: the caller's t, written when t_kparts > 1 (may be null)
  const uint64_t* t_tag;  // tagged t partials (fused), or null
  int t_kparts;
  int t_pack;             // t_tag holds tagged bf16 pairs of s_a t (see ShrinkParams)
  int r_max;
  const int* ids;
  const uint64_t* B_ptrs;  // B_a^T, bf16 [N][r_a]
  const int* ranks;
  const float* scales;
  int n_ad;
  uint16_t* y;
  int ksplit, krange, n_cb, n_tb;
  float* gpart;    // K-split partial accumulators
  int* gflag;      // [tiles][ksplit] tags of finished K-split producers
  int lora;        // add the adapter term
  int n_shrink;    // down-projection workgroups at the front of the grid
  int* ctrl;       // workspace control block
  int spin_limit;
  int* seg_build;     // non-null: workgroup 0 builds seg_indptr (here) and sorted_tok from ids
  int* sorted_build;
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
  int TT, CT, WC, WK;  // token tiles per workgroup, column tiles per wave, wave grid (columns x k)
  bool XQ;             // x is quantised by a separate pass into the workspace
  int s_cfg;           // down-projection tile shape: 0 decode, 1 prefill
  int occ = 1;         // workgroups per CU the one-tile stream kernel is built for
  bool a16 = false;    // base product on the bf16 activations as they are (bf16 MFMA)
  int KC;              // K-chunk staged in LDS
  int ksplit, krange, n_cb, n_tb, n_gemm_wg;
  // down-projection decomposition
  int s_tblk, s_ntblk, s_njg, s_jper, s_kparts, s_kpart_len, n_shrink_wg;
  int n_shrink_items;  // down-projection items (the standalone launch has one workgroup each)
  bool compact;        // fused launch: the down-projection workgroups take the items that have work
  int n_build_wg;  // 1 when the launch also builds the segments
  // workspace layout (byte offsets)
  size_t off_ctrl, off_ttag, off_gflag, off_gpart, off_xq, off_xsc, total;
};

hipError_t launch_build_segments(const int* ids, int T, int n_ad, int* seg, int* sorted, int* err, hipStream_t s);
hipError_t launch_quant(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s);
// the segment builder and the MXFP8 pre-pass in one launch (independent of each other)
hipError_t launch_quant_build(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, const int* ids, int n_ad,
                              int* seg, int* sorted, int* err, hipStream_t s);
hipError_t launch_shrink(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp);
hipError_t launch_expand(const ExpandParams& p, hipStream_t s);
hipError_t launch_layer(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp, const GemmParams& gp);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_pack_weight(int fmt, const uint8_t* q, const uint8_t* sc, int N, int K, uint8_t* qp, uint8_t* scp,
                              hipStream_t s);

}  // namespace lora

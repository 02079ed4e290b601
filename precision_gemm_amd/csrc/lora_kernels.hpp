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

// Stored adapters (lora_pack_adapter; padding zero-filled, and masked out by the kernels
// whatever it holds): B_a^T has rank_pad(r_a) columns (whole 16-byte runs of bf16); A_a is
// stored in bf16 MFMA operand order for rank tiles of 16 (a_tiles(r_a) of them): element
// (j, k) of A_a^T at a_index(j, k, K), so that the 16-byte lane loads of one rank tile and
// one 64-wide k-step read 2 KB of consecutive memory (lane l = 16 g + i: rank 16 jt + i,
// k = 64 ks + 16 g + 8 h .. + 7 for the halves h = 0, 1).
__host__ __device__ constexpr int rank_pad(int r) { return (r + 7) & ~7; }
__host__ __device__ constexpr int a_tiles(int r) { return (r + 15) >> 4; }
__host__ __device__ constexpr long a_index(int j, int k, int K) {
  return ((((long)(j >> 4) * (K >> 6) + (k >> 6)) * 2 + ((k >> 3) & 1)) * 64 + 16 * ((k >> 4) & 3) + (j & 15)) * 8 +
         (k & 7);
}
// offset (elements) of rank tile jt, k-step ks (64 wide), half h, lane l
__host__ __device__ constexpr long a_tile_off(int jt, int ks, int h, int K) {
  return (((long)jt * (K >> 6) + ks) * 2 + h) * 512;
}

// MXFP8 activations in the long-batch GEMM's operand order (k_gemm_pf), KS = K / 128:
// codes [row tile of 16][KS][half h][lane][16 B], lane l = 16 g + i holding row i at
// k = 128 ks + 64 h + 16 g .. + 15 (the scaled MFMA's operand, 1 KB per tile and half);
// scale codes [row group of 64][KS][lane][4 B], byte tt of lane l = 16 g + i the code of
// row 16 tt + i, K-block 4 ks + g (one word is the scale operand of four row tiles).
__host__ __device__ constexpr long pf_xq_off(int row, int kk, int KS) {
  return ((((long)(row >> 4) * KS + (kk >> 7)) * 2 + ((kk >> 6) & 1)) * 64 + 16 * ((kk >> 4) & 3) + (row & 15)) * 16 +
         (kk & 15);
}
__host__ __device__ constexpr long pf_xsc_off(int row, int blk, int KS) {
  return (((long)(row >> 6) * KS + (blk >> 2)) * 64 + 16 * (blk & 3) + (row & 15)) * 4 + ((row >> 4) & 3);
}

// The long-batch pre-pass (k_prep_pf) splits the down-projection's K into PF_KP parts and
// writes their partial sums as fp32 [PF_KP][T][PF_TPS]; k_gemm_pf's epilogue adds them in
// part order.
constexpr int PF_KP = 4, PF_TPS = 64;

// Workspace control block (int32 words at the start of every workspace)
enum : int {
  CTRL_EPOCH = 0,    // number of fused launches completed on this workspace (tag = epoch + 1)
  CTRL_STARTED = 1,  // workgroups of the current launch that have read the epoch
  CTRL_STATUS = 2,   // bit 0: a bounded wait gave up; bit 1: an adapter's rank was outside [1, r_max]
  CTRL_SEGREADY = 3, // tag of the launch whose segment builder has finished
  CTRL_SEGERR = 4,   // error word of the last in-launch segment build
};

struct ShrinkParams {
  const uint16_t* x;
  int T, K;
  const int* seg_indptr;
  const int* sorted_tok;
  const int* ids;          // fused launch with T <= 16: tokens found by id (may be null)
  const uint64_t* A_ptrs;  // A_a in operand order (a_index), a_tiles(r_a) rank tiles
  const int* ranks;
  int n_ad;
  int r_max;           // rank_pad of the caller's r_max: row stride of the tagged t
  int r_lim;           // the caller's r_max: largest valid rank, row stride of t_out
  float* t_out;        // plain fp32 [T][r_lim] (may be null in the fused launch)
  float* t_part;       // standalone launch with K-parts: plain fp32 partial sums [kparts][T][r_lim] (else null)
  uint64_t* t_tag;     // tagged [kparts][T][r_max] (fused launch only, else null)
  int t_pack;          // t_tag holds [T][r_max / 2] tagged bf16 pairs of s_a t (one K-part)
  const float* scales; // adapter scales (for the pairs)
  int tblk;            // tokens of one segment per workgroup item (multiple of 16)
  int n_tblk;          // token blocks per adapter
  int n_jg;            // rank groups per adapter (16 * jper ranks each)
  int jper;            // 16-rank tiles per group (1..4)
  int kparts, kpart_len;
  int item_order;      // standalone launch: 0 items in id order, 1 each XCD a contiguous run of items
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
  const float* t;         // plain t [T][r_lim] (unfused), or null; k_gemm_pf: the pre-pass's
                          // partial sums [PF_KP][T][PF_TPS] when t_kparts == PF_KP
  float* t_out;           // fused launch: the caller's t, written when t_kparts > 1 (may be null);
                          // k_gemm_pf: written by the tiles of column block 0 (may be null)
  const uint64_t* t_tag;  // tagged t partials (fused), or null
  int t_kparts;
  int t_pack;             // t_tag holds tagged bf16 pairs of s_a t (see ShrinkParams)
  int r_max;              // rank_pad of the caller's r_max (internal row stride of t)
  int r_lim;              // the caller's r_max (largest valid rank, row stride of t and t_out)
  const int* ids;
  const uint64_t* B_ptrs;  // B_a^T, bf16 [N][rank_pad(r_a)]
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
  int tile_group;     // > 0: XCD-grouped tile order, groups of this many column blocks
  int rot;            // tiles start their K walk at different chunks (spreads HBM channels)
};

struct ExpandParams {
  const float* t;      // [T][r_lim]
  int T, N, r_lim, n_ad;
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
  bool rows16 = false; // a16 long batch (FP8, N % 256 == 0): t by the rows pre-pass, then k_gemm_a16
  bool pf = false;     // long MXFP8 batch (FP8, K and N % 512 == 0, enough tiles): 128 x 512 tiles of
                       // k_gemm_pf on x in operand order (pf_xq_off, pf_xsc_off)
  int KC;              // K-chunk staged in LDS
  int ksplit, krange, n_cb, n_tb, n_gemm_wg;
  // down-projection decomposition
  int s_tblk, s_ntblk, s_njg, s_jper, s_kparts, s_kpart_len, n_shrink_wg;
  int n_shrink_items;  // down-projection items (the standalone launch has one workgroup each)
  bool compact;        // fused launch: the down-projection workgroups take the items that have work
  int n_build_wg;  // 1 when the launch also builds the segments
  // workspace layout (byte offsets); tpl: plain fp32 t of a down-projection run in the
  // pre-pass launch
  size_t off_ctrl, off_ttag, off_gflag, off_gpart, off_xq, off_xsc, off_tpl, total;
};

hipError_t launch_build_segments(const int* ids, int T, int n_ad, int* seg, int* sorted, int* err, hipStream_t s);
hipError_t launch_quant(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s);
// the same quantisation written in the long-batch GEMM's operand order (pf_xq_off, pf_xsc_off)
hipError_t launch_quant_pf(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s);
// the long-batch GEMM: 128 x 512 tiles, eight waves, W into registers, x copied to LDS (k_gemm_pf)
hipError_t launch_gemm_pf(const GemmParams& gp, hipStream_t s);
// the 16-bit-activation GEMM of a long batch: 64 x 256 tiles, FP8 W (N % 256 == 0), plain t
hipError_t launch_gemm_a16(const GemmParams& gp, hipStream_t s);
// the segment builder and the MXFP8 pre-pass in one launch (independent of each other)
// the MXFP8 pre-pass with the down-projection items (plan with 64-token items) beside it
hipError_t launch_quant_shrink(const LayerPlan& pl, const ShrinkParams& sp, const uint16_t* x, int T, int K, uint8_t* xq,
                               uint8_t* xsc, hipStream_t s);
// the pre-pass's down-projection alone over 16-position blocks of the sorted order (no
// quantisation): t_out plain, sp.ids the per-token adapter ids
hipError_t launch_shrink_rows(const ShrinkParams& sp, hipStream_t s);
hipError_t launch_quant_build(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, const int* ids, int n_ad,
                              int* seg, int* sorted, int* err, hipStream_t s);
hipError_t launch_shrink(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp);
hipError_t launch_expand(const ExpandParams& p, hipStream_t s);
// the per-token merged-weight layer (an alternative formulation to ablate against)
hipError_t launch_merged(const uint16_t* x, int T, int K, int N, int fmt, const uint8_t* wq, const void* wscale,
                         const int* ids, const uint64_t* A_rows, const uint64_t* B_ptrs, const int* ranks,
                         const float* scales, int n_ad, int r_lim, uint16_t* y, hipStream_t s);
// the standalone down-projection with an explicit configuration (tuning): TG token tiles and
// JP rank tiles per inner step, U k-steps per prefetch buffer (compiled for TG, JP in
// {1, 2, 4}, U in {1, 2}); one workgroup per item.  shrink_cfg_attr: the instance's registers
// per lane, scratch (spill) bytes per lane and LDS bytes.
hipError_t launch_shrink_cfg(int tg, int jp, int u, int grid, hipStream_t s, const ShrinkParams& sp);
hipError_t shrink_cfg_attr(int tg, int jp, int u, int* regs, int* spill, int* lds);
// the wave-reduction (BGMV) down-projection: NT positions of a segment and JP rank tiles per
// workgroup, U k-steps per buffer (compiled for NT in {1, 2, 4} with JP in {1, 2, 4} and U = 1,
// and NT = 1 with U = 2); one workgroup per item (adapter, token block, rank group)
hipError_t launch_shrink_bgmv(int nt, int jp, int u, int grid, hipStream_t s, const ShrinkParams& sp);
hipError_t shrink_bgmv_attr(int nt, int jp, int u, int* regs, int* spill, int* lds);
hipError_t launch_layer(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp, const GemmParams& gp);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_pack_weight(int fmt, const uint8_t* q, const uint8_t* sc, int N, int K, uint8_t* qp, uint8_t* scp,
                              hipStream_t s);
// Allocation-free layer call: bytes of the per-device scratch array, and its device
// address on the current device (looked up on first use, when the array is also
// zero-filled on `s`; the tagged hand-over area [tag_lo, tag_hi) is zero-filled again on
// `s` whenever it differs from the previous call's on this device).
constexpr size_t SCRATCH_BYTES = (size_t)LORA_NOALLOC_SCRATCH_BYTES;
hipError_t scratch_acquire(hipStream_t s, size_t tag_lo, size_t tag_hi, void** out);
// Backward (lora_backward.hip).  dX = dY W_d^T + s_a u A_a^T: 64 x 256 tiles, W^T packed
// by launch_pack_weight_t, A_a rows [K][rank_pad(r_a)] (launch_pack_adapter_bwd).
struct BwdDxParams {
  const uint16_t* dy;      // bf16 [T][N]
  const uint8_t* wt;       // W^T FP8 codes, packed
  const float* wsc;        // channel scales [N]
  int T, K, N;
  const float* u;          // [T][r_lim]: dY B_a^T
  int r_lim;
  const int* ids;
  const uint64_t* Ar_ptrs;
  const int* ranks;
  const float* scales;
  int n_ad;
  uint16_t* dx;            // bf16 [T][K]
  int n_tb, n_kb;          // 64-row and 256-column blocks
  int n_split, split_steps;  // the contraction over N in n_split ranges of split_steps 64-wide steps
  float* part;             // n_split > 1: fp32 partial sums [n_split][T][K] (the adapter term in range 0)
};
// dA_a = s_a X_a^T U_a [K][r_a] and dB_a = s_a T_a^T dY_a [r_a][N]: one workgroup per
// (adapter, 64 rows of K) and (adapter, 64 columns of N).
struct BwdGradParams {
  const uint16_t* x;       // bf16 [T][K]
  const uint16_t* dy;      // bf16 [T][N]
  const float* u;          // [T][r_lim]
  const float* t;          // [T][r_lim]: the forward's down-projection
  int T, K, N, r_lim;
  const int* seg_indptr;
  const int* sorted_tok;
  int empty;               // no tokens: every gradient is zero (segments not read)
  const int* ranks;
  const float* scales;
  int n_ad;
  const uint64_t* dA_ptrs;
  const uint64_t* dB_ptrs;
  int nkb, nnb;
  int* status;             // bit 1 OR-ed in for an adapter with tokens and a rank outside [1, r_lim]
};
hipError_t launch_pack_weight_t(const uint8_t* q, int N, int K, uint8_t* qt, hipStream_t s);
hipError_t launch_pack_adapter_bwd(const uint16_t* A, const uint16_t* B, int K, int N, int r, uint16_t* Bop,
                                   uint16_t* Ar, hipStream_t s);
hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s);
hipError_t launch_bwd_grad(const BwdGradParams& p, hipStream_t s);
// dx = bf16 of the partial sums added in range order (n_split > 1)
hipError_t launch_bwd_dx_reduce(const BwdDxParams& p, hipStream_t s);
// out[tok][j] = the K-parts of part [kparts][T][r_lim] added in order for j < r_a, 0 for
// r_a <= j < r_lim; tokens without a valid adapter or rank are left as they are
hipError_t launch_part_reduce(const float* part, int kparts, int T, int r_lim, const int* ids, const int* ranks,
                              int n_ad, float* out, hipStream_t s);
hipError_t launch_pack_adapter(const uint16_t* A, const uint16_t* B, int K, int N, int r, uint16_t* At, uint16_t* Bt,
                               hipStream_t s);

}  // namespace lora

// C-ABI host layer: argument checks, the tile plan, workspace layout and launches.
// Every check runs before anything is enqueued; nothing here allocates or synchronises.
#include <stdint.h>
#include <string.h>

#include "lora_kernels.hpp"

using namespace lora;

namespace {

constexpr int SPIN_LIMIT = 1 << 23;  // bounded waits in the fused launch (about a second)
// down-projection workgroups of a fused launch of 17 to 128 tokens: one per CU at most, the
// items beyond are looped over (fewer workgroups, so that GEMM workgroups could start beside
// them, measured slower: the A stream wants every CU)
constexpr int SHRINK_CAP = 256;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t round256(size_t v) { return (v + 255) & ~size_t(255); }
inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
inline int pow2_floor(long v) {
  int p = 1;
  while ((long)p * 2 <= v) p *= 2;
  return p;
}

lora_status check_sizes(int32_t T, int32_t K, int32_t N) {
  if (T < 0 || K <= 0 || N <= 0) return LORA_ERR_INVALID_ARG;
  if (T > 65536 || K % 128 != 0 || N % 64 != 0) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

lora_status check_adapters(int32_t n_adapters, int32_t r_max) {
  if (n_adapters < 1 || r_max < 1) return LORA_ERR_INVALID_ARG;
  if (n_adapters > MAX_ADAPTERS || r_max > MAX_RANK || r_max % 8 != 0) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

// Tile plan: a pure function of the sizes, so lora_workspace_bytes and every call agree.
// fused: the down-projection runs in the layer launch (its K may then be split into parts
// that the GEMM epilogue adds up); otherwise it runs alone and writes the final t.
// a16: 16-bit activations: the one-tile stream up to 16 tokens, 64 x 128 tiles with bf16 x
// staged in LDS above (where N % 128 == 0; otherwise 16-token tiles of the stream, whose
// token tiles of a column tile share an XCD's L2 for W).
LayerPlan make_plan(int T, int K, int N, int n_ad, int r_max, int fmt, bool fused = true, bool a16 = false) {
  LayerPlan pl{};
  pl.fmt = fmt;
  pl.a16 = a16;
  if (a16 && T > 16 && N % 128 == 0) {
    pl.TT = 4; pl.CT = 2; pl.WC = 4; pl.WK = 1; pl.XQ = false;
  } else if (T <= 16 || a16) {
    // one-tile stream, built for two workgroups per CU (its registers and LDS fit): the
    // down-projection's few workgroups then share CUs with the GEMM's (Llama-3-8B QKV decode:
    // 14.05 to 14.13 us per step against 14.27 to 14.44)
    pl.TT = 1; pl.CT = 2; pl.WC = 1; pl.WK = 4; pl.XQ = false; pl.occ = 2;
  } else if (T <= 64) {
    // 128 channels per workgroup: with the down-projection's workgroups the grid stays
    // within one workgroup per CU for the widest decode layers.  x is quantised once by a
    // pre-pass: every workgroup reads all of x, and MXFP8 halves those reads (measured: the
    // pass pays for its launch at 64 tokens, not at 16)
    pl.TT = 4; pl.CT = (N % 128 == 0) ? 2 : 1; pl.WC = 4; pl.WK = 1; pl.XQ = (pl.CT == 2);
  } else {
    // 128 tokens per tile: x is quantised once by a pre-pass (every column tile reads
    // it), and 128 channels per workgroup halve those reads
    pl.TT = 8; pl.WC = 4; pl.WK = 1; pl.XQ = true;
    pl.CT = (N % 128 == 0) ? 2 : 1;
    // prefill: 128 x 256 tiles (each wave 128 tokens x 64 channels: four times the MFMAs
    // per LDS read of x of the 128-channel tile), one workgroup per CU; where N is not a
    // multiple of 256, 64-token tiles with two workgroups per CU, so that one workgroup's
    // start-up and epilogue latency overlaps the other's main loop
    if (T > 128 && N % 256 == 0) {
      pl.CT = 4;
    } else if (T > 128 && pl.CT == 2) {
      pl.TT = 4;
    }
  }
  pl.KC = (pl.TT == 1) ? 2048 : ((pl.TT <= 4 && pl.CT == 1) ? 512 : (pl.CT == 4 ? 128 : 256));
  const int WN = pl.WC * pl.CT * 16;
  pl.n_cb = N / WN;
  pl.n_tb = ceil_div(T, 16 * pl.TT);
  const int tiles = pl.n_cb * pl.n_tb;
  const int max_split = std::max(1, K / pl.KC);
  // split K over workgroups only when there are too few tiles to fill the GPU: the
  // split-K hand-over adds dependent memory round trips to the critical path.  The GEMM
  // workgroups fill at most seven eighths of the 256 CUs, so that they all start beside
  // the last down-projection workgroups (measured on the 42-tile down-projection, µs per
  // step: 5 splits 112.6, 4 splits 122.4, 6 splits 131.3, 7 splits 138.7, 10 splits 135.7)
  int ks = (tiles >= 128) ? 1 : std::min(max_split, std::max(1, 224 / tiles));
  ks = std::max(ks, 1);
  pl.krange = ceil_div(ceil_div(K, ks), pl.KC) * pl.KC;
  pl.ksplit = ceil_div(K, pl.krange);
  pl.n_gemm_wg = tiles * pl.ksplit;

  // down-projection: item = (adapter, token block, group of 16*jper ranks, K-part)
  int kparts = 1;
  if (T <= 128) {
    pl.s_cfg = 0;
    pl.s_tblk = ceil_div(T, 16) * 16;
    pl.s_ntblk = 1;
    pl.s_jper = 1;
    pl.s_njg = ceil_div(r_max, 16);
    // latency-bound single-tile decode: split K so that t is ready early (measured: for the
    // 128-token shapes K-parts only add per-item start-up round trips)
    if (fused && T <= 16) kparts = std::min(4, std::max(1, K / 1024));
  } else {
    pl.s_cfg = 1;
    pl.s_tblk = 64;
    pl.s_ntblk = ceil_div(T, 64);
    pl.s_jper = 2;
    pl.s_njg = ceil_div(r_max, 32);
  }
  pl.s_kpart_len = ceil_div(ceil_div(K, kparts), 256) * 256;
  pl.s_kparts = ceil_div(K, pl.s_kpart_len);
  pl.n_shrink_items = n_ad * pl.s_ntblk * pl.s_njg * pl.s_kparts;
  // fused launch past 16 tokens: the down-projection workgroups take only the items that
  // have work (an idle workgroup still holds a CU the GEMM workgroups need).  The segments
  // of T tokens fill at most ceil(T / tblk) + min(n_ad, T) token blocks (each adapter adds
  // at most one partial block).  Short batches cap the workgroups at SHRINK_CAP.
  const int max_items = (ceil_div(T, pl.s_tblk) + std::min(n_ad, T)) * pl.s_njg * pl.s_kparts;
  pl.compact = fused && T > 16;
  pl.n_shrink_wg = pl.compact ? std::min({pl.n_shrink_items, max_items, pl.s_cfg == 1 ? 1 << 30 : SHRINK_CAP})
                              : pl.n_shrink_items;

  size_t off = 0;
  pl.off_ctrl = off;  off += 256;
  pl.off_ttag = off;  off += round256((size_t)pl.s_kparts * T * r_max * 8);
  pl.off_gflag = off; off += round256((size_t)tiles * pl.ksplit * 4);
  pl.off_gpart = off;
  if (pl.ksplit > 1) off += round256((size_t)tiles * pl.ksplit * pl.WC * pl.TT * pl.CT * 256 * 4);
  pl.off_xq = off;    if (pl.XQ) off += round256((size_t)T * K);
  pl.off_xsc = off;   if (pl.XQ) off += round256((size_t)T * (K / 32) + 8);  // + 8: padding read by a partial last chunk
  pl.total = off;
  return pl;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or format)";
    case LORA_ERR_UNSUPPORTED: return "unsupported size (see the limits in lora_lowp.h)";
    case LORA_ERR_WORKSPACE: return "workspace missing or too small";
    case LORA_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

const char* lora_version(void) { return "lora_lowp gfx950 kernels v1 (scaled-MFMA base GEMM, bf16-MFMA adapters)"; }

size_t lora_workspace_bytes(int32_t T, int32_t K, int32_t N, int32_t n_adapters, int32_t r_max) {
  if (check_sizes(T, K, N) != LORA_OK || check_adapters(n_adapters, r_max) != LORA_OK) return 0;
  if (T == 0) return 256;
  // the larger of the two plans (MXFP8 and 16-bit activations)
  return std::max(make_plan(T, K, N, n_adapters, r_max, LORA_W_FP8_E4M3).total,
                  make_plan(T, K, N, n_adapters, r_max, LORA_W_FP8_E4M3, true, true).total);
}

lora_status lora_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || !aligned16(workspace)) return LORA_ERR_INVALID_ARG;
  return launch_fill_zero(workspace, workspace_bytes, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_workspace_status(const void* workspace, int32_t* status_dev, void* stream) {
  if (!workspace || !status_dev) return LORA_ERR_INVALID_ARG;
  const char* ctrl = reinterpret_cast<const char*>(workspace);
  hipError_t e = hipMemcpyAsync(status_dev, ctrl + 8, 4, hipMemcpyDeviceToDevice, as_stream(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_workspace_segment_error(const void* workspace, int32_t* err_dev, void* stream) {
  if (!workspace || !err_dev) return LORA_ERR_INVALID_ARG;
  const char* ctrl = reinterpret_cast<const char*>(workspace);
  hipError_t e = hipMemcpyAsync(err_dev, ctrl + 4 * CTRL_SEGERR, 4, hipMemcpyDeviceToDevice, as_stream(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_build_segments(const int32_t* adapter_id, int32_t T, int32_t n_adapters, int32_t* seg_indptr,
                                int32_t* sorted_tok, int32_t* err_word, void* stream) {
  if (T < 0 || n_adapters < 1) return LORA_ERR_INVALID_ARG;
  if (T > 65536 || n_adapters > MAX_ADAPTERS) return LORA_ERR_UNSUPPORTED;
  if (!seg_indptr || !err_word) return LORA_ERR_INVALID_ARG;
  if (T > 0 && (!adapter_id || !sorted_tok)) return LORA_ERR_INVALID_ARG;
  hipError_t e = launch_build_segments(adapter_id, T, n_adapters, seg_indptr, sorted_tok, err_word, as_stream(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_quant_act_mxfp8(const uint16_t* x, int32_t T, int32_t K, uint8_t* x_q, uint8_t* x_sc,
                                 void* stream) {
  if (T < 0 || K <= 0) return LORA_ERR_INVALID_ARG;
  if (K % 32 != 0 || T > 65536) return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;
  if (!x || !x_q || !x_sc || !aligned16(x) || !aligned16(x_q)) return LORA_ERR_INVALID_ARG;
  return launch_quant(x, T, K, x_q, x_sc, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_shrink(const uint16_t* x, int32_t T, int32_t K, const int32_t* seg_indptr,
                        const int32_t* sorted_tok, const uint64_t* A_ptrs, const int32_t* ranks,
                        int32_t n_adapters, int32_t r_max, float* t, void* workspace, size_t workspace_bytes,
                        void* stream) {
  (void)workspace;
  (void)workspace_bytes;  // the standalone down-projection needs no scratch memory
  lora_status st = check_sizes(T, K, 64);
  if (st != LORA_OK) return st;
  if ((st = check_adapters(n_adapters, r_max)) != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  if (!x || !seg_indptr || !sorted_tok || !A_ptrs || !ranks || !t) return LORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(t)) return LORA_ERR_INVALID_ARG;
  const LayerPlan pl = make_plan(T, K, 64, n_adapters, r_max, LORA_W_FP8_E4M3, /*fused=*/false);
  ShrinkParams sp{};
  sp.x = x; sp.T = T; sp.K = K;
  sp.seg_indptr = seg_indptr; sp.sorted_tok = sorted_tok;
  sp.A_ptrs = A_ptrs; sp.ranks = ranks; sp.n_ad = n_adapters; sp.r_max = r_max;
  sp.ids = nullptr;  // standalone: tokens come from the segments only
  sp.t_out = t; sp.t_tag = nullptr;
  sp.tblk = pl.s_tblk; sp.n_tblk = pl.s_ntblk; sp.n_jg = pl.s_njg; sp.jper = pl.s_jper;
  sp.kparts = pl.s_kparts; sp.kpart_len = pl.s_kpart_len;
  hipError_t e = launch_shrink(pl, as_stream(stream), sp);
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_expand(const float* t, int32_t T, int32_t N, const int32_t* adapter_id, const uint64_t* B_ptrs,
                        const int32_t* ranks, const float* scales, int32_t n_adapters, int32_t r_max, uint16_t* y,
                        void* stream) {
  lora_status st = check_sizes(T, 128, N);
  if (st != LORA_OK) return st;
  if ((st = check_adapters(n_adapters, r_max)) != LORA_OK) return st;
  if (T == 0) return LORA_OK;
  if (!t || !adapter_id || !B_ptrs || !ranks || !scales || !y) return LORA_ERR_INVALID_ARG;
  if (!aligned16(t) || !aligned16(y)) return LORA_ERR_INVALID_ARG;
  ExpandParams p{};
  p.t = t; p.T = T; p.N = N; p.r_max = r_max; p.n_ad = n_adapters;
  p.ids = adapter_id; p.B_ptrs = B_ptrs; p.ranks = ranks; p.scales = scales; p.y = y;
  return launch_expand(p, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status gemm_lowp_lora_epilogue(const uint16_t* x, int32_t T, int32_t K, int32_t N, int32_t w_fmt,
                                    const uint8_t* w_q, const void* w_scale, float* t, const int32_t* adapter_id,
                                    int32_t* seg_indptr, int32_t* sorted_tok, const uint64_t* A_ptrs,
                                    const uint64_t* B_ptrs, const int32_t* ranks, const float* scales,
                                    int32_t n_adapters, int32_t r_max, uint16_t* y, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  lora_status st = check_sizes(T, K, N);
  if (st != LORA_OK) return st;
  if ((st = check_adapters(n_adapters, r_max)) != LORA_OK) return st;
  if (w_fmt != LORA_W_FP8_E4M3 && w_fmt != LORA_W_MXFP4_E2M1) return LORA_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(LORA_FUSE_SHRINK | LORA_BUILD_SEGMENTS | LORA_ACT_BF16)) return LORA_ERR_INVALID_ARG;
  const bool build = (flags & LORA_BUILD_SEGMENTS) != 0;
  if (build && !(flags & LORA_FUSE_SHRINK)) return LORA_ERR_INVALID_ARG;
  const bool a16 = (flags & LORA_ACT_BF16) != 0;
  if (build && (!seg_indptr || !adapter_id || (T > 0 && !sorted_tok))) return LORA_ERR_INVALID_ARG;
  if (T == 0) {
    if (!build) return LORA_OK;
    // an empty batch still has its (all-zero) segment offsets
    if (!workspace || !aligned16(workspace) || workspace_bytes < 256) return LORA_ERR_WORKSPACE;
    int* ctrl0 = reinterpret_cast<int*>(workspace);
    return launch_build_segments(adapter_id, 0, n_adapters, seg_indptr, sorted_tok, ctrl0 + CTRL_SEGERR,
                                 as_stream(stream)) == hipSuccess
               ? LORA_OK
               : LORA_ERR_HIP;
  }
  if (!x || !w_q || !w_scale || !y) return LORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(y)) return LORA_ERR_INVALID_ARG;
  const bool fused = (flags & LORA_FUSE_SHRINK) != 0;
  const bool lora = fused || t != nullptr;
  if (lora && (!adapter_id || !B_ptrs || !ranks || !scales)) return LORA_ERR_INVALID_ARG;
  if (fused && (!seg_indptr || !sorted_tok || !A_ptrs)) return LORA_ERR_INVALID_ARG;
  if (t && !aligned16(t)) return LORA_ERR_INVALID_ARG;
  const LayerPlan pl = make_plan(T, K, N, n_adapters, r_max, w_fmt, true, a16);
  if (!workspace || !aligned16(workspace) || workspace_bytes < pl.total) return LORA_ERR_WORKSPACE;
  char* ws = reinterpret_cast<char*>(workspace);
  hipStream_t s = as_stream(stream);

  int* ctrl = reinterpret_cast<int*>(ws + pl.off_ctrl);
  // Segments in the layer launch up to 128 tokens.  Beyond that the builder's own launch
  // costs less than making the down-projection workgroups wait for it at their start
  // (measured per step: 128 tokens x 128 adapters 190.4 us in-launch against 193.2 us;
  // 4096-token prefill 220.1 us in-launch against 218.0 us).
  const bool build_in = build && T <= 128;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + pl.off_xq);
  uint8_t* xsc = reinterpret_cast<uint8_t*>(ws + pl.off_xsc);
  if (build && !build_in && pl.XQ) {
    // the builder as a workgroup of the MXFP8 pre-pass's launch
    if (launch_quant_build(x, T, K, xq, xsc, adapter_id, n_adapters, seg_indptr, sorted_tok, ctrl + CTRL_SEGERR, s) !=
        hipSuccess)
      return LORA_ERR_HIP;
  } else {
    if (build && !build_in &&
        launch_build_segments(adapter_id, T, n_adapters, seg_indptr, sorted_tok, ctrl + CTRL_SEGERR, s) != hipSuccess)
      return LORA_ERR_HIP;
    if (pl.XQ && launch_quant(x, T, K, xq, xsc, s) != hipSuccess) return LORA_ERR_HIP;
  }

  uint64_t* ttag = reinterpret_cast<uint64_t*>(ws + pl.off_ttag);

  ShrinkParams sp{};
  if (fused) {
    sp.x = x; sp.T = T; sp.K = K;
    sp.seg_indptr = seg_indptr; sp.sorted_tok = sorted_tok;
    sp.A_ptrs = A_ptrs; sp.ranks = ranks; sp.n_ad = n_adapters; sp.r_max = r_max;
    sp.ids = adapter_id;
    sp.t_out = t;  // may be null
    sp.t_tag = ttag;
    // past 16 tokens (one K-part): t goes to the epilogue as tagged bf16 pairs of s_a t
    sp.t_pack = (pl.s_kparts == 1 && T > 16 && pl.TT != 1) ? 1 : 0;
    sp.scales = scales;
    sp.tblk = pl.s_tblk; sp.n_tblk = pl.s_ntblk; sp.n_jg = pl.s_njg; sp.jper = pl.s_jper;
    sp.kparts = pl.s_kparts; sp.kpart_len = pl.s_kpart_len;
    sp.seg_wait = build_in ? 1 : 0;
    sp.compact = pl.compact ? 1 : 0;
    sp.spin_limit = SPIN_LIMIT;
  }
  GemmParams gp{};
  gp.x = x; gp.xq = xq; gp.xsc = xsc;
  gp.T = T; gp.K = K; gp.N = N;
  gp.wq = w_q;
  gp.ws_fp8 = (w_fmt == LORA_W_FP8_E4M3) ? reinterpret_cast<const float*>(w_scale) : nullptr;
  gp.ws_fp4 = (w_fmt == LORA_W_MXFP4_E2M1) ? reinterpret_cast<const uint8_t*>(w_scale) : nullptr;
  gp.t = fused ? nullptr : t;
  gp.t_out = (fused && pl.s_kparts > 1) ? t : nullptr;
  gp.t_tag = fused ? ttag : nullptr;
  gp.t_kparts = pl.s_kparts;
  gp.t_pack = (fused && pl.s_kparts == 1 && T > 16 && pl.TT != 1) ? 1 : 0;
  gp.r_max = r_max;
  gp.ids = adapter_id; gp.B_ptrs = B_ptrs; gp.ranks = ranks; gp.scales = scales; gp.n_ad = n_adapters;
  gp.y = y;
  gp.ksplit = pl.ksplit; gp.krange = pl.krange; gp.n_cb = pl.n_cb; gp.n_tb = pl.n_tb;
  gp.gpart = reinterpret_cast<float*>(ws + pl.off_gpart);
  gp.gflag = reinterpret_cast<int*>(ws + pl.off_gflag);
  gp.lora = lora ? 1 : 0;
  gp.n_shrink = fused ? pl.n_shrink_wg : 0;
  gp.ctrl = ctrl;
  gp.spin_limit = SPIN_LIMIT;
  gp.seg_build = build_in ? seg_indptr : nullptr;
  gp.sorted_build = build_in ? sorted_tok : nullptr;
  return launch_layer(pl, s, sp, gp) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_pack_weight(int32_t w_fmt, const uint8_t* q, const uint8_t* scale, int32_t N, int32_t K,
                             uint8_t* q_packed, uint8_t* scale_packed, void* stream) {
  if (w_fmt != LORA_W_FP8_E4M3 && w_fmt != LORA_W_MXFP4_E2M1) return LORA_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return LORA_ERR_INVALID_ARG;
  if (N % 64 != 0 || K % 128 != 0) return LORA_ERR_UNSUPPORTED;
  if (!q || !q_packed || !aligned16(q) || !aligned16(q_packed)) return LORA_ERR_INVALID_ARG;
  if (w_fmt == LORA_W_MXFP4_E2M1 && (!scale || !scale_packed)) return LORA_ERR_INVALID_ARG;
  if (q == q_packed) return LORA_ERR_INVALID_ARG;  // not in place
  hipError_t e = launch_pack_weight(w_fmt, q, reinterpret_cast<const uint8_t*>(scale), N, K, q_packed, scale_packed,
                                    as_stream(stream));
  return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

/* Introspection for tests and the benchmark: the plan chosen for these sizes. */
int32_t lora_plan_info(int32_t T, int32_t K, int32_t N, int32_t n_adapters, int32_t r_max, int32_t w_fmt,
                       int32_t* out, int32_t n_out) {
  if (check_sizes(T, K, N) != LORA_OK || check_adapters(n_adapters, r_max) != LORA_OK || T == 0) return -1;
  const LayerPlan pl = make_plan(T, K, N, n_adapters, r_max, w_fmt);
  const int32_t v[] = {pl.TT, pl.CT, pl.WC, pl.WK, pl.XQ ? 1 : 0, pl.KC, pl.ksplit, pl.krange, pl.n_cb,
                       pl.n_tb, pl.n_gemm_wg, pl.s_tblk, pl.s_njg, pl.s_kparts, pl.n_shrink_wg};
  const int32_t n = (int32_t)(sizeof(v) / sizeof(v[0]));
  for (int32_t i = 0; i < n && i < n_out; ++i) out[i] = v[i];
  return n;
}

}  // extern "C"

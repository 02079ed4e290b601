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
  if (n_adapters > MAX_ADAPTERS || r_max > MAX_RANK) return LORA_ERR_UNSUPPORTED;
  return LORA_OK;
}

// Tile plan: a pure function of the sizes, so lora_workspace_bytes and every call agree.
// fused: the down-projection runs in the layer launch (its K may then be split into parts
// that the GEMM epilogue adds up); otherwise it runs alone and writes the final t.
// a16: 16-bit activations: the one-tile stream up to 16 tokens, 64 x 128 tiles with bf16 x
// staged in LDS above (where N % 128 == 0; otherwise 16-token tiles of the stream, whose
// token tiles of a column tile share an XCD's L2 for W).
LayerPlan make_plan(int T, int K, int N, int n_ad, int r_max_in, int fmt, bool fused = true, bool a16 = false) {
  // internal row stride of t: the caller's r_max rounded up to whole 16-byte runs of bf16
  const int r_max = rank_pad(r_max_in);
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
  // MXFP8 long batches with FP8 W, K and N multiples of 512 and at least 128 tiles of 128
  // tokens x 512 channels: the eight-wave tiles of k_gemm_pf (two waves per SIMD, W straight
  // into registers, x through LDS), x quantised in their operand order
  if (!a16 && fmt == LORA_W_FP8_E4M3 && T > 128 && N % 512 == 0 && K % 512 == 0 &&
      ceil_div(T, 128) * (N / 512) >= 128) {
    pl.pf = true;
    pl.TT = 8; pl.CT = 8; pl.WC = 4; pl.WK = 1; pl.XQ = true;
  }
  // 16-bit activations past 128 tokens (FP8, N % 256 == 0): the down-projection runs first,
  // over 16-position blocks of the sorted order, and writes plain fp32 t; the GEMM then has
  // the whole GPU, in 64 x 256 tiles (two workgroups per CU) whose epilogue adds the term
  pl.rows16 = a16 && T > 128 && fmt == LORA_W_FP8_E4M3 && N % 256 == 0;
  pl.KC = (pl.TT == 1) ? 2048 : ((pl.TT <= 4 && pl.CT == 1) ? 512 : (pl.CT >= 4 ? 128 : 256));
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
  int ks = (tiles >= 128 || pl.pf) ? 1 : std::min(max_split, std::max(1, 224 / tiles));
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
    // The standalone launch takes all ranks of an adapter in one item (up to 64): its x rows
    // are read once and the four rank tiles' loads are in flight together (the configuration
    // search's choice on the one-token-per-adapter down-projection: 76 -> 35 us).  In the
    // fused launch, beside the GEMM workgroups, items of 16 ranks measured faster
    // (down-projection workload 96 us per call against 122 us with 64-rank items).
    pl.s_jper = fused ? 1 : 4;
    pl.s_njg = ceil_div(r_max, 16 * pl.s_jper);
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
  // (the operand order of k_gemm_pf holds whole 128-row tiles; rows past T are never written)
  const size_t xrows = pl.pf ? (size_t)pl.n_tb * 128 : (size_t)T;
  pl.off_xq = off;    if (pl.XQ) off += round256(xrows * K);
  pl.off_xsc = off;   if (pl.XQ) off += round256(xrows * (K / 32) + 8);  // + 8: padding read by a partial last chunk
  pl.off_tpl = off;
  if (pl.pf) off += round256((size_t)PF_KP * T * PF_TPS * 4);  // the pre-pass's K-part sums of t
  else if ((pl.XQ || pl.rows16) && pl.s_cfg == 1) off += round256((size_t)T * r_max * 4);
  pl.total = off;
  return pl;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// The backward's work split for short batches, with the workspace its partial sums need.
// dX: with fewer 64-row x 256-column tiles than fill the GPU, each tile's contraction over N is
// split into ranges of an even number of 64-wide steps taken by workgroups of their own
// (towards 512 workgroups: at most 32 ranges a tile, four or more steps each).  u = dY B_a^T
// up to 128 tokens (the standalone down-projection, one item per adapter present): N is split
// into parts of at least 256 (towards 256 items, at most 32 parts).
struct BwdPlan {
  int n_split, steps;      // dX ranges
  int u_kparts, u_kpart_len;
  size_t dx_bytes, u_bytes, total;
};
BwdPlan bwd_plan(int T, int K, int N, int n_ad, int r_max) {
  const int NI = N / 64, tiles = ceil_div(T, 64) * ceil_div(K, 256);
  BwdPlan b{1, NI, 1, N, 0, 0, 0};
  if (T <= 0) return b;
  if (tiles < 384) {
    const int want = std::min({ceil_div(512, tiles), std::max(1, NI / 4), 32});
    if (want > 1) {
      int steps = ceil_div(NI, want);
      steps += steps & 1;  // even: the loop alternates two register sets
      if (ceil_div(NI, steps) > 1) {
        b.n_split = ceil_div(NI, steps);
        b.steps = steps;
        b.dx_bytes = round256((size_t)b.n_split * T * K * 4);
      }
    }
  }
  if (T <= 128) {
    const int kp = std::min({ceil_div(256, std::max(1, std::min(n_ad, T))), std::max(1, N / 256), 32});
    if (kp > 1) {
      b.u_kpart_len = ceil_div(ceil_div(N, kp), 256) * 256;
      b.u_kparts = ceil_div(N, b.u_kpart_len);
      if (b.u_kparts > 1) b.u_bytes = round256((size_t)b.u_kparts * T * r_max * 4);
      else b.u_kpart_len = N;
    }
  }
  b.total = b.dx_bytes + b.u_bytes;
  return b;
}

}  // namespace

extern "C" {

const char* lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or format)";
    case LORA_ERR_UNSUPPORTED: return "unsupported size (see the limits in lora_lowp.h)";
    case LORA_ERR_WORKSPACE: return "workspace missing or too small";
    case LORA_ERR_HIP: return "HIP launch or runtime error";
    case LORA_ERR_SCRATCH_LIMIT:
      return "sizes need more than the 32 MiB of scratch memory of gemm_lowp_lora_epilogue_noalloc";
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
  sp.A_ptrs = A_ptrs; sp.ranks = ranks; sp.n_ad = n_adapters; sp.r_max = rank_pad(r_max); sp.r_lim = r_max;
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
  p.t = t; p.T = T; p.N = N; p.r_lim = r_max; p.n_ad = n_adapters;
  p.ids = adapter_id; p.B_ptrs = B_ptrs; p.ranks = ranks; p.scales = scales; p.y = y;
  return launch_expand(p, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // extern "C"

namespace {

// The layer call.  noalloc: the workspace is this device's scratch array, acquired here
// once every argument has passed its checks (workspace and workspace_bytes are ignored).
lora_status layer_call(const uint16_t* x, int32_t T, int32_t K, int32_t N, int32_t w_fmt, const uint8_t* w_q,
                       const void* w_scale, float* t, const int32_t* adapter_id, int32_t* seg_indptr,
                       int32_t* sorted_tok, const uint64_t* A_ptrs, const uint64_t* B_ptrs, const int32_t* ranks,
                       const float* scales, int32_t n_adapters, int32_t r_max, uint16_t* y, uint32_t flags,
                       void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  lora_status st = check_sizes(T, K, N);
  if (st != LORA_OK) return st;
  if ((st = check_adapters(n_adapters, r_max)) != LORA_OK) return st;
  if (w_fmt != LORA_W_FP8_E4M3 && w_fmt != LORA_W_MXFP4_E2M1) return LORA_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(LORA_FUSE_SHRINK | LORA_BUILD_SEGMENTS | LORA_ACT_BF16)) return LORA_ERR_INVALID_ARG;
  const bool build = (flags & LORA_BUILD_SEGMENTS) != 0;
  if (build && !(flags & LORA_FUSE_SHRINK)) return LORA_ERR_INVALID_ARG;
  const bool a16 = (flags & LORA_ACT_BF16) != 0;
  if (build && (!seg_indptr || !adapter_id || (T > 0 && !sorted_tok))) return LORA_ERR_INVALID_ARG;
  if (noalloc) {
    // every argument that can be checked before touching the device, then the scratch
    const LayerPlan pl0 = make_plan(std::max(T, 1), K, N, n_adapters, r_max, w_fmt, true, a16);
    if (pl0.total > SCRATCH_BYTES) return LORA_ERR_SCRATCH_LIMIT;
    if (T > 0) {
      if (!x || !w_q || !w_scale || !y) return LORA_ERR_INVALID_ARG;
      if (!aligned16(x) || !aligned16(w_q) || !aligned16(y)) return LORA_ERR_INVALID_ARG;
      const bool lora0 = (flags & LORA_FUSE_SHRINK) != 0 || t != nullptr;
      if (lora0 && (!adapter_id || !B_ptrs || !ranks || !scales)) return LORA_ERR_INVALID_ARG;
      if ((flags & LORA_FUSE_SHRINK) && (!seg_indptr || !sorted_tok || !A_ptrs)) return LORA_ERR_INVALID_ARG;
      if (t && !aligned16(t)) return LORA_ERR_INVALID_ARG;
    } else if (!build) {
      return LORA_OK;
    }
    if (scratch_acquire(as_stream(stream), pl0.off_ttag, pl0.off_gpart, &workspace) != hipSuccess) return LORA_ERR_HIP;
    workspace_bytes = SCRATCH_BYTES;
  }
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
  // Long batches with an MXFP8 pre-pass: the down-projection items run in the pre-pass
  // launch, beside the quantisation, and write t as plain fp32; the layer launch is the
  // GEMM alone (its epilogue reads that t).  In the layer launch they would hold CUs that
  // the GEMM tiles need (prefill: 144 workgroups for ~30 us each).
  const bool pre_shrink = fused && pl.XQ && pl.s_cfg == 1;
  // (with k_gemm_pf the pre-pass writes K-part sums into the workspace, and the GEMM adds them
  // and stores the caller's t)
  float* t_pl = pre_shrink ? ((t && !pl.pf) ? t : reinterpret_cast<float*>(ws + pl.off_tpl)) : nullptr;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + pl.off_xq);
  uint8_t* xsc = reinterpret_cast<uint8_t*>(ws + pl.off_xsc);
  ShrinkParams sp{};
  auto shrink_params = [&]() {
    sp.x = x; sp.T = T; sp.K = K;
    sp.seg_indptr = seg_indptr; sp.sorted_tok = sorted_tok;
    sp.A_ptrs = A_ptrs; sp.ranks = ranks; sp.n_ad = n_adapters; sp.r_max = rank_pad(r_max); sp.r_lim = r_max;
    sp.ids = adapter_id;
    sp.scales = scales;
    sp.tblk = pl.s_tblk; sp.n_tblk = pl.s_ntblk; sp.n_jg = pl.s_njg; sp.jper = pl.s_jper;
    sp.kparts = pl.s_kparts; sp.kpart_len = pl.s_kpart_len;
    sp.compact = pl.compact ? 1 : 0;
    sp.spin_limit = SPIN_LIMIT;
  };
  if (pl.rows16) {
    float* t16 = fused ? (t ? t : reinterpret_cast<float*>(ws + pl.off_tpl)) : t;
    if (fused) {
      if (build && launch_build_segments(adapter_id, T, n_adapters, seg_indptr, sorted_tok, ctrl + CTRL_SEGERR, s) !=
                       hipSuccess)
        return LORA_ERR_HIP;
      shrink_params();
      sp.t_out = t16;
      if (launch_shrink_rows(sp, s) != hipSuccess) return LORA_ERR_HIP;
    }
    GemmParams gp{};
    gp.x = x; gp.T = T; gp.K = K; gp.N = N;
    gp.wq = w_q;
    gp.ws_fp8 = reinterpret_cast<const float*>(w_scale);
    gp.t = t16;
    gp.r_max = rank_pad(r_max);
    gp.r_lim = r_max;
    gp.ids = adapter_id; gp.B_ptrs = B_ptrs; gp.ranks = ranks; gp.scales = scales; gp.n_ad = n_adapters;
    gp.y = y;
    gp.lora = lora ? 1 : 0;
    gp.ctrl = ctrl;
    return launch_gemm_a16(gp, s) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  }
  if (pre_shrink) {
    // the segments first (above 128 tokens never in the layer launch), then the pre-pass
    if (build && launch_build_segments(adapter_id, T, n_adapters, seg_indptr, sorted_tok, ctrl + CTRL_SEGERR, s) !=
                     hipSuccess)
      return LORA_ERR_HIP;
    shrink_params();
    sp.t_out = pl.pf ? nullptr : t_pl;
    sp.t_part = pl.pf ? t_pl : nullptr;
    sp.t_tag = nullptr;
    sp.t_pack = 0;
    sp.seg_wait = 0;
    if (launch_quant_shrink(pl, sp, x, T, K, xq, xsc, s) != hipSuccess) return LORA_ERR_HIP;
    sp = ShrinkParams{};
  } else if (build && !build_in && pl.XQ && !pl.pf) {
    // the builder as a workgroup of the MXFP8 pre-pass's launch
    if (launch_quant_build(x, T, K, xq, xsc, adapter_id, n_adapters, seg_indptr, sorted_tok, ctrl + CTRL_SEGERR, s) !=
        hipSuccess)
      return LORA_ERR_HIP;
  } else {
    if (build && !build_in &&
        launch_build_segments(adapter_id, T, n_adapters, seg_indptr, sorted_tok, ctrl + CTRL_SEGERR, s) != hipSuccess)
      return LORA_ERR_HIP;
    if (pl.XQ && (pl.pf ? launch_quant_pf(x, T, K, xq, xsc, s) : launch_quant(x, T, K, xq, xsc, s)) != hipSuccess)
      return LORA_ERR_HIP;
  }

  uint64_t* ttag = reinterpret_cast<uint64_t*>(ws + pl.off_ttag);

  const bool in_launch = fused && !pre_shrink;  // the down-projection in the layer launch
  if (in_launch) {
    shrink_params();
    sp.t_out = t;  // may be null
    sp.t_tag = ttag;
    // past 16 tokens (one K-part): t goes to the epilogue as tagged bf16 pairs of s_a t
    sp.t_pack = (pl.s_kparts == 1 && T > 16 && pl.TT != 1) ? 1 : 0;
    sp.seg_wait = build_in ? 1 : 0;
  }
  GemmParams gp{};
  gp.x = x; gp.xq = xq; gp.xsc = xsc;
  gp.T = T; gp.K = K; gp.N = N;
  gp.wq = w_q;
  gp.ws_fp8 = (w_fmt == LORA_W_FP8_E4M3) ? reinterpret_cast<const float*>(w_scale) : nullptr;
  gp.ws_fp4 = (w_fmt == LORA_W_MXFP4_E2M1) ? reinterpret_cast<const uint8_t*>(w_scale) : nullptr;
  gp.t = pre_shrink ? t_pl : (fused ? nullptr : t);
  gp.t_out = ((in_launch && pl.s_kparts > 1) || (pre_shrink && pl.pf)) ? t : nullptr;
  gp.t_tag = in_launch ? ttag : nullptr;
  gp.t_kparts = pl.pf ? (pre_shrink ? PF_KP : 1) : pl.s_kparts;
  gp.t_pack = (in_launch && pl.s_kparts == 1 && T > 16 && pl.TT != 1) ? 1 : 0;
  gp.r_max = rank_pad(r_max);
  gp.r_lim = r_max;
  gp.ids = adapter_id; gp.B_ptrs = B_ptrs; gp.ranks = ranks; gp.scales = scales; gp.n_ad = n_adapters;
  gp.y = y;
  gp.ksplit = pl.ksplit; gp.krange = pl.krange; gp.n_cb = pl.n_cb; gp.n_tb = pl.n_tb;
  gp.gpart = reinterpret_cast<float*>(ws + pl.off_gpart);
  gp.gflag = reinterpret_cast<int*>(ws + pl.off_gflag);
  gp.lora = lora ? 1 : 0;
  gp.n_shrink = in_launch ? pl.n_shrink_wg : 0;
  gp.ctrl = ctrl;
  gp.spin_limit = SPIN_LIMIT;
  gp.seg_build = build_in ? seg_indptr : nullptr;
  gp.sorted_build = build_in ? sorted_tok : nullptr;
  // Long batches: every tile walks K from the same place (tiles that share W or x blocks
  // then read them at about the same time, from L2), in the XCD-grouped tile order.  Short
  // batches keep the rotation: their few tiles each read W alone, spread over HBM channels.
  const int tiles = pl.n_cb * pl.n_tb;
  const int first_gemm = (build_in ? 1 : 0) + gp.n_shrink;
  gp.rot = (T > 128) ? 0 : 1;
  gp.tile_group = 0;
  if (T > 128 && pl.ksplit == 1 && tiles % 8 == 0 && first_gemm % 8 == 0 && pl.TT != 1)
    gp.tile_group = (pl.n_cb % 4 == 0) ? 4 : ((pl.n_cb % 2 == 0) ? 2 : 1);
  if (pl.pf) return launch_gemm_pf(gp, s) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  return launch_layer(pl, s, sp, gp) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // namespace

extern "C" {

lora_status gemm_lowp_lora_epilogue(const uint16_t* x, int32_t T, int32_t K, int32_t N, int32_t w_fmt,
                                    const uint8_t* w_q, const void* w_scale, float* t, const int32_t* adapter_id,
                                    int32_t* seg_indptr, int32_t* sorted_tok, const uint64_t* A_ptrs,
                                    const uint64_t* B_ptrs, const int32_t* ranks, const float* scales,
                                    int32_t n_adapters, int32_t r_max, uint16_t* y, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return layer_call(x, T, K, N, w_fmt, w_q, w_scale, t, adapter_id, seg_indptr, sorted_tok, A_ptrs, B_ptrs, ranks,
                    scales, n_adapters, r_max, y, flags, workspace, workspace_bytes, stream, false);
}

lora_status gemm_lowp_lora_epilogue_noalloc(const uint16_t* x, int32_t T, int32_t K, int32_t N, int32_t w_fmt,
                                            const uint8_t* w_q, const void* w_scale, float* t,
                                            const int32_t* adapter_id, int32_t* seg_indptr, int32_t* sorted_tok,
                                            const uint64_t* A_ptrs, const uint64_t* B_ptrs, const int32_t* ranks,
                                            const float* scales, int32_t n_adapters, int32_t r_max, uint16_t* y,
                                            uint32_t flags, void* stream) {
  return layer_call(x, T, K, N, w_fmt, w_q, w_scale, t, adapter_id, seg_indptr, sorted_tok, A_ptrs, B_ptrs, ranks,
                    scales, n_adapters, r_max, y, flags, nullptr, 0, stream, true);
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

lora_status lora_pack_adapter(const uint16_t* A, const uint16_t* B, int32_t K, int32_t N, int32_t r, uint16_t* At,
                              uint16_t* Bt, void* stream) {
  if (K <= 0 || N <= 0 || r < 1) return LORA_ERR_INVALID_ARG;
  if (r > MAX_RANK || K % 64 != 0) return LORA_ERR_UNSUPPORTED;
  if (!A || !B || !At || !Bt || !aligned16(At) || !aligned16(Bt)) return LORA_ERR_INVALID_ARG;
  const char *a0 = reinterpret_cast<const char*>(A), *b0 = reinterpret_cast<const char*>(B);
  const char *o0 = reinterpret_cast<const char*>(At), *p0 = reinterpret_cast<const char*>(Bt);
  const size_t na = (size_t)K * r * 2, nb = (size_t)N * r * 2;
  const size_t nat = (size_t)a_tiles(r) * 16 * K * 2, nbt = (size_t)N * rank_pad(r) * 2;
  auto overlap = [](const char* x, size_t nx, const char* y, size_t ny) { return x < y + ny && y < x + nx; };
  if (overlap(a0, na, o0, nat) || overlap(a0, na, p0, nbt) || overlap(b0, nb, o0, nat) || overlap(b0, nb, p0, nbt) ||
      overlap(o0, nat, p0, nbt))
    return LORA_ERR_INVALID_ARG;  // not in place
  return launch_pack_adapter(A, B, K, N, r, At, Bt, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_pack_weight_t(int32_t w_fmt, const uint8_t* q, int32_t N, int32_t K, uint8_t* qt, void* stream) {
  if (w_fmt != LORA_W_FP8_E4M3 && w_fmt != LORA_W_MXFP4_E2M1) return LORA_ERR_INVALID_ARG;
  if (N <= 0 || K <= 0) return LORA_ERR_INVALID_ARG;
  if (w_fmt != LORA_W_FP8_E4M3 || N % 128 != 0 || K % 128 != 0) return LORA_ERR_UNSUPPORTED;
  if (!q || !qt || !aligned16(qt)) return LORA_ERR_INVALID_ARG;
  const char *a = reinterpret_cast<const char*>(q), *b = reinterpret_cast<const char*>(qt);
  const size_t n = (size_t)N * K;
  if (a < b + n && b < a + n) return LORA_ERR_INVALID_ARG;  // not in place
  return launch_pack_weight_t(q, N, K, qt, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_pack_adapter_bwd(const uint16_t* A, const uint16_t* B, int32_t K, int32_t N, int32_t r,
                                  uint16_t* Bop, uint16_t* Ar, void* stream) {
  if (K <= 0 || N <= 0 || r < 1) return LORA_ERR_INVALID_ARG;
  if (r > MAX_RANK || N % 64 != 0) return LORA_ERR_UNSUPPORTED;
  if (!A || !B || !Bop || !Ar || !aligned16(Bop) || !aligned16(Ar)) return LORA_ERR_INVALID_ARG;
  const char *a0 = reinterpret_cast<const char*>(A), *b0 = reinterpret_cast<const char*>(B);
  const char *o0 = reinterpret_cast<const char*>(Bop), *p0 = reinterpret_cast<const char*>(Ar);
  const size_t na = (size_t)K * r * 2, nb = (size_t)N * r * 2;
  const size_t nop = (size_t)a_tiles(r) * 16 * N * 2, nar = (size_t)K * rank_pad(r) * 2;
  auto overlap = [](const char* x, size_t nx, const char* y, size_t ny) { return x < y + ny && y < x + nx; };
  if (overlap(a0, na, o0, nop) || overlap(a0, na, p0, nar) || overlap(b0, nb, o0, nop) || overlap(b0, nb, p0, nar) ||
      overlap(o0, nop, p0, nar))
    return LORA_ERR_INVALID_ARG;  // not in place
  return launch_pack_adapter_bwd(A, B, K, N, r, Bop, Ar, as_stream(stream)) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_backward(const uint16_t* x, const uint16_t* dy, const float* t, int32_t T, int32_t K, int32_t N,
                          int32_t w_fmt, const uint8_t* wt_q, const float* w_scale, const int32_t* adapter_id,
                          const int32_t* seg_indptr, const int32_t* sorted_tok, const uint64_t* Bop_ptrs,
                          const uint64_t* Ar_ptrs, const int32_t* ranks, const float* scales, int32_t n_adapters,
                          int32_t r_max, uint16_t* dx, float* u, const uint64_t* dA_ptrs, const uint64_t* dB_ptrs,
                          int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  if (w_fmt != LORA_W_FP8_E4M3 && w_fmt != LORA_W_MXFP4_E2M1) return LORA_ERR_INVALID_ARG;
  if (T < 0 || K <= 0 || N <= 0) return LORA_ERR_INVALID_ARG;
  if (w_fmt != LORA_W_FP8_E4M3 || T > 65536 || K % 128 != 0 || N % 128 != 0) return LORA_ERR_UNSUPPORTED;
  lora_status st = check_adapters(n_adapters, r_max);
  if (st != LORA_OK) return st;
  if (!ranks || !scales || !dA_ptrs || !dB_ptrs) return LORA_ERR_INVALID_ARG;
  const hipStream_t s = as_stream(stream);
  BwdGradParams gp{};
  gp.x = x; gp.dy = dy; gp.u = u; gp.t = t;
  gp.T = T; gp.K = K; gp.N = N; gp.r_lim = r_max;
  gp.seg_indptr = seg_indptr; gp.sorted_tok = sorted_tok; gp.empty = (T == 0);
  gp.ranks = ranks; gp.scales = scales; gp.n_ad = n_adapters;
  gp.dA_ptrs = dA_ptrs; gp.dB_ptrs = dB_ptrs;
  gp.nkb = K / 64; gp.nnb = N / 64; gp.status = status;
  if (T == 0)  // no tokens: zero gradients
    return launch_bwd_grad(gp, s) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  if (!x || !dy || !t || !wt_q || !w_scale || !adapter_id || !seg_indptr || !sorted_tok || !Bop_ptrs || !Ar_ptrs ||
      !dx || !u)
    return LORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(wt_q) || !aligned16(w_scale) || !aligned16(dx) || !aligned16(u))
    return LORA_ERR_INVALID_ARG;
  const BwdPlan bp = bwd_plan(T, K, N, n_adapters, r_max);  // the split work's partial sums
  if (bp.total > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < bp.total)) return LORA_ERR_WORKSPACE;
  char* wsb = reinterpret_cast<char*>(workspace);
  // u = dY B_a^T: the forward's down-projection kernel over N, with B_a in A_a's place
  const LayerPlan pl = make_plan(T, N, 64, n_adapters, r_max, LORA_W_FP8_E4M3, /*fused=*/false);
  ShrinkParams sp{};
  sp.x = dy; sp.T = T; sp.K = N;
  sp.seg_indptr = seg_indptr; sp.sorted_tok = sorted_tok;
  sp.A_ptrs = Bop_ptrs; sp.ranks = ranks; sp.n_ad = n_adapters; sp.r_max = rank_pad(r_max); sp.r_lim = r_max;
  sp.ids = nullptr;
  sp.t_out = u; sp.t_tag = nullptr;
  sp.tblk = pl.s_tblk; sp.n_tblk = pl.s_ntblk; sp.n_jg = pl.s_njg; sp.jper = pl.s_jper;
  sp.kparts = pl.s_kparts; sp.kpart_len = pl.s_kpart_len;
  // above 128 tokens: the forward pre-pass's down-projection over 16-position blocks (every
  // row of dY read once, four waves per block splitting N); below, the standalone kernel
  if (T > 128) {
    sp.ids = adapter_id;
    if (launch_shrink_rows(sp, s) != hipSuccess) return LORA_ERR_HIP;
  } else if (bp.u_kparts > 1) {
    // N in parts, one item each: fp32 partial sums in the workspace, then added in order
    LayerPlan pu = pl;
    sp.kparts = bp.u_kparts; sp.kpart_len = bp.u_kpart_len;
    sp.t_out = nullptr; sp.t_part = reinterpret_cast<float*>(wsb + bp.dx_bytes);
    pu.s_kparts = bp.u_kparts; pu.s_kpart_len = bp.u_kpart_len;
    pu.n_shrink_items = n_adapters * pl.s_ntblk * pl.s_njg * bp.u_kparts;
    if (launch_shrink(pu, s, sp) != hipSuccess) return LORA_ERR_HIP;
    if (launch_part_reduce(sp.t_part, bp.u_kparts, T, r_max, adapter_id, ranks, n_adapters, u, s) != hipSuccess)
      return LORA_ERR_HIP;
  } else if (launch_shrink(pl, s, sp) != hipSuccess) {
    return LORA_ERR_HIP;
  }
  if (launch_bwd_grad(gp, s) != hipSuccess) return LORA_ERR_HIP;
  BwdDxParams dp{};
  dp.dy = dy; dp.wt = wt_q; dp.wsc = w_scale; dp.T = T; dp.K = K; dp.N = N;
  dp.u = u; dp.r_lim = r_max; dp.ids = adapter_id; dp.Ar_ptrs = Ar_ptrs; dp.ranks = ranks; dp.scales = scales;
  dp.n_ad = n_adapters; dp.dx = dx;
  dp.n_tb = ceil_div(T, 64); dp.n_kb = ceil_div(K, 256);
  dp.n_split = bp.n_split; dp.split_steps = bp.steps;
  dp.part = reinterpret_cast<float*>(wsb);
  if (launch_bwd_dx(dp, s) != hipSuccess) return LORA_ERR_HIP;
  if (dp.n_split > 1 && launch_bwd_dx_reduce(dp, s) != hipSuccess) return LORA_ERR_HIP;
  return LORA_OK;
}

size_t lora_backward_workspace_bytes(int32_t T, int32_t K, int32_t N, int32_t n_adapters, int32_t r_max) {
  if (T <= 0 || K <= 0 || N <= 0 || T > 65536 || K % 128 != 0 || N % 128 != 0) return 0;
  if (check_adapters(n_adapters, r_max) != LORA_OK) return 0;
  return bwd_plan(T, K, N, n_adapters, r_max).total;
}

lora_status lora_shrink_configured(const uint16_t* x, int32_t T, int32_t K, const int32_t* seg_indptr,
                                   const int32_t* sorted_tok, const uint64_t* A_ptrs, const int32_t* ranks,
                                   int32_t n_adapters, int32_t r_max, float* t, const int32_t* config, void* stream) {
  lora_status st = check_sizes(T, K, 64);
  if (st != LORA_OK) return st;
  if ((st = check_adapters(n_adapters, r_max)) != LORA_OK) return st;
  if (!config) return LORA_ERR_INVALID_ARG;
  const int tg = config[0], jp = config[1], u = config[2], tblk = config[3], order = config[4];
  auto in = [](int v, int a, int b, int c) { return v == a || v == b || v == c; };
  const bool bgmv = tg == 0;  // wave reductions: TBLK positions per item, 1, 2 or 4
  if (!(bgmv || in(tg, 1, 2, 4)) || !in(jp, 1, 2, 4) || (u != 1 && u != 2) || (order != 0 && order != 1))
    return LORA_ERR_UNSUPPORTED;
  if (bgmv ? (!in(tblk, 1, 2, 4) || (u == 2 && tblk != 1)) : (tblk < 16 || tblk % 16 != 0 || tblk > 65536))
    return LORA_ERR_UNSUPPORTED;
  if (T == 0) return LORA_OK;
  if (!x || !seg_indptr || !sorted_tok || !A_ptrs || !ranks || !t) return LORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(t)) return LORA_ERR_INVALID_ARG;
  ShrinkParams sp{};
  sp.x = x; sp.T = T; sp.K = K;
  sp.seg_indptr = seg_indptr; sp.sorted_tok = sorted_tok;
  sp.A_ptrs = A_ptrs; sp.ranks = ranks; sp.n_ad = n_adapters; sp.r_max = rank_pad(r_max); sp.r_lim = r_max;
  sp.ids = nullptr;
  sp.t_out = t; sp.t_tag = nullptr;
  sp.tblk = tblk; sp.n_tblk = ceil_div(T, tblk); sp.jper = jp; sp.n_jg = ceil_div(r_max, 16 * jp);
  sp.kparts = 1; sp.kpart_len = ceil_div(K, 256) * 256;
  sp.item_order = order;
  const long items = (long)n_adapters * sp.n_tblk * sp.n_jg;
  if (items > (1L << 30)) return LORA_ERR_UNSUPPORTED;
  if (bgmv)
    return launch_shrink_bgmv(tblk, jp, u, (int)items, as_stream(stream), sp) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
  return launch_shrink_cfg(tg, jp, u, (int)items, as_stream(stream), sp) == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

lora_status lora_shrink_config_info(int32_t tg, int32_t jp, int32_t u, int32_t* out) {
  if (!out) return LORA_ERR_INVALID_ARG;
  int regs = 0, spill = 0, lds = 0;
  const hipError_t e = shrink_cfg_attr(tg, jp, u, &regs, &spill, &lds);
  if (e == hipErrorInvalidValue) return LORA_ERR_UNSUPPORTED;
  if (e != hipSuccess) return LORA_ERR_HIP;
  out[0] = regs;
  out[1] = spill;
  out[2] = lds;
  return LORA_OK;
}

lora_status lora_shrink_bgmv_info(int32_t nt, int32_t jp, int32_t u, int32_t* out) {
  if (!out) return LORA_ERR_INVALID_ARG;
  int regs = 0, spill = 0, lds = 0;
  const hipError_t e = shrink_bgmv_attr(nt, jp, u, &regs, &spill, &lds);
  if (e == hipErrorInvalidValue) return LORA_ERR_UNSUPPORTED;
  if (e != hipSuccess) return LORA_ERR_HIP;
  out[0] = regs;
  out[1] = spill;
  out[2] = lds;
  return LORA_OK;
}

lora_status lora_merged_layer(const uint16_t* x, int32_t T, int32_t K, int32_t N, int32_t w_fmt, const uint8_t* w_q,
                              const void* w_scale, const int32_t* adapter_id, const uint64_t* A_rows,
                              const uint64_t* B_ptrs, const int32_t* ranks, const float* scales, int32_t n_adapters,
                              int32_t r_max, uint16_t* y, void* stream) {
  lora_status st = check_sizes(T, K, N);
  if (st != LORA_OK) return st;
  if ((st = check_adapters(n_adapters, r_max)) != LORA_OK) return st;
  if (w_fmt != LORA_W_FP8_E4M3 && w_fmt != LORA_W_MXFP4_E2M1) return LORA_ERR_INVALID_ARG;
  if (T == 0) return LORA_OK;
  if (T > 65535 * 16) return LORA_ERR_UNSUPPORTED;
  if (!x || !w_q || !w_scale || !adapter_id || !A_rows || !B_ptrs || !ranks || !scales || !y)
    return LORA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(y)) return LORA_ERR_INVALID_ARG;
  return launch_merged(x, T, K, N, w_fmt, w_q, w_scale, adapter_id, A_rows, B_ptrs, ranks, scales, n_adapters, r_max, y,
                       as_stream(stream)) == hipSuccess
             ? LORA_OK
             : LORA_ERR_HIP;
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

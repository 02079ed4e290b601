// gfx950 kernels of the fused multi-tenant LoRA layer.
//
// The layer (per token t with adapter a = adapter_id[t]):
//     y[t] = bf16( dequant(xq[t] . W) + s_a * (x[t] @ A_a) @ B_a )
// "Punica: Serving multiple LoRA finetuned LLM as one" (README, Overview) gives the
// algebra Y = X@W + (x_1@A_1@B_1, ...); the "EpiLoRA" abstract gives the schedule:
// the adapter down-projection runs first, the low-precision GEMM streams its weights
// meanwhile, and the up-projection of every tenant is added in the GEMM's epilogue.
//
// Kernels (all with 256-thread workgroups = 4 wave64 unless stated):
//   k_build_segments  one 1024-thread workgroup: stable counting sort of tokens by adapter.
//   k_quant_mxfp8     MXFP8 quantisation of bf16 activations (one thread per 32-block).
//   k_shrink          down-projection t = x @ A_a per segment on bf16 MFMA, split-K with a
//                     fixed-order last-arriver reduction (deterministic).
//   k_expand          standalone up-projection y += s_a t @ B_a (the unfused schedule).
//   k_layer           role-split launch: workgroups [0, n_shrink) run the down-projection,
//                     the rest run the scaled-MFMA base GEMM whose epilogue waits for t.
#include "device_common.hpp"
#include "lora_kernels.hpp"

namespace lora {

// ======================================================================================
// Segment builder
// ======================================================================================
__global__ __launch_bounds__(SEG_THREADS) void k_build_segments(const int* __restrict__ ids, int T, int n_ad,
                                                                int* __restrict__ seg_indptr,
                                                                int* __restrict__ sorted_tok, int* __restrict__ err) {
  __shared__ int cnt[MAX_ADAPTERS];
  __shared__ int part[SEG_THREADS];
  __shared__ int first_bad;
  const int tid = threadIdx.x;
  if (tid == 0) first_bad = 0x7fffffff;
  for (int a = tid; a < n_ad; a += SEG_THREADS) cnt[a] = 0;
  __syncthreads();
  // 1. counts (LDS atomics: order-independent)
  for (int t = tid; t < T; t += SEG_THREADS) {
    int a = ids[t];
    if (a >= 0 && a < n_ad) atomicAdd(&cnt[a], 1);
    else atomicMin(&first_bad, t);
  }
  __syncthreads();
  // 2. exclusive scan: each thread sums a contiguous slice, then a scan over threads
  const int per = (n_ad + SEG_THREADS - 1) / SEG_THREADS;
  const int lo = min(tid * per, n_ad), hi = min(lo + per, n_ad);
  int s = 0;
  for (int a = lo; a < hi; ++a) s += cnt[a];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < SEG_THREADS; off <<= 1) {
    int v = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int base = (tid > 0) ? part[tid - 1] : 0;
  for (int a = lo; a < hi; ++a) {
    int c = cnt[a];
    seg_indptr[a] = base;
    cnt[a] = base;  // becomes the write cursor of adapter a
    base += c;
  }
  if (tid == SEG_THREADS - 1) seg_indptr[n_ad] = part[SEG_THREADS - 1];
  if (tid == 0) *err = (first_bad == 0x7fffffff) ? 0 : first_bad + 1;
  __syncthreads();
  // 3. stable placement by one wave, 64 tokens at a time in token order.  Lanes with the
  //    same adapter are grouped with a ballot; a lane's slot is the cursor plus the number
  //    of lower lanes in its group, so equal ids keep their token order.
  if (tid < 64) {
    volatile int* cur = cnt;
    const int lane = tid;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int t0 = 0; t0 < T; t0 += 64) {
      const int t = t0 + lane;
      const int a = (t < T) ? ids[t] : -1;
      const bool ok = (a >= 0 && a < n_ad);
      unsigned long long pending = __ballot(ok);
      while (pending) {
        const int leader = __ffsll((long long)pending) - 1;
        const int la = __shfl(a, leader);
        const unsigned long long same = __ballot(ok && a == la);
        const int c0 = cur[la];
        if (ok && a == la) sorted_tok[c0 + __popcll(same & below)] = t;
        if (lane == leader) cur[la] = c0 + __popcll(same);
        pending &= ~same;
      }
    }
  }
}

// ======================================================================================
// MXFP8 activation quantisation (standalone; the GEMM loader calls the same functions)
// ======================================================================================
__global__ __launch_bounds__(256) void k_quant_mxfp8(const uint16_t* __restrict__ x, int T, int K,
                                                     uint8_t* __restrict__ xq, uint8_t* __restrict__ xsc) {
  const int nb = K / 32;
  const long total = (long)T * nb;
  for (long b = (long)blockIdx.x * blockDim.x + threadIdx.x; b < total; b += (long)gridDim.x * blockDim.x) {
    const long row = b / nb, kb = b % nb;
    const uint16_t* src = x + row * K + kb * 32;
    uint4 in[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) in[i] = ldg16(src + 8 * i);
    const uint32_t code = mx_block_code(in);
    uint4 out[2];
    mx_block_quant(in, code, out);
    uint8_t* dst = xq + row * K + kb * 32;
    *reinterpret_cast<uint4*>(dst) = out[0];
    *reinterpret_cast<uint4*>(dst + 16) = out[1];
    xsc[b] = (uint8_t)code;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ======================================================================================
// Down-projection ("shrink"): one workgroup per (adapter a, K-chunk c).
// A_a is stored transposed, bf16 [r_a][K].  Both MFMA operands are then rows with K
// contiguous: the x operand is 16 tokens of segment a (gathered through sorted_tok),
// the A operand is 16 ranks.  Lane (i = l%16, g = l/16) loads 32 contiguous bytes
// (k = k0+16g .. k0+16g+15) of its row and feeds them to two 16x16x32 MFMAs; both
// operands use the same k assignment, so the products pair up.  The four waves split
// the chunk's 64-wide k-steps; their sums meet in LDS in wave order, and the chunks of
// one adapter are summed in chunk order by whichever workgroup arrives last.
// ======================================================================================
template <int TG, int U>
__device__ void shrink_item(const ShrinkParams& p, int item, char* smem) {
  const int a = item / p.nchunks, c = item % p.nchunks;
  const int s0 = p.seg_indptr[a], s1 = p.seg_indptr[a + 1];
  const int L = s1 - s0;
  if (L <= 0) return;
  const int r = p.ranks[a];
  if (r < 8 || r > p.r_max || (r & 7)) return;  // unsupported rank: adapter skipped
  const uint16_t* __restrict__ A = reinterpret_cast<const uint16_t*>(p.A_ptrs[a]);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int k_begin = c * p.KC, k_end = min(p.K, k_begin + p.KC);
  const int nsteps = (k_end - k_begin) >> 6;
  const int JT = (r + 15) >> 4;
  float* red = reinterpret_cast<float*>(smem);           // [4 waves][TG][4][64 lanes][4]
  int* flag = reinterpret_cast<int*>(smem + 4 * TG * 4 * 256 * sizeof(float));
  const bool single = (p.nchunks == 1);

  const uint16_t* arow[4];
  bool av[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int j = jt * 16 + li;
    av[jt] = (jt < JT) && (j < r);
    arow[jt] = A + (long)(av[jt] ? j : 0) * p.K + 16 * g;
  }

  for (int tg0 = 0; tg0 < L; tg0 += TG * 16) {
    const int ntt = min(TG, (L - tg0 + 15) >> 4);
    const uint16_t* xrow[TG];
    bool xv[TG];
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      const int pos = tg0 + tt * 16 + li;
      xv[tt] = (tt < ntt) && (pos < L);
      xrow[tt] = p.x + (long)(xv[tt] ? p.sorted_tok[s0 + pos] : 0) * p.K + 16 * g;
    }
    v4f acc[TG][4];
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[tt][jt] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int s = wave; s < nsteps; s += 4 * U) {
      uint4 xa[U][TG][2], aa[U][4][2];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int su = s + 4 * u;
        const int k0 = k_begin + su * 64;
        const bool sv = su < nsteps;
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          const bool v = sv && xv[tt];
          xa[u][tt][0] = v ? ldg16(xrow[tt] + k0) : zero4();
          xa[u][tt][1] = v ? ldg16(xrow[tt] + k0 + 8) : zero4();
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const bool v = sv && av[jt];
          aa[u][jt][0] = v ? ldg16(arow[jt] + k0) : zero4();
          aa[u][jt][1] = v ? ldg16(arow[jt] + k0 + 8) : zero4();
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          if (tt >= ntt) continue;
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) {
            if (jt >= JT) continue;
            acc[tt][jt] = mfma_bf16_16x16x32(xa[u][tt][0], aa[u][jt][0], acc[tt][jt]);
            acc[tt][jt] = mfma_bf16_16x16x32(xa[u][tt][1], aa[u][jt][1], acc[tt][jt]);
          }
        }
    }
    // cross-wave sum in fixed wave order
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
        if (tt < ntt && jt < JT)
          *reinterpret_cast<v4f*>(red + (((wave * TG + tt) * 4 + jt) * 64 + lane) * 4) = acc[tt][jt];
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (tt >= ntt || jt >= JT || ((tt * 4 + jt) & 3) != wave) continue;
        v4f sum = *reinterpret_cast<const v4f*>(red + (((0 * TG + tt) * 4 + jt) * 64 + lane) * 4);
#pragma unroll
        for (int w = 1; w < 4; ++w) sum += *reinterpret_cast<const v4f*>(red + (((w * TG + tt) * 4 + jt) * 64 + lane) * 4);
        const int j = jt * 16 + li;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int pos = tg0 + tt * 16 + 4 * g + v;
          if (pos < L && j < r) {
            if (single) st_agent(p.t + (long)p.sorted_tok[s0 + pos] * p.r_max + j, sum[v]);
            else st_agent(p.part + ((long)c * p.T + (s0 + pos)) * p.r_max + j, sum[v]);
          }
        }
      }
    __syncthreads();
  }
  if (single) {
    // columns j in [r, r_max) of this segment's t rows are zero
    for (int idx = tid; idx < L * (p.r_max - r); idx += 256) {
      const int pos = idx / (p.r_max - r), j = r + idx % (p.r_max - r);
      st_agent(p.t + (long)p.sorted_tok[s0 + pos] * p.r_max + j, 0.f);
    }
    return;
  }
  // last-arriver reduction over the chunks of adapter a
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const int prev = add_agent(&p.ad_ctr[a], 1);
    *flag = (prev == p.nchunks - 1);
  }
  __syncthreads();
  if (!*flag) return;
  for (int idx = tid; idx < L * p.r_max; idx += 256) {
    const int pos = idx / p.r_max, j = idx % p.r_max;
    float sum = 0.f;
    if (j < r)
      for (int cc = 0; cc < p.nchunks; ++cc) sum += ld_agent(p.part + ((long)cc * p.T + (s0 + pos)) * p.r_max + j);
    st_agent(p.t + (long)p.sorted_tok[s0 + pos] * p.r_max + j, sum);
  }
  if (tid == 0) set_agent(&p.ad_ctr[a], 0);
}

template <int TG, int U>
__global__ __launch_bounds__(256) void k_shrink(ShrinkParams p) {
  extern __shared__ __align__(16) char smem[];
  shrink_item<TG, U>(p, blockIdx.x, smem);
}

// ======================================================================================
// Standalone up-projection: y[tok][n] = bf16( y[tok][n] + s_a * sum_j t[tok][j] B_a[j][n] ),
// B_a stored transposed, bf16 [N][r_a].  One workgroup per (token, 256 columns).
// ======================================================================================
__global__ __launch_bounds__(256) void k_expand(ExpandParams p) {
  __shared__ float trow[64];
  const int tok = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int a = p.ids[tok];
  if (a < 0 || a >= p.n_ad) return;
  const int r = p.ranks[a];
  if (r < 8 || r > p.r_max || (r & 7)) return;  // unsupported rank: adapter skipped
  if (threadIdx.x < 64) trow[threadIdx.x] = (threadIdx.x < r) ? p.t[(long)tok * p.r_max + threadIdx.x] : 0.f;
  __syncthreads();
  if (n >= p.N) return;
  const uint16_t* __restrict__ Bt = reinterpret_cast<const uint16_t*>(p.B_ptrs[a]) + (long)n * r;
  float acc = 0.f;
  for (int j = 0; j < r; j += 8) {
    const uint4 b = ldg16(Bt + j);
    const uint32_t w[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += trow[j + 2 * e] * bf16_lo(w[e]);
      acc += trow[j + 2 * e + 1] * bf16_hi(w[e]);
    }
  }
  uint16_t* yp = p.y + (long)tok * p.N + n;
  const float out = __uint_as_float((uint32_t)*yp << 16) + p.scales[a] * acc;
  *yp = (uint16_t)f32_to_bf16_rne(out);
}

// ======================================================================================
// Base GEMM with the LoRA epilogue.
//
// Workgroup tile: TT*16 tokens x WN = 4*CT*16 output channels over a K-range; wave w owns
// columns [w*CT*16, (w+1)*CT*16) of the tile and all its tokens.  Per K-chunk of KC:
//   1. every lane issues the loads of its W fragments for the whole chunk straight into
//      registers (each W byte is read by exactly one lane of one workgroup per K-split);
//   2. the workgroup converts the chunk of x to MXFP8 (or copies pre-quantised codes)
//      into LDS, one 32-block per thread-iteration, rows padded by 16 bytes so that the
//      16 lanes of a lane group hit distinct banks;
//   3. per 128-wide k-step each wave reads its TT x-fragments from LDS once and issues
//      TT*CT scaled MFMAs (x scale from the MX block, W scale 1.0 for FP8 or the MXFP4
//      block scale).
// K-splits write their accumulators to the workspace in lane order; the last split of a
// tile to arrive sums all of them in split order and runs the epilogue.
// Epilogue: FP8 channel scale; then, in fused mode, wait until every down-projection
// workgroup has finished (bounded spin on an agent-scope counter); then for each token
// tile and each adapter present in it, one bf16 MFMA per 32 ranks adds
// (s_a * t[tok]) @ B_a to the rows of that adapter's tokens; round to bf16 and store.
// ======================================================================================
template <int TT>
struct ChunkK {
  static constexpr int KC = (TT == 1) ? 1024 : ((TT <= 4) ? 512 : 256);
  static constexpr int STEPS = KC / 128;
  static constexpr int ROW = KC + 16;  // LDS row stride in bytes
};

template <int FMT, int TT, int CT, bool XQ>
__device__ void gemm_item(const GemmParams& p, int item, char* smem) {
  constexpr int KC = ChunkK<TT>::KC, STEPS = ChunkK<TT>::STEPS, ROW = ChunkK<TT>::ROW;
  constexpr int WN = 4 * CT * 16;
  constexpr int FMTB = (FMT == LORA_W_FP8_E4M3) ? 0 : 4;
  uint8_t* xs = reinterpret_cast<uint8_t*>(smem);               // [TT*16][ROW]
  uint8_t* ss = xs + TT * 16 * ROW;                             // [TT*16][KC/32]
  int* flag = reinterpret_cast<int*>(ss + TT * 16 * (KC / 32) + 16);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, g = lane >> 4;
  const int ks = item % p.ksplit;
  const int tile = item / p.ksplit;
  const int cb = tile % p.n_cb, tb = tile / p.n_cb;
  const int row0 = tb * TT * 16;
  const int nw0 = cb * WN + wave * CT * 16;
  const int K = p.K;

  const uint8_t* wrow[CT];
  const uint8_t* wsrow[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const long n = nw0 + ct * 16 + li;
    if (FMT == LORA_W_FP8_E4M3) {
      wrow[ct] = p.wq + n * K + 16 * g;
      wsrow[ct] = nullptr;
    } else {
      wrow[ct] = p.wq + n * (K / 2) + 16 * g;
      wsrow[ct] = p.ws_fp4 + n * (K / 32) + g;
    }
  }

  v4f acc[TT][CT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[tt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  const int kb = ks * p.krange, ke = min(K, kb + p.krange);
  for (int kc0 = kb; kc0 < ke; kc0 += KC) {
    const int kcl = min(KC, ke - kc0);
    const int nsteps = kcl >> 7;
    // 1. W fragments of the chunk
    uint4 wlo[STEPS][CT], whi[STEPS][CT];
    int wsc[STEPS][CT];
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int k = kc0 + s * 128;
        if (s < nsteps) {
          if (FMT == LORA_W_FP8_E4M3) {
            wlo[s][ct] = ldg16(wrow[ct] + k);
            whi[s][ct] = ldg16(wrow[ct] + k + 64);
            wsc[s][ct] = 127;
          } else {
            wlo[s][ct] = ldg16(wrow[ct] + k / 2);
            whi[s][ct] = zero4();
            wsc[s][ct] = wsrow[ct][k / 32];
          }
        } else {
          wlo[s][ct] = zero4();
          whi[s][ct] = zero4();
          wsc[s][ct] = 127;
        }
      }
    // 2. x chunk -> MXFP8 in LDS
    const int bpr = kcl >> 5;  // 32-blocks per row in this chunk
    const int nblk = TT * 16 * bpr;
    for (int b = tid; b < nblk; b += 256) {
      const int row = b / bpr, k32 = b - row * bpr;
      const int tok = row0 + row;
      uint4 out[2];
      uint32_t code = 0;
      if (tok < p.T) {
        if (XQ) {
          const uint8_t* src = p.xq + (long)tok * K + kc0 + k32 * 32;
          out[0] = ldg16(src);
          out[1] = ldg16(src + 16);
          code = p.xsc[(long)tok * (K / 32) + (kc0 >> 5) + k32];
        } else {
          const uint16_t* src = p.x + (long)tok * K + kc0 + k32 * 32;
          uint4 in[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) in[i] = ldg16(src + 8 * i);
          code = mx_block_code(in);
          mx_block_quant(in, code, out);
        }
      } else {
        out[0] = zero4();
        out[1] = zero4();
      }
      *reinterpret_cast<uint4*>(xs + row * ROW + k32 * 32) = out[0];
      *reinterpret_cast<uint4*>(xs + row * ROW + k32 * 32 + 16) = out[1];
      ss[row * (KC / 32) + k32] = (uint8_t)code;
    }
    __syncthreads();
    // 3. MFMAs
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (s >= nsteps) break;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int row = tt * 16 + li;
        const uint8_t* xp = xs + row * ROW + s * 128 + 16 * g;
        const uint4 alo = *reinterpret_cast<const uint4*>(xp);
        const uint4 ahi = *reinterpret_cast<const uint4*>(xp + 64);
        const int sa = ss[row * (KC / 32) + s * 4 + g];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[tt][ct] = mfma_scaled_16x16x128<FMTB>(alo, ahi, wlo[s][ct], whi[s][ct], acc[tt][ct], sa, wsc[s][ct]);
      }
    }
    __syncthreads();
  }

  // ---- K-split reduction (deterministic: summed in split order by the last arriver)
  const int ntiles = p.n_cb * p.n_tb;
  if (p.ksplit > 1) {
    constexpr int PER_WAVE = TT * CT * 256;
    float* mine = p.gpart + (((long)tile * p.ksplit + ks) * 4 + wave) * PER_WAVE;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) st_agent(mine + ((tt * CT + ct) * 64 + lane) * 4 + v, acc[tt][ct][v]);
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      const int prev = add_agent(&p.tile_ctr[tile], 1);
      *flag = (prev == p.ksplit - 1);
    }
    __syncthreads();
    if (!*flag) return;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
        for (int k2 = 0; k2 < p.ksplit; ++k2) {
          const float* src = p.gpart + (((long)tile * p.ksplit + k2) * 4 + wave) * PER_WAVE + ((tt * CT + ct) * 64 + lane) * 4;
          v4f v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = ld_agent(src + e);
          sum += v;
        }
        acc[tt][ct] = sum;
      }
    if (tid == 0) set_agent(&p.tile_ctr[tile], 0);
  }

  // ---- epilogue: channel scale
  if (FMT == LORA_W_FP8_E4M3) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float sw = p.ws_fp8[nw0 + ct * 16 + li];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[tt][ct] *= sw;
    }
  }

  // ---- epilogue: adapter up-projection
  if (p.lora) {
    if (p.n_shrink > 0) {
      if (tid == 0) {
        int spins = 0;
        while (ld_agent(p.shrink_done) < p.n_shrink) {
          __builtin_amdgcn_s_sleep(4);
          if (++spins > p.spin_limit) {
            set_agent(p.status, 1);
            break;
          }
        }
        const int prev = add_agent(p.wait_done, 1);
        if (prev == ntiles - 1) {
          set_agent(p.shrink_done, 0);
          set_agent(p.wait_done, 0);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int tok = row0 + tt * 16 + li;  // A-operand row of this lane
      const int a = (tok < p.T) ? p.ids[tok] : -1;
      const bool valid = (a >= 0 && a < p.n_ad);
      unsigned long long pending = __ballot(valid && g == 0);
      while (pending) {
        const int leader = __ffsll((long long)pending) - 1;
        const int la = __shfl(a, leader);
        const unsigned long long same = __ballot(valid && g == 0 && a == la);
        const bool mine = valid && (a == la);
        const int rk = p.ranks[la];
        const int r = (rk < 8 || rk > p.r_max || (rk & 7)) ? 0 : rk;  // unsupported rank: skipped
        const float sa = p.scales[la];
        const uint16_t* __restrict__ Bt = reinterpret_cast<const uint16_t*>(p.B_ptrs[la]);
        for (int j0 = 0; j0 < r; j0 += 32) {
          const int j = j0 + 8 * g;
          uint4 aop = zero4();
          if (mine && j < r) {
            const float* tp = p.t + (long)tok * p.r_max + j;
            float tv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tv[e] = sa * ld_agent(tp + e);
            aop.x = f32_to_bf16_rne(tv[0]) | (f32_to_bf16_rne(tv[1]) << 16);
            aop.y = f32_to_bf16_rne(tv[2]) | (f32_to_bf16_rne(tv[3]) << 16);
            aop.z = f32_to_bf16_rne(tv[4]) | (f32_to_bf16_rne(tv[5]) << 16);
            aop.w = f32_to_bf16_rne(tv[6]) | (f32_to_bf16_rne(tv[7]) << 16);
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const long n = nw0 + ct * 16 + li;
            const uint4 bop = (j < r) ? ldg16(Bt + n * r + j) : zero4();
            acc[tt][ct] = mfma_bf16_16x16x32(aop, bop, acc[tt][ct]);
          }
        }
        pending &= ~same;
      }
    }
  }

  // ---- store bf16 (round to nearest even)
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int n = nw0 + ct * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = row0 + tt * 16 + 4 * g + v;
        if (tok < p.T) p.y[(long)tok * p.N + n] = (uint16_t)f32_to_bf16_rne(acc[tt][ct][v]);
      }
    }
}

template <int FMT, int TT, int CT, bool XQ, int TG, int U>
__global__ __launch_bounds__(256) void k_layer(ShrinkParams sp, GemmParams gp) {
  extern __shared__ __align__(16) char smem[];
  const int b = blockIdx.x;
  if (b < gp.n_shrink) {
    shrink_item<TG, U>(sp, b, smem);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) add_agent(gp.shrink_done, 1);
    return;
  }
  gemm_item<FMT, TT, CT, XQ>(gp, b - gp.n_shrink, smem);
}

// ======================================================================================
// Launchers
// ======================================================================================
size_t shrink_smem_bytes(int TG) { return (size_t)4 * TG * 4 * 256 * sizeof(float) + 64; }

template <int TT>
size_t gemm_smem_bytes() {
  return (size_t)TT * 16 * ChunkK<TT>::ROW + TT * 16 * (ChunkK<TT>::KC / 32) + 64;
}

template <typename KernelT>
static hipError_t launch(KernelT kern, int grid, size_t smem, hipStream_t stream, const ShrinkParams& sp,
                         const GemmParams& gp) {
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), smem, stream, sp, gp);
  return hipGetLastError();
}

template <int FMT, int TT, int CT, bool XQ>
static hipError_t launch_layer_t(int tg, int grid, hipStream_t stream, const ShrinkParams& sp, const GemmParams& gp) {
  const size_t sm = std::max(gemm_smem_bytes<TT>(), gp.n_shrink > 0 ? shrink_smem_bytes(tg) : (size_t)0);
  if (tg == 1) return launch(k_layer<FMT, TT, CT, XQ, 1, 4>, grid, sm, stream, sp, gp);
  return launch(k_layer<FMT, TT, CT, XQ, 4, 1>, grid, sm, stream, sp, gp);
}

template <int FMT>
static hipError_t launch_layer_f(const LayerPlan& pl, int grid, hipStream_t stream, const ShrinkParams& sp,
                                 const GemmParams& gp) {
  const int tg = pl.shrink_tg;
  if (pl.TT == 1 && pl.CT == 1 && !pl.XQ) return launch_layer_t<FMT, 1, 1, false>(tg, grid, stream, sp, gp);
  if (pl.TT == 4 && pl.CT == 1 && !pl.XQ) return launch_layer_t<FMT, 4, 1, false>(tg, grid, stream, sp, gp);
  if (pl.TT == 8 && pl.CT == 1 && !pl.XQ) return launch_layer_t<FMT, 8, 1, false>(tg, grid, stream, sp, gp);
  if (pl.TT == 8 && pl.CT == 2 && !pl.XQ) return launch_layer_t<FMT, 8, 2, false>(tg, grid, stream, sp, gp);
  if (pl.TT == 8 && pl.CT == 1 && pl.XQ) return launch_layer_t<FMT, 8, 1, true>(tg, grid, stream, sp, gp);
  if (pl.TT == 8 && pl.CT == 2 && pl.XQ) return launch_layer_t<FMT, 8, 2, true>(tg, grid, stream, sp, gp);
  if (pl.TT == 8 && pl.CT == 4 && pl.XQ) return launch_layer_t<FMT, 8, 4, true>(tg, grid, stream, sp, gp);
  return hipErrorInvalidValue;
}

hipError_t launch_layer(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp, const GemmParams& gp) {
  const int grid = gp.n_shrink + pl.n_gemm_wg;
  if (pl.fmt == LORA_W_FP8_E4M3) return launch_layer_f<LORA_W_FP8_E4M3>(pl, grid, stream, sp, gp);
  return launch_layer_f<LORA_W_MXFP4_E2M1>(pl, grid, stream, sp, gp);
}

hipError_t launch_shrink(int tg, int grid, hipStream_t stream, const ShrinkParams& sp) {
  const size_t sm = shrink_smem_bytes(tg);
  if (tg == 1) {
    hipLaunchKernelGGL((k_shrink<1, 4>), dim3(grid), dim3(256), sm, stream, sp);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_shrink<4, 1>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_shrink<4, 1>), dim3(grid), dim3(256), sm, stream, sp);
  }
  return hipGetLastError();
}

hipError_t launch_build_segments(const int* ids, int T, int n_ad, int* seg, int* sorted, int* err, hipStream_t s) {
  hipLaunchKernelGGL(k_build_segments, dim3(1), dim3(SEG_THREADS), 0, s, ids, T, n_ad, seg, sorted, err);
  return hipGetLastError();
}

hipError_t launch_quant(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s) {
  const long blocks = ((long)T * (K / 32) + 255) / 256;
  const int grid = (int)std::min<long>(blocks, 8192);
  hipLaunchKernelGGL(k_quant_mxfp8, dim3(grid), dim3(256), 0, s, x, T, K, xq, xsc);
  return hipGetLastError();
}

hipError_t launch_expand(const ExpandParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_expand, dim3((p.N + 255) / 256, p.T), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const int grid = (int)std::min<size_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace lora

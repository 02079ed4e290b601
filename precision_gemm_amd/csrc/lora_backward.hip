// Backward of the multi-tenant LoRA layer on a frozen FP8 base, for gfx950.
//
// The "EpiLoRA" abstract has the trainer compute on the serving engine's FP8 weights
// (no 16-bit copy of W) with activations kept in 16 bits.  For the 16-bit-activation
// layer y[t] = x[t] W_d + s_a (x[t] A_a) B_a, with W_d frozen and the gradient dY of a
// loss with respect to y given in bf16, the chain rule over the tokens R_a of each adapter
// (the segments of "Punica" README, Overview) gives
//
//     u[t]  = dY[t] B_a^T                       (a down-projection over N)
//     dX[t] = dY[t] W_d^T + s_a u[t] A_a^T      (a GEMM over N plus an up-projection)
//     dA_a  = s_a X_a^T U_a,   dB_a = s_a T_a^T dY_a   (contractions over a segment)
//
// Kernels:
//   k_pack_weight_t     W^T in the packed order the dX GEMM reads (offline, like W's own pack).
//   k_pack_adapter_bwd  B_a in bf16 MFMA operand order over N, A_a as rows [K][rank_pad(r_a)].
//   (u)                 the forward down-projection kernel, run on dY with B_a in place of A_a.
//   k_bwd_dx            dX on bf16 MFMA: dY staged in LDS, W^T codes straight from their
//                       packed tiles and widened in registers, the adapter term added per
//                       adapter present in the tile, bf16 stores through LDS.
//   k_bwd_grad          dA and dB: per (adapter, 128 rows of K or N) item, the segment's
//                       tokens in 32-token chunks on bf16 MFMA (the fp32 side split into two
//                       bf16 terms), the waves' partial sums combined in a fixed order.
#include "device_common.hpp"
#include "lora_kernels.hpp"

namespace lora {

typedef float v2f __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------
// Packs
// ---------------------------------------------------------------------------------

// W^T for the dX GEMM, FP8: tiles (kt, ns) of 16 rows k by 64 channels n, each 1 KB:
// byte e of lane l (i = l % 16, g = l / 16) of tile (kt, ns) holds the code of
// W[n = 64 ns + 16 g + e][k = 16 kt + i], tile (kt, ns) at byte ((kt (N/64) + ns) 64 + l) 16.
// One thread per 16-byte output.
__global__ void k_pack_weight_t(const uint8_t* __restrict__ q, int N, int K, uint8_t* __restrict__ qt) {
  const long o = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int nsn = N >> 6;
  if (o >= (long)(K >> 4) * nsn * 64) return;
  const int l = (int)(o & 63);
  const long tile = o >> 6;
  const int ns = (int)(tile % nsn), kt = (int)(tile / nsn);
  const int k = 16 * kt + (l & 15), n0 = 64 * ns + 16 * (l >> 4);
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) v |= (uint32_t)q[(long)(n0 + 4 * d + e) * K + k] << (8 * e);
    w[d] = v;
  }
  *reinterpret_cast<uint4*>(qt + o * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Bop: B_a (bf16 [r][N]) in operand order over N -- element (j, n) at a_index(j, n, N), the
// layout of the forward's packed A with N in place of K, zero past r.  Ar: A_a (bf16 [K][r])
// as [K][rank_pad(r)], zero past r.  One thread per output element.
__global__ void k_pack_adapter_bwd(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int K, int N,
                                   int r, uint16_t* __restrict__ Bop, uint16_t* __restrict__ Ar) {
  const long o = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long nb = (long)a_tiles(r) * 16 * N;
  const int rp = rank_pad(r);
  if (o < nb) {
    const int e = (int)(o & 7), ji = (int)((o >> 3) & 15), gq = (int)((o >> 7) & 3), h = (int)((o >> 9) & 1);
    const long rest = o >> 10;
    const int ns = (int)(rest % (N >> 6)), jt = (int)(rest / (N >> 6));
    const int j = 16 * jt + ji, n = 64 * ns + 16 * gq + 8 * h + e;
    Bop[o] = j < r ? B[(long)j * N + n] : (uint16_t)0;
  } else if (o < nb + (long)K * rp) {
    const long q = o - nb;
    const int k = (int)(q / rp), j = (int)(q % rp);
    Ar[q] = j < r ? A[(long)k * r + j] : (uint16_t)0;
  }
}

hipError_t launch_pack_weight_t(const uint8_t* q, int N, int K, uint8_t* qt, hipStream_t s) {
  const long n16 = (long)(K / 16) * (N / 64) * 64;
  hipLaunchKernelGGL(k_pack_weight_t, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, q, N, K, qt);
  return hipGetLastError();
}

hipError_t launch_pack_adapter_bwd(const uint16_t* A, const uint16_t* B, int K, int N, int r, uint16_t* Bop,
                                   uint16_t* Ar, hipStream_t s) {
  const long total = (long)a_tiles(r) * 16 * N + (long)K * rank_pad(r);
  hipLaunchKernelGGL(k_pack_adapter_bwd, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, A, B, K, N, r, Bop,
                     Ar);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------------

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ldg16f(const float* p) { return __builtin_bit_cast(float4, ldg16(p)); }

// s = hi + lo with hi = bf16(s) and lo = bf16(s - hi): |s - hi - lo| <= 2^-9 |s - hi| <= 2^-17 |s|
// (round to nearest even at both steps), so two bf16 MFMAs carry an fp32 operand to about
// 17 bits.  Eight values -> two bf16 operands.
__device__ __forceinline__ void split8(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    h[d] = bf16x2_rne(v[2 * d], v[2 * d + 1]);
    l[d] = bf16x2_rne(v[2 * d] - bf16_lo(h[d]), v[2 * d + 1] - bf16_hi(h[d]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------------
// dX = dY W_d^T + s_a u A_a^T
//
// Workgroup tile: 64 rows (tokens) x 256 columns (k), four waves of 64 x 64, two workgroups
// per CU (their barriers are independent, so one's loads, widening and waits overlap the
// other's MFMAs).  dY W_d^T = (dY diag(s_w)) codes^T: per 64-channel step, dY [64][64] times
// the step's channel scales, rounded to bf16 (nearest even), is staged in LDS (loaded a step
// ahead, double buffered; each value scaled once per workgroup); each wave reads its four W^T
// tiles (1 KB of consecutive memory each) straight into registers, a step ahead, and widens
// the codes to bf16 exactly (one conversion per two codes); two bf16 MFMAs per 16 x 16 block
// cover the 64 channels (lane group g supplies channels 16 g .. 16 g + 7 to the first and
// 16 g + 8 .. 16 g + 15 to the second, the same assignment on both operands).
// Adapter term: the rows' s_a u[t] split into two bf16 terms and staged in LDS; for each
// adapter present in the tile (in increasing id order) and each 32 ranks, two MFMAs per
// block with the rows of other adapters zeroed and A_a rows [K][rank_pad] as the other
// operand.  Rows whose adapter id or rank is invalid get the base term only.
// Short batches (too few tiles to fill the GPU) split the contraction over N: workgroup
// (tile, range) walks its range of steps and writes fp32 partial sums, range 0 with the
// adapter term, and k_bwd_dx_reduce adds the ranges in order.
// ---------------------------------------------------------------------------------

constexpr int BX_RS = 144;              // LDS row stride (bytes): 64 bf16 + 16 bytes of bank offset
constexpr int BX_ROWS = 64;             // rows of a workgroup tile
constexpr int BX_BUF = BX_ROWS * BX_RS; // one staged step

__global__ __launch_bounds__(256, 2) void k_bwd_dx(BwdDxParams p) {
  __shared__ __align__(16) uint8_t lds[2 * BX_BUF];
  __shared__ int rid[BX_ROWS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;

  // tile order: workgroup b runs on XCD b % 8; each XCD takes a contiguous run of (tile,
  // range) items in row-block-major order, so that the column blocks of a row block (and the
  // ranges of a tile) share its L2 for dY
  const int nitems = p.n_tb * p.n_kb * p.n_split;
  int item = blockIdx.x;
  if ((nitems & 7) == 0) item = (item & 7) * (nitems >> 3) + (item >> 3);
  const int tile = item / p.n_split, split = item - tile * p.n_split;
  const int tb = tile / p.n_kb, kb = tile % p.n_kb;
  const int t0 = BX_ROWS * tb, k0w = 256 * kb + 64 * w;
  const int NI = p.N >> 6, nkt = p.K >> 4;
  // this workgroup's steps [it0, it1): an even count (split_steps is even, and so is NI)
  const int it0 = split * p.split_steps, it1 = min(NI, it0 + p.split_steps);

  // dY staging: thread loads row srow + 32 q (q = 0, 1), 16-byte part spart (8 channels)
  const int srow = tid >> 3, spart = tid & 7;
  const uint16_t* dyp[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) dyp[q] = p.dy + (long)min(t0 + srow + 32 * q, p.T - 1) * p.N + 8 * spart;
  const uint8_t* wp[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) wp[ct] = p.wt + ((long)min((k0w >> 4) + ct, nkt - 1) * NI * 64 + lane) * 16;

  // dY staging: the thread's 8 channels 64 st + 8 spart .. + 7 share their 8 scales (two rows)
  auto load_dy = [&](uint4 (&d)[2], float4 (&sv)[2], int st) {
    sv[0] = ldg16f(p.wsc + 64 * st + 8 * spart);
    sv[1] = ldg16f(p.wsc + 64 * st + 8 * spart + 4);
#pragma unroll
    for (int q = 0; q < 2; ++q) d[q] = ldg16(dyp[q] + 64 * st);
  };
  auto load_w = [&](uint4 (&wv)[4], int st) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) wv[ct] = ldg16(wp[ct] + (long)st * 1024);
  };
  // dY x channel scale -> bf16 (round to nearest even) into LDS buffer buf
  auto store_dy = [&](const uint4 (&d)[2], const float4 (&sv)[2], int buf) {
    const float sc[8] = {sv[0].x, sv[0].y, sv[0].z, sv[0].w, sv[1].x, sv[1].y, sv[1].z, sv[1].w};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t wv[4] = {d[q].x, d[q].y, d[q].z, d[q].w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = bf16x2_rne(bf16_lo(wv[e]) * sc[2 * e], bf16_hi(wv[e]) * sc[2 * e + 1]);
      *reinterpret_cast<uint4*>(lds + buf * BX_BUF + (srow + 32 * q) * BX_RS + 16 * spart) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  // W^T of a step is loaded a step ahead into one of two register sets used alternately (no
  // register copies, which would wait for the loads): N / 64 steps, an even number
  uint4 dn[2], wA[4], wB[4];
  float4 sn[2];
  load_dy(dn, sn, it0);
  load_w(wA, it0);
  store_dy(dn, sn, 0);
  __syncthreads();

  v4f acc[4][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[tt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int it, const uint4 (&wc)[4], uint4 (&wn)[4]) {
    const int nx = min(it + 1, it1 - 1);  // the last step reloads itself: uniform code
    load_dy(dn, sn, nx);
    load_w(wn, nx);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay at the top: a whole step hides them
    // W^T codes -> bf16, exact: codes e = 8 s .. 8 s + 7 of the lane's 16 are operand s
    uint4 wb[4][2];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint2 c0 = fp8x4_to_bf16(wc[ct].x), c1 = fp8x4_to_bf16(wc[ct].y);
      const uint2 c2 = fp8x4_to_bf16(wc[ct].z), c3 = fp8x4_to_bf16(wc[ct].w);
      wb[ct][0] = make_uint4(c0.x, c0.y, c1.x, c1.y);
      wb[ct][1] = make_uint4(c2.x, c2.y, c3.x, c3.y);
    }
    const uint8_t* B0 = lds + ((it - it0) & 1) * BX_BUF;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint8_t* ra = B0 + (16 * tt + i) * BX_RS + 32 * g;
      const uint4 a0 = lds16(ra), a1 = lds16(ra + 16);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[tt][ct] = mfma_bf16_16x16x32(a0, wb[ct][0], acc[tt][ct]);
        acc[tt][ct] = mfma_bf16_16x16x32(a1, wb[ct][1], acc[tt][ct]);
      }
    }
    store_dy(dn, sn, (it - it0 + 1) & 1);
    __syncthreads();
  };
  for (int it = it0; it < it1; it += 2) {
    step(it, wA, wB);
    step(it + 1, wB, wA);
  }
  const bool with_term = split == 0;  // the adapter term: once, in range 0

  // ---- adapter term
  if (with_term) {
    if (tid < BX_ROWS) {
      const int t = t0 + tid;
      int a = -1;
      if (t < p.T) {
        a = p.ids[t];
        if (a < 0 || a >= p.n_ad) {
          a = -1;
        } else {
          const int r = p.ranks[a];
          if (r < 1 || r > p.r_lim) a = -1;
        }
      }
      rid[tid] = a;
    }
    __syncthreads();
    // s_a u[t] as two bf16 terms: hi in buffer 0, lo in buffer 1, [row][64 ranks]
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = srow + 32 * q;
      const int a = rid[row];
      float v[8];
      if (a >= 0) {
        const int r = p.ranks[a];
        const float sa = p.scales[a];
        const float* urow = p.u + (long)(t0 + row) * p.r_lim;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 8 * spart + e;
          v[e] = j < r ? sa * urow[j] : 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
      }
      uint4 hi, lo;
      split8(v, hi, lo);
      *reinterpret_cast<uint4*>(lds + row * BX_RS + 16 * spart) = hi;
      *reinterpret_cast<uint4*>(lds + BX_BUF + row * BX_RS + 16 * spart) = lo;
    }
    __syncthreads();
    int prev = -1;
    for (;;) {
      const int c = rid[lane];
      int m = c > prev ? c : 0x7fffffff;
      m = wave_min(m);
      if (m == 0x7fffffff) break;
      const int a = __builtin_amdgcn_readfirstlane(m);
      prev = a;
      const int r = p.ranks[a], rp = rank_pad(r);
      const uint16_t* Ar = reinterpret_cast<const uint16_t*>(p.Ar_ptrs[a]);
      for (int rs = 0; 32 * rs < r; ++rs) {
        const int jj = 32 * rs + 8 * g;
        const int off = min(jj, rp - 8);
        uint4 bop[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int k = min(k0w + 16 * ct + i, p.K - 1);
          bop[ct] = keep_bf16(ldg16(Ar + (long)k * rp + off), r - jj);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int row = 16 * tt + i;
          const bool mine = rid[row] == a;
          const int o = row * BX_RS + 64 * rs + 16 * g;
          const uint4 ah = mine ? lds16(lds + o) : zero4();
          const uint4 al = mine ? lds16(lds + BX_BUF + o) : zero4();
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            acc[tt][ct] = mfma_bf16_16x16x32(ah, bop[ct], acc[tt][ct]);
            acc[tt][ct] = mfma_bf16_16x16x32(al, bop[ct], acc[tt][ct]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- a range of a split contraction: fp32 partial sums, not rounded
  if (p.n_split > 1) {
    float* P = p.part + (long)split * p.T * p.K;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = t0 + 16 * tt + 4 * g + v, k = k0w + 16 * ct + i;
          if (t < p.T && k < p.K) P[(long)t * p.K + k] = acc[tt][ct][v];
        }
    return;
  }

  // ---- bf16 stores through LDS, 32 rows per pass: wave w's region holds its 32 x 64 block
  uint8_t* reg = lds + w * (32 * BX_RS);
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
#pragma unroll
    for (int tq = 0; tq < 2; ++tq)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<uint16_t*>(reg + (16 * tq + 4 * g + v) * BX_RS + 2 * (16 * ct + i)) =
              (uint16_t)f32_to_bf16_rne(acc[2 * ph + tq][ct][v]);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = lane + 64 * c;           // 32 rows x 8 parts of 16 bytes
      const int row = idx >> 3, part = idx & 7;
      const int t = t0 + 32 * ph + row, k = k0w + 8 * part;
      const uint4 v = lds16(reg + row * BX_RS + 16 * part);
      if (t < p.T && k < p.K) *reinterpret_cast<uint4*>(p.dx + (long)t * p.K + k) = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------
// dA_a = s_a X_a^T U_a and dB_a = s_a T_a^T dY_a (the second computed as its transpose,
// dY_a^T T_a): G [C][r] = s M[R]^T V[R] with M bf16 [T][C], V fp32 [T][r_lim].
//
// Item (adapter a, 64 rows c0 .. c0 + 63 of C), two workgroups per CU: the segment's
// positions go in rounds of 1024 whose token indices are staged in LDS; the four waves take
// the round's 32-token chunks in turn.  Lane (i, g) loads, for tokens q = 8 g .. 8 g + 7 of
// a chunk, the 8 bytes M[tok_q][c0 + 4 i .. + 3] and transposes the 8 x 4 block in
// registers: operand m holds M[tok_q][c0 + 4 i + m] over q, the A operand of MFMA block m
// whose row i is C-row c0 + 4 i + m.  The B operand holds V[tok_q][16 jt + i] over q, split
// into two bf16 terms.  A chunk's rows and V are loaded while the previous chunk computes.
// The waves' sums are combined as ((w0 + w2) + (w1 + w3)): a fixed order, so the result is
// bitwise reproducible.
// ---------------------------------------------------------------------------------

constexpr int GR_ROWS = 64;  // rows of C per item
constexpr int GR_RS = 68;    // floats per LDS row of a 64 x 64 partial-sum slot
constexpr int GR_ROUND = 1024;

__device__ __forceinline__ uint32_t dw(const uint2& v, int d) { return d == 0 ? v.x : v.y; }

// NJT: 16-rank tiles loaded per token (ceil(r_max / 16)); every load is unconditional (clamped
// addresses, values masked at use), so the compiler's wait counts see the prefetch through.
template <int NJT>
__global__ __launch_bounds__(256, 2) void k_bwd_grad(BwdGradParams p) {
  __shared__ float red[2][GR_ROWS * GR_RS];
  __shared__ int stok[GR_ROUND];
  const int per_ad = p.nkb + p.nnb;
  const int a = blockIdx.x / per_ad, blk = blockIdx.x % per_ad;
  const bool isA = blk < p.nkb;
  const int c0 = GR_ROWS * (isA ? blk : blk - p.nkb);
  const int C = isA ? p.K : p.N;
  const uint16_t* M = isA ? p.x : p.dy;
  const float* V = isA ? p.u : p.t;
  const int r = p.ranks[a];
  const int s_beg = p.empty ? 0 : p.seg_indptr[a], s_end = p.empty ? 0 : p.seg_indptr[a + 1];
  if (r < 1 || r > p.r_lim) {
    if (threadIdx.x == 0 && blk == 0 && s_end > s_beg && p.status) or_agent(p.status, 2);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int njt = (r + 15) >> 4;

  v4f acc[4][NJT];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) acc[m][jt] = v4f{0.f, 0.f, 0.f, 0.f};

  struct Chunk {
    uint2 mr[8];
    float v[NJT][8];
  };
  int nin = 1;  // positions of the current round staged in stok (reads past them take its last)
  // loads of chunk c of the round (positions base + 32 c ..): rows of M and V; positions
  // past the segment read the round's last token and are zeroed at use
  auto load = [&](Chunk& ch, int c) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int tok = stok[min(32 * c + 8 * g + q, nin - 1)];
      ch.mr[q] = *reinterpret_cast<const uint2*>(M + (long)tok * C + c0 + 4 * i);
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) ch.v[jt][q] = V[(long)tok * p.r_lim + min(16 * jt + i, r - 1)];
    }
  };
  auto compute = [&](const Chunk& ch, int base, int c) {
    bool ok[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) ok[q] = base + 32 * c + 8 * g + q < s_end;
    uint4 op[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint2 lo2 = ok[2 * d] ? ch.mr[2 * d] : make_uint2(0u, 0u);
        const uint2 hi2 = ok[2 * d + 1] ? ch.mr[2 * d + 1] : make_uint2(0u, 0u);
        const uint32_t lo = dw(lo2, m >> 1), hi = dw(hi2, m >> 1);
        o[d] = (m & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u) : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      op[m] = make_uint4(o[0], o[1], o[2], o[3]);
    }
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      if (jt < njt) {
        const bool jok = 16 * jt + i < r;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = (ok[q] && jok) ? ch.v[jt][q] : 0.f;
        uint4 vh, vl;
        split8(v, vh, vl);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[m][jt] = mfma_bf16_16x16x32(op[m], vh, acc[m][jt]);
          acc[m][jt] = mfma_bf16_16x16x32(op[m], vl, acc[m][jt]);
        }
      }
    }
  };

  for (int base = s_beg; base < s_end; base += GR_ROUND) {
    __syncthreads();  // the previous round's tokens are no longer read
    nin = min(GR_ROUND, s_end - base);  // the round's positions: only these are staged
    for (int o = tid; o < nin; o += 256) stok[o] = p.sorted_tok[base + o];
    __syncthreads();
    const int nch = (nin + 31) / 32;  // chunks of this round
    // wave w takes chunks w, w + 4, ...; two register sets alternate, the next chunk's loads
    // in flight while one computes (the loads past the last chunk reload it, unused)
    Chunk A, B;
    load(A, min(w, nch - 1));
    for (int c = w; c < nch; c += 8) {
      load(B, min(c + 4, nch - 1));
      compute(A, base, c);
      load(A, min(c + 8, nch - 1));
      if (c + 4 < nch) compute(B, base, c + 4);
    }
  }

  // combine the waves: slot row 16 m + rho holds C-row c0 + 4 rho + m (rho = 4 g + v)
  auto put = [&](float* s) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[(16 * m + 4 * g + v) * GR_RS + 16 * jt + i] = acc[m][jt][v];
  };
  auto add = [&](const float* s) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][jt][v] += s[(16 * m + 4 * g + v) * GR_RS + 16 * jt + i];
  };
  __syncthreads();
  if (w >= 2) put(red[w - 2]);
  __syncthreads();
  if (w < 2) add(red[w]);
  __syncthreads();
  if (w == 1) put(red[0]);
  __syncthreads();
  if (w == 0) {
    add(red[0]);
    const float sa = p.scales[a];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc[m][jt] *= sa;
    put(red[1]);
  }
  __syncthreads();
  const float* fin = red[1];
  float* out = reinterpret_cast<float*>(isA ? p.dA_ptrs[a] : p.dB_ptrs[a]);
  if (isA) {  // dA_a [K][r]: rows c0 .. c0 + 63 are 64 r consecutive floats
    for (int o = tid; o < GR_ROWS * r; o += 256) {
      const int row = o / r, j = o - row * r;
      out[(long)(c0 + row) * r + j] = fin[(16 * (row & 3) + (row >> 2)) * GR_RS + j];
    }
  } else {    // dB_a [r][N]: for each rank, 64 consecutive columns
    for (int o = tid; o < GR_ROWS * r; o += 256) {
      const int j = o >> 6, col = o & 63;
      out[(long)j * p.N + c0 + col] = fin[(16 * (col & 3) + (col >> 2)) * GR_RS + j];
    }
  }
}

// dx[t][k] = bf16(sum over the ranges, in order, of the partial sums): four columns a thread
__global__ __launch_bounds__(256) void k_bwd_dx_reduce(BwdDxParams p) {
  const long q = (long)blockIdx.x * 256 + threadIdx.x;  // index of four consecutive elements
  const long n4 = (long)p.T * p.K / 4;
  if (q >= n4) return;
  const long stride = (long)p.T * p.K;
  float4 acc = *reinterpret_cast<const float4*>(p.part + 4 * q);
  for (int r = 1; r < p.n_split; ++r) {
    const float4 v = *reinterpret_cast<const float4*>(p.part + r * stride + 4 * q);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *reinterpret_cast<uint2*>(p.dx + 4 * q) = make_uint2(bf16x2_rne(acc.x, acc.y), bf16x2_rne(acc.z, acc.w));
}

// out[tok][j] = sum over the K-parts in order (j < r_a), 0 for r_a <= j < r_lim: one thread
// per element
__global__ __launch_bounds__(256) void k_part_reduce(const float* __restrict__ part, int kparts, int T, int r_lim,
                                                     const int* __restrict__ ids, const int* __restrict__ ranks,
                                                     int n_ad, float* __restrict__ out) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)T * r_lim) return;
  const int tok = (int)(idx / r_lim), j = (int)(idx - (long)tok * r_lim);
  const int a = ids[tok];
  if (a < 0 || a >= n_ad) return;
  const int r = ranks[a];
  if (r < 1 || r > r_lim) return;
  float v = 0.f;
  if (j < r)
    for (int q = 0; q < kparts; ++q) v += part[((long)q * T + tok) * r_lim + j];
  out[idx] = v;
}

hipError_t launch_part_reduce(const float* part, int kparts, int T, int r_lim, const int* ids, const int* ranks,
                              int n_ad, float* out, hipStream_t s) {
  const long n = (long)T * r_lim;
  hipLaunchKernelGGL(k_part_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, kparts, T, r_lim, ids,
                     ranks, n_ad, out);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dx, dim3(p.n_tb * p.n_kb * p.n_split), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dx_reduce(const BwdDxParams& p, hipStream_t s) {
  const long n4 = (long)p.T * p.K / 4;
  hipLaunchKernelGGL(k_bwd_dx_reduce, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_grad(const BwdGradParams& p, hipStream_t s) {
  const dim3 grid(p.n_ad * (p.nkb + p.nnb));
  switch ((p.r_lim + 15) >> 4) {
    case 1: hipLaunchKernelGGL(k_bwd_grad<1>, grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_bwd_grad<2>, grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL(k_bwd_grad<3>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(k_bwd_grad<4>, grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace lora

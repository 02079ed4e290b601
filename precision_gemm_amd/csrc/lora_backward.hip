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
// Workgroup tile: 128 rows (tokens) x 256 columns (k), four waves of 128 x 64.  Per
// 64-channel step: dY [128][64] bf16 staged in LDS (loaded a step ahead, double buffered);
// each wave reads its four W^T tiles (1 KB of consecutive memory each) straight into
// registers and widens them to bf16 as code x channel scale (rounded to nearest even: the
// dequantised weight in 16 bits); two bf16 MFMAs per 16 x 16 block cover the 64 channels
// (lane group g supplies channels 16 g .. 16 g + 7 to the first and 16 g + 8 .. 16 g + 15
// to the second, the same assignment on both operands).
// Adapter term: the rows' s_a u[t] split into two bf16 terms and staged in LDS; for each
// adapter present in the tile (in increasing id order) and each 32 ranks, two MFMAs per
// block with the rows of other adapters zeroed and A_a rows [K][rank_pad] as the other
// operand.  Rows whose adapter id or rank is invalid get the base term only.
// ---------------------------------------------------------------------------------

constexpr int BX_RS = 144;              // LDS row stride (bytes): 64 bf16 + 16 bytes of bank offset
constexpr int BX_BUF = 128 * BX_RS;     // one 128-row buffer

__global__ __launch_bounds__(256, 1) void k_bwd_dx(BwdDxParams p) {
  __shared__ __align__(16) uint8_t lds[2 * BX_BUF];
  __shared__ int rid[128];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;

  // tile order: workgroup b runs on XCD b % 8; each XCD takes a contiguous run of tiles in
  // row-block-major order, so that the column blocks of a row block share its L2 for dY
  const int ntiles = p.n_tb * p.n_kb;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
  const int tb = tile / p.n_kb, kb = tile % p.n_kb;
  const int t0 = 128 * tb, k0w = 256 * kb + 64 * w;
  const int NI = p.N >> 6, nkt = p.K >> 4;

  // dY staging: thread loads row srow + 32 q, 16-byte part spart (8 channels)
  const int srow = tid >> 3, spart = tid & 7;
  const uint16_t* dyp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) dyp[q] = p.dy + (long)min(t0 + srow + 32 * q, p.T - 1) * p.N + 8 * spart;
  const uint8_t* wp[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) wp[ct] = p.wt + ((long)min((k0w >> 4) + ct, nkt - 1) * NI * 64 + lane) * 16;
  const float* scp = p.wsc + 16 * g;

  uint4 sd[4], wc[4];
  float4 sc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sd[q] = ldg16(dyp[q]);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) wc[ct] = ldg16(wp[ct]);
#pragma unroll
  for (int e = 0; e < 4; ++e) sc[e] = ldg16f(scp + 4 * e);
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(lds + (srow + 32 * q) * BX_RS + 16 * spart) = sd[q];
  __syncthreads();

  v4f acc[8][4];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[tt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < NI; ++it) {
    // next step's loads (the last step reloads its own: uniform code, no branch)
    const int nx = min(it + 1, NI - 1);
    uint4 sdn[4], wn[4];
    float4 scn[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sdn[q] = ldg16(dyp[q] + 64 * nx);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) wn[ct] = ldg16(wp[ct] + (long)nx * 1024);
#pragma unroll
    for (int e = 0; e < 4; ++e) scn[e] = ldg16f(scp + 64 * nx + 4 * e);

    // W^T codes -> bf16 (code x channel scale)
    const float s16[16] = {sc[0].x, sc[0].y, sc[0].z, sc[0].w, sc[1].x, sc[1].y, sc[1].z, sc[1].w,
                           sc[2].x, sc[2].y, sc[2].z, sc[2].w, sc[3].x, sc[3].y, sc[3].z, sc[3].w};
    uint4 wb[4][2];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint32_t d[4] = {wc[ct].x, wc[ct].y, wc[ct].z, wc[ct].w};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * s + h], 1.0f, false);
          const v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d[2 * s + h], 1.0f, true);
          const int e0 = 8 * s + 4 * h;
          o[2 * h] = bf16x2_rne(a.x * s16[e0], a.y * s16[e0 + 1]);
          o[2 * h + 1] = bf16x2_rne(b.x * s16[e0 + 2], b.y * s16[e0 + 3]);
        }
        wb[ct][s] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    const uint8_t* B0 = lds + (it & 1) * BX_BUF;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const uint8_t* ra = B0 + (16 * tt + i) * BX_RS + 32 * g;
      const uint4 a0 = lds16(ra), a1 = lds16(ra + 16);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[tt][ct] = mfma_bf16_16x16x32(a0, wb[ct][0], acc[tt][ct]);
        acc[tt][ct] = mfma_bf16_16x16x32(a1, wb[ct][1], acc[tt][ct]);
      }
    }
    uint8_t* B1 = lds + ((it + 1) & 1) * BX_BUF;
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(B1 + (srow + 32 * q) * BX_RS + 16 * spart) = sdn[q];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) wc[ct] = wn[ct];
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = scn[e];
    __syncthreads();
  }

  // ---- adapter term
  if (tid < 128) {
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
  for (int q = 0; q < 4; ++q) {
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
    const int c0 = rid[lane], c1 = rid[lane + 64];
    int m = 0x7fffffff;
    if (c0 > prev) m = c0;
    if (c1 > prev && c1 < m) m = c1;
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
      for (int tt = 0; tt < 8; ++tt) {
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

  // ---- bf16 stores through LDS, 64 rows per pass: wave w's region holds its 64 x 64 block
  uint8_t* reg = lds + w * (64 * BX_RS);
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
#pragma unroll
    for (int tq = 0; tq < 4; ++tq)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<uint16_t*>(reg + (16 * tq + 4 * g + v) * BX_RS + 2 * (16 * ct + i)) =
              (uint16_t)f32_to_bf16_rne(acc[4 * ph + tq][ct][v]);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int idx = lane + 64 * c;           // 64 rows x 8 parts of 16 bytes
      const int row = idx >> 3, part = idx & 7;
      const int t = t0 + 64 * ph + row, k = k0w + 8 * part;
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
// Item (adapter a, 128 rows c0 .. c0 + 127 of C): the four waves take the segment's
// 32-token chunks in turn.  Lane (i, g) loads, for tokens q = 8 g .. 8 g + 7 of the chunk,
// the 16 bytes M[tok_q][c0 + 8 i .. + 7] and transposes the 8 x 8 block in registers:
// operand m holds M[tok_q][c0 + 8 i + m] over q, the A operand of MFMA block m whose row
// i is C-row c0 + 8 i + m.  The B operand holds V[tok_q][16 jt + i] over q, split into two
// bf16 terms.  The waves' sums are combined as ((w0 + w2) + (w1 + w3)): a fixed order, so
// the result is bitwise reproducible.
// ---------------------------------------------------------------------------------

constexpr int GR_RS = 68;  // floats per LDS row of a 128 x 64 partial-sum slot

__device__ __forceinline__ uint32_t dw(const uint4& v, int d) {
  return d == 0 ? v.x : (d == 1 ? v.y : (d == 2 ? v.z : v.w));
}

__global__ __launch_bounds__(256, 1) void k_bwd_grad(BwdGradParams p) {
  __shared__ float red[2][128 * GR_RS];
  const int per_ad = p.nkb + p.nnb;
  const int a = blockIdx.x / per_ad, blk = blockIdx.x % per_ad;
  const bool isA = blk < p.nkb;
  const int c0 = 128 * (isA ? blk : blk - p.nkb);
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

  v4f acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) acc[m][jt] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int p0 = s_beg + 32 * w; p0 < s_end; p0 += 128) {
    int tok[8];
    bool ok[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int pos = p0 + 8 * g + q;
      ok[q] = pos < s_end;
      tok[q] = p.sorted_tok[ok[q] ? pos : s_beg];
    }
    uint4 mr[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      mr[q] = ldg16(M + (long)tok[q] * C + c0 + 8 * i);
      if (!ok[q]) mr[q] = zero4();
    }
    uint4 op[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = dw(mr[2 * d], m >> 1), hi = dw(mr[2 * d + 1], m >> 1);
        o[d] = (m & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u) : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
      op[m] = make_uint4(o[0], o[1], o[2], o[3]);
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt < njt) {
        const int j = 16 * jt + i;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = (ok[q] && j < r) ? V[(long)tok[q] * p.r_lim + j] : 0.f;
        uint4 vh, vl;
        split8(v, vh, vl);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          acc[m][jt] = mfma_bf16_16x16x32(op[m], vh, acc[m][jt]);
          acc[m][jt] = mfma_bf16_16x16x32(op[m], vl, acc[m][jt]);
        }
      }
    }
  }

  // combine the waves: slot row 16 m + rho holds C-row c0 + 8 rho + m (rho = 4 g + v)
  auto put = [&](float* s) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[(16 * m + 4 * g + v) * GR_RS + 16 * jt + i] = acc[m][jt][v];
  };
  auto add = [&](const float* s) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[m][jt][v] += s[(16 * m + 4 * g + v) * GR_RS + 16 * jt + i];
  };
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
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[m][jt] *= sa;
    put(red[1]);
  }
  __syncthreads();
  const float* fin = red[1];
  float* out = reinterpret_cast<float*>(isA ? p.dA_ptrs[a] : p.dB_ptrs[a]);
  if (isA) {  // dA_a [K][r]: rows c0 .. c0 + 127 are 128 r consecutive floats
    for (int o = tid; o < 128 * r; o += 256) {
      const int row = o / r, j = o - row * r;
      out[(long)(c0 + row) * r + j] = fin[(16 * (row & 7) + (row >> 3)) * GR_RS + j];
    }
  } else {    // dB_a [r][N]: for each rank, 128 consecutive columns
    for (int o = tid; o < 128 * r; o += 256) {
      const int j = o >> 7, col = o & 127;
      out[(long)j * p.N + c0 + col] = fin[(16 * (col & 7) + (col >> 3)) * GR_RS + j];
    }
  }
}

hipError_t launch_bwd_dx(const BwdDxParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dx, dim3(p.n_tb * p.n_kb), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_grad(const BwdGradParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_grad, dim3(p.n_ad * (p.nkb + p.nnb)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lora

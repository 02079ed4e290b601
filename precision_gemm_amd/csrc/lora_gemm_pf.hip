// The base GEMM of a long MXFP8 batch with its adapter epilogue:
//   y[t, n] = bf16( s_w[n] * sum_k x_q[t, k] W_q[k, n] + s_a (t[t, :r_a] . B_a[:r_a, n]) )
// ("EpiLoRA" abstract: the low-precision GEMM streams its weights while the adapter
// down-projection, launched first, produces t; the up-projection of each tenant is added in
// the GEMM's epilogue.  Punica README, Overview: y = x W + x A B per token's adapter.)
//
// One workgroup of eight waves (two per SIMD) per 128-token x 512-channel tile; wave w owns
// channels 64 w .. 64 w + 63 (four column tiles) for all 128 tokens (eight row tiles): 32
// accumulators of the scaled FP8 MFMA 16x16x128, formed transposed (y^T = W^T x^T, so that a
// lane's four results are four consecutive channels of one token).  Per 128-wide k-step:
//  - W: each wave loads its own four column tiles (packed, 2 KB of consecutive memory each)
//    straight into registers a step ahead, in two alternating register sets; no W byte goes
//    through LDS, and no two waves load the same one;
//  - x: the tile's codes (16 KB, in the MFMA's operand order as the pre-pass wrote them) and
//    scale codes (two 256-byte rows whose word at lane l holds the codes of four row tiles;
//    the operand select picks the byte) are copied from memory straight into LDS (16-byte
//    direct-to-LDS loads), three stages, two steps ahead; every wave reads all of them.
// So each step reads 128 KB of LDS per CU for 256 MFMAs, half the bytes per MFMA of a tile
// whose waves share both operands through LDS.
// Epilogue: the channel scale, then for each adapter present among the tile's rows
// (ascending id) one bf16 MFMA per 32 ranks, row tile and column tile with s_a t rounded to
// bf16 (rows of other adapters zeroed) and B_a^T rows as the other operand, then 8-byte bf16
// stores.  t is the sum, in part order, of the pre-pass's partial sums over four parts of K
// (the tiles of column block 0 also store it for the caller), or the caller's t.  Workgroups are dealt to the eight XCDs in turn; XCD x takes a contiguous run of
// tiles in an order grouped by row blocks, so the tiles an XCD runs together share x and W in
// its L2.
#include "device_common.hpp"
#include "lora_kernels.hpp"

namespace lora {

constexpr int PF_BM = 128, PF_BN = 512;
constexpr int PF_XBYTES = 8 * 2 * 1024;                   // x codes of one step: 8 row tiles x 2 halves
constexpr int PF_SBYTES = 2 * 256;                        // x scale codes: 2 row groups of 64
constexpr int PF_STAGE = PF_XBYTES + PF_SBYTES;           // one of four stages (separate LDS arrays)
constexpr int PF_TRS = 128;                               // epilogue: s_a t as bf16, 64 ranks a row

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// lane l copies `size` bytes from g into LDS at l_base + size * l (l_base wave-uniform)
__device__ __forceinline__ void dma16(const void* g, void* l_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)l_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* l_base) {
  __builtin_amdgcn_global_load_lds((gptr_t)g, (lptr_t)l_base, 4, 0, 0);
}

// Buffer resource over `bytes` bytes from `base` (raw, untyped: the third word 0x00020000
// is the gfx9 data format for untyped buffer access); loads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// lane l copies `size` bytes at voff (+ soff) into LDS at l_base + size * l
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, void* l_base, int size, int voff, int soff) {
  if (size == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)l_base, 16, voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)l_base, 4, voff, soff, 0, 0);
}

// A: 16 channels (e4m3 W codes, scale 2^0); B: 16 tokens (e4m3 x codes with their e8m0
// scales, byte OPB of sb_word)
template <int OPB>
__device__ __forceinline__ v4f mfma_pf(const v8i& w, const uint4& xlo, const uint4& xhi, v4f acc, int sb_word) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, join8(xlo, xhi), acc, 0, 0, 0, 127, OPB, sb_word);
}

// Workgroup barrier of the main loop.  __syncthreads() would also make every wave wait for all
// of its direct-to-LDS copies in flight (its release covers LDS writes, which those copies
// are), taking the look-ahead away; the waits this loop needs are explicit (the copies of the
// stage about to be read), and the wave-scope fences only keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void pf_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The four x stages are separate LDS arrays, each named directly by the unrolled steps:
// the compiler then knows that a step's LDS reads do not touch the stages whose copies are
// in flight, and does not wait for those copies before the reads.
template <int S>
__device__ __forceinline__ uint8_t* pf_stage(uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3) {
  return S == 0 ? s0 : (S == 1 ? s1 : (S == 2 ? s2 : s3));
}

__global__ __launch_bounds__(512) void k_gemm_pf(GemmParams p) {
  __shared__ __align__(16) uint8_t stg0[PF_STAGE], stg1[PF_STAGE], stg2[PF_STAGE], stg3[PF_STAGE];
  __shared__ __align__(16) uint8_t tstg[PF_BM * PF_TRS];
  __shared__ int rid[PF_BM];
  const int tid = threadIdx.x, lane = tid & 63, i = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, T = p.T, KS = K >> 7;
  const int n_tb = (T + PF_BM - 1) / PF_BM, n_cb = N / PF_BN, ntiles = n_tb * n_cb;
  int L = blockIdx.x;
  if ((ntiles & 7) == 0) L = (L & 7) * (ntiles >> 3) + (L >> 3);
  const int GM = (n_tb % 8 == 0) ? 8 : ((n_tb % 4 == 0) ? 4 : ((n_tb % 2 == 0) ? 2 : 1));
  const int grp = L / (GM * n_cb), rem = L % (GM * n_cb);
  const int tb = grp * GM + rem % GM, cb = rem / GM;
  const int t0 = tb * PF_BM, nw = cb * PF_BN + 64 * w;

  // x: wave w copies row tile w (both halves) and the scale row of group w & 1 (waves w and
  // w + 2, w + 4, w + 6 write the same bytes to the same place, so each wave issues the same
  // three copies and the wait counts stay exact)
  // Buffer loads: a wave-uniform base in a buffer resource (scalar registers), the step and
  // tile in a scalar offset, one 32-bit lane offset for every load (so few vector registers
  // hold addresses beside the accumulators); each resource covers exactly its bytes.
  const int tsz = KS * 2048;  // one 16-row (16-channel) tile's whole K, bytes
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.xq + (long)(8 * tb + w) * tsz, tsz);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.xsc + (long)(2 * tb + (w & 1)) * KS * 256, KS * 256);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.wq + (long)(nw >> 4) * tsz, 4 * tsz);
  const int lo16 = 16 * lane, lo4 = 4 * lane;
  auto issue_x = [&](uint8_t* st, int ks) {
    dma_buf(rx, st + (2 * w) * 1024, 16, lo16, ks * 2048);
    dma_buf(rx, st + (2 * w + 1) * 1024, 16, lo16 + 1024, ks * 2048);
    dma_buf(rs, st + PF_XBYTES + (w & 1) * 256, 4, lo4, ks * 256);
  };
  // W: the wave's column tiles nw / 16 + ct, each loaded into one 32-byte register tuple
  auto load_w = [&](v8i (&d)[4], int ks) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int so = ct * tsz + ks * 2048;
      d[ct] = join8(ld_buf(rw, lo16, so), ld_buf(rw, lo16 + 1024, so));
    }
  };

  v4f acc[8][4];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i wr[2][4];
  // (K is a multiple of 512: KS >= 4, even)
  issue_x(stg0, 0);
  issue_x(stg1, 1);
  load_w(wr[0], 0);
  // one 128-wide step ks: register set C holds W of step ks, set 1 - C receives step ks + 1;
  // stage S = ks % 4 holds x of step ks.  Stages go in pairs: an even step waits for the
  // copies of its pair, passes the step pair's one barrier and copies the next pair
  // (steps ks + 2, ks + 3) into the other two stages, read last in the previous pair
  auto step = [&](int ks, auto set, auto stage) {
    constexpr int C = decltype(set)::value, S = decltype(stage)::value;
    uint8_t* st = pf_stage<S>(stg0, stg1, stg2, stg3);
    if (S % 2 == 0) {
      // this wave's copies of stages ks and ks + 1 have landed: only the W loads of step ks,
      // issued after them, may still be in flight; and its LDS reads of the previous pair
      // are done, so that no copy issued after the barrier can overtake one
      __builtin_amdgcn_s_waitcnt(0x0070 | 8);  // vmcnt(8) lgkmcnt(0)
      pf_barrier();
    }
    // the last steps reload W of the last step and copy the last pair again (the same
    // bytes to the same place): uniform code, exact wait counts.  W first: the MFMAs of
    // step ks + 1 then wait for these loads only, not for the copies issued after them
    load_w(wr[1 - C], min(ks + 1, KS - 1));
    if (S % 2 == 0) {
      __builtin_amdgcn_sched_barrier(0);
      issue_x(pf_stage<(S + 2) % 4>(stg0, stg1, stg2, stg3), min(ks + 2, KS - 2));
      issue_x(pf_stage<(S + 3) % 4>(stg0, stg1, stg2, stg3), min(ks + 3, KS - 1));
    }
    __builtin_amdgcn_sched_barrier(0);  // the loads stay at the top: a whole step hides them
    const int sw0 = *reinterpret_cast<const int*>(st + PF_XBYTES + 4 * lane);
    const int sw1 = *reinterpret_cast<const int*>(st + PF_XBYTES + 256 + 4 * lane);
    const v8i (&wv)[4] = wr[C];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const uint4 xl = *reinterpret_cast<const uint4*>(st + (2 * rt) * 1024 + 16 * lane);
      const uint4 xh = *reinterpret_cast<const uint4*>(st + (2 * rt + 1) * 1024 + 16 * lane);
      const int sw = rt < 4 ? sw0 : sw1;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        switch (rt & 3) {
          case 0: acc[rt][ct] = mfma_pf<0>(wv[ct], xl, xh, acc[rt][ct], sw); break;
          case 1: acc[rt][ct] = mfma_pf<1>(wv[ct], xl, xh, acc[rt][ct], sw); break;
          case 2: acc[rt][ct] = mfma_pf<2>(wv[ct], xl, xh, acc[rt][ct], sw); break;
          default: acc[rt][ct] = mfma_pf<3>(wv[ct], xl, xh, acc[rt][ct], sw); break;
        }
      }
    }
    // LDS reads one row tile ahead of the MFMAs (all of them at once would need 64 more
    // registers than the two waves per SIMD have)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int q = 0; q < 7; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // no remainder (a conditional step after the loop made the register allocator spill the
  // accumulators at the join)
  for (int ks = 0; ks < KS; ks += 4) {
    step(ks, I0{}, I0{});
    step(ks + 1, I1{}, I1{});
    step(ks + 2, I0{}, I2{});
    step(ks + 3, I1{}, I3{});
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with the stages (reused below)

  // ---- FP8 channel scales of the lane's channels (nw + 16 ct + 4 g + v)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const float4 cs = *reinterpret_cast<const float4*>(p.ws_fp8 + nw + 16 * ct + 4 * g);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) acc[rt][ct] *= v4f{cs.x, cs.y, cs.z, cs.w};
  }

  // ---- adapter term: s_a t[row] B_a for the adapter of each row
  // (without the term every row's adapter is -1 and the loops below do nothing; a branch
  // around them made the register allocator spill the accumulators at the join)
  if (tid < PF_BM) {
    const int t = t0 + tid;
    int a = -1;
    if (t < T && p.lora) {
      a = p.ids[t];
      if (a < 0 || a >= p.n_ad) {
        a = -1;
      } else {
        const int r = p.ranks[a];
        if (r < 1 || r > p.r_lim) {
          or_agent(p.ctrl + CTRL_STATUS, 2);  // reported: the adapter's term is left out
          a = -1;
        }
      }
    }
    rid[tid] = a;
  }
  __syncthreads();
  // t = the pre-pass's K-part sums added in part order; s_a t as bf16, [row][64 ranks] (zero
  // past the row's rank and for rows without an adapter): thread = (row, quarter of the
  // ranks).  The tiles of column block 0 also store t for the caller.
  {
    const int row = tid >> 2, qq = tid & 3;
    const int a = rid[row];
    const int r = a >= 0 ? p.ranks[a] : 0;
    const float sa = a >= 0 ? p.scales[a] : 0.f;
    float tv[16];
    if (p.t_kparts == PF_KP) {  // the pre-pass's partial sums, rows of PF_TPS
      const long tpart = (long)T * PF_TPS;
      const float* trow = p.t + (long)(t0 + row) * PF_TPS + 16 * qq;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (4 * c + 16 * qq < r) {
          v = *reinterpret_cast<const float4*>(trow + 4 * c);
#pragma unroll
          for (int kp = 1; kp < PF_KP; ++kp) {
            const float4 u = *reinterpret_cast<const float4*>(trow + kp * tpart + 4 * c);
            v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
          }
        }
        tv[4 * c] = v.x; tv[4 * c + 1] = v.y; tv[4 * c + 2] = v.z; tv[4 * c + 3] = v.w;
      }
    } else {  // the caller's t [T][r_lim]
      const float* trow = p.t + (long)(t0 + row) * p.r_lim + 16 * qq;
#pragma unroll
      for (int jl = 0; jl < 16; ++jl) tv[jl] = (16 * qq + jl < r) ? trow[jl] : 0.f;
    }
    uint8_t* dst = tstg + row * PF_TRS;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int jl = 8 * q + 2 * d, j = 16 * qq + jl;
        o[d] = bf16x2_rne(j < r ? sa * tv[jl] : 0.f, j + 1 < r ? sa * tv[jl + 1] : 0.f);
      }
      *reinterpret_cast<uint4*>(dst + 2 * (16 * qq + 8 * q)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (p.t_out && cb == 0 && a >= 0) {
      float* trow_out = p.t_out + (long)(t0 + row) * p.r_lim;
#pragma unroll
      for (int jl = 0; jl < 16; ++jl) {
        const int j = 16 * qq + jl;
        if (j < p.r_lim) trow_out[j] = j < r ? tv[jl] : 0.f;
      }
    }
  }
  __syncthreads();
  const int my_a0 = rid[lane], my_a1 = rid[64 + lane];
  // B slots, 4 KB per wave, over the first two stages (contiguous: stg0 then stg1)
  uint8_t* bslot = (w < 4 ? stg0 + w * 4096 : stg1 + (w - 4) * 4096);
  int prev = -1;
  for (;;) {
    int m = min(my_a0 > prev ? my_a0 : 0x7fffffff, my_a1 > prev ? my_a1 : 0x7fffffff);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = min(m, __shfl_xor(m, o, 64));
    if (m == 0x7fffffff) break;
    const int a = __builtin_amdgcn_readfirstlane(m);
    prev = a;
    const int r = p.ranks[a], rp = rank_pad(r);
    const uint16_t* Bt = reinterpret_cast<const uint16_t*>(p.B_ptrs[a]);
    for (int rs = 0; 32 * rs < r; ++rs) {
      // B_a^T of the wave's 64 channels and 32 ranks, copied into the wave's slot in
      // operand order (lane (i, g) of block ct: channel 16 ct + i, ranks 32 rs + 8 g ..):
      // no registers held while the copy is in flight beside the 128 accumulators
      const int jj = 32 * rs + 8 * g;
      const uint16_t* bsrc = Bt + (long)(nw + i) * rp + min(jj, rp - 8);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) dma16(bsrc + (long)16 * ct * rp, bslot + ct * 1024);
      __builtin_amdgcn_s_waitcnt(0);
      uint4 bop[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        bop[ct] = keep_bf16(*reinterpret_cast<const uint4*>(bslot + ct * 1024 + 16 * lane), r - jj);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        const int row = 16 * rt + i;
        const bool mine = rid[row] == a;
        if (__ballot(mine) == 0ull) continue;
        const uint4 ah = mine ? *reinterpret_cast<const uint4*>(tstg + row * PF_TRS + 64 * rs + 16 * g)
                              : zero4();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = mfma_bf16_16x16x32(bop[ct], ah, acc[rt][ct]);
      }
    }
  }

  // ---- bf16 stores: token 16 rt + i, channels nw + 16 ct + 4 g .. + 3 (8 bytes) per lane
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const int t = t0 + 16 * rt + i;
    if (t >= T) continue;
    uint16_t* yrow = p.y + (long)t * N + nw + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      *reinterpret_cast<uint2*>(yrow + 16 * ct) =
          make_uint2(bf16x2_rne(acc[rt][ct][0], acc[rt][ct][1]), bf16x2_rne(acc[rt][ct][2], acc[rt][ct][3]));
  }
}

hipError_t launch_gemm_pf(const GemmParams& gp, hipStream_t s) {
  const int grid = ((gp.T + PF_BM - 1) / PF_BM) * (gp.N / PF_BN);
  hipLaunchKernelGGL(k_gemm_pf, dim3(grid), dim3(512), 0, s, gp);
  return hipGetLastError();
}

}  // namespace lora

// gfx950 kernels of the fused multi-tenant LoRA layer.
//
// The layer (per token t with adapter a = adapter_id[t]):
//     y[t] = bf16( dequant(xq[t] . W) + s_a * (x[t] @ A_a) @ B_a )
// "Punica: Serving multiple LoRA finetuned LLM as one" (README, Overview) gives the
// algebra Y = X@W + (x_1@A_1@B_1, ...); the "EpiLoRA" abstract gives the schedule:
// the adapter down-projection runs first, the low-precision GEMM streams its weights
// meanwhile, and the up-projection of every tenant is added in the GEMM's epilogue.
//
// Kernels (256-thread workgroups = 4 wave64):
//   k_build_segments  stable counting sort of tokens by adapter (one workgroup).
//   k_quant_mxfp8     MXFP8 quantisation of bf16 activations (one thread per 32-block).
//   k_shrink          down-projection t = x @ A_a per segment on bf16 MFMA (unfused schedule).
//   k_expand          up-projection y += s_a t @ B_a as its own launch (unfused schedule).
//   k_layer           one launch for the layer: workgroups [0, n_shrink) compute the
//                     down-projection, the others the scaled-MFMA base GEMM, whose
//                     epilogue waits for t only when it needs it.  With 16-bit
//                     activations (the "EpiLoRA" abstract's engine variant) the base GEMM
//                     reads x in bf16 and runs on bf16 MFMA with W widened in registers.
//
// Hand-over between workgroups of one launch uses agent-coherent loads/stores (see
// device_common.hpp) and a per-launch tag instead of counters that need resetting:
// every workgroup first reads the workspace's launch epoch E; values handed over are
// stored together with tag = E + 1 and a reader waits until it sees that tag.  The last
// workgroup to start (counted with one relaxed atomic) advances E when it ends, which is
// safe because every workgroup has read E before being counted.  A workgroup only ever
// waits for workgroups with lower ids, and the hardware dispatches workgroups in id
// order, so waits cannot deadlock; every wait is bounded and reports a status on expiry.
#include <mutex>

#include "device_common.hpp"
#include "lora_kernels.hpp"

#include <type_traits>

namespace lora {

// ======================================================================================
// Segment builder: seg_indptr (CSR over adapter ids) and sorted_tok (stable order)
// ======================================================================================
constexpr int SEG_THREADS = 1024;  // the builder's own launch (latency-bound loops: 4 waves per SIMD)
constexpr int SEG_SCRATCH = 32;    // LDS words before cnt: 16 wave sums, then misc
constexpr int SEG_CACHE = 4096;  // batches up to this size keep their ids in LDS between the passes

// One workgroup builds the whole result.  LDS (caller's): cnt (n_ad ints), and for batches
// of up to SEG_CACHE tokens the ids (T ints), the adapters present (up to T ints) and the
// per-(adapter, token chunk) counts (up to SEG_CACHE ints).  COH: the outputs are written
// with agent-coherent stores, for workgroups of the same launch that read them.
//
// Placement of a cached batch is data-parallel: the tokens are cut into C chunks, and one
// work item per (present adapter, chunk) counts the adapter's tokens in its chunk, then,
// after a prefix over the chunks, writes their positions in token order, which keeps the
// sort stable.  About 2 * T comparisons per present adapter.  Larger batches (ids read
// from memory) are placed by one wave in token order, 64 tokens at a time.
template <bool COH, int NT>
__device__ __forceinline__ void build_segments_wg(const int* __restrict__ ids, int T, int n_ad,
                                                  int* __restrict__ seg_indptr, int* __restrict__ sorted_tok,
                                                  int* __restrict__ err, int* cnt, int* ids_s, int* pres, int* wcnt,
                                                  int* wsum, int* misc) {
  auto put = [](int* q, int v) {
    if (COH)
      set_agent(q, v);
    else
      *q = v;
  };
  int* first_bad = misc;
  int* n_pres = misc + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    *first_bad = 0x7fffffff;
    *n_pres = 0;
  }
  for (int a = tid; a < n_ad; a += NT) cnt[a] = 0;
  __syncthreads();
  // 1. counts (LDS atomics: order-independent); ids read from memory once
  const bool cached = T <= SEG_CACHE;
  for (int t = tid; t < T; t += NT) {
    const int a = ids[t];
    if (cached) ids_s[t] = a;
    if (a >= 0 && a < n_ad) atomicAdd(&cnt[a], 1);
    else atomicMin(first_bad, t);
  }
  __syncthreads();
  // 2. exclusive scan: a contiguous slice per thread, a wave scan, then the wave totals;
  //    the adapters present are listed (in any order) for the placement
  const int per = (n_ad + NT - 1) / NT;
  const int lo = min(tid * per, n_ad), hi = min(lo + per, n_ad);
  int s = 0;
  for (int a = lo; a < hi; ++a) s += cnt[a];
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = incl - s;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  for (int a = lo; a < hi; ++a) {
    const int c = cnt[a];
    put(seg_indptr + a, base);
    cnt[a] = base;  // becomes the start of adapter a
    if (cached && c > 0) pres[atomicAdd(n_pres, 1)] = a;
    base += c;
  }
  if (tid == NT - 1) put(seg_indptr + n_ad, base);
  if (tid == 0) put(err, (*first_bad == 0x7fffffff) ? 0 : *first_bad + 1);
  __syncthreads();
  // 3. stable placement
  if (cached) {
    const int np = *n_pres;
    if (np == 0) return;
    // C chunks of L tokens (L a multiple of 4: the ids are read four at a time; reads past
    // T stay inside the LDS areas and are masked)
    const int C = min(min(T, 64), max(1, min((2 * NT + np - 1) / np, SEG_CACHE / np)));
    const int L = (((T + C - 1) / C) + 3) & ~3;
    const int items = np * C;
    // (a) count of adapter pres[i] in chunk c; item = c * np + i, so that neighbouring lanes
    //     read the same ids (a broadcast, not a bank conflict); counts stored per adapter
    for (int it = tid; it < items; it += NT) {
      const int i = it % np, c = it / np, a = pres[i];
      const int t0 = c * L, t1 = min(T, t0 + L);
      int n = 0;
      for (int t = t0; t < t1; t += 4) {
        const int4 v = *reinterpret_cast<const int4*>(ids_s + t);
        n += (v.x == a) + (v.y == a && t + 1 < t1) + (v.z == a && t + 2 < t1) + (v.w == a && t + 3 < t1);
      }
      wcnt[i * C + c] = n;
    }
    __syncthreads();
    // (b) per adapter: exclusive prefix over its C <= 64 chunks, from its start; a thread
    //     per adapter for few chunks, a wave per adapter for many
    if (C <= 16) {
      for (int i = tid; i < np; i += NT) {
        int run = cnt[pres[i]];
        for (int c = 0; c < C; ++c) {
          const int n = wcnt[i * C + c];
          wcnt[i * C + c] = run;
          run += n;
        }
      }
    } else {
      for (int i = wave; i < np; i += NT / 64) {
        const int v = (lane < C) ? wcnt[i * C + lane] : 0;
        int inc = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int u = __shfl_up(inc, off);
          if (lane >= off) inc += u;
        }
        if (lane < C) wcnt[i * C + lane] = cnt[pres[i]] + inc - v;
      }
    }
    __syncthreads();
    // (c) positions, in token order within the chunk
    for (int it = tid; it < items; it += NT) {
      const int i = it % np, c = it / np, a = pres[i];
      const int t0 = c * L, t1 = min(T, t0 + L);
      int pos = wcnt[i * C + c];
      for (int t = t0; t < t1; t += 4) {
        const int4 v = *reinterpret_cast<const int4*>(ids_s + t);
        if (v.x == a) put(sorted_tok + pos++, t);
        if (v.y == a && t + 1 < t1) put(sorted_tok + pos++, t + 1);
        if (v.z == a && t + 2 < t1) put(sorted_tok + pos++, t + 2);
        if (v.w == a && t + 3 < t1) put(sorted_tok + pos++, t + 3);
      }
    }
    return;
  }
  // one wave, 64 tokens at a time in token order.  Lanes with the same adapter are grouped
  // with a ballot; a lane's slot is the cursor plus the number of lower lanes in its group,
  // so equal ids keep their token order.
  if (wave == 0) {
    volatile int* cur = cnt;
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
        if (ok && a == la) put(sorted_tok + c0 + __popcll(same & below), t);
        if (lane == leader) cur[la] = c0 + __popcll(same);
        pending &= ~same;
      }
    }
  }
}

// LDS bytes of the builder: SEG_SCRATCH words of scratch, cnt, and for cached batches the ids, the
// adapters present and the chunk counts
__host__ __device__ constexpr int seg_cnt_words(int n_ad) { return (n_ad + 3) & ~3; }  // keeps the id cache 16-byte aligned
__host__ __device__ constexpr size_t seg_lds_bytes(int T, int n_ad) {
  return 4 * (size_t)SEG_SCRATCH + 4 * (size_t)seg_cnt_words(n_ad) +
         (T <= SEG_CACHE ? 4 * (size_t)((T + 3) & ~3) + 4 * (size_t)(T < n_ad ? T : n_ad) + 4 * (size_t)SEG_CACHE + 16
                         : 0);
}

__global__ __launch_bounds__(SEG_THREADS) void k_build_segments(const int* __restrict__ ids, int T, int n_ad,
                                                                int* __restrict__ seg_indptr,
                                                                int* __restrict__ sorted_tok, int* __restrict__ err) {
  extern __shared__ __align__(16) char smem[];
  int* w = reinterpret_cast<int*>(smem);
  int* cnt = w + SEG_SCRATCH;
  int* ids_s = cnt + seg_cnt_words(n_ad);
  int* pres = ids_s + (T <= SEG_CACHE ? (T + 3) & ~3 : 0);
  int* wcnt = pres + (T <= SEG_CACHE ? min(T, n_ad) : 0);
  build_segments_wg<false, SEG_THREADS>(ids, T, n_ad, seg_indptr, sorted_tok, err, cnt, ids_s, pres, wcnt, w, w + 16);
}

// ======================================================================================
// MXFP8 activation quantisation (standalone; the GEMM loader uses the same functions)
// ======================================================================================
// One thread per 16-byte piece (8 elements): each wave reads 1 KB of x per load, and
// the four lanes holding a 32-block combine their maxima with two lane swaps.
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {  // value of lane ^ 1 (DPP quad_perm 1,0,3,2)
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {  // value of lane ^ 2 (DPP quad_perm 2,3,0,1)
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
// PK: codes and scales in the long-batch GEMM's operand order (pf_xq_off, pf_xsc_off)
template <bool PK = false>
__device__ __forceinline__ void quant_mxfp8_part(const uint16_t* __restrict__ x, int T, int K, uint8_t* __restrict__ xq,
                                                 uint8_t* __restrict__ xsc, int block, int n_blocks) {
  const long total = (long)T * (K / 8);  // a multiple of 4: whole blocks, so quads stay together
  for (long P = (long)block * blockDim.x + threadIdx.x; P < total; P += (long)n_blocks * blockDim.x) {
    const uint4 in = ldg16(x + P * 8);
    uint32_t mx = absmax8_bits(in);
    mx = max(mx, quad_swap1(mx));
    mx = max(mx, quad_swap2(mx));
    const uint32_t code = mx_code_from_bits(mx);
    if (PK) {
      const int row = (int)(P / (K >> 3)), kk = (int)(P % (K >> 3)) * 8;
      *reinterpret_cast<uint2*>(xq + pf_xq_off(row, kk, K >> 7)) = mx_piece_quant(in, code);
      if ((P & 3) == 0) xsc[pf_xsc_off(row, kk >> 5, K >> 7)] = (uint8_t)code;
    } else {
      *reinterpret_cast<uint2*>(xq + P * 8) = mx_piece_quant(in, code);
      if ((P & 3) == 0) xsc[P >> 2] = (uint8_t)code;
    }
  }
}
template <bool PK>
__global__ __launch_bounds__(256) void k_quant_mxfp8(const uint16_t* __restrict__ x, int T, int K,
                                                     uint8_t* __restrict__ xq, uint8_t* __restrict__ xsc) {
  quant_mxfp8_part<PK>(x, T, K, xq, xsc, blockIdx.x, gridDim.x);
}
// The segment builder (workgroup 0) beside the MXFP8 pre-pass (the others) in one launch:
// the two do not depend on each other, so the builder's latency hides behind the pre-pass.
// Workgroups of SEG_THREADS threads (the builder's loops are latency-bound).
__global__ __launch_bounds__(SEG_THREADS) void k_quant_build(const uint16_t* __restrict__ x, int T, int K,
                                                     uint8_t* __restrict__ xq, uint8_t* __restrict__ xsc,
                                                     const int* __restrict__ ids, int n_ad, int* __restrict__ seg_indptr,
                                                     int* __restrict__ sorted_tok, int* __restrict__ err) {
  extern __shared__ __align__(16) char smem[];
  if (blockIdx.x == 0) {
    int* w = reinterpret_cast<int*>(smem);
    int* cnt = w + SEG_SCRATCH;
    int* ids_s = cnt + seg_cnt_words(n_ad);
    int* pres = ids_s + (T <= SEG_CACHE ? (T + 3) & ~3 : 0);
    int* wcnt = pres + (T <= SEG_CACHE ? min(T, n_ad) : 0);
    build_segments_wg<false, SEG_THREADS>(ids, T, n_ad, seg_indptr, sorted_tok, err, cnt, ids_s, pres, wcnt, w, w + 16);
  } else {
    quant_mxfp8_part<false>(x, T, K, xq, xsc, blockIdx.x - 1, gridDim.x - 1);
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ======================================================================================
// Packed weight layout.  For each tile of 16 output channels (row tile nt) and each
// 128-wide k-step ks, the bytes one wave loads for the scaled MFMA's W operand are stored
// contiguously in lane order (lane l = 16g + j: channel 16nt + j, lane group g), so every
// 16-byte load instruction of the GEMM reads 1 KB of consecutive memory:
//   FP8:   [N/16][K/128][half h][lane l][16 B], lane l holds k = 128ks + 64h + 16g .. +15
//   MXFP4: [N/16][K/128][lane l][16 B],          lane l holds k = 128ks + 32g .. +31
//          scales [N/16][K/128][lane l] (1 byte), the e8m0 code of k-block 4ks + g
// One thread per 16-byte chunk of the packed codes.
// ======================================================================================
__global__ __launch_bounds__(256) void k_pack_weight(int fmt, const uint8_t* __restrict__ q,
                                                     const uint8_t* __restrict__ sc, int N, int K,
                                                     uint8_t* __restrict__ qp, uint8_t* __restrict__ scp) {
  const int ksteps = K / 128;
  const long chunks = (fmt == LORA_W_FP8_E4M3) ? (long)N * K / 16 : (long)N * K / 32;
  for (long c = (long)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += (long)gridDim.x * blockDim.x) {
    const int l = (int)(c & 63), j = l & 15, g = l >> 4;
    if (fmt == LORA_W_FP8_E4M3) {
      const int h = (int)((c >> 6) & 1);
      const long rest = c >> 7;
      const long ks = rest % ksteps, nt = rest / ksteps;
      const long n = nt * 16 + j, k = ks * 128 + h * 64 + g * 16;
      *reinterpret_cast<uint4*>(qp + c * 16) = ldg16(q + n * K + k);
    } else {
      const long rest = c >> 6;
      const long ks = rest % ksteps, nt = rest / ksteps;
      const long n = nt * 16 + j;
      *reinterpret_cast<uint4*>(qp + c * 16) = ldg16(q + n * (K / 2) + ks * 64 + g * 16);
      scp[c] = sc[n * (K / 32) + ks * 4 + g];
    }
  }
}

// ======================================================================================
// Adapter layout.  The pages state an adapter as A [K, r] and B [r, N] ("Punica" README,
// Overview: A [H1, r], B [r, H2]), both row-major here.  The kernels read them as the
// weights of the maps K -> r and r -> N in out-by-in order, along their reduction
// dimension: A^T in bf16 MFMA operand order (a_index: each 16-byte lane load of a rank
// tile reads 1 KB of consecutive memory with the others of its wave) and B^T
// [N][rank_pad(r)], the padding rows / columns zero.  One thread per output element (an
// offline step, like the packing of W).
// ======================================================================================
__global__ __launch_bounds__(256) void k_pack_adapter(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                      int K, int N, int r, uint16_t* __restrict__ At,
                                                      uint16_t* __restrict__ Bt) {
  const int r8 = rank_pad(r);
  const long na = (long)a_tiles(r) * 16 * K, total = na + (long)N * r8;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    if (i < na) {
      // i = a_index(j, k): e = k % 8, lane = 16 g + j % 16, h, ks, jt
      const int e = (int)(i & 7), lane = (int)((i >> 3) & 63), h = (int)((i >> 9) & 1);
      const long q = i >> 10;
      const int ks = (int)(q % (K >> 6)), jt = (int)(q / (K >> 6));
      const int j = jt * 16 + (lane & 15), k = ks * 64 + 16 * (lane >> 4) + 8 * h + e;
      At[i] = (j < r) ? A[(long)k * r + j] : (uint16_t)0;
    } else {
      const long q = i - na;
      const int n = (int)(q / r8), j = (int)(q % r8);
      Bt[q] = (j < r) ? B[(long)j * N + n] : (uint16_t)0;
    }
  }
}

// ======================================================================================
// Launch epoch (see the file comment)
// ======================================================================================
// thread 0 issues the epoch load before any bulk load of the workgroup
__device__ __forceinline__ int wg_epoch_load(const int* ctrl) {
  return (threadIdx.x == 0) ? ld_agent(ctrl + CTRL_EPOCH) : 0;
}

// thread 0: publish the epoch to LDS and count this workgroup as started.  The increment's
// operand goes through an empty asm statement that takes the epoch as an input, so the
// compiler waits for the epoch load before the increment is issued (a value-neutral
// dependence: the increment is always 1).
__device__ __forceinline__ int wg_epoch_publish(int* ctrl, int e, int* lds_epoch) {
  int started = 0;
  if (threadIdx.x == 0) {
    *lds_epoch = e;
    int one = 1;
    asm volatile("" : "+v"(one) : "v"(e));
    started = add_agent(ctrl + CTRL_STARTED, one);
  }
  return started;
}

// The epoch stays in [0, 2^30): tags (epoch + 1) never overflow a signed int, and a
// workspace can serve any number of launches (a tag comes back after 2^30 launches).
constexpr int EPOCH_MASK = 0x3fffffff;
__device__ __forceinline__ void wg_epoch_end(int* ctrl, int e, int started) {
  if (threadIdx.x == 0 && started == (int)gridDim.x - 1) {
    set_agent(ctrl + CTRL_STARTED, 0);
    set_agent(ctrl + CTRL_EPOCH, (e + 1) & EPOCH_MASK);
  }
}

__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}

// Bounded wait until a tagged word carries `tag`; on expiry the status word is set and the
// stale value is used, so the kernel always finishes.
__device__ __forceinline__ uint64_t wait_tag(const uint64_t* p, uint64_t v, uint32_t tag, int* ctrl, int spin_limit) {
  int spins = 0;
  while ((uint32_t)(v >> 32) != tag) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > spin_limit) {
      or_agent(ctrl + CTRL_STATUS, 1);
      break;
    }
    v = ld_agent_u64(p);
  }
  return v;
}

// ======================================================================================
// Down-projection ("shrink").  Work item = (adapter a, token block of its segment,
// group of 16*JP ranks, K-part).  A_a is stored transposed, bf16 [r_a][K], so both MFMA
// operands are rows with K contiguous: the x operand is 16 tokens of segment a (gathered
// through sorted_tok), the A operand is 16 ranks.  Lane (i = l%16, g = l/16) loads 32
// contiguous bytes (k = k0+16g .. k0+16g+15) of its row and feeds them to two 16x16x32
// MFMAs; both operands use the same k assignment, so the products pair up.  The four
// waves take interleaved 64-wide k-steps, with the loads of the next U steps in flight
// while the current ones are multiplied; the wave sums meet in LDS in wave order.
// Output: t (or its K-part) for each token of the block, in original token order.
// ======================================================================================
// In the fused launch (ctrl != null) the workgroup publishes the launch epoch once its
// first loads are in flight (or when it finds no work); the tag is read after a barrier.
// PACK: the launch may ask for t as tagged bf16 pairs (not in the one-tile stream's launch)
template <int TG, int JP, int U, bool PACK = false>
__device__ __forceinline__ void shrink_item(const ShrinkParams& p, int item, char* smem, int* ctrl, int e, int* lds_epoch,
                                            int* started, bool& published) {
  auto publish = [&]() {
    if (ctrl && !published) *started = wg_epoch_publish(ctrl, e, lds_epoch);
    published = true;
  };
  const int kp = item % p.kparts;
  int rest = item / p.kparts;
  const int jg = rest % p.n_jg;
  rest /= p.n_jg;
  const int tb = rest % p.n_tblk;
  const int a = rest / p.n_tblk;
  // With at most 16 tokens (and ids at hand) the workgroup takes all token rows and keeps
  // the rows of adapter a: no dependent loads of seg_indptr and sorted_tok before x.
  const bool direct = (p.ids != nullptr) && (p.T <= 16);
  // Segments built by workgroup 0 of this launch: wait for its tag, then read them with
  // agent-coherent loads (another XCD's L2 may hold an older copy).
  const bool coh = !direct && p.seg_wait;
  if (coh) {
    publish();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int tag = *lds_epoch + 1;
      int spins = 0;
      while (ld_agent(ctrl + CTRL_SEGREADY) != tag) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > p.spin_limit) {
          or_agent(ctrl + CTRL_STATUS, 1);
          break;
        }
      }
    }
    __syncthreads();
  }
  auto seg_at = [&](int i) { return coh ? ld_agent(p.seg_indptr + i) : p.seg_indptr[i]; };
  auto tok_at = [&](int i) { return coh ? ld_agent(p.sorted_tok + i) : p.sorted_tok[i]; };
  const int s0 = direct ? 0 : seg_at(a);
  const int L = direct ? p.T : seg_at(a + 1) - s0;
  const int tok_begin = tb * p.tblk;
  const int r = p.ranks[a];
  const int j_begin = jg * JP * 16;
  // no work: empty token block, a rank outside [1, r_max] (the GEMM epilogue reports it
  // and skips the adapter term), or ranks beyond r_a
  if (tok_begin >= L || r < 1 || r > p.r_lim || j_begin >= r) {
    publish();
    return;
  }
  const int tok_end = min(L, tok_begin + p.tblk);
  const int njt = min(JP, (r - j_begin + 15) >> 4);
  const uint16_t* __restrict__ A = reinterpret_cast<const uint16_t*>(p.A_ptrs[a]);
  // wave index as a scalar: conditions derived from it must compile to branches, since an
  // MFMA executes for every lane whatever the EXEC mask
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15,
            g = lane >> 4;
  const int k_begin = kp * p.kpart_len, k_end = min(p.K, k_begin + p.kpart_len);
  const int nsteps = (k_end - k_begin) >> 6;
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][TG][JP][64 lanes][4]

  // A_a in operand order: the lane's 16 bytes of rank tile jt for k-step ks at
  // a_tile_off(jt, ks, h) + 8 lane (rows past r_a are zero padding of the last tile; tiles
  // past the item's last read that tile and feed no output)
  const uint16_t* arow[JP];
  const int nat = a_tiles(r);
#pragma unroll
  for (int jt = 0; jt < JP; ++jt) arow[jt] = A + a_tile_off(min((j_begin >> 4) + jt, nat - 1), 0, 0, p.K) + 8 * lane;
  const int ks0 = k_begin >> 6;  // the item's first k-step

  for (int t0 = tok_begin; t0 < tok_end; t0 += TG * 16) {
    const int ntt = min(TG, (tok_end - t0 + 15) >> 4);
    const uint16_t* xrow[TG];
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      const int pos = min(t0 + tt * 16 + li, tok_end - 1);
      xrow[tt] = p.x + (long)(direct ? pos : tok_at(s0 + pos)) * p.K + k_begin + 16 * g;
    }
    v4f acc[TG][JP];
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int jt = 0; jt < JP; ++jt) acc[tt][jt] = v4f{0.f, 0.f, 0.f, 0.f};

    // Loads are unconditional with clamped (always valid) addresses: a predicated load
    // would compile to a branch that waits for it, serialising the stream.  Rows past the
    // segment or the rank read a valid row and only feed outputs that are discarded;
    // k-steps past the range are skipped at the MFMA (uniform branch).
    uint4 xa[2][U][TG][2], aa[2][U][JP][2];
    auto load = [&](int buf, int sbase) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k0 = min(sbase + 4 * u, nsteps - 1) * 64;
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          xa[buf][u][tt][0] = ldg16(xrow[tt] + k0);
          xa[buf][u][tt][1] = ldg16(xrow[tt] + k0 + 8);
        }
#pragma unroll
        for (int jt = 0; jt < JP; ++jt) {
          aa[buf][u][jt][0] = ldg16(arow[jt] + a_tile_off(0, ks0 + (k0 >> 6), 0, p.K));
          aa[buf][u][jt][1] = ldg16(arow[jt] + a_tile_off(0, ks0 + (k0 >> 6), 1, p.K));
        }
      }
    };
    auto mma = [&](int buf, int sbase) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (sbase + 4 * u >= nsteps) break;
#pragma unroll
        for (int tt = 0; tt < TG; ++tt)
#pragma unroll
          for (int jt = 0; jt < JP; ++jt) {
            if (tt >= ntt || jt >= njt) continue;
            acc[tt][jt] = mfma_bf16_16x16x32(xa[buf][u][tt][0], aa[buf][u][jt][0], acc[tt][jt]);
            acc[tt][jt] = mfma_bf16_16x16x32(xa[buf][u][tt][1], aa[buf][u][jt][1], acc[tt][jt]);
          }
      }
    };
    load(0, wave);
    for (int s = wave; s < nsteps; s += 8 * U) {
      load(1, s + 4 * U);
      mma(0, s);
      load(0, s + 8 * U);
      mma(1, s + 4 * U);
    }
    publish();  // the epoch is needed only for the stores below
    // cross-wave sum in fixed wave order
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int jt = 0; jt < JP; ++jt)
        *reinterpret_cast<v4f*>(red + (((wave * TG + tt) * JP + jt) * 64 + lane) * 4) = acc[tt][jt];
    __syncthreads();
    const uint32_t tag = ctrl ? (uint32_t)(*lds_epoch) + 1u : 0u;
    const bool pack = PACK && p.t_pack;
    const float s_a = pack ? p.scales[a] : 0.f;
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int jt = 0; jt < JP; ++jt) {
        if (tt >= ntt || jt >= njt || ((tt * JP + jt) & 3) != wave) continue;
        v4f sum = *reinterpret_cast<const v4f*>(red + (((0 * TG + tt) * JP + jt) * 64 + lane) * 4);
#pragma unroll
        for (int w = 1; w < 4; ++w)
          sum += *reinterpret_cast<const v4f*>(red + (((w * TG + tt) * JP + jt) * 64 + lane) * 4);
        const int j = j_begin + jt * 16 + li;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int pos = t0 + tt * 16 + 4 * g + v;
          float other = pack ? __shfl_xor(sum[v], 1) : 0.f;  // rank j ^ 1, same token (uniform)
          if (j + 1 >= r) other = 0.f;                             // past the rank: a padding row of A
          if (pos < tok_end && j < r && (!direct || p.ids[pos] == a)) {
            const long tok = direct ? pos : tok_at(s0 + pos);
            if (p.t_tag && pack) {
              // one K-part: s_a t of ranks j, j + 1 as two bf16 under one tag (the GEMM
              // epilogue's operands as they are)
              if ((li & 1) == 0)
                st_agent_u64(p.t_tag + tok * (p.r_max >> 1) + (j >> 1),
                             ((uint64_t)tag << 32) | bf16x2_rne(sum[v] * s_a, other * s_a));
            } else if (p.t_tag) {
              st_agent_u64(p.t_tag + ((long)kp * p.T + tok) * p.r_max + j, tagged(sum[v], tag));
            }
            if (p.t_out && p.kparts == 1) p.t_out[tok * p.r_lim + j] = sum[v];
            if (p.t_part) p.t_part[((long)kp * p.T + tok) * p.r_lim + j] = sum[v];
          }
        }
      }
    __syncthreads();
  }
  // columns j in [r, r_max) of the caller's t are zero
  if (p.t_out && jg == 0 && kp == 0 && r < p.r_lim) {
    const int w = p.r_lim - r;
    for (int idx = tid; idx < (tok_end - tok_begin) * w; idx += 256) {
      const int pos = tok_begin + idx / w;
      if (direct && p.ids[pos] != a) continue;
      const long tok = direct ? pos : tok_at(s0 + pos);
      p.t_out[tok * p.r_lim + r + idx % w] = 0.f;
    }
  }
}

template <int TG, int JP, int U>
__global__ __launch_bounds__(256) void k_shrink(ShrinkParams p) {
  extern __shared__ __align__(16) char smem[];
  int started = 0;
  bool published = false;
  // item order 1: workgroups are dealt to the eight XCDs in turn, and XCD x takes the x-th
  // eighth of the items, so that items sharing an adapter's A_a and a segment's x rows run on
  // one XCD's L2
  const int b = blockIdx.x, nb = gridDim.x;
  const int item = (p.item_order == 1 && nb % 8 == 0) ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  shrink_item<TG, JP, U>(p, item, smem, nullptr, 0, nullptr, &started, published);
}

// ======================================================================================
// Down-projection by wave reductions (BGMV) for segments of a few tokens, the standalone
// launch's alternative to the MFMA tiles above (16-token tiles, mostly padding when a segment
// holds one token).  Item (adapter a, NT consecutive positions of its segment, 16 JP ranks).
// The packed A gives lane (i, g) rank i of a 16-rank tile at k = 64 ks + 16 g .. + 15 of each
// 64-wide k-step: the lane multiplies those 16 values with the same 16 k of each token's x
// row in fp32 and keeps one partial sum per (token, rank).  The four waves take interleaved
// k-steps, U of them per buffer, two buffers in flight; at the end the four lane groups g
// are summed by two butterfly shuffles and the four waves in LDS in wave order, so t is
// deterministic.  Output as the MFMA kernel's: fp32 t in original token order, zero for
// r_a <= j < r_max.
// ======================================================================================
template <int NT, int JP, int U>
__global__ __launch_bounds__(256) void k_shrink_bgmv(ShrinkParams p) {
  __shared__ float red[4][NT][JP * 16];
  const int b = blockIdx.x, nb = gridDim.x;
  const int item = (p.item_order == 1 && nb % 8 == 0) ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  const int jg = item % p.n_jg;
  const int rest = item / p.n_jg;
  const int tb = rest % p.n_tblk;
  const int a = rest / p.n_tblk;
  const int s0 = p.seg_indptr[a];
  const int L = p.seg_indptr[a + 1] - s0;
  const int tok_begin = tb * NT;
  const int r = p.ranks[a];
  const int j_begin = jg * JP * 16;
  if (tok_begin >= L || r < 1 || r > p.r_lim) return;
  const int tok_end = min(L, tok_begin + NT);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15,
            g = lane >> 4;
  if (j_begin < r) {
    const int nsteps = p.K >> 6;
    const uint16_t* __restrict__ A = reinterpret_cast<const uint16_t*>(p.A_ptrs[a]);
    const uint16_t* arow[JP];
    const int nat = a_tiles(r);
#pragma unroll
    for (int jt = 0; jt < JP; ++jt) arow[jt] = A + a_tile_off(min((j_begin >> 4) + jt, nat - 1), 0, 0, p.K) + 8 * lane;
    const uint16_t* xrow[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) xrow[q] = p.x + (long)p.sorted_tok[s0 + min(tok_begin + q, tok_end - 1)] * p.K + 16 * g;
    float acc[NT][JP];
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int jt = 0; jt < JP; ++jt) acc[q][jt] = 0.f;
    // unconditional loads from clamped addresses (see shrink_item)
    uint4 xa[2][U][NT][2], aa[2][U][JP][2];
    auto load = [&](int buf, int sbase) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = min(sbase + 4 * u, nsteps - 1);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
          xa[buf][u][q][0] = ldg16(xrow[q] + ks * 64);
          xa[buf][u][q][1] = ldg16(xrow[q] + ks * 64 + 8);
        }
#pragma unroll
        for (int jt = 0; jt < JP; ++jt) {
          aa[buf][u][jt][0] = ldg16(arow[jt] + a_tile_off(0, ks, 0, p.K));
          aa[buf][u][jt][1] = ldg16(arow[jt] + a_tile_off(0, ks, 1, p.K));
        }
      }
    };
    auto fma_step = [&](int buf, int sbase) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (sbase + 4 * u >= nsteps) break;
#pragma unroll
        for (int jt = 0; jt < JP; ++jt) {
          float av[16];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t w[4] = {aa[buf][u][jt][h].x, aa[buf][u][jt][h].y, aa[buf][u][jt][h].z, aa[buf][u][jt][h].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              av[8 * h + 2 * d] = bf16_lo(w[d]);
              av[8 * h + 2 * d + 1] = bf16_hi(w[d]);
            }
          }
#pragma unroll
          for (int q = 0; q < NT; ++q) {
            float s = acc[q][jt];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const uint32_t w[4] = {xa[buf][u][q][h].x, xa[buf][u][q][h].y, xa[buf][u][q][h].z, xa[buf][u][q][h].w};
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                s = __builtin_fmaf(bf16_lo(w[d]), av[8 * h + 2 * d], s);
                s = __builtin_fmaf(bf16_hi(w[d]), av[8 * h + 2 * d + 1], s);
              }
            }
            acc[q][jt] = s;
          }
        }
      }
    };
    load(0, wave);
    for (int st = wave; st < nsteps; st += 8 * U) {
      load(1, st + 4 * U);
      fma_step(0, st);
      load(0, st + 8 * U);
      fma_step(1, st + 4 * U);
    }
    // the four lane groups: rank li of each group sums over its 16 k
#pragma unroll
    for (int q = 0; q < NT; ++q)
#pragma unroll
      for (int jt = 0; jt < JP; ++jt) {
        float v = acc[q][jt];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g == 0) red[wave][q][jt * 16 + li] = v;
      }
    __syncthreads();
    for (int idx = tid; idx < NT * JP * 16; idx += 256) {
      const int q = idx / (JP * 16), jj = idx % (JP * 16);
      const int j = j_begin + jj;
      const int pos = tok_begin + q;
      if (pos < tok_end && j < r && j < p.r_lim) {
        const float sum = ((red[0][q][jj] + red[1][q][jj]) + red[2][q][jj]) + red[3][q][jj];
        p.t_out[(long)p.sorted_tok[s0 + pos] * p.r_lim + j] = sum;
      }
    }
  }
  // columns j in [r, r_max) of the caller's t are zero
  if (jg == 0 && r < p.r_lim) {
    const int w = p.r_lim - r;
    for (int idx = tid; idx < (tok_end - tok_begin) * w; idx += 256) {
      const int pos = tok_begin + idx / w;
      p.t_out[(long)p.sorted_tok[s0 + pos] * p.r_lim + r + idx % w] = 0.f;
    }
  }
}

// ======================================================================================
// Standalone up-projection: y[tok][n] = bf16( y[tok][n] + s_a * sum_j t[tok][j] B_a[j][n] ),
// B_a stored transposed, bf16 [N][rank_pad(r_a)].  One workgroup per (token, 256 columns).
// ======================================================================================
__global__ __launch_bounds__(256) void k_expand(ExpandParams p) {
  __shared__ float trow[64];
  const int tok = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int a = p.ids[tok];
  if (a < 0 || a >= p.n_ad) return;
  const int r = p.ranks[a];
  if (r < 1 || r > p.r_lim) return;  // a rank outside [1, r_max]: adapter skipped
  if (threadIdx.x < 64) trow[threadIdx.x] = (threadIdx.x < r) ? p.t[(long)tok * p.r_lim + threadIdx.x] : 0.f;
  __syncthreads();
  if (n >= p.N) return;
  const int r8 = rank_pad(r);
  const uint16_t* __restrict__ Bt = reinterpret_cast<const uint16_t*>(p.B_ptrs[a]) + (long)n * r8;
  float acc = 0.f;
  for (int j = 0; j < r; j += 8) {
    const uint4 b = keep_bf16(ldg16(Bt + j), r - j);  // the padding past r_a is masked
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
// Workgroup tile: TT*16 tokens x WN = WC*CT*16 output channels over a K-range.  The four
// waves form a WC x WK grid: wave (wc, wk) owns columns [wc*CT*16, (wc+1)*CT*16) of the
// tile and the k-steps s with s % WK == wk.  Per K-chunk of KC:
//   * the x loads of the chunk are issued before its W loads (loads retire in order, so
//     x can be quantised while W is still in flight), and the loads of chunk c+1 are
//     issued before the MFMAs of chunk c;
//   * W fragments go straight from HBM into registers (each W byte is read by exactly one
//     lane of one workgroup per K-split);
//   * the workgroup converts the chunk of x to MXFP8 (or copies pre-quantised codes) into
//     LDS, rows padded by 16 bytes so the 16 lanes of a lane group hit distinct banks;
//   * per 128-wide k-step a wave reads its TT x-fragments from LDS once and issues TT*CT
//     scaled MFMAs (x scale from the MX block; W scale 1.0 for FP8, the block scale for
//     MXFP4).
// The WK wave sums meet in LDS in wave order.  With a K-split over workgroups, each split
// adds the adapter terms of its share of the tile's adapters to its own sum; the splits
// other than the last store their sums and a tagged flag, and the last split of the tile
// (highest id) waits for the flags, adds the sums in split order and stores y.
// Epilogue: FP8 channel scale; then, if the layer has adapters, the distinct adapters of
// the token block are listed, t is gathered (waiting for its tag in the fused launch) and
// stored pre-scaled as bf16 in LDS, and for each token tile and each adapter present in it
// one bf16 MFMA per 32 ranks adds (s_a t[tok]) @ B_a to the rows of that adapter's tokens,
// the B_a^T operands read from slices staged in LDS (64-row tiles) or straight from memory
// (128-row tiles); finally bf16 stores (RNE), through LDS for the chunked tiles.
// ======================================================================================
template <int TT, int CT>
struct ChunkK {
  // K-chunk: two chunks of x and W are held in registers, so the chunk shrinks as the
  // workgroup tile grows (the host plan uses the same rule)
  static constexpr int KC = (TT == 1) ? 2048 : ((TT <= 4 && CT == 1) ? 512 : (CT == 4 ? 128 : 256));
  static constexpr int STEPS = KC / 128;
  static constexpr int ROW = KC + 16;  // LDS row stride in bytes
};

// B_a^T slices of the up-projection are staged in LDS, in slots of WN x r_max bf16, up to
// a budget of bytes at a time (one batch: normally all the adapters of the tile).  Kernels
// that run two workgroups per CU stage less (each workgroup has half the LDS).
template <int OCC>
constexpr int epi_bstage() { return OCC == 2 ? 32 * 1024 : 96 * 1024; }
constexpr int TSTR = MAX_RANK + 8;  // bf16 row stride of the staged t (the pad spreads the rows over LDS banks)

template <int TT, int CT, int WC, int WK>
struct EpiLayout {
  static constexpr int ROWS = TT * 16;
  // per-row metadata of the up-projection, built during the main loop in an LDS area of
  // its own (byte offsets from that area)
  static constexpr int ROWAD = 0;                    // int [ROWS]: adapter of the row (-1: none)
  static constexpr int ROWRK = ROWAD + ROWS * 4;     // int [ROWS]: its rank
  static constexpr int ROWSC = ROWRK + ROWS * 4;     // float [ROWS]: its scale
  static constexpr int ROWBP = ROWSC + ROWS * 4;     // uint64 [ROWS]: address of its B^T
  static constexpr int ITEMS = ROWBP + ROWS * 8;     // int [2 * ROWS]: up-projection work items
  static constexpr int IOFF = ITEMS + ROWS * 8;      // int [2 * ROWS]: LDS offset of the item's B slice
  static constexpr int LROW = IOFF + ROWS * 8;       // int [ROWS]: leader rows of this split's adapters, in order
  static constexpr int LEAD = LROW + ROWS * 4;       // int [ROWS]: token tiles of the row's adapter (leader rows)
  static constexpr int LEADOF = LEAD + ROWS * 4;     // int [ROWS]: leader row of the row's adapter (-1: none)
  static constexpr int MINE = LEADOF + ROWS * 4;     // int [ROWS]: leader rows whose adapter this K-split adds
  static constexpr int RLIST = MINE + ROWS * 4;      // int [ROWS]: rows whose t this K-split needs
  static constexpr int META = RLIST + ROWS * 4;      // int [16]
  static constexpr int MD_BYTES = META + 64;
  // after the main loop, over the x staging area (offsets from the start)
  static constexpr int TB = 0;                       // bf16 [ROWS][TSTR]: s_a * t
  static constexpr int LRED = TB + ROWS * TSTR * 2;  // float [WK-1][WC][TT][CT][256]: k-wave sums
  static constexpr int POST = LRED + (WK - 1) * WC * TT * CT * 256 * 4;
  static_assert(ROWBP % 8 == 0 && LRED % 16 == 0, "epilogue LDS alignment");
};

template <int TT, int CT, int WC, int WK, int OCC, bool A16 = false>
struct GemmSmem {
  using CK = ChunkK<TT, CT>;
  // the chunked loop stages x in two buffers (chunk c + 1 is staged while chunk c is
  // multiplied); the one-tile stream does not use them.  MXFP8: codes and scale codes;
  // 16-bit activations: the bf16 rows themselves
  static constexpr int XROW16 = CK::KC * 2 + 16;
  static constexpr int XBUF =
      (A16 && TT != 1) ? TT * 16 * XROW16 : ((TT * 16 * CK::ROW + TT * 16 * (CK::KC / 32)) + 15) & ~15;
  static constexpr int MAIN = (TT == 1) ? XBUF : 2 * XBUF;
  static constexpr int RED = (WK - 1) * WC * TT * CT * 256 * 4;
  static constexpr int POST = EpiLayout<TT, CT, WC, WK>::POST;
  static constexpr int M1 = MAIN > RED ? MAIN : RED;
  static constexpr int MD = ((M1 > POST ? M1 : POST) + 15) & ~15;  // metadata area, kept through the loop
  static constexpr int STG = (MD + EpiLayout<TT, CT, WC, WK>::MD_BYTES + 1023) & ~1023;  // B staging
  // B staging budget: what is left of the workgroup's share of the 160 KB LDS, at most
  // epi_bstage (room for two slices of the widest tile at the largest rank)
  static constexpr int LDS_WG = (160 * 1024 - 1024) / OCC;
  static constexpr int BST = (epi_bstage<OCC>() < LDS_WG - STG) ? epi_bstage<OCC>() : ((LDS_WG - STG) & ~1023);
  static_assert(BST >= 2 * WC * CT * 16 * MAX_RANK * 2, "LDS too small for two B slices");
  static constexpr int BYTES = STG + BST;
};

template <int FMT, int TT, int CT, int WC, int WK, bool XQ, int KPT, int OCC, bool A16>
__device__ __forceinline__ void gemm_item(const GemmParams& p, int item, char* smem, int e, int* lds_epoch, int* started) {
  using CK = ChunkK<TT, CT>;
  constexpr int KC = CK::KC, STEPS = CK::STEPS, ROW = CK::ROW;
  constexpr int SPW = STEPS / WK;  // k-steps per wave per chunk
  constexpr int WN = WC * CT * 16;
  constexpr int FMTB = (FMT == LORA_W_FP8_E4M3) ? 0 : 4;
  constexpr int ROWS = TT * 16;
  constexpr int KP = KPT;  // K-parts of t the epilogue adds (the host plan stays within it)
  // t elements per thread per gather batch: the whole block's t (ROWS x 64) in one batch,
  // so that the gather costs one memory round trip
  constexpr int EPI_TE = (ROWS * MAX_RANK + 255) / 256;
  // gather batches (one: the main loop's staging registers are free by then)
  constexpr int EPI_PH = 1;
  constexpr int EPI_TH = EPI_TE / EPI_PH;
  static_assert(STEPS % WK == 0, "k-steps per chunk must split evenly over the k-waves");
  // x staging buffer b: [ROWS][ROW] codes, then [ROWS][KC/32] scale codes
  constexpr int XBUF = GemmSmem<TT, CT, WC, WK, OCC, A16>::XBUF;
  auto xs_of = [&](int b) { return reinterpret_cast<uint8_t*>(smem) + b * XBUF; };
  auto ss_of = [&](int b) { return reinterpret_cast<uint8_t*>(smem) + b * XBUF + ROWS * ROW; };
  // scale code of row `row`, 32-block k32 of the chunk: the TT codes a lane needs for one
  // k-step (rows li + 16 tt, block 4 sp + g) lie next to each other
  static_assert(TT == 1 || TT == 4 || TT == 8, "scale layout: four or eight token tiles");
  auto sidx = [&](int row, int k32) { return (k32 * 16 + (row & 15)) * TT + (row >> 4); };

  // wave index as a scalar (see the down-projection)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15,
            g = lane >> 4;
  const int wc = wave % WC, wk = wave / WC;
  const int ks = item % p.ksplit;
  const int tile = item / p.ksplit;
  int cb = tile % p.n_cb, tb = tile / p.n_cb;
  if (p.tile_group > 0) {
    // XCD-grouped order (the host sets it only without a K-split, with a multiple of 8
    // tiles and of 8 workgroups before the first GEMM workgroup).  Workgroups are dealt to
    // the eight XCDs in turn, so items item % 8 == x run on XCD x, in the order item / 8.
    // XCD x takes the x-th eighth of the tiles in an order that walks groups of
    // tile_group column blocks token block by token block: the tiles an XCD runs at one
    // time then share a few W column blocks and a few x row blocks in its L2.
    const int per = (p.n_cb * p.n_tb) >> 3;
    const int L = (item & 7) * per + (item >> 3);
    const int G = p.tile_group, gsz = G * p.n_tb;
    const int grp = L / gsz, r = L - grp * gsz;
    tb = r / G;
    cb = grp * G + (r - (r / G) * G);
  }
  if (TT == 1 && p.n_tb > 1) {
    // several 16-token tiles per column tile (16-bit activations past 16 tokens): the tiles
    // of one column tile take item ids 8 apart, so that they run on one XCD (workgroups are
    // dealt to the eight XCDs in turn) at about the same time and read W once into its L2.
    // Column tiles beyond the last multiple of 8 keep the plain order.
    const int full = (p.n_cb / 8) * 8;
    if (tile < full * p.n_tb) {
      const int j = tile / 8;
      tb = j % p.n_tb;
      cb = (j / p.n_tb) * 8 + tile % 8;
    } else {
      const int r = tile - full * p.n_tb, rest = p.n_cb - full;
      cb = full + r % rest;
      tb = r / rest;
    }
  }
  const int row0 = tb * ROWS;
  const int n_tile0 = cb * WN;
  const int nw0 = n_tile0 + wc * CT * 16;
  const int K = p.K;

  // packed W (see k_pack_weight): per 16-channel tile and k-step, 2 KB (FP8) or 1 KB
  // (MXFP4) in lane order, plus 64 scale bytes for MXFP4
  constexpr int WSTEP = (FMT == LORA_W_FP8_E4M3) ? 2048 : 1024;
  const uint8_t* wrow[CT];
  const uint8_t* wsrow[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const long nt = (nw0 + ct * 16) / 16;
    wrow[ct] = p.wq + nt * (K / 128) * WSTEP + lane * 16;
    wsrow[ct] = (FMT == LORA_W_FP8_E4M3) ? nullptr : p.ws_fp4 + nt * (K / 128) * 64 + lane;
  }

  v4f acc[TT][CT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[tt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  // FP8 channel scales of the lane's columns: the chunked loop loads them when it ends (no
  // registers held through it), the one-tile stream at the start
  float chan_s[CT];
  auto load_chan_s = [&]() {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) chan_s[ct] = (FMT == LORA_W_FP8_E4M3) ? p.ws_fp8[nw0 + ct * 16 + li] : 1.f;
  };
  if constexpr (TT == 1) load_chan_s();
  // adapter of row `tid` of the token block for the epilogue: the id is loaded before the
  // bulk loads, its rank, scale and B address right after the first ones (loads retire
  // in order, so none of these waits for more than the id)
  const int id_raw = p.lora ? p.ids[min(row0 + min(tid, ROWS - 1), p.T - 1)] : -1;

  const int kb = ks * p.krange, ke = min(K, kb + p.krange);
  const int nchunks = (ke - kb + KC - 1) / KC;
  // Every tile walks its K-range from a different place (chunk and step rotation), so that
  // the workgroups do not all hit the same HBM channels with rows that are K bytes apart.
  const int crot = p.rot ? tile % nchunks : 0;
  const int srot = p.rot ? (tile * 5) & (STEPS - 1) : 0;
  auto chunk_k0 = [&](int c) { return kb + ((c + crot) % nchunks) * KC; };

  // register staging, two chunks ahead: x (raw bf16 or pre-quantised) and W.
  // Pre-quantised x is read in 16-byte pieces, piece P = tid + 256 m of the chunk's rows,
  // so that each wave's load covers 1 KB of a row.  Raw bf16 x is read a 32-block per
  // thread (four 16-byte loads), so that the thread quantises the whole block itself: a
  // piece layout would need a cross-lane maximum per block, which measured slower.
  constexpr int PPR = KC / 16;               // MXFP8 pieces per row and chunk
  constexpr int NP = ROWS * PPR / 256;       // MXFP8 pieces per thread and chunk
  constexpr int NBLK = ROWS * (KC / 32) / 256;  // bf16 32-blocks per thread and chunk
  constexpr int NX = XQ ? NP : 4 * NBLK;     // 16-byte registers per chunk
  static_assert(NP >= 1 && NBLK >= 1 && NBLK * 256 == ROWS * (KC / 32), "chunk does not split evenly");
  // chunks in flight (measured on the 64-token tile: three or four are no faster than two)
  constexpr int NBUF = 2;
  static_assert(NBUF == 2, "x registers and LDS buffers alternate between two chunks");
  uint4 xr[NBUF][NX];
  // pre-quantised x: the chunk's scale codes, ROWS x SB bytes, are one load of wave 0
  // (lane l: rows SRL*l .. SRL*l + SRL - 1)
  constexpr int SB = KC / 32;
  static_assert(!XQ || ((SB == 8 || SB == 4) && (ROWS == 64 || ROWS == 128)),
                "scale staging: 4 or 8 codes per row, 64 or 128 rows");
  constexpr int SRL = (ROWS >= 64) ? ROWS / 64 : 1;
  uint2 xsc2[NBUF][SRL];
  uint4 wlo[NBUF][SPW][CT], whi[NBUF][SPW][CT];
  int wsc[NBUF][SPW][CT];

  auto load_x = [&](int buf, int c) {
    const int kc0 = chunk_k0(c);
    // unconditional loads from clamped addresses: rows past T repeat row T-1 and only
    // feed rows that are never stored; pieces and blocks past the chunk end are never
    // read back from LDS
    if (XQ) {
      const int ppr = min(KC, ke - kc0) / 16;
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int P = tid + 256 * m;
        const int row = P / PPR, pp = min(P % PPR, ppr - 1);
        const long tok = min(row0 + row, p.T - 1);
        xr[buf][m] = ldg16(p.xq + tok * K + kc0 + pp * 16);
      }
    } else {
      const int bpr = min(KC, ke - kc0) >> 5;
#pragma unroll
      for (int m = 0; m < NBLK; ++m) {
        const int b = tid + 256 * m;
        const int row = b / (KC / 32), k32 = min(b % (KC / 32), bpr - 1);
        const long tok = min(row0 + row, p.T - 1);
        const uint16_t* src = p.x + tok * K + kc0 + k32 * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[buf][4 * m + q] = ldg16(src + 8 * q);
      }
    }
    if (XQ && wave == 0) {
#pragma unroll
      for (int h = 0; h < SRL; ++h) {
        // SB / 4 four-byte loads (rows are 4-byte aligned); in a partial last chunk the second
        // may read codes past the row, which are never used (the workspace pads the array)
        const long tok = min(row0 + SRL * lane + h, p.T - 1);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(p.xsc + tok * (K / 32) + (kc0 >> 5));
        xsc2[buf][h] = make_uint2(src[0], SB == 8 ? src[1] : 0u);
      }
    }
  };
  // physical k-step of logical step s in a chunk of nsteps steps
  auto phys_step = [&](int s, int nsteps) { return (s + srot) % nsteps; };
  auto load_w = [&](int buf, int c) {
    const int kc0 = chunk_k0(c);
    const int nsteps = min(KC, ke - kc0) >> 7;
    // k-steps past the range load step 0 again; their MFMAs are skipped
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int s = wk + WK * i;
      const long ksg = (kc0 >> 7) + (s < nsteps ? phys_step(s, nsteps) : 0);  // global k-step
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if (FMT == LORA_W_FP8_E4M3) {
          wlo[buf][i][ct] = ldg16(wrow[ct] + ksg * WSTEP);
          whi[buf][i][ct] = ldg16(wrow[ct] + ksg * WSTEP + 1024);
          wsc[buf][i][ct] = 127;
        } else {
          wlo[buf][i][ct] = ldg16(wrow[ct] + ksg * WSTEP);
          whi[buf][i][ct] = zero4();
          wsc[buf][i][ct] = (int)wsrow[ct][ksg * 64];
        }
      }
    }
  };
  auto stage_x = [&](int buf) {  // x registers of buffer buf -> LDS buffer buf
    uint8_t* xs = xs_of(buf);
    uint8_t* ss = ss_of(buf);
    if constexpr (A16) {  // the bf16 blocks as they are: row stride XROW16, block k32 at 64 k32
      constexpr int XR = GemmSmem<TT, CT, WC, WK, OCC, A16>::XROW16;
#pragma unroll
      for (int m = 0; m < NBLK; ++m) {
        const int b = tid + 256 * m;
        const int row = b / (KC / 32), k32 = b % (KC / 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(xs + row * XR + k32 * 64 + 16 * q) = xr[buf][4 * m + q];
      }
      return;
    }
    if (XQ) {
#pragma unroll
      for (int m = 0; m < NP; ++m) {
        const int P = tid + 256 * m;
        const int row = P / PPR, pp = P % PPR;
        *reinterpret_cast<uint4*>(xs + row * ROW + pp * 16) = xr[buf][m];
      }
    } else {
#pragma unroll
      for (int m = 0; m < NBLK; ++m) {
        const int b = tid + 256 * m;
        const int row = b / (KC / 32), k32 = b % (KC / 32);
        const uint4 in[4] = {xr[buf][4 * m], xr[buf][4 * m + 1], xr[buf][4 * m + 2], xr[buf][4 * m + 3]};
        const uint32_t code = mx_block_code(in);
        uint4 out[2];
        mx_block_quant(in, code, out);
        *reinterpret_cast<uint4*>(xs + row * ROW + k32 * 32) = out[0];
        *reinterpret_cast<uint4*>(xs + row * ROW + k32 * 32 + 16) = out[1];
        ss[sidx(row, k32)] = (uint8_t)code;
      }
    }
    if (XQ && wave == 0) {
#pragma unroll
      for (int h = 0; h < SRL; ++h)
#pragma unroll
        for (int k32 = 0; k32 < SB; ++k32)
          ss[sidx(SRL * lane + h, k32)] =
              (uint8_t)(((k32 < 4) ? xsc2[buf][h].x : xsc2[buf][h].y) >> (8 * (k32 & 3)));
    }
  };
  auto mma_chunk_a16 = [&](int buf, int c) {
    // 16-bit activations: per k-step the lane widens its W codes of each column tile to four
    // bf16 operands once, then per token tile reads the four 8-element x pieces at the same
    // k (FP8: 16g, 16g+8, 64+16g, 72+16g; MXFP4: 32g .. 32g+31) and issues four bf16 MFMAs
    constexpr int XR = GemmSmem<TT, CT, WC, WK, OCC, A16>::XROW16;
    const uint8_t* xs = xs_of(buf);
    const int kc0 = chunk_k0(c);
    const int nsteps = min(KC, ke - kc0) >> 7;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int s = wk + WK * i;
      if (s >= nsteps) break;
      const int sp = phys_step(s, nsteps);
      uint4 wb[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if constexpr (FMT == LORA_W_FP8_E4M3) {
          const uint4 lo = wlo[buf][i][ct], hi = whi[buf][i][ct];
          const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint2 a = fp8x4_to_bf16(d[2 * m]), b = fp8x4_to_bf16(d[2 * m + 1]);
            wb[ct][m] = make_uint4(a.x, a.y, b.x, b.y);
          }
        } else {
          const float sc = __builtin_bit_cast(float, wsc[buf][i][ct] << 23);
          const uint4 lo = wlo[buf][i][ct];
          wb[ct][0] = fp4x8_to_bf16(lo.x, sc);
          wb[ct][1] = fp4x8_to_bf16(lo.y, sc);
          wb[ct][2] = fp4x8_to_bf16(lo.z, sc);
          wb[ct][3] = fp4x8_to_bf16(lo.w, sc);
        }
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint8_t* xp = xs + (tt * 16 + li) * XR + sp * 256;
        uint4 xf[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int k = (FMT == LORA_W_FP8_E4M3) ? ((m >> 1) * 64 + 16 * g + 8 * (m & 1)) : (32 * g + 8 * m);
          xf[m] = *reinterpret_cast<const uint4*>(xp + 2 * k);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[tt][ct] = mfma_bf16_16x16x32(xf[m], wb[ct][m], acc[tt][ct]);
      }
    }
  };
  auto mma_chunk = [&](int buf, int c) {  // LDS buffer and W registers of buffer buf
    if constexpr (A16) {
      mma_chunk_a16(buf, c);
      return;
    }
    const uint8_t* xs = xs_of(buf);
    const uint8_t* ss = ss_of(buf);
    const int kc0 = chunk_k0(c);
    const int nsteps = min(KC, ke - kc0) >> 7;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int s = wk + WK * i;
      if (s >= nsteps) break;
      const int sp = phys_step(s, nsteps);
      // the scale codes of the lane's TT rows for this k-step: one read (the MFMA picks
      // the byte), and the x fragment of token tile tt + 1 is read before the MFMAs of
      // tile tt go out, so that its LDS latency overlaps them
      const uint8_t* sb = ss + sidx(li, sp * 4 + g);
      uint32_t sc[2];
      if constexpr (TT == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(sb);
        sc[0] = v.x;
        sc[1] = v.y;
      } else {
        sc[0] = *reinterpret_cast<const uint32_t*>(sb);
        sc[1] = 0u;
      }
      // fragments read FD token tiles ahead of their MFMAs (measured: two ahead on the
      // 128 x 256 prefill tile, no faster, and the registers spill)
      constexpr int FD = 1;
      constexpr int FB = FD + 1;
      uint4 alo[FB], ahi[FB];
      auto frag = [&](int tt) {
        const uint8_t* xp = xs + (tt * 16 + li) * ROW + sp * 128 + 16 * g;
        alo[tt % FB] = *reinterpret_cast<const uint4*>(xp);
        ahi[tt % FB] = *reinterpret_cast<const uint4*>(xp + 64);
      };
#pragma unroll
      for (int tt = 0; tt < FD; ++tt) frag(tt);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt + FD < TT) frag(tt + FD);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[tt][ct] = mfma_scaled_16x16x128_sel<FMTB>(tt & 3, alo[tt % FB], ahi[tt % FB], wlo[buf][i][ct],
                                                         whi[buf][i][ct], acc[tt][ct], (int)sc[tt >> 2],
                                                         wsc[buf][i][ct]);
      }
      // keep that order: the scale and first FD fragments' reads, then per token tile the
      // reads FD tiles ahead before the tile's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1 + 2 * FD, 0);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt + FD < TT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, CT, 0);
      }
    }
  };

  // ---- one-token-tile decode (16 tokens, the four waves splitting K): each wave streams
  //      its own k-steps s = wk, wk+4, ... with x loaded straight into the MFMA operand
  //      layout and quantised in registers, so the main loop needs no LDS and no barrier.
  //      Lane (li, g) holds token row li at k = 16g .. 16g+15 (first half of the operand) and
  //      64+16g .. 64+16g+15 (second half); a 32-block spans the lanes g and g^1 (16 apart),
  //      which exchange their maxima.  The scale operand of lane (li, g) is the code of
  //      K-block g, held by the lanes g' with g'/2 == g%2 in their first (g < 2) or second
  //      half: lanes g = 1 and g = 2 swap one code.
  constexpr bool STREAM = (TT == 1 && WC == 1 && WK == 4 && !XQ);
  // 16-bit activations: x enters bf16 MFMAs as it is and W is widened to bf16 in
  // registers (FP8: the lane's codes are at the k of its x pieces; MXFP4: lane (li, g)
  // holds k = 32g .. 32g+31, one block, so x is read there and the block scale is
  // applied in the widening).  The one-tile stream only.
  static_assert(!A16 || STREAM || (TT == 4 && CT == 2 && !XQ), "16-bit activations: the stream or 64 x 128 tiles");
  constexpr bool A16_FP4 = A16 && FMT == LORA_W_MXFP4_E2M1;
  constexpr int SD = 4;  // k-steps of a wave in flight (measured: 2, 3 and 6 are slower)
  const int nst = (ke - kb) >> 7;
  const int nmy = (nst > wk) ? (nst - wk + 3) / 4 : 0;
  const int srot_all = (tile * 5) % (nst > 0 ? nst : 1);
  auto kstep = [&](int i) {  // physical k-step of the wave's i-th step (clamped, always valid)
    const int ic = max(min(i, nmy - 1), 0);
    const int sl = (nmy > 0) ? wk + 4 * ic : 0;
    return (sl + srot_all) % nst;
  };
  uint4 sx[SD][4];
  v8i sw[SD][CT];
  int sws[SD][CT];
  const uint16_t* xs_row = p.x + (long)min(row0 + li, p.T - 1) * K + kb + (A16_FP4 ? 32 : 16) * g;
  auto s_issue = [&](int slot, int i) {
    const int ps = kstep(i);
    const uint16_t* xp = xs_row + ps * 128;
    sx[slot][0] = ldg16(xp);
    sx[slot][1] = ldg16(xp + 8);
    sx[slot][2] = ldg16(xp + (A16_FP4 ? 16 : 64));
    sx[slot][3] = ldg16(xp + (A16_FP4 ? 24 : 72));
    const long ksg = (kb >> 7) + ps;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      if (FMT == LORA_W_FP8_E4M3) {
        sw[slot][ct] = join8(ldg16(wrow[ct] + ksg * WSTEP), ldg16(wrow[ct] + ksg * WSTEP + 1024));
        sws[slot][ct] = 127;
      } else {
        sw[slot][ct] = join8(ldg16(wrow[ct] + ksg * WSTEP), zero4());
        sws[slot][ct] = (int)wsrow[ct][ksg * 64];
      }
    }
  };
  auto s_consume_a16 = [&](int slot) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const v8i w = sw[slot][ct];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint4 b;
        if constexpr (A16_FP4) {
          // e8m0 code c as the float 2^(c - 127) (exact widening for codes 2 .. 252)
          b = fp4x8_to_bf16((uint32_t)w[m], __builtin_bit_cast(float, sws[slot][ct] << 23));
        } else {
          const uint2 lo = fp8x4_to_bf16((uint32_t)w[2 * m]), hi = fp8x4_to_bf16((uint32_t)w[2 * m + 1]);
          b = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        acc[0][ct] = mfma_bf16_16x16x32(sx[slot][m], b, acc[0][ct]);
      }
    }
  };
  auto s_consume = [&](int slot) {
    if constexpr (A16) {
      s_consume_a16(slot);
    } else {
      uint32_t m1 = max(absmax8_bits(sx[slot][0]), absmax8_bits(sx[slot][1]));
      uint32_t m2 = max(absmax8_bits(sx[slot][2]), absmax8_bits(sx[slot][3]));
      m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 16));
      m2 = max(m2, (uint32_t)__shfl_xor((int)m2, 16));
      const uint32_t c1 = mx_code_from_bits(m1), c2 = mx_code_from_bits(m2);
      const uint2 q0 = mx_piece_quant(sx[slot][0], c1), q1 = mx_piece_quant(sx[slot][1], c1);
      const uint2 q2 = mx_piece_quant(sx[slot][2], c2), q3 = mx_piece_quant(sx[slot][3], c2);
      const uint4 alo = make_uint4(q0.x, q0.y, q1.x, q1.y), ahi = make_uint4(q2.x, q2.y, q3.x, q3.y);
      const uint32_t recv = (uint32_t)__shfl_xor((int)((g == 1) ? c2 : c1), 48);
      const int sa = (int)((g == 0) ? c1 : ((g == 3) ? c2 : recv));
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        acc[0][ct] = mfma_scaled_16x16x128<FMTB>(alo, ahi, sw[slot][ct], acc[0][ct], sa, sws[slot][ct]);
    }
  };

  // chunks 0 .. NBUF-1 in flight before anything waits; chunk c + NBUF is issued into the
  // buffer of chunk c while chunk c is multiplied (x once it is staged, W after its MFMAs).
  // x of a chunk is always issued before its W (loads retire in order).
  if (STREAM) {
#pragma unroll
    for (int d = 0; d < SD; ++d) s_issue(d, d);
  } else {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {  // past the last chunk: a chunk again (never multiplied)
      load_x(u, u);
      load_w(u, u);
    }
  }
  const bool row_ok = p.lora && tid < ROWS && row0 + tid < p.T && id_raw >= 0 &&
                      id_raw < p.n_ad;
  int row_r = 0;
  float row_s = 0.f;
  uint64_t row_bp = 0;
  if (p.lora) {  // unconditional loads from a valid index
    const int ac = row_ok ? id_raw : 0;
    row_r = p.ranks[ac];
    row_s = p.scales[ac];
    row_bp = p.B_ptrs[ac];
  }
  // up-projection metadata (adapter list, work items, rows whose t is needed), built once
  // the first chunk is multiplied: its LDS latency then overlaps the loads in flight
  using EL = EpiLayout<TT, CT, WC, WK>;
  char* md = smem + GemmSmem<TT, CT, WC, WK, OCC, A16>::MD;
  int* rowad = reinterpret_cast<int*>(md + EL::ROWAD);
  int* rowrk = reinterpret_cast<int*>(md + EL::ROWRK);
  float* rowsc = reinterpret_cast<float*>(md + EL::ROWSC);
  uint64_t* rowbp = reinterpret_cast<uint64_t*>(md + EL::ROWBP);
  int* items = reinterpret_cast<int*>(md + EL::ITEMS);
  int* lead = reinterpret_cast<int*>(md + EL::LEAD);
  int* leadof = reinterpret_cast<int*>(md + EL::LEADOF);
  int* mine = reinterpret_cast<int*>(md + EL::MINE);
  int* rowlist = reinterpret_cast<int*>(md + EL::RLIST);
  int* meta = reinterpret_cast<int*>(md + EL::META);
  int* ioff = reinterpret_cast<int*>(md + EL::IOFF);
  int* lrow = reinterpret_cast<int*>(md + EL::LROW);
  char* stg = smem + GemmSmem<TT, CT, WC, WK, OCC, A16>::STG;
  const int slot = WN * p.r_max * 2;  // bytes of one B slice slot (a multiple of 512)
  constexpr int BST = GemmSmem<TT, CT, WC, WK, OCC, A16>::BST;
  const int spb = BST / slot;  // slots per batch (>= 2)
  static_assert(BST / (WN * 8 * 2) <= 256, "stage_b keeps a wave's slices one per lane");
  auto prepare_epilogue = [&]() {
    // (1) adapter, rank, scale and B address of every row; a rank outside [1, r_max]
    //     drops the row's adapter term (adapter -2: reported after the main loop)
    if (tid < ROWS) {
      const bool ok = row_ok && row_r >= 1 && row_r <= p.r_lim;
      rowad[tid] = ok ? id_raw : (row_ok ? -2 : -1);
      rowrk[tid] = ok ? row_r : 0;
      rowsc[tid] = row_s;
      rowbp[tid] = row_bp;
    }
    __syncthreads();
    // (2) work items: one per adapter present in the token block and 32 of its ranks, in
    //     order of the adapter's first row (its leader), with the set of 16-row token tiles
    //     that hold its rows; each item's B operands then serve all those tiles
    // The leader is found through a table of first rows indexed by adapter (n_ad <=
    // MAX_ADAPTERS ints, in the B staging area, which is free until the main loop ends):
    // the rows set their adapter's entry, then take the minimum with an LDS atomic.
    int my_lead = -1;
    int* first_row = reinterpret_cast<int*>(stg);
    static_assert(MAX_ADAPTERS * 4 <= BST, "first-row table in the B staging area");
    const int a_row = (tid < ROWS) ? rowad[tid] : -1;  // -1 or an adapter index below n_ad
    if (tid < ROWS) {
      lead[tid] = 0;
      mine[tid] = 0;
    }
    if (a_row >= 0) first_row[a_row] = ROWS;
    __syncthreads();
    if (a_row >= 0) atomicMin(first_row + a_row, tid);
    __syncthreads();
    if (a_row >= 0) my_lead = first_row[a_row];
    if (tid < ROWS) leadof[tid] = my_lead;
    __syncthreads();
    if (my_lead >= 0) atomicOr(lead + my_lead, 1 << (tid >> 4));
    __syncthreads();
    // With a K-split the tile's adapters are dealt round-robin (in leader order) to its
    // splits: each split adds the up-projection of its share to its own sum.
    if (wave == 0) {
      int n = 0, n_lead = 0, n_own = 0;
      for (int c0 = 0; c0 < ROWS; c0 += 64) {
        const int row = c0 + lane;
        const int mask = (row < ROWS) ? lead[row] : 0;  // non-zero only for leader rows
        const unsigned long long bl = __ballot(mask != 0);
        const int ord = n_lead + __popcll(bl & ((1ull << lane) - 1ull));
        n_lead += __popcll(bl);
        const bool own = mask != 0 && (ord % p.ksplit) == ks;
        if (own) mine[row] = 1;
        // this split's k-th adapter: B slice in slot k % spb of batch k / spb
        const unsigned long long bo = __ballot(own);
        const int k = n_own + __popcll(bo & ((1ull << lane) - 1ull));
        n_own += __popcll(bo);
        if (own) lrow[k] = row;
        // items of 32 ranks: one or two per adapter (ranks up to 64), so the inclusive prefix
        // over the lanes is two ballot counts
        static_assert(MAX_RANK <= 64, "at most two 32-rank items per adapter");
        const int nb = own ? ((rowrk[row] + 31) >> 5) : 0;
        const unsigned long long b1 = __ballot(nb >= 1), b2 = __ballot(nb >= 2);
        const unsigned long long le = (lane == 63) ? ~0ull : ((1ull << (lane + 1)) - 1ull);
        const int incl = __popcll(b1 & le) + __popcll(b2 & le);
        for (int b = 0; b < nb; ++b) {
          items[n + incl - nb + b] = row | (b << 8) | (mask << 9) | ((k / spb) << 17);
          ioff[n + incl - nb + b] = (k % spb) * slot;
        }
        n += __popcll(b1) + __popcll(b2);
      }
      // rows whose t this split needs (rows of its adapters), in row order
      int nr = 0;
      for (int c0 = 0; c0 < ROWS; c0 += 64) {
        const int row = c0 + lane;
        const bool need = row < ROWS && rowrk[row] > 0 && (p.ksplit == 1 || mine[max(leadof[row], 0)]);
        const unsigned long long bl = __ballot(need);
        if (need) rowlist[nr + __popcll(bl & ((1ull << lane) - 1ull))] = row;
        nr += __popcll(bl);
      }
      // any row whose adapter has a rank outside [1, r_max]
      bool bad = false;
      for (int c0 = 0; c0 < ROWS; c0 += 64) bad |= __ballot(c0 + lane < ROWS && rowad[c0 + lane] == -2) != 0ull;
      if (lane == 0) {
        meta[0] = n;
        meta[1] = nr;
        meta[2] = n_own;
        meta[3] = bad ? 1 : 0;
      }
    }
  };

  // ---- up-projection helpers: B slices into LDS and the t gather.  They go out as soon as
  //      the tile knows its rows' adapters: in the one-tile stream while the last k-steps
  //      are in flight, otherwise when the main loop ends (before the k-wave sums)
  uint16_t* tbuf = reinterpret_cast<uint16_t*>(smem + EL::TB);
  float* lred = reinterpret_cast<float*>(smem + EL::LRED);
  int n_items = 0, n_rows = 0, n_own = 0, n_batch = 0, nel = 0;
  auto read_meta = [&]() {
    n_items = __builtin_amdgcn_readfirstlane(meta[0]);
    n_rows = __builtin_amdgcn_readfirstlane(meta[1]);
    n_own = __builtin_amdgcn_readfirstlane(meta[2]);
    n_batch = (n_own + spb - 1) / spb;
    nel = n_rows * p.r_max;
  };

  // B_a^T rows n_tile0 .. n_tile0 + WN - 1 of one adapter are WN * r_a contiguous bf16;
  // the waves copy the slices of a batch straight into their LDS slots (16 bytes per
  // lane, 1 KB per wave load), leader k of the batch by wave k % 4
  auto stage_b = [&](int b) {
    // the wave's slices k = b*spb + wave + 4j: their rank and B address are read from LDS
    // first, one per lane, because an LDS read placed after a direct-to-LDS copy waits for
    // that copy to land (the copies would go out one memory round trip apart)
    const int kb0 = b * spb + wave, k1 = min(n_own, (b + 1) * spb);
    const int nk = (k1 > kb0) ? (k1 - kb0 + 3) / 4 : 0;  // at most spb / 4 <= 64
    int r_l = 0;
    uint64_t bp_l = 0;
    if (lane < nk) {
      const int row = lrow[kb0 + 4 * lane];
      r_l = rowrk[row];
      bp_l = rowbp[row];
    }
    for (int j = 0; j < nk; ++j) {
      const int k = kb0 + 4 * j;
      const int r = __builtin_amdgcn_readlane(r_l, j);
      const uint64_t bpu = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bp_l >> 32), j) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bp_l, j);
      const int r8 = rank_pad(r);  // the stored row length of B_a^T
      const char* src = reinterpret_cast<const char*>(bpu) + (long)n_tile0 * r8 * 2;
      char* dst = stg + (k % spb) * slot;
      const int bytes = WN * r8 * 2;
      for (int c = 0; c < bytes; c += 1024) {
        if (c + lane * 16 < bytes)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + c + lane * 16),
                                           (__attribute__((address_space(3))) void*)(dst + c), 16, 0, 0);
      }
    }
  };
  uint64_t traw[EPI_TH][KP];
  float tpl[EPI_TH];
  // element idx = tid + 256 (ph * EPI_TH + m) of the row list, one word each: row (bits
  // 0-7), rank index (8-15), the row's rank (16-23, filled in when the tags are checked);
  // all the list reads go out before the first use, so their latencies overlap
  int tinf[EPI_TH];
  auto trow = [&](int m) { return tinf[m] & 255; };
  auto tcol = [&](int m) { return (tinf[m] >> 8) & 255; };
  // (with bf16 pairs, an element is a pair of ranks: rank index = pair index)
  const bool tpack = !STREAM && p.t_tag && p.t_pack;
  auto t_elements = [&](int ph) {
    const int rm = __builtin_amdgcn_readfirstlane(tpack ? p.r_max >> 1 : p.r_max);
    const int ne = tpack ? nel >> 1 : nel;
#pragma unroll
    for (int m = 0; m < EPI_TH; ++m) {
      const int idx = min(tid + 256 * (ph * EPI_TH + m), max(ne - 1, 0));
      const int q = idx / rm;
      tinf[m] = rowlist[min(q, ROWS - 1)] | ((idx - q * rm) << 8);
    }
  };
  // t of the rows this split needs (all of them fit EPI_PH batches of EPI_TH per thread):
  // tagged partials (fused) or the caller's plain t
  auto load_t = [&](int ph) {
    t_elements(ph);
    if (nel == 0) {
      // no rows: nothing to load
    } else if (tpack) {  // half the elements: pairs of ranks
#pragma unroll
      for (int m = 0; m < EPI_TH / 2; ++m)
        traw[m][0] = ld_agent_u64(p.t_tag + (long)(row0 + trow(m)) * (p.r_max >> 1) + tcol(m));
    } else if (p.t_tag) {  // unconditional loads from clamped addresses; tags checked later
#pragma unroll
      for (int m = 0; m < EPI_TH; ++m) {
        const long addr = (long)(row0 + trow(m)) * p.r_max + tcol(m);
#pragma unroll
        for (int k2 = 0; k2 < KP; ++k2)
          traw[m][k2] = ld_agent_u64(p.t_tag + (long)min(k2, p.t_kparts - 1) * p.T * p.r_max + addr);
      }
    } else {
#pragma unroll
      for (int m = 0; m < EPI_TH; ++m) tpl[m] = p.t[(long)(row0 + trow(m)) * p.r_lim + min(tcol(m), p.r_lim - 1)];
    }
  };
  // The stream's tagged t gather, issued before its last round of k-steps is multiplied:
  // EPI_TE x KP loads per thread on every path, each from its own address (an element it
  // needs, else a distinct word of x), so that none can be merged away and the waits for
  // those k-steps do not have to assume that fewer loads went out after them.
  auto load_t_stream = [&]() {
    static_assert(!STREAM || EPI_PH == 1, "the stream gathers t in one batch");
    t_elements(0);  // list reads unconditional (a stale value is never used)
    const int rm = max(p.r_max, 1);
    const uint64_t* dummy = reinterpret_cast<const uint64_t*>(p.x);
    const uint64_t tb = reinterpret_cast<uint64_t>(p.t_tag), xb = reinterpret_cast<uint64_t>(dummy);
    const bool tag_on = p.t_tag != nullptr;
#pragma unroll
    for (int m = 0; m < EPI_TH; ++m) {
      const bool use = tag_on && tid + 256 * m < nel;
      const long elem = (long)(row0 + trow(m)) * rm + tcol(m);
#pragma unroll
      for (int k2 = 0; k2 < KP; ++k2) {
        const uint64_t a_use = tb + 8ull * (uint64_t)((long)min(k2, max(p.t_kparts, 1) - 1) * p.T * rm + elem);
        const uint64_t a_dum = xb + 8ull * (uint64_t)(m * KP + k2);
        traw[m][k2] = ld_agent_u64_at(use ? a_use : a_dum);
      }
    }
  };

  // The stream's B operands, when the tile has at most one up-projection item per wave (the
  // single-adapter decode): each wave loads its item's operands (CT x 16 bytes per lane) with
  // the t gather, instead of staging B slices in LDS after the loop.  A fixed count of
  // loads on every path (x as a dummy source), as for the t gather.
  uint4 sb[CT];
  int sb_it = 0, sb_a = -1, sb_r = 8;
  bool sb_on = false;
  auto load_b_stream = [&]() {
    sb_on = p.lora && n_items <= WK && wk < n_items;  // uniform
    const int it = items[min(wk, 2 * ROWS - 1)];
    const int row = it & 255;
    sb_it = sb_on ? it : 0;
    sb_r = sb_on ? rowrk[row] : 8;
    sb_a = sb_on ? rowad[row] : -1;
    const uint64_t bp = sb_on ? rowbp[row] : reinterpret_cast<uint64_t>(p.x);
    const int j = ((sb_it >> 8) & 1) * 32 + 8 * g;
    const int r8 = rank_pad(sb_r);
    const int jc = min(j, r8 - 8);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int nl = wc * CT * 16 + ct * 16 + li;
      const uint64_t a_b = bp + 2ull * (uint64_t)((long)(n_tile0 + nl) * r8 + jc);
      const uint64_t a_d = reinterpret_cast<uint64_t>(p.x) + 16ull * (uint64_t)ct;
      sb[ct] = ldg16(reinterpret_cast<const void*>(sb_on ? a_b : a_d));
    }
  };

  if (STREAM) {
    // Rounds of SD steps, at least two.  Every round but the last consumes its SD slots
    // and refills them (past the wave's last step a refill reloads that step, and its
    // consumption is skipped); the last round only consumes.  The loads a round issues
    // never depend on a branch, so every path holds the slots' loads in the same order
    // and the compiler's waits for slot d count only the loads issued before it (a
    // conditional round or an early exit would make it wait for all of them).
    const int nround = max((nmy + SD - 1) / SD, 2);
    auto s_round = [&](int r) {
#pragma unroll
      for (int d = 0; d < SD; ++d) {
        if (r * SD + d < nmy) s_consume(d);
        s_issue(d, (r + 1) * SD + d);
      }
    };
    s_round(0);
    // the adapters of the rows are known by now: the up-projection metadata, so that the
    // t gather can go out before the last round
    if (p.lora) {
      prepare_epilogue();
      __syncthreads();
      read_meta();
    }
    int r = 1;
    for (; r + 1 < nround; ++r) s_round(r);
    load_t_stream();
    load_b_stream();
#pragma unroll
    for (int d = 0; d < SD; ++d)
      if (r * SD + d < nmy) s_consume(d);
  }
  if (!STREAM) {
    // Rounds of NBUF chunks, at least two: every round but the last refills each buffer with
    // the chunk NBUF ahead (past the last chunk: a chunk again, never multiplied), the last
    // round only multiplies.  As in the stream, no load depends on a branch, so the waits
    // for a chunk's loads leave the later chunks' loads in flight.  x of chunk c + 1 goes
    // into its LDS buffer while chunk c is multiplied from the other one, so each chunk
    // takes one barrier; the x registers it frees are refilled with chunk c + 3.  Measured:
    // staging and refilling x ahead of the chunk's MFMAs, prefill 149.7 -> 146.3 us;
    // with the refill after them, 156.2 us.
    const int nround = max((nchunks + NBUF - 1) / NBUF, 2);
    stage_x(0);
    __syncthreads();
    load_x(0, NBUF);
    auto c_round = [&](int r, bool refill) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int c = r * NBUF + u;
        if (refill) {
          // x of c + 1 is staged and its registers refilled before the MFMAs of c go out:
          // both are independent of them (with fewer than three chunks the first round
          // already passes the last one)
          stage_x(1 - u);
          load_x(1 - u, c + NBUF + 1);
          if (c < nchunks) mma_chunk(u, c);
          load_w(u, c + NBUF);
        } else {
          if (c < nchunks) mma_chunk(u, c);
          if (u + 1 < NBUF) stage_x(1 - u);
        }
        __syncthreads();
        if (c == 0 && p.lora) {
          prepare_epilogue();
          __syncthreads();
        }
      }
    };
    int r = 0;
    for (; r + 1 < nround; ++r) c_round(r, true);
    c_round(r, false);
  }
  // adapter sums go straight into the (already scaled) accumulator of the wave that
  // multiplies the item; with k-waves the waves' parts are summed afterwards
  auto lacc = [&](int tt, int ct) -> v4f& { return acc[tt][ct]; };
  // one bf16 MFMA per item, token tile and column tile; B operands from the staged slice
  // (lane (li, g): B_a^T[n][j .. j+7], j = 32*block + 8g, zero for j >= r_a).  The item
  // descriptors of 64 items at a time sit one per lane and are read with readlane, and the
  // adapters of the lane's own rows are kept in registers, so an item issues its operand
  // reads without a chain of dependent LDS loads.
  int myad[TT];
  auto consume = [&](int it, int off, int a, int r) {  // wave-uniform descriptor
    const int jb = (it >> 8) & 1, mask = (it >> 9) & 255;
    const int j = jb * 32 + 8 * g;  // <= 56
    const bool valid = j < r;
    const int r8 = rank_pad(r);
    const int jc = min(j, r8 - 8);
    uint4 bop[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int nl = wc * CT * 16 + ct * 16 + li;
      const uint4 bv = *reinterpret_cast<const uint4*>(stg + off + (nl * r8 + jc) * 2);
      bop[ct] = keep_bf16(bv, r - j);  // zero past the rank (padding) and for j >= r
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (!((mask >> tt) & 1)) continue;  // uniform: adapter absent from this token tile
      const uint4 tv = *reinterpret_cast<const uint4*>(tbuf + (tt * 16 + li) * TSTR + j);
      const uint4 aop = (valid && myad[tt] == a) ? tv : zero4();
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) lacc(tt, ct) = mfma_bf16_16x16x32(aop, bop[ct], lacc(tt, ct));
    }
  };
  auto put = [&](int i, int j, float v) {  // t of row i, rank j: staged (scaled, bf16) and the caller's t
    tbuf[i * TSTR + j] = (uint16_t)f32_to_bf16_rne(v * rowsc[i]);
    if (p.t_out && cb == 0 && j < p.r_lim) p.t_out[(long)(row0 + i) * p.r_lim + j] = v;
  };
  if constexpr (TT != 1) load_chan_s();
  // ---- up-projection loads of the chunked path go out as soon as the main loop ends
  // B operands of the 128-row tiles straight into registers; the others stage B slices in LDS
  constexpr bool RB = !STREAM && TT >= 8;
  if (!STREAM && p.lora) {
    read_meta();
    if (!RB && n_batch > 0) stage_b(0);
    load_t(0);
  } else if (STREAM && p.lora) {
    if (n_batch > 0 && n_items > WK) stage_b(0);
    if (!p.t_tag) load_t(0);
  }

  // a rank outside [1, r_max] in this tile: bit 1 of the status word
  if (p.lora && tid == 0 && meta[3]) or_agent(p.ctrl + CTRL_STATUS, 2);
  // publish the launch epoch only now: waiting for it earlier would stall wave 0
  *started = wg_epoch_publish(p.ctrl, e, lds_epoch);
  __syncthreads();
  const uint32_t tag = (uint32_t)(*lds_epoch) + 1u;

  // ---- epilogue: channel scale (of this K-split's sum: the splits are added scaled); with
  //      k-waves every wave scales its own part, and the parts are summed after the adapter
  //      terms are added (one LDS reduction for both).  It comes after the t gather, so that
  //      the accumulators stay untouched (in AGPRs) while the gather holds its registers.
  auto scale_acc = [&]() {
    if (FMT == LORA_W_FP8_E4M3) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[tt][ct] *= chan_s[ct];
      }
    }
  };
  if (!p.lora) scale_acc();

  // ---- epilogue: adapter up-projection (this K-split's share of the adapters)
  if (p.lora) {
    // (4) t of the rows this split needs -> LDS as bf16 pre-scaled by s_a (zero beyond the
    //     row's rank); the other rows of tbuf are never selected
#pragma unroll
    for (int ph = 0; ph < EPI_PH; ++ph) {
      if (ph > 0) load_t(ph);
#pragma unroll
      for (int m = 0; m < EPI_TH; ++m) tinf[m] |= rowrk[trow(m)] << 16;  // the rows' ranks, read together
      auto trk = [&](int m) { return tinf[m] >> 16; };
      if (tpack) {
        static_assert(EPI_PH == 1 && EPI_TH % 2 == 0, "pairs: one gather batch");
#pragma unroll
        for (int m = 0; m < EPI_TH / 2; ++m) {
          if (tid + 256 * m >= (nel >> 1)) continue;
          const int i = trow(m), j = 2 * tcol(m);
          uint32_t w2 = 0u;
          if (j < trk(m))
            w2 = (uint32_t)wait_tag(p.t_tag + (long)(row0 + i) * (p.r_max >> 1) + (j >> 1), traw[m][0], tag, p.ctrl,
                                    p.spin_limit);
          *reinterpret_cast<uint32_t*>(tbuf + i * TSTR + j) = w2;
        }
      } else if (p.t_tag) {
#pragma unroll
        for (int m = 0; m < EPI_TH; ++m) {
          if (tid + 256 * (ph * EPI_TH + m) >= nel) continue;
          const int i = trow(m), j = tcol(m);
          const long addr = (long)(row0 + i) * p.r_max + j;
          float v = 0.f;
#pragma unroll
          for (int k2 = 0; k2 < KP; ++k2) {
            if (j < trk(m) && k2 < p.t_kparts) {
              const uint64_t w =
                  wait_tag(p.t_tag + (long)k2 * p.T * p.r_max + addr, traw[m][k2], tag, p.ctrl, p.spin_limit);
              v += __uint_as_float((uint32_t)w);
            }
          }
          put(i, j, v);
        }
      } else {
#pragma unroll
        for (int m = 0; m < EPI_TH; ++m) {
          if (tid + 256 * (ph * EPI_TH + m) >= nel) continue;
          put(trow(m), tcol(m), tcol(m) < trk(m) ? tpl[m] : 0.f);
        }
      }
    }
    scale_acc();
    // (5) the stream's items with their B operands in registers ...
    if (STREAM && n_items <= WK) {
      __syncthreads();  // the staged t
      if (sb_on) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) myad[tt] = rowad[tt * 16 + li];
        const int jb = (sb_it >> 8) & 1, mask = (sb_it >> 9) & 255;
        const int j = jb * 32 + 8 * g;
        const bool valid = j < sb_r;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (!((mask >> tt) & 1)) continue;
          const uint4 tv = *reinterpret_cast<const uint4*>(tbuf + (tt * 16 + li) * TSTR + j);
          const uint4 aop = (valid && myad[tt] == sb_a) ? tv : zero4();
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            lacc(tt, ct) = mfma_bf16_16x16x32(aop, keep_bf16(sb[ct], sb_r - j), lacc(tt, ct));
        }
      }
      __syncthreads();  // the area of the k-wave sums lies over the staged t
    }
    // ... the 128-row tiles' items with their B operands straight from memory in registers,
    //     IB items at a time (a lane loads exactly its operand: 16 bytes of B_a^T per column
    //     tile).  Staging the slices in LDS took a memory round trip per batch of slices:
    //     down-projection 112.5 -> 103.7 us per step this way; the 64-row gate-up tiles
    //     (about 20 rank-16 adapters each) stay faster with the LDS slices (45.4 against 46.3) ...
    if constexpr (RB) {
      __syncthreads();  // the staged t
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) myad[tt] = rowad[tt * 16 + li];
      constexpr int IB = (CT >= 4) ? 2 : 8;
      for (int i0 = 0; i0 < n_items; i0 += 64) {
        const int iq = min(i0 + lane, n_items - 1);
        const int it_l = items[iq];
        const int row_l = it_l & 255;
        const int a_l = rowad[row_l], r_l = rowrk[row_l];
        const uint64_t bp_l = rowbp[row_l];
        const int n_here = min(64, n_items - i0);
        for (int q0 = 0; q0 < n_here; q0 += IB) {
          // IB items' loads on every path (past the end: the last item again, not used)
          uint4 bop[IB][CT];
          int itq[IB], aq[IB], rq[IB];
#pragma unroll
          for (int u = 0; u < IB; ++u) {
            const int q = min(q0 + u, n_here - 1);
            itq[u] = __builtin_amdgcn_readlane(it_l, q);
            aq[u] = __builtin_amdgcn_readlane(a_l, q);
            rq[u] = __builtin_amdgcn_readlane(r_l, q);
            const uint64_t bpu =
                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bp_l >> 32), q) << 32) |
                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bp_l, q);
            const int r8 = rank_pad(rq[u]);
            const int jc = min(((itq[u] >> 8) & 1) * 32 + 8 * g, r8 - 8);
            const uint16_t* bsrc = reinterpret_cast<const uint16_t*>(bpu);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              bop[u][ct] = ldg16(bsrc + (long)(n_tile0 + wc * CT * 16 + ct * 16 + li) * r8 + jc);
          }
#pragma unroll
          for (int u = 0; u < IB; ++u) {
            if (q0 + u >= n_here) continue;  // uniform
            const int mask = (itq[u] >> 9) & 255;
            const int j = ((itq[u] >> 8) & 1) * 32 + 8 * g;
            const bool valid = j < rq[u];
            if (rq[u] & 7) {  // uniform: a rank that is not a multiple of 8 has padding to mask
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) bop[u][ct] = keep_bf16(bop[u][ct], rq[u] - j);
            }
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) {
              if (!((mask >> tt) & 1)) continue;  // uniform: adapter absent from this token tile
              const uint4 tv = *reinterpret_cast<const uint4*>(tbuf + (tt * 16 + li) * TSTR + j);
              const uint4 aop = (valid && myad[tt] == aq[u]) ? tv : zero4();
#pragma unroll
              for (int ct = 0; ct < CT; ++ct)
                lacc(tt, ct) = mfma_bf16_16x16x32(aop, valid ? bop[u][ct] : zero4(), lacc(tt, ct));
            }
          }
        }
      }
    }
    // ... otherwise per batch: wait for this wave's copies, then every wave multiplies its
    //     items (the waves sharing columns split them: item i goes to wave i % WK)
    for (int b = 0; b < ((RB || (STREAM && n_items <= WK)) ? 0 : n_batch); ++b) {
      if (b > 0) stage_b(b);
      wait_stores();  // all of this wave's memory operations, the LDS copies included
      __syncthreads();
      if (b == 0) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) myad[tt] = rowad[tt * 16 + li];
      }
      // this wave's items wk, wk + WK, ...: descriptors of 64 of them per lane load
      for (int i0 = wk; i0 < n_items; i0 += 64 * WK) {
        const int iq = min(i0 + WK * lane, n_items - 1);
        const int it_l = items[iq], off_l = ioff[iq];
        const int row_l = it_l & 255;
        const int a_l = rowad[row_l], r_l = rowrk[row_l];
        const int n_here = min(64, (n_items - i0 + WK - 1) / WK);
        for (int q = 0; q < n_here; ++q) {
          const int it = __builtin_amdgcn_readlane(it_l, q);
          if ((it >> 17) != b) continue;  // uniform
          consume(it, __builtin_amdgcn_readlane(off_l, q), __builtin_amdgcn_readlane(a_l, q),
                  __builtin_amdgcn_readlane(r_l, q));
        }
      }
      __syncthreads();  // slots are refilled by the next batch
    }
  }

  // ---- sums of the WK k-waves (base and adapter terms), in wave order, end up in the waves
  //      with wk == 0 (the area lies over the staged t, which is no longer read)
  if (WK > 1) {
    float* red = reinterpret_cast<float*>(smem);
    if (wk > 0) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          *reinterpret_cast<v4f*>(red + ((((wk - 1) * WC + wc) * TT + tt) * CT + ct) * 256 + lane * 4) = acc[tt][ct];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < WK; ++w)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[tt][ct] +=
                *reinterpret_cast<const v4f*>(red + ((((w - 1) * WC + wc) * TT + tt) * CT + ct) * 256 + lane * 4);
    }
    __syncthreads();
  }

  // ---- K-split over workgroups: producers store their (scaled, adapter-including) sums
  //      and a flag, the last split adds them in split order
  if (p.ksplit > 1) {
    constexpr int PER_WAVE = TT * CT * 256;
    const long tile_base = (long)tile * p.ksplit;
    if (ks < p.ksplit - 1) {
      if (wk == 0) {
        float* mine = p.gpart + ((tile_base + ks) * WC + wc) * PER_WAVE;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            uint64_t* d = reinterpret_cast<uint64_t*>(mine + ((tt * CT + ct) * 64 + lane) * 4);
            st_agent_u64(d, ((uint64_t)__float_as_uint(acc[tt][ct][1]) << 32) | __float_as_uint(acc[tt][ct][0]));
            st_agent_u64(d + 1, ((uint64_t)__float_as_uint(acc[tt][ct][3]) << 32) | __float_as_uint(acc[tt][ct][2]));
          }
      }
      wait_stores();
      __syncthreads();
      if (tid == 0) set_agent(p.gflag + tile_base + ks, (int)tag);
      return;
    }
    // the reducer: wait for every producer of this tile
    for (int k2 = tid; k2 < p.ksplit - 1; k2 += 256) {
      int spins = 0;
      while ((uint32_t)ld_agent(p.gflag + tile_base + k2) != tag) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > p.spin_limit) {
          or_agent(p.ctrl + CTRL_STATUS, 1);
          break;
        }
      }
    }
    __syncthreads();
    if (wk == 0) {
      // the producers' sums are added to this split's in split order; all of one split's
      // loads go out together (one memory round trip per split)
      for (int k2 = 0; k2 < p.ksplit - 1; ++k2) {
        const uint64_t* src =
            reinterpret_cast<const uint64_t*>(p.gpart + ((tile_base + k2) * WC + wc) * PER_WAVE) + lane * 2;
        uint64_t u[TT][CT][2];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            u[tt][ct][0] = ld_agent_u64(src + (tt * CT + ct) * 128);
            u[tt][ct][1] = ld_agent_u64(src + (tt * CT + ct) * 128 + 1);
          }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            acc[tt][ct][0] += __uint_as_float((uint32_t)u[tt][ct][0]);
            acc[tt][ct][1] += __uint_as_float((uint32_t)(u[tt][ct][0] >> 32));
            acc[tt][ct][2] += __uint_as_float((uint32_t)u[tt][ct][1]);
            acc[tt][ct][3] += __uint_as_float((uint32_t)(u[tt][ct][1] >> 32));
          }
      }
    }
  }

  // ---- store bf16 (round to nearest even)
  if constexpr (STREAM) {
    if (wk == 0) {
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
  } else {
    // through LDS (the B staging area, free by now): a lane's values (four rows of one
    // channel per 16x16 block) go in as bf16, then every thread stores 16 contiguous bytes
    // of a row.  A 16-byte pad per row puts the four rows a lane group writes on different
    // banks, where the tile then still fits the 16-bit offsets of the LDS writes.
    constexpr int RS = (ROWS * (WN * 2 + 16) <= 65536) ? WN * 2 + 16 : WN * 2;
    static_assert(WK == 1 && ROWS * RS <= BST, "output tile in the B staging area");
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        char* dst = stg + (tt * 16 + 4 * g) * RS + (wc * CT * 16 + ct * 16 + li) * 2;
        const uint32_t p01 = bf16x2_rne(acc[tt][ct][0], acc[tt][ct][1]);
        const uint32_t p23 = bf16x2_rne(acc[tt][ct][2], acc[tt][ct][3]);
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)p01;
        *reinterpret_cast<uint16_t*>(dst + RS) = (uint16_t)(p01 >> 16);
        *reinterpret_cast<uint16_t*>(dst + 2 * RS) = (uint16_t)p23;
        *reinterpret_cast<uint16_t*>(dst + 3 * RS) = (uint16_t)(p23 >> 16);
      }
    __syncthreads();
    constexpr int CPR = WN / 8;  // 16-byte pieces per row
    static_assert((ROWS * CPR) % 256 == 0, "output pieces split evenly over the threads");
    constexpr int RPP = 256 / CPR;  // rows per pass of the workgroup
    const int c8 = tid % CPR, r0 = tid / CPR;
    const char* src = stg + r0 * RS + c8 * 16;
    uint16_t* dst = p.y + (long)(row0 + r0) * p.N + n_tile0 + c8 * 8;
    const long step = (long)RPP * p.N;
    const int rows_left = p.T - row0 - r0;
#pragma unroll 4
    for (int i = 0; i < ROWS / RPP; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + i * RPP * RS);
      if (i * RPP < rows_left) *reinterpret_cast<uint4*>(dst + i * step) = v;
    }
  }
}

// The down-projection role of a launch: workgroup b of the n_wg that take down-projection
// items (the lowest ids of a fused layer launch, or the first workgroups of the pre-pass
// launch).  ctrl == null: a launch without the launch epoch (the pre-pass), which writes t
// as plain fp32 and publishes nothing.
template <int TG, int JP, int U, bool PACK>
__device__ __forceinline__ void shrink_role(const ShrinkParams& sp, int b, int n_wg, char* smem, int* ctrl, int e,
                                            int* lds_epoch, int& started) {
  bool published = false;
  int n_valid = b + 1, stride = 1;
  int* pre = reinterpret_cast<int*>(smem + sp.compact_off);  // [n_ad + 1] item prefix
  if (sp.compact) {
    // Most (adapter, token block, rank group) items can be empty: token blocks past the
    // end of a segment, rank groups past an adapter's rank.  The workgroups take the
    // items that have work, k = b, b + n_shrink, ..., counted per adapter from the segment
    // lengths and ranks (prefix over the adapters, in LDS after the area the
    // down-projection uses), so that no workgroup holds a CU the GEMM needs for nothing.
    // Segments built in this launch are waited for first (see shrink_item).
    const bool coh = sp.seg_wait != 0;
    if (coh) {
      started = wg_epoch_publish(ctrl, e, lds_epoch);
      published = true;
      __syncthreads();
      if (threadIdx.x == 0) {
        int spins = 0;
        while (ld_agent(ctrl + CTRL_SEGREADY) != *lds_epoch + 1) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > sp.spin_limit) {
            or_agent(ctrl + CTRL_STATUS, 1);
            break;
          }
        }
      }
      __syncthreads();
    }
    int* wsum = pre + sp.n_ad + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto count = [&](int a) {
      const int len = coh ? ld_agent(sp.seg_indptr + a + 1) - ld_agent(sp.seg_indptr + a)
                          : sp.seg_indptr[a + 1] - sp.seg_indptr[a];
      const int r = sp.ranks[a];
      const bool ok = r >= 1 && r <= sp.r_lim;
      const int nj = min(sp.n_jg, (r + 16 * JP - 1) / (16 * JP));
      return ok ? (len + sp.tblk - 1) / sp.tblk * nj * sp.kparts : 0;
    };
    const int per = (sp.n_ad + 255) / 256;
    const int lo = min(tid * per, sp.n_ad), hi = min(lo + per, sp.n_ad);
    int cnt = 0;
    for (int a = lo; a < hi; ++a) cnt += count(a);
    int inc = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(inc, off);
      if (lane >= off) inc += u;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int base = inc - cnt;
    for (int w = 0; w < wave; ++w) base += wsum[w];
    for (int a = lo; a < hi; ++a) {
      pre[a] = base;
      base += count(a);
    }
    if (tid == 255) pre[sp.n_ad] = base;
    __syncthreads();
    n_valid = __builtin_amdgcn_readfirstlane(pre[sp.n_ad]);
    stride = n_wg;
  }
  for (int k = b; k < n_valid; k += stride) {
    int item = k;
    if (sp.compact) {
      int lo_a = 0, hi_a = sp.n_ad;  // adapter a with pre[a] <= k < pre[a + 1]
      while (hi_a - lo_a > 1) {
        const int mid = (lo_a + hi_a) >> 1;
        if (__builtin_amdgcn_readfirstlane(pre[mid]) <= k) lo_a = mid; else hi_a = mid;
      }
      const int local = k - __builtin_amdgcn_readfirstlane(pre[lo_a]);
      const int nj = min(sp.n_jg, (sp.ranks[lo_a] + 16 * JP - 1) / (16 * JP));
      const int kp = local % sp.kparts, rest = local / sp.kparts;
      const int jg = rest % nj, tb = rest / nj;
      item = (tb < sp.n_tblk) ? ((lo_a * sp.n_tblk + tb) * sp.n_jg + jg) * sp.kparts + kp : -1;
    }
    if (item >= 0) shrink_item<TG, JP, U, PACK>(sp, item, smem, ctrl, e, lds_epoch, &started, published);
  }
  if (!published && ctrl) started = wg_epoch_publish(ctrl, e, lds_epoch);
}

// OCC: workgroups per CU the registers are budgeted for (2 for the 64-token prefill tile,
// so that one workgroup's epilogue and start-up latency overlap another's main loop, and
// for the one-tile stream, whose few down-projection workgroups then share CUs)
template <int FMT, int TT, int CT, int WC, int WK, bool XQ, int TG, int JP, int U, int OCC, bool A16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void k_layer(ShrinkParams sp,
                                                                                                GemmParams gp) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int lds_epoch;
  const int e = wg_epoch_load(gp.ctrl);
  const int nb = gp.seg_build ? 1 : 0;
  const int b = blockIdx.x - nb;
  int started = 0;
  if (b < 0) {
    // the batch's segments, built in this launch (workgroup 0): coherent stores, then
    // the launch's tag in the control block for down-projection workgroups that read them
    started = wg_epoch_publish(gp.ctrl, e, &lds_epoch);
    int* w = reinterpret_cast<int*>(smem);
    int* cnt = w + SEG_SCRATCH;
    int* ids_s = cnt + seg_cnt_words(gp.n_ad);
    int* pres = ids_s + (gp.T <= SEG_CACHE ? (gp.T + 3) & ~3 : 0);
    int* wcnt = pres + (gp.T <= SEG_CACHE ? min(gp.T, gp.n_ad) : 0);
    build_segments_wg<true, 256>(gp.ids, gp.T, gp.n_ad, gp.seg_build, gp.sorted_build, gp.ctrl + CTRL_SEGERR, cnt,
                                 ids_s, pres, wcnt, w, w + 16);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) set_agent(gp.ctrl + CTRL_SEGREADY, e + 1);
  } else if (b < gp.n_shrink) {
    shrink_role<TG, JP, U, TT != 1>(sp, b, gp.n_shrink, smem, gp.ctrl, e, &lds_epoch, started);
  } else {
    // K-parts of t: the single-tile decode down-projection splits K
    constexpr int KPT = (TT == 1) ? 4 : 1;
    gemm_item<FMT, TT, CT, WC, WK, XQ, KPT, OCC, A16>(gp, b - gp.n_shrink, smem, e, &lds_epoch, &started);
  }
  wg_epoch_end(gp.ctrl, e, started);
}

// ======================================================================================
// Pre-pass of a long batch whose segments are built: the MXFP8 quantisation of x and the
// adapter down-projection in one pass over x.  Workgroup b takes the 16 positions
// [16b, 16b + 16) of the sorted token order for the down-projection and the 16 rows
// [16b, 16b + 16) of x for the quantisation: the same rows where segments are runs of
// consecutive tokens (a prefill batch), so each row of x is then read from memory once for
// both.  The four waves split K in quarters.  Per 64-wide k-step lane (i, g) holds
// x[row i][k + 16g .. k + 16g + 15]: the operands of two bf16 MFMAs (rows x 32 k each) and
// half of one of the row's MX blocks (the other half in lane i + 16(g ^ 1)).  Each adapter
// present among the
// 16 positions is one pass over the quarter: t[row][j] = sum_k x[row][k] A_a^T[j][k] on bf16
// MFMA 16x16x32 for the ranks of a, with the rows of other adapters masked to zero (a tile
// of a prefill batch holds one adapter, two where a segment ends; the first pass also
// quantises).  The quarters' sums meet in LDS in wave order, so t is deterministic, and go
// out as plain fp32 for the GEMM epilogue.  The down-projection thus still runs first, on
// the bf16 x, fused with the quantisation the GEMM needs anyway, and holds no GEMM CU.
// ======================================================================================
constexpr int PREP_U = 2;       // k-steps of 64 in flight per wave
constexpr int PREP_RS = 128 + 16;  // LDS row stride (bytes) of a wave's x slot: 16 rows x 64 bf16
// One pass of a wave over its part of K: quantise (QUANT) and/or add x A_a^T for NJT rank
// tiles.  The number of loads per step is a compile-time constant and no load or store sits
// behind a branch, so the compiler's waits for step u leave the later steps' loads in
// flight.
//  - QUANT: the quantisation's rows p0 .. p0 + 15 are loaded row-contiguously, lane l taking
//    16 bytes of row 8 i + l / 8 at piece l % 8 of the step (one load covers 8 whole
//    128-byte lines); the quantiser works on those pieces (a block is a quad of lanes).
//    Without SEP the same rows are the down-projection's, and their MFMA operand layout
//    comes back through the wave's LDS slot.
//  - SEP: the down-projection's rows (which differ from the quantisation's) are loaded in
//    operand layout, lane (i, g) taking row i at 16 g .. 16 g + 15.
//  - neither: the down-projection's rows p0 .. p0 + 15 loaded row-contiguously and relayed,
//    with no quantisation (the backward's u = dY B_a^T).
//  - PRE: the contiguous rows' first PREP_U k-steps were loaded by the caller (xpre), ahead of
//    the adapter look-ups the other loads depend on.
template <bool QUANT, bool SEP, int NJT, bool PK = false, bool PRE = false>
__device__ __forceinline__ void prep_pass(uint8_t* __restrict__ xq, uint8_t* __restrict__ xsc, int K, int T, int p0,
                                          const uint16_t* x, const uint16_t* xrow_s, char* slot, bool s_mine,
                                          const uint16_t* arow0, int r, int kb, int nst, v4f (&acc)[4],
                                          const uint4 (*xpre)[2] = nullptr) {
  constexpr int U = PREP_U;
  constexpr bool RELAY = !SEP && NJT > 0;  // operands through the LDS slot
  constexpr bool CONTIG = QUANT || RELAY;  // rows p0 .. p0 + 15 loaded row-contiguously
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  if (nst <= 0) return;
  // A_a in operand order (tiles past r_a's last read that tile and are masked at the output;
  // without an adapter, r == 0, the loads read x as a stand-in and feed nothing)
  const uint16_t* arow[NJT > 0 ? NJT : 1];
  const int nat = a_tiles(r);
#pragma unroll
  for (int jt = 0; jt < NJT; ++jt) arow[jt] = arow0 + a_tile_off(r > 0 ? min(jt, nat - 1) : 0, 0, 0, K) + 8 * lane;
  // rows of the contiguous loads (clamped: lanes past the last row repeat row T - 1 and store
  // the same bytes again) and of the operand-layout loads
  const int crow0 = min(p0 + (lane >> 3), T - 1), crow1 = min(p0 + 8 + (lane >> 3), T - 1);
  const uint16_t* xc0 = x + (long)crow0 * K + 8 * (lane & 7);
  const uint16_t* xc1 = x + (long)crow1 * K + 8 * (lane & 7);
  uint4 xr[U][2], xs[U][2], ar[U][NJT > 0 ? NJT : 1][2];
  auto issue = [&](int u, int st, bool contig) {  // the clamped step is always valid
    const int k = kb + min(st, nst - 1) * 64;
    if (contig) {
      xr[u][0] = ldg16(xc0 + k);
      xr[u][1] = ldg16(xc1 + k);
    }
    if (SEP && NJT > 0) {
      xs[u][0] = ldg16(xrow_s + k);
      xs[u][1] = ldg16(xrow_s + k + 8);
    }
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      ar[u][jt][0] = ldg16(arow[jt] + a_tile_off(0, k >> 6, 0, K));
      ar[u][jt][1] = ldg16(arow[jt] + a_tile_off(0, k >> 6, 1, K));
    }
  };
  auto consume = [&](int u, int st) {
    const int k = kb + st * 64;
    uint4 xv[2] = {zero4(), zero4()};
    if (CONTIG) {
      // a block is 32 values = the pieces of a quad of lanes; all four lanes store its code
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (QUANT) {
          uint32_t mx = absmax8_bits(xr[u][i]);
          mx = max(mx, quad_swap1(mx));
          mx = max(mx, quad_swap2(mx));
          const uint32_t code = mx_code_from_bits(mx);
          const int row = i ? crow1 : crow0;
          const int kk = k + 8 * (lane & 7);
          if (PK) {
            *reinterpret_cast<uint2*>(xq + pf_xq_off(row, kk, K >> 7)) = mx_piece_quant(xr[u][i], code);
            xsc[pf_xsc_off(row, kk >> 5, K >> 7)] = (uint8_t)code;
          } else {
            *reinterpret_cast<uint2*>(xq + (long)row * K + kk) = mx_piece_quant(xr[u][i], code);
            xsc[(long)row * (K / 32) + (kk >> 5)] = (uint8_t)code;
          }
        }
        if (RELAY) *reinterpret_cast<uint4*>(slot + PREP_RS * (8 * i + (lane >> 3)) + 16 * (lane & 7)) = xr[u][i];
      }
    }
    if (RELAY) {
      xv[0] = *reinterpret_cast<const uint4*>(slot + PREP_RS * li + 32 * g);
      xv[1] = *reinterpret_cast<const uint4*>(slot + PREP_RS * li + 32 * g + 16);
    } else if (SEP && NJT > 0) {
      xv[0] = xs[u][0];
      xv[1] = xs[u][1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 xm = s_mine ? xv[h] : zero4();
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc[jt] = mfma_bf16_16x16x32(xm, ar[u][jt][h], acc[jt]);
    }
  };
  // Rounds of U steps: every round but the last consumes its U slots and refills them
  // (past the last step a refill loads that step again, never consumed); the last round only
  // consumes.
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (PRE) {
      xr[u][0] = xpre[u][0];
      xr[u][1] = xpre[u][1];
      issue(u, u, false);
    } else {
      issue(u, u, CONTIG);
    }
  }
  const int nround = (nst + U - 1) / U;
  for (int rd = 0; rd + 1 < nround; ++rd) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      consume(u, rd * U + u);
      issue(u, (rd + 1) * U + u, CONTIG);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if ((nround - 1) * U + u < nst) consume(u, (nround - 1) * U + u);
}

// NJT: rank tiles of 16 of the batch's largest rank (every adapter's pass runs them all;
// the ranks past an adapter's own read its row 0 and are masked at the output).  Q: the first
// pass also quantises x; without it the kernel is the down-projection alone (the backward's
// u = dY B_a^T, B_a in A_a's operand order), its passes relaying contiguous rows where the
// positions are consecutive tokens.
template <int NJT, bool Q, bool PK = false>
__global__ __launch_bounds__(256) void k_prep_rows(ShrinkParams sp, uint8_t* __restrict__ xq, uint8_t* __restrict__ xsc) {
  __shared__ __align__(16) float red[4][4][64][4];  // [wave][rank tile][lane][4]
  __shared__ __align__(16) char xslot[4][16 * PREP_RS];  // each wave's x relayout slot
  __shared__ int stok[16], sad[16];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15,
            g = lane >> 4;
  const int T = sp.T, K = sp.K;
  // Workgroups are dealt to the eight XCDs in turn; XCD x takes the x-th eighth of the
  // position blocks, a run of consecutive positions, so that the A_a of its one or two
  // segments stays in its L2 (in plain order every XCD would stream every adapter's A_a)
  const int nblk = gridDim.x, b = blockIdx.x;
  const int blk = (nblk % 8 == 0) ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int p0 = blk * 16;
  const int n_valid = sp.seg_indptr[sp.n_ad];  // positions of tokens with a valid adapter
  const int pos = p0 + li;
  const bool s_ok = pos < n_valid;
  const int tok_s = s_ok ? sp.sorted_tok[pos] : 0;
  const int a_s = s_ok ? sp.ids[tok_s] : -1;
  if (tid < 16) {
    stok[tid] = tok_s;
    sad[tid] = a_s;
  }
  // the down-projection's rows are the quantisation's rows (runs of consecutive tokens)
  const bool same = __ballot(s_ok && tok_s != p0 + li) == 0ull;
  // the wave's quarter of K, in steps of 64 (the last quarter may be shorter or empty)
  const int kqs = ((K >> 2) + 63) & ~63;
  const int kb = min(K, wave * kqs), nst = (min(K, kb + kqs) - kb) >> 6;
  const uint16_t* xrow_s = sp.x + (long)tok_s * K + 16 * g;
  v4f acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) acc[jt] = v4f{0.f, 0.f, 0.f, 0.f};
  // one pass per adapter present (the first also quantises); lanes 0..15 stand for the rows
  unsigned long long todo = __ballot(li == lane && s_ok);
  bool first = true;
  do {
    int a = -1, r = 0;
    if (todo) {
      const int lead = __ffsll((long long)todo) - 1;
      a = __builtin_amdgcn_readlane(a_s, lead);
      todo &= ~__ballot(li == lane && s_ok && a_s == a);
      r = sp.ranks[a];
      if (r < 1 || r > sp.r_lim) r = 0;  // reported by the GEMM epilogue; no term
    }
    // no adapter (or an invalid rank): the rows read x's row 0 and the products are masked
    const bool mine = a >= 0 && r > 0 && s_ok && a_s == a;
    const uint16_t* arow0 = reinterpret_cast<const uint16_t*>(r > 0 ? sp.A_ptrs[a] : (uint64_t)sp.x);
    char* slot = xslot[wave];
    if (!Q) {
      if (r > 0 && same)
        prep_pass<false, false, NJT>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc);
      else if (r > 0)
        prep_pass<false, true, NJT>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc);
    } else if (first && same) {
      prep_pass<true, false, NJT, PK>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc);
    } else if (first) {
      prep_pass<true, true, NJT, PK>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc);
    } else if (r > 0) {
      prep_pass<false, true, NJT>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc);
    }
    first = false;
  } while (todo);
  // the quarters' sums in wave order; wave w writes rank tile w of t (plain fp32, zero past
  // the row's rank up to r_max)
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) *reinterpret_cast<v4f*>(&red[wave][jt][lane][0]) = acc[jt];
  __syncthreads();
  if (!sp.t_out) return;
  v4f sum = *reinterpret_cast<const v4f*>(&red[0][wave][lane][0]);
#pragma unroll
  for (int w = 1; w < 4; ++w) sum += *reinterpret_cast<const v4f*>(&red[w][wave][lane][0]);
  const int j = wave * 16 + li;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    if (p0 + row >= n_valid || j >= sp.r_lim) continue;
    const int a = sad[row];
    const int r = sp.ranks[a];
    if (r < 1 || r > sp.r_lim) continue;
    sp.t_out[(long)stok[row] * sp.r_lim + j] = (j < r) ? sum[v] : 0.f;
  }
}

// The pre-pass of the long-batch GEMM k_gemm_pf: the MXFP8 quantisation of x into that GEMM's
// operand order and the down-projection t = x A_a, with K in PF_KP parts across workgroups.
// A workgroup takes 64 consecutive positions of the sorted order and one K-part; wave w takes
// positions 16 w .. 16 w + 15 (and quantises token rows p0 .. p0 + 15 over the part), so the
// four waves read the same A_a slice at about the same time and share it through the cache,
// where one workgroup per 16 positions read every adapter's whole A_a per 16 positions.  Each
// wave writes its partial sums straight to t_part [PF_KP][T][PF_TPS] (fp32, zero past the
// row's rank up to 16 NJT), which the GEMM's epilogue adds in part order.  Rows without a
// valid adapter or rank are not written (the epilogue reads no t for them).  Workgroups are
// dealt to the XCDs in turn; XCD x takes a contiguous run of (position block, part) pairs, so
// the A_a of its segments stays in its L2.
template <int NJT>
__global__ __launch_bounds__(256) void k_prep_pf(ShrinkParams sp, uint8_t* __restrict__ xq, uint8_t* __restrict__ xsc) {
  __shared__ __align__(16) char xslot[4][16 * PREP_RS];  // each wave's x relayout slot
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15,
            g = lane >> 4;
  const int T = sp.T, K = sp.K;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int L = (nblk % 8 == 0) ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int kp = L % PF_KP, p0 = (L / PF_KP) * 64 + 16 * wave;
  if (p0 >= T) return;  // wave-uniform: no rows (the kernel has no barrier)
  const int kpl = K / PF_KP, kb = kp * kpl, nst = kpl >> 6;
  // the first k-steps of the rows this wave quantises go out first: they do not depend on
  // the adapter look-ups below (the same clamped rows and steps as prep_pass's loads)
  uint4 xpre[PREP_U][2];
  {
    const uint16_t* xc0 = sp.x + (long)min(p0 + (lane >> 3), T - 1) * K + 8 * (lane & 7);
    const uint16_t* xc1 = sp.x + (long)min(p0 + 8 + (lane >> 3), T - 1) * K + 8 * (lane & 7);
#pragma unroll
    for (int u = 0; u < PREP_U; ++u) {
      const int k = kb + min(u, nst - 1) * 64;
      xpre[u][0] = ldg16(xc0 + k);
      xpre[u][1] = ldg16(xc1 + k);
    }
  }
  // the position's token and adapter are loaded beside the count of valid positions (at a
  // clamped index; used only below that count)
  const int n_valid = sp.seg_indptr[sp.n_ad];  // positions of tokens with a valid adapter
  const int pos = p0 + li;
  const int tok_c = sp.sorted_tok[min(pos, T - 1)];
  const int a_c = sp.ids[min(max(tok_c, 0), T - 1)];
  const bool s_ok = pos < n_valid;
  const int tok_s = s_ok ? tok_c : 0;
  const int a_s = s_ok ? a_c : -1;
  const bool same = __ballot(s_ok && tok_s != pos) == 0ull;
  const uint16_t* xrow_s = sp.x + (long)tok_s * K + 16 * g;
  v4f acc[4];
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) acc[jt] = v4f{0.f, 0.f, 0.f, 0.f};
  // one pass per adapter present among the wave's rows (the first also quantises)
  unsigned long long todo = __ballot(li == lane && s_ok);
  bool first = true;
  char* slot = xslot[wave];
  do {
    int a = -1, r = 0;
    if (todo) {
      const int lead = __ffsll((long long)todo) - 1;
      a = __builtin_amdgcn_readlane(a_s, lead);
      todo &= ~__ballot(li == lane && s_ok && a_s == a);
      r = sp.ranks[a];
      if (r < 1 || r > sp.r_lim) r = 0;  // reported by the GEMM epilogue; no term
    }
    const bool mine = a >= 0 && r > 0 && s_ok && a_s == a;
    const uint16_t* arow0 = reinterpret_cast<const uint16_t*>(r > 0 ? sp.A_ptrs[a] : (uint64_t)sp.x);
    if (first && same) {
      prep_pass<true, false, NJT, true, true>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc, xpre);
    } else if (first) {
      prep_pass<true, true, NJT, true, true>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc, xpre);
    } else if (r > 0) {
      prep_pass<false, true, NJT>(xq, xsc, K, T, p0, sp.x, xrow_s, slot, mine, arow0, r, kb, nst, acc);
    }
    first = false;
  } while (todo);
  // lane (i, g) holds rank 16 jt + i of rows 4 g + v
  float* tp = sp.t_part + (long)kp * T * PF_TPS;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * g + v;
    const int tok = __shfl(tok_s, row, 64), a = __shfl(a_s, row, 64);
    if (p0 + row >= n_valid) continue;
    const int r = sp.ranks[a];
    if (r < 1 || r > sp.r_lim) continue;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      const int j = 16 * jt + li;
      tp[(long)tok * PF_TPS + j] = (j < r) ? acc[jt][v] : 0.f;
    }
  }
}

// ======================================================================================
// The per-token merged-weight formulation, as an alternative to ablate against ("LoRA-Switch"
// abstract: each token's adapter is merged into the backbone weights for inference, the merges
// of all adapters fused in one kernel).  y[t] = bf16( x[t] . (W_d + s_a A_a B_a) ) with the
// merged weight formed in registers and never stored: workgroup = 16 output channels x 16
// tokens, the four waves splitting K in quarters.  Per 32-wide k-step lane (i, g) holds
// W'[n0 + i][k] for k in {k0 + 4g .. k0 + 4g + 3} and {k0 + 16 + 4g .. k0 + 16 + 4g + 3}:
// the delta A_a B_a comes from two bf16 MFMAs per 32 ranks (rows k, columns n: their output
// puts exactly those four k of column i in lane (i, g)), the base term from the W codes
// (FP8 times the channel scale, or MXFP4 times its block scale), and W' goes to bf16 as the
// A operand of the main MFMA, whose B operand reads x at the same k.  Each adapter present in
// the token tile is one pass (rows of other adapters masked); tokens without a valid adapter
// get a pass with the base weight alone.  W is read in its row-major form, A_a as A rows
// bf16 [K][rank_pad(r_a)], B_a as the packed B_a^T.
// ======================================================================================
struct MergedParams {
  const uint16_t* x;
  int T, K, N, fmt;
  const uint8_t* wq;       // row-major codes [N][K] (FP8) or [N][K/2] (MXFP4)
  const float* ws_fp8;     // [N]
  const uint8_t* ws_fp4;   // [N][K/32]
  const int* ids;
  const uint64_t* A_rows;  // per adapter: bf16 [K][rank_pad(r)]
  const uint64_t* B_ptrs;  // per adapter: bf16 [N][rank_pad(r)]
  const int* ranks;
  const float* scales;
  int n_ad, r_lim;
  uint16_t* y;
};

template <int FMT>
__global__ __launch_bounds__(256) void k_merged(MergedParams p) {
  __shared__ __align__(16) float red[4][64][4];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15,
            g = lane >> 4;
  const int K = p.K;
  const int n0 = blockIdx.x * 16, t0 = blockIdx.y * 16;
  const int n = n0 + li;
  // the lane's token (as the main MFMA's B operand: column li) and its adapter
  const int tok = min(t0 + li, p.T - 1);
  const bool tok_ok = t0 + li < p.T;
  int a_tok = tok_ok ? p.ids[tok] : -1;
  if (a_tok >= 0 && a_tok < p.n_ad) {
    const int r = p.ranks[a_tok];
    if (r < 1 || r > p.r_lim) a_tok = -2;  // no adapter term (the layer call reports it)
  } else if (tok_ok) {
    a_tok = -2;
  }
  const int kq = K >> 2, kb = wave * kq, nst = kq >> 5;  // the wave's quarter, steps of 32
  const float s_w = (FMT == LORA_W_FP8_E4M3) ? p.ws_fp8[n] : 1.f;
  const uint16_t* xrow = p.x + (long)tok * K + 4 * g;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  // passes: one per adapter present among lanes 0 .. 15, then one for tokens without one
  unsigned long long todo = __ballot(li == lane && a_tok >= 0);
  bool base_pass = __ballot(li == lane && a_tok == -2) != 0ull;
  while (todo || base_pass) {
    int a = -1, r = 0;
    if (todo) {
      a = __builtin_amdgcn_readlane(a_tok, __ffsll((long long)todo) - 1);
      todo &= ~__ballot(li == lane && a_tok == a);
      r = p.ranks[a];
    } else {
      base_pass = false;
    }
    const bool mine = (a >= 0) ? (a_tok == a) : (a_tok == -2);
    const int r8 = (a >= 0) ? rank_pad(r) : 8;
    const int nrb = (r8 + 31) >> 5;  // 32-rank blocks of the delta MFMAs
    const float s_a = (a >= 0) ? p.scales[a] : 0.f;
    // B_a^T of channel n, ranks 8g' .. 8g' + 7 per rank block (loop-invariant), masked past r
    uint4 bop[2] = {zero4(), zero4()};
    const uint16_t* arow = reinterpret_cast<const uint16_t*>(a >= 0 ? p.A_rows[a] : (uint64_t)p.x);
    if (a >= 0) {
      const uint16_t* bt = reinterpret_cast<const uint16_t*>(p.B_ptrs[a]) + (long)n * r8;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int j = 32 * rb + 8 * g;
        if (rb < nrb && j < r8) bop[rb] = keep_bf16(ldg16(bt + j), r - j);
      }
    }
    // two stages in flight: the loads of step st + 1 go out before step st is multiplied
    // (unconditional loads from clamped addresses; ranks past r_a are masked afterwards)
    struct Stage {
      uint32_t w[2];
      uint2 x0, x1;
      uint4 av[2][2];
    };
    // (without an adapter the stand-in rows are x's first eight values, stride 0)
    const int jc0 = min(8 * g, r8 - 8), jc1 = min(32 + 8 * g, r8 - 8), astr = (a >= 0) ? r8 : 0;
    auto load = [&](int st, Stage& S) {
      const int k0 = kb + min(st, nst - 1) * 32;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (FMT == LORA_W_FP8_E4M3)
          S.w[h] = *reinterpret_cast<const uint32_t*>(p.wq + (long)n * K + k0 + 16 * h + 4 * g);
        else
          S.w[h] = *reinterpret_cast<const uint16_t*>(p.wq + ((long)n * K + k0 + 16 * h + 4 * g) / 2);
        const uint16_t* ar = arow + (long)(k0 + 16 * h + li) * astr;
        S.av[h][0] = ldg16(ar + jc0);
        S.av[h][1] = ldg16(ar + jc1);
      }
      S.x0 = *reinterpret_cast<const uint2*>(xrow + k0);
      S.x1 = *reinterpret_cast<const uint2*>(xrow + k0 + 16);
    };
    auto compute = [&](const Stage& S, int st) {
      const int k0 = kb + st * 32;
      // delta^T tiles (rows k0 .. k0 + 15 and k0 + 16 .. k0 + 31, columns n0 .. n0 + 15)
      v4f d[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          if (rb < nrb) d[h] = mfma_bf16_16x16x32(keep_bf16(S.av[h][rb], r - (32 * rb + 8 * g)), bop[rb], d[h]);
      // base weight at the same k: W[n][k0 + 16h + 4g + v]
      float wv[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (FMT == LORA_W_FP8_E4M3) {
          const uint2 bf = fp8x4_to_bf16(S.w[h]);
          wv[h][0] = bf16_lo(bf.x); wv[h][1] = bf16_hi(bf.x); wv[h][2] = bf16_lo(bf.y); wv[h][3] = bf16_hi(bf.y);
        } else {
          const float sc = __uint_as_float((uint32_t)p.ws_fp4[(long)n * (K / 32) + (k0 >> 5)] << 23);
          const uint4 bf = fp4x8_to_bf16(S.w[h], sc);
          wv[h][0] = bf16_lo(bf.x); wv[h][1] = bf16_hi(bf.x); wv[h][2] = bf16_lo(bf.y); wv[h][3] = bf16_hi(bf.y);
        }
      }
      // merged weight to bf16 (the A operand: eight k of channel n for lane group g)
      uint32_t wm[4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 4; v += 2)
          wm[2 * h + v / 2] = bf16x2_rne(s_w * wv[h][v] + s_a * d[h][v], s_w * wv[h][v + 1] + s_a * d[h][v + 1]);
      // x of the lane's token at the same k (the B operand), other adapters' tokens masked
      const uint4 xv = mine ? make_uint4(S.x0.x, S.x0.y, S.x1.x, S.x1.y) : zero4();
      acc = mfma_bf16_16x16x32(make_uint4(wm[0], wm[1], wm[2], wm[3]), xv, acc);
    };
    Stage S0, S1;
    load(0, S0);
    for (int st = 0; st < nst; st += 2) {
      load(st + 1, S1);
      compute(S0, st);
      load(st + 2, S0);
      if (st + 1 < nst) compute(S1, st + 1);
    }
  }
  // the quarters' sums in wave order; lane (i, g) holds y[t0 + i][n0 + 4g + v]
  *reinterpret_cast<v4f*>(&red[wave][lane][0]) = acc;
  __syncthreads();
  if (wave == 0) {
    v4f sum = *reinterpret_cast<const v4f*>(&red[0][lane][0]);
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += *reinterpret_cast<const v4f*>(&red[w][lane][0]);
    if (tok_ok) {
#pragma unroll
      for (int v = 0; v < 4; ++v) p.y[(long)tok * p.N + n0 + 4 * g + v] = (uint16_t)f32_to_bf16_rne(sum[v]);
    }
  }
}

// ======================================================================================
// Launchers
// ======================================================================================
template <int TG, int JP, int U>
constexpr size_t shrink_smem() {
  return (size_t)4 * TG * JP * 256 * sizeof(float);
}

template <typename KernelT, typename... Args>
static hipError_t launch_kn(KernelT kern, int grid, int threads, size_t smem, hipStream_t stream, Args... args) {
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), smem, stream, args...);
  return hipGetLastError();
}
template <typename KernelT, typename... Args>
static hipError_t launch_k(KernelT kern, int grid, size_t smem, hipStream_t stream, Args... args) {
  return launch_kn(kern, grid, 256, smem, stream, args...);
}

template <int FMT, int TT, int CT, int WC, int WK, bool XQ, int TG, int JP, int U, int OCC, bool A16 = false>
static hipError_t launch_layer_t(const LayerPlan& pl, int grid, hipStream_t stream, const ShrinkParams& sp_in,
                                 const GemmParams& gp) {
  ShrinkParams sp = sp_in;
  sp.compact_off = (int)shrink_smem<TG, JP, U>();  // the block prefix lies after the down-projection's area
  const size_t sm = std::max(std::max((size_t)GemmSmem<TT, CT, WC, WK, OCC, A16>::BYTES,
                                      gp.n_shrink > 0 ? shrink_smem<TG, JP, U>() : (size_t)0),
                             std::max(gp.seg_build ? seg_lds_bytes(gp.T, gp.n_ad) : (size_t)0,
                                      sp.compact ? (size_t)sp.compact_off + 4 * (size_t)(sp.n_ad + 1) + 16 : (size_t)0));
  return launch_k(k_layer<FMT, TT, CT, WC, WK, XQ, TG, JP, U, OCC, A16>, grid, sm, stream, sp, gp);
}

// GEMM tile (TT, CT, WC, WK, XQ), down-projection shape (decode, cfg 0: one 16-rank tile,
// two-step prefetch; prefill, cfg 1: four token tiles, two rank tiles) and workgroups per CU
#define LORA_LAYER_CASE(TT_, CT_, WC_, WK_, XQ_, CFG_, TG_, JP_, U_, OCC_)                                \
  if (pl.TT == TT_ && pl.CT == CT_ && pl.WC == WC_ && pl.WK == WK_ && pl.XQ == XQ_ && pl.s_cfg == CFG_ && \
      (pl.occ == OCC_ || TT_ != 1))                                                                     \
    return launch_layer_t<FMT, TT_, CT_, WC_, WK_, XQ_, TG_, JP_, U_, OCC_>(pl, grid, stream, sp, gp);

template <int FMT>
static hipError_t launch_layer_f(const LayerPlan& pl, int grid, hipStream_t stream, const ShrinkParams& sp,
                                 const GemmParams& gp) {
  if (pl.a16) {  // 16-bit activations: the one-tile stream or 64 x 128 tiles, either down-projection shape
    if (pl.TT == 1 && pl.CT == 2 && pl.WC == 1 && pl.WK == 4 && !pl.XQ && pl.occ == 2) {
      if (pl.s_cfg == 0) return launch_layer_t<FMT, 1, 2, 1, 4, false, 1, 1, 2, 2, true>(pl, grid, stream, sp, gp);
      if (pl.s_cfg == 1) return launch_layer_t<FMT, 1, 2, 1, 4, false, 4, 2, 1, 2, true>(pl, grid, stream, sp, gp);
    }
    if (pl.TT == 4 && pl.CT == 2 && pl.WC == 4 && pl.WK == 1 && !pl.XQ && pl.occ == 1) {
      if (pl.s_cfg == 0) return launch_layer_t<FMT, 4, 2, 4, 1, false, 1, 1, 2, 1, true>(pl, grid, stream, sp, gp);
      if (pl.s_cfg == 1) return launch_layer_t<FMT, 4, 2, 4, 1, false, 4, 2, 1, 1, true>(pl, grid, stream, sp, gp);
    }
    return hipErrorInvalidValue;
  }
  LORA_LAYER_CASE(1, 2, 1, 4, false, 0, 1, 1, 2, 2)
  LORA_LAYER_CASE(4, 1, 4, 1, false, 0, 1, 1, 2, 1)
  LORA_LAYER_CASE(4, 2, 4, 1, false, 0, 1, 1, 2, 1)
  LORA_LAYER_CASE(4, 2, 4, 1, true, 0, 1, 1, 2, 1)
  LORA_LAYER_CASE(8, 1, 4, 1, true, 0, 1, 1, 2, 1)
  LORA_LAYER_CASE(8, 2, 4, 1, true, 0, 1, 1, 2, 1)
  LORA_LAYER_CASE(8, 1, 4, 1, true, 1, 4, 2, 1, 1)
  LORA_LAYER_CASE(8, 2, 4, 1, true, 1, 4, 2, 1, 1)
  LORA_LAYER_CASE(4, 2, 4, 1, true, 1, 4, 2, 1, 2)
  LORA_LAYER_CASE(8, 4, 4, 1, true, 1, 4, 2, 1, 1)
  return hipErrorInvalidValue;
}
#undef LORA_LAYER_CASE

hipError_t launch_layer(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp, const GemmParams& gp) {
  const int grid = (gp.seg_build ? 1 : 0) + gp.n_shrink + pl.n_gemm_wg;
  if (pl.fmt == LORA_W_FP8_E4M3) return launch_layer_f<LORA_W_FP8_E4M3>(pl, grid, stream, sp, gp);
  return launch_layer_f<LORA_W_MXFP4_E2M1>(pl, grid, stream, sp, gp);
}

hipError_t launch_shrink(const LayerPlan& pl, hipStream_t stream, const ShrinkParams& sp) {
  if (pl.s_cfg == 0) return launch_k(k_shrink<1, 4, 1>, pl.n_shrink_items, shrink_smem<1, 4, 1>(), stream, sp);
  if (pl.s_cfg == 1) return launch_k(k_shrink<4, 2, 1>, pl.n_shrink_items, shrink_smem<4, 2, 1>(), stream, sp);
  return hipErrorInvalidValue;
}

// compiled configurations of the standalone down-projection (tuning)
#define LORA_SHRINK_CFGS(X) \
  X(1, 1, 1) X(1, 1, 2) X(1, 2, 1) X(1, 2, 2) X(1, 4, 1) X(1, 4, 2) \
  X(2, 1, 1) X(2, 1, 2) X(2, 2, 1) X(2, 2, 2) X(2, 4, 1) X(2, 4, 2) \
  X(4, 1, 1) X(4, 1, 2) X(4, 2, 1) X(4, 2, 2) X(4, 4, 1) X(4, 4, 2)

hipError_t launch_shrink_cfg(int tg, int jp, int u, int grid, hipStream_t s, const ShrinkParams& sp) {
#define X(TG_, JP_, U_) \
  if (tg == TG_ && jp == JP_ && u == U_) return launch_k(k_shrink<TG_, JP_, U_>, grid, shrink_smem<TG_, JP_, U_>(), s, sp);
  LORA_SHRINK_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t shrink_cfg_attr(int tg, int jp, int u, int* regs, int* spill, int* lds) {
  hipFuncAttributes fa{};
  hipError_t e = hipErrorInvalidValue;
#define X(TG_, JP_, U_)                                                                       \
  if (tg == TG_ && jp == JP_ && u == U_) {                                                    \
    e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(k_shrink<TG_, JP_, U_>));   \
    *lds = (int)shrink_smem<TG_, JP_, U_>();                                                 \
  }
  LORA_SHRINK_CFGS(X)
#undef X
  if (e != hipSuccess) return e;
  *regs = fa.numRegs;
  *spill = (int)fa.localSizeBytes;
  return hipSuccess;
}
#undef LORA_SHRINK_CFGS

// compiled configurations of the wave-reduction down-projection: NT tokens, JP rank tiles,
// U k-steps per buffer
#define LORA_BGMV_CFGS(X) \
  X(1, 1, 1) X(1, 2, 1) X(1, 4, 1) X(2, 1, 1) X(2, 2, 1) X(2, 4, 1) X(4, 1, 1) X(4, 2, 1) X(4, 4, 1) \
  X(1, 1, 2) X(1, 2, 2) X(1, 4, 2)

hipError_t launch_shrink_bgmv(int nt, int jp, int u, int grid, hipStream_t s, const ShrinkParams& sp) {
#define X(NT_, JP_, U_) \
  if (nt == NT_ && jp == JP_ && u == U_) {                                                   \
    hipLaunchKernelGGL((k_shrink_bgmv<NT_, JP_, U_>), dim3(grid), dim3(256), 0, s, sp);      \
    return hipGetLastError();                                                                \
  }
  LORA_BGMV_CFGS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t shrink_bgmv_attr(int nt, int jp, int u, int* regs, int* spill, int* lds) {
  hipFuncAttributes fa{};
  hipError_t e = hipErrorInvalidValue;
#define X(NT_, JP_, U_)                                                                        \
  if (nt == NT_ && jp == JP_ && u == U_) {                                                     \
    e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(k_shrink_bgmv<NT_, JP_, U_>)); \
    *lds = 4 * NT_ * JP_ * 16 * 4;                                                             \
  }
  LORA_BGMV_CFGS(X)
#undef X
  if (e != hipSuccess) return e;
  *regs = fa.numRegs;
  *spill = (int)fa.localSizeBytes;
  return hipSuccess;
}
#undef LORA_BGMV_CFGS

hipError_t launch_build_segments(const int* ids, int T, int n_ad, int* seg, int* sorted, int* err, hipStream_t s) {
  return launch_kn(k_build_segments, 1, SEG_THREADS, seg_lds_bytes(T, n_ad), s, ids, T, n_ad, seg, sorted, err);
}

// ======================================================================================
// The 16-bit-activation GEMM of a long batch (FP8 W, N % 256 == 0; plain fp32 t from the
// down-projection launched before it, or the caller's): y = bf16(s_w (x . codes) + s_a t B_a)
// on bf16 MFMA.  A 64-token x
// 256-channel tile per workgroup, four waves of 64 x 64, two workgroups per CU (their
// barriers are independent, so one's loads, widening and waits overlap the other's MFMAs).
// Per 128-wide k-step the tile's bf16 x rows [64][128] are staged in LDS a step ahead, double
// buffered; each wave loads its four packed W tiles (2 KB of consecutive memory each) a step
// ahead into one of two alternating register sets, widens the codes exactly (one conversion
// per two codes) and issues 64 MFMAs: lane group g's 32 codes of a tile (k = 16 g .., 16 g + 8
// .., 64 + 16 g .., 72 + 16 g ..) are four operands, each paired with the x piece at the
// same k.  The loads are pinned at the top of the step.  Epilogue: the channel scale, then
// for each adapter present in the tile (in increasing id order) one bf16 MFMA per 32 ranks
// and block with s_a t rounded to bf16 (rows of other adapters zeroed) and B_a^T rows as the
// other operand, then bf16 stores through LDS.  Workgroups are dealt to the XCDs
// in turn; XCD x takes a contiguous run of tiles in row-block-major order (the column blocks
// of a row block share its x rows in L2).
// ======================================================================================
constexpr int GA_XRS = 256 + 16;      // LDS row stride of a staged step: 128 bf16 + 16 bytes
constexpr int GA_XBUF = 64 * GA_XRS;  // one staged k-step of the tile's 64 rows
constexpr int GA_ERS = 144;           // row stride of the epilogue's staging (64 bf16 + 16 bytes)

__global__ __launch_bounds__(256, 2) void k_gemm_a16(GemmParams p) {
  __shared__ __align__(16) uint8_t lds[2 * GA_XBUF];
  __shared__ int rid[64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, i = lane & 15, g = lane >> 4;
  const int K = p.K, N = p.N, T = p.T;
  const int n_tb = (T + 63) >> 6, n_cb = N >> 8;
  const int ntiles = n_tb * n_cb;
  int tile = blockIdx.x;
  if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
  const int tb = tile / n_cb, cb = tile % n_cb;
  const int t0 = 64 * tb, n0w = 256 * cb + 64 * w;
  const int NS = K >> 7;

  // staging: thread loads pieces P = tid + 256 m (m = 0..3), row P / 16 at 16 (P % 16) bytes
  const int prow = tid >> 4, ppart = tid & 15;
  const uint16_t* xrow[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) xrow[m] = p.x + (long)min(t0 + prow + 16 * m, T - 1) * K + 8 * ppart;
  const uint8_t* wrow[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) wrow[ct] = p.wq + (long)((n0w >> 4) + ct) * NS * 2048 + lane * 16;

  auto load_x = [&](uint4 (&d)[4], int st) {
#pragma unroll
    for (int m = 0; m < 4; ++m) d[m] = ldg16(xrow[m] + 128 * st);
  };
  auto load_w = [&](uint4 (&lo)[4], uint4 (&hi)[4], int st) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      lo[ct] = ldg16(wrow[ct] + (long)st * 2048);
      hi[ct] = ldg16(wrow[ct] + (long)st * 2048 + 1024);
    }
  };
  auto store_x = [&](const uint4 (&d)[4], int buf) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<uint4*>(lds + buf * GA_XBUF + (prow + 16 * m) * GA_XRS + 16 * ppart) = d[m];
  };

  uint4 xd[4], wl[2][4], wh[2][4];
  load_x(xd, 0);
  load_w(wl[0], wh[0], 0);
  store_x(xd, 0);
  __syncthreads();

  v4f acc[4][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[tt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  // one 128-wide step: register set C holds W of step it, set 1 - C receives step it + 1
  auto step = [&](int it, auto set) {
    constexpr int C = decltype(set)::value;
    const int nx = min(it + 1, NS - 1);  // the last step reloads itself: uniform code
    load_x(xd, nx);
    load_w(wl[1 - C], wh[1 - C], nx);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay at the top: a whole step hides them
    const uint8_t* B0 = lds + (it & 1) * GA_XBUF;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const uint8_t* ra = B0 + (16 * tt + i) * GA_XRS + 32 * g;
      const uint4 xa[4] = {*reinterpret_cast<const uint4*>(ra), *reinterpret_cast<const uint4*>(ra + 16),
                           *reinterpret_cast<const uint4*>(ra + 128), *reinterpret_cast<const uint4*>(ra + 144)};
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const uint2 c0 = fp8x4_to_bf16(wl[C][ct].x), c1 = fp8x4_to_bf16(wl[C][ct].y);
        const uint2 c2 = fp8x4_to_bf16(wl[C][ct].z), c3 = fp8x4_to_bf16(wl[C][ct].w);
        const uint2 c4 = fp8x4_to_bf16(wh[C][ct].x), c5 = fp8x4_to_bf16(wh[C][ct].y);
        const uint2 c6 = fp8x4_to_bf16(wh[C][ct].z), c7 = fp8x4_to_bf16(wh[C][ct].w);
        acc[tt][ct] = mfma_bf16_16x16x32(xa[0], make_uint4(c0.x, c0.y, c1.x, c1.y), acc[tt][ct]);
        acc[tt][ct] = mfma_bf16_16x16x32(xa[1], make_uint4(c2.x, c2.y, c3.x, c3.y), acc[tt][ct]);
        acc[tt][ct] = mfma_bf16_16x16x32(xa[2], make_uint4(c4.x, c4.y, c5.x, c5.y), acc[tt][ct]);
        acc[tt][ct] = mfma_bf16_16x16x32(xa[3], make_uint4(c6.x, c6.y, c7.x, c7.y), acc[tt][ct]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the next step's staging waits for its loads only here
    store_x(xd, (it + 1) & 1);
    __syncthreads();
  };
  int it = 0;
  for (; it + 1 < NS; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    step(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < NS) step(it, std::integral_constant<int, 0>{});

  // ---- epilogue: FP8 channel scale of the lane's columns
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const float cs = p.ws_fp8[n0w + 16 * ct + i];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt][ct] *= cs;
  }
  // ---- adapter term: s_a t[row] @ B_a for the adapter of each row
  const int srow = tid >> 3, spart = tid & 7;  // the epilogue's staging: rows srow + 32 q, 16-byte part spart
  if (p.lora) {
    if (tid < 64) {
      const int t = t0 + tid;
      int a = -1;
      if (t < T) {
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
    // s_a t as bf16, [row][64 ranks] in LDS (zero past the rank and for other rows)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = srow + 32 * q;
      const int a = rid[row];
      uint32_t o[4] = {0u, 0u, 0u, 0u};
      if (a >= 0) {
        const int r = p.ranks[a];
        const float sa = p.scales[a];
        const float* trow = p.t + (long)(t0 + row) * p.r_lim;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int j = 8 * spart + 2 * d;
          o[d] = bf16x2_rne(j < r ? sa * trow[j] : 0.f, j + 1 < r ? sa * trow[j + 1] : 0.f);
        }
      }
      *reinterpret_cast<uint4*>(lds + row * GA_ERS + 16 * spart) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();
    int prev = -1;
    for (;;) {
      const int c = rid[lane];
      int m = c > prev ? c : 0x7fffffff;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = min(m, __shfl_xor(m, o, 64));
      if (m == 0x7fffffff) break;
      const int a = __builtin_amdgcn_readfirstlane(m);
      prev = a;
      const int r = p.ranks[a], rp = rank_pad(r);
      const uint16_t* Bt = reinterpret_cast<const uint16_t*>(p.B_ptrs[a]);
      for (int rs = 0; 32 * rs < r; ++rs) {
        const int jj = 32 * rs + 8 * g;
        const int off = min(jj, rp - 8);
        uint4 bop[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) bop[ct] = keep_bf16(ldg16(Bt + (long)(n0w + 16 * ct + i) * rp + off), r - jj);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int row = 16 * tt + i;
          const uint4 ah = (rid[row] == a) ? *reinterpret_cast<const uint4*>(lds + row * GA_ERS + 64 * rs + 16 * g)
                                           : zero4();
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[tt][ct] = mfma_bf16_16x16x32(ah, bop[ct], acc[tt][ct]);
        }
      }
    }
    __syncthreads();
  }

  // ---- bf16 stores through LDS, 32 rows per pass: wave w's region holds its 32 x 64 block
  uint8_t* reg = lds + w * (32 * GA_ERS);
#pragma unroll
  for (int ph = 0; ph < 2; ++ph) {
#pragma unroll
    for (int tq = 0; tq < 2; ++tq)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<uint16_t*>(reg + (16 * tq + 4 * g + v) * GA_ERS + 2 * (16 * ct + i)) =
              (uint16_t)f32_to_bf16_rne(acc[2 * ph + tq][ct][v]);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = lane + 64 * c;  // 32 rows x 8 parts of 16 bytes
      const int row = idx >> 3, part = idx & 7;
      const int t = t0 + 32 * ph + row;
      const uint4 v = *reinterpret_cast<const uint4*>(reg + row * GA_ERS + 16 * part);
      if (t < T) *reinterpret_cast<uint4*>(p.y + (long)t * N + n0w + 8 * part) = v;
    }
    __syncthreads();
  }
}

hipError_t launch_gemm_a16(const GemmParams& gp, hipStream_t s) {
  const int grid = ((gp.T + 63) / 64) * (gp.N / 256);
  hipLaunchKernelGGL(k_gemm_a16, dim3(grid), dim3(256), 0, s, gp);
  return hipGetLastError();
}

hipError_t launch_quant(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s) {
  const long blocks = ((long)T * (K / 8) + 255) / 256;
  const int grid = (int)std::min<long>(blocks, 8192);
  hipLaunchKernelGGL(k_quant_mxfp8<false>, dim3(grid), dim3(256), 0, s, x, T, K, xq, xsc);
  return hipGetLastError();
}

hipError_t launch_quant_pf(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, hipStream_t s) {
  const long blocks = ((long)T * (K / 8) + 255) / 256;
  const int grid = (int)std::min<long>(blocks, 8192);
  hipLaunchKernelGGL(k_quant_mxfp8<true>, dim3(grid), dim3(256), 0, s, x, T, K, xq, xsc);
  return hipGetLastError();
}

hipError_t launch_quant_shrink(const LayerPlan& pl, const ShrinkParams& sp, const uint16_t* x, int T, int K,
                               uint8_t* xq, uint8_t* xsc, hipStream_t s) {
  (void)x; (void)K;
  const dim3 grid((T + 15) / 16), block(256);
  if (pl.pf) {  // codes and scales in k_gemm_pf's operand order, t as PF_KP partial sums
    const dim3 gpf(((T + 63) / 64) * PF_KP);
    if (!sp.t_part || K % (64 * PF_KP) != 0) return hipErrorInvalidValue;
    switch ((sp.r_lim + 15) / 16) {
      case 1: hipLaunchKernelGGL((k_prep_pf<1>), gpf, block, 0, s, sp, xq, xsc); break;
      case 2: hipLaunchKernelGGL((k_prep_pf<2>), gpf, block, 0, s, sp, xq, xsc); break;
      case 3: hipLaunchKernelGGL((k_prep_pf<3>), gpf, block, 0, s, sp, xq, xsc); break;
      case 4: hipLaunchKernelGGL((k_prep_pf<4>), gpf, block, 0, s, sp, xq, xsc); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch ((sp.r_lim + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_prep_rows<1, true>), grid, block, 0, s, sp, xq, xsc); break;
    case 2: hipLaunchKernelGGL((k_prep_rows<2, true>), grid, block, 0, s, sp, xq, xsc); break;
    case 3: hipLaunchKernelGGL((k_prep_rows<3, true>), grid, block, 0, s, sp, xq, xsc); break;
    case 4: hipLaunchKernelGGL((k_prep_rows<4, true>), grid, block, 0, s, sp, xq, xsc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_shrink_rows(const ShrinkParams& sp, hipStream_t s) {
  const dim3 grid((sp.T + 15) / 16), block(256);
  switch ((sp.r_lim + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_prep_rows<1, false>), grid, block, 0, s, sp, nullptr, nullptr); break;
    case 2: hipLaunchKernelGGL((k_prep_rows<2, false>), grid, block, 0, s, sp, nullptr, nullptr); break;
    case 3: hipLaunchKernelGGL((k_prep_rows<3, false>), grid, block, 0, s, sp, nullptr, nullptr); break;
    case 4: hipLaunchKernelGGL((k_prep_rows<4, false>), grid, block, 0, s, sp, nullptr, nullptr); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_build(const uint16_t* x, int T, int K, uint8_t* xq, uint8_t* xsc, const int* ids, int n_ad,
                              int* seg, int* sorted, int* err, hipStream_t s) {
  const long blocks = ((long)T * (K / 8) + SEG_THREADS - 1) / SEG_THREADS;
  const int grid = 1 + (int)std::min<long>(blocks, 2048);
  return launch_kn(k_quant_build, grid, SEG_THREADS, seg_lds_bytes(T, n_ad), s, x, T, K, xq, xsc, ids, n_ad, seg, sorted,
                   err);
}

hipError_t launch_expand(const ExpandParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_expand, dim3((p.N + 255) / 256, p.T), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pack_weight(int fmt, const uint8_t* q, const uint8_t* sc, int N, int K, uint8_t* qp, uint8_t* scp,
                              hipStream_t s) {
  const long chunks = (fmt == LORA_W_FP8_E4M3) ? (long)N * K / 16 : (long)N * K / 32;
  const int grid = (int)std::min<long>((chunks + 255) / 256, 16384);
  hipLaunchKernelGGL(k_pack_weight, dim3(grid), dim3(256), 0, s, fmt, q, sc, N, K, qp, scp);
  return hipGetLastError();
}

hipError_t launch_pack_adapter(const uint16_t* A, const uint16_t* B, int K, int N, int r, uint16_t* At, uint16_t* Bt,
                               hipStream_t s) {
  const long total = (long)a_tiles(r) * 16 * K + (long)rank_pad(r) * N;
  const int grid = (int)std::min<long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_pack_adapter, dim3(grid), dim3(256), 0, s, A, B, K, N, r, At, Bt);
  return hipGetLastError();
}

hipError_t launch_merged(const uint16_t* x, int T, int K, int N, int fmt, const uint8_t* wq, const void* wscale,
                         const int* ids, const uint64_t* A_rows, const uint64_t* B_ptrs, const int* ranks,
                         const float* scales, int n_ad, int r_lim, uint16_t* y, hipStream_t s) {
  MergedParams p{};
  p.x = x; p.T = T; p.K = K; p.N = N; p.fmt = fmt; p.wq = wq;
  p.ws_fp8 = (fmt == LORA_W_FP8_E4M3) ? reinterpret_cast<const float*>(wscale) : nullptr;
  p.ws_fp4 = (fmt == LORA_W_MXFP4_E2M1) ? reinterpret_cast<const uint8_t*>(wscale) : nullptr;
  p.ids = ids; p.A_rows = A_rows; p.B_ptrs = B_ptrs; p.ranks = ranks; p.scales = scales;
  p.n_ad = n_ad; p.r_lim = r_lim; p.y = y;
  const dim3 grid(N / 16, (T + 15) / 16);
  if (fmt == LORA_W_FP8_E4M3) hipLaunchKernelGGL(k_merged<LORA_W_FP8_E4M3>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(k_merged<LORA_W_MXFP4_E2M1>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const int grid = (int)std::min<size_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

// ======================================================================================
// Scratch memory of the allocation-free layer call (gemm_lowp_lora_epilogue_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.  In host code
// `scratch` names a host-side stand-in, so the kernels only ever get the device address
// that hipGetSymbolAddress returns for the current device (looked up once per device).
// ======================================================================================
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
struct ScratchState {
  void* ptr = nullptr;               // device address of this device's copy
  size_t tag_lo = 0, tag_hi = 0;     // tagged hand-over area of the last call's layout
};
ScratchState g_scratch[MAX_DEVICES];
}  // namespace

hipError_t scratch_acquire(hipStream_t s, size_t tag_lo, size_t tag_hi, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchState& st = g_scratch[dev];
  if (!st.ptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // first use on this device: the whole array starts at zero (control block, tags)
    e = launch_fill_zero(p, SCRATCH_BYTES, s);
    if (e != hipSuccess) return e;
    st.ptr = p;
  } else if (tag_lo != st.tag_lo || tag_hi != st.tag_hi) {
    // another layout: its tagged area may hold bytes of other buffers of the last layout,
    // which must not pass for tags of a later launch
    e = launch_fill_zero(reinterpret_cast<char*>(st.ptr) + tag_lo, tag_hi - tag_lo, s);
    if (e != hipSuccess) return e;
  }
  st.tag_lo = tag_lo;
  st.tag_hi = tag_hi;
  *out = st.ptr;
  return hipSuccess;
}

}  // namespace lora

// Device helpers shared by the gfx950 kernels: bf16 handling, the MXFP8 block
// quantiser, and thin wrappers over the CDNA4 matrix instructions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace lora {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs are finite; NaN maps to a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// two floats to bf16 (round to nearest even) in one word, lo in bits 0..15: the gfx950
// conversion instruction (finite values as f32_to_bf16_rne; NaN stays a quiet NaN)
// (one v_cvt_pk_bf16_f32: the vector conversion keeps both halves in one instruction)
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// ---------------------------------------------------------------------------------
// MXFP8 quantisation of one 32-element block (OCP Microscaling v1.0, e4m3 elements):
//   scale code = E + 127 with E = floor(log2 max|x|) - 8, clamped to [-127, 127];
//   element = RNE_e4m3(clamp(x * 2^-E, +-448)).
// For a bf16 maximum with biased exponent field ef >= 1, floor(log2 max) = ef - 127, so
// the code is ef - 8; zero and subnormal maxima (ef == 0) and ef <= 8 give E = -127,
// code 0.  |bits| compares as an unsigned integer in the order of |x|.
// The conversion uses v_cvt_pk_fp8_f32 (round to nearest even, OCP e4m3fn on gfx950);
// its inputs are already clamped, and it keeps the sign of zero.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mx_block_code(const uint4 (&in)[4]) {
  us2 m = {0, 0};
  const us2 mask = {0x7fff, 0x7fff};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w[4] = {in[i].x, in[i].y, in[i].z, in[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      us2 v = __builtin_bit_cast(us2, w[j]) & mask;
      m = __builtin_elementwise_max(m, v);
    }
  }
  uint32_t mx = m.x > m.y ? m.x : m.y;
  uint32_t ef = mx >> 7;
  return ef > 8u ? ef - 8u : 0u;
}


// Largest |x| of 8 bf16 (one 16-byte piece of a block), as 15-bit magnitude bits.
__device__ __forceinline__ uint32_t absmax8_bits(const uint4& in) {
  const us2 mask = {0x7fff, 0x7fff};
  us2 m = __builtin_bit_cast(us2, in.x) & mask;
  m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, in.y) & mask);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, in.z) & mask);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, in.w) & mask);
  return m.x > m.y ? m.x : m.y;
}

// Scale code of a block from its largest magnitude bits (the rule above).
__device__ __forceinline__ uint32_t mx_code_from_bits(uint32_t mx) {
  const uint32_t ef = mx >> 7;
  return ef > 8u ? ef - 8u : 0u;
}

// Element codes with the gfx950 scaled conversion: the magnitudes are first clamped to
// 448 * 2^E in the bf16 bit domain (the bits of a non-negative bf16 order as its value),
// then v_cvt_scalef32_pk_fp8_bf16 divides by its scale operand 2^E (exact) and rounds to
// nearest even.  For finite x this is RNE_e4m3(clamp(x * 2^-E, +-448)), the rule above:
// checked on the GPU against the fp32 form (multiply by 2^-E, clamp, v_cvt_pk_fp8_f32)
// for every finite bf16 pattern at scale codes 0 to 246, with no difference.
struct MxScale {
  us2 lim;   // bf16 bits of 448 * 2^E (= 1.75 * 2^(code - 119)), in both halves
  float sc;  // 2^E = 2^(code - 127) as a float (a subnormal for code 0)
};
__device__ __forceinline__ MxScale mx_scale(uint32_t code) {
  const unsigned short l = (unsigned short)(((code + 8u) << 7) | 0x60u);
  return {us2{l, l}, code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u)};
}
// Four e4m3 codes (byte i from bf16 i, low half of w0 first) of two bf16 pairs.
__device__ __forceinline__ uint32_t mx_cvt4(uint32_t w0, uint32_t w1, const MxScale& s) {
  const us2 mask = {0x7fff, 0x7fff};
  auto clampw = [&](uint32_t w) {
    const us2 m = __builtin_elementwise_min(__builtin_bit_cast(us2, w) & mask, s.lim);
    return __builtin_bit_cast(bf16x2, (w & 0x80008000u) | __builtin_bit_cast(uint32_t, m));
  };
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, clampw(w0), s.sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, clampw(w1), s.sc, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Quantise one 16-byte piece (8 bf16) of a block with the block's scale code into 8
// e4m3 codes.
__device__ __forceinline__ uint2 mx_piece_quant(const uint4& in, uint32_t code) {
  const MxScale s = mx_scale(code);
  return make_uint2(mx_cvt4(in.x, in.y, s), mx_cvt4(in.z, in.w, s));
}

// Quantise 32 bf16 (64 bytes in `in`) with scale code `code` into 32 e4m3 codes (out[2]).
__device__ __forceinline__ void mx_block_quant(const uint4 (&in)[4], uint32_t code, uint4 (&out)[2]) {
  const MxScale s = mx_scale(code);
  uint32_t r[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = mx_cvt4(in[i].x, in[i].y, s);
    r[2 * i + 1] = mx_cvt4(in[i].z, in[i].w, s);
  }
  out[0] = make_uint4(r[0], r[1], r[2], r[3]);
  out[1] = make_uint4(r[4], r[5], r[6], r[7]);
}

// ---------------------------------------------------------------------------------
// Scaled MFMA, 16x16x128, gfx950.  Operand layout (measured with a one-instruction
// probe against a CPU model, lane l, g = l / 16, row/column = l % 16):
//   fp8 operand (8 dwords): bytes 0..15 hold k = 16g .. 16g+15, bytes 16..31 hold
//                           k = 64+16g .. 64+16g+15;
//   fp4 operand (4 dwords): nibble q (byte q/2, low nibble first) holds k = 32g + q;
//   scale operand (byte 0): row/column l % 16, K-block g (k = 32g .. 32g+31);
//   result: lane l, element v -> row 4g + v, column l % 16.
// ---------------------------------------------------------------------------------
template <int FMT_B>
__device__ __forceinline__ v4f mfma_scaled_16x16x128(const uint4& alo, const uint4& ahi, const uint4& blo,
                                                     const uint4& bhi, v4f acc, int sa, int sb) {
  v8i a = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  v8i b = {(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, FMT_B, 0, sa, 0, sb);
}

// The same with the B operand already assembled as one 32-byte register tuple: loads
// written straight into the two halves of a tuple that lives across many instructions
// spare the register allocator from joining two separately allocated halves later.
template <int FMT_B>
__device__ __forceinline__ v4f mfma_scaled_16x16x128(const uint4& alo, const uint4& ahi, const v8i& b, v4f acc, int sa,
                                                     int sb) {
  v8i a = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, FMT_B, 0, sa, 0, sb);
}
// The same with the A scale taken from byte `opa` (0..3) of a word of four codes; opa is
// a constant after unrolling (the instruction encodes it).
template <int FMT_B>
__device__ __forceinline__ v4f mfma_scaled_16x16x128_sel(int opa, const uint4& alo, const uint4& ahi, const uint4& blo,
                                                         const uint4& bhi, v4f acc, int sa_word, int sb) {
  v8i a = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w, (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  v8i b = {(int)blo.x, (int)blo.y, (int)blo.z, (int)blo.w, (int)bhi.x, (int)bhi.y, (int)bhi.z, (int)bhi.w};
  if (opa == 0) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, FMT_B, 0, sa_word, 0, sb);
  if (opa == 1) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, FMT_B, 1, sa_word, 0, sb);
  if (opa == 2) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, FMT_B, 2, sa_word, 0, sb);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, FMT_B, 3, sa_word, 0, sb);
}
__device__ __forceinline__ v8i join8(const uint4& lo, const uint4& hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// bf16 MFMA 16x16x32.  A and B operands have mirrored layouts (lane l: row/column
// l % 16, eight k values for lane group l / 16), so any fixed assignment of the eight
// k values of a lane group works as long as both operands use it; the result layout
// is that of every 16x16 MFMA (row 4g + v, column l % 16).
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const uint4& a, const uint4& b, v4f acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), acc, 0,
                                                 0, 0);
}

// Widening of W codes to bf16 with the gfx950 scaled conversions (exact: e4m3 and e2m1
// values times a power of two fit bf16 unless the power leaves bf16's normal range).
// Four e4m3fn codes (byte 0 first) -> four bf16 in two dwords (element 0 in the low half).
__device__ __forceinline__ uint2 fp8x4_to_bf16(uint32_t v) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true)));
}
// Eight e2m1 codes (low nibble of byte 0 first) times `s` (a power of two) -> eight bf16.
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t v, float s) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3)));
}

// 16-byte load from global memory.  The address-space cast makes the compiler emit
// global_load (counted by vmcnt only) rather than flat_load, which also counts in lgkmcnt
// and forces full waits.
__device__ __forceinline__ uint4 ldg16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(1))) const uint4 g_uint4;
  return *(g_uint4*)(reinterpret_cast<uintptr_t>(p));
#else
  return *reinterpret_cast<const uint4*>(p);  // host pass only; never executed
#endif
}

// ---------------------------------------------------------------------------------
// Data handed between workgroups inside one launch (split-K partial sums, the
// down-projection t, arrival counters).  The eight XCDs of an MI355X each have their
// own L2, and those L2s are not coherent with each other.  An agent-scope fence would
// make plain stores visible by writing back (buffer_wbl2) or invalidating (buffer_inv)
// the entire L2 of the XCD, which stalls every workgroup streaming through it.
// Instead, every value that crosses workgroups is written with an agent-coherent store
// (relaxed agent-scope atomic store: global_store ... sc1, written through past the L2)
// and read with an agent-coherent load (global_load ... sc1).  A writer waits for its
// stores to complete (s_waitcnt vmcnt(0)) and passes a workgroup barrier before one
// thread bumps the arrival counter with a relaxed agent-scope atomic; a reader acts
// only after observing the counter.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void set_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_agent(int* p, int v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// the same from an address held as an integer: the global address space is stated, so
// the load is a global (not a flat) access
__device__ __forceinline__ uint64_t ld_agent_u64_at(uint64_t addr) {
  typedef __attribute__((address_space(1))) uint64_t g_u64;
  return __hip_atomic_load(reinterpret_cast<g_u64*>(addr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until every memory operation this wave issued has completed
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// The first n of the eight bf16 in v (element e in half e % 2 of dword e / 2), the
// others zeroed; n <= 0 gives zero, n >= 8 gives v.  Masks the padding of an adapter
// stored with a rank that is not a multiple of 8.
__device__ __forceinline__ uint4 keep_bf16(const uint4& v, int n) {
  auto m = [n](int d) -> uint32_t { return (2 * d + 1 < n) ? 0xffffffffu : ((2 * d < n) ? 0x0000ffffu : 0u); };
  return make_uint4(v.x & m(0), v.y & m(1), v.z & m(2), v.w & m(3));
}

}  // namespace lora

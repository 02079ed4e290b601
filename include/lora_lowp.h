/*
 * lora_lowp.h -- C ABI of the fused multi-tenant LoRA layer over a low-precision
 * base GEMM, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes.  "Punica: Serving multiple LoRA finetuned LLM as one"
 * (README, Overview) writes a LoRA'd layer as y = x@W + x@A@B with W [H1, H2],
 * A [H1, r], B [r, H2], and a batch whose parts x_i map to adapter i as
 * Y = X@W + (x_1@A_1@B_1, ..., x_n@A_n@B_n).  The "EpiLoRA" abstract puts W in
 * 8-bit (FP8) or 4-bit form, runs the adapter down-projection first and adds every
 * tenant's up-projection in the epilogue of the low-precision GEMM.  Here, per
 * token t with adapter a = adapter_id[t] and per-adapter scale s_a:
 *
 *     y[t, :] = bf16( dequant(xq[t] . W) + s_a * (x[t] @ A_a) @ B_a )
 *
 * with H1 = K, H2 = N, x bf16 [T, K], and xq the MXFP8 form of x (32-element
 * K-blocks: e8m0 scale 2^E with E = floor(log2 max|x|) - 8, e4m3fn elements,
 * round to nearest even, clamped to +-448 -- OCP Microscaling Formats v1.0).
 * The adapter terms use the bf16 x itself.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked [host]; the caller owns all
 *    memory.  Buffers are dense row-major with no padding and 16-byte aligned.
 *  - bf16 values are passed as their uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it; nothing is synchronised and nothing is allocated.
 *  - Argument checks run on the host before anything is enqueued; on error the
 *    call returns a non-zero lora_status and enqueues nothing.  A failed launch
 *    returns LORA_ERR_HIP.  Adapter ids outside [0, n_adapters) are data errors
 *    found on the device: lora_build_segments reports them in *err_word and
 *    leaves those tokens out of the segments; later calls skip the adapter term
 *    of such tokens.
 *  - Limits: K % 128 == 0 (whole MFMA K-steps; MX blocks are 32), N % 64 == 0,
 *    0 <= T <= 65536 (T == 0 is a no-op returning LORA_OK), 1 <= n_adapters <= 8192,
 *    r_max a multiple of 8 in [8, 64], every rank a multiple of 8 in [8, r_max].  The
 *    ranks live in device memory, so the kernels check them: an adapter whose rank
 *    breaks this rule contributes no adapter term (and its rows of t are not written).
 *
 * Data layouts:
 *  - W, FP8 (LORA_W_FP8_E4M3), row-major form: w_q uint8 [N][K] e4m3fn codes (K
 *    contiguous), w_scale float [N], one scale per output channel; dequant =
 *    w_scale[n]*code.
 *  - W, MXFP4 (LORA_W_MXFP4_E2M1), row-major form: w_q uint8 [N][K/2] e2m1 codes,
 *    element k of row n in the low nibble of byte k/2 when k is even, high nibble
 *    when odd; w_scale uint8 [N][K/32] e8m0 codes, one per 32 consecutive k.
 *  - gemm_lowp_lora_epilogue reads W in the packed form made once by
 *    lora_pack_weight (same bytes, reordered so that each 16-byte load of the GEMM
 *    reads 1 KB of consecutive memory; the FP8 channel scales stay as they are):
 *      FP8:   [N/16][K/128][h = 0,1][l = 0..63][16 B]: 16 codes of channel
 *             16*nt + l%16 at k = 128*ks + 64*h + 16*(l/16) ..
 *      MXFP4: [N/16][K/128][l][16 B]: 32 codes of channel 16*nt + l%16 at
 *             k = 128*ks + 32*(l/16) .., and scales [N/16][K/128][l] (one byte:
 *             the code of k-block 4*ks + l/16).
 *  - Adapter a: A_a [K][r_a] is stored as A_a^T, bf16 [r_a][K] (K contiguous),
 *    and B_a [r_a][N] as B_a^T, bf16 [N][r_a] (r_a contiguous) -- the weights of
 *    the linear maps K -> r_a and r_a -> N in out-by-in order, so that both matrix
 *    products read 16-byte runs along their reduction dimension.
 *    A_ptrs / B_ptrs are device arrays of n_adapters device addresses (uint64),
 *    so adapters may live anywhere in device memory.  ranks int32 [n_adapters],
 *    scales float [n_adapters].
 *  - Segments (from lora_build_segments): seg_indptr int32 [n_adapters + 1] is a
 *    CSR over adapter ids (empty adapters included), sorted_tok int32 [T] lists
 *    token indices ordered by (adapter id, token index).
 *  - t: float [T][r_max], original token order, columns j >= r_a hold zero.
 *  - y: bf16 [T][N], original token order.
 *
 * Workspace: gemm_lowp_lora_epilogue and lora_shrink take a caller-provided
 * device workspace of at least lora_workspace_bytes(...) bytes, zero-filled once
 * before first use (lora_workspace_init does that).  Every call leaves its
 * counters at zero again when it completes, so calls that share a workspace must
 * be ordered on one stream; calls that overlap in time need distinct workspaces.
 */
#ifndef LORA_LOWP_H
#define LORA_LOWP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lora_status;
enum {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARG = 1,   /* bad pointer, size, alignment or format        */
  LORA_ERR_UNSUPPORTED = 2,   /* valid but outside the limits listed above      */
  LORA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required     */
  LORA_ERR_HIP = 5            /* a HIP launch or query failed                   */
};

enum { LORA_W_FP8_E4M3 = 0, LORA_W_MXFP4_E2M1 = 1 };

/* flags for gemm_lowp_lora_epilogue */
enum {
  /* Run the adapter down-projection inside the same launch: its workgroups take the
   * lowest ids and start first, the GEMM workgroups stream W meanwhile and wait for
   * t only in their epilogue.  t (if non-NULL) receives the down-projection. */
  LORA_FUSE_SHRINK = 1u << 0,
  /* With LORA_FUSE_SHRINK: the same launch also builds the batch's segments from
   * adapter_id, exactly as lora_build_segments does (one more workgroup; the
   * down-projection workgroups that read them wait for it).  seg_indptr and
   * sorted_tok are then outputs; the error word goes to the workspace (see
   * lora_workspace_segment_error).  Meant for the first LoRA layer of a batch, so
   * that the batch needs no launch of its own for the segments.  Above 128 tokens the
   * call launches the builder just before the layer instead (the down-projection
   * would otherwise start late); the outputs are the same. */
  LORA_BUILD_SEGMENTS = 1u << 1,
  /* The engine variant that keeps activations in 16 bits ("EpiLoRA" abstract, on
   * narrowing the mismatch between generator and trainer): the base product reads the
   * bf16 x as it is, with no MXFP8 quantisation.  W is widened to bf16 in registers
   * (FP8 codes exactly; MXFP4 codes times their block scale, exact while the value
   * stays in bf16's normal range: block scale codes 2 .. 252 for any e2m1 code)
   * and the products run on bf16 MFMA with fp32 accumulation; the FP8 channel scale
   * and the adapter terms are applied as without the flag.  Any T: up to 16 tokens the
   * decode stream; above, 64-token x 128-channel tiles with bf16 x staged in LDS where
   * N % 128 == 0, else 16-token tiles of the decode stream (much slower for large T). */
  LORA_ACT_BF16 = 1u << 2
};

/* Status code as text; never NULL. */
const char* lora_status_string(lora_status s);

/* Library build identifier (gfx target and kernel set); never NULL. */
const char* lora_version(void);

/* Bytes of workspace needed by lora_shrink and gemm_lowp_lora_epilogue for these
 * sizes (any flags).  Returns 0 for sizes outside the limits. */
size_t lora_workspace_bytes(int32_t T, int32_t K, int32_t N, int32_t n_adapters, int32_t r_max);

/* Zero-fill a workspace (a fill kernel on `stream`, safe under graph capture). */
lora_status lora_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Group tokens by adapter ("Punica" README, Overview: the batch X splits into the
 * parts x_i that map to each adapter; the kernel is "Segmented" for that reason).
 * adapter_id int32 [T] -> seg_indptr int32 [n_adapters+1], sorted_tok int32 [T].
 * The result is unique: a stable counting sort.  *err_word (device int32) is set to
 * 0, or to 1 + the index of a token whose id is outside [0, n_adapters); such tokens
 * are left out (seg_indptr[n_adapters] < T).  One workgroup; deterministic. */
lora_status lora_build_segments(const int32_t* adapter_id, int32_t T, int32_t n_adapters,
                                int32_t* seg_indptr, int32_t* sorted_tok, int32_t* err_word,
                                void* stream);

/* Reorder a row-major W (codes, and for MXFP4 its block scales) into the packed form
 * that gemm_lowp_lora_epilogue reads (see "Data layouts").  An offline step, like the
 * quantisation of W itself.  FP8: scale and scale_packed are ignored (may be NULL).
 * Not in place.  N % 64 == 0, K % 128 == 0. */
lora_status lora_pack_weight(int32_t w_fmt, const uint8_t* q, const uint8_t* scale, int32_t N, int32_t K,
                             uint8_t* q_packed, uint8_t* scale_packed, void* stream);

/* MXFP8 quantisation of bf16 activations x [T][K] -> x_q uint8 [T][K] e4m3fn codes,
 * x_sc uint8 [T][K/32] e8m0 codes, by the rule in the header comment.  Bit-exact;
 * the same device function quantises x inside gemm_lowp_lora_epilogue. */
lora_status lora_quant_act_mxfp8(const uint16_t* x, int32_t T, int32_t K,
                                 uint8_t* x_q, uint8_t* x_sc, void* stream);

/* Adapter down-projection ("EpiLoRA" abstract: the down-projection is launched
 * first; "Punica" README: SGMV over segments):
 *   t[tok, j] = sum_k x[tok, k] * A_a[k, j]  for every tok in segment a, j < r_a,
 * fp32 accumulation of exact bf16 products, written in original token order,
 * zero for j >= r_a.  Fixed summation order: bitwise deterministic.  The standalone
 * down-projection needs no scratch memory: workspace may be NULL (kept in the
 * signature so that callers can pass the layer's workspace). */
lora_status lora_shrink(const uint16_t* x, int32_t T, int32_t K,
                        const int32_t* seg_indptr, const int32_t* sorted_tok,
                        const uint64_t* A_ptrs, const int32_t* ranks,
                        int32_t n_adapters, int32_t r_max,
                        float* t, void* workspace, size_t workspace_bytes, void* stream);

/* Adapter up-projection as its own launch (the unfused schedule the "EpiLoRA"
 * abstract replaces):  y[tok, :] = bf16( y[tok, :] + s_a * t[tok, :r_a] @ B_a ).
 * y is read and written in place. */
lora_status lora_expand(const float* t, int32_t T, int32_t N,
                        const int32_t* adapter_id, const uint64_t* B_ptrs,
                        const int32_t* ranks, const float* scales,
                        int32_t n_adapters, int32_t r_max,
                        uint16_t* y, void* stream);

/* The fused layer ("EpiLoRA" abstract): low-precision base GEMM on gfx950 scaled
 * MFMA (x quantised to MXFP8 in the loader; with LORA_ACT_BF16, bf16 x on bf16 MFMA
 * instead), with the epilogue applying the FP8
 * channel scale and adding s_a * t[tok] @ B_a for every token's adapter before
 * the bf16 store (round to nearest even).
 *  - flags & LORA_FUSE_SHRINK: the down-projection runs in the same launch (t is an
 *    output, may be NULL).  Otherwise t is an input (from lora_shrink); t == NULL
 *    then means "base GEMM only" and the adapter arguments may be NULL.
 *  - seg_indptr / sorted_tok: read (from lora_build_segments) unless flags has
 *    LORA_BUILD_SEGMENTS, which makes them outputs of this call.
 *  - w_fmt: LORA_W_FP8_E4M3 or LORA_W_MXFP4_E2M1; w_q (and for MXFP4 w_scale) in the
 *    packed form made by lora_pack_weight; for FP8 w_scale is float [N].
 * y is written, not accumulated into. */
lora_status gemm_lowp_lora_epilogue(const uint16_t* x, int32_t T, int32_t K, int32_t N,
                                    int32_t w_fmt, const uint8_t* w_q, const void* w_scale,
                                    float* t, const int32_t* adapter_id,
                                    int32_t* seg_indptr, int32_t* sorted_tok,
                                    const uint64_t* A_ptrs, const uint64_t* B_ptrs,
                                    const int32_t* ranks, const float* scales,
                                    int32_t n_adapters, int32_t r_max,
                                    uint16_t* y, uint32_t flags,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Device-side status word of the last gemm_lowp_lora_epilogue / lora_shrink that
 * used this workspace: copies one int32 to *status_dev (device pointer) on
 * `stream`.  0 = fine; non-zero = a bounded wait in the fused launch gave up
 * (the output is then unspecified).  Cleared by lora_workspace_init. */
lora_status lora_workspace_status(const void* workspace, int32_t* status_dev, void* stream);

/* Error word of the last segment build inside gemm_lowp_lora_epilogue
 * (LORA_BUILD_SEGMENTS) on this workspace, with the meaning of lora_build_segments'
 * err_word: copies one int32 to *err_dev (device pointer) on `stream`. */
lora_status lora_workspace_segment_error(const void* workspace, int32_t* err_dev, void* stream);

/* Introspection for tests and benchmarks: writes the tile plan chosen for these sizes
 * into out[0..n_out) (host array) as {token tiles of 16 per workgroup, column tiles of
 * 16 per wave, waves along N, waves along K, separate x-quantisation pass, K-chunk,
 * K-splits, K-range, column blocks, token blocks, GEMM workgroups, down-projection token
 * block, its rank groups, its K-parts, its workgroups} and returns the number of entries
 * (15), or -1 for sizes outside the limits.  Pure host function. */
int32_t lora_plan_info(int32_t T, int32_t K, int32_t N, int32_t n_adapters, int32_t r_max, int32_t w_fmt,
                       int32_t* out, int32_t n_out);

#ifdef __cplusplus
}
#endif

#endif /* LORA_LOWP_H */

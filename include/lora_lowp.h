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
 *    1 <= r_max <= 64, and every rank r_a in [1, r_max] (any value: ranks differ per
 *    adapter).  The ranks live in device memory, so the kernels check them: an
 *    adapter whose rank is outside [1, r_max] contributes no adapter term (its rows of
 *    t are not written) and the layer call sets bit 1 of the workspace status word
 *    (lora_workspace_status), so the error is never silent.
 *
 * Where this interface departs from the problem as the pages state it (adapter
 * A [K, r] and B [r, N] in any layout the caller likes, K a multiple of the MX block
 * of 32), and why:
 *  - Adapters are read in a packed form made once by lora_pack_adapter from A [K][r]
 *    and B [r][N] row-major (below): A in bf16 MFMA operand order, B as B^T
 *    [N][rank_pad(r)].  Both adapter products then read 16-byte runs along their
 *    reduction dimension straight into bf16 MFMA operands (for A, each wave's load of a
 *    rank tile reads 1 KB of consecutive memory), and any rank keeps those runs aligned.
 *    Like the quantisation of W, this is an offline step per adapter, not per call;
 *    it needs K % 64 == 0.
 *  - W is read in the packed form made once by lora_pack_weight (below): each 16-byte
 *    load of the GEMM then reads 1 KB of consecutive memory.
 *  - K % 128 == 0 instead of K % 32: the scaled MFMA takes 128 values of K per step;
 *    N % 64 == 0: the narrowest column tile of a workgroup is 64 channels.  Other
 *    shapes return LORA_ERR_UNSUPPORTED (they are never computed wrongly).
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
 *  - Adapter a (packed by lora_pack_adapter), as the weights of the linear maps
 *    K -> r_a and r_a -> N in out-by-in order:
 *      A: ceil(r_a/16) rank tiles of 16, each [K/64][h = 0,1][l = 0..63][8] bf16 --
 *         the 8 values of lane l = 16 g + i hold A_a[k][16 jt + i] for
 *         k = 64 ks + 16 g + 8 h .. + 7 (the bf16 MFMA operand of rank tile jt for
 *         that k-step; element (j, k) at ((((j/16) (K/64) + k/64) 2 + (k/8)%2) 64 +
 *         16 ((k/16)%4) + j%16) 8 + k%8), 16 ceil(r_a/16) K values in all;
 *      B: B_a^T, bf16 [N][rank_pad(r_a)] (ranks contiguous).
 *    Ranks j >= r_a are padding: lora_pack_adapter zero-fills them, and the kernels
 *    never let them reach a result.  16-byte aligned.
 *    A_ptrs / B_ptrs are device arrays of n_adapters device addresses (uint64),
 *    so adapters may live anywhere in device memory.  ranks int32 [n_adapters],
 *    scales float [n_adapters].
 *  - Segments (from lora_build_segments): seg_indptr int32 [n_adapters + 1] is a
 *    CSR over adapter ids (empty adapters included), sorted_tok int32 [T] lists
 *    token indices ordered by (adapter id, token index).
 *  - t: float [T][r_max] (row stride r_max), original token order, columns
 *    j >= r_a hold zero.
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
  LORA_ERR_HIP = 5,           /* a HIP launch or query failed                   */
  LORA_ERR_SCRATCH_LIMIT = 6  /* gemm_lowp_lora_epilogue_noalloc: the sizes need more
                                 scratch than LORA_NOALLOC_SCRATCH_BYTES           */
};

/* Scratch memory of gemm_lowp_lora_epilogue_noalloc, per GPU (bytes). */
#define LORA_NOALLOC_SCRATCH_BYTES (32u << 20)

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
   * N % 128 == 0, else 16-token tiles of the decode stream (much slower for large T).
   * Past 128 tokens with FP8 W and N % 256 == 0 the fused call first runs the
   * down-projection in a launch of its own (plain fp32 t, into t or the workspace) and
   * then the GEMM in 64 x 256 tiles, two workgroups per CU. */
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

/* Pack one adapter ("Punica" README, Overview: A [H1, r] and B [r, H2]) into the form
 * the layer reads (see "Data layouts"): A bf16 [K][r] row-major -> At, 16 ceil(r/16) K
 * bf16 in operand order; B bf16 [r][N] row-major -> Bt bf16 [N][rank_pad(r)]
 * (Bt[n][j] = B[j][n]); padding ranks are zero.  rank_pad(r) = (r + 7) / 8 * 8.
 * An offline step per adapter.  1 <= r <= 64 and K % 64 == 0 (else
 * LORA_ERR_UNSUPPORTED, or LORA_ERR_INVALID_ARG for r < 1); At and Bt 16-byte aligned;
 * no buffer may overlap another. */
lora_status lora_pack_adapter(const uint16_t* A, const uint16_t* B, int32_t K, int32_t N, int32_t r,
                              uint16_t* At, uint16_t* Bt, void* stream);

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
 * signature so that callers can pass the layer's workspace).  An adapter whose rank is
 * outside [1, r_max] is skipped (its rows of t are not written); the layer call that
 * consumes t reports it. */
lora_status lora_shrink(const uint16_t* x, int32_t T, int32_t K,
                        const int32_t* seg_indptr, const int32_t* sorted_tok,
                        const uint64_t* A_ptrs, const int32_t* ranks,
                        int32_t n_adapters, int32_t r_max,
                        float* t, void* workspace, size_t workspace_bytes, void* stream);

/* The standalone down-projection (lora_shrink's result, bitwise: every configuration keeps
 * the summation order) with an explicit configuration, for operator tuning ("Efficient
 * multi-tenant LoRA serving via SGMV-specific operator autotuning", abstract: tiling,
 * caching and virtual-thread scheduling of the SGMV operator chosen by a stochastic search).
 * config [host] int32[5] = {TG, JP, U, TBLK, ORDER}:
 *   TG   token tiles of 16 per inner step on bf16 MFMA (tiling)   1, 2 or 4; or 0: the
 *        wave-reduction kernel (BGMV: each lane multiplies 16 k of one rank with the tokens'
 *        x in fp32, the lane groups and waves summed by shuffles and LDS), for segments of a
 *        few tokens
 *   JP   rank tiles of 16 per workgroup item (tiling)          1, 2 or 4
 *   U    k-steps of 64 per prefetch buffer (caching)          1 or 2 (TG = 0: 2 only with TBLK 1)
 *   TBLK positions of one segment per workgroup item (scheduling): a multiple of 16, or for
 *        TG = 0: 1, 2 or 4
 *   ORDER 0: items in workgroup-id order; 1: each XCD takes a contiguous run of items
 *         (scheduling).
 * Other values return LORA_ERR_UNSUPPORTED.  Other arguments as lora_shrink.  The
 * wave-reduction kernel sums in another order than the MFMA kernels (t agrees to fp32
 * rounding, bitwise deterministic on its own). */
lora_status lora_shrink_configured(const uint16_t* x, int32_t T, int32_t K,
                                   const int32_t* seg_indptr, const int32_t* sorted_tok,
                                   const uint64_t* A_ptrs, const int32_t* ranks,
                                   int32_t n_adapters, int32_t r_max, float* t,
                                   const int32_t* config, void* stream);

/* The per-token merged-weight formulation of the layer, an alternative to ablate against
 * ("LoRA-Switch" abstract: each token's adapter is merged into the backbone weights for
 * inference, the merges fused in one kernel):
 *     y[t, :] = bf16( x[t] . (W_d + s_a A_a B_a) ),   a = adapter_id[t],
 * with the merged weight formed in registers (rounded to bf16 for the MFMA) and never
 * stored; x enters in bf16 (by the merged-weight identity this is the 16-bit activation
 * layer).  Tokens whose adapter id or rank is invalid get the base term only.
 *  - w_q, w_scale: W in its row-major form (see "Data layouts"), not packed;
 *  - A_rows: per adapter, the device address of A_a as bf16 [K][rank_pad(r_a)] row-major
 *    (the ranks past r_a read but masked);
 *  - B_ptrs: per adapter, B_a^T packed by lora_pack_adapter.
 * Limits as for the layer call; no workspace; one launch. */
lora_status lora_merged_layer(const uint16_t* x, int32_t T, int32_t K, int32_t N, int32_t w_fmt,
                              const uint8_t* w_q, const void* w_scale, const int32_t* adapter_id,
                              const uint64_t* A_rows, const uint64_t* B_ptrs,
                              const int32_t* ranks, const float* scales, int32_t n_adapters,
                              int32_t r_max, uint16_t* y, void* stream);

/* Resources of the compiled wave-reduction down-projection (TBLK = nt positions, jp, u) on the
 * current device, as lora_shrink_config_info. */
lora_status lora_shrink_bgmv_info(int32_t nt, int32_t jp, int32_t u, int32_t* out);

/* Resources of the compiled down-projection instance (TG, JP, U) on the current device:
 * out [host] int32[3] = {registers per lane, scratch (spill) bytes per lane, LDS bytes}.
 * LORA_ERR_UNSUPPORTED for a configuration that is not compiled; LORA_ERR_HIP without a
 * device. */
lora_status lora_shrink_config_info(int32_t tg, int32_t jp, int32_t u, int32_t* out);

/* Adapter up-projection as its own launch (the unfused schedule the "EpiLoRA"
 * abstract replaces):  y[tok, :] = bf16( y[tok, :] + s_a * t[tok, :r_a] @ B_a ).
 * y is read and written in place.  Tokens whose adapter id is outside
 * [0, n_adapters) or whose adapter's rank is outside [1, r_max] are left as they are. */
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

/* gemm_lowp_lora_epilogue for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same call with
 * the same arguments and results, minus the workspace.  Its scratch memory is a
 * library-owned device array of LORA_NOALLOC_SCRATCH_BYTES per GPU (32 MiB, held until
 * the process ends); the call allocates nothing and calls no allocating routine.
 *  - Sizes whose lora_workspace_bytes exceed LORA_NOALLOC_SCRATCH_BYTES return
 *    LORA_ERR_SCRATCH_LIMIT and enqueue nothing (every shape of the pages' workloads
 *    fits: the 4096-token prefill needs 22.5 MiB).
 *  - All calls on one GPU share its array: calls on one GPU must be ordered on one
 *    stream (calls that overlap in time on one GPU race).  The first call on a GPU, and
 *    a call whose sizes lay the array out differently from the previous call's on that
 *    GPU, also enqueue a fill kernel that clears the array's hand-over tags.
 *  - The device status word and the in-launch segment builder's error word live in the
 *    array and are not reported; callers that need the error word build the segments
 *    with lora_build_segments. */
lora_status gemm_lowp_lora_epilogue_noalloc(const uint16_t* x, int32_t T, int32_t K, int32_t N,
                                            int32_t w_fmt, const uint8_t* w_q, const void* w_scale,
                                            float* t, const int32_t* adapter_id,
                                            int32_t* seg_indptr, int32_t* sorted_tok,
                                            const uint64_t* A_ptrs, const uint64_t* B_ptrs,
                                            const int32_t* ranks, const float* scales,
                                            int32_t n_adapters, int32_t r_max,
                                            uint16_t* y, uint32_t flags, void* stream);

/* ---- Backward: the adapters train on the frozen low-precision base ----
 * The "EpiLoRA" abstract has the LoRA trainer compute on the serving engine's FP8 weights,
 * with no 16-bit copy of W, and keep activations in 16 bits.  For the 16-bit-activation
 * layer y[t] = x[t] W_d + s_a (x[t] A_a) B_a (W_d the dequantised W, frozen; A_a, B_a
 * trained; s_a fixed) and the gradient dY of a loss with respect to y, the chain rule over
 * each adapter's tokens R_a (its segment, "Punica" README, Overview) gives
 *     u[t]  = dY[t] B_a^T,            dX[t] = dY[t] W_d^T + s_a u[t] A_a^T,
 *     dA_a  = s_a sum_{t in R_a} x[t]^T u[t],   dB_a = s_a sum_{t in R_a} t_a[t]^T dY[t],
 * with t_a[t] = x[t] A_a the forward's down-projection.  FP8 base only (MXFP4:
 * LORA_ERR_UNSUPPORTED). */

/* W^T in the packed form lora_backward reads, from the row-major FP8 codes q uint8 [N][K]:
 * tiles of 16 rows k by 64 channels n, 1 KB each, tile (kt, ns) at byte
 * ((kt (N/64) + ns) 64 + l) 16 for lane l = 16 g + i, whose 16 bytes hold the codes of
 * W[64 ns + 16 g + e][16 kt + i], e = 0 .. 15.  An 8-bit copy made once, offline (the channel
 * scales stay as they are).  N % 128 == 0, K % 128 == 0; qt 16-byte aligned; not in place. */
lora_status lora_pack_weight_t(int32_t w_fmt, const uint8_t* q, int32_t N, int32_t K, uint8_t* qt, void* stream);

/* Pack one adapter for lora_backward from A bf16 [K][r] and B bf16 [r][N] row-major:
 *   Bop: B_a in bf16 MFMA operand order over N -- the layout lora_pack_adapter gives A, with
 *        N in place of K: element (j, n) at ((((j/16) (N/64) + n/64) 2 + (n/8)%2) 64 +
 *        16 ((n/16)%4) + j%16) 8 + n%8, 16 ceil(r/16) N values;
 *   Ar:  A_a as bf16 [K][rank_pad(r)] row-major.
 * Padding ranks are zero.  1 <= r <= 64, N % 64 == 0; Bop and Ar 16-byte aligned; no buffer
 * may overlap another.  Like lora_pack_adapter, once per adapter (after each update of it). */
lora_status lora_pack_adapter_bwd(const uint16_t* A, const uint16_t* B, int32_t K, int32_t N, int32_t r,
                                  uint16_t* Bop, uint16_t* Ar, void* stream);

/* Gradients of the layer above with respect to x, A_a and B_a.
 *  - x bf16 [T][K], dy bf16 [T][N], t float [T][r_max] (the forward's down-projection, as
 *    lora_shrink or gemm_lowp_lora_epilogue write it; columns j >= r_a are not read);
 *  - wt_q: W^T packed by lora_pack_weight_t, w_scale float [N] (the FP8 channel scales);
 *  - adapter_id int32 [T], seg_indptr / sorted_tok from lora_build_segments;
 *  - Bop_ptrs / Ar_ptrs: per adapter, device addresses of Bop and Ar (lora_pack_adapter_bwd);
 *  - outputs: dx bf16 [T][K] (round to nearest even); u float [T][r_max] (dY B_a^T, with the
 *    layout of t); per adapter dA_a float [K][r_a] and dB_a float [r_a][N] row-major at the
 *    addresses in dA_ptrs / dB_ptrs, written, not accumulated into (zero for an adapter
 *    without tokens);
 *  - status: device int32 or NULL; bit 1 is OR-ed in when an adapter with tokens has a rank
 *    outside [1, r_max] (its dA_a and dB_a are not written and its tokens get dY W_d^T only);
 *  - workspace: device memory of lora_backward_workspace_bytes(T, K, N, n_adapters, r_max)
 *    bytes, 16-byte aligned (NULL where that is 0): short batches split dX's contraction and
 *    u's over N across workgroups and keep their fp32 partial sums there (added in a fixed
 *    order, so the result does not depend on the split's timing); LORA_ERR_WORKSPACE when it
 *    is missing or short.
 * Arithmetic: dY W_d^T = (dY diag(w_scale)) codes^T on bf16 MFMA: dY times the channel scale
 * rounded to bf16 (nearest even), the FP8 codes widened exactly, fp32 accumulation; u by the forward's
 * down-projection kernel (exact bf16 products, fp32 sums); the fp32 factors u, t of the
 * adapter products enter bf16 MFMAs as two bf16 terms each (about 17 bits).  Bitwise
 * deterministic.  Tokens whose adapter id is outside [0, n_adapters) get dY W_d^T only.
 * Limits: T <= 65536 (T == 0 zero-fills the dA_a and dB_a), K % 128 == 0, N % 128 == 0,
 * 1 <= r_max <= 64; x, dy, wt_q, w_scale, dx, u 16-byte aligned. */
lora_status lora_backward(const uint16_t* x, const uint16_t* dy, const float* t, int32_t T, int32_t K, int32_t N,
                          int32_t w_fmt, const uint8_t* wt_q, const float* w_scale, const int32_t* adapter_id,
                          const int32_t* seg_indptr, const int32_t* sorted_tok, const uint64_t* Bop_ptrs,
                          const uint64_t* Ar_ptrs, const int32_t* ranks, const float* scales, int32_t n_adapters,
                          int32_t r_max, uint16_t* dx, float* u, const uint64_t* dA_ptrs, const uint64_t* dB_ptrs,
                          int32_t* status, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lora_backward needs for these sizes: 0 where the 64-token x 256-column
 * tiles of dX fill the GPU (about 6,000 or more tokens at K = 4096) and T > 128; else the
 * fp32 partial sums of the split work: dX's contraction in up to 32 ranges of N (ranges x T x
 * K x 4 bytes) and, up to 128 tokens, u = dY B_a^T in up to 32 parts of N (parts x T x r_max x
 * 4 bytes).  0 for sizes or adapter counts lora_backward does not accept. */
size_t lora_backward_workspace_bytes(int32_t T, int32_t K, int32_t N, int32_t n_adapters, int32_t r_max);

/* Device-side status word of the layer calls on this workspace since it was last
 * initialised (bits accumulate): copies one int32 to *status_dev (device pointer) on
 * `stream`.  0 = fine; bit 0 = a bounded wait in the fused launch gave up (the output
 * is then unspecified); bit 1 = a token's adapter had a rank outside [1, r_max] (that
 * adapter's term was left out).  Cleared by lora_workspace_init. */
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

/*
 * fp8bs.h -- C ABI of the MI355X (gfx950) block-scaled FP8 W8A8 GEMM library.
 *
 * The method: activations are quantized per token in 1x128 groups to OCP e4m3
 * with power-of-two (UE8M0) scales packed four to a 32-bit word; weights are
 * e4m3 with one scale per 128x128 block; the GEMM accumulates in fp32, applying
 * the two scales to each 128-wide K-block before adding it, and writes bf16.
 * Sources: vLLM DeepGEMM FP8 block GEMM benchmark post (sections 4.1-4.2:
 * quantization layouts, the three dense GEMM calls and their preconditions);
 * vLLM PR #29546 "Deepgemm fused layout kernel for activations" (quant with the
 * uint32 scale pack fused in); vLLM PR #19885 "Optimize the little operations
 * in the DeepGEMM + DeepEP low latency case" (fused SiLU-mul-quant that skips
 * padded tokens); vLLM PR #19111 "Integrate batched/masked deepgemm kernel"
 * (masked grouped GEMM over [experts, max_tokens, K] with per-expert counts).
 *
 * Conventions shared by every entry point
 *   - Data pointers are DEVICE pointers owned by the caller.  bf16 is passed as
 *     its 16-bit pattern, e4m3 as bytes (OCP E4M3FN, max 448).
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).  Every
 *     call is asynchronous and stream-ordered; nothing reads device data on the
 *     host, so masked counts never leave the device.
 *   - Return value: FP8BS_OK (0) or a negative status; on error nothing is
 *     launched.  fp8bs_status_string() names a status; after FP8BS_ERR_LAUNCH,
 *     fp8bs_last_hip_error() gives the hipError_t of the failed call (per thread).
 *   - Sizes of zero are a successful no-op, except K (see each call).
 *   - Outputs must not overlap inputs.
 *   - Alignment: every data pointer and every row of an e4m3/bf16 tensor must be
 *     16-byte aligned (FP8BS_ERR_ALIGN otherwise); scale pointers 4-byte aligned.
 *   - The device must be gfx950 (FP8BS_ERR_DEVICE otherwise).
 *
 * Packed activation-scale layout ("sf"): for K columns there are G = K/128 groups
 * per row and W = ceil(G/4) words per row.  Group g's exponent byte (e + 127,
 * where the group's scale is 2^e) sits in bits 8*(g%4)..8*(g%4)+7 of word g/4;
 * bytes of groups past G are zero.  Words are stored M-major: word w of row r is
 * sf[w*ld_sf + r] (the column-major, padded layout the benchmark post's section
 * 4.1 describes for DeepGEMM; ld_sf = round_up(M, 4) gives 16-byte columns).
 * Weight block scales ("sfb") are fp32 [ceil(N/128)][K/128], row-major: the
 * UE8M0 values the weight block quant produces (powers of two).  Every UE8M0 entry
 * point, whatever kernel it picks, reads only each scale's exponent field, i.e.
 * uses 2^floor(log2 |s|): a power of two is used as it is, any other finite scale
 * is taken as the power of two at or below its magnitude (sign and mantissa bits
 * ignored).  The float-scale entry points (fp8_block_gemm_nt_float_scales...) use
 * the whole fp32 value.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FP8BS_OK = 0,
  FP8BS_ERR_NULL = -1,   /* a required pointer is NULL                              */
  FP8BS_ERR_SHAPE = -2,  /* a size or leading dimension is out of its allowed range */
  FP8BS_ERR_ALIGN = -3,  /* a pointer or row stride breaks the alignment rule       */
  FP8BS_ERR_DEVICE = -4, /* the current device is not gfx950                        */
  FP8BS_ERR_LAUNCH = -5, /* a HIP call failed; see fp8bs_last_hip_error()           */
  FP8BS_ERR_ALLOC = -6,  /* the split-K workspace could not be allocated            */
  FP8BS_ERR_SCRATCH = -7 /* fp8_block_gemm_nt_preshuffled_noalloc: scratch too small */
};

/*
 * Per-token 1x128 group quant with the UE8M0 scale pack in the same pass
 * (PR #29546, Purpose; benchmark post section 4.1, per_token_group_quant with
 * column-major, aligned scales).  For every row r < M and group g:
 *   e = smallest integer with 448 * 2^e >= max(amax of the group, 1e-10),
 *   q[r][k] = e4m3_rne_saturating(x[r][k] * 2^-e),  byte e + 127 into sf.
 *   x   : bf16 [M][ldx], ldx >= K
 *   q   : e4m3 [M][ldq], ldq >= K, ldq % 16 == 0
 *   sf  : uint32 [ceil(K/512)][ld_sf], ld_sf >= M; entries of rows >= M untouched
 *   K % 128 == 0.
 */
int fp8_quant_group_pack(const void* x, int64_t ldx, int64_t M, int64_t K,
                         void* q, int64_t ldq, uint32_t* sf, int64_t ld_sf, void* stream);

/*
 * Fused SiLU-and-mul + the quant/pack above over a masked expert batch
 * (PR #19885, Summary item 2: outputs in the GEMM's layout, padded tokens
 * neither loaded nor computed).  For e < E and r < clamp(masked_m[e], 0, M_max):
 *   y = silu(gate) * up = gate / (1 + exp(-gate)) * up, in fp32, with gate =
 *   x[e][r][0:H] and up = x[e][r][H:2H]; then 1x128 quant/pack of y.
 *   x        : bf16 [E][M_max][2H] contiguous
 *   masked_m : int32 [E] on the device (clamped to [0, M_max] in the kernel)
 *   q        : e4m3 [E][M_max][H] contiguous
 *   sf       : uint32 [E][ceil(H/512)][M_max] contiguous
 *   H % 128 == 0.  Rows r >= count of q and sf are left untouched.
 */
int silu_mul_quant_group_pack(const void* x, const int32_t* masked_m, int64_t E, int64_t M_max,
                              int64_t H, void* q, uint32_t* sf, void* stream);

/*
 * Float-scale (non-UE8M0) format (benchmark post section 4.1: the scale of a
 * group or block is amax / fp8_max, rounded up to a power of two only when UE8M0
 * is asked for).  In IEEE fp32 with correctly rounded division:
 *   s = max(amax, 1e-10f) / 448,  q = e4m3_rne(clamp(x / s, -448, 448)).
 * fp8_quant_group_float: 1x128 groups of bf16 x [M][ldx] (ldx >= K, ldx % 8 == 0)
 *   -> q e4m3 [M][ldq] (ldq % 16 == 0), sf fp32 [K/128][ld_sf], ld_sf >= M
 *   (one float per group, M-major; entries of rows >= M untouched).
 * fp8_block_quant_128x128_float: 128x128 blocks of bf16 w [N][K] -> q e4m3 [N][K],
 *   sfb fp32 [ceil(N/128)][K/128].
 * fp8_block_gemm_nt_float_scales: C[m][n] = bf16( sum over K-blocks kb of
 *   sfa[kb][m] * sfb[n/128][kb] * (e4m3 dot product of the block) ), fp32
 *   accumulation; sfa fp32 [K/128][ld_sfa], ld_sfa >= M; other arguments and
 *   preconditions as fp8_block_gemm_nt (the scales may be any finite fp32).
 */
int fp8_quant_group_float(const void* x, int64_t ldx, int64_t M, int64_t K, void* q, int64_t ldq,
                          float* sf, int64_t ld_sf, void* stream);
int fp8_block_quant_128x128_float(const void* w, int64_t N, int64_t K, void* q, float* sfb,
                                  void* stream);
/*
 * fp8_block_gemm_nt_float_scales with the weights b in the layout of
 * fp8_weight_preshuffle (rows = N); every other argument and the result are those of
 * fp8_block_gemm_nt_float_scales.  Runs the float-scale decode kernel at every M:
 * meant for decode-sized M (M <= 64).
 */
int fp8_block_gemm_nt_float_scales_preshuffled(const void* a, const float* sfa, int64_t ld_sfa,
                                                const void* b, const float* sfb, void* c, int64_t ldc,
                                                int64_t M, int64_t N, int64_t K, void* stream);
int fp8_block_gemm_nt_float_scales(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                   const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N,
                                   int64_t K, void* stream);

/*
 * Per-token group quant written into the masked expert layout of the routed
 * tokens: the quantization half of FP8 dispatch on one GPU (PR #19885, Summary
 * item 1: DeepEP quantizes and puts the scales in DeepGEMM's layout; PR #19111
 * review: the TODO asking for a batched quant).  Token t's choice j routes pair
 * p = t * topk + j to expert topk_ids[p]; its slot is the number of earlier pairs
 * (in p order) routed to the same expert.  Pairs whose id is outside [0, E) or
 * whose slot reaches M_max get slot -1 and are not written.  Every token is
 * quantized once, exactly as fp8_quant_group_pack quantizes a row, and its e4m3
 * row and scale words are written to row `slot` of its expert.
 *   x        : bf16 [T][ldx], ldx >= K, ldx % 8 == 0;  K % 128 == 0
 *   topk_ids : int32 [T][topk] on the device, 1 <= topk <= 64
 *   q        : e4m3 [E][M_max][K];   sf : uint32 [E][ceil(K/512)][M_max]
 *   masked_m : int32 [E] out: min(pairs routed to e, M_max)
 *   slot_of  : int32 [T][topk] out: the slot of every pair, or -1
 *   1 <= E <= 1024.  Rows at or past masked_m[e] of q and sf are left untouched.
 * Two launches on `stream`: one workgroup per 1024 pairs ranks the pairs, then the
 * quantization resolves the slots (deterministic) and reads every token once.  The
 * ranks and per-chunk counts (4 * (T * topk + ceil(T * topk / 1024) * E) bytes) go
 * to the library's per-(device, stream) workspace, allocated on the first call
 * that needs it (FP8BS_ERR_ALLOC during HIP graph capture, as for the GEMMs).
 */
int fp8_quant_group_pack_to_experts(const void* x, int64_t ldx, int64_t T, int64_t K,
                                    const int32_t* topk_ids, int32_t topk, int64_t E, int64_t M_max,
                                    void* q, uint32_t* sf, int32_t* masked_m, int32_t* slot_of,
                                    void* stream);

/*
 * 128x128 weight block quant (benchmark post section 4.1, per_block_cast with
 * UE8M0: scale = block amax / 448 rounded up to a power of two).
 *   w   : bf16 [N][K] contiguous;  q : e4m3 [N][K] contiguous
 *   sfb : fp32 [ceil(N/128)][K/128]; the last row block may be partial.
 *   K % 128 == 0.
 */
int fp8_block_quant_128x128(const void* w, int64_t N, int64_t K, void* q, float* sfb, void* stream);

/*
 * Dense block-scaled GEMM, NT form (benchmark post section 4.2, fp8_gemm_nt
 * writing into a preallocated output; preconditions there: bf16 output,
 * N % 64 == 0, K % 128 == 0):
 *   C[m][n] = bf16_rne( sum_kb 2^ea[m][kb] * sfb[n/128][kb]
 *                       * sum_{k in block kb} a[m][k] * b[n][k] )
 *   a   : e4m3 [M][K] contiguous;    sfa : packed scales [ceil(K/512)][ld_sfa], ld_sfa >= M
 *   b   : e4m3 [N][K] contiguous;    sfb : fp32 [ceil(N/128)][K/128]
 *   c   : bf16 [M][ldc], ldc >= N, ldc % 8 == 0
 *   K >= 128, K % 128 == 0, N % 64 == 0.
 * Decode-sized M splits K across workgroups; the split partials live in a
 * library-owned device workspace kept per (device, stream), allocated on the
 * first call that needs it (make that call outside HIP graph capture: during
 * capture an allocation is refused with FP8BS_ERR_ALLOC).  Calls on different
 * streams never share a workspace.  A workspace that a larger call outgrows is
 * replaced but never freed, so graphs captured earlier stay valid.  A captured
 * graph keeps the workspace of the stream it was captured on: replay it in
 * stream order with the other calls on that stream (a replay running at the same
 * time as calls on the capture stream would share the split-K partials with them,
 * and for the entries that reduce inside the kernel also the arrival counters).
 */
int fp8_block_gemm_nt(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                      const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                      void* stream);

/*
 * Offline weight layout for the decode GEMM.  The weights of a block-scaled GEMM
 * are prepared once, outside the timed step (benchmark post section 4.1 quantizes
 * B before timing); this library's own pre-shuffled layout is a byte permutation
 * of the e4m3 weights [rows][K] (same size) in which every 16-byte load of the
 * decode kernel reads one contiguous kilobyte:
 *   out[((g * KB + kb) * 4 + q) * 1024 + l * 16 + i]
 *     = w[32 g + (l & 31)][128 kb + 64 (q >> 1) + 32 (l >> 5) + 16 (q & 1) + i]
 * for g < rows/32, kb < KB = K/128, q < 4, l < 64, i < 16.  The block scales are
 * unchanged.  Expert weights [E][N][K] are shuffled as rows = E*N.
 *   w, out : device, 16-byte aligned, not overlapping;  rows % 32 == 0, K % 128 == 0.
 */
int fp8_weight_preshuffle(const void* w, int64_t rows, int64_t K, void* out, void* stream);

/*
 * fp8_block_gemm_nt with the weights b in the layout of fp8_weight_preshuffle
 * (rows = N); every other argument, the result and the workspace rules are those
 * of fp8_block_gemm_nt.  M <= 64 runs the weight-streaming kernel, whose loads this
 * layout makes contiguous; larger M the ring tiles of fp8_block_gemm_nt, each weight
 * DMA instruction then moving one contiguous kilobyte (bit-identical results; at
 * prefill sizes 1-6% shorter than fp8_block_gemm_nt on the plain layout).
 */
int fp8_block_gemm_nt_preshuffled(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                  const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N,
                                  int64_t K, void* stream);

/*
 * fp8_block_gemm_nt_preshuffled for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, kernels and result are those of
 * fp8_block_gemm_nt_preshuffled (bit-identical output); the split-K scratch
 * (arrival counters and fp32 partials) is a static device array of 8 MiB per GPU
 * instead of the per-stream workspace, so this call never allocates or frees.  For
 * M <= 64 and K <= 143360 (the weight-streaming kernel) the automatic configuration
 * needs at most 64 KiB + 224 * 64 * 128 * 4 bytes (7.4 MB), for larger M none; a
 * problem needing more than 8 MiB returns FP8BS_ERR_SCRATCH without launching.  Every call on one GPU shares that array:
 * calls that overlap on one GPU (different streams, or a graph replay running
 * beside another call) race and give undefined results.  The first call on a device
 * clears the counters with a fill kernel on its stream; every call leaves them clear.
 */
int fp8_block_gemm_nt_preshuffled_noalloc(const void* a, const uint32_t* sfa, int64_t ld_sfa,
                                          const void* b, const float* sfb, void* c, int64_t ldc,
                                          int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Masked grouped GEMM (PR #19111: m_grouped GEMM, masked, over [E, max_tokens, K]
 * with per-expert valid counts; 128x128 blocks).  For each expert e and row
 * r < clamp(masked_m[e], 0, M_max), row r of C[e] is the dense NT result of
 * a[e], sfa[e], b[e], sfb[e].  Rows at or past the count are not written, and
 * workgroup tiles that start past the count issue no loads and no MFMA.
 *   a        : e4m3 [E][M_max][K];      sfa : uint32 [E][ceil(K/512)][M_max]
 *   b        : e4m3 [E][N][K];          sfb : fp32 [E][ceil(N/128)][K/128]
 *   c        : bf16 [E][M_max][N];      masked_m : int32 [E] on the device
 *   K >= 128, K % 128 == 0, N % 64 == 0.
 */
int fp8_block_gemm_grouped_masked(const void* a, const uint32_t* sfa, const void* b,
                                  const float* sfb, void* c, const int32_t* masked_m, int64_t E,
                                  int64_t M_max, int64_t N, int64_t K, void* stream);

/*
 * fp8_block_gemm_grouped_masked with the expert weights b in the layout of
 * fp8_weight_preshuffle (rows = E*N, so each expert's [N][K] block is shuffled on
 * its own); every other argument and the result are those of
 * fp8_block_gemm_grouped_masked.  K <= 20480 (a masked group never splits K, and the
 * kernels reading this layout hold the scales of at most 160 K-blocks); larger K
 * returns FP8BS_ERR_SHAPE.
 */
int fp8_block_gemm_grouped_masked_preshuffled(const void* a, const uint32_t* sfa, const void* b,
                                              const float* sfb, void* c, const int32_t* masked_m,
                                              int64_t E, int64_t M_max, int64_t N, int64_t K,
                                              void* stream);

/*
 * Contiguous grouped GEMM, the layout of the high-throughput MoE path (PR #19111
 * page, changelog: the "High-Throughput" DeepEP + DeepGEMM test).  The pages name
 * that path only; the layout is read plainly: the rows of A and C are grouped by
 * expert in runs aligned to 128 rows, and m_indices[m] names the expert of row m
 * (-1 for padding).  Every aligned 128-row block holds rows of one expert followed
 * by padding rows, or padding only.  For every row m with 0 <= m_indices[m] < E,
 * row m of C is the dense NT result of a[m], sfa, b[m_indices[m]],
 * sfb[m_indices[m]].  A block whose first row is padding or names no expert in
 * [0, E) is skipped (no loads, no MFMA, C untouched); padding rows inside a block
 * of an expert are written with that expert's result (unspecified values).
 *   a         : e4m3 [M][K];            sfa : uint32 [ceil(K/512)][ld_sfa], ld_sfa >= M
 *   b         : e4m3 [E][N][K];         sfb : fp32 [E][ceil(N/128)][K/128]
 *   c         : bf16 [M][ldc], ldc >= N, ldc % 8 == 0
 *   m_indices : int32 [M] on the device (values outside [0, E) mean padding)
 *   K >= 128, K % 128 == 0, N % 64 == 0.
 */
int fp8_block_gemm_grouped_contiguous(const void* a, const uint32_t* sfa, int64_t ld_sfa,
                                      const void* b, const float* sfb, void* c, int64_t ldc,
                                      const int32_t* m_indices, int64_t E, int64_t M, int64_t N,
                                      int64_t K, void* stream);

/*
 * Tile-table access, for tuning and for tests that cover every compiled tile
 * shape.  fp8bs_gemm_config reports what the automatic choice would be for a
 * dense (masked = 0), masked (masked = 1), contiguous grouped (masked = 2),
 * dense float-scale (masked = 3), dense pre-shuffled-weight (masked = 4),
 * masked pre-shuffled-weight (masked = 5) or dense float-scale pre-shuffled-weight
 * (masked = 6) problem: kernel index into the tile
 * table, workgroup tile bm x bn, and the number of K splits.  The _cfg variants
 * run the same GEMMs with an explicit kernel index and split count (splits is
 * clamped to [1, K/128]; the masked and contiguous forms use splits == 1 only, and
 * the contiguous form only tiles of at most 128 rows).
 */
int fp8bs_gemm_config_count(void);
int fp8bs_gemm_config(int masked, int64_t M, int64_t N, int64_t K, int32_t* kernel, int32_t* bm,
                      int32_t* bn, int32_t* splits);
/* Whether table entry `kernel` accepts a dense (masked = 0), masked (masked = 1),
 * contiguous grouped (masked = 2), dense float-scale (masked = 3), dense
 * pre-shuffled-weight (masked = 4), masked pre-shuffled-weight (masked = 5) or dense
 * float-scale pre-shuffled-weight (masked = 6) problem of this
 * shape with `splits` K splits: FP8BS_OK with its workgroup tile and the split count
 * it would use, FP8BS_ERR_SHAPE if it does not (for instance K past the entry's scale
 * tables, a masked problem that would need K splits, or a scale format the entry does
 * not read).  Host-only; launches nothing. */
int fp8bs_gemm_config_of(int32_t kernel, int masked, int64_t M, int64_t N, int64_t K, int32_t splits,
                         int32_t* bm, int32_t* bn, int32_t* splits_out);
int fp8_block_gemm_nt_cfg(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                          const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                          int32_t kernel, int32_t splits, void* stream);
int fp8_block_gemm_grouped_masked_cfg(const void* a, const uint32_t* sfa, const void* b,
                                      const float* sfb, void* c, const int32_t* masked_m, int64_t E,
                                      int64_t M_max, int64_t N, int64_t K, int32_t kernel,
                                      void* stream);
int fp8_block_gemm_grouped_contiguous_cfg(const void* a, const uint32_t* sfa, int64_t ld_sfa,
                                          const void* b, const float* sfb, void* c, int64_t ldc,
                                          const int32_t* m_indices, int64_t E, int64_t M,
                                          int64_t N, int64_t K, int32_t kernel, void* stream);
int fp8_block_gemm_nt_float_scales_cfg(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                       const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N,
                                       int64_t K, int32_t kernel, int32_t splits, void* stream);
int fp8_block_gemm_nt_preshuffled_cfg(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                      const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N,
                                      int64_t K, int32_t kernel, int32_t splits, void* stream);
int fp8_block_gemm_nt_float_scales_preshuffled_cfg(const void* a, const float* sfa, int64_t ld_sfa,
                                                    const void* b, const float* sfb, void* c, int64_t ldc,
                                                    int64_t M, int64_t N, int64_t K, int32_t kernel,
                                                    int32_t splits, void* stream);
int fp8_block_gemm_grouped_masked_preshuffled_cfg(const void* a, const uint32_t* sfa, const void* b,
                                                  const float* sfb, void* c, const int32_t* masked_m,
                                                  int64_t E, int64_t M_max, int64_t N, int64_t K,
                                                  int32_t kernel, void* stream);

/* Status helpers. */
const char* fp8bs_status_string(int status);
int fp8bs_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */

/*
 * cq.h -- C ABI of libcq: block-quantized GGUF weight x activation matmul
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages cited by title and section):
 *   - Weights stay in GGUF block form as stored: Q4_0, Q4_1, Q8_0, Q4_K
 *     (Cera README, "Quantization"; alice-llm 2.0.0 README, "Quantization
 *     Block Specs"), Q5_K and Q6_K (same table; Cera README, "Quantization";
 *     Q6_K is the type of the tied-embedding LM head, Cera README,
 *     "Performance").  The LM head runs on the weight as stored, not on a
 *     dequantized copy (Cera README, "Performance").
 *   - Activations are quantized on the fly to Q8_0 blocks of 32 (Cera
 *     README, "Quantization"; alice-llm 2.0.0 README, "The CPU Optimization
 *     Journey", Phase 4).
 *   - Each output is an integer dot inside every 32-value block with the
 *     scales applied once per block (alice-llm 2.0.0 README, "Computation
 *     Path (Q4_K)").
 *   - Decode GEMV for 1..8 activation rows: the batched LM-head verify of
 *     speculative decoding reads the weights once for all 1+k rows (cera
 *     0.5.3 README, "Speculative decoding"; alice-llm 2.0.0 README,
 *     "Batch-4 Speculative Decoding").
 *   - Batched prefill GEMM (Cera README, "Supported models").
 *   - lfm2moe-style routed expert FFN with tokens grouped by expert so that
 *     each expert's weights are read once per chunk (Cera README,
 *     "Supported models", which names grouping as the follow-up), SwiGLU
 *     between the projections (alice-llm 2.0.0 README, "The GPU
 *     Optimization Journey", phase 4).
 *
 * Block layouts (little-endian fp16 fields):
 *   Q4_0  32 values, 18 B: d, 16 bytes; byte i = element i (low nibble) and
 *         element i+16 (high nibble); value d*(q-8).
 *   Q4_1  32 values, 20 B: d, m, 16 bytes as Q4_0; value d*q + m.
 *   Q8_0  32 values, 34 B: d, 32 int8; value d*q.
 *   Q4_K  256 values, 144 B: d, dmin, 12 bytes of six-bit sub-block scales
 *         and mins, 128 bytes of nibbles (32-byte chunk c: low nibbles =
 *         sub-block 2c, high nibbles = sub-block 2c+1); value d*sc*q - dmin*m.
 *   Q5_K  256 values, 176 B: d, dmin, 12 scale bytes as Q4_K, qh[32], then
 *         128 bytes of nibbles as Q4_K; bit j of qh[l] is bit 4 of element l
 *         of sub-block j (quants 0..31); value d*sc*q - dmin*m.
 *   Q1_0  128 values, 18 B: d, then 16 bytes of sign bits; value i is bit
 *         i % 8 of byte 2 + i/8 (LSB first), +d when set, -d when clear
 *         (alice-llm 2.0.0 README, Bonsai 27B notes).  GEMV entry points only.
 *   TQ2   128 values, 34 B: d, then 32 bytes of 2-bit codes, four per byte;
 *         value i is code (byte 2 + i/4 >> 2*(i%4)) & 3, low pair first;
 *         codes 00, 01, 11 give 0, +d, -d (alice-llm 2.0.0 README, "Sparse
 *         Ternary Quantization"); 10, which that encoding never writes,
 *         reads as 0.  GEMV entry points only.
 *   Q6_K  256 values, 210 B: ql[128], qh[64], 16 signed 8-bit scales, d.
 *         In half h (128 values), element l + 32g (l < 32, quadrant g) takes
 *         a nibble of ql[64h + l] (g = 0 low, g = 2 high) or ql[64h + 32 + l]
 *         (g = 1 low, g = 3 high), bit pair g of qh[32h + l] as bits 4-5,
 *         and scale 8h + 2g + l/16; value d*scale*(q-32).
 *   A weight matrix [n][k] is n rows of k/qk consecutive blocks, row-major,
 *   no padding.  MoE expert weights are n_experts such matrices back to back.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  They must stay valid until the
 *     stream reaches the call.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     legacy default stream), performs no host synchronization, and keeps no
 *     state between calls apart from a read-only per-device property cache.
 *     Calls are thread-safe.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call returns a negative cq_status and launches nothing.  Faults
 *     raised by the GPU surface at the caller's next synchronization.
 *   - Sizes of zero (n, rows, m, n_tokens) are valid and launch nothing.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs on every run (no floating-point atomics).
 */
#ifndef CQ_H
#define CQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t (HIP declares hipStream_t as this same pointer type). */
typedef struct ihipStream_t* cq_stream_t;

/* Status codes: append-only, never renumbered. */
typedef enum {
    CQ_OK = 0,
    CQ_ERR_INVALID_ARG = -1,      /* null pointer, negative size, bad flag   */
    CQ_ERR_UNSUPPORTED_TYPE = -2, /* weight type not supported by the call   */
    CQ_ERR_SHAPE = -3,            /* k not a multiple of the block, too big  */
    CQ_ERR_ALIGNMENT = -4,        /* pointer or leading dim misaligned       */
    CQ_ERR_WORKSPACE = -5,        /* caller workspace too small or misaligned */
    CQ_ERR_HIP = -6,              /* a HIP runtime call failed               */
    CQ_ERR_NO_DEVICE = -7,        /* no gfx950 device current                */
    CQ_ERR_SCRATCH_LIMIT = -8     /* exceeds the fixed no-allocation scratch */
} cq_status;

/* Weight types, numbered as the GGUF tensor type ids. */
typedef enum { CQ_Q4_0 = 2, CQ_Q4_1 = 3, CQ_Q8_0 = 8, CQ_Q4_K = 12, CQ_Q5_K = 13,
               CQ_Q6_K = 14,
               CQ_Q1_0 = 41, /* library-assigned: the pages give no GGUF id */
               CQ_TQ2 = 42   /* library-assigned: the pages give no GGUF id */ } cq_type;

#define CQ_ABI_VERSION 2
#define CQ_GEMV_MAX_BATCH 8
#define CQ_MAX_K 65536
#define CQ_GEMV_MAX_K 32768   /* cq_gemv: up to 8 waves of 64 lanes per row */

int cq_abi_version(void);
/* Static, never-null string naming a status code. */
const char* cq_status_string(int status);
/* Values per block, bytes per block, bytes per row of k values; -1 for an
 * unknown type or a k that is not a whole number of blocks. */
int64_t cq_block_elems(int type);
int64_t cq_block_bytes(int type);
int64_t cq_row_bytes(int type, int64_t k);

/*
 * cq_quantize_q8_0 -- dynamic activation quantization to Q8_0.
 * (alice-llm 2.0.0 README, "The CPU Optimization Journey", Phase 4: block
 * amax, scale 127/amax, multiply, round to nearest even, saturate.)
 *
 * For each row r < rows and each block b < k/32 of the 32 fp32 values
 * x[r*ldx + 32b .. +31]:
 *     amax = max |x_i|;  id = 127.0f / amax;  q_i = rne(x_i * id) clamped to
 *     [-127, 127] (a zero x_i gives 0 even if id overflows);
 *     d = fp16_rne(amax / 127.0f); block = d (2 B LE) then q_0..q_31.
 * All arithmetic is single IEEE fp32 operations, so the bytes are exact and
 * reproducible on any IEEE machine.
 *   x    fp32 [rows][ldx], 16-byte aligned, ldx % 4 == 0, ldx >= k.
 *   xq   out: rows*(k/32) blocks of 34 bytes, contiguous, 2-byte aligned.
 *   k    multiple of 32, k <= CQ_MAX_K.
 * Inputs with NaN or Inf are outside the contract.
 */
int cq_quantize_q8_0(const float* x, int64_t ldx, int64_t rows, int64_t k,
                     void* xq, cq_stream_t stream);

/*
 * cq_gemv -- decode GEMV for 1..8 activation rows (speculative verify
 * rows included): y[b*ldy + i] = sum_j w_hat[i][j] * x_hat[b][j].
 *   wt     CQ_Q4_0 / CQ_Q4_1 / CQ_Q8_0 / CQ_Q4_K / CQ_Q5_K / CQ_Q6_K / CQ_Q1_0 /
 *          CQ_TQ2.
 *   w      [n][k/qk] blocks, 16-byte aligned.
 *   xq     [batch][k/32] Q8_0 blocks (as written by cq_quantize_q8_0),
 *          2-byte aligned.
 *   batch  1..CQ_GEMV_MAX_BATCH.
 *   y      fp32, row b at y + b*ldy, ldy >= n, 4-byte aligned.
 *   k      multiple of 32 (of 256 for Q4_K, Q5_K and Q6_K; of 128 for Q1_0 and TQ2),
 *          k <= CQ_GEMV_MAX_K (a longer row returns CQ_ERR_SHAPE).
 * Each row b of a batched call is bitwise equal to the batch-1 call on that
 * row alone.  Accuracy: |y - y_exact| <= 2e-5 * sum_j |w_hat*x_hat|.
 */
int cq_gemv(int wt, const void* w, int64_t n, int64_t k,
            const void* xq, int64_t batch, float* y, int64_t ldy,
            cq_stream_t stream);

/*
 * cq_gemv_swiglu -- fused decode FFN front half for 1..8 activation rows:
 *     h[b*ldh + i] = silu(g) * u,  g = sum_j Wg_hat[i][j] * x_hat[b][j],
 *                                  u = sum_j Wu_hat[i][j] * x_hat[b][j],
 * silu(z) = z / (1 + exp(-z)) evaluated in fp64 from the fp32 g and u and
 * rounded once to fp32 (alice-llm 2.0.0 README, "The GPU Optimization
 * Journey", phase 4: gate + up + silu x mul in one pass that shares the
 * activation read).  One kernel streams the gate and up rows of each output
 * in turn; g and u are bitwise the values cq_gemv returns for the two
 * matrices, so h equals SwiGLU of those up to the fp64 exp's last bit.
 *   wt          any cq_gemv type; w_gate, w_up [n][k/qk] blocks, 16-byte
 *               aligned (both matrices of the same type and shape).
 *   xq          [batch][k/32] Q8_0 blocks, 16-byte aligned.
 *   h           fp32, row b at h + b*ldh, ldh >= n, 4-byte aligned.
 *   Shapes: whole 16-byte weight rows (k a multiple of 256; Q6_K: k a
 *   multiple of 2048) with k <= 16384 (up to 4096 one wave per row, longer
 *   rows split over two or four waves); other shapes return CQ_ERR_SHAPE
 *   (use cq_gemv twice and
 *   cq_swiglu_quantize_q8_0).  An xq not 16-byte aligned returns
 *   CQ_ERR_ALIGNMENT.
 */
int cq_gemv_swiglu(int wt, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                   const void* xq, int64_t batch, float* h, int64_t ldh,
                   cq_stream_t stream);

/*
 * cq_gemm -- prefill GEMM over m activation rows:
 *     y[r*ldy + i] = sum_j w_hat[i][j] * x_hat[r][j]
 * computed as int8 MFMA products of each 32-value block with the two block
 * scales applied per block in fp32.
 *   wt     CQ_Q4_0 / CQ_Q4_1 / CQ_Q8_0 / CQ_Q4_K / CQ_Q5_K / CQ_Q6_K (Q6_K:
 *          one K = 16 MFMA step per 16-value scale group; its weight matrix
 *          must be under 2 GiB, else CQ_ERR_SHAPE).
 *   w      [n][k/qk] blocks, 16-byte aligned; xq [m][k/32] Q8_0 blocks,
 *          4-byte aligned; y fp32 [m][ldy], ldy >= n, 4-byte aligned.
 *   k      multiple of 256, k <= CQ_MAX_K.
 * Accuracy as cq_gemv.
 */
int cq_gemm(int wt, const void* w, int64_t n, int64_t k,
            const void* xq, int64_t m, float* y, int64_t ldy,
            cq_stream_t stream);

/*
 * Flags of cq_moe_gemm (one value from each pair, OR-ed):
 *   CQ_MOE_X_PER_TOKEN  pair p = t*top_k + s reads activation row t of xq
 *                       (the gate and up projections);
 *   CQ_MOE_X_PER_PAIR   pair p reads activation row p (the down projection,
 *                       whose input is the pair's own SwiGLU output);
 *   CQ_MOE_OUT_PER_PAIR y row p = the pair's product row;
 *   CQ_MOE_OUT_COMBINE  y row t = sum over s = 0..top_k-1, in slot order, of
 *                       route_w[t*top_k + s] times the pair's product row
 *                       (fp32), the routed FFN's output.
 */
#define CQ_MOE_X_PER_TOKEN 0
#define CQ_MOE_X_PER_PAIR 1
#define CQ_MOE_OUT_PER_PAIR 0
#define CQ_MOE_OUT_COMBINE 2

/*
 * cq_moe_workspace_bytes -- device workspace cq_moe_gemm needs: a status
 * word, the grouping of the n_tokens*top_k pairs by expert, and with
 * CQ_MOE_OUT_COMBINE the fp32 product rows [n_tokens*top_k][n] that the
 * slot-order combine reads (a deterministic sum without floating-point
 * atomics needs every product before the first addition).  0 on bad sizes
 * or flags.
 */
size_t cq_moe_workspace_bytes(int64_t n_tokens, int64_t top_k, int64_t n_experts, int64_t n,
                              int flags);

/*
 * cq_moe_gemm -- one routed-expert projection of a chunk of tokens, grouped
 * so that each expert's weight matrix is read once for all of its pairs
 * (Cera README, "Supported models": lfm2moe routes each token to its own 4
 * of 32 experts, and grouping tokens by expert is the follow-up it names;
 * alice-llm 2.0.0 README, "The GPU Optimization Journey", phase 6: no
 * allocation per call, the caller owns the workspace).  For every pair
 * p = t*top_k + s with e = expert_ids[p]:
 *     P[p][i] = sum_j W_e_hat[i][j] * x_hat[row][j],  i < n,
 * row = t (CQ_MOE_X_PER_TOKEN) or p (CQ_MOE_X_PER_PAIR); then y[p*ldy + i]
 * = P[p][i] (CQ_MOE_OUT_PER_PAIR) or y[t*ldy + i] = sum_s route_w[p] *
 * P[p][i] in slot order (CQ_MOE_OUT_COMBINE).
 *   wt          CQ_Q4_0 / CQ_Q4_1 / CQ_Q8_0 / CQ_Q4_K / CQ_Q5_K / CQ_Q6_K
 *               (Q6_K: each expert's matrix under 2 GiB, else CQ_ERR_SHAPE).
 *   w_experts   n_experts matrices [n][k/qk] back to back, 16-byte aligned.
 *   xq          Q8_0 rows of k/32 blocks (n_tokens rows, or n_tokens*top_k
 *               rows with CQ_MOE_X_PER_PAIR), 2-byte aligned.
 *   expert_ids  device int32 [n_tokens][top_k].
 *   route_w     device fp32 [n_tokens][top_k]; read only with
 *               CQ_MOE_OUT_COMBINE (may be NULL otherwise).
 *   y           fp32, rows of ldy >= n: n_tokens*top_k rows (per pair) or
 *               n_tokens rows (combined), 4-byte aligned.
 *   workspace   device memory, 256-byte aligned, ws_bytes >=
 *               cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags),
 *               else CQ_ERR_WORKSPACE.  Scratch, overwritten by each call;
 *               calls that share a workspace must be ordered on one stream.
 *   n_experts 1..1024, top_k 1..n_experts, n_tokens*top_k <= 2^24,
 *   k a multiple of 256, k <= CQ_MAX_K.  Accuracy as cq_gemv.
 * Expert ids live on the device and cannot be checked before the launch.
 * After the stream reaches the call, the int32 at workspace offset 0 holds
 * the number of ids outside [0, n_experts): 0 means every result is
 * complete; otherwise those pairs were computed by no expert (a combined
 * row leaves their slots out, a per-pair row of theirs is left unwritten)
 * and the caller must treat the call as failed.
 */
int cq_moe_gemm(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                const void* xq, int flags, const int32_t* expert_ids, const float* route_w,
                int64_t n_tokens, int64_t top_k, float* y, int64_t ldy, void* workspace,
                size_t ws_bytes, cq_stream_t stream);

/*
 * cq_moe_gemm_noalloc -- cq_moe_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and results, with the workspace in a
 * fixed scratch array that the library holds on each GPU it runs on from
 * first use until the process ends, and the status word (the number of
 * expert ids outside [0, n_experts), stored by the call) in the caller's
 * `status` (device int32, 4-byte aligned).  The call allocates and frees
 * nothing.
 *   Limit: cq_moe_workspace_bytes(n_tokens, top_k, n_experts, n, flags) must
 *   not exceed CQ_MOE_NOALLOC_MAX_BYTES (16 MiB, e.g. 2048 pairs of 2048
 *   combined outputs), else CQ_ERR_SCRATCH_LIMIT and nothing is launched.
 *   Every call on one GPU uses that GPU's one scratch array: calls on
 *   different streams that overlap in time race and give wrong results;
 *   order them on one stream (or with events).  The array keeps the last
 *   call's contents; each call writes everything it later reads.
 * Other arguments, results and errors as cq_moe_gemm.
 */
#define CQ_MOE_NOALLOC_MAX_BYTES (16 << 20)
int cq_moe_gemm_noalloc(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                        const void* xq, int flags, const int32_t* expert_ids,
                        const float* route_w, int64_t n_tokens, int64_t top_k,
                        float* y, int64_t ldy, int32_t* status, cq_stream_t stream);

/*
 * The routed projection in separate steps (cq_moe_gemm runs these three on
 * its workspace), for callers that share one grouping between the gate, up
 * and down projections:
 *
 * cq_moe_group -- group the (token, slot) pairs of a top-k routing table by
 * expert (stable counting sort).
 *   expert_ids  int32 [n_tokens][top_k].
 *   offsets     out int32 [n_experts + 1]: pairs of expert e are
 *               pairs[offsets[e] .. offsets[e+1]).
 *   pairs       out int32 [n_tokens*top_k]: pair ids p = t*top_k + s,
 *               ascending within each expert.
 *   status      out device int32: the number of ids outside [0, n_experts)
 *               (such pairs are in no group; 0 when the grouping is whole).
 *   n_experts <= 1024, top_k <= n_experts, n_tokens*top_k <= 2^24.
 */
int cq_moe_group(const int32_t* expert_ids, int64_t n_tokens, int64_t top_k,
                 int64_t n_experts, int32_t* offsets, int32_t* pairs, int32_t* status,
                 cq_stream_t stream);

/*
 * cq_moe_gemm_grouped -- the grouped product of cq_moe_gemm on a grouping
 * written by cq_moe_group.  For every expert e and every pair p in
 * pairs[offsets[e] .. offsets[e+1]):
 *     y[p*ldy + i] = sum_j W_e_hat[i][j] * x_hat[row][j],  i < n,
 * where row = p / top_k (x_per_pair = 0: gate/up read the token row) or
 * row = p (x_per_pair = 1: down reads the pair row).
 *   Types, w_experts, xq, k as cq_moe_gemm; y fp32 [n_tokens*top_k][ldy].
 */
int cq_moe_gemm_grouped(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                        const void* xq, int x_per_pair, const int32_t* offsets,
                        const int32_t* pairs, int64_t n_tokens, int64_t top_k,
                        float* y, int64_t ldy, cq_stream_t stream);

/*
 * cq_moe_gemm_grouped2 -- two grouped products of the same gathered
 * activation rows in one call (the routed FFN's gate and up projections,
 * which read the same token rows): y_a as cq_moe_gemm_grouped gives for
 * w_a_experts, y_b for w_b_experts, bit for bit.  Where one launch can serve
 * both (Q4_K at k = 1536 or 2048), each expert's activation rows are split
 * into the tile once for both matrices; otherwise the two products run one
 * after the other.  (Cera README, "Supported models": lfm2moe's routed FFN,
 * gate and up projections of each chosen expert followed by SwiGLU.)
 *   w_a_experts, w_b_experts  device, the layout of cq_moe_gemm_grouped's
 *                 w_experts (the same type and shape).
 *   y_a, y_b      out device fp32 [n_tokens*top_k][ldy] each; the two may not
 *                 overlap (CQ_ERR_INVALID_ARG).
 *   Other arguments, results and errors as cq_moe_gemm_grouped.
 */
int cq_moe_gemm_grouped2(int wt, const void* w_a_experts, const void* w_b_experts,
                         int64_t n_experts, int64_t n, int64_t k, const void* xq, int x_per_pair,
                         const int32_t* offsets, const int32_t* pairs, int64_t n_tokens,
                         int64_t top_k, float* y_a, float* y_b, int64_t ldy, cq_stream_t stream);

/*
 * cq_moe_gemv -- routed experts at decode: the same product as cq_moe_gemm
 * for a few tokens, taken straight from the routing table, one GEMV per
 * token-expert pair p = t*top_k + s (no grouping call):
 *     y[p*ldy + i] = sum_j W_e_hat[i][j] * x_hat[row][j],  e = expert_ids[p],
 * row = p / top_k (x_per_pair = 0) or p (x_per_pair = 1).  Each pair
 * streams its expert's matrix once, so an expert chosen by two pairs is read
 * twice: meant for decode and verify batches (Cera README, "Supported
 * models": lfm2moe's routed FFN; 1 token x top-4), where the grouped MFMA
 * path would run 16-token tiles with one live row.
 *   expert_ids  device int32 [n_tokens][top_k].
 *   status      device int32, an error counter the caller zeroes once: each
 *               pair whose id lies outside [0, n_experts) adds 1 to it, and
 *               its output row is set to 0 (no weights are read for it).
 *               The library never clears it, so one check after many calls
 *               covers them all (and graph replays need no reset node).
 *   xq          Q8_0 rows, 16-byte aligned; y fp32 [n_tokens*top_k][ldy].
 *   Shapes: as cq_gemv_swiglu with one wave per row only (k <= 4096),
 *   n_tokens*top_k <= 65535; else CQ_ERR_SHAPE.
 */
int cq_moe_gemv(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                const void* xq, int x_per_pair, const int32_t* expert_ids,
                int64_t n_tokens, int64_t top_k, float* y, int64_t ldy, int32_t* status,
                cq_stream_t stream);

/*
 * cq_moe_gemv_swiglu -- cq_moe_gemv over the gate and up expert matrices
 * fused with SwiGLU, as cq_gemv_swiglu per pair (x row = the pair's token):
 *     h[p*ldh + i] = silu(g) * u for the pair's expert.
 * status as cq_moe_gemv (an invalid id gives h = 0 for its pair).
 */
int cq_moe_gemv_swiglu(int wt, const void* w_gate_experts, const void* w_up_experts,
                       int64_t n_experts, int64_t n, int64_t k, const void* xq,
                       const int32_t* expert_ids, int64_t n_tokens, int64_t top_k,
                       float* h, int64_t ldh, int32_t* status, cq_stream_t stream);

/*
 * cq_argmax_workspace_bytes -- bytes of device workspace cq_argmax needs for
 * rows x n logits (8 bytes per 4096-value chunk of each row); 0 on bad
 * sizes.
 */
size_t cq_argmax_workspace_bytes(int64_t rows, int64_t n);

/*
 * cq_argmax -- greedy token choice on the device: idx[r] = the first index of
 * the largest of y[r*ldy + 0 .. n-1] (cera 0.5.3 README, "Speculative
 * decoding": the greedy verify compares arg-max tokens; Cera README,
 * "Performance": the verify then reads 4 bytes per row instead of the
 * logits).  -0 and +0 compare equal; rows must hold no NaN.  Deterministic
 * (a maximum of (value, first index) keys).
 *   y          fp32, 4-byte aligned (16-byte aligned rows read faster).
 *   rows       0..65535; n 1..2^31-1; ldy >= n.
 *   idx        int32 [rows].
 *   workspace  caller device memory, 8-byte aligned, ws_bytes >=
 *              cq_argmax_workspace_bytes(rows, n) (else CQ_ERR_WORKSPACE);
 *              its contents are scratch, overwritten by each call.
 */
int cq_argmax(const float* y, int64_t rows, int64_t n, int64_t ldy, int32_t* idx,
              void* workspace, size_t ws_bytes, cq_stream_t stream);

/*
 * cq_topk_softmax -- the expert router (Cera README, "Supported models":
 * each token picks its own top_k of n_experts): ids[t][0..top_k) = the
 * top_k largest logits of row t in descending order (equal logits: smaller
 * expert id first) and w[t][s] = their softmax over the chosen top_k only,
 * exp(l_s - l_0) / sum_j exp(l_j - l_0) in fp64 summed in slot order,
 * rounded once to fp32.  The output feeds cq_moe_group / cq_moe_gemv
 * (ids) and cq_moe_gemm / cq_moe_combine (w).
 *   logits     fp32 [rows][ld], ld >= n_experts, 4-byte aligned, no NaN.
 *   n_experts  1..1024; top_k 1..min(16, n_experts).
 *   ids        int32 [rows][top_k]; w fp32 [rows][top_k].
 */
int cq_topk_softmax(const float* logits, int64_t rows, int64_t n_experts, int64_t ld,
                    int64_t top_k, int32_t* ids, float* w, cq_stream_t stream);

/*
 * cq_swiglu_quantize_q8_0 -- h = silu(g) * u with silu(z) = z/(1+exp(-z))
 * (alice-llm 2.0.0 README, "The GPU Optimization Journey", phase 4: fused
 * gate/up SwiGLU), evaluated in fp64 from the fp32 inputs and rounded once
 * to fp32, then quantized to Q8_0 exactly as cq_quantize_q8_0.
 *   g, u   fp32 [rows][k], contiguous, 16-byte aligned.
 *   h_opt  optional fp32 [rows][k] output of h (NULL to skip), 16-byte
 *          aligned.
 *   hq     out: rows*(k/32) Q8_0 blocks, 2-byte aligned.
 *   k      multiple of 32, k <= CQ_MAX_K.
 */
int cq_swiglu_quantize_q8_0(const float* g, const float* u, int64_t rows, int64_t k,
                            float* h_opt, void* hq, cq_stream_t stream);

/*
 * cq_moe_combine -- y[t*ldy + i] = sum over s = 0..top_k-1, in slot order,
 * of route_w[t*top_k + s] * d[(t*top_k + s)*n + i], fp32.
 *   d  fp32 [n_tokens*top_k][n] (as written by cq_moe_gemm_grouped or
 *      cq_moe_gemv with ldy = n).
 */
int cq_moe_combine(const float* d, const float* route_w, int64_t n_tokens,
                   int64_t top_k, int64_t n, float* y, int64_t ldy,
                   cq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CQ_H */

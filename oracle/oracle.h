/*
 * oracle.h -- plain CPU reference for the block-quantized GGUF matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
 * __graft_entry__.py and the CPU-baseline leg of bench.py may load or call
 * this library.  The product path (libcq) never links, loads or calls it,
 * and the two share no source, header, table or helper.
 *
 * Everything here is deliberately slow and literal: each weight block is
 * decoded to exact fp64 values, activations are decoded the same way, and
 * dot products are accumulated in fp64.  Sources for what is computed:
 *
 *   [alice-QBS]   alice-llm 2.0.0 README, "Quantization Block Specs" table:
 *                 a Q8_0 block is 34 bytes for 32 values (an fp16 scale
 *                 then 32 signed bytes); a Q4_K super-block is 144 bytes for
 *                 256 values (fp16 d, fp16 dmin, 12 packed scale bytes, 128
 *                 bytes of 4-bit quants).
 *   [alice-Q4K]   alice-llm 2.0.0 README, "Computation Path (Q4_K)": eight
 *                 32-value sub-blocks, each with a six-bit scale and a
 *                 six-bit min; the dot is integer inside each sub-block and
 *                 the scales enter only at the end, as d*dx*(sum of
 *                 sc*q*qx) minus dmin*dx*(sum of m * activation sums).
 *   [alice-P4]    alice-llm 2.0.0 README, "The CPU Optimization Journey",
 *                 Phase 4 (i8 dynamic quantization): amax, scale = 127/amax,
 *                 multiply, round to nearest (ties to even), saturate.
 *   [cera-Q]      Cera README, "Quantization": weights in Q4_0, Q4_1, Q8_0,
 *                 Q4_K; activations dynamically quantized to Q8_0.
 *   [cera-MoE]    Cera README, "Supported models": lfm2moe's routed FFN,
 *                 each token picks its own 4 of 32 experts; grouping tokens
 *                 by expert is the stated follow-up.
 *   [alice-GPU]   alice-llm 2.0.0 README, "The GPU Optimization Journey",
 *                 phase 4: fused SwiGLU (gate + up + silu x mul).
 *   [cera-V]      cera 0.5.3 README, "Speculative decoding", and Cera README,
 *                 "Performance": greedy verification compares the target's
 *                 arg-max token with the draft, and keeping the arg-max on
 *                 the device reads a few bytes instead of the full logits.
 *   [cera-R]      Cera README, "Supported models": lfm2moe routes each token
 *                 to its own 4 of 32 experts.
 *   [alice-Q10]   alice-llm 2.0.0 README, "Bonsai 27B" notes: Q1_0 packs 128
 *                 values in 18 bytes, an fp16 scale d then 16 bytes of 1-bit
 *                 weights, each value +d or -d (1.125 bits per weight).
 *   [alice-Q5K]   alice-llm 2.0.0 README, "Quantization Block Specs" table:
 *                 a Q5_K super-block is 176 bytes for 256 values (5.5 bpw),
 *                 fields d (fp16), dmin (fp16), scales[12], qh[32], qs[128].
 *   [alice-TQ]    alice-llm 2.0.0 README, "Sparse Ternary Quantization" and
 *                 "The CPU Optimization Journey", Phase 5: packed 2-bit
 *                 weights, four per byte, 00 = 0, 01 = +1, 11 = -1, expanded
 *                 through a table [0, +1, 0, -1]; N:M structured sparsity
 *                 (8 non-zero of every 16 values).
 *   [alice-Q6K]   alice-llm 2.0.0 README, "Quantization Block Specs" table:
 *                 a Q6_K super-block is 210 bytes for 256 values, fields
 *                 ql[128], qh[64], scales[16], d (fp16); and the NEON matvec
 *                 design notes: the two high bits of each quant come from qh
 *                 through the shift-masks (qh<<4)&0x30, (qh<<2)&0x30,
 *                 qh&0x30 and (qh>>2)&0x30, one per quadrant.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - Q4_0 block: fp16 d, then 16 bytes; byte i holds element i in its low
 *     nibble and element i+16 in its high nibble; value d*(q-8).
 *   - Q4_1 block: fp16 d, fp16 m, then 16 bytes in the Q4_0 nibble order;
 *     value d*q + m.
 *   - Q4_K: the 12 scale bytes pack 8 six-bit scales and 8 six-bit mins
 *     (see oracle_q4k_scale_min); qs chunk c (32 bytes) holds sub-block 2c
 *     in low nibbles and sub-block 2c+1 in high nibbles.  Value
 *     d*sc*q - dmin*m.
 *   - Q1_0: value i of the block is bit (i % 8) of byte 2 + i/8 (least
 *     significant bit first); a set bit is +d, a clear bit -d.
 *   - Q5_K: d, dmin and the 12 scale bytes as in Q4_K (same six-bit
 *     scale/min packing); qs chunk c (32 bytes) holds the low four bits of
 *     sub-block 2c in low nibbles and of sub-block 2c+1 in high nibbles, as
 *     in Q4_K; bit j of qh[l] (l in 0..31) is bit 4 of element l of
 *     sub-block j.  Quants 0..31, value d*sc*q - dmin*m.  This is the GGUF
 *     layout (the pages give only the fields and their sizes).
 *   - Q6_K: each 128-value half h uses ql[64h..64h+63], qh[32h..32h+31]
 *     and scales[8h..8h+7].  For l in 0..31 the 6-bit quants of elements
 *     l, l+32, l+64, l+96 of the half are the low nibble of ql[l], the low
 *     nibble of ql[l+32], the high nibble of ql[l], the high nibble of
 *     ql[l+32], each joined with bit pair 0-1, 2-3, 4-5, 6-7 of qh[l] as bits
 *     4-5 (the four shift-masks above); element l + 32*g takes the signed
 *     scale byte scales[8h + 2g + l/16]; value d*scale*(q-32).  This is the
 *     GGUF layout, so real GGUF tensors decode as stored.
 *   - TQ2 (2-bit ternary): 128 values in 34 bytes, an fp16 scale d then
 *     32 bytes of 2-bit codes, four per byte; value i is code
 *     (byte 2 + i/4 >> 2*(i%4)) & 3, least significant pair first.  Codes
 *     00, 01, 11 are 0, +1, -1 [alice-TQ]; code 10, which the encoding never
 *     produces, reads as 0 (the expansion table printed with it maps index 2
 *     to 0).  Value = d * code value.  The pages print no scale placement;
 *     one scale per 128 values (the Q1_0 block size) is the reading taken.
 *   - Greedy arg-max: the first index of the largest value (NaN-free rows;
 *     -0 and +0 compare equal).
 *   - Router: the top_k largest logits in descending order (equal logits:
 *     smaller expert id first) and their softmax over those top_k only,
 *     evaluated in fp64 and rounded once to fp32.
 *   - fp16 is IEEE-754 binary16, little-endian, subnormals honoured.
 *   - Q8_0 quantization: see oracle_quantize_q8_0.
 *   - SwiGLU: h = silu(gate) * up, silu(z) = z / (1 + exp(-z)), evaluated
 *     in fp64 and rounded once to fp32.
 *
 * Status codes: 0 = ok, -1 = bad argument, -2 = unknown type, -3 = shape.
 */
#ifndef CQ_ORACLE_H
#define CQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORACLE_Q4_0 = 2,
    ORACLE_Q4_1 = 3,
    ORACLE_Q8_0 = 8,
    ORACLE_Q4_K = 12,
    ORACLE_Q5_K = 13,
    ORACLE_Q1_0 = 41,   /* library-assigned id (the pages give no GGUF type id) */
    ORACLE_Q6_K = 14,
    ORACLE_TQ2 = 42     /* 2-bit ternary, library-assigned id */
};

int oracle_abi_version(void);

/* Elements and bytes per block of a weight type; -1 for an unknown type. */
int64_t oracle_block_elems(int type);
int64_t oracle_block_bytes(int type);

/* IEEE binary16 -> exact fp64 value (all 65536 encodings, NaN kept as NaN). */
double oracle_half_to_double(uint16_t h);
/* fp32 -> binary16, round to nearest, ties to even, subnormals and overflow
 * to infinity included.  NaN becomes a quiet NaN carrying the top payload
 * bits.  */
uint16_t oracle_float_to_half(float f);
void oracle_half_to_double_n(const uint16_t* h, int64_t n, double* out);
void oracle_float_to_half_n(const float* f, int64_t n, uint16_t* out);

/* Q4_K: six-bit scale and min of sub-block j (0..7) from the 12 packed
 * bytes. */
void oracle_q4k_scale_min(const uint8_t* scales12, int j, int* sc, int* mn);

/* Decode n_elems consecutive elements (a whole number of blocks) of a
 * block-quantized tensor to exact fp64 values. */
int oracle_dequantize(int type, const uint8_t* blocks, int64_t n_elems, double* out);

/* Q8_0 activation quantizer (the bit-exact contract).  x: fp32 [rows][ldx],
 * the first k of each row used; out: rows * (k/32) blocks of 34 bytes. */
int oracle_quantize_q8_0(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* out);

/* y[i][r] = sum_k w_hat[r][k] * x_hat[i][k] and s[i][r] = sum_k |w_hat*x_hat|
 * over all m activation rows i and n weight rows r, fp64.  w: n rows of
 * k/qk blocks; xq: m rows of k/32 Q8_0 blocks.  Either of y, s may be NULL. */
int oracle_matmul(int type, const uint8_t* w, int64_t n, int64_t k,
                  const uint8_t* xq, int64_t m, double* y, double* s, int n_threads);

/* The same products at selected (activation row, weight row) pairs only. */
int oracle_matmul_sampled(int type, const uint8_t* w, int64_t n, int64_t k,
                          const uint8_t* xq, int64_t m,
                          const int64_t* act_rows, const int64_t* w_rows, int64_t count,
                          double* y, double* s, int n_threads);

/* Second, independent formulation of oracle_matmul: per 32-element block
 * (Q6_K: per 16-element scale group) an exact integer sum of quant products,
 * then the fp64 scale factors, as in [alice-Q4K] with the Q8_0 activation
 * scale of each 32-block in place of the Q8_K one. */
int oracle_matmul_factored(int type, const uint8_t* w, int64_t n, int64_t k,
                           const uint8_t* xq, int64_t m, double* y, int n_threads);

/* h[i] = fp32( silu(g[i]) * u[i] ), silu evaluated in fp64. */
void oracle_swiglu(const float* g, const float* u, int64_t n, float* h);

/* Stable counting sort of the (token, slot) pairs by expert.
 * ids: [n_tokens][top_k]; offsets: [n_experts + 1]; pairs: [n_tokens*top_k]
 * gets pair ids p = t*top_k + s, grouped by expert, ascending p within an
 * expert.  Returns -1 on an id outside [0, n_experts). */
int oracle_moe_group(const int32_t* ids, int64_t n_tokens, int64_t top_k,
                     int64_t n_experts, int32_t* offsets, int32_t* pairs);

/* Per-pair expert projection: for pair p = (t, s) with expert e = ids[p],
 * y[p][:] = W_e * x_hat[row] where row = p if x_per_pair else t.
 * w: n_experts consecutive [n][k/qk] block matrices. */
int oracle_moe_matmul(int type, const uint8_t* w, int64_t n_experts, int64_t n, int64_t k,
                      const uint8_t* xq, int x_per_pair, const int32_t* ids,
                      int64_t n_tokens, int64_t top_k, double* y, double* s, int n_threads);

/* y[t][:] = sum over slots s of route_w[t][s] * d[t*top_k + s][:], fp64;
 * s_out[t][:] = sum over s of |route_w| * s_in (either may be NULL). */
int oracle_moe_combine(const double* d, const double* s_in, const float* route_w,
                       int64_t n_tokens, int64_t top_k, int64_t n,
                       double* y, double* s_out);

/* idx[r] = first index of the largest of y[r*ldy + 0 .. n-1] [cera-V]. */
void oracle_argmax_rows(const float* y, int64_t rows, int64_t n, int64_t ldy, int32_t* idx);

/* Router [cera-R]: for each row of logits (n_experts values, row stride ld),
 * ids[t][0..top_k) = the top_k largest in descending order (ties: smaller
 * id first) and w[t][s] = exp(l_s - l_0) / sum over the top_k of
 * exp(l_j - l_0) in fp64, rounded to fp32.  Returns -1 on bad sizes. */
int oracle_topk_softmax(const float* logits, int64_t rows, int64_t n_experts, int64_t ld,
                        int64_t top_k, int32_t* ids, float* w);

#ifdef __cplusplus
}
#endif

#endif

// gemv.hip -- decode GEMV over GGUF blocks (Q4_0, Q4_1, Q8_0, Q4_K, Q5_K,
// Q6_K, Q1_0, 2-bit ternary TQ2) for 1..8 Q8_0 activation rows; the same
// streaming kernel also runs the fused gate/up + SwiGLU GEMV and the
// per-pair routed-expert GEMVs of decode.
//
// Streaming kernel (HBM-bound; the weights are read exactly once):
//  * A wave owns a contiguous range of rows.  Every row is loaded with
//    coalesced, non-temporal 16-byte loads (one KiB per wave instruction)
//    straight into registers, through a ring of P rows, so P rows are in
//    flight while one is computed.  Because GGUF rows are stored back to
//    back, a row is one contiguous byte range whatever the 18/20/34/144-byte
//    block size; it is staged in a wave-private LDS buffer and each lane
//    re-slices its own blocks out of it.
//  * Each lane owns fixed "columns" of K (one or two 32-value blocks; for
//    Q4_K / Q5_K one 32-byte nibble chunk = two 32-value sub-blocks; for
//    Q6_K a 64-value quarter super-block; for Q1_0 and TQ2 half a block) and keeps the
//    Q8_0 activation of its columns, for all batch rows, in registers.  The
//    activations are copied once per workgroup into LDS with coalesced
//    loads and unpacked from there.
//  * Per block: nibble unpack in registers, v_dot4 integer dots against the
//    activation quants, scales applied once per 32-value block in fp32
//    (alice-llm 2.0.0 README, "Computation Path (Q4_K)").  Batch rows share
//    the decoded weight registers (alice-llm 2.0.0 README, "Batch-4
//    Speculative Decoding": one accumulator register per row).
//  * Cross-lane sums: P rows x batch values are reduced together, four at a
//    time, with permlane swaps and DPP (alice-llm 2.0.0 README, "The GPU
//    Optimization Journey", phase 2: subgroup reduction instead of a
//    shared-memory tree), then stored with one instruction.
//  * The column split depends only on (type, k), never on the batch size, so
//    batch row b gives bitwise the batch-1 result.
//  * Fused modes (template flags): SW walks the gate and up rows of each
//    output in turn and stores silu(gate)*up after the reduction; MOE makes
//    grid.y a token-expert pair whose expert id, activation row and output
//    row offset the pointers at kernel start.
//  * k-split form (rows of one to four wave widths): KS = 2 or 4 waves
//    stream the same rows, each over its own k-slice, load
//    their slice's activations per lane from global memory, and add their
//    per-row sums in slice order through LDS after each group of P rows.
// Shapes the streaming kernel does not cover (longer rows, rows that are not
// whole 16-byte pieces, unaligned activations at one wave per row) use the
// general kernel: several waves per row,
// cooperative staging of row tiles in LDS, per-wave sums added in wave
// order.
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {
namespace {

enum { T_Q4_0 = 2, T_Q4_1 = 3, T_Q8_0 = 8, T_Q4_K = 12, T_Q5_K = 13, T_Q6_K = 14, T_Q1_0 = 41,
       T_TQ2 = 42 };

// Q4_K and Q5_K share the super-block header (d, dmin, 6-bit scales and
// mins) and the nibble chunks; Q5_K adds one high bit per value from qh.
template <int FMT> constexpr bool kK45 = (FMT == T_Q4_K || FMT == T_Q5_K);
// super-block formats: a lane column spans 64 values
template <int FMT> constexpr bool kSuper = kK45<FMT> || FMT == T_Q6_K;
// 128-value blocks whose lane column is half a block (64 values, two Q8_0
// activation blocks): Q1_0 and the 2-bit ternary TQ2
template <int FMT> constexpr bool kHalf128 = FMT == T_Q1_0 || FMT == T_TQ2;
// one column per lane (no two-column streaming instantiation)
template <int FMT> constexpr bool kOneCol = kSuper<FMT> || kHalf128<FMT>;

// columns per lane: a super-block column already spans 64 values, and a
// Q1_0 column (64 values, 9 bytes) carries two activation blocks, so one
template <int FMT> constexpr int kCMax = kOneCol<FMT> ? 1 : 2;
constexpr int kMaxThreads = 512;    // 8 waves

// bytes per block of the 32-value formats
template <int FMT> struct Fmt;
template <> struct Fmt<T_Q4_0> { static constexpr int BS = 18; };
template <> struct Fmt<T_Q4_1> { static constexpr int BS = 20; };
template <> struct Fmt<T_Q8_0> { static constexpr int BS = 34; };

// Activation registers of one column for one batch row.
// Integer dots start from kBias = bit pattern of 1.5*2^23: for |s| < 2^22
// the int32 kBias + s, read as a float, is exactly 12582912 + s, so
// fma(that, dx, -12582912*dx) = round(s*dx) with no int-to-float convert
// (-12582912*dx is exact: dx is an fp16 value, 11 significant bits).
constexpr int kBias = 0x4B400000;
constexpr float kBiasF = 12582912.0f;

// kBias in a scalar register the compiler cannot see through.
__device__ __forceinline__ int bias_sgpr() {
    int r;
    asm("s_mov_b32 %0, 0x4b400000" : "=s"(r));
    return r;
}

template <int FMT> struct Act {
    uint32_t q[8];  // 32 int8 quants
    float dx;       // block scale
    float ndx;      // -12582912 * dx
    float sdx;      // dx * sum(q)                  (Q4_1)
    int start;      // kBias (- 8 * sum(q) for Q4_0): start value of the dot
};
template <> struct Act<T_Q4_K> {
    uint32_t qa[8], qb[8];  // the two 32-value blocks under one nibble chunk
    float dxa, dxb;         // (Q4_K: dxb / 16, see chunk_dot_k45)
    float ndxa, ndxb;       // -12582912 * dx (of the dx held)
    float sa, sb;           // dx * sum(q) of each block
    int startb;             // Q4_K: kBias + 128 * sum(qb), the high-nibble chain's start
};
template <> struct Act<T_Q5_K> : Act<T_Q4_K> {};

// Q1_0 column (64 values): half col & 1 of block col >> 1, i.e. Q8_0
// activation blocks 2 col and 2 col + 1.
template <> struct Act<T_Q1_0> {
    uint32_t q[2][8];
    float dx[2];
    float ndx[2];      // -12582912 * dx
    int start[2];      // kBias - sum(q): start of the dot with the 0/2 sign bytes
};

// TQ2 column (64 values): half col & 1 of block col >> 1, i.e. Q8_0
// activation blocks 2 col and 2 col + 1, each quant word transposed per 16
// values (see tq2_perm16) to match the code fields of the weight bytes.
template <> struct Act<T_TQ2> {
    uint32_t q[2][8];
    float dx[2];
    float ndx[2];      // -12582912 * dx
};

// Q6_K column (64 values): half h of super-block sb, l in [16 i, 16 i + 16)
// of each of the four 32-value quadrants g; quadrant g of the half is Q8_0
// activation block 8 sb + 4 h + g, values [16 i, 16 i + 16) of it.
template <> struct Act<T_Q6_K> {
    uint32_t q[4][4];  // 16 int8 quants per quadrant
    float dx[4];
    float ndx[4];      // -12582912 * dx
    int start[4];      // kBias - 32 * sum(q): start of the dot with the 6-bit quants
};

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// First dot of a chain in the three-operand form, its start value read from a
// scalar register (S), a vector register (V) or zero (Z); the compiler's own
// choice, the accumulate-in-place form, would first copy the start value into
// the result register.
__device__ __forceinline__ int sdot4_s(uint32_t a, uint32_t b, int c) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}
__device__ __forceinline__ int sdot4_v(uint32_t a, uint32_t b, int c) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ int sdot4_z(uint32_t a, uint32_t b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// start + sum over t < 8 of the 4-byte dot w[t].x[t] (exact in int32); start
// is wave-uniform (in a scalar register) when UNIFORM.  TWO: two chains of
// four for more independent work (batch 1).
template <bool TWO, bool UNIFORM>
__device__ __forceinline__ int dot8(const uint32_t* w, const uint32_t* x, int start) {
    int s = UNIFORM ? sdot4_s(w[0], x[0], start) : sdot4_v(w[0], x[0], start);
    if constexpr (TWO) {
        int s1 = sdot4_z(w[4], x[4]);
#pragma unroll
        for (int t = 1; t < 4; ++t) {
            s = sdot4(w[t], x[t], s);
            s1 = sdot4(w[4 + t], x[4 + t], s1);
        }
        return s + s1;
    } else {
#pragma unroll
        for (int t = 1; t < 8; ++t) s = sdot4(w[t], x[t], s);
        return s;
    }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Weight rows are read through buffer descriptors: the row base and its
// length live in scalar registers, each lane adds a 32-bit offset, and the
// hardware returns zeros for bytes at or past the length without touching
// memory.  The loads carry the non-temporal hint (every weight byte is read
// once).
constexpr int kBufWord3 = 0x00020000;  // raw 32-bit dwords
constexpr int kNonTemporal = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, kBufWord3);
}

// Activation blocks through a buffer resource over the xq rows whose base is
// xq rounded down to 4 bytes and whose range is rounded up to 4 bytes (every
// dword that holds an activation byte lies in the range and in a page the
// buffer touches; nothing outside the range is read).  bo is a block's byte
// offset from that base (even).  Nine dwords from bo rounded down to 4
// cover the 34-byte block: three loads instead of seventeen 16-bit ones.
__device__ __forceinline__ void load_q8_rs(__amdgpu_buffer_rsrc_t rs, int bo, uint32_t* q,
                                           float* dx, int* sum) {
    const int b4 = bo & ~3;
    const bool odd = (bo & 2) != 0;   // d in the high half of the first dword
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, b4, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, b4 + 16, 0, 0);
    const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rs, b4 + 32, 0, 0);
    const uint32_t wd[9] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, c};
    *dx = h2f(static_cast<uint16_t>(odd ? wd[0] >> 16 : wd[0]));
    int acc = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        q[t] = odd ? wd[t + 1] : __builtin_amdgcn_alignbit(wd[t + 1], wd[t], 16);
        acc = sdot4(q[t], 0x01010101u, acc);
    }
    *sum = acc;
}

// TQ2: the 16 activation quants of values v..v+15 (four words, value v+4i+p
// in byte p of word i) rearranged so that word p holds values v+p, v+4+p,
// v+8+p, v+12+p: the order of the code fields p of four weight bytes.
__device__ __forceinline__ void tq2_perm16(const uint32_t* w, uint32_t* o) {
    const uint32_t a01l = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
    const uint32_t a01h = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
    const uint32_t a23l = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    o[0] = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(a23h, a01h, 0x07060302u);
}

// The Q8_0 activation of lane column col (its blocks and the per-block
// terms the dot chains start from) for one batch row, whose first byte is
// at offset xo from the resource base.
template <int FMT>
__device__ __forceinline__ void load_act_rs(__amdgpu_buffer_rsrc_t rs, int xo, int col, Act<FMT>& a) {
    if constexpr (kK45<FMT>) {
        int sa, sb;
        load_q8_rs(rs, xo + 2 * col * 34, a.qa, &a.dxa, &sa);
        load_q8_rs(rs, xo + (2 * col + 1) * 34, a.qb, &a.dxb, &sb);
        a.sa = a.dxa * static_cast<float>(sa);
        a.sb = a.dxb * static_cast<float>(sb);
        if constexpr (FMT == T_Q4_K) {
            a.startb = kBias + 128 * sb;
            a.dxb *= 0.0625f;
        }
        a.ndxa = -kBiasF * a.dxa;
        a.ndxb = -kBiasF * a.dxb;
    } else if constexpr (FMT == T_Q1_0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int sum;
            load_q8_rs(rs, xo + (2 * col + j) * 34, a.q[j], &a.dx[j], &sum);
            a.start[j] = kBias - sum;
            a.ndx[j] = -kBiasF * a.dx[j];
        }
    } else if constexpr (FMT == T_TQ2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int sum;
            uint32_t q[8];
            load_q8_rs(rs, xo + (2 * col + j) * 34, q, &a.dx[j], &sum);
            tq2_perm16(q, a.q[j]);
            tq2_perm16(q + 4, a.q[j] + 4);
            a.ndx[j] = -kBiasF * a.dx[j];
        }
    } else if constexpr (FMT == T_Q6_K) {
        // quadrant g: d and the 16 quants [16 i, 16 i + 16) of block
        // 8 sb + 4 h + g; five dwords from the quants' start rounded down
        const int sb = col >> 2, h = (col >> 1) & 1, i = col & 1;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int bo = xo + (8 * sb + 4 * h + g) * 34;
            const uint32_t dw = __builtin_amdgcn_raw_buffer_load_b32(rs, bo & ~3, 0, 0);
            a.dx[g] = h2f(static_cast<uint16_t>((bo & 2) ? dw >> 16 : dw));
            const int qs = bo + 2 + 16 * i, q4 = qs & ~3;
            const bool odd = (qs & 2) != 0;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, q4, 0, 0);
            const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rs, q4 + 16, 0, 0);
            const uint32_t wd[5] = {v.x, v.y, v.z, v.w, e};
            int sum = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                a.q[g][t] = odd ? __builtin_amdgcn_alignbit(wd[t + 1], wd[t], 16) : wd[t];
                sum = sdot4(a.q[g][t], 0x01010101u, sum);
            }
            a.start[g] = kBias - 32 * sum;
            a.ndx[g] = -kBiasF * a.dx[g];
        }
    } else {
        int s;
        load_q8_rs(rs, xo + col * 34, a.q, &a.dx, &s);
        a.start = (FMT == T_Q4_0) ? kBias - 8 * s : kBias;
        a.ndx = -kBiasF * a.dx;
        a.sdx = a.dx * static_cast<float>(s);
    }
}

// Byte offset, inside the staged tile, of the block that holds column col
// of tile row r.
template <int FMT>
__device__ __forceinline__ int col_offset(int row_base, int col) {
    if constexpr (FMT == T_Q4_K) return row_base + (col >> 2) * 144;
    else if constexpr (FMT == T_Q5_K) return row_base + (col >> 2) * 176;
    else if constexpr (FMT == T_Q6_K) return row_base + (col >> 2) * 210;
    else if constexpr (FMT == T_Q1_0) return row_base + (col >> 1) * 18;
    else if constexpr (FMT == T_TQ2) return row_base + (col >> 1) * 34;
    else return row_base + col * Fmt<FMT>::BS;
}

// Q6_K 6-bit quants of quadrant g (0..3) from 4 dwords of ql (the low
// nibbles of ql[l] for g = 0, of ql[l + 32] for g = 1, their high nibbles for
// g = 2, 3) and 4 dwords of qh (bit pair g of qh[l] goes to bits 4-5).
__device__ __forceinline__ uint32_t q6k_quant4(uint32_t lqa, uint32_t lqb, uint32_t hq, int g) {
    const uint32_t l = (g & 1) ? lqb : lqa;
    const uint32_t nib = (g < 2) ? (l & 0x0F0F0F0Fu) : ((l >> 4) & 0x0F0F0F0Fu);
    return nib | (((hq >> (2 * g)) & 0x03030303u) << 4);
}

// acc[j] += one Q6_K column (see Act<T_Q6_K>) of the super-block at LDS byte
// offset off (2-byte aligned): per quadrant g an integer dot of the 16 6-bit
// quants with the activation quants from kBias - 32 * sum(qx), then
// dx * d * scale.
template <int B>
__device__ __forceinline__ void q6k_column_dot(const uint8_t* lds, int off, int col,
                                               const Act<T_Q6_K>* a, float* acc) {
    const int h = (col >> 1) & 1, i = col & 1;
    uint32_t qla[4], qlb[4], qh[4], scw[2];
    lds_dwords_a2<4>(lds, off + 64 * h + 16 * i, qla);
    lds_dwords_a2<4>(lds, off + 64 * h + 32 + 16 * i, qlb);
    lds_dwords_a2<4>(lds, off + 128 + 32 * h + 16 * i, qh);
    lds_dwords_a2<2>(lds, off + 192 + 8 * h, scw);
    const float d = h2f(lds_u16(lds, off + 208));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        // signed scale byte 2 g + i of the half
        const int b = 2 * g + i;
        const int sc = static_cast<int8_t>((scw[b >> 2] >> (8 * (b & 3))) & 0xFFu);
        const float dsc = d * static_cast<float>(sc);
        uint32_t q[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) q[t] = q6k_quant4(qla[t], qlb[t], qh[t], g);
#pragma unroll
        for (int j = 0; j < B; ++j) {
            int s = sdot4_v(q[0], a[j].q[g][0], a[j].start[g]);
#pragma unroll
            for (int t = 1; t < 4; ++t) s = sdot4(q[t], a[j].q[g][t], s);
            const float sx = fmaf(__int_as_float(s), a[j].dx[g], a[j].ndx[g]);
            acc[j] = fmaf(sx, dsc, acc[j]);
        }
    }
}

// acc[j] += Q4_K / Q5_K chunk c (sub-blocks 2c, 2c+1) of the super-block
// whose 16-byte header is hdr, nibbles q[0..7] (Q5_K: the 32 qh bytes
// qh[0..7], bit j of byte l being bit 4 of value l of sub-block j), batch
// row j.  Branch-free in c (c differs between the lanes of a wave).
template <int FMT, int B>
__device__ __forceinline__ void chunk_dot_k45(const uint32_t* hdr, const uint32_t* qh, const uint32_t* q,
                                              int c, const Act<FMT>* a, float* acc) {
    const float d = h2f(hdr[0] & 0xFFFFu), dmin = h2f(hdr[0] >> 16);
    // 6-bit scale / min of sub-blocks 2c, 2c+1 as byte pairs (low byte: 2c).
    // With the 12 scale bytes S[0..11] in hdr[1..3], one byte permutation
    // per pair gathers [S[2c], S[2c+1], 0, 0] (scales, c < 2), [S[4+2c],
    // S[5+2c], 0, 0] (mins, c < 2), or [S[4+2c], S[5+2c], S[2c-4],
    // S[2c-3]] (scales, c >= 2: low four bits, then the two top bits in
    // bits 6-7 of the high bytes), [S[4+2c], S[5+2c], S[2c], S[2c+1]] (mins,
    // c >= 2: the high four bits, then the top bits).  The selector, mask
    // and shift depend on c only (loop-invariant for a lane).
    const uint32_t sel = (c < 2) ? 0x0C0C0100u + 0x0202u * c : 0x01000504u + 0x02020202u * (c - 2);
    const uint32_t msk = (c < 2) ? 0x3F3Fu : 0x0F0Fu;
    const uint32_t msh = (c < 2) ? 0u : 4u;
    const uint32_t ps = __builtin_amdgcn_perm(hdr[3], hdr[1], sel);
    const uint32_t pm = __builtin_amdgcn_perm(hdr[3], hdr[2], sel);
    const uint32_t scp = (ps & msk) | ((ps >> 18) & 0x3030u);
    const uint32_t mp = ((pm >> msh) & msk) | ((pm >> 18) & 0x3030u);
    const float ds0 = d * static_cast<float>(scp & 0xFFu), ds1 = d * static_cast<float>((scp >> 8) & 0xFFu);
    const float dm0 = dmin * static_cast<float>(mp & 0xFFu), dm1 = dmin * static_cast<float>((mp >> 8) & 0xFFu);
    // Q4_K: the high nibbles h stay in place with the top bit flipped, a
    // byte (q & 0xF0) ^ 0x80 that reads as the signed value 16h - 128 (one
    // three-input bitwise op instead of a shift and a mask); its chain starts
    // at kBias + 128 * sum(qb), so it ends at kBias + 16 * sum(h * qb), and dxb
    // is held divided by 16 (exact): the same s * dx as the plain nibbles give.
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        lo[t] = q[t] & 0x0F0F0F0Fu;
        if constexpr (FMT == T_Q4_K) hi[t] = (q[t] & 0xF0F0F0F0u) ^ 0x80808080u;
        else hi[t] = (q[t] >> 4) & 0x0F0F0F0Fu;
        if constexpr (FMT == T_Q5_K) {
            // bits 2c and 2c+1 of each qh byte become bit 4 of the low and
            // high values
            const uint32_t u = qh[t] >> (2 * c);
            lo[t] |= (u << 4) & 0x10101010u;
            hi[t] |= (u << 3) & 0x10101010u;
        }
    }
    const int bias = bias_sgpr();
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const int sa = dot8<B == 1, true>(lo, a[j].qa, bias);
        int sb;
        if constexpr (FMT == T_Q4_K) sb = dot8<B == 1, false>(hi, a[j].qb, a[j].startb);
        else sb = dot8<B == 1, true>(hi, a[j].qb, bias);
        const float xa = fmaf(__int_as_float(sa), a[j].dxa, a[j].ndxa);
        const float xb = fmaf(__int_as_float(sb), a[j].dxb, a[j].ndxb);
        float v = fmaf(xa, ds0, acc[j]);
        v = fmaf(-dm0, a[j].sa, v);
        v = fmaf(xb, ds1, v);
        acc[j] = fmaf(-dm1, a[j].sb, v);
    }
}

// acc[j] += one Q1_0 column (see Act<T_Q1_0>) of the block at LDS byte
// offset off (2-byte aligned): the 32 sign bits of each activation block
// become bytes 0 or 2 (4 bits per multiply), so the dot chain from
// kBias - sum(qx) ends at kBias + sum(+-qx); then dx, then d.
template <int B>
__device__ __forceinline__ void q10_column_dot(const uint8_t* lds, int off, int col,
                                               const Act<T_Q1_0>* a, float* acc) {
    const float d = h2f(lds_u16(lds, off));
    uint32_t bits[2];
    lds_dwords_a2<2>(lds, off + 2 + 8 * (col & 1), bits);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint32_t e[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            e[t] = (__builtin_amdgcn_ubfe(bits[j], 4 * t, 4) * 0x00408102u) & 0x02020202u;
#pragma unroll
        for (int b = 0; b < B; ++b) {
            int s = sdot4_v(e[0], a[b].q[j][0], a[b].start[j]);
#pragma unroll
            for (int t = 1; t < 8; ++t) s = sdot4(e[t], a[b].q[j][t], s);
            const float sx = fmaf(__int_as_float(s), a[b].dx[j], a[b].ndx[j]);
            acc[b] = fmaf(sx, d, acc[b]);
        }
    }
}

// acc[j] += one TQ2 column (see Act<T_TQ2>) of the block at LDS byte offset
// off (2-byte aligned).  Codes 10 become 00 first (each high bit is kept only
// where its low bit is set), then the code field p of every byte is shifted
// to the top two bits of the byte, where as a signed byte it reads 64 times
// the code value (01: 64, 11: -64, 00: 0); four such words against the
// transposed activation words give 64 * sum(t * qx) from kBias, then dx, then
// d / 64 (exact).
template <int B>
__device__ __forceinline__ void tq2_column_dot(const uint8_t* lds, int off, int col,
                                               const Act<T_TQ2>* a, float* acc) {
    const float d64 = h2f(lds_u16(lds, off)) * 0.015625f;
    uint32_t code[4];
    lds_dwords_a2<4>(lds, off + 2 + 16 * (col & 1), code);
    const int bias = bias_sgpr();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint32_t f[8];   // 16 values per code word: fields 0..3
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t c = code[2 * j + h] & ((code[2 * j + h] << 1) | 0x55555555u);
            f[4 * h + 0] = (c << 6) & 0xC0C0C0C0u;
            f[4 * h + 1] = (c << 4) & 0xC0C0C0C0u;
            f[4 * h + 2] = (c << 2) & 0xC0C0C0C0u;
            f[4 * h + 3] = c & 0xC0C0C0C0u;
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int s = dot8<B == 1, true>(f, a[b].q[j], bias);
            const float sx = fmaf(__int_as_float(s), a[b].dx[j], a[b].ndx[j]);
            acc[b] = fmaf(sx, d64, acc[b]);
        }
    }
}

// acc[j] += dot of one column of one weight row with activation row j.
template <int FMT, int B>
__device__ __forceinline__ void column_dot(const uint8_t* lds, int off, const Act<FMT>* a,
                                           float* acc, int col) {
    if constexpr (FMT == T_Q4_0) {
        const float dw = h2f(lds_u16(lds, off));
        uint32_t q[4];
        lds_dwords_a2<4>(lds, off + 2, q);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            lo[t] = q[t] & 0x0F0F0F0Fu;
            hi[t] = (q[t] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            // kBias + sum (q-8)*qx = kBias + sum q*qx - 8*sum qx (at batch 1
            // as two chains, low and high nibbles, joined at the end)
            int s = a[j].start, s1 = 0;
            int& s2 = B == 1 ? s1 : s;  // a second chain only at batch 1
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                s = sdot4(lo[t], a[j].q[t], s);
                s2 = sdot4(hi[t], a[j].q[4 + t], s2);
            }
            if (B == 1) s += s1;
            const float sx = fmaf(__int_as_float(s), a[j].dx, a[j].ndx);  // sum * dx
            acc[j] = fmaf(sx, dw, acc[j]);
        }
    } else if constexpr (FMT == T_Q4_1) {
        const uint32_t dm = *reinterpret_cast<const uint32_t*>(lds + off);  // 4-aligned
        const float dw = h2f(dm & 0xFFFFu), mw = h2f(dm >> 16);
        const uint32_t* qp = reinterpret_cast<const uint32_t*>(lds + off + 4);
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t q = qp[t];
            lo[t] = q & 0x0F0F0F0Fu;
            hi[t] = (q >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            int s = kBias, s1 = 0;  // a second chain only at batch 1
            int& s2 = B == 1 ? s1 : s;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                s = sdot4(lo[t], a[j].q[t], s);
                s2 = sdot4(hi[t], a[j].q[4 + t], s2);
            }
            if (B == 1) s += s1;
            // dx * (d * sum(q*qx) + m * sum(qx))
            const float sx = fmaf(__int_as_float(s), a[j].dx, a[j].ndx);
            acc[j] = fmaf(mw, a[j].sdx, fmaf(sx, dw, acc[j]));
        }
    } else if constexpr (FMT == T_Q8_0) {
        const float dw = h2f(lds_u16(lds, off));
        uint32_t q[8];
        lds_dwords_a2<8>(lds, off + 2, q);
#pragma unroll
        for (int j = 0; j < B; ++j) {
            int s = kBias, s1 = 0;  // a second chain only at batch 1
            int& s2 = B == 1 ? s1 : s;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                s = sdot4(q[t], a[j].q[t], s);
                s2 = sdot4(q[4 + t], a[j].q[4 + t], s2);
            }
            if (B == 1) s += s1;
            const float sx = fmaf(__int_as_float(s), a[j].dx, a[j].ndx);
            acc[j] = fmaf(sx, dw, acc[j]);
        }
    } else if constexpr (FMT == T_Q6_K) {
        q6k_column_dot<B>(lds, off, col, a, acc);
    } else if constexpr (FMT == T_Q1_0) {
        q10_column_dot<B>(lds, off, col, a, acc);
    } else if constexpr (FMT == T_TQ2) {
        tq2_column_dot<B>(lds, off, col, a, acc);
    } else if constexpr (FMT == T_Q5_K) {  // chunk c, its 32 qh bytes at off + 16
        const int c = col & 3;
        const uint4 h4 = *reinterpret_cast<const uint4*>(lds + off);  // 16-aligned
        const uint4 qh0 = *reinterpret_cast<const uint4*>(lds + off + 16);
        const uint4 qh1 = *reinterpret_cast<const uint4*>(lds + off + 32);
        const uint4 q0 = *reinterpret_cast<const uint4*>(lds + off + 48 + 32 * c);
        const uint4 q1 = *reinterpret_cast<const uint4*>(lds + off + 64 + 32 * c);
        const uint32_t hdr[4] = {h4.x, h4.y, h4.z, h4.w};
        const uint32_t qh[8] = {qh0.x, qh0.y, qh0.z, qh0.w, qh1.x, qh1.y, qh1.z, qh1.w};
        const uint32_t q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        chunk_dot_k45<T_Q5_K, B>(hdr, qh, q, c, a, acc);
    } else {  // Q4_K: column = nibble chunk c of super-block at off
        const int c = col & 3;
        const uint4 hdr = *reinterpret_cast<const uint4*>(lds + off);  // 16-aligned
        const uint4 q0 = *reinterpret_cast<const uint4*>(lds + off + 16 + 32 * c);
        const uint4 q1 = *reinterpret_cast<const uint4*>(lds + off + 32 + 32 * c);
        const float d = h2f(hdr.x & 0xFFFFu), dmin = h2f(hdr.x >> 16);
        // six-bit scale/min of sub-blocks j0 = 2c and j1 = 2c + 1 from the 12
        // scale bytes S[0..11] = hdr.y, hdr.z, hdr.w (little-endian)
        const uint32_t s03 = hdr.y, s47 = hdr.z, s8b = hdr.w;
        int sc0, m0, sc1, m1;
        if (c < 2) {  // sub-blocks 0..3: low six bits of S[j] and S[j+4]
            const int sh0 = 16 * c, sh1 = 16 * c + 8;
            sc0 = (s03 >> sh0) & 63;
            m0 = (s47 >> sh0) & 63;
            sc1 = (s03 >> sh1) & 63;
            m1 = (s47 >> sh1) & 63;
        } else {      // sub-blocks 4..7: nibble of S[j+4], top bits of S[j-4] / S[j]
            const int sh0 = 16 * (c - 2), sh1 = 16 * (c - 2) + 8;
            sc0 = ((s8b >> sh0) & 0xF) | (((s03 >> sh0) >> 6 & 3) << 4);
            m0 = ((s8b >> sh0) >> 4 & 0xF) | (((s47 >> sh0) >> 6 & 3) << 4);
            sc1 = ((s8b >> sh1) & 0xF) | (((s03 >> sh1) >> 6 & 3) << 4);
            m1 = ((s8b >> sh1) >> 4 & 0xF) | (((s47 >> sh1) >> 6 & 3) << 4);
        }
        const float ds0 = d * static_cast<float>(sc0), dm0 = dmin * static_cast<float>(m0);
        const float ds1 = d * static_cast<float>(sc1), dm1 = dmin * static_cast<float>(m1);
        const uint32_t q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        uint32_t lo[8], hi[8];   // (high nibbles as in chunk_dot_k45)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            lo[t] = q[t] & 0x0F0F0F0Fu;
            hi[t] = (q[t] & 0xF0F0F0F0u) ^ 0x80808080u;
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            int sa = kBias, sb = a[j].startb, sa1 = 0, sb1 = 0;  // four chains at batch 1
            int& sa2 = B == 1 ? sa1 : sa;
            int& sb2 = B == 1 ? sb1 : sb;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sa = sdot4(lo[t], a[j].qa[t], sa);
                sb = sdot4(hi[t], a[j].qb[t], sb);
                sa2 = sdot4(lo[4 + t], a[j].qa[4 + t], sa2);
                sb2 = sdot4(hi[4 + t], a[j].qb[4 + t], sb2);
            }
            if (B == 1) {
                sa += sa1;
                sb += sb1;
            }
            // dx*(d*sc*sum(q*qx) - dmin*m*sum(qx)) for each sub-block
            const float xa = fmaf(__int_as_float(sa), a[j].dxa, a[j].ndxa);
            const float xb = fmaf(__int_as_float(sb), a[j].dxb, a[j].ndxb);
            float v = fmaf(xa, ds0, acc[j]);
            v = fmaf(-dm0, a[j].sa, v);
            v = fmaf(xb, ds1, v);
            acc[j] = fmaf(-dm1, a[j].sb, v);
        }
    }
}

template <int FMT, int B, int RT>
__global__ __launch_bounds__(kMaxThreads) void gemv_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t rb, int ncols, int C,
        const uint8_t* __restrict__ xq, int64_t xq_row_bytes, float* __restrict__ y, int64_t ldy,
        int tile_lds_bytes) {
    extern __shared__ __align__(16) uint8_t smem[];
    float* red = reinterpret_cast<float*>(smem + tile_lds_bytes);
    const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;

    // columns of this lane and their activations, resident for the whole
    // kernel (read through a descriptor over the activation rows, base
    // rounded down and length rounded up to 4 bytes)
    const int mis = static_cast<int>(reinterpret_cast<uintptr_t>(xq) & 3);
    const __amdgpu_buffer_rsrc_t xr =
        row_rsrc(xq - mis, (mis + B * static_cast<int>(xq_row_bytes) + 3) & ~3);
    constexpr int CM = kCMax<FMT>;
    Act<FMT> act[CM][B];
    int col[CM];
    bool valid[CM];
#pragma unroll
    for (int i = 0; i < CM; ++i) {
        col[i] = (wv * C + i) * kWave + lane;
        valid[i] = (i < C) && (col[i] < ncols);
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (valid[i])
                load_act_rs<FMT>(xr, mis + j * static_cast<int>(xq_row_bytes), col[i], act[i][j]);
    }

    const int64_t total = n * rb;
    const int64_t ntiles = (n + RT - 1) / RT;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t r0 = tile * RT;
        const int rt = static_cast<int>(n - r0 < RT ? n - r0 : RT);
        const int64_t start = r0 * rb;
        const int64_t a0 = start & ~static_cast<int64_t>(15);
        const int delta = static_cast<int>(start - a0);
        const int nvec = (delta + rt * static_cast<int>(rb) + 15) >> 4;

        __syncthreads();  // the previous tile's LDS reads are done
        for (int v0 = threadIdx.x; v0 < nvec; v0 += 4 * blockDim.x) {
            uint4 val[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = v0 + u * blockDim.x;
                const int64_t g = a0 + 16 * static_cast<int64_t>(v);
                if (v < nvec && g + 16 <= total) {
                    val[u] = *reinterpret_cast<const uint4*>(w + g);
                } else if (v < nvec) {  // the matrix ends inside this vector
                    uint16_t part[8];
#pragma unroll
                    for (int p = 0; p < 8; ++p)
                        part[p] = (g + 2 * p + 2 <= total)
                                      ? *reinterpret_cast<const uint16_t*>(w + g + 2 * p) : 0;
                    val[u] = make_uint4(part[0] | (part[1] << 16), part[2] | (part[3] << 16),
                                        part[4] | (part[5] << 16), part[6] | (part[7] << 16));
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = v0 + u * blockDim.x;
                if (v < nvec) reinterpret_cast<uint4*>(smem)[v] = val[u];
            }
        }
        __syncthreads();

        float acc[RT][B];
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int j = 0; j < B; ++j) acc[r][j] = 0.0f;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (r < rt) {
                const int row_base = delta + r * static_cast<int>(rb);
#pragma unroll
                for (int i = 0; i < CM; ++i)
                    if (valid[i])
                        column_dot<FMT, B>(smem, col_offset<FMT>(row_base, col[i]), act[i],
                                           acc[r], col[i]);
            }
        }

        // reduce over the wave, then over the waves of the row in wave order
#pragma unroll
        for (int r = 0; r < RT; ++r) {
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const float s = wave_sum(acc[r][j]);
                if (nw == 1) {
                    if (lane == 0 && r < rt) y[j * ldy + r0 + r] = s;
                } else if (lane == 0) {
                    red[(wv * RT + r) * B + j] = s;
                }
            }
        }
        if (nw > 1) {
            __syncthreads();
            const int t = threadIdx.x;
            if (t < RT * B) {
                const int r = t / B, j = t - r * B;
                if (r < rt) {
                    float s = red[r * B + j];
                    for (int q = 1; q < nw; ++q) s += red[(q * RT + r) * B + j];
                    y[j * ldy + r0 + r] = s;
                }
            }
        }
    }
}

// Sum each of the V = RT*B accumulators over the 64 lanes.  Groups of four
// values are transposed across the wave with permlane32_swap /
// permlane16_swap so that each 16-lane row holds one value, then each row is
// summed with four DPP steps.  The association order is the same for every
// value slot.  Returns the sum this lane holds: value slot
// idx = 4*(lane & 15) + perm(lane >> 4) (perm swapping 1 and 2; slot r*B + j
// is row r, batch row j), nothing for lanes with lane & 15 >= ceil(V/4).
template <int RT, int B>
__device__ __forceinline__ float reduce_lanes(float (&acc)[RT][B], int lane) {
    constexpr int V = RT * B;
    constexpr int NG = (V + 3) / 4;
    static_assert(NG <= 16, "at most 64 values");
    float vals[4 * NG];
#pragma unroll
    for (int i = 0; i < 4 * NG; ++i) vals[i] = (i < V) ? acc[i / B][i % B] : 0.0f;
    float out = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const auto ab = __builtin_amdgcn_permlane32_swap(__float_as_uint(vals[4 * g]),
                                                         __float_as_uint(vals[4 * g + 1]), false, false);
        const auto cd = __builtin_amdgcn_permlane32_swap(__float_as_uint(vals[4 * g + 2]),
                                                         __float_as_uint(vals[4 * g + 3]), false, false);
        const float sab = __uint_as_float(ab[0]) + __uint_as_float(ab[1]);  // rows 0,1: a; 2,3: b
        const float scd = __uint_as_float(cd[0]) + __uint_as_float(cd[1]);  // rows 0,1: c; 2,3: d
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(sab), __float_as_uint(scd),
                                                        false, false);
        float v = __uint_as_float(q[0]) + __uint_as_float(q[1]);             // rows: a, c, b, d
        v += dpp_f<0xB1>(v);
        v += dpp_f<0x4E>(v);
        v += dpp_f<0x141>(v);
        v += dpp_f<0x140>(v);                                                // row sums
        if ((lane & 15) == g) out = v;
    }
    return out;
}

// value slot held by a lane after reduce_lanes (meaningful while it is < V)
__device__ __forceinline__ int reduced_slot(int lane) {
    const int row = lane >> 4;
    return 4 * (lane & 15) + (row == 1 ? 2 : (row == 2 ? 1 : row));
}

// Reduce (reduce_lanes) and store row r, batch j to y[j*ldy + r0 + r*rs]
// (r < rt) with one store instruction.
template <int RT, int B>
__device__ __forceinline__ void reduce_store(float (&acc)[RT][B], int rt, int64_t r0,
                                             float* __restrict__ y, int64_t ldy, int lane,
                                             int64_t rs = 1) {
    constexpr int V = RT * B;
    const float out = reduce_lanes<RT, B>(acc, lane);
    const int idx = reduced_slot(lane);
    const int r = idx / B, j = idx - (idx / B) * B;
    if (idx < V && r < rt) y[j * ldy + r0 + r * rs] = out;
}

// As reduce_store, for rows that alternate gate, up, gate, up (r0 even):
// after the reduction the lane holding gate row 2p, batch j fetches the up
// row 2p+1 of the same batch row from the lane that holds it and stores
// h[j*ldh + (r0 + 2p)/2] = silu(gate)*up.  The sums are those reduce_store
// forms (the association order does not depend on the slot).
template <int RT, int B>
__device__ __forceinline__ void reduce_swiglu(float (&acc)[RT][B], int rt, int64_t r0,
                                              float* __restrict__ h, int64_t ldh, int lane) {
    static_assert(RT % 2 == 0, "gate/up pairs");
    constexpr int V = RT * B;
    const float out = reduce_lanes<RT, B>(acc, lane);
    // value idx sits in lane 16*perm(idx % 4) + idx / 4, perm swapping 1 and 2
    const int idx = reduced_slot(lane);
    const int r = idx / B, j = idx - (idx / B) * B;
    const int pidx = (idx + B < V) ? idx + B : idx;
    const int pm = pidx & 3;
    const int plane = 16 * (pm == 1 ? 2 : (pm == 2 ? 1 : pm)) + (pidx >> 2);
    const float up = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * plane, __float_as_int(out)));
    if (idx < V && (r & 1) == 0 && r < rt)
        h[j * ldh + (r0 + r) / 2] = swiglu1(out, up);
}

// ---- streaming kernel helpers: dword windows of a staged row ---------------
// the dword at (even) byte offset O of a dword window
template <int O>
__device__ __forceinline__ uint32_t dw_at(const uint32_t* w) {
    if constexpr (O & 2) return __builtin_amdgcn_alignbit(w[(O >> 2) + 1], w[O >> 2], 16);
    else return w[O >> 2];
}
template <int O>
__device__ __forceinline__ uint32_t half_at(const uint32_t* w) {
    return (w[O >> 2] >> ((O & 2) * 8)) & 0xFFFFu;
}

// Per-lane register window of one weight row.
template <int FMT, int C> struct Win {
    static constexpr int BS = Fmt<FMT>::BS;
    static constexpr bool kMis = (C * BS) % 4 != 0;       // odd lanes start 2 bytes into a dword
    static constexpr int NDW = kMis ? (C * BS + 2 + 3) / 4 : C * BS / 4;
};
template <int C> struct Win<T_Q4_K, C> {
    static constexpr bool kMis = false;
    static constexpr int NDW = 4 + 8 * C;                  // header + C nibble chunks
};
template <int C> struct Win<T_Q5_K, C> {
    static constexpr bool kMis = false;
    static constexpr int NDW = 12 + 8 * C;                 // header + qh + C nibble chunks
};
template <int C> struct Win<T_Q1_0, C> {                 // (reads LDS directly)
    static constexpr bool kMis = false;
    static constexpr int NDW = 1;
};
template <int C> struct Win<T_TQ2, C> {                  // (reads LDS directly)
    static constexpr bool kMis = false;
    static constexpr int NDW = 1;
};
template <int C> struct Win<T_Q6_K, C> {                 // (reads LDS directly)
    static constexpr bool kMis = false;
    static constexpr int NDW = 1;
};

// acc[j] += block (32 values) at byte offset O of the window, batch row j
template <int FMT, int B, int O>
__device__ __forceinline__ void block_dot(const uint32_t* w, const Act<FMT>* a, float* acc) {
    if constexpr (FMT == T_Q8_0) {
        const float dw = h2f(half_at<O>(w));
        uint32_t q[8];
        q[0] = dw_at<O + 2>(w); q[1] = dw_at<O + 6>(w); q[2] = dw_at<O + 10>(w); q[3] = dw_at<O + 14>(w);
        q[4] = dw_at<O + 18>(w); q[5] = dw_at<O + 22>(w); q[6] = dw_at<O + 26>(w); q[7] = dw_at<O + 30>(w);
        const int bias = bias_sgpr();
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int s = dot8<B == 1, true>(q, a[j].q, bias);
            const float sx = fmaf(__int_as_float(s), a[j].dx, a[j].ndx);
            acc[j] = fmaf(sx, dw, acc[j]);
        }
    } else if constexpr (FMT == T_Q4_0) {
        const float dw = h2f(half_at<O>(w));
        const uint32_t qq[4] = {dw_at<O + 2>(w), dw_at<O + 6>(w), dw_at<O + 10>(w), dw_at<O + 14>(w)};
        uint32_t nib[8];  // low nibbles (values 0..15), then high nibbles (16..31)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            nib[t] = qq[t] & 0x0F0F0F0Fu;
            nib[4 + t] = (qq[t] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int s = dot8<B == 1, false>(nib, a[j].q, a[j].start);
            const float sx = fmaf(__int_as_float(s), a[j].dx, a[j].ndx);
            acc[j] = fmaf(sx, dw, acc[j]);
        }
    } else {  // Q4_1, O a multiple of 4
        const uint32_t dm = w[O >> 2];
        const float dw = h2f(dm & 0xFFFFu), mw = h2f(dm >> 16);
        uint32_t nib[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t q = w[(O >> 2) + 1 + t];
            nib[t] = q & 0x0F0F0F0Fu;
            nib[4 + t] = (q >> 4) & 0x0F0F0F0Fu;
        }
        const int bias = bias_sgpr();
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int s = dot8<B == 1, true>(nib, a[j].q, bias);
            const float sx = fmaf(__int_as_float(s), a[j].dx, a[j].ndx);
            acc[j] = fmaf(mw, a[j].sdx, fmaf(sx, dw, acc[j]));
        }
    }
}

template <int FMT, int B, int C, int I = 0>
__device__ __forceinline__ void row_dot(const uint32_t* w, const Act<FMT> (*act)[B], int c0,
                                        float* acc) {
    if constexpr (I < C) {
        if constexpr (FMT == T_Q4_K) {
            chunk_dot_k45<T_Q4_K, B>(w, nullptr, w + 4 + 8 * I, c0 + I, act[I], acc);
        } else if constexpr (FMT == T_Q5_K) {  // header, 32 qh bytes, chunk
            chunk_dot_k45<T_Q5_K, B>(w, w + 4, w + 12 + 8 * I, c0 + I, act[I], acc);
        } else {
            block_dot<FMT, B, I * Fmt<FMT>::BS>(w, act[I], acc);
        }
        row_dot<FMT, B, C, I + 1>(w, act, c0, acc);
    }
}

template <bool V> struct Bool { static constexpr bool value = V; };

// bytes of one lane column: a 32-value block, or a quarter super-block
// (Q6_K: 210 / 4, rounded up)
template <int FMT> constexpr int col_bytes() {
    if constexpr (FMT == T_Q4_K) return 36;
    else if constexpr (FMT == T_Q5_K) return 44;
    else if constexpr (FMT == T_Q6_K) return 53;
    else if constexpr (FMT == T_Q1_0) return 9;
    else if constexpr (FMT == T_TQ2) return 17;
    else return Fmt<FMT>::BS;
}

// bytes of the 64*C columns of one k-slice (a whole number of blocks)
template <int FMT, int C> constexpr int slice_bytes() {
    if constexpr (FMT == T_Q4_K) return kWave * C / 4 * 144;
    else if constexpr (FMT == T_Q5_K) return kWave * C / 4 * 176;
    else if constexpr (FMT == T_Q6_K) return kWave * C / 4 * 210;
    else if constexpr (FMT == T_Q1_0) return kWave * C / 2 * 18;
    else if constexpr (FMT == T_TQ2) return kWave * C / 2 * 34;
    else return kWave * C * Fmt<FMT>::BS;
}

constexpr int kGW = 4;  // waves per workgroup of the streaming kernel (one per SIMD)

// Largest activation bytes (all batch rows) one streaming workgroup stages.
template <int FMT, int B, int C>
constexpr int kActMax = B * (kSuper<FMT> || kHalf128<FMT> ? 128 : 64) * C * 34;

// Routed-expert addressing for decode (MOE): blockIdx.y is the
// token-expert pair p = t*top_k + s; its matrix is expert ids[p] of the
// n_experts back-to-back matrices of mat_bytes each, its activation row is
// xq row p (x_per_pair) or t, and its output row is y + p*ldy.  An id
// outside [0, n_experts) reads no weights (its rows stream as zeros, so its
// outputs are exactly 0) and adds 1 to *status (once per pair, from the
// pair's first workgroup).
struct MoeMap {
    const int32_t* ids;
    int64_t mat_bytes;
    int n_experts, top_k, x_per_pair;
    int32_t* status;
};

// SW: fused gate/up + SwiGLU.  Then w is the gate matrix, w2 the up matrix,
// the wave's rows are gate/up pairs (rows_q, rows_r count pairs), row 2i of
// the wave's virtual range is gate row i and row 2i+1 up row i, and y
// receives h = silu(gate)*up.
// KS > 1 (rows longer than one wave covers): the KS waves of a row stream
// take consecutive k-slices of 64*C columns of the same rows, load their
// slice's activations per lane from global memory (no shared table), and
// add their per-row sums in wave order through LDS after each group.
template <int FMT, int B, int C, int P, bool SW = false, bool MOE = false, int KS = 1>
__global__ __launch_bounds__(kWave * kGW) void gemv_stream_kernel(
        const uint8_t* __restrict__ w, int64_t rows_q, int rows_r, int64_t rb, int ncols,
        const uint8_t* __restrict__ xq, int64_t xq_row_bytes, float* __restrict__ y,
        int64_t ldy, const uint8_t* __restrict__ w2 = nullptr, MoeMap mm = {}) {
    static_assert(KS == 1 || (!MOE && kGW % KS == 0), "k-split: plain or fused GEMV, whole streams per workgroup");
    bool rows_live = true;   // false: every weight row reads as zeros
    if constexpr (MOE) {
        static_assert(B == 1, "one activation row per token-expert pair");
        const int pr = static_cast<int>(blockIdx.y);
        int e = mm.ids[pr];
        if (e < 0 || e >= mm.n_experts) {
            if (blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(mm.status, 1);
            e = 0;
            rows_live = false;
        }
        w += static_cast<int64_t>(e) * mm.mat_bytes;
        if constexpr (SW) w2 += static_cast<int64_t>(e) * mm.mat_bytes;
        xq += static_cast<int64_t>(mm.x_per_pair ? pr : pr / mm.top_k) * xq_row_bytes;
        y += static_cast<int64_t>(pr) * ldy;
    }
    using W = Win<FMT, C>;
    // 16-byte pieces per lane and row: piece j of lane l is row bytes
    // [1024 j + 16 l, +16), so every load instruction reads one contiguous KiB
    constexpr int NJ = (kWave * C * col_bytes<FMT>() + 1023) / 1024;
    constexpr int XMAX = kActMax<FMT, B, C>;
    // Converted activation blocks in lane order: slot h of column C*l + i of
    // batch row j sits at index (j*NS + h)*NP + 64*i + l, so a wave's lanes
    // read consecutive words (no bank conflicts).  A slot is one Q8_0 block
    // (Q6_K: the 16 values of one quadrant that the column covers).
    constexpr int NS = (kK45<FMT> || kHalf128<FMT>) ? 2 : FMT == T_Q6_K ? 4 : 1;  // slots per column
    constexpr int NP = kWave * C;                                  // column positions per row
    constexpr int NBMAX = KS == 1 ? B * NS * NP : 1;              // slots, all rows
    constexpr int STG = NJ * 1024 + 16;                          // staging bytes per wave
    constexpr int RAW = (KS == 1 && XMAX + 16 > kGW * STG) ? XMAX + 16 : kGW * STG;
    // raw activation copy first, the waves' row staging buffers afterwards
    __shared__ __align__(16) uint8_t raw[RAW];
    __shared__ __align__(16) u32x4 xq0[NBMAX];  // quants 0..15 (Q6_K: the slot's 16)
    __shared__ __align__(16) u32x4 xq1[NBMAX];  // quants 16..31
    __shared__ float xda[NBMAX];                // dx
    __shared__ float xau[NBMAX];                // dx*sum(q) (Q4_0, Q6_K: the integer sum)
    // (the wave index is read from lane 0 so the compiler keeps every
    // per-wave row quantity in scalar registers)
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint8_t* xs = raw;
    uint8_t* stage = raw + wv * STG;
    // global row stream g owns rows [rbeg, rend): rows_q each, one more for
    // the first rows_r (possibly none); a stream is one wave (KS = 1) or the
    // KS waves of a workgroup
    constexpr int NSTREAM = kGW / KS;
    const int slice = KS > 1 ? wv % KS : 0;
    const int64_t g = static_cast<int64_t>(blockIdx.x) * NSTREAM + wv / KS;
    constexpr int U = SW ? 2 : 1;  // rows per unit (SW: a gate/up pair)
    const int64_t rbeg = U * (g * rows_q + (g < rows_r ? g : rows_r));
    const int64_t rend = rbeg + U * (rows_q + (g < rows_r ? 1 : 0));
    const int cbase = slice * kWave * C;   // first column of this wave's slice
    const bool valid = cbase + C * lane < ncols;
    const int slice_off = slice * slice_bytes<FMT, C>();   // its first byte in a row
    // byte offsets of this lane's column data within a row
    int off, qoff = 0, c0 = 0;
    if constexpr (kK45<FMT>) {
        const int ch = valid ? C * lane : 0;
        off = (ch >> 2) * (FMT == T_Q4_K ? 144 : 176);
        c0 = ch & 3;
        qoff = off + (FMT == T_Q4_K ? 16 : 48) + 32 * c0;
    } else if constexpr (FMT == T_Q6_K) {
        c0 = valid ? C * lane : 0;               // the column
        off = (c0 >> 2) * 210;
    } else if constexpr (FMT == T_Q1_0) {
        c0 = valid ? C * lane : 0;               // first column; block c0 / 2
        off = (c0 >> 1) * 18;
    } else if constexpr (FMT == T_TQ2) {
        c0 = valid ? C * lane : 0;
        off = (c0 >> 1) * 34;
    } else {
        off = valid ? C * lane * Fmt<FMT>::BS : 0;
    }
    const int aoff = off & ~3;
    const uint32_t mis = static_cast<uint32_t>(off & 2) * 8;
    // Pieces past the row end, and every piece of a row past rend (the ring
    // runs up to P-1 rows ahead of the wave's last row), read as zeros
    // without memory traffic; they are staged or computed and never stored.
    auto load_row = [&](int64_t r, u32x4* d) {
        const bool in = r < rend && rows_live;
        const uint8_t* base;
        if constexpr (SW) base = ((r & 1) ? w2 : w) + (in ? r >> 1 : 0) * rb;
        else base = w + (in ? r : 0) * rb;
        int bytes = in ? static_cast<int>(rb) : 0;
        if constexpr (KS > 1) {
            const int left = bytes - slice_off;
            bytes = left < 0 ? 0 : (left > slice_bytes<FMT, C>() ? slice_bytes<FMT, C>() : left);
            // (the clamp is formed with a vector instruction; the value is
            // wave-uniform, and reading it back into a scalar register keeps
            // the compiler from wrapping each load in a loop over the
            // descriptor values)
            bytes = __builtin_amdgcn_readfirstlane(bytes);
            base += slice_off;
        }
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(base, bytes);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            d[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, 1024 * j + 16 * lane, 0, kNonTemporal);
    };

    // Activations: the workgroup copies all batch rows (xact bytes, a whole
    // number of 16-byte pieces at a 16-byte aligned address) into LDS with
    // coalesced loads, issued before the first P rows of each wave; the
    // copy only waits for its own loads (they are the oldest).
    const int xact = static_cast<int>(B * xq_row_bytes);
    constexpr int XPT = KS > 1 ? 1 : (XMAX / 16 + kWave * kGW - 1) / (kWave * kGW);  // pieces per thread
    u32x4 xv[XPT];
    if constexpr (KS == 1) {
#pragma unroll
        for (int t = 0; t < XPT; ++t) {
            const int pc = threadIdx.x + t * kWave * kGW;
            xv[t] = *reinterpret_cast<const u32x4*>(xq + (16 * pc < xact ? 16 * pc : 0));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // (no branch around these loads, even for a spare wave without rows,
    // whose loads read zeros: with a branch, the wait for the activation
    // copy below would also wait for these loads)
    // KS > 1: every wave of the workgroup runs the groups of its first
    // stream (the one with the most rows), so all take the same barriers;
    // a stream with fewer rows computes zeros past rend and stores nothing
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * NSTREAM;
    const int64_t rows0 = U * (rows_q + (g0 < rows_r ? 1 : 0));
    const bool has_rows = KS > 1 ? rows0 > 0 : rbeg < rend;
    u32x4 buf[P][NJ];
#pragma unroll
    for (int j = 0; j < P; ++j) load_row(rbeg + j, buf[j]);
    __builtin_amdgcn_sched_barrier(0);
    Act<FMT> act[C][B];
    if constexpr (KS > 1) {
        // each lane loads its own columns' activations (its slice of k);
        // lanes past the columns keep zeros and add exact zeros
        (void)xs;
        if (!has_rows) return;
        const int mis = static_cast<int>(reinterpret_cast<uintptr_t>(xq) & 3);
        const __amdgpu_buffer_rsrc_t xr = row_rsrc(xq - mis, (mis + xact + 3) & ~3);
#pragma unroll
        for (int i = 0; i < C; ++i)
#pragma unroll
            for (int j = 0; j < B; ++j) {
                act[i][j] = Act<FMT>{};
                if (valid)
                    load_act_rs<FMT>(xr, mis + j * static_cast<int>(xq_row_bytes), cbase + C * lane + i,
                                     act[i][j]);
            }
    } else {
#pragma unroll
    for (int t = 0; t < XPT; ++t) {
        const int pc = threadIdx.x + t * kWave * kGW;
        if (16 * pc < xact) *reinterpret_cast<u32x4*>(xs + 16 * pc) = xv[t];
    }
    __syncthreads();
    // Each activation block is converted once per workgroup: 32 quants (two
    // 16-byte words), dx, and dx*sum(q) (Q4_0: the integer sum); positions
    // past the columns get zeros, so lanes without a column add exact zeros.
    {
        const int nbr = static_cast<int>(xq_row_bytes / 34);
        constexpr int NG = B * NS * NP;
#pragma unroll
        for (int t0 = 0; t0 < NG; t0 += kWave * kGW) {
            const int gi = t0 + static_cast<int>(threadIdx.x);
            if (gi < NG) {
                const int j = gi / (NS * NP), h = (gi / NP) % NS, pp = gi % NP;
                const int col = C * (pp % kWave) + pp / kWave;
                // Q6_K: quadrant h of the column's half, values [16 i, +16)
                const int blk = FMT == T_Q6_K ? 8 * (col >> 2) + 4 * ((col >> 1) & 1) + h : col * NS + h;
                const int qofs = FMT == T_Q6_K ? 16 * (col & 1) : 0;
                uint32_t q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                float dx = 0.0f;
                if (blk < nbr) {
                    const int bo = j * static_cast<int>(xq_row_bytes) + blk * 34;
                    const int qb = bo + 2 + qofs;
                    const uint32_t* pq = reinterpret_cast<const uint32_t*>(xs + (qb & ~3));
                    const uint32_t sh = static_cast<uint32_t>(qb & 2) * 8;
                    uint32_t wd[9];
#pragma unroll
                    for (int u = 0; u < 9; ++u) wd[u] = pq[u];
#pragma unroll
                    for (int u = 0; u < 8; ++u) q[u] = __builtin_amdgcn_alignbit(wd[u + 1], wd[u], sh);
                    dx = h2f(*reinterpret_cast<const uint16_t*>(xs + bo));
                }
                if constexpr (FMT == T_TQ2) {   // code-field order, once per workgroup
                    uint32_t t[8];
                    tq2_perm16(q, t);
                    tq2_perm16(q + 4, t + 4);
#pragma unroll
                    for (int u = 0; u < 8; ++u) q[u] = t[u];
                }
                xq0[gi] = u32x4{q[0], q[1], q[2], q[3]};
                xq1[gi] = u32x4{q[4], q[5], q[6], q[7]};
                xda[gi] = dx;
                if constexpr (FMT == T_Q6_K) {
                    int sum = 0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) sum = sdot4(q[u], 0x01010101u, sum);
                    xau[gi] = __int_as_float(sum);
                } else if constexpr (FMT != T_Q8_0 && FMT != T_TQ2) {
                    int sum = 0;
#pragma unroll
                    for (int u = 0; u < 8; ++u) sum = sdot4(q[u], 0x01010101u, sum);
                    xau[gi] = (FMT == T_Q4_0 || FMT == T_Q1_0 || FMT == T_Q4_K)
                                  ? __int_as_float(sum) : dx * static_cast<float>(sum);
                }
            }
        }
    }
    __syncthreads();  // converted; the raw copy's space now serves as row staging
    if (!has_rows) return;
#pragma unroll
    for (int i = 0; i < C; ++i)
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if constexpr (FMT == T_Q1_0) {
                Act<T_Q1_0>& a = act[i][j];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int gi = (j * NS + h) * NP + kWave * i + lane;
                    const u32x4 q0 = xq0[gi], q1 = xq1[gi];
                    a.q[h][0] = q0.x; a.q[h][1] = q0.y; a.q[h][2] = q0.z; a.q[h][3] = q0.w;
                    a.q[h][4] = q1.x; a.q[h][5] = q1.y; a.q[h][6] = q1.z; a.q[h][7] = q1.w;
                    a.dx[h] = xda[gi];
                    a.ndx[h] = -kBiasF * a.dx[h];
                    a.start[h] = kBias - __float_as_int(xau[gi]);
                }
            } else if constexpr (FMT == T_TQ2) {
                Act<T_TQ2>& a = act[i][j];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int gi = (j * NS + h) * NP + kWave * i + lane;
                    const u32x4 q0 = xq0[gi], q1 = xq1[gi];
                    a.q[h][0] = q0.x; a.q[h][1] = q0.y; a.q[h][2] = q0.z; a.q[h][3] = q0.w;
                    a.q[h][4] = q1.x; a.q[h][5] = q1.y; a.q[h][6] = q1.z; a.q[h][7] = q1.w;
                    a.dx[h] = xda[gi];
                    a.ndx[h] = -kBiasF * a.dx[h];
                }
            } else if constexpr (FMT == T_Q6_K) {
                Act<T_Q6_K>& a = act[i][j];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int gi = (j * NS + g) * NP + kWave * i + lane;
                    const u32x4 q0 = xq0[gi];
                    a.q[g][0] = q0.x; a.q[g][1] = q0.y; a.q[g][2] = q0.z; a.q[g][3] = q0.w;
                    a.dx[g] = xda[gi];
                    a.ndx[g] = -kBiasF * a.dx[g];
                    a.start[g] = kBias - 32 * __float_as_int(xau[gi]);
                }
            } else if constexpr (kK45<FMT>) {
                Act<FMT>& a = act[i][j];
                const int ga = 2 * j * NP + lane, gb = ga + NP;
                const u32x4 a0 = xq0[ga], a1 = xq1[ga], b0 = xq0[gb], b1 = xq1[gb];
                a.qa[0] = a0.x; a.qa[1] = a0.y; a.qa[2] = a0.z; a.qa[3] = a0.w;
                a.qa[4] = a1.x; a.qa[5] = a1.y; a.qa[6] = a1.z; a.qa[7] = a1.w;
                a.qb[0] = b0.x; a.qb[1] = b0.y; a.qb[2] = b0.z; a.qb[3] = b0.w;
                a.qb[4] = b1.x; a.qb[5] = b1.y; a.qb[6] = b1.z; a.qb[7] = b1.w;
                a.dxa = xda[ga];
                a.dxb = xda[gb];
                if constexpr (FMT == T_Q4_K) {   // (the table holds the integer sums)
                    const int suma = __float_as_int(xau[ga]), sumb = __float_as_int(xau[gb]);
                    a.sa = a.dxa * static_cast<float>(suma);
                    a.sb = a.dxb * static_cast<float>(sumb);
                    a.startb = kBias + 128 * sumb;
                    a.dxb *= 0.0625f;
                } else {
                    a.sa = xau[ga];
                    a.sb = xau[gb];
                }
                a.ndxa = -kBiasF * a.dxa;
                a.ndxb = -kBiasF * a.dxb;
            } else {
                Act<FMT>& a = act[i][j];
                const int g = j * NP + kWave * i + lane;
                const u32x4 q0 = xq0[g], q1 = xq1[g];
                a.q[0] = q0.x; a.q[1] = q0.y; a.q[2] = q0.z; a.q[3] = q0.w;
                a.q[4] = q1.x; a.q[5] = q1.y; a.q[6] = q1.z; a.q[7] = q1.w;
                a.dx = xda[g];
                a.ndx = -kBiasF * a.dx;
                if constexpr (FMT == T_Q4_0) {
                    a.start = kBias - 8 * __float_as_int(xau[g]);
                } else {
                    a.start = kBias;
                    if constexpr (FMT == T_Q4_1) a.sdx = xau[g];
                }
            }
        }
    }

    // per-row sums of the KS slices, by group parity (KS > 1)
    __shared__ float part[KS > 1 ? 2 * kGW * P * B : 1];
    int gpar = 0;

    // One group of P rows: stage each row in LDS, refill its registers with
    // the row P further on (REFILL), compute, then reduce and store.  The
    // last group does not refill, so every row is loaded once (refills past
    // rend read zeros, computed and not stored).
    auto group = [&](int64_t r, auto refill) {
        float acc[P][B];
#pragma unroll
        for (int i = 0; i < P; ++i)
#pragma unroll
            for (int j = 0; j < B; ++j) acc[i][j] = 0.0f;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            // stage the row in LDS (one wave: LDS requests are served in
            // order, so the reads below see these writes and the next
            // row's writes come after these reads)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                *reinterpret_cast<u32x4*>(stage + 1024 * j + 16 * lane) = buf[i][j];
            // The refill goes into the registers just staged, with no branch
            // around it, so no register copy of an in-flight load (which
            // would wait for it) is ever needed.
            if constexpr (decltype(refill)::value) {
                __builtin_amdgcn_sched_barrier(0);
                load_row(r + P + i, buf[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint32_t v[W::NDW];
            if constexpr (FMT == T_Q6_K) {
                static_assert(C == 1, "one Q6_K column per lane");
                q6k_column_dot<B>(stage, off, c0, act[0], acc[i]);
            } else if constexpr (FMT == T_Q1_0) {
#pragma unroll
                for (int cc = 0; cc < C; ++cc)
                    q10_column_dot<B>(stage, ((c0 + cc) >> 1) * 18, c0 + cc, act[cc], acc[i]);
            } else if constexpr (FMT == T_TQ2) {
#pragma unroll
                for (int cc = 0; cc < C; ++cc)
                    tq2_column_dot<B>(stage, ((c0 + cc) >> 1) * 34, c0 + cc, act[cc], acc[i]);
            } else if constexpr (kK45<FMT>) {
                // header (and Q5_K's 32 qh bytes), then the C nibble chunks
                constexpr int NH = FMT == T_Q4_K ? 1 : 3;
#pragma unroll
                for (int t = 0; t < NH; ++t) {
                    const uint4 h = *reinterpret_cast<const uint4*>(stage + off + 16 * t);
                    v[4 * t] = h.x; v[4 * t + 1] = h.y; v[4 * t + 2] = h.z; v[4 * t + 3] = h.w;
                }
#pragma unroll
                for (int t = 0; t < 2 * C; ++t) {
                    const uint4 q = *reinterpret_cast<const uint4*>(stage + qoff + 16 * t);
                    v[4 * NH + 4 * t] = q.x; v[4 * NH + 1 + 4 * t] = q.y;
                    v[4 * NH + 2 + 4 * t] = q.z; v[4 * NH + 3 + 4 * t] = q.w;
                }
            } else {
#pragma unroll
                for (int t = 0; t < W::NDW; ++t)
                    v[t] = *reinterpret_cast<const uint32_t*>(stage + aoff + 4 * t);
                if constexpr (W::kMis) {
#pragma unroll
                    for (int t = 0; t + 1 < W::NDW; ++t) v[t] = __builtin_amdgcn_alignbit(v[t + 1], v[t], mis);
                    v[W::NDW - 1] >>= mis;
                }
            }
            if constexpr (FMT != T_Q6_K && !kHalf128<FMT>) row_dot<FMT, B, C>(v, act, c0, acc[i]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        const int rt = static_cast<int>(rend - r < P ? rend - r : P);
        if constexpr (KS > 1) {
            // slice sums -> LDS; after one barrier the first wave adds them in
            // slice order and stores (double-buffered by group parity, so a
            // buffer is rewritten only after every wave passed the barrier
            // that follows its reads)
            constexpr int V = P * B;
            const float out = reduce_lanes<P, B>(acc, lane);
            const int idx = reduced_slot(lane);
            float* pb = part + (gpar * NSTREAM + wv / KS) * KS * V;
            if (idx < V) pb[slice * V + idx] = out;
            __syncthreads();
            if (slice == 0) {
                float sum = 0.0f;
                if (idx < V) {
                    sum = pb[idx];
#pragma unroll
                    for (int q = 1; q < KS; ++q) sum += pb[q * V + idx];
                }
                const int rr = idx / B, jj = idx - (idx / B) * B;
                if constexpr (SW) {
                    // gate row rr (even) takes up row rr + 1 of the same batch
                    // row from the lane that holds it (as in reduce_swiglu)
                    const int pidx = (idx + B < V) ? idx + B : idx;
                    const int pm = pidx & 3;
                    const int plane = 16 * (pm == 1 ? 2 : (pm == 2 ? 1 : pm)) + (pidx >> 2);
                    const float up = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * plane, __float_as_int(sum)));
                    if (idx < V && (rr & 1) == 0 && rr < rt)
                        y[jj * ldy + (r + rr) / 2] = swiglu1(sum, up);
                } else {
                    if (idx < V && rr < rt) y[jj * ldy + r + rr] = sum;
                }
            }
            gpar ^= 1;
        } else if constexpr (SW) {
            reduce_swiglu<P, B>(acc, rt, r, y, ldy, lane);
        } else {
            reduce_store<P, B>(acc, rt, r, y, ldy, lane);
        }
    };
    int64_t r = rbeg;
    if constexpr (KS > 1) {
        const int64_t ng = (rows0 + P - 1) / P;   // workgroup-uniform
        for (int64_t i = 1; i < ng; ++i, r += P) group(r, Bool<true>{});
    } else {
        for (; r + P < rend; r += P) group(r, Bool<true>{});
    }
    group(r, Bool<false>{});
}

struct Plan {
    int ncols, C, nw, RT, tile_lds, red_bytes;
    int SC;  // > 0: streaming kernel with SC columns per lane
    int KS;  // streaming kernel: waves per row (k-slices), 1, 2 or kGW
};

constexpr int kRing = 4;  // rows in flight per wave in the streaming kernel

// stream_ok: the streaming kernel may be used (the activations are 16-byte
// aligned); it also needs weight and activation rows that are a whole number
// of 16-byte pieces.
Plan make_plan(int wt, int64_t k, int64_t rb, int batch, bool stream_ok) {
    const int64_t xrb = k / 32 * 34;
    Plan p{};
    const bool super = wt == T_Q4_K || wt == T_Q5_K || wt == T_Q6_K;
    const bool half128 = wt == T_Q1_0 || wt == T_TQ2;
    p.ncols = static_cast<int>(super || half128 ? k / 64 : k / 32);   // Q1_0, TQ2: half blocks
    p.C = (super || half128 || p.ncols <= kWave) ? 1 : 2;
    p.nw = (p.ncols + kWave * p.C - 1) / (kWave * p.C);
    // general kernel: about 16 KiB of weights per tile, at most 32 live
    // accumulators per lane
    int rt = 8;
    while (rt > 1 && (rt * rb > 20480 || rt * batch > 32)) rt >>= 1;
    if (rt == 2) rt = 1;  // instantiated tiles: 1, 4, 8
    p.RT = rt;
    p.tile_lds = static_cast<int>((rt * rb + 32 + 15) & ~15);
    p.red_bytes = p.nw > 1 ? p.nw * rt * batch * 4 : 0;
    // streaming kernel: one wave covers the row with 1 or 2 columns per lane
    // (not Q4_K with two chunks per lane: its activations alone would need
    // more than the register file at the larger batches, and every batch of
    // one (type, k) must take the same kernel)
    const int sc = (p.ncols + kWave - 1) / kWave;
    p.KS = 1;
    if (stream_ok && rb % 16 == 0 && xrb % 16 == 0 && sc <= 2 && p.ncols % sc == 0 &&
        !((super || half128) && sc == 2)) {
        p.SC = sc;
    } else if (rb % 16 == 0 && p.ncols > kWave * p.C &&
               p.ncols <= kGW * kWave * p.C && p.ncols % p.C == 0) {
        // rows of one to four wave widths: two or four waves split k
        // (activations loaded per lane, so xq's alignment does not matter).
        // k-split vs tile kernel, 4096 rows x 14336: Q8_0 b1 12.5 vs 17.1 us,
        // Q4_K b1 9.0 vs 15.1 us, Q4_K b8 18.2 vs 31.2 us; 13824 x 5120
        // (1.25 widths, two waves): Q4_K b1 13.0 vs 17.3 us.
        p.SC = p.C;
        p.KS = p.ncols <= 2 * kWave * p.C ? 2 : kGW;
    }
    return p;
}

template <typename K>
int resident_blocks_per_cu(K kernel, int threads) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1)
        nb = 1;
    return nb;
}

template <int FMT, int B, int SC, bool SW = false, bool MOE = false, int KS = 1>
int launch_stream(const uint8_t* w, int64_t n, int64_t rb, int ncols, const uint8_t* xq,
                  int64_t xrb, float* y, int64_t ldy, hipStream_t stream,
                  const uint8_t* w2 = nullptr, MoeMap mm = {}, int npairs = 1) {
    auto kern = gemv_stream_kernel<FMT, B, SC, kRing, SW, MOE, KS>;
    static const int occ = kGW * resident_blocks_per_cu(kern, kWave * kGW);
    // as many waves as fit, each with a whole number of P-row groups where
    // possible: gpw groups per wave, then the fewest waves that cover n,
    // rounded up to whole workgroups (spare waves get no rows).  Units are
    // rows, or gate/up row pairs (two per group) for SW.
    constexpr int64_t upg = SW ? kRing / 2 : kRing;  // units per group
    // (MOE: the wave slots are shared by the npairs matrices of the launch;
    // KS > 1: a row stream is KS waves)
    constexpr int NSTREAM = kGW / KS;
    const int64_t groups = (n + upg - 1) / upg;
    auto streams_for = [&](int cap) {
        const int per_cu = occ < cap ? occ : cap;
        const int64_t g = static_cast<int64_t>(device_cu_count()) * per_cu / npairs / KS;
        return g < NSTREAM ? static_cast<int64_t>(NSTREAM) : g;
    };
    // Wave slots per CU: up to 16 where they fit and every stream still gets
    // at least 8 groups (long matrices: the Q4_K 128256 x 4096 LM head at
    // batch 1 takes 45.5 against 47.4 us with 8), else up to 8 (shorter
    // streams are slower with more waves: Q4_1 14336 x 4096 at batch 1 takes
    // 8.6 us with 16 against 7.6 us with 8).
    int64_t gmax = streams_for(16);
    if ((groups + gmax - 1) / gmax < 8) gmax = streams_for(8);
    const int64_t gpw = (groups + gmax - 1) / gmax;
    const int64_t waves = (n + gpw * upg - 1) / (gpw * upg);   // row streams
    const int64_t wgs = (waves + NSTREAM - 1) / NSTREAM, nw = wgs * NSTREAM;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(wgs), static_cast<unsigned>(npairs)),
                       dim3(kWave * kGW), 0, stream, w, n / nw, static_cast<int>(n % nw), rb, ncols,
                       xq, xrb, y, ldy, w2, mm);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <int FMT, int B>
int launch_fmt_b(const Plan& p, const uint8_t* w, int64_t n, int64_t rb, const uint8_t* xq,
                 int64_t xrb, float* y, int64_t ldy, hipStream_t stream) {
    if (p.KS == 2) {
        if (p.SC == 1)
            return launch_stream<FMT, B, 1, false, false, 2>(w, n, rb, p.ncols, xq, xrb, y, ldy, stream);
        if constexpr (!kOneCol<FMT>)
            if (p.SC == 2)
                return launch_stream<FMT, B, 2, false, false, 2>(w, n, rb, p.ncols, xq, xrb, y, ldy, stream);
        return -3;
    }
    if (p.KS == kGW) {
        if (p.SC == 1)
            return launch_stream<FMT, B, 1, false, false, kGW>(w, n, rb, p.ncols, xq, xrb, y, ldy, stream);
        if constexpr (!kOneCol<FMT>)
            if (p.SC == 2)
                return launch_stream<FMT, B, 2, false, false, kGW>(w, n, rb, p.ncols, xq, xrb, y, ldy, stream);
        return -3;
    }
    if (p.SC == 1) return launch_stream<FMT, B, 1>(w, n, rb, p.ncols, xq, xrb, y, ldy, stream);
    if constexpr (!kOneCol<FMT>)  // (one column per lane for the super-block formats, Q1_0)
        if (p.SC == 2) return launch_stream<FMT, B, 2>(w, n, rb, p.ncols, xq, xrb, y, ldy, stream);
    const int64_t ntiles = (n + p.RT - 1) / p.RT;
    const int per_cu = p.nw >= 4 ? 2 : 8 / p.nw;
    int64_t grid = static_cast<int64_t>(device_cu_count()) * per_cu;
    // small workgroups (one or two waves) and up to two tiles per slot: one
    // workgroup per tile, so none runs a second tile after the others have
    // finished (Q1_0 10240 x 5120 on this kernel, batch 1: 8.1 against
    // 9.0 us); with larger
    // workgroups the extra resident ones slowed long rows at batch 8
    if (grid > ntiles || (p.nw <= 2 && ntiles <= 2 * grid)) grid = ntiles;
    const dim3 g(static_cast<unsigned>(grid)), b(p.nw * kWave);
    const size_t lds = static_cast<size_t>(p.tile_lds + p.red_bytes);
    switch (p.RT) {
        case 8:
            // make_plan keeps RT * batch <= 32, so RT = 8 exists for B <= 4 only
            if constexpr (B <= 4) {
                hipLaunchKernelGGL((gemv_kernel<FMT, B, 8>), g, b, lds, stream, w, n, rb, p.ncols,
                                   p.C, xq, xrb, y, ldy, p.tile_lds);
                break;
            } else {
                return -3;
            }
        case 4: hipLaunchKernelGGL((gemv_kernel<FMT, B, 4>), g, b, lds, stream, w, n, rb, p.ncols,
                                   p.C, xq, xrb, y, ldy, p.tile_lds); break;
        default: hipLaunchKernelGGL((gemv_kernel<FMT, B, 1>), g, b, lds, stream, w, n, rb, p.ncols,
                                    p.C, xq, xrb, y, ldy, p.tile_lds); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

template <int FMT>
int launch_fmt(const Plan& p, int batch, const uint8_t* w, int64_t n, int64_t rb,
               const uint8_t* xq, int64_t xrb, float* y, int64_t ldy, hipStream_t s) {
    switch (batch) {
        case 1: return launch_fmt_b<FMT, 1>(p, w, n, rb, xq, xrb, y, ldy, s);
        case 2: return launch_fmt_b<FMT, 2>(p, w, n, rb, xq, xrb, y, ldy, s);
        case 3: return launch_fmt_b<FMT, 3>(p, w, n, rb, xq, xrb, y, ldy, s);
        case 4: return launch_fmt_b<FMT, 4>(p, w, n, rb, xq, xrb, y, ldy, s);
        case 5: return launch_fmt_b<FMT, 5>(p, w, n, rb, xq, xrb, y, ldy, s);
        case 6: return launch_fmt_b<FMT, 6>(p, w, n, rb, xq, xrb, y, ldy, s);
        case 7: return launch_fmt_b<FMT, 7>(p, w, n, rb, xq, xrb, y, ldy, s);
        default: return launch_fmt_b<FMT, 8>(p, w, n, rb, xq, xrb, y, ldy, s);
    }
}

int64_t block_bytes_of(int wt) {
    return wt == T_Q4_0 || wt == T_Q1_0 ? 18 : wt == T_Q4_1 ? 20 : wt == T_Q8_0 || wt == T_TQ2 ? 34
           : wt == T_Q4_K ? 144 : wt == T_Q5_K ? 176 : 210;
}
int64_t block_elems_of(int wt) {
    return wt == T_Q4_K || wt == T_Q5_K || wt == T_Q6_K ? 256 : wt == T_Q1_0 || wt == T_TQ2 ? 128 : 32;
}

}  // namespace

// Returns 0, -3 (shape the kernel cannot tile) or -6 (launch failure).
int gemv_shape_ok(int wt, int64_t k, int64_t batch) {
    const int64_t bs = block_bytes_of(wt);
    const int64_t qk = block_elems_of(wt);
    const Plan p = make_plan(wt, k, k / qk * bs, static_cast<int>(batch), false);
    if (p.nw * kWave > kMaxThreads) return -3;
    if (p.tile_lds + p.red_bytes > 65536) return -3;
    return 0;
}

int launch_gemv(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t batch,
                float* y, int64_t ldy, hipStream_t stream) {
    // tall Q4_K matrices with 4096-value rows: integer dots on the matrix
    // cores (gemv_mfma.hip); the choice does not depend on the batch size
    if (wt == T_Q4_K && gemv_q4k_mfma_ok(n, k, batch, xq))
        return launch_gemv_q4k_mfma(w, n, xq, batch, y, ldy, stream);
    if (gemv_shape_ok(wt, k, batch) != 0) return -3;
    const int64_t bs = block_bytes_of(wt);
    const int64_t qk = block_elems_of(wt);
    const int64_t rb = k / qk * bs;
    const Plan p = make_plan(wt, k, rb, static_cast<int>(batch),
                             (reinterpret_cast<uintptr_t>(xq) & 15) == 0);
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int64_t xrb = k / 32 * 34;
    const int b = static_cast<int>(batch);
    switch (wt) {
        case T_Q4_0: return launch_fmt<T_Q4_0>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q4_1: return launch_fmt<T_Q4_1>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q8_0: return launch_fmt<T_Q8_0>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q4_K: return launch_fmt<T_Q4_K>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q5_K: return launch_fmt<T_Q5_K>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q6_K: return launch_fmt<T_Q6_K>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q1_0: return launch_fmt<T_Q1_0>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_TQ2: return launch_fmt<T_TQ2>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        default: return -2;
    }
}

// ---- fused gate/up GEMV + SwiGLU (decode FFN) -------------------------------
// Streaming kernel only: one wave per row (k <= 4096) with a 16-byte aligned
// xq, or its k-split form (rows of up to four wave widths, k <= 16384), and
// whole 16-byte weight rows.
int gemv_swiglu_shape_ok(int wt, int64_t k, int64_t batch) {
    if (gemv_shape_ok(wt, k, batch) != 0) return -3;
    const Plan p = make_plan(wt, k, k / block_elems_of(wt) * block_bytes_of(wt),
                             static_cast<int>(batch), true);
    return p.SC > 0 ? 0 : -3;
}

template <int FMT, int B>
int launch_sw_b(int SC, int KS, const uint8_t* wg, const uint8_t* wu, int64_t n, int64_t rb,
                int ncols, const uint8_t* xq, int64_t xrb, float* h, int64_t ldh,
                hipStream_t stream) {
    if (KS == 2) {
        if (SC == 1)
            return launch_stream<FMT, B, 1, true, false, 2>(wg, n, rb, ncols, xq, xrb, h, ldh, stream, wu);
        if constexpr (!kOneCol<FMT>)
            if (SC == 2)
                return launch_stream<FMT, B, 2, true, false, 2>(wg, n, rb, ncols, xq, xrb, h, ldh, stream, wu);
        return -3;
    }
    if (KS == kGW) {
        if (SC == 1)
            return launch_stream<FMT, B, 1, true, false, kGW>(wg, n, rb, ncols, xq, xrb, h, ldh, stream, wu);
        if constexpr (!kOneCol<FMT>)
            if (SC == 2)
                return launch_stream<FMT, B, 2, true, false, kGW>(wg, n, rb, ncols, xq, xrb, h, ldh, stream, wu);
        return -3;
    }
    if (SC == 1) return launch_stream<FMT, B, 1, true>(wg, n, rb, ncols, xq, xrb, h, ldh, stream, wu);
    if constexpr (!kOneCol<FMT>)
        if (SC == 2) return launch_stream<FMT, B, 2, true>(wg, n, rb, ncols, xq, xrb, h, ldh, stream, wu);
    return -3;
}

template <int FMT>
int launch_sw(int SC, int KS, int b, const uint8_t* wg, const uint8_t* wu, int64_t n, int64_t rb,
              int ncols, const uint8_t* xq, int64_t xrb, float* h, int64_t ldh, hipStream_t s) {
    switch (b) {
        case 1: return launch_sw_b<FMT, 1>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        case 2: return launch_sw_b<FMT, 2>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        case 3: return launch_sw_b<FMT, 3>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        case 4: return launch_sw_b<FMT, 4>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        case 5: return launch_sw_b<FMT, 5>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        case 6: return launch_sw_b<FMT, 6>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        case 7: return launch_sw_b<FMT, 7>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
        default: return launch_sw_b<FMT, 8>(SC, KS, wg, wu, n, rb, ncols, xq, xrb, h, ldh, s);
    }
}

int launch_gemv_swiglu(int wt, const void* w_gate, const void* w_up, int64_t n, int64_t k,
                       const void* xq, int64_t batch, float* h, int64_t ldh, hipStream_t stream) {
    if (gemv_swiglu_shape_ok(wt, k, batch) != 0) return -3;
    const int64_t rb = k / block_elems_of(wt) * block_bytes_of(wt);
    const Plan p = make_plan(wt, k, rb, static_cast<int>(batch), true);
    const uint8_t* wg = static_cast<const uint8_t*>(w_gate);
    const uint8_t* wu = static_cast<const uint8_t*>(w_up);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int64_t xrb = k / 32 * 34;
    const int b = static_cast<int>(batch);
    switch (wt) {
        case T_Q4_0: return launch_sw<T_Q4_0>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_Q4_1: return launch_sw<T_Q4_1>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_Q8_0: return launch_sw<T_Q8_0>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_Q4_K: return launch_sw<T_Q4_K>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_Q5_K: return launch_sw<T_Q5_K>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_Q6_K: return launch_sw<T_Q6_K>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_Q1_0: return launch_sw<T_Q1_0>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        case T_TQ2: return launch_sw<T_TQ2>(p.SC, p.KS, b, wg, wu, n, rb, p.ncols, xp, xrb, h, ldh, stream);
        default: return -2;
    }
}

// ---- routed experts at decode: one GEMV per token-expert pair ---------------
// One wave per row (k <= 4096, whole 16-byte rows, aligned xq); pairs beyond
// grid.y's range are refused.
int moe_gemv_shape_ok(int wt, int64_t k, int64_t npairs) {
    if (npairs > 65535 || gemv_swiglu_shape_ok(wt, k, 1) != 0) return -3;
    const Plan p = make_plan(wt, k, k / block_elems_of(wt) * block_bytes_of(wt), 1, true);
    return p.KS == 1 ? 0 : -3;
}

template <int FMT, bool SW>
int launch_moe_gemv_fmt(int SC, const uint8_t* w, const uint8_t* w2, int64_t n, int64_t rb,
                        int ncols, const uint8_t* xq, int64_t xrb, float* y, int64_t ldy,
                        const MoeMap& mm, int npairs, hipStream_t s) {
    if (SC == 1) return launch_stream<FMT, 1, 1, SW, true>(w, n, rb, ncols, xq, xrb, y, ldy, s, w2, mm, npairs);
    if constexpr (!kOneCol<FMT>)
        if (SC == 2) return launch_stream<FMT, 1, 2, SW, true>(w, n, rb, ncols, xq, xrb, y, ldy, s, w2, mm, npairs);
    return -3;
}

template <bool SW>
int launch_moe_gemv_any(int wt, const void* w, const void* w2, int64_t n_experts, int64_t n,
                        int64_t k, const void* xq, int x_per_pair, const int32_t* ids,
                        int64_t n_tokens, int64_t top_k, float* y, int64_t ldy, int32_t* status,
                        hipStream_t s) {
    const int64_t npairs = n_tokens * top_k;
    if (moe_gemv_shape_ok(wt, k, npairs) != 0) return -3;
    const int64_t rb = k / block_elems_of(wt) * block_bytes_of(wt);
    const Plan p = make_plan(wt, k, rb, 1, true);
    const MoeMap mm{ids, n * rb, static_cast<int>(n_experts), static_cast<int>(top_k), x_per_pair,
                    status};
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* wp2 = static_cast<const uint8_t*>(w2);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int64_t xrb = k / 32 * 34;
    const int np = static_cast<int>(npairs);
    switch (wt) {
        case T_Q4_0: return launch_moe_gemv_fmt<T_Q4_0, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_Q4_1: return launch_moe_gemv_fmt<T_Q4_1, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_Q8_0: return launch_moe_gemv_fmt<T_Q8_0, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_Q4_K: return launch_moe_gemv_fmt<T_Q4_K, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_Q5_K: return launch_moe_gemv_fmt<T_Q5_K, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_Q6_K: return launch_moe_gemv_fmt<T_Q6_K, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_Q1_0: return launch_moe_gemv_fmt<T_Q1_0, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        case T_TQ2: return launch_moe_gemv_fmt<T_TQ2, SW>(p.SC, wp, wp2, n, rb, p.ncols, xp, xrb, y, ldy, mm, np, s);
        default: return -2;
    }
}

int launch_moe_gemv(int wt, const void* w_experts, int64_t n_experts, int64_t n, int64_t k,
                    const void* xq, int x_per_pair, const int32_t* ids, int64_t n_tokens,
                    int64_t top_k, float* y, int64_t ldy, int32_t* status, hipStream_t stream) {
    return launch_moe_gemv_any<false>(wt, w_experts, nullptr, n_experts, n, k, xq, x_per_pair, ids,
                                      n_tokens, top_k, y, ldy, status, stream);
}

int launch_moe_gemv_swiglu(int wt, const void* w_gate, const void* w_up, int64_t n_experts,
                           int64_t n, int64_t k, const void* xq, const int32_t* ids,
                           int64_t n_tokens, int64_t top_k, float* h, int64_t ldh,
                           int32_t* status, hipStream_t stream) {
    return launch_moe_gemv_any<true>(wt, w_gate, w_up, n_experts, n, k, xq, 0, ids, n_tokens,
                                     top_k, h, ldh, status, stream);
}

}  // namespace cq

// gemv.hip -- decode GEMV over GGUF blocks (Q4_0, Q4_1, Q8_0, Q4_K) for
// 1..8 Q8_0 activation rows.
//
// Design (HBM-bound; the weights are read exactly once):
//  * A workgroup owns row tiles of RT consecutive weight rows.  Because GGUF
//    rows are stored back to back, a tile is one contiguous byte range; all
//    threads stage it into LDS with fully coalesced 16-byte loads (a wave
//    reads 1 KiB per instruction), whatever the 18/20/34/144-byte block
//    size.  Blocks are then re-sliced out of LDS.
//  * Each lane owns fixed "columns" of K (one 32-value block, or for Q4_K one
//    32-byte nibble chunk = two 32-value sub-blocks) and keeps the Q8_0
//    activation of its columns, for all batch rows, in registers for the
//    workgroup's lifetime; a grid-stride loop over tiles amortizes that load.
//  * Per block: nibble unpack in registers, v_dot4 integer dots against the
//    activation quants, scales applied once per 32-value block in fp32
//    (alice-llm 2.0.0 README, "Computation Path (Q4_K)").  Batch rows share
//    the decoded weight registers (alice-llm 2.0.0 README, "Batch-4
//    Speculative Decoding": one accumulator register per row).
//  * Cross-lane sums are wave64 DPP reductions (alice-llm 2.0.0 README, "The
//    GPU Optimization Journey", phase 2: subgroup reduction instead of a
//    shared-memory tree); with more than one wave per row the per-wave sums
//    meet in LDS and are added in wave order.
//  * The column split depends only on (type, k), never on the batch size, so
//    batch row b gives bitwise the batch-1 result.
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {
namespace {

enum { T_Q4_0 = 2, T_Q4_1 = 3, T_Q8_0 = 8, T_Q4_K = 12 };

// columns per lane: a Q4_K column already spans 64 values
template <int FMT> constexpr int kCMax = (FMT == T_Q4_K) ? 1 : 2;
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

template <int FMT> struct Act {
    uint32_t q[8];  // 32 int8 quants
    float dx;       // block scale
    float ndx;      // -12582912 * dx
    float sdx;      // dx * sum(q)                  (Q4_1)
    int start;      // kBias (- 8 * sum(q) for Q4_0): start value of the dot
};
template <> struct Act<T_Q4_K> {
    uint32_t qa[8], qb[8];  // the two 32-value blocks under one nibble chunk
    float dxa, dxb;
    float ndxa, ndxb;       // -12582912 * dx
    float sa, sb;           // dx * sum(q) of each block
};

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Load one 34-byte Q8_0 activation block (2-byte aligned) from global memory.
__device__ __forceinline__ void load_q8(const uint8_t* p, uint32_t* q, float* dx, int* sum) {
    const uint16_t* s = reinterpret_cast<const uint16_t*>(p);
    *dx = h2f(s[0]);
    int acc = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        q[t] = static_cast<uint32_t>(s[1 + 2 * t]) | (static_cast<uint32_t>(s[2 + 2 * t]) << 16);
        acc = sdot4(q[t], 0x01010101u, acc);
    }
    *sum = acc;
}

template <int FMT>
__device__ __forceinline__ void load_act(const uint8_t* xq_row, int col, Act<FMT>& a) {
    int s;
    load_q8(xq_row + static_cast<int64_t>(col) * 34, a.q, &a.dx, &s);
    a.start = (FMT == T_Q4_0) ? kBias - 8 * s : kBias;
    a.ndx = -kBiasF * a.dx;
    a.sdx = a.dx * static_cast<float>(s);
}
template <>
__device__ __forceinline__ void load_act<T_Q4_K>(const uint8_t* xq_row, int col, Act<T_Q4_K>& a) {
    int sa, sb;
    load_q8(xq_row + static_cast<int64_t>(2 * col) * 34, a.qa, &a.dxa, &sa);
    load_q8(xq_row + static_cast<int64_t>(2 * col + 1) * 34, a.qb, &a.dxb, &sb);
    a.sa = a.dxa * static_cast<float>(sa);
    a.sb = a.dxb * static_cast<float>(sb);
    a.ndxa = -kBiasF * a.dxa;
    a.ndxb = -kBiasF * a.dxb;
}

// Byte offset, inside the staged tile, of the block that holds column col
// of tile row r.
template <int FMT>
__device__ __forceinline__ int col_offset(int row_base, int col) {
    if constexpr (FMT == T_Q4_K) return row_base + (col >> 2) * 144;
    else return row_base + col * Fmt<FMT>::BS;
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
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            lo[t] = q[t] & 0x0F0F0F0Fu;
            hi[t] = (q[t] >> 4) & 0x0F0F0F0Fu;
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            int sa = kBias, sb = kBias, sa1 = 0, sb1 = 0;  // four chains at batch 1
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

    // columns of this lane and their activations, resident for the whole kernel
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
            if (valid[i]) load_act<FMT>(xq + j * xq_row_bytes, col[i], act[i][j]);
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

// ---- single-wave variant: one wave covers all of k (every lane owns its
// columns), so waves never wait for each other.  Each wave streams its row
// tiles HBM -> LDS with LDS-DMA (global_load_lds_dwordx4: 16 bytes per lane,
// 1 KiB per instruction, no VGPRs) through a ring of kRing wave-private
// buffers: while tile t is computed, tiles t+1 .. t+kRing-1 are in flight.
// The weights are read once, so the DMA carries the non-temporal hint.
//
// Wait accounting: every tile is exactly kDmaVec DMA instructions, each with
// at least one active lane (lanes past the tile are masked off; an
// instruction wholly past it re-loads the tile's first KiB onto the buffer's
// first KiB), and every processed tile issues exactly one global store, so
// the number of vector-memory operations issued after a tile's DMA is a
// compile-time constant and an explicit s_waitcnt vmcnt(N) suffices.  The
// DMA is issued from inline assembly: the compiler then does not model it,
// and places no waits of its own for it (its waits for its own loads can
// only become more conservative); all waits for the DMA are the explicit
// ones below.
constexpr int kRing = 2;                           // buffers per wave
constexpr int kTileCap = 9232;                     // tile bytes incl. up to 15 lead bytes
constexpr int kDmaVec = (kTileCap + 1023) / 1024;  // 1-KiB DMA instructions per tile
constexpr int kDmaBufBytes = kTileCap + 64;        // + read slack past the last block
constexpr int kWavesPerCu = 8;                     // most waves per CU (kRing buffers each)
// waves per CU launched: Q8_0's per-tile work (two unaligned 34-byte blocks
// per lane and row) runs best with six, the others with eight
template <int FMT> constexpr int kWaveGrid = FMT == T_Q8_0 ? 6 : kWavesPerCu;
static_assert(kRing >= 2 && kRing <= 4, "ring depth");
static_assert(kRing * kWavesPerCu * kDmaBufBytes <= 160 * 1024, "LDS per CU");
static_assert(kDmaVec * 64 * 16 >= kTileCap && (kDmaVec - 1) * 1024 < kTileCap, "instruction count");

template <int N>
__device__ __forceinline__ void wait_vmem() {      // s_waitcnt vmcnt(N)
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS byte offset of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    typedef const __attribute__((address_space(3))) uint8_t* lds_ptr;
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(p)));
}

// One LDS-DMA instruction: each active lane copies the 16 bytes at gaddr (its
// own) to LDS[lds_base + 16*lane]; lds_base must be wave-uniform.  M0 carries
// the LDS base; it is saved and restored around the instruction, with one
// wait state between the M0 write and the DMA that reads it.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gaddr), "s"(lds_base)
        : "memory");
}

// Stage bytes [a0, a0 + 16*nvec) of w (a0 16-aligned, 1 <= nvec,
// 16*nvec <= kTileCap, a0 + 16*nvec <= size of w) into buf with exactly
// kDmaVec DMA instructions.  Instruction u covers vectors 64u .. 64u+63 with
// the lanes past nvec masked off; an instruction with 64u >= nvec instead
// re-loads the tile's own first vectors (lanes < nvec) onto the same bytes of
// the buffer, so every instruction has lane 0 active and none writes past
// 16*nvec.
__device__ __forceinline__ void dma_tile(const uint8_t* __restrict__ w, int64_t a0, int nvec,
                                         uint8_t* buf, int lane) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_offset(buf));
#pragma unroll
    for (int u = 0; u < kDmaVec; ++u) {
        if (u * kWave < nvec) {               // wave-uniform
            const int v = u * kWave + lane;
            if (v < nvec) dma16(w + a0 + 16 * static_cast<int64_t>(v), base + u * kWave * 16);
        } else {
            // the tile's first vectors again, onto the same bytes (lanes past
            // nvec masked as above, lane 0 always active)
            if (lane < nvec) dma16(w + a0 + 16 * static_cast<int64_t>(lane), base);
        }
    }
}

// Sum each of the V = RT*B accumulators over the 64 lanes and store row r,
// batch j to y[j*ldy + r0 + r] (r < rt) with one store instruction.
// Groups of four values are transposed across the wave with
// permlane32_swap / permlane16_swap so that each 16-lane row holds one
// value, then each row is summed with four DPP steps.  The association
// order is the same for every value slot.
template <int RT, int B>
__device__ __forceinline__ void reduce_store(float (&acc)[RT][B], int rt, int64_t r0,
                                             float* __restrict__ y, int64_t ldy, int lane) {
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
    const int row = lane >> 4, g = lane & 15;
    const int idx = 4 * g + (row == 1 ? 2 : (row == 2 ? 1 : row));
    const int r = idx / B, j = idx - (idx / B) * B;
    if (g < NG && idx < V && r < rt) y[j * ldy + r0 + r] = out;
}

template <int FMT, int B, int RT>
__global__ __launch_bounds__(kWave) void gemv_wave_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t rb, int ncols, int C,
        const uint8_t* __restrict__ xq, int64_t xq_row_bytes, float* __restrict__ y,
        int64_t ldy) {
    __shared__ __align__(16) uint8_t ring[kRing][kDmaBufBytes];
    const int lane = threadIdx.x;

    constexpr int CM = kCMax<FMT>;
    int col[CM];
    bool valid[CM];
#pragma unroll
    for (int i = 0; i < CM; ++i) {
        col[i] = i * kWave + lane;
        valid[i] = (i < C) && (col[i] < ncols);
    }
    Act<FMT> act[CM][B];  // loaded once the first tiles are in flight

    const int64_t G = gridDim.x;
    const int64_t ntiles = (n + RT - 1) / RT;
    const int64_t nt = ntiles > blockIdx.x ? (ntiles - blockIdx.x + G - 1) / G : 0;
    auto tile_of = [&](int64_t i) { return blockIdx.x + i * G; };
    auto issue = [&](int64_t i, uint8_t* buf) {
        const int64_t r0 = tile_of(i) * RT;
        const int rt = static_cast<int>(n - r0 < RT ? n - r0 : RT);
        const int64_t a0 = (r0 * rb) & ~static_cast<int64_t>(15);
        const int nvec = (static_cast<int>(r0 * rb - a0) + rt * static_cast<int>(rb) + 15) >> 4;
        wait_lds_all();  // earlier reads of this buffer have completed
        dma_tile(w, a0, nvec, buf, lane);
    };
    auto process = [&](int64_t i, const uint8_t* buf) {
        const int64_t r0 = tile_of(i) * RT;
        const int rt = static_cast<int>(n - r0 < RT ? n - r0 : RT);
        const int delta = static_cast<int>(r0 * rb - ((r0 * rb) & ~static_cast<int64_t>(15)));
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
                for (int c = 0; c < CM; ++c)
                    if (valid[c])
                        column_dot<FMT, B>(buf, col_offset<FMT>(row_base, col[c]), act[c],
                                           acc[r], col[c]);
            }
        }
        reduce_store<RT, B>(acc, rt, r0, y, ldy, lane);
    };
    // Tile i lives in buffer i % kRing.  Step i issues tile i+kRing-1 (into
    // the buffer computed in step i-1), waits for tile i, computes it and
    // stores its outputs.  Vector-memory operations issued after tile i's DMA
    // by the time of that wait: the DMAs of tiles i+1 .. i+kRing-1 and the
    // stores of the min(i, kRing-1) steps before i.  Once no tile is left to
    // issue, the wait drains everything.
    constexpr int kAhead = (kRing - 1) * kDmaVec;
    auto step = [&](int64_t i, const uint8_t* cur, uint8_t* nxt) {
        if (i + kRing - 1 < nt) {
            issue(i + kRing - 1, nxt);
            const int64_t stores = i < kRing - 1 ? i : kRing - 1;
            if (stores == 0) wait_vmem<kAhead>();
            else if (stores == 1) wait_vmem<kAhead + 1>();
            else if (stores == 2) wait_vmem<kAhead + 2>();
            else wait_vmem<kAhead + 3>();
        } else {
            wait_vmem<0>();
        }
        process(i, cur);
    };
#pragma unroll
    for (int d = 0; d < kRing - 1; ++d)
        if (d < nt) issue(d, ring[d]);
    // the activations are loaded after the first tiles are in flight, so the
    // latencies overlap (their loads only add completed operations to the
    // counts above, which stay upper bounds).  Unconditional loads (an
    // unused column reads column 0 and is never consumed) keep all of them in
    // flight together.
#pragma unroll
    for (int i = 0; i < CM; ++i)
#pragma unroll
        for (int j = 0; j < B; ++j)
            load_act<FMT>(xq + j * xq_row_bytes, valid[i] ? col[i] : 0, act[i][j]);
    for (int64_t i = 0; i < nt; i += kRing) {
        step(i, ring[0], ring[kRing - 1]);
        if (i + 1 >= nt) break;
        step(i + 1, ring[1], ring[0]);
        if constexpr (kRing > 2) {
            if (i + 2 >= nt) break;
            step(i + 2, ring[2], ring[1]);
        }
        if constexpr (kRing > 3) {
            if (i + 3 >= nt) break;
            step(i + 3, ring[3], ring[2]);
        }
    }
}

struct Plan {
    int ncols, C, nw, RT, tile_lds, red_bytes;
    bool wave;  // single-wave LDS-DMA kernel
};

// wave_ok: the single-wave LDS-DMA kernel may be used (the matrix is a whole
// number of 16-byte vectors, so no tile ends inside a vector).
Plan make_plan(int wt, int64_t k, int64_t rb, int batch, bool wave_ok) {
    Plan p{};
    p.ncols = static_cast<int>(wt == T_Q4_K ? k / 64 : k / 32);
    p.C = (wt == T_Q4_K || p.ncols <= kWave) ? 1 : 2;
    p.nw = (p.ncols + kWave * p.C - 1) / (kWave * p.C);
    // rows per tile: about 16 KiB of weights per tile, at most 32 live
    // accumulators per lane
    int rt = 8;
    while (rt > 1 && (rt * rb > 20480 || rt * batch > 32)) rt >>= 1;
    if (rt == 2) rt = 1;  // instantiated tiles: 1, 4, 8
    if (p.nw == 1 && wave_ok) {  // single-wave kernel: tiles bounded by its LDS buffers
        static constexpr int kRts[] = {8, 4, 3, 2, 1};
        for (int cand : kRts) {
            if (cand * rb + 15 <= kTileCap && cand * batch <= 32) {
                rt = cand;
                p.wave = true;
                break;
            }
        }
    }
    p.RT = rt;
    p.tile_lds = static_cast<int>((rt * rb + 32 + 15) & ~15);
    p.red_bytes = p.nw > 1 ? p.nw * rt * batch * 4 : 0;
    return p;
}

template <int FMT, int B>
int launch_fmt_b(const Plan& p, const uint8_t* w, int64_t n, int64_t rb, const uint8_t* xq,
                 int64_t xrb, float* y, int64_t ldy, hipStream_t stream) {
    const int64_t ntiles = (n + p.RT - 1) / p.RT;
    if (p.wave) {
        int64_t grid = static_cast<int64_t>(device_cu_count()) * kWaveGrid<FMT>;
        if (grid > ntiles) grid = ntiles;
        const dim3 g(static_cast<unsigned>(grid)), b(kWave);
        switch (p.RT) {
            case 8:
                if constexpr (B <= 4) {
                    hipLaunchKernelGGL((gemv_wave_kernel<FMT, B, 8>), g, b, 0, stream, w, n, rb,
                                       p.ncols, p.C, xq, xrb, y, ldy);
                    break;
                } else {
                    return -3;
                }
            case 4: hipLaunchKernelGGL((gemv_wave_kernel<FMT, B, 4>), g, b, 0, stream, w, n, rb,
                                       p.ncols, p.C, xq, xrb, y, ldy); break;
            case 3: hipLaunchKernelGGL((gemv_wave_kernel<FMT, B, 3>), g, b, 0, stream, w, n, rb,
                                       p.ncols, p.C, xq, xrb, y, ldy); break;
            case 2: hipLaunchKernelGGL((gemv_wave_kernel<FMT, B, 2>), g, b, 0, stream, w, n, rb,
                                       p.ncols, p.C, xq, xrb, y, ldy); break;
            default: hipLaunchKernelGGL((gemv_wave_kernel<FMT, B, 1>), g, b, 0, stream, w, n, rb,
                                        p.ncols, p.C, xq, xrb, y, ldy); break;
        }
        return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    const int per_cu = p.nw >= 4 ? 2 : 8 / p.nw;
    int64_t grid = static_cast<int64_t>(device_cu_count()) * per_cu;
    if (grid > ntiles) grid = ntiles;
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

}  // namespace

// Returns 0, -3 (shape the kernel cannot tile) or -6 (launch failure).
int gemv_shape_ok(int wt, int64_t k, int64_t batch) {
    const int64_t bs = wt == T_Q4_0 ? 18 : wt == T_Q4_1 ? 20 : wt == T_Q8_0 ? 34 : 144;
    const int64_t qk = wt == T_Q4_K ? 256 : 32;
    const Plan p = make_plan(wt, k, k / qk * bs, static_cast<int>(batch), false);
    if (p.nw * kWave > kMaxThreads) return -3;
    if (!p.wave && p.tile_lds + p.red_bytes > 65536) return -3;
    return 0;
}

int launch_gemv(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t batch,
                float* y, int64_t ldy, hipStream_t stream) {
    if (gemv_shape_ok(wt, k, batch) != 0) return -3;
    const int64_t bs = wt == T_Q4_0 ? 18 : wt == T_Q4_1 ? 20 : wt == T_Q8_0 ? 34 : 144;
    const int64_t qk = wt == T_Q4_K ? 256 : 32;
    const int64_t rb = k / qk * bs;
    const Plan p = make_plan(wt, k, rb, static_cast<int>(batch), (n * rb) % 16 == 0);
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int64_t xrb = k / 32 * 34;
    const int b = static_cast<int>(batch);
    switch (wt) {
        case T_Q4_0: return launch_fmt<T_Q4_0>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q4_1: return launch_fmt<T_Q4_1>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q8_0: return launch_fmt<T_Q8_0>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        case T_Q4_K: return launch_fmt<T_Q4_K>(p, b, wp, n, rb, xp, xrb, y, ldy, stream);
        default: return -2;
    }
}

}  // namespace cq

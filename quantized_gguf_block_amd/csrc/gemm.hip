// gemm.hip -- prefill GEMM over GGUF blocks with int8 MFMA on gfx950.
//
//   y[m][n] = sum over 32-value blocks b of dx[m,b] * dw[n,b] * I[m,n,b],
//   I[m,n,b] = sum_i wq[n, 32b+i] * xq[m, 32b+i]   (exact int32)
//
// (alice-llm 2.0.0 README, "Computation Path (Q4_K)": integer dot inside
// each 32-value block, scales applied once per block.)
//
// Tiling: a 256-thread workgroup owns 128 tokens x 128 weight rows and walks
// k in steps of 4 blocks (128 values).  Per step the weight blocks are
// decoded once into signed int8 rows in LDS (Q4_0: q-8, Q4_1 / Q4_K: q,
// Q5_K: q with its qh bit, Q6_K: q-32) and the Q8_0 activation blocks are
// split into int8 rows plus fp32 scales.  Q6_K's 16-value scale groups take
// one v_mfma_i32_32x32x16_i8 each (two rescales per 32 values).
// Each wave computes 64 x 64 outputs as 2 x 2 tiles of
// v_mfma_i32_32x32x32_i8: one MFMA is exactly one 32-value block.
//
// Scale application: the MFMA accumulator starts from the bit pattern of
// 1.5*2^23 (12582912.0f), so the int32 result read as a float is exactly
// 12582912 + I (|I| < 2^22).  Then t = fma(D, dx, -12582912*dx) = round(I*dx)
// (the subtrahend is exact: dx has 11 significant bits) and
// acc = fma(t, dw, acc): two VALU FMAs per output and block, no convert.
// With packed-FP32 instructions disabled this VALU work, not the MFMA, is
// the bound: 2 lane-FMAs per output per block against 1/128 of a CU-clock
// of MFMA time, i.e. at most a quarter of the int8 MFMA peak.
//
// Q4_1 and Q4_K also carry an additive term per block, sum_b (dx*sum(xq))[m,b]
// * c[n,b] with c = m (Q4_1) or -dmin*min (Q4_K).  That is itself a matrix
// product over blocks; it is accumulated with fp32 MFMA
// (v_mfma_f32_32x32x2_f32, two blocks per instruction) into the same
// accumulators, so it costs MFMA time, not VALU time.
#include "cq_device.h"
#include "cq_internal.h"

namespace cq {
namespace {

enum { T_Q4_0 = 2, T_Q4_1 = 3, T_Q8_0 = 8, T_Q4_K = 12, T_Q5_K = 13, T_Q6_K = 14 };

// Q4_K and Q5_K share the super-block header and nibble chunks (Q5_K adds a
// high bit per value from qh[32])
template <int FMT> constexpr bool kK45 = (FMT == T_Q4_K || FMT == T_Q5_K);

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int KB = 4;            // 32-value blocks per k step
constexpr int ROW = KB * 32 + 16;  // LDS row stride of the int8 tiles (16 B pad)
constexpr int kThreads = 256;
constexpr int kBias = 0x4B400000;
constexpr float kBiasF = 12582912.0f;

template <int FMT> constexpr bool kHasOffset = (FMT == T_Q4_1 || kK45<FMT>);

// Workgroup tile of BM tokens x BN weight rows: 4 waves arranged WMW x WNW,
// each wave MI x NI tiles of 32 x 32.
template <int WMW, int WNW, int MI, int NI>
struct Tile {
    static constexpr int BM = WMW * MI * 32;
    static constexpr int BN = WNW * NI * 32;
    static_assert(WMW * WNW == 4, "four waves");
    static_assert(BN == 128 && BM <= 128, "staging assumes 128 weight rows, <= 128 tokens");
};

template <int BM, int BN>
struct Smem {
    int8_t w[BN * ROW];       // decoded weight quants, row n, k within the step
    int8_t x[BM * ROW];       // activation quants
    float dw[KB][BN];         // weight block scale (Q4_K: d*sc; Q6_K: d*sc of values 0..15)
    float dw2[KB][BN];        // Q6_K: d*sc of values 16..31
    float dx[KB][BM];         // activation block scale
    float cw[KB][BN];         // Q4_1: m; Q4_K: -dmin*min  (additive weight term)
    float sx[KB][BM];         // dx * sum of the block's activation quants
    int xrow[BM];             // activation row of each tile row (-1: none)
    int yrow[BM];             // output row of each tile row
};

__device__ __forceinline__ uint32_t nib_lo_s8(uint32_t v) {   // low nibbles as q-8
    return ((v & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t nib_hi_s8(uint32_t v) {
    return (((v >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u;
}
__device__ __forceinline__ uint32_t nib_lo(uint32_t v) { return v & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t v) { return (v >> 4) & 0x0F0F0F0Fu; }

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Bytes [off, off+4*N) of a little-endian byte stream held in dwords
// w[0..] (off even, known at compile time after unrolling).
template <int N>
__device__ __forceinline__ void extract(const uint32_t* w, int off, uint32_t* out) {
#pragma unroll
    for (int t = 0; t < N; ++t) {
        const int o = off + 4 * t;
        out[t] = (o & 2) ? __builtin_amdgcn_alignbit(w[(o >> 2) + 1], w[o >> 2], 16) : w[o >> 2];
    }
}
__device__ __forceinline__ uint32_t half_at(const uint32_t* w, int off) {
    return (w[off >> 2] >> ((off & 2) * 8)) & 0xFFFFu;
}

// ---- staging of one k step --------------------------------------------------
// Two threads per row: thread t stages row t/2, blocks 2*(t%2) and
// 2*(t%2)+1 of the step.  Staging is split into the global loads (into
// registers) and the decode into LDS, so the loads of step ks+1 are in flight
// while step ks is computed.  The loads are unconditional: a weight row past
// n reads row n-1 and a tile row without an activation row reads row 0; the
// outputs of such rows are never stored.  (A load under a branch is merged
// with the other branch's value by a register copy, which waits for it at
// once.)
template <int FMT> struct WRaw {      // two 32-value blocks of one row
    static constexpr int BS = (FMT == T_Q4_0) ? 18 : (FMT == T_Q4_1) ? 20 : 34;
    uint32_t v[(2 * BS) / 4];
};
template <> struct WRaw<T_Q4_K> {     // super-block header + one 32-byte chunk
    uint32_t hdr[4], q[8];
};
template <> struct WRaw<T_Q5_K> {     // header, the 32 qh bytes, one 32-byte chunk
    uint32_t hdr[4], qh[8], q[8];
};
template <> struct WRaw<T_Q6_K> {     // one 32-byte ql run and the qh bytes of a half
    uint32_t ql[9], qh[9];            // dword-aligned covers (see load_weights)
    uint32_t sc0, sc1;                // scale byte pairs of the two quadrants
    uint32_t d;                       // fp16 d
    uint32_t sh;                      // 16 when the runs start 2 bytes into a dword
};
struct XRaw {                         // two Q8_0 activation blocks
    uint32_t v[17];
};

template <int FMT>
__device__ __forceinline__ void load_weights(WRaw<FMT>& r, const uint8_t* __restrict__ w, int64_t n,
                                             int64_t rb, int64_t n0, int kstep) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    const int64_t gn = n0 + row < n ? n0 + row : n - 1;
    if constexpr (FMT == T_Q6_K) {
        // A k step is one 128-value half h of super-block sb; this thread
        // decodes quadrants g = half and half + 2 of it, which share the ql
        // run [64h + 32*half, +32) (low and high nibbles).  Super-blocks are
        // 210 bytes, so the runs may start 2 bytes into a dword: the dwords
        // covering them are loaded through a buffer descriptor over the
        // matrix (reads past it return zeros) and re-aligned when stored.
        const int h = kstep & 1;
        const uintptr_t wa = reinterpret_cast<uintptr_t>(w);
        const uint8_t* wal = reinterpret_cast<const uint8_t*>(wa & ~static_cast<uintptr_t>(3));
        const int delta = static_cast<int>(wa & 3);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(wal), 0, static_cast<int>(delta + n * rb), 0x00020000);
        const int base = delta + static_cast<int>(gn * rb) + (kstep >> 1) * 210;
        const int mis = base & 2;
        r.sh = static_cast<uint32_t>(mis) * 8;
        const int aql = base + 64 * h + 32 * half - mis, aqh = base + 128 + 32 * h - mis;
#pragma unroll
        for (int i = 0; i < 9; ++i) {
            r.ql[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, aql + 4 * i, 0, 0);
            r.qh[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, aqh + 4 * i, 0, 0);
        }
        r.sc0 = __builtin_amdgcn_raw_buffer_load_b16(rs, base + 192 + 8 * h + 2 * half, 0, 0);
        r.sc1 = __builtin_amdgcn_raw_buffer_load_b16(rs, base + 196 + 8 * h + 2 * half, 0, 0);
        r.d = __builtin_amdgcn_raw_buffer_load_b16(rs, base + 208, 0, 0);
    } else if constexpr (kK45<FMT>) {
        // a 256-value super-block spans two k steps; this step holds nibble
        // chunks 2*(kstep&1) and +1, this thread chunk c (sub-blocks 2c, 2c+1)
        constexpr int SB = FMT == T_Q4_K ? 144 : 176, QS = FMT == T_Q4_K ? 16 : 48;
        const int c = 2 * (kstep & 1) + half;
        const uint8_t* p = w + gn * rb + static_cast<int64_t>(kstep >> 1) * SB;
        const uint4 hv = *reinterpret_cast<const uint4*>(p);
        r.hdr[0] = hv.x; r.hdr[1] = hv.y; r.hdr[2] = hv.z; r.hdr[3] = hv.w;
        if constexpr (FMT == T_Q5_K) {
            const uint4 h0 = *reinterpret_cast<const uint4*>(p + 16);
            const uint4 h1 = *reinterpret_cast<const uint4*>(p + 32);
            r.qh[0] = h0.x; r.qh[1] = h0.y; r.qh[2] = h0.z; r.qh[3] = h0.w;
            r.qh[4] = h1.x; r.qh[5] = h1.y; r.qh[6] = h1.z; r.qh[7] = h1.w;
        }
        const uint4 v0 = *reinterpret_cast<const uint4*>(p + QS + 32 * c);
        const uint4 v1 = *reinterpret_cast<const uint4*>(p + QS + 16 + 32 * c);
        r.q[0] = v0.x; r.q[1] = v0.y; r.q[2] = v0.z; r.q[3] = v0.w;
        r.q[4] = v1.x; r.q[5] = v1.y; r.q[6] = v1.z; r.q[7] = v1.w;
    } else {
        constexpr int BS = WRaw<FMT>::BS;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(
            w + gn * rb + (static_cast<int64_t>(kstep) * KB + 2 * half) * BS);
#pragma unroll
        for (int i = 0; i < (2 * BS) / 4; ++i) r.v[i] = p[i];
    }
}

template <int FMT, class S>
__device__ __forceinline__ void store_weights(S& s, const WRaw<FMT>& r, int kstep) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    if constexpr (FMT == T_Q6_K) {
        const float d = h2f(r.d);
        uint32_t ql[8], qh[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ql[i] = __builtin_amdgcn_alignbit(r.ql[i + 1], r.ql[i], r.sh);
            qh[i] = __builtin_amdgcn_alignbit(r.qh[i + 1], r.qh[i], r.sh);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int g = half + 2 * e;       // quadrant = local block of the step
            const uint32_t scp = e ? r.sc1 : r.sc0;  // signed scales of values 0..15, 16..31
            s.dw[g][row] = d * static_cast<float>(static_cast<int8_t>(scp & 0xFFu));
            s.dw2[g][row] = d * static_cast<float>(static_cast<int8_t>((scp >> 8) & 0xFFu));
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t nib = e ? (ql[i] >> 4) & 0x0F0F0F0Fu : ql[i] & 0x0F0F0F0Fu;
                const uint32_t v = nib | (((qh[i] >> (2 * g)) & 0x03030303u) << 4);   // 0..63
                o[i] = (v + 0x60606060u) ^ 0x80808080u;   // v - 32 per byte, no carries
            }
            uint4* d4 = reinterpret_cast<uint4*>(s.w + row * ROW + 32 * g);
            d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    } else if constexpr (kK45<FMT>) {
        const int c = 2 * (kstep & 1) + half;
        const float d = h2f(r.hdr[0] & 0xFFFFu), dmin = h2f(r.hdr[0] >> 16);
        const uint32_t S0 = r.hdr[1], S1 = r.hdr[2], S2 = r.hdr[3];
#pragma unroll
        for (int e = 0; e < 2; ++e) {             // sub-block j = 2c + e -> local block 2*half + e
            const int j = 2 * c + e;
            int sc, mn;
            if (j < 4) {
                sc = (S0 >> (8 * j)) & 63;
                mn = (S1 >> (8 * j)) & 63;
            } else {
                const int sh = 8 * (j - 4);
                sc = ((S2 >> sh) & 0xF) | ((((S0 >> sh) >> 6) & 3) << 4);
                mn = (((S2 >> sh) >> 4) & 0xF) | ((((S1 >> sh) >> 6) & 3) << 4);
            }
            const int b = 2 * half + e;
            s.dw[b][row] = d * static_cast<float>(sc);
            s.cw[b][row] = -(dmin * static_cast<float>(mn));
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                o[i] = e ? nib_hi(r.q[i]) : nib_lo(r.q[i]);
                // Q5_K: bit j of qh byte l is bit 4 of value l of sub-block j
                if constexpr (FMT == T_Q5_K) o[i] |= ((r.qh[i] >> j) & 0x01010101u) << 4;
            }
            uint4* d4 = reinterpret_cast<uint4*>(s.w + row * ROW + 32 * b);
            d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    } else {
        constexpr int BS = WRaw<FMT>::BS;
#pragma unroll
        for (int bl = 0; bl < 2; ++bl) {
            const int b = 2 * half + bl;
            uint32_t o[8];
            s.dw[b][row] = h2f(half_at(r.v, bl * BS));
            if constexpr (FMT == T_Q8_0) {
                extract<8>(r.v, bl * BS + 2, o);
            } else {
                uint32_t q[4];
                extract<4>(r.v, bl * BS + (FMT == T_Q4_0 ? 2 : 4), q);
                if constexpr (FMT == T_Q4_1) s.cw[b][row] = h2f(half_at(r.v, bl * BS + 2));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = (FMT == T_Q4_0) ? nib_lo_s8(q[i]) : nib_lo(q[i]);
                    o[4 + i] = (FMT == T_Q4_0) ? nib_hi_s8(q[i]) : nib_hi(q[i]);
                }
            }
            uint4* d4 = reinterpret_cast<uint4*>(s.w + row * ROW + 32 * b);
            d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

// Activations: threads t < 2*BM stage tile row t/2 (activation row
// s.xrow[t/2]), blocks 2*(t%2) and +1 of the step.
template <int BM, class S>
__device__ __forceinline__ void load_acts(XRaw& r, const S& s, const uint8_t* __restrict__ xq,
                                          int64_t xrb, int kstep) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    if (2 * BM < kThreads && row >= BM) return;
    const int gm = s.xrow[row] < 0 ? 0 : s.xrow[row];
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        xq + static_cast<int64_t>(gm) * xrb + (static_cast<int64_t>(kstep) * KB + 2 * half) * 34);
#pragma unroll
    for (int i = 0; i < 17; ++i) r.v[i] = p[i];
}

template <int FMT, int BM, class S>
__device__ __forceinline__ void store_acts(S& s, const XRaw& r) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    if (2 * BM < kThreads && row >= BM) return;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
        const int b = 2 * half + bl;
        uint32_t o[8];
        extract<8>(r.v, bl * 34 + 2, o);
        const float dx = h2f(half_at(r.v, bl * 34));
        s.dx[b][row] = dx;
        if constexpr (kHasOffset<FMT>) {
            int sum = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum = sdot4(o[i], 0x01010101u, sum);
            s.sx[b][row] = dx * static_cast<float>(sum);
        }
        uint4* d4 = reinterpret_cast<uint4*>(s.x + row * ROW + 32 * b);
        d4[0] = make_uint4(o[0], o[1], o[2], o[3]);
        d4[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

// One workgroup tile: y[yrow[r]][n0 + c] for tile rows r with xrow[r] >= 0,
// over all of k.  Weights: rows n0.. of w (n rows, rb bytes per row).
template <int FMT, int WMW, int WNW, int MI, int NI, bool kAllLive = false>
__device__ __forceinline__ void mma_tile(Smem<Tile<WMW, WNW, MI, NI>::BM, 128>& s,
                                         const uint8_t* __restrict__ w, int64_t n, int64_t k,
                                         int64_t rb, int64_t n0, const uint8_t* __restrict__ xq,
                                         int rows, float* __restrict__ y, int64_t ldy) {
    constexpr int BM = Tile<WMW, WNW, MI, NI>::BM;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv / WNW, wn = wv % WNW;     // wave tile: tokens wm*MI*32.., rows wn*NI*32..
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t xrb = k / 32 * 34;
    // token sub-tiles of this wave that hold at least one real row
    int mi_live = 0;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
        if ((wm * MI + mi) * 32 < rows) mi_live = mi + 1;

    v16f acc[MI][NI];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = kBias;

    const int ksteps = static_cast<int>(k / (32 * KB));
    WRaw<FMT> wr;
    XRaw xr;
    load_weights<FMT>(wr, w, n, rb, n0, 0);
    __syncthreads();  // the row maps written by the caller are visible
    load_acts<BM>(xr, s, xq, xrb, 0);
    for (int ks = 0; ks < ksteps; ++ks) {
        __syncthreads();  // the previous step's reads of the tiles are done
        store_weights<FMT>(s, wr, ks);
        store_acts<FMT, BM>(s, xr);
        __syncthreads();
        // next step's loads (the last step reloads itself: no branch)
        const int kn = ks + 1 < ksteps ? ks + 1 : ks;
        load_weights<FMT>(wr, w, n, rb, n0, kn);
        load_acts<BM>(xr, s, xq, xrb, kn);
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            v4i A[NI], Bv[MI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                A[ni] = *reinterpret_cast<const v4i*>(s.w + ((wn * NI + ni) * 32 + l32) * ROW + 32 * b + 16 * h);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                Bv[mi] = *reinterpret_cast<const v4i*>(s.x + ((wm * MI + mi) * 32 + l32) * ROW + 32 * b + 16 * h);
            float dx[MI], ndx[MI];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                dx[mi] = s.dx[b][(wm * MI + mi) * 32 + l32];
                ndx[mi] = -kBiasF * dx[mi];
            }
            if constexpr (FMT == T_Q6_K) {
                // 16-value scale groups: one v_mfma_i32_32x32x16_i8 per
                // half block, each rescaled with its own d*sc
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    long A2[NI], B2[MI];
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni)
                        A2[ni] = *reinterpret_cast<const long*>(
                            s.w + ((wn * NI + ni) * 32 + l32) * ROW + 32 * b + 16 * hh + 8 * h);
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        B2[mi] = *reinterpret_cast<const long*>(
                            s.x + ((wm * MI + mi) * 32 + l32) * ROW + 32 * b + 16 * hh + 8 * h);
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        float dwv[16];
                        const float* dsrc = hh ? &s.dw2[b][0] : &s.dw[b][0];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 d4 = *reinterpret_cast<const float4*>(dsrc + (wn * NI + ni) * 32 + 8 * q + 4 * h);
                            dwv[4 * q] = d4.x; dwv[4 * q + 1] = d4.y; dwv[4 * q + 2] = d4.z; dwv[4 * q + 3] = d4.w;
                        }
#pragma unroll
                        for (int mi = 0; mi < MI; ++mi) {
                            if (!kAllLive && mi >= mi_live) break;
                            const v16i D = __builtin_amdgcn_mfma_i32_32x32x16_i8(A2[ni], B2[mi], bias, 0, 0, 0);
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float tq = fmaf(__int_as_float(D[r]), dx[mi], ndx[mi]);
                                acc[mi][ni][r] = fmaf(tq, dwv[r], acc[mi][ni][r]);
                            }
                        }
                    }
                }
            } else if constexpr (kAllLive) {
                // every (ni, mi) tile is live: the MFMA of the next tile is
                // issued before the rescale of the current one, so the
                // rescale does not wait for the MFMA it follows
                constexpr int NT = NI * MI;
                float dwv[NI][16];
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 d4 = *reinterpret_cast<const float4*>(&s.dw[b][(wn * NI + ni) * 32 + 8 * q + 4 * h]);
                        dwv[ni][4 * q] = d4.x; dwv[ni][4 * q + 1] = d4.y;
                        dwv[ni][4 * q + 2] = d4.z; dwv[ni][4 * q + 3] = d4.w;
                    }
                v16i D[2];
                D[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[0], Bv[0], bias, 0, 0, 0);
#pragma unroll
                for (int p = 0; p < NT; ++p) {
                    const int ni = p / MI, mi = p % MI;
                    if (p + 1 < NT)
                        D[(p + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[(p + 1) / MI], Bv[(p + 1) % MI],
                                                                             bias, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float tq = fmaf(__int_as_float(D[p & 1][r]), dx[mi], ndx[mi]);
                        acc[mi][ni][r] = fmaf(tq, dwv[ni][r], acc[mi][ni][r]);
                    }
                }
            } else {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    float dwv[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 d4 = *reinterpret_cast<const float4*>(&s.dw[b][(wn * NI + ni) * 32 + 8 * q + 4 * h]);
                        dwv[4 * q] = d4.x; dwv[4 * q + 1] = d4.y; dwv[4 * q + 2] = d4.z; dwv[4 * q + 3] = d4.w;
                    }
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) {
                        if (mi >= mi_live) break;
                        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[ni], Bv[mi], bias, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float tq = fmaf(__int_as_float(D[r]), dx[mi], ndx[mi]);
                            acc[mi][ni][r] = fmaf(tq, dwv[r], acc[mi][ni][r]);
                        }
                    }
                }
            }
        }
        if constexpr (kHasOffset<FMT>) {
            // additive term: acc[n][m] += sum_b cw[b][n] * sx[b][m], two blocks
            // per fp32 MFMA (A: rows n, k = block; B: columns m)
#pragma unroll
            for (int b2 = 0; b2 < KB; b2 += 2) {
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const float a = s.cw[b2 + h][(wn * NI + ni) * 32 + l32];
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi) {
                        if (!kAllLive && mi >= mi_live) break;
                        const float bx = s.sx[b2 + h][(wm * MI + mi) * 32 + l32];
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bx, acc[mi][ni], 0, 0, 0);
                    }
                }
            }
        }
    }

    // epilogue: lane holds tile row (wm*MI + mi)*32 + l32 and weight rows
    // n0 + (wn*NI + ni)*32 + 8q + 4h + e (register 4q + e)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int r = (wm * MI + mi) * 32 + l32;
        if (r >= rows || s.xrow[r] < 0) continue;
        float* yr = y + static_cast<int64_t>(s.yrow[r]) * ldy;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t gn = n0 + (wn * NI + ni) * 32 + 8 * q + 4 * h;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (gn + e < n) yr[gn + e] = acc[mi][ni][4 * q + e];
            }
        }
    }
}

// Dense GEMM with one LDS buffer (the formats whose scale tables do not
// leave room for two buffers at two workgroups per CU): 128 x 128 tiles,
// 2 x 2 waves of 64 x 64.
// Workgroup g of G -> tile index (token tile = tile % tiles_m, weight tile =
// tile / tiles_m).  Workgroups are dealt round-robin over the 8 XCDs; each
// XCD takes a contiguous range of weight tiles with all their token tiles,
// walked in bands of two token tiles across the XCD's weight tiles, so the
// workgroups resident on an XCD at once share a few token tiles and all of
// its weight tiles in that XCD's L2 (the L2 fetches at 2048 tokens drop from
// about 3.0x to 1.9x the operand bytes).  Grids that do not split evenly keep
// the plain contiguous order.
__device__ __forceinline__ int tile_of(int g, int G, int tiles_m) {
    const int per_xcd = G / 8;
    if (g >= 8 * per_xcd) return g;
    const int l = g / 8;
    if (per_xcd % tiles_m != 0 || tiles_m % 2 != 0) return (g % 8) * per_xcd + l;
    const int nl = per_xcd / tiles_m;          // weight tiles of this XCD
    const int band = l / (2 * nl), rem = l % (2 * nl);
    return ((g % 8) * nl + rem / 2) * tiles_m + 2 * band + (rem & 1);
}

template <int FMT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t k, int64_t rb,
        const uint8_t* __restrict__ xq, int64_t m, float* __restrict__ y, int64_t ldy,
        int tiles_m, int tiles_total) {
    using T = Tile<2, 2, 2, 2>;
    __shared__ __align__(16) Smem<T::BM, 128> s;
    const int G = gridDim.x, g = blockIdx.x;
    const int tile = tile_of(g, G, tiles_m);
    if (tile >= tiles_total) return;
    const int64_t m0 = static_cast<int64_t>(tile % tiles_m) * T::BM;
    const int64_t n0 = static_cast<int64_t>(tile / tiles_m) * T::BN;
    if (threadIdx.x < T::BM) {
        const int64_t gm = m0 + threadIdx.x;
        s.xrow[threadIdx.x] = gm < m ? static_cast<int>(gm) : -1;
        s.yrow[threadIdx.x] = static_cast<int>(gm);
    }
    const int rows = static_cast<int>(m - m0 < T::BM ? m - m0 : T::BM);
    // every token sub-tile is computed (rows past m hold row 0's data and are
    // not stored): straight-line MFMA code keeps the accumulators in place
    mma_tile<FMT, 2, 2, 2, 2, true>(s, w, n, k, rb, n0, xq, rows, y, ldy);
}

// ---- dense GEMM, double-buffered LDS -----------------------------------------
// The same 128 x 128 workgroup tile, 2 x 2 waves of 64 x 64 and k step of
// four blocks, with two LDS buffers: while step ks is computed from one, the
// decoded weights and split activations of step ks+1 are stored into the
// other (their global loads were issued a step earlier), so each step needs
// one barrier instead of two.  Two buffers of padded rows (the 16-byte pad
// keeps the MFMA operand reads of eight rows at one offset on distinct
// banks) and the two scale tables take 80 KB, so two workgroups share a CU:
// this path serves Q4_0 and Q8_0 (Q4_1 / K-quants need more tables).
constexpr int RW2 = KB * 32 + 16;

template <int FMT>
struct Smem2 {
    int8_t w[128 * RW2];
    int8_t x[128 * RW2];
    float dw[KB][128];
    float dx[KB][128];
};

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * RW2 + (chunk << 4); }  // byte offset of 16-byte chunk

template <int FMT>
__device__ __forceinline__ void store_w2(Smem2<FMT>& s, const WRaw<FMT>& r) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
    constexpr int BS = WRaw<FMT>::BS;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
        const int b = 2 * half + bl;
        uint32_t o[8];
        if constexpr (FMT == T_Q8_0) {
            s.dw[b][row] = h2f(half_at(r.v, bl * BS));
            extract<8>(r.v, bl * BS + 2, o);
        } else {
            // Q4_0: each nibble q goes to the top of its byte with the top
            // bit flipped, (q << 4 or q) & 0xF0 ^ 0x80 = the signed byte
            // 16 (q - 8) (a shift and one three-input bitwise op, or just the
            // latter), so the MFMA sums 16 x the integer dot; the block scale
            // is held divided by 16 (exact), and t = D*dx - bias*dx rounds
            // to 16 x the plain t, so the products are bitwise unchanged.
            s.dw[b][row] = h2f(half_at(r.v, bl * BS)) * 0.0625f;
            uint32_t q[4];
            extract<4>(r.v, bl * BS + 2, q);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[i] = ((q[i] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;
                o[4 + i] = (q[i] & 0xF0F0F0F0u) ^ 0x80808080u;
            }
        }
        *reinterpret_cast<uint4*>(s.w + lds_off(row, 2 * b)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(s.w + lds_off(row, 2 * b + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

template <int FMT>
__device__ __forceinline__ void store_x2(Smem2<FMT>& s, const XRaw& r) {
    const int t = threadIdx.x, row = t >> 1, half = t & 1;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
        const int b = 2 * half + bl;
        uint32_t o[8];
        extract<8>(r.v, bl * 34 + 2, o);
        s.dx[b][row] = h2f(half_at(r.v, bl * 34));
        *reinterpret_cast<uint4*>(s.x + lds_off(row, 2 * b)) = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(s.x + lds_off(row, 2 * b + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

__device__ __forceinline__ void load_x2(XRaw& r, const uint8_t* __restrict__ xq, int64_t xrb,
                                        int64_t gm, int kstep) {
    const int half = threadIdx.x & 1;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        xq + gm * xrb + (static_cast<int64_t>(kstep) * KB + 2 * half) * 34);
#pragma unroll
    for (int i = 0; i < 17; ++i) r.v[i] = p[i];
}

// one 32-value block of the step: 2 x 2 MFMA tiles of this wave, rescaled
template <int FMT>
__device__ __forceinline__ void mma_block2(const Smem2<FMT>& s, int b, int wm, int wn, int l32, int h,
                                           const v16i& bias, v16f (&acc)[2][2]) {
    v4i A[2], Bv[2];
    float dx[2], ndx[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int r = (wn * 2 + ni) * 32 + l32;
        A[ni] = *reinterpret_cast<const v4i*>(s.w + lds_off(r, 2 * b + h));
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int r = (wm * 2 + mi) * 32 + l32;
        Bv[mi] = *reinterpret_cast<const v4i*>(s.x + lds_off(r, 2 * b + h));
        dx[mi] = s.dx[b][r];
        ndx[mi] = -kBiasF * dx[mi];
    }
    float dwv[2][16];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 d4 = *reinterpret_cast<const float4*>(&s.dw[b][(wn * 2 + ni) * 32 + 8 * q + 4 * h]);
            dwv[ni][4 * q] = d4.x; dwv[ni][4 * q + 1] = d4.y;
            dwv[ni][4 * q + 2] = d4.z; dwv[ni][4 * q + 3] = d4.w;
        }
    v16i D[2];
    D[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[0], Bv[0], bias, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int ni = p / 2, mi = p % 2;
        if (p + 1 < 4)
            D[(p + 1) & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[(p + 1) / 2], Bv[(p + 1) % 2], bias, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float tq = fmaf(__int_as_float(D[p & 1][r]), dx[mi], ndx[mi]);
            acc[mi][ni][r] = fmaf(tq, dwv[ni][r], acc[mi][ni][r]);
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads, 2) void gemm2_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t k, int64_t rb,
        const uint8_t* __restrict__ xq, int64_t m, float* __restrict__ y, int64_t ldy,
        int tiles_m, int tiles_total) {
    __shared__ __align__(16) Smem2<FMT> sm[2];
    const int G = gridDim.x, g = blockIdx.x;
    const int tile = tile_of(g, G, tiles_m);
    if (tile >= tiles_total) return;
    const int64_t m0 = static_cast<int64_t>(tile % tiles_m) * 128;
    const int64_t n0 = static_cast<int64_t>(tile / tiles_m) * 128;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t xrb = k / 32 * 34;
    const int64_t gm = m0 + (threadIdx.x >> 1) < m ? m0 + (threadIdx.x >> 1) : m - 1;
    const int ksteps = static_cast<int>(k / (32 * KB));

    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = kBias;
    v16f acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    WRaw<FMT> wr;
    XRaw xr;
    load_weights<FMT>(wr, w, n, rb, n0, 0);
    load_x2(xr, xq, xrb, gm, 0);
    store_w2<FMT>(sm[0], wr);
    store_x2<FMT>(sm[0], xr);
    const int k1 = ksteps > 1 ? 1 : 0;
    load_weights<FMT>(wr, w, n, rb, n0, k1);
    load_x2(xr, xq, xrb, gm, k1);
    __syncthreads();
    for (int ks = 0; ks < ksteps; ++ks) {
        const Smem2<FMT>& cur = sm[ks & 1];
        if (ks + 1 < ksteps) {
            store_w2<FMT>(sm[(ks + 1) & 1], wr);
            store_x2<FMT>(sm[(ks + 1) & 1], xr);
        }
        const int kn = ks + 2 < ksteps ? ks + 2 : ksteps - 1;
        load_weights<FMT>(wr, w, n, rb, n0, kn);
        load_x2(xr, xq, xrb, gm, kn);
#pragma unroll
        for (int b = 0; b < KB; ++b) mma_block2<FMT>(cur, b, wm, wn, l32, h, bias, acc);
        __syncthreads();
    }
    // epilogue: lane holds token row (wm*2 + mi)*32 + l32 and weight rows
    // n0 + (wn*2 + ni)*32 + 8q + 4h + e (register 4q + e)
    const bool vec = (ldy & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int64_t gr = m0 + (wm * 2 + mi) * 32 + l32;
        if (gr >= m) continue;
        float* yr = y + gr * ldy;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t gn = n0 + (wn * 2 + ni) * 32 + 8 * q + 4 * h;
                if (vec && gn + 3 < n) {
                    *reinterpret_cast<float4*>(yr + gn) =
                        make_float4(acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                                    acc[mi][ni][4 * q + 3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (gn + e < n) yr[gn + e] = acc[mi][ni][4 * q + e];
                }
            }
        }
    }
}

// Grouped expert GEMM: workgroup (n tile, expert); 64 x 128 tiles, 1 x 4
// waves of 64 x 32, looping over the expert's rows 64 at a time.  The
// activation rows are gathered through the grouped pair list.
template <int FMT>
__global__ __launch_bounds__(kThreads, 2) void moe_gemm_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t k, int64_t rb,
        const uint8_t* __restrict__ xq, int x_per_pair, const int32_t* __restrict__ offsets,
        const int32_t* __restrict__ pairs, int np, int top_k, float* __restrict__ y, int64_t ldy) {
    using T = Tile<1, 4, 2, 1>;
    __shared__ __align__(16) Smem<T::BM, 128> s;
    const int e = blockIdx.y;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * T::BN;
    // defensive clamps: offsets and pairs come from device memory
    int off = offsets[e], end = offsets[e + 1];
    off = off < 0 ? 0 : (off > np ? np : off);
    end = end < off ? off : (end > np ? np : end);
    const uint8_t* we = w + static_cast<int64_t>(e) * n * rb;
    for (int base = off; base < end; base += T::BM) {
        const int rows = end - base < T::BM ? end - base : T::BM;
        __syncthreads();  // the previous tile's epilogue has read xrow / yrow
        if (threadIdx.x < T::BM) {
            int xr = -1, yr = 0;
            if (static_cast<int>(threadIdx.x) < rows) {
                const int p = pairs[base + threadIdx.x];
                if (p >= 0 && p < np) {
                    xr = x_per_pair ? p : p / top_k;
                    yr = p;
                }
            }
            s.xrow[threadIdx.x] = xr;
            s.yrow[threadIdx.x] = yr;
        }
        mma_tile<FMT, 1, 4, 2, 1>(s, we, n, k, rb, n0, xq, rows, y, ldy);
    }
}

// ---- streaming grouped GEMM for Q4_K expert weights ---------------------------
// The routed FFN is bound by streaming each expert's weights once, so here
// the weights sit on the MFMA's B side (columns = weight rows) and every lane
// loads its own weight row straight from HBM into registers.  With
// v_mfma_i32_16x16x32_i8 a lane (row j = lane%16, quarter g = lane/16) holds
// 8 of the 32 values of a block, so for super-block s it loads the 16-byte
// header and bytes [8g, 8g+8) of each of the four 32-byte nibble chunks:
// exactly the B operands of the eight sub-block MFMAs (low nibbles give
// sub-block 2c, high nibbles 2c+1).  The next super-block's loads are issued
// before the current one is computed; no barrier is involved.  The expert's
// gathered Q8_0 activation rows (up to 64 per pass, in 16-row MFMA tiles so
// padding stays small) are the A side, split per super-block into a
// double-buffered LDS tile by all 256 threads (one barrier per super-block).
// Per sub-block: D = mfma(act, w) from the float bias, t = fma(D, d*sc,
// -12582912*d*sc) = round(I*d*sc) (exact subtrahend: d*sc has 17 significant
// bits), acc = fma(t, dx, acc); the -dmin*m * dx*sum(qx) term goes through
// v_mfma_f32_16x16x4_f32, four sub-blocks at a time.
constexpr int kSbTok = 64;             // tokens per pass
// LDS row stride of the activation tile: 264 bytes (66 dwords) puts the
// 8-byte MFMA operand reads of 16 consecutive token rows on distinct banks
// (the 272-byte stride paired rows j and j + 8 on one bank)
constexpr int kSbRow = 8 * 32 + 8;
constexpr int kSbRows = 64;            // weight rows per workgroup (16 per wave)

typedef float v4f __attribute__((ext_vector_type(4)));

struct ActTile {
    int8_t x[kSbTok * kSbRow];
    float dx[8][kSbTok];
    float sx[8][kSbTok + 16];   // rows padded: the four sub-block rows one
                                // read instruction touches fall on distinct banks
};

struct StreamSmem {
    ActTile t[2];
    int xrow[kSbTok];
    int yrow[kSbTok];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct ARegs {            // two Q8_0 activation blocks (68 bytes)
    u32x4 v[4];
    uint32_t t;
};

struct WRegs {            // one lane's share of one Q4_K super-block
    u32x4 hdr;            // d, dmin, 12 scale bytes
    u32x2 q[4];           // 8 bytes of each 32-byte nibble chunk
};

// Load activation blocks 2q, 2q+1 of super-block sb for tile row r (thread
// t: r = t/4, q = t%4).  Unconditional: a row that holds no pair reads the
// pass's first token row instead (loaded anyway, and not one row shared by
// every workgroup), and its outputs are never stored.  (A load under a
// branch is merged with the other branch's value by a register copy, which
// waits for the load at once.)
__device__ __forceinline__ void issue_acts(const StreamSmem& s, const uint8_t* __restrict__ xq,
                                           int64_t xrb, int sb, ARegs& a) {
    const int t = threadIdx.x, r = t >> 2, q = t & 3;
    const int gm = s.xrow[r] >= 0 ? s.xrow[r] : s.xrow[0];
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        xq + static_cast<int64_t>(gm < 0 ? 0 : gm) * xrb + (static_cast<int64_t>(sb) * 8 + 2 * q) * 34);
#pragma unroll
    for (int i = 0; i < 4; ++i) a.v[i] = u32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
    a.t = p[16];
}

// Load super-block sb of this lane's weight row (a lane past the last row
// reads row 0 of the expert and stores nothing).
__device__ __forceinline__ void issue_w(const uint8_t* __restrict__ row, int sb, int g, WRegs& r) {
    const uint8_t* p = row + static_cast<int64_t>(sb) * 144;
    r.hdr = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const u32x2*>(p + 16 + 32 * c + 8 * g);
}

// Split two loaded blocks into the tile: int8 values, dx and dx*sum(q).
__device__ __forceinline__ void store_acts(ActTile& at, const ARegs& a) {
    const int t = threadIdx.x, r = t >> 2, q = t & 3;
    uint32_t v[17];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[4 * i] = a.v[i].x;
        v[4 * i + 1] = a.v[i].y;
        v[4 * i + 2] = a.v[i].z;
        v[4 * i + 3] = a.v[i].w;
    }
    v[16] = a.t;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
        const int b = 2 * q + bl;
        uint32_t o[8];
        extract<8>(v, bl * 34 + 2, o);
        const float dx = h2f(half_at(v, bl * 34));
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) sum = sdot4(o[i], 0x01010101u, sum);
        at.dx[b][r] = dx;
        at.sx[b][r] = dx * static_cast<float>(sum);
        uint2* d2 = reinterpret_cast<uint2*>(at.x + r * kSbRow + 32 * b);   // 8-byte aligned rows
        d2[0] = make_uint2(o[0], o[1]);
        d2[1] = make_uint2(o[2], o[3]);
        d2[2] = make_uint2(o[4], o[5]);
        d2[3] = make_uint2(o[6], o[7]);
    }
}

constexpr int kStreamThreads = 256;    // 4 waves x 16 weight rows; 4 stagers per token row
static_assert(kStreamThreads == 4 * kSbTok, "every thread stages two activation blocks");

struct StreamLane {
    const uint8_t* wrow;   // this lane's weight row (expert already applied)
    bool row_ok;
    int g, j16;            // lane / 16 and lane % 16
    int64_t gn;            // this lane's weight row index
};

// One super-block: MT 16-token tiles against this wave's 16 weight rows.
template <int MT>
__device__ __forceinline__ void stream_sb(const ActTile& at, const WRegs& cur, const StreamLane& L,
                                          const v4i& bias, v4f (&acc)[MT]) {
    const float d = h2f(cur.hdr.x & 0xFFFFu), dmin = h2f(cur.hdr.x >> 16);
    // the eight 6-bit scales (bytes of sc03, sc47) and this lane's mins of
    // sub-blocks g and 4 + g, unpacked a dword at a time
    const uint32_t sc03 = cur.hdr.y & 0x3F3F3F3Fu;
    const uint32_t sc47 = (cur.hdr.w & 0x0F0F0F0Fu) | ((cur.hdr.y >> 2) & 0x30303030u);
    const uint32_t mn03 = cur.hdr.z & 0x3F3F3F3Fu;
    const uint32_t mn47 = ((cur.hdr.w >> 4) & 0x0F0F0F0Fu) | ((cur.hdr.z >> 2) & 0x30303030u);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x2 qv = cur.q[c];
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const int j = 2 * c + e2;         // sub-block = local block index
            const long Bw = static_cast<long>(
                (static_cast<uint64_t>(((e2 ? qv.y >> 4 : qv.y) & 0x0F0F0F0Fu)) << 32) |
                ((e2 ? qv.x >> 4 : qv.x) & 0x0F0F0F0Fu));
            const uint32_t scw = j < 4 ? sc03 : sc47;
            const float dwj = d * static_cast<float>((scw >> (8 * (j & 3))) & 0xFFu);
            const float ndwj = -kBiasF * dwj;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const long A = *reinterpret_cast<const long*>(at.x + (16 * mt + L.j16) * kSbRow + 32 * j + 8 * L.g);
                const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, Bw, bias, 0, 0, 0);
                const float4 dx = *reinterpret_cast<const float4*>(&at.dx[j][16 * mt + 4 * L.g]);
                acc[mt][0] = fmaf(fmaf(__int_as_float(D[0]), dwj, ndwj), dx.x, acc[mt][0]);
                acc[mt][1] = fmaf(fmaf(__int_as_float(D[1]), dwj, ndwj), dx.y, acc[mt][1]);
                acc[mt][2] = fmaf(fmaf(__int_as_float(D[2]), dwj, ndwj), dx.z, acc[mt][2]);
                acc[mt][3] = fmaf(fmaf(__int_as_float(D[3]), dwj, ndwj), dx.w, acc[mt][3]);
            }
        }
    }
    // -dmin*m * dx*sum(qx): A = dx*sum(q) [tokens][4 sub-blocks],
    // B = -dmin*m [4 sub-blocks][weight rows]
#pragma unroll
    for (int j4 = 0; j4 < 8; j4 += 4) {
        const uint32_t mw = j4 == 0 ? mn03 : mn47;      // sub-block j4 + g of this lane's row
        const float bm = -(dmin * static_cast<float>(__builtin_amdgcn_ubfe(mw, 8 * L.g, 8)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float ax = at.sx[j4 + L.g][16 * mt + L.j16];
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ax, bm, acc[mt], 0, 0, 0);
        }
    }
}

// One pass over up to 16*MT gathered token rows (row maps already in LDS).
// Weight super-block sb is loaded into register set sb % 3 two steps before it
// is used; the sets rotate by unrolling, so no set is copied.  The loads for
// later super-blocks are written before the compute of the current one; past
// the last super-block they repeat the current one and the store fills the
// idle tile, so no load or store sits under a branch.
template <int MT>
__device__ __forceinline__ void stream_pass(StreamSmem& s, const StreamLane& L, int nsb,
                                            const uint8_t* __restrict__ xq, int64_t xrb, int rows,
                                            float* __restrict__ y, int64_t ldy) {
    v4i bias;
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = kBias;
    ARegs av;
    WRegs w0, w1, w2;
    // only the token rows of the MT live tiles are staged: 16 rows per wave
    const bool stager = MT == 4 || __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)) < MT;
    if (stager) issue_acts(s, xq, xrb, 0, av);
    issue_w(L.wrow, 0, L.g, w0);
    issue_w(L.wrow, nsb > 1 ? 1 : 0, L.g, w1);
    if (stager) store_acts(s.t[0], av);
    __syncthreads();

    v4f acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][r] = 0.0f;

#define CQ_STREAM_STEP(SB, CUR, FILL)                                             \
    {                                                                                   \
        const int sb_ = (SB);                                                           \
        if (stager) issue_acts(s, xq, xrb, sb_ + 1 < nsb ? sb_ + 1 : sb_, av);          \
        issue_w(L.wrow, sb_ + 2 < nsb ? sb_ + 2 : sb_, L.g, FILL);                      \
        stream_sb<MT>(s.t[sb_ & 1], CUR, L, bias, acc);                                 \
        if (stager) store_acts(s.t[(sb_ + 1) & 1], av);                                 \
        __syncthreads();                                                                \
    }
    for (int sb = 0; sb < nsb; sb += 3) {
        CQ_STREAM_STEP(sb, w0, w2)
        if (sb + 1 >= nsb) break;
        CQ_STREAM_STEP(sb + 1, w1, w0)
        if (sb + 2 >= nsb) break;
        CQ_STREAM_STEP(sb + 2, w2, w1)
    }
#undef CQ_STREAM_STEP
    // epilogue: lane = weight row gn, register r = token row 4g + r of tile mt
    if (L.row_ok) {
        const int lim = rows - 4 * L.g;           // token row 4g + c is live when c < lim
        const int* xr = s.xrow + 4 * L.g;
        const int* yr = s.yrow + 4 * L.g;
        float* yc = y + L.gn;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * mt + r;
                if (c < lim && xr[c] >= 0) yc[static_cast<int64_t>(yr[c]) * ldy] = acc[mt][r];
            }
        }
    }
}

__global__ __launch_bounds__(kStreamThreads, 3) void moe_stream_q4k_kernel(
        const uint8_t* __restrict__ w, int64_t n, int64_t k, int64_t rb,
        const uint8_t* __restrict__ xq, int x_per_pair, const int32_t* __restrict__ offsets,
        const int32_t* __restrict__ pairs, int np, int top_k, float* __restrict__ y, int64_t ldy) {
    __shared__ __align__(16) StreamSmem s;
    const int e = blockIdx.y;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    StreamLane L;
    L.j16 = lane & 15;
    L.g = lane >> 4;
    L.gn = static_cast<int64_t>(blockIdx.x) * kSbRows + 16 * wv + L.j16;
    L.row_ok = L.gn < n;
    L.wrow = w + (static_cast<int64_t>(e) * n + (L.row_ok ? L.gn : 0)) * rb;
    const int nsb = static_cast<int>(k / 256);
    const int64_t xrb = k / 32 * 34;
    int off = offsets[e], end = offsets[e + 1];
    off = off < 0 ? 0 : (off > np ? np : off);
    end = end < off ? off : (end > np ? np : end);

    for (int base = off; base < end; base += kSbTok) {
        const int rows = end - base < kSbTok ? end - base : kSbTok;
        __syncthreads();  // the previous pass is done with the tile and row maps
        if (threadIdx.x < kSbTok) {
            int xr = -1, yr = 0;
            if (static_cast<int>(threadIdx.x) < rows) {
                const int p = pairs[base + threadIdx.x];
                if (p >= 0 && p < np) {
                    xr = x_per_pair ? p : p / top_k;
                    yr = p;
                }
            }
            s.xrow[threadIdx.x] = xr;
            s.yrow[threadIdx.x] = yr;
        }
        __syncthreads();
        switch ((rows + 15) >> 4) {     // 16-token tiles holding real rows
            case 1: stream_pass<1>(s, L, nsb, xq, xrb, rows, y, ldy); break;
            case 2: stream_pass<2>(s, L, nsb, xq, xrb, rows, y, ldy); break;
            case 3: stream_pass<3>(s, L, nsb, xq, xrb, rows, y, ldy); break;
            default: stream_pass<4>(s, L, nsb, xq, xrb, rows, y, ldy); break;
        }
    }
}


// ---- routed experts, whole-k activation tile ---------------------------------
// For k of NSB super-blocks (the lfm2moe projections: 2048 and 1536), a
// workgroup of NW waves owns NW*16*rpl weight rows of one expert and splits
// the expert's gathered Q8_0 activation rows (up to 16*MTMAX per pass) for
// the whole of k into LDS at once, behind one barrier; each wave then runs
// its rpl groups of 16 rows over every super-block with no further barrier.
// A wave's weights pass through a ring of RING register sets of one
// super-block each: set s % RING is refilled, as soon as it has been used,
// with super-block s + RING of the group, or of the wave's next group.  The
// arithmetic per super-block is that of stream_sb, in the same order, so
// the results are those of moe_stream_q4k_kernel bit for bit.  With PAIR
// the row groups run over two matrices that read the same activation rows
// (w, then w2: the routed FFN's gate and up), so one split serves both.
// (lfm2moe shapes, 256 tokens, top 4 of 32, C harness: gate/up 29.4
// against 34.0 us, down 28.7 against 37.4 us; gate + up in one launch 48
// against 59 us for two.)
constexpr int kSxRow = 80;   // sx row stride (floats): four rows of one read on distinct banks

template <int NSB, int T>
struct WholeSmem {           // NSB super-blocks of T token rows
    int8_t x[NSB][T * kSbRow];
    float dx[NSB * 8][T];
    float sx[NSB * 8][kSxRow];
    int xrow[T];
    int yrow[T];
};

// Issue the loads of activation block pair item (token row r = item % T,
// pair q = item / T: blocks 2q and 2q+1); a tile row past the pass's rows
// reads the pass's first token row.  Consecutive threads take consecutive
// token rows, so their dx and sum stores below fall on consecutive banks.
template <int NSB, int T>
__device__ __forceinline__ void issue_pair(const WholeSmem<NSB, T>& s, const uint8_t* __restrict__ xq,
                                           int64_t xrb, int item, ARegs& a) {
    const int r = item % T, q = item / T;
    const int gm = s.xrow[r] >= 0 ? s.xrow[r] : s.xrow[0];
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        xq + static_cast<int64_t>(gm < 0 ? 0 : gm) * xrb + static_cast<int64_t>(2 * q) * 34);
#pragma unroll
    for (int i = 0; i < 4; ++i) a.v[i] = u32x4{p[4 * i], p[4 * i + 1], p[4 * i + 2], p[4 * i + 3]};
    a.t = p[16];
}

// Split a loaded pair into the tile: int8 values, dx and dx*sum(q).
template <int NSB, int T>
__device__ __forceinline__ void store_pair(WholeSmem<NSB, T>& s, int item, const ARegs& a) {
    const int r = item % T, q = item / T;
    const int sb = q >> 2;
    uint32_t v[17];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[4 * i] = a.v[i].x;
        v[4 * i + 1] = a.v[i].y;
        v[4 * i + 2] = a.v[i].z;
        v[4 * i + 3] = a.v[i].w;
    }
    v[16] = a.t;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
        const int b = 2 * (q & 3) + bl;   // sub-block within the super-block
        uint32_t o[8];
        extract<8>(v, bl * 34 + 2, o);
        const float dx = h2f(half_at(v, bl * 34));
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) sum = sdot4(o[i], 0x01010101u, sum);
        s.dx[8 * sb + b][r] = dx;
        s.sx[8 * sb + b][r] = dx * static_cast<float>(sum);
        uint2* d2 = reinterpret_cast<uint2*>(s.x[sb] + r * kSbRow + 32 * b);
        d2[0] = make_uint2(o[0], o[1]);
        d2[1] = make_uint2(o[2], o[3]);
        d2[2] = make_uint2(o[4], o[5]);
        d2[3] = make_uint2(o[6], o[7]);
    }
}

// This lane's row of group grp (a row past n reads row 0 of the expert and
// is not stored).
__device__ __forceinline__ StreamLane group_lane(const uint8_t* __restrict__ w, int64_t n, int64_t rb,
                                                 int e, int64_t grp, int lane) {
    StreamLane L;
    L.j16 = lane & 15;
    L.g = lane >> 4;
    L.gn = grp * 16 + L.j16;
    L.row_ok = L.gn < n;
    L.wrow = w + (static_cast<int64_t>(e) * n + (L.row_ok ? L.gn : 0)) * rb;
    return L;
}

// Store group outputs: lane = weight row, register r = token row 4g + r of
// tile mt.
template <int MT, int NSB, int T>
__device__ __forceinline__ void store_group(const WholeSmem<NSB, T>& s, const StreamLane& L, int rows,
                                            const v4f (&acc)[MT], float* __restrict__ y, int64_t ldy) {
    if (!L.row_ok) return;
    const int lim = rows - 4 * L.g;
    const int* xr = s.xrow + 4 * L.g;
    const int* yr = s.yrow + 4 * L.g;
    float* yc = y + L.gn;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * mt + r;
            if (c < lim && xr[c] >= 0) yc[static_cast<int64_t>(yr[c]) * ldy] = acc[mt][r];
        }
}

// stream_sb on a WholeSmem super-block, from this lane's LDS positions:
// ax = its A-operand bytes of token row j16 (x + j16*kSbRow + 8g), pdx =
// dx row 0 at token 4g, psx = sx row g at token j16.  Each MFMA is issued
// before the rescale of the previous one, so the rescale never waits for
// the MFMA it follows.
template <int MT, int T>
__device__ __forceinline__ void whole_sb(const int8_t* ax, const float* pdx, const float* psx,
                                         const WRegs& cur, int g, const v4i& bias, v4f (&acc)[MT]) {
    const float d = h2f(cur.hdr.x & 0xFFFFu), dmin = h2f(cur.hdr.x >> 16);
    const uint32_t sc03 = cur.hdr.y & 0x3F3F3F3Fu;
    const uint32_t sc47 = (cur.hdr.w & 0x0F0F0F0Fu) | ((cur.hdr.y >> 2) & 0x30303030u);
    const uint32_t mn03 = cur.hdr.z & 0x3F3F3F3Fu;
    const uint32_t mn47 = ((cur.hdr.w >> 4) & 0x0F0F0F0Fu) | ((cur.hdr.z >> 2) & 0x30303030u);
    // B operand of sub-block j: low (j even) or high nibbles of chunk j/2
    auto bw = [&](int j) {
        const u32x2 qv = cur.q[j >> 1];
        const uint32_t sh = (j & 1) ? 4u : 0u;
        return static_cast<long>((static_cast<uint64_t>((qv.y >> sh) & 0x0F0F0F0Fu) << 32) |
                                  ((qv.x >> sh) & 0x0F0F0F0Fu));
    };
    auto amat = [&](int q) {
        return *reinterpret_cast<const long*>(ax + 16 * (q % MT) * kSbRow + 32 * (q / MT));
    };
    // MFMA q = j*MT + mt; the next one is issued before this one's rescale
    constexpr int NQ = 8 * MT;
    v4i D[2];
    D[0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(amat(0), bw(0), bias, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int j = q / MT, mt = q % MT;
        if (q + 1 < NQ)
            D[(q + 1) & 1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(amat(q + 1), bw((q + 1) / MT), bias, 0, 0, 0);
        const uint32_t scw = j < 4 ? sc03 : sc47;
        const float dwj = d * static_cast<float>((scw >> (8 * (j & 3))) & 0xFFu);
        const float ndwj = -kBiasF * dwj;
        const float4 dx = *reinterpret_cast<const float4*>(pdx + j * T + 16 * mt);
        const v4i& Dq = D[q & 1];
        acc[mt][0] = fmaf(fmaf(__int_as_float(Dq[0]), dwj, ndwj), dx.x, acc[mt][0]);
        acc[mt][1] = fmaf(fmaf(__int_as_float(Dq[1]), dwj, ndwj), dx.y, acc[mt][1]);
        acc[mt][2] = fmaf(fmaf(__int_as_float(Dq[2]), dwj, ndwj), dx.z, acc[mt][2]);
        acc[mt][3] = fmaf(fmaf(__int_as_float(Dq[3]), dwj, ndwj), dx.w, acc[mt][3]);
    }
#pragma unroll
    for (int j4 = 0; j4 < 8; j4 += 4) {
        const uint32_t mw = j4 == 0 ? mn03 : mn47;
        const float bm = -(dmin * static_cast<float>(__builtin_amdgcn_ubfe(mw, 8 * g, 8)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float ax4 = psx[j4 * kSxRow + 16 * mt];
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ax4, bm, acc[mt], 0, 0, 0);
        }
    }
}

// The groups of one pass (the tile is staged; the first D super-blocks of
// group 0 are in flight).  Register set s % D holds super-block s; after it
// is used it is refilled with super-block s + D of the group, or s + D - NSB
// of the next one.
// Group grp of a workgroup's list: the first gmat groups are row groups of
// w (output y), the next gmat those of w2 (output y2), when w2 is given.
struct GroupRef {
    const uint8_t* w;
    float* y;
    int64_t rg;   // row group within the matrix
};

template <bool PAIR>
__device__ __forceinline__ GroupRef group_ref(const uint8_t* w, const uint8_t* w2, float* y, float* y2,
                                              int64_t gmat, int64_t grp) {
    const bool second = PAIR && grp >= gmat;
    return GroupRef{second ? w2 : w, second ? y2 : y, second ? grp - gmat : grp};
}

template <int MT, int NSB, int D, int T, bool PAIR>
__device__ __forceinline__ void whole_groups(const WholeSmem<NSB, T>& s, WRegs (&wr)[D],
                                             const uint8_t* __restrict__ w, const uint8_t* __restrict__ w2,
                                             int64_t gmat, int64_t n, int64_t rb, int e,
                                             int64_t grp0, int nw, int rpl, int lane, int rows,
                                             float* __restrict__ y, float* __restrict__ y2, int64_t ldy) {
    static_assert(NSB % D == 0, "whole sets per group");
    v4i bias;
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = kBias;
    for (int i = 0; i < rpl; ++i) {
        const GroupRef G = group_ref<PAIR>(w, w2, y, y2, gmat, grp0 + static_cast<int64_t>(i) * nw);
        const StreamLane L = group_lane(G.w, n, rb, e, G.rg, lane);
        // past the last group the refills repeat this group's first sets
        StreamLane Ln = L;
        if (i + 1 < rpl) {
            const GroupRef Gn = group_ref<PAIR>(w, w2, y, y2, gmat, grp0 + static_cast<int64_t>(i + 1) * nw);
            Ln = group_lane(Gn.w, n, rb, e, Gn.rg, lane);
        }
        v4f acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][r] = 0.0f;
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            // The tile spans more than the 64 KiB an LDS instruction's
            // offset field reaches; with the lane offsets opaque here, their
            // sums with each super-block's address are formed per super-block
            // instead of one address register per (super-block, tile,
            // sub-block) being held across the loop (which spilled).
            int ox = L.j16 * kSbRow + 8 * L.g, od = 4 * L.g, os = L.g * kSxRow + L.j16;
            asm volatile("" : "+v"(ox), "+v"(od), "+v"(os));
            whole_sb<MT, T>(s.x[sb] + ox, &s.dx[8 * sb][0] + od, &s.sx[8 * sb][0] + os, wr[sb % D], L.g, bias, acc);
            if (sb + D < NSB) issue_w(L.wrow, sb + D, L.g, wr[sb % D]);
            else issue_w(Ln.wrow, sb + D - NSB, Ln.g, wr[sb % D]);
            __builtin_amdgcn_sched_barrier(0);
        }
        store_group<MT>(s, L, rows, acc, G.y, ldy);
    }
}

template <int NW, int NSB, int MTMAX, int RING, bool PAIR>
__global__ __launch_bounds__(NW * 64, NW / 4) void moe_whole_q4k_kernel(
        const uint8_t* __restrict__ w, const uint8_t* __restrict__ w2, int64_t gmat, int64_t n,
        int64_t rb, int rpl, const uint8_t* __restrict__ xq, int x_per_pair,
        const int32_t* __restrict__ offsets, const int32_t* __restrict__ pairs, int np, int top_k,
        float* __restrict__ y, float* __restrict__ y2, int64_t ldy) {
    constexpr int T = 16 * MTMAX;
    constexpr int NT = NW * 64;
    constexpr int UMAX = T * 4 * NSB / NT;   // block pairs per thread
    static_assert(UMAX * NT == T * 4 * NSB, "every thread stages whole pairs");
    __shared__ __align__(16) WholeSmem<NSB, T> s;
    const int e = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t grp0 = static_cast<int64_t>(blockIdx.x) * NW * rpl + wv;
    const int64_t xrb = static_cast<int64_t>(NSB) * 8 * 34;
    int off = offsets[e], end = offsets[e + 1];
    off = off < 0 ? 0 : (off > np ? np : off);
    end = end < off ? off : (end > np ? np : end);

    for (int base = off; base < end; base += T) {
        const int rows = end - base < T ? end - base : T;
        const int mt = (rows + 15) >> 4;          // 16-token tiles holding real rows
        __syncthreads();  // the previous pass is done with the tile and row maps
        if (threadIdx.x < T) {
            int xr = -1, yr = 0;
            if (static_cast<int>(threadIdx.x) < rows) {
                const int p = pairs[base + threadIdx.x];
                if (p >= 0 && p < np) {
                    xr = x_per_pair ? p : p / top_k;
                    yr = p;
                }
            }
            s.xrow[threadIdx.x] = xr;
            s.yrow[threadIdx.x] = yr;
        }
        __syncthreads();
        // activation loads first, then the weights of group 0: the split waits
        // for the (older) activation loads only
        ARegs av[UMAX];
#pragma unroll
        for (int u = 0; u < UMAX; ++u) {
            const int item = static_cast<int>(threadIdx.x) + u * NT;
            issue_pair<NSB, T>(s, xq, xrb, item, av[u]);
        }
        constexpr int D = RING;
        WRegs wr[D];
        {
            const GroupRef G0 = group_ref<PAIR>(w, w2, y, y2, gmat, grp0);
            const StreamLane L0 = group_lane(G0.w, n, rb, e, G0.rg, lane);
#pragma unroll
            for (int sb = 0; sb < D; ++sb) issue_w(L0.wrow, sb, L0.g, wr[sb]);
        }
#pragma unroll
        for (int u = 0; u < UMAX; ++u) {
            const int item = static_cast<int>(threadIdx.x) + u * NT;
            store_pair<NSB, T>(s, item, av[u]);
        }
        __syncthreads();
        switch (mt) {
            case 1: whole_groups<1, NSB, D, T, PAIR>(s, wr, w, w2, gmat, n, rb, e, grp0, NW, rpl, lane, rows, y, y2, ldy); break;
            case 2: whole_groups<2, NSB, D, T, PAIR>(s, wr, w, w2, gmat, n, rb, e, grp0, NW, rpl, lane, rows, y, y2, ldy); break;
            case 3: whole_groups<3, NSB, D, T, PAIR>(s, wr, w, w2, gmat, n, rb, e, grp0, NW, rpl, lane, rows, y, y2, ldy); break;
            default:
                if constexpr (MTMAX >= 4) whole_groups<4, NSB, D, T, PAIR>(s, wr, w, w2, gmat, n, rb, e, grp0, NW, rpl, lane, rows, y, y2, ldy);
                break;
        }
    }
}

}  // namespace

// Q6_K weights are read through one buffer descriptor per matrix (expert),
// with 31-bit byte offsets
static bool q6k_range_ok(int wt, int64_t n, int64_t k) {
    return wt != T_Q6_K || n * (k / 256) * 210 + 4 <= 0x7FFFFFFFll;
}

int gemm_shape_ok(int wt, int64_t n, int64_t k) {
    return (k % 256 == 0 && q6k_range_ok(wt, n, k)) ? 0 : -3;
}

int launch_gemm(int wt, const void* w, int64_t n, int64_t k, const void* xq, int64_t m, float* y,
                int64_t ldy, hipStream_t stream) {
    const int64_t bs = wt == T_Q4_0 ? 18 : wt == T_Q4_1 ? 20 : wt == T_Q8_0 ? 34 : wt == T_Q4_K ? 144
                       : wt == T_Q5_K ? 176 : 210;
    const int64_t qk = wt == T_Q4_K || wt == T_Q5_K || wt == T_Q6_K ? 256 : 32;
    const int64_t rb = k / qk * bs;
    if (!q6k_range_ok(wt, n, k)) return -3;
    const int64_t tiles_m = (m + 127) / 128, tiles_n = (n + 127) / 128;
    const int64_t tiles = tiles_m * tiles_n;
    if (tiles > 0x7FFFFFFF) return -3;
    const dim3 g(static_cast<unsigned>(tiles)), b(kThreads);
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int tm = static_cast<int>(tiles_m), tt = static_cast<int>(tiles);
    switch (wt) {
        case T_Q4_0: hipLaunchKernelGGL(gemm2_kernel<T_Q4_0>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q4_1: hipLaunchKernelGGL(gemm_kernel<T_Q4_1>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q8_0: hipLaunchKernelGGL(gemm2_kernel<T_Q8_0>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q4_K: hipLaunchKernelGGL(gemm_kernel<T_Q4_K>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q5_K: hipLaunchKernelGGL(gemm_kernel<T_Q5_K>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        case T_Q6_K: hipLaunchKernelGGL(gemm_kernel<T_Q6_K>, g, b, 0, stream, wp, n, k, rb, xp, m, y, ldy, tm, tt); break;
        default: return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// The whole-k Q4_K kernel for k of 8 or 6 super-blocks: one workgroup per
// CU, the experts' row groups (of w, then of w2 when given) spread over the
// CUs (gpw groups per workgroup, rpl per wave).  Returns false (nothing
// launched) for other k.
static bool launch_moe_whole(const uint8_t* wp, const uint8_t* wp2, int64_t n_experts, int64_t n,
                             int64_t k, int64_t rb, const uint8_t* xp, int x_per_pair,
                             const int32_t* offsets, const int32_t* pairs, int npi, int tk, float* y,
                             float* y2, int64_t ldy, hipStream_t stream) {
    const int64_t nsb = k / 256;
    if (nsb != 8 && nsb != 6) return false;
    const int nw = nsb == 8 ? 12 : 8;
    const int64_t gmat = (n + 15) / 16;
    const int64_t groups = wp2 ? 2 * gmat : gmat;
    int64_t wpe = device_cu_count() / n_experts;
    wpe = wpe < 1 ? 1 : (wpe > groups ? groups : wpe);
    const int64_t gpw = (groups + wpe - 1) / wpe;
    const int64_t rpl = (gpw + nw - 1) / nw;
    const int64_t wgs = (groups + nw * rpl - 1) / (nw * rpl);
    const dim3 gw(static_cast<unsigned>(wgs), static_cast<unsigned>(n_experts));
    const int rp = static_cast<int>(rpl);
    // (the two-matrix launch is its own instantiation, so a kernel trace
    // tells it from the single-matrix one)
    if (nsb == 8 && wp2)
        hipLaunchKernelGGL((moe_whole_q4k_kernel<12, 8, 3, 2, true>), gw, dim3(12 * 64), 0, stream, wp, wp2,
                           gmat, n, rb, rp, xp, x_per_pair, offsets, pairs, npi, tk, y, y2, ldy);
    else if (nsb == 8)
        hipLaunchKernelGGL((moe_whole_q4k_kernel<12, 8, 3, 2, false>), gw, dim3(12 * 64), 0, stream, wp, wp2,
                           gmat, n, rb, rp, xp, x_per_pair, offsets, pairs, npi, tk, y, y2, ldy);
    else if (wp2)
        hipLaunchKernelGGL((moe_whole_q4k_kernel<8, 6, 4, 3, true>), gw, dim3(8 * 64), 0, stream, wp, wp2,
                           gmat, n, rb, rp, xp, x_per_pair, offsets, pairs, npi, tk, y, y2, ldy);
    else
        hipLaunchKernelGGL((moe_whole_q4k_kernel<8, 6, 4, 3, false>), gw, dim3(8 * 64), 0, stream, wp, wp2,
                           gmat, n, rb, rp, xp, x_per_pair, offsets, pairs, npi, tk, y, y2, ldy);
    return true;
}

int moe_shape_ok(int wt, int64_t n, int64_t k) {
    return (k % 256 == 0 && q6k_range_ok(wt, n, k)) ? 0 : -3;
}

int launch_moe_gemm(int wt, const void* w, int64_t n_experts, int64_t n, int64_t k,
                    const void* xq, int x_per_pair, const int32_t* offsets,
                    const int32_t* pairs, int64_t n_tokens, int64_t top_k, float* y,
                    int64_t ldy, hipStream_t stream) {
    const int64_t bs = wt == T_Q4_0 ? 18 : wt == T_Q4_1 ? 20 : wt == T_Q8_0 ? 34 : wt == T_Q4_K ? 144
                       : wt == T_Q5_K ? 176 : 210;
    const int64_t qk = wt == T_Q4_K || wt == T_Q5_K || wt == T_Q6_K ? 256 : 32;
    const int64_t rb = k / qk * bs;
    if (!q6k_range_ok(wt, n, k)) return -3;
    const int64_t tiles_n = (n + 127) / 128;
    const int64_t np = n_tokens * top_k;
    if (tiles_n > 0x7FFFFFFF || np > 0x7FFFFFFF) return -3;
    const dim3 g(static_cast<unsigned>(tiles_n), static_cast<unsigned>(n_experts)), b(kThreads);
    const uint8_t* wp = static_cast<const uint8_t*>(w);
    const uint8_t* xp = static_cast<const uint8_t*>(xq);
    const int npi = static_cast<int>(np), tk = static_cast<int>(top_k);
    switch (wt) {
        case T_Q4_0: hipLaunchKernelGGL(moe_gemm_kernel<T_Q4_0>, g, b, 0, stream, wp, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk, y, ldy); break;
        case T_Q4_1: hipLaunchKernelGGL(moe_gemm_kernel<T_Q4_1>, g, b, 0, stream, wp, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk, y, ldy); break;
        case T_Q8_0: hipLaunchKernelGGL(moe_gemm_kernel<T_Q8_0>, g, b, 0, stream, wp, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk, y, ldy); break;
        case T_Q5_K: hipLaunchKernelGGL(moe_gemm_kernel<T_Q5_K>, g, b, 0, stream, wp, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk, y, ldy); break;
        case T_Q6_K: hipLaunchKernelGGL(moe_gemm_kernel<T_Q6_K>, g, b, 0, stream, wp, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk, y, ldy); break;
        case T_Q4_K: {
            if (launch_moe_whole(wp, nullptr, n_experts, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk,
                                 y, nullptr, ldy, stream))
                break;
            const dim3 gs(static_cast<unsigned>((n + kSbRows - 1) / kSbRows), static_cast<unsigned>(n_experts));
            hipLaunchKernelGGL(moe_stream_q4k_kernel, gs, dim3(kStreamThreads), 0, stream, wp, n, k, rb, xp, x_per_pair, offsets, pairs, npi, tk, y, ldy);
            break;
        }
        default: return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Two grouped products over the same activation rows (w -> y, w2 -> y2):
// one launch over both matrices where the whole-k kernel applies (one
// split of each expert's activation rows serves both), else two launches.
int launch_moe_gemm2(int wt, const void* w, const void* w2, int64_t n_experts, int64_t n, int64_t k,
                     const void* xq, int x_per_pair, const int32_t* offsets, const int32_t* pairs,
                     int64_t n_tokens, int64_t top_k, float* y, float* y2, int64_t ldy,
                     hipStream_t stream) {
    if (wt == T_Q4_K) {
        const int64_t rb = k / 256 * 144;
        const int64_t np = n_tokens * top_k;
        if (np > 0x7FFFFFFF) return -3;
        if (launch_moe_whole(static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(w2), n_experts, n,
                             k, rb, static_cast<const uint8_t*>(xq), x_per_pair, offsets, pairs,
                             static_cast<int>(np), static_cast<int>(top_k), y, y2, ldy, stream))
            return hipGetLastError() == hipSuccess ? 0 : -6;
    }
    if (int rc = launch_moe_gemm(wt, w, n_experts, n, k, xq, x_per_pair, offsets, pairs, n_tokens, top_k,
                                 y, ldy, stream))
        return rc;
    return launch_moe_gemm(wt, w2, n_experts, n, k, xq, x_per_pair, offsets, pairs, n_tokens, top_k, y2,
                           ldy, stream);
}

}  // namespace cq

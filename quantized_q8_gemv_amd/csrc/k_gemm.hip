// k_gemm.hip -- Q8_0 x f32 matrix-matrix product on MFMA (prefill).
//
// Prefill runs every projection on T token rows at once ("生成一个 token",
// section "prefill 和 decode：同一个 forward，不同的路": several input rows take
// the matrix-matrix kernel). Y[T][N] = U[T][K] . W[N][K]^T with W in Q8_0.
//
// gfx950 has v_mfma_f32_16x16x32_f16, whose K = 32 is exactly one Q8_0 block.
// Per 32-wide block and 16x16 output tile:
//   * B = the block's int8 values as f16 (exact: |q| <= 127);
//   * A = the activations as an f16 pair hi + lo (u = hi + lo to ~2^-22
//     relative); two MFMAs accumulate (hi + lo) . q in f32;
//   * the block's f16 scale d (one per output column = one per lane) is then
//     applied in f32: acc += d * tile.
// The result is f32-accurate up to summation order; the int8 values are never
// rounded and the scale is never folded into f16.
//
// Activations arrive already split: the RMSNorm kernel, the attention kernel
// and the gate/up epilogue write their outputs as an f16 hi plane [T][K]
// followed by an f16 lo plane, so a K step of A is a plain copy. (The single-op
// entry point passes f32 activations; that variant splits them on the way into
// LDS.)
//
// Workgroup tile TM tokens x TN output rows, 4 waves in 2 x 2, K in steps of
// 64 (one block pair per row, 68 bytes, 4-byte aligned). Software pipeline:
// the global loads of the next few K steps are in flight in registers while
// the MFMAs of the current step run from LDS (a step's MFMA work is far
// shorter than a global round trip); two LDS buffers, one barrier per step.

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int GK = 64;     // weights per K step (two Q8_0 blocks)
constexpr int LPAD = 64;   // halves per LDS row of a tile (64 weights of K, 8 chunks of 16 bytes)

// Half offset of (row, col) in an LDS tile, col inside one 16-byte chunk
// (col % 8 + the access width <= 8). Chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7): the 16 rows a fragment read takes (16-byte lanes, one
// chunk each) and the rows a store covers then fall on distinct bank groups,
// with no padding.
__device__ __forceinline__ int lds_h(int row, int col) {
    return row * LPAD + ((((col >> 3) ^ (row >> 1)) & 7) << 3) + (col & 7);
}

// The same with the row's key (row >> 1) & 7 given: a thread's store rows
// differ by multiples of 16, so its key is fixed and kept in one register.
__device__ __forceinline__ int lds_hk(int row, int col, int key) {
    return row * LPAD + ((((col >> 3) ^ key) & 7) << 3) + (col & 7);
}

// Column offset of a lane's fragment chunk (half-block hb, lane group
// lane / 16) in tile rows of the form 16 i + lane % 16: their swizzle key is
// (lane % 16) / 2 for every i.
__device__ __forceinline__ int frag_col(int hb, int lane) {
    return ((((hb * 4 + (lane >> 4)) ^ ((lane & 15) >> 1)) & 7) << 3);
}

enum GemmEpi { G_STORE = 0, G_ACCUM = 1, G_QKV = 2, G_GATEUP = 3, G_PART = 4 };

struct GemmArgs {
    const void *A;         // A32: f32 [T][K]; else f16 hi plane [T][K] then lo plane [T][K]
    const uint8_t *W[3];   // matrices (q, k, v | gate, up | single)
    int Nm[3];             // rows of each matrix
    int tiles[3];          // row tiles of each matrix (QKV)
    int T, K, rowbytes;
    // G_STORE / G_ACCUM
    float *Y;              // [T][N]
    // G_QKV
    const StepState *st;
    const float2 *rope;
    float *q, *kc, *vc;
    int QD, hd, max_seq;
    int rope_neox;         // 1: q and k are written unrotated
    // G_GATEUP: h = silu(gate) * up as f16 hi plane [T][F] then lo plane
    _Float16 *h;
    // G_PART: K split over gridDim.z slices; slice z writes its sum to part[z][T][N]
    float *part;
    int splits;
    ActScale sc;           // activation scaling (see ActScale)
};

template <int TM, int TN>
struct Cfg {
    static constexpr int WM = TM / 2, WN = TN / 2;       // wave tile
    static constexpr int MS = WM / 16, NS = WN / 16;     // MFMA tiles per wave
    static constexpr int AP = TM * 16 / kThreads;        // 16-byte A pieces per thread per step
    static constexpr int BU = TN * 4 / kThreads;         // B quarter rows per thread per step
    static constexpr int A_HALVES = TM * LPAD;
    static constexpr int B_HALVES = TN * LPAD;
    static constexpr size_t BUF = sizeof(_Float16) * (2 * A_HALVES + B_HALVES) + sizeof(float) * TN * 2;
    // LDS buffers: one when a single K step of loads is in flight (grids
    // that fill the chip: a second barrier per step, but half the LDS, so
    // more workgroups per CU; 7B-class 512-token prefill 28.2 -> 27.1 ms,
    // 135M 4000-token 11.9 -> 11.0 ms, 203-token 1.84 -> 1.86 ms; with one
    // buffer for the large tile only, 27.3 and 11.4 ms), two for the
    // small-grid walk that keeps several steps in flight
    static constexpr bool one_buffer(int st) { return st == 1; }
    static constexpr size_t lds(int st) { return (one_buffer(st) ? 1 : 2) * BUF; }
    static_assert(AP >= 1 && BU >= 1 && MS >= 1 && NS >= 1, "tile too small");
    static_assert(BUF % 16 == 0, "LDS buffer alignment");
    static_assert(size_t(TM) * WN * sizeof(float) <= BUF, "gate/up exchange fits");
};

struct GBuf {
    _Float16 *ahi, *alo, *bq;
    float *bd;
};

template <int TM, int TN>
__device__ inline GBuf gbuf(uint8_t *smem, int k) {
    using C = Cfg<TM, TN>;
    GBuf b;
    uint8_t *p = smem + size_t(k) * C::BUF;
    b.ahi = reinterpret_cast<_Float16 *>(p);
    b.alo = b.ahi + C::A_HALVES;
    b.bq = b.alo + C::A_HALVES;
    b.bd = reinterpret_cast<float *>(b.bq + C::B_HALVES);
    return b;
}

// Dwords a thread loads per B quarter row and step: a Q8_0 quarter is 16
// values and a scale or a dword of slack (5), a Q5_0 quarter reads its whole
// 22-byte block from the dword-aligned floor (6).
template <int FMT>
constexpr int quarter_dwords() { return FMT == F_Q5_0 ? 6 : 5; }

template <int FMT>
constexpr int pair_bytes() { return FMT == F_Q5_0 ? kQ5PairBytes : kPairBytes; }

// Registers holding one K step of global data in flight.
template <int TM, int TN, int FMT>
struct GRegs {
    u32x4 a[Cfg<TM, TN>::AP];
    uint32_t b[Cfg<TM, TN>::BU][quarter_dwords<FMT>()];
};

// First dword of quarter qd (block qd / 2, values 16 (qd % 2) .. +15) of a
// block pair. Q8_0, 68 bytes: 0 -> d0 + q0..15 of block 0 (dwords 0..4), 1 ->
// q16..31 + d1 (4..8), 2 -> q0..15 of block 1 (9..13, the last unused), 3 ->
// q16..31 of block 1 (12..16, the first unused). Q5_0, 44 bytes: block 0 is
// bytes 0..21 (dwords 0..5), block 1 bytes 22..43 (dwords 5..10); both
// quarters of a block read the whole block (the fifth bits and the nibbles
// of values j and j + 16 share bytes).
template <int FMT>
__device__ inline int quarter_base(int qd) {
    if (FMT == F_Q5_0) return qd < 2 ? 0 : 5;
    return qd == 0 ? 0 : qd == 1 ? 4 : qd == 2 ? 9 : 12;
}

// Buffer-load sources of a thread: one resource per operand and a fixed byte
// offset per piece; a K step adds a uniform offset. Rows past the end of A or
// W get an offset past the resource's size, so the hardware range check
// returns zeros (no branches; those rows' results are never stored).
constexpr uint32_t kOutOfRange = 0x80000000u;   // resources are < kOutOfRange bytes
constexpr int kRsrcWord3 = 0x00020000;           // raw buffer, 32-bit data format

template <int TM, int TN>
struct GSrc {
    __amdgpu_buffer_rsrc_t ra;
    __amdgpu_buffer_rsrc_t rb[Cfg<TM, TN>::BU];
    uint32_t aoff[Cfg<TM, TN>::AP];
    uint32_t boff[Cfg<TM, TN>::BU];
};

// A-side (activation) sources: shared by the Q8_0 and the K-format kernels.
template <bool A32, int TM, int TN>
__device__ inline void a_setup(const GemmArgs &a, int m0, __amdgpu_buffer_rsrc_t &ra, uint32_t *aoff) {
    using C = Cfg<TM, TN>;
    const int tid = threadIdx.x;
    const uint32_t abytes = uint32_t(size_t(a.T) * a.K * 4);  // f32, or two f16 planes
    ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.A), 0, int(abytes), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int c = tid + i * kThreads;
        if (A32) {
            const int m = c >> 4;
            aoff[i] = m0 + m < a.T ? uint32_t((size_t(m0 + m) * a.K + (c & 15) * 4) * 4) : kOutOfRange;
        } else {
            const int plane = c / (TM * 8), rr = c - plane * (TM * 8);
            const int m = rr >> 3;
            aoff[i] = m0 + m < a.T
                          ? uint32_t((size_t(plane) * a.T * a.K + size_t(m0 + m) * a.K + (rr & 7) * 8) * 2)
                          : kOutOfRange;
        }
    }
}

template <bool A32, int TM, int TN, int EPI, int FMT>
__device__ inline void g_setup(const GemmArgs &a, int m0, int row0, const int nvalid[2],
                               const uint8_t *const Wb[2], GSrc<TM, TN> &g) {
    using C = Cfg<TM, TN>;
    const int tid = threadIdx.x;
    a_setup<A32, TM, TN>(a, m0, g.ra, g.aoff);
#pragma unroll
    for (int i = 0; i < C::BU; ++i) {
        const int u = tid + i * kThreads;
        const int b = u >> 2, qd = u & 3;
        // wave-uniform: a wave's B rows all come from one matrix
        const int part = (EPI == G_GATEUP) ? __builtin_amdgcn_readfirstlane(b >= TN / 2 ? 1 : 0) : 0;
        const int rr = (EPI == G_GATEUP) ? (b - part * (TN / 2)) : b;
        const uint8_t *W = part ? Wb[1] : Wb[0];
        g.rb[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), 0,
                                                    int(uint32_t(row0 + nvalid[part]) * uint32_t(a.rowbytes)),
                                                    kRsrcWord3);
        g.boff[i] = rr < nvalid[part] ? uint32_t(row0 + rr) * uint32_t(a.rowbytes) + quarter_base<FMT>(qd) * 4
                                      : kOutOfRange;
    }
}

template <bool A32, int TM, int TN>
__device__ inline void a_load(__amdgpu_buffer_rsrc_t ra, const uint32_t *aoff, int ks, u32x4 *ra_out) {
    using C = Cfg<TM, TN>;
    const int sa = ks * GK * (A32 ? 4 : 2);
#pragma unroll
    for (int i = 0; i < C::AP; ++i) ra_out[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i], sa, 0);
}

template <bool A32, int TM, int TN, int FMT>
__device__ inline void g_load(const GSrc<TM, TN> &g, int ks, GRegs<TM, TN, FMT> &r) {
    using C = Cfg<TM, TN>;
    a_load<A32, TM, TN>(g.ra, g.aoff, ks, r.a);
    const int sb = ks * pair_bytes<FMT>();
#pragma unroll
    for (int i = 0; i < C::BU; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(g.rb[i], g.boff[i], sb, 0);
        r.b[i][0] = v.x;
        r.b[i][1] = v.y;
        r.b[i][2] = v.z;
        r.b[i][3] = v.w;
        if constexpr (FMT == F_Q5_0) {
            const uint2 t = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(g.rb[i], g.boff[i] + 16, sb, 0));
            r.b[i][4] = t.x;
            r.b[i][5] = t.y;
        } else {
            r.b[i][4] = __builtin_amdgcn_raw_buffer_load_b32(g.rb[i], g.boff[i] + 16, sb, 0);
        }
    }
}

// Four unsigned bytes u (one dword) -> 4 exact f16 values u - zero: place
// each byte in the mantissa of 1024.0 (f16 bits 0x6400 | u) and subtract
// 1024 + zero. Q8_0 passes its int8 values biased to q + 128 (zero 128), Q5_0
// its 5-bit codes (zero 16).
template <int ZERO>
__device__ inline void u4_to_half(uint32_t x, half2v &lo, half2v &hi) {
    const uint32_t l = __builtin_amdgcn_perm(0x64646464u, x, 0x05010400u);
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, x, 0x07030602u);
    const half2v bias = {static_cast<_Float16>(1024.0f + ZERO), static_cast<_Float16>(1024.0f + ZERO)};
    lo = __builtin_bit_cast(half2v, l) - bias;
    hi = __builtin_bit_cast(half2v, h) - bias;
}

// Step ks of the A tile, registers -> LDS. f32 input (A32) is split into an
// f16 pair here; a value outside the pair's range (|v| >= 2^15, or not
// finite) sets sc.range_flag. Split planes are copied, and when `resc` (some
// row of the tile has a nonzero row exponent sc.eg) block b of row t is
// first multiplied by 2^(eg[t] - el[t][b]): every block of a row then carries
// the row's common exponent, which the epilogue takes out (exact powers of
// two; a block far below the row's largest may lose bits to f16 subnormals).
template <bool A32, int TM, int TN>
__device__ inline void a_store(const u32x4 *ra, _Float16 *ahi, _Float16 *alo, const GemmArgs &a, int m0, int ks,
                               bool resc) {
    using C = Cfg<TM, TN>;
    const int tid = threadIdx.x;
    // row keys: A32 rows tid / 16 + 16 i, else tid / 8 + (0 or 32)
    static_assert(kThreads % 256 == 0 && (TM * 8) % 256 == 0, "store rows differ by multiples of 16");
    const int key = A32 ? (tid >> 5) & 7 : (tid >> 4) & 7;
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int c = tid + i * kThreads;
        if (A32) {
            const int m = c >> 4, c4 = c & 15;
            const float4 v = __builtin_bit_cast(float4, ra[i]);
            const float vv[4] = {v.x, v.y, v.z, v.w};
            _Float16 hi[4], lo[4];
            bool bad = false;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                bad |= !(fabsf(vv[k]) < kPairRange);
                hi[k] = static_cast<_Float16>(vv[k]);
                lo[k] = static_cast<_Float16>(vv[k] - static_cast<float>(hi[k]));
            }
            if (bad && a.sc.range_flag) *a.sc.range_flag = 1u;
            *reinterpret_cast<uint2 *>(ahi + lds_hk(m, c4 * 4, key)) = __builtin_bit_cast(uint2, hi);
            *reinterpret_cast<uint2 *>(alo + lds_hk(m, c4 * 4, key)) = __builtin_bit_cast(uint2, lo);
        } else {
            // thread tid stores chunk tid % 8 of rows tid / 8 + a multiple of 32
            // (per i, known at compile time) of the hi or the lo plane
            constexpr int kPlaneRows = TM * 8;
            const int plane = (i * kThreads) / kPlaneRows;
            const int m = (tid >> 3) + ((i * kThreads) % kPlaneRows) / 8, p = tid & 7;
            u32x4 v = ra[i];
            if (resc && m0 + m < a.T) {
                const int t = m0 + m;
                const int dexp = a.sc.eg[t] - int(a.sc.el[size_t(t) * a.sc.el_stride + 2 * ks + (p >> 2)]);
                if (dexp != 0) {
                    half8 h = __builtin_bit_cast(half8, v);
#pragma unroll
                    for (int k = 0; k < 8; ++k) h[k] = static_cast<_Float16>(ldexpf(static_cast<float>(h[k]), dexp));
                    v = __builtin_bit_cast(u32x4, h);
                }
            }
            const int off = (tid >> 3) * LPAD + (((p ^ key) & 7) << 3);   // this thread's chunk in row tid / 8
            *reinterpret_cast<u32x4 *>((plane ? alo : ahi) + off + ((i * kThreads) % kPlaneRows) / 8 * LPAD) = v;
        }
    }
}

// Whether some row of the tile starting at m0 carries a nonzero row exponent
// (then its A blocks are brought to the row's exponent on their way to LDS).
template <int TM>
__device__ inline bool tile_rescales(const GemmArgs &a, int m0) {
    int any = 0;
    if (a.sc.eg && threadIdx.x < TM && m0 + int(threadIdx.x) < a.T) any = a.sc.eg[m0 + threadIdx.x] != 0;
    return __syncthreads_or(any) != 0;
}

// The factors that take the rows' scaling out of a product: sc.rs[t] (the
// normalised input's per-row factor) times 2^-eg[t] (the row exponent, 0
// where rows are not rescaled), for the rows t = m0 + wm*WM + ms*16 +
// 4*(lane/16) + i this lane's accumulators hold (1 past T). Loaded at the
// start of the kernel, so the epilogue does not wait for them.
template <int TM, int TN>
struct RowFactors {
    float f[Cfg<TM, TN>::MS][4];
    __device__ __forceinline__ void load(const GemmArgs &a, int m0, int wm, int lane) {
        using C = Cfg<TM, TN>;
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = min(m0 + wm * C::WM + ms * 16 + 4 * (lane >> 4) + i, a.T - 1);
                const float r = a.sc.rs ? a.sc.rs[t] : 1.0f;
                f[ms][i] = a.sc.eg ? ldexpf(r, -a.sc.eg[t]) : r;
            }
    }
};

template <bool A32, int TM, int TN, int FMT>
__device__ inline void g_store(const GRegs<TM, TN, FMT> &r, const GBuf &bf, const GemmArgs &a, int m0, int ks,
                               bool resc) {
    using C = Cfg<TM, TN>;
    const int tid = threadIdx.x;
    a_store<A32, TM, TN>(r.a, bf.ahi, bf.alo, a, m0, ks, resc);
#pragma unroll
    for (int i = 0; i < C::BU; ++i) {
        const int u = tid + i * kThreads;
        const int b = u >> 2, qd = u & 3;
        const uint32_t *w = r.b[i];
        half2v v[8];
        if constexpr (FMT == F_Q5_0) {
            // block 0 (qd 0, 1): d in bytes 0..1, the fifth-bit word and the
            // nibbles 2 bytes into a dword; block 1 (qd 2, 3): d in bytes 2..3,
            // word and nibbles dword-aligned. Quarter qd & 1 takes the high
            // nibbles and bits 16..31 of the word.
            const bool blk1 = qd >= 2, hi = qd & 1;
            const uint32_t qh = blk1 ? w[1] : __builtin_amdgcn_alignbyte(w[1], w[0], 2);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t qs = blk1 ? w[k + 2] : __builtin_amdgcn_alignbyte(w[k + 2], w[k + 1], 2);
                u4_to_half<16>(q5_bytes(qs, qh, k, hi), v[2 * k], v[2 * k + 1]);
            }
        } else {
            const uint32_t shift = qd < 2 ? 2u : 0u;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t q4 = qd == 3 ? w[k + 1] : __builtin_amdgcn_alignbyte(w[k + 1], w[k], shift);
                u4_to_half<128>(q4 ^ 0x80808080u, v[2 * k], v[2 * k + 1]);
            }
        }
        const u32x4 s0 = u32x4{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                               __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
        const u32x4 s1 = u32x4{__builtin_bit_cast(uint32_t, v[4]), __builtin_bit_cast(uint32_t, v[5]),
                               __builtin_bit_cast(uint32_t, v[6]), __builtin_bit_cast(uint32_t, v[7])};
        // rows tid / 4 + 64 i: this thread's two chunks in row tid / 4, plus
        // i * 64 rows
        const int col = (tid & 2) * 16 + (tid & 1) * 16, key = (tid >> 3) & 7;
        const int rofs = i * (kThreads / 4) * LPAD;
        *reinterpret_cast<u32x4 *>(bf.bq + lds_hk(tid >> 2, col, key) + rofs) = s0;
        *reinterpret_cast<u32x4 *>(bf.bq + lds_hk(tid >> 2, col + 8, key) + rofs) = s1;
        if (FMT == F_Q5_0) {
            if (qd == 0) bf.bd[b * 2 + 0] = half_bits_to_float(w[0] & 0xffffu);
            if (qd == 2) bf.bd[b * 2 + 1] = half_bits_to_float(w[0] >> 16);
        } else {
            if (qd == 0) bf.bd[b * 2 + 0] = half_bits_to_float(w[0] & 0xffffu);
            if (qd == 1) bf.bd[b * 2 + 1] = half_bits_to_float(w[4] >> 16);
        }
    }
}

// FMT: the weights' block format, Q8_0 or Q5_0 (a pair of 64 weights per K
// step either way; only the B tile's load and decode differ).
//
// The large-tile Q8_0 q/k/v and gate/up kernels of grids that fill the chip
// are held to 128 VGPRs (4 waves per SIMD instead of 3, with the row factors
// loaded in the epilogue instead of at the start: 7B-class 512-token prefill
// 27.5 -> 26.9 ms); the accumulating and the Q5_0 kernels would spill there.
template <int FMT, int EPI, int TM, int ST>
constexpr bool gemm_four_waves() {
    return FMT == F_Q8_0 && ST == 1 && TM == 64 && (EPI == G_QKV || EPI == G_GATEUP);
}

template <int FMT, int EPI, int TM, int TN, bool A32, int ST>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(gemm_four_waves<FMT, EPI, TM, ST>() ? 4 : 1)))
void k_gemm_q8(GemmArgs a) {
    using C = Cfg<TM, TN>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = blockIdx.x * TM;

    // Which weight rows feed B rows [0, TN) of this tile.
    int mat = 0, row0 = 0;
    const uint8_t *Wb[2] = {nullptr, nullptr};
    int nvalid[2] = {0, 0};
    if (EPI == G_GATEUP) {
        row0 = blockIdx.y * (TN / 2);
        Wb[0] = a.W[0];
        Wb[1] = a.W[1];
        nvalid[0] = nvalid[1] = min(TN / 2, a.Nm[0] - row0);
    } else {
        int t = blockIdx.y;
        if (EPI == G_QKV) {
            while (mat < 2 && t >= a.tiles[mat]) t -= a.tiles[mat++];
        }
        row0 = t * TN;
        Wb[0] = a.W[mat];
        nvalid[0] = min(TN, a.Nm[mat] - row0);
    }

    f32x4 acc[C::MS][C::NS];
#pragma unroll
    for (int i = 0; i < C::MS; ++i)
#pragma unroll
        for (int j = 0; j < C::NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // S register stages: the loads of steps ks+1 .. ks+S are in flight while
    // step ks is computed (the loop is unrolled by S so each stage is a fixed
    // set of registers).
    constexpr int S = ST;
    int kfirst = 0, nsteps = a.K / GK;
    if (EPI == G_PART) {  // this workgroup's slice of the K steps
        const int all = nsteps;
        kfirst = int(blockIdx.z) * all / a.splits;
        nsteps = (int(blockIdx.z) + 1) * all / a.splits - kfirst;
    }
    GSrc<TM, TN> src;
    g_setup<A32, TM, TN, EPI, FMT>(a, m0, row0, nvalid, Wb, src);
    // only products of the gate/up output (o-type epilogues) see per-block
    // exponents; q/k/v and gate/up read the normalised rows (row factors only)
    constexpr bool kResc = !A32 && EPI != G_QKV && EPI != G_GATEUP;
    const bool resc = kResc ? tile_rescales<TM>(a, m0) : false;
    constexpr bool kLateRows = gemm_four_waves<FMT, EPI, TM, ST>();
    RowFactors<TM, TN> rf;
    if (!kLateRows) rf.load(a, m0, wm, lane);
    // Every stage issues its loads unconditionally (steps past the end
    // re-read the last step, whose registers are never stored): with no
    // branch around them the compiler can wait for the oldest stage alone
    // instead of draining every load in flight.
    GRegs<TM, TN, FMT> regs[S];
#pragma unroll
    for (int j = 0; j < S; ++j) g_load<A32, TM, TN, FMT>(src, kfirst + min(j, nsteps - 1), regs[j]);
    for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int ks = k0 + j;
            if (ks >= nsteps) break;
            constexpr bool kOne = C::one_buffer(S);
            const GBuf bf = gbuf<TM, TN>(smem, kOne ? 0 : (ks & 1));
            if (kOne) __syncthreads();   // (one buffer) every wave is done with the previous step
            g_store<A32, TM, TN, FMT>(regs[j], bf, a, m0, kfirst + ks, resc);
            __syncthreads();
            if (S == 1) {
                if (ks + 1 < nsteps) g_load<A32, TM, TN, FMT>(src, kfirst + ks + 1, regs[j]);
            } else {
                g_load<A32, TM, TN, FMT>(src, kfirst + min(ks + S, nsteps - 1), regs[j]);
            }
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                half8 bfr[C::NS];
                float dsc[C::NS];
                const int fc = frag_col(hb, lane);
#pragma unroll
                for (int ns = 0; ns < C::NS; ++ns) {
                    const int col = wn * C::WN + ns * 16 + (lane & 15);
                    bfr[ns] = *reinterpret_cast<const half8 *>(bf.bq + col * LPAD + fc);
                    dsc[ns] = bf.bd[col * 2 + hb];
                }
#pragma unroll
                for (int ms = 0; ms < C::MS; ++ms) {
                    const int row = wm * C::WM + ms * 16 + (lane & 15);
                    const half8 ah = *reinterpret_cast<const half8 *>(bf.ahi + row * LPAD + fc);
                    const half8 al = *reinterpret_cast<const half8 *>(bf.alo + row * LPAD + fc);
#pragma unroll
                    for (int ns = 0; ns < C::NS; ++ns) {
                        f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bfr[ns], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bfr[ns], t, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[ms][ns][i] = fmaf(dsc[ns], t[i], acc[ms][ns][i]);
                    }
                }
            }
        }
    }

    if (kLateRows) rf.load(a, m0, wm, lane);
    // ---- epilogue: acc[ms][ns][i] is (m, c) with
    //      m = wm*WM + ms*16 + 4*(lane/16) + i, c = wn*WN + ns*16 + lane%16
    if (EPI == G_GATEUP) {
        // waves with wn = 1 hold the up rows: pass them to the wn = 0 waves through LDS
        __syncthreads();  // every wave is done with the K-step buffers
        float *ub = reinterpret_cast<float *>(smem);  // TM x WN f32
        if (wn == 1) {
#pragma unroll
            for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < C::NS; ++ns)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = wm * C::WM + ms * 16 + 4 * (lane >> 4) + i;
                        const int c = ns * 16 + (lane & 15);
                        ub[m * C::WN + c] = acc[ms][ns][i];
                    }
        }
        __syncthreads();
        if (wn == 0) {
            // h = silu(g) * up in f32, then per (row, 32-column block) the
            // exponent that keeps the block's largest |h| below 2^15 (0 when it
            // already is): the block's 32 columns are ns = 2bb, 2bb + 1 of the
            // 16 lanes sharing lane >> 4.
            const size_t plane = size_t(a.T) * a.Nm[0];
#pragma unroll
            for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = wm * C::WM + ms * 16 + 4 * (lane >> 4) + i;
                    const int t = m0 + m;
                    const float f = rf.f[ms][i];
                    float hv[C::NS];
#pragma unroll
                    for (int ns = 0; ns < C::NS; ++ns) {
                        const int c = ns * 16 + (lane & 15);
                        const float h = silu(acc[ms][ns][i] * f) * (ub[m * C::WN + c] * f);
                        hv[ns] = (t < a.T && c < nvalid[0]) ? h : 0.f;
                    }
#pragma unroll
                    for (int bb = 0; bb < (C::NS + 1) / 2; ++bb) {
                        float mx = fabsf(hv[2 * bb]);
                        if (2 * bb + 1 < C::NS) mx = fmaxf(mx, fabsf(hv[2 * bb + 1]));
                        mx = row16_max_dpp(mx);
                        int e = 0;
                        if (!(mx < kPairRange)) e = isfinite(mx) ? max(14 - ilogbf(mx), -126) : -126;
                        // el[t][.] was cleared with eg[t] by the norm kernel: only
                        // nonzero exponents are written
                        if (e != 0 && t < a.T && a.sc.el_out && (lane & 15) == 0 && 32 * bb < nvalid[0]) {
                            a.sc.el_out[size_t(t) * a.sc.el_stride + (row0 >> 5) + bb] = int8_t(e);
                            atomicMin(a.sc.eg_out + t, e);
                        }
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int ns = 2 * bb + q;
                            const int c = ns * 16 + (lane & 15);
                            if (ns < C::NS && t < a.T && c < nvalid[0])
                                store_hilo(a.h, plane, size_t(t) * a.Nm[0] + row0 + c, ldexpf(hv[ns], e));
                        }
                    }
                }
        }
        return;
    }
    // q/k/v: each value is range-checked here, where it is written (the
    // prefill attention splits Q, K and V into f16 pairs)
    bool bad = false;
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < C::NS; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = wm * C::WM + ms * 16 + 4 * (lane >> 4) + i;
                const int c = wn * C::WN + ns * 16 + (lane & 15);
                const float v = acc[ms][ns][i] * rf.f[ms][i];
                if (EPI == G_QKV) {
                    // rope pairs (2j, 2j+1) sit in adjacent lanes
                    const float partner = __shfl_xor(v, 1, 64);
                    if (m0 + m >= a.T || c >= nvalid[0]) continue;
                    const int row = row0 + c;
                    const int d = row % a.hd;
                    const int t = m0 + m;
                    if (mat == 2 || a.rope_neox) {
                        float *dst = mat == 0 ? a.q + size_t(t) * a.QD + row
                                              : (mat == 1 ? a.kc : a.vc) +
                                                    (size_t(row / a.hd) * a.max_seq + a.st->slot + t) * a.hd + d;
                        if (mat == 2) bad |= !(fabsf(v) < kPairRange);   // (NEOX q, k: checked once rotated)
                        *dst = v;
                    } else {
                        const float2 cs = a.rope[size_t(a.st->pos + t) * (a.hd / 2) + (d >> 1)];
                        const float r = (d & 1) ? (partner * cs.y + v * cs.x) : (v * cs.x - partner * cs.y);
                        bad |= !(fabsf(r) < kPairRange);
                        if (mat == 0)
                            a.q[size_t(t) * a.QD + row] = r;
                        else
                            a.kc[(size_t(row / a.hd) * a.max_seq + a.st->slot + t) * a.hd + d] = r;
                    }
                } else if (EPI == G_PART) {
                    if (m0 + m >= a.T || c >= nvalid[0]) continue;
                    a.part[(size_t(blockIdx.z) * a.T + m0 + m) * a.Nm[0] + row0 + c] = v;
                } else {
                    if (m0 + m >= a.T || c >= nvalid[0]) continue;
                    float *dst = a.Y + size_t(m0 + m) * a.Nm[0] + row0 + c;
                    *dst = (EPI == G_ACCUM) ? *dst + v : v;
                }
            }
    if (EPI == G_QKV && bad && a.sc.range_flag) *a.sc.range_flag = 1u;
}

// ---- 256-weight block formats (Q4_K, Q6_K), 64 weights per K step.
//
// Q4_K, step ks of a row: block ks/4, chunk c = ks%4 = sub-block 2c (low
// nibbles of bytes 32c..32c+31) and sub-block 2c+1 (their high nibbles). A
// sub-block holds (d*s)*q - dmin*m with q in 0..15: the MFMAs take q as f16
// (exact), the product d*s is applied in f32 per sub-block as the Q8_0 scale
// is, and the min term needs each token's activation sum over the sub-block,
// which one more MFMA pair against a B of ones gives (shared by all rows).
// Q6_K, step ks: block ks/4, half h = (ks%4)/2, k-pair kk = ks%2: values
// 32k + l of half h for k = 2kk, 2kk+1, each 16 with its own int8 scale. The
// MFMA's 32 k-rows span two scales (B lanes 0..31 hold k-rows 0..15, lanes
// 32..63 rows 16..31), so each step's B is used twice with the other half's
// lanes zeroed. Q6_K blocks are 210 bytes and start 2-byte aligned: pieces are
// loaded from the dword-aligned floor and re-aligned with alignbyte.

template <int FMT, int TN>
struct KB {
    static constexpr int TPR = FMT == F_Q4_K ? 2 : 4;    // threads per row and step
    static constexpr int BU = (TN * TPR + kThreads - 1) / kThreads;
    static constexpr int NW = FMT == F_Q4_K ? 8 : 12;     // dwords a thread loads per row and step
};

template <int TM, int TN>
struct KCfg {
    using C = Cfg<TM, TN>;
    static constexpr size_t BUF = sizeof(_Float16) * (2 * C::A_HALVES + C::B_HALVES) + sizeof(float) * TN * 4;
    static constexpr size_t LDS = 2 * BUF;
    static_assert(BUF % 16 == 0, "LDS buffer alignment");
};

template <int FMT, int TM, int TN>
struct KSrc {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t aoff[Cfg<TM, TN>::AP];
    uint32_t rowoff[KB<FMT, TN>::BU];   // byte offset of the thread's row in W, or kOutOfRange
};

template <int FMT, int TM, int TN>
struct KRegs {
    u32x4 a[Cfg<TM, TN>::AP];
    uint32_t b[KB<FMT, TN>::BU][KB<FMT, TN>::NW];
};

// Byte offsets of a Q6_K thread piece (row offset ro, step ks, 16-column group
// qd). d is read with a 16-bit load: the dword holding it may reach past the
// end of the matrix (a dword-aligned last block), where the range check would
// return zero.
struct Q6Piece {
    uint32_t ql, qh, sc, d;
};
__device__ inline Q6Piece q6_piece(uint32_t ro, int ks, int qd) {
    const uint32_t blk = ro + uint32_t(ks >> 2) * kQ6KBytes;
    const int h = (ks >> 1) & 1, kk = ks & 1;
    Q6Piece p;
    p.ql = blk + 64 * h + 16 * qd;
    p.qh = blk + 128 + 32 * h + 16 * (qd & 1);
    p.sc = blk + 192 + 8 * h + 4 * kk + qd;
    p.d = blk + 208;
    return p;
}

template <int FMT, int TM, int TN>
__device__ inline void kb_load(const KSrc<FMT, TM, TN> &g, int ks, KRegs<FMT, TM, TN> &r) {
    using B = KB<FMT, TN>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < B::BU; ++i) {
        const int part = (tid + i * kThreads) % B::TPR;
        const uint32_t ro = g.rowoff[i];
        uint32_t *w = r.b[i];
        if (FMT == F_Q4_K) {
            const uint32_t blk = ro + uint32_t(ks >> 2) * kQ4KBytes;
            const u32x4 hd = __builtin_amdgcn_raw_buffer_load_b128(g.rb, blk, 0, 0);
            const u32x4 qs = __builtin_amdgcn_raw_buffer_load_b128(g.rb, blk + 16 + 32 * (ks & 3) + 16 * part, 0, 0);
            w[0] = hd.x; w[1] = hd.y; w[2] = hd.z; w[3] = hd.w;
            w[4] = qs.x; w[5] = qs.y; w[6] = qs.z; w[7] = qs.w;
        } else {
            const Q6Piece p = q6_piece(ro, ks, part);
            const u32x4 l = __builtin_amdgcn_raw_buffer_load_b128(g.rb, p.ql & ~3u, 0, 0);
            const u32x4 h = __builtin_amdgcn_raw_buffer_load_b128(g.rb, p.qh & ~3u, 0, 0);
            w[0] = l.x; w[1] = l.y; w[2] = l.z; w[3] = l.w;
            w[4] = __builtin_amdgcn_raw_buffer_load_b32(g.rb, (p.ql & ~3u) + 16, 0, 0);
            w[5] = h.x; w[6] = h.y; w[7] = h.z; w[8] = h.w;
            w[9] = __builtin_amdgcn_raw_buffer_load_b32(g.rb, (p.qh & ~3u) + 16, 0, 0);
            w[10] = __builtin_amdgcn_raw_buffer_load_b32(g.rb, p.sc & ~3u, 0, 0);
            w[11] = __builtin_amdgcn_raw_buffer_load_b16(g.rb, p.d, 0, 0);   // 2-byte aligned; see q6_piece
        }
    }
}

// Four bytes (each 0..255) -> four f16 values 1024 + byte (two half2).
__device__ inline void bytes_to_half_biased(uint32_t w, half2v &lo, half2v &hi) {
    lo = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, w, 0x05010400u));
    hi = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, w, 0x07030602u));
}

// 16 small unsigned values (4 dwords of bytes) minus `bias` + 1024, as f16, to LDS.
__device__ inline void store16(const uint32_t *v, float bias, _Float16 *bq, int row, int col) {
    const half2v b = {static_cast<_Float16>(1024.0f + bias), static_cast<_Float16>(1024.0f + bias)};
    half2v o[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bytes_to_half_biased(v[k], o[2 * k], o[2 * k + 1]);
        o[2 * k] = o[2 * k] - b;
        o[2 * k + 1] = o[2 * k + 1] - b;
    }
    *reinterpret_cast<u32x4 *>(bq + lds_h(row, col)) =
        u32x4{__builtin_bit_cast(uint32_t, o[0]), __builtin_bit_cast(uint32_t, o[1]), __builtin_bit_cast(uint32_t, o[2]),
              __builtin_bit_cast(uint32_t, o[3])};
    *reinterpret_cast<u32x4 *>(bq + lds_h(row, col + 8)) =
        u32x4{__builtin_bit_cast(uint32_t, o[4]), __builtin_bit_cast(uint32_t, o[5]), __builtin_bit_cast(uint32_t, o[6]),
              __builtin_bit_cast(uint32_t, o[7])};
}

template <int FMT, int TM, int TN>
__device__ inline void kb_store(const KSrc<FMT, TM, TN> &g, int ks, const KRegs<FMT, TM, TN> &r, _Float16 *bq,
                                float *bd) {
    using B = KB<FMT, TN>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < B::BU; ++i) {
        const int u = tid + i * kThreads;
        if (B::BU * kThreads > TN * B::TPR && u >= TN * B::TPR) break;
        const int b = u / B::TPR, part = u % B::TPR;
        const uint32_t *w = r.b[i];
        if (FMT == F_Q4_K) {
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = w[4 + e] & 0x0f0f0f0fu;
                hi[e] = (w[4 + e] >> 4) & 0x0f0f0f0fu;
            }
            store16(lo, 0.f, bq, b, 16 * part);
            store16(hi, 0.f, bq, b, 32 + 16 * part);
            if (part == 0) {
                const int c = ks & 3;
                const float d = half_bits_to_float(w[0]), dmin = half_bits_to_float(w[0] >> 16);
                uint32_t s0, m0, s1, m1;
                q4k_scale_min(2 * c, w[1], w[2], w[3], s0, m0);
                q4k_scale_min(2 * c + 1, w[1], w[2], w[3], s1, m1);
                *reinterpret_cast<float4 *>(bd + b * 4) =
                    make_float4(d * float(s0), d * float(s1), dmin * float(m0), dmin * float(m1));
            }
        } else {
            const Q6Piece p = q6_piece(g.rowoff[i], ks, part);
            const uint32_t sh = p.ql & 3u;   // the block's misalignment (0 or 2), same for every piece
            const int kk = ks & 1;
            const uint32_t hshift = 2u * (2 * kk + (part >> 1));
            uint32_t q6[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t l = __builtin_amdgcn_alignbyte(w[e + 1], w[e], sh);
                const uint32_t h = __builtin_amdgcn_alignbyte(w[e + 6], w[e + 5], sh);
                const uint32_t nib = (kk ? (l >> 4) : l) & 0x0f0f0f0fu;
                q6[e] = nib | (((h >> hshift) & 0x03030303u) << 4);
            }
            store16(q6, 32.f, bq, b, 16 * part);
            const int scv = static_cast<int8_t>((w[10] >> (8 * (p.sc & 3u))) & 0xffu);
            const float d = half_bits_to_float(w[11]);
            bd[b * 4 + part] = d * float(scv);
        }
    }
}

template <int FMT, int EPI, int TM, int TN, bool A32>
__global__ __launch_bounds__(kThreads) void k_gemm_kq(GemmArgs a) {
    using C = Cfg<TM, TN>;
    using KC = KCfg<TM, TN>;
    using B = KB<FMT, TN>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int m0 = blockIdx.x * TM;
    const int row0 = blockIdx.y * TN;
    const int nvalid = min(TN, a.Nm[0] - row0);

    KSrc<FMT, TM, TN> src;
    a_setup<A32, TM, TN>(a, m0, src.ra, src.aoff);
    src.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(a.W[0]), 0,
                                               int(uint32_t(a.Nm[0]) * uint32_t(a.rowbytes)), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < B::BU; ++i) {
        const int u = tid + i * kThreads;
        const int b = u / B::TPR;
        src.rowoff[i] = (u < TN * B::TPR && b < nvalid) ? uint32_t(row0 + b) * uint32_t(a.rowbytes) : kOutOfRange;
    }

    f32x4 acc[C::MS][C::NS];
#pragma unroll
    for (int i = 0; i < C::MS; ++i)
#pragma unroll
        for (int j = 0; j < C::NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = a.K / GK;
    const bool resc = A32 ? false : tile_rescales<TM>(a, m0);
    RowFactors<TM, TN> rf;
    rf.load(a, m0, wm, lane);
    KRegs<FMT, TM, TN> regs;
    a_load<A32, TM, TN>(src.ra, src.aoff, 0, regs.a);
    kb_load<FMT, TM, TN>(src, 0, regs);
    const _Float16 one = static_cast<_Float16>(1.0f);
    const half8 ones = {one, one, one, one, one, one, one, one};
    const half8 zeros = {};
    for (int ks = 0; ks < nsteps; ++ks) {
        uint8_t *p = smem + size_t(ks & 1) * KC::BUF;
        _Float16 *ahi = reinterpret_cast<_Float16 *>(p), *alo = ahi + C::A_HALVES, *bq = alo + C::A_HALVES;
        float *bd = reinterpret_cast<float *>(bq + C::B_HALVES);
        a_store<A32, TM, TN>(regs.a, ahi, alo, a, m0, ks, resc);
        kb_store<FMT, TM, TN>(src, ks, regs, bq, bd);
        __syncthreads();
        if (ks + 1 < nsteps) {
            a_load<A32, TM, TN>(src.ra, src.aoff, ks + 1, regs.a);
            kb_load<FMT, TM, TN>(src, ks + 1, regs);
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            half8 bfr[C::NS], bfr1[C::NS];
            float s0[C::NS], s1[C::NS];
            const int fc = frag_col(hb, lane);
#pragma unroll
            for (int ns = 0; ns < C::NS; ++ns) {
                const int col = wn * C::WN + ns * 16 + (lane & 15);
                const half8 v = *reinterpret_cast<const half8 *>(bq + col * LPAD + fc);
                if (FMT == F_Q4_K) {
                    bfr[ns] = v;
                    s0[ns] = bd[col * 4 + hb];          // d * s
                    s1[ns] = -bd[col * 4 + 2 + hb];     // -dmin * m
                } else {
                    bfr[ns] = lane < 32 ? v : zeros;    // k-rows 0..15: scale 2hb
                    bfr1[ns] = lane < 32 ? zeros : v;   // k-rows 16..31: scale 2hb + 1
                    s0[ns] = bd[col * 4 + 2 * hb];
                    s1[ns] = bd[col * 4 + 2 * hb + 1];
                }
            }
#pragma unroll
            for (int ms = 0; ms < C::MS; ++ms) {
                const int row = wm * C::WM + ms * 16 + (lane & 15);
                const half8 ah = *reinterpret_cast<const half8 *>(ahi + row * LPAD + fc);
                const half8 al = *reinterpret_cast<const half8 *>(alo + row * LPAD + fc);
                if (FMT == F_Q4_K) {
                    f32x4 sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ones, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, ones, sx, 0, 0, 0);
#pragma unroll
                    for (int ns = 0; ns < C::NS; ++ns) {
                        f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bfr[ns], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        t = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bfr[ns], t, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[ms][ns][i] = fmaf(s0[ns], t[i], acc[ms][ns][i]);
                            acc[ms][ns][i] = fmaf(s1[ns], sx[i], acc[ms][ns][i]);
                        }
                    }
                } else {
#pragma unroll
                    for (int ns = 0; ns < C::NS; ++ns) {
                        f32x4 t0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bfr[ns], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        t0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bfr[ns], t0, 0, 0, 0);
                        f32x4 t1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bfr1[ns], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        t1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bfr1[ns], t1, 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[ms][ns][i] = fmaf(s0[ns], t0[i], acc[ms][ns][i]);
                            acc[ms][ns][i] = fmaf(s1[ns], t1[i], acc[ms][ns][i]);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < C::NS; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = wm * C::WM + ms * 16 + 4 * (lane >> 4) + i;
                const int c = wn * C::WN + ns * 16 + (lane & 15);
                if (m0 + m >= a.T || c >= nvalid) continue;
                float *dst = a.Y + size_t(m0 + m) * a.Nm[0] + row0 + c;
                const float v = acc[ms][ns][i] * rf.f[ms][i];
                *dst = (EPI == G_ACCUM) ? *dst + v : v;
            }
}

// u = x / sqrt(mean(x^2) + eps) * w for each token row, written as the f16
// hi plane [T][K] followed by the lo plane, each row multiplied first by the
// power of two 2^e that puts its largest |u| in [2^14, 2^15) (exact; the
// pair then holds every value with its 22 bits, however large or small the
// row); rs[row] = 2^-e for the products' epilogues (1 for a zero row). One
// workgroup per row. With splits > 0 the residual add of a split-K product
// happens here first: x += part[0] + part[1] + ... (that order), written back
// to x. With u NULL only that add is done. eg_zero (if set) is cleared for the
// row: the row exponent of planes a later kernel of the layer writes.
__global__ __launch_bounds__(kThreads) void k_rms_split(float *x, int T, int K, const float *w,
                                                        float eps, _Float16 *u, const float *part,
                                                        int splits, float *rs, int *eg_zero, int8_t *el_zero,
                                                        int el_n) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    float4 *xr = reinterpret_cast<float4 *>(x + row * K);
    const int n4 = K / 4;
    float ss = 0.f;
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        float4 v = xr[e];
        if (splits > 0) {
            const float4 *pr = reinterpret_cast<const float4 *>(part) + row * n4 + e;
            float4 p = pr[0];
            for (int z = 1; z < splits; ++z) {
                const float4 q = pr[size_t(z) * T * n4];
                p.x += q.x; p.y += q.y; p.z += q.z; p.w += q.w;
            }
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
            xr[e] = v;
        }
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    if (eg_zero && threadIdx.x == 0) eg_zero[row] = 0;
    if (el_zero)
        for (int b = threadIdx.x; b < el_n; b += kThreads) el_zero[row * el_n + b] = 0;
    if (!u) return;
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
    float mx = 0.f;
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        const float4 v = xr[e];
        const float4 g = reinterpret_cast<const float4 *>(w)[e];
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x * r * g.x), fabsf(v.y * r * g.y)),
                             fmaxf(fabsf(v.z * r * g.z), fabsf(v.w * r * g.w))));
    }
    mx = wave_max(mx);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int ex = (mx > 0.f && isfinite(mx)) ? min(max(14 - ilogbf(mx), -126), 126) : 0;
    if (rs && threadIdx.x == 0) rs[row] = ldexpf(1.0f, -ex);
    const size_t plane = size_t(T) * K;
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        const float4 v = xr[e];
        const float4 g = reinterpret_cast<const float4 *>(w)[e];
        const float vv[4] = {ldexpf(v.x * r * g.x, ex), ldexpf(v.y * r * g.y, ex), ldexpf(v.z * r * g.z, ex),
                             ldexpf(v.w * r * g.w, ex)};
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hi[k] = static_cast<_Float16>(vv[k]);
            lo[k] = static_cast<_Float16>(vv[k] - static_cast<float>(hi[k]));
        }
        *reinterpret_cast<uint2 *>(u + row * K + e * 4) = __builtin_bit_cast(uint2, hi);
        *reinterpret_cast<uint2 *>(u + plane + row * K + e * 4) = __builtin_bit_cast(uint2, lo);
    }
}

int row_tiles(int n, int tn) { return (n + tn - 1) / tn; }

// Tile choice: the large tile (64 x 128) when it gives at least 1.5
// workgroups per CU, otherwise the small one (32 x 64: short prompts, narrow
// matrices). Measured on the 7B-class 512-token prefill: a threshold of 256
// (o and down on large tiles, one workgroup per CU) gave 28.6 ms, 512 (qkv on
// small tiles too) 28.4 ms, 384 27.5 ms; 1024 also moved gate/up at 203
// tokens to small tiles (15.5 -> 17.3 ms for that prefill).
bool large_tiles(int T, int n_tiles_large) {
    return long((T + 63) / 64) * n_tiles_large >= 384;
}

// K steps of global loads in flight per workgroup: one when the grid fills
// the chip (more registers would cost occupancy), several when it is small
// (short prompts of small models: a few workgroups each walking all of K,
// where every step would otherwise wait a full memory round trip).
constexpr int kSmallGridStages = 4;

template <int FMT, int EPI, int TM, int TN, bool A32, int ST>
hipError_t launch_st(const GemmArgs &a, dim3 grid, hipStream_t s) {
    using C = Cfg<TM, TN>;
    constexpr size_t lds = C::lds(ST);
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_q8<FMT, EPI, TM, TN, A32, ST>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_gemm_q8<FMT, EPI, TM, TN, A32, ST>), grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

template <int EPI, int TM, int TN, bool A32, int FMT = F_Q8_0>
hipError_t launch_cfg(const GemmArgs &a, int ytiles, hipStream_t s) {
    // buffer resources address < 2 GiB (offsets past that read as zeros)
    if (size_t(a.T) * a.K * 4 >= kOutOfRange) return hipErrorInvalidValue;
    for (int i = 0; i < 3; ++i)
        if (a.W[i] && size_t(a.Nm[i]) * a.rowbytes >= kOutOfRange) return hipErrorInvalidValue;
    const dim3 grid((a.T + TM - 1) / TM, ytiles, EPI == G_PART ? a.splits : 1);
    if constexpr (TM == 32)
        if (long(grid.x) * grid.y * grid.z < 256)
            return launch_st<FMT, EPI, TM, TN, A32, kSmallGridStages>(a, grid, s);
    return launch_st<FMT, EPI, TM, TN, A32, 1>(a, grid, s);
}

template <int EPI, bool A32, int FMT = F_Q8_0>
hipError_t launch_plain(const GemmArgs &a, int N, hipStream_t s) {
    if (large_tiles(a.T, row_tiles(N, 128))) return launch_cfg<EPI, 64, 128, A32, FMT>(a, row_tiles(N, 128), s);
    return launch_cfg<EPI, 32, 64, A32, FMT>(a, row_tiles(N, 64), s);
}

template <int FMT, int EPI, int TM, int TN, bool A32>
hipError_t launch_kq_cfg(const GemmArgs &a, hipStream_t s) {
    using KC = KCfg<TM, TN>;
    if (size_t(a.T) * a.K * 4 >= kOutOfRange || size_t(a.Nm[0]) * a.rowbytes + 64 >= kOutOfRange)
        return hipErrorInvalidValue;
    if (KC::LDS > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_kq<FMT, EPI, TM, TN, A32>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(KC::LDS));
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.T + TM - 1) / TM, row_tiles(a.Nm[0], TN));
    hipLaunchKernelGGL((k_gemm_kq<FMT, EPI, TM, TN, A32>), grid, dim3(kThreads), KC::LDS, s, a);
    return hipGetLastError();
}

template <int FMT, int EPI, bool A32>
hipError_t launch_kq_plain(const GemmArgs &a, hipStream_t s) {
    if (large_tiles(a.T, row_tiles(a.Nm[0], 128))) return launch_kq_cfg<FMT, EPI, 64, 128, A32>(a, s);
    return launch_kq_cfg<FMT, EPI, 32, 64, A32>(a, s);
}

template <int FMT>
hipError_t launch_kq_fmt(const GemmArgs &a, bool a_split, int accumulate, hipStream_t s) {
    if (a_split)
        return accumulate ? launch_kq_plain<FMT, G_ACCUM, false>(a, s) : launch_kq_plain<FMT, G_STORE, false>(a, s);
    return accumulate ? launch_kq_plain<FMT, G_ACCUM, true>(a, s) : launch_kq_plain<FMT, G_STORE, true>(a, s);
}

GemmArgs gemm_base(const void *A, int T, int K, int fmt = F_Q8_0) {
    GemmArgs a{};
    a.A = A; a.T = T; a.K = K;
    a.rowbytes = int(fmt_row_bytes(fmt, K));
    return a;
}

bool pair_format(int fmt) { return fmt == F_Q8_0 || fmt == F_Q5_0; }

}  // namespace

hipError_t launch_rms_split(float *x, int T, int K, const float *w, float eps, _Float16 *u,
                            const float *part, int splits, hipStream_t s, float *rs, int *eg_zero, int8_t *el_zero,
                            int el_n) {
    hipLaunchKernelGGL(k_rms_split, dim3(T), dim3(kThreads), 0, s, x, T, K, w, eps, u, part, splits, rs, eg_zero,
                       el_zero, el_n);
    return hipGetLastError();
}

// Split-K applies while the plain 32 x 64 grid has fewer than kSplitKWgs
// workgroups. The slices bring it to about 256 workgroups (512 for rows of
// 4096 weights or more, whose K walk is long), at least 2 slices, at most 8.
// Measured at the 135M shape (K = 576 / 1536) and the 7B-class one
// (K = 4096 / 14336) for prompts of 13 to 1024 tokens.
constexpr int kSplitKWgs = 512;

int gemm_splitk_max_tokens(int N) {
    return std::min(kSplitKMaxTokens, 32 * ((kSplitKWgs - 1) / row_tiles(N, 64)));
}

// Wide matrices (N >= 2048) past 64 tokens (two tile rows) whose 64 x 128 grid is
// still short of the large-tile threshold: large tiles split over K instead
// of small tiles (their LDS traffic per MFMA is half), 2 to 8 slices towards
// kSplitKWgs workgroups, as many as the partials buffer holds.
bool splitk_large(int N, int T) { return N >= 2048 && T > 64 && !large_tiles(T, row_tiles(N, 128)); }

int gemm_splitk(int N, int K, int T) {
    if (splitk_large(N, T)) {
        const long wgs = long(row_tiles(T, 64)) * row_tiles(N, 128);
        const long want = std::max(2L, (kSplitKWgs + wgs - 1) / wgs);
        const long fit = long(kSplitKMax) * gemm_splitk_max_tokens(N) / T;
        const long sk = std::min<long>({want, long(kSplitKMax), long(K / GK), fit});
        return sk >= 2 ? int(sk) : 1;
    }
    if (T > gemm_splitk_max_tokens(N)) return 1;
    const long wgs = long(row_tiles(T, 32)) * row_tiles(N, 64);
    if (wgs >= kSplitKWgs || large_tiles(T, row_tiles(N, 128))) return 1;
    const long target = K >= 4096 ? 512 : 256;
    const long want = std::max(2L, (target + wgs - 1) / wgs);
    return int(std::max(1L, std::min<long>({want, long(kSplitKMax), long(K / GK)})));
}

hipError_t launch_gemm_part(const uint8_t *W, int N, int K, const _Float16 *A, int T, int splits, float *part,
                            hipStream_t s, const ActScale &sc, int fmt) {
    // (the partials part[splits][T][N] must fit the buffer sized for
    // kSplitKMax slices of gemm_splitk_max_tokens(N) rows)
    if (splits < 1 || splits > kSplitKMax || splits > K / GK ||
        long(splits) * T > long(kSplitKMax) * gemm_splitk_max_tokens(N) || !pair_format(fmt))
        return hipErrorInvalidValue;
    GemmArgs a = gemm_base(A, T, K, fmt);
    a.W[0] = W; a.Nm[0] = N; a.part = part; a.splits = splits; a.sc = sc;
    if (splitk_large(N, T))
        return fmt == F_Q5_0 ? launch_cfg<G_PART, 64, 128, false, F_Q5_0>(a, row_tiles(N, 128), s)
                             : launch_cfg<G_PART, 64, 128, false>(a, row_tiles(N, 128), s);
    return fmt == F_Q5_0 ? launch_cfg<G_PART, 32, 64, false, F_Q5_0>(a, row_tiles(N, 64), s)
                         : launch_cfg<G_PART, 32, 64, false>(a, row_tiles(N, 64), s);
}

hipError_t launch_gemm_matmul(const uint8_t *W, int N, int K, const void *A, bool a_split, int T,
                              int accumulate, float *Y, hipStream_t s, const ActScale &sc, int fmt) {
    if (!pair_format(fmt)) return hipErrorInvalidValue;
    GemmArgs a = gemm_base(A, T, K, fmt);
    a.W[0] = W; a.Nm[0] = N; a.Y = Y; a.sc = sc;
    if (fmt == F_Q5_0) {
        if (a_split)
            return accumulate ? launch_plain<G_ACCUM, false, F_Q5_0>(a, N, s)
                              : launch_plain<G_STORE, false, F_Q5_0>(a, N, s);
        return accumulate ? launch_plain<G_ACCUM, true, F_Q5_0>(a, N, s) : launch_plain<G_STORE, true, F_Q5_0>(a, N, s);
    }
    if (a_split)
        return accumulate ? launch_plain<G_ACCUM, false>(a, N, s) : launch_plain<G_STORE, false>(a, N, s);
    return accumulate ? launch_plain<G_ACCUM, true>(a, N, s) : launch_plain<G_STORE, true>(a, N, s);
}

hipError_t launch_gemm_kq(int fmt, const uint8_t *W, int N, int K, const void *A, bool a_split, int T,
                          int accumulate, float *Y, hipStream_t s, const ActScale &sc) {
    if (K % kQKK || (fmt != F_Q4_K && fmt != F_Q6_K)) return hipErrorInvalidValue;
    GemmArgs a{};
    a.A = A; a.T = T; a.K = K; a.sc = sc;
    a.rowbytes = int(fmt_row_bytes(fmt, K));
    a.W[0] = W; a.Nm[0] = N; a.Y = Y;
    return fmt == F_Q4_K ? launch_kq_fmt<F_Q4_K>(a, a_split, accumulate, s)
                         : launch_kq_fmt<F_Q6_K>(a, a_split, accumulate, s);
}

constexpr long kQkvLargeWgs = 512;   // (768 measured slower at 700 and 900 tokens)

template <int FMT>
hipError_t launch_qkv_fmt(const GemmArgs &a, int tiles, int yt, hipStream_t s) {
    if (tiles == 2) return launch_cfg<G_QKV, 64, 128, false, FMT>(a, yt, s);
    if (tiles == 1) return launch_cfg<G_QKV, 64, 64, false, FMT>(a, yt, s);
    return launch_cfg<G_QKV, 32, 64, false, FMT>(a, yt, s);
}

// q, k and v in one launch when they share a block format; otherwise one
// launch per run of matrices of one format (the other matrices get no row
// tiles, so the kernel's tile -> matrix walk skips them).
hipError_t launch_gemm_qkv(const Dims &d, const LayerPtrs &w, const _Float16 *u, const StepState *st,
                           const float2 *rope, float *q, float *kc, float *vc, int T, hipStream_t s,
                           const ActScale &sc) {
    const int QD = d.nh * d.hd, KVD = d.nkv * d.hd;
    const int fm[3] = {w.fq, w.fk, w.fv};
    for (int i = 0; i < 3; ++i)
        if (!pair_format(fm[i])) return hipErrorInvalidValue;
    const int n128 = row_tiles(QD, 128) + 2 * row_tiles(KVD, 128);
    // 64 x 128 tiles from 2 workgroups per CU; 64 x 64 between the
    // large-tile threshold and that
    const int tiles = !large_tiles(T, n128) ? 0 : long((T + 63) / 64) * n128 >= kQkvLargeWgs ? 2 : 1;
    const int tn = tiles == 2 ? 128 : 64;
    for (int first = 0; first < 3;) {
        int last = first;
        while (last + 1 < 3 && fm[last + 1] == fm[first]) ++last;
        GemmArgs a = gemm_base(u, T, d.H, fm[first]);
        a.sc = sc;
        a.W[0] = w.wq; a.W[1] = w.wk; a.W[2] = w.wv;
        a.Nm[0] = QD; a.Nm[1] = KVD; a.Nm[2] = KVD;
        a.st = st; a.rope = rope; a.q = q; a.kc = kc; a.vc = vc;
        a.QD = QD; a.hd = d.hd; a.max_seq = d.max_seq; a.rope_neox = d.rope_neox;
        int yt = 0;
        for (int i = 0; i < 3; ++i) {
            a.tiles[i] = (i >= first && i <= last) ? row_tiles(a.Nm[i], tn) : 0;
            if (!a.tiles[i]) a.W[i] = nullptr;
            yt += a.tiles[i];
        }
        const hipError_t e = fm[first] == F_Q5_0 ? launch_qkv_fmt<F_Q5_0>(a, tiles, yt, s)
                                                 : launch_qkv_fmt<F_Q8_0>(a, tiles, yt, s);
        if (e != hipSuccess) return e;
        first = last + 1;
    }
    return hipSuccess;
}

template <int FMT>
hipError_t launch_gateup_fmt(const GemmArgs &a, hipStream_t s) {
    const int F = a.Nm[0];
    if (large_tiles(a.T, row_tiles(F, 64))) return launch_cfg<G_GATEUP, 64, 128, false, FMT>(a, row_tiles(F, 64), s);
    return launch_cfg<G_GATEUP, 32, 64, false, FMT>(a, row_tiles(F, 32), s);
}

hipError_t launch_gemm_gateup(const Dims &d, const LayerPtrs &w, const _Float16 *u, _Float16 *h, int T,
                              hipStream_t s, const ActScale &sc) {
    if (!pair_format(w.fg) || w.fu != w.fg) return hipErrorInvalidValue;
    GemmArgs a = gemm_base(u, T, d.H, w.fg);
    a.sc = sc;
    a.W[0] = w.wg; a.W[1] = w.wu; a.Nm[0] = d.F; a.Nm[1] = d.F; a.h = h;
    return w.fg == F_Q5_0 ? launch_gateup_fmt<F_Q5_0>(a, s) : launch_gateup_fmt<F_Q8_0>(a, s);
}

}  // namespace q8l

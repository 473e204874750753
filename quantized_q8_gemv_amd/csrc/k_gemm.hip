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
constexpr int LPAD = 72;   // halves per LDS row (64 + 8)

enum GemmEpi { G_STORE = 0, G_ACCUM = 1, G_QKV = 2, G_GATEUP = 3 };

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
    static constexpr size_t LDS = 2 * BUF;
    static constexpr int STAGES = 1;                     // K steps of global loads in flight
    static_assert(AP >= 1 && BU >= 1 && MS >= 1 && NS >= 1, "tile too small");
    static_assert(BUF % 16 == 0, "LDS buffer alignment");
    static_assert(size_t(TM) * WN * sizeof(float) <= LDS, "gate/up exchange fits");
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

// Registers holding one K step of global data in flight.
template <int TM, int TN>
struct GRegs {
    u32x4 a[Cfg<TM, TN>::AP];
    uint32_t b[Cfg<TM, TN>::BU][5];
};

// Quarter qd of a 68-byte block pair (dwords): 0 -> d0 + q0..15 of block 0
// (dwords 0..4), 1 -> q16..31 + d1 (4..8), 2 -> q0..15 of block 1 (9..13, the
// last unused), 3 -> q16..31 of block 1 (12..16, the first unused).
__device__ inline int quarter_base(int qd) { return qd == 0 ? 0 : qd == 1 ? 4 : qd == 2 ? 9 : 12; }

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

template <bool A32, int TM, int TN, int EPI>
__device__ inline void g_setup(const GemmArgs &a, int m0, int row0, const int nvalid[2],
                               const uint8_t *const Wb[2], GSrc<TM, TN> &g) {
    using C = Cfg<TM, TN>;
    const int tid = threadIdx.x;
    const uint32_t abytes = uint32_t(size_t(a.T) * a.K * 4);  // f32, or two f16 planes
    g.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.A), 0, int(abytes), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int c = tid + i * kThreads;
        if (A32) {
            const int m = c >> 4;
            g.aoff[i] = m0 + m < a.T ? uint32_t((size_t(m0 + m) * a.K + (c & 15) * 4) * 4) : kOutOfRange;
        } else {
            const int plane = c / (TM * 8), rr = c - plane * (TM * 8);
            const int m = rr >> 3;
            g.aoff[i] = m0 + m < a.T
                            ? uint32_t((size_t(plane) * a.T * a.K + size_t(m0 + m) * a.K + (rr & 7) * 8) * 2)
                            : kOutOfRange;
        }
    }
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
        g.boff[i] = rr < nvalid[part] ? uint32_t(row0 + rr) * uint32_t(a.rowbytes) + quarter_base(qd) * 4
                                      : kOutOfRange;
    }
}

template <bool A32, int TM, int TN>
__device__ inline void g_load(const GSrc<TM, TN> &g, int ks, GRegs<TM, TN> &r) {
    using C = Cfg<TM, TN>;
    const int sa = ks * GK * (A32 ? 4 : 2);
    const int sb = ks * kPairBytes;
#pragma unroll
    for (int i = 0; i < C::AP; ++i) r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(g.ra, g.aoff[i], sa, 0);
#pragma unroll
    for (int i = 0; i < C::BU; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(g.rb[i], g.boff[i], sb, 0);
        r.b[i][0] = v.x;
        r.b[i][1] = v.y;
        r.b[i][2] = v.z;
        r.b[i][3] = v.w;
        r.b[i][4] = __builtin_amdgcn_raw_buffer_load_b32(g.rb[i], g.boff[i] + 16, sb, 0);
    }
}

// int8 x 4 (one dword) -> 4 exact f16 values: bias each byte to an unsigned
// value u = q + 128, place it in the mantissa of 1024.0 (f16 bits 0x6400 | u)
// and subtract 1152 = 1024 + 128.
__device__ inline void q4_to_half(uint32_t w, half2v &lo, half2v &hi) {
    const uint32_t x = w ^ 0x80808080u;
    const uint32_t l = __builtin_amdgcn_perm(0x64646464u, x, 0x05010400u);
    const uint32_t h = __builtin_amdgcn_perm(0x64646464u, x, 0x07030602u);
    const half2v bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
    lo = __builtin_bit_cast(half2v, l) - bias;
    hi = __builtin_bit_cast(half2v, h) - bias;
}

template <bool A32, int TM, int TN>
__device__ inline void g_store(const GRegs<TM, TN> &r, const GBuf &bf) {
    using C = Cfg<TM, TN>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::AP; ++i) {
        const int c = tid + i * kThreads;
        if (A32) {
            const int m = c >> 4, c4 = c & 15;
            const float4 v = __builtin_bit_cast(float4, r.a[i]);
            const float vv[4] = {v.x, v.y, v.z, v.w};
            _Float16 hi[4], lo[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                hi[k] = static_cast<_Float16>(vv[k]);
                lo[k] = static_cast<_Float16>(vv[k] - static_cast<float>(hi[k]));
            }
            *reinterpret_cast<uint2 *>(bf.ahi + m * LPAD + c4 * 4) = __builtin_bit_cast(uint2, hi);
            *reinterpret_cast<uint2 *>(bf.alo + m * LPAD + c4 * 4) = __builtin_bit_cast(uint2, lo);
        } else {
            const int plane = c / (TM * 8), rr = c - plane * (TM * 8);
            const int m = rr >> 3, p = rr & 7;
            *reinterpret_cast<u32x4 *>((plane ? bf.alo : bf.ahi) + m * LPAD + p * 8) = r.a[i];
        }
    }
#pragma unroll
    for (int i = 0; i < C::BU; ++i) {
        const int u = tid + i * kThreads;
        const int b = u >> 2, qd = u & 3;
        const uint32_t *w = r.b[i];
        const uint32_t shift = qd < 2 ? 2u : 0u;
        half2v v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t q4 = qd == 3 ? w[k + 1] : __builtin_amdgcn_alignbyte(w[k + 1], w[k], shift);
            q4_to_half(q4, v[2 * k], v[2 * k + 1]);
        }
        const u32x4 s0 = u32x4{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                               __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
        const u32x4 s1 = u32x4{__builtin_bit_cast(uint32_t, v[4]), __builtin_bit_cast(uint32_t, v[5]),
                               __builtin_bit_cast(uint32_t, v[6]), __builtin_bit_cast(uint32_t, v[7])};
        _Float16 *dst = bf.bq + b * LPAD + (qd >> 1) * 32 + (qd & 1) * 16;
        *reinterpret_cast<u32x4 *>(dst) = s0;
        *reinterpret_cast<u32x4 *>(dst + 8) = s1;
        if (qd == 0) bf.bd[b * 2 + 0] = half_bits_to_float(w[0] & 0xffffu);
        if (qd == 1) bf.bd[b * 2 + 1] = half_bits_to_float(w[4] >> 16);
    }
}

template <int EPI, int TM, int TN, bool A32>
__global__ __launch_bounds__(kThreads) void k_gemm_q8(GemmArgs a) {
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

    // S register stages: the loads of steps ks+1 .. ks+S-1 are in flight while
    // step ks is computed (the loop is unrolled by S so each stage is a fixed
    // set of registers).
    constexpr int S = C::STAGES;
    const int nsteps = a.K / GK;
    GSrc<TM, TN> src;
    g_setup<A32, TM, TN, EPI>(a, m0, row0, nvalid, Wb, src);
    GRegs<TM, TN> regs[S];
#pragma unroll
    for (int j = 0; j < S; ++j)
        if (j < nsteps) g_load<A32, TM, TN>(src, j, regs[j]);
    for (int k0 = 0; k0 < nsteps; k0 += S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const int ks = k0 + j;
            if (ks >= nsteps) break;
            const GBuf bf = gbuf<TM, TN>(smem, ks & 1);
            g_store<A32, TM, TN>(regs[j], bf);
            __syncthreads();
            if (ks + S < nsteps) g_load<A32, TM, TN>(src, ks + S, regs[j]);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                half8 bfr[C::NS];
                float dsc[C::NS];
#pragma unroll
                for (int ns = 0; ns < C::NS; ++ns) {
                    const int col = wn * C::WN + ns * 16 + (lane & 15);
                    bfr[ns] = *reinterpret_cast<const half8 *>(bf.bq + col * LPAD + hb * 32 + 8 * (lane >> 4));
                    dsc[ns] = bf.bd[col * 2 + hb];
                }
#pragma unroll
                for (int ms = 0; ms < C::MS; ++ms) {
                    const int row = wm * C::WM + ms * 16 + (lane & 15);
                    const half8 ah = *reinterpret_cast<const half8 *>(bf.ahi + row * LPAD + hb * 32 + 8 * (lane >> 4));
                    const half8 al = *reinterpret_cast<const half8 *>(bf.alo + row * LPAD + hb * 32 + 8 * (lane >> 4));
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
            const size_t plane = size_t(a.T) * a.Nm[0];
#pragma unroll
            for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
                for (int ns = 0; ns < C::NS; ++ns)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = wm * C::WM + ms * 16 + 4 * (lane >> 4) + i;
                        const int c = ns * 16 + (lane & 15);
                        if (m0 + m < a.T && c < nvalid[0]) {
                            const float g = acc[ms][ns][i], u = ub[m * C::WN + c];
                            store_hilo(a.h, plane, size_t(m0 + m) * a.Nm[0] + row0 + c, silu(g) * u);
                        }
                    }
        }
        return;
    }
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < C::NS; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = wm * C::WM + ms * 16 + 4 * (lane >> 4) + i;
                const int c = wn * C::WN + ns * 16 + (lane & 15);
                const float v = acc[ms][ns][i];
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
                        *dst = v;
                    } else {
                        const float2 cs = a.rope[size_t(a.st->pos + t) * (a.hd / 2) + (d >> 1)];
                        const float r = (d & 1) ? (partner * cs.y + v * cs.x) : (v * cs.x - partner * cs.y);
                        if (mat == 0)
                            a.q[size_t(t) * a.QD + row] = r;
                        else
                            a.kc[(size_t(row / a.hd) * a.max_seq + a.st->slot + t) * a.hd + d] = r;
                    }
                } else {
                    if (m0 + m >= a.T || c >= nvalid[0]) continue;
                    float *dst = a.Y + size_t(m0 + m) * a.Nm[0] + row0 + c;
                    *dst = (EPI == G_ACCUM) ? *dst + v : v;
                }
            }
}

// u = x / sqrt(mean(x^2) + eps) * w for each token row, written as the f16
// hi plane [T][K] followed by the lo plane. One workgroup per row.
__global__ __launch_bounds__(kThreads) void k_rms_split(const float *x, int T, int K, const float *w,
                                                        float eps, _Float16 *u) {
    __shared__ float red[4];
    const size_t row = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + row * K);
    const int n4 = K / 4;
    float ss = 0.f;
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        const float4 v = xr[e];
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
    const size_t plane = size_t(T) * K;
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        const float4 v = xr[e];
        const float4 g = reinterpret_cast<const float4 *>(w)[e];
        const float vv[4] = {v.x * r * g.x, v.y * r * g.y, v.z * r * g.z, v.w * r * g.w};
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

// Tile choice: the large tile (64 x 128) when it still gives every CU a
// workgroup, otherwise the small one (32 x 64: short prompts, narrow matrices).
bool large_tiles(int T, int n_tiles_large) {
    return long((T + 63) / 64) * n_tiles_large >= 256;
}

template <int EPI, int TM, int TN, bool A32>
hipError_t launch_cfg(const GemmArgs &a, int ytiles, hipStream_t s) {
    using C = Cfg<TM, TN>;
    // buffer resources address < 2 GiB (offsets past that read as zeros)
    if (size_t(a.T) * a.K * 4 >= kOutOfRange) return hipErrorInvalidValue;
    for (int i = 0; i < 3; ++i)
        if (a.W[i] && size_t(a.Nm[i]) * a.rowbytes >= kOutOfRange) return hipErrorInvalidValue;
    if (C::LDS > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_q8<EPI, TM, TN, A32>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(C::LDS));
        if (e != hipSuccess) return e;
    }
    dim3 grid((a.T + TM - 1) / TM, ytiles);
    hipLaunchKernelGGL((k_gemm_q8<EPI, TM, TN, A32>), grid, dim3(kThreads), C::LDS, s, a);
    return hipGetLastError();
}

template <int EPI, bool A32>
hipError_t launch_plain(const GemmArgs &a, int N, hipStream_t s) {
    if (large_tiles(a.T, row_tiles(N, 128))) return launch_cfg<EPI, 64, 128, A32>(a, row_tiles(N, 128), s);
    return launch_cfg<EPI, 32, 64, A32>(a, row_tiles(N, 64), s);
}

GemmArgs gemm_base(const void *A, int T, int K) {
    GemmArgs a{};
    a.A = A; a.T = T; a.K = K;
    a.rowbytes = K / kQK * kQBytes;
    return a;
}

}  // namespace

hipError_t launch_rms_split(const float *x, int T, int K, const float *w, float eps, _Float16 *u,
                            hipStream_t s) {
    hipLaunchKernelGGL(k_rms_split, dim3(T), dim3(kThreads), 0, s, x, T, K, w, eps, u);
    return hipGetLastError();
}

hipError_t launch_gemm_matmul(const uint8_t *W, int N, int K, const void *A, bool a_split, int T,
                              int accumulate, float *Y, hipStream_t s) {
    GemmArgs a = gemm_base(A, T, K);
    a.W[0] = W; a.Nm[0] = N; a.Y = Y;
    if (a_split)
        return accumulate ? launch_plain<G_ACCUM, false>(a, N, s) : launch_plain<G_STORE, false>(a, N, s);
    return accumulate ? launch_plain<G_ACCUM, true>(a, N, s) : launch_plain<G_STORE, true>(a, N, s);
}

hipError_t launch_gemm_qkv(const Dims &d, const LayerPtrs &w, const _Float16 *u, const StepState *st,
                           const float2 *rope, float *q, float *kc, float *vc, int T, hipStream_t s) {
    GemmArgs a = gemm_base(u, T, d.H);
    const int QD = d.nh * d.hd, KVD = d.nkv * d.hd;
    a.W[0] = w.wq; a.W[1] = w.wk; a.W[2] = w.wv;
    a.Nm[0] = QD; a.Nm[1] = KVD; a.Nm[2] = KVD;
    a.st = st; a.rope = rope; a.q = q; a.kc = kc; a.vc = vc;
    a.QD = QD; a.hd = d.hd; a.max_seq = d.max_seq; a.rope_neox = d.rope_neox;
    const bool large = large_tiles(T, row_tiles(QD, 128) + 2 * row_tiles(KVD, 128));
    const int tn = large ? 128 : 64;
    for (int i = 0; i < 3; ++i) a.tiles[i] = row_tiles(a.Nm[i], tn);
    const int yt = a.tiles[0] + a.tiles[1] + a.tiles[2];
    return large ? launch_cfg<G_QKV, 64, 128, false>(a, yt, s) : launch_cfg<G_QKV, 32, 64, false>(a, yt, s);
}

hipError_t launch_gemm_gateup(const Dims &d, const LayerPtrs &w, const _Float16 *u, _Float16 *h, int T,
                              hipStream_t s) {
    GemmArgs a = gemm_base(u, T, d.H);
    a.W[0] = w.wg; a.W[1] = w.wu; a.Nm[0] = d.F; a.Nm[1] = d.F; a.h = h;
    if (large_tiles(T, row_tiles(d.F, 64))) return launch_cfg<G_GATEUP, 64, 128, false>(a, row_tiles(d.F, 64), s);
    return launch_cfg<G_GATEUP, 32, 64, false>(a, row_tiles(d.F, 32), s);
}

}  // namespace q8l

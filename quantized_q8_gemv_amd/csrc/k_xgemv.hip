// k_xgemv.hip -- single-token products for rows of 2048 to 4096 weights (32
// to 64 pairs), and for longer rows in 2 or 4 slices, one wave per row.
//
// Lane l of a wave takes pair l (64 weights: 68 bytes of Q8_0 or 44 of Q5_0)
// of every row it computes, read with 16-byte loads, and keeps the pair's 64
// activations in registers for the whole kernel: the 64 lanes hold the whole
// activation row. The workgroup stages that row once in LDS (with the
// RMSNorm in front where the product has one), each lane takes its 64
// values, and from then on every wave works alone: it walks its rows (row r,
// r + waves, ...) with the next D rows' weights in flight while one is
// computed; the weights of its first rows are requested before the
// activation row is read. Compared with staging weight tiles through LDS,
// there are no barriers in the row loop and no activation reads from LDS per
// pair.
//
// Arithmetic per row: lane l's pair product d_A * s_A + d_B * s_B (each block
// sum in four interleaved partial sums, as the other GEMVs), then the 64
// lanes summed by wave_sum_dpp. Rows longer than 64 pairs (the down
// projection of 7B-class models) are cut into S = 2 or 4 slices of at most
// 64 pairs, taken by S waves of one workgroup; their sums meet in LDS and are
// added in slice order.
//
// Output rows shorter than 32 pairs take the same per-lane pair layout with
// several rows per wave (k_xlmhead_short). Used for the o, gate/up, down and
// output products of a decode step. The
// q/k/v product stays on the LDS-staged kernel, which measured faster at the
// 7B-class shape (10.0 us against 11.1 for a version of this design with the
// rope and cache-write epilogue).

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int kWavesX = kThreads / 64;
constexpr uint32_t kNoRow = 0x80000000u;  // a buffer offset past every resource: the load returns zeros
constexpr int kXRows = 32;                // rows one wave computes at most (slice sums kept in LDS)

template <int FMT>
struct LPair {
    uint32_t w[FMT == F_Q5_0 ? 11 : 17];
};

template <int FMT>
constexpr uint32_t lp_bytes() { return FMT == F_Q5_0 ? kQ5PairBytes : kPairBytes; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint8_t *W, int N, uint32_t rowbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(W), 0, int(uint32_t(N) * rowbytes),
                                             0x00020000);
}

template <int FMT>
__device__ __forceinline__ void lp_load(__amdgpu_buffer_rsrc_t rs, uint32_t off, LPair<FMT> &o) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0);
    o.w[0] = a.x; o.w[1] = a.y; o.w[2] = a.z; o.w[3] = a.w;
    o.w[4] = b.x; o.w[5] = b.y; o.w[6] = b.z; o.w[7] = b.w;
    if constexpr (FMT == F_Q5_0) {
        const u32x3 c = __builtin_amdgcn_raw_buffer_load_b96(rs, off + 32, 0, 0);
        o.w[8] = c.x; o.w[9] = c.y; o.w[10] = c.z;
    } else {
        const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32, 0, 0);
        const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 48, 0, 0);
        o.w[8] = c.x; o.w[9] = c.y; o.w[10] = c.z; o.w[11] = c.w;
        o.w[12] = d.x; o.w[13] = d.y; o.w[14] = d.z; o.w[15] = d.w;
        o.w[16] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 64, 0, 0);
    }
}

// The lane's activations: its pair's 64 values and, for Q5_0 rows, their two
// block sums (taken once; see xpair_dot_q5s).
struct XAct {
    float v[64];
    float sA, sB;
    __device__ __forceinline__ void sums() {
        sA = sB = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            sA += v[i];
            sB += v[32 + i];
        }
    }
};

template <int FMT>
__device__ __forceinline__ float lp_dot(const LPair<FMT> &p, const XAct &x) {
    if constexpr (FMT == F_Q5_0)
        return xpair_dot_q5s(p.w, x.v, x.sA, x.sB);
    else
        return xpair_dot_q8(p.w, x.v);
}

// The 64 activations of pair p (x[64 p + i]); zeros when !on. The loads are
// unconditional (a clamped pair) so that none is sunk into a branch.
__device__ __forceinline__ void xl_load(const float *x, int p, bool on, float (&v)[64]) {
    const f32x4 *src = reinterpret_cast<const f32x4 *>(x + size_t(on ? p : 0) * kPairWeights);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f32x4 t = src[i];
        v[4 * i] = on ? t.x : 0.f;
        v[4 * i + 1] = on ? t.y : 0.f;
        v[4 * i + 2] = on ? t.z : 0.f;
        v[4 * i + 3] = on ? t.w : 0.f;
    }
}

// The activation row staged once per workgroup: its 256 threads read the row
// (f32 x, or the token's Q8_0 embedding row dequantized as d * q; workgroup
// 0 then writes that row to xres) with coalesced 16-byte loads, take the
// RMSNorm when norm_w is set (sum of squares per thread in element order,
// then the waves in order), and leave u in LDS; each lane then reads the 64
// values of pair `pair` (zeros when !on). One read of the row per workgroup
// instead of per wave.
constexpr int kXPad = 68;  // floats per staged pair (the pair stride spreads the lanes over the LDS banks)

struct XStage {
    float u[64 * kXPad];
    float red[kWavesX];
};

// The 64 staged values of pair p (zeros when !on).
__device__ __forceinline__ void xl_take(const XStage &L, int p, bool on, float (&v)[64]) {
    const f32x4 *src = reinterpret_cast<const f32x4 *>(L.u + (on ? p : 0) * kXPad);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const f32x4 t = src[i];
        v[4 * i] = on ? t.x : 0.f;
        v[4 * i + 1] = on ? t.y : 0.f;
        v[4 * i + 2] = on ? t.z : 0.f;
        v[4 * i + 3] = on ? t.w : 0.f;
    }
}

__device__ __forceinline__ void xl_stage(XStage &L, const float *x, const uint8_t *erow, bool evalid, float *xres,
                                         const float *norm_w, int P, float eps, float (&v)[64], int pair, bool on) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n4 = P * 16;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid + i * kThreads;
        if (e < n4) {
            f32x4 t;
            if (erow) {
                const uint8_t *blk = erow + size_t(e >> 3) * kQBytes;   // 8 float4 per 32-weight block
                const int i0 = 2 + (e & 7) * 4;
                const float d = half_bits_to_float(uint32_t(blk[0]) | (uint32_t(blk[1]) << 8));
                t.x = evalid ? d * static_cast<float>(static_cast<int8_t>(blk[i0])) : 0.f;
                t.y = evalid ? d * static_cast<float>(static_cast<int8_t>(blk[i0 + 1])) : 0.f;
                t.z = evalid ? d * static_cast<float>(static_cast<int8_t>(blk[i0 + 2])) : 0.f;
                t.w = evalid ? d * static_cast<float>(static_cast<int8_t>(blk[i0 + 3])) : 0.f;
                if (xres && blockIdx.x == 0) reinterpret_cast<f32x4 *>(xres)[e] = t;
            } else {
                t = reinterpret_cast<const f32x4 *>(x)[e];
            }
            ss = fmaf(t.x, t.x, ss);
            ss = fmaf(t.y, t.y, ss);
            ss = fmaf(t.z, t.z, ss);
            ss = fmaf(t.w, t.w, ss);
            *reinterpret_cast<f32x4 *>(L.u + (e >> 4) * kXPad + (e & 15) * 4) = t;
        }
    }
    if (norm_w) {
        ss = wave_sum_dpp(ss);
        if (lane == 0) L.red[wv] = ss;
        __syncthreads();
        const float tot = (L.red[0] + L.red[1]) + (L.red[2] + L.red[3]);
        const float r = 1.0f / sqrtf(tot / static_cast<float>(P * kPairWeights) + eps);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * kThreads;
            if (e < n4) {
                f32x4 *up = reinterpret_cast<f32x4 *>(L.u + (e >> 4) * kXPad + (e & 15) * 4);
                const f32x4 w = reinterpret_cast<const f32x4 *>(norm_w)[e];
                f32x4 t = *up;
                t.x = t.x * r * w.x;
                t.y = t.y * r * w.y;
                t.z = t.z * r * w.z;
                t.w = t.w * r * w.w;
                *up = t;
            }
        }
    }
    __syncthreads();
    xl_take(L, pair, on, v);
}

// ---------------------------------------------------------------- o, down, op

struct XMatmulArgs {
    const uint8_t *W;
    const float *x;  // [K]
    float *y;        // [N]
    int N, P, accumulate;
};

// S waves of a workgroup per row (slice s = wave % S holds pairs s * SP ..
// s * SP + SP - 1, SP = ceil(P / S)); 4 / S row groups per workgroup. Rows
// in flight per wave: 2 for whole rows (short kernels, where the first
// rows' latency is most of the time), 1 for sliced ones (measured on the
// 7B-class o and down projections).
template <int FMT, int S>
__device__ __forceinline__ void xmatmul_body(XMatmulArgs a) {
    constexpr int D = S == 1 ? 2 : 1, GW = 4 / S;
    __shared__ float red[4][kXRows];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int gi = wv / S, sl = wv % S;
    const int ng = int(gridDim.x) * GW;       // row groups in the grid
    const int g = int(blockIdx.x) * GW + gi;  // this wave's group: rows g, g + ng, ...
    const int SP = (a.P + S - 1) / S;
    const int p = sl * SP + lane;
    const bool on = lane < SP && p < a.P;
    const uint32_t rowbytes = uint32_t(a.P) * lp_bytes<FMT>();
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.W, a.N, rowbytes);
    auto off = [&](int r) { return (r < a.N && on) ? uint32_t(r) * rowbytes + uint32_t(p) * lp_bytes<FMT>() : kNoRow; };
    LPair<FMT> w[D];
    float yv[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
        lp_load<FMT>(rs, off(g + k * ng), w[k]);
        yv[k] = (S == 1 && a.accumulate) ? a.y[min(g + k * ng, a.N - 1)] : 0.f;
    }
    XAct v;
    if constexpr (S == 1) {
        __shared__ XStage L;
        xl_stage(L, a.x, nullptr, false, nullptr, nullptr, a.P, 0.f, v.v, lane, lane < a.P);
    } else {
        xl_load(a.x, p, on, v.v);
    }
    if (FMT == F_Q5_0) v.sums();
    for (int k0 = 0; g + k0 * ng < a.N; k0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int k = k0 + j, r = g + k * ng;
            if (r >= a.N) break;
            const float part = lp_dot<FMT>(w[j], v);
            const float y0 = yv[j];
            const int rn = g + (k + D) * ng;
            lp_load<FMT>(rs, off(rn), w[j]);
            if (S == 1 && a.accumulate) yv[j] = a.y[min(rn, a.N - 1)];
            const float s = wave_sum_dpp(part);
            if (S == 1) {
                if (lane == 0) a.y[r] = a.accumulate ? y0 + s : s;
            } else if (lane == 0) {
                red[wv][k] = s;
            }
        }
    }
    if constexpr (S > 1) {
        __syncthreads();
        const int t = threadIdx.x;
        if (t < GW * kXRows) {
            const int gt = t / kXRows, k = t - gt * kXRows;
            const int r = int(blockIdx.x) * GW + gt + k * ng;
            if (r < a.N) {
                float s = red[gt * S][k];
#pragma unroll
                for (int q = 1; q < S; ++q) s += red[gt * S + q][k];
                a.y[r] = a.accumulate ? a.y[r] + s : s;
            }
        }
    }
}

template <int S>
__global__ __launch_bounds__(kThreads) void k_xmatmul1(XMatmulArgs a) { xmatmul_body<F_Q8_0, S>(a); }
template <int S>
__global__ __launch_bounds__(kThreads) void k_xmatmul1_q5(XMatmulArgs a) { xmatmul_body<F_Q5_0, S>(a); }

// ---------------------------------------------------------------- gate/up

struct XGateUpArgs {
    const uint8_t *wg, *wu;
    const float *norm_w;
    const float *x;
    float *h;
    int F, P;
    float eps;
};

template <int FMT>
__device__ __forceinline__ void xgateup_body(XGateUpArgs a) {
    constexpr int D = 1;   // (2 gave 27.0 us against 25.9 on the 7B-class gate/up)
    const int lane = threadIdx.x & 63;
    const int nw = int(gridDim.x) * kWavesX;
    const int g = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * kWavesX + int(threadIdx.x >> 6));
    const bool on = lane < a.P;
    const uint32_t rowbytes = uint32_t(a.P) * lp_bytes<FMT>();
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc(a.wg, a.F, rowbytes), ru = rows_rsrc(a.wu, a.F, rowbytes);
    auto off = [&](int r) { return (r < a.F && on) ? uint32_t(r) * rowbytes + uint32_t(lane) * lp_bytes<FMT>() : kNoRow; };
    LPair<FMT> wg[D], wu[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
        lp_load<FMT>(rg, off(g + k * nw), wg[k]);
        lp_load<FMT>(ru, off(g + k * nw), wu[k]);
    }
    XAct v;
    __shared__ XStage L;
    xl_stage(L, a.x, nullptr, false, nullptr, a.norm_w, a.P, a.eps, v.v, lane, lane < a.P);
    if (FMT == F_Q5_0) v.sums();
    for (int k0 = 0; g + k0 * nw < a.F; k0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int k = k0 + j, f = g + k * nw;
            if (f >= a.F) break;
            const float pg = lp_dot<FMT>(wg[j], v), pu = lp_dot<FMT>(wu[j], v);
            const int fn = g + (k + D) * nw;
            lp_load<FMT>(rg, off(fn), wg[j]);
            lp_load<FMT>(ru, off(fn), wu[j]);
            const float gs = wave_sum_dpp(pg), us = wave_sum_dpp(pu);
            if (lane == 0) a.h[f] = silu(gs) * us;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_xgateup1(XGateUpArgs a) { xgateup_body<F_Q8_0>(a); }
__global__ __launch_bounds__(kThreads) void k_xgateup1_q5(XGateUpArgs a) { xgateup_body<F_Q5_0>(a); }

// ---------------------------------------------------------------- output layer

// logits[r] = W_out[r] . rmsnorm(x) for every row, and per workgroup the
// (largest logit, lowest row among equals) pair, merged later by
// k_argmax_finish. Q8_0 only.
struct XLmHeadArgs {
    const uint8_t *W;
    const float *norm_w;
    const float *x;
    StepState *st;
    float *partials;  // [gridDim.x][2]
    int V, P;
    float eps;
};

__global__ __launch_bounds__(kThreads) void k_xlmhead1(XLmHeadArgs a) {
    constexpr int D = 1;
    __shared__ float s_v[kWavesX];
    __shared__ uint32_t s_i[kWavesX];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int nw = int(gridDim.x) * kWavesX;
    const int g = int(blockIdx.x) * kWavesX + wv;
    const bool on = lane < a.P;
    const uint32_t rowbytes = uint32_t(a.P) * kPairBytes;
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.W, a.V, rowbytes);
    auto off = [&](int r) { return (r < a.V && on) ? uint32_t(r) * rowbytes + uint32_t(lane) * kPairBytes : kNoRow; };
    LPair<F_Q8_0> w[D];
#pragma unroll
    for (int k = 0; k < D; ++k) lp_load<F_Q8_0>(rs, off(g + k * nw), w[k]);
    XAct v;
    __shared__ XStage L;
    xl_stage(L, a.x, nullptr, false, nullptr, a.norm_w, a.P, a.eps, v.v, lane, lane < a.P);
    float *logits = a.st->logits_out;
    float bv = -INFINITY;
    uint32_t bi = uint32_t(g);
    for (int k0 = 0; g + k0 * nw < a.V; k0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int k = k0 + j, r = g + k * nw;
            if (r >= a.V) break;
            const float part = lp_dot<F_Q8_0>(w[j], v);
            lp_load<F_Q8_0>(rs, off(g + (k + D) * nw), w[j]);
            const float s = wave_sum_dpp(part);
            if (lane == 0) logits[r] = s;
            argmax_merge(bv, bi, s, uint32_t(r));
        }
    }
    if (lane == 0) {
        s_v[wv] = bv;
        s_i[wv] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v0 = s_v[0];
        uint32_t i0 = s_i[0];
        for (int w2 = 1; w2 < kWavesX; ++w2) argmax_merge(v0, i0, s_v[w2], s_i[w2]);
        a.partials[2 * blockIdx.x] = v0;
        a.partials[2 * blockIdx.x + 1] = __uint_as_float(i0);
    }
}

// Rows of P < 32 pairs: a wave takes R = 64 / P rows at a time, lane
// l = P * rr + i holding pair i of row rr (lanes from R * P on idle), so each
// 16-byte load moves a whole pair per lane (Q8_0: 17 dwords of 64 weights)
// instead of a byte. Each lane's pair product goes to the wave's row of LDS;
// lane rr < R then adds its row's P products in pair order. A wave takes the
// row groups g, g + waves, ..., kXsGroups of them at most, all loaded before
// the first is computed.
constexpr int kXsGroups = 2;

__global__ __launch_bounds__(kThreads) void k_xlmhead_short(XLmHeadArgs a) {
    constexpr int D = kXsGroups;
    __shared__ float s_v[kWavesX];
    __shared__ uint32_t s_i[kWavesX];
    __shared__ float s_part[kWavesX][64];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int P = a.P, R = 64 / P;
    const int nw = int(gridDim.x) * kWavesX;
    const int g = int(blockIdx.x) * kWavesX + wv;
    const int rr = lane / P, pi = lane - rr * P;
    const bool on = rr < R;
    const int ngroups = (a.V + R - 1) / R;
    const uint32_t rowbytes = uint32_t(P) * kPairBytes;
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.W, a.V, rowbytes);
    auto off = [&](int grp) {
        const int r = grp * R + rr;
        return (on && r < a.V) ? uint32_t(r) * rowbytes + uint32_t(pi) * kPairBytes : kNoRow;
    };
    LPair<F_Q8_0> w[D];
#pragma unroll
    for (int k = 0; k < D; ++k) lp_load<F_Q8_0>(rs, off(g + k * nw), w[k]);
    XAct v;
    __shared__ XStage L;
    xl_stage(L, a.x, nullptr, false, nullptr, a.norm_w, P, a.eps, v.v, pi, on);
    float *logits = a.st->logits_out;
    float *pw = s_part[wv];
    float bv = -INFINITY;
    uint32_t bi = uint32_t(min(g * R, a.V - 1));   // a valid row even if every logit is NaN
    for (int k0 = 0; g + k0 * nw < ngroups; k0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int k = k0 + j, grp = g + k * nw;
            if (grp >= ngroups) break;
            const float part = lp_dot<F_Q8_0>(w[j], v);
            lp_load<F_Q8_0>(rs, off(g + (k + D) * nw), w[j]);
            pw[lane] = part;
            __builtin_amdgcn_wave_barrier();
            const int r = grp * R + lane;
            if (lane < R && r < a.V) {
                float sum = pw[lane * P];
                for (int i = 1; i < P; ++i) sum += pw[lane * P + i];
                logits[r] = sum;
                argmax_merge(bv, bi, sum, uint32_t(r));
            }
            __builtin_amdgcn_wave_barrier();   // the row is rewritten for the next group
        }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
        s_v[wv] = bv;
        s_i[wv] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v0 = s_v[0];
        uint32_t i0 = s_i[0];
        for (int w2 = 1; w2 < kWavesX; ++w2) argmax_merge(v0, i0, s_v[w2], s_i[w2]);
        a.partials[2 * blockIdx.x] = v0;
        a.partials[2 * blockIdx.x + 1] = __uint_as_float(i0);
    }
}

// Workgroups for about `per_cu` per compute unit, at least enough that no wave
// computes more than kXRows rows.
int xgrid(int units, int waves_per_unit, int per_cu) {
    const int min_wgs = (units * waves_per_unit + kWavesX * kXRows - 1) / (kWavesX * kXRows);
    return std::max(1, std::max(min_wgs, std::min(256 * per_cu, (units * waves_per_unit + kWavesX - 1) / kWavesX)));
}

bool rows_fit(int N, int P, int fmt) {
    return uint64_t(N) * uint64_t(P) * uint64_t(fmt == F_Q5_0 ? kQ5PairBytes : kPairBytes) < kNoRow;
}

}  // namespace

bool xgemv_fits(int K) {
    if (K % kPairWeights) return false;
    const int P = K / kPairWeights;
    return P >= kXMinPairs && P <= 64;
}

int xgemv_slices(int K) {
    if (K % kPairWeights) return 0;
    const int P = K / kPairWeights;
    if (P < kXMinPairs) return 0;
    return P <= 64 ? 1 : P <= 128 ? 2 : P <= 256 ? 4 : 0;
}

hipError_t launch_xmatmul(const uint8_t *W, int N, int K, const float *x, int accumulate, float *y, hipStream_t s,
                          int fmt) {
    const int S = xgemv_slices(K);
    const int P = K / kPairWeights;
    if (S == 0 || (fmt != F_Q8_0 && fmt != F_Q5_0) || !rows_fit(N, P, fmt)) return hipErrorNotSupported;
    XMatmulArgs a;
    a.W = W; a.x = x; a.y = y; a.N = N; a.P = P; a.accumulate = accumulate;
    const int grid = xgrid(N, S, S == 1 ? 1 : 2);
    const bool q5 = fmt == F_Q5_0;
    if (S == 1) hipLaunchKernelGGL(q5 ? k_xmatmul1_q5<1> : k_xmatmul1<1>, dim3(grid), dim3(kThreads), 0, s, a);
    else if (S == 2) hipLaunchKernelGGL(q5 ? k_xmatmul1_q5<2> : k_xmatmul1<2>, dim3(grid), dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(q5 ? k_xmatmul1_q5<4> : k_xmatmul1<4>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_xgateup(const Dims &dm, const LayerPtrs &w, const float *x, float *h, hipStream_t s) {
    const int P = dm.H / kPairWeights;
    if (!xgemv_fits(dm.H) || w.fg != w.fu || (w.fg != F_Q8_0 && w.fg != F_Q5_0) || !rows_fit(dm.F, P, w.fg))
        return hipErrorNotSupported;
    XGateUpArgs a;
    a.wg = w.wg; a.wu = w.wu; a.norm_w = w.ffn_norm; a.x = x; a.h = h; a.F = dm.F; a.P = P; a.eps = dm.eps;
    // four workgroups per CU: one resident round at this kernel's register
    // use (7B-class gate/up 26.0 -> 25.0 us; 2, 3, 5, 6 and 7 measured slower)
    const int grid = xgrid(dm.F, 1, 4);
    hipLaunchKernelGGL(w.fg == F_Q5_0 ? k_xgateup1_q5 : k_xgateup1, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

int xlmhead_short_blocks(int V, int K) {
    if (K % kPairWeights) return 0;
    const int P = K / kPairWeights;
    if (P < 1 || P >= kXMinPairs || !rows_fit(V, P, F_Q8_0)) return 0;
    const int ngroups = (V + 64 / P - 1) / (64 / P);
    return std::max(1, (ngroups + kWavesX * kXsGroups - 1) / (kWavesX * kXsGroups));
}

hipError_t launch_xlmhead(const Dims &dm, const uint8_t *Wout, const float *out_norm, const float *x_last,
                          StepState *st, float *partials, int n_partials, hipStream_t s) {
    const int P = dm.H / kPairWeights;
    const bool short_rows = xlmhead_short_blocks(dm.V, dm.H) > 0;
    if ((!short_rows && !xgemv_fits(dm.H)) || !rows_fit(dm.V, P, F_Q8_0) || n_partials < 1)
        return hipErrorNotSupported;
    XLmHeadArgs a;
    a.W = Wout; a.norm_w = out_norm; a.x = x_last; a.st = st; a.partials = partials;
    a.V = dm.V; a.P = P; a.eps = dm.eps;
    hipLaunchKernelGGL(short_rows ? k_xlmhead_short : k_xlmhead1, dim3(n_partials), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace q8l

// k_wgemv.hip -- single-token Q8_0 products for short rows, one wave per
// group of rows, without LDS or barriers.
//
// A decode step of a small model is a chain of GEMVs that each move a few
// hundred KB: the time of such a kernel is its chain of dependent steps, not
// its bytes. Here every wave works alone. Lane l of a wave takes, for each
// 64-weight pair i of a row (K = 64 P), weight p = 64 i + l: byte l % 32 of
// Q8_0 block 2i + l / 32 and that block's f16 scale. It also loads the
// activation values at the same positions p, so the lanes of one wave hold
// the whole activation row between them: the RMSNorm's sum of squares is a
// wave reduction, the normalised values stay in registers, and the dot
// products need nothing from other waves. Every load of the wave (weights,
// scales, activations, norm weights, split-K partial sums, the residual it
// adds to) is issued at the start, so the kernel costs about one memory
// round trip plus a short arithmetic chain.
//
// Arithmetic per row: acc = sum over i (in order) of (d * q) * u in each lane
// (d * q is exact in f32), then the 64 lanes summed by wave_sum_dpp. Q5_0
// rows (22-byte blocks) are read the same way: the lane's weight j = l % 32
// of its block is nibble j / 16 of byte 6 + j % 16 with fifth bit j of the
// word at byte 2, q = (nibble | bit << 4) - 16; each wave picks its matrix's
// format once, before any load (a template of the whole wave's work). The
// epilogues are those of the LDS-staged kernels: rope and the KV-cache write
// (q/k/v), SiLU(gate) * up (gate/up), the residual add (o, down).

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

constexpr int kWaves = kThreads / 64;

// The activation row at this lane's positions (p = 64 i + lane), plus any
// split-K partial sums (in index order); workgroup 0's first wave writes the
// summed row to ps.xout. RowIn::issue starts every load (the row and the
// first NB partial rows) and RowIn::finish adds them up, so that other loads
// can be issued in between. Loads are used without conditions (a load used
// only under a condition would be moved into it): partial rows past n
// re-read the last one and are dropped by a select.
template <int P>
struct RowIn {
    static constexpr int NB = (64 / P) < 1 ? 1 : (64 / P) > 4 ? 4 : (64 / P);   // partial rows per batch
    float v[P];
    float t[NB][P];

    __device__ __forceinline__ void issue(const float *x, const PartSrc &ps) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] = x[i * 64 + lane];
        if (ps.n > 0) {
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const float *pr = ps.part + size_t(min(k, ps.n - 1)) * ps.stride;
#pragma unroll
                for (int i = 0; i < P; ++i) t[k][i] = pr[i * 64 + lane];
            }
        }
    }

    __device__ __forceinline__ void finish(const PartSrc &ps) {
        const int lane = threadIdx.x & 63;
        if (ps.n == 0) return;
        float acc[P];
#pragma unroll
        for (int i = 0; i < P; ++i) acc[i] = t[0][i];
        for (int i0 = 0; i0 < ps.n; i0 += NB) {
            if (i0 > 0) {
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const float *pr = ps.part + size_t(min(i0 + k, ps.n - 1)) * ps.stride;
#pragma unroll
                    for (int i = 0; i < P; ++i) t[k][i] = pr[i * 64 + lane];
                }
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
#pragma unroll
                for (int i = 0; i < P; ++i) {
                    const float s = acc[i] + t[k][i];
                    acc[i] = (i0 + k > 0 && i0 + k < ps.n) ? s : acc[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] += acc[i];
        if (ps.xout && blockIdx.x == 0 && threadIdx.x < 64) {
#pragma unroll
            for (int i = 0; i < P; ++i) ps.xout[i * 64 + lane] = v[i];
        }
    }
};

// u = v / sqrt(mean(v^2) + eps) * w, in place (sum of squares in position
// order within the lane, then wave_sum_dpp).
template <int P>
__device__ __forceinline__ void rms_norm(float (&v)[P], const float (&w)[P], float eps) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) ss = fmaf(v[i], v[i], ss);
    ss = wave_sum_dpp(ss);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(P * 64) + eps);
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = v[i] * r * w[i];
}

// This lane's weights and scales of one row (row bytes at `row`), as loaded:
// Q8_0 the int8, Q5_0 the nibble byte and the fifth-bit word.
template <int P, int FMT>
struct RowRegs {
    int q[P];
    uint32_t d[P];
    uint32_t h[FMT == F_Q5_0 ? P : 1];
};

template <int P, int FMT>
__device__ __forceinline__ void load_weights(const uint8_t *row, RowRegs<P, FMT> &r) {
    const int lane = threadIdx.x & 63;
    if (FMT == F_Q5_0) {
        // d and the fifth-bit word from the two dwords at the block's dword
        // floor (block 0 of a pair: d = bytes 0..1, word = bytes 2..5; block
        // 1, bytes 22..43: d = bytes 22..23, word = bytes 24..27): two dword
        // loads and the value byte, where three 16-bit loads took longer
        const int b1 = lane >> 5, j = lane & 31;
        const uint32_t *w = reinterpret_cast<const uint32_t *>(row) + b1 * 5;
        const uint8_t *qb = row + b1 * kQ5Bytes + 6 + (j & 15);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t lo = w[i * (kQ5PairBytes / 4)], hi = w[i * (kQ5PairBytes / 4) + 1];
            r.d[i] = b1 ? lo >> 16 : lo & 0xffffu;
            r.h[i] = b1 ? hi : __builtin_amdgcn_alignbyte(hi, lo, 2);
            r.q[i] = qb[i * kQ5PairBytes];
        }
    } else {
        const uint8_t *b = row + (lane >> 5) * kQBytes;
        const int o = 2 + (lane & 31);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            r.d[i] = *reinterpret_cast<const uint16_t *>(b + i * kPairBytes);
            r.q[i] = static_cast<int8_t>(b[i * kPairBytes + o]);
        }
    }
}

template <int P, int FMT>
__device__ __forceinline__ float weight(const RowRegs<P, FMT> &r, int i) {
    if (FMT == F_Q5_0) {
        // d * (u - 16) as one FMA, u the 5-bit code: exact (an f16 times an
        // integer below 2^5 needs 16 bits)
        const uint32_t j = threadIdx.x & 31;
        const uint32_t u = (__builtin_amdgcn_ubfe(r.h[i], j, 1) << 4) | __builtin_amdgcn_ubfe(uint32_t(r.q[i]), 4 * (j >> 4), 4);
        const float d = half_bits_to_float(r.d[i]);
        return fmaf(static_cast<float>(u), d, -16.0f * d);
    }
    return half_bits_to_float(r.d[i]) * static_cast<float>(r.q[i]);
}

template <int P, int FMT>
__device__ __forceinline__ float row_dot(const RowRegs<P, FMT> &r, const float (&u)[P]) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) acc = fmaf(weight<P, FMT>(r, i), u[i], acc);
    return wave_sum_dpp(acc);
}

template <int P>
__device__ __forceinline__ size_t row_bytes_of(int fmt) {
    return size_t(P) * (fmt == F_Q5_0 ? kQ5PairBytes : kPairBytes);
}

// ---------------------------------------------------------------- q/k/v

// Wave w of workgroup b takes the row pair (2e, 2e + 1), e = 4 b + w, of the
// stacked q, k, v rows (QD + 2 KVD rows; pairs never straddle two matrices:
// QD and KVD are even). Layer 0 of a step: the input row is the token's
// embedding, dequantized here (x = d * q per block), and workgroup 0's first
// wave writes it to xres.
struct WQkvArgs {
    const uint8_t *wq, *wk, *wv;
    const float *norm_w;
    const float *x;
    const StepState *st;
    const float2 *rope;
    float *q, *kc, *vc;
    int QD, KVD, hd, max_seq;
    float eps;
    int rope_neox;
    const uint8_t *embed;
    float *xres;
    int V;
    PartSrc ps;
    int fmt[3];   // WFmt of q, k, v (Q8_0 or Q5_0)
};

template <int P, int FMT>
__device__ __forceinline__ void wqkv_body(const WQkvArgs &a, int kind, int lrow) {
    const int lane = threadIdx.x & 63;
    const uint8_t *W = kind == 0 ? a.wq : kind == 1 ? a.wk : a.wv;
    const size_t rowbytes = row_bytes_of<P>(FMT);
    RowRegs<P, FMT> r0, r1;
    load_weights<P, FMT>(W + size_t(lrow) * rowbytes, r0);
    load_weights<P, FMT>(W + size_t(lrow + 1) * rowbytes, r1);
    float w[P];
#pragma unroll
    for (int i = 0; i < P; ++i) w[i] = a.norm_w[i * 64 + lane];
    RowIn<P> in;
    float (&v)[P] = in.v;
    if (!a.embed) in.issue(a.x, a.ps);
    // the step state (a scalar load) and the rope factors that depend on it
    // come after the independent loads, so none of those waits for them
    const int pos = a.st->pos, slot = a.st->slot;
    const int d = lrow % a.hd;
    const bool rot = kind != 2 && !a.rope_neox;
    const float2 cs = a.rope[size_t(pos) * (a.hd / 2) + (d >> 1)];
    if (a.embed) {
        const uint32_t tok = a.st->token;
        const bool valid = tok < uint32_t(a.V);
        RowRegs<P, F_Q8_0> er;
        load_weights<P, F_Q8_0>(a.embed + (valid ? size_t(tok) : 0) * row_bytes_of<P>(F_Q8_0), er);
#pragma unroll
        for (int i = 0; i < P; ++i) v[i] = valid ? half_bits_to_float(er.d[i]) * static_cast<float>(er.q[i]) : 0.f;
        if (blockIdx.x == 0 && threadIdx.x < 64) {
#pragma unroll
            for (int i = 0; i < P; ++i) a.xres[i * 64 + lane] = v[i];
        }
    } else {
        in.finish(a.ps);
    }
    rms_norm<P>(v, w, a.eps);
    const float a0 = row_dot<P, FMT>(r0, v), a1 = row_dot<P, FMT>(r1, v);
    // (an empty use here keeps the rope load where it was issued, at the
    // start: a load used only inside the branch below would be moved into it)
    asm volatile("" : : "v"(cs.x), "v"(cs.y));
    const float b0 = rot ? a0 * cs.x - a1 * cs.y : a0;
    const float b1 = rot ? a0 * cs.y + a1 * cs.x : a1;
    if (lane == 0) {
        float *dst = kind == 0   ? a.q + lrow
                     : kind == 1 ? a.kc + (size_t(lrow / a.hd) * a.max_seq + slot) * a.hd + d
                                 : a.vc + (size_t(lrow / a.hd) * a.max_seq + slot) * a.hd + d;
        dst[0] = b0;
        dst[1] = b1;
    }
}

template <int P, int PM>
__device__ __forceinline__ void wqkv_kernel(WQkvArgs a) {
    const int e = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int N = a.QD + 2 * a.KVD;
    if (2 * e >= N) return;   // (no barriers in this kernel)
    const int row = 2 * e;
    const int kind = row < a.QD ? 0 : row < a.QD + a.KVD ? 1 : 2;
    const int lrow = kind == 0 ? row : kind == 1 ? row - a.QD : row - a.QD - a.KVD;
    const bool q5 = PM == PM_Q5 || (PM == PM_MIXED && (kind == 0 ? a.fmt[0] == F_Q5_0
                                                        : kind == 1 ? a.fmt[1] == F_Q5_0
                                                                    : a.fmt[2] == F_Q5_0));
    if (q5)
        wqkv_body<P, F_Q5_0>(a, kind, lrow);
    else
        wqkv_body<P, F_Q8_0>(a, kind, lrow);
}

// One kernel per block-format mode (PairMode).
template <int P>
__global__ __launch_bounds__(kThreads) void k_wqkv1(WQkvArgs a) { wqkv_kernel<P, PM_Q8>(a); }
template <int P>
__global__ __launch_bounds__(kThreads) void k_wqkv1_q5(WQkvArgs a) { wqkv_kernel<P, PM_Q5>(a); }
template <int P>
__global__ __launch_bounds__(kThreads) void k_wqkv1_mixed(WQkvArgs a) { wqkv_kernel<P, PM_MIXED>(a); }

// ---------------------------------------------------------------- gate/up

struct WGateUpArgs {
    const uint8_t *wg, *wu;
    const float *norm_w;
    const float *x;
    float *h;
    int F;
    float eps;
    PartSrc ps;
};

// Wave w of workgroup b: row f = 4 b + w of gate and of up; h[f] = SiLU(g) * u.
template <int P, int FMT>
__device__ __forceinline__ void wgateup_body(const WGateUpArgs &a, int f) {
    const int lane = threadIdx.x & 63;
    const size_t rowbytes = row_bytes_of<P>(FMT);
    RowRegs<P, FMT> rg, ru;
    load_weights<P, FMT>(a.wg + size_t(f) * rowbytes, rg);
    load_weights<P, FMT>(a.wu + size_t(f) * rowbytes, ru);
    float w[P];
#pragma unroll
    for (int i = 0; i < P; ++i) w[i] = a.norm_w[i * 64 + lane];
    RowIn<P> in;
    in.issue(a.x, a.ps);
    in.finish(a.ps);
    rms_norm<P>(in.v, w, a.eps);
    const float g = row_dot<P, FMT>(rg, in.v), u = row_dot<P, FMT>(ru, in.v);
    if (lane == 0) a.h[f] = silu(g) * u;
}

template <int P, int FMT>
__device__ __forceinline__ void wgateup_kernel(const WGateUpArgs &a) {
    const int f = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (f >= a.F) return;
    wgateup_body<P, FMT>(a, f);
}

template <int P>
__global__ __launch_bounds__(kThreads) void k_wgateup1(WGateUpArgs a) { wgateup_kernel<P, F_Q8_0>(a); }
template <int P>
__global__ __launch_bounds__(kThreads) void k_wgateup1_q5(WGateUpArgs a) { wgateup_kernel<P, F_Q5_0>(a); }

// ---------------------------------------------------------------- o, down

struct WMatmulArgs {
    const uint8_t *W;
    const float *x;
    float *y;
    int N, accumulate;
};

// Wave w of workgroup b: rows 2e, 2e + 1 (e = 4 b + w); y[row] (+)= W[row] . x.
template <int P, int FMT>
__device__ __forceinline__ void wmatmul_body(const WMatmulArgs &a, int row) {
    const int lane = threadIdx.x & 63;
    const bool two = row + 1 < a.N;
    const size_t rowbytes = row_bytes_of<P>(FMT);
    RowRegs<P, FMT> r0, r1;
    load_weights<P, FMT>(a.W + size_t(row) * rowbytes, r0);
    load_weights<P, FMT>(a.W + size_t(two ? row + 1 : row) * rowbytes, r1);
    const float y0 = a.accumulate ? a.y[row] : 0.f;
    const float y1 = a.accumulate ? a.y[two ? row + 1 : row] : 0.f;
    RowIn<P> in;
    in.issue(a.x, PartSrc{});
    const float s0 = row_dot<P, FMT>(r0, in.v), s1 = row_dot<P, FMT>(r1, in.v);
    asm volatile("" : : "v"(y0), "v"(y1));   // keeps the residual loads at the start (see k_wqkv1)
    const float o0 = a.accumulate ? y0 + s0 : s0, o1 = a.accumulate ? y1 + s1 : s1;
    if (lane == 0) {
        a.y[row] = o0;
        if (two) a.y[row + 1] = o1;
    }
}

template <int P, int FMT>
__device__ __forceinline__ void wmatmul_kernel(const WMatmulArgs &a) {
    const int e = blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int row = 2 * e;
    if (row >= a.N) return;
    wmatmul_body<P, FMT>(a, row);
}

template <int P>
__global__ __launch_bounds__(kThreads) void k_wmatmul1(WMatmulArgs a) { wmatmul_kernel<P, F_Q8_0>(a); }
template <int P>
__global__ __launch_bounds__(kThreads) void k_wmatmul1_q5(WMatmulArgs a) { wmatmul_kernel<P, F_Q5_0>(a); }

template <class F>
bool dispatch_p(int P, F &&f) {
    switch (P) {
        case 1: f(std::integral_constant<int, 1>{}); return true;
        case 2: f(std::integral_constant<int, 2>{}); return true;
        case 4: f(std::integral_constant<int, 4>{}); return true;
        case 8: f(std::integral_constant<int, 8>{}); return true;
        case 9: f(std::integral_constant<int, 9>{}); return true;
        case 12: f(std::integral_constant<int, 12>{}); return true;
        case 16: f(std::integral_constant<int, 16>{}); return true;
        case 24: f(std::integral_constant<int, 24>{}); return true;
        default: return false;
    }
}

}  // namespace

bool wgemv_fits(int K) {
    if (K % kPairWeights) return false;
    return dispatch_p(K / kPairWeights, [](auto) {});
}

hipError_t launch_wqkv(const Dims &dm, const LayerPtrs &w, const float *x, const StepState *st, const float2 *rope,
                       float *q, float *kc, float *vc, hipStream_t s, const uint8_t *embed, float *xres,
                       const PartSrc &ps) {
    WQkvArgs a;
    a.wq = w.wq; a.wk = w.wk; a.wv = w.wv; a.norm_w = w.attn_norm; a.x = x; a.st = st; a.rope = rope;
    a.q = q; a.kc = kc; a.vc = vc;
    a.QD = dm.nh * dm.hd; a.KVD = dm.nkv * dm.hd; a.hd = dm.hd; a.max_seq = dm.max_seq;
    a.eps = dm.eps; a.rope_neox = dm.rope_neox;
    a.embed = embed; a.xres = xres; a.V = dm.V; a.ps = ps;
    a.fmt[0] = w.fq; a.fmt[1] = w.fk; a.fmt[2] = w.fv;
    const int pairs = (a.QD + 2 * a.KVD) / 2;
    const int grid = (pairs + kWaves - 1) / kWaves;
    const int pm = pair_mode(w.fq, w.fk, w.fv);
    if (!dispatch_p(dm.H / kPairWeights, [&](auto p) {
            constexpr int P = decltype(p)::value;
            if (pm == PM_Q8) hipLaunchKernelGGL(k_wqkv1<P>, dim3(grid), dim3(kThreads), 0, s, a);
            else if (pm == PM_Q5) hipLaunchKernelGGL(k_wqkv1_q5<P>, dim3(grid), dim3(kThreads), 0, s, a);
            else hipLaunchKernelGGL(k_wqkv1_mixed<P>, dim3(grid), dim3(kThreads), 0, s, a);
        }))
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_wgateup(const Dims &dm, const LayerPtrs &w, const float *x, float *h, hipStream_t s,
                          const PartSrc &ps) {
    WGateUpArgs a;
    a.wg = w.wg; a.wu = w.wu; a.norm_w = w.ffn_norm; a.x = x; a.h = h; a.F = dm.F; a.eps = dm.eps; a.ps = ps;
    const int grid = (dm.F + kWaves - 1) / kWaves;
    if (!dispatch_p(dm.H / kPairWeights, [&](auto p) {
            constexpr int P = decltype(p)::value;
            if (w.fg == F_Q5_0) hipLaunchKernelGGL(k_wgateup1_q5<P>, dim3(grid), dim3(kThreads), 0, s, a);
            else hipLaunchKernelGGL(k_wgateup1<P>, dim3(grid), dim3(kThreads), 0, s, a);
        }))
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_wmatmul(const uint8_t *W, int N, int K, const float *x, int accumulate, float *y, hipStream_t s,
                          int fmt) {
    WMatmulArgs a;
    a.W = W; a.x = x; a.y = y; a.N = N; a.accumulate = accumulate;
    const int grid = ((N + 1) / 2 + kWaves - 1) / kWaves;
    if (!dispatch_p(K / kPairWeights, [&](auto p) {
            constexpr int P = decltype(p)::value;
            if (fmt == F_Q5_0) hipLaunchKernelGGL(k_wmatmul1_q5<P>, dim3(grid), dim3(kThreads), 0, s, a);
            else hipLaunchKernelGGL(k_wmatmul1<P>, dim3(grid), dim3(kThreads), 0, s, a);
        }))
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace q8l

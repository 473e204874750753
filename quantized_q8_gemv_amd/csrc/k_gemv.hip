// k_gemv.hip -- Q8_0 x f32 matrix-vector (and few-token) products for gfx950.
//
// One kernel family covers every projection of the forward pass ("量化 llama
// 的一次前向": q/k/v, o, gate/up, down and the output layer are each one
// quantized matmul). A decode step multiplies each weight matrix by a single
// activation row, so the work is a stream of 34-byte Q8_0 blocks from HBM.
//
// Workgroup layout (256 threads = 4 wave64):
//   * the workgroup owns NR consecutive rows of one or two matrices and walks
//     K in chunks of PC block pairs (a pair = 2 blocks = 68 bytes, always
//     4-byte aligned because K is a multiple of 64);
//   * each chunk of weights is copied HBM -> LDS with coalesced 16-byte loads
//     when aligned (4-byte loads otherwise) -- the 34-byte blocks are not
//     16-byte aligned, so lanes cannot decode straight from their own loads;
//   * the activation chunk is staged in LDS, with RMSNorm applied on the way
//     when the projection has a norm in front (each workgroup recomputes the
//     row's sum of squares; it is K floats from L2, far less than its weights);
//   * thread u decodes pair u of the tile (17 dwords, stride 17 -> no LDS bank
//     conflicts) and accumulates d * sum(q * x) per block in f32 for each of
//     up to MAXT tokens;
//   * per-row partials are reduced in a fixed order (lane-strided sum, then a
//     butterfly), so results are bitwise reproducible run to run.
// The epilogue fuses the op that follows the projection: rope + KV-cache
// write (q/k/v), SiLU(gate)*up (gate/up), residual add (o, down), or the
// greedy argmax (output layer).

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

constexpr int kXPad = 68;  // floats per staged 64-weight activation pair (bank padding)

struct CoreArgs {
    const uint8_t *W[2];
    int nmat;
    GemvShape sh;
    int N;
    int row0;
    int Tc;
    const float *X;  // token t at X + t * ldx
    int ldx;
    const float *norm_w;
    float eps;
};

struct Lds {
    uint32_t *wt;   // nmat*NR*PC*17 dwords (reused for partials)
    float *xs;      // MAXT*PC*kXPad
    float *outv;    // MAXT*nmat*NR
    float *rinv;    // MAXT
    float *red;     // 4
};

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

__host__ __device__ inline size_t lds_bytes(const GemvShape &sh, int nmat, int maxt) {
    size_t wt = size_t(nmat) * sh.NR * sh.PC * kPairBytes;
    size_t part = size_t(maxt) * nmat * sh.NR * sh.PC * 4;
    size_t b = align16(std::max(wt, part));
    b += align16(size_t(maxt) * sh.PC * kXPad * 4);
    b += align16(size_t(maxt) * nmat * sh.NR * 4);
    b += align16(size_t(maxt) * 4) + 16;
    return b;
}

__device__ inline Lds carve(uint8_t *smem, const GemvShape &sh, int nmat, int maxt) {
    Lds l;
    size_t wt = size_t(nmat) * sh.NR * sh.PC * kPairBytes;
    size_t part = size_t(maxt) * nmat * sh.NR * sh.PC * 4;
    size_t off = 0;
    l.wt = reinterpret_cast<uint32_t *>(smem + off);
    off += align16(wt > part ? wt : part);
    l.xs = reinterpret_cast<float *>(smem + off);
    off += align16(size_t(maxt) * sh.PC * kXPad * 4);
    l.outv = reinterpret_cast<float *>(smem + off);
    off += align16(size_t(maxt) * nmat * sh.NR * 4);
    l.rinv = reinterpret_cast<float *>(smem + off);
    off += align16(size_t(maxt) * 4);
    l.red = reinterpret_cast<float *>(smem + off);
    return l;
}

// Copy rows [row0, row0+nrows), pairs [c*PC, (c+1)*PC) of one matrix to LDS
// as a flat [row][pair] array of 17-dword pairs.
__device__ inline void load_tile(const uint8_t *W, const GemvShape &sh, int row0, int nrows,
                                 int c, uint32_t *dst) {
    const int tid = threadIdx.x;
    const uint8_t *base = W + size_t(row0) * sh.rowbytes + size_t(c) * sh.PC * kPairBytes;
    if (sh.PC == sh.P) {
        const int nbytes = nrows * sh.rowbytes;
        if (((reinterpret_cast<uintptr_t>(base) | reinterpret_cast<uintptr_t>(dst) | nbytes) & 15) == 0) {
            const u32x4 *s4 = reinterpret_cast<const u32x4 *>(base);
            u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
            for (int i = tid; i < nbytes / 16; i += kThreads) d4[i] = __builtin_nontemporal_load(s4 + i);
        } else {
            const uint32_t *s1 = reinterpret_cast<const uint32_t *>(base);
            for (int i = tid; i < nbytes / 4; i += kThreads) dst[i] = __builtin_nontemporal_load(s1 + i);
        }
    } else {
        const int slice = sh.PC * (kPairBytes / 4);
        const int total = nrows * slice;
        for (int i = tid; i < total; i += kThreads) {
            const int r = i / slice;
            const int w = i - r * slice;
            const uint32_t *s1 = reinterpret_cast<const uint32_t *>(base + size_t(r) * sh.rowbytes);
            dst[i] = __builtin_nontemporal_load(s1 + w);
        }
    }
}

// Computes outv[(t*nmat + m)*NR + r] = sum_k W_m[row0+r][k] * U[t][k].
template <int MAXT>
__device__ void gemv_core(const CoreArgs &a, const Lds &l) {
    const int tid = threadIdx.x;
    const GemvShape &sh = a.sh;
    const int nrows = min(sh.NR, a.N - a.row0);
    const int per_mat = nrows * sh.PC;
    const int units = a.nmat * per_mat;

    if (a.norm_w) {
        for (int t = 0; t < a.Tc; ++t) {
            float ss = 0.f;
            const float *xr = a.X + size_t(t) * a.ldx;
            for (int k = tid; k < sh.K; k += kThreads) {
                float v = xr[k];
                ss = fmaf(v, v, ss);
            }
            ss = block_sum(ss, l.red);
            if (tid == 0) l.rinv[t] = 1.0f / sqrtf(ss / static_cast<float>(sh.K) + a.eps);
        }
        __syncthreads();
    }

    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.f;

    int up = 0;
    if (tid < units) {
        const int rem = tid % per_mat;
        up = rem % sh.PC;
    }
    const int nchunks = sh.P / sh.PC;
    for (int c = 0; c < nchunks; ++c) {
        for (int m = 0; m < a.nmat; ++m)
            load_tile(a.W[m], sh, a.row0, nrows, c, l.wt + size_t(m) * per_mat * (kPairBytes / 4));
        const int n4 = a.Tc * sh.PC * 16;
        for (int e = tid; e < n4; e += kThreads) {
            const int t = e / (sh.PC * 16);
            const int rem = e - t * sh.PC * 16;
            const int p = rem >> 4;
            const int i4 = rem & 15;
            const int k = (c * sh.PC + p) * kPairWeights + i4 * 4;
            float4 v = *reinterpret_cast<const float4 *>(a.X + size_t(t) * a.ldx + k);
            if (a.norm_w) {
                const float r = l.rinv[t];
                const float4 w = *reinterpret_cast<const float4 *>(a.norm_w + k);
                v.x = v.x * r * w.x;
                v.y = v.y * r * w.y;
                v.z = v.z * r * w.z;
                v.w = v.w * r * w.w;
            }
            *reinterpret_cast<float4 *>(l.xs + (size_t(t) * sh.PC + p) * kXPad + i4 * 4) = v;
        }
        __syncthreads();
        if (tid < units) {
            PairQ pq;
            decode_pair(l.wt + size_t(tid) * (kPairBytes / 4), pq);
#pragma unroll
            for (int t = 0; t < MAXT; ++t) {
                if (t < a.Tc) {
                    const float *x = l.xs + (size_t(t) * sh.PC + up) * kXPad;
                    acc[t] = fmaf(pq.dA, block_dot(pq.q, x), acc[t]);
                    acc[t] = fmaf(pq.dB, block_dot(pq.q + 32, x + 32), acc[t]);
                }
            }
        }
        __syncthreads();
    }

    float *part = reinterpret_cast<float *>(l.wt);
    if (tid < units) {
#pragma unroll
        for (int t = 0; t < MAXT; ++t)
            if (t < a.Tc) part[size_t(t) * units + tid] = acc[t];
    }
    __syncthreads();
    const int lane = tid & 63, wid = tid >> 6;
    const int items = a.Tc * a.nmat * nrows;
    for (int it = wid; it < items; it += 4) {
        const int t = it / (a.nmat * nrows);
        const int rem = it - t * a.nmat * nrows;  // m * nrows + r
        const float *src = part + size_t(t) * units + size_t(rem) * sh.PC;
        float v = 0.f;
        for (int p = lane; p < sh.PC; p += 64) v += src[p];
        v = wave_sum(v);
        if (lane == 0) {
            const int m = rem / nrows, r = rem - m * nrows;
            l.outv[(t * a.nmat + m) * sh.NR + r] = v;
        }
    }
    __syncthreads();
}

// ---------------------------------------------------------------- q/k/v

struct QkvArgs {
    const uint8_t *wq, *wk, *wv;
    const float *norm_w;
    const float *x;  // [T][H]
    const StepState *st;
    const float2 *rope;  // [max_seq][hd/2]
    float *q;            // [T][QD]
    float *kc, *vc;      // this layer's [nkv][max_seq][hd]
    GemvShape sh;
    int tq, tk;          // tiles of q, of k (v has tk too)
    int QD, KVD, hd, max_seq, T;
    float eps;
};

template <int MAXT>
__global__ __launch_bounds__(kThreads) void k_qkv(QkvArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds l = carve(smem, a.sh, 1, MAXT);
    int tile = blockIdx.x, kind;
    const uint8_t *W;
    int N;
    if (tile < a.tq) {
        kind = 0; W = a.wq; N = a.QD;
    } else if (tile < a.tq + a.tk) {
        kind = 1; W = a.wk; N = a.KVD; tile -= a.tq;
    } else {
        kind = 2; W = a.wv; N = a.KVD; tile -= a.tq + a.tk;
    }
    const int t0 = blockIdx.y * MAXT;
    CoreArgs c;
    c.W[0] = W; c.W[1] = nullptr; c.nmat = 1; c.sh = a.sh; c.N = N;
    c.row0 = tile * a.sh.NR; c.Tc = min(MAXT, a.T - t0);
    c.X = a.x + size_t(t0) * a.sh.K; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<MAXT>(c, l);

    const int nrows = min(a.sh.NR, N - c.row0);
    const int half = nrows >> 1;
    const int pos0 = a.st->pos + t0, slot0 = a.st->slot + t0;
    for (int e = threadIdx.x; e < c.Tc * half; e += kThreads) {
        const int t = e / half;
        const int r = 2 * (e - t * half);
        const float a0 = l.outv[t * a.sh.NR + r], a1 = l.outv[t * a.sh.NR + r + 1];
        const int row = c.row0 + r;
        const int d = row % a.hd;
        if (kind == 2) {
            float *dst = a.vc + (size_t(row / a.hd) * a.max_seq + slot0 + t) * a.hd + d;
            dst[0] = a0;
            dst[1] = a1;
        } else {
            const float2 cs = a.rope[size_t(pos0 + t) * (a.hd / 2) + (d >> 1)];
            const float b0 = a0 * cs.x - a1 * cs.y;
            const float b1 = a0 * cs.y + a1 * cs.x;
            float *dst = (kind == 0)
                             ? a.q + size_t(t0 + t) * a.QD + row
                             : a.kc + (size_t(row / a.hd) * a.max_seq + slot0 + t) * a.hd + d;
            dst[0] = b0;
            dst[1] = b1;
        }
    }
}

// ---------------------------------------------------------------- gate/up

struct GateUpArgs {
    const uint8_t *wg, *wu;
    const float *norm_w;
    const float *x;
    float *h;  // [T][F]
    GemvShape sh;
    int F, T;
    float eps;
};

template <int MAXT>
__global__ __launch_bounds__(kThreads) void k_gateup(GateUpArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds l = carve(smem, a.sh, 2, MAXT);
    const int t0 = blockIdx.y * MAXT;
    CoreArgs c;
    c.W[0] = a.wg; c.W[1] = a.wu; c.nmat = 2; c.sh = a.sh; c.N = a.F;
    c.row0 = blockIdx.x * a.sh.NR; c.Tc = min(MAXT, a.T - t0);
    c.X = a.x + size_t(t0) * a.sh.K; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<MAXT>(c, l);
    const int nrows = min(a.sh.NR, a.F - c.row0);
    for (int e = threadIdx.x; e < c.Tc * nrows; e += kThreads) {
        const int t = e / nrows, r = e - t * nrows;
        const float g = l.outv[(t * 2 + 0) * a.sh.NR + r];
        const float u = l.outv[(t * 2 + 1) * a.sh.NR + r];
        a.h[size_t(t0 + t) * a.F + c.row0 + r] = silu(g) * u;
    }
}

// ---------------------------------------------------------------- generic (o, down, op)

struct MatmulArgs {
    const uint8_t *W;
    const float *norm_w;
    const float *x;
    float *y;  // [T][N]
    GemvShape sh;
    int N, T, accumulate;
    float eps;
};

template <int MAXT>
__global__ __launch_bounds__(kThreads) void k_matmul(MatmulArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds l = carve(smem, a.sh, 1, MAXT);
    const int t0 = blockIdx.y * MAXT;
    CoreArgs c;
    c.W[0] = a.W; c.W[1] = nullptr; c.nmat = 1; c.sh = a.sh; c.N = a.N;
    c.row0 = blockIdx.x * a.sh.NR; c.Tc = min(MAXT, a.T - t0);
    c.X = a.x + size_t(t0) * a.sh.K; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<MAXT>(c, l);
    const int nrows = min(a.sh.NR, a.N - c.row0);
    for (int e = threadIdx.x; e < c.Tc * nrows; e += kThreads) {
        const int t = e / nrows, r = e - t * nrows;
        float *dst = a.y + size_t(t0 + t) * a.N + c.row0 + r;
        const float v = l.outv[t * a.sh.NR + r];
        *dst = a.accumulate ? *dst + v : v;
    }
}

// ---------------------------------------------------------------- output layer + argmax

struct LmHeadArgs {
    const uint8_t *W;
    const float *norm_w;
    const float *x;      // [H], the last position
    StepState *st;
    float *partials;     // [gridDim.x][2] (value, index bits)
    uint32_t *counter;
    GemvShape sh;
    int V;
    float eps;
};

// Final reduction of per-workgroup (value, index) partials; called by the
// last workgroup to finish. Fixed order: thread-strided, then butterflies.
__device__ void argmax_finish(const float *partials, int n, float *red, uint32_t *redi,
                              float &bv, uint32_t &bi) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float v = -INFINITY;
    uint32_t i = 0xffffffffu;
    for (int b = tid; b < n; b += kThreads) {
        const float ov = __builtin_nontemporal_load(partials + 2 * b);
        const uint32_t oi = __float_as_uint(__builtin_nontemporal_load(partials + 2 * b + 1));
        argmax_merge(v, i, ov, oi);
    }
    wave_argmax(v, i);
    if (lane == 0) {
        red[wid] = v;
        redi[wid] = i;
    }
    __syncthreads();
    bv = red[0];
    bi = redi[0];
    for (int w = 1; w < 4; ++w) argmax_merge(bv, bi, red[w], redi[w]);
}

__global__ __launch_bounds__(kThreads) void k_lmhead(LmHeadArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds l = carve(smem, a.sh, 1, 1);
    __shared__ float s_red[4];
    __shared__ uint32_t s_redi[4];
    __shared__ int s_last;
    CoreArgs c;
    c.W[0] = a.W; c.W[1] = nullptr; c.nmat = 1; c.sh = a.sh; c.N = a.V;
    c.row0 = blockIdx.x * a.sh.NR; c.Tc = 1;
    c.X = a.x; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<1>(c, l);
    const int nrows = min(a.sh.NR, a.V - c.row0);
    float *logits = a.st->logits_out;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    for (int r = tid; r < nrows; r += kThreads) {
        const float v = l.outv[r];
        logits[c.row0 + r] = v;
        argmax_merge(bv, bi, v, uint32_t(c.row0 + r));
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
        s_red[wid] = bv;
        s_redi[wid] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        float v = s_red[0];
        uint32_t i = s_redi[0];
        for (int w = 1; w < 4; ++w) argmax_merge(v, i, s_red[w], s_redi[w]);
        a.partials[2 * blockIdx.x] = v;
        a.partials[2 * blockIdx.x + 1] = __uint_as_float(i);
        __threadfence();
        const uint32_t prev = atomicAdd(a.counter, 1u);
        s_last = (prev == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    float v;
    uint32_t i;
    argmax_finish(a.partials, gridDim.x, s_red, s_redi, v, i);
    if (tid == 0) {
        StepState *st = a.st;
        if (st->argmax_out) *st->argmax_out = i;
        if (st->advance) {
            if (st->ids_out) st->ids_out[st->step] = i;
            st->token = i;
            st->pos += 1;
            st->slot += 1;
            st->step += 1;
        }
        *a.counter = 0u;  // ready for the next launch (no memset node needed)
    }
}

__global__ __launch_bounds__(kThreads) void k_argmax(const float *x, int64_t n, uint32_t *out,
                                                     float *partials, uint32_t *counter) {
    __shared__ float s_red[4];
    __shared__ uint32_t s_redi[4];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t per = 4096;
    const int64_t b0 = int64_t(blockIdx.x) * per;
    const int64_t e = min(n, b0 + per);
    float bv = -INFINITY;
    uint32_t bi = 0xffffffffu;
    for (int64_t j = b0 + tid; j < e; j += kThreads) argmax_merge(bv, bi, x[j], uint32_t(j));
    wave_argmax(bv, bi);
    if (lane == 0) {
        s_red[wid] = bv;
        s_redi[wid] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        float v = s_red[0];
        uint32_t i = s_redi[0];
        for (int w = 1; w < 4; ++w) argmax_merge(v, i, s_red[w], s_redi[w]);
        partials[2 * blockIdx.x] = v;
        partials[2 * blockIdx.x + 1] = __uint_as_float(i);
        __threadfence();
        s_last = (atomicAdd(counter, 1u) == gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    float v;
    uint32_t i;
    argmax_finish(partials, gridDim.x, s_red, s_redi, v, i);
    if (tid == 0) {
        *out = i;
        *counter = 0u;
    }
}

// ---------------------------------------------------------------- host side

int divisor_at_most(int P, int cap) {
    for (int d = std::min(P, cap); d >= 1; --d)
        if (P % d == 0) return d;
    return 1;
}

// Pick pairs-per-chunk and rows-per-workgroup for an N x K matrix.
//   maxt:        tokens per workgroup (LDS for the staged activations)
//   nmat:        matrices processed together
//   target_wgs:  aim for at least this many workgroups
//   nr_mult:     rows per workgroup must be a multiple of this (2 for rope pairs)
GemvShape choose_shape(int N, int K, int maxt, int nmat, int target_wgs, int nr_mult) {
    GemvShape s;
    s.K = K;
    s.P = K / kPairWeights;
    s.rowbytes = s.P * kPairBytes;
    const int lds_cap_pairs = std::max(1, (40 * 1024) / (maxt * kXPad * 4));
    s.PC = divisor_at_most(s.P, std::min(lds_cap_pairs, kThreads / nmat));
    int nr = kThreads / (nmat * s.PC);
    const int want = (N + target_wgs - 1) / target_wgs;
    nr = std::min(nr, std::max(want, 1));
    // prefer 16-byte aligned whole-row tiles (4 rows of any K are aligned)
    if (nr >= 4) nr -= nr % 4;
    nr = std::max(nr_mult, nr - nr % nr_mult);
    s.NR = nr;
    return s;
}

static hipError_t set_lds(const void *fn, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

}  // namespace

hipError_t launch_qkv(const Dims &d, const LayerPtrs &w, const float *x, const StepState *st,
                      const float2 *rope, float *q, float *kc, float *vc, int T, hipStream_t s) {
    const int maxt = T == 1 ? 1 : kMaxTokChunk;
    QkvArgs a;
    a.wq = w.wq; a.wk = w.wk; a.wv = w.wv; a.norm_w = w.attn_norm; a.x = x; a.st = st;
    a.rope = rope; a.q = q; a.kc = kc; a.vc = vc;
    a.QD = d.nh * d.hd; a.KVD = d.nkv * d.hd; a.hd = d.hd; a.max_seq = d.max_seq; a.T = T;
    a.eps = d.eps;
    a.sh = choose_shape(a.QD + 2 * a.KVD, d.H, maxt, 1, 512, 2);
    a.tq = (a.QD + a.sh.NR - 1) / a.sh.NR;
    a.tk = (a.KVD + a.sh.NR - 1) / a.sh.NR;
    dim3 grid(a.tq + 2 * a.tk, (T + maxt - 1) / maxt);
    const size_t lds = lds_bytes(a.sh, 1, maxt);
    if (maxt == 1) {
        hipLaunchKernelGGL(k_qkv<1>, grid, dim3(kThreads), lds, s, a);
    } else {
        hipLaunchKernelGGL(k_qkv<kMaxTokChunk>, grid, dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gateup(const Dims &d, const LayerPtrs &w, const float *x, float *h, int T,
                         hipStream_t s) {
    const int maxt = T == 1 ? 1 : kMaxTokChunk;
    GateUpArgs a;
    a.wg = w.wg; a.wu = w.wu; a.norm_w = w.ffn_norm; a.x = x; a.h = h; a.F = d.F; a.T = T;
    a.eps = d.eps;
    a.sh = choose_shape(d.F, d.H, maxt, 2, 512, 1);
    dim3 grid((d.F + a.sh.NR - 1) / a.sh.NR, (T + maxt - 1) / maxt);
    const size_t lds = lds_bytes(a.sh, 2, maxt);
    if (maxt == 1) {
        hipLaunchKernelGGL(k_gateup<1>, grid, dim3(kThreads), lds, s, a);
    } else {
        hipLaunchKernelGGL(k_gateup<kMaxTokChunk>, grid, dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_matmul(const uint8_t *W, int N, int K, const float *X, int T,
                         const float *norm_w, float eps, int accumulate, float *Y,
                         hipStream_t s) {
    const int maxt = T == 1 ? 1 : kMaxTokChunk;
    MatmulArgs a;
    a.W = W; a.norm_w = norm_w; a.x = X; a.y = Y; a.N = N; a.T = T; a.accumulate = accumulate;
    a.eps = eps;
    a.sh = choose_shape(N, K, maxt, 1, 512, 1);
    dim3 grid((N + a.sh.NR - 1) / a.sh.NR, (T + maxt - 1) / maxt);
    const size_t lds = lds_bytes(a.sh, 1, maxt);
    if (maxt == 1) {
        hipLaunchKernelGGL(k_matmul<1>, grid, dim3(kThreads), lds, s, a);
    } else {
        hipLaunchKernelGGL(k_matmul<kMaxTokChunk>, grid, dim3(kThreads), lds, s, a);
    }
    return hipGetLastError();
}

static int lmhead_nr(int V, int K) { return choose_shape(V, K, 1, 1, 1024, 1).NR; }

hipError_t launch_lmhead(const Dims &d, const uint8_t *Wout, const float *out_norm,
                         const float *x_last, StepState *st, float *partials, uint32_t *counter,
                         hipStream_t s) {
    LmHeadArgs a;
    a.W = Wout; a.norm_w = out_norm; a.x = x_last; a.st = st; a.partials = partials;
    a.counter = counter; a.V = d.V; a.eps = d.eps;
    a.sh = choose_shape(d.V, d.H, 1, 1, 1024, 1);
    dim3 grid((d.V + a.sh.NR - 1) / a.sh.NR);
    hipLaunchKernelGGL(k_lmhead, grid, dim3(kThreads), lds_bytes(a.sh, 1, 1), s, a);
    return hipGetLastError();
}

size_t lmhead_partials_bytes(int V, int K) {
    const int nr = lmhead_nr(V, K);
    return size_t((V + nr - 1) / nr) * 8;
}

size_t argmax_partials_bytes(int64_t n) { return size_t((n + 4095) / 4096) * 8; }

hipError_t launch_argmax(const float *x, int64_t n, uint32_t *out, float *partials,
                         uint32_t *counter, hipStream_t s) {
    const unsigned grid = unsigned((n + 4095) / 4096);
    hipLaunchKernelGGL(k_argmax, dim3(grid), dim3(kThreads), 0, s, x, n, out, partials, counter);
    return hipGetLastError();
}

}  // namespace q8l

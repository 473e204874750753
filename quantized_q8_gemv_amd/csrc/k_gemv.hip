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

// Decode o-projection after a multi-split attention: the activation row is
// merged from the attention's split partials instead of read from X. (Kept out
// of CoreArgs: a larger CoreArgs is copied through scratch memory.)
struct MergeSrc {
    const float *part;       // [nh][splits][hd + 2]: (max, sum, unnormalised o)
    int splits, hd;
    const StepState *st;     // active splits from the cache length
};

struct Lds {
    uint32_t *wt;   // nmat*NR*PC*17 dwords (reused for partials)
    float *xs;      // MAXT*PC*kXPad
    float *outv;    // max(MAXT*nmat*NR, 4*MAXT); also the norm prologue's scratch
    float *rinv;    // MAXT
    float *red;     // 4
};

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

__host__ __device__ inline size_t lds_bytes(const GemvShape &sh, int nmat, int maxt) {
    size_t wt = size_t(nmat) * sh.NR * sh.PC * kPairBytes;
    size_t part = size_t(maxt) * nmat * sh.NR * sh.PC * 4;
    size_t b = align16(std::max(wt, part));
    b += align16(size_t(maxt) * sh.PC * kXPad * 4);
    b += align16(std::max(size_t(maxt) * nmat * sh.NR, size_t(4) * maxt) * 4);
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
    off += align16((size_t(maxt) * nmat * sh.NR > size_t(4) * maxt ? size_t(maxt) * nmat * sh.NR
                                                                 : size_t(4) * maxt) * 4);
    l.rinv = reinterpret_cast<float *>(smem + off);
    off += align16(size_t(maxt) * 4);
    l.red = reinterpret_cast<float *>(smem + off);
    return l;
}

// Weight tile staging. A workgroup's tile for chunk c is nmat x nrows row
// slices of PC pairs; in LDS it is one flat [m][r][p] array of 17-dword
// pairs. Loads are issued into registers first (so they are in flight while
// the workgroup does other work) and written to LDS later.
constexpr int kMaxV4 = 5;   // 16-byte loads per thread (tile <= 256 pairs = 17408 bytes)

struct WStage {
    u32x4 v[kMaxV4];
};

// Block format of the pairs a kernel instance decodes (PairMode): fixed for
// PM_Q8 / PM_Q5, the tile's own (sh.pb) for PM_MIXED.
template <int PM>
__device__ __forceinline__ bool pm_q5(const GemvShape &sh) {
    return PM == PM_Q5 || (PM == PM_MIXED && sh.pb == kQ5PairBytes);
}
template <int PM>
__device__ __forceinline__ int pm_pair_bytes(const GemvShape &sh) {
    return PM == PM_Q8 ? kPairBytes : PM == PM_Q5 ? kQ5PairBytes : sh.pb;
}
template <int PM>
__device__ __forceinline__ int pm_pair_dwords(const GemvShape &sh) {
    return pm_pair_bytes<PM>(sh) / 4;
}

// Whether chunk tiles can be moved with 16-byte loads (all pieces 16-byte
// aligned and whole). Otherwise (only ragged edge tiles of some shapes) the
// tile is copied with 4-byte loads at store time (pairs are 4-byte aligned).
__device__ inline bool tile_vec(const CoreArgs &a, int nrows) {
    const GemvShape &sh = a.sh;
    if (sh.PC == sh.P) return ((size_t(a.row0) * sh.rowbytes) % 16 == 0) && ((nrows * sh.rowbytes) % 16 == 0);
    return (sh.PC % 4 == 0) && (sh.P % 4 == 0);
}

template <int PM>
__device__ inline const uint8_t *tile_src(const CoreArgs &a, int nrows, int c, int i, int unit) {
    // i indexes `unit`-byte pieces of the flat tile
    const GemvShape &sh = a.sh;
    if (sh.PC == sh.P) {
        const int per_mat = nrows * sh.rowbytes / unit;
        const int m = i >= per_mat ? 1 : 0;
        return a.W[m] + size_t(a.row0) * sh.rowbytes + size_t(i - m * per_mat) * unit;
    }
    const int pb = pm_pair_bytes<PM>(sh);
    const int per_row = sh.PC * pb / unit;
    const int per_mat = nrows * per_row;
    const int m = i >= per_mat ? 1 : 0;
    const int ii = i - m * per_mat;
    const int r = ii / per_row, j = ii - r * per_row;
    return a.W[m] + size_t(a.row0 + r) * sh.rowbytes + size_t(c) * sh.PC * pb + size_t(j) * unit;
}

template <int PM>
__device__ inline void stage_issue(const CoreArgs &a, int nrows, int c, bool vec, WStage &st) {
    if (!vec) return;
    const int tid = threadIdx.x;
    const int n16 = a.nmat * nrows * a.sh.PC * pm_pair_bytes<PM>(a.sh) / 16;
#pragma unroll
    for (int k = 0; k < kMaxV4; ++k) {
        const int i = tid + k * kThreads;
        if (i < n16)
            st.v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(tile_src<PM>(a, nrows, c, i, 16)));
    }
}

template <int PM>
__device__ inline void stage_store(const CoreArgs &a, int nrows, int c, bool vec, const WStage &st,
                                   uint32_t *wt) {
    const int tid = threadIdx.x;
    const int bytes = a.nmat * nrows * a.sh.PC * pm_pair_bytes<PM>(a.sh);
    if (vec) {
        u32x4 *d = reinterpret_cast<u32x4 *>(wt);
#pragma unroll
        for (int k = 0; k < kMaxV4; ++k) {
            const int i = tid + k * kThreads;
            if (i < bytes / 16) d[i] = st.v[k];
        }
    } else {
#pragma unroll 1
        for (int i = tid; i < bytes / 4; i += kThreads)
            wt[i] = *reinterpret_cast<const uint32_t *>(tile_src<PM>(a, nrows, c, i, 4));
    }
}

// Computes outv[(t*nmat + m)*NR + r] = sum_k W_m[row0+r][k] * U[t][k].
//   U = X, or rmsnorm(X) * norm_w when norm_w is set.
// Timeline: chunk-0 weight loads are issued first; the activation row is
// read (and its norm computed) while they are in flight; chunk c+1's loads
// are issued before chunk c is computed.
template <int MAXT, bool MULTI, int PM>
__device__ void gemv_core(const CoreArgs &a, const Lds &l) {
    const int tid = threadIdx.x;
    const GemvShape &sh = a.sh;
    const int nrows = min(sh.NR, a.N - a.row0);
    const int per_mat = nrows * sh.PC;
    const int units = a.nmat * per_mat;
    const int nchunks = MULTI ? sh.P / sh.PC : 1;
    const bool x_full = (nchunks == 1);   // the whole activation row fits in one staging
    const bool vec = tile_vec(a, nrows);

    WStage st;
    stage_issue<PM>(a, nrows, 0, vec, st);

    // Stage x for chunk c (all of K when x_full); rinv must be ready if norm.
    auto stage_x = [&](int c, bool normalize) {
        const int n4 = a.Tc * sh.PC * 16;
        for (int e = tid; e < n4; e += kThreads) {
            const int t = e / (sh.PC * 16);
            const int rem = e - t * sh.PC * 16;
            const int p = rem >> 4;
            const int i4 = rem & 15;
            const int k = (c * sh.PC + p) * kPairWeights + i4 * 4;
            float4 v = *reinterpret_cast<const float4 *>(a.X + size_t(t) * a.ldx + k);
            if (normalize) {
                const float r = l.rinv[t];
                const float4 w = *reinterpret_cast<const float4 *>(a.norm_w + k);
                v.x = v.x * r * w.x;
                v.y = v.y * r * w.y;
                v.z = v.z * r * w.z;
                v.w = v.w * r * w.w;
            }
            *reinterpret_cast<float4 *>(l.xs + (size_t(t) * sh.PC + p) * kXPad + i4 * 4) = v;
        }
    };

    if (a.norm_w) {
        // Sum of squares for every token at once: all activation loads are in
        // flight together, then one reduction (per-token partials in fixed order).
        float ss[MAXT];
#pragma unroll
        for (int t = 0; t < MAXT; ++t) ss[t] = 0.f;
        const int n4row = x_full ? sh.PC * 16 : sh.K / 4;
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            if (t < a.Tc) {
                for (int e = tid; e < n4row; e += kThreads) {
                    const float4 v = *reinterpret_cast<const float4 *>(a.X + size_t(t) * a.ldx + e * 4);
                    if (x_full) {
                        const int p = e >> 4, i4 = e & 15;
                        *reinterpret_cast<float4 *>(l.xs + (size_t(t) * sh.PC + p) * kXPad + i4 * 4) = v;
                    }
                    ss[t] = fmaf(v.x, v.x, ss[t]);
                    ss[t] = fmaf(v.y, v.y, ss[t]);
                    ss[t] = fmaf(v.z, v.z, ss[t]);
                    ss[t] = fmaf(v.w, v.w, ss[t]);
                }
            }
        }
        float *red = l.outv;  // MAXT * nmat * NR >= 4 * MAXT floats of scratch until the end
        const int lane0 = tid & 63, wid0 = tid >> 6;
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            const float v = wave_sum(ss[t]);
            if (lane0 == 0) red[wid0 * MAXT + t] = v;
        }
        __syncthreads();
        if (tid < a.Tc) {
            const float tot = (red[tid] + red[MAXT + tid]) + (red[2 * MAXT + tid] + red[3 * MAXT + tid]);
            l.rinv[tid] = 1.0f / sqrtf(tot / static_cast<float>(sh.K) + a.eps);
        }
        __syncthreads();
        if (x_full) {
            const int n4 = a.Tc * sh.PC * 16;
            for (int e = tid; e < n4; e += kThreads) {
                const int t = e / (sh.PC * 16);
                const int rem = e - t * sh.PC * 16;
                const int p = rem >> 4, i4 = rem & 15;
                float4 *xp = reinterpret_cast<float4 *>(l.xs + (size_t(t) * sh.PC + p) * kXPad + i4 * 4);
                const float4 w = *reinterpret_cast<const float4 *>(a.norm_w + p * kPairWeights + i4 * 4);
                const float r = l.rinv[t];
                float4 v = *xp;
                v.x = v.x * r * w.x;
                v.y = v.y * r * w.y;
                v.z = v.z * r * w.z;
                v.w = v.w * r * w.w;
                *xp = v;
            }
        }
    } else if (x_full) {
        stage_x(0, false);
    }

    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = 0.f;
    int up = 0;
    if (tid < units) up = (tid % per_mat) % sh.PC;

    for (int c = 0; c < nchunks; ++c) {
        if (!x_full) stage_x(c, a.norm_w != nullptr);
        stage_store<PM>(a, nrows, c, vec, st, l.wt);
        if (MULTI && c + 1 < nchunks) stage_issue<PM>(a, nrows, c + 1, vec, st);
        __syncthreads();
        if (tid < units) {
            const uint32_t *wp = l.wt + size_t(tid) * pm_pair_dwords<PM>(sh);
            const bool q5 = pm_q5<PM>(sh);
            if constexpr (MAXT == 1) {
                float dA, sA, dB, sB;
                if (q5)
                    pair_dot1_q5(wp, l.xs + size_t(up) * kXPad, dA, sA, dB, sB);
                else
                    pair_dot1(wp, l.xs + size_t(up) * kXPad, dA, sA, dB, sB);
                acc[0] = fmaf(dA, sA, acc[0]);
                acc[0] = fmaf(dB, sB, acc[0]);
            } else {
                PairQ pq;
                if (q5)
                    decode_pair_q5(wp, pq);
                else
                    decode_pair(wp, pq);
#pragma unroll
                for (int t = 0; t < MAXT; ++t) {
                    if (t < a.Tc) {
                        const float *x = l.xs + (size_t(t) * sh.PC + up) * kXPad;
                        acc[t] = fmaf(pq.dA, block_dot(pq.q, x), acc[t]);
                        acc[t] = fmaf(pq.dB, block_dot(pq.q + 32, x + 32), acc[t]);
                    }
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
    int rope_neox;       // 1: q and k are written unrotated (a separate kernel rotates them)
    // Decode of layer 0: the input row is the token's embedding (Q8_0 row of
    // embed, token from st), dequantized here; workgroup 0 also writes it to
    // xres (the residual). NULL: the row is read from x.
    const uint8_t *embed;
    float *xres;
    int V;
    PartSrc ps;          // decode: split-K partials added to x first (n = 0: none)
    int pb[3];           // pair bytes of q, k, v (68 Q8_0, 44 Q5_0)
    // several tokens (a prefill): set to 1 when a written q, k or v value is
    // outside the f16 pairs' range of the prefill attention (NEOX q and k are
    // checked by the kernel that rotates them)
    uint32_t *range_flag;
};

template <int MAXT, bool MULTI, int PM>
__device__ __forceinline__ void qkv_multi(QkvArgs a) {
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
    c.sh.pb = (kind == 0 ? a.pb[0] : kind == 1 ? a.pb[1] : a.pb[2]);
    c.sh.rowbytes = a.sh.P * (kind == 0 ? a.pb[0] : kind == 1 ? a.pb[1] : a.pb[2]);
    c.row0 = tile * a.sh.NR; c.Tc = min(MAXT, a.T - t0);
    c.X = a.x + size_t(t0) * a.sh.K; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<MAXT, MULTI, PM>(c, l);

    const int nrows = min(a.sh.NR, N - c.row0);
    const int half = nrows >> 1;
    const int pos0 = a.st->pos + t0, slot0 = a.st->slot + t0;
    bool bad = false;
    for (int e = threadIdx.x; e < c.Tc * half; e += kThreads) {
        const int t = e / half;
        const int r = 2 * (e - t * half);
        const float a0 = l.outv[t * a.sh.NR + r], a1 = l.outv[t * a.sh.NR + r + 1];
        const int row = c.row0 + r;
        const int d = row % a.hd;
        if (kind == 2 || a.rope_neox) {
            float *dst = kind == 0   ? a.q + size_t(t0 + t) * a.QD + row
                         : kind == 1 ? a.kc + (size_t(row / a.hd) * a.max_seq + slot0 + t) * a.hd + d
                                     : a.vc + (size_t(row / a.hd) * a.max_seq + slot0 + t) * a.hd + d;
            if (kind == 2) bad |= !(fabsf(a0) < kPairRange) || !(fabsf(a1) < kPairRange);
            dst[0] = a0;
            dst[1] = a1;
        } else {
            const float2 cs = a.rope[size_t(pos0 + t) * (a.hd / 2) + (d >> 1)];
            const float b0 = a0 * cs.x - a1 * cs.y;
            const float b1 = a0 * cs.y + a1 * cs.x;
            float *dst = (kind == 0)
                             ? a.q + size_t(t0 + t) * a.QD + row
                             : a.kc + (size_t(row / a.hd) * a.max_seq + slot0 + t) * a.hd + d;
            bad |= !(fabsf(b0) < kPairRange) || !(fabsf(b1) < kPairRange);
            dst[0] = b0;
            dst[1] = b1;
        }
    }
    if (bad && a.range_flag) *a.range_flag = 1u;
}

// One kernel per block-format mode (PairMode) of each body below.
template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_qkv(QkvArgs a) { qkv_multi<MAXT, MULTI, PM_Q8>(a); }
template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_qkv_q5(QkvArgs a) { qkv_multi<MAXT, MULTI, PM_Q5>(a); }
template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_qkv_mixed(QkvArgs a) { qkv_multi<MAXT, MULTI, PM_MIXED>(a); }

// ---------------------------------------------------------------- gate/up

struct GateUpArgs {
    const uint8_t *wg, *wu;
    const float *norm_w;
    const float *x;
    float *h;  // [T][F]
    GemvShape sh;
    int F, T;
    float eps;
    PartSrc ps;  // decode: split-K partials added to x first (n = 0: none)
};

template <int MAXT, bool MULTI, int PM>
__device__ __forceinline__ void gateup_multi(const GateUpArgs &a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds l = carve(smem, a.sh, 2, MAXT);
    const int t0 = blockIdx.y * MAXT;
    CoreArgs c;
    c.W[0] = a.wg; c.W[1] = a.wu; c.nmat = 2; c.sh = a.sh; c.N = a.F;
    c.row0 = blockIdx.x * a.sh.NR; c.Tc = min(MAXT, a.T - t0);
    c.X = a.x + size_t(t0) * a.sh.K; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<MAXT, MULTI, PM>(c, l);
    const int nrows = min(a.sh.NR, a.F - c.row0);
    for (int e = threadIdx.x; e < c.Tc * nrows; e += kThreads) {
        const int t = e / nrows, r = e - t * nrows;
        const float g = l.outv[(t * 2 + 0) * a.sh.NR + r];
        const float u = l.outv[(t * 2 + 1) * a.sh.NR + r];
        a.h[size_t(t0 + t) * a.F + c.row0 + r] = silu(g) * u;
    }
}

template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_gateup(GateUpArgs a) { gateup_multi<MAXT, MULTI, PM_Q8>(a); }
template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_gateup_q5(GateUpArgs a) { gateup_multi<MAXT, MULTI, PM_Q5>(a); }

// ---------------------------------------------------------------- generic (o, down, op)

struct MatmulArgs {
    const uint8_t *W;
    const float *norm_w;
    const float *x;
    float *y;  // [T][N]
    GemvShape sh;
    int N, T, accumulate;
    float eps;
    const float *mpart;      // decode only: merge x from attention partials (see CoreArgs)
    int msplits, mhd;
    const StepState *mst;
};

template <int MAXT, bool MULTI, int PM>
__device__ __forceinline__ void matmul_multi(const MatmulArgs &a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds l = carve(smem, a.sh, 1, MAXT);
    const int t0 = blockIdx.y * MAXT;
    CoreArgs c;
    c.W[0] = a.W; c.W[1] = nullptr; c.nmat = 1; c.sh = a.sh; c.N = a.N;
    c.row0 = blockIdx.x * a.sh.NR; c.Tc = min(MAXT, a.T - t0);
    c.X = a.x + size_t(t0) * a.sh.K; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    gemv_core<MAXT, MULTI, PM>(c, l);
    const int nrows = min(a.sh.NR, a.N - c.row0);
    for (int e = threadIdx.x; e < c.Tc * nrows; e += kThreads) {
        const int t = e / nrows, r = e - t * nrows;
        float *dst = a.y + size_t(t0 + t) * a.N + c.row0 + r;
        const float v = l.outv[t * a.sh.NR + r];
        *dst = a.accumulate ? *dst + v : v;
    }
}

template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_matmul(MatmulArgs a) { matmul_multi<MAXT, MULTI, PM_Q8>(a); }
template <int MAXT, bool MULTI>
__global__ __launch_bounds__(kThreads) void k_matmul_q5(MatmulArgs a) { matmul_multi<MAXT, MULTI, PM_Q5>(a); }

// ---------------------------------------------------------------- output layer + argmax

struct LmHeadArgs {
    const uint8_t *W;
    const float *norm_w;
    const float *x;      // [H], the last position
    StepState *st;
    float *partials;     // [gridDim.x][2] (value, index bits)
    GemvShape sh;
    int V;
    float eps;
    PartSrc ps;          // split-K partials added to x first (n = 0: none)
};

// Merge n (value, index) partials in a fixed order; lowest index on ties.
__device__ void argmax_reduce(const float *partials, int n, float &bv, uint32_t &bi) {
    __shared__ float red[4];
    __shared__ uint32_t redi[4];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float v = -INFINITY;
    uint32_t i = 0xffffffffu;
    for (int b = tid; b < n; b += kThreads)
        argmax_merge(v, i, partials[2 * b], __float_as_uint(partials[2 * b + 1]));
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

// One workgroup: final argmax of the output layer, then the step state
// update used by on-device generation (the picked id becomes the next input).
__global__ __launch_bounds__(kThreads) void k_argmax_finish(const float *partials, int n, StepState *st) {
    float v;
    uint32_t i;
    argmax_reduce(partials, n, v, i);
    if (threadIdx.x == 0) {
        if (st->argmax_out) *st->argmax_out = i;
        if (st->advance) {
            if (st->ids_out) st->ids_out[st->step] = i;
            st->token = i;
            st->pos += 1;
            st->slot += 1;
            st->step += 1;
        }
    }
}

// Standalone argmax: per-workgroup partials, then a one-workgroup merge.
__global__ __launch_bounds__(kThreads) void k_argmax_part(const float *x, int64_t n, float *partials) {
    __shared__ float s_red[4];
    __shared__ uint32_t s_redi[4];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t per = 4096;
    const int64_t b0 = int64_t(blockIdx.x) * per;
    const int64_t e = min(n, b0 + per);
    float bv = -INFINITY;
    uint32_t bi = uint32_t(b0);
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
    }
}

__global__ __launch_bounds__(kThreads) void k_argmax_out(const float *partials, int n, uint32_t *out) {
    float v;
    uint32_t i;
    argmax_reduce(partials, n, v, i);
    if (threadIdx.x == 0) *out = i;
}

// ---------------------------------------------------------------- decode (T = 1)
//
// A decode workgroup stages the whole activation row once (normalised when
// a norm comes first) and then walks row tiles
// blockIdx.x, blockIdx.x + gridDim.x, ...: the next tile's weights are issued
// into registers while the current tile is computed, so the weight stream
// never waits on the activation staging and the row is read once per
// workgroup instead of once per tile.

struct Lds1 {
    uint32_t *wt;   // nmat*NR*PC*17 dwords (reused for partials)
    float *xs;      // P*kXPad: the whole activation row
    float *outv;    // max(nmat*NR, 4)
    float *red;     // 4
};

__host__ __device__ inline size_t lds1_bytes(const GemvShape &sh, int nmat) {
    size_t b = align16(size_t(nmat) * sh.NR * sh.PC * kPairBytes);
    b += align16(size_t(sh.P) * kXPad * 4);
    b += align16((size_t(nmat) * sh.NR > 4 ? size_t(nmat) * sh.NR : 4) * 4);
    b += 16;
    return b;
}

__device__ inline Lds1 carve1(uint8_t *smem, const GemvShape &sh, int nmat) {
    Lds1 l;
    size_t off = 0;
    l.wt = reinterpret_cast<uint32_t *>(smem + off);
    off += align16(size_t(nmat) * sh.NR * sh.PC * kPairBytes);
    l.xs = reinterpret_cast<float *>(smem + off);
    off += align16(size_t(sh.P) * kXPad * 4);
    l.outv = reinterpret_cast<float *>(smem + off);
    off += align16((size_t(nmat) * sh.NR > 4 ? size_t(nmat) * sh.NR : 4) * 4);
    l.red = reinterpret_cast<float *>(smem + off);
    return l;
}

// The attention output, merged from the split partials of the decode
// attention, into xs in pair layout: for head h and split s with (m_s, l_s,
// o_s), o[d] = sum_s w_s o_s[d] / sum_s w_s l_s with w_s = exp(m_s - M), M the
// largest m_s, sums in split order (what k_attn_combine computes). Every
// split's values are loaded before any is used, and before the number of
// splits in use (from the step state) is known: indexes past the launch's
// splits re-read its last one, and splits past the ones in use are not
// summed.
__device__ void stage_merged1(const CoreArgs &a, const MergeSrc &ms, const Lds1 &l) {
    const int hd = ms.hd, S = ms.splits;
    const int C = attn_chunk(hd);
    const int n4 = a.sh.P * 16;
    for (int e = threadIdx.x; e < n4; e += kThreads) {
        const int k = 4 * e, h = k / hd, d = k - h * hd;
        const float *pb = ms.part + size_t(h) * S * (hd + 2);
        float m[kMergeMaxSplits], ls[kMergeMaxSplits], o[kMergeMaxSplits][4];
#pragma unroll
        for (int s = 0; s < kMergeMaxSplits; ++s) {
            const float *ps = pb + size_t(min(s, S - 1)) * (hd + 2);
            m[s] = ps[0];
            ls[s] = ps[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[s][i] = ps[2 + d + i];
        }
        const int active = min((ms.st->slot + 1 + C - 1) / C, S);
        float M = m[0];
#pragma unroll
        for (int s = 1; s < kMergeMaxSplits; ++s)
            if (s < active) M = fmaxf(M, m[s]);
        float sum = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kMergeMaxSplits; ++s) {
            if (s < active) {
                const float w = expf(m[s] - M);
                sum = fmaf(w, ls[s], sum);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, o[s][i], acc[i]);
            }
        }
        const float inv = 1.0f / sum;
        *reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4) =
            float4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    }
}

constexpr int kStage4 = 4;   // float4 of the row per thread held in registers (rows of <= 4096)

// The whole row u (K values) into xs in pair layout; the caller syncs.
// With a norm and rows of 1025 to kStage4 * 1024 values, the row and the norm
// weights are loaded into registers together (one memory round trip before
// the sum of squares instead of a second one after it); the arithmetic is
// the same, in the same order, as the general path below. Measured: 7B-class
// decode (rows of 4096) 2601 -> 2554 us/token; with the 135M shape's rows of
// 576 it was slower (694 -> 700), so short rows keep the general path.
constexpr int kPartBatch = 4;   // split-K partial rows loaded together (all in flight before the sum)

// v + (p_0 + p_1 + ... + p_{n-1}) for the float4 at e (partials summed in
// index order, then added to v); kPartBatch loads are issued before any is
// used (indexes past n re-read the last partial and are not summed).
__device__ __forceinline__ float4 add_partials(float4 v, const PartSrc &ps, int e) {
    const float *pp = ps.part + size_t(e) * 4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < ps.n; i0 += kPartBatch) {
        float4 t[kPartBatch];
#pragma unroll
        for (int i = 0; i < kPartBatch; ++i)
            t[i] = *reinterpret_cast<const float4 *>(pp + size_t(min(i0 + i, ps.n - 1)) * ps.stride);
#pragma unroll
        for (int i = 0; i < kPartBatch; ++i) {
            if (i0 + i == 0) {
                acc = t[0];
            } else if (i0 + i < ps.n) {
                acc.x += t[i].x;
                acc.y += t[i].y;
                acc.z += t[i].z;
                acc.w += t[i].w;
            }
        }
    }
    return make_float4(v.x + acc.x, v.y + acc.y, v.z + acc.z, v.w + acc.w);
}

__device__ void stage_row1(const CoreArgs &a, const Lds1 &l, PartSrc ps = PartSrc{}) {
    const int tid = threadIdx.x;
    const int n4 = a.sh.P * 16;
    if (a.norm_w && ps.n == 0 && n4 > kThreads && n4 <= kStage4 * kThreads) {
        float4 xv[kStage4], wv[kStage4];
#pragma unroll
        for (int i = 0; i < kStage4; ++i) {   // indexes past the row re-read its last float4 (unused)
            const int e = min(tid + i * kThreads, n4 - 1);
            xv[i] = *reinterpret_cast<const float4 *>(a.X + size_t(e) * 4);
            wv[i] = *reinterpret_cast<const float4 *>(a.norm_w + size_t(e) * 4);
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < kStage4; ++i) {
            if (tid + i * kThreads < n4) {
                const float4 v = xv[i];
                ss = fmaf(v.x, v.x, ss);
                ss = fmaf(v.y, v.y, ss);
                ss = fmaf(v.z, v.z, ss);
                ss = fmaf(v.w, v.w, ss);
            }
        }
        ss = block_sum(ss, l.red);
        const float r = 1.0f / sqrtf(ss / static_cast<float>(a.sh.K) + a.eps);
#pragma unroll
        for (int i = 0; i < kStage4; ++i) {
            const int e = tid + i * kThreads;
            if (e < n4) {
                float4 v = xv[i];
                const float4 w = wv[i];
                v.x = v.x * r * w.x;
                v.y = v.y * r * w.y;
                v.z = v.z * r * w.z;
                v.w = v.w * r * w.w;
                *reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4) = v;
            }
        }
        return;
    }
    if (n4 <= kThreads) {
        // Rows of at most kThreads float4: one per thread, its norm weights
        // (and any partial sums) loaded with it, so the row costs one memory
        // round trip; the values and their order are the general path's.
        const int e = tid;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f), w = v;
        if (e < n4) {
            v = *reinterpret_cast<const float4 *>(a.X + size_t(e) * 4);
            if (a.norm_w) w = *reinterpret_cast<const float4 *>(a.norm_w + size_t(e) * 4);
            if (ps.n > 0) {
                v = add_partials(v, ps, e);
                if (ps.xout && blockIdx.x == 0) *reinterpret_cast<float4 *>(ps.xout + size_t(e) * 4) = v;
            }
        }
        float4 *xp = reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4);
        if (!a.norm_w) {
            if (e < n4) *xp = v;
            return;
        }
        float ss = 0.f;
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
        ss = block_sum(ss, l.red);
        const float r = 1.0f / sqrtf(ss / static_cast<float>(a.sh.K) + a.eps);
        if (e < n4) {
            v.x = v.x * r * w.x;
            v.y = v.y * r * w.y;
            v.z = v.z * r * w.z;
            v.w = v.w * r * w.w;
            *xp = v;
        }
        return;
    }
    float ss = 0.f;
    for (int e = tid; e < n4; e += kThreads) {
        float4 v = *reinterpret_cast<const float4 *>(a.X + size_t(e) * 4);
        if (ps.n > 0) {
            v = add_partials(v, ps, e);
            if (ps.xout && blockIdx.x == 0) *reinterpret_cast<float4 *>(ps.xout + size_t(e) * 4) = v;
        }
        *reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4) = v;
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    if (!a.norm_w) return;
    ss = block_sum(ss, l.red);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(a.sh.K) + a.eps);
    for (int e = tid; e < n4; e += kThreads) {
        float4 *xp = reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4);
        const float4 w = *reinterpret_cast<const float4 *>(a.norm_w + size_t(e) * 4);
        float4 v = *xp;
        v.x = v.x * r * w.x;
        v.y = v.y * r * w.y;
        v.z = v.z * r * w.z;
        v.w = v.w * r * w.w;
        *xp = v;
    }
}

// Products of a small single-chunk tile (the whole row staged): wave w takes
// rows w, w + 4, ... of the tile; lane l takes the row's weights l, l + 64,
// ... (byte l % 32 of block 2i + l / 32 for pair i) and accumulates
// (d * q) * u (d * q is exact in f32) in pair order; the lanes are summed
// by wave_sum_dpp. Fewer barriers and a short chain per lane, for tiles that
// would leave most threads idle one pair per thread.
template <int PM>
__device__ __forceinline__ void rows_dot1(const CoreArgs &c, const Lds1 &l, int nrows) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const GemvShape &sh = c.sh;
    const int items = c.nmat * nrows;
    constexpr int W = kThreads / 64;
    auto put = [&](int it, float v) {
        if (lane == 0) {
            const int m = it / nrows, r = it - m * nrows;
            l.outv[m * sh.NR + r] = v;
        }
    };
    if (pm_q5<PM>(sh)) {
        // Q5_0: weight j = lane % 32 of block 2i + lane / 32 (nibble j / 16 of
        // byte 6 + j % 16, fifth bit j of the word at byte 2)
        const uint8_t *wt = reinterpret_cast<const uint8_t *>(l.wt) + (lane >> 5) * kQ5Bytes;
        const int j = lane & 31;
        for (int it = wid; it < items; it += W) {
            const uint8_t *row = wt + size_t(it) * sh.PC * kQ5PairBytes;
            float acc = 0.f;
#pragma unroll 4
            for (int i = 0; i < sh.P; ++i) {
                const uint8_t *blk = row + i * kQ5PairBytes;
                const float d = half_bits_to_float(*reinterpret_cast<const uint16_t *>(blk));
                const uint32_t qh = uint32_t(*reinterpret_cast<const uint16_t *>(blk + 2)) |
                                    (uint32_t(*reinterpret_cast<const uint16_t *>(blk + 4)) << 16);
                const int q5 = ((blk[6 + (j & 15)] >> (4 * (j >> 4))) & 15) | int(((qh >> j) & 1u) << 4);
                acc = fmaf(d * static_cast<float>(q5 - 16), l.xs[i * kXPad + lane], acc);
            }
            put(it, wave_sum_dpp(acc));
        }
        return;
    }
    const uint8_t *wt = reinterpret_cast<const uint8_t *>(l.wt) + (lane >> 5) * kQBytes;
    const int o = lane & 31;
    int it = wid;
    // rows it and it + W together while both exist (one read of u for two rows)
    for (; it + W < items; it += 2 * W) {
        const uint8_t *ra = wt + size_t(it) * sh.PC * kPairBytes;
        const uint8_t *rb = wt + size_t(it + W) * sh.PC * kPairBytes;
        float acc = 0.f, acc2 = 0.f;
#pragma unroll 8
        for (int i = 0; i < sh.P; ++i) {
            const uint8_t *ba = ra + i * kPairBytes, *bb = rb + i * kPairBytes;
            const float u = l.xs[i * kXPad + lane];
            const float da = half_bits_to_float(*reinterpret_cast<const uint16_t *>(ba));
            const float db = half_bits_to_float(*reinterpret_cast<const uint16_t *>(bb));
            acc = fmaf(da * static_cast<float>(static_cast<int8_t>(ba[2 + o])), u, acc);
            acc2 = fmaf(db * static_cast<float>(static_cast<int8_t>(bb[2 + o])), u, acc2);
        }
        put(it, wave_sum_dpp(acc));
        put(it + W, wave_sum_dpp(acc2));
    }
    for (; it < items; it += W) {
        const uint8_t *row = wt + size_t(it) * sh.PC * kPairBytes;
        float acc = 0.f;
#pragma unroll 8
        for (int i = 0; i < sh.P; ++i) {
            const uint8_t *blk = row + i * kPairBytes;
            const float d = half_bits_to_float(*reinterpret_cast<const uint16_t *>(blk));
            const float q = static_cast<float>(static_cast<int8_t>(blk[2 + o]));
            acc = fmaf(d * q, l.xs[i * kXPad + lane], acc);
        }
        put(it, wave_sum_dpp(acc));
    }
}

// One row tile: outv[m*NR + r] = sum_k W_m[row0+r][k] * u[k]. Chunk 0 of this
// tile is already in `st`; the next tile's chunk 0 is issued during the last
// chunk (when has_next).
template <bool MULTI, int PM>
__device__ void tile_run1(const CoreArgs &c, const Lds1 &l, int nrows, bool vec, WStage &st,
                          const CoreArgs &n, int nn, bool nvec, bool has_next) {
    const int tid = threadIdx.x;
    const GemvShape &sh = c.sh;
    const int per_mat = nrows * sh.PC;
    const int units = c.nmat * per_mat;
    if constexpr (!MULTI) {
        if (2 * units <= kThreads) {
            stage_store<PM>(c, nrows, 0, vec, st, l.wt);
            if (has_next) stage_issue<PM>(n, nn, 0, nvec, st);
            __syncthreads();
            rows_dot1<PM>(c, l, nrows);
            __syncthreads();
            return;
        }
    }
    const int nchunks = MULTI ? sh.P / sh.PC : 1;
    const int up = tid < units ? (tid % per_mat) % sh.PC : 0;
    float acc = 0.f;
    for (int ch = 0; ch < nchunks; ++ch) {
        stage_store<PM>(c, nrows, ch, vec, st, l.wt);
        if (MULTI && ch + 1 < nchunks)
            stage_issue<PM>(c, nrows, ch + 1, vec, st);
        else if (has_next)
            stage_issue<PM>(n, nn, 0, nvec, st);
        __syncthreads();
        if (tid < units) {
            float dA, sA, dB, sB;
            const uint32_t *wp = l.wt + size_t(tid) * pm_pair_dwords<PM>(sh);
            const float *xp = l.xs + size_t(ch * sh.PC + up) * kXPad;
            if (pm_q5<PM>(sh))
                pair_dot1_q5(wp, xp, dA, sA, dB, sB);
            else
                pair_dot1(wp, xp, dA, sA, dB, sB);
            acc = fmaf(dA, sA, acc);
            acc = fmaf(dB, sB, acc);
        }
        __syncthreads();
    }
    float *part = reinterpret_cast<float *>(l.wt);
    if (tid < units) part[tid] = acc;
    __syncthreads();
    const int lane = tid & 63, wid = tid >> 6;
    const int items = c.nmat * nrows;
    for (int it = wid; it < items; it += 4) {
        const float *src = part + size_t(it) * sh.PC;
        float v = 0.f;
        for (int p = lane; p < sh.PC; p += 64) v += src[p];
        v = wave_sum(v);
        if (lane == 0) {
            const int m = it / nrows, r = it - m * nrows;
            l.outv[m * sh.NR + r] = v;
        }
    }
    __syncthreads();
}

__device__ inline int tile_rows(const CoreArgs &c) { return min(c.sh.NR, c.N - c.row0); }

// The workgroup's tiles blockIdx.x, +G, +2G, ... (G = gridDim.x) with two
// tiles' weights in flight: tile t + 2G is issued as soon as tile t's
// weights are in LDS, into the registers tile t used (two register stages,
// alternating). The activation row is staged while the first two tiles load.
// epi(tile, rows) consumes outv after each tile.
template <bool MULTI, bool MERGE, int PM, class Epi>
__device__ __forceinline__ void walk_tiles2(const CoreArgs &c, const Lds1 &l, int ntiles, Epi &&epi,
                                            const MergeSrc *ms = nullptr, PartSrc ps = PartSrc{}) {
    const int G = int(gridDim.x);
    auto at = [&](int t, CoreArgs &x, int &nr, bool &v) {
        x = c;
        x.row0 = t * c.sh.NR;
        nr = t < ntiles ? tile_rows(x) : 0;
        v = nr > 0 ? tile_vec(x, nr) : false;
    };
    int t = blockIdx.x;
    CoreArgs ca, cb, n;
    int na, nb, nn;
    bool va, vb, nv;
    at(t, ca, na, va);
    at(t + G, cb, nb, vb);
    WStage sa, sb;
    if (na > 0) stage_issue<PM>(ca, na, 0, va, sa);
    if (nb > 0) stage_issue<PM>(cb, nb, 0, vb, sb);
    if constexpr (MERGE)
        stage_merged1(c, *ms, l);
    else
        stage_row1(c, l, ps);
    while (t < ntiles) {
        at(t + 2 * G, n, nn, nv);
        tile_run1<MULTI, PM>(ca, l, na, va, sa, n, nn, nv, nn > 0);
        epi(ca, na);
        ca = n; na = nn; va = nv;
        t += G;
        if (t >= ntiles) break;
        at(t + 2 * G, n, nn, nv);
        tile_run1<MULTI, PM>(cb, l, nb, vb, sb, n, nn, nv, nn > 0);
        epi(cb, nb);
        cb = n; nb = nn; vb = nv;
        t += G;
    }
}

// Layer 0 of a decode step: the embedding of the step's token (x = d * q per
// 32-weight block, as the embedding kernel computes it) staged and
// normalised as stage_row1's general path does (same values, same order);
// workgroup 0 writes the row to x, the residual the o-projection adds to. A
// token id past the vocabulary (only reachable through a device-side token)
// gives a zero row, as the embedding kernel does.
__device__ void stage_embed1(const QkvArgs &a, const CoreArgs &c, const Lds1 &l) {
    const int tid = threadIdx.x;
    const int n4 = c.sh.P * 16, H = c.sh.K;
    const uint32_t tok = a.st->token;
    const bool valid = tok < uint32_t(a.V);
    const uint8_t *row = a.embed + (valid ? size_t(tok) : 0) * (size_t(H) / kQK * kQBytes);
    float ss = 0.f;
    for (int e = tid; e < n4; e += kThreads) {
        const uint8_t *blk = row + size_t(e >> 3) * kQBytes;   // 8 float4 per 32-weight block
        const int i0 = (e & 7) * 4;
        const float d = half_bits_to_float(uint32_t(blk[0]) | (uint32_t(blk[1]) << 8));
        float4 v;
        v.x = valid ? d * static_cast<float>(static_cast<int8_t>(blk[2 + i0])) : 0.f;
        v.y = valid ? d * static_cast<float>(static_cast<int8_t>(blk[3 + i0])) : 0.f;
        v.z = valid ? d * static_cast<float>(static_cast<int8_t>(blk[4 + i0])) : 0.f;
        v.w = valid ? d * static_cast<float>(static_cast<int8_t>(blk[5 + i0])) : 0.f;
        *reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4) = v;
        if (blockIdx.x == 0) *reinterpret_cast<float4 *>(a.xres + size_t(e) * 4) = v;
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
        ss = fmaf(v.z, v.z, ss);
        ss = fmaf(v.w, v.w, ss);
    }
    ss = block_sum(ss, l.red);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(c.sh.K) + c.eps);
    for (int e = tid; e < n4; e += kThreads) {
        float4 *xp = reinterpret_cast<float4 *>(l.xs + (e >> 4) * kXPad + (e & 15) * 4);
        const float4 w = *reinterpret_cast<const float4 *>(c.norm_w + size_t(e) * 4);
        float4 v = *xp;
        v.x = v.x * r * w.x;
        v.y = v.y * r * w.y;
        v.z = v.z * r * w.z;
        v.w = v.w * r * w.w;
        *xp = v;
    }
}

template <bool MULTI, int PM>
__device__ __forceinline__ void qkv_one(const QkvArgs &a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds1 l = carve1(smem, a.sh, 1);
    const int ntiles = a.tq + 2 * a.tk;
    auto ref = [&](int tile, int &kind) {
        CoreArgs c{};
        c.nmat = 1; c.sh = a.sh; c.Tc = 1; c.X = a.x; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
        if (tile < a.tq) {
            kind = 0; c.W[0] = a.wq; c.N = a.QD;
        } else if (tile < a.tq + a.tk) {
            kind = 1; c.W[0] = a.wk; c.N = a.KVD; tile -= a.tq;
        } else {
            kind = 2; c.W[0] = a.wv; c.N = a.KVD; tile -= a.tq + a.tk;
        }
        c.row0 = tile * a.sh.NR;
        c.sh.pb = (kind == 0 ? a.pb[0] : kind == 1 ? a.pb[1] : a.pb[2]);
        c.sh.rowbytes = a.sh.P * (kind == 0 ? a.pb[0] : kind == 1 ? a.pb[1] : a.pb[2]);
        return c;
    };
    int tile = blockIdx.x, kind;
    CoreArgs c = ref(tile, kind);
    int nrows = tile_rows(c);
    bool vec = tile_vec(c, nrows);
    WStage st;
    stage_issue<PM>(c, nrows, 0, vec, st);
    const int pos = a.st->pos, slot = a.st->slot;   // in flight with the weights and the row
    if (a.embed)
        stage_embed1(a, c, l);
    else
        stage_row1(c, l, a.ps);
    for (; tile < ntiles; tile += gridDim.x) {
        const bool has_next = tile + int(gridDim.x) < ntiles;
        int nkind = 0;
        CoreArgs n = has_next ? ref(tile + gridDim.x, nkind) : c;
        const int nn = has_next ? tile_rows(n) : 0;
        const bool nvec = has_next ? tile_vec(n, nn) : false;
        // Thread e writes rows 2e, 2e + 1 of the tile (nrows <= NR <= kThreads,
        // so one pair per thread); its rope factors are loaded before the
        // products, not after them.
        const int e = threadIdx.x;
        const bool rot = kind != 2 && !a.rope_neox;
        float2 cs = make_float2(1.f, 0.f);
        if (rot && e < nrows / 2) cs = a.rope[size_t(pos) * (a.hd / 2) + (((c.row0 + 2 * e) % a.hd) >> 1)];
        tile_run1<MULTI, PM>(c, l, nrows, vec, st, n, nn, nvec, has_next);
        if (e < nrows / 2) {
            const int r = 2 * e;
            const float a0 = l.outv[r], a1 = l.outv[r + 1];
            const int row = c.row0 + r;
            const int d = row % a.hd;
            if (!rot) {
                float *dst = kind == 0   ? a.q + row
                             : kind == 1 ? a.kc + (size_t(row / a.hd) * a.max_seq + slot) * a.hd + d
                                         : a.vc + (size_t(row / a.hd) * a.max_seq + slot) * a.hd + d;
                dst[0] = a0;
                dst[1] = a1;
            } else {
                const float b0 = a0 * cs.x - a1 * cs.y;
                const float b1 = a0 * cs.y + a1 * cs.x;
                float *dst = (kind == 0) ? a.q + row
                                         : a.kc + (size_t(row / a.hd) * a.max_seq + slot) * a.hd + d;
                dst[0] = b0;
                dst[1] = b1;
            }
        }
        c = n; nrows = nn; vec = nvec; kind = nkind;
    }
}

template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_qkv1(QkvArgs a) { qkv_one<MULTI, PM_Q8>(a); }
template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_qkv1_q5(QkvArgs a) { qkv_one<MULTI, PM_Q5>(a); }
template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_qkv1_mixed(QkvArgs a) { qkv_one<MULTI, PM_MIXED>(a); }

template <bool MULTI, int PM>
__device__ __forceinline__ void gateup_one(const GateUpArgs &a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds1 l = carve1(smem, a.sh, 2);
    const int ntiles = (a.F + a.sh.NR - 1) / a.sh.NR;
    CoreArgs c{};
    c.W[0] = a.wg; c.W[1] = a.wu; c.nmat = 2; c.sh = a.sh; c.N = a.F; c.Tc = 1;
    c.X = a.x; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    walk_tiles2<MULTI, false, PM>(
        c, l, ntiles,
        [&](const CoreArgs &t, int nrows) {
            for (int r = threadIdx.x; r < nrows; r += kThreads)
                a.h[t.row0 + r] = silu(l.outv[r]) * l.outv[a.sh.NR + r];
        },
        nullptr, a.ps);
}

template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_gateup1(GateUpArgs a) { gateup_one<MULTI, PM_Q8>(a); }
template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_gateup1_q5(GateUpArgs a) { gateup_one<MULTI, PM_Q5>(a); }

// Large K (several chunks), no norm: chunk-outer, tile-inner. Only one
// activation chunk is in LDS at a time (so more workgroups fit per CU); each
// thread keeps one accumulator per tile of its workgroup (at most kTilesPerWg)
// across chunks; the tiles are reduced and written at the end.
// The last chunk may be shorter than PC pairs (PC need not divide P: a
// multiple of 4 pairs keeps every piece 16-byte aligned). Thread u always
// takes pair u % PC of row u / PC, so its accumulator stays on one row; in
// LDS a tile keeps a row stride of PC pairs.
constexpr int kTilesPerWg = 8;
constexpr int kMaxX4 = 10;   // float4 of one activation chunk per thread (chunks of <= 160 pairs)

__device__ inline int chunk_pairs(const GemvShape &sh, int c) { return min(sh.PC, sh.P - c * sh.PC); }

// Piece i (of `unit` bytes) of chunk c's tile: source address and LDS byte offset.
template <int PM>
__device__ inline const uint8_t *ctile_src(const uint8_t *W, const GemvShape &sh, int row0, int pcc, int c, int i,
                                           int unit) {
    const int pb = pm_pair_bytes<PM>(sh);
    const int per_row = pcc * pb / unit;
    const int r = i / per_row, j = i - r * per_row;
    return W + size_t(row0 + r) * sh.rowbytes + size_t(c) * sh.PC * pb + size_t(j) * unit;
}
template <int PM>
__device__ inline int ctile_dst(const GemvShape &sh, int pcc, int i, int unit) {
    const int pb = pm_pair_bytes<PM>(sh);
    const int per_row = pcc * pb / unit;
    const int r = i / per_row, j = i - r * per_row;
    return r * sh.PC * pb + j * unit;
}
__device__ inline bool ctile_vec(const GemvShape &sh, int pcc) {
    return (pcc % 4 == 0) && (sh.PC % 4 == 0) && (sh.P % 4 == 0);
}
template <int PM>
__device__ inline void ctile_issue(const uint8_t *W, const GemvShape &sh, int row0, int nrows, int c, WStage &st) {
    const int pcc = chunk_pairs(sh, c);
    if (!ctile_vec(sh, pcc)) return;
    const int n16 = nrows * pcc * pm_pair_bytes<PM>(sh) / 16;
#pragma unroll
    for (int k = 0; k < kMaxV4; ++k) {
        const int i = threadIdx.x + k * kThreads;
        if (i < n16)
            st.v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ctile_src<PM>(W, sh, row0, pcc, c, i, 16)));
    }
}
template <int PM>
__device__ inline void ctile_store(const uint8_t *W, const GemvShape &sh, int row0, int nrows, int c,
                                   const WStage &st, uint32_t *wt) {
    const int pcc = chunk_pairs(sh, c);
    const int pb = pm_pair_bytes<PM>(sh);
    uint8_t *base = reinterpret_cast<uint8_t *>(wt);
    if (ctile_vec(sh, pcc)) {
        const int n16 = nrows * pcc * pb / 16;
#pragma unroll
        for (int k = 0; k < kMaxV4; ++k) {
            const int i = threadIdx.x + k * kThreads;
            if (i < n16) *reinterpret_cast<u32x4 *>(base + ctile_dst<PM>(sh, pcc, i, 16)) = st.v[k];
        }
    } else {
#pragma unroll 1
        for (int i = threadIdx.x; i < nrows * pcc * pb / 4; i += kThreads)
            *reinterpret_cast<uint32_t *>(base + ctile_dst<PM>(sh, pcc, i, 4)) =
                *reinterpret_cast<const uint32_t *>(ctile_src<PM>(W, sh, row0, pcc, c, i, 4));
    }
}

__host__ __device__ inline size_t lds1c_bytes(const GemvShape &sh) {
    return align16(size_t(sh.NR) * sh.PC * sh.pb) + align16(size_t(sh.PC) * kXPad * 4) +
           align16(size_t(sh.NR > 4 ? sh.NR : 4) * 4) + 16;
}

template <bool Q5>
__global__ __launch_bounds__(kThreads) void k_matmul1_chunked(MatmulArgs a) {
    constexpr int PM = Q5 ? PM_Q5 : PM_Q8;
    extern __shared__ __align__(16) uint8_t smem[];
    const GemvShape &sh = a.sh;
    uint32_t *wt = reinterpret_cast<uint32_t *>(smem);
    float *xs = reinterpret_cast<float *>(smem + align16(size_t(sh.NR) * sh.PC * pm_pair_bytes<PM>(sh)));
    float *outv = xs + align16(size_t(sh.PC) * kXPad * 4) / 4;
    const int tid = threadIdx.x;
    const int ntiles = (a.N + sh.NR - 1) / sh.NR;
    const int nchunks = (sh.P + sh.PC - 1) / sh.PC;
    const bool q5 = pm_q5<PM>(sh);
    int my_tiles = 0;
    for (int k = 0; k < kTilesPerWg; ++k) my_tiles += (int(blockIdx.x) + k * int(gridDim.x) < ntiles) ? 1 : 0;
    float acc[kTilesPerWg];
#pragma unroll
    for (int k = 0; k < kTilesPerWg; ++k) acc[k] = 0.f;

    int row0 = int(blockIdx.x) * sh.NR;
    int nrows = min(sh.NR, a.N - row0);
    WStage st;
    // The next chunk's activations are loaded into registers while the
    // current chunk's tiles are computed (indexes past a short last chunk
    // re-read its last float4; those registers are not stored).
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x4 xr[kMaxX4];
    {
        const int last = chunk_pairs(sh, 0) * 16 - 1;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(a.x);
#pragma unroll
        for (int i = 0; i < kMaxX4; ++i) xr[i] = src[min(tid + i * kThreads, last)];
    }
    ctile_issue<PM>(a.W, sh, row0, nrows, 0, st);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int pcc = chunk_pairs(sh, ch);
        __syncthreads();  // the previous chunk's activations are no longer read
        const int n4 = pcc * 16;
#pragma unroll
        for (int i = 0; i < kMaxX4; ++i) {
            const int e = tid + i * kThreads;
            if (e < n4) *reinterpret_cast<f32x4 *>(xs + (e >> 4) * kXPad + (e & 15) * 4) = xr[i];
        }
        if (ch + 1 < nchunks) {
            const int last = chunk_pairs(sh, ch + 1) * 16 - 1;
            const f32x4 *src = reinterpret_cast<const f32x4 *>(a.x + size_t(ch + 1) * sh.PC * kPairWeights);
#pragma unroll
            for (int i = 0; i < kMaxX4; ++i) xr[i] = src[min(tid + i * kThreads, last)];
        }
#pragma unroll
        for (int k = 0; k < kTilesPerWg; ++k) {
            if (k < my_tiles) {
                // the next (tile, chunk) in stream order
                int nk = k + 1, nch = ch;
                if (nk >= my_tiles) { nk = 0; ++nch; }
                const bool has_next = nch < nchunks;
                const int nrow0 = (int(blockIdx.x) + nk * int(gridDim.x)) * sh.NR;
                const int nn = has_next ? min(sh.NR, a.N - nrow0) : 0;
                ctile_store<PM>(a.W, sh, row0, nrows, ch, st, wt);
                if (has_next) ctile_issue<PM>(a.W, sh, nrow0, nn, nch, st);
                __syncthreads();
                const int r = tid / sh.PC, p = tid - r * sh.PC;
                if (r < nrows && p < pcc) {
                    float dA, sA, dB, sB;
                    if (q5)
                        pair_dot1_q5(wt + size_t(tid) * (kQ5PairBytes / 4), xs + size_t(p) * kXPad, dA, sA, dB, sB);
                    else
                        pair_dot1(wt + size_t(tid) * (kPairBytes / 4), xs + size_t(p) * kXPad, dA, sA, dB, sB);
                    acc[k] = fmaf(dA, sA, acc[k]);
                    acc[k] = fmaf(dB, sB, acc[k]);
                }
                __syncthreads();
                row0 = nrow0; nrows = nn;
            }
        }
    }
    // reduce and write each tile
    float *part = reinterpret_cast<float *>(wt);
    const int lane = tid & 63, wid = tid >> 6;
#pragma unroll
    for (int k = 0; k < kTilesPerWg; ++k) {
        if (k < my_tiles) {
            const int row0 = (int(blockIdx.x) + k * int(gridDim.x)) * sh.NR;
            const int nr = min(sh.NR, a.N - row0);
            if (tid < nr * sh.PC) part[tid] = acc[k];
            __syncthreads();
            for (int r = wid; r < nr; r += 4) {
                float v = 0.f;
                for (int p = lane; p < sh.PC; p += 64) v += part[r * sh.PC + p];
                v = wave_sum(v);
                if (lane == 0) outv[r] = v;
            }
            __syncthreads();
            for (int r = tid; r < nr; r += kThreads) {
                float *dst = a.y + row0 + r;
                *dst = a.accumulate ? *dst + outv[r] : outv[r];
            }
            __syncthreads();
        }
    }
}


template <bool MULTI, bool MERGE, int PM>
__device__ __forceinline__ void matmul_one(const MatmulArgs &a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds1 l = carve1(smem, a.sh, 1);
    const int ntiles = (a.N + a.sh.NR - 1) / a.sh.NR;
    CoreArgs c{};
    c.W[0] = a.W; c.nmat = 1; c.sh = a.sh; c.N = a.N; c.Tc = 1;
    c.X = a.x; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    const MergeSrc ms{a.mpart, a.msplits, a.mhd, a.mst};
    walk_tiles2<MULTI, MERGE, PM>(
        c, l, ntiles,
        [&](const CoreArgs &t, int nrows) {
            for (int r = threadIdx.x; r < nrows; r += kThreads) {
                float *dst = a.y + t.row0 + r;
                *dst = a.accumulate ? *dst + l.outv[r] : l.outv[r];
            }
        },
        &ms);
}

template <bool MULTI, bool MERGE = false>
__global__ __launch_bounds__(kThreads) void k_matmul1(MatmulArgs a) { matmul_one<MULTI, MERGE, PM_Q8>(a); }
template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_matmul1_q5(MatmulArgs a) { matmul_one<MULTI, false, PM_Q5>(a); }

template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_lmhead1(LmHeadArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const Lds1 l = carve1(smem, a.sh, 1);
    __shared__ float s_red[4];
    __shared__ uint32_t s_redi[4];
    const int ntiles = (a.V + a.sh.NR - 1) / a.sh.NR;
    CoreArgs c{};
    c.W[0] = a.W; c.nmat = 1; c.sh = a.sh; c.N = a.V; c.Tc = 1;
    c.X = a.x; c.ldx = a.sh.K; c.norm_w = a.norm_w; c.eps = a.eps;
    int tile = blockIdx.x;
    c.row0 = tile * a.sh.NR;
    int nrows = tile_rows(c);
    bool vec = tile_vec(c, nrows);
    WStage st;
    stage_issue<PM_Q8>(c, nrows, 0, vec, st);
    stage_row1(c, l, a.ps);
    float *logits = a.st->logits_out;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    float bv = -INFINITY;
    uint32_t bi = uint32_t(c.row0);
    for (; tile < ntiles; tile += gridDim.x) {
        const bool has_next = tile + int(gridDim.x) < ntiles;
        CoreArgs n = c;
        n.row0 = (tile + gridDim.x) * a.sh.NR;
        const int nn = has_next ? tile_rows(n) : 0;
        const bool nvec = has_next ? tile_vec(n, nn) : false;
        tile_run1<MULTI, PM_Q8>(c, l, nrows, vec, st, n, nn, nvec, has_next);
        for (int r = tid; r < nrows; r += kThreads) {
            const float v = l.outv[r];
            logits[c.row0 + r] = v;
            argmax_merge(bv, bi, v, uint32_t(c.row0 + r));
        }
        c = n; nrows = nn; vec = nvec;
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
//   fmt:         the matrix's block format (Q8_0 or Q5_0: 68- or 44-byte pairs;
//                both need the same row alignment, P * align a multiple of 4)
GemvShape choose_shape(int N, int K, int maxt, int nmat, int target_wgs, int nr_mult, int fmt = F_Q8_0) {
    GemvShape s;
    s.K = K;
    s.P = K / kPairWeights;
    s.pb = fmt == F_Q5_0 ? kQ5PairBytes : kPairBytes;
    s.rowbytes = s.P * s.pb;
    const int lds_cap_pairs = std::max(1, (40 * 1024) / (maxt * kXPad * 4));
    s.PC = divisor_at_most(s.P, std::min(lds_cap_pairs, kThreads / nmat));
    const int cap = kThreads / (nmat * s.PC);
    const int want = (N + target_wgs - 1) / target_wgs;
    int nr = std::min(cap, std::max(want, 1));
    // Whole-row tiles move with 16-byte loads only when the tile is a
    // multiple of 16 bytes: round the row count up to that multiple (4 rows of
    // any K are), else down to a multiple of 4.
    int align = 1;
    if (s.PC == s.P)
        while ((align * s.rowbytes) % 16) ++align;
    if (nr >= 4) nr -= nr % 4;
    if (nr % align && ((nr + align - 1) / align) * align <= cap) nr = ((nr + align - 1) / align) * align;
    nr = std::max(nr_mult, nr - nr % nr_mult);
    s.NR = nr;
    return s;
}

// Shape for the chunk-outer kernel. When the dividing chunk size is not a
// multiple of 4 pairs (its tiles would move with 4-byte loads; e.g. K = 11008,
// 172 pairs = 4 * 43) but the row is, take a multiple of 4 that need not
// divide P: the best use of the 256 threads over the chunks, less a small cost
// per chunk, at least 32 pairs per chunk.
GemvShape chunked_shape(GemvShape s) {
    if (s.PC % 4 == 0 || s.P % 4) return s;
    const int cap = std::max(1, (40 * 1024) / (kXPad * 4));
    double best = -1.0;
    int best_pc = s.PC;
    for (int pc = 32; pc <= std::min(cap, kThreads); pc += 4) {
        const int nr = kThreads / pc;
        const int nch = (s.P + pc - 1) / pc;
        const double score = double(s.P) * nr / (double(nch) * kThreads) - 0.03 * nch;
        if (score >= best) {
            best = score;
            best_pc = pc;
        }
    }
    s.PC = best_pc;
    s.NR = kThreads / best_pc;
    return s;
}

// Decode grid: one workgroup per tile up to what the chip holds at once (by
// LDS use), beyond that workgroups loop over tiles.
int grid1(int ntiles, size_t lds) {
    const size_t per_cu = std::max<size_t>(1, std::min<size_t>(8, (160 * 1024) / std::max<size_t>(lds, 1)));
    return std::max(1, std::min(ntiles, int(256 * per_cu)));
}

static hipError_t set_lds(const void *fn, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
}

}  // namespace

hipError_t launch_qkv(const Dims &d, const LayerPtrs &w, const float *x, const StepState *st,
                      const float2 *rope, float *q, float *kc, float *vc, int T, hipStream_t s,
                      const uint8_t *embed, float *xres, const PartSrc &ps, uint32_t *range_flag) {
    const int maxt = T == 1 ? 1 : kMaxTokChunk;
    if (embed && (T != 1 || !xres)) return hipErrorInvalidValue;
    if (ps.n > 0 && (T != 1 || embed)) return hipErrorInvalidValue;
    if (T == 1 && wgemv_fits(d.H)) return launch_wqkv(d, w, x, st, rope, q, kc, vc, s, embed, xres, ps);
    QkvArgs a;
    a.ps = ps;
    a.range_flag = T > 1 ? range_flag : nullptr;
    a.embed = embed; a.xres = xres; a.V = d.V;
    a.wq = w.wq; a.wk = w.wk; a.wv = w.wv; a.norm_w = w.attn_norm; a.x = x; a.st = st;
    a.rope = rope; a.q = q; a.kc = kc; a.vc = vc;
    a.QD = d.nh * d.hd; a.KVD = d.nkv * d.hd; a.hd = d.hd; a.max_seq = d.max_seq; a.T = T;
    a.eps = d.eps; a.rope_neox = d.rope_neox;
    a.sh = choose_shape(a.QD + 2 * a.KVD, d.H, maxt, 1, 512, 2);
    a.pb[0] = w.fq == F_Q5_0 ? kQ5PairBytes : kPairBytes;
    a.pb[1] = w.fk == F_Q5_0 ? kQ5PairBytes : kPairBytes;
    a.pb[2] = w.fv == F_Q5_0 ? kQ5PairBytes : kPairBytes;
    a.tq = (a.QD + a.sh.NR - 1) / a.sh.NR;
    a.tk = (a.KVD + a.sh.NR - 1) / a.sh.NR;
    const int pm = pair_mode(w.fq, w.fk, w.fv);
    const bool multi = a.sh.PC != a.sh.P;
    if (T == 1) {  // decode: row-looping kernel
        const size_t lds = lds1_bytes(a.sh, 1);
        const int g = grid1(a.tq + 2 * a.tk, lds);
        auto kern = pm == PM_Q8 ? (multi ? k_qkv1<true> : k_qkv1<false>)
                  : pm == PM_Q5 ? (multi ? k_qkv1_q5<true> : k_qkv1_q5<false>)
                                : (multi ? k_qkv1_mixed<true> : k_qkv1_mixed<false>);
        hipLaunchKernelGGL(kern, dim3(g), dim3(kThreads), lds, s, a);
        return hipGetLastError();
    }
    dim3 grid(a.tq + 2 * a.tk, (T + maxt - 1) / maxt);
    const size_t lds = lds_bytes(a.sh, 1, maxt);
    auto kern = pm == PM_Q8 ? (multi ? k_qkv<kMaxTokChunk, true> : k_qkv<kMaxTokChunk, false>)
              : pm == PM_Q5 ? (multi ? k_qkv_q5<kMaxTokChunk, true> : k_qkv_q5<kMaxTokChunk, false>)
                            : (multi ? k_qkv_mixed<kMaxTokChunk, true> : k_qkv_mixed<kMaxTokChunk, false>);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_gateup(const Dims &d, const LayerPtrs &w, const float *x, float *h, int T,
                         hipStream_t s, const PartSrc &ps) {
    const int maxt = T == 1 ? 1 : kMaxTokChunk;
    if (ps.n > 0 && T != 1) return hipErrorInvalidValue;
    if (T == 1 && wgemv_fits(d.H)) return launch_wgateup(d, w, x, h, s, ps);
    if (T == 1 && ps.n == 0) {
        const hipError_t e = launch_xgateup(d, w, x, h, s);
        if (e != hipErrorNotSupported) return e;
    }
    GateUpArgs a;
    a.ps = ps;
    a.wg = w.wg; a.wu = w.wu; a.norm_w = w.ffn_norm; a.x = x; a.h = h; a.F = d.F; a.T = T;
    a.eps = d.eps;
    a.sh = choose_shape(d.F, d.H, maxt, 2, 512, 1, w.fg);
    const bool q5 = w.fg == F_Q5_0;
    const bool multi = a.sh.PC != a.sh.P;
    if (T == 1) {
        const size_t lds = lds1_bytes(a.sh, 2);
        const int g = grid1((d.F + a.sh.NR - 1) / a.sh.NR, lds);
        auto kern = q5 ? (multi ? k_gateup1_q5<true> : k_gateup1_q5<false>)
                       : (multi ? k_gateup1<true> : k_gateup1<false>);
        hipLaunchKernelGGL(kern, dim3(g), dim3(kThreads), lds, s, a);
        return hipGetLastError();
    }
    dim3 grid((d.F + a.sh.NR - 1) / a.sh.NR, (T + maxt - 1) / maxt);
    const size_t lds = lds_bytes(a.sh, 2, maxt);
    auto kern = q5 ? (multi ? k_gateup_q5<kMaxTokChunk, true> : k_gateup_q5<kMaxTokChunk, false>)
                   : (multi ? k_gateup<kMaxTokChunk, true> : k_gateup<kMaxTokChunk, false>);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_matmul(const uint8_t *W, int N, int K, const float *X, int T,
                         const float *norm_w, float eps, int accumulate, float *Y,
                         hipStream_t s, int fmt) {
    if (fmt != F_Q8_0 && fmt != F_Q5_0) return hipErrorInvalidValue;
    const int maxt = T == 1 ? 1 : kMaxTokChunk;
    MatmulArgs a{};
    a.W = W; a.norm_w = norm_w; a.x = X; a.y = Y; a.N = N; a.T = T; a.accumulate = accumulate;
    a.eps = eps;
    a.sh = choose_shape(N, K, maxt, 1, 512, 1, fmt);
    if (T == 1 && !norm_w && wgemv_fits(K)) return launch_wmatmul(W, N, K, X, accumulate, Y, s, fmt);
    if (T == 1 && !norm_w) {
        const hipError_t e = launch_xmatmul(W, N, K, X, accumulate, Y, s, fmt);
        if (e != hipErrorNotSupported) return e;
    }
    const bool q5 = fmt == F_Q5_0;
    const bool multi = a.sh.PC != a.sh.P;
    if (T == 1) {
        if (a.sh.PC != a.sh.P && !norm_w) {  // large K: chunk-outer walk
            a.sh = chunked_shape(a.sh);
            if (a.sh.PC * 16 > kMaxX4 * kThreads) return hipErrorInvalidValue;  // activation chunk > registers
            const size_t lds = lds1c_bytes(a.sh);
            const int ntiles = (N + a.sh.NR - 1) / a.sh.NR;
            const int g = std::max(grid1(ntiles, lds), (ntiles + kTilesPerWg - 1) / kTilesPerWg);
            hipLaunchKernelGGL(q5 ? k_matmul1_chunked<true> : k_matmul1_chunked<false>, dim3(g), dim3(kThreads), lds,
                               s, a);
            return hipGetLastError();
        }
        const size_t lds = lds1_bytes(a.sh, 1);
        const int g = grid1((N + a.sh.NR - 1) / a.sh.NR, lds);
        auto kern = q5 ? (multi ? k_matmul1_q5<true> : k_matmul1_q5<false>)
                       : (multi ? k_matmul1<true> : k_matmul1<false>);
        hipLaunchKernelGGL(kern, dim3(g), dim3(kThreads), lds, s, a);
        return hipGetLastError();
    }
    dim3 grid((N + a.sh.NR - 1) / a.sh.NR, (T + maxt - 1) / maxt);
    const size_t lds = lds_bytes(a.sh, 1, maxt);
    auto kern = q5 ? (multi ? k_matmul_q5<kMaxTokChunk, true> : k_matmul_q5<kMaxTokChunk, false>)
                   : (multi ? k_matmul<kMaxTokChunk, true> : k_matmul<kMaxTokChunk, false>);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_oproj_merged(const uint8_t *W, int N, int K, const float *part, int n_splits, int hd,
                               const StepState *st, float *Y, hipStream_t s) {
    if (n_splits < 1 || n_splits > kMergeMaxSplits || K % hd || hd % 4) return hipErrorInvalidValue;
    MatmulArgs a{};
    a.W = W; a.x = nullptr; a.y = Y; a.N = N; a.T = 1; a.accumulate = 1;
    a.mpart = part; a.msplits = n_splits; a.mhd = hd; a.mst = st;
    a.sh = choose_shape(N, K, 1, 1, 512, 1);
    if (a.sh.PC != a.sh.P) return hipErrorInvalidValue;  // the merged row is staged whole
    const size_t lds = lds1_bytes(a.sh, 1);
    const hipError_t e = set_lds(reinterpret_cast<const void *>(&k_matmul1<false, true>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_matmul1<false, true>), dim3(grid1((N + a.sh.NR - 1) / a.sh.NR, lds)), dim3(kThreads), lds,
                       s, a);
    return hipGetLastError();
}

static int lmhead_blocks(int V, int K) {
    if (const int xs = xlmhead_short_blocks(V, K)) return xs;
    const GemvShape sh = choose_shape(V, K, 1, 1, 1024, 1);
    return grid1((V + sh.NR - 1) / sh.NR, lds1_bytes(sh, 1));
}

hipError_t launch_lmhead(const Dims &d, const uint8_t *Wout, const float *out_norm,
                         const float *x_last, StepState *st, float *partials, hipStream_t s, const PartSrc &ps) {
    LmHeadArgs a;
    a.ps = ps;
    a.W = Wout; a.norm_w = out_norm; a.x = x_last; a.st = st; a.partials = partials;
    a.V = d.V; a.eps = d.eps;
    a.sh = choose_shape(d.V, d.H, 1, 1, 1024, 1);
    const int nb = lmhead_blocks(d.V, d.H);
    if (ps.n == 0) {
        const hipError_t e = launch_xlmhead(d, Wout, out_norm, x_last, st, partials, nb, s);
        if (e != hipErrorNotSupported) return e;
    }
    const size_t lds = lds1_bytes(a.sh, 1);
    if (a.sh.PC != a.sh.P)
        hipLaunchKernelGGL(k_lmhead1<true>, dim3(nb), dim3(kThreads), lds, s, a);
    else
        hipLaunchKernelGGL(k_lmhead1<false>, dim3(nb), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_argmax_finish(const Dims &d, const float *partials, StepState *st,
                                hipStream_t s) {
    hipLaunchKernelGGL(k_argmax_finish, dim3(1), dim3(kThreads), 0, s, partials,
                       lmhead_blocks(d.V, d.H), st);
    return hipGetLastError();
}

size_t lmhead_partials_bytes(int V, int K) { return size_t(lmhead_blocks(V, K)) * 8; }

size_t argmax_partials_bytes(int64_t n) { return size_t((n + 4095) / 4096) * 8; }

hipError_t launch_argmax(const float *x, int64_t n, uint32_t *out, float *partials, hipStream_t s) {
    const int grid = int((n + 4095) / 4096);
    hipLaunchKernelGGL(k_argmax_part, dim3(grid), dim3(kThreads), 0, s, x, n, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_out, dim3(1), dim3(kThreads), 0, s, (const float *)partials, grid, out);
    return hipGetLastError();
}

}  // namespace q8l

// k_gemm.hip -- Q8_0 x f32 matrix-matrix product on MFMA (prefill, T > 16).
//
// Prefill runs every projection on T token rows at once ("生成一个 token",
// section "prefill 和 decode：同一个 forward，不同的路": several input rows take
// the matrix-matrix kernel). Y[T][N] = U[T][K] . W[N][K]^T with W in Q8_0.
//
// gfx950 has v_mfma_f32_16x16x32_f16, whose K = 32 is exactly one Q8_0 block.
// Per 32-wide block and 16x16 output tile:
//   * B = the block's int8 values as f16 (exact: |q| <= 127);
//   * A = the activations split as f16 hi + f16 lo (u = hi + lo to ~2^-22
//     relative), two MFMAs accumulate (hi + lo) . q in f32;
//   * the block's f16 scale d (one per output column = one per lane) is then
//     applied in f32: acc += d * tile.
// The result is f32-accurate up to summation order; the int8 values are never
// rounded and the scale is never folded into f16.
//
// Workgroup tile: 64 tokens x 128 output rows, K in steps of 64 (one block
// pair per row, 68 bytes, 4-byte aligned). Per step: activations f32 -> hi/lo
// f16 in LDS (RMSNorm applied on the way when the projection has one), raw
// Q8_0 pairs -> LDS -> f16 values + f32 scales in LDS. 4 waves, each owns a
// 64 x 32 slice (4 x 2 MFMA tiles).

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int GM = 64;     // tokens per workgroup tile
constexpr int GN = 128;    // output rows per workgroup tile
constexpr int GK = 64;     // weights per K step (two Q8_0 blocks)
constexpr int LPAD = 72;   // halves per LDS row (64 + 8)

enum GemmEpi { G_STORE = 0, G_ACCUM = 1, G_QKV = 2, G_GATEUP = 3 };

struct GemmArgs {
    const float *X;        // [T][K] f32 activations
    const float *rinv;     // [T] RMSNorm factors (with norm_w) or null
    const float *norm_w;   // [K] or null
    const uint8_t *W[3];   // matrices (q, k, v | gate, up | single)
    int Nm[3];             // rows of each matrix
    int tiles[3];          // N tiles of each matrix (QKV); GATEUP: tiles of 64 rows
    int T, K, rowbytes;
    // G_STORE / G_ACCUM
    float *Y;              // [T][N]
    // G_QKV
    const StepState *st;
    const float2 *rope;
    float *q, *kc, *vc;
    int QD, hd, max_seq;
    // G_GATEUP
    float *h;              // [T][F]
};

struct GemmLds {
    _Float16 ahi[GM * LPAD];
    _Float16 alo[GM * LPAD];
    _Float16 bq[GN * LPAD];
    float bd[GN * 2];
    uint32_t braw[GN * 17];
};

template <int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm_q8(GemmArgs a) {
    __shared__ __align__(16) GemmLds L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = blockIdx.x * GM;

    // Which weight row feeds B row b of this tile (b in [0, GN)).
    int mat = 0, row0 = 0, rows_in_tile = GN;
    const uint8_t *Wb[2] = {nullptr, nullptr};
    int nvalid[2] = {0, 0};
    if (EPI == G_GATEUP) {
        row0 = blockIdx.y * (GN / 2);
        Wb[0] = a.W[0];
        Wb[1] = a.W[1];
        nvalid[0] = nvalid[1] = min(GN / 2, a.Nm[0] - row0);
    } else {
        int t = blockIdx.y;
        if (EPI == G_QKV) {
            while (mat < 2 && t >= a.tiles[mat]) t -= a.tiles[mat++];
        }
        row0 = t * GN;
        Wb[0] = a.W[mat];
        nvalid[0] = min(GN, a.Nm[mat] - row0);
        rows_in_tile = nvalid[0];
    }
    (void)rows_in_tile;

    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = a.K / GK;
    for (int ks = 0; ks < nsteps; ++ks) {
        // activations: 64 rows x 64 f32 -> hi/lo f16
        for (int e = tid; e < GM * 16; e += kThreads) {
            const int m = e >> 4, c4 = e & 15;
            const int k = ks * GK + c4 * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + m < a.T) {
                v = *reinterpret_cast<const float4 *>(a.X + size_t(m0 + m) * a.K + k);
                if (a.norm_w) {
                    const float r = a.rinv[m0 + m];
                    const float4 w = *reinterpret_cast<const float4 *>(a.norm_w + k);
                    v.x = v.x * r * w.x;
                    v.y = v.y * r * w.y;
                    v.z = v.z * r * w.z;
                    v.w = v.w * r * w.w;
                }
            }
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16 hi = static_cast<_Float16>(vv[i]);
                const _Float16 lo = static_cast<_Float16>(vv[i] - static_cast<float>(hi));
                L.ahi[m * LPAD + c4 * 4 + i] = hi;
                L.alo[m * LPAD + c4 * 4 + i] = lo;
            }
        }
        // raw Q8_0 pairs: GN rows x 17 dwords
        for (int e = tid; e < GN * 17; e += kThreads) {
            const int b = e / 17, j = e - b * 17;
            const int part = (EPI == G_GATEUP) ? (b >= GN / 2) : 0;
            const int r = (EPI == G_GATEUP) ? (b - part * (GN / 2)) : b;
            uint32_t v = 0;
            if (r < nvalid[part])
                v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(
                    Wb[part] + size_t(row0 + r) * a.rowbytes + size_t(ks) * kPairBytes) + j);
            L.braw[e] = v;
        }
        __syncthreads();
        // decode: int8 -> f16 values, f16 scales -> f32
        for (int e = tid; e < GN * 16; e += kThreads) {
            const int b = e >> 4, j = e & 15;
            const uint32_t *raw = L.braw + b * 17;
            const uint32_t q4 = (j < 8) ? __builtin_amdgcn_alignbyte(raw[j + 1], raw[j], 2) : raw[9 + (j - 8)];
            _Float16 *dst = L.bq + b * LPAD + 4 * j;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[i] = static_cast<_Float16>(static_cast<float>(static_cast<int8_t>((q4 >> (8 * i)) & 0xffu)));
            if (j == 0) L.bd[b * 2 + 0] = half_bits_to_float(raw[0]);
            if (j == 8) L.bd[b * 2 + 1] = half_bits_to_float(raw[8] >> 16);
        }
        __syncthreads();
        // MFMA: wave owns columns [wave*32, wave*32 + 32)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            half8 bf[2];
            float dsc[2];
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const int col = wave * 32 + ns * 16 + (lane & 15);
                bf[ns] = *reinterpret_cast<const half8 *>(L.bq + col * LPAD + hb * 32 + 8 * (lane >> 4));
                dsc[ns] = L.bd[col * 2 + hb];
            }
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                const int row = ms * 16 + (lane & 15);
                const half8 ah = *reinterpret_cast<const half8 *>(L.ahi + row * LPAD + hb * 32 + 8 * (lane >> 4));
                const half8 al = *reinterpret_cast<const half8 *>(L.alo + row * LPAD + hb * 32 + 8 * (lane >> 4));
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bf[ns], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bf[ns], t, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[ms][ns][i] = fmaf(dsc[ns], t[i], acc[ms][ns][i]);
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: acc[ms][ns][i] is (m, c) = (ms*16 + 4*(lane/16) + i, wave*32 + ns*16 + lane%16)
    if (EPI == G_GATEUP) {
        // waves 2, 3 hold the up rows: pass them to waves 0, 1 through LDS
        float *ub = reinterpret_cast<float *>(L.ahi);  // 64 x 64 f32 = 16 KB (ahi+alo)
        if (wave >= 2) {
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = ms * 16 + 4 * (lane >> 4) + i;
                        const int c = (wave - 2) * 32 + ns * 16 + (lane & 15);
                        ub[m * 64 + c] = acc[ms][ns][i];
                    }
        }
        __syncthreads();
        if (wave < 2) {
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = ms * 16 + 4 * (lane >> 4) + i;
                        const int c = wave * 32 + ns * 16 + (lane & 15);
                        if (m0 + m < a.T && c < nvalid[0]) {
                            const float g = acc[ms][ns][i], u = ub[m * 64 + c];
                            a.h[size_t(m0 + m) * a.Nm[0] + row0 + c] = silu(g) * u;
                        }
                    }
        }
        return;
    }
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = ms * 16 + 4 * (lane >> 4) + i;
                const int c = wave * 32 + ns * 16 + (lane & 15);
                const float v = acc[ms][ns][i];
                if (EPI == G_QKV) {
                    // rope pairs (2j, 2j+1) sit in adjacent lanes
                    const float partner = __shfl_xor(v, 1, 64);
                    if (m0 + m >= a.T || c >= nvalid[0]) continue;
                    const int row = row0 + c;
                    const int d = row % a.hd;
                    const int t = m0 + m;
                    if (mat == 2) {
                        a.vc[(size_t(row / a.hd) * a.max_seq + a.st->slot + t) * a.hd + d] = v;
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

// rinv[t] = 1 / sqrt(mean(x[t]^2) + eps), one workgroup per row.
__global__ __launch_bounds__(kThreads) void k_rms_rows(const float *x, int K, float eps, float *rinv) {
    __shared__ float red[4];
    const float *xr = x + size_t(blockIdx.x) * K;
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += kThreads) ss = fmaf(xr[k], xr[k], ss);
    ss = block_sum(ss, red);
    if (threadIdx.x == 0) rinv[blockIdx.x] = 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
}

}  // namespace

hipError_t launch_rms_rows(const float *x, int T, int K, float eps, float *rinv, hipStream_t s) {
    hipLaunchKernelGGL(k_rms_rows, dim3(T), dim3(kThreads), 0, s, x, K, eps, rinv);
    return hipGetLastError();
}

static GemmArgs gemm_base(const float *X, const float *rinv, const float *norm_w, int T, int K) {
    GemmArgs a{};
    a.X = X; a.rinv = rinv; a.norm_w = norm_w; a.T = T; a.K = K;
    a.rowbytes = K / kQK * kQBytes;
    return a;
}

hipError_t launch_gemm_matmul(const uint8_t *W, int N, int K, const float *X, int T,
                              const float *rinv, const float *norm_w, int accumulate, float *Y,
                              hipStream_t s) {
    GemmArgs a = gemm_base(X, rinv, norm_w, T, K);
    a.W[0] = W; a.Nm[0] = N; a.Y = Y;
    dim3 grid((T + GM - 1) / GM, (N + GN - 1) / GN);
    if (accumulate)
        hipLaunchKernelGGL(k_gemm_q8<G_ACCUM>, grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL(k_gemm_q8<G_STORE>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_qkv(const Dims &d, const LayerPtrs &w, const float *x, const float *rinv,
                           const StepState *st, const float2 *rope, float *q, float *kc, float *vc,
                           int T, hipStream_t s) {
    GemmArgs a = gemm_base(x, rinv, w.attn_norm, T, d.H);
    const int QD = d.nh * d.hd, KVD = d.nkv * d.hd;
    a.W[0] = w.wq; a.W[1] = w.wk; a.W[2] = w.wv;
    a.Nm[0] = QD; a.Nm[1] = KVD; a.Nm[2] = KVD;
    for (int i = 0; i < 3; ++i) a.tiles[i] = (a.Nm[i] + GN - 1) / GN;
    a.st = st; a.rope = rope; a.q = q; a.kc = kc; a.vc = vc;
    a.QD = QD; a.hd = d.hd; a.max_seq = d.max_seq;
    dim3 grid((T + GM - 1) / GM, a.tiles[0] + a.tiles[1] + a.tiles[2]);
    hipLaunchKernelGGL(k_gemm_q8<G_QKV>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_gateup(const Dims &d, const LayerPtrs &w, const float *x, const float *rinv,
                              float *h, int T, hipStream_t s) {
    GemmArgs a = gemm_base(x, rinv, w.ffn_norm, T, d.H);
    a.W[0] = w.wg; a.W[1] = w.wu; a.Nm[0] = d.F; a.Nm[1] = d.F; a.h = h;
    dim3 grid((T + GM - 1) / GM, (d.F + GN / 2 - 1) / (GN / 2));
    hipLaunchKernelGGL(k_gemm_q8<G_GATEUP>, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace q8l

// k_kquant.hip -- Q4_K / Q6_K x f32 matrix-vector product (one token).
//
// Files in the 4-bit "K" mix store some projections in 256-weight blocks
// ("速度", section "CPU GGUF": the Q4_K_M file of the 135M model holds its
// 1536-wide down projections as Q4K and Q6K). Decoding multiplies each such
// matrix by one activation row, so the work is a stream of blocks from HBM:
//   Q4_K (144 B / 256 weights): f16 d, f16 dmin, 12 bytes of 6-bit scales and
//        mins for eight 32-weight sub-blocks, 128 bytes of 4-bit values;
//        weight = d * s * q - dmin * m.
//   Q6_K (210 B / 256 weights): 128 bytes of low 4 bits, 64 bytes of high 2
//        bits, sixteen int8 scales (one per 16 weights), f16 d;
//        weight = d * sc * (q - 32).
//
// Layout: each wave owns R consecutive rows and walks their blocks; the
// workgroup (4 waves) stages the activation row in LDS once per K chunk,
// together with its sums over each 16 weights (the min term of Q4_K and the
// -32 offset of Q6_K are such sums times a per-block constant). A lane takes
// one "piece" of a block per iteration and the same piece of each of the
// wave's R rows, so activation values read from LDS serve R rows:
//   Q4_K piece p (8 per block), c = p/2, l0 = 16 (p%2): value bytes
//        32c + l0 .. +15, whose low nibbles are weights 64c + l0 + i
//        (sub-block 2c) and high nibbles 64c + 32 + l0 + i (sub-block 2c+1),
//        plus the 16-byte header (d, dmin, scales);
//   Q6_K piece p (4 per block), h = p/2, l0 = 16 (p%2): weights
//        128h + 32k + l0 + i for k = 0..3, i.e. low-bit bytes 64h + l0 + i
//        (k = 0 low nibble, k = 2 high) and 64h + 32 + l0 + i (k = 1, 3),
//        high-bit bytes 32h + l0 + i (bits 2k, 2k+1), the half's 8 scales and
//        d. Q6_K blocks start 2-byte aligned: pieces are loaded from the
//        dword-aligned floor and re-aligned with alignbyte.
// Loads go through one buffer resource over the matrix; rows past N read as
// zeros through its range check. Per-row partials are reduced over the wave
// in a fixed order (results are reproducible run to run).

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

constexpr int kKqMaxChunk = 15360;             // activation floats staged per K chunk (60 KB + sums)
constexpr uint32_t kKqOut = 0x80000000u;       // offset past any resource: loads return 0
constexpr int kKqWord3 = 0x00020000;           // raw buffer, 32-bit data format

struct KqArgs {
    const uint8_t *W;
    int N, K, rowbytes;
    int kc;              // K chunk (multiple of 256)
    const float *X;      // [K]
    float *Y;            // [N]
    int accumulate;
};

template <int FMT>
struct KqFmt {
    static constexpr int PER = FMT == F_Q4_K ? 8 : 4;        // pieces per block
    static constexpr int NW = FMT == F_Q4_K ? 8 : 19;        // dwords a piece loads
    static constexpr int BYTES = FMT == F_Q4_K ? kQ4KBytes : kQ6KBytes;
    static constexpr int U = FMT == F_Q4_K ? 2 : 1;          // pieces per lane per register stage
};

template <int FMT>
__device__ inline void kq_piece_load(__amdgpu_buffer_rsrc_t rs, uint32_t blk, int p, uint32_t *w) {
    if (FMT == F_Q4_K) {
        const u32x4 hd = __builtin_amdgcn_raw_buffer_load_b128(rs, blk, 0, 0);
        const u32x4 qs = __builtin_amdgcn_raw_buffer_load_b128(rs, blk + 16 + 16 * p, 0, 0);
        w[0] = hd.x; w[1] = hd.y; w[2] = hd.z; w[3] = hd.w;
        w[4] = qs.x; w[5] = qs.y; w[6] = qs.z; w[7] = qs.w;
    } else {
        const int h = p >> 1, l0 = 16 * (p & 1);
        const uint32_t base = blk & ~3u;    // piece offsets below are multiples of 4
        const uint32_t offs[3] = {base + 64 * h + l0, base + 64 * h + 32 + l0, base + 128 + 32 * h + l0};
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, offs[k], 0, 0);
            w[5 * k + 0] = v.x; w[5 * k + 1] = v.y; w[5 * k + 2] = v.z; w[5 * k + 3] = v.w;
            w[5 * k + 4] = __builtin_amdgcn_raw_buffer_load_b32(rs, offs[k] + 16, 0, 0);
        }
        const uint32_t so = base + 192 + 8 * h;   // the third dword is used only when misaligned
        w[15] = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 0, 0);
        w[16] = __builtin_amdgcn_raw_buffer_load_b32(rs, so + 4, 0, 0);
        w[17] = __builtin_amdgcn_raw_buffer_load_b32(rs, so + 8, 0, 0);
        // d: a 16-bit load at its own address (a dword there would reach past
        // the matrix's last block when that block is dword-aligned)
        w[18] = __builtin_amdgcn_raw_buffer_load_b16(rs, blk + 208, 0, 0);
    }
}

__device__ __forceinline__ float ubyte(uint32_t v, int b) { return static_cast<float>((v >> (8 * b)) & 0xffu); }

// A word of small values whose known-zero bits the compiler should not see:
// otherwise it turns each byte conversion into a bit-field extract plus a
// conversion of byte 0, instead of one conversion of byte b. An empty asm
// statement, no instruction; not volatile, so it does not fence the
// scheduler (a volatile one cost a third of the kernel's speed).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Q4_K piece p of block j (of the staged chunk) against the staged activations.
__device__ inline float q4k_piece_dot(const uint32_t *w, int p, const float *xs, const float *x16, int j) {
    const int c = p >> 1, l0 = 16 * (p & 1);
    const float d = half_bits_to_float(w[0]), dmin = half_bits_to_float(w[0] >> 16);
    // scales and mins of sub-blocks 2c and 2c+1, branch-free (c differs across
    // the wave's lanes): for c < 2 the low 6 bits of bytes 2c(+1) and 2c(+1)+4;
    // for c >= 2 a nibble of byte 2c(+1)+4 below the top two bits of byte
    // 2c(+1)-4 (scale) or 2c(+1) (min)
    const bool hi = c >= 2;
    const int sh = 16 * (c & 1);
    const uint32_t s03 = w[1] >> sh, s47 = w[2] >> sh, s811 = w[3] >> sh;
    const uint32_t lo_s = hi ? s811 : s03, lo_m = hi ? (s811 >> 4) : s47;
    const uint32_t mask = hi ? 0x0f0fu : 0x3f3fu;
    const uint32_t top_s = hi ? ((s03 >> 2) & 0x3030u) : 0u, top_m = hi ? ((s47 >> 2) & 0x3030u) : 0u;
    const uint32_t sc = (lo_s & mask) | top_s, mn = (lo_m & mask) | top_m;   // byte 0: sub-block 2c, byte 1: 2c+1
    const uint32_t s0 = sc & 0xffu, s1 = (sc >> 8) & 0xffu, m0 = mn & 0xffu, m1 = (mn >> 8) & 0xffu;
    const int xl = j * kQKK + 64 * c + l0;
    const float *xa = xs + xl, *xb = xs + xl + 32;
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = opaque(w[4 + e] & 0x0f0f0f0fu), hi = opaque((w[4 + e] >> 4) & 0x0f0f0f0fu);
        const float4 va = *reinterpret_cast<const float4 *>(xa + 4 * e);
        const float4 vb = *reinterpret_cast<const float4 *>(xb + 4 * e);
        a0 = fmaf(ubyte(lo, 0), va.x, a0);
        a1 = fmaf(ubyte(lo, 1), va.y, a1);
        a0 = fmaf(ubyte(lo, 2), va.z, a0);
        a1 = fmaf(ubyte(lo, 3), va.w, a1);
        b0 = fmaf(ubyte(hi, 0), vb.x, b0);
        b1 = fmaf(ubyte(hi, 1), vb.y, b1);
        b0 = fmaf(ubyte(hi, 2), vb.z, b0);
        b1 = fmaf(ubyte(hi, 3), vb.w, b1);
    }
    const float ra = (d * float(s0)) * (a0 + a1) - (dmin * float(m0)) * x16[xl >> 4];
    const float rb = (d * float(s1)) * (b0 + b1) - (dmin * float(m1)) * x16[(xl + 32) >> 4];
    return ra + rb;
}

// Q6_K piece p of block j; `blk` is the block's byte offset (its low two bits
// give the re-alignment).
__device__ inline float q6k_piece_dot(const uint32_t *w, uint32_t blk, int p, const float *xs, const float *x16,
                                      int j) {
    const uint32_t sh = blk & 3u;
    const int h = p >> 1, odd = p & 1;
    uint32_t A[4], B[4], Hb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        A[e] = __builtin_amdgcn_alignbyte(w[e + 1], w[e], sh);
        B[e] = __builtin_amdgcn_alignbyte(w[e + 6], w[e + 5], sh);
        Hb[e] = __builtin_amdgcn_alignbyte(w[e + 11], w[e + 10], sh);
    }
    const uint32_t S0 = __builtin_amdgcn_alignbyte(w[16], w[15], sh);   // scales 8h + 0..3
    const uint32_t S1 = __builtin_amdgcn_alignbyte(w[17], w[16], sh);   // scales 8h + 4..7
    const float d = half_bits_to_float(w[18]);
    const int xl = j * kQKK + 128 * h + 16 * odd;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float *xk = xs + xl + 32 * k;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lowsrc = (k & 1) ? B[e] : A[e];
            const uint32_t nib = (k >= 2 ? (lowsrc >> 4) : lowsrc) & 0x0f0f0f0fu;
            const uint32_t q = opaque(nib | (((Hb[e] >> (2 * k)) & 0x03030303u) << 4));
            const float4 v = *reinterpret_cast<const float4 *>(xk + 4 * e);
            s0 = fmaf(ubyte(q, 0), v.x, s0);
            s1 = fmaf(ubyte(q, 1), v.y, s1);
            s0 = fmaf(ubyte(q, 2), v.z, s0);
            s1 = fmaf(ubyte(q, 3), v.w, s1);
        }
        // scale 2k + odd of the half: byte (2k + odd) of S0:S1
        const uint32_t sw = k < 2 ? S0 : S1;
        const float sc = static_cast<float>(static_cast<int8_t>((sw >> (8 * (2 * (k & 1) + odd))) & 0xffu));
        acc = fmaf(sc, (s0 + s1) - 32.f * x16[(xl + 32 * k) >> 4], acc);
    }
    return d * acc;
}

// One stage: kU pieces per lane (each for the wave's R rows) starting at item i0.
template <int FMT, int R>
__device__ inline void kq_issue(__amdgpu_buffer_rsrc_t rs, const uint32_t *roff, uint32_t blk0, int items, int i0,
                                int lane, int p, uint32_t (&w)[KqFmt<FMT>::U][R][KqFmt<FMT>::NW]) {
    using F = KqFmt<FMT>;
#pragma unroll
    for (int u = 0; u < F::U; ++u) {
        const int it = i0 + 64 * u + lane;
        const uint32_t bo = blk0 + uint32_t(it / F::PER) * F::BYTES;
#pragma unroll
        for (int r = 0; r < R; ++r) kq_piece_load<FMT>(rs, it < items ? roff[r] + bo : kKqOut, p, w[u][r]);
    }
}

template <int FMT, int R>
__device__ inline void kq_compute(const uint32_t *roff, uint32_t blk0, int items, int i0, int lane, int p,
                                  const float *xs, const float *x16, const uint32_t (&w)[KqFmt<FMT>::U][R][KqFmt<FMT>::NW],
                                  float *acc) {
    using F = KqFmt<FMT>;
#pragma unroll
    for (int u = 0; u < F::U; ++u) {
        const int it = i0 + 64 * u + lane;
        if (it < items) {
            const int j = it / F::PER;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (FMT == F_Q4_K)
                    acc[r] += q4k_piece_dot(w[u][r], p, xs, x16, j);
                else
                    acc[r] += q6k_piece_dot(w[u][r], roff[r] + blk0 + uint32_t(j) * F::BYTES, p, xs, x16, j);
            }
        }
    }
}

template <int FMT, int R>
__global__ __launch_bounds__(kThreads) void k_kq_gemv(KqArgs a) {
    using F = KqFmt<FMT>;
    constexpr int STEP = 64 * F::U;   // items per stage
    extern __shared__ __align__(16) float xs[];   // a.kc activations, then a.kc / 16 sums
    float *x16 = xs + a.kc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row0 = (blockIdx.x * 4 + wave) * R;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(a.W), 0, int(uint32_t(a.N) * uint32_t(a.rowbytes)), kKqWord3);
    uint32_t roff[R];
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        roff[r] = row0 + r < a.N ? uint32_t(row0 + r) * uint32_t(a.rowbytes) : kKqOut;
        acc[r] = 0.f;
    }
    const int p = lane % F::PER;   // the same piece of every block for this lane
    uint32_t w0[F::U][R][F::NW], w1[F::U][R][F::NW];
    for (int k0 = 0; k0 < a.K; k0 += a.kc) {
        const int kn = min(a.kc, a.K - k0);
        const uint32_t blk0 = uint32_t(k0 / kQKK) * F::BYTES;
        const int items = kn / kQKK * F::PER;
        // the first stage's weights do not depend on the activations: in flight during the staging
        kq_issue<FMT, R>(rs, roff, blk0, items, 0, lane, p, w0);
        __syncthreads();   // the previous chunk is consumed
        for (int i = tid; i < kn / 16; i += kThreads) {
            const float4 *src = reinterpret_cast<const float4 *>(a.X + k0 + 16 * i);
            const float4 v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
            float4 *dst = reinterpret_cast<float4 *>(xs + 16 * i);
            dst[0] = v0; dst[1] = v1; dst[2] = v2; dst[3] = v3;
            x16[i] = (((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w))) +
                     (((v2.x + v2.y) + (v2.z + v2.w)) + ((v3.x + v3.y) + (v3.z + v3.w)));
        }
        __syncthreads();
        // two register stages: the next stage's loads are issued before this one is computed
        for (int i0 = 0; i0 < items; i0 += 2 * STEP) {
            if (i0 + STEP < items) kq_issue<FMT, R>(rs, roff, blk0, items, i0 + STEP, lane, p, w1);
            kq_compute<FMT, R>(roff, blk0, items, i0, lane, p, xs, x16, w0, acc);
            if (i0 + STEP >= items) break;
            if (i0 + 2 * STEP < items) kq_issue<FMT, R>(rs, roff, blk0, items, i0 + 2 * STEP, lane, p, w0);
            kq_compute<FMT, R>(roff, blk0, items, i0 + STEP, lane, p, xs, x16, w1, acc);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float v = wave_sum(acc[r]);
        if (lane == 0 && row0 + r < a.N) {
            float *dst = a.Y + row0 + r;
            *dst = a.accumulate ? *dst + v : v;
        }
    }
}

template <int FMT, int R>
hipError_t launch_kq_r(const KqArgs &a, hipStream_t s) {
    const size_t lds = size_t(a.kc) * 4 + size_t(a.kc / 16) * 4;
    const int grid = (a.N + 4 * R - 1) / (4 * R);
    hipLaunchKernelGGL((k_kq_gemv<FMT, R>), dim3(grid), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kq_gemv(int fmt, const uint8_t *W, int N, int K, const float *X, int accumulate, float *Y,
                          hipStream_t s) {
    if ((fmt != F_Q4_K && fmt != F_Q6_K) || N < 1 || K < kQKK || K % kQKK) return hipErrorInvalidValue;
    KqArgs a;
    a.W = W; a.N = N; a.K = K; a.X = X; a.Y = Y; a.accumulate = accumulate;
    a.rowbytes = int(fmt_row_bytes(fmt, K));
    if (uint64_t(N) * uint64_t(a.rowbytes) + 64 >= kKqOut) return hipErrorInvalidValue;
    a.kc = std::min(K, kKqMaxChunk);
    // two rows per wave once that still gives every CU two workgroups
    const bool two = N >= 2 * 256 * 4 * 2;
    if (fmt == F_Q4_K) return two ? launch_kq_r<F_Q4_K, 2>(a, s) : launch_kq_r<F_Q4_K, 1>(a, s);
    return two ? launch_kq_r<F_Q6_K, 2>(a, s) : launch_kq_r<F_Q6_K, 1>(a, s);
}

}  // namespace q8l

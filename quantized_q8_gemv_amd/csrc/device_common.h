// device_common.h -- device helpers shared by the kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8l_internal.h"

namespace q8l {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// IEEE binary16 bit pattern -> f32 (exact; subnormal scales stay subnormal in
// f16 and become normal f32 values).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(bits & 0xffffu)));
}

__device__ __forceinline__ float sbyte(uint32_t v, int b) {
    return static_cast<float>(static_cast<int>(static_cast<int8_t>((v >> (8 * b)) & 0xffu)));
}

// Decode one pair of Q8_0 blocks (68 bytes = 17 dwords at a 4-byte aligned
// address): block A = bytes [0, 34), block B = bytes [34, 68). The int8
// payload of A starts at byte 2, so its dwords are re-aligned with alignbyte;
// B's payload starts at byte 36 and is dword-aligned.
struct PairQ {
    float dA, dB;
    float q[64];
};

__device__ __forceinline__ void decode_pair(const uint32_t *w, PairQ &o) {
    uint32_t r[17];
#pragma unroll
    for (int i = 0; i < 17; ++i) r[i] = w[i];
    o.dA = half_bits_to_float(r[0]);
    o.dB = half_bits_to_float(r[8] >> 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t a = __builtin_amdgcn_alignbyte(r[j + 1], r[j], 2);
        uint32_t b = r[9 + j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o.q[4 * j + e] = sbyte(a, e);
            o.q[32 + 4 * j + e] = sbyte(b, e);
        }
    }
}

// One pair against one activation row, decoding on the fly (no 64-float
// array: keeps register use low). Same summation order as decode_pair +
// block_dot: per block four interleaved partial sums, (s0 + s1) + (s2 + s3).
__device__ __forceinline__ void pair_dot1(const uint32_t *w, const float *x, float &dA, float &sA,
                                          float &dB, float &sB) {
    uint32_t prev = w[0];
    dA = half_bits_to_float(prev);
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t nxt = w[j + 1];
        const uint32_t q = __builtin_amdgcn_alignbyte(nxt, prev, 2);
        const float4 xv = *reinterpret_cast<const float4 *>(x + 4 * j);
        s0 = fmaf(sbyte(q, 0), xv.x, s0);
        s1 = fmaf(sbyte(q, 1), xv.y, s1);
        s2 = fmaf(sbyte(q, 2), xv.z, s2);
        s3 = fmaf(sbyte(q, 3), xv.w, s3);
        prev = nxt;
    }
    sA = (s0 + s1) + (s2 + s3);
    dB = half_bits_to_float(prev >> 16);
    s0 = s1 = s2 = s3 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t q = w[9 + j];
        const float4 xv = *reinterpret_cast<const float4 *>(x + 32 + 4 * j);
        s0 = fmaf(sbyte(q, 0), xv.x, s0);
        s1 = fmaf(sbyte(q, 1), xv.y, s1);
        s2 = fmaf(sbyte(q, 2), xv.z, s2);
        s3 = fmaf(sbyte(q, 3), xv.w, s3);
    }
    sB = (s0 + s1) + (s2 + s3);
}

// Q5_0 (22-byte blocks: f16 d, a 32-bit word of fifth bits, 16 bytes of
// nibbles; weight i < 16 is the low nibble of byte i, weight i + 16 its high
// nibble, bit i of the word is weight i's fifth bit, q = 5-bit value - 16).
// The 5-bit values of weights 4j .. 4j + 3 (hi = false) or 16 + 4j .. 16 +
// 4j + 3 (hi = true) as four bytes: the nibbles of dword j of the block's 16
// value bytes with their fifth bits placed at bit 4 of each byte (the four
// bits times 0x204081 land at bits 0, 8, 16 and 24).
__device__ __forceinline__ uint32_t q5_bytes(uint32_t qs, uint32_t qh, int j, bool hi) {
    const uint32_t nib = (hi ? qs >> 4 : qs) & 0x0f0f0f0fu;
    const uint32_t b = (qh >> (4 * j + (hi ? 16 : 0))) & 0xfu;
    return nib | (((b * 0x204081u) & 0x01010101u) << 4);
}

__device__ __forceinline__ float ubyte_f(uint32_t v, int b) { return static_cast<float>((v >> (8 * b)) & 0xffu); }

// One pair of Q5_0 blocks (44 bytes = 11 dwords at a 4-byte aligned
// address): block A = bytes [0, 22) (its fifth-bit word and values start 2
// bytes into a dword and are re-aligned with alignbyte), block B = bytes
// [22, 44) (d in the high half of dword 5, the word and values dword-aligned).
// Decoded into the Q8_0 pair form (d and the 64 integers as floats).
__device__ __forceinline__ void decode_pair_q5(const uint32_t *w, PairQ &o) {
    uint32_t r[11];
#pragma unroll
    for (int i = 0; i < 11; ++i) r[i] = w[i];
    o.dA = half_bits_to_float(r[0]);
    o.dB = half_bits_to_float(r[5] >> 16);
    const uint32_t qhA = __builtin_amdgcn_alignbyte(r[1], r[0], 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t qa = __builtin_amdgcn_alignbyte(r[j + 2], r[j + 1], 2);
        const uint32_t qb = r[7 + j];
        const uint32_t la = q5_bytes(qa, qhA, j, false), ha = q5_bytes(qa, qhA, j, true);
        const uint32_t lb = q5_bytes(qb, r[6], j, false), hb = q5_bytes(qb, r[6], j, true);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o.q[4 * j + e] = ubyte_f(la, e) - 16.0f;
            o.q[16 + 4 * j + e] = ubyte_f(ha, e) - 16.0f;
            o.q[32 + 4 * j + e] = ubyte_f(lb, e) - 16.0f;
            o.q[48 + 4 * j + e] = ubyte_f(hb, e) - 16.0f;
        }
    }
}

// d * sum_i q[i] x[i] over one 32-weight block, in a fixed order: four
// interleaved partial sums, then (s0 + s1) + (s2 + s3).
__device__ __forceinline__ float block_dot(const float *q, const float *x) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
        float4 xv = *reinterpret_cast<const float4 *>(x + i);
        s0 = fmaf(q[i + 0], xv.x, s0);
        s1 = fmaf(q[i + 1], xv.y, s1);
        s2 = fmaf(q[i + 2], xv.z, s2);
        s3 = fmaf(q[i + 3], xv.w, s3);
    }
    return (s0 + s1) + (s2 + s3);
}

// One Q5_0 pair against one activation row, decoding on the fly (as
// pair_dot1; same values and summation order as decode_pair_q5 + block_dot:
// weights 0..15 of a block are the low nibbles, 16..31 the high ones).
__device__ __forceinline__ float q5_block_dot(const uint32_t qs[4], uint32_t qh, const float *x) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t u = q5_bytes(qs[j], qh, j, h != 0);
            const float4 xv = *reinterpret_cast<const float4 *>(x + 16 * h + 4 * j);
            s0 = fmaf(ubyte_f(u, 0) - 16.0f, xv.x, s0);
            s1 = fmaf(ubyte_f(u, 1) - 16.0f, xv.y, s1);
            s2 = fmaf(ubyte_f(u, 2) - 16.0f, xv.z, s2);
            s3 = fmaf(ubyte_f(u, 3) - 16.0f, xv.w, s3);
        }
    return (s0 + s1) + (s2 + s3);
}

__device__ __forceinline__ void pair_dot1_q5(const uint32_t *w, const float *x, float &dA, float &sA, float &dB,
                                             float &sB) {
    const uint32_t r0 = w[0], r1 = w[1];
    dA = half_bits_to_float(r0);
    uint32_t qa[4];
    qa[0] = __builtin_amdgcn_alignbyte(w[2], r1, 2);
#pragma unroll
    for (int j = 1; j < 4; ++j) qa[j] = __builtin_amdgcn_alignbyte(w[j + 2], w[j + 1], 2);
    sA = q5_block_dot(qa, __builtin_amdgcn_alignbyte(r1, r0, 2), x);
    dB = half_bits_to_float(w[5] >> 16);
    uint32_t qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = w[7 + j];
    sB = q5_block_dot(qb, w[6], x + 32);
}

// The same pair products with the pair's 64 activations in registers
// (x[i] = activation i of the pair): returns dA * sA + dB * sB, with sA, sB
// summed as in pair_dot1 / pair_dot1_q5.
__device__ __forceinline__ float xpair_dot_q8(const uint32_t (&w)[17], const float (&x)[64]) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t q = __builtin_amdgcn_alignbyte(w[j + 1], w[j], 2);
        s0 = fmaf(sbyte(q, 0), x[4 * j], s0);
        s1 = fmaf(sbyte(q, 1), x[4 * j + 1], s1);
        s2 = fmaf(sbyte(q, 2), x[4 * j + 2], s2);
        s3 = fmaf(sbyte(q, 3), x[4 * j + 3], s3);
    }
    const float sA = (s0 + s1) + (s2 + s3);
    s0 = s1 = s2 = s3 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t q = w[9 + j];
        s0 = fmaf(sbyte(q, 0), x[32 + 4 * j], s0);
        s1 = fmaf(sbyte(q, 1), x[33 + 4 * j], s1);
        s2 = fmaf(sbyte(q, 2), x[34 + 4 * j], s2);
        s3 = fmaf(sbyte(q, 3), x[35 + 4 * j], s3);
    }
    const float sB = (s0 + s1) + (s2 + s3);
    return fmaf(half_bits_to_float(w[8] >> 16), sB, half_bits_to_float(w[0]) * sA);
}

__device__ __forceinline__ float xblock_dot_q5(const uint32_t (&qs)[4], uint32_t qh, const float (&x)[64], int x0) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t u = q5_bytes(qs[j], qh, j, h != 0);
            const int i = x0 + 16 * h + 4 * j;
            s0 = fmaf(ubyte_f(u, 0) - 16.0f, x[i], s0);
            s1 = fmaf(ubyte_f(u, 1) - 16.0f, x[i + 1], s1);
            s2 = fmaf(ubyte_f(u, 2) - 16.0f, x[i + 2], s2);
            s3 = fmaf(ubyte_f(u, 3) - 16.0f, x[i + 3], s3);
        }
    return (s0 + s1) + (s2 + s3);
}

// The same with the activation block sums xs = sum x[0..31], sum x[32..63]
// taken once (the activations stay while the rows change): sum (u - 16) x =
// sum u x - 16 xs, one conversion and one FMA per weight (u the 5-bit code;
// the rounding differs from the form above by the order of the terms only).
__device__ __forceinline__ float xblock_dot_q5u(const uint32_t (&qs)[4], uint32_t qh, const float (&x)[64], int x0,
                                                float xs) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t u = q5_bytes(qs[j], qh, j, h != 0);
            const int i = x0 + 16 * h + 4 * j;
            s0 = fmaf(ubyte_f(u, 0), x[i], s0);
            s1 = fmaf(ubyte_f(u, 1), x[i + 1], s1);
            s2 = fmaf(ubyte_f(u, 2), x[i + 2], s2);
            s3 = fmaf(ubyte_f(u, 3), x[i + 3], s3);
        }
    return fmaf(-16.0f, xs, (s0 + s1) + (s2 + s3));
}

__device__ __forceinline__ float xpair_dot_q5s(const uint32_t (&w)[11], const float (&x)[64], float xsA, float xsB) {
    uint32_t qa[4], qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        qa[j] = __builtin_amdgcn_alignbyte(w[j + 2], w[j + 1], 2);
        qb[j] = w[7 + j];
    }
    const float sA = xblock_dot_q5u(qa, __builtin_amdgcn_alignbyte(w[1], w[0], 2), x, 0, xsA);
    const float sB = xblock_dot_q5u(qb, w[6], x, 32, xsB);
    return fmaf(half_bits_to_float(w[5] >> 16), sB, half_bits_to_float(w[0]) * sA);
}

__device__ __forceinline__ float xpair_dot_q5(const uint32_t (&w)[11], const float (&x)[64]) {
    uint32_t qa[4], qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        qa[j] = __builtin_amdgcn_alignbyte(w[j + 2], w[j + 1], 2);
        qb[j] = w[7 + j];
    }
    const float sA = xblock_dot_q5(qa, __builtin_amdgcn_alignbyte(w[1], w[0], 2), x, 0);
    const float sB = xblock_dot_q5(qb, w[6], x, 32);
    return fmaf(half_bits_to_float(w[5] >> 16), sB, half_bits_to_float(w[0]) * sA);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// v of a lane combined with the lane `ctrl` selects (a DPP move; row_mask,
// bank_mask all lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a wave, in a fixed order, without LDS: within
// each 16-lane row by DPP (neighbours, pairs of neighbours, mirrored halves
// of 8, mirrored halves of 16: every lane of a row ends with the row's sum,
// the same bits in each since a + b == b + a), then the four row sums read
// from lanes 0, 16, 32, 48 and added as (r0 + r1) + (r2 + r3). Every lane
// gets the result.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v);   // row_half_mirror
    v += dpp_f<0x140>(v);   // row_mirror
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Largest of v over the 64 lanes, by the same DPP pattern as wave_sum_dpp
// (max is exact, so the order does not matter); every lane gets it.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Largest of v over each 16-lane row (lanes 16r .. 16r + 15), every lane
// of the row gets it.
__device__ __forceinline__ float row16_max_dpp(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    return fmaxf(v, dpp_f<0x140>(v));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Sum of v over the 256-thread workgroup in a fixed order; every thread gets
// the result. `red` is 4 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    v = wave_sum_dpp(v);
    __syncthreads();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Larger value wins; on equal values the lower index wins.
__device__ __forceinline__ void argmax_merge(float &v, uint32_t &i, float ov, uint32_t oi) {
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

__device__ __forceinline__ void wave_argmax(float &v, uint32_t &i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float ov = __shfl_xor(v, off, 64);
        uint32_t oi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(i), off, 64));
        argmax_merge(v, i, ov, oi);
    }
}

// Scale s and min m (6 bits each) of Q4_K sub-block j (0..7) from the block's
// 12 packed bytes (dwords s03 = bytes 0..3, s47 = 4..7, s811 = 8..11): for
// j < 4 the low 6 bits of bytes j and j + 4; for j >= 4 the low / high nibble
// of byte j + 4 with the top two bits of byte j - 4 / j above it.
__device__ __forceinline__ void q4k_scale_min(int j, uint32_t s03, uint32_t s47, uint32_t s811, uint32_t &sc,
                                              uint32_t &mn) {
    const int sh = 8 * (j & 3);
    if (j < 4) {
        sc = (s03 >> sh) & 63u;
        mn = (s47 >> sh) & 63u;
    } else {
        sc = ((s811 >> sh) & 15u) | (((s03 >> (sh + 6)) & 3u) << 4);
        mn = ((s811 >> (sh + 4)) & 15u) | (((s47 >> (sh + 6)) & 3u) << 4);
    }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Magnitudes an f16 pair (hi + lo) holds with its 22 bits: hi = f16(v)
// overflows at 65520, and keeping below 2^15 leaves lo a normal f16 for
// every |v| >= 2^-3.
constexpr float kPairRange = 32768.0f;

// v as an f16 pair: hi = f16(v) at hi[i], lo = f16(v - hi) at hi[plane + i]
// (the layout the matrix-matrix kernel reads its activations in).
__device__ __forceinline__ void store_hilo(_Float16 *hi, size_t plane, size_t i, float v) {
    const _Float16 h = static_cast<_Float16>(v);
    hi[i] = h;
    hi[plane + i] = static_cast<_Float16>(v - static_cast<float>(h));
}

}  // namespace q8l

// k_misc.hip -- step state, rope table and token embedding kernels.

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

// Writes the per-call state (position, slot, token count, output pointers)
// and up to kInlineTokens token ids. Values come in as kernel arguments, so
// the host buffer they were read from can be reused as soon as the launch
// call returns.
__global__ __launch_bounds__(kThreads) void k_set_state(SetStateArgs a, StepState *st,
                                                       uint32_t *tok_buf) {
    const int tid = threadIdx.x;
    for (int i = tid; i < a.tok_count; i += kThreads) tok_buf[a.tok_offset + i] = a.tokens[i];
    if (tid == 0 && a.set_header) {
        st->pos = a.pos;
        st->slot = a.slot;
        st->T = a.T;
        st->step = a.step;
        st->token = a.tokens[0];
        st->advance = a.advance;
        st->logits_out = a.logits_out;
        st->argmax_out = a.argmax_out;
        st->ids_out = a.ids_out;
    }
}

// The rope table the pages describe ("量化 llama 的一次前向", section
// "from_gguf：键名写死了 llama."): max_seq rows x hd/2 pairs, built once.
// Angle of pair j at position p: f32(p) * f32(theta^(-2j/hd)) rounded to f32
// (one rounding, as a K = 1 f32 matmul gives); cos and sin of that angle are
// evaluated in f64 and stored as f32.
__global__ __launch_bounds__(kThreads) void k_rope_table(float2 *table, int max_seq, int hd,
                                                        double theta) {
    const int half = hd / 2;
    const int64_t n = int64_t(max_seq) * half;
    for (int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x; e < n;
         e += int64_t(gridDim.x) * kThreads) {
        const int p = int(e / half), j = int(e % half);
        const float inv_freq = static_cast<float>(pow(theta, -2.0 * double(j) / double(hd)));
        const float ang = static_cast<float>(p) * inv_freq;
        table[e] = make_float2(static_cast<float>(cos(double(ang))),
                               static_cast<float>(sin(double(ang))));
    }
}

// x[t] = dequant(E[token_t]) -- one workgroup per token, one thread per
// block of 32 weights at a time.
__global__ __launch_bounds__(kThreads) void k_embed(const uint8_t *E, int H, int V,
                                                   const StepState *st, const uint32_t *tok_buf,
                                                   int from_state_token, float *x) {
    const int t = blockIdx.x;
    const uint32_t tok = from_state_token ? st->token : tok_buf[t];
    const int nb = H / kQK;
    float *dst = x + size_t(t) * H;
    if (tok >= uint32_t(V)) {  // only reachable through a device-side token; write zeros
        for (int e = threadIdx.x; e < H; e += kThreads) dst[e] = 0.f;
        return;
    }
    const uint8_t *row = E + size_t(tok) * nb * kQBytes;
    for (int e = threadIdx.x; e < H; e += kThreads) {
        const int b = e / kQK, i = e - b * kQK;
        const uint8_t *blk = row + size_t(b) * kQBytes;
        const uint32_t dbits = uint32_t(blk[0]) | (uint32_t(blk[1]) << 8);
        dst[e] = half_bits_to_float(dbits) * static_cast<float>(static_cast<int8_t>(blk[2 + i]));
    }
}

// An empty kernel: the launch-and-event overhead that timings subtract.
__global__ void k_noop() {}

// The NEOX rope convention ("量化 llama 的一次前向", section "RoPE：两种约定，按架构名
// 选"): dimension j of a head is rotated with dimension j + hd/2 by the table's
// angle for pair j. One workgroup per (token, head); heads [0, nh) are the
// token's q row, heads [nh, nh + nkv) its new key slot in the cache.
// (range_flag, when set: 1 if a rotated value is outside the f16 pairs'
// range of the prefill attention)
__global__ __launch_bounds__(kThreads) void k_rope_neox(const StepState *st, const float2 *rope, float *q,
                                                       float *kc, int nh, int hd, int max_seq, uint32_t *range_flag) {
    const int t = blockIdx.x, h = blockIdx.y;
    const int half = hd / 2;
    float *v = h < nh ? q + (size_t(t) * nh + h) * hd
                      : kc + (size_t(h - nh) * max_seq + st->slot + t) * hd;
    const float2 *cs = rope + size_t(st->pos + t) * half;
    bool bad = false;
    for (int j = threadIdx.x; j < half; j += kThreads) {
        const float x0 = v[j], x1 = v[j + half];
        const float y0 = x0 * cs[j].x - x1 * cs[j].y, y1 = x0 * cs[j].y + x1 * cs[j].x;
        bad |= !(fabsf(y0) < kPairRange) || !(fabsf(y1) < kPairRange);
        v[j] = y0;
        v[j + half] = y1;
    }
    if (bad && range_flag) *range_flag = 1u;
}

// Range check of cached K and V before a prefill reads them: positions
// [lo, hi) of every layer's cache (written by decode steps, whose f32
// arithmetic does not check them). Sets *range_flag to 1 when a value is
// outside the f16 pairs' range. Grid: (float4 chunks of one position range,
// 2 * n_layer * nkv cache rows).
__global__ __launch_bounds__(kThreads) void k_kv_range(const float *kc, const float *vc, size_t layer_stride,
                                                      int nkv, int max_seq, int hd, int lo, int hi,
                                                      uint32_t *range_flag) {
    const int r = blockIdx.y;                  // (cache, layer, kv head)
    const int which = r & 1, lh = r >> 1;
    const int l = lh / nkv, g = lh - l * nkv;
    const float *base = (which ? vc : kc) + size_t(l) * layer_stride + (size_t(g) * max_seq + lo) * hd;
    const size_t n4 = size_t(hi - lo) * hd / 4;
    bool bad = false;
    for (size_t e = size_t(blockIdx.x) * kThreads + threadIdx.x; e < n4; e += size_t(gridDim.x) * kThreads) {
        const float4 v = reinterpret_cast<const float4 *>(base)[e];
        bad |= !(fabsf(v.x) < kPairRange) || !(fabsf(v.y) < kPairRange) || !(fabsf(v.z) < kPairRange) ||
               !(fabsf(v.w) < kPairRange);
    }
    if (bad) *range_flag = 1u;
}

}  // namespace

hipError_t launch_set_state(const SetStateArgs &a, StepState *st, uint32_t *tok_buf,
                            hipStream_t s) {
    hipLaunchKernelGGL(k_set_state, dim3(1), dim3(kThreads), 0, s, a, st, tok_buf);
    return hipGetLastError();
}

hipError_t launch_rope_table(float2 *table, int max_seq, int hd, double theta, hipStream_t s) {
    const int64_t n = int64_t(max_seq) * (hd / 2);
    const unsigned grid = unsigned(std::min<int64_t>((n + kThreads - 1) / kThreads, 4096));
    hipLaunchKernelGGL(k_rope_table, dim3(grid), dim3(kThreads), 0, s, table, max_seq, hd, theta);
    return hipGetLastError();
}

hipError_t launch_embed(const uint8_t *E, int H, int V, const StepState *st,
                        const uint32_t *tok_buf, int T, int from_state_token, float *x,
                        hipStream_t s) {
    hipLaunchKernelGGL(k_embed, dim3(T), dim3(kThreads), 0, s, E, H, V, st, tok_buf,
                       from_state_token, x);
    return hipGetLastError();
}

hipError_t launch_noop(hipStream_t s) {
    hipLaunchKernelGGL(k_noop, dim3(1), dim3(64), 0, s);
    return hipGetLastError();
}

hipError_t launch_rope_neox(const Dims &d, const StepState *st, const float2 *rope, float *q, float *kc,
                            int T, hipStream_t s, uint32_t *range_flag) {
    hipLaunchKernelGGL(k_rope_neox, dim3(T, d.nh + d.nkv), dim3(64), 0, s, st, rope, q, kc, d.nh, d.hd,
                       d.max_seq, T > 1 ? range_flag : nullptr);
    return hipGetLastError();
}

hipError_t launch_kv_range(const float *kc, const float *vc, size_t layer_stride, int n_layer, int nkv, int max_seq,
                           int hd, int lo, int hi, uint32_t *range_flag, hipStream_t s) {
    if (hi <= lo || !range_flag) return hipSuccess;
    const size_t n4 = size_t(hi - lo) * hd / 4;
    const int gx = int(std::min<size_t>((n4 + kThreads - 1) / kThreads, 64));
    hipLaunchKernelGGL(k_kv_range, dim3(gx, 2 * n_layer * nkv), dim3(kThreads), 0, s, kc, vc, layer_stride, nkv,
                       max_seq, hd, lo, hi, range_flag);
    return hipGetLastError();
}

}  // namespace q8l

// k_attn.hip -- grouped-query attention over the preallocated KV cache.
//
// Semantics ("量化 llama 的一次前向", section "forward_attn：自己拼 KV";
// "生成一个 token", section "prefill 和 decode：同一个 forward，不同的路"):
// scores q.k / sqrt(hd); query head h reads KV head h / (n_head / n_head_kv)
// (each KV head serves a run of consecutive query heads); softmax over keys;
// weighted sum of values. A single query (decode) sees every cached key with
// no mask; T > 1 queries see keys j <= prefix + i (prefix = cached positions
// before the call) -- the mask whose first `prefix` columns are open and whose
// last T columns are a causal triangle, applied here as a predicate instead
// of a mask tensor, and without copying KV heads.
//
// Decode: the cache is split into chunks of keys; one workgroup handles one
// chunk for all query heads of one KV head (K/V are read once per group),
// keeps scores and softmax in LDS, and writes (max, sum, unnormalised o)
// partials. The partials are merged in split order by k_attn_combine, so the
// result does not depend on timing and no device-wide atomics are needed;
// when the cache fits one split, the workgroup writes the normalised output
// itself (the merge of one split is that division).
//
// Prefill (head size 64 or 128): one workgroup per (64 queries, head) on
// MFMA, key blocks of 64 staged in LDS as f16 pairs, online softmax per
// query; long prompts cut each query block's keys into up to kMaxPfSplits
// ranges on separate workgroups, merged in range order by
// k_attn_prefill_merge. Other head sizes: one workgroup per (32 queries,
// head) in f32 (k_attn_prefill).

#include <algorithm>

#include "device_common.h"

namespace q8l {

namespace {

struct DecodeLds {
    float *q;    // G * hd
    float *k;    // chunk * (hd + 4): rows padded to keep 16-byte reads conflict-free
    float *v;    // chunk * hd
    float *p;    // (kThreads / 64) * chunk: each wave's softmax numerators
};

constexpr int kKvPer = 4;   // float4 per thread of a K (or V) tile: 64 x 64 or 32 x 128 floats
constexpr int kQPer = 2;    // float4 per thread of a group's queries (G * hd <= 2048 floats)
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline DecodeLds carve_decode(uint8_t *smem, int G, int hd) {
    const int C = attn_chunk(hd);
    DecodeLds L;
    float *p = reinterpret_cast<float *>(smem);
    L.q = p; p += G * hd;
    L.k = p; p += C * (hd + kKPad);
    L.v = p; p += C * hd;
    L.p = p;
    return L;
}

// The G query heads of KV group g against keys [j0, j0 + nk) of the cache
// (nk <= the split size, <= 64): q and the key/value tile are staged in LDS
// by the whole workgroup, then wave w takes heads w, w + 4, ...:
//   scores  lane j: q_h . k_j (four partial sums over d, then
//           (s0 + s1) + (s2 + s3)), times the scale;
//   softmax max over the lanes, e_j = exp(s_j - max), l = sum of e_j
//           (DPP reductions, no barrier);
//   output  lane d (and d + 64): sum over j in key order of e_j * v_j[d],
//           e_j read back (four at a time) from the wave's row of L.p.
// out(h, d, acc, max, l) receives each unnormalised output.
template <class Out>
__device__ __forceinline__ void attn_group_split(const AttnDecodeArgs &a, const DecodeLds &L, int g, int j0,
                                                 int nk, Out &&out) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int hd = a.hd, G = a.nh / a.nkv;
    const int C = attn_chunk(hd);
    // 16-byte loads (hd % 8 == 0; the cache and the V tile are 16-byte aligned)
    const f32x4 *qg = reinterpret_cast<const f32x4 *>(a.q + size_t(g) * G * hd);
    const f32x4 *kb = reinterpret_cast<const f32x4 *>(a.kc + (size_t(g) * a.kv_stride + j0) * hd);
    const f32x4 *vb = reinterpret_cast<const f32x4 *>(a.vc + (size_t(g) * a.kv_stride + j0) * hd);
    // Every load of q and of the tile is issued before the first LDS store,
    // so they cost one memory round trip together (G * hd <= kQPer * kThreads
    // float4 of q; chunk * hd <= kKvPer * kThreads float4 of K and of V). The
    // tile's loads cover the whole chunk that the cache holds from j0 on (not
    // only the nk keys in use, which are known only from the step state), so
    // the issue does not wait for that state. Indexes past q or past the
    // cache re-read the last float4 (in bounds), and every loaded register is
    // stored without a condition (q's extra copies onto its last float4,
    // the tile's onto rows past nk that are never read): a load used under a
    // condition would be sunk into it, one round trip per load.
    const int nq4 = G * hd / 4;
    const int last = min(C, a.kv_stride - j0) * hd / 4 - 1;
    f32x4 qr[kQPer], kr[kKvPer], vr[kKvPer];
#pragma unroll
    for (int i = 0; i < kQPer; ++i) qr[i] = qg[min(tid + i * kThreads, nq4 - 1)];
#pragma unroll
    for (int i = 0; i < kKvPer; ++i) {
        const int e4 = min(tid + i * kThreads, last);
        kr[i] = kb[e4];
        vr[i] = vb[e4];
    }
#pragma unroll
    for (int i = 0; i < kQPer; ++i) reinterpret_cast<f32x4 *>(L.q)[min(tid + i * kThreads, nq4 - 1)] = qr[i];
    // Destinations past the chunk (head sizes whose chunk is under 4096
    // floats) go to its last float4: every such store carries the value
    // loaded from index `last`, which is also what that slot's own thread
    // loaded (min(C * hd / 4 - 1, last) == last whenever the cache is short).
    const int tile4 = C * hd / 4 - 1;
#pragma unroll
    for (int i = 0; i < kKvPer; ++i) {
        const int e = 4 * min(tid + i * kThreads, tile4), j = e / hd, d = e - j * hd;
        *reinterpret_cast<f32x4 *>(L.k + j * (hd + kKPad) + d) = kr[i];
        *reinterpret_cast<f32x4 *>(L.v + e) = vr[i];
    }
    __syncthreads();
    for (int h = wid; h < G; h += kThreads / 64) {
        const float *qh = L.q + h * hd;
        float sc = -INFINITY;
        if (lane < nk) {
            const float *kj = L.k + lane * (hd + kKPad);
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 4
            for (int d = 0; d < hd; d += 4) {
                const float4 qv = *reinterpret_cast<const float4 *>(qh + d);
                const float4 kv = *reinterpret_cast<const float4 *>(kj + d);
                s0 = fmaf(qv.x, kv.x, s0);
                s1 = fmaf(qv.y, kv.y, s1);
                s2 = fmaf(qv.z, kv.z, s2);
                s3 = fmaf(qv.w, kv.w, s3);
            }
            sc = ((s0 + s1) + (s2 + s3)) * a.scale;
        }
        const float mx = wave_max_dpp(sc);
        const float e = lane < nk ? expf(sc - mx) : 0.f;
        const float l = wave_sum_dpp(e);
        float *pw = L.p + wid * C;   // this wave's row: written and read by the wave alone
        if (lane < C) pw[lane] = e;
        __builtin_amdgcn_wave_barrier();
        for (int d = lane; d < hd; d += 64) {
            float acc = 0.f;
            int j = 0;
#pragma unroll 2
            for (; j + 4 <= nk; j += 4) {
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(pw + j);
                acc = fmaf(e4.x, L.v[j * hd + d], acc);
                acc = fmaf(e4.y, L.v[(j + 1) * hd + d], acc);
                acc = fmaf(e4.z, L.v[(j + 2) * hd + d], acc);
                acc = fmaf(e4.w, L.v[(j + 3) * hd + d], acc);
            }
            for (; j < nk; ++j) acc = fmaf(pw[j], L.v[j * hd + d], acc);
            out(h, d, acc, mx, l);
        }
        __builtin_amdgcn_wave_barrier();   // the row is rewritten for the wave's next head
    }
}

__global__ __launch_bounds__(kThreads) void k_attn_decode(AttnDecodeArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int s = blockIdx.x, g = blockIdx.y;
    const int hd = a.hd, G = a.nh / a.nkv;
    const int C = attn_chunk(hd);
    const int kv_len = a.kv_len_arg >= 0 ? a.kv_len_arg : a.st->slot + 1;
    const int active = min((kv_len + C - 1) / C, a.n_splits);
    if (s >= active) return;
    const DecodeLds L = carve_decode(smem, G, hd);
    const int j0 = s * C;
    attn_group_split(a, L, g, j0, min(C, kv_len - j0), [&](int h, int d, float acc, float mx, float l) {
        if (a.o) {  // the only split: its normalised output (what the merge of one split computes)
            a.o[size_t(g * G + h) * hd + d] = acc / l;
            return;
        }
        float *pp = a.part + (size_t(g * G + h) * a.n_splits + s) * (hd + 2);
        pp[2 + d] = acc;
        if (d == 0) {
            pp[0] = mx;
            pp[1] = l;
        }
    });
}

// Decode attention of a cache that fits one split, fused with the
// o-projection as a sum over KV groups: workgroup (g, row chunk) computes the
// normalised output of group g's heads and multiplies it by the matching
// columns of W_o (this group's G*hd columns, whole 64-weight pairs) for its
// rows, writing part[g][row] = sum over those columns. The residual add of
// sum_g part[g] is the prologue of the next kernel with a norm in front. Every
// workgroup of a group recomputes the same attention (at most one split of
// keys: a few KB of K/V from L2); the workgroup's W_o pairs are loaded into
// registers first and are in flight during the attention. FMT: W_o's block
// format (Q8_0 or Q5_0 pairs).
template <int FMT>
__device__ __forceinline__ void attn_o_body(const AttnODecodeArgs &b) {
    constexpr int PB = FMT == F_Q5_0 ? kQ5PairBytes : kPairBytes;
    extern __shared__ __align__(16) uint8_t smem[];
    const AttnDecodeArgs &a = b.at;
    const int tid = threadIdx.x;
    const int g = blockIdx.x % a.nkv, r0 = (blockIdx.x / a.nkv) * b.rows;
    const int hd = a.hd, G = a.nh / a.nkv, C = attn_chunk(hd);
    const int Pg = G * hd / kPairWeights;   // pairs of this group's columns in one row of W_o
    const int P = a.nh * hd / kPairWeights; // pairs per row
    const int nr = min(b.rows, b.N - r0);
    const int units = nr * Pg;              // <= kThreads (host-checked)
    uint32_t w[PB / 4];
    if (tid < units) {
        const int r = tid / Pg, p = tid - r * Pg;
        const uint32_t *src =
            reinterpret_cast<const uint32_t *>(b.wo + (size_t(r0 + r) * P + size_t(g) * Pg + p) * PB);
#pragma unroll
        for (int i = 0; i < PB / 4; ++i) w[i] = src[i];
    }
    const DecodeLds L = carve_decode(smem, G, hd);
    float *xs = reinterpret_cast<float *>(smem + attn_o_xs_offset(G, hd));  // Pg * kOPad: the group's output
    float *red = xs + Pg * kOPad;                                           // units
    const int kv_len = min(a.st->slot + 1, C);
    attn_group_split(a, L, g, 0, kv_len, [&](int h, int d, float acc, float, float l) {
        const int k = h * hd + d;
        xs[(k / kPairWeights) * kOPad + (k % kPairWeights)] = acc / l;
    });
    __syncthreads();
    if (tid < units) {
        float dA, sA, dB, sB;
        if (FMT == F_Q5_0)
            pair_dot1_q5(w, xs + (tid % Pg) * kOPad, dA, sA, dB, sB);
        else
            pair_dot1(w, xs + (tid % Pg) * kOPad, dA, sA, dB, sB);
        red[tid] = fmaf(dB, sB, dA * sA);
    }
    __syncthreads();
    for (int r = tid; r < nr; r += kThreads) {
        float v = red[r * Pg];
        for (int p = 1; p < Pg; ++p) v += red[r * Pg + p];
        b.part[size_t(g) * b.N + r0 + r] = v;
    }
}

__global__ __launch_bounds__(kThreads) void k_attn_o1(AttnODecodeArgs b) { attn_o_body<F_Q8_0>(b); }
__global__ __launch_bounds__(kThreads) void k_attn_o1_q5(AttnODecodeArgs b) { attn_o_body<F_Q5_0>(b); }

// Merge the split partials of the decode attention into O: one workgroup per
// query head. The split weights w_s = exp(m_s - M) (M = max over splits) are
// computed once per split into LDS; then o[d] = sum_s w_s o_s[d] / sum_s w_s l_s,
// every sum in split order (the result does not depend on timing).
constexpr int kCombinePre = 32;   // partial outputs per thread loaded before the weights are known

__global__ __launch_bounds__(kThreads) void k_attn_combine(const float *part, int n_splits,
                                                          int active, int hd, float *o,
                                                          const StepState *st) {
    extern __shared__ float w[];  // n_splits
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int h = blockIdx.x;
    const float *pb = part + size_t(h) * n_splits * (hd + 2);
    // Many splits: kThreads / hd interleaved slices of the splits (slice j:
    // splits j, j + P, ...), each summed in split order, then the slices in
    // order -- P shorter dependent chains instead of one of `active` steps
    // (135M, 63 splits: 997 -> 979 us/token; with 17 splits the extra
    // exchange cost more than it saved). Otherwise thread d sums every split.
    // In graph replay (st set) the choice follows the launch's split count,
    // a power of two of which more than half are in use, so it is the same
    // as from the count in use without waiting for it.
    const bool sliced = (st ? n_splits > 32 : active > 32) && hd <= kThreads && kThreads % hd == 0;
    const int P = sliced ? kThreads / hd : 1;
    const int j = sliced ? tid / hd : 0, d = sliced ? tid - j * hd : tid;
    const bool outs = d < hd && j < P;
    // This thread's first kCombinePre partial outputs and its first split's
    // (max, sum), requested before the count in use is known (a read of the
    // step state: a round trip of its own), so that they arrive together
    // (in bounds: clamped to the launch's splits; those past the count in
    // use are never summed)
    float pre[kCombinePre];
#pragma unroll
    for (int k = 0; k < kCombinePre; ++k)
        pre[k] = pb[size_t(min(j + k * P, n_splits - 1)) * (hd + 2) + 2 + min(d, hd - 1)];
    const int t0 = min(tid, n_splits - 1);
    const float m0 = pb[size_t(t0) * (hd + 2)], l0 = pb[size_t(t0) * (hd + 2) + 1];
    if (st) {  // graph replay: the cache length comes from the step state
        const int C = attn_chunk(hd);
        active = min((st->slot + 1 + C - 1) / C, n_splits);
    }
    float mx = tid < active ? m0 : -INFINITY;
    for (int t = tid + kThreads; t < active; t += kThreads) mx = fmaxf(mx, pb[size_t(t) * (hd + 2)]);
    mx = wave_max(mx);
    if (lane == 0) red[wid] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float ls = 0.f;
    if (tid < active) {
        const float wt = expf(m0 - mx);
        w[tid] = wt;
        ls = fmaf(wt, l0, ls);
    }
    for (int t = tid + kThreads; t < active; t += kThreads) {
        const float wt = expf(pb[size_t(t) * (hd + 2)] - mx);
        w[t] = wt;
        ls = fmaf(wt, pb[size_t(t) * (hd + 2) + 1], ls);
    }
    ls = block_sum(ls, red);  // its barriers also publish w[]
    const float inv = 1.0f / ls;
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kCombinePre; ++k)
        if (j + k * P < active) acc = fmaf(w[j + k * P], pre[k], acc);
    for (int t = j + kCombinePre * P; t < active; t += P) acc = fmaf(w[t], pb[size_t(t) * (hd + 2) + 2 + d], acc);
    if (sliced) {
        __shared__ float acc_s[kThreads];
        acc_s[tid] = acc;
        __syncthreads();
        if (j == 0) {
            float sum = acc_s[d];
            for (int q = 1; q < P; ++q) sum += acc_s[q * hd + d];
            o[size_t(h) * hd + d] = sum * inv;
        }
        return;
    }
    if (outs) o[size_t(h) * hd + d] = acc * inv;
}

constexpr int kQB = 32;   // queries per prefill workgroup
constexpr int kKT = 32;   // keys per prefill tile

__global__ __launch_bounds__(kThreads) void k_attn_prefill(AttnPrefillArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int qi = tid >> 3, sub = tid & 7;
    const int hd = a.hd, G = a.nh / a.nkv;
    const int h = blockIdx.y, g = h / G;
    const int q0 = blockIdx.x * kQB;
    const int nq = min(kQB, a.T - q0);
    const int prefix = a.kv_len - a.T;
    const int row_stride = a.nh * hd;

    float *Qs = reinterpret_cast<float *>(smem);       // kQB * (hd + 1)
    float *Ks = Qs + kQB * (hd + 1);                    // kKT * (hd + 1)
    float *Vs = Ks + kKT * (hd + 1);                    // kKT * hd
    float *Ps = Vs + kKT * hd;                          // kQB * kKT

    for (int e = tid; e < kQB * hd; e += kThreads) {
        const int i = e / hd, d = e - i * hd;
        Qs[i * (hd + 1) + d] = (i < nq) ? a.q[size_t(q0 + i) * row_stride + h * hd + d] : 0.f;
    }
    const int ndim = hd / 8;  // output dims per thread (hd % 8 == 0)
    float o[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = 0.f;
    float m = -INFINITY, lsum = 0.f;
    const int my_last = prefix + q0 + qi;                  // last visible key of this row
    const int blk_last = prefix + q0 + nq - 1;             // last key any row sees
    const float *kb = a.kc + size_t(g) * a.kv_stride * hd;
    const float *vb = a.vc + size_t(g) * a.kv_stride * hd;

    for (int j0 = 0; j0 <= blk_last; j0 += kKT) {
        const int nk = min(kKT, blk_last + 1 - j0);
        __syncthreads();
        for (int e = tid; e < kKT * hd; e += kThreads) {
            const int j = e / hd, d = e - j * hd;
            const bool in = j < nk;
            Ks[j * (hd + 1) + d] = in ? kb[size_t(j0 + j) * hd + d] : 0.f;
            Vs[e] = in ? vb[size_t(j0 + j) * hd + d] : 0.f;
        }
        __syncthreads();
        float sv[kKT / 8];
        float tmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < kKT / 8; ++u) {
            const int jj = sub + 8 * u;
            const int j = j0 + jj;
            float sc = -INFINITY;
            if (qi < nq && jj < nk && j <= my_last) {
                const float *qr = Qs + qi * (hd + 1);
                const float *kr = Ks + jj * (hd + 1);
                float s0 = 0.f, s1 = 0.f;
                for (int d = 0; d < hd; d += 2) {
                    s0 = fmaf(qr[d], kr[d], s0);
                    s1 = fmaf(qr[d + 1], kr[d + 1], s1);
                }
                sc = (s0 + s1) * a.scale;
            }
            sv[u] = sc;
            tmax = fmaxf(tmax, sc);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 4, 64));
        const float m_new = fmaxf(m, tmax);
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < kKT / 8; ++u) {
            const float pv = (sv[u] == -INFINITY) ? 0.f : expf(sv[u] - m_new);
            Ps[qi * kKT + sub + 8 * u] = pv;
            psum += pv;
        }
        psum += __shfl_xor(psum, 1, 64);
        psum += __shfl_xor(psum, 2, 64);
        psum += __shfl_xor(psum, 4, 64);
        lsum = lsum * alpha + psum;
        m = m_new;
        __syncthreads();
        const float *pr = Ps + qi * kKT;
        for (int k = 0; k < ndim; ++k) {
            const int d = sub + 8 * k;
            float acc = 0.f;
            for (int jj = 0; jj < nk; ++jj) acc = fmaf(pr[jj], Vs[jj * hd + d], acc);
            o[k] = o[k] * alpha + acc;
        }
    }
    if (qi < nq) {
        const size_t base = size_t(q0 + qi) * row_stride + h * hd;
        if (a.o_split) {
            const size_t plane = size_t(a.T) * row_stride;
            bool bad = false;
            for (int k = 0; k < ndim; ++k) {
                bad |= !(fabsf(o[k] / lsum) < kPairRange);
                store_hilo(a.o_split, plane, base + sub + 8 * k, o[k] / lsum);
            }
            if (bad && a.range_flag) *a.range_flag = 1u;
        } else {
            for (int k = 0; k < ndim; ++k) a.o[base + sub + 8 * k] = o[k] / lsum;
        }
    }
}

// ---------------------------------------------------------------- prefill on MFMA
//
// One workgroup = 64 queries of one head; each wave owns 16 queries. Per
// block of 64 keys:
//   S^T[key][query] = K . Q^T   (contraction over hd, 3 f16 MFMAs per 32:
//                                 Kh.Qh + Kl.Qh + Kh.Ql, Q pre-scaled)
//   online softmax per query column in f32 (each lane holds one query)
//   O^T[d][query] += V^T . P^T  (contraction over keys)
// In the S^T accumulator a lane holds keys 4*(l/16)+i of one 16-key tile for
// query l%16. The P^T . V contraction runs over keys in the order
// slot 8*(l/16)+j -> key (j < 4 ? 4*(l/16)+j : 16 + 4*(l/16)+j-4) of each
// 32-key step, so the S accumulators are the B operand as they stand and only
// the V^T operand is gathered in that order from LDS.

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FQ = 64;    // queries per workgroup
constexpr int kPfMinChunk = 4;   // key blocks per range at least (shorter prompts are not split)
constexpr int FK = 64;    // keys per block

template <int HD>
struct FlashLds {
    _Float16 kh[FK * (HD + 8)];     // K [key][d]
    _Float16 kl[FK * (HD + 8)];
    _Float16 vh[HD * (FK + 8)];     // V^T [d][slot]: keys in P^T slot order
    _Float16 vl[HD * (FK + 8)];
};

__device__ __forceinline__ void split16(float v, _Float16 &hi, _Float16 &lo) {
    hi = static_cast<_Float16>(v);
    lo = static_cast<_Float16>(v - static_cast<float>(hi));
}

// Four values as f16 pairs. (Q, K and V are range-checked where they are
// written: the q/k/v kernels of a prefill, and a check of the cached
// positions a decode step wrote before a prefill reads them.)
__device__ __forceinline__ void split4(const float v[4], uint2 &hi, uint2 &lo) {
    _Float16 h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split16(v[i], h[i], l[i]);
    hi = __builtin_bit_cast(uint2, h);
    lo = __builtin_bit_cast(uint2, l);
}

// Slot of key k (0..FK-1, a multiple of 4) in the P^T operand order: within a
// 32-key step, keys 4g..4g+3 sit in slots 8g..8g+3 and keys 16+4g..16+4g+3 in
// slots 8g+4..8g+7.
__device__ __forceinline__ int key_slot(int k) {
    const int kk = k & 31;
    return (k & ~31) + 8 * ((kk & 15) >> 2) + 4 * (kk >> 4);
}

// One key block of K and V in registers (loaded a block ahead).
template <int HD>
struct KvRegs {
    float4 k[FK * HD / 4 / kThreads];
    float v[FK * HD / kThreads];
};

template <int HD>
__device__ __forceinline__ void kv_load(const float *kb, const float *vb, int j0, int blk_last, KvRegs<HD> &r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < FK * HD / 4 / kThreads; ++i) {
        const int e = tid + i * kThreads;
        const int j = e / (HD / 4), d4 = (e - j * (HD / 4)) * 4;
        r.k[i] = (j0 + j <= blk_last) ? *reinterpret_cast<const float4 *>(kb + size_t(j0 + j) * HD + d4)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < FK * HD / 4 / kThreads; ++i) {
        const int e = tid + i * kThreads;       // (quad of keys, d): consecutive threads, consecutive d
        const int quad = e / HD, d = e - quad * HD;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = j0 + 4 * quad + t;
            r.v[4 * i + t] = (key <= blk_last) ? vb[size_t(key) * HD + d] : 0.f;
        }
    }
}

template <int HD>
__device__ __forceinline__ void kv_store(const KvRegs<HD> &r, FlashLds<HD> &L) {
    constexpr int LD = HD + 8, LV = FK + 8;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < FK * HD / 4 / kThreads; ++i) {
        const int e = tid + i * kThreads;
        const int j = e / (HD / 4), d4 = (e - j * (HD / 4)) * 4;
        const float kk[4] = {r.k[i].x, r.k[i].y, r.k[i].z, r.k[i].w};
        uint2 hi, lo;
        split4(kk, hi, lo);
        *reinterpret_cast<uint2 *>(L.kh + j * LD + d4) = hi;
        *reinterpret_cast<uint2 *>(L.kl + j * LD + d4) = lo;
    }
#pragma unroll
    for (int i = 0; i < FK * HD / 4 / kThreads; ++i) {
        const int e = tid + i * kThreads;
        const int quad = e / HD, d = e - quad * HD;
        uint2 hi, lo;
        split4(&r.v[4 * i], hi, lo);
        const int slot = key_slot(4 * quad);
        *reinterpret_cast<uint2 *>(L.vh + d * LV + slot) = hi;
        *reinterpret_cast<uint2 *>(L.vl + d * LV + slot) = lo;
    }
}

// Key blocks of FK that query block qb (queries qb * FQ ..) reaches.
__host__ __device__ inline int prefix_blocks(int prefix, int qb, int T) {
    return (prefix + min((qb + 1) * FQ, T) - 1) / FK + 1;
}

// KS: query blocks may split their key range (a.pf_chunk > 0); without it
// every workgroup takes a whole query block.
template <int HD, bool KS>
__global__ __launch_bounds__(kThreads) void k_attn_prefill_mfma(AttnPrefillArgs a) {
    __shared__ __align__(16) FlashLds<HD> L;
    constexpr int LD = HD + 8, LV = FK + 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.nh / a.nkv;
    const int h = blockIdx.y, g = h / G;
    const int prefix = a.kv_len - a.T;
    // causal work grows with the query block: start the longest blocks first.
    // With key splits, workgroup x takes key range sp of the query blocks
    // taken from the last one down (ns ranges of pf_chunk key blocks each).
    const int nqb = (a.T + FQ - 1) / FQ;
    int qb = nqb - 1 - int(blockIdx.x), sp = 0, ns = 1;
    if constexpr (KS) {
        int w = blockIdx.x;
        for (qb = nqb - 1;; --qb) {
            ns = (prefix_blocks(prefix, qb, a.T) + a.pf_chunk - 1) / a.pf_chunk;
            if (w < ns || qb == 0) break;
            w -= ns;
        }
        if (w >= ns) return;   // (past the work: the grid is sized to it)
        sp = w;
    }
    const int q0 = qb * FQ;
    const int row_stride = a.nh * HD;
    const int qi = q0 + wave * 16 + (lane & 15);   // this lane's query
    const int grp = lane >> 4;

    // Q^T fragments (B operand): lane holds Q[qi][32*s + 8*grp + j], pre-scaled
    // by 1/sqrt(hd) * log2(e) so that the softmax runs on exp2
    const float qscale = a.scale * 1.4426950408889634f;
    half8 qh[HD / 32], ql[HD / 32];
#pragma unroll
    for (int s = 0; s < HD / 32; ++s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float v = (qi < a.T) ? a.q[size_t(qi) * row_stride + h * HD + 32 * s + 8 * grp + j] * qscale : 0.f;
            _Float16 hi, lo;
            split16(v, hi, lo);
            qh[s][j] = hi;
            ql[s][j] = lo;
        }

    f32x4 o[HD / 16];
#pragma unroll
    for (int t = 0; t < HD / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.f;
    const int last_q = min(q0 + FQ, a.T) - 1;
    const int blk_last = prefix + last_q;                // last key any query of the block sees
    const float *kb = a.kc + size_t(g) * a.kv_stride * HD;
    const float *vb = a.vc + size_t(g) * a.kv_stride * HD;

    // this workgroup's keys: all of the block's, or key blocks
    // [sp * pf_chunk, (sp + 1) * pf_chunk)
    const int j_first = ns > 1 ? sp * a.pf_chunk * FK : 0;
    const int j_last = ns > 1 ? min(blk_last, (sp + 1) * a.pf_chunk * FK - 1) : blk_last;
    KvRegs<HD> kv;
    kv_load<HD>(kb, vb, j_first, j_last, kv);
    for (int j0 = j_first; j0 <= j_last; j0 += FK) {
        __syncthreads();  // the previous block's LDS tiles are no longer read
        kv_store<HD>(kv, L);
        __syncthreads();
        if (j0 + FK <= j_last) kv_load<HD>(kb, vb, j0 + FK, j_last, kv);
        // S^T for 4 key tiles of 16
        f32x4 st[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            const int key = kt * 16 + (lane & 15);
#pragma unroll
            for (int s = 0; s < HD / 32; ++s) {
                const half8 ah = *reinterpret_cast<const half8 *>(L.kh + key * LD + 32 * s + 8 * grp);
                const half8 al = *reinterpret_cast<const half8 *>(L.kl + key * LD + 32 * s + 8 * grp);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, qh[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, qh[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, ql[s], acc, 0, 0, 0);
            }
            st[kt] = acc;
        }
        // mask keys beyond the causal limit of this query (or beyond kv_len):
        // only blocks that reach past the first query's limit need it
        if (j0 + FK - 1 > prefix + q0) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = j0 + kt * 16 + 4 * grp + i;
                    const bool vis = key <= prefix + qi && key <= blk_last;
                    st[kt][i] = vis ? st[kt][i] : -INFINITY;
                }
        }
        float bmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, st[kt][i]);
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        // Scores are in log2 units (Q carries log2(e)). Key 0 is visible to
        // every query, so with the whole key range m_new is finite and
        // exp2(-inf) = 0 handles masked keys and the first block's alpha. A
        // later key range can hold no visible key of a query yet (m_new still
        // -inf): its exponentials are taken against 0 instead and give 0.
        const float m_new = fmaxf(m, bmax);
        const float m_ref = KS && m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
        float psum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(st[kt][i] - m_ref);
                st[kt][i] = p;
                psum += p;
            }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        lsum = lsum * alpha + psum;
        m = m_new;
        // P^T as the B operand for two 32-key steps: keys {kt=2s, kt=2s+1}
        half8 ph[2], pl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = (j < 4) ? st[2 * s][j] : st[2 * s + 1][j - 4];
                _Float16 hi, lo;
                split16(p, hi, lo);
                ph[s][j] = hi;
                pl[s][j] = lo;
            }
#pragma unroll
        for (int t = 0; t < HD / 16; ++t) {
            f32x4 acc = o[t] * alpha;
            const int d = t * 16 + (lane & 15);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const half8 vh = *reinterpret_cast<const half8 *>(L.vh + d * LV + 32 * s + 8 * grp);
                const half8 vl = *reinterpret_cast<const half8 *>(L.vl + d * LV + 32 * s + 8 * grp);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, ph[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(vl, ph[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh, pl[s], acc, 0, 0, 0);
            }
            o[t] = acc;
        }
    }
    if (KS && ns > 1) {   // one key range of several: (max in log2 units, sum, unnormalised o)
        if (qi < a.T) {
            float *pp = a.pf_part + ((size_t(h) * a.T + qi) * kMaxPfSplits + sp) * (HD + 2);
#pragma unroll
            for (int t = 0; t < HD / 16; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) pp[2 + t * 16 + 4 * grp + i] = o[t][i];
            if (grp == 0) {
                pp[0] = m;
                pp[1] = lsum;
            }
        }
        return;
    }
    if (qi < a.T) {
        const float inv = 1.0f / lsum;
        const size_t base = size_t(qi) * row_stride + h * HD;
        if (a.o_split) {
            const size_t plane = size_t(a.T) * row_stride;
            bool bad = false;   // an output outside the f16 pairs' range
#pragma unroll
            for (int t = 0; t < HD / 16; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ov = o[t][i] * inv;
                    bad |= !(fabsf(ov) < kPairRange);
                    store_hilo(a.o_split, plane, base + t * 16 + 4 * grp + i, ov);
                }
            if (bad && a.range_flag) *a.range_flag = 1u;
        } else {
            float *dst = a.o + base;
#pragma unroll
            for (int t = 0; t < HD / 16; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[t * 16 + 4 * grp + i] = o[t][i] * inv;
        }
    }
}

// Merge of the key ranges of the query blocks that were split: one wave per
// (query, head), queries from q_begin; lane d (and d + 64) of the output.
// o = sum_s w_s o_s / sum_s w_s l_s, w_s = exp2(m_s - M), M the largest m_s,
// sums in range order (the result does not depend on timing). Written as the
// attention kernel writes an unsplit block (f32, or the f16 pair planes with
// the range check).
template <int HD>
__global__ __launch_bounds__(kThreads) void k_attn_prefill_merge(AttnPrefillArgs a, int q_begin) {
    constexpr int DL = HD / 64;   // output values per lane
    const int lane = threadIdx.x & 63;
    const int qi = q_begin + int(blockIdx.x) * (kThreads / 64) + int(threadIdx.x >> 6), h = blockIdx.y;
    if (qi >= a.T) return;   // (no barriers in this kernel)
    const int prefix = a.kv_len - a.T;
    const int ns = (prefix_blocks(prefix, qi / FQ, a.T) + a.pf_chunk - 1) / a.pf_chunk;
    if (ns <= 1) return;     // written by the attention kernel itself
    const float *pp = a.pf_part + (size_t(h) * a.T + qi) * kMaxPfSplits * (HD + 2);
    float ms[kMaxPfSplits], ls[kMaxPfSplits], ov[kMaxPfSplits][DL];
#pragma unroll
    for (int s = 0; s < kMaxPfSplits; ++s) {
        const float *ps = pp + size_t(min(s, ns - 1)) * (HD + 2);
        ms[s] = ps[0];
        ls[s] = ps[1];
#pragma unroll
        for (int j = 0; j < DL; ++j) ov[s][j] = ps[2 + lane + 64 * j];
    }
    float M = ms[0];
#pragma unroll
    for (int s = 1; s < kMaxPfSplits; ++s)
        if (s < ns) M = fmaxf(M, ms[s]);
    float L = 0.f, acc[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxPfSplits; ++s) {
        if (s < ns) {
            const float w = __builtin_amdgcn_exp2f(ms[s] - M);
            L = fmaf(w, ls[s], L);
#pragma unroll
            for (int j = 0; j < DL; ++j) acc[j] = fmaf(w, ov[s][j], acc[j]);
        }
    }
    const float inv = 1.0f / L;
    const int row_stride = a.nh * HD;
    const size_t base = size_t(qi) * row_stride + h * HD;
    if (a.o_split) {
        const size_t plane = size_t(a.T) * row_stride;
        bool bad = false;
#pragma unroll
        for (int j = 0; j < DL; ++j) {
            const float v = acc[j] * inv;
            bad |= !(fabsf(v) < kPairRange);
            store_hilo(a.o_split, plane, base + lane + 64 * j, v);
        }
        if (bad && a.range_flag) *a.range_flag = 1u;
    } else {
#pragma unroll
        for (int j = 0; j < DL; ++j) a.o[base + lane + 64 * j] = acc[j] * inv;
    }
}

}  // namespace

int attn_prefill_chunk(int kv_len) {
    const int nb = (kv_len + FK - 1) / FK;
    const int c = (nb + kMaxPfSplits - 1) / kMaxPfSplits;
    return c >= kPfMinChunk ? c : 0;
}

int attn_decode_splits(int kv_len, int hd) {
    const int C = attn_chunk(hd);
    return (kv_len + C - 1) / C;
}

hipError_t launch_attn_decode(const AttnDecodeArgs &a, hipStream_t s) {
    const size_t lds = attn_decode_lds(a.nh / a.nkv, a.hd);
    hipLaunchKernelGGL(k_attn_decode, dim3(a.n_splits, a.nkv), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

size_t attn_o_lds(int G, int hd, int rows) {
    const int Pg = G * hd / kPairWeights;
    return attn_o_xs_offset(G, hd) + sizeof(float) * (size_t(Pg) * kOPad + size_t(rows) * Pg);
}

bool attn_o_fits(const Dims &d) {
    const int G = d.nh / d.nkv;
    return (G * d.hd) % kPairWeights == 0 && G * d.hd / kPairWeights <= kThreads;
}

int attn_o_rows(const Dims &d) {
    const int Pg = d.nh / d.nkv * d.hd / kPairWeights;
    const int want = (kAttnOWgs + d.nkv - 1) / d.nkv;          // row chunks per group
    const int rows = (d.H + want - 1) / want;
    return std::max(1, std::min(rows, kThreads / Pg));
}

hipError_t launch_attn_o(const AttnDecodeArgs &a, const uint8_t *wo, int N, float *part, hipStream_t s, int fmt) {
    Dims d{};
    d.H = N; d.nh = a.nh; d.nkv = a.nkv; d.hd = a.hd;
    if (!attn_o_fits(d) || (fmt != F_Q8_0 && fmt != F_Q5_0)) return hipErrorInvalidValue;
    AttnODecodeArgs b;
    b.at = a;
    b.wo = wo; b.N = N; b.part = part;

    b.rows = attn_o_rows(d);
    const int chunks = (N + b.rows - 1) / b.rows;
    hipLaunchKernelGGL(fmt == F_Q5_0 ? k_attn_o1_q5 : k_attn_o1, dim3(chunks * a.nkv), dim3(kThreads),
                       attn_o_lds(a.nh / a.nkv, a.hd, b.rows), s, b);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const float *part, int n_splits, int kv_len, int nh, int hd,
                               float *o, const StepState *st, hipStream_t s) {
    const int active = std::min((kv_len + attn_chunk(hd) - 1) / attn_chunk(hd), n_splits);
    const size_t lds = size_t(n_splits) * sizeof(float);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_combine, dim3(nh), dim3(kThreads), lds, s, part, n_splits, active, hd, o, st);
    return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnPrefillArgs &a, hipStream_t s) {
    if (a.hd == 64 || a.hd == 128) {
        const int nqb = (a.T + FQ - 1) / FQ, prefix = a.kv_len - a.T;
        // key splits: the workgroups of every query block, and the first
        // query whose block is split
        int wgs = nqb, q_split = a.T;
        if (a.pf_part && a.pf_chunk > 0) {
            if (a.pf_chunk * kMaxPfSplits < prefix_blocks(prefix, nqb - 1, a.T)) return hipErrorInvalidValue;
            wgs = 0;
            for (int qb = 0; qb < nqb; ++qb) {
                const int ns = (prefix_blocks(prefix, qb, a.T) + a.pf_chunk - 1) / a.pf_chunk;
                wgs += ns;
                if (ns > 1 && q_split == a.T) q_split = qb * FQ;
            }
        }
        AttnPrefillArgs b = a;
        const bool ks = a.pf_part && a.pf_chunk > 0;
        if (!ks) b.pf_chunk = 0;
        dim3 grid(wgs, a.nh);
        void (*kern)(AttnPrefillArgs);
        if (a.hd == 64)
            kern = ks ? k_attn_prefill_mfma<64, true> : k_attn_prefill_mfma<64, false>;
        else
            kern = ks ? k_attn_prefill_mfma<128, true> : k_attn_prefill_mfma<128, false>;
        hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, b);
        if (q_split < a.T) {
            const dim3 mgrid((a.T - q_split + kThreads / 64 - 1) / (kThreads / 64), a.nh);
            if (a.hd == 64)
                hipLaunchKernelGGL(k_attn_prefill_merge<64>, mgrid, dim3(kThreads), 0, s, b, q_split);
            else
                hipLaunchKernelGGL(k_attn_prefill_merge<128>, mgrid, dim3(kThreads), 0, s, b, q_split);
        }
        return hipGetLastError();
    }
    const size_t lds = sizeof(float) * (size_t(kQB) * (a.hd + 1) + size_t(kKT) * (a.hd + 1) +
                                        size_t(kKT) * a.hd + size_t(kQB) * kKT);
    dim3 grid((a.T + kQB - 1) / kQB, a.nh);
    hipLaunchKernelGGL(k_attn_prefill, grid, dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace q8l

// noalloc.hip -- the single-token attention entry point for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// q8l_op_attention takes its split-KV partial results in a caller workspace;
// this variant keeps them in a file-scope device array instead. Each device
// the library runs on holds its own copy of the array until the process ends.
// Host code never passes the array's name to a kernel (on the host that name
// is only a stand-in, not a device address): the device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and the
// looked-up pointer is what the kernels receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/q8l.h"
#include "q8l_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[Q8L_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
hipError_t scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

using namespace q8l;

extern "C" q8l_status q8l_op_attention_noalloc(const float *Q, const float *K, const float *V, int32_t T,
                                               int32_t kv_len, int32_t kv_stride, int32_t n_head,
                                               int32_t n_head_kv, int32_t hd, float *O, void *stream) {
    if (!Q || !K || !V || !O || T < 1 || kv_len < T || kv_stride < kv_len || n_head < 1 || n_head_kv < 1 ||
        n_head % n_head_kv || n_head / n_head_kv > kMaxGroup || hd % 8 || hd > 128 ||
        (reinterpret_cast<uintptr_t>(Q) & 15) || (reinterpret_cast<uintptr_t>(K) & 15) ||
        (reinterpret_cast<uintptr_t>(V) & 15))
        return Q8L_E_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (T == 1) {
        // the partials [n_head][splits][hd + 2] f32 must fit the array
        const int splits = (kv_len + attn_chunk(hd) - 1) / attn_chunk(hd);
        if (size_t(n_head) * splits * (hd + 2) * sizeof(float) > size_t(Q8L_NOALLOC_SCRATCH_BYTES))
            return Q8L_E_INVALID_ARG;
        void *part = nullptr;
        if ((e = scratch_on_current_device(&part)) != hipSuccess) return Q8L_E_HIP;
        AttnDecodeArgs a;
        a.q = Q; a.kc = K; a.vc = V;
        a.part = static_cast<float *>(part);
        a.st = nullptr; a.kv_len_arg = kv_len; a.kv_stride = kv_stride;
        a.nh = n_head; a.nkv = n_head_kv; a.hd = hd;
        a.n_splits = splits;
        a.scale = 1.0f / sqrtf(float(hd));
        a.o = nullptr;
        e = launch_attn_decode(a, s);
        if (e == hipSuccess) e = launch_attn_combine(a.part, a.n_splits, kv_len, n_head, hd, O, nullptr, s);
    } else {
        // several queries: the prefill kernel uses no scratch memory
        AttnPrefillArgs a;
        a.q = Q; a.kc = K; a.vc = V; a.o = O; a.o_split = nullptr; a.T = T; a.kv_len = kv_len;
        a.kv_stride = kv_stride; a.nh = n_head; a.nkv = n_head_kv; a.hd = hd; a.scale = 1.0f / sqrtf(float(hd));
        e = launch_attn_prefill(a, s);
    }
    return e == hipSuccess ? Q8L_OK : Q8L_E_HIP;
}

/*
 * q8l.h -- C ABI of the MI355X (gfx950) quantized Llama forward library.
 *
 * The library runs the forward pass of a Llama-shaped model whose projection
 * weights are Q8_0 blocks, as the page "量化 llama 的一次前向" (one forward of
 * quantized llama) traces it through candle's quantized_llama:
 *   token embedding -> per layer [RMSNorm -> q/k/v projections -> interleaved
 *   rope at index_pos -> KV-cache append -> grouped-query attention ->
 *   o-projection + residual -> RMSNorm -> gate/up projections, SiLU(gate)*up,
 *   down projection + residual] -> final RMSNorm -> last position ->
 *   output layer (the embedding when output.weight is absent).
 * Its calls follow the interface that page and "生成一个 token" (generating one
 * token) describe: build a model from named tensors (section "建模型：按名字取
 * 张量"), forward(tokens, index_pos) -> logits of the last position (section
 * "forward：mask 什么时候建"), and clear_kv_cache (section "换 prompt 要不要
 * clear_kv_cache").
 *
 * Conventions for every call:
 *   - Device pointers are HIP device memory on the current device. The
 *     library never frees memory it did not allocate; bound tensors and the
 *     workspace are BORROWED and must outlive the model.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls that take a stream enqueue work and return without waiting;
 *     results are valid after the stream is synchronized.
 *   - Errors are returned as q8l_status; q8l_last_error() gives a message.
 *     An error found by argument or state checks leaves the model unchanged
 *     and enqueues nothing. A HIP launch failure returns Q8L_E_HIP.
 *   - A model is not re-entrant: a forward mutates its KV cache. Two models
 *     may be used from different threads.
 *
 * Q8_0 layout: a row of K weights (K a multiple of 64 for this library) is
 * K/32 blocks of 34 bytes, each an IEEE binary16 scale d (little-endian)
 * followed by 32 signed 8-bit values q; weight = d * q. Matrices are
 * row-major [out, in] with blocks along `in`. The pages fix the block size
 * through the model file's byte count ("生成一个 token", sections 实验程序
 * and 读 GGUF); the field order is the GGUF convention.
 */
#ifndef Q8L_H
#define Q8L_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8L_OK = 0,
    Q8L_E_INVALID_ARG = 1,    /* bad pointer, size, count, token id, or index_pos < 0 */
    Q8L_E_MISSING_TENSOR = 2, /* finalize: a required tensor was never bound */
    Q8L_E_SHAPE = 3,          /* bind: rows/cols/nbytes do not match the config */
    Q8L_E_POS_RANGE = 4,      /* index_pos + T > max_seq_len (the rope table bound) */
    Q8L_E_POS_MISMATCH = 5,   /* T > 1 and index_pos != cached positions */
    Q8L_E_KV_FULL = 6,        /* cached positions + T > max_seq_len */
    Q8L_E_NOT_FINALIZED = 7,  /* forward before finalize, or bind after it */
    Q8L_E_HIP = 8,            /* a HIP call failed (message has the HIP error) */
    Q8L_E_FORMAT = 9,         /* GGUF: malformed or unsupported file content */
    Q8L_E_MISSING_KEY = 10,   /* GGUF: a required metadata key is absent */
    Q8L_E_IO = 11,            /* GGUF: the file cannot be opened or read */
    Q8L_E_RANGE = 12          /* an earlier prefill met a value outside its f16 pairs' range (see q8l_forward) */
} q8l_status;

/* Q4_K and Q6_K: the 256-weight block formats of the 4-bit "K" file mix
 * ("速度", section "CPU GGUF": 144 and 210 bytes per 256 weights by its
 * Q4_K_M tensor table; bit layouts as in the public GGUF block definitions).
 * Q4_K block: f16 d, f16 dmin, 12 bytes packing eight 6-bit scales s_j and
 * mins m_j, 128 bytes of 4-bit values q; weight = d*s_j*q - dmin*m_j per
 * 32-weight sub-block j. Q6_K block: 128 bytes of low 4 bits, 64 bytes of
 * high 2 bits, 16 int8 scales (one per 16 weights), f16 d;
 * weight = d*scale*(q - 32). */
typedef enum { Q8L_F32 = 0, Q8L_Q8_0 = 1, Q8L_Q4_K = 2, Q8L_Q6_K = 3, Q8L_Q5_0 = 4 } q8l_dtype;

/*
 * Model hyper-parameters: the llama.* metadata keys the page "生成一个 token"
 * (section 读 GGUF) prints, plus the rope table length (4096 in candle, page
 * "量化 llama 的一次前向", section "from_gguf：键名写死了 llama."), the norm eps
 * and the rope base. Requirements: n_head % n_head_kv == 0 with at most 16
 * query heads per KV head, head_dim a multiple of 8 and <= 128, n_embd, n_ff
 * and n_head*head_dim multiples of 64, max_seq_len >= 1.
 */
typedef struct q8l_config {
    int32_t n_layer;      /* llama.block_count */
    int32_t n_embd;       /* llama.embedding_length (H) */
    int32_t n_head;       /* llama.attention.head_count */
    int32_t n_head_kv;    /* llama.attention.head_count_kv */
    int32_t head_dim;     /* per-head width */
    int32_t n_ff;         /* llama.feed_forward_length */
    int32_t n_vocab;      /* rows of token_embd */
    int32_t max_seq_len;  /* rope table rows = KV cache slots (4096) */
    double rms_eps;       /* RMSNorm epsilon (1e-5) */
    double rope_theta;    /* rope base (10000) */
    int32_t tied_output;  /* 1: the output layer is token_embd */
    int32_t rope_type;    /* Q8L_ROPE_NORM: pairs (2j, 2j+1), llama's rope_i;
                             Q8L_ROPE_NEOX: pairs (j, j + head_dim/2) ("量化 llama 的一次
                             前向", section "RoPE：两种约定，按架构名选"); same angles */
} q8l_config;

#define Q8L_ROPE_NORM 0
#define Q8L_ROPE_NEOX 1

typedef struct q8l_model q8l_model;

/* Bytes of device workspace the model needs: KV cache
 * [n_layer][2][n_head_kv][max_seq_len][head_dim] f32, the rope table,
 * activations for up to max_seq_len tokens, attention partials (decode
 * splits; the key ranges of long prefills), split-K partial sums of the
 * prefill o and down projections, and counters.
 * Returns 0 for an invalid config. */
size_t q8l_workspace_bytes(const q8l_config *cfg);

/* Create a host-side model object; no HIP calls. Q8L_E_INVALID_ARG for a bad
 * config. The object is owned by the caller and freed with q8l_destroy. */
q8l_status q8l_create(const q8l_config *cfg, q8l_model **out);

/*
 * Bind one tensor by its GGUF name (page "生成一个 token", section 建模型):
 *   token_embd.weight              Q8_0 [n_vocab, n_embd]
 *   blk.{i}.attn_norm.weight       F32  [1, n_embd]
 *   blk.{i}.attn_q.weight          Q8_0 [n_head*head_dim, n_embd]
 *   blk.{i}.attn_k.weight          Q8_0 [n_head_kv*head_dim, n_embd]
 *   blk.{i}.attn_v.weight          Q8_0 [n_head_kv*head_dim, n_embd]
 *   blk.{i}.attn_output.weight     Q8_0 [n_embd, n_head*head_dim]
 *   blk.{i}.ffn_norm.weight        F32  [1, n_embd]
 *   blk.{i}.ffn_gate.weight        Q8_0 [n_ff, n_embd]
 *   blk.{i}.ffn_up.weight          Q8_0 [n_ff, n_embd]
 *   blk.{i}.ffn_down.weight        Q8_0 [n_embd, n_ff]
 *   output_norm.weight             F32  [1, n_embd]
 *   output.weight                  Q8_0 [n_vocab, n_embd]  (untied models only)
 * attn_output and ffn_down may instead be Q4_K or Q6_K when their cols are a
 * multiple of 256 (as files of the 4-bit mix store the down projection), and
 * every blk.{i} projection (attn_q, attn_k, attn_v, attn_output, ffn_gate,
 * ffn_up, ffn_down) may be Q5_0
 * (22-byte blocks: f16 d, a 32-bit little-endian word whose bit i is weight
 * i's fifth bit, 16 bytes whose low nibbles are weights 0..15 and high
 * nibbles 16..31; weight = d * ((nibble | bit << 4) - 16)) -- the 4-bit mix
 * stores most of the 135M model's projections so ("速度", section "CPU
 * GGUF"). Each matrix's format is taken from its binding; ffn_gate and
 * ffn_up of a layer must share one (Q8L_E_SHAPE from q8l_finalize otherwise).
 * `dev_ptr` holds the raw bytes (blocks exactly as in the file, rows back to
 * back; F32 little-endian), 16-byte aligned, borrowed. Q8L_E_SHAPE when the
 * dtype, rows, cols or nbytes (rows*cols/32*34 for Q8_0, rows*cols/32*22 for
 * Q5_0, rows*cols/256*144 for Q4_K, rows*cols/256*210 for Q6_K, rows*cols*4
 * for F32) do not match;
 * Q8L_E_INVALID_ARG for an unknown name, NULL or misaligned pointer;
 * Q8L_E_NOT_FINALIZED after finalize (weights are fixed once finalized).
 * Binding a name twice replaces the earlier pointer.
 */
q8l_status q8l_bind_tensor(q8l_model *m, const char *name, q8l_dtype dtype, int64_t rows,
                           int64_t cols, const void *dev_ptr, size_t nbytes);

/* Bind the device workspace (>= q8l_workspace_bytes, 256-byte aligned,
 * borrowed). Q8L_E_INVALID_ARG if too small, NULL or misaligned. */
q8l_status q8l_bind_workspace(q8l_model *m, void *dev_ptr, size_t nbytes);

/*
 * Check that every required tensor (9 per layer + token_embd + output_norm,
 * + output.weight when untied) and the workspace are bound -- else
 * Q8L_E_MISSING_TENSOR naming the first missing one -- then build the rope
 * table on the device, set the cached-position count to 0 and prepare the
 * decode graphs. Enqueued on `stream`.
 */
q8l_status q8l_finalize(q8l_model *m, void *stream);

/*
 * forward(tokens, index_pos): run T = n_tokens tokens starting at position
 * index_pos and write the logits of the LAST position to logits_dev
 * (f32[n_vocab], device) and, if argmax_dev is not NULL, the index of the
 * largest logit (lowest index on ties) to *argmax_dev (a uint32 the device
 * can address: device memory, or pinned host memory by its device address,
 * which the last kernel writes directly, so a per-token readback needs no
 * copy).
 * `tokens_host` is host memory (read before the call returns).
 * Checks, in this order, before anything is enqueued or changed:
 *   1. n_tokens >= 1, tokens < n_vocab, index_pos >= 0, logits_dev != NULL
 *                                                        else Q8L_E_INVALID_ARG
 *   2. index_pos + T <= max_seq_len                      else Q8L_E_POS_RANGE
 *   3. index_pos == 0 drops the cache (cached positions := 0), as candle does
 *   4. T > 1 requires index_pos == cached positions      else Q8L_E_POS_MISMATCH
 *      (candle fails these as a broadcast error; page "量化 llama 的一次前向",
 *      section "index_pos 传错"). T == 1 is NOT checked, as in candle: rope
 *      uses index_pos, the new key/value go to the next free slot and the
 *      single query attends to every cached position without a mask.
 *   5. cached positions + T <= max_seq_len               else Q8L_E_KV_FULL
 * Then enqueue the forward; cached positions += T.
 *
 * Prefill arithmetic (T >= 2 runs on the matrix cores): int8 weights exact in
 * f16, activations as f16 pairs hi + lo (22 bits), f32 accumulation. The
 * normalised rows are scaled per token by a power of two and the gate/up
 * output per token and 32-wide block (only when a value would reach 2^15),
 * both taken out exactly in f32, so those pairs keep 22 bits at any
 * magnitude. q, k, v, the attention output and the few f32 inputs that are
 * split on the way must stay below 2^15 in magnitude: when one does not, the
 * model's NEXT forward or generate call returns Q8L_E_RANGE once (that
 * prefill's logits are not exact) and does nothing else. q, k and v are
 * checked where a prefill writes them; cached keys and values that decode
 * steps wrote (single-token steps compute in f32 and check nothing) are
 * checked when a prefill that appends to the cache first reads them.
 */
q8l_status q8l_forward(q8l_model *m, const uint32_t *tokens_host, int32_t n_tokens,
                       int32_t index_pos, float *logits_dev, uint32_t *argmax_dev,
                       void *stream);

/*
 * Greedy generation on the device: starting from the token at *token_dev
 * (device uint32), run `n_steps` single-token forwards at positions
 * index_pos, index_pos+1, ..., each feeding its argmax to the next step
 * without a host round trip, and write the n_steps picked ids to ids_dev
 * (device uint32[n_steps]). logits_dev (optional, f32[n_vocab]) receives the
 * last step's logits. This is the caller's loop of single-token forwards and
 * argmax readbacks (page "生成一个 token", section 实验程序), with each step's
 * checks (as in q8l_forward with T == 1) done up front for all steps.
 */
q8l_status q8l_generate(q8l_model *m, const uint32_t *token_dev, int32_t index_pos,
                        int32_t n_steps, uint32_t *ids_dev, float *logits_dev, void *stream);

/* Drop the KV cache: cached positions := 0 (page "量化 llama 的一次前向",
 * section "换 prompt 要不要 clear_kv_cache"). No memory is freed or cleared. */
q8l_status q8l_clear_kv_cache(q8l_model *m);

/* Number of cached positions (-1 for NULL). */
int32_t q8l_cache_len(const q8l_model *m);

/* Message for the last error on this model ("" if none; static string for NULL). */
const char *q8l_last_error(const q8l_model *m);

/* Free the host object and the graphs it owns (not bound memory). */
void q8l_destroy(q8l_model *m);

/* ------------------------------------------------------------------------
 * Single-op entry points: the hot path's building blocks on caller buffers,
 * for tests and microbenchmarks. All pointers are device memory; all enqueue
 * on `stream`.
 * ------------------------------------------------------------------------ */

/*
 * Q8_0 matrix-vector / small matrix product (the decode projection; page
 * "生成一个 token", section "prefill 和 decode：同一个 forward，不同的路":
 * one input row uses the matrix-vector kernel):
 *   Y[t][n] = sum_k W[n][k] * U[t][k],  t < T, n < N,
 * with U = X (norm_w NULL) or U[t] = X[t] / sqrt(mean(X[t]^2) + eps) * norm_w
 * (RMSNorm fused in front). W is Q8_0 [N][K] (16-byte aligned), X f32 [T][K],
 * Y f32 [T][N]. When `accumulate` is 1, Y += the product (residual add).
 * K must be a multiple of 64; 1 <= T <= 2^20. With norm_w set, or T <= 16
 * (the multi-token matrix-vector kernel), the arithmetic is f32. Larger
 * T without norm_w runs the MFMA matrix-matrix kernel on X split into f16
 * pairs: the product is then within about 2^-22 relative per element only
 * while every |X| < 2^15 (this entry point does not scale X and reports no
 * range error; the model's forward scales its activations itself).
 */
q8l_status q8l_op_matmul_q8_0(const void *W, int64_t N, int64_t K, const float *X, int64_t T,
                              const float *norm_w, double eps, int32_t accumulate, float *Y,
                              void *stream);

/*
 * The same product for a Q5_0 matrix (22-byte blocks as described at
 * q8l_bind; the 4-bit mix of the 135M model stores its 576-wide projections
 * so, "速度", section "CPU GGUF"):
 *   Y[t][n] (+)= sum_k W[n][k] * X[t][k].
 * W: N rows of K/32 blocks back to back (16-byte aligned), X f32 [T][K]
 * (16-byte aligned), Y f32 [T][N]; accumulate 1 adds to Y. K must be a
 * multiple of 64; 1 <= T <= 2^20. T <= 16 runs the matrix-vector kernels in
 * f32; larger T the MFMA matrix-matrix kernel on X split into f16 pairs
 * (exact to about 2^-22 relative while every |X| < 2^15, as for
 * q8l_op_matmul_q8_0). Q8L_E_INVALID_ARG for a NULL or misaligned pointer,
 * sizes out of range, or a matrix or activation block of 2 GiB or more.
 */
q8l_status q8l_op_matmul_q5_0(const void *W, int64_t N, int64_t K, const float *X, int64_t T,
                              int32_t accumulate, float *Y, void *stream);

/*
 * The same product for a Q4_K or Q6_K matrix (dtype Q8L_Q4_K / Q8L_Q6_K; the
 * pages time it on the down projection's shape, [203, 1536] x [1536, 576] and
 * [1, 1536] x [1536, 576], "速度", section "CPU GGUF"):
 *   Y[t][n] (+)= sum_k W[n][k] * X[t][k].
 * W: N rows of K/256 blocks back to back (16-byte aligned), X f32 [T][K]
 * (16-byte aligned), Y f32 [T][N]; accumulate 1 adds to Y. K must be a
 * multiple of 256. T = 1 runs the matrix-vector kernel, T > 1 the MFMA
 * matrix-matrix kernel on X split into f16 pairs (as for q8l_op_matmul_q8_0,
 * exact to about 2^-22 relative while every |X| < 2^15). Q8L_E_INVALID_ARG for a NULL or misaligned pointer,
 * another dtype, sizes out of range, or a matrix or activation block of 2 GiB
 * or more.
 */
q8l_status q8l_op_matmul_kq(const void *W, int32_t dtype, int64_t N, int64_t K, const float *X, int64_t T,
                            int32_t accumulate, float *Y, void *stream);

/*
 * Attention of T queries over kv_len cached keys with grouped heads:
 *   Q f32 [T][n_head][hd]; K, V f32 [n_head_kv][kv_stride][hd] (slot j of
 *   group g at (g*kv_stride + j)*hd); O f32 [T][n_head][hd].
 * Query head h reads KV group h / (n_head/n_head_kv). Scores are
 * q.k / sqrt(hd); when T > 1, query t sees keys j <= kv_len - T + t (the
 * causal mask offset by the cached prefix); when T == 1 it sees all kv_len.
 * Q, K and V must be 16-byte aligned (Q8L_E_INVALID_ARG otherwise).
 */
q8l_status q8l_op_attention(const float *Q, const float *K, const float *V, int32_t T,
                            int32_t kv_len, int32_t kv_stride, int32_t n_head,
                            int32_t n_head_kv, int32_t hd, float *O, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Bytes of workspace q8l_op_attention needs for these sizes. */
size_t q8l_op_attention_workspace(int32_t T, int32_t kv_len, int32_t n_head, int32_t n_head_kv,
                                  int32_t hd);

/* Size of the device array q8l_op_attention_noalloc keeps its partial results
 * in (per device): 4 MiB holds the single-query split partials
 * [n_head][ceil(kv_len / C)][head_dim + 2] f32 (C = 64 keys for head_dim <= 64,
 * else 32), e.g. 32 heads of 128 over 4096 keys = 2.1 MB. */
#define Q8L_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * q8l_op_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments (minus the workspace),
 * layouts and results -- bitwise, the same kernels -- as q8l_op_attention.
 * The single-query case (T == 1) keeps its split partials in a static device
 * array of Q8L_NOALLOC_SCRATCH_BYTES that each device holds until the process
 * ends; the call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine). T > 1 uses no scratch memory.
 * Errors: Q8L_E_INVALID_ARG as for q8l_op_attention, and when T == 1 and the
 * partials would exceed Q8L_NOALLOC_SCRATCH_BYTES; Q8L_E_HIP if the array's
 * device address cannot be looked up or a launch fails.
 * Every call on one device shares that device's array and leaves its
 * contents behind (each call writes every partial it reads): calls that
 * overlap in time on one device (two streams, or two host threads) race on
 * it, so the caller must serialise them.
 */
q8l_status q8l_op_attention_noalloc(const float *Q, const float *K, const float *V, int32_t T,
                                    int32_t kv_len, int32_t kv_stride, int32_t n_head,
                                    int32_t n_head_kv, int32_t hd, float *O, void *stream);

/* Largest element of x (f32[n], device), lowest index on ties, to *out.
 * workspace_bytes >= 8 * ceil(n / 4096). */
q8l_status q8l_op_argmax(const float *x, int64_t n, uint32_t *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Measurement: launch each kernel of one decode step on its own, once
 * untimed and then `reps` times back to back between two HIP events on
 * `stream`, and write the mean time per launch in milliseconds to
 * ms_out[kind] (ms_out holds 9 floats), kinds
 *   0 embedding (-1: the step has no embedding kernel, the first q/k/v
 *   kernel dequantizes the token's row; the slot's launches warm the GPU up
 *   for the kinds after it), 1 q/k/v (+norm, rope, KV write;
 *   as layers after the first run it), 2 attention (split
 *   partials, or the normalised output when the cache fits one split; when
 *   the step fuses the one-split attention with the o-projection, that
 *   fused kernel), 3 o-projection (+residual; as in the step at this length:
 *   with 2..8 splits and few partial bytes it merges them in its prologue,
 *   with more the merge is a kernel of its own, not timed here; -1 when it
 *   is part of kind 2), 4 gate/up (+norm, SiLU*up; after the fused kernel
 *   it first adds that kernel's per-group partial sums to the residual),
 *   5 down (+residual), 6 output layer (+norm, per-workgroup
 *   argmax), 7 argmax merge, 8 an empty kernel (the dispatch gap between
 *   back-to-back launches, included in every other entry).
 * The r-th launch of a per-layer kind (1 to 5) uses layer r mod n_layer's
 * weights and cache, so the weights come from beyond the L2 as they do in a
 * step, where each layer's weights are read once; attention runs over
 * cache_len + 1 keys. The residual stream, the next KV slot of every layer
 * and the logits buffer are scratch afterwards: the next forward rewrites
 * them before use.
 * The cache length is unchanged. Blocks until the timings are read back.
 * Q8L_E_INVALID_ARG if reps < 1 or the cache is full.
 */
q8l_status q8l_time_decode_kernels(q8l_model *m, int32_t reps, float *ms_out, void *stream);

/* Version string of the library build. */
const char *q8l_version(void);

/* ---------------------------------------------------------------- GGUF model files
 *
 * Reading a model file: the step before the forward. "生成一个 token", section
 * "读 GGUF：130 ms，只读头部": the header, metadata key/values and tensor
 * directory are read and the start of the tensor data is recorded, no weight
 * is read; section "建模型：按名字取张量": each tensor is found by name and its
 * raw bytes are read from the data region (Q8_0 bytes stay as they are, so
 * binding them is a copy). The byte format is the public GGUF specification
 * (versions 2 and 3, little-endian, data aligned to general.alignment, 32 by
 * default). Host-only calls: no device memory is touched. A handle holds the
 * open file; it is not thread-safe. Errors: Q8L_E_IO (open/read), Q8L_E_FORMAT
 * (bad magic, unsupported version, truncated or inconsistent directory,
 * tensor types other than F32 and Q8_0 when read), Q8L_E_MISSING_KEY.
 */
typedef struct q8l_gguf q8l_gguf;

/* Parse the header, metadata and tensor directory of `path`. On failure *out
 * is NULL and q8l_gguf_open_error() describes the problem (per thread). */
q8l_status q8l_gguf_open(const char *path, q8l_gguf **out);
const char *q8l_gguf_open_error(void);
const char *q8l_gguf_last_error(const q8l_gguf *g);
void q8l_gguf_close(q8l_gguf *g);

/* Directory facts ("读 GGUF" prints: file size, data start, key and tensor counts). */
uint32_t q8l_gguf_version(const q8l_gguf *g);
int64_t q8l_gguf_n_kv(const q8l_gguf *g);
int64_t q8l_gguf_n_tensors(const q8l_gguf *g);
uint64_t q8l_gguf_data_offset(const q8l_gguf *g);   /* absolute file offset */
uint64_t q8l_gguf_file_size(const q8l_gguf *g);

/* A numeric metadata value (any integer or float type, as double), or a
 * string value copied NUL-terminated into buf (Q8L_E_INVALID_ARG if it does not
 * fit). Q8L_E_MISSING_KEY if the key is absent or of another kind. */
q8l_status q8l_gguf_get_number(const q8l_gguf *g, const char *key, double *out);
q8l_status q8l_gguf_get_string(const q8l_gguf *g, const char *key, char *buf, size_t buf_bytes);

/* Model config from the llama.* keys ("量化 llama 的一次前向", section "from_gguf：
 * 键名写死了 llama."): block_count, embedding_length, attention.head_count,
 * attention.head_count_kv, feed_forward_length, rope.dimension_count (must
 * equal embedding_length / head_count), attention.layer_norm_rms_epsilon
 * (all required: Q8L_E_MISSING_KEY, message "cannot find <key> in metadata"),
 * rope.freq_base (optional, 10000). n_vocab = rows of token_embd.weight;
 * tied_output = 1 when output.weight is absent (section "建模型"); rope_type
 * from general.architecture (section "RoPE：两种约定，按架构名选": qwen, qwen2,
 * falcon, phi3, stablelm and gptneox pair j with j + hd/2, every other
 * architecture 2j with 2j+1). max_seq_len is the caller's (4096 in candle). */
q8l_status q8l_gguf_config(q8l_gguf *g, int32_t max_seq_len, q8l_config *cfg);

/* Index of the tensor called `name`, or -1. */
int64_t q8l_gguf_find_tensor(const q8l_gguf *g, const char *name);
/* Tensor `index`: name (valid while the handle is open), dtype (a q8l_dtype, or
 * -1 with Q8L_E_FORMAT for other types), rows x cols (cols = the innermost
 * dimension), absolute file offset and byte size as read. Any output may be
 * NULL. Q5_0 tensors of the seven blk.{i} projections with rows of at least
 * 2048 weights are read as they are (dtype Q8L_Q5_0, 22 bytes per 32
 * weights). Q4_0 tensors, Q5_0 tensors of shorter rows (whose single-token
 * products are faster in Q8_0) and Q5_0 tensors of the other roles
 * (token_embd, output) are read as Q8_0
 * (32-weight blocks of an f16 scale times 4- or 5-bit integers; sizes pinned
 * by "速度", section "CPU GGUF"): dtype Q8L_Q8_0, size rows*cols/32*34, each
 * block converted exactly (same scale, int8 = the block's integer). Q4_K and
 * Q6_K tensors are read as they are (dtype Q8L_Q4_K / Q8L_Q6_K). Other block
 * formats are listed but not read (dtype -1). */
q8l_status q8l_gguf_tensor_info(const q8l_gguf *g, int64_t index, const char **name, int32_t *dtype,
                                int64_t *rows, int64_t *cols, uint64_t *offset, uint64_t *nbytes);
/* Read tensor `index`'s bytes into host memory; nbytes must equal its size as read. */
q8l_status q8l_gguf_read_tensor(q8l_gguf *g, int64_t index, void *host_dst, size_t nbytes);
/* The tensor's type id in the file (the GGUF numbering: 0 F32, 2 Q4_0, 6 Q5_0, 8 Q8_0, 12 Q4_K,
 * 14 Q6_K, ...), or -1. */
int32_t q8l_gguf_tensor_file_type(const q8l_gguf *g, int64_t index);

#ifdef __cplusplus
}
#endif

#endif /* Q8L_H */

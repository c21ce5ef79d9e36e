/*
 * gqa.h -- C ABI of libgqa.so: fused grouped-query scaled-dot-product
 * attention on one AMD Instinct MI355X (gfx950).
 *
 * Every entry point computes, for each request b, query head h and query
 * row i,
 *
 *   out[b,h,i,:] = sum_{j in J} softmax_j(scale * <q[b,h,i,:], k[b,g,j,:]>) v[b,g,j,:]
 *
 * where g = h / (Hq/Hkv) (query heads come in contiguous groups that share
 * one KV head) and J is the set of visible keys defined per entry point.
 * K and V are read unexpanded, straight from a preallocated cache, and no
 * score matrix is ever written to memory.
 *
 * Sources (web pages; section names as printed there):
 *  - "2x faster Qwen2 decode on Metal in Candle", sections "Why Qwen2 Was
 *    Running at Half Speed" and "Why It Matters: 7x KV Expansion": the fused
 *    single-token kernel attends over the original KV heads through a GQA
 *    stride instead of materialising one K/V copy per query head.
 *  - "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x
 *    faster...", section "Cause and workaround", points 1-3: K/V are passed
 *    before repeat_kv, with Hq divisible by Hkv; with
 *    more than one query the causal mask is applied in-kernel with the
 *    queries aligned to the end of the keys; the single-query kernel reads K
 *    and V through the head stride and needs each head's rows to be
 *    contiguous.  Same page, end of "Cause and workaround": a device the
 *    kernel does not support gets an explicit error, not a fallback.
 *  - VeloxQuant-MLX "attention" posts, Result 4 and Part 4: the decode
 *    kernel's grid carries a request (B) axis; the quantized path takes the
 *    queries, the cache's codes, scales and biases, the group size and the
 *    scale, and dequantizes inside the kernel.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named q, k, v, out, kv_lens, codes, scales, biases and
 *    workspace are DEVICE pointers owned by the caller.  The library keeps no
 *    reference after the call returns and allocates no memory.
 *  - Tensors are dense and row-major in the stated shapes; every pointer must
 *    be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    and the call returns without synchronising.  `out` is fully overwritten
 *    when the work runs.
 *  - Every argument check runs on the host before anything is enqueued, so a
 *    call that returns an error has enqueued nothing.  Errors are status codes;
 *    nothing aborts or throws across the ABI.
 *  - `scale` is the float multiplier of the dot products (normally
 *    1/sqrt(D)); it must be finite.
 *  - Accumulation is fp32 for every storage dtype.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_NULL = 1,        /* a required pointer is NULL */
    GQA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
    GQA_ERR_UNSUPPORTED = 3, /* dtype, head dim or device not supported */
    GQA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    GQA_ERR_HIP = 5,         /* the HIP runtime reported an error */
    GQA_ERR_ALIGN = 6        /* a pointer is not 16-byte aligned */
} gqa_status_t;

typedef enum gqa_dtype {
    GQA_F32 = 0,
    GQA_BF16 = 1,
    GQA_F16 = 2
} gqa_dtype_t;

/* Version of this ABI (bumped on any incompatible change). */
int gqa_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char *gqa_status_string(int status);

/*
 * Workspaces.  A workspace must be zero-filled before its first use.  It
 * begins with a region of 16 MiB that holds the decode (max, sum) pairs and
 * the prefill arrival counters; the other partial results follow it.  Every
 * call leaves, once its work has completed, the 16 MiB region zero-filled
 * and every 32-bit word after it with its lowest bit clear: decode
 * publishes its partial results with that bit set in every word (which is
 * how they are recognised) and the workgroup that consumes them zeroes them;
 * prefill writes its partial results with that bit clear and returns its
 * counters to zero.  One workspace may therefore serve any sequence of
 * decode and prefill calls of any sizes, as long as it is large enough for
 * each call and their work does not overlap in time.
 *
 * Bytes of device workspace the decode entry points need for these sizes:
 * the 16 MiB region plus one fp32 partial output per (request, query head,
 * split).  Returns 0 when the sizes are invalid, which includes (max, sum)
 * pairs that would not fit the region (8 bytes per request, query head and
 * split; at most 64 splits).  The value depends only on the arguments.
 */
size_t gqa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int s_cap);

/*
 * Prepare a workspace for its first use: zero-fills `bytes` bytes at
 * `workspace` with a kernel on `stream`.  Every entry point leaves the
 * workspace ready for the next call (see above), so this is needed once per
 * allocation (a zero-filled allocation needs no call).  Two calls whose work
 * may overlap in time must not share a workspace.
 */
int gqa_workspace_init(void *workspace, size_t bytes, void *stream);

/*
 * Single-token decode over a preallocated KV cache, every request with the
 * same length.
 *
 *   q, out  [B, Hq, 1, D]        dtype
 *   k, v    [B, Hkv, s_cap, D]   dtype, rows 0..kv_len-1 valid (others never read)
 *   visible keys J = { j : j < kv_len }   (no mask: one query token)
 *
 * Requires B >= 1, Hkv >= 1, Hq % Hkv == 0, D in {64, 128},
 * 1 <= kv_len <= s_cap, dtype in {GQA_F32, GQA_BF16, GQA_F16},
 * workspace_bytes >= gqa_decode_workspace_bytes(B, Hq, Hkv, D, s_cap) and a
 * workspace prepared as described at gqa_workspace_init.
 * The split of the KV length depends only on (s_cap, Hq, Hkv), so the output
 * for request b is bit-identical to gqa_decode_attend_batched with
 * kv_lens[b] = kv_len and the same s_cap.
 */
int gqa_decode_attend(const void *q, const void *k, const void *v, void *out,
                      int B, int Hq, int Hkv, int D, int kv_len, int s_cap,
                      float scale, int dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Batched decode: as gqa_decode_attend, but request b attends over its own
 * first kv_lens[b] cache rows.  kv_lens is a DEVICE array of B int32 values;
 * the host cannot check it, so the kernel clamps each value to [0, s_cap].
 * A request with length 0 gets an all-zero output row.
 */
int gqa_decode_attend_batched(const void *q, const void *k, const void *v, void *out,
                              const int32_t *kv_lens,
                              int B, int Hq, int Hkv, int D, int s_cap,
                              float scale, int dtype,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace gqa_prefill_causal needs for these sizes: the
 * 16 MiB region (one u32 arrival counter per request, query head and 128-row
 * block that is split into key chunks) plus the fp32 partial results of
 * those chunks; when no row block is split, the region alone.  Returns
 * 0 when the sizes are invalid.  The value depends only on the arguments.
 * Like the decode workspace it must start zero-filled (torch.zeros, or
 * gqa_workspace_init once per allocation).
 */
size_t gqa_prefill_workspace_bytes(int B, int Hq, int Hkv, int D, int Tq, int Tk);

/*
 * Causal prefill with the queries aligned to the end of the keys.
 *
 *   q, out  [B, Hq, Tq, D]       dtype
 *   k, v    [B, Hkv, s_cap, D]   dtype, rows 0..Tk-1 valid (others never read)
 *   visible keys for query row i: J_i = { j : j <= i + (Tk - Tq) }
 *
 * so a chunk of Tq queries at offset Tk - Tq sees every earlier key.
 * Requires B >= 1, Hkv >= 1, Hq % Hkv == 0, D in {64, 128},
 * 1 <= Tq <= Tk <= s_cap, Tq <= 131072, dtype in {GQA_BF16, GQA_F16} (products on the
 * matrix cores, fp32 accumulation; probabilities are rounded to the input
 * dtype before the second product), and a caller-owned, 16-byte aligned
 * workspace of at least gqa_prefill_workspace_bytes(B, Hq, Hkv, D, Tq, Tk)
 * bytes (GQA_ERR_WORKSPACE otherwise).  Two calls whose work may overlap in
 * time must not share a workspace.  The result does not depend on timing:
 * the key chunks of a row block are merged in chunk order.
 */
int gqa_prefill_causal(const void *q, const void *k, const void *v, void *out,
                       int B, int Hq, int Hkv, int D, int Tq, int Tk, int s_cap,
                       float scale, int dtype,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode over a 4-bit group-affine quantized KV cache.
 *
 *   q, out                 [B, Hq, 1, D]                 f16
 *   k_codes, v_codes       [B, Hkv, s_cap, D/2]          uint8; element 2j of
 *                          a row is the low nibble of byte j, element 2j+1 the
 *                          high nibble
 *   k_scales, k_biases,
 *   v_scales, v_biases     [B, Hkv, s_cap, D/group_size] f16
 *
 * Element e of a row with code c has the value s*c + b (s, b of group
 * e / group_size), rounded once to float32, exactly as gqa_dequant_q4
 * returns it; attention then proceeds as in gqa_decode_attend.
 * Requires D in {64, 128}, group_size in {32, 64, 128} dividing D,
 * 1 <= kv_len <= s_cap, and a workspace as for gqa_decode_attend (same size
 * function).
 */
int gqa_decode_attend_q4(const void *q,
                         const uint8_t *k_codes, const void *k_scales, const void *k_biases,
                         const uint8_t *v_codes, const void *v_scales, const void *v_biases,
                         void *out, int B, int Hq, int Hkv, int D, int group_size,
                         int kv_len, int s_cap, float scale,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dequantize n_rows cache rows to float32 with the device routine that
 * gqa_decode_attend_q4 applies to every element (a check hook: its output
 * can be compared bit for bit with the definition above).
 *
 *   codes [n_rows, D/2] uint8, scales/biases [n_rows, D/group_size] f16,
 *   out [n_rows, D] float32.
 *
 * Requires D in {64, 128}, group_size in {32, 64, 128} dividing D and
 * n_rows >= 0 (0 enqueues nothing).
 */
int gqa_dequant_q4(const uint8_t *codes, const void *scales, const void *biases, float *out,
                   int n_rows, int D, int group_size, void *stream);

/*
 * Measurement helper, not part of the attention path: reads `bytes` bytes at
 * `src` once with coalesced 16-byte loads (the plain streaming read that
 * bounds any HBM-bound kernel), so that a benchmark can time the achievable
 * read rate exactly as it times the decode kernels.  Stores nothing in
 * practice: one 32-bit word at `sink` (device memory) is written only if the
 * data fold to one fixed value.  Requires bytes > 0 and a multiple of 16,
 * src and sink 16-byte aligned.
 */
int gqa_read_probe(const void *src, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */

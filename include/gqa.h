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
 * Each entry point below cites the web page passage that defines it (page
 * title and section as printed there).  The pages:
 *  - "2x faster Qwen2 decode on Metal in Candle" (the Candle decode page);
 *  - "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x
 *    faster and lowers its peak from 3,403 MiB to 1,470 MiB" (the Fornace
 *    prefill page);
 *  - the VeloxQuant-MLX blog posts tagged "attention": "Batching Decode
 *    Attention Across Requests Got Us 3.83x Real Throughput..." and
 *    "Batching Decode Attention Across Layers Sounded Great -- Until the
 *    Residual Stream Said No" (the VeloxQuant posts).
 * A device other than gfx950 gets GQA_ERR_UNSUPPORTED rather than a
 * fallback, as the Fornace page's engine refuses to load its fused path
 * where the kernel does not exist ("Cause and workaround", last paragraph).
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
    GQA_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
    GQA_ERR_SCRATCH = 7      /* sizes exceed the allocation-free entry point's scratch */
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
 * Decode merges never depend on every workgroup of a launch being resident
 * at once: a workgroup waits for others only after all of them have
 * started, so calls on other streams, other processes or a CU mask cannot
 * stall one.  The waits are bounded all the same; should one ever give up
 * (the protocol makes that unreachable), that merge writes NaN and marks
 * the workspace poisoned (a word in the last 64 bytes of the 16 MiB
 * region), and every later decode merge on it writes NaN too, rather than
 * reading what the abandoned call left behind, until the workspace is
 * zero-filled again (gqa_workspace_init).
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
 * Defined by the Candle decode page, "Why It Matters: 7x KV Expansion on
 * Every Decode Step" (the fused kernel attends over the original KV heads
 * through a GQA stride instead of a copy per query head), and the Fornace
 * prefill page, "Cause and workaround", points 1 and 3 (K/V given before
 * repeat_kv; the one-token kernel reads each KV head's rows contiguously
 * through the head stride).
 *
 *   q, out  [B, Hq, 1, D]        dtype
 *   k, v    [B, Hkv, s_cap, D]   dtype, rows 0..kv_len-1 valid (others never read)
 *   visible keys J = { j : j < kv_len }   (no mask: one query token)
 *
 * Requires B >= 1, Hkv >= 1, Hq % Hkv == 0, D in {64, 128},
 * 1 <= kv_len <= s_cap, dtype in {GQA_F32, GQA_BF16, GQA_F16},
 * workspace_bytes >= gqa_decode_workspace_bytes(B, Hq, Hkv, D, s_cap) and a
 * workspace prepared as described at gqa_workspace_init.
 * The split of the KV length depends only on (s_cap, Hq, Hkv, D), so the output
 * for request b is bit-identical to gqa_decode_attend_batched with
 * kv_lens[b] = kv_len and the same s_cap.
 */
int gqa_decode_attend(const void *q, const void *k, const void *v, void *out,
                      int B, int Hq, int Hkv, int D, int kv_len, int s_cap,
                      float scale, int dtype,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_decode_attend without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It allocates nothing and calls
 * no allocating routine: its partial results live in a scratch array of
 * 8 MiB built into the library (one per GPU, held until the process ends):
 * 512 KiB for the (max, sum) and control words (which must fit 512 KiB less
 * 64 bytes) and 7.5 MiB for the fp32 partial outputs (B * Hq * splits * D * 4
 * bytes; e.g. the 28/4-head, D = 128 geometry up to B = 8 at s_cap = 4096).
 * Larger sizes return GQA_ERR_SCRATCH.  Same kernels and split plan as
 * gqa_decode_attend, so the output is bit-identical to it.  The first call
 * on a device also zero-fills the array with a kernel on `stream` (make that
 * first call outside any graph capture).  Every call on one GPU shares that
 * GPU's array: calls that may overlap in time on one GPU race and must not
 * be issued (serialize them on one stream); each call leaves the array
 * ready for the next.
 */
int gqa_decode_attend_noalloc(const void *q, const void *k, const void *v, void *out,
                              int B, int Hq, int Hkv, int D, int kv_len, int s_cap,
                              float scale, int dtype, void *stream);

/*
 * Batched decode: as gqa_decode_attend, but request b attends over its own
 * first kv_lens[b] cache rows.  Defined by the VeloxQuant posts ("Part 4:
 * the other half of the lever actually works": the decode kernel's grid
 * carries a request axis, B x H_kv x S_q threadgroups; "Where this leaves
 * things": variable-length concurrent requests).  kv_lens is a DEVICE array of B int32 values;
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
 * 0 when the sizes are invalid.  The value depends on the arguments and on
 * the compute-unit count of the current HIP device (the chunking sizes the
 * launch to the device; 256 when no device can be queried), so size the
 * workspace with the device current that the call will run on.  It is not
 * monotone in Tq and Tk (a shorter prompt may be cut into more key chunks):
 * a workspace shared by calls of several sizes takes the largest of their
 * values.
 * Like the decode workspace it must start zero-filled (torch.zeros, or
 * gqa_workspace_init once per allocation).
 */
size_t gqa_prefill_workspace_bytes(int B, int Hq, int Hkv, int D, int Tq, int Tk);

/*
 * Causal prefill with the queries aligned to the end of the keys.
 *
 * Defined by the Fornace prefill page, "Cause and workaround": one kernel
 * reads the grouped KV heads directly (point 1), applies the causal mask
 * inside the kernel with the queries aligned to the end of the keys so that
 * a chunk at an offset sees every earlier key (point 2), and never stores
 * the [Hq, T, T] score matrix ("Why it matters").
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
 * Decode and causal prefill with a sliding window and attention sinks.  The
 * pages' fused kernels leave both out -- the Fornace prefill page, "What
 * this does not prove": no sliding window is applied (Qwen2.5's window never
 * masks a position, other models can differ); the VeloxQuant posts, "Part
 * 4": the SDPA call the fused decode path intercepts carries `sinks` -- and
 * models that use them need them in the same fused pass:
 *
 *   window > 0   only the `window` most recent keys up to a query's own
 *                position are visible: key j is visible to row i iff
 *                last - window < j <= last, last = i + (Tk - Tq) for
 *                prefill and kv_lens[b] - 1 for decode (0: no window);
 *   sinks        NULL, or a DEVICE float array [Hq]: one logit per query
 *                head, in the units of scale * <q, k>, that joins the
 *                softmax normaliser and carries no value:
 *                out = sum_j e^{s_j} v_j / (e^{sinks[h]} + sum_j e^{s_j}).
 *
 * gqa_decode_attend_ex is gqa_decode_attend_batched with these options (its
 * split plan covers min(window, s_cap) rows, so a call's workspace is at
 * most gqa_decode_workspace_bytes(B, Hq, Hkv, D, s_cap)); with window = 0
 * and sinks = NULL its output is bit-identical to the batched entry point.
 * gqa_prefill_causal_ex is gqa_prefill_causal with these options and needs
 * gqa_prefill_workspace_bytes_ex(..., window) bytes of workspace.  Errors,
 * layouts and workspaces as for the entry points they extend;
 * GQA_ERR_SHAPE for window < 0.
 */
int gqa_decode_attend_ex(const void *q, const void *k, const void *v, void *out,
                         const int32_t *kv_lens, int B, int Hq, int Hkv, int D, int s_cap,
                         float scale, int dtype, int window, const float *sinks,
                         void *workspace, size_t workspace_bytes, void *stream);
size_t gqa_prefill_workspace_bytes_ex(int B, int Hq, int Hkv, int D, int Tq, int Tk, int window);
int gqa_prefill_causal_ex(const void *q, const void *k, const void *v, void *out,
                          int B, int Hq, int Hkv, int D, int Tq, int Tk, int s_cap,
                          float scale, int dtype, int window, const float *sinks,
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
 * Defined by the VeloxQuant posts ("Part 4": the fused decode call takes
 * the queries, the cache's codes, scales and biases, the group size and the
 * scale, and dequantizes inside the kernel; "The setup": the fused
 * group-affine decode+attention kernel behind the KIVI-style cache).
 *
 * Element e of a row with code c has the value s*c + b (s, b of group
 * e / group_size); the result is attention over those values, as in
 * gqa_decode_attend.  The kernel does not form s*c + b per element: per
 * group it uses
 *     q . k         = s * sum_e q_e c_e + b * sum_e q_e
 *     sum_r p_r v_r = sum_r (p_r s_r) c_r + sum_r p_r b_r
 * with the code products on the matrix cores (fp32 sums), and it rounds two
 * kinds of intermediate values to f16: the query elements that face a high
 * nibble (divided by 16; exact unless |q| < 2^-10) and each probability
 * times its row's scale, p_r s_r (and p_r s_r / 16 for high nibbles).  With
 * one visible key (kv_len = 1) the output is that key's dequantized value
 * row, s*c + b rounded once to float32 (as gqa_dequant_q4 returns it), then
 * rounded to f16: bit for bit.
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
 * Append new tokens' K and V rows to a preallocated dense cache (the step
 * before each decode call).  The Fornace prefill page runs decode over a
 * preallocated KV cache ("What was measured and how"; "What it means if you
 * run models on your own hardware": use the fused kernel with a preallocated
 * cache), into which each new token's rows are written in place.
 *
 *   k_new, v_new      [B, Hkv, T_new, D]   dtype
 *   k_cache, v_cache  [B, Hkv, s_cap, D]   dtype
 *   kv_lens           [B] int32 (DEVICE): rows already in request b's cache
 *   new_lens          [B] int32 (DEVICE) or NULL: receives
 *                     min(p_b + T_new, s_cap)
 *
 * Request b's new row t goes to cache row p_b + t, p_b = kv_lens[b] clamped
 * to [0, s_cap]; rows that would land at or past s_cap are dropped.  Nothing
 * else in the caches changes; the copy is exact.  new_lens must not be
 * kv_lens (every workgroup reads the old lengths).  Requires D in {64, 128},
 * dtype in {GQA_F32, GQA_BF16, GQA_F16}, T_new >= 1, 16-byte aligned
 * pointers.
 */
int gqa_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                  const int32_t *kv_lens, int32_t *new_lens,
                  int B, int Hkv, int D, int T_new, int s_cap, int dtype, void *stream);

/*
 * Append new tokens' K and V rows to a 4-bit cache, quantizing only the new
 * rows (the VeloxQuant posts, "Part 4": re-quantizing the whole K/V history
 * every decode step cost ~25 ms/step against a ~12 ms/step kernel; the fix
 * quantizes only the newly aged rows).  Layouts as in gqa_decode_attend_q4;
 * k_new, v_new [B, Hkv, T_new, D] in `dtype` (GQA_F32, GQA_BF16 or GQA_F16);
 * kv_lens, new_lens and the placement of rows as in gqa_kv_append.
 *
 * Each group of group_size elements of a new row is encoded with the
 * min-max group-affine map, in float32 on the exactly widened inputs:
 *   scale = f16((max - min) / 15), bias = f16(min)   (round to nearest even;
 *           a zero minimum or step is stored as +0)
 *   code  = clamp(rint((x - bias) / scale), 0, 15)   (ties to even; 0 when
 *           the scale is 0)
 * Inputs must be finite, with the minimum and (max - min) / 15 within the
 * f16 range.  Requires D in {64, 128}, group_size in {32, 64, 128} dividing
 * D, T_new >= 1, 16-byte aligned pointers.
 */
int gqa_kv_append_q4(const void *k_new, const void *v_new, int dtype,
                     uint8_t *k_codes, void *k_scales, void *k_biases,
                     uint8_t *v_codes, void *v_scales, void *v_biases,
                     const int32_t *kv_lens, int32_t *new_lens,
                     int B, int Hkv, int D, int group_size, int T_new, int s_cap, void *stream);

/*
 * 4-bit cache with a float16 residual window.
 *
 * The VeloxQuant posts ("What this means in practice", and the caveats
 * after the real-model results) point out that a production KIVI cache
 * keeps the most recent tokens in float16 and only older ones quantized,
 * which their test cache did not.  Reading taken here (block flush): with
 * residual capacity R, a request of n tokens holds positions [0, n_q),
 * n_q = R * floor(n / R), in the 4-bit arrays (layouts as in
 * gqa_decode_attend_q4, s_cap rows per KV head) and positions [n_q, n) as
 * exact float16 rows at slots 0 .. n - n_q - 1 of
 *
 *   k_res, v_res   [B, Hkv, R, D]   f16
 *
 * kv_lens [B] int32 (DEVICE) holds n per request (clamped to [0, s_cap]).
 * R must be a positive multiple of 64.
 */

/* Workspace bytes for gqa_decode_attend_q4r (0 if the sizes are invalid). */
size_t gqa_decode_q4r_workspace_bytes(int B, int Hq, int Hkv, int D, int s_cap, int R);

/*
 * Decode over a residual-window 4-bit cache: attention of q [B, Hq, 1, D]
 * f16 over every token of each request, the 4-bit rows dequantized as in
 * gqa_decode_attend_q4 and the residual rows as they are; out [B, Hq, 1, D]
 * f16.  One launch: the 4-bit rows are split as in gqa_decode_attend_q4,
 * and the residual rows of each (request, head tile) are one more split,
 * streamed as float16 rows by the dense decode path and merged with the
 * others.  A request with no tokens gets zeros.  Requires D in {64, 128},
 * group_size in {32, 64, 128} dividing D, and a zero-initialised workspace
 * of gqa_decode_q4r_workspace_bytes (calls leave it as they found it, so it
 * is reused without clearing).
 */
int gqa_decode_attend_q4r(const void *q,
                          const uint8_t *k_codes, const void *k_scales, const void *k_biases,
                          const uint8_t *v_codes, const void *v_scales, const void *v_biases,
                          const void *k_res, const void *v_res, void *out, const int32_t *kv_lens,
                          int B, int Hq, int Hkv, int D, int group_size, int R, int s_cap, float scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Append new float16 rows k_new, v_new [B, Hkv, T_new, D] to a
 * residual-window 4-bit cache (the VeloxQuant posts' "Part 4": encode only
 * rows that age, never the whole history).  Request b's rows take
 * positions n .. n + T_new - 1 (n = kv_lens[b] clamped to [0, s_cap]; rows
 * at or past s_cap are dropped) and new_lens[b] (DEVICE, or NULL) receives
 * n' = min(n + T_new, s_cap).  Positions [n_q(n), n_q(n')) are encoded
 * into the 4-bit arrays with the quantizer of gqa_kv_append_q4 (from the
 * residual, or straight from the new rows that age at once) and positions
 * [max(n, n_q(n')), n') are copied to their residual slots; other rows and
 * slots are left unchanged.  Several workgroups per (request, KV head)
 * share the encoding; when the copies would overwrite residual slots that
 * the encoding reads (a flush that keeps new rows, old residual not empty),
 * one workgroup encodes and then copies, so the update is exact whatever
 * T_new is.  new_lens
 * must not be kv_lens.  Requires D in {64, 128}, group_size in
 * {32, 64, 128} dividing D, R a positive multiple of 64, T_new >= 1,
 * finite inputs, 16-byte aligned pointers.
 */
int gqa_kv_append_q4r(const void *k_new, const void *v_new,
                      uint8_t *k_codes, void *k_scales, void *k_biases,
                      uint8_t *v_codes, void *v_scales, void *v_biases,
                      void *k_res, void *v_res,
                      const int32_t *kv_lens, int32_t *new_lens,
                      int B, int Hkv, int D, int group_size, int R, int T_new, int s_cap, void *stream);

/*
 * Causal prefill of a chunk over a residual-window 4-bit cache (the
 * VeloxQuant posts' caveats above, with the chunked prefill of the Fornace
 * page's "Cause and workaround": a chunk of Tq queries at the end of Tk
 * tokens sees every earlier token).  Every request holds Tk tokens (the
 * chunk's own rows already appended, e.g. by gqa_kv_append_q4r), so
 * positions [0, n_q), n_q = R * floor(Tk / R), are read from the 4-bit
 * arrays and [n_q, Tk) from the residual.  Query row i attends to
 * positions j <= i + Tk - Tq.
 *
 *   q, out   [B, Hq, Tq, D]  f16
 *
 * The kernel is gqa_prefill_causal's with the 4-bit tiles dequantized on
 * the way into LDS: each value s*c + b is formed in float32 (one rounding,
 * as gqa_dequant_q4) and rounded to f16, the type the matrix cores read.
 * Workspace: gqa_prefill_workspace_bytes(B, Hq, Hkv, D, Tq, Tk).  Requires
 * D in {64, 128}, group_size in {32, 64, 128} dividing D, R a positive
 * multiple of 64, 1 <= Tq <= Tk <= s_cap.
 */
int gqa_prefill_causal_q4r(const void *q,
                           const uint8_t *k_codes, const void *k_scales, const void *k_biases,
                           const uint8_t *v_codes, const void *v_scales, const void *v_biases,
                           const void *k_res, const void *v_res, void *out,
                           int B, int Hq, int Hkv, int D, int group_size, int R, int Tq, int Tk, int s_cap,
                           float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dequantize n_rows cache rows to float32: s*c + b per element, rounded once
 * (a check hook for the encoding the 4-bit entry points share; its output
 * can be compared bit for bit with that definition).  The attention kernel
 * does not call it: it applies scales and biases around the code products
 * (see gqa_decode_attend_q4).
 *
 *   codes [n_rows, D/2] uint8, scales/biases [n_rows, D/group_size] f16,
 *   out [n_rows, D] float32.
 *
 * Requires D in {64, 128}, group_size in {32, 64, 128} dividing D and
 * n_rows >= 0 (0 enqueues nothing).
 */
int gqa_dequant_q4(const uint8_t *codes, const void *scales, const void *biases, float *out,
                   int n_rows, int D, int group_size, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */

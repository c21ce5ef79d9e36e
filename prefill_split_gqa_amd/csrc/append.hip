// append.hip -- writing new tokens' K/V rows into a preallocated cache.
//
// The step that runs before every decode call.  The Fornace prefill page
// ("What was measured and how", "What it means if you run models on your own
// hardware") runs decode over a preallocated KV cache, whose rows the new
// tokens are written into in place; the VeloxQuant-MLX "attention" posts
// ("Part 4") found that re-quantizing the whole growing K/V history every
// decode step cost ~25 ms/step against a ~12 ms/step attention kernel, and
// fixed it by quantizing only the newly aged rows.  Here both are kernels:
//
//  * dense append: request b's T_new new rows go to cache rows
//    p_b .. p_b + T_new - 1, p_b = kv_lens[b] clamped to [0, s_cap]; rows that
//    would land at or past s_cap are dropped; new_lens[b] = min(p_b + T_new,
//    s_cap) when asked for.  A plain copy: 16 bytes per lane, coalesced.
//  * 4-bit append: the same rows, each encoded on the way in with the
//    min-max group-affine quantizer (per group of `group` elements along D:
//    scale = f16((max - min) / 15), bias = f16(min), code = clamp(rint((x -
//    bias) / scale), 0, 15), float32 arithmetic, ties to even; code 0 where
//    the scale is 0; a zero minimum or step is stored as +0).  Only the new
//    rows are touched.
//
//  * 4-bit append with a float16 residual window: a request of n tokens
//    holds positions [0, n_q) 4-bit, n_q = R * floor(n / R), and positions
//    [n_q, n) as exact float16 rows in a residual buffer of R rows (slot p -
//    n_q).  New float16 rows join the residual; when it fills, its rows and
//    any new rows that age at once are encoded as one block (the VeloxQuant
//    posts, "What this means in practice": a production KIVI cache keeps the
//    recent tokens in float16).  Several workgroups per (request, KV head)
//    share the encoding; a slot that is both read (aged) and rewritten (new)
//    in one append is handled by a single workgroup, read before a barrier
//    and written after it.
//
// All are bound by HBM (a few hundred KB per call at the workloads' sizes);
// one lane handles 8 consecutive elements of a row (one 16-byte load of
// 16-bit inputs, two of fp32), the lanes of one group reduce its minimum and
// maximum with butterfly shuffles, and each lane writes its 8 codes as one
// 32-bit word.  Device lengths are read by every lane that needs them; the
// host cannot check them, so they are clamped.

#include <algorithm>

#include "common.h"

namespace gqa {

namespace {

__device__ __forceinline__ int clamp_len(int n, int s_cap) { return n < 0 ? 0 : (n > s_cap ? s_cap : n); }

// ---------------------------------------------------------------------------
// Dense append
// ---------------------------------------------------------------------------
__global__ void kv_append_kernel(const uint4 *__restrict__ k_new, const uint4 *__restrict__ v_new,
                                 uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache,
                                 const int32_t *__restrict__ kv_lens, int32_t *__restrict__ new_lens, int Hkv,
                                 int T_new, int s_cap, int vec_per_row, long n_vec)
{
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += (long)gridDim.x * blockDim.x) {
        const int c = (int)(i % vec_per_row);
        const long row = i / vec_per_row;  // (b, h, t)
        const int t = (int)(row % T_new);
        const long bh = row / T_new;
        const int b = (int)(bh / Hkv);
        const int p = clamp_len(kv_lens[b], s_cap);
        if (new_lens && c == 0 && t == 0 && bh % Hkv == 0) new_lens[b] = min(p + T_new, s_cap);
        if (p + t >= s_cap) continue;
        const long dst = (bh * s_cap + p + t) * vec_per_row + c;
        k_cache[dst] = k_new[i];
        v_cache[dst] = v_new[i];
    }
}

// ---------------------------------------------------------------------------
// 4-bit append
// ---------------------------------------------------------------------------
template <typename T> struct Load8;
template <> struct Load8<f16_t> {
    __device__ __forceinline__ static void run(const void *row, int lane8, float *x)
    {
        const uint4 w = ((const uint4 *)row)[lane8];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = f16_bits_to_f32(ws[i] & 0xFFFFu);
            x[2 * i + 1] = f16_bits_to_f32(ws[i] >> 16);
        }
    }
};
template <> struct Load8<bf16_t> {
    __device__ __forceinline__ static void run(const void *row, int lane8, float *x)
    {
        const uint4 w = ((const uint4 *)row)[lane8];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_bits_to_f32(ws[i] & 0xFFFFu);
            x[2 * i + 1] = bf16_bits_to_f32(ws[i] >> 16);
        }
    }
};
template <> struct Load8<float> {
    __device__ __forceinline__ static void run(const void *row, int lane8, float *x)
    {
        const float4 a = ((const float4 *)row)[2 * lane8];
        const float4 b = ((const float4 *)row)[2 * lane8 + 1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x)
{
    const _Float16 h = (_Float16)x;  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Min-max encoding of the 8 elements x of one lane; the LPG lanes of a
// group (aligned, a power of two) reduce its minimum and maximum together,
// so every lane of a group must take part.  Returns the lane's 8 codes as
// one word (element i: nibble i) and the group's f16 scale and bias.
template <int LPG>
__device__ __forceinline__ uint32_t q4_encode8(const float (&x)[8], uint16_t &sh, uint16_t &bh16)
{
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        lo = fminf(lo, x[i]);
        hi = fmaxf(hi, x[i]);
    }
#pragma unroll
    for (int m = 1; m < LPG; m <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, m, 64));
        hi = fmaxf(hi, __shfl_xor(hi, m, 64));
    }
    lo = lo == 0.0f ? 0.0f : lo;  // a zero minimum or step is stored as +0
    float step = (hi - lo) / 15.0f;
    step = step == 0.0f ? 0.0f : step;
    sh = f32_to_f16_bits(step);
    bh16 = f32_to_f16_bits(lo);
    const float s = f16_bits_to_f32(sh);
    const float bias = f16_bits_to_f32(bh16);
    uint32_t word = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t c = 0u;
        if (s != 0.0f) {
            const float k = __builtin_rintf((x[i] - bias) / s);
            c = k < 0.0f ? 0u : (k > 15.0f ? 15u : (uint32_t)k);
        }
        word |= c << (4 * i);  // element 8*lane8 + i: nibble i (low nibble = even element)
    }
    return word;
}

// One row of D elements per D/8 lanes; LPG = group/8 lanes per group (a
// power of two, aligned within the wave), whose minimum and maximum are
// reduced with xor shuffles.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void kv_append_q4_kernel(const void *__restrict__ k_new, const void *__restrict__ v_new,
                                                           uint8_t *__restrict__ k_codes, uint16_t *__restrict__ k_scales,
                                                           uint16_t *__restrict__ k_biases, uint8_t *__restrict__ v_codes,
                                                           uint16_t *__restrict__ v_scales, uint16_t *__restrict__ v_biases,
                                                           const int32_t *__restrict__ kv_lens,
                                                           int32_t *__restrict__ new_lens, int Hkv, int T_new,
                                                           int s_cap, long n_rows)
{
    constexpr int LPR = D / 8;   // lanes per row
    constexpr int LPG = G / 8;   // lanes per group
    constexpr int NG = D / G;    // groups per row
    static_assert(LPR <= 64 && (64 % LPR) == 0 && (LPG & (LPG - 1)) == 0 && LPG <= LPR, "lane layout");
    const long gl = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long row = gl / LPR;     // (b, h, t) of the new rows
    const int lane8 = (int)(gl % LPR);
    const bool live = row < n_rows;
    const long r = live ? row : n_rows - 1;  // lanes past the last row shadow it (their writes are dropped)
    const int t = (int)(r % T_new);
    const long bh = r / T_new;
    const int b = (int)(bh / Hkv);
    const int p = clamp_len(kv_lens[b], s_cap);
    if (live && new_lens && lane8 == 0 && t == 0 && bh % Hkv == 0) new_lens[b] = min(p + T_new, s_cap);
    const bool store = live && p + t < s_cap;
    const long dst = bh * s_cap + p + t;  // cache row
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const void *src = (const char *)(which ? v_new : k_new) + r * (long)D * sizeof(T);
        float x[8];
        Load8<T>::run(src, lane8, x);
        uint16_t sh, bh16;
        const uint32_t word = q4_encode8<LPG>(x, sh, bh16);
        if (store) {
            uint8_t *codes = which ? v_codes : k_codes;
            ((uint32_t *)(codes + dst * (D / 2)))[lane8] = word;
            if ((lane8 % LPG) == 0) {
                const int g = lane8 / LPG;
                (which ? v_scales : k_scales)[dst * NG + g] = sh;
                (which ? v_biases : k_biases)[dst * NG + g] = bh16;
            }
        }
    }
}

// Residual-window append: workgroups (request b, KV head, j), j < NB.  With
// n the request's tokens before and n2 after the append, positions
// [n_q(n), n_q(n2)) are encoded (from residual slot p - n_q(n) while p < n,
// else from new row p - n), then positions [max(n, n_q(n2)), n2) are copied
// to residual slot p - n_q(n2).  The copies overwrite slots the encoding
// reads only when a flush keeps new rows in the residual and the old
// residual was not empty (an append of several rows); then workgroup j = 0
// does both in order, with a barrier between, and the others stop.
// Otherwise the NB workgroups share the encoding row by row and j = 0 also
// copies.  Rows are spread over a workgroup's lanes, D/8 lanes per row; a
// lane past the last row of a pass shadows the row before it and stores
// nothing.
template <int D, int G>
__global__ __launch_bounds__(256) void kv_append_q4r_kernel(const f16_t *__restrict__ k_new, const f16_t *__restrict__ v_new,
                                                            uint8_t *__restrict__ k_codes, uint16_t *__restrict__ k_scales,
                                                            uint16_t *__restrict__ k_biases, uint8_t *__restrict__ v_codes,
                                                            uint16_t *__restrict__ v_scales, uint16_t *__restrict__ v_biases,
                                                            uint4 *__restrict__ k_res, uint4 *__restrict__ v_res,
                                                            const int32_t *__restrict__ kv_lens,
                                                            int32_t *__restrict__ new_lens, int Hkv, int T_new,
                                                            int s_cap, int R)
{
    constexpr int LPR = D / 8;   // lanes per row
    constexpr int LPG = G / 8;   // lanes per group
    constexpr int NG = D / G;    // groups per row
    constexpr int RPP = 256 / LPR;  // rows per pass
    static_assert(LPR <= 64 && (64 % LPR) == 0 && (LPG & (LPG - 1)) == 0 && LPG <= LPR, "lane layout");
    const int bh = (int)blockIdx.x;
    const int j = (int)blockIdx.y, nb = (int)gridDim.y;
    const int b = bh / Hkv;
    const int n = clamp_len(kv_lens[b], s_cap);
    const int n2 = min(n + T_new, s_cap);
    const int nq_old = n - n % R, nq_new = n2 - n2 % R;
    const bool ordered = nq_new > nq_old && n > nq_old && n2 > nq_new;
    if (ordered && j != 0) return;
    const int step = ordered ? 1 : nb;  // passes of this workgroup: j, j + step, ...
    if (new_lens && j == 0 && threadIdx.x == 0 && bh % Hkv == 0) new_lens[b] = n2;
    const int lane8 = (int)threadIdx.x % LPR;
    const int rsub = (int)threadIdx.x / LPR;
    const size_t res0 = (size_t)bh * R;        // residual row of slot 0
    const size_t new0 = (size_t)bh * T_new;    // new row 0
    const size_t cache0 = (size_t)bh * s_cap;  // cache row of position 0

    // aged rows -> 4-bit
    for (int p0 = nq_old + j * RPP; p0 < nq_new; p0 += step * RPP) {
        const bool live = p0 + rsub < nq_new;
        const int p = live ? p0 + rsub : nq_new - 1;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const f16_t *src = p < n ? (const f16_t *)(which ? v_res : k_res) + (res0 + (p - nq_old)) * D
                                     : (which ? v_new : k_new) + (new0 + (p - n)) * D;
            float x[8];
            Load8<f16_t>::run(src, lane8, x);
            uint16_t sh, bh16;
            const uint32_t word = q4_encode8<LPG>(x, sh, bh16);
            if (live) {
                const size_t dst = cache0 + p;
                ((uint32_t *)((which ? v_codes : k_codes) + dst * (D / 2)))[lane8] = word;
                if ((lane8 % LPG) == 0) {
                    (which ? v_scales : k_scales)[dst * NG + lane8 / LPG] = sh;
                    (which ? v_biases : k_biases)[dst * NG + lane8 / LPG] = bh16;
                }
            }
        }
    }
    if (j != 0) return;
    __syncthreads();  // (ordered) every aged residual slot has been read

    // new rows that stay float16 -> residual
    const int keep0 = max(n, nq_new);
    for (int p0 = keep0; p0 < n2; p0 += RPP) {
        const int p = p0 + rsub;
        if (p < n2) {
            const size_t src = (new0 + (p - n)) * LPR + lane8;  // 16-byte units
            const size_t dst = (res0 + (p - nq_new)) * LPR + lane8;
            k_res[dst] = ((const uint4 *)k_new)[src];
            v_res[dst] = ((const uint4 *)v_new)[src];
        }
    }
}

template <typename T, int D>
hipError_t launch_q4_append_d(const void *kn, const void *vn, uint8_t *kc, void *ks, void *kb, uint8_t *vc, void *vs,
                              void *vb, const int32_t *lens, int32_t *new_lens, int B, int Hkv, int group, int T_new,
                              int s_cap, hipStream_t st)
{
    const long n_rows = (long)B * Hkv * T_new;
    const long lanes = n_rows * (D / 8);
    const unsigned blocks = (unsigned)((lanes + 255) / 256);
#define GQA_Q4A(G)                                                                                                  \
    hipLaunchKernelGGL((kv_append_q4_kernel<T, D, G>), dim3(blocks), dim3(256), 0, st, kn, vn, kc, (uint16_t *)ks, \
                       (uint16_t *)kb, vc, (uint16_t *)vs, (uint16_t *)vb, lens, new_lens, Hkv, T_new, s_cap, n_rows)
    if (group == 32) GQA_Q4A(32);
    else if (group == 64) GQA_Q4A(64);
    else if constexpr (D == 128) {
        if (group == 128) GQA_Q4A(128);
        else return hipErrorInvalidValue;
    } else return hipErrorInvalidValue;
#undef GQA_Q4A
    return hipGetLastError();
}

template <typename T>
hipError_t launch_q4_append_t(int D, const void *kn, const void *vn, uint8_t *kc, void *ks, void *kb, uint8_t *vc,
                              void *vs, void *vb, const int32_t *lens, int32_t *new_lens, int B, int Hkv, int group,
                              int T_new, int s_cap, hipStream_t st)
{
    if (D == 64) return launch_q4_append_d<T, 64>(kn, vn, kc, ks, kb, vc, vs, vb, lens, new_lens, B, Hkv, group, T_new, s_cap, st);
    if (D == 128) return launch_q4_append_d<T, 128>(kn, vn, kc, ks, kb, vc, vs, vb, lens, new_lens, B, Hkv, group, T_new, s_cap, st);
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_q4r_append_d(const void *kn, const void *vn, uint8_t *kc, void *ks, void *kb, uint8_t *vc, void *vs,
                               void *vb, void *kr, void *vr, const int32_t *lens, int32_t *new_lens, int B, int Hkv,
                               int group, int R, int T_new, int s_cap, hipStream_t st)
{
    // workgroups per (request, KV head): enough passes for the most rows one
    // append can encode (a full residual plus the new rows), at most 64
    const long rows = (long)R + T_new;
    const unsigned nb = (unsigned)std::min<long>(64, (rows + 256 / (D / 8) - 1) / (256 / (D / 8)));
#define GQA_Q4R(G)                                                                                                 \
    hipLaunchKernelGGL((kv_append_q4r_kernel<D, G>), dim3(B * Hkv, nb), dim3(256), 0, st, (const f16_t *)kn,      \
                       (const f16_t *)vn, kc, (uint16_t *)ks, (uint16_t *)kb, vc, (uint16_t *)vs, (uint16_t *)vb, \
                       (uint4 *)kr, (uint4 *)vr, lens, new_lens, Hkv, T_new, s_cap, R)
    if (group == 32) GQA_Q4R(32);
    else if (group == 64) GQA_Q4R(64);
    else if constexpr (D == 128) {
        if (group == 128) GQA_Q4R(128);
        else return hipErrorInvalidValue;
    } else return hipErrorInvalidValue;
#undef GQA_Q4R
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append_q4r(const void *k_new, const void *v_new, uint8_t *k_codes, void *k_scales,
                                void *k_biases, uint8_t *v_codes, void *v_scales, void *v_biases, void *k_res,
                                void *v_res, const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D,
                                int group, int R, int T_new, int s_cap, hipStream_t s)
{
    if (D == 64)
        return launch_q4r_append_d<64>(k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, k_res,
                                       v_res, kv_lens, new_lens, B, Hkv, group, R, T_new, s_cap, s);
    if (D == 128)
        return launch_q4r_append_d<128>(k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, k_res,
                                        v_res, kv_lens, new_lens, B, Hkv, group, R, T_new, s_cap, s);
    return hipErrorInvalidValue;
}

hipError_t launch_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                            const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D, int T_new, int s_cap,
                            int elem_bytes, hipStream_t s)
{
    const int vec_per_row = D * elem_bytes / 16;
    const long n_vec = (long)B * Hkv * T_new * vec_per_row;
    long blocks = (n_vec + 255) / 256;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint4 *)k_new,
                       (const uint4 *)v_new, (uint4 *)k_cache, (uint4 *)v_cache, kv_lens, new_lens, Hkv, T_new, s_cap,
                       vec_per_row, n_vec);
    return hipGetLastError();
}

hipError_t launch_kv_append_q4(int dtype, const void *k_new, const void *v_new, uint8_t *k_codes, void *k_scales,
                               void *k_biases, uint8_t *v_codes, void *v_scales, void *v_biases,
                               const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D, int group, int T_new,
                               int s_cap, hipStream_t s)
{
    if (dtype == 0)
        return launch_q4_append_t<float>(D, k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases,
                                         kv_lens, new_lens, B, Hkv, group, T_new, s_cap, s);
    if (dtype == 1)
        return launch_q4_append_t<bf16_t>(D, k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases,
                                          kv_lens, new_lens, B, Hkv, group, T_new, s_cap, s);
    if (dtype == 2)
        return launch_q4_append_t<f16_t>(D, k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases,
                                         kv_lens, new_lens, B, Hkv, group, T_new, s_cap, s);
    return hipErrorInvalidValue;
}

}  // namespace gqa

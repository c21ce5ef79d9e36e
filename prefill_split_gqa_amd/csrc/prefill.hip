// prefill.hip -- causal grouped-query prefill on the gfx950 matrix cores.
//
// "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x faster",
// section "Cause and workaround": one pass reads the grouped KV heads
// directly, applies the causal mask inside the kernel with the queries
// aligned to the end of the keys (row i sees keys j <= i + Tk - Tq), and never
// stores the score matrix.
//
// Work decomposition: a workgroup of 4 waves owns 128 query rows of one query
// head (32 rows per wave) and walks the visible keys in tiles of 64.  Each K
// tile is staged row-major in LDS and each V tile transposed (V^T, keys
// contiguous), double-buffered, with the next tile's global loads in flight
// while the current tile is computed.
//
// Per tile and wave, on v_mfma_f32_32x32x16 (bf16 or f16 inputs, fp32 sums):
//   S^T[key][row] = K Q^T          (A = K rows from LDS, B = Q rows in registers)
//   online softmax per row in fp32 (exp2 with scale*log2(e) folded in; the
//   reference max is only raised when a score exceeds it by more than 2^8)
//   O^T[d][row] += V^T P^T         (A = V^T from LDS, B = P in registers)
// Computing S transposed makes its accumulator layout (a lane holds keys of
// one row) exactly the layout the second product wants for P, so P never
// leaves registers.  Only tiles that cross the diagonal are masked.
// Workgroups are issued longest-row-block first to shorten the causal tail.

#include <type_traits>

#include "common.h"

namespace gqa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Per-dtype matrix-core product, fp32 -> 16-bit pair conversion (one
// v_cvt_pk per pair) and the sum of a packed pair (v_dot2 against 1.0).
template <typename T> struct MfmaOps;
template <> struct MfmaOps<bf16_t> {
    typedef bf16x8_t vec;
    __device__ __forceinline__ static f32x16_t mfma(vec a, vec b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi)
    {
        const f32x2_t x = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
    }
    __device__ __forceinline__ static float sum2(uint32_t w, float acc)
    {
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
    }
};
template <> struct MfmaOps<f16_t> {
    typedef f16x8_t vec;
    __device__ __forceinline__ static f32x16_t mfma(vec a, vec b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi)
    {
        const f32x2_t x = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
    }
    __device__ __forceinline__ static float sum2(uint32_t w, float acc)
    {
        const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), one, acc, false);
    }
};

template <typename V> __device__ __forceinline__ V as_vec(uint4 x) { return __builtin_bit_cast(V, x); }

// Position of key kk (0..63 within a tile) in a V^T row in LDS.  Each
// 16-key block is stored as keys [0-3, 8-11, 4-7, 12-15]: the eight keys
// that lane group lg of the second product pairs with its P values (keys
// 4lg..4lg+3 and 8+4lg..8+4lg+3 of the block, the order in which the score
// accumulator holds them) then sit in eight consecutive elements.
__device__ __forceinline__ int vt_pos(int kk)
{
    const int w = kk & 15, a = w >> 2;
    return (kk & ~15) + 8 * (a & 1) + 4 * (a >> 1) + (w & 3);
}

constexpr int kPfBM = 128;   // query rows per workgroup
constexpr int kPfBN = 64;    // keys per tile
constexpr int kPfThreads = 256;
constexpr int kPfKPad = 8;   // 16-bit elements of padding per K row in LDS
constexpr int kPfVPad = 8;   // per V^T row

// Online softmax of one 64-key tile for the wave's 32 rows.
//
// st holds S^T (raw q.k) in the accumulator layout: lane (ln, lg) has, for
// sub-tile u and register j, key key0 + 32u + 8(j/4) + (j%4) of row ln,
// where key0 already includes the 4*lg lane offset.  With sigma the sign of
// the scale, the running maximum m_run is kept over the oriented raw scores
// sigma*s, so that one fused multiply-add per score gives the log2-domain
// exponent: exp2(s*qs - |qs|*m_run).  m_run is raised only when a tile's
// maximum exceeds it by more than thr (2^8 in the exponent), and the running
// output and sum are rescaled then.  The probabilities are rounded to the
// 16-bit input type in pairs (the B operand of the second product) and the
// row sum adds exactly the rounded values.
template <typename Ops, bool NEG, bool MASK, int NDB>
__device__ __forceinline__ void softmax_tile(f32x16_t (&st)[2], uint32_t (&pw)[2][8], f32x16_t (&acc)[NDB],
                                             float &m_run, float &l_part, float qs, float thr, int key0, int my_lim)
{
    constexpr float kInf = __builtin_huge_valf();
    float tmax = -kInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float e = NEG ? -st[u][j] : st[u][j];
            if (MASK && key0 + 32 * u + 8 * (j >> 2) + (j & 3) > my_lim) e = -kInf;
            tmax = fmaxf(tmax, e);
        }
    {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));  // both halves of the row
    }
    if (__any(tmax > m_run + thr)) {
        const float mn = fmaxf(m_run, tmax);
        const float al = m_run == -kInf ? 0.0f : fast_exp2(fabsf(qs) * (m_run - mn));
        m_run = mn;
        l_part *= al;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[db][j] *= al;
    }
    const float mq = -fabsf(qs) * m_run;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            float p0 = fast_exp2(__builtin_fmaf(st[u][j], qs, mq));
            float p1 = fast_exp2(__builtin_fmaf(st[u][j + 1], qs, mq));
            if (MASK) {
                const int kk = key0 + 32 * u + 8 * (j >> 2) + (j & 3);
                if (kk > my_lim) p0 = 0.0f;
                if (kk + 1 > my_lim) p1 = 0.0f;
            }
            const uint32_t w = Ops::pack2(p0, p1);
            pw[u][j / 2] = w;
            l_part = Ops::sum2(w, l_part);
        }
}

template <typename T, int D, bool NEG>
__global__ __launch_bounds__(kPfThreads) void prefill_causal_kernel(const uint16_t *__restrict__ q,
                                                                    const uint16_t *__restrict__ k,
                                                                    const uint16_t *__restrict__ v,
                                                                    uint16_t *__restrict__ out, int Hq, int Hkv,
                                                                    int Tq, int Tk, int s_cap, float qscale,
                                                                    int n_rb)
{
    typedef MfmaOps<T> Ops;
    typedef typename Ops::vec vec;
    constexpr int KS = D + kPfKPad;      // K row stride in LDS (elements)
    constexpr int VS = kPfBN + kPfVPad;  // V^T row stride in LDS (elements)
    constexpr int NKB = D / 16;          // k-blocks of the QK^T product
    constexpr int NDB = D / 32;          // 32-wide d-blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kPfBN * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VS];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ln = lane & 31, lg = lane >> 5;

    // longest row blocks first, every head's before the next length
    const int bx = blockIdx.x;
    const int h = bx % Hq;
    const int rb = n_rb - 1 - bx / Hq;
    const int b = blockIdx.y;
    const int G = Hq / Hkv;
    const int g = h / G;
    const int off = Tk - Tq;
    const int r0 = rb * kPfBM;
    const int rw0 = r0 + wave * 32;                 // first row of this wave
    const int row_hi = min(r0 + kPfBM, Tq);         // one past the last valid row of the block
    const int kend = min(Tk, row_hi + off);         // keys any valid row of the block can see
    const int n_tiles = (kend + kPfBN - 1) / kPfBN;

    const uint16_t *qh = q + ((size_t)b * Hq + h) * (size_t)Tq * D;
    const uint16_t *kh = k + ((size_t)b * Hkv + g) * (size_t)s_cap * D;
    const uint16_t *vh = v + ((size_t)b * Hkv + g) * (size_t)s_cap * D;
    // rows at or past Tq (queries) and Tk (keys) read as zeros
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, (size_t)Tq * D * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, (size_t)Tk * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh, (size_t)Tk * D * 2);

    // Q rows of this wave as MFMA B operands: lane (row ln, group lg) holds
    // dims [16*kb + 8*lg, +8) of its row.
    vec qreg[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
        qreg[kb] = as_vec<vec>(__builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, ((rw0 + ln) * D + kb * 16 + lg * 8) * 2, 0, 0)));

    // global -> register staging of one K/V tile
    constexpr int K_ITEMS = kPfBN * D / 8;          // 16-byte pieces per K tile
    constexpr int K_PER_T = K_ITEMS / kPfThreads;
    constexpr int V_ITEMS = (kPfBN / 2) * (D / 8);  // (key pair, 8-dim chunk)
    constexpr int V_PER_T = V_ITEMS / kPfThreads;
    static_assert(K_ITEMS % kPfThreads == 0 && V_ITEMS % kPfThreads == 0, "tile/thread mismatch");
    uint4 kreg[K_PER_T], vreg[V_PER_T][2];

    auto load_tile = [&](int kt) {
        const int k0 = kt * kPfBN;
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int idx = tid + i * kPfThreads;
            const int key = k0 + idx / (D / 8), c8 = idx % (D / 8);
            kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (key * D + c8 * 8) * 2, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = tid + i * kPfThreads;
            const int kp = idx % (kPfBN / 2), c8 = idx / (kPfBN / 2);
            const int key = k0 + 2 * kp;
            vreg[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (key * D + c8 * 8) * 2, 0, 0));
            vreg[i][1] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, ((key + 1) * D + c8 * 8) * 2, 0, 0));
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int idx = tid + i * kPfThreads;
            const int key = idx / (D / 8), c8 = idx % (D / 8);
            *(uint4 *)(&Ks[buf][key * KS + c8 * 8]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = tid + i * kPfThreads;
            const int kp = idx % (kPfBN / 2), c8 = idx / (kPfBN / 2);
            const int pos = vt_pos(2 * kp);
            const uint32_t *a = (const uint32_t *)&vreg[i][0];
            const uint32_t *c = (const uint32_t *)&vreg[i][1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // dims 8*c8 + 2w (low halves) and 8*c8 + 2w + 1 (high halves)
                const uint32_t lo = (a[w] & 0xFFFFu) | (c[w] << 16);
                const uint32_t hi = (a[w] >> 16) | (c[w] & 0xFFFF0000u);
                *(uint32_t *)(&Vt[buf][(c8 * 8 + 2 * w) * VS + pos]) = lo;
                *(uint32_t *)(&Vt[buf][(c8 * 8 + 2 * w + 1) * VS + pos]) = hi;
            }
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] = 0.0f;
    float m_run = -__builtin_huge_valf();  // running max of the oriented raw scores of this lane's row
    float l_part = 0.0f;
    const float aq = fabsf(qscale);
    const float thr = aq > 0.0f ? fminf(8.0f / aq, 3.0e38f) : 3.0e38f;  // lazy-rescale threshold, raw units
    const int my_row = rw0 + ln;
    const int my_lim = my_row + off;  // last visible key of this lane's row

    // One tile of the wave's rows.  All LDS fragments a product needs are
    // read before its first matrix instruction, and the V^T fragments before
    // the softmax, so that LDS latency hides behind the products and the
    // exponentials instead of stalling each instruction.
    auto compute_tile = [&](int buf, int k0, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        f32x16_t st[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) st[u][j] = 0.0f;
        // ---- S^T = K Q^T for two 32-key sub-tiles ----
        if constexpr (D == 64) {
            uint4 kf[2][NKB];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    kf[u][kb] = *(const uint4 *)(&Ks[buf][(u * 32 + ln) * KS + kb * 16 + lg * 8]);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) st[u] = Ops::mfma(as_vec<vec>(kf[u][kb]), qreg[kb], st[u]);
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                uint4 kf[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    kf[kb] = *(const uint4 *)(&Ks[buf][(u * 32 + ln) * KS + kb * 16 + lg * 8]);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) st[u] = Ops::mfma(as_vec<vec>(kf[kb]), qreg[kb], st[u]);
            }
        }
        // ---- V^T fragments (keys stored in MFMA operand order: one 16-byte read each) ----
        constexpr int VF = D == 64 ? 4 : 1;  // 16-key blocks fetched ahead of the softmax
        uint4 vf[4][NDB];
#pragma unroll
        for (int t = 0; t < VF; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                vf[t][db] = *(const uint4 *)(&Vt[buf][(db * 32 + ln) * VS + 16 * t + 8 * lg]);
        asm volatile("" ::: "memory");
        // ---- online softmax ----
        uint32_t pw[2][8];
        softmax_tile<Ops, NEG, MASK>(st, pw, acc, m_run, l_part, qscale, thr, k0 + 4 * lg, my_lim);
        // ---- O^T += V^T P^T, four 16-key k-blocks ----
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int u = t >> 1, hh = t & 1;
            const uint4 pb = make_uint4(pw[u][hh * 4 + 0], pw[u][hh * 4 + 1], pw[u][hh * 4 + 2], pw[u][hh * 4 + 3]);
            if (t >= VF) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vf[t][db] = *(const uint4 *)(&Vt[buf][(db * 32 + ln) * VS + 16 * t + 8 * lg]);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = Ops::mfma(as_vec<vec>(vf[t][db]), as_vec<vec>(pb), acc[db]);
        }
    };

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    // Tiles every row of the block sees in full: no mask and no skip.
    const int n_full = min(n_tiles, max(0, (r0 + off + 1) / kPfBN));
    int kt = 0;
    for (; kt < n_full; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) load_tile(kt + 1);
        compute_tile(buf, kt * kPfBN, std::false_type());
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }
    // Tiles crossing the diagonal of the block: masked, and skipped by waves
    // whose rows see none of their keys.
    for (; kt < n_tiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) load_tile(kt + 1);
        const int k0 = kt * kPfBN;
        if (k0 <= rw0 + 31 + off) compute_tile(buf, k0, std::true_type());
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- normalise and store: lane holds O^T[d][row] for d = 32db + 8i + 4lg + r ----
    float l_tot = l_part + __shfl_xor(l_part, 32, 64);
    if (my_row < Tq) {
        const float inv = 1.0f / l_tot;
        uint16_t *orow = out + (((size_t)b * Hq + h) * (size_t)Tq + my_row) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = db * 32 + 8 * i + 4 * lg;
                uint2 w;
                w.x = Ops::pack2(acc[db][4 * i + 0] * inv, acc[db][4 * i + 1] * inv);
                w.y = Ops::pack2(acc[db][4 * i + 2] * inv, acc[db][4 * i + 3] * inv);
                *(uint2 *)(orow + d) = w;
            }
    }
}

template <typename T, int D>
static hipError_t launch_pf(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv,
                            int Tq, int Tk, int s_cap, float scale, hipStream_t s)
{
    const int n_rb = (Tq + kPfBM - 1) / kPfBM;
    const float qscale = scale * 1.4426950408889634f;
    dim3 grid(n_rb * Hq, B);
    if (qscale < 0.0f)
        hipLaunchKernelGGL((prefill_causal_kernel<T, D, true>), grid, dim3(kPfThreads), 0, s, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)out, Hq, Hkv, Tq, Tk, s_cap,
                           qscale, n_rb);
    else
        hipLaunchKernelGGL((prefill_causal_kernel<T, D, false>), grid, dim3(kPfThreads), 0, s, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)out, Hq, Hkv, Tq, Tk, s_cap,
                           qscale, n_rb);
    return hipGetLastError();
}

hipError_t launch_prefill(int dtype, int D, const void *q, const void *k, const void *v, void *out, int B,
                          int Hq, int Hkv, int Tq, int Tk, int s_cap, float scale, hipStream_t s)
{
    if (dtype == 1) {
        if (D == 64) return launch_pf<bf16_t, 64>(q, k, v, out, B, Hq, Hkv, Tq, Tk, s_cap, scale, s);
        if (D == 128) return launch_pf<bf16_t, 128>(q, k, v, out, B, Hq, Hkv, Tq, Tk, s_cap, scale, s);
    } else if (dtype == 2) {
        if (D == 64) return launch_pf<f16_t, 64>(q, k, v, out, B, Hq, Hkv, Tq, Tk, s_cap, scale, s);
        if (D == 128) return launch_pf<f16_t, 128>(q, k, v, out, B, Hq, Hkv, Tq, Tk, s_cap, scale, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gqa

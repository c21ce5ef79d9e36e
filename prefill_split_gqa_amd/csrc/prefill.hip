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

#include "common.h"

namespace gqa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

template <typename T> struct MfmaOps;
template <> struct MfmaOps<bf16_t> {
    typedef bf16x8_t vec;
    __device__ __forceinline__ static f32x16_t mfma(vec a, vec b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi)
    {
        __bf16 a = (__bf16)lo, b = (__bf16)hi;
        return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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
        _Float16 a = (_Float16)lo, b = (_Float16)hi;
        return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
};

template <typename V> __device__ __forceinline__ V as_vec(uint4 x) { return __builtin_bit_cast(V, x); }

constexpr int kPfBM = 128;   // query rows per workgroup
constexpr int kPfBN = 64;    // keys per tile
constexpr int kPfThreads = 256;
constexpr int kPfKPad = 8;   // 16-bit elements of padding per K row in LDS
constexpr int kPfVPad = 8;   // per V^T row

template <typename T, int D>
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
    const int wave = tid >> 6, lane = tid & 63;
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

    // Q rows of this wave as MFMA B operands: lane (row ln, group lg) holds
    // dims [16*kb + 8*lg, +8) of its row.
    vec qreg[NKB];
    {
        const int row = rw0 + ln;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (row < Tq) x = *(const uint4 *)(qh + (size_t)row * D + kb * 16 + lg * 8);
            qreg[kb] = as_vec<vec>(x);
        }
    }

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
            kreg[i] = key < Tk ? *(const uint4 *)(kh + (size_t)key * D + c8 * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = tid + i * kPfThreads;
            const int kp = idx % (kPfBN / 2), c8 = idx / (kPfBN / 2);
            const int key = k0 + 2 * kp;
            vreg[i][0] = key < Tk ? *(const uint4 *)(vh + (size_t)key * D + c8 * 8) : make_uint4(0, 0, 0, 0);
            vreg[i][1] = key + 1 < Tk ? *(const uint4 *)(vh + (size_t)(key + 1) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
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
            const uint32_t *a = (const uint32_t *)&vreg[i][0];
            const uint32_t *c = (const uint32_t *)&vreg[i][1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // dims 8*c8 + 2w (low halves) and 8*c8 + 2w + 1 (high halves)
                const uint32_t lo = (a[w] & 0xFFFFu) | (c[w] << 16);
                const uint32_t hi = (a[w] >> 16) | (c[w] & 0xFFFF0000u);
                *(uint32_t *)(&Vt[buf][(c8 * 8 + 2 * w) * VS + 2 * kp]) = lo;
                *(uint32_t *)(&Vt[buf][(c8 * 8 + 2 * w + 1) * VS + 2 * kp]) = hi;
            }
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] = 0.0f;
    float m_ref = -__builtin_huge_valf();
    float l_part = 0.0f;
    const int my_row = rw0 + ln;
    const int my_lim = my_row + off;  // last visible key of this lane's row

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = 0; kt < n_tiles; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) load_tile(kt + 1);
        const int k0 = kt * kPfBN;

        if (k0 <= rw0 + 31 + off) {  // some row of this wave sees this tile
            // ---- S^T = K Q^T for two 32-key sub-tiles ----
            f32x16_t st[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int j = 0; j < 16; ++j) st[u][j] = 0.0f;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const uint4 x = *(const uint4 *)(&Ks[buf][(u * 32 + ln) * KS + kb * 16 + lg * 8]);
                    st[u] = Ops::mfma(as_vec<vec>(x), qreg[kb], st[u]);
                }
            }
            // ---- scale to log2 units, mask, tile max ----
            const bool diag = k0 + kPfBN - 1 > rw0 + off;
            float tmax = -__builtin_huge_valf();
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    float t = st[u][j] * qscale;
                    if (diag) {
                        const int key = k0 + u * 32 + 8 * (j >> 2) + 4 * lg + (j & 3);
                        if (key > my_lim) t = -__builtin_huge_valf();
                    }
                    st[u][j] = t;
                    tmax = fmaxf(tmax, t);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            // ---- lazy rescale of the running output ----
            const bool need = tmax > m_ref + 8.0f;
            if (__any(need)) {
                const float mn = fmaxf(m_ref, tmax);
                const float al = (mn == m_ref) ? 1.0f : fast_exp2(m_ref - mn);
                m_ref = mn;
                l_part *= al;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[db][j] *= al;
            }
            // ---- probabilities -> 16-bit B operands ----
            uint32_t pw[2][8];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                    const float p0 = fast_exp2(st[u][j] - m_ref);
                    const float p1 = fast_exp2(st[u][j + 1] - m_ref);
                    l_part += p0 + p1;
                    pw[u][j / 2] = Ops::pack2(p0, p1);
                }
            // ---- O^T += V^T P^T, four 16-key k-blocks ----
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int u = t >> 1, hh = t & 1;
                const uint4 pb = make_uint4(pw[u][hh * 4 + 0], pw[u][hh * 4 + 1], pw[u][hh * 4 + 2], pw[u][hh * 4 + 3]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint16_t *vrow = &Vt[buf][(db * 32 + ln) * VS + 16 * t + 4 * lg];
                    const uint2 lo = *(const uint2 *)(vrow);
                    const uint2 hi = *(const uint2 *)(vrow + 8);
                    const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    acc[db] = Ops::mfma(as_vec<vec>(va), as_vec<vec>(pb), acc[db]);
                }
            }
        }
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
    hipLaunchKernelGGL((prefill_causal_kernel<T, D>), grid, dim3(kPfThreads), 0, s, (const uint16_t *)q,
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

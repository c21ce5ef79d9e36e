// decode.hip -- split-K single-token grouped-query attention for gfx950.
//
// One workgroup (8 waves, 512 lanes) handles one split of the KV length for
// one KV head and GT of the query heads that share it ("Why It Matters: 7x
// KV Expansion" on the Candle decode page: the fused kernel reads each KV
// head once through a GQA stride; here the heads of a group share the load).
//
// Lane layout: each key row is read by a 16-lane row-group with 16-byte
// (or 8-byte) coalesced loads; a wave reads 4 consecutive rows per load
// instruction and the workgroup 32 rows per step.  Each lane owns D/16
// elements of the row; a dot product is finished with four DPP steps inside
// the 16-lane row.  Each row-group keeps its own online-softmax state
// (reference max, sum, output slice) in registers; the reference max is only
// raised when a score exceeds it by more than 2^8 (log2 domain), so the
// rescale of the output registers is rare and the result is exact up to
// rounding.  Two 64-row chunks of K and V are in flight per workgroup.
//
// End of a workgroup: the four row-groups of a wave are merged with the
// gfx950 cross-half lane swaps (a reduce-scatter: after two swap+add steps
// each lane owns a quarter of the wave's output slice), the eight waves
// through LDS, giving one (max, sum, output) partial per split.  The last
// workgroup of a (request, head tile) to finish merges every split's
// partial with the log-sum-exp rule, in split order, so results do not
// depend on timing.
//
// Cross-workgroup exchange without cache maintenance: on gfx950 each XCD has
// its own L2, and a device-scope fence writes back / invalidates that L2
// (tens of microseconds across a full launch).  Instead, every value that
// crosses workgroups is written and read with device-scope (sc1) accesses,
// which are coherent at device scope by themselves; the writer waits for its
// stores to complete before taking its ticket with a device-scope atomic
// add, and the merger only reads after its ticket shows that every partial
// was published.
//
// The 4-bit cache variant (VeloxQuant-MLX "attention" posts, Part 4: codes,
// scales, biases and the group size go to the kernel, which dequantizes in
// registers) replaces the row loads by code/scale/bias loads and the
// unpacking by the group-affine dequant below; everything else is shared.

#include "common.h"

namespace gqa {

// ---------------------------------------------------------------------------
// Group-affine 4-bit dequant of one element: scale * code + bias, one
// rounding (scale * code is exact in fp32, so this equals the fused
// multiply-add).  The dequant check entry point calls this same function.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float q4_dequant_value(float scale, float bias, uint32_t code)
{
    return __builtin_fmaf(scale, (float)code, bias);
}

// Dense K/V rows of D elements of type T.
template <typename T, int D>
struct DenseKV {
    static constexpr int EPL = D / 16;                            // elements per lane
    static constexpr int BPL = D * (int)sizeof(T) / 16;           // bytes per lane
    static constexpr int U = BPL >= 16 ? 16 : BPL;                // bytes per load
    static constexpr int NU = BPL / U;                            // loads per lane per row
    static constexpr int EU = U / (int)sizeof(T);                 // elements per load
    static constexpr int WPU = U / 4;                             // words per load
    struct Raw { uint32_t w[NU * WPU]; };

    __device__ __forceinline__ static int dim(int lr, int e) { return ((e / EU) * 16 + lr) * EU + (e % EU); }

    struct Src {
        const T *base;  // row 0 of this (request, KV head)
    };
    __device__ __forceinline__ static Src make_src(const DecodeArgs &a, bool is_v, size_t head_row0, int)
    {
        return Src{(const T *)(is_v ? a.v : a.k) + head_row0 * D};
    }

    __device__ __forceinline__ static void load(Raw &r, const Src &s, int row, int lr)
    {
        const char *p = (const char *)(s.base + (size_t)row * D);
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const char *pj = p + (size_t)(j * 16 + lr) * U;
            if constexpr (U == 16) {
                uint4 x = *(const uint4 *)pj;
                r.w[j * 4 + 0] = x.x; r.w[j * 4 + 1] = x.y; r.w[j * 4 + 2] = x.z; r.w[j * 4 + 3] = x.w;
            } else {
                uint2 x = *(const uint2 *)pj;
                r.w[j * 2 + 0] = x.x; r.w[j * 2 + 1] = x.y;
            }
        }
    }
    __device__ __forceinline__ static void zero(Raw &r)
    {
#pragma unroll
        for (int i = 0; i < NU * WPU; ++i) r.w[i] = 0;
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float *x)
    {
        constexpr int PW = Unpack<T>::per_word;
#pragma unroll
        for (int i = 0; i < NU * WPU; ++i) Unpack<T>::run(r.w[i], x + i * PW);
    }
    // a query row has the same element type and lane layout as a K row
    __device__ __forceinline__ static void load_q(float *x, const void *q, size_t row, int lr)
    {
        Raw r;
        Src qs{(const T *)q + row * D};
        load(r, qs, 0, lr);
        unpack(r, x);
    }
};

// 4-bit group-affine K/V rows: D/2 bytes of codes plus D/group f16 scales and
// biases.  Lane lr owns the D/16 consecutive elements starting at lr*D/16.
template <int D>
struct Q4KV {
    static constexpr int EPL = D / 16;
    static constexpr int CB = EPL / 2;  // code bytes per lane (4 or 2)
    struct Raw { uint32_t codes; uint32_t sb; };  // sb: scale bits | bias bits << 16

    __device__ __forceinline__ static int dim(int lr, int e) { return lr * EPL + e; }

    struct Src {
        const uint8_t *codes;
        const uint16_t *scales, *biases;
        int n_groups;      // D / group
        int lane_group;    // group index of this lane's elements
    };
    __device__ __forceinline__ static Src make_src(const DecodeArgs &a, bool is_v, size_t head_row0, int lr)
    {
        Src r;
        r.n_groups = D / a.group;
        r.lane_group = (lr * EPL) / a.group;
        r.codes = (const uint8_t *)(is_v ? a.v : a.k) + head_row0 * (D / 2);
        r.scales = (const uint16_t *)(is_v ? a.v_scales : a.k_scales) + head_row0 * r.n_groups;
        r.biases = (const uint16_t *)(is_v ? a.v_biases : a.k_biases) + head_row0 * r.n_groups;
        return r;
    }

    __device__ __forceinline__ static void load(Raw &r, const Src &s, int row, int lr)
    {
        const uint8_t *c = s.codes + (size_t)row * (D / 2) + lr * CB;
        if constexpr (CB == 4) r.codes = *(const uint32_t *)c;
        else r.codes = *(const uint16_t *)c;
        const size_t gi = (size_t)row * s.n_groups + s.lane_group;
        r.sb = (uint32_t)s.scales[gi] | ((uint32_t)s.biases[gi] << 16);
    }
    __device__ __forceinline__ static void zero(Raw &r) { r.codes = 0; r.sb = 0; }
    // f16 query: the lane's D/16 consecutive elements in one vector load
    __device__ __forceinline__ static void load_q(float *x, const void *q, size_t row, int lr)
    {
        const uint16_t *p = (const uint16_t *)q + row * D + lr * EPL;
        uint32_t w[EPL / 2];
        if constexpr (EPL == 8) {
            const uint4 v = *(const uint4 *)p;
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else {
            const uint2 v = *(const uint2 *)p;
            w[0] = v.x; w[1] = v.y;
        }
#pragma unroll
        for (int i = 0; i < EPL / 2; ++i) Unpack<f16_t>::run(w[i], x + 2 * i);
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float *x)
    {
        const float sc = f16_bits_to_f32(r.sb & 0xFFFFu);
        const float bi = f16_bits_to_f32(r.sb >> 16);
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = q4_dequant_value(sc, bi, (r.codes >> (4 * e)) & 0xFu);
    }
};

// Output stores of 4 consecutive elements.
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d)
{
    *(float4 *)p = make_float4(a, b, c, d);
}
template <typename T16>
__device__ __forceinline__ void store4(T16 *p, float a, float b, float c, float d)
{
    T16 t[4];
    store_elem(&t[0], a); store_elem(&t[1], b); store_elem(&t[2], c); store_elem(&t[3], d);
    uint2 w;
    w.x = (uint32_t)t[0].bits | ((uint32_t)t[1].bits << 16);
    w.y = (uint32_t)t[2].bits | ((uint32_t)t[3].bits << 16);
    *(uint2 *)p = w;
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazyRescale = 8.0f;  // log2 units
constexpr int kSC1 = 16;              // cache policy bit: device-scope coherence

__device__ __forceinline__ float rel_weight(float m_part, float m_total)
{
    return m_part == kNegInf ? 0.0f : fast_exp2(m_part - m_total);
}

// gfx950 cross-half swaps (see the file header).
__device__ __forceinline__ void swap32(float a, float b, float &lo, float &hi)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float a, float b, float &lo, float &hi)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
// max / sum over the 4 row-groups of a wave (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rowgroup_max(float x)
{
    float a, b;
    swap32(x, x, a, b);
    x = fmaxf(a, b);
    swap16(x, x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float rowgroup_sum(float x)
{
    float a, b;
    swap32(x, x, a, b);
    x = a + b;
    swap16(x, x, a, b);
    return a + b;
}

// Waits until this workgroup's device-scope stores have completed, then
// takes a ticket; true in every thread of the last of `expected` arrivals.
__device__ __forceinline__ bool take_ticket(unsigned *counter, unsigned expected, int *s_flag)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();                // ... and so have every other wave's
    if (threadIdx.x == 0) {
        const unsigned t = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = (t == expected - 1);
        if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

template <class KV, typename TQ, int D, int GT>
__global__ __launch_bounds__(kDecodeThreads) void decode_splitk_kernel(DecodeArgs a)
{
    constexpr int EPL = D / 16;
    constexpr int RC = 2;                     // rows per row-group per chunk
    constexpr int CHUNK = RC * kDecodeRowGroups;
    constexpr int NW = kDecodeThreads / 64;   // waves
    constexpr int NF = GT * EPL;              // output registers per lane
    constexpr int NQ = GT * D / 4;            // 4-wide output items
    static_assert(KV::EPL == EPL, "lane layout mismatch");
    static_assert(NF % 4 == 0 && NQ <= kDecodeThreads, "tile shape");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, rgq = lane >> 4, lr = lane & 15;
    const int rg = wave * 4 + rgq;  // row-group within the workgroup
    const int s = blockIdx.x, ht = blockIdx.y, b = blockIdx.z;
    const DecodePlan &P = a.plan;

    int n = a.kv_len;
    if (a.kv_lens) {
        n = a.kv_lens[b];
        n = n < 0 ? 0 : (n > a.s_cap ? a.s_cap : n);
    }
    const int n_split = (n + P.L - 1) / P.L;
    const int g = ht / P.ht_per_kv;
    const int h0 = g * P.G + (ht % P.ht_per_kv) * GT;
    TQ *out = (TQ *)a.out + ((size_t)b * a.Hq + h0) * D;

    if (n == 0) {  // empty request: defined as an all-zero output
        if (s == 0)
            for (int idx = tid; idx < GT * D; idx += kDecodeThreads) store_elem(out + idx, 0.0f);
        return;
    }
    if (s >= n_split) return;
    const int start = s * P.L;
    const int end = min(start + P.L, n);

    const size_t head_row0 = ((size_t)b * a.Hkv + g) * (size_t)a.s_cap;
    const typename KV::Src src = KV::make_src(a, false, head_row0, lr);
    const typename KV::Src srcv = KV::make_src(a, true, head_row0, lr);

    typename KV::Raw kr[2][RC], vr[2][RC];
    auto load_chunk = [&](int buf, int c0) {
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) {
            const int row = c0 + rr * kDecodeRowGroups + rg;
            if (row < end) {
                KV::load(kr[buf][rr], src, row, lr);
                KV::load(vr[buf][rr], srcv, row, lr);
            } else {
                KV::zero(kr[buf][rr]);
                KV::zero(vr[buf][rr]);
            }
        }
    };
    load_chunk(0, start);

    // Queries of the GT heads, pre-multiplied by scale*log2(e).
    float qf[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        KV::load_q(qf[h], a.q, (size_t)b * a.Hq + h0 + h, lr);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[h][e] *= a.qscale;
    }

    float m[GT], l[GT], o[GT][EPL];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        m[h] = kNegInf;
        l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] = 0.0f;
    }

    auto process_chunk = [&](int buf, int c0) {
        float sc[RC][GT];
        bool valid[RC];
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) {
            valid[rr] = (c0 + rr * kDecodeRowGroups + rg) < end;
            float kf[EPL];
            KV::unpack(kr[buf][rr], kf);
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf(qf[h][e], kf[e], acc);
                acc = row16_sum(acc);
                sc[rr][h] = valid[rr] ? acc : kNegInf;
            }
        }
        bool need = false;
        float mc[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            mc[h] = sc[0][h];
#pragma unroll
            for (int rr = 1; rr < RC; ++rr) mc[h] = fmaxf(mc[h], sc[rr][h]);
            need |= mc[h] > m[h] + kLazyRescale;
        }
        if (__any(need)) {
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                const float mn = fmaxf(m[h], mc[h]);
                const float al = (mn == m[h]) ? 1.0f : fast_exp2(m[h] - mn);
                m[h] = mn;
                l[h] *= al;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[h][e] *= al;
            }
        }
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) {
            float vf[EPL];
            KV::unpack(vr[buf][rr], vf);
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                const float p = valid[rr] ? fast_exp2(sc[rr][h] - m[h]) : 0.0f;
                l[h] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[h][e] = __builtin_fmaf(p, vf[e], o[h][e]);
            }
        }
    };

    // Two-deep register pipeline over the chunks of this split.
    for (int c0 = start; c0 < end; c0 += 2 * CHUNK) {
        const int c1 = c0 + CHUNK;
        if (c1 < end) load_chunk(1, c1);
        process_chunk(0, c0);
        if (c1 >= end) break;
        if (c1 + CHUNK < end) load_chunk(0, c1 + CHUNK);
        process_chunk(1, c1);
    }

    // ---- merge the 4 row-groups of each wave ----
    __shared__ __attribute__((aligned(16))) float so[NW][GT][D];
    __shared__ float sm[NW][GT], sl[NW][GT];
    __shared__ int s_last;
    float of[NF];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        const float mw = rowgroup_max(m[h]);
        const float al = rel_weight(m[h], mw);
        const float lw = rowgroup_sum(l[h] * al);
#pragma unroll
        for (int e = 0; e < EPL; ++e) of[h * EPL + e] = o[h][e] * al;
        if (lane == 0) { sm[wave][h] = mw; sl[wave][h] = lw; }
    }
    float w1[NF / 2], w2[NF / 4];
#pragma unroll
    for (int f = 0; f < NF / 2; ++f) {
        float lo, hi;
        swap32(of[f], of[f + NF / 2], lo, hi);
        w1[f] = lo + hi;
    }
#pragma unroll
    for (int f = 0; f < NF / 4; ++f) {
        float lo, hi;
        swap16(w1[f], w1[f + NF / 4], lo, hi);
        w2[f] = lo + hi;
    }
    {
        const int fbase = (lane >> 5) * (NF / 2) + ((lane >> 4) & 1) * (NF / 4);
#pragma unroll
        for (int f = 0; f < NF / 4; ++f) {
            const int ff = fbase + f;
            so[wave][ff / EPL][KV::dim(lr, ff % EPL)] = w2[f];
        }
    }
    __syncthreads();

    // ---- workgroup partial: 4 consecutive dims per item ----
    const int col = b * P.HT + ht;
    const int qh = tid / (D / 4), qd = (tid % (D / 4)) * 4;
    float Mw = kNegInf, Lw = 0.0f, O0 = 0.0f, O1 = 0.0f, O2 = 0.0f, O3 = 0.0f;
    if (tid < NQ) {
#pragma unroll
        for (int w = 0; w < NW; ++w) Mw = fmaxf(Mw, sm[w][qh]);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float wt = rel_weight(sm[w][qh], Mw);
            const float4 x = *(const float4 *)&so[w][qh][qd];
            Lw += wt * sl[w][qh];
            O0 += wt * x.x; O1 += wt * x.y; O2 += wt * x.z; O3 += wt * x.w;
        }
    }
    if (n_split == 1) {
        if (tid < NQ) store4(out + (size_t)qh * D + qd, O0 / Lw, O1 / Lw, O2 / Lw, O3 / Lw);
        return;
    }

    // ---- publish the partial with device-scope stores ----
    const __amdgpu_buffer_rsrc_t ws_o =
        __builtin_amdgcn_make_buffer_rsrc(a.part_o, 0, (int)(P.off_ml - P.off_o), 0x00020000);
    const __amdgpu_buffer_rsrc_t ws_ml =
        __builtin_amdgcn_make_buffer_rsrc(a.part_ml, 0, (int)(P.off_cnt - P.off_ml), 0x00020000);
    const size_t colbase = (size_t)col * P.n_split_max;
    if (tid < NQ) {
        const int off_o = (int)((((colbase + s) * GT + qh) * D + qd) * 4);
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, make_float4(O0, O1, O2, O3)), ws_o,
            off_o, 0, kSC1);
        if (qd == 0) {
            const int off_ml = (int)(((colbase + s) * GT + qh) * 2 * 4);
            __builtin_amdgcn_raw_buffer_store_b64(
                __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, make_float2(Mw, Lw)), ws_ml,
                off_ml, 0, kSC1);
        }
    }
    if (!take_ticket(&a.cnt[col], (unsigned)n_split, &s_last)) return;

    // ---- last arrival: merge every split's partial in one round trip ----
    // Thread t handles output item t % 256 over the splits of half t / 256
    // (up to kDecodeMaxSplits / 2 each); the (max, sum) pairs of every split
    // are staged in LDS by the same round trip.  The merge order is fixed:
    // each half sums its splits in order, then half 0 adds half 1.
    constexpr int HALF = kDecodeMaxSplits / 2;
    static_assert(kDecodeThreads == 512 && NQ <= 256, "merge layout");
    __shared__ float2 sml[kDecodeMaxSplits][GT];
    __shared__ float4 sacc[256];
    __shared__ float sls[256];
    const int item = tid & 255, hf = tid >> 8;
    const int mh = item / (D / 4), md = (item % (D / 4)) * 4;
    const int s_first = hf * HALF;
    const int s_count = max(0, min(HALF, n_split - s_first));
    float4 po[HALF];
    if (item < NQ) {
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
            const int sj = j < s_count ? s_first + j : 0;
            const int off_o = (int)((((colbase + sj) * GT + mh) * D + md) * 4);
            po[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ws_o, off_o, 0, kSC1));
        }
    }
    if (tid < n_split * GT) {
        const int ms = tid / GT, mhh = tid % GT;
        const int off_ml = (int)(((colbase + ms) * GT + mhh) * 2 * 4);
        sml[ms][mhh] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ws_ml, off_ml, 0, kSC1));
    }
    __syncthreads();
    float M = kNegInf;
    if (item < NQ)
        for (int j = 0; j < n_split; ++j) M = fmaxf(M, sml[j][mh].x);
    float Ls = 0.0f;
    float4 R = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (item < NQ) {
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
            if (j >= s_count) continue;
            const float2 ml = sml[s_first + j][mh];
            const float w = rel_weight(ml.x, M);
            Ls += w * ml.y;
            R.x += w * po[j].x; R.y += w * po[j].y; R.z += w * po[j].z; R.w += w * po[j].w;
        }
    }
    if (hf == 1) { sacc[item] = R; sls[item] = Ls; }
    __syncthreads();
    if (hf == 0 && item < NQ) {
        const float4 R1 = sacc[item];
        Ls += sls[item];
        R.x += R1.x; R.y += R1.y; R.z += R1.z; R.w += R1.w;
        store4(out + (size_t)mh * D + md, R.x / Ls, R.y / Ls, R.z / Ls, R.w / Ls);
    }
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
template <class KV, typename TQ, int D, int GT>
static hipError_t launch_one(int B, const DecodeArgs &a, hipStream_t stream)
{
    const int gx = a.kv_lens ? a.plan.n_split_max : (a.kv_len + a.plan.L - 1) / a.plan.L;
    dim3 grid(gx, a.plan.HT, B);
    hipLaunchKernelGGL((decode_splitk_kernel<KV, TQ, D, GT>), grid, dim3(kDecodeThreads), 0, stream, a);
    return hipGetLastError();
}

template <class KV, typename TQ, int D>
static hipError_t dispatch_gt(int B, const DecodeArgs &a, hipStream_t s)
{
    switch (a.plan.GT) {
    case 1: return launch_one<KV, TQ, D, 1>(B, a, s);
    case 2: return launch_one<KV, TQ, D, 2>(B, a, s);
    case 3: return launch_one<KV, TQ, D, 3>(B, a, s);
    case 4: return launch_one<KV, TQ, D, 4>(B, a, s);
    case 5: return launch_one<KV, TQ, D, 5>(B, a, s);
    case 6: return launch_one<KV, TQ, D, 6>(B, a, s);
    case 7: return launch_one<KV, TQ, D, 7>(B, a, s);
    case 8: return launch_one<KV, TQ, D, 8>(B, a, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int D>
static hipError_t dispatch_dense(int B, const DecodeArgs &a, hipStream_t s)
{
    return dispatch_gt<DenseKV<T, D>, T, D>(B, a, s);
}

hipError_t launch_decode(int dtype, int D, int B, const DecodeArgs &a, hipStream_t s)
{
    if (D == 128) {
        if (dtype == 0) return dispatch_dense<float, 128>(B, a, s);
        if (dtype == 1) return dispatch_dense<bf16_t, 128>(B, a, s);
        if (dtype == 2) return dispatch_dense<f16_t, 128>(B, a, s);
    } else if (D == 64) {
        if (dtype == 0) return dispatch_dense<float, 64>(B, a, s);
        if (dtype == 1) return dispatch_dense<bf16_t, 64>(B, a, s);
        if (dtype == 2) return dispatch_dense<f16_t, 64>(B, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode_q4(int D, int group, int B, const DecodeArgs &a, hipStream_t s)
{
    if (group != a.group) return hipErrorInvalidValue;
    if (D == 128) return dispatch_gt<Q4KV<128>, f16_t, 128>(B, a, s);
    if (D == 64) return dispatch_gt<Q4KV<64>, f16_t, 64>(B, a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Dequant check hook: one thread per element, same dequant function.
// ---------------------------------------------------------------------------
__global__ void dequant_q4_kernel(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                                  float *out, long n_elems, int D, int group)
{
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_elems) return;
    const long row = i / D;
    const int e = (int)(i % D);
    const uint32_t byte = codes[row * (D / 2) + e / 2];
    const uint32_t code = (e & 1) ? (byte >> 4) : (byte & 0xFu);
    const long gi = row * (D / group) + e / group;
    out[i] = q4_dequant_value(f16_bits_to_f32(scales[gi]), f16_bits_to_f32(biases[gi]), code);
}

hipError_t launch_dequant_q4(const uint8_t *codes, const void *scales, const void *biases, float *out,
                             int n_rows, int D, int group, hipStream_t s)
{
    const long n = (long)n_rows * D;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    const long blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(dequant_q4_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, codes,
                       (const uint16_t *)scales, (const uint16_t *)biases, out, n, D, group);
    return hipGetLastError();
}

// Zero-fill with a kernel (kept out of hipMemsetAsync so that callers may
// capture it in a graph).
__global__ void fill_zero_kernel(uint32_t *p, size_t n_words)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s)
{
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)p, words);
    return hipGetLastError();
}

}  // namespace gqa

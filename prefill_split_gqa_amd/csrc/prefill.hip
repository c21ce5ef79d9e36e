// prefill.hip -- causal grouped-query prefill on the gfx950 matrix cores.
//
// "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x faster",
// section "Cause and workaround": one pass reads the grouped KV heads
// directly, applies the causal mask inside the kernel with the queries
// aligned to the end of the keys (row i sees keys j <= i + Tk - Tq), and never
// stores the score matrix.
//
// Work decomposition: a workgroup owns 128 query rows of one query head and
// has 8 waves: row-wave w (32 rows) appears twice, once in each half of the
// workgroup, and the two halves walk the first and the second half of the
// visible key tiles (64 keys each) side by side.  At the end the second
// half's running (output, max, sum) goes through LDS and is merged into the
// first half's, which normalises and stores.  Splitting the keys halves the
// longest chain of dependent tiles (the last row block sees every key) while
// the merge costs one LDS round trip.  Each half stages its K tiles row-major
// in LDS and its V tiles transposed (V^T, keys contiguous), double-buffered,
// with the next tile's global loads in flight while the current tile is
// computed.
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

constexpr int kPfBM = 128;          // query rows per workgroup (4 row-waves of 32)
constexpr int kPfBN = 64;           // keys per tile
constexpr int kPfHalfThreads = 256; // one key half: 4 waves
constexpr int kPfThreads = 512;     // two key halves
constexpr int kPfKPad = 8;          // 16-bit elements of padding per K row in LDS
constexpr int kPfVPad = 8;          // per V^T row

// LDS layout: for each key half, two buffers of [K tile | V^T tile]; after
// the key loop the same memory holds the second half's partial results.
template <int D> struct PfSmem {
    static constexpr int KS = D + kPfKPad;      // K row stride (elements)
    static constexpr int VS = kPfBN + kPfVPad;  // V^T row stride (elements)
    static constexpr int K_ELEMS = kPfBN * KS;
    static constexpr int BUF = K_ELEMS + D * VS;
    static constexpr int TOTAL = 2 * 2 * BUF;
    static constexpr int MERGE_FLOATS = 4 * (D / 32) * 16 * 64 + 4 * 64 * 2;
    static_assert(MERGE_FLOATS * 4 <= TOTAL * 2, "merge area exceeds the tile buffers");
};

// Softmax part of one 64-key tile for the wave's 32 rows, in place.
//
// st holds S^T (raw q.k) in the accumulator layout: lane (ln, lg) has, for
// sub-tile u and register j, key 32u + 8(j/4) + 4lg + (j%4) of the tile, row
// ln.  Masked keys already hold sigma*(-inf), sigma the sign of the scale.
// The running maximum m_run is kept over the oriented raw scores sigma*s, so
// that one fused multiply-add per score gives the log2-domain exponent
// exp2(s*qs - |qs|*m_run).  m_run is raised only when a tile's maximum
// exceeds it by more than thr (2^8 in the exponent); the running output and
// sum are rescaled then.  On return st holds the probabilities (fp32).
template <bool NEG, int NDB>
__device__ __forceinline__ void softmax_inplace(f32x16_t (&st)[2], f32x16_t (&acc)[NDB], float &m_run,
                                                float &l_part, float qs, float thr)
{
    constexpr float kInf = __builtin_huge_valf();
    float tmax = -kInf;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, NEG ? -st[u][j] : st[u][j]);
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
    // a row that has seen no visible key yet (all -inf so far) gets p = 0
    const float mq = m_run == -kInf ? 0.0f : -fabsf(qs) * m_run;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 16; ++j) st[u][j] = fast_exp2(__builtin_fmaf(st[u][j], qs, mq));
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
    typedef PfSmem<D> L;
    constexpr int KS = L::KS;
    constexpr int VS = L::VS;
    constexpr int NKB = D / 16;  // k-blocks of the QK^T product
    constexpr int NDB = D / 32;  // 32-wide d-blocks of the output
    constexpr float kInf = __builtin_huge_valf();
    __shared__ __attribute__((aligned(16))) uint16_t smem[L::TOTAL];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2;  // which half of the key tiles this wave walks
    const int rw = wave & 3;     // row-wave within the block
    const int htid = tid & (kPfHalfThreads - 1);
    const int lane = tid & 63;
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
    const int rw0 = r0 + rw * 32;                   // first row of this wave
    const int row_hi = min(r0 + kPfBM, Tq);         // one past the last valid row of the block
    const int kend = min(Tk, row_hi + off);         // keys any valid row of the block can see
    const int n_tiles = (kend + kPfBN - 1) / kPfBN;
    const int n = (n_tiles + 1) / 2;                // steps; the first half has n tiles, the second the rest
    const int t_begin = half ? n : 0;
    const int n_full = min(n_tiles, max(0, (r0 + off + 1) / kPfBN));  // tiles every row sees in full
    uint16_t *const hsm = smem + half * 2 * L::BUF;  // this half's two buffers

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

    // global -> register -> LDS staging of K and V tiles by the 256 threads
    // of a half.  Tile indices past the end load zeros (range-checked
    // buffers) or keys no valid row sees, into buffers nobody reads any more,
    // so neither step branches.
    constexpr int K_ITEMS = kPfBN * D / 8;          // 16-byte pieces per K tile
    constexpr int K_PER_T = K_ITEMS / kPfHalfThreads;
    constexpr int V_ITEMS = (kPfBN / 2) * (D / 8);  // (key pair, 8-dim chunk)
    constexpr int V_PER_T = V_ITEMS / kPfHalfThreads;
    static_assert(K_ITEMS % kPfHalfThreads == 0 && V_ITEMS % kPfHalfThreads == 0, "tile/thread mismatch");
    uint4 kreg[2][K_PER_T], vreg[2][V_PER_T][2];  // two staging sets: loads run two steps ahead

    auto load_k = [&](int kt, int set) {
        const int k0 = kt * kPfBN;
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int idx = htid + i * kPfHalfThreads;
            const int key = k0 + idx / (D / 8), c8 = idx % (D / 8);
            kreg[set][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (key * D + c8 * 8) * 2, 0, 0));
        }
    };
    auto load_v = [&](int kt, int set) {
        const int k0 = kt * kPfBN;
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = htid + i * kPfHalfThreads;
            const int kp = idx % (kPfBN / 2), c8 = idx / (kPfBN / 2);
            const int key = k0 + 2 * kp;
            vreg[set][i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (key * D + c8 * 8) * 2, 0, 0));
            vreg[set][i][1] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, ((key + 1) * D + c8 * 8) * 2, 0, 0));
        }
    };
    auto k_buf = [&](int buf) { return hsm + buf * L::BUF; };
    auto v_buf = [&](int buf) { return hsm + buf * L::BUF + L::K_ELEMS; };
    auto store_k = [&](int buf, int set) {
        uint16_t *Ks = k_buf(buf);
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int idx = htid + i * kPfHalfThreads;
            const int key = idx / (D / 8), c8 = idx % (D / 8);
            *(uint4 *)(&Ks[key * KS + c8 * 8]) = kreg[set][i];
        }
    };
    auto store_v = [&](int buf, int set) {
        uint16_t *Vt = v_buf(buf);
#pragma unroll
        for (int i = 0; i < V_PER_T; ++i) {
            const int idx = htid + i * kPfHalfThreads;
            const int kp = idx % (kPfBN / 2), c8 = idx / (kPfBN / 2);
            const int pos = vt_pos(2 * kp);
            const uint32_t *a = (const uint32_t *)&vreg[set][i][0];
            const uint32_t *c = (const uint32_t *)&vreg[set][i][1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // dims 8*c8 + 2w (low halves of the two keys) and 8*c8 + 2w + 1 (high halves)
                *(uint32_t *)(&Vt[(c8 * 8 + 2 * w) * VS + pos]) = __builtin_amdgcn_perm(c[w], a[w], 0x05040100u);
                *(uint32_t *)(&Vt[(c8 * 8 + 2 * w + 1) * VS + pos]) = __builtin_amdgcn_perm(c[w], a[w], 0x07060302u);
            }
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] = 0.0f;
    f32x16_t st[2];  // S^T of the current tile, then its probabilities
    float m_run = -kInf;  // running max of the oriented raw scores of this lane's row
    float l_part = 0.0f;
    const float aq = fabsf(qscale);
    const float thr = fminf(8.0f / aq, 3.0e38f);  // lazy-rescale threshold, raw units (qscale != 0)
    const int my_row = rw0 + ln;
    const int my_lim = my_row + off;  // last visible key of this lane's row

    // Keys of a tile that crosses the diagonal get sigma*(-inf) where masked.
    auto mask_tile = [&](int kt) {
        if (kt >= n_full) {
            // (kept a real branch: the empty asm stops the compiler from
            // turning the mask into selects executed on every tile)
            asm volatile("");
            const int key0 = kt * kPfBN + 4 * lg;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (key0 + 32 * u + 8 * (j >> 2) + (j & 3) > my_lim) st[u][j] = NEG ? kInf : -kInf;
        }
    };
    // S^T = K Q^T for tile kt from K fragments already in registers
    auto qk_frags = [&](int kt, const uint4 (&kf)[2][NKB]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) st[u][j] = 0.0f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u) st[u] = Ops::mfma(as_vec<vec>(kf[u][kb]), qreg[kb], st[u]);
        mask_tile(kt);
    };
    // S^T = K Q^T for tile kt (this half's K buffer buf)
    auto qk = [&](int kt, int buf) {
        const uint16_t *Ks = k_buf(buf);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) st[u][j] = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint4 kf[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb] = *(const uint4 *)(&Ks[(u * 32 + ln) * KS + kb * 16 + lg * 8]);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) st[u] = Ops::mfma(as_vec<vec>(kf[kb]), qreg[kb], st[u]);
        }
        mask_tile(kt);
    };

    // The two phases of step s of a half (tile t_begin + s):
    //   V(s): LDS stores of K(s+1), V(s) (loaded two steps earlier, staging
    //         set s&1); loads of K(s+3), V(s+2) issued into the same set;
    //         softmax of tile s in place
    //   M(s): P of tile s rounded to 16 bits and summed; O^T += V^T P^T;
    //         S^T of tile s+1
    // K runs one tile ahead of V: M(s) reads K buffer (s+1)&1 and V buffer
    // s&1; V(s) writes the same two buffers, whose previous tiles M(s-1)
    // read.  A global load has two whole steps to arrive before its store.
    // SET is s&1, a template argument so that the staging registers are
    // named statically (the step loop is unrolled by two).
    auto v_phase = [&](int s, auto set_tag) {
        constexpr int SET = decltype(set_tag)::value;
        if (s > 0) {
            store_k((s + 1) & 1, SET);
            store_v(s & 1, SET);
        }
        load_k(t_begin + s + 3, SET);
        load_v(t_begin + s + 2, SET);
        softmax_inplace<NEG>(st, acc, m_run, l_part, qscale, thr);
    };
    auto m_phase = [&](int s) {
        const uint16_t *Vt = v_buf(s & 1);
        const uint16_t *Ks = k_buf((s + 1) & 1);
        // D = 64: every LDS fragment of the phase is requested up front (64
        // registers), so the reads overlap each other instead of each
        // matrix instruction waiting for the one it needs.
        constexpr bool PRE = D == 64;
        uint4 vf[4][NDB], kf[2][NKB];
        if constexpr (PRE) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    vf[t][db] = *(const uint4 *)(&Vt[(db * 32 + ln) * VS + 16 * t + 8 * lg]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    kf[u][kb] = *(const uint4 *)(&Ks[(u * 32 + ln) * KS + kb * 16 + lg * 8]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // P of tile s to 16 bits (paired conversion) and its row sums (four
        // independent partial sums); O^T += V^T P^T in four 16-key k-blocks
        float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int u = t >> 1, hh = t & 1;
            uint32_t pw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pw[i] = Ops::pack2(st[u][8 * hh + 2 * i], st[u][8 * hh + 2 * i + 1]);
                lsum[i] = Ops::sum2(pw[i], lsum[i]);
            }
            const uint4 pb = make_uint4(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if constexpr (!PRE) vf[t][db] = *(const uint4 *)(&Vt[(db * 32 + ln) * VS + 16 * t + 8 * lg]);
                acc[db] = Ops::mfma(as_vec<vec>(vf[t][db]), as_vec<vec>(pb), acc[db]);
            }
        }
        l_part += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
        // S^T of tile s+1
        if constexpr (PRE) {
            qk_frags(t_begin + s + 1, kf);
        } else {
            qk(t_begin + s + 1, (s + 1) & 1);
        }
    };

    // prologue: K and V of tile 0, K of tile 1 into LDS; K of tile 2 and V
    // of tile 1 in flight into staging set 1 (stored by V(1))
    load_k(t_begin, 0);
    load_v(t_begin, 0);
    store_k(0, 0);
    store_v(0, 0);
    load_k(t_begin + 1, 0);
    store_k(1, 0);
    load_k(t_begin + 2, 1);
    load_v(t_begin + 1, 1);
    __syncthreads();

    // Ping-pong: the second half runs one phase behind the first, so on each
    // SIMD one wave issues matrix instructions while the other (same row
    // block, other key half) runs the softmax.  Both halves run the same
    // sequence qk(0) | V(0) | M(0) | ... | V(n-1) | M(n-1), one barrier
    // after each phase; the second half passes one extra barrier before it
    // starts and the first half one after it ends (a barrier only counts
    // arrivals, so the waves need not be at the same instruction).  The
    // second half has one tile fewer when n_tiles is odd; its extra tile
    // holds keys at or past kend, masked for every valid row.
    // phase_end() is a barrier that the compiler may not move work across:
    // the phases only overlap as intended if each stays between its barriers.
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    if (half == 1) phase_end();
    qk(t_begin, 0);
    phase_end();
    int s = 0;
    for (; s + 1 < n; s += 2) {
        v_phase(s, std::integral_constant<int, 0>());
        phase_end();
        m_phase(s);
        phase_end();
        v_phase(s + 1, std::integral_constant<int, 1>());
        phase_end();
        m_phase(s + 1);
        phase_end();
    }
    if (s < n) {
        v_phase(s, std::integral_constant<int, 0>());
        phase_end();
        m_phase(s);
        phase_end();
    }
    if (half == 0) phase_end();

    // ---- merge the second half's partial results into the first half ----
    // (the last phase ended on a barrier, so the tile buffers are free)
    float *xo = (float *)smem;                   // [row-wave][NDB*16 registers][64 lanes]
    float *xml = xo + 4 * NDB * 16 * 64;         // [row-wave][64 lanes][max, sum]
    if (half == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) xo[((rw * NDB + db) * 16 + j) * 64 + lane] = acc[db][j];
        xml[(rw * 64 + lane) * 2 + 0] = m_run;
        xml[(rw * 64 + lane) * 2 + 1] = l_part;
    }
    __syncthreads();
    if (half == 1) return;
    {
        const float mB = xml[(rw * 64 + lane) * 2 + 0];
        const float lB = xml[(rw * 64 + lane) * 2 + 1];
        const float m = fmaxf(m_run, mB);
        const float wA = m_run == -__builtin_huge_valf() ? 0.0f : fast_exp2(aq * (m_run - m));
        const float wB = mB == -__builtin_huge_valf() ? 0.0f : fast_exp2(aq * (mB - m));
        l_part = wA * l_part + wB * lB;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[db][j] = wA * acc[db][j] + wB * xo[((rw * NDB + db) * 16 + j) * 64 + lane];
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
    // A zero scale (uniform weights over the visible keys) is run as the
    // smallest normal scale: every exponent is then below 2^-80 in
    // magnitude, exp2 of it rounds to exactly 1, and masked keys (-inf)
    // still give 0 rather than inf*0.
    float qscale = scale * 1.4426950408889634f;
    if (qscale == 0.0f) qscale = 1.17549435e-38f;
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

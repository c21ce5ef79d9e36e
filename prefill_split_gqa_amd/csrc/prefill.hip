// prefill.hip -- causal grouped-query prefill on the gfx950 matrix cores.
//
// "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x faster",
// section "Cause and workaround": a single kernel takes K and V with their
// original (grouped) heads, applies the causal mask inside the kernel with
// the queries aligned to the end of the keys (row i sees keys
// j <= i + Tk - Tq), and never stores the score matrix.
//
// Work decomposition.  A workgroup has 4 waves and owns 128 query rows of
// one query head (32 rows per wave) and a contiguous range ("chunk") of the
// 64-key tiles those rows can see.  Short row blocks are one chunk; the long
// ones near the end of the causal triangle are cut into chunks of at most
// ch tiles, ch chosen so that the launch has about three workgroups per CU
// for D = 64 (four are resident).  The host sorts the (row block,
// chunk) items longest first into a table passed with the launch, so the
// long items start first and the short ones fill in behind them.  The
// chunks of a split row block meet through the workspace: each stores its
// partial (output, max, sum) and takes a ticket from a counter; the last
// to arrive merges all partials in chunk order, normalises and stores.
//
// Per tile, on v_mfma_f32_32x32x16 (bf16 or f16 inputs, fp32 sums), each
// wave computes for its 32 rows:
//   S^T[key][row] = K Q^T          (A = K rows from LDS, B = Q rows in registers)
//   online softmax per row in fp32 (exp2 with scale*log2(e) folded in; the
//   reference max is only raised when a score exceeds it by more than 2^8)
//   O^T[d][row] += V^T P^T         (A = V^T fragments from LDS, B = P in registers)
// Computing S transposed makes its accumulator layout (a lane holds keys of
// one row) exactly the layout the second product wants for P, so P never
// leaves registers.  With four workgroups per CU each SIMD runs four waves,
// so one wave's matrix instructions overlap other waves' exponentials.
//
// Data movement.  K and V tiles go from HBM straight into LDS with buffer
// loads that write LDS (no staging registers), row-major, each row's 16-byte
// chunks XOR-swizzled and every 8 rows padded by 64 bytes, so that the
// fragment reads below avoid bank conflicts.  K fragments are plain 16-byte
// reads; V^T fragments come from the transposing LDS read
// (ds_read_b64_tr_b16), which hands each lane four 16-bit values of one
// column from four consecutive rows.  Rows past Tk load as zeros (buffer
// range check).  K and V are double-buffered: the loads of tile t+1 run
// while tile t is computed, and one barrier per tile hands the buffers
// over.  Only tiles that cross a wave's diagonal are masked, and a wave
// skips the arithmetic of tiles it cannot see at all (the end of a row
// block's diagonal, or a last row block with fewer than 128 valid rows).
//
// Sliding window and sinks: tiles wholly before a wave's first visible key
// are skipped, tiles across it masked, and a sink logit joins the final
// normaliser.  A 4-bit cache with a float16 residual window (VeloxQuant
// posts; a chunked prefill reading the quantized cache): key tiles below
// the 4-bit row count are loaded as codes, scales and biases into registers
// and dequantized into the tile buffers at the end of the step; the others
// come from the residual rows by the same LDS DMA as a dense cache.

#include <algorithm>
#include <type_traits>
#include <utility>
#include <vector>

#include "common.h"

namespace gqa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8v_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

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
    __device__ __forceinline__ static uint4 pack8(f32x8_t x)
    {
        return __builtin_bit_cast(uint4, __builtin_convertvector(x, bf16x8v_t));
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
    __device__ __forceinline__ static uint4 pack8(f32x8_t x)
    {
        return __builtin_bit_cast(uint4, __builtin_convertvector(x, f16x8v_t));
    }
};

template <typename V> __device__ __forceinline__ V as_vec(uint4 x) { return __builtin_bit_cast(V, x); }

constexpr int kPfBM = 128;       // query rows per workgroup: 4 row-waves of 32 rows
constexpr int kPfBN = 64;        // keys per tile
constexpr int kPfThreads = 256;  // 4 waves
constexpr int kPfMaxItems = 1024;     // (row block, key chunk) work items in the launch table
constexpr int kPfMinChunk = 3;        // fewest key tiles per chunk
constexpr int kPfMaxSplit = 7;        // most chunks of a row block the floor allows: each partial costs a write and a read
constexpr float kPfSumLimit = 1024.0f;  // a lane's probability sum that needs the exact path

// The launch's work items, longest first: entry r is (row block << 6) |
// chunk; grid block x runs item x / (B * Hq) for request and head
// x % (B * Hq).  ch is the most key tiles a chunk holds; row blocks rb0 and
// later (those with more than ch tiles) are split, each into at most max_nc
// chunks.
struct PfItems {
    int n;
    int ch;
    int rb0;
    int max_nc;
    unsigned short e[kPfMaxItems];
};

// LDS layout (bytes).  A tile is 64 rows of D 16-bit elements: groups of 8
// rows (8 * ROW bytes) followed by 64 bytes of padding.  K buffers 0, 1 then
// V buffers 0, 1.
template <int D> struct PfLds {
    static constexpr int ROW = D * 2;
    static constexpr int GROUP = 8 * ROW + 64;
    static constexpr int TILE = 8 * GROUP;
    static constexpr int TOTAL = 4 * TILE;
};

// Partial result of one key chunk in the workspace: the 4 waves' fp32 O^T
// accumulators, 16 bytes per lane and access ([wave][d-block][j/4][lane]
// [j%4]), then each lane's (max, sum).
template <int D> struct PfSlot {
    static constexpr int O_FLOATS = 4 * (D / 32) * 16 * 64;
    static constexpr int ML_FLOATS = 4 * 64 * 2;
    static constexpr int BYTES = (O_FLOATS + ML_FLOATS) * 4;
};

// XOR applied to the 16-byte chunk index of a row, from the row's position
// in its group of 8.  Any 8 consecutive rows get 8 distinct values (the K
// fragment reads: 8 rows, one chunk each), and any 4 consecutive rows that
// start at a multiple of 4 get distinct values of swz >> 1 (the transposing
// V reads: 4 rows, an aligned pair of chunks each).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <int D> __device__ __forceinline__ int tile_off(int row, int chunk)
{
    typedef PfLds<D> L;
    return (row >> 3) * L::GROUP + (row & 7) * L::ROW + ((chunk ^ swz(row & 7)) << 4);
}

// Reference maximum of one 64-key tile for one 32-row block.
//
// st holds S^T (raw q.k) in the accumulator layout: lane (ln, lg) has, for
// sub-tile u and register j, key 32u + 8(j/4) + 4lg + (j%4) of the tile, row
// ln.  Masked keys already hold sigma*(-inf), sigma the sign of the scale.
// The running maximum m_run is kept over the oriented raw scores sigma*s, so
// that one fused multiply-add per score gives the log2-domain exponent
// exp2(s*qs - |qs|*m_run).  m_run is raised only when the tile's maximum
// exceeds it by more than thr (2^8 in the exponent); the running output and
// sum are rescaled then.  Returns the exponent offset -|qs|*m_run (0 for a
// row that has seen no visible key yet, whose probabilities are then 0).
template <bool NEG, int NDB>
__device__ __forceinline__ float softmax_max(const f32x16_t (&st)[2], f32x16_t (&acc)[NDB], float &m_run,
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
    return m_run == -kInf ? 0.0f : -fabsf(qs) * m_run;
}

template <typename T, int D, bool NEG, bool Q4 = false>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? (Q4 ? 3 : 4) : 2))) void prefill_causal_kernel(const uint16_t *__restrict__ q,
                                                                    const uint16_t *__restrict__ k,
                                                                    const uint16_t *__restrict__ v,
                                                                    uint16_t *__restrict__ out, int Hq, int Hkv,
                                                                    int Tq, int Tk, int s_cap, float qscale,
                                                                    int n_rb, unsigned char *__restrict__ ws,
                                                                    int B, int window, const float *__restrict__ sinks,
                                                                    PfItems items, Q4Source q4)
{
    typedef MfmaOps<T> Ops;
    typedef typename Ops::vec vec;
    typedef PfLds<D> L;
    typedef PfSlot<D> SL;
    constexpr int NRW = 4;             // row-waves
    constexpr int NKB = D / 16;        // k-blocks of the QK^T product
    constexpr int NDB = D / 32;        // 32-wide d-blocks of the output
    constexpr int CPR = D / 8;         // 16-byte chunks per row
    constexpr int RPI = 1024 / L::ROW; // rows per LDS-writing load (64 lanes x 16 bytes)
    constexpr int IPT = kPfBN / RPI;   // such loads per tile
    constexpr int IPW = 2 * IPT / NRW; // loads per wave per step (one K and one V tile)
    constexpr float kInf = __builtin_huge_valf();
    static_assert(2 * IPT % NRW == 0 && IPT % IPW == 0, "load split");
    __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = wave;  // row-wave
    const int lane = tid & 63;
    const int ln = lane & 31, lg = lane >> 5;

    // work item (row block, key chunk) and (request, head) of this workgroup
    const int bh = blockIdx.x % (B * Hq);
    const int item = items.e[blockIdx.x / (B * Hq)];
    const int rb = item >> 6, chunk = item & 63;
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int G = Hq / Hkv;
    const int g = h / G;
    const int off = Tk - Tq;
    const int r0 = rb * kPfBM;
    const int rw0 = r0 + rw * 32;                   // first row of this wave
    const int row_hi = min(r0 + kPfBM, Tq);         // one past the last valid row of the block
    const int kend = min(Tk, row_hi + off);         // keys any valid row of the block can see
    // with a window, row i sees keys i + off - window < j <= i + off: the
    // block's first row sets its first tile
    const int t_lo = window > 0 ? max(0, r0 + off - window + 1) / kPfBN : 0;
    const int n_tiles = (kend + kPfBN - 1) / kPfBN - t_lo;
    const int nc = (n_tiles + items.ch - 1) / items.ch;  // chunks of this row block
    const int per = (n_tiles + nc - 1) / nc;        // tiles per chunk
    const int t_begin = t_lo + min(n_tiles, chunk * per);
    const int n = min(n_tiles, chunk * per + per) - min(n_tiles, chunk * per);
    // Per wave (wave-uniform): tiles below n_full are visible in full to
    // every row of the wave, so they need no mask; tiles from w_end on are
    // masked for every row of the wave (or the wave has no valid row), so it
    // skips their arithmetic and only takes part in the loads and barriers.
    // With a window, tiles below w_begin are below every row's first visible
    // key (skipped like those past w_end), and tiles below lo_full cross
    // some row's first visible key (masked).
    const int t_hi = t_lo + n_tiles;
    const int n_full = min(t_hi, (rw0 + off + 1) / kPfBN);
    const int w_end = rw0 < row_hi ? min(t_hi, (min(rw0 + 31, row_hi - 1) + off) / kPfBN + 1) : 0;
    const int w_begin = window > 0 ? max(0, rw0 + off - window + 1) / kPfBN : 0;
    const int lo_full =
        window > 0 ? (max(0, min(rw0 + 31, max(row_hi - 1, rw0)) + off - window + 1) + kPfBN - 1) / kPfBN : 0;
    const int my_row = rw0 + ln;
    const int my_lim = my_row + off;  // last visible key of this lane's row
    const int my_lo = window > 0 ? my_row + off - window + 1 : -0x7FFFFFFF;  // first visible key

    const uint16_t *qh = q + ((size_t)b * Hq + h) * (size_t)Tq * D;
    const uint16_t *kh = k + ((size_t)b * Hkv + g) * (size_t)s_cap * D;
    const uint16_t *vh = v + ((size_t)b * Hkv + g) * (size_t)s_cap * D;
    // With a 4-bit cache, k and v hold the float16 residual: key position
    // p >= n_q is its row p - n_q.
    const int row_base = Q4 ? q4.n_q : 0;
    // rows at or past Tq (queries) and Tk (keys) read as zeros
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, (size_t)Tq * D * 2);
    const BufDesc dk = buf_desc(kh, (size_t)(Tk - row_base) * D * 2);
    const BufDesc dv = buf_desc(vh, (size_t)(Tk - row_base) * D * 2);

    // Q rows of this wave as MFMA B operands: lane (row ln, group lg) holds
    // dims [16*kb + 8*lg, +8) of its row.
    vec qreg[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
        qreg[kb] = as_vec<vec>(__builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, ((rw0 + ln) * D + kb * 16 + lg * 8) * 2, 0, 0)));

    // ---- tile loads: HBM -> LDS, IPW loads of 1 KB per wave and step ----
    // Load i of a tile covers rows [i*RPI, i*RPI + RPI); lane l writes the
    // 16 bytes at LDS position (row i*RPI + l/CPR, slot l%CPR), which hold
    // the row's chunk slot ^ swz(row & 7).  The 4 waves share the K and V
    // loads of one tile.
    const bool loads_v = rw * IPW >= IPT;  // this wave's share of a step's loads: all K or all V
    int dma_voff[IPW];                     // lane part of each load's byte offset
    unsigned dma_lds[IPW];                 // LDS destination of each load in buffer 0
#pragma unroll
    for (int ii = 0; ii < IPW; ++ii) {
        const int i = rw * IPW + ii;  // 0 .. 2*IPT-1: K loads, then V loads
        const int row_first = (loads_v ? i - IPT : i) * RPI;
        const int row = row_first + lane / CPR;
        const int cslot = (lane % CPR) ^ swz(row & 7);
        dma_voff[ii] = (row * D + cslot * 8) * 2;
        dma_lds[ii] = (unsigned)(uintptr_t)(lds_void_t *)(smem + (loads_v ? 2 : 0) * L::TILE +
                                                          (row_first >> 3) * L::GROUP + (row_first & 7) * L::ROW);
    }
    auto issue_dma = [&](int kt, int buf) {
        const int toff = (kt * kPfBN - row_base) * D * 2;
#pragma unroll
        for (int ii = 0; ii < IPW; ++ii)
            lds_load16(loads_v ? dv : dk, dma_lds[ii] + buf * L::TILE, dma_voff[ii] + toff);
    };

    // ---- 4-bit tiles: HBM -> registers -> dequantized f16 in LDS ----
    // Tiles below n_q (a multiple of the tile) are 4-bit.  Their codes,
    // scales and biases are loaded into registers when the tile's loads are
    // issued, and dequantized (s * c + b in fp32, one rounding, then to f16)
    // into the tile buffer at the end of the step, in the layout the DMA
    // path writes.  Thread t handles 8-element chunks t + 256 i of the tile
    // (16 consecutive threads cover one row's codes, coalesced).
    constexpr int QCPT = Q4 ? D / 32 : 1;  // chunks per thread and tile (K or V)
    constexpr int QLPR = D / 8;            // chunks per row
    const int q4_ng = Q4 ? D / q4.group : 1;
    const int q4_gshift = Q4 ? __builtin_ctz((unsigned)q4.group / 8u) : 0;  // chunk -> group
    // (without a 4-bit cache these resources are empty and never used)
    const size_t q4_head = Q4 ? ((size_t)b * Hkv + g) * (size_t)q4.s_cap : 0;
    const size_t q4_nq = Q4 ? (size_t)q4.n_q : 0;
    auto q4_rsrc = [&](const void *base, size_t per_row) {
        return Q4 ? make_rsrc((const char *)base + q4_head * per_row, q4_nq * per_row) : make_rsrc(kh, 0);
    };
    const __amdgpu_buffer_rsrc_t rkc = q4_rsrc(q4.k_codes, D / 2), rvc = q4_rsrc(q4.v_codes, D / 2);
    const __amdgpu_buffer_rsrc_t rks = q4_rsrc(q4.k_scales, q4_ng * 2), rkb = q4_rsrc(q4.k_biases, q4_ng * 2);
    const __amdgpu_buffer_rsrc_t rvs = q4_rsrc(q4.v_scales, q4_ng * 2), rvb = q4_rsrc(q4.v_biases, q4_ng * 2);
    // (scales and biases stay in registers of their own: combining them
    // at issue would wait for the loads there)
    uint32_t qk_w[QCPT], qv_w[QCPT];
    uint32_t qk_s[QCPT], qk_b[QCPT], qv_s[QCPT], qv_b[QCPT];
    bool q4_pending = false;
    auto issue_q4 = [&](int kt) {
#pragma unroll
        for (int i = 0; i < QCPT; ++i) {
            const int c = tid + 256 * i;
            const int row = kt * kPfBN + c / QLPR, cc = c % QLPR;
            const int coff = row * (D / 2) + cc * 4;
            const int soff = (row * q4_ng + (cc >> q4_gshift)) * 2;
            qk_w[i] = __builtin_amdgcn_raw_buffer_load_b32(rkc, coff, 0, 0);
            qv_w[i] = __builtin_amdgcn_raw_buffer_load_b32(rvc, coff, 0, 0);
            qk_s[i] = __builtin_amdgcn_raw_buffer_load_b16(rks, soff, 0, 0);
            qk_b[i] = __builtin_amdgcn_raw_buffer_load_b16(rkb, soff, 0, 0);
            qv_s[i] = __builtin_amdgcn_raw_buffer_load_b16(rvs, soff, 0, 0);
            qv_b[i] = __builtin_amdgcn_raw_buffer_load_b16(rvb, soff, 0, 0);
        }
    };
    auto commit_q4 = [&](int buf) {
#pragma unroll
        for (int i = 0; i < QCPT; ++i) {
            const int c = tid + 256 * i;
            const int row = c / QLPR, cc = c % QLPR;
#pragma unroll
            for (int which = 0; which < 2; ++which) {
                const uint32_t w = which ? qv_w[i] : qk_w[i];
                const float sc = f16_bits_to_f32(which ? qv_s[i] : qk_s[i]);
                const float bi = f16_bits_to_f32(which ? qv_b[i] : qk_b[i]);
                // even nibbles to the bytes of lo, odd ones to those of hi:
                // each code then converts with one byte-to-float instruction
                // (the masks are opaque to the compiler, which would
                // otherwise fold them back into one bit-field extract per
                // code)
                uint32_t lo, hi;
                asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(lo) : "v"(w));
                asm("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(hi) : "v"(w >> 4));
                f32x8_t x;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = __builtin_fmaf(sc, (float)((((e & 1) ? hi : lo) >> (8 * (e >> 1))) & 0xFFu), bi);
                *(uint4 *)(smem + (2 * which + buf) * L::TILE + tile_off<D>(row, cc)) = MfmaOps<f16_t>::pack8(x);
            }
        }
    };
    auto issue_tile_loads = [&](int kt, int buf) {
        if constexpr (Q4) {
            if (kt * kPfBN < row_base) {
                issue_q4(kt);
                q4_pending = true;
                return;
            }
        }
        issue_dma(kt, buf);
    };
    // end of a step: a 4-bit tile whose loads were issued goes into buffer buf
    auto finish_tile_loads = [&](int buf) {
        if constexpr (Q4) {
            if (q4_pending) {
                commit_q4(buf);
                q4_pending = false;
            }
        }
        (void)buf;
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] = 0.0f;
    float m_run = -kInf;  // running max of the oriented raw scores of this lane's row
    float l_part = 0.0f;
    const float aq = fabsf(qscale);
    const float thr = fminf(8.0f / aq, 3.0e38f);  // lazy-rescale threshold, raw units (qscale != 0)

    // Lane-dependent LDS byte offsets of the fragments within a tile; the
    // rest of each address (buffer, sub-tile, row group) is a constant the
    // reads take as an immediate offset.
    //   K, row u*32 + ln, chunk 2kb + lg:  tile_off(ln, 2kb + lg) + u*4*GROUP
    //   V, rows 16t + 8h + 4lg + j/4:     voff[db] + (2t + h)*GROUP
    int koff[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) koff[kb] = tile_off<D>(ln, 2 * kb + lg);
    int voff[NDB];
    {
        const int gam = lane >> 4, j = lane & 15;
        const int row0 = 4 * lg + (j >> 2);  // < 8: rows 16t + 8h + row0 share its swizzle
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            voff[db] = tile_off<D>(row0, 4 * db + 2 * (gam & 1) + ((j & 3) >> 1)) + (j & 1) * 8;
    }
    // K fragment (A operand of S^T): key row u*32 + ln, dims kb*16 + lg*8 .. +8
    auto k_frag = [&](const unsigned char *Kt, int u, int kb) {
        return *(const uint4 *)(Kt + koff[kb] + u * 4 * L::GROUP);
    };
    // V^T fragment (A operand of O^T += V^T P^T) for k-block t, d-block db.
    // The operand's slots 0..3 are keys 16t + 4lg + 0..3 and slots 4..7 keys
    // 16t + 8 + 4lg + 0..3 of column d = 32db + (lane % 32), matching the
    // order in which P sits in the score accumulator.  A transposing read
    // gives output lane i (of 16) element i%4 of the 8 bytes named by source
    // lane 4k + i/4 as its slot k, so source lane j names row
    // 16t + 8h + 4lg + j/4 (h: which half of the slots) at column
    // 32db + 16*((lane/16)%2) + 4*(j%4).
    auto v_frag = [&](const unsigned char *Vt, int t, int db) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t *)(Vt + voff[db] + (2 * t) * L::GROUP));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t *)(Vt + voff[db] + (2 * t + 1) * L::GROUP));
        const uint2 a = __builtin_bit_cast(uint2, lo), c = __builtin_bit_cast(uint2, hi);
        return make_uint4(a.x, a.y, c.x, c.y);
    };

    // One tile of the wave's 32 rows from buffer buf: S^T = K Q^T, mask (tiles
    // crossing the diagonal), online softmax, O^T += V^T P^T.  Fragments are
    // read from LDS as they are needed; the waves of the other workgroups on
    // the CU (four workgroups per CU for D = 64) hide the latency.
    // S^T of tile kt from K buffer Kt, masked where the tile crosses the
    // diagonal.
    auto scores = [&](const unsigned char *Kt, int kt, f32x16_t (&st)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int j = 0; j < 16; ++j) st[u][j] = 0.0f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) st[u] = Ops::mfma(as_vec<vec>(k_frag(Kt, u, kb)), qreg[kb], st[u]);
        }
        if (kt >= n_full || kt < lo_full) {
            // (kept a real branch: the empty asm stops the compiler from
            // turning the mask into selects executed on every tile)
            asm volatile("");
            const int key0 = kt * kPfBN + 4 * lg;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = key0 + 32 * u + 8 * (j >> 2) + (j & 3);
                    if (key > my_lim || key < my_lo) st[u][j] = NEG ? kInf : -kInf;
                }
        }
    };
    // Probabilities exp2(s*qs + mq), rounded to 16 bits in four 16-key
    // blocks (one vector conversion each), and this lane's sum of the
    // rounded values (independent partial sums).
    auto probs = [&](f32x16_t (&st)[2], float mq, uint4 (&pb)[4]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) st[u][j] = fast_exp2(__builtin_fmaf(st[u][j], qscale, mq));
        float lsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x8_t x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = st[t >> 1][8 * (t & 1) + i];
            pb[t] = Ops::pack8(x);
            lsum[0] = Ops::sum2(pb[t].x, lsum[0]);
            lsum[1] = Ops::sum2(pb[t].y, lsum[1]);
            lsum[2] = Ops::sum2(pb[t].z, lsum[2]);
            lsum[3] = Ops::sum2(pb[t].w, lsum[3]);
        }
        return (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };
    // One tile of the wave's 32 rows from buffer buf.  Once every row has a
    // reference maximum, the probabilities are taken against it directly,
    // without the tile's maximum: the lane's sum of them bounds each one, so
    // a sum at most kPfSumLimit proves none exceeds it.  Otherwise (the
    // first tile, or scores that outgrew the reference) the tile's scores are
    // formed again from LDS and go through the exact path: maximum, lazy
    // rescale, probabilities.  P V is issued after the test.
    auto tile_step = [&](int kt, int buf) {
        const unsigned char *Kt = smem + buf * L::TILE;
        const unsigned char *Vt = smem + (2 + buf) * L::TILE;
        f32x16_t st[2];
        scores(Kt, kt, st);
        uint4 pb[4];
        float lt = 0.0f;
        bool exact = __any(m_run == -kInf);
        if (!exact) {
            lt = probs(st, -aq * m_run, pb);
            exact = __any(lt > kPfSumLimit);
            if (exact) scores(Kt, kt, st);
        }
        if (exact) {
            const float mq = softmax_max<NEG>(st, acc, m_run, l_part, qscale, thr);
            lt = probs(st, mq, pb);
        }
        l_part += lt;
        // O^T += V^T P^T in four 16-key k-blocks
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = Ops::mfma(as_vec<vec>(v_frag(Vt, t, db)), as_vec<vec>(pb[t]), acc[db]);
    };

    // Step s: the loads of tile t+1 go to the buffer that step s-1 read
    // (every wave has passed the barrier that ended step s-1); tile t is
    // computed from the other buffer; the step ends by waiting for its own
    // loads and a barrier.
    if (n > 0) issue_tile_loads(t_begin, 0);
    finish_tile_loads(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int s = 0; s < n; s += 2) {  // unrolled by two: buffer indices are constants
        issue_tile_loads(t_begin + s + 1, 1);
        if (t_begin + s < w_end && t_begin + s >= w_begin) tile_step(t_begin + s, 0);
        finish_tile_loads(1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (s + 1 < n) {
            issue_tile_loads(t_begin + s + 2, 0);
            if (t_begin + s + 1 < w_end && t_begin + s + 1 >= w_begin) tile_step(t_begin + s + 1, 1);
            finish_tile_loads(0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // ---- key chunks of a long row block: merge through the workspace ----
    // Every chunk stores its partial with device-scope stores, waits for
    // them, and takes a ticket; the chunk that arrives last merges all of
    // them in chunk order (so the result does not depend on timing), writes
    // the output and returns the counter to zero.  Partial words are written
    // with their lowest bit clear (at most one unit in the last place), so
    // what they leave behind never looks like a published decode word.  Counters sit in the
    // workspace's flag region, partials after it, both indexed by the split
    // row block (nc > 1 exactly for row blocks rb0 and later: the tile count
    // grows with the row block).
    if (nc > 1) {
        const size_t split_rb = ((size_t)b * Hq + h) * (n_rb - items.rb0) + (rb - items.rb0);
        unsigned *counter = (unsigned *)ws + split_rb;
        unsigned char *slots = ws + kWsFlagBytes + split_rb * items.max_nc * SL::BYTES;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(slots, (size_t)nc * SL::BYTES);
        typedef __attribute__((ext_vector_type(4))) unsigned u4;
        typedef __attribute__((ext_vector_type(2))) unsigned u2;
        auto o_off = [&](int c, int db, int qd) { return c * SL::BYTES + (((rw * NDB + db) * 4 + qd) * 64 + lane) * 16; };
        auto ml_off = [&](int c) { return c * SL::BYTES + (SL::O_FLOATS + (rw * 64 + lane) * 2) * 4; };
        const unsigned clr = ~1u;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u4, make_float4(acc[db][4 * qd], acc[db][4 * qd + 1], acc[db][4 * qd + 2],
                                                       acc[db][4 * qd + 3])) & clr,
                    rs, o_off(chunk, db, qd), 0, kSC1);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, make_float2(m_run, l_part)) & clr, rs,
                                              ml_off(chunk), 0, kSC1);
        __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
        __syncthreads();                // ... and so have every other thread's
        __shared__ int s_last;
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == (unsigned)(nc - 1);
        __syncthreads();
        if (!s_last) return;
        // Combine the chunks in chunk order with a running maximum.  This
        // workgroup's own partial is not re-read from the workspace: it is
        // parked in the (now idle) tile buffers exactly as it was stored
        // (lowest bits clear), so the result does not depend on which chunk
        // merges, and folded from there in its turn; the others are loaded
        // two per round trip.  Each lane parks and reads back only its own
        // words ([wave][d-block][register][lane]; 4 KB per d-block and wave).
        static_assert(4 * NDB * 16 * 64 * 4 <= L::TOTAL, "own partial fits the tile buffers");
        float *own_lds = (float *)smem + (rw * NDB * 16) * 64 + lane;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                own_lds[(db * 16 + j) * 64] = __uint_as_float(__float_as_uint(acc[db][j]) & clr);
        asm volatile("" ::: "memory");  // read them back from LDS, not kept live in registers
        const float own_m = __uint_as_float(__float_as_uint(m_run) & clr);
        const float own_l = __uint_as_float(__float_as_uint(l_part) & clr);
        float M = -kInf, Lsum = 0.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[db][j] = 0.0f;
        auto load_part = [&](int c, float &mc, float &lc, f32x16_t (&oc)[NDB]) {
            const float2 ml = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs, ml_off(c), 0, kSC1));
            mc = ml.x;
            lc = ml.y;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const float4 x =
                        __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, o_off(c, db, qd), 0, kSC1));
                    oc[db][4 * qd] = x.x; oc[db][4 * qd + 1] = x.y; oc[db][4 * qd + 2] = x.z; oc[db][4 * qd + 3] = x.w;
                }
        };
        auto fold = [&](float mc, float lc, const f32x16_t (&oc)[NDB]) {
            const float Mn = fmaxf(M, mc);
            const float wa = M == -kInf ? 0.0f : fast_exp2(aq * (M - Mn));
            const float wb = mc == -kInf ? 0.0f : fast_exp2(aq * (mc - Mn));
            M = Mn;
            // one rounded product and one fused multiply-add, spelled out, so
            // that every call site rounds alike (which site folds a chunk
            // depends on which chunk merges)
            Lsum = __builtin_fmaf(lc, wb, __fmul_rn(Lsum, wa));
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[db][j] = __builtin_fmaf(oc[db][j], wb, __fmul_rn(acc[db][j], wa));
        };
        auto fold_own = [&]() {
            f32x16_t oc[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) oc[db][j] = own_lds[(db * 16 + j) * 64];
            fold(own_m, own_l, oc);
            asm volatile("" ::: "memory");
        };
        // the i-th other chunk is i below this one's index, i + 1 from it on
        bool own_done = false;
        for (int i = 0; i < nc - 1; i += 2) {
            const int c0 = i < chunk ? i : i + 1;
            const int c1 = i + 1 < chunk ? i + 1 : i + 2;
            const bool two = i + 1 < nc - 1;
            if (!own_done && chunk < c0) {  // before the loads: fewer registers live
                fold_own();
                own_done = true;
            }
            float m0, l0, m1 = -kInf, l1 = 0.0f;
            f32x16_t o0[NDB], o1[NDB];
            load_part(c0, m0, l0, o0);
            if (two) load_part(c1, m1, l1, o1);
            fold(m0, l0, o0);
            if (two) {
                if (!own_done && chunk < c1) {
                    fold_own();
                    own_done = true;
                }
                fold(m1, l1, o1);
            }
        }
        if (!own_done) fold_own();
        m_run = M;
        l_part = Lsum;
        if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }

    // ---- normalise and store: lane holds O^T[d][row] for d = 32db + 8i + 4lg + r ----
    // A sink logit joins the normaliser: relative to the row's reference
    // exponent it is e = sink * log2(e) - |qs| * m_run (log2 units); when
    // e > 0 both the sum and the output are scaled by 2^-e first.
    const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
    if (my_row < Tq) {
        float inv = 1.0f / l_tot;
        if (sinks) {
            const float e = sinks[h] * 1.4426950408889634f - aq * m_run;
            const float mx = fmaxf(e, 0.0f);
            const float down = fast_exp2(-mx);
            inv = down / __builtin_fmaf(l_tot, down, fast_exp2(e - mx));
        }
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

// ---- work decomposition (host) ----
// Key tiles of row block rb (the keys its valid rows can see; with a
// window, from the first row's first visible key on).
static int pf_row_tiles(int rb, int Tq, int Tk, int window)
{
    const int row_hi = std::min((rb + 1) * kPfBM, Tq);
    const int t_lo = window > 0 ? std::max(0, rb * kPfBM + Tk - Tq - window + 1) / kPfBN : 0;
    return (std::min(Tk, row_hi + Tk - Tq) + kPfBN - 1) / kPfBN - t_lo;
}

// Chunking of the causal triangle.  The most key tiles per chunk, ch, is
// the smallest value that gives about one slot's share of the tiles per
// chunk (3 shares per CU for D = 64, 2 for D = 128; the items,
// issued longest first, then finish close together), but at least
// kPfMinChunk tiles and a 1/kPfMaxSplit share of the longest row block,
// with the launch table's item count, the chunks per row
// block and the split row blocks' counters within their limits.  Every
// limit is monotone in ch and met once no row block is split.
struct PfPlan {
    int n_rb, ch, rb0, max_nc, n_items;
};

static PfPlan pf_plan_for(int Tq, int Tk, int window, int ch)
{
    PfPlan p;
    p.n_rb = (Tq + kPfBM - 1) / kPfBM;
    p.ch = ch;
    p.rb0 = p.n_rb;
    p.max_nc = 1;
    p.n_items = 0;
    for (int rb = p.n_rb - 1; rb >= 0; --rb) {
        const int nc = (pf_row_tiles(rb, Tq, Tk, window) + ch - 1) / ch;
        if (nc > 1) p.rb0 = rb;
        p.max_nc = std::max(p.max_nc, nc);
        p.n_items += nc;
    }
    return p;
}

static bool pf_plan_fits(const PfPlan &p, int B, int Hq)
{
    return p.n_items <= kPfMaxItems && p.max_nc <= 63 &&
           (size_t)B * Hq * (p.n_rb - p.rb0) * 4 <= kWsFlagBytes - kWsTailBytes;
}

// n_cus: compute units of the device the launch runs on.
static PfPlan pf_plan(int B, int Hq, int D, int Tq, int Tk, int window, int n_cus)
{
    // Shares of 3 workgroups per CU for D = 64, although 4 are resident:
    // longer chunks and fewer merges measured 0.8 us faster at T = 4097
    // (0.5B geometry), the same at T = 2049 and for a 256-query chunk.
    const long slots = (long)(D == 64 ? 3 : 2) * n_cus;
    const int n_rb = (Tq + kPfBM - 1) / kPfBM;
    long total = 0;
    int max_nt = 0;
    for (int rb = 0; rb < n_rb; ++rb) {
        const int nt = pf_row_tiles(rb, Tq, Tk, window);
        total += nt;
        max_nt = std::max(max_nt, nt);
    }
    total *= (long)B * Hq;
    // The floor: short prompts split into short chunks (T = 513, 0.5B
    // geometry: 154 workgroups of at most 3 tiles instead of 70 whole row
    // blocks, 10.7 us against 11.6), but no row block into more than
    // kPfMaxSplit chunks (without that cap, a 256-query chunk's 65-tile rows
    // split 22 ways and took 28.5 us against 18.7).
    const long min_chunk = std::max<long>(kPfMinChunk, (max_nt + kPfMaxSplit - 1) / kPfMaxSplit);
    int lo = (int)std::min<long>(std::max(min_chunk, (total + slots - 1) / std::max(slots, 1L)), 1 << 30);
    int hi = std::max(lo, max_nt);  // no split: always fits
    if (pf_plan_fits(pf_plan_for(Tq, Tk, window, lo), B, Hq)) return pf_plan_for(Tq, Tk, window, lo);
    while (hi - lo > 1) {  // invariant: lo does not fit, hi does
        const int mid = lo + (hi - lo) / 2;
        if (pf_plan_fits(pf_plan_for(Tq, Tk, window, mid), B, Hq)) hi = mid; else lo = mid;
    }
    return pf_plan_for(Tq, Tk, window, hi);
}

// The (row block, chunk) items sorted longest first (ties: longer row block
// first, so that the chunks that merge run early), as the launch table.
static void pf_items(const PfPlan &p, int Tq, int Tk, int window, PfItems *it)
{
    std::vector<std::pair<int, int>> v;  // (sort key, entry)
    for (int rb = 0; rb < p.n_rb; ++rb) {
        const int nt = pf_row_tiles(rb, Tq, Tk, window);
        const int nc = (nt + p.ch - 1) / p.ch, per = (nt + nc - 1) / nc;
        for (int c = 0; c < nc; ++c) {
            const int t0 = std::min(nt, c * per), len = std::min(nt, t0 + per) - t0;
            v.push_back({-(len * 1048576 + nt * 64 + (63 - c)), (rb << 6) | c});
        }
    }
    std::sort(v.begin(), v.end());
    it->n = (int)v.size();
    it->ch = p.ch;
    it->rb0 = p.rb0;
    it->max_nc = p.max_nc;
    for (int i = 0; i < it->n; ++i) it->e[i] = (unsigned short)v[i].second;
}

// Flag region, then one partial slot per chunk of every split row block.
size_t prefill_workspace_bytes(int B, int Hq, int D, int Tq, int Tk, int window, int n_cus)
{
    const PfPlan p = pf_plan(B, Hq, D, Tq, Tk, window, n_cus);
    const size_t slot = D == 64 ? PfSlot<64>::BYTES : PfSlot<128>::BYTES;
    const size_t split_cols = (size_t)B * Hq * (p.n_rb - p.rb0);
    return kWsFlagBytes + (p.max_nc > 1 ? split_cols * p.max_nc * slot : 0);
}

template <typename T, int D, bool Q4 = false>
static hipError_t launch_pf(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv,
                            int Tq, int Tk, int s_cap, float scale, void *ws, int window, const float *sinks,
                            int n_cus, hipStream_t s, Q4Source src = Q4Source{})
{
    const PfPlan plan = pf_plan(B, Hq, D, Tq, Tk, window, n_cus);
    PfItems items;
    pf_items(plan, Tq, Tk, window, &items);
    // A zero scale (uniform weights over the visible keys) is run as the
    // smallest normal scale: every exponent is then below 2^-80 in
    // magnitude, exp2 of it rounds to exactly 1, and masked keys (-inf)
    // still give 0 rather than inf*0.
    float qscale = scale * 1.4426950408889634f;
    if (qscale == 0.0f) qscale = 1.17549435e-38f;
    dim3 grid((unsigned)(items.n * B * Hq));
    if (qscale < 0.0f)
        hipLaunchKernelGGL((prefill_causal_kernel<T, D, true, Q4>), grid, dim3(kPfThreads), 0, s,
                           (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)out, Hq, Hkv,
                           Tq, Tk, s_cap, qscale, plan.n_rb, (unsigned char *)ws, B, window, sinks, items, src);
    else
        hipLaunchKernelGGL((prefill_causal_kernel<T, D, false, Q4>), grid, dim3(kPfThreads), 0, s,
                           (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)out, Hq, Hkv,
                           Tq, Tk, s_cap, qscale, plan.n_rb, (unsigned char *)ws, B, window, sinks, items, src);
    return hipGetLastError();
}

hipError_t launch_prefill(int dtype, int D, const void *q, const void *k, const void *v, void *out, int B,
                          int Hq, int Hkv, int Tq, int Tk, int s_cap, float scale, void *ws, int window,
                          const float *sinks, int n_cus, hipStream_t s)
{
#define GQA_PF(T, DD) launch_pf<T, DD>(q, k, v, out, B, Hq, Hkv, Tq, Tk, s_cap, scale, ws, window, sinks, n_cus, s)
    if (dtype == 1) {
        if (D == 64) return GQA_PF(bf16_t, 64);
        if (D == 128) return GQA_PF(bf16_t, 128);
    } else if (dtype == 2) {
        if (D == 64) return GQA_PF(f16_t, 64);
        if (D == 128) return GQA_PF(f16_t, 128);
    }
#undef GQA_PF
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_q4r(int D, const void *q, const void *k_res, const void *v_res, void *out, int B, int Hq,
                              int Hkv, int Tq, int Tk, int R, float scale, void *ws, const Q4Source &src, int n_cus,
                              hipStream_t s)
{
    if (D == 64)
        return launch_pf<f16_t, 64, true>(q, k_res, v_res, out, B, Hq, Hkv, Tq, Tk, R, scale, ws, 0, nullptr, n_cus, s,
                                          src);
    if (D == 128)
        return launch_pf<f16_t, 128, true>(q, k_res, v_res, out, B, Hq, Hkv, Tq, Tk, R, scale, ws, 0, nullptr, n_cus,
                                           s, src);
    return hipErrorInvalidValue;
}

}  // namespace gqa

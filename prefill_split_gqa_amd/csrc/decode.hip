// decode.hip -- split-K single-token grouped-query attention for gfx950.
//
// Every decode launch splits the KV length of each (request, KV head) into
// splits of L rows; one workgroup handles one split for GT of the query
// heads that share the KV head ("Why It Matters: 7x KV Expansion" on the
// Candle decode page: the fused kernel reads each KV head once through a GQA
// stride; here the heads of a group share the load).  Each split publishes
// one (max, sum, output) partial per query head, and the partials are merged
// in the same launch (below).
//
// Dense caches (fp32, bf16, f16) run on the matrix cores: decode_mfma_kernel,
// 4 waves, each taking 16-row blocks of the split (its comment has the
// operand layouts).
//
// The float16 residual rows of a residual-window 4-bit cache are one split of
// the 4-bit kernel's launch, streamed on the SIMD lanes (dense_split, 8
// waves): each key row is read by a 32-lane row-group with 16-byte (or
// 8-byte) coalesced loads; a wave reads 2 rows per load instruction and the
// workgroup 16 rows per step.  Each lane owns D/32 elements of the row; a
// dot product is finished with four DPP steps inside a 16-lane row and one
// gfx950 row swap (v_permlane16_swap).  Each row-group keeps its own
// online-softmax state in registers; the two row-groups of a wave are merged
// with the gfx950 cross-half lane swap (v_permlane32_swap), the eight waves
// through LDS.
//
// In both, the reference maximum of the online softmax is only raised when a
// score exceeds it by more than 2^8 (log2 domain), so the rescale of the
// output registers is rare and the result is exact up to rounding; the query
// rows are staged in LDS once per workgroup; K and V are read through buffer
// resources bounded to the split, so a row past its end reads as zeros and
// loads are issued unconditionally.
//
// Cross-split merge: one CU can pull only ~70 GB/s, so a single workgroup
// reading every split's partial would be the tail of the launch.  Instead
// each (request, query head) is merged by a whole workgroup that waits until
// every split of its (request, head tile) has published its partial for that
// head, reads only that head's slice and merges it with the log-sum-exp rule
// in a fixed order (results do not depend on timing).  The designated merger
// of query head hh is split hh mod n_split when the whole grid can be
// resident (it merges right after publishing its own partial), otherwise a
// merge workgroup placed after every split in the grid.  A split publishes
// its outputs and its (max, sum) pair with one store each and no wait: every
// fp32 word is written with its lowest mantissa bit set, so in the
// zero-filled workspace a word with that bit set has been published.  The
// merge polls the words it needs (one round trip once they have landed) and
// zeroes them after reading, leaving the workspace ready for the next call.
//
// Waiting without co-residency.  A workgroup may wait without bound for
// other workgroups only once it has proof that all of them have started: a
// started split is resident (or done) and never waits before publishing, so
// its partial always lands, whatever else shares the device (other kernels,
// other streams, a CU mask).  The splits count themselves in groups of
// kSplitGroup, one word per group (an atomic add first thing); the split
// that completes its group adds one to the (request, head tile)'s tile word:
//   bits 0..3   groups whose splits have all started;
//   bits 4..7   heads whose designated merger has decided;
//   bits 8+hh   set by head hh's designated merger when it decides.
// A designated merger decides with exactly one add, (1 << 4) | (1 << (8 +
// hh)) (a split merging in place makes it once its streaming is done -- the
// matrix-core kernel once its partial is published -- for all of its heads
// at once): if the add finds every group counted, it has
// its proof and merges; otherwise it leaves the head, and the split that
// completed the last group -- whose add comes after in the word's order, and
// so finds the head's bit set -- merges it after its own split, with proof.
// The adds to one word are totally ordered, so each head is merged exactly
// once and no workgroup waits without proof.  Every group and every head
// adds exactly once, so the add that leaves the word at its final value
// (all groups, all heads, every bit) returns it to zero; each group
// completer zeroes its group word.  The waits are still bounded: a merge
// that gives up (not reachable by the argument above) writes NaN and sets
// the workspace's poison word, and every later merge on that workspace
// writes NaN instead of trusting stale words, until the workspace is
// zero-filled again.

// Cross-workgroup exchange without cache maintenance: on gfx950 each XCD has
// its own L2, and a device-scope fence writes back / invalidates that L2
// (tens of microseconds across a full launch).  Instead, every value that
// crosses workgroups is written and read with device-scope (sc1) accesses,
// which are coherent at device scope by themselves; each 32-bit word is
// written whole, and the merge accepts a word only once its tag bit is set.
//
// The 4-bit cache variant (VeloxQuant-MLX "attention" posts, Part 4: codes,
// scales, biases and the group size go to the kernel, which dequantizes
// inside it) has a kernel of its own on the matrix cores (below); the split
// plan, the partials and the merge are shared.  With a float16 residual
// window (the same posts, "What this means in practice": recent tokens kept
// unquantized), the residual rows of each (request, head tile) are one more
// split of that launch, streamed by the dense path (dense_split) and merged
// with the 4-bit splits.
//
// Sliding window and sinks (the Fornace prefill page, "What this does not
// prove", and the SDPA signature in the VeloxQuant posts, Part 4): a window
// moves each request's first visible row (the splits cover only the window),
// and a sink logit joins the normaliser where the partials are combined.

#include "common.h"

#include <type_traits>

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

// K/V rows are read with buffer loads whose resource covers exactly the
// rows [0, end) of this (request, KV head): a row past the split's end reads
// as zeros without a branch (and without a memory access), so every load of a
// chunk is issued unconditionally.

// Dense K/V rows of D elements of type T.
template <typename T, int D>
struct DenseKV {
    static constexpr int EPL = D / kDecodeLPR;                    // elements per lane
    static constexpr int BPL = D * (int)sizeof(T) / kDecodeLPR;   // bytes per lane
    static constexpr int U = BPL >= 16 ? 16 : BPL;                // bytes per load
    static constexpr int NU = BPL / U;                            // loads per lane per row
    static constexpr int EU = U / (int)sizeof(T);                 // elements per load
    static constexpr int WPU = U / 4;                             // words per load
    static constexpr int ROW = D * (int)sizeof(T);                // bytes per row
    struct Raw { uint32_t w[NU * WPU]; };

    __device__ __forceinline__ static int dim(int lr, int e) { return ((e / EU) * kDecodeLPR + lr) * EU + (e % EU); }

    struct Src {
        __amdgpu_buffer_rsrc_t rs;  // rows [0, end) of this (request, KV head)
    };
    __device__ __forceinline__ static Src make_src(const void *base, size_t head_row0, int end)
    {
        return Src{make_rsrc((const T *)base + head_row0 * D, (size_t)end * ROW)};
    }

    __device__ __forceinline__ static void load(Raw &r, const Src &s, int row, int lr)
    {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int off = row * ROW + (j * kDecodeLPR + lr) * U;
            if constexpr (U == 16) {
                auto x = __builtin_amdgcn_raw_buffer_load_b128(s.rs, off, 0, 0);
                r.w[j * 4 + 0] = x[0]; r.w[j * 4 + 1] = x[1]; r.w[j * 4 + 2] = x[2]; r.w[j * 4 + 3] = x[3];
            } else if constexpr (U == 8) {
                auto x = __builtin_amdgcn_raw_buffer_load_b64(s.rs, off, 0, 0);
                r.w[j * 2 + 0] = x[0]; r.w[j * 2 + 1] = x[1];
            } else {
                r.w[j] = __builtin_amdgcn_raw_buffer_load_b32(s.rs, off, 0, 0);
            }
        }
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float *x)
    {
        constexpr int PW = Unpack<T>::per_word;
#pragma unroll
        for (int i = 0; i < NU * WPU; ++i) Unpack<T>::run(r.w[i], x + i * PW);
    }
    // a query row has the same element type and lane layout as a K row; the
    // workgroup's query rows are staged in LDS (sq) first
    typedef Raw QRaw;
    __device__ __forceinline__ static void load_q_lds(QRaw &r, const uint32_t *sq, int h, int lr)
    {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const uint32_t *pj = sq + (h * ROW + (j * kDecodeLPR + lr) * U) / 4;
#pragma unroll
            for (int w = 0; w < WPU; ++w) r.w[j * WPU + w] = pj[w];
        }
    }
    __device__ __forceinline__ static void unpack_q(const QRaw &r, float *x) { unpack(r, x); }
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
// max / sum over the 2 row-groups of a wave (lanes l and l^32)
__device__ __forceinline__ float rowgroup_max(float x)
{
    float a, b;
    swap32(x, x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float rowgroup_sum(float x)
{
    float a, b;
    swap32(x, x, a, b);
    return a + b;
}

// max / sum over the 4 lanes l % 16 == j (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float max4q(float x)
{
    float a, b;
    swap16(x, x, a, b);
    x = fmaxf(a, b);
    swap32(x, x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float sum4q(float x)
{
    float a, b;
    swap16(x, x, a, b);
    x = a + b;
    swap32(x, x, a, b);
    return a + b;
}

constexpr unsigned kMergeSpinLimit = 1u << 22;  // polls before a merge workgroup gives up
constexpr unsigned kStartPolls = 256;           // tile word reads of a merge workgroup before it decides

// Kernel launch shape of the decode grid: streaming workgroups first, then
// merge workgroups (one per request and query head).
struct DecodeGrid {
    int gx;        // splits per (request, head tile) in the grid
    int n_stream;  // gx * HT * B splits; merge workgroups (if any) follow
    int inplace;   // 1: the splits merge themselves (no merge workgroups)
    int B;         // requests
};

// Rows of request b that its query sees: its length (device lengths are
// clamped to [0, s_cap]); with a window, only the last `window` of them,
// which start at row *lo.
// The cache a launch reads (a compile-time mode, so that plain launches
// carry none of it): kResNone a plain cache; kResQ4 a 4-bit cache with a
// float16 residual window, whose residual rows are one more split.
enum ResMode { kResNone = 0, kResQ4 = 1 };

// Rows of request b the splits of length L cover (with a residual window:
// its 4-bit rows, whole blocks of the residual's size).
template <int RES>
__device__ __forceinline__ int request_len(const DecodeArgs &a, int b)
{
    int n = a.kv_len;
    if (a.kv_lens) {
        n = a.kv_lens[b];
        n = n < 0 ? 0 : (n > a.s_cap ? a.s_cap : n);
    }
    if constexpr (RES == kResQ4) n -= n % a.res_cap;
    return n;
}

// Float16 residual rows of request b (kResQ4): the rest of its tokens.
__device__ __forceinline__ int residual_rows(const DecodeArgs &a, int b)
{
    int n = a.kv_lens[b];
    n = n < 0 ? 0 : (n > a.s_cap ? a.s_cap : n);
    return n % a.res_cap;
}

// Splits of request b, whose split-covered rows are n: pieces of L rows, and
// with a residual window one more for the residual rows if there are any.
template <int RES>
__device__ __forceinline__ int request_splits(const DecodeArgs &a, int b, int n)
{
    const int ns = (n + a.plan.L - 1) / a.plan.L;
    if constexpr (RES == kResQ4) return ns + (residual_rows(a, b) > 0 ? 1 : 0);
    return ns;
}

__device__ __forceinline__ int windowed(const DecodeArgs &a, int n, int *lo)
{
    *lo = a.window > 0 && n > a.window ? n - a.window : 0;
    return n - *lo;
}

// With per-request lengths and at most kDecodePackMaxB requests, the
// working splits are packed at the front of the grid: request b's
// HT * max(1, n_split(b)) items (head tile major, split minor) follow those
// of requests 0 .. b-1, so no workgroup slot goes to a split past its
// request's length (a request of length 0 keeps one item per head tile,
// which writes its zero output).  Every wave derives the same mapping:
// lane r reads request r's length, the items are prefix-summed across the
// lanes, and a ballot finds the request holding item i.  The split
// boundaries, and so the results, are those of the strided mapping.
constexpr int kDecodePackMaxB = 64;
struct SplitItem {
    int b, ht, s, n;  // request, head tile, split, clamped length
};
template <int RES>
__device__ __forceinline__ bool packed_item(const DecodeArgs &a, int B, int i, SplitItem *it)
{
    const DecodePlan &P = a.plan;
    const int lane = threadIdx.x & 63;
    int n = 0, lo;
    if (lane < B) n = windowed(a, request_len<RES>(a, lane), &lo);
    const int ns = (n + P.L - 1) / P.L;
    const int items = lane < B ? P.HT * (ns > 1 ? ns : 1) : 0;
    int incl = items;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    const int b = __popcll(__ballot(incl <= i));  // requests whose items all precede item i
    if (b >= B) return false;                      // past the working items
    const int start = __shfl(incl - items, b, 64);
    const int nb = __shfl(n, b, 64);
    const int local = i - start;
    const int nsb = (nb + P.L - 1) / P.L > 1 ? (nb + P.L - 1) / P.L : 1;
    it->b = __builtin_amdgcn_readfirstlane(b);
    it->n = __builtin_amdgcn_readfirstlane(nb);
    it->ht = __builtin_amdgcn_readfirstlane(local / nsb);
    it->s = __builtin_amdgcn_readfirstlane(local % nsb);
    return true;
}

template <typename TQ, int D, int GT, int RES, int NT = kDecodeThreads>
__device__ void merge_head(const DecodeArgs &a, int m, int n_split);
template <typename TQ, int D, int GT, int RES, int NT = kDecodeThreads>
__device__ void merge_heads(const DecodeArgs &a, int col, int n_split, unsigned heads);
template <typename TQ, int D, int GT, int RES, int NT = kDecodeThreads>
__device__ void merge_workgroup(const DecodeArgs &a, int m);

// Control words (see the file header): the tile word of (request, head
// tile) col, and the word of its split group g.
constexpr unsigned kTwGroups = 0xFu;    // bits 0..3
constexpr int kTwDecidedShift = 4;      // bits 4..7
constexpr int kTwHeadShift = 8;         // bits 8..15
constexpr unsigned kNoTicket = ~0u;
__device__ __forceinline__ unsigned *tile_word(const DecodeArgs &a, int col)
{
    return a.ctrl + (size_t)col * kCtrlWords * kCtrlStride;
}
__device__ __forceinline__ unsigned *group_word(const DecodeArgs &a, int col, int g)
{
    return tile_word(a, col) + (1 + g) * kCtrlStride;
}
__device__ __forceinline__ unsigned split_groups(int n_split)
{
    return (unsigned)(n_split + kSplitGroup - 1) / kSplitGroup;
}

// First thing a split of a multi-split (request, head tile) does: count
// itself in its group.
__device__ __forceinline__ unsigned group_add(const DecodeArgs &a, int col, int s)
{
    return __hip_atomic_fetch_add(group_word(a, col, s / kSplitGroup), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Given its group add's result t: the split that completed its group zeroes
// the group word and counts the group in the tile word, returning that add's
// result (awaited at the end); kNoTicket for the others.
__device__ __forceinline__ unsigned group_done(const DecodeArgs &a, int col, int s, int n_split, unsigned t)
{
    const int g = s / kSplitGroup;
    const int gs = min(kSplitGroup, n_split - g * kSplitGroup);
    if (t != (unsigned)gs - 1u) return kNoTicket;
    __hip_atomic_store(group_word(a, col, g), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __hip_atomic_fetch_add(tile_word(a, col), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A designated merger's one add for the heads in `heads`; the result shows
// whether every group had started when it landed.
__device__ __forceinline__ unsigned tile_decision_add(unsigned heads)
{
    return ((unsigned)__popc(heads) << kTwDecidedShift) | (heads << kTwHeadShift);
}
__device__ __forceinline__ unsigned decide(const DecodeArgs &a, int col, unsigned heads)
{
    return __hip_atomic_fetch_add(tile_word(a, col), tile_decision_add(heads), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}
// After an add to the tile word that left it at `after`: the last add
// (every group, every head counted) returns it to zero.
template <int GT>
__device__ __forceinline__ void tile_word_last(const DecodeArgs &a, int col, int n_split, unsigned after)
{
    const unsigned all = (1u << GT) - 1u;
    if ((after & 0xFFFFu) == (split_groups(n_split) | ((unsigned)GT << kTwDecidedShift) | (all << kTwHeadShift)))
        __hip_atomic_store(tile_word(a, col), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Heads a split designates itself merger of when the splits merge in place.
template <int GT> __device__ __forceinline__ unsigned inplace_heads(int s, int n_split)
{
    unsigned h = 0u;
    for (int hh = s; hh < GT; hh += n_split) h |= 1u << hh;
    return h;
}

// The heads a split of (request, head tile) col merges once it has published
// (see the file header), from the results of its adds to the tile word
// (thread 0).  ticket_heads: if its group completion (`ticket`; kNoTicket
// if it completed no group) counted the last group, the heads whose
// designated mergers decided before that.  decided_heads: the heads it is
// the designated merger of (own_heads, in place), if its decision add
// (result `decision`) found every group counted.
template <int GT>
__device__ __forceinline__ unsigned ticket_heads(const DecodeArgs &a, int col, int n_split, unsigned ticket)
{
    if (ticket == kNoTicket) return 0u;
    const unsigned all = (1u << GT) - 1u;
    const unsigned after = ticket + 1u;
    tile_word_last<GT>(a, col, n_split, after);
    return (after & kTwGroups) == split_groups(n_split) ? (ticket >> kTwHeadShift) & all : 0u;
}
template <int GT>
__device__ __forceinline__ unsigned decided_heads(const DecodeArgs &a, int col, int n_split, unsigned own_heads,
                                                  unsigned decision)
{
    if (own_heads == 0u) return 0u;
    tile_word_last<GT>(a, col, n_split, decision + tile_decision_add(own_heads));
    return (decision & kTwGroups) == split_groups(n_split) ? own_heads : 0u;
}
// Both, for a split that decided when its streaming was done and reads the
// results before its last barrier, ahead of its publish (the SIMD-lane and
// 4-bit kernels: waiting there for the adds' round trips does not also wait
// for the publish stores).
template <int GT>
__device__ __forceinline__ unsigned tile_heads(const DecodeArgs &a, int col, int n_split, unsigned own_heads,
                                               unsigned decision, unsigned ticket)
{
    return ticket_heads<GT>(a, col, n_split, ticket) | decided_heads<GT>(a, col, n_split, own_heads, decision);
}

// The matrix-core kernel's designated merger (own_heads != 0, uniform)
// decides once its partial is published instead: thread 0 adds to the tile
// word after its publish stores, so that the add's round trip delays only
// this workgroup's own merges, never a publish that the tile's other
// mergers wait for (measured: 7B geometry, 4096 rows, 9.02 -> 8.94 us; the
// 4-bit kernel measured 0.3 us slower this way).  Adds the heads kept to
// *s_heads (LDS) and ends with a barrier.
template <int GT>
__device__ __forceinline__ void decide_after_publish(const DecodeArgs &a, int col, int n_split, unsigned own_heads,
                                                     unsigned *s_heads)
{
    if (own_heads == 0u) return;
    if (threadIdx.x == 0) *s_heads |= decided_heads<GT>(a, col, n_split, own_heads, decide(a, col, own_heads));
    __syncthreads();
}

// Published partials carry a tag: every fp32 word is written with its
// lowest mantissa bit set, so a published word can be told from a word of
// the zero-filled workspace without a separate flag, and a publisher never
// waits for its stores.  The tag moves a value by at most one unit in the
// last place; the reference maximum is tagged before the weights relative
// to it are taken, so it costs nothing there.
typedef __attribute__((ext_vector_type(4))) unsigned tag_u4_t;
typedef __attribute__((ext_vector_type(2))) unsigned tag_u2_t;
__device__ __forceinline__ float tagged_f32(float x) { return __uint_as_float(__float_as_uint(x) | 1u); }
__device__ __forceinline__ bool is_tagged4(tag_u4_t w) { return (w[0] & w[1] & w[2] & w[3] & 1u) != 0u; }
__device__ __forceinline__ bool is_tagged2(tag_u2_t w) { return (w[0] & w[1] & 1u) != 0u; }

// End of a streaming workgroup.  so [waves][GT][SOD] (rows of D floats at
// a stride of SOD), sm and sl [waves][GT] hold, per wave and query head, the
// unnormalised output row, its reference maximum (log2 domain; -inf for a
// wave that saw no row) and its sum of weights.  The waves are combined;
// with a single split the output is written, otherwise the split's partial
// is published with tagged device-scope stores (its outputs and its (max,
// sum) pair), with no wait.
// A sink logit (natural units of the scaled scores) in the log2 units of
// the kernels' scores; -inf without sinks.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float sink_log2(const DecodeArgs &a, int h)
{
    return a.sinks ? a.sinks[h] * kLog2e : kNegInf;
}

template <typename TQ, int D, int GT, int RES, int SOD = D, int NT = kDecodeThreads>
__device__ __forceinline__ void finish_split(const DecodeArgs &a, const float *so, const float *sm, const float *sl,
                                             int col, int s, int n_split, TQ *out, int h0)
{
    constexpr int NW = NT / 64;
    constexpr int NQ = GT * D / 4;  // 4-wide output items
    static_assert(NQ <= NT, "one output item per thread");
    const DecodePlan &P = a.plan;
    const int tid = threadIdx.x;
    const int qh = tid / (D / 4), qd = (tid % (D / 4)) * 4;
    float Mw = kNegInf, Lw = 0.0f, O0 = 0.0f, O1 = 0.0f, O2 = 0.0f, O3 = 0.0f;
    if (tid < NQ) {
        // every read first, then the arithmetic
        float mw[NW], lw[NW];
        float4 xw[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = sm[w * GT + qh];
            lw[w] = sl[w * GT + qh];
            xw[w] = *(const float4 *)&so[(w * GT + qh) * SOD + qd];
        }
#pragma unroll
        for (int w = 0; w < NW; ++w) Mw = fmaxf(Mw, mw[w]);
        // a single split normalises here, sink included; several publish
        // their partials and the merge adds the sink
        const float s2 = n_split == 1 ? sink_log2(a, h0 + qh) : kNegInf;
        Mw = fmaxf(Mw, s2);
        if (n_split > 1) Mw = tagged_f32(Mw);  // finite: every split has a row
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float wt = rel_weight(mw[w], Mw);
            Lw += wt * lw[w];
            O0 += wt * xw[w].x; O1 += wt * xw[w].y; O2 += wt * xw[w].z; O3 += wt * xw[w].w;
        }
        Lw += rel_weight(s2, Mw);
    }
    if (n_split == 1) {
        if (tid < NQ) store4(out + (size_t)qh * D + qd, O0 / Lw, O1 / Lw, O2 / Lw, O3 / Lw);
        return;
    }
    const __amdgpu_buffer_rsrc_t ws_o =
        __builtin_amdgcn_make_buffer_rsrc(a.part_o, 0, (int)P.o_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ws_ml =
        __builtin_amdgcn_make_buffer_rsrc(a.part_ml, 0, (int)P.ml_bytes, kRsrcWord3);
    const size_t colbase = (size_t)col * P.n_split_max;
    if (tid < NQ) {
        const int off_o = (int)((((colbase + s) * GT + qh) * D + qd) * 4);
        const tag_u4_t w = {__float_as_uint(O0) | 1u, __float_as_uint(O1) | 1u, __float_as_uint(O2) | 1u,
                            __float_as_uint(O3) | 1u};
        __builtin_amdgcn_raw_buffer_store_b128(w, ws_o, off_o, 0, kSC1);
        if (qd == 0) {
            const int off_ml = (int)(((colbase + s) * GT + qh) * 2 * 4);
            const tag_u2_t wm = {__float_as_uint(Mw), __float_as_uint(Lw) | 1u};
            __builtin_amdgcn_raw_buffer_store_b64(wm, ws_ml, off_ml, 0, kSC1);
        }
    }
}

// One split of a dense KV cache (or of a 4-bit cache's float16 residual):
// rows [start, end) of the KV head whose row 0 is row head_row0 of kbase /
// vbase, for query heads h0 .. h0 + GT - 1 of request b (head tile ht);
// split s of the (request, head tile)'s n_split.  Streams the rows,
// publishes the split's partial and takes part in the merge.
template <class KV, typename TQ, int D, int GT, int RES>
__device__ __forceinline__ void dense_split(const DecodeArgs &a, const DecodeGrid &grid, const void *kbase,
                                            const void *vbase, size_t head_row0, int s, int n_split, int start,
                                            int end, int b, int ht, int h0, TQ *out)
{
    constexpr int EPL = D / kDecodeLPR;
    constexpr int RC = 2;                     // rows per row-group per chunk
    constexpr int CHUNK = RC * kDecodeRowGroups;
    constexpr int NW = kDecodeThreads / 64;   // waves
    constexpr int NF = GT * EPL;              // output registers per lane
    constexpr int NQ = GT * D / 4;            // 4-wide output items
    static_assert(KV::EPL == EPL, "lane layout mismatch");
    static_assert(NF % 2 == 0 && NQ <= kDecodeThreads && kDecodeLPR == 32, "tile shape");

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, rgq = lane >> 5, lr = lane & 31;
    const int rg = wave * 2 + rgq;  // row-group (half wave) within the workgroup
    const DecodePlan &P = a.plan;

    const typename KV::Src src = KV::make_src(kbase, head_row0, end);
    const typename KV::Src srcv = KV::make_src(vbase, head_row0, end);

    typename KV::Raw kr[2][RC], vr[2][RC];
    auto load_chunk = [&](int buf, int c0) {
#pragma unroll
        for (int rr = 0; rr < RC; ++rr) {
            const int row = c0 + rr * kDecodeRowGroups + rg;  // rows >= end read as zero
            KV::load(kr[buf][rr], src, row, lr);
            KV::load(vr[buf][rr], srcv, row, lr);
        }
    };

    // Issue order matters: vector-memory waits are in order, so the queries
    // go first (their wait then does not wait for K/V), then the first two
    // chunks, all before anything is consumed.  The GT query rows are read
    // once per workgroup (16 bytes per thread) and staged in LDS: loading
    // them per wave would push as many bytes through each CU's load path as
    // the K/V split itself.
    constexpr int QB = GT * D * (int)sizeof(TQ);  // bytes of this workgroup's query rows
    __shared__ __attribute__((aligned(16))) uint32_t sq[QB / 4];
    // (every load below is unconditional -- threads past the query block
    // re-read its first 16 bytes, rows past the split read as zero -- so the
    // compiler's in-order wait counts stay exact)
    const bool q_loader = tid < QB / 16;
    const uint4 qv = *((const uint4 *)((const char *)a.q + ((size_t)b * a.Hq + h0) * D * sizeof(TQ)) +
                       (q_loader ? tid : 0));
    // this split counts itself in its group right after the query load
    // (its result is awaited after the queries, before any K/V wait)
    const int col = b * P.HT + ht;
    unsigned gticket = 0u;
    if (n_split > 1 && tid == 0) gticket = group_add(a, col, s);
    asm volatile("" ::: "memory");  // keep the query load ahead of the K/V loads
    load_chunk(0, start);
    load_chunk(1, start + CHUNK);
    if (q_loader) *((uint4 *)sq + tid) = qv;
    __syncthreads();
    unsigned ticket = kNoTicket;  // a group completer's tile word add (awaited at the end)
    if (n_split > 1 && tid == 0) ticket = group_done(a, col, s, n_split, gticket);

    // Queries of the GT heads, pre-multiplied by scale*log2(e) (every LDS
    // read issued before the first is used).
    float qf[GT][EPL];
    {
        typename KV::QRaw qraw[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) KV::load_q_lds(qraw[h], sq, h, lr);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            KV::unpack_q(qraw[h], qf[h]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) qf[h][e] *= a.qscale;
        }
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
                acc = row32_sum(acc);
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

    // Two-deep register pipeline over the chunks of this split: chunks c and
    // c+1 are in flight while chunk c is consumed.
    for (int c0 = start; c0 < end; c0 += 2 * CHUNK) {
        const int c1 = c0 + CHUNK;
        process_chunk(0, c0);
        if (c1 >= end) break;
        const bool more = c1 + CHUNK < end;  // uniform
        if (more) load_chunk(0, c1 + CHUNK);
        process_chunk(1, c1);
        if (more) load_chunk(1, c1 + 2 * CHUNK);
    }

    // in place, split s is the designated merger of heads s, s + n_split, ...,
    // and decides for them now (the add's result is needed at the last
    // barrier)
    const unsigned own = n_split > 1 && grid.inplace ? inplace_heads<GT>(s, n_split) : 0u;
    unsigned decision = 0u;
    if (tid == 0 && own != 0u) decision = decide(a, col, own);

    // ---- merge the 2 row-groups of each wave ----
    __shared__ __attribute__((aligned(16))) float so[NW][GT][D];
    __shared__ float sm[NW][GT], sl[NW][GT];
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
    {
        // reduce-scatter: lanes of the low half keep of[0, NF/2), the high half of[NF/2, NF)
        const int fbase = (lane >> 5) * (NF / 2);
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
            float lo, hi;
            swap32(of[f], of[f + NF / 2], lo, hi);
            const int ff = fbase + f;
            so[wave][ff / EPL][KV::dim(lr, ff % EPL)] = lo + hi;
        }
    }
    __shared__ unsigned s_heads;
    if (tid == 0) s_heads = n_split > 1 ? tile_heads<GT>(a, col, n_split, own, decision, ticket) : 0u;
    __syncthreads();

    finish_split<TQ, D, GT, RES>(a, &so[0][0][0], &sm[0][0], &sl[0][0], col, s, n_split, out, h0);
    if (n_split > 1) merge_heads<TQ, D, GT, RES>(a, col, n_split, s_heads);
}

// ===========================================================================
// Dense KV cache on the matrix cores
// ===========================================================================
//
// One workgroup of 4 waves (one per SIMD) per (request, head tile, split),
// with the split plan, the partials and the merge above.  Wave w takes the
// 16-row blocks w, w + 4, ... of the split, two blocks in flight, read
// straight from HBM into registers in the layouts the matrix instructions
// take, so that no key or value ever moves between lanes.  With lane l,
// j = l % 16 and k = l / 16:
//   S^T[row][head] = K Q^T: A = K row j of the block (16-byte pieces k,
//     k + 4, ... of the row), B = query head j in the same element order
//     (zero past the tile's heads).  fp32 caches take
//     v_mfma_f32_16x16x4_f32 (one element of each piece per instruction),
//     16-bit caches v_mfma_f32_16x16x32_{bf16,f16} (a whole piece).  The
//     lane then holds head j, rows 4k .. 4k + 3 of the block.
//   Online softmax (log2 domain) with the lazy reference maximum, shared by
//     the four lanes of a head.
//   O^T[d][head] += V^T P^T with v_mfma_f32_16x16x4_f32, in four steps v
//     over the rows 4k + v: A = V[row 4k + v][the lane's dimensions] (16
//     lanes read a whole row, 16 or 8 consecutive bytes each), B = the
//     lane's own p of that row.  Values of 16-bit caches are widened to
//     fp32 in registers; p stays fp32.
// At the end each wave holds, per head, its reference maximum, its sum of
// weights and its output row; the workgroup combines the 4 waves through
// LDS (finish_split) and publishes the split's partial.
constexpr int kMfThreads = 256;
constexpr int kMfWaves = kMfThreads / 64;
constexpr int kMfRows = 16;  // rows per block

typedef float mf_f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 mf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 mf_f16x8_t __attribute__((ext_vector_type(8)));

template <typename T, int D>
struct MfKV {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int ROW = D * ES;                         // bytes per row
    static constexpr int KE = 16 / ES;                         // elements per 16-byte K piece
    static constexpr int NK = D / (4 * KE);                    // K pieces per lane (of the lane's row)
    static constexpr int VU = ROW / 16 >= 16 ? 16 : ROW / 16;  // bytes per V load
    static constexpr int NVL = ROW / 16 / VU;                  // V loads per lane and row
    static constexpr int VE = VU / ES;                         // elements per V load
    static constexpr int NTILE = D / 16;                       // 16-dimension output tiles
    static_assert(NK >= 1 && NVL * VE * 16 == D && NTILE == NVL * VE, "operand layout");
    struct Blk {
        u32x4_t k[NK];
        uint32_t v[4][NVL][VU / 4];
    };
    // Block of rows r0 .. r0 + 15 (rows at or past the resources' end read
    // as zeros): lane (j, k) reads K row r0 + j, pieces k + 4t, and V rows
    // r0 + 4k + v, bytes VU * (16h + j) .. of each.
    __device__ __forceinline__ static void load(Blk &bk, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                                int r0, int j, int k)
    {
#pragma unroll
        for (int t = 0; t < NK; ++t)
            bk.k[t] = __builtin_bit_cast(u32x4_t,
                                         __builtin_amdgcn_raw_buffer_load_b128(rk, (r0 + j) * ROW + 64 * t + 16 * k, 0, 0));
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int h = 0; h < NVL; ++h) {
                const int off = (r0 + 4 * k + v) * ROW + VU * (16 * h + j);
                if constexpr (VU == 16) {
                    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
                    bk.v[v][h][0] = x[0]; bk.v[v][h][1] = x[1]; bk.v[v][h][2] = x[2]; bk.v[v][h][3] = x[3];
                } else {
                    const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0);
                    bk.v[v][h][0] = x[0]; bk.v[v][h][1] = x[1];
                }
            }
    }
    // element e of V load (v, h), widened to fp32
    __device__ __forceinline__ static float v_elem(const Blk &bk, int v, int h, int e)
    {
        if constexpr (ES == 4) {
            return __uint_as_float(bk.v[v][h][e]);
        } else if constexpr (__is_same(T, bf16_t)) {
            const uint32_t w = bk.v[v][h][e / 2];
            return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
        } else {
            const uint32_t w = bk.v[v][h][e / 2];
            return f16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
        }
    }
};

// S^T of one block: fp32 elements one per instruction, 16-bit pieces whole.
template <typename T, int D>
struct MfQK;
template <int D>
struct MfQK<float, D> {
    typedef MfKV<float, D> M;
    float q[M::NK][4];  // query element 4(k + 4t) + e of head j, times scale * log2(e)
    __device__ __forceinline__ void init(const uint32_t *sq, int j, int k, bool valid, float qscale)
    {
#pragma unroll
        for (int t = 0; t < M::NK; ++t) {
            const uint4 x = *(const uint4 *)(sq + j * D + 4 * (k + 4 * t));
            q[t][0] = valid ? __uint_as_float(x.x) * qscale : 0.0f;
            q[t][1] = valid ? __uint_as_float(x.y) * qscale : 0.0f;
            q[t][2] = valid ? __uint_as_float(x.z) * qscale : 0.0f;
            q[t][3] = valid ? __uint_as_float(x.w) * qscale : 0.0f;
        }
    }
    __device__ __forceinline__ mf_f32x4_t scores(const typename M::Blk &bk) const
    {
        mf_f32x4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
#pragma unroll
        for (int t = 0; t < M::NK; ++t) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bk.k[t][0]), q[t][0], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bk.k[t][1]), q[t][1], c1, 0, 0, 0);
            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bk.k[t][2]), q[t][2], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bk.k[t][3]), q[t][3], c1, 0, 0, 0);
        }
        return c0 + c1;
    }
};
template <typename T16, int D>
struct MfQK16 {
    typedef MfKV<T16, D> M;
    typedef typename std::conditional<__is_same(T16, bf16_t), mf_bf16x8_t, mf_f16x8_t>::type op_t;
    op_t q[M::NK];  // query elements 8(k + 4t) .. + 7 of head j
    float qscale;
    __device__ __forceinline__ void init(const uint32_t *sq, int j, int k, bool valid, float qs)
    {
#pragma unroll
        for (int t = 0; t < M::NK; ++t) {
            uint4 x = *(const uint4 *)(sq + (j * D) / 2 + 4 * (k + 4 * t));
            if (!valid) x = make_uint4(0u, 0u, 0u, 0u);
            q[t] = __builtin_bit_cast(op_t, x);
        }
        qscale = qs;
    }
    __device__ __forceinline__ mf_f32x4_t scores(const typename M::Blk &bk) const
    {
        mf_f32x4_t c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
#pragma unroll
        for (int t = 0; t < M::NK; ++t) {
            if constexpr (__is_same(T16, bf16_t)) {
                if (t & 1) c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(op_t, bk.k[t]), q[t], c1, 0, 0, 0);
                else c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(op_t, bk.k[t]), q[t], c0, 0, 0, 0);
            } else {
                if (t & 1) c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(op_t, bk.k[t]), q[t], c1, 0, 0, 0);
                else c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(op_t, bk.k[t]), q[t], c0, 0, 0, 0);
            }
        }
        return (c0 + c1) * qscale;
    }
};
template <int D> struct MfQK<bf16_t, D> : MfQK16<bf16_t, D> {};
template <int D> struct MfQK<f16_t, D> : MfQK16<f16_t, D> {};

template <typename T, int D, int GT>
__global__ __launch_bounds__(kMfThreads) void decode_mfma_kernel(DecodeArgs a, DecodeGrid grid)
{
    constexpr int RES = kResNone;
    typedef MfKV<T, D> M;
    static_assert(GT <= 16, "one matrix column per query head");
    if ((int)blockIdx.x >= grid.n_stream) {
        merge_workgroup<T, D, GT, RES, kMfThreads>(a, (int)blockIdx.x - grid.n_stream);
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, j = lane & 15, k = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const DecodePlan &P = a.plan;
    int s, ht, b;
    if (a.kv_lens && grid.B <= kDecodePackMaxB) {
        SplitItem it;
        if (!packed_item<RES>(a, grid.B, (int)blockIdx.x, &it)) return;
        s = it.s; ht = it.ht; b = it.b;
    } else {
        s = (int)blockIdx.x % grid.gx;
        ht = ((int)blockIdx.x / grid.gx) % P.HT;
        b = (int)blockIdx.x / (grid.gx * P.HT);
    }
    int lo;  // first visible row (a window's start)
    const int n = windowed(a, request_len<RES>(a, b), &lo);
    const int n_split = (n + P.L - 1) / P.L;
    const int gk = ht / P.ht_per_kv;
    const int h0 = gk * P.G + (ht % P.ht_per_kv) * GT;
    T *out = (T *)a.out + ((size_t)b * a.Hq + h0) * D;

    if (n == 0) {  // empty request: defined as an all-zero output
        if (s == 0)
            for (int idx = tid; idx < GT * D; idx += kMfThreads) store_elem(out + idx, 0.0f);
        return;
    }
    if (s >= n_split) return;
    const int start = s * P.L;
    const int end = min(start + P.L, n);
    const int nblk = (end - start + kMfRows - 1) / kMfRows;

    const size_t head_row0 = ((size_t)b * a.Hkv + gk) * (size_t)a.s_cap + lo;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const T *)a.k + head_row0 * D, (size_t)end * M::ROW);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const T *)a.v + head_row0 * D, (size_t)end * M::ROW);

    // The query rows first (one 16-byte load per thread, staged in LDS), then
    // this split's group add, then the first blocks of every wave, all before
    // anything is consumed.  A block past the split reads zeros without
    // touching memory.
    constexpr int QB = GT * D * (int)sizeof(T);
    static_assert(QB <= 16 * kMfThreads, "query rows: one 16-byte load per thread");
    __shared__ __attribute__((aligned(16))) uint32_t sq[QB / 4];
    const bool q_loader = tid < QB / 16;
    const uint4 qv = *((const uint4 *)((const char *)a.q + ((size_t)b * a.Hq + h0) * D * sizeof(T)) +
                       (q_loader ? tid : 0));
    const int col = b * P.HT + ht;
    unsigned gticket = 0u;
    if (n_split > 1 && tid == 0) gticket = group_add(a, col, s);
    asm volatile("" ::: "memory");

    MfQK<T, D> qk;
    mf_f32x4_t o[M::NTILE];
#pragma unroll
    for (int t = 0; t < M::NTILE; ++t) o[t] = mf_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_ref = kNegInf, l_run = 0.0f;
    unsigned ticket = kNoTicket;  // a group completer's tile word add (awaited at the end)

    auto block = [&](const typename M::Blk &bk, int r0) {
        const mf_f32x4_t sv = qk.scores(bk);
        float sc[4] = {sv[0], sv[1], sv[2], sv[3]};
        if (r0 + kMfRows > end) {  // the split's last block: rows past its end
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (r0 + 4 * k + v >= end) sc[v] = kNegInf;
        }
        const float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        if (__any(bm > m_ref + kLazyRescale)) {
            const float mn = fmaxf(m_ref, max4q(bm));  // finite: the block's first row is valid
            const float al = rel_weight(m_ref, mn);
            m_ref = mn;
            l_run *= al;
#pragma unroll
            for (int t = 0; t < M::NTILE; ++t) o[t] *= al;
        }
        float p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            p[v] = fast_exp2(sc[v] - m_ref);
            l_run += p[v];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int h = 0; h < M::NVL; ++h)
#pragma unroll
                for (int e = 0; e < M::VE; ++e)
                    o[h * M::VE + e] =
                        __builtin_amdgcn_mfma_f32_16x16x4f32(M::v_elem(bk, v, h, e), p[v], o[h * M::VE + e], 0, 0, 0);
    };

    // Every wave's first block, and its second when the split has more than
    // one block per wave (a wave past the split's blocks reads zeros);
    // refills in the loop are unconditional (past the split they read zeros).
    typename M::Blk bk0, bk1;
    const bool two = nblk > kMfWaves;  // uniform
    M::load(bk0, rk, rv, start + wave * kMfRows, j, k);
    if (two) M::load(bk1, rk, rv, start + (wave + kMfWaves) * kMfRows, j, k);
    if (q_loader) *((uint4 *)sq + tid) = qv;
    __syncthreads();
    if (n_split > 1 && tid == 0) ticket = group_done(a, col, s, n_split, gticket);
    qk.init(sq, j < GT ? j : 0, k, j < GT, a.qscale);

    // Two-deep register pipeline over this wave's blocks.
    for (int kb = wave; kb < nblk; kb += 2 * kMfWaves) {
        block(bk0, start + kb * kMfRows);
        if (!two) break;
        M::load(bk0, rk, rv, start + (kb + 2 * kMfWaves) * kMfRows, j, k);
        if (kb + kMfWaves >= nblk) break;
        block(bk1, start + (kb + kMfWaves) * kMfRows);
        M::load(bk1, rk, rv, start + (kb + 3 * kMfWaves) * kMfRows, j, k);
    }

    // ---- the 4 waves' partials through LDS ----
    constexpr int SOD = D + 4;  // row stride (floats): the heads' rows start in distinct banks
    __shared__ __attribute__((aligned(16))) float so[kMfWaves * GT * SOD];
    __shared__ float sm[kMfWaves * GT], sl[kMfWaves * GT];
    l_run = sum4q(l_run);
    if (j < GT) {
        float *row = so + (wave * GT + j) * SOD;
#pragma unroll
        for (int h = 0; h < M::NVL; ++h)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int e4 = 0; e4 < M::VE; e4 += 4)
                    *(float4 *)&row[16 * M::VE * h + M::VE * (4 * k + v) + e4] =
                        make_float4(o[h * M::VE + e4][v], o[h * M::VE + e4 + 1][v], o[h * M::VE + e4 + 2][v],
                                    o[h * M::VE + e4 + 3][v]);
        if (k == 0) {
            sm[wave * GT + j] = m_ref;
            sl[wave * GT + j] = l_run;
        }
    }
    __shared__ unsigned s_heads;
    if (tid == 0) s_heads = n_split > 1 ? ticket_heads<GT>(a, col, n_split, ticket) : 0u;
    __syncthreads();

    finish_split<T, D, GT, RES, SOD, kMfThreads>(a, so, sm, sl, col, s, n_split, out, h0);
    if (n_split > 1) {
        // in place, split s is the designated merger of heads s, s + n_split, ...
        decide_after_publish<GT>(a, col, n_split, grid.inplace ? inplace_heads<GT>(s, n_split) : 0u, &s_heads);
        merge_heads<T, D, GT, RES, kMfThreads>(a, col, n_split, s_heads);
    }
}

// Sum over the lanes of a wave that share lane % CPW (CPW a power of two
// below 16): rotations by CPW, 2 CPW, ... inside each 16-lane row, then the
// two row swaps.  Every lane of the group ends with the same value.
template <int CPW> __device__ __forceinline__ float colgroup_sum(float x)
{
    if constexpr (CPW <= 1) x += dpp_f32<0x121>(x);  // row_ror:1
    if constexpr (CPW <= 2) x += dpp_f32<0x122>(x);  // row_ror:2
    if constexpr (CPW <= 4) x += dpp_f32<0x124>(x);  // row_ror:4
    if constexpr (CPW <= 8) x += dpp_f32<0x128>(x);  // row_ror:8
    return sum4q(x);
}

// Merge of item m = (request b, head tile ht) * GT + hh: the partials of
// the n_split splits of (b, ht) for query head h0 + hh, combined by a whole
// workgroup (one that has published its own split, or a merge workgroup).  Wave w owns the
// 4-wide output columns w*CPW .. w*CPW + CPW - 1; lane (c = lane % CPW,
// sg = lane / CPW) handles column c of the splits sg + k*LPC and polls
// those output slices itself.  Wave 0 polls the (max, sum) pairs (lane j:
// split j) and leaves each split's weight and the reciprocal of the total
// weight in LDS; each wave then scales its slices and sums its lanes with
// cross-lane steps.
//
template <typename TQ, int D, int GT, int RES, int NT>
__device__ void merge_head(const DecodeArgs &a, int m, int n_split)
{
    constexpr int D4 = D / 4;                     // 4-wide output columns
    constexpr int NW = NT / 64;                   // waves
    constexpr int CPW = D4 / NW;                  // columns per wave
    constexpr int LPC = 64 / CPW;                 // lanes per column
    constexpr int PER = kDecodeMaxSplits / LPC;   // splits per lane
    static_assert(CPW * NW == D4 && CPW < 16 && LPC * PER == kDecodeMaxSplits, "merge layout");
    static_assert(kDecodeMaxSplits <= 64, "every split's (max, sum) pair is polled by a lane of wave 0");
    __shared__ __attribute__((aligned(16))) float sw[LPC][PER];  // weight of split sg + k * LPC at [sg][k]
    __shared__ int s_go;
    __shared__ float s_inv;
    const DecodePlan &P = a.plan;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c = lane % CPW, sg = lane / CPW;
    const int d4 = wave * CPW + c;
    __syncthreads();  // a previous merge in this workgroup is done with the shared arrays
    const int hh = m % GT;
    const int col = m / GT;
    const int ht = col % P.HT;
    const int b = col / P.HT;
    if (n_split <= 1) return;  // written directly by the streaming workgroup
    const int g = ht / P.ht_per_kv;
    const int h = g * P.G + (ht % P.ht_per_kv) * GT + hh;
    TQ *out = (TQ *)a.out + ((size_t)b * a.Hq + h) * D;

    // Wait until every split has published this head's partial (the caller
    // holds the proof that every split has started): each thread polls the
    // tagged words it needs -- the (max, sum) pair of split tid (tid <
    // n_split) and its output slices of splits sg + k * LPC -- and zeroes
    // them once read, leaving the workspace as it found it.
    const size_t colbase = (size_t)col * P.n_split_max;
    const __amdgpu_buffer_rsrc_t ws_ml = make_rsrc(a.part_ml + colbase * GT * 2, (size_t)n_split * GT * 8);
    const __amdgpu_buffer_rsrc_t ws_o = make_rsrc(a.part_o + colbase * GT * D, (size_t)n_split * GT * D * 4);
    auto o_off = [&](int k) { return (int)(((((size_t)sg + (size_t)k * LPC) * GT + hh) * D + d4 * 4) * 4); };
    if (tid == 0) s_go = 1;
    __syncthreads();
    // a poisoned workspace (an earlier merge gave up) is not trusted; every
    // thread reads the word (one line), so that its round trip overlaps the
    // first poll's instead of preceding it
    const unsigned poisoned = __hip_atomic_load(a.poison, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tag_u4_t po[PER];
    tag_u2_t mlw = {0u, 0u};
    unsigned need = tid < n_split ? 1u << PER : 0u;  // bit k: slice k, bit PER: the pair
#pragma unroll
    for (int k = 0; k < PER; ++k)
        if (sg + k * LPC < n_split) need |= 1u << k;
    // Every poll issues all of this thread's loads before looking at any of
    // them (one round trip per poll).  Loads of splits past n_split fall
    // outside the resources' ranges: they read zero and touch no memory.
    unsigned pend = need;
    for (unsigned it = 0;; ++it) {
        // the words change under this loop: every poll must read memory again
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < PER; ++k)
            po[k] = __builtin_bit_cast(tag_u4_t, __builtin_amdgcn_raw_buffer_load_b128(ws_o, o_off(k), 0, kSC1));
        mlw = __builtin_bit_cast(tag_u2_t, __builtin_amdgcn_raw_buffer_load_b64(ws_ml, (tid * GT + hh) * 8, 0, kSC1));
        unsigned ok = is_tagged2(mlw) ? 1u << PER : 0u;
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (is_tagged4(po[k])) ok |= 1u << k;
        pend = need & ~ok;
        if (pend == 0u || it + 1 >= kMergeSpinLimit) break;
        __builtin_amdgcn_s_sleep(2);
    }
    if (pend != 0u) {
        s_go = 0;
        __hip_atomic_store(a.poison, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (poisoned != 0u) {
        s_go = 0;
    } else {
        // consume: every word read goes back to zero
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (sg + k * LPC < n_split)
                __builtin_amdgcn_raw_buffer_store_b128(tag_u4_t{0u, 0u, 0u, 0u}, ws_o, o_off(k), 0, kSC1);
        if (tid < n_split) __builtin_amdgcn_raw_buffer_store_b64(tag_u2_t{0u, 0u}, ws_ml, (tid * GT + hh) * 8, 0, kSC1);
    }
    // Wave 0 (lane j: split j) forms the maximum over the splits (and the
    // sink), each split's weight and the reciprocal of the total weight, and
    // leaves them in LDS, weights [sg][k] for split sg + k * LPC; every
    // thread then scales and adds its output slices.
    if (tid < 64) {
        const float2 ml = __builtin_bit_cast(float2, mlw);
        const bool in = tid < n_split;
        float mx = in ? ml.x : kNegInf;
        mx = fmaxf(mx, dpp_f32<0xB1>(mx));
        mx = fmaxf(mx, dpp_f32<0x4E>(mx));
        mx = fmaxf(mx, dpp_f32<0x141>(mx));
        mx = fmaxf(mx, dpp_f32<0x140>(mx));
        mx = max4q(mx);
        const float s2 = sink_log2(a, h);
        const float M = fmaxf(mx, s2);
        const float w = in ? fast_exp2(ml.x - M) : 0.0f;  // every split's maximum is finite
        sw[tid % LPC][tid / LPC] = w;
        float lw = w * ml.y;
        lw = row16_sum(lw);
        {
            float lo, hi;
            swap16(lw, lw, lo, hi);
            lw = lo + hi;
            swap32(lw, lw, lo, hi);
            lw = lo + hi;
        }
        if (tid == 0) s_inv = 1.0f / (lw + rel_weight(s2, M));
    }
    __syncthreads();
    if (!s_go) {  // not reachable (see the file header); never pass silently
        if (sg == 0) store4(out + d4 * 4, __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
        return;
    }
    float4 R = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float wk[PER];  // slots past the splits have weight 0 (and their words read as zero)
#pragma unroll
    for (int k = 0; k < PER; ++k) wk[k] = sw[sg][k];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const float4 x = __builtin_bit_cast(float4, po[k]);
        R.x += wk[k] * x.x; R.y += wk[k] * x.y; R.z += wk[k] * x.z; R.w += wk[k] * x.w;
    }
    R.x = colgroup_sum<CPW>(R.x);
    R.y = colgroup_sum<CPW>(R.y);
    R.z = colgroup_sum<CPW>(R.z);
    R.w = colgroup_sum<CPW>(R.w);
    const float inv = s_inv;
    if (sg == 0) store4(out + d4 * 4, R.x * inv, R.y * inv, R.z * inv, R.w * inv);
}

// The merges of heads (a bit per head of the tile) by a split that has
// published its own partial.
template <typename TQ, int D, int GT, int RES, int NT>
__device__ void merge_heads(const DecodeArgs &a, int col, int n_split, unsigned heads)
{
    for (int hh = 0; hh < GT; ++hh)
        if (heads & (1u << hh)) merge_head<TQ, D, GT, RES, NT>(a, col * GT + hh, n_split);
}

// A merge workgroup (placed after every split in the grid): the designated
// merger of item m = (request, head tile) * GT + head.  Thread 0 waits a
// bounded time for the tile word to count every group (it waits for starts
// only that long), then decides with its one add.
template <typename TQ, int D, int GT, int RES, int NT>
__device__ void merge_workgroup(const DecodeArgs &a, int m)
{
    __shared__ int s_go;
    const int col = m / GT, hh = m % GT;
    const int b = col / a.plan.HT;
    int lo;
    const int n = windowed(a, request_len<RES>(a, b), &lo);
    const int n_split = request_splits<RES>(a, b, n);
    if (n_split <= 1) return;  // written directly by the streaming workgroup
    if (threadIdx.x == 0) {
        const unsigned n_groups = split_groups(n_split);
        for (unsigned it = 0; it < kStartPolls; ++it) {
            if ((__hip_atomic_load(tile_word(a, col), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kTwGroups) ==
                n_groups)
                break;
            __builtin_amdgcn_s_sleep(2);
        }
        const unsigned old = decide(a, col, 1u << hh);
        tile_word_last<GT>(a, col, n_split, old + tile_decision_add(1u << hh));
        s_go = (old & kTwGroups) == n_groups ? 1 : 0;
    }
    __syncthreads();
    if (s_go) merge_head<TQ, D, GT, RES, NT>(a, m, n_split);
}

// ===========================================================================
// 4-bit group-affine cache on the matrix cores
// ===========================================================================
//
// With codes c, and scale s and bias b per group of G elements of a row,
// both products of the attention factor per group:
//     q . k          = s * sum_e q_e c_e + b * sum_e q_e
//     sum_r p_r v_r  = sum_r (p_r s_r) c_r + sum_r p_r b_r
// so the matrix cores multiply the codes themselves, and the scales and
// biases are applied per row and group in fp32 around them (the products
// equal those with dequantized K and V, up to rounding).
//
// Codes as f16 operands.  A 4-bit code c in bits 0..3 of a 16-bit lane is
// the f16 subnormal c * 2^-24, which v_mfma_f32_16x16x32_f16 multiplies
// exactly; a code in bits 4..7 is 16c * 2^-24, and the matching entry of
// the other operand is divided by 16 instead.  A word of 8 codes (nibble n
// = element n) thus becomes a full 8-slot operand with four masks and one
// shift, in the slot order (n0, n4, 16 n1, 16 n5, n2, n6, 16 n3, 16 n7), and
// the factor 2^24 is restored in fp32.
//
// Work.  One workgroup per (request, head tile, split), as the dense
// kernel; each wave takes 32-row steps of the split in turn (wave w: steps
// w, w + 8, ...), each staged into the wave's own LDS buffer (two per
// wave) by buffer loads that write LDS: codes of K and V in 16-byte pieces,
// scales and biases one 16-bit value per lane.  Per step, with lane l
// (l % 16 = j, l / 16 = qg):
//   S^T[row][head] = K Q^T per group: A = the K codes of row j of a 16-row
//     block (the lane's G/8 bytes of each group), B = the queries of head j
//     in the same slot order (zero for j >= GT);
//   scores in the log2 domain, scale * log2(e) folded in; the lane holds
//     head j and rows 4qg..4qg+3 of both 16-row blocks; online softmax with
//     an exact running maximum (so every p <= 1 and p * s fits f16);
//   O^T[d][head] += V^T (p s)^T: A = V codes of column d = 16n + j for the
//     lane's 8 rows, which ds_read_b64_tr_b4 delivers directly (lane i of a
//     16-lane group receives nibble i of the 8 bytes each of the group's 16
//     lanes names: here 8 rows at two 16-column blocks), B = p * s of the
//     same 8 rows in f16, one operand per group.
// The lane's rows of the second product (4qg + r of each block) are exactly
// the rows its scores hold, so P never leaves registers.  At the end each
// wave holds, per head, O = 2^24 O^T + sum_r p_r b_r, its maximum and its sum.

typedef _Float16 q4f16x8_t __attribute__((ext_vector_type(8)));
typedef float q4f32x4_t __attribute__((ext_vector_type(4)));
typedef int q4i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) q4i32x2_t lds_q4i32x2_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

constexpr int kQ4Rows = 32;                     // rows per wave step (two 16-row blocks)
constexpr int kQ4Waves = kDecodeThreads / 64;   // waves per workgroup

// LDS staging of one step: offsets in bytes within one buffer.
template <int D, int G>
struct Q4Stage {
    static constexpr int NG = D / G;                        // groups per row
    static constexpr int ROWB = D / 2;                      // code bytes per row
    static constexpr int CDMA = kQ4Rows * ROWB / 1024;      // 16-byte loads per step and code array
    // V rows 16..31 start VHALF bytes after rows 0..15 (D = 128: 32 bytes of
    // padding, so the transposing reads of the two blocks use other banks)
    static constexpr int VHALF = D == 128 ? 16 * ROWB + 32 : 16 * ROWB;
    static constexpr int SDMA = (kQ4Rows * NG + 63) / 64;   // 16-bit loads per step and scale/bias array
    static constexpr int SB = SDMA * 256;                   // bytes per scale/bias array (a dword per value)
    static constexpr int K = 0;
    static constexpr int V = kQ4Rows * ROWB;
    static constexpr int KS = V + VHALF + 16 * ROWB;
    static constexpr int KB = KS + SB;
    static constexpr int VS = KB + SB;
    static constexpr int VB = VS + SB;
    static constexpr int BYTES = VB + SB;
    static constexpr int NL = 2 * CDMA + 4 * SDMA;          // loads per step
    static_assert(CDMA * 1024 == kQ4Rows * ROWB, "code block");
};

// 8 codes (one word, nibble n = element n) as an f16 MFMA operand, slots
// (n0, n4, 16 n1, 16 n5, n2, n6, 16 n3, 16 n7) times 2^-24.
__device__ __forceinline__ q4f16x8_t q4_operand(uint32_t w)
{
    const uint32_t h = w >> 8;
    const u32x4_t x = {w & 0x000F000Fu, w & 0x00F000F0u, h & 0x000F000Fu, h & 0x00F000F0u};
    return __builtin_bit_cast(q4f16x8_t, x);
}

template <int D, int G, int GT, int RES>
__global__ __launch_bounds__(kDecodeThreads) void decode_q4_kernel(DecodeArgs a, DecodeGrid grid)
{
    typedef Q4Stage<D, G> S;
    constexpr int NG = S::NG;
    constexpr int TPG = G / 32;      // code words per lane, group and row
    constexpr int NT = D / 32;       // code words per lane and row (= k-blocks of the first product)
    constexpr int NDB = D / 16;      // 16-column blocks of the output
    static_assert(GT <= 16 && G % 32 == 0 && D % G == 0, "tile shape");

    if ((int)blockIdx.x >= grid.n_stream) {
        merge_workgroup<f16_t, D, GT, RES>(a, (int)blockIdx.x - grid.n_stream);
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63, j = lane & 15, qg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const DecodePlan &P = a.plan;
    const int s = (int)blockIdx.x % grid.gx;
    const int ht = ((int)blockIdx.x / grid.gx) % P.HT;
    const int b = (int)blockIdx.x / (grid.gx * P.HT);

    int lo;
    const int n = windowed(a, request_len<RES>(a, b), &lo);
    const int n_split = request_splits<RES>(a, b, n);
    const int g = ht / P.ht_per_kv;
    const int h0 = g * P.G + (ht % P.ht_per_kv) * GT;
    f16_t *out = (f16_t *)a.out + ((size_t)b * a.Hq + h0) * D;

    if (n_split == 0) {  // empty request: defined as an all-zero output
        if (s == 0)
            for (int idx = tid; idx < GT * D; idx += kDecodeThreads) store_elem(out + idx, 0.0f);
        return;
    }
    if (s >= n_split) return;
    if constexpr (RES == kResQ4) {
        // the last split of a residual-window cache: its float16 residual
        // rows, through the dense path (the same partial and merge)
        const int n_r = residual_rows(a, b);
        if (n_r > 0 && s == n_split - 1) {
            dense_split<DenseKV<f16_t, D>, f16_t, D, GT, RES>(a, grid, a.k_res, a.v_res,
                                                              ((size_t)b * a.Hkv + g) * (size_t)a.res_cap, s,
                                                              n_split, 0, n_r, b, ht, h0, out);
            return;
        }
    }
    const int start = s * P.L;
    const int end = min(start + P.L, n);
    const int nst = (end - start + kQ4Rows - 1) / kQ4Rows;

    // sources bounded to rows [0, end) of this (request, KV head): rows past
    // the split's end stage as zeros (and are masked below)
    const size_t head_row0 = ((size_t)b * a.Hkv + g) * (size_t)a.s_cap + lo;
    const BufDesc dk = buf_desc((const uint8_t *)a.k + head_row0 * S::ROWB, (size_t)end * S::ROWB);
    const BufDesc dv = buf_desc((const uint8_t *)a.v + head_row0 * S::ROWB, (size_t)end * S::ROWB);
    const BufDesc dks = buf_desc((const uint16_t *)a.k_scales + head_row0 * NG, (size_t)end * NG * 2);
    const BufDesc dkb = buf_desc((const uint16_t *)a.k_biases + head_row0 * NG, (size_t)end * NG * 2);
    const BufDesc dvs = buf_desc((const uint16_t *)a.v_scales + head_row0 * NG, (size_t)end * NG * 2);
    const BufDesc dvb = buf_desc((const uint16_t *)a.v_biases + head_row0 * NG, (size_t)end * NG * 2);

    __shared__ __attribute__((aligned(16))) unsigned char smem[kQ4Waves * 2 * S::BYTES];
    constexpr int SOD = D + 4;  // wave-output row stride (floats): the 16 heads' rows start in distinct banks
    static_assert(kQ4Waves * 2 * S::BYTES >= kQ4Waves * GT * SOD * 4, "wave outputs alias the staging buffers");
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_u8_t *)smem;
    const int wbuf = wave * 2 * S::BYTES;  // this wave's two buffers

    auto issue = [&](int st, int buf) {
        const int r0 = start + st * kQ4Rows;
        const unsigned base = lds0 + (unsigned)(wbuf + buf * S::BYTES);
#pragma unroll
        for (int i = 0; i < S::CDMA; ++i) lds_load16(dk, base + S::K + 1024 * i, r0 * S::ROWB + 1024 * i + 16 * lane);
#pragma unroll
        for (int i = 0; i < S::CDMA; ++i)
            lds_load16(dv, base + S::V + S::VHALF * i, r0 * S::ROWB + 1024 * i + 16 * lane);
#pragma unroll
        for (int i = 0; i < S::SDMA; ++i) {
            const int off = (r0 * NG + 64 * i + lane) * 2;
            lds_load_u16(dks, base + S::KS + 256 * i, off);
            lds_load_u16(dkb, base + S::KB + 256 * i, off);
            lds_load_u16(dvs, base + S::VS + 256 * i, off);
            lds_load_u16(dvb, base + S::VB + 256 * i, off);
        }
    };

    // The workgroup's query rows go to LDS by the same kind of load (the
    // first QDMA waves, 1 KB each), ahead of each wave's first two steps;
    // those waves wait for their query piece only, then the workgroup meets.
    // (With every load issued this way, the only waits are the explicit
    // ones: the first step is computed while the second is still arriving.)
    constexpr int QB = GT * D * 2;
    constexpr int QDMA = (QB + 1023) / 1024;
    __shared__ __attribute__((aligned(16))) uint16_t sq[QDMA * 512];
    if (wave < QDMA) {
        const BufDesc dq = buf_desc((const char *)a.q + ((size_t)b * a.Hq + h0) * D * 2, QB);
        lds_load16(dq, (unsigned)(uintptr_t)(lds_u8_t *)sq + 1024 * wave, 1024 * wave + 16 * lane);
    }
    // The group add comes first (thread 0), and wave 0 waits for it (and
    // its query piece) before issuing its steps (measured: 1 us faster at
    // 16384 rows than letting it overlap them); its result is used right
    // after the query barrier.
    const int col = b * P.HT + ht;
    unsigned gticket = 0u, ticket = kNoTicket;
    if (n_split > 1 && tid == 0) {
        gticket = group_add(a, col, s);
        asm volatile("s_waitcnt vmcnt(0)" ::"v"(gticket) : "memory");
    }
    const bool two = wave + kQ4Waves < nst;
    if (wave < nst) issue(wave, 0);
    if (two) issue(wave + kQ4Waves, 1);
    if (wave < QDMA) {
        if (two)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * S::NL) : "memory");
        else if (wave < nst)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::NL) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    // the group add's result is in (waited above): a group completer counts
    // its group now, early in the split
    if (n_split > 1 && tid == 0) ticket = group_done(a, col, s, n_split, gticket);

    // B operands of the first product: head j, slot order of q4_operand,
    // entries facing a 16c slot divided by 16; and per group the sum of the
    // head's query elements (times scale * log2(e)) for the bias term.
    q4f16x8_t qop[NT];
    float qs[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) qs[gg] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int gg = t / TPG;
        const int d0 = gg * G + qg * (G / 4) + 8 * (t % TPG);
        // one 16-byte read of a valid row (lanes of padding heads read row 0
        // and zero the values), not eight predicated 16-bit reads
        const uint4 raw = *(const uint4 *)&sq[(j < GT ? j : 0) * D + d0];
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x[e] = j < GT ? f16_bits_to_f32(rw[e / 2] >> (16 * (e & 1))) : 0.0f;
            qs[gg] += x[e];
        }
        const float r = 0.0625f;
        const q4f16x8_t op = {(_Float16)x[0], (_Float16)x[4], (_Float16)(x[1] * r), (_Float16)(x[5] * r),
                              (_Float16)x[2], (_Float16)x[6], (_Float16)(x[3] * r), (_Float16)(x[7] * r)};
        qop[t] = op;
    }
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) qs[gg] = sum4q(qs[gg]) * a.qscale;
    const float C = a.qscale * 16777216.0f;  // scale * log2(e) * 2^24

    // transposing-read address of this lane: row R(j % 8) of the step
    // (4qg + 0..3 in block 0, then in block 1), 8-byte column chunk j / 8
    int voff;
    {
        const int rr = j & 7;
        const int row = rr < 4 ? 4 * qg + rr : 16 + 4 * qg + (rr - 4);
        voff = S::V + (row < 16 ? row * S::ROWB : S::VHALF + (row - 16) * S::ROWB) + 8 * (j >> 3);
    }

    q4f32x4_t o[NDB];
#pragma unroll
    for (int nb = 0; nb < NDB; ++nb) o[nb] = q4f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = kNegInf, l_run = 0.0f, bsum[NG];
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) bsum[gg] = 0.0f;

    auto step = [&](int boff, int r0) {
        const unsigned char *bp = smem + boff;
        // ---- S^T = K Q^T, one accumulator per 16-row block and group ----
        q4f32x4_t acc[2][NG];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                const unsigned char *kp = bp + S::K + (16 * u + j) * S::ROWB + gg * (G / 2) + qg * (G / 8);
                uint32_t w[TPG];
                if constexpr (TPG == 4) {
                    const uint4 x = *(const uint4 *)kp;
                    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
                } else if constexpr (TPG == 2) {
                    const uint2 x = *(const uint2 *)kp;
                    w[0] = x.x; w[1] = x.y;
                } else {
                    w[0] = *(const uint32_t *)kp;
                }
                q4f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int tt = 0; tt < TPG; ++tt)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(q4_operand(w[tt]), qop[gg * TPG + tt], c, 0, 0, 0);
                acc[u][gg] = c;
            }
        }
        // ---- scores (log2 domain); rows past the split's end masked ----
        float sc[2][4];
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t *ks = (const uint32_t *)(bp + S::KS) + (16 * u + 4 * qg) * NG;
            const uint32_t *kb = (const uint32_t *)(bp + S::KB) + (16 * u + 4 * qg) * NG;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = 0.0f, y = 0.0f;
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    x = __builtin_fmaf(f16_bits_to_f32(ks[r * NG + gg]), acc[u][gg][r], x);
                    y = __builtin_fmaf(f16_bits_to_f32(kb[r * NG + gg]), qs[gg], y);
                }
                sc[u][r] = __builtin_fmaf(C, x, y);
            }
        }
        if (r0 + kQ4Rows > end) {  // the split's last step: rows past its end
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (r0 + 16 * u + 4 * qg + r >= end) sc[u][r] = kNegInf;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[u][r]);
        mx = max4q(mx);  // finite: the step's first row is valid
        if (m_run == kNegInf) {  // first step of this wave: nothing to rescale
            m_run = mx;
        } else if (__any(mx > m_run)) {
            const float mn = fmaxf(m_run, mx);
            const float al = fast_exp2(m_run - mn);  // 1 where unchanged
            m_run = mn;
            l_run *= al;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) bsum[gg] *= al;
#pragma unroll
            for (int nb = 0; nb < NDB; ++nb) o[nb] *= al;
        }
        // ---- probabilities, V-bias sums, and p * s as f16 operands ----
        float pr[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t *vb = (const uint32_t *)(bp + S::VB) + (16 * u + 4 * qg) * NG;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pr[u][r] = fast_exp2(sc[u][r] - m_run);
                l_run += pr[u][r];
#pragma unroll
                for (int gg = 0; gg < NG; ++gg)
                    bsum[gg] = __builtin_fmaf(pr[u][r], f16_bits_to_f32(vb[r * NG + gg]), bsum[gg]);
            }
        }
        q4f16x8_t pop[NG];
        {
            const uint32_t *vs0 = (const uint32_t *)(bp + S::VS) + (4 * qg) * NG;
            const uint32_t *vs1 = (const uint32_t *)(bp + S::VS) + (16 + 4 * qg) * NG;
            float pf[2][4];  // p, divided by 16 for the rows that face 16c slots
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) pf[u][r] = (r & 1) ? pr[u][r] * 0.0625f : pr[u][r];
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                _Float16 e[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    e[2 * r] = (_Float16)__builtin_fmaf(pf[0][r], f16_bits_to_f32(vs0[r * NG + gg]), 0.0f);
                    e[2 * r + 1] = (_Float16)__builtin_fmaf(pf[1][r], f16_bits_to_f32(vs1[r * NG + gg]), 0.0f);
                }
                const q4f16x8_t op = {e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]};
                pop[gg] = op;
            }
        }
        // ---- O^T += V^T (p s)^T ----
#pragma unroll
        for (int pp = 0; pp < D / 32; ++pp) {
            const q4i32x2_t w2 =
                __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_q4i32x2_t *)((lds_u8_t *)smem + boff + voff + 16 * pp));
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int nb = 2 * pp + hh;
                o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(q4_operand((uint32_t)w2[hh]), pop[(16 * nb) / G], o[nb],
                                                               0, 0, 0);
            }
        }
    };

    // Steps of this wave, two buffers: step st + 8 is in flight while st is
    // computed; the buffer of st is refilled with st + 16 afterwards.
    int it = 0;
    for (int st = wave; st < nst; st += kQ4Waves, ++it) {
        const int buf = it & 1;
        if (st + kQ4Waves < nst)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(S::NL) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        step(wbuf + buf * S::BYTES, start + st * kQ4Rows);
        if (st + 2 * kQ4Waves < nst) issue(st + 2 * kQ4Waves, buf);
    }

    const unsigned own = n_split > 1 && grid.inplace ? inplace_heads<GT>(s, n_split) : 0u;
    unsigned decision = 0u;
    if (tid == 0 && own != 0u) decision = decide(a, col, own);

    // ---- wave totals, then the workgroup's combination ----
    l_run = sum4q(l_run);
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) bsum[gg] = sum4q(bsum[gg]);
    __shared__ float sm[kQ4Waves * GT], sl[kQ4Waves * GT];
    __syncthreads();  // every wave is done with its staging buffers
    float *so = (float *)smem;  // [waves][GT][SOD]
    if (j < GT) {
#pragma unroll
        for (int nb = 0; nb < NDB; ++nb) {
            const float bb = bsum[(16 * nb) / G];
            *(float4 *)&so[(wave * GT + j) * SOD + 16 * nb + 4 * qg] =
                make_float4(16777216.0f * o[nb][0] + bb, 16777216.0f * o[nb][1] + bb, 16777216.0f * o[nb][2] + bb,
                            16777216.0f * o[nb][3] + bb);
        }
        if (qg == 0) {
            sm[wave * GT + j] = m_run;
            sl[wave * GT + j] = l_run;
        }
    }
    __shared__ unsigned s_heads;
    if (tid == 0) s_heads = n_split > 1 ? tile_heads<GT>(a, col, n_split, own, decision, ticket) : 0u;
    __syncthreads();
    finish_split<f16_t, D, GT, RES, SOD>(a, so, sm, sl, col, s, n_split, out, h0);
    if (n_split > 1) merge_heads<f16_t, D, GT, RES>(a, col, n_split, s_heads);
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
// Grid of a decode launch; returns the number of merge workgroups.  When
// every split can be resident at once (no more splits than compute units;
// each kernel holds at least one workgroup per CU), the splits merge the
// heads themselves right after publishing.  Otherwise a split that waited
// would hold a CU that later splits need, so dedicated merge workgroups
// follow every split in the grid instead.
static int decode_grid(int B, int GT, const DecodeArgs &a, DecodeGrid *g)
{
    g->gx = a.kv_lens ? a.plan.n_split_max : (a.kv_len + a.plan.L - 1) / a.plan.L;
    g->n_stream = g->gx * a.plan.HT * B;
    g->B = B;
    const bool several = a.plan.n_split_max > 1 && g->gx > 1;
    g->inplace = g->n_stream <= a.n_cus ? 1 : 0;
    return several && !g->inplace ? B * a.plan.HT * GT : 0;
}

template <typename T, int D, int GT>
static hipError_t launch_dense(int B, const DecodeArgs &a, hipStream_t stream)
{
    DecodeGrid g;
    const int n_merge = decode_grid(B, GT, a, &g);
    hipLaunchKernelGGL((decode_mfma_kernel<T, D, GT>), dim3(g.n_stream + n_merge), dim3(kMfThreads), 0, stream, a, g);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t dispatch_dense(int B, const DecodeArgs &a, hipStream_t s)
{
    switch (a.plan.GT) {
    case 1: return launch_dense<T, D, 1>(B, a, s);
    case 2: return launch_dense<T, D, 2>(B, a, s);
    case 3: return launch_dense<T, D, 3>(B, a, s);
    case 4: return launch_dense<T, D, 4>(B, a, s);
    case 5: return launch_dense<T, D, 5>(B, a, s);
    case 6: return launch_dense<T, D, 6>(B, a, s);
    case 7: return launch_dense<T, D, 7>(B, a, s);
    case 8: return launch_dense<T, D, 8>(B, a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(int dtype, int D, int B, const DecodeArgs &a, hipStream_t s)
{
    if (a.res_cap != 0) return hipErrorInvalidValue;
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

template <int D, int G, int GT, int RES>
static hipError_t launch_q4(int B, const DecodeArgs &a, hipStream_t stream)
{
    DecodeGrid g;
    const int n_merge = decode_grid(B, GT, a, &g);
    hipLaunchKernelGGL((decode_q4_kernel<D, G, GT, RES>), dim3(g.n_stream + n_merge), dim3(kDecodeThreads), 0,
                       stream, a, g);
    return hipGetLastError();
}

template <int D, int G, int RES>
static hipError_t dispatch_q4_gt(int B, const DecodeArgs &a, hipStream_t s)
{
    switch (a.plan.GT) {
    case 1: return launch_q4<D, G, 1, RES>(B, a, s);
    case 2: return launch_q4<D, G, 2, RES>(B, a, s);
    case 3: return launch_q4<D, G, 3, RES>(B, a, s);
    case 4: return launch_q4<D, G, 4, RES>(B, a, s);
    case 5: return launch_q4<D, G, 5, RES>(B, a, s);
    case 6: return launch_q4<D, G, 6, RES>(B, a, s);
    case 7: return launch_q4<D, G, 7, RES>(B, a, s);
    case 8: return launch_q4<D, G, 8, RES>(B, a, s);
    default: return hipErrorInvalidValue;
    }
}

template <int D, int G>
static hipError_t dispatch_q4(int B, const DecodeArgs &a, hipStream_t s)
{
    if (a.res_cap > 0) {  // a residual-window cache: device lengths, residual rows
        if (!a.kv_lens || !a.k_res || !a.v_res) return hipErrorInvalidValue;
        return dispatch_q4_gt<D, G, kResQ4>(B, a, s);
    }
    return dispatch_q4_gt<D, G, kResNone>(B, a, s);
}

hipError_t launch_decode_q4(int D, int group, int B, const DecodeArgs &a, hipStream_t s)
{
    if (group != a.group) return hipErrorInvalidValue;
    if (D == 128 && group == 32) return dispatch_q4<128, 32>(B, a, s);
    if (D == 128 && group == 64) return dispatch_q4<128, 64>(B, a, s);
    if (D == 128 && group == 128) return dispatch_q4<128, 128>(B, a, s);
    if (D == 64 && group == 32) return dispatch_q4<64, 32>(B, a, s);
    if (D == 64 && group == 64) return dispatch_q4<64, 64>(B, a, s);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Dequant check hook: a grid-stride loop over the elements, same dequant function.
// ---------------------------------------------------------------------------
__global__ void dequant_q4_kernel(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                                  float *out, long n_elems, int D, int group)
{
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n_elems; i += (long)gridDim.x * blockDim.x) {
        const long row = i / D;
        const int e = (int)(i % D);
        const uint32_t byte = codes[row * (D / 2) + e / 2];
        const uint32_t code = (e & 1) ? (byte >> 4) : (byte & 0xFu);
        const long gi = row * (D / group) + e / group;
        out[i] = q4_dequant_value(f16_bits_to_f32(scales[gi]), f16_bits_to_f32(biases[gi]), code);
    }
}

hipError_t launch_dequant_q4(const uint8_t *codes, const void *scales, const void *biases, float *out,
                             int n_rows, int D, int group, hipStream_t s)
{
    const long n = (long)n_rows * D;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    long blocks = (n + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(dequant_q4_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, codes,
                       (const uint16_t *)scales, (const uint16_t *)biases, out, n, D, group);
    return hipGetLastError();
}

}  // namespace gqa

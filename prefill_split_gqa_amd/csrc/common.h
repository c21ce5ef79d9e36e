// common.h -- internal definitions shared by the gfx950 kernels and the C-ABI
// layer of libgqa.so.  Not installed; the public interface is include/gqa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// ---------------------------------------------------------------------------
// Storage types.  bf16 and f16 travel as raw 16-bit words so that loads stay
// plain integer vector loads; conversion to fp32 happens in registers.
// ---------------------------------------------------------------------------
struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b)
{
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
    return (float)h;
}

// fp32 -> storage, round to nearest even (gfx950 converts natively).
template <typename T> __device__ __forceinline__ void store_elem(T *p, float x);
template <> __device__ __forceinline__ void store_elem<float>(float *p, float x) { *p = x; }
template <> __device__ __forceinline__ void store_elem<bf16_t>(bf16_t *p, float x)
{
    __bf16 h = (__bf16)x;
    p->bits = __builtin_bit_cast(uint16_t, h);
}
template <> __device__ __forceinline__ void store_elem<f16_t>(f16_t *p, float x)
{
    _Float16 h = (_Float16)x;
    p->bits = __builtin_bit_cast(uint16_t, h);
}

// Unpack the 32-bit words of a loaded vector into fp32 elements.
template <typename T> struct Unpack;
template <> struct Unpack<float> {
    static constexpr int per_word = 1;
    __device__ __forceinline__ static void run(uint32_t w, float *out) { out[0] = __uint_as_float(w); }
};
template <> struct Unpack<bf16_t> {
    static constexpr int per_word = 2;
    __device__ __forceinline__ static void run(uint32_t w, float *out)
    {
        out[0] = __uint_as_float(w << 16);
        out[1] = __uint_as_float(w & 0xFFFF0000u);
    }
};
template <> struct Unpack<f16_t> {
    static constexpr int per_word = 2;
    __device__ __forceinline__ static void run(uint32_t w, float *out)
    {
        out[0] = f16_bits_to_f32(w & 0xFFFFu);
        out[1] = f16_bits_to_f32(w >> 16);
    }
};

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// DPP row controls (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1 (lane^1),
// quad_perm [2,3,0,1] = 0x4E (lane^2), row_half_mirror = 0x141,
// row_mirror = 0x140.  The four steps below sum a value over each
// 16-lane row.
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp_f32(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    x += dpp_f32<0x141>(x);
    x += dpp_f32<0x140>(x);
    return x;
}

// Sum over each 32-lane half of the wave: the 16-lane sum, then the two
// rows of the half added with the gfx950 row swap (which hands each row the
// other row's value).
__device__ __forceinline__ float row32_sum(float x)
{
    x = row16_sum(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask)
{
    return __shfl_xor(x, mask, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resources: a load whose byte offset falls outside [0, bytes)
// returns zeros and touches no memory, which lets tiles past the end of a
// sequence be loaded without a branch.
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 data format
constexpr int kSC1 = 16;                 // cache policy bit of buffer accesses: device-scope coherence

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, size_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

// Buffer loads that write LDS (buffer_load_... lds): lane l's data at byte
// offset voff goes to LDS address lds_base + 16*l (16-byte loads) or
// lds_base + 4*l (16-bit loads, zero-extended to a dword); an offset outside
// the descriptor's range writes zeros (the whole offset is in the vector
// register, where the range check applies, per dword).  They are issued from
// inline assembly so that the compiler does not treat them as pending LDS
// stores (it would otherwise wait for every one of them at each workgroup
// barrier); the kernels wait for them themselves (s_waitcnt vmcnt) before
// the data is read.  The compiler's hazard recognizer cannot see inside
// inline assembly, so each block starts with the wait states a vector
// memory instruction needs after a VALU write of an SGPR it reads (5: the
// descriptor or M0 may have just been reloaded with v_readlane) and after
// an SALU write of M0 (1).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
struct BufDesc { u32x4_t w; };

__device__ __forceinline__ BufDesc buf_desc(const void *base, size_t bytes)
{
    const unsigned long long a = (unsigned long long)(uintptr_t)base;
    BufDesc d;
    d.w[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
    d.w[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32)) & 0xFFFFu;  // stride 0
    d.w[2] = __builtin_amdgcn_readfirstlane((unsigned)bytes);
    d.w[3] = kRsrcWord3;
    return d;
}

__device__ __forceinline__ void lds_load16(const BufDesc &d, unsigned lds_base, int voff)
{
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(d.w), "{m0}"(lds_base)
                 : "memory");
}

__device__ __forceinline__ void lds_load_u16(const BufDesc &d, unsigned lds_base, int voff)
{
    asm volatile("s_nop 4\n\tbuffer_load_ushort %0, %1, 0 offen lds" ::"v"(voff), "s"(d.w), "{m0}"(lds_base)
                 : "memory");
}

// ---------------------------------------------------------------------------
// Decode split plan.  The host sizes the workspace and the grid from it and
// the kernel derives every index from the same numbers, so a request's split
// boundaries depend only on (s_cap, Hq, Hkv, D) -- never on B or on the other
// requests' lengths.
// ---------------------------------------------------------------------------
constexpr int kDecodeThreads = 512;     // 8 waves
constexpr int kDecodeLPR = 32;          // lanes per key row (a row-group)
constexpr int kDecodeRowGroups = kDecodeThreads / kDecodeLPR;
constexpr int kDecodeMaxSplits = 64;    // partials merged by one workgroup (one round trip)
constexpr long kDecodeOneSplitElems = 8192;  // a KV head this small is one split (see make_decode_plan)
// Workgroups a plan aims for at full length: the matrix-core dense kernel's
// 4-wave workgroups co-reside 2 or 3 per CU (measured best, batched Qwen3-4B
// geometry, B = 1..8: 320 against 256, 384 and 512); the 4-bit kernel's
// 8-wave ones one per CU.
constexpr int kDecodeTargetWGs = 320;
constexpr int kDecodeQ4TargetWGs = 256;

// Every workspace begins with a flag region of fixed size.  The words that
// workgroups use to meet one another (decode (max, sum) words, prefill
// arrival counters) live only there, and every call leaves the ones it used
// at zero; partial results go after the region.  Because the region's place
// and size never depend on a call's sizes, the partial results of one call
// can never land where another call, of any sizes, looks for its flags.
constexpr size_t kWsFlagBytes = (size_t)16 << 20;
// The last kWsTailBytes of the region are never used for per-call words:
// they hold the poison word (offset kWsPoisonOff), set only if a decode
// merge ever had to give up waiting (then every later decode merge on that
// workspace writes NaN instead of trusting what it reads, until the
// workspace is zero-filled again).
constexpr size_t kWsTailBytes = 64;
constexpr size_t kWsPoisonOff = kWsFlagBytes - 16;

struct DecodePlan {
    int G;            // query heads per KV head
    int GT;           // query heads handled by one workgroup (divides G, <= 8)
    int ht_per_kv;    // G / GT
    int HT;           // Hkv * ht_per_kv: workgroup columns per request
    int L;            // keys per split (multiple of kDecodeRowGroups)
    int n_split_max;  // ceil(s_cap / L)
    // workspace layout: (max, sum) words at offset 0 (flag region), then
    // kCtrlWords control words per (request, head tile) at off_ctrl (also in
    // the flag region), partial outputs from kWsFlagBytes on
    size_t ml_bytes, off_ctrl, ctrl_bytes, off_o, o_bytes, bytes;
};

// Control words of one (request, head tile): a tile word, then one word per
// group of kSplitGroup splits (at most kDecodeMaxSplits / kSplitGroup),
// each on a 128-byte line of its own: many workgroups adding to one word at
// once queue behind each other in the memory system (measured: 64 adds on
// one word at the start of the launch cost 2.4 us of a 11.4 us decode, on
// separate lines nothing).  Groups of 16 (at most 4 per tile) measured
// 0.13 us faster than groups of 8 at the 7B headline and on the 4-bit decode
// (fewer group completions add to the tile word); 32 was no better.
constexpr int kSplitGroup = 16;
static_assert(kDecodeMaxSplits / kSplitGroup <= 15, "the tile word counts groups in 4 bits");
constexpr int kCtrlStride = 32;  // words
constexpr int kCtrlWords = 1 + kDecodeMaxSplits / kSplitGroup;

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// extra_splits: splits per (request, head tile) beyond those of the rows
// (a residual-window cache's float16 residual is one).
// min_per: the fewest rows per row-group a split gets (see below).
inline bool make_decode_plan(int B, int Hq, int Hkv, int D, int s_cap, int target_wgs, int max_splits,
                             DecodePlan *p, int extra_splits = 0, int min_per = 2)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || s_cap < 1 || Hq % Hkv || target_wgs < 1 || max_splits < 1)
        return false;
    p->G = Hq / Hkv;
    p->GT = 1;
    for (int t = 8; t >= 1; --t)
        if (p->G % t == 0) { p->GT = t; break; }
    p->ht_per_kv = p->G / p->GT;
    p->HT = Hkv * p->ht_per_kv;
    long ns = target_wgs / p->HT - extra_splits;  // the extra splits count against the target
    // A KV head of at most kDecodeOneSplitElems elements per K (and V) is one
    // split: the merge round trip costs more than streaming it in one
    // workgroup (measured, 0.5B geometry, 128 rows of 64: 5.6 us against
    // 6.7 us with 8 splits; at 128 rows of 128 the split plan stays ahead).
    if ((long)s_cap * D <= kDecodeOneSplitElems) ns = 1;
    if (ns < 1) ns = 1;
    if (ns > max_splits) ns = max_splits;
    const long rows = kDecodeRowGroups;
    long per = (s_cap + rows * ns - 1) / (rows * ns);  // rows per row-group per split
    // At least min_per rows per row-group as long as that still gives every
    // query head of a tile a split to merge it.  The 4-bit kernel takes 2
    // (32-row steps: shorter splits would leave half of each step's loads
    // empty); the matrix-core dense kernel takes 1 (16-row blocks: at 7B
    // geometry 16-row splits measured 0.1 us faster at KV lengths 512 and
    // 1024 than 32-row ones, and the same elsewhere).
    if (per < min_per && (s_cap + min_per * rows - 1) / (min_per * rows) >= p->GT) per = min_per;
    p->L = (int)(per * rows);
    p->n_split_max = (int)((s_cap + p->L - 1) / p->L) + extra_splits;
    const size_t parts = (size_t)B * p->HT * p->n_split_max * p->GT;  // (request, query head, split)
    p->ml_bytes = parts * 2 * 4;
    p->off_ctrl = align_up(p->ml_bytes, 128);
    p->ctrl_bytes = (size_t)B * p->HT * kCtrlWords * kCtrlStride * 4;
    p->off_o = kWsFlagBytes;
    p->o_bytes = parts * (size_t)D * 4;
    p->bytes = align_up(p->off_o + p->o_bytes, 256);
    // the flags and control words must fit their region (its tail is
    // reserved); partials are addressed with 32-bit offsets
    return p->off_ctrl + p->ctrl_bytes <= kWsFlagBytes - kWsTailBytes && p->o_bytes < ((size_t)1 << 31);
}

// Arguments of the split-K decode kernels (passed by value).
struct DecodeArgs {
    const void *q;
    const void *k;       // dense K, or 4-bit codes
    const void *v;       // dense V, or 4-bit codes
    const void *k_scales, *k_biases, *v_scales, *v_biases;  // 4-bit cache only
    void *out;
    const int32_t *kv_lens;  // device lengths, or nullptr
    int kv_len;              // uniform length when kv_lens == nullptr
    int Hq, Hkv, s_cap;
    int group;               // 4-bit cache group size (0 for dense caches)
    int window;              // > 0: only the last `window` rows of each request are visible
    const float *sinks;      // per query head softmax sink logits, or nullptr
    float qscale;            // scale * log2(e)
    DecodePlan plan;
    float *part_o, *part_ml; // per split: [GT][D] outputs, [GT][2] (max, sum)
    unsigned *ctrl;          // kCtrlWords control words per (request, head tile)
    unsigned *poison;        // the workspace's poison word
    size_t ws_bytes;
    int n_cus;               // compute units of the device (launch shape)
    // A 4-bit cache with a float16 residual window (res_cap > 0 rows per KV
    // head in k_res / v_res): a request of n tokens (clamped to s_cap) holds
    // n - n % res_cap rows 4-bit and n % res_cap rows in the residual.
    int res_cap;
    const void *k_res, *v_res;
};

// Launchers (defined in the .hip files; return a hipError_t).
hipError_t launch_decode(int dtype, int D, int B, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_q4(int D, int group, int B, const DecodeArgs &a, hipStream_t s);
hipError_t launch_dequant_q4(const uint8_t *codes, const void *scales, const void *biases, float *out,
                             int n_rows, int D, int group, hipStream_t s);
hipError_t launch_prefill(int dtype, int D, const void *q, const void *k, const void *v, void *out,
                          int B, int Hq, int Hkv, int Tq, int Tk, int s_cap, float scale, void *ws, int window,
                          const float *sinks, int n_cus, hipStream_t s);
size_t prefill_workspace_bytes(int B, int Hq, int D, int Tq, int Tk, int window, int n_cus);
// A 4-bit cache with a float16 residual as the prefill kernel reads it:
// key positions [0, n_q) from the 4-bit arrays (s_cap rows per KV head,
// group-affine, f16 scale and bias per group), later positions from the
// float16 residual rows (passed as k and v, R rows per KV head).
struct Q4Source {
    const uint8_t *k_codes, *v_codes;
    const uint16_t *k_scales, *k_biases, *v_scales, *v_biases;
    int n_q, group, s_cap;
};
hipError_t launch_prefill_q4r(int D, const void *q, const void *k_res, const void *v_res, void *out, int B, int Hq,
                              int Hkv, int Tq, int Tk, int R, float scale, void *ws, const Q4Source &src, int n_cus,
                              hipStream_t s);
hipError_t launch_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                            const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D, int T_new, int s_cap,
                            int elem_bytes, hipStream_t s);
hipError_t launch_kv_append_q4(int dtype, const void *k_new, const void *v_new, uint8_t *k_codes, void *k_scales,
                               void *k_biases, uint8_t *v_codes, void *v_scales, void *v_biases,
                               const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D, int group, int T_new,
                               int s_cap, hipStream_t s);
hipError_t launch_kv_append_q4r(const void *k_new, const void *v_new, uint8_t *k_codes, void *k_scales,
                                void *k_biases, uint8_t *v_codes, void *v_scales, void *v_biases, void *k_res,
                                void *v_res, const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D,
                                int group, int R, int T_new, int s_cap, hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_read_probe(const void *src, size_t bytes, void *sink, hipStream_t s);

}  // namespace gqa

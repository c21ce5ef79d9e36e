// gqa_abi.hip -- the extern "C" entry points declared in include/gqa.h.
//
// Every check on sizes, pointers and dtypes runs before the first HIP call,
// so an invalid call returns a status without touching the device (and can be
// exercised on a machine with no GPU).  The device check (gfx950 only; the
// decode page's companion finding returns an explicit error on a device the
// fused kernel does not support rather than falling back) runs next, then the
// kernels are enqueued on the caller's stream.

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/gqa.h"
#include "../../include/gqa_bench.h"
#include "common.h"

using namespace gqa;

namespace {

constexpr int kAbiVersion = 4;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// four_bit: the 4-bit kernel's plan (fewer workgroups and at least two rows
// per row-group: never more splits, so a dense plan's workspace fits it too)
bool plan_decode(int B, int Hq, int Hkv, int D, int s_cap, DecodePlan *p, bool four_bit = false)
{
    if (!make_decode_plan(B, Hq, Hkv, D, s_cap, four_bit ? kDecodeQ4TargetWGs : kDecodeTargetWGs, kDecodeMaxSplits,
                          p, 0, four_bit ? 2 : 1))
        return false;
    // grid limits, and buffer-resource ranges of the partial arrays
    return p->HT <= 65535 && p->n_split_max <= 65535 && p->bytes < ((size_t)1 << 31);
}

// 1 = gfx950, 0 = other device, -1 = HIP error; *cus = the device's compute
// units.  Cached per device ordinal.
int device_supported(int *cus = nullptr)
{
    static std::mutex mu;
    static int cache[64], n_cus[64];
    static bool init = false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (!init) {
        for (int &c : cache) c = 2;  // unknown
        init = true;
    }
    if (dev < 0 || dev >= 64) return -1;
    if (cache[dev] == 2) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
        n_cus[dev] = prop.multiProcessorCount;
        cache[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    if (cus) *cus = n_cus[dev];
    return cache[dev];
}

// Compute units of the current device, for launch plans whose sizes the
// host needs before it can launch (workspace sizes); 256 (the gfx950 parts)
// when no device can be queried.
int plan_cus()
{
    int cus = 0;
    return device_supported(&cus) == 1 && cus > 0 ? cus : 256;
}

int check_device(int *cus = nullptr)
{
    const int d = device_supported(cus);
    if (d < 0) return GQA_ERR_HIP;
    if (d == 0) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_HIP; }

bool dense_dtype(int dtype) { return dtype == GQA_F32 || dtype == GQA_BF16 || dtype == GQA_F16; }

// plan_rows: the rows the split plan covers (s_cap, or a window's length)
int check_decode_common(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv, int D,
                        int s_cap, float scale, void *ws, size_t ws_bytes, DecodePlan *plan, int plan_rows = 0,
                        bool four_bit = false)
{
    if (!q || !k || !v || !out) return GQA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || s_cap < 1) return GQA_ERR_SHAPE;
    if (!std::isfinite(scale)) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    // a KV head's rows are addressed with 32-bit buffer offsets
    if (B > 65535 || (size_t)s_cap * D * 4 >= ((size_t)1 << 31)) return GQA_ERR_SHAPE;
    if (!plan_decode(B, Hq, Hkv, D, plan_rows > 0 ? plan_rows : s_cap, plan, four_bit)) return GQA_ERR_SHAPE;
    if (!ws || ws_bytes < plan->bytes) return GQA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ws)) return GQA_ERR_ALIGN;
    return GQA_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode entry point: a file-scope device
// array (one per GPU), laid out like a workspace with a smaller flag
// region: (max, sum) words and control words at the front, the poison word
// at the end of that region, partial outputs after it.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr size_t kScratchFlagBytes = (size_t)512 << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

bool scratch_fits(const DecodePlan &p)
{
    return p.off_ctrl + p.ctrl_bytes <= kScratchFlagBytes - kWsTailBytes && p.o_bytes <= kScratchBytes - kScratchFlagBytes;
}

// Device address of `scratch` on the current device: taken with
// hipGetSymbolAddress once per device (with that device current) and kept;
// the first call on a device also zero-fills the array on `stream` (a
// kernel, not a memset).  The array's host-side name is never used as an
// address.  nullptr on a HIP error.
unsigned char *scratch_address(hipStream_t stream)
{
    static std::mutex mu;
    static unsigned char *addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        if (launch_fill_zero(ptr, kScratchBytes, stream) != hipSuccess) return nullptr;
        addr[dev] = (unsigned char *)ptr;
    }
    return addr[dev];
}

// Residual-window 4-bit decode: one launch, whose splits are those of the
// 4-bit rows plus one for the float16 residual rows (at most 63 + 1, so the
// merge still reads every partial in one round).
bool q4r_residual_ok(int D, int R) { return R >= 64 && R % 64 == 0 && (size_t)R * D * 4 < ((size_t)1 << 31); }

bool plan_q4r(int B, int Hq, int Hkv, int D, int s_cap, DecodePlan *p)
{
    if (!make_decode_plan(B, Hq, Hkv, D, s_cap, kDecodeQ4TargetWGs, kDecodeMaxSplits - 1, p, 1)) return false;
    return p->HT <= 65535 && p->n_split_max <= kDecodeMaxSplits && p->bytes < ((size_t)1 << 31);
}

void fill_ws(DecodeArgs &a, void *ws)
{
    char *base = (char *)ws;
    a.part_o = (float *)(base + a.plan.off_o);
    a.part_ml = (float *)base;  // the flag region
    a.ctrl = (unsigned *)(base + a.plan.off_ctrl);
    a.poison = (unsigned *)(base + kWsPoisonOff);
    a.ws_bytes = a.plan.bytes;
}

}  // namespace

extern "C" {

int gqa_abi_version(void) { return kAbiVersion; }

const char *gqa_status_string(int status)
{
    switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "sizes are inconsistent or out of range";
    case GQA_ERR_UNSUPPORTED: return "dtype, head dimension or device not supported";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_HIP: return "HIP runtime error";
    case GQA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case GQA_ERR_SCRATCH: return "sizes exceed the built-in scratch of the allocation-free entry point";
    default: return "unknown status";
    }
}

size_t gqa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int s_cap)
{
    if (D != 64 && D != 128) return 0;
    DecodePlan p;
    if (!plan_decode(B, Hq, Hkv, D, s_cap, &p)) return 0;
    return p.bytes;
}

int gqa_workspace_init(void *workspace, size_t bytes, void *stream)
{
    if (!workspace) return GQA_ERR_NULL;
    if (!aligned16(workspace)) return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return hip_status(launch_fill_zero(workspace, bytes, (hipStream_t)stream));
}

int gqa_decode_attend(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv, int D,
                      int kv_len, int s_cap, float scale, int dtype, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    DecodePlan plan;
    if (int st = check_decode_common(q, k, v, out, B, Hq, Hkv, D, s_cap, scale, workspace, workspace_bytes, &plan))
        return st;
    if (kv_len < 1 || kv_len > s_cap) return GQA_ERR_SHAPE;
    if (!dense_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    DecodeArgs a{};
    a.n_cus = cus;
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.kv_lens = nullptr; a.kv_len = kv_len;
    a.Hq = Hq; a.Hkv = Hkv; a.s_cap = s_cap; a.group = 0;
    a.qscale = scale * 1.4426950408889634f;
    a.plan = plan;
    fill_ws(a, workspace);
    return hip_status(launch_decode(dtype, D, B, a, (hipStream_t)stream));
}

int gqa_decode_attend_noalloc(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv,
                              int D, int kv_len, int s_cap, float scale, int dtype, void *stream)
{
    if (!q || !k || !v || !out) return GQA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || s_cap < 1) return GQA_ERR_SHAPE;
    if (!std::isfinite(scale)) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (B > 65535 || (size_t)s_cap * D * 4 >= ((size_t)1 << 31)) return GQA_ERR_SHAPE;
    DecodePlan plan;
    if (!plan_decode(B, Hq, Hkv, D, s_cap, &plan)) return GQA_ERR_SHAPE;
    if (!scratch_fits(plan)) return GQA_ERR_SCRATCH;
    if (kv_len < 1 || kv_len > s_cap) return GQA_ERR_SHAPE;
    if (!dense_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_ALIGN;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    unsigned char *base = scratch_address((hipStream_t)stream);
    if (!base) return GQA_ERR_HIP;
    DecodeArgs a{};
    a.n_cus = cus;
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.kv_lens = nullptr; a.kv_len = kv_len;
    a.Hq = Hq; a.Hkv = Hkv; a.s_cap = s_cap; a.group = 0;
    a.qscale = scale * 1.4426950408889634f;
    a.plan = plan;
    a.part_ml = (float *)base;
    a.ctrl = (unsigned *)(base + plan.off_ctrl);
    a.poison = (unsigned *)(base + kScratchFlagBytes - 16);
    a.part_o = (float *)(base + kScratchFlagBytes);
    a.ws_bytes = kScratchBytes;
    return hip_status(launch_decode(dtype, D, B, a, (hipStream_t)stream));
}

int gqa_decode_attend_batched(const void *q, const void *k, const void *v, void *out, const int32_t *kv_lens,
                              int B, int Hq, int Hkv, int D, int s_cap, float scale, int dtype, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    if (!kv_lens) return GQA_ERR_NULL;
    DecodePlan plan;
    if (int st = check_decode_common(q, k, v, out, B, Hq, Hkv, D, s_cap, scale, workspace, workspace_bytes, &plan))
        return st;
    if (!aligned16(kv_lens)) return GQA_ERR_ALIGN;
    if (!dense_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    DecodeArgs a{};
    a.n_cus = cus;
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.kv_lens = kv_lens; a.kv_len = 0;
    a.Hq = Hq; a.Hkv = Hkv; a.s_cap = s_cap; a.group = 0;
    a.qscale = scale * 1.4426950408889634f;
    a.plan = plan;
    fill_ws(a, workspace);
    return hip_status(launch_decode(dtype, D, B, a, (hipStream_t)stream));
}

int gqa_decode_attend_ex(const void *q, const void *k, const void *v, void *out, const int32_t *kv_lens, int B,
                         int Hq, int Hkv, int D, int s_cap, float scale, int dtype, int window, const float *sinks,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (!kv_lens) return GQA_ERR_NULL;
    if (window < 0) return GQA_ERR_SHAPE;
    DecodePlan plan;
    const int rows = window > 0 && window < s_cap ? window : s_cap;
    if (int st = check_decode_common(q, k, v, out, B, Hq, Hkv, D, s_cap, scale, workspace, workspace_bytes, &plan,
                                     rows))
        return st;
    if (!aligned16(kv_lens) || !aligned16(sinks)) return GQA_ERR_ALIGN;
    if (!dense_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    DecodeArgs a{};
    a.n_cus = cus;
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.kv_lens = kv_lens; a.kv_len = 0;
    a.Hq = Hq; a.Hkv = Hkv; a.s_cap = s_cap; a.group = 0;
    a.window = window; a.sinks = sinks;
    a.qscale = scale * 1.4426950408889634f;
    a.plan = plan;
    fill_ws(a, workspace);
    return hip_status(launch_decode(dtype, D, B, a, (hipStream_t)stream));
}

size_t gqa_prefill_workspace_bytes_ex(int B, int Hq, int Hkv, int D, int Tq, int Tk, int window)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Tq < 1 || Tq > Tk || window < 0) return 0;
    if (D != 64 && D != 128) return 0;
    return prefill_workspace_bytes(B, Hq, D, Tq, Tk, window, plan_cus());
}

size_t gqa_prefill_workspace_bytes(int B, int Hq, int Hkv, int D, int Tq, int Tk)
{
    return gqa_prefill_workspace_bytes_ex(B, Hq, Hkv, D, Tq, Tk, 0);
}

int gqa_prefill_causal_ex(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv, int D,
                          int Tq, int Tk, int s_cap, float scale, int dtype, int window, const float *sinks,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k || !v || !out) return GQA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return GQA_ERR_SHAPE;
    if (Tq < 1 || Tq > Tk || Tk > s_cap || window < 0) return GQA_ERR_SHAPE;
    if (!std::isfinite(scale)) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (dtype != GQA_BF16 && dtype != GQA_F16) return GQA_ERR_UNSUPPORTED;
    // the launch table names row blocks in 10 bits, and the 1-D grid has at
    // most 1024 items per (request, head)
    if (Tq > 1024 * 128 || (long)B * Hq * 1024 >= (1L << 31)) return GQA_ERR_SHAPE;
    // a head's rows (plus the tile past the end that a prefetch names) are
    // addressed with 32-bit byte offsets
    if ((size_t)(s_cap + 512) * D * 2 >= ((size_t)1 << 31)) return GQA_ERR_SHAPE;
    const int cus = plan_cus();
    const size_t need = prefill_workspace_bytes(B, Hq, D, Tq, Tk, window, cus);
    if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(workspace) ||
        !aligned16(sinks))
        return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return hip_status(launch_prefill(dtype, D, q, k, v, out, B, Hq, Hkv, Tq, Tk, s_cap, scale, workspace, window,
                                     sinks, cus, (hipStream_t)stream));
}

int gqa_prefill_causal_q4r(const void *q, const uint8_t *k_codes, const void *k_scales, const void *k_biases,
                           const uint8_t *v_codes, const void *v_scales, const void *v_biases, const void *k_res,
                           const void *v_res, void *out, int B, int Hq, int Hkv, int D, int group_size, int R, int Tq,
                           int Tk, int s_cap, float scale, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!q || !k_codes || !k_scales || !k_biases || !v_codes || !v_scales || !v_biases || !k_res || !v_res || !out)
        return GQA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return GQA_ERR_SHAPE;
    if (Tq < 1 || Tq > Tk || Tk > s_cap) return GQA_ERR_SHAPE;
    if (!std::isfinite(scale)) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (group_size != 32 && group_size != 64 && group_size != 128) return GQA_ERR_UNSUPPORTED;
    if (D % group_size != 0 || !q4r_residual_ok(D, R)) return GQA_ERR_SHAPE;
    if (Tq > 1024 * 128 || (long)B * Hq * 1024 >= (1L << 31)) return GQA_ERR_SHAPE;
    if ((size_t)(s_cap + 512) * D * 2 >= ((size_t)1 << 31) || (size_t)(R + 512) * D * 2 >= ((size_t)1 << 31))
        return GQA_ERR_SHAPE;
    const int cus = plan_cus();
    const size_t need = prefill_workspace_bytes(B, Hq, D, Tq, Tk, 0, cus);
    if (!workspace || workspace_bytes < need) return GQA_ERR_WORKSPACE;
    if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) || !aligned16(k_biases) ||
        !aligned16(v_scales) || !aligned16(v_biases) || !aligned16(k_res) || !aligned16(v_res) || !aligned16(out) ||
        !aligned16(workspace))
        return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    Q4Source src;
    src.k_codes = k_codes; src.v_codes = v_codes;
    src.k_scales = (const uint16_t *)k_scales; src.k_biases = (const uint16_t *)k_biases;
    src.v_scales = (const uint16_t *)v_scales; src.v_biases = (const uint16_t *)v_biases;
    src.n_q = Tk - Tk % R;
    src.group = group_size;
    src.s_cap = s_cap;
    return hip_status(launch_prefill_q4r(D, q, k_res, v_res, out, B, Hq, Hkv, Tq, Tk, R, scale, workspace, src, cus,
                                         (hipStream_t)stream));
}

int gqa_prefill_causal(const void *q, const void *k, const void *v, void *out, int B, int Hq, int Hkv, int D,
                       int Tq, int Tk, int s_cap, float scale, int dtype, void *workspace, size_t workspace_bytes,
                       void *stream)
{
    return gqa_prefill_causal_ex(q, k, v, out, B, Hq, Hkv, D, Tq, Tk, s_cap, scale, dtype, 0, nullptr, workspace,
                                 workspace_bytes, stream);
}

int gqa_decode_attend_q4(const void *q, const uint8_t *k_codes, const void *k_scales, const void *k_biases,
                         const uint8_t *v_codes, const void *v_scales, const void *v_biases, void *out, int B,
                         int Hq, int Hkv, int D, int group_size, int kv_len, int s_cap, float scale,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (!k_scales || !k_biases || !v_scales || !v_biases) return GQA_ERR_NULL;
    DecodePlan plan;
    if (int st = check_decode_common(q, k_codes, v_codes, out, B, Hq, Hkv, D, s_cap, scale, workspace,
                                     workspace_bytes, &plan, 0, true))
        return st;
    if (kv_len < 1 || kv_len > s_cap) return GQA_ERR_SHAPE;
    if (group_size != 32 && group_size != 64 && group_size != 128) return GQA_ERR_UNSUPPORTED;
    if (D % group_size != 0) return GQA_ERR_SHAPE;
    if (!aligned16(k_scales) || !aligned16(k_biases) || !aligned16(v_scales) || !aligned16(v_biases))
        return GQA_ERR_ALIGN;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    DecodeArgs a{};
    a.n_cus = cus;
    a.q = q; a.k = k_codes; a.v = v_codes; a.out = out;
    a.k_scales = k_scales; a.k_biases = k_biases; a.v_scales = v_scales; a.v_biases = v_biases;
    a.kv_lens = nullptr; a.kv_len = kv_len;
    a.Hq = Hq; a.Hkv = Hkv; a.s_cap = s_cap; a.group = group_size;
    a.qscale = scale * 1.4426950408889634f;
    a.plan = plan;
    fill_ws(a, workspace);
    return hip_status(launch_decode_q4(D, group_size, B, a, (hipStream_t)stream));
}

size_t gqa_decode_q4r_workspace_bytes(int B, int Hq, int Hkv, int D, int s_cap, int R)
{
    if ((D != 64 && D != 128) || !q4r_residual_ok(D, R)) return 0;
    DecodePlan p;
    if (!plan_q4r(B, Hq, Hkv, D, s_cap, &p)) return 0;
    return p.bytes;
}

int gqa_decode_attend_q4r(const void *q, const uint8_t *k_codes, const void *k_scales, const void *k_biases,
                          const uint8_t *v_codes, const void *v_scales, const void *v_biases, const void *k_res,
                          const void *v_res, void *out, const int32_t *kv_lens, int B, int Hq, int Hkv, int D,
                          int group_size, int R, int s_cap, float scale, void *workspace, size_t workspace_bytes,
                          void *stream)
{
    if (!k_scales || !k_biases || !v_scales || !v_biases || !k_res || !v_res || !kv_lens) return GQA_ERR_NULL;
    DecodePlan plan;
    // (the common checks, with the workspace size checked against this plan below)
    if (int st = check_decode_common(q, k_codes, v_codes, out, B, Hq, Hkv, D, s_cap, scale, workspace,
                                     ~(size_t)0, &plan))
        return st;
    if (!q4r_residual_ok(D, R) || !plan_q4r(B, Hq, Hkv, D, s_cap, &plan)) return GQA_ERR_SHAPE;
    if (group_size != 32 && group_size != 64 && group_size != 128) return GQA_ERR_UNSUPPORTED;
    if (D % group_size != 0) return GQA_ERR_SHAPE;
    if (workspace_bytes < plan.bytes) return GQA_ERR_WORKSPACE;
    if (!aligned16(k_scales) || !aligned16(k_biases) || !aligned16(v_scales) || !aligned16(v_biases) ||
        !aligned16(k_res) || !aligned16(v_res) || !aligned16(kv_lens))
        return GQA_ERR_ALIGN;
    int cus = 0;
    if (int st = check_device(&cus)) return st;
    DecodeArgs a{};
    a.n_cus = cus;
    a.q = q; a.k = k_codes; a.v = v_codes; a.out = out;
    a.k_scales = k_scales; a.k_biases = k_biases; a.v_scales = v_scales; a.v_biases = v_biases;
    a.kv_lens = kv_lens; a.kv_len = 0;
    a.Hq = Hq; a.Hkv = Hkv; a.s_cap = s_cap; a.group = group_size;
    a.res_cap = R; a.k_res = k_res; a.v_res = v_res;
    a.qscale = scale * 1.4426950408889634f;
    a.plan = plan;
    fill_ws(a, workspace);
    return hip_status(launch_decode_q4(D, group_size, B, a, (hipStream_t)stream));
}

int gqa_kv_append_q4r(const void *k_new, const void *v_new, uint8_t *k_codes, void *k_scales, void *k_biases,
                      uint8_t *v_codes, void *v_scales, void *v_biases, void *k_res, void *v_res,
                      const int32_t *kv_lens, int32_t *new_lens, int B, int Hkv, int D, int group_size, int R,
                      int T_new, int s_cap, void *stream)
{
    if (!k_new || !v_new || !k_codes || !k_scales || !k_biases || !v_codes || !v_scales || !v_biases || !k_res ||
        !v_res || !kv_lens)
        return GQA_ERR_NULL;
    if (B < 1 || Hkv < 1 || T_new < 1 || s_cap < 1 || B > 65535 || (long)B * Hkv > 0x7FFFFFFFL) return GQA_ERR_SHAPE;
    if ((const void *)new_lens == (const void *)kv_lens) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (group_size != 32 && group_size != 64 && group_size != 128) return GQA_ERR_UNSUPPORTED;
    if (D % group_size != 0) return GQA_ERR_SHAPE;
    if (!q4r_residual_ok(D, R)) return GQA_ERR_SHAPE;
    if ((long)B * Hkv * (long)(s_cap > T_new ? s_cap : T_new) * D * 4 >= (1L << 46)) return GQA_ERR_SHAPE;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_codes) || !aligned16(v_codes) ||
        !aligned16(k_scales) || !aligned16(k_biases) || !aligned16(v_scales) || !aligned16(v_biases) ||
        !aligned16(k_res) || !aligned16(v_res) || !aligned16(kv_lens) || !aligned16(new_lens))
        return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return hip_status(launch_kv_append_q4r(k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases,
                                           k_res, v_res, kv_lens, new_lens, B, Hkv, D, group_size, R, T_new, s_cap,
                                           (hipStream_t)stream));
}

int gqa_kv_append(const void *k_new, const void *v_new, void *k_cache, void *v_cache, const int32_t *kv_lens,
                  int32_t *new_lens, int B, int Hkv, int D, int T_new, int s_cap, int dtype, void *stream)
{
    if (!k_new || !v_new || !k_cache || !v_cache || !kv_lens) return GQA_ERR_NULL;
    if (B < 1 || Hkv < 1 || T_new < 1 || s_cap < 1) return GQA_ERR_SHAPE;
    if ((const void *)new_lens == (const void *)kv_lens) return GQA_ERR_SHAPE;  // every lane reads kv_lens
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (!dense_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
    const int elem = dtype == GQA_F32 ? 4 : 2;
    if ((long)B * Hkv * (long)(s_cap > T_new ? s_cap : T_new) * D * elem >= (1L << 46)) return GQA_ERR_SHAPE;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(kv_lens) ||
        !aligned16(new_lens))
        return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return hip_status(launch_kv_append(k_new, v_new, k_cache, v_cache, kv_lens, new_lens, B, Hkv, D, T_new, s_cap,
                                       elem, (hipStream_t)stream));
}

int gqa_kv_append_q4(const void *k_new, const void *v_new, int dtype, uint8_t *k_codes, void *k_scales,
                     void *k_biases, uint8_t *v_codes, void *v_scales, void *v_biases, const int32_t *kv_lens,
                     int32_t *new_lens, int B, int Hkv, int D, int group_size, int T_new, int s_cap, void *stream)
{
    if (!k_new || !v_new || !k_codes || !k_scales || !k_biases || !v_codes || !v_scales || !v_biases || !kv_lens)
        return GQA_ERR_NULL;
    if (B < 1 || Hkv < 1 || T_new < 1 || s_cap < 1) return GQA_ERR_SHAPE;
    if ((const void *)new_lens == (const void *)kv_lens) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (group_size != 32 && group_size != 64 && group_size != 128) return GQA_ERR_UNSUPPORTED;
    if (D % group_size != 0) return GQA_ERR_SHAPE;
    if (!dense_dtype(dtype)) return GQA_ERR_UNSUPPORTED;
    if ((long)B * Hkv * (long)(s_cap > T_new ? s_cap : T_new) * D * 4 >= (1L << 46)) return GQA_ERR_SHAPE;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_codes) || !aligned16(v_codes) ||
        !aligned16(k_scales) || !aligned16(k_biases) || !aligned16(v_scales) || !aligned16(v_biases) ||
        !aligned16(kv_lens) || !aligned16(new_lens))
        return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return hip_status(launch_kv_append_q4(dtype, k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales,
                                          v_biases, kv_lens, new_lens, B, Hkv, D, group_size, T_new, s_cap,
                                          (hipStream_t)stream));
}

int gqa_dequant_q4(const uint8_t *codes, const void *scales, const void *biases, float *out, int n_rows, int D,
                   int group_size, void *stream)
{
    if (!codes || !scales || !biases || !out) return GQA_ERR_NULL;
    if (n_rows < 0) return GQA_ERR_SHAPE;
    if (D != 64 && D != 128) return GQA_ERR_UNSUPPORTED;
    if (group_size != 32 && group_size != 64 && group_size != 128) return GQA_ERR_UNSUPPORTED;
    if (D % group_size != 0) return GQA_ERR_SHAPE;
    if (int st = check_device()) return st;
    return hip_status(launch_dequant_q4(codes, scales, biases, out, n_rows, D, group_size, (hipStream_t)stream));
}

int gqa_read_probe(const void *src, size_t bytes, void *sink, void *stream)
{
    if (!src || !sink) return GQA_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || bytes / 16 / 1024 >= ((size_t)1 << 32)) return GQA_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(sink)) return GQA_ERR_ALIGN;
    if (int st = check_device()) return st;
    return hip_status(launch_read_probe(src, bytes, sink, (hipStream_t)stream));
}

}  // extern "C"

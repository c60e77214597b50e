// api.hip -- the C ABI: argument validation, workspace layout and the launch
// sequence of the whole layer. No allocation, no synchronisation, no device
// reads on the host: every call only enqueues kernels on the caller's stream.
//
// Error convention after the FlashInfer PR #6986 analysis, section 1:
// shape queries (check_shape / is_supported) answer without failing; the run
// entry points return a status and launch nothing when validation fails.
#include <mutex>

#include "common.hpp"

namespace moe {

int device_cu_count()
{
    static int cache[64];
    static std::once_flag once[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::call_once(once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev] = n;
    });
    return cache[dev];
}

namespace {

std::mutex g_override_mu;
moe_launch_override g_override = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};

}  // namespace

moe_launch_override launch_override()
{
    std::lock_guard<std::mutex> lock(g_override_mu);
    return g_override;
}

// The grouped GEMM descriptor of the layer's gate/up or down projection
// (sizes, expected rows under uniform routing, code layout); the caller fills
// in the pointers.
GemmLaunch layer_gemm_args(const moe_shape &sh, moe_gemm_kind kind)
{
    GemmLaunch g{};
    g.kind = kind;
    g.top_k = sh.top_k;
    g.num_experts = sh.num_local_experts;
    g.max_rows = sh.num_tokens * sh.top_k;
    // expected local rows: the routed slots that land on this GPU's experts
    g.expected_rows = (int)((long long)g.max_rows * sh.num_local_experts / sh.num_experts);
    if (kind == MOE_GEMM_W2) {
        g.K = sh.inter;
        g.N = sh.hidden;
    } else {
        g.K = sh.hidden;
        g.N = 2 * sh.inter;
    }
    g.a_bytes = (size_t)g.max_rows * g.K * 2;
    g.w_tiled = sh.weight_layout == MOE_WEIGHTS_TILED;
    return g;
}

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_shape(const moe_shape *sh)
{
    if (!sh)
        return MOE_ERR_NULL;
    if (sh->group_size != kGroup)
        return MOE_ERR_UNSUPPORTED;
    if (sh->num_tokens < 0 || sh->num_tokens > kMaxTokens)
        return MOE_ERR_SHAPE;
    if (sh->hidden < kGroup || sh->hidden > kMaxDim || sh->hidden % kGroup)
        return MOE_ERR_SHAPE;
    if (sh->inter < kGroup || sh->inter > kMaxDim || sh->inter % kGroup)
        return MOE_ERR_SHAPE;
    if (sh->num_experts < 1 || sh->num_experts > kMaxExperts)
        return MOE_ERR_SHAPE;
    if (sh->num_local_experts < 1 || sh->num_local_experts > kMaxExperts)
        return MOE_ERR_SHAPE;
    if (sh->expert_begin < 0 || sh->expert_begin + sh->num_local_experts > sh->num_experts)
        return MOE_ERR_SHAPE;
    if (sh->top_k < 1 || sh->top_k > kMaxTopK || sh->top_k > sh->num_experts)
        return MOE_ERR_SHAPE;
    if (sh->weight_layout != MOE_WEIGHTS_PLAIN && sh->weight_layout != MOE_WEIGHTS_TILED)
        return MOE_ERR_UNSUPPORTED;
    // activation-sized arrays are addressed with 32-bit buffer offsets
    const long long rows = (long long)sh->num_tokens * sh->top_k;
    const long long widest = sh->hidden > sh->inter ? sh->hidden : sh->inter;
    if (rows * widest * 2 >= (1LL << 31))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Forward workspace layout (each region 256-byte aligned).
struct Workspace {
    int32_t *ids;
    float *w;
    int32_t *counts;
    int32_t *offsets;
    int32_t *perm;
    int32_t *inv_perm;
    uint16_t *h;
    uint16_t *y;
    int32_t *part;    // per-range expert counts of the parallel permutation (many tokens)
    int32_t *pres;    // small-batch path: slot index if the slot's expert is local, else -1
    size_t bytes;
};

// nsh shared experts add nsh*T rows after the T*k routed rows and nsh
// experts after the E_loc routed ones.
Workspace carve(const moe_shape &sh, void *base, int nsh = 0)
{
    const size_t Sr = (size_t)sh.num_tokens * sh.top_k;
    const size_t S = Sr + (size_t)nsh * sh.num_tokens;
    const size_t E = (size_t)sh.num_local_experts + nsh;
    char *p = static_cast<char *>(base);
    size_t off = 0;
    Workspace ws{};
    auto take = [&](size_t bytes) {
        char *r = p ? p + off : nullptr;
        off += align_up(bytes);
        return r;
    };
    ws.ids = reinterpret_cast<int32_t *>(take(Sr * 4));
    ws.w = reinterpret_cast<float *>(take(Sr * 4));
    ws.counts = reinterpret_cast<int32_t *>(take(E * 4));
    ws.offsets = reinterpret_cast<int32_t *>(take((E + 1) * 4));
    ws.perm = reinterpret_cast<int32_t *>(take(S * 4));
    ws.inv_perm = reinterpret_cast<int32_t *>(take(Sr * 4));
    ws.h = reinterpret_cast<uint16_t *>(take(S * (size_t)sh.inter * 2));
    ws.y = reinterpret_cast<uint16_t *>(take(S * (size_t)sh.hidden * 2));
    ws.part = reinterpret_cast<int32_t *>(take(permute_workspace_bytes(sh)));
    ws.pres = reinterpret_cast<int32_t *>(take(Sr * 4));
    ws.bytes = off;
    return ws;
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The W4A4 (MXFP4) entry points: the same limits, with 32-element scale
// blocks and plain (row-major) codes.
moe_status check_shape_mx(const moe_shape *sh)
{
    if (!sh)
        return MOE_ERR_NULL;
    if (sh->group_size != 32 || (sh->weight_layout != MOE_WEIGHTS_PLAIN && sh->weight_layout != MOE_WEIGHTS_TILED))
        return MOE_ERR_UNSUPPORTED;
    moe_shape s = *sh;
    s.group_size = kGroup;
    return check_shape(&s);
}

// W4A4 layer workspace: the W4A16 layer's regions plus the quantized x and h.
struct MxWorkspace {
    Workspace base;
    uint8_t *xq, *xs, *hq, *hs;
    size_t bytes;
};

MxWorkspace carve_mx(const moe_shape &sh, void *p)
{
    MxWorkspace w{};
    w.base = carve(sh, p);
    char *b = static_cast<char *>(p);
    size_t off = w.base.bytes;
    auto take = [&](size_t bytes) {
        char *r = b ? b + off : nullptr;
        off += align_up(bytes);
        return reinterpret_cast<uint8_t *>(r);
    };
    const size_t T = (size_t)sh.num_tokens, S = T * sh.top_k;
    w.xq = take(T * sh.hidden / 2);
    w.xs = take(T * sh.hidden / 32);
    w.hq = take(S * sh.inter / 2);
    w.hs = take(S * sh.inter / 32);
    w.bytes = off;
    return w;
}

constexpr int32_t kMaxDenseDim = 65536;   // N and K of the dense GEMM


}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_status_str(moe_status s)
{
    switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: sizes inconsistent or out of range";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: configuration not supported";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: pointer misaligned";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    }
    return "unknown moe_status";
}

moe_status moe_w4a16_check_shape(const moe_shape *shape) { return check_shape(shape); }

moe_status moe_w4a16_set_launch_override(const moe_launch_override *ov)
{
    std::lock_guard<std::mutex> lock(g_override_mu);
    if (ov)
        g_override = *ov;
    else
        g_override = moe_launch_override{-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
    return MOE_OK;
}

int moe_w4a16_is_supported(const moe_shape *shape) { return check_shape(shape) == MOE_OK ? 1 : 0; }

size_t moe_w4a16_workspace_size(const moe_shape *shape)
{
    if (check_shape(shape) != MOE_OK)
        return 0;
    return carve(*shape, nullptr).bytes;
}

size_t moe_w4a16_workspace_size_shared(const moe_shape *shape, int32_t num_shared)
{
    if (check_shape(shape) != MOE_OK || num_shared < 1 || num_shared > kMaxSharedExperts)
        return 0;
    return carve(*shape, nullptr, num_shared).bytes;
}

size_t moe_permute_workspace_size(const moe_shape *shape)
{
    if (check_shape(shape) != MOE_OK)
        return 0;
    return permute_workspace_bytes(*shape);
}

moe_status moe_route(const moe_shape *shape, const float *logits, int32_t *topk_ids, float *topk_w,
                     void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    if (shape->num_tokens == 0)
        return MOE_OK;
    if (!logits || !topk_ids || !topk_w)
        return MOE_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
        return MOE_ERR_ALIGN;
    return from_hip(launch_route(*shape, logits, topk_ids, topk_w, static_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const moe_shape *shape, const int32_t *topk_ids, const uint16_t *x,
                       int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_perm,
                       uint16_t *x_perm, void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    if (!counts || !offsets)
        return MOE_ERR_NULL;
    const size_t need = permute_workspace_bytes(*shape);
    if (need && !workspace)
        return MOE_ERR_NULL;
    if (workspace_bytes < need)
        return MOE_ERR_WORKSPACE;
    if (need && !aligned(workspace, 4))
        return MOE_ERR_ALIGN;
    if ((x == nullptr) != (x_perm == nullptr))
        return MOE_ERR_NULL;
    if (shape->num_tokens > 0 && (!topk_ids || !perm || !inv_perm))
        return MOE_ERR_NULL;
    if (x && (!aligned(x, 16) || !aligned(x_perm, 16)))
        return MOE_ERR_ALIGN;
    if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(topk_ids, 4) || !aligned(perm, 4) ||
        !aligned(inv_perm, 4))
        return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_permute(*shape, topk_ids, counts, offsets, perm, inv_perm, s, 0,
                                  static_cast<int32_t *>(workspace));
    if (e == hipSuccess && x && shape->num_tokens > 0)
        e = launch_gather(*shape, x, perm, offsets, x_perm, s);
    return from_hip(e);
}

moe_status moe_grouped_gemm_w4a16(const moe_shape *shape, moe_gemm_kind kind, const uint16_t *a,
                                  const int32_t *a_row_index, const int32_t *offsets,
                                  const uint8_t *wq, const uint16_t *s, void *c, moe_dtype c_dtype,
                                  void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    if (kind != MOE_GEMM_W13_SWIGLU && kind != MOE_GEMM_W2 && kind != MOE_GEMM_W13_RAW)
        return MOE_ERR_UNSUPPORTED;
    if (c_dtype != MOE_BF16 && c_dtype != MOE_F32)
        return MOE_ERR_UNSUPPORTED;
    if (kind == MOE_GEMM_W13_SWIGLU && c_dtype != MOE_BF16)
        return MOE_ERR_UNSUPPORTED;
    if (shape->num_tokens == 0)
        return MOE_OK;
    if (!a || !offsets || !wq || !s || !c)
        return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(wq, 16) || !aligned(c, 16) || !aligned(s, 2) ||
        !aligned(offsets, 4) || (a_row_index && !aligned(a_row_index, 4)))
        return MOE_ERR_ALIGN;
    GemmLaunch g = layer_gemm_args(*shape, kind);
    g.a = a;
    g.a_row_index = a_row_index;
    if (a_row_index)
        g.a_bytes = (size_t)shape->num_tokens * g.K * 2;
    g.offsets = offsets;
    g.wq = wq;
    g.s = s;
    g.c = c;
    g.c_f32 = c_dtype == MOE_F32;
    return from_hip(launch_grouped_gemm(g, static_cast<hipStream_t>(stream)));
}

moe_status moe_w4a16_dense_gemm(int32_t M, int32_t N, int32_t K, const uint16_t *a, const uint8_t *wq,
                                const uint16_t *s, void *c, moe_dtype c_dtype, int32_t weight_layout,
                                void *stream)
{
    if (M < 0 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0 || N > kMaxDenseDim || K > kMaxDenseDim)
        return MOE_ERR_SHAPE;
    if ((size_t)N * (K / 2) >= (size_t(1) << 31) || (size_t)M * K * 2 >= (size_t(1) << 31))
        return MOE_ERR_UNSUPPORTED;                       // beyond one buffer descriptor's range
    if (c_dtype != MOE_BF16 && c_dtype != MOE_F32)
        return MOE_ERR_UNSUPPORTED;
    if (weight_layout != MOE_WEIGHTS_PLAIN && weight_layout != MOE_WEIGHTS_TILED)
        return MOE_ERR_UNSUPPORTED;
    if (M == 0)
        return MOE_OK;
    if (!a || !wq || !s || !c)
        return MOE_ERR_NULL;
    if (!aligned(a, 16) || !aligned(wq, 16) || !aligned(c, 16) || !aligned(s, 2))
        return MOE_ERR_ALIGN;
    // one expert holding every row: the grouped GEMM with offsets {0, M}
    // passed by value (nothing to read from device memory)
    GemmLaunch g{};
    g.kind = MOE_GEMM_W2;
    g.top_k = 1;
    g.num_experts = 1;
    g.max_rows = M;
    g.expected_rows = M;
    g.K = K;
    g.N = N;
    g.a = a;
    g.a_row_index = nullptr;
    g.a_bytes = (size_t)M * K * 2;
    g.offsets = nullptr;
    g.dense_rows = M;
    g.wq = wq;
    g.s = s;
    g.c = c;
    g.c_f32 = c_dtype == MOE_F32;
    g.w_tiled = weight_layout == MOE_WEIGHTS_TILED;
    return from_hip(launch_grouped_gemm(g, static_cast<hipStream_t>(stream)));
}

moe_status moe_finalize(const moe_shape *shape, const void *y, moe_dtype y_dtype,
                        const float *topk_w, const int32_t *inv_perm, void *out, moe_dtype out_dtype,
                        void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    if ((y_dtype != MOE_BF16 && y_dtype != MOE_F32) || (out_dtype != MOE_BF16 && out_dtype != MOE_F32))
        return MOE_ERR_UNSUPPORTED;
    if (shape->num_tokens == 0)
        return MOE_OK;
    if (!y || !topk_w || !inv_perm || !out)
        return MOE_ERR_NULL;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(topk_w, 4) || !aligned(inv_perm, 4))
        return MOE_ERR_ALIGN;
    return from_hip(launch_finalize(*shape, y, y_dtype == MOE_F32, topk_w, inv_perm, out,
                                    out_dtype == MOE_F32, static_cast<hipStream_t>(stream)));
}

moe_status moe_w4a16_pack_weights(const moe_shape *shape, moe_gemm_kind kind, const uint8_t *wq,
                                  uint8_t *wq_tiled, void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    if (kind != MOE_GEMM_W13_SWIGLU && kind != MOE_GEMM_W2 && kind != MOE_GEMM_W13_RAW)
        return MOE_ERR_UNSUPPORTED;
    if (!wq || !wq_tiled)
        return MOE_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(wq_tiled, 16))
        return MOE_ERR_ALIGN;
    const int N = kind == MOE_GEMM_W2 ? shape->hidden : 2 * shape->inter;
    const int K = kind == MOE_GEMM_W2 ? shape->inter : shape->hidden;
    const size_t bytes = (size_t)shape->num_local_experts * N * (K / 2);
    const uintptr_t a = reinterpret_cast<uintptr_t>(wq), b = reinterpret_cast<uintptr_t>(wq_tiled);
    if (a < b + bytes && b < a + bytes)
        return MOE_ERR_UNSUPPORTED;                       // in place or overlapping
    return from_hip(launch_pack_weights(shape->num_local_experts, N, K, shape->inter,
                                        kind == MOE_GEMM_W13_SWIGLU, wq, wq_tiled,
                                        static_cast<hipStream_t>(stream)));
}

// The layer's general path builds the permutation inside the gate/up GEMM
// (no permutation launch) up to this many tokens; past it the separate
// permutation, whose one workgroup scales better than every GEMM workgroup
// redoing it. The launch override's perm_in_gemm_max_tokens changes it.
static bool perm_in_gemm_fits(const moe_shape &sh)
{
    const int ov = launch_override().perm_in_gemm_max_tokens;
    return sh.num_tokens <= (ov >= 0 ? ov : 512);
}

// The layer, with nsh >= 0 shared experts folded into the same launches:
// the permutation appends one T-row segment per shared expert, the grouped
// GEMMs see E_loc + nsh experts (the last nsh read the shared weights) and
// the finalize adds the shared rows after the routed slots.
static moe_status forward_impl(const moe_shape *shape, int nsh, const uint16_t *x, const float *router_logits,
                               const uint8_t *w13_q, const uint16_t *s13, const uint8_t *w2_q, const uint16_t *s2,
                               const uint8_t *w13_sh, const uint16_t *s13_sh, const uint8_t *w2_sh,
                               const uint16_t *s2_sh, uint16_t *out, void *workspace, size_t workspace_bytes,
                               void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    const moe_shape &sh = *shape;
    if (nsh < 0 || nsh > kMaxSharedExperts)
        return MOE_ERR_UNSUPPORTED;
    const long long rows = (long long)sh.num_tokens * (sh.top_k + nsh);
    if (rows * (sh.hidden > sh.inter ? sh.hidden : sh.inter) * 2 >= (1LL << 31))
        return MOE_ERR_UNSUPPORTED;
    if (sh.num_tokens == 0)
        return MOE_OK;
    if (!x || !router_logits || !w13_q || !s13 || !w2_q || !s2 || !out || !workspace)
        return MOE_ERR_NULL;
    if (nsh > 0 && (!w13_sh || !s13_sh || !w2_sh || !s2_sh))
        return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w13_q, 16) || !aligned(w2_q, 16) ||
        !aligned(s13, 2) || !aligned(s2, 2) || !aligned(router_logits, 4) || !aligned(workspace, kAlign))
        return MOE_ERR_ALIGN;
    if (nsh > 0 && (!aligned(w13_sh, 16) || !aligned(w2_sh, 16) || !aligned(s13_sh, 2) || !aligned(s2_sh, 2)))
        return MOE_ERR_ALIGN;
    Workspace ws = carve(sh, workspace, nsh);
    if (workspace_bytes < ws.bytes)
        return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (decode_path_fits(sh, nsh)) {
        // small batch: routing inside the gate/up GEMM, h and y in slot order,
        // no permutation; the combine inside the down GEMM for the fewest tokens
        e = launch_decode_gate_up(sh, router_logits, x, w13_q, s13, ws.ids, ws.w, ws.pres, ws.h, s);
        if (e == hipSuccess) {
            if (decode_combine_fits(sh)) {
                e = launch_decode_down_combine(sh, ws.ids, ws.w, ws.pres, ws.h, w2_q, s2, out, s);
            } else {
                e = launch_decode_down(sh, ws.ids, ws.pres, ws.h, w2_q, s2, ws.y, s);
                if (e == hipSuccess)
                    e = launch_finalize(sh, ws.y, false, ws.w, ws.pres, out, false, s, true);
            }
        }
        return from_hip(e);
    }
    // The gate/up GEMM of the general path (the pointers the layer gives it).
    GemmLaunch g1 = layer_gemm_args(sh, MOE_GEMM_W13_SWIGLU);
    g1.a = x;
    g1.a_row_index = ws.perm;
    g1.a_bytes = (size_t)sh.num_tokens * sh.hidden * 2;
    g1.offsets = ws.offsets;
    g1.wq = w13_q;
    g1.s = s13;
    g1.c = ws.h;
    g1.c_f32 = false;
    // Up to a few hundred tokens the gate/up GEMM builds the permutation
    // itself from the routing ids (every workgroup, in LDS) and stores its
    // tables for the down GEMM and the finalize: one launch fewer. Measured
    // on MI355X (Qwen3-30B-A3B layer; its EP shard): 17-32 tokens 0.6-0.7 us
    // (2.2-2.5 us) faster than routing inside the permutation, 64 and 256
    // tokens 2.0-3.3 and 2.6-2.8 us (5.3-7.4 and 1.9-2.6 us) faster than the
    // separate permutation, 512 tokens 1.9 us.
    auto with_shared = [&](GemmLaunch &g, const uint8_t *wq_sh, const uint16_t *s_sh) {
        if (nsh == 0)
            return;
        g.e_routed = g.num_experts;
        g.num_experts += nsh;
        g.max_rows += nsh * sh.num_tokens;
        g.expected_rows += nsh * sh.num_tokens;
        g.wq_sh = wq_sh;
        g.s_sh = s_sh;
    };
    with_shared(g1, w13_sh, s13_sh);
    // (with shared experts the GEMM appends their T-row segments, as the
    // separate permutation does)
    const bool perm_in_gemm = perm_in_gemm_fits(sh) && gemm_ids_supported(g1, sh.num_tokens);
    if (perm_in_gemm) {
        e = launch_route(sh, router_logits, ws.ids, ws.w, s);
    } else if (route_permute_fusable(sh)) {
        e = launch_route_permute(sh, router_logits, ws.ids, ws.w, ws.counts, ws.offsets, ws.perm, ws.inv_perm, s,
                                 nsh);
    } else {
        e = launch_route(sh, router_logits, ws.ids, ws.w, s);
        if (e == hipSuccess)
            e = launch_permute(sh, ws.ids, ws.counts, ws.offsets, ws.perm, ws.inv_perm, s, nsh, ws.part);
    }
    if (e == hipSuccess && perm_in_gemm) {
        IdsSource src{ws.ids, sh.num_tokens, sh.expert_begin, ws.counts, ws.offsets, ws.perm, ws.inv_perm};
        e = launch_gemm_ids(g1, src, s);
    } else if (e == hipSuccess) {
        e = launch_grouped_gemm(g1, s);
    }
    // every slot local (and no shared rows): the down GEMM writes y in slot
    // order and the finalize reads it without the inv_perm indirection
    const bool y_slot = sh.num_local_experts == sh.num_experts && nsh == 0;
    if (e == hipSuccess) {
        GemmLaunch g = layer_gemm_args(sh, MOE_GEMM_W2);
        with_shared(g, w2_sh, s2_sh);
        g.a = ws.h;
        g.a_row_index = nullptr;
        g.a_bytes = (size_t)g.max_rows * sh.inter * 2;
        g.offsets = ws.offsets;
        g.wq = w2_q;
        g.s = s2;
        g.c = ws.y;
        g.c_row_index = y_slot ? ws.perm : nullptr;
        g.c_f32 = false;
        e = launch_grouped_gemm(g, s);
    }
    if (e == hipSuccess)
        e = launch_finalize(sh, ws.y, false, ws.w, ws.inv_perm, out, false, s, y_slot, nsh,
                            ws.offsets + sh.num_local_experts);
    return from_hip(e);
}

moe_status moe_w4a16_forward(const moe_shape *shape, const uint16_t *x, const float *router_logits,
                             const uint8_t *w13_q, const uint16_t *s13, const uint8_t *w2_q,
                             const uint16_t *s2, uint16_t *out, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    return forward_impl(shape, 0, x, router_logits, w13_q, s13, w2_q, s2, nullptr, nullptr, nullptr, nullptr, out,
                        workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// The layer without a caller workspace: its intermediates live in a
// file-scope device array (one copy per GPU, held until the process ends).
// Host code never passes the array's name to a kernel: that name is only a
// host-side stand-in. Its device address is looked up once per device, with
// that device current, and kept; kernels get that address as their workspace.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static void *g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

// Device address of this device's scratch array (NULL on failure, with the
// HIP error in *err). The lookup runs on the first call on each device.
static void *scratch_address(hipError_t *err)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void *ptr = nullptr;
        const hipError_t r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = r;
        g_scratch_ptr[dev] = r == hipSuccess ? ptr : nullptr;
    });
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}

moe_status moe_w4a16_forward_noalloc(const moe_shape *shape, const uint16_t *x, const float *router_logits,
                                     const uint8_t *w13_q, const uint16_t *s13, const uint8_t *w2_q,
                                     const uint16_t *s2, uint16_t *out, void *stream)
{
    moe_status st = check_shape(shape);
    if (st != MOE_OK)
        return st;
    if (carve(*shape, nullptr).bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_WORKSPACE;                         // beyond the fixed scratch array
    if (shape->num_tokens == 0)
        return MOE_OK;
    hipError_t err = hipSuccess;
    void *ws = scratch_address(&err);
    if (!ws)
        return MOE_ERR_HIP;
    // nothing in the workspace has to start at zero: every kernel of the
    // layer writes each intermediate before any kernel reads it
    return forward_impl(shape, 0, x, router_logits, w13_q, s13, w2_q, s2, nullptr, nullptr, nullptr, nullptr, out,
                        ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_mxfp4_quantize(int64_t rows, int32_t K, const uint16_t *x, uint8_t *codes, uint8_t *scales,
                              void *stream)
{
    if (rows < 0 || K < 32 || K % 32 != 0 || K > 65536)
        return MOE_ERR_SHAPE;
    if (rows * (int64_t)K * 2 >= (1LL << 40))
        return MOE_ERR_UNSUPPORTED;
    if (rows == 0)
        return MOE_OK;
    if (!x || !codes || !scales)
        return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(codes, 16))
        return MOE_ERR_ALIGN;
    return from_hip(launch_mx_quantize(rows, K, x, codes, scales, nullptr, static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm_mxfp4(const moe_shape *shape, moe_gemm_kind kind, const uint8_t *a_codes,
                                  const uint8_t *a_scales, const int32_t *a_row_index, const int32_t *offsets,
                                  const uint8_t *wq, const uint8_t *ws, void *c, moe_dtype c_dtype, void *stream)
{
    moe_status st = check_shape_mx(shape);
    if (st != MOE_OK)
        return st;
    if (kind != MOE_GEMM_W13_SWIGLU && kind != MOE_GEMM_W2 && kind != MOE_GEMM_W13_RAW)
        return MOE_ERR_UNSUPPORTED;
    if ((c_dtype != MOE_BF16 && c_dtype != MOE_F32) || (kind == MOE_GEMM_W13_SWIGLU && c_dtype != MOE_BF16))
        return MOE_ERR_UNSUPPORTED;
    if (shape->num_tokens == 0)
        return MOE_OK;
    if (!a_codes || !a_scales || !offsets || !wq || !ws || !c)
        return MOE_ERR_NULL;
    if (!aligned(a_codes, 16) || !aligned(wq, 16) || !aligned(c, 16) || !aligned(a_scales, 4) || !aligned(ws, 4) ||
        !aligned(offsets, 4) || (a_row_index && !aligned(a_row_index, 4)))
        return MOE_ERR_ALIGN;
    GemmLaunch g0 = layer_gemm_args(*shape, kind);
    MxGemmLaunch g{};
    g.kind = kind;
    g.a = a_codes;
    g.as = a_scales;
    g.a_row_index = a_row_index;
    g.a_rows = a_row_index ? shape->num_tokens : (long long)shape->num_tokens * shape->top_k;
    g.top_k = shape->top_k;
    g.offsets = offsets;
    g.num_experts = shape->num_local_experts;
    g.wq = wq;
    g.ws = ws;
    g.c = c;
    g.c_f32 = c_dtype == MOE_F32;
    g.K = g0.K;
    g.N = g0.N;
    g.max_rows = g0.max_rows;
    g.expected_rows = g0.expected_rows;
    g.w_tiled = shape->weight_layout == MOE_WEIGHTS_TILED;
    return from_hip(launch_mx_grouped_gemm(g, static_cast<hipStream_t>(stream)));
}

moe_status moe_mxfp4_pack_weights(const moe_shape *shape, moe_gemm_kind kind, const uint8_t *wq, uint8_t *wq_tiled,
                                  void *stream)
{
    moe_status st = check_shape_mx(shape);
    if (st != MOE_OK)
        return st;
    if (kind != MOE_GEMM_W13_SWIGLU && kind != MOE_GEMM_W2 && kind != MOE_GEMM_W13_RAW)
        return MOE_ERR_UNSUPPORTED;
    if (!wq || !wq_tiled)
        return MOE_ERR_NULL;
    if (!aligned(wq, 16) || !aligned(wq_tiled, 16))
        return MOE_ERR_ALIGN;
    const int N = kind == MOE_GEMM_W2 ? shape->hidden : 2 * shape->inter;
    const int K = kind == MOE_GEMM_W2 ? shape->inter : shape->hidden;
    const size_t bytes = (size_t)shape->num_local_experts * N * (K / 2);
    const uintptr_t a = reinterpret_cast<uintptr_t>(wq), b = reinterpret_cast<uintptr_t>(wq_tiled);
    if (a < b + bytes && b < a + bytes)
        return MOE_ERR_UNSUPPORTED;                       // in place or overlapping
    return from_hip(launch_pack_weights(shape->num_local_experts, N, K, shape->inter, kind == MOE_GEMM_W13_SWIGLU,
                                        wq, wq_tiled, static_cast<hipStream_t>(stream), false));
}

size_t moe_w4a4_workspace_size(const moe_shape *shape)
{
    if (check_shape_mx(shape) != MOE_OK)
        return 0;
    moe_shape s = *shape;
    s.group_size = kGroup;
    return carve_mx(s, nullptr).bytes;
}

moe_status moe_w4a4_forward(const moe_shape *shape, const uint16_t *x, const float *router_logits,
                            const uint8_t *w13_q, const uint8_t *w13_s, const uint8_t *w2_q, const uint8_t *w2_s,
                            uint16_t *out, void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status st = check_shape_mx(shape);
    if (st != MOE_OK)
        return st;
    moe_shape sh = *shape;
    sh.group_size = kGroup;                               // the shared launchers read no group size
    if (sh.num_tokens == 0)
        return MOE_OK;
    if (!x || !router_logits || !w13_q || !w13_s || !w2_q || !w2_s || !out || !workspace)
        return MOE_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w13_q, 16) || !aligned(w2_q, 16) || !aligned(w13_s, 4) ||
        !aligned(w2_s, 4) || !aligned(router_logits, 4) || !aligned(workspace, kAlign))
        return MOE_ERR_ALIGN;
    MxWorkspace mw = carve_mx(sh, workspace);
    if (workspace_bytes < mw.bytes)
        return MOE_ERR_WORKSPACE;
    const Workspace &ws = mw.base;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    const int S = sh.num_tokens * sh.top_k;
    const bool y_slot = sh.num_local_experts == sh.num_experts;
    // the gate/up GEMM; h requantized (only the R routed rows, R =
    // offsets[E_loc] on the device): in the GEMM's epilogue, or by the
    // quantize kernel after it
    const GemmLaunch g0 = layer_gemm_args(sh, MOE_GEMM_W13_SWIGLU);
    MxGemmLaunch g1{};
    g1.kind = MOE_GEMM_W13_SWIGLU;
    g1.a = mw.xq;
    g1.as = mw.xs;
    g1.a_row_index = ws.perm;
    g1.a_rows = sh.num_tokens;
    g1.top_k = sh.top_k;
    g1.offsets = ws.offsets;
    g1.num_experts = sh.num_local_experts;
    g1.wq = w13_q;
    g1.ws = w13_s;
    g1.c = ws.h;
    g1.K = g0.K;
    g1.N = g0.N;
    g1.max_rows = g0.max_rows;
    g1.expected_rows = g0.expected_rows;
    g1.w_tiled = sh.weight_layout == MOE_WEIGHTS_TILED;
    g1.cq = mw.hq;
    g1.cs = mw.hs;
    // the down GEMM: the requantized h, y bf16
    const GemmLaunch gd = layer_gemm_args(sh, MOE_GEMM_W2);
    MxGemmLaunch g2{};
    g2.kind = MOE_GEMM_W2;
    g2.a = mw.hq;
    g2.as = mw.hs;
    g2.a_rows = S;
    g2.top_k = sh.top_k;
    g2.offsets = ws.offsets;
    g2.num_experts = sh.num_local_experts;
    g2.wq = w2_q;
    g2.ws = w2_s;
    g2.c = ws.y;
    g2.c_row_index = y_slot ? ws.perm : nullptr;
    g2.K = gd.K;
    g2.N = gd.N;
    g2.max_rows = gd.max_rows;
    g2.expected_rows = gd.expected_rows;
    g2.w_tiled = sh.weight_layout == MOE_WEIGHTS_TILED;
    // Small batch (as in the W4A16 layer): the gate/up GEMM routes the tokens
    // and quantizes their x rows itself, h and y rows are the slots t*k + j,
    // no permutation; three launches.
    const moe_launch_override ov = launch_override();
    const int small_max = ov.decode_max_tokens >= 0 ? ov.decode_max_tokens : 16;
    if (sh.num_tokens <= small_max && S <= kDecMaxSlots && sh.num_experts <= 256 && mx_small_supported(g1) &&
        mx_small_supported(g2)) {
        e = launch_mx_small(g1, MxSmallSource{router_logits, sh.num_experts, sh.num_tokens, sh.expert_begin, x,
                                              ws.ids, ws.w, ws.pres}, s);
        if (e == hipSuccess)
            e = launch_mx_small(g2, MxSmallSource{nullptr, sh.num_experts, sh.num_tokens, sh.expert_begin, nullptr,
                                                  ws.ids, ws.w, ws.pres}, s);
        if (e == hipSuccess)
            e = launch_finalize(sh, ws.y, false, ws.w, ws.pres, out, false, s, true);
        return from_hip(e);
    }
    // as in the W4A16 layer: up to a few hundred tokens the gate/up GEMM
    // builds the permutation from the routing ids (no permutation launch)
    const bool perm_in_gemm = perm_in_gemm_fits(sh) && mx_gemm_ids_supported(g1, sh.num_tokens);
    if (perm_in_gemm) {
        g1.ids = ws.ids;
        g1.T = sh.num_tokens;
        g1.begin = sh.expert_begin;
        g1.counts_out = ws.counts;
        g1.offsets_out = ws.offsets;
        g1.perm_out = ws.perm;
        g1.inv_perm_out = ws.inv_perm;
    }
    // x is quantized by the routing launch (the quantize kernel's bits)
    if (perm_in_gemm) {
        e = launch_route(sh, router_logits, ws.ids, ws.w, s, x, mw.xq, mw.xs);
    } else if (route_permute_fusable(sh)) {
        e = launch_route_permute(sh, router_logits, ws.ids, ws.w, ws.counts, ws.offsets, ws.perm, ws.inv_perm, s, 0,
                                 x, mw.xq, mw.xs);
    } else {
        e = launch_route(sh, router_logits, ws.ids, ws.w, s, x, mw.xq, mw.xs);
        if (e == hipSuccess)
            e = launch_permute(sh, ws.ids, ws.counts, ws.offsets, ws.perm, ws.inv_perm, s, 0, ws.part);
    }
    if (e == hipSuccess)
        e = launch_mx_grouped_gemm(g1, s);
    if (e == hipSuccess)
        e = launch_mx_grouped_gemm(g2, s);
    if (e == hipSuccess)
        e = launch_finalize(sh, ws.y, false, ws.w, ws.inv_perm, out, false, s, y_slot);
    return from_hip(e);
}

moe_status moe_w4a16_forward_shared(const moe_shape *shape, int32_t num_shared, const uint16_t *x,
                                    const float *router_logits, const uint8_t *w13_q, const uint16_t *s13,
                                    const uint8_t *w2_q, const uint16_t *s2, const uint8_t *w13_sh,
                                    const uint16_t *s13_sh, const uint8_t *w2_sh, const uint16_t *s2_sh,
                                    uint16_t *out, void *workspace, size_t workspace_bytes, void *stream)
{
    if (num_shared < 1)
        return MOE_ERR_UNSUPPORTED;
    return forward_impl(shape, num_shared, x, router_logits, w13_q, s13, w2_q, s2, w13_sh, s13_sh, w2_sh, s2_sh, out,
                        workspace, workspace_bytes, stream);
}

}  // extern "C"

// The C ABI of include/moe.h: host-side argument checks, workspace carving and stream-ordered
// launches. Nothing here allocates device memory or synchronises the stream.
#include <mutex>
#include <string.h>

#include "kernels.h"

using namespace moe;

namespace {

constexpr int kMaxE = 1024, kMaxK = kMaxTopK, kMaxH = 16384, kMaxI = 4096, kMaxT = 1 << 20;
// (The router is the GEMV, weights read once for all tokens, up to kGemvMaxT tokens of kernels.h,
// and the bf16x3 MFMA GEMM above.)

// moe_layer takes the decode kernels up to this many tokens by default (when they fit the shape):
// the crossover measured on the 8K-prefill layer shape (H 2048, 256 experts top-8 + shared, 4-bit):
// the decode kernels win up to 6 tokens, the grouped GEMMs (on packed codes) from 7;
// moe_layer_desc.decode_max_tokens overrides it (up to 8).
constexpr int kLayerDecodeMaxT = 6;
constexpr int kDecodeMaxT = 8;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_desc(const moe_layer_desc* d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->fmt != MOE_Q8_B32 && d->fmt != MOE_Q4_B32 && d->fmt != MOE_Q2_B32) return MOE_ERR_INVALID_ARG;
    if (d->hidden < 32 || d->hidden > kMaxH || d->hidden % 32) return MOE_ERR_INVALID_ARG;
    if (d->inter < 32 || d->inter > kMaxI || d->inter % 32) return MOE_ERR_INVALID_ARG;
    if (d->shared_inter < 0 || d->shared_inter > kMaxI || d->shared_inter % 32) return MOE_ERR_INVALID_ARG;
    if (d->num_experts < 1 || d->num_experts > kMaxE) return MOE_ERR_INVALID_ARG;
    if (d->top_k < 1 || d->top_k > kMaxK || d->top_k > d->num_experts) return MOE_ERR_INVALID_ARG;
    if (d->decode_max_tokens < 0 || d->decode_max_tokens > kDecodeMaxT) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_T(int32_t T) { return (T >= 1 && T <= kMaxT) ? MOE_OK : MOE_ERR_INVALID_ARG; }

bool qmat_ok(const moe_qmat& q) { return q.codes && q.scales && aligned16(q.codes) && ((uintptr_t)q.scales & 1u) == 0; }

moe_status check_expert_weights(const moe_layer_desc* d, const moe_layer_weights* w) {
    if (!w) return MOE_ERR_INVALID_ARG;
    if (!qmat_ok(w->gate) || !qmat_ok(w->up) || !qmat_ok(w->down)) return MOE_ERR_INVALID_ARG;
    if (d->shared_inter > 0 && (!qmat_ok(w->sh_gate) || !qmat_ok(w->sh_up) || !qmat_ok(w->sh_down)))
        return MOE_ERR_INVALID_ARG;
    if (w->prefill_codes && !aligned16(w->prefill_codes)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status check_router_weights(const moe_layer_weights* w) {
    if (!w || !w->w_router || !aligned16(w->w_router)) return MOE_ERR_INVALID_ARG;
    if (w->router_bias && ((uintptr_t)w->router_bias & 3u)) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

LayerView view(const moe_layer_desc* d, const moe_layer_weights* w) {
    LayerView L;
    L.H = d->hidden; L.I = d->inter; L.E = d->num_experts; L.k = d->top_k; L.Is = d->shared_inter; L.fmt = d->fmt;
    L.w_router = w->w_router; L.bias = w->router_bias;
    L.g_codes = (const uint8_t*)w->gate.codes; L.g_scales = w->gate.scales;
    L.u_codes = (const uint8_t*)w->up.codes; L.u_scales = w->up.scales;
    L.d_codes = (const uint8_t*)w->down.codes; L.d_scales = w->down.scales;
    const bool sh = d->shared_inter > 0;
    L.sg_codes = sh ? (const uint8_t*)w->sh_gate.codes : nullptr; L.sg_scales = sh ? w->sh_gate.scales : nullptr;
    L.su_codes = sh ? (const uint8_t*)w->sh_up.codes : nullptr; L.su_scales = sh ? w->sh_up.scales : nullptr;
    L.sd_codes = sh ? (const uint8_t*)w->sh_down.codes : nullptr; L.sd_scales = sh ? w->sh_down.scales : nullptr;
    L.pk = (const uint8_t*)w->prefill_codes;
    return L;
}

LayerView shape_view(const moe_layer_desc* d) {
    LayerView L{};
    L.H = d->hidden; L.I = d->inter; L.E = d->num_experts; L.k = d->top_k; L.Is = d->shared_inter; L.fmt = d->fmt;
    return L;
}

// ------------------------------------------------------------------ workspace layouts

struct RouteWs { float* logits; float* part; };
RouteWs carve_route(const moe_layer_desc* d, int T, void* base, size_t* bytes) {
    Carve c(base);
    RouteWs r;
    r.logits = c.take<float>((size_t)T * d->num_experts);
    const size_t pb = T > kGemvMaxT ? router_scratch_bytes(T, d->hidden, d->num_experts) : 0;
    r.part = pb ? c.take<float>(pb / sizeof(float)) : nullptr;
    if (bytes) *bytes = c.bytes();
    return r;
}

struct PermWs { int32_t* chunks; };
PermWs carve_perm(const moe_layer_desc* d, int T, void* base, size_t* bytes) {
    Carve c(base);
    PermWs r;
    r.chunks = c.take<int32_t>(perm_scratch_ints(T, d->num_experts));
    if (bytes) *bytes = c.bytes();
    return r;
}

struct DecodeWs { float* h; };
DecodeWs carve_decode(const moe_layer_desc* d, int T, void* base, size_t* bytes) {
    Carve c(base);
    DecodeWs r;
    r.h = c.take<float>(decode_scratch_floats(shape_view(d), T));
    if (bytes) *bytes = c.bytes();
    return r;
}

struct PrefillWs { void* scratch; };
PrefillWs carve_prefill_ws(const moe_layer_desc* d, int T, void* base, size_t* bytes) {
    Carve c(base);
    PrefillWs r;
    r.scratch = c.take<char>(prefill_scratch_bytes(shape_view(d), T));
    if (bytes) *bytes = c.bytes();
    return r;
}

// moe_layer's regime: the decode kernels for 1 <= T <= kLayerDecodeMaxT when they fit the shape (T k
// <= 64 pairs, and their LDS holds x and every chosen pair's activations), the grouped-GEMM path
// otherwise.
bool layer_uses_decode(const moe_layer_desc* d, int T) {
    const int tmax = d->decode_max_tokens > 0 ? d->decode_max_tokens : kLayerDecodeMaxT;
    return T <= tmax && decode_fits(shape_view(d), T, true);
}

struct LayerWs {
    float* logits;
    int32_t* ids;
    float* p;
    _Float16* y_rows;    // y_sorted (prefill), [T*k][H], fp16 inside the fused layer
    _Float16* y_shared;  // [T][H]
    int32_t *offsets, *perm, *inv, *chunks;  // prefill only
    float* h;          // decode only
    void* prefill;     // prefill only
    float* router_part;  // prefill only: split-K partial sums of the router GEMM (may be null)
};
LayerWs carve_layer(const moe_layer_desc* d, int T, void* base, size_t* bytes) {
    Carve c(base);
    LayerWs r{};
    const size_t P = (size_t)T * d->top_k;
    r.logits = c.take<float>((size_t)T * d->num_experts);
    r.ids = c.take<int32_t>(P);
    r.p = c.take<float>(P);
    if (layer_uses_decode(d, T)) {
        r.h = c.take<float>(decode_scratch_floats(shape_view(d), T));
    } else {
        r.y_rows = c.take<_Float16>(P * d->hidden);
        r.y_shared = c.take<_Float16>((size_t)T * d->hidden);
        r.offsets = c.take<int32_t>((size_t)d->num_experts + 1);
        r.perm = c.take<int32_t>(P);
        r.inv = c.take<int32_t>(P);
        r.chunks = c.take<int32_t>(perm_scratch_ints(T, d->num_experts));
        r.prefill = c.take<char>(prefill_scratch_bytes(shape_view(d), T));
        const size_t pb = T > kGemvMaxT ? router_scratch_bytes(T, d->hidden, d->num_experts) : 0;
        r.router_part = pb ? c.take<float>(pb / sizeof(float)) : nullptr;
    }
    if (bytes) *bytes = c.bytes();
    return r;
}

moe_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return MOE_OK;
    if (!ws || !aligned16(ws)) return MOE_ERR_INVALID_ARG;
    return ws_bytes >= need ? MOE_OK : MOE_ERR_WORKSPACE;
}

// ------------------------------------------------------------------ static workspace

// moe_layer_static's workspace: a file-scope device array (each GPU holds its own copy from load
// until the process ends). Host code never uses the array's name as an address: its device address
// comes from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's copy of scratch (nullptr and a status on failure).
void* static_scratch(moe_status* st) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *st = MOE_ERR_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            *st = MOE_ERR_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *st = MOE_OK;
    return g_scratch_ptr[dev];
}

#define MOE_TRY(expr)                   \
    do {                                \
        moe_status _st = (expr);        \
        if (_st != MOE_OK) return _st;  \
    } while (0)

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

size_t moe_prefill_codes_bytes(const moe_layer_desc* d) {
    if (check_desc(d) != MOE_OK) return 0;
    return (size_t)packed_offsets(shape_view(d)).total;
}

moe_status moe_pack_prefill_codes(const moe_layer_desc* d, const moe_layer_weights* w, void* dst, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_expert_weights(d, w));
    if (!dst || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
    LayerView L = view(d, w);
    L.pk = nullptr;
    return launch_pack_codes(L, static_cast<uint8_t*>(dst), (hipStream_t)stream);
}

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

moe_status moe_workspace_size(const moe_layer_desc* d, int32_t T, moe_call call, size_t* bytes) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    if (!bytes) return MOE_ERR_INVALID_ARG;
    size_t b = 0;
    switch (call) {
        case MOE_CALL_ROUTE: carve_route(d, T, nullptr, &b); break;
        case MOE_CALL_PERMUTE: carve_perm(d, T, nullptr, &b); break;
        case MOE_CALL_EXPERTS_DECODE:
            if (!decode_fits(shape_view(d), T, false)) return MOE_ERR_UNSUPPORTED;
            carve_decode(d, T, nullptr, &b);
            break;
        case MOE_CALL_EXPERTS_PREFILL:
            carve_prefill_ws(d, T, nullptr, &b);
            break;
        case MOE_CALL_COMBINE: b = 0; break;
        case MOE_CALL_LAYER:
            carve_layer(d, T, nullptr, &b);
            break;
        default: return MOE_ERR_INVALID_ARG;
    }
    *bytes = b;
    return MOE_OK;
}

moe_status moe_route(const moe_layer_desc* d, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                     float* logits, int32_t* ids, float* p, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    MOE_TRY(check_router_weights(w));
    if (!x || !aligned16(x) || !ids || !p) return MOE_ERR_INVALID_ARG;
    if (logits && ((uintptr_t)logits & 3u)) return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    carve_route(d, T, nullptr, &need);
    const bool split = T > kGemvMaxT && router_scratch_bytes(T, d->hidden, d->num_experts) > 0;
    if (!logits || split) MOE_TRY(check_ws(ws, ws_bytes, need));
    const RouteWs rw = (!logits || split) ? carve_route(d, T, ws, nullptr) : RouteWs{nullptr, nullptr};
    float* lg = logits ? logits : rw.logits;
    hipStream_t s = (hipStream_t)stream;
    if (T > kGemvMaxT)
        return launch_route_topk(w->w_router, w->router_bias, x, T, d->hidden, d->num_experts, d->top_k, lg, ids, p,
                                 rw.part, s);
    MOE_TRY(launch_route_gemv(w->w_router, w->router_bias, x, T, d->hidden, d->num_experts, lg, s));
    return launch_topk(lg, T, d->num_experts, d->top_k, ids, p, s);
}

moe_status moe_permute(const moe_layer_desc* d, const int32_t* ids, int32_t T, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    if (!ids || !offsets || !perm || !inv) return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    carve_perm(d, T, nullptr, &need);
    MOE_TRY(check_ws(ws, ws_bytes, need));
    return launch_permute(ids, T, d->top_k, d->num_experts, offsets, perm, inv, carve_perm(d, T, ws, nullptr).chunks,
                          (hipStream_t)stream);
}

moe_status moe_experts_decode(const moe_layer_desc* d, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                              const int32_t* ids, float* y_pairs, float* y_shared, void* ws, size_t ws_bytes,
                              void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    if (!decode_fits(shape_view(d), T, false)) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_expert_weights(d, w));
    if (!x || !aligned16(x) || !ids || !y_pairs || !aligned16(y_pairs)) return MOE_ERR_INVALID_ARG;
    if (d->shared_inter > 0 && (!y_shared || !aligned16(y_shared))) return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    carve_decode(d, T, nullptr, &need);
    MOE_TRY(check_ws(ws, ws_bytes, need));
    const DecodeWs dw = carve_decode(d, T, ws, nullptr);
    return launch_decode_experts(view(d, w), x, T, nullptr, const_cast<int32_t*>(ids), nullptr, dw.h, nullptr, y_pairs,
                                 y_shared, (hipStream_t)stream);
}

moe_status moe_experts_prefill(const moe_layer_desc* d, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                               const int32_t* offsets, const int32_t* perm, float* y_sorted, float* y_shared, void* ws,
                               size_t ws_bytes, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    MOE_TRY(check_expert_weights(d, w));
    if (!x || !aligned16(x) || !offsets || !perm || !y_sorted) return MOE_ERR_INVALID_ARG;
    if (d->shared_inter > 0 && !y_shared) return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    carve_prefill_ws(d, T, nullptr, &need);
    MOE_TRY(check_ws(ws, ws_bytes, need));
    return launch_prefill_experts(view(d, w), x, T, offsets, perm, y_sorted, y_shared, PrefillOut::kF32,
                                  carve_prefill_ws(d, T, ws, nullptr).scratch, (hipStream_t)stream);
}

moe_status moe_experts_prefill_f16(const moe_layer_desc* d, const moe_layer_weights* w, const uint16_t* x,
                                   int32_t T, const int32_t* offsets, const int32_t* perm, uint16_t* y_sorted,
                                   uint16_t* y_shared, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    MOE_TRY(check_expert_weights(d, w));
    if (!x || !aligned16(x) || !offsets || !perm || !y_sorted || !aligned16(y_sorted)) return MOE_ERR_INVALID_ARG;
    if (d->shared_inter > 0 && (!y_shared || !aligned16(y_shared))) return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    carve_prefill_ws(d, T, nullptr, &need);
    MOE_TRY(check_ws(ws, ws_bytes, need));
    return launch_prefill_experts(view(d, w), x, T, offsets, perm, y_sorted, y_shared, PrefillOut::kF16,
                                  carve_prefill_ws(d, T, ws, nullptr).scratch, (hipStream_t)stream);
}

moe_status moe_combine(const moe_layer_desc* d, int32_t T, const float* p, const float* y_rows,
                       const int32_t* row_of_pair, const float* y_shared, float* out, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    if (!p || !y_rows || !out || !aligned16(y_rows) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if (y_shared && !aligned16(y_shared)) return MOE_ERR_INVALID_ARG;
    return launch_combine(T, d->top_k, d->hidden, p, y_rows, row_of_pair, y_shared, out, (hipStream_t)stream);
}

moe_status moe_kv_encode(const uint16_t* src, int32_t rows, int32_t D, int8_t* codes, uint16_t* scales,
                         void* stream) {
    if (rows < 0 || D < 32 || D > 65536 || D % 32 != 0) return MOE_ERR_INVALID_ARG;
    if (rows == 0) return MOE_OK;
    if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes) || ((uintptr_t)scales & 1u))
        return MOE_ERR_INVALID_ARG;
    return launch_kv_encode(src, rows, D, codes, scales, (hipStream_t)stream);
}

moe_status moe_kv_gather(const int8_t* codes, const uint16_t* scales, int32_t n_rows, int32_t D, const int32_t* idx,
                         int32_t n_idx, float* out, void* stream) {
    if (n_rows < 0 || n_idx < 0 || D < 32 || D > 65536 || D % 32 != 0) return MOE_ERR_INVALID_ARG;
    if (n_idx == 0) return MOE_OK;
    if (!idx || !out || ((uintptr_t)idx & 3u) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if (n_rows > 0 && (!codes || !scales || !aligned16(codes) || ((uintptr_t)scales & 1u)))
        return MOE_ERR_INVALID_ARG;
    return launch_kv_gather(codes, scales, n_rows, D, idx, n_idx, out, (hipStream_t)stream);
}

moe_status moe_layer(const moe_layer_desc* d, const moe_layer_weights* w, const uint16_t* x, int32_t T, float* out,
                     float* logits, int32_t* ids, float* p, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    MOE_TRY(check_router_weights(w));
    MOE_TRY(check_expert_weights(d, w));
    if (!x || !aligned16(x) || !out || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if ((logits && ((uintptr_t)logits & 3u)) || (ids && ((uintptr_t)ids & 3u)) || (p && ((uintptr_t)p & 3u)))
        return MOE_ERR_INVALID_ARG;
    size_t need = 0;
    carve_layer(d, T, nullptr, &need);
    MOE_TRY(check_ws(ws, ws_bytes, need));
    const LayerWs lw = carve_layer(d, T, ws, nullptr);
    float* lg = logits ? logits : lw.logits;
    int32_t* id = ids ? ids : lw.ids;
    float* pr = p ? p : lw.p;
    const LayerView L = view(d, w);
    hipStream_t s = (hipStream_t)stream;
    if (layer_uses_decode(d, T)) {
        MOE_TRY(launch_route_gemv(w->w_router, w->router_bias, x, T, L.H, L.E, lg, s));
        return launch_decode_experts(L, x, T, lg, id, pr, lw.h, out, nullptr, nullptr, s);
    }
    // the expert outputs between the down GEMM and the combine are fp16 rows here (half the bytes
    // of the largest stream), at each token's activation scale; the combine sums and unscales them
    // in fp32
    const _Float16* ysh = d->shared_inter > 0 ? lw.y_shared : nullptr;
    if (T <= kGemvMaxT) MOE_TRY(launch_route_gemv(w->w_router, w->router_bias, x, T, L.H, L.E, lg, s));
    if (route_small_fits(L, T)) {
        // small batches: top-k, permutation, tile list and x conversion in one kernel
        MOE_TRY(launch_route_small(L, x, T, lg, id, pr, lw.offsets, lw.perm, lw.inv, lw.prefill, s));
        MOE_TRY(launch_prefill_experts(L, x, T, lw.offsets, lw.perm, lw.y_rows, lw.y_shared, PrefillOut::kF16Scaled,
                                       lw.prefill, s, true));
    } else {
        if (T <= kGemvMaxT) MOE_TRY(launch_topk(lg, T, L.E, L.k, id, pr, s));
        else MOE_TRY(launch_route_topk(w->w_router, w->router_bias, x, T, L.H, L.E, L.k, lg, id, pr, lw.router_part, s));
        MOE_TRY(launch_permute(id, T, L.k, L.E, lw.offsets, lw.perm, lw.inv, lw.chunks, s));
        MOE_TRY(launch_prefill_experts(L, x, T, lw.offsets, lw.perm, lw.y_rows, lw.y_shared, PrefillOut::kF16Scaled,
                                       lw.prefill, s));
    }
    return launch_combine_f16(T, L.k, L.H, pr, lw.y_rows, lw.inv, ysh, prefill_token_exps(L, T, lw.prefill), out, s);
}

moe_status moe_layer_static(const moe_layer_desc* d, const moe_layer_weights* w, const uint16_t* x, int32_t T,
                            float* out, float* logits, int32_t* ids, float* p, void* stream) {
    MOE_TRY(check_desc(d));
    MOE_TRY(check_T(T));
    size_t need = 0;
    carve_layer(d, T, nullptr, &need);
    if (need > kStaticScratchBytes) return MOE_ERR_UNSUPPORTED;
    moe_status st = MOE_OK;
    void* ws = static_scratch(&st);
    if (st != MOE_OK) return st;
    return moe_layer(d, w, x, T, out, logits, ids, p, ws, kStaticScratchBytes, stream);
}

size_t moe_layer_static_max_bytes(void) { return kStaticScratchBytes; }

}  // extern "C"

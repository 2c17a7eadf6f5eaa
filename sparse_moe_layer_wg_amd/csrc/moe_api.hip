// C ABI of the MoE layer: host-side validation, workspace carving and the
// launch sequence.  Everything here runs on the host; nothing is allocated,
// copied or synchronised.
#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

#include <math.h>

#include <atomic>
#include <mutex>

// Scratch of moe_gate_noalloc, for callers that cannot allocate: a
// device-side array of the code object, so each GPU the library runs on holds
// its own copy from the module's load until the process ends.  Host code
// never uses this name as an address (on the host it is only a stand-in for
// the symbol): the device address is looked up with hipGetSymbolAddress,
// once per device, and that pointer is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

using namespace moe;

struct Plan {
    int S, d, h, E, k, C, nb;
    bool bf16;
    bool dropless;  // compact expert segments, no drops (C = S bounds every expert)
    bool reroute;   // dropped assignments offered to alternative experts
    int crows;      // rows of counts: k, or k + 1 with re-routing
    size_t rows;    // rows of the dispatch buffer / expert output: E*C or S*k
    size_t es;      // bytes per activation element
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Row of assignment (e, slot) in xd/out is e*row_stride + slot, valid for
// slot < row_limit: padded buffers [E,C,d], or compact ones where the slot is
// already the global row.
int row_stride(const Plan& p) { return p.dropless ? 0 : p.C; }
int row_limit(const Plan& p) { return p.dropless ? (int)p.rows : p.C; }

// Validates the config; fills the plan.  INVALID_ARG for values outside the
// definition, UNSUPPORTED for valid shapes the kernels do not handle.
moe_status make_plan(const moe_config* c, Plan* pl) {
    if (!c) return MOE_ERR_INVALID_ARG;
    if (c->flags & ~(MOE_CFG_DROPLESS | MOE_CFG_REROUTE)) return MOE_ERR_INVALID_ARG;
    const bool dropless = (c->flags & MOE_CFG_DROPLESS) != 0;
    const bool reroute = (c->flags & MOE_CFG_REROUTE) != 0;
    if (dropless && reroute) return MOE_ERR_INVALID_ARG;   // dropless drops nothing
    if (c->S < 0 || c->d_model < 1 || c->d_ff < 1 || c->E < 1 || c->k < 1 || c->k > c->E)
        return MOE_ERR_INVALID_ARG;
    if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (c->capacity < 0) return MOE_ERR_INVALID_ARG;
    double C;
    if (dropless) {
        // Top-k experts are distinct, so no expert receives more than S rows.
        if (c->capacity != 0) return MOE_ERR_INVALID_ARG;
        C = c->S;
    } else if (c->capacity > 0) {
        C = c->capacity;
    } else {
        if (!(c->capacity_factor > 0.0) || !isfinite(c->capacity_factor))
            return MOE_ERR_INVALID_ARG;
        // C = ceil(cf * k * S / E), evaluated left to right in fp64.
        C = ceil(c->capacity_factor * (double)c->k * (double)c->S / (double)c->E);
    }
    if (C > 2147483647.0) return MOE_ERR_UNSUPPORTED;
    if (c->E > kMaxE || c->k > kMaxK || c->k * c->E > 16384) return MOE_ERR_UNSUPPORTED;
    const bool bf16 = c->act_dtype == MOE_BF16;
    const int q = bf16 ? 64 : 4;
    if (c->d_model % q != 0 || c->d_ff % q != 0) return MOE_ERR_UNSUPPORTED;
    const double wide = (double)(c->d_model > c->d_ff ? c->d_model : c->d_ff);
    const double rows = dropless ? (double)c->S * c->k : (double)c->E * C;
    if (rows * wide >= 2147483648.0) return MOE_ERR_UNSUPPORTED;
    if ((double)c->S * wide >= 2147483648.0 || (double)c->S * c->E >= 2147483648.0)
        return MOE_ERR_UNSUPPORTED;
    // one expert's weight matrix is addressed with 32-bit byte offsets
    if ((double)c->d_model * c->d_ff * (bf16 ? 2.0 : 4.0) >= 4294967296.0)
        return MOE_ERR_UNSUPPORTED;
    pl->S = c->S;
    pl->d = c->d_model;
    pl->h = c->d_ff;
    pl->E = c->E;
    pl->k = c->k;
    pl->C = (int)C;
    pl->nb = (int)ceil_div(c->S, kTokBlock);
    pl->bf16 = bf16;
    pl->dropless = dropless;
    pl->reroute = reroute;
    pl->crows = c->k + (reroute ? 1 : 0);
    pl->rows = (size_t)rows;
    pl->es = bf16 ? 2 : 4;
    return MOE_OK;
}

// Two expert GEMMs, 8 tile counters each (one per XCD chunk).
constexpr int kTileCounters = 16;

// Workspace layout, every region 256-byte aligned:
//   [route]  logits, idx, w, slot, counts, losses, hist, ppart, zpart, psum, occ,
//            mt_start + m-tile experts, expert segment starts [E], GEMM tile
//            counters, inverse slot map [R], squared row norms of x [S] and
//            of the router weight [E]; with re-routing also the overflow
//            offers [S,k] x 2 and their tile histograms [E,k,nb]
//   [ffn]    H [R,h]
//   [layer]  one [R,d] buffer (dispatch buffer and expert output)
// with R = rows: E*C padded, S*k compact (dropless).
struct Carve {
    size_t logits, idx, w, slot, counts, losses, hist, ppart, zpart, psum, occ, mt_start, seg, ctr,
        inv, xn2, wn2, offer_e, offer_r, rhist;
    size_t route_end, H, ffn_end, xo, end;
};

size_t up(size_t v) { return (v + 255) & ~size_t(255); }

Carve carve(const Plan& p) {
    Carve c{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = up(o + bytes);
        return at;
    };
    c.logits = take((size_t)p.S * p.E * 4);
    c.idx = take((size_t)p.S * p.k * 4);
    c.w = take((size_t)p.S * p.k * 4);
    c.slot = take((size_t)p.S * p.k * 4);
    c.counts = take((size_t)p.crows * p.E * 4);
    c.losses = take(2 * 4);
    c.hist = take((size_t)p.E * p.k * p.nb * 4);
    c.ppart = take((size_t)p.nb * p.E * 4);
    c.zpart = take((size_t)p.nb * 4);
    c.psum = take((size_t)p.E * 8);
    c.occ = take((size_t)p.E * 4);
    c.mt_start = take(((size_t)p.E + 1 + mtile_table_len(p.E, p.C, p.rows)) * 4);
    c.seg = take((size_t)p.E * 4);
    c.ctr = take(kTileCounters * 4);
    c.inv = take(p.rows * 4);
    c.xn2 = take((size_t)p.S * 4);
    c.wn2 = take((size_t)p.E * 4);
    if (p.reroute) {
        c.offer_e = take((size_t)p.S * p.k * 4);
        c.offer_r = take((size_t)p.S * p.k * 4);
        c.rhist = take((size_t)p.E * p.k * p.nb * 4);
    }
    c.route_end = o;
    c.H = take(p.rows * p.h * p.es);
    c.ffn_end = o;
    c.xo = take(p.rows * p.d * p.es);
    c.end = o;
    return c;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Router margin per unit of logit scale: a top-k decision closer than
// 32 * 2^-24 * (|x_s| max_j |w_j| + max_j |b_j| / 8) is re-evaluated in fp64.
// For unit-scale rows (|x_s| about sqrt(d), |w_j| about 1) that is 32 ulps
// of 1.0 times sqrt(d), the growth of fp32 accumulation error over d terms.
constexpr float kRefineTau = 32.0f / 16777216.0f;

#define MOE_TRY(call)                                  \
    do {                                               \
        if ((call) != hipSuccess) return MOE_ERR_HIP;  \
    } while (0)

void record(hipEvent_t* ev, int i, hipStream_t st) {
    if (ev && ev[i]) (void)hipEventRecord(ev[i], st);
}

// Router + slots for a planned layer.  logits: device array (input when
// logits_in).  Writes topk_idx/topk_w/slot/counts/losses; leaves occ and
// mt_start in the workspace.
moe_status run_gate(const Plan& p, const Carve& cv, const void* x, const float* wg,
                    const float* bg, float* logits, bool logits_in, int32_t* topk_idx,
                    float* topk_w, int32_t* slot, int32_t* counts, float* losses, void* ws,
                    int32_t* inv, hipEvent_t* ev, hipStream_t st) {
    int32_t* hist = at<int32_t>(ws, cv.hist);
    float* ppart = at<float>(ws, cv.ppart);
    float* zpart = at<float>(ws, cv.zpart);
    double* psum = at<double>(ws, cv.psum);
    int32_t* occ = at<int32_t>(ws, cv.occ);
    int32_t* mt = at<int32_t>(ws, cv.mt_start);
    float* xn2 = at<float>(ws, cv.xn2);
    float* wn2 = at<float>(ws, cv.wn2);
    if (!logits_in)
        MOE_TRY(launch_gate_logits(x, p.bf16, wg, bg, logits, xn2, wn2, p.S, p.d, p.E, st));
    record(ev, 1, st);
    RouteParams rp{};
    rp.logits = logits;
    rp.x = logits_in ? nullptr : x;
    rp.x_bf16 = p.bf16;
    rp.wg = logits_in ? nullptr : wg;
    rp.bg = logits_in ? nullptr : bg;
    rp.S = p.S;
    rp.d = p.d;
    rp.E = p.E;
    rp.k = p.k;
    rp.nb = p.nb;
    rp.tau = logits_in ? 0.f : kRefineTau;
    rp.xn2 = xn2;
    rp.wn2 = wn2;
    rp.topk_idx = topk_idx;
    rp.topk_w = topk_w;
    rp.hist = hist;
    rp.ppart = ppart;
    rp.zpart = zpart;
    MOE_TRY(launch_route(rp, st));
    record(ev, 2, st);
    MOE_TRY(launch_slot_scan(hist, p.E, p.k, p.nb, p.C, counts, occ, ppart, psum, st));
    record(ev, 3, st);
    MOE_TRY(launch_positions_finalize(topk_idx, hist, p.S, p.E, p.k, p.nb, p.C, p.dropless, slot,
                                      inv, psum, zpart, counts, occ,
                                      gemm_block_m(p.bf16, p.S, p.E, p.k), losses, mt,
                                      at<int32_t>(ws, cv.seg), at<int32_t>(ws, cv.ctr),
                                      kTileCounters, st));
    if (p.reroute)
        MOE_TRY(launch_reroute(logits, topk_idx, slot, inv, counts, occ, mt,
                               at<int32_t>(ws, cv.ctr), kTileCounters, p.S, p.E, p.k, p.nb, p.C,
                               gemm_block_m(p.bf16, p.S, p.E, p.k), at<int32_t>(ws, cv.offer_e),
                               at<int32_t>(ws, cv.offer_r), at<int32_t>(ws, cv.rhist), st));
    record(ev, 4, st);
    return MOE_OK;
}

// Both expert GEMMs.  a_rows: NULL (GEMM 1 reads the dispatch buffer xd) or
// the inverse slot map (GEMM 1 gathers its rows from the token rows in xd).
// seg: the experts' first rows in compact (dropless) buffers.
moe_status run_ffn(const Plan& p, const void* xd, const int32_t* a_rows, const void* w1,
                   const void* b1, const void* w2, const void* b2, void* out, const int32_t* occ,
                   const int32_t* mt, const int32_t* seg, int32_t* ctr, void* H, hipEvent_t* ev,
                   hipStream_t st) {
    GemmParams g{};
    g.occ = occ;
    g.row0 = p.dropless ? seg : nullptr;
    g.mt_start = mt;
    g.mt_expert = mt + p.E + 1;
    g.tile_ctr = ctr;
    g.a_rows = a_rows;
    g.E = p.E;
    g.C = p.C;
    g.A = xd;
    g.B = w1;
    g.bias = b1;
    g.Cout = H;
    g.N = p.h;
    g.K = p.d;
    g.relu = true;
    MOE_TRY(launch_expert_gemm(g, p.bf16, gemm_block_m(p.bf16, p.S, p.E, p.k), st));
    record(ev, 6, st);
    g.tile_ctr = ctr + 8;
    g.a_rows = nullptr;
    g.A = H;
    g.B = w2;
    g.bias = b2;
    g.Cout = out;
    g.N = p.d;
    g.K = p.h;
    g.relu = false;
    MOE_TRY(launch_expert_gemm(g, p.bf16, gemm_block_m(p.bf16, p.S, p.E, p.k), st));
    record(ev, 7, st);
    return MOE_OK;
}

// Device address of the current device's copy of `scratch`, looked up with
// hipGetSymbolAddress the first time a device asks and kept per device.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

moe_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
                return MOE_ERR_HIP;
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return MOE_OK;
}

// moe_gate's body.  use_static: the scratch is this device's static array
// (ws ignored) and a shape whose scratch exceeds it is refused.
moe_status gate_call(const moe_config* cfg, const void* x, const float* w_gate,
                     const float* gate_bias, float* logits, int32_t* topk_idx, float* topk_w,
                     int32_t* slot, int32_t* counts, float* losses, uint32_t flags, void* ws,
                     size_t ws_bytes, bool use_static, hipStream_t stream) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s != MOE_OK) return s;
    if (flags & ~MOE_GATE_LOGITS_IN) return MOE_ERR_INVALID_ARG;
    const bool logits_in = (flags & MOE_GATE_LOGITS_IN) != 0;
    if (!counts || !losses) return MOE_ERR_INVALID_ARG;
    if (p.S > 0 && (!topk_idx || !topk_w || !slot)) return MOE_ERR_INVALID_ARG;
    if (p.S > 0 && (logits_in ? !logits : (!x || !w_gate))) return MOE_ERR_INVALID_ARG;
    if (!logits_in && (!aligned(x, 16) || !aligned(w_gate, 16))) return MOE_ERR_INVALID_ARG;
    if (p.S == 0) {
        MOE_TRY(launch_zero_outputs(counts, p.crows * p.E, losses, stream));
        return MOE_OK;
    }
    const Carve cv = carve(p);
    if (use_static) {
        if (cv.route_end > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
        s = scratch_address(&ws);
        if (s != MOE_OK) return s;
    } else {
        if (!ws || !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
        if (ws_bytes < cv.route_end) return MOE_ERR_WORKSPACE;
    }
    float* L = logits ? logits : at<float>(ws, cv.logits);
    return run_gate(p, cv, x, w_gate, gate_bias, L, logits_in, topk_idx, topk_w, slot, counts,
                    losses, ws, nullptr, nullptr, stream);
}

}  // namespace

extern "C" {

int32_t moe_capacity(const moe_config* cfg) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s == MOE_ERR_INVALID_ARG) return -1;
    if (s != MOE_OK) {
        // Valid but unsupported configs still have a capacity.
        if (cfg->flags & MOE_CFG_DROPLESS) return cfg->S;
        if (cfg->capacity > 0) return cfg->capacity;
        double C = ceil(cfg->capacity_factor * (double)cfg->k * (double)cfg->S / (double)cfg->E);
        return C > 2147483647.0 ? -1 : (int32_t)C;
    }
    return p.C;
}

int64_t moe_dispatch_rows(const moe_config* cfg) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s == MOE_ERR_INVALID_ARG) return -1;
    if (s != MOE_OK) {
        const int32_t C = moe_capacity(cfg);
        if (C < 0) return -1;
        return (cfg->flags & MOE_CFG_DROPLESS) ? (int64_t)cfg->S * cfg->k
                                               : (int64_t)cfg->E * C;
    }
    return (int64_t)p.rows;
}

moe_status moe_workspace_bytes(const moe_config* cfg, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s != MOE_OK) return s;
    *bytes = carve(p).end;
    return MOE_OK;
}

const char* moe_status_string(int32_t status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype not supported";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch failed";
        case MOE_ERR_SCRATCH_LIMIT:
            return "MOE_ERR_SCRATCH_LIMIT: shape needs more than the static scratch "
                   "(MOE_STATIC_SCRATCH_BYTES)";
        default: return "unknown moe_status";
    }
}

moe_status moe_gate(const moe_config* cfg, const void* x, const float* w_gate,
                    const float* gate_bias, float* logits, int32_t* topk_idx, float* topk_w,
                    int32_t* slot, int32_t* counts, float* losses, uint32_t flags, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
    return gate_call(cfg, x, w_gate, gate_bias, logits, topk_idx, topk_w, slot, counts, losses,
                     flags, ws, ws_bytes, false, stream);
}

moe_status moe_gate_noalloc(const moe_config* cfg, const void* x, const float* w_gate,
                            const float* gate_bias, float* logits, int32_t* topk_idx,
                            float* topk_w, int32_t* slot, int32_t* counts, float* losses,
                            uint32_t flags, hipStream_t stream) {
    return gate_call(cfg, x, w_gate, gate_bias, logits, topk_idx, topk_w, slot, counts, losses,
                     flags, nullptr, MOE_STATIC_SCRATCH_BYTES, true, stream);
}

moe_status moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                        const int32_t* slot, void* xd, hipStream_t stream) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s != MOE_OK) return s;
    if (p.S == 0) return MOE_OK;
    if (!x || !topk_idx || !slot || !xd) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(xd, 16)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_dispatch(x, topk_idx, slot, xd, p.S, p.d, p.k, p.E, row_stride(p),
                            row_limit(p), (int)p.es, stream));
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* xd, const int32_t* counts,
                          const void* w1, const void* b1, const void* w2, const void* b2,
                          void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s != MOE_OK) return s;
    if (!xd || !counts || !w1 || !w2 || !out) return MOE_ERR_INVALID_ARG;
    for (const void* q : {xd, w1, b1, w2, b2, (const void*)out})
        if (q && !aligned(q, 16)) return MOE_ERR_INVALID_ARG;
    if (p.C == 0) return MOE_OK;
    if (!ws || !aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
    const Carve cv = carve(p);
    if (ws_bytes < cv.ffn_end) return MOE_ERR_WORKSPACE;
    int32_t* occ = at<int32_t>(ws, cv.occ);
    int32_t* mt = at<int32_t>(ws, cv.mt_start);
    int32_t* ctr = at<int32_t>(ws, cv.ctr);
    int32_t* seg = at<int32_t>(ws, cv.seg);
    const int bm = gemm_block_m(p.bf16, p.S, p.E, p.k);
    MOE_TRY(launch_occupancy(counts, p.E, p.k, p.C, bm, strip_rows(bm), occ, mt,
                             p.dropless ? seg : nullptr, (int)p.rows, ctr, kTileCounters,
                             stream, p.reroute));
    return run_ffn(p, xd, nullptr, w1, b1, w2, b2, out, occ, mt, seg, ctr, at<void>(ws, cv.H),
                   nullptr, stream);
}

moe_status moe_combine(const moe_config* cfg, const void* out, const int32_t* topk_idx,
                       const int32_t* slot, const float* topk_w, void* y, hipStream_t stream) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s != MOE_OK) return s;
    if (p.S == 0) return MOE_OK;
    if (!out || !topk_idx || !slot || !topk_w || !y) return MOE_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(y, 16)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(launch_combine(out, topk_idx, slot, topk_w, y, p.S, p.d, p.k, p.E, row_stride(p),
                           row_limit(p), p.bf16, stream));
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_config* cfg, const void* x, const float* w_gate,
                             const float* gate_bias, const void* w1, const void* b1,
                             const void* w2, const void* b2, void* y, float* logits,
                             int32_t* topk_idx, float* topk_w, int32_t* slot, int32_t* counts,
                             float* losses, void* xd, void* out, void* hidden, void* ws,
                             size_t ws_bytes,
                             hipEvent_t* stage_events, hipStream_t stream) {
    Plan p;
    moe_status s = make_plan(cfg, &p);
    if (s != MOE_OK) return s;
    if (!w_gate || !w1 || !w2 || !ws) return MOE_ERR_INVALID_ARG;
    if (p.S > 0 && (!x || !y)) return MOE_ERR_INVALID_ARG;
    for (const void* q : {x, (const void*)w_gate, w1, b1, w2, b2, (const void*)y,
                          (const void*)xd, (const void*)out, (const void*)hidden})
        if (q && !aligned(q, 16)) return MOE_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
    const Carve cv = carve(p);
    if (ws_bytes < cv.end) return MOE_ERR_WORKSPACE;
    hipEvent_t* ev = stage_events;
    record(ev, 0, stream);
    if (p.S == 0) {
        MOE_TRY(launch_zero_outputs(counts, counts ? p.crows * p.E : 0, losses, stream));
        for (int i = 1; i < MOE_NUM_STAGE_EVENTS; ++i) record(ev, i, stream);
        return MOE_OK;
    }
    float* L = logits ? logits : at<float>(ws, cv.logits);
    int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, cv.idx);
    float* w = topk_w ? topk_w : at<float>(ws, cv.w);
    int32_t* sl = slot ? slot : at<int32_t>(ws, cv.slot);
    int32_t* cnt = counts ? counts : at<int32_t>(ws, cv.counts);
    float* los = losses ? losses : at<float>(ws, cv.losses);
    void* XD = xd ? xd : at<void>(ws, cv.xo);
    void* OUT = out ? out : (xd ? at<void>(ws, cv.xo) : XD);

    // Without a requested dispatch buffer (and for bf16 activations), GEMM 1
    // gathers its rows straight from x through the inverse slot map, so the
    // permute costs no separate pass over HBM.
    // (The gather offsets are 32-bit: x must stay below 4 GiB.)
    const bool fuse = xd == nullptr && p.bf16 && (size_t)p.S * p.d * p.es < ((size_t)1 << 32);
    int32_t* inv = fuse ? at<int32_t>(ws, cv.inv) : nullptr;
    s = run_gate(p, cv, x, w_gate, gate_bias, L, false, idx, w, sl, cnt, los, ws, inv, ev, stream);
    if (s != MOE_OK) return s;
    if (!fuse)
        MOE_TRY(launch_dispatch(x, idx, sl, XD, p.S, p.d, p.k, p.E, row_stride(p), row_limit(p),
                                (int)p.es, stream));
    record(ev, 5, stream);
    s = run_ffn(p, fuse ? x : XD, inv, w1, b1, w2, b2, OUT, at<int32_t>(ws, cv.occ),
                at<int32_t>(ws, cv.mt_start), at<int32_t>(ws, cv.seg), at<int32_t>(ws, cv.ctr),
                hidden ? hidden : at<void>(ws, cv.H), ev, stream);
    if (s != MOE_OK) return s;
    MOE_TRY(launch_combine(OUT, idx, sl, w, y, p.S, p.d, p.k, p.E, row_stride(p), row_limit(p),
                           p.bf16, stream));
    record(ev, 8, stream);
    return MOE_OK;
}

}  // extern "C"

namespace {

// Tile counters of the backward: GEMM 1 recompute, wgrad 2, dgrad 2, wgrad 1,
// dgrad 1 (8 each).
constexpr int kBwdCounters = 40;

// Backward workspace, every region 256-byte aligned:
//   occ [E], forward m-tile list (E+1 + table), backward m-tile list
//   (E+1 + table), seg [E], tile counters, inv [R], dw [S,k] fp32,
//   dl [S,E] fp32, router weight-gradient partials, the router dx GEMM's
//   operands and tables, H then dU [R,h], dO then dX
//   [R,d], the dispatched rows of x [R,d]   (R = rows)
struct BwdCarve {
    size_t occ, mt_fwd, mt_bwd, seg, ctr, inv, dw, dl, rgrad, H, G, X, end;
};

BwdCarve bwd_carve(const Plan& p) {
    BwdCarve c{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = up(o + bytes);
        return at;
    };
    const size_t tab = ((size_t)p.E + 1 + mtile_table_len(p.E, p.C, p.rows)) * 4;
    c.occ = take((size_t)p.E * 4);
    c.mt_fwd = take(tab);
    c.mt_bwd = take(tab);
    c.seg = take((size_t)p.E * 4);
    c.ctr = take(kBwdCounters * 4);
    c.inv = take(p.rows * 4);
    c.dw = take((size_t)p.S * p.k * 4);
    c.dl = take((size_t)p.S * p.E * 4);
    c.rgrad = take(router_grads_workspace(p.S, p.d, p.E));
    c.H = take(p.rows * p.h * 2);
    c.G = take(p.rows * p.d * 2);
    c.X = take(p.rows * p.d * 2);
    c.end = o;
    return c;
}

// The backward runs bf16 activations only, and gathers token rows of x with
// 32-bit offsets (x under 4 GiB), as the fused forward does.
moe_status bwd_plan(const moe_config* cfg, Plan* p) {
    moe_status s = make_plan(cfg, p);
    if (s != MOE_OK) return s;
    if (!p->bf16) return MOE_ERR_UNSUPPORTED;
    if ((size_t)p->S * p->d * 2 >= ((size_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_backward_workspace_bytes(const moe_config* cfg, size_t* bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    Plan p;
    moe_status s = bwd_plan(cfg, &p);
    if (s != MOE_OK) return s;
    *bytes = bwd_carve(p).end;
    return MOE_OK;
}

moe_status moe_layer_backward(const moe_config* cfg, const void* x, const float* w_gate,
                              const void* w1, const void* b1, const void* w2,
                              const float* logits, const int32_t* topk_idx, const float* topk_w,
                              const int32_t* slot, const int32_t* counts, const void* out,
                              const void* hidden, const void* dy, float g_aux, float g_z,
                              void* dx, float* dw_gate,
                              float* db_gate, void* dw1, void* db1, void* dw2, void* db2,
                              void* ws, size_t ws_bytes, hipEvent_t* stage_events,
                              hipStream_t stream) {
    Plan p;
    moe_status s = bwd_plan(cfg, &p);
    if (s != MOE_OK) return s;
    if (!w_gate || !w1 || !w2 || !dw_gate || !dw1 || !dw2 || !ws) return MOE_ERR_INVALID_ARG;
    if (p.S > 0 && (!x || !logits || !topk_idx || !topk_w || !slot || !counts || !out || !dy ||
                    !dx))
        return MOE_ERR_INVALID_ARG;
    if (!counts) return MOE_ERR_INVALID_ARG;
    if (!isfinite(g_aux) || !isfinite(g_z)) return MOE_ERR_INVALID_ARG;
    for (const void* q : {x, (const void*)w_gate, w1, b1, w2, out, hidden, dy, (const void*)dx,
                          (const void*)dw1, (const void*)db1, (const void*)dw2, (const void*)db2,
                          (const void*)dw_gate})
        if (q && !aligned(q, 16)) return MOE_ERR_INVALID_ARG;
    if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
    const BwdCarve cv = bwd_carve(p);
    if (ws_bytes < cv.end) return MOE_ERR_WORKSPACE;
    const size_t E = p.E, d = p.d, h = p.h;
    hipEvent_t* ev = stage_events;
    record(ev, 0, stream);
    if (p.S == 0) {
        // no tokens: every gradient is zero
        MOE_TRY(launch_zero_bytes(dw_gate, E * d * 4, stream));
        MOE_TRY(launch_zero_bytes(db_gate, db_gate ? E * 4 : 0, stream));
        MOE_TRY(launch_zero_bytes(dw1, E * h * d * 2, stream));
        MOE_TRY(launch_zero_bytes(db1, db1 ? E * h * 2 : 0, stream));
        MOE_TRY(launch_zero_bytes(dw2, E * d * h * 2, stream));
        MOE_TRY(launch_zero_bytes(db2, db2 ? E * d * 2 : 0, stream));
        for (int i = 1; i < MOE_NUM_BWD_EVENTS; ++i) record(ev, i, stream);
        return MOE_OK;
    }
    int32_t* occ = at<int32_t>(ws, cv.occ);
    int32_t* mt_fwd = at<int32_t>(ws, cv.mt_fwd);
    int32_t* mt_bwd = at<int32_t>(ws, cv.mt_bwd);
    int32_t* seg = at<int32_t>(ws, cv.seg);
    int32_t* ctr = at<int32_t>(ws, cv.ctr);
    int32_t* inv = at<int32_t>(ws, cv.inv);
    float* dwk = at<float>(ws, cv.dw);
    float* dl = at<float>(ws, cv.dl);
    void* H = at<void>(ws, cv.H);
    void* G = at<void>(ws, cv.G);
    const int32_t* row0 = p.dropless ? seg : nullptr;
    const int stride = row_stride(p), limit = row_limit(p);

    // occupancies, both m-tile lists, segment starts, zeroed tile counters,
    // and the inverse slot map (row -> token)
    const int bm = gemm_block_m(true, p.S, p.E, p.k);
    MOE_TRY(launch_occupancy(counts, p.E, p.k, p.C, bm, strip_rows(bm), occ, mt_fwd,
                             p.dropless ? seg : nullptr, (int)p.rows, ctr, kBwdCounters, stream,
                             p.reroute));
    MOE_TRY(launch_occupancy(counts, p.E, p.k, p.C, 256, 0, occ, mt_bwd,
                             p.dropless ? seg : nullptr, (int)p.rows, nullptr, 0, stream,
                             p.reroute));
    MOE_TRY(launch_inverse_rows(topk_idx, slot, p.S, p.k, p.E, stride, limit, inv, stream));
    // the expert rows of x, written once: dW1's K-major operand reads them
    // as plain rows (a gather there would put a dependent index load in
    // front of every row load)
    void* X = at<void>(ws, cv.X);
    MOE_TRY(launch_dispatch(x, topk_idx, slot, X, p.S, p.d, p.k, p.E, stride, limit, 2, stream));
    record(ev, 1, stream);

    // H = ReLU(x W1^T + b1): the forward's, or computed again (rows gathered
    // from x) exactly as the forward does
    const void* Hs = hidden;
    if (!hidden) {
        GemmParams g{};
        g.occ = occ;
        g.mt_start = mt_fwd;
        g.mt_expert = mt_fwd + p.E + 1;
        g.tile_ctr = ctr;
        g.a_rows = inv;
        g.row0 = row0;
        g.E = p.E;
        g.C = p.C;
        g.A = x;
        g.B = w1;
        g.bias = b1;
        g.Cout = H;
        g.N = p.h;
        g.K = p.d;
        g.relu = true;
        MOE_TRY(launch_expert_gemm(g, true, bm, stream));
        Hs = H;
    }
    record(ev, 2, stream);

    // combine and router backward
    MOE_TRY(launch_combine_bwd(dy, out, topk_idx, slot, topk_w, G, dwk, p.S, p.d, p.k, p.E, stride,
                               limit, stream));
    MOE_TRY(launch_router_bwd(logits, topk_idx, topk_w, dwk, counts, g_aux, g_z, dl, p.S, p.E, p.k,
                              p.reroute, stream));
    record(ev, 3, stream);

    BwdGemmParams b{};
    b.occ = occ;
    b.row0 = row0;
    b.E = p.E;
    b.C = p.C;
    b.rows = p.rows;
    // dW2 = dO^T H (reads H before dgrad 2 may overwrite it); db2 = column
    // sums of dO in the same pass
    b.A = G;
    b.B = Hs;
    b.b_rows = nullptr;
    b.bias_grad = db2;
    b.Cout = dw2;
    b.M = p.d;
    b.N = p.h;
    b.tile_ctr = ctr + 8;
    MOE_TRY(launch_bwd_gemm(b, true, false, stream));
    record(ev, 4, stream);
    // dU = (dO W2) * [H > 0], into H's workspace buffer (in place when H
    // was recomputed there)
    b.mt_start = mt_bwd;
    b.mt_expert = mt_bwd + p.E + 1;
    b.A = G;
    b.B = w2;
    b.mask = Hs;
    b.bias_grad = nullptr;
    b.Cout = H;
    b.N = p.h;
    b.K = p.d;
    b.tile_ctr = ctr + 16;
    MOE_TRY(launch_bwd_gemm(b, false, true, stream));
    record(ev, 5, stream);
    // dW1 = dU^T X; db1 = column sums of dU
    b.A = H;
    b.B = X;
    b.b_rows = nullptr;
    b.bias_grad = db1;
    b.mask = nullptr;
    b.Cout = dw1;
    b.M = p.h;
    b.N = p.d;
    b.tile_ctr = ctr + 24;
    MOE_TRY(launch_bwd_gemm(b, true, false, stream));
    record(ev, 6, stream);
    // dX = dU W1, over dO's buffer (dO is no longer needed)
    b.A = H;
    b.B = w1;
    b.b_rows = nullptr;
    b.bias_grad = nullptr;
    b.Cout = G;
    b.N = p.d;
    b.K = p.h;
    b.tile_ctr = ctr + 32;
    MOE_TRY(launch_bwd_gemm(b, false, false, stream));
    record(ev, 7, stream);

    // dx = dispatch backward + dl Wg; dWg = dl^T x; dbg = colsum dl
    MOE_TRY(launch_router_grads(dl, w_gate, x, G, topk_idx, slot, dx, dw_gate, db_gate, p.S, p.d,
                                p.E, p.k, stride, limit, at<void>(ws, cv.rgrad), stream));
    record(ev, 8, stream);
    return MOE_OK;
}

}  // extern "C"

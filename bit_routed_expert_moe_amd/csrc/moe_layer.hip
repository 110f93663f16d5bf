// moe_layer.hip -- host side of libmoe_layer.so: handle, validation, workspace
// layout and kernel launches behind the C ABI declared in include/moe_layer.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "moe_internal.h"
#include "../../include/moe_layer.h"

namespace moe {
hipError_t launch_route(const RouteArgs& a, int T, int act_bf16, hipStream_t s);
hipError_t launch_prep(const RouteArgs& a, int T, int act_bf16, hipStream_t s);
hipError_t launch_topk(const RouteArgs& a, int T, hipStream_t s);
hipError_t launch_gate_up(const FfnArgs& a, int T, int xparts, int n_units, hipStream_t s);
hipError_t launch_down(const FfnArgs& a, int T, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_clear_word(uint32_t* p, hipStream_t s);
hipError_t launch_fetch(const FetchArgs& f, hipStream_t s);
hipError_t launch_prefill_prep(const PrefillArgs& a, int act_bf16, hipStream_t s);
hipError_t launch_prefill_group(const PrefillArgs& a, hipStream_t s);
hipError_t launch_route_tiles(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_gate_up(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_down(const PrefillArgs& a, hipStream_t s);
hipError_t launch_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* sink, hipStream_t s);
}  // namespace moe

using namespace moe;

// HBM expert-slot cache of one layer: n_slots device records filled on a
// side stream from a pinned host pool of all E records.  LFU: every selection
// adds one to its expert's count (never decayed); a miss always enters, into a
// free slot if any (lowest index), otherwise replacing the resident expert that
// the current token did not select with the smallest count, then the least
// recently used, then the lowest slot.
struct SlotCache {
    int n_slots = 0;
    std::vector<int32_t> slot_of;     // [E], -1 when not resident
    std::vector<int32_t> expert_in;   // [n_slots], -1 when free
    std::vector<uint64_t> count;      // [E]
    std::vector<uint64_t> last_use;   // [n_slots]
    std::vector<char> pinned;         // [n_slots]
    std::vector<char> prefetched;     // [n_slots]: entered by a prefetch, not yet selected
    std::vector<char> side_writing;   // [n_slots]: a copy into the slot may be pending on `side`
    int policy = MOE_CACHE_LFU;
    uint64_t tick = 0, hits = 0, misses = 0;
    uint64_t prefetch_issued = 0, prefetch_used = 0;
    bool side_pending = false;        // prefetch copies on `side` not yet waited for
    hipStream_t side = nullptr;
    hipEvent_t ev_ids = nullptr, ev_copies = nullptr;
    hipEvent_t ev_read = nullptr;     // after the last kernels that read the slots
    bool read_recorded = false;
    int32_t* h_ids = nullptr;         // pinned staging [k]
    int32_t* h_slots = nullptr;       // pinned staging [k]
};

struct moe_layer {
    moe_layer_desc d;
    moe_layer_weights w;
    SlotCache cache;
    size_t rec_bytes;
    size_t shared_rec_bytes;
    int bits;             // code width of the expert records: 4 or 2
    size_t d_off;         // down segments of a routed record (after its gate/up segments)
    size_t d_off_shared;  // ... and of the shared record
    int NG;        // H / 64
    int blk_r;     // I / 32
    int blk_s;     // Is / 32
    int blk_max;
    int xparts;    // fp16 parts per activation: 1 for bf16, 2 for fp32
    int gi;        // input groups per routed down item
    int gis;       // input groups per shared down item
    int n_items;   // down items per output tile
    int n_otiles;  // H / 64
    int gpw_gu, gpw_dn;
    int sh_split;  // pieces per shared 32-row block (kSharedSplit or 1)
    int gpw_sh;    // input groups per wave in a shared piece
    int gu_waves;  // waves per gate/up workgroup
    int spin_limit; // fused routing: polls of the logit words before computing them locally
    // the host pool as the device addresses it (null: not mapped; misses are
    // then copied on the side stream)
    const uint8_t* host_pool_dev = nullptr;
};

namespace moe {
LaunchStamp* g_stamp = nullptr;  // see launch_kernel
}  // namespace moe

// Scratch of moe_layer_forward_noalloc: the workspace of one call, in a
// static device array (one copy per GPU, held until the process ends).  Host
// code never uses the array's name as an address: each device's copy is
// located once with hipGetSymbolAddress and that pointer is passed to the
// kernels.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

// ---- per-launch event timing (moe_profile_*) ----
enum { K_ROUTE = 0, K_PREP = 1, K_GATE_UP = 2, K_DOWN = 3, K_COMBINE = 4, K_TOPK = 5,
       K_PF_PREP = 6, K_PF_GROUP = 7, K_PF_GATE_UP = 8, K_PF_DOWN = 9, K_STREAM = 10 };
struct ProfRec {
    int kid;
    hipEvent_t a, b;
};
std::vector<ProfRec> g_prof;
size_t g_prof_n = 0;
bool g_prof_on = false;

template <typename F>
hipError_t timed(int kid, hipStream_t s, F&& launch) {
    if (!(g_prof_on && g_prof_n < g_prof.size())) return launch();
    ProfRec* r = &g_prof[g_prof_n++];
    r->kid = kid;
    LaunchStamp st{r->a, r->b, false};
    g_stamp = &st;
    hipError_t e = launch();
    g_stamp = nullptr;
    if (!st.used) {  // nothing launched: an empty interval
        (void)hipEventRecord(r->a, s);
        (void)hipEventRecord(r->b, s);
    }
    return e;
}

moe_status fail(moe_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct WsLayout {
    size_t err, flog, dctr, pred_ids, pred_w, xpairs, xK, xX, xinv, logits, hpairs, hK, hHs, hinv, dpart,
        x16, x16b, pxsum, pxinv, pair_tok, pair_slot, tiles, n_tiles, h16, phsum, phinv, eo, shp, total;
    int tile_cap;
};

// Tokens per pass of the grouped path: bounded so that every byte offset into
// the fp16 activation and h buffers fits the kernels' 32-bit buffer offsets.
int grouped_chunk(const moe_layer* L) {
    const int64_t lim = (int64_t)0x7FFFFFFF;
    const int64_t Imax = std::max(L->d.inter, L->d.shared_inter);
    int64_t c = 8192;
    c = std::min(c, lim / ((int64_t)(L->d.top_k + 1) * Imax * 2));
    c = std::min(c, lim / ((int64_t)L->xparts * L->d.hidden * 2));
    return (int)std::max<int64_t>(c, kPrefillMinTokens);
}

WsLayout ws_layout(const moe_layer* L, int T) {
    WsLayout o{};
    const int H = L->d.hidden, k = L->d.top_k;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    // counters first, at offsets and extents that depend neither on T nor on
    // the layer's shape: every call leaves them at zero, so a workspace
    // zero-filled once serves calls of any size, of any layer it is large
    // enough for
    o.err = take(4);
    o.flog = take((size_t)(kPrefillMinTokens - 1) * kMaxExperts * 4);  // fused routing's logit words
    o.dctr = take((size_t)(kPrefillMinTokens - 1) * (kMaxHidden / 64) * kCounterStride * 4);
    o.pred_ids = take((size_t)L->d.top_k * 4);  // moe_cache_prefetch's selection
    o.pred_w = take((size_t)L->d.top_k * 4);
    o.logits = take((size_t)T * L->d.n_experts * 4);
    if (T < kPrefillMinTokens) {  // per-token (decode) path
        o.xpairs = take((size_t)T * (H / 2) * L->xparts * 4);
        o.xK = take((size_t)T * L->NG * 4);
        o.xX = take((size_t)T * L->NG * 4);
        o.xinv = take((size_t)T * L->NG * 4);
        const size_t nslot = (size_t)T * (k + 1) * L->blk_max;
        o.hpairs = take(nslot * 16 * kHParts * 4);
        o.hK = take(nslot * 4);
        o.hHs = take(nslot * 4);
        o.hinv = take(nslot * 4);
        o.dpart = take((size_t)T * L->n_otiles * L->n_items * 64 * 4);
        o.shp = take((size_t)T * L->blk_s * L->sh_split * 64 * 4);
    } else {  // grouped path, one chunk of at most grouped_chunk(L) tokens at a time
        const size_t Tg = (size_t)std::min(T, grouped_chunk(L));
        const size_t P = Tg * k;
        const int Imax = std::max(L->d.inter, L->d.shared_inter);
        o.tile_cap = (int)(std::min<size_t>((size_t)L->d.n_experts, P) + (P + kTileRows - 1) / kTileRows +
                           (Tg + kTileRows - 1) / kTileRows);
        o.x16 = take((size_t)L->xparts * Tg * H * 2);
        o.x16b = take(L->bits == 2 ? (size_t)L->xparts * Tg * H * 2 : 0);  // 2-bit slot order
        o.pxsum = take(Tg * (H / 64) * 4);
        o.pxinv = take(Tg * 4);
        o.pair_tok = take(P * 4);
        o.pair_slot = take(P * 4);
        o.tiles = take((size_t)o.tile_cap * 16);
        o.n_tiles = take(4);
        o.h16 = take((P + Tg) * Imax * 2);
        o.phsum = take((P + Tg) * (Imax / 64) * 4);
        o.phinv = take((P + Tg) * (Imax / 64) * 4);
        o.eo = take(Tg * (k + 1) * H * 4);
    }
    o.total = off;
    return o;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_device_ptr(const void* p, const char* name) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(MOE_ERR_ARG, std::string(name) + " is not a HIP allocation");
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(MOE_ERR_ARG, std::string(name) + " is not device memory");
    return MOE_OK;
}

RouteArgs route_args(const moe_layer* L, const void* x, int32_t* ids, float* w, uint8_t* ws,
                     const WsLayout& o, int prep, int T) {
    RouteArgs a{};
    a.x = x;
    a.rq = L->w.router_q;
    a.rs = L->w.router_scale;
    a.logits = (float*)(ws + o.logits);
    a.ids = ids;
    a.w = w;
    a.xpairs = (uint32_t*)(ws + o.xpairs);
    a.xK = (float*)(ws + o.xK);
    a.xX = (float*)(ws + o.xX);
    a.xinv = (float*)(ws + o.xinv);
    a.H = L->d.hidden;
    a.E = L->d.n_experts;
    a.k = L->d.top_k;
    a.prep = prep;
    a.T = T;
    a.gate = L->d.gate_fn == MOE_SIGMOID_TOPK ? 1 : 0;
    a.bias = L->w.selection_bias;
    a.rscale = L->d.routed_scale > 0.0f ? L->d.routed_scale : 1.0f;
    a.bits = L->bits;
    return a;
}

FfnArgs ffn_args(const moe_layer* L, const int32_t* ids, const float* w, uint8_t* ws,
                 const WsLayout& o, float* y, float* eo, bool select) {
    FfnArgs a{};
    if (select) {  // k_gate_up selects from the logits and writes ids/w itself
        a.logits = (const float*)(ws + o.logits);
        a.ids_out = const_cast<int32_t*>(ids);
        a.w_out = const_cast<float*>(w);
    }
    a.gate = L->d.gate_fn == MOE_SIGMOID_TOPK ? 1 : 0;
    a.bias = L->w.selection_bias;
    a.rscale = L->d.routed_scale > 0.0f ? L->d.routed_scale : 1.0f;
    a.experts = L->w.experts;
    a.shared = L->w.shared;
    a.rec_bytes = L->rec_bytes;
    a.bits = L->bits;
    a.d_off = L->d_off;
    a.d_off_shared = L->d_off_shared;
    if (L->cache.n_slots) {
        a.slots = L->w.slots;
    }
    a.ids = ids;
    a.w = w;
    a.xpairs = (const uint32_t*)(ws + o.xpairs);
    a.xK = (const float*)(ws + o.xK);
    a.xX = (const float*)(ws + o.xX);
    a.xinv = (const float*)(ws + o.xinv);
    a.hpairs = (uint32_t*)(ws + o.hpairs);
    a.hK = (float*)(ws + o.hK);
    a.hHs = (float*)(ws + o.hHs);
    a.hinv = (float*)(ws + o.hinv);
    a.dpart = (float*)(ws + o.dpart);
    a.n_units = L->d.top_k * L->blk_r + L->sh_split * L->blk_s;
    a.shp = (float*)(ws + o.shp);
    a.sh_split = L->sh_split;
    a.gpw_sh = L->gpw_sh;
    a.dctr = (uint32_t*)(ws + o.dctr);
    a.y = y;
    a.eo = eo;
    a.err = (uint32_t*)(ws + o.err);
    a.H = L->d.hidden;
    a.I = L->d.inter;
    a.Is = L->d.shared_inter;
    a.E = L->d.n_experts;
    a.k = L->d.top_k;
    a.blk_r = L->blk_r;
    a.blk_s = L->blk_s;
    a.blk_max = L->blk_max;
    a.gpw_gu = L->gpw_gu;
    a.gu_waves = L->gu_waves;
    a.n_otiles = L->n_otiles;
    a.n_items = L->n_items;
    a.gi = L->gi;
    a.gis = L->gis;
    a.gpw_dn = L->gpw_dn;
    return a;
}

PrefillArgs prefill_args(const moe_layer* L, const void* x, const int32_t* ids, uint8_t* ws,
                         const WsLayout& o, int T, float* eo) {
    PrefillArgs a{};
    a.x = x;
    a.ids = ids;
    a.experts = L->w.experts;
    a.shared = L->w.shared;
    a.rec_bytes = L->rec_bytes;
    a.rec_bytes_shared = L->shared_rec_bytes;
    a.x16 = (uint16_t*)(ws + o.x16);
    a.x16b = (uint16_t*)(ws + o.x16b);
    a.bits = L->bits;
    a.d_off = L->d_off;
    a.d_off_shared = L->d_off_shared;
    a.xsum = (float*)(ws + o.pxsum);
    a.xinv = (float*)(ws + o.pxinv);
    a.pair_tok = (int32_t*)(ws + o.pair_tok);
    a.pair_slot = (int32_t*)(ws + o.pair_slot);
    a.tiles = (int4*)(ws + o.tiles);
    a.n_tiles = (int32_t*)(ws + o.n_tiles);
    a.h16 = (uint16_t*)(ws + o.h16);
    a.hsum = (float*)(ws + o.phsum);
    a.hinv = (float*)(ws + o.phinv);
    a.eo = eo;
    a.err = (uint32_t*)(ws + o.err);
    a.H = L->d.hidden;
    a.E = L->d.n_experts;
    a.I = L->d.inter;
    a.Is = L->d.shared_inter;
    a.k = L->d.top_k;
    a.T = T;
    a.P = T * L->d.top_k;
    a.Imax = std::max(L->d.inter, L->d.shared_inter);
    a.tile_cap = o.tile_cap;
    a.xparts = L->xparts;
    a.rq = L->w.router_q;
    a.rs = L->w.router_scale;
    a.logits = (float*)(ws + o.logits);
    return a;
}

// The grouped path over T tokens in chunks.  With `route`, each chunk is
// routed first (prepared activations -> router tiles -> top-k into ids, w);
// with `ffn`, the experts run: expert_out given -> per-slot outputs written
// there; else each chunk's outputs go to the workspace and are combined into
// y with w.
moe_status grouped_ffn(const moe_layer* L, const void* x, int T, int32_t* ids, float* w, float* y,
                       float* expert_out, uint8_t* ws, const WsLayout& o, hipStream_t s, bool route,
                       bool ffn) {
    const int H = L->d.hidden, k = L->d.top_k, C = grouped_chunk(L);
    const size_t esz = L->d.act_dtype == MOE_BF16 ? 2 : 4;
    hipError_t e;
    for (int c0 = 0; c0 < T; c0 += C) {
        const int Tc = std::min(C, T - c0);
        const void* xc = (const uint8_t*)x + (size_t)c0 * H * esz;
        int32_t* ic = ids + (size_t)c0 * k;
        float* eo = expert_out ? expert_out + (size_t)c0 * (k + 1) * H : (float*)(ws + o.eo);
        const PrefillArgs pa = prefill_args(L, xc, ic, ws, o, Tc, eo);
        if ((e = timed(K_PF_PREP, s, [&] { return launch_prefill_prep(pa, L->d.act_dtype == MOE_BF16, s); })) != hipSuccess)
            return hip_fail(e, "prefill prep launch");
        if (route) {
            if ((e = timed(K_ROUTE, s, [&] { return launch_route_tiles(pa, s); })) != hipSuccess)
                return hip_fail(e, "router launch");
            RouteArgs ra = route_args(L, xc, ic, w + (size_t)c0 * k, ws, o, 0, Tc);
            if ((e = timed(K_TOPK, s, [&] { return launch_topk(ra, Tc, s); })) != hipSuccess)
                return hip_fail(e, "top-k launch");
        }
        if (!ffn) continue;
        if ((e = timed(K_PF_GROUP, s, [&] { return launch_prefill_group(pa, s); })) != hipSuccess)
            return hip_fail(e, "grouping launch");
        if ((e = timed(K_PF_GATE_UP, s, [&] { return launch_prefill_gate_up(pa, s); })) != hipSuccess)
            return hip_fail(e, "grouped gate/up launch");
        if ((e = timed(K_PF_DOWN, s, [&] { return launch_prefill_down(pa, s); })) != hipSuccess)
            return hip_fail(e, "grouped down launch");
        if (!expert_out) {
            CombineArgs ca{eo, w + (size_t)c0 * k, y + (size_t)c0 * H, H, k, Tc, 0};
            if ((e = timed(K_COMBINE, s, [&] { return launch_combine(ca, s); })) != hipSuccess)
                return hip_fail(e, "combine launch");
        }
    }
    return MOE_OK;
}

// The per-token FFN: gate/up units [first, first + n), then the down stage
// that writes y and/or the per-slot outputs.
hipError_t decode_units(const moe_layer* L, const FfnArgs& fa, int T, int first, int n, hipStream_t s) {
    FfnArgs a = fa;
    a.unit_offset = first;
    return timed(K_GATE_UP, s, [&] { return launch_gate_up(a, T, L->xparts, n, s); });
}

hipError_t decode_finish(const FfnArgs& fa, int T, hipStream_t s) {
    return timed(K_DOWN, s, [&] { return launch_down(fa, T, s); });
}

// Routing inside the gate/up launch: when the gate/up units first read the
// router units' logit words, in ticks of the 100 MHz device clock after they
// start.  Reading the words before the router units have stored them delays
// the hand-off by about 1 us (a re-read waits behind the weight streams that
// have started meanwhile), and each tick past the router units' span is lost,
// so the first read waits for about that span: 1.5 us plus 0.25 us per round
// of 16-byte router loads per lane (hidden / 1024).  The router units run in
// parallel, one row per wave, so the expert count hardly matters.  Measured
// best delays: hidden 256 (32 experts) 160 ticks, 2816 (128) 220, 4096 (256
// and 1024) 220-300; the rule gives 175, 225 and 250.
int logit_delay_ticks(const moe_layer_desc& d) {
    const int rounds = (d.hidden + 1023) / 1024;
    return 150 + 25 * rounds;
}

moe_status check_call(const moe_layer* L, const void* x, int32_t T, const void* ws) {
    if (!L) return fail(MOE_ERR_ARG, "null layer handle");
    if (!x) return fail(MOE_ERR_ARG, "null activations");
    if (!ws) return fail(MOE_ERR_ARG, "null workspace");
    if (T <= 0 || T > (1 << 20)) return fail(MOE_ERR_ARG, "n_tokens out of range");
    if (!aligned(x, 16) || !aligned(ws, 256)) return fail(MOE_ERR_ALIGN, "x needs 16-byte and workspace 256-byte alignment");
    return MOE_OK;
}

// The slot to evict: a resident expert that is neither pinned nor among the
// `n` ids in `keep`; LFU: smallest count, then least recently used, then
// lowest slot; LRU: least recently used, then lowest slot.  -1 if none.
int victim_slot(const SlotCache& c, const int32_t* keep, int n) {
    int slot = -1;
    for (int q = 0; q < c.n_slots; ++q) {
        const int r = c.expert_in[q];
        if (r < 0 || c.pinned[q]) continue;
        bool kept = false;
        for (int jj = 0; jj < n; ++jj) kept |= keep[jj] == r;
        if (kept) continue;
        if (slot < 0) {
            slot = q;
            continue;
        }
        const int rs = c.expert_in[slot];
        const bool better = c.policy == MOE_CACHE_LRU
                                ? c.last_use[q] < c.last_use[slot]
                                : (c.count[r] < c.count[rs] ||
                                   (c.count[r] == c.count[rs] && c.last_use[q] < c.last_use[slot]));
        if (better) slot = q;
    }
    return slot;
}

// Routed + shared FFN of one decode token through the slot cache.  ids are on
// the device (written earlier on `s`).  They are copied to pinned host memory,
// and the shared expert's gate/up units are queued before the host waits for
// them: those need no selection, so they run meanwhile.  The host then
// updates the policy's state, has the missing records copied into their slots
// (k_fetch on `s`, or copies on the side stream behind pending prefetches),
// and queues the routed gate/up and the down kernel behind the copies.
// ev_ids marks the point after every earlier reader of the slots: copies on
// the side stream wait for it.
moe_status cached_ffn(moe_layer* L, const int32_t* ids, FfnArgs fa, const WsLayout& o,
                      uint8_t* ws, hipStream_t s) {
    SlotCache& c = L->cache;
    const int k = L->d.top_k;
    const int routed_units = k * L->blk_r;
    hipError_t e = hipMemcpyAsync(c.h_ids, ids, sizeof(int32_t) * k, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(c.ev_ids, s);
    if (e != hipSuccess) return hip_fail(e, "reading the selected experts");
    if ((e = decode_units(L, fa, 1, routed_units, L->sh_split * L->blk_s, s)) != hipSuccess)
        return hip_fail(e, "gate/up launch");
    if ((e = hipEventSynchronize(c.ev_ids)) != hipSuccess) return hip_fail(e, "reading the selected experts");
    ++c.tick;
    for (int j = 0; j < k; ++j) {
        const int ex = c.h_ids[j];
        if (ex < 0 || ex >= L->d.n_experts)
            return fail(MOE_ERR_ARG, "selected expert id out of range");
    }
    bool copies = false;
    // misses copied by a kernel on `s` when the pool is device-mapped, except
    // into a slot that a pending side-stream copy may still be writing (a
    // prefetched expert evicted before use): that miss goes to the side
    // stream, behind the copy
    FetchArgs fetch{};
    fetch.src = L->host_pool_dev;
    fetch.dst = L->w.slots;
    fetch.rec_bytes = L->rec_bytes;
    for (int j = 0; j < k; ++j) {
        const int ex = c.h_ids[j];
        c.count[ex] += 1;
        int slot = c.slot_of[ex];
        if (slot >= 0) {
            ++c.hits;
            if (c.prefetched[slot]) {
                ++c.prefetch_used;
                c.prefetched[slot] = 0;
            }
        } else {
            ++c.misses;
            for (int q = 0; q < c.n_slots && slot < 0; ++q)
                if (c.expert_in[q] < 0) slot = q;
            if (slot < 0) {
                slot = victim_slot(c, c.h_ids, k);
                c.slot_of[c.expert_in[slot]] = -1;
            }
            c.expert_in[slot] = ex;
            c.slot_of[ex] = slot;
            c.prefetched[slot] = 0;
            if (L->host_pool_dev && !c.side_writing[slot]) {
                fetch.src_rec[fetch.n] = ex;
                fetch.dst_slot[fetch.n] = slot;
                ++fetch.n;
            } else {
                if (!copies) {  // the side stream must not overwrite a slot still being read
                    if ((e = hipStreamWaitEvent(c.side, c.ev_ids, 0)) != hipSuccess)
                        return hip_fail(e, "side stream wait");
                    copies = true;
                }
                e = hipMemcpyAsync(L->w.slots + (size_t)slot * L->rec_bytes,
                                   L->w.host_pool + (size_t)ex * L->rec_bytes, L->rec_bytes,
                                   hipMemcpyHostToDevice, c.side);
                if (e != hipSuccess) return hip_fail(e, "expert copy into its slot");
            }
        }
        c.last_use[slot] = c.tick;
        c.h_slots[j] = slot;
    }
    for (int j = 0; j < k; ++j) fa.slot_of[j] = c.h_slots[j];  // by value: no copy to the device
    if (fetch.n && (e = launch_fetch(fetch, s)) != hipSuccess) return hip_fail(e, "expert fetch launch");
    if (copies || c.side_pending) {  // this call's copies and any earlier prefetch copies
        if ((e = hipEventRecord(c.ev_copies, c.side)) != hipSuccess ||
            (e = hipStreamWaitEvent(s, c.ev_copies, 0)) != hipSuccess)
            return hip_fail(e, "copy ordering");
        c.side_pending = false;
        std::fill(c.side_writing.begin(), c.side_writing.end(), 0);
    }
    if ((e = decode_units(L, fa, 1, 0, routed_units, s)) != hipSuccess)
        return hip_fail(e, "gate/up launch");
    if ((e = decode_finish(fa, 1, s)) != hipSuccess) return hip_fail(e, "down launch");
    if ((e = hipEventRecord(c.ev_read, s)) != hipSuccess) return hip_fail(e, "slot read ordering");
    c.read_recorded = true;
    return MOE_OK;
}

// Slots for the predicted experts pred[0..n) (host), their copies on the side
// stream once the kernels that last read this layer's slots have finished
// (later work on the caller's stream, such as other layers, is not waited for).
moe_status prefetch_place(moe_layer* L, const int32_t* pred, int n) {
    SlotCache& c = L->cache;
    bool waited = false;
    for (int j = 0; j < n; ++j) {
        const int ex = pred[j];
        if (c.slot_of[ex] >= 0) continue;
        int slot = -1;
        for (int q = 0; q < c.n_slots && slot < 0; ++q)
            if (c.expert_in[q] < 0) slot = q;
        if (slot < 0) {
            slot = victim_slot(c, pred, n);
            if (slot < 0) break;  // every other slot pinned or predicted
            c.slot_of[c.expert_in[slot]] = -1;
        }
        c.expert_in[slot] = ex;
        c.slot_of[ex] = slot;
        c.prefetched[slot] = 1;
        c.last_use[slot] = c.tick;
        hipError_t e = hipSuccess;
        if (!waited) {  // a slot being replaced may still be read by this layer's last call
            if (c.read_recorded && (e = hipStreamWaitEvent(c.side, c.ev_read, 0)) != hipSuccess)
                return hip_fail(e, "side stream wait");
            waited = true;
        }
        // DMA copies: they run beside the other layers' kernels without
        // taking CUs (a copy kernel there slowed those kernels down)
        e = hipMemcpyAsync(L->w.slots + (size_t)slot * L->rec_bytes,
                           L->w.host_pool + (size_t)ex * L->rec_bytes, L->rec_bytes,
                           hipMemcpyHostToDevice, c.side);
        if (e != hipSuccess) return hip_fail(e, "prefetch copy into its slot");
        ++c.prefetch_issued;
        c.side_pending = true;
        c.side_writing[slot] = 1;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_expert_record_bytes(int32_t hidden, int32_t inter) {
    return moe_expert_record_bytes_bits(hidden, inter, 4);
}

size_t moe_expert_record_bytes_bits(int32_t hidden, int32_t inter, int32_t bits) {
    if (hidden <= 0 || inter <= 0 || hidden % 64 || inter % 64 || (bits != 4 && bits != 2)) return 0;
    // codes (bits/8 bytes per weight) + one fp16 (scale, bias) pair per 64 weights
    return (size_t)(bits == 4 ? 27 : 15) * hidden * inter / 16;
}

moe_status moe_layer_create(const moe_layer_desc* desc, const moe_layer_weights* w,
                            moe_layer_t* out) {
    if (!desc || !w || !out) return fail(MOE_ERR_ARG, "null argument");
    *out = nullptr;
    const moe_layer_desc& d = *desc;
    if (d.group != 64) return fail(MOE_ERR_SHAPE, "group must be 64");
    if (d.hidden <= 0 || d.hidden % 64 || d.hidden > kMaxHidden)
        return fail(MOE_ERR_SHAPE, "hidden must be a positive multiple of 64, at most 8192");
    if (d.inter <= 0 || d.inter % 64 || d.inter > 64 * kMaxDownGroups)
        return fail(MOE_ERR_SHAPE, "inter must be a positive multiple of 64, at most 4096");
    if (d.shared_inter < 0 || d.shared_inter % 64 || d.shared_inter > 16384)
        return fail(MOE_ERR_SHAPE, "shared_inter must be 0 or a multiple of 64, at most 16384");
    if (d.n_experts < 1 || d.n_experts > kMaxExperts)
        return fail(MOE_ERR_SHAPE, "n_experts must be in 1..1024");
    if (d.top_k < 1 || d.top_k > kMaxTopK || d.top_k > d.n_experts)
        return fail(MOE_ERR_SHAPE, "top_k must be in 1..min(16, n_experts)");
    if (d.act_dtype != MOE_F32 && d.act_dtype != MOE_BF16)
        return fail(MOE_ERR_ARG, "act_dtype must be MOE_F32 or MOE_BF16");
    if (d.gate_fn != MOE_SOFTMAX_TOPK && d.gate_fn != MOE_SIGMOID_TOPK)
        return fail(MOE_ERR_ARG, "gate_fn must be MOE_SOFTMAX_TOPK or MOE_SIGMOID_TOPK");
    if (!(d.routed_scale >= 0.0f) || !(d.routed_scale < 3.0e38f))
        return fail(MOE_ERR_ARG, "routed_scale must be finite and >= 0");
    if (d.gate_fn == MOE_SOFTMAX_TOPK && d.routed_scale != 0.0f && d.routed_scale != 1.0f)
        return fail(MOE_ERR_ARG, "routed_scale applies to MOE_SIGMOID_TOPK only");
    if (d.gate_fn == MOE_SOFTMAX_TOPK && w->selection_bias)
        return fail(MOE_ERR_ARG, "selection_bias applies to MOE_SIGMOID_TOPK only");
    if (w->selection_bias && !aligned(w->selection_bias, 4))
        return fail(MOE_ERR_ALIGN, "selection_bias needs 4-byte alignment");
    if (d.n_slots < 0 || d.n_slots > (1 << 20)) return fail(MOE_ERR_SHAPE, "bad n_slots");
    if (d.n_slots > 0 && d.n_slots < d.top_k)
        return fail(MOE_ERR_SHAPE, "n_slots must be at least top_k");
    if (d.cache_policy != MOE_CACHE_LFU && d.cache_policy != MOE_CACHE_LRU)
        return fail(MOE_ERR_ARG, "cache_policy must be MOE_CACHE_LFU or MOE_CACHE_LRU");
    if (d.n_slots == 0 && d.cache_policy != MOE_CACHE_LFU)
        return fail(MOE_ERR_ARG, "cache_policy applies to a slot cache only");
    if (d.bits != 0 && d.bits != 4 && d.bits != 2) return fail(MOE_ERR_ARG, "bits must be 4 or 2 (0 reads as 4)");
    if (d.n_slots == 0 && (w->host_pool || w->slots))
        return fail(MOE_ERR_ARG, "host_pool/slots must be NULL when n_slots = 0");
    if (d.n_slots > 0 && (!w->host_pool || !w->slots))
        return fail(MOE_ERR_ARG, "n_slots > 0 needs host_pool and slots");
    if (!w->router_q || !w->router_scale || (!w->experts && d.n_slots == 0))
        return fail(MOE_ERR_ARG, "router_q, router_scale and experts are required");
    if ((w->slots && !aligned(w->slots, 16)) || (w->host_pool && !aligned(w->host_pool, 16)))
        return fail(MOE_ERR_ALIGN, "slots and host_pool need 16-byte alignment");
    if ((d.shared_inter > 0) != (w->shared != nullptr))
        return fail(MOE_ERR_ARG, "shared must be given exactly when shared_inter > 0");
    if (!aligned(w->router_q, 16) || (w->experts && !aligned(w->experts, 16)) ||
        (w->shared && !aligned(w->shared, 16)) || !aligned(w->router_scale, 2))
        return fail(MOE_ERR_ALIGN, "router_q, experts and shared need 16-byte alignment");
    moe_status st;
    if ((st = check_device_ptr(w->router_q, "router_q")) != MOE_OK) return st;
    if ((st = check_device_ptr(w->router_scale, "router_scale")) != MOE_OK) return st;
    if (w->experts && (st = check_device_ptr(w->experts, "experts")) != MOE_OK) return st;
    if (w->shared && (st = check_device_ptr(w->shared, "shared")) != MOE_OK) return st;
    if (w->slots && (st = check_device_ptr(w->slots, "slots")) != MOE_OK) return st;
    if (w->selection_bias && (st = check_device_ptr(w->selection_bias, "selection_bias")) != MOE_OK)
        return st;
    const uint8_t* host_pool_dev = nullptr;
    if (w->host_pool) {
        hipPointerAttribute_t attr;
        if (hipPointerGetAttributes(&attr, w->host_pool) != hipSuccess ||
            attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return fail(MOE_ERR_NOT_PINNED, "host_pool must be page-locked host memory (hipHostMalloc)");
        }
        host_pool_dev = (const uint8_t*)attr.devicePointer;
    }

    moe_layer* L = new (std::nothrow) moe_layer();
    if (!L) return fail(MOE_ERR_NOMEM, "host allocation failed");
    L->d = d;
    L->w = *w;
    L->host_pool_dev = host_pool_dev;
    L->bits = d.bits == 2 ? 2 : 4;
    L->rec_bytes = moe_expert_record_bytes_bits(d.hidden, d.inter, L->bits);
    L->shared_rec_bytes = d.shared_inter ? moe_expert_record_bytes_bits(d.hidden, d.shared_inter, L->bits) : 0;
    // gate/up segments first: (I/32) blocks x (H/64) groups, each segment the
    // group's codes (64 rows x 64 inputs) and its 64 (scale, bias) pairs
    const size_t seg = (size_t)64 * 64 * L->bits / 8 + 256;
    L->d_off = (size_t)(d.inter / 32) * (d.hidden / 64) * seg;
    L->d_off_shared = (size_t)(d.shared_inter / 32) * (d.hidden / 64) * seg;
    L->NG = d.hidden / 64;
    L->blk_r = d.inter / 32;
    L->blk_s = d.shared_inter / 32;
    L->blk_max = std::max(L->blk_r, L->blk_s);
    L->xparts = d.act_dtype == MOE_F32 ? 2 : 1;
    L->gi = d.inter / 64;
    const int sg = d.shared_inter / 64;
    L->gis = std::max(L->gi, (sg + kMaxSharedItems - 1) / kMaxSharedItems);
    L->n_items = d.top_k + (sg + L->gis - 1) / L->gis;
    L->gpw_dn = (std::max(L->gi, L->gis) + kWaves - 1) / kWaves;
    L->n_otiles = d.hidden / 64;
    L->gu_waves = d.hidden <= kGuSmallHMax ? kGuWavesSmallH : kGuWavesLargeH;
    L->spin_limit = kRouteSpinLimit;
    if (const char* sl = std::getenv("MOE_ROUTE_SPIN_LIMIT")) {  // test hook: -1 computes the logits locally
        char* end = nullptr;
        const long v = std::strtol(sl, &end, 10);
        if (end != sl && *end == '\0' && v >= -1 && v <= kRouteSpinLimit) L->spin_limit = (int)v;
    }
    L->gpw_gu = (L->NG + L->gu_waves - 1) / L->gu_waves;
    // the shared blocks in slices of H where the units have 4 waves; the piece
    // counts reuse the down stage's arrival counters ([T][n_otiles] of them)
    {
        const int per_wave = ((L->NG + kSharedSplit - 1) / kSharedSplit + L->gu_waves - 1) / L->gu_waves;
        const bool split = L->gu_waves == kGuWavesLargeH && L->blk_s > 0 && L->blk_s <= kMaxHidden / 64 &&
                           per_wave <= kPieceMaxGroups;
        L->sh_split = split ? kSharedSplit : 1;
        L->gpw_sh = split ? per_wave : 0;
    }
    if (L->gpw_gu > kMaxGateUpGroupsPerWave || std::max(L->gi, L->gis) > kMaxDownGroups) {
        delete L;
        return fail(MOE_ERR_SHAPE, "shape exceeds the kernels' per-wave register tiles");
    }
    if (d.n_slots > 0) {
        SlotCache& c = L->cache;
        c.n_slots = d.n_slots;
        c.slot_of.assign(d.n_experts, -1);
        c.expert_in.assign(d.n_slots, -1);
        c.count.assign(d.n_experts, 0);
        c.last_use.assign(d.n_slots, 0);
        c.pinned.assign(d.n_slots, 0);
        c.prefetched.assign(d.n_slots, 0);
        c.side_writing.assign(d.n_slots, 0);
        c.policy = d.cache_policy;
        hipError_t e = hipStreamCreateWithFlags(&c.side, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c.ev_ids, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c.ev_copies, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c.ev_read, hipEventDisableTiming);
        if (e == hipSuccess) e = hipHostMalloc((void**)&c.h_ids, sizeof(int32_t) * d.top_k, 0);
        if (e == hipSuccess) e = hipHostMalloc((void**)&c.h_slots, sizeof(int32_t) * d.top_k, 0);
        if (e != hipSuccess) {
            moe_layer_destroy(L);
            return hip_fail(e, "slot cache setup");
        }
    }
    *out = L;
    return MOE_OK;
}

moe_status moe_layer_destroy(moe_layer_t layer) {
    if (!layer) return fail(MOE_ERR_ARG, "null layer handle");
    SlotCache& c = layer->cache;
    if (c.side) (void)hipStreamSynchronize(c.side);
    if (c.h_ids) (void)hipHostFree(c.h_ids);
    if (c.h_slots) (void)hipHostFree(c.h_slots);
    if (c.ev_ids) (void)hipEventDestroy(c.ev_ids);
    if (c.ev_copies) (void)hipEventDestroy(c.ev_copies);
    if (c.ev_read) (void)hipEventDestroy(c.ev_read);
    if (c.side) (void)hipStreamDestroy(c.side);
    delete layer;
    return MOE_OK;
}

size_t moe_workspace_bytes(moe_layer_t layer, int32_t n_tokens) {
    if (!layer || n_tokens <= 0) return 0;
    return ws_layout(layer, n_tokens).total;
}

moe_status moe_route_topk(moe_layer_t L, const void* x, int32_t T, int32_t* ids, float* w,
                          void* workspace, void* stream) {
    moe_status st = check_call(L, x, T, workspace);
    if (st != MOE_OK) return st;
    if (!ids || !w) return fail(MOE_ERR_ARG, "null ids or w");
    const WsLayout o = ws_layout(L, T);
    hipStream_t s = (hipStream_t)stream;
    if (T >= kPrefillMinTokens)  // the grouped path's router (MFMA tiles), as the forward call
        return grouped_ffn(L, x, T, ids, w, nullptr, nullptr, (uint8_t*)workspace, o, s, true, false);
    RouteArgs a = route_args(L, x, ids, w, (uint8_t*)workspace, o, 0, T);
    hipError_t e = timed(K_ROUTE, s, [&] { return launch_route(a, T, L->d.act_dtype == MOE_BF16, s); });
    if (e != hipSuccess) return hip_fail(e, "router launch");
    e = timed(K_TOPK, s, [&] { return launch_topk(a, T, s); });
    return e == hipSuccess ? MOE_OK : hip_fail(e, "top-k launch");
}

moe_status moe_expert_ffn(moe_layer_t L, const void* x, int32_t T, const int32_t* ids,
                          void* workspace, float* expert_out, void* stream) {
    moe_status st = check_call(L, x, T, workspace);
    if (st != MOE_OK) return st;
    if (L->cache.n_slots && T != 1) return fail(MOE_ERR_STATE, "the slot cache runs one token per call");
    if (!ids || !expert_out) return fail(MOE_ERR_ARG, "null ids or expert_out");
    const WsLayout o = ws_layout(L, T);
    uint8_t* ws = (uint8_t*)workspace;
    hipStream_t s = (hipStream_t)stream;
    if (T >= kPrefillMinTokens) {
        return grouped_ffn(L, x, T, const_cast<int32_t*>(ids), nullptr, nullptr, expert_out, ws, o, s,
                           false, true);
    }
    RouteArgs ra = route_args(L, x, nullptr, nullptr, ws, o, 1, T);
    hipError_t e = timed(K_PREP, s, [&] { return launch_prep(ra, T, L->d.act_dtype == MOE_BF16, s); });
    if (e != hipSuccess) return hip_fail(e, "prep launch");
    FfnArgs fa = ffn_args(L, ids, nullptr, ws, o, nullptr, expert_out, false);
    if (L->cache.n_slots) return cached_ffn(L, ids, fa, o, ws, s);
    if ((e = decode_units(L, fa, T, 0, fa.n_units, s)) != hipSuccess) return hip_fail(e, "gate/up launch");
    if ((e = decode_finish(fa, T, s)) != hipSuccess) return hip_fail(e, "down launch");
    return MOE_OK;
}

moe_status moe_combine(moe_layer_t L, const float* expert_out, const float* w, int32_t T,
                       void* y, int32_t y_dtype, void* stream) {
    if (!L) return fail(MOE_ERR_ARG, "null layer handle");
    if (!expert_out || !w || !y) return fail(MOE_ERR_ARG, "null expert_out, w or y");
    if (T <= 0) return fail(MOE_ERR_ARG, "n_tokens out of range");
    if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return fail(MOE_ERR_ARG, "bad y_dtype");
    CombineArgs a{expert_out, w, y, L->d.hidden, L->d.top_k, T, y_dtype == MOE_BF16};
    hipError_t e = timed(K_COMBINE, (hipStream_t)stream, [&] { return launch_combine(a, (hipStream_t)stream); });
    return e == hipSuccess ? MOE_OK : hip_fail(e, "combine launch");
}

moe_status moe_layer_forward(moe_layer_t L, const void* x, int32_t T, int32_t* ids, float* w,
                             float* y, void* workspace, void* stream) {
    moe_status st = check_call(L, x, T, workspace);
    if (st != MOE_OK) return st;
    if (L->cache.n_slots && T != 1) return fail(MOE_ERR_STATE, "the slot cache runs one token per call");
    if (!ids || !w || !y) return fail(MOE_ERR_ARG, "null ids, w or y");
    const WsLayout o = ws_layout(L, T);
    uint8_t* ws = (uint8_t*)workspace;
    hipStream_t s = (hipStream_t)stream;
    if (T >= kPrefillMinTokens) return grouped_ffn(L, x, T, ids, w, y, nullptr, ws, o, s, true, true);
    hipError_t e;
    FfnArgs fa = ffn_args(L, ids, w, ws, o, y, nullptr, true);
    if (L->cache.n_slots || L->d.hidden > kFusedMaxHidden) {
        RouteArgs ra = route_args(L, x, ids, w, ws, o, 1, T);
        if ((e = timed(K_ROUTE, s, [&] { return launch_route(ra, T, L->d.act_dtype == MOE_BF16, s); })) != hipSuccess)
            return hip_fail(e, "router launch");
        if (L->cache.n_slots) {
            if ((e = timed(K_TOPK, s, [&] { return launch_topk(ra, T, s); })) != hipSuccess)
                return hip_fail(e, "top-k launch");
            return cached_ffn(L, ids, ffn_args(L, ids, w, ws, o, y, nullptr, false), o, ws, s);
        }
    } else {  // resident, hidden <= kFusedMaxHidden: routing inside the gate/up launch
        fa.logits = nullptr;
        fa.route_units = (L->d.n_experts + L->gu_waves - 1) / L->gu_waves;
        fa.x = x;
        fa.rq = L->w.router_q;
        fa.rs = L->w.router_scale;
        fa.flog = (uint32_t*)(ws + o.flog);
        fa.spin_limit = L->spin_limit;
        fa.logit_delay = logit_delay_ticks(L->d);
    }
    if ((e = decode_units(L, fa, T, 0, fa.n_units, s)) != hipSuccess) return hip_fail(e, "gate/up launch");
    if ((e = decode_finish(fa, T, s)) != hipSuccess) return hip_fail(e, "down launch");
    return MOE_OK;
}

moe_status moe_stack_forward(const moe_layer_t* layers, int32_t n_layers, const void* x,
                             int64_t x_stride, int32_t T, int32_t* ids, float* w, float* y,
                             int64_t y_stride, void* workspace, void* stream) {
    if (!layers || n_layers <= 0) return fail(MOE_ERR_ARG, "no layers");
    if (T <= 0) return fail(MOE_ERR_ARG, "n_tokens out of range");
    // every layer's ids/w rows sit at l * T * top_k and its x at l * x_stride
    // elements of one activation dtype: the layers must agree on both, and
    // each layer's [T][H] block must fit in its stride
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer* L = layers[l];
        if (!L) return fail(MOE_ERR_ARG, "null layer handle in stack");
        if (L->d.top_k != layers[0]->d.top_k || L->d.act_dtype != layers[0]->d.act_dtype)
            return fail(MOE_ERR_SHAPE, "stack layers must share top_k and act_dtype");
        if ((int64_t)T * L->d.hidden > x_stride || (int64_t)T * L->d.hidden > y_stride)
            return fail(MOE_ERR_SHAPE, "x_stride and y_stride must hold n_tokens * hidden elements");
    }
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer* L = layers[l];
        const size_t esz = L->d.act_dtype == MOE_BF16 ? 2 : 4;
        const void* xl = (const uint8_t*)x + (size_t)l * x_stride * esz;
        moe_status st = moe_layer_forward(layers[l], xl, T, ids + (size_t)l * T * L->d.top_k,
                                          w + (size_t)l * T * L->d.top_k,
                                          y + (size_t)l * y_stride, workspace, stream);
        if (st != MOE_OK) return st;
    }
    return MOE_OK;
}

namespace {
// Per-device address of `scratch` and whether its counters still need the
// one clear of their first use (or a clear after a failed call).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_dirty[kMaxDevices] = {};

__global__ void k_clear_words(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The current device's scratch address (looked up on its first use there).
moe_status scratch_for_current_device(uint8_t** out, int* dev_out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_STATE, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = (uint8_t*)ptr;
        g_scratch_dirty[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    *dev_out = dev;
    return MOE_OK;
}
}  // namespace

moe_status moe_layer_forward_noalloc(moe_layer_t L, const void* x, int32_t T, int32_t* ids, float* w,
                                     float* y, void* stream) {
    if (!L) return fail(MOE_ERR_ARG, "null layer handle");
    if (T <= 0 || T > (1 << 20)) return fail(MOE_ERR_ARG, "n_tokens out of range");
    const size_t need = ws_layout(L, T).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_SHAPE, "this call needs " + std::to_string(need) + " bytes of scratch; the "
                                   "allocation-free entry holds " + std::to_string(kScratchBytes));
    uint8_t* ws = nullptr;
    int dev = -1;
    moe_status st = scratch_for_current_device(&ws, &dev);
    if (st != MOE_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (g_scratch_dirty[dev]) {
        // counters, logit words and the error word must start at zero: they
        // are the scratch's first bytes, below the offsets that depend on T
        const size_t words = ws_layout(L, 1).pred_ids / 4;
        hipLaunchKernelGGL(k_clear_words, dim3(64), dim3(256), 0, s, (uint32_t*)ws, words);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
        g_scratch_dirty[dev] = false;
    }
    st = moe_layer_forward(L, x, T, ids, w, y, ws, stream);
    if (st == MOE_ERR_HIP) g_scratch_dirty[dev] = true;  // a partial call may leave counters set
    return st;
}

moe_status moe_cache_usage(moe_layer_t L, uint64_t* counts) {
    if (!L || !counts) return fail(MOE_ERR_ARG, "null argument");
    if (!L->cache.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    std::copy(L->cache.count.begin(), L->cache.count.end(), counts);
    return MOE_OK;
}

moe_status moe_cache_pin_hottest(moe_layer_t L, const uint64_t* counts, int32_t n, void* stream) {
    if (!L) return fail(MOE_ERR_ARG, "null layer handle");
    const SlotCache& c = L->cache;
    if (!c.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    if (n < 0 || n > c.n_slots - L->d.top_k) return fail(MOE_ERR_ARG, "n must be in 0..n_slots - top_k");
    const int E = L->d.n_experts;
    const uint64_t* u = counts ? counts : c.count.data();
    std::vector<int32_t> order(E);
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [u](int32_t a, int32_t b) { return u[a] > u[b]; });
    return moe_cache_pin(L, order.data(), n, stream);
}

moe_status moe_cache_stats(moe_layer_t L, uint64_t* hits, uint64_t* misses) {
    if (!L || !hits || !misses) return fail(MOE_ERR_ARG, "null argument");
    if (!L->cache.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    *hits = L->cache.hits;
    *misses = L->cache.misses;
    return MOE_OK;
}

moe_status moe_cache_pin(moe_layer_t L, const int32_t* experts, int32_t n, void* stream) {
    if (!L) return fail(MOE_ERR_ARG, "null layer handle");
    SlotCache& c = L->cache;
    if (!c.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    if (n < 0 || n > c.n_slots - L->d.top_k) return fail(MOE_ERR_ARG, "n must be in 0..n_slots - top_k");
    if (n > 0 && !experts) return fail(MOE_ERR_ARG, "null experts");
    for (int i = 0; i < n; ++i) {
        if (experts[i] < 0 || experts[i] >= L->d.n_experts) return fail(MOE_ERR_ARG, "expert id out of range");
        for (int j = 0; j < i; ++j)
            if (experts[j] == experts[i]) return fail(MOE_ERR_ARG, "duplicate expert id");
    }
    hipStream_t s = (hipStream_t)stream;
    if (c.side_pending) {  // a prefetch copy may still be writing a slot this call replaces
        hipError_t e = hipEventRecord(c.ev_copies, c.side);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, c.ev_copies, 0);
        if (e != hipSuccess) return hip_fail(e, "copy ordering");
        c.side_pending = false;
        std::fill(c.side_writing.begin(), c.side_writing.end(), 0);
    }
    std::fill(c.pinned.begin(), c.pinned.end(), 0);
    ++c.tick;
    for (int i = 0; i < n; ++i) {
        const int ex = experts[i];
        int slot = c.slot_of[ex];
        if (slot < 0) {
            for (int q = 0; q < c.n_slots && slot < 0; ++q)
                if (c.expert_in[q] < 0) slot = q;
            if (slot < 0) {
                slot = victim_slot(c, experts, n);  // never one of the set being pinned
                c.slot_of[c.expert_in[slot]] = -1;
            }
            c.expert_in[slot] = ex;
            c.slot_of[ex] = slot;
            hipError_t e = hipMemcpyAsync(L->w.slots + (size_t)slot * L->rec_bytes,
                                          L->w.host_pool + (size_t)ex * L->rec_bytes, L->rec_bytes,
                                          hipMemcpyHostToDevice, s);
            if (e != hipSuccess) return hip_fail(e, "pinned expert copy");
        }
        c.pinned[slot] = 1;
        c.prefetched[slot] = 0;
        c.last_use[slot] = c.tick;
    }
    return MOE_OK;
}

moe_status moe_cache_prefetch(moe_layer_t L, const void* x_hint, int32_t n_predict, void* workspace,
                              int32_t* predicted, void* stream) {
    moe_status st = check_call(L, x_hint, 1, workspace);
    if (st != MOE_OK) return st;
    SlotCache& c = L->cache;
    if (!c.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    const int k = L->d.top_k;
    if (n_predict < 1 || n_predict > k) return fail(MOE_ERR_ARG, "n_predict must be in 1..top_k");
    const WsLayout o = ws_layout(L, 1);
    uint8_t* ws = (uint8_t*)workspace;
    hipStream_t s = (hipStream_t)stream;
    int32_t* pid = (int32_t*)(ws + o.pred_ids);
    RouteArgs a = route_args(L, x_hint, pid, (float*)(ws + o.pred_w), ws, o, 0, 1);
    hipError_t e = timed(K_ROUTE, s, [&] { return launch_route(a, 1, L->d.act_dtype == MOE_BF16, s); });
    if (e == hipSuccess) e = timed(K_TOPK, s, [&] { return launch_topk(a, 1, s); });
    if (e != hipSuccess) return hip_fail(e, "lookahead router launch");
    e = hipMemcpyAsync(c.h_ids, pid, sizeof(int32_t) * k, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(c.ev_ids, s);
    if (e == hipSuccess) e = hipEventSynchronize(c.ev_ids);
    if (e != hipSuccess) return hip_fail(e, "reading the predicted experts");
    for (int j = 0; j < n_predict; ++j)
        if (c.h_ids[j] < 0 || c.h_ids[j] >= L->d.n_experts)
            return fail(MOE_ERR_ARG, "predicted expert id out of range");
    if (predicted) std::copy(c.h_ids, c.h_ids + n_predict, predicted);
    return prefetch_place(L, c.h_ids, n_predict);
}

moe_status moe_cache_prefetch_ids(moe_layer_t L, const int32_t* experts, int32_t n, void* stream) {
    if (!L) return fail(MOE_ERR_ARG, "null layer handle");
    SlotCache& c = L->cache;
    if (!c.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    if (n < 1 || n > L->d.top_k) return fail(MOE_ERR_ARG, "n must be in 1..top_k");
    if (!experts) return fail(MOE_ERR_ARG, "null experts");
    for (int i = 0; i < n; ++i) {
        if (experts[i] < 0 || experts[i] >= L->d.n_experts) return fail(MOE_ERR_ARG, "expert id out of range");
        for (int j = 0; j < i; ++j)
            if (experts[j] == experts[i]) return fail(MOE_ERR_ARG, "duplicate expert id");
    }
    (void)stream;  // the copies are ordered by the layer's own slot reads
    return prefetch_place(L, experts, n);
}

moe_status moe_cache_prefetch_stats(moe_layer_t L, uint64_t* issued, uint64_t* used) {
    if (!L || !issued || !used) return fail(MOE_ERR_ARG, "null argument");
    if (!L->cache.n_slots) return fail(MOE_ERR_STATE, "layer has no slot cache");
    *issued = L->cache.prefetch_issued;
    *used = L->cache.prefetch_used;
    return MOE_OK;
}

moe_status moe_poll_device_error(moe_layer_t L, void* workspace, void* stream) {
    if (!L || !workspace) return fail(MOE_ERR_ARG, "null layer or workspace");
    hipStream_t s = (hipStream_t)stream;
    uint32_t* errp = (uint32_t*)((uint8_t*)workspace + ws_layout(L, 1).err);
    uint32_t host = 0;
    hipError_t e = hipMemcpyAsync(&host, errp, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = launch_clear_word(errp, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "device error poll");
    return host ? fail(MOE_ERR_DEVICE, "a kernel saw an expert id outside [0, n_experts)") : MOE_OK;
}

moe_status moe_stream_read(const void* src, size_t bytes, int32_t n_blocks, uint32_t* sink, void* stream) {
    if (!src || !sink) return fail(MOE_ERR_ARG, "null src or sink");
    if (bytes == 0 || bytes % 16) return fail(MOE_ERR_ARG, "bytes must be a positive multiple of 16");
    if (n_blocks < 1 || n_blocks > (1 << 20)) return fail(MOE_ERR_ARG, "n_blocks must be in 1..2^20");
    if (!aligned(src, 16) || !aligned(sink, 4)) return fail(MOE_ERR_ALIGN, "src needs 16-byte alignment");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = timed(K_STREAM, s, [&] { return launch_stream_read(src, bytes, n_blocks, sink, s); });
    return e == hipSuccess ? MOE_OK : hip_fail(e, "stream read launch");
}

moe_status moe_profile_start(int32_t capacity) {
    if (capacity <= 0 || capacity > (1 << 22)) return fail(MOE_ERR_ARG, "bad profile capacity");
    for (auto& r : g_prof) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    g_prof.clear();
    g_prof_n = 0;
    try {
        g_prof.resize((size_t)capacity);
    } catch (...) {
        return fail(MOE_ERR_NOMEM, "profile buffer");
    }
    for (auto& r : g_prof) {
        hipError_t e = hipEventCreate(&r.a);
        if (e == hipSuccess) e = hipEventCreate(&r.b);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    }
    g_prof_on = true;
    return MOE_OK;
}

moe_status moe_profile_stop(void) {
    g_prof_on = false;
    return MOE_OK;
}

int32_t moe_profile_read(int32_t* kernel_ids, float* ms, int32_t max_records) {
    if (!kernel_ids || !ms || max_records < 0) return fail(MOE_ERR_ARG, "null profile output");
    const int32_t n = (int32_t)std::min<size_t>(g_prof_n, (size_t)max_records);
    for (int32_t i = 0; i < n; ++i) {
        hipError_t e = hipEventSynchronize(g_prof[i].b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_prof[i].a, g_prof[i].b);
        if (e != hipSuccess) return hip_fail(e, "profile read");
        kernel_ids[i] = g_prof[i].kid;
    }
    g_prof_n = 0;
    return n;
}

const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_ARG: return "MOE_ERR_ARG";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        case MOE_ERR_NOMEM: return "MOE_ERR_NOMEM";
        case MOE_ERR_NOT_PINNED: return "MOE_ERR_NOT_PINNED";
        case MOE_ERR_STATE: return "MOE_ERR_STATE";
        case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

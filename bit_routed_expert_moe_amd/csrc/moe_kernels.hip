// moe_kernels.hip -- gfx950 kernels of the routed-expert MoE layer.
//
//   k_route       router GEMV (int8 rows x activations), one row per wave,
//                 every load issued before any use; extra workgroups beside
//                 the router prepare the activations for the FFN kernels (four
//                 64-input groups per wave).  The API route and the slot-cache
//                 path use it; the resident forward routes inside k_gate_up.
//   k_topk        exact top-k and gate weights from the logits (API route and
//                 the grouped path).
//   k_prep        activation preparation alone (API expert FFN).
//   k_gate_up     one workgroup per (token, expert slot, block of 32 rows of
//                 I).  For routed slots in the fused path it first selects its
//                 expert itself (exact top-k over the logits, a radix select);
//                 then it streams the 64-row gate/up tile, h = silu(g) * u, and
//                 writes h prepared as fp16 pairs for the down kernel.  In the
//                 resident forward the router runs in the same launch: leading
//                 router units store the logits, the gate/up units prepare x in
//                 LDS while those land and read them as they arrive (no kernel
//                 boundary between routing and the expert stream).
//   k_down        one workgroup per (token, 64 output rows, work item), a work
//                 item being one routed expert or a k-slice of the shared one;
//                 the last item to finish for an output tile sums the items in
//                 a fixed order into per-expert outputs and/or the combined y.
//   k_combine     y = sum_j w_j * eo_j + eo_shared.
//
// Every weight byte is read once per token with 16-byte nontemporal loads,
// lane = row of a 64-row tile, so one wave instruction reads 1 KB of
// contiguous record bytes.  Small inputs (activations, logits) are loaded
// before the weights so that the weights can be consumed in arrival order.
// Sums across waves and workgroups are done in a fixed order: reruns are
// bit-identical.  The hand-offs inside a kernel (k_down's last arrival,
// k_gate_up's router units to its gate/up units, the last shared piece of a
// block in k_gate_up) use agent-scope coherent stores and loads (plus an
// arrival counter in k_down and for the pieces), so no L2 write-back or
// invalidate is needed.
#include "moe_device.h"
#include <type_traits>

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// activation preparation, four 64-input groups g0..g0+3 per wave: the 16
// lanes of row r (lanes 16r..16r+15) take group g0 + r, lane m of the row its
// inputs 4m..4m+3.  Each group gets its own power-of-two scale 2^e so that its
// largest value lands below 2^14 in fp16.  4-bit weights: odd positions of
// each 8-set are also divided by 16 to pair with the x16 nibble slots, pairs
// (a_p, a_{p+4}) per 8-set; 2-bit weights: pairs (a_j, a_{j+8}) per 16-set
// with pair j's in-place factor.  Writes each group's 32*XP pair dwords,
// K = 1024 * sum of the fp16 values (in double), X = sum of the inputs and
// inv = 2^-e, for groups below NG.  Sums run in a fixed order (a lane's four
// inputs in order, then the row's DPP tree; lane 0 of the row writes).
// xrow, pairs, K, X, inv are the token's own.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float row_max(float v) {  // max over the lane's row of 16
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    return fmaxf(v, dpp<0x128>(v));
}
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x124>(v);
    return v + dpp<0x128>(v);
}
__device__ __forceinline__ double row_sum_d(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x124>(v);
    return v + dpp_f64<0x128>(v);
}
// the lane's four inputs of group g: x[64 g + 4 m ...] (one 8- or 16-byte load);
// element by element through scalars (a bit-cast of a vector element reads
// element 0 with this compiler)
template <bool BF16>
__device__ __forceinline__ void load_act4(const void* xrow, int g, float (&v)[4]) {
    const int i0 = 64 * g + 4 * (threadIdx.x & 15);
    if (BF16) {
        const u32x2 w = *(const u32x2*)((const uint16_t*)xrow + i0);
        const uint32_t w0 = w[0], w1 = w[1];
        v[0] = __builtin_bit_cast(float, w0 << 16);
        v[1] = __builtin_bit_cast(float, w0 & 0xFFFF0000u);
        v[2] = __builtin_bit_cast(float, w1 << 16);
        v[3] = __builtin_bit_cast(float, w1 & 0xFFFF0000u);
    } else {
        const u32x4 w = *(const u32x4*)((const float*)xrow + i0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t wi = w[i];
            v[i] = __builtin_bit_cast(float, wi);
        }
    }
}
// the four groups' arithmetic, v = this lane's inputs
template <int XP, int BITS>
__device__ __forceinline__ void prep_quad_v(const float (&v)[4], int NG, int g0, uint32_t* pairs, float* K, float* X,
                                            float* inv) {
    const int lane = threadIdx.x & 63, m = lane & 15, g = g0 + (lane >> 4);
    const int e = act_exponent(row_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])))));
    uint32_t h[2] = {0u, 0u}, l[2] = {0u, 0u};
    double kd = 0.0;
    float xs = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sh = BITS == 4 ? ((i & 1) ? -4 : 0) : crumb_scale_log2(4 * (m & 1) + i);
        const float vs = v[i] * ldexpf(1.0f, e + sh);
        const _Float16 hi = (_Float16)vs;
        const _Float16 lo = (_Float16)(vs - (float)hi);
        h[i >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, hi) << (16 * (i & 1));
        l[i >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, lo) << (16 * (i & 1));
        kd += (double)(float)hi + (XP == 2 ? (double)(float)lo : 0.0);
        xs += v[i];
    }
    kd = row_sum_d(kd);
    xs = row_sum(xs);
    // partner lane with the other members of this lane's pairs: m ^ 1 (8-sets
    // over two lanes), m ^ 2 (16-sets over four lanes, j and j + 8)
    constexpr int CTRL = BITS == 4 ? 0xB1 : 0x4E;
    const bool writer = BITS == 4 ? (m & 1) == 0 : (m & 2) == 0;
    uint32_t* gp = pairs + (size_t)g * 32 * XP;
    // 4-bit: 8-set m/2, 4 pair dwords per part; 2-bit: 16-set m/4, 8 pair dwords per part, 4(m & 1) onward
    const int off = BITS == 4 ? (m >> 1) * XP * 4 : (m >> 2) * XP * 8 + 4 * (m & 1);
    const int part_stride = BITS == 4 ? 4 : 8;
#pragma unroll
    for (int part = 0; part < XP; ++part) {
        const uint32_t w01 = part ? l[0] : h[0], w23 = part ? l[1] : h[1];
        const uint32_t q01 = dpp_u32<CTRL>(w01), q23 = dpp_u32<CTRL>(w23);
        const u32x4 pd = {(w01 & 0xFFFFu) | (q01 << 16), (w01 >> 16) | (q01 & 0xFFFF0000u),
                          (w23 & 0xFFFFu) | (q23 << 16), (w23 >> 16) | (q23 & 0xFFFF0000u)};
        if (writer && g < NG) *(u32x4*)(gp + off + part * part_stride) = pd;
    }
    if (m == 0 && g < NG) {
        K[g] = (float)(1024.0 * kd);
        X[g] = xs;
        inv[g] = ldexpf(1.0f, -e);
    }
}
template <int XP, bool BF16, int BITS>
__device__ void prep_quad(const void* xrow, int NG, int g0, uint32_t* pairs, float* K, float* X, float* inv) {
    float v[4];
    load_act4<BF16>(xrow, min(g0 + (int)((threadIdx.x & 63) >> 4), NG - 1), v);
    prep_quad_v<XP, BITS>(v, NG, g0, pairs, K, X, inv);
}

// ---------------------------------------------------------------------------
// exact top-k over E <= 64*Q logits, then the renormalised softmax gates.
// Order: logit descending, ties to the lower id.  All threads of the
// workgroup must call it (it synchronises the workgroup once).
//   1. (wave 0) order-preserving 32-bit keys u (larger logit -> larger u);
//   2. (wave 0) threshold search, most significant bit first: T grows while
//      #{u >= T} >= k, and the search stops at the first T with exactly k
//      keys >= T (else it ends at the k-th largest key); up to 32 steps of
//      one compare per key slot, a ballot and a scalar popcount (two bits a
//      step measured no faster: it triples the scalar work per step);
//   3. (wave 0) the selection = every key above T plus the lowest ids among
//      the keys equal to T, as many as are needed, written to LDS in id order;
//   4. (every wave, after the barrier) lane j < k ranks entry j: the entries
//      with a larger key, and the earlier entries with an equal key, are
//      ahead of it.
// Only wave 0 selects; one barrier publishes the selection.  Returns the id
// of rank `want` (if >= 0; -1 when no entry has that rank).  ids_out / w_out (workgroup-uniform) get the
// selection in rank order and the gates.
// ---------------------------------------------------------------------------
struct alignas(16) TopkScratch {
    uint32_t key[kMaxTopK];
    int id[kMaxTopK];
    float val[kMaxTopK];
};

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);  // -0 -> +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Gate functions: 0 = softmax over the selected logits (selection by logit);
// 1 = sigmoid router (selection by logistic score + bias, gates = rscale *
// score / sum of the selection's scores).
struct GateFn {
    int kind;
    const float* bias;  // [E] or nullptr
    float rscale;
};

__device__ __forceinline__ int ballot_count(bool v) {
    return __builtin_popcountll(__builtin_amdgcn_ballot_w64(v));
}

// The selection from logits held by wave 0: lg0[q] on lane l is the logit of
// id l + 64 q (any value where that id is >= E).  Waves other than 0 pass
// anything.
template <int Q>
__device__ __forceinline__ int topk_select_v(const float (&lg0)[Q], int E, int k, int want, TopkScratch& sm,
                                             int32_t* ids_out, float* w_out, GateFn gf) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        float lv[Q];  // logit (softmax) or score (sigmoid) of each key slot
        uint32_t u[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) lv[q] = lg0[q];
        if (gf.kind == 1) {
            float bv[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) bv[q] = gf.bias ? gf.bias[min(lane + 64 * q, E - 1)] : 0.0f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                lv[q] = __builtin_amdgcn_rcpf(1.0f + expf(-lv[q]));  // score; 1-ulp reciprocal
                u[q] = order_key(lv[q] + bv[q]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < Q; ++q) u[q] = order_key(lv[q]);
        }
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (lane + 64 * q >= E) u[q] = 0u;  // 0: below every key
        // once exactly k keys are >= T the selection is fixed: the keys equal
        // to T (if any) are then all taken below, so the search may stop there
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int n = 0;
#pragma unroll
            for (int q = 0; q < Q; ++q) n += ballot_count(u[q] >= cand);
            if (n >= k) {
                T = cand;
                if (n == k) break;
            }
        }
        int gt = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) gt += ballot_count(u[q] > T);
        const int need = k - gt;  // keys equal to T to take, lowest ids first
        int before = 0, pos0 = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint64_t eqm = __builtin_amdgcn_ballot_w64(u[q] == T && lane + 64 * q < E);
            const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(eqm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eqm, 0u));
            const bool take = u[q] > T || ((eqm >> lane) & 1 && before + below < need);
            const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
            if (take) {
                const int pos = pos0 + __builtin_amdgcn_mbcnt_hi((uint32_t)(tm >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)tm, 0u));
                sm.key[pos] = u[q];
                sm.id[pos] = lane + 64 * q;
                sm.val[pos] = lv[q];
            }
            before += __builtin_popcountll(eqm);
            pos0 += __builtin_popcountll(tm);
        }
        if (lane >= k && lane < kMaxTopK) sm.key[lane] = 0u;  // below every selected key
    }
    __syncthreads();
    // entry j (lane j < k): its rank among the k entries (held in id order):
    // the entries ahead of it are those with a larger (key, -position), one
    // 64-bit compare each; the zero keys past k are behind every entry
    uint32_t keys[kMaxTopK];
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) keys[i] = sm.key[i];
    const int mine = min(lane, kMaxTopK - 1);
    const int my_id = sm.id[mine];
    const uint64_t mc = ((uint64_t)sm.key[mine] << 32) | (uint32_t)(kMaxTopK - 1 - mine);
    int rank = 0;
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) rank += (((uint64_t)keys[i] << 32) | (uint32_t)(kMaxTopK - 1 - i)) > mc ? 1 : 0;
    const bool valid = lane < k;
    if (ids_out && threadIdx.x < 64) {
        const float v = valid ? sm.val[mine] : 0.0f;
        float ex;
        if (gf.kind == 1) {
            ex = v;  // the unbiased score
        } else {
            const uint64_t top = __builtin_amdgcn_ballot_w64(valid && rank == 0);
            const float mx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v),
                                                                                  __builtin_ctzll(top)));
            ex = valid ? expf(v - mx) : 0.0f;
        }
        const float z = wave_sum(ex);
        if (valid) {
            ids_out[rank] = my_id;
            w_out[rank] = gf.kind == 1 ? gf.rscale * (ex / z) : ex / z;
        }
    }
    if (want < 0) return -1;
    const uint64_t m = __builtin_amdgcn_ballot_w64(valid && rank == want);
    return m ? __builtin_amdgcn_readlane(my_id, __builtin_ctzll(m)) : -1;
}

// The selection from logits lg [E] in memory (loaded by wave 0, clamped ids).
template <int Q>
__device__ __forceinline__ int topk_select(const float* lg, int E, int k, int want, TopkScratch& sm, int32_t* ids_out,
                                           float* w_out, GateFn gf) {
    float lv[Q] = {};
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < Q; ++q) lv[q] = lg[min(lane + 64 * q, E - 1)];
    }
    return topk_select_v<Q>(lv, E, k, want, sm, ids_out, w_out, gf);
}

// ---------------------------------------------------------------------------
// One router row per wave: the logit of expert e for token t, the int8 row
// times the activations in fp32 (lane = 16-byte chunk of the row, chunks
// accumulated per lane in a fixed order, then a fixed-order wave sum), times
// the row's fp16 scale.  Every load is issued before any use (CPL = chunk
// rounds per lane held in registers, H <= 1024 * CPL).  All lanes return the
// logit.  k_route and the fused router units of k_gate_up use it, and
// router_row_rolled repeats its arithmetic in the same order, so every path
// gets the same bits.
// ---------------------------------------------------------------------------
constexpr int kRouterChunksPerLane = kMaxHidden / 16 / 64;  // 16-byte chunks per lane

__device__ __forceinline__ float router_chunk(uint32_t q, const float* xf, float acc) {
#pragma unroll
    for (int bsel = 0; bsel < 4; ++bsel) acc = fmaf((float)(int)(int8_t)(q >> (8 * bsel)), xf[bsel], acc);
    return acc;
}

template <bool BF16>
__device__ __forceinline__ void unpack_x16(const u32x4 (&xr)[BF16 ? 2 : 4], float (&xf)[16]) {
#pragma unroll
    for (int v = 0; v < (BF16 ? 2 : 4); ++v) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t word = xr[v][d];
            if (BF16) {
                xf[8 * v + 2 * d] = __builtin_bit_cast(float, word << 16);
                xf[8 * v + 2 * d + 1] = __builtin_bit_cast(float, word & 0xFFFF0000u);
            } else {
                xf[4 * v + d] = __builtin_bit_cast(float, word);
            }
        }
    }
}

template <bool BF16, int CPL = kRouterChunksPerLane>
__device__ __forceinline__ float router_row(const void* x, int t, int H, const int8_t* rq, const uint16_t* rs,
                                            int e) {
    const int lane = threadIdx.x & 63;
    const int nch = H / 16;
    constexpr int XV = BF16 ? 2 : 4;  // 16-byte loads per 16 activations
    const int ncl = (nch + 63) / 64;  // chunk rounds in use (uniform)
    u32x4 wr[CPL], xr[CPL][XV];
    const u32x4* row = (const u32x4*)(rq + (size_t)e * H);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        if (i < ncl) wr[i] = ldg_nt(row + min(lane + 64 * i, nch - 1));
    const u32x4* xb = (const u32x4*)((const uint8_t*)x + (size_t)t * H * (BF16 ? 2 : 4));
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (i < ncl) {
            const int c = min(lane + 64 * i, nch - 1);
#pragma unroll
            for (int v = 0; v < XV; ++v) xr[i][v] = xb[c * XV + v];
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (lane + 64 * i < nch) {
            float xf[16];
            unpack_x16<BF16>(xr[i], xf);
#pragma unroll
            for (int d = 0; d < 4; ++d) acc = router_chunk(wr[i][d], xf + 4 * d, acc);
        }
    }
    return wave_sum(acc) * (float)__builtin_bit_cast(_Float16, rs[e]);
}

// router_row one chunk round at a time (few registers, one round trip per
// round): the same operations in the same order, so the same bits.
template <bool BF16>
__device__ float router_row_rolled(const void* x, int t, int H, const int8_t* rq, const uint16_t* rs, int e) {
    const int lane = threadIdx.x & 63;
    const int nch = H / 16;
    constexpr int XV = BF16 ? 2 : 4;
    const u32x4* row = (const u32x4*)(rq + (size_t)e * H);
    const u32x4* xb = (const u32x4*)((const uint8_t*)x + (size_t)t * H * (BF16 ? 2 : 4));
    float acc = 0.0f;
    for (int c = lane; c < nch; c += 64) {
        const u32x4 w = row[c];
        u32x4 xr[XV];
#pragma unroll
        for (int v = 0; v < XV; ++v) xr[v] = xb[c * XV + v];
        float xf[16];
        unpack_x16<BF16>(xr, xf);
#pragma unroll
        for (int d = 0; d < 4; ++d) acc = router_chunk(w[d], xf + 4 * d, acc);
    }
    return wave_sum(acc) * (float)__builtin_bit_cast(_Float16, rs[e]);
}

// k_route: grid (ceil(E/4) router blocks [+ prep blocks], T); one router row
// per wave (measured: 3 % less per decode step than two rows, 7 % less than 4).
template <int XP, bool BF16, int BITS>
__global__ __launch_bounds__(kBlock) void k_route(RouteArgs a) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int rb = (a.E + kWaves - 1) / kWaves;
    if ((int)blockIdx.x >= rb) {  // activation preparation blocks (one token each, four groups a wave)
        const int g0 = 4 * (((int)blockIdx.x - rb) * kWaves + wave), NG = a.H / 64, t = blockIdx.y;
        if (g0 < NG)
            prep_quad<XP, BF16, BITS>((const uint8_t*)a.x + (size_t)t * a.H * (BF16 ? 2 : 4), NG, g0,
                                      a.xpairs + (size_t)t * (a.H / 2) * XP, a.xK + (size_t)t * NG,
                                      a.xX + (size_t)t * NG, a.xinv + (size_t)t * NG);
        return;
    }
    const int e = blockIdx.x * kWaves + wave;
    if (e >= a.E) return;
    const float v = router_row<BF16>(a.x, blockIdx.y, a.H, a.rq, a.rs, e);
    if (lane == 0) a.logits[(size_t)blockIdx.y * a.E + e] = v;
}

// Wave 0 of a fused gate/up workgroup: the logits of token t as the router
// units store them.  A stored word is the logit's bits inverted, so it is
// never 0 (a finite logit is never all ones) and 0 means "not yet written";
// the wave re-reads its words, with agent-scope loads that see the stores of
// every XCD, until none is 0.  After spin_limit re-reads (at once when it is
// negative) it computes the logits itself with router_row: the same bits, and
// a wait that ends however the workgroups are scheduled.
template <int Q, bool BF16>
__device__ __forceinline__ void fused_logits(const FfnArgs& a, int t, float (&lv)[Q]) {
    const int lane = threadIdx.x & 63;
    uint32_t* fl = a.flog + (size_t)t * a.E;
    if (a.spin_limit >= 0) {
        for (int it = 0;; ++it) {
            uint32_t w[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q)
                w[q] = __hip_atomic_load(fl + min(lane + 64 * q, a.E - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool miss = false;
#pragma unroll
            for (int q = 0; q < Q; ++q) miss |= w[q] == 0u;
            if (!__builtin_amdgcn_ballot_w64(miss)) {
#pragma unroll
                for (int q = 0; q < Q; ++q) lv[q] = __builtin_bit_cast(float, ~w[q]);
                return;
            }
            if (it >= a.spin_limit) break;
            __builtin_amdgcn_s_sleep(2);
        }
    }
    for (int e = 0; e < a.E; ++e) {
        const float v = router_row_rolled<BF16>(a.x, t, a.H, a.rq, a.rs, e);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (e == lane + 64 * q) lv[q] = v;
    }
}

// k_topk: grid (T), one wave per token: ids/w from the logits.
template <int Q>
__global__ __launch_bounds__(64) void k_topk(RouteArgs a) {
    __shared__ TopkScratch sm;
    const int t = blockIdx.x;
    topk_select<Q>(a.logits + (size_t)t * a.E, a.E, a.k, -1, sm, a.ids + (size_t)t * a.k, a.w + (size_t)t * a.k,
                   GateFn{a.gate, a.bias, a.rscale});
}

// k_prep: grid (ceil(H/256), T); one wave per 64-input group.
template <int XP, bool BF16, int BITS>
__global__ __launch_bounds__(kBlock) void k_prep(RouteArgs a) {
    const int g0 = 4 * (blockIdx.x * kWaves + wave_id()), NG = a.H / 64, t = blockIdx.y;
    if (g0 < NG)
        prep_quad<XP, BF16, BITS>((const uint8_t*)a.x + (size_t)t * a.H * (BF16 ? 2 : 4), NG, g0,
                                  a.xpairs + (size_t)t * (a.H / 2) * XP, a.xK + (size_t)t * NG, a.xX + (size_t)t * NG,
                                  a.xinv + (size_t)t * NG);
}

// ---------------------------------------------------------------------------
// k_gate_up: grid (k*blk_r + sh_split*blk_s, T).  Lane = row of the 64-row GU
// tile (rows 0..31 gate, 32..63 up); waves split the H/64 input groups.  With
// 4-wave units each shared 32-row block is sh_split units, one slice of H
// each: the slices' gate/up sums meet in the last slice to arrive, which
// computes h.  (A unit per shared block was a third unit on a quarter of the
// CUs, and a CU streams at most about 25 GB/s: those CUs finished last.)
// ---------------------------------------------------------------------------
template <int XP, int MAXG, int Q, int BITS, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gate_up(FfnArgs a) {
    constexpr int kGuBlock = 64 * WAVES;
    // 16-byte vectors of prepared activations per thread, at the largest hidden
    // size the wave count is used for
    constexpr int kXPrepVecsPerThread =
        (WAVES == kGuWavesSmallH ? kGuSmallHMax : kMaxHidden) / 8 * 2 / kGuBlock;
    extern __shared__ uint32_t smem[];
    const int H = a.H, NG = H / 64;
    uint32_t* xp = smem;                                 // [H/2*XP]
    float* sK = (float*)(xp + (H / 2) * XP);             // [NG]
    float* sX = sK + NG;                                 // [NG]
    float* sI = sX + NG;                                 // [NG]
    float* red = sI + NG;                                // [WAVES][64]
    __shared__ TopkScratch s_topk;

    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int t = blockIdx.y;
    // routing inside this launch serves the hidden sizes of the 8-wave units
    constexpr bool FUSABLE = WAVES == kGuWavesSmallH;
    static_assert(kFusedMaxHidden <= kGuSmallHMax, "fused routing needs the 8-wave units");
    const int route_units = FUSABLE ? a.route_units : 0;
    if ((int)blockIdx.x < route_units) {  // fused router unit: one logit per wave
        const int e = blockIdx.x * WAVES + wave;
        if (e < a.E) {
            constexpr int CPL = kFusedMaxHidden / 16 / 64;  // chunk rounds per lane
            const float v = router_row<XP == 1, CPL>(a.x, t, H, a.rq, a.rs, e);
            if (lane == 0)
                __hip_atomic_store(a.flog + (size_t)t * a.E + e, ~__builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    const uint64_t t_launch = wall_clock64();  // 100 MHz device clock
    const int u = blockIdx.x - route_units + a.unit_offset;
    const bool fused = route_units > 0;
    const bool routed = u < a.k * a.blk_r;
    const int j = routed ? u / a.blk_r : a.k;
    // a shared unit is one slice (piece) of H of a 32-row block when sh_split > 1
    const int S = routed ? 1 : a.sh_split;
    const int vs = u - a.k * a.blk_r;
    const int b = routed ? u - j * a.blk_r : vs / S;
    const int piece = routed ? 0 : vs - b * S;

    // 1. the prepared activations of token t: into registers first, or with
    // fused routing prepared here, straight into LDS (the same arithmetic as
    // the preparation blocks; each wave loads all of its groups' inputs
    // first, then works through them)
    const int nvec = (H / 8) * XP;  // 16-byte vectors of pairs
    const int gq = min((int)threadIdx.x, NG - 1);
    u32x4 xv[kXPrepVecsPerThread];
    float kx = 0.0f, xx = 0.0f, xi = 0.0f;
    if (fused) {
        constexpr int R = (kFusedMaxHidden / 256 + WAVES - 1) / WAVES;  // four-group rounds per wave at most
        const uint8_t* xrow = (const uint8_t*)a.x + (size_t)t * H * (XP == 1 ? 2 : 4);
        float v[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) load_act4<XP == 1>(xrow, min(4 * (wave + WAVES * r) + (lane >> 4), NG - 1), v[r]);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (4 * (wave + WAVES * r) < NG) prep_quad_v<XP, BITS>(v[r], NG, 4 * (wave + WAVES * r), xp, sK, sX, sI);
    } else {
        const u32x4* gx = (const u32x4*)(a.xpairs + (size_t)t * (H / 2) * XP);
        // Loads are unconditional with clamped addresses so that the number of
        // loads in flight is static and every use waits only for its own data.
#pragma unroll
        for (int i = 0; i < kXPrepVecsPerThread; ++i)
            xv[i] = gx[min((int)threadIdx.x + kGuBlock * i, nvec - 1)];
        kx = a.xK[(size_t)t * NG + gq];
        xx = a.xX[(size_t)t * NG + gq];
        xi = a.xinv[(size_t)t * NG + gq];
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. which expert
    bool bad = false;
    const uint8_t* rec;
    if (routed) {
        int e;
        const bool first = u == 0;
        int32_t* ids_out = first ? a.ids_out + (size_t)t * a.k : nullptr;
        float* w_out = first ? a.w_out + (size_t)t * a.k : nullptr;
        if (fused) {
            float lv[Q] = {};
            if (wave == 0) {
                // first read no earlier than the router units' span (bounded wait)
                while (wall_clock64() - t_launch < (uint64_t)a.logit_delay) __builtin_amdgcn_s_sleep(1);
                fused_logits<Q, XP == 1>(a, t, lv);
            }
            e = topk_select_v<Q>(lv, a.E, a.k, j, s_topk, ids_out, w_out, GateFn{a.gate, a.bias, a.rscale});
        } else if (a.logits) {
            e = topk_select<Q>(a.logits + (size_t)t * a.E, a.E, a.k, j, s_topk, ids_out, w_out,
                               GateFn{a.gate, a.bias, a.rscale});
        } else {
            e = a.ids[(size_t)t * a.k + j];
        }
        if (e < 0 || e >= a.E) {
            bad = true;
            e = 0;
        }
        rec = a.slots ? a.slots + (size_t)a.slot_of[j] * a.rec_bytes
                      : a.experts + (size_t)e * a.rec_bytes;
    } else {
        rec = a.shared;
    }
    // the block's H/64 segments, one per 64-input group: NW 1 KB chunks of
    // codes (16 bytes per tile row: 32 nibbles, or 64 2-bit codes) and then
    // the 64 rows' (scale, bias) pairs, 4 bytes per row
    constexpr int NW = BITS == 4 ? 2 : 1;
    constexpr int SEG = NW * 1024 + 256;
    const uint8_t* tile = rec + (size_t)SEG * NG * b + (size_t)lane * 16;
    const uint8_t* sbt = rec + (size_t)SEG * NG * b + NW * 1024 + (size_t)lane * 4;
    int g0, g1;
    if (S == 1) {
        g0 = wave * a.gpw_gu;
        g1 = min(NG, g0 + a.gpw_gu);
    } else {  // this piece's slice of the input groups, split over the waves
        const int r1 = (piece + 1) * NG / S;
        g0 = piece * NG / S + wave * a.gpw_sh;
        g1 = min(r1, g0 + a.gpw_sh);
    }
    const int glast = max(g1 - 1, 0);  // clamp of the loads past this wave's groups (re-reads)

    // 3. weight stream: a ring of kDepth groups in flight per wave.  Loads are
    // unconditional (clamped to a valid group) and kept in program order, so
    // each group's compute waits only for that group's loads.
    constexpr int DK = WAVES == kGuWavesLargeH && BITS == 4 ? kDepthLargeH : kDepth;
    constexpr int D = DK < MAXG ? DK : MAXG;
    u32x4 W[D][NW];
    uint32_t SB[D];
#pragma unroll
    for (int q = 0; q < D; ++q) {
        const int g = min(g0 + q, glast);
#pragma unroll
        for (int c = 0; c < NW; ++c) W[q][c] = ldg_nt((const u32x4*)(tile + (size_t)g * SEG + c * 1024));
        SB[q] = ldg_nt((const uint32_t*)(sbt + (size_t)g * SEG));
        __builtin_amdgcn_sched_barrier(0);
    }
    // 4. activations to LDS (waits only for the loads issued before the weights)
    if (!fused) {
#pragma unroll
        for (int i = 0; i < kXPrepVecsPerThread; ++i) {
            const int v = threadIdx.x + kGuBlock * i;
            if (v < nvec) ((u32x4*)xp)[v] = xv[i];
        }
        if ((int)threadIdx.x < NG) {
            sK[threadIdx.x] = kx;
            sX[threadIdx.x] = xx;
            sI[threadIdx.x] = xi;
        }
    }
    __syncthreads();

    // 5. dequantised dot products, group by group as the weights arrive (a
    // shared piece's waves hold at most kPieceMaxGroups groups: its own
    // unrolled copy, so that every copy's waits stay exact)
    float rs = 0.0f, rb = 0.0f;
    auto stream = [&](auto mg) {
        constexpr int MG = decltype(mg)::value;
#pragma unroll
        for (int q = 0; q < MG; ++q) {
            const int slot = q % D;
            const int g = g0 + q;
            if (g < g1) {
                float a0 = 0.0f, a1 = 0.0f;
                if constexpr (BITS == 4) {
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const u32x4 wv = W[slot][half];
                        const uint32_t* xc = xp + (size_t)(2 * g + half) * 16 * XP;
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
#pragma unroll
                            for (int p = 0; p < XP; ++p) dot_nib8(wv[m], xc + (m * XP + p) * 4, a0, a1);
                        }
                    }
                } else {
                    const u32x4 wv = W[slot][0];
                    const uint32_t* xc = xp + (size_t)g * 32 * XP;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
#pragma unroll
                        for (int p = 0; p < XP; ++p) dot_crumb16(wv[m], xc + (m * XP + p) * 8, a0, a1);
                    }
                }
                rs = fmaf(f16lo(SB[slot]) * sI[g], (a0 + a1) - sK[g], rs);
                rb = fmaf(f16hi(SB[slot]), sX[g], rb);
            }
            if (q + D < MG) {  // refill the slot just consumed
                const int gn = min(g0 + q + D, glast);
#pragma unroll
                for (int c = 0; c < NW; ++c) W[slot][c] = ldg_nt((const u32x4*)(tile + (size_t)gn * SEG + c * 1024));
                SB[slot] = ldg_nt((const uint32_t*)(sbt + (size_t)gn * SEG));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (WAVES == kGuWavesLargeH && S > 1)  // pieces only with 4-wave units
        stream(std::integral_constant<int, (kPieceMaxGroups < MAXG ? kPieceMaxGroups : MAXG)>{});
    else
        stream(std::integral_constant<int, MAXG>{});
    red[wave * 64 + lane] = rs + rb;
    __syncthreads();
    if (wave != 0) return;

    // 6. wave 0: gate/up sums in wave order (of a shared block split into
    // pieces: each piece's sums, then in the last piece to arrive their sums
    // in piece order), h = silu(g) * u, then h prepared
    float gsum = 0.0f, usum = 0.0f;
    if (WAVES != kGuWavesLargeH || S == 1) {
        if (lane < 32) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                gsum += red[w * 64 + lane];
                usum += red[w * 64 + 32 + lane];
            }
        }
    } else {
        float pv = 0.0f;  // lane < 32: gate row lane, else up row lane - 32
#pragma unroll
        for (int w = 0; w < WAVES; ++w) pv += red[w * 64 + lane];
        float* P = a.shp + ((size_t)t * a.blk_s + b) * S * 64;
        __hip_atomic_store(P + piece * 64 + lane, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);  // the coherent store above has completed
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        uint32_t* ctr = a.dctr + ((size_t)t * a.blk_s + b) * kCounterStride;
        uint32_t prev = 0;
        if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __shfl(prev, 0, 64);
        if (prev != (uint32_t)S - 1) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        for (int q = 0; q < S; ++q) {
            const float gq = __hip_atomic_load(P + q * 64 + (lane & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const float uq = __hip_atomic_load(P + q * 64 + 32 + (lane & 31), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
            gsum += gq;
            usum += uq;
        }
        if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float h = 0.0f;
    if (lane < 32) h = bad ? __builtin_nanf("") : gsum / (1.0f + expf(-gsum)) * usum;
    if (bad && lane == 0) atomicOr(a.err, 1u);
    const float mx = wave_max(lane < 32 ? fabsf(h) : 0.0f);
    const int e = act_exponent(mx);
    // h pairs as the activations: (h_p, h_{p+4}) per 8-set with odd p / 16 for
    // nibbles; (h_p, h_{p+8}) per 16-set with pair p % 8's factor for 2-bit codes
    constexpr int SET = BITS == 4 ? 8 : 16, PD = SET / 2;
    const int p = lane % SET, set = lane / SET;
    const int sh = BITS == 4 ? ((p & 1) ? -4 : 0) : crumb_scale_log2(p & 7);
    const float v = h * ldexpf(1.0f, e + sh);
    const _Float16 hh = (_Float16)v;
    const _Float16 hl = (_Float16)(v - (float)hh);
    double kd = lane < 32 ? (double)(float)hh + (kHParts == 2 ? (double)(float)hl : 0.0) : 0.0;
    kd = wave_sum_d(kd);
    const float hs = wave_sum(lane < 32 ? h : 0.0f);
    const uint32_t bh = __builtin_bit_cast(uint16_t, hh), bl = __builtin_bit_cast(uint16_t, hl);
    const uint32_t ph = __shfl_down(bh, PD, 64), pl = __shfl_down(bl, PD, 64);
    const size_t slot = ((size_t)t * (a.k + 1) + j) * a.blk_max + b;
    uint32_t* hp = a.hpairs + slot * (16 * kHParts);
    if (lane < 32 && p < PD) {
        hp[(set * kHParts + 0) * PD + p] = bh | (ph << 16);
        if (kHParts == 2) hp[(set * kHParts + 1) * PD + p] = bl | (pl << 16);
    }
    if (lane == 0) {
        a.hK[slot] = bad ? __builtin_nanf("") : (float)(1024.0 * kd);
        a.hHs[slot] = hs;
        a.hinv[slot] = ldexpf(1.0f, -e);
    }
}

// ---------------------------------------------------------------------------
// k_down: grid (n_otiles * n_items, T).  Lane = output row of a 64-row tile;
// waves split the item's input groups (64 inputs of I = two h blocks).
// ---------------------------------------------------------------------------
template <int MAXG, int BITS, int RING>
__global__ __launch_bounds__(kBlock) void k_down(FfnArgs a) {
    extern __shared__ uint32_t smem[];
    const int H = a.H;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int t = blockIdx.y;
    if (a.flog && blockIdx.x == 0) {  // the fused router's words back to "not written"
        for (int i = threadIdx.x; i < a.E; i += kBlock)
            __hip_atomic_store(a.flog + (size_t)t * a.E + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int ot = blockIdx.x / a.n_items, item = blockIdx.x - ot * a.n_items;
    int j, ga, gb;
    const uint8_t* rec;
    if (item < a.k) {
        j = item;
        int e = a.ids[(size_t)t * a.k + j];
        if (e < 0 || e >= a.E) e = 0;  // h of this slot is NaN already
        rec = a.slots ? a.slots + (size_t)a.slot_of[j] * a.rec_bytes
                      : a.experts + (size_t)e * a.rec_bytes;
        ga = 0;
        gb = a.I / 64;
    } else {
        j = a.k;
        rec = a.shared;
        ga = (item - a.k) * a.gis;
        gb = min(ga + a.gis, a.Is / 64);
    }
    const int o = ot * 64 + lane;
    const int g0 = ga + wave * a.gpw_dn;
    const int g1 = min(gb, g0 + a.gpw_dn);
    // the output tile's down segments, one per 64-input group of I: the codes
    // (two 1 KB chunks of 32 nibbles per row, or one of 64 2-bit codes per
    // row), then the 64 rows' (scale, bias) pairs
    constexpr int NW = BITS == 4 ? 2 : 1;
    constexpr int SEG = NW * 1024 + 256;
    const int ngi = (item < a.k ? a.I : a.Is) / 64;
    const uint8_t* dseg = rec + (item < a.k ? a.d_off : a.d_off_shared) + (size_t)SEG * ngi * ot;
    const uint8_t* dcodes = dseg + (size_t)lane * 16;
    const uint8_t* dsb = dseg + NW * 1024 + (size_t)lane * 4;

    // h of (t, j), blocks [2ga, 2gb): loaded before the weights
    const int nb = 2 * (gb - ga);
    uint32_t* sp = smem;                             // [nb][16*kHParts]
    float* sK = (float*)(sp + nb * 16 * kHParts);    // [nb]
    float* sH = sK + nb;                             // [nb]
    float* sI = sH + nb;                             // [nb]
    float* red = sI + nb;                            // [4][64]
    const size_t slot0 = ((size_t)t * (a.k + 1) + j) * a.blk_max + 2 * ga;
    // at most 2 * kMaxDownGroups h blocks per item (<= kBlock), 4*kHParts vectors each
    constexpr int HV = (2 * kMaxDownGroups * 4 * kHParts + kBlock - 1) / kBlock;
    const u32x4* gp = (const u32x4*)(a.hpairs + slot0 * 16 * kHParts);
    const int nvec = nb * 4 * kHParts;
    // unconditional loads with clamped addresses (static count in flight)
    u32x4 hv[HV];
#pragma unroll
    for (int i = 0; i < HV; ++i) hv[i] = gp[min((int)threadIdx.x + kBlock * i, nvec - 1)];
    const int bq = min((int)threadIdx.x, nb - 1);
    const float hk = a.hK[slot0 + bq];
    const float hs = a.hHs[slot0 + bq];
    const float hi = a.hinv[slot0 + bq];
    __builtin_amdgcn_sched_barrier(0);

    // a ring of DD groups in flight per wave (every group at once when a wave
    // has at most RING groups)
    constexpr int DD = MAXG > RING ? RING : MAXG;
    u32x4 W[DD][NW];
    uint32_t SB[DD];
#pragma unroll
    for (int q = 0; q < DD; ++q) {
        const int g = min(g0 + q, gb - 1);  // past this wave's range: re-read a valid group
#pragma unroll
        for (int c = 0; c < NW; ++c) W[q][c] = ldg_nt((const u32x4*)(dcodes + (size_t)g * SEG + c * 1024));
        SB[q] = ldg_nt((const uint32_t*)(dsb + (size_t)g * SEG));
        __builtin_amdgcn_sched_barrier(0);  // keep issue order = consumption order
    }
#pragma unroll
    for (int i = 0; i < HV; ++i) {
        const int v = threadIdx.x + kBlock * i;
        if (v < nvec) ((u32x4*)sp)[v] = hv[i];
    }
    if ((int)threadIdx.x < nb) {
        sK[threadIdx.x] = hk;
        sH[threadIdx.x] = hs;
        sI[threadIdx.x] = hi;
    }
    __syncthreads();

    float row = 0.0f;
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
        const int g = g0 + q;
        const int slot = q % DD;
        if (g < g1) {
            float part = 0.0f;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int lb = 2 * (g - ga) + half;  // local h block
                const uint32_t* hc = sp + (size_t)lb * 16 * kHParts;
                float a0 = 0.0f, a1 = 0.0f;
                if constexpr (BITS == 4) {
                    const u32x4 wv = W[slot][half];  // 32 nibbles: inputs 32 half .. of the group
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t wm = wv[m];
#pragma unroll
                        for (int p = 0; p < kHParts; ++p)
                            dot_nib8(wm, hc + (m * kHParts + p) * 4, a0, a1);
                    }
                } else {
                    const u32x4 wv = W[slot][0];  // 64 codes: dwords 2 half, 2 half + 1 hold this half
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        const uint32_t wm = wv[2 * half + m];
#pragma unroll
                        for (int p = 0; p < kHParts; ++p)
                            dot_crumb16(wm, hc + (m * kHParts + p) * 8, a0, a1);
                    }
                }
                part = fmaf((a0 + a1) - sK[lb], sI[lb], part);
            }
            const int lb0 = 2 * (g - ga);
            row = fmaf(f16lo(SB[slot]), part, row);
            row = fmaf(f16hi(SB[slot]), sH[lb0] + sH[lb0 + 1], row);
        }
        if (q + DD < MAXG) {  // refill the slot just consumed
            const int gn = min(g0 + q + DD, gb - 1);
#pragma unroll
            for (int c = 0; c < NW; ++c) W[slot][c] = ldg_nt((const u32x4*)(dcodes + (size_t)gn * SEG + c * 1024));
            SB[slot] = ldg_nt((const uint32_t*)(dsb + (size_t)gn * SEG));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    red[wave * 64 + lane] = row;
    __syncthreads();
    if (wave != 0) return;

    // wave 0: this item's partial, then the arrival count for the output tile
    float r = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) r += red[w * 64 + lane];
    float* dp = a.dpart + ((size_t)t * a.n_otiles + ot) * a.n_items * 64 + lane;
    __hip_atomic_store(dp + item * 64, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // the coherent store above has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    uint32_t* ctr = a.dctr + ((size_t)t * a.n_otiles + ot) * kCounterStride;
    uint32_t prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0, 64);
    if (prev != (uint32_t)a.n_items - 1) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // last arrival: load every item's partial and the gate weights first, then
    // sum the items in a fixed order
    float pv[kMaxItems], wv[kMaxTopK];
#pragma unroll
    for (int it = 0; it < kMaxItems; ++it)
        pv[it] = __hip_atomic_load(dp + min(it, a.n_items - 1) * 64, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj)
        wv[jj] = a.w ? a.w[(size_t)t * a.k + min(jj, a.k - 1)] : 0.0f;
    float ys = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kMaxTopK; ++jj) {
        if (jj < a.k) {
            if (a.eo) a.eo[((size_t)t * (a.k + 1) + jj) * H + o] = pv[jj];
            ys = fmaf(wv[jj], pv[jj], ys);
        }
    }
    float es = 0.0f;
#pragma unroll
    for (int it = 0; it < kMaxItems; ++it)
        if (it >= a.k && it < a.n_items) es += pv[it];
    if (a.eo) a.eo[((size_t)t * (a.k + 1) + a.k) * H + o] = es;
    if (a.y) a.y[(size_t)t * H + o] = ys + es;
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// k_combine: grid (ceil(H/256), T)
__global__ __launch_bounds__(kBlock) void k_combine(CombineArgs a) {
    const int t = blockIdx.y, o = blockIdx.x * kBlock + threadIdx.x;
    if (o >= a.H) return;
    float ys = 0.0f;
    for (int j = 0; j < a.k; ++j)
        ys = fmaf(a.w[(size_t)t * a.k + j], a.eo[((size_t)t * (a.k + 1) + j) * a.H + o], ys);
    ys = ys + a.eo[((size_t)t * (a.k + 1) + a.k) * a.H + o];
    if (a.y_bf16)
        ((uint16_t*)a.y)[(size_t)t * a.H + o] = f32_to_bf16(ys);
    else
        ((float*)a.y)[(size_t)t * a.H + o] = ys;
}

__global__ void k_clear_word(uint32_t* p) { *p = 0u; }

// k_fetch: grid (blocks per record, n).  Each workgroup copies an interleaved
// share of one record's 16-byte vectors, four loads in flight per thread
// (the loads cross PCIe: enough must be outstanding to cover its latency,
// and not so many that they slow each other down).
__global__ __launch_bounds__(kBlock) void k_fetch(FetchArgs f) {
    const int r = blockIdx.y;
    const u32x4* src = (const u32x4*)(f.src + (size_t)f.src_rec[r] * f.rec_bytes);
    u32x4* dst = (u32x4*)(f.dst + (size_t)f.dst_slot[r] * f.rec_bytes);
    const size_t nv = f.rec_bytes / 16, stride = (size_t)gridDim.x * kBlock;
    for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < nv; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * stride < nv) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i + u * stride < nv) dst[i + u * stride] = v[u];
    }
}

// ---------------------------------------------------------------------------
// host-side launchers (called from moe_layer.hip)
// ---------------------------------------------------------------------------
// Router blocks, then (with a.prep) activation preparation blocks running
// beside them, one token per block row.
hipError_t launch_route(const RouteArgs& a, int T, int act_bf16, hipStream_t s) {
    const int rpb = kWaves;  // one router row per wave
    const int nb = (a.E + rpb - 1) / rpb + (a.prep ? ((a.H / 64 + 3) / 4 + kWaves - 1) / kWaves : 0);
    const dim3 grid(nb, T);
    if (a.bits == 2) {
        if (act_bf16) launch_kernel(k_route<1, true, 2>, grid, dim3(kBlock), 0, s, a);
        else launch_kernel(k_route<2, false, 2>, grid, dim3(kBlock), 0, s, a);
    } else {
        if (act_bf16) launch_kernel(k_route<1, true, 4>, grid, dim3(kBlock), 0, s, a);
        else launch_kernel(k_route<2, false, 4>, grid, dim3(kBlock), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const RouteArgs& a, int T, hipStream_t s) {
    if (a.E <= 64) launch_kernel(k_topk<1>, dim3(T), dim3(64), 0, s, a);
    else if (a.E <= 128) launch_kernel(k_topk<2>, dim3(T), dim3(64), 0, s, a);
    else if (a.E <= 256) launch_kernel(k_topk<4>, dim3(T), dim3(64), 0, s, a);
    else launch_kernel(k_topk<16>, dim3(T), dim3(64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prep(const RouteArgs& a, int T, int act_bf16, hipStream_t s) {
    const dim3 grid(((a.H / 64 + 3) / 4 + kWaves - 1) / kWaves, T);  // four groups per wave
    if (a.bits == 2) {
        if (act_bf16) launch_kernel(k_prep<1, true, 2>, grid, dim3(kBlock), 0, s, a);
        else launch_kernel(k_prep<2, false, 2>, grid, dim3(kBlock), 0, s, a);
    } else {
        if (act_bf16) launch_kernel(k_prep<1, true, 4>, grid, dim3(kBlock), 0, s, a);
        else launch_kernel(k_prep<2, false, 4>, grid, dim3(kBlock), 0, s, a);
    }
    return hipGetLastError();
}

template <int XP, int Q, int BITS>
static hipError_t launch_gu_xq(const FfnArgs& a, int T, int n_units, hipStream_t s) {
    const dim3 grid(a.route_units + n_units, T);
    const int NG = a.H / 64;
    const size_t sh = ((size_t)(a.H / 2) * XP + 3 * NG + a.gu_waves * 64) * 4;
    const int m = a.gpw_gu;  // groups per wave: <= 8 with 8 waves, 17..32 with 4 (H > 4096)
#define MOE_GU(MG, W) launch_kernel(k_gate_up<XP, MG, Q, BITS, W>, grid, dim3(64 * W), sh, s, a)
    if (a.gu_waves == kGuWavesSmallH) {
        if (m <= 4) MOE_GU(4, kGuWavesSmallH);
        else MOE_GU(8, kGuWavesSmallH);
    } else {
        if (m <= 24) MOE_GU(24, kGuWavesLargeH);
        else MOE_GU(32, kGuWavesLargeH);
    }
#undef MOE_GU
    return hipGetLastError();
}

template <int XP, int BITS>
static hipError_t launch_gu_xb(const FfnArgs& a, int T, int n, hipStream_t s) {
    if ((!a.logits && !a.route_units) || a.E <= 64) return launch_gu_xq<XP, 1, BITS>(a, T, n, s);  // Q = 1: no selection
    if (a.E <= 128) return launch_gu_xq<XP, 2, BITS>(a, T, n, s);
    if (a.E <= 256) return launch_gu_xq<XP, 4, BITS>(a, T, n, s);
    return launch_gu_xq<XP, 16, BITS>(a, T, n, s);
}

template <int XP>
static hipError_t launch_gu_xp(const FfnArgs& a, int T, int n, hipStream_t s) {
    return a.bits == 2 ? launch_gu_xb<XP, 2>(a, T, n, s) : launch_gu_xb<XP, 4>(a, T, n, s);
}

// units [a.unit_offset, a.unit_offset + n_units) of the k*blk_r routed + blk_s shared units
hipError_t launch_gate_up(const FfnArgs& a, int T, int xparts, int n_units, hipStream_t s) {
    if (n_units <= 0) return hipSuccess;
    return xparts == 2 ? launch_gu_xp<2>(a, T, n_units, s) : launch_gu_xp<1>(a, T, n_units, s);
}

hipError_t launch_down(const FfnArgs& a, int T, hipStream_t s) {
    const dim3 grid(a.n_otiles * a.n_items, T);
    const int nb = 2 * max(a.gi, a.gis);  // blocks staged per item (upper bound)
    const size_t sh = ((size_t)nb * (16 * kHParts + 3) + kWaves * 64) * 4;
    const int m = a.gpw_dn;
    // one group in flight per wave for 4-bit records above hidden 4096 (the
    // largest down grids), else kDnRing
    const bool ring1 = a.bits == 4 && a.H > kGuSmallHMax;
#define MOE_DN(MG)                                                                                   \
    (a.bits == 2 ? launch_kernel(k_down<MG, 2, kDnRing>, grid, dim3(kBlock), sh, s, a)              \
                 : (ring1 ? launch_kernel(k_down<MG, 4, 1>, grid, dim3(kBlock), sh, s, a)           \
                          : launch_kernel(k_down<MG, 4, kDnRing>, grid, dim3(kBlock), sh, s, a)))
    if (m <= 2) MOE_DN(2);
    else if (m <= 4) MOE_DN(4);
    else if (m <= 8) MOE_DN(8);
    else MOE_DN(16);
#undef MOE_DN
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    const dim3 grid((a.H + kBlock - 1) / kBlock, a.T);
    launch_kernel(k_combine, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fetch(const FetchArgs& f, hipStream_t s) {
    if (f.n <= 0) return hipSuccess;
    launch_kernel(k_fetch, dim3(kFetchBlocksPerRecord, f.n), dim3(kBlock), 0, s, f);
    return hipGetLastError();
}

hipError_t launch_clear_word(uint32_t* p, hipStream_t s) {
    launch_kernel(k_clear_word, dim3(1), dim3(1), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe

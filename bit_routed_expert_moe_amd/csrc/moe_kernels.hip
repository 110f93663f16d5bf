// moe_kernels.hip -- gfx950 kernels of the routed-expert MoE layer.
//
//   k_route       router GEMV (int8 rows x activations), then, in the last
//                 workgroup to finish for a token, exact top-k and the gate
//                 weights; optionally prepares the activations for the FFN.
//   k_prep        activation preparation alone (for moe_expert_ffn).
//   k_gate_up     one workgroup per (token, expert slot, block of 32 rows of
//                 I): streams the 64-row gate/up tile, h = silu(g) * u, writes
//                 h prepared as fp16 pairs for the down kernel.
//   k_down        one workgroup per (token, 64 output rows, work item), a work
//                 item being one routed expert or a k-slice of the shared one;
//                 the last item to finish for an output tile sums the items in
//                 a fixed order into per-expert outputs and/or the combined y.
//   k_combine     y = sum_j w_j * eo_j + eo_shared.
//
// Every weight byte is read once per token with 16-byte loads, lane = row of a
// 64-row tile, so one wave instruction reads 1 KB of contiguous record bytes.
// Sums across waves and workgroups are done in a fixed order: reruns are
// bit-identical.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// activation preparation (all threads of the block take part)
// xs: the vector in LDS as fp32; writes pairs/K/X/inv for one vector.
// ---------------------------------------------------------------------------
template <int XP>
__device__ void prep_vector(const float* xs, int n, float max_abs, uint32_t* pairs, float* Kg,
                            float* Xg, float* inv_out) {
    const int e = act_exponent(max_abs);
    const float sc = ldexpf(1.0f, e);
    const int nsets = n / 8;
    for (int s0 = 0; s0 < nsets; s0 += kBlock) {
        const int s = s0 + (int)threadIdx.x;
        const bool ok = s < nsets;
        double ksum = 0.0;
        float xsum = 0.0f;
        if (ok) {
            uint32_t hi[8], lo[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const float a = xs[8 * s + p];
                const float v = a * sc * ((p & 1) ? 0.0625f : 1.0f);
                const _Float16 h = (_Float16)v;
                const float hf = (float)h;
                const _Float16 l = (_Float16)(v - hf);
                hi[p] = __builtin_bit_cast(uint16_t, h);
                lo[p] = __builtin_bit_cast(uint16_t, l);
                ksum += (double)hf;
                if (XP == 2) ksum += (double)(float)l;
                xsum += a;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                pairs[(s * XP + 0) * 4 + m] = hi[m] | (hi[m + 4] << 16);
                if (XP == 2) pairs[(s * XP + 1) * 4 + m] = lo[m] | (lo[m + 4] << 16);
            }
        }
        // sum the 8 sets of each 64-group: 8 consecutive threads
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            ksum += __shfl_xor(ksum, off, 64);
            xsum += __shfl_xor(xsum, off, 64);
        }
        if (ok && (s & 7) == 0) {
            Kg[s >> 3] = (float)(1024.0 * ksum);
            Xg[s >> 3] = xsum;
        }
    }
    if (threadIdx.x == 0) *inv_out = ldexpf(1.0f, -e);
}

// loads x[t] into LDS as fp32 and returns max |x| (block-wide)
template <bool BF16>
__device__ float stage_x(const void* x, int t, int H, float* xs, float* red4) {
    float mx = 0.0f;
    for (int i = threadIdx.x; i < H; i += kBlock) {
        const float v = BF16 ? bf16_to_f32(((const uint16_t*)x)[(size_t)t * H + i])
                             : ((const float*)x)[(size_t)t * H + i];
        xs[i] = v;
        mx = fmaxf(mx, fabsf(v));
    }
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
    return mx;
}

// ---------------------------------------------------------------------------
// exact top-k over E <= 1024 logits by one wave, then the renormalised softmax
// gates.  Order: logit descending, ties to the lower id.
// ---------------------------------------------------------------------------
__device__ void topk_softmax_wave(const float* lg, int E, int k, int32_t* ids_out, float* w_out) {
    const int lane = threadIdx.x & 63;
    float v[kMaxExperts / 64];
#pragma unroll
    for (int q = 0; q < kMaxExperts / 64; ++q) {
        const int e = lane + 64 * q;
        v[q] = e < E ? lg[e] : -INFINITY;
    }
    uint32_t taken = 0;
    float sel_l = -INFINITY;
    int sel_id = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < kMaxExperts / 64; ++q) {
            const int e = lane + 64 * q;
            const bool cand = e < E && !((taken >> q) & 1u);
            if (cand && (v[q] > bv || (v[q] == bv && e < bi))) {
                bv = v[q];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
            sel_l = bv;
            sel_id = bi;
        }
    }
    const float m = __shfl(sel_l, 0, 64);  // the first pick is the largest
    const float ex = lane < k ? expf(sel_l - m) : 0.0f;
    float z = 0.0f;
    for (int j = 0; j < k; ++j) z += __shfl(ex, j, 64);
    if (lane < k) {
        ids_out[lane] = sel_id;
        w_out[lane] = ex / z;
    }
}

// ---------------------------------------------------------------------------
// k_route: grid (ceil(E/4), T), one router row per wave.
// ---------------------------------------------------------------------------
template <int XP, bool BF16>
__global__ __launch_bounds__(kBlock) void k_route(RouteArgs a) {
    extern __shared__ float xs[];  // [H]
    __shared__ float red4[kWaves];
    __shared__ int is_last;
    const int t = blockIdx.y;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const float mx = stage_x<BF16>(a.x, t, a.H, xs, red4);

    const int e = blockIdx.x * kRouterRowsPerBlock + wave;
    if (e < a.E) {
        const u32x4* row = (const u32x4*)(a.rq + (size_t)e * a.H);
        float acc = 0.0f;
        for (int c = lane; c < a.H / 16; c += 64) {
            const u32x4 q = ldg_nt(row + c);
            const float* xv = xs + 16 * c;
            const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
#pragma unroll
                for (int bsel = 0; bsel < 4; ++bsel) {
                    const int qv = (int)(int8_t)(qq[d] >> (8 * bsel));
                    acc = fmaf((float)qv, xv[4 * d + bsel], acc);
                }
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            a.logits[(size_t)t * a.E + e] = acc * (float)__builtin_bit_cast(_Float16, a.rs[e]);
            __threadfence();
        }
    }
    if (a.prep && blockIdx.x == 0) {
        prep_vector<XP>(xs, a.H, mx, a.xpairs + (size_t)t * (a.H / 2) * XP,
                        a.xK + (size_t)t * (a.H / 64), a.xX + (size_t)t * (a.H / 64), a.xinv + t);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t prev = atomicAdd(a.ctr + t, 1u);
        is_last = prev == gridDim.x - 1;
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    if (wave == 0) {
        topk_softmax_wave(a.logits + (size_t)t * a.E, a.E, a.k, a.ids + (size_t)t * a.k,
                          a.w + (size_t)t * a.k);
        if (lane == 0) a.ctr[t] = 0;
    }
}

// k_prep: grid (T); prepares x[t] for the FFN kernels.
template <int XP, bool BF16>
__global__ __launch_bounds__(kBlock) void k_prep(RouteArgs a) {
    extern __shared__ float xs[];
    __shared__ float red4[kWaves];
    const int t = blockIdx.x;
    const float mx = stage_x<BF16>(a.x, t, a.H, xs, red4);
    prep_vector<XP>(xs, a.H, mx, a.xpairs + (size_t)t * (a.H / 2) * XP,
                    a.xK + (size_t)t * (a.H / 64), a.xX + (size_t)t * (a.H / 64), a.xinv + t);
}

// ---------------------------------------------------------------------------
// k_gate_up: grid (k*blk_r + blk_s, T).  Lane = row of the 64-row GU tile
// (rows 0..31 gate, 32..63 up); waves split the H/64 input groups.
// ---------------------------------------------------------------------------
template <int XP, int MAXG>
__global__ __launch_bounds__(kBlock) void k_gate_up(FfnArgs a) {
    extern __shared__ uint32_t smem[];
    const int H = a.H, NG = H / 64;
    uint32_t* xp = smem;                                 // [H/2*XP]
    float* sK = (float*)(xp + (H / 2) * XP);             // [NG]
    float* sX = sK + NG;                                 // [NG]
    float* red = sX + NG;                                // [4][64]
    __shared__ float s_inv;

    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int t = blockIdx.y, u = blockIdx.x;
    int j, b, Ie;
    const uint8_t* rec;
    bool bad = false;
    if (u < a.k * a.blk_r) {
        j = u / a.blk_r;
        b = u - j * a.blk_r;
        int e = a.ids[(size_t)t * a.k + j];
        if (e < 0 || e >= a.E) {
            bad = true;
            e = 0;
        }
        rec = a.experts + (size_t)e * a.rec_bytes;
        Ie = a.I;
    } else {
        j = a.k;
        b = u - a.k * a.blk_r;
        rec = a.shared;
        Ie = a.Is;
    }
    const uint8_t* tile = rec + (size_t)48 * H * b + (size_t)lane * 16;
    const uint8_t* sbt = rec + (size_t)3 * H * Ie / 2 + (size_t)12 * H * (b >> 1) +
                         (size_t)4 * H * (b & 1) + (size_t)lane * 4;
    const int g0 = wave * a.gpw_gu;
    const int g1 = min(NG, g0 + a.gpw_gu);

    // issue every weight load of this wave before touching LDS
    u32x4 W[2 * MAXG];
    uint32_t SB[MAXG];
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
        const int g = g0 + q;
        if (g < g1) {
            W[2 * q] = ldg_nt((const u32x4*)(tile + (size_t)(2 * g) * 1024));
            W[2 * q + 1] = ldg_nt((const u32x4*)(tile + (size_t)(2 * g + 1) * 1024));
            SB[q] = ldg_nt((const uint32_t*)(sbt + (size_t)g * 256));
        }
    }
    // stage the prepared activations of token t
    {
        const uint32_t* gx = a.xpairs + (size_t)t * (H / 2) * XP;
        for (int i = threadIdx.x; i < (H / 2) * XP; i += kBlock) xp[i] = gx[i];
        for (int i = threadIdx.x; i < NG; i += kBlock) {
            sK[i] = a.xK[(size_t)t * NG + i];
            sX[i] = a.xX[(size_t)t * NG + i];
        }
        if (threadIdx.x == 0) s_inv = a.xinv[t];
    }
    __syncthreads();

    float rs = 0.0f, rb = 0.0f;
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
        const int g = g0 + q;
        if (g < g1) {
            float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const u32x4 wv = W[2 * q + half];
                const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
                const uint32_t* xc = xp + (size_t)(2 * g + half) * 16 * XP;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
#pragma unroll
                    for (int p = 0; p < XP; ++p) dot_nib8(wd[m], xc + (m * XP + p) * 4, a0, a1);
                }
            }
            rs = fmaf(f16lo(SB[q]), (a0 + a1) - sK[g], rs);
            rb = fmaf(f16hi(SB[q]), sX[g], rb);
        }
    }
    red[wave * 64 + lane] = fmaf(rs, s_inv, rb);
    __syncthreads();
    if (wave != 0) return;

    // wave 0: gate/up sums in wave order, h = silu(g) * u, then h prepared
    float h = 0.0f;
    if (lane < 32) {
        float g = 0.0f, uu = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            g += red[w * 64 + lane];
            uu += red[w * 64 + 32 + lane];
        }
        h = bad ? __builtin_nanf("") : g / (1.0f + expf(-g)) * uu;
    }
    if (bad && lane == 0) atomicOr(a.err, 1u);
    const float mx = wave_max(lane < 32 ? fabsf(h) : 0.0f);
    const int e = act_exponent(mx);
    const int p = lane & 7, set = lane >> 3;
    const float v = h * ldexpf(1.0f, e) * ((p & 1) ? 0.0625f : 1.0f);
    const _Float16 hh = (_Float16)v;
    const _Float16 hl = (_Float16)(v - (float)hh);
    double kd = lane < 32 ? (double)(float)hh + (kHParts == 2 ? (double)(float)hl : 0.0) : 0.0;
    kd = wave_sum_d(kd);
    const float hs = wave_sum(lane < 32 ? h : 0.0f);
    const uint32_t bh = __builtin_bit_cast(uint16_t, hh), bl = __builtin_bit_cast(uint16_t, hl);
    const uint32_t ph = __shfl_down(bh, 4, 64), pl = __shfl_down(bl, 4, 64);
    const size_t slot = ((size_t)t * (a.k + 1) + j) * a.blk_max + b;
    uint32_t* hp = a.hpairs + slot * (16 * kHParts);
    if (lane < 32 && p < 4) {
        hp[(set * kHParts + 0) * 4 + p] = bh | (ph << 16);
        if (kHParts == 2) hp[(set * kHParts + 1) * 4 + p] = bl | (pl << 16);
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
// mode bit 0: write per-expert outputs eo; bit 1: write combined y.
// ---------------------------------------------------------------------------
template <int MAXG>
__global__ __launch_bounds__(kBlock) void k_down(FfnArgs a) {
    extern __shared__ uint32_t smem[];
    __shared__ int is_last;
    const int H = a.H;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int t = blockIdx.y;
    const int ot = blockIdx.x / a.n_items, item = blockIdx.x - ot * a.n_items;
    int j, ga, gb, Ie;
    const uint8_t* rec;
    if (item < a.k) {
        j = item;
        int e = a.ids[(size_t)t * a.k + j];
        if (e < 0 || e >= a.E) e = 0;  // h of this slot is NaN already
        rec = a.experts + (size_t)e * a.rec_bytes;
        Ie = a.I;
        ga = 0;
        gb = a.I / 64;
    } else {
        j = a.k;
        rec = a.shared;
        Ie = a.Is;
        ga = (item - a.k) * a.gi;
        gb = min(ga + a.gi, a.Is / 64);
    }
    const int o = ot * 64 + lane;
    const int g0 = ga + wave * a.gpw_dn;
    const int g1 = min(gb, g0 + a.gpw_dn);
    const uint8_t* dblk = rec + (size_t)32 * H + (size_t)o * 16;
    const uint8_t* dsb = rec + (size_t)3 * H * Ie / 2 + (size_t)8 * H + (size_t)o * 4;

    u32x4 W[2 * MAXG];
    uint32_t SB[MAXG];
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
        const int g = g0 + q;
        if (g < g1) {
            W[2 * q] = ldg_nt((const u32x4*)(dblk + (size_t)48 * H * (2 * g)));
            W[2 * q + 1] = ldg_nt((const u32x4*)(dblk + (size_t)48 * H * (2 * g + 1)));
            SB[q] = ldg_nt((const uint32_t*)(dsb + (size_t)12 * H * g));
        }
    }
    // stage h of (t, j), blocks [2ga, 2gb)
    const int nb = 2 * (gb - ga);
    uint32_t* sp = smem;                             // [nb][16*kHParts]
    float* sK = (float*)(sp + nb * 16 * kHParts);    // [nb]
    float* sH = sK + nb;                             // [nb]
    float* sI = sH + nb;                             // [nb]
    float* red = sI + nb;                            // [4][64]
    {
        const size_t slot0 = ((size_t)t * (a.k + 1) + j) * a.blk_max + 2 * ga;
        const uint32_t* gp = a.hpairs + slot0 * 16 * kHParts;
        for (int i = threadIdx.x; i < nb * 16 * kHParts; i += kBlock) sp[i] = gp[i];
        for (int i = threadIdx.x; i < nb; i += kBlock) {
            sK[i] = a.hK[slot0 + i];
            sH[i] = a.hHs[slot0 + i];
            sI[i] = a.hinv[slot0 + i];
        }
    }
    __syncthreads();

    float row = 0.0f;
#pragma unroll
    for (int q = 0; q < MAXG; ++q) {
        const int g = g0 + q;
        if (g < g1) {
            float part = 0.0f;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int lb = 2 * (g - ga) + half;  // local h block
                const u32x4 wv = W[2 * q + half];
                const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
                const uint32_t* hc = sp + (size_t)lb * 16 * kHParts;
                float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
#pragma unroll
                    for (int p = 0; p < kHParts; ++p)
                        dot_nib8(wd[m], hc + (m * kHParts + p) * 4, a0, a1);
                }
                part = fmaf((a0 + a1) - sK[lb], sI[lb], part);
            }
            const int lb0 = 2 * (g - ga);
            row = fmaf(f16lo(SB[q]), part, row);
            row = fmaf(f16hi(SB[q]), sH[lb0] + sH[lb0 + 1], row);
        }
    }
    red[wave * 64 + lane] = row;
    __syncthreads();
    if (wave == 0) {
        float r = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) r += red[w * 64 + lane];
        a.dpart[(((size_t)t * a.n_otiles + ot) * a.n_items + item) * 64 + lane] = r;
        __threadfence();
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t prev = atomicAdd(a.dctr + (size_t)t * a.n_otiles + ot, 1u);
        is_last = prev == (uint32_t)a.n_items - 1;
    }
    __syncthreads();
    if (!is_last || wave != 0) return;
    __threadfence();
    const float* dp = a.dpart + ((size_t)t * a.n_otiles + ot) * a.n_items * 64 + lane;
    float ys = 0.0f;
    for (int jj = 0; jj < a.k; ++jj) {
        const float v = dp[jj * 64];
        if (a.eo) a.eo[((size_t)t * (a.k + 1) + jj) * H + o] = v;
        ys = fmaf(a.w ? a.w[(size_t)t * a.k + jj] : 0.0f, v, ys);
    }
    float es = 0.0f;
    for (int it = a.k; it < a.n_items; ++it) es += dp[it * 64];
    if (a.eo) a.eo[((size_t)t * (a.k + 1) + a.k) * H + o] = es;
    if (a.y) a.y[(size_t)t * H + o] = ys + es;
    if (lane == 0) a.dctr[(size_t)t * a.n_otiles + ot] = 0;
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

// ---------------------------------------------------------------------------
// host-side launchers (called from moe_layer.hip)
// ---------------------------------------------------------------------------
hipError_t launch_route(const RouteArgs& a, int T, int act_bf16, hipStream_t s) {
    const dim3 grid((a.E + kRouterRowsPerBlock - 1) / kRouterRowsPerBlock, T);
    const size_t sh = (size_t)a.H * sizeof(float);
    if (act_bf16)
        hipLaunchKernelGGL((k_route<1, true>), grid, dim3(kBlock), sh, s, a);
    else
        hipLaunchKernelGGL((k_route<2, false>), grid, dim3(kBlock), sh, s, a);
    return hipGetLastError();
}

hipError_t launch_prep(const RouteArgs& a, int T, int act_bf16, hipStream_t s) {
    const size_t sh = (size_t)a.H * sizeof(float);
    if (act_bf16)
        hipLaunchKernelGGL((k_prep<1, true>), dim3(T), dim3(kBlock), sh, s, a);
    else
        hipLaunchKernelGGL((k_prep<2, false>), dim3(T), dim3(kBlock), sh, s, a);
    return hipGetLastError();
}

template <int XP>
static hipError_t launch_gu_xp(const FfnArgs& a, int T, hipStream_t s) {
    const dim3 grid(a.k * a.blk_r + a.blk_s, T);
    const int NG = a.H / 64;
    const size_t sh = ((size_t)(a.H / 2) * XP + 2 * NG + kWaves * 64) * 4;
    const int m = a.gpw_gu;
#define MOE_GU(MG) hipLaunchKernelGGL((k_gate_up<XP, MG>), grid, dim3(kBlock), sh, s, a)
    if (m <= 4) MOE_GU(4);
    else if (m <= 8) MOE_GU(8);
    else if (m <= 12) MOE_GU(12);
    else if (m <= 16) MOE_GU(16);
    else if (m <= 24) MOE_GU(24);
    else MOE_GU(32);
#undef MOE_GU
    return hipGetLastError();
}

hipError_t launch_gate_up(const FfnArgs& a, int T, int xparts, hipStream_t s) {
    return xparts == 2 ? launch_gu_xp<2>(a, T, s) : launch_gu_xp<1>(a, T, s);
}

hipError_t launch_down(const FfnArgs& a, int T, hipStream_t s) {
    const dim3 grid(a.n_otiles * a.n_items, T);
    const int nb = 2 * a.gi;  // blocks staged per item (upper bound)
    const size_t sh = ((size_t)nb * (16 * kHParts + 3) + kWaves * 64) * 4;
    const int m = a.gpw_dn;
#define MOE_DN(MG) hipLaunchKernelGGL((k_down<MG>), grid, dim3(kBlock), sh, s, a)
    if (m <= 2) MOE_DN(2);
    else if (m <= 4) MOE_DN(4);
    else if (m <= 8) MOE_DN(8);
    else MOE_DN(16);
#undef MOE_DN
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    const dim3 grid((a.H + kBlock - 1) / kBlock, a.T);
    hipLaunchKernelGGL(k_combine, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_clear_word(uint32_t* p, hipStream_t s) {
    hipLaunchKernelGGL(k_clear_word, dim3(1), dim3(1), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe

// moe_prefill.hip -- multi-token (prefill) path: experts grouped by selection
// and run as MFMA grouped dequant GEMMs, so that each selected expert's
// weights are streamed once per chunk and applied to every token routed to it.
//
//   k_prep_tokens   per (token, 64-input group): fp16 parts of x * 2^e, with
//                   e chosen so the group's largest value is below 2^14; the
//                   group's input sum and 2^-e.
//   k_group         one workgroup: (token, slot) pairs sorted by expert
//                   (stable), and a tile list of at most 16 rows per tile;
//                   the shared expert adds tiles of 16 consecutive tokens.
//   k_gu_grouped    per (tile, 64 rows of I): each wave computes gate and up
//                   for 16 rows of I over all of H with v_mfma_f32_16x16x32_f16;
//                   h = silu(gate) * up, stored as fp16 with a per-(row,
//                   64-group) power-of-two scale, plus the group's sum of h.
//   k_down_grouped  per (tile, 64 outputs): each wave computes 16 outputs over
//                   all of I; writes each row's expert output (unweighted).
// The combine is the decode path's k_combine (fixed order, shared last).
//
// Numerics follow the affine group quantisation directly: the MFMA operand B
// holds the exact integer codes q (nibble | 0x6400 is fp16 1024 + q, minus
// 1024), so per 64-input group
//     sum_i (s q_i + b) x_i = s * sum_i q_i x_i + b * sum_i x_i,
// with the group's scale s and bias b applied in fp32 after its two MFMA
// steps.  Activations enter as fp16 (bf16 inputs exactly; fp32 inputs as a
// hi + lo pair), so the only fp16 rounding beyond the inputs is that of h.
//
// Nibble order: one dword holds 8 inputs, input 2m in the low nibble of byte m.
// The unpack yields them in the order (0,4,1,5,2,6,3,7) with the odd inputs
// scaled by 16; activations are stored in that order ("slot order") with odd
// inputs divided by 16, which is exact in fp16.
//
// MFMA 16x16x32 f16 operand layout (lane l): A[l%16][8*(l/16)+i],
// B[8*(l/16)+i][l%16], D[4*(l/16)+r][l%16].
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kPfDepth = 4;  // 64-input groups in flight per wave

// slot of input p (0..7) within its 8: inverse of (0,4,1,5,2,6,3,7)
__device__ __forceinline__ int slot_of(int p) { return p < 4 ? 2 * p : 2 * (p - 4) + 1; }

// 8 nibbles of one dword -> the 8 exact codes as fp16, in slot order, odd
// inputs times 16.
__device__ __forceinline__ half8 codes8(uint32_t w) {
    const uint32_t M = 0x64006400u;
    const uint32_t w8 = w >> 8;
    const half2v off = {(_Float16)1024.0f, (_Float16)1024.0f};
    const half2v p0 = __builtin_bit_cast(half2v, (w & 0x000F000Fu) | M) - off;   // q0, q4
    const half2v p1 = __builtin_bit_cast(half2v, (w & 0x00F000F0u) | M) - off;   // 16q1, 16q5
    const half2v p2 = __builtin_bit_cast(half2v, (w8 & 0x000F000Fu) | M) - off;  // q2, q6
    const half2v p3 = __builtin_bit_cast(half2v, (w8 & 0x00F000F0u) | M) - off;  // 16q3, 16q7
    half8 o;
    o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
    o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
    return o;
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, uint32_t w, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), codes8(w), c, 0, 0, 0);
}

// max / sum over the 16 lanes of a DPP row; lane 0 of each row gets a value
// whose summation order is fixed.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    return fmaxf(v, dpp<0x128>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x124>(v);
    return v + dpp<0x128>(v);
}

// ---------------------------------------------------------------------------
// k_prep_tokens: grid (ceil(H/256), T), 256 threads; wave = one 64-input group.
// ---------------------------------------------------------------------------
template <int XP, bool BF16>
__global__ __launch_bounds__(kBlock) void k_prep_tokens(PrefillArgs a) {
    const int t = blockIdx.y, H = a.H, NG = H / 64;
    const int g = blockIdx.x * kWaves + wave_id(), lane = threadIdx.x & 63;
    if (g >= NG) return;
    const size_t gi = (size_t)t * H + 64 * g + lane;
    const float v = BF16 ? bf16_to_f32(((const uint16_t*)a.x)[gi]) : ((const float*)a.x)[gi];
    const int e = act_exponent(wave_max(fabsf(v)));
    const int p = lane & 7;
    const float vs = v * ldexpf(1.0f, e) * ((p & 1) ? 0.0625f : 1.0f);
    const uint16_t hi = f16bits(vs);
    const size_t dst = (size_t)t * H + 64 * g + (lane & ~7) + slot_of(p);
    a.x16[dst] = hi;
    if (XP == 2) {
        const float r = vs - (float)__builtin_bit_cast(_Float16, hi);
        a.x16[(size_t)a.T * H + dst] = f16bits(r);
    }
    const double xs = wave_sum_d((double)v);
    if (lane == 0) {
        a.xsum[(size_t)t * NG + g] = (float)xs;
        a.xinv[(size_t)t * NG + g] = ldexpf(1.0f, -e);
    }
}

// ---------------------------------------------------------------------------
// k_group: one workgroup of 256 threads.
// tiles[i] = {expert (or -1 = shared), first row, rows, 0}; rows of a routed
// tile are positions in the expert-sorted pair list, rows of a shared tile are
// tokens.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_group(PrefillArgs a) {
    __shared__ int hist[kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];
    __shared__ int running[kMaxExperts];
    __shared__ int chunk_e[kBlock];
    __shared__ int tile_base[kMaxExperts + 1];
    const int E = a.E, P = a.T * a.k, tid = threadIdx.x;
    for (int e = tid; e < E; e += kBlock) {
        hist[e] = 0;
        running[e] = 0;
    }
    __syncthreads();
    for (int p = tid; p < P; p += kBlock) {
        int e = a.ids[p];
        if (e < 0 || e >= E) {  // flagged; the slot's output is poisoned by k_down_grouped
            atomicOr(a.err, 1u);
            e = 0;
        }
        atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0, tiles = 0;
        for (int e = 0; e < E; ++e) {
            offs[e] = run;
            run += hist[e];
            tile_base[e] = tiles;
            tiles += (hist[e] + kTileRows - 1) / kTileRows;
        }
        offs[E] = run;
        tile_base[E] = tiles;
    }
    __syncthreads();
    // stable scatter, 256 pairs at a time
    for (int p0 = 0; p0 < P; p0 += kBlock) {
        const int p = p0 + tid;
        int e = -1;
        if (p < P) {
            e = a.ids[p];
            e = (e < 0 || e >= E) ? 0 : e;
        }
        chunk_e[tid] = e;
        __syncthreads();
        if (p < P) {
            int rank = 0;
            for (int q = 0; q < tid; ++q) rank += chunk_e[q] == e;
            const int pos = offs[e] + running[e] + rank;
            a.pair_tok[pos] = p / a.k;
            a.pair_slot[pos] = p % a.k;
        }
        __syncthreads();
        if (p < P) atomicAdd(&running[e], 1);
        __syncthreads();
    }
    // tiles
    for (int e = tid; e < E; e += kBlock) {
        const int n = hist[e];
        for (int i = 0; i * kTileRows < n; ++i) {
            int4 tl;
            tl.x = e;
            tl.y = offs[e] + i * kTileRows;
            tl.z = min(kTileRows, n - i * kTileRows);
            tl.w = 0;
            a.tiles[tile_base[e] + i] = tl;
        }
    }
    const int routed_tiles = tile_base[E];
    const int shared_tiles = a.Is ? (a.T + kTileRows - 1) / kTileRows : 0;
    for (int i = tid; i < shared_tiles; i += kBlock) {
        int4 tl;
        tl.x = -1;
        tl.y = i * kTileRows;
        tl.z = min(kTileRows, a.T - i * kTileRows);
        tl.w = 0;
        a.tiles[routed_tiles + i] = tl;
    }
    if (tid == 0) a.n_tiles[0] = routed_tiles + shared_tiles;
}

// ---------------------------------------------------------------------------
// k_gu_grouped: grid (tile capacity, max(I, Is)/64), 256 threads.
// Workgroup (tile, g) covers rows [64g, 64g+64) of I: GU tiles 2g and 2g+1.
// Wave w: GU tile 2g + (w >> 1), gate rows 16*(w & 1) + n and the matching up
// rows 32 + 16*(w & 1) + n, over all 64-input groups of H.
// ---------------------------------------------------------------------------
template <int XP>
__global__ __launch_bounds__(kBlock) void k_gu_grouped(PrefillArgs a) {
    extern __shared__ float dsm[];  // [H/64][16] group sums, then [H/64][16] 2^-e
    __shared__ int s_tok[kTileRows];
    __shared__ float s_mx[kWaves][kTileRows];
    __shared__ float s_hs[kWaves][kTileRows];
    const int tidx = blockIdx.x;
    if (tidx >= a.n_tiles[0]) return;
    const int4 tl = a.tiles[tidx];
    const bool shared = tl.x < 0;
    const int Ie = shared ? a.Is : a.I;
    const int g = blockIdx.y;
    if (g >= Ie / 64) return;
    const int H = a.H, NG = H / 64;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int n = lane & 15, kq = lane >> 4;
    const int tt = wave >> 1, hf = wave & 1;
    float* sX = dsm;
    float* sXi = dsm + NG * kTileRows;

    // rows of the tile: token of each, then the tokens' group sums and scales
    for (int i = threadIdx.x; i < NG * kTileRows; i += kBlock) {
        const int m = i & (kTileRows - 1), jg = i >> 4;
        const int tok = m < tl.z ? (shared ? tl.y + m : a.pair_tok[tl.y + m]) : -1;
        sX[i] = tok < 0 ? 0.0f : a.xsum[(size_t)tok * NG + jg];
        sXi[i] = tok < 0 ? 0.0f : a.xinv[(size_t)tok * NG + jg];
        if (jg == 0) s_tok[m] = tok;
    }
    __syncthreads();

    const uint8_t* rec = shared ? a.shared : a.experts + (size_t)tl.x * a.rec_bytes;
    const int b = 2 * g + tt, rg = 16 * hf + n, ru = 32 + rg;
    const uint8_t* wg = rec + (size_t)48 * H * b + rg * 16 + kq * 4;
    const uint8_t* wu = rec + (size_t)48 * H * b + ru * 16 + kq * 4;
    const uint8_t* sbt = rec + (size_t)3 * H * Ie / 2 + (size_t)12 * H * g + (size_t)4 * H * tt;
    const int tok_n = max(s_tok[n], 0);  // padded rows compute on token 0; discarded
    const uint16_t* xr = a.x16 + (size_t)tok_n * H + 8 * kq;
    const size_t xpart = (size_t)a.T * H;

    // ring of kPfDepth groups: per group 2 chunks of A (per part), gate and up
    // code dwords of both chunks, and the gate and up scale/bias pairs
    u32x4 A[kPfDepth][2][XP];
    uint32_t WG[kPfDepth][2], WU[kPfDepth][2], SG[kPfDepth], SU[kPfDepth];
    auto load = [&](int q, int jg) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int p = 0; p < XP; ++p)
                A[q][c][p] = *(const u32x4*)(xr + p * xpart + 64 * jg + 32 * c);
            WG[q][c] = ldg_nt((const uint32_t*)(wg + (size_t)(2 * jg + c) * 1024));
            WU[q][c] = ldg_nt((const uint32_t*)(wu + (size_t)(2 * jg + c) * 1024));
        }
        SG[q] = *(const uint32_t*)(sbt + (size_t)jg * 256 + rg * 4);
        SU[q] = *(const uint32_t*)(sbt + (size_t)jg * 256 + ru * 4);
    };
#pragma unroll
    for (int q = 0; q < kPfDepth; ++q) {
        load(q, min(q, NG - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    for (int j0 = 0; j0 < NG; j0 += kPfDepth) {
#pragma unroll
        for (int q = 0; q < kPfDepth; ++q) {
            const int jg = j0 + q;
            if (jg < NG) {
                f32x4 pg = {0, 0, 0, 0}, pu = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int p = 0; p < XP; ++p) {
                        pg = mfma(A[q][c][p], WG[q][c], pg);
                        pu = mfma(A[q][c][p], WU[q][c], pu);
                    }
                const f32x4 xi = *(const f32x4*)&sXi[jg * kTileRows + 4 * kq];
                const f32x4 xs = *(const f32x4*)&sX[jg * kTileRows + 4 * kq];
                const float sg = f16lo(SG[q]), bg = f16hi(SG[q]);
                const float su = f16lo(SU[q]), bu = f16hi(SU[q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    accg[r] = fmaf(bg, xs[r], fmaf(sg, pg[r] * xi[r], accg[r]));
                    accu[r] = fmaf(bu, xs[r], fmaf(su, pu[r] * xi[r], accu[r]));
                }
            }
            load(q, min(jg + kPfDepth, NG - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // h = silu(gate) * up for rows 4kq + r, column 32*tt + 16*hf + n of the group
    float h[4], mx[4], hs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float gv = accg[r];
        h[r] = s_tok[4 * kq + r] < 0 ? 0.0f : gv / (1.0f + expf(-gv)) * accu[r];
        mx[r] = row16_max(fabsf(h[r]));
        hs[r] = row16_sum(h[r]);
    }
    if (n == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s_mx[wave][4 * kq + r] = mx[r];
            s_hs[wave][4 * kq + r] = hs[r];
        }
    }
    __syncthreads();
    const int NGi = a.Imax / 64;
    const int col = 64 * g + 32 * tt + 16 * hf + n;
    const int hcol = (col & ~7) + slot_of(n & 7);
    const float odd = (n & 1) ? 0.0625f : 1.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= tl.z) continue;
        const float M = fmaxf(fmaxf(s_mx[0][m], s_mx[1][m]), fmaxf(s_mx[2][m], s_mx[3][m]));
        const int e = act_exponent(M);
        const size_t hrow = shared ? (size_t)a.P + tl.y + m : (size_t)(tl.y + m);
        a.h16[hrow * a.Imax + hcol] = f16bits(h[r] * ldexpf(1.0f, e) * odd);
        if (wave == 0 && n == 0) {
            a.hsum[hrow * NGi + g] = ((s_hs[0][m] + s_hs[1][m]) + s_hs[2][m]) + s_hs[3][m];
            a.hinv[hrow * NGi + g] = ldexpf(1.0f, -e);
        }
    }
}

// ---------------------------------------------------------------------------
// k_down_grouped: grid (tile capacity, H/64), 256 threads.  Wave w computes
// outputs o0 + 16w + n over all 64-groups of I.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_down_grouped(PrefillArgs a) {
    extern __shared__ float dsm[];  // [Ie/64][16] group sums of h, then [Ie/64][16] 2^-e
    __shared__ int s_row[kTileRows];
    const int tidx = blockIdx.x;
    if (tidx >= a.n_tiles[0]) return;
    const int4 tl = a.tiles[tidx];
    const bool shared = tl.x < 0;
    const int Ie = shared ? a.Is : a.I;
    const int NGe = Ie / 64, NGi = a.Imax / 64;
    const int H = a.H;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int n = lane & 15, kq = lane >> 4;
    float* sH = dsm;
    float* sHi = dsm + NGe * kTileRows;
    for (int i = threadIdx.x; i < NGe * kTileRows; i += kBlock) {
        const int m = i & (kTileRows - 1), jg = i >> 4;
        const int row = m < tl.z ? (shared ? a.P + tl.y + m : tl.y + m) : -1;
        sH[i] = row < 0 ? 0.0f : a.hsum[(size_t)row * NGi + jg];
        sHi[i] = row < 0 ? 0.0f : a.hinv[(size_t)row * NGi + jg];
        if (jg == 0) s_row[m] = row;
    }
    __syncthreads();
    const uint8_t* rec = shared ? a.shared : a.experts + (size_t)tl.x * a.rec_bytes;
    const int o = blockIdx.y * 64 + 16 * wave + n;
    const uint8_t* wd = rec + (size_t)32 * H + (size_t)o * 16 + kq * 4;
    const uint8_t* sbd = rec + (size_t)3 * H * Ie / 2 + (size_t)8 * H + (size_t)o * 4;
    const uint16_t* hr = a.h16 + (size_t)max(s_row[n], 0) * a.Imax + 8 * kq;

    u32x4 A[kPfDepth][2];
    uint32_t W[kPfDepth][2], SB[kPfDepth];
    auto load = [&](int q, int jg) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            A[q][c] = *(const u32x4*)(hr + 64 * jg + 32 * c);
            W[q][c] = ldg_nt((const uint32_t*)(wd + (size_t)48 * H * (2 * jg + c)));
        }
        SB[q] = *(const uint32_t*)(sbd + (size_t)12 * H * jg);
    };
#pragma unroll
    for (int q = 0; q < kPfDepth; ++q) {
        load(q, min(q, NGe - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 acc = {0, 0, 0, 0};
    for (int j0 = 0; j0 < NGe; j0 += kPfDepth) {
#pragma unroll
        for (int q = 0; q < kPfDepth; ++q) {
            const int jg = j0 + q;
            if (jg < NGe) {
                f32x4 pd = {0, 0, 0, 0};
                pd = mfma(A[q][0], W[q][0], pd);
                pd = mfma(A[q][1], W[q][1], pd);
                const f32x4 hi = *(const f32x4*)&sHi[jg * kTileRows + 4 * kq];
                const f32x4 hsum = *(const f32x4*)&sH[jg * kTileRows + 4 * kq];
                const float sd = f16lo(SB[q]), bd = f16hi(SB[q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(bd, hsum[r], fmaf(sd, pd[r] * hi[r], acc[r]));
            }
            load(q, min(jg + kPfDepth, NGe - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= tl.z) continue;
        float v = acc[r];
        int t, j;
        if (shared) {
            t = tl.y + m;
            j = a.k;
        } else {
            t = a.pair_tok[tl.y + m];
            j = a.pair_slot[tl.y + m];
            const int e = a.ids[(size_t)t * a.k + j];
            if (e < 0 || e >= a.E) v = __builtin_nanf("");
        }
        a.eo[((size_t)t * (a.k + 1) + j) * H + o] = v;
    }
}

__global__ void k_zero_shared_rows(PrefillArgs a) {  // no shared expert: eo[:, k, :] = 0
    const int t = blockIdx.y, o = blockIdx.x * kBlock + threadIdx.x;
    if (o < a.H) a.eo[((size_t)t * (a.k + 1) + a.k) * a.H + o] = 0.0f;
}

hipError_t launch_prefill_prep(const PrefillArgs& a, int act_bf16, hipStream_t s) {
    const dim3 grid((a.H / 64 + kWaves - 1) / kWaves, a.T);
    if (a.xparts == 1 && act_bf16)
        hipLaunchKernelGGL((k_prep_tokens<1, true>), grid, dim3(kBlock), 0, s, a);
    else if (a.xparts == 1)
        hipLaunchKernelGGL((k_prep_tokens<1, false>), grid, dim3(kBlock), 0, s, a);
    else if (act_bf16)
        hipLaunchKernelGGL((k_prep_tokens<2, true>), grid, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL((k_prep_tokens<2, false>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_ffn(const PrefillArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_group, dim3(1), dim3(kBlock), 0, s, a);
    const dim3 gu(a.tile_cap, a.Imax / 64);
    const size_t lds_gu = (size_t)(a.H / 64) * kTileRows * 8, lds_dn = (size_t)(a.Imax / 64) * kTileRows * 8;
    if (a.xparts == 1)
        hipLaunchKernelGGL((k_gu_grouped<1>), gu, dim3(kBlock), lds_gu, s, a);
    else
        hipLaunchKernelGGL((k_gu_grouped<2>), gu, dim3(kBlock), lds_gu, s, a);
    hipLaunchKernelGGL(k_down_grouped, dim3(a.tile_cap, a.H / 64), dim3(kBlock), lds_dn, s, a);
    if (!a.Is) hipLaunchKernelGGL(k_zero_shared_rows, dim3((a.H + kBlock - 1) / kBlock, a.T), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

// moe_prefill.hip -- multi-token (prefill) path: experts grouped by selection
// and run as MFMA grouped dequant GEMMs, so that each selected expert's
// weights are streamed once per call and applied to every token routed to it.
//
//   k_prep_tokens   per token: fp16 parts of x * 2^e, with one e per token
//                   chosen so that its largest value is below 2^14; the exact
//                   sum of each 64-input group of x * 2^e.
//   k_route_tiles   router logits as 16-token x 16-expert MFMA tiles over the
//                   prepared activations and the int8 rows turned exactly into
//                   fp16 (k_topk then selects).
//   k_group         one workgroup: (token, slot) pairs grouped by expert
//                   (in any order within an expert: no row of a tile
//                   depends on another), and a tile list of at most 16 rows;
//                   the shared expert adds tiles of 16 consecutive tokens.
//   k_gu_grouped    per (tile, 128 rows of I): wave = one 64-row group of I
//                   (gate and up: 8 MFMA N-tiles of 16) over one half of H;
//                   the two halves are added in a fixed order, then
//                   h = silu(gate) * up is stored as fp16 with a per-(row,
//                   64-group) power-of-two scale, plus the group's sum of h.
//   k_down_grouped  per (tile, 512 outputs): wave = 128 outputs (8 MFMA
//                   N-tiles) over all of I; writes each row's expert output
//                   (unweighted).
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
// 2-bit records: a 16-byte run of a tile row is a whole 64-input group, and
// after the lane transpose a lane holds dword kq (inputs 16kq .. 16kq+15) of
// its rows.  Its codes are taken in place as pairs (q_j, q_{8+j}) scaled by
// 4^j (j < 5; j >= 5 from the dword shifted by 10, scaled by 4^(j-5)); MFMA
// step s of the group uses the pairs j = 4s .. 4s+3.  The activations (and h)
// of that group are stored in the matching 2-bit slot order: input
// 16kq + 8u + j at position 32(j/4) + 8kq + 2(j%4) + u, times the inverse
// power of 4 (exact).
//
// Streams: weights, scale/bias pairs and activations are read with buffer
// loads whose per-lane offsets are loop invariant (the loop advances a scalar
// offset), weights with the nontemporal hint.  A workgroup's waves read the
// same activation rows, which stay in the CU's L1.
//
// MFMA 16x16x32 f16 operand layout (lane l): A[l%16][8*(l/16)+i],
// B[8*(l/16)+i][l%16], D[4*(l/16)+r][l%16].
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kNtGu = 8;  // MFMA N-tiles per wave in k_gu_grouped (64 rows of I, gate + up)
constexpr int kNtDn = 8;  // MFMA N-tiles per wave in k_down_grouped (128 outputs)
constexpr int kAuxNT = 2; // buffer-load cache policy: nontemporal
constexpr int kGuDepth = 2;  // 64-input groups in flight per wave, k_gu_grouped
constexpr int kDnDepth = 2;  // 64-input groups in flight per wave, k_down_grouped
// Scalar offset for ring refills past a wave's last group: with any per-lane
// offset (< 2^28 in a record) the sum lies beyond every record (records are
// under 2^28 bytes) without wrapping 32 bits, so the buffer load is dropped
// (returns 0, no memory traffic) instead of fetching a group again.
constexpr int kPastEnd = 0x7FFFF000;

// slot of input p (0..7) within its 8: inverse of (0,4,1,5,2,6,3,7)
__device__ __forceinline__ int slot_of(int p) { return p < 4 ? 2 * p : 2 * (p - 4) + 1; }

// Unpack constants kept in VGPRs so that each nibble pair costs one
// v_and_or_b32 (a VOP3 cannot take two literal constants).
struct Unpack {
    uint32_t lo, hi, magic;
    __device__ __forceinline__ Unpack() {
        asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(lo));
        asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(hi));
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));
    }
    // 8 of the 16 2-bit codes of one dword (pairs j = 4s .. 4s+3, s = 0 or 1)
    // as fp16 4^j q (4^(j-5) q for j >= 5), in the 2-bit slot order
    template <int S>
    __device__ __forceinline__ half8 crumbs(uint32_t w) const {
        const half2v off = {(_Float16)1024.0f, (_Float16)1024.0f};
        half2v p0, p1, p2, p3;
        if (S == 0) {
            p0 = __builtin_bit_cast(half2v, (w & 0x00030003u) | magic) - off;  // q0, q8
            p1 = __builtin_bit_cast(half2v, (w & 0x000C000Cu) | magic) - off;  // 4 q1, 4 q9
            p2 = __builtin_bit_cast(half2v, (w & 0x00300030u) | magic) - off;  // 16 q2, 16 q10
            p3 = __builtin_bit_cast(half2v, (w & 0x00C000C0u) | magic) - off;  // 64 q3, 64 q11
        } else {
            const uint32_t v = w >> 10;
            p0 = __builtin_bit_cast(half2v, (w & 0x03000300u) | magic) - off;  // 256 q4, 256 q12
            p1 = __builtin_bit_cast(half2v, (v & 0x00030003u) | magic) - off;  // q5, q13
            p2 = __builtin_bit_cast(half2v, (v & 0x000C000Cu) | magic) - off;  // 4 q6, 4 q14
            p3 = __builtin_bit_cast(half2v, (v & 0x00300030u) | magic) - off;  // 16 q7, 16 q15
        }
        half8 o;
        o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
        o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
        return o;
    }
    // 8 nibbles of one dword -> the exact codes as fp16, in slot order, odd
    // inputs times 16
    __device__ __forceinline__ half8 codes(uint32_t w) const {
        const uint32_t w8 = w >> 8;
        const half2v off = {(_Float16)1024.0f, (_Float16)1024.0f};
        const half2v p0 = __builtin_bit_cast(half2v, (w & lo) | magic) - off;   // q0, q4
        const half2v p1 = __builtin_bit_cast(half2v, (w & hi) | magic) - off;   // 16q1, 16q5
        const half2v p2 = __builtin_bit_cast(half2v, (w8 & lo) | magic) - off;  // q2, q6
        const half2v p3 = __builtin_bit_cast(half2v, (w8 & hi) | magic) - off;  // 16q3, 16q7
        half8 o;
        o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
        o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
        return o;
    }
};

__device__ __forceinline__ f32x4 mfma(u32x4 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)min(bytes, (size_t)0x7FFFFFFF),
                                             0x00020000);
}
template <int AUX = 0>
__device__ __forceinline__ uint32_t bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ u32x4 bload4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}

// Lane-group moves on the wave's four 16-lane row groups (gfx950
// v_permlane16_swap / v_permlane32_swap; all 64 lanes must be active).
// xpose4: row group g, register j holds M[g][j] -> row group g, register t
// holds M[t][g].  A wave's 16-byte load of rows 16g + n (lane n of group g)
// becomes, in lane n of group g, dword g of rows n, 16 + n, 32 + n, 48 + n:
// the MFMA B operand of four N-tiles.
__device__ __forceinline__ u32x4 xpose4(u32x4 d) {
    const auto s01 = __builtin_amdgcn_permlane16_swap(d[0], d[1], false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(d[2], d[3], false, false);
    const auto s02 = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(s01[1], s23[1], false, false);
    return u32x4{s02[0], s13[0], s02[1], s13[1]};
}
// bcast4: register t of every row group <- v of row group t (same lane n).
__device__ __forceinline__ u32x4 bcast4(uint32_t v) {
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
    return u32x4{b[0], c[0], b[1], c[1]};
}

// max / sum over the 16 lanes of a DPP row.  Every lane of the row gets the
// max; the sum's rounding order differs between lanes, so only one lane's
// sum is used.
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
// k_prep_tokens: grid (T), 256 threads.
// ---------------------------------------------------------------------------
template <int XP, bool BF16, int BITS>
__global__ __launch_bounds__(kBlock) void k_prep_tokens(PrefillArgs a) {
    __shared__ float row[kMaxHidden];
    __shared__ float red4[kWaves];
    const int t = blockIdx.x, H = a.H, NG = H / 64;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    // the token's row into LDS with 16-byte loads, and its largest magnitude
    float mx = 0.0f;
    constexpr int PER = BF16 ? 8 : 4;                 // values per 16-byte load
    constexpr int NV = kMaxHidden / PER / kBlock;     // loads per thread at the largest hidden size
    const u32x4* src = (const u32x4*)((const uint8_t*)a.x + (size_t)t * H * (BF16 ? 2 : 4));
    u32x4 w[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {  // every load issued before the first wait
        w[j] = src[min((int)threadIdx.x + j * kBlock, H / PER - 1)];  // past the row: a repeat, unused
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = threadIdx.x + j * kBlock;
        if (v >= H / PER) break;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t u = w[j][d];  // bit-cast a scalar copy, never a vector element lvalue
            if (BF16) {
                const float f0 = __builtin_bit_cast(float, u << 16);
                const float f1 = __builtin_bit_cast(float, u & 0xFFFF0000u);
                row[v * 8 + 2 * d] = f0;
                row[v * 8 + 2 * d + 1] = f1;
                mx = fmaxf(mx, fmaxf(fabsf(f0), fabsf(f1)));
            } else {
                const float f = __builtin_bit_cast(float, u);
                row[v * 4 + d] = f;
                mx = fmaxf(mx, fabsf(f));
            }
        }
    }
    mx = wave_max(mx);
    if (lane == 0) red4[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
    const int e = act_exponent(mx);
    const float sc = ldexpf(1.0f, e);
    const int p = lane & 7;
    for (int g = wave; g < NG; g += kWaves) {
        const float vs = row[64 * g + lane] * sc;  // exact: a power-of-two scaling
        const float vq = vs * ((p & 1) ? 0.0625f : 1.0f);
        const uint16_t hi = f16bits(vq);
        const size_t dst = (size_t)t * H + 64 * g + (lane & ~7) + slot_of(p);
        a.x16[dst] = hi;
        if (XP == 2) a.x16[(size_t)a.T * H + dst] = f16bits(vq - (float)__builtin_bit_cast(_Float16, hi));
        if (BITS == 2) {  // the 2-bit slot order for the gate/up operand
            const int j = lane & 7;
            const float v2 = vs * ldexpf(1.0f, crumb_scale_log2(j));
            const uint16_t h2 = f16bits(v2);
            const size_t d2 = (size_t)t * H + 64 * g + 32 * (j >> 2) + 8 * (lane >> 4) + 2 * (j & 3) +
                              ((lane >> 3) & 1);
            a.x16b[d2] = h2;
            if (XP == 2) a.x16b[(size_t)a.T * H + d2] = f16bits(v2 - (float)__builtin_bit_cast(_Float16, h2));
        }
        const double gs = wave_sum_d((double)vs);
        if (lane == 0) a.xsum[(size_t)t * NG + g] = (float)gs;
    }
    if (threadIdx.x == 0) a.xinv[t] = ldexpf(1.0f, -e);
}

// ---------------------------------------------------------------------------
// k_route_tiles: router logits of many tokens.  Grid (ceil(E/16), ceil(T/16)),
// 64*NW threads; the workgroup computes a 16-token x 16-expert tile, wave w
// over the 64-input units [w*U/NW, (w+1)*U/NW), the NW partial sums added in
// wave order.  A = the prepared fp16 activations (slot order, odd inputs / 16,
// token scale 2^e); B = the int8 router bytes turned into fp16 in the same slot
// order with odd inputs x16: byte b + 128 in the mantissa of 1024.0 (or of
// 16384.0, where one mantissa step is 16) minus 1152 (or 18432) is b (or 16 b)
// exactly.  Products are exact in fp32; logit = sum * 2^-e * scale.
// Within a 64-input unit, lane quarter kq owns inputs [16 kq, 16 kq + 16): one
// 16-byte router load and two 16-byte activation loads per lane, the unit's two
// MFMA steps taking the first and the second 8 of them.  (A lane owning 8
// inputs of each 32-input step instead touches twice the cache lines per load
// and measured no faster with 4, 8 or 16 waves.)
// ---------------------------------------------------------------------------

__device__ __forceinline__ half8 router_b(uint32_t lo4, uint32_t hi4) {
    const uint32_t u0 = lo4 ^ 0x80808080u, u1 = hi4 ^ 0x80808080u;  // bytes b + 128
    // inputs (0,4) (1,5) (2,6) (3,7) into the low bytes of two halves
    const uint32_t d0 = __builtin_amdgcn_perm(u1, u0, 0x0C040C00u);
    const uint32_t d1 = __builtin_amdgcn_perm(u1, u0, 0x0C050C01u);
    const uint32_t d2 = __builtin_amdgcn_perm(u1, u0, 0x0C060C02u);
    const uint32_t d3 = __builtin_amdgcn_perm(u1, u0, 0x0C070C03u);
    const half2v o1 = {(_Float16)1152.0f, (_Float16)1152.0f}, o16 = {(_Float16)18432.0f, (_Float16)18432.0f};
    const half2v p0 = __builtin_bit_cast(half2v, d0 | 0x64006400u) - o1;   // b0, b4
    const half2v p1 = __builtin_bit_cast(half2v, d1 | 0x74007400u) - o16;  // 16 b1, 16 b5
    const half2v p2 = __builtin_bit_cast(half2v, d2 | 0x64006400u) - o1;   // b2, b6
    const half2v p3 = __builtin_bit_cast(half2v, d3 | 0x74007400u) - o16;  // 16 b3, 16 b7
    half8 o;
    o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
    o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
    return o;
}

template <int XP, int NW, int D>
__global__ __launch_bounds__(64 * NW) void k_route_tiles(PrefillArgs a) {
    __shared__ float red[NW][kTileRows][kTileRows + 1];
    const int H = a.H, nu = H / 64;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int n = lane & 15, kq = lane >> 4;
    const int e0 = blockIdx.x * kTileRows, t0 = blockIdx.y * kTileRows;
    const int u0 = wave * nu / NW, u1 = (wave + 1) * nu / NW;
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x16, (size_t)XP * a.T * H * 2);
    const __amdgpu_buffer_rsrc_t rr = rsrc(a.rq, (size_t)a.E * H);
    const int xpart = a.T * H * 2;
    const int xo = (min(t0 + n, a.T - 1) * H + 16 * kq) * 2;  // rows past T compute on token T-1; discarded
    const int ro = min(e0 + n, a.E - 1) * H + 16 * kq;
    u32x4 A[D][XP][2];
    u32x4 B[D];
    auto load = [&](int q, int u) {
        const int uc = min(u, u1 - 1);
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            A[q][p][0] = bload4(rx, xo, p * xpart + 128 * uc);
            A[q][p][1] = bload4(rx, xo, p * xpart + 128 * uc + 16);
        }
        B[q] = bload4(rr, ro, 64 * uc);
    };
    f32x4 acc = {0, 0, 0, 0};
    if (u1 > u0) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            load(q, u0 + q);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int ub = u0; ub < u1; ub += D) {
#pragma unroll
            for (int q = 0; q < D; ++q) {
                if (ub + q < u1) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const half8 b = router_b(B[q][2 * j], B[q][2 * j + 1]);
#pragma unroll
                        for (int p = 0; p < XP; ++p) acc = mfma(A[q][p][j], b, acc);
                    }
                }
                load(q, ub + q + D);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * kq + r][n] = acc[r];
    __syncthreads();
    if (threadIdx.x >= kTileRows * kTileRows) return;
    const int m = threadIdx.x >> 4, ei = threadIdx.x & 15;  // token m, expert ei of the tile
    const int t = t0 + m, e = e0 + ei;
    if (t < a.T && e < a.E) {
        float v = red[0][m][ei];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][m][ei];
        a.logits[(size_t)t * a.E + e] = v * a.xinv[t] * (float)__builtin_bit_cast(_Float16, a.rs[e]);
    }
}

// ---------------------------------------------------------------------------
// k_group: one workgroup of 256 threads.
// tiles[i] = {expert (or -1 = shared), first row, rows, 0}; rows of a routed
// tile are positions in the expert-sorted pair list, rows of a shared tile are
// tokens.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_group(PrefillArgs a) {
    constexpr int R = 16;  // pair ids loaded per thread per batch (kBlock * R pairs in one round trip)
    __shared__ int hist[kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];       // exclusive prefix sums of hist
    __shared__ int tile_base[kMaxExperts + 1];  // exclusive prefix sums of the tile counts
    __shared__ int running[kMaxExperts];
    __shared__ int scan[2][kBlock];
    const int E = a.E, P = a.T * a.k, tid = threadIdx.x;
    for (int e = tid; e < E; e += kBlock) {
        hist[e] = 0;
        running[e] = 0;
    }
    __syncthreads();
    auto load_ids = [&](int base, int* v) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int p = base + tid + kBlock * i;
            v[i] = p < P ? a.ids[p] : 0;
        }
    };
    for (int base = 0; base < P; base += kBlock * R) {
        int v[R];
        load_ids(base, v);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (base + tid + kBlock * i >= P) continue;
            int e = v[i];
            if (e < 0 || e >= E) {  // flagged; the slot's output is poisoned by k_down_grouped
                atomicOr(a.err, 1u);
                e = 0;
            }
            atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    // exclusive prefix sums of the pair and tile counts: thread tid owns
    // experts [4 tid, 4 tid + 4), a Hillis-Steele scan over the threads
    int pc[4], tc[4], ps = 0, ts = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        pc[j] = e < E ? hist[e] : 0;
        tc[j] = (pc[j] + kTileRows - 1) / kTileRows;
        ps += pc[j];
        ts += tc[j];
    }
    scan[0][tid] = ps;
    scan[1][tid] = ts;
    __syncthreads();
    for (int d = 1; d < kBlock; d <<= 1) {
        const int p0 = tid >= d ? scan[0][tid - d] : 0, t0 = tid >= d ? scan[1][tid - d] : 0;
        __syncthreads();
        scan[0][tid] += p0;
        scan[1][tid] += t0;
        __syncthreads();
    }
    int po = scan[0][tid] - ps, to = scan[1][tid] - ts;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * tid + j;
        if (e < E) {
            offs[e] = po;
            tile_base[e] = to;
        }
        po += pc[j];
        to += tc[j];
    }
    if (tid == kBlock - 1) {
        offs[E] = scan[0][tid];
        tile_base[E] = scan[1][tid];
    }
    __syncthreads();
    // scatter: each pair takes the next free position of its expert.  The
    // order of an expert's pairs does not change any result (every row of a
    // grouped tile is computed on its own, and written to its own (token,
    // slot)), so the positions come from an LDS atomic per pair.
    for (int base = 0; base < P; base += kBlock * R) {
        int v[R];
        load_ids(base, v);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int p = base + tid + kBlock * i;
            if (p >= P) continue;
            const int e = (v[i] < 0 || v[i] >= E) ? 0 : v[i];
            const int pos = offs[e] + atomicAdd(&running[e], 1);
            a.pair_tok[pos] = p / a.k;
            a.pair_slot[pos] = p % a.k;
        }
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
// k_gu_grouped: grid (tile capacity, ceil(max(I, Is)/128)), 256 threads.
// Wave w: 64-row group gi = 2*blockIdx.y + (w & 1) of I (GU tiles 2gi and
// 2gi+1: N-tiles 0-1 gate and 2-3 up of the first, 4-7 of the second) over
// the half (w >> 1) of the 64-input groups of H.
// Dynamic LDS: [H/64][16] group sums of the rows' activations, then the
// partial sums of the upper-half waves, [2][8][64] float4.
// ---------------------------------------------------------------------------
template <int XP, int BITS>
__global__ __launch_bounds__(kBlock) void k_gu_grouped(PrefillArgs a) {
    extern __shared__ float dsm[];
    __shared__ int s_tok[kTileRows];
    __shared__ float s_xinv[kTileRows];
    const int tidx = blockIdx.x;
    if (tidx >= a.n_tiles[0]) return;
    const int4 tl = a.tiles[tidx];
    const bool shared = tl.x < 0;
    const int Ie = shared ? a.Is : a.I;
    if (2 * (int)blockIdx.y * 64 >= Ie) return;
    const int H = a.H, NG = H / 64;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int n = lane & 15, kq = lane >> 4;
    const int gi = 2 * blockIdx.y + (wave & 1), kh = wave >> 1;
    const bool active = gi * 64 < Ie;
    float* sX = dsm;
    f32x4* red = (f32x4*)(dsm + NG * kTileRows);

    for (int i = threadIdx.x; i < NG * kTileRows; i += kBlock) {
        const int m = i & (kTileRows - 1), jg = i >> 4;
        const int tok = m < tl.z ? (shared ? tl.y + m : a.pair_tok[tl.y + m]) : -1;
        sX[i] = tok < 0 ? 0.0f : a.xsum[(size_t)tok * NG + jg];
        if (jg == 0) {
            s_tok[m] = tok;
            s_xinv[m] = tok < 0 ? 0.0f : a.xinv[tok];
        }
    }
    __syncthreads();

    f32x4 acc[kNtGu];
#pragma unroll
    for (int nt = 0; nt < kNtGu; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
    const int j0 = kh * NG / 2, j1 = (kh + 1) * NG / 2;
    if (active && j1 > j0) {
        const uint8_t* rec = shared ? a.shared : a.experts + (size_t)tl.x * a.rec_bytes;
        const __amdgpu_buffer_rsrc_t rw = rsrc(rec, shared ? a.rec_bytes_shared : a.rec_bytes);
        const __amdgpu_buffer_rsrc_t rx = rsrc(BITS == 2 ? a.x16b : a.x16, (size_t)XP * a.T * H * 2);
        // per-lane offsets (bytes): row 16*kq + n of each GU tile (codes and
        // scale/bias pair; one 16-byte load covers a 1 KB chunk of a tile per
        // wave), and the lane's activations; the rest of each address is
        // uniform and goes in the scalar offset.  A 64-input group's segment
        // is two chunks of nibbles or one chunk of 2-bit codes, then the 64
        // rows' (scale, bias) pairs.
        constexpr int NC = BITS == 4 ? 2 : 1;
        constexpr int SEG = NC * 1024 + 256;
        const int tb = SEG * NG;  // bytes of a 32-row block's segments
        const int rl = 16 * kq + n;
        const int wo[2] = {tb * (2 * gi) + rl * 16, tb * (2 * gi + 1) + rl * 16};
        const int so[2] = {tb * (2 * gi) + NC * 1024 + rl * 4, tb * (2 * gi + 1) + NC * 1024 + rl * 4};
        const int xo = (max(s_tok[n], 0) * H + 8 * kq) * 2;
        const int xpart = a.T * H * 2;
        const Unpack up;
        struct Regs {
            u32x4 A[2][XP];
            u32x4 W[2][NC];  // [GU tile][chunk], rows 16*kq + n
            uint32_t SB[2];
        };
        auto load = [&](Regs& R, int jg) {  // jg >= j1: a refill past the end
            const bool live = jg < j1;
            const int ja = min(jg, j1 - 1);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int p = 0; p < XP; ++p) R.A[c][p] = bload4(rx, xo, p * xpart + 128 * ja + 64 * c);
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    R.W[t2][c] = bload4<kAuxNT>(rw, wo[t2], live ? SEG * jg + 1024 * c : kPastEnd);
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) R.SB[t2] = bload(rw, so[t2], live ? SEG * jg : kPastEnd);
        };
        auto compute = [&](const Regs& R, int jg) {
            const f32x4 xs = *(const f32x4*)&sX[jg * kTileRows + 4 * kq];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const u32x4 w0 = xpose4(R.W[t2][0]), w1 = xpose4(R.W[t2][NC - 1]);
                const u32x4 sb = bcast4(R.SB[t2]);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int nt = 4 * t2 + t;
                    f32x4 pg = {0, 0, 0, 0};
                    const half8 q0 = BITS == 4 ? up.codes(w0[t]) : up.crumbs<0>(w0[t]);
                    const half8 q1 = BITS == 4 ? up.codes(w1[t]) : up.crumbs<1>(w0[t]);
#pragma unroll
                    for (int p = 0; p < XP; ++p) pg = mfma(R.A[0][p], q0, pg);
#pragma unroll
                    for (int p = 0; p < XP; ++p) pg = mfma(R.A[1][p], q1, pg);
                    const float sc = f16lo(sb[t]), bi = f16hi(sb[t]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[nt][r] = fmaf(sc, pg[r], fmaf(bi, xs[r], acc[nt][r]));
                }
            }
        };
        // ring of kGuDepth groups in flight (also for 2-bit groups: deeper measured slower)
        constexpr int GD = kGuDepth;
        Regs R[GD];
#pragma unroll
        for (int q = 0; q < GD; ++q) {
            load(R[q], j0 + q);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int jb = j0; jb < j1; jb += GD) {
#pragma unroll
            for (int q = 0; q < GD; ++q) {
                if (jb + q < j1) compute(R[q], jb + q);
                load(R[q], jb + q + GD);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // upper half of H: to LDS; lower half adds it (fixed order: lower + upper)
    if (kh == 1) {
#pragma unroll
        for (int nt = 0; nt < kNtGu; ++nt) red[((wave & 1) * kNtGu + nt) * 64 + lane] = acc[nt];
    }
    __syncthreads();
    if (kh == 1 || !active) return;
#pragma unroll
    for (int nt = 0; nt < kNtGu; ++nt) acc[nt] += red[((wave & 1) * kNtGu + nt) * 64 + lane];

    // h = silu(gate) * up: rows 4kq + r, columns i = 64gi + 32*t2 + 16*hh + n
    float h[4][4], mx[4], hs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float xi = s_xinv[4 * kq + r];
        mx[r] = 0.0f;
        hs[r] = 0.0f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {  // c4 = 2*t2 + hh
            const int ntg = 4 * (c4 >> 1) + (c4 & 1);
            const float gv = acc[ntg][r] * xi, uv = acc[ntg + 2][r] * xi;
            const float v = s_tok[4 * kq + r] < 0 ? 0.0f : gv / (1.0f + expf(-gv)) * uv;
            h[r][c4] = v;
            mx[r] = fmaxf(mx[r], fabsf(v));
            hs[r] += v;
        }
        mx[r] = row16_max(mx[r]);
        hs[r] = row16_sum(hs[r]);
    }
    const int NGi = a.Imax / 64;
    // column 16*c4 + n of the group at pslot + pstride*c4, times the slot's factor
    const float odd = BITS == 4 ? ((n & 1) ? 0.0625f : 1.0f) : ldexpf(1.0f, crumb_scale_log2(n & 7));
    const int pslot = BITS == 4 ? (n & ~7) + slot_of(n & 7) : 32 * ((n & 7) >> 2) + 2 * (n & 3) + (n >> 3);
    constexpr int pstride = BITS == 4 ? 16 : 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= tl.z) continue;
        const int e = act_exponent(mx[r]);
        const float sc = ldexpf(1.0f, e) * odd;
        const size_t hrow = shared ? (size_t)a.P + tl.y + m : (size_t)(tl.y + m);
        uint16_t* hp = a.h16 + hrow * a.Imax + 64 * gi + pslot;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) hp[pstride * c4] = f16bits(h[r][c4] * sc);
        if (n == 0) {
            a.hsum[hrow * NGi + gi] = hs[r];
            a.hinv[hrow * NGi + gi] = ldexpf(1.0f, -e);
        }
    }
}

// ---------------------------------------------------------------------------
// k_down_grouped: grid (tile capacity, ceil(H/512)), 256 threads.  Wave w:
// outputs o0 = 512*blockIdx.y + 128w + [0, 128) (two 64-row halves of N-tiles
// of 16) over all of I; a wave visit reads 2 KB of contiguous record bytes.
// Dynamic LDS: [Ie/64][16] group sums of h, then [Ie/64][16] 2^-e of h.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_down_grouped(PrefillArgs a) {
    extern __shared__ float dsm[];
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
    const int o0 = 512 * blockIdx.y + 128 * wave;
    if (o0 >= H) return;
    const bool hi_ok = o0 + 128 <= H;  // the second 64-row half exists (H is a multiple of 64)
    const uint8_t* rec = shared ? a.shared : a.experts + (size_t)tl.x * a.rec_bytes;
    const __amdgpu_buffer_rsrc_t rw = rsrc(rec, shared ? a.rec_bytes_shared : a.rec_bytes);
    const __amdgpu_buffer_rsrc_t rh = rsrc(a.h16, (size_t)(a.P + a.T) * a.Imax * 2);
    // lane row o0 + 64*hh + 16*kq + n, row 16*kq + n of output tile
    // o0/64 + hh: one 16-byte load covers 64 rows of a 1 KB chunk of a down
    // segment (32 nibbles per row, or the group's 64 2-bit codes), one dword
    // load their scale/bias pairs
    constexpr int NC = BITS == 4 ? 2 : 1;
    constexpr int SEG = NC * 1024 + 256;
    const int ts = SEG * NGe;  // bytes of an output tile's segments
    const int dof = (int)(shared ? a.d_off_shared : a.d_off) + ts * (o0 / 64);
    const int wo = dof + (16 * kq + n) * 16;
    const int so = dof + NC * 1024 + (16 * kq + n) * 4;
    const int ho = (max(s_row[n], 0) * a.Imax + 8 * kq) * 2;
    const Unpack up;
    f32x4 acc[kNtDn];
#pragma unroll
    for (int nt = 0; nt < kNtDn; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
    struct Regs {
        u32x4 A[2];
        u32x4 W[2][2];  // [output tile][chunk] (2-bit: the group's 16 bytes in W[tile][0])
        uint32_t SB[2];
    };
    auto load = [&](Regs& R, int jg) {  // jg >= NGe: a refill past the end
        const int ja = min(jg, NGe - 1);
#pragma unroll
        for (int c = 0; c < 2; ++c) R.A[c] = bload4(rh, ho, 128 * ja + 64 * c);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bool live = jg < NGe && (hh == 0 || hi_ok);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                R.W[hh][c] = bload4<kAuxNT>(rw, wo, live ? ts * hh + SEG * jg + 1024 * c : kPastEnd);
            R.SB[hh] = bload(rw, so, live ? ts * hh + SEG * jg : kPastEnd);
        }
    };
    auto compute = [&](const Regs& R, int jg) {
        const f32x4 hi = *(const f32x4*)&sHi[jg * kTileRows + 4 * kq];
        const f32x4 hsum = *(const f32x4*)&sH[jg * kTileRows + 4 * kq];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const u32x4 w0 = xpose4(R.W[hh][0]);
            const u32x4 w1 = BITS == 4 ? xpose4(R.W[hh][1]) : w0;
            const u32x4 sb = bcast4(R.SB[hh]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int nt = 4 * hh + t;
                f32x4 pd = {0, 0, 0, 0};
                pd = mfma(R.A[0], BITS == 4 ? up.codes(w0[t]) : up.crumbs<0>(w0[t]), pd);
                pd = mfma(R.A[1], BITS == 4 ? up.codes(w1[t]) : up.crumbs<1>(w0[t]), pd);
                const float sd = f16lo(sb[t]), bd = f16hi(sb[t]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[nt][r] = fmaf(bd, hsum[r], fmaf(sd, pd[r] * hi[r], acc[nt][r]));
            }
        }
    };
    constexpr int DD = kDnDepth;
    Regs R[DD];
#pragma unroll
    for (int q = 0; q < DD; ++q) {
        load(R[q], q);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int jb = 0; jb < NGe; jb += DD) {
#pragma unroll
        for (int q = 0; q < DD; ++q) {
            if (jb + q < NGe) compute(R[q], jb + q);
            load(R[q], jb + q + DD);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= tl.z) continue;
        int t, j;
        bool bad = false;
        if (shared) {
            t = tl.y + m;
            j = a.k;
        } else {
            t = a.pair_tok[tl.y + m];
            j = a.pair_slot[tl.y + m];
            const int e = a.ids[(size_t)t * a.k + j];
            bad = e < 0 || e >= a.E;
        }
        float* dst = a.eo + ((size_t)t * (a.k + 1) + j) * H + o0 + n;
#pragma unroll
        for (int nt = 0; nt < kNtDn; ++nt)
            if (nt < 4 || hi_ok) dst[16 * nt] = bad ? __builtin_nanf("") : acc[nt][r];
    }
}

__global__ void k_zero_shared_rows(PrefillArgs a) {  // no shared expert: eo[:, k, :] = 0
    const int t = blockIdx.y, o = blockIdx.x * kBlock + threadIdx.x;
    if (o < a.H) a.eo[((size_t)t * (a.k + 1) + a.k) * a.H + o] = 0.0f;
}

template <int BITS>
static void launch_prep_bits(const PrefillArgs& a, int act_bf16, hipStream_t s) {
    const dim3 grid(a.T);
    if (a.xparts == 1 && act_bf16)
        launch_kernel(k_prep_tokens<1, true, BITS>, grid, dim3(kBlock), 0, s, a);
    else if (a.xparts == 1)
        launch_kernel(k_prep_tokens<1, false, BITS>, grid, dim3(kBlock), 0, s, a);
    else if (act_bf16)
        launch_kernel(k_prep_tokens<2, true, BITS>, grid, dim3(kBlock), 0, s, a);
    else
        launch_kernel(k_prep_tokens<2, false, BITS>, grid, dim3(kBlock), 0, s, a);
}

hipError_t launch_prefill_prep(const PrefillArgs& a, int act_bf16, hipStream_t s) {
    if (a.bits == 2)
        launch_prep_bits<2>(a, act_bf16, s);
    else
        launch_prep_bits<4>(a, act_bf16, s);
    return hipGetLastError();
}

hipError_t launch_route_tiles(const PrefillArgs& a, hipStream_t s) {
    const dim3 grid((a.E + kTileRows - 1) / kTileRows, (a.T + kTileRows - 1) / kTileRows);
    constexpr int NW = 4, D = 4;  // waves per tile, 64-input units in flight per wave
    if (a.xparts == 1)
        launch_kernel(k_route_tiles<1, NW, D>, grid, dim3(64 * NW), 0, s, a);
    else
        launch_kernel(k_route_tiles<2, NW, D>, grid, dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_group(const PrefillArgs& a, hipStream_t s) {
    launch_kernel(k_group, dim3(1), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_gate_up(const PrefillArgs& a, hipStream_t s) {
    const dim3 grid(a.tile_cap, (a.Imax + 127) / 128);
    const size_t lds = (size_t)(a.H / 64) * kTileRows * 4 + (size_t)2 * kNtGu * 64 * 16;
    if (a.xparts == 1 && a.bits == 2)
        launch_kernel(k_gu_grouped<1, 2>, grid, dim3(kBlock), lds, s, a);
    else if (a.xparts == 1)
        launch_kernel(k_gu_grouped<1, 4>, grid, dim3(kBlock), lds, s, a);
    else if (a.bits == 2)
        launch_kernel(k_gu_grouped<2, 2>, grid, dim3(kBlock), lds, s, a);
    else
        launch_kernel(k_gu_grouped<2, 4>, grid, dim3(kBlock), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_down(const PrefillArgs& a, hipStream_t s) {
    const size_t lds = (size_t)(a.Imax / 64) * kTileRows * 8;
    const dim3 grid(a.tile_cap, (a.H + 511) / 512);
    if (a.bits == 2)
        launch_kernel(k_down_grouped<2>, grid, dim3(kBlock), lds, s, a);
    else
        launch_kernel(k_down_grouped<4>, grid, dim3(kBlock), lds, s, a);
    if (!a.Is) launch_kernel(k_zero_shared_rows, dim3((a.H + kBlock - 1) / kBlock, a.T), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

// moe_prefill.hip -- multi-token (prefill) path: experts grouped by selection
// and run as MFMA grouped dequant GEMMs, so that each selected expert's
// weights are streamed once per call and applied to every token routed to it.
//
//   k_prep_tokens   per token: fp16 parts of x * 2^e, with one e per token
//                   chosen so that its largest value is below 2^14; the exact
//                   sum of each 64-input group of x * 2^e.
//   k_group         one workgroup: (token, slot) pairs sorted by expert
//                   (stable), and a tile list of at most 16 rows per tile;
//                   the shared expert adds tiles of 16 consecutive tokens.
//   k_gu_grouped    per (tile, 128 rows of I): wave = one 64-row group of I
//                   (gate and up: 8 MFMA N-tiles of 16) over one half of H;
//                   the two halves are added in a fixed order, then
//                   h = silu(gate) * up is stored as fp16 with a per-(row,
//                   64-group) power-of-two scale, plus the group's sum of h.
//   k_down_grouped  per (tile, 256 outputs): wave = 64 outputs over all of I;
//                   writes each row's expert output (unweighted).
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
constexpr int kNtDn = 4;  // MFMA N-tiles per wave in k_down_grouped (64 outputs)
constexpr int kAuxNT = 2; // buffer-load cache policy: nontemporal
constexpr int kGuDepth = 2;  // 64-input groups in flight per wave, k_gu_grouped
constexpr int kDnDepth = 4;  // 64-input groups in flight per wave, k_down_grouped

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
template <int XP, bool BF16>
__global__ __launch_bounds__(kBlock) void k_prep_tokens(PrefillArgs a) {
    __shared__ float red4[kWaves];
    const int t = blockIdx.x, H = a.H, NG = H / 64;
    const int wave = wave_id(), lane = threadIdx.x & 63;
    auto load = [&](int i) {
        const size_t gi = (size_t)t * H + i;
        return BF16 ? bf16_to_f32(((const uint16_t*)a.x)[gi]) : ((const float*)a.x)[gi];
    };
    float mx = 0.0f;
    for (int i = threadIdx.x; i < H; i += kBlock) mx = fmaxf(mx, fabsf(load(i)));
    mx = wave_max(mx);
    if (lane == 0) red4[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
    const int e = act_exponent(mx);
    const float sc = ldexpf(1.0f, e);
    const int p = lane & 7;
    for (int g = wave; g < NG; g += kWaves) {
        const float vs = load(64 * g + lane) * sc;  // exact: a power-of-two scaling
        const float vq = vs * ((p & 1) ? 0.0625f : 1.0f);
        const uint16_t hi = f16bits(vq);
        const size_t dst = (size_t)t * H + 64 * g + (lane & ~7) + slot_of(p);
        a.x16[dst] = hi;
        if (XP == 2) a.x16[(size_t)a.T * H + dst] = f16bits(vq - (float)__builtin_bit_cast(_Float16, hi));
        const double gs = wave_sum_d((double)vs);
        if (lane == 0) a.xsum[(size_t)t * NG + g] = (float)gs;
    }
    if (threadIdx.x == 0) a.xinv[t] = ldexpf(1.0f, -e);
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
// k_gu_grouped: grid (tile capacity, ceil(max(I, Is)/128)), 256 threads.
// Wave w: 64-row group gi = 2*blockIdx.y + (w & 1) of I (GU tiles 2gi and
// 2gi+1: N-tiles 0-1 gate and 2-3 up of the first, 4-7 of the second) over
// the half (w >> 1) of the 64-input groups of H.
// Dynamic LDS: [H/64][16] group sums of the rows' activations, then the
// partial sums of the upper-half waves, [2][8][64] float4.
// ---------------------------------------------------------------------------
template <int XP>
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
        const __amdgpu_buffer_rsrc_t rx = rsrc(a.x16, (size_t)XP * a.T * H * 2);
        // per-lane offsets (bytes): row 16*kq + n of each GU tile (codes and
        // scale/bias pair; one 16-byte load covers a 1 KB chunk of a tile per
        // wave), and the lane's activations; the rest of each address is
        // uniform and goes in the scalar offset
        const int rl = 16 * kq + n;
        const int wo[2] = {48 * H * (2 * gi) + rl * 16, 48 * H * (2 * gi + 1) + rl * 16};
        const int so[2] = {3 * H * Ie / 2 + 12 * H * gi + rl * 4, 3 * H * Ie / 2 + 12 * H * gi + 4 * H + rl * 4};
        const int xo = (max(s_tok[n], 0) * H + 8 * kq) * 2;
        const int xpart = a.T * H * 2;
        const Unpack up;
        struct Regs {
            u32x4 A[2][XP];
            u32x4 W[2][2];  // [GU tile][chunk], rows 16*kq + n
            uint32_t SB[2];
        };
        auto load = [&](Regs& R, int jg) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int p = 0; p < XP; ++p) R.A[c][p] = bload4(rx, xo, p * xpart + 128 * jg + 64 * c);
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                for (int c = 0; c < 2; ++c) R.W[t2][c] = bload4<kAuxNT>(rw, wo[t2], 2048 * jg + 1024 * c);
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) R.SB[t2] = bload(rw, so[t2], 256 * jg);
        };
        auto compute = [&](const Regs& R, int jg) {
            const f32x4 xs = *(const f32x4*)&sX[jg * kTileRows + 4 * kq];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const u32x4 w0 = xpose4(R.W[t2][0]), w1 = xpose4(R.W[t2][1]);
                const u32x4 sb = bcast4(R.SB[t2]);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int nt = 4 * t2 + t;
                    f32x4 pg = {0, 0, 0, 0};
                    const half8 q0 = up.codes(w0[t]), q1 = up.codes(w1[t]);
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
        // ring of kGuDepth groups in flight; refills are clamped to the last
        // group (re-reads of it are cache hits)
        Regs R[kGuDepth];
#pragma unroll
        for (int q = 0; q < kGuDepth; ++q) {
            load(R[q], min(j0 + q, j1 - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int jb = j0; jb < j1; jb += kGuDepth) {
#pragma unroll
            for (int q = 0; q < kGuDepth; ++q) {
                if (jb + q < j1) compute(R[q], jb + q);
                load(R[q], min(jb + q + kGuDepth, j1 - 1));
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
    const float odd = (n & 1) ? 0.0625f : 1.0f;
    const int pslot = (n & ~7) + slot_of(n & 7);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * kq + r;
        if (m >= tl.z) continue;
        const int e = act_exponent(mx[r]);
        const float sc = ldexpf(1.0f, e) * odd;
        const size_t hrow = shared ? (size_t)a.P + tl.y + m : (size_t)(tl.y + m);
        uint16_t* hp = a.h16 + hrow * a.Imax + 64 * gi + pslot;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) hp[16 * c4] = f16bits(h[r][c4] * sc);
        if (n == 0) {
            a.hsum[hrow * NGi + gi] = hs[r];
            a.hinv[hrow * NGi + gi] = ldexpf(1.0f, -e);
        }
    }
}

// ---------------------------------------------------------------------------
// k_down_grouped: grid (tile capacity, ceil(H/256)), 256 threads.  Wave w:
// outputs o0 = 256*blockIdx.y + 64w + [0, 64) (N-tiles of 16) over all of I.
// Dynamic LDS: [Ie/64][16] group sums of h, then [Ie/64][16] 2^-e of h.
// ---------------------------------------------------------------------------
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
    const int o0 = 256 * blockIdx.y + 64 * wave;
    if (o0 >= H) return;
    const uint8_t* rec = shared ? a.shared : a.experts + (size_t)tl.x * a.rec_bytes;
    const __amdgpu_buffer_rsrc_t rw = rsrc(rec, shared ? a.rec_bytes_shared : a.rec_bytes);
    const __amdgpu_buffer_rsrc_t rh = rsrc(a.h16, (size_t)(a.P + a.T) * a.Imax * 2);
    // lane row o0 + 16*kq + n: one 16-byte load covers the wave's 64 rows of a
    // down chunk, one dword load their scale/bias pairs
    const int rl = o0 + 16 * kq + n;
    const int wo = 32 * H + rl * 16;
    const int so = 3 * H * Ie / 2 + 8 * H + rl * 4;
    const int ho = (max(s_row[n], 0) * a.Imax + 8 * kq) * 2;
    const Unpack up;
    f32x4 acc[kNtDn];
#pragma unroll
    for (int nt = 0; nt < kNtDn; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
    struct Regs {
        u32x4 A[2];
        u32x4 W[2];
        uint32_t SB;
    };
    auto load = [&](Regs& R, int jg) {
#pragma unroll
        for (int c = 0; c < 2; ++c) R.A[c] = bload4(rh, ho, 128 * jg + 64 * c);
#pragma unroll
        for (int c = 0; c < 2; ++c) R.W[c] = bload4<kAuxNT>(rw, wo, 48 * H * (2 * jg + c));
        R.SB = bload(rw, so, 12 * H * jg);
    };
    auto compute = [&](const Regs& R, int jg) {
        const f32x4 hi = *(const f32x4*)&sHi[jg * kTileRows + 4 * kq];
        const f32x4 hsum = *(const f32x4*)&sH[jg * kTileRows + 4 * kq];
        const u32x4 w0 = xpose4(R.W[0]), w1 = xpose4(R.W[1]);
        const u32x4 sb = bcast4(R.SB);
#pragma unroll
        for (int nt = 0; nt < kNtDn; ++nt) {
            f32x4 pd = {0, 0, 0, 0};
            pd = mfma(R.A[0], up.codes(w0[nt]), pd);
            pd = mfma(R.A[1], up.codes(w1[nt]), pd);
            const float sd = f16lo(sb[nt]), bd = f16hi(sb[nt]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[nt][r] = fmaf(bd, hsum[r], fmaf(sd, pd[r] * hi[r], acc[nt][r]));
        }
    };
    Regs R[kDnDepth];
#pragma unroll
    for (int q = 0; q < kDnDepth; ++q) {
        load(R[q], min(q, NGe - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int jb = 0; jb < NGe; jb += kDnDepth) {
#pragma unroll
        for (int q = 0; q < kDnDepth; ++q) {
            if (jb + q < NGe) compute(R[q], jb + q);
            load(R[q], min(jb + q + kDnDepth, NGe - 1));
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
        for (int nt = 0; nt < kNtDn; ++nt) dst[16 * nt] = bad ? __builtin_nanf("") : acc[nt][r];
    }
}

__global__ void k_zero_shared_rows(PrefillArgs a) {  // no shared expert: eo[:, k, :] = 0
    const int t = blockIdx.y, o = blockIdx.x * kBlock + threadIdx.x;
    if (o < a.H) a.eo[((size_t)t * (a.k + 1) + a.k) * a.H + o] = 0.0f;
}

hipError_t launch_prefill_prep(const PrefillArgs& a, int act_bf16, hipStream_t s) {
    const dim3 grid(a.T);
    if (a.xparts == 1 && act_bf16)
        launch_kernel(k_prep_tokens<1, true>, grid, dim3(kBlock), 0, s, a);
    else if (a.xparts == 1)
        launch_kernel(k_prep_tokens<1, false>, grid, dim3(kBlock), 0, s, a);
    else if (act_bf16)
        launch_kernel(k_prep_tokens<2, true>, grid, dim3(kBlock), 0, s, a);
    else
        launch_kernel(k_prep_tokens<2, false>, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_group(const PrefillArgs& a, hipStream_t s) {
    launch_kernel(k_group, dim3(1), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_gate_up(const PrefillArgs& a, hipStream_t s) {
    const dim3 grid(a.tile_cap, (a.Imax + 127) / 128);
    const size_t lds = (size_t)(a.H / 64) * kTileRows * 4 + (size_t)2 * kNtGu * 64 * 16;
    if (a.xparts == 1)
        launch_kernel(k_gu_grouped<1>, grid, dim3(kBlock), lds, s, a);
    else
        launch_kernel(k_gu_grouped<2>, grid, dim3(kBlock), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_down(const PrefillArgs& a, hipStream_t s) {
    const size_t lds = (size_t)(a.Imax / 64) * kTileRows * 8;
    launch_kernel(k_down_grouped, dim3(a.tile_cap, (a.H + 255) / 256), dim3(kBlock), lds, s, a);
    if (!a.Is) launch_kernel(k_zero_shared_rows, dim3((a.H + kBlock - 1) / kBlock, a.T), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

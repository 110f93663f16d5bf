// moe_internal.h -- launch arguments shared by the host side of the library
// (moe_layer.hip) and its kernels (moe_kernels.hip).  Not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kBlock = 256;        // threads per workgroup (4 waves of 64)
constexpr int kWaves = kBlock / 64;
// Waves of a k_gate_up workgroup (they split H): 8 up to hidden 4096 (at
// most 8 groups of 64 inputs per wave), else 4 (measured: 8 waves save 1.5-4 %
// per layer at hidden 2816, 4 waves are 1 % faster at hidden 6144).
constexpr int kGuWavesSmallH = 8, kGuWavesLargeH = 4, kGuSmallHMax = 4096;
// Polls of the router's logit words that a fused gate/up workgroup makes
// before it computes the logits itself (each poll waits for its load, well
// under a microsecond): a bound on the wait, never reached when the router
// units run beside the gate/up units.
constexpr int kRouteSpinLimit = 1 << 14;
// Largest hidden size routed inside the gate/up launch: there every gate/up
// workgroup prepares its own activations, a few groups per wave (measured:
// 2 % less per decode step at hidden 2816; at hidden 6144 the separate router
// launch is 16 % faster).
constexpr int kFusedMaxHidden = kGuSmallHMax;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kMaxHidden = 8192;
constexpr int kHParts = 1;         // fp16 parts used for the intermediate h
constexpr int kMaxDownGroups = 64; // input groups (of I) per down work item
constexpr int kMaxGateUpGroupsPerWave = 32;
// Shared 32-row blocks split into this many slices of H (4-wave units only):
// the shared expert's gate/up then runs on every CU while the routed units
// select, instead of as a third unit on a quarter of the CUs
constexpr int kSharedSplit = 4;
constexpr int kPieceMaxGroups = 8;  // input groups per wave in a shared piece, at most
constexpr int kCounterStride = 64;  // arrival counters 256 bytes apart (own cache lines)
// Weight groups in flight per wave in k_gate_up.  Shallow on purpose: with one
// wave per SIMD and every wave's loads queued at once, deeper rings delay each
// wave's first groups behind the others' later ones (measured: 3 beats 4, 6, 8
// and 12 at hidden 2816 and 6144, for 4-bit and 2-bit records).
constexpr int kDepth = 3;
constexpr int kDepthLargeH = 2;  // the same for 4-bit records with 4-wave workgroups (hidden
                                 // above 4096): 2.5 % per layer at hidden 6144 (2-bit groups,
                                 // half the bytes, keep 3)
constexpr int kMaxSharedItems = 8;  // down work items of the shared expert
// k_down: groups in flight per wave.  2 beats 4 and all-at-once; above hidden
// 4096 (864 down workgroups at hidden 6144) 4-bit records keep only 1 in
// flight: 3 % less down time there, while at hidden 2816 one in flight is
// 10 % slower.
constexpr int kDnRing = 2;
constexpr int kMaxItems = kMaxTopK + kMaxSharedItems;

// Prepared activations of one vector of length n (n multiple of 64):
//   pairs [n/8][parts][4] dwords  (fp16 pairs, see moe_device.h)
//   K     [n/64] float            1024 * sum of the fp16 values per group
//   X     [n/64] float            sum of the unscaled values per group
//   inv   [n/64] float            2^-e, e the group's scale exponent
struct RouteArgs {
    const void* x;           // [T][H] activations
    const int8_t* rq;        // [E][H]
    const uint16_t* rs;      // [E] fp16
    float* logits;           // [T][E]
    int32_t* ids;            // [T][k]
    float* w;                // [T][k]
    uint32_t* xpairs;        // [T][H/2*XP] (written only if prep != 0)
    float* xK;               // [T][H/64]
    float* xX;               // [T][H/64]
    float* xinv;             // [T][H/64]
    const float* bias;       // [E] selection bias (sigmoid gate) or nullptr
    float rscale;            // sigmoid gate: routed scaling factor
    int H, E, k, prep, T;
    int gate;                // 0 softmax, 1 sigmoid
    int bits;                // weight code width: 4 or 2 (activation pair order)
};

struct FfnArgs {
    const uint8_t* experts;  // E records
    const uint8_t* shared;   // shared record or nullptr
    size_t rec_bytes;
    const uint8_t* slots;    // slot cache: n_slots records (nullptr = resident pool)
    int32_t slot_of[kMaxTopK];  // with slots (one token per call): the slot of each selected expert
    int unit_offset;         // k_gate_up: first unit of this launch (split launches)
    const int32_t* ids;      // [T][k] selection (read by k_down; by k_gate_up unless logits)
    const float* w;          // [T][k] gate weights (fused combine only)
    const float* logits;     // [T][E]: if set, k_gate_up selects the experts itself
    // fused routing (route_units > 0, hidden <= kFusedMaxHidden): the first
    // route_units workgroups of each token row compute the router logits, one
    // row per wave, into flog; the gate/up units prepare x themselves and
    // select from flog
    int route_units;
    const void* x;           // [T][H] activations
    const int8_t* rq;        // [E][H] router rows
    const uint16_t* rs;      // [E] fp16 row scales
    uint32_t* flog;          // [T][E] logits stored bit-inverted, 0 = not yet written;
                             // k_down returns the words to 0 when set
    int spin_limit;          // polls before computing the logits locally (< 0: none)
    int logit_delay;         // ticks of the 100 MHz device clock after its start before a
                             // gate/up unit first reads the logit words (logit_delay_ticks)
    const float* bias;       // [E] selection bias (sigmoid gate) or nullptr
    float rscale;            // sigmoid gate: routed scaling factor
    int gate;                // 0 softmax, 1 sigmoid
    int32_t* ids_out;        // [T][k] written by k_gate_up's first workgroup when logits is set
    float* w_out;            // [T][k]
    const uint32_t* xpairs;  // prepared x, as in RouteArgs
    const float* xK;
    const float* xX;
    const float* xinv;
    uint32_t* hpairs;        // [T][k+1][blk_max][16*kHParts]
    float* hK;               // [T][k+1][blk_max]
    float* hHs;              // [T][k+1][blk_max]
    float* hinv;             // [T][k+1][blk_max]
    float* dpart;            // [T][n_otiles][n_items][64]
    int n_units;             // k*blk_r + sh_split*blk_s
    uint32_t* dctr;          // [T][n_otiles][kCounterStride] (k_gate_up: [T][blk_s] piece counts)
    float* shp;              // [T][blk_s][sh_split][64] gate/up sums of the shared pieces
    int sh_split;            // pieces per shared 32-row block (each a slice of H), or 1
    int gpw_sh;              // input groups per wave in a shared piece
    float* y;                // [T][H] fused output (or nullptr)
    float* eo;               // [T][k+1][H] per-expert outputs (or nullptr)
    uint32_t* err;           // device error word
    int H, I, Is, E, k;
    int blk_r;               // I/32  (gate/up units per routed expert)
    int blk_s;               // Is/32 (32-row blocks of the shared expert; sh_split units each)
    int blk_max;             // max(blk_r, blk_s)
    int gpw_gu;              // input groups per wave in the gate/up kernel
    int gu_waves;            // waves per gate/up workgroup
    int n_otiles;            // H/64
    int n_items;             // down work items per output tile: k + shared k-slices
    int gi;                  // input groups (of I) per routed down item (= I/64)
    int gis;                 // input groups per shared down item
    int gpw_dn;              // input groups per wave in the down kernel
    int bits;                // weight code width: 4 or 2
    size_t d_off;            // start of a routed record's down segments
    size_t d_off_shared;     // the same for the shared record
};

constexpr int kTileRows = 16;         // rows (tokens) per MFMA tile in the prefill path
constexpr int kPrefillMinTokens = 4;  // calls with at least this many tokens group by expert

struct PrefillArgs {
    const void* x;           // [T][H] activations
    const int32_t* ids;      // [T][k]
    const uint8_t* experts;
    const uint8_t* shared;
    size_t rec_bytes;
    size_t rec_bytes_shared;
    uint16_t* x16;           // [XP][T][H] fp16 parts of x * 2^e (one e per token), slot order
    uint16_t* x16b;          // 2-bit records: the same in the 2-bit slot order (gate/up operand)
    float* xsum;             // [T][H/64] sum of each group of x * 2^e
    float* xinv;             // [T] 2^-e
    int32_t* pair_tok;       // [P] token of each expert-sorted (token, slot) pair
    int32_t* pair_slot;      // [P] slot j of each sorted pair
    int4* tiles;             // [tile_cap] {expert or -1 (shared), first row, rows, 0}
    int32_t* n_tiles;        // [1]
    uint16_t* h16;           // [P + T][Imax] fp16 h * 2^e (per 64-group e), slot order
    float* hsum;             // [P + T][Imax/64]
    float* hinv;             // [P + T][Imax/64]
    float* eo;               // [T][k+1][H] per-slot expert outputs
    uint32_t* err;           // device error word
    const int8_t* rq;        // router [E][H] (k_route_tiles)
    const uint16_t* rs;      // router row scales [E] fp16
    float* logits;           // [T][E] out (k_route_tiles)
    size_t d_off, d_off_shared;  // down segments of a routed / the shared record
    int H, E, I, Is, k, T, P, Imax, tile_cap, xparts, bits;
};

// k_fetch workgroups per record: 4 to 16 measured alike on the out-of-core
// stack, 64 and more 7 % slower (too many host reads in flight at once)
constexpr int kFetchBlocksPerRecord = 8;
// Missed experts' records copied by a kernel from the pinned host pool (read
// over PCIe through its device mapping) into their HBM slots.
struct FetchArgs {
    const uint8_t* src;          // host pool, device-mapped address
    uint8_t* dst;                // slots
    size_t rec_bytes;            // a multiple of 16
    int n;                       // records to copy (<= kMaxTopK)
    int32_t src_rec[kMaxTopK];   // expert index in the pool
    int32_t dst_slot[kMaxTopK];  // slot index
};

struct CombineArgs {
    const float* eo;  // [T][k+1][H]
    const float* w;   // [T][k]
    void* y;          // [T][H]
    int H, k, T, y_bf16;
};

// Per-launch timing: when the host layer sets g_stamp around one launcher
// call, the first kernel that launcher starts is dispatched with
// hipExtLaunchKernelGGL so that the event pair holds that dispatch's own start
// and end (no marker packets in between).  Null when profiling is off.
struct LaunchStamp {
    hipEvent_t start, stop;
    bool used;
};
extern LaunchStamp* g_stamp;

template <typename... P, typename... A>
inline void launch_kernel(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A... args) {
    if (g_stamp && !g_stamp->used) {
        g_stamp->used = true;
        hipExtLaunchKernelGGL(k, grid, block, (uint32_t)lds, s, g_stamp->start, g_stamp->stop, 0,
                              static_cast<P>(args)...);
    } else {
        hipLaunchKernelGGL(k, grid, block, lds, s, static_cast<P>(args)...);
    }
}

}  // namespace moe

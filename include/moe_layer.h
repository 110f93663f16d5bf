/*
 * moe_layer.h -- C ABI of the MI355X routed-expert MoE layer library
 * (libmoe_layer.so, built for gfx950).
 *
 * One layer of a mixture-of-experts FFN at decode, as the out-of-core engines
 * on the source pages run it: an 8-bit router, exact top-k expert selection
 * with gate weights renormalised over the selection, a SwiGLU FFN per selected
 * expert over affine 4-bit group-64 weights (one fp16 scale and one fp16 bias
 * per 64 inputs) dequantised on use, and an always-resident shared expert
 * added to the weighted sum of the routed outputs.
 *   - exact top-8 routed experts: Inferno README, "Current Scope"
 *   - 8-bit router, MLX affine 4-bit group-64 experts, shared expert computed
 *     while routed experts are fetched, outputs combined afterwards:
 *     TurboFieldfare article, "Arsitektur eksekusi yang mengurangi memori" and
 *     "Proses pembuatan token"
 *   - gate, up and down matrices of an expert stored next to each other:
 *     Inferno README, "Model" (ExpertPack)
 *   - dequantisation on use, batch-union of experts in prefill: Colibri README,
 *     "What's implemented"
 *   - never run an expert whose weights are missing, never substitute zeros:
 *     Colibri analysis report, section 6
 *
 * Conventions
 *   - Every pointer argument named as "device" must point to GPU memory
 *     (hipMalloc / torch CUDA tensors) on the current device.  Host pointers
 *     are named "host".  Nothing here takes ownership of caller memory.
 *   - Compute calls enqueue work on `stream` (a hipStream_t; NULL = the
 *     default stream) and return without waiting.  Argument errors are
 *     detected on the host before anything is enqueued; faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - A handle is not thread-safe; calls on one handle must be issued from one
 *     thread and, while they share a workspace, on one stream.
 *   - Status codes are int32: MOE_OK (0) or a negative MOE_ERR_*.
 *     moe_last_error() gives a thread-local detail string for the last failure.
 *
 * Packed expert record (hidden H, intermediate I; H and I multiples of 64).
 * Matrices G (gate) and U (up) are [I][H] with input dim H; D (down) is [H][I]
 * with input dim I.  Inputs are quantised in groups of 64 consecutive inputs:
 * W = scale * q + bias, q in 0..15, one fp16 (scale, bias) pair per row and
 * group.  The record is a sequence of 3*H*I/4096 segments of 2304 bytes; a
 * segment covers one tile of 64 rows x 64 inputs:
 *     +0     codes: [half c < 2][row r < 64][16 bytes], the 16 bytes holding
 *            inputs [32c, 32c+32) of the tile's row r, input 2m of those 32
 *            in the low nibble of byte m and 2m+1 in its high nibble
 *     +2048  (scale, bias) fp16 pairs of the 64 rows, in row order
 *   gate/up segments first: segment b*(H/64) + g (b < I/32, g < H/64) holds
 *     inputs [64g, 64g+64) of tile rows r < 32 = G row 32b+r and r >= 32 =
 *     U row 32b+r-32
 *   down segments next: segment (I/32)*(H/64) + t*(I/64) + g (t < H/64,
 *     g < I/64) holds inputs [64g, 64g+64) of D rows 64t+r
 *   Record size: 27*H*I/16 bytes (0.5625 bytes per weight).  A layer's routed
 *   records lie back to back: record e at experts + e * moe_expert_record_bytes.
 *   Keeping each group's pairs beside its codes makes every 64-input step of
 *   a weight stream one contiguous 2.25 KB read (the gate, up and down
 *   matrices of an expert stored next to each other: Inferno README, "Model",
 *   ExpertPack).
 * 2-bit records (desc.bits = 2): W = scale * q + bias, q in 0..3; segments of
 * 1280 bytes: codes [row r < 64][16 bytes] holding the tile's 64 inputs of row
 * r, input 4m+j in bits [2j, 2j+2) of byte m, then the 64 pairs at +1024.
 * (Colibri README, "What's implemented", names packed int2 among its CPU
 * quantisation kernels; the layout here is our own.)  Record size:
 * 15*H*I/16 bytes (0.3125 bytes per weight); moe_expert_record_bytes_bits
 * gives either size.
 * Router: rows q[E][H] int8, row-major, and one fp16 scale per row;
 *   logit_e = scale_e * sum_h q[e][h] * x_h.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_ARG = -1,        /* null or inconsistent argument                    */
    MOE_ERR_SHAPE = -2,      /* H or I not a multiple of 64, top_k > n_experts... */
    MOE_ERR_ALIGN = -3,      /* pointer not 16-byte aligned                      */
    MOE_ERR_HIP = -4,        /* a HIP runtime call failed (detail in last_error) */
    MOE_ERR_NOMEM = -5,      /* host or device allocation failed                 */
    MOE_ERR_NOT_PINNED = -6, /* host pool is not page-locked host memory         */
    MOE_ERR_STATE = -7,      /* call not valid for this handle's configuration   */
    MOE_ERR_DEVICE = -8      /* a kernel reported bad input (e.g. expert id out of range) */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };                 /* activation / output dtypes */
enum { MOE_SOFTMAX_TOPK = 0, MOE_SIGMOID_TOPK = 1 }; /* gate functions            */
enum { MOE_CACHE_LFU = 0, MOE_CACHE_LRU = 1 };       /* slot cache replacement    */

typedef struct moe_layer_desc {
    int32_t hidden;        /* H, multiple of 64, <= 8192                          */
    int32_t n_experts;     /* E routed experts, 1..1024                           */
    int32_t inter;         /* I, routed expert intermediate size, multiple of 64, <= 4096 */
    int32_t top_k;         /* k, 1..min(E, 16)                                    */
    int32_t shared_inter;  /* intermediate size of the shared expert, 0 = none    */
    int32_t group;         /* quantisation group; must be 64                      */
    int32_t act_dtype;     /* MOE_F32 or MOE_BF16 activations x                   */
    int32_t gate_fn;       /* MOE_SOFTMAX_TOPK: w = softmax of the selected logits
                              (selection by logit).  MOE_SIGMOID_TOPK: scores
                              s_e = 1 / (1 + exp(-logit_e)); selection by s_e + b_e
                              (b = weights.selection_bias, zero if NULL); w_j =
                              routed_scale * s_j / sum over the selection of s.  The
                              DeepSeek-V3-style router that the Colibri README ("What's
                              implemented") names for GLM (noaux_tc,
                              routed_scaling_factor); one expert group.            */
    int32_t n_slots;       /* 0 = every routed record resident in HBM; otherwise the
                              number of HBM expert slots of the slot cache (>= top_k) */
    float routed_scale;    /* MOE_SIGMOID_TOPK: the routed scaling factor (> 0; 0 reads
                              as 1); must be 0 or 1 with MOE_SOFTMAX_TOPK           */
    int32_t cache_policy;  /* n_slots > 0: MOE_CACHE_LFU or MOE_CACHE_LRU (see
                              moe_cache_stats); must be MOE_CACHE_LFU otherwise     */
    int32_t bits;          /* width of the expert weight codes: 4 (0 reads as 4) or 2;
                              router rows stay int8                                */
    int32_t reserved[4];
} moe_layer_desc;

typedef struct moe_layer_weights {
    const int8_t* router_q;       /* device, [E][H] int8                              */
    const uint16_t* router_scale; /* device, [E] fp16 bits                            */
    const uint8_t* experts;       /* device, E packed records back to back            */
    const uint8_t* shared;        /* device, one packed record of (H, shared_inter), or NULL */
    const uint8_t* host_pool;     /* n_slots > 0: page-locked host memory (hipHostMalloc)
                                     holding all E records back to back; else NULL */
    uint8_t* slots;               /* n_slots > 0: device, n_slots records; else NULL.
                                     The library overwrites slots as experts enter. */
    const float* selection_bias;  /* MOE_SIGMOID_TOPK only: device, [E] fp32 correction
                                     bias added to the scores for selection (not to the
                                     gates), or NULL; must be NULL with MOE_SOFTMAX_TOPK */
} moe_layer_weights;

typedef struct moe_layer* moe_layer_t;

/* Bytes of one packed 4-bit record of (hidden, inter): 27*hidden*inter/16, or 0
 * if either is not a positive multiple of 64. */
size_t moe_expert_record_bytes(int32_t hidden, int32_t inter);

/* Bytes of one packed record of (hidden, inter) with `bits`-wide codes (4 or 2):
 * 27*hidden*inter/16 or 15*hidden*inter/16; 0 for a bad shape or width. */
size_t moe_expert_record_bytes_bits(int32_t hidden, int32_t inter, int32_t bits);

/* Validates desc and weights and builds a handle for one MoE layer: its
 * router, its routed experts' packed records and the shared expert's record
 * (the per-layer expert set the engines on the pages keep: Inferno README,
 * "Model" and "Memory Strategy"; TurboFieldfare article, "Arsitektur
 * eksekusi yang mengurangi memori").  Fails at creation on any inconsistent
 * shape or pointer rather than falling back to another path later (Colibri
 * analysis report, section 6).  The handle borrows the weight pointers (they
 * must outlive it) and owns only host metadata.  Launches nothing.
 * Errors: ARG, SHAPE, ALIGN, STATE, NOMEM. */
moe_status moe_layer_create(const moe_layer_desc* desc, const moe_layer_weights* w,
                            moe_layer_t* out);
moe_status moe_layer_destroy(moe_layer_t layer);

/* Device workspace bytes needed by the compute calls for n_tokens tokens.
 * The workspace must be zero-filled before its first use; its arrival
 * counters and the fused router's logit words sit at fixed offsets at its
 * start and every call returns them to zero, so it can be reused without
 * clearing, for any n_tokens it is large enough for (after a call that
 * returned MOE_ERR_HIP, zero-fill it again).  Two calls that overlap in time
 * must not share a workspace. */
size_t moe_workspace_bytes(moe_layer_t layer, int32_t n_tokens);

/* Router + exact top-k + gates for n_tokens tokens: the 8-bit router on the
 * token's activations (TurboFieldfare article, "Arsitektur eksekusi ...": the
 * router is 8-bit; "Proses pembuatan token": it runs first, on resident
 * weights) and the exact top-k (Inferno README, "Current Scope": exact top-8,
 * no approximate routing), gates renormalised over the selection.
 *   x   device [T][H] in desc.act_dtype
 *   ids device [T][k] int32 out: selected experts, by logit descending, ties to
 *       the lower id
 *   w   device [T][k] fp32 out: exp(l_j - l_max) / sum over the selection
 *       (MOE_SIGMOID_TOPK: routed_scale * s_j / sum of s over the selection; ids
 *       then in the order of s + bias descending, ties to the lower id)
 * Errors: ARG, ALIGN, HIP. */
moe_status moe_route_topk(moe_layer_t layer, const void* x, int32_t n_tokens, int32_t* ids,
                          float* w, void* workspace, void* stream);

/* Calls of 4 or more tokens (prefill chunks; the pages run prompts in chunks of
 * up to 128 tokens so that a fetched expert serves several rows: TurboFieldfare
 * article, "Proses pembuatan token"; Colibri analysis report, section 2,
 * "Union"; Colibri README, "What's implemented", batch-union MoE) take the
 * grouped path: the (token, slot) pairs are sorted by expert and every selected
 * expert's record is read once per call and applied to all of its tokens with
 * MFMA.  Results agree with the per-token path within the stated tolerance, not
 * bit for bit; within each path a token's result does not depend on the other
 * tokens of its call. */

/* Per-expert SwiGLU outputs for the given selection: each selected expert's
 * gate, up and down matrices dequantised on use from the affine group-64
 * record (TurboFieldfare article, "Arsitektur eksekusi ...": MLX affine 4-bit
 * group 64; Colibri README, "What's implemented": dequantisation on use),
 * h = silu(G x) * (U x), y_e = D h, and the shared expert's the same way.
 *   ids        device [T][k] int32 (values outside [0, E) set the device error
 *              flag, see moe_poll_device_error, and make that slot's output NaN)
 *   expert_out device [T][k+1][H] fp32 out: row j < k is D_e silu(G_e x)*(U_e x)
 *              for e = ids[t][j]; row k is the shared expert (zeros if none)
 * Errors: ARG, ALIGN, HIP. */
moe_status moe_expert_ffn(moe_layer_t layer, const void* x, int32_t n_tokens,
                          const int32_t* ids, void* workspace, float* expert_out, void* stream);

/* The combine: y[t] = sum_{j<k} w[t][j] * expert_out[t][j] + expert_out[t][k]
 * (routed outputs weighted by their gates, the shared expert's added with
 * weight 1: TurboFieldfare article, "Proses pembuatan token", shared and
 * routed outputs combined after the expert reads), summed in that order.  y device [T][H] of y_dtype (MOE_F32 or MOE_BF16, round to
 * nearest even).  Errors: ARG, ALIGN, HIP. */
moe_status moe_combine(moe_layer_t layer, const float* expert_out, const float* w,
                       int32_t n_tokens, void* y, int32_t y_dtype, void* stream);

/* The whole layer in one call: route, experts, combine, with the per-expert
 * outputs reduced inside the FFN kernels (no expert_out round trip).
 * ids, w as moe_route_topk; y device [T][H] fp32.  Errors: ARG, ALIGN, HIP.
 * Up to hidden 4096 a resident layer routes inside its gate/up launch: leading
 * workgroups compute the logits while the gate/up workgroups prepare the
 * activations, then read the logits as they land.  A gate/up workgroup that
 * has polled for them MOE_ROUTE_SPIN_LIMIT times (environment variable read
 * by moe_layer_create, default 16384, -1 = at once) computes them itself,
 * with the same arithmetic: results never depend on it. */
moe_status moe_layer_forward(moe_layer_t layer, const void* x, int32_t n_tokens, int32_t* ids,
                             float* w, float* y, void* workspace, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: the same kernels and results (bit for bit), with the workspace
 * taken from a static device array of the library (8 MiB, one copy per GPU,
 * held until the process ends) instead of a caller's buffer.  Calls no
 * hipMalloc, hipFree or other allocating routine.  A call whose workspace
 * (moe_workspace_bytes(layer, n_tokens)) exceeds 8 MiB returns MOE_ERR_SHAPE
 * before anything is enqueued; every per-token call (n_tokens <= 3) at any
 * shape moe_layer_create accepts fits.  The first call on a device (and the
 * first after a call that returned MOE_ERR_HIP) enqueues a small clear
 * kernel for the array's counters before the layer; every call returns them
 * to zero.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (other streams, other threads) race and must not be issued.
 * Errors: ARG, SHAPE, ALIGN, HIP. */
moe_status moe_layer_forward_noalloc(moe_layer_t layer, const void* x, int32_t n_tokens, int32_t* ids,
                                     float* w, float* y, void* stream);

/* n_layers layers one after another on one stream, layer l reading x_l and
 * writing y_l (strides in elements: x_stride for x, y_stride for y, k-strided
 * ids/w per layer), each layer ordered after the previous one's output.  The
 * layers must share top_k and act_dtype (their ids/w rows sit at l*T*top_k and
 * their x at l*x_stride elements of one dtype), and x_stride and y_stride must
 * each hold n_tokens*hidden elements of every layer (else MOE_ERR_SHAPE, checked
 * before anything is enqueued).  The workspace must be sized for the largest
 * layer.  The decode engines on the pages run their layers in this order, one
 * token at a time (TurboFieldfare article, "Proses pembuatan token").  Errors as
 * moe_layer_forward, plus SHAPE. */
moe_status moe_stack_forward(const moe_layer_t* layers, int32_t n_layers, const void* x,
                             int64_t x_stride, int32_t n_tokens, int32_t* ids, float* w,
                             float* y, int64_t y_stride, void* workspace, void* stream);

/* HBM expert-slot cache (n_slots > 0), the out-of-core decode of the pages:
 * TurboFieldfare article, "Proses pembuatan token" (the 8 ids are matched
 * against a 16-slot LFU per layer, misses are read while the shared expert is
 * computed, outputs combined after the reads); Inferno README, "Memory
 * Strategy" (hit: execute from the slot; miss: read, place in a slot, execute).
 * With a slot cache, moe_layer_forward and moe_expert_ffn take one token per
 * call (else MOE_ERR_STATE) and synchronise the host on that token's expert
 * ids.  Policy: each selection adds one to its expert's count (never
 * decayed); a miss always enters, into the lowest free slot if any, else in
 * place of a resident expert that is neither selected by the current token nor
 * pinned (moe_cache_pin): MOE_CACHE_LFU takes the one with the smallest count,
 * then the least recently used, then the lowest slot; MOE_CACHE_LRU (the
 * per-layer LRU of the Colibri README) the least recently used, then the
 * lowest slot.
 * Misses are copied into their slots by a kernel on the call's stream that
 * reads host_pool through its device mapping (or, when the pool has none, or
 * into a slot that a pending prefetch copy may still be writing, on a side
 * stream owned by the handle, behind that copy; the routed kernels wait for
 * the side stream).  The shared expert's
 * gate/up is queued before the host waits for the ids, so it runs during that
 * wait rather than beside the copies.  The handle owns the side
 * stream, two events and two small page-locked staging buffers.  Results are
 * bit-identical to the resident path for the same records.
 * moe_cache_stats returns the hits and misses so far.  Errors: ARG, STATE. */
moe_status moe_cache_stats(moe_layer_t layer, uint64_t* hits, uint64_t* misses);

/* Pins experts into the slot cache: a static hot set chosen by the caller
 * (for instance the most used experts of a statistics pass), as the pinned
 * hot-store of the Colibri README.  experts: host [n] distinct ids in [0, E);
 * 0 <= n <= n_slots - top_k (a token's misses always find an unpinned slot).
 * Replaces any previous pinned set.  Experts not resident are copied from
 * host_pool into free or evicted unpinned slots on `stream` (ordered after
 * the work already on it); pinned slots are never evicted.  Pinning counts as
 * neither hit nor miss.  Errors: ARG, STATE (no slot cache), HIP. */
moe_status moe_cache_pin(moe_layer_t layer, const int32_t* experts, int32_t n, void* stream);

/* Usage-learned pinning: the persistent usage heatmap of the Colibri README
 * ("Learn", `.coli_usage`), which pins the hottest experts at startup.  The
 * heatmap is the handle's per-expert selection count (+1 per selection, hit
 * or miss, never decayed: the LFU's own counts).
 *   moe_cache_usage: counts  host [E], receives the counts.  Errors: ARG, STATE.
 *   moe_cache_pin_hottest: pins the n experts with the largest counts in
 *     `counts` (host [E]: a heatmap saved by an earlier run, or NULL for this
 *     handle's own), ties to the lower id, exactly as moe_cache_pin would pin
 *     that list (same n limits, slots, copies on `stream`, errors).
 * Errors: ARG, STATE (no slot cache), HIP. */
moe_status moe_cache_usage(moe_layer_t layer, uint64_t* counts);
moe_status moe_cache_pin_hottest(moe_layer_t layer, const uint64_t* counts, int32_t n, void* stream);

/* Router lookahead: starts copying the experts this layer is predicted to
 * select before its own router runs, from a hint vector that is available
 * earlier -- the next layer's router applied to the current layer's state, as
 * the experimental router-lookahead prefetch of the Colibri README (PILOT=1)
 * and the Colibri analysis report (section 5) describe.
 *   x_hint     device [H], the layer's act_dtype: one token's hint vector.
 *   n_predict  1..top_k: how many of the hint's top-k experts to fetch.
 *   workspace  as for the compute calls (moe_workspace_bytes(layer, 1) or more).
 *   predicted  host [n_predict] or NULL: receives the predicted ids, rank order.
 * Runs the router and top-k on x_hint on `stream`, waits on the host for the
 * predicted ids, and copies every predicted expert that is not resident from
 * host_pool into a free slot, else into the slot the cache policy would evict
 * (never a pinned slot or another predicted expert; with none left the rest
 * are skipped), on the handle's side stream (DMA copies), ordered after the layer's own
 * earlier kernels that read its slots (not after other work on `stream`).
 * The next compute call on the layer waits for those copies
 * before it reads any slot.  Prefetching changes only which experts are
 * resident: results stay bit-identical, and hits and misses are counted at the
 * compute calls as before (a prefetched expert that is then selected is a
 * hit).  moe_cache_prefetch_stats returns the copies issued and how many of
 * the prefetched experts were selected before being evicted.
 * Errors: ARG, ALIGN, STATE (no slot cache), HIP. */
moe_status moe_cache_prefetch(moe_layer_t layer, const void* x_hint, int32_t n_predict,
                              void* workspace, int32_t* predicted, void* stream);

/* The same prefetch for predicted ids the caller already holds on the host
 * (for instance from moe_route_topk on the hint and an asynchronous copy that
 * the caller has seen complete): no router launch and no host wait.
 *   experts  host [n] distinct ids in [0, E), most confident first; 1 <= n <= top_k.
 * Copies are ordered as for moe_cache_prefetch; `stream` is the layer's
 * stream (unused by the copies themselves).  Errors: ARG, STATE, HIP. */
moe_status moe_cache_prefetch_ids(moe_layer_t layer, const int32_t* experts, int32_t n,
                                  void* stream);
moe_status moe_cache_prefetch_stats(moe_layer_t layer, uint64_t* issued, uint64_t* used);

/* Reads and clears the device error flag kept in `workspace` (synchronises
 * `stream`).  MOE_OK if no kernel reported bad input since the last poll,
 * MOE_ERR_DEVICE otherwise. */
moe_status moe_poll_device_error(moe_layer_t layer, void* workspace, void* stream);

/* Measurement reference (not part of the layer): reads `bytes` bytes of device
 * memory at `src` (16-byte aligned, bytes a positive multiple of 16) with the
 * 16-byte nontemporal loads the expert kernels use, `n_blocks` workgroups of
 * 256 threads each reading one contiguous slice, and no arithmetic beyond an
 * XOR of the loaded words.  Its rate is what this chip's HBM delivers to a
 * plain read-only stream of that size, the achievable figure the expert
 * kernels' rates are set against.  sink: device, one 32-bit word, written only
 * when the XOR equals a fixed value the data practically never produce (so the
 * loads cannot be removed).  Kernel id 10 in the profile records.  Enqueued on
 * `stream`.  Errors: ARG, ALIGN, HIP. */
moe_status moe_stream_read(const void* src, size_t bytes, int32_t n_blocks, uint32_t* sink, void* stream);

/* Measurement support.  While profiling is on, the library dispatches the
 * first kernel of each launch step with hipExtLaunchKernelGGL carrying a
 * start/stop hipEvent pair, so the pair holds that dispatch's own start and
 * end on its launch stream (up to `capacity` launches).  moe_profile_read
 * synchronises those events and writes,
 * per recorded launch, the kernel id (0 router, 1 activation prep, 2 gate/up,
 * 3 down with in-place combine, 4 combine, 5 top-k; for calls of 4 or more
 * tokens: 6 activation prep, 7 grouping by expert, 8 grouped gate/up, 9 grouped
 * down; 10 moe_stream_read) and the elapsed milliseconds;
 * it returns the number of records (or a negative status) and clears them.
 * Profiling state is process-wide and not thread-safe; do not profile inside
 * stream capture.  Errors: ARG, HIP, NOMEM. */
moe_status moe_profile_start(int32_t capacity);
moe_status moe_profile_stop(void);
int32_t moe_profile_read(int32_t* kernel_ids, float* ms, int32_t max_records);

const char* moe_status_str(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */

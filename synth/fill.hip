// fill.hip -- GPU implementation of the synthetic expert-record generator
// defined in synth/__init__.py (SplitMix64 counter streams; Steele, Lea and
// Flood, OOPSLA 2014).  Input infrastructure only: it writes random bytes and
// random fp16 scale/bias pairs, and computes nothing of the MoE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __host__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// key(seed, layer, kind, index): fold k = mix64((k ^ p) + gamma) from k = 0
__device__ __host__ inline uint64_t key4(uint64_t seed, uint64_t layer, uint64_t kind, uint64_t idx) {
    uint64_t k = 0;
    k = mix64((k ^ seed) + kGamma);
    k = mix64((k ^ layer) + kGamma);
    k = mix64((k ^ kind) + kGamma);
    k = mix64((k ^ idx) + kGamma);
    return k;
}

__device__ inline double unit_uniform(uint64_t u) { return (double)(u >> 11) * 0x1.0p-53; }

// double -> fp32 -> fp16, each step round-to-nearest-even.  The empty asm keeps
// the compiler from fusing the two roundings into one (a different result on
// fp16 ties).
__device__ inline uint16_t f16_bits(double v) {
    float f = (float)v;
    asm volatile("" : "+v"(f));
    const _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// grid (blocks, n_records); record r is expert first_index + r (or the shared
// expert's index when first_index < 0), written at dst + r * stride.  A record
// is segments of seg_code code bytes followed by 256 bytes (64 pairs) of
// (scale, bias): code word i (8 bytes) goes to segment i / (seg_code / 8),
// pair j to segment j / 64.
__global__ void k_fill_records(uint8_t* dst, int64_t stride, int64_t nib_bytes, int64_t npairs,
                               int64_t seg_code, uint64_t seed, int layer, int first_index) {
    const int r = blockIdx.y;
    const uint64_t idx = first_index < 0 ? 0xFFFFull : (uint64_t)(first_index + r);
    const uint64_t kn = key4(seed, layer, 1, idx), ks = key4(seed, layer, 2, idx),
                   kb = key4(seed, layer, 3, idx);
    uint8_t* rec = dst + (size_t)r * stride;
    const int64_t seg = seg_code + 256, wps = seg_code / 8;  // segment bytes, code words per segment
    const int64_t n64 = nib_bytes / 8;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n64; i += step)
        *(uint64_t*)(rec + (i / wps) * seg + (i % wps) * 8) = mix64(kn + (uint64_t)(i + 1) * kGamma);
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < npairs; j += step) {
        const double us = unit_uniform(mix64(ks + (uint64_t)(j + 1) * kGamma));
        const double ub = unit_uniform(mix64(kb + (uint64_t)(j + 1) * kGamma));
        const double s = __dadd_rn(1e-3, __dmul_rn(9e-3, us));
        const double b = __dmul_rn(-8e-3, ub);
        *(uint32_t*)(rec + (j / 64) * seg + seg_code + (j % 64) * 4) =
            (uint32_t)f16_bits(s) | ((uint32_t)f16_bits(b) << 16);
    }
}
}  // namespace

extern "C" int synth_fill_records(void* dst, int64_t stride, int hidden, int inter, uint64_t seed,
                                  int layer, int first_index, int n_records, void* stream, int bits) {
    if (!dst || hidden <= 0 || inter <= 0 || hidden % 64 || inter % 64 || n_records <= 0 ||
        n_records > 65535 || (bits != 4 && bits != 2))
        return -1;
    const int64_t nib = (int64_t)3 * hidden * inter * bits / 8;  // code region bytes
    const int64_t npairs = (int64_t)3 * hidden * inter / 64;
    if (stride < nib + 4 * npairs) return -1;
    int64_t want = (nib / 8 + 255) / 256;
    const int blocks = (int)(want < 1024 ? (want < 1 ? 1 : want) : 1024);
    const int64_t seg_code = (int64_t)64 * 64 * bits / 8;  // code bytes per segment
    hipLaunchKernelGGL(k_fill_records, dim3(blocks, n_records), dim3(256), 0,
                       (hipStream_t)stream, (uint8_t*)dst, stride, nib, npairs, seg_code, seed, layer,
                       first_index);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

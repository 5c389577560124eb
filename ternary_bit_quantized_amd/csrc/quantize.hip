// Weight-side conversions on the GPU: the reference quantizer (f32 -> Q2_0) and the
// reader of the legacy group-128 packing (-> Q2_0 with group 64).
//
// aisvetem.cz, "Llama.cpp umi dvoubitovy Q2_0 i na kartach NVIDIA":
//  * section "Na bezny model to neni": the reference quantizer takes the block's
//    largest |w| as the scale and puts every weight on the nearest of the four levels;
//  * sections "Osmnact bajtu na ctyriasedesat vah" and "Sest procent, o ktera se vedl
//    spor": the merged format groups 64 weights in 18 bytes, the older packing 128
//    weights in 34 bytes.
//
// Quantizer: four threads per block, one per 32-bit code word (16 weights).  The
// scale is the half nearest to max|w| (ties to even, the hardware conversion); the
// nearest level is chosen by comparing w with the midpoints -d/2, d/2 and 3d/2, all
// exact in f32, so a weight exactly between two levels goes to the one nearer zero
// (code 1 at +-d/2, code 2 at 3d/2).  |w| <= max|w| < 1.5 d, so code 3 never occurs.
// A block whose scale rounds to 0 gets code 1 everywhere.
//
// Group-128 reader: a legacy block is a half scale and eight little-endian code
// words, code i of word w belonging to weight 16w+i (the group-64 convention,
// extended to 128 weights); its two halves become two group-64 blocks with the same
// scale.  Pure byte moves.
#include "q2_0_internal.h"

namespace q2_0 {

namespace {

__device__ __forceinline__ void store_u32_as_u16x2(uint16_t *p, uint32_t v) {
    p[0] = (uint16_t)v;
    p[1] = (uint16_t)(v >> 16);
}

template <bool kVec>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ src, int64_t ld, int nb,
                                                       int64_t n_blocks, uint8_t *__restrict__ w) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = t >> 2;
    const int word = (int)(t & 3);
    const bool live = blk < n_blocks;
    const int64_t b = live ? blk : n_blocks - 1;   // the tail's lanes redo the last block and store nothing
    const int64_t m = b / nb, kb = b - m * nb;
    const float *p = src + m * ld + kb * kBlockWeights + 16 * word;
    float v[16];
    if (kVec) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4_t f = reinterpret_cast<const float4_t *>(p)[q];
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = p[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // the four threads of a block are consecutive lanes
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const _Float16 dh = (_Float16)amax;
    const float d = (float)dh, hd = 0.5f * d, h3 = d + hd;
    uint32_t codes = 0;
    if (d != 0.f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t q = (v[i] < -hd) ? 0u : (v[i] <= hd) ? 1u : (v[i] <= h3) ? 2u : 3u;
            codes |= q << (2 * i);
        }
    } else {
        codes = 0x55555555u;   // code 1 everywhere
    }
    if (live) {
        uint16_t *out = reinterpret_cast<uint16_t *>(w + blk * kBlockBytes);
        if (word == 0) out[0] = __builtin_bit_cast(uint16_t, dh);
        store_u32_as_u16x2(out + 1 + 2 * word, codes);
    }
}

// One thread per output (group-64) block: 9 half-words copied.
__global__ __launch_bounds__(256) void repack_g128_kernel(const uint8_t *__restrict__ w128, int64_t n_out,
                                                          uint8_t *__restrict__ w) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= n_out) return;
    const int64_t j = o >> 1;
    const int h = (int)(o & 1);
    const uint16_t *s = reinterpret_cast<const uint16_t *>(w128 + j * 34);
    uint16_t *d = reinterpret_cast<uint16_t *>(w + o * kBlockBytes);
    d[0] = s[0];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[1 + i] = s[1 + 8 * h + i];
}

}  // namespace

hipError_t launch_quantize(const float *src, int64_t M, int nb, int64_t ld, uint8_t *w, hipStream_t s) {
    const int64_t n_blocks = M * nb;
    const int64_t threads = n_blocks * 4;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (((uintptr_t)src % 16 == 0) && (ld % 4 == 0))
        quantize_kernel<true><<<grid, 256, 0, s>>>(src, ld, nb, n_blocks, w);
    else
        quantize_kernel<false><<<grid, 256, 0, s>>>(src, ld, nb, n_blocks, w);
    return hipGetLastError();
}

hipError_t launch_repack_g128(const uint8_t *w128, int64_t M, int64_t K, uint8_t *w, hipStream_t s) {
    const int64_t n_out = M * (K / kBlockWeights);
    const dim3 grid((unsigned)((n_out + 255) / 256));
    repack_g128_kernel<<<grid, 256, 0, s>>>(w128, n_out, w);
    return hipGetLastError();
}

}  // namespace q2_0

// get_rows: gather Q2_0 rows and dequantize them to f32, bit-exact.
//
// bisque.today, "WebGPU: add Q2_0 support", the paragraph on its three shaders: the
// gather shader expands selected rows to f32, 64 values per block, code q giving the
// weight (q - 1) * d.
//
// One thread per 32-bit code word (16 weights): it reads the block's half scale and
// its word, and writes 16 floats as 4 x 16-byte stores when the output row allows.
// Each output is the IEEE product f32(q - 1) * f32(d); there is no FMA and no
// rewrite such as q*d - d, so signs of zero and NaN/inf follow the product.
#include "q2_0_internal.h"

namespace q2_0 {

template <bool kVecStore>
__global__ __launch_bounds__(256) void get_rows_kernel(const uint8_t *__restrict__ w, int64_t M,
                                                       int nb, const int32_t *__restrict__ ids,
                                                       int64_t n_ids, float *__restrict__ out,
                                                       int64_t ld_out) {
    const int words = nb * 4;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= words) return;
    for (int64_t r = blockIdx.y; r < n_ids; r += gridDim.y) {
        float *o = out + r * ld_out + (int64_t)t * 16;
        const int64_t id = ids[r];
        float v[16];
        if (id < 0 || id >= M) {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = __builtin_nanf("");
        } else {
            const uint16_t *blk16 =
                reinterpret_cast<const uint16_t *>(w + (id * nb + (t >> 2)) * kBlockBytes);
            const float d = half_bits_to_float(blk16[0]);
            const uint32_t q = load_word_u16x2(blk16, t & 3);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = (float)((int)((q >> (2 * i)) & 3u) - 1) * d;
        }
        if (kVecStore) {
            float4_t *o4 = reinterpret_cast<float4_t *>(o);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_nontemporal_store(float4_t{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]},
                                            o4 + j);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] = v[i];
        }
    }
}

hipError_t launch_get_rows(const uint8_t *w, int64_t M, int nb, const int32_t *ids, int64_t n_ids,
                           float *out, int64_t ld_out, hipStream_t s) {
    const int words = nb * 4;
    // at most 256 rows at a time (a workgroup per CU), each workgroup looping over its
    // rows: 2048 rows of 4096 took 14.9 us, against 16.9 with a workgroup per row and
    // 19.3 with 128 at a time
    dim3 grid((words + 255) / 256, (unsigned)(n_ids < 256 ? n_ids : 256));
    const bool vec = ((uintptr_t)out % 16 == 0) && (ld_out % 4 == 0);
    if (vec)
        get_rows_kernel<true><<<grid, 256, 0, s>>>(w, M, nb, ids, n_ids, out, ld_out);
    else
        get_rows_kernel<false><<<grid, 256, 0, s>>>(w, M, nb, ids, n_ids, out, ld_out);
    return hipGetLastError();
}

}  // namespace q2_0

// K0: int8 quantisation of W2 with one fp32 scale per row (vLLM PR #62958, Overview), and the
// Philox test hook. Load-time work; HBM-bound (reads V*256 elements, writes V*256 + 4V bytes).
#include "device_common.hpp"
#include "internal.hpp"

namespace dspark {

// Set when a row holds a NaN or infinity; one copy per device.
__device__ unsigned int g_quant_nonfinite;

// One wave per row; lane l owns elements 4l .. 4l+3, so loads and the 256-byte row store are
// contiguous across the wave. s = absmax / 127 and q = rint(w / s) use IEEE fp32 division
// (the default for HIP fp32 '/' without fast-math) and round half to even.
template <int DT>
__global__ __launch_bounds__(256) void quantize_w2_kernel(const void* __restrict__ w2, int64_t V,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ s) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int64_t row = (int64_t)blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
    if (row >= V) return;
    const float4 w = load4_as_f32<DT>(w2, row * RANK + lane * 4);
    const bool finite = isfinite(w.x) && isfinite(w.y) && isfinite(w.z) && isfinite(w.w);
    if (__any(!finite) && lane == 0) atomicOr(&g_quant_nonfinite, 1u);
    float a = fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w)));
    a = wave_max_nonneg_f32(a);
    uint32_t packed = 0;
    float sv = 0.0f;
    if (a > 0.0f) {
        sv = a / 127.0f;
        const float v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r = rintf(v[i] / sv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            packed |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * i);
        }
    }
    reinterpret_cast<uint32_t*>(q + row * RANK)[lane] = packed;
    if (lane == 0) s[row] = sv;
}

int launch_quantize(const void* w2, int dtype, int64_t V, int8_t* q, float* s, hipStream_t stream) {
    const unsigned int zero = 0;
    if (hipMemcpyToSymbolAsync(HIP_SYMBOL(g_quant_nonfinite), &zero, sizeof(zero), 0,
                               hipMemcpyHostToDevice, stream) != hipSuccess)
        return DSPARK_ERR_LAUNCH;
    const int rows_per_block = 4;
    const dim3 grid((unsigned)((V + rows_per_block - 1) / rows_per_block));
    const dim3 block(rows_per_block * WAVE);
    switch (dtype) {
        case DSPARK_F32: quantize_w2_kernel<DT_F32><<<grid, block, 0, stream>>>(w2, V, q, s); break;
        case DSPARK_BF16: quantize_w2_kernel<DT_BF16><<<grid, block, 0, stream>>>(w2, V, q, s); break;
        default: quantize_w2_kernel<DT_F16><<<grid, block, 0, stream>>>(w2, V, q, s); break;
    }
    if (hipGetLastError() != hipSuccess) return DSPARK_ERR_LAUNCH;
    unsigned int flag = 0;
    if (hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_quant_nonfinite), sizeof(flag), 0,
                                 hipMemcpyDeviceToHost, stream) != hipSuccess)
        return DSPARK_ERR_LAUNCH;
    if (hipStreamSynchronize(stream) != hipSuccess) return DSPARK_ERR_LAUNCH;
    return flag ? DSPARK_ERR_NONFINITE : DSPARK_OK;
}

__global__ void philox_words_kernel(uint64_t seed, uint64_t position, int64_t v0, int64_t n,
                                    uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = noise_word(seed, position, (uint32_t)(v0 + i));
}

int launch_philox_words(uint64_t seed, uint64_t position, int64_t v0, int64_t n, uint32_t* out,
                        hipStream_t stream) {
    const int threads = 256;
    philox_words_kernel<<<(unsigned)((n + threads - 1) / threads), threads, 0, stream>>>(
        seed, position, v0, n, out);
    return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

}  // namespace dspark

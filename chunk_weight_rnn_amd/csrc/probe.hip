// Microbenchmarks of the chip's own ceilings, for comparison with the vendor
// peaks the roofline is priced against: bf16 MFMA throughput (the two shapes
// the kernels use) and HBM read bandwidth.  Built as a separate library; not
// part of the chunk-update ABI.
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every wavefront runs `iters` rounds of NA independent accumulations, so
// consecutive MFMAs never wait for each other's results; the sums are stored
// so that nothing is optimised away.
template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1e-3f * (float)(lane + e));
        b[e] = (__bf16)(1e-3f * (float)(lane - e));
    }
    float s = 0.f;
    if (SHAPE == 0 || SHAPE == 2) {  // v_mfma_f32_16x16x32_bf16 (8 or 16 independent accumulators)
        constexpr int NA = SHAPE == 0 ? 8 : 16;
        f32x4 acc[NA] = {};
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int k = 0; k < NA; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < NA; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[k][e];
    } else if (SHAPE == 3) {  // v_mfma_f32_16x16x16_bf16 (the K = 16 form)
        constexpr int NA = 8;
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        i16x4 a4, b4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a4[e] = __builtin_bit_cast(short, a[e]);
            b4[e] = __builtin_bit_cast(short, b[e]);
        }
        f32x4 acc[NA] = {};
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int k = 0; k < NA; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, acc[k], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < NA; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[k][e];
    } else {  // v_mfma_f32_32x32x16_bf16
        constexpr int NA = 4;
        f32x16 acc[NA] = {};
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int k = 0; k < NA; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
#pragma unroll
        for (int k = 0; k < NA; ++k)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[k][e];
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Grid-stride 16-byte loads over n4 float4 elements; one partial sum per thread.
__global__ __launch_bounds__(256) void read_probe_kernel(const f32x4* src, size_t n4, float* out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) acc += src[i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

// Flops of one launch: grid * 4 wavefronts * iters * flops per round: shape 0
// 8 x 16x16x32, shape 1 4 x 32x32x16, shape 2 16 x 16x16x32, shape 3
// 8 x 16x16x16 (2 M N K each).  `out` holds grid * 256 floats.
// Returns a hipError_t code.
extern "C" __attribute__((visibility("default"))) int e2ttt_probe_mfma(int shape, int iters, float* out, int grid,
                                                                       void* stream) {
    if (iters < 1 || grid < 1 || !out) return (int)hipErrorInvalidValue;
    if (shape == 0)
        hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    else if (shape == 1)
        hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    else if (shape == 2)
        hipLaunchKernelGGL(mfma_probe_kernel<2>, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    else if (shape == 3)
        hipLaunchKernelGGL(mfma_probe_kernel<3>, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, out, iters);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// Reads n4 float4 (16 bytes each) from src once; `out` holds grid * 256 floats.
extern "C" __attribute__((visibility("default"))) int e2ttt_probe_read(const void* src, size_t n4, float* out, int grid,
                                                                       void* stream) {
    if (!src || !out || grid < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, (const f32x4*)src,
                       n4, out);
    return (int)hipGetLastError();
}

// Microbenchmarks of the chip's own ceilings, for comparison with the vendor
// peaks the roofline is priced against: bf16 MFMA throughput (the shapes the
// kernels use), how far one SIMD overlaps MFMA and VALU work of different
// wavefronts, LDS bandwidth per compute unit and HBM read bandwidth.  Built
// as a separate library; not part of the chunk-update ABI.
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

// MFMA and VALU on one SIMD.  512-thread workgroups, 8 wavefronts, two per
// SIMD: with mode bit 1 wavefronts 0-3 each run `iters` rounds of 16
// independent 16x16x32 bf16 MFMAs; with mode bit 2 wavefronts 4-7 each run
// `iters` rounds of 16 V dependent-free fp32 FMAs (8 independent chains).
// Mode 3 runs both, so the time against modes 1 and 2 alone shows how far the
// SIMD overlaps one wavefront's MFMAs with another's VALU work.
template <int V>
__global__ __launch_bounds__(512) void overlap_probe_kernel(int mode, int iters, float* out) {
    const int wave = threadIdx.x >> 6;
    float r = 0.f;
    if (wave < 4 && (mode & 1)) {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(1e-3f * (float)threadIdx.x);
            b[e] = (__bf16)(1e-3f * (float)e);
        }
        f32x4 acc[16] = {};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) r += acc[i][0];
    } else if (wave >= 4 && (mode & 2)) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 1e-3f * (float)threadIdx.x + (float)i;
        const float fa = 0.999f, fb = 1e-3f;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 16 * V; ++i) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(x[i & 7]) : "v"(fa), "v"(fb));
#pragma unroll
        for (int i = 0; i < 8; ++i) r += x[i];
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// LDS bandwidth of one compute unit: the first `nwaves` wavefronts of a
// 768-thread workgroup each issue `iters` x 16 conflict-free LDS accesses,
// mode 0 ds_read_b128, 1 ds_read_b64_tr_b16 (8 bytes per lane), 2
// ds_write_b128.  Every access stays inside the 64 KB buffer.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
template <int MODE>
__global__ __launch_bounds__(768) void lds_probe_kernel(int nwaves, int iters, unsigned* out) {
    constexpr int BYTES = 64 * 1024;
    __shared__ __attribute__((aligned(16))) unsigned char buf[BYTES];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < BYTES / 4; i += blockDim.x) ((unsigned*)buf)[i] = (unsigned)i;
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (wave < nwaves) {
        const int base = (wave * 1024 + lane * 16) & (BYTES - 1);
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                int off = (base + k * 4096) & (BYTES - 1);  // 16-byte aligned, at most BYTES - 16
                asm volatile("" : "+v"(off));
                if (MODE == 0) {
                    acc ^= *(const u32x4*)(buf + off);
                } else if (MODE == 1) {
                    const int o2 = (off & ~511) + lane * 8;  // 64 lanes x 8 bytes, consecutive
                    const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(buf + o2));
                    const unsigned long long w = __builtin_bit_cast(unsigned long long, v);
                    acc[0] ^= (unsigned)w;
                    acc[1] ^= (unsigned)(w >> 32);
                } else {
                    *(u32x4*)(buf + off) = acc;
                    acc[0] += 1u;
                }
            }
        }
    }
    __syncthreads();
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ buf[(threadIdx.x * 16) & (BYTES - 1)];
}

}  // namespace

// mode 1, 2 or 3 (see overlap_probe_kernel), v 2 or 4; `out` holds grid * 512 floats.
extern "C" __attribute__((visibility("default"))) int e2ttt_probe_overlap(int mode, int v, int iters, float* out,
                                                                          int grid, void* stream) {
    if (mode < 1 || mode > 3 || iters < 1 || grid < 1 || !out) return (int)hipErrorInvalidValue;
    if (v == 2)
        hipLaunchKernelGGL(overlap_probe_kernel<2>, dim3((unsigned)grid), dim3(512), 0, (hipStream_t)stream, mode, iters,
                           out);
    else if (v == 4)
        hipLaunchKernelGGL(overlap_probe_kernel<4>, dim3((unsigned)grid), dim3(512), 0, (hipStream_t)stream, mode, iters,
                           out);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

// Bytes per launch: grid * nwaves * iters * 16 * (1024, 512, 1024 for modes 0, 1, 2);
// nwaves 1..12; `out` holds grid * 768 words.
extern "C" __attribute__((visibility("default"))) int e2ttt_probe_lds(int mode, int nwaves, int iters, unsigned* out,
                                                                      int grid, void* stream) {
    if (mode < 0 || mode > 2 || nwaves < 1 || nwaves > 12 || iters < 1 || grid < 1 || !out)
        return (int)hipErrorInvalidValue;
    if (mode == 0)
        hipLaunchKernelGGL(lds_probe_kernel<0>, dim3((unsigned)grid), dim3(768), 0, (hipStream_t)stream, nwaves, iters, out);
    else if (mode == 1)
        hipLaunchKernelGGL(lds_probe_kernel<1>, dim3((unsigned)grid), dim3(768), 0, (hipStream_t)stream, nwaves, iters, out);
    else
        hipLaunchKernelGGL(lds_probe_kernel<2>, dim3((unsigned)grid), dim3(768), 0, (hipStream_t)stream, nwaves, iters, out);
    return (int)hipGetLastError();
}

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

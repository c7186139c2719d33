// Portable fp32 chunk loop: every fast-weight kind and loss, any shape with
// D <= 256 and Hd <= 1024.  It serves the fp32-I/O workloads (linear and MLP
// fast weights, where MSE couples all hidden units so a head cannot be split
// across workgroups) and every shape the SwiGLU MFMA path does not take.
//
// The chunk update follows "Rethinking Expressivity and Efficiency in
// Test-Time Training" (abstract; atlas summary "Approach"):
//   1. output of every token of the chunk from the chunk-start weights,
//   2. per-token backward factors at the chunk-start weights,
//   3. the two coefficient-weighted gradient aggregations
//        G^M = sum_i cM_i g_i,   G^W = sum_i cW_i g_i   (cM, cW from logscan),
//   4. M <- Bb*M + G^M,  W <- A*W - gamma*M_old - G^W.
//
// One 1024-thread workgroup per (b, h).  The state lives in the W_end / M_end
// buffers (fp32, L2-resident) and G^M, G^W in a per-head workspace slice.
// Tokens are staged through LDS in blocks of TB; every contraction is a plain
// fp32 dot product (no reassociation beyond the per-thread loop order).
#include <math.h>

#include "e2ttt_internal.h"

namespace e2ttt {
namespace {

constexpr int NT = 1024;  // 16 wavefronts: the fp32 loops are latency-bound

struct GenericArgs {
    int64_t T, D, Hd, C, nc, P;
    int64_t ldc;  // row stride of cM / cW (tokens, >= T)
    int loss, TB;
    int nomom;  // no momentum: M0 / M are not used (the scalar kernels already have beta = 0)
    int wlds;   // 1: the chunk-start weights are copied to LDS after the token rows
    const void* q;
    const void* k;
    const void* v;
    const float* cM;
    const float* cW;
    const float* scal;
    const float* W0;
    const float* M0;
    void* out;
    float* W;
    float* M;
    float* gacc;
    float* save;  // [BH][nc][2][P] chunk-start W, M (may be null)
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigm(x); }
__device__ __forceinline__ float dsilu_f(float x) {
    const float s = sigm(x);
    return s * (1.f + x * (1.f - s));
}

template <int KIND, typename TIO, bool WLDS>
__global__ __launch_bounds__(NT) void generic_kernel(GenericArgs a) {
    extern __shared__ float smem[];
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int D = (int)a.D, Hd = (int)a.Hd, TB = a.TB;
    const int64_t P = a.P;
    float* xs = smem;             // [TB][D]  q or k
    float* vs = xs + TB * D;      // [TB][D]
    float* dys = vs + TB * D;     // [TB][D]  dL/dy
    float* h1s = dys + TB * D;    // [TB][Hd]
    float* h3s = h1s + TB * Hd;   // [TB][Hd]
    float* us = h3s + TB * Hd;    // [TB][Hd]
    float* cms = us + TB * Hd;    // [TB]
    float* cws = cms + TB;        // [TB]
    float* wl = cws + TB;         // [P] chunk-start weights (when a.wlds)

    float* W = a.W + bh * P;
    float* M = a.nomom ? nullptr : a.M + bh * P;
    float* GM = a.gacc + bh * 2 * P;
    float* GW = GM + P;
    const float* W0 = a.W0 + bh * P;
    const float* M0 = a.nomom ? nullptr : a.M0 + bh * P;
    const TIO* q = (const TIO*)a.q + bh * a.T * D;
    const TIO* k = (const TIO*)a.k + bh * a.T * D;
    const TIO* v = (const TIO*)a.v + bh * a.T * D;
    TIO* out = (TIO*)a.out + bh * a.T * D;

    for (int64_t p = tid; p < P; p += NT) {
        W[p] = W0[p];
        if (M) M[p] = M0[p];
        GM[p] = 0.f;
        GW[p] = 0.f;
    }
    __syncthreads();

    // matrix views of the chunk-start weights: the LDS copy when it fits,
    // else the state buffer itself (read-only until step 4).  The LDS copy
    // pads every matrix row by one float, so that lanes reading one column of
    // consecutive rows hit distinct banks (rows of D or Hd floats are a
    // multiple of the 64 banks otherwise).
    const int pad = WLDS ? 1 : 0;
    const int64_t sD = D + pad, sH = Hd + pad;    // row strides of D- and Hd-wide rows
    const float* Wr = WLDS ? wl : W;
    const float* Wl = Wr;                         // linear  [D][D]     (rows of D)
    const float* W1 = Wr;                         // mlp [Hd][D] (rows of D); swiglu [D][Hd] (rows of Hd)
    const float* W3 = Wr + (int64_t)D * sH;       // swiglu [D][Hd]
    const float* W2m = Wr + (int64_t)Hd * sD;     // mlp [D][Hd]         (rows of Hd)
    const float* W2s = Wr + 2 * (int64_t)D * sH;  // swiglu [Hd][D]      (rows of D)

    for (int64_t c = 0; c < a.nc; ++c) {
        const int64_t t0 = c * a.C;
        const int64_t Cc = min(a.C, a.T - t0);  // the last chunk may be shorter
        if (a.save) {  // chunk-start state for the backward pass
            float* sv = a.save + (bh * a.nc + c) * 2 * P;
            for (int64_t p = tid; p < P; p += NT) {
                sv[p] = W[p];
                sv[P + p] = M ? M[p] : 0.f;
            }
        }
        if (WLDS) {  // packed index -> padded (row, column)
            for (int64_t p = tid; p < P; p += NT) {
                int64_t o;
                if (KIND == E2TTT_LINEAR) {
                    o = (p / D) * sD + p % D;
                } else if (KIND == E2TTT_MLP) {
                    const int64_t n1 = (int64_t)Hd * D;
                    o = p < n1 ? (p / D) * sD + p % D : n1 + Hd + ((p - n1) / Hd) * sH + (p - n1) % Hd;
                } else {
                    const int64_t n1 = (int64_t)D * Hd;
                    o = p < 2 * n1 ? (p / Hd) * sH + p % Hd : 2 * D * sH + ((p - 2 * n1) / D) * sD + (p - 2 * n1) % D;
                }
                wl[o] = W[p];
            }
            __syncthreads();
        }
        // ---- 1. outputs from the chunk-start weights
        for (int64_t b0 = 0; b0 < Cc; b0 += TB) {
            const int nt = (int)min((int64_t)TB, Cc - b0);
            for (int i = tid; i < nt * D; i += NT) xs[i] = to_f32(q[(t0 + b0) * D + i]);
            __syncthreads();
            if (KIND == E2TTT_LINEAR) {
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) acc += Wl[r * sD + d] * xs[t * D + d];
                    out[(t0 + b0) * D + i] = from_f32<TIO>(acc);
                }
            } else if (KIND == E2TTT_MLP) {
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) acc += W1[j * sD + d] * xs[t * D + d];
                    us[t * Hd + j] = silu_f(acc);
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) acc += W2m[r * sH + j] * us[t * Hd + j];
                    out[(t0 + b0) * D + i] = from_f32<TIO>(acc);
                }
            } else {
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float a1 = 0.f, a3 = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) {
                        const float x = xs[t * D + d];
                        a1 += x * W1[d * sH + j];
                        a3 += x * W3[d * sH + j];
                    }
                    us[t * Hd + j] = silu_f(a1) * a3;
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) acc += us[t * Hd + j] * W2s[j * sD + r];
                    out[(t0 + b0) * D + i] = from_f32<TIO>(acc);
                }
            }
            __syncthreads();
        }

        // ---- 2-3. backward factors at the chunk-start weights, aggregated into G
        for (int64_t b0 = 0; b0 < Cc; b0 += TB) {
            const int nt = (int)min((int64_t)TB, Cc - b0);
            for (int i = tid; i < nt * D; i += NT) {
                xs[i] = to_f32(k[(t0 + b0) * D + i]);
                vs[i] = to_f32(v[(t0 + b0) * D + i]);
            }
            for (int i = tid; i < TB; i += NT) {
                cms[i] = i < nt ? a.cM[bh * a.ldc + t0 + b0 + i] : 0.f;
                cws[i] = i < nt ? a.cW[bh * a.ldc + t0 + b0 + i] : 0.f;
            }
            __syncthreads();
            if (KIND == E2TTT_LINEAR) {
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float g = -vs[i];
                    if (a.loss == E2TTT_LOSS_MSE) {
                        float acc = 0.f;
                        #pragma unroll 4
                        for (int d = 0; d < D; ++d) acc += Wl[r * sD + d] * xs[t * D + d];
                        g = acc - vs[i];
                    }
                    dys[i] = g;
                }
                __syncthreads();
                for (int64_t p = tid; p < P; p += NT) {
                    const int r = (int)(p / D), d = (int)(p % D);
                    float gm = 0.f, gw = 0.f;
                    #pragma unroll 4
                    for (int t = 0; t < nt; ++t) {
                        const float g = dys[t * D + r] * xs[t * D + d];
                        gm += cms[t] * g;
                        gw += cws[t] * g;
                    }
                    GM[p] += gm;
                    GW[p] += gw;
                }
            } else if (KIND == E2TTT_MLP) {
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) acc += W1[j * sD + d] * xs[t * D + d];
                    h1s[i] = acc;          // z
                    us[i] = silu_f(acc);   // a
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float g = -vs[i];
                    if (a.loss == E2TTT_LOSS_MSE) {
                        float acc = 0.f;
                        #pragma unroll 4
                        for (int j = 0; j < Hd; ++j) acc += W2m[r * sH + j] * us[t * Hd + j];
                        g = acc - vs[i];
                    }
                    dys[i] = g;
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) acc += W2m[r * sH + j] * dys[t * D + r];
                    h3s[i] = acc * dsilu_f(h1s[i]);  // dz
                }
                __syncthreads();
                const int64_t n1 = (int64_t)Hd * D;
                for (int64_t p = tid; p < P; p += NT) {
                    float gm = 0.f, gw = 0.f;
                    if (p < n1) {
                        const int j = (int)(p / D), d = (int)(p % D);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const float g = h3s[t * Hd + j] * xs[t * D + d];
                            gm += cms[t] * g;
                            gw += cws[t] * g;
                        }
                    } else {
                        const int r = (int)((p - n1) / Hd), j = (int)((p - n1) % Hd);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const float g = dys[t * D + r] * us[t * Hd + j];
                            gm += cms[t] * g;
                            gw += cws[t] * g;
                        }
                    }
                    GM[p] += gm;
                    GW[p] += gw;
                }
            } else {
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float a1 = 0.f, a3 = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) {
                        const float x = xs[t * D + d];
                        a1 += x * W1[d * sH + j];
                        a3 += x * W3[d * sH + j];
                    }
                    h1s[i] = a1;
                    h3s[i] = a3;
                    us[i] = silu_f(a1) * a3;
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float g = -vs[i];
                    if (a.loss == E2TTT_LOSS_MSE) {
                        float acc = 0.f;
                        #pragma unroll 4
                        for (int j = 0; j < Hd; ++j) acc += us[t * Hd + j] * W2s[j * sD + r];
                        g = acc - vs[i];
                    }
                    dys[i] = g;
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float du = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) du += dys[t * D + r] * W2s[j * sD + r];
                    const float x1 = h1s[i], x3 = h3s[i];
                    h1s[i] = du * x3 * dsilu_f(x1);  // dh1
                    h3s[i] = du * silu_f(x1);        // dh3
                }
                __syncthreads();
                const int64_t n1 = (int64_t)D * Hd;
                for (int64_t p = tid; p < P; p += NT) {
                    float gm = 0.f, gw = 0.f;
                    if (p < 2 * n1) {
                        const float* fac = p < n1 ? h1s : h3s;
                        const int64_t pp = p < n1 ? p : p - n1;
                        const int d = (int)(pp / Hd), j = (int)(pp % Hd);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const float g = xs[t * D + d] * fac[t * Hd + j];
                            gm += cms[t] * g;
                            gw += cws[t] * g;
                        }
                    } else {
                        const int j = (int)((p - 2 * n1) / D), r = (int)((p - 2 * n1) % D);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const float g = us[t * Hd + j] * dys[t * D + r];
                            gm += cms[t] * g;
                            gw += cws[t] * g;
                        }
                    }
                    GM[p] += gm;
                    GW[p] += gw;
                }
            }
            __syncthreads();
        }

        // ---- 4. state transition with the chunk-start momentum
        const float* sc = a.scal + (bh * a.nc + c) * 4;
        const float A = sc[0], Bb = sc[1], gamma = sc[2];
        for (int64_t p = tid; p < P; p += NT) {
            const float w = W[p], m = M ? M[p] : 0.f;
            W[p] = A * w - gamma * m - GW[p];
            if (M) M[p] = Bb * m + GM[p];
            GM[p] = 0.f;
            GW[p] = 0.f;
        }
        __syncthreads();
    }
}

template <int KIND, typename TIO, bool WLDS>
hipError_t launch_one(const e2ttt_desc& d, const GenericArgs& a, size_t shmem, hipStream_t s) {
    const void* f = (const void*)generic_kernel<KIND, TIO, WLDS>;
    if (shmem > 64 * 1024 && hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((generic_kernel<KIND, TIO, WLDS>), dim3((unsigned)(d.B * d.H)), dim3(NT), shmem, s, a);
    return hipGetLastError();
}

template <int KIND>
hipError_t launch_kind(const e2ttt_desc& d, const GenericArgs& a, size_t shmem, hipStream_t s) {
    if (d.io_dtype == E2TTT_BF16)
        return a.wlds ? launch_one<KIND, __bf16, true>(d, a, shmem, s) : launch_one<KIND, __bf16, false>(d, a, shmem, s);
    return a.wlds ? launch_one<KIND, float, true>(d, a, shmem, s) : launch_one<KIND, float, false>(d, a, shmem, s);
}

// LDS the portable kernels may use per workgroup (of gfx950's 160 KB)
constexpr size_t kLdsBudget = 144 * 1024;

}  // namespace

int generic_token_block(const e2ttt_desc& d) {
    const int64_t Hd = d.kind == E2TTT_LINEAR ? 0 : d.Hd;
    for (int tb = 16; tb >= 1; tb >>= 1)
        if ((3 * d.D + 3 * Hd + 2) * tb * 4 <= 64 * 1024) return tb;
    return 1;
}

hipError_t launch_generic(const e2ttt_desc& d, const void* q, const void* k, const void* v, const float* cM,
                          const float* cW, int64_t ldc, const float* scal, const float* W0, const float* M0, void* out,
                          float* W_end, float* M_end, float* gacc, hipStream_t s, float* save) {
    GenericArgs a;
    a.T = d.T;
    a.D = d.D;
    a.Hd = d.kind == E2TTT_LINEAR ? 0 : d.Hd;
    a.C = d.chunk;
    a.nc = (d.T + d.chunk - 1) / d.chunk;
    a.ldc = ldc;
    a.P = e2ttt_param_count(&d);
    a.loss = d.loss;
    a.TB = generic_token_block(d);
    a.nomom = (d.flags & E2TTT_FLAG_NO_MOMENTUM) ? 1 : 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.cM = cM;
    a.cW = cW;
    a.scal = scal;
    a.W0 = W0;
    a.M0 = M0;
    a.out = out;
    a.W = W_end;
    a.M = M_end;
    a.gacc = gacc;
    a.save = save;
    size_t shmem = (size_t)(3 * a.D + 3 * a.Hd + 2) * a.TB * sizeof(float);
    // the weights with every row padded by one float
    const int64_t Dd = a.D, H = a.Hd;
    const int64_t Ppad = d.kind == E2TTT_LINEAR ? Dd * (Dd + 1)
                         : d.kind == E2TTT_MLP  ? H * (Dd + 1) + Dd * (H + 1)
                                                : 2 * Dd * (H + 1) + H * (Dd + 1);
    a.wlds = shmem + (size_t)Ppad * sizeof(float) <= kLdsBudget ? 1 : 0;
    if (a.wlds) shmem += (size_t)Ppad * sizeof(float);
    switch (d.kind) {
        case E2TTT_LINEAR: return launch_kind<E2TTT_LINEAR>(d, a, shmem, s);
        case E2TTT_MLP: return launch_kind<E2TTT_MLP>(d, a, shmem, s);
        default: return launch_kind<E2TTT_SWIGLU>(d, a, shmem, s);
    }
}

}  // namespace e2ttt

// e2ttt_logscan: the two scalar kernels of the E2-TTT closed form.
//
// "Rethinking Expressivity and Efficiency in Test-Time Training", atlas
// summary "Approach" (two scalar kernels -- momentum and weight -- evaluated
// with log-space cumulative sums) and arxivlens "Results" (log-space suffix
// and ratio sums are the closed form's only overhead).
//
// For one chunk of tokens i = 0..C-1 with gates alpha_i, beta_i:
//   Sa_i = sum_{s>i} log alpha_s,  Sb_i = sum_{s>i} log beta_s   (suffix sums)
//   m_i  = exp(Sb_i)                                (momentum kernel)
//   w_i  = sum_{tau>=i} exp(Sa_tau) * prod_{s=i+1..tau} beta_s   (weight kernel)
// The weight kernel obeys the reverse recurrence w_i = a_i + beta_{i+1} w_{i+1}
// (w_{C-1} = 1), which in log space is lw_i = Sa_i (+) (log beta_{i+1} + lw_{i+1})
// with (+) = logaddexp.  Each step is the map z -> x (+) (y + z); maps compose
// as (x1, y1) o (x2, y2) = (x1 (+) (y1 + x2), y1 + y2), so the recurrence is a
// reverse scan.  Every value stays <= log C, and -inf (alpha = 0 or beta = 0)
// passes through without NaN because (+) maps (-inf, -inf) to -inf.  The
// "ratio" form exp(Sb_i) * sum exp(Sa - Sb) is avoided: it overflows fp32 once
// sum log(alpha/beta) exceeds ~88, which chunks of 1024 tokens reach.
//
// Mapping: one 64-lane wavefront per chunk, 4 chunks per 256-thread block.
// Lane l owns the contiguous tokens [l*npl, (l+1)*npl); lane-local sequential
// passes plus wavefront shuffle scans combine them.
#include <math.h>

#include "e2ttt_internal.h"

namespace e2ttt {
namespace {

__device__ __forceinline__ float log_add_exp(float a, float b) {
    const float m = fmaxf(a, b);
    if (m == -INFINITY) return -INFINITY;
    return m + log1pf(expf(fminf(a, b) - m));
}

__global__ __launch_bounds__(256) void logscan_kernel(int64_t total_chunks, int64_t nc, int64_t T, int C,
                                                      int npl, const float* __restrict__ eta,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, float* __restrict__ cM,
                                                      float* __restrict__ cW, float* __restrict__ scal) {
    const int lane = threadIdx.x & 63;
    const int64_t gc = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gc >= total_chunks) return;  // uniform per wavefront
    const int64_t bh = gc / nc, c = gc % nc;
    const size_t base = (size_t)bh * T + (size_t)c * C;
    const float* al = alpha + base;
    const float* be = beta + base;
    const float* et = eta + base;
    const int lo = lane * npl;
    const int hi = min(lo + npl, C);

    // pass 1: lane sums of log alpha, log beta
    float sa = 0.f, sb = 0.f;
    for (int t = lo; t < hi; ++t) {
        sa += logf(al[t]);
        sb += logf(be[t]);
    }
    // inclusive reverse scan over lanes: ra = sum over lanes >= lane
    float ra = sa, rb = sb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float oa = __shfl_down(ra, off, 64);
        const float ob = __shfl_down(rb, off, 64);
        if (lane + off < 64) {
            ra += oa;
            rb += ob;
        }
    }
    const float tot_a = __shfl(ra, 0, 64);
    const float tot_b = __shfl(rb, 0, 64);
    float base_a = __shfl_down(ra, 1, 64);  // sum over lanes > lane
    float base_b = __shfl_down(rb, 1, 64);
    if (lane == 63) base_a = base_b = 0.f;

    // pass 2: compose the lane's maps f_t(z) = Sa_t (+) (log beta_{t+1} + z), last token first
    float X = -INFINITY, Y = 0.f;  // identity map
    {
        float Sa = base_a;
        for (int t = hi - 1; t >= lo; --t) {
            const float y = (t + 1 < C) ? logf(be[t + 1]) : -INFINITY;
            X = log_add_exp(Sa, y + X);
            Y = y + Y;
            Sa += logf(al[t]);
        }
    }
    // inclusive reverse scan of the maps: R_lane = F_lane o F_lane+1 o ... o F_63
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float oX = __shfl_down(X, off, 64);
        const float oY = __shfl_down(Y, off, 64);
        if (lane + off < 64) {
            X = log_add_exp(X, Y + oX);
            Y = Y + oY;
        }
    }
    // lw at the first token of the next lane; the chunk's last map is constant,
    // so applying the right-hand composition to -inf gives its x component
    float z = __shfl_down(X, 1, 64);
    if (lane == 63) z = -INFINITY;

    // pass 3: per-token coefficients
    float Sa = base_a, Sb = base_b;
    for (int t = hi - 1; t >= lo; --t) {
        const float y = (t + 1 < C) ? logf(be[t + 1]) : -INFINITY;
        const float lw = log_add_exp(Sa, y + z);
        z = lw;
        const float e = et[t];
        cM[base + t] = expf(Sb) * e;
        cW[base + t] = expf(lw) * e;
        Sa += logf(al[t]);
        Sb += logf(be[t]);
        if (t == 0) {
            float* s = scal + gc * 4;
            s[0] = expf(tot_a);
            s[1] = expf(tot_b);
            s[2] = expf(logf(be[0]) + lw);  // gamma = beta_first * w_first
            s[3] = 0.f;
        }
    }
}

}  // namespace

hipError_t launch_logscan(int64_t BH, int64_t T, int64_t chunk, const float* eta, const float* alpha,
                          const float* beta, float* cM, float* cW, float* scal, hipStream_t s) {
    const int64_t nc = T / chunk;
    const int64_t total = BH * nc;
    if (total == 0) return hipSuccess;
    const int npl = (int)((chunk + 63) / 64);
    const int64_t blocks = (total + 3) / 4;
    hipLaunchKernelGGL(logscan_kernel, dim3((unsigned)blocks), dim3(256), 0, s, total, nc, T, (int)chunk, npl,
                       eta, alpha, beta, cM, cW, scal);
    return hipGetLastError();
}

}  // namespace e2ttt

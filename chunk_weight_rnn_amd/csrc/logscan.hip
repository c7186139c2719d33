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
// A ragged last chunk (T % C != 0) takes the same passes over its tokens.
//
// Mapping: chunks of up to 256 tokens take one 64-lane wavefront each, 4
// chunks per 256-thread block; chunks of up to 1024 tokens take the four
// wavefronts of a block, a quarter of the chunk each.  Lane l of a wavefront
// owns npl <= 4 contiguous tokens; lane-local sequential passes plus
// wavefront shuffle scans combine them, and the four wavefronts of a long
// chunk exchange their partial results through LDS.  The lane's gates stay
// in registers and the logs are base-2 hardware log / exp; longer chunks use
// a variant that re-reads its tokens and uses natural-log library functions.
//
// Variants (flags):
//   no momentum: W_t = alpha_t W_{t-1} - eta_t g_t, i.e. beta = 0 throughout:
//     m_i = [i = C-1], w_i = exp(Sa_i), Bb = gamma = 0 (beta is not read);
//   chunk average (the pages' chunk-averaged ablation, atlas summary
//     "Surprising findings"): m_i and w_i are replaced by their mean over the
//     chunk before the multiplication by eta_i; A, Bb, gamma are unchanged.
#include <math.h>

#include "e2ttt_internal.h"
#include "scan_wave.h"

namespace e2ttt {
namespace {

constexpr int MAXNPL = 4;  // tokens per lane: 4 waves per chunk take chunks up to 1024 tokens

// One wave per chunk (NW = 1, four chunks per block) or four (NW = 4, one
// chunk per block); the chunk's passes are scan::scan_chunk (scan_wave.h).
template <int NW, int MAXN>
__global__ __launch_bounds__(256) void logscan_kernel(int64_t total_chunks, int64_t nc, int64_t T, int C,
                                                      int npl, int nomom, int avg, const float* __restrict__ eta,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, float* __restrict__ cM,
                                                      float* __restrict__ cW, int64_t ldc,
                                                      float* __restrict__ scal) {
    __shared__ float xs[3][NW][2];  // per wave: (sum log2 alpha, sum log2 beta), map (X, Y), (sum m, sum w)
    const int lane = threadIdx.x & 63;
    const int w = NW == 1 ? 0 : (int)(threadIdx.x >> 6);
    const int64_t gc = NW == 1 ? (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6) : (int64_t)blockIdx.x;
    if (gc >= total_chunks) return;  // uniform per wavefront (NW = 1) or per block (NW = 4)
    scan::scan_chunk<NW, MAXN>(lane, w, gc / nc, gc % nc, nc, T, C, npl, nomom, avg, eta, alpha, beta, cM, cW, ldc,
                               scal, xs);
}

// Any chunk length (tokens per lane not bounded): the same three passes with
// the lane's tokens re-read from memory and natural-log libm functions.
__device__ __forceinline__ float log_add_exp(float a, float b) {
    const float m = fmaxf(a, b);
    if (m == -INFINITY) return -INFINITY;
    return m + log1pf(expf(fminf(a, b) - m));
}

__global__ __launch_bounds__(256) void logscan_kernel_any(int64_t total_chunks, int64_t nc, int64_t T, int C,
                                                      int npl, int nomom, int avg, const float* __restrict__ eta,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, float* __restrict__ cM,
                                                      float* __restrict__ cW, int64_t ldc,
                                                      float* __restrict__ scal) {
    const int lane = threadIdx.x & 63;
    const int64_t gc = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gc >= total_chunks) return;  // uniform per wavefront
    const int64_t bh = gc / nc, c = gc % nc;
    const size_t base = (size_t)bh * T + (size_t)c * C;     // inputs: rows of T tokens
    const size_t obase = (size_t)bh * ldc + (size_t)c * C;  // outputs: rows of ldc tokens
    if (c == nc - 1 && T + lane < ldc) {                    // zero padding after the sequence
        cM[(size_t)bh * ldc + T + lane] = 0.f;
        cW[(size_t)bh * ldc + T + lane] = 0.f;
    }
    C = (int)min((int64_t)C, T - c * (int64_t)C);  // this chunk's length (the last may be shorter)
    const float* al = alpha + base;
    const float* be = nomom ? nullptr : beta + base;
    auto logb = [&](int t) { return nomom ? -INFINITY : logf(be[t]); };
    const float* et = eta + base;
    const int lo = lane * npl;
    const int hi = min(lo + npl, C);

    // pass 1: lane sums of log alpha, log beta
    float sa = 0.f, sb = 0.f;
    for (int t = lo; t < hi; ++t) {
        sa += logf(al[t]);
        sb += logb(t);
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
            const float y = (t + 1 < C) ? logb(t + 1) : -INFINITY;
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

    // pass 3: per-token coefficients (with the chunk average: their sums)
    float Sa = base_a, Sb = base_b, sum_m = 0.f, sum_w = 0.f;
    for (int t = hi - 1; t >= lo; --t) {
        const float y = (t + 1 < C) ? logb(t + 1) : -INFINITY;
        const float lw = log_add_exp(Sa, y + z);
        z = lw;
        const float e = et[t];
        const float mt = expf(Sb), wt = expf(lw);
        sum_m += mt;
        sum_w += wt;
        if (!avg) {
            cM[obase + t] = mt * e;
            cW[obase + t] = wt * e;
        }
        Sa += logf(al[t]);
        Sb += logb(t);
        if (t == 0) {
            float* s = scal + gc * 4;
            s[0] = expf(tot_a);
            s[1] = expf(tot_b);
            s[2] = expf(logb(0) + lw);  // gamma = beta_first * w_first
            s[3] = 0.f;
        }
    }
    if (avg) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sum_m += __shfl_xor(sum_m, off, 64);
            sum_w += __shfl_xor(sum_w, off, 64);
        }
        const float mm = sum_m / (float)C, mw = sum_w / (float)C;
        for (int t = lo; t < hi; ++t) {
            cM[obase + t] = mm * et[t];
            cW[obase + t] = mw * et[t];
        }
    }
}

}  // namespace

hipError_t launch_logscan(int64_t BH, int64_t T, int64_t chunk, int flags, const float* eta, const float* alpha,
                          const float* beta, float* cM, float* cW, int64_t ldc, float* scal, hipStream_t s) {
    const int nomom = (flags & E2TTT_FLAG_NO_MOMENTUM) ? 1 : 0;
    const int avg = (flags & E2TTT_FLAG_CHUNK_AVG) ? 1 : 0;
    const int64_t nc = (T + chunk - 1) / chunk;  // the last chunk may be shorter
    const int64_t total = BH * nc;
    if (total == 0) return hipSuccess;
    const int npl = (int)((chunk + 63) / 64);
    const int64_t blocks = (total + 3) / 4;
    if (npl <= 4)  // one wave per chunk, four chunks per block
        hipLaunchKernelGGL((logscan_kernel<1, 4>), dim3((unsigned)blocks), dim3(256), 0, s, total, nc, T, (int)chunk,
                           npl, nomom, avg, eta, alpha, beta, cM, cW, ldc, scal);
    else if (npl <= 4 * MAXNPL)  // four waves per chunk
        hipLaunchKernelGGL((logscan_kernel<4, MAXNPL>), dim3((unsigned)total), dim3(256), 0, s, total, nc, T,
                           (int)chunk, (npl + 3) / 4, nomom, avg, eta, alpha, beta, cM, cW, ldc, scal);
    else
        hipLaunchKernelGGL(logscan_kernel_any, dim3((unsigned)blocks), dim3(256), 0, s, total, nc, T, (int)chunk,
                           npl, nomom, avg, eta, alpha, beta, cM, cW, ldc, scal);
    return hipGetLastError();
}

}  // namespace e2ttt

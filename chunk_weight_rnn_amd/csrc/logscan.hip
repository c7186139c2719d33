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

namespace e2ttt {
namespace {

// Everything below works in base-2 logs with the hardware log2 / exp2
// (v_log_f32 / v_exp_f32): l = log2(x), so products become sums and
// logaddexp becomes m + log2(1 + 2^(min - m)).
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_add_exp2(float a, float b) {
    const float m = fmaxf(a, b);
    if (m == -INFINITY) return -INFINITY;
    return m + lg2(1.f + ex2(fminf(a, b) - m));
}

constexpr int MAXNPL = 4;  // tokens per lane: 4 waves per chunk take chunks up to 1024 tokens

// NW wavefronts per chunk: wave w takes the chunk's tokens [w L, (w + 1) L),
// L = 64 npl, npl <= MAXN tokens per lane.  With NW = 1 a block of four waves
// takes four chunks; with NW = 4 one chunk, and the waves exchange through
// LDS what the later waves contribute to each pass: the sums of log alpha
// and log beta (pass 1), the composition of the later waves' maps (pass 2)
// and, for chunk averages, the sums of m and w.  (One wave per chunk of 1024
// tokens left three quarters of the chip idle and each wave's chain 16
// tokens long.)
template <int NW, int MAXN>
__global__ __launch_bounds__(256) void logscan_kernel(int64_t total_chunks, int64_t nc, int64_t T, int C,
                                                      int npl, int nomom, int avg, const float* __restrict__ eta,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, float* __restrict__ cM,
                                                      float* __restrict__ cW, int64_t ldc,
                                                      float* __restrict__ scal) {
    static_assert(NW == 1 || NW == 4, "waves per chunk");
    __shared__ float xs[3][NW][2];  // per wave: (sum log2 alpha, sum log2 beta), map (X, Y), (sum m, sum w)
    const int lane = threadIdx.x & 63;
    const int w = NW == 1 ? 0 : (int)(threadIdx.x >> 6);
    const int64_t gc = NW == 1 ? (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6) : (int64_t)blockIdx.x;
    if (gc >= total_chunks) return;  // uniform per wavefront (NW = 1) or per block (NW = 4)
    const int64_t bh = gc / nc, c = gc % nc;
    const size_t base = (size_t)bh * T + (size_t)c * C;     // inputs: rows of T tokens
    const size_t obase = (size_t)bh * ldc + (size_t)c * C;  // outputs: rows of ldc tokens
    if (w == 0 && c == nc - 1 && T + lane < ldc) {          // zero padding after the sequence
        cM[(size_t)bh * ldc + T + lane] = 0.f;
        cW[(size_t)bh * ldc + T + lane] = 0.f;
    }
    C = (int)min((int64_t)C, T - c * (int64_t)C);  // this chunk's length (the last may be shorter)
    const int L = 64 * npl;                         // tokens per wave
    const int lo = w * L + lane * npl;              // the lane's first token

    // the lane's tokens: log2 alpha, log2 beta (beta of the next token too), eta
    float la[MAXN], lb[MAXN], lbn[MAXN], et[MAXN];
#pragma unroll
    for (int u = 0; u < MAXN; ++u) {
        if (u < npl && lo + u < C) {
            la[u] = lg2(alpha[base + lo + u]);
            lb[u] = nomom ? -INFINITY : lg2(beta[base + lo + u]);
            et[u] = eta[base + lo + u];
        } else {
            la[u] = 0.f;
            lb[u] = 0.f;
            et[u] = 0.f;
        }
    }
    // log2 beta of token t+1: the first token of the next lane for the last
    // one, of the next wave's first lane (read directly) for lane 63
    float lb_next_lane = __shfl_down(lb[0], 1, 64);
    if (lane == 63) {
        const int t1 = (w + 1) * L;
        lb_next_lane = (NW > 1 && t1 < C && !nomom) ? lg2(beta[base + t1]) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < MAXN; ++u) {
        if (u + 1 < npl) lbn[u] = lb[u + 1];
        else lbn[u] = lb_next_lane;
        if (lo + u + 1 >= C) lbn[u] = -INFINITY;  // the chunk's last token has no successor
        else if (nomom) lbn[u] = -INFINITY;
    }

    // pass 1: lane sums, then the inclusive reverse scan over lanes (and waves)
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int u = 0; u < MAXN; ++u) {
        sa += la[u];
        sb += lb[u];
    }
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
    float tot_a = __shfl(ra, 0, 64);
    float tot_b = __shfl(rb, 0, 64);
    float base_a = __shfl_down(ra, 1, 64);  // sum over lanes > lane
    float base_b = __shfl_down(rb, 1, 64);
    if (lane == 63) base_a = base_b = 0.f;
    if constexpr (NW > 1) {
        if (lane == 0) {
            xs[0][w][0] = tot_a;
            xs[0][w][1] = tot_b;
        }
        __syncthreads();
        float la_later = 0.f, lb_later = 0.f;
        tot_a = tot_b = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            tot_a += xs[0][v][0];
            tot_b += xs[0][v][1];
            if (v > w) {
                la_later += xs[0][v][0];
                lb_later += xs[0][v][1];
            }
        }
        base_a += la_later;
        base_b += lb_later;
    }

    // pass 2: compose the lane's maps f_t(z) = Sa_t (+) (log2 beta_{t+1} + z), last token first
    float X = -INFINITY, Y = 0.f;  // identity map
    {
        float Sa = base_a;
#pragma unroll
        for (int u = MAXN - 1; u >= 0; --u) {
            if (u < npl && lo + u < C) {
                X = log2_add_exp2(Sa, lbn[u] + X);
                Y = lbn[u] + Y;
                Sa += la[u];
            }
        }
    }
    // inclusive reverse scan of the maps: R_lane = F_lane o F_lane+1 o ... o F_63
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float oX = __shfl_down(X, off, 64);
        const float oY = __shfl_down(Y, off, 64);
        if (lane + off < 64) {
            X = log2_add_exp2(X, Y + oX);
            Y = Y + oY;
        }
    }
    // lw at the first token of the next lane: the composition of the later
    // lanes R_lane+1 and of the later waves G, applied to -inf (the chunk's
    // last map is constant); G(-inf) is G's x component
    float xg = -INFINITY;
    if constexpr (NW > 1) {
        if (lane == 0) {
            xs[1][w][0] = X;
            xs[1][w][1] = Y;
        }
        __syncthreads();
        float gy = 0.f;  // G = W_w+1 o ... o W_NW-1, folded from the right
#pragma unroll
        for (int v = NW - 1; v > 0; --v) {
            if (v > w) {
                xg = log2_add_exp2(xs[1][v][0], xs[1][v][1] + xg);
                gy = xs[1][v][1] + gy;
            }
        }
        (void)gy;
    }
    float nX = __shfl_down(X, 1, 64), nY = __shfl_down(Y, 1, 64);
    if (lane == 63) {
        nX = -INFINITY;
        nY = 0.f;
    }
    float z = log2_add_exp2(nX, nY + xg);

    // pass 3: per-token kernels m, w
    float mv[MAXN], wv[MAXN];
    float Sa = base_a, Sb = base_b, sum_m = 0.f, sum_w = 0.f;
#pragma unroll
    for (int u = MAXN - 1; u >= 0; --u) {
        mv[u] = wv[u] = 0.f;
        if (u < npl && lo + u < C) {
            const float lw = log2_add_exp2(Sa, lbn[u] + z);
            z = lw;
            mv[u] = ex2(Sb);
            wv[u] = ex2(lw);
            sum_m += mv[u];
            sum_w += wv[u];
            Sa += la[u];
            Sb += lb[u];
            if (lo + u == 0) {
                float* sp = scal + gc * 4;
                sp[0] = ex2(tot_a);
                sp[1] = ex2(tot_b);
                sp[2] = ex2(lb[0] + lw);  // gamma = beta_first * w_first
                sp[3] = 0.f;
            }
        }
    }
    if (avg) {  // chunk means of m and w for every token
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sum_m += __shfl_xor(sum_m, off, 64);
            sum_w += __shfl_xor(sum_w, off, 64);
        }
        if constexpr (NW > 1) {
            if (lane == 0) {
                xs[2][w][0] = sum_m;
                xs[2][w][1] = sum_w;
            }
            __syncthreads();
            sum_m = sum_w = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                sum_m += xs[2][v][0];
                sum_w += xs[2][v][1];
            }
        }
#pragma unroll
        for (int u = 0; u < MAXN; ++u) {
            mv[u] = sum_m / (float)C;
            wv[u] = sum_w / (float)C;
        }
    }
    // coefficients cM = m eta, cW = w eta
#pragma unroll
    for (int u = 0; u < MAXN; ++u) {
        if (u < npl && lo + u < C) {
            cM[obase + lo + u] = mv[u] * et[u];
            cW[obase + lo + u] = wv[u] * et[u];
        }
    }
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

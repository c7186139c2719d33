// The scalar kernels of one chunk, computed by one wavefront (or by NW
// wavefronts of a workgroup that share the chunk): the body of the scan
// kernel in logscan.hip, also run inside the SwiGLU chunk loop's prologue.
// The method, the log-space reverse scan and the variants are described in
// logscan.hip.
#pragma once

#include <math.h>

#include "e2ttt_internal.h"

namespace e2ttt {
namespace scan {

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

// NW wavefronts per chunk: wave w takes the chunk's tokens [w L, (w + 1) L),
// L = 64 npl, npl <= MAXN tokens per lane.  With NW = 1 a block of four waves
// takes four chunks; with NW = 4 one chunk, and the waves exchange through
// LDS what the later waves contribute to each pass: the sums of log alpha
// and log beta (pass 1), the composition of the later waves' maps (pass 2)
// and, for chunk averages, the sums of m and w.  (One wave per chunk of 1024
// tokens left three quarters of the chip idle and each wave's chain 16
// tokens long.)
//
// The gates of the lane's tokens of chunk c of row bh (alpha, beta, eta;
// 1 / 1 / 0 past the chunk), loaded apart from the passes so that a caller
// can issue the loads early.
template <int MAXN>
struct Gates {
    float a[MAXN], b[MAXN], e[MAXN];
};

template <int NW, int MAXN>
__device__ __forceinline__ void load_gates(int lane, int w, int64_t bh, int64_t c, int64_t T, int C, int npl,
                                           int nomom, const float* __restrict__ eta, const float* __restrict__ alpha,
                                           const float* __restrict__ beta, Gates<MAXN>& g) {
    const size_t base = (size_t)bh * T + (size_t)c * C;
    C = (int)min((int64_t)C, T - c * (int64_t)C);
    const int lo = w * 64 * npl + lane * npl;
#pragma unroll
    for (int u = 0; u < MAXN; ++u) {
        const bool in = u < npl && lo + u < C;
        g.a[u] = in ? alpha[base + lo + u] : 1.f;
        g.b[u] = in && !nomom ? beta[base + lo + u] : 1.f;
        g.e[u] = in ? eta[base + lo + u] : 0.f;
    }
}

// Chunk c of row bh (gc = bh nc + c its index in scal) from its loaded
// gates; xs: the workgroup's exchange area, used only with NW > 1.
template <int NW, int MAXN>
__device__ __forceinline__ void scan_chunk_from(int lane, int w, int64_t bh, int64_t c, int64_t nc, int64_t T, int C,
                                                int npl, int nomom, int avg, const Gates<MAXN>& gt,
                                                const float* __restrict__ beta, float* __restrict__ cM,
                                                float* __restrict__ cW, int64_t ldc, float* __restrict__ scal,
                                                float (*xs)[NW][2]) {
    static_assert(NW == 1 || NW == 4, "waves per chunk");
    const int64_t gc = bh * nc + c;
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
            la[u] = lg2(gt.a[u]);
            lb[u] = nomom ? -INFINITY : lg2(gt.b[u]);
            et[u] = gt.e[u];
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


// Both steps in turn.
template <int NW, int MAXN>
__device__ __forceinline__ void scan_chunk(int lane, int w, int64_t bh, int64_t c, int64_t nc, int64_t T, int C,
                                           int npl, int nomom, int avg, const float* __restrict__ eta,
                                           const float* __restrict__ alpha, const float* __restrict__ beta,
                                           float* __restrict__ cM, float* __restrict__ cW, int64_t ldc,
                                           float* __restrict__ scal, float (*xs)[NW][2]) {
    Gates<MAXN> g;
    load_gates<NW, MAXN>(lane, w, bh, c, T, C, npl, nomom, eta, alpha, beta, g);
    scan_chunk_from<NW, MAXN>(lane, w, bh, c, nc, T, C, npl, nomom, avg, g, beta, cM, cW, ldc, scal, xs);
}

}  // namespace scan
}  // namespace e2ttt

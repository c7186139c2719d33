// Portable fp32 backward of the chunk update: every fast-weight kind and loss
// (the shapes of the portable forward).  It is the vector-Jacobian product of
// the chunk update of "Rethinking Expressivity and Efficiency in Test-Time
// Training" (abstract; atlas summary "Approach"), the same derivative as the
// SwiGLU MFMA backward, written for all three fast weights.
//
// Per (b, h) and chunk c, from the last to the first, with the chunk-start
// state W_c, M_c (saved by the forward recompute) and the cotangents lW, lM of
// the chunk end.  For token t with coefficients cM, cW let
// Lam = cM lM - cW lW; the objective's chunk terms are
//   J = sum_t <dout_t, f_{W_c}(q_t)> + sum_t <Lam_t, g_t(W_c)>
// and the update is
//   dW_c = A lW + dJ/dW,  dM_c = Bb lM - gamma lW,
//   dcM_t = <lM, g_t>,  dcW_t = -<lW, g_t>,
//   dA = <lW, W_c>,  dBb = <lM, M_c>,  dgamma = -<lW, M_c>,
// with dq_t, dk_t, dv_t = dJ/dq_t, dJ/dk_t, dJ/dv_t.  <Lam, g_t> is the
// derivative of token t's loss along Lam, so dJ/d(W, k, v) holds the second
// derivatives of the fast-weight loss:
//
// linear (y = W k, dy = y - v or -v, g = dy k^T), s = Lam k:
//   <Lam, g> = s . dy;  dk = Lam^T dy [+ W^T s];  dv = -s;  dW += [s k^T]
// mlp (z = W1 k, a = silu(z), y = W2 a, e = W2^T dy, dz = e silu'(z),
// g = (dz k^T, dy a^T)), p1 = Lam1 k, p2 = Lam2 a:
//   <Lam, g> = dy . p2 + dz . p1;  Gy = p2 + W2 (silu'(z) p1);
//   Ja = Lam2^T dy [+ W2^T Gy];  Jz = e p1 silu''(z) + Ja silu'(z);
//   dk = Lam1^T dz + W1^T Jz;  dv = -Gy;
//   dW1 += Jz k^T;  dW2 += dy (silu'(z) p1)^T [+ Gy a^T]
// swiglu (row vectors; h1 = k W1, h3 = k W3, u = silu(h1) h3, y = u W2,
// du = dy W2^T, dh1 = du h3 silu'(h1), dh3 = du silu(h1),
// g = (k^T dh1, k^T dh3, u^T dy)), P1 = k Lam1, P3 = k Lam3, Q2 = Lam2 dy^T:
//   <Lam, g> = P1 . dh1 + P3 . dh3 + u . Q2;  E = P1 h3 silu' + P3 silu;
//   Gy = u Lam2 + E W2;  Ju = Q2 [+ Gy W2^T];
//   Jh1 = P1 du h3 silu'' + P3 du silu' + Ju h3 silu';  Jh3 = P1 du silu' + Ju silu;
//   dk = Jh1 W1^T + Jh3 W3^T + dh1 Lam1^T + dh3 Lam3^T;  dv = -Gy;
//   dW1 += k^T Jh1;  dW3 += k^T Jh3;  dW2 += E^T dy [+ u^T Gy]
// ([...] only for the MSE loss) and the output path, the gradient of
// <dout, f_W(q)>, as in any MLP backward.
//
// One 1024-thread workgroup per (b, h); tokens in blocks through LDS; every
// contraction is a plain fp32 loop.  The cotangents are updated in place in
// the dW0 / dM0 buffers; dJ/dW accumulates in a per-head workspace slice.
#include <math.h>

#include "e2ttt_internal.h"

namespace e2ttt {
namespace {

constexpr int NT = 1024;  // 16 wavefronts: the fp32 loops are latency-bound

struct GBwdArgs {
    int64_t T, D, Hd, C, nc, P, ldc;
    int loss, TB, mom;
    const void *q, *k, *v, *dout;
    const float *cM, *cW, *scal;
    const float* save;        // [BH][nc][2][P] chunk-start W, M
    const float *dW_end, *dM_end;
    float *lamW, *lamM;       // [BH][P] working cotangents (the dW0 / dM0 outputs)
    float* dacc;              // [BH][P] dJ/dW of the current chunk
    void *dq, *dk, *dv;
    float *dcM, *dcW;         // [BH][ldc]
    float* dpart;             // [BH][nc][4]
};

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const __bf16* p, int64_t i) { return (float)p[i]; }
__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(__bf16* p, int64_t i, float x) { p[i] = (__bf16)x; }

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigm(x); }
__device__ __forceinline__ float dsilu_f(float x) {
    const float s = sigm(x);
    return s * (1.f + x * (1.f - s));
}
__device__ __forceinline__ float d2silu_f(float x) {
    const float s = sigm(x);
    return s * (1.f - s) * (2.f + x * (1.f - 2.f * s));
}

// sum over the workgroup of three values (result in every thread)
__device__ void block_sum3(float& a, float& b, float& c, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
        c += __shfl_xor(c, o);
    }
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) {
        red[3 * w] = a;
        red[3 * w + 1] = b;
        red[3 * w + 2] = c;
    }
    __syncthreads();
    a = b = c = 0.f;
    for (int i = 0; i < NT / 64; ++i) {
        a += red[3 * i];
        b += red[3 * i + 1];
        c += red[3 * i + 2];
    }
    __syncthreads();
}

// floats of LDS per token for each kind: D-sized and Hd-sized rows
__host__ __device__ constexpr int rows_d(int kind) { return kind == E2TTT_LINEAR ? 8 : kind == E2TTT_MLP ? 8 : 6; }
__host__ __device__ constexpr int rows_h(int kind) { return kind == E2TTT_LINEAR ? 0 : kind == E2TTT_MLP ? 7 : 13; }

// Packed parameter index -> index in the row-padded copy, and its size.
template <int KIND>
__device__ __forceinline__ int64_t padded_index(int64_t p, int64_t D, int64_t Hd) {
    if (KIND == E2TTT_LINEAR) return (p / D) * (D + 1) + p % D;
    if (KIND == E2TTT_MLP) {
        const int64_t n1 = Hd * D;
        return p < n1 ? (p / D) * (D + 1) + p % D : Hd * (D + 1) + ((p - n1) / Hd) * (Hd + 1) + (p - n1) % Hd;
    }
    const int64_t n1 = D * Hd;
    return p < 2 * n1 ? (p / Hd) * (Hd + 1) + p % Hd : 2 * D * (Hd + 1) + ((p - 2 * n1) / D) * (D + 1) + (p - 2 * n1) % D;
}
template <int KIND>
__host__ __device__ constexpr int64_t padded_count(int64_t D, int64_t Hd) {
    return KIND == E2TTT_LINEAR ? D * (D + 1) : KIND == E2TTT_MLP ? Hd * (D + 1) + D * (Hd + 1) : 2 * D * (Hd + 1) + Hd * (D + 1);
}

// CACHE: 0 nothing in LDS, 1 W_c, 2 W_c and the cotangents lW, lM (copied per
// chunk after the token rows, rows padded); the rest is read from global
// memory.
template <int KIND, typename TIO, int CACHE>
__global__ __launch_bounds__(NT) void generic_bwd_kernel(GBwdArgs a) {
    extern __shared__ float smem[];
    __shared__ float red[3 * NT / 64];
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int D = (int)a.D, Hd = (int)a.Hd, TB = a.TB;
    const int64_t P = a.P;
    const bool mse = a.loss == E2TTT_LOSS_MSE;
    const bool mom = a.mom != 0;
    // token-block rows: D-sized x rows_d, Hd-sized x rows_h, then cM, cW
    float* rd = smem;
    float* rh = smem + rows_d(KIND) * TB * D;
    auto RD = [&](int i) { return rd + i * TB * D; };
    auto RH = [&](int i) { return rh + i * TB * Hd; };
    float* cms = rh + rows_h(KIND) * TB * Hd;
    float* cws = cms + TB;
    float* cache = cws + TB;  // W_c (CACHE >= 1), lW and lM (CACHE >= 2), rows padded
    // Row strides of the weights (w*) and cotangents (l*): the LDS copies pad
    // every row by one float, so that lanes reading one column of consecutive
    // rows hit distinct banks.
    const int64_t wD = D + (CACHE > 0), wH = Hd + (CACHE > 0);
    const int64_t lD = D + (CACHE > 1), lH = Hd + (CACHE > 1);
    const int64_t PP = padded_count<KIND>(D, Hd);

    const TIO* q = (const TIO*)a.q + bh * a.T * D;
    const TIO* k = (const TIO*)a.k + bh * a.T * D;
    const TIO* v = (const TIO*)a.v + bh * a.T * D;
    const TIO* dout = (const TIO*)a.dout + bh * a.T * D;
    TIO* dq = (TIO*)a.dq + bh * a.T * D;
    TIO* dk = (TIO*)a.dk + bh * a.T * D;
    TIO* dv = (TIO*)a.dv + bh * a.T * D;
    float* LW = a.lamW + bh * P;
    float* LM = mom ? a.lamM + bh * P : nullptr;
    float* DJ = a.dacc + bh * P;

    for (int64_t p = tid; p < P; p += NT) {
        LW[p] = a.dW_end[bh * P + p];
        if (mom) LM[p] = a.dM_end[bh * P + p];
    }
    __syncthreads();

    for (int64_t c = a.nc - 1; c >= 0; --c) {
        const float* Wc = a.save + (bh * a.nc + c) * 2 * P;
        const float* Mc = Wc + P;
        const int64_t t0 = c * a.C;
        const int64_t Cc = min(a.C, a.T - t0);
        {
            float sA = 0.f, sB = 0.f, sG = 0.f;
            for (int64_t p = tid; p < P; p += NT) {
                DJ[p] = 0.f;
                const float lw = LW[p];
                sA += lw * Wc[p];
                if (mom) {
                    sB += LM[p] * Mc[p];
                    sG -= lw * Mc[p];
                }
            }
            block_sum3(sA, sB, sG, red);
            if (tid == 0) {
                float* dp = a.dpart + (bh * a.nc + c) * 4;
                dp[0] = sA;
                dp[1] = sB;
                dp[2] = sG;
            }
        }
        if (CACHE > 0) {  // packed index -> padded (row, column), as in the portable forward
            for (int64_t p = tid; p < P; p += NT) {
                const int64_t o = padded_index<KIND>(p, D, Hd);
                cache[o] = Wc[p];
                if (CACHE > 1) cache[PP + o] = LW[p];
                if (CACHE > 1 && mom) cache[2 * PP + o] = LM[p];
            }
            __syncthreads();
        }
        const float* Wr = CACHE > 0 ? cache : Wc;
        const float* LWr = CACHE > 1 ? cache + PP : LW;
        const float* LMr = CACHE > 1 ? cache + 2 * PP : LM;
        for (int64_t b0 = 0; b0 < Cc; b0 += TB) {
            const int nt = (int)min((int64_t)TB, Cc - b0);
            const int64_t tb = t0 + b0;  // first token of the block
            float* xk = RD(0);
            float* xv = RD(1);
            float* xq = RD(2);
            float* xo = RD(3);
            for (int i = tid; i < nt * D; i += NT) {
                xk[i] = ld(k, tb * D + i);
                xv[i] = ld(v, tb * D + i);
                xq[i] = ld(q, tb * D + i);
                xo[i] = ld(dout, tb * D + i);
            }
            for (int i = tid; i < nt; i += NT) {
                cms[i] = mom ? a.cM[bh * a.ldc + tb + i] : 0.f;
                cws[i] = a.cW[bh * a.ldc + tb + i];
            }
            __syncthreads();

            if (KIND == E2TTT_LINEAR) {
                // W [D][D] (y_r = sum_d W[r][d] k_d)
                float* dy = RD(4);
                float* sM = RD(5);
                float* sW = RD(6);
                float* s = RD(7);
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float y = 0.f, pm = 0.f, pw = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) {
                        const float x = xk[t * D + d];
                        y += Wr[r * wD + d] * x;
                        pw += LWr[r * lD + d] * x;
                        if (mom) pm += LMr[r * lD + d] * x;
                    }
                    dy[i] = mse ? y - xv[i] : -xv[i];
                    sM[i] = pm;
                    sW[i] = pw;
                }
                __syncthreads();
                for (int t = tid; t < nt; t += NT) {
                    float gm = 0.f, gw = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) {
                        gm += sM[t * D + r] * dy[t * D + r];
                        gw += sW[t * D + r] * dy[t * D + r];
                    }
                    if (mom) a.dcM[bh * a.ldc + tb + t] = gm;
                    a.dcW[bh * a.ldc + tb + t] = -gw;
                }
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D;
                    s[i] = cms[t] * sM[i] - cws[t] * sW[i];
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, d = i % D;
                    float gk = 0.f, gq = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) {
                        const float w = Wr[r * wD + d];
                        const float lam = cms[t] * (mom ? LMr[r * lD + d] : 0.f) - cws[t] * LWr[r * lD + d];
                        gk += lam * dy[t * D + r] + (mse ? w * s[t * D + r] : 0.f);
                        gq += w * xo[t * D + r];
                    }
                    st(dk, tb * D + i, gk);
                    st(dv, tb * D + i, -s[i]);
                    st(dq, tb * D + i, gq);
                }
                for (int64_t p = tid; p < P; p += NT) {
                    const int r = (int)(p / D), d = (int)(p % D);
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int t = 0; t < nt; ++t)
                        acc += (mse ? s[t * D + r] * xk[t * D + d] : 0.f) + xo[t * D + r] * xq[t * D + d];
                    DJ[p] += acc;
                }
            } else if (KIND == E2TTT_MLP) {
                // W1 [Hd][D] at 0, W2 [D][Hd] at Hd*D (column vectors)
                const int64_t o2 = (int64_t)Hd * D;     // packed offset of W2
                const int64_t w2o = Hd * wD, l2o = Hd * lD;  // ... in the (padded) weights / cotangents
                float* dy = RD(4);
                float* gy = RD(5);
                float* p2M = RD(6);
                float* p2W = RD(7);
                float* z = RH(0);
                float* e = RH(1);   // W2^T dy
                float* p1M = RH(2);
                float* p1W = RH(3);
                float* jz = RH(4);
                float* zq = RH(5);
                float* dzq = RH(6);
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float zz = 0.f, zzq = 0.f, pm = 0.f, pw = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) {
                        const float w1 = Wr[j * wD + d];
                        zz += w1 * xk[t * D + d];
                        zzq += w1 * xq[t * D + d];
                        pw += LWr[j * lD + d] * xk[t * D + d];
                        if (mom) pm += LMr[j * lD + d] * xk[t * D + d];
                    }
                    z[i] = zz;
                    zq[i] = zzq;
                    p1M[i] = pm;
                    p1W[i] = pw;
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float y = 0.f, pm = 0.f, pw = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) {
                        const float aj = silu_f(z[t * Hd + j]);
                        y += Wr[w2o + r * wH + j] * aj;
                        pw += LWr[l2o + r * lH + j] * aj;
                        if (mom) pm += LMr[l2o + r * lH + j] * aj;
                    }
                    dy[i] = mse ? y - xv[i] : -xv[i];
                    p2M[i] = pm;
                    p2W[i] = pw;
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float ee = 0.f, eq = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) {
                        const float w2 = Wr[w2o + r * wH + j];
                        ee += w2 * dy[t * D + r];
                        eq += w2 * xo[t * D + r];
                    }
                    e[i] = ee;
                    dzq[i] = eq * dsilu_f(zq[i]);
                }
                __syncthreads();
                for (int t = tid; t < nt; t += NT) {
                    float gm = 0.f, gw = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) {
                        gm += dy[t * D + r] * p2M[t * D + r];
                        gw += dy[t * D + r] * p2W[t * D + r];
                    }
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) {
                        const float dz = e[t * Hd + j] * dsilu_f(z[t * Hd + j]);
                        gm += dz * p1M[t * Hd + j];
                        gw += dz * p1W[t * Hd + j];
                    }
                    if (mom) a.dcM[bh * a.ldc + tb + t] = gm;
                    a.dcW[bh * a.ldc + tb + t] = -gw;
                }
                __syncthreads();  // the projections are overwritten next
                // combined projections p = cM pM - cW pW (in place of the M rows)
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd;
                    p1M[i] = cms[t] * p1M[i] - cws[t] * p1W[i];
                }
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D;
                    p2M[i] = cms[t] * p2M[i] - cws[t] * p2W[i];
                }
                __syncthreads();
                const float* p1 = p1M;
                const float* p2 = p2M;
                for (int i = tid; i < nt * D; i += NT) {  // Gy = p2 + W2 (silu'(z) p1)
                    const int t = i / D, r = i % D;
                    float acc = p2[i];
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j)
                        acc += Wr[w2o + r * wH + j] * dsilu_f(z[t * Hd + j]) * p1[t * Hd + j];
                    gy[i] = acc;
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {  // Ja, Jz
                    const int t = i / Hd, j = i % Hd;
                    float ja = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) {
                        const int64_t ow = w2o + r * wH + j, ol = l2o + r * lH + j;
                        const float lam = cms[t] * (mom ? LMr[ol] : 0.f) - cws[t] * LWr[ol];
                        ja += lam * dy[t * D + r] + (mse ? Wr[ow] * gy[t * D + r] : 0.f);
                    }
                    const float zz = z[i];
                    jz[i] = e[i] * p1[i] * d2silu_f(zz) + ja * dsilu_f(zz);
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, d = i % D;
                    float gk = 0.f, gq = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) {
                        const int64_t ow = j * wD + d, ol = j * lD + d;
                        const float dz = e[t * Hd + j] * dsilu_f(z[t * Hd + j]);
                        const float lam = cms[t] * (mom ? LMr[ol] : 0.f) - cws[t] * LWr[ol];
                        gk += lam * dz + Wr[ow] * jz[t * Hd + j];
                        gq += Wr[ow] * dzq[t * Hd + j];
                    }
                    st(dk, tb * D + i, gk);
                    st(dv, tb * D + i, -gy[i]);
                    st(dq, tb * D + i, gq);
                }
                for (int64_t p = tid; p < P; p += NT) {
                    float acc = 0.f;
                    if (p < o2) {
                        const int j = (int)(p / D), d = (int)(p % D);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) acc += jz[t * Hd + j] * xk[t * D + d] + dzq[t * Hd + j] * xq[t * D + d];
                    } else {
                        const int r = (int)((p - o2) / Hd), j = (int)((p - o2) % Hd);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const float zz = z[t * Hd + j];
                            acc += dy[t * D + r] * dsilu_f(zz) * p1[t * Hd + j] + xo[t * D + r] * silu_f(zq[t * Hd + j]) +
                                   (mse ? gy[t * D + r] * silu_f(zz) : 0.f);
                        }
                    }
                    DJ[p] += acc;
                }
            } else {
                // W1, W3 [D][Hd] at 0, D*Hd; W2 [Hd][D] at 2*D*Hd (row vectors)
                const int64_t o3 = (int64_t)D * Hd, o2 = 2 * (int64_t)D * Hd;  // packed offsets of W3, W2
                const int64_t w3o = D * wH, w2o = 2 * D * wH, l3o = D * lH, l2o = 2 * D * lH;
                float* dy = RD(4);
                float* gy = RD(5);
                float* h1 = RH(0);
                float* h3 = RH(1);
                float* P1 = RH(2);   // P1M, then combined P1
                float* E = RH(3);    // P1W, then E
                float* P3 = RH(4);   // P3M, then combined P3
                float* Ju = RH(5);   // P3W, then Ju
                float* Q2 = RH(6);   // Q2M, then combined Q2
                float* Jh1 = RH(7);  // Q2W, then Jh1
                float* du = RH(8);
                float* hq1 = RH(9);
                float* hq3 = RH(10);
                float* hdo = RH(11);
                float* Jh3 = RH(12);
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float a1 = 0.f, a3 = 0.f, q1 = 0.f, q3 = 0.f, m1 = 0.f, w1 = 0.f, m3 = 0.f, w3 = 0.f;
                    #pragma unroll 4
                    for (int d = 0; d < D; ++d) {
                        const int64_t ow = d * wH + j, ol = d * lH + j;
                        const float x = xk[t * D + d], y = xq[t * D + d];
                        a1 += x * Wr[ow];
                        a3 += x * Wr[w3o + ow];
                        q1 += y * Wr[ow];
                        q3 += y * Wr[w3o + ow];
                        w1 += x * LWr[ol];
                        w3 += x * LWr[l3o + ol];
                        if (mom) {
                            m1 += x * LMr[ol];
                            m3 += x * LMr[l3o + ol];
                        }
                    }
                    h1[i] = a1;
                    h3[i] = a3;
                    hq1[i] = q1;
                    hq3[i] = q3;
                    P1[i] = m1;
                    E[i] = w1;
                    P3[i] = m3;
                    Ju[i] = w3;
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, r = i % D;
                    float y = 0.f;
                    if (mse)
                        #pragma unroll 4
                        for (int j = 0; j < Hd; ++j)
                            y += silu_f(h1[t * Hd + j]) * h3[t * Hd + j] * Wr[w2o + j * wD + r];
                    dy[i] = mse ? y - xv[i] : -xv[i];
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {
                    const int t = i / Hd, j = i % Hd;
                    float u_ = 0.f, qm = 0.f, qw = 0.f, ho = 0.f;
                    #pragma unroll 4
                    for (int r = 0; r < D; ++r) {
                        const int64_t ow = w2o + j * wD + r, ol = l2o + j * lD + r;
                        const float g = dy[t * D + r];
                        u_ += g * Wr[ow];
                        qw += LWr[ol] * g;
                        if (mom) qm += LMr[ol] * g;
                        ho += xo[t * D + r] * Wr[ow];
                    }
                    du[i] = u_;
                    Q2[i] = qm;
                    Jh1[i] = qw;
                    hdo[i] = ho;
                }
                __syncthreads();
                for (int t = tid; t < nt; t += NT) {
                    float gm = 0.f, gw = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) {
                        const int i = t * Hd + j;
                        const float x1 = h1[i], x3 = h3[i];
                        const float s1 = dsilu_f(x1), act = silu_f(x1);
                        const float dh1 = du[i] * x3 * s1, dh3 = du[i] * act, u_ = act * x3;
                        gm += P1[i] * dh1 + P3[i] * dh3 + u_ * Q2[i];
                        gw += E[i] * dh1 + Ju[i] * dh3 + u_ * Jh1[i];
                    }
                    if (mom) a.dcM[bh * a.ldc + tb + t] = gm;
                    a.dcW[bh * a.ldc + tb + t] = -gw;
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {  // combined projections and E
                    const int t = i / Hd;
                    const float cm = cms[t], cw = cws[t];
                    const float p1 = cm * P1[i] - cw * E[i], p3 = cm * P3[i] - cw * Ju[i], q2 = cm * Q2[i] - cw * Jh1[i];
                    const float x1 = h1[i];
                    P1[i] = p1;
                    P3[i] = p3;
                    Q2[i] = q2;
                    E[i] = p1 * h3[i] * dsilu_f(x1) + p3 * silu_f(x1);
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {  // Gy = u Lam2 + E W2
                    const int t = i / D, r = i % D;
                    float acc = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) {
                        const int64_t ow = w2o + j * wD + r, ol = l2o + j * lD + r;
                        const float lam = cms[t] * (mom ? LMr[ol] : 0.f) - cws[t] * LWr[ol];
                        acc += silu_f(h1[t * Hd + j]) * h3[t * Hd + j] * lam + E[t * Hd + j] * Wr[ow];
                    }
                    gy[i] = acc;
                }
                __syncthreads();
                for (int i = tid; i < nt * Hd; i += NT) {  // Ju, Jh1, Jh3
                    const int t = i / Hd, j = i % Hd;
                    float ju = Q2[i];
                    if (mse)
                        #pragma unroll 4
                        for (int r = 0; r < D; ++r) ju += gy[t * D + r] * Wr[w2o + j * wD + r];
                    const float x1 = h1[i], x3 = h3[i];
                    const float s1 = dsilu_f(x1), s2 = d2silu_f(x1), act = silu_f(x1);
                    Ju[i] = ju;
                    Jh1[i] = P1[i] * du[i] * x3 * s2 + P3[i] * du[i] * s1 + ju * x3 * s1;
                    Jh3[i] = P1[i] * du[i] * s1 + ju * act;
                }
                __syncthreads();
                for (int i = tid; i < nt * D; i += NT) {
                    const int t = i / D, d = i % D;
                    float gk = 0.f, gq = 0.f;
                    #pragma unroll 4
                    for (int j = 0; j < Hd; ++j) {
                        const int64_t ow = d * wH + j, ol = d * lH + j;
                        const int h = t * Hd + j;
                        const float x1 = h1[h], x3 = h3[h];
                        const float dh1 = du[h] * x3 * dsilu_f(x1), dh3 = du[h] * silu_f(x1);
                        const float l1 = cms[t] * (mom ? LMr[ol] : 0.f) - cws[t] * LWr[ol];
                        const float l3 = cms[t] * (mom ? LMr[l3o + ol] : 0.f) - cws[t] * LWr[l3o + ol];
                        gk += Jh1[h] * Wr[ow] + Jh3[h] * Wr[w3o + ow] + dh1 * l1 + dh3 * l3;
                        const float y1 = hq1[h], y3 = hq3[h];
                        gq += hdo[h] * y3 * dsilu_f(y1) * Wr[ow] + hdo[h] * silu_f(y1) * Wr[w3o + ow];
                    }
                    st(dk, tb * D + i, gk);
                    st(dv, tb * D + i, -gy[i]);
                    st(dq, tb * D + i, gq);
                }
                for (int64_t p = tid; p < P; p += NT) {
                    float acc = 0.f;
                    if (p < o2) {
                        const bool three = p >= o3;
                        const int64_t pp = three ? p - o3 : p;
                        const int d = (int)(pp / Hd), j = (int)(pp % Hd);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const int h = t * Hd + j;
                            const float y1 = hq1[h], y3 = hq3[h];
                            const float dq_ = three ? hdo[h] * silu_f(y1) : hdo[h] * y3 * dsilu_f(y1);
                            acc += xk[t * D + d] * (three ? Jh3[h] : Jh1[h]) + xq[t * D + d] * dq_;
                        }
                    } else {
                        const int j = (int)((p - o2) / D), r = (int)((p - o2) % D);
                        #pragma unroll 4
                        for (int t = 0; t < nt; ++t) {
                            const int h = t * Hd + j;
                            const float u_ = silu_f(h1[h]) * h3[h];
                            const float uq = silu_f(hq1[h]) * hq3[h];
                            acc += E[h] * dy[t * D + r] + uq * xo[t * D + r] + (mse ? u_ * gy[t * D + r] : 0.f);
                        }
                    }
                    DJ[p] += acc;
                }
            }
            __syncthreads();
        }
        // cotangents of the chunk start (uses the chunk-end lW in both)
        const float* sc = a.scal + (bh * a.nc + c) * 4;
        const float A = sc[0], Bb = sc[1], gamma = sc[2];
        for (int64_t p = tid; p < P; p += NT) {
            const float lw = LW[p];
            LW[p] = A * lw + DJ[p];
            if (mom) LM[p] = Bb * LM[p] - gamma * lw;
        }
        __syncthreads();
    }
}

template <int KIND, typename TIO, int CACHE>
hipError_t launch_bwd_one(const e2ttt_desc& d, const GBwdArgs& a, size_t shmem, hipStream_t s) {
    const void* f = (const void*)generic_bwd_kernel<KIND, TIO, CACHE>;
    if (shmem > 64 * 1024 && hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((generic_bwd_kernel<KIND, TIO, CACHE>), dim3((unsigned)(d.B * d.H)), dim3(NT), shmem, s, a);
    return hipGetLastError();
}

template <int KIND, typename TIO>
hipError_t launch_bwd_cache(const e2ttt_desc& d, const GBwdArgs& a, int cache, size_t shmem, hipStream_t s) {
    switch (cache) {
        case 2: return launch_bwd_one<KIND, TIO, 2>(d, a, shmem, s);
        case 1: return launch_bwd_one<KIND, TIO, 1>(d, a, shmem, s);
        default: return launch_bwd_one<KIND, TIO, 0>(d, a, shmem, s);
    }
}

template <int KIND>
hipError_t launch_bwd_kind(const e2ttt_desc& d, const GBwdArgs& a, int cache, size_t shmem, hipStream_t s) {
    if (d.io_dtype == E2TTT_BF16) return launch_bwd_cache<KIND, __bf16>(d, a, cache, shmem, s);
    return launch_bwd_cache<KIND, float>(d, a, cache, shmem, s);
}

// LDS the portable kernels may use per workgroup (of gfx950's 160 KB)
constexpr size_t kLdsBudget = 144 * 1024;

int floats_per_token(const e2ttt_desc& d) {
    const int64_t Hd = d.kind == E2TTT_LINEAR ? 0 : d.Hd;
    const int kind = d.kind;
    return (int)(rows_d(kind) * d.D + rows_h(kind) * Hd + 2);
}

}  // namespace

int generic_bwd_token_block(const e2ttt_desc& d) {
    const int f = floats_per_token(d);
    for (int tb = 16; tb >= 1; tb >>= 1)
        if ((int64_t)f * tb * 4 <= 64 * 1024) return tb;
    return 0;  // not even one token fits
}

hipError_t launch_generic_backward(const e2ttt_desc& d, const GenericBwdBuffers& b, hipStream_t s) {
    GBwdArgs a;
    a.T = d.T;
    a.D = d.D;
    a.Hd = d.kind == E2TTT_LINEAR ? 0 : d.Hd;
    a.C = d.chunk;
    a.nc = (d.T + d.chunk - 1) / d.chunk;
    a.P = e2ttt_param_count(&d);
    a.ldc = b.ldc;
    a.loss = d.loss;
    a.TB = generic_bwd_token_block(d);
    a.mom = (d.flags & E2TTT_FLAG_NO_MOMENTUM) ? 0 : 1;
    a.q = b.q;
    a.k = b.k;
    a.v = b.v;
    a.dout = b.dout;
    a.cM = b.cM;
    a.cW = b.cW;
    a.scal = b.scal;
    a.save = b.save;
    a.dW_end = b.dW_end;
    a.dM_end = b.dM_end;
    a.lamW = b.dW0;
    a.lamM = b.dM0;
    a.dacc = b.dacc;
    a.dq = b.dq;
    a.dk = b.dk;
    a.dv = b.dv;
    a.dcM = b.dcM;
    a.dcW = b.dcW;
    a.dpart = b.dpart;
    size_t shmem = (size_t)floats_per_token(d) * a.TB * sizeof(float);
    // cache as many of W_c, lW, lM as fit next to the token rows (a smaller
    // token block would cost more than the cache saves: every block re-reads
    // and re-writes the dJ/dW accumulators)
    const int64_t Hd0 = d.kind == E2TTT_LINEAR ? 0 : d.Hd;
    const int64_t PP = d.kind == E2TTT_LINEAR ? padded_count<E2TTT_LINEAR>(d.D, Hd0)
                       : d.kind == E2TTT_MLP  ? padded_count<E2TTT_MLP>(d.D, Hd0)
                                              : padded_count<E2TTT_SWIGLU>(d.D, Hd0);
    int cache = 0;
    for (int c = 2; c >= 1 && cache == 0; --c) {
        const int arrays = c == 1 ? 1 : (a.mom ? 3 : 2);  // W_c; or W_c, lW (and lM)
        const size_t need = ((size_t)floats_per_token(d) * a.TB + (size_t)arrays * PP) * sizeof(float);
        if (need <= kLdsBudget) {
            cache = c;
            shmem = need;
        }
    }
    hipError_t e;
    switch (d.kind) {
        case E2TTT_LINEAR: e = launch_bwd_kind<E2TTT_LINEAR>(d, a, cache, shmem, s); break;
        case E2TTT_MLP: e = launch_bwd_kind<E2TTT_MLP>(d, a, cache, shmem, s); break;
        default: e = launch_bwd_kind<E2TTT_SWIGLU>(d, a, cache, shmem, s); break;
    }
    if (e != hipSuccess) return e;
    return launch_bwd_scalar(d, b.eta, b.alpha, b.beta, b.dcM, b.dcW, b.ldc, b.dpart, 1, b.deta, b.dalpha, b.dbeta,
                             s);
}

}  // namespace e2ttt

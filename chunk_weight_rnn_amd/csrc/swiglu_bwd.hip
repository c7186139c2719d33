// SwiGLU fast weight, negative-dot loss, bf16 q/k/v: the backward pass of the
// E2-TTT chunk update on CDNA4 (gfx950).
//
// Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
// (abstract; atlas summary "Approach"): the forward pass takes, per chunk,
// gradients at the chunk-start weights W_c, two weighted aggregations with the
// per-token coefficients cM = eta*m, cW = eta*w, and the transition
//   M_{c+1} = Bb M_c + sum_t cM_t g_t,   W_{c+1} = A W_c - gamma M_c - sum_t cW_t g_t,
// and emits out_t = f_{W_c}(q_t).  This file is its vector-Jacobian product.
//
// Reverse over chunks with the state cotangents (lW, lM) of (W_{c+1}, M_{c+1})
// (initially dW_end, dM_end).  Per token t and hidden unit j of chunk c, at
// W_c (row vectors; W1, W3 [D x Hd], W2 [Hd x D]):
//   h1 = k W1, h3 = k W3, du = -v W2^T, a = silu(h1), s = silu'(h1),
//   s2 = silu''(h1), u = a h3, dh1 = du h3 s, dh3 = du a;
//   projections of the cotangents: pX1 = k lX1, pX3 = k lX3, pX2 = v lX2^T
//   (X in {W, M}), combined P = cM pM - cW pW;
//   E  = P1 h3 s + P3 a                          (d/d du)
//   F1 = du P1 h3 s2 + (du P3 - h3 P2) s          (d/d h1)
//   F3 = du P1 s - a P2                           (d/d h3)
//   dcM_t = sum_j pM1 dh1 + pM3 dh3 - u pM2,   dcW_t = -(same with pW)
//   dk_t = sum_j F1 W1[:,j] + F3 W3[:,j] + dh1 (cM lM1 - cW lW1)[:,j]
//                                        + dh3 (cM lM3 - cW lW3)[:,j]
//   dv_t = sum_j -E W2[j,:] - u (cM lM2 - cW lW2)[j,:]
//   output path: hq1 = q W1, hq3 = q W3, hdo = do W2^T, uq = silu(hq1) hq3,
//   dhq1 = hdo hq3 silu'(hq1), dhq3 = hdo silu(hq1),
//   dq_t = sum_j dhq1 W1[:,j] + dhq3 W3[:,j]
// and per chunk
//   dW1 = sum_t k_t^T F1 + q_t^T dhq1,  dW3 = sum_t k_t^T F3 + q_t^T dhq3,
//   dW2 = sum_t -E^T v_t + uq^T do_t,
//   lW <- A lW + dW,   lM <- Bb lM - gamma lW_old,
//   dA = <lW_old, W_c>,  dBb = <lM_old, M_c>,  dgamma = -<lW_old, M_c>.
// The chunk-start states come from a forward recompute (bf16 snapshots of W_c
// and M_c); the scalar kernels' backward turns dcM, dcW, dA, dBb, dgamma into
// d eta, d alpha, d beta.
//
// Kernels, per chunk from the last to the first:
//   token kernel  (one workgroup per 64 tokens): projections at W_c and the
//                 cotangents (16x16x32 MFMA, hidden units 16 at a time through
//                 LDS), the elementwise terms, and dk, dv, dq, dcM, dcW summed
//                 over all hidden units (pairs of 16-unit products as one
//                 16x16x32 MFMA); E, F1, F3, dhq1, dhq3,
//                 uq go to a per-chunk buffer for
//   weight kernel (one workgroup per 64 hidden units): the chunk's dW by a
//                 contraction over its tokens (16x16x32 MFMA, token rows
//                 through LDS and the gfx950 transpose read) and the state
//                 cotangent update, in fp32, with bf16 copies for the next
//                 token kernel;
// then one scalar kernel for the whole sequence.
#include "e2ttt_internal.h"

namespace e2ttt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int D = 128;             // head dim
constexpr int NT = 256;            // 4 wavefronts per workgroup
constexpr int US = 16;             // hidden units per token-kernel step
constexpr int TB = 64;             // tokens per token-kernel workgroup
constexpr int ROWB = D * 2;        // one bf16 row of D
constexpr int STEPB = US * ROWB;   // one matrix's rows of a token-kernel step (4 KB)
constexpr int NMAT = 9;            // W1^T, W3^T, W2, lW1^T, lW3^T, lW2, lM1^T, lM3^T, lM2
constexpr int WS = 64;             // hidden units per weight-kernel workgroup
constexpr int KT = 32;             // tokens per weight-kernel step
constexpr int KTB = KT * ROWB;     // one token matrix's rows of a weight-kernel step (8 KB)
constexpr int NQ = 6;              // per (token, unit) terms handed to the weight kernel
constexpr int RSRC_W3 = 0x00020000;  // dword 3 of a raw buffer resource (32-bit format, no swizzle)

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x16: A lane (row l%16, k 4(l/16)..+3), B lane (column l%16, same k)
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                      0, 0, 0);
}

// Two K = 16 products into one 16x16x32 MFMA: k-slots 0..3 of lane group g
// take a's and b's units 4g..4g+3, slots 4..7 the second pair's.
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = lo[e];
        r[4 + e] = hi[e];
    }
    return r;
}

__device__ __forceinline__ float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// 16-byte chunk swizzles of 256-byte LDS rows: logical chunk c of row t sits
// at physical chunk c ^ swz(t).  The LDS has 64 four-byte banks.
// ds_read_b128 serves 16 lanes per cycle, lanes 8a .. 8a+7 together with
// 32+8a .. 32+8a+7 (this grouping reproduces the measured conflict counts of
// every kernel here); the transpose read ds_read_b64_tr_b16 serves lanes 0..31,
// then 32..63.
//   swz_u: hidden-unit stage [16 rows].  Row fragments (b128): lanes
//          (row r, column-chunk group g) with rows 8h .. 8h+7 and groups g,
//          g + 2 together, i.e. chunks c ^ swz(r) and c ^ 2 ^ swz(r): the 8
//          values swz(r) must not contain a pair differing only in bit 1.
//          Transpose fragments: 8 rows per cycle (0..7, 8..15), each at an
//          aligned chunk pair that lands on pair n ^ (swz(r) >> 1), so
//          swz(r) >> 1 must differ across those 8 rows.  Bits 1..3 of
//          swz(r) = r mod 8 and bit 0 = bit 1 meet both.
//   swz_t: token stage [32 rows], transpose reads only: rows {0..3, 8..11}
//          and {4..7, 12..15} per cycle, swz(r) >> 1 distinct within each.
__device__ __forceinline__ int swz_u(int t) { return ((t & 7) << 1) | (t & 1); }
__device__ __forceinline__ int swz_t(int t) { return ((t & 3) << 1) | (t & 8) | ((t >> 2) & 1); }

// (base and size must be the same in every lane; the words are read from
// the first lane so that the descriptor lives in scalar registers)
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, unsigned num_bytes) {
    const unsigned long long p = (unsigned long long)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((unsigned)p);
    r[1] = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xFFFFu);
    r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
    r[3] = RSRC_W3;
    return r;
}

// HBM -> LDS copy of 16 bytes per lane: lane L reads base + voff (zeros at or
// past the resource's size) and writes LDS byte lds + 16 L.  Its completion is
// waited for explicitly with wait_vm; the instruction writes no register.
__device__ __forceinline__ void copy16(u32x4 rsrc, unsigned lds, unsigned voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Wait for a step's stage copies but not for the kStoresAfterCopy global
// stores each wave issues after them in the previous step (vector memory
// operations complete in issue order, so vmcnt(k) leaves the last k pending).
constexpr int kStoresAfterCopy = 12;  // three put_inter calls of four stores
__device__ __forceinline__ void wait_stage(int step) {
    if (step == 0)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else
        __builtin_amdgcn_s_waitcnt(0x0F70 | kStoresAfterCopy);  // vmcnt(12)
}

__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Workgroup id -> logical id such that consecutive logical ids (the slices or
// token blocks of one head, which read the same operands) share an XCD:
// hardware ids go round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_remap(int nwg, int on) {
    const int b = blockIdx.x;
    return on ? (b % 8) * (nwg / 8) + b / 8 : b;
}

// B fragment of a 16x16x16 MFMA from a hidden-major [16 units][D] stage
// (swizzled rows): lane (p, g) gets rows 4g + e (e = 0..3), column d0 + p,
// by the transpose read (lane p's result slot e comes from the 8 bytes that
// lane 4e + p/4 of its 16-lane group addresses, element p%4).
__device__ __forceinline__ bf16x4 tr_units(const unsigned char* stage, int lane, int n) {
    const int p = lane & 15, g = lane >> 4;
    const int row = 4 * g + (p >> 2);
    const int q = p & 3;
    const unsigned char* a = stage + row * ROWB + 16 * ((2 * n + (q >> 1)) ^ swz_u(row)) + 8 * (q & 1);
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a);
}

// B fragment of a 16x16x32 MFMA from a token-major [32 tokens][D] stage:
// lane (p, g) gets tokens 8g + e (e = 0..7), column 16 n + p.
__device__ __forceinline__ bf16x8 tr_tokens(const unsigned char* stage, int lane, int n) {
    const int p = lane & 15, g = lane >> 4;
    const int q = p & 3;
    bf16x8 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 8 * g + 4 * h + (p >> 2);
        const unsigned char* a = stage + row * ROWB + 16 * ((2 * n + (q >> 1)) ^ swz_t(row & 15)) + 8 * (q & 1);
        const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a);
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 * h + e] = v[e];
    }
    return r;
}

// ---------------------------------------------------------------------------
// token kernel
struct TokArgs {
    const __bf16 *k, *v, *q, *dout;  // [BH][T][D]
    const float *cM, *cW;            // [BH][ldc]
    const __bf16* snapW;             // [BH][nc][3][Hd][D]: W1^T, W3^T, W2 of each chunk start
    const __bf16* lam;               // [BH][6][Hd][D]: lW1^T, lW3^T, lW2, lM1^T, lM3^T, lM2
    __bf16* inter;                   // [BH][6][Hd][C]: F1, F3, -E, dhq1, dhq3, uq
    __bf16 *dq, *dk, *dv;            // [BH][T][D]
    float *dcM, *dcW;                // [BH][ldc]
    float* part;                     // U > 1: [3][BH][T][U][D] dk, dv, dq and [2][BH][ldc][U] dcM, dcW partial sums
    int64_t T, ldc, BH;
    int Hd, C, nc, c, nb;            // nb: 64-token blocks of chunk c
    int U;                           // parts of the hidden units, one workgroup each
    int nwg, xcd_map;
};

template <bool MOM>
__global__ void __launch_bounds__(NT) bwd_tok_kernel(TokArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char stage[2 * NMAT * STEPB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tl = lane & 15, g = lane >> 4;
    const int lid = xcd_remap(a.nwg, a.xcd_map);
    const int64_t bh = lid / (a.nb * a.U);
    const int blk = (lid / a.U) % a.nb;
    const int part = lid % a.U;  // hidden units part * Hd / U .. of the head
    const int64_t T = a.T;
    const int Hd = a.Hd;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int64_t tc0 = (int64_t)a.c * a.C + blk * TB + 16 * w;  // the wave's first token
    const int64_t t = tc0 + tl;                                  // this lane's token (projections)
    const bool tin = t < T;
    const int tcl = blk * TB + 16 * w + tl;                      // ... within the chunk
    constexpr int nmat = MOM ? NMAT : 6;

    const u32x4 wrs = buffer_rsrc(a.snapW + (bh * a.nc + a.c) * P, (unsigned)(P * 2));
    const u32x4 lrs = buffer_rsrc(a.lam + bh * 2 * P, (unsigned)(2 * P * 2));
    const unsigned stage_lds = lds_addr(stage);
    // rows j0 .. j0+15 of matrices 0 .. nm-1 into stage buffer b: 4 copies per
    // matrix (4 rows each), spread over the 4 waves
    auto issue = [&](int j0, int b, int nm) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        for (int ii = w; ii < 4 * nm; ii += 4) {
            const int mi = ii >> 2, rq = ii & 3;
            const int row = 4 * rq + (ln >> 4);
            const unsigned off = (unsigned)((mi < 3 ? mi : mi - 3) * Hd * D + (j0 + row) * D) * 2u +
                                 16u * (unsigned)((ln & 15) ^ swz_u(row));
            copy16(mi < 3 ? wrs : lrs, stage_lds + (unsigned)((b * NMAT + mi) * STEPB + 4 * rq * ROWB), off);
        }
    };
    // A fragment of a projection: row j0 + tl of matrix mi, d = 32 kk + 8 g .. +7
    auto afrag = [&](const unsigned char* sb, int mi, int kk) {
        return *(const bf16x8*)(sb + mi * STEPB + tl * ROWB + 16 * ((4 * kk + g) ^ swz_u(tl)));
    };
    auto load_tok = [&](const __bf16* X, bf16x8 (&f)[4]) {
        const __bf16* row = X + (bh * T + (tin ? t : 0)) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            f[kk] = *(const bf16x8*)(row + 32 * kk);
            if (!tin) f[kk] = bf16x8{};
        }
    };
    __bf16* const inter = a.inter + bh * NQ * (int64_t)Hd * a.C;
    auto put_inter = [&](int qi, int j0, const float (&x)[4]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) inter[((int64_t)qi * Hd + j0 + 4 * g + r) * a.C + tcl] = (__bf16)x[r];
    };
    auto store_tok = [&](__bf16* X, const f32x4 (&acc)[8]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t tt = tc0 + 4 * g + r;
            if (tt < T) {
#pragma unroll
                for (int n = 0; n < 8; ++n) X[(bh * T + tt) * D + 16 * n + tl] = (__bf16)acc[n][r];
            }
        }
    };
    const int nsteps = Hd / a.U / US;
    const int jp = part * (Hd / a.U);  // the workgroup's first hidden unit
    // with U > 1 the sums over hidden units (dk, dv, dq, dcM, dcW) leave as
    // fp32 partial sums of this part, added up in a fixed order afterwards
    // (the U parts of one row side by side, so that the sum reads one stream)
    const int64_t BHTDU = a.BH * T * D * a.U;
    float* const pdc = a.part + 3 * BHTDU + part;  // [2][BH][ldc][U]
    auto part_tok = [&](int which, const f32x4 (&acc)[8]) {
        float* const X = a.part + which * BHTDU + (int64_t)part * D;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t tt = tc0 + 4 * g + r;
            if (tt < T) {
#pragma unroll
                for (int n = 0; n < 8; ++n) X[(bh * T + tt) * a.U * D + 16 * n + tl] = acc[n][r];
            }
        }
    };

    // ---------------- pass A: k / v side (needs W_c and the cotangents)
    {
        const float cm = MOM ? a.cM[bh * a.ldc + tcl + (int64_t)a.c * a.C] : 0.f;
        const float cw = a.cW[bh * a.ldc + tcl + (int64_t)a.c * a.C];
        bf16x8 xk[4], xv[4];
        load_tok(a.k, xk);
        load_tok(a.v, xv);
        f32x4 dk[8], dv[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) dk[n] = dv[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        float sM = 0.f, sW = 0.f;
        issue(jp, 0, nmat);
        for (int js = 0; js < nsteps; ++js) {
            wait_stage(js);
            barrier_lds();
            if (js + 1 < nsteps) issue(jp + US * (js + 1), (js + 1) & 1, nmat);
            const unsigned char* sb = stage + (js & 1) * NMAT * STEPB;
            const int j0 = jp + US * js;
            f32x4 pr[NMAT];
#pragma unroll
            for (int mi = 0; mi < nmat; ++mi) pr[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int mi = 0; mi < nmat; ++mi) {
                    const bool vside = (mi == 2 || mi == 5 || mi == 8);
                    pr[mi] = mfma32(afrag(sb, mi, kk), vside ? xv[kk] : xk[kk], pr[mi]);
                }
            }
            // elementwise: lane holds units j0 + 4g + r of token tl
            float F1[4], F3[4], nE[4];
            bf16x4 aF1, aF3, aW1, aW3, aM1, aM3, anE, aW2, aM2;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float h1 = pr[0][r], h3 = pr[1][r], du = -pr[2][r];
                const float sg = fast_sigmoid(h1);
                const float act = h1 * sg;
                const float s1 = sg * (1.f + h1 * (1.f - sg));
                const float s2 = sg * (1.f - sg) * (2.f + h1 * (1.f - 2.f * sg));
                const float u = act * h3, dh1 = du * h3 * s1, dh3 = du * act;
                float P1 = -cw * pr[3][r], P3 = -cw * pr[4][r], P2 = -cw * pr[5][r];
                if (MOM) {
                    P1 += cm * pr[6][r];
                    P3 += cm * pr[7][r];
                    P2 += cm * pr[8][r];
                }
                const float E = P1 * h3 * s1 + P3 * act;
                F1[r] = du * P1 * h3 * s2 + (du * P3 - h3 * P2) * s1;
                F3[r] = du * P1 * s1 - act * P2;
                nE[r] = -E;
                sW -= pr[3][r] * dh1 + pr[4][r] * dh3 - u * pr[5][r];
                if (MOM) sM += pr[6][r] * dh1 + pr[7][r] * dh3 - u * pr[8][r];
                aF1[r] = (__bf16)F1[r];
                aF3[r] = (__bf16)F3[r];
                anE[r] = (__bf16)nE[r];
                aW1[r] = (__bf16)(-cw * dh1);
                aW3[r] = (__bf16)(-cw * dh3);
                aW2[r] = (__bf16)(cw * u);
                aM1[r] = (__bf16)(cm * dh1);
                aM3[r] = (__bf16)(cm * dh3);
                aM2[r] = (__bf16)(-cm * u);
            }
            put_inter(0, j0, F1);
            put_inter(1, j0, F3);
            put_inter(2, j0, nE);
            // token side: contraction over the step's 16 units, the B fragments
            // of column tile n + 1 read while tile n's MFMAs run
            bf16x4 bf[NMAT];
#pragma unroll
            for (int mi = 0; mi < nmat; ++mi) bf[mi] = tr_units(sb + mi * STEPB, lane, 0);
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                bf16x4 cur[NMAT];
#pragma unroll
                for (int mi = 0; mi < nmat; ++mi) cur[mi] = bf[mi];
                if (n + 1 < 8) {
#pragma unroll
                    for (int mi = 0; mi < nmat; ++mi) bf[mi] = tr_units(sb + mi * STEPB, lane, n + 1);
                }
                // pairs of K = 16 terms as one K = 32 product each
                dk[n] = mfma32(cat8(aF1, aF3), cat8(cur[0], cur[1]), dk[n]);
                dk[n] = mfma32(cat8(aW1, aW3), cat8(cur[3], cur[4]), dk[n]);
                dv[n] = mfma32(cat8(anE, aW2), cat8(cur[2], cur[5]), dv[n]);
                if (MOM) {
                    dk[n] = mfma32(cat8(aM1, aM3), cat8(cur[6], cur[7]), dk[n]);
                    dv[n] = mfma16(aM2, cur[8], dv[n]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (a.U == 1) {
            store_tok(a.dk, dk);
            store_tok(a.dv, dv);
        } else {
            part_tok(0, dk);
            part_tok(1, dv);
        }
        sW += __shfl_xor(sW, 16);
        sW += __shfl_xor(sW, 32);
        if (MOM) {
            sM += __shfl_xor(sM, 16);
            sM += __shfl_xor(sM, 32);
        }
        if (g == 0) {
            const int64_t o = bh * a.ldc + (int64_t)a.c * a.C + tcl;
            if (a.U == 1) {
                a.dcW[o] = sW;
                if (MOM) a.dcM[o] = sM;
            } else {
                pdc[(a.BH * a.ldc + o) * a.U] = sW;
                if (MOM) pdc[o * a.U] = sM;
            }
        }
    }
    barrier_lds();  // every wave is done with the stage buffers

    // ---------------- pass B: output path (needs W_c only)
    {
        bf16x8 xq[4], xd[4];
        load_tok(a.q, xq);
        load_tok(a.dout, xd);
        f32x4 dq[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) dq[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        issue(jp, 0, 3);
        for (int js = 0; js < nsteps; ++js) {
            wait_stage(js);
            barrier_lds();
            if (js + 1 < nsteps) issue(jp + US * (js + 1), (js + 1) & 1, 3);
            const unsigned char* sb = stage + (js & 1) * NMAT * STEPB;
            const int j0 = jp + US * js;
            f32x4 pr[3];
#pragma unroll
            for (int mi = 0; mi < 3; ++mi) pr[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                pr[0] = mfma32(afrag(sb, 0, kk), xq[kk], pr[0]);
                pr[1] = mfma32(afrag(sb, 1, kk), xq[kk], pr[1]);
                pr[2] = mfma32(afrag(sb, 2, kk), xd[kk], pr[2]);
            }
            float d1[4], d3[4], uq[4];
            bf16x4 a1, a3;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float h1 = pr[0][r], h3 = pr[1][r], hdo = pr[2][r];
                const float sg = fast_sigmoid(h1);
                const float act = h1 * sg;
                const float s1 = sg * (1.f + h1 * (1.f - sg));
                d1[r] = hdo * h3 * s1;
                d3[r] = hdo * act;
                uq[r] = act * h3;
                a1[r] = (__bf16)d1[r];
                a3[r] = (__bf16)d3[r];
            }
            put_inter(3, j0, d1);
            put_inter(4, j0, d3);
            put_inter(5, j0, uq);
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                dq[n] = mfma32(cat8(a1, a3), cat8(tr_units(sb + 0 * STEPB, lane, n), tr_units(sb + 1 * STEPB, lane, n)),
                               dq[n]);
                if (n & 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (a.U == 1)
            store_tok(a.dq, dq);
        else
            part_tok(2, dq);
    }
}

// The U parts' partial sums of the reverse loop, added in part order: dk, dv,
// dq to bf16, dcM and dcW (the padded rows too) in fp32.
struct ReduceArgs {
    const float* part;  // [3][BH][T][U][D], then [2][BH][ldc][U]
    __bf16 *dk, *dv, *dq;
    float *dcM, *dcW;
    int64_t BHTD, BHL;  // B*H*T*D, B*H*ldc
    int U, mom;
};

__global__ void __launch_bounds__(256) bwd_part_reduce_kernel(ReduceArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
#pragma unroll
    for (int which = 0; which < 3; ++which) {
        const float* const src = a.part + which * a.BHTD * a.U;
        __bf16* const dst = which == 0 ? a.dk : which == 1 ? a.dv : a.dq;
        for (int64_t e = 4 * i0; e < a.BHTD; e += 4 * stride) {
            const float* const p = src + (e / D) * a.U * D + e % D;  // row e / D, columns e % D .. + 3
            f32x4 sum = *(const f32x4*)p;
            for (int u = 1; u < a.U; ++u) sum += *(const f32x4*)(p + u * D);
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (__bf16)sum[r];
            *(bf16x4*)(dst + e) = o;
        }
    }
    const float* const pdc = a.part + 3 * a.BHTD * a.U;
    for (int which = a.mom ? 0 : 1; which < 2; ++which) {  // 0: dcM, 1: dcW
        float* const dst = which == 0 ? a.dcM : a.dcW;
        for (int64_t e = i0; e < a.BHL; e += stride) {
            const float* const p = pdc + (which * a.BHL + e) * a.U;
            float sum = p[0];
            for (int u = 1; u < a.U; ++u) sum += p[u];
            dst[e] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// weight kernel
struct WtArgs {
    const __bf16 *k, *v, *q, *dout;  // [BH][T][D]
    const __bf16* inter;             // [BH][6][Hd][C]
    const __bf16 *snapW, *snapM;     // [BH][nc][3][Hd][D]
    const float* scal;               // [BH][nc][4]: A, Bb, gamma
    float *lamW, *lamM;              // [BH][3][Hd][D] fp32 state cotangents, hidden-major, updated in place
    __bf16* lam;                     // [BH][6][Hd][D] bf16 copies (token kernel operands)
    float* dpart;                    // [BH][nc][nsl][4]: partial dA, dBb, dgamma
    int64_t T;
    int Hd, C, nc, c, nsl, nsteps;   // nsteps: 32-token steps of chunk c (whole 64-token blocks)
    int nwg, xcd_map;
};

template <bool MOM>
__global__ void __launch_bounds__(NT) bwd_wt_kernel(WtArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char stage[2 * 4 * KTB];
    __shared__ float red[4][4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = lane & 15, g = lane >> 4;
    const int lid = xcd_remap(a.nwg, a.xcd_map);
    const int64_t bh = lid / a.nsl;
    const int sl = lid % a.nsl;
    const int Hd = a.Hd;
    const int64_t T = a.T;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int j0 = WS * sl + 16 * w;  // the wave's 16 hidden units
    const unsigned xbytes = (unsigned)(T * D * 2);
    const u32x4 rs[4] = {buffer_rsrc(a.k + bh * T * D, xbytes), buffer_rsrc(a.q + bh * T * D, xbytes),
                         buffer_rsrc(a.v + bh * T * D, xbytes), buffer_rsrc(a.dout + bh * T * D, xbytes)};
    const unsigned stage_lds = lds_addr(stage);
    const int64_t tbase = (int64_t)a.c * a.C;
    // token rows of step s (32 rows of k, q, v, do) into buffer b: 8 copies
    // per matrix (4 rows each), spread over the waves
    auto issue = [&](int s, int b) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int x8 = 0; x8 < 8; ++x8) {
            const int mat = x8 >> 1, rq = 4 * (x8 & 1) + w;  // (matrix index stays compile-time)
            const int row = 4 * rq + (ln >> 4);
            const unsigned off = (unsigned)((tbase + KT * s + row) * D) * 2u + 16u * (unsigned)((ln & 15) ^ swz_t(row & 15));
            copy16(rs[mat], stage_lds + (unsigned)((b * 4 + mat) * KTB + 4 * rq * ROWB), off);
        }
    };
    // A fragments: rows j0 + p of the six per-(token, unit) terms, tokens
    // 32 s + 8 g .. +7
    const __bf16* const inter = a.inter + (bh * NQ * Hd + j0 + p) * (int64_t)a.C + 8 * g;
    auto load_frags = [&](int s, bf16x8 (&f)[NQ]) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) f[qi] = *(const bf16x8*)(inter + (int64_t)qi * Hd * a.C + KT * s);
    };
    f32x4 acc[3][8];
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 fa[NQ];
    load_frags(0, fa);
    issue(0, 0);
    for (int s = 0; s < a.nsteps; ++s) {
        wait_vm0();
        barrier_lds();
        bf16x8 fn[NQ];
        if (s + 1 < a.nsteps) {
            issue(s + 1, (s + 1) & 1);
            load_frags(s + 1, fn);
        }
        const unsigned char* sb = stage + (s & 1) * 4 * KTB;
        bf16x8 nb4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) nb4[x] = tr_tokens(sb + x * KTB, lane, 0);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const bf16x8 bk = nb4[0], bq = nb4[1], bv = nb4[2], bd = nb4[3];
            if (n + 1 < 8) {
#pragma unroll
                for (int x = 0; x < 4; ++x) nb4[x] = tr_tokens(sb + x * KTB, lane, n + 1);
            }
            acc[0][n] = mfma32(fa[0], bk, acc[0][n]);
            acc[0][n] = mfma32(fa[3], bq, acc[0][n]);
            acc[1][n] = mfma32(fa[1], bk, acc[1][n]);
            acc[1][n] = mfma32(fa[4], bq, acc[1][n]);
            acc[2][n] = mfma32(fa[2], bv, acc[2][n]);
            acc[2][n] = mfma32(fa[5], bd, acc[2][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s + 1 < a.nsteps) {
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) fa[qi] = fn[qi];
        }
    }

    // State cotangents, one matrix at a time: the accumulators (lane: units
    // j0 + 4g + r, d = 16 n + p) are parked as a [64 units][D] fp32 tile in
    // the idle stage buffer (row stride 132 floats: conflict-free), then the
    // whole workgroup walks the tile row by row, 4 d per thread, so that every
    // global access covers whole rows (fp32 cotangents 512 B, bf16 snapshots
    // and copies 256 B per unit).
    const f32x4 sc = *(const f32x4*)(a.scal + (bh * a.nc + a.c) * 4);
    const float A = sc[0], Bb = sc[1], gam = sc[2];
    const int64_t ws0 = (int64_t)WS * sl;  // the workgroup's first unit
    float* const lamW = a.lamW + bh * P;
    float* const lamM = MOM ? a.lamM + bh * P : nullptr;
    const __bf16* const snw = a.snapW + (bh * a.nc + a.c) * P;
    const __bf16* const snm = MOM ? a.snapM + (bh * a.nc + a.c) * P : nullptr;
    __bf16* const cpW = a.lam + bh * 2 * P;
    __bf16* const cpM = a.lam + bh * 2 * P + P;
    const bool copies = a.c > 0;  // chunk 0's cotangents are final: no token kernel reads them
    constexpr int TS = 132;       // parked tile row stride (floats)
    float* const tile = (float*)stage;
    float sA = 0.f, sB = 0.f, sG = 0.f;
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int m = 0; m < 3; ++m) {
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) tile[(16 * w + 4 * g + r) * TS + 16 * n + p] = acc[m][n][r];
        __syncthreads();
#pragma unroll 2
        for (int e = tid; e < WS * D / 4; e += NT) {
            const int jj = e / (D / 4), d4 = 4 * (e % (D / 4));
            const int64_t hm = ((int64_t)m * Hd + ws0 + jj) * D + d4;
            const f32x4 an = *(const f32x4*)(tile + jj * TS + d4);
            const f32x4 lw = *(const f32x4*)(lamW + hm);
            const bf16x4 wc = *(const bf16x4*)(snw + hm);
            f32x4 lm = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x4 mc = bf16x4{};
            if (MOM) {
                lm = *(const f32x4*)(lamM + hm);
                mc = *(const bf16x4*)(snm + hm);
            }
            f32x4 nw, nm;
            bf16x4 bw, bm;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sA += lw[r] * (float)wc[r];
                nw[r] = A * lw[r] + an[r];
                bw[r] = (__bf16)nw[r];
                if (MOM) {
                    sB += lm[r] * (float)mc[r];
                    sG -= lw[r] * (float)mc[r];
                    nm[r] = Bb * lm[r] - gam * lw[r];
                    bm[r] = (__bf16)nm[r];
                }
            }
            *(f32x4*)(lamW + hm) = nw;
            if (MOM) *(f32x4*)(lamM + hm) = nm;
            if (copies) {
                *(bf16x4*)(cpW + hm) = bw;
                if (MOM) *(bf16x4*)(cpM + hm) = bm;
            }
        }
        __syncthreads();  // the tile is rewritten for the next matrix
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        sA += __shfl_xor(sA, o);
        sB += __shfl_xor(sB, o);
        sG += __shfl_xor(sG, o);
    }
    if (lane == 0) {
        red[w][0] = sA;
        red[w][1] = sB;
        red[w][2] = sG;
    }
    __syncthreads();
    if (tid < 3) {
        const float v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
        a.dpart[((bh * a.nc + a.c) * a.nsl + sl) * 4 + tid] = v;
    }
}

// ---------------------------------------------------------------------------
// Layout changes of the state cotangents between the packed parameter layout
// (W1, W3 [D][Hd], W2 [Hd][D]) and the hidden-major working layout ([3][Hd][D]):
// W1 / W3 are transposed through LDS 64 units at a time, W2 is hidden-major
// already.  TO_HIDDEN: packed dW_end / dM_end -> fp32 working copy + bf16
// copies; else the working copy -> packed dW0 / dM0.
struct LayoutArgs {
    const float *srcW, *srcM;  // [BH][P]
    float *dstW, *dstM;        // [BH][P]
    __bf16* cp;                // [BH][2P] bf16 copies (TO_HIDDEN only)
    int Hd, nsl, nx;           // nx: 2 with momentum (W and M), else 1
};

template <bool TO_HIDDEN>
__global__ void __launch_bounds__(NT) bwd_layout_kernel(LayoutArgs a) {
    __shared__ float tile[D][WS + 1];
    const int64_t bh = blockIdx.x / (a.nx * a.nsl);
    const int x = (blockIdx.x / a.nsl) % a.nx;  // 0: W, 1: M
    const int sl = blockIdx.x % a.nsl;
    const int Hd = a.Hd;
    const int64_t P = 3 * (int64_t)D * Hd;
    const float* src = (x ? a.srcM : a.srcW) + bh * P;
    float* dst = (x ? a.dstM : a.dstW) + bh * P;
    __bf16* cp = TO_HIDDEN ? a.cp + bh * 2 * P + x * P : nullptr;
    const int j0 = WS * sl;
    for (int m = 0; m < 2; ++m) {
        const int64_t pk = (int64_t)m * D * Hd + j0;            // packed: + d * Hd + j
        const int64_t hmb = ((int64_t)m * Hd + j0) * D;         // hidden-major: + j * D + d
        for (int e = threadIdx.x; e < D * WS / 4; e += NT) {
            if (TO_HIDDEN) {  // 16-byte reads along the packed rows
                const int d = e / (WS / 4), j4 = 4 * (e % (WS / 4));
                const f32x4 v = *(const f32x4*)(src + pk + (int64_t)d * Hd + j4);
#pragma unroll
                for (int i = 0; i < 4; ++i) tile[d][j4 + i] = v[i];
            } else {  // 16-byte reads along the hidden-major rows
                const int jj = e / (D / 4), d4 = 4 * (e % (D / 4));
                const f32x4 v = *(const f32x4*)(src + hmb + (int64_t)jj * D + d4);
#pragma unroll
                for (int i = 0; i < 4; ++i) tile[d4 + i][jj] = v[i];
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < D * WS / 4; e += NT) {
            if (TO_HIDDEN) {  // 16-byte writes along the hidden-major rows
                const int jj = e / (D / 4), d4 = 4 * (e % (D / 4));
                f32x4 v;
                bf16x4 b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = tile[d4 + i][jj];
                    b[i] = (__bf16)v[i];
                }
                *(f32x4*)(dst + hmb + (int64_t)jj * D + d4) = v;
                *(bf16x4*)(cp + hmb + (int64_t)jj * D + d4) = b;
            } else {  // 16-byte writes along the packed rows
                const int d = e / (WS / 4), j4 = 4 * (e % (WS / 4));
                f32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = tile[d][j4 + i];
                *(f32x4*)(dst + pk + (int64_t)d * Hd + j4) = v;
            }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < WS * D / 4; e += NT) {
        const int64_t o = 2 * (int64_t)D * Hd + (int64_t)j0 * D + 4 * e;
        const f32x4 v = *(const f32x4*)(src + o);
        *(f32x4*)(dst + o) = v;
        if (TO_HIDDEN) {
            bf16x4 b;
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i] = (__bf16)v[i];
            *(bf16x4*)(cp + o) = b;
        }
    }
}

// ---------------------------------------------------------------------------
// scalar kernels' backward, one workgroup (one wavefront) per (b, h, chunk).
// With a_i = prod_{s>i} alpha_s, m_i = prod_{s>i} beta_s and
// w_i = a_i + beta_{i+1} w_{i+1} (w_last = 1), A = alpha_0 a_0, Bb = beta_0 m_0,
// gamma = beta_0 w_0, the adjoints run forward through the chunk from
// Wb_{-1} = dgamma, Mb_{-1} = dBb, Ab_{-1} = dA:
//   Wb_i = dw_i + beta_i Wb_{i-1},  Mb_i = dm_i + beta_i Mb_{i-1},  Ab_i = Wb_i + alpha_i Ab_{i-1},
//   dalpha_i = Ab_{i-1} a_i,  dbeta_i = Wb_{i-1} w_i + Mb_{i-1} m_i,
// with dm_i = eta_i dcM_i, dw_i = eta_i dcW_i and deta_i = m_i dcM_i + w_i dcW_i
// (chunk average: m_i, w_i replaced by their means mb, wb; then
// deta_i = mb dcM_i + wb dcW_i and dm_i = sum_t eta_t dcM_t / C for every i).
// Every recurrence is affine, x_i = u_i + v_i x_{i-1} (or its mirror image for
// the suffix quantities): each lane folds its segment of consecutive tokens
// into one map, a log-step shuffle scan composes the maps across the wave,
// and each lane then replays its segment from its incoming value.
struct ScalArgs {
    const float *eta, *alpha, *beta;  // [BH][T]
    const float *dcM, *dcW;           // [BH][ldc]
    const float* dpart;               // [BH][nc][nsl][4]
    float *deta, *dalpha, *dbeta;     // [BH][T]
    int64_t T, ldc;
    int C, nc, nsl, mom, avg;
};

// composition of affine maps x -> u + v x: (u, v) after (u', v')
__device__ __forceinline__ void compose(float& u, float& v, float u2, float v2) {
    u = u + v * u2;
    v = v * v2;
}

// inclusive scan of maps over lanes: from the right (lane l gets
// f_l o f_{l+1} o ... o f_63) or from the left (f_l o ... o f_0)
template <bool RIGHT>
__device__ __forceinline__ void scan_maps(float& u, float& v, int lane) {
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        float u2 = RIGHT ? __shfl_down(u, k) : __shfl_up(u, k);
        float v2 = RIGHT ? __shfl_down(v, k) : __shfl_up(v, k);
        const bool in = RIGHT ? lane + k < 64 : lane >= k;
        if (!in) {
            u2 = 0.f;
            v2 = 1.f;
        }
        compose(u, v, u2, v2);
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__global__ void __launch_bounds__(64) bwd_scalar_kernel(ScalArgs a) {
    extern __shared__ float sh[];
    const int C = a.C;
    float* al = sh;
    float* be = sh + C;
    float* et = sh + 2 * C;
    float* gm = sh + 3 * C;  // dcM, then d eta
    float* gw = sh + 4 * C;  // dcW
    float* va = sh + 5 * C;  // a_i, then d alpha
    float* vm = sh + 6 * C;  // m_i, then d beta
    float* vw = sh + 7 * C;  // w_i
    const int64_t bh = blockIdx.x / a.nc;
    const int c = blockIdx.x % a.nc;
    const int lane = threadIdx.x;
    const int64_t t0 = (int64_t)c * C;
    const int Cc = (int)((a.T - t0) < C ? (a.T - t0) : C);
    const int64_t base = bh * a.T + t0;
    const int64_t cb = bh * a.ldc + t0;
    for (int i = lane; i < Cc; i += 64) {
        al[i] = a.alpha[base + i];
        be[i] = a.mom ? a.beta[base + i] : 0.f;
        et[i] = a.eta[base + i];
        gm[i] = a.mom ? a.dcM[cb + i] : 0.f;
        gw[i] = a.dcW[cb + i];
    }
    __syncthreads();
    float dA = 0.f, dB = 0.f, dG = 0.f;
    const float* dp = a.dpart + (bh * a.nc + c) * a.nsl * 4;
    for (int s = 0; s < a.nsl; ++s) {
        dA += dp[4 * s];
        dB += dp[4 * s + 1];
        dG += dp[4 * s + 2];
    }
    const int L = (Cc + 63) / 64;  // tokens per lane
    const int i0 = lane * L < Cc ? lane * L : Cc;
    const int i1 = i0 + L < Cc ? i0 + L : Cc;
    auto bnext = [&](int i) { return i + 1 < Cc ? be[i + 1] : 0.f; };

    // a_i, m_i: suffix products (segment products scanned from the right)
    float pa = 1.f, pb = 1.f;
    for (int i = i0; i < i1; ++i) {
        pa *= al[i];
        pb *= be[i];
    }
    {
        float u = 0.f, v = pa, u2 = 0.f, v2 = pb;  // products as maps x -> v x
        scan_maps<true>(u, v, lane);
        scan_maps<true>(u2, v2, lane);
        float ra = __shfl_down(v, 1), rm = __shfl_down(v2, 1);
        if (lane == 63) ra = rm = 1.f;
        for (int i = i1 - 1; i >= i0; --i) {
            va[i] = ra;
            vm[i] = rm;
            ra *= al[i];
            rm *= be[i];
        }
    }
    // w_i = a_i + beta_{i+1} w_{i+1}: the segment as w_{i0} = X + Y w_{i1}
    {
        float X = 0.f, Y = 1.f;
        for (int i = i1 - 1; i >= i0; --i) {
            const float bn = bnext(i);
            X = va[i] + bn * X;
            Y = bn * Y;
        }
        scan_maps<true>(X, Y, lane);
        float wv = __shfl_down(X, 1);  // w of the next segment's first token (maps applied to 0)
        if (lane == 63) wv = 0.f;
        for (int i = i1 - 1; i >= i0; --i) {
            wv = va[i] + bnext(i) * wv;
            vw[i] = wv;
        }
    }
    float mb = 0.f, wb = 0.f, dmb = 0.f, dwb = 0.f;
    if (a.avg) {
        float sm = 0.f, sw = 0.f, sdm = 0.f, sdw = 0.f;
        for (int i = i0; i < i1; ++i) {
            sm += vm[i];
            sw += vw[i];
            sdm += et[i] * gm[i];
            sdw += et[i] * gw[i];
        }
        const float inv = 1.f / (float)Cc;
        mb = wave_sum(sm) * inv;
        wb = wave_sum(sw) * inv;
        dmb = wave_sum(sdm) * inv;
        dwb = wave_sum(sdw) * inv;
    }
    auto dm_of = [&](int i) { return a.avg ? dmb : et[i] * gm[i]; };
    auto dw_of = [&](int i) { return a.avg ? dwb : et[i] * gw[i]; };

    // Wb, Mb: segment maps from the left, applied to dgamma / dBb
    float Wi, Mi;  // Wb_{i0-1}, Mb_{i0-1}
    {
        float uw = 0.f, vwm = 1.f, um = 0.f, vmm = 1.f;
        for (int i = i0; i < i1; ++i) {
            uw = dw_of(i) + be[i] * uw;
            vwm = be[i] * vwm;
            um = dm_of(i) + be[i] * um;
            vmm = be[i] * vmm;
        }
        scan_maps<false>(uw, vwm, lane);
        scan_maps<false>(um, vmm, lane);
        float ue = __shfl_up(uw, 1), ve = __shfl_up(vwm, 1), ume = __shfl_up(um, 1), vme = __shfl_up(vmm, 1);
        if (lane == 0) {
            ue = ume = 0.f;
            ve = vme = 1.f;
        }
        Wi = ue + ve * dG;
        Mi = ume + vme * dB;
    }
    // Ab: Ab_i = Wb_i + alpha_i Ab_{i-1}, from dA
    float Ai;  // Ab_{i0-1}
    {
        float ua = 0.f, vaa = 1.f, wbv = Wi;
        for (int i = i0; i < i1; ++i) {
            wbv = dw_of(i) + be[i] * wbv;
            ua = wbv + al[i] * ua;
            vaa = al[i] * vaa;
        }
        scan_maps<false>(ua, vaa, lane);
        float ue = __shfl_up(ua, 1), ve = __shfl_up(vaa, 1);
        if (lane == 0) {
            ue = 0.f;
            ve = 1.f;
        }
        Ai = ue + ve * dA;
    }
    // replay: gradients of every token of the segment
    for (int i = i0; i < i1; ++i) {
        const float de = a.avg ? mb * gm[i] + wb * gw[i] : vm[i] * gm[i] + vw[i] * gw[i];
        const float da = Ai * va[i];
        const float db = Wi * vw[i] + Mi * vm[i];
        Wi = dw_of(i) + be[i] * Wi;
        Mi = dm_of(i) + be[i] * Mi;
        Ai = Wi + al[i] * Ai;
        gm[i] = de;
        va[i] = da;
        vm[i] = db;
    }
    __syncthreads();
    for (int i = lane; i < Cc; i += 64) {
        a.deta[base + i] = gm[i];
        a.dalpha[base + i] = va[i];
        if (a.mom) a.dbeta[base + i] = vm[i];
    }
}

}  // namespace

int64_t swiglu_bwd_inter_elems(const e2ttt_desc& d) { return (int64_t)NQ * d.Hd * d.chunk; }

// Parts of the hidden units in the token kernel: a head's chunk gives
// B·H·(chunk/64) workgroups; small grids split each one's hidden units over
// 2 or 4 workgroups (shorter chains, more of the 256 compute units busy).
int swiglu_bwd_unit_parts(const e2ttt_desc& d) {
    const int64_t span = d.chunk < d.T ? d.chunk : d.T;
    const int64_t wg = d.B * d.H * ((span + TB - 1) / TB);
    if (wg * 4 <= 256 && d.Hd % (4 * US) == 0) return 4;
    if (wg * 2 <= 256 && d.Hd % (2 * US) == 0) return 2;
    return 1;
}

int64_t swiglu_bwd_part_elems(const e2ttt_desc& d, int64_t ldc) {
    const int U = swiglu_bwd_unit_parts(d);
    if (U == 1) return 0;
    const int64_t BH = d.B * d.H;
    return (int64_t)U * (3 * BH * d.T * D + 2 * BH * ldc);
}

hipError_t launch_swiglu_backward(const e2ttt_desc& d, const BwdBuffers& b, hipStream_t s, hipEvent_t ev_loop) {
    const int64_t BH = d.B * d.H;
    const bool mom = !(d.flags & E2TTT_FLAG_NO_MOMENTUM);
    const int Hd = (int)d.Hd, C = (int)d.chunk;
    const int nc = (int)((d.T + d.chunk - 1) / d.chunk);
    const int nsl = Hd / WS;
    const int nx = mom ? 2 : 1;
    const int U = swiglu_bwd_unit_parts(d);
    if (U > 1 && !b.part) return hipErrorInvalidValue;
    {  // working copy and bf16 copies of dW_end, dM_end
        LayoutArgs la{b.dW_end, b.dM_end, b.lamW, b.lamM, (__bf16*)b.lam, Hd, nsl, nx};
        hipLaunchKernelGGL(bwd_layout_kernel<true>, dim3((unsigned)(BH * nx * nsl)), dim3(NT), 0, s, la);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    for (int c = nc - 1; c >= 0; --c) {
        const int Cc = (int)((d.T - (int64_t)c * C) < C ? (d.T - (int64_t)c * C) : C);
        const int nb = (Cc + TB - 1) / TB;
        TokArgs ta;
        ta.k = (const __bf16*)b.k;
        ta.v = (const __bf16*)b.v;
        ta.q = (const __bf16*)b.q;
        ta.dout = (const __bf16*)b.dout;
        ta.cM = b.cM;
        ta.cW = b.cW;
        ta.snapW = (const __bf16*)b.snapW;
        ta.lam = (const __bf16*)b.lam;
        ta.inter = (__bf16*)b.inter;
        ta.dq = (__bf16*)b.dq;
        ta.dk = (__bf16*)b.dk;
        ta.dv = (__bf16*)b.dv;
        ta.dcM = b.dcM;
        ta.dcW = b.dcW;
        ta.part = b.part;
        ta.T = d.T;
        ta.ldc = b.ldc;
        ta.BH = BH;
        ta.Hd = Hd;
        ta.C = C;
        ta.nc = nc;
        ta.c = c;
        ta.nb = nb;
        ta.U = U;
        ta.nwg = (int)(BH * nb * U);
        ta.xcd_map = ta.nwg % 8 == 0 ? 1 : 0;
        if (mom)
            hipLaunchKernelGGL(bwd_tok_kernel<true>, dim3((unsigned)ta.nwg), dim3(NT), 0, s, ta);
        else
            hipLaunchKernelGGL(bwd_tok_kernel<false>, dim3((unsigned)ta.nwg), dim3(NT), 0, s, ta);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        WtArgs wa;
        wa.k = (const __bf16*)b.k;
        wa.v = (const __bf16*)b.v;
        wa.q = (const __bf16*)b.q;
        wa.dout = (const __bf16*)b.dout;
        wa.inter = (const __bf16*)b.inter;
        wa.snapW = (const __bf16*)b.snapW;
        wa.snapM = (const __bf16*)b.snapM;
        wa.scal = b.scal;
        wa.lamW = b.lamW;
        wa.lamM = b.lamM;
        wa.lam = (__bf16*)b.lam;
        wa.dpart = b.dpart;
        wa.T = d.T;
        wa.Hd = Hd;
        wa.C = C;
        wa.nc = nc;
        wa.c = c;
        wa.nsl = nsl;
        wa.nsteps = nb * (TB / KT);
        wa.nwg = (int)(BH * nsl);
        wa.xcd_map = wa.nwg % 8 == 0 ? 1 : 0;
        if (mom)
            hipLaunchKernelGGL(bwd_wt_kernel<true>, dim3((unsigned)wa.nwg), dim3(NT), 0, s, wa);
        else
            hipLaunchKernelGGL(bwd_wt_kernel<false>, dim3((unsigned)wa.nwg), dim3(NT), 0, s, wa);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    {  // chunk 0's state cotangents -> packed dW0, dM0
        LayoutArgs la{b.lamW, b.lamM, b.dW0, b.dM0, nullptr, Hd, nsl, nx};
        hipLaunchKernelGGL(bwd_layout_kernel<false>, dim3((unsigned)(BH * nx * nsl)), dim3(NT), 0, s, la);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (U > 1) {  // the parts' dk, dv, dq, dcM, dcW
        ReduceArgs ra{b.part, (__bf16*)b.dk, (__bf16*)b.dv, (__bf16*)b.dq, b.dcM, b.dcW, BH * d.T * D, BH * b.ldc, U,
                      mom ? 1 : 0};
        hipLaunchKernelGGL(bwd_part_reduce_kernel, dim3(4096), dim3(256), 0, s, ra);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    if (ev_loop && hipEventRecord(ev_loop, s) != hipSuccess) return hipErrorLaunchFailure;
    return launch_bwd_scalar(d, b.eta, b.alpha, b.beta, b.dcM, b.dcW, b.ldc, b.dpart, nsl, b.deta, b.dalpha, b.dbeta,
                             s);
}

hipError_t launch_bwd_scalar(const e2ttt_desc& d, const float* eta, const float* alpha, const float* beta,
                             const float* dcM, const float* dcW, int64_t ldc, const float* dpart, int nsl,
                             float* deta, float* dalpha, float* dbeta, hipStream_t s) {
    const int64_t BH = d.B * d.H;
    const int C = (int)d.chunk;
    const int nc = (int)((d.T + d.chunk - 1) / d.chunk);
    ScalArgs sa;
    sa.eta = eta;
    sa.alpha = alpha;
    sa.beta = beta;
    sa.dcM = dcM;
    sa.dcW = dcW;
    sa.dpart = dpart;
    sa.deta = deta;
    sa.dalpha = dalpha;
    sa.dbeta = dbeta;
    sa.T = d.T;
    sa.ldc = ldc;
    sa.C = C;
    sa.nc = nc;
    sa.nsl = nsl;
    sa.mom = (d.flags & E2TTT_FLAG_NO_MOMENTUM) ? 0 : 1;
    sa.avg = (d.flags & E2TTT_FLAG_CHUNK_AVG) ? 1 : 0;
    hipLaunchKernelGGL(bwd_scalar_kernel, dim3((unsigned)(BH * nc)), dim3(64), (size_t)8 * C * sizeof(float), s, sa);
    return hipGetLastError();
}

}  // namespace e2ttt

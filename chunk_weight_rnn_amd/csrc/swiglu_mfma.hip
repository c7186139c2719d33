// SwiGLU fast weight, negative-dot loss, bf16 q/k/v/out, fp32 state: the
// CDNA4 (gfx950) MFMA path of the E2-TTT chunk update.
//
// Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
// (abstract; atlas summary "Approach"): gradients at the chunk-start weights,
// two scalar kernels, two weighted gradient aggregations, and the chunk
// output from the chunk-start weights (arxivlens "Limitations").
//
// Per (b, h) and chunk, with K, V, Q the chunk's [C x D] token rows, the
// chunk-start weights W1, W3 [D x Hd], W2 [Hd x D] and per-token coefficients
// cM = eta*m, cW = eta*w from e2ttt_logscan:
//   grad:       H1 = K W1, H3 = K W3, dU = -V W2^T                      [C x Hd]
//               U = silu(H1)*H3, dH3 = dU*silu(H1), dH1 = dU*H3*silu'(H1)
//   aggregate:  G1 = K^T diag(c) dH1, G3 = K^T diag(c) dH3,
//               G2^T = V^T diag(-c) U           for c in {cM, cW}
//   epilogue:   M <- Bb*M + G^M,   W <- A*W - gamma*M_old - G^W
//   apply:      out = (silu(Q W1) * (Q W3)) W2
//
// Because dL/dy = -v does not depend on W, hidden unit j's gradient touches
// only column j of W1, W3 and row j of W2: a head's hidden units split into
// independent slices of 64.  One workgroup (4 wavefronts, one per SIMD) owns
// one (b, h, slice) for the whole sequence and keeps that slice's fp32 W and M
// (6 x 128 x 64 values) resident as MFMA accumulators of the aggregation GEMM
// across all chunks.  The epilogue therefore never touches HBM: W and M are
// rescaled in registers at each chunk start and the aggregation MFMAs
// accumulate straight into them.
//
// The output needs every hidden unit of the head, so the loop kernel writes a
// bf16 snapshot of each chunk-start weight slice and a second, fully
// parallel kernel computes every chunk's output from the snapshots.
#include "e2ttt_internal.h"

namespace e2ttt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;   // head dim
constexpr int S = 64;    // hidden units per workgroup slice
constexpr int CB = 64;   // tokens per block inside a chunk
constexpr int NT = 256;  // 4 wavefronts

// LDS pitches (bf16 elements); +8 keeps 16-byte row accesses bank-conflict free
constexpr int PW = D + 8;   // weight slices [S][PW]
constexpr int PK = CB + 8;  // K^T, V^T [D][PK]
constexpr int PDT = CB + 8; // scaled backward factors [S][PDT]

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 pack4(float a, float b, float c, float d) {
    bf16x4 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    r[2] = (__bf16)c;
    r[3] = (__bf16)d;
    return r;
}

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + __expf(-x)); }

struct LoopArgs {
    const __bf16* k;
    const __bf16* v;
    const float* cM;
    const float* cW;
    const float* scal;
    const float* W0;
    const float* M0;
    float* W_end;
    float* M_end;
    __bf16* snap;
    int64_t T;
    int Hd, C, nc, nsl, nwg, xcd_map;
};

struct alignas(16) Lds {
    __bf16 wsl[3][S][PW];  // chunk-start weights: W1^T, W3^T, W2 rows of the slice
    __bf16 kt[D][PK];      // K^T of the current token block
    __bf16 vt[D][PK];      // V^T
    __bf16 dt[6][S][PDT];  // c-scaled factors, hidden-major: 1M 1W 3M 3W 2M 2W
};

// tile element (lane l, register r) of a 32x32 MFMA accumulator:
//   col = l % 32, row = 8*(r/4) + 4*(l/32) + r%4

// Aggregation over one token block.  The wave owns row tiles {rt0, rt0+1} of
// D and hidden half h of the slice for all three matrices: acc[rr][2m] and
// acc[rr][2m+1] are the M and W parts of matrix m (0: W1, 1: W3, 2: W2^T).
__device__ __forceinline__ void aggregate_block(f32x16 (&acc)[2][6], const Lds& L, int lane, int rt0, int h) {
    const int li = lane & 31, lg = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < CB / 16; ++ks) {
        const int kc = 16 * ks + 8 * lg;
        bf16x8 ak[2], av[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            ak[rr] = *(const bf16x8*)&L.kt[32 * (rt0 + rr) + li][kc];
            av[rr] = *(const bf16x8*)&L.vt[32 * (rt0 + rr) + li][kc];
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const bf16x8 bm = *(const bf16x8*)&L.dt[2 * m][32 * h + li][kc];
            const bf16x8 bw = *(const bf16x8*)&L.dt[2 * m + 1][32 * h + li][kc];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const bf16x8 a = (m < 2) ? ak[rr] : av[rr];
                acc[rr][2 * m] = mfma32(a, bm, acc[rr][2 * m]);
                acc[rr][2 * m + 1] = mfma32(a, bw, acc[rr][2 * m + 1]);
            }
        }
    }
}

// State tiles <-> packed fp32 parameters (W1 [D][Hd] | W3 [D][Hd] | W2 [Hd][D]).
// Element (lane, r) of the tile for pair p and row tile rt sits at
//   mat < 2: mat*D*Hd + d*Hd + j      mat == 2: 2*D*Hd + j*D + d
// with d = 32 rt + 8 (r/4) + 4 lg + r%4 and j = j0 + 32 h + li.  Addresses
// are split into a wave-uniform base plus one 32-bit lane offset
// (laneA = 4 lg Hd + li for [d][j], laneB = li D + 4 lg for [j][d]).
template <bool STORE>
__device__ __forceinline__ void state_io(f32x16 (&acc)[2][6], float* W, float* M, int rt0, int h, int j0, int Hd,
                                         unsigned laneA, unsigned laneB) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int mat = p;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dr = 32 * (rt0 + rr) + 8 * (r / 4) + (r % 4);  // uniform part of d
                float* wb;
                float* mb;
                unsigned lo;
                if (mat < 2) {
                    const int64_t ub = (int64_t)mat * D * Hd + (int64_t)dr * Hd + j0 + 32 * h;
                    wb = W + ub;
                    mb = M + ub;
                    lo = laneA;
                } else {
                    const int64_t ub = 2 * (int64_t)D * Hd + (int64_t)(j0 + 32 * h) * D + dr;
                    wb = W + ub;
                    mb = M + ub;
                    lo = laneB;
                }
                if (STORE) {
                    mb[lo] = acc[rr][2 * p][r];
                    wb[lo] = acc[rr][2 * p + 1][r];
                } else {
                    acc[rr][2 * p][r] = mb[lo];
                    acc[rr][2 * p + 1][r] = wb[lo];
                }
            }
        }
    }
}

// Chunk start: write the bf16 weights (LDS operand slices and the global
// snapshot W1^T [Hd][D] | W3^T [Hd][D] | W2 [Hd][D], all hidden-major), then
// rescale the state: W <- A W - gamma M, M <- Bb M.
__device__ __forceinline__ void chunk_start(f32x16 (&acc)[2][6], Lds& L, __bf16* snap, int lane, int rt0, int h,
                                            int j0, int Hd, float A, float Bb, float gamma) {
    const int li = lane & 31, lg = lane >> 5;
    const int jl = 32 * h + li;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        __bf16* base = snap + (int64_t)m * Hd * D + (int64_t)(j0 + 32 * h) * D + 32 * rt0 + li * D + 4 * lg;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const f32x16 w = acc[rr][2 * m + 1];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const bf16x4 v4 = pack4(w[4 * qd], w[4 * qd + 1], w[4 * qd + 2], w[4 * qd + 3]);
                *(bf16x4*)&L.wsl[m][jl][32 * (rt0 + rr) + 8 * qd + 4 * lg] = v4;
                *(bf16x4*)&base[32 * rr + 8 * qd] = v4;
            }
            const f32x16 mm = acc[rr][2 * m];
            acc[rr][2 * m + 1] = A * w - gamma * mm;
            acc[rr][2 * m] = Bb * mm;
        }
    }
}

__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
swiglu_loop_kernel(LoopArgs a) {
    __shared__ Lds L;
    __shared__ alignas(16) float cbuf[2][2][CB];  // per-token cM, cW of a block, double-buffered
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int lane = tid & 63;
    const int li = lane & 31, lg = lane >> 5;

    // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
    // remap to keep the slices of one head (which read the same K/V) on one XCD.
    int L_id = blockIdx.x;
    if (a.xcd_map) L_id = (blockIdx.x % 8) * (a.nwg / 8) + blockIdx.x / 8;
    const int64_t bh = L_id / a.nsl;
    const int j0 = (L_id % a.nsl) * S;
    const int Hd = a.Hd;
    const int64_t T = a.T;
    const int64_t P = 3 * (int64_t)D * Hd;

    const __bf16* kb = a.k + bh * T * D;
    const __bf16* vb = a.v + bh * T * D;
    const float* cMb = a.cM + bh * T;
    const float* cWb = a.cW + bh * T;

    // state ownership: wave -> row tiles (of D) {rt0, rt0+1} x hidden half hh of the slice
    const int rt0 = 2 * (wave & 1);
    const int hh = wave >> 1;
    // grad ownership: wave -> token rows [32*gr, +32) x hidden cols [32*gc, +32) of the slice
    const int gr = wave >> 1, gc = wave & 1;

    const unsigned laneA = (unsigned)(4 * lg * Hd + li);
    const unsigned laneB = (unsigned)(li * D + 4 * lg);
    const unsigned laneK = (unsigned)(li * D + 8 * lg);  // A-operand rows of K / V

    f32x16 acc[2][6];
    state_io<false>(acc, (float*)a.W0 + bh * P, (float*)a.M0 + bh * P, rt0, hh, j0, Hd, laneA, laneB);

    const int nblk = (int)(T / CB);
    const int bpc = a.C / CB;

    // A operands of the next block's grad GEMMs (K and V rows), prefetched
    bf16x8 ka[8], va[8];
    auto prefetch = [&](int blk) {
        const __bf16* kr = kb + ((int64_t)blk * CB + 32 * gr) * D;
        const __bf16* vr = vb + ((int64_t)blk * CB + 32 * gr) * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            ka[ks] = *(const bf16x8*)&kr[laneK + 16 * ks];
            va[ks] = *(const bf16x8*)&vr[laneK + 16 * ks];
        }
    };
    prefetch(0);
    if (wave == 0) {
        cbuf[0][0][lane] = cMb[lane];
        cbuf[0][1][lane] = cWb[lane];
    }

    for (int blk = 0; blk < nblk; ++blk) {
        const int c = blk / bpc;
        if (blk % bpc == 0) {
            const float* sc = a.scal + (bh * a.nc + c) * 4;
            const float A = sc[0], Bb = sc[1], gamma = sc[2];
            __bf16* snap = a.snap + (bh * a.nc + c) * P;
            chunk_start(acc, L, snap, lane, rt0, hh, j0, Hd, A, Bb, gamma);
            __syncthreads();
        }

        // ---- K^T (waves with gc == 0) or V^T (gc == 1) of token rows gr into LDS,
        // transposed out of the A-operand registers: lane holds row t = 32 gr + li,
        // d = 16 ks + 8 lg + e
        if (gc == 0) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) L.kt[16 * ks + 8 * lg + e][32 * gr + li] = ka[ks][e];
        } else {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) L.vt[16 * ks + 8 * lg + e][32 * gr + li] = va[ks][e];
        }

        // ---- grad: H1, H3, V W2^T for token rows gr, hidden cols gc
        f32x16 h1 = {}, h3 = {}, hv = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int kc = 16 * ks + 8 * lg;
            const bf16x8 b1 = *(const bf16x8*)&L.wsl[0][32 * gc + li][kc];
            const bf16x8 b3 = *(const bf16x8*)&L.wsl[1][32 * gc + li][kc];
            const bf16x8 b2 = *(const bf16x8*)&L.wsl[2][32 * gc + li][kc];
            h1 = mfma32(ka[ks], b1, h1);
            h3 = mfma32(ka[ks], b3, h3);
            hv = mfma32(va[ks], b2, hv);
        }
        // ---- elementwise backward and coefficient scaling -> LDS (hidden-major)
        {
            const int jl = 32 * gc + li;
            const float(*cb)[CB] = cbuf[blk & 1];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int tcol = 32 * gr + 8 * qd + 4 * lg;
                const f32x4 cm4 = *(const f32x4*)&cb[0][tcol];
                const f32x4 cw4 = *(const f32x4*)&cb[1][tcol];
                float o[6][4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * qd + e;
                    const float x1 = h1[r], x3 = h3[r], du = -hv[r];
                    const float sg = sigm(x1);
                    const float s1 = x1 * sg;
                    const float u = s1 * x3;
                    const float dh3 = du * s1;
                    const float dh1 = du * x3 * sg * (1.f + x1 * (1.f - sg));
                    const float cm = cm4[e], cw = cw4[e];
                    o[0][e] = cm * dh1;
                    o[1][e] = -cw * dh1;
                    o[2][e] = cm * dh3;
                    o[3][e] = -cw * dh3;
                    o[4][e] = -cm * u;
                    o[5][e] = cw * u;
                }
#pragma unroll
                for (int ty = 0; ty < 6; ++ty)
                    *(bf16x4*)&L.dt[ty][jl][tcol] = pack4(o[ty][0], o[ty][1], o[ty][2], o[ty][3]);
            }
        }
        __syncthreads();

        // ---- prefetch the next block (K/V rows to registers, coefficients to LDS)
        const bool more = blk + 1 < nblk;
        float cm_n = 0.f, cw_n = 0.f;
        if (more) {
            prefetch(blk + 1);
            if (wave == 0) {
                cm_n = cMb[(int64_t)(blk + 1) * CB + lane];
                cw_n = cWb[(int64_t)(blk + 1) * CB + lane];
            }
        }

        // ---- aggregation into the resident state
        aggregate_block(acc, L, lane, rt0, hh);
        if (more && wave == 0) {
            cbuf[(blk + 1) & 1][0][lane] = cm_n;
            cbuf[(blk + 1) & 1][1][lane] = cw_n;
        }
        __syncthreads();
    }

    float* We = a.W_end + bh * P;
    float* Me = a.M_end + bh * P;
    state_io<true>(acc, We, Me, rt0, hh, j0, Hd, laneA, laneB);
}

// ---------------------------------------------------------------------------
// apply: out = (silu(Q W1) * (Q W3)) W2 from the chunk-start snapshot.
// Snapshot layout per (b, h, chunk), bf16: W1^T [Hd][D] | W3^T [Hd][D] | W2 [Hd][D].
// One wavefront per 32 tokens; hidden units streamed through LDS 64 at a time.
// Computed transposed (H^T = W1^T Q^T, out^T = W2^T U^T) so that U^T leaves
// the first MFMA in exactly the register layout the second one consumes.
// ---------------------------------------------------------------------------
struct ApplyArgs {
    const __bf16* q;
    const __bf16* snap;
    __bf16* out;
    int64_t T;
    int Hd, C, nc, rbc;  // rbc: row blocks per chunk
};

constexpr int HB = 64;
constexpr int PA1 = D + 8;   // [HB][PA1] for W1^T / W3^T rows
constexpr int PA2 = HB + 8;  // [D][PA2] for W2^T columns

template <int NWA>
__global__ __launch_bounds__(64 * NWA) void swiglu_apply_kernel(ApplyArgs a) {
    __shared__ __bf16 lw1[HB][PA1];
    __shared__ __bf16 lw3[HB][PA1];
    __shared__ __bf16 lw2[D][PA2];
    constexpr int NTA = 64 * NWA;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 31, lg = lane >> 5;
    const int64_t wg = blockIdx.x;
    const int64_t bh = wg / ((int64_t)a.nc * a.rbc);
    const int rem = (int)(wg % ((int64_t)a.nc * a.rbc));
    const int c = rem / a.rbc, rb = rem % a.rbc;
    const int Hd = a.Hd;
    const int64_t t0 = (int64_t)c * a.C + (int64_t)rb * 32 * NWA + 32 * wave;
    const int64_t P = 3 * (int64_t)D * Hd;
    const __bf16* sn = a.snap + (bh * a.nc + c) * P;
    const __bf16* qb = a.q + bh * a.T * D;

    bf16x8 qf[8];  // Q^T as B operand: col = token, k = d
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)&qb[(t0 + li) * D + 16 * ks + 8 * lg];

    f32x16 oacc[4] = {};
    for (int hb = 0; hb < Hd; hb += HB) {
        // stage W1^T, W3^T rows [hb, hb+64) and W2^T columns [hb, hb+64)
        for (int i = tid; i < HB * (D / 8); i += NTA) {
            const int r = i / (D / 8), c8 = (i % (D / 8)) * 8;
            *(bf16x8*)&lw1[r][c8] = *(const bf16x8*)&sn[(int64_t)(hb + r) * D + c8];
            *(bf16x8*)&lw3[r][c8] = *(const bf16x8*)&sn[(int64_t)Hd * D + (int64_t)(hb + r) * D + c8];
        }
        // W2 rows [hb, hb+64) transposed into lw2[d][j]: lanes run over j so the
        // 2-byte LDS writes of one instruction land in consecutive columns
        for (int i = tid; i < HB * (D / 8); i += NTA) {
            const int r = i % HB, c8 = (i / HB) * 8;
            const bf16x8 w8 = *(const bf16x8*)&sn[2 * (int64_t)Hd * D + (int64_t)(hb + r) * D + c8];
#pragma unroll
            for (int e = 0; e < 8; ++e) lw2[c8 + e][r] = w8[e];
        }
        __syncthreads();
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            f32x16 x1 = {}, x3 = {};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int kc = 16 * ks + 8 * lg;
                x1 = mfma32(*(const bf16x8*)&lw1[32 * jt + li][kc], qf[ks], x1);
                x3 = mfma32(*(const bf16x8*)&lw3[32 * jt + li][kc], qf[ks], x3);
            }
            // U^T tile: rows j = 32 jt + 8(r/4) + 4 lg + r%4, col = token
            bf16x8 ub[2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 8 * s + e;
                    const float h = x1[r];
                    ub[s][e] = (__bf16)(h * sigm(h) * x3[r]);
                }
            // k-step s covers j = 32 jt + 16 s + {0..15}; lane group lg holds
            // j offsets {4lg..4lg+3, 8+4lg..8+4lg+3}; the A operand matches it.
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int jb = 32 * jt + 16 * s + 4 * lg;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const u32x2 lo = *(const u32x2*)&lw2[32 * dt + li][jb];
                    const u32x2 hi = *(const u32x2*)&lw2[32 * dt + li][jb + 8];
                    u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, av), ub[s], oacc[dt]);
                }
            }
        }
        __syncthreads();
    }
    __bf16* ob = a.out + bh * a.T * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d = 32 * dt + 8 * qd + 4 * lg;
            *(bf16x4*)&ob[(t0 + li) * D + d] =
                pack4(oacc[dt][4 * qd], oacc[dt][4 * qd + 1], oacc[dt][4 * qd + 2], oacc[dt][4 * qd + 3]);
        }
}

}  // namespace

bool swiglu_mfma_supported(const e2ttt_desc& d) {
    return d.kind == E2TTT_SWIGLU && d.loss == E2TTT_LOSS_NEGDOT && d.io_dtype == E2TTT_BF16 && d.D == D &&
           d.Hd >= S && d.Hd % S == 0 && d.Hd <= 4096 && d.chunk % CB == 0;
}

hipError_t launch_swiglu_mfma(const e2ttt_desc& d, const void* q, const void* k, const void* v, const float* cM,
                              const float* cW, const float* scal, const float* W0, const float* M0, void* out,
                              float* W_end, float* M_end, void* snap, hipStream_t s, hipEvent_t ev_mid) {
    const int64_t BH = d.B * d.H;
    LoopArgs la;
    la.k = (const __bf16*)k;
    la.v = (const __bf16*)v;
    la.cM = cM;
    la.cW = cW;
    la.scal = scal;
    la.W0 = W0;
    la.M0 = M0;
    la.W_end = W_end;
    la.M_end = M_end;
    la.snap = (__bf16*)snap;
    la.T = d.T;
    la.Hd = (int)d.Hd;
    la.C = (int)d.chunk;
    la.nc = (int)(d.T / d.chunk);
    la.nsl = (int)(d.Hd / S);
    la.nwg = (int)(BH * la.nsl);
    la.xcd_map = (la.nwg % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL(swiglu_loop_kernel, dim3((unsigned)la.nwg), dim3(NT), 0, s, la);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_mid && (e = hipEventRecord(ev_mid, s)) != hipSuccess) return e;

    ApplyArgs aa;
    aa.q = (const __bf16*)q;
    aa.snap = (const __bf16*)snap;
    aa.out = (__bf16*)out;
    aa.T = d.T;
    aa.Hd = (int)d.Hd;
    aa.C = (int)d.chunk;
    aa.nc = (int)(d.T / d.chunk);
    if (d.chunk % 128 == 0) {
        aa.rbc = (int)(d.chunk / 128);
        hipLaunchKernelGGL(swiglu_apply_kernel<4>, dim3((unsigned)(BH * aa.nc * aa.rbc)), dim3(256), 0, s, aa);
    } else {
        aa.rbc = (int)(d.chunk / 64);
        hipLaunchKernelGGL(swiglu_apply_kernel<2>, dim3((unsigned)(BH * aa.nc * aa.rbc)), dim3(128), 0, s, aa);
    }
    return hipGetLastError();
}

}  // namespace e2ttt

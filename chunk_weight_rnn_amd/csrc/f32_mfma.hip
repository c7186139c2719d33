// fp32 MFMA chunk loop for the linear and MLP fast weights with fp32 q/k/v/out
// on CDNA4 (gfx950): every contraction of the chunk update runs on
// v_mfma_f32_16x16x4f32 (fp32 operands, fp32 accumulation).
//
// Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
// (abstract; atlas summary "Approach" and "Key results": an MLP fast weight).
// Per (b, h) and chunk, with K, V, Q the chunk's [C x D] token rows and the
// chunk-start weights (W for linear; W1 [Hd x D], W2 [D x Hd] for the MLP):
//   output:     O = Q W^T                     | O = silu(Q W1^T) W2^T
//   forward:    Y = K W^T                     | Z = K W1^T, A = silu(Z), Y = A W2^T
//   loss:       dY = Y - V (MSE)  or  dY = -V (negative dot product)
//   backward:                                 | dZ = (dY W2) * silu'(Z)
//   aggregate:  G_W  = dY^T diag(c) K         | G_W2 = dY^T diag(c) A, G_W1 = dZ^T diag(c) K
//               for c in {cM, cW} (per-token coefficients from e2ttt_logscan)
//   transition: M <- Bb M + G^M,  W <- A W - gamma M_old - G^W
//
// One workgroup of 8 wavefronts per (b, h): the MLP's hidden units are coupled
// through Y, so a head is not split.  The state (W and M) stays in MFMA
// accumulator registers for the whole sequence as 16x16 tiles spread over the
// wavefronts; its aggregation MFMAs accumulate into it directly.  Per chunk
// the chunk-start weights are written to LDS once; per block of up to 64
// tokens the token rows and the intermediates (silu(Z), dY, then dZ) go
// through LDS between the stages.
//
// LDS matrices hold fp32 rows of RS floats (RS a multiple of 64) with element
// (r, c) at r * RS + (c ^ swz(r)).  An MFMA operand read touches either 16
// rows x 4 columns or 4 rows x 16 columns (the same matrix is contracted over
// its rows in one product and over its columns in another); the swizzle puts
// both patterns on 64 distinct banks.
#include "e2ttt_internal.h"

namespace e2ttt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 8;          // wavefronts per workgroup
constexpr int NT = 64 * NW;    // threads per workgroup
constexpr int TBMAX = 64;      // tokens per block
constexpr int MAXT = 4;        // 16x16 tiles per wavefront per matrix
constexpr int MAXY = 2;        // 16x16 tiles per wavefront of a [TB x D] product (D <= 64)

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 4) | (((r >> 2) & 3) << 2); }

// a matrix in LDS
struct Lm {
    float* p;
    int rs;  // row stride in floats (a multiple of 64)
    __device__ __forceinline__ float& at(int r, int c) const { return p[r * rs + (c ^ swz(r))]; }
    __device__ __forceinline__ f32x4* row4(int r, int c4) const {  // 4 floats from column 4 c4, 16-byte aligned
        return (f32x4*)&p[r * rs + ((4 * c4) ^ swz(r))];
    }
};

__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

struct F32Args {
    const float* q;
    const float* k;
    const float* v;
    const float* cM;
    const float* cW;
    const float* scal;
    const float* W0;
    const float* M0;
    float* out;
    float* W;
    float* M;
    float* save;  // [BH][nc][2][P] chunk-start W, M (may be null)
    int64_t T, ldc, P;
    int D, Hd, C, nc, TB;
    int rsd, rsh;  // LDS row strides for D- and Hd-wide rows
};

// tile s of a matrix with ncol 16-wide column tiles: (row tile, column tile)
__device__ __forceinline__ int tr(int s, int ncol) { return s / ncol; }
__device__ __forceinline__ int tc(int s, int ncol) { return s % ncol; }

template <int KIND, int LOSS, bool MOM>
__global__ __launch_bounds__(NT) void f32_chunk_kernel(F32Args a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    int jl = lane & 15, g = lane >> 4;  // made opaque per chunk below (no per-lane address outlives a chunk)
    const int64_t bh = blockIdx.x;
    const int D = a.D, Hd = KIND == E2TTT_MLP ? a.Hd : 0, TB = a.TB;
    const int64_t P = a.P, T = a.T;
    const bool mlp = KIND == E2TTT_MLP;

    // ---------------------------------------------------------------- LDS
    // MLP:    W1s [Hd][rsd] | W2s [D][rsh] | Xs [TB][rsd] | As [TB][rsh] | Ks [TB][rsd] | c [2][TB]
    // linear: Ws [D][rsd]                  | Xs [TB][rsd] |              | Ks [TB][rsd] | c [2][TB]
    // Xs holds a block's Q rows, then (once the output stage has read them) dY;
    // Ks its K rows.
    float* p = lds;
    const Lm W1s{p, a.rsd};
    p += (mlp ? Hd : D) * a.rsd;
    const Lm W2s{p, a.rsh};
    p += mlp ? D * a.rsh : 0;
    const Lm Xs{p, a.rsd};
    p += TB * a.rsd;
    const Lm As{p, a.rsh};
    p += mlp ? TB * a.rsh : 0;
    const Lm Ks{p, a.rsd};
    p += TB * a.rsd;
    const Lm& dYs = Xs;
    float* cms = p;
    float* cws = p + TB;

    // ---------------------------------------------------------------- state
    // matrix 0: W1 [Hd x D] (linear: W [D x D]); matrix 1: W2 [D x Hd].
    // Tile s of matrix m is held by wave s % NW in slot s / NW; lane (jl, g)
    // register r holds element (16 tr + 4g + r, 16 tc + jl).
    const int nr0 = mlp ? Hd / 16 : D / 16, nc0 = D / 16;  // tile rows / columns of matrix 0
    const int nr1 = D / 16, nc1 = mlp ? Hd / 16 : 1;       // of matrix 1 (linear: none)
    const int ns0 = nr0 * nc0, ns1 = mlp ? nr1 * nc1 : 0;
    const int64_t off1 = (int64_t)(mlp ? Hd : D) * D;  // packed offset of matrix 1
    const int cols0 = D, cols1 = Hd;                    // packed row lengths
    f32x4 w0[MAXT], m0[MAXT], w1[MAXT], m1[MAXT];
    auto gidx0 = [&](int s, int r) { return (int64_t)(16 * tr(s, nc0) + 4 * g + r) * cols0 + 16 * tc(s, nc0) + jl; };
    auto gidx1 = [&](int s, int r) {
        return off1 + (int64_t)(16 * tr(s, nc1) + 4 * g + r) * cols1 + 16 * tc(s, nc1) + jl;
    };
    {
        const float* W0 = a.W0 + bh * P;
        const float* M0 = MOM ? a.M0 + bh * P : nullptr;
#pragma unroll
        for (int q = 0; q < MAXT; ++q) {
            const int s0 = wave + NW * q;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                w0[q][r] = s0 < ns0 ? W0[gidx0(s0, r)] : 0.f;
                m0[q][r] = (MOM && s0 < ns0) ? M0[gidx0(s0, r)] : 0.f;
                w1[q][r] = s0 < ns1 ? W0[gidx1(s0, r)] : 0.f;
                m1[q][r] = (MOM && s0 < ns1) ? M0[gidx1(s0, r)] : 0.f;
            }
        }
    }

    const float* qh = a.q + bh * T * D;
    const float* kh = a.k + bh * T * D;
    const float* vh = a.v + bh * T * D;
    float* oh = a.out + bh * T * D;
    const float* cMh = a.cM + bh * a.ldc;
    const float* cWh = a.cW + bh * a.ldc;

    // rows [t, t + nb) of q and k [T][D] -> Xs and Ks, zero rows nb .. TB-1
    auto load_rows = [&](int64_t t, int nb) {
        const int n4 = D / 4;
        for (int i = tid; i < TB * n4; i += NT) {
            const int r = i / n4, c4 = i % n4;
            f32x4 q4 = {0.f, 0.f, 0.f, 0.f}, k4 = q4;
            if (r < nb) {
                q4 = *(const f32x4*)&qh[(t + r) * D + 4 * c4];
                k4 = *(const f32x4*)&kh[(t + r) * D + 4 * c4];
            }
            *Xs.row4(r, c4) = q4;
            *Ks.row4(r, c4) = k4;
        }
    };

    // [TB x N] = X_lds [TB x K] * B^T where B_lds is [N][K] (contraction over
    // columns of both): tiles s = wave + NW q of (TB/16) x (N/16); the result
    // tiles go to fn(q, row tile, col tile, acc).
    auto gemm_rows = [&](const Lm& X, const Lm& B, int N, int K, auto&& fn) {
        const int ncn = N / 16, nst = (TB / 16) * ncn;
        f32x4 acc[MAXT];
        int ti[MAXT], tj[MAXT];
#pragma unroll
        for (int q = 0; q < MAXT; ++q) {
            acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int s = wave + NW * q;
            ti[q] = s < nst ? tr(s, ncn) : 0;
            tj[q] = s < nst ? tc(s, ncn) : 0;
        }
        // k-slot (g, j) of MFMA j in group m is k = 16 m + 4 g + j: each lane
        // reads its 4 k of a group with one 16-byte LDS read per operand.
        // When the column tiles divide the wavefronts, all of a wave's tiles
        // share one column tile and its B operand is read once.
        if (NW % ncn == 0) {
            for (int m = 0; m < K / 16; ++m) {
                f32x4 av[MAXT];
                const f32x4 bv = *B.row4(16 * tj[0] + jl, 4 * m + g);
#pragma unroll
                for (int q = 0; q < MAXT; ++q)
                    if (wave + NW * q < nst) av[q] = *X.row4(16 * ti[q] + jl, 4 * m + g);
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < MAXT; ++q)
                        if (wave + NW * q < nst) acc[q] = mfma(av[q][j], bv[j], acc[q]);
            }
        } else {
            for (int m = 0; m < K / 16; ++m) {
#pragma unroll
                for (int q = 0; q < MAXT; ++q) {
                    if (wave + NW * q < nst) {
                        const f32x4 av = *X.row4(16 * ti[q] + jl, 4 * m + g);
                        const f32x4 bv = *B.row4(16 * tj[q] + jl, 4 * m + g);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[q] = mfma(av[j], bv[j], acc[q]);
                    }
                }
            }
        }
#pragma unroll
        for (int q = 0; q < MAXT; ++q)
            if (wave + NW * q < nst) fn(q, ti[q], tj[q], acc[q]);
    };

    const int nchunks = a.nc;
    for (int c = 0; c < nchunks; ++c) {
        // per-lane tile coordinates are re-derived in every chunk, so that the
        // compiler does not keep dozens of per-tile addresses live across the loop
        asm volatile("" : "+v"(jl), "+v"(g));
        const int64_t t0 = (int64_t)c * a.C;
        const int Cc = (int)min((int64_t)a.C, T - t0);  // the last chunk may be shorter
        __syncthreads();  // the previous chunk's last reads of the weight snapshot are done
        if (a.save) {     // chunk-start state for the backward pass
            float* sv = a.save + (bh * nchunks + c) * 2 * P;
#pragma unroll
            for (int q = 0; q < MAXT; ++q) {
                const int s0 = wave + NW * q;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (s0 < ns0) {
                        sv[gidx0(s0, r)] = w0[q][r];
                        sv[P + gidx0(s0, r)] = MOM ? m0[q][r] : 0.f;
                    }
                    if (s0 < ns1) {
                        sv[gidx1(s0, r)] = w1[q][r];
                        sv[P + gidx1(s0, r)] = MOM ? m1[q][r] : 0.f;
                    }
                }
            }
        }
        // chunk-start weights -> LDS
#pragma unroll
        for (int q = 0; q < MAXT; ++q) {
            const int s0 = wave + NW * q;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (s0 < ns0) W1s.at(16 * tr(s0, nc0) + 4 * g + r, 16 * tc(s0, nc0) + jl) = w0[q][r];
                if (s0 < ns1) W2s.at(16 * tr(s0, nc1) + 4 * g + r, 16 * tc(s0, nc1) + jl) = w1[q][r];
            }
        }
        // transition of the state with the chunk-start momentum; the
        // aggregations below then add G^M to M and subtract G^W from W
        {
            const f32x4 sc = *(const f32x4*)(a.scal + (bh * nchunks + c) * 4);
            const float A = sc[0], Bb = sc[1], gamma = sc[2];
#pragma unroll
            for (int q = 0; q < MAXT; ++q) {
                if (MOM) {
                    w0[q] = A * w0[q] - gamma * m0[q];
                    m0[q] = Bb * m0[q];
                    w1[q] = A * w1[q] - gamma * m1[q];
                    m1[q] = Bb * m1[q];
                } else {
                    w0[q] = A * w0[q];
                    w1[q] = A * w1[q];
                }
            }
        }

        for (int tb0 = 0; tb0 < Cc; tb0 += TB) {
            const int nb = min(TB, Cc - tb0);
            const int64_t tt = t0 + tb0;  // first token of the block
            // ---------------------------------------------------- output
            // the block's Q and K rows, coefficients and this wave's V elements
            // are loaded together: one load latency is exposed per block
            float vr[MAXY][4];  // V at this wave's Y tiles (tiles s = wave + NW q of [TB x D])
            {
                const int ncn = D / 16, nst = (TB / 16) * ncn;
#pragma unroll
                for (int q = 0; q < MAXY; ++q) {
                    const int s = wave + NW * q;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * tr(s, ncn) + 4 * g + r;
                        vr[q][r] = (s < nst && row < nb) ? vh[(tt + row) * D + 16 * tc(s, ncn) + jl] : 0.f;
                    }
                }
            }
            load_rows(tt, nb);
            for (int i = tid; i < TB; i += NT) {
                cms[i] = (MOM && i < nb) ? cMh[tt + i] : 0.f;
                cws[i] = i < nb ? cWh[tt + i] : 0.f;
            }
            __syncthreads();
            auto store_out = [&](int, int ti, int tj, f32x4 o) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * ti + 4 * g + r;
                    if (row < nb) oh[(tt + row) * D + 16 * tj + jl] = o[r];
                }
            };
            if (mlp) {
                // Aq = silu(Q W1^T) -> As
                gemm_rows(Xs, W1s, Hd, D, [&](int, int ti, int tj, f32x4 z) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) As.at(16 * ti + 4 * g + r, 16 * tj + jl) = z[r] * sigm(z[r]);
                });
                __syncthreads();
                gemm_rows(As, W2s, D, Hd, store_out);  // O = Aq W2^T (W2s rows are W2[d][:])
            } else {
                gemm_rows(Xs, W1s, D, D, store_out);  // O = Q W^T
            }
            __syncthreads();
            // ---------------------------------------------------- forward
            float sp[MAXT][4];  // silu'(Z) of this wave's Z tiles
            auto to_dy = [&](int q, int ti, int tj, f32x4 y) {  // dL/dy of this wave's Y tiles -> dYs
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * ti + 4 * g + r, col = 16 * tj + jl;
                    dYs.at(row, col) = LOSS == E2TTT_LOSS_MSE ? y[r] - vr[q & (MAXY - 1)][r] : -vr[q & (MAXY - 1)][r];
                }
            };
            if (mlp) {
                gemm_rows(Ks, W1s, Hd, D, [&](int q, int ti, int tj, f32x4 z) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float s = sigm(z[r]);
                        As.at(16 * ti + 4 * g + r, 16 * tj + jl) = z[r] * s;
                        sp[q][r] = s * (1.f + z[r] * (1.f - s));
                    }
                });
                __syncthreads();
                if (LOSS == E2TTT_LOSS_MSE) {
                    gemm_rows(As, W2s, D, Hd, to_dy);  // Y = A W2^T
                } else {
                    const int ncn = D / 16, nst = (TB / 16) * ncn;
#pragma unroll
                    for (int q = 0; q < MAXY; ++q) {
                        const int s = wave + NW * q;
                        if (s < nst) to_dy(q, tr(s, ncn), tc(s, ncn), f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                }
            } else {
                if (LOSS == E2TTT_LOSS_MSE) {
                    gemm_rows(Ks, W1s, D, D, to_dy);  // Y = K W^T
                } else {
                    const int ncn = D / 16, nst = (TB / 16) * ncn;
#pragma unroll
                    for (int q = 0; q < MAXY; ++q) {
                        const int s = wave + NW * q;
                        if (s < nst) to_dy(q, tr(s, ncn), tc(s, ncn), f32x4{0.f, 0.f, 0.f, 0.f});
                    }
                }
            }
            __syncthreads();
            // ---------------------------------------------------- aggregation, matrix 1
            // MLP W2 [D x Hd]: M += (cM dY)^T A, W -= (cW dY)^T A
            if (mlp) {
#pragma unroll 2
                for (int kk = 0; kk < TB / 4; ++kk) {
                    const int tok = 4 * kk + g;
                    const float cm = cms[tok], cw = cws[tok];
#pragma unroll
                    for (int q = 0; q < MAXT; ++q) {
                        const int s = wave + NW * q;
                        if (s < ns1) {
                            const float y = dYs.at(tok, 16 * tr(s, nc1) + jl);
                            const float b = As.at(tok, 16 * tc(s, nc1) + jl);
                            if (MOM) m1[q] = mfma(cm * y, b, m1[q]);
                            w1[q] = mfma(-cw * y, b, w1[q]);
                        }
                    }
                }
                __syncthreads();  // every wave is done with A
                // ------------------------------------------------ backward: dZ = (dY W2) * silu'(Z) -> As
                const int ncn = Hd / 16, nst = (TB / 16) * ncn;
                f32x4 dz[MAXT];
#pragma unroll
                for (int q = 0; q < MAXT; ++q) dz[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
                for (int kk = 0; kk < D / 4; ++kk) {
#pragma unroll
                    for (int q = 0; q < MAXT; ++q) {
                        const int s = wave + NW * q;
                        if (s < nst)
                            dz[q] = mfma(dYs.at(16 * tr(s, ncn) + jl, 4 * kk + g),
                                         W2s.at(4 * kk + g, 16 * tc(s, ncn) + jl), dz[q]);
                    }
                }
#pragma unroll
                for (int q = 0; q < MAXT; ++q) {
                    const int s = wave + NW * q;
                    if (s < nst)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            As.at(16 * tr(s, ncn) + 4 * g + r, 16 * tc(s, ncn) + jl) = dz[q][r] * sp[q][r];
                }
                __syncthreads();
            }
            // matrix 0: MLP W1 [Hd x D]: M += (cM dZ)^T K, W -= (cW dZ)^T K;
            //           linear W [D x D]: M += (cM dY)^T K, W -= (cW dY)^T K
            {
                const Lm& G = mlp ? As : dYs;
#pragma unroll 2
                for (int kk = 0; kk < TB / 4; ++kk) {
                    const int tok = 4 * kk + g;
                    const float cm = cms[tok], cw = cws[tok];
#pragma unroll
                    for (int q = 0; q < MAXT; ++q) {
                        const int s = wave + NW * q;
                        if (s < ns0) {
                            const float x = G.at(tok, 16 * tr(s, nc0) + jl);
                            const float b = Ks.at(tok, 16 * tc(s, nc0) + jl);
                            if (MOM) m0[q] = mfma(cm * x, b, m0[q]);
                            w0[q] = mfma(-cw * x, b, w0[q]);
                        }
                    }
                }
            }
            __syncthreads();  // Xs, As, dYs are rewritten by the next block
        }
    }
    // final state
    asm volatile("" : "+v"(jl), "+v"(g));
    {
        float* W = a.W + bh * P;
        float* M = MOM ? a.M + bh * P : nullptr;
#pragma unroll
        for (int q = 0; q < MAXT; ++q) {
            const int s0 = wave + NW * q;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (s0 < ns0) {
                    W[gidx0(s0, r)] = w0[q][r];
                    if (MOM) M[gidx0(s0, r)] = m0[q][r];
                }
                if (s0 < ns1) {
                    W[gidx1(s0, r)] = w1[q][r];
                    if (MOM) M[gidx1(s0, r)] = m1[q][r];
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// The MLP split over its hidden units: for heads too few to fill the chip,
// the hidden units of a head go to S = Hd / 16 workgroups (16 units each),
// which run the whole sequence in one launch.  Step L (L = 0 .. nc) finishes
// chunk L - 1 and starts chunk L:
//   finish: Y = sum of the S slices' partial Y (fixed order), dY = Y - V;
//           dZ_s = (dY W2_s) silu'(Z_s); the slice's aggregations
//           G_W2_s = dY^T diag(c) A_s, G_W1_s = dZ_s^T diag(c) K and its
//           transition; the output rows r = s, s + S, ... as the sum of the
//           slices' partial outputs;
//   start:  Z_s = K W1_s^T, A_s = silu(Z_s) (kept for the finish), the
//           partial Y_s = A_s W2_s^T and the partial output
//           silu(Q W1_s^T) W2_s^T.
// The slices of a head meet once per step: a slice publishes its partial sums
// (stores, a device-scope release, then an increment of the head's arrival
// counter) and the next step's finish waits until all S slices have arrived.
// Partial sums are double-buffered by chunk parity: a slice overwrites a
// buffer only after every slice has arrived once more, i.e. has finished
// reading it.  A slice's state stays in registers for the whole sequence,
// and its K rows, A_s and chunk-start W2_s stay in LDS from the start of a
// chunk to its finish.
//
// All S workgroups of a head must run at the same time: the launch holds at
// most one workgroup per compute unit.  A wait gives up after 10 s of wall
// time (which only a device that cannot run the whole grid at once could
// reach); it then raises the flag word after the counters, stops waiting for
// the rest of the call and the workgroup writes NaN into its final state.
// The counters and the flag are zeroed by a one-workgroup kernel before the
// loop on the same stream.
// ---------------------------------------------------------------------------
constexpr int SNW = 8;         // wavefronts per split workgroup: two groups of 4
constexpr int SNT = 64 * SNW;
constexpr int HS = 16;         // hidden units per split workgroup
constexpr int SMAX = 8;        // slices per head (Hd <= 128)
constexpr int RPT = 2;         // 16-byte pieces of a [TB][D] block per thread (TB * D <= 4096)
// A slice writes output rows sl, sl + S, ...: with S >= 2 at most TB / 2 rows
// of D / 4 pieces, one piece per thread.
static_assert(SNT >= (64 / 2) * (64 / 4), "output rows of a slice: one 16-byte piece per thread");
constexpr uint64_t kSpinTicks = 1000000000ull;  // 10 s of the 100 MHz wall clock

struct SplitArgs {
    const float* q;
    const float* k;
    const float* v;
    const float* cM;
    const float* cW;
    const float* scal;
    const float* W0;
    const float* M0;
    float* out;
    float* W;
    float* M;
    float* save;   // [BH][nc][2][P] chunk-start W, M (may be null)
    float* ypart;  // [2][BH][S][TB][D] partial Y of each slice (parity of the chunk)
    float* opart;  // [2][BH][S][TB][D] partial outputs
    unsigned* sync;  // [BH] arrival counters, then the time-out flag
    int64_t T, ldc, P;
    int D, Hd, C, nc, TB, S;
    int xcd_map, nwg;
};

__global__ void split_sync_init(unsigned* sync, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) sync[i] = 0u;
}

template <int LOSS, bool MOM>
__global__ void __attribute__((amdgpu_flat_work_group_size(SNT, SNT), amdgpu_waves_per_eu(2, 2)))
f32_split_kernel(SplitArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ unsigned gave_up;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, jl = lane & 15, g = lane >> 4;
    // the S slices of one head run on one XCD (consecutive ids land on
    // different XCDs, so remap)
    int L_id = blockIdx.x;
    if (a.xcd_map) L_id = (blockIdx.x % 8) * (a.nwg / 8) + blockIdx.x / 8;
    const int64_t bh = L_id / a.S;
    const int sl = L_id % a.S;  // this workgroup's slice: hidden units 16 sl .. 16 sl + 15
    const int D = a.D, Hd = a.Hd, TB = a.TB, S = a.S;
    const int64_t P = a.P, T = a.T;
    const int nd = D / 16;  // tiles along D
    const int64_t off1 = (int64_t)Hd * D;
    unsigned* const cnt = a.sync + bh;      // this head's arrival counter
    unsigned* const flag = a.sync + a.nwg / S;  // after the BH counters

    // LDS: W1s [16][64] | W2s [D][64] | Ks [TB][64] | Qs [TB][64] (Q, or dY) | Ab [TB][64] (A, or dZ) | Aq [TB][64] | c [2][TB]
    float* p = lds;
    const Lm W1s{p, 64};
    p += HS * 64;
    const Lm W2s{p, 64};
    p += D * 64;
    const Lm Ks{p, 64};
    p += TB * 64;
    const Lm Qs{p, 64};
    p += TB * 64;
    const Lm Ab{p, 64};
    p += TB * 64;
    const Lm Aq{p, 64};
    p += TB * 64;
    float* cms = p;
    float* cws = p + TB;

    // Two groups of four wavefronts, wl = wave % 4 within the group:
    //   group 0 holds the W1_s tile (units, d 16 wl ..) and its momentum, and
    //     computes token tile wl's dA / dZ, its G_W1 tile, Z and partial Y;
    //   group 1 holds the W2_s tile (d 16 wl .., units) and its momentum, and
    //     computes its G_W2 tile, token tile wl's Zq and partial output.
    // So the W2 aggregation overlaps dA, and Z overlaps Zq.
    const int grp = wave >> 2, wl = wave & 3;
    const bool st = wl < nd;
    const bool tt = wl < TB / 16;  // owns token tile wl
    f32x4 w = {0.f, 0.f, 0.f, 0.f}, m = w;
    // packed index of element r of this wave's state tile
    auto ix = [&](int r, int jl_, int g_) {
        return grp == 0 ? (int64_t)(HS * sl + 4 * g_ + r) * D + 16 * wl + jl_
                        : off1 + (int64_t)(16 * wl + 4 * g_ + r) * Hd + HS * sl + jl_;
    };
    if (st) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w[r] = a.W0[bh * P + ix(r, jl, g)];
            if (MOM) m[r] = a.M0[bh * P + ix(r, jl, g)];
        }
    }
    if (tid == 0) gave_up = 0u;
    const int64_t slot = bh * S + sl;
    const size_t part = (size_t)TB * D;                // floats of one slice's partial
    const size_t parity = (size_t)(gridDim.x) * part;  // all slices' partials of one chunk parity
    const int n4 = D / 4;
    float sp[4] = {0.f, 0.f, 0.f, 0.f};  // group 0: silu'(Z) of the chunk last started at token tile wl (rows 16 wl + 4g + r, unit jl)

    // until all S slices of the head have arrived `target` times in total.
    // The cache maintenance of a device-scope acquire (invalidation) and
    // release (L2 write-back) acts on whole caches, so one wavefront of the
    // workgroup issues it, ordered with the others' accesses by the
    // workgroup barrier (and, for the release, their own wait for their stores).
    auto wait_head = [&](unsigned target) {
        if (tid == 0 && !gave_up) {
            const uint64_t t0 = wall_clock64();
            while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                    wall_clock64() - t0 > kSpinTicks) {
                    __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    gave_up = 1u;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        if (wave == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
    };
    // this slice's partial sums of the step are visible device-wide, then it arrives
    auto publish = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's stores are done
        __syncthreads();
        if (wave == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (tid == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    for (int L = 0; L <= a.nc; ++L) {
        // lane coordinates re-derived in every step: otherwise the compiler
        // keeps dozens of per-lane 64-bit addresses live across the loop
        int tid_s = threadIdx.x;
        asm volatile("" : "+v"(tid_s));
        const int tid = tid_s, lane = tid & 63, jl = lane & 15, g = lane >> 4;
        auto rows = [&](const float* x, int64_t t, int nb, f32x4 (&v4)[RPT]) {
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int i = tid + SNT * u, r = i / n4;
                v4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (i < TB * n4 && r < nb) v4[u] = *(const f32x4*)&x[(bh * T + t + r) * D + 4 * (i % n4)];
            }
        };
        // the columns 16 wl .. 16 wl + 15 of a chunk's rows (wave wl < nd of a
        // group; 4 pieces of 4 floats per lane): piece p = lane + 64 u is row
        // p / 4, column chunk 4 wl + p % 4
        auto rows_tile = [&](const float* x, int64_t t, int nb, f32x4 (&v4)[4]) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pc = lane + 64 * u, r = pc >> 2, c4 = 4 * wl + (pc & 3);
                v4[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (st && r < TB && r < nb) v4[u] = *(const f32x4*)&x[(bh * T + t + r) * D + 4 * c4];
            }
        };
        const bool fin = L >= 1, sta = L < a.nc;
        const int cf = L - 1, cs = L;  // the chunk finished, the chunk started
        const int64_t tf = (int64_t)cf * a.C, ts = (int64_t)cs * a.C;
        const int nbf = fin ? (int)min((int64_t)a.C, T - tf) : 0, nbs = sta ? (int)min((int64_t)a.C, T - ts) : 0;
        const int nr = fin ? (nbf - sl + S - 1) / S : 0;  // output rows r = sl, sl + S, ... of the finished chunk
        const int orow = sl + S * (tid / n4), oc4 = tid % n4;

        // ------------------------------------------------------------ the step's loads: own rows first
        f32x4 vf[RPT];
        f32x4 xs[4];  // the started chunk's K rows (group 0) or Q rows (group 1), columns of d-tile wl
        f32x4 ysum[RPT];                    // the finished chunk's Y summed over the slices (fixed order)
        f32x4 osum = {0.f, 0.f, 0.f, 0.f};  // one piece of its output rows
        float cmv = 0.f, cwv = 0.f;
        if (fin) {
            rows(a.v, tf, nbf, vf);
            if (tid < TB && tid < nbf) {
                if (MOM) cmv = a.cM[bh * a.ldc + tf + tid];
                cwv = a.cW[bh * a.ldc + tf + tid];
            }
        }
        if (sta) rows_tile(grp == 0 ? a.k : a.q, ts, nbs, xs);
        if (fin) {
            wait_head((unsigned)(S * L));  // every slice has published chunk L - 1
            const float* yp = a.ypart + (size_t)(cf & 1) * parity + (size_t)bh * S * part;
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int i = tid + SNT * u;
                f32x4 ys[SMAX];
#pragma unroll
                for (int s2 = 0; s2 < SMAX; ++s2)
                    if (s2 < S && i < TB * n4) ys[s2] = *(const f32x4*)&yp[s2 * part + 4 * i];
                ysum[u] = ys[0];
#pragma unroll
                for (int s2 = 1; s2 < SMAX; ++s2)
                    if (s2 < S) ysum[u] += ys[s2];
            }
            if (tid < nr * n4) {
                const float* op = a.opart + (size_t)(cf & 1) * parity + (size_t)bh * S * part;
                f32x4 os[SMAX];
#pragma unroll
                for (int s2 = 0; s2 < SMAX; ++s2)
                    if (s2 < S) os[s2] = *(const f32x4*)&op[s2 * part + orow * D + 4 * oc4];
                osum = os[0];
#pragma unroll
                for (int s2 = 1; s2 < SMAX; ++s2)
                    if (s2 < S) osum += os[s2];
            }
        }

        // ------------------------------------------------------------ finish chunk L - 1
        // (Ks, Ab and W2s still hold its K rows, A_s and chunk-start W2_s)
        if (fin) {
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int i = tid + SNT * u;
                if (i < TB * n4) *Qs.row4(i / n4, i % n4) = LOSS == E2TTT_LOSS_MSE ? ysum[u] - vf[u] : -vf[u];  // dY
            }
            if (tid < TB) {
                cms[tid] = cmv;
                cws[tid] = cwv;
            }
            if (tid < nr * n4) *(f32x4*)&a.out[(bh * T + tf + orow) * D + 4 * oc4] = osum;
            __syncthreads();
            // transition with the chunk-start momentum; the aggregations add G
            {
                const f32x4 sc = *(const f32x4*)(a.scal + (bh * a.nc + cf) * 4);
                if (MOM) {
                    w = sc[0] * w - sc[2] * m;
                    m = sc[1] * m;
                } else {
                    w = sc[0] * w;
                }
            }
            // (the short contractions below run on 4 independent accumulators,
            // k-step kk on accumulator kk % 4, summed in a fixed order)
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            if (grp == 0) {
                // dA = dY W2_s on token tile wl, dZ = dA silu'(Z), parked in Aq
                if (tt) {
                    f32x4 acc[4] = {z4, z4, z4, z4};
                    for (int k4 = 0; k4 < D / 16; ++k4)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int kk = 4 * k4 + j;
                            acc[j] = mfma(Qs.at(16 * wl + jl, 4 * kk + g), W2s.at(4 * kk + g, jl), acc[j]);
                        }
                    const f32x4 dz = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) Aq.at(16 * wl + 4 * g + r, jl) = dz[r] * sp[r];
                }
            } else if (st) {
                // G_W2_s tile (d 16 wl .., units): M += (cM dY)^T A, W -= (cW dY)^T A
                f32x4 am[4] = {z4, z4, z4, z4}, aw[4] = {z4, z4, z4, z4};
                for (int k4 = 0; k4 < TB / 16; ++k4)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int tok = 16 * k4 + 4 * j + g;
                        const float y = Qs.at(tok, 16 * wl + jl), b = Ab.at(tok, jl);
                        if (MOM) am[j] = mfma(cms[tok] * y, b, am[j]);
                        aw[j] = mfma(-cws[tok] * y, b, aw[j]);
                    }
                if (MOM) m += (am[0] + am[1]) + (am[2] + am[3]);
                w += (aw[0] + aw[1]) + (aw[2] + aw[3]);
            }
            __syncthreads();  // dZ is in Aq; dY, A and W2s are no longer read
            if (grp == 0 && st) {
                // G_W1_s tile (units, d 16 wl ..): M += (cM dZ)^T K, W -= (cW dZ)^T K
                f32x4 am[4] = {z4, z4, z4, z4}, aw[4] = {z4, z4, z4, z4};
                for (int k4 = 0; k4 < TB / 16; ++k4)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int tok = 16 * k4 + 4 * j + g;
                        const float x = Aq.at(tok, jl), b = Ks.at(tok, 16 * wl + jl);
                        if (MOM) am[j] = mfma(cms[tok] * x, b, am[j]);
                        aw[j] = mfma(-cws[tok] * x, b, aw[j]);
                    }
                if (MOM) m += (am[0] + am[1]) + (am[2] + am[3]);
                w += (aw[0] + aw[1]) + (aw[2] + aw[3]);
            }
        }
        if (!sta) break;

        // ------------------------------------------------------------ start chunk L
        if (a.save && st) {  // chunk-start state for the backward pass
            float* sv = a.save + (bh * a.nc + cs) * 2 * P;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sv[ix(r, jl, g)] = w[r];
                sv[P + ix(r, jl, g)] = MOM ? m[r] : 0.f;
            }
        }
        if (st) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (grp == 0)
                    W1s.at(4 * g + r, 16 * wl + jl) = w[r];
                else
                    W2s.at(16 * wl + 4 * g + r, jl) = w[r];
            }
        }
        // group 1 writes Q rows and W2s while group 0 still reads K rows and
        // dZ for its W1 aggregation.  Group 0's wavefront wl writes the K-row
        // columns of its own d-tile, the only ones its W1 aggregation reads,
        // after that aggregation.
        if (st) {
            const Lm& Xs = grp == 0 ? Ks : Qs;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pc = lane + 64 * u, r = pc >> 2;
                if (r < TB) *Xs.row4(r, 4 * wl + (pc & 3)) = xs[u];
            }
        }
        __syncthreads();
        // group 0: Z_s = K W1_s^T on token tile wl, A_s = silu(Z_s) into Ab,
        // then the partial Y_s = A_s W2_s^T of those rows; group 1 the same
        // with Q: Zq, silu(Zq) into Aq, the partial output.  Each wavefront
        // reads back only the rows it wrote.
        if (tt) {
            const Lm& X = grp == 0 ? Ks : Qs;
            const Lm& Act = grp == 0 ? Ab : Aq;
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            f32x4 za[4] = {z4, z4, z4, z4};
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
                if (mm < D / 16) {
                    const f32x4 xv = *X.row4(16 * wl + jl, 4 * mm + g);
                    const f32x4 wv = *W1s.row4(jl, 4 * mm + g);
#pragma unroll
                    for (int j = 0; j < 4; ++j) za[j] = mfma(xv[j], wv[j], za[j]);
                }
            }
            const f32x4 z = (za[0] + za[1]) + (za[2] + za[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * wl + 4 * g + r;
                const float s1 = sigm(z[r]);
                Act.at(row, jl) = z[r] * s1;
                if (grp == 0) sp[r] = s1 * (1.f + z[r] * (1.f - s1));
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's rows are written
            asm volatile("" ::: "memory");
            float* dst = (grp == 0 ? a.ypart : a.opart) + (size_t)(cs & 1) * parity + (size_t)slot * part;
            const f32x4 av = *Act.row4(16 * wl + jl, g);
            for (int tj = 0; tj < nd; ++tj) {
                const f32x4 wv = *W2s.row4(16 * tj + jl, g);
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) y = mfma(av[j], wv[j], y);
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * wl + 4 * g + r) * D + 16 * tj + jl] = y[r];
            }
        }
        publish();
    }
    if (gave_up)  // the synchronisation was abandoned: mark the result invalid
        w = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    if (st) {
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        const int jl_e = lane_e & 15, g_e = lane_e >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            a.W[bh * P + ix(r, jl_e, g_e)] = w[r];
            if (MOM) a.M[bh * P + ix(r, jl_e, g_e)] = m[r];
        }
    }
}

constexpr size_t kLdsMax = 160 * 1024;

int rs_of(int64_t cols) { return (int)((cols + 63) / 64 * 64); }

int f32_block(const e2ttt_desc& d) { return (int)(d.chunk >= TBMAX ? TBMAX : (d.chunk + 15) / 16 * 16); }

size_t f32_lds_bytes(const e2ttt_desc& d) {
    const int64_t TB = f32_block(d), rsd = rs_of(d.D);
    if (d.kind == E2TTT_MLP) {
        const int64_t rsh = rs_of(d.Hd);
        return (size_t)(d.Hd * rsd + d.D * rsh + TB * rsd + TB * rsh + TB * rsd + 2 * TB) * 4;
    }
    return (size_t)(d.D * rsd + 2 * TB * rsd + 2 * TB) * 4;
}

template <int KIND, int LOSS>
hipError_t launch_kl(const e2ttt_desc& d, const F32Args& a, hipStream_t s) {
    const size_t shmem = f32_lds_bytes(d);
    const bool mom = !(d.flags & E2TTT_FLAG_NO_MOMENTUM);
    const void* f = mom ? (const void*)f32_chunk_kernel<KIND, LOSS, true> : (const void*)f32_chunk_kernel<KIND, LOSS, false>;
    if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem) != hipSuccess)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(d.B * d.H)), block(NT);
    if (mom)
        hipLaunchKernelGGL((f32_chunk_kernel<KIND, LOSS, true>), grid, block, shmem, s, a);
    else
        hipLaunchKernelGGL((f32_chunk_kernel<KIND, LOSS, false>), grid, block, shmem, s, a);
    return hipGetLastError();
}

}  // namespace

bool f32_mfma_supported(const e2ttt_desc& d) {
    if (d.io_dtype != E2TTT_F32) return false;
    if (d.kind != E2TTT_LINEAR && d.kind != E2TTT_MLP) return false;
    if (d.D < 16 || d.D % 16 || d.D > 64) return false;
    const int64_t TB = f32_block(d);
    const int64_t nsd = d.D / 16;
    if (d.kind == E2TTT_MLP) {
        if (d.Hd < 16 || d.Hd % 16) return false;
        const int64_t nsh = d.Hd / 16;
        // state, Z / dZ and output tiles per wavefront
        if (nsh * nsd > NW * MAXT || (TB / 16) * nsh > NW * MAXT || (TB / 16) * nsd > NW * MAXT) return false;
    } else {
        if (nsd * nsd > NW * MAXT || (TB / 16) * nsd > NW * MAXT) return false;
    }
    return f32_lds_bytes(d) <= kLdsMax;
}

bool f32_split(const e2ttt_desc& d) {
    if (d.kind != E2TTT_MLP || !f32_mfma_supported(d)) return false;
    if (d.chunk > TBMAX || d.Hd / HS < 2 || d.Hd / HS > SMAX) return false;
    // worth it while the heads leave most of the chip idle and the slices of
    // all heads fit on the compute units at once
    return d.B * d.H * (d.Hd / HS) <= 256;
}

size_t f32_split_bytes(const e2ttt_desc& d) {
    if (!f32_split(d)) return 0;
    const size_t BH = (size_t)(d.B * d.H), S = (size_t)(d.Hd / HS), TB = (size_t)f32_block(d);
    // partial Y and outputs (two parities), the heads' arrival counters and the flag
    return (4 * (2 * BH * S * TB * d.D * 2 + BH + 1) + 255) / 256 * 256;
}

namespace {
size_t split_lds_bytes(const e2ttt_desc& d) {
    const size_t TB = (size_t)f32_block(d);
    return (HS * 64 + d.D * 64 + 4 * TB * 64 + 2 * TB) * 4;
}

template <int LOSS, bool MOM>
hipError_t launch_split(const e2ttt_desc& d, SplitArgs a, hipStream_t s) {
    const size_t shmem = split_lds_bytes(d);
    const void* f = (const void*)f32_split_kernel<LOSS, MOM>;
    if (shmem > 64 * 1024 && hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem) != hipSuccess)
        return hipErrorInvalidValue;
    const int nsync = a.nwg / a.S + 1;
    hipLaunchKernelGGL(split_sync_init, dim3(1), dim3(256), 0, s, a.sync, nsync);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((f32_split_kernel<LOSS, MOM>), dim3((unsigned)a.nwg), dim3(SNT), shmem, s, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_f32_mfma(const e2ttt_desc& d, const void* q, const void* k, const void* v, const float* cM,
                           const float* cW, int64_t ldc, const float* scal, const float* W0, const float* M0, void* out,
                           float* W_end, float* M_end, hipStream_t s, float* save, void* split_ws) {
    // the hidden-slice split needs all its workgroups resident at once (one per
    // compute unit); on a device with fewer compute units the heads run whole
    int ncu = 0;
    if (f32_split(d)) {
        const hipError_t e = device_cu_count(&ncu);
        if (e != hipSuccess) return e;
    }
    if (f32_split(d) && d.B * d.H * (d.Hd / HS) <= ncu) {
        SplitArgs a;
        a.q = (const float*)q;
        a.k = (const float*)k;
        a.v = (const float*)v;
        a.cM = cM;
        a.cW = cW;
        a.scal = scal;
        a.W0 = W0;
        a.M0 = M0;
        a.out = (float*)out;
        a.W = W_end;
        a.M = M_end;
        a.save = save;
        a.T = d.T;
        a.ldc = ldc;
        a.P = e2ttt_param_count(&d);
        a.D = (int)d.D;
        a.Hd = (int)d.Hd;
        a.C = (int)d.chunk;
        a.nc = (int)((d.T + d.chunk - 1) / d.chunk);
        a.TB = f32_block(d);
        a.S = (int)(d.Hd / HS);
        a.nwg = (int)(d.B * d.H * a.S);
        a.xcd_map = a.nwg % 8 == 0 ? 1 : 0;
        const size_t part = (size_t)a.nwg * a.TB * a.D;
        a.ypart = (float*)split_ws;
        a.opart = a.ypart + 2 * part;
        a.sync = (unsigned*)(a.opart + 2 * part);
        const bool mom = !(d.flags & E2TTT_FLAG_NO_MOMENTUM);
        if (d.loss == E2TTT_LOSS_MSE)
            return mom ? launch_split<E2TTT_LOSS_MSE, true>(d, a, s) : launch_split<E2TTT_LOSS_MSE, false>(d, a, s);
        return mom ? launch_split<E2TTT_LOSS_NEGDOT, true>(d, a, s) : launch_split<E2TTT_LOSS_NEGDOT, false>(d, a, s);
    }
    F32Args a;
    a.q = (const float*)q;
    a.k = (const float*)k;
    a.v = (const float*)v;
    a.cM = cM;
    a.cW = cW;
    a.scal = scal;
    a.W0 = W0;
    a.M0 = M0;
    a.out = (float*)out;
    a.W = W_end;
    a.M = M_end;
    a.save = save;
    a.T = d.T;
    a.ldc = ldc;
    a.P = e2ttt_param_count(&d);
    a.D = (int)d.D;
    a.Hd = d.kind == E2TTT_MLP ? (int)d.Hd : 0;
    a.C = (int)d.chunk;
    a.nc = (int)((d.T + d.chunk - 1) / d.chunk);
    a.TB = f32_block(d);
    a.rsd = rs_of(d.D);
    a.rsh = d.kind == E2TTT_MLP ? rs_of(d.Hd) : 64;
    if (d.kind == E2TTT_MLP)
        return d.loss == E2TTT_LOSS_MSE ? launch_kl<E2TTT_MLP, E2TTT_LOSS_MSE>(d, a, s)
                                        : launch_kl<E2TTT_MLP, E2TTT_LOSS_NEGDOT>(d, a, s);
    return d.loss == E2TTT_LOSS_MSE ? launch_kl<E2TTT_LINEAR, E2TTT_LOSS_MSE>(d, a, s)
                                    : launch_kl<E2TTT_LINEAR, E2TTT_LOSS_NEGDOT>(d, a, s);
}

}  // namespace e2ttt

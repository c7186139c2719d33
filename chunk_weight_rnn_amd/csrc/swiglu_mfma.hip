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
// across all chunks: the epilogue never touches HBM.
//
// gfx950 specifics used here:
//   * K and V token blocks are copied HBM -> LDS by global_load_lds_dwordx4
//     (no registers), one block ahead of use, into a row-major layout;
//   * the grad GEMMs read K/V rows from it with ds_read_b128 and the
//     aggregation reads K^T / V^T fragments from the same buffer with the
//     LDS transpose read ds_read_b64_tr_b16 (within a 16-lane group, lane p
//     loads row p/4, columns 4(p%4)..+3, and lane i receives 4 consecutive
//     rows of column i), so nothing is ever written transposed;
//   * every LDS layout uses an XOR swizzle of 16-byte chunks instead of
//     padding, chosen so both the row reads and the transpose reads are
//     bank-conflict free.
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
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int D = 128;   // head dim
constexpr int S = 64;    // hidden units per workgroup slice
constexpr int CB = 64;   // tokens per block inside a chunk
constexpr int NT = 256;  // 4 wavefronts

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

__device__ __forceinline__ float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// 16-byte chunk swizzle of a 256-byte row t (row-major [t][128] bf16): the 8
// rows read at one chunk by 8 lanes of ds_read_b128 land in 8 different bank
// groups, and so do the 4 rows x 2 chunks of one 16-lane transpose read.
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// 32x16 MFMA operand fragment transposed out of a swizzled row-major
// [rows][128] bf16 LDS buffer: operand row = source column col0 + lane%32,
// operand k 0..3 = source rows rbase0..+3, k 4..7 = source rows rbase1..+3.
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* buf, int rbase0, int rbase1, int col0, int lane) {
    const int p = lane & 15, G = lane >> 4;
    const int col = col0 + 16 * (G & 1) + 4 * (p & 3);
    const int chunk = col >> 3;
    const int half = p & 1;
    const int r0 = rbase0 + (p >> 2);
    const int r1 = rbase1 + (p >> 2);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(buf + r0 * 256 + 16 * (chunk ^ swz(r0)) + 8 * half));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(buf + r1 * 256 + 16 * (chunk ^ swz(r1)) + 8 * half));
    bf16x8 r;
    r[0] = lo[0];
    r[1] = lo[1];
    r[2] = lo[2];
    r[3] = lo[3];
    r[4] = hi[0];
    r[5] = hi[1];
    r[6] = hi[2];
    r[7] = hi[3];
    return r;
}

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

// LDS of the loop kernel (bytes): exactly the 160 KB of a gfx950 CU
constexpr int KV_BYTES = 64 * 256;             // one [64 tokens][128] bf16 matrix
constexpr int OFF_KV = 0;                      // [2 buffers][K, V]
constexpr int OFF_DT = OFF_KV + 4 * KV_BYTES;  // [6][64 hidden][64 tokens] bf16 scaled factors
constexpr int DT_BYTES = 6 * 64 * 128;
constexpr int OFF_WS = OFF_DT + DT_BYTES;      // [3][64 hidden][128 d] bf16 chunk-start weights
constexpr int LOOP_LDS = OFF_WS + 3 * 64 * 256;
static_assert(LOOP_LDS == 160 * 1024, "loop kernel LDS budget");

__device__ __forceinline__ int kv_off(int buf, int mat, int t, int chunk) {
    return OFF_KV + (2 * buf + mat) * KV_BYTES + t * 256 + 16 * (chunk ^ swz(t));
}
// scaled factors: row j holds 64 tokens = 8 chunks, swizzled by j
__device__ __forceinline__ int dt_off(int ty, int j, int chunk) {
    return OFF_DT + ty * 8192 + j * 128 + 16 * (chunk ^ (j & 7));
}
// chunk-start weight slices W1^T, W3^T, W2 rows: [3][64 hidden][128 d], swizzled by j
__device__ __forceinline__ int ws_off(int m, int j, int chunk) {
    return OFF_WS + m * 16384 + j * 256 + 16 * (chunk ^ (j & 7));
}

// tile element (lane l, register r) of a 32x32 MFMA accumulator:
//   col = l % 32, row = 8*(r/4) + 4*(l/32) + r%4
//
// State ownership: wave w owns row tiles {rt0, rt0+1} (rt0 = 2(w&1)) of D
// and hidden half hh = w>>1 of the slice, for all three matrices:
// acc[rr][2m] / acc[rr][2m+1] are the M / W parts of matrix m
// (0: W1, 1: W3, 2: W2 held transposed as [d][j]).

// State tiles <-> packed fp32 parameters (W1 [D][Hd] | W3 [D][Hd] | W2 [Hd][D]).
template <bool STORE>
__device__ __forceinline__ void state_io(f32x16 (&acc)[2][6], float* W, float* M, int rt0, int h, int j0, int Hd,
                                         unsigned laneA, unsigned laneB) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dr = 32 * (rt0 + rr) + 8 * (r / 4) + (r % 4);  // uniform part of d
                float* wb;
                float* mb;
                unsigned lo;
                if (p < 2) {
                    const int64_t ub = (int64_t)p * D * Hd + (int64_t)dr * Hd + j0 + 32 * h;
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

__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
swiglu_loop_kernel(LoopArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[LOOP_LDS];
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

    const int rt0 = 2 * (wave & 1), hh = wave >> 1;  // state / aggregation ownership
    const int gr = wave >> 1, gc = wave & 1;         // grad: token rows 32gr.., hidden cols 32gc..

    // HBM -> LDS copy of one token block's K and V rows: wave w moves rows
    // [16w, 16w+16) of both, 4 rows (1 KB) per instruction; lane L writes row
    // r0 + L/16 at physical chunk L%16, which holds logical chunk (L%16)^swz(row).
    auto issue_kv = [&](int blk, int buf) {
        const int64_t tb = (int64_t)blk * CB;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const __bf16* src = m == 0 ? kb : vb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r0 = 16 * wave + 4 * i;
                const int row = r0 + (lane >> 4);
                const int c = (lane & 15) ^ swz(row);
                __builtin_amdgcn_global_load_lds((const void*)(src + (tb + row) * D + 8 * c),
                                                 (lds_void_t*)(smem + OFF_KV + (2 * buf + m) * KV_BYTES + r0 * 256),
                                                 16, 0, 0);
            }
        }
    };

    f32x16 acc[2][6];
    const unsigned laneA = (unsigned)(4 * lg * Hd + li);
    const unsigned laneB = (unsigned)(li * D + 4 * lg);
    state_io<false>(acc, (float*)a.W0 + bh * P, (float*)a.M0 + bh * P, rt0, hh, j0, Hd, laneA, laneB);

    const int nblk = (int)(T / CB);
    const int bpc = a.C / CB;

    issue_kv(0, 0);
    wait_vmem();
    __syncthreads();

    for (int blk = 0; blk < nblk; ++blk) {
        const int buf = blk & 1;
        const bool more = blk + 1 < nblk;
        if (blk % bpc == 0) {
            // ---- chunk start: bf16 weights -> LDS operand slices + global snapshot; rescale state
            const int c = blk / bpc;
            const float* sc = a.scal + (bh * a.nc + c) * 4;
            const float A = sc[0], Bb = sc[1], gamma = sc[2];
            __bf16* snap = a.snap + (bh * a.nc + c) * P;
            const int jl = 32 * hh + li;
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                __bf16* base = snap + (int64_t)m * Hd * D + (int64_t)(j0 + 32 * hh) * D + 32 * rt0 + li * D + 4 * lg;
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const f32x16 w = acc[rr][2 * m + 1];
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        const bf16x4 v4 = pack4(w[4 * qd], w[4 * qd + 1], w[4 * qd + 2], w[4 * qd + 3]);
                        *(bf16x4*)(smem + ws_off(m, jl, 4 * (rt0 + rr) + qd) + 8 * lg) = v4;
                        *(bf16x4*)&base[32 * rr + 8 * qd] = v4;
                    }
                    const f32x16 mm = acc[rr][2 * m];
                    acc[rr][2 * m + 1] = A * w - gamma * mm;
                    acc[rr][2 * m] = Bb * mm;
                }
            }
            __syncthreads();
        }

        // ---- next block's K/V copy runs behind this block's work
        if (more) issue_kv(blk + 1, buf ^ 1);
        // ---- this block's coefficients (cM, cW of the lane's 16 tokens)
        f32x4 cm4[4], cw4[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int64_t t = (int64_t)blk * CB + 32 * gr + 8 * qd + 4 * lg;
            cm4[qd] = *(const f32x4*)&cMb[t];
            cw4[qd] = *(const f32x4*)&cWb[t];
        }

        // ---- grad: H1, H3, V W2^T for token rows gr, hidden cols gc
        f32x16 h1 = {}, h3 = {}, hv = {};
        {
            const int t = 32 * gr + li;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int jw = 32 * gc + li;
                const bf16x8 ak = *(const bf16x8*)(smem + kv_off(buf, 0, t, 2 * ks + lg));
                const bf16x8 av = *(const bf16x8*)(smem + kv_off(buf, 1, t, 2 * ks + lg));
                h1 = mfma32(ak, *(const bf16x8*)(smem + ws_off(0, jw, 2 * ks + lg)), h1);
                h3 = mfma32(ak, *(const bf16x8*)(smem + ws_off(1, jw, 2 * ks + lg)), h3);
                hv = mfma32(av, *(const bf16x8*)(smem + ws_off(2, jw, 2 * ks + lg)), hv);
            }
        }
        // ---- elementwise backward and coefficient scaling -> LDS (hidden-major)
        // du = -hv: 1M = -cm*a, 1W = cw*a, 3M = -cm*b, 3W = cw*b, 2M = -cm*u,
        // 2W = cw*u, where a = hv*h3*silu'(h1), b = hv*silu(h1)
        {
            const int jl = 32 * gc + li;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                float o[6][4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * qd + e;
                    const float x1 = h1[r], x3 = h3[r], y = hv[r];
                    const float sg = fast_sigmoid(x1);
                    const float s1 = x1 * sg;
                    const float u = s1 * x3;
                    const float ds = sg + s1 * (1.f - sg);
                    const float av = y * x3 * ds;
                    const float bv = y * s1;
                    const float ncm = -cm4[qd][e], cw = cw4[qd][e];
                    o[0][e] = ncm * av;
                    o[1][e] = cw * av;
                    o[2][e] = ncm * bv;
                    o[3][e] = cw * bv;
                    o[4][e] = ncm * u;
                    o[5][e] = cw * u;
                }
#pragma unroll
                for (int ty = 0; ty < 6; ++ty)
                    *(bf16x4*)(smem + dt_off(ty, jl, 4 * gr + qd) + 8 * lg) =
                        pack4(o[ty][0], o[ty][1], o[ty][2], o[ty][3]);
            }
        }
        __syncthreads();

        // ---- aggregation into the resident state
        {
            const unsigned char* kbuf = smem + OFF_KV + (2 * buf) * KV_BYTES;
            const unsigned char* vbuf = kbuf + KV_BYTES;
            const int jl = 32 * hh + li;
#pragma unroll
            for (int ks = 0; ks < CB / 16; ++ks) {
                const int rb0 = 16 * ks + 8 * lg, rb1 = rb0 + 4;
                bf16x8 ak[2], av[2];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    ak[rr] = tr_frag(kbuf, rb0, rb1, 32 * (rt0 + rr), lane);
                    av[rr] = tr_frag(vbuf, rb0, rb1, 32 * (rt0 + rr), lane);
                }
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    const bf16x8 bm = *(const bf16x8*)(smem + dt_off(2 * m, jl, 2 * ks + lg));
                    const bf16x8 bw = *(const bf16x8*)(smem + dt_off(2 * m + 1, jl, 2 * ks + lg));
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const bf16x8 x = (m < 2) ? ak[rr] : av[rr];
                        acc[rr][2 * m] = mfma32(x, bm, acc[rr][2 * m]);
                        acc[rr][2 * m + 1] = mfma32(x, bw, acc[rr][2 * m + 1]);
                    }
                }
            }
        }
        wait_vmem();  // this wave's share of the next block's K/V has landed
        __syncthreads();
    }

    float* We = a.W_end + bh * P;
    float* Me = a.M_end + bh * P;
    state_io<true>(acc, We, Me, rt0, hh, j0, Hd, laneA, laneB);
}

// ---------------------------------------------------------------------------
// apply: out = (silu(Q W1) * (Q W3)) W2 from the chunk-start snapshot.
// Snapshot layout per (b, h, chunk), bf16, all hidden-major:
//   W1^T [Hd][D] | W3^T [Hd][D] | W2 [Hd][D].
// One wavefront per 32 tokens; hidden units stream through LDS 32 at a time
// (double-buffered, HBM -> LDS copies).  Computed transposed (H^T = W1^T Q^T,
// out^T = W2^T U^T) so that U^T leaves the first MFMA in the register layout
// the second one consumes; the W2^T operand comes from the hidden-major stage
// through the transpose read.
// ---------------------------------------------------------------------------
struct ApplyArgs {
    const __bf16* q;
    const __bf16* snap;
    __bf16* out;
    int64_t T;
    int Hd, C, nc, rbc;  // rbc: workgroups per chunk
};

constexpr int HB = 32;                     // hidden units per stage
constexpr int STAGE_BYTES = 3 * HB * 256;  // W1^T, W3^T, W2 rows of the stage

template <int NWA>
__global__ __launch_bounds__(64 * NWA) void swiglu_apply_kernel(ApplyArgs a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE_BYTES];
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

    // stage hb -> buffer: 24 instructions of 4 rows (1 KB), spread over the waves
    auto issue_stage = [&](int hb, int sbuf) {
#pragma unroll
        for (int i = wave; i < 24; i += NWA) {
            const int m = i >> 3, r0 = 4 * (i & 7);
            const int row = r0 + (lane >> 4);
            const int cch = (lane & 15) ^ swz(row);
            __builtin_amdgcn_global_load_lds((const void*)(sn + (int64_t)m * Hd * D + (int64_t)(hb + row) * D + 8 * cch),
                                             (lds_void_t*)(smem + sbuf * STAGE_BYTES + m * HB * 256 + r0 * 256), 16,
                                             0, 0);
        }
    };

    issue_stage(0, 0);
    bf16x8 qf[8];  // Q^T as B operand: col = token, k = d
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)&qb[(t0 + li) * D + 16 * ks + 8 * lg];
    wait_vmem();
    __syncthreads();

    f32x16 oacc[4] = {};
    const int nhb = Hd / HB;
    for (int ih = 0; ih < nhb; ++ih) {
        const int sbuf = ih & 1;
        if (ih + 1 < nhb) issue_stage((ih + 1) * HB, sbuf ^ 1);
        const unsigned char* st = smem + sbuf * STAGE_BYTES;
        f32x16 x1 = {}, x3 = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int ch = (2 * ks + lg) ^ swz(li);
            x1 = mfma32(*(const bf16x8*)(st + li * 256 + 16 * ch), qf[ks], x1);
            x3 = mfma32(*(const bf16x8*)(st + HB * 256 + li * 256 + 16 * ch), qf[ks], x3);
        }
        // U^T tile: rows j = 8(r/4) + 4 lg + r%4, col = token
        bf16x8 ub[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 8 * s + e;
                const float h = x1[r];
                ub[s][e] = (__bf16)(h * fast_sigmoid(h) * x3[r]);
            }
        // k-step s covers j = 16 s + {0..15}; lane group lg holds j offsets
        // {4lg..4lg+3, 8+4lg..8+4lg+3}; the transpose read fetches W2 rows in that order.
        const unsigned char* w2 = st + 2 * HB * 256;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int jb = 16 * s + 4 * lg;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) oacc[dt] = mfma32(tr_frag(w2, jb, jb + 8, 32 * dt, lane), ub[s], oacc[dt]);
        }
        wait_vmem();
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
    const unsigned nck = (unsigned)(BH * aa.nc);
    if (d.chunk % 256 == 0) {
        aa.rbc = (int)(d.chunk / 256);
        hipLaunchKernelGGL(swiglu_apply_kernel<8>, dim3(nck * aa.rbc), dim3(512), 0, s, aa);
    } else if (d.chunk % 128 == 0) {
        aa.rbc = (int)(d.chunk / 128);
        hipLaunchKernelGGL(swiglu_apply_kernel<4>, dim3(nck * aa.rbc), dim3(256), 0, s, aa);
    } else {
        aa.rbc = (int)(d.chunk / 64);
        hipLaunchKernelGGL(swiglu_apply_kernel<2>, dim3(nck * aa.rbc), dim3(128), 0, s, aa);
    }
    return hipGetLastError();
}

}  // namespace e2ttt

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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// dword 3 of a raw buffer resource (gfx9 family: 32-bit data format, no swizzle)
constexpr int RSRC_W3 = 0x00020000;

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

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (__bf16)lo[e];
        r[4 + e] = (__bf16)hi[e];
    }
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

// LDS of the loop kernel: two buffers of one token block each (TBK = 64 SB
// tokens): K [TBK][128] bf16 | V [TBK][128] bf16 | cM [TBK] f32 | cW [TBK] f32
// (| unused up to 1 KB) | (A, Bb, gamma, -) of the block's chunk.
// Rows are 256 bytes; 16-byte chunk c of row t sits at physical chunk
// c ^ swz4(t).  The LDS has 64 four-byte banks (256 bytes per clock):
// ds_read_b128 serves 16 lanes at a time, here 16 consecutive rows at one
// chunk, which swz4 (a permutation of the 16 chunks over t mod 16) spreads
// over all 64 banks; ds_read_b64_tr_b16 serves 32 lanes at a time, here 8
// consecutive rows x 4 chunks x one 8-byte half per chunk pair, which swz4
// (bits 0, 2, 3 of the permutation taken from the row, bit 1 from row bit 3)
// also spreads over all 64 banks.
__device__ __forceinline__ int swz4(int t) { return (t & 1) | ((t & 6) << 1) | ((t & 8) >> 2); }

__device__ __forceinline__ int row_off(int t, int chunk) { return t * 256 + 16 * (chunk ^ swz4(t)); }

// Row permutation of the state tiles.  Accumulator tile i (16 rows of d)
// holds, in its row 4g + r (lane group g, register r),
//   d = 32(i/2) + 8g + 4((g & 1) ^ (i & 1)) + r.
// Tiles 2kk and 2kk+1 together give lane group g exactly d = 32kk + 8g + 0..7,
// which is the k-slot order of a natural 16x16x32 operand: the chunk-start
// weights become grad operands by a conversion in registers, while the
// aggregation's K^T / V^T operands pick the same d order in the transpose read.
__device__ __forceinline__ int state_d(int i, int g) { return 32 * (i >> 1) + 8 * g + 4 * ((g & 1) ^ (i & 1)); }

// K^T / V^T aggregation operand for state tile i and the 32 tokens tb..tb+31 of
// the LDS block: operand row rho = l%16 is d = state_d(i, rho/4) + rho%4,
// k-slot e < 4 is token tb + 4(l/16) + e, e >= 4 is token tb + 16 + 4(l/16) + e-4.
// ds_read_b64_tr_b16: within a 16-lane group lane p fetches 4 values of
// token row p/4 at d quad p%4, and lane i receives 4 token rows of quad
// i/4, element i%4.
__device__ __forceinline__ bf16x8 trT(const unsigned char* buf, int i, int tb, int lane) {
    const int p = lane & 15, g = lane >> 4, q = p & 3;
    const int dq = 32 * (i >> 1) + 8 * q + 4 * ((q & 1) ^ (i & 1));
    const int chunk = dq >> 3, half = (dq >> 2) & 1;
    const int r0 = tb + 4 * g + (p >> 2), r1 = r0 + 16;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(buf + r0 * 256 + 16 * (chunk ^ swz4(r0)) + 8 * half));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(buf + r1 * 256 + 16 * (chunk ^ swz4(r1)) + 8 * half));
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = lo[e];
        r[4 + e] = hi[e];
    }
    return r;
}

// State tiles <-> packed fp32 parameters (W1 [D][Hd] | W3 [D][Hd] | W2 [Hd][D]).
// acc[m][0] / acc[m][1] are the M / W parts of matrix m (0: W1, 1: W3, 2: W2
// held transposed as [d][j]); tile element (i, r) of lane (jl, g) is
// d = state_d(i, g) + r, hidden unit j = j0 + jl.
template <bool STORE>
__device__ __forceinline__ void state_io(f32x4 (&acc)[3][2][8], float* W, float* M, int64_t j, int g, int Hd) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t d = state_d(i, g);
            if (m < 2) {
                const int64_t o = (int64_t)m * D * Hd + d * Hd + j;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (STORE) {
                        M[o + r * Hd] = acc[m][0][i][r];
                        W[o + r * Hd] = acc[m][1][i][r];
                    } else {
                        acc[m][0][i][r] = M[o + r * Hd];
                        acc[m][1][i][r] = W[o + r * Hd];
                    }
                }
            } else {
                const int64_t o = 2 * (int64_t)D * Hd + j * D + d;
                if (STORE) {
                    *(f32x4*)&M[o] = acc[m][0][i];
                    *(f32x4*)&W[o] = acc[m][1][i];
                } else {
                    acc[m][0][i] = *(const f32x4*)&M[o];
                    acc[m][1][i] = *(const f32x4*)&W[o];
                }
            }
        }
    }
}

// One workgroup = one (b, h, 64-unit hidden slice) for the whole sequence.
// Wavefront w owns hidden units j0 + 16w .. +15 of the slice in all three
// matrices: their fp32 M and W (6 x 128 x 16 per wave) stay in accumulator
// registers, and the chunk-start weights as bf16 grad operands.  Tokens go
// through LDS in blocks of SB sub-blocks of 64; per sub-block every wave runs
//   grad:      H1, H3 = K W1, K W3 and HV = V W2^T for its 16 units
//              (16x16x32 MFMA, K/V rows from LDS),
//   backward:  the six coefficient-scaled factors, converted in registers
//              straight into the aggregation's B operand,
//   aggregate: state += K^T F1, K^T F3, V^T F2 (K^T, V^T by transpose reads),
// so the only data the waves share is the K/V/coefficient block in LDS, and
// one barrier per block guards its double buffer.
//
// Within a block the three stages run as one software pipeline of
// 16 SB + 12 steps; sub-block s occupies local steps ls = step - 16 s:
//   ls  0..15  grad of tile ls/4, k-step ls%4       (3 MFMA)
//   ls  4..19  backward of tile ls/4 - 1, row ls%4 (VALU)
//   ls 12..27  aggregation step u = ls - 12         (6 MFMA)
// so the MFMA-only head of one sub-block overlaps the backward of the
// previous one.  sched_barrier keeps every step's work together; grad
// fragments are read two steps ahead, aggregation fragments two, coefficients
// one, and the next block's HBM->LDS copies are spread over the first steps.
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
swiglu_loop_kernel(LoopArgs a) {
    constexpr int SB = 1;                        // 64-token sub-blocks per LDS block
    constexpr int TBK = CB * SB;                 // tokens per LDS block
    constexpr int KVB = TBK * 256;               // one [TBK][128] bf16 matrix
    constexpr int COB = 1024 + 16;               // cM | cW (| unused) | (A, Bb, gamma, -)
    constexpr int BUFB = 2 * KVB + COB;
    constexpr int BOFF = 5;                      // backward of tile t starts at local step 4 t + BOFF
    constexpr int AOFF = 4 + 2 * 4 + BOFF - 4;   // aggregation step u runs at local step AOFF + u
    constexpr int NSTEP = 16 * (SB - 1) + AOFF + 16;
    constexpr int NKV = 4 * SB;                  // copy instructions per matrix per wave
    constexpr int AGG_AHEAD = SB == 1 ? 2 : 1;   // aggregation fragments are read this many steps ahead
    // Two LDS buffers as separate arrays: the compiler can then tell the
    // next block's in-flight HBM->LDS copies from this block's LDS reads.
    __shared__ __attribute__((aligned(16))) unsigned char lds0[BUFB];
    __shared__ __attribute__((aligned(16))) unsigned char lds1[BUFB];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int jl = lane & 15, g = lane >> 4;

    // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
    // remap to keep the slices of one head (which read the same K/V) on one XCD.
    int L_id = blockIdx.x;
    if (a.xcd_map) L_id = (blockIdx.x % 8) * (a.nwg / 8) + blockIdx.x / 8;
    const int64_t bh = L_id / a.nsl;
    const int Hd = a.Hd;
    const int64_t j = (int64_t)(L_id % a.nsl) * S + 16 * wave + jl;  // this lane's hidden unit
    const int64_t T = a.T;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int nblk = (int)(T / TBK);
    const int bpc = a.C / TBK;

    // HBM -> LDS copies of one block (buffer / MUBUF form of the direct
    // load: unlike the global form it is not a FLAT instruction, so while it
    // is in flight the compiler still waits for individual LDS reads).  Lane L
    // of a copy writes 16 bytes at destination + 16 L.  Wave w moves K and V
    // rows [TBK/4 w, TBK/4 (w+1)), 4 rows per instruction: lane L loads
    // row r0 + L/16, chunk (L%16) ^ swz4(row), which lands at physical chunk
    // L%16.  Wave 0 also moves the block's cM and cW (one instruction; cM and
    // cW are addressed from one resource based at cM) and the (A, Bb, gamma)
    // of the block's chunk.  Copies past the end of the sequence (the block
    // after the last) fall outside the resources' ranges and read zeros.
    const __bf16* kb = a.k + bh * T * D;
    const __bf16* vb = a.v + bh * T * D;
    const float* cMb = a.cM + bh * T;
    const unsigned cw_rel = (unsigned)((const char*)(a.cW + bh * T) - (const char*)cMb);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, (int)(T * D * 2), RSRC_W3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, (int)(T * D * 2), RSRC_W3);
    const __amdgpu_buffer_rsrc_t crs =
        __builtin_amdgcn_make_buffer_rsrc((void*)cMb, 0, (int)(cw_rel + T * 4), RSRC_W3);
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.scal + bh * a.nc * 4), 0, a.nc * 16, RSRC_W3);
    unsigned koff[NKV];
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
        const int row = (TBK / 4) * wave + 4 * i + (lane >> 4);
        koff[i] = (unsigned)(row * D + 8 * ((lane & 15) ^ swz4(row))) * 2u;
    }
    const unsigned coff = lane < 16 * SB ? 16u * lane
                        : lane < 32 * SB ? cw_rel + 16u * (lane - 16 * SB)
                                         : 16u * (lane - 32 * SB);
    // copy instruction n (0 <= n < 2 NKV + 1) of block blk into dst
    auto issue = [&](int n, int blk, unsigned char* dst) {
        const unsigned tbb = (unsigned)blk * TBK * D * 2;
        if (n < 2 * NKV) {
            const int m = n & 1, i = n >> 1;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(m ? vrs : krs,
                                                     (lds_void_t*)(dst + m * KVB + ((TBK / 4) * wave + 4 * i) * 256),
                                                     16, koff[i], tbb, 0, 0);
        } else if (wave == 0) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, (lds_void_t*)(dst + 2 * KVB), 16, coff,
                                                     (unsigned)blk * TBK * 4, 0, 0);
        }
    };
    auto issue_scal = [&](int blk, unsigned char* dst) {
        if (wave == 0 && lane == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void_t*)(dst + 2 * KVB + 1024), 16, 0,
                                                     (unsigned)(blk / bpc) * 16, 0, 0);
    };

    f32x4 acc[3][2][8];
    state_io<false>(acc, (float*)a.W0 + bh * P, (float*)a.M0 + bh * P, j, g, Hd);

    const bool godd = (g & 1) != 0;
    bf16x8 wb[3][4];  // chunk-start weights as grad B operands: k-slot e of lane group g is d = 32kk + 8g + e

#pragma unroll
    for (int n = 0; n < 2 * NKV + 1; ++n) issue(n, 0, lds0);
    issue_scal(0, lds0);
    wait_vmem();
    __syncthreads();

    auto block = [&](int blk, const unsigned char* kbuf, unsigned char* next) {
        const unsigned char* vbuf = kbuf + KVB;
        const float* cob = (const float*)(kbuf + 2 * KVB);
        if (blk % bpc == 0) {
            // ---- chunk start: grad operands + bf16 snapshot from W, then rescale the state
            const int c = blk / bpc;
            const f32x4 sc = *(const f32x4*)&cob[256];
            const float A = sc[0], Bb = sc[1], gamma = sc[2];
            __bf16* snap = a.snap + (bh * a.nc + c) * P + j * D + 8 * g;
#pragma unroll
            for (int m = 0; m < 3; ++m) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x4 t0 = pack4(acc[m][1][2 * kk][0], acc[m][1][2 * kk][1], acc[m][1][2 * kk][2],
                                            acc[m][1][2 * kk][3]);
                    const bf16x4 t1 = pack4(acc[m][1][2 * kk + 1][0], acc[m][1][2 * kk + 1][1],
                                            acc[m][1][2 * kk + 1][2], acc[m][1][2 * kk + 1][3]);
                    const bf16x4 lo = godd ? t1 : t0, hi = godd ? t0 : t1;
                    bf16x8 w8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w8[e] = lo[e];
                        w8[4 + e] = hi[e];
                    }
                    wb[m][kk] = w8;
                    *(bf16x8*)&snap[(int64_t)m * Hd * D + 32 * kk] = w8;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const f32x4 mm = acc[m][0][i];
                    acc[m][1][i] = A * acc[m][1][i] - gamma * mm;
                    acc[m][0][i] = Bb * mm;
                }
            }
        }
        issue_scal(blk + 1, next);

        // f[s][x][h]: factors of sub-block s; x = 1M, 1W, 3M, 3W, 2M, 2W; h = 32-token half
        bf16x8 f[SB][6][2];
        f32x4 hg[SB][4][3];     // grad accumulators per sub-block and tile
        float ob[SB][6];        // backward outputs of the last even token row
        bf16x2 pr[SB][6][4];    // packed factor pairs of the current tile pair
        f32x4 cm[SB], cw[SB];   // coefficients of the tile being processed
        f32x4 cmn[SB], cwn[SB]; // ... and of the next one (read a step early)
        auto gfrag = [&](const unsigned char* b, int gs) {  // grad step gs = 16 s + 4 ti + kk
            const int s = gs >> 4, l = gs & 15;
            return *(const bf16x8*)(b + row_off(64 * s + 16 * (l >> 2) + jl, 4 * (l & 3) + g));
        };
        auto afrag = [&](const unsigned char* b, int s, int u) { return trT(b, u & 7, 64 * s + 32 * (u >> 3), lane); };
        // backward for token row r of tile ti of sub-block s:
        // du = -hv: 1M = -cm*a, 1W = cw*a, 3M = -cm*b, 3W = cw*b, 2M = -cm*u,
        // 2W = cw*u, where a = hv*h3*silu'(h1), b = hv*silu(h1)
        auto backward = [&](int s, int ti, int r) {
            if (r == 0) {
                cm[s] = cmn[s];
                cw[s] = cwn[s];
            }
            const float x1 = hg[s][ti][0][r], x3 = hg[s][ti][1][r], y = hg[s][ti][2][r];
            const float sg = fast_sigmoid(x1);
            const float s1 = x1 * sg;
            const float u = s1 * x3;
            const float ds = sg + s1 * (1.f - sg);
            const float av = y * x3 * ds;
            const float bv = y * s1;
            const float ncm = -cm[s][r], cwr = cw[s][r];
            float o[6];
            o[0] = ncm * av;
            o[1] = cwr * av;
            o[2] = ncm * bv;
            o[3] = cwr * bv;
            o[4] = ncm * u;
            o[5] = cwr * u;
            if ((r & 1) == 0) {
#pragma unroll
                for (int x = 0; x < 6; ++x) ob[s][x] = o[x];
                return;
            }
            // rows r-1, r of the tile -> bf16 pair at position r/2 of the tile's half
#pragma unroll
            for (int x = 0; x < 6; ++x) {
                bf16x2 p2;
                p2[0] = (__bf16)ob[s][x];
                p2[1] = (__bf16)o[x];
                pr[s][x][(ti & 1) * 2 + (r >> 1)] = p2;
            }
            if (r == 3 && (ti & 1)) {
#pragma unroll
                for (int x = 0; x < 6; ++x) {
                    bf16x8 v8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v8[2 * e] = pr[s][x][e][0];
                        v8[2 * e + 1] = pr[s][x][e][1];
                    }
                    f[s][x][ti >> 1] = v8;
                }
            }
        };
        auto agg = [&](int s, int u, bf16x8 kt, bf16x8 vt) {
            const int h = u >> 3, i = u & 7;
            acc[0][0][i] = mfma16(kt, f[s][0][h], acc[0][0][i]);
            acc[0][1][i] = mfma16(kt, f[s][1][h], acc[0][1][i]);
            acc[1][0][i] = mfma16(kt, f[s][2][h], acc[1][0][i]);
            acc[1][1][i] = mfma16(kt, f[s][3][h], acc[1][1][i]);
            acc[2][0][i] = mfma16(vt, f[s][4][h], acc[2][0][i]);
            acc[2][1][i] = mfma16(vt, f[s][5][h], acc[2][1][i]);
        };

        bf16x8 gk = gfrag(kbuf, 0), gv = gfrag(vbuf, 0);
        bf16x8 gk2 = gfrag(kbuf, 1), gv2 = gfrag(vbuf, 1);
        bf16x8 tk[3], tv[3];  // aggregation fragments, ring of 3
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            // ---- copies for the next block, LDS reads for later steps
            if (st < 2 * NKV + 1) issue(st, blk + 1, next);
            const bf16x8 ak = gk, av = gv;
            gk = gk2;
            gv = gv2;
            if (st + 2 < 16 * SB) {
                gk2 = gfrag(kbuf, st + 2);
                gv2 = gfrag(vbuf, st + 2);
            }
#pragma unroll
            for (int s = 0; s < SB; ++s) {
                const int ls = st - 16 * s;  // coefficients of tile ls/4 one step before its backward
                const int lb = ls + 1 - BOFF;
                if (lb >= 0 && lb < 16 && (lb & 3) == 0) {
                    cmn[s] = *(const f32x4*)&cob[64 * s + 16 * (lb >> 2) + 4 * g];
                    cwn[s] = *(const f32x4*)&cob[64 * SB + 64 * s + 16 * (lb >> 2) + 4 * g];
                }
            }
#pragma unroll
            for (int s = 0; s < SB; ++s) {
                const int ur = st + AGG_AHEAD - 16 * s - AOFF;
                if (ur >= 0 && ur < 16) {
                    tk[(16 * s + ur) % 3] = afrag(kbuf, s, ur);
                    tv[(16 * s + ur) % 3] = afrag(vbuf, s, ur);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // ---- grad MFMAs
            if (st < 16 * SB) {
                const int s = st >> 4, ti = (st >> 2) & 3, kk = st & 3;
                if (kk == 0) {
                    hg[s][ti][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    hg[s][ti][1] = hg[s][ti][0];
                    hg[s][ti][2] = hg[s][ti][0];
                }
                hg[s][ti][0] = mfma16(ak, wb[0][kk], hg[s][ti][0]);
                hg[s][ti][1] = mfma16(ak, wb[1][kk], hg[s][ti][1]);
                hg[s][ti][2] = mfma16(av, wb[2][kk], hg[s][ti][2]);
            }
#pragma unroll
            for (int s = 0; s < SB; ++s) {
                const int ls = st - 16 * s;
                // ---- aggregation MFMAs
                if (ls >= AOFF && ls < AOFF + 16)
                    agg(s, ls - AOFF, tk[(ls + 16 * s - AOFF) % 3], tv[(ls + 16 * s - AOFF) % 3]);
                // ---- backward of the previous tile, one token row per step
                if (ls >= BOFF && ls < BOFF + 16) backward(s, (ls - BOFF) >> 2, (ls - BOFF) & 3);
            }
            // issue order within the step: each MFMA followed by up to three
            // VALU instructions, which run while the MFMA executes
#pragma unroll
            for (int k = 0; k < 9; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmem();  // this wave's share of the next block has landed
        __syncthreads();
    };
    for (int blk = 0; blk < nblk; blk += 2) {
        block(blk, lds0, lds1);
        if (blk + 1 < nblk) block(blk + 1, lds1, lds0);
    }

    state_io<true>(acc, a.W_end + bh * P, a.M_end + bh * P, j, g, Hd);
}

// ---------------------------------------------------------------------------
// apply: out = (silu(Q W1) * (Q W3)) W2 from the chunk-start snapshot.
// Snapshot layout per (b, h, chunk), bf16, all hidden-major:
//   W1^T [Hd][D] | W3^T [Hd][D] | W2 [Hd][D].
// One wavefront per 32 tokens; hidden units stream through LDS 32 at a time
// in a ring of three stages (two copies in flight while one is consumed).
// Computed transposed (H^T = W1^T Q^T, out^T = W2^T U^T) so that U^T leaves
// the first MFMA in the register layout the second one consumes; the W2^T
// operand comes from the hidden-major stage through the transpose read.
// ---------------------------------------------------------------------------
struct ApplyArgs {
    const __bf16* q;
    const __bf16* snap;
    __bf16* out;
    int64_t T;
    int Hd, C, nc, rbc;  // rbc: items per chunk
    int nb;              // B H
};

constexpr int HB = 32;                     // hidden units per stage
constexpr int STAGE_BYTES = 3 * HB * 256;  // W1^T, W3^T, W2 rows of the stage

// Stage rows are 256 bytes with 16-byte chunk c of row t at physical chunk
// c ^ swza(t).  The grad-style row reads (16 consecutive rows at one chunk)
// see a permutation of all 16 chunks, and each 32-lane half of a 32x32
// transpose fragment (4 consecutive rows x 4 chunks x 2 halves) sees four
// disjoint 4-chunk groups: conflict-free on the 64 four-byte banks.
__device__ __forceinline__ int swza(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// 32x16 MFMA operand fragment transposed out of a swizzled row-major
// [rows][128] bf16 stage: operand row = source column col0 + lane%32,
// operand k 0..3 = source rows rbase0..+3, k 4..7 = source rows rbase1..+3.
__device__ __forceinline__ bf16x8 tr_frag_a(const unsigned char* buf, int rbase0, int rbase1, int col0, int lane) {
    const int p = lane & 15, G = lane >> 4;
    const int col = col0 + 16 * (G & 1) + 4 * (p & 3);
    const int chunk = col >> 3;
    const int half = p & 1;
    const int r0 = rbase0 + (p >> 2);
    const int r1 = rbase1 + (p >> 2);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(buf + r0 * 256 + 16 * (chunk ^ swza(r0)) + 8 * half));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(buf + r1 * 256 + 16 * (chunk ^ swza(r1)) + 8 * half));
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = lo[e];
        r[4 + e] = hi[e];
    }
    return r;
}

// direct HBM->LDS copy of 16 bytes per lane (buffer form; lane L writes
// dst + 16 L); offsets at or past num_bytes read zeros
__device__ __forceinline__ void lds_copy16(const void* base, int num_bytes, unsigned char* dst, unsigned voff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, num_bytes, RSRC_W3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, 0, 0, 0);
}

// Persistent: every workgroup walks a list of items (an item = 32 NWA tokens
// of one chunk) so the stage copies never stop between items.  Each
// wavefront copies its own 32 query rows of the next item into its own LDS
// rows while the current item runs.
template <int NWA>
__global__ __launch_bounds__(64 * NWA) void swiglu_apply_kernel(ApplyArgs a) {
    // three stage buffers as separate arrays, so the compiler can tell copies
    // in flight from the reads of the stage being consumed
    __shared__ __attribute__((aligned(16))) unsigned char sb0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sb1[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char sb2[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char qs[NWA * 32 * 256];  // [wave][32 tokens][128] bf16
    constexpr int NI = 24 / NWA;  // stage copy instructions per wave per stage
    constexpr int NQ = 8;         // query copy instructions per wave per item (32 rows, 4 per copy)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 31, lg = lane >> 5;
    const int Hd = a.Hd;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int nhb = Hd / HB;
    const int64_t nitems = (int64_t)a.nb * a.nc * a.rbc;
    // items of this workgroup: blockIdx.x + k gridDim.x
    const int nmine = (int)((nitems - blockIdx.x + gridDim.x - 1) / gridDim.x);
    unsigned char* qw = qs + wave * 32 * 256;

    struct Item {
        const __bf16* sn;  // snapshot of the item's chunk
        int64_t tok;       // first token (global row in q / out) of this wave
        int nrec;          // bytes the copies may read (0 past the last item: zeros)
    };
    auto item = [&](int k) {
        Item it;
        const int64_t x = blockIdx.x + (int64_t)k * gridDim.x;
        const bool ok = k < nmine;
        const int64_t xx = ok ? x : 0;
        const int64_t bh = xx / ((int64_t)a.nc * a.rbc);
        const int rem = (int)(xx % ((int64_t)a.nc * a.rbc));
        const int c = rem / a.rbc, rb = rem % a.rbc;
        it.sn = a.snap + (bh * a.nc + c) * P;
        it.tok = bh * a.T + (int64_t)c * a.C + (int64_t)rb * 32 * NWA + 32 * wave;
        it.nrec = ok ? (int)(P * 2) : 0;
        return it;
    };

    // stage copies: 24 copies of 4 rows (1 KB), NI per wave
    unsigned voff[NI];
    int mrow[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int i = wave + NWA * n;
        const int m = i >> 3, r0 = 4 * (i & 7);
        const int row = r0 + (lane >> 4);
        voff[n] = (unsigned)((m * Hd * D + row * D + 8 * ((lane & 15) ^ swza(row))) * 2);
        mrow[n] = m * HB * 256 + r0 * 256;
    }
    // global stage index gs = k nhb + ih
    auto issue_stage = [&](int gs, unsigned char* buf) {
        const Item it = item(gs / nhb);
        const unsigned ho = (unsigned)((gs % nhb) * HB * D * 2);
#pragma unroll
        for (int n = 0; n < NI; ++n) lds_copy16(it.sn, it.nrec, buf + mrow[n], voff[n] + ho);
    };
    // the wave's 32 query rows of item k, row-major with the stage swizzle
    auto issue_q = [&](int k) {
        const Item it = item(k);
        const int qrec = k < nmine ? 32 * D * 2 : 0;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int row = 4 * n + (lane >> 4);
            const unsigned vo = (unsigned)((row * D + 8 * ((lane & 15) ^ swza(row))) * 2);
            lds_copy16(a.q + it.tok * D, qrec, qw + 4 * n * 256, vo);
        }
    };

    bf16x8 qf[8];  // Q^T as B operand: col = token, k = d
    f32x16 oacc[4] = {};
    issue_q(0);
    issue_stage(0, sb0);
    issue_stage(1, sb1);

    auto stage = [&](int gs, const unsigned char* st, unsigned char* refill) {
        const int ih = gs % nhb;
        // this stage's copies (and, at an item start, the item's queries)
        // landed: the loads issued after them are the next stage's copies and,
        // within two stages of an item start, the next item's queries.  (Loads
        // complete in order; a count that ignores later stores only waits longer.)
        if (ih == 1 || ih == 2)
            __builtin_amdgcn_s_waitcnt(((NI + NQ) & 15) | (((NI + NQ) >> 4) << 14) | 0x0F70);
        else
            __builtin_amdgcn_s_waitcnt((NI & 15) | ((NI >> 4) << 14) | 0x0F70);
        __syncthreads();
        issue_stage(gs + 2, refill);  // refill = buffer of stage gs - 1, free after the barrier
        if (ih == 0) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(qw + li * 256 + 16 * ((2 * ks + lg) ^ swza(li)));
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the query rows are in registers
            issue_q(gs / nhb + 1);
        }
        f32x16 x1 = {}, x3 = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int ch = (2 * ks + lg) ^ swza(li);
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
            for (int dt = 0; dt < 4; ++dt)
                oacc[dt] = mfma32(tr_frag_a(w2, jb, jb + 8, 32 * dt, lane), ub[s], oacc[dt]);
        }
        if (ih == nhb - 1) {
            const int64_t tok = item(gs / nhb).tok;
            __bf16* ob = a.out + tok * D;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int d = 32 * dt + 8 * qd + 4 * lg;
                    *(bf16x4*)&ob[li * D + d] =
                        pack4(oacc[dt][4 * qd], oacc[dt][4 * qd + 1], oacc[dt][4 * qd + 2], oacc[dt][4 * qd + 3]);
                }
                oacc[dt] = f32x16{};
            }
        }
    };
    const int nst = nmine * nhb;
    for (int gs = 0; gs < nst; gs += 3) {
        stage(gs, sb0, sb2);
        if (gs + 1 < nst) stage(gs + 1, sb1, sb0);
        if (gs + 2 < nst) stage(gs + 2, sb2, sb1);
    }
    wait_vmem();  // copies past the last item (zeros) land before the LDS goes away
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
    aa.nb = (int)BH;
    // persistent grid: one workgroup per compute unit (the LDS of one fills it)
    int dev = 0, ncu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t nck = BH * aa.nc;
    auto grid = [&](int64_t items) { return dim3((unsigned)(items < ncu ? items : ncu)); };
    if (d.chunk % 256 == 0) {
        aa.rbc = (int)(d.chunk / 256);
        hipLaunchKernelGGL(swiglu_apply_kernel<8>, grid(nck * aa.rbc), dim3(512), 0, s, aa);
    } else if (d.chunk % 128 == 0) {
        aa.rbc = (int)(d.chunk / 128);
        hipLaunchKernelGGL(swiglu_apply_kernel<4>, grid(nck * aa.rbc), dim3(256), 0, s, aa);
    } else {
        aa.rbc = (int)(d.chunk / 64);
        hipLaunchKernelGGL(swiglu_apply_kernel<2>, grid(nck * aa.rbc), dim3(128), 0, s, aa);
    }
    return hipGetLastError();
}

}  // namespace e2ttt

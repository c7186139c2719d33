// SwiGLU fast weight, negative-dot loss, bf16 k/v, fp32 state: the chunk loop
// of the E2-TTT update on CDNA4 (gfx950), with the state and the gradient
// work on separate wavefronts.
//
// Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
// (abstract; atlas summary "Approach"): per chunk, gradients at the
// chunk-start weights, two scalar kernels, two weighted gradient
// aggregations, and a closed-form transition of (W, M).
//
// Per (b, h) and chunk, with K, V the chunk's [C x D] token rows, the
// chunk-start weights W1, W3 [D x Hd], W2 [Hd x D] and per-token coefficients
// cM = eta*m, cW = eta*w from e2ttt_logscan:
//   grad:       H1 = K W1, H3 = K W3, dU = -V W2^T                      [C x Hd]
//               U = silu(H1)*H3, dH3 = dU*silu(H1), dH1 = dU*H3*silu'(H1)
//   aggregate:  G1 = K^T diag(c) dH1, G3 = K^T diag(c) dH3,
//               G2^T = V^T diag(-c) U           for c in {cM, cW}
//   epilogue:   M <- Bb*M + G^M,   W <- A*W - gamma*M_old - G^W
//
// dL/dy = -v does not depend on W, so hidden unit j's gradient touches only
// column j of W1, W3 and row j of W2: a head's hidden units split into
// independent slices of 64, and one workgroup owns one (b, h, slice) for the
// whole sequence.
//
// Workgroup = 8 wavefronts, two per SIMD, in two roles over the same 16-unit
// groups u = 0..3 (the precise form: 4 wavefronts over a 32-unit slice,
// u = 0..1; grids that leave compute units idle take the block-slot kernel
// further below):
//   state wave u (wave u):      the group's fp32 W and M (6 x 128 x 16 values)
//                               as MFMA accumulators; per 32 tokens it scales
//                               the gradient wave's factors by the tokens'
//                               coefficients and adds K^T F and V^T F (48
//                               MFMAs), with K^T / V^T read from the row-major
//                               token block by the gfx950 LDS transpose read;
//                               it also issues the HBM -> LDS token copies;
//   gradient wave u (wave 4+u): the group's chunk-start weights as bf16 MFMA
//                               operands; per 32 tokens H1, H3, HV (24 MFMAs)
//                               and the backward to three unscaled fp32
//                               factors (VALU), handed over through LDS, so
//                               that each aggregation operand is rounded to
//                               bf16 once, after its scaling.
// The gradient wave runs one 32-token half-block ahead of the state wave and
// issues the next half-block's grad MFMAs before the current one's backward;
// one barrier per half-block separates the roles.  Sharing a SIMD, one wave's
// VALU work and LDS waits overlap the other's MFMAs.  At a chunk boundary the
// gradient waves wait one extra half-block: the next chunk's grad operands
// are the state after the previous chunk's last aggregation.
//
// Precise form (E2TTT_FLAG_PRECISE): the chunk-start weights in the grad
// products, the factors handed to the state waves and the coefficient-scaled
// aggregation operands are hi/lo bf16 pairs (16 significant bits), each
// product two MFMAs into the same fp32 accumulator.  On 32-unit slices, one
// wavefront per SIMD, with a 24 KB exchange area per unit group.
//
// LDS (150.5 KB; 123 KB for 32-unit slices): three 64-token K/V/coefficient
// blocks (the state waves' block, the gradient waves' block, one in flight
// from HBM) and per unit group a 12 KB exchange area: two half-block factor
// sets, or at a chunk boundary the 12 bf16 grad operands.  HBM -> LDS copies
// are waited for one slot before their first reader, so a barrier never
// waits on them.
#include <type_traits>

#include "e2ttt_internal.h"
#include "scan_wave.h"

namespace e2ttt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int D = 128;             // head dim
constexpr int CB = 64;             // tokens per LDS block
constexpr int KVB = CB * 256;      // one [64][128] bf16 token block
constexpr int COB = 1024;          // cM [64] f32 | cW [64] f32 | spare
constexpr int KVBUF = 2 * KVB + COB;
constexpr int NBUF = 3;            // token blocks resident in LDS
// Exchange area per unit group: two half-block factor sets, or at a chunk
// boundary the 12 bf16 grad operand fragments (64 lanes x 16 B each).  The
// factors go over in fp32 (3 x 2 KB a set), so that they are rounded to bf16
// once, after the coefficient scaling.  The precise form (PRE) hands every
// operand over as a hi/lo bf16 pair: twice the operand fragments, twice the
// area.
template <bool PRE> constexpr int XW = (PRE ? 24 : 12) * 1024;
template <bool PRE> constexpr int FACB = 6 * 1024;  // one half-block factor set
constexpr int RSRC_W3 = 0x00020000;  // dword 3 of a raw buffer resource (32-bit format, no swizzle)

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 pack4(f32x4 v) {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (__bf16)v[e];
    return r;
}

__device__ __forceinline__ float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): together 16
// significant bits, against 8 for hi alone.  hi / lo are summed by two
// MFMAs into one fp32 accumulator.
__device__ __forceinline__ void split4(f32x4 v, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)v[e];
        lo[e] = (__bf16)(v[e] - (float)hi[e]);
    }
}

// 16-byte chunk swizzle of 256-byte token rows: chunk c of row t sits at
// physical chunk c ^ swz4(t).  The LDS has 64 four-byte banks: ds_read_b128
// serves 16 lanes at a time (here 16 consecutive rows at one chunk, which
// swz4 spreads over all 64 banks) and ds_read_b64_tr_b16 32 lanes (8 rows x
// 4 chunks x one 8-byte half, also spread over all 64 banks by swz4).
__device__ __forceinline__ int swz4(int t) { return (t & 1) | ((t & 6) << 1) | ((t & 8) >> 2); }

// Row permutation of the state tiles: accumulator tile i (16 rows of d) holds
// in its row 4g + r (lane group g, register r) d = state_d(i, g) + r.  Tiles
// 2kk and 2kk+1 together give lane group g exactly d = 32kk + 8g + 0..7, the
// k-slot order of a natural 16x16x32 operand, so the chunk-start weights become
// grad operands by a conversion in registers.
__device__ __forceinline__ int state_d(int i, int g) { return 32 * (i >> 1) + 8 * g + 4 * ((g & 1) ^ (i & 1)); }

__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, unsigned num_bytes) {
    const unsigned long long p = (unsigned long long)base;
    u32x4 r;
    r[0] = (unsigned)p;
    r[1] = (unsigned)(p >> 32) & 0xFFFFu;
    r[2] = num_bytes;
    r[3] = RSRC_W3;
    return r;
}

// HBM -> LDS copy of 16 bytes per lane: lane L reads base + voff (zeros at or
// past the resource's num_records) and writes LDS byte lds + 16 L.  Written
// as an instruction the compiler does not track, so it inserts no wait for
// it anywhere; completion is waited for explicitly with wait_vm (no register
// is written by the instruction).  M0 carries the LDS address; nothing else in
// this kernel uses M0.
__device__ __forceinline__ void copy16(u32x4 rsrc, unsigned lds, unsigned voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) (N < 16), nothing else
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt");
    __builtin_amdgcn_s_waitcnt(N | 0x0F70);
}

// Workgroup barrier that waits for this wave's LDS accesses but not for its
// HBM -> LDS copies in flight.
__device__ __forceinline__ void slot_barrier() {
    __builtin_amdgcn_sched_barrier(0);  // no instruction moves across a slot boundary
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
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
    __bf16* snapM;  // bf16 chunk-start momentum snapshots (SAVEM instantiation only)
    int64_t T;
    int64_t ldc;  // row stride of cM / cW (T rounded up to a whole block, zero padded)
    int Hd, C, nc, nsl, nwg, xcd_map;
    // fold: the chunk loop computes the scalar kernels itself (cM, cW, scal
    // from eta, alpha, beta) before its first slot, instead of a separate scan
    // launch before it (two more workgroup barriers); avg: chunk-averaged
    // kernels
    const float *eta, *alpha, *beta;
    int fold, avg;
};

// State tiles <-> packed fp32 parameters (W1 [D][Hd] | W3 [D][Hd] | W2 [Hd][D]).
// acc[m][0] / acc[m][1] are the M / W parts of matrix m (0: W1, 1: W3, 2: W2
// held transposed as [d][j]); tile element (i, r) of lane (jl, g) is
// d = state_d(i, g) + r, hidden unit j.  Without momentum M is not touched.
// NT tiles from tile t0 on (a state wave that holds only some rows of d).
template <bool STORE, bool MOM, int NT>
__device__ __forceinline__ void state_io(f32x4 (&acc)[3][2][NT], float* W, float* M, int64_t j, int g, int Hd,
                                         int t0 = 0, int part = 3) {
#pragma unroll
    for (int m = 0; m < 3; ++m) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int64_t d = state_d(t0 + i, g);
            if (m < 2) {
                const int64_t o = (int64_t)m * D * Hd + d * Hd + j;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (STORE) {
                        if (MOM) M[o + r * Hd] = acc[m][0][i][r];
                        W[o + r * Hd] = acc[m][1][i][r];
                    } else {
                        if (part & 2) acc[m][0][i][r] = MOM ? M[o + r * Hd] : 0.f;
                        if (part & 1) acc[m][1][i][r] = W[o + r * Hd];
                    }
                }
            } else {
                const int64_t o = 2 * (int64_t)D * Hd + j * D + d;
                if (STORE) {
                    if (MOM) *(f32x4*)&M[o] = acc[m][0][i];
                    *(f32x4*)&W[o] = acc[m][1][i];
                } else {
                    if (part & 2) acc[m][0][i] = MOM ? *(const f32x4*)&M[o] : f32x4{0.f, 0.f, 0.f, 0.f};
                    if (part & 1) acc[m][1][i] = *(const f32x4*)&W[o];
                }
            }
        }
    }
}

// UG: 16-unit groups per workgroup (4: a 64-unit slice, 8 wavefronts, two
// per SIMD; 2 for small grids: a 32-unit slice whose 4 wavefronts each get a
// SIMD of their own, and a head's hidden units over more workgroups).
// SPREAD: the gradient waves store the weight snapshots, a few fragments per
// half-block (short chunks); else the state waves store them at the chunk
// boundary.
// PRE (precise form): every bf16 MFMA operand that is not an input -- the
// chunk-start weights in the grad products and the coefficient-scaled
// factors in the aggregation -- is a hi/lo bf16 pair summed by two MFMAs,
// and the gradient waves hand the factors over as hi/lo pairs too.  Twice the
// MFMAs and operand registers: 32-unit slices, one wavefront per SIMD (up to
// 512 registers each).  The chunk-start weight snapshot for the output stays
// the hi part.
template <bool MOM, bool SAVEM, int UG, bool SPREAD, bool PRE>
__global__ void __attribute__((amdgpu_flat_work_group_size(128 * UG, 128 * UG),
                               amdgpu_waves_per_eu(PRE ? 1 : 2, PRE ? 1 : 2)))
swiglu_loop_kernel(LoopArgs a) {
    static_assert(UG == 2 || UG == 4, "unit groups per workgroup");
    static_assert(!PRE || (UG == 2 && !SAVEM), "the precise form: 32-unit slices, weight snapshots only");
    constexpr int XWB = XW<PRE>;
    constexpr int FSET = FACB<PRE>;
    constexpr int S = 16 * UG;     // hidden units per workgroup slice
    constexpr int RPW = CB / UG;   // token rows each state wave copies per block
    // MOM = false: the recurrence without momentum; the scalar kernels then
    // have beta = 0 (cM unused, gamma = Bb = 0) and the M half of the state,
    // its aggregation MFMAs and its HBM traffic are compiled out.
    // SAVEM: also write a bf16 snapshot of every chunk's start momentum, in
    // the layout of the weight snapshot (for the backward pass).
    __shared__ __attribute__((aligned(16))) unsigned char kvs[NBUF * KVBUF];
    __shared__ __attribute__((aligned(16))) unsigned char xch[UG * XWB];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int u = wave & (UG - 1);
    const int lane = tid & 63;
    const int jl = lane & 15, g = lane >> 4;

    // XCD-aware placement: consecutive workgroup ids go to different XCDs, so
    // remap to keep the slices of one head (which read the same K/V) on one XCD.
    int L_id = blockIdx.x;
    if (a.xcd_map) L_id = (blockIdx.x % 8) * (a.nwg / 8) + blockIdx.x / 8;
    const int64_t bh = L_id / a.nsl;
    const int Hd = a.Hd;
    const int64_t j = (int64_t)(L_id % a.nsl) * S + 16 * u + jl;  // this lane's hidden unit
    const int64_t T = a.T;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int nblk = (int)((T + CB - 1) / CB);  // the last block may be partial (rows past T read as zeros)
    const int nh = a.C / 32;                     // half-blocks per chunk
    // half-blocks of chunk c: nh, except a shorter last chunk
    const int nh_last = (int)((T - (int64_t)(a.nc - 1) * a.C + 31) / 32);
    auto halves = [&](int c) { return c == a.nc - 1 ? nh_last : nh; };
    const int nc = a.nc;
    unsigned char* const xw = xch + u * XWB;  // this unit group's exchange area
    const int xl = 16 * lane;                // this lane's 16 bytes in an exchange fragment

    if (wave < UG) {
        // ------------------------------------------------------------ state wave
        // K^T / V^T fragment offsets for state tile i (16x16x32 A operand, rows
        // d in state_d order, k = 32 tokens of a half-block): lane (p, g)
        // transposes from token row tb + 4g + p/4 (k-slots 0..3) and 16 rows
        // further (4..7), d quad q = p%4 -> d = 32(i/2) + 8q + 4((q^i)&1).
        // Tiles 2t and 2t+1 share the chunk and take opposite 8-byte halves:
        // toff(2t) = te[t], toff(2t+1) = te[t] + tdelta.
        int te[4], tdelta;
        {
            const int p = lane & 15, q = p & 3;
            const int r0 = 4 * g + (p >> 2);
            const int h0 = 8 * (q & 1);
#pragma unroll
            for (int t = 0; t < 4; ++t) te[t] = r0 * 256 + 16 * ((4 * t + q) ^ swz4(r0)) + h0;
            tdelta = 8 - 2 * h0;
        }
        // HBM -> LDS copies of block X into buffer X % 3, issued by the state
        // waves (they have the slack): wave u moves K and V rows RPW u .. + RPW-1, 4
        // rows per instruction (lane L: row + L/16, chunk (L%16) ^ swz4(row),
        // landing at physical chunk L%16); wave 0 also moves the block's cM and
        // cW (one resource based at cM).
        const __bf16* kbase = a.k + bh * T * D;
        const __bf16* vbase = a.v + bh * T * D;
        const float* cMb = a.cM + bh * a.ldc;
        const unsigned cw_rel = (unsigned)((const char*)(a.cW + bh * a.ldc) - (const char*)cMb);
        const u32x4 krs = buffer_rsrc(kbase, (unsigned)(T * D * 2));
        const u32x4 vrs = buffer_rsrc(vbase, (unsigned)(T * D * 2));
        const u32x4 crs = buffer_rsrc(cMb, cw_rel + (unsigned)(a.ldc * 4));
        const unsigned kvs_lds = lds_addr(kvs);
        // (kv / coef: which parts; the folded scan copies a block's
        // coefficients only once it has written them)
        auto issue_block = [&](int X, bool kv = true, bool coef = true) {
            // per-lane offsets recomputed here rather than kept in registers
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const unsigned dst = kvs_lds + (unsigned)((X % NBUF) * KVBUF);
            const unsigned tb = (unsigned)X * CB * D * 2;
            if (kv) {
#pragma unroll
                for (int i = 0; i < RPW / 4; ++i) {
                    const int row = RPW * u + 4 * i + (ln >> 4);
                    const unsigned ko = (unsigned)(row * D + 8 * ((ln & 15) ^ swz4(row))) * 2u + tb;
                    copy16(krs, dst + (RPW * u + 4 * i) * 256, ko);
                    copy16(vrs, dst + KVB + (RPW * u + 4 * i) * 256, ko);
                }
            }
            if (coef && u == 0) {
                const unsigned coff = ln < 16 ? 16u * ln : ln < 32 ? cw_rel + 16u * (ln - 16) : 16u * (ln - 32);
                copy16(crs, dst + 2 * KVB, coff + (unsigned)X * CB * 4);
            }
        };
        // HBM -> LDS schedule: block b + 1 is issued in the slot of half-block
        // 2b - 1 (its buffer's last reader, the state waves' half-block 2b - 3,
        // finished a slot earlier) and has landed by the end of the slot of
        // half-block 2b, before the slot that reads half-block 2b + 2.
        auto copy_step = [&](int h) {
            if (h & 1) {
                const int X = (h + 3) >> 1;
                if (X < nblk) issue_block(X);
            } else {
                wait_vm<0>();
            }
        };

        const bool fold = a.fold != 0;
        issue_block(0, true, !fold);
        if (nblk > 1) issue_block(1, true, !fold);
        if (fold) slot_barrier();  // the gradient waves' gate loads are out
        // The chunk-start W first, then M: the hand-over below waits only for
        // W (loads complete in order), and M lands during the first slot,
        // where these waves only rescale while the gradient waves start.
        f32x4 acc[3][2][8];
        state_io<false, MOM, 8>(acc, (float*)a.W0 + bh * P, nullptr, j, g, Hd, 0, 1);
        state_io<false, MOM, 8>(acc, nullptr, MOM ? (float*)a.M0 + bh * P : nullptr, j, g, Hd, 0, 2);

        // chunk-start weights -> grad operands (exchange area) + bf16 snapshot
        // (with SPREAD the gradient waves store the snapshot instead)
        const bool godd = (g & 1) != 0;
        auto grad_operands = [&](int c) {
            unsigned char* snap = (unsigned char*)(a.snap + (bh * nc + c) * P);
            unsigned snap_lane = (unsigned)(j * D + 8 * g) * 2u;  // byte offset within a snapshot
            asm volatile("" : "+v"(snap_lane));                  // (recomputed per call, not kept live)
#pragma unroll
            for (int m = 0; m < 3; ++m) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    bf16x4 t0, t1, r0, r1;  // hi parts; lo parts (PRE)
                    if (PRE) {
                        split4(acc[m][1][2 * kk], t0, r0);
                        split4(acc[m][1][2 * kk + 1], t1, r1);
                    } else {
                        t0 = pack4(acc[m][1][2 * kk]);
                        t1 = pack4(acc[m][1][2 * kk + 1]);
                    }
                    const bf16x4 lo = godd ? t1 : t0, hi = godd ? t0 : t1;
                    bf16x8 w8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w8[e] = lo[e];
                        w8[4 + e] = hi[e];
                    }
                    *(bf16x8*)(xw + (4 * m + kk) * 1024 + xl) = w8;
                    if (PRE) {  // the lo parts, 12 fragments further on
                        const bf16x4 rlo = godd ? r1 : r0, rhi = godd ? r0 : r1;
                        bf16x8 l8;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            l8[e] = rlo[e];
                            l8[4 + e] = rhi[e];
                        }
                        *(bf16x8*)(xw + (12 + 4 * m + kk) * 1024 + xl) = l8;
                    }
                    if (!SPREAD) *(bf16x8*)(snap + (snap_lane + (unsigned)(m * Hd * D + 32 * kk) * 2u)) = w8;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // SAVEM: the bf16 snapshot of chunk c's start momentum, stored in the
        // chunk's first slot before its rescale (not with the grad operands,
        // so that the first hand-over waits for W only)
        auto momentum_snapshot = [&](int c) {
            unsigned char* snapm = (unsigned char*)(a.snapM + (bh * nc + c) * P);
            unsigned snap_lane = (unsigned)(j * D + 8 * g) * 2u;
            asm volatile("" : "+v"(snap_lane));
#pragma unroll
            for (int m = 0; m < 3; ++m) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x4 s0 = pack4(acc[m][0][2 * kk]), s1 = pack4(acc[m][0][2 * kk + 1]);
                    const bf16x4 mlo = godd ? s1 : s0, mhi = godd ? s0 : s1;
                    bf16x8 m8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        m8[e] = mlo[e];
                        m8[4 + e] = mhi[e];
                    }
                    *(bf16x8*)(snapm + (snap_lane + (unsigned)(m * Hd * D + 32 * kk) * 2u)) = m8;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        // W <- A W - gamma M, M <- Bb M with chunk c's scalars
        auto rescale = [&](int c) {
            const f32x4 sc = *(const f32x4*)(a.scal + (bh * nc + c) * 4);
            const float A = sc[0], Bb = sc[1], gamma = sc[2];
#pragma unroll
            for (int m = 0; m < 3; ++m) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (MOM) {
                        const f32x4 mm = acc[m][0][i];
                        acc[m][1][i] = A * acc[m][1][i] - gamma * mm;
                        acc[m][0][i] = Bb * mm;
                    } else {
                        acc[m][1][i] = A * acc[m][1][i];
                    }
                }
            }
        };
        // state += K^T F, V^T F over half-block h (tokens 32h .. 32h+31).  The
        // gradient wave hands over the unscaled factors a, b, u; here they are
        // scaled by the tokens' coefficients into the six aggregation operands
        // 1M = -cM a, 1W = cW a, 3M = -cM b, 3W = cW b, 2M = -cM u, 2W = cW u
        // (M += G^M with G^M = sum cM g, W += -G^W; du = -hv).
        auto aggregate = [&](int h) {
            const unsigned char* kb = kvs + ((h >> 1) % NBUF) * KVBUF + (h & 1) * 32 * 256;
            const unsigned char* fb = xw + (h & 1) * FSET + xl;
            const float* cob = (const float*)(kvs + ((h >> 1) % NBUF) * KVBUF + 2 * KVB) + (h & 1) * 32 + 4 * g;
            const f32x4 cm0 = *(const f32x4*)cob, cm1 = *(const f32x4*)(cob + 16);
            const f32x4 cw0 = *(const f32x4*)(cob + 64), cw1 = *(const f32x4*)(cob + 80);
            // the factor's 8 fp32 values: k-slots 0..3 and 4..7 in two 1 KB halves
            auto scale = [&](f32x4 x0, f32x4 x1, bf16x8& fm, bf16x8& fw) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = e < 4 ? x0[e] : x1[e - 4];
                    fm[e] = (__bf16)(-(e < 4 ? cm0[e] : cm1[e - 4]) * x);
                    fw[e] = (__bf16)((e < 4 ? cw0[e] : cw1[e - 4]) * x);
                }
            };
            // PRE: the factor is hi + lo of its fp32 value, and each scaled
            // operand is split into hi / lo again
            auto scale_pre = [&](bf16x8 raw, bf16x8 rawlo, bf16x8& fm, bf16x8& fw, bf16x8& fml, bf16x8& fwl) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (float)raw[e] + (float)rawlo[e];
                    const float ym = -(e < 4 ? cm0[e] : cm1[e - 4]) * x;
                    const float yw = (e < 4 ? cw0[e] : cw1[e - 4]) * x;
                    fm[e] = (__bf16)ym;
                    fw[e] = (__bf16)yw;
                    fml[e] = (__bf16)(ym - (float)fm[e]);
                    fwl[e] = (__bf16)(yw - (float)fw[e]);
                }
            };
            auto scale_any = [&](int x, bf16x8& fm, bf16x8& fw, bf16x8& fml, bf16x8& fwl) {
                if (PRE)
                    scale_pre(*(const bf16x8*)(fb + x * 1024), *(const bf16x8*)(fb + (3 + x) * 1024), fm, fw, fml,
                              fwl);
                else
                    scale(*(const f32x4*)(fb + x * 2048), *(const f32x4*)(fb + x * 2048 + 1024), fm, fw);
            };
            auto frag = [&](int i, int mat) {  // mat 0: K^T, 1: V^T
                const unsigned char* p = kb + mat * KVB + (i & 1 ? te[i >> 1] + tdelta : te[i >> 1]);
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 4096));
                bf16x8 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r[e] = lo[e];
                    r[4 + e] = hi[e];
                }
                return r;
            };
            // K^T part (W1, W3: 4 MFMAs per fragment, 8 with PRE), then V^T
            // part (W2: 2, or 4)
            bf16x8 f[4], fl[4];  // scaled operands; their lo parts (PRE)
            scale_any(0, f[0], f[1], fl[0], fl[1]);
            scale_any(1, f[2], f[3], fl[2], fl[3]);
            bf16x8 t = frag(0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // the fragment of tile i + 1 is read while tile i's MFMAs run
                const bf16x8 tn = i + 1 < 8 ? frag(i + 1, 0) : frag(0, 1);
                if (MOM) acc[0][0][i] = mfma16(t, f[0], acc[0][0][i]);
                acc[0][1][i] = mfma16(t, f[1], acc[0][1][i]);
                if (MOM) acc[1][0][i] = mfma16(t, f[2], acc[1][0][i]);
                acc[1][1][i] = mfma16(t, f[3], acc[1][1][i]);
                if (PRE) {
                    if (MOM) acc[0][0][i] = mfma16(t, fl[0], acc[0][0][i]);
                    acc[0][1][i] = mfma16(t, fl[1], acc[0][1][i]);
                    if (MOM) acc[1][0][i] = mfma16(t, fl[2], acc[1][0][i]);
                    acc[1][1][i] = mfma16(t, fl[3], acc[1][1][i]);
                }
                if (i == 7) scale_any(2, f[0], f[1], fl[0], fl[1]);
                t = tn;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bf16x8 tn = t;
                if (i + 1 < 8) tn = frag(i + 1, 1);
                if (MOM) acc[2][0][i] = mfma16(t, f[0], acc[2][0][i]);
                acc[2][1][i] = mfma16(t, f[1], acc[2][1][i]);
                if (PRE) {
                    if (MOM) acc[2][0][i] = mfma16(t, fl[0], acc[2][0][i]);
                    acc[2][1][i] = mfma16(t, fl[1], acc[2][1][i]);
                }
                t = tn;
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // Slots, as seen from the gradient waves: half-block hh for hh = 0 ..
        // nhalf-1, with one extra slot before each chunk start hh > 0.  Here:
        // a chunk's rescale runs in the slot of its first half-block, half-block
        // hh-1 is aggregated in hh's slot, and the chunk's last half-block in the
        // extra slot, which also hands over the next chunk's grad operands.
        // (Nested loops with unconditional state updates keep every state tile
        // in one register tuple for the whole sequence.)
        grad_operands(0);  // (its reads of W have waited for blocks 0 and 1's copies, issued before)
        if (fold) {
            slot_barrier();  // the gradient waves have written every chunk's coefficients
            issue_block(0, false, true);  // blocks 0 and 1's, landing beside the momentum loads
            if (nblk > 1) issue_block(1, false, true);
            wait_vm<0>();  // and have landed
        }
        slot_barrier();
        for (int c = 0;; ++c) {
            if (SAVEM) momentum_snapshot(c);
            rescale(c);
            copy_step(c * nh);
            slot_barrier();
            const int nhc = halves(c);
            for (int k = 1; k < nhc; ++k) {
                aggregate(c * nh + k - 1);
                copy_step(c * nh + k);
                slot_barrier();
            }
            aggregate(c * nh + nhc - 1);
            if (c + 1 == nc) break;
            grad_operands(c + 1);
            slot_barrier();
        }
        // lane indices re-derived here so that no prologue address survives the loop
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        state_io<true, MOM, 8>(acc, a.W_end + bh * P, MOM ? a.M_end + bh * P : nullptr, (int64_t)(L_id % a.nsl) * S + 16 * u + (lane_e & 15),
                       lane_e >> 4, Hd);
    } else {
        // ------------------------------------------------------------ gradient wave
        // K / V row fragments (16x16x32 A operand): lane (jl, g) reads token row
        // tb + 16 ti + jl, d = 32kk + 8g .. +7
        int goff[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) goff[kk] = jl * 256 + 16 * ((4 * kk + g) ^ swz4(jl));

        bf16x8 wb[3][4];  // chunk-start weights: k-slot e of lane group g is d = 32kk + 8g + e
        bf16x8 wl[3][4];  // PRE: their lo parts
        auto load_operands = [&]() {
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    wb[m][kk] = *(const bf16x8*)(xw + (4 * m + kk) * 1024 + xl);
                    if (PRE) wl[m][kk] = *(const bf16x8*)(xw + (12 + 4 * m + kk) * 1024 + xl);
                }
        };
        // grad MFMAs of half-block h: H1, H3, HV tiles of its two 16-token rows.
        // The 16 K / V row fragments are read first (one LDS round trip), then
        // the 24 MFMAs consume them.
        typedef f32x4 grad_acc[2][3];
        struct grad_frags {
            bf16x8 k[4][2], v[4][2];
        };
        auto grad_read = [&](int h, grad_frags& fr) {
            const unsigned char* kb = kvs + ((h >> 1) % NBUF) * KVBUF + (h & 1) * 32 * 256;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    fr.k[kk][ti] = *(const bf16x8*)(kb + goff[kk] + 16 * ti * 256);
                    fr.v[kk][ti] = *(const bf16x8*)(kb + KVB + goff[kk] + 16 * ti * 256);
                }
        };
        auto grad_mfma = [&](const grad_frags& fr, grad_acc& hg) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
                    hg[ti][0] = mfma16(fr.k[kk][ti], wb[0][kk], kk ? hg[ti][0] : z);
                    hg[ti][1] = mfma16(fr.k[kk][ti], wb[1][kk], kk ? hg[ti][1] : z);
                    hg[ti][2] = mfma16(fr.v[kk][ti], wb[2][kk], kk ? hg[ti][2] : z);
                }
                if (PRE) {
#pragma unroll
                    for (int ti = 0; ti < 2; ++ti) {
                        hg[ti][0] = mfma16(fr.k[kk][ti], wl[0][kk], hg[ti][0]);
                        hg[ti][1] = mfma16(fr.k[kk][ti], wl[1][kk], hg[ti][1]);
                        hg[ti][2] = mfma16(fr.v[kk][ti], wl[2][kk], hg[ti][2]);
                    }
                }
            }
        };
        // backward of half-block h from its grad tiles: the three unscaled
        // factors a = hv h3 silu'(h1) (W1), b = hv silu(h1) (W3), u = silu(h1) h3
        // (W2), with hv = V W2^T = -du, go to factor set h % 2.  k-slot e of a
        // factor fragment is token 32h + 16 (e/4) + 4g + e%4, the token order of
        // the transpose read.
        auto backward = [&](int h, const grad_acc& hg) {
            bf16x8 f[3], fl[3];  // PRE: factors as hi / lo parts
            f32x4 f32[3][2];     // otherwise in fp32, k-slots 0..3 and 4..7
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x1 = hg[ti][0][r], x3 = hg[ti][1][r], y = hg[ti][2][r];
                    const float sg = fast_sigmoid(x1);
                    const float s1 = x1 * sg;
                    const float ds = sg + s1 * (1.f - sg);
                    const int e = 4 * ti + r;
                    const float fv[3] = {y * x3 * ds, y * s1, s1 * x3};
#pragma unroll
                    for (int x = 0; x < 3; ++x) {
                        if (PRE) {
                            f[x][e] = (__bf16)fv[x];
                            fl[x][e] = (__bf16)(fv[x] - (float)f[x][e]);
                        } else {
                            f32[x][ti][r] = fv[x];
                        }
                    }
                }
            }
            unsigned char* fb = xw + (h & 1) * FSET + xl;
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                if (PRE) {
                    *(bf16x8*)(fb + x * 1024) = f[x];
                    *(bf16x8*)(fb + (3 + x) * 1024) = fl[x];
                } else {
                    *(f32x4*)(fb + x * 2048) = f32[x][0];
                    *(f32x4*)(fb + x * 2048 + 1024) = f32[x][1];
                }
            }
        };
        // With SPREAD (short chunks, whose chunk-boundary slots are a
        // large share of all slots) the gradient waves store the chunk's bf16
        // snapshot from wb, which holds it in the exchange area's lane layout
        // (fragment f = 4m + kk), a few fragments per half-block: fragments
        // f0 .. f1-1 here.  Otherwise the state waves store it at the chunk
        // boundary, which costs less on long chunks.
        auto store_snap = [&](int c, int f0, int f1) {
            unsigned char* snap = (unsigned char*)(a.snap + (bh * nc + c) * P);
            unsigned snap_lane = (unsigned)(j * D + 8 * g) * 2u;
            asm volatile("" : "+v"(snap_lane));
#pragma unroll
            for (int f = 0; f < 12; ++f)
                if (f >= f0 && f < f1)
                    *(bf16x8*)(snap + (snap_lane + (unsigned)((f >> 2) * Hd * D + 32 * (f & 3)) * 2u)) = wb[f >> 2][f & 3];
            __builtin_amdgcn_sched_barrier(0);
        };
        // The folded scan: while the state waves load the state, gradient wave
        // u computes the scalar kernels of chunks u and u + UG of its head (the
        // launcher folds only calls of at most UG chunks; every slice of the
        // head writes the same values), then waits for its stores, so that the
        // state waves' coefficient copies after the next barrier and the
        // rescales read them.  Its gate loads go out before the state waves
        // start the state load (the first barrier), so that they do not queue
        // behind it.
        if (a.fold) {
            const int npl = (a.C + 63) / 64, nm = MOM ? 0 : 1;
            scan::Gates<4> g0, g1;
            const int c0 = u, c1 = u + UG;
            if (c0 < nc) scan::load_gates<1, 4>(lane, 0, bh, c0, T, a.C, npl, nm, a.eta, a.alpha, a.beta, g0);
            if (c1 < nc) scan::load_gates<1, 4>(lane, 0, bh, c1, T, a.C, npl, nm, a.eta, a.alpha, a.beta, g1);
            slot_barrier();
            if (c0 < nc)
                scan::scan_chunk_from<1, 4>(lane, 0, bh, c0, nc, T, a.C, npl, nm, a.avg, g0, a.beta, (float*)a.cM,
                                            (float*)a.cW, a.ldc, (float*)a.scal, nullptr);
            if (c1 < nc)
                scan::scan_chunk_from<1, 4>(lane, 0, bh, c1, nc, T, a.C, npl, nm, a.avg, g1, a.beta, (float*)a.cM,
                                            (float*)a.cW, a.ldc, (float*)a.scal, nullptr);
            wait_vm<0>();
            slot_barrier();
        }
        // Slots as in the state waves' loop.  The grad MFMAs of the next
        // half-block are issued before the backward of the current one, so they
        // run in the MFMA pipe while the backward runs on the VALU; only a
        // chunk's first half-block waits for its own MFMAs.
        slot_barrier();
        for (int c = 0; c < nc; ++c) {
            if (c > 0) slot_barrier();  // the state waves finish the previous chunk
            load_operands();
            grad_acc hg;
            {
                grad_frags fr;
                grad_read(c * nh, fr);
                grad_mfma(fr, hg);
            }
            const int nhc = halves(c);
            for (int k = 0; k + 1 < nhc; ++k) {
                if (SPREAD) store_snap(c, 12 * k / nhc, 12 * (k + 1) / nhc);
                const int hh = c * nh + k;
                // next half-block's fragments, this one's backward with the next
                // one's MFMAs slotted in between its VALU work, factor writes last
                grad_frags fr;
                grad_read(hh + 1, fr);
                grad_acc hn;
                grad_mfma(fr, hn);
                backward(hh, hg);
                constexpr int NGM = PRE ? 48 : 24;  // grad MFMAs per half-block
                constexpr int VPM = PRE ? 4 : 5;    // VALU instructions slotted between two of them
                __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads: fragments
#pragma unroll
                for (int q = 0; q < NGM; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
                }
                __builtin_amdgcn_sched_group_barrier(0x200, 6, 0);  // LDS writes: factors
                slot_barrier();
#pragma unroll
                for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                    for (int m = 0; m < 3; ++m) hg[ti][m] = hn[ti][m];
            }
            if (SPREAD) store_snap(c, 12 * (nhc - 1) / nhc, 12);
            backward(c * nh + nhc - 1, hg);
            slot_barrier();
        }
    }
}


// ---------------------------------------------------------------------------
// Small grids (16- or 32-unit slices that all fit on the chip at once): block
// slots.  When the grid leaves compute units idle, a slot's length is the
// latency of one wavefront's chain, not the chip's throughput.  Every
// gradient of a chunk is taken at the chunk-start weights, so the tokens of a
// chunk need no order among themselves; only the aggregation into the state
// has to finish before the chunk boundary.  This kernel gives each slot a
// whole 64-token block and each 16-unit group eight wavefronts, so a chunk of
// C tokens takes C/64 + 1 slots (the 64-unit kernel: C/32 + 1).  Per unit
// group u (UG groups per workgroup, two or four wavefronts per SIMD):
//   state wave hf (wave 8u + hf, hf = 0..3): rows d = 32 hf .. 32 hf + 31 of the
//       group's six state matrices (tiles 2 hf, 2 hf + 1: 48 accumulator
//       registers); per block 24 MFMAs (12 without momentum) of K^T F and V^T F
//       over the block's two half-blocks; it also issues the HBM -> LDS copies;
//   gradient wave ti (wave 8u + 4 + ti): tokens 16 ti .. 16 ti + 15 of every
//       block: H1, H3, HV (12 MFMAs), the backward and the scaling by the
//       tokens' coefficients in fp32, written into its quarter of the block's
//       factor set.
// The state wave of SIMD s and the gradient wave of SIMD s overlap each
// other's MFMAs, VALU work and LDS waits.
//
// Slots (one barrier each): the slot of block X holds the gradient waves'
// work on X and the state waves' aggregation of block X - 1; a chunk's first
// slot holds the state waves' rescale instead, and a boundary slot after the
// chunk's last block holds the aggregation of that block and the hand-over.
// One unit group: four LDS blocks; block X + 2 is copied during the slot of
// block X, into the buffer block X - 2 left (its last reader, the state
// waves, finished in the slot before), and waited for at the end of the slot
// of block X + 1, so each copy has two slots to land.  Two unit groups (their
// own factor sets, the token blocks shared): three LDS blocks, block X + 1
// copied during the slot of block X and waited for at its end.
//
// Hand-over: at a chunk boundary each state wave writes the operand
// fragments of its rows of d (k-step hf of every matrix) and stores the
// snapshot.  With momentum the operands go into the factor set that the
// chunk's first block will use (12 KB, not read in the boundary slot), so the
// chunk's first slot starts with a barrier after the gradient waves have
// loaded them; without momentum they have an area of their own, and the
// same barrier is kept so that both forms share one schedule.
//
// LDS: four (one group) or three (two groups) 64-token blocks with their
// coefficients, 33 KB each; per unit group two factor sets (24 KB, or 12 KB
// and the 12 KB operand area without momentum): 156 KB or 147 KB.
template <bool MOM, bool SAVEM, int UG>
__global__ void __attribute__((amdgpu_flat_work_group_size(512 * UG, 512 * UG), amdgpu_waves_per_eu(2 * UG, 2 * UG)))
swiglu_loop_bs_kernel(LoopArgs a) {
    static_assert(UG == 1 || UG == 2, "unit groups per workgroup");
    constexpr int NF = MOM ? 6 : 3;        // factor fragments per half-block
    constexpr int FSET = 2 * NF * 1024;    // one block's factor set (two half-blocks)
    constexpr int GSZ = 2 * FSET + (MOM ? 0 : 12 * 1024);  // a unit group's factor sets (and operand area)
    constexpr int NB = UG == 1 ? 4 : 3;    // LDS token blocks
    constexpr int LEAD = NB - 2;           // blocks a copy runs ahead of the slot that issues it
    constexpr int RPW = CB / (4 * UG);     // token rows each state wave copies per block
    __shared__ __attribute__((aligned(16))) unsigned char kvs[NB * KVBUF];
    __shared__ __attribute__((aligned(16))) unsigned char fxs_all[UG * GSZ];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int u = wave >> 3;   // unit group
    const int lw = wave & 7;   // wave within the group: 0..3 state, 4..7 gradient
    unsigned char* const fxs = fxs_all + u * GSZ;
    const int lane = tid & 63;
    const int jl = lane & 15, g = lane >> 4;
    const int xl = 16 * lane;

    int L_id = blockIdx.x;
    if (a.xcd_map) L_id = (blockIdx.x % 8) * (a.nwg / 8) + blockIdx.x / 8;
    const int64_t bh = L_id / a.nsl;
    const int Hd = a.Hd;
    const int64_t j = (int64_t)(L_id % a.nsl) * 16 * UG + 16 * u + jl;  // this lane's hidden unit
    const int64_t T = a.T;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int nblk = (int)((T + CB - 1) / CB);
    const int nbc = a.C / CB;  // blocks per chunk
    const int nc = a.nc;
    const int nb_last = (int)((T - (int64_t)(nc - 1) * a.C + CB - 1) / CB);
    auto blocks = [&](int c) { return c == nc - 1 ? nb_last : nbc; };
    // chunk c's grad operands: with momentum the factor set of its first block
    auto opnd = [&](int c) { return MOM ? fxs + ((c * nbc) & 1) * FSET : fxs + 2 * FSET; };

    if (lw < 4) {
        // ------------------------------------------------------------ state wave
        const int hf = lw;
        const int cw = 4 * u + hf;  // this wave's share of the block copies
        int te, tdelta;  // transpose-read offset of this wave's rows of d (tile 2 hf; + tdelta: 2 hf + 1)
        {
            const int p = lane & 15, q = p & 3;
            const int r0 = 4 * g + (p >> 2);
            const int h0 = 8 * (q & 1);
            te = r0 * 256 + 16 * ((4 * hf + q) ^ swz4(r0)) + h0;
            tdelta = 8 - 2 * h0;
        }
        const __bf16* kbase = a.k + bh * T * D;
        const __bf16* vbase = a.v + bh * T * D;
        const float* cMb = a.cM + bh * a.ldc;
        const unsigned cw_rel = (unsigned)((const char*)(a.cW + bh * a.ldc) - (const char*)cMb);
        const u32x4 krs = buffer_rsrc(kbase, (unsigned)(T * D * 2));
        const u32x4 vrs = buffer_rsrc(vbase, (unsigned)(T * D * 2));
        const u32x4 crs = buffer_rsrc(cMb, cw_rel + (unsigned)(a.ldc * 4));
        const unsigned kvs_lds = lds_addr(kvs);
        // rows RPW cw .. + RPW - 1 of block X's K and V (rows past T read as
        // zeros), and copy wave 0 the block's coefficients: 2 RPW / 4 copies,
        // one more for copy wave 0
        // (kv / coef: which parts, as in the 64-unit kernel)
        auto issue_block = [&](int X, bool kv = true, bool coef = true) {
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const unsigned dst = kvs_lds + (unsigned)((X % NB) * KVBUF);
            const unsigned tb = (unsigned)X * CB * D * 2;
            if (kv) {
#pragma unroll
                for (int i = 0; i < RPW / 4; ++i) {
                    const int row = RPW * cw + 4 * i + (ln >> 4);
                    const unsigned ko = (unsigned)(row * D + 8 * ((ln & 15) ^ swz4(row))) * 2u + tb;
                    copy16(krs, dst + (RPW * cw + 4 * i) * 256, ko);
                    copy16(vrs, dst + KVB + (RPW * cw + 4 * i) * 256, ko);
                }
            }
            if (coef && cw == 0) {
                const unsigned coff = ln < 16 ? 16u * ln : ln < 32 ? cw_rel + 16u * (ln - 16) : 16u * (ln - 32);
                copy16(crs, dst + 2 * KVB, coff + (unsigned)X * CB * 4);
            }
        };
        // every copy older than this wave's copies of one block has landed
        auto wait_all_but_block = [&]() {
            if (cw == 0)
                wait_vm<2 * (RPW / 4) + 1>();
            else
                wait_vm<2 * (RPW / 4)>();
        };
        // the slot of block X copies block X + LEAD at its start; at its end
        // block X + 1 has landed (with LEAD = 2 the copy of block X + 2 may
        // still be in flight)
        auto issue_next = [&](int X) {
            if (X + LEAD < nblk) issue_block(X + LEAD);
        };
        auto slot_end = [&](int X) {
            if (LEAD == 2 && X + 2 < nblk)
                wait_all_but_block();
            else
                wait_vm<0>();
        };

        // With the folded scan (see the gradient waves): the coefficients of
        // blocks 0 and 1 are copied once the scan has written them.
        const bool fold = a.fold != 0;
        issue_block(0, true, !fold);
        if (LEAD == 2 && nblk > 1) issue_block(1, true, !fold);
        if (fold) slot_barrier();  // the gradient waves' gate loads are out
        f32x4 acc[3][2][2];
        state_io<false, MOM, 2>(acc, (float*)a.W0 + bh * P, MOM ? (float*)a.M0 + bh * P : nullptr, j, g, Hd, 2 * hf);

        const bool godd = (g & 1) != 0;
        // chunk c's grad operands (k-step hf of each matrix) and snapshot rows
        auto operands = [&](int c) {
            unsigned char* const od = opnd(c);
            unsigned char* snap = (unsigned char*)(a.snap + (bh * nc + c) * P);
            unsigned snap_lane = (unsigned)(j * D + 8 * g) * 2u;
            asm volatile("" : "+v"(snap_lane));
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const bf16x4 t0 = pack4(acc[m][1][0]), t1 = pack4(acc[m][1][1]);
                const bf16x4 lo = godd ? t1 : t0, hi = godd ? t0 : t1;
                bf16x8 w8;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    w8[e] = lo[e];
                    w8[4 + e] = hi[e];
                }
                *(bf16x8*)(od + (4 * m + hf) * 1024 + xl) = w8;
                *(bf16x8*)(snap + (snap_lane + (unsigned)(m * Hd * D + 32 * hf) * 2u)) = w8;
                if (SAVEM) {
                    unsigned char* snapm = (unsigned char*)(a.snapM + (bh * nc + c) * P);
                    const bf16x4 s0 = pack4(acc[m][0][0]), s1 = pack4(acc[m][0][1]);
                    const bf16x4 mlo = godd ? s1 : s0, mhi = godd ? s0 : s1;
                    bf16x8 m8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        m8[e] = mlo[e];
                        m8[4 + e] = mhi[e];
                    }
                    *(bf16x8*)(snapm + (snap_lane + (unsigned)(m * Hd * D + 32 * hf) * 2u)) = m8;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // (the chunk scalars through the scalar cache: a vector load here would
        // make the compiler wait for the block copies in flight before it)
        auto rescale = [&](int c) {
            typedef const __attribute__((address_space(4))) f32x4 const_f32x4;
            const f32x4 sc = *(const_f32x4*)(a.scal + (bh * nc + c) * 4);
            const float A = sc[0], Bb = sc[1], gamma = sc[2];
#pragma unroll
            for (int m = 0; m < 3; ++m) {
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    if (MOM) {
                        const f32x4 mm = acc[m][0][i];
                        acc[m][1][i] = A * acc[m][1][i] - gamma * mm;
                        acc[m][0][i] = Bb * mm;
                    } else {
                        acc[m][1][i] = A * acc[m][1][i];
                    }
                }
            }
        };
        // state rows += K^T F, V^T F over both half-blocks of block X with the
        // operands of factor set X % 2: (-cM a, cW a, -cM b, cW b, -cM u, cW u),
        // without momentum (cW a, cW b, cW u)
        auto aggregate = [&](int X) {
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) {
                const unsigned char* kb = kvs + (X % NB) * KVBUF + hl * 32 * 256;
                const unsigned char* fb = fxs + (X & 1) * FSET + hl * NF * 1024 + xl;
                bf16x8 f[NF];
#pragma unroll
                for (int x = 0; x < NF; ++x) f[x] = *(const bf16x8*)(fb + x * 1024);
                auto frag = [&](int i, int mat) {
                    const unsigned char* p = kb + mat * KVB + (i ? te + tdelta : te);
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p + 4096));
                    bf16x8 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        r[e] = lo[e];
                        r[4 + e] = hi[e];
                    }
                    return r;
                };
                const bf16x8 k0 = frag(0, 0), k1 = frag(1, 0), v0 = frag(0, 1), v1 = frag(1, 1);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bf16x8 t = i ? k1 : k0;
                    if (MOM) {
                        acc[0][0][i] = mfma16(t, f[0], acc[0][0][i]);
                        acc[0][1][i] = mfma16(t, f[1], acc[0][1][i]);
                        acc[1][0][i] = mfma16(t, f[2], acc[1][0][i]);
                        acc[1][1][i] = mfma16(t, f[3], acc[1][1][i]);
                    } else {
                        acc[0][1][i] = mfma16(t, f[0], acc[0][1][i]);
                        acc[1][1][i] = mfma16(t, f[1], acc[1][1][i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const bf16x8 t = i ? v1 : v0;
                    if (MOM) {
                        acc[2][0][i] = mfma16(t, f[4], acc[2][0][i]);
                        acc[2][1][i] = mfma16(t, f[5], acc[2][1][i]);
                    } else {
                        acc[2][1][i] = mfma16(t, f[2], acc[2][1][i]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        operands(0);
        if (fold) {
            slot_barrier();  // the scan's coefficients are written
            issue_block(0, false, true);
            if (LEAD == 2 && nblk > 1) issue_block(1, false, true);
            wait_vm<0>();  // blocks 0 and 1 with their coefficients have landed
        } else if (LEAD == 2 && nblk > 1) {
            wait_all_but_block();  // block 0 has landed
        } else {
            wait_vm<0>();
        }
        slot_barrier();
        // (nested loops with unconditional state updates keep every state
        // tile in one register tuple for the whole sequence)
        for (int c = 0;; ++c) {
            const int X0 = c * nbc;
            const int n = blocks(c);
            rescale(c);
            slot_barrier();  // the gradient waves have loaded the chunk's operands
            issue_next(X0);  // the slot of block X0
            slot_end(X0);
            slot_barrier();
            for (int k = 1; k < n; ++k) {  // the slot of block X0 + k
                issue_next(X0 + k);
                aggregate(X0 + k - 1);
                slot_end(X0 + k);
                slot_barrier();
            }
            aggregate(X0 + n - 1);  // the boundary slot
            if (c + 1 == nc) break;
            operands(c + 1);
            slot_barrier();
        }
        wait_vm<0>();
        int lane_e = lane;
        asm volatile("" : "+v"(lane_e));
        state_io<true, MOM, 2>(acc, a.W_end + bh * P, MOM ? a.M_end + bh * P : nullptr,
                               (int64_t)(L_id % a.nsl) * 16 * UG + 16 * u + (lane_e & 15), lane_e >> 4, Hd, 2 * hf);
    } else {
        // ------------------------------------------------------------ gradient wave
        const int ti = lw - 4;  // token rows 16 ti .. 16 ti + 15 of every block
        int goff[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) goff[kk] = jl * 256 + 16 * ((4 * kk + g) ^ swz4(jl)) + 16 * ti * 256;
        bf16x8 wb[3][4];  // chunk-start weights: k-slot e of lane group g is d = 32kk + 8g + e
        typedef f32x4 grad_acc[3];
        typedef bf16x8 rows[4];  // K or V row fragments of this wave's 16 tokens
        auto read_rows = [&](int X, int mat, rows& fr) {
            const unsigned char* kb = kvs + (X % NB) * KVBUF + mat * KVB;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fr[kk] = *(const bf16x8*)(kb + goff[kk]);
        };
        // backward of this wave's tokens of block X and the scaling:
        // a = hv h3 silu'(h1), b = hv silu(h1), u = silu(h1) h3 (hv = V W2^T =
        // -du) times the tokens' cM and cW, into k-slots 4 (ti % 2) .. + 3 of
        // the fragments of half-block ti / 2 in factor set X % 2 (k-slot e of a
        // fragment is token 16 (e/4) + 4g + e%4 of the half-block, the token
        // order of the transpose read)
        auto backward = [&](int X, const grad_acc& hg) {
            const float* cob = (const float*)(kvs + (X % NB) * KVBUF + 2 * KVB) + 16 * ti + 4 * g;
            const f32x4 cm = *(const f32x4*)cob, cw = *(const f32x4*)(cob + 64);
            float fa[4], fb[4], fu[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x1 = hg[0][r], x3 = hg[1][r], y = hg[2][r];
                const float sg = fast_sigmoid(x1);
                const float s1 = x1 * sg;
                const float ds = sg + s1 * (1.f - sg);
                fa[r] = y * x3 * ds;
                fb[r] = y * s1;
                fu[r] = s1 * x3;
            }
            unsigned char* const fo = fxs + (X & 1) * FSET + (ti >> 1) * NF * 1024 + xl + 8 * (ti & 1);
            auto put = [&](int x, const float (&v)[4], bool mom) {
                bf16x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = (__bf16)(mom ? -cm[e] * v[e] : cw[e] * v[e]);
                *(bf16x4*)(fo + x * 1024) = r;
            };
            if (MOM) {
                put(0, fa, true);
                put(1, fa, false);
                put(2, fb, true);
                put(3, fb, false);
                put(4, fu, true);
                put(5, fu, false);
            } else {
                put(0, fa, false);
                put(1, fb, false);
                put(2, fu, false);
            }
        };
        // The folded scan (calls of at most four chunks): gradient wave ti of
        // unit group 0 computes chunk ti's scalar kernels while the state
        // waves load the state, its gate loads issued before that load, as in
        // the 64-unit kernel (every slice of the head writes the same values).
        if (a.fold) {
            const int npl = (a.C + 63) / 64, nm = MOM ? 0 : 1;
            const bool mine = u == 0 && ti < nc;
            scan::Gates<4> gt;
            if (mine) scan::load_gates<1, 4>(lane, 0, bh, ti, T, a.C, npl, nm, a.eta, a.alpha, a.beta, gt);
            slot_barrier();
            if (mine)
                scan::scan_chunk_from<1, 4>(lane, 0, bh, ti, nc, T, a.C, npl, nm, a.avg, gt, a.beta, (float*)a.cM,
                                            (float*)a.cW, a.ldc, (float*)a.scal, nullptr);
            wait_vm<0>();
            slot_barrier();
        }
        slot_barrier();
        for (int c = 0; c < nc; ++c) {
            const unsigned char* const od = opnd(c);
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) wb[m][kk] = *(const bf16x8*)(od + (4 * m + kk) * 1024 + xl);
            slot_barrier();  // every gradient wave has its operands (the factors may overwrite them)
            const int X0 = c * nbc;
            const int n = blocks(c);
            for (int k = 0; k < n; ++k) {  // the slot of block X0 + k
                const int X = X0 + k;
                grad_acc hg;
                rows fk, fv;
                read_rows(X, 0, fk);
                read_rows(X, 1, fv);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
                    hg[0] = mfma16(fk[kk], wb[0][kk], kk ? hg[0] : z);
                    hg[1] = mfma16(fk[kk], wb[1][kk], kk ? hg[1] : z);
                    hg[2] = mfma16(fv[kk], wb[2][kk], kk ? hg[2] : z);
                }
                backward(X, hg);
                slot_barrier();
            }
            if (c + 1 < nc) slot_barrier();  // the boundary slot: the state waves hand over the next operands
        }
    }
}

}  // namespace

// Smaller slices only while their grid still fits on the chip at once: a
// slot takes about as long either way, so a second round of workgroups would
// cost more than the smaller slices gain.  16- and 32-unit slices take the
// block-slot kernel (eight wavefronts per unit group, a 64-token block per
// slot).
static int loop_unit_groups(int64_t BH, int64_t Hd, int ncu) {
    if (BH * (Hd / 16) <= ncu) return 1;
    return BH * (Hd / 32) <= ncu ? 2 : 4;
}

// Whether the chunk loop computes the scalar kernels itself (see the
// gradient waves' prologue): chunks of at most 256 tokens (one wavefront per
// chunk) and at most one chunk per gradient wavefront (of unit group 0 in the
// block-slot kernel).
// That is a streaming call of one or a few chunks, where the separate scan
// launch is a large share of the call.  With more chunks per wavefront the
// folded scan costs the loop about what the launch costs (1.3B-shaped
// workload, 8 chunks of 256 tokens, two per wavefront: call time equal within
// noise, loop 4 us longer).
bool swiglu_loop_scans(const e2ttt_desc& d) {
    int ncu = 0;
    if (device_cu_count(&ncu) != hipSuccess) return false;
    const bool pre = (d.flags & E2TTT_FLAG_PRECISE) != 0;
    const int ug = pre ? 2 : loop_unit_groups(d.B * d.H, d.Hd, ncu);
    const int64_t nc = (d.T + d.chunk - 1) / d.chunk;
    if (!pre && ug <= 2) return d.chunk <= 256 && nc >= 1 && nc <= 4;  // the block-slot kernel: group 0's 4 waves
    return d.chunk <= 256 && nc >= 1 && nc <= ug;
}

hipError_t launch_swiglu_loop(const e2ttt_desc& d, const void* k, const void* v, const float* cM, const float* cW,
                              int64_t ldc, const float* scal, const float* W0, const float* M0, float* W_end, float* M_end,
                              void* snap, void* snapM, hipStream_t s, const float* eta, const float* alpha,
                              const float* beta, bool fold) {
    const int64_t BH = d.B * d.H;
    LoopArgs la;
    la.eta = eta;
    la.alpha = alpha;
    la.beta = beta;
    la.fold = fold ? 1 : 0;
    la.avg = (d.flags & E2TTT_FLAG_CHUNK_AVG) ? 1 : 0;
    if (fold && (!eta || !alpha || (!(d.flags & E2TTT_FLAG_NO_MOMENTUM) && !beta) || !swiglu_loop_scans(d)))
        return hipErrorInvalidValue;
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
    la.snapM = (__bf16*)snapM;
    la.T = d.T;
    la.Hd = (int)d.Hd;
    la.C = (int)d.chunk;
    la.nc = (int)((d.T + d.chunk - 1) / d.chunk);  // the last chunk may be shorter
    la.ldc = ldc;
    // 16-unit groups per workgroup: 32-unit slices (each wavefront gets a SIMD
    // of its own) on grids small enough for them, else 64-unit slices
    int ncu = 0;
    hipError_t e;
    if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
    const bool pre = (d.flags & E2TTT_FLAG_PRECISE) != 0;
    if (pre && snapM) return hipErrorInvalidValue;  // the precise form keeps no momentum snapshots
    const int ug = pre ? 2 : loop_unit_groups(BH, d.Hd, ncu);
    la.nsl = (int)(d.Hd / (16 * ug));
    la.nwg = (int)(BH * la.nsl);
    la.xcd_map = (la.nwg % 8 == 0) ? 1 : 0;
    if (!pre && ug <= 2) {  // small grids: block slots, 16- or 32-unit slices
        const bool nm = (d.flags & E2TTT_FLAG_NO_MOMENTUM) != 0;
        // block slots: eight wavefronts per 16-unit group, a 64-token block per slot
        auto go_bs = [&](auto UGc) {
            constexpr int U = decltype(UGc)::value;
            const dim3 g1((unsigned)la.nwg), b1(512 * U);
            if (nm)
                hipLaunchKernelGGL((swiglu_loop_bs_kernel<false, false, U>), g1, b1, 0, s, la);
            else if (snapM)
                hipLaunchKernelGGL((swiglu_loop_bs_kernel<true, true, U>), g1, b1, 0, s, la);
            else
                hipLaunchKernelGGL((swiglu_loop_bs_kernel<true, false, U>), g1, b1, 0, s, la);
        };
        if (ug == 1)
            go_bs(std::integral_constant<int, 1>{});
        else
            go_bs(std::integral_constant<int, 2>{});
        return hipGetLastError();
    }
    const dim3 grid((unsigned)la.nwg), block((unsigned)(128 * ug));
    const bool nomom = (d.flags & E2TTT_FLAG_NO_MOMENTUM) != 0;
    // short chunks: the snapshot stores spread over the gradient waves' half-blocks
    const bool spread = d.chunk <= 64;
    auto go = [&](auto UGc, auto SPc) {
        constexpr int U = decltype(UGc)::value;
        constexpr bool SP = decltype(SPc)::value;
        if (nomom)
            hipLaunchKernelGGL((swiglu_loop_kernel<false, false, U, SP, false>), grid, block, 0, s, la);
        else if (snapM)
            hipLaunchKernelGGL((swiglu_loop_kernel<true, true, U, SP, false>), grid, block, 0, s, la);
        else
            hipLaunchKernelGGL((swiglu_loop_kernel<true, false, U, SP, false>), grid, block, 0, s, la);
    };
    auto go_pre = [&](auto SPc) {
        constexpr bool SP = decltype(SPc)::value;
        if (nomom)
            hipLaunchKernelGGL((swiglu_loop_kernel<false, false, 2, SP, true>), grid, block, 0, s, la);
        else
            hipLaunchKernelGGL((swiglu_loop_kernel<true, false, 2, SP, true>), grid, block, 0, s, la);
    };
    auto go_ug = [&](auto SPc) {
        if (pre)
            go_pre(SPc);
        else
            go(std::integral_constant<int, 4>{}, SPc);
    };
    if (spread)
        go_ug(std::true_type{});
    else
        go_ug(std::false_type{});
    return hipGetLastError();
}

}  // namespace e2ttt

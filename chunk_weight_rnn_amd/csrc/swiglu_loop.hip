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
// groups u = 0..3 (on small grids 4 wavefronts over a 32-unit slice, u = 0..1):
//   state wave u (wave u):      the group's fp32 W and M (6 x 128 x 16 values)
//                               as MFMA accumulators; per 32 tokens it scales
//                               the gradient wave's factors by the tokens'
//                               coefficients and adds K^T F and V^T F (48
//                               MFMAs), with K^T / V^T read from the row-major
//                               token block by the gfx950 LDS transpose read;
//                               it also issues the HBM -> LDS token copies;
//   gradient wave u (wave 4+u): the group's chunk-start weights as bf16 MFMA
//                               operands; per 32 tokens H1, H3, HV (24 MFMAs)
//                               and the backward to three unscaled bf16
//                               factors (VALU), handed over through LDS.
// The gradient wave runs one 32-token half-block ahead of the state wave and
// issues the next half-block's grad MFMAs before the current one's backward;
// one barrier per half-block separates the roles.  Sharing a SIMD, one wave's
// VALU work and LDS waits overlap the other's MFMAs.  At a chunk boundary the
// gradient waves wait one extra half-block: the next chunk's grad operands
// are the state after the previous chunk's last aggregation.
//
// LDS (150.5 KB; 123 KB for 32-unit slices): three 64-token K/V/coefficient
// blocks (the state waves' block, the gradient waves' block, one in flight
// from HBM) and per unit group a 12 KB exchange area: two half-block factor
// sets, or at a chunk boundary the 12 bf16 grad operands.  HBM -> LDS copies
// are waited for one slot before their first reader, so a barrier never
// waits on them.
#include <type_traits>

#include "e2ttt_internal.h"

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
constexpr int XW = 12 * 1024;      // exchange area per unit group
constexpr int FACB = 3 * 1024;     // one half-block factor set (3 x 64 lanes x 16 B)
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
};

// State tiles <-> packed fp32 parameters (W1 [D][Hd] | W3 [D][Hd] | W2 [Hd][D]).
// acc[m][0] / acc[m][1] are the M / W parts of matrix m (0: W1, 1: W3, 2: W2
// held transposed as [d][j]); tile element (i, r) of lane (jl, g) is
// d = state_d(i, g) + r, hidden unit j.  Without momentum M is not touched.
template <bool STORE, bool MOM>
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
                        if (MOM) M[o + r * Hd] = acc[m][0][i][r];
                        W[o + r * Hd] = acc[m][1][i][r];
                    } else {
                        acc[m][0][i][r] = MOM ? M[o + r * Hd] : 0.f;
                        acc[m][1][i][r] = W[o + r * Hd];
                    }
                }
            } else {
                const int64_t o = 2 * (int64_t)D * Hd + j * D + d;
                if (STORE) {
                    if (MOM) *(f32x4*)&M[o] = acc[m][0][i];
                    *(f32x4*)&W[o] = acc[m][1][i];
                } else {
                    acc[m][0][i] = MOM ? *(const f32x4*)&M[o] : f32x4{0.f, 0.f, 0.f, 0.f};
                    acc[m][1][i] = *(const f32x4*)&W[o];
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
template <bool MOM, bool SAVEM, int UG, bool SPREAD>
__global__ void __attribute__((amdgpu_flat_work_group_size(128 * UG, 128 * UG), amdgpu_waves_per_eu(2, 2)))
swiglu_loop_kernel(LoopArgs a) {
    static_assert(UG == 2 || UG == 4, "unit groups per workgroup");
    constexpr int S = 16 * UG;     // hidden units per workgroup slice
    constexpr int RPW = CB / UG;   // token rows each state wave copies per block
    // MOM = false: the recurrence without momentum; the scalar kernels then
    // have beta = 0 (cM unused, gamma = Bb = 0) and the M half of the state,
    // its aggregation MFMAs and its HBM traffic are compiled out.
    // SAVEM: also write a bf16 snapshot of every chunk's start momentum, in
    // the layout of the weight snapshot (for the backward pass).
    __shared__ __attribute__((aligned(16))) unsigned char kvs[NBUF * KVBUF];
    __shared__ __attribute__((aligned(16))) unsigned char xch[UG * XW];
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
    unsigned char* const xw = xch + u * XW;  // this unit group's exchange area
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
        auto issue_block = [&](int X) {
            // per-lane offsets recomputed here rather than kept in registers
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const unsigned dst = kvs_lds + (unsigned)((X % NBUF) * KVBUF);
            const unsigned tb = (unsigned)X * CB * D * 2;
#pragma unroll
            for (int i = 0; i < RPW / 4; ++i) {
                const int row = RPW * u + 4 * i + (ln >> 4);
                const unsigned ko = (unsigned)(row * D + 8 * ((ln & 15) ^ swz4(row))) * 2u + tb;
                copy16(krs, dst + (RPW * u + 4 * i) * 256, ko);
                copy16(vrs, dst + KVB + (RPW * u + 4 * i) * 256, ko);
            }
            if (u == 0) {
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

        issue_block(0);
        if (nblk > 1) issue_block(1);
        f32x4 acc[3][2][8];
        state_io<false, MOM>(acc, (float*)a.W0 + bh * P, MOM ? (float*)a.M0 + bh * P : nullptr, j, g, Hd);

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
                    const bf16x4 t0 = pack4(acc[m][1][2 * kk]), t1 = pack4(acc[m][1][2 * kk + 1]);
                    const bf16x4 lo = godd ? t1 : t0, hi = godd ? t0 : t1;
                    bf16x8 w8;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w8[e] = lo[e];
                        w8[4 + e] = hi[e];
                    }
                    *(bf16x8*)(xw + (4 * m + kk) * 1024 + xl) = w8;
                    if (!SPREAD) *(bf16x8*)(snap + (snap_lane + (unsigned)(m * Hd * D + 32 * kk) * 2u)) = w8;
                    if (SAVEM) {
                        unsigned char* snapm = (unsigned char*)(a.snapM + (bh * nc + c) * P);
                        const bf16x4 s0 = pack4(acc[m][0][2 * kk]), s1 = pack4(acc[m][0][2 * kk + 1]);
                        const bf16x4 mlo = godd ? s1 : s0, mhi = godd ? s0 : s1;
                        bf16x8 m8;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            m8[e] = mlo[e];
                            m8[4 + e] = mhi[e];
                        }
                        *(bf16x8*)(snapm + (snap_lane + (unsigned)(m * Hd * D + 32 * kk) * 2u)) = m8;
                    }
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
            const unsigned char* fb = xw + (h & 1) * FACB + xl;
            const float* cob = (const float*)(kvs + ((h >> 1) % NBUF) * KVBUF + 2 * KVB) + (h & 1) * 32 + 4 * g;
            const f32x4 cm0 = *(const f32x4*)cob, cm1 = *(const f32x4*)(cob + 16);
            const f32x4 cw0 = *(const f32x4*)(cob + 64), cw1 = *(const f32x4*)(cob + 80);
            auto scale = [&](bf16x8 raw, bf16x8& fm, bf16x8& fw) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = (float)raw[e];
                    fm[e] = (__bf16)(-(e < 4 ? cm0[e] : cm1[e - 4]) * x);
                    fw[e] = (__bf16)((e < 4 ? cw0[e] : cw1[e - 4]) * x);
                }
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
            // K^T part (W1, W3: 4 MFMAs per fragment), then V^T part (W2: 2)
            bf16x8 f[4];
            scale(*(const bf16x8*)fb, f[0], f[1]);
            scale(*(const bf16x8*)(fb + 1024), f[2], f[3]);
            bf16x8 t = frag(0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // the fragment of tile i + 1 is read while tile i's MFMAs run
                const bf16x8 tn = i + 1 < 8 ? frag(i + 1, 0) : frag(0, 1);
                if (MOM) acc[0][0][i] = mfma16(t, f[0], acc[0][0][i]);
                acc[0][1][i] = mfma16(t, f[1], acc[0][1][i]);
                if (MOM) acc[1][0][i] = mfma16(t, f[2], acc[1][0][i]);
                acc[1][1][i] = mfma16(t, f[3], acc[1][1][i]);
                if (i == 7) scale(*(const bf16x8*)(fb + 2 * 1024), f[0], f[1]);
                t = tn;
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bf16x8 tn = t;
                if (i + 1 < 8) tn = frag(i + 1, 1);
                if (MOM) acc[2][0][i] = mfma16(t, f[0], acc[2][0][i]);
                acc[2][1][i] = mfma16(t, f[1], acc[2][1][i]);
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
        grad_operands(0);
        wait_vm<0>();  // blocks 0 and 1 have landed
        slot_barrier();
        for (int c = 0;; ++c) {
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
        state_io<true, MOM>(acc, a.W_end + bh * P, MOM ? a.M_end + bh * P : nullptr, (int64_t)(L_id % a.nsl) * S + 16 * u + (lane_e & 15),
                       lane_e >> 4, Hd);
    } else {
        // ------------------------------------------------------------ gradient wave
        // K / V row fragments (16x16x32 A operand): lane (jl, g) reads token row
        // tb + 16 ti + jl, d = 32kk + 8g .. +7
        int goff[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) goff[kk] = jl * 256 + 16 * ((4 * kk + g) ^ swz4(jl));

        bf16x8 wb[3][4];  // chunk-start weights: k-slot e of lane group g is d = 32kk + 8g + e
        auto load_operands = [&]() {
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) wb[m][kk] = *(const bf16x8*)(xw + (4 * m + kk) * 1024 + xl);
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
            }
        };
        // backward of half-block h from its grad tiles: the three unscaled
        // factors a = hv h3 silu'(h1) (W1), b = hv silu(h1) (W3), u = silu(h1) h3
        // (W2), with hv = V W2^T = -du, go to factor set h % 2.  k-slot e of a
        // factor fragment is token 32h + 16 (e/4) + 4g + e%4, the token order of
        // the transpose read.
        auto backward = [&](int h, const grad_acc& hg) {
            bf16x8 f[3];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x1 = hg[ti][0][r], x3 = hg[ti][1][r], y = hg[ti][2][r];
                    const float sg = fast_sigmoid(x1);
                    const float s1 = x1 * sg;
                    const float ds = sg + s1 * (1.f - sg);
                    const int e = 4 * ti + r;
                    f[0][e] = (__bf16)(y * x3 * ds);
                    f[1][e] = (__bf16)(y * s1);
                    f[2][e] = (__bf16)(s1 * x3);
                }
            }
            unsigned char* fb = xw + (h & 1) * FACB + xl;
#pragma unroll
            for (int x = 0; x < 3; ++x) *(bf16x8*)(fb + x * 1024) = f[x];
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
                __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads: fragments
#pragma unroll
                for (int q = 0; q < 24; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                }
                __builtin_amdgcn_sched_group_barrier(0x200, 3, 0);  // LDS writes: factors
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

}  // namespace

// 32-unit slices only while their grid still fits on the chip at once: a
// slot takes about as long either way, so a second round of workgroups would
// cost more than the smaller slices gain.  (16-unit slices measured slower
// than both.)
static int loop_unit_groups(int64_t BH, int64_t Hd, int ncu) {
    return BH * (Hd / 32) <= ncu ? 2 : 4;
}

hipError_t launch_swiglu_loop(const e2ttt_desc& d, const void* k, const void* v, const float* cM, const float* cW,
                              int64_t ldc, const float* scal, const float* W0, const float* M0, float* W_end, float* M_end,
                              void* snap, void* snapM, hipStream_t s) {
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
    la.snapM = (__bf16*)snapM;
    la.T = d.T;
    la.Hd = (int)d.Hd;
    la.C = (int)d.chunk;
    la.nc = (int)((d.T + d.chunk - 1) / d.chunk);  // the last chunk may be shorter
    la.ldc = ldc;
    // 16-unit groups per workgroup: 32-unit slices (each wavefront gets a SIMD
    // of its own) on grids small enough for them, else 64-unit slices
    int dev = 0, ncu = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int ug = loop_unit_groups(BH, d.Hd, ncu);
    la.nsl = (int)(d.Hd / (16 * ug));
    la.nwg = (int)(BH * la.nsl);
    la.xcd_map = (la.nwg % 8 == 0) ? 1 : 0;
    const dim3 grid((unsigned)la.nwg), block((unsigned)(128 * ug));
    const bool nomom = (d.flags & E2TTT_FLAG_NO_MOMENTUM) != 0;
    // short chunks: the snapshot stores spread over the gradient waves' half-blocks
    const bool spread = d.chunk <= 64;
    auto go = [&](auto UGc, auto SPc) {
        constexpr int U = decltype(UGc)::value;
        constexpr bool SP = decltype(SPc)::value;
        if (nomom)
            hipLaunchKernelGGL((swiglu_loop_kernel<false, false, U, SP>), grid, block, 0, s, la);
        else if (snapM)
            hipLaunchKernelGGL((swiglu_loop_kernel<true, true, U, SP>), grid, block, 0, s, la);
        else
            hipLaunchKernelGGL((swiglu_loop_kernel<true, false, U, SP>), grid, block, 0, s, la);
    };
    auto go_ug = [&](auto SPc) {
        if (ug == 4)
            go(std::integral_constant<int, 4>{}, SPc);
        else
            go(std::integral_constant<int, 2>{}, SPc);
    };
    if (spread)
        go_ug(std::true_type{});
    else
        go_ug(std::false_type{});
    return hipGetLastError();
}

}  // namespace e2ttt

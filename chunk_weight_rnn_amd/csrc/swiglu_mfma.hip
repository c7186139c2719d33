// SwiGLU fast weight, negative-dot loss, bf16 q/k/v/out: the CDNA4 (gfx950)
// MFMA path of the E2-TTT chunk update, and its output kernel.
//
// Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
// (abstract; atlas summary "Approach"): gradients at the chunk-start weights,
// two scalar kernels, two weighted gradient aggregations, and the chunk
// output from the chunk-start weights (arxivlens "Limitations").
//
//   apply:      out = (silu(Q W1) * (Q W3)) W2     (W = chunk-start weights)
//
// The chunk loop (swiglu_loop.hip) keeps each 64-unit hidden slice's state
// on chip and writes a bf16 snapshot of every chunk's start weights; the
// output needs all hidden units of a head, so this second, fully parallel
// kernel computes every chunk's output from the snapshots.
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
constexpr int S = 64;    // hidden units per loop-kernel slice
constexpr int CB = 64;   // tokens per loop-kernel block

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
        int nrows;         // rows of this wave inside the sequence (a short last chunk has fewer)
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
        const int64_t tl = (int64_t)c * a.C + (int64_t)rb * 32 * NWA + 32 * wave;  // token within the sequence
        it.tok = bh * a.T + tl;
        it.nrec = ok ? (int)(P * 2) : 0;
        it.nrows = ok ? (int)(a.T - tl < 0 ? 0 : (a.T - tl > 32 ? 32 : a.T - tl)) : 0;
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
        const int qrec = it.nrows * D * 2;  // rows past the sequence read zeros
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
            const Item it = item(gs / nhb);
            __bf16* ob = a.out + it.tok * D;
            const bool row_ok = li < it.nrows;  // no stores past the sequence
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int d = 32 * dt + 8 * qd + 4 * lg;
                    if (row_ok)
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
    // the chunk loop addresses each head's K / V rows through 32-bit buffer
    // offsets, so one head's rows must stay below 2 GiB (T < 8M tokens)
    return d.kind == E2TTT_SWIGLU && d.loss == E2TTT_LOSS_NEGDOT && d.io_dtype == E2TTT_BF16 && d.D == D &&
           d.Hd >= S && d.Hd % S == 0 && d.Hd <= 4096 && d.chunk % CB == 0 && d.T * D * 2 < ((int64_t)1 << 31);
}

hipError_t launch_swiglu_mfma(const e2ttt_desc& d, const void* q, const void* k, const void* v, const float* cM,
                              const float* cW, int64_t ldc, const float* scal, const float* W0, const float* M0, void* out,
                              float* W_end, float* M_end, void* snap, void* snapM, hipStream_t s, hipEvent_t ev_mid) {
    const int64_t BH = d.B * d.H;
    hipError_t e = launch_swiglu_loop(d, k, v, cM, cW, ldc, scal, W0, M0, W_end, M_end, snap, snapM, s);
    if (e != hipSuccess) return e;
    if (ev_mid && (e = hipEventRecord(ev_mid, s)) != hipSuccess) return e;

    ApplyArgs aa;
    aa.q = (const __bf16*)q;
    aa.snap = (const __bf16*)snap;
    aa.out = (__bf16*)out;
    aa.T = d.T;
    aa.Hd = (int)d.Hd;
    aa.C = (int)d.chunk;
    aa.nc = (int)((d.T + d.chunk - 1) / d.chunk);  // the last chunk may be shorter
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

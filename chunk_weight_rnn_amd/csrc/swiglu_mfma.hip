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
#include <type_traits>

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
// in a ring of stages (all but one in flight while one is consumed).
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
    int hord;            // 1: the chunk loop placed heads by XCD (B H a multiple of 8), see apply_head
};

// The head of the output kernels' r-th group of items.  Heads are visited in
// the reverse of the order in which the chunk loop's workgroups were
// dispatched, so that the snapshots written last are read first, while the
// 256 MB last-level cache may still hold them.  With B H a multiple of 8 the
// loop places the slices of head x (B H / 8) + i on XCD x and dispatches the
// heads in the order (i, x); otherwise in head order (a permutation either
// way: only the cache hits depend on it).
__device__ __forceinline__ int64_t apply_head(int64_t r, int64_t BH, int hord) {
    const int64_t n = BH - 1 - r;  // the head's dispatch rank in the chunk loop
    return hord ? (n % 8) * (BH / 8) + n / 8 : n;
}

constexpr int HB = 32;                     // hidden units per stage
constexpr int STAGE_BYTES = 3 * HB * 256;  // W1^T, W3^T, W2 rows of the stage

// Stage rows are 256 bytes with 16-byte chunk c of row t at physical chunk
// c ^ swza(t).  The grad-style row reads (16 consecutive rows at one chunk)
// see a permutation of all 16 chunks, and each 32-lane half of a 32x32
// transpose fragment (4 consecutive rows x 4 chunks x 2 halves) sees four
// disjoint 4-chunk groups: conflict-free on the 64 four-byte banks.
__device__ __forceinline__ int swza(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

// Per-lane byte offset, within a stage's W2 block, of one half of a 32x16
// MFMA operand fragment transposed out of the swizzled row-major [rows][128]
// bf16 rows: operand row = W2 column 32 dt + lane%32, operand k 0..3 = W2
// rows 16 s + 4 lg + {0..3} (hi = 0) and k 4..7 the same + 8 (hi = 1).  The
// k-step s adds 16 rows, 4096 bytes, and does not change the swizzle.
__device__ __forceinline__ unsigned tr_offset(int dt, int hi, int lane) {
    const int p = lane & 15, G = lane >> 4;
    const int r = 4 * (G >> 1) + 8 * hi + (p >> 2);
    const int chunk = 4 * dt + 2 * (G & 1) + ((p & 3) >> 1);
    return (unsigned)(r * 256 + 16 * (chunk ^ swza(r)) + 8 * (p & 1));
}

__device__ __forceinline__ bf16x8 tr_frag_at(const unsigned char* base, unsigned off0, unsigned off1) {
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + off0));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + off1));
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = lo[e];
        r[4 + e] = hi[e];
    }
    return r;
}

// Wave-uniform values the compiler cannot prove uniform (loop-carried
// cursors): read from the first lane so buffer descriptors stay in SGPRs.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (void*)(((uint64_t)hi << 32) | lo);
}

// direct HBM->LDS copy of 16 bytes per lane (buffer form; lane L writes
// dst + 16 L); offsets at or past num_bytes read zeros
__device__ __forceinline__ void lds_copy16(const void* base, int num_bytes, unsigned char* dst, unsigned voff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), 0, uniform(num_bytes), RSRC_W3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, voff, 0, 0, 0);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) with every other counter left alone (N < 64)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that waits for this wave's LDS accesses but not for its
// HBM -> LDS copies in flight (__syncthreads would wait for every load).
__device__ __forceinline__ void stage_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The stage ring: separate LDS objects, so that the compiler can tell the
// copies in flight from the reads of the stage being consumed.
__shared__ __attribute__((aligned(16))) unsigned char apply_sb0[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) unsigned char apply_sb1[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) unsigned char apply_sb2[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) unsigned char apply_sb3[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) unsigned char apply_sb4[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) unsigned char apply_sb5[STAGE_BYTES];
constexpr int NS_MAX = 6;

template <int I>
__device__ __forceinline__ unsigned char* stage_buf() {
    static_assert(I >= 0 && I < NS_MAX, "stage ring index");
    if constexpr (I == 0) return apply_sb0;
    else if constexpr (I == 1) return apply_sb1;
    else if constexpr (I == 2) return apply_sb2;
    else if constexpr (I == 3) return apply_sb3;
    else if constexpr (I == 4) return apply_sb4;
    else return apply_sb5;
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// LDS of a compute unit, and workgroups of the output kernel per compute unit
constexpr int LDS_PER_CU = 160 * 1024;
template <int NS>
constexpr int apply_wg_per_cu() { return LDS_PER_CU / (NS * STAGE_BYTES); }

// Persistent: every workgroup walks a list of items (an item = 32 NWA tokens
// of one chunk) so the stage copies never stop between items.  NS stage
// buffers form a ring with NS - 1 stages in flight while one is consumed.
// Each wavefront loads its own 32 query rows of the next item straight into
// registers while the current item runs.
template <int NWA, int NS>
__global__ __launch_bounds__(64 * NWA) void swiglu_apply_kernel(ApplyArgs a) {
    constexpr int NI = 24 / NWA;  // stage copy instructions per wave per stage
    constexpr int NQ = 8;         // query loads per wave per item (16 bytes per lane each)
    static_assert(NS >= 3 && NS <= NS_MAX, "stage ring size");
    static_assert((NS - 2) * NI + 3 * NQ < 64, "wait counts must fit vmcnt");
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 31, lg = lane >> 5;
    const int Hd = a.Hd;
    const int64_t P = 3 * (int64_t)D * Hd;
    const int nhb = Hd / HB;
    const int64_t nitems = (int64_t)a.nb * a.nc * a.rbc;
    // items of this workgroup: blockIdx.x + k gridDim.x
    const int nmine = (int)((nitems - blockIdx.x + gridDim.x - 1) / gridDim.x);

    struct Item {
        const __bf16* sn;  // snapshot of the item's chunk
        int64_t tok;       // first token (global row in q / out) of this wave
        int nrec;          // bytes the copies may read (0 past the last item: zeros)
        int nrows;         // rows of this wave inside the sequence (a short last chunk has fewer)
    };
    auto item = [&](int k) __attribute__((always_inline)) {
        Item it;
        const int64_t x = blockIdx.x + (int64_t)k * gridDim.x;
        const bool ok = k < nmine;
        const int64_t xx = ok ? x : 0;
        const int64_t bh = apply_head(xx / ((int64_t)a.nc * a.rbc), a.nb, a.hord);
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
    // The copy stream runs NS - 1 stages ahead of the computation.  Each
    // stream keeps a cursor (item, stage within the item), so an item's
    // position (64-bit divisions, done by the scalar unit) is worked out once
    // per item rather than at every stage.
    Item citem = item(0);
    int ck = 0, cih = 0;
    auto issue_next_copy = [&](unsigned char* buf) __attribute__((always_inline)) {
        const unsigned ho = (unsigned)(cih * HB * D * 2);
#pragma unroll
        for (int n = 0; n < NI; ++n) lds_copy16(citem.sn, citem.nrec, buf + mrow[n], voff[n] + ho);
        if (++cih == nhb) {
            cih = 0;
            citem = item(++ck);
        }
    };
    // Q^T as the B operand of the first product (col = token li, k = d):
    // lane (li, lg) holds q[li][16 ks + 8 lg .. + 7] for k-step ks.  Rows past
    // the sequence read zeros.
    auto load_q = [&](const Item& it, bf16x8(&dst)[8]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.q + it.tok * D), 0, uniform(it.nrows * D * 2), RSRC_W3);
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, (li * D + 16 * ks + 8 * lg) * 2, 0, 0);
            dst[ks] = __builtin_bit_cast(bf16x8, w);
        }
    };

    // per-lane LDS offsets of the stage reads, the same for every buffer of the ring
    unsigned rd_off[8], tr_off[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) rd_off[ks] = (unsigned)(li * 256 + 16 * ((2 * ks + lg) ^ swza(li)));
#pragma unroll
    for (int i = 0; i < 8; ++i) tr_off[i] = tr_offset(i >> 1, i & 1, lane);

    bf16x8 qf[8], qn[8];
    f32x16 oacc[4] = {};
    Item cur = item(0), nxt = cur;  // the item being computed, and the next one
    load_q(cur, qn);                // the first item's queries precede every copy
    static_for<0, NS - 1>([&](auto I) __attribute__((always_inline)) { issue_next_copy(stage_buf<decltype(I)::value>()); });

    int ih = 0;          // stage within the current item
    unsigned qmask = 0;  // bit j: a query batch was issued j + 1 stages ago (j < NS - 1)
    int k = 0;           // current item
    auto stage = [&](const unsigned char* st, unsigned char* refill) __attribute__((always_inline)) {
        // This stage's copies landed once at most the loads issued after them
        // are outstanding: the copies of the next NS - 2 stages and the query
        // batches of the last NS - 1 stages.  (Loads complete in order; the
        // output stores are not counted, which only waits longer.)
        switch (__builtin_popcount(qmask)) {
            case 0: wait_vm<(NS - 2) * NI>(); break;
            case 1: wait_vm<(NS - 2) * NI + NQ>(); break;
            case 2: wait_vm<(NS - 2) * NI + 2 * NQ>(); break;
            default: wait_vm<(NS - 2) * NI + 3 * NQ>(); break;
        }
        stage_barrier();
        issue_next_copy(refill);  // refill = buffer of the previous stage, free after the barrier
        qmask = (qmask << 1) & ((1u << (NS - 1)) - 1);
        if (ih == 0) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) qf[ks] = qn[ks];
            nxt = item(k + 1);
            load_q(nxt, qn);
            qmask |= 1;
        }
        // The offsets are opaque to the optimiser here, so each read adds its
        // offset to this stage's buffer instead of the kernel keeping the
        // addresses of every buffer of the ring in registers.
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(rd_off[i]), "+v"(tr_off[i]));
        f32x16 x1 = {}, x3 = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            x1 = mfma32(*(const bf16x8*)(st + rd_off[ks]), qf[ks], x1);
            x3 = mfma32(*(const bf16x8*)(st + HB * 256 + rd_off[ks]), qf[ks], x3);
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
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                oacc[dt] = mfma32(tr_frag_at(w2 + 4096 * s, tr_off[2 * dt], tr_off[2 * dt + 1]), ub[s], oacc[dt]);
        if (++ih == nhb) {
            __bf16* ob = a.out + cur.tok * D;
            const bool row_ok = li < cur.nrows;  // no stores past the sequence
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
            ih = 0;
            ++k;
            cur = nxt;
        }
    };
    const int nst = nmine * nhb;
    for (int gs = 0; gs < nst; gs += NS) {
        static_for<0, NS>([&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            if (gs + i < nst) stage(stage_buf<i>(), stage_buf<(i + NS - 1) % NS>());
        });
    }
    wait_vmem();  // copies past the last item (zeros) land before the LDS goes away
}


// ---------------------------------------------------------------------------
// The output kernel for Hd = 256 (items of eight stages) and chunks of a
// multiple of 256 tokens: a four-stage ring, so that every item starts at
// ring buffer 0 and a loop iteration is straight-line code over two items
// (the query registers alternate between them, so no register copy has to
// wait for query loads).
//
// Each item's memory traffic besides the stage copies is spread over its
// first stages: the next item's eight query loads in its first two stages
// (four a stage: each a whole 128-byte line of every query row; two a stage
// over four stages fetched 15% more than the queries from HBM), and two of
// the previous item's eight output stores in each of its first four.  Every wait on the
// in-order memory counter therefore allows exactly the operations issued
// after the stage's copies (vm_allowed below).  (The six-stage ring moved an
// item's start through its unrolled loop; the compiler then had to assume
// the query loads had just been issued, and its wait for them drained every
// copy in flight, while the item's 16 stores went out at once from every
// workgroup and the next stage's wait, which did not count them, waited for
// them as well.)
//
// The outputs leave through LDS: each wavefront writes its 32 x 128 tile
// there in halves of 64 columns and reads it back as rows, so that a store
// instruction writes eight 128-byte row segments instead of 16-byte pieces
// of 32 rows.  They are buffer stores whose range ends at the last row inside
// the sequence: every lane issues them (so the counts hold), and the
// hardware drops rows past it; the first item's stand-in stores have an
// empty range.
// ---------------------------------------------------------------------------
__shared__ __attribute__((aligned(16))) unsigned char apply_ost[8 * 32 * 128];

// Memory operations a stage at item position p (0..7) lets stay in flight
// at its wait: issued after its copies (three stages earlier) are the copies
// of the two stages between, and the query loads (four at positions 0 and
// 1) and output stores (two at positions 0..3) among those three positions.
__host__ __device__ constexpr int vm_allowed(int p, int ni) {
    int n = 2 * ni;
    for (int x = p - 3; x < p; ++x) {
        const int y = (x + 8) % 8;
        n += (y < 2 ? 4 : 0) + (y < 4 ? 2 : 0);
    }
    return n;
}

template <int NWA>
__global__ __launch_bounds__(64 * NWA) void swiglu_apply_h256_kernel(ApplyArgs a) {
    constexpr int NS = 4;         // ring buffers
    constexpr int NHB = 8;        // stages per item (Hd = 256)
    constexpr int NI = 24 / NWA;  // stage copy instructions per wave per stage
    static_assert(vm_allowed(3, NI) < 64, "wait counts must fit vmcnt");
    static_assert(NWA * 32 * 128 <= (int)sizeof(apply_ost), "output staging");
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 31, lg = lane >> 5;
    constexpr int Hd = NHB * HB;
    constexpr int64_t P = 3 * (int64_t)D * Hd;
    const int64_t nitems = (int64_t)a.nb * a.nc * a.rbc;
    const int nmine = (int)((nitems - blockIdx.x + gridDim.x - 1) / gridDim.x);

    struct Item {
        const __bf16* sn;  // snapshot of the item's chunk
        int64_t tok;       // first token (global row in q / out) of this wave
        int nrec;          // bytes the copies may read (0 past the last item: zeros)
        int nrows;         // rows of this wave inside the sequence
    };
    auto item = [&](int k) __attribute__((always_inline)) {
        Item it;
        const int64_t x = blockIdx.x + (int64_t)k * gridDim.x;
        const bool ok = k < nmine;
        const int64_t xx = ok ? x : 0;
        const int64_t bh = apply_head(xx / ((int64_t)a.nc * a.rbc), a.nb, a.hord);
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
    // the copy stream, NS - 1 stages ahead of the computation (across items)
    Item citem = item(0);
    int ck = 0, cih = 0;
    auto issue_next_copy = [&](unsigned char* buf) __attribute__((always_inline)) {
        const unsigned ho = (unsigned)(cih * HB * D * 2);
#pragma unroll
        for (int n = 0; n < NI; ++n) lds_copy16(citem.sn, citem.nrec, buf + mrow[n], voff[n] + ho);
        if (++cih == NHB) {
            cih = 0;
            citem = item(++ck);
        }
    };
    // Q^T as the B operand of the first product (as in swiglu_apply_kernel):
    // k-steps ks0, ks0 + 1 of an item's queries
    auto q_rsrc = [&](const Item& it) __attribute__((always_inline)) {
        return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.q + it.tok * D), 0, uniform(it.nrows * D * 2), RSRC_W3);
    };
    auto load_q2 = [&](__amdgpu_buffer_rsrc_t r, int ks0, bf16x8(&dst)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = ks0; ks < ks0 + 2; ++ks) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, (li * D + 16 * ks + 8 * lg) * 2, 0, 0);
            dst[ks] = __builtin_bit_cast(bf16x8, w);
        }
    };

    unsigned rd_off[8], tr_off[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) rd_off[ks] = (unsigned)(li * 256 + 16 * ((2 * ks + lg) ^ swza(li)));
#pragma unroll
    for (int i = 0; i < 8; ++i) tr_off[i] = tr_offset(i >> 1, i & 1, lane);

    // output pieces: piece 4 h + i is row 8 i + 2 ((L >> 3) & 3) + (L >> 5),
    // columns 64 h + 8 (L & 7) .. + 7 of lane L
    const int orow = 2 * ((lane >> 3) & 3) + (lane >> 5), ocol = 8 * (lane & 7);
    unsigned char* const ost = apply_ost + wave * (32 * 128);  // this wave's output staging
    bf16x8 qa[8], qb[8];
    u32x4 vout[8];                                               // the previous item's output pieces
    __amdgpu_buffer_rsrc_t orsrc = q_rsrc(Item{a.q, 0, 0, 0});  // their range: empty before the first item
    f32x16 oacc[4] = {};
    Item cur = item(0);
    int k = 0;
    {
        const __amdgpu_buffer_rsrc_t r = q_rsrc(cur);  // the first item's queries precede every copy
#pragma unroll
        for (int ks = 0; ks < 8; ks += 2) load_q2(r, ks, qa);
    }
    static_for<0, NS - 1>([&](auto I) __attribute__((always_inline)) { issue_next_copy(stage_buf<decltype(I)::value>()); });

    // the stage at item position p (ring buffer p % 4) on queries qu; at
    // positions 0 and 1 also four of the next item's query loads into qn, at
    // positions 0..3 two of the previous item's output stores
    auto stage = [&](auto Pc, const bf16x8(&qu)[8], bf16x8(&qn)[8], __amdgpu_buffer_rsrc_t qr)
        __attribute__((always_inline)) {
        constexpr int p = decltype(Pc)::value;
        constexpr int I = p % NS;
        const unsigned char* st = stage_buf<I>();
        wait_vm<vm_allowed(p, NI)>();
        stage_barrier();
        issue_next_copy(stage_buf<(I + NS - 1) % NS>());  // the buffer the previous stage read
        if constexpr (p < 2) {
            load_q2(qr, 4 * p, qn);
            load_q2(qr, 4 * p + 2, qn);
        }
        if constexpr (p < 4) {
#pragma unroll
            for (int j = 2 * p; j < 2 * p + 2; ++j)
                __builtin_amdgcn_raw_buffer_store_b128(vout[j], orsrc, ((8 * (j & 3) + orow) * D + 64 * (j >> 2) + ocol) * 2, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(rd_off[i]), "+v"(tr_off[i]));
        f32x16 x1 = {}, x3 = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            x1 = mfma32(*(const bf16x8*)(st + rd_off[ks]), qu[ks], x1);
            x3 = mfma32(*(const bf16x8*)(st + HB * 256 + rd_off[ks]), qu[ks], x3);
        }
        bf16x8 ub[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = 8 * s2 + e;
                const float h = x1[r];
                ub[s2][e] = (__bf16)(h * fast_sigmoid(h) * x3[r]);
            }
        const unsigned char* w2 = st + 2 * HB * 256;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                oacc[dt] = mfma32(tr_frag_at(w2 + 4096 * s2, tr_off[2 * dt], tr_off[2 * dt + 1]), ub[s2], oacc[dt]);
    };
    // The item's outputs into vout through the staging, in two halves of 64
    // columns.  Staging row t holds token t's 128 bytes of the half, 16-byte
    // chunk c at physical chunk c ^ ((t >> 1) & 7); written by lane (li, lg)
    // in 8-byte pieces (columns 32 dt + 8 qd + 4 lg ..), read back as the
    // output pieces, so that the two 8-lane groups a 128-bit read serves
    // together see rows of opposite parity.
    auto item_end = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int dd = 0; dd < 2; ++dd)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x16& o = oacc[2 * h + dd];
                    const int c = 4 * dd + qd;
                    *(bf16x4*)(ost + li * 128 + 16 * (c ^ ((li >> 1) & 7)) + 8 * lg) =
                        pack4(o[4 * qd], o[4 * qd + 1], o[4 * qd + 2], o[4 * qd + 3]);
                }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 8 * i + orow;
                vout[4 * h + i] = *(const u32x4*)(ost + row * 128 + 16 * ((ocol >> 3) ^ ((row >> 1) & 7)));
            }
        }
        orsrc = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.out + cur.tok * D), 0, uniform(cur.nrows * D * 2), RSRC_W3);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
    };
    // one item on the queries in qu, loading the next item's into qn
    auto one_item = [&](const bf16x8(&qu)[8], bf16x8(&qn)[8]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t qr = q_rsrc(item(k + 1));
        static_for<0, NHB>([&](auto Pc) __attribute__((always_inline)) { stage(Pc, qu, qn, qr); });
        item_end();
        cur = item(++k);
    };
    while (true) {
        one_item(qa, qb);
        if (k >= nmine) break;
        one_item(qb, qa);
        if (k >= nmine) break;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)  // the last item's outputs
        __builtin_amdgcn_raw_buffer_store_b128(vout[j], orsrc, ((8 * (j & 3) + orow) * D + 64 * (j >> 2) + ocol) * 2, 0, 0);
    wait_vmem();  // and the copies past the last item (zeros) land before the LDS goes away
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
                              float* W_end, float* M_end, void* snap, void* snapM, hipStream_t s, hipEvent_t ev_mid,
                              const float* eta, const float* alpha, const float* beta, bool fold) {
    const int64_t BH = d.B * d.H;
    hipError_t e = launch_swiglu_loop(d, k, v, cM, cW, ldc, scal, W0, M0, W_end, M_end, snap, snapM, s, eta, alpha,
                                      beta, fold);
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
    aa.hord = (BH % 8 == 0) ? 1 : 0;  // the loop's XCD placement (its grid is then a multiple of 8)
    // persistent grid: as many workgroups as the compute units hold at once
    int ncu = 0;
    if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
    const int64_t nck = BH * aa.nc;
    auto grid = [&](int64_t items, int per_cu) {
        const int64_t cap = (int64_t)ncu * per_cu;
        return dim3((unsigned)(items < cap ? items : cap));
    };
    if (d.chunk % 256 == 0 && d.Hd == 8 * HB) {
        aa.rbc = (int)(d.chunk / 256);
        hipLaunchKernelGGL((swiglu_apply_h256_kernel<8>), grid(nck * aa.rbc, 1), dim3(512), 0, s, aa);
    } else if (d.chunk % 256 == 0) {
        aa.rbc = (int)(d.chunk / 256);
        hipLaunchKernelGGL((swiglu_apply_kernel<8, 6>), grid(nck * aa.rbc, apply_wg_per_cu<6>()), dim3(512), 0, s, aa);
    } else if (d.chunk % 128 == 0) {
        aa.rbc = (int)(d.chunk / 128);
        hipLaunchKernelGGL((swiglu_apply_kernel<4, 3>), grid(nck * aa.rbc, apply_wg_per_cu<3>()), dim3(256), 0, s, aa);
    } else {
        aa.rbc = (int)(d.chunk / 64);
        hipLaunchKernelGGL((swiglu_apply_kernel<2, 3>), grid(nck * aa.rbc, apply_wg_per_cu<3>()), dim3(128), 0, s, aa);
    }
    return hipGetLastError();
}

}  // namespace e2ttt

// Host side of the C ABI declared in include/e2ttt.h: descriptor and pointer
// validation (pure host code, callable without a GPU), workspace layout and
// dispatch of the device kernels on the caller's stream.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "e2ttt_internal.h"

// Scratch of e2ttt_chunk_forward_noalloc: a file-scope device array, one copy
// per GPU, allocated when the code object loads and held until the process
// ends.  Host code never uses its name as an address: the address of the
// current device's copy comes from hipGetSymbolAddress (scratch_address).
static __device__ __align__(256) unsigned char scratch[E2TTT_NOALLOC_SCRATCH_BYTES];

namespace e2ttt {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];  // per device, filled on its first no-allocation call
std::mutex scratch_mu;
}  // namespace

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
static hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(scratch_mu);
        p = scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t device_cu_count(int* ncu) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];  // 0 = not queried yet
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *ncu = c;
            return hipSuccess;
        }
    }
    int n = 0;
    if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if (n < 1) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    *ncu = n;
    return hipSuccess;
}

static bool desc_ok(const e2ttt_desc* d) {
    if (!d) return false;
    if (d->kind < E2TTT_LINEAR || d->kind > E2TTT_SWIGLU) return false;
    if (d->loss < E2TTT_LOSS_MSE || d->loss > E2TTT_LOSS_NEGDOT) return false;
    if (d->io_dtype < E2TTT_F32 || d->io_dtype > E2TTT_BF16) return false;
    if (d->B < 0 || d->H < 0 || d->T < 0 || d->D < 1 || d->chunk < 1) return false;
    if (d->chunk > INT32_MAX) return false;  // kernels take the chunk length as a 32-bit int
    if (d->kind != E2TTT_LINEAR && d->Hd < 1) return false;
    if (d->flags & ~(E2TTT_FLAG_FORCE_GENERIC | E2TTT_FLAG_NO_MOMENTUM | E2TTT_FLAG_CHUNK_AVG |
                     E2TTT_FLAG_SAVE_STATES | E2TTT_FLAG_PRECISE))
        return false;
    // keep every product used for indexing far from int64 overflow
    const int64_t lim = (int64_t)1 << 40;
    if (d->B > lim || d->H > lim || d->T > lim || d->D > 65536 || d->Hd > 65536) return false;
    if (d->B * d->H > lim || d->B * d->H * d->T > lim) return false;
    return true;
}

// The fields e2ttt_logscan reads: sizes, the chunk length and the flags
// (kind, loss, dtype, D and Hd are ignored there).
static bool logscan_desc_ok(const e2ttt_desc* d) {
    if (!d) return false;
    if (d->B < 0 || d->H < 0 || d->T < 0 || d->chunk < 1 || d->chunk > INT32_MAX) return false;
    if (d->flags & ~(E2TTT_FLAG_FORCE_GENERIC | E2TTT_FLAG_NO_MOMENTUM | E2TTT_FLAG_CHUNK_AVG |
                     E2TTT_FLAG_SAVE_STATES | E2TTT_FLAG_PRECISE))
        return false;
    const int64_t lim = (int64_t)1 << 40;
    if (d->B > lim || d->H > lim || d->T > lim || d->B * d->H > lim || d->B * d->H * d->T > lim) return false;
    return true;
}

// 0: portable fp32 kernel, 1: SwiGLU bf16 MFMA path, 2: the same with hi/lo
// bf16 operands (E2TTT_FLAG_PRECISE), 3: fp32 MFMA path (linear / MLP, fp32
// I/O, one workgroup per head), 4: the same for the MLP split over hidden
// slices (few heads)
static int path_of(const e2ttt_desc& d) {
    if (d.flags & E2TTT_FLAG_FORCE_GENERIC) return 0;
    if (swiglu_mfma_supported(d)) return (d.flags & E2TTT_FLAG_PRECISE) ? 2 : 1;
    if (f32_mfma_supported(d)) return f32_split(d) ? 4 : 3;
    return 0;
}

// A forward with E2TTT_FLAG_SAVE_STATES leaves what its backward reads: the
// bf16 snapshots for the MFMA backward, the fp32 chunk-start states for the
// portable backward (written by both fp32 forward paths).
static bool save_compatible(int fwd_path, int bwd_path) {
    return (fwd_path == 1 && bwd_path == 1) || ((fwd_path == 0 || fwd_path >= 3) && bwd_path == 0);
}

static bool generic_supported(const e2ttt_desc& d) {
    if (d.D > 256) return false;
    if (d.kind != E2TTT_LINEAR && d.Hd > 1024) return false;
    return true;
}

// ---------------------------------------------------------------- backward
// 1: SwiGLU MFMA backward, 0: portable fp32 backward, -1: unsupported
static int backward_path(const e2ttt_desc& d) {
    if (d.chunk > 2048) return -1;  // the scalar backward stages one chunk in LDS
    // a precise forward is differentiated by the portable fp32 backward
    if (!(d.flags & (E2TTT_FLAG_FORCE_GENERIC | E2TTT_FLAG_PRECISE)) && swiglu_mfma_supported(d) &&
        d.T * d.D * 2 < ((int64_t)1 << 31) && 6 * d.Hd * d.D * 2 < ((int64_t)1 << 31))  // 32-bit copy offsets
        return 1;
    if (generic_supported(d) && generic_bwd_token_block(d) > 0) return 0;
    return -1;
}

struct BwdWorkspace {
    size_t cM, cW, scal, snapW, snapM, lamW, lamM, lam, inter, dcM, dcW, dpart, part, split, total;
    size_t save, gacc;  // portable path: chunk-start states, forward G accumulators / dJ/dW
    int64_t ldc;
};

static BwdWorkspace bwd_workspace_layout(const e2ttt_desc& d) {
    BwdWorkspace w{};
    if (backward_path(d) == 0) {
        const size_t BH = (size_t)(d.B * d.H);
        const size_t nc = (size_t)((d.T + d.chunk - 1) / d.chunk);
        const size_t P = (size_t)e2ttt_param_count(&d);
        w.ldc = (d.T + 63) / 64 * 64;
        const size_t ldc = (size_t)w.ldc;
        size_t off = 0;
        auto take = [&](size_t bytes) {
            const size_t o = off;
            off += align_up(bytes);
            return o;
        };
        w.cM = take(BH * ldc * 4);
        w.cW = take(BH * ldc * 4);
        w.scal = take(BH * nc * 4 * 4);
        w.save = take(BH * nc * 2 * P * 4);
        w.gacc = take(BH * 2 * P * 4);
        w.dcM = take(BH * ldc * 4);
        w.dcW = take(BH * ldc * 4);
        w.dpart = take(BH * nc * 4 * 4);
        w.split = take(f32_split_bytes(d));  // the fp32 MFMA forward's partial sums (recompute / saved forward)
        w.total = (BH * (size_t)d.T == 0) ? 0 : off;
        return w;
    }
    const size_t BH = (size_t)(d.B * d.H);
    const size_t nc = (size_t)((d.T + d.chunk - 1) / d.chunk);
    const size_t P = (size_t)e2ttt_param_count(&d);
    const bool mom = !(d.flags & E2TTT_FLAG_NO_MOMENTUM);
    w.ldc = (d.T + 63) / 64 * 64;
    const size_t ldc = (size_t)w.ldc;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return o;
    };
    w.cM = take(BH * ldc * 4);
    w.cW = take(BH * ldc * 4);
    w.scal = take(BH * nc * 4 * 4);
    w.snapW = take(BH * nc * P * 2);
    w.snapM = mom ? take(BH * nc * P * 2) : 0;
    w.lamW = take(BH * P * 4);
    w.lamM = mom ? take(BH * P * 4) : 0;
    w.lam = take(BH * 2 * P * 2);
    w.inter = take(BH * (size_t)swiglu_bwd_inter_elems(d) * 2);
    w.dcM = take(BH * ldc * 4);
    w.dcW = take(BH * ldc * 4);
    w.dpart = take(BH * nc * (size_t)(d.Hd / 64) * 4 * 4);
    w.part = take((size_t)swiglu_bwd_part_elems(d, w.ldc) * 4);
    w.total = (BH * (size_t)d.T == 0) ? 0 : off;
    return w;
}

// byte sizes of the backward's 19 tensors: q, k, v, eta, alpha, beta, W0, M0,
// dout, dW_end, dM_end (inputs), dq, dk, dv, deta, dalpha, dbeta, dW0, dM0
static void bwd_sizes(const e2ttt_desc& d, size_t bytes[19]) {
    const size_t BH = (size_t)(d.B * d.H);
    const size_t es = d.io_dtype == E2TTT_BF16 ? 2 : 4;
    const size_t P = (size_t)e2ttt_param_count(&d);
    const bool mom = !(d.flags & E2TTT_FLAG_NO_MOMENTUM);
    const size_t x = BH * d.T * d.D * es, g = BH * d.T * 4, st = BH * P * 4;
    const size_t tmp[19] = {x, x, x, g, g, mom ? g : 0, st, mom ? st : 0, x, st, mom ? st : 0,
                            x, x, x, g, g, mom ? g : 0, st, mom ? st : 0};
    for (int i = 0; i < 19; ++i) bytes[i] = tmp[i];
}


Workspace workspace_layout(const e2ttt_desc& d, int path) {
    Workspace w{};
    const size_t BH = (size_t)(d.B * d.H);
    const size_t T = (size_t)d.T;
    const size_t nc = (size_t)((d.T + d.chunk - 1) / d.chunk);  // the last chunk may be shorter
    const size_t P = (size_t)e2ttt_param_count(&d);
    w.ldc = (d.T + 63) / 64 * 64;
    const size_t ldc = (size_t)w.ldc;
    (void)T;
    size_t off = 0;
    w.cM = off;
    off += align_up(BH * ldc * sizeof(float));
    w.cW = off;
    off += align_up(BH * ldc * sizeof(float));
    w.scal = off;
    off += align_up(BH * nc * 4 * sizeof(float));
    w.gacc = w.snap = off;
    if (path == 0)
        off += align_up(BH * 2 * P * sizeof(float));  // portable path: G accumulators
    else if (path == 1 || path == 2)
        off += align_up(BH * nc * P * 2);  // bf16 chunk-start snapshots
    // path 3 (fp32 MFMA) keeps its state and aggregations on chip, except
    // for the hidden-slice split, whose partial sums pass through here
    w.split = off;
    if (path == 4) off += align_up(f32_split_bytes(d));
    w.total = (BH * T == 0) ? 0 : off;
    return w;
}

struct Range {
    uintptr_t lo, hi;
};

static bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

}  // namespace e2ttt

using namespace e2ttt;

extern "C" {

int64_t e2ttt_param_count(const e2ttt_desc* d) {
    if (!d) return -1;
    switch (d->kind) {
        case E2TTT_LINEAR: return d->D * d->D;
        case E2TTT_MLP: return 2 * d->D * d->Hd;
        case E2TTT_SWIGLU: return 3 * d->D * d->Hd;
        default: return -1;
    }
}

size_t e2ttt_workspace_size(const e2ttt_desc* d) {
    if (!desc_ok(d)) return (size_t)-1;
    if (d->flags & E2TTT_FLAG_SAVE_STATES) return bwd_workspace_layout(*d).total;  // shared with the backward
    return workspace_layout(*d, path_of(*d)).total;
}

int e2ttt_path(const e2ttt_desc* d) {
    if (!desc_ok(d)) return -E2TTT_ERR_INVALID_ARG;
    return path_of(*d);
}

int e2ttt_validate(const e2ttt_desc* d, const void* const ptrs[11]) {
    if (!desc_ok(d) || !ptrs) return E2TTT_ERR_INVALID_ARG;
    if (path_of(*d) == 0 && !generic_supported(*d)) return E2TTT_ERR_UNSUPPORTED;
    if ((d->flags & E2TTT_FLAG_SAVE_STATES) && !save_compatible(path_of(*d), backward_path(*d)))
        return E2TTT_ERR_UNSUPPORTED;
    const size_t BH = (size_t)(d->B * d->H);
    const size_t es = d->io_dtype == E2TTT_BF16 ? 2 : 4;
    const size_t P = (size_t)e2ttt_param_count(d);
    const bool mom = !(d->flags & E2TTT_FLAG_NO_MOMENTUM);  // beta, M0, M_end unused without momentum
    const size_t bytes[11] = {BH * d->T * d->D * es, BH * d->T * d->D * es, BH * d->T * d->D * es,
                              BH * d->T * 4,         BH * d->T * 4,         mom ? BH * d->T * 4 : 0,
                              BH * P * 4,            mom ? BH * P * 4 : 0,  BH * d->T * d->D * es,
                              BH * P * 4,            mom ? BH * P * 4 : 0};
    const size_t align[11] = {16, 16, 16, 4, 4, 4, 16, 16, 16, 16, 16};
    for (int i = 0; i < 11; ++i) {
        if (bytes[i] == 0) continue;
        if (!ptrs[i]) return E2TTT_ERR_INVALID_ARG;
        if ((uintptr_t)ptrs[i] % align[i]) return E2TTT_ERR_INVALID_ARG;
    }
    Range r[11];
    for (int i = 0; i < 11; ++i) r[i] = {(uintptr_t)ptrs[i], (uintptr_t)ptrs[i] + bytes[i]};
    // outputs: 8 = out, 9 = W_end, 10 = M_end
    for (int o = 8; o < 11; ++o) {
        if (bytes[o] == 0) continue;
        for (int i = 0; i < 11; ++i) {
            if (i == o || bytes[i] == 0) continue;
            if (o == 9 && i == 6 && ptrs[9] == ptrs[6]) continue;   // W_end == W0: in place
            if (o == 10 && i == 7 && ptrs[10] == ptrs[7]) continue;  // M_end == M0: in place
            if (overlap(r[o], r[i])) return E2TTT_ERR_ALIAS;
        }
    }
    return E2TTT_OK;
}

int e2ttt_chunk_forward(const e2ttt_desc* d, const void* q, const void* k, const void* v, const float* eta,
                        const float* alpha, const float* beta, const float* W0, const float* M0, void* out,
                        float* W_end, float* M_end, void* workspace, size_t workspace_bytes, void* stream) {
    return e2ttt_chunk_forward_events(d, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, workspace,
                                      workspace_bytes, stream, nullptr);
}

int e2ttt_chunk_forward_events(const e2ttt_desc* d, const void* q, const void* k, const void* v, const float* eta,
                               const float* alpha, const float* beta, const float* W0, const float* M0, void* out,
                               float* W_end, float* M_end, void* workspace, size_t workspace_bytes, void* stream,
                               void* const events[4]) {
    const void* ptrs[11] = {q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end};
    const int st = e2ttt_validate(d, ptrs);
    if (st != E2TTT_OK) return st;
    const int path = path_of(*d);
    const bool save = (d->flags & E2TTT_FLAG_SAVE_STATES) != 0;
    Workspace ws = workspace_layout(*d, path);
    const BwdWorkspace bws = bwd_workspace_layout(*d);
    if (save) {  // the backward's layout: its leading sections are the forward's
        ws.cM = bws.cM;
        ws.cW = bws.cW;
        ws.scal = bws.scal;
        ws.snap = bws.snapW;
        ws.gacc = bws.gacc;
        ws.split = bws.split;
        ws.total = bws.total;
    }
    if (ws.total > 0) {
        if (!workspace || workspace_bytes < ws.total || (uintptr_t)workspace % kAlign) return E2TTT_ERR_WORKSPACE;
        const Range wr{(uintptr_t)workspace, (uintptr_t)workspace + ws.total};
        const size_t BH = (size_t)(d->B * d->H);
        const size_t es = d->io_dtype == E2TTT_BF16 ? 2 : 4;
        const size_t P = (size_t)e2ttt_param_count(d);
        const bool mom = !(d->flags & E2TTT_FLAG_NO_MOMENTUM);
        const size_t bytes[11] = {BH * d->T * d->D * es, BH * d->T * d->D * es, BH * d->T * d->D * es,
                                  BH * d->T * 4, BH * d->T * 4, mom ? BH * d->T * 4 : 0, BH * P * 4,
                                  mom ? BH * P * 4 : 0, BH * d->T * d->D * es, BH * P * 4,
                                  mom ? BH * P * 4 : 0};
        for (int i = 0; i < 11; ++i)
            if (bytes[i] && overlap(wr, Range{(uintptr_t)ptrs[i], (uintptr_t)ptrs[i] + bytes[i]}))
                return E2TTT_ERR_ALIAS;
    }
    hipStream_t s = (hipStream_t)stream;
    const int64_t BH = d->B * d->H;
    if (BH == 0) return E2TTT_OK;
    const size_t P = (size_t)e2ttt_param_count(d);
    if (d->T == 0) {
        if (W_end != W0 && hipMemcpyAsync(W_end, W0, BH * P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return E2TTT_ERR_HIP;
        if (!(d->flags & E2TTT_FLAG_NO_MOMENTUM) && M_end != M0 &&
            hipMemcpyAsync(M_end, M0, BH * P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return E2TTT_ERR_HIP;
        return E2TTT_OK;
    }
    char* wsb = (char*)workspace;
    float* cM = (float*)(wsb + ws.cM);
    float* cW = (float*)(wsb + ws.cW);
    float* scal = (float*)(wsb + ws.scal);
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (events)
        for (int i = 0; i < 4; ++i) ev[i] = (hipEvent_t)events[i];
    if (ev[0] && hipEventRecord(ev[0], s) != hipSuccess) return E2TTT_ERR_HIP;
    // the SwiGLU chunk loop computes the scalar kernels itself where it can
    const bool fold = (path == 1 || path == 2) && swiglu_loop_scans(*d);
    if (!fold &&
        launch_logscan(BH, d->T, d->chunk, d->flags, eta, alpha, beta, cM, cW, ws.ldc, scal, s) != hipSuccess)
        return E2TTT_ERR_HIP;
    if (ev[1] && hipEventRecord(ev[1], s) != hipSuccess) return E2TTT_ERR_HIP;
    hipError_t e;
    const bool mom = !(d->flags & E2TTT_FLAG_NO_MOMENTUM);
    if (path == 1 || path == 2) {
        e = launch_swiglu_mfma(*d, q, k, v, cM, cW, ws.ldc, scal, W0, M0, out, W_end, M_end, wsb + ws.snap,
                               save && mom ? wsb + bws.snapM : nullptr, s, ev[2], eta, alpha, beta, fold);
    } else if (path == 3 || path == 4) {
        e = launch_f32_mfma(*d, q, k, v, cM, cW, ws.ldc, scal, W0, M0, out, W_end, M_end, s,
                            save ? (float*)(wsb + bws.save) : nullptr, wsb + ws.split);
        if (e == hipSuccess && ev[2]) e = hipEventRecord(ev[2], s);
    } else {
        e = launch_generic(*d, q, k, v, cM, cW, ws.ldc, scal, W0, M0, out, W_end, M_end, (float*)(wsb + ws.gacc),
                           s, save ? (float*)(wsb + bws.save) : nullptr);
        if (e == hipSuccess && ev[2]) e = hipEventRecord(ev[2], s);
    }
    if (e == hipSuccess && ev[3]) e = hipEventRecord(ev[3], s);
    return e == hipSuccess ? E2TTT_OK : E2TTT_ERR_HIP;
}

int e2ttt_chunk_forward_noalloc(const e2ttt_desc* d, const void* q, const void* k, const void* v, const float* eta,
                                const float* alpha, const float* beta, const float* W0, const float* M0, void* out,
                                float* W_end, float* M_end, void* stream) {
    const void* ptrs[11] = {q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end};
    const int st = e2ttt_validate(d, ptrs);
    if (st != E2TTT_OK) return st;
    // saved states would not survive the next call on this GPU
    if (d->flags & E2TTT_FLAG_SAVE_STATES) return E2TTT_ERR_INVALID_ARG;
    const size_t need = e2ttt_workspace_size(d);
    if (need > (size_t)E2TTT_NOALLOC_SCRATCH_BYTES) return E2TTT_ERR_SCRATCH_LIMIT;  // before any device call
    void* ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess) return E2TTT_ERR_HIP;
    return e2ttt_chunk_forward_events(d, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws,
                                      need > 0 ? (size_t)E2TTT_NOALLOC_SCRATCH_BYTES : 0, stream, nullptr);
}

size_t e2ttt_backward_workspace_size(const e2ttt_desc* d) {
    if (!desc_ok(d)) return (size_t)-1;
    return bwd_workspace_layout(*d).total;
}

int e2ttt_validate_backward(const e2ttt_desc* d, const void* const ptrs[19]) {
    if (!desc_ok(d) || !ptrs) return E2TTT_ERR_INVALID_ARG;
    if (backward_path(*d) < 0) return E2TTT_ERR_UNSUPPORTED;
    size_t bytes[19];
    bwd_sizes(*d, bytes);
    for (int i = 0; i < 19; ++i) {
        if (bytes[i] == 0) continue;
        if (!ptrs[i]) return E2TTT_ERR_INVALID_ARG;
        const bool scalar = (i >= 3 && i <= 5) || (i >= 14 && i <= 16);  // [B][H][T] fp32
        if ((uintptr_t)ptrs[i] % (scalar ? 4 : 16)) return E2TTT_ERR_INVALID_ARG;
    }
    for (int o = 11; o < 19; ++o) {
        if (bytes[o] == 0) continue;
        const Range ro{(uintptr_t)ptrs[o], (uintptr_t)ptrs[o] + bytes[o]};
        for (int i = 0; i < 19; ++i) {
            if (i == o || bytes[i] == 0) continue;
            if (overlap(ro, Range{(uintptr_t)ptrs[i], (uintptr_t)ptrs[i] + bytes[i]})) return E2TTT_ERR_ALIAS;
        }
    }
    return E2TTT_OK;
}

int e2ttt_chunk_backward(const e2ttt_desc* d, const void* q, const void* k, const void* v, const float* eta,
                         const float* alpha, const float* beta, const float* W0, const float* M0, const void* dout,
                         const float* dW_end, const float* dM_end, void* dq, void* dk, void* dv, float* deta,
                         float* dalpha, float* dbeta, float* dW0, float* dM0, void* workspace,
                         size_t workspace_bytes, void* stream) {
    return e2ttt_chunk_backward_events(d, q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end, dq, dk, dv, deta,
                                       dalpha, dbeta, dW0, dM0, workspace, workspace_bytes, stream, nullptr);
}

int e2ttt_chunk_backward_events(const e2ttt_desc* d, const void* q, const void* k, const void* v, const float* eta,
                                const float* alpha, const float* beta, const float* W0, const float* M0,
                                const void* dout, const float* dW_end, const float* dM_end, void* dq, void* dk,
                                void* dv, float* deta, float* dalpha, float* dbeta, float* dW0, float* dM0,
                                void* workspace, size_t workspace_bytes, void* stream, void* const events[4]) {
    const void* ptrs[19] = {q,  k,  v,  eta,  alpha,  beta,  W0,  M0,  dout, dW_end,
                            dM_end, dq, dk, dv, deta, dalpha, dbeta, dW0, dM0};
    const int st = e2ttt_validate_backward(d, ptrs);
    if (st != E2TTT_OK) return st;
    const BwdWorkspace ws = bwd_workspace_layout(*d);
    if (ws.total > 0) {
        if (!workspace || workspace_bytes < ws.total || (uintptr_t)workspace % kAlign) return E2TTT_ERR_WORKSPACE;
        const Range wr{(uintptr_t)workspace, (uintptr_t)workspace + ws.total};
        size_t bytes[19];
        bwd_sizes(*d, bytes);
        for (int i = 0; i < 19; ++i)
            if (bytes[i] && overlap(wr, Range{(uintptr_t)ptrs[i], (uintptr_t)ptrs[i] + bytes[i]}))
                return E2TTT_ERR_ALIAS;
    }
    hipStream_t s = (hipStream_t)stream;
    const int64_t BH = d->B * d->H;
    if (BH == 0) return E2TTT_OK;
    const bool mom = !(d->flags & E2TTT_FLAG_NO_MOMENTUM);
    const size_t P = (size_t)e2ttt_param_count(d);
    if (d->T == 0) {  // the state passes through unchanged
        if (hipMemcpyAsync(dW0, dW_end, BH * P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess) return E2TTT_ERR_HIP;
        if (mom && hipMemcpyAsync(dM0, dM_end, BH * P * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
            return E2TTT_ERR_HIP;
        return E2TTT_OK;
    }
    char* wsb = (char*)workspace;
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (events)
        for (int i = 0; i < 4; ++i) ev[i] = (hipEvent_t)events[i];
    if (ev[0] && hipEventRecord(ev[0], s) != hipSuccess) return E2TTT_ERR_HIP;
    if (backward_path(*d) == 0) {
        // portable path: recompute saving every chunk's start state (outputs
        // into dq, end state into dW0 / dM0, both overwritten below)
        float* cM = (float*)(wsb + ws.cM);
        float* cW = (float*)(wsb + ws.cW);
        float* scal = (float*)(wsb + ws.scal);
        float* save = (float*)(wsb + ws.save);
        if (!(d->flags & E2TTT_FLAG_SAVE_STATES)) {  // else a forward call left them in the workspace
            if (launch_logscan(BH, d->T, d->chunk, d->flags, eta, alpha, beta, cM, cW, ws.ldc, scal, s) != hipSuccess)
                return E2TTT_ERR_HIP;
            // the forward path e2ttt_chunk_forward takes, so that a saved forward
            // and this recompute leave the same states
            const hipError_t fe =
                path_of(*d) >= 3
                    ? launch_f32_mfma(*d, q, k, v, cM, cW, ws.ldc, scal, W0, M0, dq, dW0, dM0, s, save,
                                      wsb + ws.split)
                    : launch_generic(*d, q, k, v, cM, cW, ws.ldc, scal, W0, M0, dq, dW0, dM0,
                                     (float*)(wsb + ws.gacc), s, save);
            if (fe != hipSuccess) return E2TTT_ERR_HIP;
        }
        if (ev[1] && hipEventRecord(ev[1], s) != hipSuccess) return E2TTT_ERR_HIP;
        GenericBwdBuffers g;
        g.q = q;
        g.k = k;
        g.v = v;
        g.dout = dout;
        g.eta = eta;
        g.alpha = alpha;
        g.beta = beta;
        g.cM = cM;
        g.cW = cW;
        g.scal = scal;
        g.save = save;
        g.dW_end = dW_end;
        g.dM_end = dM_end;
        g.dacc = (float*)(wsb + ws.gacc);
        g.dcM = (float*)(wsb + ws.dcM);
        g.dcW = (float*)(wsb + ws.dcW);
        g.dpart = (float*)(wsb + ws.dpart);
        g.dq = dq;
        g.dk = dk;
        g.dv = dv;
        g.deta = deta;
        g.dalpha = dalpha;
        g.dbeta = dbeta;
        g.dW0 = dW0;
        g.dM0 = dM0;
        g.ldc = ws.ldc;
        hipError_t e = launch_generic_backward(*d, g, s);
        if (e == hipSuccess && ev[2]) e = hipEventRecord(ev[2], s);
        if (e == hipSuccess && ev[3]) e = hipEventRecord(ev[3], s);
        return e == hipSuccess ? E2TTT_OK : E2TTT_ERR_HIP;
    }
    // forward recompute: scalar kernels and the chunk loop (chunk-start
    // snapshots of W and M); its end state goes to dW0 / dM0, which the
    // backward overwrites
    float* cM = (float*)(wsb + ws.cM);
    float* cW = (float*)(wsb + ws.cW);
    float* scal = (float*)(wsb + ws.scal);
    if (!(d->flags & E2TTT_FLAG_SAVE_STATES)) {  // else a forward call left them in the workspace
        if (launch_logscan(BH, d->T, d->chunk, d->flags, eta, alpha, beta, cM, cW, ws.ldc, scal, s) != hipSuccess)
            return E2TTT_ERR_HIP;
        if (launch_swiglu_loop(*d, k, v, cM, cW, ws.ldc, scal, W0, M0, dW0, dM0, wsb + ws.snapW,
                               mom ? wsb + ws.snapM : nullptr, s) != hipSuccess)
            return E2TTT_ERR_HIP;
    }
    if (ev[1] && hipEventRecord(ev[1], s) != hipSuccess) return E2TTT_ERR_HIP;
    BwdBuffers b;
    b.q = q;
    b.k = k;
    b.v = v;
    b.dout = dout;
    b.eta = eta;
    b.alpha = alpha;
    b.beta = beta;
    b.cM = cM;
    b.cW = cW;
    b.scal = scal;
    b.snapW = wsb + ws.snapW;
    b.snapM = mom ? wsb + ws.snapM : nullptr;
    b.dW_end = dW_end;
    b.dM_end = dM_end;
    b.lamW = (float*)(wsb + ws.lamW);
    b.lamM = mom ? (float*)(wsb + ws.lamM) : nullptr;
    b.lam = wsb + ws.lam;
    b.inter = wsb + ws.inter;
    b.dcM = (float*)(wsb + ws.dcM);
    b.dcW = (float*)(wsb + ws.dcW);
    b.dpart = (float*)(wsb + ws.dpart);
    b.part = swiglu_bwd_part_elems(*d, ws.ldc) > 0 ? (float*)(wsb + ws.part) : nullptr;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.deta = deta;
    b.dalpha = dalpha;
    b.dbeta = dbeta;
    b.dW0 = dW0;
    b.dM0 = dM0;
    b.ldc = ws.ldc;
    hipError_t e = launch_swiglu_backward(*d, b, s, ev[2]);
    if (e == hipSuccess && ev[3]) e = hipEventRecord(ev[3], s);
    return e == hipSuccess ? E2TTT_OK : E2TTT_ERR_HIP;
}

int e2ttt_logscan(const e2ttt_desc* d, const float* eta, const float* alpha, const float* beta, float* cM,
                  float* cW, float* scal, void* stream) {
    if (!logscan_desc_ok(d)) return E2TTT_ERR_INVALID_ARG;
    const int64_t BH = d->B * d->H;
    if (BH * d->T == 0) return E2TTT_OK;
    if (!eta || !alpha || !cM || !cW || !scal) return E2TTT_ERR_INVALID_ARG;
    if (!beta && !(d->flags & E2TTT_FLAG_NO_MOMENTUM)) return E2TTT_ERR_INVALID_ARG;
    const float* const ptrs[6] = {eta, alpha, beta, cM, cW, scal};
    for (const float* p : ptrs)
        if ((uintptr_t)p % alignof(float)) return E2TTT_ERR_INVALID_ARG;
    return launch_logscan(BH, d->T, d->chunk, d->flags, eta, alpha, beta, cM, cW, d->T, scal, (hipStream_t)stream) ==
                   hipSuccess
               ? E2TTT_OK
               : E2TTT_ERR_HIP;
}

const char* e2ttt_status_string(int s) {
    switch (s) {
        case E2TTT_OK: return "ok";
        case E2TTT_ERR_INVALID_ARG: return "invalid argument";
        case E2TTT_ERR_UNSUPPORTED: return "unsupported shape";
        case E2TTT_ERR_ALIAS: return "output aliases another buffer";
        case E2TTT_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case E2TTT_ERR_HIP: return "HIP launch failed";
        case E2TTT_ERR_SCRATCH_LIMIT: return "call needs more scratch than the no-allocation entry point holds";
        default: return "unknown status";
    }
}

}  // extern "C"

// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/e2ttt.h"

namespace e2ttt {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of the workspace sections for one call.
struct Workspace {
    size_t cM, cW, scal;  // logscan outputs (fp32; cM / cW rows of ldc tokens)
    int64_t ldc;          // T rounded up to a whole 64-token block
    size_t gacc;          // portable path: per-head gradient accumulators (fp32, 2*P)
    size_t snap;          // MFMA path: bf16 chunk-start weight snapshots (B*H*nc*P)
    size_t split;         // fp32 MFMA path, MLP split over hidden slices: partial sums
    size_t total;
};

Workspace workspace_layout(const e2ttt_desc& d, int path);

// Compute units of the current device, queried once per device and cached
// (launch sizing reads it on every call).
hipError_t device_cu_count(int* ncu);

// Launchers (return hipError_t of the launch).
// cM / cW rows have stride ldc >= T; entries T .. ldc-1 are written as zeros.
hipError_t launch_logscan(int64_t BH, int64_t T, int64_t chunk, int flags, const float* eta, const float* alpha,
                          const float* beta, float* cM, float* cW, int64_t ldc, float* scal, hipStream_t s);

// save (may be null): [BH][nc][2][P] fp32, every chunk's start W and M.
hipError_t launch_generic(const e2ttt_desc& d, const void* q, const void* k, const void* v,
                          const float* cM, const float* cW, int64_t ldc, const float* scal, const float* W0,
                          const float* M0, void* out, float* W_end, float* M_end, float* gacc,
                          hipStream_t s, float* save = nullptr);

// fp32-MFMA chunk loop for the linear and MLP fast weights with fp32 I/O
// (D and Hd multiples of 16, a head's state within 32 16x16 tiles per
// matrix); save as launch_generic's.
bool f32_mfma_supported(const e2ttt_desc& d);
// Whether the MLP is split over hidden slices (one workgroup per slice for
// the whole sequence, the slices of a head meeting once per chunk), and the
// workspace bytes the split needs (0 otherwise).
bool f32_split(const e2ttt_desc& d);
size_t f32_split_bytes(const e2ttt_desc& d);
hipError_t launch_f32_mfma(const e2ttt_desc& d, const void* q, const void* k, const void* v, const float* cM,
                           const float* cW, int64_t ldc, const float* scal, const float* W0, const float* M0, void* out,
                           float* W_end, float* M_end, hipStream_t s, float* save, void* split_ws);

// SwiGLU / negative-dot / bf16 / D == 128 / Hd % 64 == 0 / chunk % 64 == 0.
bool swiglu_mfma_supported(const e2ttt_desc& d);
// Chunk loop of the SwiGLU path: final state and the bf16 chunk-start weight
// snapshots [BH][nc][W1^T | W3^T | W2] (each [Hd][D]); with snapM non-null
// (momentum only) also the chunk-start momentum snapshots in the same layout.
// With fold the loop writes cM, cW and scal itself from eta, alpha, beta
// (no separate launch_logscan before it); only where swiglu_loop_scans(d).
bool swiglu_loop_scans(const e2ttt_desc& d);
hipError_t launch_swiglu_loop(const e2ttt_desc& d, const void* k, const void* v, const float* cM, const float* cW,
                              int64_t ldc, const float* scal, const float* W0, const float* M0, float* W_end, float* M_end,
                              void* snap, void* snapM, hipStream_t s, const float* eta = nullptr,
                              const float* alpha = nullptr, const float* beta = nullptr, bool fold = false);
// ev_mid (may be null) is recorded between the chunk-loop and output launches;
// snapM (may be null) receives the momentum snapshots; fold as for
// launch_swiglu_loop.
hipError_t launch_swiglu_mfma(const e2ttt_desc& d, const void* q, const void* k, const void* v,
                              const float* cM, const float* cW, int64_t ldc, const float* scal, const float* W0,
                              const float* M0, void* out, float* W_end, float* M_end, void* snap, void* snapM,
                              hipStream_t s, hipEvent_t ev_mid, const float* eta = nullptr,
                              const float* alpha = nullptr, const float* beta = nullptr, bool fold = false);

// Backward pass of the SwiGLU path (same shape support, chunk <= 2048).
struct BwdBuffers {
    const void *q, *k, *v, *dout;      // [BH][T][D] bf16
    const float *eta, *alpha, *beta;   // [BH][T]
    const float *cM, *cW, *scal;       // scalar-kernel outputs of the recompute
    const void *snapW, *snapM;         // bf16 chunk-start snapshots of the recompute
    const float *dW_end, *dM_end;      // [BH][P] state cotangents
    float *lamW, *lamM;                // [BH][P] fp32 working state cotangents (hidden-major)
    void* lam;                         // [BH][2P] bf16 copies
    void* inter;                       // [BH][6][Hd][chunk] bf16 per-chunk terms
    float *dcM, *dcW;                  // [BH][ldc]
    float* dpart;                      // [BH][nc][Hd/64][4]
    float* part;                       // swiglu_bwd_part_elems floats (null when that is 0)
    void *dq, *dk, *dv;                // [BH][T][D] bf16
    float *deta, *dalpha, *dbeta;      // [BH][T]
    float *dW0, *dM0;                  // [BH][P]
    int64_t ldc;
};
// ev_loop (may be null) is recorded after the reverse chunk loop, before the
// scalar kernels' backward.
hipError_t launch_swiglu_backward(const e2ttt_desc& d, const BwdBuffers& b, hipStream_t s, hipEvent_t ev_loop);
int64_t swiglu_bwd_inter_elems(const e2ttt_desc& d);  // per (b, h)
// token-kernel hidden-unit parts (1, 2 or 4) and the fp32 partial sums they need
int swiglu_bwd_unit_parts(const e2ttt_desc& d);
int64_t swiglu_bwd_part_elems(const e2ttt_desc& d, int64_t ldc);

// Scalar kernels' backward: d eta, d alpha, d beta from dcM, dcW (per token)
// and the partial dA, dBb, dgamma in dpart [BH][nc][nsl][4].
hipError_t launch_bwd_scalar(const e2ttt_desc& d, const float* eta, const float* alpha, const float* beta,
                             const float* dcM, const float* dcW, int64_t ldc, const float* dpart, int nsl,
                             float* deta, float* dalpha, float* dbeta, hipStream_t s);

// Backward of the portable path (every kind and loss).
struct GenericBwdBuffers {
    const void *q, *k, *v, *dout;
    const float *eta, *alpha, *beta;
    const float *cM, *cW, *scal;
    const float* save;                // [BH][nc][2][P] chunk-start W, M
    const float *dW_end, *dM_end;
    float* dacc;                      // [BH][P]
    float *dcM, *dcW;                 // [BH][ldc]
    float* dpart;                     // [BH][nc][4]
    void *dq, *dk, *dv;
    float *deta, *dalpha, *dbeta, *dW0, *dM0;
    int64_t ldc;
};
int generic_bwd_token_block(const e2ttt_desc& d);  // 0: the shape does not fit
hipError_t launch_generic_backward(const e2ttt_desc& d, const GenericBwdBuffers& b, hipStream_t s);

}  // namespace e2ttt

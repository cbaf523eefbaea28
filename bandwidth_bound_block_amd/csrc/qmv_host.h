// Host-side helpers shared by the entry points of libqmv.so: the thread-local
// error message, argument checks and per-device launch facts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "qmv.h"

namespace qmv {

// Records the message for qmv_last_error() and returns code.
int32_t fail(int32_t code, const char* fmt, ...);
// Clears the message (called on every successful return).
int32_t ok();

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Workgroups of `kernel` (block threads, dynamic LDS bytes) that fit on one
// compute unit at once (cached per kernel and LDS size; at least 1).
int resident_wgs(const void* kernel, int threads, size_t lds);

// Raises the dynamic LDS limit of `kernel` to what a workgroup of lds_total
// bytes leaves beside the kernel's static LDS, once per kernel and device
// (thread-safe).  Returns QMV_OK with that limit in *dyn_max, else QMV_EHIP
// with the message set (prefixed by `what`).
int32_t lds_limit(const void* kernel, size_t lds_total, const char* what, size_t* dyn_max);

// Maps the status of the launch just issued to a return code.
int32_t check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Up to kMaxSegs matrices with the same number of columns that read one
// activation vector, run as one batch-1 matvec over their concatenated
// rows (each matrix's blocks and outputs stay in its own buffers).
constexpr int kMaxSegs = 4;
struct RowSegs {
    const uint8_t* W[kMaxSegs];
    float* y[kMaxSegs];
    int64_t end[kMaxSegs];   // cumulative row counts: rows of matrix i are [end[i-1], end[i])
    int32_t n;
};

// Runs segs with the contiguous-chunk batch-1 kernel of format fmt when it
// applies (whole 64-block steps, W and x 16-byte aligned): returns true and
// the launch status in *rc, else false and launches nothing.  Without
// force, only where that kernel measured faster than per-block loads.
bool group_matvec_contig(qmv_fmt fmt, const RowSegs& segs, int nb, const float* x, hipStream_t st, bool force,
                         int32_t* rc);

// The entry points of one block format (its kernels are compiled in a
// translation unit of their own).  x_type: QMV_X_F32 / QMV_X_F16 /
// QMV_X_BF16; path: QMV_PATH_*; swiglu: the MoE gate||up variant.
struct FormatOps {
    int32_t (*matvec)(const char* name, const void* W, int64_t N, int64_t K, const void* x, int32_t x_type,
                      int64_t ldx, int32_t batch, float* y, int64_t ldy, void* stream, int32_t path);
    int32_t (*dequant)(const void* W, int64_t N, int64_t K, float* out, void* stream);
    int32_t (*moe)(const char* name, bool swiglu, const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K,
                   const int32_t* ids, int32_t batch, int32_t top_k, const void* x, int32_t x_type, int64_t xs_tok,
                   int64_t xs_slot, float* y, void* stream);
    int32_t (*moe_combine)(const void* Wx, int64_t estride, int32_t E, int64_t N, int64_t K, const int32_t* ids,
                           const float* wts, int32_t batch, int32_t top_k, const float* x, int64_t xs_tok,
                           int64_t xs_slot, float* out, void* stream);
    bool (*group_contig)(const RowSegs& segs, int nb, const float* x, hipStream_t st, bool force, int32_t* rc);
    // qmv_chain for formats without the persistent chain kernels (nullptr
    // for the others): stage groups and stages as separate launches
    int32_t (*chain)(const char* name, const qmv_chain_stage* stages, int32_t n_stages, void* stream);
};
const FormatOps& ops_q8_0();
const FormatOps& ops_q4_0();
const FormatOps& ops_q4_1();
const FormatOps& ops_q4_k();   // qmv_q4k.hip
const FormatOps& ops_q6_k();   // qmv_q6k.hip
// The table of fmt, or nullptr for an unknown format.
const FormatOps* format_ops(qmv_fmt fmt);

// The batch-1 chain of qmv_chain as one weight stream across dependency
// levels (qmv_decode.hip).  Applies when every stage has n_cols a multiple
// of 2048 and 16-byte aligned W and x, and the staged x, partial sums and
// load ring fit the LDS: then returns true and the launch status in *rc;
// else false and launches nothing.  ws: the 40 KB workspace (flag words
// 9216.. and the error word 2).
bool decode_chain(qmv_fmt fmt, const qmv_chain_stage* stages, int32_t n_stages, unsigned* ws, hipStream_t st,
                  int32_t* rc);

// Batch 2..8 on the matrix cores (bf16 MFMA with the activations split into
// two bf16 pieces).  Applies when n_cols is a multiple of 256, W is 16-byte
// aligned, x is aligned to 4 elements and ldx is a multiple of 4: then returns true and the
// launch status in *rc; else false and launches nothing.  variant: 0 for
// the default workgroup shape, else (waves << 8) | waves-per-tile (tuning).
// x_type: QMV_X_F32 / QMV_X_F16 / QMV_X_BF16 (x holds that element type).
bool batch_matvec_mma(qmv_fmt fmt, const uint8_t* W, int64_t N, int nb, const void* x, int32_t x_type, int64_t ldx,
                      int B, float* y, int64_t ldy, hipStream_t st, int variant, int32_t* rc);
// Whether QMV_PATH_AUTO takes the matrix-core kernel for this shape.
bool use_mfma(qmv_fmt fmt, int64_t N, int nb, int B);

}  // namespace qmv

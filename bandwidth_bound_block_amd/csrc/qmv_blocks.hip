// C entry points of the block-format (Q8_0 / Q4_0 / Q4_1 / Q4_K / Q6_K)
// matvec, MoE and dequant paths: argument routing to the format's FormatOps
// table (the kernels themselves are in qmv_blocks_impl.h, compiled once per
// 32-weight format, qmv_q4k.hip and qmv_q6k.hip).
#include "qmv_host.h"

namespace qmv {

const FormatOps* format_ops(qmv_fmt fmt) {
    switch (fmt) {
    case QMV_Q8_0: return &ops_q8_0();
    case QMV_Q4_0: return &ops_q4_0();
    case QMV_Q4_1: return &ops_q4_1();
    case QMV_Q4_K: return &ops_q4_k();
    case QMV_Q6_K: return &ops_q6_k();
    default: return nullptr;
    }
}

bool group_matvec_contig(qmv_fmt fmt, const RowSegs& segs, int nb, const float* x, hipStream_t st, bool force,
                         int32_t* rc) {
    const FormatOps* ops = format_ops(fmt);
    return ops && ops->group_contig(segs, nb, x, st, force, rc);
}

}  // namespace qmv

extern "C" int32_t qmv_q8_0(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::ops_q8_0().matvec("qmv_q8_0", W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream,
                                  QMV_PATH_AUTO);
}
extern "C" int32_t qmv_q4_0(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::ops_q4_0().matvec("qmv_q4_0", W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream,
                                  QMV_PATH_AUTO);
}
extern "C" int32_t qmv_q4_1(const void* W, int64_t n_rows, int64_t n_cols, const float* x, int64_t ldx, int32_t batch,
                            float* y, int64_t ldy, void* stream) {
    return qmv::ops_q4_1().matvec("qmv_q4_1", W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream,
                                  QMV_PATH_AUTO);
}
extern "C" int32_t qmv_matvec_xt(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols, const void* x,
                                 int32_t x_type, int64_t ldx, int32_t batch, float* y, int64_t ldy, int32_t path,
                                 void* stream) {
    const char* name = "qmv_matvec_xt";
    if (path != QMV_PATH_AUTO && path != QMV_PATH_FMA && path != QMV_PATH_MFMA)
        return qmv::fail(QMV_EINVAL, "%s: unknown path %d", name, (int)path);
    const qmv::FormatOps* ops = qmv::format_ops(fmt);
    if (!ops) return qmv::fail(QMV_EUNSUPPORTED, "%s: unknown format %d", name, (int)fmt);
    return ops->matvec(name, W, n_rows, n_cols, x, x_type, ldx, batch, y, ldy, stream, path);
}
extern "C" int32_t qmv_matvec_path(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols, const float* x,
                                   int64_t ldx, int32_t batch, float* y, int64_t ldy, int32_t path, void* stream) {
    const char* name = "qmv_matvec_path";
    if (path != QMV_PATH_AUTO && path != QMV_PATH_FMA && path != QMV_PATH_MFMA)
        return qmv::fail(QMV_EINVAL, "%s: unknown path %d", name, (int)path);
    const qmv::FormatOps* ops = qmv::format_ops(fmt);
    if (!ops) return qmv::fail(QMV_EUNSUPPORTED, "%s: unknown format %d", name, (int)fmt);
    return ops->matvec(name, W, n_rows, n_cols, x, QMV_X_F32, ldx, batch, y, ldy, stream, path);
}
extern "C" int32_t qmv_dequant(qmv_fmt fmt, const void* W, int64_t n_rows, int64_t n_cols, float* out, void* stream) {
    const qmv::FormatOps* ops = qmv::format_ops(fmt);
    if (!ops) return qmv::fail(QMV_EUNSUPPORTED, "qmv_dequant: unknown format %d", (int)fmt);
    return ops->dequant(W, n_rows, n_cols, out, stream);
}

namespace qmv {
namespace {
int32_t moe_entry(const char* name, bool swiglu, qmv_fmt fmt, const void* W, int64_t estride, int32_t E, int64_t N,
                  int64_t K, const int32_t* ids, int32_t batch, int32_t top_k, const void* x, int32_t x_type,
                  int64_t xs_tok, int64_t xs_slot, float* y, void* stream) {
    const FormatOps* ops = format_ops(fmt);
    if (!ops) return fail(QMV_EUNSUPPORTED, "%s: unknown format %d", name, (int)fmt);
    return ops->moe(name, swiglu, W, estride, E, N, K, ids, batch, top_k, x, x_type, xs_tok, xs_slot, y, stream);
}
}  // namespace
}  // namespace qmv

extern "C" int32_t qmv_moe(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes, int32_t n_experts,
                           int64_t n_rows, int64_t n_cols, const int32_t* expert_ids, int32_t batch, int32_t top_k,
                           const float* x, int64_t x_stride_token, int64_t x_stride_slot, float* y, void* stream) {
    return qmv::moe_entry("qmv_moe", false, fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids,
                          batch, top_k, x, QMV_X_F32, x_stride_token, x_stride_slot, y, stream);
}

extern "C" int32_t qmv_moe_xt(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes, int32_t n_experts,
                              int64_t n_rows, int64_t n_cols, const int32_t* expert_ids, int32_t batch, int32_t top_k,
                              const void* x, int32_t x_type, int64_t x_stride_token, int64_t x_stride_slot, float* y,
                              void* stream) {
    return qmv::moe_entry("qmv_moe_xt", false, fmt, W_experts, expert_stride_bytes, n_experts, n_rows, n_cols,
                          expert_ids, batch, top_k, x, x_type, x_stride_token, x_stride_slot, y, stream);
}

extern "C" int32_t qmv_moe_swiglu(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes, int32_t n_experts,
                                  int64_t n_ff, int64_t n_cols, const int32_t* expert_ids, int32_t batch,
                                  int32_t top_k, const float* x, int64_t x_stride_token, int64_t x_stride_slot,
                                  float* h, void* stream) {
    return qmv::moe_entry("qmv_moe_swiglu", true, fmt, W_experts, expert_stride_bytes, n_experts, n_ff, n_cols,
                          expert_ids, batch, top_k, x, QMV_X_F32, x_stride_token, x_stride_slot, h, stream);
}

extern "C" int32_t qmv_moe_swiglu_xt(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes,
                                     int32_t n_experts, int64_t n_ff, int64_t n_cols, const int32_t* expert_ids,
                                     int32_t batch, int32_t top_k, const void* x, int32_t x_type,
                                     int64_t x_stride_token, int64_t x_stride_slot, float* h, void* stream) {
    return qmv::moe_entry("qmv_moe_swiglu_xt", true, fmt, W_experts, expert_stride_bytes, n_experts, n_ff, n_cols,
                          expert_ids, batch, top_k, x, x_type, x_stride_token, x_stride_slot, h, stream);
}

extern "C" int32_t qmv_moe_combine(qmv_fmt fmt, const void* W_experts, int64_t expert_stride_bytes, int32_t n_experts,
                                   int64_t n_rows, int64_t n_cols, const int32_t* expert_ids, const float* weights,
                                   int32_t batch, int32_t top_k, const float* x, int64_t x_stride_token,
                                   int64_t x_stride_slot, float* out, void* stream) {
    const qmv::FormatOps* ops = qmv::format_ops(fmt);
    if (!ops) return qmv::fail(QMV_EUNSUPPORTED, "qmv_moe_combine: unknown format %d", (int)fmt);
    return ops->moe_combine(W_experts, expert_stride_bytes, n_experts, n_rows, n_cols, expert_ids, weights, batch,
                            top_k, x, x_stride_token, x_stride_slot, out, stream);
}

// eqlinear_api.hip -- the C ABI of libeqlinear (declared in include/eqlinear.h):
// plan metadata, argument validation and kernel dispatch.  Validation runs
// before any HIP call so the error paths can be exercised without a GPU.
#include <new>

#include "../../include/eqlinear.h"
#include "eq_launch.h"

struct eqlinear_plan_s {
    int kind;
    int dtype;
    int N;
    int C_in, C_out;
};

namespace {


bool dtype_ok(int dt) { return dt == EQL_F32 || dt == EQL_BF16 || dt == EQL_F16; }

// The plan dtype is the launchers' element-type code (eql::kIo*).
static_assert(EQL_F32 == eql::kIoF32 && EQL_BF16 == eql::kIoBF16 && EQL_F16 == eql::kIoF16, "type codes");

size_t elem_size(const eqlinear_plan_s* p) { return p->dtype == EQL_F32 ? 4 : 2; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

eqlinear_status hip_status(hipError_t e) { return e == hipSuccess ? EQL_OK : EQL_ERR_HIP; }

int64_t in_width(const eqlinear_plan_s* p) {
    return p->kind == EQL_KIND_CN ? (int64_t)p->N * p->C_in : p->C_in;
}
int64_t out_width(const eqlinear_plan_s* p) {
    return p->kind == EQL_KIND_CN ? (int64_t)p->N * p->C_out : p->C_out;
}

// Widths are capped so every per-row offset fits an int in the kernels.
constexpr int64_t kMaxWidth = 1 << 20;

// Irreps of the dihedral group of the regular n-gon: 1-D ones (A1, A2, and B1,
// B2 for even n) and 2-D ones E_k.
int dihedral_one_dim(int n) { return n % 2 == 0 ? 4 : 2; }
int dihedral_two_dim(int n) { return n % 2 == 0 ? n / 2 - 1 : (n - 1) / 2; }

}  // namespace

extern "C" {

const char* eqlinear_status_string(eqlinear_status s) {
    switch (s) {
        case EQL_OK: return "EQL_OK";
        case EQL_ERR_INVALID: return "EQL_ERR_INVALID: invalid argument";
        case EQL_ERR_UNSUPPORTED: return "EQL_ERR_UNSUPPORTED: not supported by the library";
        case EQL_ERR_HIP: return "EQL_ERR_HIP: HIP runtime or kernel launch error";
        case EQL_ERR_NOMEM: return "EQL_ERR_NOMEM: host allocation failed";
    }
    return "EQL_ERR_UNKNOWN: unknown status code";
}

eqlinear_status eqlinear_plan(eqlinear_plan_t* out, int N, int C_in, int C_out,
                              eqlinear_dtype dt) {
    if (!out) return EQL_ERR_INVALID;
    *out = nullptr;
    if (N < 1 || N > 16 || C_in < 1 || C_out < 1 || !dtype_ok((int)dt)) return EQL_ERR_INVALID;
    if ((int64_t)N * C_in > kMaxWidth || (int64_t)N * C_out > kMaxWidth) return EQL_ERR_INVALID;
    eqlinear_plan_s* p = new (std::nothrow) eqlinear_plan_s{EQL_KIND_CN, (int)dt, N, C_in, C_out};
    if (!p) return EQL_ERR_NOMEM;
    *out = p;
    return EQL_OK;
}

eqlinear_status eqlinear_dihedral_plan(eqlinear_plan_t* out, int n, int C_in, int C_out, eqlinear_dtype dt) {
    if (!out) return EQL_ERR_INVALID;
    *out = nullptr;
    if (n < 2 || n > 12) return EQL_ERR_INVALID;
    const int G = 2 * n;  // group order: the plan's N
    if (C_in < G || C_out < G || C_in % G || C_out % G || !dtype_ok((int)dt)) return EQL_ERR_INVALID;
    if (C_in > kMaxWidth || C_out > kMaxWidth) return EQL_ERR_INVALID;
    eqlinear_plan_s* p = new (std::nothrow) eqlinear_plan_s{EQL_KIND_D8, (int)dt, G, C_in, C_out};
    if (!p) return EQL_ERR_NOMEM;
    *out = p;
    return EQL_OK;
}

eqlinear_status eqlinear_d8_plan(eqlinear_plan_t* out, int C_in, int C_out, eqlinear_dtype dt) {
    return eqlinear_dihedral_plan(out, 4, C_in, C_out, dt);
}

eqlinear_status eqlinear_plan_destroy(eqlinear_plan_t plan) {
    if (!plan) return EQL_ERR_INVALID;
    delete plan;
    return EQL_OK;
}

eqlinear_status eqlinear_plan_info(eqlinear_plan_t p, eqlinear_info* out) {
    if (!p || !out) return EQL_ERR_INVALID;
    eqlinear_info in{};
    in.kind = p->kind;
    in.dtype = p->dtype;
    in.N = p->N;
    in.C_in = p->C_in;
    in.C_out = p->C_out;
    const int64_t ci = p->C_in, co = p->C_out;
    if (p->kind == EQL_KIND_CN) {
        const int N = p->N;
        const int complex_bins = (N - 1) / 2;
        const int real_bins = 1 + (N % 2 == 0 && N > 1 ? 1 : 0);
        in.bins = N / 2 + 1;
        in.planes = N;
        in.has_nyquist = (N % 2 == 0 && N > 1) ? 1 : 0;
        in.params = (int64_t)N * ci * co;
        in.w_hat_elems = in.params;
        in.real_gemms = real_bins + 4 * complex_bins;
        in.macs_per_token = in.real_gemms * ci * co;
        in.dense_macs_per_token = (int64_t)N * N * ci * co;
    } else {
        const int n = p->N / 2;
        const int64_t mi = ci / p->N, mo = co / p->N;
        const int n1 = dihedral_one_dim(n), n2 = dihedral_two_dim(n);
        in.bins = n1 + n2;  // irrep blocks
        in.planes = 0;
        in.has_nyquist = 0;
        in.params = n1 * mi * mo + n2 * (2 * mi) * (2 * mo);
        in.w_hat_elems = in.params;
        in.real_gemms = 0;
        in.macs_per_token = n1 * mi * mo + 2 * n2 * (2 * mi) * (2 * mo);
        in.dense_macs_per_token = ci * co;
    }
    *out = in;
    return EQL_OK;
}

size_t eqlinear_w_hat_elems(eqlinear_plan_t p) {
    if (!p) return 0;
    eqlinear_info in;
    if (eqlinear_plan_info(p, &in) != EQL_OK) return 0;
    return (size_t)in.w_hat_elems;
}

eqlinear_status eqlinear_weight_fft(eqlinear_plan_t p, const void* w, void* w_hat) {
    if (!p || !w || !w_hat || p->kind != EQL_KIND_CN) return EQL_ERR_INVALID;
    if (!aligned16(w) || !aligned16(w_hat)) return EQL_ERR_INVALID;
    const size_t bytes = eqlinear_w_hat_elems(p) * elem_size(p);
    if (overlaps(w, bytes, w_hat, bytes)) return EQL_ERR_INVALID;
    hipError_t e = eql::launch_weight_dft(p->N, p->dtype, w, w_hat, p->C_in,
                                          p->C_out, nullptr);
    if (e != hipSuccess) return EQL_ERR_HIP;
    return hip_status(hipStreamSynchronize(nullptr));
}

eqlinear_status eqlinear_forward_tiled(eqlinear_plan_t p, const void* x, const void* w_hat,
                                      void* y, int64_t T, void* stream, int tile) {
    if (!p || p->kind != EQL_KIND_CN) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!x || !w_hat || !y) return EQL_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w_hat) || !aligned16(y)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t xb = (size_t)T * in_width(p) * es, yb = (size_t)T * out_width(p) * es;
    const size_t wb = eqlinear_w_hat_elems(p) * es;
    if (overlaps(x, xb, y, yb) || overlaps(w_hat, wb, y, yb)) return EQL_ERR_INVALID;
    if (tile < -1 || tile > 17) return EQL_ERR_INVALID;
    return hip_status(eql::launch_cn_forward(p->N, p->dtype, x, w_hat, y, T, p->C_in,
                                             p->C_out, (hipStream_t)stream, tile));
}

eqlinear_status eqlinear_forward(eqlinear_plan_t p, const void* x, const void* w_hat, void* y,
                                 int64_t T, void* stream) {
    return eqlinear_forward_tiled(p, x, w_hat, y, T, stream, -1);
}

eqlinear_status eqlinear_forward_bias_act(eqlinear_plan_t p, const void* x, const void* w_hat, const void* bias,
                                          int act, void* y, int64_t T, void* stream, int tile) {
    if (!p || p->kind != EQL_KIND_CN) return EQL_ERR_INVALID;
    if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!x || !w_hat || !y) return EQL_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w_hat) || !aligned16(y)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t xb = (size_t)T * in_width(p) * es, yb = (size_t)T * out_width(p) * es;
    const size_t wb = eqlinear_w_hat_elems(p) * es, bb = (size_t)p->C_out * es;
    if (overlaps(x, xb, y, yb) || overlaps(w_hat, wb, y, yb)) return EQL_ERR_INVALID;
    if (bias && (((uintptr_t)bias % es) != 0 || overlaps(bias, bb, y, yb))) return EQL_ERR_INVALID;
    if (tile < -1 || tile > 17) return EQL_ERR_INVALID;
    return hip_status(eql::launch_cn_forward(p->N, p->dtype, x, w_hat, y, T, p->C_in, p->C_out,
                                             (hipStream_t)stream, tile, eql::Epi{bias, act}));
}

eqlinear_status eqlinear_d8_bias_act(eqlinear_plan_t p, const void* y_in, const void* bias, int act, void* y_out,
                                     int64_t T, void* stream) {
    if (!p || p->kind != EQL_KIND_D8) return EQL_ERR_INVALID;
    if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!y_in || !y_out || !aligned16(y_in) || !aligned16(y_out)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t yb = (size_t)T * p->C_out * es, bb = (size_t)(p->C_out / p->N) * es;
    if (y_in != y_out && overlaps(y_in, yb, y_out, yb)) return EQL_ERR_INVALID;  // in place, or apart
    if (bias && (((uintptr_t)bias % es) != 0 || overlaps(bias, bb, y_out, yb))) return EQL_ERR_INVALID;
    return hip_status(eql::launch_dn_round_trip(p->N / 2, p->dtype, y_in, y_out, bias, act,
                                                p->C_out / p->N, T, (hipStream_t)stream));
}

eqlinear_status eqlinear_d8_regular_forward(eqlinear_plan_t p, const void* x_reg, const void* wb, const void* bias,
                                            int act, void* y_reg, int64_t T, void* stream) {
    if (!p || p->kind != EQL_KIND_D8) return EQL_ERR_INVALID;
    if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (p->dtype == EQL_F32) return EQL_ERR_UNSUPPORTED;
    const int mi = p->C_in / p->N, mo = p->C_out / p->N;
    if (mi % 8 || mo % 8) return EQL_ERR_UNSUPPORTED;
    if (T == 0) return EQL_OK;
    if (!x_reg || !wb || !y_reg) return EQL_ERR_INVALID;
    if (!aligned16(x_reg) || !aligned16(wb) || !aligned16(y_reg)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t xb = (size_t)T * p->C_in * es, yb = (size_t)T * p->C_out * es;
    const size_t wbb = eqlinear_w_hat_elems(p) * es, bb = (size_t)mo * es;
    if (overlaps(x_reg, xb, y_reg, yb) || overlaps(wb, wbb, y_reg, yb)) return EQL_ERR_INVALID;
    if (bias && (((uintptr_t)bias % es) != 0 || overlaps(bias, bb, y_reg, yb))) return EQL_ERR_INVALID;
    const hipError_t e = eql::launch_dn_regular(p->N / 2, p->dtype, x_reg, wb, bias, act, y_reg, T, mi, mo,
                                                (int64_t)eqlinear_w_hat_elems(p), (hipStream_t)stream);
    return e == hipErrorNotSupported ? EQL_ERR_UNSUPPORTED : hip_status(e);
}

eqlinear_status eqlinear_d8_to_fourier(eqlinear_plan_t p, const void* x_reg, void* x_four, int64_t T,
                                       void* stream) {
    if (!p || p->kind != EQL_KIND_D8) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!x_reg || !x_four || !aligned16(x_reg) || !aligned16(x_four)) return EQL_ERR_INVALID;
    const size_t b = (size_t)T * p->C_in * elem_size(p);
    if (overlaps(x_reg, b, x_four, b)) return EQL_ERR_INVALID;
    return hip_status(eql::launch_dn_to_fourier(p->N / 2, p->dtype, x_reg, x_four, p->C_in / p->N,
                                                T, (hipStream_t)stream));
}

eqlinear_status eqlinear_d8_to_regular(eqlinear_plan_t p, const void* y_four, void* y_reg, int64_t T,
                                       void* stream) {
    if (!p || p->kind != EQL_KIND_D8) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!y_four || !y_reg || !aligned16(y_four) || !aligned16(y_reg)) return EQL_ERR_INVALID;
    const size_t b = (size_t)T * p->C_out * elem_size(p);
    if (overlaps(y_four, b, y_reg, b)) return EQL_ERR_INVALID;
    return hip_status(eql::launch_dn_to_regular(p->N / 2, p->dtype, y_four, y_reg, p->C_out / p->N,
                                                T, (hipStream_t)stream));
}

eqlinear_status eqlinear_w_hat_adjoint(eqlinear_plan_t p, const void* w_hat, void* w_hat_adj, void* stream) {
    if (!p || p->kind != EQL_KIND_CN || !w_hat || !w_hat_adj) return EQL_ERR_INVALID;
    if (!aligned16(w_hat) || !aligned16(w_hat_adj)) return EQL_ERR_INVALID;
    const size_t b = eqlinear_w_hat_elems(p) * elem_size(p);
    if (overlaps(w_hat, b, w_hat_adj, b)) return EQL_ERR_INVALID;
    return hip_status(eql::launch_w_hat_adjoint(p->N, p->dtype, w_hat, w_hat_adj, p->C_in, p->C_out,
                                                (hipStream_t)stream));
}

eqlinear_status eqlinear_backward_data(eqlinear_plan_t p, const void* dy, const void* w_hat_adj, void* dx,
                                       int64_t T, void* stream) {
    if (!p || p->kind != EQL_KIND_CN) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!dy || !w_hat_adj || !dx) return EQL_ERR_INVALID;
    if (!aligned16(dy) || !aligned16(w_hat_adj) || !aligned16(dx)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t dyb = (size_t)T * out_width(p) * es, dxb = (size_t)T * in_width(p) * es;
    const size_t wb = eqlinear_w_hat_elems(p) * es;
    if (overlaps(dy, dyb, dx, dxb) || overlaps(w_hat_adj, wb, dx, dxb)) return EQL_ERR_INVALID;
    // the layer with C_in and C_out exchanged, run by the forward kernels
    return hip_status(eql::launch_cn_forward(p->N, p->dtype, dy, w_hat_adj, dx, T, p->C_out, p->C_in,
                                             (hipStream_t)stream, -1));
}

size_t eqlinear_backward_weight_workspace(eqlinear_plan_t p, int64_t T) {
    if (!p || p->kind != EQL_KIND_CN || T < 0) return 0;
    return eql::backward_weight_workspace(p->N, p->dtype, T, p->C_in, p->C_out);
}

eqlinear_status eqlinear_backward_weight(eqlinear_plan_t p, const void* x, const void* dy, float* dw, int64_t T,
                                         void* workspace, size_t workspace_bytes, void* stream) {
    if (!p || p->kind != EQL_KIND_CN || !dw) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (!aligned16(dw)) return EQL_ERR_INVALID;
    const size_t dwb = eqlinear_w_hat_elems(p) * sizeof(float);
    if (T > 0) {
        if (!x || !dy || !workspace) return EQL_ERR_INVALID;
        if (!aligned16(x) || !aligned16(dy) || ((uintptr_t)workspace & 255u) != 0) return EQL_ERR_INVALID;
        const size_t need = eql::backward_weight_workspace(p->N, p->dtype, T, p->C_in, p->C_out);
        if (workspace_bytes < need) return EQL_ERR_INVALID;
        const size_t es = elem_size(p);
        const size_t xb = (size_t)T * in_width(p) * es, dyb = (size_t)T * out_width(p) * es;
        if (overlaps(dw, dwb, x, xb) || overlaps(dw, dwb, dy, dyb) || overlaps(dw, dwb, workspace, need) ||
            overlaps(workspace, need, x, xb) || overlaps(workspace, need, dy, dyb))
            return EQL_ERR_INVALID;
    }
    const hipError_t e = eql::launch_cn_backward_weight(p->N, p->dtype, x, dy, dw, T, p->C_in, p->C_out,
                                                        workspace, workspace_bytes, (hipStream_t)stream);
    return e == hipErrorNotSupported ? EQL_ERR_UNSUPPORTED : hip_status(e);
}

eqlinear_status eqlinear_backward_weight_noalloc(eqlinear_plan_t p, const void* x, const void* dy, float* dw,
                                                 int64_t T, void* stream) {
    if (!p || p->kind != EQL_KIND_CN || !dw) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (!aligned16(dw)) return EQL_ERR_INVALID;
    const size_t dwb = eqlinear_w_hat_elems(p) * sizeof(float);
    if (T > 0) {
        if (!x || !dy) return EQL_ERR_INVALID;
        if (!aligned16(x) || !aligned16(dy)) return EQL_ERR_INVALID;
        const size_t es = elem_size(p);
        const size_t xb = (size_t)T * in_width(p) * es, dyb = (size_t)T * out_width(p) * es;
        if (overlaps(dw, dwb, x, xb) || overlaps(dw, dwb, dy, dyb)) return EQL_ERR_INVALID;
        // the library-held scratch has a fixed size: larger shapes are refused here
        if (eql::backward_weight_workspace(p->N, p->dtype, T, p->C_in, p->C_out) > eql::kNoAllocScratchBytes)
            return EQL_ERR_UNSUPPORTED;
    }
    // the scratch array used is the current device's: the stream must be one of its streams
    if (stream) {
        int cur = -1, sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
            return EQL_ERR_HIP;
        if (cur != sdev) return EQL_ERR_INVALID;
    }
    const hipError_t e = eql::launch_cn_backward_weight_noalloc(p->N, p->dtype, x, dy, dw, T, p->C_in, p->C_out,
                                                                (hipStream_t)stream);
    if (e == hipErrorOutOfMemory) return EQL_ERR_UNSUPPORTED;
    return e == hipErrorNotSupported ? EQL_ERR_UNSUPPORTED : hip_status(e);
}

eqlinear_status eqlinear_d8_forward(eqlinear_plan_t p, const void* x, const void* wb, void* y,
                                    int64_t T, void* stream) {
    if (!p || p->kind != EQL_KIND_D8) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!x || !wb || !y) return EQL_ERR_INVALID;
    if (!aligned16(x) || !aligned16(wb) || !aligned16(y)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t xb = (size_t)T * p->C_in * es, yb = (size_t)T * p->C_out * es;
    const size_t wbb = eqlinear_w_hat_elems(p) * es;
    if (overlaps(x, xb, y, yb) || overlaps(wb, wbb, y, yb)) return EQL_ERR_INVALID;
    const int n = p->N / 2, mi = p->C_in / p->N, mo = p->C_out / p->N;
    const int n1 = dihedral_one_dim(n), n2 = dihedral_two_dim(n);
    eql::GemmJobs jobs{};
    jobs.njobs = n1 + 2 * n2;  // <= kMaxGemmJobs for n <= 12
    for (int b = 0; b < n1; ++b)  // A1, A2 (, B1, B2)
        jobs.j[b] = eql::GemmJob{b * mi, b * mo, mi, mo, (int64_t)b * mo * mi, mi, 0, 0, 0, 0};
    for (int k = 0; k < n2; ++k)  // W of E_{k+1} on its coordinate 0 and 1
        for (int c = 0; c < 2; ++c)
            jobs.j[n1 + 2 * k + c] =
                eql::GemmJob{n1 * mi + 4 * k * mi + 2 * c * mi, n1 * mo + 4 * k * mo + 2 * c * mo, 2 * mi, 2 * mo,
                             (int64_t)n1 * mo * mi + (int64_t)k * 4 * mo * mi, 2 * mi, 0, 0, 0, 0};
    if (p->dtype == EQL_BF16 || p->dtype == EQL_F16) {
        // widest output tile that the 1-D blocks fill: 160, 96, 80 or 32 channels
        const int cb = mo % 160 == 0 ? 10 : (mo % 96 == 0 ? 6 : (mo % 80 == 0 ? 5 : 2));
        const hipError_t e = eql::launch_d8_fast(p->dtype, jobs, x, wb, y, T, p->C_in, p->C_out,
                                                 (int64_t)eqlinear_w_hat_elems(p), cb, (hipStream_t)stream);
        if (e != hipErrorNotSupported) return hip_status(e);
    }
    return hip_status(eql::launch_gemm_rows(p->dtype, jobs, x, wb, y, T, p->C_in,
                                            p->C_out, (hipStream_t)stream));
}

eqlinear_status eqlinear_expand_dense(eqlinear_plan_t p, const void* w, void* w_dense,
                                      void* stream) {
    if (!p || !w || !w_dense) return EQL_ERR_INVALID;
    if (!aligned16(w) || !aligned16(w_dense)) return EQL_ERR_INVALID;
    const size_t es = elem_size(p);
    const size_t wb = eqlinear_w_hat_elems(p) * es;
    const size_t db = (size_t)in_width(p) * out_width(p) * es;
    if (overlaps(w, wb, w_dense, db)) return EQL_ERR_INVALID;
    hipError_t e;
    if (p->kind == EQL_KIND_CN)
        e = eql::launch_cn_expand(p->N, p->dtype, w, w_dense, p->C_in, p->C_out,
                                  (hipStream_t)stream);
    else
        e = eql::launch_dn_expand(p->N / 2, p->dtype, w, w_dense, p->C_in, p->C_out,
                                  (hipStream_t)stream);
    return hip_status(e);
}

eqlinear_status eqlinear_dense_forward(eqlinear_plan_t p, const void* x, const void* w_dense,
                                       void* y, int64_t T, void* stream) {
    if (!p) return EQL_ERR_INVALID;
    if (T < 0) return EQL_ERR_INVALID;
    if (T == 0) return EQL_OK;
    if (!x || !w_dense || !y) return EQL_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w_dense) || !aligned16(y)) return EQL_ERR_INVALID;
    const int64_t K = in_width(p), M = out_width(p);
    const size_t es = elem_size(p);
    const size_t xb = (size_t)T * K * es, yb = (size_t)T * M * es, db = (size_t)K * M * es;
    if (overlaps(x, xb, y, yb) || overlaps(w_dense, db, y, yb)) return EQL_ERR_INVALID;
    eql::GemmJobs jobs{};
    jobs.njobs = 1;
    jobs.j[0] = eql::GemmJob{0, 0, (int)K, (int)M, 0, (int)K, 0, 0, 0, 0};
    return hip_status(eql::launch_gemm_rows(p->dtype, jobs, x, w_dense, y, T, (int)K,
                                            (int)M, (hipStream_t)stream));
}

}  // extern "C"

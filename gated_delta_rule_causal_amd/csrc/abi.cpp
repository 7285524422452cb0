// C ABI of liblinattn.so: host-side validation and dispatch to the gfx950
// kernels.  The public contract (argument meaning, layouts, ownership, error
// behaviour) is documented in include/linattn.h.
#include "linattn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kernels.hpp"

namespace {

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kParallelMaxT = 8192;

bool valid_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};

bool overlaps(Span a, Span b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Sizes: all element counts are computed in 64 bits; the bound keeps every
// per-tensor byte count far below 2^63 and every head index within a grid
// dimension.
bool sizes_ok(long long B, long long H, long long T) {
    if (B < 0 || H < 0 || T < 0) return false;
    if (B * H > 0x7fffffffLL) return false;
    if (T > (1LL << 30)) return false;
    return B * H * T <= (1LL << 40);
}

size_t io_size(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

// hipErrorInvalidConfiguration is what the launchers return for a grid of
// 2^32 or more work-items (sizes that pass the bounds above but are more than
// one launch can hold): a shape the library cannot run.
la_status from_hip(hipError_t e) {
    return e == hipSuccess ? LA_OK : e == hipErrorInvalidConfiguration ? LA_ERR_SHAPE : LA_ERR_HIP;
}

// Copy S0 -> S_out (zero-fill when S0 is NULL) for empty sequences.
__global__ void state_copy_kernel(const float* src, float* dst, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

la_status copy_state(const float* src, float* dst, size_t n, hipStream_t s) {
    if (dst == nullptr || n == 0 || src == dst) return LA_OK;
    const unsigned blocks = static_cast<unsigned>((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(state_copy_kernel, dim3(blocks), dim3(256), 0, s, src, dst, n);
    return from_hip(hipGetLastError());
}

// seg_base and snap_base of a packed batch, [N+1] ints each, rounded to 256 bytes
// seg_base, snap_base ([N+1] each) and the sequences longest first ([N])
size_t varlen_table_bytes(int N) { return N > 0 ? ((3 * static_cast<size_t>(N) + 2) * sizeof(int) + 255) / 256 * 256 : 0; }

size_t la_prefill_ws(int dtype, int B, int H, int T, int dk, int dv, int form, int chunk) {
    if (form == LA_FORM_CHUNKED && la::la_mfma_supported(dtype, dk, dv, chunk))
        return la::la_mfma_workspace_bytes(B, H, T, dk, dv, chunk);
    return 0;
}

size_t gdn_prefill_ws(int dtype, int B, int H, int T, int dk, int dv, int form, int chunk) {
    if (form == LA_FORM_CHUNKED && la::gdn_mfma_supported(dtype, dk, dv, chunk))
        return la::gdn_mfma_workspace_bytes(B, H, T, dk, dv, chunk);
    return 0;
}

// Which kernel family a chunked call uses; -1 when none fits.
int la_chunked_path(int dtype, int dk, int dv, int chunk) {
    if (la::la_mfma_supported(dtype, dk, dv, chunk)) return 1;
    if (la::la_chunked_generic_lds_bytes(dk, dv, chunk) <= kMaxLds) return 0;
    return -1;
}
int gdn_chunked_path(int dtype, int dk, int dv, int chunk) {
    if (la::gdn_mfma_supported(dtype, dk, dv, chunk)) return 1;
    if (la::gdn_chunked_generic_lds_bytes(dk, dv, chunk) <= kMaxLds) return 0;
    return -1;
}

}  // namespace

extern "C" {

int la_abi_version(void) { return LA_ABI_VERSION; }

const char* la_status_str(la_status s) {
    switch (s) {
        case LA_OK: return "LA_OK";
        case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
        case LA_ERR_SHAPE: return "LA_ERR_SHAPE: a size is negative, unsupported or too large";
        case LA_ERR_DTYPE: return "LA_ERR_DTYPE: dtype must be LA_F32 or LA_BF16";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: valid arguments, combination not implemented";
        case LA_ERR_ALIGN: return "LA_ERR_ALIGN: a pointer is not 16-byte aligned";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
        case LA_ERR_HIP: return "LA_ERR_HIP: the HIP runtime reported an error";
        case LA_ERR_ARG: return "LA_ERR_ARG: bad enum value or overlapping buffers";
        default: return "unknown la_status";
    }
}

size_t la_workspace_bytes(int fn, int dtype, int B, int H, int T, int dk, int dv, int form, int chunk) {
    const size_t bad = static_cast<size_t>(-1);
    if (dtype != LA_F32 && dtype != LA_BF16) return bad;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv)) return bad;
    if (fn == LA_FN_DECODE_STEP) return 0;  // form and chunk do not apply
    if (form == LA_FORM_CHUNKED && !valid_chunk(chunk)) return bad;
    switch (fn) {
        case LA_FN_LIN_ATTN_PREFILL:
            if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT && form != LA_FORM_PARALLEL) return bad;
            if (form == LA_FORM_CHUNKED && la_chunked_path(dtype, dk, dv, chunk) < 0) return bad;
            return la_prefill_ws(dtype, B, H, T, dk, dv, form, chunk);
        case LA_FN_GDN_PREFILL:
            if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return bad;
            if (form == LA_FORM_CHUNKED && gdn_chunked_path(dtype, dk, dv, chunk) < 0) return bad;
            return gdn_prefill_ws(dtype, B, H, T, dk, dv, form, chunk);
        case LA_FN_GLA_PREFILL:
            if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return bad;
            if (form == LA_FORM_CHUNKED && !la::la_mfma_supported(dtype, dk, dv, chunk)) return bad;
            return form == LA_FORM_CHUNKED ? la::la_mfma_workspace_bytes(B, H, T, dk, dv, chunk) : 0;
        case LA_FN_KDA_PREFILL:
            if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return bad;
            if (form == LA_FORM_CHUNKED && !la::kda_mfma_supported(dtype, dk, dv, chunk)) return bad;
            return form == LA_FORM_CHUNKED ? la::kda_mfma_workspace_bytes(B, H, T) : 0;
        case LA_FN_GDN_VARLEN:   // B = number of sequences, T = total tokens
            if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return bad;
            if (form == LA_FORM_CHUNKED && !la::gdn_mfma_supported(dtype, dk, dv, chunk)) return bad;
            return form == LA_FORM_CHUNKED ? la::gdn_mfma_varlen_workspace_bytes(B, H, T) : varlen_table_bytes(B);
        case LA_FN_PREFILL_VARLEN:   // every kind: the largest of their needs
            if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return bad;
            if (form == LA_FORM_CHUNKED && !la::gdn_mfma_supported(dtype, dk, dv, chunk)) return bad;
            if (form == LA_FORM_RECURRENT) return varlen_table_bytes(B);
            return std::max({la::gdn_mfma_varlen_workspace_bytes(B, H, T), la::kda_mfma_varlen_workspace_bytes(B, H, T),
                             la::la_mfma_varlen_workspace_bytes(B, H, T)});
        default:
            return bad;
    }
}

la_status lin_attn_prefill(int dtype, int B, int H, int T, int dk, int dv, const void* q,
                           const void* k, const void* v, const float* S0, const float* z0, void* o,
                           float* S_out, float* z_out, int form, int chunk, void* workspace,
                           size_t ws_bytes, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT && form != LA_FORM_PARALLEL) return LA_ERR_ARG;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (form == LA_FORM_CHUNKED && !valid_chunk(chunk)) return LA_ERR_SHAPE;
    if (form == LA_FORM_PARALLEL && T > kParallelMaxT) return LA_ERR_SHAPE;
    const size_t heads = static_cast<size_t>(B) * H;
    if (heads == 0) return LA_OK;
    const size_t es = io_size(dtype);
    const size_t nqk = heads * T * dk * es, nv = heads * T * dv * es;
    const size_t nS = heads * dv * dk * sizeof(float), nz = heads * dk * sizeof(float);
    if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr)) return LA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(S0),
                          static_cast<const void*>(z0), static_cast<const void*>(S_out),
                          static_cast<const void*>(z_out), static_cast<const void*>(workspace)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    if (form == LA_FORM_PARALLEL && (S0 != nullptr || z0 != nullptr)) return LA_ERR_ARG;
    // outputs must not overlap inputs, except the documented in-place states
    const Span in[] = {{q, nqk}, {k, nqk}, {v, nv}, {S0, nS}, {z0, nz}};
    const Span outs[] = {{o, T > 0 ? nv : 0}, {S_out, nS}, {z_out, nz}};
    for (const Span& a : outs)
        for (const Span& b : in) {
            if ((a.p == S_out && b.p == S0 && S_out == S0) || (a.p == z_out && b.p == z0 && z_out == z0)) continue;
            if (overlaps(a, b)) return LA_ERR_ARG;
        }
    if (overlaps(outs[0], outs[1]) || overlaps(outs[0], outs[2]) || overlaps(outs[1], outs[2])) return LA_ERR_ARG;
    int path = 0;
    if (form == LA_FORM_CHUNKED) {
        path = la_chunked_path(dtype, dk, dv, chunk);
        if (path < 0) return LA_ERR_UNSUPPORTED;
    }
    const size_t need = la_prefill_ws(dtype, B, H, T, dk, dv, form, chunk);
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    if (need > 0) {
        const Span w{workspace, need};
        for (const Span& b : in)
            if (overlaps(w, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (overlaps(w, b)) return LA_ERR_ARG;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        la_status st = copy_state(S0, S_out, heads * dv * dk, s);
        if (st != LA_OK) return st;
        return copy_state(z0, z_out, heads * dk, s);
    }
    const int nh = static_cast<int>(heads);
    switch (form) {
        case LA_FORM_PARALLEL:
            return from_hip(la::launch_la_parallel(dtype, nh, T, dk, dv, q, k, v, o, S_out, z_out, s));
        case LA_FORM_RECURRENT:
            return from_hip(la::launch_recurrent(la::kNormalized, dtype, nh, T, dk, dv, q, k, v, nullptr,
                                                 nullptr, S0, S_out, z0, z_out, o, s));
        default:
            if (path == 1)
                return from_hip(la::launch_la_mfma(B, H, T, q, k, v, S0, z0, o, S_out, z_out, workspace, s));
            return from_hip(la::launch_la_chunked_generic(dtype, nh, T, dk, dv, chunk, q, k, v, S0, z0, o,
                                                          S_out, z_out, s));
    }
}

}  // extern "C"

namespace {

// gdn_prefill with either the caller's workspace or (own_ws) the library's
// array, taken only after every argument has been validated.
la_status gdn_prefill_impl(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, const float* S0, void* o,
                           float* S_out, int form, int chunk, void* workspace, size_t ws_bytes, bool own_ws,
                           void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return LA_ERR_ARG;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (form == LA_FORM_CHUNKED && !valid_chunk(chunk)) return LA_ERR_SHAPE;
    const size_t heads = static_cast<size_t>(B) * H;
    if (heads == 0) return LA_OK;
    const size_t es = io_size(dtype);
    const size_t nqk = heads * T * dk * es, nv = heads * T * dv * es, ng = heads * T * sizeof(float);
    const size_t nS = heads * dv * dk * sizeof(float);
    if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || alpha == nullptr ||
                  beta == nullptr))
        return LA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(alpha),
                          static_cast<const void*>(beta), static_cast<const void*>(S0),
                          static_cast<const void*>(S_out), static_cast<const void*>(workspace)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {{q, nqk}, {k, nqk}, {v, nv}, {alpha, ng}, {beta, ng}, {S0, nS}};
    const Span outs[] = {{o, T > 0 ? nv : 0}, {S_out, nS}};
    for (const Span& a : outs)
        for (const Span& b : in) {
            if (a.p == S_out && b.p == S0 && S_out == S0) continue;
            if (overlaps(a, b)) return LA_ERR_ARG;
        }
    if (overlaps(outs[0], outs[1])) return LA_ERR_ARG;
    int path = 0;
    if (form == LA_FORM_CHUNKED) {
        path = gdn_chunked_path(dtype, dk, dv, chunk);
        if (path < 0) return LA_ERR_UNSUPPORTED;
    }
    const size_t need = gdn_prefill_ws(dtype, B, H, T, dk, dv, form, chunk);
    if (own_ws && need > 0) {
        if (need > la::gdn_scratch_bytes()) return LA_ERR_WORKSPACE;
        if (la::gdn_scratch(&workspace) != hipSuccess) return LA_ERR_HIP;
        ws_bytes = need;
    }
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    if (need > 0 && (overlaps({workspace, need}, outs[0]) || overlaps({workspace, need}, outs[1]) ||
                     overlaps({workspace, need}, Span{S0, nS})))
        return LA_ERR_ARG;
    for (const Span& b : in)
        if (need > 0 && overlaps({workspace, need}, b)) return LA_ERR_ARG;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) return copy_state(S0, S_out, heads * dv * dk, s);
    const int nh = static_cast<int>(heads);
    if (form == LA_FORM_RECURRENT)
        return from_hip(la::launch_recurrent(la::kGatedDelta, dtype, nh, T, dk, dv, q, k, v, alpha, beta,
                                             S0, S_out, nullptr, nullptr, o, s));
    if (path == 1)
        return from_hip(la::launch_gdn_mfma(B, H, T, q, k, v, alpha, beta, S0, o, S_out, workspace, s));
    return from_hip(la::launch_gdn_chunked_generic(dtype, nh, T, dk, dv, chunk, q, k, v, alpha, beta, S0,
                                                   o, S_out, s));
}

}  // namespace

extern "C" {

la_status gdn_prefill(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, const float* S0, void* o,
                      float* S_out, int form, int chunk, void* workspace, size_t ws_bytes,
                      void* stream) {
    return gdn_prefill_impl(dtype, B, H, T, dk, dv, q, k, v, alpha, beta, S0, o, S_out, form, chunk, workspace,
                            ws_bytes, false, stream);
}

la_status gdn_prefill_noalloc(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
                              const void* v, const float* alpha, const float* beta, const float* S0, void* o,
                              float* S_out, int form, int chunk, void* stream) {
    return gdn_prefill_impl(dtype, B, H, T, dk, dv, q, k, v, alpha, beta, S0, o, S_out, form, chunk, nullptr, 0,
                            true, stream);
}

la_status gla_prefill(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
                      const void* v, const float* alpha, const float* S0, void* o, float* S_out, int form,
                      int chunk, void* workspace, size_t ws_bytes, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return LA_ERR_ARG;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (form == LA_FORM_CHUNKED && !valid_chunk(chunk)) return LA_ERR_SHAPE;
    const size_t heads = static_cast<size_t>(B) * H;
    if (heads == 0) return LA_OK;
    const size_t es = io_size(dtype);
    const size_t nqk = heads * T * dk * es, nv = heads * T * dv * es, ng = heads * T * sizeof(float);
    const size_t nS = heads * dv * dk * sizeof(float);
    if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || alpha == nullptr))
        return LA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(alpha),
                          static_cast<const void*>(S0), static_cast<const void*>(S_out),
                          static_cast<const void*>(workspace)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {{q, nqk}, {k, nqk}, {v, nv}, {alpha, ng}, {S0, nS}};
    const Span outs[] = {{o, T > 0 ? nv : 0}, {S_out, nS}};
    for (const Span& a : outs)
        for (const Span& b : in) {
            if (a.p == S_out && b.p == S0 && S_out == S0) continue;
            if (overlaps(a, b)) return LA_ERR_ARG;
        }
    if (overlaps(outs[0], outs[1])) return LA_ERR_ARG;
    if (form == LA_FORM_CHUNKED && !la::la_mfma_supported(dtype, dk, dv, chunk)) return LA_ERR_UNSUPPORTED;
    const size_t need = form == LA_FORM_CHUNKED ? la::la_mfma_workspace_bytes(B, H, T, dk, dv, chunk) : 0;
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    if (need > 0) {
        const Span w{workspace, need};
        for (const Span& b : in)
            if (overlaps(w, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (overlaps(w, b)) return LA_ERR_ARG;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) return copy_state(S0, S_out, heads * dv * dk, s);
    if (form == LA_FORM_RECURRENT)
        return from_hip(la::launch_recurrent(la::kGated, dtype, static_cast<int>(heads), T, dk, dv, q, k, v, alpha,
                                             nullptr, S0, S_out, nullptr, nullptr, o, s));
    return from_hip(la::launch_gla_mfma(B, H, T, q, k, v, alpha, S0, o, S_out, workspace, s));
}

la_status gdn_preprocess(int dtype, int B, int T, int H, int dk, int dv, const void* x, const float* conv_w,
                         const float* a_logit, const float* b_logit, const void* conv_state, void* conv_state_out,
                         void* q, void* k, void* v, float* alpha, float* beta, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (static_cast<long long>(H) * (2 * dk + dv) > 0x7fffffffLL) return LA_ERR_SHAPE;
    // one workgroup of 256 threads per (sequence, head, 128-token tile, part of q / k / v): the
    // grid's work items must fit 32 bits
    if (static_cast<long long>(B) * H * ((T + 127) / 128 > 0 ? (T + 127) / 128 : 1) * 3 * 256 > 0xffffffffLL)
        return LA_ERR_SHAPE;
    if (B == 0 || H == 0) return LA_OK;
    const size_t es = io_size(dtype);
    const size_t C = static_cast<size_t>(H) * (2 * dk + dv);
    const size_t rows = static_cast<size_t>(B) * T;
    if (conv_w == nullptr) return LA_ERR_NULL;
    if (T > 0 && (x == nullptr || a_logit == nullptr || b_logit == nullptr || q == nullptr || k == nullptr ||
                  v == nullptr || alpha == nullptr || beta == nullptr))
        return LA_ERR_NULL;
    for (const void* p : {x, static_cast<const void*>(conv_w), static_cast<const void*>(a_logit),
                          static_cast<const void*>(b_logit), conv_state, static_cast<const void*>(conv_state_out),
                          static_cast<const void*>(q), static_cast<const void*>(k), static_cast<const void*>(v),
                          static_cast<const void*>(alpha), static_cast<const void*>(beta)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const size_t nx = rows * C * es, nl = rows * H * sizeof(float), nst = static_cast<size_t>(B) * 3 * C * es;
    const size_t nqk = rows * H * dk * es, nv = rows * H * dv * es;
    const Span in[] = {{x, nx}, {conv_w, C * 4 * sizeof(float)}, {a_logit, nl}, {b_logit, nl}, {conv_state, nst}};
    const Span outs[] = {{conv_state_out, nst}, {q, nqk}, {k, nqk}, {v, nv}, {alpha, nl}, {beta, nl}};
    for (const Span& a : outs) {
        for (const Span& b : in)
            if (overlaps(a, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (&a != &b && overlaps(a, b)) return LA_ERR_ARG;
    }
    if (T == 0 && conv_state_out == nullptr) return LA_OK;
    return from_hip(la::launch_gdn_preprocess(dtype, B, T, H, dk, dv, x, conv_w, a_logit, b_logit, conv_state,
                                              conv_state_out, q, k, v, alpha, beta,
                                              static_cast<hipStream_t>(stream)));
}

la_status gdn_preprocess_varlen(int dtype, int N, int T_total, int H, int dk, int dv, const int* cu_seqlens,
                                const void* x, const float* conv_w, const float* a_logit, const float* b_logit,
                                const void* conv_state, void* conv_state_out, void* q, void* k, void* v, float* alpha,
                                float* beta, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (!sizes_ok(N, H, T_total) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (static_cast<long long>(H) * (2 * dk + dv) > 0x7fffffffLL) return LA_ERR_SHAPE;
    if (static_cast<long long>(H) * ((T_total + 127) / 128 > 0 ? (T_total + 127) / 128 : 1) * 3 * 256 > 0xffffffffLL)
        return LA_ERR_SHAPE;
    if (N == 0 || H == 0) return LA_OK;
    if (cu_seqlens == nullptr || conv_w == nullptr) return LA_ERR_NULL;
    if (T_total > 0 && (x == nullptr || a_logit == nullptr || b_logit == nullptr || q == nullptr || k == nullptr ||
                        v == nullptr || alpha == nullptr || beta == nullptr))
        return LA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return LA_ERR_ALIGN;
    for (const void* p : {x, static_cast<const void*>(conv_w), static_cast<const void*>(a_logit),
                          static_cast<const void*>(b_logit), conv_state, static_cast<const void*>(conv_state_out),
                          static_cast<const void*>(q), static_cast<const void*>(k), static_cast<const void*>(v),
                          static_cast<const void*>(alpha), static_cast<const void*>(beta)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const size_t es = io_size(dtype);
    const size_t C = static_cast<size_t>(H) * (2 * dk + dv);
    const size_t rows = static_cast<size_t>(T_total);
    const size_t nx = rows * C * es, nl = rows * H * sizeof(float), nst = static_cast<size_t>(N) * 3 * C * es;
    const size_t nqk = rows * H * dk * es, nv = rows * H * dv * es;
    const Span in[] = {{x, nx}, {conv_w, C * 4 * sizeof(float)}, {a_logit, nl}, {b_logit, nl}, {conv_state, nst},
                       {cu_seqlens, (static_cast<size_t>(N) + 1) * sizeof(int)}};
    const Span outs[] = {{conv_state_out, nst}, {q, nqk}, {k, nqk}, {v, nv}, {alpha, nl}, {beta, nl}};
    for (const Span& a : outs) {
        for (const Span& b : in)
            if (overlaps(a, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (&a != &b && overlaps(a, b)) return LA_ERR_ARG;
    }
    return from_hip(la::launch_gdn_preprocess_varlen(dtype, N, T_total, H, dk, dv, cu_seqlens, x, conv_w, a_logit,
                                                     b_logit, conv_state, conv_state_out, q, k, v, alpha, beta,
                                                     static_cast<hipStream_t>(stream)));
}

la_status gdn_prefill_varlen(int dtype, int N, int H, int T_total, int dk, int dv, const int* cu_seqlens,
                             const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                             const float* S0, void* o, float* S_out, int snap_interval, int snap_count,
                             float* S_snap, int form, int chunk, void* workspace, size_t ws_bytes, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return LA_ERR_ARG;
    if (!sizes_ok(N, H, T_total) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (static_cast<long long>(T_total) * H > 0x7fffffffLL) return LA_ERR_SHAPE;
    if (snap_interval < 0 || snap_count < 0) return LA_ERR_SHAPE;
    if (form == LA_FORM_CHUNKED) {
        if (!valid_chunk(chunk)) return LA_ERR_SHAPE;
        if (!la::gdn_mfma_supported(dtype, dk, dv, chunk)) return LA_ERR_UNSUPPORTED;
        if (snap_interval % la::kMfmaChunk != 0) return LA_ERR_SHAPE;
    }
    if (N == 0 || H == 0) return LA_OK;
    if (cu_seqlens == nullptr) return LA_ERR_NULL;
    if (T_total > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || alpha == nullptr ||
                        beta == nullptr))
        return LA_ERR_NULL;
    if (snap_interval > 0 && snap_count > 0 && S_snap == nullptr) return LA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return LA_ERR_ALIGN;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(alpha),
                          static_cast<const void*>(beta), static_cast<const void*>(S0),
                          static_cast<const void*>(S_out), static_cast<const void*>(S_snap),
                          static_cast<const void*>(workspace)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const size_t es = io_size(dtype);
    const size_t rows = static_cast<size_t>(H) * T_total;
    const size_t nS = static_cast<size_t>(N) * H * dv * dk * sizeof(float);
    const size_t nsnap = snap_interval > 0 ? static_cast<size_t>(snap_count) * H * dv * dk * sizeof(float) : 0;
    const Span in[] = {{q, rows * dk * es}, {k, rows * dk * es}, {v, rows * dv * es}, {alpha, rows * sizeof(float)},
                       {beta, rows * sizeof(float)}, {S0, nS}, {cu_seqlens, (static_cast<size_t>(N) + 1) * sizeof(int)}};
    const Span outs[] = {{o, rows * dv * es}, {S_out, nS}, {S_snap, nsnap}};
    for (const Span& a : outs)
        for (const Span& b : in) {
            if (a.p == S_out && b.p == S0 && S_out == S0) continue;
            if (overlaps(a, b)) return LA_ERR_ARG;
        }
    if (overlaps(outs[0], outs[1]) || overlaps(outs[0], outs[2]) || overlaps(outs[1], outs[2])) return LA_ERR_ARG;
    const size_t need = form == LA_FORM_CHUNKED ? la::gdn_mfma_varlen_workspace_bytes(N, H, T_total)
                                                : varlen_table_bytes(N);
    if (workspace == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    {
        const Span w{workspace, need};
        for (const Span& b : in)
            if (overlaps(w, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (overlaps(w, b)) return LA_ERR_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (form == LA_FORM_CHUNKED)
        return from_hip(la::launch_gdn_mfma_varlen(N, H, T_total, cu_seqlens, q, k, v, alpha, beta, S0, o, S_out,
                                                   S_snap ? snap_interval : 0, snap_count, S_snap, workspace, s));
    int* tab = static_cast<int*>(workspace);
    la::Packed pk;
    pk.cu = cu_seqlens;
    pk.snap_base = tab + (N + 1);
    pk.H = H;
    pk.Ttot = T_total;
    pk.snap = S_snap ? snap_interval : 0;
    pk.snap_cap = snap_count;
    pk.S_snap = S_snap;
    pk.seq_order = tab + 2 * (N + 1);
    const hipError_t e = la::launch_varlen_table(N, T_total, 1, pk.snap, cu_seqlens, tab, s, nullptr, 0,
                                                 tab + 2 * (N + 1));
    if (e != hipSuccess) return LA_ERR_HIP;
    return from_hip(la::launch_recurrent(la::kGatedDelta, dtype, N * H, T_total, dk, dv, q, k, v, alpha, beta, S0,
                                         S_out, nullptr, nullptr, o, s, pk));
}

la_status lin_attn_prefill_varlen(int kind, int dtype, int N, int H, int T_total, int dk, int dv,
                                  const int* cu_seqlens, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, const float* S0, const float* z0, void* o,
                                  float* S_out, float* z_out, int snap_interval, int snap_count, float* S_snap,
                                  float* z_snap, int form, int chunk, void* workspace, size_t ws_bytes,
                                  void* stream) {
    if (kind != LA_KIND_NORMALIZED && kind != LA_KIND_GATED_DELTA && kind != LA_KIND_GATED && kind != LA_KIND_KDA)
        return LA_ERR_ARG;
    const bool has_z = kind == LA_KIND_NORMALIZED;
    if (!has_z && (z0 != nullptr || z_out != nullptr || z_snap != nullptr)) return LA_ERR_ARG;
    if (kind == LA_KIND_GATED_DELTA)
        return gdn_prefill_varlen(dtype, N, H, T_total, dk, dv, cu_seqlens, q, k, v, alpha, beta, S0, o, S_out,
                                  snap_interval, snap_count, S_snap, form, chunk, workspace, ws_bytes, stream);
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return LA_ERR_ARG;
    if (kind == LA_KIND_NORMALIZED && (alpha != nullptr || beta != nullptr)) return LA_ERR_ARG;
    if (kind == LA_KIND_GATED && beta != nullptr) return LA_ERR_ARG;
    if (!sizes_ok(N, H, T_total) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (static_cast<long long>(T_total) * H > 0x7fffffffLL) return LA_ERR_SHAPE;
    if (snap_interval < 0 || snap_count < 0) return LA_ERR_SHAPE;
    if (form == LA_FORM_CHUNKED) {   // the block forms, on the matrix cores
        if (!valid_chunk(chunk)) return LA_ERR_SHAPE;
        const bool ok = kind == LA_KIND_KDA ? la::kda_mfma_supported(dtype, dk, dv, chunk)
                                            : la::la_mfma_supported(dtype, dk, dv, chunk);
        if (!ok) return LA_ERR_UNSUPPORTED;
        if (snap_interval % la::kMfmaChunk != 0) return LA_ERR_SHAPE;
    }
    if (N == 0 || H == 0) return LA_OK;
    if (cu_seqlens == nullptr) return LA_ERR_NULL;
    if (T_total > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr)) return LA_ERR_NULL;
    if (T_total > 0 && kind != LA_KIND_NORMALIZED && alpha == nullptr) return LA_ERR_NULL;
    if (T_total > 0 && kind == LA_KIND_KDA && beta == nullptr) return LA_ERR_NULL;
    const bool snaps = snap_interval > 0 && snap_count > 0 && S_snap != nullptr;
    if (snap_interval > 0 && snap_count > 0 && S_snap == nullptr) return LA_ERR_NULL;
    if (snaps && has_z && z_snap == nullptr) return LA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return LA_ERR_ALIGN;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(alpha),
                          static_cast<const void*>(beta), static_cast<const void*>(S0), static_cast<const void*>(z0),
                          static_cast<const void*>(S_out), static_cast<const void*>(z_out),
                          static_cast<const void*>(S_snap), static_cast<const void*>(z_snap),
                          static_cast<const void*>(workspace)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const size_t es = io_size(dtype);
    const size_t rows = static_cast<size_t>(H) * T_total;
    const size_t nS = static_cast<size_t>(N) * H * dv * dk * sizeof(float);
    const size_t nz = static_cast<size_t>(N) * H * dk * sizeof(float);
    const size_t nsnap = snaps ? static_cast<size_t>(snap_count) * H * dv * dk * sizeof(float) : 0;
    const size_t nzsnap = snaps && has_z ? static_cast<size_t>(snap_count) * H * dk * sizeof(float) : 0;
    const size_t na = rows * (kind == LA_KIND_KDA ? dk : 1) * sizeof(float);
    const Span in[] = {{q, rows * dk * es}, {k, rows * dk * es}, {v, rows * dv * es}, {alpha, na},
                       {beta, rows * sizeof(float)}, {S0, nS}, {z0, nz},
                       {cu_seqlens, (static_cast<size_t>(N) + 1) * sizeof(int)}};
    const Span outs[] = {{o, rows * dv * es}, {S_out, nS}, {z_out, has_z ? nz : 0}, {S_snap, nsnap},
                         {z_snap, nzsnap}};
    for (const Span& a : outs) {
        for (const Span& b : in) {
            if (a.p == S_out && b.p == S0 && S_out == S0) continue;   // in-place state update
            if (a.p == z_out && b.p == z0 && z_out == z0) continue;
            if (overlaps(a, b)) return LA_ERR_ARG;
        }
        for (const Span& b : outs)
            if (&a != &b && overlaps(a, b)) return LA_ERR_ARG;
    }
    const size_t need = form != LA_FORM_CHUNKED ? varlen_table_bytes(N)
                        : kind == LA_KIND_KDA  ? la::kda_mfma_varlen_workspace_bytes(N, H, T_total)
                                               : la::la_mfma_varlen_workspace_bytes(N, H, T_total);
    if (workspace == nullptr || ws_bytes < need) return LA_ERR_WORKSPACE;
    {
        const Span w{workspace, need};
        for (const Span& b : in)
            if (overlaps(w, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (overlaps(w, b)) return LA_ERR_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (form == LA_FORM_CHUNKED && kind == LA_KIND_KDA)
        return from_hip(la::launch_kda_mfma_varlen(N, H, T_total, cu_seqlens, q, k, v, alpha, beta, S0, o, S_out,
                                                   snaps ? snap_interval : 0, snap_count, snaps ? S_snap : nullptr,
                                                   workspace, s));
    if (form == LA_FORM_CHUNKED)
        return from_hip(la::launch_la_mfma_varlen(kind == LA_KIND_GATED, N, H, T_total, cu_seqlens, q, k, v, alpha,
                                                  S0, z0, o, S_out, z_out, snaps ? snap_interval : 0, snap_count,
                                                  snaps ? S_snap : nullptr, snaps && has_z ? z_snap : nullptr,
                                                  workspace, s));
    int* tab = static_cast<int*>(workspace);
    la::Packed pk;
    pk.cu = cu_seqlens;
    pk.snap_base = tab + (N + 1);
    pk.H = H;
    pk.Ttot = T_total;
    pk.snap = snaps ? snap_interval : 0;
    pk.snap_cap = snap_count;
    pk.S_snap = snaps ? S_snap : nullptr;
    pk.z_snap = snaps && has_z ? z_snap : nullptr;
    pk.seq_order = tab + 2 * (N + 1);
    const hipError_t e = la::launch_varlen_table(N, T_total, 1, pk.snap, cu_seqlens, tab, s, nullptr, 0,
                                                 tab + 2 * (N + 1));
    if (e != hipSuccess) return LA_ERR_HIP;
    const int k_kind = kind == LA_KIND_GATED ? la::kGated : kind == LA_KIND_KDA ? la::kKda : la::kNormalized;
    return from_hip(la::launch_recurrent(k_kind, dtype, N * H, T_total, dk, dv, q, k, v, alpha, beta, S0, S_out,
                                         has_z ? z0 : nullptr, has_z ? z_out : nullptr, o, s, pk));
}

la_status kda_prefill(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const float* S0, void* o, float* S_out, int form,
                      int chunk, void* workspace, size_t ws_bytes, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (form != LA_FORM_CHUNKED && form != LA_FORM_RECURRENT) return LA_ERR_ARG;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    if (form == LA_FORM_CHUNKED && !valid_chunk(chunk)) return LA_ERR_SHAPE;
    const size_t heads = static_cast<size_t>(B) * H;
    if (heads == 0) return LA_OK;
    const size_t es = io_size(dtype);
    const size_t nqk = heads * T * dk * es, nv = heads * T * dv * es;
    const size_t na = heads * T * dk * sizeof(float), nb = heads * T * sizeof(float);
    const size_t nS = heads * dv * dk * sizeof(float);
    if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || alpha == nullptr ||
                  beta == nullptr))
        return LA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(alpha),
                          static_cast<const void*>(beta), static_cast<const void*>(S0),
                          static_cast<const void*>(S_out), static_cast<const void*>(workspace)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const Span in[] = {{q, nqk}, {k, nqk}, {v, nv}, {alpha, na}, {beta, nb}, {S0, nS}};
    const Span outs[] = {{o, T > 0 ? nv : 0}, {S_out, nS}};
    for (const Span& a : outs)
        for (const Span& b : in) {
            if (a.p == S_out && b.p == S0 && S_out == S0) continue;
            if (overlaps(a, b)) return LA_ERR_ARG;
        }
    if (overlaps(outs[0], outs[1])) return LA_ERR_ARG;
    if (form == LA_FORM_CHUNKED && !la::kda_mfma_supported(dtype, dk, dv, chunk)) return LA_ERR_UNSUPPORTED;
    const size_t need = form == LA_FORM_CHUNKED ? la::kda_mfma_workspace_bytes(B, H, T) : 0;
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    if (need > 0) {
        const Span w{workspace, need};
        for (const Span& b : in)
            if (overlaps(w, b)) return LA_ERR_ARG;
        for (const Span& b : outs)
            if (overlaps(w, b)) return LA_ERR_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) return copy_state(S0, S_out, heads * dv * dk, s);
    if (form == LA_FORM_CHUNKED)
        return from_hip(la::launch_kda_mfma(B, H, T, q, k, v, alpha, beta, S0, o, S_out, workspace, s));
    return from_hip(la::launch_recurrent(la::kKda, dtype, static_cast<int>(heads), T, dk, dv, q, k, v, alpha, beta,
                                         S0, S_out, nullptr, nullptr, o, s));
}

namespace {

// Shared checks of the two halves of the chunked matrix-core gated-delta path.
la_status gdn_split_common(int dtype, int B, int H, int T, int dk, int dv, int chunk, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, const void* ws, size_t ws_bytes,
                           size_t* heads_out) {
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (!sizes_ok(B, H, T) || !valid_dim(dk) || !valid_dim(dv) || !valid_chunk(chunk)) return LA_ERR_SHAPE;
    if (!la::gdn_mfma_supported(dtype, dk, dv, chunk)) return LA_ERR_UNSUPPORTED;
    *heads_out = static_cast<size_t>(B) * H;
    if (*heads_out == 0 || T == 0) return LA_OK;
    if (q == nullptr || k == nullptr || v == nullptr || alpha == nullptr || beta == nullptr) return LA_ERR_NULL;
    for (const void* p : {q, k, v, static_cast<const void*>(alpha), static_cast<const void*>(beta)})
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const size_t need = la::gdn_mfma_workspace_bytes(B, H, T, dk, dv, chunk);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return LA_ERR_WORKSPACE;
    if (ws != nullptr && !aligned16(ws)) return LA_ERR_ALIGN;
    const size_t nqk = *heads_out * T * dk * 2, nv = *heads_out * T * dv * 2, ng = *heads_out * T * sizeof(float);
    const Span w{ws, need};
    for (const Span& b : {Span{q, nqk}, Span{k, nqk}, Span{v, nv}, Span{alpha, ng}, Span{beta, ng}})
        if (overlaps(w, b)) return LA_ERR_ARG;
    return LA_OK;
}

}  // namespace

la_status gdn_prefill_prep(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, int chunk, void* workspace,
                           size_t ws_bytes, void* stream) {
    size_t heads = 0;
    const la_status st =
        gdn_split_common(dtype, B, H, T, dk, dv, chunk, q, k, v, alpha, beta, workspace, ws_bytes, &heads);
    if (st != LA_OK || heads == 0 || T == 0) return st;
    return from_hip(la::launch_gdn_mfma_prep(B, H, T, q, k, v, alpha, beta, workspace,
                                             static_cast<hipStream_t>(stream)));
}

la_status gdn_prefill_scan(int dtype, int B, int H, int T, int dk, int dv, const void* q, const void* k,
                           const void* v, const float* alpha, const float* beta, const float* S0, void* o,
                           float* S_out, int chunk, void* workspace, size_t ws_bytes, void* stream) {
    size_t heads = 0;
    const la_status st =
        gdn_split_common(dtype, B, H, T, dk, dv, chunk, q, k, v, alpha, beta, workspace, ws_bytes, &heads);
    if (st != LA_OK || heads == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (S0 != nullptr && !aligned16(S0)) return LA_ERR_ALIGN;
        if (S_out != nullptr && !aligned16(S_out)) return LA_ERR_ALIGN;
        return copy_state(S0, S_out, heads * dv * dk, s);
    }
    if (o == nullptr) return LA_ERR_NULL;
    for (const void* p : {static_cast<const void*>(o), static_cast<const void*>(S0), static_cast<const void*>(S_out)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const size_t nqk = heads * T * dk * 2, nv = heads * T * dv * 2, ng = heads * T * sizeof(float);
    const size_t nS = heads * dv * dk * sizeof(float);
    const Span ws{workspace, la::gdn_mfma_workspace_bytes(B, H, T, dk, dv, chunk)};
    const Span outs[] = {{o, nv}, {S_out, nS}};
    for (const Span& a : outs) {
        for (const Span& b : {Span{q, nqk}, Span{k, nqk}, Span{v, nv}, Span{alpha, ng}, Span{beta, ng}, ws})
            if (overlaps(a, b)) return LA_ERR_ARG;
        if (!(a.p == S_out && S_out == S0) && overlaps(a, Span{S0, nS})) return LA_ERR_ARG;
    }
    if (overlaps(outs[0], outs[1])) return LA_ERR_ARG;
    if (overlaps(ws, Span{S0, nS})) return LA_ERR_ARG;
    return from_hip(la::launch_gdn_mfma_scan(B, H, T, q, k, v, alpha, beta, S0, o, S_out, workspace, s));
}

la_status lin_attn_decode_step(int kind, int dtype, int N, int H, int dk, int dv, const void* q,
                               const void* k, const void* v, const float* alpha, const float* beta,
                               float* S, float* z, void* o, void* stream) {
    if (kind != LA_KIND_NORMALIZED && kind != LA_KIND_GATED_DELTA && kind != LA_KIND_GATED && kind != LA_KIND_KDA)
        return LA_ERR_ARG;
    if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_DTYPE;
    if (!sizes_ok(N, H, 1) || !valid_dim(dk) || !valid_dim(dv)) return LA_ERR_SHAPE;
    const size_t heads = static_cast<size_t>(N) * H;
    if (heads == 0) return LA_OK;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || S == nullptr) return LA_ERR_NULL;
    if (kind == LA_KIND_GATED_DELTA || kind == LA_KIND_KDA) {
        if (alpha == nullptr || beta == nullptr) return LA_ERR_NULL;
        if (z != nullptr) return LA_ERR_ARG;
    } else if (kind == LA_KIND_GATED) {
        if (alpha == nullptr) return LA_ERR_NULL;
        if (beta != nullptr || z != nullptr) return LA_ERR_ARG;
    } else {
        if (z == nullptr) return LA_ERR_NULL;
        if (alpha != nullptr || beta != nullptr) return LA_ERR_ARG;
    }
    for (const void* p : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(alpha),
                          static_cast<const void*>(beta), static_cast<const void*>(S),
                          static_cast<const void*>(z)})
        if (p != nullptr && !aligned16(p)) return LA_ERR_ALIGN;
    const size_t es = io_size(dtype);
    const Span outs[] = {{o, heads * dv * es}, {S, heads * dv * dk * sizeof(float)}, {z, heads * dk * sizeof(float)}};
    const Span in[] = {{q, heads * dk * es}, {k, heads * dk * es}, {v, heads * dv * es},
                       {alpha, heads * (kind == LA_KIND_KDA ? dk : 1) * sizeof(float)}, {beta, heads * sizeof(float)}};
    for (const Span& a : outs)
        for (const Span& b : in)
            if (overlaps(a, b)) return LA_ERR_ARG;
    if (overlaps(outs[0], outs[1]) || overlaps(outs[0], outs[2]) || overlaps(outs[1], outs[2])) return LA_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int k_kind = kind == LA_KIND_GATED_DELTA ? la::kGatedDelta
                       : kind == LA_KIND_GATED ? la::kGated
                       : kind == LA_KIND_KDA   ? la::kKda
                                               : la::kNormalized;
    return from_hip(la::launch_recurrent(k_kind, dtype, static_cast<int>(heads), 1, dk, dv, q, k, v, alpha,
                                         beta, S, S, z, z, o, s));
}

}  // extern "C"

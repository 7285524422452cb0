// Chunked forms in plain fp32 arithmetic on the vector ALUs.
//
// These kernels evaluate the chunked forms exactly as written, with every
// product in fp32, for shapes the bf16 matrix-core kernels do not cover
// (fp32 activations, small head dims, other chunk lengths).  One block per
// head walks the chunks in order; the carried state and the current chunk
// live in LDS.
//
// Linear attention (page "Linear attention and hybrids", section "Three forms
// of one computation", chunk equation; block flowchart):
//   A = tril(phi(Q_b) phi(K_b)^T); num = A V_b + phi(Q_b) S^T;
//   den = rowsum(A) + phi(Q_b) z; O_b = num / den; S += V_b^T phi(K_b);
//   z += colsum phi(K_b).
// Gated delta rule (same page, section "Delta rule and Gated DeltaNet",
// Gated DeltaNet equation), chunkwise by unrolling the recurrence inside a
// chunk of c tokens with entry state S: g = cumsum(log alpha) (chunk-local),
// Gamma_ij = exp(g_i - g_j);
//   L_ij = beta_i Gamma_ij k_i.k_j (j < i);  (I + L) [W | Ut] =
//   [diag(beta e^g) K | diag(beta) V] solved by forward substitution;
//   U = Ut - W S^T;  A = (Q K^T) * Gamma, lower triangle with diagonal;
//   O = diag(e^g) Q S^T + A U;  S <- e^{g_c} S + U^T diag(e^{g_c - g}) K.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int kThreads = 256;

template <class IO>
__global__ __launch_bounds__(kThreads) void la_chunked_generic_kernel(
    int T, int DK, int DV, int C, const typename IO::T* __restrict__ q,
    const typename IO::T* __restrict__ k, const typename IO::T* __restrict__ v, const float* S0,
    const float* z0, typename IO::T* __restrict__ o, float* S_out, float* z_out) {
    extern __shared__ float lds[];
    float* S = lds;                 // [DV][DK]
    float* z = S + DV * DK;         // [DK]
    float* fq = z + DK;             // [C][DK]
    float* fk = fq + C * DK;        // [C][DK]
    float* vv = fk + C * DK;        // [C][DV]
    float* A = vv + C * DV;         // [C][C]
    float* den = A + C * C;         // [C]
    const int head = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t hs = static_cast<size_t>(head) * DV * DK;
    for (int e = tid; e < DV * DK; e += kThreads) S[e] = S0 ? S0[hs + e] : 0.f;
    for (int e = tid; e < DK; e += kThreads) z[e] = z0 ? z0[static_cast<size_t>(head) * DK + e] : 0.f;

    for (int a = 0; a < T; a += C) {
        const int c = min(C, T - a);
        const size_t tk = (static_cast<size_t>(head) * T + a) * DK;
        const size_t tv = (static_cast<size_t>(head) * T + a) * DV;
        __syncthreads();
        for (int e = tid; e < c * DK; e += kThreads) {
            fq[e] = phi(IO::load(q, tk + e));
            fk[e] = phi(IO::load(k, tk + e));
        }
        for (int e = tid; e < c * DV; e += kThreads) vv[e] = IO::load(v, tv + e);
        __syncthreads();
        for (int e = tid; e < c * c; e += kThreads) {
            const int i = e / c, j = e % c;
            float acc = 0.f;
            if (j <= i)
                for (int p = 0; p < DK; ++p) acc = fmaf(fq[i * DK + p], fk[j * DK + p], acc);
            A[i * C + j] = acc;
        }
        __syncthreads();
        for (int i = tid; i < c; i += kThreads) {
            float acc = 0.f;
            for (int j = 0; j <= i; ++j) acc += A[i * C + j];
            for (int p = 0; p < DK; ++p) acc = fmaf(fq[i * DK + p], z[p], acc);
            den[i] = acc;
        }
        __syncthreads();
        for (int e = tid; e < c * DV; e += kThreads) {
            const int i = e / DV, r = e % DV;
            float acc = 0.f;
            for (int j = 0; j <= i; ++j) acc = fmaf(A[i * C + j], vv[j * DV + r], acc);
            for (int p = 0; p < DK; ++p) acc = fmaf(fq[i * DK + p], S[r * DK + p], acc);
            IO::store(o, tv + e, acc / den[i]);
        }
        __syncthreads();
        for (int e = tid; e < DV * DK; e += kThreads) {
            const int r = e / DK, p = e % DK;
            float acc = S[e];
            for (int j = 0; j < c; ++j) acc = fmaf(vv[j * DV + r], fk[j * DK + p], acc);
            S[e] = acc;
        }
        for (int p = tid; p < DK; p += kThreads) {
            float acc = z[p];
            for (int j = 0; j < c; ++j) acc += fk[j * DK + p];
            z[p] = acc;
        }
    }
    __syncthreads();
    if (S_out)
        for (int e = tid; e < DV * DK; e += kThreads) S_out[hs + e] = S[e];
    if (z_out)
        for (int e = tid; e < DK; e += kThreads) z_out[static_cast<size_t>(head) * DK + e] = z[e];
}

template <class IO>
__global__ __launch_bounds__(kThreads) void gdn_chunked_generic_kernel(
    int T, int DK, int DV, int C, const typename IO::T* __restrict__ q,
    const typename IO::T* __restrict__ k, const typename IO::T* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, const float* S0,
    typename IO::T* __restrict__ o, float* S_out) {
    extern __shared__ float lds[];
    float* S = lds;               // [DV][DK]
    float* Qs = S + DV * DK;      // [C][DK]
    float* Ks = Qs + C * DK;      // [C][DK]
    float* W = Ks + C * DK;       // [C][DK]
    float* U = W + C * DK;        // [C][DV]  (holds V, then Ut, then U)
    float* L = U + C * DV;        // [C][C]   (L, then the decay-masked Q K^T)
    float* g = L + C * C;         // [C]
    float* bt = g + C;            // [C]
    const int head = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t hs = static_cast<size_t>(head) * DV * DK;
    for (int e = tid; e < DV * DK; e += kThreads) S[e] = S0 ? S0[hs + e] : 0.f;

    for (int a = 0; a < T; a += C) {
        const int c = min(C, T - a);
        const size_t tk = (static_cast<size_t>(head) * T + a) * DK;
        const size_t tv = (static_cast<size_t>(head) * T + a) * DV;
        const size_t tg = static_cast<size_t>(head) * T + a;
        __syncthreads();
        for (int e = tid; e < c * DK; e += kThreads) {
            Qs[e] = IO::load(q, tk + e);
            Ks[e] = IO::load(k, tk + e);
        }
        for (int e = tid; e < c * DV; e += kThreads) U[e] = IO::load(v, tv + e);
        if (tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < c; ++i) {
                acc += __logf(alpha[tg + i]);
                g[i] = acc;
                bt[i] = beta[tg + i];
            }
        }
        __syncthreads();
        // L (strictly lower) and the right-hand sides diag(beta e^g) K, diag(beta) V
        for (int e = tid; e < c * c; e += kThreads) {
            const int i = e / c, j = e % c;
            float acc = 0.f;
            if (j < i) {
                for (int p = 0; p < DK; ++p) acc = fmaf(Ks[i * DK + p], Ks[j * DK + p], acc);
                acc *= bt[i] * __expf(g[i] - g[j]);
            }
            L[i * C + j] = acc;
        }
        for (int e = tid; e < c * DK; e += kThreads) W[e] = bt[e / DK] * __expf(g[e / DK]) * Ks[e];
        for (int e = tid; e < c * DV; e += kThreads) U[e] *= bt[e / DV];
        __syncthreads();
        // forward substitution, one right-hand-side column per thread
        for (int col = tid; col < DK + DV; col += kThreads) {
            float* X = col < DK ? W + col : U + (col - DK);
            const int ld = col < DK ? DK : DV;
            for (int i = 1; i < c; ++i) {
                float acc = X[i * ld];
                for (int j = 0; j < i; ++j) acc = fmaf(-L[i * C + j], X[j * ld], acc);
                X[i * ld] = acc;
            }
        }
        __syncthreads();
        // U = Ut - W S^T ; decay-masked Q K^T into L
        for (int e = tid; e < c * DV; e += kThreads) {
            const int i = e / DV, r = e % DV;
            float acc = U[e];
            for (int p = 0; p < DK; ++p) acc = fmaf(-W[i * DK + p], S[r * DK + p], acc);
            U[e] = acc;
        }
        for (int e = tid; e < c * c; e += kThreads) {
            const int i = e / c, j = e % c;
            float acc = 0.f;
            if (j <= i) {
                for (int p = 0; p < DK; ++p) acc = fmaf(Qs[i * DK + p], Ks[j * DK + p], acc);
                acc *= __expf(g[i] - g[j]);
            }
            L[i * C + j] = acc;
        }
        __syncthreads();
        // O = diag(e^g) Q S^T + A U
        for (int e = tid; e < c * DV; e += kThreads) {
            const int i = e / DV, r = e % DV;
            float qs = 0.f;
            for (int p = 0; p < DK; ++p) qs = fmaf(Qs[i * DK + p], S[r * DK + p], qs);
            float acc = __expf(g[i]) * qs;
            for (int j = 0; j <= i; ++j) acc = fmaf(L[i * C + j], U[j * DV + r], acc);
            IO::store(o, tv + e, acc);
        }
        __syncthreads();
        // S <- e^{g_c} S + U^T diag(e^{g_c - g}) K
        const float gc = g[c - 1];
        for (int e = tid; e < DV * DK; e += kThreads) {
            const int r = e / DK, p = e % DK;
            float acc = __expf(gc) * S[e];
            for (int j = 0; j < c; ++j) acc = fmaf(U[j * DV + r] * __expf(gc - g[j]), Ks[j * DK + p], acc);
            S[e] = acc;
        }
    }
    __syncthreads();
    if (S_out)
        for (int e = tid; e < DV * DK; e += kThreads) S_out[hs + e] = S[e];
}

}  // namespace

size_t la_chunked_generic_lds_bytes(int dk, int dv, int chunk) {
    return sizeof(float) * (static_cast<size_t>(dv) * dk + dk + 2 * chunk * dk + chunk * dv +
                            chunk * chunk + chunk);
}

size_t gdn_chunked_generic_lds_bytes(int dk, int dv, int chunk) {
    return sizeof(float) * (static_cast<size_t>(dv) * dk + 3 * chunk * dk + chunk * dv +
                            chunk * chunk + 2 * chunk);
}

hipError_t launch_la_chunked_generic(int dtype, int heads, int T, int dk, int dv, int chunk,
                                     const void* q, const void* k, const void* v, const float* S0,
                                     const float* z0, void* o, float* S_out, float* z_out,
                                     hipStream_t stream) {
    if (heads <= 0) return hipSuccess;
    if (!grid_fits(heads, kThreads)) return hipErrorInvalidConfiguration;
    const size_t lds = la_chunked_generic_lds_bytes(dk, dv, chunk);
    if (dtype == kBF16) {
        auto kern = la_chunked_generic_kernel<IoBF16>;
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(heads), dim3(kThreads), lds, stream, T, dk, dv, chunk,
                           static_cast<const u16*>(q), static_cast<const u16*>(k),
                           static_cast<const u16*>(v), S0, z0, static_cast<u16*>(o), S_out, z_out);
    } else {
        auto kern = la_chunked_generic_kernel<IoF32>;
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(heads), dim3(kThreads), lds, stream, T, dk, dv, chunk,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), S0, z0, static_cast<float*>(o), S_out, z_out);
    }
    return hipGetLastError();
}

hipError_t launch_gdn_chunked_generic(int dtype, int heads, int T, int dk, int dv, int chunk,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta, const float* S0,
                                      void* o, float* S_out, hipStream_t stream) {
    if (heads <= 0) return hipSuccess;
    if (!grid_fits(heads, kThreads)) return hipErrorInvalidConfiguration;
    const size_t lds = gdn_chunked_generic_lds_bytes(dk, dv, chunk);
    if (dtype == kBF16) {
        auto kern = gdn_chunked_generic_kernel<IoBF16>;
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(heads), dim3(kThreads), lds, stream, T, dk, dv, chunk,
                           static_cast<const u16*>(q), static_cast<const u16*>(k),
                           static_cast<const u16*>(v), alpha, beta, S0, static_cast<u16*>(o), S_out);
    } else {
        auto kern = gdn_chunked_generic_kernel<IoF32>;
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(heads), dim3(kThreads), lds, stream, T, dk, dv, chunk,
                           static_cast<const float*>(q), static_cast<const float*>(k),
                           static_cast<const float*>(v), alpha, beta, S0, static_cast<float*>(o), S_out);
    }
    return hipGetLastError();
}

}  // namespace la

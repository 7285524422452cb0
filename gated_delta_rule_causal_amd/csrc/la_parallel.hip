// Normalised causal linear attention, masked parallel form, fp32 arithmetic.
//
// Page "Linear attention and hybrids", section "Three forms of one
// computation", form 1: A = phi(Q) phi(K)^T with future keys masked out,
// each output row is (A_i V) / sum(A_i).  Cost grows with T^2, so this form
// is for short sequences.
//
// Grid: (heads, ceil(T / 64)).  Block: 256 threads = 64 query rows x 4 groups
// of value columns.  Key/value tiles of 64 tokens are staged in LDS with phi
// already applied; each thread keeps phi(q_i) in registers.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int kRows = 64;

template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void la_parallel_kernel(int T, const typename IO::T* __restrict__ q,
                                                          const typename IO::T* __restrict__ k,
                                                          const typename IO::T* __restrict__ v,
                                                          typename IO::T* __restrict__ o) {
    constexpr int CG = DV / 4;  // value columns per thread
    __shared__ float fk_s[kRows][DK + 1];
    __shared__ float v_s[kRows][DV + 1];
    const int head = blockIdx.x;
    const int qi = threadIdx.x % kRows;
    const int cg = threadIdx.x / kRows;
    const int i = blockIdx.y * kRows + qi;
    const size_t hk = static_cast<size_t>(head) * T * DK;
    const size_t hv = static_cast<size_t>(head) * T * DV;

    float fq[DK];
#pragma unroll
    for (int p = 0; p < DK; ++p) fq[p] = i < T ? phi(IO::load(q, hk + static_cast<size_t>(i) * DK + p)) : 0.f;
    float num[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) num[c] = 0.f;
    float den = 0.f;

    const int last_tile = blockIdx.y;  // key tiles after the query tile are fully masked
    for (int jt = 0; jt <= last_tile; ++jt) {
        __syncthreads();
        for (int e = threadIdx.x; e < kRows * DK; e += blockDim.x) {
            const int jj = e / DK, p = e % DK, j = jt * kRows + jj;
            fk_s[jj][p] = j < T ? phi(IO::load(k, hk + static_cast<size_t>(j) * DK + p)) : 0.f;
        }
        for (int e = threadIdx.x; e < kRows * DV; e += blockDim.x) {
            const int jj = e / DV, c = e % DV, j = jt * kRows + jj;
            v_s[jj][c] = j < T ? IO::load(v, hv + static_cast<size_t>(j) * DV + c) : 0.f;
        }
        __syncthreads();
        const int jmax = min(kRows, i - jt * kRows + 1);  // keys j <= i only
        for (int jj = 0; jj < jmax; ++jj) {
            float a = 0.f;
#pragma unroll
            for (int p = 0; p < DK; ++p) a = fmaf(fq[p], fk_s[jj][p], a);
            den += a;
#pragma unroll
            for (int c = 0; c < CG; ++c) num[c] = fmaf(a, v_s[jj][cg * CG + c], num[c]);
        }
    }
    if (i < T) {
        const float rden = 1.f / den;
#pragma unroll
        for (int c = 0; c < CG; ++c) IO::store(o, hv + static_cast<size_t>(i) * DV + cg * CG + c, num[c] * rden);
    }
}

// Final state of the whole sequence: S = sum_t v_t phi(k_t)^T, z = sum_t phi(k_t)
// (the sums S_i, z_i of the kernel-trick equation at i = T).  Block per
// (head, row); threads over the dk columns.
template <class IO>
__global__ __launch_bounds__(128) void la_final_state_kernel(int T, int DK, int DV,
                                                             const typename IO::T* __restrict__ k,
                                                             const typename IO::T* __restrict__ v,
                                                             float* S_out, float* z_out) {
    const int head = blockIdx.x;
    const int r = blockIdx.y;  // r == DV is the normaliser row
    const int p = threadIdx.x;
    if (p >= DK) return;
    const size_t hk = static_cast<size_t>(head) * T * DK;
    const size_t hv = static_cast<size_t>(head) * T * DV;
    float acc = 0.f;
    for (int t = 0; t < T; ++t) {
        const float f = phi(IO::load(k, hk + static_cast<size_t>(t) * DK + p));
        acc = r < DV ? fmaf(IO::load(v, hv + static_cast<size_t>(t) * DV + r), f, acc) : acc + f;
    }
    if (r < DV) {
        if (S_out) S_out[(static_cast<size_t>(head) * DV + r) * DK + p] = acc;
    } else if (z_out) {
        z_out[static_cast<size_t>(head) * DK + p] = acc;
    }
}

template <class IO, int DK, int DV>
hipError_t launch_shape(int heads, int T, const void* q, const void* k, const void* v, void* o,
                        hipStream_t stream) {
    using E = typename IO::T;
    dim3 grid(heads, (T + kRows - 1) / kRows), block(256);
    hipLaunchKernelGGL((la_parallel_kernel<IO, DK, DV>), grid, block, 0, stream, T,
                       static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v),
                       static_cast<E*>(o));
    return hipGetLastError();
}

template <class IO, int DK>
hipError_t launch_dv(int heads, int T, int dv, const void* q, const void* k, const void* v, void* o,
                     hipStream_t stream) {
    switch (dv) {
        case 16: return launch_shape<IO, DK, 16>(heads, T, q, k, v, o, stream);
        case 32: return launch_shape<IO, DK, 32>(heads, T, q, k, v, o, stream);
        case 64: return launch_shape<IO, DK, 64>(heads, T, q, k, v, o, stream);
        case 128: return launch_shape<IO, DK, 128>(heads, T, q, k, v, o, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class IO>
hipError_t launch_io(int heads, int T, int dk, int dv, const void* q, const void* k, const void* v,
                     void* o, float* S_out, float* z_out, hipStream_t stream) {
    if (!grid_fits(heads, 256)) return hipErrorInvalidConfiguration;   // both kernels: x = heads
    hipError_t e;
    switch (dk) {
        case 16: e = launch_dv<IO, 16>(heads, T, dv, q, k, v, o, stream); break;
        case 32: e = launch_dv<IO, 32>(heads, T, dv, q, k, v, o, stream); break;
        case 64: e = launch_dv<IO, 64>(heads, T, dv, q, k, v, o, stream); break;
        case 128: e = launch_dv<IO, 128>(heads, T, dv, q, k, v, o, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (S_out != nullptr || z_out != nullptr) {
        using E = typename IO::T;
        dim3 grid(heads, dv + 1), block(128);
        hipLaunchKernelGGL(la_final_state_kernel<IO>, grid, block, 0, stream, T, dk, dv,
                           static_cast<const E*>(k), static_cast<const E*>(v), S_out, z_out);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_la_parallel(int dtype, int heads, int T, int dk, int dv, const void* q,
                              const void* k, const void* v, void* o, float* S_out, float* z_out,
                              hipStream_t stream) {
    if (heads <= 0 || T <= 0) return hipSuccess;
    return dtype == kBF16 ? launch_io<IoBF16>(heads, T, dk, dv, q, k, v, o, S_out, z_out, stream)
                          : launch_io<IoF32>(heads, T, dk, dv, q, k, v, o, S_out, z_out, stream);
}

}  // namespace la

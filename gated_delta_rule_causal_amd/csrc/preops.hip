// Pre-operations in front of a Gated DeltaNet layer, fused into one pass:
// kernel-4 causal depthwise convolution over time, per-head L2 normalisation
// of q and k, sigmoid gates, and the change of layout from token-major
// projections [B, T, channels] to the head-major rows [B, H, T, d] the
// prefill kernels read.
//
// Source: page "Linear attention and hybrids", section "2025 hybrids:
// Qwen3-Next and Kimi Linear" (a short causal depthwise convolution over time
// with kernel 4 before q, k and v), section "Memory must forget: decay and
// gates" (the gate is a sigmoid of the input).  Per channel c and token t:
//     y_t[c] = sum_{i<4} w[c][i] x_{t-3+i}[c]
// with the three tokens before the first taken from a carried state (zeros
// without one); q and k are then divided by their per-head Euclidean norm;
// alpha = sigma(a_logit), beta = sigma(b_logit).
//
// Work split: one workgroup per (sequence, head, tile of 128 tokens), 256
// threads, which produce the tile's q, then k, then v rows.  For one part
// (D channels) a lane owns 8 consecutive channels and TPL consecutive tokens
// (D/8 lanes per token row): it loads its channels of the TPL + 3 rows its
// outputs need (its tokens and the three before them: the previous tile, the
// carried state, or zeros) with 16-byte loads, all issued before the first
// is used, then convolves, normalises (the D/8 lanes of a q or k row are an
// aligned lane group and reduce its sum of squares with xor shuffles) and
// writes each output row piece with one 16-byte nontemporal store (nothing
// here reads the outputs back).  The heads of one tile are neighbours in the
// launch order, so the workgroups in flight read whole projection rows
// between them.  HBM traffic: one read of the projections (the three history
// rows of a tile come from the caches) and one write of the head-major
// tensors.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int kTile = 128;
constexpr int kThreads = 256;

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// 8 consecutive elements of one input row, as loaded (16-byte aligned).
template <class E>
struct Raw;
template <>
struct Raw<u16> {
    uint4 u;
    __device__ __forceinline__ void load(const u16* p) { u = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void get(float* x) const {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <>
struct Raw<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const float4*>(p)[0];
        b = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ __forceinline__ void get(float* x) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
};

__device__ __forceinline__ void nt_store16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4v v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4v*>(p));
}
__device__ __forceinline__ void store8(float* p, const float* x) {
    nt_store16(p, __float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
    nt_store16(p + 4, __float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7]));
}
__device__ __forceinline__ void store8(u16* p, const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i])) |
               (static_cast<uint32_t>(f32_to_bf16_bits(x[2 * i + 1])) << 16);
    nt_store16(p, w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// One part of the tile: the head's D channels starting at channel cbase of
// the projection, written to dst = the head's rows [T, D].  With NORM every
// output row is divided by its Euclidean norm (a zero row stays zero).
// Called by every thread of the workgroup with len > 0 (the xor reductions
// need whole waves).
// Packed batch: sequence n is tokens cu[n] .. cu[n+1] of the projections
// (one sequence axis, B = 1); a tap before its sequence's first token reads
// row 3 + (tap - start) of that sequence's carried state st[n] ([3][C]), or
// zero when there is none.  cu == nullptr: the uniform layout.
template <class E>
struct Seqs {
    const int* cu;
    int N;
    const E* st;
};

// The window of one part: this lane's channels of the TPL + 3 rows its outputs
// need, and the kernel weights of those channels.  conv_load issues every load
// (a row the outputs do not need reads row t0, which exists, so no load sits
// in a branch); conv_store convolves, normalises and stores.
template <int D, class E>
struct Window {
    static constexpr int L = D / 8;                                          // lanes per token row
    static constexpr int TPL = kTile * L / kThreads >= 1 ? kTile * L / kThreads : 1;   // tokens per lane
    static constexpr int NL = kTile / TPL * L;                               // lanes in use
    static_assert(NL <= kThreads && NL % kWave == 0, "lane layout");
    Raw<E> raw[TPL + 3];
    float4 w[8];
};

template <int D, class E>
__device__ __forceinline__ void conv_load(Window<D, E>& win, const E* __restrict__ xb, const E* st,
                                          const float* __restrict__ w, int C, int cbase, int t0, int len, int tid) {
    using W = Window<D, E>;
    if (tid >= W::NL) return;                                         // whole waves
    const int m = tid % W::L;
    const int jb = (tid / W::L) * W::TPL;                             // first token of this lane in the tile
    const int c0 = cbase + 8 * m;
#pragma unroll
    for (int e = 0; e < 8; ++e) win.w[e] = *reinterpret_cast<const float4*>(w + static_cast<size_t>(c0 + e) * 4);
    // window rows r = 0 .. TPL + 2 hold token t0 + jb - 3 + r
#pragma unroll
    for (int r = 0; r < W::TPL + 3; ++r) {
        const int ts = t0 + jb - 3 + r;                               // >= -3
        const bool in_tile = jb + r - 3 < len;                        // later rows feed no stored output
        const bool from_state = in_tile && ts < 0 && st != nullptr;
        const int row = in_tile && ts >= 0 ? ts : t0;
        const E* src = from_state ? st + static_cast<size_t>(3 + ts) * C : xb + static_cast<size_t>(row) * C;
        win.raw[r].load(src + c0);
    }
    // keep the scheduler from unpacking the first rows (and so waiting for
    // them) before every load above has been issued
    __builtin_amdgcn_sched_barrier(0);
}

// One part of the tile: the head's D channels starting at channel cbase of
// the projection, written to dst = the head's rows [T, D].  With NORM every
// output row is divided by its Euclidean norm (a zero row stays zero).
// Called by every thread of the workgroup with len > 0 (the xor reductions
// need whole waves).  PACKED: the packed-batch layout of Seqs.
template <int D, bool NORM, bool PACKED, class E>
__device__ __forceinline__ void conv_store(const Window<D, E>& win, const E* st, int C, int cbase, int t0, int len,
                                           int T, E* __restrict__ dst, int tid, const Seqs<E>& sq) {
    using W = Window<D, E>;
    if (tid >= W::NL) return;                                         // whole waves
    const int m = tid % W::L;
    const int jb = (tid / W::L) * W::TPL;
    const int c0 = cbase + 8 * m;
    float wv[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        wv[e][0] = win.w[e].x; wv[e][1] = win.w[e].y; wv[e][2] = win.w[e].z; wv[e][3] = win.w[e].w;
    }
    float xr[W::TPL + 3][8];
#pragma unroll
    for (int r = 0; r < W::TPL + 3; ++r) {
        win.raw[r].get(xr[r]);
        // before the first token, without a carried state: zeros
        const bool live = t0 + jb - 3 + r >= 0 || st != nullptr;
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[r][e] = live ? xr[r][e] : 0.f;
    }
    // packed batch: the sequence of this lane's first token (binary search)
    int n = 0;
    if constexpr (PACKED) {
        const int tf = t0 + jb;
        int lo = 0, hi = sq.N;   // the last n with cu[n] <= tf
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sq.cu[mid] <= tf) lo = mid; else hi = mid;
        }
        n = lo;
    }
#pragma unroll
    for (int s = 0; s < W::TPL; ++s) {
        float tap[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) tap[i][e] = xr[s + i][e];
        if constexpr (PACKED) {
            const int t = t0 + jb + s;
            while (n + 1 < sq.N && sq.cu[n + 1] <= t) ++n;
            const int d = max(0, t - min(max(sq.cu[n], 0), T));   // position inside its sequence
            if (d < 3) {   // taps before the sequence start: its carried state (or zero)
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    if (i < 3 - d) {
                        if (sq.st != nullptr) {
                            Raw<E> rs;
                            rs.load(sq.st + (static_cast<size_t>(n) * 3 + d + i) * C + c0);
                            rs.get(tap[i]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) tap[i][e] = 0.f;
                        }
                    }
                }
            }
        }
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = wv[e][0] * tap[0][e];
            acc = fmaf(wv[e][1], tap[1][e], acc);
            acc = fmaf(wv[e][2], tap[2][e], acc);
            y[e] = fmaf(wv[e][3], tap[3][e], acc);
        }
        if constexpr (NORM) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
            ss = group_sum<W::L>(ss);
            const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= inv;
        }
        const int j = jb + s;
        if (j < len) store8(dst + static_cast<size_t>(t0 + j) * D + 8 * m, y);
    }
}

template <class IO, int DK, int DV, bool PACKED>
__global__ __launch_bounds__(kThreads) void gdn_preprocess_kernel(
    int T, int H, int tiles, const int* cu, int N, const typename IO::T* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ a_logit, const float* __restrict__ b_logit, const typename IO::T* st_in,
    typename IO::T* st_out, typename IO::T* __restrict__ q, typename IO::T* __restrict__ k,
    typename IO::T* __restrict__ v, float* __restrict__ alpha, float* __restrict__ beta) {
    using E = typename IO::T;
    const int C = H * (2 * DK + DV);
    // the three parts (q, k, v) of a (tile, head) are neighbouring workgroups,
    // and the heads of a tile follow each other
    const int part = blockIdx.x % 3;
    const int rest = blockIdx.x / 3;
    const int h = rest % H;
    const int tile = (rest / H) % tiles;
    const int b = rest / (H * tiles);
    const int t0 = tile * kTile;
    const int len = max(0, min(kTile, T - t0));
    const E* xb = x + static_cast<size_t>(b) * T * C;
    // packed batch: one sequence axis; states are per sequence and handled in conv_part
    const Seqs<E> sq{cu, N, cu ? st_in : nullptr};
    const E* st = (st_in && !cu) ? st_in + static_cast<size_t>(b) * 3 * C : nullptr;
    const size_t row0 = (static_cast<size_t>(b) * H + h) * T;   // row (b, h, t = 0) of the outputs
    const int tid = threadIdx.x;

    if (len > 0) {   // (T == 0: only the state below)
        // one part per workgroup: a workgroup's window loads never wait
        // behind its own stores of another part (loads and stores share one
        // counter), and the parts of neighbouring workgroups overlap
        if (part == 0) {
            Window<DK, E> wq;
            conv_load<DK>(wq, xb, st, w, C, h * DK, t0, len, tid);
            conv_store<DK, true, PACKED>(wq, st, C, h * DK, t0, len, T, q + row0 * DK, tid, sq);
            for (int j = tid; j < len; j += kThreads) {
                const size_t li = (static_cast<size_t>(b) * T + t0 + j) * H + h;
                alpha[row0 + t0 + j] = sigmoid(a_logit[li]);
                beta[row0 + t0 + j] = sigmoid(b_logit[li]);
            }
        } else if (part == 1) {
            Window<DK, E> wk;
            conv_load<DK>(wk, xb, st, w, C, H * DK + h * DK, t0, len, tid);
            conv_store<DK, true, PACKED>(wk, st, C, H * DK + h * DK, t0, len, T, k + row0 * DK, tid, sq);
        } else {
            Window<DV, E> wv;
            conv_load<DV>(wv, xb, st, w, C, 2 * H * DK + h * DV, t0, len, tid);
            conv_store<DV, false, PACKED>(wv, st, C, 2 * H * DK + h * DV, t0, len, T, v + row0 * DV, tid, sq);
        }
    }
    // carried state: the last three tokens of [state; x], this head's channels
    // (packed batches: written per sequence by gdn_state_out_kernel)
    if (st_out != nullptr && cu == nullptr && tile == tiles - 1) {
        // this part's channels
        const int nch = part == 2 ? DV : DK;
        const int cb = part == 0 ? h * DK : part == 1 ? H * DK + h * DK : 2 * H * DK + h * DV;
        for (int e = tid; e < 3 * nch; e += kThreads) {
            const int r = e / nch, c = cb + e % nch;
            const int ts = T - 3 + r;
            float val = 0.f;
            if (ts >= 0)
                val = IO::load(xb, static_cast<size_t>(ts) * C + c);
            else if (st != nullptr)
                val = IO::load(st, static_cast<size_t>(3 + ts) * C + c);
            IO::store(st_out + static_cast<size_t>(b) * 3 * C, static_cast<size_t>(r) * C + c, val);
        }
    }
}

// Packed batch: the next conv state of every sequence, the last three
// tokens of [state; its tokens].
template <class IO>
__global__ __launch_bounds__(256) void gdn_state_out_kernel(int N, int T, int C, const int* cu,
                                                            const typename IO::T* __restrict__ x,
                                                            const typename IO::T* st_in, typename IO::T* st_out) {
    const size_t total = static_cast<size_t>(N) * 3 * C;
    for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < total;
         e += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int c = static_cast<int>(e % C);
        const int j = static_cast<int>((e / C) % 3);
        const int n = static_cast<int>(e / (static_cast<size_t>(3) * C));
        const int s0 = min(max(cu[n], 0), T), e1 = max(min(max(cu[n + 1], 0), T), s0);
        const int src = e1 - 3 + j;
        float val = 0.f;
        if (src >= s0)
            val = IO::load(x, static_cast<size_t>(src) * C + c);
        else if (st_in != nullptr)
            val = IO::load(st_in, (static_cast<size_t>(n) * 3 + 3 + (src - s0)) * C + c);
        IO::store(st_out, e, val);
    }
}

template <class IO, int DK>
hipError_t launch_dv(int B, int T, int H, int dv, const int* cu, int N, const void* x, const float* w,
                     const float* al, const float* bl, const void* st_in, void* st_out, void* q, void* k, void* v,
                     float* alpha, float* beta, hipStream_t stream) {
    using E = typename IO::T;
    const int tiles = T > 0 ? (T + kTile - 1) / kTile : 1;   // T == 0: one workgroup per head writes the state
    const long long blocks = static_cast<long long>(B) * H * tiles * 3;
    if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, T, H, tiles, cu, N, static_cast<const E*>(x), w, al, bl,
                           static_cast<const E*>(st_in), static_cast<E*>(st_out), static_cast<E*>(q),
                           static_cast<E*>(k), static_cast<E*>(v), alpha, beta);
        return hipGetLastError();
    };
    const bool packed = cu != nullptr;
    switch (dv) {
        case 16: return packed ? go(gdn_preprocess_kernel<IO, DK, 16, true>) : go(gdn_preprocess_kernel<IO, DK, 16, false>);
        case 32: return packed ? go(gdn_preprocess_kernel<IO, DK, 32, true>) : go(gdn_preprocess_kernel<IO, DK, 32, false>);
        case 64: return packed ? go(gdn_preprocess_kernel<IO, DK, 64, true>) : go(gdn_preprocess_kernel<IO, DK, 64, false>);
        case 128:
            return packed ? go(gdn_preprocess_kernel<IO, DK, 128, true>) : go(gdn_preprocess_kernel<IO, DK, 128, false>);
        default: return hipErrorInvalidValue;
    }
}

template <class IO>
hipError_t launch_io(int B, int T, int H, int dk, int dv, const int* cu, int N, const void* x, const float* w,
                     const float* al, const float* bl, const void* st_in, void* st_out, void* q, void* k, void* v,
                     float* alpha, float* beta, hipStream_t stream) {
    hipError_t e;
    switch (dk) {
        case 16: e = launch_dv<IO, 16>(B, T, H, dv, cu, N, x, w, al, bl, st_in, st_out, q, k, v, alpha, beta, stream); break;
        case 32: e = launch_dv<IO, 32>(B, T, H, dv, cu, N, x, w, al, bl, st_in, st_out, q, k, v, alpha, beta, stream); break;
        case 64: e = launch_dv<IO, 64>(B, T, H, dv, cu, N, x, w, al, bl, st_in, st_out, q, k, v, alpha, beta, stream); break;
        case 128: e = launch_dv<IO, 128>(B, T, H, dv, cu, N, x, w, al, bl, st_in, st_out, q, k, v, alpha, beta, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || cu == nullptr || st_out == nullptr) return e;
    using E = typename IO::T;
    const int C = H * (2 * dk + dv);
    const size_t total = static_cast<size_t>(N) * 3 * C;
    const unsigned blocks = static_cast<unsigned>((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(gdn_state_out_kernel<IO>, dim3(blocks), dim3(256), 0, stream, N, T, C, cu,
                       static_cast<const E*>(x), static_cast<const E*>(st_in), static_cast<E*>(st_out));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_preprocess(int dtype, int B, int T, int H, int dk, int dv, const void* x, const float* w,
                                 const float* a_logit, const float* b_logit, const void* st_in, void* st_out,
                                 void* q, void* k, void* v, float* alpha, float* beta, hipStream_t stream) {
    if (B <= 0 || H <= 0) return hipSuccess;
    return dtype == kBF16 ? launch_io<IoBF16>(B, T, H, dk, dv, nullptr, 0, x, w, a_logit, b_logit, st_in, st_out, q,
                                              k, v, alpha, beta, stream)
                          : launch_io<IoF32>(B, T, H, dk, dv, nullptr, 0, x, w, a_logit, b_logit, st_in, st_out, q,
                                             k, v, alpha, beta, stream);
}

hipError_t launch_gdn_preprocess_varlen(int dtype, int N, int T, int H, int dk, int dv, const int* cu, const void* x,
                                        const float* w, const float* a_logit, const float* b_logit,
                                        const void* st_in, void* st_out, void* q, void* k, void* v, float* alpha,
                                        float* beta, hipStream_t stream) {
    if (N <= 0 || H <= 0) return hipSuccess;
    if (T == 0 && st_out == nullptr) return hipSuccess;
    // (T == 0: one workgroup per head runs with nothing to convolve; the states pass through)
    return dtype == kBF16 ? launch_io<IoBF16>(1, T, H, dk, dv, cu, N, x, w, a_logit, b_logit, st_in, st_out, q, k, v,
                                              alpha, beta, stream)
                          : launch_io<IoF32>(1, T, H, dk, dv, cu, N, x, w, a_logit, b_logit, st_in, st_out, q, k, v,
                                             alpha, beta, stream);
}

}  // namespace la

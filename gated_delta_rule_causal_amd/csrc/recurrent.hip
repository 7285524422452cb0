// Token-by-token recurrence with the state held in registers.
//
// One kernel template serves both kinds of recurrence on the page "Linear
// attention and hybrids":
//   * kGatedDelta - section "Delta rule and Gated DeltaNet", Gated DeltaNet
//     equation: S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//     o_t = S_t q_t.  Expanded per state row s_i (value channel i):
//       u = s_i.k,  p = s_i.q,  c = beta (v_i - alpha u),
//       s_i <- alpha s_i + c k,   o_i = alpha p + c (k.q)
//     so each row is read once and written once per token.
//   * kGated - section "Memory must forget: decay and gates", the decay
//     equation with the input-dependent gate alpha_t in place of gamma:
//       S_t = alpha_t S_{t-1} + v_t k_t^T,  o_t = S_t q_t, per row
//       p = s_i.q,  s_i <- alpha s_i + v_i k,  o_i = alpha p + v_i (k.q)
//   * kKda - same section, Kimi Delta Attention: the scalar gate becomes a
//     per-channel decay Diag(alpha_t) on the key side of S,
//     S_t = S_{t-1} Diag(alpha_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T; per row
//       d = s_i * alpha (elementwise),  u = d.k,  p = d.q,  c = beta (v_i - u),
//       s_i <- d + c k,   o_i = p + c (k.q)
//   * kNormalized - section "Three forms of one computation", recurrent form:
//       s_i <- s_i + v_i phi(k),  z <- z + phi(k),  o_i = s_i.phi(q) / z.phi(q)
// With T = 1 it is the decode step (the state streams from HBM and back,
// in place); with T > 1 it is the recurrent prefill form.
//
// Rows of S evolve independently (each new row depends only on the same old
// row and the token), so a block owns SPLIT-th of one head's rows and splits
// them over lane groups: LPR = dk/8 lanes per row, 8 fp32 state elements per
// lane held as two float4 (columns [4l, 4l+4) and [dk/2 + 4l, dk/2 + 4l + 4)
// for lane l of the group, so one load instruction covers 256 contiguous
// bytes of a row).  Dot products reduce over the LPR lanes by DPP.  The
// kinds without a normaliser cut each head's rows over two or more blocks
// (more blocks, fewer registers); the normalised kind does so only when z is
// not updated in place: every block then keeps its own copy of z (it depends
// on k alone) and the block holding row 0 writes it, while an in-place z
// (always so in the decode step) needs one block per head, so that no block
// can overwrite z before another has read it.
// The state is touched exactly once per call, so its loads and stores carry
// the nontemporal hint: the decode step streams the whole state through HBM
// and nothing it moves is reused by the next kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int kThreads = 256;

template <int DK>
struct RowSlice {
    static constexpr int LPR = DK / 8;
    static constexpr int RG = kThreads / LPR;  // row groups per block
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_state8(const float* row, int c0, int c1, float* s) {
    const f32x4v a = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(row + c0));
    const f32x4v b = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(row + c1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        s[e] = a[e];
        s[4 + e] = b[e];
    }
}

__device__ __forceinline__ void store_state8(float* row, int c0, int c1, const float* s) {
    const f32x4v a = {s[0], s[1], s[2], s[3]};
    const f32x4v b = {s[4], s[5], s[6], s[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4v*>(row + c0));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4v*>(row + c1));
}

template <class IO>
__device__ __forceinline__ void load_slice(const typename IO::T* p, size_t base, int c0, int c1,
                                           float* out) {
    IO::load4(p, base + c0, out);
    IO::load4(p, base + c1, out + 4);
}

// A block of TB tokens of one head's inputs in LDS: k, q [TB][DK], v [TB][DV]
// (DV <= 128), the gates (alpha [TB] or, per key channel, [TB][DK]; beta
// [TB]).  The workgroup copies a block cooperatively in 16-byte pieces: load()
// issues the global loads of block tokens t0 .. t0+TB-1 into registers, and
// store() writes them to LDS; rows past the sequence's end (Tn tokens) are
// neither read nor written.  Every token row of k, q, v and of a per-channel
// alpha is a whole number of 16-byte pieces (DK, DV >= 16), contiguous in
// global memory and in LDS.
template <int KIND, class IO, int DK>
struct Stage {
    static constexpr int TB = 16;
    using E = typename IO::T;
    static constexpr int KA = KIND == kKda ? DK : 1;
    struct Tiles {
        E k[TB * DK], q[TB * DK], v[TB * 128];
        float a[TB * KA], b[TB];
    };
    static constexpr int KROW = DK * static_cast<int>(sizeof(E)) / 16;    // pieces per row of k, q
    static constexpr int KPT = (TB * KROW + kThreads - 1) / kThreads;       // pieces per thread
    static constexpr int VPT = (TB * 128 * static_cast<int>(sizeof(E)) / 16 + kThreads - 1) / kThreads;
    static constexpr int AROW = KA * 4 / 16;                                 // per-channel alpha only
    static constexpr int APT = KIND == kKda ? (TB * AROW + kThreads - 1) / kThreads : 0;
    struct Regs {
        uint4 k[KPT], q[KPT], v[VPT], a[APT > 0 ? APT : 1];
        float as, bs;
    };
    static __device__ __forceinline__ void load(Regs& r, const E* q, const E* k, const E* v, const float* alpha,
                                                const float* beta, size_t tok0, int t0, int Tn, int DV) {
        const int tid = threadIdx.x, nt = min(TB, Tn - t0), vrow = DV * static_cast<int>(sizeof(E)) / 16;
        const char* kb = reinterpret_cast<const char*>(k + (tok0 + t0) * DK);
        const char* qb = reinterpret_cast<const char*>(q + (tok0 + t0) * DK);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int p = tid + i * kThreads;
            if (p < nt * KROW) {
                r.k[i] = *reinterpret_cast<const uint4*>(kb + 16 * static_cast<size_t>(p));
                r.q[i] = *reinterpret_cast<const uint4*>(qb + 16 * static_cast<size_t>(p));
            }
        }
        const char* vb = reinterpret_cast<const char*>(v + (tok0 + t0) * DV);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int p = tid + i * kThreads;
            if (p < nt * vrow) r.v[i] = *reinterpret_cast<const uint4*>(vb + 16 * static_cast<size_t>(p));
        }
        if constexpr (KIND == kKda) {
            const char* ab = reinterpret_cast<const char*>(alpha + (tok0 + t0) * DK);
#pragma unroll
            for (int i = 0; i < APT; ++i) {
                const int p = tid + i * kThreads;
                if (p < nt * AROW) r.a[i] = *reinterpret_cast<const uint4*>(ab + 16 * static_cast<size_t>(p));
            }
        }
        if constexpr (KIND == kGated || KIND == kGatedDelta) {
            if (tid < nt) r.as = alpha[tok0 + t0 + tid];
        }
        if constexpr (KIND == kGatedDelta || KIND == kKda) {
            if (tid < nt) r.bs = beta[tok0 + t0 + tid];
        }
    }
    static __device__ __forceinline__ void store(const Regs& r, Tiles& s, int t0, int Tn, int DV) {
        const int tid = threadIdx.x, nt = min(TB, Tn - t0), vrow = DV * static_cast<int>(sizeof(E)) / 16;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int p = tid + i * kThreads;
            if (p < nt * KROW) {
                reinterpret_cast<uint4*>(s.k)[p] = r.k[i];
                reinterpret_cast<uint4*>(s.q)[p] = r.q[i];
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int p = tid + i * kThreads;
            if (p < nt * vrow) reinterpret_cast<uint4*>(s.v)[p] = r.v[i];
        }
        if constexpr (KIND == kKda) {
#pragma unroll
            for (int i = 0; i < APT; ++i) {
                const int p = tid + i * kThreads;
                if (p < nt * AROW) reinterpret_cast<uint4*>(s.a)[p] = r.a[i];
            }
        }
        if constexpr (KIND == kGated || KIND == kGatedDelta) {
            if (tid < nt) s.a[tid] = r.as;
        }
        if constexpr (KIND == kGatedDelta || KIND == kKda) {
            if (tid < nt) s.b[tid] = r.bs;
        }
    }
};

template <int KIND, class IO, int DK, int R, int SPLIT, bool ONE>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(
    int T, int DV, const typename IO::T* __restrict__ q, const typename IO::T* __restrict__ k,
    const typename IO::T* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, const float* S0, float* S_out, const float* z0, float* z_out,
    typename IO::T* __restrict__ o, Packed pk) {
    constexpr int LPR = RowSlice<DK>::LPR;
    constexpr int RG = RowSlice<DK>::RG;
    int head = blockIdx.x / SPLIT;   // state index (packed: sequence * H + head)
    // token rows of this head: [head][T] (uniform) or tokens cu[n].. of row
    // block h of [H][Ttot] (packed batch)
    size_t tok0 = static_cast<size_t>(head) * T;
    int Tn = T, hh = 0, snap0 = 0;
    if (!ONE && pk.cu != nullptr) {   // (the decode step never runs a packed batch)
        const int ni = head / pk.H;
        hh = head - ni * pk.H;
        const int n = pk.seq_order ? pk.seq_order[ni] : ni;
        head = n * pk.H + hh;
        const int t0 = min(max(pk.cu[n], 0), pk.Ttot), t1 = min(max(pk.cu[n + 1], 0), pk.Ttot);
        Tn = t1 > t0 ? t1 - t0 : 0;
        tok0 = static_cast<size_t>(hh) * pk.Ttot + t0;
        snap0 = pk.snap_base ? pk.snap_base[n] : 0;
    }
    const int li = threadIdx.x % LPR;
    const int rg = threadIdx.x / LPR + (blockIdx.x % SPLIT) * RG * R;  // first row of this lane group
    const int c0 = 4 * li;
    const int c1 = DK / 2 + 4 * li;
    const size_t sbase = static_cast<size_t>(head) * DV * DK;

    // ---- carried state: R rows per lane group, 8 columns per lane
    float s[R][8];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int r = rg + RG * j;
        if (S0 != nullptr && r < DV) {
            load_state8(S0 + sbase + static_cast<size_t>(r) * DK, c0, c1, s[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
        }
    }
    float z[8];
    if constexpr (KIND == kNormalized) {
        const size_t zb = static_cast<size_t>(head) * DK;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = 0.f;
        if (z0 != nullptr) {
            const float4 a = *reinterpret_cast<const float4*>(z0 + zb + c0);
            const float4 b = *reinterpret_cast<const float4*>(z0 + zb + c1);
            z[0] = a.x; z[1] = a.y; z[2] = a.z; z[3] = a.w;
            z[4] = b.x; z[5] = b.y; z[6] = b.z; z[7] = b.w;
        }
    }

    // ---- token inputs, prefetched one token ahead.  The decode step reads
    // them from global memory; the prefill stages blocks of TB tokens through
    // LDS (Stage below), so the wait for HBM is paid once per block, not once
    // per token of the serial chain.
    float kn[8], qn[8], vn[R], an = 1.f, bn = 0.f, avn[8];
    using St = Stage<KIND, IO, DK>;
    __shared__ __attribute__((aligned(16))) typename St::Tiles st[ONE ? 1 : 2];
    typename St::Regs sr;
    auto fetch = [&](int t) {
        if constexpr (ONE) {
            const size_t tk = (tok0 + t) * DK;
            const size_t tv = (tok0 + t) * DV;
            load_slice<IO>(k, tk, c0, c1, kn);
            load_slice<IO>(q, tk, c0, c1, qn);
            if constexpr (KIND == kKda) load_slice<IoF32>(alpha, tk, c0, c1, avn);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int r = rg + RG * j;
                vn[j] = r < DV ? IO::load(v, tv + r) : 0.f;
            }
            if constexpr (KIND == kGated || KIND == kGatedDelta) an = alpha[tok0 + t];
            if constexpr (KIND == kGatedDelta || KIND == kKda) bn = beta[tok0 + t];
        } else {
            const typename St::Tiles& b = st[(t / St::TB) & 1];
            const int tl = t % St::TB;
            load_slice<IO>(b.k, static_cast<size_t>(tl) * DK, c0, c1, kn);
            load_slice<IO>(b.q, static_cast<size_t>(tl) * DK, c0, c1, qn);
            if constexpr (KIND == kKda) load_slice<IoF32>(b.a, static_cast<size_t>(tl) * DK, c0, c1, avn);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int r = rg + RG * j;
                vn[j] = r < DV ? IO::load(b.v, static_cast<size_t>(tl) * DV + r) : 0.f;
            }
            if constexpr (KIND == kGated || KIND == kGatedDelta) an = b.a[tl];
            if constexpr (KIND == kGatedDelta || KIND == kKda) bn = b.b[tl];
        }
    };
    if constexpr (!ONE) {
        // block 0 into LDS, block 1 in flight in registers
        if (Tn > 0) {
            St::load(sr, q, k, v, alpha, beta, tok0, 0, Tn, DV);
            St::store(sr, st[0], 0, Tn, DV);
            __syncthreads();
            if (Tn > St::TB) St::load(sr, q, k, v, alpha, beta, tok0, St::TB, Tn, DV);
        }
    }
    if (ONE || Tn > 0) fetch(0);

    const int steps = ONE ? 1 : Tn;  // ONE: the decode step (T = 1), no prefetch path
    for (int t = 0; t < steps; ++t) {
        float kc[8], qc[8], vc[R], ac[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) { kc[e] = kn[e]; qc[e] = qn[e]; }
        if constexpr (KIND == kKda) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ac[e] = avn[e];
        }
#pragma unroll
        for (int j = 0; j < R; ++j) vc[j] = vn[j];
        const float a = an, b = bn;
        if constexpr (!ONE) {
            if (t + 1 < Tn) {
                if ((t + 1) % St::TB == 0) {
                    // next block: registers -> LDS (the copy it replaces was last
                    // read before the previous block's barrier), then the block
                    // after it into registers
                    St::store(sr, st[((t + 1) / St::TB) & 1], t + 1, Tn, DV);
                    __syncthreads();
                    if (t + 1 + St::TB < Tn) St::load(sr, q, k, v, alpha, beta, tok0, t + 1 + St::TB, Tn, DV);
                }
                fetch(t + 1);
            }
        }
        const size_t to = (tok0 + t) * DV;

        if constexpr (KIND == kGated) {
            (void)b;
            float kq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) kq = fmaf(kc[e], qc[e], kq);
            kq = group_sum<LPR>(kq);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) p = fmaf(s[j][e], qc[e], p);
                p = group_sum<LPR>(p);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[j][e] = fmaf(a, s[j][e], vc[j] * kc[e]);
                const int r = rg + RG * j;
                if (li == 0 && r < DV) IO::store(o, to + r, fmaf(a, p, vc[j] * kq));
            }
        } else if constexpr (KIND == kGatedDelta) {
            float kq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) kq = fmaf(kc[e], qc[e], kq);
            kq = group_sum<LPR>(kq);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float u = 0.f, p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u = fmaf(s[j][e], kc[e], u);
                    p = fmaf(s[j][e], qc[e], p);
                }
                u = group_sum<LPR>(u);
                p = group_sum<LPR>(p);
                const float c = b * (vc[j] - a * u);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[j][e] = fmaf(a, s[j][e], c * kc[e]);
                const int r = rg + RG * j;
                if (li == 0 && r < DV) IO::store(o, to + r, fmaf(a, p, c * kq));
            }
        } else if constexpr (KIND == kKda) {
            (void)a;
            float kq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) kq = fmaf(kc[e], qc[e], kq);
            kq = group_sum<LPR>(kq);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float u = 0.f, p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    s[j][e] *= ac[e];
                    u = fmaf(s[j][e], kc[e], u);
                    p = fmaf(s[j][e], qc[e], p);
                }
                u = group_sum<LPR>(u);
                p = group_sum<LPR>(p);
                const float c = b * (vc[j] - u);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[j][e] = fmaf(c, kc[e], s[j][e]);
                const int r = rg + RG * j;
                if (li == 0 && r < DV) IO::store(o, to + r, fmaf(c, kq, p));
            }
        } else {
            float fk[8], fq[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { fk[e] = phi(kc[e]); fq[e] = phi(qc[e]); }
            float den = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                z[e] += fk[e];
                den = fmaf(z[e], fq[e], den);
            }
            den = group_sum<LPR>(den);
            const float rden = 1.f / den;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float num = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    s[j][e] = fmaf(vc[j], fk[e], s[j][e]);
                    num = fmaf(s[j][e], fq[e], num);
                }
                num = group_sum<LPR>(num);
                const int r = rg + RG * j;
                if (li == 0 && r < DV) IO::store(o, to + r, num * rden);
            }
        }
        // packed batches: the state after every pk.snap tokens
        if (!ONE && pk.snap > 0 && (t + 1) % pk.snap == 0) {
            const int js = snap0 + (t + 1) / pk.snap - 1;
            if (js < pk.snap_cap) {
                float* dst = pk.S_snap + (static_cast<size_t>(js) * pk.H + hh) * DV * DK;
#pragma unroll
                for (int j = 0; j < R; ++j) {
                    const int r = rg + RG * j;
                    if (r < DV) store_state8(dst + static_cast<size_t>(r) * DK, c0, c1, s[j]);
                }
                if constexpr (KIND == kNormalized) {
                    if (rg == 0 && pk.z_snap != nullptr) {   // every lane group holds the same z
                        float* zp = pk.z_snap + (static_cast<size_t>(js) * pk.H + hh) * DK;
                        *reinterpret_cast<float4*>(zp + c0) = make_float4(z[0], z[1], z[2], z[3]);
                        *reinterpret_cast<float4*>(zp + c1) = make_float4(z[4], z[5], z[6], z[7]);
                    }
                }
            }
        }
    }

    // ---- write back the state (same lanes that read it: in-place safe)
    if (S_out != nullptr) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int r = rg + RG * j;
            if (r < DV) store_state8(S_out + sbase + static_cast<size_t>(r) * DK, c0, c1, s[j]);
        }
    }
    if constexpr (KIND == kNormalized) {
        if (z_out != nullptr) {
            __syncthreads();  // every lane group has read z0 before it is overwritten
            if (rg == 0) {
                float* zp = z_out + static_cast<size_t>(head) * DK;
                *reinterpret_cast<float4*>(zp + c0) = make_float4(z[0], z[1], z[2], z[3]);
                *reinterpret_cast<float4*>(zp + c1) = make_float4(z[4], z[5], z[6], z[7]);
            }
        }
    }
}

template <int KIND, class IO, int DK, bool ONE>
hipError_t launch_rows(int heads, int T, int dv, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* S0, float* S_out,
                     const float* z0, float* z_out, void* o, const Packed& pk, hipStream_t stream) {
    using E = typename IO::T;
    constexpr int RG = RowSlice<DK>::RG;
    // A head's rows go to 2 blocks (the normalised kind: only when z is not
    // updated in place); a token-serial prefill over few heads splits further (up to 8 blocks
    // of at least one row group each) so that about 512 blocks run, and a
    // packed batch always splits as far as it can: its longest sequence runs
    // on after the others have finished, and fewer rows per wave shorten
    // that sequence's per-token chain.
    const bool z_in_place = KIND == kNormalized && (ONE || (z0 != nullptr && z0 == z_out));
    int split = (!z_in_place && dv >= 2 * RG) ? 2 : 1;
    if (!ONE && split == 2)
        while (split < 8 && dv >= 2 * split * RG &&
               (pk.cu != nullptr || static_cast<long long>(heads) * split < 512))
            split *= 2;
    const int R = (dv / split + RG - 1) / RG;
    if (!grid_fits(static_cast<long long>(heads) * split, kThreads)) return hipErrorInvalidConfiguration;
    dim3 grid(static_cast<unsigned>(heads) * split), block(kThreads);
    auto args = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, stream, T, dv, static_cast<const E*>(q),
                           static_cast<const E*>(k), static_cast<const E*>(v), alpha, beta, S0,
                           S_out, z0, z_out, static_cast<E*>(o), pk);
        return hipGetLastError();
    };
    {
        if (split == 2) {
            switch (R) {
                case 1: return args(recurrent_kernel<KIND, IO, DK, 1, 2, ONE>);
                case 2: return args(recurrent_kernel<KIND, IO, DK, 2, 2, ONE>);
                case 4: return args(recurrent_kernel<KIND, IO, DK, 4, 2, ONE>);
                default: return hipErrorInvalidValue;
            }
        }
        if constexpr (!ONE) {
            if (split == 4) {
                switch (R) {
                    case 1: return args(recurrent_kernel<KIND, IO, DK, 1, 4, ONE>);
                    case 2: return args(recurrent_kernel<KIND, IO, DK, 2, 4, ONE>);
                    default: return hipErrorInvalidValue;
                }
            }
            if (split == 8) {
                if (R == 1) return args(recurrent_kernel<KIND, IO, DK, 1, 8, ONE>);
                return hipErrorInvalidValue;
            }
        }
    }
    switch (R) {
        case 1: return args(recurrent_kernel<KIND, IO, DK, 1, 1, ONE>);
        case 2: return args(recurrent_kernel<KIND, IO, DK, 2, 1, ONE>);
        case 4: return args(recurrent_kernel<KIND, IO, DK, 4, 1, ONE>);
        case 8: return args(recurrent_kernel<KIND, IO, DK, 8, 1, ONE>);
        default: return hipErrorInvalidValue;
    }
}

template <int KIND, class IO, int DK>
hipError_t launch_dk(int heads, int T, int dv, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* S0, float* S_out,
                     const float* z0, float* z_out, void* o, const Packed& pk, hipStream_t stream) {
    if (T == 1 && pk.cu == nullptr)
        return launch_rows<KIND, IO, DK, true>(heads, T, dv, q, k, v, alpha, beta, S0, S_out, z0, z_out, o, pk, stream);
    return launch_rows<KIND, IO, DK, false>(heads, T, dv, q, k, v, alpha, beta, S0, S_out, z0, z_out, o, pk, stream);
}

template <int KIND, class IO>
hipError_t launch_io(int heads, int T, int dk, int dv, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* S0, float* S_out,
                     const float* z0, float* z_out, void* o, const Packed& pk, hipStream_t stream) {
    switch (dk) {
        case 16: return launch_dk<KIND, IO, 16>(heads, T, dv, q, k, v, alpha, beta, S0, S_out, z0, z_out, o, pk, stream);
        case 32: return launch_dk<KIND, IO, 32>(heads, T, dv, q, k, v, alpha, beta, S0, S_out, z0, z_out, o, pk, stream);
        case 64: return launch_dk<KIND, IO, 64>(heads, T, dv, q, k, v, alpha, beta, S0, S_out, z0, z_out, o, pk, stream);
        case 128: return launch_dk<KIND, IO, 128>(heads, T, dv, q, k, v, alpha, beta, S0, S_out, z0, z_out, o, pk, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_recurrent(int kind, int dtype, int heads, int T, int dk, int dv, const void* q,
                            const void* k, const void* v, const float* alpha, const float* beta,
                            const float* S0, float* S_out, const float* z0, float* z_out, void* o,
                            hipStream_t stream, const Packed& pk) {
    if (heads <= 0 || (T <= 0 && pk.cu == nullptr)) return hipSuccess;
    const bool bf = dtype == kBF16;
    switch (kind) {
        case kGated:
            return bf ? launch_io<kGated, IoBF16>(heads, T, dk, dv, q, k, v, alpha, nullptr, S0, S_out, nullptr,
                                                  nullptr, o, pk, stream)
                      : launch_io<kGated, IoF32>(heads, T, dk, dv, q, k, v, alpha, nullptr, S0, S_out, nullptr,
                                                 nullptr, o, pk, stream);
        case kKda:
            return bf ? launch_io<kKda, IoBF16>(heads, T, dk, dv, q, k, v, alpha, beta, S0, S_out, nullptr, nullptr,
                                                o, pk, stream)
                      : launch_io<kKda, IoF32>(heads, T, dk, dv, q, k, v, alpha, beta, S0, S_out, nullptr, nullptr, o,
                                               pk, stream);
        case kGatedDelta:
            return bf ? launch_io<kGatedDelta, IoBF16>(heads, T, dk, dv, q, k, v, alpha, beta, S0, S_out, nullptr,
                                                       nullptr, o, pk, stream)
                      : launch_io<kGatedDelta, IoF32>(heads, T, dk, dv, q, k, v, alpha, beta, S0, S_out, nullptr,
                                                      nullptr, o, pk, stream);
        default:
            return bf ? launch_io<kNormalized, IoBF16>(heads, T, dk, dv, q, k, v, nullptr, nullptr, S0, S_out, z0,
                                                       z_out, o, pk, stream)
                      : launch_io<kNormalized, IoF32>(heads, T, dk, dv, q, k, v, nullptr, nullptr, S0, S_out, z0,
                                                      z_out, o, pk, stream);
    }
}

}  // namespace la

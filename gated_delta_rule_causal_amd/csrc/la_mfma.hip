// Normalised causal linear attention, chunked form, on the CDNA4 matrix
// cores: bf16 activations, fp32 state and normaliser, d_k = d_v = 128,
// chunk C = 64.
//
// Source: page "Linear attention and hybrids", section "Three forms of one
// computation", chunk equation and block flowchart (plus the same
// normalisation as the recurrent form): per block b,
//     A   = tril(phi(Q_b) phi(K_b)^T)                 (diagonal included)
//     num = A V_b + phi(Q_b) S^T,   den = rowsum(A) + phi(Q_b) z
//     O_b = num / den,   then  S += V_b^T phi(K_b),  z += colsum phi(K_b)
//
// The sequence of every head is cut into G segments of whole blocks so that
// B*H*G workgroups fill the chip (S and z are sums over tokens, so a segment's
// contribution does not depend on what came before):
//  * la_chunked_mfma_kernel<false> (segments 0..G-2): the segment's
//    contributions dS = sum V_b^T phi(K_b), dz = sum colsum phi(K_b);
//  * la_combine_kernel: entering states by prefix sums, S0 + dS_0 + ... ;
//  * la_chunked_mfma_kernel<true> (every segment): outputs from the entering
//    state, and the final state in the last segment.
// A packed batch of sequences of different lengths runs the same three
// kernels with each sequence cut into its own segments: a table built on the
// device maps a workgroup to (sequence, head, segment), and the output pass
// also writes state snapshots at whole blocks (S, and z for the normalised
// kind), since it holds the running state after every block.
// One workgroup (4 waves) walks the blocks of its segment in order; the
// kernels are held to 256 registers per lane so that two workgroups share a
// CU (about 512 segments in flight, one hiding the other's latencies).  Each wave
// owns 32 value channels of the state, P = S_rows^T (d_k x 32, fp32) in
// accumulator registers; the state update is a plain accumulation
// P += phi(K_b)^T V_b on MFMA and, as in the gated-delta scan, accumulator
// tiles feed the next product as B operands through a permuted contraction
// index.  Per block the tiles phi(Q), phi(K) and V are staged row-major in
// LDS with phi applied on the way in (the products that contract over tokens
// read them with the transposing LDS load); the next block's raw q/k/v are
// prefetched into registers while the current block computes.
// z lives in LDS and is only written back by this workgroup, so an in-place
// update of z is race-free.
//
// GATED selects the scalar-gated, unnormalised variant of the same page
// (section "Memory must forget: decay and gates": the decay equation with an
// input-dependent gate alpha_t): S_t = alpha_t S_{t-1} + v_t k_t^T,
// o_t = S_t q_t, no feature map and no normaliser.  With g the chunk-local
// cumsum of log alpha (a DPP scan per wave), a chunk is
//     A = tril(Q K^T) * Gamma,  Gamma_ij = e^{g_i - g_j}
//     O = diag(e^g) Q S^T + A V,   S <- e^{g_c} S + V^T diag(e^{g_c - g}) K
// and a segment's contribution is (decay m = e^{sum of log alpha}, dS), with
// entering states P_{s+1} = m_s P_s + dS_s.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int C = 64;
constexpr int D = 128;
constexpr int LDR = D + 24;  // row-major [C][LDR] bf16 tiles (304-B rows: see the gated-delta kernels)
constexpr int LDT = C + 8;   // 64-wide [C][LDT] bf16 tiles (144-B rows)
constexpr int kThreads = 256;
constexpr int kItems = C * D / 8 / kThreads;  // 16-byte loads per thread per tile
constexpr int kTargetBlocks = 512;           // workgroups that fill the chip (two per CU)
constexpr size_t kMat = static_cast<size_t>(D) * D;

// Workspace record per (head, segment) slot: entering state P (state layout
// [d_v][d_k]) and normaliser zP, then the segment's contributions dS, dz.
constexpr size_t kRec = 2 * kMat + 2 * D;
__device__ __forceinline__ size_t ws_P(size_t slot) { return slot * kRec; }
__device__ __forceinline__ size_t ws_zP(size_t slot) { return ws_P(slot) + kMat; }
__device__ __forceinline__ size_t ws_dS(size_t slot) { return ws_P(slot) + kMat + D; }
__device__ __forceinline__ size_t ws_dz(size_t slot) { return ws_P(slot) + 2 * kMat + D; }

// Where the segments of a call live: a uniform batch (BH heads of T tokens,
// G segments of SEGC chunks each, slot of segment s of head bh at bh G + s),
// or a packed batch (cu != nullptr: N sequences back to back in each of H
// heads of Ttot tokens; seg_base[n] = segments of the sequences before n,
// built on the device; slot of segment s of sequence n in head h at
// h Gcap + seg_base[n] + s).
struct LGeo {
    int BH, T, NC, G, SEGC;
    const int* cu;
    const int* seg_base;
    const int* snap_base;
    const int* order;   // packed: segments longest first (workgroup i takes order[i])
    int N, H, Ttot, Gcap;
    int snap, snap_cap;   // packed: snapshots of (S, z) after every `snap` tokens (a multiple of C)
    float* S_snap;
    float* z_snap;
};

// One (sequence, head, segment) work item.
struct LItem {
    size_t head_tok;   // token row of the sequence's first token (this head)
    size_t slot0;      // slot of the sequence's segment 0
    size_t state;      // index of the sequence's state in S0 / S_out (and z)
    int T, G, seg, n0, n1, snap0, h;
};

__device__ __forceinline__ int lclamp(int t, int Ttot) { return t < 0 ? 0 : t > Ttot ? Ttot : t; }

// The item of workgroup blk: OUT, every segment; else segments 0..G-2 (the
// last segment's contribution is never needed).  False: nothing to do.
template <bool PACKED>
__device__ __forceinline__ bool la_item(const LGeo& g, int blk, bool out, LItem& it) {
    if constexpr (!PACKED) {
        const int per = out ? g.G : g.G - 1;
        const int bh = blk / per;
        if (bh >= g.BH) return false;
        it.seg = blk - bh * per;
        it.G = g.G;
        it.T = g.T;
        it.head_tok = static_cast<size_t>(bh) * g.T;
        it.slot0 = static_cast<size_t>(bh) * g.G;
        it.state = bh;
        it.snap0 = 0;
        it.h = 0;
    } else {
        const int h = blk % g.H, i = blk / g.H;
        if (i >= min(g.seg_base[g.N], g.Gcap)) return false;
        const int gs = g.order ? g.order[i] : i;
        int lo = 0, hi = g.N;   // seg_base[lo] <= gs < seg_base[hi]; every sequence has a segment
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.seg_base[mid] <= gs) lo = mid; else hi = mid;
        }
        it.seg = gs - g.seg_base[lo];
        it.G = g.seg_base[lo + 1] - g.seg_base[lo];
        if (!out && it.seg == it.G - 1) return false;
        if (g.seg_base[lo + 1] > g.Gcap) return false;   // a bad table never overruns the workspace
        const int t0 = lclamp(g.cu[lo], g.Ttot), t1 = lclamp(g.cu[lo + 1], g.Ttot);
        it.T = t1 > t0 ? t1 - t0 : 0;
        it.head_tok = static_cast<size_t>(h) * g.Ttot + t0;
        it.slot0 = static_cast<size_t>(h) * g.Gcap + g.seg_base[lo];
        it.state = static_cast<size_t>(lo) * g.H + h;
        it.snap0 = g.snap_base ? g.snap_base[lo] : 0;
        it.h = h;
    }
    it.n0 = it.seg * g.SEGC;
    it.n1 = min((it.T + C - 1) / C, it.n0 + g.SEGC);
    return true;
}

__device__ __forceinline__ int perm_row(int t, int rr) {
    return 32 * (t >> 1) + 8 * (rr >> 2) + 4 * (t & 1) + (rr & 3);
}

__device__ __forceinline__ bf16x8 lds8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// x + (x of the lane the DPP control selects, 0 where there is none).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes without LDS: shifts inside 16-lane
// rows, then lane 15 into rows 1 and 3 and lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x = dpp_add<0x111, 0xf>(x);
    x = dpp_add<0x112, 0xf>(x);
    x = dpp_add<0x114, 0xf>(x);
    x = dpp_add<0x118, 0xf>(x);
    x = dpp_add<0x142, 0xa>(x);
    return dpp_add<0x143, 0xc>(x);
}

// OUT = false: segment contributions only (no q, no outputs), from a zero state.
// GATED: the scalar-gated variant (alpha used, z0/z_out unused).
// PACKED: a packed batch (geo.cu set; a copy of the kernel so that the
// uniform batch carries none of its table lookups).
template <bool GATED, bool OUT, bool PACKED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void la_chunked_mfma_kernel(
    LGeo geo, const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* S0, const float* z0, float* ws, u16* __restrict__ o, float* S_out,
    float* z_out) {
    __shared__ __attribute__((aligned(16))) u16 fQ[C][LDR];
    __shared__ __attribute__((aligned(16))) u16 fK[C][LDR];
    __shared__ __attribute__((aligned(16))) u16 Vs[C][LDR];
    __shared__ __attribute__((aligned(16))) u16 As[C][LDT];
    __shared__ float zs[D], dens[C];
    // normalised kind: per 16-row group of a chunk, the column sums of phi(K)
    // that the staging threads formed (padded rows: fewer bank conflicts)
    __shared__ float zpart[GATED ? 1 : D][17];
    __shared__ float gs[C], egs[C], eks[C];   // GATED: chunk-local g, e^g, e^{g_c - g}

    LItem it;
    if (!la_item<PACKED>(geo, blockIdx.x, OUT, it)) return;
    const int G = it.G, seg = it.seg, n0 = it.n0, n1 = it.n1, T = it.T;
    const size_t slot = it.slot0 + seg;
    // entering state: S0 itself when the sequence is one segment, else the
    // prefix sum from the workspace (segment 0 included, so S_out may alias S0)
    const float* Sin = !OUT ? nullptr
                       : G == 1 ? (S0 ? S0 + it.state * kMat : nullptr)
                                : ws + ws_P(slot);
    const float* zin = (!OUT || GATED) ? nullptr
                       : G == 1 ? (z0 ? z0 + it.state * D : nullptr)
                                : ws + ws_zP(slot);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: MFMAs sit in branches on it
    const int lane = tid & 63;
    const int r = lane & 15;
    const int g = lane >> 4;

    // ---- state: wave w owns value channels 32w + 16nb + r (nb = 0, 1)
    f32x4 P[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int vc = 32 * w + 16 * nb + r;
        const float* srow = Sin ? Sin + static_cast<size_t>(vc) * D : nullptr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int d0 = 32 * s + 8 * g;
            if (srow) {
                const float4 a = *reinterpret_cast<const float4*>(srow + d0);
                const float4 b = *reinterpret_cast<const float4*>(srow + d0 + 4);
                P[nb][2 * s] = f32x4{a.x, a.y, a.z, a.w};
                P[nb][2 * s + 1] = f32x4{b.x, b.y, b.z, b.w};
            } else {
                P[nb][2 * s] = zero4();
                P[nb][2 * s + 1] = zero4();
            }
        }
    }
    if (tid < D) zs[tid] = zin ? zin[tid] : 0.f;

    // ---- raw chunk prefetch: item e = tid + kThreads * it -> row = e / 16, c8 = 8 (e % 16):
    //      16 lanes read one 256-byte row, so a wave-wide load is 1 KiB contiguous
    uint4 rq[kItems], rk[kItems], rv[kItems];
    float ra = 1.f;   // GATED: alpha of token `lane` of the chunk (1 past the end)
    float decay = 1.f;  // GATED: product of the gates seen so far in this segment
    const size_t head = it.head_tok * D;
    auto fetch = [&](int n) {
        const int t0 = n * C;
        const int len = min(C, T - t0);
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int e = tid + kThreads * it;
            const int row = e >> 4, c8 = 8 * (e & 15);
            if constexpr (!GATED) {
                // every load issued (rows past the end read the last row and
                // are zeroed when staged): see the peeled first chunk below
                const size_t gi = head + static_cast<size_t>(t0 + min(row, len - 1)) * D + c8;
                if (OUT) rq[it] = *reinterpret_cast<const uint4*>(q + gi);
                rk[it] = *reinterpret_cast<const uint4*>(k + gi);
                rv[it] = *reinterpret_cast<const uint4*>(v + gi);
            } else {
                rq[it] = rk[it] = rv[it] = make_uint4(0, 0, 0, 0);
                if (row < len) {
                    const size_t gi = head + static_cast<size_t>(t0 + row) * D + c8;
                    if (OUT) rq[it] = *reinterpret_cast<const uint4*>(q + gi);
                    rk[it] = *reinterpret_cast<const uint4*>(k + gi);
                    rv[it] = *reinterpret_cast<const uint4*>(v + gi);
                }
            }
        }
        if (GATED) ra = lane < len ? alpha[it.head_tok + t0 + lane] : 1.f;
    };
    if (n1 > n0) fetch(n0);   // (an empty sequence has no chunk to load)
    // this wave's rows of the state (value channels 32w + 16nb + r) into a [d_v][d_k] fp32 matrix
    auto store_P = [&](float* dst) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            float* srow = dst + static_cast<size_t>(32 * w + 16 * nb + r) * D;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int d0 = 32 * s + 8 * g;
                *reinterpret_cast<float4*>(srow + d0) =
                    make_float4(P[nb][2 * s][0], P[nb][2 * s][1], P[nb][2 * s][2], P[nb][2 * s][3]);
                *reinterpret_cast<float4*>(srow + d0 + 4) =
                    make_float4(P[nb][2 * s + 1][0], P[nb][2 * s + 1][1], P[nb][2 * s + 1][2], P[nb][2 * s + 1][3]);
            }
        }
    };
    // packed batches: slot of the snapshot taken after chunk n, or -1
    auto snap_slot = [&](int n) {
        const int end = (n + 1) * C;
        if (!OUT || !PACKED || geo.snap <= 0 || end > T || end % geo.snap != 0) return -1;
        const int js = it.snap0 + end / geo.snap - 1;
        return js < geo.snap_cap ? js : -1;
    };

    // One chunk.  Normalised kind: the first chunk is peeled off the loop, so
    // every path into the loop ends with the same loads and stores and the
    // wait for a chunk's loads is a count that leaves the previous chunk's
    // output stores in flight (with both paths merged at the loop head the
    // compiler waits for everything).  The gated kind measured slower peeled.
    auto chunk = [&](int n) {
        const int t0 = n * C;
        const int len = min(C, T - t0);
        lds_barrier();  // the previous block's LDS tiles are no longer read
        // GATED: g for token `lane` (alpha of token `lane` is in ra); e^{g_c - g}
        // scales the rows of V for the state update
        float ek = 1.f, egc = 1.f;
        if constexpr (GATED) {
            const float gx = wave_prefix_sum(__logf(ra));
            const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gx), C - 1));
            ek = __expf(gl - gx);
            egc = __expf(gl);
            if (w == 0) {
                gs[lane] = gx;
                egs[lane] = __expf(gx);
                eks[lane] = ek;
            }
        }
        // ---- stage phi(Q), phi(K), phi(K)^T, V^T (padded rows stay zero: phi is
        //      applied only to real tokens, so they add nothing to A, S or z);
        //      GATED: Q, K, (e^{g_c - g} K)^T, V^T
        // (a whole chunk, the usual case, takes a copy of the loop without the
        // row masks: len is uniform over the workgroup)
        auto stage = [&](auto whole) {
        float zp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // this thread's rows of its 8 channels
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
            const int e = tid + kThreads * it;
            const int row = e >> 4, c8 = 8 * (e & 15);
            const bool real = decltype(whole)::value || row < len;
            const uint32_t wq[4] = {rq[it].x, rq[it].y, rq[it].z, rq[it].w};
            const uint32_t wk[4] = {rk[it].x, rk[it].y, rk[it].z, rk[it].w};
            float xq[8], xk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t bq = (j & 1) ? (wq[j >> 1] & 0xffff0000u) : (wq[j >> 1] << 16);
                const uint32_t bk = (j & 1) ? (wk[j >> 1] & 0xffff0000u) : (wk[j >> 1] << 16);
                if (GATED) {
                    xq[j] = __uint_as_float(bq);
                    xk[j] = __uint_as_float(bk);
                } else {
                    xq[j] = real ? phi(__uint_as_float(bq)) : 0.f;
                    xk[j] = real ? phi(__uint_as_float(bk)) : 0.f;
                }
            }
            const bf16x8 pq = pack8(xq[0], xq[1], xq[2], xq[3], xq[4], xq[5], xq[6], xq[7]);
            const bf16x8 pk = pack8(xk[0], xk[1], xk[2], xk[3], xk[4], xk[5], xk[6], xk[7]);
            if (OUT) *reinterpret_cast<bf16x8*>(&fQ[row][c8]) = pq;
            *reinterpret_cast<bf16x8*>(&fK[row][c8]) = pk;
            *reinterpret_cast<uint4*>(&Vs[row][c8]) = real ? rv[it] : make_uint4(0, 0, 0, 0);
            if (!GATED) {
#pragma unroll
                for (int j = 0; j < 8; ++j) zp[j] += xk[j];
            }
        }
        if (!GATED) {   // rows (tid >> 4) + 16 it of channels 8 (tid & 15) .. +7
#pragma unroll
            for (int j = 0; j < 8; ++j) zpart[8 * (tid & 15) + j][tid >> 4] = zp[j];
        }
        };
        if (len == C)
            stage(std::true_type{});
        else
            stage(std::false_type{});
        if constexpr (GATED) {
            if (n + 1 < n1) fetch(n + 1);
        } else {
            fetch(min(n + 1, n1 - 1));
        }
        lds_barrier();

        // ---- A = tril(phi(Q) phi(K)^T), row tile w, and its row sums (fp32)
        if constexpr (OUT) {
            // A is formed transposed (phi(K) tile times phi(Q) tile) so that the
            // lane holds 4 consecutive columns of one row: A[16w + r][16ct + 4g ..]
            // (one 8-byte LDS write per tile, row sums over the 4 g lanes)
            const int row = 16 * w + r;
            float rs = 0.f;
            for (int ct = 0; ct < 4; ++ct) {
                uint2 bits = make_uint2(0, 0);
                if (ct <= w) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        acc = mfma16x16x32(lds8(&fK[16 * ct + r][32 * s + 8 * g]),
                                           lds8(&fQ[16 * w + r][32 * s + 8 * g]), acc);
                    float a4[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int col = 16 * ct + 4 * g + i;
                        a4[i] = col > row ? 0.f
                                : GATED ? acc[i] * __expf(fminf(gs[row] - gs[col], 0.f))
                                        : acc[i];
                        rs += a4[i];
                    }
                    bits = make_uint2(pack_bf16x2(a4[0], a4[1]), pack_bf16x2(a4[2], a4[3]));
                }
                *reinterpret_cast<uint2*>(&As[row][16 * ct + 4 * g]) = bits;
            }
            if (!GATED) {
                // den = rowsum(A) + phi(Q) z (z of the previous blocks): the 4
                // lanes of a row split its columns and the 128 channels
                rs += __shfl_xor(rs, 16, kWave);
                rs += __shfl_xor(rs, 32, kWave);
                float d0 = 0.f, d1 = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c0 = 32 * g + 8 * j;
                    const uint4 u = *reinterpret_cast<const uint4*>(&fQ[row][c0]);
                    const float4 za = *reinterpret_cast<const float4*>(&zs[c0]);
                    const float4 zb = *reinterpret_cast<const float4*>(&zs[c0 + 4]);
                    d0 = fmaf(__uint_as_float(u.x << 16), za.x, d0);
                    d1 = fmaf(__uint_as_float(u.x & 0xffff0000u), za.y, d1);
                    d0 = fmaf(__uint_as_float(u.y << 16), za.z, d0);
                    d1 = fmaf(__uint_as_float(u.y & 0xffff0000u), za.w, d1);
                    d0 = fmaf(__uint_as_float(u.z << 16), zb.x, d0);
                    d1 = fmaf(__uint_as_float(u.z & 0xffff0000u), zb.y, d1);
                    d0 = fmaf(__uint_as_float(u.w << 16), zb.z, d0);
                    d1 = fmaf(__uint_as_float(u.w & 0xffff0000u), zb.w, d1);
                }
                float dot = d0 + d1;
                dot += __shfl_xor(dot, 16, kWave);
                dot += __shfl_xor(dot, 32, kWave);
                if (g == 0) dens[row] = rs + dot;
            }
        }
        if constexpr (OUT) lds_barrier();   // A and den complete
        // ---- z += colsum phi(K) from the 16 row-group sums of the staging
        //      (read again only after the next loop-top barrier)
        if (!GATED && tid < D) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                a0 += zpart[tid][i];
                a1 += zpart[tid][i + 1];
            }
            const float zn = zs[tid] + (a0 + a1);
            zs[tid] = zn;
            const int js = snap_slot(n);
            if (js >= 0) geo.z_snap[(static_cast<size_t>(js) * geo.H + it.h) * D + tid] = zn;
        }

        // ---- this wave's 32 value channels: outputs, then the state update
        // V as B operands (tokens 32 s2 + 8 g .. +7 of value channel 32 w + 16 nb + r),
        // read transposed from its row-major tile; GATED: Ve has the rows
        // scaled by e^{g_c - g} for the state update
        bf16x8 Pb[2][4], Vb[2][2], Ve[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int s = 0; s < 4; ++s) Pb[nb][s] = pack_acc_pair(P[nb][2 * s], P[nb][2 * s + 1]);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                Vb[nb][s2] = tr_operand(Vs, 32 * s2, [&](int aa) { return 32 * w + 16 * nb + 4 * aa; }, lane);
                if constexpr (GATED) {
                    const float4 e0 = *reinterpret_cast<const float4*>(&eks[32 * s2 + 8 * g]);
                    const float4 e1 = *reinterpret_cast<const float4*>(&eks[32 * s2 + 8 * g + 4]);
                    const float ee[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
                    float x[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) x[j] = static_cast<float>(Vb[nb][s2][j]) * ee[j];
                    Ve[nb][s2] = pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
                } else {
                    Ve[nb][s2] = Vb[nb][s2];
                }
            }
        }
#pragma unroll
        for (int m = 0; m < (OUT ? 4 : 0); ++m) {
            f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a = lds8(&fQ[16 * m + r][32 * s + 8 * g]);
                acc[0] = mfma16x16x32(a, Pb[0][s], acc[0]);
                acc[1] = mfma16x16x32(a, Pb[1][s], acc[1]);
            }
            if (GATED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float eg = egs[16 * m + 4 * g + i];
                    acc[0][i] *= eg;
                    acc[1][i] *= eg;
                }
            }
#pragma unroll
            for (int s2 = 0; s2 <= (m >> 1); ++s2) {
                const bf16x8 a = lds8(&As[16 * m + r][32 * s2 + 8 * g]);
                acc[0] = mfma16x16x32(a, Vb[0][s2], acc[0]);
                acc[1] = mfma16x16x32(a, Vb[1][s2], acc[1]);
            }
            // staged in this wave's own 32 columns of V (read into Vb above,
            // by this wave only)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * m + 4 * g + i;
                const float rden = GATED ? 1.f : __builtin_amdgcn_rcpf(dens[row]);
                Vs[row][32 * w + r] = f32_to_bf16_bits(acc[0][i] * rden);
                Vs[row][32 * w + 16 + r] = f32_to_bf16_bits(acc[1][i] * rden);
            }
        }
        if constexpr (OUT) {
            // 16-byte global stores: 64 rows x 4 pieces of this wave's 32 channels
            wave_fence();
#pragma unroll
            for (int pass = 0; pass < C * 4 / kWave; ++pass) {
                const int e = pass * kWave + lane, c8 = 8 * (e & 3);
                if constexpr (!GATED) {   // every store issued: rows past the end write the last row again
                    const int row = min(e >> 2, len - 1);
                    *reinterpret_cast<uint4*>(o + head + static_cast<size_t>(t0 + row) * D + 32 * w + c8) =
                        *reinterpret_cast<const uint4*>(&Vs[row][32 * w + c8]);
                } else if ((e >> 2) < len) {
                    const int row = e >> 2;
                    *reinterpret_cast<uint4*>(o + head + static_cast<size_t>(t0 + row) * D + 32 * w + c8) =
                        *reinterpret_cast<const uint4*>(&Vs[row][32 * w + c8]);
                }
            }
        }
        if (GATED) {
            decay *= egc;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                P[0][t] *= egc;
                P[1][t] *= egc;
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                // (phi(K) or K)^T rows in the permuted order, read transposed
                const bf16x8 a =
                    tr_operand(fK, 32 * s2, [&](int aa) { return 32 * (t >> 1) + 8 * aa + 4 * (t & 1); }, lane);
                P[0][t] = mfma16x16x32(a, Ve[0][s2], P[0][t]);
                P[1][t] = mfma16x16x32(a, Ve[1][s2], P[1][t]);
            }
        }
        const int js = snap_slot(n);
        if (js >= 0) store_P(geo.S_snap + (static_cast<size_t>(js) * geo.H + it.h) * kMat);
    };
    if (n1 > n0) {
        int nstart = n0;
        if constexpr (!GATED) {
            chunk(n0);
            nstart = n0 + 1;
        }
        for (int n = nstart; n < n1; ++n) chunk(n);
    }

    // OUT: final state of the last segment; otherwise the segment's contributions
    float* Sdst = OUT ? (seg == G - 1 && S_out ? S_out + it.state * kMat : nullptr) : ws + ws_dS(slot);
    float* zdst = OUT ? (seg == G - 1 && z_out ? z_out + it.state * D : nullptr) : ws + ws_dz(slot);
    if (Sdst) store_P(Sdst);
    lds_barrier();
    if (GATED) {
        // the segment's total decay in slot 0 of the dz record (z is unused)
        if (!OUT && tid == 0) zdst[0] = decay;
    } else if (zdst && tid < D) {
        zdst[tid] = zs[tid];
    }
}

// Entering states of every segment: P_0 = S0 (or 0), P_{s+1} = P_s + dS_s, and
// the same for z; GATED: P_{s+1} = m_s P_s + dS_s with the segment decay m_s.
// 16 workgroups per head, 4 consecutive floats per thread.  The contributions
// of up to kBatch segments are loaded before any of them is added, so the
// chain of additions waits for one memory latency per batch instead of one
// per segment.
constexpr int kBatch = 8;

template <bool GATED>
__global__ __launch_bounds__(kThreads) void la_combine_kernel(LGeo geo, const float* S0, const float* z0, float* ws) {
    // item: a head (uniform) or a (sequence, head) pair (packed)
    const int item = blockIdx.x >> 4;
    int G;
    size_t slot0, state;
    if (geo.cu == nullptr) {
        if (item >= geo.BH) return;
        G = geo.G;
        slot0 = static_cast<size_t>(item) * G;
        state = item;
    } else {
        if (item >= geo.N * geo.H) return;
        const int sq = item / geo.H, h = item - sq * geo.H;
        G = geo.seg_base[sq + 1] - geo.seg_base[sq];
        if (G < 2 || geo.seg_base[sq + 1] > geo.Gcap) return;   // one segment: the output pass reads S0 itself
        slot0 = static_cast<size_t>(h) * geo.Gcap + geo.seg_base[sq];
        state = item;
    }
    const int part = blockIdx.x & 15;
    const size_t e = (static_cast<size_t>(part) * kThreads + threadIdx.x) * 4;   // < kMat
    float4 run = S0 ? *reinterpret_cast<const float4*>(S0 + state * kMat + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < G; s0 += kBatch) {
        float4 d[kBatch];
        float m[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int s = min(s0 + j, G - 2);   // (G >= 2) clamped: loads past the last map are unused
            d[j] = *reinterpret_cast<const float4*>(ws + ws_dS(slot0 + s) + e);
            m[j] = GATED ? ws[ws_dz(slot0 + s)] : 1.f;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int s = s0 + j;
            if (s < G) {
                *reinterpret_cast<float4*>(ws + ws_P(slot0 + s) + e) = run;
                if (s + 1 < G) {
                    run.x = fmaf(m[j], run.x, d[j].x); run.y = fmaf(m[j], run.y, d[j].y);
                    run.z = fmaf(m[j], run.z, d[j].z); run.w = fmaf(m[j], run.w, d[j].w);
                }
            }
        }
    }
    if (!GATED && part == 0 && threadIdx.x < D) {
        float zr = z0 ? z0[state * D + threadIdx.x] : 0.f;
        for (int s0 = 0; s0 < G; s0 += kBatch) {
            float dz[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) dz[j] = ws[ws_dz(slot0 + min(s0 + j, G - 2)) + threadIdx.x];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int s = s0 + j;
                if (s < G) {
                    ws[ws_zP(slot0 + s) + threadIdx.x] = zr;
                    if (s + 1 < G) zr += dz[j];
                }
            }
        }
    }
}

struct Plan {
    int NC, G, SEGC;
};

// Segments per head so that B*H*G workgroups roughly fill the chip.
Plan make_plan(int BH, int T) {
    Plan p;
    p.NC = (T + C - 1) / C;
    int G = kTargetBlocks / (BH > 0 ? BH : 1);
    if (G < 1) G = 1;
    if (G > p.NC) G = p.NC;
    p.SEGC = (p.NC + G - 1) / G;
    p.G = (p.NC + p.SEGC - 1) / p.SEGC;  // every segment non-empty
    return p;
}

}  // namespace

bool la_mfma_supported(int dtype, int dk, int dv, int chunk) {
    static_assert(C == kMfmaChunk, "the matrix-core kernels share one block length");
    return dtype == kBF16 && dk == D && dv == D && mfma_chunk_ok(chunk);
}

size_t la_mfma_workspace_bytes(int B, int H, int T, int, int, int) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return 0;
    const Plan p = make_plan(BH, T);
    return p.G == 1 ? 0 : static_cast<size_t>(BH) * p.G * kRec * sizeof(float);
}

namespace {

template <bool GATED, bool PACKED>
hipError_t launch_geo(const LGeo& g, long long state_blocks, long long combine_items, long long out_blocks,
                      const void* q, const void* k, const void* v, const float* alpha, const float* S0,
                      const float* z0, void* o, float* S_out, float* z_out, float* ws, hipStream_t stream) {
    if (!grid_fits(state_blocks, kThreads) || !grid_fits(state_blocks > 0 ? combine_items * 16 : 0, kThreads) ||
        !grid_fits(out_blocks, kThreads))
        return hipErrorInvalidConfiguration;
    const u16 *q16 = static_cast<const u16*>(q), *k16 = static_cast<const u16*>(k), *v16 = static_cast<const u16*>(v);
    if (state_blocks > 0) {
        hipLaunchKernelGGL((la_chunked_mfma_kernel<GATED, false, PACKED>), dim3(static_cast<unsigned>(state_blocks)),
                           dim3(kThreads), 0, stream, g, q16, k16, v16, alpha, S0, z0, ws, nullptr, nullptr, nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(la_combine_kernel<GATED>, dim3(static_cast<unsigned>(combine_items) * 16), dim3(kThreads),
                           0, stream, g, S0, z0, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((la_chunked_mfma_kernel<GATED, true, PACKED>), dim3(static_cast<unsigned>(out_blocks)),
                       dim3(kThreads), 0, stream, g, q16, k16, v16, alpha, S0, z0, ws, static_cast<u16*>(o), S_out,
                       z_out);
    return hipGetLastError();
}

template <bool GATED>
hipError_t launch_segmented(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                            const float* S0, const float* z0, void* o, float* S_out, float* z_out, void* workspace,
                            hipStream_t stream) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return hipSuccess;
    const Plan p = make_plan(BH, T);
    LGeo g{};
    g.BH = BH;
    g.T = T;
    g.NC = p.NC;
    g.G = p.G;
    g.SEGC = p.SEGC;
    const long long bh = BH;
    return launch_geo<GATED, false>(g, p.G > 1 ? bh * (p.G - 1) : 0, bh, bh * p.G, q, k, v, alpha, S0, z0, o, S_out,
                                    z_out, static_cast<float*>(workspace), stream);
}

// ---- packed batches: plan on the host from N and Ttot only (the sequence
// lengths stay on the device).  SEGC is chosen so that about kTargetBlocks
// (segment, head) items exist; Gcap bounds the total segment count,
// sum ceil(NC_n / SEGC) <= (Ttot / C + N) / SEGC + N.
struct LVarPlan {
    int SEGC, Gcap;
    size_t table_bytes;
};

LVarPlan make_lvar_plan(int N, int H, int Ttot) {
    LVarPlan p;
    const long long chunks = static_cast<long long>(Ttot) / C + N;
    long long segc = (chunks * H + kTargetBlocks - 1) / kTargetBlocks;
    if (segc < 1) segc = 1;
    p.SEGC = static_cast<int>(segc);
    p.Gcap = static_cast<int>(chunks / segc + N + 1);
    // seg_base, snap_base ([N+1] each), order ([Gcap])
    p.table_bytes = ((2 * (static_cast<size_t>(N) + 1) + p.Gcap) * sizeof(int) + 255) / 256 * 256;
    return p;
}

template <bool GATED>
hipError_t launch_packed(int N, int H, int Ttot, const int* cu, const void* q, const void* k, const void* v,
                         const float* alpha, const float* S0, const float* z0, void* o, float* S_out, float* z_out,
                         int snap, int snap_cap, float* S_snap, float* z_snap, void* workspace, hipStream_t stream) {
    if (N <= 0 || H <= 0) return hipSuccess;
    const LVarPlan p = make_lvar_plan(N, H, Ttot);
    int* tab = static_cast<int*>(workspace);
    LGeo g{};
    g.SEGC = p.SEGC;
    g.cu = cu;
    g.seg_base = tab;
    g.snap_base = tab + (N + 1);
    g.order = tab + 2 * (N + 1);
    g.N = N;
    g.H = H;
    g.Ttot = Ttot;
    g.Gcap = p.Gcap;
    g.snap = S_snap ? snap : 0;
    g.snap_cap = snap_cap;
    g.S_snap = S_snap;
    g.z_snap = z_snap;
    // (segment, head) items, a bound; the extra workgroups exit.  Every grid
    // is checked before the table kernel runs.
    const long long blocks = static_cast<long long>(p.Gcap) * H, items = static_cast<long long>(N) * H;
    if (!grid_fits(blocks, kThreads) || !grid_fits(items * 16, kThreads)) return hipErrorInvalidConfiguration;
    const hipError_t e = launch_varlen_table(N, Ttot, p.SEGC, g.snap, cu, tab, stream, tab + 2 * (N + 1), p.Gcap);
    if (e != hipSuccess) return e;
    float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.table_bytes);
    return launch_geo<GATED, true>(g, blocks, items, blocks, q, k, v, alpha, S0, z0, o, S_out, z_out, ws, stream);
}

}  // namespace

hipError_t launch_la_mfma(int B, int H, int T, const void* q, const void* k, const void* v, const float* S0,
                          const float* z0, void* o, float* S_out, float* z_out, void* workspace, hipStream_t stream) {
    return launch_segmented<false>(B, H, T, q, k, v, nullptr, S0, z0, o, S_out, z_out, workspace, stream);
}

hipError_t launch_gla_mfma(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                           const float* S0, void* o, float* S_out, void* workspace, hipStream_t stream) {
    return launch_segmented<true>(B, H, T, q, k, v, alpha, S0, nullptr, o, S_out, nullptr, workspace, stream);
}

size_t la_mfma_varlen_workspace_bytes(int N, int H, int Ttot) {
    if (N <= 0 || H <= 0) return 0;
    const LVarPlan p = make_lvar_plan(N, H, Ttot);
    return p.table_bytes + static_cast<size_t>(H) * p.Gcap * kRec * sizeof(float);
}

hipError_t launch_la_mfma_varlen(bool gated, int N, int H, int Ttot, const int* cu, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* S0, const float* z0, void* o,
                                 float* S_out, float* z_out, int snap, int snap_cap, float* S_snap, float* z_snap,
                                 void* workspace, hipStream_t stream) {
    return gated ? launch_packed<true>(N, H, Ttot, cu, q, k, v, alpha, S0, nullptr, o, S_out, nullptr, snap, snap_cap,
                                       S_snap, nullptr, workspace, stream)
                 : launch_packed<false>(N, H, Ttot, cu, q, k, v, nullptr, S0, z0, o, S_out, z_out, snap, snap_cap,
                                        S_snap, z_snap, workspace, stream);
}

}  // namespace la

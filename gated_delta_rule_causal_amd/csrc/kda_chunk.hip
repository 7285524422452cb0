// Chunked Kimi Delta Attention (per-channel decay) on the matrix cores, as
// two kernels: a fully parallel pass that turns every chunk of 64 tokens into
// the tiles of its affine state map, and a scan that runs the chunks of a
// head in order, one workgroup per 16 value channels.
//
// Source: page "Linear attention and hybrids", section "Delta rule and Gated
// DeltaNet": KDA replaces the scalar gate of the Gated DeltaNet equation by
// Diag(alpha_t), acting on the key side of S (d_v x d_k):
//     S_t = S_{t-1} Diag(alpha_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t
// The chunk form (not printed on the page) follows by unrolling the equation
// inside a chunk with entry state S0, g_r = sum_{s<=r} log alpha_s per
// channel (chunk-local) and Gamma_rj = e^{g_r - g_j} elementwise:
//     L_rj = beta_r sum_c k_r[c] Gamma_rj[c] k_j[c]   (j < r)
//     A_rj = sum_c q_r[c] Gamma_rj[c] k_j[c]            (j <= r)
//     W = (I + L)^{-1} diag(beta) (K * e^g),  Ut = (I + L)^{-1} diag(beta) V
//     U = Ut - W S0^T,  O = (Q * e^g) S0^T + A U
//     S_c = S0 Diag(e^{g_c}) + U^T (K * e^{g_c - g})
// With the transposed state P = S^T (d_k x d_v) every value channel (column
// of P) evolves on its own: P <- Diag(e^{g_c}) P + Kt^T (Ut - W P), which is
// what lets the scan split a head over workgroups.
//
// Tile pass (one workgroup per chunk, 256 threads, two workgroups per CU).
// g by sums over 4-token blocks plus their exclusive prefix; the decayed products L and A as MFMA products of scaled copies
// K * e^{g - g_m}, K * e^{g_m - g}, Q * e^{g - g_m} (g_m: the chunk's middle
// token, so every factor lies within e^{+-80} whenever the chunk's decay span
// is at most 80 in every channel; chunks with a larger span take an exact
// path with one exponential per term); then T = (I + L)^{-1} on the matrix
// cores (the four diagonal 16x16 blocks by the nilpotent product form in
// registers, the blocks below them as three independent MFMA chains) and W,
// Ut as plain products with T.  Per chunk it writes W, Q * e^g (64 x 128),
// A (64 x 64), (K * e^{g_c - g})^T and Ut^T (128 x 64) in bf16 and e^{g_c}
// (128 fp32): 74 240 bytes.
//
// Scan (one workgroup per (head, 16 value channels), 4 waves).  Wave w owns
// token rows 16w.. of X = W P, U and O and key rows 32w.. of P (fp32 in its
// accumulators); P^T and U^T (bf16) are shared through LDS, two barriers per
// chunk.  The tiles of chunks n+1 and n+2 are loaded while chunk n runs, each
// wave-wide load one contiguous run of the record.  The eight
// workgroups of a head take block indices eight apart, so they run on one XCD
// and read each chunk's tiles from that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int C = 64;           // tokens per chunk
constexpr int D = 128;          // d_k = d_v
constexpr int LDB = D + 8;      // bf16 row stride of the tile pass's LDS tiles
constexpr int LDT = C + 8;      // bf16 row stride of the 64-wide T tile
constexpr int kTileThreads = 256;
constexpr int kScanThreads = 256;
constexpr float kMaxSpan = 80.f;   // largest decay span of the factored fast path

// per-chunk record (bytes)
constexpr size_t oW = 0;              // W       [64][128] bf16, fragment order (frag8)
constexpr size_t oQ = 16384;          // Q e^g   [64][128] bf16, frag8
constexpr size_t oA = 32768;          // A       [64][64]  bf16 (zero above the diagonal), frag8
constexpr size_t oKt = 40960;         // Kt^T    [128][64] bf16, frag8
constexpr size_t oUt = 57344;         // Ut^T    [128][64] bf16, frag4
constexpr size_t oDec = 73728;        // e^{g_c} [128] fp32
constexpr size_t kRecord = 74240;

// The bf16 tiles of the record are stored in the order the scan's MFMA
// operands read them, so each wave-wide load is one contiguous run (1 KiB for
// a 16-byte piece per lane) instead of 16 half cache lines.
//   frag8: 16 x 32 blocks (row-block major), inside a block lane (r, g) =
//          16 g + r holds row r, columns 8g .. 8g+7 (16 bytes);
//   frag4: 16 x 16 blocks, lane 16 g + r holds row r, columns 4g .. 4g+3.
// Element offsets for a tile with `ncols` columns:
__host__ __device__ constexpr int frag8(int row, int col, int ncols) {
    return ((((row >> 4) * (ncols >> 5) + (col >> 5)) * 64 + ((col >> 3) & 3) * 16 + (row & 15)) << 3) + (col & 7);
}
__host__ __device__ constexpr int frag4(int row, int col, int ncols) {
    return ((((row >> 4) * (ncols >> 4) + (col >> 4)) * 64 + ((col >> 2) & 3) * 16 + (row & 15)) << 2) + (col & 3);
}
static_assert(frag8(17, 40, 128) == ((4 + 1) * 64 + 16 + 1) * 8, "frag8 block order");
static_assert(frag4(17, 21, 64) == ((4 + 1) * 64 + 16 + 1) * 4 + 1, "frag4 block order");

__device__ __forceinline__ float bf(u16 b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16_bits(a)) | (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ======================================================== geometry
// Where the chunks of a call live: a uniform batch (BH heads of T tokens, NC
// chunks each, record of chunk n of head bh at bh * NC + n) or a packed batch
// (cu != nullptr: N sequences back to back in every one of H heads of Ttot
// tokens; chunk_base[n] = chunks of the sequences before n, built on the
// device; the record of chunk j of sequence n in head h at
// h * cap + chunk_base[n] + j, cap bounding the total chunk count).
struct KGeo {
    int BH, T, NC;
    const int* cu;
    const int* chunk_base;
    const int* snap_base;
    const int* seq_order;   // packed: sequences longest first (the scan takes them in that order)
    int N, H, Ttot, cap;
    int snap, snap_cap;   // snapshots of P after every `snap` tokens (a multiple of C), slots below snap_cap
    float* S_snap;
};

__device__ __forceinline__ int kclamp(int t, int Ttot) { return t < 0 ? 0 : t > Ttot ? Ttot : t; }

// Sequence of global chunk gc of a packed batch (chunk_base non-decreasing,
// chunk_base[0] = 0 <= gc < chunk_base[N]).
__device__ __forceinline__ int chunk_seq(const KGeo& g, int gc) {
    int lo = 0, hi = g.N;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (g.chunk_base[mid] <= gc) lo = mid; else hi = mid;
    }
    return lo;
}

// ======================================================== tile pass
// LDS of the tile pass, about 79 KiB so that two workgroups share a CU (one
// loads its chunk while the other computes).  The raw k, v, q pieces and the
// decay sums stay in the registers of the thread that loaded them; the three
// scaled copies, then the exact path's g and k, then the right-hand sides of
// W and Ut take turns in one region.
struct TileSmem {
    union {
        struct {
            u16 Kp[C][LDB];     // k e^{g - g_m}
            u16 Km[C][LDB];     // k e^{g_m - g}
            u16 Qp[C][LDB];     // q e^{g - g_m}
        } f;                    // fast path, L and A
        struct {
            float g[C][D];      // chunk-local cumulative log decay
            u16 K[C][LDB];      // raw k
        } x;                    // exact path, L and A
        struct {
            u16 Xw[C][LDB];     // beta k e^g
            u16 Xv[C][LDB];     // beta v
            u16 Kc[C][LDB];     // k e^{g_c - g}
        } r;                    // right-hand sides and (K e^{g_c - g})^T
        float part[16][D];      // log-decay sums of 4-token blocks, then their exclusive prefix
    };
    u16 Tm[C][LDT];       // T = (I + L)^{-1} (bf16, lower triangular)
    float L[C][C + 4];    // beta_r L_rj (strictly lower)
    float beta[C];
    float g0[D], gm[D], gc[D];   // g at tokens 0, C/2 - 1 and C - 1
    int span;             // max decay span over channels (float bits, >= 0)
};
static_assert(sizeof(TileSmem) <= 80 * 1024, "two tile workgroups per CU");

__global__ __launch_bounds__(kTileThreads) void kda_tile_kernel(KGeo geo, const u16* __restrict__ q,
                                                                const u16* __restrict__ k,
                                                                const u16* __restrict__ v,
                                                                const float* __restrict__ alpha,
                                                                const float* __restrict__ beta,
                                                                unsigned char* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) TileSmem sm;
    int len;
    size_t row0;   // first token row of the chunk
    unsigned char* rec;
    if (geo.cu == nullptr) {
        const int bh = blockIdx.x / geo.NC, n = blockIdx.x % geo.NC;
        if (bh >= geo.BH) return;
        len = min(C, geo.T - n * C);
        row0 = static_cast<size_t>(bh) * geo.T + n * C;
        rec = ws + (static_cast<size_t>(bh) * geo.NC + n) * kRecord;
    } else {
        const int h = blockIdx.x % geo.H, gc = blockIdx.x / geo.H;
        if (gc >= geo.chunk_base[geo.N] || gc >= geo.cap) return;
        const int sq = chunk_seq(geo, gc), j = gc - geo.chunk_base[sq];
        const int t0 = kclamp(geo.cu[sq], geo.Ttot), t1 = kclamp(geo.cu[sq + 1], geo.Ttot);
        len = min(C, (t1 > t0 ? t1 - t0 : 0) - j * C);
        if (len <= 0) return;   // an empty sequence counts one chunk in the table and has none
        row0 = static_cast<size_t>(h) * geo.Ttot + t0 + static_cast<size_t>(j) * C;
        rec = ws + (static_cast<size_t>(h) * geo.cap + gc) * kRecord;
    }
    const int tid = threadIdx.x;

    // Thread (tb, cg) owns tokens 4 tb .. 4 tb + 3 and channels 8 cg .. 8 cg + 7
    // of every per-token tile: 16 threads cover one 256-byte row of k, v, q.
    const int tb = tid >> 4, c0 = (tid & 15) * 8;
    uint4 kr[4], vr[4], qr[4];
    float g[4][8];   // running log decay of the owned tokens (local sums first)
    if (tid == 0) sm.span = 0;
    {
        float4 al[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // rows past the sequence: alpha = 1, k = v = q = 0
            const int t = 4 * tb + j;
            al[j][0] = al[j][1] = make_float4(1.f, 1.f, 1.f, 1.f);
            kr[j] = vr[j] = qr[j] = make_uint4(0, 0, 0, 0);
            if (t < len) {
                al[j][0] = *reinterpret_cast<const float4*>(alpha + (row0 + t) * D + c0);
                al[j][1] = *reinterpret_cast<const float4*>(alpha + (row0 + t) * D + c0 + 4);
                const size_t gi = (row0 + t) * D + c0;
                kr[j] = *reinterpret_cast<const uint4*>(k + gi);
                vr[j] = *reinterpret_cast<const uint4*>(v + gi);
                qr[j] = *reinterpret_cast<const uint4*>(q + gi);
            }
        }
        if (tid < C) sm.beta[tid] = tid < len ? beta[row0 + tid] : 0.f;
        float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float la[8] = {__logf(al[j][0].x), __logf(al[j][0].y), __logf(al[j][0].z), __logf(al[j][0].w),
                                 __logf(al[j][1].x), __logf(al[j][1].y), __logf(al[j][1].z), __logf(al[j][1].w)};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                run[i] += la[i];
                g[j][i] = run[i];
            }
            if (tb == 0 && j == 0) {
                *reinterpret_cast<float4*>(&sm.g0[c0]) = make_float4(la[0], la[1], la[2], la[3]);
                *reinterpret_cast<float4*>(&sm.g0[c0 + 4]) = make_float4(la[4], la[5], la[6], la[7]);
            }
        }
        *reinterpret_cast<float4*>(&sm.part[tb][c0]) = make_float4(run[0], run[1], run[2], run[3]);
        *reinterpret_cast<float4*>(&sm.part[tb][c0 + 4]) = make_float4(run[4], run[5], run[6], run[7]);
    }
    __syncthreads();
    if (tid < D) {   // exclusive prefix of the 16 block sums, one channel per thread; g_m, g_c, e^{g_c}, span
        float acc = 0.f, gmid = 0.f;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            if (b == C / 2 / 4) gmid = acc;   // blocks of tokens 0 .. C/2 - 1
            const float x = sm.part[b][tid];
            sm.part[b][tid] = acc;
            acc += x;
        }
        sm.gm[tid] = gmid;
        sm.gc[tid] = acc;
        reinterpret_cast<float*>(rec + oDec)[tid] = __expf(acc);
        // largest span of the two half-chunks over the channels: one atomic per wave
        float sp = fmaxf(fmaxf(sm.g0[tid] - gmid, gmid - acc), 0.f);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) sp = fmaxf(sp, __shfl_xor(sp, off, kWave));
        if ((tid & 63) == 0) atomicMax(&sm.span, __float_as_int(sp));
    }
    __syncthreads();
    const bool fast = __int_as_float(sm.span) <= kMaxSpan;
    float gmv[8], gcv[8];
    {
        const float4 p0 = *reinterpret_cast<const float4*>(&sm.part[tb][c0]);
        const float4 p1 = *reinterpret_cast<const float4*>(&sm.part[tb][c0 + 4]);
        const float pre[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) g[j][i] += pre[i];
        const float4 m0 = *reinterpret_cast<const float4*>(&sm.gm[c0]);
        const float4 m1 = *reinterpret_cast<const float4*>(&sm.gm[c0 + 4]);
        const float4 e0 = *reinterpret_cast<const float4*>(&sm.gc[c0]);
        const float4 e1 = *reinterpret_cast<const float4*>(&sm.gc[c0 + 4]);
        const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        const float cv[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            gmv[i] = mv[i];
            gcv[i] = cv[i];
        }
    }
    __syncthreads();   // every thread has read its block prefix: the region now takes the tiles

    // ---- elementwise: Q e^g to the record; the scaled copies (fast path) or
    // g and raw k (exact path) into LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * tb + j;
        float kv[8], qv[8];
        unpack8(kr[j], kv);
        unpack8(qr[j], qv);
        float qe[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qe[i] = qv[i] * __expf(g[j][i]);
        *reinterpret_cast<bf16x8*>(rec + oQ + static_cast<size_t>(frag8(t, c0, D)) * 2) =
            pack8(qe[0], qe[1], qe[2], qe[3], qe[4], qe[5], qe[6], qe[7]);
        if (fast) {
            float kp[8], km[8], qp[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float up = __expf(g[j][i] - gmv[i]);
                kp[i] = kv[i] * up;
                km[i] = kv[i] * __expf(gmv[i] - g[j][i]);
                qp[i] = qv[i] * up;
            }
            *reinterpret_cast<bf16x8*>(&sm.f.Kp[t][c0]) = pack8(kp[0], kp[1], kp[2], kp[3], kp[4], kp[5], kp[6], kp[7]);
            *reinterpret_cast<bf16x8*>(&sm.f.Km[t][c0]) = pack8(km[0], km[1], km[2], km[3], km[4], km[5], km[6], km[7]);
            *reinterpret_cast<bf16x8*>(&sm.f.Qp[t][c0]) = pack8(qp[0], qp[1], qp[2], qp[3], qp[4], qp[5], qp[6], qp[7]);
        } else {
            *reinterpret_cast<float4*>(&sm.x.g[t][c0]) = make_float4(g[j][0], g[j][1], g[j][2], g[j][3]);
            *reinterpret_cast<float4*>(&sm.x.g[t][c0 + 4]) = make_float4(g[j][4], g[j][5], g[j][6], g[j][7]);
            *reinterpret_cast<uint4*>(&sm.x.K[t][c0]) = kr[j];
        }
    }
    __syncthreads();

    // ---- L (beta-scaled, strictly lower) into LDS, A (lower incl. diagonal) to the record
    u16* Arec = reinterpret_cast<u16*>(rec + oA);
    if (fast) {
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15, gg = lane >> 4;
        // 10 lower tile pairs (I >= J) x {L, A}: wave w takes items w, w+4, ...
        // A is formed transposed (K e^{g_m - g} times Q e^{g - g_m}) so each lane
        // holds 4 consecutive columns of one row: 8-byte stores into the record.
        for (int item = w; item < 20; item += 4) {
            const int p = item >> 1;
            const bool isA = item & 1;
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= p) ++I;
            const int J = p - I * (I + 1) / 2;
            bf16x8 xa[4], xb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                xa[s] = lds_bf16x8(isA ? &sm.f.Km[16 * J + r][32 * s + 8 * gg] : &sm.f.Kp[16 * I + r][32 * s + 8 * gg]);
                xb[s] = lds_bf16x8(isA ? &sm.f.Qp[16 * I + r][32 * s + 8 * gg] : &sm.f.Km[16 * J + r][32 * s + 8 * gg]);
            }
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma16x16x32(xa[s], xb[s], acc);
            if (isA) {
                // lane holds A[row = 16 I + r][cols 16 J + 4 gg .. +3]
                const int row = 16 * I + r, col = 16 * J + 4 * gg;
                float a4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a4[i] = col + i <= row ? acc[i] : 0.f;
                *reinterpret_cast<uint2*>(Arec + frag8(row, col, C)) = make_uint2(pack2(a4[0], a4[1]), pack2(a4[2], a4[3]));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * I + 4 * gg + i, col = 16 * J + r;
                    sm.L[row][col] = col < row ? sm.beta[row] * acc[i] : 0.f;
                }
            }
        }
    } else {
        // exact path: one exponential per term (raw q read from memory: rows
        // past the sequence are zero)
        for (int e = tid; e < C * C; e += kTileThreads) {
            const int row = e / C, col = e % C;
            float sl = 0.f, sa = 0.f;
            if (col <= row) {
                const u16* qrow = q + (row0 + min(row, len - 1)) * D;
                const float qs = row < len ? 1.f : 0.f;
                for (int c = 0; c < D; ++c) {
                    const float f = __expf(sm.x.g[row][c] - sm.x.g[col][c]) * bf(sm.x.K[col][c]);
                    sl = fmaf(bf(sm.x.K[row][c]), f, sl);
                    sa = fmaf(qs * bf(qrow[c]), f, sa);
                }
            }
            sm.L[row][col] = col < row ? sm.beta[row] * sl : 0.f;
            Arec[frag8(row, col, C)] = f32_to_bf16_bits(col <= row ? sa : 0.f);
        }
    }
    // the six 16x16 tiles above the diagonal tiles of A are zero (8-byte stores)
    {
        const int lane = tid & 63, wv = tid >> 6;
        for (int blk = wv; blk < 6; blk += 4) {
            const int I = blk < 3 ? 0 : blk < 5 ? 1 : 2, J = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
            *reinterpret_cast<uint2*>(Arec + frag8(16 * I + (lane & 15), 16 * J + 4 * (lane >> 4), C)) = make_uint2(0, 0);
        }
    }
    __syncthreads();

    // ---- T = (I + L)^{-1} on the matrix cores (L fp32 in LDS, beta-scaled,
    // strictly lower), then W = T diag(beta) (K e^g) and Ut = T diag(beta) V as
    // plain products.  The scaled copies are no longer read: the two
    // right-hand sides and K e^{g_c - g} take their place.
    u16 (*Tm)[LDT] = sm.Tm;
    u16 (*Xw)[LDB] = sm.r.Xw;
    u16 (*Xv)[LDB] = sm.r.Xv;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15, gg = lane >> 4;
    {
        // diagonal block w: N = -L_ww and its transpose, both in the accumulator layout
        f32x4 N, Nt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int a_ = 16 * w + 4 * gg + i, b_ = 16 * w + r;
            N[i] = r < 4 * gg + i ? -sm.L[a_][b_] : 0.f;
            Nt[i] = 4 * gg + i < r ? -sm.L[b_][a_] : 0.f;
        }
        const f32x4 Tb = unit_lower_inverse(N, Nt, r, gg);
#pragma unroll
        for (int i = 0; i < 4; ++i) Tm[16 * w + 4 * gg + i][16 * w + r] = f32_to_bf16_bits(Tb[i]);
        // blocks (0,1) and (2,3) above the diagonal are read by 32-wide slices
        if (w < 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Tm[32 * w + 4 * gg + i][32 * w + 16 + r] = 0;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // from the pieces this thread loaded
        const int t = 4 * tb + j;
        const float bt = sm.beta[t];
        float kx[8], vx[8];
        unpack8(kr[j], kx);
        unpack8(vr[j], vx);
        float xw[8], xv[8], xk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xw[i] = bt * kx[i] * __expf(g[j][i]);
            xv[i] = bt * vx[i];
            xk[i] = kx[i] * __expf(gcv[i] - g[j][i]);
        }
        *reinterpret_cast<bf16x8*>(&Xw[t][c0]) = pack8(xw[0], xw[1], xw[2], xw[3], xw[4], xw[5], xw[6], xw[7]);
        *reinterpret_cast<bf16x8*>(&Xv[t][c0]) = pack8(xv[0], xv[1], xv[2], xv[3], xv[4], xv[5], xv[6], xv[7]);
        *reinterpret_cast<bf16x8*>(&sm.r.Kc[t][c0]) = pack8(xk[0], xk[1], xk[2], xk[3], xk[4], xk[5], xk[6], xk[7]);
    }
    __syncthreads();
    // (K e^{g_c - g})^T: a transposed read gives lane (r, g) 8 consecutive
    // tokens of one channel, one 16-byte piece of the record's [128][64] tile
    {
        u16* Kt = reinterpret_cast<u16*>(rec + oKt);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int item = 4 * w + j, dt = item >> 1, s = item & 1;   // 16 channels x 32 tokens
            const bf16x8 x = tr_operand(sm.r.Kc, 32 * s, [&](int aa) { return 16 * dt + 4 * aa; }, lane);
            *reinterpret_cast<bf16x8*>(Kt + frag8(16 * dt + r, 32 * s + 8 * gg, C)) = x;
        }
    }
    // below-diagonal blocks of T, T_ij = T_ii sum_{j<=k<i} (-L_ik) T_kj, as
    // three independent chains on waves 0-2 (T_10, T_20, T_30; T_21, T_31; T_32)
    {
        auto nl = [&](int i, int j) {   // A operand of -L_ij (bf16)
            const float4 x = *reinterpret_cast<const float4*>(&sm.L[16 * i + r][16 * j + 4 * gg]);
            return to_bf16x4(f32x4{-x.x, -x.y, -x.z, -x.w});
        };
        auto ta = [&](int i) { return lds_short4(&Tm[16 * i + r][16 * i + 4 * gg]); };
        auto tb = [&](int i) {          // B operand of T_ii
            short4v x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = static_cast<short>(Tm[16 * i + 4 * gg + e][16 * i + r]);
            return x;
        };
        auto put = [&](int i, int j, short4v t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[16 * i + 4 * gg + e][16 * j + r] = static_cast<u16>(t[e]);
        };
        auto solve = [&](short4v a, f32x4 y) { return to_bf16x4(mfma16x16x16(a, to_bf16x4(y), zero4())); };
        if (w == 0) {
            const short4v t00 = tb(0);
            const short4v l10 = nl(1, 0), l20 = nl(2, 0), l21 = nl(2, 1), l30 = nl(3, 0), l31 = nl(3, 1), l32 = nl(3, 2);
            const short4v a1 = ta(1), a2 = ta(2), a3 = ta(3);
            const short4v t10 = solve(a1, mfma16x16x16(l10, t00, zero4()));
            const short4v t20 = solve(a2, mfma16x16x16(l21, t10, mfma16x16x16(l20, t00, zero4())));
            const short4v t30 =
                solve(a3, mfma16x16x16(l32, t20, mfma16x16x16(l31, t10, mfma16x16x16(l30, t00, zero4()))));
            put(1, 0, t10);
            put(2, 0, t20);
            put(3, 0, t30);
        } else if (w == 1) {
            const short4v t11 = tb(1);
            const short4v l21 = nl(2, 1), l31 = nl(3, 1), l32 = nl(3, 2);
            const short4v a2 = ta(2), a3 = ta(3);
            const short4v t21 = solve(a2, mfma16x16x16(l21, t11, zero4()));
            const short4v t31 = solve(a3, mfma16x16x16(l32, t21, mfma16x16x16(l31, t11, zero4())));
            put(2, 1, t21);
            put(3, 1, t31);
        } else if (w == 2) {
            const short4v t22 = tb(2);
            const short4v l32 = nl(3, 2), a3 = ta(3);
            put(3, 2, solve(a3, mfma16x16x16(l32, t22, zero4())));
        }
    }
    __syncthreads();
    // W^T = Xw^T T^T and Ut = T Xv on the matrix cores; wave w takes the
    // 16-token column tile w of W^T and the 16-token row tile w of Ut.
    // T is lower triangular: slices s > w/2 of its rows are zero.
    {
        const int tt = w;
        u16* Wrec = reinterpret_cast<u16*>(rec + oW);
        u16* Urec = reinterpret_cast<u16*>(rec + oUt);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            f32x4 accw = zero4(), accu = zero4();
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                if (s > (tt >> 1)) break;
                const bf16x8 trow = lds_bf16x8(&Tm[16 * tt + r][32 * s + 8 * gg]);
                // W^T[d][tok] = sum_j Xw[j][d] T[tok][j]: A = Xw^T (transposed read), B = T rows
                const bf16x8 xw = tr_operand(Xw, 32 * s, [&](int aa) { return 16 * dt + 4 * aa; }, lane);
                accw = mfma16x16x32(xw, trow, accw);
                // Ut[tok][v] = sum_j T[tok][j] Xv[j][v]: A = T rows, B = Xv (transposed read)
                const bf16x8 xv = tr_operand(Xv, 32 * s, [&](int aa) { return 16 * dt + 4 * aa; }, lane);
                accu = mfma16x16x32(trow, xv, accu);
            }
            // accw: lane holds W[tok = 16 tt + r][d = 16 dt + 4 gg .. +3];
            // accu: lane holds Ut[tok = 16 tt + 4 gg .. +3][v = 16 dt + r] = Ut^T[v][tok ..]
            *reinterpret_cast<uint2*>(Wrec + frag8(16 * tt + r, 16 * dt + 4 * gg, D)) =
                make_uint2(pack2(accw[0], accw[1]), pack2(accw[2], accw[3]));
            *reinterpret_cast<uint2*>(Urec + frag4(16 * dt + r, 16 * tt + 4 * gg, C)) =
                make_uint2(pack2(accu[0], accu[1]), pack2(accu[2], accu[3]));
        }
    }
}

// ======================================================== scan
struct ScanSmem {
    u16 PT[16][D + 8];    // P^T (bf16): [value column][key channel]
    u16 UT[16][C + 8];    // U^T (bf16): [value column][token]
    u16 Os[4][16][20];    // each wave's 16 x 16 output tile, turned into row pieces
};

struct ChunkOps {
    uint4 W[4], Q[4], A[2], K[2][2];
    uint2 U;
    float4 d[2];
};

__device__ __forceinline__ void load_ops(ChunkOps& op, const unsigned char* rec, int w, int cb, int r, int gg) {
    const u16* W = reinterpret_cast<const u16*>(rec + oW);
    const u16* Q = reinterpret_cast<const u16*>(rec + oQ);
    const u16* A = reinterpret_cast<const u16*>(rec + oA);
    const u16* K = reinterpret_cast<const u16*>(rec + oKt);
    const u16* U = reinterpret_cast<const u16*>(rec + oUt);
    const float* d = reinterpret_cast<const float*>(rec + oDec);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        op.W[s] = *reinterpret_cast<const uint4*>(W + frag8(16 * w + r, 32 * s + 8 * gg, D));
        op.Q[s] = *reinterpret_cast<const uint4*>(Q + frag8(16 * w + r, 32 * s + 8 * gg, D));
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        op.A[s] = *reinterpret_cast<const uint4*>(A + frag8(16 * w + r, 32 * s + 8 * gg, C));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            op.K[mt][s] = *reinterpret_cast<const uint4*>(K + frag8(32 * w + 16 * mt + r, 32 * s + 8 * gg, C));
    }
    op.U = *reinterpret_cast<const uint2*>(U + frag4(16 * cb + r, 16 * w + 4 * gg, C));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) op.d[mt] = *reinterpret_cast<const float4*>(d + 32 * w + 16 * mt + 4 * gg);
}

__device__ __forceinline__ void scan_chunk(ScanSmem& sm, const ChunkOps& op, f32x4 (&P)[2], int w, int r, int gg,
                                           u16* __restrict__ o, size_t orow, int len, int cb) {
    // X = W P and Q e^g P from P^T (all key channels)
    f32x4 X = zero4(), O = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 p = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.PT[r][32 * s + 8 * gg]));
        X = mfma16x16x32(as_bf16x8(op.W[s]), p, X);
        O = mfma16x16x32(as_bf16x8(op.Q[s]), p, O);
    }
    // U = Ut - X for tokens 16w + 4gg + i, value column r
    const float ut[4] = {__uint_as_float(op.U.x << 16), __uint_as_float(op.U.x & 0xffff0000u),
                         __uint_as_float(op.U.y << 16), __uint_as_float(op.U.y & 0xffff0000u)};
    float u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = ut[i] - X[i];
    *reinterpret_cast<uint2*>(&sm.UT[r][16 * w + 4 * gg]) = make_uint2(pack2(u[0], u[1]), pack2(u[2], u[3]));
    lds_barrier();
    bf16x8 ub[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) ub[s] = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.UT[r][32 * s + 8 * gg]));
    // P <- Diag(e^{g_c}) P + Kt^T U (key rows 32w + 16mt + 4gg + i): first,
    // since the next chunk waits for P^T
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const float dd[4] = {op.d[mt].x, op.d[mt].y, op.d[mt].z, op.d[mt].w};
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = dd[i] * P[mt][i];
#pragma unroll
        for (int s = 0; s < 2; ++s) acc = mfma16x16x32(as_bf16x8(op.K[mt][s]), ub[s], acc);
        P[mt] = acc;
        *reinterpret_cast<uint2*>(&sm.PT[r][32 * w + 16 * mt + 4 * gg]) =
            make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]));
    }
    // O += A U.  The lane holds O[16w + 4gg + i][r]; the wave's tile goes
    // through its own LDS block so each lane stores 4 columns of one row.
#pragma unroll
    for (int s = 0; s < 2; ++s) O = mfma16x16x32(as_bf16x8(op.A[s]), ub[s], O);
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.Os[w][4 * gg + i][r] = f32_to_bf16_bits(O[i]);
    wave_fence();
    const int lane = 16 * gg + r, orw = lane >> 2, ocl = 4 * (lane & 3);
    const uint2 orow_bits = *reinterpret_cast<const uint2*>(&sm.Os[w][orw][ocl]);
    lds_barrier();
    if (16 * w + orw < len)
        *reinterpret_cast<uint2*>(o + (orow + 16 * w + orw) * D + 16 * cb + ocl) = orow_bits;
}

__global__ __launch_bounds__(kScanThreads) void kda_scan_kernel(KGeo geo, const unsigned char* __restrict__ ws,
                                                                const float* S0, u16* __restrict__ o, float* S_out) {
    __shared__ __attribute__((aligned(16))) ScanSmem sm;
    // the 8 column blocks of a head take block indices 8 apart (one XCD)
    const int i = blockIdx.x;
    const int bh = (i >> 6) * 8 + (i & 7);   // head (uniform) or sequence * H + head (packed)
    const int cb = (i >> 3) & 7;
    int T, NC, hh = 0, snap0 = 0;
    const unsigned char* rec0;
    size_t orow, state = bh;   // index of the (sequence, head) state in S0 / S_out
    if (geo.cu == nullptr) {
        if (bh >= geo.BH) return;
        T = geo.T;
        NC = geo.NC;
        rec0 = ws + static_cast<size_t>(bh) * NC * kRecord;
        orow = static_cast<size_t>(bh) * T;
    } else {
        if (bh >= geo.N * geo.H) return;
        const int si = bh / geo.H;
        hh = bh - si * geo.H;
        const int sq = geo.seq_order ? geo.seq_order[si] : si;
        state = static_cast<size_t>(sq) * geo.H + hh;
        const int t0 = kclamp(geo.cu[sq], geo.Ttot), t1 = kclamp(geo.cu[sq + 1], geo.Ttot);
        T = t1 > t0 ? t1 - t0 : 0;
        // a table that is not non-decreasing can promise more chunks than the
        // workspace holds: those are never read
        const int base = geo.chunk_base[sq];
        NC = min((T + C - 1) / C, min(geo.chunk_base[sq + 1], geo.cap) - base);
        if (NC < 0) NC = 0;
        rec0 = ws + (static_cast<size_t>(hh) * geo.cap + base) * kRecord;
        orow = static_cast<size_t>(hh) * geo.Ttot + t0;
        snap0 = geo.snap_base ? geo.snap_base[sq] : 0;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, gg = lane >> 4;
    const size_t sbase = state * D * D;
    // P[key c][value col] = S0[col][c]: this lane holds c = 32w + 16mt + 4gg + i, col = 16cb + r
    f32x4 P[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (S0) x = *reinterpret_cast<const float4*>(S0 + sbase + static_cast<size_t>(16 * cb + r) * D + 32 * w +
                                                      16 * mt + 4 * gg);
        P[mt] = f32x4{x.x, x.y, x.z, x.w};
        *reinterpret_cast<uint2*>(&sm.PT[r][32 * w + 16 * mt + 4 * gg]) =
            make_uint2(pack2(x.x, x.y), pack2(x.z, x.w));
    }
    __syncthreads();
    // tiles of chunks n+1 and n+2 are in flight while chunk n runs (three
    // register sets in rotation; indices past the end reload the last chunk)
    ChunkOps a, b, c;
    auto rec = [&](int m) { return rec0 + static_cast<size_t>(min(m, NC - 1)) * kRecord; };
    auto run = [&](const ChunkOps& op, int m) {
        scan_chunk(sm, op, P, w, r, gg, o, orow + static_cast<size_t>(m) * C, min(C, T - m * C), cb);
        // packed batches: the state after every geo.snap tokens
        const int end = (m + 1) * C;
        if (geo.snap > 0 && end <= T && end % geo.snap == 0) {
            const int js = snap0 + end / geo.snap - 1;
            if (js < geo.snap_cap) {
                float* dst = geo.S_snap + (static_cast<size_t>(js) * geo.H + hh) * D * D;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    *reinterpret_cast<float4*>(dst + static_cast<size_t>(16 * cb + r) * D + 32 * w + 16 * mt +
                                               4 * gg) = make_float4(P[mt][0], P[mt][1], P[mt][2], P[mt][3]);
            }
        }
    };
    if (NC > 0) {
        load_ops(a, rec(0), w, cb, r, gg);
        load_ops(b, rec(1), w, cb, r, gg);
    }
    int n = 0;
    for (; n + 3 <= NC; n += 3) {   // no branches around the chunks: the wait counts stay exact
        load_ops(c, rec(n + 2), w, cb, r, gg);
        run(a, n);
        load_ops(a, rec(n + 3), w, cb, r, gg);
        run(b, n + 1);
        load_ops(b, rec(n + 4), w, cb, r, gg);
        run(c, n + 2);
    }
    if (n < NC) run(a, n);
    if (n + 1 < NC) run(b, n + 1);
    if (S_out) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            *reinterpret_cast<float4*>(S_out + sbase + static_cast<size_t>(16 * cb + r) * D + 32 * w + 16 * mt +
                                       4 * gg) = make_float4(P[mt][0], P[mt][1], P[mt][2], P[mt][3]);
    }
}

}  // namespace

bool kda_mfma_supported(int dtype, int dk, int dv, int chunk) {
    static_assert(C == kMfmaChunk, "the matrix-core kernels share one block length");
    return dtype == kBF16 && dk == D && dv == D && mfma_chunk_ok(chunk);
}

size_t kda_mfma_workspace_bytes(int B, int H, int T) {
    if (B <= 0 || H <= 0 || T <= 0) return 0;
    return static_cast<size_t>(B) * H * ((T + C - 1) / C) * kRecord;
}

hipError_t kda_launch(const KGeo& g, long long tile_blocks, long long scan_items, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                      unsigned char* ws, hipStream_t stream) {
    if (!grid_fits(tile_blocks, kTileThreads) || !grid_fits((scan_items + 7) / 8 * 64, kScanThreads))
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kda_tile_kernel, dim3(static_cast<unsigned>(tile_blocks)), dim3(kTileThreads), 0, stream, g,
                       static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v), alpha, beta,
                       ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_scan_kernel, dim3(static_cast<unsigned>((scan_items + 7) / 8) * 64), dim3(kScanThreads), 0,
                       stream, g, ws, S0, static_cast<u16*>(o), S_out);
    return hipGetLastError();
}

hipError_t launch_kda_mfma(int B, int H, int T, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                           void* workspace, hipStream_t stream) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return hipSuccess;
    KGeo g{};
    g.BH = BH;
    g.T = T;
    g.NC = (T + C - 1) / C;
    return kda_launch(g, static_cast<long long>(BH) * g.NC, BH, q, k, v, alpha, beta, S0, o, S_out,
                      static_cast<unsigned char*>(workspace), stream);
}

// Packed batches: a device-built table (chunk_base, snap_base: [N+1] each;
// the sequences longest first: [N]) ahead of the records; at most Ttot / C + N
// chunks per head.
static size_t kda_table_bytes(int N) { return ((3 * static_cast<size_t>(N) + 2) * sizeof(int) + 255) / 256 * 256; }

size_t kda_mfma_varlen_workspace_bytes(int N, int H, int Ttot) {
    if (N <= 0 || H <= 0) return 0;
    const size_t table = kda_table_bytes(N);
    const size_t cap = static_cast<size_t>(Ttot) / C + N;
    return table + static_cast<size_t>(H) * cap * kRecord;
}

hipError_t launch_kda_mfma_varlen(int N, int H, int Ttot, const int* cu, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                                  int snap, int snap_cap, float* S_snap, void* workspace, hipStream_t stream) {
    if (N <= 0 || H <= 0) return hipSuccess;
    const size_t table = kda_table_bytes(N);
    int* tab = static_cast<int*>(workspace);
    KGeo g{};
    g.cu = cu;
    g.chunk_base = tab;
    g.snap_base = tab + (N + 1);
    g.seq_order = tab + 2 * (N + 1);
    g.N = N;
    g.H = H;
    g.Ttot = Ttot;
    g.cap = Ttot / C + N;
    g.snap = S_snap ? snap : 0;
    g.snap_cap = snap_cap;
    g.S_snap = S_snap;
    // every grid checked before the table kernel runs
    const long long tiles = static_cast<long long>(g.cap) * H, items = static_cast<long long>(N) * H;
    if (!grid_fits(tiles, kTileThreads) || !grid_fits((items + 7) / 8 * 64, kScanThreads))
        return hipErrorInvalidConfiguration;
    // chunk_base: one "segment" per chunk (an empty sequence counts one)
    const hipError_t e = launch_varlen_table(N, Ttot, 1, g.snap, cu, tab, stream, nullptr, 0, tab + 2 * (N + 1));
    if (e != hipSuccess) return e;
    return kda_launch(g, tiles, items, q, k, v, alpha, beta, S0, o, S_out, static_cast<unsigned char*>(workspace) + table,
                      stream);
}

}  // namespace la

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
// Tile pass (one workgroup per chunk, 256 threads).  g by a per-channel
// running sum; the decayed products L and A as MFMA products of scaled copies
// K * e^{g - g_m}, K * e^{g_m - g}, Q * e^{g - g_m} (g_m: the chunk's middle
// token, so every factor lies within e^{+-80} whenever the chunk's decay span
// is at most 80 in every channel; chunks with a larger span take an exact
// path with one exponential per term); then [W | Ut] by forward substitution
// in fp32, one column per thread.  Per chunk it writes W, Q * e^g (64 x 128),
// A (64 x 64), (K * e^{g_c - g})^T and Ut^T (128 x 64) in bf16 and e^{g_c}
// (128 fp32): 74 240 bytes.
//
// Scan (one workgroup per (head, 16 value channels), 4 waves).  Wave w owns
// token rows 16w.. of X = W P, U and O and key rows 32w.. of P (fp32 in its
// accumulators); P^T and U^T (bf16) are shared through LDS, two barriers per
// chunk.  The tiles of chunk n+1 are loaded while chunk n runs.  The eight
// workgroups of a head take block indices eight apart, so they run on one XCD
// and read each chunk's tiles from that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int C = 64;           // tokens per chunk
constexpr int D = 128;          // d_k = d_v
constexpr int LDB = D + 8;      // bf16 row stride of the tile pass's LDS tiles
constexpr int kTileThreads = 256;
constexpr int kScanThreads = 256;
constexpr float kMaxSpan = 80.f;   // largest decay span of the factored fast path

// per-chunk record (bytes)
constexpr size_t oW = 0;              // W       [64][128] bf16
constexpr size_t oQ = 16384;          // Q e^g   [64][128] bf16
constexpr size_t oA = 32768;          // A       [64][64]  bf16 (zero above the diagonal)
constexpr size_t oKt = 40960;         // Kt^T    [128][64] bf16
constexpr size_t oUt = 57344;         // Ut^T    [128][64] bf16
constexpr size_t oDec = 73728;        // e^{g_c} [128] fp32
constexpr size_t kRecord = 74240;

__device__ __forceinline__ float bf(u16 b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16_bits(a)) | (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// ======================================================== tile pass
struct TileSmem {
    u16 K[C][LDB];        // raw k
    u16 V[C][LDB];        // raw v
    u16 Qp[C][LDB];       // raw q, then q e^{g - g_m} (fast path)
    u16 Kp[C][LDB];       // k e^{g - g_m}
    u16 Km[C][LDB];       // k e^{g_m - g}
    float g[C][D];        // chunk-local cumulative log decay
    float L[C][C + 4];    // beta_r L_rj (strictly lower)
    float beta[C];
    int span;             // max decay span over channels (float bits, >= 0)
};

__global__ __launch_bounds__(kTileThreads) void kda_tile_kernel(int BH, int T, int NC, bool scalar_gate,
                                                                const u16* __restrict__ q, const u16* __restrict__ k,
                                                                const u16* __restrict__ v,
                                                                const float* __restrict__ alpha,
                                                                const float* __restrict__ beta,
                                                                unsigned char* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) TileSmem sm;
    const int bh = blockIdx.x / NC, n = blockIdx.x % NC;
    if (bh >= BH) return;
    const int tid = threadIdx.x;
    const int t0 = n * C;
    const int len = min(C, T - t0);
    const size_t row0 = static_cast<size_t>(bh) * T + t0;   // first token row of the chunk
    unsigned char* rec = ws + (static_cast<size_t>(bh) * NC + n) * kRecord;

    if (tid == 0) sm.span = 0;
    // ---- every input load of the chunk first (coalesced 16-byte pieces): log
    // alpha into g, raw k, v, q tiles; then the running sums of g
    {
        float4 al[8];
        uint4 kk[4], vv[4], qq[4];
#pragma unroll
        for (int it = 0; it < 8; ++it) {           // alpha: 64 x 128 fp32 = 2048 float4
            const int e = it * kTileThreads + tid, t = e >> 5, c4 = (e & 31) * 4;
            al[it] = make_float4(1.f, 1.f, 1.f, 1.f);
            if (t < len) {
                if (scalar_gate) {
                    const float a = alpha[row0 + t];
                    al[it] = make_float4(a, a, a, a);
                } else {
                    al[it] = *reinterpret_cast<const float4*>(alpha + (row0 + t) * D + c4);
                }
            }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {           // k, v, q: 64 x 128 bf16 = 1024 pieces each
            const int e = it * kTileThreads + tid, t = e >> 4, c8 = (e & 15) * 8;
            kk[it] = vv[it] = qq[it] = make_uint4(0, 0, 0, 0);
            if (t < len) {
                const size_t gi = (row0 + t) * D + c8;
                kk[it] = *reinterpret_cast<const uint4*>(k + gi);
                vv[it] = *reinterpret_cast<const uint4*>(v + gi);
                qq[it] = *reinterpret_cast<const uint4*>(q + gi);
            }
        }
        if (tid < C) sm.beta[tid] = tid < len ? beta[row0 + tid] : 0.f;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int e = it * kTileThreads + tid, t = e >> 5, c4 = (e & 31) * 4;
            *reinterpret_cast<float4*>(&sm.g[t][c4]) =
                make_float4(__logf(al[it].x), __logf(al[it].y), __logf(al[it].z), __logf(al[it].w));
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int e = it * kTileThreads + tid, t = e >> 4, c8 = (e & 15) * 8;
            *reinterpret_cast<uint4*>(&sm.K[t][c8]) = kk[it];
            *reinterpret_cast<uint4*>(&sm.V[t][c8]) = vv[it];
            *reinterpret_cast<uint4*>(&sm.Qp[t][c8]) = qq[it];
        }
    }
    __syncthreads();
    if (tid < D) {   // running sum over the chunk's tokens, one channel per thread
        float acc = 0.f;
#pragma unroll 16
        for (int t = 0; t < C; ++t) {
            acc += sm.g[t][tid];
            sm.g[t][tid] = acc;
        }
    }
    __syncthreads();
    if (tid < D) {
        const float s = fmaxf(sm.g[0][tid] - sm.g[31][tid], sm.g[31][tid] - sm.g[C - 1][tid]);
        atomicMax(&sm.span, __float_as_int(fmaxf(s, 0.f)));
    }
    __syncthreads();
    const bool fast = __int_as_float(sm.span) <= kMaxSpan;

    // ---- elementwise: scaled copies, Q e^g, Kt^T, e^{g_c}
    for (int e = tid; e < C * D / 8; e += kTileThreads) {
        const int t = e / (D / 8), c0 = (e % (D / 8)) * 8;
        uint32_t wq[4], wp[4], wm[4], wqp[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            float kp[2], km[2], qp[2], qe[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = c0 + i + h;
                const float gr = sm.g[t][c], gm = sm.g[31][c];
                const float kv = bf(sm.K[t][c]), qv = bf(sm.Qp[t][c]);
                const float up = __expf(gr - gm);
                kp[h] = kv * up;
                km[h] = kv * __expf(gm - gr);
                qp[h] = qv * up;
                qe[h] = qv * __expf(gr);
            }
            wp[i / 2] = pack2(kp[0], kp[1]);
            wm[i / 2] = pack2(km[0], km[1]);
            wqp[i / 2] = pack2(qp[0], qp[1]);
            wq[i / 2] = pack2(qe[0], qe[1]);
        }
        *reinterpret_cast<uint4*>(rec + oQ + (static_cast<size_t>(t) * D + c0) * 2) = make_uint4(wq[0], wq[1], wq[2], wq[3]);
        if (fast) {
            *reinterpret_cast<uint4*>(&sm.Kp[t][c0]) = make_uint4(wp[0], wp[1], wp[2], wp[3]);
            *reinterpret_cast<uint4*>(&sm.Km[t][c0]) = make_uint4(wm[0], wm[1], wm[2], wm[3]);
        }
        // q e^{g - g_m} replaces raw q only on the fast path (the exact path reads raw q)
        if (fast) *reinterpret_cast<uint4*>(&sm.Qp[t][c0]) = make_uint4(wqp[0], wqp[1], wqp[2], wqp[3]);
    }
    for (int e = tid; e < D * (C / 8); e += kTileThreads) {
        const int c = e / (C / 8), tb = (e % (C / 8)) * 8;
        const float gc = sm.g[C - 1][c];
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2)
            w[i / 2] = pack2(bf(sm.K[tb + i][c]) * __expf(gc - sm.g[tb + i][c]),
                             bf(sm.K[tb + i + 1][c]) * __expf(gc - sm.g[tb + i + 1][c]));
        *reinterpret_cast<uint4*>(rec + oKt + (static_cast<size_t>(c) * C + tb) * 2) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (tid < D) reinterpret_cast<float*>(rec + oDec)[tid] = __expf(sm.g[C - 1][tid]);
    __syncthreads();

    // ---- L (beta-scaled, strictly lower) into LDS, A (lower incl. diagonal) to the record
    u16* Arec = reinterpret_cast<u16*>(rec + oA);
    if (fast) {
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15, gg = lane >> 4;
        // 10 lower tile pairs (I >= J) x {L, A}: wave w takes items w, w+4, ...
        for (int item = w; item < 20; item += 4) {
            const int p = item >> 1;
            const bool isA = item & 1;
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= p) ++I;
            const int J = p - I * (I + 1) / 2;
            f32x4 acc = zero4();
            const u16 (*X)[LDB] = isA ? sm.Qp : sm.Kp;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&X[16 * I + r][32 * s + 8 * gg]));
                const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Km[16 * J + r][32 * s + 8 * gg]));
                acc = mfma16x16x32(a, b, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * I + 4 * gg + i, col = 16 * J + r;
                if (isA) {
                    Arec[row * C + col] = f32_to_bf16_bits(col <= row ? acc[i] : 0.f);
                } else {
                    sm.L[row][col] = col < row ? sm.beta[row] * acc[i] : 0.f;
                }
            }
        }
    } else {
        // exact path: one exponential per term
        for (int e = tid; e < C * C; e += kTileThreads) {
            const int row = e / C, col = e % C;
            float sl = 0.f, sa = 0.f;
            if (col <= row) {
                for (int c = 0; c < D; ++c) {
                    const float f = __expf(sm.g[row][c] - sm.g[col][c]) * bf(sm.K[col][c]);
                    sl = fmaf(bf(sm.K[row][c]), f, sl);
                    sa = fmaf(bf(sm.Qp[row][c]), f, sa);
                }
            }
            sm.L[row][col] = col < row ? sm.beta[row] * sl : 0.f;
            Arec[row * C + col] = f32_to_bf16_bits(col <= row ? sa : 0.f);
        }
    }
    // tiles above the diagonal block row of A are zero
    for (int e = tid; e < C * C; e += kTileThreads) {
        const int row = e / C, col = e % C;
        if (col / 16 > row / 16) Arec[row * C + col] = 0;
    }
    __syncthreads();

    // ---- [W | Ut] = (I + L)^{-1} diag(beta) [K e^g | V]: column tid, forward substitution
    {
        const int col = tid;
        float x[C];
#pragma unroll
        for (int r = 0; r < C; ++r)
            x[r] = col < D ? sm.beta[r] * bf(sm.K[r][col]) * __expf(sm.g[r][col]) : sm.beta[r] * bf(sm.V[r][col - D]);
        // (right-hand sides first, then the sweep: one fused loop made the
        // compiler keep every right-hand side live and spill)
        // row r + 1 of L is read while row r is used (software pipelined:
        // otherwise every row waits for its own LDS reads)
        float4 cur[C / 4], nxt[C / 4];
        cur[0] = *reinterpret_cast<const float4*>(&sm.L[1][0]);
#pragma unroll
        for (int r = 1; r < C; ++r) {
            if (r + 1 < C) {
#pragma unroll
                for (int j4 = 0; j4 < (r + 4) / 4; ++j4) nxt[j4] = *reinterpret_cast<const float4*>(&sm.L[r + 1][4 * j4]);
            }
            float acc[4] = {x[r], 0.f, 0.f, 0.f};   // four chains: the sums are not one long dependency
#pragma unroll
            for (int j = 0; j < r; ++j) {
                const float4 l = cur[j >> 2];
                const float lj = (j & 3) == 0 ? l.x : (j & 3) == 1 ? l.y : (j & 3) == 2 ? l.z : l.w;
                acc[j & 3] = fmaf(-lj, x[j], acc[j & 3]);
            }
            x[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
            for (int j4 = 0; j4 < C / 4; ++j4) cur[j4] = nxt[j4];
        }
        if (col < D) {
            u16* W = reinterpret_cast<u16*>(rec + oW);
#pragma unroll
            for (int r = 0; r < C; ++r) W[r * D + col] = f32_to_bf16_bits(x[r]);
        } else {
            unsigned char* ut = rec + oUt + static_cast<size_t>(col - D) * C * 2;
#pragma unroll
            for (int r = 0; r < C; r += 8)
                *reinterpret_cast<uint4*>(ut + r * 2) =
                    make_uint4(pack2(x[r], x[r + 1]), pack2(x[r + 2], x[r + 3]), pack2(x[r + 4], x[r + 5]),
                               pack2(x[r + 6], x[r + 7]));
        }
    }
}

// ======================================================== scan
struct ScanSmem {
    u16 PT[16][D + 8];    // P^T (bf16): [value column][key channel]
    u16 UT[16][C + 8];    // U^T (bf16): [value column][token]
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
        op.W[s] = *reinterpret_cast<const uint4*>(W + (16 * w + r) * D + 32 * s + 8 * gg);
        op.Q[s] = *reinterpret_cast<const uint4*>(Q + (16 * w + r) * D + 32 * s + 8 * gg);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        op.A[s] = *reinterpret_cast<const uint4*>(A + (16 * w + r) * C + 32 * s + 8 * gg);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            op.K[mt][s] = *reinterpret_cast<const uint4*>(K + (32 * w + 16 * mt + r) * C + 32 * s + 8 * gg);
    }
    op.U = *reinterpret_cast<const uint2*>(U + (16 * cb + r) * C + 16 * w + 4 * gg);
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
    // O += A U; store rows inside the sequence
#pragma unroll
    for (int s = 0; s < 2; ++s) O = mfma16x16x32(as_bf16x8(op.A[s]), ub[s], O);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 16 * w + 4 * gg + i;
        if (t < len) o[(orow + t) * D + 16 * cb + r] = f32_to_bf16_bits(O[i]);
    }
    // P <- Diag(e^{g_c}) P + Kt^T U (key rows 32w + 16mt + 4gg + i)
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
    lds_barrier();
}

__global__ __launch_bounds__(kScanThreads) void kda_scan_kernel(int BH, int T, int NC,
                                                                const unsigned char* __restrict__ ws,
                                                                const float* S0, u16* __restrict__ o, float* S_out) {
    __shared__ __attribute__((aligned(16))) ScanSmem sm;
    // the 8 column blocks of a head take block indices 8 apart (one XCD)
    const int i = blockIdx.x;
    const int bh = (i >> 6) * 8 + (i & 7);
    const int cb = (i >> 3) & 7;
    if (bh >= BH) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, gg = lane >> 4;
    const size_t sbase = static_cast<size_t>(bh) * D * D;
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
    const unsigned char* rec0 = ws + static_cast<size_t>(bh) * NC * kRecord;
    const size_t orow = static_cast<size_t>(bh) * T;
    // tiles of chunks n+1 and n+2 are in flight while chunk n runs (three
    // register sets in rotation; indices past the end reload the last chunk)
    ChunkOps a, b, c;
    auto rec = [&](int m) { return rec0 + static_cast<size_t>(min(m, NC - 1)) * kRecord; };
    auto run = [&](const ChunkOps& op, int m) {
        scan_chunk(sm, op, P, w, r, gg, o, orow + static_cast<size_t>(m) * C, min(C, T - m * C), cb);
    };
    load_ops(a, rec(0), w, cb, r, gg);
    load_ops(b, rec(1), w, cb, r, gg);
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
    return dtype == kBF16 && dk == D && dv == D && chunk == C;
}

size_t kda_mfma_workspace_bytes(int B, int H, int T) {
    if (B <= 0 || H <= 0 || T <= 0) return 0;
    return static_cast<size_t>(B) * H * ((T + C - 1) / C) * kRecord;
}

hipError_t launch_kda_mfma(int B, int H, int T, bool scalar_gate, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                           void* workspace, hipStream_t stream) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return hipSuccess;
    const int NC = (T + C - 1) / C;
    auto* ws = static_cast<unsigned char*>(workspace);
    hipLaunchKernelGGL(kda_tile_kernel, dim3(static_cast<unsigned>(BH) * NC), dim3(kTileThreads), 0, stream, BH, T, NC,
                       scalar_gate, static_cast<const u16*>(q), static_cast<const u16*>(k),
                       static_cast<const u16*>(v), alpha, beta, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_scan_kernel, dim3(static_cast<unsigned>((BH + 7) / 8) * 64), dim3(kScanThreads), 0, stream,
                       BH, T, NC, ws, S0, static_cast<u16*>(o), S_out);
    return hipGetLastError();
}

}  // namespace la

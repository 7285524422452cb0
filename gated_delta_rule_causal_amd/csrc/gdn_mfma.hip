// Gated delta rule, chunkwise, on the CDNA4 matrix cores: bf16 activations,
// fp32 state, d_k = d_v = 128, chunk C = 64.
//
// Source: page "Linear attention and hybrids", section "Delta rule and Gated
// DeltaNet", Gated DeltaNet equation
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// The page names a sequence-parallel evaluation but prints none; the chunk
// form used here follows from unrolling the equation inside a chunk of c
// tokens with entry state S (rows = value channels).  With g = chunk-local
// cumsum(log alpha), Gamma_ij = exp(g_i - g_j):
//     L_ij = beta_i Gamma_ij (k_i . k_j) for j < i          (strictly lower)
//     W    = (I + L)^{-1} diag(beta e^g) K                   (c x d_k)
//     Ut   = (I + L)^{-1} diag(beta) V                       (c x d_v)
//     A    = (Q K^T) * Gamma, lower triangle incl. diagonal  (c x c)
//     U    = Ut - W S^T
//     O    = diag(e^g) Q S^T + A U
//     S   <- e^{g_c} S + U^T diag(e^{g_c - g}) K
// Written on P = S^T (d_k x d_v) a chunk is the affine map
//     P <- M P + N,   M = e^{g_c} I - K~^T W,   N = K~^T Ut,   K~ = diag(e^{g_c-g}) K,
// and a run of chunks composes to one such map.
//
// The sequence of every head is cut into G segments of whole chunks so that
// B*H*G workgroups fill the chip.  Three kernels, one workgroup per (head,
// segment) in the two big ones (the map kernel 12 waves: 8 carry state
// columns, 4 stage tiles; the output kernel 8 waves: 4 and 4):
//  * gdn_map_kernel     - segments 0..G-2: for each chunk, recompute its
//    state-independent tiles in LDS and push the augmented state [N | M]
//    (d_k x 256, starting from [0 | I]) through the chunk map; emits the
//    segment's (M, N).
//  * gdn_combine_kernel - per head, the entering state of every segment:
//    P_0 = S0, P_{s+1} = M_s P_s + N_s (split bf16 products, fp32 sums).
//  * gdn_out_kernel     - every segment from its entering state: recompute
//    the chunk tiles, outputs O, and the final state of the last segment.
// The map pass needs one workgroup fewer per head than the output pass; a
// whole gdn_prefill call can instead give segment 0 (whose entering state is
// S0) to gdn_lead_map_kernel, which runs it beside the maps of segments
// 1..G-2 and writes P_1; the combine then starts from P_1 and the output pass
// runs segments 1..G-1, so both passes fill the chip with one more segment.
// Per chunk, the state-independent tiles (chunk-local prefix sum of log alpha
// with a wave scan; K K^T and Q K^T on v_mfma_f32_16x16x32_bf16; the four
// 16x16 diagonal blocks of I + L inverted in registers by the product form
// (I + N)(I + N^2)(I + N^4)(I + N^8), N = -L_bb nilpotent, on
// v_mfma_f32_16x16x16_bf16 (the first squaring from split bf16 pairs); the
// rest of the unit lower-triangular solve as blocked v_mfma_f32_16x16x16_bf16
// products) never leave LDS.  The state slice of each wave stays in MFMA
// accumulator registers for the whole segment: an accumulator tile is fed
// back as the B operand of the next product by permuting the contraction
// index (pack_acc_pair), so no state crosses lanes.  The next chunk's raw
// q/k/v are loaded into registers while the current chunk computes.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // d_k = d_v
// bf16 row stride of 128-wide LDS tiles (304 B).  Measured on gfx950 LDS: any
// stride of 136 u16 or more (16-byte multiple, not a power of two) serves the
// 16-row x 16-byte operand reads at full rate; 152 also halves the bank
// conflicts of the transposing reads of K in the state update (the four
// column groups of a lane quad are 16 bytes apart there).
constexpr int LDQ = D + 24;
constexpr int LDA = C + 8;   // bf16 row stride of 64-wide LDS tiles (144 B)
constexpr int kThreads = 512;                 // 8 waves per workgroup
constexpr int kTargetBlocks = 256;            // workgroups that fill the chip (one per CU)

// Row permutation shared by the state tiles and the chunk tiles: accumulator
// tile t, lane group gg, register i  <->  index 32(t/2) + 8 gg + 4(t%2) + i.
// Two consecutive tiles therefore hold 8 consecutive indices per lane group,
// which is exactly one K = 32 operand slice of that lane (pack_acc_pair).
__device__ __forceinline__ int perm_row(int t, int rr) {
    return 32 * (t >> 1) + 8 * (rr >> 2) + 4 * (t & 1) + (rr & 3);
}

// ------------------------------------------------------------------ LDS
// Gate vectors of one chunk.
struct Gates {
    float g[C], b[C], eg[C], sw[C], ek[C];  // g, beta, e^g, beta e^g, e^{g_c - g}
};

// Raw chunk inputs held in registers between chunks.  Each 16-byte piece is
// one of the sixteen in a 256-byte row, so the global loads are contiguous
// and the LDS stores conflict-free.  NTHR threads (tid 0 .. NTHR-1) share the
// work, NI pieces each.  Piece it of thread tid:
//   WAVE_ROWS = false: rows interleaved over all threads, row = (tid + NTHR it) / 16;
//   WAVE_ROWS = true:  wave u holds rows 16u .. 16u+15 (NTHR = 256, four waves),
//                      so a wave can use its own rows right after writing them.
// Every wave also holds the gates of all 64 tokens, one per lane.
template <int NTHR, bool WAVE_ROWS = false>
struct RawChunk {
    static constexpr int NI = C * D / 8 / NTHR;
    static_assert(!WAVE_ROWS || NTHR == 256, "wave-owned rows need four waves");
    uint4 q[NI], k[NI], v[NI];
    float a, b;
    static __device__ __forceinline__ int row(int tid, int it) {
        return WAVE_ROWS ? 16 * (tid >> 6) + 4 * it + ((tid & 63) >> 4) : (tid + NTHR * it) >> 4;
    }
    static __device__ __forceinline__ int col(int tid) { return (tid & 15) * 8; }
};

// WITH_Q / WITH_K / WITH_V select the tensors loaded (the gates come with k).
// Every load is issued, rows past the end of the sequence (len >= 1 tokens
// from t0) reading its last row: they are zeroed when staged.  With no
// branches around the loads, the wait before a staging step covers only the
// loads it consumes, and the others stay in flight.
template <bool WITH_Q, bool WITH_K, bool WITH_V, int NTHR, bool WR>
__device__ __forceinline__ void fetch_chunk(RawChunk<NTHR, WR>& rc, const u16* __restrict__ q, const u16* __restrict__ k,
                                            const u16* __restrict__ v, const float* __restrict__ alpha,
                                            const float* __restrict__ beta, size_t head_tok, int t0, int len,
                                            int tid) {
    using RC = RawChunk<NTHR, WR>;
#pragma unroll
    for (int it = 0; it < RC::NI; ++it) {
        const int row = min(RC::row(tid, it), len - 1), c8 = RC::col(tid);
        const size_t gi = (head_tok + t0 + row) * D + c8;
        if (WITH_Q) rc.q[it] = *reinterpret_cast<const uint4*>(q + gi);
        if (WITH_K) rc.k[it] = *reinterpret_cast<const uint4*>(k + gi);
        if (WITH_V) rc.v[it] = *reinterpret_cast<const uint4*>(v + gi);
    }
    if (WITH_K) {
        const int t = min(tid & 63, len - 1);
        rc.a = alpha[head_tok + t0 + t];
        rc.b = beta[head_tok + t0 + t];
    }
}

// One tensor's raw rows (rc.q, rc.k or rc.v) into a row-major LDS tile, rows
// len.. (past the end of the sequence) as zeros.
template <class RC, int NI>
__device__ __forceinline__ void stage_rows(u16 (*X)[LDQ], const uint4 (&raw)[NI], int tid, int len) {
    if (len >= C) {   // a whole chunk (len is uniform): no rows to clear
#pragma unroll
        for (int it = 0; it < NI; ++it)
            *reinterpret_cast<uint4*>(&X[RC::row(tid, it)][RC::col(tid)]) = raw[it];
        return;
    }
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int row = RC::row(tid, it);
        *reinterpret_cast<uint4*>(&X[row][RC::col(tid)]) = row < len ? raw[it] : make_uint4(0, 0, 0, 0);
    }
}

// Gates of the chunk, one token per lane: g = inclusive scan of log alpha
// over the wave.
struct GateRegs {
    float g, b, eg, ek;
};

// x + (x of the lane selected by the DPP control, 0 where there is none or
// the row is masked off).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWMASK, 0xf, true));
}

// Tokens past the end of the sequence (lane >= len) take alpha = 1 (log 0)
// and beta = 0: with their zero rows they change nothing.
__device__ __forceinline__ GateRegs chunk_gates(float a, float b, int len) {
    const bool in = static_cast<int>(threadIdx.x & 63) < len;
    b = in ? b : 0.f;
    // inclusive scan without LDS: shifts by 1, 2, 4, 8 inside each 16-lane
    // row, then lane 15 added into rows 1 and 3 and lane 31 into rows 2 and 3
    float x = in ? __logf(a) : 0.f;
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa>(x);   // row_bcast:15
    x = dpp_add<0x143, 0xc>(x);   // row_bcast:31
    const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), C - 1));
    return GateRegs{x, b, __expf(x), __expf(gl - x)};
}

// Gate vectors of token t (one lane each).
__device__ __forceinline__ void write_gates(Gates& gt, const GateRegs& gr, int t) {
    gt.g[t] = gr.g;
    gt.b[t] = gr.b;
    gt.eg[t] = gr.eg;
    gt.sw[t] = gr.b * gr.eg;
    gt.ek[t] = gr.ek;
}

// B operand (K = 16) of a diagonal block of Tm: lane (r, g) holds T[4g+i][r].
__device__ __forceinline__ short4v tdiag_b(const u16 (*Tm)[LDA], int blk, int r, int g) {
    short4v x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = static_cast<short>(Tm[16 * blk + 4 * g + i][16 * blk + r]);
    return x;
}

// Everything one 16x16 tile (rt, ct) of X Y^T (two row-major 64 x 128 LDS
// operands) and its epilogue read from LDS: four K = 32 slices of row
// 16 rt + r of X and of row 16 ct + r of Y, g and beta of rows 16 rt + 4 g ..
// +3 and of column 16 ct + r.  Loading it all before the products keeps the
// reads in flight together instead of one round trip per product.
struct TileOps {
    bf16x8 x[4], y[4];
    float4 gr, br;
    float gc, bc;
};

__device__ __forceinline__ void load_tile(TileOps& o, const u16 (*X)[LDQ], const u16 (*Y)[LDQ], const Gates& gt,
                                          int rt, int ct, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.x[s] = lds_bf16x8(&X[16 * rt + r][32 * s + 8 * g]);
        o.y[s] = lds_bf16x8(&Y[16 * ct + r][32 * s + 8 * g]);
    }
    o.gr = *reinterpret_cast<const float4*>(&gt.g[16 * rt + 4 * g]);
    o.br = *reinterpret_cast<const float4*>(&gt.b[16 * rt + 4 * g]);
    o.gc = gt.g[16 * ct + r];
    o.bc = gt.b[16 * ct + r];
}

__device__ __forceinline__ f32x4 dot_tile(const TileOps& o) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16x16x32(o.x[s], o.y[s], acc);
    return acc;
}

__device__ __forceinline__ float f4get(const float4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// 16x16 block coordinates.  Blocks below the diagonal, 0..5:
// (1,0) (2,0) (2,1) (3,0) (3,1) (3,2); blocks on or below it, 0..9, in row order.
__device__ __forceinline__ int below_row(int t) { return 1 + (t >= 1) + (t >= 3); }
__device__ __forceinline__ int below_col(int t) { const int rt = below_row(t); return t - rt * (rt - 1) / 2; }
__device__ __forceinline__ int lower_row(int t) { return (t >= 1) + (t >= 3) + (t >= 6); }
__device__ __forceinline__ int lower_col(int t) { const int rt = lower_row(t); return t - rt * (rt + 1) / 2; }

// ---- step 1: L = beta Gamma (K K^T) below the diagonal, and the inverses of
// the diagonal 16x16 blocks of I + L.
//
// Diagonal block b: K K^T is symmetric there, so one accumulator tile yields
// both L_bb and its transpose; the inverse is formed in registers and stored
// in bf16 into Tm.
__device__ __forceinline__ void step1_diag(const u16 (*Ks)[LDQ], u16 (*Tm)[LDA], const Gates& gt, int b, int lane) {
    const int r = lane & 15, g = lane >> 4;
    TileOps o;
    load_tile(o, Ks, Ks, gt, b, b, lane);
    const f32x4 acc = dot_tile(o);
    f32x4 N, Nt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float gr = f4get(o.gr, i), br = f4get(o.br, i);
        N[i] = r < 4 * g + i ? -br * __expf(fminf(gr - o.gc, 0.f)) * acc[i] : 0.f;
        Nt[i] = 4 * g + i < r ? -o.bc * __expf(fminf(o.gc - gr, 0.f)) * acc[i] : 0.f;
    }
    const f32x4 Tb = unit_lower_inverse(N, Nt, r, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) Tm[16 * b + 4 * g + i][16 * b + r] = f32_to_bf16_bits(Tb[i]);
}

// Below-diagonal blocks ta and tb (numbering above): -L in bf16 into Lb.  With
// two = false, tb is formed and dropped, which keeps the code free of
// branches around the matrix-core instructions.
__device__ __forceinline__ void step1_below(const u16 (*Ks)[LDQ], u16 (*Lb)[LDA], const Gates& gt, int ta, int tb,
                                            bool two, int lane) {
    const int r = lane & 15, g = lane >> 4;
    TileOps o[2];
    load_tile(o[0], Ks, Ks, gt, below_row(ta), below_col(ta), lane);
    load_tile(o[1], Ks, Ks, gt, below_row(tb), below_col(tb), lane);
    const f32x4 acc[2] = {dot_tile(o[0]), dot_tile(o[1])};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j == 1 && !two) break;
        const int t = j ? tb : ta;
        const int rt = below_row(t), ct = below_col(t);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Lb[16 * rt + 4 * g + i][16 * ct + r] =
                f32_to_bf16_bits(-f4get(o[j].br, i) * __expf(fminf(f4get(o[j].gr, i) - o[j].gc, 0.f)) * acc[j][i]);
    }
}

// ---- step 2: (I + L)^{-1} below the diagonal,
//     T_ij = T_ii * sum_{j<=k<i} (-L_ik) T_kj,
// as three independent chains, one per wave: part 0 forms T_10, T_20, T_30;
// part 1 T_21, T_31; part 2 T_32.  Every LDS operand is read first.  The
// part is a template argument: each wave runs straight-line code of its own.
template <int PART>
__device__ __forceinline__ void step2_inverse_below(u16 (*Tm)[LDA], const u16 (*Lb)[LDA], int lane) {
    const int r = lane & 15, g = lane >> 4;
    auto nl = [&](int i, int j) { return lds_short4(&Lb[16 * i + r][16 * j + 4 * g]); };
    auto ta = [&](int i) { return lds_short4(&Tm[16 * i + r][16 * i + 4 * g]); };
    auto put = [&](int i, int j, short4v t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[16 * i + 4 * g + e][16 * j + r] = static_cast<u16>(t[e]);
    };
    auto solve = [&](short4v a, f32x4 y) { return to_bf16x4(mfma16x16x16(a, to_bf16x4(y), zero4())); };
    if constexpr (PART == 0) {
        const short4v t00 = tdiag_b(Tm, 0, r, g);
        const short4v l10 = nl(1, 0), l20 = nl(2, 0), l21 = nl(2, 1), l30 = nl(3, 0), l31 = nl(3, 1), l32 = nl(3, 2);
        const short4v a1 = ta(1), a2 = ta(2), a3 = ta(3);
        const short4v t10 = solve(a1, mfma16x16x16(l10, t00, zero4()));
        const short4v t20 = solve(a2, mfma16x16x16(l21, t10, mfma16x16x16(l20, t00, zero4())));
        const short4v t30 =
            solve(a3, mfma16x16x16(l32, t20, mfma16x16x16(l31, t10, mfma16x16x16(l30, t00, zero4()))));
        put(1, 0, t10);
        put(2, 0, t20);
        put(3, 0, t30);
    } else if constexpr (PART == 1) {
        const short4v t11 = tdiag_b(Tm, 1, r, g);
        const short4v l21 = nl(2, 1), l31 = nl(3, 1), l32 = nl(3, 2);
        const short4v a2 = ta(2), a3 = ta(3);
        const short4v t21 = solve(a2, mfma16x16x16(l21, t11, zero4()));
        const short4v t31 = solve(a3, mfma16x16x16(l32, t21, mfma16x16x16(l31, t11, zero4())));
        put(2, 1, t21);
        put(3, 1, t31);
    } else {
        const short4v t22 = tdiag_b(Tm, 2, r, g);
        const short4v l32 = nl(3, 2), a3 = ta(3);
        put(3, 2, solve(a3, mfma16x16x16(l32, t22, zero4())));
    }
}

// A = (Q K^T) * Gamma on and below the diagonal: blocks t0 .. t0+NB-1 of the
// 0..9 numbering, the operands of block j+1 read while block j is formed.
template <int NB>
__device__ __forceinline__ void step2_qk(const u16 (*Qs)[LDQ], const u16 (*Ks)[LDQ], u16 (*As)[LDA], const Gates& gt,
                                         int t0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    TileOps o[2];
    load_tile(o[0], Qs, Ks, gt, lower_row(t0), lower_col(t0), lane);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int t = t0 + j;
        if (j + 1 < NB) load_tile(o[(j + 1) & 1], Qs, Ks, gt, lower_row(t + 1), lower_col(t + 1), lane);
        const TileOps& c = o[j & 1];
        const f32x4 acc = dot_tile(c);
        const int rt = lower_row(t), ct = lower_col(t);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * g + i, col = 16 * ct + r;
            const float e = __expf(fminf(f4get(c.gr, i) - c.gc, 0.f)) * acc[i];
            As[row][col] = f32_to_bf16_bits(col <= row ? e : 0.f);
        }
    }
}

// Zero block z (the transpose of below-diagonal block z) of a 64 x 64 tile.
__device__ __forceinline__ void zero_above(u16 (*X)[LDA], int z, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) X[16 * below_col(z) + 4 * g + i][16 * below_row(z) + r] = 0;
}

// ---- scan of one chunk for the NT 16-wide state tiles a wave owns (columns
// col0 + 16 nt + r of P).
//
// O = Q P (the inter-chunk part of the outputs, before the e^g row scaling;
// WITH_Q only) and X = K P, rows in the permuted order, in one pass over the
// packed state.  Sixteen steps (K-slice s, row tile m); the LDS operands of
// step i + AHEAD are read before the products of step i, so each wait for a
// read is covered by AHEAD steps of matrix-core work (a read issued right
// before its products left the whole LDS latency exposed).
template <int NT, bool WITH_Q>
__device__ __forceinline__ void scan_qk(const u16 (*Qs)[LDQ], const u16 (*Ks)[LDQ], const f32x4 (&P)[NT][8], int lane,
                                        f32x4 (&O)[NT][4], f32x4 (&X)[NT][4]) {
    const int r = lane & 15, g = lane >> 4;
    constexpr int AHEAD = WITH_Q ? 2 : 4, NBUF = AHEAD + 1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int m = 0; m < 4; ++m) O[nt][m] = X[nt][m] = zero4();
    bf16x8 ak[NBUF], aq[NBUF];
    auto load = [&](int i) {
        const int s = i >> 2, m = i & 3;
        ak[i % NBUF] = lds_bf16x8(&Ks[perm_row(m, r)][32 * s + 8 * g]);
        if constexpr (WITH_Q) aq[i % NBUF] = lds_bf16x8(&Qs[perm_row(m, r)][32 * s + 8 * g]);
    };
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) load(i);
    bf16x8 pb[NT];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int s = i >> 2, m = i & 3;
        if (i + AHEAD < 16) load(i + AHEAD);
        if (m == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) pb[nt] = pack_acc_pair(P[nt][2 * s], P[nt][2 * s + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of these products
        if constexpr (WITH_Q) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O[nt][m] = mfma16x16x32(aq[i % NBUF], pb[nt], O[nt][m]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) X[nt][m] = mfma16x16x32(ak[i % NBUF], pb[nt], X[nt][m]);
    }
}

// Right-hand side of the chunk's triangular system, diag(beta) (V - diag(e^g) K P)
// (without the V term when WITH_V is false: the M part of a segment map),
// packed as the B operands of two K = 32 slices: lane (r, g) of slice s2 holds
// tokens 32 s2 + 8 g .. +7 of value column col0 + 16 nt + r.  V is read
// transposed from its row-major tile.
template <int NT, bool WITH_V>
__device__ __forceinline__ void scan_rhs(const u16 (*Vs)[LDQ], const Gates& gt, const f32x4 (&X)[NT][4], int col0,
                                         int lane, bf16x8 (&Xb)[NT][2]) {
    const int g = lane >> 4;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int t0 = 32 * s2 + 8 * g;
        const float4 b0 = *reinterpret_cast<const float4*>(&gt.b[t0]), b1 = *reinterpret_cast<const float4*>(&gt.b[t0 + 4]);
        const float4 w0 = *reinterpret_cast<const float4*>(&gt.sw[t0]), w1 = *reinterpret_cast<const float4*>(&gt.sw[t0 + 4]);
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = -ww[i] * X[nt][2 * s2][i];
                x[4 + i] = -ww[4 + i] * X[nt][2 * s2 + 1][i];
            }
            if constexpr (WITH_V) {
                const bf16x8 vv = tr_operand(Vs, 32 * s2, [&](int aa) { return col0 + 16 * nt + 4 * aa; }, lane);
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] += bb[j] * static_cast<float>(vv[j]);
            }
            Xb[nt][s2] = pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
        }
    }
}

// The A operands a lower-triangular 64 x 64 tile (Tm or A) contributes to a
// product with a 64-row right-hand side: row tile m (chunk rows
// 32(m/2)..+31, permuted) needs K-slices s2 <= m/2, six pieces in all, read
// in one go so that their LDS latency overlaps (and, issued early, the work
// before their products).
struct TriOps {
    bf16x8 a[6];
};
__device__ __forceinline__ constexpr int tri_idx(int m, int s2) { return m < 2 ? m : 2 + 2 * (m - 2) + s2; }

__device__ __forceinline__ void load_tri(TriOps& t, const u16 (*X)[LDA], int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int s2 = 0; s2 <= (m >> 1); ++s2) t.a[tri_idx(m, s2)] = lds_bf16x8(&X[perm_row(m, r)][32 * s2 + 8 * g]);
}

// U = (I + L)^{-1} times that right-hand side (rows permuted), returned packed
// with the rows scaled by e^{g_c - g} (for the state update, which then reads
// K itself) and, WITH_UB, as is (for A U).
template <int NT, bool WITH_UB>
__device__ __forceinline__ void scan_solve(const TriOps& tm, const Gates& gt, const bf16x8 (&Xb)[NT][2], int lane,
                                           bf16x8 (&Ub)[NT][2], bf16x8 (&Ue)[NT][2]) {
    const int g = lane >> 4;
    f32x4 U[NT][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) U[nt][m] = zero4();
#pragma unroll
        for (int s2 = 0; s2 <= (m >> 1); ++s2)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) U[nt][m] = mfma16x16x32(tm.a[tri_idx(m, s2)], Xb[nt][s2], U[nt][m]);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int t0 = 32 * s2 + 8 * g;
        const float4 e0 = *reinterpret_cast<const float4*>(&gt.ek[t0]), e1 = *reinterpret_cast<const float4*>(&gt.ek[t0 + 4]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const f32x4 lo = U[nt][2 * s2], hi = U[nt][2 * s2 + 1];
            if constexpr (WITH_UB) Ub[nt][s2] = pack_acc_pair(lo, hi);
            Ue[nt][s2] = pack8(lo[0] * e0.x, lo[1] * e0.y, lo[2] * e0.z, lo[3] * e0.w, hi[0] * e1.x, hi[1] * e1.y,
                               hi[2] * e1.z, hi[3] * e1.w);
        }
    }
}

// O <- diag(e^g) O + A U, stored for the rows that exist.
template <int NT>
__device__ __forceinline__ void scan_out(const TriOps& am, const Gates& gt, f32x4 (&O)[NT][4],
                                         const bf16x8 (&Ub)[NT][2], int col0, int lane, u16* __restrict__ o,
                                         size_t o_row0, int len, u16 (*Os)[LDQ]) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float elo = gt.eg[32 * s2 + 8 * g + i], ehi = gt.eg[32 * s2 + 8 * g + 4 + i];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                O[nt][2 * s2][i] *= elo;
                O[nt][2 * s2 + 1][i] *= ehi;
            }
        }
    // row tile m (chunk rows 32(m/2)..+31) needs column slices s2 <= m/2
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int s2 = 0; s2 <= (m >> 1); ++s2)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O[nt][m] = mfma16x16x32(am.a[tri_idx(m, s2)], Ub[nt][s2], O[nt][m]);
    // Outputs go through LDS (Os: this wave's 16 NT columns of a free 64-row
    // tile) so that every global store is 16 contiguous bytes.
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = perm_row(m, 4 * g + i);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) Os[row][col0 + 16 * nt + r] = f32_to_bf16_bits(O[nt][m][i]);
        }
    wave_fence();   // this wave's LDS writes before its reads of other lanes' values
    constexpr int P8 = 2 * NT;   // 16-byte pieces per row of this wave's columns
#pragma unroll
    for (int pass = 0; pass < C * P8 / kWave; ++pass) {
        const int e = pass * kWave + lane, row = e / P8, c8 = 8 * (e % P8);
        if (row < len)
            *reinterpret_cast<uint4*>(o + (o_row0 + row) * D + col0 + c8) =
                *reinterpret_cast<const uint4*>(&Os[row][col0 + c8]);
    }
}

// P <- e^{g_c} P + Kx^T U, Kx^T read transposed in the permuted row order
// (Kx = K~ with U as is, or Kx = K with U's rows scaled by e^{g_c - g}).
template <int NT>
__device__ __forceinline__ void scan_update(const u16 (*Kx)[LDQ], const Gates& gt, f32x4 (&P)[NT][8],
                                            const bf16x8 (&Ub)[NT][2], int lane) {
    const float egc = gt.eg[C - 1];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) P[nt][t] *= egc;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8 a = tr_operand(Kx, 32 * s2, [&](int aa) { return 32 * (t >> 1) + 8 * aa + 4 * (t & 1); }, lane);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) P[nt][t] = mfma16x16x32(a, Ub[nt][s2], P[nt][t]);
        }
    }
}

// State slice <-> memory.  Memory layout is the state's: row = column of P
// (value channel, or map column), 128 fp32 per row over d.  Lane (r, g) of
// tile pair (2s, 2s+1) holds d = 32s + 8g .. 32s + 8g + 7 of row `col`.
template <int NT>
__device__ __forceinline__ void load_state(f32x4 (&P)[NT][8], const float* rows, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const float* row = rows ? rows + static_cast<size_t>(col0 + 16 * nt + r) * D : nullptr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (row) {
                const float4 a = *reinterpret_cast<const float4*>(row + 32 * s + 8 * g);
                const float4 b = *reinterpret_cast<const float4*>(row + 32 * s + 8 * g + 4);
                P[nt][2 * s] = f32x4{a.x, a.y, a.z, a.w};
                P[nt][2 * s + 1] = f32x4{b.x, b.y, b.z, b.w};
            } else {
                P[nt][2 * s] = zero4();
                P[nt][2 * s + 1] = zero4();
            }
        }
    }
}

template <int NT>
__device__ __forceinline__ void store_state(const f32x4 (&P)[NT][8], float* rows, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float* row = rows + static_cast<size_t>(col0 + 16 * nt + r) * D;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            *reinterpret_cast<float4*>(row + 32 * s + 8 * g) =
                make_float4(P[nt][2 * s][0], P[nt][2 * s][1], P[nt][2 * s][2], P[nt][2 * s][3]);
            *reinterpret_cast<float4*>(row + 32 * s + 8 * g + 4) =
                make_float4(P[nt][2 * s + 1][0], P[nt][2 * s + 1][1], P[nt][2 * s + 1][2], P[nt][2 * s + 1][3]);
        }
    }
}

// A segment map M is stored split, M = hi + lo with hi = bf16(M) and
// lo = bf16(M - hi), the two bf16 operands the combine multiplies with, in
// the order its MFMA operands read them: 64-lane blocks of 16 bytes, block
// (w, mt, ks) holding, for lane 16 g + r, M[32 w + 16 mt + r][32 ks + 8 g .. +7];
// hi in the first half of the matrix's space, lo in the second.  Every
// wave-wide load of the combine is then one contiguous 1 KiB run, and the
// combine does no splitting of its own.
constexpr int kMapHalf = D * D;   // bf16 elements of each half
__device__ __forceinline__ int map_frag(int row, int col) {
    const int blk = ((row >> 5) * 2 + ((row >> 4) & 1)) * 4 + (col >> 5);
    const int ln = ((col >> 3) & 3) * 16 + (row & 15);
    return ((blk * 64 + ln) << 3) + (col & 7);
}

// The slice of M a map carrier holds, written in that order.
template <int NT>
__device__ __forceinline__ void store_map_frag(const f32x4 (&P)[NT][8], u16* M, int col0, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int at = map_frag(perm_row(t, 4 * g + i), col0 + 16 * nt + r);
                const float x = P[nt][t][i];
                const u16 hi = f32_to_bf16_bits(x);
                M[at] = hi;
                M[kMapHalf + at] = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
            }
}

// ---- workspace: per (head, segment) three 128 x 128 fp32 matrices' room:
// the entering state P_s and N_s in the state's row layout ([value
// channel][d]), and M_s as two bf16 halves in the combine's operand order
// (map_frag).
constexpr size_t kMat = static_cast<size_t>(D) * D;
__device__ __forceinline__ size_t ws_P(size_t slot) { return slot * 3 * kMat; }
__device__ __forceinline__ size_t ws_N(size_t slot) { return ws_P(slot) + kMat; }
__device__ __forceinline__ size_t ws_M(size_t slot) { return ws_P(slot) + 2 * kMat; }

// ============================================================ work items
// Every (sequence, head) runs as G segments of SEGC chunks; a map or output
// workgroup takes one segment.  Two layouts:
// * uniform (cu == nullptr): BH = B*H sequences of T tokens, rows [BH][T][d],
//   gates [BH][T], states [BH][d][d], G segments each;
// * packed: N sequences, sequence n = tokens cu[n] .. cu[n+1] of every head's
//   rows [H][Ttot][d] (gates [H][Ttot]), states [N][H][d][d]; the segment
//   count varies per sequence, seg_base[n] numbers the segments of all
//   sequences in order (built on the device), and the workspace slots of head
//   h start at h * Gcap (Gcap bounds the total segment count).  The state
//   after every snap tokens of a sequence (snap a multiple of C, 0 for none)
//   is written to S_snap[snap_base[n] + j][h] for the first snap_cap slots.
struct Geo {
    int BH, T, G, SEGC;
    int L0;     // chunks of segment 0 (SEGC unless lead)
    int lead;   // uniform only: segment 0 runs in the map pass (1) or with the others (0)
    const int* cu;
    const int* seg_base;
    const int* snap_base;
    const int* order;   // packed: segments longest first (workgroup i takes order[i])
    int N, H, Ttot, Gcap;
    int snap, snap_cap;
    float* S_snap;
};

struct Item {
    size_t head_tok;  // row of the sequence's first token (this head) in q/k/v/o and alpha/beta
    int len;          // tokens of the sequence
    int seg, G;       // this segment and the sequence's segment count
    int n0, n1;       // chunks of the segment
    size_t slot0;     // workspace slot of the sequence's segment 0
    size_t state;     // index of the sequence's state in S0 / S_out
    int snap0, h;     // first snapshot of the sequence, head
};

__device__ __forceinline__ int clamp_tok(int t, int Ttot) { return t < 0 ? 0 : t > Ttot ? Ttot : t; }

// The work item of workgroup blk (maps: the last segment of a sequence has no
// map and its workgroup has nothing to do).  False: nothing to do.
__device__ __forceinline__ bool find_item(const Geo& g, int blk, bool maps, Item& it) {
    if (g.cu == nullptr) {
        // with a lead segment, segment 0 is neither mapped nor run here
        const int per = (maps ? g.G - 1 : g.G) - g.lead;
        const int bh = blk / per;
        if (bh >= g.BH) return false;
        it.seg = g.lead + blk - bh * per;
        it.G = g.G;
        it.len = g.T;
        it.head_tok = static_cast<size_t>(bh) * g.T;
        it.slot0 = static_cast<size_t>(bh) * g.G;
        it.state = bh;
        it.snap0 = 0;
        it.h = 0;
    } else {
        const int h = blk % g.H, i = blk / g.H;
        if (i >= min(g.seg_base[g.N], g.Gcap)) return false;
        const int gs = g.order ? g.order[i] : i;
        int lo = 0, hi = g.N;  // seg_base[lo] <= gs < seg_base[hi]; every sequence has a segment
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (g.seg_base[mid] <= gs) lo = mid; else hi = mid;
        }
        it.seg = gs - g.seg_base[lo];
        it.G = g.seg_base[lo + 1] - g.seg_base[lo];
        if (maps && it.seg == it.G - 1) return false;
        // a table that is not non-decreasing can ask for more segments than
        // the workspace holds: such sequences are skipped, never overrun
        if (g.seg_base[lo + 1] > g.Gcap) return false;
        const int t0 = clamp_tok(g.cu[lo], g.Ttot), t1 = clamp_tok(g.cu[lo + 1], g.Ttot);
        it.len = t1 > t0 ? t1 - t0 : 0;
        it.head_tok = static_cast<size_t>(h) * g.Ttot + t0;
        it.slot0 = static_cast<size_t>(h) * g.Gcap + g.seg_base[lo];
        it.state = static_cast<size_t>(lo) * g.H + h;
        it.snap0 = g.snap_base ? g.snap_base[lo] : 0;
        it.h = h;
    }
    it.n0 = it.seg == 0 ? 0 : g.L0 + (it.seg - 1) * g.SEGC;
    it.n1 = min((it.len + C - 1) / C, it.n0 + (it.seg == 0 ? g.L0 : g.SEGC));
    return true;
}

// Segment 0 of head bh of a uniform batch (the lead segment).
__device__ __forceinline__ void lead_item(const Geo& g, int bh, Item& it) {
    it.seg = 0;
    it.G = g.G;
    it.len = g.T;
    it.head_tok = static_cast<size_t>(bh) * g.T;
    it.slot0 = static_cast<size_t>(bh) * g.G;
    it.state = bh;
    it.snap0 = 0;
    it.h = 0;
    it.n0 = 0;
    it.n1 = min((g.T + C - 1) / C, g.L0);
}

// ============================================================ segment maps
// LDS of the map kernel: k and the gates in three copies (chunk n for the
// carriers, n+1 for the stagers, n+2 being written), v and (I + L)^{-1} in two
// by chunk parity.
struct MapTiles {
    u16 Ks[3][C][LDQ];    // chunk m in copy m % 3
    u16 Vs[2][C][LDQ];    // chunk m in copy m & 1
    u16 Tm[2][C][LDA];    // chunk m in copy m & 1
    u16 Lb[C][LDA];
    Gates gt[3];          // chunk m in copy m % 3
};

constexpr int kMapThreads = 768;   // 8 state carriers + 4 stagers

// Waves 0-7 carry the augmented state [N | M] (d_k x 256, starting from
// [0 | I]): waves 0-3 the N columns (value channels 32w..32w+31, with V),
// waves 4-7 the M columns (no V term).  Per chunk, like the output kernel
// without Q, A and the outputs:
//     carriers:  K P, staging | B1 | right-hand side (reads v), solve | B2 |
//                update | B0
//     stagers:   diagonal inverse blocks of chunk n+1 | B1 |
//                L below the diagonal | B2 | inverse below the diagonal (three waves) | B0
// The carriers also stage the inputs, in the first phase, which the stagers'
// diagonal blocks bound: waves 0-3 k and the gates of chunk n+2, waves 4-7 v
// of chunk n+1.
__device__ __forceinline__ void map_body(MapTiles& sm, const Item& it, const u16* __restrict__ k,
                                        const u16* __restrict__ v, const float* __restrict__ alpha,
                                        const float* __restrict__ beta, float* __restrict__ ws) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the branches below are scalar
    const int n0 = it.n0, n1 = it.n1, T = it.len;
    const size_t head_tok = it.head_tok;
    using RC = RawChunk<256, true>;
    if (w < 8) {
        const int r = lane & 15, g = lane >> 4;
        const bool npart = w < 4;
        const int col0 = 32 * (w & 3);
        f32x4 P[2][8];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    P[nt][t][i] = (!npart && perm_row(t, 4 * g + i) == col0 + 16 * nt + r) ? 1.f : 0.f;
        // inputs: waves 0-3 load k and the gates, waves 4-7 v into rc.k (the
        // gates that come with it are not used); chunk n + ahead is staged in
        // the first phase of chunk n, where the carriers' products are shorter
        // than the stagers' diagonal inverse blocks, every index past the
        // segment clamped to its last chunk (no branch around the loads; a
        // clamped copy rewrites a tile with the values it already holds)
        const bool kpart = npart;
        const int ptid = tid & 255, ahead = kpart ? 2 : 1;
        const u16* src = kpart ? k : v;
        RC rc;
        auto fetch = [&](int m) {
            m = min(m, n1 - 1);
            fetch_chunk<false, true, false>(rc, nullptr, src, nullptr, alpha, beta, head_tok, m * C, min(C, T - m * C),
                                            ptid);
        };
        auto stage = [&](int m) {
            m = min(m, n1 - 1);
            const int len = min(C, T - m * C);
            if (kpart) {
                write_gates(sm.gt[m % 3], chunk_gates(rc.a, rc.b, len), lane);
                stage_rows<RC>(sm.Ks[m % 3], rc.k, ptid, len);
            } else {
                stage_rows<RC>(sm.Vs[m & 1], rc.k, ptid, len);
            }
        };
        fetch(n0);
        stage(n0);
        fetch(n0 + 1);
        lds_barrier();  // k, gates and v of chunk n0 staged
        lds_barrier();  // B1, B2, B0 of the stagers' chunk n0
        lds_barrier();
        if (kpart) {   // k of chunk n0 + 1 before the stagers start on it
            stage(n0 + 1);
            fetch(n0 + 2);
        }
        lds_barrier();
        for (int n = n0; n < n1; ++n) {
            const int c3 = n % 3, cb = n & 1;
            const Gates& gt = sm.gt[c3];
            f32x4 O[2][4], X[2][4];
            bf16x8 Xb[2][2], Ub[2][2], Ue[2][2];
            scan_qk<2, false>(nullptr, sm.Ks[c3], P, lane, O, X);
            stage(n + ahead);
            fetch(n + ahead + 1);
            lds_barrier();  // B1
            if (npart)
                scan_rhs<2, true>(sm.Vs[cb], gt, X, col0, lane, Xb);
            else
                scan_rhs<2, false>(sm.Vs[cb], gt, X, col0, lane, Xb);
            TriOps tm;
            load_tri(tm, sm.Tm[cb], lane);
            scan_solve<2, false>(tm, gt, Xb, lane, Ub, Ue);
            lds_barrier();  // B2
            scan_update<2>(sm.Ks[c3], gt, P, Ue, lane);
            lds_barrier();  // B0
        }
        if (npart)
            store_state<2>(P, ws + ws_N(it.slot0 + it.seg), col0, lane);
        else
            store_map_frag<2>(P, reinterpret_cast<u16*>(ws + ws_M(it.slot0 + it.seg)), col0, lane);
    } else {
        const int u = w - 8;
        // The blocks (0,1) and (2,3) above the diagonal of Tm are read by
        // 32-wide operand slices and must be zero; nothing else writes them.
        zero_above(sm.Tm[u & 1], (u & 2) ? 5 : 0, lane);
        lds_barrier();  // the carriers staged chunk n0
        for (int m = n0; m < n1; ++m) {
            const int c3 = m % 3, cb = m & 1;
            step1_diag(sm.Ks[c3], sm.Tm[cb], sm.gt[c3], u, lane);
            lds_barrier();  // B1
            step1_below(sm.Ks[c3], sm.Lb, sm.gt[c3], u, u < 2 ? u + 4 : u, u < 2, lane);
            lds_barrier();  // B2
            if (u == 0)
                step2_inverse_below<0>(sm.Tm[cb], sm.Lb, lane);
            else if (u == 1)
                step2_inverse_below<1>(sm.Tm[cb], sm.Lb, lane);
            else if (u == 2)
                step2_inverse_below<2>(sm.Tm[cb], sm.Lb, lane);
            lds_barrier();  // B0
        }
        lds_barrier();  // B1, B2, B0 of the carriers' last chunk
        lds_barrier();
        lds_barrier();
    }
}


__global__ __launch_bounds__(kMapThreads) void gdn_map_kernel(Geo geo, const u16* __restrict__ k,
                                                              const u16* __restrict__ v,
                                                              const float* __restrict__ alpha,
                                                              const float* __restrict__ beta, float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) MapTiles sm;
    Item it;
    if (!find_item(geo, blockIdx.x, true, it)) return;
    map_body(sm, it, k, v, alpha, beta, ws);
}

// ============================================================ combine
// One workgroup (4 waves) per (head, 16 value channels): P_0 = S0,
// P_{s+1} = M_s P_s + N_s, writing every P_s that the output pass reads (from
// P_1 on when the lead kernel has run segment 0 and written P_1).  The products run on MFMA with
// both operands split into bf16 high and low parts (hi*hi + hi*lo + lo*hi),
// which keeps about 16 significant bits.  Wave w owns d rows 32w..32w+31.
constexpr int kCombineThreads = 256;

__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    float h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        h[j] = bf16_bits_to_f32(f32_to_bf16_bits(x[j]));
        l[j] = x[j] - h[j];
    }
    hi = pack8(h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]);
    lo = pack8(l[0], l[1], l[2], l[3], l[4], l[5], l[6], l[7]);
}

__global__ __launch_bounds__(kCombineThreads) void gdn_combine_kernel(Geo geo, const float* S0,
                                                                      float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) float Ps[2][16][D + 4];  // P_s by parity: [value channel][j]
    // Workgroups are dealt to the 8 XCDs round-robin (each XCD has its own
    // L2): the 8 column tiles of one (sequence, head) take block indices 8
    // apart, so all of them land on one XCD and share its maps in that L2.
    const int i = blockIdx.x;
    const int bh = (i >> 6) * 8 + (i & 7);   // (sequence, head) pair
    const int tile = (i >> 3) & 7;
    int G;
    size_t slot0, state;
    if (geo.cu == nullptr) {
        if (bh >= geo.BH) return;
        G = geo.G;
        slot0 = static_cast<size_t>(bh) * G;
        state = bh;
    } else {
        if (bh >= geo.N * geo.H) return;
        const int n = bh / geo.H, h = bh % geo.H;
        G = geo.seg_base[n + 1] - geo.seg_base[n];
        if (geo.seg_base[n + 1] > geo.Gcap) return;   // (see find_item)
        slot0 = static_cast<size_t>(h) * geo.Gcap + geo.seg_base[n];
        state = bh;
    }
    // with a lead segment the chain starts from P_1, which pass 1 wrote
    const int s0 = geo.cu == nullptr ? geo.lead : 0;
    if (G < 2 + s0) return;   // a single segment starts from S0 itself (or P_1 is the last state needed)
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    // P_0 = S0 (zeros when absent), or P_1, for value channels 16 tile .. +15
    for (int e = tid; e < 16 * D / 4; e += kCombineThreads) {
        const int rl = e / (D / 4), d4 = (e % (D / 4)) * 4;
        const size_t off = static_cast<size_t>(16 * tile + rl) * D + d4;
        const float4 x = s0 ? *reinterpret_cast<const float4*>(ws + ws_P(slot0 + 1) + off)
                         : S0 ? *reinterpret_cast<const float4*>(S0 + state * kMat + off)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(&Ps[0][rl][d4]) = x;
        if (!s0) *reinterpret_cast<float4*>(ws + ws_P(slot0) + off) = x;
    }
    // The maps (M_s, N_s) do not depend on the states: they are loaded two
    // steps ahead into a ring of two register sets (M already split into its
    // bf16 halves by the map kernel).  Lane (r, g) of wave w uses rows
    // d = 32w + 16mt + r of M (8 columns per k-step) and rows
    // d = 32w + 16mt + 4g .. +3 of column v = r of N.
    bf16x8 mh[2][2][4], ml[2][2][4];
    f32x4 nv[2][2];
    auto load_maps = [&](int st, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        const u16* Mh = reinterpret_cast<const u16*>(ws + ws_M(slot0 + st));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                // M[32w + 16mt + r][32ks + 8g .. +7] in the operand order of map_frag
                const size_t at = static_cast<size_t>(((w * 2 + mt) * 4 + ks) * 64 + lane) * 8;
                mh[B][mt][ks] = *reinterpret_cast<const bf16x8*>(Mh + at);
                ml[B][mt][ks] = *reinterpret_cast<const bf16x8*>(Mh + kMapHalf + at);
            }
            const float4 x = *reinterpret_cast<const float4*>(ws + ws_N(slot0 + st) +
                                                              static_cast<size_t>(16 * tile + r) * D + 32 * w +
                                                              16 * mt + 4 * g);
            nv[B][mt] = f32x4{x.x, x.y, x.z, x.w};
        }
    };
    // step s: P_{s+1} = M_s P_s + N_s with the maps in ring slot B = (s - s0) & 1
    auto step = [&](int s, auto bufc) {
        constexpr int B = decltype(bufc)::value;
        lds_barrier();
        f32x4 acc[2] = {nv[B][0], nv[B][1]};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 ph, pl;
            split8(&Ps[B][r][32 * ks + 8 * g], ph, pl);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                acc[mt] = mfma16x16x32(mh[B][mt][ks], ph, acc[mt]);
                acc[mt] = mfma16x16x32(mh[B][mt][ks], pl, acc[mt]);
                acc[mt] = mfma16x16x32(ml[B][mt][ks], ph, acc[mt]);
            }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            // lane holds P_{s+1}[d = 32w+16mt+4g+i][v = r]
            const int d0 = 32 * w + 16 * mt + 4 * g;
            const float4 x = make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]);
            *reinterpret_cast<float4*>(&Ps[B ^ 1][r][d0]) = x;
            *reinterpret_cast<float4*>(ws + ws_P(slot0 + s + 1) + static_cast<size_t>(16 * tile + r) * D + d0) = x;
        }
        if (s + 2 <= G - 2) load_maps(s + 2, bufc);   // the maps two steps on, into the slot just used
    };
    using b0 = std::integral_constant<int, 0>;
    using b1 = std::integral_constant<int, 1>;
    load_maps(s0, b0{});
    if (s0 + 1 <= G - 2) load_maps(s0 + 1, b1{});
    for (int s = s0; s + 1 < G; s += 2) {
        step(s, b0{});
        if (s + 2 < G) step(s + 1, b1{});
    }
}

// ============================================================ outputs
// LDS of the output kernel.  Chunk m's k, (I + L)^{-1}, A and gates sit in
// copy m & 1: the stagers fill copy m+1 while the state carriers read copy m.
// q and v have one copy each; each is rewritten only after the carriers' last
// read of the previous chunk's.
struct OutTiles {
    u16 Ks[2][C][LDQ];
    u16 Qs[C][LDQ];
    u16 Vs[C][LDQ];
    u16 Os[C][LDQ];      // output staging (state carriers)
    u16 Tm[2][C][LDA];   // (I + L)^{-1}
    u16 As[2][C][LDA];   // decay-masked Q K^T
    u16 Lb[C][LDA];      // -L (stagers only)
    Gates gt[2];
};

// Waves 0-3 carry the state (32 value channels each) and compute, per chunk,
//     O = diag(e^g) Q P + A U,   U = (I + L)^{-1} diag(beta) (V - diag(e^g) K P),
//     P <- e^{g_c} P + K^T diag(e^{g_c - g}) U
// (the chunk form above with W and Ut folded: W P = (I + L)^{-1} diag(beta e^g) K P,
// so no chunk-sized W or Ut tile is formed).  Waves 4-7 stage chunk m+1 and
// form its state-independent tiles (L, (I + L)^{-1}, A) while the carriers run
// chunk m.  Every chunk has three barriers, met by both roles:
//     carriers:  Q P and K P | B1 | right-hand side (reads v), solve, diagonal inverse
//                blocks of chunk n+1 | B2 | outputs, update | B0
//     stagers:   k + gates of chunk n+1 | B1 | L below the diagonal, q | B2 |
//                inverse below the diagonal (three waves), A, v | B0
// The stagers run one chunk ahead: they stage chunk n0 while the carriers
// wait, and wait through the carriers' last chunk.
template <int NCAR>
__device__ __forceinline__ void out_body(OutTiles& sm, const Geo& geo, const Item& it, const u16* __restrict__ q,
                                        const u16* __restrict__ k, const u16* __restrict__ v,
                                        const float* __restrict__ alpha, const float* __restrict__ beta,
                                        const float* Sin, float* Send, u16* __restrict__ o) {
    constexpr int NT = 128 / 16 / NCAR;   // 16-column tiles per carrier
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the branches below are scalar
    const int n0 = it.n0, n1 = it.n1, T = it.len;
    const size_t head_tok = it.head_tok;
    if (w < NCAR) {
        const int col0 = 16 * NT * w;
        f32x4 P[NT][8];
        load_state<NT>(P, Sin, col0, lane);
        // diagonal block w of (I + L)^{-1} of chunk m (staged before the last B1), waves 0-3
        auto diag = [&](int m) {
            if (NCAR == 4 || w < 4) step1_diag(sm.Ks[m & 1], sm.Tm[m & 1], sm.gt[m & 1], w, lane);
        };
        lds_barrier();  // B1, B2, B0 of chunk n0's staging
        diag(n0);
        lds_barrier();
        lds_barrier();
        for (int n = n0; n < n1; ++n) {
            const int cb = n & 1;
            const Gates& gt = sm.gt[cb];
            f32x4 O[NT][4], X[NT][4];
            bf16x8 Xb[NT][2], Ub[NT][2], Ue[NT][2];
            scan_qk<NT, true>(sm.Qs, sm.Ks[cb], P, lane, O, X);
            lds_barrier();  // B1
            TriOps tm, am;
            load_tri(tm, sm.Tm[cb], lane);
            scan_rhs<NT, true>(sm.Vs, gt, X, col0, lane, Xb);
            scan_solve<NT, true>(tm, gt, Xb, lane, Ub, Ue);
            load_tri(am, sm.As[cb], lane);   // A of chunk n was formed during chunk n - 1
            if (n + 1 < n1) diag(n + 1);
            lds_barrier();  // B2
            const int t0 = n * C;
            scan_out<NT>(am, gt, O, Ub, col0, lane, o, head_tok + t0, min(C, T - t0), sm.Os);
            scan_update<NT>(sm.Ks[cb], gt, P, Ue, lane);
            // snapshot of the state after chunk n (packed batches)
            const int end = (n + 1) * C;
            if (geo.snap > 0 && end <= T && end % geo.snap == 0) {
                const int j = it.snap0 + end / geo.snap - 1;
                if (j < geo.snap_cap)
                    store_state<NT>(P, geo.S_snap + (static_cast<size_t>(j) * geo.H + it.h) * kMat, col0, lane);
            }
            lds_barrier();  // B0
        }
        if (Send) store_state<NT>(P, Send, col0, lane);
    } else {
        const int ptid = tid - 64 * NCAR;
        const int u = w - NCAR;
        // The blocks (0,1) and (2,3) above the diagonal of Tm and A are read by
        // 32-wide operand slices and must be zero; nothing else writes them.
        zero_above((u & 2) ? sm.As[u & 1] : sm.Tm[u & 1], 0, lane);
        zero_above((u & 2) ? sm.As[u & 1] : sm.Tm[u & 1], 5, lane);
        // Each tensor of chunk m+1 is fetched right after the same tensor of
        // chunk m is staged (the last chunk fetches itself again).
        using RC = RawChunk<256, true>;
        RC rc;
        using yes = std::true_type;
        using no = std::false_type;
        auto fetch = [&](int m, auto with_q, auto with_k, auto with_v) {
            fetch_chunk<decltype(with_q)::value, decltype(with_k)::value, decltype(with_v)::value>(
                rc, q, k, v, alpha, beta, head_tok, m * C, min(C, T - m * C), ptid);
        };
        // the same issue order as inside the loop (k and gates, q, v), so the
        // wait before each staging step is as short there as on every later chunk
        fetch(n0, no{}, yes{}, no{});
        __builtin_amdgcn_sched_barrier(0);
        fetch(n0, yes{}, no{}, no{});
        __builtin_amdgcn_sched_barrier(0);
        fetch(n0, no{}, no{}, yes{});
        __builtin_amdgcn_sched_barrier(0);
        for (int m = n0; m < n1; ++m) {
            const int cb = m & 1, len = min(C, T - m * C), mn = min(m + 1, n1 - 1);
            write_gates(sm.gt[cb], chunk_gates(rc.a, rc.b, len), lane);
            stage_rows<RC>(sm.Ks[cb], rc.k, ptid, len);
            fetch(mn, no{}, yes{}, no{});
            lds_barrier();  // B1
            step1_below(sm.Ks[cb], sm.Lb, sm.gt[cb], u, u < 2 ? u + 4 : u, u < 2, lane);
            stage_rows<RC>(sm.Qs, rc.q, ptid, len);
            fetch(mn, yes{}, no{}, no{});
            lds_barrier();  // B2
            // the inverse in three parts (waves 0-2) and blocks 0..9 of A:
            // waves 0 and 1 two each, waves 2 and 3 three each
            if (u == 0)
                step2_inverse_below<0>(sm.Tm[cb], sm.Lb, lane);
            else if (u == 1)
                step2_inverse_below<1>(sm.Tm[cb], sm.Lb, lane);
            else if (u == 2)
                step2_inverse_below<2>(sm.Tm[cb], sm.Lb, lane);
            if (u < 2)
                step2_qk<2>(sm.Qs, sm.Ks[cb], sm.As[cb], sm.gt[cb], 2 * u, lane);
            else
                step2_qk<3>(sm.Qs, sm.Ks[cb], sm.As[cb], sm.gt[cb], 3 * u - 2, lane);
            stage_rows<RC>(sm.Vs, rc.v, ptid, len);
            fetch(mn, no{}, no{}, yes{});
            lds_barrier();  // B0
        }
        lds_barrier();  // B1, B2, B0 of the last chunk's scan
        lds_barrier();
        lds_barrier();
    }
}

__global__ __launch_bounds__(kThreads) void gdn_out_kernel(Geo geo, const u16* __restrict__ q,
                                                           const u16* __restrict__ k, const u16* __restrict__ v,
                                                           const float* __restrict__ alpha,
                                                           const float* __restrict__ beta, const float* S0,
                                                           const float* __restrict__ ws, u16* __restrict__ o,
                                                           float* S_out) {
    __shared__ __attribute__((aligned(16))) OutTiles sm;
    Item it;
    if (!find_item(geo, blockIdx.x, false, it)) return;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float* S0h = S0 ? S0 + it.state * kMat : nullptr;
    float* Send = it.seg == it.G - 1 && S_out ? S_out + it.state * kMat : nullptr;
    if (it.n0 >= it.n1) {   // an empty sequence: its state passes through
        if (w < 4 && S_out) {
            f32x4 P[2][8];
            load_state<2>(P, S0h, 32 * w, threadIdx.x & 63);
            store_state<2>(P, S_out + it.state * kMat, 32 * w, threadIdx.x & 63);
        }
        return;
    }
    // entering state: S0 itself when the sequence is one segment, else the
    // combined state (segment 0 included, so S_out may alias S0)
    out_body<4>(sm, geo, it, q, k, v, alpha, beta, it.G == 1 ? S0h : ws + ws_P(it.slot0 + it.seg), Send, o);
}

// ---- pass 1 with a lead segment (uniform batches).  The map pass has one
// workgroup fewer per head than the output pass (the last segment needs no
// map), so it leaves CUs idle; with a lead segment, workgroups 0..BH-1 run
// segment 0 of their head from S0 instead (its outputs, and its final state
// P_1 into the workspace), while the others compute the maps of segments
// 1..G-2.  The output pass then runs segments 1..G-1.  Both roles use the
// map kernel's 768 threads: the lead role runs the output kernel's work with
// eight carriers of 16 value channels (and the four stagers).
union PassOneTiles {
    MapTiles m;
    OutTiles o;
};

__global__ __launch_bounds__(kMapThreads) void gdn_lead_map_kernel(Geo geo, const u16* __restrict__ q,
                                                                   const u16* __restrict__ k,
                                                                   const u16* __restrict__ v,
                                                                   const float* __restrict__ alpha,
                                                                   const float* __restrict__ beta, const float* S0,
                                                                   float* __restrict__ ws, u16* __restrict__ o) {
    __shared__ __attribute__((aligned(16))) PassOneTiles sm;
    Item it;
    const int blk = blockIdx.x;
    if (blk < geo.BH) {
        lead_item(geo, blk, it);
        out_body<8>(sm.o, geo, it, q, k, v, alpha, beta, S0 ? S0 + it.state * kMat : nullptr,
                    ws + ws_P(it.slot0 + 1), o);
        return;
    }
    if (!find_item(geo, blk - geo.BH, true, it)) return;
    map_body(sm.m, it, k, v, alpha, beta, ws);
}

struct Plan {
    int NC, G, SEGC;
    int L0, lead;   // chunks of segment 0; whether it runs in the map pass
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
    p.L0 = p.SEGC;
    p.lead = 0;
    return p;
}

// Expected time of a plan, in output-pass chunk times: the longest map-pass
// workgroup, the combine chain and the longest output-pass workgroup.  Per
// chunk, measured against an output-pass chunk: a map chunk 0.94-1.045 (taken
// as 1), a lead chunk (eight 16-channel carriers) 1.25 (taken as 1.3, so that
// the lead segment does not set the pace), a combine step 0.45.
double plan_cost(const Plan& p) {
    if (p.G < 2) return p.NC;
    if (!p.lead) return p.SEGC + 0.45 * (p.G - 1) + p.SEGC;
    const double pass1 = std::max(1.3 * p.L0, p.G > 2 ? 1.0 * p.SEGC : 0.0);
    return pass1 + 0.45 * (p.G - 2) + p.SEGC;
}

// The plan of a whole prefill call: with a lead segment (segment 0 in the map
// pass, G = slots + 1 segments, segments 1..G-1 of SEGC chunks and segment 0
// of the rest) when that is expected to be at least 3% faster, else the plain
// plan.  gdn_prefill_prep / gdn_prefill_scan always use the plain plan (the
// lead segment needs S0 and writes o, which prep does not take).
Plan make_step_plan(int BH, int T) {
    Plan best = make_plan(BH, T);
    if (best.G < 2 || BH <= 0) return best;
    const int slots = kTargetBlocks / BH;
    if (slots < 2) return best;
    const double plain = plan_cost(best);
    double best_cost = 0.97 * plain;
    for (int S = (best.NC + slots) / (slots + 1); S >= 1 && slots * S < best.NC; ++S) {
        Plan q;
        q.NC = best.NC;
        q.G = slots + 1;
        q.SEGC = S;
        q.L0 = best.NC - slots * S;
        q.lead = 1;
        if (q.L0 < 1) continue;
        const double c = plan_cost(q);
        if (c < best_cost) {
            best_cost = c;
            best = q;
        }
    }
    return best;
}

Geo uniform_geo(const Plan& p, int BH, int T) {
    Geo g{};
    g.BH = BH;
    g.T = T;
    g.G = p.G;
    g.SEGC = p.SEGC;
    g.L0 = p.L0;
    g.lead = p.lead;
    return g;
}

// ---- packed batches: plan on the host from N and Ttot only (the sequence
// lengths stay on the device).  A sequence of NC chunks gets ceil(NC/SEGC)
// segments (one when empty); SEGC is chosen so that about kTargetBlocks
// (segment, head) items exist, and Gcap bounds the total segment count:
// sum ceil(NC_n / SEGC) <= (Ttot / C + N) / SEGC + N.
struct VarPlan {
    int SEGC, Gcap;
    size_t table_bytes;   // seg_base and snap_base, [N+1] each, rounded to 256 bytes
};

VarPlan make_var_plan(int N, int H, int Ttot) {
    VarPlan p;
    const long long chunks = static_cast<long long>(Ttot) / C + N;   // >= sum of per-sequence chunk counts
    long long segc = (chunks * H + kTargetBlocks - 1) / kTargetBlocks;
    if (segc < 1) segc = 1;
    p.SEGC = static_cast<int>(segc);
    p.Gcap = static_cast<int>(chunks / segc + N + 1);
    // seg_base, snap_base ([N+1] each), order ([Gcap])
    p.table_bytes = ((2 * (static_cast<size_t>(N) + 1) + p.Gcap) * sizeof(int) + 255) / 256 * 256;
    return p;
}

// seg_base and snap_base by a block-wide exclusive scan over the sequences;
// with `order`, then a counting sort of the segments by descending chunk count
// (bins in LDS, positions taken with LDS atomics: the order within a bin is
// arbitrary, and every workgroup computes the same thing whatever its place).
constexpr int kPlanThreads = 1024;

// Inclusive prefix sum over the plan kernel's threads: a shuffle scan in each
// wave, then one over the wave totals (tot: kPlanThreads / 64 ints of LDS,
// not shared with another scan in flight).
__device__ __forceinline__ int plan_scan(int x, int* tot) {
    constexpr int kWaves = kPlanThreads / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) tot[wv] = x;
    __syncthreads();
    if (wv == 0) {
        int t = lane < kWaves ? tot[lane] : 0;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const int y = __shfl_up(t, d, 64);
            if (lane >= d) t += y;
        }
        if (lane < kWaves) tot[lane] = t;
    }
    __syncthreads();
    return wv > 0 ? x + tot[wv - 1] : x;
}

__global__ __launch_bounds__(kPlanThreads) void gdn_varlen_plan_kernel(int N, int Ttot, int SEGC, int snap,
                                                                       const int* __restrict__ cu, int* seg_base,
                                                                       int* snap_base, int* order, int cap,
                                                                       int* seq_order) {
    __shared__ int hist[kPlanThreads];
    __shared__ int tot[4][kPlanThreads / 64];
    const int tid = threadIdx.x;
    const int per = (N + kPlanThreads - 1) / kPlanThreads;
    const int a = min(N, tid * per), b = min(N, a + per);
    auto counts = [&](int n, int& segs, int& snaps, int& nc) {
        const int t0 = clamp_tok(cu[n], Ttot), t1 = clamp_tok(cu[n + 1], Ttot);
        const int len = t1 > t0 ? t1 - t0 : 0;
        nc = (len + C - 1) / C;
        segs = nc > 0 ? (nc + SEGC - 1) / SEGC : 1;
        snaps = snap > 0 ? len / snap : 0;
    };
    int ss = 0, sn = 0;
    for (int n = a; n < b; ++n) {
        int g, z, nc;
        counts(n, g, z, nc);
        ss += g;
        sn += z;
    }
    const int ss_incl = plan_scan(ss, tot[0]);
    const int sn_incl = plan_scan(sn, tot[1]);
    const int gb0 = ss_incl - ss;   // exclusive
    int gb = gb0, zb = sn_incl - sn;
    for (int n = a; n < b; ++n) {
        seg_base[n] = gb;
        snap_base[n] = zb;
        int g, z, nc;
        counts(n, g, z, nc);
        gb += g;
        zb += z;
    }
    if (tid == kPlanThreads - 1) {
        seg_base[N] = ss_incl;
        snap_base[N] = sn_incl;
    }
    if (order == nullptr && seq_order == nullptr) return;
    // ---- longest first: bin kPlanThreads - 1 - chunks (chunk counts past the
    // last bin share it), histogram, exclusive scan, scatter
    auto sort_by_chunks = [&](auto&& each, int* t) {
        __syncthreads();   // the previous scatter's atomics are done
        hist[tid] = 0;
        __syncthreads();
        each([&](int, int bin) { atomicAdd(&hist[bin], 1); });
        __syncthreads();
        const int own = hist[tid];
        const int incl = plan_scan(own, t);
        hist[tid] = incl - own;   // exclusive: the first position of bin tid
        __syncthreads();
    };
    auto bin_of = [&](int chunks) { return kPlanThreads - 1 - min(max(chunks, 0), kPlanThreads - 1); };
    // sequences (seq_order: every sequence, by its chunk count)
    auto each_sequence = [&](auto&& fn) {
        for (int n = a; n < b; ++n) {
            int g, z, nc;
            counts(n, g, z, nc);
            fn(n, bin_of(nc));
        }
    };
    if (seq_order) {
        sort_by_chunks(each_sequence, tot[2]);
        each_sequence([&](int n, int bin) { seq_order[atomicAdd(&hist[bin], 1)] = n; });
    }
    if (order == nullptr) return;
    auto each_segment = [&](auto&& fn) {
        int base = gb0;
        for (int n = a; n < b; ++n) {
            int g, z, nc;
            counts(n, g, z, nc);
            for (int s = 0; s < g && base + s < cap; ++s) {
                const int ch = min(SEGC, nc - s * SEGC);   // 0 for an empty sequence
                fn(base + s, bin_of(ch));
            }
            base += g;
        }
    };
    sort_by_chunks(each_segment, tot[3]);
    each_segment([&](int gs, int bin) { order[atomicAdd(&hist[bin], 1)] = gs; });
}

hipError_t launch_all(const Geo& g, long long map_blocks, long long combine_items, long long out_blocks,
                      const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                      const float* S0, void* o, float* S_out, float* ws, bool prep, bool scan, hipStream_t stream) {
    if (!grid_fits(prep ? map_blocks : 0, kMapThreads) ||
        !grid_fits(scan ? (combine_items + 7) / 8 * 64 : 0, kCombineThreads) ||
        !grid_fits(scan ? out_blocks : 0, kThreads))
        return hipErrorInvalidConfiguration;
    if (prep && map_blocks > 0) {
        hipLaunchKernelGGL(gdn_map_kernel, dim3(static_cast<unsigned>(map_blocks)), dim3(kMapThreads), 0, stream, g,
                           static_cast<const u16*>(k), static_cast<const u16*>(v), alpha, beta, ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!scan) return hipSuccess;
    if (combine_items > 0) {
        hipLaunchKernelGGL(gdn_combine_kernel, dim3(static_cast<unsigned>((combine_items + 7) / 8) * 64),
                           dim3(kCombineThreads), 0, stream, g, S0, ws);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gdn_out_kernel, dim3(static_cast<unsigned>(out_blocks)), dim3(kThreads), 0, stream, g,
                       static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v), alpha, beta,
                       S0, ws, static_cast<u16*>(o), S_out);
    return hipGetLastError();
}

hipError_t launch_uniform(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                          const float* beta, const float* S0, void* o, float* S_out, void* workspace, bool prep,
                          bool scan, hipStream_t stream) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return hipSuccess;
    const Geo g = uniform_geo(prep && scan ? make_step_plan(BH, T) : make_plan(BH, T), BH, T);
    float* ws = static_cast<float*>(workspace);
    if (g.lead) {   // (G >= 3 by construction: slots >= 2)
        const long long blocks = static_cast<long long>(BH) * (g.G - 1);
        if (!grid_fits(blocks, kMapThreads) || !grid_fits((BH + 7LL) / 8 * 64, kCombineThreads) ||
            !grid_fits(blocks, kThreads))
            return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(gdn_lead_map_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kMapThreads), 0,
                           stream, g, static_cast<const u16*>(q), static_cast<const u16*>(k),
                           static_cast<const u16*>(v), alpha, beta, S0, ws, static_cast<u16*>(o));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_all(g, 0, BH, blocks, q, k, v, alpha, beta, S0, o, S_out, ws, false, true, stream);
    }
    const bool multi = g.G > 1;
    const long long bh = BH;
    return launch_all(g, multi ? bh * (g.G - 1) : 0, multi ? bh : 0, bh * g.G, q, k, v, alpha, beta, S0, o, S_out,
                      ws, prep, scan, stream);
}

// ---- a workspace held by the library, for callers that cannot allocate.
// The plain uniform plan makes at most kTargetBlocks (head, segment) items and
// the lead plan BH (slots + 1) with slots = kTargetBlocks / BH >= 2, so at
// most kTargetBlocks + kTargetBlocks / 2: kScratchBytes (72 MiB) covers every
// uniform call.  The array is part of the code object: each device the
// library runs on holds its own copy from the first launch until the process
// ends.  Host code must not use the
// array's name as an address (on the host it is only a stand-in); the device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current, and is kept per device.
constexpr size_t kScratchBytes = static_cast<size_t>(kTargetBlocks + kTargetBlocks / 2) * 3 * kMat * sizeof(float);
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex scratch_mutex;
void* scratch_ptr[kScratchDevices];

}  // namespace

size_t gdn_scratch_bytes() { return kScratchBytes; }

hipError_t gdn_scratch(void** out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

bool gdn_mfma_supported(int dtype, int dk, int dv, int chunk) {
    static_assert(C == kMfmaChunk, "the matrix-core kernels share one block length");
    return dtype == kBF16 && dk == D && dv == D && mfma_chunk_ok(chunk);
}

size_t gdn_mfma_workspace_bytes(int B, int H, int T, int, int, int) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return 0;
    // one size for gdn_prefill (plain or lead plan) and prep / scan (plain)
    const Plan p = make_plan(BH, T), s = make_step_plan(BH, T);
    const int G = std::max(p.G, s.G);
    if (G == 1) return 0;
    return static_cast<size_t>(BH) * G * 3 * kMat * sizeof(float);
}

hipError_t launch_gdn_mfma_prep(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, void* workspace, hipStream_t stream) {
    return launch_uniform(B, H, T, q, k, v, alpha, beta, nullptr, nullptr, nullptr, workspace, true, false, stream);
}

hipError_t launch_gdn_mfma_scan(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* S0, void* o, float* S_out, void* workspace,
                                hipStream_t stream) {
    return launch_uniform(B, H, T, q, k, v, alpha, beta, S0, o, S_out, workspace, false, true, stream);
}

hipError_t launch_gdn_mfma(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S0, void* o, float* S_out, void* workspace,
                           hipStream_t stream) {
    return launch_uniform(B, H, T, q, k, v, alpha, beta, S0, o, S_out, workspace, true, true, stream);
}

hipError_t launch_varlen_table(int N, int Ttot, int segc, int snap, const int* cu, int* tab, hipStream_t stream,
                               int* order, int cap, int* seq_order) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(gdn_varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, N, Ttot, segc < 1 ? 1 : segc,
                       snap, cu, tab, tab + (N + 1), order, order ? cap : 0, seq_order);
    return hipGetLastError();
}

size_t gdn_mfma_varlen_workspace_bytes(int N, int H, int Ttot) {
    if (N <= 0 || H <= 0) return 0;
    const VarPlan p = make_var_plan(N, H, Ttot);
    return p.table_bytes + static_cast<size_t>(H) * p.Gcap * 3 * kMat * sizeof(float);
}

hipError_t launch_gdn_mfma_varlen(int N, int H, int Ttot, const int* cu, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                                  int snap, int snap_cap, float* S_snap, void* workspace, hipStream_t stream) {
    if (N <= 0 || H <= 0) return hipSuccess;
    const VarPlan p = make_var_plan(N, H, Ttot);
    int* tab = static_cast<int*>(workspace);
    Geo g{};
    g.SEGC = p.SEGC;
    g.L0 = p.SEGC;
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
    // (segment, head) items, a bound; the extra workgroups exit.  Every grid
    // is checked before the table kernel runs.
    const long long blocks = static_cast<long long>(p.Gcap) * H, items = static_cast<long long>(N) * H;
    if (!grid_fits(blocks, kMapThreads) || !grid_fits(blocks, kThreads) ||
        !grid_fits((items + 7) / 8 * 64, kCombineThreads))
        return hipErrorInvalidConfiguration;
    const hipError_t e = launch_varlen_table(N, Ttot, p.SEGC, g.snap, cu, tab, stream, tab + 2 * (N + 1), p.Gcap);
    if (e != hipSuccess) return e;
    float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.table_bytes);
    return launch_all(g, blocks, items, blocks, q, k, v, alpha, beta, S0, o, S_out, ws, true, true, stream);
}

}  // namespace la

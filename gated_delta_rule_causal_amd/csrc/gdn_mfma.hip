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
//
// Two kernels:
//  * gdn_prep_kernel - one workgroup per chunk, fully parallel over (b, h,
//    chunk).  Everything that does not depend on the carried state: the
//    gates' prefix sum, K K^T and Q K^T on MFMA, the unit lower-triangular
//    solve (16x16 diagonal blocks inverted by substitution in fp32, the rest
//    as blocked MFMA products), and the workspace tiles W, K~^T =
//    (diag(e^{g_c-g}) K)^T, Ut^T, A and e^g.
//  * gdn_scan_kernel - one wavefront per (b, h, 16-wide value tile), walking
//    the chunks in order.  The wave's slice of the state, P = S_tile^T
//    (d_k x 16, fp32), never leaves its accumulator registers: an MFMA
//    accumulator tile is fed back as the B operand of the next product by
//    permuting the contraction index (see pack_acc_pair in common.hpp), so
//    X = W P, U = Ut - X, P <- e^{g_c} P + K~^T U and O = e^g (Q P) + A U need
//    no cross-lane data movement.  Workgroups are mapped so that all eight
//    value tiles of one head run on the same XCD and share its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace la {

namespace {

constexpr int C = 64;        // chunk length
constexpr int D = 128;       // d_k = d_v
constexpr int LDQ = D + 8;   // bf16 row stride of the staged q/k/v tiles (272 B: conflict-free 16-B reads)
constexpr int LDA = C + 8;   // bf16 row stride of 64-wide tiles
constexpr int kPrepThreads = 256;

// ---- workspace layout, per chunk (all offsets in bytes) -------------------
constexpr size_t kOffW = 0;                                  // W      [C][D]  bf16
constexpr size_t kOffKt = kOffW + size_t(C) * D * 2;          // K~^T   [D][C]  bf16
constexpr size_t kOffUt = kOffKt + size_t(D) * C * 2;         // Ut^T   [D][C]  bf16
constexpr size_t kOffA = kOffUt + size_t(D) * C * 2;          // A      [C][C]  bf16
constexpr size_t kOffEg = kOffA + size_t(C) * C * 2;          // e^{g_i} [C] fp32, then e^{g_c}
constexpr size_t kChunkBytes = kOffEg + 512;

typedef short short4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16(short4v a, short4v b, f32x4 c) {
    // v_mfma_f32_16x16x16_bf16: lane (r = l%16, g = l/16) holds A[r][4g..4g+3],
    // B[4g..4g+3][r]; the accumulator holds D[4g..4g+3][r].  K = 16 equals the
    // accumulator's row span, so an accumulator tile is directly a B operand.
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short4v to_bf16x4(f32x4 x) {
    short4v r;
    r[0] = static_cast<short>(f32_to_bf16_bits(x[0]));
    r[1] = static_cast<short>(f32_to_bf16_bits(x[1]));
    r[2] = static_cast<short>(f32_to_bf16_bits(x[2]));
    r[3] = static_cast<short>(f32_to_bf16_bits(x[3]));
    return r;
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const u16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ short4v lds_short4(const u16* p) { return *reinterpret_cast<const short4v*>(p); }

// ============================================================ prep kernel
__global__ __launch_bounds__(kPrepThreads) void gdn_prep_kernel(
    int T, int NC, const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, unsigned char* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) u16 Qs[C][LDQ];   // later: staging of W
    __shared__ __attribute__((aligned(16))) u16 Ks[C][LDQ];
    __shared__ __attribute__((aligned(16))) u16 Vs[C][LDQ];
    __shared__ __attribute__((aligned(16))) u16 Lb[C][LDA];   // -L as bf16 (blocks below the diagonal)
    __shared__ __attribute__((aligned(16))) u16 As[C][LDA];   // decay-masked Q K^T
    __shared__ __attribute__((aligned(16))) u16 Ts[4][16][24];  // inverses of the diagonal blocks of I + L
    __shared__ float Ld[4][16][17];                           // diagonal blocks of L, fp32
    __shared__ float gs[C], bs[C], egs[C];

    const int chunk = blockIdx.x;
    const int bh = chunk / NC;
    const int n = chunk - bh * NC;
    const int t0 = n * C;
    const int len = min(C, T - t0);
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int r = lane & 15;
    const int g = lane >> 4;
    unsigned char* wsc = ws + static_cast<size_t>(chunk) * kChunkBytes;

    // ---- 1. stage the chunk's q, k, v (rows past the sequence end are zero)
    const size_t base = (static_cast<size_t>(bh) * T + t0) * D;
    for (int e = tid; e < C * D / 8; e += kPrepThreads) {
        const int row = e >> 4, c8 = (e & 15) * 8;
        uint4 vq = make_uint4(0, 0, 0, 0), vk = vq, vv = vq;
        if (row < len) {
            const size_t gi = base + static_cast<size_t>(row) * D + c8;
            vq = *reinterpret_cast<const uint4*>(q + gi);
            vk = *reinterpret_cast<const uint4*>(k + gi);
            vv = *reinterpret_cast<const uint4*>(v + gi);
        }
        *reinterpret_cast<uint4*>(&Qs[row][c8]) = vq;
        *reinterpret_cast<uint4*>(&Ks[row][c8]) = vk;
        *reinterpret_cast<uint4*>(&Vs[row][c8]) = vv;
    }
    if (w == 0) {
        // chunk-local g_i = sum_{j<=i} log alpha_j; padded tokens: alpha = 1, beta = 0
        const size_t gi = static_cast<size_t>(bh) * T + t0 + lane;
        float x = lane < len ? __logf(alpha[gi]) : 0.f;
        const float bt = lane < len ? beta[gi] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        gs[lane] = x;
        bs[lane] = bt;
        egs[lane] = __expf(x);
    }
    __syncthreads();

    // ---- 2. K K^T and Q K^T for row tile w; L and A in their final forms
    for (int ct = 0; ct < 4; ++ct) {
        if (ct <= w) {
            f32x4 acck = zero4(), accq = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 ak = lds_bf16x8(&Ks[16 * w + r][32 * s + 8 * g]);
                const bf16x8 aq = lds_bf16x8(&Qs[16 * w + r][32 * s + 8 * g]);
                const bf16x8 bk = lds_bf16x8(&Ks[16 * ct + r][32 * s + 8 * g]);
                acck = mfma16x16x32(ak, bk, acck);
                accq = mfma16x16x32(aq, bk, accq);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * w + 4 * g + i, col = 16 * ct + r;
                const float dec = __expf(fminf(gs[row] - gs[col], 0.f));
                const float lval = col < row ? bs[row] * dec * acck[i] : 0.f;
                const float aval = col <= row ? dec * accq[i] : 0.f;
                Lb[row][col] = f32_to_bf16_bits(-lval);
                As[row][col] = f32_to_bf16_bits(aval);
                if (ct == w) Ld[w][4 * g + i][r] = lval;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) As[16 * w + 4 * g + i][16 * ct + r] = 0;
        }
    }
    __syncthreads();

    // ---- 3. wave 0: inverses of the four 16x16 diagonal blocks of I + L by
    //         forward substitution, one column per lane, fp32.
    //         waves 1-3: emit K~^T, A and e^g to the workspace.
    if (w == 0) {
        const int b = lane >> 4, c = lane & 15;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float val = rr == c ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < rr; ++j) val = fmaf(-Ld[b][rr][j], x[j], val);
            x[rr] = val;
            Ts[b][rr][c] = f32_to_bf16_bits(val);
        }
    } else {
        const int t3 = tid - 64;
        const float gl = gs[C - 1];
        for (int e = t3; e < D * (C / 8); e += kPrepThreads - 64) {
            const int d = e >> 3, c0 = (e & 7) * 8;
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                x[j] = bf16_bits_to_f32(Ks[c0 + j][d]) * __expf(gl - gs[c0 + j]);
            *reinterpret_cast<bf16x8*>(wsc + kOffKt + (static_cast<size_t>(d) * C + c0) * 2) =
                pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
        }
        for (int e = t3; e < C * (C / 8); e += kPrepThreads - 64) {
            const int row = e >> 3, c8 = (e & 7) * 8;
            *reinterpret_cast<uint4*>(wsc + kOffA + (static_cast<size_t>(row) * C + c8) * 2) =
                *reinterpret_cast<const uint4*>(&As[row][c8]);
        }
        // e^g, e^{g_c}, and 16 zero bytes at byte 272 (the source of padded q rows in the scan)
        float* egw = reinterpret_cast<float*>(wsc + kOffEg);
        if (t3 < C) egw[t3] = egs[t3];
        if (t3 == C) egw[C] = egs[C - 1];
        if (t3 > C && t3 <= C + 3 + 4) egw[t3] = 0.f;
    }
    __syncthreads();

    // ---- 4. blocked forward substitution on MFMA.  Waves 0,1 solve for the
    //         64-column halves of W, waves 2,3 for those of Ut:
    //         X_rb = T_rb,rb (RHS_rb - sum_{kb<rb} L_rb,kb X_kb)
    {
        const bool isW = w < 2;
        const int cb = (w & 1) * 64;
        const u16(*src)[LDQ] = isW ? Ks : Vs;
        short4v Xb[4][4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            f32x4 acc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rb + 4 * g + i;
                const float sc = isW ? bs[row] * egs[row] : bs[row];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[nt][i] = sc * bf16_bits_to_f32(src[row][cb + 16 * nt + r]);
            }
#pragma unroll
            for (int kb = 0; kb < rb; ++kb) {
                const short4v a = lds_short4(&Lb[16 * rb + r][16 * kb + 4 * g]);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[nt] = mfma16x16x16(a, Xb[kb][nt], acc[nt]);
            }
            const short4v tb = lds_short4(&Ts[rb][r][4 * g]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const f32x4 out = mfma16x16x16(tb, to_bf16x4(acc[nt]), zero4());
                Xb[rb][nt] = to_bf16x4(out);
                if (isW) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Qs[16 * rb + 4 * g + i][cb + 16 * nt + r] = static_cast<u16>(Xb[rb][nt][i]);
                } else {
                    *reinterpret_cast<short4v*>(
                        wsc + kOffUt + (static_cast<size_t>(cb + 16 * nt + r) * C + 16 * rb + 4 * g) * 2) =
                        Xb[rb][nt];
                }
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < C * D / 8; e += kPrepThreads) {
        const int row = e >> 4, c8 = (e & 15) * 8;
        *reinterpret_cast<uint4*>(wsc + kOffW + (static_cast<size_t>(row) * D + c8) * 2) =
            *reinterpret_cast<const uint4*>(&Qs[row][c8]);
    }
}

// ============================================================ scan kernel
// Row permutation shared by the state tiles and the chunk tiles: accumulator
// tile t, lane group gg, register i  <->  index 32(t/2) + 8 gg + 4(t%2) + i.
// Two consecutive tiles therefore hold 8 consecutive indices per lane group,
// which is exactly one K = 32 operand slice of that lane (pack_acc_pair).
__device__ __forceinline__ int perm_row(int t, int rr) {
    return 32 * (t >> 1) + 8 * (rr >> 2) + 4 * (t & 1) + (rr & 3);
}

// One workgroup per (head, 16-wide value tile), four waves with fixed roles:
//   wave 0    - the scan: state in accumulator registers, operands from LDS;
//   waves 1,2 - copy the next chunk's operands global -> LDS with the direct
//               LDS-load instruction (no registers), double-buffered, each
//               1-KiB fragment laid out exactly as the MFMA lanes read it;
//   wave 3    - touches the workspace kPrefetchAhead chunks ahead so that
//               the copies are served from L2.
// Every role runs its own loop with the same number of barriers.
constexpr int kScanThreads = 256;
constexpr int kFragW = 0;     // W        (m, s)    16 fragments
constexpr int kFragQ = 16;    // Q        (m, s)    16
constexpr int kFragA = 32;    // A        lower (m, s2) blocks: 6
constexpr int kFragKt = 38;   // K~^T     (t, s2)   16
constexpr int kFragU = 54;    // Ut^T rows of this value tile (s2): 2
constexpr int kNumFrag = 56;
constexpr int kEgBytes = 272;                       // e^g (64), e^{g_c}, pad: 17 lanes x 16 B
constexpr int kBufBytes = kNumFrag * 1024 + kEgBytes;
constexpr int kZeroOff = 272;                       // 16 zero bytes inside each chunk's e^g area
constexpr int kPrefetchAhead = 6;
constexpr int kWsLines = static_cast<int>((kChunkBytes + 127) / 128);

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 4, 0, 0);
}
__device__ __forceinline__ void wait_vm0() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unconstrained
}

__device__ __forceinline__ int afrag_m(int idx) { return idx < 2 ? idx : 2 + ((idx - 2) >> 1); }
__device__ __forceinline__ int afrag_s(int idx) { return idx < 2 ? 0 : ((idx - 2) & 1); }

__global__ __launch_bounds__(kScanThreads) void gdn_scan_kernel(int BH, int T, int NC, const u16* __restrict__ q,
                                                                const unsigned char* __restrict__ ws,
                                                                const float* S0, float* S_out,
                                                                u16* __restrict__ o) {
    __shared__ __attribute__((aligned(16))) unsigned char sbuf[2][kBufBytes];
    __shared__ __attribute__((aligned(16))) unsigned char scratch[256];

    // blockIdx -> (head, value tile) such that the 8 tiles of a head share an XCD
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int j = blk >> 3;
    const int tile = j & 7;
    const int bh = (j >> 3) * 8 + xcd;
    if (bh >= BH) return;  // uniform over the workgroup
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int g = lane >> 4;
    const size_t qhead = static_cast<size_t>(bh) * T * D;
    const unsigned char* wsh = ws + static_cast<size_t>(bh) * NC * kChunkBytes;

    if (w == 0) {
        // ------------------------------------------------------------ scan
        const int vcol = 16 * tile + r;
        f32x4 P[8];
        {
            const float* srow = S0 ? S0 + (static_cast<size_t>(bh) * D + vcol) * D : nullptr;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int d0 = 32 * s + 8 * g;
                if (srow) {
                    const float4 a = *reinterpret_cast<const float4*>(srow + d0);
                    const float4 b = *reinterpret_cast<const float4*>(srow + d0 + 4);
                    P[2 * s] = f32x4{a.x, a.y, a.z, a.w};
                    P[2 * s + 1] = f32x4{b.x, b.y, b.z, b.w};
                } else {
                    P[2 * s] = zero4();
                    P[2 * s + 1] = zero4();
                }
            }
        }
        __syncthreads();
        for (int n = 0; n < NC; ++n) {
            const unsigned char* B = sbuf[n & 1];
            auto frag = [&](int f) { return *reinterpret_cast<const bf16x8*>(B + f * 1024 + lane * 16); };
            const float* eg = reinterpret_cast<const float*>(B + kNumFrag * 1024);
            const int t0 = n * C;
            const int len = min(C, T - t0);

            bf16x8 Pb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) Pb[s] = pack_acc_pair(P[2 * s], P[2 * s + 1]);
            // X = W P
            f32x4 X[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                X[m] = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) X[m] = mfma16x16x32(frag(kFragW + 4 * m + s), Pb[s], X[m]);
            }
            // U = Ut - X
            f32x4 U[4];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                // decode the 8 bf16 with integer ops (element extraction from
                // __bf16 vectors is avoided throughout)
                const uint4 raw = *reinterpret_cast<const uint4*>(B + (kFragU + s2) * 1024 + lane * 16);
                const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = wds[i >> 1], hi = wds[2 + (i >> 1)];
                    const float u_lo = __uint_as_float((i & 1) ? (lo & 0xffff0000u) : (lo << 16));
                    const float u_hi = __uint_as_float((i & 1) ? (hi & 0xffff0000u) : (hi << 16));
                    U[2 * s2][i] = u_lo - X[2 * s2][i];
                    U[2 * s2 + 1][i] = u_hi - X[2 * s2 + 1][i];
                }
            }
            bf16x8 Ub[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) Ub[s2] = pack_acc_pair(U[2 * s2], U[2 * s2 + 1]);
            // O = e^g (Q P) + A U  (padded Q rows were copied as zeros)
            f32x4 O[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                O[m] = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) O[m] = mfma16x16x32(frag(kFragQ + 4 * m + s), Pb[s], O[m]);
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    O[2 * s2][i] *= eg[32 * s2 + 8 * g + i];
                    O[2 * s2 + 1][i] *= eg[32 * s2 + 8 * g + 4 + i];
                }
            }
#pragma unroll
            for (int idx = 0; idx < 6; ++idx) {
                const int m = afrag_m(idx), s2 = afrag_s(idx);
                O[m] = mfma16x16x32(frag(kFragA + idx), Ub[s2], O[m]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = perm_row(m, 4 * g + i);
                    if (row < len) o[qhead + static_cast<size_t>(t0 + row) * D + vcol] = f32_to_bf16_bits(O[m][i]);
                }
            // P <- e^{g_c} P + K~^T U
            const float egc = eg[C];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                P[t] *= egc;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) P[t] = mfma16x16x32(frag(kFragKt + 2 * t + s2), Ub[s2], P[t]);
            }
            __syncthreads();
        }
        if (S_out) {
            float* srow = S_out + (static_cast<size_t>(bh) * D + vcol) * D;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int d0 = 32 * s + 8 * g;
                *reinterpret_cast<float4*>(srow + d0) =
                    make_float4(P[2 * s][0], P[2 * s][1], P[2 * s][2], P[2 * s][3]);
                *reinterpret_cast<float4*>(srow + d0 + 4) =
                    make_float4(P[2 * s + 1][0], P[2 * s + 1][1], P[2 * s + 1][2], P[2 * s + 1][3]);
            }
        }
    } else if (w <= 2) {
        // --------------------------------------------------- operand copies
        const int half = w - 1;
        auto issue = [&](int n) {
            unsigned char* B = sbuf[n & 1];
            const unsigned char* wsc = wsh + static_cast<size_t>(n) * kChunkBytes;
            const int t0 = n * C;
            const int len = min(C, T - t0);
            for (int f = half; f < kNumFrag; f += 2) {
                const void* src;
                if (f < kFragQ) {
                    const int m = (f - kFragW) >> 2, s = (f - kFragW) & 3;
                    src = wsc + kOffW + (static_cast<size_t>(perm_row(m, r)) * D + 32 * s + 8 * g) * 2;
                } else if (f < kFragA) {
                    const int m = (f - kFragQ) >> 2, s = (f - kFragQ) & 3;
                    const int row = perm_row(m, r);
                    src = row < len ? static_cast<const void*>(q + qhead + static_cast<size_t>(t0 + row) * D + 32 * s + 8 * g)
                                    : static_cast<const void*>(wsc + kOffEg + kZeroOff);
                } else if (f < kFragKt) {
                    const int idx = f - kFragA;
                    src = wsc + kOffA + (static_cast<size_t>(perm_row(afrag_m(idx), r)) * C + 32 * afrag_s(idx) + 8 * g) * 2;
                } else if (f < kFragU) {
                    const int idx = f - kFragKt;
                    src = wsc + kOffKt + (static_cast<size_t>(perm_row(idx >> 1, r)) * C + 32 * (idx & 1) + 8 * g) * 2;
                } else {
                    const int s2 = f - kFragU;
                    src = wsc + kOffUt + (static_cast<size_t>(16 * tile + r) * C + 32 * s2 + 8 * g) * 2;
                }
                dma16(src, B + f * 1024);
            }
            if (half == 0 && lane < kEgBytes / 16) dma16(wsc + kOffEg + lane * 16, B + kNumFrag * 1024);
        };
        issue(0);
        wait_vm0();
        __syncthreads();
        for (int n = 0; n < NC; ++n) {
            if (n + 1 < NC) issue(n + 1);
            wait_vm0();
            __syncthreads();
        }
    } else {
        // -------------------------------------------------- L2 prefetcher
        auto touch = [&](int n) {
            const unsigned char* wsc = wsh + static_cast<size_t>(n) * kChunkBytes;
            for (int l = lane; l < kWsLines; l += 64) dma4(wsc + static_cast<size_t>(l) * 128, scratch);
            const int t0 = n * C;
            const int len = min(C, T - t0);
            if (lane < len) {
                const u16* qrow = q + qhead + static_cast<size_t>(t0 + lane) * D;
                dma4(qrow, scratch);
                dma4(qrow + 64, scratch);
            }
        };
        // This wave shares nothing through LDS (its copies land in a scratch
        // area nobody reads), so it joins the barriers without the release
        // fence of __syncthreads, which would wait for its loads to land.
        for (int n = 1; n <= kPrefetchAhead && n < NC; ++n) touch(n);
        __builtin_amdgcn_s_barrier();
        for (int n = 0; n < NC; ++n) {
            if (n + kPrefetchAhead + 1 < NC) touch(n + kPrefetchAhead + 1);
            __builtin_amdgcn_s_barrier();
        }
        wait_vm0();
    }
}

}  // namespace

bool gdn_mfma_supported(int dtype, int dk, int dv, int chunk) {
    return dtype == kBF16 && dk == D && dv == D && chunk == C;
}

size_t gdn_mfma_workspace_bytes(int B, int H, int T, int, int, int) {
    const size_t nc = (static_cast<size_t>(T) + C - 1) / C;
    return static_cast<size_t>(B) * H * nc * kChunkBytes;
}

hipError_t launch_gdn_mfma_prep(int B, int H, int T, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, void* workspace, hipStream_t stream) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return hipSuccess;
    const int NC = (T + C - 1) / C;
    hipLaunchKernelGGL(gdn_prep_kernel, dim3(static_cast<unsigned>(BH) * NC), dim3(kPrepThreads), 0, stream, T,
                       NC, static_cast<const u16*>(q), static_cast<const u16*>(k), static_cast<const u16*>(v),
                       alpha, beta, static_cast<unsigned char*>(workspace));
    return hipGetLastError();
}

hipError_t launch_gdn_mfma_scan(int B, int H, int T, const void* q, const float* S0, void* o, float* S_out,
                                const void* workspace, hipStream_t stream) {
    const int BH = B * H;
    if (BH <= 0 || T <= 0) return hipSuccess;
    const int NC = (T + C - 1) / C;
    const unsigned scan_blocks = static_cast<unsigned>((BH * 8 + 63) / 64 * 64);
    hipLaunchKernelGGL(gdn_scan_kernel, dim3(scan_blocks), dim3(kScanThreads), 0, stream, BH, T, NC,
                       static_cast<const u16*>(q), static_cast<const unsigned char*>(workspace), S0, S_out,
                       static_cast<u16*>(o));
    return hipGetLastError();
}

hipError_t launch_gdn_mfma(int B, int H, int T, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                           void* workspace, hipStream_t stream) {
    const hipError_t e = launch_gdn_mfma_prep(B, H, T, q, k, v, alpha, beta, workspace, stream);
    if (e != hipSuccess) return e;
    return launch_gdn_mfma_scan(B, H, T, q, S0, o, S_out, workspace, stream);
}

}  // namespace la

// Internal launcher interface between the C ABI (abi.cpp) and the kernel
// translation units.  Not part of the public ABI.  Every launcher enqueues on
// `stream`, relies on abi.cpp's validation of the arguments, and returns the
// hipError_t of the launch; the one check of its own is the size of each grid
// (grid_fits), for which it returns hipErrorInvalidConfiguration before
// launching anything more.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

enum Kind { kNormalized = 0, kGatedDelta = 1, kGated = 2, kKda = 3 };
enum Dtype { kF32 = 0, kBF16 = 1 };
// Block length of every matrix-core chunk kernel (bf16, d_k = d_v = 128).
// They serve any requested chunk length: the chunk form's result does not
// depend on the block length beyond rounding, and smaller blocks would only
// leave the matrix cores idler.
constexpr int kMfmaChunk = 64;
__host__ __device__ inline bool mfma_chunk_ok(int chunk) {
    return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128;
}

// A one-dimensional launch holds fewer than 2^32 work-items: blocks of
// `threads` each, counted in 64 bits (the block counts of very many heads or
// chunks would wrap in 32).
inline bool grid_fits(long long blocks, long long threads) {
    return blocks >= 0 && threads > 0 && blocks <= 0xffffffffLL / threads;
}

// ---- token-by-token recurrence, one block per head (recurrent.hip) --------
// heads = B*H (or N*H for a decode step); T >= 1.  q,k [heads,T,dk];
// v,o [heads,T,dv]; alpha [heads,T] (gated kinds; [heads,T,dk] per channel
// for KDA), beta [heads,T] (gated delta and KDA); S0/S_out
// [heads,dv,dk] (may alias); z0/z_out [heads,dk] (normalized only, may alias).
// Packed batch (cu != nullptr): heads = N*H; head i = n*H + h runs tokens
// cu[n]..cu[n+1] of row block h of [H][Ttot][d] (gates [H][Ttot]) with state
// i, T is ignored, and after every `snap` tokens (0: never) the state goes to
// S_snap[snap_base[n] + j][h] for the first snap_cap slots.  With seq_order,
// block group i takes sequence seq_order[i / H] (longest first).
struct Packed {
    const int* cu = nullptr;
    const int* snap_base = nullptr;
    const int* seq_order = nullptr;
    int H = 0, Ttot = 0, snap = 0, snap_cap = 0;
    float* S_snap = nullptr;
    float* z_snap = nullptr;   // normalised kind: z at the same positions as S_snap
};
hipError_t launch_recurrent(int kind, int dtype, int heads, int T, int dk, int dv,
                            const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta,
                            const float* S0, float* S_out, const float* z0, float* z_out,
                            void* o, hipStream_t stream, const Packed& pk = Packed{});
// The packed-batch table of seg_base / snap_base ([N+1] ints each, at tab and
// tab + N + 1) on the device, from cu (1 workgroup).  With order != nullptr
// (room for cap ints) it also lists the first min(segments, cap) segments,
// numbered as seg_base numbers them, longest first: a workgroup per segment
// taken in that order starts the long chains first.  With seq_order != nullptr
// (room for N ints) it lists the sequences longest first.
hipError_t launch_varlen_table(int N, int Ttot, int segc, int snap, const int* cu, int* tab, hipStream_t stream,
                               int* order = nullptr, int cap = 0, int* seq_order = nullptr);

// ---- normalised linear attention, masked parallel form (la_parallel.hip) -
hipError_t launch_la_parallel(int dtype, int heads, int T, int dk, int dv,
                              const void* q, const void* k, const void* v, void* o,
                              float* S_out, float* z_out, hipStream_t stream);

// ---- chunked forms with fp32 arithmetic on the vector ALUs (chunked_generic.hip)
// One block per head; state and the current chunk live in LDS.
size_t la_chunked_generic_lds_bytes(int dk, int dv, int chunk);
hipError_t launch_la_chunked_generic(int dtype, int heads, int T, int dk, int dv, int chunk,
                                     const void* q, const void* k, const void* v,
                                     const float* S0, const float* z0, void* o,
                                     float* S_out, float* z_out, hipStream_t stream);
size_t gdn_chunked_generic_lds_bytes(int dk, int dv, int chunk);
hipError_t launch_gdn_chunked_generic(int dtype, int heads, int T, int dk, int dv, int chunk,
                                      const void* q, const void* k, const void* v,
                                      const float* alpha, const float* beta,
                                      const float* S0, void* o, float* S_out, hipStream_t stream);

// ---- bf16 matrix-core paths (dk = dv = 128, chunk = 64) -------------------
// Gated delta (gdn_mfma.hip): the sequence of each head is cut into
// segments; prep = the affine map of every segment but the last, scan = the
// entering state of every segment and then outputs.  The workspace holds the
// per-(head, segment) state and map; gdn_mfma_workspace_bytes sizes it.
bool gdn_mfma_supported(int dtype, int dk, int dv, int chunk);
size_t gdn_mfma_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);
hipError_t launch_gdn_mfma(int B, int H, int T, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S0,
                           void* o, float* S_out, void* workspace, hipStream_t stream);
hipError_t launch_gdn_mfma_prep(int B, int H, int T, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, void* workspace,
                                hipStream_t stream);
hipError_t launch_gdn_mfma_scan(int B, int H, int T, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* S0, void* o,
                                float* S_out, void* workspace, hipStream_t stream);

// The library's own workspace for the chunked gated-delta path (one array per
// device, in the code object): its size, and its device address on the
// current device (looked up once per device).
size_t gdn_scratch_bytes();
hipError_t gdn_scratch(void** out);

// Packed batch of N sequences (rows [H][Ttot][d], gates [H][Ttot], states
// [N][H][d][d], sequence n = tokens cu[n]..cu[n+1] on the device), with state
// snapshots after every `snap` tokens (a multiple of the chunk; 0 for none)
// into S_snap [snap_cap][H][d][d].  The workspace (gdn_mfma_varlen_workspace_
// bytes) holds the device-built segment table and the segment maps.
size_t gdn_mfma_varlen_workspace_bytes(int N, int H, int Ttot);
hipError_t launch_gdn_mfma_varlen(int N, int H, int Ttot, const int* cu, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                                  int snap, int snap_cap, float* S_snap, void* workspace, hipStream_t stream);

// Chunked KDA (kda_chunk.hip): a per-chunk tile pass into the workspace, then
// a column-parallel scan.  alpha [B,H,T,128] per channel.
bool kda_mfma_supported(int dtype, int dk, int dv, int chunk);
size_t kda_mfma_workspace_bytes(int B, int H, int T);
size_t kda_mfma_varlen_workspace_bytes(int N, int H, int Ttot);
size_t la_mfma_varlen_workspace_bytes(int N, int H, int Ttot);
hipError_t launch_la_mfma_varlen(bool gated, int N, int H, int Ttot, const int* cu, const void* q, const void* k,
                                 const void* v, const float* alpha, const float* S0, const float* z0, void* o,
                                 float* S_out, float* z_out, int snap, int snap_cap, float* S_snap, float* z_snap,
                                 void* workspace, hipStream_t stream);
hipError_t launch_kda_mfma_varlen(int N, int H, int Ttot, const int* cu, const void* q, const void* k, const void* v,
                                  const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                                  int snap, int snap_cap, float* S_snap, void* workspace, hipStream_t stream);
hipError_t launch_kda_mfma(int B, int H, int T, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, const float* S0, void* o, float* S_out,
                           void* workspace, hipStream_t stream);

// Normalised linear attention, chunked, bf16 in/out (la_mfma.hip).
bool la_mfma_supported(int dtype, int dk, int dv, int chunk);
size_t la_mfma_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);
hipError_t launch_la_mfma(int B, int H, int T, const void* q, const void* k, const void* v,
                          const float* S0, const float* z0, void* o, float* S_out, float* z_out,
                          void* workspace, hipStream_t stream);
// Scalar-gated (unnormalised) linear attention, same kernels and workspace
// as the normalised path (la_mfma_supported / la_mfma_workspace_bytes).
hipError_t launch_gla_mfma(int B, int H, int T, const void* q, const void* k, const void* v, const float* alpha,
                           const float* S0, void* o, float* S_out, void* workspace, hipStream_t stream);

// ---- fused pre-operations of a Gated DeltaNet layer (preops.hip) ---------
// x [B,T,H*(2dk+dv)] token-major (q | k | v channel blocks), w [C,4] fp32,
// a_logit/b_logit [B,T,H] fp32, conv state [B,3,C] (I/O dtype; NULL = zeros,
// st_out NULL = not written, never the same memory as st_in); outputs q,k
// [B,H,T,dk], v [B,H,T,dv], alpha/beta [B,H,T] fp32.  T may be 0.
hipError_t launch_gdn_preprocess(int dtype, int B, int T, int H, int dk, int dv, const void* x, const float* w,
                                 const float* a_logit, const float* b_logit, const void* st_in, void* st_out,
                                 void* q, void* k, void* v, float* alpha, float* beta, hipStream_t stream);
// Packed batch: N sequences on one token axis of T tokens (cu [N+1] on the
// device), states [N,3,C]; outputs [H,T,d] and [H,T].
hipError_t launch_gdn_preprocess_varlen(int dtype, int N, int T, int H, int dk, int dv, const int* cu, const void* x,
                                        const float* w, const float* a_logit, const float* b_logit,
                                        const void* st_in, void* st_out, void* q, void* k, void* v, float* alpha,
                                        float* beta, hipStream_t stream);

}  // namespace la

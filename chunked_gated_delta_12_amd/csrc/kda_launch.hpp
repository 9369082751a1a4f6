// kda_launch.hpp -- internal host-side launchers of the libkda kernels.
// Arguments are validated by the C ABI layer before any of these is called;
// each returns the hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Segmentation of a sequence of `nchunks` 16-token chunks into `nseg`
// contiguous runs of `seg_len` chunks (the last one possibly shorter).
struct SegPlan {
    int nchunks;
    int seg_len;
    int nseg;
};
SegPlan plan_segments(int T, int requested);

// Workspace bytes of a chunked prefill with `nseg` segments of `nchunks` chunks in all.
size_t chunk_workspace_bytes(int B, int H, int dk, int dv, int nseg, int nchunks);

hipError_t launch_gate(int B, int T, int H, int dk, const float* theta, float* g, float* gcum,
                       hipStream_t stream);

// z: pre-activation of the output gate (o's layout and type), or NULL for none.
hipError_t launch_decode(bool f32, int B, int H, int d, const void* q, const void* k,
                         const void* v, const float* theta, const float* beta, float* S,
                         const void* z, void* o, hipStream_t stream);

// Segment map kernel of the chunked prefill: the widened end state [N | M] of
// every segment but the last (N fp32 into ws_n, M in the input type into ws_m,
// both [segment][head][d_k][d]), T' = (I + A)^-1 diag(beta) of every chunk into ws_t.
hipError_t launch_chunk_map(bool f32, int B, int T, int H, int d, const SegPlan& plan, const void* k,
                            const void* v, const float* theta, const float* beta, float* ws_n,
                            void* ws_m, void* ws_t, hipStream_t stream);

// Per-chunk workspace of the bf16 backward pass (one chunk of one sequence), in bf16
// elements: the start state as row-product operand fragments (checkpoint chunks
// only: every CKPT-th chunk of a segment, counted from its first), U by 16-column
// tiles ([d/16][64 lanes (g, li)][tokens 4g .. 4g+3 of column 16 tile + li]),
// T^T [16][16].  The state area of every other chunk holds the previous chunk's
// Kend (operand fragments [d/16][64 lanes] x 8 bytes) and Gamma_C (fp32 per
// channel) instead, at the byte offsets below: the backward sweep rebuilds a
// chunk's start state from the checkpoint before it with those and the U's.
template <int D>
struct BwdChunkWs {
    static constexpr int CKPT = 2;
    static constexpr int64_t WS_S = (int64_t)D * D;
    static constexpr int64_t WS_U = 16 * (int64_t)D;
    static constexpr int64_t WSC = WS_S + WS_U + 256;
    static constexpr uint32_t KE_BYTES = (uint32_t)(D / 16) * 64u * 8u;
    static constexpr uint32_t GC_OFF = KE_BYTES;
};

// The forward chain of the bf16 backward pass on the map kernel's producer and
// consumer wavefronts (d = 64 or 128): from each segment's start state (s_start,
// [segment][batch*head][d][d] fp32, or NULL for zero), it writes every chunk's
// saved operands into the backward workspace's chunk area ws_b
// ([batch*head][chunk] of BwdChunkWs<d>::WSC elements).
hipError_t launch_chunk_save(int B, int T, int H, int d, const SegPlan& plan, const void* k, const void* v,
                             const float* theta, const float* beta, const float* s_start, void* ws_b,
                             hipStream_t stream);

// Gradient segment maps of the bf16 backward pass (d = 64 or 128): for every segment
// but the first, the end value [N | M] of the carried-gradient chain over it from
// [0 | I], in reverse segment order (N fp32, then M bf16 after the nseg N blocks,
// [map][batch*head][d][d]); T' of every chunk from ws_t ([batch*head][chunk][16][16]).
hipError_t launch_grad_map(int B, int T, int H, int d, const SegPlan& plan, const void* q, const void* k,
                           const float* theta, const void* dout, const void* ws_t, float* maps,
                           hipStream_t stream);

// Output pass of a segmented bf16 prefill with producer and consumer
// wavefronts (d = 32, 64 or 128: chunk_out_supported): o from each segment's
// start state in ws_start and each chunk's T' in ws_t, scaled by the output gate
// sigmoid(z) when z is not NULL; S_T (nullable) from the last segment.
bool chunk_out_supported(int d);
hipError_t launch_chunk_out(int B, int T, int H, int d, const SegPlan& plan, const void* q, const void* k,
                            const void* v, const float* theta, const void* ws_t, const float* ws_start,
                            const void* z, void* o, float* S_T, hipStream_t stream);

// z: pre-activation of the output gate (o's layout and type), or NULL for none.
// unbounded: the ablation with the gate -softplus(theta) and position-wise fp32
// diagonal tiles (one segment, z NULL).
hipError_t launch_chunk_fwd(bool f32, int B, int T, int H, int d, const SegPlan& plan,
                            const void* q, const void* k, const void* v, const float* theta,
                            const float* beta, const float* S0, const void* z, void* o, float* S_T,
                            void* workspace, hipStream_t stream, bool unbounded = false);

// Backward pass of the chunked prefill (one workgroup per sequence and head):
// fp32 gradients dq, dk, dv, dtheta, dbeta and dS0 (nullable); the workspace
// holds every chunk's start state (chunk_bwd_workspace_bytes).
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int d);
hipError_t launch_chunk_bwd(bool f32, int B, int T, int H, int d, const void* q, const void* k,
                            const void* v, const float* theta, const float* beta, const float* S0,
                            const void* dout, const float* dS_T, float* dq, float* dk, float* dv,
                            float* dtheta, float* dbeta, float* dS0, void* workspace, hipStream_t stream);

// The same backward pass for bf16 inputs at d = 64 and 128 on the bf16 matrix
// cores (kda_bwd2.hip), with nseg segments of seg_len chunks per sequence; its
// workspace (every chunk's start state, U and T^T in bf16, and the segment maps
// and boundary values) takes chunk_bwd2_workspace_bytes.
size_t chunk_bwd2_workspace_bytes(int B, int T, int H, int d, int nseg);
hipError_t launch_chunk_bwd2(int B, int T, int H, int d, int nseg, int seg_len, const void* q, const void* k,
                             const void* v, const float* theta, const float* beta, const float* S0,
                             const void* dout, const float* dS_T, float* dq, float* dk, float* dv,
                             float* dtheta, float* dbeta, float* dS0, void* workspace, hipStream_t stream);
// Chains affine segment maps X_{s+1} = M_s X_s + N_s of every head on the bf16
// matrix cores (the forward's combine kernel, kda_chunk.hip): N fp32 and M bf16,
// both [segment][batch*head][d][d]; writes X_s for every segment to out (X_0 =
// init, or zero when NULL).  d = 64 or 128.
hipError_t launch_state_combine(int d, int BH, int nseg, const float* init, const float* ws_n, const void* ws_m,
                                float* out, hipStream_t stream);

}  // namespace kda

// kda_gate.hip -- the bounded gate g = -5 * sigmoid(theta) and its 16-token
// chunk-local inclusive prefix sum ("Architecture Deep Dive: Kimi K3...",
// section 3.2, equation 1; "Kimi K3 Deep Dive...", lower-bounded log-decay).
//
// Elementwise and HBM-bound: 4 bytes read and up to 8 bytes written per
// element.  One thread owns one channel of one (batch, chunk, head) and walks
// the chunk's 16 tokens; consecutive threads own consecutive channels, so
// every load and store of a wavefront is a contiguous 256-byte run.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

__global__ void __launch_bounds__(256) gate_kernel(int B, int T, int H, int dk, int nchunks,
                                                   const float* __restrict__ theta,
                                                   float* __restrict__ g, float* __restrict__ gcum) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_b = (int64_t)nchunks * H * dk;
    if (idx >= (int64_t)B * per_b) return;
    const int b = (int)(idx / per_b);
    int64_t rem = idx - (int64_t)b * per_b;
    const int n = (int)(rem / ((int64_t)H * dk));
    rem -= (int64_t)n * H * dk;          // = h * dk + c
    const int t0 = n * CHUNK;
    const int tn = min(CHUNK, T - t0);
    int64_t off = ((int64_t)b * T + t0) * H * dk + rem;
    const int64_t stride = (int64_t)H * dk;
    float run = 0.0f;
    for (int p = 0; p < tn; ++p, off += stride) {
        const float x = gate_logdecay(theta[off]);
        run += x;
        if (g) g[off] = x;
        if (gcum) gcum[off] = run;
    }
}

hipError_t launch_gate(int B, int T, int H, int dk, const float* theta, float* g, float* gcum,
                       hipStream_t stream) {
    const int nchunks = (int)(((int64_t)T + CHUNK - 1) / CHUNK);
    const int64_t n = (int64_t)B * nchunks * H * dk;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, B, T, H, dk,
                       nchunks, theta, g, gcum);
    return hipGetLastError();
}

}  // namespace kda

// kda_decode.hip -- one decode step of the gated delta rule for every
// (batch, head), state updated in place ("Kimi K3" explainer, "Across the
// sequence": a fixed-size recurrent state that each token reads, partly
// forgets and writes).
//
// With alpha = exp(g) per channel and D = Diag(alpha), one step is
//     a = (D S)^T k = S^T (alpha*k),   b = (D S)^T q = S^T (alpha*q)
//     u = beta (v - a),   o = S'^T q = b + (k.q) u,   S' = alpha*S + k u^T
// so the fp32 state is read once and written once: a pure HBM stream of
// 8*dk*dv bytes per head (plus ~1.5 KB of token data).  One workgroup owns
// one head; each thread keeps a [RPT x 4] slab of S in registers between the
// read and the write, and every load/store is a 16-byte vector access with a
// wavefront covering contiguous rows.  A state larger than the last-level cache
// is read and written with the non-temporal (streaming) hint: measured on MI355X
// at 512 MiB - 1 GiB of state, 5-12% faster than plain accesses; a state that fits
// keeps plain accesses, which let it stay in that cache between steps.  With the
// output gate ("Kimi K3"
// explainer, "Across the sequence") o is multiplied by sigmoid(z) in fp32
// before it is rounded.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
struct DecodeCfg {
    static constexpr int NTHR = (D * D / 4) < 256 ? (D * D / 4) : 256;
    static constexpr int CG = D / 4;         // float4 column groups per row
    static constexpr int RG = NTHR / CG;     // row groups
    static constexpr int RPT = D / RG;       // rows per thread
};

// MI355X's last-level cache (Infinity Cache), 256 MiB: states above it stream.
constexpr size_t kLastLevelCacheBytes = (size_t)256 << 20;

template <typename E, int D, bool STREAM>
__global__ void __launch_bounds__(DecodeCfg<D>::NTHR)
decode_kernel(const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
              const float* __restrict__ theta, const float* __restrict__ beta,
              float* __restrict__ S, const E* __restrict__ z, E* __restrict__ o) {
    typedef DecodeCfg<D> C;
    __shared__ alignas(16) float s_alpha[D];
    __shared__ alignas(16) float s_ak[D];
    __shared__ alignas(16) float s_aq[D];
    __shared__ alignas(16) float s_k[D];
    __shared__ alignas(16) float s_kq[D];
    __shared__ alignas(16) float s_pa[C::RG][D];
    __shared__ alignas(16) float s_pb[C::RG][D];
    __shared__ alignas(16) float s_u[D];
    __shared__ float s_dot;

    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % C::CG, rg = tid / C::CG;
    float* Sh = S + bh * D * D;

    // 1. stream this thread's rows of the state into registers
    f32x4 s[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
        const f32x4* p = reinterpret_cast<const f32x4*>(Sh + (rg + C::RG * i) * D + 4 * cg);
        if constexpr (STREAM) s[i] = __builtin_nontemporal_load(p);
        else s[i] = *p;
    }

    // 2. per-channel gate and scaled key/query
    if (tid < D) {
        const float a = __expf(gate_logdecay(theta[bh * D + tid]));
        const float kk = to_f(k[bh * D + tid]);
        const float qq = to_f(q[bh * D + tid]);
        s_alpha[tid] = a;
        s_ak[tid] = a * kk;
        s_aq[tid] = a * qq;
        s_k[tid] = kk;
        s_kq[tid] = kk * qq;
    }
    __syncthreads();

    // 3. k.q on wave 0 (fixed summation order), partial column sums elsewhere
    if (tid < 64) {
        float x = 0.0f;
        for (int c = tid; c < D; c += 64) x += s_kq[c];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
        if (tid == 0) s_dot = x;
    }
    float pa[4] = {0, 0, 0, 0}, pb[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
        const int r = rg + C::RG * i;
        const float ak = s_ak[r], aq = s_aq[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pa[j] += s[i][j] * ak;
            pb[j] += s[i][j] * aq;
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s_pa[rg][4 * cg + j] = pa[j];
        s_pb[rg][4 * cg + j] = pb[j];
    }
    __syncthreads();

    // 4. finish the reductions per column: u and o
    if (tid < D) {
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int r = 0; r < C::RG; ++r) {
            a += s_pa[r][tid];
            b += s_pb[r][tid];
        }
        const float u = beta[bh] * (to_f(v[bh * D + tid]) - a);
        s_u[tid] = u;
        float ov = b + s_dot * u;
        if (z) ov *= out_sigmoid(to_f(z[bh * D + tid]));   // output gate, if given
        o[bh * D + tid] = from_f<E>(ov);
    }
    __syncthreads();

    // 5. S' = alpha*S + k u^T, written back over S
    const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cg]);
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
        const int r = rg + C::RG * i;
        const float a = s_alpha[r], kk = s_k[r];
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = a * s[i][j] + kk * u4[j];
        f32x4* p = reinterpret_cast<f32x4*>(Sh + r * D + 4 * cg);
        if constexpr (STREAM) __builtin_nontemporal_store(w, p);
        else *p = w;
    }
}

template <typename E, int D>
static hipError_t launch_decode_t(int B, int H, const void* q, const void* k, const void* v,
                                  const float* theta, const float* beta, float* S, const void* z,
                                  void* o, hipStream_t stream) {
    const bool stream_state = (size_t)B * H * D * D * sizeof(float) > kLastLevelCacheBytes;
    if (stream_state)
        hipLaunchKernelGGL((decode_kernel<E, D, true>), dim3((unsigned)(B * H)), dim3(DecodeCfg<D>::NTHR), 0,
                           stream, (const E*)q, (const E*)k, (const E*)v, theta, beta, S, (const E*)z,
                           (E*)o);
    else
        hipLaunchKernelGGL((decode_kernel<E, D, false>), dim3((unsigned)(B * H)), dim3(DecodeCfg<D>::NTHR), 0,
                           stream, (const E*)q, (const E*)k, (const E*)v, theta, beta, S, (const E*)z,
                           (E*)o);
    return hipGetLastError();
}

hipError_t launch_decode(bool f32, int B, int H, int d, const void* q, const void* k,
                         const void* v, const float* theta, const float* beta, float* S,
                         const void* z, void* o, hipStream_t stream) {
#define KDA_DEC(E, D) return launch_decode_t<E, D>(B, H, q, k, v, theta, beta, S, z, o, stream)
    if (f32) {
        switch (d) {
            case 16: KDA_DEC(float, 16);
            case 32: KDA_DEC(float, 32);
            case 64: KDA_DEC(float, 64);
            case 128: KDA_DEC(float, 128);
        }
    } else {
        switch (d) {
            case 16: KDA_DEC(bf16, 16);
            case 32: KDA_DEC(bf16, 32);
            case 64: KDA_DEC(bf16, 64);
            case 128: KDA_DEC(bf16, 128);
        }
    }
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda

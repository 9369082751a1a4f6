// kda_chunk.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The sequence is cut into 16-token chunks ("Kimi K3 Deep Dive...", "The
// Problem: The Diagonal-Block Dilemma").  Within a chunk, with start state S,
// G the inclusive chunk-local cumulative log-decay and Gamma = exp(G):
//     K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma, Kend = K*Gamma_C/Gamma
//     A  = StrictLower(diag(beta) K+ K-^T),   T = (I + A)^-1
//     W  = T diag(beta) K+,   Ut = T diag(beta) V,   U = Ut - W S
//     O  = Q+ S + LowerIncl(Q+ K-^T) U,   S' = Diag(Gamma_C) S + Kend^T U.
// Only K- carries an inverse decay, and the bounded gate keeps it below
// exp(16*5) = 5.5e34 ("Architecture Deep Dive: Kimi K3...", section 3.2), so
// the diagonal tiles A and LowerIncl(Q+ K-^T) are plain dense bf16 matrix-core
// products like every other tile -- no position-wise fallback.
//
// A chunk maps the state affinely, S' = M S + N (M = Diag(Gamma_C) - Kend^T W,
// N = Kend^T Ut).  To expose parallelism beyond batch*heads, each sequence is
// cut into segments of whole chunks:
//   map kernel     one workgroup per (segment but the last, head): runs the
//                  chunk scan over its segment with the state widened to
//                  [N | M], started from [0 | I], and stores the result;
//   combine kernel one workgroup per head: start state of every segment,
//                  S_{s+1} = M_s S_s + N_s (sequential over segments);
//   out kernel     one workgroup per (segment, head): the chunk scan from the
//                  segment's true start state, writing o (and S_T for the
//                  last segment).
// With one segment only the out kernel runs, straight from S0.
//
// Workgroup = 4 wavefronts.  Per chunk: the gate and all decay-scaled operand
// tiles are formed once in LDS; A, T, W are shared by the workgroup; the state
// columns are split into 16-column tiles across the wavefronts, each tile
// living in fp32 accumulator registers for the whole segment.  All products
// are 16x16 matrix-core tiles (bf16 operands, fp32 accumulation; fp32
// operands in the validation dtype).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D, bool MAP>
struct ChunkCfg {
    static constexpr int NW = 4;                   // wavefronts per workgroup
    static constexpr int NTHR = 64 * NW;
    static constexpr int NCOL = MAP ? 2 * D : D;   // state columns carried
    static constexpr int NT = NCOL / 16;           // 16-column tiles
    static constexpr int TPW = (NT + NW - 1) / NW; // tiles per wavefront (max)
    static constexpr int KT = D / 16;              // 16-row tiles along d_k
    static constexpr int LDR = D + 8;              // padded row of [16][D] tiles
    static constexpr int LDC = 20;                 // padded row of [D][16] tiles
    static constexpr int PPT = D >= 32 ? D / 32 : 1;  // tokens per thread, gate stage
    static constexpr int NPG = CHUNK / PPT;           // token groups, gate stage
    static constexpr int NACT = (D / 2) * NPG;        // active threads, gate stage
    static_assert(NACT <= NTHR, "gate stage mapping");
};

template <typename E, int D, bool MAP>
struct ChunkSmem {
    typedef ChunkCfg<D, MAP> C;
    alignas(16) E kp_row[16 * C::LDR];             // beta*K+          [token][ch]
    alignas(16) E km_row[16 * C::LDR];             // K-               [token][ch]
    alignas(16) E qp_row[MAP ? 8 : 16 * C::LDR];   // Q+               [token][ch]
    alignas(16) E wn_row[16 * C::LDR];             // -W               [token][ch]
    alignas(16) E kp_col[D * C::LDC];              // (beta*K+)^T      [ch][token]
    alignas(16) E ke_col[D * C::LDC];              // Kend^T           [ch][token]
    alignas(16) E vb_col[D * C::LDC];              // (beta*V)^T       [col][token]
    alignas(16) E t_row[16 * C::LDC];              // T                [token][token]
    alignas(16) E aqk_row[MAP ? 8 : 16 * C::LDC];  // LowerIncl(Q+K-^T)[token][token]
    alignas(16) float akk[16 * 17];                // StrictLower(beta K+ K-^T), fp32
    alignas(16) float gc[D];                       // Gamma_C per channel
    alignas(16) float part[C::NPG * D];            // per-group partial sums of g
};

template <typename E, int D, bool MAP>
__global__ void __launch_bounds__(256)
chunk_kernel(int T, int H, int BH, int nchunks, int seg_len, int nseg,
             const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
             const float* __restrict__ theta, const float* __restrict__ beta,
             const float* S0, const float* __restrict__ ws_start, float* __restrict__ ws_mn,
             E* __restrict__ o, float* S_T) {
    typedef ChunkCfg<D, MAP> C;
    typedef Ops<E> MM;
    typedef typename MM::BFrag BFrag;
    __shared__ ChunkSmem<E, D, MAP> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int nblk_seg = MAP ? nseg - 1 : nseg;
    const int bh = blockIdx.x / nblk_seg, seg = blockIdx.x % nblk_seg;
    const int b = bh / H, h = bh % H;
    const int c0 = seg * seg_len;
    const int c1 = min(nchunks, c0 + seg_len);

    // gate-stage mapping: channel pair cp, token group pgi
    const int cp = tid % (D / 2), pgi = tid / (D / 2);
    const int ch = 2 * cp;
    const bool gact = tid < C::NACT;
    const int64_t tok_stride = (int64_t)H * D;
    const int64_t head_base = (int64_t)b * T * H * D + (int64_t)h * D;

    // ---- state tiles: S[jj][t] = rows 16t.., columns 16*(wave + NW*jj)..
    f32x4 S[C::TPW][C::KT];
    const float* src = nullptr;
    if constexpr (!MAP) src = ws_start ? ws_start + ((int64_t)seg * BH + bh) * D * D
                                       : (S0 ? S0 + (int64_t)bh * D * D : nullptr);
#pragma unroll
    for (int jj = 0; jj < C::TPW; ++jj) {
        const int jt = wave + C::NW * jj;
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * t + 4 * g + i;
                float x = 0.0f;
                if constexpr (MAP) {
                    if (jt >= D / 16 && jt - D / 16 == t && 4 * g + i == r) x = 1.0f;
                } else {
                    if (src && jt < C::NT) x = src[(int64_t)row * D + 16 * jt + r];
                }
                S[jj][t][i] = x;
            }
        }
    }

    // ---- prefetch registers for one chunk (this thread's gate-stage elements)
    f32x2 th_r[C::PPT], k_r[C::PPT], q_r[C::PPT], v_r[C::PPT];
    float b_r[C::PPT];
    auto load_chunk = [&](int n) {
        const int t0 = n * CHUNK;
#pragma unroll
        for (int p = 0; p < C::PPT; ++p) {
            const int t = t0 + pgi * C::PPT + p;
            const bool ok = gact && t < T;
            const int64_t off = head_base + (int64_t)t * tok_stride + ch;
            th_r[p] = ok ? *reinterpret_cast<const f32x2*>(theta + off) : f32x2{0.0f, 0.0f};
            k_r[p] = ok ? load_pair(k + off) : f32x2{0.0f, 0.0f};
            if constexpr (!MAP) q_r[p] = ok ? load_pair(q + off) : f32x2{0.0f, 0.0f};
            v_r[p] = ok ? load_pair(v + off) : f32x2{0.0f, 0.0f};
            b_r[p] = ok ? beta[((int64_t)b * T + t) * H + h] : 0.0f;
        }
    };

    load_chunk(c0);
    for (int n = c0; n < c1; ++n) {
        const int t0 = n * CHUNK;
        // ---------------- stage 1: gate, cumulative decay, scaled operand tiles
        float G0[C::PPT], G1[C::PPT];
        {
            float run0 = 0.0f, run1 = 0.0f;
#pragma unroll
            for (int p = 0; p < C::PPT; ++p) {
                const bool ok = gact && (t0 + pgi * C::PPT + p < T);
                run0 += ok ? gate_logdecay(th_r[p][0]) : 0.0f;   // padding tokens: g = 0
                run1 += ok ? gate_logdecay(th_r[p][1]) : 0.0f;
                G0[p] = run0;
                G1[p] = run1;
            }
            if (gact) {
                sm.part[pgi * D + ch] = run0;
                sm.part[pgi * D + ch + 1] = run1;
            }
        }
        __syncthreads();
        if (gact) {
            float off0 = 0.0f, off1 = 0.0f, tot0 = 0.0f, tot1 = 0.0f;
#pragma unroll
            for (int gi = 0; gi < C::NPG; ++gi) {
                const float x0 = sm.part[gi * D + ch], x1 = sm.part[gi * D + ch + 1];
                if (gi < pgi) { off0 += x0; off1 += x1; }
                tot0 += x0;
                tot1 += x1;
            }
            if (pgi == 0) {
                sm.gc[ch] = __expf(tot0);
                sm.gc[ch + 1] = __expf(tot1);
            }
#pragma unroll
            for (int p = 0; p < C::PPT; ++p) {
                const int pos = pgi * C::PPT + p;
                const float Ga = G0[p] + off0, Gb = G1[p] + off1;
                const float eGa = __expf(Ga), eGb = __expf(Gb);
                const float emGa = __expf(-Ga), emGb = __expf(-Gb);
                const float eEa = __expf(tot0 - Ga), eEb = __expf(tot1 - Gb);
                const float ka = k_r[p][0], kb = k_r[p][1], bt = b_r[p];
                const float kpa = bt * ka * eGa, kpb = bt * kb * eGb;
                store_pair(&sm.kp_row[pos * C::LDR + ch], kpa, kpb);
                sm.kp_col[ch * C::LDC + pos] = from_f<E>(kpa);
                sm.kp_col[(ch + 1) * C::LDC + pos] = from_f<E>(kpb);
                store_pair(&sm.km_row[pos * C::LDR + ch], ka * emGa, kb * emGb);
                if constexpr (!MAP)
                    store_pair(&sm.qp_row[pos * C::LDR + ch], q_r[p][0] * eGa, q_r[p][1] * eGb);
                sm.ke_col[ch * C::LDC + pos] = from_f<E>(ka * eEa);
                sm.ke_col[(ch + 1) * C::LDC + pos] = from_f<E>(kb * eEb);
                sm.vb_col[ch * C::LDC + pos] = from_f<E>(bt * v_r[p][0]);
                sm.vb_col[(ch + 1) * C::LDC + pos] = from_f<E>(bt * v_r[p][1]);
            }
        }
        if (n + 1 < c1) load_chunk(n + 1);   // overlaps the rest of this chunk
        __syncthreads();

        // ---------------- stage 2: diagonal tiles as dense products
        if (wave == 0) {
            const f32x4 a = MM::template mm_ll<D>(sm.kp_row, C::LDR, sm.km_row, C::LDR,
                                                  f32x4{0, 0, 0, 0}, r, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                sm.akk[row * 17 + r] = (r < row) ? a[i] : 0.0f;     // mask by select
            }
        } else if (!MAP && wave == 1) {
            const f32x4 a = MM::template mm_ll<D>(sm.qp_row, C::LDR, sm.km_row, C::LDR,
                                                  f32x4{0, 0, 0, 0}, r, g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                sm.aqk_row[row * C::LDC + r] = from_f<E>((r <= row) ? a[i] : 0.0f);
            }
        }
        __syncthreads();

        // ---------------- stage 3: T = (I + A)^-1 by forward substitution (fp32)
        if (wave == 0 && lane < 16) {
            const int j = lane;   // this lane solves column j
            float tc[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float acc = (rr == j) ? 1.0f : 0.0f;
#pragma unroll
                for (int s = 0; s < rr; ++s) acc -= sm.akk[rr * 17 + s] * tc[s];
                tc[rr] = acc;
                sm.t_row[rr * C::LDC + j] = from_f<E>(acc);
            }
        }
        __syncthreads();

        // ---------------- stage 4: W (shared) and Ut (per column tile)
        for (int tile = wave; tile < C::KT; tile += C::NW) {
            const f32x4 w = MM::template mm_ll<16>(sm.kp_col + tile * 16 * C::LDC, C::LDC, sm.t_row,
                                                   C::LDC, f32x4{0, 0, 0, 0}, r, g);
            // w[i] = W[token r][ch 16*tile + 4g + i]
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.wn_row[r * C::LDR + 16 * tile + 4 * g + i] = from_f<E>(-w[i]);
        }
        f32x4 ut[C::TPW];
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NW * jj;
            ut[jj] = f32x4{0, 0, 0, 0};
            if (jt < D / 16)   // value columns; the M part of a widened state has Ut = 0
                ut[jj] = MM::template mm_ll<16>(sm.t_row, C::LDC, sm.vb_col + jt * 16 * C::LDC, C::LDC,
                                                ut[jj], r, g);
        }
        __syncthreads();

        // ---------------- stage 5: inter-chunk step for this wavefront's column tiles
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NW * jj;
            if (jt >= C::NT) continue;
            BFrag sb[C::KT];
#pragma unroll
            for (int t = 0; t < C::KT; ++t) sb[t] = MM::to_b(S[jj][t]);
            const f32x4 u = MM::template mm_la<D>(sm.wn_row, C::LDR, sb, ut[jj], r, g);  // Ut - W S
            const BFrag ub = MM::to_b(u);
            if constexpr (!MAP) {
                f32x4 oo = MM::template mm_la<D>(sm.qp_row, C::LDR, sb, f32x4{0, 0, 0, 0}, r, g);
                oo = MM::template mm_la<16>(sm.aqk_row, C::LDC, &ub, oo, r, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t0 + 4 * g + i;
                    if (t < T) o[head_base + (int64_t)t * tok_stride + 16 * jt + r] = from_f<E>(oo[i]);
                }
            }
#pragma unroll
            for (int t = 0; t < C::KT; ++t) {
                const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[16 * t + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) S[jj][t][i] *= gcv[i];
                S[jj][t] = MM::template mm_la<16>(sm.ke_col + 16 * t * C::LDC, C::LDC, &ub, S[jj][t], r, g);
            }
        }
        __syncthreads();
    }

    // ---- write the segment's final state
#pragma unroll
    for (int jj = 0; jj < C::TPW; ++jj) {
        const int jt = wave + C::NW * jj;
        if (jt >= C::NT) continue;
#pragma unroll
        for (int t = 0; t < C::KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * t + 4 * g + i;
                if constexpr (MAP) {
                    ws_mn[(((int64_t)seg * BH + bh) * D + row) * (2 * D) + 16 * jt + r] = S[jj][t][i];
                } else {
                    if (S_T && seg == nseg - 1)
                        S_T[((int64_t)bh * D + row) * D + 16 * jt + r] = S[jj][t][i];
                }
            }
    }
}

// Start state of every segment: S_0 = S0 (or 0), S_{s+1} = M_s S_s + N_s, where
// [N_s | M_s] is the widened end state the map kernel stored for segment s.
// One workgroup per head; 16-column tiles of the state across its wavefronts.
template <typename E, int D>
__global__ void __launch_bounds__(256)
combine_kernel(int BH, int nseg, const float* S0, const float* __restrict__ ws_mn,
               float* __restrict__ ws_start) {
    constexpr int NW = 4, NT = D / 16, TPW = (NT + NW - 1) / NW, KT = D / 16;
    typedef Ops<E> MM;
    typedef typename MM::BFrag BFrag;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x;

    f32x4 S[TPW][KT];
#pragma unroll
    for (int jj = 0; jj < TPW; ++jj) {
        const int jt = wave + NW * jj;
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * t + 4 * g + i;
                S[jj][t][i] = (S0 && jt < NT) ? S0[((int64_t)bh * D + row) * D + 16 * jt + r] : 0.0f;
            }
    }
    auto store = [&](int s) {
        float* dst = ws_start + ((int64_t)s * BH + bh) * D * D;
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
            const int jt = wave + NW * jj;
            if (jt >= NT) continue;
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(int64_t)(16 * t + 4 * g + i) * D + 16 * jt + r] = S[jj][t][i];
        }
    };
    store(0);
    for (int s = 0; s + 1 < nseg; ++s) {
        const float* X = ws_mn + ((int64_t)s * BH + bh) * D * (2 * D);   // [D][2D] = [N | M]
#pragma unroll
        for (int jj = 0; jj < TPW; ++jj) {
            const int jt = wave + NW * jj;
            if (jt >= NT) continue;
            BFrag sb[KT];
#pragma unroll
            for (int t = 0; t < KT; ++t) sb[t] = MM::to_b(S[jj][t]);
#pragma unroll
            for (int rt = 0; rt < KT; ++rt) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = X[(int64_t)(16 * rt + 4 * g + i) * (2 * D) + 16 * jt + r];
                S[jj][rt] = MM::template mm_ga<D>(X + (int64_t)16 * rt * (2 * D) + D, 2 * D, sb, acc, r, g);
            }
        }
        store(s + 1);
    }
}

// ----------------------------------------------------------------------------- host side
SegPlan plan_segments(int T, int requested) {
    SegPlan p;
    p.nchunks = (T + CHUNK - 1) / CHUNK;
    int want = requested < 1 ? 1 : requested;
    if (want > p.nchunks) want = p.nchunks;
    p.seg_len = (p.nchunks + want - 1) / want;
    p.nseg = (p.nchunks + p.seg_len - 1) / p.seg_len;
    return p;
}

size_t chunk_workspace_bytes(int B, int H, int dk, int dv, int nseg) {
    if (nseg <= 1) return 0;
    const size_t bh = (size_t)B * H;
    const size_t mn = (size_t)(nseg - 1) * bh * dk * (size_t)(dv + dk);
    const size_t st = (size_t)nseg * bh * dk * dv;
    return (mn + st) * sizeof(float);
}

template <typename E, int D>
static hipError_t launch_chunk_t(int B, int T, int H, const SegPlan& p, const void* q,
                                 const void* k, const void* v, const float* theta,
                                 const float* beta, const float* S0, void* o, float* S_T,
                                 void* workspace, hipStream_t stream) {
    const int BH = B * H;
    float* ws_mn = nullptr;
    float* ws_start = nullptr;
    if (p.nseg > 1) {
        ws_mn = reinterpret_cast<float*>(workspace);
        ws_start = ws_mn + (size_t)(p.nseg - 1) * BH * D * (2 * D);
        hipLaunchKernelGGL((chunk_kernel<E, D, true>), dim3((unsigned)(BH * (p.nseg - 1))), dim3(256), 0,
                           stream, T, H, BH, p.nchunks, p.seg_len, p.nseg, (const E*)q, (const E*)k,
                           (const E*)v, theta, beta, (const float*)nullptr, (const float*)nullptr, ws_mn,
                           (E*)nullptr, (float*)nullptr);
        hipLaunchKernelGGL((combine_kernel<E, D>), dim3((unsigned)BH), dim3(256), 0, stream, BH, p.nseg,
                           S0, (const float*)ws_mn, ws_start);
    }
    hipLaunchKernelGGL((chunk_kernel<E, D, false>), dim3((unsigned)(BH * p.nseg)), dim3(256), 0, stream, T,
                       H, BH, p.nchunks, p.seg_len, p.nseg, (const E*)q, (const E*)k, (const E*)v, theta,
                       beta, S0, (const float*)ws_start, (float*)nullptr, (E*)o, S_T);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(bool f32, int B, int T, int H, int d, const SegPlan& plan,
                            const void* q, const void* k, const void* v, const float* theta,
                            const float* beta, const float* S0, void* o, float* S_T,
                            void* workspace, hipStream_t stream) {
#define KDA_CH(E, D) \
    return launch_chunk_t<E, D>(B, T, H, plan, q, k, v, theta, beta, S0, o, S_T, workspace, stream)
    if (f32) {
        switch (d) {
            case 16: KDA_CH(float, 16);
            case 32: KDA_CH(float, 32);
            case 64: KDA_CH(float, 64);
            case 128: KDA_CH(float, 128);
        }
    } else {
        switch (d) {
            case 16: KDA_CH(bf16, 16);
            case 32: KDA_CH(bf16, 32);
            case 64: KDA_CH(bf16, 64);
            case 128: KDA_CH(bf16, 128);
        }
    }
#undef KDA_CH
    return hipErrorInvalidValue;
}

}  // namespace kda

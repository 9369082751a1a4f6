// kda_bwd.hip -- backward pass of the chunked KDA prefill on gfx950.
//
// Gradients of L = sum_t <do_t, o_t> + <dS_T, S_T> with respect to q, k, v, theta,
// beta and S0, evaluated chunk by chunk.  With the forward quantities of a chunk
// (kda_chunk.hip; "Kimi K3 Deep Dive...", "The Problem: The Diagonal-Block
// Dilemma"; the bounded gate of "Architecture Deep Dive: Kimi K3...", section
// 3.2) -- start state S, K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma, Kend =
// K*Gamma_C/Gamma, A = StrictLower(diag(beta) K+ K-^T), T = (I + A)^-1,
// Y = V - K+ S, U = T diag(beta) Y, A_qk = LowerIncl(Q+ K-^T) -- and the
// gradients dO of the chunk's outputs and dS' of its end state:
//     dU = A_qk^T dO + Kend dS',   Z = T^T dU,   dY = diag(beta) Z,   dV = dY
//     dS = Diag(Gamma_C) dS' + Q+^T dO - K+^T dY          (to the previous chunk)
//     dA_qk = LowerIncl(dO U^T),   dA = StrictLower(-Z U^T)
//     dQ+ = dO S^T + dA_qk K-,     dK+ = -dY S^T + diag(beta) dA K-
//     dK- = dA_qk^T Q+ + (diag(beta) dA)^T K+,   dKend = U dS'^T
//     dbeta = rowsum(dA * K+ K-^T) + rowsum(Z * Y),   dGamma_C = rowsum(dS' * S)
// then the chain through the decay scalings to K, Q and the chunk-local
// cumulative log-decay, whose reverse prefix sum over the chunk gives dg, and
// dtheta = dg * (-5) sigmoid(theta) (1 - sigmoid(theta)).
//
// Two kernels evaluate it.  bwd_kernel (d = 16 and 32) is the plain fp32
// vector-unit form: one workgroup per (batch, head) walks the chunks forward,
// saving every chunk's start state, then backward.  bwd_mfma_kernel (d = 64
// and 128) runs every product on the fp32 matrix cores and, for few long
// sequences, splits them into segments joined by their affine maps
// (bwd_combine_kernel chains them).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

// ---------------------------------------------------------------------------- bwd_kernel
// One workgroup of 256 threads per (batch, head).  The state recurrences act on
// columns separately, so S and dS' live in registers by column (TPC threads
// per column, RPT rows each); products over the state's columns read S rows
// from the workspace and dS' rows from LDS; every row-space gradient element
// has one owning thread, so results are deterministic.
template <int D>
struct BwdCfg {
    static constexpr int NTHR = 256;
    static constexpr int TPC = NTHR / D;     // threads per state column
    static constexpr int RPT = D / TPC;      // state rows per thread
    static constexpr int LDS_ = D + 1;       // row stride of the staged dS'
    // row-space work: thread owns channel i = tid / RT and tokens th*TT .. +TT-1
    static constexpr int RT = NTHR / D;      // threads per channel
    static constexpr int TT = CHUNK / RT;    // tokens per thread
    static_assert(TPC >= 1 && TPC <= 16 && RPT >= 1 && RT * TT == CHUNK, "mappings");
};

template <int D>
struct BwdSmem {
    float gam[CHUNK][D];      // Gamma
    float kp[CHUNK][D];       // K+
    float km[CHUNK][D];       // K-
    float qp[CHUNK][D];       // Q+
    float ke[CHUNK][D];       // Kend
    float dO[CHUNK][D];       // incoming output gradient
    float U[CHUNK][D];
    float Z[CHUNK][D];        // T^T dU
    float dU[CHUNK][D];       // A_qk^T dO + Kend dS'
    float Y[CHUNK][D];        // V - K+ S
    float dS[D * BwdCfg<D>::LDS_];   // dS' of the chunk, row-major
    float KK[CHUNK][CHUNK];   // K+ K-^T
    float A[CHUNK][CHUNK];    // StrictLower(diag(beta) K+ K-^T)
    float Tm[CHUNK][CHUNK + 1];
    float Aqk[CHUNK][CHUNK];
    float dAqk[CHUNK][CHUNK];
    float dA[CHUNK][CHUNK];
    float gc[D], beta[CHUNK];
};

template <typename E, int D>
__global__ void __launch_bounds__(BwdCfg<D>::NTHR)
bwd_kernel(int T, int H, int nchunks, const E* __restrict__ q, const E* __restrict__ k,
           const E* __restrict__ v, const float* __restrict__ theta, const float* __restrict__ beta,
           const float* __restrict__ S0, const E* __restrict__ dout, const float* __restrict__ dS_T,
           float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv,
           float* __restrict__ dtheta, float* __restrict__ dbeta, float* __restrict__ dS0,
           float* __restrict__ ws) {
    typedef BwdCfg<D> C;
    __shared__ BwdSmem<D> sm;
    const int tid = threadIdx.x;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int64_t tstr = (int64_t)H * D;                              // elements between tokens
    const int64_t hb = (int64_t)b * T * H * D + (int64_t)h * D;       // token 0 of this head
    const int64_t bstr = H;                                            // beta: between tokens
    const int64_t bb = (int64_t)b * T * H + h;
    float* Ssave = ws + (int64_t)bh * nchunks * D * D;                 // chunk start states

    // column-space mapping: column j, rows r0 .. r0 + RPT - 1
    const int j = tid / C::TPC, pc = tid % C::TPC, r0 = pc * C::RPT;
    // row-space mapping: channel i, tokens t0 .. t0 + TT - 1
    const int ich = tid / C::RT, t0r = (tid % C::RT) * C::TT;

    constexpr float LOG2E = 1.4426950408889634f;

    float S[C::RPT], dS[C::RPT];
#pragma unroll
    for (int r = 0; r < C::RPT; ++r) {
        S[r] = S0 ? S0[((int64_t)bh * D + r0 + r) * D + j] : 0.0f;
        dS[r] = dS_T ? dS_T[((int64_t)bh * D + r0 + r) * D + j] : 0.0f;
    }

    // sum over the TPC threads of one column (adjacent lanes)
    auto colsum = [&](float x) {
#pragma unroll
        for (int o = 1; o < C::TPC; o <<= 1) x += __shfl_xor(x, o);
        return x;
    };

    // gate, decay tiles and the chunk's small matrices (KK, A, T, A_qk); padding
    // tokens of a partial chunk get g = 0, k = q = v = beta = 0
    auto prepare = [&](int n) {
        const int tc = n * CHUNK;
        const int nv = min(CHUNK, T - tc);
        if (tid < D) {
            const int c = tid;
            float G = 0.0f;
            float gam[CHUNK];
#pragma unroll
            for (int t = 0; t < CHUNK; ++t) {
                float g2 = 0.0f;
                if (t < nv) {
                    const float th = theta[hb + (tc + t) * tstr + c];
                    g2 = G_MIN * LOG2E * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th));
                }
                G += g2;
                gam[t] = __builtin_amdgcn_exp2f(G);
            }
            const float gC = gam[CHUNK - 1];
#pragma unroll
            for (int t = 0; t < CHUNK; ++t) {
                const float kk = t < nv ? to_f(k[hb + (tc + t) * tstr + c]) : 0.0f;
                const float qq = t < nv ? to_f(q[hb + (tc + t) * tstr + c]) : 0.0f;
                const float ig = __builtin_amdgcn_rcpf(gam[t]);   // <= e^80: the bound
                sm.gam[t][c] = gam[t];
                sm.kp[t][c] = kk * gam[t];
                sm.km[t][c] = kk * ig;
                sm.qp[t][c] = qq * gam[t];
                sm.ke[t][c] = kk * (gC * ig);
            }
            sm.gc[c] = gC;
        }
        if (tid < CHUNK) sm.beta[tid] = tid < nv ? beta[bb + (int64_t)(tc + tid) * bstr] : 0.0f;
        __syncthreads();
        if (tid < CHUNK * CHUNK) {   // one (t, s) entry per thread
            const int t = tid / CHUNK, s = tid % CHUNK;
            float kk = 0.0f, qk = 0.0f;
            for (int c = 0; c < D; ++c) {
                kk = fmaf(sm.kp[t][c], sm.km[s][c], kk);
                qk = fmaf(sm.qp[t][c], sm.km[s][c], qk);
            }
            sm.KK[t][s] = kk;
            sm.A[t][s] = s < t ? sm.beta[t] * kk : 0.0f;
            sm.Aqk[t][s] = s <= t ? qk : 0.0f;
        }
        __syncthreads();
        if (tid < CHUNK) {   // T = (I + A)^-1, column tid, forward substitution
            const int cj = tid;
            float x[CHUNK];
#pragma unroll
            for (int r = 0; r < CHUNK; ++r) {
                float a = (r == cj) ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < CHUNK; ++s2)
                    if (s2 < r) a = fmaf(-sm.A[r][s2], x[s2], a);
                x[r] = a;
            }
#pragma unroll
            for (int r = 0; r < CHUNK; ++r) sm.Tm[r][cj] = x[r];
        }
        __syncthreads();
    };

    // Y = V - K+ S and U = T diag(beta) Y for this thread's column, into sm.Y and sm.U
    // (written by the first thread of the column; its partners are in the same wavefront)
    auto forward_cols = [&](int n) {
        const int tc = n * CHUNK;
        const int nv = min(CHUNK, T - tc);
        if (pc == 0) {   // V into Y first: the loads are independent and all in flight at once
#pragma unroll
            for (int t = 0; t < CHUNK; ++t) sm.Y[t][j] = t < nv ? to_f(v[hb + (tc + t) * tstr + j]) : 0.0f;
        }
        for (int t = 0; t < CHUNK; ++t) {
            float a = 0.0f;
#pragma unroll
            for (int r = 0; r < C::RPT; ++r) a = fmaf(sm.kp[t][r0 + r], S[r], a);
            a = colsum(a);
            if (pc == 0) sm.Y[t][j] -= a;
        }
        wave_lds_sync();
        for (int t = 0; t < CHUNK; ++t) {
            float a = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < CHUNK; ++s2) a = fmaf(sm.Tm[t][s2], sm.beta[s2] * sm.Y[s2][j], a);
            if (pc == 0) sm.U[t][j] = a;
        }
        wave_lds_sync();
    };

    // ---------------- forward sweep: save every chunk's start state
    for (int n = 0; n < nchunks; ++n) {
        prepare(n);
#pragma unroll
        for (int r = 0; r < C::RPT; ++r) Ssave[((int64_t)n * D + r0 + r) * D + j] = S[r];
        forward_cols(n);
#pragma unroll
        for (int r = 0; r < C::RPT; ++r) S[r] *= sm.gc[r0 + r];
        for (int t = 0; t < CHUNK; ++t) {
            const float u = sm.U[t][j];
#pragma unroll
            for (int r = 0; r < C::RPT; ++r) S[r] = fmaf(sm.ke[t][r0 + r], u, S[r]);
        }
        __syncthreads();   // before the next chunk's tiles overwrite these
    }

    // ---------------- backward sweep
    for (int n = nchunks - 1; n >= 0; --n) {
        const int tc = n * CHUNK;
        const int nv = min(CHUNK, T - tc);
        prepare(n);
        for (int x = tid; x < CHUNK * D; x += C::NTHR) {
            const int t = x / D, c = x % D;
            sm.dO[t][c] = t < nv ? to_f(dout[hb + (tc + t) * tstr + c]) : 0.0f;
        }
        const float* Sn = Ssave + (int64_t)n * D * D;
#pragma unroll
        for (int r = 0; r < C::RPT; ++r) {
            S[r] = Sn[(r0 + r) * D + j];
            sm.dS[(r0 + r) * C::LDS_ + j] = dS[r];
        }
        __syncthreads();

        forward_cols(n);
        // dU = A_qk^T dO + Kend dS',  Z = T^T dU,  dV = dY = diag(beta) Z
        for (int t = 0; t < CHUNK; ++t) {
            float a = 0.0f;
#pragma unroll
            for (int r = 0; r < C::RPT; ++r) a = fmaf(sm.ke[t][r0 + r], dS[r], a);
            a = colsum(a);
#pragma unroll
            for (int s2 = 0; s2 < CHUNK; ++s2) a = fmaf(sm.Aqk[s2][t], sm.dO[s2][j], a);
            if (pc == 0) sm.dU[t][j] = a;
        }
        wave_lds_sync();
        for (int t = 0; t < CHUNK; ++t) {
            float a = 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < CHUNK; ++s2) a = fmaf(sm.Tm[s2][t], sm.dU[s2][j], a);
            if (pc == 0) {
                sm.Z[t][j] = a;
                if (t < nv) dv[hb + (tc + t) * tstr + j] = sm.beta[t] * a;
            }
        }
        wave_lds_sync();
        // dS <- Diag(Gamma_C) dS' + Q+^T dO - K+^T dY   (dS' itself is staged in LDS)
#pragma unroll
        for (int r = 0; r < C::RPT; ++r) dS[r] *= sm.gc[r0 + r];
        for (int t = 0; t < CHUNK; ++t) {
            const float o = sm.dO[t][j], zy = sm.beta[t] * sm.Z[t][j];
#pragma unroll
            for (int r = 0; r < C::RPT; ++r) dS[r] = fmaf(sm.qp[t][r0 + r], o, fmaf(-sm.kp[t][r0 + r], zy, dS[r]));
        }
        __syncthreads();

        if (tid < CHUNK * CHUNK) {   // dA_qk = LowerIncl(dO U^T), dA = StrictLower(-Z U^T): one entry per thread
            const int t = tid / CHUNK, s = tid % CHUNK;
            float a = 0.0f, z = 0.0f;
            for (int c = 0; c < D; ++c) {
                a = fmaf(sm.dO[t][c], sm.U[s][c], a);
                z = fmaf(sm.Z[t][c], sm.U[s][c], z);
            }
            sm.dAqk[t][s] = s <= t ? a : 0.0f;
            sm.dA[t][s] = s < t ? -z : 0.0f;
        }
        __syncthreads();
        if (tid < CHUNK) {   // dbeta
            const int t = tid;
            float a = 0.0f;
            for (int s2 = 0; s2 < CHUNK; ++s2) a = fmaf(sm.dA[t][s2], sm.KK[t][s2], a);
            for (int c = 0; c < D; ++c) a = fmaf(sm.Z[t][c], sm.Y[t][c], a);
            if (t < nv) dbeta[bb + (int64_t)(tc + t) * bstr] = a;
        }

        {   // row space: channel ich, tokens t0r .. t0r + TT - 1
            const int c = ich;
            const float* Srow = Sn + (int64_t)c * D;
            const float* dSrow = &sm.dS[c * C::LDS_];
            // the products over the state's columns, each S and dS' row element read once
            float dgc = 0.0f;
            float dqp[C::TT], dkp[C::TT], dke[C::TT];
#pragma unroll
            for (int u = 0; u < C::TT; ++u) dqp[u] = dkp[u] = dke[u] = 0.0f;
            // the S row in blocks of 16, each fetched with four 16-byte loads in flight together
            for (int jb = 0; jb < D; jb += 16) {
                f32x4 s4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) s4[e] = *reinterpret_cast<const f32x4*>(Srow + jb + 4 * e);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jj = jb + e;
                    const float sv = s4[e >> 2][e & 3], dsv = dSrow[jj];
                    dgc = fmaf(dsv, sv, dgc);
#pragma unroll
                    for (int u = 0; u < C::TT; ++u) {
                        const int t = t0r + u;
                        dqp[u] = fmaf(sm.dO[t][jj], sv, dqp[u]);
                        dkp[u] = fmaf(-sm.beta[t] * sm.Z[t][jj], sv, dkp[u]);
                        dke[u] = fmaf(sm.U[t][jj], dsv, dke[u]);
                    }
                }
            }
            float dG[C::TT], kesum = 0.0f;
#pragma unroll
            for (int u = 0; u < C::TT; ++u) {
                const int t = t0r + u;
                float dkm = 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < CHUNK; ++s2) {
                    dqp[u] = fmaf(sm.dAqk[t][s2], sm.km[s2][c], dqp[u]);
                    dkp[u] = fmaf(sm.beta[t] * sm.dA[t][s2], sm.km[s2][c], dkp[u]);
                    dkm = fmaf(sm.dAqk[s2][t], sm.qp[s2][c], dkm);
                    dkm = fmaf(sm.beta[s2] * sm.dA[s2][t], sm.kp[s2][c], dkm);
                }
                const float gm = sm.gam[t][c], gC = sm.gc[c];
                const float ig = __builtin_amdgcn_rcpf(gm);
                if (t < nv) {
                    dk[hb + (tc + t) * tstr + c] = dkp[u] * gm + dkm * ig + dke[u] * (gC * ig);
                    dq[hb + (tc + t) * tstr + c] = dqp[u] * gm;
                }
                const float ked = dke[u] * sm.ke[t][c];
                kesum += ked;
                dG[u] = dkp[u] * sm.kp[t][c] - dkm * sm.km[t][c] + dqp[u] * sm.qp[t][c] - ked;
            }
            // the chunk's last row also carries the end decay: d(G_C) = sum_t dKend*Kend + dGamma_C*Gamma_C
            float ktot = kesum;
#pragma unroll
            for (int o = 1; o < C::RT; o <<= 1) ktot += __shfl_xor(ktot, o);
            if (t0r + C::TT == CHUNK) dG[C::TT - 1] += ktot + dgc * sm.gc[c];
            // reverse prefix sum over the chunk's tokens: within the thread, then across
            // the RT threads of the channel (adjacent lanes, later tokens in higher lanes)
            float suf = 0.0f;
#pragma unroll
            for (int u = C::TT - 1; u >= 0; --u) {
                suf += dG[u];
                dG[u] = suf;
            }
            // the totals of the threads of this channel that hold later tokens
            const int rl = tid % C::RT;
            float later = 0.0f;
#pragma unroll
            for (int o = 1; o < C::RT; ++o) {
                const float x = __shfl_down(suf, o);
                if (rl + o < C::RT) later += x;
            }
#pragma unroll
            for (int u = 0; u < C::TT; ++u) {
                const int t = t0r + u;
                if (t < nv) {
                    const float th = theta[hb + (tc + t) * tstr + c];
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th));
                    dtheta[hb + (tc + t) * tstr + c] = (dG[u] + later) * G_MIN * sg * (1.0f - sg);
                }
            }
        }
        __syncthreads();   // before the next chunk overwrites the tiles
    }
    if (dS0) {
#pragma unroll
        for (int r = 0; r < C::RPT; ++r) dS0[((int64_t)bh * D + r0 + r) * D + j] = dS[r];
    }
}

// ----------------------------------------------------------------------------
// Matrix-core version for d = 64 and 128.  Same algebra and the same two sweeps;
// the products run as fp32 16x16x4 matrix-core steps and the state lives in
// the accumulator layout: wavefront w owns the column tiles w*NCW .. w*NCW+NCW-1
// of S (forward sweep) and of dS' (backward sweep), lane (g = lane/16, li =
// lane%16) holding rows 4g..4g+3 of column li of each 16x16 tile.  That layout
// is the B operand of a step that contracts over the tile's rows (step i takes
// row 4g+i), so K+ S, Kend dS', T' Y, T^T dU and the rank-16 state updates
// read the state, U, dU and dY straight from registers.  The forward sweep
// saves every chunk's start state (row-major) and its U and Y tiles; the
// backward sweep reads them back for the products over the state's columns
// (dO S^T, dY S^T, U dS'^T), which run with the tokens as rows and the state's
// rows as columns.  Deterministic: every output element has one owner and a
// fixed summation order.
template <int D>
struct BmCfg {
    static constexpr int NT = D / 16;     // 16-wide tiles along a state dimension
    static constexpr int NW = D == 128 ? 8 : 4;   // wavefronts
    static constexpr int NTHR = 64 * NW;
    static constexpr int NCW = NT / NW;   // column tiles per wavefront
    static constexpr int LDR = D + 4;     // row stride of the [16][D] tiles: rows start 4 banks apart
    static constexpr int LS = CHUNK + 4;  // row stride of the 16x16 matrices
    static constexpr int64_t CW = (int64_t)D * D + 2 * CHUNK * D;   // workspace floats per chunk
    static constexpr int EPT = CHUNK * D / NTHR;  // elements of a [16][D] tile per thread
    static_assert(NCW >= 1 && NT % NW == 0, "d = 64 or 128");
};

// N consecutive elements of E, loaded as one unit (16-byte aligned at most)
template <typename E, int N>
struct alignas(N * sizeof(E) >= 16 ? 16 : N * sizeof(E)) Row {
    E x[N];
};

template <int D>
struct BmSmem {
    typedef BmCfg<D> C;
    float kp[CHUNK][C::LDR];   // K+
    float km[CHUNK][C::LDR];   // K-
    float qp[CHUNK][C::LDR];   // Q+
    float ke[CHUNK][C::LDR];   // Kend
    float gam[CHUNK][C::LDR];  // Gamma
    float dO[CHUNK][C::LDR];
    float U[CHUNK][C::LDR];
    float Z[CHUNK][C::LDR];    // T^T dU
    float Y[CHUNK][C::LDR];    // V - K+ S (backward sweep); V (forward sweep)
    float dsg[CHUNK][C::LDR];  // d g / d theta = G_MIN sigmoid(theta) (1 - sigmoid(theta))
    float X[D][C::LDR];        // dS' of the chunk
    float KK[CHUNK][C::LS];    // K+ K-^T
    float A[CHUNK][C::LS];     // StrictLower(diag(beta) K+ K-^T)
    float Tm[CHUNK][C::LS];    // (I + A)^-1
    float Aqk[CHUNK][C::LS];
    float dAqk[CHUNK][C::LS];
    float dA[CHUNK][C::LS];
    float gpart[4][D];         // the gate's partial sums over each quarter of the chunk
    float zyw[BmCfg<D>::NW][CHUNK];   // rowsum(Z * Y) over each wavefront's columns
    float gc[D], beta[CHUNK];
};

// MODE 0: both sweeps over one segment of chunks, from the state at its start
// (Sinit) and the gradient at its end (Xinit), writing the gradients.
// MODE 1 and 2 are the segment maps: the forward sweep (1) or the chain of
// the carried gradient alone (2) over one segment, run on the widened state
// [0 | I] (d x 2d), whose end value [N | M] gives the segment's affine map
// (end = M start + N for the state; start = M end + N for the gradient).
// They write it, row-major, to maps.  The carried gradient does not depend on
// the state, so both maps are independent of each other.
enum { BWD_FULL = 0, BWD_FMAP = 1, BWD_BMAP = 2 };

template <typename E, int D, int MODE>
__global__ void __launch_bounds__(BmCfg<D>::NTHR)
bwd_mfma_kernel(int T, int H, int BH, int nchunks, int seg_len, const E* __restrict__ q,
                const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ theta,
                const float* __restrict__ beta, const float* __restrict__ Sinit, const E* __restrict__ dout,
                const float* __restrict__ Xinit, float* __restrict__ dq, float* __restrict__ dk,
                float* __restrict__ dv, float* __restrict__ dtheta, float* __restrict__ dbeta,
                float* __restrict__ dS0, float* __restrict__ ws, float* __restrict__ maps) {
    typedef BmCfg<D> C;
    constexpr bool FULL = MODE == BWD_FULL;
    constexpr int NCX = FULL ? C::NCW : 2 * C::NCW;   // column tiles per wavefront (widened in the maps)
    constexpr int WD = FULL ? D : 2 * D;              // columns of the state
    __shared__ BmSmem<D> sm;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, li = lane & 15;
    const int bh = blockIdx.x % BH, seg = blockIdx.x / BH, b = bh / H, h = bh % H;
    const int n_lo = seg * seg_len, n_hi = min(nchunks, n_lo + seg_len);
    const int64_t sb = ((int64_t)seg * BH + bh) * D * D;              // this segment's start / end matrix
    const int64_t tstr = (int64_t)H * D;                              // elements between tokens
    const int64_t hb = (int64_t)b * T * H * D + (int64_t)h * D;       // token 0 of this head
    const int64_t bb = (int64_t)b * T * H + h;                        // beta of token 0
    float* wsh = ws + (int64_t)bh * nchunks * C::CW;
    constexpr float LOG2E = 1.4426950408889634f;
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto ld4 = [](const float* p) { return *reinterpret_cast<const f32x4*>(p); };

    // raw inputs of one chunk, loaded into registers a chunk ahead and written
    // to LDS when that chunk starts: theta, k, q, then v (forward sweep) or
    // dO and the saved U and Y tiles (backward sweep), and beta.  Thread tid
    // holds token xt, channels xc .. xc + EPT - 1; padding tokens read as zero.
    const int xt = tid * C::EPT / D, xc = tid * C::EPT % D;
    struct Raw {
        Row<float, C::EPT> th, u, y;
        Row<E, C::EPT> k, q, x;
        float b;
    };
    auto zero_row = [](auto& r) {
#pragma unroll
        for (int e = 0; e < C::EPT; ++e) r.x[e] = 0.0f;
    };
    auto load_raw = [&](int m, bool bwd, Raw& r) {
        const int tm = m * CHUNK;
        const int nvm = min(CHUNK, T - tm);
        if (xt < nvm) {
            const int64_t off = hb + (tm + xt) * tstr + xc;
            r.th = *reinterpret_cast<const Row<float, C::EPT>*>(theta + off);
            r.k = *reinterpret_cast<const Row<E, C::EPT>*>(k + off);
            r.q = *reinterpret_cast<const Row<E, C::EPT>*>(q + off);
            r.x = *reinterpret_cast<const Row<E, C::EPT>*>((bwd ? dout : v) + off);
        } else {
            zero_row(r.th);
            zero_row(r.k);
            zero_row(r.q);
            zero_row(r.x);
        }
        if (FULL && bwd) {
            const float* wsm = wsh + (int64_t)m * C::CW + (int64_t)D * D + xt * D + xc;
            r.u = *reinterpret_cast<const Row<float, C::EPT>*>(wsm);
            r.y = *reinterpret_cast<const Row<float, C::EPT>*>(wsm + CHUNK * D);
        }
        r.b = (tid < nvm) ? beta[bb + (int64_t)(tm + tid) * H] : 0.0f;
    };
    auto store_raw = [&](const Raw& r, bool bwd) {
#pragma unroll
        for (int e = 0; e < C::EPT; ++e) {
            sm.gam[xt][xc + e] = r.th.x[e];          // theta until the gate overwrites it
            sm.kp[xt][xc + e] = to_f(r.k.x[e]);      // k until the gate overwrites it
            sm.qp[xt][xc + e] = to_f(r.q.x[e]);      // q until the gate overwrites it
            if (bwd) {
                sm.dO[xt][xc + e] = to_f(r.x.x[e]);
                if (FULL) {
                    sm.U[xt][xc + e] = r.u.x[e];
                    sm.Y[xt][xc + e] = r.y.x[e];
                }
            } else {
                sm.Y[xt][xc + e] = to_f(r.x.x[e]);   // V
            }
        }
        if (tid < CHUNK) sm.beta[tid] = r.b;
    };

    // nprod (1 or 2) 16x16 products over the d channels, P0 = A0 Bm^T and P1 = A1 Bm^T
    // (token rows in LDS).  The contraction is split over the wavefronts, the first
    // half (all, for one product) on P0, the second on P1, each over its own channel
    // blocks; the partial tiles meet in scratch ([wavefront][16][16], an LDS array not
    // in use at that point) and finish(p, t, s, value) takes each summed element.
    auto small_products = [&](const float(*A0)[C::LDR], const float(*A1)[C::LDR], const float(*Bm)[C::LDR],
                              float* scratch, int nprod, auto finish) {
        const int wpp = C::NW / nprod, pr = w / wpp, wl = w % wpp, kpw = C::NT / wpp;
        const float(*Am)[C::LDR] = pr == 0 ? A0 : A1;
        f32x4 acc = zero4;
        for (int j = 0; j < kpw; ++j) {
            const int kb = wl * kpw + j;
            const f32x4 a4 = ld4(&Am[li][16 * kb + 4 * g]), b4 = ld4(&Bm[li][16 * kb + 4 * g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma_k4(a4[i], b4[i], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) scratch[w * 256 + (4 * g + r) * 16 + li] = acc[r];
        lds_barrier();
        for (int e = tid; e < nprod * 256; e += C::NTHR) {
            const int p = e >> 8, ts = e & 255;
            float v = 0.0f;
            for (int x = 0; x < wpp; ++x) v += scratch[(p * wpp + x) * 256 + ts];
            finish(p, ts >> 4, ts & 15, v);
        }
    };

    // gate, decay tiles, KK, A, T and (backward sweep) A_qk and dg/dtheta of the
    // chunk whose raw inputs are in LDS
    auto prepare = [&](bool bwd, int nv) {
        static_assert(C::NTHR == 4 * D, "four threads per channel");
        lds_barrier();
        // the gate: four threads per channel c, tokens 4 part .. 4 part + 3 each; the
        // running sum of the log-decay restarts at the chunk and takes the totals of
        // the lower quarters from LDS
        const int c = tid % D, part = tid / D;
        float gl[4], sgv[4], Gl = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 4 * part + u;
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * sm.gam[t][c]));
            sgv[u] = sg;
            if (t < nv) Gl += G_MIN * LOG2E * sg;
            gl[u] = Gl;
        }
        sm.gpart[part][c] = Gl;
        lds_barrier();
        float off = 0.0f, tot = 0.0f;
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
            const float x = sm.gpart[p2][c];
            if (p2 < part) off += x;
            tot += x;
        }
        const float gC = __builtin_amdgcn_exp2f(tot);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 4 * part + u;
            const float gm = __builtin_amdgcn_exp2f(off + gl[u]);
            const float kk = sm.kp[t][c], qq = sm.qp[t][c];
            const float ig = __builtin_amdgcn_rcpf(gm);   // <= e^80: the bound
            sm.gam[t][c] = gm;
            sm.kp[t][c] = kk * gm;
            sm.km[t][c] = kk * ig;
            sm.qp[t][c] = qq * gm;
            sm.ke[t][c] = kk * (gC * ig);
            if (bwd) sm.dsg[t][c] = G_MIN * sgv[u] * (1.0f - sgv[u]);
        }
        if (part == 0) sm.gc[c] = gC;
        lds_barrier();
        // KK = K+ K-^T and (backward sweep) A_qk = Q+ K-^T; Z is not in use yet
        small_products(sm.kp, sm.qp, sm.km, &sm.Z[0][0], bwd ? 2 : 1, [&](int p, int t, int s2, float x) {
            if (p == 0) {
                sm.KK[t][s2] = x;
                sm.A[t][s2] = s2 < t ? sm.beta[t] * x : 0.0f;
            } else {
                sm.Aqk[t][s2] = s2 <= t ? x : 0.0f;
            }
        });
        lds_barrier();
        if (tid < CHUNK) {   // T = (I + A)^-1, column tid, forward substitution
            const int cj = tid;
            float x[CHUNK];
#pragma unroll
            for (int r = 0; r < CHUNK; ++r) {
                float a = (r == cj) ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < CHUNK; ++s2)
                    if (s2 < r) a = fmaf(-sm.A[r][s2], x[s2], a);
                x[r] = a;
            }
#pragma unroll
            for (int r = 0; r < CHUNK; ++r) sm.Tm[r][cj] = x[r];
        }
        lds_barrier();
    };

    // ---------------- forward sweep: S in registers, every chunk's S, U, Y saved
    // the widened state starts as [0 | I]
    auto init_state = [&](f32x4 (&W)[C::NT][NCX], const float* init) {
#pragma unroll
        for (int rt = 0; rt < C::NT; ++rt)
#pragma unroll
            for (int cw = 0; cw < NCX; ++cw)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * rt + 4 * g + r, col = 16 * (w * NCX + cw) + li;
                    if (FULL) W[rt][cw][r] = init ? init[sb + (int64_t)row * D + col] : 0.0f;
                    else W[rt][cw][r] = (col - D == row) ? 1.0f : 0.0f;
                }
    };
    auto store_map = [&](const f32x4 (&W)[C::NT][NCX]) {
        float* mp = maps + ((int64_t)seg * BH + bh) * D * WD;
#pragma unroll
        for (int rt = 0; rt < C::NT; ++rt)
#pragma unroll
            for (int cw = 0; cw < NCX; ++cw)
#pragma unroll
                for (int r = 0; r < 4; ++r) mp[(int64_t)(16 * rt + 4 * g + r) * WD + 16 * (w * NCX + cw) + li] = W[rt][cw][r];
    };
    Raw raw;
    if (MODE != BWD_BMAP) {
    f32x4 St[C::NT][NCX];
    init_state(St, Sinit);
    load_raw(n_lo, false, raw);
    for (int n = n_lo; n < n_hi; ++n) {
        const int nv = min(CHUNK, T - n * CHUNK);
        store_raw(raw, false);
        if (n + 1 < n_hi) load_raw(n + 1, false, raw);   // in flight during this chunk
        prepare(false, nv);
        float* wsn = wsh + (int64_t)n * C::CW;
#pragma unroll
        for (int cw = 0; cw < NCX; ++cw) {
            const int col = 16 * (w * NCX + cw) + li;
            if (FULL) {
#pragma unroll
                for (int rt = 0; rt < C::NT; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) wsn[(16 * rt + 4 * g + r) * D + col] = St[rt][cw][r];
            }
            // P = K+ S: A[t][c] = K+[li][c], B[c][j] = S tile rows
            f32x4 p = zero4;
#pragma unroll
            for (int rt = 0; rt < C::NT; ++rt) {
                const f32x4 a4 = ld4(&sm.kp[li][16 * rt + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) p = mfma_k4(a4[i], St[rt][cw][i], p);
            }
            f32x4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = (col < D ? sm.Y[4 * g + r][col] : 0.0f) - p[r];   // V - K+ S
            // U = T diag(beta) Y: A[t][s] = T[li][s] beta[s], B[s][j] = Y rows
            f32x4 u = zero4;
            const f32x4 t4 = ld4(&sm.Tm[li][4 * g]);
#pragma unroll
            for (int i = 0; i < 4; ++i) u = mfma_k4(t4[i] * sm.beta[4 * g + i], y[i], u);
            if (FULL) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    wsn[(int64_t)D * D + (4 * g + r) * D + col] = u[r];
                    wsn[(int64_t)D * D + CHUNK * D + (4 * g + r) * D + col] = y[r];
                }
            }
            // S <- Diag(Gamma_C) S + Kend^T U: A[c][t] = Kend[t][c], B[t][j] = U rows
#pragma unroll
            for (int rt = 0; rt < C::NT; ++rt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) St[rt][cw][r] *= sm.gc[16 * rt + 4 * g + r];
#pragma unroll
                for (int i = 0; i < 4; ++i) St[rt][cw] = mfma_k4(sm.ke[4 * g + i][16 * rt + li], u[i], St[rt][cw]);
            }
        }
        lds_barrier();   // before the next chunk's tiles overwrite these
    }
    if (MODE == BWD_FMAP) {
        store_map(St);
        return;
    }
    }
    __syncthreads();   // the saved states, U and Y are in memory before the backward sweep reads them

    // ---------------- backward sweep: dS' in registers
    f32x4 Xt[C::NT][NCX];
    init_state(Xt, Xinit);
    load_raw(n_hi - 1, true, raw);
    for (int n = n_hi - 1; n >= n_lo; --n) {
        const int tc = n * CHUNK;
        const int nv = min(CHUNK, T - tc);
        const float* wsn = wsh + (int64_t)n * C::CW;
        store_raw(raw, true);
        if (n > n_lo) load_raw(n - 1, true, raw);   // in flight during this chunk
        if (FULL) {
#pragma unroll
            for (int rt = 0; rt < C::NT; ++rt)
#pragma unroll
                for (int cw = 0; cw < NCX; ++cw)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm.X[16 * rt + 4 * g + r][16 * (w * NCX + cw) + li] = Xt[rt][cw][r];
        }
        prepare(true, nv);

        // column space: dU, Z, dV and the carried gradient, per owned column tile
#pragma unroll
        for (int cw = 0; cw < NCX; ++cw) {
            const int col = 16 * (w * NCX + cw) + li;
            float dob[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) dob[i] = col < D ? sm.dO[4 * g + i][col] : 0.0f;
            // dU = A_qk^T dO + Kend dS'
            f32x4 du = zero4;
#pragma unroll
            for (int i = 0; i < 4; ++i) du = mfma_k4(sm.Aqk[4 * g + i][li], dob[i], du);
#pragma unroll
            for (int rt = 0; rt < C::NT; ++rt) {
                const f32x4 a4 = ld4(&sm.ke[li][16 * rt + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) du = mfma_k4(a4[i], Xt[rt][cw][i], du);
            }
            // Z = T^T dU,  dY = diag(beta) Z = dV
            f32x4 z = zero4;
#pragma unroll
            for (int i = 0; i < 4; ++i) z = mfma_k4(sm.Tm[4 * g + i][li], du[i], z);
            f32x4 dy;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                dy[r] = sm.beta[t] * z[r];
                if (FULL) {
                    sm.Z[t][col] = z[r];
                    if (t < nv) dv[hb + (tc + t) * tstr + col] = dy[r];
                }
            }
            if (FULL) {   // rowsum(Z * Y) over this column tile (NCW = 1): the 16 lanes of a lane group
                static_assert(!FULL || C::NCW == 1, "one column tile per wavefront");
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float zy = z[r] * sm.Y[4 * g + r][col];
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) zy += __shfl_xor(zy, o);
                    if (li == 0) sm.zyw[w][4 * g + r] = zy;
                }
            }
            // dS' <- Diag(Gamma_C) dS' + Q+^T dO - K+^T dY
#pragma unroll
            for (int rt = 0; rt < C::NT; ++rt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Xt[rt][cw][r] *= sm.gc[16 * rt + 4 * g + r];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Xt[rt][cw] = mfma_k4(sm.qp[4 * g + i][16 * rt + li], dob[i], Xt[rt][cw]);
                    Xt[rt][cw] = mfma_k4(-sm.kp[4 * g + i][16 * rt + li], dy[i], Xt[rt][cw]);
                }
            }
        }
        if (!FULL) {
            lds_barrier();   // before the next chunk overwrites the tiles
            continue;
        }
        // the S rows of this lane's channels, in flight across the next barriers
        f32x4 srow[C::NCW][C::NT];
#pragma unroll
        for (int cw = 0; cw < C::NCW; ++cw)
#pragma unroll
            for (int kb = 0; kb < C::NT; ++kb)
                srow[cw][kb] = ld4(wsn + (int64_t)(16 * (w * C::NCW + cw) + li) * D + 16 * kb + 4 * g);
        lds_barrier();   // Z complete

        // dA_qk = LowerIncl(dO U^T), dA = StrictLower(-Z U^T); Y is no longer needed
        small_products(sm.dO, sm.Z, sm.U, &sm.Y[0][0], 2, [&](int p, int t, int s2, float x) {
            if (p == 0) sm.dAqk[t][s2] = s2 <= t ? x : 0.0f;
            else sm.dA[t][s2] = s2 < t ? -x : 0.0f;
        });
        lds_barrier();
        if (tid < CHUNK) {   // dbeta = rowsum(dA * K+ K-^T) + rowsum(Z * Y)
            const int t = tid;
            float a = 0.0f;
#pragma unroll
            for (int x = 0; x < C::NW; ++x) a += sm.zyw[x][t];
#pragma unroll
            for (int s2 = 0; s2 < CHUNK; ++s2) a = fmaf(sm.dA[t][s2], sm.KK[t][s2], a);
            if (t < nv) dbeta[bb + (int64_t)(tc + t) * H] = a;
        }

        // row space: channel tiles owned like the column tiles; rows are tokens,
        // step i contracts state column 16kb + 4g + i (S and dS' rows as B operands)
#pragma unroll
        for (int cw = 0; cw < C::NCW; ++cw) {
            const int cc = 16 * (w * C::NCW + cw) + li;   // this lane's channel
            f32x4 aq = zero4, ak = zero4, ae = zero4, am = zero4;   // dQ+, dK+, dKend, dK-
            float dgc = 0.0f;
            const float nbl = -sm.beta[li];
#pragma unroll
            for (int kb = 0; kb < C::NT; ++kb) {
                const f32x4 s4 = srow[cw][kb];
                const f32x4 x4 = ld4(&sm.X[cc][16 * kb + 4 * g]);
                const f32x4 o4 = ld4(&sm.dO[li][16 * kb + 4 * g]);
                const f32x4 z4 = ld4(&sm.Z[li][16 * kb + 4 * g]);
                const f32x4 u4 = ld4(&sm.U[li][16 * kb + 4 * g]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    aq = mfma_k4(o4[i], s4[i], aq);
                    ak = mfma_k4(nbl * z4[i], s4[i], ak);
                    ae = mfma_k4(u4[i], x4[i], ae);
                    dgc = fmaf(x4[i], s4[i], dgc);
                }
            }
            // + dA_qk K-, + diag(beta) dA K-;  dK- = dA_qk^T Q+ + (diag(beta) dA)^T K+
            const f32x4 daq4 = ld4(&sm.dAqk[li][4 * g]), da4 = ld4(&sm.dA[li][4 * g]);
            const float bl = sm.beta[li];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 4 * g + i;
                const float kmv = sm.km[s][cc];
                aq = mfma_k4(daq4[i], kmv, aq);
                ak = mfma_k4(bl * da4[i], kmv, ak);
                am = mfma_k4(sm.dAqk[s][li], sm.qp[s][cc], am);
                am = mfma_k4(sm.beta[s] * sm.dA[s][li], sm.kp[s][cc], am);
            }
            dgc += __shfl_xor(dgc, 16);
            dgc += __shfl_xor(dgc, 32);
            // chain through the decay scalings; lane holds tokens 4g..4g+3 of channel cc
            const float gC = sm.gc[cc];
            float dG[4], kesum = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                const float gm = sm.gam[t][cc], ig = __builtin_amdgcn_rcpf(gm);
                if (t < nv) {
                    dk[hb + (tc + t) * tstr + cc] = ak[r] * gm + am[r] * ig + ae[r] * (gC * ig);
                    dq[hb + (tc + t) * tstr + cc] = aq[r] * gm;
                }
                const float ked = ae[r] * sm.ke[t][cc];
                kesum += ked;
                dG[r] = ak[r] * sm.kp[t][cc] - am[r] * sm.km[t][cc] + aq[r] * sm.qp[t][cc] - ked;
            }
            kesum += __shfl_xor(kesum, 16);
            kesum += __shfl_xor(kesum, 32);
            // the chunk's last token also carries the end decay: d(G_C) = sum_t dKend*Kend + dGamma_C*Gamma_C
            if (g == 3) dG[3] += kesum + dgc * gC;
            // reverse prefix sum over the chunk's tokens: within the lane, then the
            // totals of the lane groups holding later tokens
            float suf = 0.0f;
#pragma unroll
            for (int r = 3; r >= 0; --r) {
                suf += dG[r];
                dG[r] = suf;
            }
            float later = 0.0f;
#pragma unroll
            for (int o = 1; o < 4; ++o) {
                const float x = __shfl_down(suf, 16 * o);
                if (g + o < 4) later += x;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                if (t < nv) dtheta[hb + (tc + t) * tstr + cc] = (dG[r] + later) * sm.dsg[t][cc];
            }
        }
        lds_barrier();   // before the next chunk overwrites the tiles
    }
    if (!FULL) {
        store_map(Xt);
    } else if (dS0 && seg == 0) {
#pragma unroll
        for (int rt = 0; rt < C::NT; ++rt)
#pragma unroll
            for (int cw = 0; cw < NCX; ++cw)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dS0[((int64_t)bh * D + 16 * rt + 4 * g + r) * D + 16 * (w * NCX + cw) + li] = Xt[rt][cw][r];
    }
}

// Chains the segment maps of one head along its segments, 16 state columns per
// workgroup (the maps act on columns separately).  With [N_s | M_s] the map of
// segment s: forward, Y_0 = init and Y_{s+1} = M_s Y_s + N_s (the state at
// each segment's start); reverse, Y_{nseg-1} = init and Y_{s-1} = M_s Y_s + N_s
// (the carried gradient at each segment's end).  Writes every Y_s to out.
template <int D>
__global__ void __launch_bounds__(256)
bwd_combine_kernel(int BH, int nseg, int reverse, const float* __restrict__ maps,
                   const float* __restrict__ init, float* __restrict__ out) {
    constexpr int NT = D / 16, R = D / 16;   // column tiles; rows per thread
    __shared__ float Ys[D][17];
    const int bh = blockIdx.x / NT, ct = blockIdx.x % NT;
    const int tid = threadIdx.x, cl = tid & 15, r0 = (tid >> 4) * R;
    const int col = 16 * ct + cl;
    float y[R];
#pragma unroll
    for (int r = 0; r < R; ++r) y[r] = init ? init[((int64_t)bh * D + r0 + r) * D + col] : 0.0f;
    int s = reverse ? nseg - 1 : 0;
    for (int step = 0;; ++step) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            Ys[r0 + r][cl] = y[r];
            out[(((int64_t)s * BH + bh) * D + r0 + r) * D + col] = y[r];
        }
        if (step == nseg - 1) break;
        __syncthreads();
        const float* mp = maps + ((int64_t)s * BH + bh) * D * 2 * D;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = mp[(int64_t)(r0 + r) * 2 * D + col];   // N_s
        for (int kk = 0; kk < D; kk += 4) {
            float yk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) yk[e] = Ys[kk + e][cl];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const f32x4 m4 = *reinterpret_cast<const f32x4*>(mp + (int64_t)(r0 + r) * 2 * D + D + kk);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[r] = fmaf(m4[e], yk[e], acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) y[r] = acc[r];
        s += reverse ? -1 : 1;
        __syncthreads();
    }
}

// Segments of the matrix-core backward: one per workgroup slot the heads leave
// free, at least 16 chunks each, used only when they give four or more
// workgroups per head (the maps cost about as much again as the pass itself).
static int bwd_segments(int BH, int nchunks, int d, int* seg_len) {
    *seg_len = nchunks;
    if ((d != 64 && d != 128) || BH > 64 || nchunks < 64) return 1;
    const int want = (256 + BH - 1) / BH;
    int L = (nchunks + want - 1) / want;
    if (L < 16) L = 16;
    *seg_len = L;
    return (nchunks + L - 1) / L;
}

// The size serves both input types: the fp32 kernels' layout (fp32 chunk states,
// U and Y) and, for d = 64 and 128, the bf16 kernel's (kda_bwd2.hip).
size_t chunk_bwd_workspace_bytes(int B, int T, int H, int d) {
    const size_t nchunks = ((size_t)T + CHUNK - 1) / CHUNK;
    const size_t BH = (size_t)B * H;
    // every chunk's start state; the matrix-core kernel also keeps its U and Y tiles
    size_t n = nchunks * BH * ((size_t)d * d + 2 * CHUNK * (size_t)d);
    int L;
    const size_t nseg = bwd_segments((int)BH, (int)nchunks, d, &L);
    // segmented: both maps of every segment (d x 2d), the states at the segments'
    // starts and the carried gradients at their ends (d x d)
    if (nseg > 1) n += nseg * BH * (4 * (size_t)d * d + 2 * (size_t)d * d);
    size_t bytes = n * sizeof(float);
    if (d == 64 || d == 128) {
        const size_t b2 = chunk_bwd2_workspace_bytes(B, T, H, d, (int)nseg);
        if (b2 > bytes) bytes = b2;
    }
    return bytes;
}

hipError_t launch_chunk_bwd(bool f32, int B, int T, int H, int d, const void* q, const void* k,
                            const void* v, const float* theta, const float* beta, const float* S0,
                            const void* dout, const float* dS_T, float* dq, float* dk, float* dv,
                            float* dtheta, float* dbeta, float* dS0, void* workspace, hipStream_t stream) {
    const int nchunks = (int)(((int64_t)T + CHUNK - 1) / CHUNK);
    const int BH = B * H;
    int L;
    const int nseg = bwd_segments(BH, nchunks, d, &L);
    if (!f32 && (d == 64 || d == 128))   // bf16 inputs: the bf16 matrix-core kernel
        return launch_chunk_bwd2(B, T, H, d, nseg, L, q, k, v, theta, beta, S0, dout, dS_T, dq, dk, dv, dtheta,
                                 dbeta, dS0, workspace, stream);
    float* wsf = (float*)workspace;
    const size_t DD = (size_t)d * d;
    float* mapF = wsf + (size_t)nchunks * BH * (DD + 2 * CHUNK * (size_t)d);
    float* mapB = mapF + (size_t)nseg * BH * 2 * DD;
    float* Sst = mapB + (size_t)nseg * BH * 2 * DD;
    float* Xen = Sst + (size_t)nseg * BH * DD;
#define KDA_BWD_MODE(E, D, MODE, GRID, SI, XI, MP)                                                        \
    hipLaunchKernelGGL((bwd_mfma_kernel<E, D, MODE>), dim3((unsigned)(GRID)), dim3(BmCfg<D>::NTHR), 0, stream, \
                       T, H, BH, nchunks, L, (const E*)q, (const E*)k, (const E*)v, theta, beta, SI,          \
                       (const E*)dout, XI, dq, dk, dv, dtheta, dbeta, dS0, wsf, MP)
#define KDA_BWD_MFMA(E, D)                                                                              \
    if (nseg == 1) {                                                                                    \
        KDA_BWD_MODE(E, D, BWD_FULL, BH, S0, dS_T, nullptr);                                            \
    } else {                                                                                            \
        KDA_BWD_MODE(E, D, BWD_FMAP, nseg * BH, nullptr, nullptr, mapF);                                \
        KDA_BWD_MODE(E, D, BWD_BMAP, nseg * BH, nullptr, nullptr, mapB);                                \
        hipLaunchKernelGGL((bwd_combine_kernel<D>), dim3((unsigned)(BH * (D / 16))), dim3(256), 0, stream, \
                           BH, nseg, 0, (const float*)mapF, S0, Sst);                                   \
        hipLaunchKernelGGL((bwd_combine_kernel<D>), dim3((unsigned)(BH * (D / 16))), dim3(256), 0, stream, \
                           BH, nseg, 1, (const float*)mapB, dS_T, Xen);                                 \
        KDA_BWD_MODE(E, D, BWD_FULL, nseg * BH, (const float*)Sst, (const float*)Xen, nullptr);         \
    }                                                                                                   \
    return hipGetLastError()
#define KDA_BWD(E, D)                                                                                  \
    hipLaunchKernelGGL((bwd_kernel<E, D>), dim3((unsigned)BH), dim3(BwdCfg<D>::NTHR), 0, stream, T, H,  \
                       nchunks,                                                                         \
                       (const E*)q, (const E*)k, (const E*)v, theta, beta, S0, (const E*)dout, dS_T, dq, \
                       dk, dv, dtheta, dbeta, dS0, (float*)workspace);                                  \
    return hipGetLastError()
    if (f32) {
        switch (d) {
            case 16: KDA_BWD(float, 16);
            case 32: KDA_BWD(float, 32);
            case 64: KDA_BWD_MFMA(float, 64);
            case 128: KDA_BWD_MFMA(float, 128);
        }
    } else {
        switch (d) {
            case 16: KDA_BWD(bf16, 16);
            case 32: KDA_BWD(bf16, 32);
            case 64: KDA_BWD_MFMA(bf16, 64);
            case 128: KDA_BWD_MFMA(bf16, 128);
        }
    }
#undef KDA_BWD
#undef KDA_BWD_MFMA
#undef KDA_BWD_MODE
    return hipErrorInvalidValue;
}

}  // namespace kda

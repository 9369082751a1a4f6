// kda_chunk.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The sequence is cut into 16-token chunks ("Kimi K3 Deep Dive...", "The
// Problem: The Diagonal-Block Dilemma").  Within a chunk, with start state S,
// G the inclusive chunk-local cumulative log-decay and Gamma = exp(G):
//     K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma, Kend = K*Gamma_C/Gamma
//     A  = StrictLower(diag(beta) K+ K-^T),   T = (I + A)^-1
//     W  = T diag(beta) K+,   Ut = T diag(beta) V,   U = Ut - W S
//     O  = Q+ S + LowerIncl(Q+ K-^T) U,   S' = Diag(Gamma_C) S + Kend^T U.
// The kernels evaluate U as T (beta*V - beta*K+ S): the products with the
// state then do not wait for T, and W is never formed.
// Only K- carries an inverse decay, and the bounded gate keeps it below
// exp(16*5) = 5.5e34 ("Architecture Deep Dive: Kimi K3...", section 3.2), so
// the diagonal tiles A and LowerIncl(Q+ K-^T) are plain dense bf16 matrix-core
// products like every other tile -- no position-wise fallback.
//
// A chunk maps the state affinely, S' = M S + N (M = Diag(Gamma_C) - Kend^T W,
// N = Kend^T Ut).  To expose parallelism beyond batch*heads, each sequence is
// cut into segments of whole chunks:
//   map kernel     (kda_map.hip) one workgroup per (segment, head): runs the
//                  chunk scan over its segment with the state widened to
//                  [N | M], started from [0 | I], stores the result and
//                  publishes every chunk's T' = T diag(beta);
//   combine kernel start state of every segment, S_{s+1} = M_s S_s + N_s
//                  (sequential over segments);
//   out kernel     one workgroup per (segment, head): the chunk scan from the
//                  segment's true start state, writing o (and S_T for the
//                  last segment).
// With one segment only the out kernel runs, straight from S0, and solves for
// T itself.
//
// The out kernel runs workgroups of 4 wavefronts, two per compute unit.  Per
// chunk: the gate and all decay-scaled operand tiles are formed once in LDS;
// A and T are shared by the workgroup; the state columns are split into
// 16-column tiles across the wavefronts, each tile living in fp32 accumulator
// registers for the whole segment.  The next chunk's inputs are loaded while the current one is being
// processed, and each chunk's o tile is written out during the next chunk.  All products
// are 16x16 matrix-core tiles (bf16 operands, fp32 accumulation; fp32
// operands in the validation dtype).
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D, int NW_>
struct ChunkCfg {
    static constexpr int NW = NW_;                 // wavefronts per workgroup
    static constexpr int NTHR = 64 * NW;
    static constexpr int NCOL = D;                 // state columns carried
    static constexpr int NT = NCOL / 16;           // 16-column tiles
    static constexpr int TPW = (NT + NW - 1) / NW; // tiles per wavefront (max)
    static constexpr int KT = D / 16;              // 16-row tiles along d_k
    static constexpr int LDR = D + 8;              // padded row of [16][D] tiles
    static constexpr int LDC = 20;                 // padded row of [D][16] tiles
    // Gate stage: a thread owns one channel pair and PPT consecutive tokens; the
    // NPG token groups of a pair sit in the same wavefront (PW pairs per
    // wavefront), so the prefix over the chunk runs on cross-lane shuffles.
    static constexpr int PPT = D / (8 * NW) > 1 ? D / (8 * NW) : 1;  // tokens per thread
    static constexpr int NPG = CHUNK / PPT;           // token groups per pair
    static constexpr int PW = 64 / NPG;               // channel pairs per wavefront
    static constexpr int NACT = (D / 2) * NPG;        // active threads
    static_assert(NACT <= NTHR, "gate stage mapping");
    static_assert(NPG <= 64 && 64 % NPG == 0, "gate stage mapping");
    static_assert(PPT == 1 || PPT == 2 || PPT == 4, "gate stage column writes");
};

// UNB: the ablation with the unbounded gate, which also keeps the raw q tile and
// the in-chunk cumulative log-decay (base 2) for the position-wise diagonal tiles.
template <typename E, int D, int NW, bool UNB = false>
struct ChunkSmem {
    typedef ChunkCfg<D, NW> C;
    static constexpr int LDP = Ops<E>::PAD_ROW;    // padded K = 16 operand rows
    // operand rows [16][D]: bf16 D + 4 elements (a stride of 2 (mod 4) dwords keeps
    // the pairs of 8-byte operand reads free of bank conflicts); o_tile keeps
    // C::LDR, whose rows are 16-byte aligned for the o stores
    static constexpr int LDQ = sizeof(E) == 2 ? D + 4 : D + 8;
    alignas(16) E kn_row[16 * LDQ];                // -K+ = -K*Gamma           [token][ch]
    alignas(16) E km_row[16 * LDQ];                // K- = K/Gamma (UNB: raw K) [token][ch]
    alignas(16) E qp_row[16 * LDQ];                // Q+ = Q*Gamma             [token][ch]
    alignas(16) E o_tile[16 * C::LDR];             // o of the chunk           [token][col]
    alignas(16) E ke_pad[D * LDP];                 // Kend^T, padded           [ch][token]
    alignas(16) E v_col[D * C::LDC];               // V^T                      [col][token]
    alignas(16) E t_pad[16 * LDP];                 // T = (I + A)^-1, padded   [token][token]
    alignas(16) E aqk_pad[16 * LDP];               // LowerIncl(Q+K-^T), padded [token][token]
    alignas(16) float akk_t[16 * 20];              // StrictLower(beta K+ K-^T)^T, fp32
    alignas(16) float gc[D];                       // Gamma_C per channel
    alignas(16) E q_row[UNB ? 16 * LDQ : 8];       // UNB: raw Q               [token][ch]
    alignas(16) float g_row[UNB ? 16 * (D + 4) : 4];   // UNB: G2 = log2 Gamma  [token][ch]
};

// Store units of the o tile: SU bytes per thread and store (4, 8 or 16).
template <int SU> struct StoreUnit;
template <> struct StoreUnit<4> { typedef uint32_t T; };
template <> struct StoreUnit<8> { typedef uint64_t T; };
template <> struct StoreUnit<16> { typedef f32x4 T; };

// One store unit by buffer load (zero outside the resource).
template <int SU> __device__ __forceinline__ typename StoreUnit<SU>::T ld_unit(Rsrc r, uint32_t voff);
template <> __device__ __forceinline__ uint32_t ld_unit<4>(Rsrc r, uint32_t voff) {
    return buf_ld32(r, voff, 0u);
}
template <> __device__ __forceinline__ uint64_t ld_unit<8>(Rsrc r, uint32_t voff) {
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0));
}
template <> __device__ __forceinline__ f32x4 ld_unit<16>(Rsrc r, uint32_t voff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// The output gate on one store unit of o: every element times sigmoid of the
// matching element of z, in fp32, rounded once to the storage type.
template <typename E, typename U>
__device__ __forceinline__ U gate_unit(U ou, U zu) {
    constexpr int N = (int)(sizeof(U) / sizeof(E));
    typedef E V __attribute__((__vector_size__(sizeof(U))));
    const V ov = __builtin_bit_cast(V, ou), zv = __builtin_bit_cast(V, zu);
    V r;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const E oe = ov[i], ze = zv[i];
        r[i] = from_f<E>(to_f(oe) * out_sigmoid(to_f(ze)));
    }
    return __builtin_bit_cast(U, r);
}

// N consecutive values as one store of the storage type.
template <typename E, int N>
__device__ __forceinline__ void store_run(E* p, const float* x) {
    typedef E V __attribute__((__vector_size__(N * sizeof(E))));
    V v;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = from_f<E>(x[i]);
    *reinterpret_cast<V*>(p) = v;
}

// Four values of an accumulator tile as one store of the storage type.
template <typename E>
__device__ __forceinline__ void store4(E* p, f32x4 x) {
    typedef E V __attribute__((__vector_size__(4 * sizeof(E))));
    V v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = from_f<E>(x[i]);
    *reinterpret_cast<V*>(p) = v;
}

// Scatter PPT loaded pairs (channel c, c+1 of consecutive tokens) into two
// token runs, one per channel, without a round trip through fp32.
template <typename E, int N>
__device__ __forceinline__ void store_pair_runs(E* pa, E* pb, const typename Pair<E>::T* x) {
    typedef E V __attribute__((__vector_size__(N * sizeof(E))));
    V a, b;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        a[i] = x[i][0];
        b[i] = x[i][1];
    }
    *reinterpret_cast<V*>(pa) = a;
    *reinterpret_cast<V*>(pb) = b;
}

// TWS: several segments; the kernel reads each chunk's T' = T diag(beta) from
// ws_t (published by the map kernel) instead of forming A and solving for T.
// GATE: o is scaled by the output gate sigmoid(z) ("Kimi K3" explainer,
// "Across the sequence"); z has o's layout.
// UNB: the ablation of the bound -- the conventional unbounded log-decay
// g = -softplus(theta) ("Kimi K3 Deep Dive...", "The Design: Putting a Lower
// Bound on Log-Decay").  K- = K/Gamma is then unbounded and may overflow, so
// the two diagonal tiles are formed position by position in fp32 from the raw
// K, Q and the cumulative log-decay ("Architecture Deep Dive: Kimi K3...",
// section 3.1): A[t][s] = sum_c x_t[c] k_s[c] 2^(G2_t[c] - G2_s[c]), s <= t, whose
// exponents are never positive.  Every other factor stays <= 1.
template <typename E, int D, int NW, bool TWS, bool GATE, bool UNB = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(8 / NW)))
chunk_kernel(int T, int H, int BH, int nchunks, int seg_len, int nseg,
             const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
             const float* __restrict__ theta, const float* __restrict__ beta,
             const float* S0, const float* __restrict__ ws_start,
             const E* ws_t, const E* __restrict__ z, E* __restrict__ o, float* S_T) {
    typedef ChunkCfg<D, NW> C;
    typedef ChunkSmem<E, D, NW, UNB> SM;
    typedef Ops<E> MM;
    static_assert(!UNB || (!TWS && !GATE && C::NTHR == 256), "the ablation runs one segment, one thread per tile entry");
    typedef typename MM::BFrag BFrag;
    typedef typename MM::PFrag PFrag;
    constexpr int LDP = SM::LDP;
    __shared__ SM sm;

    // wave index as a scalar, so that branches on it stay scalar branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int b = bh / H, h = bh % H;
    const int c0 = seg * seg_len;
    const int c1 = min(nchunks, c0 + seg_len);
    const int c_full = min(c1, T / CHUNK);         // chunks [c0, c_full) hold 16 tokens

    // gate-stage mapping: channel pair cp, token group pgi (tokens pgi*PPT ..)
    const int cp = wave * C::PW + lane % C::PW, pgi = lane / C::PW;
    const int ch = 2 * cp;
    constexpr bool ALL_ACT = C::NACT == C::NTHR;
    const bool gact = ALL_ACT || cp < D / 2;
    const int64_t tok_stride = (int64_t)H * D;
    const int64_t head_base = (int64_t)b * T * H * D + (int64_t)h * D;

    // The padded operand tiles carry zeros in the upper half of every group;
    // only the lower halves are rewritten per chunk.
    for (int i = tid; i < D * LDP; i += C::NTHR) sm.ke_pad[i] = from_f<E>(0.0f);
    for (int i = tid; i < 16 * LDP; i += C::NTHR) {
        sm.t_pad[i] = from_f<E>(0.0f);
        sm.aqk_pad[i] = from_f<E>(0.0f);
    }

    // ---- state tiles: S[jj][t] = rows 16t.., columns 16*(wave + NW*jj)..
    f32x4 S[C::TPW][C::KT];
    const float* src = nullptr;
    src = ws_start ? ws_start + ((int64_t)seg * BH + bh) * D * D
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
                if (src && jt < C::NT) x = src[(int64_t)row * D + 16 * jt + r];
                S[jj][t][i] = x;
            }
        }
    }

    // ---- prefetch registers for one chunk (this thread's gate-stage elements).
    // Buffer loads with scalar bases; the loads stay in flight until the
    // chunk's gate stage.  Idle lanes read a valid element and ignore it.
    typedef typename Pair<E>::T RawPair;
    typedef typename BufQuad<E>::T TQuad;
    struct Pref {
        f32x2 th[C::PPT];
        RawPair k[C::PPT], q[C::PPT], v[C::PPT];
    };
    // Inputs used only after the gate stage -- T[r][4g .. 4g+3] (TWS) and beta
    // of tokens 4g .. 4g+3 (the rows of this lane's tiles) -- have a set of
    // their own, refilled for the next chunk as soon as the current chunk is
    // done with them.
    TQuad t_l;
    float b_l[4];
    // Prefetch distance in chunks: two register sets where registers allow it
    // (the out kernel that reads T), one otherwise.
    constexpr int PFD = TWS ? 2 : 1;
    Pref pa, pb;
    const uint32_t lane_tok = (uint32_t)(pgi * C::PPT);          // first token of this lane in a chunk
    const uint32_t lane_ch = gact ? (uint32_t)ch : 0u;
    const uint32_t tstr = (uint32_t)tok_stride;                  // elements between tokens
    // Per-lane element offsets of this lane's tokens inside a chunk (loop
    // invariant).  Each load carries its full offset in the lane register, so a
    // resource sized to the chunk's valid tokens returns zeros for the padding
    // tokens of the final, partial chunk and every chunk runs the same loads.
    uint32_t el_off[C::PPT], b_off[4];
#pragma unroll
    for (int p = 0; p < C::PPT; ++p) el_off[p] = (lane_tok + (uint32_t)p) * tstr + lane_ch;
#pragma unroll
    for (int i = 0; i < 4; ++i) b_off[i] = (uint32_t)(4 * g + i) * (uint32_t)H * 4u;
    auto load_chunk = [&](int n, Pref& d) {
        const int t0 = n * CHUNK;
        const uint32_t nvalid = (uint32_t)min(CHUNK, T - t0);             // uniform
        const int64_t base = head_base + (int64_t)t0 * tok_stride;       // uniform
        const uint32_t span = nvalid * tstr;                             // elements of valid tokens
        const Rsrc rth = make_rsrc(theta + base, span * 4u);
        const Rsrc rk = make_rsrc(k + base, span * (uint32_t)sizeof(E));
        const Rsrc rq = make_rsrc(q + base, span * (uint32_t)sizeof(E));
        const Rsrc rv = make_rsrc(v + base, span * (uint32_t)sizeof(E));
#pragma unroll
        for (int p = 0; p < C::PPT; ++p) {
            d.th[p] = buf_ld_f2(rth, el_off[p] * 4u, 0u);
            d.k[p] = BufPair<E>::ld(rk, el_off[p] * (uint32_t)sizeof(E), 0u);
            d.q[p] = BufPair<E>::ld(rq, el_off[p] * (uint32_t)sizeof(E), 0u);
            d.v[p] = BufPair<E>::ld(rv, el_off[p] * (uint32_t)sizeof(E), 0u);
        }
    };
    auto load_late = [&](int n) {
        const int t0 = n * CHUNK;
        const uint32_t nvalid = (uint32_t)min(CHUNK, T - t0);             // uniform
        if constexpr (!TWS) {
            const Rsrc rb = make_rsrc(beta + ((int64_t)b * T + t0) * H + h, nvalid * (uint32_t)H * 4u);
#pragma unroll
            for (int i = 0; i < 4; ++i) b_l[i] = __builtin_bit_cast(float, buf_ld32(rb, b_off[i], 0u));
        } else {
            t_l = BufQuad<E>::ld(make_rsrc(ws_t + ((int64_t)bh * nchunks + n) * 256),
                                 (uint32_t)(r * 16 + 4 * g) * (uint32_t)sizeof(E), 0u);
        }
    };


    // ---- write the o tile of chunk n (staged in LDS) with coalesced stores.
    // Every thread stores the same number of units for a full chunk, so no
    // branch guards the stores in the main loop; rows past T only occur in
    // the final chunk, which is stored after the loop with a row mask.
    constexpr int OB = 16 * D * (int)sizeof(E);             // bytes of one o tile
    constexpr int SU = OB / C::NTHR >= 16 ? 16 : (OB / C::NTHR >= 8 ? 8 : 4);
    constexpr int UPR = D * (int)sizeof(E) / SU;            // units per row
    constexpr int NU = OB / SU;                             // units per tile
    constexpr int UPT = (NU + C::NTHR - 1) / C::NTHR;       // units per thread
    typedef typename StoreUnit<SU>::T Unit;
    // With the output gate, z of the units a thread stores for chunk n is loaded
    // during chunk n's gate stage (load_z) and used when that tile is stored
    // during the next chunk; a thread without a unit reads offset 0 and ignores it.
    Unit z_l[UPT];
    auto load_z = [&](int n) {
        const int t0 = n * CHUNK;
        const uint32_t nvalid = (uint32_t)min(CHUNK, T - t0);
        const Rsrc rz = make_rsrc(z + head_base + (int64_t)t0 * tok_stride,
                                  nvalid * (uint32_t)tok_stride * (uint32_t)sizeof(E));
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int u = tid + C::NTHR * j;
            const int row = u / UPR, ce = (u % UPR) * (SU / (int)sizeof(E));
            const bool has = NU % C::NTHR == 0 || u < NU;
            z_l[j] = ld_unit<SU>(rz, has ? ((uint32_t)row * (uint32_t)tok_stride + (uint32_t)ce) * (uint32_t)sizeof(E) : 0u);
        }
    };
    auto store_o = [&](int n, bool masked) {
        const int t0 = n * CHUNK;
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const int u = tid + C::NTHR * j;
            const int row = u / UPR, ce = (u % UPR) * (SU / (int)sizeof(E));
            if ((NU % C::NTHR == 0 || u < NU) && (!masked || t0 + row < T)) {
                Unit val = *reinterpret_cast<const Unit*>(&sm.o_tile[row * C::LDR + ce]);
                if constexpr (GATE) val = gate_unit<E>(val, z_l[j]);
                *reinterpret_cast<Unit*>(o + head_base + (int64_t)(t0 + row) * tok_stride + ce) = val;
            }
        }
    };

    // Gate arithmetic in base 2: g2 = g*log2(e), G2 its in-chunk prefix sum,
    // Gamma = 2^G2.
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float GMIN2 = G_MIN * LOG2E;

    // ---- one chunk.  PARTIAL: the final chunk with fewer than 16 tokens; its
    // padding tokens get g = 0, beta = k = q = v = 0, which leave the state unchanged.
    auto chunk = [&](auto partial_tag, int n, Pref& cur) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
        const int t0 = n * CHUNK;
        // ---------------- stage 1: gate, cumulative decay, scaled operand tiles
        float G0[C::PPT], G1[C::PPT];
        float run0 = 0.0f, run1 = 0.0f;
#pragma unroll
        for (int p = 0; p < C::PPT; ++p) {
            float ga, gb;
            if constexpr (UNB) {   // -softplus(theta) log2(e) = -(max(theta, 0) log2(e) + log2(1 + 2^(-|theta| log2(e))))
                const float x0 = cur.th[p][0], x1 = cur.th[p][1];
                ga = -(fmaxf(x0, 0.0f) * LOG2E + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * fabsf(x0))));
                gb = -(fmaxf(x1, 0.0f) * LOG2E + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * fabsf(x1))));
            } else {
                ga = GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * cur.th[p][0]));
                gb = GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * cur.th[p][1]));
            }
            if (PARTIAL || !ALL_ACT) {
                const bool ok = gact && (!PARTIAL || t0 + pgi * C::PPT + p < T);
                ga = ok ? ga : 0.0f;
                gb = ok ? gb : 0.0f;
            }
            run0 += ga;
            run1 += gb;
            G0[p] = run0;
            G1[p] = run1;
        }
        // inclusive scan of the group totals across the NPG lanes of this pair
        float inc0 = run0, inc1 = run1;
#pragma unroll
        for (int d = 1; d < C::NPG; d <<= 1) {
            const float u0 = __shfl_up(inc0, d * C::PW), u1 = __shfl_up(inc1, d * C::PW);
            if (pgi >= d) { inc0 += u0; inc1 += u1; }
        }
        const float tot0 = __shfl(inc0, (C::NPG - 1) * C::PW + lane % C::PW);
        const float tot1 = __shfl(inc1, (C::NPG - 1) * C::PW + lane % C::PW);
        if (gact) {
            const float off0 = inc0 - run0, off1 = inc1 - run1;
            const float eC0 = __builtin_amdgcn_exp2f(tot0), eC1 = __builtin_amdgcn_exp2f(tot1);
            if (pgi == 0) {
                sm.gc[ch] = eC0;
                sm.gc[ch + 1] = eC1;
            }
            float kea[C::PPT], keb[C::PPT];
            RawPair vr[C::PPT];
#pragma unroll
            for (int p = 0; p < C::PPT; ++p) {
                const int pos = pgi * C::PPT + p;
                const float Ga = G0[p] + off0, Gb = G1[p] + off1;
                const float eGa = __builtin_amdgcn_exp2f(Ga), eGb = __builtin_amdgcn_exp2f(Gb);
                float ka = to_f(cur.k[p][0]), kb = to_f(cur.k[p][1]);
                float qa = to_f(cur.q[p][0]), qb = to_f(cur.q[p][1]);
                vr[p] = cur.v[p];
                if (PARTIAL && !(t0 + pos < T)) {   // padding token: k = q = v = 0
                    ka = kb = qa = qb = 0.0f;
                    vr[p][0] = vr[p][1] = from_f<E>(0.0f);
                }
                if constexpr (UNB) {
                    // Kend = k 2^(G_C - G) directly (1/Gamma may overflow); raw k, q and G2
                    // for the position-wise diagonal tiles
                    kea[p] = ka * __builtin_amdgcn_exp2f(tot0 - Ga);
                    keb[p] = kb * __builtin_amdgcn_exp2f(tot1 - Gb);
                    store_pair(&sm.km_row[pos * SM::LDQ + ch], ka, kb);
                    store_pair(&sm.q_row[pos * SM::LDQ + ch], qa, qb);
                    *reinterpret_cast<f32x2*>(&sm.g_row[pos * (D + 4) + ch]) = f32x2{Ga, Gb};
                } else {
                    const float emGa = __builtin_amdgcn_exp2f(-Ga), emGb = __builtin_amdgcn_exp2f(-Gb);
                    const float kma = ka * emGa, kmb = kb * emGb;
                    kea[p] = kma * eC0;                 // k * exp(G_C - G), every factor <= 1 in range
                    keb[p] = kmb * eC1;
                    store_pair(&sm.km_row[pos * SM::LDQ + ch], kma, kmb);
                }
                store_pair(&sm.kn_row[pos * SM::LDQ + ch], -ka * eGa, -kb * eGb);
                store_pair(&sm.qp_row[pos * SM::LDQ + ch], qa * eGa, qb * eGb);
            }
            const int pos0 = pgi * C::PPT;
            const int kp = 8 * (pos0 >> 2) + (pos0 & 3);   // padded slot of token pos0
            store_run<E, C::PPT>(&sm.ke_pad[ch * LDP + kp], kea);
            store_run<E, C::PPT>(&sm.ke_pad[(ch + 1) * LDP + kp], keb);
            store_pair_runs<E, C::PPT>(&sm.v_col[ch * C::LDC + pos0], &sm.v_col[(ch + 1) * C::LDC + pos0], vr);
        }
        if (n > c0) store_o(n - 1, false);   // the previous chunk is always a full one
        // z of this chunk (used when its o tile is stored, during the next chunk) is
        // issued before the prefetch: loads retire in order, and waiting for z must
        // not mean waiting for the prefetch as well
        if constexpr (GATE) load_z(n);
        if (n + PFD < c1) load_chunk(n + PFD, cur);   // in flight until that chunk's gate stage
        lds_barrier();

        // beta of rows 4g+i (zero past T: loads of padding tokens return zero)
        f32x4 btv = f32x4{0, 0, 0, 0};
        if constexpr (!TWS) btv = f32x4{b_l[0], b_l[1], b_l[2], b_l[3]};

        // ---------------- stage 2: diagonal tiles, then the state-side products
        // for every column tile, overlapped with the triangular solve:
        //   Y   = beta*(V - K+ S)      (so that U = T Y = Ut - W S)
        //   O1^T = S^T Q+^T
        if constexpr (UNB) {
            // Position-wise diagonal tiles in fp32: thread (t, s) forms A[t][s] and
            // A_qk[t][s] for s <= t; both share the decay weight of every channel.
            const int tt = tid >> 4, ss = tid & 15;
            float dkk = 0.0f, dqk = 0.0f;
            if (ss <= tt) {
                const float* Gt = &sm.g_row[tt * (D + 4)];
                const float* Gs = &sm.g_row[ss * (D + 4)];
                const E* kt = &sm.km_row[tt * SM::LDQ];
                const E* ks = &sm.km_row[ss * SM::LDQ];
                const E* qt = &sm.q_row[tt * SM::LDQ];
                for (int c = 0; c < D; c += 4) {
                    const f32x4 gt = *reinterpret_cast<const f32x4*>(Gt + c);
                    const f32x4 gs = *reinterpret_cast<const f32x4*>(Gs + c);
                    const auto k4t = ld_quad(kt + c), k4s = ld_quad(ks + c), q4t = ld_quad(qt + c);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float kw = to_f(k4s[i]) * __builtin_amdgcn_exp2f(gt[i] - gs[i]);   // weight <= 1
                        dkk = fmaf(to_f(k4t[i]), kw, dkk);
                        dqk = fmaf(to_f(q4t[i]), kw, dqk);
                    }
                }
            }
            // beta of row tt: lanes 16*wave .. hold beta of rows 4*wave + i in b_l[i]
            float bt = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = __shfl(b_l[i], 16 * wave);
                bt = (tt - 4 * wave == i) ? x : bt;
            }
            sm.akk_t[ss * 20 + tt] = ss < tt ? bt * dkk : 0.0f;
            sm.aqk_pad[tt * LDP + 8 * (ss >> 2) + (ss & 3)] = from_f<E>(ss <= tt ? dqk : 0.0f);
            lds_barrier();
        } else if (!TWS && wave == 0) {
            // A = StrictLower(beta K+ K-^T), kept transposed in LDS: akk_t[col][row]
            const f32x4 a = MM::template mm_ll<D>(sm.kn_row, SM::LDQ, sm.km_row, SM::LDQ,
                                                  f32x4{0, 0, 0, 0}, r, g);
            f32x4 m;
#pragma unroll
            for (int i = 0; i < 4; ++i) m[i] = (r < 4 * g + i) ? -btv[i] * a[i] : 0.0f;   // mask by select
            *reinterpret_cast<f32x4*>(&sm.akk_t[r * 20 + 4 * g]) = m;
        } else if (wave == (TWS ? 0 : 1)) {
            // A_qk^T = K- Q+^T; lane (g, r) holds A_qk[r][4g+i], i.e. four
            // consecutive k-slots of row r of the padded tile
            const f32x4 a = MM::template mm_ll<D>(sm.km_row, SM::LDQ, sm.qp_row, SM::LDQ,
                                                  f32x4{0, 0, 0, 0}, r, g);
            f32x4 m;
#pragma unroll
            for (int i = 0; i < 4; ++i) m[i] = (4 * g + i <= r) ? a[i] : 0.0f;
            store4<E>(&sm.aqk_pad[r * LDP + 8 * g], m);
        }
        // Tiles of this wavefront: jt = wave + NW*jj for jj < nv (wave-uniform).
        const int nv = C::NT % C::NW == 0 ? C::TPW : (wave < C::NT ? min(C::TPW, (C::NT - 1 - wave) / C::NW + 1) : 0);
        f32x4 y[C::TPW], o1[C::TPW];
        BFrag sb[C::TPW * C::KT];
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NW * jj;
#pragma unroll
            for (int t = 0; t < C::KT; ++t) sb[jj * C::KT + t] = MM::to_b(S[jj][t]);
            f32x4 yc = f32x4{0, 0, 0, 0};
            if (jj < nv && jt < D / 16) {   // value columns; the M part of a widened state has V = 0
                const int cb = (16 * jt + r) * C::LDC + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) yc[i] = to_f(sm.v_col[cb + i]);
            }
            y[jj] = yc;
            o1[jj] = f32x4{0, 0, 0, 0};
        }
        MM::template mm_la_n<D, C::TPW>(sm.kn_row, SM::LDQ, sb, y, nv, r, g);
        MM::template mm_al_n<D, C::TPW>(sb, sm.qp_row, SM::LDQ, o1, nv, r, g);
        // The products above are issued before the solve starts (matrix cores
        // run them while the solve proceeds); keeping the two apart in the
        // instruction stream also keeps their registers from being live at once.
        __builtin_amdgcn_sched_barrier(0);
        if (!TWS && wave == 0) {
            // T = (I + A)^-1, column j per lane, right-looking substitution: once
            // x[s] is final, every later row subtracts A[r][s] x[s].  (The LDS
            // round trip stays inside this wavefront, which executes in order.)
            const int j = lane & 15;
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == j) ? 1.0f : 0.0f;
#pragma unroll
            for (int s = 0; s < 15; ++s) {
                f32x4 col[4];
#pragma unroll
                for (int c = s / 4; c < 4; ++c)
                    col[c] = *reinterpret_cast<const f32x4*>(&sm.akk_t[s * 20 + 4 * c]);
                const float xs = x[s];
#pragma unroll
                for (int rr = s + 1; rr < 16; ++rr) x[rr] = fmaf(-col[rr >> 2][rr & 3], xs, x[rr]);
            }
            if (lane < 16) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) sm.t_pad[rr * LDP + 8 * (j >> 2) + (j & 3)] = from_f<E>(x[rr]);
            }
        }
        lds_barrier();

        // ---------------- stage 3: U = T Y, output, state update per column tile
        // (operand fragments shared by the tiles are loaded once)
        PFrag up[C::TPW];
        {
            PFrag tf;
            if constexpr (TWS) tf = MM::pad(t_l);
            else tf = MM::ld_p(&sm.t_pad[r * LDP], g);
            PFrag qf;
            qf = MM::ld_p(&sm.aqk_pad[r * LDP], g);
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                if (jj >= nv) continue;
                const int jt = wave + C::NW * jj;
                f32x4 yy = y[jj];
                if constexpr (!TWS) {   // the published T' already carries diag(beta)
#pragma unroll
                    for (int i = 0; i < 4; ++i) yy[i] *= btv[i];
                }
                up[jj] = MM::to_p(MM::mm16(tf, MM::to_p(yy), f32x4{0, 0, 0, 0}));
                // O^T = O1^T + U^T A_qk^T: lane (g, r) holds o[token r][16jt + 4g + i]
                const f32x4 ot = MM::mm16(up[jj], qf, o1[jj]);
                store4<E>(&sm.o_tile[r * C::LDR + 16 * jt + 4 * g], ot);
            }
        }
        if (n + 1 < c1) load_late(n + 1);   // T and beta are no longer needed for this chunk
#pragma unroll
        for (int t = 0; t < C::KT; ++t) {
            const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[16 * t + 4 * g]);
            const PFrag kf = MM::ld_p(&sm.ke_pad[(16 * t + r) * LDP], g);
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                if (jj >= nv) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) S[jj][t][i] *= gcv[i];
                S[jj][t] = MM::mm16(kf, up[jj], S[jj][t]);
            }
        }
        lds_barrier();
    };

    load_chunk(c0, pa);
    load_late(c0);
    if (PFD == 2 && c0 + 1 < c1) load_chunk(c0 + 1, pb);
    // Retire every load issued so far (start state, first chunk) before the
    // loop: otherwise the compiler's wait-counter analysis carries them into the
    // loop and makes uses of the state registers wait for the next chunk's
    // prefetch as well.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();   // zero-filled padding visible to every wavefront
    // chunk m uses register set pa if (m - c0) is even, pb otherwise
    int n = c0;
    if constexpr (PFD == 2) {
        for (; n + 1 < c_full; n += 2) {
            chunk(std::false_type{}, n, pa);
            chunk(std::false_type{}, n + 1, pb);
        }
    }
    for (; n < c_full; ++n) chunk(std::false_type{}, n, pa);   // at most one left when PFD == 2
    if (c_full < c1) {
        if (PFD == 2 && ((c_full - c0) & 1)) chunk(std::true_type{}, c_full, pb);
        else chunk(std::true_type{}, c_full, pa);
    }
    store_o(c1 - 1, true);

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
                if (S_T && seg == nseg - 1)
                    S_T[((int64_t)bh * D + row) * D + 16 * jt + r] = S[jj][t][i];
            }
    }
}

// Start state of every segment: S_0 = S0 (or 0), S_{s+1} = M_s S_s + N_s, where
// [N_s | M_s] is the widened end state the map kernel stored for segment s (N_s
// in fp32, M_s in the operand type: every step streams all of M_s through the
// compute unit, so its size sets the pace).
// Columns of the state are independent, so one workgroup owns one 16-column
// tile of one head, and each of its wavefronts one 16-row tile of it.  The
// column tile is shared through LDS (transposed, rounded to the operand type)
// at every step; the row of M_s and the N_s tile a wavefront needs are fetched
// two steps ahead into a three-slot register ring.  Every step runs the same
// loads and stores: a fetch past the last map reads zeros and a store past the
// last start state is dropped (buffer resources of size zero), so the loop
// holds no conditional memory access that would make the compiler wait for the
// prefetch.
constexpr int COMBINE_XCDS = 8;   // accelerator complex dies of an MI355X

template <typename E, int D>
struct CombineCfg {
    static constexpr int KT = D / 16, NT = D / 16;
    static constexpr int NW = KT;                    // one wavefront per 16-row tile
    static constexpr int LDT = D + 8;                // padded row of the transposed tile
    // bf16: a wavefront's 16 rows of M_s are one contiguous block of 32D bytes,
    // fetched with whole-wavefront 16-byte loads and laid out as operand
    // fragments through the wavefront's own LDS rows
    static constexpr int MB = 16 * D * 2;            // bytes of the block
    static constexpr int NML = MB >= 1024 ? MB / 1024 : 1;   // 16-byte loads per lane
    static constexpr int LDM = D + 8;                // padded LDS row of the block
};

template <typename E, int D>
__global__ void __launch_bounds__(64 * (D / 16))
combine_kernel(int BH, int nseg, const float* S0, const float* __restrict__ ws_n,
               const E* __restrict__ ws_m, float* __restrict__ ws_start) {
    typedef CombineCfg<E, D> C;
    __shared__ alignas(16) E st[16 * C::LDT];   // st[col][row]: the state column tile
    // each wavefront's rows of M_s (bf16 only)
    __shared__ alignas(16) E mw[sizeof(E) == 2 ? C::NW * 16 * C::LDM : 8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int rt = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wavefront's row tile
    const int r = lane & 15, g = lane >> 4;
    // Workgroups are dealt to the 8 XCDs round-robin by index; all column tiles
    // of one head go to the same XCD so that its L2 serves the segment maps
    // (read by every tile) once from HBM.
    const int xcd = blockIdx.x % COMBINE_XCDS, i = blockIdx.x / COMBINE_XCDS;
    const int bh = xcd + COMBINE_XCDS * (i / C::NT), jt = i % C::NT;
    if (bh >= BH) return;
    const int nsteps = nseg - 1;

    // M row 16rt + r as operand fragments: bf16, per 32-column block kb, columns
    // 32kb + 4g .. +3 and 32kb + 16 + 4g .. +3 (the k-map of Ops<bf16>::mm_la);
    // fp32, per 16-column tile t, columns 16t + 4g .. +3
    constexpr bool BF = sizeof(E) == 2;
    constexpr int NMF = BF ? (D >= 32 ? D / 32 : 1) : C::KT;
    typedef typename std::conditional<BF, bf16x8, f32x4>::type MFrag;
    typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
    struct Pref {
        // bf16: the raw block, 16 bytes per lane per load; fp32: operand fragments
        typename std::conditional<BF, u32x4, MFrag>::type m[BF ? C::NML : NMF];
        float n[4];       // N rows 16rt + 4g + i, column 16jt + r
    };
    auto fetch = [&](int s, Pref& pf) {
        const bool in = s < nsteps;
        const Rsrc xn = make_rsrc(ws_n + ((int64_t)s * BH + bh) * D * D, in ? (uint32_t)(D * D * 4) : 0u);
        const Rsrc xm = make_rsrc(ws_m + ((int64_t)s * BH + bh) * D * D, in ? (uint32_t)(D * D * sizeof(E)) : 0u);
        const uint32_t row = (uint32_t)(16 * rt + r) * D;
        if constexpr (BF) {
            const uint32_t blk = (uint32_t)(16 * rt) * D * 2u;   // this wavefront's rows
#pragma unroll
            for (int i = 0; i < C::NML; ++i)
                pf.m[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    xm, (int)(blk + (uint32_t)(i * 64 + lane) * 16u), 0, 0));
        } else {
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
                pf.m[t] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    xm, (int)((row + 16 * t + 4 * g) * 4), 0, 0));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            pf.n[q] = __builtin_bit_cast(float, buf_ld32(xn, (uint32_t)(((16 * rt + 4 * g + q) * D + 16 * jt + r) * 4), 0u));
    };
    auto publish = [&](int s, f32x4 acc) {   // acc: rows 16rt + 4g + i, column 16jt + r
        const Rsrc dst = make_rsrc(ws_start + ((int64_t)s * BH + bh) * D * D,
                                   s <= nsteps ? (uint32_t)(D * D * 4) : 0u);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 16 * rt + 4 * g + q;
            const float val = acc[q];   // (a bit cast of the vector element itself read element 0)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), dst,
                                                  (int)((row * D + 16 * jt + r) * 4), 0, 0);
            st[r * C::LDT + row] = from_f<E>(acc[q]);
        }
    };

    f32x4 acc;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        acc[q] = S0 ? S0[((int64_t)bh * D + 16 * rt + 4 * g + q) * D + 16 * jt + r] : 0.0f;
    Pref ring0, ring1, ring2;
    fetch(0, ring0);
    fetch(1, ring1);
    publish(0, acc);
    // Retire the loads above before the loop, so that the wait counting inside it
    // only sees the loop's own prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();

    // one step: S <- M_s S + N_s, using the prefetched slot `cur`, refilling `nxt2`
    auto step = [&](int s, const Pref& cur, Pref& nxt2) {
        // Keep each step's instructions in its own step: converting the next
        // step's rows early would wait for a fetch issued only one step before.
        __builtin_amdgcn_sched_barrier(0);
        fetch(s + 2, nxt2);
        f32x4 a = f32x4{cur.n[0], cur.n[1], cur.n[2], cur.n[3]};
        if constexpr (BF) {   // bf16 operands, k-map of the accumulator-as-B form
            // the raw block into this wavefront's LDS rows, then row r as fragments
            bf16* mwv = (bf16*)&mw[rt * 16 * C::LDM];
#pragma unroll
            for (int i = 0; i < C::NML; ++i) {
                const int e = (i * 64 + lane) * 8;        // element offset in the block
                if (C::MB >= 1024 || e < 16 * D)
                    *reinterpret_cast<u32x4*>(&mwv[(e / D) * C::LDM + e % D]) = cur.m[i];
            }
            wave_lds_sync();
            if constexpr (D == 16) {
                a = mfma_k16(ld_b4(&mwv[r * C::LDM + 4 * g]), ld_b4((const bf16*)&st[r * C::LDT + 4 * g]), a);
            } else {
#pragma unroll
                for (int kb = 0; kb < D / 32; ++kb) {
                    const bf16* mp = &mwv[r * C::LDM + 32 * kb + 4 * g];
                    const bf16* bp = (const bf16*)&st[r * C::LDT + 32 * kb + 4 * g];
                    a = mfma_k32(cat8(ld_b4(mp), ld_b4(mp + 16)), cat8(ld_b4(bp), ld_b4(bp + 16)), a);
                }
            }
        } else {                          // fp32 operands: step (t, i) contracts row 16t + 4g + i
#pragma unroll
            for (int t = 0; t < C::KT; ++t) {
                const f32x4 b = *reinterpret_cast<const f32x4*>(&st[r * C::LDT + 16 * t + 4 * g]);
#pragma unroll
                for (int q = 0; q < 4; ++q) a = mfma_k4(cur.m[t][q], b[q], a);
            }
        }
        lds_barrier();              // every wavefront has read the old column tile
        publish(s + 1, a);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Whole rounds of three steps; the at most two steps past the last map read
    // zeros and store nothing.
    for (int s = 0; s < nsteps; s += 3) {
        step(s, ring0, ring2);
        step(s + 1, ring1, ring0);
        step(s + 2, ring2, ring1);
    }
}

// ----------------------------------------------------------------------------- host side
SegPlan plan_segments(int T, int requested) {
    SegPlan p;
    p.nchunks = (int)(((int64_t)T + CHUNK - 1) / CHUNK);
    int want = requested < 1 ? 1 : requested;
    if (want > p.nchunks) want = p.nchunks;
    p.seg_len = (p.nchunks + want - 1) / want;
    p.nseg = (p.nchunks + p.seg_len - 1) / p.seg_len;
    return p;
}

size_t chunk_workspace_bytes(int B, int H, int dk, int dv, int nseg, int nchunks) {
    if (nseg <= 1) return 0;
    const size_t bh = (size_t)B * H;
    const size_t mn = (size_t)(nseg - 1) * bh * dk * (size_t)(dv + dk);
    const size_t st = (size_t)nseg * bh * dk * dv;
    const size_t tt = (size_t)nchunks * bh * CHUNK * CHUNK;   // T per chunk, sized for fp32
    return (mn + st + tt) * sizeof(float);
}

// Wavefronts per workgroup: four, so that two workgroups share a compute unit
// and one's gate/solve phases overlap the other's matrix-core phases.
constexpr int CHUNK_NW_OUT = 4;

template <typename E, int D>
static hipError_t launch_chunk_t(int B, int T, int H, const SegPlan& p, const void* q,
                                 const void* k, const void* v, const float* theta,
                                 const float* beta, const float* S0, const void* z, void* o,
                                 float* S_T, void* workspace, hipStream_t stream, bool unbounded) {
    const int BH = B * H;
    if (unbounded) {   // the ablation: one segment, no output gate
        hipLaunchKernelGGL((chunk_kernel<E, D, CHUNK_NW_OUT, false, false, true>), dim3((unsigned)BH),
                           dim3(64 * CHUNK_NW_OUT), 0, stream, T, H, BH, p.nchunks, p.nchunks, 1,
                           (const E*)q, (const E*)k, (const E*)v, theta, beta, S0, (const float*)nullptr,
                           (const E*)nullptr, (const E*)nullptr, (E*)o, S_T);
        return hipGetLastError();
    }
    float* ws_start = nullptr;
    E* ws_t = nullptr;
    if (p.nseg > 1) {
        // segment maps: N (fp32) then M (input type, in a region sized for fp32)
        float* ws_n = reinterpret_cast<float*>(workspace);
        E* ws_m = reinterpret_cast<E*>(ws_n + (size_t)(p.nseg - 1) * BH * D * D);
        ws_start = ws_n + (size_t)(p.nseg - 1) * BH * D * (2 * D);
        ws_t = reinterpret_cast<E*>(ws_start + (size_t)p.nseg * BH * D * D);
        const hipError_t e = launch_chunk_map(std::is_same<E, float>::value, B, T, H, D, p, k, v, theta,
                                              beta, ws_n, ws_m, ws_t, stream);
        if (e != hipSuccess) return e;
        const int heads_per_xcd = (BH + COMBINE_XCDS - 1) / COMBINE_XCDS;
        hipLaunchKernelGGL((combine_kernel<E, D>), dim3((unsigned)(COMBINE_XCDS * heads_per_xcd * (D / 16))),
                           dim3(64 * (D / 16)), 0, stream,
                           BH, p.nseg,
                           S0, (const float*)ws_n, (const E*)ws_m, ws_start);
    }
    const bool gate = z != nullptr;
#define KDA_OUT(TWS_, GATE_, GRID, WS_START, WS_T)                                                        \
    hipLaunchKernelGGL((chunk_kernel<E, D, CHUNK_NW_OUT, TWS_, GATE_>), dim3((unsigned)(GRID)),           \
                       dim3(64 * CHUNK_NW_OUT), 0, stream, T, H, BH, p.nchunks, p.seg_len, p.nseg,         \
                       (const E*)q, (const E*)k, (const E*)v, theta, beta, S0, (const float*)(WS_START),   \
                       (const E*)(WS_T), (const E*)z, (E*)o, S_T)
    if (p.nseg > 1 && std::is_same<E, bf16>::value && chunk_out_supported(D)) {
        // bf16: the output pass with producer and consumer wavefronts (kda_out.hip)
        return launch_chunk_out(B, T, H, D, p, q, k, v, theta, ws_t, ws_start, z, o, S_T, stream);
    }
    if (p.nseg > 1) {
        if (gate) KDA_OUT(true, true, BH * p.nseg, ws_start, ws_t);
        else KDA_OUT(true, false, BH * p.nseg, ws_start, ws_t);
    } else {
        if (gate) KDA_OUT(false, true, BH, nullptr, nullptr);
        else KDA_OUT(false, false, BH, nullptr, nullptr);
    }
#undef KDA_OUT
    return hipGetLastError();
}

hipError_t launch_state_combine(int d, int BH, int nseg, const float* init, const float* ws_n, const void* ws_m,
                                float* out, hipStream_t stream) {
    const int heads_per_xcd = (BH + COMBINE_XCDS - 1) / COMBINE_XCDS;
#define KDA_COMB(D)                                                                                          \
    hipLaunchKernelGGL((combine_kernel<bf16, D>), dim3((unsigned)(COMBINE_XCDS * heads_per_xcd * (D / 16))),   \
                       dim3(64 * (D / 16)), 0, stream, BH, nseg, init, ws_n, (const bf16*)ws_m, out);         \
    return hipGetLastError()
    switch (d) {
        case 64: KDA_COMB(64);
        case 128: KDA_COMB(128);
    }
#undef KDA_COMB
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(bool f32, int B, int T, int H, int d, const SegPlan& plan,
                            const void* q, const void* k, const void* v, const float* theta,
                            const float* beta, const float* S0, const void* z, void* o, float* S_T,
                            void* workspace, hipStream_t stream, bool unbounded) {
#define KDA_CH(E, D) \
    return launch_chunk_t<E, D>(B, T, H, plan, q, k, v, theta, beta, S0, z, o, S_T, workspace, stream, unbounded)
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

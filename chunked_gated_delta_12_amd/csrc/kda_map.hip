// kda_map.hip -- segment map kernel of the chunked prefill on gfx950.
//
// A chunk maps the state affinely, S' = M S + N ("Kimi K3 Deep Dive...", "The
// Problem: The Diagonal-Block Dilemma" gives the chunk form; see kda_chunk.hip
// for the algebra).  For every segment but the last, this kernel runs the chunk
// scan with the state widened to [N | M], started from [0 | I], and stores the
// end state (N in fp32, M in the operand type).  For every chunk of every
// segment it also publishes
//     T' = (I + A)^-1 diag(beta),   A = StrictLower(diag(beta) K+ K-^T),
// so that the out kernel forms U = T' (V - K+ S) without a triangular solve.
//
// bf16 at d = 128 (the prefill's shape) builds the same map by walking each
// segment backward: with F_m the chunk's linear part and Z the product of the F's
// of the chunks already walked (I at the start), N <- N + Z Kend^T T' V and
// Z <- Z F_m, M = Z at the segment's start.  Only Z is rescaled by the decay and
// the update of N is 16 deep, so a chunk costs the consumers about half the
// widened forward chain; and the walk ends on each segment's first chunks, which
// the out kernel reads first.  The other types and sizes run the forward chain.
//
// Wavefront roles.  Everything a chunk needs apart from the state -- the
// gate, the decay-scaled tiles, A and T' -- is formed by NPW producer
// wavefronts, one chunk each, into LDS slots.  NCW consumer wavefronts hold
// the state tiles in registers and run only the state chain
//     Y = V - K+ S,   U = T' Y,   S <- Diag(Gamma_C) S + Kend^T U
// over the NPW chunks the producers finished in the previous step.  The slots
// are double buffered, so a single barrier per step of NPW chunks separates
// the two roles, and the consumers run NPW chunks back to back between
// barriers.  A producer lane owns one channel pair of its chunk for all its
// tokens (all 16 when d_k = 128), so the in-chunk prefix of the log-decay stays
// inside the lane; its next chunk's inputs are loaded while it forms A and T'.
//
// SAVE mode (bf16, d = 64 and 128) serves the backward pass: the same chain, not
// widened, from each segment's given start state, writing for every chunk the
// operands the backward sweep reads (kda_launch.hpp, BwdChunkWs): the start state
// of every CKPT-th chunk of the segment (the checkpoints) as row-product operand
// fragments, U and T^T of every chunk, and the Kend and Gamma_C the other chunks'
// states are rebuilt from.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename E, int D, bool SAVE = false>
struct MapCfg {
    static constexpr int NT = SAVE ? D / 16 : D / 8;      // 16-column tiles of [N | M] (SAVE: of S)
    // consumer wavefronts: eight for bf16; four for fp32 (the validation type),
    // whose wider operands need two wavefronts' registers per SIMD
    static constexpr int NCWMAX = sizeof(E) == 2 ? 8 : 4;
    static constexpr int NCW = NT < NCWMAX ? NT : NCWMAX;
    static constexpr int TPW = NT / NCW;                  // state tiles per consumer
    static constexpr int NPW = sizeof(E) == 2 ? 4 : 2;    // producer wavefronts = chunks per step
    static constexpr int NW = NCW + NPW;
    static constexpr int KT = D / 16;                     // 16-row tiles along d_k
    // padded [16][D] rows.  bf16: D + 4 elements, a row stride of 2 (mod 4) dwords,
    // for which the pairs of 8-byte operand reads (k = 4g.., 16 + 4g..) of 16 rows
    // meet no bank conflict; with D + 8 they meet about eight per read on gfx950
    static constexpr int LDR = sizeof(E) == 2 ? D + 4 : D + 8;
    static constexpr int LDK = 20;                        // padded [.][16] rows
    static constexpr int PPL = D / 2 < 64 ? D / 2 : 64;   // channel pairs of a producer
    static constexpr int NTG = 64 / PPL;                  // token groups (lanes per pair)
    static constexpr int TPL = CHUNK / NTG;               // tokens per producer lane
    static_assert(NT % NCW == 0, "state tiles split evenly");
    static_assert(PPL * 2 == D, "one producer wavefront covers all channels");
    // The map by a backward walk (bf16 at d = 128, not SAVE): see the kernel.  Consumer w
    // holds rows 16w.. of Z and N.
    static constexpr bool REV = !SAVE && sizeof(E) == 2 && D == 128;
    static_assert(!REV || (NCW == D / 16 && NTG == 1), "backward walk: one row slab per consumer");
};

// What the consumers read for one chunk.
template <typename E, int D, bool REV = false>
struct MapSlot {
    typedef MapCfg<E, D> C;
    alignas(16) E kn_row[16 * C::LDR];   // -K+ = -K*Gamma            [token][ch]
    alignas(16) E ke_col[D * C::LDK];    // Kend^T = (K*Gamma_C/Gamma)^T [ch][token]
    alignas(16) E v_col[D * C::LDK];     // V^T                       [ch][token]
    alignas(16) E t_row[16 * C::LDK];    // T' = (I + A)^-1 diag(beta) [row][k]
    alignas(16) float gc[D];             // Gamma_C per channel
};
// The backward walk's operands: Kend rows, -K+^T and V^T columns, T'^T.
template <typename E, int D>
struct MapSlot<E, D, true> {
    typedef MapCfg<E, D> C;
    alignas(16) E ke_row[16 * C::LDR];   // Kend = K*Gamma_C/Gamma     [token][ch]
    alignas(16) E kn_col[D * C::LDK];    // -K+^T                     [ch][token]
    alignas(16) E v_col[D * C::LDK];     // V^T                       [ch][token]
    alignas(16) E tt_row[16 * C::LDK];   // T'^T                      [col][row]
    alignas(16) float gc[D];             // Gamma_C per channel
};
// Private to one producer wavefront.
template <typename E, int D, bool REV = false>
struct MapScratch {
    alignas(16) E km_row[16 * MapCfg<E, D>::LDR];   // K- = K/Gamma     [token][ch]
};
template <typename E, int D>
struct MapScratch<E, D, true> {
    alignas(16) E km_row[16 * MapCfg<E, D>::LDR];   // K- = K/Gamma     [token][ch]
    alignas(16) E kn_row[16 * MapCfg<E, D>::LDR];   // -K+ = -K*Gamma   [token][ch]
    alignas(16) E t_row[16 * MapCfg<E, D>::LDK];    // T', for its publication [row][col]
};
template <typename E, int D, bool SAVE = false>
struct MapSmem {
    static constexpr bool REV = MapCfg<E, D, SAVE>::REV;
    MapSlot<E, D, REV> slot[2 * MapCfg<E, D, SAVE>::NPW];
    MapScratch<E, D, REV> scr[MapCfg<E, D, SAVE>::NPW];
};

// N elements as 8-byte stores (4-byte when the run is shorter).
template <typename E, int N>
__device__ __forceinline__ void store_run8(E* p, const E* x) {
    constexpr int B = N * (int)sizeof(E);
    constexpr int U = B >= 8 ? 8 : B;
    constexpr int EPU = U / (int)sizeof(E);
    typedef E V __attribute__((__vector_size__(U)));
#pragma unroll
    for (int u = 0; u < B / U; ++u) {
        V w;
#pragma unroll
        for (int i = 0; i < EPU; ++i) w[i] = x[u * EPU + i];
        *reinterpret_cast<V*>(p + u * EPU) = w;
    }
}

// The LDS-side operand of a K = 16 product, row [.][16] at p (k = 4g .. 4g+3 at
// p).  bf16: the upper four k-slots of the 16x16x32 operand take the next four
// stored elements instead of zeros, saving the register copies that padding
// would cost.  They are finite (data, or row padding zeroed at the start) and
// meet the zero slots of the register-side operand, so they add exact zeros.
__device__ __forceinline__ bf16x8 ld_k16(const bf16* p) { return cat8(ld_b4(p), ld_b4(p + 4)); }
__device__ __forceinline__ f32x4 ld_k16(const float* p) { return ld_quad(p); }

// x[i] -= A[4g+i][4B+J] * xj for the lane's row group g: the coefficient is lane 4B+J of
// the lane's own row of 16 lanes.
template <int B, int J>
__device__ __forceinline__ void tri_axpy(float (&x)[4], const float (&am)[4], float xj) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = fmaf(-row_lane<4 * B + J>(am[i]), xj, x[i]);
}

// One block of four rows of the unit lower triangular solve (I + A) x = e_r, one
// right-hand side per lane column r.  Lane (g, r) holds x[i] = row 4g+i and
// am[i] = A[4g+i][r] (zero on and above the diagonal).  Row block B is finished
// first on its own lanes, then its four values go to every row and the rows below
// subtract their share.
template <int B>
__device__ __forceinline__ void tri_block(float (&x)[4], const float (&am)[4], int g, int lane) {
    const bool own = g == B;
    // within the block: A[4B+i][4B+j] is zero for i <= j, so the update of rows
    // up to j leaves them unchanged; other rows take a zero multiplier
    tri_axpy<B, 0>(x, am, own ? x[0] : 0.0f);
    tri_axpy<B, 1>(x, am, own ? x[1] : 0.0f);
    tri_axpy<B, 2>(x, am, own ? x[2] : 0.0f);
    if constexpr (B < 3) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] = row_to_all<B>(x[j], lane);
            p[j] = g > B ? p[j] : 0.0f;   // rows above B hold zero coefficients; row B is done
        }
        tri_axpy<B, 0>(x, am, p[0]);
        tri_axpy<B, 1>(x, am, p[1]);
        tri_axpy<B, 2>(x, am, p[2]);
        tri_axpy<B, 3>(x, am, p[3]);
    }
}

template <typename E, int D, bool SAVE = false>
__global__ void __launch_bounds__((64 * MapCfg<E, D, SAVE>::NW))
map_kernel(int T, int H, int BH, int nchunks, int seg_len, int nseg,
           const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ theta,
           const float* __restrict__ beta, float* __restrict__ ws_n, E* __restrict__ ws_m,
           E* __restrict__ ws_t, const float* __restrict__ s_start, bf16* __restrict__ ws_b) {
    typedef MapCfg<E, D, SAVE> C;
    typedef BwdChunkWs<D> BW;
    static_assert(!SAVE || (sizeof(E) == 2 && (D == 64 || D == 128) && C::TPW == 1),
                  "SAVE: bf16 at d = 64 and 128, one state tile per consumer");
    typedef Ops<E> MM;
    typedef typename MM::BFrag BFrag;
    typedef typename MM::PFrag PFrag;
    constexpr bool REV = C::REV;
    typedef MapSlot<E, D, REV> Slot;
    __shared__ MapSmem<E, D, SAVE> sm;

    // wave index as a scalar, so that branches on it stay scalar branches
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // segment-major: the workgroups resident at once cover every head of a run of
    // segments, so that concurrent reads of a token row (all heads of it) meet in DRAM
    const int bh = blockIdx.x % BH, seg = blockIdx.x / BH;
    const int b = bh / H, h = bh % H;
    const int c0 = seg * seg_len;
    const int c1 = min(nchunks, c0 + seg_len);
    const int nsteps = (c1 - c0 + C::NPW - 1) / C::NPW;
    const int tend = min(T, c1 * CHUNK);            // the segment's tokens end here
    const bool last = !SAVE && seg == nseg - 1;     // publishes T' only
    // SAVE: the backward workspace of chunk m of this sequence, and the resource of its
    // first `bytes` (none outside the segment: stores through it are dropped)
    auto bws = [&](int m) { return ws_b + ((int64_t)bh * nchunks + m) * BW::WSC; };
    auto bws_rsrc = [&](int m, bool on, uint32_t bytes) {
        return make_rsrc(bws(on ? m : c0), on ? bytes : 0u);
    };

    // zero the padding columns 16 .. LDK-1 of the [.][16] tiles read by ld_k16
    for (int i = tid; i < 2 * C::NPW * (D + 16); i += 64 * C::NW) {
        Slot& sl = sm.slot[i / (D + 16)];
        const int row = i % (D + 16);
        E* pad;
        if constexpr (REV) pad = row < D ? &sl.kn_col[row * C::LDK + 16] : &sl.tt_row[(row - D) * C::LDK + 16];
        else pad = row < D ? &sl.ke_col[row * C::LDK + 16] : &sl.t_row[(row - D) * C::LDK + 16];
#pragma unroll
        for (int j = 0; j < C::LDK - 16; ++j) pad[j] = from_f<E>(0.0f);
    }

    if (wave >= C::NCW) {
        // =================================================================== producer
        const int pw = wave - C::NCW;
        // The producers' chunk is the critical path of every step: let the SIMD
        // issue their instructions first and the consumers' in the gaps.
        __builtin_amdgcn_s_setprio(3);
        MapScratch<E, D, REV>& scr = sm.scr[pw];
        const int p = lane % C::PPL, tg = lane / C::PPL;
        const int ch = 2 * p, tok0 = tg * C::TPL;
        const uint32_t tstr = (uint32_t)(H * D);   // elements between tokens
        const int64_t head_base = (int64_t)b * T * H * D + (int64_t)h * D;
        typedef typename Pair<E>::T RawPair;
        typedef typename BufQuad<E>::T Quad;

        // Inputs of one chunk, loaded a step ahead.  Resources are sized to the
        // chunk's tokens inside the segment: loads of the rest return zeros, and
        // a chunk past the segment's end reads as all padding.
        f32x2 th[C::TPL];
        RawPair kr[C::TPL], vr[C::TPL];
        float bl[4], br;
        auto load = [&](int m) {
            // the backward walk's chunks before the segment read as padding
            const bool before = REV && m < c0;
            const int t0 = (before ? c0 : m) * CHUNK;
            // uniform; kept in a scalar register so the resources below stay scalar
            const uint32_t nv = __builtin_amdgcn_readfirstlane(before ? 0 : max(0, min(CHUNK, tend - t0)));
            const int64_t base = head_base + (int64_t)t0 * tstr;
            const uint32_t span = nv * tstr;
            const Rsrc rth = make_rsrc(theta + base, span * 4u);
            const Rsrc rk = make_rsrc(k + base, span * (uint32_t)sizeof(E));
            const Rsrc rv = make_rsrc(v + base, span * (uint32_t)sizeof(E));
#pragma unroll
            for (int t = 0; t < C::TPL; ++t) {
                const uint32_t el = (uint32_t)(tok0 + t) * tstr + (uint32_t)ch;
                th[t] = buf_ld_f2(rth, el * 4u, 0u);
                kr[t] = BufPair<E>::ld(rk, el * (uint32_t)sizeof(E), 0u);
                vr[t] = BufPair<E>::ld(rv, el * (uint32_t)sizeof(E), 0u);
            }
        };
        // beta of the chunk, loaded once the current chunk's beta is used up
        auto load_beta = [&](int m) {
            const bool before = REV && m < c0;
            const int t0 = (before ? c0 : m) * CHUNK;
            const uint32_t nv = __builtin_amdgcn_readfirstlane(before ? 0 : max(0, min(CHUNK, tend - t0)));
            const Rsrc rb = make_rsrc(beta + ((int64_t)b * T + t0) * H + h, nv * (uint32_t)H * 4u);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bl[i] = __builtin_bit_cast(float, buf_ld32(rb, (uint32_t)(4 * g + i) * (uint32_t)H * 4u, 0u));
            br = __builtin_bit_cast(float, buf_ld32(rb, (uint32_t)r * (uint32_t)H * 4u, 0u));
        };

        constexpr float LOG2E = 1.4426950408889634f;
        constexpr float GMIN2 = G_MIN * LOG2E;

        auto produce = [&](int m, Slot& sl) {
            const int t0 = m * CHUNK;
            const int nv = (REV && m < c0) ? 0 : max(0, min(CHUNK, tend - t0));
            E kea[C::TPL], keb[C::TPL], va[C::TPL], vb[C::TPL];
            E kna[4], knb[4];   // backward walk: -K+ of the lane's channels, four tokens at a time
            float eCa, eCb;
            if constexpr (C::NTG == 1) {
                // The lane holds all 16 tokens of its channel pair, so the decay is
                // formed as products: per-token factor gamma = 2^(g2) (1 for padding
                // tokens), Gamma_t = prefix product, Kend = k * (suffix product after
                // t) = k Gamma_C / Gamma_t, and K- = Kend / Gamma_C.  Three
                // transcendentals per element instead of four.
                float gma[C::TPL], gmb[C::TPL];
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    gma[t] = __builtin_amdgcn_exp2f(GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][0])));
                    gmb[t] = __builtin_amdgcn_exp2f(GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][1])));
                }
                if (nv < CHUNK) {   // the segment's partial last chunk: padding tokens do not decay
#pragma unroll
                    for (int t = 0; t < C::TPL; ++t) {
                        gma[t] = t < nv ? gma[t] : 1.0f;
                        gmb[t] = t < nv ? gmb[t] : 1.0f;
                    }
                }
                float Pa = 1.0f, Pb = 1.0f;   // Gamma_t
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    Pa *= gma[t];
                    Pb *= gmb[t];
                    const float ka = to_f(kr[t][0]), kb = to_f(kr[t][1]);   // zero for padding tokens
                    if constexpr (REV) {
                        kna[t & 3] = from_f<E>(-ka * Pa);
                        knb[t & 3] = from_f<E>(-kb * Pb);
                        store_pair(&scr.kn_row[t * C::LDR + ch], -ka * Pa, -kb * Pb);
                        if ((t & 3) == 3) {   // -K+^T columns, tokens t-3 .. t (8-byte aligned)
                            *reinterpret_cast<bf16x4*>(&sl.kn_col[ch * C::LDK + tok0 + t - 3]) =
                                bf16x4{kna[0], kna[1], kna[2], kna[3]};
                            *reinterpret_cast<bf16x4*>(&sl.kn_col[(ch + 1) * C::LDK + tok0 + t - 3]) =
                                bf16x4{knb[0], knb[1], knb[2], knb[3]};
                        }
                    } else {
                        store_pair(&sl.kn_row[t * C::LDR + ch], -ka * Pa, -kb * Pb);
                    }
                }
                eCa = Pa;
                eCb = Pb;
                // 1 / Gamma_C <= e^80: the bound keeps it finite in fp32
                const float ia = __builtin_amdgcn_rcpf(eCa), ib = __builtin_amdgcn_rcpf(eCb);
                float Qa = 1.0f, Qb = 1.0f;   // product of gamma over the tokens after t
#pragma unroll
                for (int t = C::TPL - 1; t >= 0; --t) {
                    const float ka = to_f(kr[t][0]), kb = to_f(kr[t][1]);
                    const float xa = ka * Qa, xb = kb * Qb;   // Kend, |Kend| <= |k|
                    store_pair(&scr.km_row[t * C::LDR + ch], xa * ia, xb * ib);
                    if constexpr (REV) store_pair(&sl.ke_row[t * C::LDR + ch], xa, xb);
                    kea[t] = from_f<E>(xa);
                    keb[t] = from_f<E>(xb);
                    va[t] = vr[t][0];
                    vb[t] = vr[t][1];
                    if constexpr (sizeof(E) == 4) {   // fp32: column elements one at a time (registers)
                        sl.ke_col[ch * C::LDK + t] = kea[t];
                        sl.ke_col[(ch + 1) * C::LDK + t] = keb[t];
                        sl.v_col[ch * C::LDK + t] = va[t];
                        sl.v_col[(ch + 1) * C::LDK + t] = vb[t];
                    }
                    Qa *= gma[t];
                    Qb *= gmb[t];
                }
            } else {
                // ---- log-decay in base 2 (zero for padding tokens) and its in-lane prefix
                float Ga[C::TPL], Gb[C::TPL];
                float sa = 0.0f, sb = 0.0f;
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    float ga = GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][0]));
                    float gb = GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][1]));
                    const bool ok = tok0 + t < nv;
                    sa += ok ? ga : 0.0f;
                    sb += ok ? gb : 0.0f;
                    Ga[t] = sa;
                    Gb[t] = sb;
                }
                // prefix across the token groups of a pair (d_k < 128 only)
                float offa = 0.0f, offb = 0.0f, tota = sa, totb = sb;
                if constexpr (C::NTG > 1) {
                    float ia = sa, ib = sb;
#pragma unroll
                    for (int d = 1; d < C::NTG; d <<= 1) {
                        const float ua = __shfl_up(ia, d * C::PPL), ub = __shfl_up(ib, d * C::PPL);
                        if (tg >= d) { ia += ua; ib += ub; }
                    }
                    offa = ia - sa;
                    offb = ib - sb;
                    tota = __shfl(ia, (C::NTG - 1) * C::PPL + p);
                    totb = __shfl(ib, (C::NTG - 1) * C::PPL + p);
                }
                eCa = __builtin_amdgcn_exp2f(tota);
                eCb = __builtin_amdgcn_exp2f(totb);
                // ---- scaled tiles: -K+ and K- rows, Kend^T and V^T columns, Gamma_C
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    const int pos = tok0 + t;
                    const float xa = Ga[t] + offa, xb = Gb[t] + offb;
                    const float eGa = __builtin_amdgcn_exp2f(xa), eGb = __builtin_amdgcn_exp2f(xb);
                    const float emGa = __builtin_amdgcn_exp2f(-xa), emGb = __builtin_amdgcn_exp2f(-xb);
                    const float ka = to_f(kr[t][0]), kb = to_f(kr[t][1]);   // zero for padding tokens
                    const float kma = ka * emGa, kmb = kb * emGb;
                    store_pair(&sl.kn_row[pos * C::LDR + ch], -ka * eGa, -kb * eGb);
                    store_pair(&scr.km_row[pos * C::LDR + ch], kma, kmb);
                    kea[t] = from_f<E>(kma * eCa);   // k * exp(G_C - G) <= |k|
                    keb[t] = from_f<E>(kmb * eCb);
                    va[t] = vr[t][0];
                    vb[t] = vr[t][1];
                    if constexpr (sizeof(E) == 4) {   // fp32: column elements one at a time (registers)
                        sl.ke_col[ch * C::LDK + pos] = kea[t];
                        sl.ke_col[(ch + 1) * C::LDK + pos] = keb[t];
                        sl.v_col[ch * C::LDK + pos] = va[t];
                        sl.v_col[(ch + 1) * C::LDK + pos] = vb[t];
                    }
                }
            }
            if constexpr (sizeof(E) == 2) {   // bf16: packed runs of the lane's tokens
                if constexpr (!REV) {
                    store_run8<E, C::TPL>(&sl.ke_col[ch * C::LDK + tok0], kea);
                    store_run8<E, C::TPL>(&sl.ke_col[(ch + 1) * C::LDK + tok0], keb);
                }
                store_run8<E, C::TPL>(&sl.v_col[ch * C::LDK + tok0], va);
                store_run8<E, C::TPL>(&sl.v_col[(ch + 1) * C::LDK + tok0], vb);
            }
            *reinterpret_cast<f32x2*>(&sl.gc[ch]) = f32x2{eCa, eCb};   // token groups write equal values
            if constexpr (SAVE) {
                // a chunk whose successor is no checkpoint leaves its Kend (fragments:
                // wavefront c/16, lane 16 (token group) + c%16, 4 tokens of channel c) and
                // Gamma_C in that successor's state area
                const Rsrc rk = bws_rsrc(m + 1, (m - c0) % BW::CKPT != BW::CKPT - 1 && m + 1 < c1,
                                         BW::KE_BYTES + 4u * D);
#pragma unroll
                for (int q4 = 0; q4 < C::TPL / 4; ++q4) {
                    const int gq = tok0 / 4 + q4;
                    buf_st_quad(bf16x4{kea[4 * q4], kea[4 * q4 + 1], kea[4 * q4 + 2], kea[4 * q4 + 3]}, rk,
                                (uint32_t)(((ch >> 4) * 64 + gq * 16 + (ch & 15)) * 8));
                    buf_st_quad(bf16x4{keb[4 * q4], keb[4 * q4 + 1], keb[4 * q4 + 2], keb[4 * q4 + 3]}, rk,
                                (uint32_t)((((ch + 1) >> 4) * 64 + gq * 16 + ((ch + 1) & 15)) * 8));
                }
                typedef uint32_t U2 __attribute__((__vector_size__(8)));
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(U2, f32x2{eCa, eCb}), rk,
                                                      (int)(BW::GC_OFF + (uint32_t)ch * 4u), 0, 0);
            }
            load(REV ? m - C::NPW : m + C::NPW);   // in flight while A and T' are formed
            wave_lds_sync();

            // ---- A = StrictLower(diag(beta) K+ K-^T): lane (g, r) holds A[4g+i][r]
            const E* kn_rows;
            if constexpr (REV) kn_rows = scr.kn_row;
            else kn_rows = sl.kn_row;
            const f32x4 a = MM::template mm_ll<D>(kn_rows, C::LDR, scr.km_row, C::LDR,
                                                  f32x4{0, 0, 0, 0}, r, g);
            float am[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) am[i] = (r < 4 * g + i) ? -bl[i] * a[i] : 0.0f;   // beta of row 4g+i

            // ---- T = (I + A)^-1 by forward substitution in registers: lane (g, r)
            // holds rows 4g .. 4g+3 of column r.  A[4g+i][s] is lane s of the
            // lane's own row; each finished block of four rows is copied to the
            // rows below it.
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * g + i == r) ? 1.0f : 0.0f;
            tri_block<0>(x, am, g, lane);
            tri_block<1>(x, am, g, lane);
            tri_block<2>(x, am, g, lane);
            tri_block<3>(x, am, g, lane);
            // T' = T diag(beta): column r scaled by beta_r.  The backward walk's consumers
            // take T'^T, whose row r is this lane's column, and T' itself goes to the
            // publication through a tile (rows 4g .. 4g+3 from lane group g).
            E* t_pub;
            if constexpr (REV) {
                t_pub = scr.t_row;
                *reinterpret_cast<bf16x4*>(&sl.tt_row[r * C::LDK + 4 * g]) =
                    bf16x4{(bf16)(x[0] * br), (bf16)(x[1] * br), (bf16)(x[2] * br), (bf16)(x[3] * br)};
            } else {
                t_pub = sl.t_row;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) t_pub[(4 * g + i) * C::LDK + r] = from_f<E>(x[i] * br);
            load_beta(REV ? m - C::NPW : m + C::NPW);
            wave_lds_sync();
            if constexpr (SAVE) {
                // T^T row r (column r of T) for the backward sweep: lane group g stores
                // elements 4g .. 4g+3
                const Rsrc rt = bws_rsrc(m, m < c1, (uint32_t)BW::WSC * 2u);
                const uint32_t o = (uint32_t)(BW::WS_S + BW::WS_U) * 2u + (uint32_t)r * 32u + (uint32_t)g * 8u;
                buf_st_quad(bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]}, rt, o);
            } else {
                // publish T' of chunks inside the segment: lane (g, r) stores T'[r][4g .. 4g+3]
                const Quad tq = ld_quad(&t_pub[r * C::LDK + 4 * g]);
                const bool inside = m >= c0 && m < c1;
                const Rsrc rt = make_rsrc(ws_t + ((int64_t)bh * nchunks + (inside ? m : c0)) * 256,
                                          inside ? 256u * (uint32_t)sizeof(E) : 0u);
                buf_st_quad(tq, rt, (uint32_t)(r * 16 + 4 * g) * (uint32_t)sizeof(E));
            }
        };

        // step s takes chunk c0 + s NPW + pw, or c1 - 1 - (s NPW + pw) in the backward walk
        auto chunk_at = [&](int st) { return REV ? c1 - 1 - (st * C::NPW + pw) : c0 + st * C::NPW + pw; };
        load(chunk_at(0));
        load_beta(chunk_at(0));
        // Retire the first chunk's loads before the loop: the compiler's
        // wait-counter analysis would otherwise merge them with the loop's own
        // prefetch and wait for everything at the top of every step.
        __builtin_amdgcn_s_waitcnt(0);
        for (int s = 0; s < nsteps; ++s) {
            produce(chunk_at(s), sm.slot[(s & 1) * C::NPW + pw]);
            lds_barrier();
        }
        lds_barrier();   // the consumers' last step
    } else if constexpr (REV) {
        // ==================================================== consumer, backward walk
        // The segment's map is F_{L-1} .. F_0 (chunk m: S -> F_m S + G_m with
        // F_m = Diag(Gamma_C) - Kend^T T' K+ and G_m = Kend^T T' V).  Walking its chunks
        // from the last, with Z = F_{L-1} .. F_{m+1} (I at the start) and W = Z Kend^T T':
        //     N <- N + W V,   Z <- Z Diag(Gamma_C) - W K+,
        // and at the segment's start M = Z.  Only Z is rescaled by the decay, and W
        // is 16 columns wide, so a chunk costs about half the widened forward chain.
        // Consumer w holds rows 16w.. of Z (as Z^T tiles, the operand of Kend Z^T) and
        // of N: Zt[t], lane (g, r): Z[16w + r][16t + 4g + i]; Nt[j], lane (g, r):
        // N[16w + 4g + i][16j + r].
        f32x4 Zt[C::KT], Nt[C::KT];
#pragma unroll
        for (int t = 0; t < C::KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Zt[t][i] = (t == wave && 4 * g + i == r) ? 1.0f : 0.0f;
                Nt[t][i] = 0.0f;
            }
        // One chunk of the walk: Z^T <- Diag(Gamma_C) Z^T + (-K+^T) W^T with
        // W = Z Kend^T T'.  Returns W's operand fragment: lane (g, r) holds
        // W[16w + r][token 4g + i].  The chunk's LDS operands are read ahead of their
        // products, so that the reads overlap one another and the products instead
        // of each waiting in turn.
        auto chain_rev = [&](const Slot& sl) -> bf16x4 {
            bf16x8 ka[D / 32];   // Kend rows in mm_la's k-map: block kb, slots 32kb + 4g + (0..3, 16..19)
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) {
                const bf16* a = &sl.ke_row[r * C::LDR + 32 * kb + 4 * g];
                ka[kb] = cat8(ld_b4(a), ld_b4(a + 16));
            }
            // T'^T row r and the -K+^T rows as 16-byte reads: slots 4..7 hold the
            // next four tokens (or the zeroed padding columns), which meet the zero
            // slots of the padded register operand
            const PFrag tt = ld_k16(&sl.tt_row[r * C::LDK + 4 * g]);
            f32x4 gcv[C::KT];
#pragma unroll
            for (int t = 0; t < C::KT; ++t) gcv[t] = *reinterpret_cast<const f32x4*>(&sl.gc[16 * t + 4 * g]);
            // P = Kend Z^T (tokens x the slab's rows of Z), over all channels
            BFrag zb[C::KT];
#pragma unroll
            for (int t = 0; t < C::KT; ++t) zb[t] = MM::to_b(Zt[t]);
            f32x4 pz = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kb = 0; kb < D / 32; ++kb) pz = mfma_k32(ka[kb], cat8(zb[2 * kb], zb[2 * kb + 1]), pz);
            PFrag kn[C::KT];
#pragma unroll
            for (int t = 0; t < C::KT; ++t) kn[t] = ld_k16(&sl.kn_col[(16 * t + r) * C::LDK + 4 * g]);
            // Diag(Gamma_C) Z^T while P is formed
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) Zt[t][i] *= gcv[t][i];
            // W^T = T'^T P
            const f32x4 wt = MM::mm16(tt, MM::to_p(pz), f32x4{0, 0, 0, 0});
            const bf16x4 wb = MM::to_b(wt);
            const PFrag wp = MM::pad(wb);
#pragma unroll
            for (int t = 0; t < C::KT; ++t) Zt[t] = MM::mm16(kn[t], wp, Zt[t]);
            return wb;
        };
        static_assert(C::NPW % 2 == 0, "the walk's chunks pair up for the N update");
        for (int s = 0; s <= nsteps; ++s) {
            if (s > 0 && !last) {
                // slot pp holds chunk c1 - 1 - ((s - 1) NPW + pp): descending.
                // N <- N + W V over two chunks at a time, as one K = 32 product:
                // slots 0..3 of a lane group are the first chunk's tokens 4g..4g+3,
                // slots 4..7 the second's, in both operands.
                const Slot* sp = &sm.slot[((s - 1) & 1) * C::NPW];
#pragma unroll
                for (int pp = 0; pp < C::NPW; pp += 2) {
                    const bf16x4 w0 = chain_rev(sp[pp]);
                    const bf16x4 w1 = chain_rev(sp[pp + 1]);
                    const bf16x8 wpair = cat8(w0, w1);
#pragma unroll
                    for (int j = 0; j < C::KT; ++j) {
                        const int o = (16 * j + r) * C::LDK + 4 * g;
                        Nt[j] = mfma_k32(wpair, cat8(ld_b4(&sp[pp].v_col[o]), ld_b4(&sp[pp + 1].v_col[o])), Nt[j]);
                    }
                }
            }
            lds_barrier();
        }
        if (!last) {
            // M = Z in the operand type the combine kernel uses, N in fp32,
            // both [segment][head][row][column]
            const int64_t rb = ((int64_t)seg * BH + bh) * D;
#pragma unroll
            for (int t = 0; t < C::KT; ++t) {
                *reinterpret_cast<bf16x4*>(&ws_m[(rb + 16 * wave + r) * D + 16 * t + 4 * g]) = MM::to_b(Zt[t]);
#pragma unroll
                for (int i = 0; i < 4; ++i) ws_n[(rb + 16 * wave + 4 * g + i) * D + 16 * t + r] = Nt[t][i];
            }
        }
    } else {
        // =================================================================== consumer
        // state tiles: S[jj][t] = rows 16t.., columns 16*(wave + NCW*jj).. of [N | M]
        // (SAVE: of S, from the segment's start state)
        f32x4 S[C::TPW][C::KT];
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NCW * jj;
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (SAVE)
                        S[jj][t][i] = s_start ? s_start[(((int64_t)seg * BH + bh) * D + 16 * t + 4 * g + i) * D + 16 * jt + r]
                                              : 0.0f;
                    else
                        S[jj][t][i] = (jt >= D / 16 && jt - D / 16 == t && 4 * g + i == r) ? 1.0f : 0.0f;
                }
        }
        // SAVE: the identity as a padded K = 16 operand (lane (g, r): I[4g + i][r])
        typename MM::PFrag eye{};
        if constexpr (SAVE)
            eye = MM::pad(bf16x4{(bf16)(4 * g == r ? 1.0f : 0.0f), (bf16)(4 * g + 1 == r ? 1.0f : 0.0f),
                                 (bf16)(4 * g + 2 == r ? 1.0f : 0.0f), (bf16)(4 * g + 3 == r ? 1.0f : 0.0f)});

        auto chain = [&](const Slot& sl, int m) {
            if constexpr (SAVE) {
                // The start state of a checkpoint chunk, as row-product fragments: fragment
                // (channel tile c, block kb, lane (gl, rl)) holds S[16c + rl][32kb + 4gl ..+3]
                // and S[16c + rl][32kb + 16 + 4gl ..+3]; this wavefront's tile (columns
                // 16jt ..) fills the 8-byte half (jt & 1) of the fragments of block jt / 2.
                // A state tile in accumulator form (lane (g, r): rows 4g + i, column r), taken
                // as the padded A operand, is its transpose; times the identity it comes back
                // as an accumulator that holds S[16t + r][16jt + 4g + i] in lane (g, r), this
                // lane's half fragment.  The bf16 values pass through exactly.
                // Only checkpoint chunks store.  The step's chunks are unrolled and NPW is a
                // multiple of CKPT, so the test is a constant in each unrolled copy.
                static_assert(C::NPW % BW::CKPT == 0, "checkpoints at fixed places of a step");
                if ((m - c0) % BW::CKPT == 0) {
                    const Rsrc rs = bws_rsrc(m, m < c1, (uint32_t)BW::WS_S * 2u);
                    const int jt = wave;
#pragma unroll
                    for (int t = 0; t < C::KT; ++t) {
                        const f32x4 tr = MM::mm16(MM::pad(MM::to_b(S[0][t])), eye, f32x4{0, 0, 0, 0});
                        buf_st_quad(MM::to_b(tr), rs,
                                    (uint32_t)((((t * (D / 32) + (jt >> 1)) * 64 + g * 16 + r) * 16) + 8 * (jt & 1)));
                    }
                }
            }
            // Y = V - K+ S   (the M part of the widened state has V = 0)
            f32x4 y[C::TPW];
            BFrag sb[C::TPW * C::KT];
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const int jt = wave + C::NCW * jj;
#pragma unroll
                for (int t = 0; t < C::KT; ++t) sb[jj * C::KT + t] = MM::to_b(S[jj][t]);
                f32x4 yc = f32x4{0, 0, 0, 0};
                if (jt < D / 16) {
                    const auto vq = ld_quad(&sl.v_col[(16 * jt + r) * C::LDK + 4 * g]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) yc[i] = to_f(vq[i]);
                }
                y[jj] = yc;
            }
            MM::template mm_la_n<D, C::TPW>(sl.kn_row, C::LDR, sb, y, C::TPW, r, g);
            // U = T' Y
            const PFrag tf = ld_k16(&sl.t_row[r * C::LDK + 4 * g]);
            PFrag up[C::TPW];
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const f32x4 ua = MM::mm16(tf, MM::to_p(y[jj]), f32x4{0, 0, 0, 0});
                up[jj] = MM::to_p(ua);
                if constexpr (SAVE) {   // U of this column tile: [tile][lane][tokens 4g ..], 8 bytes per lane
                    const Rsrc ru = bws_rsrc(m, m < c1, (uint32_t)BW::WSC * 2u);
                    buf_st_quad(bf16x4{(bf16)ua[0], (bf16)ua[1], (bf16)ua[2], (bf16)ua[3]}, ru,
                                (uint32_t)(BW::WS_S * 2 + (wave * 64 + lane) * 8));
                }
            }
            // fp32 operands are the state registers themselves: keep the update
            // below from being scheduled into the products above, which would
            // need a second copy of the state
            if constexpr (sizeof(E) == 4) __builtin_amdgcn_sched_barrier(0);
            // S <- Diag(Gamma_C) S + Kend^T U
#pragma unroll
            for (int t = 0; t < C::KT; ++t) {
                const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sl.gc[16 * t + 4 * g]);
                const PFrag kf = ld_k16(&sl.ke_col[(16 * t + r) * C::LDK + 4 * g]);
#pragma unroll
                for (int jj = 0; jj < C::TPW; ++jj) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[jj][t][i] *= gcv[i];
                    S[jj][t] = MM::mm16(kf, up[jj], S[jj][t]);
                }
            }
        };

        for (int s = 0; s <= nsteps; ++s) {
            if (s > 0 && !last) {
                // unrolled: a loop back-edge between two chunks would separate the
                // state products of one from the reads of the next, and the
                // compiler has been seen to under-count matrix-core wait states
                // across back-edges
#pragma unroll
                for (int pp = 0; pp < C::NPW; ++pp) chain(sm.slot[((s - 1) & 1) * C::NPW + pp], c0 + (s - 1) * C::NPW + pp);
            }
            lds_barrier();
        }

        if (!last && !SAVE) {
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const int jt = wave + C::NCW * jj;
#pragma unroll
                for (int t = 0; t < C::KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * t + 4 * g + i;
                        const int64_t rb = (((int64_t)seg * BH + bh) * D + row) * D;
                        // N in fp32; M already in the operand type the combine kernel uses
                        if (jt < D / 16) ws_n[rb + 16 * jt + r] = S[jj][t][i];
                        else ws_m[rb + 16 * (jt - D / 16) + r] = from_f<E>(S[jj][t][i]);
                    }
            }
        }
    }
}

template <typename E, int D>
static hipError_t launch_map_t(int B, int H, int T, const SegPlan& p, const void* k, const void* v,
                               const float* theta, const float* beta, float* ws_n, void* ws_m, void* ws_t,
                               hipStream_t stream) {
    typedef MapCfg<E, D> C;
    const int BH = B * H;
    hipLaunchKernelGGL((map_kernel<E, D>), dim3((unsigned)(BH * p.nseg)), dim3(64 * C::NW), 0, stream,
                       T, H, BH, p.nchunks, p.seg_len, p.nseg, (const E*)k, (const E*)v, theta, beta,
                       ws_n, (E*)ws_m, (E*)ws_t, (const float*)nullptr, (bf16*)nullptr);
    return hipGetLastError();
}

hipError_t launch_chunk_save(int B, int T, int H, int d, const SegPlan& p, const void* k, const void* v,
                             const float* theta, const float* beta, const float* s_start, void* ws_b,
                             hipStream_t stream) {
    const int BH = B * H;
#define KDA_SAVE(D)                                                                                        \
    hipLaunchKernelGGL((map_kernel<bf16, D, true>), dim3((unsigned)(BH * p.nseg)),                         \
                       dim3(64 * MapCfg<bf16, D, true>::NW), 0, stream, T, H, BH, p.nchunks, p.seg_len, p.nseg, \
                       (const bf16*)k, (const bf16*)v, theta, beta, (float*)nullptr, (bf16*)nullptr,        \
                       (bf16*)nullptr, s_start, (bf16*)ws_b);                                              \
    return hipGetLastError()
    switch (d) {
        case 64: KDA_SAVE(64);
        case 128: KDA_SAVE(128);
    }
#undef KDA_SAVE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_map(bool f32, int B, int T, int H, int d, const SegPlan& plan, const void* k,
                            const void* v, const float* theta, const float* beta, float* ws_n, void* ws_m,
                            void* ws_t, hipStream_t stream) {
#define KDA_MAP(E, D) return launch_map_t<E, D>(B, H, T, plan, k, v, theta, beta, ws_n, ws_m, ws_t, stream)
    if (f32) {
        switch (d) {
            case 16: KDA_MAP(float, 16);
            case 32: KDA_MAP(float, 32);
            case 64: KDA_MAP(float, 64);
            case 128: KDA_MAP(float, 128);
        }
    } else {
        switch (d) {
            case 16: KDA_MAP(bf16, 16);
            case 32: KDA_MAP(bf16, 32);
            case 64: KDA_MAP(bf16, 64);
            case 128: KDA_MAP(bf16, 128);
        }
    }
#undef KDA_MAP
    return hipErrorInvalidValue;
}

}  // namespace kda

// kda_out.hip -- output pass of the segmented chunked prefill on gfx950 (bf16).
//
// The chunk algebra is the one of kda_chunk.hip ("Kimi K3 Deep Dive...", "The
// Problem: The Diagonal-Block Dilemma"; the bounded gate of "Architecture Deep
// Dive: Kimi K3...", section 3.2, keeps K- = K/Gamma below exp(80), so every
// tile is a dense bf16 matrix-core product).  This kernel runs once the map and
// combine kernels have produced each segment's true start state (ws_start) and
// each chunk's T' = (I + A)^-1 diag(beta) (ws_t).  One workgroup per (segment,
// head) walks the segment's chunks and writes o (and S_T for the last segment).
//
// Wavefront roles.  Per step of NPW = 2 chunks:
//   producers  two wavefronts per chunk, one per half of the d_k channels.  A
//              lane owns one channel pair for TPL consecutive tokens.  They form
//              the gate g = -5 sigmoid(theta) and its decay as running products
//              (Gamma within the lane, one exchange across the lane's token
//              groups), the tiles -K+, Q+, Kend^T, V^T and Gamma_C, copy T', and
//              each forms the part of A_qk = LowerIncl(Q+ K-^T) that its own
//              channels contribute -- so the two never wait for each other.
//              Their inputs are loaded two steps ahead (two register sets).  They
//              also write out the o tiles staged two steps earlier, each the
//              columns of its own channel half.
//   consumers  hold the state in fp32 accumulator registers (two 16-column
//              tiles each at d_v = 128) and run only the chain
//                  Y = V - K+ S,  O1^T = S^T Q+^T,  U = T' Y,
//                  O^T = O1^T + U^T (A_qk,0 + A_qk,1)^T,
//                  S <- Diag(Gamma_C) S + Kend^T U,
//              staging each o tile in LDS.
// LDS slots are double buffered, so one workgroup barrier per step separates the
// roles, as in the map kernel (kda_map.hip).  The launcher merges pairs of map
// segments when that keeps the whole grid resident at one workgroup per compute
// unit: concurrent reads of a token row then cover every head, which was worth
// more than any change to the roles' arithmetic.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
struct OutCfg {
    static constexpr int NT = D / 16;                 // 16-column state tiles
    // consumer wavefronts: two tiles each at d_v = 128, so that every LDS operand
    // fragment of the state products is read once per two tiles
    static constexpr int NCW = NT < 4 ? NT : 4;
    static constexpr int TPW = NT / NCW;              // state tiles per consumer
    static constexpr int NPW = 2;                     // chunks per step
    static constexpr int NSP = 2;                     // producer wavefronts per chunk
    static constexpr int NW = NCW + NPW * NSP;
    static constexpr int KT = D / 16;                 // 16-row tiles along d_k
    // [16][D] rows: D + 4 elements (a stride of 2 (mod 4) dwords, for which the
    // pairs of 8-byte operand reads meet no bank conflict)
    static constexpr int LDR = D + 4;
    static constexpr int LDK = 20;                    // padded [.][16] rows
    static constexpr int CH = D / NSP;                // channels of one producer
    static constexpr int PPH = CH / 2;                // its channel pairs
    static constexpr int NTG = 64 / PPH;              // token groups (lanes per pair)
    static constexpr int TPL = CHUNK / NTG;           // tokens per producer lane
    static_assert(D >= 32 && D <= 128, "channel halves of at least 16");
    static_assert(NT % NCW == 0 && NTG * PPH == 64 && TPL * NTG == CHUNK, "lane mappings");
};

// What the consumers read for one chunk, and the o tiles they stage for the
// producers to write out: o_st, [token][column] with a row of D + 4 elements (a
// stride of 2 (mod 32) dwords), on which the consumers' 8-byte writes of
// 16 rows and the producers' reads of whole token rows meet no bank conflict.
template <int D>
struct OutSlot {
    typedef OutCfg<D> C;
    alignas(16) bf16 kn_row[16 * C::LDR];            // -K+ = -K*Gamma             [token][ch]
    alignas(16) bf16 qp_row[16 * C::LDR];            // Q+ = Q*Gamma               [token][ch]
    alignas(16) bf16 ke_col[D * C::LDK];             // Kend^T = (K*Gamma_C/Gamma)^T [ch][token]
    alignas(16) bf16 v_col[D * C::LDK];              // V^T                        [ch][token]
    alignas(16) bf16 t_row[16 * C::LDK];             // T' = (I + A)^-1 diag(beta) [row][k]
    alignas(16) bf16 aqk[C::NSP][16 * C::LDK];       // A_qk over each channel half [token][token]
    alignas(16) float gc[D];                         // Gamma_C per channel
    alignas(16) bf16 o_st[16 * (D + 4)];             // the staged o               [token][column]
};
template <int D>
struct OutSmem {
    OutSlot<D> slot[2 * OutCfg<D>::NPW];
    alignas(16) bf16 km_row[OutCfg<D>::NPW][16 * OutCfg<D>::LDR];   // K- = K/Gamma of a chunk in production
};

// The LDS side of a K = 16 product, k = 4g .. 4g+3 at p: the upper four k-slots
// of the 16x16x32 operand take the next four stored elements, which are finite
// (data, or row padding zeroed at the start) and meet the zero slots of the
// register-side operand, so they add exact zeros.
__device__ __forceinline__ bf16x8 out_ldk16(const bf16* p) { return cat8(ld_b4(p), ld_b4(p + 4)); }

__device__ __forceinline__ void out_store4(bf16* p, f32x4 x) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

// N consecutive bf16 values as stores of up to 8 bytes.
template <int N>
__device__ __forceinline__ void out_store_run(bf16* p, const bf16* x) {
    constexpr int U = N >= 4 ? 4 : N;   // elements per store
    typedef bf16 V __attribute__((__vector_size__(U * sizeof(bf16))));
#pragma unroll
    for (int u = 0; u < N / U; ++u) {
        V w;
#pragma unroll
        for (int i = 0; i < U; ++i) w[i] = x[u * U + i];
        *reinterpret_cast<V*>(p + u * U) = w;
    }
}

// The output gate on one store unit of bf16 o: every value times sigmoid of the
// matching value of z, in fp32, rounded once.
template <typename U>
__device__ __forceinline__ U out_gate(U ou, U zu) {
    constexpr int N = (int)(sizeof(U) / sizeof(bf16));
    typedef bf16 V __attribute__((__vector_size__(sizeof(U))));
    const V ov = __builtin_bit_cast(V, ou), zv = __builtin_bit_cast(V, zu);
    V res;
#pragma unroll
    for (int i = 0; i < N; ++i) res[i] = (bf16)((float)ov[i] * out_sigmoid((float)zv[i]));
    return __builtin_bit_cast(U, res);
}

template <int D, bool GATE>
__global__ void __launch_bounds__(64 * OutCfg<D>::NW)
out_kernel(int T, int H, int BH, int nchunks, int seg_len, int nseg, int smul, const bf16* __restrict__ q,
           const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ theta,
           const bf16* __restrict__ ws_t, const float* __restrict__ ws_start, const bf16* __restrict__ z,
           bf16* __restrict__ o, float* __restrict__ S_T) {
    typedef OutCfg<D> C;
    typedef Ops<bf16> MM;
    typedef MM::BFrag BFrag;
    typedef MM::PFrag PFrag;
    typedef OutSlot<D> Slot;
    __shared__ OutSmem<D> sm;

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

    // zero the padding columns 16 .. LDK-1 of the tiles read by out_ldk16
    constexpr int PADROWS = D + 16 * (1 + C::NSP);
    for (int i = tid; i < 2 * C::NPW * PADROWS; i += 64 * C::NW) {
        Slot& sl = sm.slot[i / PADROWS];
        const int row = i % PADROWS;
        bf16* pad = row < D ? &sl.ke_col[row * C::LDK + 16]
                            : (row < D + 16 ? &sl.t_row[(row - D) * C::LDK + 16]
                                            : &sl.aqk[(row - D - 16) / 16][((row - D - 16) % 16) * C::LDK + 16]);
#pragma unroll
        for (int j = 0; j < C::LDK - 16; ++j) pad[j] = (bf16)0.0f;
    }

    if (wave >= C::NCW) {
        // =================================================================== producer
        const int pwv = wave - C::NCW;
        const int pp = pwv / C::NSP, hf = pwv % C::NSP;   // chunk of the step, channel half
        // The producers' chunks pace every step: let the SIMD issue their
        // instructions first and the consumers' in the gaps.
        __builtin_amdgcn_s_setprio(3);
        const int p = lane % C::PPH, tg = lane / C::PPH;
        const int ch = hf * C::CH + 2 * p, tok0 = tg * C::TPL;
        const uint32_t tstr = (uint32_t)(H * D);          // elements between tokens
        const int64_t head_base = (int64_t)b * T * H * D + (int64_t)h * D;
        bf16* km = sm.km_row[pp];

        // Inputs of one chunk, loaded a step ahead.  Resources are sized to the
        // chunk's tokens inside the segment: loads of the rest return zeros, and
        // a chunk past the segment's end reads as all padding (T' = 0 too).
        // Two register sets, used by alternate steps: a chunk's inputs are loaded
        // two steps ahead, so that a whole step of other work hides their latency.
        struct Pref {
            f32x2 th[C::TPL];
            bf16x2 kr[C::TPL], vr[C::TPL], qr[C::TPL];
            bf16x4 tl;   // T'[r][4g .. 4g+3]
        };
        Pref pa, pb;
        auto load = [&](int m, Pref& d) {
            f32x2* th = d.th;
            bf16x2 *kr = d.kr, *vr = d.vr, *qr = d.qr;
            bf16x4& tl = d.tl;
            const int t0 = m * CHUNK;
            // uniform; kept in a scalar register so the resources below stay scalar
            const uint32_t nv = __builtin_amdgcn_readfirstlane(max(0, min(CHUNK, tend - t0)));
            const int64_t base = head_base + (int64_t)t0 * tstr;
            const uint32_t span = nv * tstr;
            const Rsrc rth = make_rsrc(theta + base, span * 4u);
            const Rsrc rk = make_rsrc(k + base, span * 2u);
            const Rsrc rv = make_rsrc(v + base, span * 2u);
            const Rsrc rq = make_rsrc(q + base, span * 2u);
#pragma unroll
            for (int t = 0; t < C::TPL; ++t) {
                const uint32_t el = (uint32_t)(tok0 + t) * tstr + (uint32_t)ch;
                // the inputs' last reads: non-temporal
                th[t] = buf_ld_f2<kCpStream>(rth, el * 4u, 0u);
                kr[t] = BufPair<bf16>::ld<kCpStream>(rk, el * 2u, 0u);
                vr[t] = BufPair<bf16>::ld<kCpStream>(rv, el * 2u, 0u);
                qr[t] = BufPair<bf16>::ld<kCpStream>(rq, el * 2u, 0u);
            }
            const Rsrc rt = make_rsrc(ws_t + ((int64_t)bh * nchunks + m) * 256, m < c1 ? 512u : 0u);
            tl = BufQuad<bf16>::ld(rt, (uint32_t)(r * 16 + 4 * g) * 2u, 0u);
        };

        // o tiles.  Each producer writes out the columns of its own channel half of
        // the chunk staged in its slot, so neither producer of a chunk waits for the other.
        // Units of UE elements, UPH per token row of the half, one per lane and pass.
        constexpr int UE = D / 2 >= 64 ? 8 : 4;          // elements per unit (16 or 8 bytes)
        constexpr int UPH = (D / 2) / UE;                // units per token row of a half
        constexpr int NUH = 16 * UPH / 64;               // units per lane
        static_assert(NUH >= 1 && 16 * UPH % 64 == 0, "whole units per lane");
        typedef uint32_t Unit __attribute__((__vector_size__(UE * 2)));
        auto unit_tc = [&](int jj, int& t, int& col) {   // token and column of this lane's unit jj
            const int u = lane + 64 * jj;
            t = u / UPH;
            col = hf * (D / 2) + (u % UPH) * UE;
        };
        auto unit_off = [&](int jj) {   // byte offset of unit jj inside a chunk of o
            int t, col;
            unit_tc(jj, t, col);
            return (int)(((uint32_t)t * tstr + (uint32_t)col) * 2u);
        };
        // o (and z) of chunk mo: the resource covers the chunk's valid tokens (none
        // when !valid), so rows past the segment or past T are dropped or read as zero
        auto o_rsrc = [&](const bf16* base, int mo, bool valid) {
            const int t0 = mo * CHUNK;
            const uint32_t nv = __builtin_amdgcn_readfirstlane(valid ? max(0, min(CHUNK, tend - t0)) : 0);
            return make_rsrc(base + head_base + (int64_t)t0 * tstr, nv * tstr * 2u);
        };
        Unit zl[GATE ? NUH : 1];   // GATE: z of the units stored next
        auto load_z = [&](int mo, bool valid) {
            const Rsrc rz = o_rsrc(z, mo, valid);
#pragma unroll
            for (int jj = 0; jj < NUH; ++jj) {
                if constexpr (UE == 8)
                    zl[jj] = __builtin_bit_cast(Unit, __builtin_amdgcn_raw_buffer_load_b128(rz, unit_off(jj), 0, kCpStream));
                else
                    zl[jj] = __builtin_bit_cast(Unit, __builtin_amdgcn_raw_buffer_load_b64(rz, unit_off(jj), 0, kCpStream));
            }
        };
        auto store_o = [&](int mo, const Slot& sl, bool valid) {
            const Rsrc ro = o_rsrc(o, mo, valid);
#pragma unroll
            for (int jj = 0; jj < NUH; ++jj) {
                int t, col;
                unit_tc(jj, t, col);
                // 8-byte halves: the staged rows are 8-byte aligned
                const bf16* sp = &sl.o_st[t * (D + 4) + col];
                Unit val;
                if constexpr (UE == 8) {
                    typedef uint32_t U2 __attribute__((__vector_size__(8)));
                    const U2 lo = *reinterpret_cast<const U2*>(sp), hi = *reinterpret_cast<const U2*>(sp + 4);
                    val = Unit{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    val = *reinterpret_cast<const Unit*>(sp);
                }
                if constexpr (GATE) val = out_gate<Unit>(val, zl[jj]);
                // o is written once and not read back here: non-temporal
                if constexpr (UE == 8)
                    __builtin_amdgcn_raw_buffer_store_b128(val, ro, unit_off(jj), 0, kCpStream);
                else
                    __builtin_amdgcn_raw_buffer_store_b64(val, ro, unit_off(jj), 0, kCpStream);
            }
        };

        constexpr float LOG2E = 1.4426950408889634f;
        constexpr float GMIN2 = G_MIN * LOG2E;

        auto produce = [&](int m, Slot& sl, Pref& cur) {
            const f32x2* th = cur.th;
            const bf16x2 *kr = cur.kr, *vr = cur.vr, *qr = cur.qr;
            const int nv = max(0, min(CHUNK, tend - m * CHUNK));
            // per-token decay factor gamma = 2^(g log2 e), 1 for padding tokens
            float ga[C::TPL], gb[C::TPL];
#pragma unroll
            for (int t = 0; t < C::TPL; ++t) {
                const bool ok = tok0 + t < nv;
                const float xa = __builtin_amdgcn_exp2f(GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][0])));
                const float xb = __builtin_amdgcn_exp2f(GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][1])));
                ga[t] = ok ? xa : 1.0f;
                gb[t] = ok ? xb : 1.0f;
            }
            // in-lane inclusive prefix products and the lane's total
            float Pa[C::TPL], Pb[C::TPL];
#pragma unroll
            for (int t = 0; t < C::TPL; ++t) {
                Pa[t] = t ? Pa[t - 1] * ga[t] : ga[t];
                Pb[t] = t ? Pb[t - 1] * gb[t] : gb[t];
            }
            // across the NTG token groups of the pair (lanes p + PPH*tg): inclusive
            // prefix (ia) and suffix (sa) products of the group totals
            float ia = Pa[C::TPL - 1], ib = Pb[C::TPL - 1], sa = ia, sb = ib;
#pragma unroll
            for (int d = 1; d < C::NTG; d <<= 1) {
                const float ua = __shfl_up(ia, d * C::PPH), ub = __shfl_up(ib, d * C::PPH);
                const float wa = __shfl_down(sa, d * C::PPH), wb = __shfl_down(sb, d * C::PPH);
                if (tg >= d) { ia *= ua; ib *= ub; }
                if (tg + d < C::NTG) { sa *= wa; sb *= wb; }
            }
            // exclusive prefix (groups before) and suffix (groups after) of this lane's group
            float ea = __shfl_up(ia, C::PPH), eb = __shfl_up(ib, C::PPH);
            float fa = __shfl_down(sa, C::PPH), fb = __shfl_down(sb, C::PPH);
            if (tg == 0) { ea = 1.0f; eb = 1.0f; }
            if (tg == C::NTG - 1) { fa = 1.0f; fb = 1.0f; }
            // Gamma_C, taken from the first group so that every lane of the pair uses the same value
            const float gCa = __shfl(sa, p), gCb = __shfl(sb, p);
            // 1 / Gamma_C <= e^80: the bound keeps it finite in fp32
            const float iCa = __builtin_amdgcn_rcpf(gCa), iCb = __builtin_amdgcn_rcpf(gCb);

            bf16 kea[C::TPL], keb[C::TPL], va[C::TPL], vb[C::TPL];
            float Qa = fa, Qb = fb;   // product of gamma over the chunk's tokens after t
#pragma unroll
            for (int t = C::TPL - 1; t >= 0; --t) {
                const int pos = tok0 + t;
                const float Ga = ea * Pa[t], Gb = eb * Pb[t];                    // Gamma_t
                const float ka = (float)kr[t][0], kb = (float)kr[t][1];          // zero for padding tokens
                const float xa = ka * Qa, xb = kb * Qb;                          // Kend, |Kend| <= |k|
                store_pair(&sl.kn_row[pos * C::LDR + ch], -ka * Ga, -kb * Gb);
                store_pair(&sl.qp_row[pos * C::LDR + ch], (float)qr[t][0] * Ga, (float)qr[t][1] * Gb);
                store_pair(&km[pos * C::LDR + ch], xa * iCa, xb * iCb);          // K- = Kend / Gamma_C
                kea[t] = (bf16)xa;
                keb[t] = (bf16)xb;
                va[t] = vr[t][0];
                vb[t] = vr[t][1];
                Qa *= ga[t];
                Qb *= gb[t];
            }
            out_store_run<C::TPL>(&sl.ke_col[ch * C::LDK + tok0], kea);
            out_store_run<C::TPL>(&sl.ke_col[(ch + 1) * C::LDK + tok0], keb);
            out_store_run<C::TPL>(&sl.v_col[ch * C::LDK + tok0], va);
            out_store_run<C::TPL>(&sl.v_col[(ch + 1) * C::LDK + tok0], vb);
            if (tg == 0) *reinterpret_cast<f32x2*>(&sl.gc[ch]) = f32x2{gCa, gCb};
            // both producers of the chunk write the same T'
            *reinterpret_cast<bf16x4*>(&sl.t_row[r * C::LDK + 4 * g]) = cur.tl;
            load(m + 2 * C::NPW, cur);   // the chunk two steps on
            wave_lds_sync();

            // ---- this half's part of A_qk = LowerIncl(Q+ K-^T); lane (g, r) holds
            // the contraction over channels [hf*CH, hf*CH + CH) of A_qk[r][4g+i]
            const f32x4 a = MM::template mm_ll<C::CH>(km + hf * C::CH, C::LDR, sl.qp_row + hf * C::CH, C::LDR,
                                                      f32x4{0, 0, 0, 0}, r, g);
            f32x4 am;
#pragma unroll
            for (int i = 0; i < 4; ++i) am[i] = (4 * g + i <= r) ? a[i] : 0.0f;   // mask by select
            out_store4(&sl.aqk[hf][r * C::LDK + 4 * g], am);
            // GATE: z of this producer's previous chunk, whose o is stored at the
            // start of the next step (issued last, where it adds the fewest live
            // registers; the prefetch it queues behind is needed right after that
            // store anyway)
            if constexpr (GATE) load_z(m - C::NPW, m - C::NPW >= c0);
        };

        load(c0 + pp, pa);
        load(c0 + C::NPW + pp, pb);
        // Retire the first two steps' loads before the loop: the compiler's
        // wait-counter analysis would otherwise merge them with the loop's own
        // prefetch and wait for everything at the top of every step.
        __builtin_amdgcn_s_waitcnt(0);
        // step s uses register set pa when s is even, pb when odd
        auto step = [&](int s, Pref& cur) {
            Slot& sl = sm.slot[(s & 1) * C::NPW + pp];
            // the slot's previous chunk (step s - 2) was consumed in the last step
            store_o(c0 + (s - 2) * C::NPW + pp, sl, s >= 2);
            produce(c0 + s * C::NPW + pp, sl, cur);
            lds_barrier();
        };
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            step(s, pa);
            step(s + 1, pb);
        }
        if (s < nsteps) step(s, pa);
        lds_barrier();   // the consumers' last step
        // the o tiles of the last two steps
        store_o(c0 + (nsteps - 2) * C::NPW + pp, sm.slot[(nsteps & 1) * C::NPW + pp], nsteps >= 2);
        if constexpr (GATE) load_z(c0 + (nsteps - 1) * C::NPW + pp, true);
        store_o(c0 + (nsteps - 1) * C::NPW + pp, sm.slot[((nsteps - 1) & 1) * C::NPW + pp], true);
    } else {
        // =================================================================== consumer
        // state tiles S[jj][t]: rows 16t.., columns 16*(wave + NCW*jj).., from the
        // segment's start state
        f32x4 S[C::TPW][C::KT];
        const float* src = ws_start + ((int64_t)seg * smul * BH + bh) * D * D;
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NCW * jj;
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[jj][t][i] = src[(16 * t + 4 * g + i) * D + 16 * jt + r];
        }

        auto chain = [&](Slot& sl) {
            // Y = V - K+ S and O1^T = S^T Q+^T, from the chunk's start state
            f32x4 y[C::TPW], o1[C::TPW];
            BFrag sb[C::TPW * C::KT];
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const int jt = wave + C::NCW * jj;
#pragma unroll
                for (int t = 0; t < C::KT; ++t) sb[jj * C::KT + t] = MM::to_b(S[jj][t]);
                const bf16x4 vq = ld_b4(&sl.v_col[(16 * jt + r) * C::LDK + 4 * g]);
                y[jj] = f32x4{(float)vq[0], (float)vq[1], (float)vq[2], (float)vq[3]};
                o1[jj] = f32x4{0, 0, 0, 0};
            }
            MM::template mm_la_n<D, C::TPW>(sl.kn_row, C::LDR, sb, y, C::TPW, r, g);
            MM::template mm_al_n<D, C::TPW>(sb, sl.qp_row, C::LDR, o1, C::TPW, r, g);
            // U = T' Y
            const PFrag tf = out_ldk16(&sl.t_row[r * C::LDK + 4 * g]);
            PFrag up[C::TPW];
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) up[jj] = MM::to_p(MM::mm16(tf, MM::to_p(y[jj]), f32x4{0, 0, 0, 0}));
            // O^T = O1^T + U^T A_qk^T over both channel halves: lane (g, r) holds
            // o[token r][16jt + 4g + i], staged for the producers
            const PFrag qf0 = out_ldk16(&sl.aqk[0][r * C::LDK + 4 * g]);
            const PFrag qf1 = out_ldk16(&sl.aqk[1][r * C::LDK + 4 * g]);
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const int jt = wave + C::NCW * jj;
                const f32x4 ot = MM::mm16(up[jj], qf1, MM::mm16(up[jj], qf0, o1[jj]));
                out_store4(&sl.o_st[r * (D + 4) + 16 * jt + 4 * g], ot);
            }
            // S <- Diag(Gamma_C) S + Kend^T U
#pragma unroll
            for (int t = 0; t < C::KT; ++t) {
                const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sl.gc[16 * t + 4 * g]);
                const PFrag kf = out_ldk16(&sl.ke_col[(16 * t + r) * C::LDK + 4 * g]);
#pragma unroll
                for (int jj = 0; jj < C::TPW; ++jj) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[jj][t][i] *= gcv[i];
                    S[jj][t] = MM::mm16(kf, up[jj], S[jj][t]);
                }
            }
        };

        for (int s = 0; s <= nsteps; ++s) {
            if (s > 0) {
                // unrolled: a loop back-edge between two chunks would separate the
                // state products of one from the reads of the next
#pragma unroll
                for (int pp = 0; pp < C::NPW; ++pp) chain(sm.slot[((s - 1) & 1) * C::NPW + pp]);
            }
            lds_barrier();
        }

        if (seg == nseg - 1 && S_T) {
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const int jt = wave + C::NCW * jj;
#pragma unroll
                for (int t = 0; t < C::KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S_T[((int64_t)bh * D + 16 * t + 4 * g + i) * D + 16 * jt + r] = S[jj][t][i];
            }
        }
    }
}

template <int D>
static hipError_t launch_out_t(int B, int H, int T, const SegPlan& p, const void* q, const void* k,
                               const void* v, const float* theta, const void* ws_t, const float* ws_start,
                               const void* z, void* o, float* S_T, hipStream_t stream) {
    typedef OutCfg<D> C;
    const int BH = B * H;
    // One workgroup per compute unit: when the map segments give more workgroups
    // than the chip holds at once, pairs of consecutive segments are merged, so
    // that the whole grid (every head) is resident in one round.
    const int smul = (BH * p.nseg > 256 && p.nseg % 2 == 0) ? 2 : 1;
    const int nseg_o = p.nseg / smul, seg_len_o = p.seg_len * smul;
#define KDA_OUTK(GATE_)                                                                                     \
    hipLaunchKernelGGL((out_kernel<D, GATE_>), dim3((unsigned)(BH * nseg_o)), dim3(64 * C::NW), 0, stream, \
                       T, H, BH, p.nchunks, seg_len_o, nseg_o, smul, (const bf16*)q, (const bf16*)k,       \
                       (const bf16*)v, theta, (const bf16*)ws_t, ws_start, (const bf16*)z, (bf16*)o, S_T)
    if (z) KDA_OUTK(true);
    else KDA_OUTK(false);
#undef KDA_OUTK
    return hipGetLastError();
}

bool chunk_out_supported(int d) { return d == 32 || d == 64 || d == 128; }

hipError_t launch_chunk_out(int B, int T, int H, int d, const SegPlan& plan, const void* q, const void* k,
                            const void* v, const float* theta, const void* ws_t, const float* ws_start,
                            const void* z, void* o, float* S_T, hipStream_t stream) {
#define KDA_OUTD(D) return launch_out_t<D>(B, H, T, plan, q, k, v, theta, ws_t, ws_start, z, o, S_T, stream)
    switch (d) {
        case 32: KDA_OUTD(32);
        case 64: KDA_OUTD(64);
        case 128: KDA_OUTD(128);
    }
#undef KDA_OUTD
    return hipErrorInvalidValue;
}

}  // namespace kda

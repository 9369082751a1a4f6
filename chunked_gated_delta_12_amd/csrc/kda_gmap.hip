// kda_gmap.hip -- gradient segment maps of the bf16 backward pass on gfx950.
//
// The carried gradient of the backward pass (kda_bwd2.hip) runs through a
// chunk, in reverse, as
//     dU = A_qk^T dO + Kend dS',   -dY = -T'^T dU,
//     dS = Diag(Gamma_C) dS' + Q+^T dO + K+^T (-dY)
// (T' = (I + A)^-1 diag(beta) as the forward pass's map kernel publishes it;
// "Kimi K3 Deep Dive...", "The Problem: The Diagonal-Block Dilemma" for the chunk
// form, the bounded gate of "Architecture Deep Dive: Kimi K3...", section 3.2).
// It does not involve the forward state, and it is affine in dS', so a segment
// maps the gradient at its end to the gradient at its start,
//     dS_start = M dS_end + N.
// This kernel runs the chain over each segment but the first with the gradient
// widened to [N | M] (d x 2d), started from [0 | I], and stores the end value in
// reverse segment order (N fp32, M bf16, [map][batch*head][d][d]), so that the
// combine kernel chains the gradients forward.
//
// Wavefront roles as in the map kernel (kda_map.hip): NPW producer wavefronts
// form one chunk each per step -- the gate, K+^T, Q+^T and dO^T columns, Kend
// rows, Gamma_C, A_qk = LowerIncl(Q+ K-^T) and -T'^T -- into double-buffered
// LDS slots, and the consumer wavefronts hold the widened gradient's 16-column
// tiles in accumulator registers and run only the chain above, over the chunks
// the producers finished in the previous step, one barrier per step.  The
// producers walk their segment from its last chunk to its first.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
struct GmapCfg {
    static constexpr int NT = D / 8;                 // 16-column tiles of [N | M]
    static constexpr int NCW = NT < 8 ? NT : 8;      // consumer wavefronts
    static constexpr int TPW = NT / NCW;             // tiles per consumer
    static constexpr int NPW = 3;                    // producer wavefronts = chunks per step
    static constexpr int NW = NCW + NPW;
    static constexpr int KT = D / 16;                // 16-row tiles along d
    static constexpr int LDR = D + 4;                // [16][D] rows (no bank conflict on operand reads)
    static constexpr int LDK = 20;                   // [.][16] rows
    static constexpr int PPL = D / 2 < 64 ? D / 2 : 64;   // channel pairs of a producer
    static constexpr int NTG = 64 / PPL;             // token groups (lanes per pair)
    static constexpr int TPL = CHUNK / NTG;          // tokens per producer lane
    static_assert(NT % NCW == 0 && PPL * 2 == D && TPL % 4 == 0, "lane mappings");
};

// What the consumers read for one chunk.
template <int D>
struct GmapSlot {
    typedef GmapCfg<D> C;
    alignas(16) bf16 ke_row[16 * C::LDR];   // Kend = K*Gamma_C/Gamma     [token][ch]
    alignas(16) bf16 kp_col[D * C::LDK];    // K+^T                       [ch][token]
    alignas(16) bf16 qp_col[D * C::LDK];    // Q+^T                       [ch][token]
    alignas(16) bf16 do_col[D * C::LDK];    // dO^T                       [column][token]
    alignas(16) bf16 nt_row[16 * C::LDK];   // -T'^T                      [row][k]
    alignas(16) bf16 aq_row[16 * C::LDK];   // A_qk^T                     [t][s]
    alignas(16) float gc[D];                // Gamma_C per channel
};
// Private to one producer wavefront: the rows of A_qk's product.
template <int D>
struct GmapScratch {
    alignas(16) bf16 qp_row[16 * GmapCfg<D>::LDR];   // Q+ = Q*Gamma   [token][ch]
    alignas(16) bf16 km_row[16 * GmapCfg<D>::LDR];   // K- = K/Gamma   [token][ch]
};
template <int D>
struct GmapSmem {
    GmapSlot<D> slot[2 * GmapCfg<D>::NPW];
    GmapScratch<D> scr[GmapCfg<D>::NPW];
};

// The LDS side of a K = 16 product read as a whole 16x16x32 operand: the upper
// four k-slots take the next four stored elements (finite: data, or row padding
// zeroed at the start), which meet zero slots of the register side.
__device__ __forceinline__ bf16x8 gm_ldk16(const bf16* p) { return cat8(ld_b4(p), ld_b4(p + 4)); }

template <int D>
__global__ void __launch_bounds__(64 * GmapCfg<D>::NW)
gmap_kernel(int T, int H, int BH, int nchunks, int seg_len, int nseg, const bf16* __restrict__ q,
            const bf16* __restrict__ k, const float* __restrict__ theta, const bf16* __restrict__ dout,
            const bf16* __restrict__ ws_t, float* __restrict__ maps) {
    typedef GmapCfg<D> C;
    typedef GmapSlot<D> Slot;
    typedef Ops<bf16> MM;
    __shared__ GmapSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    // segment-major numbering, as in the map kernel
    const int bh = blockIdx.x % BH, seg = blockIdx.x / BH;
    if (seg == 0) return;   // the first segment's map is never used (whole workgroup, before any barrier)
    const int b = bh / H, h = bh % H;
    const int c0 = seg * seg_len;
    const int c1 = min(nchunks, c0 + seg_len);
    const int nsteps = (c1 - c0 + C::NPW - 1) / C::NPW;
    const int tend = min(T, c1 * CHUNK);
    // the chunk a producer handles at step s, from the segment's last chunk down
    // (below c0: all padding)
    auto chunk_of = [&](int s, int pp) { return c1 - 1 - (s * C::NPW + pp); };

    // zero the padding columns 16 .. LDK-1 of the [.][16] tiles read by gm_ldk16
    for (int i = tid; i < 2 * C::NPW * (D + 16); i += 64 * C::NW) {
        Slot& sl = sm.slot[i / (D + 16)];
        const int row = i % (D + 16);
        bf16* pad = row < D ? &sl.kp_col[row * C::LDK + 16] : &sl.nt_row[(row - D) * C::LDK + 16];
#pragma unroll
        for (int j = 0; j < C::LDK - 16; ++j) pad[j] = (bf16)0.0f;
    }

    if (wave >= C::NCW) {
        // =================================================================== producer
        const int pw = wave - C::NCW;
        __builtin_amdgcn_s_setprio(3);
        GmapScratch<D>& scr = sm.scr[pw];
        const int p = lane % C::PPL, tg = lane / C::PPL;
        const int ch = 2 * p, tok0 = tg * C::TPL;
        const uint32_t tstr = (uint32_t)(H * D);
        const int64_t head_base = (int64_t)b * T * H * D + (int64_t)h * D;

        // Inputs of one chunk, loaded a step ahead: resources cover the chunk's tokens
        // inside the sequence (none below the segment), so padding reads zero.
        f32x2 th[C::TPL];
        bf16x2 kr[C::TPL], qr[C::TPL], dr[C::TPL];
        bf16x4 tl;   // T'[r][4g .. 4g+3]
        auto load = [&](int m) {
            const bool in = m >= c0;
            const int t0 = (in ? m : c0) * CHUNK;
            const uint32_t nv = __builtin_amdgcn_readfirstlane(in ? max(0, min(CHUNK, tend - t0)) : 0);
            const int64_t base = head_base + (int64_t)t0 * tstr;
            const uint32_t span = nv * tstr;
            const Rsrc rth = make_rsrc(theta + base, span * 4u);
            const Rsrc rk = make_rsrc(k + base, span * 2u);
            const Rsrc rq = make_rsrc(q + base, span * 2u);
            const Rsrc rd = make_rsrc(dout + base, span * 2u);
#pragma unroll
            for (int t = 0; t < C::TPL; ++t) {
                const uint32_t el = (uint32_t)(tok0 + t) * tstr + (uint32_t)ch;
                th[t] = buf_ld_f2(rth, el * 4u, 0u);
                kr[t] = BufPair<bf16>::ld(rk, el * 2u, 0u);
                qr[t] = BufPair<bf16>::ld(rq, el * 2u, 0u);
                dr[t] = BufPair<bf16>::ld(rd, el * 2u, 0u);
            }
            const Rsrc rt = make_rsrc(ws_t + ((int64_t)bh * nchunks + (in ? m : c0)) * 256, in ? 512u : 0u);
            tl = BufQuad<bf16>::ld(rt, (uint32_t)(r * 16 + 4 * g) * 2u, 0u);
        };

        constexpr float LOG2E = 1.4426950408889634f;
        constexpr float GMIN2 = G_MIN * LOG2E;

        auto produce = [&](int m, Slot& sl) {
            const int nv = m >= c0 ? max(0, min(CHUNK, tend - m * CHUNK)) : 0;
            // K+^T, Q+^T and dO^T column elements of tokens tok0 + 4u .. +3, stored as soon as
            // a unit of four is complete (few live registers)
            bf16x4 kpa, kpb, qpa, qpb, da, db;
            auto put = [&](int t, float kxa, float kxb, float qxa, float qxb) {
                const int e = t & 3;
                kpa[e] = (bf16)kxa;
                kpb[e] = (bf16)kxb;
                qpa[e] = (bf16)qxa;
                qpb[e] = (bf16)qxb;
                da[e] = dr[t][0];
                db[e] = dr[t][1];
                if (e == 3) {
                    const int c = tok0 + t - 3;
                    *reinterpret_cast<bf16x4*>(&sl.kp_col[ch * C::LDK + c]) = kpa;
                    *reinterpret_cast<bf16x4*>(&sl.kp_col[(ch + 1) * C::LDK + c]) = kpb;
                    *reinterpret_cast<bf16x4*>(&sl.qp_col[ch * C::LDK + c]) = qpa;
                    *reinterpret_cast<bf16x4*>(&sl.qp_col[(ch + 1) * C::LDK + c]) = qpb;
                    *reinterpret_cast<bf16x4*>(&sl.do_col[ch * C::LDK + c]) = da;
                    *reinterpret_cast<bf16x4*>(&sl.do_col[(ch + 1) * C::LDK + c]) = db;
                }
            };
            float eCa, eCb;
            if constexpr (C::NTG == 1) {
                // all 16 tokens of the channel pair in the lane: the decay as products
                float gma[C::TPL], gmb[C::TPL];
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    gma[t] = __builtin_amdgcn_exp2f(GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][0])));
                    gmb[t] = __builtin_amdgcn_exp2f(GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][1])));
                }
                if (nv < CHUNK) {   // padding tokens do not decay
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
                    const float ka = (float)kr[t][0], kb = (float)kr[t][1];
                    const float qa = (float)qr[t][0], qb = (float)qr[t][1];
                    put(t, ka * Pa, kb * Pb, qa * Pa, qb * Pb);
                    store_pair(&scr.qp_row[t * C::LDR + ch], qa * Pa, qb * Pb);
                }
                eCa = Pa;
                eCb = Pb;
                const float ia = __builtin_amdgcn_rcpf(eCa), ib = __builtin_amdgcn_rcpf(eCb);
                float Qa = 1.0f, Qb = 1.0f;   // product of gamma over the tokens after t
#pragma unroll
                for (int t = C::TPL - 1; t >= 0; --t) {
                    const float ka = (float)kr[t][0], kb = (float)kr[t][1];
                    const float xa = ka * Qa, xb = kb * Qb;   // Kend
                    store_pair(&sl.ke_row[t * C::LDR + ch], xa, xb);
                    store_pair(&scr.km_row[t * C::LDR + ch], xa * ia, xb * ib);   // K- = Kend / Gamma_C
                    Qa *= gma[t];
                    Qb *= gmb[t];
                }
            } else {
                // log-decay in base 2 (zero for padding tokens), its prefix in the lane and
                // across the token groups of the pair
                float Ga[C::TPL], Gb[C::TPL];
                float sa = 0.0f, sb = 0.0f;
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    const float ga = GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][0]));
                    const float gb = GMIN2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th[t][1]));
                    const bool ok = tok0 + t < nv;
                    sa += ok ? ga : 0.0f;
                    sb += ok ? gb : 0.0f;
                    Ga[t] = sa;
                    Gb[t] = sb;
                }
                float ia = sa, ib = sb;
#pragma unroll
                for (int d = 1; d < C::NTG; d <<= 1) {
                    const float ua = __shfl_up(ia, d * C::PPL), ub = __shfl_up(ib, d * C::PPL);
                    if (tg >= d) { ia += ua; ib += ub; }
                }
                const float offa = ia - sa, offb = ib - sb;
                const float tota = __shfl(ia, (C::NTG - 1) * C::PPL + p), totb = __shfl(ib, (C::NTG - 1) * C::PPL + p);
                eCa = __builtin_amdgcn_exp2f(tota);
                eCb = __builtin_amdgcn_exp2f(totb);
#pragma unroll
                for (int t = 0; t < C::TPL; ++t) {
                    const int pos = tok0 + t;
                    const float xa = Ga[t] + offa, xb = Gb[t] + offb;
                    const float eGa = __builtin_amdgcn_exp2f(xa), eGb = __builtin_amdgcn_exp2f(xb);
                    const float emGa = __builtin_amdgcn_exp2f(-xa), emGb = __builtin_amdgcn_exp2f(-xb);
                    const float ka = (float)kr[t][0], kb = (float)kr[t][1];
                    const float qa = (float)qr[t][0], qb = (float)qr[t][1];
                    const float kma = ka * emGa, kmb = kb * emGb;
                    put(t, ka * eGa, kb * eGb, qa * eGa, qb * eGb);
                    store_pair(&scr.qp_row[pos * C::LDR + ch], qa * eGa, qb * eGb);
                    store_pair(&scr.km_row[pos * C::LDR + ch], kma, kmb);
                    store_pair(&sl.ke_row[pos * C::LDR + ch], kma * eCa, kmb * eCb);   // Kend <= |k|
                }
            }
            *reinterpret_cast<f32x2*>(&sl.gc[ch]) = f32x2{eCa, eCb};   // token groups write equal values
            // -T'^T: lane (g, r) holds T'[r][4g .. 4g+3]
#pragma unroll
            for (int i = 0; i < 4; ++i) sl.nt_row[(4 * g + i) * C::LDK + r] = (bf16)(-(float)tl[i]);
            load(m - C::NPW);   // in flight while A_qk is formed
            wave_lds_sync();
            // A_qk = LowerIncl(Q+ K-^T): lane (g, r) holds A_qk[4g + i][r] = A_qk^T[r][4g + i]
            const f32x4 a = MM::template mm_ll<D>(scr.qp_row, C::LDR, scr.km_row, C::LDR, f32x4{0, 0, 0, 0}, r, g);
            *reinterpret_cast<bf16x4*>(&sl.aq_row[r * C::LDK + 4 * g]) =
                bf16x4{(bf16)(r <= 4 * g ? a[0] : 0.0f), (bf16)(r <= 4 * g + 1 ? a[1] : 0.0f),
                       (bf16)(r <= 4 * g + 2 ? a[2] : 0.0f), (bf16)(r <= 4 * g + 3 ? a[3] : 0.0f)};
        };

        load(chunk_of(0, pw));
        __builtin_amdgcn_s_waitcnt(0);   // retire the first loads before the loop
        for (int s = 0; s < nsteps; ++s) {
            produce(chunk_of(s, pw), sm.slot[(s & 1) * C::NPW + pw]);
            lds_barrier();
        }
        lds_barrier();   // the consumers' last step
    } else {
        // =================================================================== consumer
        // gradient tiles X[jj][t]: rows 16t.., columns 16*(wave + NCW*jj).. of [N | M],
        // from [0 | I]
        f32x4 X[C::TPW][C::KT];
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NCW * jj;
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    X[jj][t][i] = (jt >= D / 16 && jt - D / 16 == t && 4 * g + i == r) ? 1.0f : 0.0f;
        }

        auto chain = [&](const Slot& sl) {
            // dU = A_qk^T dO (N part only) + Kend dS'
            f32x4 du[C::TPW];
            bf16x4 xb[C::TPW * C::KT];
            bf16x4 dof[C::TPW];
            const bf16x4 aqf = ld_b4(&sl.aq_row[r * C::LDK + 4 * g]);
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) {
                const int jt = wave + C::NCW * jj;
#pragma unroll
                for (int t = 0; t < C::KT; ++t) xb[jj * C::KT + t] = MM::to_b(X[jj][t]);
                du[jj] = f32x4{0, 0, 0, 0};
                if (jt < D / 16) {   // dO[4g .. 4g+3][16jt + r]
                    dof[jj] = ld_b4(&sl.do_col[(16 * jt + r) * C::LDK + 4 * g]);
                    du[jj] = mfma_k16(aqf, dof[jj], du[jj]);
                }
            }
            MM::template mm_la_n<D, C::TPW>(sl.ke_row, C::LDR, xb, du, C::TPW, r, g);
            // -dY = -T'^T dU
            const bf16x8 tf = gm_ldk16(&sl.nt_row[r * C::LDK + 4 * g]);
            bf16x4 nd[C::TPW];
#pragma unroll
            for (int jj = 0; jj < C::TPW; ++jj) nd[jj] = MM::to_b(mfma_k32(tf, MM::to_p(du[jj]), f32x4{0, 0, 0, 0}));
            // dS' <- Diag(Gamma_C) dS' + K+^T (-dY) + Q+^T dO (N part only)
#pragma unroll
            for (int t = 0; t < C::KT; ++t) {
                const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sl.gc[16 * t + 4 * g]);
                const bf16* kp = &sl.kp_col[(16 * t + r) * C::LDK + 4 * g];
                const bf16x8 kf = gm_ldk16(kp);
#pragma unroll
                for (int jj = 0; jj < C::TPW; ++jj) {
                    const int jt = wave + C::NCW * jj;
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[jj][t][i] *= gcv[i];
                    if (jt < D / 16) {
                        const bf16x8 aop = cat8(ld_b4(kp), ld_b4(&sl.qp_col[(16 * t + r) * C::LDK + 4 * g]));
                        X[jj][t] = mfma_k32(aop, cat8(nd[jj], dof[jj]), X[jj][t]);
                    } else {
                        X[jj][t] = mfma_k32(kf, MM::pad(nd[jj]), X[jj][t]);
                    }
                }
            }
        };

        for (int s = 0; s <= nsteps; ++s) {
            if (s > 0) {
#pragma unroll
                for (int pp = 0; pp < C::NPW; ++pp) chain(sm.slot[((s - 1) & 1) * C::NPW + pp]);
            }
            lds_barrier();
        }

        // [N | M] in reverse segment order: N fp32, then (after the nseg N blocks) M bf16
        const int slot = nseg - 1 - seg;
#pragma unroll
        for (int jj = 0; jj < C::TPW; ++jj) {
            const int jt = wave + C::NCW * jj;
#pragma unroll
            for (int t = 0; t < C::KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * t + 4 * g + i;
                    const int64_t rb = (((int64_t)slot * BH + bh) * D + row) * D;
                    if (jt < D / 16) maps[rb + 16 * jt + r] = X[jj][t][i];
                    else reinterpret_cast<bf16*>(maps + (int64_t)nseg * BH * D * D)[rb + 16 * (jt - D / 16) + r] =
                             (bf16)X[jj][t][i];
                }
        }
    }
}

hipError_t launch_grad_map(int B, int T, int H, int d, const SegPlan& p, const void* q, const void* k,
                           const float* theta, const void* dout, const void* ws_t, float* maps,
                           hipStream_t stream) {
    const int BH = B * H;
#define KDA_GMAP(D)                                                                                     \
    hipLaunchKernelGGL((gmap_kernel<D>), dim3((unsigned)(BH * p.nseg)), dim3(64 * GmapCfg<D>::NW), 0, stream, \
                       T, H, BH, p.nchunks, p.seg_len, p.nseg, (const bf16*)q, (const bf16*)k, theta,        \
                       (const bf16*)dout, (const bf16*)ws_t, maps);                                          \
    return hipGetLastError()
    switch (d) {
        case 64: KDA_GMAP(64);
        case 128: KDA_GMAP(128);
    }
#undef KDA_GMAP
    return hipErrorInvalidValue;
}

}  // namespace kda

// kda_bwd2.hip -- backward pass of the chunked KDA prefill for bf16 inputs at
// d = 64 and 128, on the bf16 matrix cores (16x16x32, fp32 accumulation).
//
// The chunk algebra is the one of kda_bwd.hip ("Kimi K3 Deep Dive...", "The
// Problem: The Diagonal-Block Dilemma" for the chunk form; the bounded gate of
// "Architecture Deep Dive: Kimi K3...", section 3.2).  Per chunk, with start
// state S, K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma, Kend = K*Gamma_C/Gamma,
// T = (I + StrictLower(diag(beta) K+ K-^T))^-1, Y = V - K+ S, U = T diag(beta) Y,
// A_qk = LowerIncl(Q+ K-^T), and the gradients dO of its outputs and dS' of its
// end state:
//     dU = A_qk^T dO + Kend dS',  Z = T^T dU,  dY = diag(beta) Z = dV
//     dS = Diag(Gamma_C) dS' + Q+^T dO - K+^T dY            (to the previous chunk)
//     dQ+ = dO S^T + dA_qk K-,   dK+ = diag(beta) (dA K- - Z S^T)
//     dK- = dA_qk^T Q+ + (diag(beta) dA)^T K+,   dKend = U dS'^T
//     dA_qk = LowerIncl(dO U^T),  dA = StrictLower(-Z U^T)
//     dbeta = rowsum(dA * K+ K-^T) + rowsum(Z * V) - rowsum(K+ * (Z S^T))
// (the last two terms are rowsum(Z * Y), with Y = V - K+ S expanded so that Y
// need not be kept), then the chain through the decay scalings to K, Q and the
// chunk-local cumulative log-decay as in kda_bwd.hip.
//
// Layout of the work.  The forward chain runs first, on the map kernel's
// producer and consumer wavefronts (kda_map.hip, SAVE mode), and writes for
// every chunk the operands this kernel reads: the start state in bf16 at every
// CKPT-th chunk of the segment (the checkpoints, counted from its first chunk),
// laid out as the operand fragments the row products load (16 bytes per lane,
// coalesced); U (by column tiles) and T^T (bf16) of every chunk; and, in the
// unused state area of every other chunk, the previous chunk's Kend (bf16) and
// Gamma_C (fp32).  So this kernel neither runs the state chain over whole
// segments nor solves the triangular system.
//
// Here one workgroup per (segment, batch, head) runs the backward sweep, D/16
// wavefronts; wavefront w owns state tile w: columns 16w.. of the carried
// gradient dS' in the column products (rows in accumulator registers), and
// channels 16w.. in the row products.  Products that contract over the state's
// columns (dO S^T, Z S^T, U dS'^T) take the saved state fragments and an LDS copy
// of dS' (bf16, row-major, every chunk).  The start state of chunk c + r (c a
// checkpoint, r < CKPT) is rebuilt from the checkpoint's by r steps of the chain,
//     S_{m+1} = Diag(Gamma_C) S_m + Kend^T U_m   (chunk m's operands),
// from the very bf16 operands the forward chain used; the checkpoint's state is
// loaded once per run of CKPT chunks and kept in LDS.  CKPT = 2 halves the state
// traffic of saving every chunk's (the largest item of the pass's) for one step
// per two chunks.  The steps sit on the sweep's critical path: with CKPT = 4 (six
// steps per four chunks) the sweep lost more time than the forward chain's
// fewer stores saved.
//
// For few long sequences the segments' start states and end gradients come from
// affine segment maps: the state maps from the forward pass's map kernel
// (kda_map.hip, which also publishes every chunk's T' = T diag(beta)), the
// gradient maps from kda_gmap.hip; the forward pass's combine kernel chains both
// (the gradient's in reverse segment order).
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
struct B2Cfg {
    static constexpr int NT = D / 16;        // 16-wide tiles along a state dimension
    static constexpr int NW = NT;            // wavefronts: one tile each
    static constexpr int NTHR = 64 * NW;
    static constexpr int KB = D / 32;        // 32-deep contraction blocks over D
    static constexpr int LDR = D + 4;        // bf16 row stride of [16][D] tiles
    static constexpr int LDK = 20;           // bf16 row stride of [.][16] tiles
    static constexpr int LS = 20;            // fp32 row stride of 16x16 tiles
    static constexpr int LRB = D + 8;        // bf16 row stride of the staged inputs
    static constexpr int LRF = D + 4;        // fp32 row stride of the staged theta
    // workspace of one chunk of one sequence (kda_launch.hpp): the start state as
    // row-product operand fragments (checkpoints), U by column tiles, and T^T
    // [16][16]; in the state area of every other chunk the previous chunk's Kend as
    // the operand fragments of a rebuild step ([wavefront][lane], 4 tokens of one
    // channel, 8 bytes), then its Gamma_C (fp32 per channel)
    typedef BwdChunkWs<D> W;
    static constexpr int64_t WS_S = W::WS_S, WS_U = W::WS_U, WSC = W::WSC;
    static constexpr int CKPT = W::CKPT;      // chunks per saved start state
    static constexpr int NRB = CKPT - 1;      // most rebuild steps of one chunk
    static constexpr uint32_t KE_BYTES = W::KE_BYTES, GC_OFF = W::GC_OFF;
    static_assert(KE_BYTES == (uint32_t)NW * 64u * 8u, "one 8-byte Kend fragment per lane");
    static_assert(KE_BYTES + 4 * D <= 2 * WS_S, "Kend and Gamma_C fit in a state area");
    static_assert(D == 64 || D == 128, "d = 64 or 128");
};

template <int D>
struct B2Smem {
    typedef B2Cfg<D> C;
    alignas(16) bf16 kp[16 * C::LDR];    // K+   [token][channel]
    alignas(16) bf16 km[16 * C::LDR];    // K-
    alignas(16) bf16 ke[16 * C::LDR];    // Kend
    alignas(16) bf16 kpT[D * C::LDK];    // K+^T [channel][token]
    alignas(16) bf16 kmT[D * C::LDK];    // K-^T
    alignas(16) bf16 U[16 * C::LDR];     // U [token][value column]
    struct {
        alignas(16) bf16 Xs[D * C::LDR];    // dS' of the chunk's end [channel][column]
    } u;
    struct {
        alignas(16) bf16 qp[16 * C::LDR];    // Q+
        alignas(16) bf16 qpT[D * C::LDK];    // Q+^T
        alignas(16) bf16 dO[16 * C::LDR];    // dO [token][column]
        alignas(16) bf16 Z[16 * C::LDR];     // Z = T^T dU [token][column]
    } b;
    alignas(16) bf16 stash[D * D];       // the checkpoint's start-state fragments [w][kb][lane]
    alignas(16) bf16 upT[C::NRB][D * C::LDK];   // U^T of the chunks a start state is rebuilt from [column][token]
    alignas(16) bf16 ttT[16 * C::LDK];   // T^T (BMAP: T'^T)
    alignas(16) float KK[16 * C::LS];    // K+ K-^T [t][s]
    // dA_qk and dA as the bf16 operand fragments of the chain rule's products, [lane][4]:
    // dA_qk^T, dA_qk, (diag(beta) dA)^T, dA
    alignas(16) bf16 fq[4][64 * 4];
    alignas(16) float dA[16 * C::LS];
    alignas(16) float gc[D];             // Gamma_C per channel
    float zv[C::NW][16];                 // rowsum(Z * V) over each wavefront's columns
    float kz[C::NW][16];                 // rowsum(K+ * (Z S^T)) over each wavefront's channels
    // the next chunk's inputs, staged row-major: one 16-byte read per thread and tensor
    // from memory; each lane then takes its channel of tokens 4g .. 4g+3, theta by 4-byte
    // reads (rows padded so that the four lane groups meet different banks) and the bf16
    // tensors by 8-byte row reads through the identity product
    struct {
        alignas(16) bf16 k[16 * C::LRB];
        alignas(16) bf16 q[16 * C::LRB];
        alignas(16) bf16 o[16 * C::LRB];   // dO
        alignas(16) bf16 v[16 * C::LRB];
        alignas(16) float th[16 * C::LRF];
        float bt[16];
    } in;
    // each wavefront's gradient block [token][its 16 channels] on its way to one 16-byte
    // store per lane (rows of 20: the four lane groups' writes meet different banks)
    alignas(16) float gst[C::NW][16 * 20];
};


__device__ __forceinline__ bf16x4 bq(f32x4 x) { return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]}; }
__device__ __forceinline__ bf16x4 bq4(float a, float b, float c, float d) {
    return bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
// one 4-byte value (dbeta of a token)
__device__ __forceinline__ void buf_st32(float x, Rsrc r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, (int)voff, (int)soff, 0);
}
typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
// CP = kCpStream for the checkpoint states: each lane's own 16 bytes, read once
template <int CP = 0>
__device__ __forceinline__ bf16x8 buf_ld_b8(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, CP));
}
__device__ __forceinline__ bf16x4 buf_ld_b4(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void buf_st_b4(bf16x4 x, Rsrc r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ void buf_st_b8(bf16x8 x, Rsrc r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)voff, (int)soff, 0);
}

// Sum over the 16 lanes of a row (lane & 15), in every lane of the row, by DPP
// lane swaps (xor 1, xor 2, half-row mirror, row mirror) on the vector unit.
__device__ __forceinline__ float rowsum16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}
typedef __bf16 bf16v2 __attribute__((ext_vector_type(2)));
// x . y over 8 bf16 pairs, accumulated in fp32 (packed bf16 dot products)
__device__ __forceinline__ float dot8(bf16x8 x, bf16x8 y, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf16v2{x[2 * i], x[2 * i + 1]}, bf16v2{y[2 * i], y[2 * i + 1]}, acc, false);
    return acc;
}

// 16x16 product P = A B^T over the D channels, A and B row-major [16][LDR] in
// LDS: lane (g, r) gets P[4g + i][r].  k-map: block kb, slot i of group g is
// channel 32kb + 4g + i, slot 4 + i channel 32kb + 16 + 4g + i.
template <int D>
__device__ __forceinline__ f32x4 small_abt(const bf16* A, const bf16* B, int r, int g) {
    constexpr int LDR = B2Cfg<D>::LDR;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < D / 32; ++kb) {
        const int o = r * LDR + 32 * kb + 4 * g;
        acc = mfma_k32(cat8(ld_b4(A + o), ld_b4(A + o + 16)), cat8(ld_b4(B + o), ld_b4(B + o + 16)), acc);
    }
    return acc;
}

template <int D>
__global__ void __launch_bounds__(B2Cfg<D>::NTHR)
bwd2_kernel(int T, int H, int BH, int nchunks, int seg_len, const bf16* __restrict__ q,
            const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ theta,
            const float* __restrict__ beta, const bf16* __restrict__ dout,
            const float* __restrict__ Xinit, float* __restrict__ dq, float* __restrict__ dk,
            float* __restrict__ dv, float* __restrict__ dtheta, float* __restrict__ dbeta,
            float* __restrict__ dS0, bf16* __restrict__ ws) {
    typedef B2Cfg<D> C;
    constexpr int NCX = 1;   // column tiles of dS' per wavefront
    constexpr int NT = C::NT, KB = C::KB, LDR = C::LDR, LDK = C::LDK, LS = C::LS;
    constexpr float LOG2E = 1.4426950408889634f;
    constexpr float GMIN2 = G_MIN * LOG2E;
    __shared__ B2Smem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Wavefronts w and w + NW/2 share a SIMD, and the older one wins its issue
    // arbitration: the younger half, left as the critical path of every phase, issues
    // at a raised priority instead.
    if (w >= C::NW / 2) __builtin_amdgcn_s_setprio(1);
    // Lane-derived indices.  The lane group g is re-derived at the top of every chunk
    // from an opaque copy of the lane id (relane), so that the address arithmetic built
    // on it is recomputed inside the loop instead of being hoisted out of it, which would
    // keep dozens of loop-invariant address registers alive (with g, li and ch all
    // hoisted the kernel needs 256 VGPRs and spills).  The addresses that depend on the
    // column li and channel ch alone stay hoisted: 220 VGPRs, no scratch.
    int g = lane >> 4;
    const int li = lane & 15;
    const int bh = blockIdx.x % BH, seg = blockIdx.x / BH, b = bh / H, h = bh % H;
    const int n_lo = seg * seg_len, n_hi = min(nchunks, n_lo + seg_len);
    const uint32_t tstr = (uint32_t)(H * D);                          // elements between tokens
    const int64_t hb = (int64_t)b * T * H * D + (int64_t)h * D;      // token 0 of this head
    const int64_t bb = (int64_t)b * T * H + h;                       // beta of token 0
    bf16* wsh = ws + (int64_t)bh * nchunks * C::WSC;
    const int ch = 16 * w + li;   // this lane's channel (gate, row products) and value column (column products)
    auto relane = [&]() {
        int lv = lane;
        asm volatile("" : "+v"(lv));
        g = lv >> 4;
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // Between the lanes' layout and row-major [16][D] tiles on the matrix cores.  A product
    // with the identity turns an A operand, lane (g, li) holding row li at k-slots
    // 4g .. 4g+3, into an accumulator, lane (g, r) holding rows 4g .. 4g+3 of column r.
    // So a 16x16 block formed in the lanes' layout (tokens 4g .. 4g+3 of column li) comes
    // back as row pieces (row r, columns 4g .. 4g+3: one 8-byte LDS write per lane), and
    // 8-byte row pieces read from a staged tile come back in the lanes' layout, in fp32.
    // Two blocks share one A operand, each product taking one of them through the
    // identity in its half of the k-slots (the other half of B is zero).  bf16 values
    // pass through exactly.  The matrix cores are idle most of the chunk, and a block
    // pair costs two 8-byte LDS accesses per lane instead of eight 2-byte ones.
    const bf16x4 eyeb = bq4(4 * g == li ? 1.0f : 0.0f, 4 * g + 1 == li ? 1.0f : 0.0f,
                            4 * g + 2 == li ? 1.0f : 0.0f, 4 * g + 3 == li ? 1.0f : 0.0f);
    const bf16x4 zb4 = bq4(0.0f, 0.0f, 0.0f, 0.0f);
    // blocks x0, x1 to columns 16w .. of the row-major tiles t0, t1 (rows of stride LDR)
    auto tr_rows = [&](bf16x4 x0, bf16* t0, bf16x4 x1, bf16* t1) {
        const bf16x8 a = cat8(x0, x1);
        const int o = li * LDR + 16 * w + 4 * g;
        *reinterpret_cast<bf16x4*>(&t0[o]) = bq(mfma_k32(a, cat8(eyeb, zb4), zero4));
        *reinterpret_cast<bf16x4*>(&t1[o]) = bq(mfma_k32(a, cat8(zb4, eyeb), zero4));
    };
    // the other way: columns 16w .. of the staged input tiles t0, t1 (rows of stride LRB),
    // lane (g, li) getting tokens 4g .. 4g+3 of channel 16w + li
    auto from_rows = [&](const bf16* t0, const bf16* t1, f32x4& x0, f32x4& x1) {
        const int o = li * C::LRB + 16 * w + 4 * g;
        const bf16x8 a = cat8(ld_b4(&t0[o]), ld_b4(&t1[o]));
        x0 = mfma_k32(a, cat8(eyeb, zb4), zero4);
        x1 = mfma_k32(a, cat8(zb4, eyeb), zero4);
    };

    // ------------------------------------------------------------ raw inputs of a chunk
    // The workgroup reads a chunk's k, q, dO, v and theta as 16-byte pieces, one per
    // thread and tensor (the first half of the wavefronts k and dO, the second q and v),
    // and beta by token; stage_raw puts them in LDS, from where lane (g, li) takes channel
    // ch of tokens 4g .. 4g+3.  Padding tokens read zero.
    struct Raw {
        u32x4 a, b, c;   // 16 bytes of k or q, of dO or v, of theta
        float bt;        // beta of token lane % 16
    };
    const bool hw = w >= C::NW / 2;                          // wave-uniform
    const int jb = (w % (C::NW / 2)) * 64 + lane;            // piece of a [16][D] bf16 tile
    // Unconditional: a chunk outside the segment (the one after the last, or before the
    // first) reads zeros through resources of size zero, so no load sits under a branch
    // (which would make the compiler wait for every outstanding access at the join).
    auto load_raw = [&](int m, Raw& r) {
        const int tm = m * CHUNK;
        const bool inside = m >= n_lo && m < n_hi;
        const uint32_t nv = __builtin_amdgcn_readfirstlane(inside ? max(0, min(CHUNK, T - tm)) : 0);
        const int64_t base = hb + (int64_t)tm * tstr;
        const uint32_t span = nv * tstr;
        const uint32_t pb = ((uint32_t)(jb / (D / 8)) * tstr + (uint32_t)(jb % (D / 8)) * 8u) * 2u;
        const uint32_t pt = ((uint32_t)(tid / (D / 4)) * tstr + (uint32_t)(tid % (D / 4)) * 4u) * 4u;
        const Rsrc ra = make_rsrc((hw ? q : k) + base, span * 2u);
        const Rsrc rv = make_rsrc((hw ? v : dout) + base, span * 2u);
        const Rsrc rth = make_rsrc(theta + base, span * 4u);
        const Rsrc rb = make_rsrc(beta + bb + (int64_t)tm * H, nv * (uint32_t)H * 4u);
        r.a = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)pb, 0, 0);
        r.b = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)pb, 0, 0);
        r.c = __builtin_amdgcn_raw_buffer_load_b128(rth, (int)pt, 0, 0);
        r.bt = __builtin_bit_cast(float, buf_ld32(rb, (uint32_t)(lane & 15) * (uint32_t)H * 4u, 0u));
    };
    // Every thread writes (beta: equal duplicates), so that no branch sits around the
    // registers of loads in flight.
    auto stage_raw = [&](const Raw& r) {
        const int eb = (jb / (D / 8)) * C::LRB + (jb % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(&(hw ? sm.in.q : sm.in.k)[eb]) = r.a;
        *reinterpret_cast<u32x4*>(&(hw ? sm.in.v : sm.in.o)[eb]) = r.b;
        *reinterpret_cast<u32x4*>(&sm.in.th[(tid / (D / 4)) * C::LRF + (tid % (D / 4)) * 4]) = r.c;
        sm.in.bt[lane & 15] = r.bt;
    };
    // A gradient of the chunk, x[i] of token 4g + i and channel ch, as one 16-byte store
    // per lane: lane l writes channels 16w + 4(l % 4) .. +3 of token l / 4.  A wavefront
    // fills half of each 128-byte line it touches; the default cache policy lets the two
    // halves merge before they are written back (the non-temporal hint wrote them apart:
    // 0.5 GB more per B = 32 call, for no measurable time).
    auto store_grad = [&](const float (&x)[4], Rsrc r) {
        float* gw = sm.gst[w];
#pragma unroll
        for (int i = 0; i < 4; ++i) gw[(4 * g + i) * 20 + li] = x[i];
        wave_lds_sync();
        const f32x4 y = *reinterpret_cast<const f32x4*>(&gw[(lane >> 2) * 20 + 4 * (lane & 3)]);
        wave_lds_sync();   // read before the next block's writes
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), r,
                                               (int)(((uint32_t)(lane >> 2) * tstr + (uint32_t)(16 * w + 4 * (lane & 3))) * 4u),
                                               0, 0);
    };

    // ------------------------------------------------------------ the gate of a chunk
    // Per lane: channel ch, tokens 4g+i.  The in-chunk prefix of the log-decay (base
    // 2) runs inside the lane and then over the four lane groups.
    struct Gate {
        float gam[4], igam[4], gC, dsg[4], kf[4], qf[4];
    };
    auto gate = [&](int nv, Gate& G, bool want_q) {
        float g2[4], sgv[4];
        {
            f32x4 kf, qf;
            from_rows(sm.in.k, sm.in.q, kf, qf);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                G.kf[i] = kf[i];
                G.qf[i] = want_q ? qf[i] : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float th = sm.in.th[(4 * g + i) * C::LRF + ch];
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-LOG2E * th));
            sgv[i] = sg;
            g2[i] = (4 * g + i < nv) ? GMIN2 * sg : 0.0f;   // padding tokens do not decay
        }
        float pre[4], run = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run += g2[i];
            pre[i] = run;
        }
        const float t0 = __shfl(run, li), t1 = __shfl(run, 16 + li), t2 = __shfl(run, 32 + li),
                    t3 = __shfl(run, 48 + li);
        const float off = (g > 0 ? t0 : 0.0f) + (g > 1 ? t1 : 0.0f) + (g > 2 ? t2 : 0.0f);
        G.gC = __builtin_amdgcn_exp2f(((t0 + t1) + t2) + t3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gm = __builtin_amdgcn_exp2f(off + pre[i]);
            G.gam[i] = gm;
            G.igam[i] = __builtin_amdgcn_rcpf(gm);   // <= e^80: the bound keeps it finite
            G.dsg[i] = G_MIN * sgv[i] * (1.0f - sgv[i]);
        }
    };

    // ------------------------------------------------------------ carried gradient
    // X = dS': tile rt holds rows 16rt + 4g + i of column 16w + li.  Its start value
    // (zero when init is NULL: a resource of size zero).
    const int nseg = (nchunks + seg_len - 1) / seg_len;
    auto init_state = [&](f32x4 (&Wt)[NT][NCX], const float* init, int64_t off) {
        const Rsrc ri = make_rsrc(init ? init + off : init, init ? (uint32_t)(D * D * 4) : 0u);
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Wt[rt][0][i] = __builtin_bit_cast(float, buf_ld32(ri, (uint32_t)((16 * rt + 4 * g + i) * D + ch) * 4u, 0u));
    };

    Raw raw = {};

    // ============================================================ backward sweep
    {
        f32x4 X[NT][NCX];                 // dS' by value-column tiles
        // the carried gradient at the segment's end: the combine wrote the segments'
        // end values in reverse order (one segment: dS_T itself)
        init_state(X, Xinit, ((int64_t)(nseg - 1 - seg) * BH + bh) * D * D);
        // chunk-saved operands, loaded a chunk ahead with the raw inputs
        bf16x8 sfn[KB];                   // start-state fragments of this lane's channel tile
        bf16x4 ufn = {};                  // U of tile w, tokens 4g.., column 16w + li
        bf16x4 tfn = {};                  // 4 elements of T^T
        // operands of the rebuild steps of the chunk's start state: step j goes from
        // chunk c + j to c + j + 1 (c the checkpoint) with chunk c + j's U (tile w, as
        // ufn), Kend (tokens 4g.., channel ch) and Gamma_C of channel ch
        bf16x4 ufp[C::NRB], kep[C::NRB];
        float gcp[C::NRB];
        // chunk m's saved operands (zeros through resources of size zero outside the
        // segment).  Chunk m = c + r (r < CKPT) needs r rebuild steps from the checkpoint
        // c.  The first chunk the sweep meets in a run c .. c + CKPT - 1 (its last one,
        // or the segment's last chunk) loads the checkpoint's state and keeps it in LDS
        // for the rest of the run; the others load no state.
        auto load_saved = [&](int m) {
            const bool inside = m >= n_lo && m < n_hi;
            const int mm = inside ? m : n_lo;   // an address inside the workspace either way
            const int r = (mm - n_lo) % C::CKPT;
            const bool top = inside && (m == n_hi - 1 || r == C::CKPT - 1);
            const bf16* wsm = wsh + (int64_t)mm * C::WSC;
            const bf16* wsc = wsm - (int64_t)r * C::WSC;   // the checkpoint chunk
            {
                const Rsrc rws = make_rsrc(wsc, top ? (uint32_t)C::WS_S * 2u : 0u);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    sfn[kb] = buf_ld_b8<kCpStream>(rws, (uint32_t)lane * 16u, (uint32_t)((w * KB + kb) * 64) * 16u);
                // U, stored by column tiles: [tile][lane (g, li)][tokens 4g .. 4g+3], 8 bytes per lane
                const Rsrc ru = make_rsrc(wsm + C::WS_S, inside ? (uint32_t)C::WS_U * 2u : 0u);
                ufn = buf_ld_b4(ru, (uint32_t)lane * 8u, (uint32_t)w * 512u);
#pragma unroll
                for (int j = 0; j < C::NRB; ++j) {
                    const bool on = inside && j < r;
                    // chunk c + j's U; its Kend and Gamma_C in chunk c + j + 1's state area
                    const bf16* wj = on ? wsc + (int64_t)j * C::WSC : wsc;
                    const Rsrc rup = make_rsrc(wj + C::WS_S, on ? (uint32_t)C::WS_U * 2u : 0u);
                    ufp[j] = buf_ld_b4(rup, (uint32_t)lane * 8u, (uint32_t)w * 512u);
                    const Rsrc rke = make_rsrc(on ? wj + C::WSC : wsc, on ? C::KE_BYTES + 4u * D : 0u);
                    kep[j] = buf_ld_b4(rke, (uint32_t)lane * 8u, (uint32_t)w * 512u);
                    gcp[j] = __builtin_bit_cast(float, buf_ld32(rke, (uint32_t)ch * 4u, C::GC_OFF));
                }
            }
            // T^T, saved by the forward chain: lane l loads row l/4, columns 4(l%4) .. +3;
            // every wavefront loads it and writes the same values
            const Rsrc rt = make_rsrc(wsm + C::WS_S + C::WS_U, inside ? 512u : 0u);
            tfn = buf_ld_b4(rt, (uint32_t)lane * 8u, 0u);
        };
        load_raw(n_hi - 1, raw);
        load_saved(n_hi - 1);
        __builtin_amdgcn_s_waitcnt(0);   // retire the first loads before the loop
        stage_raw(raw);
        lds_barrier();
        for (int n = n_hi - 1; n >= n_lo; --n) {
            relane();
            const int tc = n * CHUNK;
            const int nv = min(CHUNK, T - tc);
            Gate G;
            gate(nv, G, true);
            float of[4], vf[4], bt[4];
            {
                f32x4 o4, v4;
                from_rows(sm.in.o, sm.in.v, o4, v4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    of[i] = o4[i];
                    vf[i] = v4[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bt[i] = sm.in.bt[4 * g + i];
            }
            // tiles of the chunk (the saved rebuild operands and T^T first: their registers are
            // reloaded next; U goes with dO below)
            // (no branch around registers of pending loads: every thread writes, the
            // duplicates with equal values)
            {
                // U^T of the chunks of the rebuild steps (zeros for steps the chunk has not)
#pragma unroll
                for (int j = 0; j < C::NRB; ++j)
                    *reinterpret_cast<bf16x4*>(&sm.upT[j][ch * LDK + 4 * g]) = ufp[j];
            }
            *reinterpret_cast<bf16x4*>(&sm.ttT[(lane >> 2) * LDK + 4 * (lane & 3)]) = tfn;
            load_raw(n - 1, raw);   // in flight during this chunk
            // K+, K-, Q+ and Kend of this lane's channel and tokens (recomputed in the chain rule)
            auto kpv = [&](int i) { return G.kf[i] * G.gam[i]; };
            auto kmv = [&](int i) { return G.kf[i] * G.igam[i]; };
            auto qpv = [&](int i) { return G.qf[i] * G.gam[i]; };
            auto kev = [&](int i) { return G.kf[i] * (G.gC * G.igam[i]); };
            {
                const bf16x4 kpb = bq4(kpv(0), kpv(1), kpv(2), kpv(3));
                const bf16x4 kmb = bq4(kmv(0), kmv(1), kmv(2), kmv(3));
                const bf16x4 qpb = bq4(qpv(0), qpv(1), qpv(2), qpv(3));
                tr_rows(kpb, sm.kp, kmb, sm.km);
                tr_rows(bq4(kev(0), kev(1), kev(2), kev(3)), sm.ke, qpb, sm.b.qp);
                tr_rows(bq4(of[0], of[1], of[2], of[3]), sm.b.dO, ufn, sm.U);
                *reinterpret_cast<bf16x4*>(&sm.kpT[ch * LDK + 4 * g]) = kpb;
                *reinterpret_cast<bf16x4*>(&sm.kmT[ch * LDK + 4 * g]) = kmb;
                *reinterpret_cast<bf16x4*>(&sm.b.qpT[ch * LDK + 4 * g]) = qpb;
            }
            if (g == 0) sm.gc[ch] = G.gC;
            {   // dS' of the chunk's end, row-major, for the products over its columns
#pragma unroll
                for (int rt = 0; rt < NT; rt += 2)
                    tr_rows(bq(X[rt][0]), &sm.u.Xs[16 * rt * LDR], bq(X[rt + 1][0]), &sm.u.Xs[16 * (rt + 1) * LDR]);
            }
            lds_barrier();

            {
                // ---- the chunk's start state as row-product fragments: the checkpoint's
                // (loaded by the first chunk of its run to be met, kept in LDS for the rest),
                // then r steps S_{m+1} = Diag(Gamma_C) S_m + Kend^T U_m (chunk m's operands),
                // with the state transposed: tile jt of S^T holds value columns
                // 16jt + 4g + i of channel ch
                bf16* stw = &sm.stash[(w * KB * 64 + lane) * 8];   // this lane's fragments, block kb at +512 kb
                const int r = (n - n_lo) % C::CKPT;
                if (n == n_hi - 1 || r == C::CKPT - 1) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) *reinterpret_cast<bf16x8*>(stw + kb * 512) = sfn[kb];
                } else {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) sfn[kb] = *reinterpret_cast<const bf16x8*>(stw + kb * 512);
                }
#pragma unroll
                for (int j = 0; j < C::NRB; ++j) {
                    if (j < r) {
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            f32x4 hv[2];
#pragma unroll
                            for (int hh = 0; hh < 2; ++hh) {
                                f32x4 c;
#pragma unroll
                                for (int i = 0; i < 4; ++i) c[i] = gcp[j] * (float)sfn[kb][4 * hh + i];
                                hv[hh] = mfma_k16(ld_b4(&sm.upT[j][(16 * (2 * kb + hh) + li) * LDK + 4 * g]), kep[j], c);
                            }
                            sfn[kb] = cat8(bq(hv[0]), bq(hv[1]));
                        }
                    }
                }
            }

            // ---- A_qk = LowerIncl(Q+ K-^T), formed by every wavefront: lane (g, li) holds
            // A_qk[4g + i][li], which is its A_qk^T operand fragment (row li, k = 4g + i)
            bf16x4 aqT;
            {
                const f32x4 aq = small_abt<D>(sm.b.qp, sm.km, li, g);
                aqT = bq4(li <= 4 * g ? aq[0] : 0.0f, li <= 4 * g + 1 ? aq[1] : 0.0f,
                          li <= 4 * g + 2 ? aq[2] : 0.0f, li <= 4 * g + 3 ? aq[3] : 0.0f);
            }

            // ---- column products: dU, Z, dY = dV, and dS' <- Diag(Gamma_C) dS' + Q+^T dO - K+^T dY
            float zvp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cx = 0; cx < NCX; ++cx) {
                f32x4 du = zero4;
                // A_qk^T dO
                    du = mfma_k16(aqT, bq4(of[0], of[1], of[2], of[3]), du);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int o = li * LDR + 32 * kb + 4 * g;
                    du = mfma_k32(cat8(ld_b4(&sm.ke[o]), ld_b4(&sm.ke[o + 16])),
                                  cat8(bq(X[2 * kb][cx]), bq(X[2 * kb + 1][cx])), du);
                }
                // Z = T^T dU and -dY = -diag(beta) Z
                const f32x4 z = mfma_k16(ld_b4(&sm.ttT[li * LDK + 4 * g]), bq(du), zero4);
                f32x4 ndy;
#pragma unroll
                for (int i = 0; i < 4; ++i) ndy[i] = -bt[i] * z[i];
                {
                    const Rsrc rdv = make_rsrc(dv + hb + (int64_t)tc * tstr, (uint32_t)nv * tstr * 4u);
                    const float dvv[4] = {-ndy[0], -ndy[1], -ndy[2], -ndy[3]};
                    store_grad(dvv, rdv);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sm.b.Z[(4 * g + i) * LDR + ch] = (bf16)z[i];
                        zvp[i] = z[i] * vf[i];
                    }
                }
                const bf16x4 ob = bq4(of[0], of[1], of[2], of[3]);
                const bf16x8 bop = cat8(ob, bq(ndy));
#pragma unroll
                for (int rt = 0; rt < NT; ++rt) {
                    const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[16 * rt + 4 * g]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[rt][cx][i] *= gcv[i];
                    const int o = (16 * rt + li) * LDK + 4 * g;
                    X[rt][cx] = mfma_k32(cat8(ld_b4(&sm.b.qpT[o]), ld_b4(&sm.kpT[o])), bop, X[rt][cx]);
                }
            }
            // rowsum(Z * V) over this wavefront's 16 columns
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = rowsum16(zvp[i]);
                if (li == 0) sm.zv[w][4 * g + i] = s;
            }
            lds_barrier();

            // ---- dA_qk = LowerIncl(dO U^T) (wave 0), dA = StrictLower(-Z U^T) (wave 1),
            // KK = K+ K-^T (wave 2, for dbeta); everyone: the row products over the state's
            // columns, dO S^T, U dS'^T and Z S^T, and dGamma_C = rowsum(dS' * S).  Waves 0
            // and 1 leave dA_qk and dA as the bf16 fragments every wave's chain-rule products
            // load (lane (g, li) of the accumulator holds row 4g + i of column li, the
            // transposed operand; the operand itself comes through the identity product)
            if (w == 2) {
                const f32x4 kk = small_abt<D>(sm.kp, sm.km, li, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.KK[(4 * g + i) * LS + li] = kk[i];
            }
            if (w == 0) {
                const f32x4 x = small_abt<D>(sm.b.dO, sm.U, li, g);
                const bf16x4 xb = bq4(li <= 4 * g ? x[0] : 0.0f, li <= 4 * g + 1 ? x[1] : 0.0f,
                                      li <= 4 * g + 2 ? x[2] : 0.0f, li <= 4 * g + 3 ? x[3] : 0.0f);
                *reinterpret_cast<bf16x4*>(&sm.fq[0][(16 * g + li) * 4]) = xb;
                *reinterpret_cast<bf16x4*>(&sm.fq[1][(16 * g + li) * 4]) =
                    bq(mfma_k32(cat8(xb, xb), cat8(eyeb, zb4), zero4));
            }
            if (w == 1) {
                const f32x4 x = small_abt<D>(sm.b.Z, sm.U, li, g);
                float da[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    da[i] = (li < 4 * g + i) ? -x[i] : 0.0f;
                    sm.dA[(4 * g + i) * LS + li] = da[i];
                }
                const bf16x4 db = bq4(da[0], da[1], da[2], da[3]);
                *reinterpret_cast<bf16x4*>(&sm.fq[2][(16 * g + li) * 4]) =
                    bq4(bt[0] * da[0], bt[1] * da[1], bt[2] * da[2], bt[3] * da[3]);
                *reinterpret_cast<bf16x4*>(&sm.fq[3][(16 * g + li) * 4]) =
                    bq(mfma_k32(cat8(db, db), cat8(eyeb, zb4), zero4));
            }
            f32x4 zs = zero4, aqv = zero4, aev = zero4;
            float dgc = 0.0f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int o = li * LDR + 32 * kb + 4 * g;
                zs = mfma_k32(cat8(ld_b4(&sm.b.Z[o]), ld_b4(&sm.b.Z[o + 16])), sfn[kb], zs);
                aqv = mfma_k32(cat8(ld_b4(&sm.b.dO[o]), ld_b4(&sm.b.dO[o + 16])), sfn[kb], aqv);
                const int ox = ch * LDR + 32 * kb + 4 * g;   // dS' row ch, the k-slots of this lane
                const bf16x8 xb = cat8(ld_b4(&sm.u.Xs[ox]), ld_b4(&sm.u.Xs[ox + 16]));
                aev = mfma_k32(cat8(ld_b4(&sm.U[o]), ld_b4(&sm.U[o + 16])), xb, aev);
                dgc = dot8(xb, sfn[kb], dgc);
            }
            dgc += __shfl_xor(dgc, 16);
            dgc += __shfl_xor(dgc, 32);
            // this chunk's saved operands are used up: the previous chunk's load while the
            // rest of this one runs
            load_saved(n - 1);
            lds_barrier();

            // ---- the rest of the row products and the chain rule; lane (g, li): channel ch, tokens 4g+i
            const bf16x4 kmb = ld_b4(&sm.kmT[ch * LDK + 4 * g]);
            const int fo = (16 * g + li) * 4;
            const f32x4 aqp = mfma_k16(ld_b4(&sm.fq[1][fo]), kmb, zero4);   // dA_qk K-
            const f32x4 dak = mfma_k16(ld_b4(&sm.fq[3][fo]), kmb, zero4);   // dA K-
            const bf16x8 qk = cat8(ld_b4(&sm.b.qpT[ch * LDK + 4 * g]), ld_b4(&sm.kpT[ch * LDK + 4 * g]));
            // dA_qk^T Q+ + (diag(beta) dA)^T K+
            const f32x4 amv = mfma_k32(cat8(ld_b4(&sm.fq[0][fo]), ld_b4(&sm.fq[2][fo])), qk, zero4);
            const Rsrc rq = make_rsrc(dq + hb + (int64_t)tc * tstr, (uint32_t)nv * tstr * 4u);
            const Rsrc rk = make_rsrc(dk + hb + (int64_t)tc * tstr, (uint32_t)nv * tstr * 4u);
            const Rsrc rt_ = make_rsrc(dtheta + hb + (int64_t)tc * tstr, (uint32_t)nv * tstr * 4u);
            // The intra-chunk (pair) parts of dK+, dQ+ and dK- each reach the log-decay of
            // two tokens with opposite signs, which cancel in its reverse prefix sum; they
            // cancel to fp32 accuracy only when both sides use the bf16 values the products
            // used, so those parts are multiplied by the rounded K+, K- and Q+.
            auto rb = [](float x) { return (float)(bf16)x; };
            float dG[4], kes = 0.0f, kzp[4], dkv[4], dqv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float aks = -bt[i] * zs[i], akp = bt[i] * dak[i];   // dK+: state part, pair part
                const float gm = G.gam[i], ig = G.igam[i];
                dkv[i] = (aks + akp) * gm + amv[i] * ig + aev[i] * (G.gC * ig);
                dqv[i] = (aqv[i] + aqp[i]) * gm;
                const float ked = aev[i] * kev(i);
                kes += ked;
                const float kpb = rb(kpv(i));
                dG[i] = aks * kpv(i) + akp * kpb - amv[i] * rb(kmv(i)) + aqv[i] * qpv(i) + aqp[i] * rb(qpv(i)) - ked;
                kzp[i] = zs[i] * kpb;   // rowsum(K+ * (Z S^T)) with the K+ the forward's Y used
            }
            store_grad(dkv, rk);
            store_grad(dqv, rq);
            kes += __shfl_xor(kes, 16);
            kes += __shfl_xor(kes, 32);
            // the chunk's last token also carries the end decay: d(G_C) = sum_t dKend Kend + dGamma_C Gamma_C
            if (g == 3) dG[3] += kes + dgc * G.gC;
            float suf = 0.0f;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                suf += dG[i];
                dG[i] = suf;
            }
            const float s1 = __shfl(suf, 16 + li), s2 = __shfl(suf, 32 + li), s3 = __shfl(suf, 48 + li);
            const float later = (g < 1 ? s1 : 0.0f) + (g < 2 ? s2 : 0.0f) + (g < 3 ? s3 : 0.0f);
            float dth[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) dth[i] = (dG[i] + later) * G.dsg[i];
            store_grad(dth, rt_);
            // rowsum(K+ * (Z S^T)) over this wavefront's 16 channels
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = rowsum16(kzp[i]);
                if (li == 0) sm.kz[w][4 * g + i] = s;
            }
            // the previous chunk's inputs (every read of this chunk's is behind the first barrier)
            stage_raw(raw);
            lds_barrier();
            if (w < 4) {
                // dbeta = rowsum(dA * KK) + rowsum(Z * V) - rowsum(K+ * (Z S^T)), on the first
                // four wavefronts only: they reach the next chunk's first barrier well before
                // the others, which start that chunk's tiles at once.  Wavefront w forms tokens
                // 4w .. 4w+3, one per lane group; lane li takes term s = li of each sum, and
                // the 16 lanes of the group add them up and store the value (equal duplicates).
                // The next writes of dA, KK, zv and kz follow the next chunk's first barrier.
                const int t = 4 * w + g;
                float a = sm.dA[t * LS + li] * sm.KK[t * LS + li];
                if (li < C::NW) a += sm.zv[li][t] - sm.kz[li][t];
                a = rowsum16(a);
                const Rsrc rb = make_rsrc(dbeta + bb + (int64_t)tc * H, (uint32_t)nv * (uint32_t)H * 4u);
                buf_st32(a, rb, (uint32_t)t * (uint32_t)H * 4u, 0u);
            }
        }
        if (dS0 && seg == 0) {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) dS0[((int64_t)bh * D + 16 * rt + 4 * g + i) * D + ch] = X[rt][0][i];
        }
    }
}

size_t chunk_bwd2_workspace_bytes(int B, int T, int H, int d, int nseg) {
    const size_t nchunks = ((size_t)T + CHUNK - 1) / CHUNK;
    const size_t BH = (size_t)B * H;
    const size_t DD = (size_t)d * d;
    size_t n = nchunks * BH * (DD + 16 * (size_t)d + 256) * sizeof(bf16);
    n = (n + 255) & ~(size_t)255;
    if (nseg > 1) n += (size_t)nseg * BH * (4 * DD + 2 * DD) * sizeof(float);
    return n;
}

hipError_t launch_chunk_bwd2(int B, int T, int H, int d, int nseg, int seg_len, const void* q, const void* k,
                             const void* v, const float* theta, const float* beta, const float* S0,
                             const void* dout, const float* dS_T, float* dq, float* dk, float* dv,
                             float* dtheta, float* dbeta, float* dS0, void* workspace, hipStream_t stream) {
    const int nchunks = (int)(((int64_t)T + CHUNK - 1) / CHUNK);
    const int BH = B * H;
    const size_t DD = (size_t)d * d;
    bf16* wsb = (bf16*)workspace;
    size_t off = (size_t)nchunks * BH * (DD + 16 * (size_t)d + 256) * sizeof(bf16);
    off = (off + 255) & ~(size_t)255;
    // per direction: N (fp32) then M (bf16, in a region sized for fp32), [map][BH][d][d]
    float* mapF = (float*)((char*)workspace + off);
    float* mapB = mapF + (size_t)nseg * BH * 2 * DD;
    float* Sst = mapB + (size_t)nseg * BH * 2 * DD;    // state at every segment's start
    float* Xen = Sst + (size_t)nseg * BH * DD;         // carried gradient at the segments' ends, reversed
#define KDA_B2(D, GRID, XI)                                                                             \
    hipLaunchKernelGGL((bwd2_kernel<D>), dim3((unsigned)(GRID)), dim3(B2Cfg<D>::NTHR), 0, stream, T, H,      \
                       BH, nchunks, seg_len, (const bf16*)q, (const bf16*)k, (const bf16*)v, theta, beta,      \
                       (const bf16*)dout, XI, dq, dk, dv, dtheta, dbeta, dS0, wsb)
    SegPlan plan;
    plan.nchunks = nchunks;
    plan.seg_len = seg_len;
    plan.nseg = nseg;
    // One segment: the forward chain's saved operands from the map kernel's SAVE mode,
    // then the backward sweep.  Several: the state maps and every chunk's T' (into the
    // chunk area, which the SAVE pass overwrites only later) from the prefill's map
    // kernel, the gradient maps, both chains combined, then SAVE and the backward sweep
    // from the segments' boundary values.
#define KDA_B2_ALL(D)                                                                                     \
    if (nseg == 1) {                                                                                      \
        hipError_t e = launch_chunk_save(B, T, H, D, plan, k, v, theta, beta, S0, wsb, stream);           \
        if (e != hipSuccess) return e;                                                                    \
        KDA_B2(D, BH, dS_T);                                                                              \
    } else {                                                                                              \
        hipError_t e = launch_chunk_map(false, B, T, H, D, plan, k, v, theta, beta, mapF,                  \
                                        mapF + (size_t)nseg * BH * DD, wsb, stream);                      \
        if (e != hipSuccess) return e;                                                                    \
        e = launch_grad_map(B, T, H, D, plan, q, k, theta, dout, wsb, mapB, stream);                    \
        if (e != hipSuccess) return e;                                                                    \
        e = launch_state_combine(D, BH, nseg, S0, mapF, mapF + (size_t)nseg * BH * DD, Sst, stream);      \
        if (e == hipSuccess)                                                                              \
            e = launch_state_combine(D, BH, nseg, dS_T, mapB, mapB + (size_t)nseg * BH * DD, Xen, stream);  \
        if (e == hipSuccess) e = launch_chunk_save(B, T, H, D, plan, k, v, theta, beta, Sst, wsb, stream); \
        if (e != hipSuccess) return e;                                                                    \
        KDA_B2(D, nseg * BH, (const float*)Xen);                                                          \
    }                                                                                                     \
    return hipGetLastError()
    switch (d) {
        case 64: KDA_B2_ALL(64);
        case 128: KDA_B2_ALL(128);
    }
#undef KDA_B2_ALL
#undef KDA_B2
    return hipErrorInvalidValue;
}

}  // namespace kda

// kda_device.hpp -- device-side building blocks shared by the libkda kernels
// (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (64-lane wavefront, lane = 16*g + r,
// r = lane & 15, g = lane >> 4):
//   * a 16x16 fp32 accumulator tile D holds D[4*g + i][r] in element i (i = 0..3);
//   * the A operand of a 16x16xK product supplies row r of A, the B operand
//     supplies column r of B; lane group g supplies a group of consecutive
//     k-slots (1 slot for K = 4 fp32, 4 for K = 16 bf16, 8 for K = 32 bf16).
// Which logical contraction index sits in which (g, slot) only has to agree
// between A and B, so every product below states the index map it uses.
// An accumulator tile, read as B, puts row 4*g + i in slot i -- the same map a
// 16x16x16 bf16 B operand uses -- so recurrent state and per-chunk results feed
// the next product straight from registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));

constexpr int CHUNK = 16;       // tokens per chunk
constexpr float G_MIN = -5.0f;  // lower bound of the log-decay

// ---------------------------------------------------------------- gate
// g = G_MIN * sigmoid(theta); saturates to exactly 0 for theta -> -inf and
// G_MIN for theta -> +inf.
__device__ __forceinline__ float gate_logdecay(float theta) {
    const float e = __expf(-theta);
    return G_MIN * __builtin_amdgcn_rcpf(1.0f + e);
}

// Output gate sigmoid(z) = 1 / (1 + e^-z) ("Kimi K3" explainer, "Across the
// sequence": a per-channel sigmoid gate on the attention output), from the
// hardware base-2 exponential and reciprocal.  It saturates to exactly 0 and
// 1 in the tails (e^-z overflowing to inf gives 0), never NaN for finite z.
__device__ __forceinline__ float out_sigmoid(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// ---------------------------------------------------------------- synchronisation
// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, for which the compiler waits until every outstanding
// global load has returned -- which would drain loads issued early on purpose.
// Use this where the wavefronts exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wavefront's LDS writes before its following LDS reads of other
// lanes' data.  A wavefront's LDS instructions execute in issue order, so only
// the compiler has to be kept from moving accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- lane exchange
// A wavefront's 64 lanes as four rows of 16.

// Lane N of each row, copied to every lane of that row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_lane(float v) {
    static_assert(N >= 0 && N < 16, "lane within a row");
    // every lane has a source lane, so the instruction's old value is never taken
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf,
                                                              false));
}

// Row R, copied to all four rows: lane n of every row takes lane n of row R
// (ds_bpermute: through the LDS crossbar, no memory and no VALU work).
template <int R>
__device__ __forceinline__ float row_to_all(float v, int lane) {
    static_assert(R >= 0 && R < 4, "row of a wavefront");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((R * 16 + (lane & 15)) * 4,
                                                                  __builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }  // RNE

// Two adjacent elements of a storage type, loaded/stored as one unit.
template <typename E> struct Pair;
template <> struct Pair<float> { typedef f32x2 T; };
template <> struct Pair<bf16> { typedef bf16x2 T; };

template <typename E>
__device__ __forceinline__ f32x2 load_pair(const E* p) {
    typename Pair<E>::T v = *reinterpret_cast<const typename Pair<E>::T*>(p);
    return f32x2{to_f(v[0]), to_f(v[1])};
}
template <typename E>
__device__ __forceinline__ void store_pair(E* p, float a, float b) {
    typename Pair<E>::T v;
    v[0] = from_f<E>(a);
    v[1] = from_f<E>(b);
    *reinterpret_cast<typename Pair<E>::T*>(p) = v;
}

// ---------------------------------------------------------------- MFMA wrappers
// K = 16 bf16 products run on the 16x16x32 instruction with the upper four
// k-slots of each lane group zeroed on both operands.  The legacy 16x16x16
// bf16 instruction is not used: results read right after it (at the wait
// states the compiler inserts for it) came back stale on gfx950.
__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    const bf16x4 z = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- buffer loads
// Global loads through a buffer resource: the base address lives in scalar
// registers and the per-lane offset is a loop-invariant 32-bit register, so a
// load costs no vector address arithmetic.  A load whose per-lane byte offset
// is at or past the resource's size returns zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes = 0xffffffffu) {
    // dword3 0x00020000: 32-bit data format, the raw-buffer setting for gfx9 parts.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of a buffer access (the builtins' last operand): kCpStream sets the
// non-temporal ("nt") bit, for data a kernel touches once and nothing reads soon after.
constexpr int kCpStream = 2;
template <int CP = 0>
__device__ __forceinline__ uint32_t buf_ld32(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, CP);
}
template <int CP = 0>
__device__ __forceinline__ f32x2 buf_ld_f2(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, CP));
}
// Four adjacent storage elements as one load.
template <typename E> struct BufQuad;
template <> struct BufQuad<bf16> {
    typedef bf16x4 T;
    static __device__ __forceinline__ T ld(Rsrc r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
    }
};
template <> struct BufQuad<float> {
    typedef f32x4 T;
    static __device__ __forceinline__ T ld(Rsrc r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    }
};

// Two adjacent storage elements as one load.
template <typename E> struct BufPair;
template <> struct BufPair<bf16> {
    template <int CP = 0>
    static __device__ __forceinline__ bf16x2 ld(Rsrc r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(bf16x2, buf_ld32<CP>(r, voff, soff));
    }
};
template <> struct BufPair<float> {
    template <int CP = 0>
    static __device__ __forceinline__ f32x2 ld(Rsrc r, uint32_t voff, uint32_t soff) {
        return buf_ld_f2<CP>(r, voff, soff);
    }
};

__device__ __forceinline__ bf16x4 ld_b4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ bf16x8 ld_b8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Four consecutive elements from LDS, in the register form Ops<E>::pad takes.
__device__ __forceinline__ bf16x4 ld_quad(const bf16* p) { return ld_b4(p); }
__device__ __forceinline__ f32x4 ld_quad(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Four consecutive elements to global memory through a buffer resource (a
// store at or past the resource's size is dropped).
__device__ __forceinline__ void buf_st_quad(bf16x4 x, Rsrc r, uint32_t voff) {
    typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, (int)voff, 0, 0);
}
__device__ __forceinline__ void buf_st_quad(f32x4 x, Rsrc r, uint32_t voff) {
    typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)voff, 0, 0);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------- 16x16 products
// Ops<E> evaluates D += A * B for 16x16 output tiles with operands of element
// type E (bf16: bf16 matrix cores, fp32 accumulate; float: fp32 matrix cores).
//
// mm_ll<K>(A, lda, Bt, ldb, acc): A is 16 x K row-major at A (leading dim lda),
//   B is K x 16 given transposed, Bt[n][k] = B[k][n], row-major at Bt.
// mm_la<K>(A, lda, Bf, acc): A as above; B is K x 16 held as K/16 accumulator
//   tiles converted with to_b (tile t holds B rows 16t..16t+15).
template <typename E> struct Ops;

template <> struct Ops<bf16> {
    typedef bf16x4 BFrag;
    static __device__ __forceinline__ BFrag to_b(f32x4 x) {
        return BFrag{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    }
    // k-map: K = 16: slot s of group g is k = 4g + s;
    //        K >= 32: block kb, slot s of group g is k = 32kb + 8g + s.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_ll(const bf16* A, int lda, const bf16* Bt, int ldb,
                                                  f32x4 acc, int r, int g) {
        if constexpr (K == 16) {
            acc = mfma_k16(ld_b4(A + r * lda + 4 * g), ld_b4(Bt + r * ldb + 4 * g), acc);
        } else {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {   // 8-byte halves: rows need only 8-byte alignment
                const bf16* a = A + r * lda + 32 * kb + 8 * g;
                const bf16* b = Bt + r * ldb + 32 * kb + 8 * g;
                acc = mfma_k32(cat8(ld_b4(a), ld_b4(a + 4)), cat8(ld_b4(b), ld_b4(b + 4)), acc);
            }
        }
        return acc;
    }
    // k-map: K = 16: k = 4g + s;  K >= 32: block kb, slot s < 4 is k = 32kb + 4g + s
    //        (tile 2kb), slot s >= 4 is k = 32kb + 16 + 4g + (s - 4) (tile 2kb + 1).
    template <int K>
    static __device__ __forceinline__ f32x4 mm_la(const bf16* A, int lda, const BFrag* Bf,
                                                  f32x4 acc, int r, int g) {
        if constexpr (K == 16) {
            acc = mfma_k16(ld_b4(A + r * lda + 4 * g), Bf[0], acc);
        } else {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                const bf16* a = A + r * lda + 32 * kb + 4 * g;
                acc = mfma_k32(cat8(ld_b4(a), ld_b4(a + 16)), cat8(Bf[2 * kb], Bf[2 * kb + 1]), acc);
            }
        }
        return acc;
    }

    // mm_la with the operands' roles exchanged: D += B^T A^T, i.e. the B
    // fragments (accumulator tiles of a K x 16 matrix X) act as the A operand
    // (rows of X^T) and rows of the LDS matrix A act as the B operand.  Same k-map.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_al(const BFrag* Bf, const bf16* A, int lda,
                                                  f32x4 acc, int r, int g) {
        if constexpr (K == 16) {
            acc = mfma_k16(Bf[0], ld_b4(A + r * lda + 4 * g), acc);
        } else {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                const bf16* a = A + r * lda + 32 * kb + 4 * g;
                acc = mfma_k32(cat8(Bf[2 * kb], Bf[2 * kb + 1]), cat8(ld_b4(a), ld_b4(a + 16)), acc);
            }
        }
        return acc;
    }

    // K = 16 products against "padded" LDS tiles: row m of the 16 x 16 operand
    // is stored as 4 groups of 8 elements, group g holding k = 4g .. 4g+3 and
    // four zeros, so one 16-byte load yields a complete 16x16x32 operand.
    typedef bf16x8 PFrag;   // a register operand in the same padded form
    // elements per padded row: 32 + 8.  (A 24-dword stride would free the 16-byte
    // reads of these rows from their bank conflicts, about four per read, but the
    // larger tiles measured slower in the kernel that uses them.)
    static constexpr int PAD_ROW = 40;
    static __device__ __forceinline__ PFrag to_p(f32x4 x) {
        const bf16x4 z = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
        return cat8(to_b(x), z);
    }
    // D += A B, A from the padded LDS row at Arow, B a register fragment.
    static __device__ __forceinline__ f32x4 mm16_pa(const bf16* Arow, PFrag b, f32x4 acc, int g) {
        return mfma_k32(ld_b8(Arow + 8 * g), b, acc);
    }
    // D += A B, A a register fragment, B from the padded LDS row at Brow (column r of B).
    static __device__ __forceinline__ f32x4 mm16_ap(PFrag a, const bf16* Brow, f32x4 acc, int g) {
        return mfma_k32(a, ld_b8(Brow + 8 * g), acc);
    }
    // The padded operand of one lane, loaded once and reused by several products.
    static __device__ __forceinline__ PFrag ld_p(const bf16* row, int g) { return ld_b8(row + 8 * g); }
    // Four k-slots held in registers, padded to an operand.
    static __device__ __forceinline__ PFrag pad(bf16x4 x) {
        const bf16x4 z = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
        return cat8(x, z);
    }
    static __device__ __forceinline__ f32x4 mm16(PFrag a, PFrag b, f32x4 acc) { return mfma_k32(a, b, acc); }

    // mm_la and mm_al over NTL column tiles at once (tiles n < nv only): each
    // fragment of the LDS operand is loaded once and used by every tile.
    // Bf holds the tiles' fragments as Bf[n * (K / 16) + t].
    template <int K, int NTL>
    static __device__ __forceinline__ void mm_la_n(const bf16* A, int lda, const BFrag* Bf, f32x4* acc,
                                                   int nv, int r, int g) {
        if constexpr (K == 16) {
            const bf16x4 a = ld_b4(A + r * lda + 4 * g);
#pragma unroll
            for (int n = 0; n < NTL; ++n)
                if (n < nv) acc[n] = mfma_k16(a, Bf[n], acc[n]);
        } else {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                const bf16* ap = A + r * lda + 32 * kb + 4 * g;
                const bf16x8 a = cat8(ld_b4(ap), ld_b4(ap + 16));
#pragma unroll
                for (int n = 0; n < NTL; ++n)
                    if (n < nv) acc[n] = mfma_k32(a, cat8(Bf[n * (K / 16) + 2 * kb], Bf[n * (K / 16) + 2 * kb + 1]), acc[n]);
            }
        }
    }
    template <int K, int NTL>
    static __device__ __forceinline__ void mm_al_n(const BFrag* Bf, const bf16* A, int lda, f32x4* acc,
                                                   int nv, int r, int g) {
        if constexpr (K == 16) {
            const bf16x4 a = ld_b4(A + r * lda + 4 * g);
#pragma unroll
            for (int n = 0; n < NTL; ++n)
                if (n < nv) acc[n] = mfma_k16(Bf[n], a, acc[n]);
        } else {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                const bf16* ap = A + r * lda + 32 * kb + 4 * g;
                const bf16x8 a = cat8(ld_b4(ap), ld_b4(ap + 16));
#pragma unroll
                for (int n = 0; n < NTL; ++n)
                    if (n < nv) acc[n] = mfma_k32(cat8(Bf[n * (K / 16) + 2 * kb], Bf[n * (K / 16) + 2 * kb + 1]), a, acc[n]);
            }
        }
    }

    // As mm_la, with A read from global fp32 memory (row-major, leading dim lda)
    // and rounded to bf16 on the fly.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_ga(const float* A, int64_t lda, const BFrag* Bf,
                                                  f32x4 acc, int r, int g) {
        if constexpr (K == 16) {
            acc = mfma_k16(to_b(*reinterpret_cast<const f32x4*>(A + r * lda + 4 * g)), Bf[0], acc);
        } else {
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                const float* a = A + r * lda + 32 * kb + 4 * g;
                const bf16x4 lo = to_b(*reinterpret_cast<const f32x4*>(a));
                const bf16x4 hi = to_b(*reinterpret_cast<const f32x4*>(a + 16));
                acc = mfma_k32(cat8(lo, hi), cat8(Bf[2 * kb], Bf[2 * kb + 1]), acc);
            }
        }
        return acc;
    }
};

template <> struct Ops<float> {
    typedef f32x4 BFrag;
    static __device__ __forceinline__ BFrag to_b(f32x4 x) { return x; }
    // k-map: step kk, group g is k = 4kk + g.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_ll(const float* A, int lda, const float* Bt, int ldb,
                                                  f32x4 acc, int r, int g) {
#pragma unroll
        for (int kk = 0; kk < K / 4; ++kk)
            acc = mfma_k4(A[r * lda + 4 * kk + g], Bt[r * ldb + 4 * kk + g], acc);
        return acc;
    }
    // k-map: step (t, i), group g is k = 16t + 4g + i.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_la(const float* A, int lda, const BFrag* Bf,
                                                  f32x4 acc, int r, int g) {
#pragma unroll
        for (int t = 0; t < K / 16; ++t) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(A + r * lda + 16 * t + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma_k4(a[i], Bf[t][i], acc);
        }
        return acc;
    }

    // Exchanged roles, as in the bf16 version.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_al(const BFrag* Bf, const float* A, int lda,
                                                  f32x4 acc, int r, int g) {
#pragma unroll
        for (int t = 0; t < K / 16; ++t) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(A + r * lda + 16 * t + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma_k4(Bf[t][i], a[i], acc);
        }
        return acc;
    }

    // Padded K = 16 tiles (see the bf16 version); in fp32 only the first four
    // elements of each group are used, one k-step per element.
    typedef f32x4 PFrag;
    static constexpr int PAD_ROW = 36;
    static __device__ __forceinline__ PFrag to_p(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 mm16_pa(const float* Arow, PFrag b, f32x4 acc, int g) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(Arow + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mfma_k4(a[i], b[i], acc);
        return acc;
    }
    static __device__ __forceinline__ f32x4 mm16_ap(PFrag a, const float* Brow, f32x4 acc, int g) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(Brow + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mfma_k4(a[i], b[i], acc);
        return acc;
    }
    static __device__ __forceinline__ PFrag ld_p(const float* row, int g) {
        return *reinterpret_cast<const f32x4*>(row + 8 * g);
    }
    static __device__ __forceinline__ PFrag pad(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 mm16(PFrag a, PFrag b, f32x4 acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mfma_k4(a[i], b[i], acc);
        return acc;
    }

    // Multi-tile forms, as in the bf16 version.
    template <int K, int NTL>
    static __device__ __forceinline__ void mm_la_n(const float* A, int lda, const BFrag* Bf, f32x4* acc,
                                                   int nv, int r, int g) {
#pragma unroll
        for (int t = 0; t < K / 16; ++t) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(A + r * lda + 16 * t + 4 * g);
#pragma unroll
            for (int n = 0; n < NTL; ++n)
                if (n < nv) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[n] = mfma_k4(a[i], Bf[n * (K / 16) + t][i], acc[n]);
                }
        }
    }
    template <int K, int NTL>
    static __device__ __forceinline__ void mm_al_n(const BFrag* Bf, const float* A, int lda, f32x4* acc,
                                                   int nv, int r, int g) {
#pragma unroll
        for (int t = 0; t < K / 16; ++t) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(A + r * lda + 16 * t + 4 * g);
#pragma unroll
            for (int n = 0; n < NTL; ++n)
                if (n < nv) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[n] = mfma_k4(Bf[n * (K / 16) + t][i], a[i], acc[n]);
                }
        }
    }

    // As mm_la, with A read from global fp32 memory.
    template <int K>
    static __device__ __forceinline__ f32x4 mm_ga(const float* A, int64_t lda, const BFrag* Bf,
                                                  f32x4 acc, int r, int g) {
#pragma unroll
        for (int t = 0; t < K / 16; ++t) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(A + r * lda + 16 * t + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = mfma_k4(a[i], Bf[t][i], acc);
        }
        return acc;
    }
};

}  // namespace kda

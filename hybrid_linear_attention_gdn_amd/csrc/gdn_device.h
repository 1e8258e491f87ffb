// Device-side definitions shared by the gfx950 Gated DeltaNet kernels.
//
// Matrix-core tiles use v_mfma_f32_16x16x32_f16 (wave64).  Operand fragment
// of that instruction: lane l holds 8 values of row/column (l % 16) for the
// 8 contraction slots of lane group (l / 16).  Accumulator: lane l holds rows
// 4 * (l / 16) + e, e = 0..3, of column (l % 16).  A contraction index may be
// permuted freely as long as both operands use the same permutation; the
// kernels use that to feed accumulators back as operands without an LDS
// round trip (see the slot maps below).
//
// bfloat16 inputs are widened to fp16 on load.  Every bf16 value in
// [2^-14, 65504] is exact in fp16 (8 significant bits fit in 11); smaller
// magnitudes lose at most 2^-25 absolutely.  fp16 operands keep derived
// quantities (the UT-transform rows, corrected writes U', chunk states) to an
// 11-bit mantissa, where bf16 would carry only 8: in a numerical model of the
// chunkwise form bf16 operands cost ~2.8e-3 relative L2 on outputs and
// ~2.1e-3 on states, fp16 ~3.5e-4 on both.  fp16 and bf16 share the MFMA
// peak rate on CDNA4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_sizes.h"

namespace gdn {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Workspace regions are chunk-slot-major: unit (slot, head) sits at slot *
// heads + head, so the units of all heads for one chunk are contiguous (a
// few large pages per chunk step for the state recurrence, whose 256 or more
// workgroups walk the chunks in step).
struct ChunkWorkspace {
    f16* tu;
    f16* p;
    float* dg;
    f16* kt;
    f16* qf;
    float* junk;
    int n_slots;
    int group;     // value heads per q/k head
    int h_v, h_qk;

    __device__ __forceinline__ size_t vunit(int slot, int h) const { return (size_t)slot * h_v + h; }
    // K^T and Q fragments are per q/k head j
    __device__ __forceinline__ size_t kunit(int slot, int j) const { return (size_t)slot * h_qk + j; }
};

// Cache-policy operand of a direct global-to-LDS copy
// (__builtin_amdgcn_global_load_lds): 0 ordinary, 2 non-temporal (the line
// is not kept for reuse).
constexpr int kCopyCached = 0;
constexpr int kCopyNonTemporal = 2;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ f16x8 bf16x8_to_f16x8(u16x8 b) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<f16>(bf16_to_f32(b[i]));
    return r;
}

__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Same tile on raw bfloat16 operands (used where both operands are inputs).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 value split as hi + lo in fp16: hi = x rounded toward zero to fp16
// (two values per packed conversion), lo = fp16(x - hi), where x - hi is
// exact in fp32 and |x - hi| < ulp16(hi): 21 significant bits between them
// for |x| in the fp16 normal range.  lo is formed as fma(hi, m, x) with
// m = -1 hidden from the optimiser, which otherwise folds the product into
// a subtraction: the mixed-precision fma then takes hi as fp16 straight
// from the packed register and rounds into an fp16 half, 7 VALU
// instructions per four values instead of 12 (widen, subtract, pack), with
// the same result (x - hi is exact, so either way it is rounded once).
struct Split16 {
    f16x4 hi, lo;
};

typedef f16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ Split16 split16(f32x4 x) {
    const f16x2 h01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x[0], x[1]));
    const f16x2 h23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x[2], x[3]));
    float m = -1.f;
    asm("" : "+s"(m));
    Split16 s;
    s.hi = f16x4{h01[0], h01[1], h23[0], h23[1]};
    s.lo = f16x4{static_cast<f16>(__builtin_fmaf(static_cast<float>(h01[0]), m, x[0])),
                 static_cast<f16>(__builtin_fmaf(static_cast<float>(h01[1]), m, x[1])),
                 static_cast<f16>(__builtin_fmaf(static_cast<float>(h23[0]), m, x[2])),
                 static_cast<f16>(__builtin_fmaf(static_cast<float>(h23[1]), m, x[3]))};
    return s;
}

// 16x16x16 product of split fp32 operands in fragment form (A: lane l holds
// row l%16, k = 4 (l/16) + e; B: k = 4 (l/16) + e, column l%16) on fp16
// matrix cores: hi*hi + hi*lo + lo*hi, error ~2^-21 relative.
__device__ __forceinline__ f32x4 mfma_split16(Split16 a, Split16 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(a.hi, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16f16(a.lo, b.hi, c, 0, 0, 0);
    return c;
}

// exp(x) through the hardware base-2 exponential; used for decay factors
// exp(G_r - G_s) with non-positive arguments (relative error ~1e-6).
__device__ __forceinline__ float exp_f(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ f16x8 cat_to_f16(f32x4 lo, f32x4 hi) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = static_cast<f16>(lo[e]);
        r[e + 4] = static_cast<f16>(hi[e]);
    }
    return r;
}

// Chunk slots.  Sequence n owns slots n + cu[n] / 64 ... + ceil(len_n / 64) - 1;
// consecutive sequences never overlap because the base grows by at least
// 1 + floor(len_n / 64) >= ceil(len_n / 64).  Slots in the gaps are unused.
// The slot count needed is at most N + T / 64 + 1, known on the host.
__device__ __forceinline__ int slot_base(const int32_t* cu, int n) {
    return n + cu[n] / kChunk;
}

// Map a chunk slot to (sequence, first token, length).  Returns false for an
// unused slot.  Every thread computes the same answer (uniform loads).
__device__ __forceinline__ bool resolve_slot(const int32_t* __restrict__ cu, int n_seqs, int slot,
                                             int& seq, int& t0, int& len) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_base(cu, mid) <= slot) lo = mid; else hi = mid - 1;
    }
    const int c = slot - slot_base(cu, lo);
    const int start = cu[lo], end = cu[lo + 1];
    const int first = start + c * kChunk;
    if (c < 0 || first >= end) return false;
    seq = lo;
    t0 = first;
    len = min(kChunk, end - first);
    return true;
}

}  // namespace gdn

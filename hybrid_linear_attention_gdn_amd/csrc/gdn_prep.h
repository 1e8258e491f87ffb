// Stage 1 of the chunked Gated DeltaNet prefill for gfx950: intra-chunk
// preparation (the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page, section 2,
// first of its three stages).  Per chunk of 64 positions and value head it
// forms the decay cumsum, A = strictly-lower(beta_r e^{G_r-G_s} K K^T), the UT
// transform Tm = (I + A)^{-1}, TU = Tm diag(beta) and P = M o Q K^T, and
// writes them, with the fp16 K^T and Q of each q/k head, in the matrix-core
// fragment order the state kernel reads.  W = TU diag(e^G) K and U = TU V are
// formed by the state kernel on chip (the algebra is restated in
// gdn_chunk.hip): 6 KB of TU per chunk and value head instead of 32 KB of W
// and U through memory.
//
// One workgroup serves kH value heads of one q/k head (two when the heads per
// q/k head are even): they share the chunk's K and Q rows and the raw Grams
// K K^T and K Q^T, and differ only in beta and the decay.  At 32 value / 16
// q/k heads that is 1008 workgroups for a 4000-token chunk batch, which four
// workgroups per CU run in one round, where one workgroup per value head took
// two, each paying the full latency of its input loads.
//
// The kernel is a template over its store kind: ordinary stores, or
// non-temporal ones for workspaces too large to stay cached until the state
// kernel reads them.  Each kind is instantiated in a translation unit of its
// own (gdn_prep.hip, gdn_prep_stream.hip): with both in one unit the compiler
// allocated registers differently for both, with 25 spill operations instead
// of 2, and the ordinary kind ran 5 us slower at T = 4000.
#pragma once

#include "gdn_device.h"

namespace gdn {

namespace {

// LDS row stride (floats) of the fp32 64 x 64 A / Tm: rows 4 apart (the rows
// of one accumulator store) fall 16 banks apart
constexpr int kTA = 68;

// Row-major [pos][dim] bf16 tiles, 128 dims per row, no padding: 16-byte
// chunk c (dims 8 c .. 8 c + 7) of row r sits at chunk c ^ (r % 16), so the
// 16 rows read at the same dims by a fragment load hit 16 different banks.
// Returns the element offset of chunk c of row r.
__device__ __forceinline__ int rsw(int r, int c) {
    return r * kDim + ((c ^ (r & 15)) << 3);
}

typedef short p16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) p16x4 lds_p16x4;

// K^T as the A fragment (d_k tile i, position step qq) of the state update:
// lane (gq, ln) holds K[p][16 i + ln] at the position slots p = 32 qq +
// 16 (s / 4) + 4 gq + s % 4, widened to fp16.  Read from the bf16 K rows in
// LDS with two transpose reads (ds_read_b64_tr_b16): in each group of 16
// lanes that instruction hands lane l element l % 4 of the 8-byte granules
// addressed by lanes l / 4 + 4 e, e = 0..3, so lane l addresses row
// 32 qq + 16 h + 4 gq + l / 4 at dims 16 i + 4 (l % 4) .. + 3 and receives
// rows 32 qq + 16 h + 4 gq + e of dim 16 i + l.
__device__ __forceinline__ f16x8 kt_frag(const uint16_t* Kr, int i, int qq, int gq, int ln) {
    f16x8 f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 32 * qq + 16 * h + 4 * gq + (ln >> 2);
        const int a = 4 * i + (ln & 3);                     // 8-byte granule of the row
        const p16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_p16x4*)(Kr + rsw(row, a >> 1) + 4 * (a & 1)));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[4 * h + e] = static_cast<f16>(bf16_to_f32(static_cast<uint16_t>(x[e])));
    }
    return f;
}

// ---------------------------------------------------------------------------
// Stage 1 helpers.  The Gram blocks (p, jt), jt <= p, of row tiles of K, and
// P's row tile p (owned by wave p, which holds Q's row tile p), spread so that
// every wave runs five 16 x 16 x 128 products and their decay factors: wave
// w computes P's blocks (w, 0..w) and the Gram blocks listed here.
// A store of prep's intermediates: ordinary, or non-temporal when the
// workspace is too large to stay in the last-level cache until the state
// kernel reads it (then its lines would only evict others on the way).
template <bool kStream, typename T>
__device__ __forceinline__ void put(T* p, T x) {
    if constexpr (kStream) __builtin_nontemporal_store(x, p);
    else *p = x;
}

template <int W> struct GramBlocks;
template <> struct GramBlocks<0> { static constexpr int n = 4, p[4] = {1, 2, 3, 3}, jt[4] = {0, 0, 0, 1}; };
template <> struct GramBlocks<1> { static constexpr int n = 3, p[4] = {1, 2, 3, 0}, jt[4] = {1, 1, 2, 0}; };
template <> struct GramBlocks<2> { static constexpr int n = 2, p[4] = {2, 3, 0, 0}, jt[4] = {2, 3, 0, 0}; };
template <> struct GramBlocks<3> { static constexpr int n = 1, p[4] = {0, 0, 0, 0}, jt[4] = {0, 0, 0, 0}; };

// Where the transposed diagonal block A_ii goes: block (0, 1 + i) for i < 3,
// (1, 2) for i = 3 (above the diagonal, which nothing else uses).
__device__ __forceinline__ int diag_row_block(int i) { return i < 3 ? 0 : 1; }
__device__ __forceinline__ int diag_col_block(int i) { return i < 3 ? 1 + i : 2; }

// One head's A values of a Gram block: A_rs for rows r = 16 p + 4 gq + e,
// column s = 16 jt + ln (0 for s >= r), from the raw K K^T accumulator.
__device__ __forceinline__ f32x4 a_values(const f32x4& acc, const float* Gs, const float* Bs, int p, int jt, int gq,
                                          int ln) {
    const int s = 16 * jt + ln;
    const float gsv = Gs[s];
    f32x4 av;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * p + 4 * gq + e;
        av[e] = (s < r) ? Bs[r] * exp_f(Gs[r] - gsv) * acc[e] : 0.f;
    }
    return av;
}

// Store a block of A values into an A buffer (row stride kTA); a diagonal
// block goes transposed to its place above the diagonal.
__device__ __forceinline__ void put_a(float* Ab, const f32x4& av, int p, int jt, int gq, int ln) {
    if (jt < p) {
#pragma unroll
        for (int e = 0; e < 4; ++e) Ab[(16 * p + 4 * gq + e) * kTA + 16 * jt + ln] = av[e];
    } else {
        *reinterpret_cast<f32x4*>(Ab + (16 * diag_row_block(p) + ln) * kTA + 16 * diag_col_block(p) + 4 * gq) = av;
    }
}

// The products of wave W for kH value heads: the raw Gram blocks once, with
// each head's A values of them (head 0's into av, to be stored once every
// wave has read its K tiles from head 0's A buffer; the other heads' straight
// into their own, still unused, A buffers), and P's row tile W per head,
// stored to pdst[hh].  K row tiles come from Kr (row-major bf16,
// chunk-swizzled), the wave's own from kown.
template <int W, bool kStream, int kH>
__device__ __forceinline__ void prep_products(f32x4 (&av)[4], const bf16x8 (&kown)[4], const bf16x8 (&qf)[4],
                                              const uint16_t* Kr, float* const (&Ab)[kH], const float* const (&Gs)[kH],
                                              const float* const (&Bs)[kH], f16* const (&pdst)[kH],
                                              int lane, int gq, int ln) {
    bf16x8 kt[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            kt[t][kk] = t == W ? kown[kk]
                               : __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(Kr + rsw(16 * t + ln, 4 * kk + gq)));
    using B = GramBlocks<W>;
#pragma unroll
    for (int i = 0; i < B::n; ++i) {
        const int p = B::p[i], jt = B::jt[i];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};   // exact bf16 inputs
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc = mfma_bf16(kt[p][kk], kt[jt][kk], acc);
        av[i] = a_values(acc, Gs[0], Bs[0], p, jt, gq, ln);
#pragma unroll
        for (int hh = 1; hh < kH; ++hh) put_a(Ab[hh], a_values(acc, Gs[hh], Bs[hh], p, jt, gq, ln), p, jt, gq, ln);
    }
    // P = M o (Q K^T) for row tile W, M_rs = e^{G_r - G_s} (s <= r), computed
    // as (K Q^T)[s][r] so that the accumulators of two position tiles stack
    // into the A fragment of P over position slots, which is how the output
    // stage reads it: block (p, qq) at 2 p (p < 2) or 2 + 2 (p - 2) + qq;
    // blocks (0, 1) and (1, 1) are zero and not stored.
    const int r = 16 * W + ln;
    f32x4 dt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        dt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (jt > W) continue;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) dt[jt] = mfma_bf16(kt[jt][kk], qf[kk], dt[jt]);
    }
    constexpr int f0 = W < 2 ? W : 2 * W - 2;
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
        const float gr = Gs[hh][r];
        f32x4 m[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sp = 16 * jt + 4 * gq + e;
                m[jt][e] = (jt <= W && sp <= r) ? exp_f(gr - Gs[hh][sp]) * dt[jt][e] : 0.f;
            }
        put<kStream>(reinterpret_cast<f16x8*>(pdst[hh] + ((size_t)f0 * 64 + lane) * 8), cat_to_f16(m[0], m[1]));
        if constexpr (W >= 2)
            put<kStream>(reinterpret_cast<f16x8*>(pdst[hh] + ((size_t)(f0 + 1) * 64 + lane) * 8), cat_to_f16(m[2], m[3]));
    }
}

// Head 0's A values of wave W's Gram blocks into its A buffer.
template <int W>
__device__ __forceinline__ void store_a(float* Ab, const f32x4 (&av)[4], int gq, int ln) {
    using B = GramBlocks<W>;
#pragma unroll
    for (int i = 0; i < B::n; ++i) put_a(Ab, av[i], B::p[i], B::jt[i], gq, ln);
}

// Tm_ii = (I + A_ii)^{-1} of diagonal block i of one head, in place in its A
// buffer.  N = A_ii is strictly lower, so N^16 = 0 and (I + N)^{-1} =
// sum_p (-N)^p = (I - N)(I + N^2)(I + N^4)(I + N^8): eight 16x16x16 products
// in six dependent steps.  A product's accumulator Xc (lane (gq, ln) holds
// X[4 gq + e][ln]) is X's B operand and X^T's A operand, so a power is also
// formed transposed where the next product needs it as an A operand.  Split
// fp16 operands (~2^-21 relative per product); for |N_rs| <= 1 every power
// and partial product stays below 2^14, inside fp16 range.
__device__ __forceinline__ void diag_inverse(float* Ab, int ib, int gq, int ln) {
    const float* at = Ab + 16 * diag_row_block(ib) * kTA + 16 * diag_col_block(ib);   // at[t * kTA + r] = A_ii[r][t]
    const f32x4 nb = *reinterpret_cast<const f32x4*>(at + ln * kTA + 4 * gq);           // N[4 gq + e][ln]
    f32x4 na;                                                                           // N[ln][4 gq + e]
#pragma unroll
    for (int e = 0; e < 4; ++e) na[e] = at[(4 * gq + e) * kTA + ln];
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const Split16 sna = split16(na), snb = split16(nb);
    const f32x4 n2 = mfma_split16(sna, snb, z);            // N^2
    const f32x4 n2t = mfma_split16(snb, sna, z);           // (N^2)^T
    const Split16 s2 = split16(n2), s2t = split16(n2t);
    const f32x4 n4 = mfma_split16(s2t, s2, z);             // N^4
    const f32x4 n4t = mfma_split16(s2, s2t, z);            // (N^4)^T
    const Split16 s4t = split16(n4t);
    const f32x4 n8 = mfma_split16(s4t, split16(n4), z);     // N^8
    f32x4 acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = (4 * gq + e == ln ? 1.f : 0.f) + n4[e] + n8[e];
    acc = mfma_split16(s4t, split16(n8), acc);             // (I + N^4)(I + N^8)
    acc = mfma_split16(s2t, split16(acc), acc);            // (I + N^2)(I + N^4)(I + N^8)
    const f32x4 t = mfma_split16(split16(-na), split16(acc), acc);   // (I - N)(...)
#pragma unroll
    for (int e = 0; e < 4; ++e) Ab[(16 * ib + 4 * gq + e) * kTA + 16 * ib + ln] = t[e];
}

// One block column JB of the off-diagonal solve of one head's Tm = (I + A)^{-1}:
// Tm_ij = -Tm_ii sum_{k=JB}^{i-1} A_ik Tm_kJB for i = JB+1..3, with 16x16x16
// products on the matrix cores (split fp16 operands, ~fp32 accuracy).  A
// product's accumulator is already the B operand of the next one, so the
// column chain stays in registers.  offcol_load reads the blocks the column
// needs (Tm_JBJB, Tm_ii, A_ik), offcol_solve forms and stores the column's Tm
// blocks over A's; every read of a head's blocks must precede every store.
struct OffCol {
    Split16 tcol[4];   // Tm_{k, JB} in accumulator (= B operand) layout, k >= JB
    f32x4 aik[4][4];   // A_ik, A-operand layout
    f32x4 tii[4];      // Tm_ii, A-operand layout
};

template <int JB>
__device__ __forceinline__ void offcol_load(OffCol& o, const float* A, int gq, int ln) {
    f32x4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = A[(16 * JB + 4 * gq + e) * kTA + 16 * JB + ln];
    o.tcol[JB] = split16(t);
#pragma unroll
    for (int i2 = JB + 1; i2 < 4; ++i2) {
        o.tii[i2] = *reinterpret_cast<const f32x4*>(A + (16 * i2 + ln) * kTA + 16 * i2 + 4 * gq);
#pragma unroll
        for (int kb = JB; kb < i2; ++kb)
            o.aik[i2][kb] = *reinterpret_cast<const f32x4*>(A + (16 * i2 + ln) * kTA + 16 * kb + 4 * gq);
    }
}

template <int JB>
__device__ __forceinline__ void offcol_solve(OffCol& o, float* A, int gq, int ln) {
#pragma unroll
    for (int i2 = JB + 1; i2 < 4; ++i2) {
        f32x4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = JB; kb < i2; ++kb) xs = mfma_split16(split16(o.aik[i2][kb]), o.tcol[kb], xs);
        const f32x4 y = mfma_split16(split16(o.tii[i2]), split16(xs), f32x4{0.f, 0.f, 0.f, 0.f});
        o.tcol[i2] = split16(-y);
#pragma unroll
        for (int e = 0; e < 4; ++e) A[(16 * i2 + 4 * gq + e) * kTA + 16 * JB + ln] = -y[e];
    }
}

// ---------------------------------------------------------------------------
// Stage 1: intra-chunk preparation.  One workgroup per (chunk slot of the
// range slot_lo .. slot_hi - 1, group of kH value heads of one q/k head); 36 KB of LDS
// and at most 128 registers per lane so that four workgroups share a CU.
// The UT transform of each head runs in place in its A buffer: A, then
// Tm = (I + A)^{-1}, read out as the fp16 fragments of Tm diag(beta).
// kStream: the intermediates go out as non-temporal stores.
// ---------------------------------------------------------------------------
template <bool kStream, int kH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void gdn_chunk_prep(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int n_seqs, int h_qk, int h_v, ChunkWorkspace ws, int slot_lo, int slot_hi)
{
    static_assert(kH == 1 || kH == 2, "one or two value heads per workgroup");
    // chunk slot slot_lo + x of the batch; its intermediates go to workspace
    // slot x (the range's own slots)
    const int ls = blockIdx.x;
    const int slot = slot_lo + ls;
    const int h0 = kH * blockIdx.y;                   // the workgroup's first value head
    int seq, t0, len;
    if (slot >= slot_hi || !resolve_slot(cu, n_seqs, slot, seq, t0, len)) return;
    const int j = h0 / ws.group;
    const bool first = h0 % ws.group == 0;            // holds the q/k head's first value head

    // Per head: A buffer (K rows (16 KB bf16) in head 0's and Q rows in the
    // second until the products have read them, then A, then Tm; Q rows in
    // head 0's at the end), beta and G.  Two buffers also at kH = 1.
    __shared__ __attribute__((aligned(16))) float Abuf[kH < 2 ? 2 : kH][kChunk * kTA];
    __shared__ __attribute__((aligned(16))) float Bsh[kH][kChunk];
    __shared__ float Gsh[kH][kChunk];
    __shared__ __attribute__((aligned(16))) float vsink[64];   // target of the value-line touches, never read

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int gq = lane >> 4;
    const int ln = lane & 15;
    float* Ab[kH];
    const float* Gs[kH];
    const float* Bs[kH];
    f16* pdst[kH];
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
        Ab[hh] = Abuf[hh];
        Gs[hh] = Gsh[hh];
        Bs[hh] = Bsh[hh];
        pdst[hh] = ws.p + ws.vunit(ls, h0 + hh) * kPElems;
    }

    // ---- The decay inputs (wave hh for head hh, one lane per position),
    //      loaded first so that their latency hides under the K and Q loads.
    float g_in = 0.f, b_in = 0.f;
    if (wave < kH && lane < len) {
        g_in = g[(size_t)(t0 + lane) * h_v + h0 + wave];
        b_in = beta[(size_t)(t0 + lane) * h_v + h0 + wave];
    }

    // ---- The chunk's K and Q rows, the only global reads of the inputs, by
    //      direct-to-LDS copies of whole rows (bf16, row-major, chunk-swizzled:
    //      K in head 0's A buffer, Q in the second one, both still free), so
    //      that every wave can read the row tiles its Gram rows need and the
    //      K^T fragments can be read from them transposed.  Each wave then
    //      takes its own row tile of K and Q (rows 16 w + ln, dims 32 kk +
    //      8 gq .. +7) into registers.  Pad rows of a short chunk are zero
    //      (they copy the last row, and the owning wave clears them).
    //      Measured against 16-byte register loads of the row tiles: prep at
    //      T = 131072 650 -> 630 us, varlen batch 130 -> 124 us.  The copies
    //      are non-temporal: nothing reads these rows again, and kept in the
    //      caches they would only push out lines the state kernel reads next
    //      (dirty ones among them, written back on the way).  Measured: cold
    //      prep 42 -> 36 us at T = 4000, 122 -> 95 us on the varlen batch,
    //      630 -> 576 us at T = 131072; back-to-back repeats of one layer,
    //      which could reuse cached rows, lose 3 us.
    uint16_t* Kr = reinterpret_cast<uint16_t*>(Abuf[0]);   // [pos][dim] bf16, chunk-swizzled
    bf16x8 kown[4], qf[4];
    {
        uint16_t* Qs = reinterpret_cast<uint16_t*>(Abuf[1]);   // Q rows, until the products
        // wave w copies rows 16 w .. 16 w + 15 of K and Q, four rows (1 KB)
        // per instruction: lane l of copy i takes row r = 16 w + 4 i + l / 16
        // into chunk slot l % 16, i.e. global chunk (l % 16) ^ (r % 16)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * wave + 4 * i + (lane >> 4);
            const int c = (lane & 15) ^ (r & 15);
            const size_t off = ((size_t)(t0 + min(r, len - 1)) * h_qk + j) * kDim + 8 * c;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(k + off),
                                             reinterpret_cast<void*>(Kr + (16 * wave + 4 * i) * kDim), 16, 0,
                                             kCopyNonTemporal);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(q + off),
                                             reinterpret_cast<void*>(Qs + (16 * wave + 4 * i) * kDim), 16, 0,
                                             kCopyNonTemporal);
        }
        __builtin_amdgcn_s_waitcnt(0);
        const int r = 16 * wave + ln;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u16x8 kb = {0, 0, 0, 0, 0, 0, 0, 0};
            u16x8 qb = {0, 0, 0, 0, 0, 0, 0, 0};
            if (r < len) {
                kb = *reinterpret_cast<const u16x8*>(Kr + rsw(r, 4 * kk + gq));
                qb = *reinterpret_cast<const u16x8*>(Qs + rsw(r, 4 * kk + gq));
            } else {
                *reinterpret_cast<u16x8*>(Kr + rsw(r, 4 * kk + gq)) = kb;     // pad rows are zero
            }
            kown[kk] = __builtin_bit_cast(bf16x8, kb);
            qf[kk] = __builtin_bit_cast(bf16x8, qb);
        }
    }
    // ---- decay cumsum (wave hh for head hh, one lane per position) and the
    //      decay vectors
    if (wave < kH) {
        float x = g_in;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float gc = __shfl(x, kChunk - 1, 64);
        const float eg = exp_f(x);
        const float dc = exp_f(gc - x);
        Gsh[wave][lane] = x;
        Bsh[wave][lane] = b_in;
        float* dg = ws.dg + ws.vunit(ls, h0 + wave) * kGElems;
        put<kStream>(&dg[lane], lane == kChunk - 1 ? eg : dc);
        put<kStream>(&dg[kChunk + lane], eg);
    }
    __syncthreads();

    // ---- K^T as A-operand fragments of the state update (which applies the
    //      decay e^{G_C - G} to U' instead): fragment (i, qq) = 2 i + qq, read
    //      transposed from the K rows.  The value heads of a q/k head share
    //      it; the workgroup with the first one writes it.
    if (first) {
        f16* kdst = ws.kt + ws.kunit(ls, j) * kKtElems;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int f = wave + 4 * it;
            put<kStream>(reinterpret_cast<f16x8*>(kdst + ((size_t)f * 64 + lane) * 8), kt_frag(Kr, f >> 1, f & 1, gq, ln));
        }
    }

    // ---- The Gram blocks of A = strictly lower (beta_r e^{G_r-G_s} K K^T) and
    //      P's row tile, balanced over the waves (prep_products); then, once
    //      every wave has read its K tiles from head 0's A buffer, head 0's A
    //      into it.
    f32x4 av[4];
    switch (wave) {
        case 0: prep_products<0, kStream, kH>(av, kown, qf, Kr, Ab, Gs, Bs, pdst, lane, gq, ln); break;
        case 1: prep_products<1, kStream, kH>(av, kown, qf, Kr, Ab, Gs, Bs, pdst, lane, gq, ln); break;
        case 2: prep_products<2, kStream, kH>(av, kown, qf, Kr, Ab, Gs, Bs, pdst, lane, gq, ln); break;
        default: prep_products<3, kStream, kH>(av, kown, qf, Kr, Ab, Gs, Bs, pdst, lane, gq, ln); break;
    }
    // ---- Touch this chunk's value rows of the workgroup's heads (two
    //      128-byte lines per row and head) into the last-level cache with
    //      4-byte direct-to-LDS copies into a sink nobody reads, drained at
    //      the end: the state kernel gathers them on its serial path, where
    //      HBM misses stall the recurrence (measured: 79 -> 60 us for the
    //      recurrence after a cold 4000-token prep).  Issued once the
    //      products are done, so that they stream in under the UT transform,
    //      which makes no global accesses, instead of queueing ahead of the
    //      workgroup's own stores (measured: cold prep 47.8 -> 45.0 us at
    //      T = 4000).  Not with streaming stores: a workspace that large
    //      outgrows the cache before the state kernel gets there.
    if (!kStream && wave == 3) {
        const int row = min(lane, len - 1);
#pragma unroll
        for (int hh = 0; hh < kH; ++hh) {
            const uint16_t* vl = v + ((size_t)(t0 + row) * h_v + h0 + hh) * kDim;
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vl), reinterpret_cast<void*>(vsink), 4, 0, 0);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vl + 64), reinterpret_cast<void*>(vsink), 4, 0, 0);
        }
    }
    __syncthreads();                                  // K rows in head 0's A buffer are consumed
    switch (wave) {
        case 0: store_a<0>(Ab[0], av, gq, ln); break;
        case 1: store_a<1>(Ab[0], av, gq, ln); break;
        case 2: store_a<2>(Ab[0], av, gq, ln); break;
        default: store_a<3>(Ab[0], av, gq, ln); break;
    }
    __syncthreads();

    // ---- Tm = (I + A)^{-1}, blocked by 16, in place, per head.
    //  (1) Diagonal blocks: block i on wave i.
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) diag_inverse(Ab[hh], wave, gq, ln);
    __syncthreads();
    //  (2) Below the diagonal, by block columns (offcol_*): column 0 is a
    //      chain of nine split products, column 1 of five, column 2 of two.
    //      With two heads, waves 0 and 1 take column 0 of head 0 and head 1,
    //      waves 2 and 3 columns 1 and 2 of head 0 and head 1, so that no
    //      wave runs more than one nine-product chain; with one head, wave j
    //      takes column j.
    {
        OffCol oa, ob;
        if constexpr (kH == 2) {
            switch (wave) {
                case 0: offcol_load<0>(oa, Ab[0], gq, ln); break;
                case 1: offcol_load<0>(oa, Ab[1], gq, ln); break;
                case 2: offcol_load<1>(oa, Ab[0], gq, ln); offcol_load<2>(ob, Ab[0], gq, ln); break;
                default: offcol_load<1>(oa, Ab[1], gq, ln); offcol_load<2>(ob, Ab[1], gq, ln); break;
            }
            __syncthreads();
            switch (wave) {
                case 0: offcol_solve<0>(oa, Ab[0], gq, ln); break;
                case 1: offcol_solve<0>(oa, Ab[1], gq, ln); break;
                case 2: offcol_solve<1>(oa, Ab[0], gq, ln); offcol_solve<2>(ob, Ab[0], gq, ln); break;
                default: offcol_solve<1>(oa, Ab[1], gq, ln); offcol_solve<2>(ob, Ab[1], gq, ln); break;
            }
        } else {
            switch (wave) {
                case 0: offcol_load<0>(oa, Ab[0], gq, ln); break;
                case 1: offcol_load<1>(oa, Ab[0], gq, ln); break;
                case 2: offcol_load<2>(oa, Ab[0], gq, ln); break;
                default: break;
            }
            __syncthreads();
            switch (wave) {
                case 0: offcol_solve<0>(oa, Ab[0], gq, ln); break;
                case 1: offcol_solve<1>(oa, Ab[0], gq, ln); break;
                case 2: offcol_solve<2>(oa, Ab[0], gq, ln); break;
                default: break;
            }
        }
    }
    __syncthreads();

    // ---- TU = Tm diag(beta) as A fragments over positions of its six nonzero
    //      (row tile, K-step) blocks, in the order of P's: wave w writes row
    //      tile w.  Entry (r, s) = Tm[r][s] beta_s for s <= r; blocks above the
    //      diagonal block are zero (the A buffer holds leftovers there), and
    //      inside a diagonal block the inverse is exactly lower triangular
    //      (every power of a strictly lower N is strictly lower).  The state
    //      kernel forms W = TU diag(e^G) K and U = TU V on chip from these
    //      6 KB, the K^T fragments and the value rows.
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
        const int pt = wave;
        const int r = 16 * pt + ln;
        f16* tdst = ws.tu + ws.vunit(ls, h0 + hh) * kTuElems;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            if (qq == 1 && pt < 2) continue;          // blocks (0, 1) and (1, 1) are zero
            const int f = pt < 2 ? pt : 2 + 2 * (pt - 2) + qq;
            f16x8 fr;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int s0 = 32 * qq + 16 * half + 4 * gq;      // slots 4 half .. 4 half + 3
                const bool live = (s0 >> 4) <= pt;
                const f32x4 t = live ? *reinterpret_cast<const f32x4*>(Ab[hh] + r * kTA + s0) : f32x4{0.f, 0.f, 0.f, 0.f};
                const f32x4 b = *reinterpret_cast<const f32x4*>(Bs[hh] + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) fr[4 * half + e] = static_cast<f16>(t[e] * b[e]);
            }
            put<kStream>(reinterpret_cast<f16x8*>(tdst + ((size_t)f * 64 + lane) * 8), fr);
        }
    }

    // ---- Q as A fragments over the chunk state's d_k slots, (p, qq = wave),
    //      for the output stage's Q H0; the value heads of a q/k head share
    //      them and the workgroup with the first one writes them.  The rows
    //      go through LDS (head 0's A buffer, free once TU has been read out
    //      of it) because a lane's slots span two 16-dim runs held by
    //      different lanes.
    if (first) {
        __syncthreads();                              // every read of head 0's Tm is done
        uint16_t* Qr = reinterpret_cast<uint16_t*>(Abuf[0]);   // [pos][dim] bf16, chunk-swizzled
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            *reinterpret_cast<u16x8*>(Qr + rsw(16 * wave + ln, 4 * kk + gq)) = __builtin_bit_cast(u16x8, qf[kk]);
        __syncthreads();
        f16* qdst = ws.qf + ws.kunit(ls, j) * kQfElems;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = 16 * p + ln;
            const int d0 = 32 * wave + 4 * gq;        // slots 0..3
            const int d1 = d0 + 16;                   // slots 4..7
            const u16x4 lo = *reinterpret_cast<const u16x4*>(Qr + rsw(row, d0 >> 3) + (d0 & 7));
            const u16x4 hi = *reinterpret_cast<const u16x4*>(Qr + rsw(row, d1 >> 3) + (d1 & 7));
            f16x8 fr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fr[e] = static_cast<f16>(bf16_to_f32(lo[e]));
                fr[e + 4] = static_cast<f16>(bf16_to_f32(hi[e]));
            }
            put<kStream>(reinterpret_cast<f16x8*>(qdst + ((p * 4 + wave) * 64 + lane) * 8), fr);
        }
    }
    // drain the value-line touches before the workgroup's LDS goes away
    if (!kStream && wave == 3) __builtin_amdgcn_s_waitcnt(0);
}

// Grid width of a prep launch: the chunk slots rounded up to a multiple of 8.
// Workgroup (slot, y) has the linear index slot + width * y and runs on XCD
// index % 8, so with the width a multiple of 8 every value head of a chunk
// slot runs on the same XCD, and the value heads of a q/k head, which read
// the same q and k rows, share that XCD's L2.  The padding workgroups find
// no chunk and leave at once.
__host__ __forceinline__ unsigned slots_x8(int n_slots) { return ((unsigned)n_slots + 7u) & ~7u; }

// Value heads per prep workgroup (prep_value_heads in gdn_sizes.h).
__host__ __forceinline__ int prep_heads(int h_qk, int h_v) { return prep_value_heads(h_qk, h_v); }

}  // namespace

}  // namespace gdn

// Stage 1 of the chunked Gated DeltaNet prefill for gfx950: intra-chunk
// preparation (the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page, section 2,
// first of its three stages).  Per chunk of 64 positions and value head it
// forms the decay cumsum, A = strictly-lower(beta_r e^{G_r-G_s} K K^T), the UT
// transform Tm = (I + A)^{-1}, TU = Tm diag(beta) and P = M o Q K^T, and
// writes them, with the fp16 K^T and Q of each q/k head, in the matrix-core
// fragment order the state kernel reads.  W = TU diag(e^G) K and U = TU V are
// formed by the state kernel on chip (the algebra is restated in
// gdn_chunk.hip): 6 KB of TU per chunk and value head instead of 32 KB of W
// and U through memory, and prep no longer reads V.
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

// Transposed [dim][pos] fp16 tiles, 64 positions per row, no padding.  Rows
// are written one position per lane, four dims 8 apart at a time, and read as
// 16-byte runs of 8 positions, 16 consecutive dims at a time.  XOR-ing the
// position's 8-block index (bits 3-5) with (d & 7) ^ 2 ((d >> 3) & 3) keeps
// every 8-aligned run contiguous, puts the four written rows on different
// banks and gives eight consecutive read rows eight different 8-blocks.
__device__ __forceinline__ int tsw(int d, int t) {
    return d * kChunk + (t ^ ((((d & 7) ^ (((d >> 3) & 3) << 1)) & 7) << 3));
}

// Row-major [pos][dim] bf16 tiles, 128 dims per row, no padding: 16-byte
// chunk c (dims 8 c .. 8 c + 7) of row r sits at chunk c ^ (r % 16), so the
// 16 rows read at the same dims by a fragment load hit 16 different banks.
// Returns the element offset of chunk c of row r.
__device__ __forceinline__ int rsw(int r, int c) {
    return r * kDim + ((c ^ (r & 15)) << 3);
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

// The products of wave W: the A values of its Gram blocks into av (A_rs for
// rows r = 16 p + 4 gq + e, column s = 16 jt + ln; 0 for s >= r), and P's
// row tile W, stored to pdst.  K row tiles come from Kr (row-major bf16,
// chunk-swizzled), the wave's own from kown.
template <int W, bool kStream>
__device__ __forceinline__ void prep_products(f32x4 (&av)[4], const bf16x8 (&kown)[4], const bf16x8 (&qf)[4],
                                              const uint16_t* Kr, const float* Gs, const float* Bs, f16* pdst,
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
        const int s = 16 * jt + ln;
        const float gsv = Gs[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * p + 4 * gq + e;
            av[i][e] = (s < r) ? Bs[r] * exp_f(Gs[r] - gsv) * acc[e] : 0.f;
        }
    }
    // P = M o (Q K^T) for row tile W, M_rs = e^{G_r - G_s} (s <= r), computed
    // as (K Q^T)[s][r] so that the accumulators of two position tiles stack
    // into the A fragment of P over position slots, which is how the output
    // stage reads it: block (p, qq) at 2 p (p < 2) or 2 + 2 (p - 2) + qq;
    // blocks (0, 1) and (1, 1) are zero and not stored.
    const int r = 16 * W + ln;
    const float gr = Gs[r];
    f32x4 dt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        dt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (jt > W) continue;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) dt[jt] = mfma_bf16(kt[jt][kk], qf[kk], dt[jt]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int sp = 16 * jt + 4 * gq + e;
            dt[jt][e] = (sp <= r) ? exp_f(gr - Gs[sp]) * dt[jt][e] : 0.f;
        }
    }
    constexpr int f0 = W < 2 ? W : 2 * W - 2;
    put<kStream>(reinterpret_cast<f16x8*>(pdst + ((size_t)f0 * 64 + lane) * 8), cat_to_f16(dt[0], dt[1]));
    if constexpr (W >= 2)
        put<kStream>(reinterpret_cast<f16x8*>(pdst + ((size_t)(f0 + 1) * 64 + lane) * 8), cat_to_f16(dt[2], dt[3]));
}

// A values of wave W's Gram blocks into the A buffer (row stride kTA); a
// diagonal block goes transposed to its place above the diagonal.
template <int W>
__device__ __forceinline__ void store_a(float* Ab, const f32x4 (&av)[4], int gq, int ln) {
    using B = GramBlocks<W>;
#pragma unroll
    for (int i = 0; i < B::n; ++i) {
        const int p = B::p[i], jt = B::jt[i];
        if (jt < p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Ab[(16 * p + 4 * gq + e) * kTA + 16 * jt + ln] = av[i][e];
        } else {
            *reinterpret_cast<f32x4*>(Ab + (16 * diag_row_block(p) + ln) * kTA + 16 * diag_col_block(p) + 4 * gq) = av[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Stage 1: intra-chunk preparation.  One workgroup per (chunk slot, value
// head); 35 KB of LDS and at most 128 registers per lane so that four
// workgroups share a CU.  The UT transform runs in place in the A buffer: A,
// then Tm = (I + A)^{-1}, read out as the fp16 fragments of Tm diag(beta).
// kStream: the intermediates go out as non-temporal stores.
// ---------------------------------------------------------------------------
template <bool kStream>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void gdn_chunk_prep(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int n_seqs, int h_qk, int h_v, ChunkWorkspace ws)
{
    const int slot = blockIdx.x;
    const int h = blockIdx.y;
    int seq, t0, len;
    if (!resolve_slot(cu, n_seqs, slot, seq, t0, len)) return;
    const int j = h / (h_v / h_qk);

    // K^T [dim][pos] (swizzled), then Q rows: one buffer, so that four
    // workgroups (35 KB of LDS each) share a CU
    __shared__ __attribute__((aligned(16))) f16 KsT[kDim * kChunk];
    __shared__ __attribute__((aligned(16))) float Ab[kChunk * kTA];  // K rows (16 KB), then A, then Tm
    __shared__ __attribute__((aligned(16))) float Bs[kChunk];  // beta
    __shared__ float Gs[kChunk];     // G
    __shared__ __attribute__((aligned(16))) float vsink[64];   // target of the value-line touches, never read

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int gq = lane >> 4;
    const int ln = lane & 15;
    const size_t wsidx = ws.vunit(slot, h);

    // ---- This wave's row tile of K and Q (rows 16 w + ln, dims 32 kk + 8 gq
    //      .. +7), the only global reads of the inputs: K goes to LDS
    //      row-major (bf16, in the A buffer, which is still free) so that every
    //      wave can read the row tiles its Gram rows need, and, for the first
    //      value head of a q/k head, which writes the K^T fragments,
    //      transposed (fp16).  Q stays in registers.  Pad rows are zero.
    uint16_t* Kr = reinterpret_cast<uint16_t*>(Ab);   // [pos][dim] bf16, chunk-swizzled
    // ---- Touch this chunk's value rows of head h (two 128-byte lines per
    //      row) into the last-level cache with 4-byte direct-to-LDS copies
    //      into a sink nobody reads, drained at the end: the state kernel
    //      gathers them on its serial path, where HBM misses stall the
    //      recurrence (measured: 79 -> 60 us for the recurrence after a cold
    //      4000-token prep).  Not with streaming stores: a workspace that
    //      large outgrows the cache before the state kernel gets there.
    if (!kStream && wave == 3) {
        const int row = min(lane, len - 1);
        const uint16_t* vl = v + ((size_t)(t0 + row) * h_v + h) * kDim;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vl), reinterpret_cast<void*>(vsink), 4, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vl + 64), reinterpret_cast<void*>(vsink), 4, 0, 0);
    }
    bf16x8 kown[4], qf[4];
    {
        const int r = 16 * wave + ln;
        const size_t krow = ((size_t)(t0 + r) * h_qk + j) * kDim;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u16x8 kb = {0, 0, 0, 0, 0, 0, 0, 0};
            u16x8 qb = {0, 0, 0, 0, 0, 0, 0, 0};
            if (r < len) {
                kb = *reinterpret_cast<const u16x8*>(k + krow + 32 * kk + 8 * gq);
                qb = *reinterpret_cast<const u16x8*>(q + krow + 32 * kk + 8 * gq);
            }
            kown[kk] = __builtin_bit_cast(bf16x8, kb);
            qf[kk] = __builtin_bit_cast(bf16x8, qb);
            *reinterpret_cast<u16x8*>(Kr + rsw(r, 4 * kk + gq)) = kb;
            if (h % ws.group == 0) {
                const f16x8 kt8 = bf16x8_to_f16x8(kb);
#pragma unroll
                for (int e = 0; e < 8; ++e) KsT[tsw(32 * kk + 8 * gq + e, r)] = kt8[e];
            }
        }
    }
    // ---- decay cumsum (wave 0, one lane per position) and the decay vectors
    if (wave == 0) {
        const bool in = lane < len;
        float x = in ? g[(size_t)(t0 + lane) * h_v + h] : 0.f;
        const float bt = in ? beta[(size_t)(t0 + lane) * h_v + h] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float gc = __shfl(x, kChunk - 1, 64);
        const float eg = exp_f(x);
        const float dc = exp_f(gc - x);
        Gs[lane] = x;
        Bs[lane] = bt;
        put<kStream>(&ws.dg[wsidx * kGElems + lane], lane == kChunk - 1 ? eg : dc);
        put<kStream>(&ws.dg[wsidx * kGElems + kChunk + lane], eg);
    }
    __syncthreads();

    // ---- K^T as A-operand fragments of the state update (which applies the
    //      decay e^{G_C - G} to U' instead): fragment (i, qq), lane (gq, ln) =
    //      K[p][16 i + ln] at the position slots p(gq, s) of K-step qq.  The
    //      value heads of a q/k head share it; the first one writes it.
    if (h % ws.group == 0) {
        f16* kdst = ws.kt + ws.kunit(slot, j) * kKtElems;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int f = wave + 4 * it;          // fragment index i * 2 + qq
            const int i = f >> 1, qq = f & 1;
            const int d = 16 * i + ln;
            const f16x4 lo = *reinterpret_cast<const f16x4*>(KsT + tsw(d, 32 * qq + 4 * gq));
            const f16x4 hi = *reinterpret_cast<const f16x4*>(KsT + tsw(d, 32 * qq + 16 + 4 * gq));
            const f16x8 fr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            put<kStream>(reinterpret_cast<f16x8*>(kdst + ((size_t)f * 64 + lane) * 8), fr);
        }
    }

    // ---- The Gram blocks of A = strictly lower (beta_r e^{G_r-G_s} K K^T) and
    //      P's row tile, balanced over the waves (prep_products); then, once
    //      every wave has read its K tiles from the A buffer, A into it.
    f32x4 av[4];
    switch (wave) {
        case 0: prep_products<0, kStream>(av, kown, qf, Kr, Gs, Bs, ws.p + wsidx * kPElems, lane, gq, ln); break;
        case 1: prep_products<1, kStream>(av, kown, qf, Kr, Gs, Bs, ws.p + wsidx * kPElems, lane, gq, ln); break;
        case 2: prep_products<2, kStream>(av, kown, qf, Kr, Gs, Bs, ws.p + wsidx * kPElems, lane, gq, ln); break;
        default: prep_products<3, kStream>(av, kown, qf, Kr, Gs, Bs, ws.p + wsidx * kPElems, lane, gq, ln); break;
    }
    __syncthreads();                                  // K rows in the A buffer are consumed
    switch (wave) {
        case 0: store_a<0>(Ab, av, gq, ln); break;
        case 1: store_a<1>(Ab, av, gq, ln); break;
        case 2: store_a<2>(Ab, av, gq, ln); break;
        default: store_a<3>(Ab, av, gq, ln); break;
    }
    __syncthreads();

    // ---- Tm = (I + A)^{-1}, blocked by 16, in place.
    //  (1) Diagonal blocks Tm_ii = (I + A_ii)^{-1}: wave i, lane c % 16 holds
    //      column c of x = (I + A_ii)^{-1} e_c.  Forward substitution by
    //      columns of A_ii: once x_t is final, x_r -= A_rt x_t for r > t (each
    //      x_r sees the same subtractions in the same order as the row form).
    {
        const int ib = wave;
        const float* at = Ab + 16 * diag_row_block(ib) * kTA + 16 * diag_col_block(ib);   // at[t * kTA + r] = A_ii[r][t]
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
        for (int t = 0; t < 15; ++t) {
            float col[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 c4 = *reinterpret_cast<const f32x4*>(at + t * kTA + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) col[4 * q4 + e] = c4[e];
            }
#pragma unroll
            for (int r = t + 1; r < 16; ++r) x[r] -= col[r] * x[t];
        }
        if (gq == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Ab[(16 * ib + r) * kTA + 16 * ib + ln] = x[r];
        }
    }
    __syncthreads();
    //  (2) Below the diagonal, block column j on wave j, rows i = j+1..3:
    //      Tm_ij = -Tm_ii sum_{k=j}^{i-1} A_ik Tm_kj, with 16x16x16 products on
    //      the matrix cores (split fp16 operands, ~fp32 accuracy).  A product's
    //      accumulator is already the B operand of the next one, so the column
    //      chain stays in registers.  Every A_ik a wave needs is read before
    //      any wave overwrites A blocks with Tm blocks.
    Split16 tcol[4];   // Tm_{k, jb} in accumulator (= B operand) layout, k >= jb
    f32x4 aik[4][4];   // A_ik, A-operand layout
    f32x4 tii[4];      // Tm_ii, A-operand layout
    const int jb = wave;
    if (wave < 3) {
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) {
            if (kb != jb) continue;
            f32x4 t;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = Ab[(16 * kb + 4 * gq + e) * kTA + 16 * kb + ln];
            tcol[kb] = split16(t);
        }
#pragma unroll
        for (int i2 = 1; i2 < 4; ++i2) {
            if (i2 <= jb) continue;
            tii[i2] = *reinterpret_cast<const f32x4*>(Ab + (16 * i2 + ln) * kTA + 16 * i2 + 4 * gq);
#pragma unroll
            for (int kb = 0; kb < i2; ++kb) {
                if (kb < jb) continue;
                aik[i2][kb] = *reinterpret_cast<const f32x4*>(Ab + (16 * i2 + ln) * kTA + 16 * kb + 4 * gq);
            }
        }
    }
    __syncthreads();
    if (wave < 3) {
#pragma unroll
        for (int i2 = 1; i2 < 4; ++i2) {
            if (i2 <= jb) continue;
            f32x4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < i2; ++kb) {
                if (kb < jb) continue;
                xs = mfma_split16(split16(aik[i2][kb]), tcol[kb], xs);
            }
            const f32x4 y = mfma_split16(split16(tii[i2]), split16(xs), f32x4{0.f, 0.f, 0.f, 0.f});
            tcol[i2] = split16(-y);
#pragma unroll
            for (int e = 0; e < 4; ++e) Ab[(16 * i2 + 4 * gq + e) * kTA + 16 * jb + ln] = -y[e];
        }
    }
    __syncthreads();

    // ---- TU = Tm diag(beta) as A fragments over positions of its six nonzero
    //      (row tile, K-step) blocks, in the order of P's: wave w writes row
    //      tile w.  Entry (r, s) = Tm[r][s] beta_s for s <= r; blocks above the
    //      diagonal block are zero (the A buffer holds leftovers there), and
    //      inside a diagonal block the solve left exact zeros above the
    //      diagonal.  The state kernel forms W = TU diag(e^G) K and U = TU V on
    //      chip from these 6 KB, the K^T fragments and the value rows.
    {
        const int pt = wave;
        const int r = 16 * pt + ln;
        f16* tdst = ws.tu + wsidx * kTuElems;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            if (qq == 1 && pt < 2) continue;          // blocks (0, 1) and (1, 1) are zero
            const int f = pt < 2 ? pt : 2 + 2 * (pt - 2) + qq;
            f16x8 fr;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int s0 = 32 * qq + 16 * half + 4 * gq;      // slots 4 half .. 4 half + 3
                const bool live = (s0 >> 4) <= pt;
                const f32x4 t = live ? *reinterpret_cast<const f32x4*>(Ab + r * kTA + s0) : f32x4{0.f, 0.f, 0.f, 0.f};
                const f32x4 b = *reinterpret_cast<const f32x4*>(Bs + s0);
#pragma unroll
                for (int e = 0; e < 4; ++e) fr[4 * half + e] = static_cast<f16>(t[e] * b[e]);
            }
            put<kStream>(reinterpret_cast<f16x8*>(tdst + ((size_t)f * 64 + lane) * 8), fr);
        }
    }

    // ---- Q as A fragments over the chunk state's d_k slots, (p, qq = wave),
    //      for the output stage's Q H0; the value heads of a q/k head share
    //      them and the first one writes them.  The rows go through LDS (in
    //      the K^T space, free once the fragments above have been read) because
    //      a lane's slots span two 16-dim runs held by different lanes.
    if (h % ws.group == 0) {
        __syncthreads();                              // every read of K^T is done
        uint16_t* Qr = reinterpret_cast<uint16_t*>(KsT);   // [pos][dim] bf16, chunk-swizzled
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            *reinterpret_cast<u16x8*>(Qr + rsw(16 * wave + ln, 4 * kk + gq)) = __builtin_bit_cast(u16x8, qf[kk]);
        __syncthreads();
        f16* qdst = ws.qf + ws.kunit(slot, j) * kQfElems;
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
// Workgroup (slot, h) has the linear index slot + width * h and runs on XCD
// index % 8, so with the width a multiple of 8 every value head of a chunk
// slot runs on the same XCD, and the value heads of a q/k head, which read
// the same q and k rows, share that XCD's L2.  The padding workgroups find
// no chunk and leave at once.
__host__ __forceinline__ unsigned slots_x8(int n_slots) { return ((unsigned)n_slots + 7u) & ~7u; }

}  // namespace

}  // namespace gdn

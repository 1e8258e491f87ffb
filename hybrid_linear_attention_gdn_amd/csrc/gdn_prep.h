// Stage 1 of the chunked Gated DeltaNet prefill for gfx950: intra-chunk
// preparation (the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page, section 2,
// first of its three stages).  Per chunk of 64 positions and value head it
// forms the decay cumsum, A = strictly-lower(beta_r e^{G_r-G_s} K K^T), the UT
// transform Tm = (I + A)^{-1}, W = Tm diag(beta e^G) K, U = Tm diag(beta) V
// and P = M o Q K^T, and writes them in the matrix-core fragment order the
// state kernel reads (the algebra is restated in gdn_chunk.hip).
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

constexpr int kTS = 72;   // LDS row stride (halves) of 64-wide fp16 tiles
// LDS row stride (floats) of the fp32 64 x 64 A / Tm: rows 4 apart (the rows
// of one accumulator store) fall 16 banks apart
constexpr int kTA = 68;
constexpr int kQS = 136;  // LDS row stride (halves) of 128-wide tiles

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
// then Tm = (I + A)^{-1}, then the fp16 rows of Tm diag(beta e^G) and
// Tm diag(beta).  kStream: the intermediates go out as non-temporal stores.
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

    // K^T [dim][pos] (swizzled), then V^T, then Q rows: one buffer, so that
    // four workgroups (35 KB of LDS each) share a CU
    __shared__ __attribute__((aligned(16))) f16 KsT[kDim * kChunk];
    __shared__ __attribute__((aligned(16))) float Ab[kChunk * kTS];  // A, then Tm, then TW | TU
    __shared__ __attribute__((aligned(16))) float Bs[kChunk];  // beta
    __shared__ __attribute__((aligned(16))) float Bw[kChunk];  // beta e^G
    __shared__ float Gs[kChunk];     // G

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int gq = lane >> 4;
    const int ln = lane & 15;
    const size_t wsidx = ws.vunit(slot, h);

    // ---- This wave's row tile of K, Q and V (rows 16 w + ln, dims 32 kk +
    //      8 gq .. +7), the only global reads of the inputs: K and V go to LDS
    //      transposed (fp16) for the products over positions; K also goes to
    //      LDS row-major (bf16, in the A buffer, which is still free) so that
    //      every wave can read the row tiles its Gram rows need.  Q stays in
    //      registers.  V is loaded after the UT transform, into the K^T space
    //      once W has been formed.  Pad rows are zero.
    uint16_t* Kr = reinterpret_cast<uint16_t*>(Ab);   // [pos][dim] bf16, chunk-swizzled
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
            const f16x8 kt8 = bf16x8_to_f16x8(kb);
#pragma unroll
            for (int e = 0; e < 8; ++e) KsT[tsw(32 * kk + 8 * gq + e, r)] = kt8[e];
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
        Bw[lane] = bt * eg;
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

    // ---- TW = Tm diag(beta e^G), TU = Tm diag(beta) as fp16, in place; blocks
    //      above the diagonal are zero.
    f16* TWs = reinterpret_cast<f16*>(Ab);          // [pos][t]
    f16* TUs = TWs + kChunk * kTS;                  // [pos][t]
    {
        // thread: row r = idx / 16, columns t .. t + 3 (one 16-block)
        f32x4 tv[4];
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx >> 4, t = (idx & 15) * 4;
            tv[it] = ((t >> 4) > (r >> 4)) ? f32x4{0.f, 0.f, 0.f, 0.f}
                                            : *reinterpret_cast<const f32x4*>(Ab + r * kTA + t);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int idx = tid + 256 * it;
            const int r = idx >> 4, t = (idx & 15) * 4;
            const f32x4 bw = *reinterpret_cast<const f32x4*>(Bw + t);
            const f32x4 bs = *reinterpret_cast<const f32x4*>(Bs + t);
            f16x4 tw, tu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tw[e] = static_cast<f16>(tv[it][e] * bw[e]);
                tu[e] = static_cast<f16>(tv[it][e] * bs[e]);
            }
            *reinterpret_cast<f16x4*>(TWs + r * kTS + t) = tw;
            *reinterpret_cast<f16x4*>(TUs + r * kTS + t) = tu;
        }
    }
    __syncthreads();

    // ---- W = TW K (positions on lanes), then U = TU V (d_v on lanes), with V^T
    //      in the K^T space in between.  Wave w owns d_k tiles 2w, 2w+1 and
    //      d_v tiles 2w, 2w+1.
    {
        f32x4 wacc[2][4];   // W^T[d_k tile 2w + a][pos tile p]: positions on lanes
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int p = 0; p < 4; ++p) wacc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f16x8 kfr[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                kfr[a] = *reinterpret_cast<const f16x8*>(KsT + tsw(16 * (2 * wave + a) + ln, 32 * kt + 8 * gq));
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f16x8 tw = *reinterpret_cast<const f16x8*>(TWs + (16 * p + ln) * kTS + 32 * kt + 8 * gq);
#pragma unroll
                for (int a = 0; a < 2; ++a) wacc[a][p] = mfma_f16(kfr[a], tw, wacc[a][p]);
            }
        }
        // -W fragments (p, qq = wave): stacked d_k tiles 2w, 2w+1 of W^T
        f16* wdst = ws.w + wsidx * kWElems;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f16x8 fr = cat_to_f16(-wacc[0][p], -wacc[1][p]);
            put<kStream>(reinterpret_cast<f16x8*>(wdst + ((p * 4 + wave) * 64 + lane) * 8), fr);
        }
    }
    // ---- This wave's row tile of V, loaded after W (out of the register peak
    //      of the W products; the other workgroups on the CU cover the wait)
    //      and written to LDS once every wave is done with K^T.
    u16x8 vrow[4];
    {
        const int r = 16 * wave + ln;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            vrow[kk] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (r < len) vrow[kk] = *reinterpret_cast<const u16x8*>(v + ((size_t)(t0 + r) * h_v + h) * kDim + 32 * kk + 8 * gq);
        }
    }
    __syncthreads();                                  // every read of K^T is done
    f16* VsT = KsT;                                   // V^T [dim][pos], swizzled
    {
        const int r = 16 * wave + ln;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const f16x8 vt8 = bf16x8_to_f16x8(vrow[kk]);
#pragma unroll
            for (int e = 0; e < 8; ++e) VsT[tsw(32 * kk + 8 * gq + e, r)] = vt8[e];
        }
    }
    __syncthreads();
    {
        f32x4 uacc[4][2];   // U[pos tile p][d_v tile 2w + a]: d_v on lanes
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int p = 0; p < 4; ++p) uacc[p][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f16x8 vfr[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                vfr[a] = *reinterpret_cast<const f16x8*>(VsT + tsw(16 * (2 * wave + a) + ln, 32 * kt + 8 * gq));
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const f16x8 tu = *reinterpret_cast<const f16x8*>(TUs + (16 * p + ln) * kTS + 32 * kt + 8 * gq);
#pragma unroll
                for (int a = 0; a < 2; ++a) uacc[p][a] = mfma_f16(tu, vfr[a], uacc[p][a]);
            }
        }
        // U accumulator fragments (ct, p)
        f16* udst = ws.u + wsidx * kUElems;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int ct = 2 * wave + a;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f16x4 fr;
#pragma unroll
                for (int e = 0; e < 4; ++e) fr[e] = static_cast<f16>(uacc[p][a][e]);
                put<kStream>(reinterpret_cast<f16x4*>(udst + ((ct * 4 + p) * 64 + lane) * 4), fr);
            }
        }
    }

    // ---- Q as A fragments over the chunk state's d_k slots, (p, qq = wave),
    //      for the output stage's Q H0; the value heads of a q/k head share
    //      them and the first one writes them.  The rows go through LDS (in
    //      the K^T / V^T space, free once the products above have read it) because
    //      a lane's slots span two 16-dim runs held by different lanes.
    if (h % ws.group == 0) {
        __syncthreads();                              // every read of V^T is done
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

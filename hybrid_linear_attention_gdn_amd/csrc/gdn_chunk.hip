// Chunked Gated DeltaNet prefill for gfx950, chunk length 64.
//
// The stages follow the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page,
// section 2 ("GDN prefill"): intra-chunk preparation, inter-chunk state
// recurrence with the state resident in matrix-core accumulators and the
// next chunk prefetched, and the output, which here runs inside the
// recurrence's workgroups (two kernels; a segment scan for the
// chunk-parallel path).  The chunkwise algebra (state
// H = S^T, d_k x d_v; chunk positions r, s; incoming state H0):
//
//   G_r  = sum_{t<=r} g_t              A_rs = beta_r e^{G_r-G_s} k_r.k_s  (s < r)
//   Tm   = (I + A)^{-1}                W = Tm diag(beta e^G) K,  U = Tm diag(beta) V
//   U'   = U - W H0                    H_C = e^{G_C} H0 + K^T diag(e^{G_C-G}) U'
//   O    = diag(e^G) Q H0 + (M o Q K^T) U',   M_rs = e^{G_r-G_s} (s <= r)
//
// Every exponent is a difference G_r - G_s with s <= r, hence <= 0.
//
// Prep's results live in the caller's workspace in matrix-core fragment
// order, written exactly as their consumers' operands need: Tm diag(beta)
// (TU), from which the state kernel forms -W (A fragments of W H0) and U
// on chip; K^T as A fragments of the state update; Q and P as A fragments
// of the output's (Q H0) and (P U'); the decay vectors.  Within the state
// kernel the chain wave hands the chunk state H0 and U' to the output wave
// through LDS, as B fragments of (Q H0) and (P U').
// Contraction slot maps (lane group gq = lane / 16, slot s = 0..7):
//   dim a(gq, s)   = 32 qq + 16 (s / 4) + 4 gq + s % 4   for K-step qq over d_k
//   pos p(gq, s)   = 32 qq + 16 (s / 4) + 4 gq + s % 4   for K-step qq over positions
// which is exactly how two stacked 16x16 accumulator tiles sit in a lane.
//
// Stage 1 (prep) is in gdn_prep.h; this file holds the state recurrence with
// the output, the segment scan and the host-side launch of the prefill.

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

// ---------------------------------------------------------------------------
// Stage 2: inter-chunk state recurrence with the output.  One workgroup per
// (sequence, value head, 16-column tile), its waves specialised:
//   * the chain wave keeps the tile's 128 x 16 slice of the state in
//     accumulator registers (8 tiles of 16 d_k rows) for the whole sequence.
//     Per chunk it runs the 32 matrix-core products of U' = U - W H0 and
//     H_C = e^{G_C} H0 + K^T D U', the dependency from chunk to chunk (-W and
//     U from the W wave, K^T and the decay vector from the copy ring, all in
//     LDS), and hands U' and the new state, rounded to fp16 as B operands, to
//     the output wave through double-buffered LDS slots;
//   * the output wave forms O = diag(e^G) (Q H0) + P U' on its own SIMD:
//     the Q H0 half in the interval of the chunk (Q fragments by register
//     loads one interval ahead, e^G from the ring), the P U' half one
//     interval later, when U' has been handed over (P by register loads in
//     the chunk's interval); it stores O to global memory;
//   * two W waves (one for a tile pair) form, one chunk ahead of the chain,
//     -W = -TU diag(e^G) K (48 products: -W^T = K^T (TU diag(-e^G))^T from
//     the K^T and TU fragments in the ring) and the tile's U = TU V (six
//     products from the tile's value rows in the ring, read transposed),
//     each wave about half of both, so that W and U, 32 KB per chunk and
//     value head, never go through memory: prep stores only the 6 KB of TU;
//   * the copy wave issues direct global-to-LDS copies of K^T, TU, the decay
//     vectors and the tile's value rows into a ring of kStages stages, and
//     touches the operands of a chunk two beyond those (Q and P included)
//     into L2.
// The waves meet at one barrier per chunk.  The copy wave issues a fixed
// number of copies per chunk, so one memory-counter wait makes a stage ready
// before that barrier.  The eight tiles of a head run on one XCD so that its
// L2 serves the shared fragments.  An affine map has no output: its
// workgroups have chain, W and copy waves.  When a batch has more tiles
// than the GPU has CUs, so that the workgroups run in rounds, a workgroup
// takes a pair of adjacent tiles: two chain waves on two SIMDs share the
// ring and the W wave's -W (the W wave forms both tiles' U), and one output
// wave forms both tiles' output from one set of Q and P fragments, which
// halves the operand traffic per tile and the number of rounds.
// ---------------------------------------------------------------------------
constexpr int kVRowElems = 16;                               // halves of one tile's row of V
constexpr int kHbElems = 4 * 64 * 8;                         // halves of the state's four B fragments
constexpr int kUbElems = 2 * 64 * 8;                         // halves of U''s two B fragments
constexpr int kUaccElems = 4 * 64 * 4;                       // floats of a tile's U accumulators

template <int kChains>
struct StateStage {
    static constexpr int kTiles = kChains;
    f16 k[kKtElems];                                         // K^T A fragments
    f16 tu[kTuElems];                                        // TU fragments
    float dg[kGElems];        // e^{G_C - G_r} (r < 63) and e^{G_C} in entry 63; then e^{G_r}
    uint16_t v[kChains][kChunk * kVRowElems];                // the tiles' value rows, bf16 [pos][16]
};

// Copies per chunk: 1 KB pieces (16 B per lane) of K^T (16) and TU (6), the
// two 256 B decay vectors (4 B per lane), and per tile the 64 value rows of
// 32 B (two 16-byte halves per row, 32 rows per copy).
template <int kChains>
constexpr int copies_per_chunk() { return 16 + 6 + 2 + 2 * kChains; }

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Wait for this wave's LDS operations, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Where one chunk's operands come from.  vu / ku: workspace units of the
// value head and of its q/k head; vrow: the chunk's first token row of v
// (value head h, column 0); len: its valid rows.
struct ChunkSrc {
    size_t vu, ku;
    const uint16_t* vrow;
    int len;
};

// One chunk's copies into a stage.  Value rows past the chunk's end read its
// last valid row instead: TU's columns for those positions are zero, so they
// contribute nothing, and no read leaves the sequence.
template <typename Stage>
__device__ __forceinline__ void state_copy(Stage& st, const ChunkWorkspace& ws, const ChunkSrc& s,
                                           const int* ct, size_t row_stride, int lane) {
    // (the operands go through void pointers: typed ones make the host pass
    //  of this template reject the builtin, and typed 4-byte copies tripped a
    //  code-generation fault of the ROCm 7.2 compiler in this kernel)
    constexpr int kChains = Stage::kTiles;
    // Sources as a wave-uniform base plus a 32-bit per-lane byte offset, the
    // addressing form that needs no 64-bit vector add per copy (measured: the
    // copy wave's vector instructions per chunk 59 -> 28, recurrence after a
    // cache flush at T = 4000 60.5 -> 58.2 us).  Row offsets stay below 2^32:
    // at most 63 rows of at most 65535 value heads x 256 bytes.
    const char* kb = reinterpret_cast<const char*>(ws.kt + s.ku * kKtElems);
    const char* tb = reinterpret_cast<const char*>(ws.tu + s.vu * kTuElems);
    const char* gb = reinterpret_cast<const char*>(ws.dg + s.vu * kGElems);
    unsigned lo = 16u * lane;
    asm("" : "+v"(lo));   // kept 32-bit: hoisted, it became a 64-bit offset added per copy
#pragma unroll
    for (int piece = 0; piece < 16; ++piece)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kb + 4096 * (piece >> 2) + (lo + 1024u * (piece & 3))),
                                         reinterpret_cast<void*>(st.k + piece * 512), 16, 0, 0);
#pragma unroll
    for (int piece = 0; piece < 6; ++piece)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tb + 4096 * (piece >> 2) + (lo + 1024u * (piece & 3))),
                                         reinterpret_cast<void*>(st.tu + piece * 512), 16, 0, 0);
#pragma unroll
    for (int half = 0; half < 2; ++half)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gb + ((lo >> 2) + 4u * kChunk * half)),
                                         reinterpret_cast<void*>(st.dg + kChunk * half), 4, 0, 0);
    const unsigned rbytes = (unsigned)(row_stride * 2);
#pragma unroll
    for (int r = 0; r < kChains; ++r) {
        const char* vb = reinterpret_cast<const char*>(s.vrow + kVRowElems * ct[r]);
#pragma unroll
        for (int piece = 0; piece < 2; ++piece) {
            const unsigned row = (unsigned)min(32 * piece + (lane >> 1), s.len - 1);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vb + (row * rbytes + 16u * (lane & 1))),
                                             reinterpret_cast<void*>(st.v[r] + piece * 512), 16, 0, 0);
        }
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The tile's value rows of one chunk (bf16 [pos][16] in the stage) as the B
// fragment of U = TU V over the position slots of K-step qq, column ln,
// widened to fp16: two LDS transpose reads (ds_read_b64_tr_b16).  In each
// group of 16 lanes that instruction hands lane l element l % 4 of the
// 8-byte granules addressed by lanes l / 4 + 4 e, e = 0..3.  Lane l of group
// gq addresses row 32 qq + 16 h + 4 gq + l / 4 at granule l % 4, so it
// receives rows 32 qq + 16 h + 4 gq + e of column l: position slots 4 h + e.
__device__ __forceinline__ f16x8 v_frag(const uint16_t* vrows, int qq, int gq, int ln) {
    f16x8 f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 32 * qq + 16 * h + 4 * gq + (ln >> 2);
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(vrows + row * kVRowElems + 4 * (ln & 3)));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            f[4 * h + e] = static_cast<f16>(__uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(x[e])) << 16));
    }
    return f;
}

// Touch one chunk's operands into L2 ahead of their copies and loads, with
// 4-byte direct-to-LDS copies into a sink nobody reads (one cache line per
// lane), two per tile: the 352 shared lines of K^T, Q, TU and P split over
// the 8 column tiles of a head (44 per tile; lanes past 44 repeat a line),
// and a quarter of the value-row lines that hold the tile's columns: a
// 128-byte line of a value row holds the columns of four tiles, so tile ct
// touches the rows r with r % 4 == ct % 4 (16 lines, four lanes a line) and
// the four tiles together cover all 64 (measured against each tile touching
// all 64: recurrence at T = 131072 2.19 -> 2.06 ms, varlen batch 281 -> 273
// us, T = 4000 unchanged).  A direct copy, unlike a register load,
// is invisible to the compiler's counter waits, so the copy wave's own
// single wait still covers it.  (Issued from a W wave, which never waits for
// its memory counter, the value touches were slower: a touch that waits on
// HBM holds one of the CU's outstanding-request slots the copies need.)
__device__ __forceinline__ void touch_shared(const ChunkWorkspace& ws, const ChunkSrc& s, int ct, int lane,
                                             float* sink) {
    const int line = ct * 44 + min(lane, 43);
    const int off = (line & 127) * 64;                       // halves
    const f16* base = line < 128 ? ws.kt + s.ku * kKtElems + off
                    : line < 256 ? ws.qf + s.ku * kQfElems + off
                    : line < 304 ? ws.tu + s.vu * kTuElems + (line - 256) * 64
                                 : ws.p + s.vu * kPElems + (line - 304) * 64;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base), reinterpret_cast<void*>(sink), 4, 0, 0);
}

__device__ __forceinline__ void touch_values(const ChunkSrc& s, int ct, size_t row_stride, int lane, float* sink) {
    const unsigned row = (unsigned)min(4 * (lane >> 2) + (ct & 3), s.len - 1);
    const char* vb = reinterpret_cast<const char*>(s.vrow + kVRowElems * ct);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vb + row * (unsigned)(row_stride * 2)),
                                     reinterpret_cast<void*>(sink), 4, 0, 0);
}

// Q's 16 fragments of one chunk, as sixteen 16-byte register loads.
struct QFrag {
    f16x8 f[16];
};

__device__ __forceinline__ QFrag load_q(const ChunkWorkspace& ws, size_t ku, int lane) {
    const f16* src = ws.qf + ku * kQfElems;
    QFrag qf;
#pragma unroll
    for (int f = 0; f < 16; ++f) qf.f[f] = *reinterpret_cast<const f16x8*>(src + (f * 64 + lane) * 8);
    return qf;
}

// P's six nonzero A fragments of one chunk, as six 16-byte register loads.
struct PFrag {
    f16x8 f[6];
};

__device__ __forceinline__ PFrag load_p(const ChunkWorkspace& ws, size_t vu, int lane) {
    const f16* src = ws.p + vu * kPElems;
    PFrag pf;
#pragma unroll
    for (int f = 0; f < 6; ++f) pf.f[f] = *reinterpret_cast<const f16x8*>(src + (f * 64 + lane) * 8);
    return pf;
}

// The (row tile, K-step) blocks of TU's six nonzero fragments, in storage order.
__device__ __forceinline__ constexpr int tu_pt(int f) { return f < 2 ? f : 2 + ((f - 2) >> 1); }
__device__ __forceinline__ constexpr int tu_qq(int f) { return f < 2 ? 0 : (f - 2) & 1; }

// A W wave's step for one chunk (stage st): the chain's A fragments of -W
// over d_k K-steps kQd0 .. kQd1 - 1 into wdst.
//   -W^T[d][r] = sum_s K^T[d][s] (-e^{G_s} TU[r][s]): A = the K^T fragment
//   (d_k tile i, K-step qq), B = TU's fragment (row tile pt, K-step qq) with
//   each position slot scaled by -e^{G_s} (an A and a B fragment share one
//   lane layout); the accumulators of d_k tiles 2 qq', 2 qq' + 1 stacked are
//   the chain's A fragment (p, qq') of -W.  The scaling is a packed fp16
//   product: TU is fp16 already and the product is rounded to fp16 as the
//   operand anyway; e^{G_s} below fp16's normal range (G_s < -9.7) loses
//   relative precision there, where the entries' share of W is as small.
template <int kQd0, int kQd1, typename Stage>
__device__ __forceinline__ void w_chunk(const Stage& st, f16* wdst, int lane, int gq) {
    f16x8 ng[2];                                             // -e^{G_s} over the slots of K-step qq
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(&st.dg[kChunk + 32 * qq + 4 * gq]);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(&st.dg[kChunk + 32 * qq + 16 + 4 * gq]);
        ng[qq] = cat_to_f16(-g0, -g1);
    }
    f16x8 twb[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) twb[f] = *reinterpret_cast<const f16x8*>(&st.tu[(f * 64 + lane) * 8]) * ng[tu_qq(f)];
#pragma unroll
    for (int qd = kQd0; qd < kQd1; ++qd) {
        f16x8 ka[2][2];                                      // K^T fragments (i = 2 qd + a, K-step qq)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
                ka[a][qq] = *reinterpret_cast<const f16x8*>(&st.k[(((2 * qd + a) * 2 + qq) * 64 + lane) * 8]);
        f32x4 acc[2][4];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 6; ++f)
#pragma unroll
            for (int a = 0; a < 2; ++a) acc[a][tu_pt(f)] = mfma_f16(ka[a][tu_qq(f)], twb[f], acc[a][tu_pt(f)]);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            *reinterpret_cast<f16x8*>(&wdst[((p * 4 + qd) * 64 + lane) * 8]) = cat_to_f16(acc[0][p], acc[1][p]);
    }
}

// Row tiles kPt0 .. kPt1 - 1 of a tile's U = TU V for one chunk into udst
// as fp32 accumulator fragments (rows 16 p + 4 gq + e, column ln of the
// tile): A = TU's fragment, B = the tile's values over the same position
// slots (v_frag).  Row tiles 0-1 need only K-step 0.
template <int kPt0, int kPt1, typename Stage>
__device__ __forceinline__ void u_part(const Stage& st, int r, float* udst, int lane, int gq, int ln) {
    constexpr int kQq = kPt1 > 2 ? 2 : 1;
    f16x8 vb[2];
#pragma unroll
    for (int qq = 0; qq < kQq; ++qq) vb[qq] = v_frag(st.v[r], qq, gq, ln);
    f32x4 u[4];
#pragma unroll
    for (int p = kPt0; p < kPt1; ++p) u[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        if (tu_pt(f) < kPt0 || tu_pt(f) >= kPt1) continue;
        u[tu_pt(f)] = mfma_f16(*reinterpret_cast<const f16x8*>(&st.tu[(f * 64 + lane) * 8]), vb[tu_qq(f)],
                               u[tu_pt(f)]);
    }
#pragma unroll
    for (int p = kPt0; p < kPt1; ++p) *reinterpret_cast<f32x4*>(&udst[(p * 64 + lane) * 4]) = u[p];
}

// The chain wave's step for one chunk: H0 (fp32 accumulators H, its fp16 B
// fragments hb) -> H_C, and hb <- fp16 B fragments of H_C.  -W comes from
// wsrc, U (fp32 accumulator fragments) from usrc, K^T and the decay vector
// from the stage.  With the output, U' goes to ub and H_C's fragments to hd
// for the output wave.
template <bool kOut, bool kSnap, typename Stage>
__device__ __forceinline__ void chain_chunk(f32x4 (&H)[8], f16x8 (&hb)[4], const Stage& st,
                                            const f16* wsrc, const float* usrc, f16* ub, f16* hd, float* snap,
                                            bool use_u, int lane, int gq, int ln) {
    // U' = U + (-W) H0: the fragments are read before the burst, whose 4
    // accumulator chains interleave
    f32x4 acc[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
        acc[p] = use_u ? *reinterpret_cast<const f32x4*>(&usrc[(p * 64 + lane) * 4]) : f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8 wa[4][4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int p = 0; p < 4; ++p) wa[qq][p] = *reinterpret_cast<const f16x8*>(&wsrc[((p * 4 + qq) * 64 + lane) * 8]);
    f16x8 ka[2][8];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int i = 0; i < 8; ++i) ka[qq][i] = *reinterpret_cast<const f16x8*>(&st.k[((i * 2 + qq) * 64 + lane) * 8]);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[p] = mfma_f16(wa[qq][p], hb[qq], acc[p]);
    if constexpr (kOut) {
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
            *reinterpret_cast<f16x8*>(&ub[(qq * 64 + lane) * 8]) = cat_to_f16(acc[2 * qq], acc[2 * qq + 1]);
    }
    // diag(e^{G_C - G}) U' as B fragments (position slots), the B operand of
    // the update  H <- e^{G_C} H + K^T (diag(e^{G_C - G}) U')
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        f32x4 dc = *reinterpret_cast<const f32x4*>(&st.dg[16 * p + 4 * gq]);
        if (p == 3 && gq == 3) dc[3] = 1.f;      // row 63: G_C - G_63 = 0
        acc[p] *= dc;
    }
    f16x8 up[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) up[qq] = cat_to_f16(acc[2 * qq], acc[2 * qq + 1]);
    const float gam = st.dg[kChunk - 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) H[i] *= gam;
    // eight independent accumulator chains, interleaved
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int i = 0; i < 8; ++i) H[i] = mfma_f16(ka[qq][i], up[qq], H[i]);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) hb[qq] = cat_to_f16(H[2 * qq], H[2 * qq + 1]);
    if constexpr (kOut) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<f16x8*>(&hd[(qq * 64 + lane) * 8]) = hb[qq];
    }
    if constexpr (kSnap) {
        // non-temporal: 64 KB per head and chunk that this launch never reads
        // back, kept from evicting the chunks touched ahead in L2 (measured:
        // 122 -> 103 us per 4000-token prefill)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                __builtin_nontemporal_store(H[i][e], &snap[(size_t)(16 * i + 4 * gq + e) * kDim + ln]);
    }
}

// The output is formed transposed, O^T = H0^T Q^T + U'^T P^T, so that an
// accumulator lane holds 4 consecutive columns of one output row (a 16-byte
// store) instead of 4 rows of one column.  The operands are the same
// registers: an A and a B fragment share one lane layout, so the stacked
// state and U' fragments serve as H0^T and U'^T, and the Q and P fragments
// as Q^T and P^T.  oacc[p] holds output rows 16 p + ln, columns 4 gq .. +3
// of the tile.

// The output wave's first half of a chunk: diag(e^G) (Q H0) into oacc.
__device__ __forceinline__ void out_begin(f32x4 (&oacc)[4], const float* dg, const QFrag& qf, const f16* hsrc,
                                          int lane, int ln) {
    f16x8 hb[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) hb[qq] = *reinterpret_cast<const f16x8*>(&hsrc[(qq * 64 + lane) * 8]);
    f16x8 qa[4][4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int p = 0; p < 4; ++p) qa[qq][p] = qf.f[p * 4 + qq];
#pragma unroll
    for (int p = 0; p < 4; ++p) oacc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int p = 0; p < 4; ++p) oacc[p] = mfma_f16(hb[qq], qa[qq][p], oacc[p]);
#pragma unroll
    for (int p = 0; p < 4; ++p) oacc[p] *= dg[kChunk + 16 * p + ln];
}

// The output wave's second half: + P U', then the stores of the output rows
// t0 .. t0 + len - 1 of the tile.  out_tile points at column 0 of the tile
// (row 0 of the chunk); rows past len go to the sink so that the number of
// stores never changes.  nt: non-temporal stores (wave-uniform).
__device__ __forceinline__ void out_end(f32x4 (&oacc)[4], const PFrag& pf, const f16* usrc, float* out_tile,
                                        size_t row_stride, int len, float* junk, bool nt, int lane, int gq, int ln) {
    f16x8 ua[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) ua[qq] = *reinterpret_cast<const f16x8*>(&usrc[(qq * 64 + lane) * 8]);
    oacc[0] = mfma_f16(ua[0], pf.f[0], oacc[0]);
    oacc[1] = mfma_f16(ua[0], pf.f[1], oacc[1]);
    oacc[2] = mfma_f16(ua[0], pf.f[2], oacc[2]);
    oacc[3] = mfma_f16(ua[0], pf.f[4], oacc[3]);
    oacc[2] = mfma_f16(ua[1], pf.f[3], oacc[2]);
    oacc[3] = mfma_f16(ua[1], pf.f[5], oacc[3]);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = 16 * p + ln;
        float* d = row < len ? out_tile + (size_t)row * row_stride + 4 * gq : junk + 4 * lane;
        if (nt) __builtin_nontemporal_store(oacc[p], reinterpret_cast<f32x4*>(d));
        else *reinterpret_cast<f32x4*>(d) = oacc[p];
    }
}

// ---------------------------------------------------------------------------
// Segments of a sequence (the chunk-parallel affine scan).  A sequence of
// nch chunks is cut into nseg = max(1, ceil(nch / sc)) segments of sc chunks.
// Over one segment the recurrence is affine in its incoming state,
// H_end = Phi H_start + R, and the maps compose: (Phi2, R2) o (Phi1, R1) =
// (Phi2 Phi1, Phi2 R1 + R2).  Segment s of sequence n has the index
// seg_base(n) + s, seg_base(n) = n + slot_base(n) / sc; consecutive
// sequences never overlap and every index is below n + (n + T/64 + 1) / sc + 1.
// ---------------------------------------------------------------------------
struct SegArgs {
    int seg_chunks;          // sc
    int n_segslots;
    const float* hstart;     // [segslot][h_v][128][128]: incoming state of every segment of a
                             // sequence with two or more (segment 0's copied from s0 by the scan)
    float* maps;             // [segslot][h_v][2][128][128]: Phi, R of segments s < nseg - 1
    int stream_out;          // the output goes out as non-temporal stores
    // Whole sequences: the launch runs the chunks whose slots lie in
    // slot_lo .. slot_hi - 1, whose intermediates sit in workspace slots
    // 0 .. slot_hi - slot_lo - 1.  A sequence that starts before slot_lo
    // takes its incoming state from carry, one that goes on past slot_hi
    // leaves its state there ([seq][h_v][128][128]); null when the launch
    // covers every slot.
    int slot_lo, slot_hi;
    float* carry;
};

__device__ __forceinline__ int seg_base(const int32_t* cu, int n, int sc) {
    return n + slot_base(cu, n) / sc;
}

__device__ __forceinline__ int seg_count(int nch, int sc) {
    return max(1, (nch + sc - 1) / sc);
}

// Map a segment slot to (sequence, segment, segment count); false if unused.
__device__ __forceinline__ bool resolve_segslot(const int32_t* __restrict__ cu, int n_seqs, int gs, int sc,
                                                int& seq, int& sg, int& nseg) {
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg_base(cu, mid, sc) <= gs) lo = mid; else hi = mid - 1;
    }
    const int nch = (cu[lo + 1] - cu[lo] + kChunk - 1) / kChunk;
    sg = gs - seg_base(cu, lo, sc);
    nseg = seg_count(nch, sc);
    seq = lo;
    return sg >= 0 && sg < nseg;
}

enum : int {
    kModeWhole = 0,          // whole sequences, with the output
    kModeWholeSnap = 1,      // the same, plus the state after every chunk
    kModeSegment = 2,        // one segment per workgroup, from its incoming state, with the output
    kModeMap = 3,            // the affine map (Phi, R) of one segment, no output
    kModeWholePair = 4,      // whole sequences, two column tiles per workgroup, with the output
    kModeSegmentPair = 5,    // segments, two column tiles per workgroup, with the output
    kModeMapPair = 6,        // segment maps, two column tiles (of Phi or of R) per workgroup
};

__host__ __device__ constexpr bool mode_pair(int mode) {
    return mode == kModeWholePair || mode == kModeSegmentPair || mode == kModeMapPair;
}

// The mode a tile-pair mode runs per tile.
__host__ __device__ constexpr int mode_base(int mode) {
    return mode == kModeWholePair ? kModeWhole : mode == kModeSegmentPair ? kModeSegment
                                               : mode == kModeMapPair ? kModeMap : mode;
}

// W waves of a state workgroup: two (about half of -W and U each) for one
// tile, whose interval is short; one for a tile pair, whose longer interval
// it fits.
__host__ __device__ constexpr int w_waves(int mode) { return mode_pair(mode) ? 1 : 2; }

// Threads of a state workgroup: chain, output, W and copy waves; an affine
// map has no output wave; a tile pair has two chain waves.
__host__ __device__ constexpr int state_threads(int mode) {
    return 64 * ((mode_pair(mode) ? 2 : 1) + (mode_base(mode) == kModeMap ? 0 : 1) + w_waves(mode) + 1);
}

// Stages of the copy ring.  The W wave uses a chunk's stage one interval
// before the chain, so a chunk must have landed two intervals ahead: with
// four stages its copies are issued three intervals ahead (one interval to
// land); a tile pair's larger stages leave room for three, issued two ahead
// and waited for in the same interval.
__host__ __device__ constexpr int ring_stages(int mode) { return mode_pair(mode) ? 3 : 4; }

// Workgroups of a state launch over `units` units of kTiles tiles each.
constexpr unsigned state_grid(int units, int tiles) { return 8u * tiles * 2u * (unsigned)((units + 15) / 16); }

// Grid: state_grid(U, kTiles) workgroups; U = n_seqs * h_v for whole
// sequences, n_segslots * h_v for segments; kTiles = 8 column tiles or 4
// tile pairs, for a map 16 (8 of Phi, 8 of R) or 8 pairs.  Workgroup b runs on XCD x = b % 8
// (round-robin dispatch); with m = b / 8 it takes tile m % kTiles of unit
// 16 (g / 2) + 2 x + g % 2, g = m / kTiles.  All tiles of a unit share an
// XCD, and so do units 2i and 2i + 1, the two value heads of a q/k head at
// two value heads per q/k head, whose K^T and Q fragments one L2 then
// serves; consecutive unit pairs go to different XCDs.
template <int kMode>
__global__ __launch_bounds__(state_threads(kMode)) void gdn_chunk_state(
    const int32_t* __restrict__ cu, int n_seqs, int h_v, const uint16_t* __restrict__ v,
    const float* s0, float* s_final, float* __restrict__ out, float* __restrict__ chunk_states,
    ChunkWorkspace ws, SegArgs sa)
{
    constexpr int kBase = mode_base(kMode);
    constexpr bool kOut = kBase != kModeMap;
    constexpr bool kSnap = kBase == kModeWholeSnap;
    constexpr bool kPair = mode_pair(kMode);
    constexpr int kChains = kPair ? 2 : 1;                   // chain waves: roles 0 .. kChains - 1
    constexpr int kTiles = (kBase == kModeMap ? 16 : 8) / kChains;
    constexpr bool kSeg = kBase == kModeSegment || kBase == kModeMap;
    constexpr int kStages = ring_stages(kMode);
    constexpr int kAhead = kStages - 1;                      // copies issued this many chunks ahead
    constexpr int kCopies = copies_per_chunk<kChains>();
    constexpr int kTouches = 2 * kChains;                    // the copy wave's touches per chunk
    constexpr int kTouchAhead = kAhead + 2;                  // chunks ahead of use that the touches reach
    constexpr int kOutRole = kChains;                        // when kOut
    constexpr int kWRole = kChains + (kOut ? 1 : 0);         // first W wave
    constexpr int kWWaves = w_waves(kMode);
    constexpr int kCopyRole = kWRole + kWWaves;
    static_assert(state_threads(kMode) == 64 * (kCopyRole + 1), "one wave per role");
    const int b = blockIdx.x;
    const int m = b >> 3;
    const int gu = m / kTiles;
    const int unit = ((gu >> 1) << 4) + ((b & 7) << 1) + (gu & 1);
    const int tile = m % kTiles;
    int seq, h, sg = 0, nseg = 1, gs = 0;
    if constexpr (!kSeg) {
        if (unit >= n_seqs * h_v) return;
        seq = unit / h_v;
        h = unit % h_v;
    } else {
        if (unit >= sa.n_segslots * h_v) return;
        gs = unit / h_v;
        h = unit % h_v;
        if (!resolve_segslot(cu, n_seqs, gs, sa.seg_chunks, seq, sg, nseg)) return;
        if (kBase == kModeMap && sg >= nseg - 1) return;    // the last segment needs no map
    }
    const int j = h / ws.group;

    const int lane = threadIdx.x & 63;
    // roles: chain waves first (one per column tile), then the output wave,
    // the W wave and the copy wave
    const int role = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = lane >> 4;
    const int ln = lane & 15;
    // tile of chain wave r among the unit's tiles (a map's 0-7 are Phi's,
    // 8-15 R's), and its column tile (the output wave takes all of them)
    auto gtile_of = [&](int r) { return kPair ? 2 * tile + r : tile; };
    auto tile_of = [&](int r) { return kBase == kModeMap ? gtile_of(r) & 7 : kPair ? 2 * tile + r : (tile & 7); };
    auto phi_of = [&](int r) { return kBase == kModeMap && gtile_of(r) < 8; };   // a map's Phi tile: no U

    __shared__ __attribute__((aligned(16))) StateStage<kChains> stage[kStages];
    __shared__ __attribute__((aligned(16))) f16 wbuf[2][kWElems];                  // W wave -> chain: -W
    __shared__ __attribute__((aligned(16))) float uin[kChains][2][kUaccElems];      // W wave -> chain: U
    __shared__ __attribute__((aligned(16))) f16 hbuf[kOut ? kChains : 1][2][kOut ? kHbElems : 8];  // chain -> output
    __shared__ __attribute__((aligned(16))) f16 ubuf[kOut ? kChains : 1][2][kOut ? kUbElems : 8];  // chain -> output
    __shared__ __attribute__((aligned(16))) float touch_sink[64];   // target of the L2 touches, never read

    const int start = cu[seq];
    const int end = cu[seq + 1];
    const int nchunks = (end - start + kChunk - 1) / kChunk;
    const int slot0 = slot_base(cu, seq);
    const int c_begin = kSeg ? sg * sa.seg_chunks : max(0, sa.slot_lo - slot0);
    const int c_end = kSeg ? min(c_begin + sa.seg_chunks, nchunks) : min(nchunks, sa.slot_hi - slot0);
    // a whole sequence with no chunk in the launch's slots has nothing to do
    // here (an empty one is handled by the launch that holds its slot)
    if (!kSeg && (nchunks > 0 ? c_begin >= c_end : slot0 < sa.slot_lo || slot0 >= sa.slot_hi)) return;
    const int wslot0 = kSeg ? slot0 : slot0 - sa.slot_lo;     // workspace slot of chunk 0
    auto vidx = [&](int c) { return ws.vunit(wslot0 + min(c, c_end - 1), h); };
    auto kidx = [&](int c) { return ws.kunit(wslot0 + min(c, c_end - 1), j); };
    const size_t vstride = (size_t)h_v * kDim;                // elements between token rows of v
    // chunk c's operands; chunks past the last one are clamped to it
    auto src_of = [&](int c) {
        const int cc = min(c, c_end - 1);
        const int t0 = start + kChunk * cc;
        ChunkSrc s;
        s.vu = ws.vunit(wslot0 + cc, h);
        s.ku = ws.kunit(wslot0 + cc, j);
        s.vrow = v + (size_t)t0 * vstride + (size_t)h * kDim;
        s.len = min(kChunk, end - t0);
        return s;
    };
    auto stage_of = [&](int c) -> StateStage<kChains>& { return stage[(c - c_begin) % kStages]; };
    const size_t sbase = ((size_t)seq * h_v + h) * kDim * kDim;
    const size_t gbase = ((size_t)gs * h_v + h) * kDim * kDim;

    // Barriers: P (the first chunk has landed), then B_0 .. B_n for n chunks;
    // in the interval between B_i and B_{i+1} the chain and the output work on
    // chunk i, the W wave forms chunk i + 1's -W and U (chunk c_begin's
    // between P and B_0) and the copy wave fills the stage of chunk i + kAhead.
    if (role < kChains) {
        const int ct = tile_of(role);
        const bool phi = phi_of(role);
        const int col = 16 * ct + ln;
        f32x4 H[8];
        if (kBase == kModeMap) {
            // Phi starts at the identity (tiles 0-7), R at zero (tiles 8-15)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    H[i][e] = (phi && 16 * i + 4 * gq + e == col) ? 1.f : 0.f;
        } else if (kSeg && nseg > 1) {
            // every segment of a split sequence starts from its copy in
            // hstart, segment 0 included: the last segment's workgroups may
            // write final_state while segment 0's still run, and final_state
            // may alias initial_state
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    H[i][e] = sa.hstart[gbase + (size_t)(16 * i + 4 * gq + e) * kDim + col];
        } else if (!kSeg && c_begin > 0) {
            // carried over from the launch that ran the chunks before
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    H[i][e] = sa.carry[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col];
        } else if (s0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    H[i][e] = s0[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) H[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __builtin_amdgcn_s_waitcnt(0);
        f16x8 hb[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) hb[qq] = cat_to_f16(H[2 * qq], H[2 * qq + 1]);
        if (c_end > c_begin) {
            if constexpr (kOut) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<f16x8*>(&hbuf[role][0][(qq * 64 + lane) * 8]) = hb[qq];
            }
            lds_barrier();                                   // P
            lds_barrier();                                   // B_0
            for (int c = c_begin; c < c_end; ++c) {
                const int i = c - c_begin;
                // tile base (column 16 ct); each lane adds its column ln
                float* snap = kSnap ? chunk_states + ((size_t)(slot0 + c) * h_v + h) * kDim * kDim + 16 * ct
                                    : nullptr;
                // U'(c) and H0(c + 1) for the output wave; the buffers it
                // reads in this interval are the other ones
                chain_chunk<kOut, kSnap>(H, hb, stage_of(c), wbuf[i & 1], uin[role][i & 1],
                                                  ubuf[kOut ? role : 0][i & 1], hbuf[kOut ? role : 0][(i + 1) & 1],
                                                  snap, !phi, lane, gq, ln);
                lds_barrier();                               // B_{i+1}
            }
        }
        if (kBase == kModeMap) {
            float* dst = sa.maps + (gbase * 2 + (phi ? 0 : (size_t)kDim * kDim));
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(size_t)(16 * i + 4 * gq + e) * kDim + col] = H[i][e];
        } else if (!kSeg && c_end < nchunks) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) sa.carry[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col] = H[i][e];
        } else if (s_final && sg == nseg - 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s_final[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col] = H[i][e];
        }
    } else if (kOut && role == kOutRole) {
        // the output wave: Q H0 of chunk c between B_c and B_{c+1}, from the
        // state the chain wave handed over before B_c; P U' of chunk c one
        // interval later, from the U' handed over before B_{c+1}.  Q and P
        // come by register loads.
        if (c_end > c_begin) {
            // unrolled by two so that the loaded fragments never need a
            // register copy (which would wait for the loads): Q of chunk c
            // is loaded one interval ahead, P of chunk c in its interval
            QFrag q0 = load_q(ws, kidx(c_begin), lane), q1;
            PFrag p0, p1;
            f32x4 oacc[kChains][4];
            auto end_of = [&](int cc, const PFrag& pf) {
                const int t0 = start + kChunk * cc;
#pragma unroll
                for (int r = 0; r < kChains; ++r)
                    out_end(oacc[r], pf, ubuf[r][(cc - c_begin) & 1],
                            out + ((size_t)t0 * h_v + h) * kDim + 16 * tile_of(r), (size_t)h_v * kDim,
                            min(kChunk, end - t0), ws.junk, sa.stream_out != 0, lane, gq, ln);
            };
            auto begin_of = [&](int cc, const QFrag& qf) {
#pragma unroll
                for (int r = 0; r < kChains; ++r)
                    out_begin(oacc[r], stage_of(cc).dg, qf, hbuf[r][(cc - c_begin) & 1], lane, ln);
            };
            lds_barrier();                                   // P
            lds_barrier();                                   // B_0
            for (int c = c_begin; c < c_end; c += 2) {
                if (c > c_begin) end_of(c - 1, p1);
                p0 = load_p(ws, vidx(c), lane);
                q1 = load_q(ws, kidx(c + 1), lane);          // clamped past the end
                begin_of(c, q0);
                lds_barrier();                               // B_{c+1}
                if (c + 1 == c_end) break;
                end_of(c, p0);
                p1 = load_p(ws, vidx(c + 1), lane);
                q0 = load_q(ws, kidx(c + 2), lane);
                begin_of(c + 1, q1);
                lds_barrier();                               // B_{c+2}
            }
            if (((c_end - 1 - c_begin) & 1) == 0) end_of(c_end - 1, p0);
            else end_of(c_end - 1, p1);
        }
    } else if (role < kCopyRole) {
        // the W waves: chunk c_begin's -W and U between P and B_0, chunk
        // c + 1's between B_c and B_{c+1}.  With two W waves the first takes
        // d_k K-steps 0-1 of -W and row tiles 0-1 of U, the second the rest.
        if (c_end > c_begin) {
            const bool first = role == kWRole;
            lds_barrier();                                   // P
            for (int c = c_begin; c <= c_end; ++c) {
                const int i = c - c_begin;
                if (c < c_end) {
                    const StateStage<kChains>& st = stage_of(c);
                    if (kWWaves == 1) {
                        w_chunk<0, 4>(st, wbuf[i & 1], lane, gq);
#pragma unroll
                        for (int r = 0; r < kChains; ++r)
                            if (!phi_of(r)) u_part<0, 4>(st, r, uin[r][i & 1], lane, gq, ln);
                    } else if (first) {
                        w_chunk<0, 2>(st, wbuf[i & 1], lane, gq);
#pragma unroll
                        for (int r = 0; r < kChains; ++r)
                            if (!phi_of(r)) u_part<0, 2>(st, r, uin[r][i & 1], lane, gq, ln);
                    } else {
                        w_chunk<2, 4>(st, wbuf[i & 1], lane, gq);
#pragma unroll
                        for (int r = 0; r < kChains; ++r)
                            if (!phi_of(r)) u_part<2, 4>(st, r, uin[r][i & 1], lane, gq, ln);
                    }
                }
                lds_barrier();                               // B_i
            }
        }
    } else if (c_end > c_begin) {
        // the copy wave.  Copies for chunks past the last one are issued too
        // (clamped, never used) so that the number of copies per chunk never
        // changes.  The touches go out after the copies: loads complete in
        // issue order, and the copies must not wait behind touches that go
        // to HBM.
        int cts[kChains];
#pragma unroll
        for (int r = 0; r < kChains; ++r) cts[r] = tile_of(r);
#pragma unroll
        for (int a = 0; a < kAhead; ++a) state_copy(stage_of(c_begin + a), ws, src_of(c_begin + a), cts, vstride, lane);
        // the touches an interval before B_0 would have issued, so that every
        // wait below counts the same operations after the chunk it waits for
#pragma unroll
        for (int r = 0; r < kChains; ++r) {
            touch_shared(ws, src_of(c_begin + kTouchAhead - 1), cts[r], lane, touch_sink);
            touch_values(src_of(c_begin + kTouchAhead - 1), cts[r], vstride, lane, touch_sink);
        }
        wait_vmcnt<(kAhead - 1) * kCopies + kTouches>();     // chunk c_begin has landed
        lds_barrier();                                       // P
        wait_vmcnt<(kAhead - 2) * kCopies + kTouches>();     // chunk c_begin + 1 has landed
        lds_barrier();                                       // B_0
        for (int c = c_begin; c < c_end; ++c) {
            // between B_i and B_{i+1}: chunk c + 2 must land for the W waves
            state_copy(stage_of(c + kAhead), ws, src_of(c + kAhead), cts, vstride, lane);
#pragma unroll
            for (int r = 0; r < kChains; ++r) {
                touch_shared(ws, src_of(c + kTouchAhead), cts[r], lane, touch_sink);
                touch_values(src_of(c + kTouchAhead), cts[r], vstride, lane, touch_sink);
            }
            // outstanding after chunk c + 2's copies: the previous interval's
            // touches (four ahead) when the copies run three ahead, then this
            // interval's copies and touches
            if constexpr (kAhead == 3) wait_vmcnt<2 * kTouches + kCopies>();
            else wait_vmcnt<kTouches>();
            lds_barrier();                                   // B_{i+1}
        }
        // drain the copies past the end before the workgroup's LDS goes away
        __builtin_amdgcn_s_waitcnt(0);
    }
}

// ---------------------------------------------------------------------------
// Scan over segments: the incoming state of segment s + 1 is Phi_s H_s + R_s,
// in fp32.  One workgroup of 256 threads per (sequence, value head, 16-column
// tile); Phi_s goes through LDS, the tile's state stays there.  Thread t
// computes column t % 16 of rows t / 16 + 16 i.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gdn_chunk_seg_scan(
    const int32_t* __restrict__ cu, int n_seqs, int h_v, const float* s0, SegArgs sa)
{
    const int b = blockIdx.x;
    const int ct = b & 7;
    const int unit = b >> 3;
    if (unit >= n_seqs * h_v) return;
    const int seq = unit / h_v;
    const int h = unit % h_v;
    const int nch = (cu[seq + 1] - cu[seq] + kChunk - 1) / kChunk;
    const int nseg = seg_count(nch, sa.seg_chunks);
    if (nseg <= 1) return;
    const int g0 = seg_base(cu, seq, sa.seg_chunks);
    const int tid = threadIdx.x;
    const int c = tid & 15;
    const int r0 = tid >> 4;
    constexpr int kPS = kDim + 1;                     // padded row of Phi in LDS

    __shared__ float Phi[kDim * kPS];
    __shared__ float Ht[kDim * 16];
    const size_t sbase = ((size_t)seq * h_v + h) * kDim * kDim;
    float* hs0 = const_cast<float*>(sa.hstart) + ((size_t)g0 * h_v + h) * kDim * kDim;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = r0 + 16 * i;
        const float x = s0 ? s0[sbase + (size_t)r * kDim + 16 * ct + c] : 0.f;
        Ht[r * 16 + c] = x;
        hs0[(size_t)r * kDim + 16 * ct + c] = x;      // segment 0's incoming state
    }
    for (int sg = 0; sg + 1 < nseg; ++sg) {
        const size_t mbase = ((size_t)(g0 + sg) * h_v + h) * 2 * kDim * kDim;
        const float* phi = sa.maps + mbase;
        const float* rr = sa.maps + mbase + (size_t)kDim * kDim;
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {                // 128 x 128 fp32, 16 B per thread per pass
            const int idx = tid + 256 * i;            // float4 index
            const int r = idx >> 5, k4 = (idx & 31) * 4;
            const f32x4 x = *reinterpret_cast<const f32x4*>(phi + (size_t)r * kDim + k4);
#pragma unroll
            for (int e = 0; e < 4; ++e) Phi[r * kPS + k4 + e] = x[e];
        }
        __syncthreads();
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = rr[(size_t)(r0 + 16 * i) * kDim + 16 * ct + c];
        for (int k = 0; k < kDim; ++k) {
            const float hk = Ht[k * 16 + c];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(Phi[(r0 + 16 * i) * kPS + k], hk, acc[i]);
        }
        __syncthreads();                              // every read of Phi and Ht is done
        float* dst = const_cast<float*>(sa.hstart) + ((size_t)(g0 + sg + 1) * h_v + h) * kDim * kDim;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = r0 + 16 * i;
            Ht[r * 16 + c] = acc[i];
            dst[(size_t)r * kDim + 16 * ct + c] = acc[i];
        }
        __syncthreads();
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Compute units of the current device (host query, no device work).
static int state_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// The whole-sequence recurrence (single tiles, or tile pairs once the tiles
// outnumber the CUs) over the chunk slots sa.slot_lo .. sa.slot_hi - 1.
static void launch_state_whole(const int32_t* cu, int n_seqs, int h_v, const uint16_t* v, const float* s0,
                               float* s_final, float* out, float* chunk_states, const ChunkWorkspace& ws,
                               const SegArgs& sa, hipStream_t stream) {
    const int units = n_seqs * h_v;
    const dim3 grid(state_grid(units, 8));
    if (chunk_states)
        hipLaunchKernelGGL(gdn_chunk_state<kModeWholeSnap>, grid, dim3(state_threads(kModeWholeSnap)), 0, stream,
                           cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
    else if (8 * units > state_cus())
        // more tiles than CUs: the workgroups run in rounds, and a pair of
        // tiles sharing one copy ring halves them
        hipLaunchKernelGGL(gdn_chunk_state<kModeWholePair>, dim3(state_grid(units, 4)),
                           dim3(state_threads(kModeWholePair)), 0, stream,
                           cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
    else
        hipLaunchKernelGGL(gdn_chunk_state<kModeWhole>, grid, dim3(state_threads(kModeWhole)), 0, stream,
                           cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
}

hipError_t launch_chunk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const int32_t* cu,
                            int n_seqs, int64_t total_tokens, int h_qk, int h_v,
                            const float* s0, float* out, float* s_final, float* chunk_states,
                            const ChunkWorkspace& ws, int n_slots, int stage_mask,
                            const SegLaunch* seg, int range, float* carry, hipStream_t stream)
{
    // Streaming stores of prep's intermediates once they outgrow what the
    // 256 MB last-level cache keeps for the state kernel.  Measured crossover
    // between 114 MB (T = 4000: ordinary stores 13 us faster per layer) and
    // 170 MB (T = 6000: streaming 2 us faster; 8-10% from 227 MB on).
    const bool stream_inter = (size_t)n_slots * chunk_slot_bytes(h_qk, h_v) > kStreamWorkspaceBytes;

    // One sequence whose intermediates outgrow the last-level cache runs
    // range by range (the caller decides, and lays the workspace out for one
    // range): prep of a range of chunk slots, then the recurrence over them,
    // the state handed from range to range in fp32 through `carry`, so that
    // each range's intermediates are written into and read from the cache,
    // and the next range overwrites them there.  The arithmetic is that of
    // the single pass, bit for bit.  A range is one full round of prep
    // workgroups (64 chunks at 32 value / 16 q/k heads), so that no round
    // runs part-empty.  Measured at T = 131072 against the single pass (prep
    // with streaming stores, then the recurrence with every operand from
    // HBM), on several MI355X: 2.76-2.88 -> 2.68-2.80 ms per layer after a
    // cache flush, -2% to +7% back to back, and 2.13 -> 1.94 ms at 16 value
    // / 8 q/k heads.
    if (range > 0) {
        const int nch = (int)((total_tokens + kChunk - 1) / kChunk);
        SegArgs sa = {};
        sa.stream_out = 1;
        sa.carry = carry;
        for (int lo = 0; lo < nch; lo += range) {
            const int hi = min(nch, lo + range);
            const hipError_t e = launch_prep(q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, lo, hi, stream);
            if (e != hipSuccess) return e;
            sa.slot_lo = lo;
            sa.slot_hi = hi;
            launch_state_whole(cu, n_seqs, h_v, v, s0, s_final, out, nullptr, ws, sa, stream);
        }
        return hipGetLastError();
    }

    if ((stage_mask & 1) && total_tokens > 0) {
        const hipError_t e = stream_inter
                                 ? launch_prep_stream(q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, 0, n_slots, stream)
                                 : launch_prep(q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, 0, n_slots, stream);
        if (e != hipSuccess) return e;
    }
    if ((stage_mask & 2) && n_seqs > 0) {
        SegArgs sa = {};
        // While the intermediates stay in the last-level cache (prep stores
        // them ordinarily), the output goes around it, so that it neither
        // evicts them nor, after other work, makes the cache write back
        // dirty lines to take it in (measured at T = 4000: recurrence 59.0 ->
        // 56.3 us cold, 92.7 -> 90.5 us per layer warm).  Once they come
        // from HBM anyway, ordinary stores were faster (varlen batch 268 ->
        // 292 us, T = 131072 2.04 -> 2.18 ms with non-temporal ones).
        sa.stream_out = !stream_inter;
        sa.slot_lo = 0;
        sa.slot_hi = n_slots;
        if (!seg) {
            launch_state_whole(cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa, stream);
        } else {
            sa.seg_chunks = seg->seg_chunks;
            sa.n_segslots = seg->n_segslots;
            sa.hstart = seg->hstart;
            sa.maps = seg->maps;
            const int units = seg->n_segslots * h_v;
            // Tile pairs once the active tiles outnumber the CUs, as for
            // whole sequences.  The segment slots overcount the segments, so
            // the choice uses an estimate that is exact for one sequence:
            // its ceil(T / 64) chunks make ceil(chunks / sc) segments, each
            // further sequence at most one more.
            const long long chunks = (total_tokens + kChunk - 1) / kChunk;
            const long long segs = (n_seqs - 1) + (chunks + seg->seg_chunks - 1) / seg->seg_chunks;
            const long long cus = state_cus();
            if (16 * (segs - n_seqs) * h_v > cus)
                hipLaunchKernelGGL(gdn_chunk_state<kModeMapPair>, dim3(state_grid(units, 8)),
                                   dim3(state_threads(kModeMapPair)), 0, stream,
                                   cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
            else
                hipLaunchKernelGGL(gdn_chunk_state<kModeMap>, dim3(state_grid(units, 16)),
                                   dim3(state_threads(kModeMap)), 0, stream,
                                   cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
            hipLaunchKernelGGL(gdn_chunk_seg_scan, dim3(8 * n_seqs * h_v), dim3(256), 0, stream,
                               cu, n_seqs, h_v, s0, sa);
            if (8 * segs * h_v > cus)
                hipLaunchKernelGGL(gdn_chunk_state<kModeSegmentPair>, dim3(state_grid(units, 4)),
                                   dim3(state_threads(kModeSegmentPair)), 0, stream,
                                   cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
            else
                hipLaunchKernelGGL(gdn_chunk_state<kModeSegment>, dim3(state_grid(units, 8)),
                                   dim3(state_threads(kModeSegment)), 0, stream,
                                   cu, n_seqs, h_v, v, s0, s_final, out, chunk_states, ws, sa);
        }
    }
    return hipGetLastError();
}

}  // namespace gdn

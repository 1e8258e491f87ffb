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
// Intermediates live in the caller's workspace in matrix-core fragment
// order, written by each producer exactly as its consumer's operand needs:
//   prep  -> -W as A fragments of (W H), U as accumulators of U' = U - W H,
//            K^T as A fragments of the state update, Q and P as A fragments
//            of the output's (Q H0) and (P U')
//   state -> chunk state H0 and U' as B fragments of (Q H0) and (P U')
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
// Stage 2: inter-chunk state recurrence with the output.  One workgroup of
// three waves per (sequence, value head, 16-column tile), specialised:
//   * the chain wave keeps the tile's 128 x 16 slice of the state in
//     accumulator registers (8 tiles of 16 d_k rows) for the whole sequence.
//     Per chunk it runs the 32 matrix-core products of U' = U - W H0 and
//     H_C = e^{G_C} H0 + K^T D U', the dependency from chunk to chunk (-W,
//     K^T and the decay vector from LDS, its U fragments by register loads
//     one chunk ahead), and hands U' and the new state, rounded to fp16 as B
//     operands, to the output wave through double-buffered LDS slots;
//   * the output wave forms O = diag(e^G) (Q H0) + P U' on its own SIMD:
//     the Q H0 half in the interval of the chunk (Q fragments by register
//     loads one interval ahead, e^G from the stage), the P U' half one
//     interval later, when U' has been handed over (P by register loads in
//     the chunk's interval); it stores O to global memory.  Taking Q
//     straight to its registers keeps 16 KB per chunk off the copy wave and
//     out of LDS;
//   * the copy wave issues direct global-to-LDS copies of -W, K^T and the
//     decay vectors into a ring of three stages, two chunks ahead, and
//     touches the operands of the chunk two beyond those (Q, U and P
//     included) into L2.
// The waves meet at one barrier per chunk.  The copy wave issues a fixed
// number of copies per chunk, so one memory-counter wait makes a stage ready
// before that barrier.  The eight tiles of a head run on one XCD so that its
// L2 serves the shared fragments.  An affine map has no output: its
// workgroups have a chain and a copy wave only.  When a batch has more tiles
// than the GPU has CUs, so that the workgroups run in rounds, a workgroup
// takes a pair of adjacent tiles: two chain waves on two SIMDs share the
// copy ring (-W, K^T and the decay vectors are the same for both) and one
// output wave forms both tiles' output from one set of Q and P fragments,
// which halves the operand traffic per tile and the number of rounds.
// ---------------------------------------------------------------------------
constexpr int kStages = 3;
constexpr int kUTile = 4 * 64 * 4;                           // halves of U fragments per column tile
constexpr int kHbElems = 4 * 64 * 8;                         // halves of the state's four B fragments
constexpr int kUbElems = 2 * 64 * 8;                         // halves of U''s two B fragments
constexpr int kCopiesPerChunk = 16 + 16 + 2;                 // -W, K^T, decay vectors

struct StateStage {
    f16 w[kWElems];
    f16 k[kKtElems];
    float dg[kGElems];        // e^{G_C - G_r} (r < 63) and e^{G_C} in entry 63; then e^{G_r}
};

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

// One chunk's copies: 1 KB pieces (16 B per lane) of -W and K^T, and the
// two 256 B decay vectors (4 B per lane).
__device__ __forceinline__ void state_copy(StateStage& st, const ChunkWorkspace& ws, size_t vu, size_t ku,
                                           int lane) {
    const f16* wsrc = ws.w + vu * kWElems;
    const f16* ksrc = ws.kt + ku * kKtElems;
    const float* gsrc = ws.dg + vu * kGElems;
#pragma unroll
    for (int piece = 0; piece < 16; ++piece) {
        __builtin_amdgcn_global_load_lds(wsrc + (piece * 64 + lane) * 8, st.w + piece * 512, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(ksrc + (piece * 64 + lane) * 8, st.k + piece * 512, 16, 0, 0);
    }
    // (the casts keep these 4-byte copies from tripping a code-generation
    //  fault of the ROCm 7.2 compiler in this kernel)
#pragma unroll
    for (int half = 0; half < 2; ++half)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(gsrc + kChunk * half + lane),
                                         reinterpret_cast<void*>(st.dg + kChunk * half), 4, 0, 0);
}

// Touch one chunk's operands into L2 two chunks before their copies, with
// 4-byte direct-to-LDS copies into a sink nobody reads (one cache line per
// lane).  First copy: the 384 lines of -W, K^T and Q, split over the 8
// column tiles of a head (lanes 0-47), and the 16 lines of the tile's own U
// (lanes 48-63).  Second copy: the 48 lines of P, 6 per tile (lanes past 6
// repeat a line).  A direct copy, unlike a register load, is invisible to the
// compiler's counter waits, so the copy wave's own single wait still covers
// it.  It pays where the operands come from HBM (long sequences).
constexpr int kTouchesPerChunk = 2;

__device__ __forceinline__ void state_touch(const ChunkWorkspace& ws, size_t vu, size_t ku, int ct, int lane,
                                            float* sink) {
    const f16* base;
    if (lane < 48) {
        const int line = ct * 48 + lane;
        const int arr = line >> 7, off = (line & 127) * 64;      // halves
        base = (arr == 0 ? ws.w + vu * kWElems : arr == 1 ? ws.kt + ku * kKtElems : ws.qf + ku * kQfElems) + off;
    } else {
        base = ws.u + vu * kUElems + (size_t)ct * kUTile + (lane - 48) * 64;
    }
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base), reinterpret_cast<void*>(sink), 4, 0, 0);
    const f16* pl = ws.p + vu * kPElems + (ct * 6 + min(lane, 5)) * 64;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(pl), reinterpret_cast<void*>(sink), 4, 0, 0);
}

// The tile's U fragments of one chunk, as four 8-byte register loads.
struct UFrag {
    f16x4 f[4];
};

__device__ __forceinline__ UFrag load_u(const ChunkWorkspace& ws, size_t vu, int ct, int lane) {
    const f16* src = ws.u + vu * kUElems + (size_t)ct * kUTile;
    UFrag u;
#pragma unroll
    for (int p = 0; p < 4; ++p) u.f[p] = *reinterpret_cast<const f16x4*>(src + (p * 64 + lane) * 4);
    return u;
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

// The chain wave's step for one chunk: H0 (fp32 accumulators H, its fp16 B
// fragments hb) -> H_C, and hb <- fp16 B fragments of H_C.  With the output,
// U' goes to ub and H_C's fragments to hd for the output wave.
template <bool kOut, bool kSnap>
__device__ __forceinline__ void chain_chunk(f32x4 (&H)[8], f16x8 (&hb)[4], const StateStage& st, const UFrag& u,
                                            f16* ub, f16* hd, float* snap, bool use_u, int lane, int gq, int ln) {
    // U' = U + (-W) H0: the fragments are read before the burst, whose 4
    // accumulator chains interleave
    f32x4 acc[4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[p][e] = use_u ? static_cast<float>(u.f[p][e]) : 0.f;
    f16x8 wa[4][4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int p = 0; p < 4; ++p) wa[qq][p] = *reinterpret_cast<const f16x8*>(&st.w[((p * 4 + qq) * 64 + lane) * 8]);
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
__device__ __forceinline__ void out_begin(f32x4 (&oacc)[4], const StateStage& st, const QFrag& qf, const f16* hsrc,
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
    for (int p = 0; p < 4; ++p) oacc[p] *= st.dg[kChunk + 16 * p + ln];
}

// The output wave's second half: + P U', then the stores of the output rows
// t0 .. t0 + len - 1 of the tile.  out_tile points at column 0 of the tile
// (row 0 of the chunk); rows past len go to the sink so that the number of
// stores never changes.
__device__ __forceinline__ void out_end(f32x4 (&oacc)[4], const PFrag& pf, const f16* usrc, float* out_tile,
                                        size_t row_stride, int len, float* junk, int lane, int gq, int ln) {
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
        *reinterpret_cast<f32x4*>(d) = oacc[p];
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

// Threads of a state workgroup: chain, output and copy waves; an affine map
// has no output wave; a tile pair has two chain waves.
__host__ __device__ constexpr int state_threads(int mode) {
    return 64 * ((mode_pair(mode) ? 2 : 1) + (mode_base(mode) == kModeMap ? 0 : 1) + 1);
}

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
    const int32_t* __restrict__ cu, int n_seqs, int h_v,
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
    constexpr int kCopyRole = state_threads(kMode) / 64 - 1;
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
    // then the copy wave
    const int role = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = lane >> 4;
    const int ln = lane & 15;
    // tile of chain wave r among the unit's tiles (a map's 0-7 are Phi's,
    // 8-15 R's), and its column tile (the output wave takes all of them)
    auto gtile_of = [&](int r) { return kPair ? 2 * tile + r : tile; };
    auto tile_of = [&](int r) { return kBase == kModeMap ? gtile_of(r) & 7 : kPair ? 2 * tile + r : (tile & 7); };

    __shared__ __attribute__((aligned(16))) StateStage stage[kStages];
    __shared__ __attribute__((aligned(16))) f16 hbuf[kChains][2][kHbElems];  // chain -> output: fp16 state
    __shared__ __attribute__((aligned(16))) f16 ubuf[kChains][2][kUbElems];  // chain -> output: fp16 U'
    __shared__ __attribute__((aligned(16))) float touch_sink[64];   // target of the L2 touches, never read

    const int start = cu[seq];
    const int end = cu[seq + 1];
    const int nchunks = (end - start + kChunk - 1) / kChunk;
    const int c_begin = kSeg ? sg * sa.seg_chunks : 0;
    const int c_end = kSeg ? min(c_begin + sa.seg_chunks, nchunks) : nchunks;
    const int slot0 = slot_base(cu, seq);
    auto vidx = [&](int c) { return ws.vunit(slot0 + min(c, c_end - 1), h); };
    auto kidx = [&](int c) { return ws.kunit(slot0 + min(c, c_end - 1), j); };
    const size_t sbase = ((size_t)seq * h_v + h) * kDim * kDim;
    const size_t gbase = ((size_t)gs * h_v + h) * kDim * kDim;

    if (role < kChains) {
        const int ct = tile_of(role);
        const bool phi = gtile_of(role) < 8;                 // a map's Phi tile
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
        const bool use_u = !(kBase == kModeMap && phi);      // Phi: the homogeneous part
        if (c_end > c_begin) {
            if constexpr (kOut) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) *reinterpret_cast<f16x8*>(&hbuf[role][0][(qq * 64 + lane) * 8]) = hb[qq];
            }
            UFrag un = load_u(ws, vidx(c_begin), ct, lane);
            lds_barrier();                                   // B_0: the first chunk has landed
            for (int c = c_begin; c < c_end; ++c) {
                const UFrag uc = un;
                un = load_u(ws, vidx(c + 1), ct, lane);       // clamped past the end
                // tile base (column 16 ct); each lane adds its column ln
                float* snap = kSnap ? chunk_states + ((size_t)(slot0 + c) * h_v + h) * kDim * kDim + 16 * ct
                                    : nullptr;
                // U'(c) and H0(c + 1) for the output wave; the buffers it
                // reads in this interval are the other ones
                chain_chunk<kOut, kSnap>(H, hb, stage[(c - c_begin) % kStages], uc, ubuf[role][(c - c_begin) & 1],
                                         hbuf[role][(c - c_begin + 1) & 1], snap, use_u, lane, gq, ln);
                lds_barrier();                               // B_{c+1}
            }
        }
        if (kBase == kModeMap) {
            float* dst = sa.maps + (gbase * 2 + (phi ? 0 : (size_t)kDim * kDim));
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(size_t)(16 * i + 4 * gq + e) * kDim + col] = H[i][e];
        } else if (s_final && sg == nseg - 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s_final[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col] = H[i][e];
        }
    } else if (role < kCopyRole) {
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
                            min(kChunk, end - t0), ws.junk, lane, gq, ln);
            };
            auto begin_of = [&](int cc, const QFrag& qf) {
#pragma unroll
                for (int r = 0; r < kChains; ++r)
                    out_begin(oacc[r], stage[(cc - c_begin) % kStages], qf, hbuf[r][(cc - c_begin) & 1], lane, ln);
            };
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
    } else if (c_end > c_begin) {
        // copies for chunks past the last one are issued too (clamped, never
        // used) so the number of copies per chunk never changes
        constexpr int kCopies = kCopiesPerChunk;
        state_copy(stage[0], ws, vidx(c_begin), kidx(c_begin), lane);
        state_copy(stage[1], ws, vidx(c_begin + 1), kidx(c_begin + 1), lane);
        wait_vmcnt<kCopies>();                               // the first chunk has landed
        lds_barrier();                                       // B_0
        for (int c = c_begin; c < c_end; ++c) {
            // between B_c and B_{c+1}: the chain and output waves work on chunk c
            // the touches go out before the copies for one tile of whole
            // sequences, after them for segments, maps and tile pairs (whose
            // four touches would delay the copies): measured
            constexpr bool kTouchFirst = kMode == kModeWhole || kMode == kModeWholeSnap;
            if constexpr (kTouchFirst) state_touch(ws, vidx(c + 4), kidx(c + 4), tile_of(0), lane, touch_sink);
            state_copy(stage[(c - c_begin + 2) % kStages], ws, vidx(c + 2), kidx(c + 2), lane);
            if constexpr (!kTouchFirst) {
#pragma unroll
                for (int r = 0; r < kChains; ++r) state_touch(ws, vidx(c + 4), kidx(c + 4), tile_of(r), lane, touch_sink);
            }
            wait_vmcnt<kCopies + kChains * kTouchesPerChunk>();  // chunk c + 1 has landed
            lds_barrier();                                   // B_{c+1}
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

// Workspace intermediates above which prep streams its stores.
constexpr size_t kStreamWorkspaceBytes = (size_t)160 << 20;

hipError_t launch_chunk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const int32_t* cu,
                            int n_seqs, int64_t total_tokens, int h_qk, int h_v,
                            const float* s0, float* out, float* s_final, float* chunk_states,
                            const ChunkWorkspace& ws, int n_slots, int stage_mask,
                            const SegLaunch* seg, hipStream_t stream)
{
    if ((stage_mask & 1) && total_tokens > 0) {
        // Streaming stores once the intermediates outgrow what the 256 MB
        // last-level cache keeps for the state kernel.  Measured crossover
        // between 114 MB (T = 4000: ordinary stores 13 us faster per layer)
        // and 170 MB (T = 6000: streaming 2 us faster; 8-10% from 227 MB on).
        const size_t inter = (size_t)n_slots * ((size_t)h_v * ((kWElems + kUElems + kPElems) * sizeof(f16) +
                                                               kGElems * sizeof(float)) +
                                                (size_t)h_qk * (kKtElems + kQfElems) * sizeof(f16));
        const hipError_t e = inter > kStreamWorkspaceBytes
                                 ? launch_prep_stream(q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, n_slots, stream)
                                 : launch_prep(q, k, v, g, beta, cu, n_seqs, h_qk, h_v, ws, n_slots, stream);
        if (e != hipSuccess) return e;
    }
    if ((stage_mask & 2) && n_seqs > 0) {
        SegArgs sa = {};
        if (!seg) {
            const int units = n_seqs * h_v;
            const dim3 grid(state_grid(units, 8));
            if (chunk_states)
                hipLaunchKernelGGL(gdn_chunk_state<kModeWholeSnap>, grid, dim3(state_threads(kModeWholeSnap)), 0, stream,
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
            else if (8 * units > state_cus())
                // more tiles than CUs: the workgroups run in rounds, and a
                // pair of tiles sharing one copy ring halves them
                hipLaunchKernelGGL(gdn_chunk_state<kModeWholePair>, dim3(state_grid(units, 4)),
                                   dim3(state_threads(kModeWholePair)), 0, stream,
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
            else
                hipLaunchKernelGGL(gdn_chunk_state<kModeWhole>, grid, dim3(state_threads(kModeWhole)), 0, stream,
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
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
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
            else
                hipLaunchKernelGGL(gdn_chunk_state<kModeMap>, dim3(state_grid(units, 16)),
                                   dim3(state_threads(kModeMap)), 0, stream,
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
            hipLaunchKernelGGL(gdn_chunk_seg_scan, dim3(8 * n_seqs * h_v), dim3(256), 0, stream,
                               cu, n_seqs, h_v, s0, sa);
            if (8 * segs * h_v > cus)
                hipLaunchKernelGGL(gdn_chunk_state<kModeSegmentPair>, dim3(state_grid(units, 4)),
                                   dim3(state_threads(kModeSegmentPair)), 0, stream,
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
            else
                hipLaunchKernelGGL(gdn_chunk_state<kModeSegment>, dim3(state_grid(units, 8)),
                                   dim3(state_threads(kModeSegment)), 0, stream,
                                   cu, n_seqs, h_v, s0, s_final, out, chunk_states, ws, sa);
        }
    }
    return hipGetLastError();
}

}  // namespace gdn

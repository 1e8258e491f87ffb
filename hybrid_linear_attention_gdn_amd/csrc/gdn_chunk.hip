// Chunked Gated DeltaNet prefill for gfx950: three kernels, chunk length 64.
//
// The split follows the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page,
// section 2 ("GDN prefill"): intra-chunk preparation, inter-chunk state
// recurrence with the state resident in matrix-core accumulators and the
// next chunk prefetched, then the output.  The chunkwise algebra (state
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
//   prep  -> -W as A fragments of (W H), U as accumulators of U' = U - W H
//   state -> chunk state H0 and U' as B fragments of (Q H0) and (P U')
// Contraction slot maps (lane group gq = lane / 16, slot s = 0..7):
//   dim a(gq, s)   = 32 qq + 16 (s / 4) + 4 gq + s % 4   for K-step qq over d_k
//   pos p(gq, s)   = 32 qq + 16 (s / 4) + 4 gq + s % 4   for K-step qq over positions
// which is exactly how two stacked 16x16 accumulator tiles sit in a lane.

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

constexpr int kTS = 72;   // LDS row stride (halves or floats) of 64-wide tiles
constexpr int kQS = 136;  // LDS row stride (halves) of 128-wide tiles

// ---------------------------------------------------------------------------
// Stage 1: intra-chunk preparation.  One workgroup per (chunk slot, value head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gdn_chunk_prep(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int n_seqs, int h_qk, int h_v, ChunkWorkspace ws)
{
    const int slot = blockIdx.x;
    const int h = blockIdx.y;
    int seq, t0, len;
    if (!resolve_slot(cu, n_seqs, slot, seq, t0, len)) return;
    const int j = h / (h_v / h_qk);

    __shared__ __attribute__((aligned(16))) f16 KsT[kDim * kTS];   // K^T [dim][pos]
    __shared__ __attribute__((aligned(16))) f16 VsT[kDim * kTS];   // V^T [dim][pos]
    __shared__ __attribute__((aligned(16))) float Ab[kChunk * kTS]; // A fp32, then TW | TU fp16
    __shared__ __attribute__((aligned(16))) float Tb[kChunk * kTS]; // Tm = (I + A)^{-1} fp32
    __shared__ float Gs[kChunk];
    __shared__ float Bs[kChunk];
    __shared__ float Bw[kChunk];                                     // beta e^G

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int gq = lane >> 4;
    const int ln = lane & 15;

    // ---- load K, V (bf16 -> fp16), transposed into LDS; pad rows are zero
    for (int i = tid; i < kChunk * 16; i += 256) {
        const int r = i >> 4;
        const int c8 = (i & 15) * 8;
        u16x8 kb = {0, 0, 0, 0, 0, 0, 0, 0};
        u16x8 vb = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < len) {
            kb = *reinterpret_cast<const u16x8*>(k + ((size_t)(t0 + r) * h_qk + j) * kDim + c8);
            vb = *reinterpret_cast<const u16x8*>(v + ((size_t)(t0 + r) * h_v + h) * kDim + c8);
        }
        const f16x8 kf = bf16x8_to_f16x8(kb);
        const f16x8 vf = bf16x8_to_f16x8(vb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            KsT[(c8 + e) * kTS + r] = kf[e];
            VsT[(c8 + e) * kTS + r] = vf[e];
        }
    }
    if (tid < kChunk) {
        const bool in = tid < len;
        Gs[tid] = in ? g[(size_t)(t0 + tid) * h_v + h] : 0.f;
        Bs[tid] = in ? beta[(size_t)(t0 + tid) * h_v + h] : 0.f;
    }
    __syncthreads();

    // ---- K^T as A-operand fragments of the state update K^T X, written once
    //      per (slot, q/k head) by the first value head of the group:
    //      fragment (i, qq), lane (gq, ln) = K^T[16 i + ln][p(gq, s)] for K-step qq
    const size_t wsidx = (size_t)slot * h_v + h;
    if (h % (h_v / h_qk) == 0) {
        f16* kdst = ws.kt + ((size_t)slot * h_qk + j) * kKtElems;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int f = wave + 4 * it;          // fragment index i * 2 + qq
            const int i = f >> 1, qq = f & 1;
            const f16* krow = KsT + (16 * i + ln) * kTS + 32 * qq + 4 * gq;
            const f16x4 lo = *reinterpret_cast<const f16x4*>(krow);
            const f16x4 hi = *reinterpret_cast<const f16x4*>(krow + 16);
            const f16x8 fr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<f16x8*>(kdst + ((size_t)f * 64 + lane) * 8) = fr;
        }
    }

    // ---- decay cumsum within the chunk (wave 0, one lane per position)
    if (wave == 0) {
        float x = Gs[lane];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float gc = __shfl(x, kChunk - 1, 64);
        const float eg = exp_f(x);
        Gs[lane] = x;
        Bw[lane] = Bs[lane] * eg;
        float* gdst = ws.gcum + wsidx * kGElems;
        gdst[lane] = exp_f(gc - x);
        gdst[64 + lane] = eg;
        gdst[128 + lane] = x;
    }
    __syncthreads();

    // ---- A = strictly lower (beta_r e^{G_r-G_s} K K^T); wave w owns row tile w.
    //      Operands straight from global memory: K rows, 8 dims per lane.
    {
        const int p = wave;
        f16x8 afr[4];
        const int ra = 16 * p + ln;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u16x8 b = {0, 0, 0, 0, 0, 0, 0, 0};
            if (ra < len)
                b = *reinterpret_cast<const u16x8*>(k + ((size_t)(t0 + ra) * h_qk + j) * kDim + 32 * kk + 8 * gq);
            afr[kk] = bf16x8_to_f16x8(b);
        }
        for (int jt = 0; jt <= p; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int rb = 16 * jt + ln;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u16x8 b = {0, 0, 0, 0, 0, 0, 0, 0};
                if (rb < len)
                    b = *reinterpret_cast<const u16x8*>(k + ((size_t)(t0 + rb) * h_qk + j) * kDim + 32 * kk + 8 * gq);
                acc = mfma_f16(afr[kk], bf16x8_to_f16x8(b), acc);
            }
            const int s = 16 * jt + ln;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * p + 4 * gq + e;
                Ab[r * kTS + s] = (s < r) ? Bs[r] * exp_f(Gs[r] - Gs[s]) * acc[e] : 0.f;
            }
        }
    }
    __syncthreads();

    // ---- Tm = (I + A)^{-1}, blocked by 16 (A strictly lower triangular).
    //  (1) Diagonal blocks Tm_ii = (I + A_ii)^{-1}: wave i, lane c % 16 holds
    //      column c; x_r = delta_rc - sum_{t<r} A_rt x_t (x_t = 0 for t < c).
    //  (2) Below the diagonal, block column j on wave j, rows i = j+1..3:
    //      Tm_ij = -Tm_ii sum_{k=j}^{i-1} A_ik Tm_kj, with 16x16x16 products on
    //      the matrix cores (split fp16 operands, ~fp32 accuracy).  A product's
    //      accumulator is already the B operand of the next one, so the column
    //      chain never leaves registers.
    {
        const int ib = wave;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == ln) ? 1.f : 0.f;
            const float* arow = Ab + (16 * ib + r) * kTS + 16 * ib;
#pragma unroll
            for (int t = 0; t < r; ++t) acc -= arow[t] * x[t];
            x[r] = acc;
        }
        if (gq == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Tb[(16 * ib + r) * kTS + 16 * ib + ln] = x[r];
        }
    }
    __syncthreads();
    if (wave < 3) {
        const int jb = wave;
        f32x4 tcol[4];     // Tm_{k, jb} in accumulator (= B operand) layout, k >= jb
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) tcol[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            if (kb == jb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) tcol[kb][e] = Tb[(16 * kb + 4 * gq + e) * kTS + 16 * kb + ln];
            }
#pragma unroll
        for (int i2 = 1; i2 < 4; ++i2) {
            if (i2 <= jb) continue;
            f32x4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < i2; ++kb) {
                if (kb < jb) continue;
                const f32x4 aik = *reinterpret_cast<const f32x4*>(Ab + (16 * i2 + ln) * kTS + 16 * kb + 4 * gq);
                xs = mfma_split16(aik, tcol[kb], xs);
            }
            const f32x4 tii = *reinterpret_cast<const f32x4*>(Tb + (16 * i2 + ln) * kTS + 16 * i2 + 4 * gq);
            const f32x4 y = mfma_split16(tii, xs, f32x4{0.f, 0.f, 0.f, 0.f});
            tcol[i2] = -y;
#pragma unroll
            for (int e = 0; e < 4; ++e) Tb[(16 * i2 + 4 * gq + e) * kTS + 16 * jb + ln] = -y[e];
        }
    }
    __syncthreads();

    // ---- TW = Tm diag(beta e^G), TU = Tm diag(beta) in fp16 over the dead A
    //      buffer; blocks above the diagonal are zero.
    f16* TWs = reinterpret_cast<f16*>(Ab);          // [pos][t]
    f16* TUs = TWs + kChunk * kTS;                  // [pos][t]
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int idx = tid + 256 * it;
        const int r = idx >> 6, t = idx & 63;
        const float tm = ((t >> 4) > (r >> 4)) ? 0.f : Tb[r * kTS + t];
        TWs[r * kTS + t] = static_cast<f16>(tm * Bw[t]);
        TUs[r * kTS + t] = static_cast<f16>(tm * Bs[t]);
    }
    __syncthreads();

    // ---- W^T = K^T TW^T and U = TU V.  Wave w owns dim/col tiles 2w, 2w+1.
    {
        f32x4 wacc[2][4];
        f32x4 uacc[4][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                wacc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};
                uacc[p][a] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f16x8 kfr[2], vfr[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int d = 16 * (2 * wave + a) + ln;
                kfr[a] = *reinterpret_cast<const f16x8*>(KsT + d * kTS + 32 * kt + 8 * gq);
                vfr[a] = *reinterpret_cast<const f16x8*>(VsT + d * kTS + 32 * kt + 8 * gq);
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int row = 16 * p + ln;
                const f16x8 tw = *reinterpret_cast<const f16x8*>(TWs + row * kTS + 32 * kt + 8 * gq);
                const f16x8 tu = *reinterpret_cast<const f16x8*>(TUs + row * kTS + 32 * kt + 8 * gq);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    wacc[a][p] = mfma_f16(kfr[a], tw, wacc[a][p]);   // W^T[dim][pos]
                    uacc[p][a] = mfma_f16(tu, vfr[a], uacc[p][a]);   // U[pos][col]
                }
            }
        }
        // -W fragments (p, qq = wave): stacked dim tiles 2w, 2w+1 of W^T
        f16* wdst = ws.w + wsidx * kWElems;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f16x8 fr = cat_to_f16(-wacc[0][p], -wacc[1][p]);
            *reinterpret_cast<f16x8*>(wdst + ((p * 4 + wave) * 64 + lane) * 8) = fr;
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
                *reinterpret_cast<f16x4*>(udst + ((ct * 4 + p) * 64 + lane) * 4) = fr;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Stage 2: inter-chunk state recurrence.  One workgroup per (sequence, value
// head, 64-column block); wave w owns 16 state columns for the whole sequence
// and keeps them in accumulator registers (8 tiles of 16 d_k rows).
//
// Per chunk the workgroup reads 42 KB: -W fragments (16 KB), K^T fragments
// (16 KB), the U fragments of its 4 column tiles (8 KB) and the decay
// vectors.  They arrive by direct global-to-LDS copies (no registers) into a
// ring of three LDS stages, two chunks ahead of the chunk being computed.
// Every wave issues the same fixed number of copies per chunk, so one
// explicit memory-counter wait plus a barrier makes a stage complete.
//
// Each chunk's results for the output stage (its incoming state and U') are
// stored at the top of the next chunk from one of two register sets that
// alternate, so a store always has a whole chunk to retire before its data
// registers are rewritten; vector-memory counters retire in order and a
// store's data registers cannot be reused before it has.
// ---------------------------------------------------------------------------
constexpr int kStages = 3;
constexpr int kStageU = 4 * 4 * 64 * 4;          // halves: U fragments of 4 column tiles
constexpr int kCopiesPerChunk = 4 + 4 + 2 + 2;    // per wave: -W, K^T, U, decay vectors

struct StateStage {
    f16 w[kWElems];
    f16 k[kKtElems];
    f16 u[kStageU];
    float g[4][2 * kChunk];   // per-wave copy of e^{G_C - G_r} and e^{G_r}
};

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One chunk's copies for this wave: 1 KB pieces (16 B per lane) of -W, K^T
// and U, and the two 256 B decay vectors (4 B per lane) into the wave's copy.
__device__ __forceinline__ void state_copy(StateStage& st, const ChunkWorkspace& ws, size_t wsidx,
                                           size_t ktidx, int cb, int wave, int lane) {
    const f16* wsrc = ws.w + wsidx * kWElems;
    const f16* ksrc = ws.kt + ktidx * kKtElems;
    const f16* usrc = ws.u + wsidx * kUElems + (size_t)cb * kStageU;
    const float* gsrc = ws.gcum + wsidx * kGElems;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int piece = wave * 4 + i;
        __builtin_amdgcn_global_load_lds(wsrc + (piece * 64 + lane) * 8, st.w + piece * 512, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(ksrc + (piece * 64 + lane) * 8, st.k + piece * 512, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int piece = wave * 2 + i;
        __builtin_amdgcn_global_load_lds(usrc + (piece * 64 + lane) * 8, st.u + piece * 512, 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_global_load_lds(gsrc + i * 64 + lane, &st.g[wave][i * 64], 4, 0, 0);
}

// Results of one chunk that the output stage needs.
struct StateOut {
    f16x8 hb[4];   // incoming chunk state, B fragments over d_k
    f16x8 up[2];   // U', B fragments over positions
};

__device__ __forceinline__ void state_store(const StateOut& o, const ChunkWorkspace& ws, size_t wsidx,
                                            int ct, int lane) {
    f16* hdst = ws.hc + wsidx * kHcElems;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
        *reinterpret_cast<f16x8*>(hdst + ((ct * 4 + qq) * 64 + lane) * 8) = o.hb[qq];
    f16* udst = ws.up + wsidx * kUpElems;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
        *reinterpret_cast<f16x8*>(udst + ((ct * 2 + qq) * 64 + lane) * 8) = o.up[qq];
}

// One chunk of the recurrence for this wave's 16 columns.
__device__ __forceinline__ void state_chunk(f32x4 (&H)[8], const StateStage& st, StateOut& o,
                                            int wave, int lane, int gq) {
    // U accumulator fragments of this wave's column tile
    f32x4 acc[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f16x4 uf = *reinterpret_cast<const f16x4*>(&st.u[((wave * 4 + p) * 64 + lane) * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[p][e] = static_cast<float>(uf[e]);
    }
    // incoming chunk state as B fragments (d_k slots), kept for the output stage
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) o.hb[qq] = cat_to_f16(H[2 * qq], H[2 * qq + 1]);
    // U' = U + (-W) H
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f16x8 wa = *reinterpret_cast<const f16x8*>(&st.w[((p * 4 + qq) * 64 + lane) * 8]);
            acc[p] = mfma_f16(wa, o.hb[qq], acc[p]);
        }
    // U' as B fragments (position slots), kept for the output stage
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) o.up[qq] = cat_to_f16(acc[2 * qq], acc[2 * qq + 1]);
    // X = diag(e^{G_C - G}) U';   H <- e^{G_C} H + K^T X
    const float* dec = st.g[wave];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[p][e] *= dec[16 * p + 4 * gq + e];
    f16x8 xb[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) xb[qq] = cat_to_f16(acc[2 * qq], acc[2 * qq + 1]);
    const float gam = dec[kChunk + kChunk - 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) H[i] *= gam;
    // eight independent accumulator chains, interleaved
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f16x8 ka = *reinterpret_cast<const f16x8*>(&st.k[((i * 2 + qq) * 64 + lane) * 8]);
            H[i] = mfma_f16(ka, xb[qq], H[i]);
        }
}

__global__ __launch_bounds__(256) void gdn_chunk_state(
    const int32_t* __restrict__ cu, int n_seqs, int h_qk, int h_v,
    const float* __restrict__ s0, float* __restrict__ s_final, ChunkWorkspace ws)
{
    const int nh = blockIdx.x;
    const int seq = nh / h_v;
    const int h = nh % h_v;
    const int cb = blockIdx.y;
    const int j = h / (h_v / h_qk);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int gq = lane >> 4;
    const int ln = lane & 15;
    const int ct = cb * 4 + wave;        // column tile 0..7
    const int col = 16 * ct + ln;

    __shared__ __attribute__((aligned(16))) StateStage stage[kStages];

    const int start = cu[seq];
    const int end = cu[seq + 1];
    const int nchunks = (end - start + kChunk - 1) / kChunk;
    const int slot0 = slot_base(cu, seq);
    const int last = nchunks - 1;
    auto widx = [&](int c) { return (size_t)(slot0 + min(c, last)) * h_v + h; };
    auto kidx = [&](int c) { return (size_t)(slot0 + min(c, last)) * h_qk + j; };

    // ---- incoming state
    f32x4 H[8];
    const size_t sbase = ((size_t)seq * h_v + h) * kDim * kDim;
    if (s0) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                H[i][e] = s0[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) H[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // settle the initial-state loads before the copies start counting
    __builtin_amdgcn_s_waitcnt(0);

    if (nchunks > 0) {
        // copies are issued for chunks past the last one too (clamped to the
        // last chunk, never used) so the count in flight is always the same
        state_copy(stage[0], ws, widx(0), kidx(0), cb, wave, lane);
        state_copy(stage[1], ws, widx(1), kidx(1), cb, wave, lane);
        StateOut pa, pb;
        int c = 0;
        for (;;) {
            // chunk c (even) -> pa
            wait_vmcnt<kCopiesPerChunk>();      // this wave's copies of chunk c have landed
            wg_barrier();                       // ... and every other wave's
            if (c > 0) state_store(pb, ws, widx(c - 1), ct, lane);
            state_copy(stage[(c + 2) % kStages], ws, widx(c + 2), kidx(c + 2), cb, wave, lane);
            state_chunk(H, stage[c % kStages], pa, wave, lane, gq);
            if (++c >= nchunks) break;
            // chunk c (odd) -> pb
            wait_vmcnt<kCopiesPerChunk>();
            wg_barrier();
            state_store(pa, ws, widx(c - 1), ct, lane);
            state_copy(stage[(c + 2) % kStages], ws, widx(c + 2), kidx(c + 2), cb, wave, lane);
            state_chunk(H, stage[c % kStages], pb, wave, lane, gq);
            if (++c >= nchunks) break;
        }
        if (nchunks & 1) state_store(pa, ws, widx(last), ct, lane);
        else state_store(pb, ws, widx(last), ct, lane);
        // drain the copies of the two chunks past the end before the workgroup
        // exits (the LDS they target must stay allocated until they land)
        __builtin_amdgcn_s_waitcnt(0);
    }

    if (s_final) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s_final[sbase + (size_t)(16 * i + 4 * gq + e) * kDim + col] = H[i][e];
    }
}

// ---------------------------------------------------------------------------
// Stage 3: output.  One workgroup per (chunk slot, value head).
//   O = diag(e^G) Q H0 + P U',   P = M o (Q K^T)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gdn_chunk_out(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ cu, int n_seqs, int h_qk, int h_v,
    float* __restrict__ out, ChunkWorkspace ws)
{
    const int slot = blockIdx.x;
    const int h = blockIdx.y;
    int seq, t0, len;
    if (!resolve_slot(cu, n_seqs, slot, seq, t0, len)) return;
    const int j = h / (h_v / h_qk);

    __shared__ __attribute__((aligned(16))) f16 Qs[kChunk * kQS];   // Q [pos][dim]
    __shared__ __attribute__((aligned(16))) f16 Ks[kChunk * kQS];   // K [pos][dim]
    __shared__ __attribute__((aligned(16))) f16 Ps[kChunk * kTS];   // P [pos][pos]
    __shared__ float Gs[kChunk];   // G_r
    __shared__ float Es[kChunk];   // e^{G_r}

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int gq = lane >> 4;
    const int ln = lane & 15;
    const size_t wsidx = (size_t)slot * h_v + h;

    for (int i = tid; i < kChunk * 16; i += 256) {
        const int r = i >> 4;
        const int c8 = (i & 15) * 8;
        u16x8 qb = {0, 0, 0, 0, 0, 0, 0, 0};
        u16x8 kb = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < len) {
            qb = *reinterpret_cast<const u16x8*>(q + ((size_t)(t0 + r) * h_qk + j) * kDim + c8);
            kb = *reinterpret_cast<const u16x8*>(k + ((size_t)(t0 + r) * h_qk + j) * kDim + c8);
        }
        *reinterpret_cast<f16x8*>(Qs + r * kQS + c8) = bf16x8_to_f16x8(qb);
        *reinterpret_cast<f16x8*>(Ks + r * kQS + c8) = bf16x8_to_f16x8(kb);
    }
    if (tid < kChunk) {
        Gs[tid] = ws.gcum[wsidx * kGElems + 128 + tid];
        Es[tid] = ws.gcum[wsidx * kGElems + 64 + tid];
    }
    __syncthreads();

    // ---- P = M o (Q K^T); wave w owns row tile w, zero above the diagonal
    {
        const int p = wave;
        f16x8 qa[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qa[kk] = *reinterpret_cast<const f16x8*>(Qs + (16 * p + ln) * kQS + 32 * kk + 8 * gq);
        for (int jt = 0; jt < 4; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (jt <= p) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const f16x8 kb = *reinterpret_cast<const f16x8*>(Ks + (16 * jt + ln) * kQS + 32 * kk + 8 * gq);
                    acc = mfma_f16(qa[kk], kb, acc);
                }
            }
            const int s = 16 * jt + ln;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * p + 4 * gq + e;
                Ps[r * kTS + s] = static_cast<f16>((s <= r) ? acc[e] * exp_f(Gs[r] - Gs[s]) : 0.f);
            }
        }
    }
    __syncthreads();

    // ---- O tiles: wave w owns column tiles 2w, 2w+1, all four row tiles
    f32x4 o[4][2];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a) o[p][a] = f32x4{0.f, 0.f, 0.f, 0.f};

    const f16* hsrc = ws.hc + wsidx * kHcElems;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        f16x8 hb[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            hb[a] = *reinterpret_cast<const f16x8*>(hsrc + (((2 * wave + a) * 4 + qq) * 64 + lane) * 8);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f16* qrow = Qs + (16 * p + ln) * kQS;
            const f16x4 lo = *reinterpret_cast<const f16x4*>(qrow + 32 * qq + 4 * gq);
            const f16x4 hi = *reinterpret_cast<const f16x4*>(qrow + 32 * qq + 16 + 4 * gq);
            const f16x8 qa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int a = 0; a < 2; ++a) o[p][a] = mfma_f16(qa, hb[a], o[p][a]);
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float f = Es[16 * p + 4 * gq + e];
            o[p][0][e] *= f;
            o[p][1][e] *= f;
        }

    const f16* usrc = ws.up + wsidx * kUpElems;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        f16x8 ub[2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
            ub[a] = *reinterpret_cast<const f16x8*>(usrc + (((2 * wave + a) * 2 + qq) * 64 + lane) * 8);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const f16* prow = Ps + (16 * p + ln) * kTS;
            const f16x4 lo = *reinterpret_cast<const f16x4*>(prow + 32 * qq + 4 * gq);
            const f16x4 hi = *reinterpret_cast<const f16x4*>(prow + 32 * qq + 16 + 4 * gq);
            const f16x8 pa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int a = 0; a < 2; ++a) o[p][a] = mfma_f16(pa, ub[a], o[p][a]);
        }
    }

#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * p + 4 * gq + e;
            if (r < len) {
                float* orow = out + ((size_t)(t0 + r) * h_v + h) * kDim;
#pragma unroll
                for (int a = 0; a < 2; ++a) orow[16 * (2 * wave + a) + ln] = o[p][a][e];
            }
        }
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_chunk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const int32_t* cu,
                            int n_seqs, int64_t total_tokens, int h_qk, int h_v,
                            const float* s0, float* out, float* s_final,
                            const ChunkWorkspace& ws, int n_slots, int stage_mask,
                            hipStream_t stream)
{
    if ((stage_mask & 1) && total_tokens > 0) {
        hipLaunchKernelGGL(gdn_chunk_prep, dim3(n_slots, h_v), dim3(256), 0, stream,
                           k, v, g, beta, cu, n_seqs, h_qk, h_v, ws);
    }
    if ((stage_mask & 2) && n_seqs > 0) {
        hipLaunchKernelGGL(gdn_chunk_state, dim3(n_seqs * h_v, kDim / 64), dim3(256), 0, stream,
                           cu, n_seqs, h_qk, h_v, s0, s_final, ws);
    }
    if ((stage_mask & 4) && total_tokens > 0) {
        hipLaunchKernelGGL(gdn_chunk_out, dim3(n_slots, h_v), dim3(256), 0, stream,
                           q, k, cu, n_seqs, h_qk, h_v, out, ws);
    }
    return hipGetLastError();
}

}  // namespace gdn

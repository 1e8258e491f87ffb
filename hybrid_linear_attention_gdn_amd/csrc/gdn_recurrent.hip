// Per-token Gated DeltaNet update for decode and speculative verify (gfx950).
//
// The verify step of the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page
// (section 1) runs 1 + K query tokens per request through every layer; the
// "Qwen3.8-27B on one RTX 3090" page keeps one state snapshot per
// speculative token so the state can roll back to the last accepted one.
// Per request and value head, for each new token (state H = S^T, d_k x d_v):
//
//   H <- alpha H;  delta = beta (v - H^T k);  H <- H + k delta^T;  o = H^T q
//
// The work is a stream of fp32 state: 64 KB read per (request, head) and,
// when snapshots are kept, 64 KB written per token.  One workgroup of 256
// threads owns 64 state columns of one (request, head); thread (row group
// rg = tid / 16, column quad cq = tid % 16) holds rows rg + 16 i (i = 0..7)
// of 4 adjacent columns as float4 in registers for all tokens.  Column sums
// over d_k reduce across the 4 row groups of a wave with lane shuffles and
// across the 4 waves through LDS.  Rows are contiguous 256-byte runs per
// 16 lanes, so every state load and store is a full 16-byte access.

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

__device__ __forceinline__ float4 shfl_xor4(float4 x, int m) {
    return make_float4(__shfl_xor(x.x, m, 64), __shfl_xor(x.y, m, 64),
                       __shfl_xor(x.z, m, 64), __shfl_xor(x.w, m, 64));
}

__device__ __forceinline__ float4 operator+(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
    return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}

// State storage: fp32, or fp16 (the "Qwen3.8-27B on one RTX 3090" page,
// section "Exploiter l'architecture hybride", keeps the per-request state in
// fp16).  Arithmetic is fp32 either way; fp16 stores round to nearest even.
__device__ __forceinline__ float4 load_state4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load_state4(const f16* p) {
    const f16x4 x = *reinterpret_cast<const f16x4*>(p);
    return make_float4(static_cast<float>(x[0]), static_cast<float>(x[1]),
                       static_cast<float>(x[2]), static_cast<float>(x[3]));
}
__device__ __forceinline__ void store_state4(float* p, float4 s) {
    *reinterpret_cast<float4*>(p) = s;
}
__device__ __forceinline__ void store_state4(f16* p, float4 s) {
    const f16x4 x = {static_cast<f16>(s.x), static_cast<f16>(s.y), static_cast<f16>(s.z), static_cast<f16>(s.w)};
    *reinterpret_cast<f16x4*>(p) = x;
}
// The outgoing state, which this launch never reads back: non-temporal, so
// that a large batch of states streams past the caches (measured: 128
// requests with separate in and out states, 106 -> 82 us).
__device__ __forceinline__ void stream_state4(float* p, float4 s) {
    const f32x4 x = {s.x, s.y, s.z, s.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

struct RecurrentArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    float* out;
    int h_qk, h_v;
    // contiguous layout: request r owns rows r * n_tok .. + n_tok - 1
    int n_tok;
    const void* s_in;
    void* s_out;
    void* inter;
    int save;
    // slot-pool layout
    const int32_t* cu_tokens;
    int64_t total_tokens;
    int max_tok;
    void* pool;
    int64_t pool_slots;
    const int32_t* table;      // [R][max_tok + 1]
    const int32_t* accepted;   // [R] or null
};

template <typename StateT, bool kPooled>
__global__ __launch_bounds__(256) void gdn_recurrent_kernel(RecurrentArgs a)
{
    const int rh = blockIdx.x;
    const int req = rh / a.h_v;
    const int h = rh % a.h_v;
    const int j = h / (a.h_v / a.h_qk);
    const int h_qk = a.h_qk, h_v = a.h_v;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int cq = tid & 15;
    const int rg = tid >> 4;
    const int col0 = 64 * blockIdx.y + 4 * cq;
    constexpr size_t kHeadElems = (size_t)kDim * kDim;

    // Token inputs are staged in LDS a block of kTokBlock tokens at a time, so
    // the token loop issues no global loads between its state stores: on this
    // GPU loads and stores retire in one in-order counter, and a load issued
    // behind a token's snapshot stores would wait for all of them.
    constexpr int kTokBlock = 16;
    __shared__ float kqs[kTokBlock][2][kDim];   // k, q per staged token
    __shared__ float4 vs[kTokBlock][16];        // this workgroup's 64 columns of v
    __shared__ float gs[kTokBlock], bs[kTokBlock];
    __shared__ int wss[kTokBlock];              // pool layout: write slot per token
    __shared__ float4 red[2][4][16];            // per-wave column partials (prediction, output)

    // Load order: everything that does not depend on a slot index first.
    // (1) the request's token range and accepted count; (2) the incoming slot
    // and the first block of token inputs; (3) the state.  The write slots are
    // checked while the state loads are in flight.
    int64_t t_begin;
    int n;
    const int32_t* row = nullptr;       // this request's slot-table row
    int rs = 0;
    if constexpr (kPooled) {
        // Every index below is checked before it is used to address memory.
        const int64_t tb = a.cu_tokens[req], te = a.cu_tokens[req + 1];
        const int col = a.accepted ? a.accepted[req] : 0;
        if (tb < 0 || te < tb || te > a.total_tokens || te - tb > a.max_tok) return;  // rows unknown
        t_begin = tb;
        n = (int)(te - tb);
        row = a.table + (size_t)req * (a.max_tok + 1);
        rs = (col >= 0 && col <= a.max_tok) ? row[col] : -1;
    } else {
        t_begin = (int64_t)req * a.n_tok;
        n = a.n_tok;
    }

    // Stage token inputs [blk, blk + nb) in LDS: loads into registers first
    // (stage_load), the LDS writes later (stage_store), so that other loads
    // can be issued in between.
    struct Staged {
        u16x8 kq[2];
        u16x4 v;
        float g, b;
        int w;
    };
    auto stage_load = [&](int blk, int nb) {
        Staged st = {};
        const int idx = tid;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {     // nb <= 16: k, q in two passes of 8 tokens
            const int i2 = idx + 256 * pass;
            if (i2 < nb * 32) {
                const int tt = i2 >> 5, e = (i2 & 31) * 8;
                const size_t t = (size_t)(t_begin + blk + tt);
                const uint16_t* srcp = e < kDim ? a.k + (t * h_qk + j) * kDim + e
                                                : a.q + (t * h_qk + j) * kDim + e - kDim;
                st.kq[pass] = *reinterpret_cast<const u16x8*>(srcp);
            }
        }
        if (idx < nb * 16) {
            const int tt = idx >> 4, c4 = idx & 15;
            const size_t t = (size_t)(t_begin + blk + tt);
            st.v = *reinterpret_cast<const u16x4*>(a.v + (t * h_v + h) * kDim + 64 * blockIdx.y + 4 * c4);
        }
        if (idx < nb) {
            const size_t t = (size_t)(t_begin + blk + idx);
            st.g = a.g[t * h_v + h];
            st.b = a.beta[t * h_v + h];
            if constexpr (kPooled) st.w = row[1 + blk + idx];
        }
        return st;
    };
    auto stage_store = [&](const Staged& st, int nb) {
        const int idx = tid;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int i2 = idx + 256 * pass;
            if (i2 < nb * 32) {
                const int tt = i2 >> 5, e = (i2 & 31) * 8;
                float* d = &kqs[tt][0][0] + e;
#pragma unroll
                for (int c = 0; c < 8; ++c) d[c] = bf16_to_f32(st.kq[pass][c]);
            }
        }
        if (idx < nb * 16) {
            const int tt = idx >> 4, c4 = idx & 15;
            vs[tt][c4] = make_float4(bf16_to_f32(st.v[0]), bf16_to_f32(st.v[1]), bf16_to_f32(st.v[2]), bf16_to_f32(st.v[3]));
        }
        if (idx < nb) {
            gs[idx] = exp_f(st.g);
            bs[idx] = st.b;
            wss[idx] = st.w;
        }
    };

    const int nb0 = min(kTokBlock, n);
    Staged st0 = stage_load(0, nb0);

    const StateT* src;
    if constexpr (kPooled) {
        int bad = (rs < 0 || rs >= a.pool_slots) ? 1 : 0;
        for (int t = tid; t < n; t += 256) bad |= (row[1 + t] >= a.pool_slots) ? 1 : 0;
        if (__syncthreads_or(bad)) {
            // invalid slot index: NaN outputs, no state read or written
            const float nan = __builtin_nanf("");
            for (int idx = tid; idx < n * 16; idx += 256)
                *reinterpret_cast<float4*>(a.out + ((t_begin + idx / 16) * h_v + h) * kDim + 64 * blockIdx.y + 4 * (idx % 16)) =
                    make_float4(nan, nan, nan, nan);
            return;
        }
        src = static_cast<const StateT*>(a.pool) + ((size_t)rs * h_v + h) * kHeadElems;
    } else {
        src = static_cast<const StateT*>(a.s_in) + ((size_t)req * h_v + h) * kHeadElems;
    }

    float4 S[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = load_state4(src + (size_t)(rg + 16 * i) * kDim + col0);

    for (int blk = 0; blk < n; blk += kTokBlock) {
        const int nb = min(kTokBlock, n - blk);
        if (blk > 0) {
            __syncthreads();   // previous block's staged inputs are consumed
            stage_store(stage_load(blk, nb), nb);
        } else {
            stage_store(st0, nb);
        }
        __syncthreads();

        for (int tt = 0; tt < nb; ++tt) {
            const int tau = blk + tt;
            const size_t t = (size_t)(t_begin + tau);
            const float alpha = gs[tt];
            const float b = bs[tt];
            const float4 vv = vs[tt][cq];

            float kr[8], qr[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kr[i] = kqs[tt][0][rg + 16 * i];
                qr[i] = kqs[tt][1][rg + 16 * i];
            }

            // decay and prediction p = (alpha H)^T k over this thread's rows
            float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                S[i] = make_float4(S[i].x * alpha, S[i].y * alpha, S[i].z * alpha, S[i].w * alpha);
                p = fma4(kr[i], S[i], p);
            }
            p = p + shfl_xor4(p, 16);
            p = p + shfl_xor4(p, 32);
            if ((tid & 63) < 16) red[0][wave][cq] = p;
            __syncthreads();
            p = red[0][0][cq] + red[0][1][cq] + red[0][2][cq] + red[0][3][cq];

            // delta = beta (v - p); H += k delta^T; o = H^T q
            const float4 d = make_float4(b * (vv.x - p.x), b * (vv.y - p.y), b * (vv.z - p.z), b * (vv.w - p.w));
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                S[i] = fma4(kr[i], d, S[i]);
                o = fma4(qr[i], S[i], o);
            }
            o = o + shfl_xor4(o, 16);
            o = o + shfl_xor4(o, 32);
            if ((tid & 63) < 16) red[1][wave][cq] = o;

            StateT* dst = nullptr;
            if constexpr (kPooled) {
                const int ws = wss[tt];
                if (ws >= 0) dst = static_cast<StateT*>(a.pool) + ((size_t)ws * h_v + h) * kHeadElems;
            } else if (a.save) {
                dst = static_cast<StateT*>(a.inter) + (((size_t)req * n + tau) * h_v + h) * kHeadElems;
            }
            if (dst) {
#pragma unroll
                for (int i = 0; i < 8; ++i) store_state4(dst + (size_t)(rg + 16 * i) * kDim + col0, S[i]);
            }
            __syncthreads();
            if (tid < 16) {
                const float4 os = red[1][0][cq] + red[1][1][cq] + red[1][2][cq] + red[1][3][cq];
                *reinterpret_cast<float4*>(a.out + (t * h_v + h) * kDim + col0) = os;
            }
        }
    }

    if constexpr (!kPooled) {
        if (a.s_out) {
            StateT* dst = static_cast<StateT*>(a.s_out) + ((size_t)req * h_v + h) * kHeadElems;
#pragma unroll
            for (int i = 0; i < 8; ++i) stream_state4(dst + (size_t)(rg + 16 * i) * kDim + col0, S[i]);
        }
    }
}

}  // namespace

hipError_t launch_recurrent_step(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* g, const float* beta, int n_req, int n_tok,
                                 int h_qk, int h_v, const float* s_in, float* s_out,
                                 float* out, float* inter, int save, hipStream_t stream)
{
    RecurrentArgs a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.out = out;
    a.h_qk = h_qk; a.h_v = h_v;
    a.n_tok = n_tok; a.s_in = s_in; a.s_out = s_out; a.inter = inter; a.save = save;
    hipLaunchKernelGGL((gdn_recurrent_kernel<float, false>), dim3(n_req * h_v, kDim / 64), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_recurrent_step_slots(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const float* g, const float* beta, const int32_t* cu_tokens,
                                       int n_req, int max_tok, int64_t total_tokens, int h_qk, int h_v,
                                       void* pool, int state_f16, int64_t pool_slots,
                                       const int32_t* table, const int32_t* accepted,
                                       float* out, hipStream_t stream)
{
    RecurrentArgs a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.out = out;
    a.h_qk = h_qk; a.h_v = h_v;
    a.cu_tokens = cu_tokens; a.total_tokens = total_tokens; a.max_tok = max_tok;
    a.pool = pool; a.pool_slots = pool_slots; a.table = table; a.accepted = accepted;
    const dim3 grid(n_req * h_v, kDim / 64);
    if (state_f16)
        hipLaunchKernelGGL((gdn_recurrent_kernel<f16, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((gdn_recurrent_kernel<float, true>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gdn

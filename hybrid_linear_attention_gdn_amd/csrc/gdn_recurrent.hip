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

__global__ __launch_bounds__(256) void gdn_recurrent_step_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    int n_tok, int h_qk, int h_v,
    const float* s_in, float* s_out, float* __restrict__ out,
    float* __restrict__ inter, int save)
{
    const int rh = blockIdx.x;
    const int req = rh / h_v;
    const int h = rh % h_v;
    const int j = h / (h_v / h_qk);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int cq = tid & 15;
    const int rg = tid >> 4;
    const int col0 = 64 * blockIdx.y + 4 * cq;

    __shared__ float kq[2][kDim];       // k, q of the current token
    __shared__ float4 red[2][4][16];    // per-wave column partials (prediction, output)

    const size_t sbase = ((size_t)req * h_v + h) * kDim * kDim;
    float4 S[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        S[i] = *reinterpret_cast<const float4*>(s_in + sbase + (size_t)(rg + 16 * i) * kDim + col0);

    for (int tau = 0; tau < n_tok; ++tau) {
        const size_t t = (size_t)req * n_tok + tau;
        if (tid < kDim) kq[0][tid] = bf16_to_f32(k[(t * h_qk + j) * kDim + tid]);
        else kq[1][tid - kDim] = bf16_to_f32(q[(t * h_qk + j) * kDim + tid - kDim]);
        const float alpha = exp_f(g[t * h_v + h]);
        const float b = beta[t * h_v + h];
        const u16x4 vb = *reinterpret_cast<const u16x4*>(v + (t * h_v + h) * kDim + col0);
        const float4 vv = make_float4(bf16_to_f32(vb[0]), bf16_to_f32(vb[1]),
                                      bf16_to_f32(vb[2]), bf16_to_f32(vb[3]));
        __syncthreads();

        float kr[8], qr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kr[i] = kq[0][rg + 16 * i];
            qr[i] = kq[1][rg + 16 * i];
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

        if (save) {
            float* dst = inter + (((size_t)req * n_tok + tau) * h_v + h) * kDim * kDim;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<float4*>(dst + (size_t)(rg + 16 * i) * kDim + col0) = S[i];
        }
        __syncthreads();
        if (tid < 16) {
            const float4 os = red[1][0][cq] + red[1][1][cq] + red[1][2][cq] + red[1][3][cq];
            *reinterpret_cast<float4*>(out + (t * h_v + h) * kDim + col0) = os;
        }
    }

    if (s_out) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<float4*>(s_out + sbase + (size_t)(rg + 16 * i) * kDim + col0) = S[i];
    }
}

}  // namespace

hipError_t launch_recurrent_step(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* g, const float* beta, int n_req, int n_tok,
                                 int h_qk, int h_v, const float* s_in, float* s_out,
                                 float* out, float* inter, int save, hipStream_t stream)
{
    hipLaunchKernelGGL(gdn_recurrent_step_kernel, dim3(n_req * h_v, kDim / 64), dim3(256), 0, stream,
                       q, k, v, g, beta, n_tok, h_qk, h_v, s_in, s_out, out, inter, save);
    return hipGetLastError();
}

}  // namespace gdn

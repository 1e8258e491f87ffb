// C ABI of libgdn.so: host-side validation, workspace carving and launches.
// Validation reads only host values; nothing here touches device memory or
// synchronises, except the checks GDN_DEBUG_CHECKS turns on.  See
// include/gdn.h for the contract.

#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn_launch.h"
#include "gdn_validate.h"

using gdn::aligned16;
using gdn::fail;
using gdn::kAlign;
using gdn::Layout;
using gdn::ok;

namespace {

// GDN_DEBUG_CHECKS (any value but "" or "0") makes every entry point copy its
// inputs to the host and check the device-content preconditions before any
// launch: a debugging aid that synchronises the stream and allocates host
// memory, never meant for a timed or captured call.
bool debug_checks() {
    const char* e = getenv("GDN_DEBUG_CHECKS");
    return e && *e && strcmp(e, "0") != 0;
}

template <typename T>
hipError_t to_host(std::vector<T>& dst, const void* src, size_t n) {
    dst.resize(n);
    if (n == 0 || !src) return hipSuccess;
    return hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost);
}

gdn_status debug_check_chunk(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const int32_t* cu, const float* s0, const gdn_dims* d, void* stream) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    const size_t T = (size_t)d->total_tokens, N = (size_t)d->n_seqs;
    const size_t nqk = T * d->n_heads_qk * d->d_k, nv = T * d->n_heads_v * d->d_v, ng = T * d->n_heads_v;
    std::vector<uint16_t> hq, hk, hv;
    std::vector<float> hg, hb, hs;
    std::vector<int32_t> hc;
    if (e == hipSuccess) e = to_host(hc, cu, N + 1);
    if (e == hipSuccess) e = to_host(hq, q, nqk);
    if (e == hipSuccess) e = to_host(hk, k, nqk);
    if (e == hipSuccess) e = to_host(hv, v, nv);
    if (e == hipSuccess) e = to_host(hg, g, ng);
    if (e == hipSuccess) e = to_host(hb, beta, ng);
    if (e == hipSuccess && s0) e = to_host(hs, s0, N * d->n_heads_v * d->d_k * d->d_v);
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "GDN_DEBUG_CHECKS copy: %s", hipGetErrorString(e));
    return gdn_check_chunk_inputs_host(hq.data(), hk.data(), hv.data(), hg.data(), hb.data(), hc.data(),
                                       s0 ? hs.data() : nullptr, d);
}

gdn_status debug_check_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const float* state_in, int64_t n_states, const gdn_dims* d, void* stream) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    const size_t T = (size_t)d->total_tokens;
    const size_t nqk = T * d->n_heads_qk * d->d_k, nv = T * d->n_heads_v * d->d_v, ng = T * d->n_heads_v;
    std::vector<uint16_t> hq, hk, hv;
    std::vector<float> hg, hb, hs;
    if (e == hipSuccess) e = to_host(hq, q, nqk);
    if (e == hipSuccess) e = to_host(hk, k, nqk);
    if (e == hipSuccess) e = to_host(hv, v, nv);
    if (e == hipSuccess) e = to_host(hg, g, ng);
    if (e == hipSuccess) e = to_host(hb, beta, ng);
    if (e == hipSuccess && state_in) e = to_host(hs, state_in, (size_t)n_states * d->n_heads_v * d->d_k * d->d_v);
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "GDN_DEBUG_CHECKS copy: %s", hipGetErrorString(e));
    return gdn_check_step_inputs_host(hq.data(), hk.data(), hv.data(), hg.data(), hb.data(),
                                      state_in ? hs.data() : nullptr, n_states, d);
}

#define GDN_REQUIRE_PTR(p)                                                              \
    do {                                                                                \
        if (!(p)) return fail(GDN_ERR_INVALID_VALUE, "%s is NULL", #p);                 \
        if (!aligned16(p)) return fail(GDN_ERR_MISALIGNED, "%s is not 16-byte aligned", #p); \
    } while (0)

#define GDN_OPTIONAL_PTR(p)                                                             \
    do {                                                                                \
        if ((p) && !aligned16(p)) return fail(GDN_ERR_MISALIGNED, "%s is not 16-byte aligned", #p); \
    } while (0)

}  // namespace

// The prefill entry points' common body (also behind the no-allocation
// variant in gdn_noalloc.hip, which passes its own scratch as the workspace).
gdn_status gdn::chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, const float* initial_state, float* out,
                          float* final_state, float* chunk_states, const gdn_dims* dims,
                          void* workspace, size_t workspace_bytes, int stage_mask, void* stream,
                          const char* what, int32_t seg_chunks) {
    if (stage_mask < 1 || stage_mask > 3)
        return fail(GDN_ERR_INVALID_VALUE, "stage_mask = %d is outside 1..3", stage_mask);
    gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    if (dims->n_seqs == 0) return ok();   // nothing to do, nothing to write
    GDN_REQUIRE_PTR(cu_seqlens);
    GDN_OPTIONAL_PTR(initial_state);
    GDN_OPTIONAL_PTR(final_state);
    GDN_OPTIONAL_PTR(chunk_states);
    if (dims->total_tokens > 0) {
        GDN_REQUIRE_PTR(q);
        GDN_REQUIRE_PTR(k);
        GDN_REQUIRE_PTR(v);
        GDN_REQUIRE_PTR(g);
        GDN_REQUIRE_PTR(beta);
        GDN_REQUIRE_PTR(out);
    }
    // one long sequence through gdn_chunk_fwd runs range by range, in a
    // workspace laid out for one range
    const int range = (stage_mask == 3 && !chunk_states && seg_chunks == 0) ? gdn::chunk_range(dims) : 0;
    const Layout L = range ? gdn::range_layout(dims, range) : gdn::workspace_layout(dims, seg_chunks);
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", L.total);
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(GDN_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, L.total);
    const int64_t slots = gdn::n_chunk_slots(dims);
    if (debug_checks() && (stage_mask & 1)) {
        s = debug_check_chunk(q, k, v, g, beta, cu_seqlens, initial_state, dims, stream);
        if (s != GDN_SUCCESS) return s;
    }

    char* base = static_cast<char*>(workspace);
    gdn::ChunkWorkspace ws;
    ws.tu = reinterpret_cast<gdn::f16*>(base + L.tu);
    ws.p = reinterpret_cast<gdn::f16*>(base + L.p);
    ws.dg = reinterpret_cast<float*>(base + L.dg);
    ws.kt = reinterpret_cast<gdn::f16*>(base + L.kt);
    ws.qf = reinterpret_cast<gdn::f16*>(base + L.qf);
    ws.junk = reinterpret_cast<float*>(base + L.junk);
    ws.n_slots = (int)slots;
    ws.group = dims->n_heads_v / dims->n_heads_qk;
    ws.h_v = dims->n_heads_v;
    ws.h_qk = dims->n_heads_qk;

    gdn::SegLaunch seg;
    if (seg_chunks > 0) {
        const int64_t segslots = gdn::n_seg_slots(dims, seg_chunks);
        if (segslots * dims->n_heads_v > gdn::kMaxHeadUnits)
            return fail(GDN_ERR_INVALID_VALUE, "%lld segments x H_v exceed %lld (segment_chunks too small)",
                        (long long)segslots, gdn::kMaxHeadUnits);
        seg.seg_chunks = seg_chunks;
        seg.n_segslots = (int)segslots;
        seg.maps = reinterpret_cast<float*>(base + L.maps);
        seg.hstart = reinterpret_cast<float*>(base + L.hstart);
    }
    const hipError_t e = gdn::launch_chunk_fwd(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        g, beta, cu_seqlens, dims->n_seqs, dims->total_tokens, dims->n_heads_qk, dims->n_heads_v,
        initial_state, out, final_state, chunk_states, ws, (int)slots, stage_mask,
        seg_chunks > 0 ? &seg : nullptr, range, reinterpret_cast<float*>(base + L.carry),
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

using gdn::chunk_fwd_impl;

extern "C" {

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const int32_t* cu_seqlens,
                         const float* initial_state,
                         float* out,
                         float* final_state,
                         const gdn_dims* dims,
                         void* workspace, size_t workspace_bytes,
                         void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, nullptr,
                          dims, workspace, workspace_bytes, 3, stream, "gdn_chunk_fwd");
}

gdn_status gdn_chunk_fwd_snapshots(const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const int32_t* cu_seqlens,
                                   const float* initial_state,
                                   float* out,
                                   float* final_state,
                                   float* chunk_states,
                                   const gdn_dims* dims,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (dims && dims->n_seqs > 0 && !chunk_states)
        return fail(GDN_ERR_INVALID_VALUE, "chunk_states is NULL");
    return chunk_fwd_impl(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, chunk_states,
                          dims, workspace, workspace_bytes, 3, stream, "gdn_chunk_fwd_snapshots");
}


gdn_status gdn_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const int32_t* cu_seqlens,
                                   const float* initial_state,
                                   float* out,
                                   float* final_state,
                                   int32_t segment_chunks,
                                   const gdn_dims* dims,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (segment_chunks < 1) return fail(GDN_ERR_INVALID_VALUE, "segment_chunks = %d must be positive", segment_chunks);
    return chunk_fwd_impl(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, nullptr,
                          dims, workspace, workspace_bytes, 3, stream, "gdn_chunk_fwd_segmented", segment_chunks);
}

gdn_status gdn_chunk_fwd_stages(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const int32_t* cu_seqlens,
                                const float* initial_state,
                                float* out,
                                float* final_state,
                                const gdn_dims* dims,
                                void* workspace, size_t workspace_bytes,
                                int stage_mask,
                                void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, nullptr,
                          dims, workspace, workspace_bytes, stage_mask, stream, "gdn_chunk_fwd_stages");
}

gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              int32_t n_requests, int32_t tokens_per_request,
                              const float* state_in,
                              float* state_out,
                              float* out,
                              float* intermediate_states,
                              int save_intermediate_states,
                              const gdn_dims* dims,
                              void* stream) {
    gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    if (n_requests < 0 || tokens_per_request < 0)
        return fail(GDN_ERR_INVALID_VALUE, "negative n_requests (%d) or tokens_per_request (%d)",
                    n_requests, tokens_per_request);
    if (dims->n_seqs != n_requests)
        return fail(GDN_ERR_INVALID_VALUE, "dims->n_seqs = %d differs from n_requests = %d",
                    dims->n_seqs, n_requests);
    if (dims->total_tokens != (int64_t)n_requests * tokens_per_request)
        return fail(GDN_ERR_INVALID_VALUE, "dims->total_tokens = %lld differs from %d x %d",
                    (long long)dims->total_tokens, n_requests, tokens_per_request);
    if (n_requests == 0) return ok();
    GDN_REQUIRE_PTR(state_in);
    GDN_OPTIONAL_PTR(state_out);
    GDN_OPTIONAL_PTR(intermediate_states);
    if (save_intermediate_states && !intermediate_states)
        return fail(GDN_ERR_INVALID_VALUE, "intermediate_states is NULL but save_intermediate_states is set");
    if (!save_intermediate_states && intermediate_states)
        return fail(GDN_ERR_INVALID_VALUE, "intermediate_states given but save_intermediate_states is 0");
    if (!state_out && !save_intermediate_states)
        return fail(GDN_ERR_INVALID_VALUE, "state_out is NULL and no intermediate states are saved");
    if (tokens_per_request > 0) {
        GDN_REQUIRE_PTR(q);
        GDN_REQUIRE_PTR(k);
        GDN_REQUIRE_PTR(v);
        GDN_REQUIRE_PTR(g);
        GDN_REQUIRE_PTR(beta);
        GDN_REQUIRE_PTR(out);
    }
    if (debug_checks()) {
        s = debug_check_step(q, k, v, g, beta, state_in, n_requests, dims, stream);
        if (s != GDN_SUCCESS) return s;
    }
    const hipError_t e = gdn::launch_recurrent_step(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        g, beta, n_requests, tokens_per_request, dims->n_heads_qk, dims->n_heads_v,
        state_in, state_out, out, intermediate_states, save_intermediate_states ? 1 : 0,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "gdn_recurrent_step launch: %s", hipGetErrorString(e));
    return ok();
}

gdn_status gdn_recurrent_step_slots(const void* q, const void* k, const void* v,
                                    const float* g, const float* beta,
                                    const int32_t* cu_tokens,
                                    int32_t n_requests, int32_t max_tokens,
                                    void* state_pool, int32_t state_dtype, int64_t pool_slots,
                                    const int32_t* slot_table,
                                    const int32_t* num_accepted,
                                    float* out,
                                    const gdn_dims* dims,
                                    void* stream) {
    gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    if (n_requests < 0 || max_tokens < 0)
        return fail(GDN_ERR_INVALID_VALUE, "negative n_requests (%d) or max_tokens (%d)", n_requests, max_tokens);
    if (dims->n_seqs != n_requests)
        return fail(GDN_ERR_INVALID_VALUE, "dims->n_seqs = %d differs from n_requests = %d",
                    dims->n_seqs, n_requests);
    if (state_dtype != GDN_STATE_F32 && state_dtype != GDN_STATE_F16)
        return fail(GDN_ERR_INVALID_VALUE, "state_dtype = %d is not a gdn_state_dtype", state_dtype);
    if (pool_slots <= 0) return fail(GDN_ERR_INVALID_VALUE, "pool_slots = %lld must be positive", (long long)pool_slots);
    if (n_requests == 0) return ok();
    GDN_REQUIRE_PTR(state_pool);
    if (!cu_tokens) return fail(GDN_ERR_INVALID_VALUE, "cu_tokens is NULL");
    if (!slot_table) return fail(GDN_ERR_INVALID_VALUE, "slot_table is NULL");
    if ((reinterpret_cast<uintptr_t>(cu_tokens) & 3u) || (reinterpret_cast<uintptr_t>(slot_table) & 3u) ||
        (reinterpret_cast<uintptr_t>(num_accepted) & 3u))
        return fail(GDN_ERR_MISALIGNED, "int32 index arrays must be 4-byte aligned");
    if (dims->total_tokens > 0) {
        GDN_REQUIRE_PTR(q);
        GDN_REQUIRE_PTR(k);
        GDN_REQUIRE_PTR(v);
        GDN_REQUIRE_PTR(g);
        GDN_REQUIRE_PTR(beta);
        GDN_REQUIRE_PTR(out);
    }
    if (debug_checks()) {
        s = debug_check_step(q, k, v, g, beta, nullptr, 0, dims, stream);
        if (s != GDN_SUCCESS) return s;
    }
    const hipError_t e = gdn::launch_recurrent_step_slots(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        g, beta, cu_tokens, n_requests, max_tokens, dims->total_tokens, dims->n_heads_qk, dims->n_heads_v,
        state_pool, state_dtype == GDN_STATE_F16 ? 1 : 0, pool_slots, slot_table, num_accepted, out,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "gdn_recurrent_step_slots launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// C ABI of libgdn.so: host-side validation, workspace carving and launches.
// Validation reads only host values; nothing here touches device memory or
// synchronises.  See include/gdn.h for the contract.

#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "gdn_launch.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

gdn_status ok() {
    g_last_error[0] = '\0';
    return GDN_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Launch-size limits.  A dispatch holds at most 2^32 work-items per grid
// dimension: the state launch runs 8 column tiles of 192 threads (an affine
// map 16 of 128, the segment scan 8 of 256) per (sequence or segment, value
// head) pair, prep 256 threads per chunk slot with the value heads as the
// second grid dimension (at most 65535 workgroups there).
constexpr long long kMaxHeadUnits = 1LL << 21;
constexpr long long kMaxChunkSlots = 1LL << 24;
constexpr int kMaxValueHeads = 65535;

int64_t n_chunk_slots(const gdn_dims* d) {
    return (int64_t)d->n_seqs + d->total_tokens / gdn::kChunk + 1;
}

gdn_status check_dims(const gdn_dims* d) {
    if (!d) return fail(GDN_ERR_INVALID_VALUE, "dims is NULL");
    if (d->n_seqs < 0) return fail(GDN_ERR_INVALID_VALUE, "n_seqs = %d is negative", d->n_seqs);
    if (d->total_tokens < 0)
        return fail(GDN_ERR_INVALID_VALUE, "total_tokens = %lld is negative", (long long)d->total_tokens);
    if (d->total_tokens > 0x7fffffffLL)
        return fail(GDN_ERR_INVALID_VALUE, "total_tokens = %lld exceeds int32 cu_seqlens", (long long)d->total_tokens);
    if (d->n_seqs == 0 && d->total_tokens != 0)
        return fail(GDN_ERR_INVALID_VALUE, "total_tokens = %lld with no sequences", (long long)d->total_tokens);
    if (d->n_heads_qk <= 0 || d->n_heads_v <= 0)
        return fail(GDN_ERR_INVALID_VALUE, "head counts must be positive (H_qk = %d, H_v = %d)",
                    d->n_heads_qk, d->n_heads_v);
    if (d->n_heads_v % d->n_heads_qk != 0)
        return fail(GDN_ERR_INVALID_VALUE, "H_v = %d is not a multiple of H_qk = %d",
                    d->n_heads_v, d->n_heads_qk);
    if (d->d_k <= 0 || d->d_v <= 0)
        return fail(GDN_ERR_INVALID_VALUE, "head dims must be positive (d_k = %d, d_v = %d)", d->d_k, d->d_v);
    if (d->d_k != gdn::kDim || d->d_v != gdn::kDim)
        return fail(GDN_ERR_NOT_SUPPORTED, "only d_k = d_v = 128 is supported (got %d, %d)", d->d_k, d->d_v);
    if (d->n_heads_v > kMaxValueHeads)
        return fail(GDN_ERR_INVALID_VALUE, "H_v = %d exceeds %d", d->n_heads_v, kMaxValueHeads);
    const long long nh = (long long)d->n_seqs * d->n_heads_v;
    if (nh > kMaxHeadUnits)
        return fail(GDN_ERR_INVALID_VALUE, "n_seqs * H_v = %lld exceeds %lld", nh, kMaxHeadUnits);
    if (n_chunk_slots(d) > kMaxChunkSlots)
        return fail(GDN_ERR_INVALID_VALUE, "%lld chunk slots (N + T/64 + 1) exceed %lld",
                    (long long)n_chunk_slots(d), kMaxChunkSlots);
    return GDN_SUCCESS;
}

struct Layout {
    size_t w, u, p, dg, kt, qf, junk, maps, hstart, total;
};

// Segment slots of the segment-parallel recurrence (see gdn_chunk.hip).
int64_t n_seg_slots(const gdn_dims* d, int32_t seg_chunks) {
    return (int64_t)d->n_seqs + n_chunk_slots(d) / seg_chunks + 1;
}

Layout workspace_layout(const gdn_dims* d, int32_t seg_chunks = 0) {
    const size_t units = (size_t)n_chunk_slots(d) * (size_t)d->n_heads_v;
    Layout L;
    size_t off = 0;
    const size_t qk_units = (size_t)n_chunk_slots(d) * (size_t)d->n_heads_qk;
    L.w = off;  off += round_up(units * gdn::kWElems * sizeof(gdn::f16));
    L.u = off;  off += round_up(units * gdn::kUElems * sizeof(gdn::f16));
    L.p = off;  off += round_up(units * gdn::kPElems * sizeof(gdn::f16));
    L.dg = off; off += round_up(units * gdn::kGElems * sizeof(float));
    L.kt = off; off += round_up(qk_units * gdn::kKtElems * sizeof(gdn::f16));
    L.qf = off; off += round_up(qk_units * gdn::kQfElems * sizeof(gdn::f16));
    L.junk = off; off += round_up(gdn::kJunkBytes);
    L.maps = L.hstart = off;
    if (seg_chunks > 0) {
        const size_t per = (size_t)n_seg_slots(d, seg_chunks) * (size_t)d->n_heads_v * gdn::kDim * gdn::kDim * sizeof(float);
        L.maps = off;   off += round_up(2 * per);
        L.hstart = off; off += round_up(per);
    }
    L.total = off;
    return L;
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

extern "C" {

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_SUCCESS: return "success";
        case GDN_ERR_INVALID_VALUE: return "invalid value";
        case GDN_ERR_NOT_SUPPORTED: return "not supported";
        case GDN_ERR_MISALIGNED: return "misaligned pointer";
        case GDN_ERR_WORKSPACE: return "workspace too small";
        case GDN_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* gdn_get_last_error(void) { return g_last_error; }

gdn_status gdn_chunk_fwd_workspace_size(const gdn_dims* dims, size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_VALUE, "bytes is NULL");
    const gdn_status s = check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    *bytes = workspace_layout(dims).total;
    return ok();
}

gdn_status gdn_chunk_state_slots(const gdn_dims* dims, int64_t* n_slots) {
    if (!n_slots) return fail(GDN_ERR_INVALID_VALUE, "n_slots is NULL");
    const gdn_status s = check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    *n_slots = n_chunk_slots(dims);
    return ok();
}

namespace {

gdn_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, const float* initial_state, float* out,
                          float* final_state, float* chunk_states, const gdn_dims* dims,
                          void* workspace, size_t workspace_bytes, int stage_mask, void* stream,
                          const char* what, int32_t seg_chunks = 0) {
    if (stage_mask < 1 || stage_mask > 3)
        return fail(GDN_ERR_INVALID_VALUE, "stage_mask = %d is outside 1..3", stage_mask);
    gdn_status s = check_dims(dims);
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
    const Layout L = workspace_layout(dims, seg_chunks);
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes required)", L.total);
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(GDN_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
        return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, L.total);
    const int64_t slots = n_chunk_slots(dims);

    char* base = static_cast<char*>(workspace);
    gdn::ChunkWorkspace ws;
    ws.w = reinterpret_cast<gdn::f16*>(base + L.w);
    ws.u = reinterpret_cast<gdn::f16*>(base + L.u);
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
        const int64_t segslots = n_seg_slots(dims, seg_chunks);
        if (segslots * dims->n_heads_v > kMaxHeadUnits)
            return fail(GDN_ERR_INVALID_VALUE, "%lld segments x H_v exceed %lld (segment_chunks too small)",
                        (long long)segslots, kMaxHeadUnits);
        seg.seg_chunks = seg_chunks;
        seg.n_segslots = (int)segslots;
        seg.maps = reinterpret_cast<float*>(base + L.maps);
        seg.hstart = reinterpret_cast<float*>(base + L.hstart);
    }
    const hipError_t e = gdn::launch_chunk_fwd(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        g, beta, cu_seqlens, dims->n_seqs, dims->total_tokens, dims->n_heads_qk, dims->n_heads_v,
        initial_state, out, final_state, chunk_states, ws, (int)slots, stage_mask,
        seg_chunks > 0 ? &seg : nullptr, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

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

gdn_status gdn_chunk_fwd_segmented_workspace_size(const gdn_dims* dims, int32_t segment_chunks, size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_VALUE, "bytes is NULL");
    if (segment_chunks < 1) return fail(GDN_ERR_INVALID_VALUE, "segment_chunks = %d must be positive", segment_chunks);
    const gdn_status s = check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    *bytes = workspace_layout(dims, segment_chunks).total;
    return ok();
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
    gdn_status s = check_dims(dims);
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
    gdn_status s = check_dims(dims);
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
    const hipError_t e = gdn::launch_recurrent_step_slots(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        g, beta, cu_tokens, n_requests, max_tokens, dims->total_tokens, dims->n_heads_qk, dims->n_heads_v,
        state_pool, state_dtype == GDN_STATE_F16 ? 1 : 0, pool_slots, slot_table, num_accepted, out,
        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "gdn_recurrent_step_slots launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

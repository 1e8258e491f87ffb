// Host-only part of the C ABI (no HIP calls): see gdn_validate.h.

#include "gdn_validate.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

namespace gdn {

namespace {

thread_local char g_last_error[512] = "";

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr size_t kHalf = 2;           // bytes of an fp16 workspace element
constexpr float kF16Max = 65504.f;    // largest finite fp16

// bfloat16 bits -> float (exact)
float bf16_value(uint16_t b) {
    const uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

}  // namespace

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

int64_t n_chunk_slots(const gdn_dims* d) {
    return (int64_t)d->n_seqs + d->total_tokens / kChunk + 1;
}

// Segment slots of the segment-parallel recurrence (see gdn_chunk.hip).
int64_t n_seg_slots(const gdn_dims* d, int32_t seg_chunks) {
    return (int64_t)d->n_seqs + n_chunk_slots(d) / seg_chunks + 1;
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
    if (d->d_k != kDim || d->d_v != kDim)
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

namespace {

// The intermediates' regions for `slots` chunk slots, then the sink.
Layout slot_regions(const gdn_dims* d, int64_t slots, size_t& off) {
    const size_t units = (size_t)slots * (size_t)d->n_heads_v;
    const size_t qk_units = (size_t)slots * (size_t)d->n_heads_qk;
    Layout L = {};
    off = 0;
    L.tu = off; off += round_up(units * kTuElems * kHalf);
    L.p = off;  off += round_up(units * kPElems * kHalf);
    L.dg = off; off += round_up(units * kGElems * sizeof(float));
    L.kt = off; off += round_up(qk_units * kKtElems * kHalf);
    L.qf = off; off += round_up(qk_units * kQfElems * kHalf);
    L.junk = off; off += round_up(kJunkBytes);
    return L;
}

}  // namespace

Layout range_layout(const gdn_dims* d, int range) {
    size_t off = 0;
    Layout L = slot_regions(d, range, off);
    L.maps = L.hstart = L.carry = off;
    off += round_up((size_t)d->n_heads_v * kDim * kDim * sizeof(float));
    L.total = off;
    return L;
}

int chunk_range(const gdn_dims* d) {
    if (d->n_seqs != 1 ||
        (size_t)n_chunk_slots(d) * chunk_slot_bytes(d->n_heads_qk, d->n_heads_v) <= kStreamWorkspaceBytes)
        return 0;
    const int64_t nch = (d->total_tokens + kChunk - 1) / kChunk;
    const int range = (int)(nch < range_slots(d->n_heads_qk, d->n_heads_v) ? nch : range_slots(d->n_heads_qk, d->n_heads_v));
    // (with few chunks of very many heads one range is the whole sequence,
    //  and the single pass needs no more room)
    return range_layout(d, range).total < workspace_layout(d).total ? range : 0;
}

Layout workspace_layout(const gdn_dims* d, int32_t seg_chunks) {
    size_t off = 0;
    Layout L = slot_regions(d, n_chunk_slots(d), off);
    L.carry = off;
    L.maps = L.hstart = off;
    if (seg_chunks > 0) {
        const size_t per = (size_t)n_seg_slots(d, seg_chunks) * (size_t)d->n_heads_v * kDim * kDim * sizeof(float);
        L.maps = off;   off += round_up(2 * per);
        L.hstart = off; off += round_up(per);
    }
    L.total = off;
    return L;
}

gdn_status check_cu_seqlens(const int32_t* cu, int32_t n_seqs, int64_t total_tokens) {
    if (n_seqs < 0) return fail(GDN_ERR_INVALID_VALUE, "n_seqs = %d is negative", n_seqs);
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens[0] = %d, must be 0", cu[0]);
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu[n + 1] < cu[n])
            return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens decreases at %d (%d -> %d)", n, cu[n], cu[n + 1]);
    if ((int64_t)cu[n_seqs] != total_tokens)
        return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens[%d] = %d differs from total_tokens = %lld",
                    n_seqs, cu[n_seqs], (long long)total_tokens);
    return GDN_SUCCESS;
}

gdn_status check_gates(const float* g, const float* beta, int64_t count) {
    for (int64_t i = 0; i < count; ++i) {
        if (!isfinite(g[i]) || g[i] > 0.f)
            return fail(GDN_ERR_INVALID_VALUE, "g[%lld] = %g: the log-decay must be finite and <= 0",
                        (long long)i, (double)g[i]);
        if (!isfinite(beta[i]))
            return fail(GDN_ERR_INVALID_VALUE, "beta[%lld] = %g is not finite", (long long)i, (double)beta[i]);
    }
    return GDN_SUCCESS;
}

gdn_status check_bf16_operand(const uint16_t* x, int64_t count, const char* name) {
    for (int64_t i = 0; i < count; ++i) {
        const float f = bf16_value(x[i]);
        if (!isfinite(f) || fabsf(f) > kF16Max)
            return fail(GDN_ERR_INVALID_VALUE,
                        "%s[%lld] = %g: matrix-core operands are fp16, |x| must stay <= 65504",
                        name, (long long)i, (double)f);
    }
    return GDN_SUCCESS;
}

gdn_status check_state_values(const float* s, int64_t count, const char* name, bool fp16_operand) {
    for (int64_t i = 0; i < count; ++i) {
        if (!isfinite(s[i]))
            return fail(GDN_ERR_INVALID_VALUE, "%s[%lld] = %g is not finite", name, (long long)i, (double)s[i]);
        if (fp16_operand && fabsf(s[i]) > kF16Max)
            return fail(GDN_ERR_INVALID_VALUE,
                        "%s[%lld] = %g: the chunked path rounds states to fp16 operands, |x| must stay <= 65504",
                        name, (long long)i, (double)s[i]);
    }
    return GDN_SUCCESS;
}

}  // namespace gdn

using gdn::fail;
using gdn::ok;

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

const char* gdn_get_last_error(void) { return gdn::g_last_error; }

gdn_status gdn_chunk_fwd_workspace_size(const gdn_dims* dims, size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_VALUE, "bytes is NULL");
    const gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    *bytes = gdn::workspace_layout(dims).total;
    return ok();
}

gdn_status gdn_chunk_fwd_min_workspace_size(const gdn_dims* dims, size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_VALUE, "bytes is NULL");
    const gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    const int range = gdn::chunk_range(dims);
    *bytes = range ? gdn::range_layout(dims, range).total : gdn::workspace_layout(dims).total;
    return ok();
}

gdn_status gdn_chunk_state_slots(const gdn_dims* dims, int64_t* n_slots) {
    if (!n_slots) return fail(GDN_ERR_INVALID_VALUE, "n_slots is NULL");
    const gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    *n_slots = gdn::n_chunk_slots(dims);
    return ok();
}

gdn_status gdn_chunk_fwd_segmented_workspace_size(const gdn_dims* dims, int32_t segment_chunks, size_t* bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_VALUE, "bytes is NULL");
    if (segment_chunks < 1) return fail(GDN_ERR_INVALID_VALUE, "segment_chunks = %d must be positive", segment_chunks);
    const gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    *bytes = gdn::workspace_layout(dims, segment_chunks).total;
    return ok();
}

gdn_status gdn_check_chunk_inputs_host(const void* q, const void* k, const void* v,
                                       const float* g, const float* beta,
                                       const int32_t* cu_seqlens,
                                       const float* initial_state,
                                       const gdn_dims* dims) {
    gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    if (dims->n_seqs == 0) return ok();
    if (!cu_seqlens) return fail(GDN_ERR_INVALID_VALUE, "cu_seqlens is NULL");
    if ((s = gdn::check_cu_seqlens(cu_seqlens, dims->n_seqs, dims->total_tokens)) != GDN_SUCCESS) return s;
    const int64_t T = dims->total_tokens;
    if (T > 0) {
        if (!q || !k || !v || !g || !beta) return fail(GDN_ERR_INVALID_VALUE, "a token input is NULL");
        const int64_t nqk = T * dims->n_heads_qk * dims->d_k, nv = T * dims->n_heads_v * dims->d_v;
        if ((s = gdn::check_bf16_operand(static_cast<const uint16_t*>(q), nqk, "q")) != GDN_SUCCESS) return s;
        if ((s = gdn::check_bf16_operand(static_cast<const uint16_t*>(k), nqk, "k")) != GDN_SUCCESS) return s;
        if ((s = gdn::check_bf16_operand(static_cast<const uint16_t*>(v), nv, "v")) != GDN_SUCCESS) return s;
        if ((s = gdn::check_gates(g, beta, T * dims->n_heads_v)) != GDN_SUCCESS) return s;
    }
    if (initial_state) {
        const int64_t n = (int64_t)dims->n_seqs * dims->n_heads_v * dims->d_k * dims->d_v;
        if ((s = gdn::check_state_values(initial_state, n, "initial_state", true)) != GDN_SUCCESS) return s;
    }
    return ok();
}

gdn_status gdn_check_step_inputs_host(const void* q, const void* k, const void* v,
                                      const float* g, const float* beta,
                                      const float* state_in, int64_t n_states,
                                      const gdn_dims* dims) {
    gdn_status s = gdn::check_dims(dims);
    if (s != GDN_SUCCESS) return s;
    if (n_states < 0) return fail(GDN_ERR_INVALID_VALUE, "n_states = %lld is negative", (long long)n_states);
    const int64_t T = dims->total_tokens;
    if (T > 0) {
        if (!q || !k || !v || !g || !beta) return fail(GDN_ERR_INVALID_VALUE, "a token input is NULL");
        const int64_t nqk = T * dims->n_heads_qk * dims->d_k, nv = T * dims->n_heads_v * dims->d_v;
        if ((s = gdn::check_bf16_operand(static_cast<const uint16_t*>(q), nqk, "q")) != GDN_SUCCESS) return s;
        if ((s = gdn::check_bf16_operand(static_cast<const uint16_t*>(k), nqk, "k")) != GDN_SUCCESS) return s;
        if ((s = gdn::check_bf16_operand(static_cast<const uint16_t*>(v), nv, "v")) != GDN_SUCCESS) return s;
        if ((s = gdn::check_gates(g, beta, T * dims->n_heads_v)) != GDN_SUCCESS) return s;
    }
    if (state_in && n_states > 0) {
        const int64_t n = n_states * dims->n_heads_v * dims->d_k * dims->d_v;
        if ((s = gdn::check_state_values(state_in, n, "state_in", false)) != GDN_SUCCESS) return s;
    }
    return ok();
}

}  // extern "C"

// Host-side part of the C ABI that needs no GPU: status and error text, size
// checks, the workspace layout, and the device-content precondition checks
// run on host copies.  Built with a plain C++ compiler as well as hipcc, so
// that it can be exercised under AddressSanitizer and UBSan on the CPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_sizes.h"

namespace gdn {

gdn_status fail(gdn_status s, const char* fmt, ...);
gdn_status ok();
bool aligned16(const void* p);

constexpr size_t kAlign = 256;   // workspace alignment and region rounding

// Launch-size limits.  A dispatch holds at most 2^32 work-items per grid
// dimension: the state launch runs 8 column tiles of 192 threads (an affine
// map 16 of 128, the segment scan 8 of 256) per (sequence or segment, value
// head) pair, prep 256 threads per chunk slot with the value heads as the
// second grid dimension (at most 65535 workgroups there).
constexpr long long kMaxHeadUnits = 1LL << 21;
constexpr long long kMaxChunkSlots = 1LL << 24;
constexpr int kMaxValueHeads = 65535;

int64_t n_chunk_slots(const gdn_dims* d);
int64_t n_seg_slots(const gdn_dims* d, int32_t seg_chunks);
gdn_status check_dims(const gdn_dims* d);

struct Layout {
    size_t tu, p, dg, kt, qf, junk, maps, hstart, carry, total;
};
// Every chunk slot's intermediates (the single pass; with seg_chunks > 0
// the segment maps and incoming states too).
Layout workspace_layout(const gdn_dims* d, int32_t seg_chunks = 0);
// Chunks per range when gdn_chunk_fwd runs the batch range by range (one
// sequence whose intermediates exceed kStreamWorkspaceBytes: range_slots
// of them, at most the sequence's chunks), else 0 (the single pass).
int chunk_range(const gdn_dims* d);
// The workspace of range-by-range execution: one range's intermediates and
// the state carried between ranges.
Layout range_layout(const gdn_dims* d, int range);

// Device-content preconditions on host copies (see gdn_check_*_host in gdn.h).
gdn_status check_cu_seqlens(const int32_t* cu, int32_t n_seqs, int64_t total_tokens);
gdn_status check_gates(const float* g, const float* beta, int64_t count);
gdn_status check_bf16_operand(const uint16_t* x, int64_t count, const char* name);
gdn_status check_state_values(const float* s, int64_t count, const char* name, bool fp16_operand);

}  // namespace gdn

// Sizes shared by the kernels and the host-side validation (no HIP types, so
// the host part of the library also builds with a plain C++ compiler).
#pragma once

#include <stddef.h>

namespace gdn {

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kDim = 128;   // d_k = d_v

// Per (chunk slot, value head) element counts of the workspace regions, all
// in matrix-core fragment order (two bytes per element except kGElems).
// TU = Tm diag(beta), the UT transform's rows scaled by beta, and
// P = M o (Q K^T): A fragments over positions of their six nonzero (row tile,
// K-step) blocks (0,0) (1,0) (2,0) (2,1) (3,0) (3,1) (both lower triangular)
constexpr size_t kTuElems = 6 * 64 * 8;
constexpr size_t kPElems = 6 * 64 * 8;
// decay vectors: e^{G_C - G_r} for r < 63 (the factor of row 63 is 1) with
// e^{G_C} in entry 63, then e^{G_r} for r = 0..63 (fp32)
constexpr size_t kGElems = 128;
// Per (chunk slot, q/k head): K^T as A fragments of the state update
// [d_k tile][pos step][lane][8], and Q as A fragments over d_k [p][qq][lane][8]
constexpr size_t kKtElems = 8 * 2 * 64 * 8;
constexpr size_t kQfElems = 4 * 4 * 64 * 8;
constexpr size_t kJunkBytes = 1024;         // sink for the lanes of masked-off stores

// -W as A fragments of W H0 [p][qq][lane][8]: formed on chip from K^T and TU
// (LDS only, not a workspace region)
constexpr size_t kWElems = 16 * 64 * 8;

// Workspace bytes of one chunk slot (all heads): TU, P and the decay vectors
// per value head, K^T and Q per q/k head.
constexpr size_t chunk_slot_bytes(int h_qk, int h_v) {
    return (size_t)h_v * ((kTuElems + kPElems) * 2 + kGElems * 4) + (size_t)h_qk * (kKtElems + kQfElems) * 2;
}

// Intermediates above which prep streams its stores past the caches, and
// above which one sequence runs range by range.
constexpr size_t kStreamWorkspaceBytes = (size_t)160 << 20;

// Value heads per prep workgroup: two when the value heads of a q/k head
// pair up (an even number of them), else one.
constexpr int prep_value_heads(int h_qk, int h_v) { return (h_v / h_qk) % 2 == 0 ? 2 : 1; }

// Chunk slots per range when one sequence runs range by range: one full
// round of prep workgroups (four per CU on the 256 CUs of an MI355X), a
// multiple of 8, at least 8.
constexpr int range_slots(int h_qk, int h_v) {
    const int per_slot = h_v / prep_value_heads(h_qk, h_v);      // prep workgroups per chunk slot
    const int r = (4 * 256 / per_slot) & ~7;
    return r < 8 ? 8 : r;
}

}  // namespace gdn

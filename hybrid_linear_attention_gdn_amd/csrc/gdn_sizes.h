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

}  // namespace gdn

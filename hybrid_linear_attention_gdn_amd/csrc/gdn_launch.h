// Host-side launchers of the gfx950 kernels (called by the C ABI layer).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_device.h"

namespace gdn {

// Segment-parallel recurrence: segments of seg_chunks chunks, their affine
// maps and incoming states in caller memory (sizes from the host).
struct SegLaunch {
    int seg_chunks;
    int n_segslots;
    float* hstart;      // [n_segslots][h_v][128][128]
    float* maps;        // [n_segslots][h_v][2][128][128]
};

// Enqueues the intra-chunk preparation of chunk slots slot_lo .. slot_hi - 1
// (one workgroup per chunk slot and pair of value heads sharing a q/k head,
// or per value head when they do not pair up) on `stream`, with ordinary or
// with non-temporal stores of the intermediates, which go to workspace slots
// 0 .. slot_hi - slot_lo - 1.
hipError_t launch_prep(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g, const float* beta,
                       const int32_t* cu, int n_seqs, int h_qk, int h_v, const ChunkWorkspace& ws, int slot_lo,
                       int slot_hi, hipStream_t stream);
hipError_t launch_prep_stream(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                              const float* beta, const int32_t* cu, int n_seqs, int h_qk, int h_v,
                              const ChunkWorkspace& ws, int slot_lo, int slot_hi, hipStream_t stream);

// Enqueues the chunked prefill on `stream`: prep (stage bit 0) and the state
// recurrence with the output (stage bit 1); chunk_states may be null; seg
// null runs each sequence's recurrence in one workgroup per column tile.
// range > 0 runs one sequence range by range (both stages): prep and the
// recurrence over `range` chunk slots at a time, the workspace regions
// holding one range's slots and `carry` the state between ranges
// ([h_v][128][128] fp32).
hipError_t launch_chunk_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const float* g, const float* beta, const int32_t* cu,
                            int n_seqs, int64_t total_tokens, int h_qk, int h_v,
                            const float* s0, float* out, float* s_final, float* chunk_states,
                            const ChunkWorkspace& ws, int n_slots, int stage_mask,
                            const SegLaunch* seg, int range, float* carry, hipStream_t stream);

// Body of the prefill entry points: host validation, workspace carving into
// the regions above, and the launches (seg_chunks > 0: segment-parallel).
gdn_status chunk_fwd_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, const float* initial_state, float* out,
                          float* final_state, float* chunk_states, const gdn_dims* dims,
                          void* workspace, size_t workspace_bytes, int stage_mask, void* stream,
                          const char* what, int32_t seg_chunks = 0);

// Enqueues the per-token recurrent update on `stream`.
hipError_t launch_recurrent_step(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const float* g, const float* beta, int n_req, int n_tok,
                                 int h_qk, int h_v, const float* s_in, float* s_out,
                                 float* out, float* inter, int save, hipStream_t stream);

// Enqueues the per-token update over a pool of state slots (fp32 or fp16).
hipError_t launch_recurrent_step_slots(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const float* g, const float* beta, const int32_t* cu_tokens,
                                       int n_req, int max_tok, int64_t total_tokens, int h_qk, int h_v,
                                       void* pool, int state_f16, int64_t pool_slots,
                                       const int32_t* table, const int32_t* accepted,
                                       float* out, hipStream_t stream);

}  // namespace gdn

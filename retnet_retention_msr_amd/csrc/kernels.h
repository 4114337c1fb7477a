// Host-side launchers of the retention kernels. Each returns the HIP status of
// the launch (hipGetLastError after enqueueing); arguments were validated by
// the C ABI before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace ret {

// Sizes shared by the launchers.
struct Dims {
  int B, H, N, dk, dv;
};

// Recurrent decode step (one token): state <- gamma*state + k^T v, o = q.state.
hipError_t launch_decode_step(int dtype, const void* q, const void* k, const void* v, float* state,
                              void* o, int B, int H, int dk, int dv, const HeadDecay& decay,
                              const GnArgs& gn, hipStream_t stream);

// Generic (VALU, any element type) chunk-state walk: writes the fp32 state in
// force before every chunk to `chunk_states` [B*H][nchunks][dk][dv] and the final
// state to state_out (if non-null).
hipError_t launch_generic_state_walk(int dtype, const void* k, const void* v, const float* state_in,
                                     float* state_out, float* chunk_states, const Dims& d, int chunk,
                                     const HeadDecay& decay, hipStream_t stream);

// Generic (VALU) output rows: intra-chunk causal part plus, when chunk_states
// is non-null, the cross-chunk read-out of the state before the row's chunk.
// With chunk >= N and no states this is the parallel form.
// `accumulate`: add the values already in o (partial results summed over
// launches) instead of overwriting them.
hipError_t launch_generic_chunk_out(int dtype, const void* q, const void* k, const void* v,
                                    const float* chunk_states, bool state_for_chunk0, void* o,
                                    const Dims& d, int chunk, const HeadDecay& decay, const GnArgs& gn,
                                    bool accumulate, hipStream_t stream);

// bf16 MFMA chunk-state walk: writes the bf16 state before every chunk in a
// [B*H][nchunks][dv][dk] (dk fastest) layout, and the fp32 final state.
// chunks_per_seg < nchunks splits each sequence into chunk-aligned segments
// walked in parallel; seg_states (fp32 [B*H][nseg][dk][dv]) then holds the
// segments' end states and the final state before it is copied to state_out.
hipError_t launch_mfma_state_walk(const uint16_t* k, const uint16_t* v, const float* state_in,
                                  float* state_out, uint16_t* chunk_states, float* seg_states, int chunks_per_seg,
                                  const Dims& d, int chunk, const HeadDecay& decay, hipStream_t stream);

// k-tile height of the walk is 32 * walk_k_tiles(dk); walk_tiles_per_head is
// the number of workgroups per head and segment for `heads` = B*H heads.
// walk_wide: the full-dk walk takes 256 v columns per workgroup, used when
// those workgroups alone are enough to fill the GPU (the walk is then not
// segmented); otherwise 128.
int walk_k_tiles(int dk);
bool walk_wide(int64_t heads, int dk, int dv);
int walk_tiles_per_head(int64_t heads, int dk, int dv);

// bf16 MFMA output: per 64-row query block, intra-chunk causal product plus the
// read-out of the bf16 chunk state (when chunk_states is non-null), then the
// optional GroupNorm. With chunk >= N and no states this is the parallel form.
hipError_t launch_mfma_chunk_out(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* chunk_states, bool state_for_chunk0, uint16_t* o,
                                 const Dims& d, int chunk, const HeadDecay& decay, const GnArgs& gn,
                                 bool accumulate, hipStream_t stream);

// Whether the MFMA kernels implement these sizes.
bool mfma_supports(int dk, int dv);

// Backward-pass data movement (d.B, d.H, d.N are used; rows are tokens).
// split_rows: src [B*H, N, D] read once, written to up to three targets, each
// cut into parts of width part_w (the last may be narrower), part p at
// dst + p * part_stride elements as [B*H, N, w_p], rows token-reversed within
// each head when `flip`.
struct SplitTarget {
  void* dst;
  int part_w;
  int64_t part_stride;
  bool flip;
};
hipError_t launch_split_rows(int dtype, const void* src, const SplitTarget* targets, int ntargets, const Dims& d,
                             int D, hipStream_t stream);
// sum_parts: dst [B*H, N, W] = sum of nparts buffers [B*H, N, W] (part_stride
// elements apart), read token-reversed when `flip`; fp32 sums.
hipError_t launch_sum_parts(int dtype, const void* parts, void* dst, const Dims& d, int W, int nparts,
                            int64_t part_stride, bool flip, hipStream_t stream);
// state_prep: fp32 [B*H, R, C] times a per-head factor (head_factor: host
// array of H floats, nullptr = 1), or its transpose split into parts of
// part_w rows ([B*H, w_p, R] each, part_stride elements apart).
hipError_t launch_state_prep(const float* src, float* dst, int B, int H, int R, int C, bool transpose, int part_w,
                             int64_t part_stride, const float* head_factor, hipStream_t stream);

}  // namespace ret

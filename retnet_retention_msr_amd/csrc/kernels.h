// Host-side launchers of the retention kernels and the planning functions of
// the C ABI. Each launcher returns the HIP status of the launch
// (hipGetLastError after enqueueing); arguments were validated by the C ABI
// before these are called. This header is plain host C++ (HIP runtime API
// types only), so the validation and planning code that includes it also
// builds with a host compiler alone.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace ret {

constexpr int kMaxHeads = 256;

// log2(gamma_h) per head, computed on the host in double precision and
// rounded once to float. A decay power gamma^e is formed as exp2(e * log2g).
struct HeadDecay {
  float log2g[kMaxHeads];
};

struct GnArgs {
  int enabled;
  float eps;
  const float* weight;  // [H*dv] or nullptr
  const float* bias;    // [H*dv] or nullptr
  const void* gate;     // like O (element type of the inputs), or nullptr
};

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
// The full-dk walk form covers these dk.
bool walk_full_dk(int dk);
// Whether a segmented walk runs once from zero plus the fix-up pass (true) or
// twice (segment end states first, then every segment from its true start).
bool walk_fixup_segments(int chunk, int dk, int dv);

// bf16 MFMA output: per 64-row query block, intra-chunk causal product plus the
// read-out of the bf16 chunk state (when chunk_states is non-null), then the
// optional GroupNorm. With chunk >= N and no states this is the parallel form.
hipError_t launch_mfma_chunk_out(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* chunk_states, bool state_for_chunk0, uint16_t* o,
                                 const Dims& d, int chunk, const HeadDecay& decay, const GnArgs& gn,
                                 bool accumulate, hipStream_t stream);

// Whether the MFMA kernels implement these sizes.
bool mfma_supports(int dk, int dv);

// Single-pass chunkwise kernel (fused.hip): one workgroup per (head, 256-column
// v tile) walks the chunks with its state slab in registers; GroupNorm
// statistics are exchanged between the v tiles of a head through a small
// workspace (fused_workspace_bytes). Covers dk 128 and 256, dv a multiple of
// 256 up to 1024, chunk a multiple of 64. With chunks_per_seg below the chunk
// count the sequences are cut into segments of that many chunks, each walked
// by its own workgroups from the state seg_states gives it: fp32
// [B*H][nseg][dk][dv], slot s < nseg-1 the end state of segment s started
// from zero (segment 0 from state_in), as launch_segment_ends leaves it.
// `layout` (optional) reads q and k with row pitches ldq, ldk (elements),
// takes every sequence in reverse token order (logical row t at memory row
// N-1-t, for q, k, v and o alike), and may add a second retention of the same
// sizes and pitches to the launch (its own operands, output, starting state
// and order; no final state): the units of the two run side by side. It
// excludes segments and the gate; reverse order needs (N-1)*max(ldq, ldk,
// dv)*2 below 2^30; with a second retention the workspace holds the exchange
// words of twice the units.
struct FusedJob {
  const uint16_t* q = nullptr;
  const uint16_t* k = nullptr;
  const uint16_t* v = nullptr;
  uint16_t* o = nullptr;
  const float* state_in = nullptr;
  bool reverse = false;
};
struct FusedLayout {
  int ldq = 0, ldk = 0;  // 0: dk
  bool reverse = false;
  const FusedJob* second = nullptr;
};
bool fused_supports(int dk, int dv, int chunk);
size_t fused_workspace_bytes(int64_t heads, int dv);
hipError_t launch_fused_chunkwise(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                  const float* state_in, float* state_out, void* workspace, const Dims& d, int chunk,
                                  const HeadDecay& decay, const GnArgs& gn, bool accumulate, hipStream_t stream,
                                  int chunks_per_seg = 0, const float* seg_states = nullptr,
                                  const FusedLayout* layout = nullptr);
// End states of segments 0..nseg-2 (segments of chunks_per_seg chunks), each
// walked from zero (segment 0 from state_in), into seg_states [B*H][nseg][dk][dv]
// (the MFMA state walk's first mode; dk 128 or 256, dv a multiple of 128).
hipError_t launch_segment_ends(const uint16_t* k, const uint16_t* v, const float* state_in, float* seg_states,
                               int chunks_per_seg, const Dims& d, int chunk, const HeadDecay& decay,
                               hipStream_t stream);

// xPos rotation (xpos.hip): the pairs (x[2i], x[2i+1]) of every position n
// of q (and of k, unless null) multiplied, as complex numbers, by
// exp(i (pos0 + n) theta_i); theta is a host array of d/2 angles, d <= 2 *
// kMaxXposPairs. Outputs may be the inputs (in place). BH = B * H heads of N
// positions, [BH][N][d] contiguous.
constexpr int kMaxXposPairs = 128;
hipError_t launch_xpos_rotate(int dtype, const void* q, const void* k, void* q_out, void* k_out, const float* theta,
                              int BH, int N, int d, int64_t pos0, hipStream_t stream);

// Device-to-device copy of `bytes` bytes on `stream`.
hipError_t copy_device(void* dst, const void* src, size_t bytes, hipStream_t stream);

// Bytes of the library-owned device scratch (scratch.hip) that the
// allocation-free chunkwise entry point uses instead of a caller workspace.
constexpr size_t kScratchBytes = size_t{64} << 20;

// Device address of this GPU's copy of the scratch (the current device's),
// looked up with hipGetSymbolAddress on the first call per device and kept.
hipError_t scratch_pointer(void** out);

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

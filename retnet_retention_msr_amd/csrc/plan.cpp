// Planning functions of the C ABI: which kernels cover which sizes, and how
// the state walk is tiled. Pure host code (no HIP calls), shared by the
// launchers in mfma.hip and by the validation and planning in api.cpp.
#include <cstdint>

#include "kernels.h"

namespace ret {

// v columns per workgroup of the narrow walk forms (both walk kernels).
constexpr int kWalkNarrowVT = 128;

bool mfma_supports(int dk, int dv) {
  return dk % 32 == 0 && dk >= 32 && dk <= 256 && (dv == 128 || dv == 256 || dv == 512);
}

int walk_k_tiles(int dk) { return (dk % 64 == 0) ? 2 : 1; }

// A segmented walk either runs twice (segment end states from zero, then every
// segment from its true start) or once from zero followed by a fix-up pass
// that reads and rewrites the chunk states of segments 1.. (2 x 2 bytes per
// state element and chunk, against 2 (dk + dv) bytes per token for a second
// walk's K and V). Measured on B1 H16 dk256 dv512: the fix-up wins from
// chunk 256 on (where it moves up to twice the bytes of a second walk, which
// is latency-bound) and loses at 64 and 128.
bool walk_fixup_segments(int chunk, int dk, int dv) {
  return 1LL * dk * dv < static_cast<int64_t>(chunk) * (dk + dv);
}

// The full-dk walk covers dk = 128 and 256 with one workgroup per 128 v columns.
bool walk_full_dk(int dk) { return dk == 128 || dk == 256; }

// 256 v columns per workgroup (each K row then crosses from L2 to LDS dv/256
// times instead of dv/128, and a wave's 64 x 128 accumulator slab halves the
// LDS operand reads per product) when those workgroups alone fill the GPU;
// with fewer heads, 128-column workgroups and segments give more parallelism.
constexpr int64_t kWalkWideBlocks = 256;
bool walk_wide(int64_t heads, int dk, int dv) {
  return walk_full_dk(dk) && dv % 256 == 0 && heads * (dv / 256) >= kWalkWideBlocks;
}

int walk_tiles_per_head(int64_t heads, int dk, int dv) {
  if (walk_full_dk(dk)) return dv / (walk_wide(heads, dk, dv) ? 256 : kWalkNarrowVT);
  return (dk / (32 * walk_k_tiles(dk))) * (dv / kWalkNarrowVT);
}

// The single-pass kernel: dk 128 or 256 (its state slab, 32 columns by dk
// rows per wave, fits the register budget), v tiles of 256 columns (at most
// four per head: the GroupNorm merge), query blocks of 64 rows.
bool fused_supports(int dk, int dv, int chunk) {
  return (dk == 128 || dk == 256) && dv % 256 == 0 && dv / 256 <= 4 && chunk % 64 == 0;
}

// Its workspace: per (head, v tile) two mailbox slots of 64 rows, each row
// two tagged 64-bit words (mean, sum of squared deviations): 2 KiB.
size_t fused_workspace_bytes(int64_t heads, int dv) {
  const size_t units = static_cast<size_t>(heads) * (dv / 256);
  return units * 2 * 64 * 2 * sizeof(uint64_t);
}

}  // namespace ret

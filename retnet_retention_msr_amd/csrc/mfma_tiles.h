// Device helpers shared by the MFMA retention kernels (gfx950): operand
// loads in the v_mfma_f32_32x32x16_bf16 / 16x16x32 layouts, buffer
// descriptors, direct global->LDS copies, the swizzled LDS tile layouts and
// lane-exchange reductions.
//
// MFMA 32x32x16 operand layouts (lane l of 64):
//   A[i][kk]: i = l % 32, kk = 8*(l/32) + 0..7
//   B[kk][j]: j = l % 32, kk = 8*(l/32) + 0..7
//   D[i][j] : j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4 for accumulator r = 0..15
#pragma once

#include <cstdint>

#include "common.h"

namespace ret {
namespace {

constexpr int kXcds = 8;

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Transposed operand from a row-major LDS tile: lane l receives
// tile[row0 + 8*(l/32) + i][col0 + l%32] for i = 0..7 (an MFMA A or B operand
// whose contraction index runs down the tile's rows). Two ds_read_b64_tr_b16:
// within each 16-lane group, lane j points at row (j/4) and columns 4*(j%4)..+3
// of a 4 x 16 block; lane i then holds column i of that block's four rows.
__device__ __forceinline__ bf16x8 ld_tr8(const uint16_t* tile, int pitch, int row0, int col0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = tile + (row0 + 8 * (g >> 1) + (j >> 2)) * pitch + col0 + 16 * (g & 1) + 4 * (j & 3);
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p + 4 * pitch));
  const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Logical workgroup index such that consecutive logical indices share an XCD.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
  const int full = (nblocks / kXcds) * kXcds;
  if (b >= full) return b;
  return (b % kXcds) * (full / kXcds) + b / kXcds;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferConfig = 0x00020000;  // raw buffer descriptor word 3 for gfx9-family loads
constexpr int kOutOfRange = 0x40000000;     // an offset past any tile: the load returns zero

// Buffer descriptor over `nbytes` bytes at `base`; loads past the end return zero.
// `base` and `nbytes` must be the same in every lane of the wave: they are
// read from the first active lane, so the descriptor lives in scalar
// registers (otherwise the compiler wraps each load in a loop over the
// distinct descriptors of the wave).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, static_cast<short>(0), __builtin_amdgcn_readfirstlane(nbytes),
                                           kBufferConfig);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0);
}

// Wait until this wave's global loads (including the direct LDS copies) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for outstanding global loads and stores (or copies into LDS).
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// gamma^e through the hardware exp2 (results below the normal range flush to 0).
__device__ __forceinline__ float gpow(float log2g, float e) { return __builtin_amdgcn_exp2f(e * log2g); }

__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, int byte_offset, const bf16x8& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_offset, 0, 0);
}


// Reduce-scatter of 32 values over the 32 lanes of each half-wave, in VALU
// lane exchanges only: afterwards lane l holds, for slot l%32, the sum over
// the 32 lanes of its half. Each level pairs every lane with one whose bit
// (16, 8, 4, 2, 1) differs and that shares the bits already processed; the
// lane keeps the half of its slots its own bit selects and adds the partner's
// copy of that half. Level 16 uses v_permlane16_swap (rows 1/3 exchanged with
// rows 0/2); levels 8, 4, 2, 1 use DPP row rotate by 8, row half-mirror
// (lane i <-> 7-i within eight), and quad permutes [2,3,0,1] and [1,0,3,2].
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int M, int CTRL>
__device__ __forceinline__ void rs_level(float* x, int lane) {
  const bool hi = lane & M;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const float mine = hi ? x[j + M] : x[j], other = hi ? x[j] : x[j + M];
    x[j] = mine + dpp_f<CTRL>(other);
  }
}
__device__ __forceinline__ float reduce_scatter32(float (&x)[32], int lane) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j + 16]), false, false);
    x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  rs_level<8, 0x128>(x, lane);  // row_ror:8
  rs_level<4, 0x141>(x, lane);  // row_half_mirror
  rs_level<2, 0x4E>(x, lane);   // quad_perm [2,3,0,1]
  rs_level<1, 0xB1>(x, lane);   // quad_perm [1,0,3,2]
  return x[0];
}

// Offset (elements) of 16-byte granule `g` of row `row` in a 32 x 256 K block
// stored without padding: granules are XOR-swizzled with the row so that 16
// rows read at the same column hit 16 different bank groups.
__device__ __forceinline__ int k_swz(int row, int g) { return row * 256 + ((g ^ (row & 15)) << 3); }

// Position of 16-byte granule `g` of row `row` in an unpadded X tile (V rows or
// chunk-state rows): rows r..r+3 of a transposed read land in four different
// 64-byte bank groups.
__device__ __forceinline__ int x_pos(int row, int g) { return g ^ ((row & 3) << 2); }

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// lds_chunk + 16*l (the chunk address must be the same in every lane); the
// global side is `byte_offset` into the descriptor's range (zeros past it).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint16_t* lds_chunk, int byte_offset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_chunk), 16, byte_offset, 0, 0, 0);
}
// The same with a wave-uniform part of the offset in a scalar register.
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, uint16_t* lds_chunk, int byte_offset,
                                       int uniform_offset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_chunk), 16, byte_offset, uniform_offset, 0, 0);
}

}  // namespace

struct OutArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* chunk_states;  // [B*H][nchunks][dk][dv] or null
  uint16_t* o;
  int state_for_chunk0;
  int H, N, dk, dv, chunk, nchunks, nqb;
  int nblocks;                   // B * H * nqb query blocks
};

// Workgroups of `kernel` (launched with `threads` threads) resident on the
// current device at once: CUs times workgroups per CU, cached per device and
// kernel slot `which` (0 .. kResidentSlots-1).
constexpr int kResidentSlots = 14;
hipError_t resident_workgroups(const void* kernel, int threads, int which, int* out);

}  // namespace ret

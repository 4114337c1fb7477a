// bf16 retention kernels on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulate).
//
// Method ("RetNet - Retentive Network - A Successor to Transformer for LLMs",
// Key Equations: parallel form and chunkwise recurrent form; Key components,
// 1. Retention for the chunk-state carry). For chunk i of length L, local row j:
//   O_[i] = (Q_[i] K_[i]^T (*) D) V_[i] + diag(gamma^(j+1)) Q_[i] R_{i-1}
//   R_i   = gamma^L R_{i-1} + K_[i]^T diag(gamma^(L-1-j)) V_[i]
//
// Two kernels:
//  * state walk: one workgroup per (head, 32*MT-row k-tile, 128-column v-tile,
//    sequence segment) keeps its tile of R in MFMA accumulators (fp32) and
//    walks the chunks in order. Before each chunk it stores R as bf16 ([k][v],
//    v fastest, like V); then it applies the carry and accumulates
//    K^T (zeta V) over 64-row key blocks. Long sequences with few heads are
//    cut into chunk-aligned segments: a first launch computes each segment's
//    end state (segment 0 from state_in, the others from zero), the second
//    starts every segment from the earlier segments' end states, each decayed
//    to its start, and writes the chunk states.
//  * output: one workgroup per (head, 64-row query block) with the full dv
//    row. It reads out the stored chunk state in 64-row slices (O = Q R), scales
//    the rows by gamma^(j+1), then loops over the 64-row key blocks of its chunk
//    up to the diagonal: S^T = K Q^T, the decay gamma^(n-m) (zero above the
//    diagonal) applied to the fp32 scores in registers, scores rounded to bf16
//    through LDS, then O += A V. The per-head GroupNorm and the bf16 store close
//    it. The N x N mask never exists in memory; with one chunk spanning the
//    sequence this is the parallel form.
//
// Data movement: every tile (K, V, state slice) is copied row-major into LDS
// with 16-byte accesses; the next tile's global loads are issued into registers
// before the current tile's matrix work so their latency is hidden. Operands
// that need a transposed view (V and the state as B operands, K^T as the walk's
// A operand) are fetched with ds_read_b64_tr_b16, which hands each lane four
// consecutive rows of one column. Workgroups that share K/V/state tiles get
// consecutive logical indices and are placed on the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs), so the re-reads hit one L2.
//
// MFMA 32x32x16 operand layouts used throughout (lane l of 64):
//   A[i][kk]: i = l % 32, kk = 8*(l/32) + 0..7
//   B[kk][j]: j = l % 32, kk = 8*(l/32) + 0..7
//   D[i][j] : j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4 for accumulator r = 0..15
#include <type_traits>
#include <algorithm>
#include <atomic>
#include <cstdint>

#include "kernels.h"
#include "mfma_tiles.h"

namespace ret {

namespace {

constexpr int kThreads = 256;  // four waves
constexpr int kRows = 64;      // query / key block height

// Register staging of one ROWS-row tile of a row-major bf16 matrix with NTHR
// threads: thread t owns 16-byte pieces t, t+NTHR, ... of a tile COLS wide
// (row = piece / (COLS/8)); COLS is a compile-time width so the piece layout
// costs shifts only. Rows at or past `rows_valid`, and columns at or past
// `cols_valid`, read as zero (buffer range check / out-of-range offset).
template <int MAXP, int NTHR, int COLS, int ROWS = kRows>
struct TileRegs {
  static constexpr int kPerRow = COLS / 8;
  u32x4 p[MAXP];

  __device__ __forceinline__ static int row_of(int m) { return (static_cast<int>(threadIdx.x) + NTHR * m) / kPerRow; }
  __device__ __forceinline__ static int col_of(int m) { return ((static_cast<int>(threadIdx.x) + NTHR * m) % kPerRow) * 8; }

  __device__ __forceinline__ void load(const uint16_t* src, int stride, int rows_valid, int cols_valid) {
    const int nbytes = rows_valid > 0 ? ((rows_valid - 1) * stride + cols_valid) * 2 : 0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, nbytes);
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      const int row = row_of(m), col = col_of(m);
      const int off = (row < ROWS && col < cols_valid) ? (row * stride + col) * 2 : kOutOfRange;
      p[m] = buffer_load16(r, off);
    }
  }

  // Store piece m into LDS [row][col] with the given pitch (elements).
  __device__ __forceinline__ void store_piece(uint16_t* dst, int pitch, int m) const {
    if (row_of(m) < ROWS) *reinterpret_cast<u32x4*>(dst + row_of(m) * pitch + col_of(m)) = p[m];
  }

  // Store into LDS [row][col] with the given pitch (elements).
  __device__ __forceinline__ void store(uint16_t* dst, int pitch) const {
#pragma unroll
    for (int m = 0; m < MAXP; ++m)
      if (row_of(m) < ROWS) *reinterpret_cast<u32x4*>(dst + row_of(m) * pitch + col_of(m)) = p[m];
  }

  // Store with row r multiplied by scale[m] (one factor per owned piece's row).
  __device__ __forceinline__ void store_scaled(uint16_t* dst, int pitch, const float (&scale)[MAXP]) const {
#pragma unroll
    for (int m = 0; m < MAXP; ++m) {
      if (row_of(m) < ROWS) {
        u32x4 v = p[m];
        const float z = scale[m];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = pack_bf16x2(__uint_as_float(v[e] << 16) * z, __uint_as_float(v[e] & 0xffff0000u) * z);
        *reinterpret_cast<u32x4*>(dst + row_of(m) * pitch + col_of(m)) = v;
      }
    }
  }
};


// ---------------------------------------------------------------------------
// State walk
// ---------------------------------------------------------------------------
constexpr int kWalkVT = 128;   // v columns per workgroup: 32 per wave
constexpr int kWalkPitch = 160;  // LDS pitch of the K and V tiles (320 B: rows 64 B apart mod 256)

struct WalkArgs {
  const uint16_t* k;
  const uint16_t* v;
  const float* state_in;
  float* state_out;
  uint16_t* chunk_states;  // [B*H][nchunks][dk][dv]
  float* seg_states;       // [B*H][nseg][dk][dv]
  int H, N, dk, dv, chunk, nchunks, nseg, chunks_per_seg;
  int nkt, nvt;
  // 0: end state of segments 0..nseg-2; 1: write chunk states from the true
  // start; 2: every segment from zero (segment 0 from state_in), chunk states
  // and end states written (walk_fixup_kernel then makes them true).
  int mode;
};

template <int MT>
__global__ void __launch_bounds__(kThreads) mfma_state_walk_kernel(WalkArgs a, HeadDecay decay) {
  constexpr int KT = 32 * MT;
  constexpr int PIECES = (kRows * KT / 8 + kThreads - 1) / kThreads;
  constexpr int VPIECES = kRows * kWalkVT / 8 / kThreads;
  constexpr int kPitchWK = KT <= 128 ? kWalkPitch : KT + 32;  // K tile pitch: rows 64 B apart mod 256
  __shared__ __attribute__((aligned(16))) uint16_t sK[kRows * kPitchWK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kRows * kWalkPitch];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nseg_launch = (a.mode == 0) ? a.nseg - 1 : a.nseg;
  const int nblocks = gridDim.x;
  int idx = xcd_logical_block(blockIdx.x, nblocks);
  const int vt = idx % a.nvt;
  idx /= a.nvt;
  const int kt = idx % a.nkt;
  idx /= a.nkt;
  const int seg = idx % nseg_launch;
  const int64_t bh = idx / nseg_launch;
  const int h = static_cast<int>(bh % a.H);
  const float lg = decay.log2g[h];
  const int k0 = kt * KT, v0 = vt * kWalkVT;
  const int c_begin = seg * a.chunks_per_seg;
  const int c_end = min(a.nchunks, c_begin + a.chunks_per_seg);
  const int64_t dkdv = static_cast<int64_t>(a.dk) * a.dv;

  floatx16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx16{};

  const int vcol = v0 + wave * 32 + (lane & 31);  // this lane's state column
  if (seg == 0 && a.state_in) {
    // Segment 0 starts from state_in (in both modes, so U_0 carries its decayed share).
    const float* S0 = a.state_in + bh * dkdv;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = S0[static_cast<int64_t>(k0 + mt * 32 + acc_row(r, lane)) * a.dv + vcol];
  } else if (a.mode == 1) {
    // True state at a later segment's start p: sum over earlier segments s' of
    // gamma^(p - end_s') U_s', where U_0 already includes state_in.
    const int p = c_begin * a.chunk;
    for (int s = 0; s < seg; ++s) {
      const int end_s = (s + 1) * a.chunks_per_seg * a.chunk;
      const float f = gpow(lg, static_cast<float>(p - end_s));
      const float* U = a.seg_states + (bh * a.nseg + s) * dkdv;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[mt][r] = fmaf(f, U[static_cast<int64_t>(k0 + mt * 32 + acc_row(r, lane)) * a.dv + vcol], acc[mt][r]);
    }
  }

  // The state came in through loads straight into the accumulators; finish
  // them here so no later MFMA has to wait on the vector-memory counter for
  // them (the compiler cannot tell that the first tile's wait covers them).
  wait_vmem();

  const uint16_t* kb = a.k + bh * static_cast<int64_t>(a.N) * a.dk + k0;
  const uint16_t* vb = a.v + bh * static_cast<int64_t>(a.N) * a.dv + v0;

  // Tiles are (chunk, 64-row block) pairs in sequence order.
  TileRegs<PIECES, kThreads, KT> rk;
  TileRegs<VPIECES, kThreads, kWalkVT> rv;
  // zeta_t = gamma^(L-1-t) = gamma^(L-1-t0) * gamma^(-r) for row r of a tile at t0;
  // it scales whichever of the K and V tiles is smaller. The gamma^(-r) factors
  // of this thread's rows are fixed (r <= 63, so <= 7.4).
  constexpr bool kScaleK = KT < kWalkVT;
  constexpr int ZP = kScaleK ? PIECES : VPIECES;
  float zrow[ZP];
#pragma unroll
  for (int m = 0; m < ZP; ++m) {
    const int row = kScaleK ? TileRegs<PIECES, kThreads, KT>::row_of(m) : TileRegs<VPIECES, kThreads, kWalkVT>::row_of(m);
    zrow[m] = gpow(lg, -static_cast<float>(row));
  }
  int c = c_begin, t0 = 0;
  if (c < c_end) {
    const int L = min(a.chunk, a.N - c * a.chunk);
    rk.load(kb + static_cast<int64_t>(c * a.chunk) * a.dk, a.dk, min(kRows, L), KT);
    rv.load(vb + static_cast<int64_t>(c * a.chunk) * a.dv, a.dv, min(kRows, L), kWalkVT);
  }
  while (c < c_end) {
    const int cs = c * a.chunk;
    const int L = min(a.chunk, a.N - cs);
    if (t0 == 0) {
      if (a.mode >= 1) {
        // Store R_{c-1} as bf16, [k][v] layout; 32 lanes cover 64 contiguous bytes of a row.
        uint16_t* dst = a.chunk_states + ((bh * a.nchunks + c) * a.dk + k0) * static_cast<int64_t>(a.dv) + vcol;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dst[static_cast<int64_t>(mt * 32 + acc_row(r, lane)) * a.dv] = f32_to_bf16(acc[mt][r]);
      }
      const float carry = gpow(lg, static_cast<float>(L));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= carry;
    }
    __syncthreads();
    {
      const float z0 = gpow(lg, static_cast<float>(L - 1 - t0));
      float z[ZP];
#pragma unroll
      for (int m = 0; m < ZP; ++m) z[m] = z0 * zrow[m];
      if constexpr (kScaleK) {
        rk.store_scaled(sK, kPitchWK, z);
        rv.store(sV, kWalkPitch);
      } else {
        rk.store(sK, kPitchWK);
        rv.store_scaled(sV, kWalkPitch, z);
      }
    }
    __syncthreads();

    // Advance and prefetch the next tile while this one is multiplied.
    int nc = c, nt0 = t0 + kRows;
    if (nt0 >= L) {
      nc = c + 1;
      nt0 = 0;
    }
    if (nc < c_end) {
      const int ncs = nc * a.chunk;
      const int nL = min(a.chunk, a.N - ncs);
      const int nvalid = min(kRows, nL - nt0);
      rk.load(kb + static_cast<int64_t>(ncs + nt0) * a.dk, a.dk, nvalid, KT);
      rv.load(vb + static_cast<int64_t>(ncs + nt0) * a.dv, a.dv, nvalid, kWalkVT);
    }

#pragma unroll
    for (int s = 0; s < kRows / 16; ++s) {
      const bf16x8 b = ld_tr8(sV, kWalkPitch, s * 16, wave * 32, lane);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 av = ld_tr8(sK, kPitchWK, s * 16, mt * 32, lane);
        acc[mt] = mfma32(av, b, acc[mt]);
      }
    }
    c = nc;
    t0 = nt0;
  }

  // Modes 0 and 2 store the segment's end state. Mode 1 stores the final
  // state: to state_out when there is one segment, else into the spare last
  // segment slot (the host copies it to state_out afterwards, so state_out may
  // alias state_in while other segments still read it).
  float* out = nullptr;
  if (a.mode != 1) out = a.seg_states + (bh * a.nseg + seg) * dkdv;
  else if (seg == a.nseg - 1) {
    if (a.nseg > 1) out = a.seg_states + (bh * a.nseg + seg) * dkdv;
    else if (a.state_out) out = a.state_out + bh * dkdv;
  }
  if (out) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        out[static_cast<int64_t>(k0 + mt * 32 + acc_row(r, lane)) * a.dv + vcol] = acc[mt][r];
  }
}

// ---------------------------------------------------------------------------
// State walk, full-dk form (dk = 128 or 256)
// ---------------------------------------------------------------------------
// One workgroup of eight waves per (head, 64*NTW-column v tile, segment) owns
// the whole dk x 64*NTW slab of R: wave (kw, vw) keeps rows 32*MTW*kw.. and
// columns 32*NTW*vw.. (MTW x NTW accumulator tiles), so each V row is read once
// and each K row once per v tile. 64-key blocks are double-buffered in LDS
// (register staging, zeta applied to V rows on the way), one barrier per block.
// The V tile is unpadded with its 16-byte granules XOR-swizzled by the row, so
// the transposed operand reads of four consecutive rows hit four bank groups.
constexpr int kWalk2Threads = 512;
constexpr int kWalk2VT = 128;      // v columns per workgroup at NTW = 2
constexpr int kWalk2PP = 36;       // store patch pitch: 72 B, 32 rows start on distinct bank pairs


template <int MTW, int NTW>
__global__ void __launch_bounds__(kWalk2Threads) mfma_state_walk2_kernel(WalkArgs a, HeadDecay decay) {
  constexpr int NT = kWalk2Threads;
  constexpr int DK = 128 * MTW;
  constexpr int PK = DK + 32;                  // sK pitch: rows 64 B apart mod 256
  constexpr int KP = kRows * DK / 8 / NT;      // 16-byte pieces per thread of a K block
  constexpr int VT = 64 * NTW;                 // v columns per workgroup
  constexpr int VGPR = VT / 8;                 // 16-byte granules per V row
  constexpr int VP = kRows * VT / 8 / NT;      // ... of a V block
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kRows * PK];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kRows * VT];
  __shared__ __attribute__((aligned(16))) uint16_t sPatch[8][32 * kWalk2PP];  // per-wave store patch

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = wave & 3, vw = wave >> 2;
  const int nseg_launch = (a.mode == 0) ? a.nseg - 1 : a.nseg;
  int idx = xcd_logical_block(blockIdx.x, gridDim.x);
  const int vt = idx % a.nvt;
  idx /= a.nvt;
  const int seg = idx % nseg_launch;
  const int64_t bh = idx / nseg_launch;
  const int h = static_cast<int>(bh % a.H);
  const float lg = decay.log2g[h];
  const int v0 = vt * VT;
  const int krow0 = kw * 32 * MTW;                 // this wave's first state row
  const int vcol = v0 + vw * 32 * NTW + (lane & 31);  // state column of accumulator tile 0
  const int c_begin = seg * a.chunks_per_seg;
  const int c_end = min(a.nchunks, c_begin + a.chunks_per_seg);
  const int64_t dkdv = static_cast<int64_t>(DK) * a.dv;

  floatx16 acc[MTW][NTW];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = floatx16{};

  auto state_at = [&](const float* S, int mt, int nt, int r) -> float {
    return S[static_cast<int64_t>(krow0 + mt * 32 + acc_row(r, lane)) * a.dv + vcol + 32 * nt];
  };
  if (seg == 0 && a.state_in) {
    // Segment 0 starts from state_in (in both modes, so U_0 carries its decayed share).
    const float* S0 = a.state_in + bh * dkdv;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][nt][r] = state_at(S0, mt, nt, r);
  } else if (a.mode == 1) {
    // True state at a later segment's start p: sum over earlier segments s' of
    // gamma^(p - end_s') U_s', where U_0 already includes state_in.
    const int p = c_begin * a.chunk;
    for (int s = 0; s < seg; ++s) {
      const int end_s = (s + 1) * a.chunks_per_seg * a.chunk;
      const float f = gpow(lg, static_cast<float>(p - end_s));
      const float* U = a.seg_states + (bh * a.nseg + s) * dkdv;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mt][nt][r] = fmaf(f, state_at(U, mt, nt, r), acc[mt][nt][r]);
    }
  }

  // The state came in through loads straight into the accumulators; finish
  // them here so no later MFMA has to wait on the vector-memory counter for
  // them (the compiler cannot tell that the first block's wait covers them).
  wait_vmem();

  const uint16_t* kb = a.k + bh * static_cast<int64_t>(a.N) * DK;
  const uint16_t* vb = a.v + bh * static_cast<int64_t>(a.N) * a.dv + v0;
  TileRegs<KP, NT, DK> rk;
  TileRegs<VP, NT, VT> rv;
  // zeta_t = gamma^(L-1-t) = gamma^(L-1-t0) * gamma^(-r) for row r of a block
  // at t0; the gamma^(-r) factors of this thread's V rows are fixed.
  float zrow[VP];
#pragma unroll
  for (int m = 0; m < VP; ++m) zrow[m] = gpow(lg, -static_cast<float>(TileRegs<VP, NT, VT>::row_of(m)));
  // LDS positions of this thread's V pieces in the swizzled tile, and the
  // per-lane parts of the transposed V operand reads (rows 8*(lane/32) +
  // (lane%16)/4 of columns 32*NTW*vw + 32nt + 16*((lane/16)%2) + 4*(lane%4)..;
  // a step of 16 rows or 4 rows keeps the swizzle).
  int vput[VP];
#pragma unroll
  for (int m = 0; m < VP; ++m) {
    const int row = TileRegs<VP, NT, VT>::row_of(m), g = TileRegs<VP, NT, VT>::col_of(m) / 8;
    vput[m] = row * VT + (x_pos(row, g) << 3);
  }
  int vread[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int g = lane >> 4, j = lane & 15;
    const int row = 8 * (g >> 1) + (j >> 2);
    const int col = vw * 32 * NTW + 32 * nt + 16 * (g & 1) + 4 * (j & 3);
    vread[nt] = row * VT + (x_pos(row, col >> 3) << 3) + (col & 7);
  }

  // Blocks are (chunk, 64-row block) pairs in sequence order; `load` fetches
  // block (c, t0) into registers, `put` stores it scaled into LDS buffer b.
  auto load = [&](int c, int t0) {
    const int cs = c * a.chunk;
    const int L = min(a.chunk, a.N - cs);
    const int nvalid = min(kRows, L - t0);
    rk.load(kb + static_cast<int64_t>(cs + t0) * DK, DK, nvalid, DK);
    rv.load(vb + static_cast<int64_t>(cs + t0) * a.dv, a.dv, nvalid, VT);
  };
  auto put = [&](int c, int t0, int b) {
    const int L = min(a.chunk, a.N - c * a.chunk);
    const float z0 = gpow(lg, static_cast<float>(L - 1 - t0));
    float z[VP];
#pragma unroll
    for (int m = 0; m < VP; ++m) z[m] = z0 * zrow[m];
    rk.store(sK[b], PK);
    // V rows scaled by zeta into their swizzled places.
#pragma unroll
    for (int m = 0; m < VP; ++m) {
      u32x4 w = rv.p[m];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16x2(__uint_as_float(w[e] << 16) * z[m], __uint_as_float(w[e] & 0xffff0000u) * z[m]);
      *reinterpret_cast<u32x4*>(sV[b] + vput[m]) = w;
    }
  };
  auto advance = [&](int& c, int& t0) {
    t0 += kRows;
    if (t0 >= min(a.chunk, a.N - c * a.chunk)) {
      ++c;
      t0 = 0;
    }
  };

  int c = c_begin, t0 = 0;       // block being multiplied
  int nc = c, nt0 = t0;          // block in the registers
  if (c < c_end) {
    load(c, t0);
    put(c, t0, 0);
    advance(nc, nt0);
    if (nc < c_end) load(nc, nt0);
  }
  __syncthreads();
  int buf = 0;
  while (c < c_end) {
    if (t0 == 0) {
      const int L = min(a.chunk, a.N - c * a.chunk);
      if (a.mode >= 1) {
        // Store R_{c-1} as bf16 ([k][v], v fastest). Each 32x32 accumulator tile
        // goes through this wave's LDS patch, stored transposed (a lane's four
        // consecutive rows of one column in one 8-byte write), and comes back
        // with the transposed LDS read as eight consecutive v columns of one k
        // row per lane: two 16-byte stores per lane and tile.
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(a.chunk_states + (bh * a.nchunks + c) * dkdv, static_cast<int>(dkdv * 2));
        uint16_t* patch = sPatch[wave];
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              uint2 w;
              w.x = pack_bf16x2(acc[mt][nt][4 * g], acc[mt][nt][4 * g + 1]);
              w.y = pack_bf16x2(acc[mt][nt][4 * g + 2], acc[mt][nt][4 * g + 3]);
              *reinterpret_cast<uint2*>(patch + (lane & 31) * kWalk2PP + 8 * g + 4 * (lane >> 5)) = w;
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const bf16x8 v8 = ld_tr8(patch, kWalk2PP, 16 * half, 0, lane);
              const int row = krow0 + mt * 32 + (lane & 31);
              const int col = v0 + vw * 32 * NTW + nt * 32 + 16 * half + 8 * (lane >> 5);
              buffer_store16(rs, (row * a.dv + col) * 2, v8);
            }
          }
      }
      const float carry = gpow(lg, static_cast<float>(L));
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] *= carry;
    }
    // U += K^T (zeta V) over the block's 64 keys.
    auto multiply = [&]() {
      const uint16_t* kt = sK[buf];
      const uint16_t* vt_ = sV[buf];
#pragma unroll
      for (int s = 0; s < kRows / 16; ++s) {
        bf16x8 bv[NTW], av[MTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vt_ + vread[nt] + s * 16 * VT));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vt_ + vread[nt] + (s * 16 + 4) * VT));
          bv[nt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) av[mt] = ld_tr8(kt, PK, s * 16, krow0 + mt * 32, lane);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = mfma32(av[mt], bv[nt], acc[mt][nt]);
      }
    };
    // The next block goes into the other buffer (read one block ago), the
    // one after into the registers.
    auto stage = [&]() {
      if (nc < c_end) {
        put(nc, nt0, buf ^ 1);
        int fc = nc, ft0 = nt0;
        advance(fc, ft0);
        if (fc < c_end) load(fc, ft0);
      }
    };
    // The two waves on each SIMD take the two halves in opposite order, so
    // one's matrix work overlaps the other's staging.
    if (wave < 4) {
      multiply();
      stage();
    } else {
      stage();
      multiply();
    }
    __syncthreads();
    c = nc;
    t0 = nt0;
    advance(nc, nt0);
    buf ^= 1;
  }

  // Modes 0 and 2 store the segment's end state. Mode 1 stores the final
  // state: to state_out when there is one segment, else into the spare last
  // segment slot (the host copies it to state_out afterwards, so state_out may
  // alias state_in while other segments still read it).
  float* out = nullptr;
  if (a.mode != 1) out = a.seg_states + (bh * a.nseg + seg) * dkdv;
  else if (seg == a.nseg - 1) {
    if (a.nseg > 1) out = a.seg_states + (bh * a.nseg + seg) * dkdv;
    else if (a.state_out) out = a.state_out + bh * dkdv;
  }
  if (out) {
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          out[static_cast<int64_t>(krow0 + mt * 32 + acc_row(r, lane)) * a.dv + vcol + 32 * nt] = acc[mt][nt][r];
  }
}

// ---------------------------------------------------------------------------
// Segment fix-up after a mode-2 walk
// ---------------------------------------------------------------------------
// Segment 0 was walked from the true start, the others from zero. The true
// state at the start of segment s >= 1 is S_s = gamma^len_{s-1} S_{s-1} +
// U_{s-1} with S_1 = U_0 (U = the stored end states), and the true state
// before chunk c of segment s is the stored one plus gamma^(chunk (c - c_s))
// S_s: only full chunks precede a stored state. One thread per head and eight
// consecutive state elements walks the segments in order, rewrites the bf16
// chunk states of segments 1.. in place and writes the final state.
constexpr int kFixThreads = 256;

struct FixArgs {
  uint16_t* chunk_states;  // [B*H][nchunks][dk][dv]
  const float* seg_states; // [B*H][nseg][dk][dv]
  float* state_out;        // [B*H][dk][dv] or null
  int64_t heads;
  int H, N, chunk, nchunks, nseg, chunks_per_seg, dkdv;
};

__global__ void __launch_bounds__(kFixThreads) walk_fixup_kernel(FixArgs a, HeadDecay decay) {
  const int per_head = a.dkdv / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kFixThreads + threadIdx.x;
  if (idx >= a.heads * per_head) return;
  const int64_t bh = idx / per_head;
  const int e0 = static_cast<int>(idx % per_head) * 8;
  const float lg = decay.log2g[bh % a.H];
  const float* U = a.seg_states + bh * a.nseg * static_cast<int64_t>(a.dkdv) + e0;
  float S[8];
  {
    const floatx4 lo = *reinterpret_cast<const floatx4*>(U);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(U + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S[e] = lo[e];
      S[e + 4] = hi[e];
    }
  }
  for (int s = 1; s < a.nseg; ++s) {
    const int c_s = s * a.chunks_per_seg;
    const int c_e = min(a.nchunks, c_s + a.chunks_per_seg);
    for (int c = c_s; c < c_e; ++c) {
      const float f = gpow(lg, static_cast<float>((c - c_s) * a.chunk));
      u32x4* p = reinterpret_cast<u32x4*>(a.chunk_states + (bh * a.nchunks + c) * static_cast<int64_t>(a.dkdv) + e0);
      u32x4 v = *p;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = pack_bf16x2(fmaf(f, S[2 * e], __uint_as_float(v[e] << 16)),
                           fmaf(f, S[2 * e + 1], __uint_as_float(v[e] & 0xffff0000u)));
      *p = v;
    }
    const float g = gpow(lg, static_cast<float>(min(a.N, c_e * a.chunk) - c_s * a.chunk));
    const float* Us = U + static_cast<int64_t>(s) * a.dkdv;
    const floatx4 lo = *reinterpret_cast<const floatx4*>(Us);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(Us + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      S[e] = fmaf(g, S[e], lo[e]);
      S[e + 4] = fmaf(g, S[e + 4], hi[e]);
    }
  }
  if (a.state_out) {
    float* o = a.state_out + bh * static_cast<int64_t>(a.dkdv) + e0;
    *reinterpret_cast<floatx4*>(o) = floatx4{S[0], S[1], S[2], S[3]};
    *reinterpret_cast<floatx4*>(o + 4) = floatx4{S[4], S[5], S[6], S[7]};
  }
}

// ---------------------------------------------------------------------------
// Output
// ---------------------------------------------------------------------------
constexpr int kTile = 32;      // rows of a staged tile: 32 keys of V, or 32 rows of the chunk state

// Buffer set P of three (P is a compile-time step phase).
template <int P>
__device__ __forceinline__ uint16_t* pick3(uint16_t* b0, uint16_t* b1, uint16_t* b2) {
  return P == 0 ? b0 : (P == 1 ? b1 : b2);
}

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// One workgroup per CU, looping over 64-row query blocks (head, rows q0..q0+63);
// wave w owns value columns [32*NVT*w, 32*NVT*(w+1)) of all 64 rows (2 x NVT
// accumulator tiles).
//
// Block order: the blocks are split into one contiguous range per XCD (so the
// query blocks of a chunk, which read the same K, V and state, meet in one
// L2), and the workgroups of an XCD take the range in groups of their count,
// each workgroup one block per group. The work per block grows along the
// chunk, so the assignment within a group moves between groups: rotated by one
// place per group when there are several chunks (every workgroup sweeps the
// positions of a chunk), reversed on every other group when one chunk spans
// the sequence (the parallel form: a workgroup that drew a late, long block
// next draws an early, short one).
//
// A block's work is a sequence of steps, each multiplying a 32-row bf16 tile
// X in LDS into O as O += A X: first the dk/32 slices of the stored chunk
// state (A = the matching 32 columns of Q, the cross-chunk read-out), then the
// 32-key blocks of the chunk up to the diagonal (A = the decayed scores of that
// block, X = its V rows).
//
// Scores of a key block, S^T = K Q^T (32 keys x 64 queries), are formed one
// step ahead: wave (tt, qt) computes the 16 x 16 tile of keys 16*tt.. and
// queries 16*qt.. on 16x16x32 MFMAs, K from LDS, its 16 query rows held in
// registers for the whole block; it applies gamma^(n-m) (zero above the
// diagonal) and writes the bf16 scores to the score buffer of the next step. A
// state step's A operand, the 64 x 32 Q slice, is copied into the score buffer
// of its step in the same layout, so both kinds of step read A alike, and the
// waves take their score tiles' query rows from those slices as they pass (a
// block without state slices loads them once instead).
//
// Tiles travel straight from global memory into LDS (buffer loads with an LDS
// destination) two steps ahead, in three buffer sets (X tile + K block, and a
// score buffer): the copies of step i+2 go into the set step i-1 read, and step
// i ends by waiting for all but its own copies, then one barrier. The sets are
// distinct LDS arrays chosen at compile time per step phase (i mod 3), so the
// LDS reads of a step never wait for the copies in flight. The next block's
// first copies and Q rows are requested before the current block's GroupNorm
// and store, which use no buffer those copies write.
template <int NVT, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) mfma_chunk_out_kernel(OutArgs a, HeadDecay decay, GnArgs gn) {
  constexpr int DV = WAVES * 32 * NVT;
  constexpr int SW = 8 / WAVES;                    // 16 x 16 score tiles per wave (8 per key block)
  constexpr int XCH = kTile * DV * 2 / 1024;       // 1-KiB chunks of an X tile
  constexpr int KCH = kTile * 256 * 2 / 1024;      // ... of a K block (dk <= 256)
  constexpr int XI = XCH / WAVES, KI = KCH / WAVES;  // chunks copied per wave
  constexpr int GPR = DV / 8;                      // 16-byte granules per X row
  constexpr int PT = kRows * kTile;                // elements of a score tile
  constexpr int QCH = PT * 2 / 1024;               // 1-KiB chunks of a Q slice (16 rows each)
  constexpr int XK = kTile * DV + kTile * 256;     // elements of one X + K buffer
  constexpr int OSTORES = 2 * NVT * 8;             // 4-byte O stores per lane and block
  static_assert(XI >= 1 && KI >= 1 && XCH % WAVES == 0 && KCH % WAVES == 0 && QCH <= WAVES, "layout");
  static_assert((WAVES * 64 / GPR) % 4 == 0, "X copy offsets");
  static_assert(XI + KI + 1 <= 7, "copies per step");
  static_assert(OSTORES <= 48, "O stores must fit the vector-memory counter");
  // X tile at 0 and K block at kTile*DV of each buffer set (copied at the same step).
  __shared__ __attribute__((aligned(1024))) uint16_t sXK0[XK];
  __shared__ __attribute__((aligned(1024))) uint16_t sXK1[XK];
  __shared__ __attribute__((aligned(1024))) uint16_t sXK2[XK];
  // Scores (or a Q slice), row-major with 64-byte rows of four 16-byte
  // granules, granule g of row r at slot g ^ ((r / 4) % 4) (p_off below), so the
  // 16-byte operand reads of 16 consecutive rows hit 16 different bank groups.
  __shared__ __attribute__((aligned(1024))) uint16_t sP0[PT];
  __shared__ __attribute__((aligned(1024))) uint16_t sP1[PT];
  __shared__ __attribute__((aligned(1024))) uint16_t sP2[PT];
  static_assert(sizeof(sP2) >= (WAVES + 2) * kRows * sizeof(float), "GroupNorm statistics reuse sP2");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: copy targets in scalars
  const int l32 = lane & 31;
  const int l16 = lane & 15;
  const int vcol0 = wave * 32 * NVT;
  const int dk = a.dk;

  // Transposed X operands (B of the output product, the contraction index
  // down the tile's rows), two ds_read_b64_tr_b16 each as in ld_tr8, from the
  // unpadded swizzled X tile: lane l points at row 16s + 8*(l/32) + (l%16)/4
  // (and that row + 4, same swizzle) and columns vcol0 + 32nt +
  // 16*((l/16)%2) + 4*(l%4).., at xo[nt] + 16s*DV (+ 4*DV). The empty asm keeps
  // each read's address one constant offset away from its buffer, so every
  // read keeps the buffer's alias information and never waits for copies into
  // the other buffers.
  int xo[NVT];
#pragma unroll
  for (int nt = 0; nt < NVT; ++nt) {
    const int g = lane >> 4, j = lane & 15;
    const int row = 8 * (g >> 1) + (j >> 2);
    const int col = vcol0 + 32 * nt + 16 * (g & 1) + 4 * (j & 3);
    xo[nt] = row * DV + (x_pos(row, col >> 3) << 3) + (col & 7);
    asm volatile("" : "+v"(xo[nt]));
  }
  auto ld_x = [&](const uint16_t* tile, int s, int nt) __attribute__((always_inline)) {
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(tile + xo[nt] + 16 * s * DV));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(tile + xo[nt] + (16 * s + 4) * DV));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Per-lane source offsets of the copies, fixed for the kernel. X tile: lane
  // l of 1-KiB piece c = wave + WAVES*m holds granule 64c + l of the swizzled
  // tile; the row advances by a multiple of four per m, so the swizzle
  // (row % 4) is that of m = 0 and piece m lies m*WAVES KiB further.
  int xoff;
  {
    const int flat = wave * 64 + lane;
    const int row = flat / GPR, pos = flat % GPR;
    xoff = (row * GPR + x_pos(row, pos)) * 16;
  }
  // K block: piece c holds rows 2c and 2c+1, granules swizzled with the row (zero past dk).
  int koff[KI];
#pragma unroll
  for (int m = 0; m < KI; ++m) {
    const int row = 2 * (wave + WAVES * m) + (lane >> 5), pos = lane & 31;
    const int g = pos ^ (row & 15);
    koff[m] = g * 8 < dk ? (row * dk + g * 8) * 2 : kOutOfRange;
  }
  // Score-buffer element offset of granule g (8 columns) of row r.
  auto p_off = [](int r, int g) __attribute__((always_inline)) { return r * kTile + ((g ^ ((r >> 2) & 3)) << 3); };
  // Q slice: piece w (one per wave below QCH) holds rows 16w..16w+15, lane l
  // slot l%4 of row 16w + l/4, so each lane reads 16 of the row's 64
  // contiguous bytes (the granule that lands in that slot).
  int qsoff;
  {
    const int row = wave * 16 + (lane >> 2), slot = lane & 3;
    qsoff = (row * dk + 8 * (slot ^ ((row >> 2) & 3))) * 2;
  }
  // Per-lane score-buffer offsets (elements), fixed for the kernel and kept
  // opaque (see xo): the A operand of step half s and query tile qt (rows
  // qt*32 + lane%32, granule 2s + lane/32), and the Q rows of score tile j
  // (rows ((wave + WAVES*j) % 4)*16 + lane%16, granule lane/16).
  int pa[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      pa[s2][qt] = p_off(qt * 32 + l32, 2 * s2 + (lane >> 5));
      asm volatile("" : "+v"(pa[s2][qt]));
    }
  int pq[SW];
#pragma unroll
  for (int j = 0; j < SW; ++j) {
    pq[j] = p_off(((wave + WAVES * j) & 3) * 16 + l16, lane >> 4);
    asm volatile("" : "+v"(pq[j]));
  }
  // Score tile rows of Q: row (u % 4)*16 + lane%16 of tile u = wave + WAVES*j,
  // from granule lane/16 on.
  int qfoff[SW];
#pragma unroll
  for (int j = 0; j < SW; ++j) qfoff[j] = (((wave + WAVES * j) & 3) * 16 + l16) * dk * 2 + 16 * (lane >> 4);
  // K reads of score tile j: granule 4s + lane/16 of row 16*tt + lane%16. For
  // s and s+4 the swizzled granules differ by 16 (the row's XOR touches
  // granule bits 0-3 only), so four per-lane offsets serve all eight reads.
  int kread[SW][4];
#pragma unroll
  for (int j = 0; j < SW; ++j)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kread[j][s] = k_swz(((wave + WAVES * j) >> 2) * 16 + l16, 4 * s + (lane >> 4));
      asm volatile("" : "+v"(kread[j][s]));
    }

  const int nx = min(kXcds, static_cast<int>(gridDim.x));
  const int xcd = blockIdx.x % nx, slot = blockIdx.x / nx;
  const int nwg = (static_cast<int>(gridDim.x) - xcd + nx - 1) / nx;
  const int per = (a.nblocks + nx - 1) / nx;
  const int lo = min(a.nblocks, xcd * per), hi = min(a.nblocks, lo + per);
  auto block_of = [&](int it) __attribute__((always_inline)) {
    const int pos = a.nchunks > 1 ? (slot + it) % nwg : ((it & 1) ? nwg - 1 - slot : slot);
    const int L = lo + it * nwg + pos;
    return L < hi ? L : -1;
  };

  struct Blk {
    int64_t bh;
    int h, q0, cs, qvalid, nkb, ns, ntiles;
    float lg;
    const uint16_t *kbase, *vbase, *rbase, *qbase;
  };
  auto setup = [&](int L, Blk& b) __attribute__((always_inline)) {
    b.bh = L / a.nqb;
    const int qb = L % a.nqb;
    b.h = static_cast<int>(b.bh % a.H);
    b.lg = decay.log2g[b.h];
    b.q0 = qb * kRows;
    const int c = b.q0 / a.chunk;
    b.cs = c * a.chunk;
    b.qvalid = min(kRows, a.N - b.q0);
    const int kend = min(b.q0 + kRows, a.N);
    b.nkb = (kend - b.cs + kTile - 1) / kTile;  // 32-key blocks of the chunk up to the diagonal
    const bool has_state = a.chunk_states && (c > 0 || a.state_for_chunk0);
    b.ns = has_state ? dk / kTile : 0;          // state slices (dk is a multiple of 32)
    b.ntiles = b.ns + b.nkb;
    b.kbase = a.k + b.bh * static_cast<int64_t>(a.N) * dk;
    b.vbase = a.v + b.bh * static_cast<int64_t>(a.N) * DV;
    b.rbase = has_state ? a.chunk_states + (b.bh * a.nchunks + c) * static_cast<int64_t>(dk) * DV : nullptr;
    b.qbase = a.q + (b.bh * a.N + b.q0) * static_cast<int64_t>(dk);
  };

  // X tile `it` of block b (it < ntiles) into buffer set `dst`.
  auto copy_x = [&](const Blk& b, int it, uint16_t* dst) __attribute__((always_inline)) {
    const uint16_t* src;
    int rows;
    if (it < b.ns) {
      src = b.rbase + static_cast<int64_t>(it * kTile) * DV;
      rows = kTile;
    } else {
      const int t0 = b.cs + (it - b.ns) * kTile;
      src = b.vbase + static_cast<int64_t>(t0) * DV;
      rows = min(kTile, a.N - t0);
    }
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, rows * DV * 2);
#pragma unroll
    for (int m = 0; m < XI; ++m) dma16s(r, dst + (wave + WAVES * m) * 512, xoff, m * WAVES * 1024);
  };
  // K block kb of block b (0 <= kb < nkb) into buffer set `dst`.
  auto copy_k = [&](const Blk& b, int kb, uint16_t* dst) __attribute__((always_inline)) {
    const int t0 = b.cs + kb * kTile;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(b.kbase + static_cast<int64_t>(t0) * dk, min(kTile, a.N - t0) * dk * 2);
#pragma unroll
    for (int m = 0; m < KI; ++m) dma16(r, dst + kTile * DV + (wave + WAVES * m) * 512, koff[m]);
  };
  // Columns 32s..32s+31 of the block's Q rows (zero past N) into score buffer
  // `dst`; waves below QCH copy 16 rows each.
  auto copy_qs = [&](const Blk& b, int s, uint16_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(b.qbase, b.qvalid * dk * 2);
    dma16s(r, dst + wave * 512, qsoff, s * kTile * 2);
  };
  // The 16 query rows of each of this wave's score tiles as 16x16x32 B
  // operands (zero past N and past dk): step s holds Q columns 32s.. . A block
  // with state slices takes them from the slices as they pass through LDS
  // (each Q element then leaves HBM once); a block without loads them here.
  bf16x8 qf[SW][8];
  auto load_qf = [&](const Blk& b) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(b.qbase, b.qvalid * dk * 2);
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      // Granule 4s + lane/16 of the row; step s lies past dk for every lane
      // or for none (dk is a multiple of 32), so that test is uniform.
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qf[j][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, qfoff[j], s * 32 < dk ? s * 64 : kOutOfRange, 0));
    }
  };
  // Everything the first two steps of block b need. Step j reads X_j, its A
  // operand (Q slice or scores) and the K block of its scores (key block
  // j+1-ns) from buffer sets j % 3; with no state slice the block starts at
  // step -1 (set 2), which only forms the scores of key block 0.
  auto first_copies = [&](const Blk& b) __attribute__((always_inline)) {
    if (b.ns > 0) {
#pragma unroll
      for (int j = 0; j < SW; ++j)
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[j][s] = bf16x8{};
      copy_x(b, 0, sXK0);
      copy_x(b, 1, sXK1);  // ntiles > ns
      if (wave < QCH) {
        copy_qs(b, 0, sP0);
        if (b.ns > 1) copy_qs(b, 1, sP1);
      }
      if (b.ns <= 2) copy_k(b, 0, b.ns == 2 ? sXK1 : sXK0);
      if (b.ns == 1 && b.nkb > 1) copy_k(b, 1, sXK1);
    } else {
      load_qf(b);
      copy_k(b, 0, sXK2);
      copy_x(b, 0, sXK0);
      if (b.nkb > 1) copy_k(b, 1, sXK0);
    }
  };

  int it = 0;
  int L = block_of(0);
  if (L < 0) return;  // no block for this workgroup (uniform)
  Blk cur;
  setup(L, cur);
  first_copies(cur);
  wait_vmem();
  __syncthreads();

  for (;;) {
    floatx16 acc[2][NVT];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) acc[qt][nt] = floatx16{};

    const int ns = cur.ns, ntiles = cur.ntiles, nkb = cur.nkb;

    // Decay of score (query q, key t): gamma^(q - t) = gamma^(q0 - t0) *
    // gamma^(ql - tl - r), the first factor uniform per key block, the second
    // fixed per lane for the whole block (q = q0 + ql, t = t0 + tl + r below).
    float flane[SW][4];
#pragma unroll
    for (int j = 0; j < SW; ++j) {
      const int u = wave + WAVES * j;
      const int dl0 = (u & 3) * 16 + l16 - ((u >> 2) * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int r = 0; r < 4; ++r) flane[j][r] = gpow(cur.lg, static_cast<float>(dl0 - r));
    }

    auto score_reads = [&](const uint16_t* kt, bf16x8 (&kfr)[SW][8]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < SW; ++j)
#pragma unroll
        for (int s = 0; s < 8; ++s) kfr[j][s] = ld8(kt + kread[j][s & 3] + 128 * (s >> 2));
    };
    // Decay, mask and store the scores of key block kb (S^T tiles in sacc).
    auto score_out = [&](int kb, const floatx4 (&sacc)[SW], uint16_t* pdst) __attribute__((always_inline)) {
      const int dq = cur.q0 - (cur.cs + kb * kTile);
      const float fblock = gpow(cur.lg, static_cast<float>(dq));
#pragma unroll
      for (int j = 0; j < SW; ++j) {
        const int u = wave + WAVES * j;
        const int qt = u & 3, tt = u >> 2;
        // sacc[r] = S^T[t][q]: t = tt*16 + 4*(lane/16) + r, q = qt*16 + lane%16.
        const int ql = qt * 16 + l16;
        const int tl = tt * 16 + 4 * (lane >> 4);
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = ql - tl - r >= -dq ? sacc[j][r] * (fblock * flane[j][r]) : 0.f;
        uint2 w;
        w.x = pack_bf16x2(x[0], x[1]);
        w.y = pack_bf16x2(x[2], x[3]);
        *reinterpret_cast<uint2*>(pdst + p_off(ql, tl >> 3) + (tl & 7)) = w;
      }
    };

    // Scale chunk-local row j of the read-out by xi_j = gamma^(j+1).
    // Row j = jb + 32qt + 8(r/4) + r%4 for accumulator r of query tile qt,
    // jb = q0 - cs + 4*(lane/32). (The empty asm keeps the 32 factors from
    // being computed ahead of the tile loop and held in registers through it.)
    auto xi_scale = [&]() __attribute__((always_inline)) {
      float lg = cur.lg;
      int jb = cur.q0 - cur.cs + 1 + 4 * (lane >> 5);
      asm volatile("" : "+v"(lg), "+v"(jb));
      const float fjb = static_cast<float>(jb);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float xi = gpow(lg, fjb + static_cast<float>(qt * 32 + 8 * (r >> 2) + (r & 3)));
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) acc[qt][nt][r] *= xi;
        }
    };

    // Wait for all but this step's n copies (memory operations complete in order).
    auto wait_keep = [&](int n) __attribute__((always_inline)) {
      switch (n) {
        case 1: wait_vm_keep<1>(); break;
        case 2: wait_vm_keep<2>(); break;
        case 3: wait_vm_keep<3>(); break;
        case 4: wait_vm_keep<4>(); break;
        case 5: wait_vm_keep<5>(); break;
        case 6: wait_vm_keep<6>(); break;
        case 7: wait_vm_keep<7>(); break;
        default: wait_vm_keep<0>(); break;
      }
    };

    // Step i (buffer phase PH = i mod 3): read the operands of tile i (A from
    // the step's score buffer: the Q slice of a state tile or the scores of a
    // key block) and the K block of the scores of key block i+1-ns; start the
    // copies of step i+2 into the buffers step i-1 read; O += A X_i; the
    // scores; wait for all but this step's copies; barrier.
    auto step = [&](int i, auto ph_tag) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph_tag)::value;
      constexpr int PN = (PH + 1) % 3, PF = (PH + 2) % 3;
      uint16_t* xkcur = pick3<PH>(sXK0, sXK1, sXK2);
      uint16_t* xkfar = pick3<PF>(sXK0, sXK1, sXK2);
      uint16_t* pcur = pick3<PH>(sP0, sP1, sP2);
      uint16_t* pnext = pick3<PN>(sP0, sP1, sP2);
      uint16_t* pfar = pick3<PF>(sP0, sP1, sP2);
      const int kb = i + 1 - ns;
      const bool sc = kb >= 0 && kb < nkb;
      bf16x8 av[2][2], bv[2][NVT];
      if (i >= 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) av[s][qt] = ld8(pcur + pa[s][qt]);
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) bv[s][nt] = ld_x(xkcur, s, nt);
        }
      }
      if (i >= 0 && i < ns) {
        // This slice's columns of the score tiles' query rows.
#pragma unroll
        for (int j = 0; j < SW; ++j) {
          const bf16x8 v = ld8(pcur + pq[j]);
          switch (i) {
            case 0: qf[j][0] = v; break;
            case 1: qf[j][1] = v; break;
            case 2: qf[j][2] = v; break;
            case 3: qf[j][3] = v; break;
            case 4: qf[j][4] = v; break;
            case 5: qf[j][5] = v; break;
            case 6: qf[j][6] = v; break;
            default: qf[j][7] = v; break;
          }
        }
      }
      bf16x8 kfr[SW][8];
      if (sc) score_reads(xkcur + kTile * DV, kfr);
      __builtin_amdgcn_sched_barrier(0);
      const bool cx = i + 2 < ntiles;
      if (cx) copy_x(cur, i + 2, xkfar);
      const int kn = i + 3 - ns;
      const bool ck = kn >= 0 && kn < nkb;
      if (ck) copy_k(cur, kn, xkfar);
      const bool cq = i + 2 < ns && wave < QCH;
      if (cq) copy_qs(cur, i + 2, pfar);
      __builtin_amdgcn_sched_barrier(0);
      if (i >= 0) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) {
            acc[0][nt] = mfma32(av[s][0], bv[s][nt], acc[0][nt]);
            acc[1][nt] = mfma32(av[s][1], bv[s][nt], acc[1][nt]);
          }
      }
      floatx4 sacc[SW];
      if (sc) {
#pragma unroll
        for (int j = 0; j < SW; ++j) {
          sacc[j] = floatx4{};
#pragma unroll
          for (int s = 0; s < 8; ++s) sacc[j] = mfma16(kfr[j][s], qf[j][s], sacc[j]);  // zero past dk
        }
      }
      if (sc) score_out(kb, sacc, pnext);
      wait_keep((cx ? XI : 0) + (ck ? KI : 0) + (cq ? 1 : 0));
      lds_barrier();
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    using H2 = std::integral_constant<int, 2>;

    int i = 0;
    if (ns == 0) step(-1, H2{});
    for (;;) {
      if (i >= ntiles) break;
      if (i == ns && ns > 0) xi_scale();
      step(i++, H0{});
      if (i >= ntiles) break;
      if (i == ns && ns > 0) xi_scale();
      step(i++, H1{});
      if (i >= ntiles) break;
      if (i == ns && ns > 0) xi_scale();
      step(i++, H2{});
    }

    // This block's output rows; then the next block takes over `cur` and its
    // first copies go out before this block's GroupNorm and store (which use
    // no buffer those copies write: the statistics live in sP2).
    uint16_t* const oblk = a.o + (cur.bh * a.N + cur.q0) * static_cast<int64_t>(DV);
    const int oq = cur.qvalid;
    // GroupNorm weight and bias of this wave's columns, requested before the
    // next block's copies so that waiting for them does not wait for those.
    const bool affine = gn.enabled && (gn.weight || gn.bias);
    float w[NVT], bb[NVT];
    if (affine) {
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        const int vcol = vcol0 + nt * 32 + l32;
        w[nt] = gn.weight ? gn.weight[cur.h * DV + vcol] : 1.f;
        bb[nt] = gn.bias ? gn.bias[cur.h * DV + vcol] : 0.f;
      }
    }
    const int Ln = block_of(++it);
    if (Ln >= 0) {
      setup(Ln, cur);
      first_copies(cur);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Optional per-head GroupNorm over the DV columns of each row.
    if (gn.enabled) {
      float* s_stat = reinterpret_cast<float*>(sP2);  // [WAVES][64], then mean[64], rstd[64]
      float* s_mean = s_stat + WAVES * kRows;        // the mean, later -mean * rstd
      float* s_rstd = s_mean + kRows;
      // Each lane holds 32 row slots (query tile qt, accumulator r); a
      // reduce-scatter over the 32 lanes sharing them leaves lane l with the
      // wave's sum for slot l%32; one thread per row then adds the waves.
      const int my_slot = lane & 31;
      const int my_row = (my_slot >> 4) * 32 + acc_row(my_slot & 15, lane);
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        float x[32];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float mean = pass == 0 ? 0.f : s_mean[qt * 32 + acc_row(r, lane)];
            float t = 0.f;
#pragma unroll
            for (int nt = 0; nt < NVT; ++nt) {
              const float d = acc[qt][nt][r] - mean;
              t += pass == 0 ? d : d * d;
            }
            x[qt * 16 + r] = t;
          }
        s_stat[wave * kRows + my_row] = reduce_scatter32(x, lane);
        lds_barrier();  // the next block's copies stay in flight
        if (threadIdx.x < kRows) {
          float t = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < WAVES; ++w2) t += s_stat[w2 * kRows + threadIdx.x];
          t /= DV;
          if (pass == 0) {
            s_mean[threadIdx.x] = t;
          } else {
            const float rstd = 1.0f / sqrtf(t + gn.eps);
            s_rstd[threadIdx.x] = rstd;
            s_mean[threadIdx.x] = -s_mean[threadIdx.x] * rstd;
          }
        }
        lds_barrier();
      }
      // (x - mean) * rstd as one multiply-add per value, then the affine map.
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = qt * 32 + acc_row(r, lane);
          const float rstd = s_rstd[row], shift = s_mean[row];
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) acc[qt][nt][r] = fmaf(acc[qt][nt][r], rstd, shift);
        }
      if (affine) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int nt = 0; nt < NVT; ++nt) acc[qt][nt][r] = fmaf(acc[qt][nt][r], w[nt], bb[nt]);
      }
    }

    // Store: accumulators r and r+1 of a lane are rows rho and rho+1 of one
    // column. Packed to bf16 pairs, one exchange with the neighbouring lane
    // (DPP) and a byte permute give each lane two adjacent columns of one row
    // (the even lane row rho, the odd lane row rho+1), written as one 4-byte
    // store. Rows go out in groups of eight (qt*32 + 8g ..), each through a
    // descriptor whose range ends at the block's last valid row, so the lane
    // offsets are the same for every group.
    {
      const bool odd = lane & 1;
      const int voff = ((4 * (lane >> 5) + (odd ? 1 : 0)) * DV + vcol0 + (l32 & ~1)) * 2;
      // v_perm byte selectors over {neighbour (bytes 4-7), own (bytes 0-3)}:
      // even lanes take both low halves, odd lanes both high halves.
      const unsigned sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = qt * 32 + 8 * g;
          const __amdgpu_buffer_rsrc_t r = make_rsrc(oblk + row0 * DV, min(max(oq - row0, 0), 8) * DV * 2);
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
              // accumulators 4g + 2hp (row row0 + 4*(lane/32) + 2hp) and the next row
              const int rr = 4 * g + 2 * hp;
              const unsigned own = pack_bf16x2(acc[qt][nt][rr], acc[qt][nt][rr + 1]);
              const unsigned nbr = __builtin_amdgcn_update_dpp(0u, own, 0xB1, 0xf, 0xf, true);  // quad_perm [1,0,3,2]
              const unsigned packed = __builtin_amdgcn_perm(nbr, own, sel);
              __builtin_amdgcn_raw_buffer_store_b32(packed, r, voff + (2 * hp * DV + nt * 32) * 2, 0, 0);
            }
        }
    }

    if (Ln < 0) break;
    // The next block's copies and loads were issued before this block's O
    // stores: wait for everything but those stores.
    wait_vm_keep<OSTORES>();
    lds_barrier();
  }
}

}  // namespace

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
  if (walk_full_dk(dk)) return dv / (walk_wide(heads, dk, dv) ? 256 : kWalk2VT);
  return (dk / (32 * walk_k_tiles(dk))) * (dv / kWalkVT);
}

hipError_t launch_mfma_state_walk(const uint16_t* k, const uint16_t* v, const float* state_in, float* state_out,
                                  uint16_t* chunk_states, float* seg_states, int chunks_per_seg, const Dims& d,
                                  int chunk, const HeadDecay& decay, hipStream_t stream) {
  WalkArgs a;
  a.k = k;
  a.v = v;
  a.state_in = state_in;
  a.state_out = state_out;
  a.chunk_states = chunk_states;
  a.seg_states = seg_states;
  a.H = d.H;
  a.N = d.N;
  a.dk = d.dk;
  a.dv = d.dv;
  a.chunk = chunk;
  a.nchunks = (d.N + chunk - 1) / chunk;
  a.chunks_per_seg = chunks_per_seg;
  a.nseg = (a.nchunks + chunks_per_seg - 1) / chunks_per_seg;
  const bool full = walk_full_dk(d.dk);
  const int MT = walk_k_tiles(d.dk);
  a.nkt = full ? 1 : d.dk / (32 * MT);
  const bool wide = walk_wide(static_cast<int64_t>(d.B) * d.H, d.dk, d.dv);
  a.nvt = d.dv / (full ? (wide ? 256 : kWalk2VT) : kWalkVT);
  const int64_t per_seg = static_cast<int64_t>(d.B) * d.H * a.nkt * a.nvt;
  auto walk = [&](int mode) -> hipError_t {
    a.mode = mode;
    const int64_t nblocks = per_seg * (mode == 0 ? a.nseg - 1 : a.nseg);
    const dim3 grid(static_cast<unsigned>(nblocks));
    if (full && d.dk == 256 && wide) mfma_state_walk2_kernel<2, 4><<<grid, kWalk2Threads, 0, stream>>>(a, decay);
    else if (full && d.dk == 256) mfma_state_walk2_kernel<2, 2><<<grid, kWalk2Threads, 0, stream>>>(a, decay);
    else if (full && wide) mfma_state_walk2_kernel<1, 4><<<grid, kWalk2Threads, 0, stream>>>(a, decay);
    else if (full) mfma_state_walk2_kernel<1, 2><<<grid, kWalk2Threads, 0, stream>>>(a, decay);
    else if (MT == 2) mfma_state_walk_kernel<2><<<grid, kThreads, 0, stream>>>(a, decay);
    else mfma_state_walk_kernel<1><<<grid, kThreads, 0, stream>>>(a, decay);
    return hipGetLastError();
  };
  if (a.nseg > 1 && walk_fixup_segments(chunk, d.dk, d.dv)) {
    // One walk of every segment (segment 0 from state_in, the rest from zero),
    // then the fix-up pass.
    hipError_t e = walk(2);
    if (e != hipSuccess) return e;
    FixArgs f;
    f.chunk_states = chunk_states;
    f.seg_states = seg_states;
    f.state_out = state_out;
    f.heads = static_cast<int64_t>(d.B) * d.H;
    f.H = d.H;
    f.N = d.N;
    f.chunk = chunk;
    f.nchunks = a.nchunks;
    f.nseg = a.nseg;
    f.chunks_per_seg = chunks_per_seg;
    f.dkdv = d.dk * d.dv;
    const int64_t threads = f.heads * (f.dkdv / 8);
    walk_fixup_kernel<<<dim3(static_cast<unsigned>((threads + kFixThreads - 1) / kFixThreads)), kFixThreads, 0,
                        stream>>>(f, decay);
    return hipGetLastError();
  }
  for (int mode = (a.nseg > 1 ? 0 : 1); mode <= 1; ++mode) {
    const hipError_t e = walk(mode);
    if (e != hipSuccess) return e;
  }
  if (a.nseg > 1 && state_out) {
    // The final state of every head sits in its segment slot nseg-1: one strided copy.
    const size_t row = static_cast<size_t>(d.dk) * d.dv * sizeof(float);
    const hipError_t e = hipMemcpy2DAsync(state_out, row, seg_states + static_cast<size_t>(a.nseg - 1) * d.dk * d.dv,
                                          row * a.nseg, row, static_cast<size_t>(d.B) * d.H,
                                          hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t resident_workgroups(const void* kernel, int threads, int which, int* out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][kResidentSlots];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cache[dev][which].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
  if (e != hipSuccess) return e;
  const int n = std::max(1, cus * per_cu);
  if (dev >= 0 && dev < kMaxDevices) cache[dev][which].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

hipError_t launch_mfma_chunk_out(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* chunk_states, bool state_for_chunk0, uint16_t* o, const Dims& d,
                                 int chunk, const HeadDecay& decay, const GnArgs& gn, hipStream_t stream) {
  OutArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.chunk_states = chunk_states;
  a.o = o;
  a.state_for_chunk0 = state_for_chunk0 ? 1 : 0;
  a.H = d.H;
  a.N = d.N;
  a.dk = d.dk;
  a.dv = d.dv;
  a.chunk = chunk;
  a.nchunks = (d.N + chunk - 1) / chunk;
  a.nqb = (d.N + kRows - 1) / kRows;
  const int64_t nblocks = static_cast<int64_t>(d.B) * d.H * a.nqb;
  if (nblocks > INT32_MAX) return hipErrorInvalidValue;
  a.nblocks = static_cast<int>(nblocks);
  if (a.nblocks == 0) return hipSuccess;
  // As many workgroups as are resident at once (each loops over its blocks).
  auto launch = [&](auto kernel, int threads, int which) -> hipError_t {
    int wgs = 0;
    const hipError_t e = resident_workgroups(reinterpret_cast<const void*>(kernel), threads, which, &wgs);
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(wgs, nblocks)));
    kernel<<<grid, threads, 0, stream>>>(a, decay, gn);
    return hipGetLastError();
  };
  switch (d.dv) {
    case 128: return launch(mfma_chunk_out_kernel<1, 4>, 256, 0);
    case 256: return launch(mfma_chunk_out_kernel<1, 8>, 512, 1);
    default: return launch(mfma_chunk_out_kernel<2, 8>, 512, 2);
  }
}

}  // namespace ret

// bf16 retention chunk-state walk on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Method ("RetNet - Retentive Network - A Successor to Transformer for LLMs",
// Key Equations: parallel form and chunkwise recurrent form; Key components,
// 1. Retention for the chunk-state carry). For chunk i of length L, local row j:
//   O_[i] = (Q_[i] K_[i]^T (*) D) V_[i] + diag(gamma^(j+1)) Q_[i] R_{i-1}
//   R_i   = gamma^L R_{i-1} + K_[i]^T diag(gamma^(L-1-j)) V_[i]
//
// The chunk-state walk (the output kernel that reads its states is in
// mfma_out.hip): one workgroup per (head, 32*MT-row k-tile, v-tile, sequence
// segment) keeps its tile of R in MFMA accumulators (fp32) and walks the
// chunks in order. Before each chunk it stores R as bf16 ([k][v], v fastest,
// like V); then it applies the carry and accumulates K^T (zeta V) over 64-row
// key blocks. Long sequences with few heads are cut into chunk-aligned
// segments: a first launch computes each segment's end state (segment 0 from
// state_in, the others from zero), the second starts every segment from the
// earlier segments' end states, each decayed to its start, and writes the
// chunk states.
//
// Data movement: every tile (K, V) is copied row-major into LDS with 16-byte
// accesses; the next tile's global loads are issued into registers before the
// current tile's matrix work so their latency is hidden. Operands that need a
// transposed view (V as the B operand, K^T as the A operand) are fetched with
// ds_read_b64_tr_b16, which hands each lane four consecutive rows of one
// column. Workgroups that share K/V/state tiles get
// consecutive logical indices and are placed on the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs), so the re-reads hit one L2.
//
// MFMA 32x32x16 operand layouts used throughout (lane l of 64):
//   A[i][kk]: i = l % 32, kk = 8*(l/32) + 0..7
//   B[kk][j]: j = l % 32, kk = 8*(l/32) + 0..7
//   D[i][j] : j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4 for accumulator r = 0..15
#include <type_traits>
#include <algorithm>
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
  // of this thread's rows are fixed (r <= 63: at most 2^63 for gamma > 1/2;
  // smaller decays take one exp2 per row instead).
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
      float z[ZP];
      if (lg > -1.0f) {
        const float z0 = gpow(lg, static_cast<float>(L - 1 - t0));
#pragma unroll
        for (int m = 0; m < ZP; ++m) z[m] = z0 * zrow[m];
      } else {
        // gamma <= 1/2: gamma^(-r) may leave the float range; one exp2 per row
        // (rows past the chunk end are zero and take exponent 0).
#pragma unroll
        for (int m = 0; m < ZP; ++m) {
          const int row = kScaleK ? TileRegs<PIECES, kThreads, KT>::row_of(m)
                                  : TileRegs<VPIECES, kThreads, kWalkVT>::row_of(m);
          z[m] = gpow(lg, static_cast<float>(max(L - 1 - t0 - row, 0)));
        }
      }
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
  // at t0; the gamma^(-r) factors of this thread's V rows are fixed (at most
  // 2^63 for gamma > 1/2; smaller decays take one exp2 per row instead).
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
    float z[VP];
    if (lg > -1.0f) {
      const float z0 = gpow(lg, static_cast<float>(L - 1 - t0));
#pragma unroll
      for (int m = 0; m < VP; ++m) z[m] = z0 * zrow[m];
    } else {
      // gamma <= 1/2: gamma^(-r) may leave the float range; one exp2 per row
      // (rows past the chunk end are zero and take exponent 0).
#pragma unroll
      for (int m = 0; m < VP; ++m)
        z[m] = gpow(lg, static_cast<float>(max(L - 1 - t0 - TileRegs<VP, NT, VT>::row_of(m), 0)));
    }
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

}  // namespace

namespace {

// One walk launch in `mode` (grid: every head, k tile, v tile and launched segment).
hipError_t launch_walk_mode(WalkArgs& a, int mode, const Dims& d, const HeadDecay& decay, hipStream_t stream) {
  const bool full = walk_full_dk(d.dk);
  const bool wide = walk_wide(static_cast<int64_t>(d.B) * d.H, d.dk, d.dv);
  const int MT = walk_k_tiles(d.dk);
  const int64_t per_seg = static_cast<int64_t>(d.B) * d.H * a.nkt * a.nvt;
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
}

WalkArgs walk_args(const uint16_t* k, const uint16_t* v, const float* state_in, float* state_out,
                   uint16_t* chunk_states, float* seg_states, int chunks_per_seg, const Dims& d, int chunk) {
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
  a.mode = 0;
  return a;
}

}  // namespace

hipError_t launch_segment_ends(const uint16_t* k, const uint16_t* v, const float* state_in, float* seg_states,
                               int chunks_per_seg, const Dims& d, int chunk, const HeadDecay& decay,
                               hipStream_t stream) {
  WalkArgs a = walk_args(k, v, state_in, nullptr, nullptr, seg_states, chunks_per_seg, d, chunk);
  if (a.nseg < 2) return hipSuccess;
  return launch_walk_mode(a, 0, d, decay, stream);
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

}  // namespace ret

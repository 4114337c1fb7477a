// bf16 retention output kernel on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// Method ("RetNet - Retentive Network - A Successor to Transformer for LLMs",
// Key Equations: parallel form and chunkwise recurrent form). For chunk i of
// length L, local row j:
//   O_[i] = (Q_[i] K_[i]^T (*) D) V_[i] + diag(gamma^(j+1)) Q_[i] R_{i-1}
// with R_{i-1} the bf16 chunk state the state walk stored before chunk i.
//
// One workgroup per (head, 64-row query block) with the full dv row: the
// cross-chunk read-out O = Q R over 32-row slices of the stored state, scaled
// by gamma^(j+1), then the key blocks of its chunk up to the diagonal:
// S^T = K Q^T, the decay gamma^(n-m) (zero above the diagonal) applied to the
// fp32 scores in registers, scores rounded to bf16 through LDS, O += A V. The
// per-head GroupNorm and the bf16 store close it. The N x N mask never exists
// in memory; with one chunk spanning the sequence this is the parallel form.
//
// This file is compiled on its own, with the iterative ILP scheduler
// (-amdgpu-sched-strategy=iterative-ilp), which measured faster here than the
// default and slower on the state walk.
//
// MFMA 32x32x16 operand layouts used throughout (lane l of 64):
//   A[i][kk]: i = l % 32, kk = 8*(l/32) + 0..7
//   B[kk][j]: j = l % 32, kk = 8*(l/32) + 0..7
//   D[i][j] : j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4 for accumulator r = 0..15
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "kernels.h"
#include "mfma_tiles.h"

namespace ret {

namespace {

constexpr int kRows = 64;  // query / key block height

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
//
// EPI (a separate instance each, so the extra registers do not weigh on the
// plain one): 0 stores the result; 1 multiplies it (after the GroupNorm) by
// swish(gate); 2 adds the bf16 values already in O (partial results of one
// product accumulated over several launches, in fp32 before rounding).
template <int NVT, int WAVES, int EPI>
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
    // Decay, mask and store the scores of key block kb (S^T tiles in sacc):
    // the block factor times the lane factor, or, for heads with gamma <= 1/2
    // (never on the 1 - 2^(-5-h) schedule), one exp2 per score, since the lane
    // factor (down to gamma^-35) would leave the float range.
    const bool split_decay = cur.lg > -1.0f;
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
        if (split_decay) {
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = ql - tl - r >= -dq ? sacc[j][r] * (fblock * flane[j][r]) : 0.f;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            x[r] = ql - tl - r >= -dq ? sacc[j][r] * gpow(cur.lg, static_cast<float>(dq + ql - tl - r)) : 0.f;
        }
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
    // Gate values, or the values already in O, as bf16 pairs at exactly the
    // positions this lane stores, also requested before the next block's
    // copies. Rows past the block's last valid row read as zero through the
    // descriptors' ranges.
    constexpr bool gated = EPI != 0;
    const int voff = ((4 * (lane >> 5) + (lane & 1)) * DV + vcol0 + (l32 & ~1)) * 2;
    uint32_t gv[2][4][NVT][2];
    if constexpr (gated) {
      const uint16_t* gbase = EPI == 1 ? static_cast<const uint16_t*>(gn.gate) : a.o;
      const uint16_t* gblk = gbase + (cur.bh * a.N + cur.q0) * static_cast<int64_t>(DV);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = qt * 32 + 8 * g;
          const __amdgpu_buffer_rsrc_t r = make_rsrc(gblk + row0 * DV, min(max(oq - row0, 0), 8) * DV * 2);
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
            for (int hp = 0; hp < 2; ++hp)
              gv[qt][g][nt][hp] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + (2 * hp * DV + nt * 32) * 2, 0, 0);
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
    // column. One exchange with the neighbouring lane (DPP) gives each lane
    // two adjacent columns of one row (the even lane row rho, the odd lane row
    // rho+1), written as one 4-byte store of a bf16 pair. Without a gate the
    // pair is exchanged already packed (then a byte permute picks the halves);
    // with a gate it is exchanged in fp32 and multiplied by swish of the gate
    // pair at the same position before rounding. Rows go out in groups of
    // eight (qt*32 + 8g ..), each through a descriptor whose range ends at the
    // block's last valid row, so the lane offsets are the same for every group.
    {
      const bool odd = lane & 1;
      // v_perm byte selectors over {neighbour (bytes 4-7), own (bytes 0-3)}:
      // even lanes take both low halves, odd lanes both high halves.
      const unsigned sel = odd ? 0x03020706u : 0x05040100u;
      auto store_rows = [&](auto epi_tag) __attribute__((always_inline)) {
        constexpr int kEpi = decltype(epi_tag)::value;
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
                unsigned packed;
                if constexpr (kEpi != 0) {
                  // the even lane sends its row rho+1 value, the odd lane its row rho value
                  const float a0 = acc[qt][nt][rr], a1 = acc[qt][nt][rr + 1];
                  const float send = odd ? a0 : a1;
                  const float recv = __builtin_bit_cast(
                      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xf, 0xf, true));
                  const float lo = odd ? recv : a0, hi = odd ? a1 : recv;
                  const uint32_t gp = gv[qt][g][nt][hp];
                  const float g_lo = __uint_as_float(gp << 16), g_hi = __uint_as_float(gp & 0xffff0000u);
                  if constexpr (kEpi == 1) {
                    packed = pack_bf16x2(lo * swish(g_lo), hi * swish(g_hi));
                  } else {
                    packed = pack_bf16x2(lo + g_lo, hi + g_hi);
                  }
                } else {
                  const unsigned own = pack_bf16x2(acc[qt][nt][rr], acc[qt][nt][rr + 1]);
                  const unsigned nbr = __builtin_amdgcn_update_dpp(0u, own, 0xB1, 0xf, 0xf, true);  // quad_perm [1,0,3,2]
                  packed = __builtin_amdgcn_perm(nbr, own, sel);
                }
                __builtin_amdgcn_raw_buffer_store_b32(packed, r, voff + (2 * hp * DV + nt * 32) * 2, 0, 0);
              }
          }
      };
      store_rows(std::integral_constant<int, EPI>{});
    }

    if (Ln < 0) break;
    // The next block's copies and loads were issued before this block's O
    // stores: wait for everything but those stores.
    wait_vm_keep<OSTORES>();
    lds_barrier();
  }
}

}  // namespace

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
                                 int chunk, const HeadDecay& decay, const GnArgs& gn, bool accumulate,
                                 hipStream_t stream) {
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
  const int epi = (gn.enabled && gn.gate) ? 1 : (accumulate ? 2 : 0);
  switch (d.dv) {
    case 128:
      return epi == 1   ? launch(mfma_chunk_out_kernel<1, 4, 1>, 256, 3)
             : epi == 2 ? launch(mfma_chunk_out_kernel<1, 4, 2>, 256, 6)
                        : launch(mfma_chunk_out_kernel<1, 4, 0>, 256, 0);
    case 256:
      return epi == 1   ? launch(mfma_chunk_out_kernel<1, 8, 1>, 512, 4)
             : epi == 2 ? launch(mfma_chunk_out_kernel<1, 8, 2>, 512, 7)
                        : launch(mfma_chunk_out_kernel<1, 8, 0>, 512, 1);
    default:
      return epi == 1   ? launch(mfma_chunk_out_kernel<2, 8, 1>, 512, 5)
             : epi == 2 ? launch(mfma_chunk_out_kernel<2, 8, 2>, 512, 8)
                        : launch(mfma_chunk_out_kernel<2, 8, 0>, 512, 2);
  }
}

}  // namespace ret

// Single-pass bf16 chunkwise retention on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// Method ("RetNet - Retentive Network - A Successor to Transformer for LLMs",
// Key Equations: chunkwise recurrent form; Key components, 1. Retention). For
// chunk i of length L, local row j:
//   O_[i] = (Q_[i] K_[i]^T (*) D) V_[i] + diag(gamma^(j+1)) Q_[i] R_{i-1}
//   R_i   = gamma^L R_{i-1} + K_[i]^T diag(gamma^(L-1-j)) V_[i]
// then the per-head GroupNorm ("What Is RetNet ? ...", How is this dual
// representation achieved?: GroupNorm after retention) and, optionally, the
// swish gate of the gated block (Key components, 4. block).
//
// One workgroup of eight waves owns (head, 256-column v tile) and walks the
// chunks in order, with its dk x 256 slab of R in fp32 MFMA accumulators for
// the whole sequence: wave w keeps columns 32w..32w+31 of every state row
// (dk/32 accumulator tiles). R never leaves the registers, and each Q, K and V
// element crosses from HBM once per workgroup that needs it (Q and K by the
// dv/256 workgroups of a head, which sit on one XCD so the second read is an
// L2 hit).
//
// Per 64-row query block of a chunk:
//   read-out  O = Q R_{i-1}: A = Q from LDS, B = the wave's state tile rounded
//             to bf16 in registers (v_permlane32_swap turns the accumulator
//             row order into the operand's contraction order), then the rows
//             are scaled by xi_j = gamma^(j+1);
//   key steps for the 32-key blocks of the chunk up to the diagonal: the
//             scores of the next block S^T = K Q^T on 16x16x32 MFMAs (one
//             16 x 16 tile per wave, Q and K from LDS), decayed by
//             gamma^(q-t) and masked in registers, rounded to bf16 into a
//             score buffer; O += S V with V the block's rows of this v tile;
//   GroupNorm: the mean and sum of squared deviations of each row over the
//             workgroup's 256 columns are published to the other v tiles of
//             the head through a small workspace mailbox; the merge (Chan's
//             pairwise formula in a fixed order, so every v tile gets the same
//             bits), the normalisation and the store of this block happen
//             after the next block's read-out, so waiting for the other
//             workgroups overlaps matrix work.
// After the chunk's last query block, the update pass R = gamma^L R + K^T
// (zeta V) streams the chunk's 32-key blocks once more (zeta applied to the V
// operand in registers).
//
// The v tiles of a head exchange GroupNorm statistics, so they must run at the
// same time: the kernel is launched cooperatively (all workgroups resident),
// each workgroup taking units u = r*G + (its index) for rounds r, the v tiles
// of a head being consecutive units (G a multiple of their count). Waits are
// bounded.
//
// LDS: the query block's Q (32 KiB), three buffer sets of a V tile and a K
// block (32 KiB each) copied straight from global memory two steps ahead
// (buffer loads with an LDS destination), three score buffers, GroupNorm
// statistics: about 143 KiB, one workgroup per CU.
//
// MFMA 32x32x16 operand layouts (lane l of 64):
//   A[i][kk]: i = l % 32, kk = 8*(l/32) + 0..7
//   B[kk][j]: j = l % 32, kk = 8*(l/32) + 0..7
//   D[i][j] : j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4 for accumulator r = 0..15
// MFMA 16x16x32: A[i][kk]: i = l % 16, kk = 8*(l/16) + 0..7; B likewise with
// j = l % 16; D[i][j]: j = l % 16, i = 4*(l/16) + r for r = 0..3.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "kernels.h"
#include "mfma_tiles.h"

namespace ret {

namespace {

constexpr int kRowsF = 64;      // query block rows
constexpr int kTileF = 32;      // key block rows
constexpr int kWavesF = 8;
constexpr int kThreadsF = 64 * kWavesF;
constexpr int kVT = 256;        // v columns per workgroup (32 per wave)
constexpr int kPitch = 256;     // LDS pitch (elements) of the Q block and K blocks (dk <= 256)
// One mailbox slot: per row a 64-bit word (mean, tag) and one (M2, tag), the
// tag (upper half) being the exchange number + 1; 64 rows, 1 KiB.
constexpr int kMailWords = 2 * kRowsF;
constexpr int kQCopies = 8;             // Q-block copies per copying wave (waves 0-3)
constexpr int kGnWave = 7;              // the wave that publishes and merges GroupNorm statistics
constexpr int kOStores = 16;            // 4-byte O stores per lane and query block

struct FusedArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const float* state_in;  // [B*H][dk][dv] or null
  float* state_out;       // [B*H][dk][dv] or null
  uint64_t* mail;         // [units][2 slots][kMailWords], zeroed before the launch
  // Sequences cut into nseg segments of chunks_per_seg chunks (nseg = 1: whole
  // sequences): seg_states[bh][s] holds the state reached at the end of
  // segment s < nseg - 1 when it starts from zero (segment 0 from state_in).
  const float* seg_states;
  int nseg, chunks_per_seg;
  // Row pitches (elements) of q and k (dk when they are whole tensors). With
  // `reverse` every sequence is taken in reverse token order: logical row t
  // of q, k, v and o is memory row N-1-t (a reverse-time retention without
  // reversed copies).
  int ldq, ldk, reverse;
  // A second retention of the same sizes in the same launch: units from
  // job_units on take q2, k2, v2, o2, state_in2 and reverse2 (no final
  // state, no segments). job_units = units when there is none.
  const uint16_t* q2;
  const uint16_t* k2;
  const uint16_t* v2;
  uint16_t* o2;
  const float* state_in2;
  int reverse2, job_units;
  int H, N, dk, dv, chunk, nchunks, nvt, units;
  int spin_limit;         // polls of a partner's flag before giving up on it
};

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void vm_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
// The same for a wave-uniform n (0..31): a branch per value, the wait count
// being an immediate.
template <int... Ns>
__device__ __forceinline__ void vm_keep_table(int n, std::integer_sequence<int, Ns...>) {
  ((n == Ns ? (vm_keep<Ns>(), 0) : 0), ...);
}
__device__ __forceinline__ void vm_keep_n(int n) {
  vm_keep_table(n < 31 ? n : 31, std::make_integer_sequence<int, 32>{});
}

template <int P>
__device__ __forceinline__ uint16_t* pick(uint16_t* b0, uint16_t* b1, uint16_t* b2) {
  return P == 0 ? b0 : (P == 1 ? b1 : b2);
}

// Rows 16s..16s+15 of a 32 x 32 state tile (accumulator order) as the B
// operand of the read-out, contraction index in natural order: a lane holds
// rows 4g..4g+3 and 8+4g..8+4g+3 (g = l/32) of the 16; one v_permlane32_swap
// per register pair gives lanes 0-31 rows 0..7 and lanes 32-63 rows 8..15.
__device__ __forceinline__ bf16x8 state_operand(const floatx16& t, int s) {
  uint32_t p0 = pack_bf16x2(t[8 * s + 0], t[8 * s + 1]);
  uint32_t p1 = pack_bf16x2(t[8 * s + 2], t[8 * s + 3]);
  uint32_t p2 = pack_bf16x2(t[8 * s + 4], t[8 * s + 5]);
  uint32_t p3 = pack_bf16x2(t[8 * s + 6], t[8 * s + 7]);
  // Swap the upper half-wave's rows 4g.. (p0, p1) with the lower half-wave's rows 8+4g.. (p2, p3).
  const auto x0 = __builtin_amdgcn_permlane32_swap(p0, p2, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(p1, p3, false, false);
  u32x4 u;
  u[0] = x0[0];
  u[1] = x1[0];
  u[2] = x0[1];
  u[3] = x1[1];
  return __builtin_bit_cast(bf16x8, u);
}

// GEN: the general layout (row pitches, reverse order, a second retention);
// the plain instances fold those to dk, forward order and one retention,
// keeping the registers they would hold.
template <int MT, int EPI, bool GEN>
__global__ void __launch_bounds__(kThreadsF, 1) fused_chunk_kernel(FusedArgs a, HeadDecay decay, GnArgs gn) {
  constexpr int XK = kTileF * kVT + kTileF * kPitch;  // V tile at 0, K block after it
  constexpr int PT = kRowsF * kTileF;                 // score tile (64 queries x 32 keys)
  constexpr int DKMAX = 32 * MT;
  __shared__ __attribute__((aligned(1024))) uint16_t sQ[kRowsF * kPitch];
  __shared__ __attribute__((aligned(1024))) uint16_t sXK0[XK];
  __shared__ __attribute__((aligned(1024))) uint16_t sXK1[XK];
  __shared__ __attribute__((aligned(1024))) uint16_t sXK2[XK];
  __shared__ __attribute__((aligned(1024))) uint16_t sP0[PT];
  __shared__ __attribute__((aligned(1024))) uint16_t sP1[PT];
  __shared__ __attribute__((aligned(1024))) uint16_t sP2[PT];
  // Per-wave row partials [8][64], then mean [64] and sum of squared deviations [64]
  // of this workgroup's columns, then the merged shift [64] and 1/std [64].
  __shared__ __attribute__((aligned(16))) float sG[kWavesF * kRowsF + 4 * kRowsF];
  __shared__ __attribute__((aligned(16))) float sGw[kWavesF * kRowsF];
  // GroupNorm weight and bias of the unit's 256 columns.
  __shared__ float sAff[2 * kVT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int l16 = lane & 15;
  const int vcol0 = wave * 32;  // this wave's columns within the v tile
  const int dk = a.dk, dv = a.dv;
  const int ldq = GEN ? a.ldq : dk, ldk = GEN ? a.ldk : dk;

  // ---- per-lane LDS offsets (elements), fixed for the kernel; the empty asm
  // keeps each read one opaque offset away from its array, so the compiler
  // keeps the array's alias information and never waits for copies into the
  // other buffers.
  // Transposed V operand (B of S V and of the update): two ds_read_b64_tr_b16,
  // rows 16s + 8*(l/32) + (l%16)/4 (and +4) of the swizzled V tile, columns
  // vcol0 + 16*((l/16)%2) + 4*(l%4)..
  int xo;
  {
    const int g = lane >> 4, j = lane & 15;
    const int row = 8 * (g >> 1) + (j >> 2);
    const int col = vcol0 + 16 * (g & 1) + 4 * (j & 3);
    xo = row * kVT + (x_pos(row, col >> 3) << 3) + (col & 7);
    asm volatile("" : "+v"(xo));
  }
  auto ld_v = [&](const uint16_t* tile, int s) __attribute__((always_inline)) {
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(tile + xo + 16 * s * kVT));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(tile + xo + (16 * s + 4) * kVT));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Score-buffer element offset of granule g (8 columns) of row r (64-byte
  // rows, granules XOR-swizzled by (r/4)%4).
  auto p_off = [](int r, int g) __attribute__((always_inline)) { return r * kTileF + ((g ^ ((r >> 2) & 3)) << 3); };
  // A operand of S V: score rows qt*32 + l%32, granule 2s + l/32 (the two
  // query tiles are 1024 elements apart with the same swizzle).
  int pa[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    pa[s] = p_off(l32, 2 * s + (lane >> 5));
    asm volatile("" : "+v"(pa[s]));
  }
  // This wave's score tile: queries 16*(wave%4).., keys 16*(wave/4)..
  const int sq = wave & 3, st = wave >> 2;
  // Score operands: K rows 16*st + l%16 and Q rows 16*sq + l%16, granule
  // 4s + l/16 (k_swz layout); s and s+4 differ by 128 elements.
  int kread[4], qread[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kread[s] = k_swz(st * 16 + l16, 4 * s + (lane >> 4));
    qread[s] = k_swz(sq * 16 + l16, 4 * s + (lane >> 4));
    asm volatile("" : "+v"(kread[s]), "+v"(qread[s]));
  }
  // Read-out A operand: Q row qt*32 + l%32, granule 4i + 2s + l/32 of that
  // row (row % 16 = l % 16 for both qt): base + ((4i + 2s) ^ (l16 & 14)) | gbit.
  int qro_row = l32 * kPitch;
  asm volatile("" : "+v"(qro_row));
  // Update A operand (K^T): two ds_read_b64_tr_b16 from a K block stored in
  // the V tiles' layout (granules x_pos-swizzled), rows 16s + 8*(l/32) +
  // (l%16)/4 (and +4), columns 32mt + 16*((l/16)%2) + 4*(l%4)... The row's
  // swizzle bits (row % 4 = (l%16)/4) are the same for every s and for +4, so
  // granule 4mt + c of column block mt sits at 4*((mt%4) ^ ((l%16)/4)) + c
  // (+16 for mt >= 4): four per-lane offsets, the rest immediate.
  // (Computed at the start of each update pass: an empty asm on the lane
  // number keeps them out of the registers held through the key steps.)
  auto kt_offsets = [&](int (&ktx)[4]) __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const int rq = (l & 15) >> 2;
    const int rbase = 8 * (l >> 5) + rq;
    const int c3 = 2 * ((l >> 4) & 1) + ((l & 3) >> 1);
    const int c7 = 4 * (l & 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      ktx[m] = rbase * kVT + 8 * (4 * (m ^ rq) + c3) + c7;
      asm volatile("" : "+v"(ktx[m]));
    }
  };
  auto ld_kt = [&](const int (&ktx)[4], const uint16_t* kblk, int s, int mt) __attribute__((always_inline)) {
    const uint16_t* p = kblk + ktx[mt & 3] + 16 * s * kVT + 128 * (mt >> 2);
    const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
    const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p + 4 * kVT));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- copy offsets (bytes into the source), fixed for the kernel.
  // A 1-KiB piece c of a K block or the Q block holds rows 2c, 2c+1; lane l
  // fills slot l%32 of row 2c + l/32 with source granule slot ^ (row % 16)
  // (zero past dk). Pieces c = wave + 8m: the row advances by 16m, so the
  // swizzle is that of m = 0 and piece m lies 16m rows further.
  int kqoff;
  {
    const int row = 2 * wave + (lane >> 5);
    const int g = (lane & 31) ^ (row & 15);
    kqoff = g * 8 < dk ? (row * ldk + g * 8) * 2 : kOutOfRange;
  }
  // The Q block is copied by waves 0-3 only (pieces c = wave + 4m, m = 0..7,
  // rows 2c, 2c+1): wave 7, which publishes the GroupNorm statistics and so
  // waits for all its memory operations, never has a Q copy in flight. Row
  // 2*wave + 8m + l/32 takes the swizzle of m even or odd.
  auto q_offsets = [&](int (&qoff)[2]) __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int row = 2 * (wave & 3) + 8 * par + (l >> 5);
      const int g = (l & 31) ^ (row & 15);
      qoff[par] = g * 8 < dk ? (row * ldq + g * 8) * 2 : kOutOfRange;
    }
  };
  // The same pieces of a K block in the V tiles' layout (the update pass):
  // source granule x_pos(row, slot), zero past dk.
  // (Computed at each use, as above.)
  auto kx_offset = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const int row = 2 * wave + (l >> 5);
    const int pos = x_pos(row, l & 31);
    return pos * 8 < dk ? (row * ldk + pos * 8) * 2 : kOutOfRange;
  };
  // A piece c of a V tile: lane l fills granule 64c + l of the swizzled tile,
  // row 2c + l/32, slot l%32, taking source granule x_pos(row, slot) of the
  // row (the swizzle is an involution); pieces m lie 16m rows further.
  int voff;
  {
    const int row = 2 * wave + (lane >> 5);
    const int pos = x_pos(row, lane & 31);
    voff = (row * dv + pos * 8) * 2;
  }

  // ---- work assignment
  const int G = gridDim.x;
  const int lwg = xcd_logical_block(blockIdx.x, G);

  for (int unit = lwg; unit < a.units; unit += G) {
    // Unit = (retention, head, segment, v tile), v tile fastest: the v tiles
    // of a segment (which exchange GroupNorm statistics) are neighbours.
    const bool second = GEN && unit >= a.job_units;
    const int ju = second ? unit - a.job_units : unit;
    const uint16_t* const jq = second ? a.q2 : a.q;
    const uint16_t* const jk = second ? a.k2 : a.k;
    const uint16_t* const jv = second ? a.v2 : a.v;
    uint16_t* const jo = second ? a.o2 : a.o;
    const int vt = ju % a.nvt;
    const int seg = (ju / a.nvt) % a.nseg;
    const int64_t bh = ju / a.nvt / a.nseg;
    const int h = static_cast<int>(bh % a.H);
    const float lg = decay.log2g[h];
    // This unit's rows: [row0, row0 + Nu) of the head's sequence, chunks
    // counted from row0 (segments start on chunk boundaries).
    const int row0 = seg * a.chunks_per_seg * a.chunk;
    const int Nu = min(a.chunks_per_seg * a.chunk, a.N - row0);
    const int ncu = (Nu + a.chunk - 1) / a.chunk;
    const int64_t rbase = bh * static_cast<int64_t>(a.N) + row0;  // first row in [B*H*N]
    const bool rev = GEN && (second ? a.reverse2 : a.reverse) != 0;
    // Forward: the unit's first row. Reverse: the head's memory row 0 (the
    // unit's logical row t sits at memory row N-1-t).
    const int64_t mrow = rev ? bh * static_cast<int64_t>(a.N) : rbase;
    const uint16_t* qh = jq + mrow * ldq;
    const uint16_t* kh = jk + mrow * ldk;
    const uint16_t* vh = jv + mrow * dv + vt * kVT;
    uint16_t* oh = jo + mrow * dv + vt * kVT;
    const int nm1 = a.N - 1 - row0;  // reverse: memory row of logical row t is nm1 - t
    float* const state_out = seg == a.nseg - 1 && !second ? a.state_out : nullptr;
    const int64_t dkdv = static_cast<int64_t>(dk) * dv;
    uint64_t* mymail = a.mail + static_cast<int64_t>(unit) * 2 * kMailWords;
    const int group0 = unit - vt;  // first unit of this head's v tiles
    // Powers of gamma: for gamma > 1/2 a power is split into a per-block
    // exp2 and per-lane factors gamma^(-e), e <= 35 (at most 2^35); smaller
    // decays (never on the 1 - 2^(-5-h) schedule) take one exp2 per value,
    // since those factors would leave the float range.
    const bool split_decay = lg > -1.0f;

    // R in accumulators: tile mt holds state rows 32mt.., column
    // vt * 256 + vcol0 + l32 (this lane's).
    floatx16 R[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) R[mt] = floatx16{};
    // The state this unit starts from: state_in for the first segment; for a
    // later one starting at row0, sum over earlier segments s' of
    // gamma^(row0 - end_s') U_s' (U_0 already carries state_in).
    const float* const state_in = second ? a.state_in2 : a.state_in;
    const bool has_in = seg > 0 || state_in != nullptr;
    const int nsrc = seg > 0 ? seg : (state_in ? 1 : 0);
    // The state moves between HBM and the accumulators through LDS, four
    // 32-row tiles (32 KiB of fp32 each) at a time in sQ and the three buffer
    // sets: the copies are whole 1-KiB rows, and a lane's 16 accumulator
    // values lie at constant offsets from one per-lane LDS address.
    uint16_t* const stage[4] = {sQ, sXK0, sXK1, sXK2};
    const int acc_lds = (4 * (lane >> 5)) * kVT + vcol0 + l32;  // float index of accumulator 0
    for (int src = 0; src < nsrc; ++src) {
      const float* sbase = (seg > 0 ? a.seg_states + (bh * a.nseg + src) * dkdv : state_in + bh * dkdv) + vt * kVT;
      const float fsrc = seg > 0 ? gpow(lg, static_cast<float>(row0 - (src + 1) * a.chunks_per_seg * a.chunk)) : 1.f;
#pragma unroll
      for (int g4 = 0; g4 < MT; g4 += 4) {
#pragma unroll
        for (int t = 0; t < 4 && g4 + t < MT; ++t) {
          // Rows 32(g4+t) + 4*wave + m, m = 0..3: one 1-KiB row per copy.
          const __amdgpu_buffer_rsrc_t r = make_rsrc(sbase + static_cast<int64_t>(32 * (g4 + t)) * dv,
                                                     (31 * dv + kVT) * 4);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            dma16s(r, stage[t] + (4 * wave + m) * 512, lane * 16, (4 * wave + m) * dv * 4);
        }
        wait_vmem();
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4 && g4 + t < MT; ++t) {
          const float* f = reinterpret_cast<const float*>(stage[t]) + acc_lds;
#pragma unroll
          for (int r = 0; r < 16; ++r) R[g4 + t][r] = fmaf(fsrc, f[(8 * (r >> 2) + (r & 3)) * kVT], R[g4 + t][r]);
        }
        __syncthreads();
      }
    }

    // Copies.
    // (Waves 0-3 only; kQCopies copies each.)
    // In reverse order a copy's descriptor spans the head's rows and each
    // lane's offset carries its memory row nm1 - (t0 + r): rows before the
    // head's first (logical rows past the end) come out negative, past the
    // descriptor's range as unsigned numbers, and so read as zero.
    const int rev_q_range = ((a.N - 1) * ldq + dk) * 2;
    const int rev_k_range = ((a.N - 1) * ldk + dk) * 2;
    const int rev_v_range = ((a.N - 1) * dv + kVT) * 2;
    // Row r of a tile's piece layout and the byte offset of its column part
    // (the same permutations as the forward offsets above).
    auto rev_row = [&](int pieces_per_row_step) __attribute__((always_inline)) {
      int l = lane;
      asm volatile("" : "+v"(l));
      return 2 * (wave & (pieces_per_row_step - 1)) + (l >> 5);
    };
    auto copy_q = [&](int q0) __attribute__((always_inline)) {
      if (wave < 4) {
        if (!rev) {
          int qoff[2];
          q_offsets(qoff);
          const int rows = min(kRowsF, Nu - q0);
          const __amdgpu_buffer_rsrc_t r =
              make_rsrc(qh + static_cast<int64_t>(q0) * ldq, ((rows - 1) * ldq + dk) * 2);
#pragma unroll
          for (int m = 0; m < 8; ++m) dma16s(r, sQ + (wave + 4 * m) * 512, qoff[m & 1], 8 * (m & ~1) * ldq * 2);
        } else {
          const __amdgpu_buffer_rsrc_t r = make_rsrc(qh, rev_q_range);
          const int row = rev_row(4);
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int rr = row + 8 * m;
            const int g = (lane & 31) ^ (rr & 15);
            const int off = g * 8 < dk ? ((nm1 - q0 - rr) * ldq + g * 8) * 2 : kOutOfRange;
            dma16s(r, sQ + (wave + 4 * m) * 512, off, 0);
          }
        }
      }
    };
    auto copy_k = [&](int t0, uint16_t* set) __attribute__((always_inline)) {
      if (!rev) {
        const int rows = min(kTileF, Nu - t0);
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(kh + static_cast<int64_t>(t0) * ldk, ((rows - 1) * ldk + dk) * 2);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          dma16s(r, set + kTileF * kVT + (wave + kWavesF * m) * 512, kqoff, m * 16 * ldk * 2);
      } else {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(kh, rev_k_range);
        const int row = rev_row(8);
        const int g = (lane & 31) ^ (row & 15);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int off = g * 8 < dk ? ((nm1 - t0 - row - 16 * m) * ldk + g * 8) * 2 : kOutOfRange;
          dma16s(r, set + kTileF * kVT + (wave + kWavesF * m) * 512, off, 0);
        }
      }
    };
    // K block at t0 for the update pass: into the V-tile slot layout of `set`'s K part.
    auto copy_kx = [&](int t0, uint16_t* set) __attribute__((always_inline)) {
      if (!rev) {
        const int kxoff = kx_offset();
        const int rows = min(kTileF, Nu - t0);
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(kh + static_cast<int64_t>(t0) * ldk, ((rows - 1) * ldk + dk) * 2);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          dma16s(r, set + kTileF * kVT + (wave + kWavesF * m) * 512, kxoff, m * 16 * ldk * 2);
      } else {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(kh, rev_k_range);
        const int row = rev_row(8);
        const int pos = x_pos(row, lane & 31);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int off = pos * 8 < dk ? ((nm1 - t0 - row - 16 * m) * ldk + pos * 8) * 2 : kOutOfRange;
          dma16s(r, set + kTileF * kVT + (wave + kWavesF * m) * 512, off, 0);
        }
      }
    };
    auto copy_v = [&](int t0, uint16_t* set) __attribute__((always_inline)) {
      if (!rev) {
        const int rows = min(kTileF, Nu - t0);
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(vh + static_cast<int64_t>(t0) * dv, ((rows - 1) * dv + kVT) * 2);
#pragma unroll
        for (int m = 0; m < 2; ++m) dma16s(r, set + (wave + kWavesF * m) * 512, voff, m * 16 * dv * 2);
      } else {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(vh, rev_v_range);
        const int row = rev_row(8);
        const int pos = x_pos(row, lane & 31);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          dma16s(r, set + (wave + kWavesF * m) * 512, ((nm1 - t0 - row - 16 * m) * dv + pos * 8) * 2, 0);
      }
    };

    int ex = 0;  // exchanges published by this unit
    // O stores issued after the latest copies and not yet waited for: the next
    // two waits (the top of the block and its first key step, or the update
    // pass's first) leave them in flight.
    int pend_st = 0;

    // GroupNorm weight and bias of the unit's columns, kept in LDS (read at
    // each store) rather than in two registers for the whole unit. Written
    // before the first block's barriers; the previous unit ended with one.
    const bool affine = gn.enabled && (gn.weight || gn.bias);
    if (affine && threadIdx.x < kVT) {
      const int col = vt * kVT + threadIdx.x;
      sAff[threadIdx.x] = gn.weight ? gn.weight[h * dv + col] : 1.f;
      sAff[kVT + threadIdx.x] = gn.bias ? gn.bias[h * dv + col] : 0.f;
    }

    // Local statistics of a finished block (rows over this workgroup's 256
    // columns): two passes through LDS (mean, then the sum of squared
    // deviations about it), then publication to the other v tiles.
    auto local_stats = [&](const floatx16 (&acc)[2]) __attribute__((always_inline)) {
      float* s_wmean = sG;                  // [8 waves][64 rows]: row means over the wave's 32 columns
      float* s_wm2 = sGw;                   // [8 waves][64 rows]: sums of squared deviations about them
      float* s_mean = sG + kWavesF * kRowsF;
      float* s_m2 = s_mean + kRowsF;
      const int my_slot = lane & 31;
      const int my_row = (my_slot >> 4) * 32 + acc_row(my_slot & 15, lane);
      {
        float x[32];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int e = 0; e < 16; ++e) x[qt * 16 + e] = acc[qt][e];
        // The wave's own slots: written and read back by this wave only (its
        // LDS operations complete in order), so no barrier.
        s_wmean[wave * kRowsF + my_row] = reduce_scatter32(x, lane) * (1.0f / 32);
      }
      {
        float x[32];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const floatx4 m = *reinterpret_cast<const floatx4*>(s_wmean + wave * kRowsF + qt * 32 + 8 * g +
                                                                4 * (lane >> 5));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float d = acc[qt][4 * g + e] - m[e];
              x[qt * 16 + 4 * g + e] = d * d;
            }
          }
        s_wm2[wave * kRowsF + my_row] = reduce_scatter32(x, lane);
      }
      lds_barrier();
      if (wave == kGnWave) {
        // Row `lane`: the eight waves' (mean, M2) over 32 columns each merged
        // in a fixed order: mean of the means, M2 = sum M2_w + 32 sum (m_w - mean)^2.
        float mw[kWavesF], msum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kWavesF; ++w2) {
          mw[w2] = s_wmean[w2 * kRowsF + lane];
          msum += mw[w2];
        }
        const float mean = msum * (1.0f / kWavesF);
        float m2 = 0.f, dev = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kWavesF; ++w2) {
          m2 += s_wm2[w2 * kRowsF + lane];
          const float d = mw[w2] - mean;
          dev += d * d;
        }
        s_mean[lane] = mean;
        s_m2[lane] = m2 + 32.0f * dev;
      }
      if (a.nvt > 1 && wave == kGnWave) {
        // Publish (mean, M2) of row `lane` into slot ex % 2 as two tagged
        // 64-bit words (each written at once, so a reader that sees the tag
        // sees its value; no ordering between the words is needed).
        uint64_t* slot = mymail + (ex & 1) * kMailWords;
        const uint64_t tag = static_cast<uint64_t>(ex + 1) << 32;
        __hip_atomic_store(slot + 2 * lane, tag | __float_as_uint(s_mean[lane]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(slot + 2 * lane + 1, tag | __float_as_uint(s_m2[lane]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      ++ex;
    };

    float* const s_shift = sG + kWavesF * kRowsF + 2 * kRowsF;
    float* const s_rstd = s_shift + kRowsF;
    // Merge the statistics of all v tiles for exchange e (fixed order, so every
    // v tile computes the same bits) into each row's shift and 1/std in LDS.
    auto gn_merge = [&](int e) __attribute__((always_inline)) {
      float* s_mean = sG + kWavesF * kRowsF;
      float* s_m2 = s_mean + kRowsF;
      if (gn.enabled) {
        if (wave == kGnWave) {
          const int row = lane;
          float mean_v[4], m2_v[4];
          const int nv = a.nvt;
#pragma unroll
          for (int v2 = 0; v2 < 4; ++v2) {
            mean_v[v2] = 0.f;
            m2_v[v2] = 0.f;
            if (v2 >= nv) continue;
            if (v2 == vt) {
              mean_v[v2] = s_mean[row];
              m2_v[v2] = s_m2[row];
              continue;
            }
            // Row `row` of v tile v2's slot e % 2, polled until both words
            // carry tag e + 1 (bounded: after spin_limit polls the values are
            // taken as they are).
            const uint64_t* slot = a.mail + (static_cast<int64_t>(group0 + v2) * 2 + (e & 1)) * kMailWords;
            const uint32_t want = static_cast<uint32_t>(e + 1);
            uint64_t w0, w1;
            int spins = 0;
            for (;;) {
              w0 = __hip_atomic_load(slot + 2 * row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              w1 = __hip_atomic_load(slot + 2 * row + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              const bool ok = static_cast<uint32_t>(w0 >> 32) == want && static_cast<uint32_t>(w1 >> 32) == want;
              if (__builtin_amdgcn_ballot_w64(!ok) == 0 || ++spins > a.spin_limit) break;
              __builtin_amdgcn_s_sleep(1);
            }
            mean_v[v2] = __uint_as_float(static_cast<uint32_t>(w0));
            m2_v[v2] = __uint_as_float(static_cast<uint32_t>(w1));
          }
          float msum = 0.f;
#pragma unroll
          for (int v2 = 0; v2 < 4; ++v2)
            if (v2 < nv) msum += mean_v[v2];
          const float mean = msum / static_cast<float>(nv);
          float m2 = 0.f, dev = 0.f;
#pragma unroll
          for (int v2 = 0; v2 < 4; ++v2) {
            if (v2 >= nv) continue;
            m2 += m2_v[v2];
            const float d = mean_v[v2] - mean;
            dev += d * d;
          }
          m2 += dev * static_cast<float>(kVT);
          const float var = m2 / static_cast<float>(kVT * nv);
          const float rstd = 1.0f / sqrtf(var + gn.eps);
          s_rstd[row] = rstd;
          s_shift[row] = -mean * rstd;
        }
        lds_barrier();
      }
    };
    // Gate values, or the values already in O, at exactly the positions this
    // lane stores (rows past the block's end read as zero).
    // (Recomputed where it is used: an empty asm keeps it from being hoisted
    // into a register held for the whole unit.)
    auto store_offset = [&]() __attribute__((always_inline)) {
      int l = lane;
      asm volatile("" : "+v"(l));
      return ((4 * (l >> 5) + (l & 1)) * dv + vcol0 + ((l & 31) & ~1)) * 2;
    };
    // Reverse order: the lane's row in a group of 8 and its column byte
    // offset (memory row nm1 - (pq0 + row0 + that row)).
    auto rev_store = [&](int& rr, int& cb) __attribute__((always_inline)) {
      int l = lane;
      asm volatile("" : "+v"(l));
      rr = 4 * (l >> 5) + (l & 1);
      cb = (vcol0 + ((l & 31) & ~1)) * 2;
    };
    auto load_epi = [&](uint32_t (&gv)[2][4][2], int pq0, int pqvalid) __attribute__((always_inline)) {
      if constexpr (EPI != 0) {
        const uint16_t* gbase = EPI == 1 ? static_cast<const uint16_t*>(gn.gate) : jo;
        if (!rev) {
          const int so = store_offset();
          const uint16_t* gblk = gbase + (rbase + pq0) * static_cast<int64_t>(dv) + vt * kVT;
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int row0 = qt * 32 + 8 * g;
              const int nrows = min(max(pqvalid - row0, 0), 8);
              const __amdgpu_buffer_rsrc_t r =
                  make_rsrc(gblk + row0 * dv, nrows > 0 ? ((nrows - 1) * dv + kVT) * 2 : 0);
#pragma unroll
              for (int hp = 0; hp < 2; ++hp)
                gv[qt][g][hp] = __builtin_amdgcn_raw_buffer_load_b32(r, so + 2 * hp * dv * 2, 0, 0);
            }
        } else {
          int rr, cb;
          rev_store(rr, cb);
          const __amdgpu_buffer_rsrc_t r = make_rsrc(gbase + mrow * dv + vt * kVT, rev_v_range);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
              for (int hp = 0; hp < 2; ++hp) {
                // Rows past the block's end lie before the head's first row:
                // negative offsets, out of the descriptor's range, read as zero.
                const int row = pq0 + qt * 32 + 8 * g + rr + 2 * hp;
                gv[qt][g][hp] = __builtin_amdgcn_raw_buffer_load_b32(r, (nm1 - row) * dv * 2 + cb, 0, 0);
              }
        }
      }
    };
    // Normalise a block's accumulators (rows pq0.., pqvalid valid) and store
    // them: kOStores stores per lane.
    auto store_block = [&](floatx16 (&opend)[2], const uint32_t (&gv)[2][4][2], int pq0, int pqvalid)
        __attribute__((always_inline)) {
      uint16_t* oblk = rev ? oh : oh + static_cast<int64_t>(pq0) * dv;
      int so, rr = 0, cb = 0;
      if (!rev) so = store_offset();
      else {
        rev_store(rr, cb);
        so = 0;
      }
      // Normalise and store four rows of a lane at a time (rows row0 +
      // 4*(l/32) + 0..3 are accumulators 4g..4g+3): their 1/std and shift are
      // one 16-byte LDS read each. As bf16 pairs: one DPP exchange with the
      // neighbouring lane gives each lane two adjacent columns of one row.
      const bool odd = lane & 1;
      const unsigned sel = odd ? 0x03020706u : 0x05040100u;
      float gw = 1.f, gb = 0.f;
      if (affine) {
        gw = sAff[vcol0 + l32];
        gb = sAff[kVT + vcol0 + l32];
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = qt * 32 + 8 * g;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = opend[qt][4 * g + e];
          if (gn.enabled) {
            const floatx4 rs = *reinterpret_cast<const floatx4*>(s_rstd + row0 + 4 * (lane >> 5));
            const floatx4 sh = *reinterpret_cast<const floatx4*>(s_shift + row0 + 4 * (lane >> 5));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              y[e] = fmaf(y[e], rs[e], sh[e]);
              if (affine) y[e] = fmaf(y[e], gw, gb);
            }
          }
          const int nrows = min(max(pqvalid - row0, 0), 8);
          // Reverse: one descriptor over the head's rows; rows past the
          // block's end get negative offsets and their stores are dropped.
          const __amdgpu_buffer_rsrc_t r =
              rev ? make_rsrc(oblk, rev_v_range)
                  : make_rsrc(oblk + row0 * dv, nrows > 0 ? ((nrows - 1) * dv + kVT) * 2 : 0);
#pragma unroll
          for (int hp = 0; hp < 2; ++hp) {
            const int off = rev ? (nm1 - (pq0 + row0 + rr + 2 * hp)) * dv * 2 + cb : so + 2 * hp * dv * 2;
            unsigned packed;
            if constexpr (EPI != 0) {
              const float a0 = y[2 * hp], a1 = y[2 * hp + 1];
              const float send = odd ? a0 : a1;
              const float recv = __builtin_bit_cast(
                  float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0xB1, 0xf, 0xf, true));
              const float lo = odd ? recv : a0, hi = odd ? a1 : recv;
              const uint32_t gp = gv[qt][g][hp];
              const float g_lo = __uint_as_float(gp << 16), g_hi = __uint_as_float(gp & 0xffff0000u);
              if constexpr (EPI == 1) packed = pack_bf16x2(lo * swish(g_lo), hi * swish(g_hi));
              else packed = pack_bf16x2(lo + g_lo, hi + g_hi);
            } else {
              const unsigned own = pack_bf16x2(y[2 * hp], y[2 * hp + 1]);
              const unsigned nbr = __builtin_amdgcn_update_dpp(0u, own, 0xB1, 0xf, 0xf, true);
              packed = __builtin_amdgcn_perm(nbr, own, sel);
            }
            __builtin_amdgcn_raw_buffer_store_b32(packed, r, off, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- chunks
    int cs = 0;
    if (ncu > 0) {
      // First query block's Q and the first key-step copies of chunk 0.
      copy_q(0);
      copy_k(0, sXK2);
      copy_v(0, sXK0);
      if (min(a.chunk, Nu) > kTileF) copy_k(kTileF, sXK0);
    }
    for (int c = 0; c < ncu; ++c, cs += a.chunk) {
      const int L = min(a.chunk, Nu - cs);
      const int nqb = (L + kRowsF - 1) / kRowsF;
      const bool last_chunk = c + 1 == ncu;
      for (int qb = 0; qb < nqb; ++qb) {
        const int q0 = cs + qb * kRowsF;
        const int qvalid = min(kRowsF, Nu - q0);
        const int kend = min(q0 + kRowsF, Nu);
        const int nkb = (kend - cs + kTileF - 1) / kTileF;  // key blocks up to the diagonal

        floatx16 acc[2];
        acc[0] = floatx16{};
        acc[1] = floatx16{};
        // Q of this block is in sQ once its four copies land; the key steps'
        // first copies (K_0, V_0 and K_1) may stay in flight.
        vm_keep_n(2 + 2 + (nkb > 1 ? 2 : 0) + pend_st);
        lds_barrier();

        // Read-out of R_{c-1}: O = Q R, rows scaled by xi_j = gamma^(j+1).
        // Step j = 2i + s multiplies Q columns 32i + 16s.. by state rows
        // 32i + 16s..; the A operands of step j+1 are read while step j's
        // state operand is formed and multiplied.
        if (c > 0 || has_in) {
          // (Offsets kept from being hoisted out of the block loop, where the
          // 16 of them would hold registers for the whole kernel.)
          // (The lane number formed again here: two registers held across the
          // block loop for these cost spill reloads in the read-out.)
          const int ln = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
          int qx = ln & 14, qg = ((ln >> 5) ^ ln) & 1;
          asm volatile("" : "+v"(qx), "+v"(qg));
          auto ld_qa = [&](int j, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
            const int i = j >> 1, s = j & 1;
            const int gr = (((4 * (i & 3) + 2 * s) ^ qx) | qg) + 16 * (i >> 2);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) dst[qt] = ld8(sQ + qro_row + qt * 32 * kPitch + (gr << 3));
          };
          bf16x8 an[2];
          ld_qa(0, an);
#pragma unroll
          for (int j = 0; j < 2 * MT; ++j) {
            const int i = j >> 1, s = j & 1;
            const bf16x8 a0 = an[0], a1 = an[1];
            if (j + 1 < 2 * MT) ld_qa(j + 1, an);
            // R is constant across the query blocks of a chunk; the empty asm
            // on the elements converted here keeps the conversion in the block
            // loop (hoisted out of it, the packed operands would hold 4
            // registers each for the whole chunk).
#pragma unroll
            for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(R[i][8 * s + e]));
            const bf16x8 b = state_operand(R[i], s);
            acc[0] = mfma32(a0, b, acc[0]);
            acc[1] = mfma32(a1, b, acc[1]);
            __builtin_amdgcn_sched_barrier(0);
          }
          // xi of the lane's rows jb + 32qt + 8b + i (i = 0..3, b = 0..3):
          // gamma^jb, then consecutive rows one factor gamma apart and groups
          // 8 rows apart gamma^5 from the previous group's last row (16
          // rounded products at most, about 1e-6 relative; factors that
          // underflow are below any output's rounding).
          float lgv = lg;
          int jb = q0 - cs + 1 + 4 * (lane >> 5);
          asm volatile("" : "+v"(lgv), "+v"(jb));
          const float fjb = static_cast<float>(jb);
          const float g1 = gpow(lgv, 1.0f), g5 = gpow(lgv, 5.0f);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            float xi = gpow(lgv, fjb + static_cast<float>(32 * qt));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[qt][r] *= xi;
              xi *= (r & 3) == 3 ? g5 : g1;
            }
          }
        }


        // Decay of score (query q, key t): gamma^(q - t) = gamma^(q0 - t0) *
        // gamma^(ql - tl - r): the first factor per key block, the second
        // fixed per lane for the block (q = q0 + ql, t = t0 + tl + r).
        float flane[4];
        {
          const int dl0 = sq * 16 + l16 - (st * 16 + 4 * (lane >> 4));
#pragma unroll
          for (int r = 0; r < 4; ++r) flane[r] = gpow(lg, static_cast<float>(dl0 - r));
        }
        auto score_out = [&](int kb, const floatx4& sacc, uint16_t* pdst) __attribute__((always_inline)) {
          const int dq = q0 - (cs + kb * kTileF);
          const float fblock = gpow(lg, static_cast<float>(dq));
          // sacc[r] = S^T[t][q]: t = st*16 + 4*(lane/16) + r, q = sq*16 + lane%16.
          const int ql = sq * 16 + l16;
          const int tl = st * 16 + 4 * (lane >> 4);
          float x[4];
          if (split_decay) {
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = ql - tl - r >= -dq ? sacc[r] * (fblock * flane[r]) : 0.f;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x[r] = ql - tl - r >= -dq ? sacc[r] * gpow(lg, static_cast<float>(dq + ql - tl - r)) : 0.f;
          }
          uint2 w;
          w.x = pack_bf16x2(x[0], x[1]);
          w.y = pack_bf16x2(x[2], x[3]);
          *reinterpret_cast<uint2*>(pdst + p_off(ql, tl >> 3) + (tl & 7)) = w;
        };
        // Scores of key block kb from the K block in `kset` and Q in sQ (16x16x32, dk/32 steps).
        auto scores = [&](int kb, const uint16_t* kset, uint16_t* pdst) __attribute__((always_inline)) {
          const uint16_t* kt = kset + kTileF * kVT;
          floatx4 sacc = floatx4{};
          // dk/32 steps of 32 columns, four at a time (steps s and s+4 are 128
          // elements apart in the swizzled rows), on two accumulators (even
          // and odd steps) so consecutive MFMAs do not wait for each other.
          floatx4 sodd = floatx4{};
          constexpr int NS = DKMAX / 32;
          bf16x8 kc = ld8(kt + kread[0]), qc = ld8(sQ + qread[0]);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            bf16x8 kn = kc, qn = qc;
            if (s + 1 < NS) {
              kn = ld8(kt + kread[(s + 1) & 3] + 128 * ((s + 1) >> 2));
              qn = ld8(sQ + qread[(s + 1) & 3] + 128 * ((s + 1) >> 2));
            }
            if (s & 1) sodd = mfma16(kc, qc, sodd);
            else sacc = mfma16(kc, qc, sacc);
            kc = kn;
            qc = qn;
            __builtin_amdgcn_sched_barrier(0);
          }
          sacc += sodd;
          score_out(kb, sacc, pdst);
        };

        // Where the next Q block goes: the next query block of this chunk, or
        // the first of the next chunk (the update pass does not read sQ).
        const bool last_qb = qb + 1 == nqb;
        const int next_q = !last_qb ? q0 + kRowsF : (!last_chunk ? cs + a.chunk : -1);

        // Key step i (buffer phase PH = i mod 3): set PH holds V_i and K_{i+1};
        // the scores of block i are in score buffer PH. O += S_i V_i; the scores
        // of block i+1 into score buffer PH+1; copies of V_{i+2}, K_{i+3} into
        // set PH+2 (read at step i-1); wait for all but those; barrier. The
        // last step computes no scores, so sQ is free from its start: the next
        // Q block's copies go out then.
        auto step = [&](int i, auto ph_tag) __attribute__((always_inline)) {
          constexpr int PH = decltype(ph_tag)::value;
          constexpr int PN = (PH + 1) % 3, PF = (PH + 2) % 3;
          uint16_t* xcur = pick<PH>(sXK0, sXK1, sXK2);
          uint16_t* xfar = pick<PF>(sXK0, sXK1, sXK2);
          uint16_t* pcur = pick<PH>(sP0, sP1, sP2);
          uint16_t* pnext = pick<PN>(sP0, sP1, sP2);
          bf16x8 av[2], bv;
          if (i >= 0) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) av[qt] = ld8(pcur + pa[0] + 1024 * qt);
            bv = ld_v(xcur, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          const bool cv = i + 2 < nkb;
          if (cv) copy_v(cs + (i + 2) * kTileF, xfar);
          const bool ck = i + 3 < nkb;
          if (ck) copy_k(cs + (i + 3) * kTileF, xfar);
          const bool cq = i == nkb - 1 && next_q >= 0;
          if (cq) copy_q(next_q);
          __builtin_amdgcn_sched_barrier(0);
          if (i >= 0) {
            acc[0] = mfma32(av[0], bv, acc[0]);
            acc[1] = mfma32(av[1], bv, acc[1]);
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) av[qt] = ld8(pcur + pa[1] + 1024 * qt);
            bv = ld_v(xcur, 1);
            acc[0] = mfma32(av[0], bv, acc[0]);
            acc[1] = mfma32(av[1], bv, acc[1]);
          }
          if (i + 1 < nkb) scores(i + 1, xcur, pnext);
          vm_keep_n((cv ? 2 : 0) + (ck ? 2 : 0) + (cq && wave < 4 ? kQCopies : 0) + (i < 0 ? pend_st : 0));
          lds_barrier();
        };
        using H0 = std::integral_constant<int, 0>;
        using H1 = std::integral_constant<int, 1>;
        using H2 = std::integral_constant<int, 2>;
        // The first scores read K_0, whose pieces every wave copied after this
        // block's Q: wait for it (V_0 and K_1, and the previous block's
        // stores, may stay in flight), then a barrier, so that no wave reads
        // another's piece before it lands. The read-out above hid most of
        // its latency.
        vm_keep_n(2 + (nkb > 1 ? 2 : 0) + pend_st);
        lds_barrier();
        step(-1, H2{});
        pend_st = 0;  // step 0's wait covers them
        for (int i = 0;;) {
          if (i >= nkb) break;
          step(i++, H0{});
          if (i >= nkb) break;
          step(i++, H1{});
          if (i >= nkb) break;
          step(i++, H2{});
        }

        // GroupNorm: this workgroup's row statistics, their exchange with the
        // other v tiles of the head and the merge; then the next key steps'
        // first copies (or, after the chunk's last block, the update pass's
        // first blocks) go out before this block's stores, so the waits for
        // those copies do not wait for the stores as well.
        if (gn.enabled) local_stats(acc);
        const bool do_update = last_qb && !(last_chunk && state_out == nullptr);
        if (!last_qb) {
          copy_k(cs, sXK2);
          copy_v(cs, sXK0);
          if (min(q0 + 2 * kRowsF, Nu) - cs > kTileF) copy_k(cs + kTileF, sXK0);
        } else if (do_update) {
          copy_kx(cs, sXK0);
          copy_v(cs, sXK0);
          if (L > kTileF) {
            copy_kx(cs + kTileF, sXK1);
            copy_v(cs + kTileF, sXK1);
          }
        }
        uint32_t gv[2][4][2];
        load_epi(gv, q0, qvalid);
        gn_merge(ex - 1);
        store_block(acc, gv, q0, qvalid);
        pend_st = kOStores;
      }

      // ---- update pass: R = gamma^L R + sum over the chunk's key blocks of
      // K^T (zeta V), zeta_t = gamma^(L-1-t) (t local). Set j % 3 holds V_j and K_j.
      const bool do_update = !(last_chunk && state_out == nullptr);
      if (do_update) {
        const int nkc = (L + kTileF - 1) / kTileF;
        const float carry = gpow(lg, static_cast<float>(L));
        int ktx[4];
        kt_offsets(ktx);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) R[mt] *= carry;
        // Step j (phase PH = j mod 3): set PH holds V_j and K_j. B = zeta V with
        // zeta_t = gamma^(L-1-t) (t local; rows past the chunk are zero and
        // take 0), A = K^T; copies of block j+2 into set PH+2; wait; barrier.
        auto ustep = [&](int j, auto ph_tag) __attribute__((always_inline)) {
          constexpr int PH = decltype(ph_tag)::value;
          constexpr int PF = (PH + 2) % 3;
          uint16_t* xcur = pick<PH>(sXK0, sXK1, sXK2);
          uint16_t* xfar = pick<PF>(sXK0, sXK1, sXK2);
          const uint16_t* kblk = xcur + kTileF * kVT;
          bf16x8 bz[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const u32x4 u = __builtin_bit_cast(u32x4, ld_v(xcur, s));
            // Element e of the operand is local row tb + e.
            const int e0 = L - 1 - (j * kTileF + 16 * s + 8 * (lane >> 5));
            float ze[8];
            if (split_decay) {
              // gamma^(e0 - e) = gamma^e0 times powers of 1/gamma (at most 2^7).
              const float ginv = gpow(lg, -1.0f);
              float zi = gpow(lg, static_cast<float>(max(e0, 0)));
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                ze[e] = e <= e0 ? zi : 0.f;
                zi *= ginv;
              }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) ze[e] = e <= e0 ? gpow(lg, static_cast<float>(e0 - e)) : 0.f;
            }
            u32x4 z;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              z[e2] = pack_bf16x2(__uint_as_float(u[e2] << 16) * ze[2 * e2],
                                  __uint_as_float(u[e2] & 0xffff0000u) * ze[2 * e2 + 1]);
            bz[s] = __builtin_bit_cast(bf16x8, z);
          }
          __builtin_amdgcn_sched_barrier(0);
          const bool cn = j + 2 < nkc;
          if (cn) {
            copy_kx(cs + (j + 2) * kTileF, xfar);
            copy_v(cs + (j + 2) * kTileF, xfar);
          }
          __builtin_amdgcn_sched_barrier(0);
          bf16x8 c0 = ld_kt(ktx, kblk, 0, 0), c1 = ld_kt(ktx, kblk, 0, 1);
#pragma unroll
          for (int p = 0; p < MT; ++p) {
            const int s = (2 * p) / MT, mt = (2 * p) % MT;
            bf16x8 n0 = c0, n1 = c1;
            if (p + 1 < MT) {
              n0 = ld_kt(ktx, kblk, (2 * p + 2) / MT, (2 * p + 2) % MT);
              n1 = ld_kt(ktx, kblk, (2 * p + 3) / MT, (2 * p + 3) % MT);
            }
            R[mt] = mfma32(c0, bz[s], R[mt]);
            R[mt + 1] = mfma32(c1, bz[s], R[mt + 1]);
            c0 = n0;
            c1 = n1;
            __builtin_amdgcn_sched_barrier(0);
          }
          vm_keep_n((cn ? 4 : 0) + (j == 0 ? pend_st : 0));
          lds_barrier();
        };
        // Block 0 complete; block 1 (and the last block's stores) may stay in flight.
        vm_keep_n((nkc > 1 ? 4 : 0) + pend_st);
        lds_barrier();
        using U0 = std::integral_constant<int, 0>;
        using U1 = std::integral_constant<int, 1>;
        using U2 = std::integral_constant<int, 2>;
        for (int j = 0;;) {
          if (j >= nkc) break;
          ustep(j++, U0{});
          pend_st = 0;
          if (j >= nkc) break;
          ustep(j++, U1{});
          if (j >= nkc) break;
          ustep(j++, U2{});
        }
      }
      if (!last_chunk) {
        // The next chunk's first key-step copies (its first Q block went out
        // during this chunk's last key step).
        const int ncs = cs + a.chunk;
        copy_k(ncs, sXK2);
        copy_v(ncs, sXK0);
        if (min(a.chunk, Nu - ncs) > kTileF) copy_k(ncs + kTileF, sXK0);
      }
    }
    if (state_out) {
      float* obase = state_out + bh * dkdv + vt * kVT;
      wait_vmem();
      __syncthreads();
#pragma unroll
      for (int g4 = 0; g4 < MT; g4 += 4) {
#pragma unroll
        for (int t = 0; t < 4 && g4 + t < MT; ++t) {
          float* f = reinterpret_cast<float*>(stage[t]) + acc_lds;
#pragma unroll
          for (int r = 0; r < 16; ++r) f[(8 * (r >> 2) + (r & 3)) * kVT] = R[g4 + t][r];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4 && g4 + t < MT; ++t) {
          const __amdgpu_buffer_rsrc_t r = make_rsrc(obase + static_cast<int64_t>(32 * (g4 + t)) * dv,
                                                     (31 * dv + kVT) * 4);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int row = 4 * wave + m;
            const u32x4 val = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(stage[t]) + row * kVT +
                                                              4 * lane);
            __builtin_amdgcn_raw_buffer_store_b128(val, r, lane * 16, row * dv * 4, 0);
          }
        }
        __syncthreads();
      }
    }
    // Everything of this unit is done before the buffers take the next one.
    wait_vmem();
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t copy_device(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, stream);
}

hipError_t launch_fused_chunkwise(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                  const float* state_in, float* state_out, void* workspace, const Dims& d, int chunk,
                                  const HeadDecay& decay, const GnArgs& gn, bool accumulate, hipStream_t stream,
                                  int chunks_per_seg, const float* seg_states, const FusedLayout* layout) {
  FusedArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.state_in = state_in;
  a.state_out = state_out;
  const int64_t heads = static_cast<int64_t>(d.B) * d.H;
  const int nchunks = (d.N + chunk - 1) / chunk;
  a.chunks_per_seg = chunks_per_seg > 0 && chunks_per_seg < nchunks ? chunks_per_seg : nchunks;
  a.nseg = (nchunks + a.chunks_per_seg - 1) / a.chunks_per_seg;
  a.seg_states = seg_states;
  if (a.nseg > 1 && !seg_states) return hipErrorInvalidValue;
  const FusedLayout plain;
  const FusedLayout& lay = layout ? *layout : plain;
  const FusedJob* two = lay.second;
  if (a.nseg > 1 && (lay.reverse || two)) return hipErrorInvalidValue;
  if (two && state_out) return hipErrorInvalidValue;  // the second retention leaves no final state
  if (lay.reverse || (two && two->reverse)) {
    // Reverse order addresses a head's rows from one descriptor with 32-bit
    // offsets; rows past the end must come out beyond its range.
    const int64_t widest = std::max<int64_t>({lay.ldq > 0 ? lay.ldq : d.dk, lay.ldk > 0 ? lay.ldk : d.dk, d.dv});
    if ((static_cast<int64_t>(d.N) - 1) * widest * 2 + widest * 2 >= (int64_t{1} << 30)) return hipErrorInvalidValue;
  }
  a.ldq = lay.ldq > 0 ? lay.ldq : d.dk;
  a.ldk = lay.ldk > 0 ? lay.ldk : d.dk;
  a.reverse = lay.reverse ? 1 : 0;
  a.q2 = two ? two->q : nullptr;
  a.k2 = two ? two->k : nullptr;
  a.v2 = two ? two->v : nullptr;
  a.o2 = two ? two->o : nullptr;
  a.state_in2 = two ? two->state_in : nullptr;
  a.reverse2 = two && two->reverse ? 1 : 0;
  a.nvt = d.dv / kVT;
  a.job_units = static_cast<int>(heads * a.nseg * a.nvt);
  a.units = a.job_units * (two ? 2 : 1);
  a.mail = static_cast<uint64_t*>(workspace);
  a.H = d.H;
  a.N = d.N;
  a.dk = d.dk;
  a.dv = d.dv;
  a.chunk = chunk;
  a.nchunks = (d.N + chunk - 1) / chunk;
  a.spin_limit = 1 << 22;
  // The exchange words are read only by the GroupNorm exchange between the v
  // tiles of a head; a call without it leaves them untouched.
  hipError_t e = hipSuccess;
  if (gn.enabled && a.nvt > 1) {
    const int mail_ints = a.units * 2 * kMailWords * 2;
    zero_ints_kernel<<<dim3((mail_ints + 255) / 256), 256, 0, stream>>>(reinterpret_cast<int*>(a.mail), mail_ints);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  const int epi = (gn.enabled && gn.gate) ? 1 : (accumulate ? 2 : 0);
  const void* fn = nullptr;
  const bool gen = layout != nullptr;
  if (gen && epi == 1) return hipErrorInvalidValue;  // the general layout has no gated instance
#define RET_FUSED_PICK(MTV)                                                                            \
  fn = gen          ? (epi == 2 ? reinterpret_cast<const void*>(fused_chunk_kernel<MTV, 2, true>)      \
                                : reinterpret_cast<const void*>(fused_chunk_kernel<MTV, 0, true>))     \
       : epi == 1   ? reinterpret_cast<const void*>(fused_chunk_kernel<MTV, 1, false>)                 \
       : epi == 2   ? reinterpret_cast<const void*>(fused_chunk_kernel<MTV, 2, false>)                 \
                    : reinterpret_cast<const void*>(fused_chunk_kernel<MTV, 0, false>)
  if (d.dk == 256) {
    RET_FUSED_PICK(8);
  } else {
    RET_FUSED_PICK(4);
  }
#undef RET_FUSED_PICK
  int slot = (d.dk == 256 ? 9 : 10) + (gen ? 3 : 0);  // 12, 13: the general-layout instances
  int resident = 0;
  e = resident_workgroups(fn, kThreadsF, slot, &resident);
  if (e != hipSuccess) return e;
  int G = std::min(a.units, resident);
  G -= G % a.nvt;  // the v tiles of a head run in the same round
  if (G <= 0) return hipErrorInvalidConfiguration;
  HeadDecay dc = decay;
  GnArgs g = gn;
  void* args[] = {&a, &dc, &g};
  // Only the GroupNorm exchange needs the v tiles of a head resident together.
  if (a.nvt > 1 && gn.enabled) {
    e = hipLaunchCooperativeKernel(fn, dim3(G), dim3(kThreadsF), args, 0, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
  }
  e = hipLaunchKernel(fn, dim3(G), dim3(kThreadsF), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace ret

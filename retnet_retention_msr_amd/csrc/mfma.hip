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
//    walks the chunks in order. Before each chunk it stores R as bf16 in a
//    [v][k] layout (k fastest), which is exactly the B-operand layout of the
//    read-out; then it applies the carry and accumulates K^T (zeta V) with K
//    and zeta*V staged transposed in LDS. Long sequences with few heads are cut
//    into chunk-aligned segments: a first launch computes each segment's local
//    end state from zero, the second starts every segment from the sum of the
//    earlier segments' end states, each decayed to its start.
//  * output: one workgroup per (head, 64-row query block) with the full dv row.
//    It reads out the stored chunk state, then loops over the 64-row key
//    blocks of its chunk up to the diagonal: S^T = K Q^T on the MFMAs, the
//    decay gamma^(n-m) (zero above the diagonal) applied to the fp32 scores
//    in registers, scores rounded to bf16 into LDS, then O += A V. The per-head
//    GroupNorm and the bf16 store close it. The N x N mask never exists in
//    memory; with one chunk spanning the sequence this is the parallel form.
//
// MFMA 32x32x16 operand layouts used throughout (lane l of 64):
//   A[i][kk]: i = l % 32, kk = 8*(l/32) + 0..7   (16 contiguous bytes)
//   B[kk][j]: j = l % 32, kk = 8*(l/32) + 0..7
//   D[i][j] : j = l % 32, i = 8*(r/4) + 4*(l/32) + r%4 for accumulator r = 0..15
#include "kernels.h"

namespace ret {

namespace {

constexpr int kThreads = 256;  // four waves
constexpr int kRows = 64;      // query / key block height
constexpr int kPitchT = 72;    // LDS pitch (elements) of transposed tiles: 64 + 8 pad
constexpr int kPitchQK = 264;  // LDS pitch of row-major Q/K tiles: 256 + 8 pad

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Row-major copy of `nvalid` rows (of 64) x `ncols` columns into LDS [t][c]
// with pitch P; rows past nvalid are zero.
template <int P>
__device__ __forceinline__ void stage_rows(uint16_t* dst, const uint16_t* src, int64_t stride, int nvalid,
                                           int ncols) {
  const int octets = ncols >> 3;
  for (int i = threadIdx.x; i < kRows * octets; i += kThreads) {
    const int t = i / octets, co = i - t * octets;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (t < nvalid) val = *reinterpret_cast<const uint4*>(src + t * stride + co * 8);
    *reinterpret_cast<uint4*>(dst + t * P + co * 8) = val;
  }
}

// Transposed copy: dst[c][t] = src[t][c] (times row_scale(t) when kScale),
// 4 rows x 8 columns per work item: four 16-byte loads, eight 8-byte LDS stores.
template <bool kScale>
__device__ __forceinline__ void stage_transposed(uint16_t* dst, const uint16_t* src, int64_t stride, int nvalid,
                                                 int ncols, float scale_log2g, int scale_last) {
  const int octets = ncols >> 3;
  for (int i = threadIdx.x; i < (kRows / 4) * octets; i += kThreads) {
    const int tq = i / octets, co = i - tq * octets;
    uint16_t x[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * tq + j;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (t < nvalid) val = *reinterpret_cast<const uint4*>(src + t * stride + co * 8);
      const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[j][2 * e] = static_cast<uint16_t>(w[e] & 0xffffu);
        x[j][2 * e + 1] = static_cast<uint16_t>(w[e] >> 16);
      }
      if (kScale) {
        // zeta_t = gamma^(L-1-t) for the chunk-local row t
        const float z = (t < nvalid) ? exp2f(static_cast<float>(scale_last - t) * scale_log2g) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = f32_to_bf16(bf16_to_f32(x[j][e]) * z);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint2 w;
      w.x = static_cast<uint32_t>(x[0][e]) | (static_cast<uint32_t>(x[1][e]) << 16);
      w.y = static_cast<uint32_t>(x[2][e]) | (static_cast<uint32_t>(x[3][e]) << 16);
      *reinterpret_cast<uint2*>(dst + (co * 8 + e) * kPitchT + 4 * tq) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// State walk
// ---------------------------------------------------------------------------
constexpr int kWalkVT = 128;  // v columns per workgroup: 32 per wave

struct WalkArgs {
  const uint16_t* k;
  const uint16_t* v;
  const float* state_in;
  float* state_out;
  uint16_t* chunk_states;  // [B*H][nchunks][dv][dk]
  float* seg_states;       // [B*H][nseg][dk][dv]
  int H, N, dk, dv, chunk, nchunks, nseg, chunks_per_seg;
  int nkt, nvt;
  int mode;  // 0: local end state of segments 0..nseg-2; 1: write chunk states from the true start
};

template <int MT>
__global__ void __launch_bounds__(kThreads) mfma_state_walk_kernel(WalkArgs a, HeadDecay decay) {
  constexpr int KT = 32 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t sKt[KT * kPitchT];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[kWalkVT * kPitchT];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int idx = blockIdx.x;
  const int vt = idx % a.nvt;
  idx /= a.nvt;
  const int kt = idx % a.nkt;
  idx /= a.nkt;
  const int nseg_launch = (a.mode == 0) ? a.nseg - 1 : a.nseg;
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
      const float f = exp2f(static_cast<float>(p - end_s) * lg);
      const float* U = a.seg_states + (bh * a.nseg + s) * dkdv;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[mt][r] = fmaf(f, U[static_cast<int64_t>(k0 + mt * 32 + acc_row(r, lane)) * a.dv + vcol], acc[mt][r]);
    }
  }

  const uint16_t* kb = a.k + bh * static_cast<int64_t>(a.N) * a.dk;
  const uint16_t* vb = a.v + bh * static_cast<int64_t>(a.N) * a.dv;

  for (int c = c_begin; c < c_end; ++c) {
    const int cs = c * a.chunk;
    const int L = min(a.chunk, a.N - cs);
    if (a.mode == 1) {
      // Store R_{c-1} as bf16 in [v][k] layout: 4 consecutive k per 8-byte store.
      uint16_t* dst = a.chunk_states + ((bh * a.nchunks + c) * a.dv + vcol) * static_cast<int64_t>(a.dk) + k0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 w;
          w.x = pack_bf16x2(acc[mt][4 * g + 0], acc[mt][4 * g + 1]);
          w.y = pack_bf16x2(acc[mt][4 * g + 2], acc[mt][4 * g + 3]);
          *reinterpret_cast<uint2*>(dst + mt * 32 + 8 * g + 4 * (lane >> 5)) = w;
        }
    }
    const float carry = exp2f(static_cast<float>(L) * lg);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] *= carry;

    for (int t0 = 0; t0 < L; t0 += kRows) {
      const int nvalid = min(kRows, L - t0);
      __syncthreads();
      stage_transposed<false>(sKt, kb + static_cast<int64_t>(cs + t0) * a.dk + k0, a.dk, nvalid, KT, 0.f, 0);
      stage_transposed<true>(sVt, vb + static_cast<int64_t>(cs + t0) * a.dv + v0, a.dv, nvalid, kWalkVT, lg,
                             L - 1 - t0);
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kRows / 16; ++s) {
        const bf16x8 b = ld8(sVt + (wave * 32 + (lane & 31)) * kPitchT + s * 16 + 8 * (lane >> 5));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 av = ld8(sKt + (mt * 32 + (lane & 31)) * kPitchT + s * 16 + 8 * (lane >> 5));
          acc[mt] = mfma32(av, b, acc[mt]);
        }
      }
    }
  }

  // Mode 0 stores the segment's end state. Mode 1 stores the final state: to
  // state_out when there is one segment, else into the spare last segment slot
  // (the host copies it to state_out afterwards, so state_out may alias
  // state_in while other segments still read it).
  float* out = nullptr;
  if (a.mode == 0) out = a.seg_states + (bh * a.nseg + seg) * dkdv;
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
// Output
// ---------------------------------------------------------------------------
struct OutArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* chunk_states;  // [B*H][nchunks][dv][dk] or null
  uint16_t* o;
  int state_for_chunk0;
  int H, N, dk, dv, chunk, nchunks, nqb;
};

template <int NT>
__global__ void __launch_bounds__(kThreads) mfma_chunk_out_kernel(OutArgs a, HeadDecay decay, GnArgs gn) {
  constexpr int DV = 128 * NT;   // dv handled by the workgroup
  constexpr int WV = 32 * NT;    // columns per wave
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kRows * kPitchQK];
  __shared__ __attribute__((aligned(16))) uint16_t sK[kRows * kPitchQK];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[DV * kPitchT];
  __shared__ __attribute__((aligned(16))) uint16_t sA[kRows * kPitchT];
  __shared__ float s_stat[4][kRows];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 31;
  const int lk = 8 * (lane >> 5);
  const int64_t bh = blockIdx.x / a.nqb;
  const int qb = blockIdx.x % a.nqb;
  const int h = static_cast<int>(bh % a.H);
  const float lg = decay.log2g[h];
  const int q0 = qb * kRows;
  const int c = q0 / a.chunk;
  const int cs = c * a.chunk;
  const int dk = a.dk;
  const uint16_t* qbase = a.q + bh * static_cast<int64_t>(a.N) * dk;
  const uint16_t* kbase = a.k + bh * static_cast<int64_t>(a.N) * dk;
  const uint16_t* vbase = a.v + bh * static_cast<int64_t>(a.N) * DV;

  stage_rows<kPitchQK>(sQ, qbase + static_cast<int64_t>(q0) * dk, dk, min(kRows, a.N - q0), dk);
  __syncthreads();

  floatx16 acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx16{};

  // Cross-chunk read-out: O = diag(gamma^(j+1)) Q R_{c-1}, R read as bf16 B operands.
  if (a.chunk_states && (c > 0 || a.state_for_chunk0)) {
    const uint16_t* Rt = a.chunk_states + (bh * a.nchunks + c) * static_cast<int64_t>(DV) * dk;
    for (int s = 0; s < dk / 16; ++s) {
      const bf16x8 a0 = ld8(sQ + lrow * kPitchQK + s * 16 + lk);
      const bf16x8 a1 = ld8(sQ + (32 + lrow) * kPitchQK + s * 16 + lk);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int vcol = wave * WV + nt * 32 + lrow;
        const bf16x8 b = ld8(Rt + static_cast<int64_t>(vcol) * dk + s * 16 + lk);
        acc[0][nt] = mfma32(a0, b, acc[0][nt]);
        acc[1][nt] = mfma32(a1, b, acc[1][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = q0 + mt * 32 + acc_row(r, lane) - cs;  // chunk-local row
        const float xi = exp2f(static_cast<float>(j + 1) * lg);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt][r] *= xi;
      }
  }

  // Intra-chunk causal part over key blocks cs/64 .. qb.
  const int tt = wave >> 1, qt = wave & 1;  // this wave's 32x32 tile of S^T
  for (int tb = cs / kRows; tb <= qb; ++tb) {
    const int t0 = tb * kRows;
    const int nvalid = min(kRows, a.N - t0);
    __syncthreads();
    stage_rows<kPitchQK>(sK, kbase + static_cast<int64_t>(t0) * dk, dk, nvalid, dk);
    stage_transposed<false>(sVt, vbase + static_cast<int64_t>(t0) * DV, DV, nvalid, DV, 0.f, 0);
    __syncthreads();

    floatx16 sacc = floatx16{};
    for (int s = 0; s < dk / 16; ++s) {
      const bf16x8 ak = ld8(sK + (tt * 32 + lrow) * kPitchQK + s * 16 + lk);
      const bf16x8 bq = ld8(sQ + (qt * 32 + lrow) * kPitchQK + s * 16 + lk);
      sacc = mfma32(ak, bq, sacc);
    }
    // sacc[r] = S^T[t][q], t = tt*32 + acc_row(r), q = qt*32 + lrow. Apply gamma^(q-t), zero if t > q.
    const int qa = q0 + qt * 32 + lrow;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + tt * 32 + 8 * g + 4 * (lane >> 5) + e;
        const int d = qa - t;
        x[e] = (d >= 0) ? sacc[4 * g + e] * exp2f(static_cast<float>(d) * lg) : 0.f;
      }
      uint2 w;
      w.x = pack_bf16x2(x[0], x[1]);
      w.y = pack_bf16x2(x[2], x[3]);
      *reinterpret_cast<uint2*>(sA + (qt * 32 + lrow) * kPitchT + tt * 32 + 8 * g + 4 * (lane >> 5)) = w;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kRows / 16; ++s) {
      const bf16x8 a0 = ld8(sA + lrow * kPitchT + s * 16 + lk);
      const bf16x8 a1 = ld8(sA + (32 + lrow) * kPitchT + s * 16 + lk);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 b = ld8(sVt + (wave * WV + nt * 32 + lrow) * kPitchT + s * 16 + lk);
        acc[0][nt] = mfma32(a0, b, acc[0][nt]);
        acc[1][nt] = mfma32(a1, b, acc[1][nt]);
      }
    }
  }

  // Epilogue: optional per-head GroupNorm over the DV columns of each row, then bf16 store.
  if (gn.enabled) {
    float mean[2][16], rstd[2][16];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      float part[2][16];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float d = pass == 0 ? acc[mt][nt][r] : acc[mt][nt][r] - mean[mt][r];
            s += pass == 0 ? d : d * d;
          }
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) s += __shfl_xor(s, off, 64);
          part[mt][r] = s;
        }
      __syncthreads();
      if (lrow == 0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s_stat[wave][mt * 32 + acc_row(r, lane)] = part[mt][r];
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mt * 32 + acc_row(r, lane);
          const float tot = (s_stat[0][row] + s_stat[1][row] + s_stat[2][row] + s_stat[3][row]) / DV;
          if (pass == 0) mean[mt][r] = tot;
          else rstd[mt][r] = 1.0f / sqrtf(tot + gn.eps);
        }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int vcol = wave * WV + nt * 32 + lrow;
      const float w = gn.weight ? gn.weight[h * DV + vcol] : 1.f;
      const float bb = gn.bias ? gn.bias[h * DV + vcol] : 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mt][nt][r] = (acc[mt][nt][r] - mean[mt][r]) * rstd[mt][r] * w + bb;
    }
  }

  uint16_t* obase = a.o + (bh * a.N + q0) * static_cast<int64_t>(DV);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mt * 32 + acc_row(r, lane);
      if (q0 + row < a.N) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int vcol = wave * WV + nt * 32 + lrow;
          obase[static_cast<int64_t>(row) * DV + vcol] = f32_to_bf16(acc[mt][nt][r]);
        }
      }
    }
}

}  // namespace

bool mfma_supports(int dk, int dv) {
  return dk % 32 == 0 && dk >= 32 && dk <= 256 && (dv == 128 || dv == 256 || dv == 512);
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
  const int MT = walk_k_tiles(d.dk);
  a.nkt = d.dk / (32 * MT);
  a.nvt = d.dv / kWalkVT;
  const int64_t per_seg = static_cast<int64_t>(d.B) * d.H * a.nkt * a.nvt;
  for (int mode = (a.nseg > 1 ? 0 : 1); mode <= 1; ++mode) {
    a.mode = mode;
    const int64_t nblocks = per_seg * (mode == 0 ? a.nseg - 1 : a.nseg);
    const dim3 grid(static_cast<unsigned>(nblocks));
    if (MT == 4) mfma_state_walk_kernel<4><<<grid, kThreads, 0, stream>>>(a, decay);
    else if (MT == 2) mfma_state_walk_kernel<2><<<grid, kThreads, 0, stream>>>(a, decay);
    else mfma_state_walk_kernel<1><<<grid, kThreads, 0, stream>>>(a, decay);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.nseg > 1 && state_out) {
    // Final state sits in segment slot nseg-1 of every head: copy it out.
    const int64_t dkdv = static_cast<int64_t>(d.dk) * d.dv;
    for (int64_t bh = 0; bh < static_cast<int64_t>(d.B) * d.H; ++bh) {
      const hipError_t e = hipMemcpyAsync(state_out + bh * dkdv, seg_states + (bh * a.nseg + a.nseg - 1) * dkdv,
                                          dkdv * sizeof(float), hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

int walk_k_tiles(int dk) { return (dk % 128 == 0) ? 4 : ((dk % 64 == 0) ? 2 : 1); }

int walk_tiles_per_head(int dk, int dv) { return (dk / (32 * walk_k_tiles(dk))) * (dv / kWalkVT); }

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
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(d.B) * d.H * a.nqb));
  switch (d.dv) {
    case 128: mfma_chunk_out_kernel<1><<<grid, kThreads, 0, stream>>>(a, decay, gn); break;
    case 256: mfma_chunk_out_kernel<2><<<grid, kThreads, 0, stream>>>(a, decay, gn); break;
    default: mfma_chunk_out_kernel<4><<<grid, kThreads, 0, stream>>>(a, decay, gn); break;
  }
  return hipGetLastError();
}

}  // namespace ret

// Generic retention kernels on the vector ALUs, for any element type.
//
// They compute in fp32 and serve fp32 inputs, and bf16 inputs whose sizes the
// MFMA kernels do not cover. They follow "RetNet - Retentive Network - A
// Successor to Transformer for LLMs", Key Equations (parallel and chunkwise
// recurrent forms) and Key components, 1. Retention (the chunk-state carry):
//
//   state walk:  R_i = gamma^L R_{i-1} + sum_j zeta_j k_j^T v_j ,
//                zeta_j = gamma^(L-1-j), j the row inside chunk i of length L;
//                the state before every chunk is written out for the read-out.
//   output row:  o_n = sum_{m in chunk(n), m <= n} gamma^(n-m) (q_n . k_m) v_m
//                      + gamma^(j+1) q_n R_{i-1}          (j = n - chunk start)
//
// With one chunk spanning the sequence and no state the output kernel is the
// parallel form. These kernels favour simplicity over speed.
#include "common.h"
#include "kernels.h"

namespace ret {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// State walk. Grid: (B*H, ceil(dv/64)). Thread (rg, col) with col = tid % 64,
// rg = tid / 64 owns state column v0 + col and rows rg, rg+4, ..., in registers.
// ---------------------------------------------------------------------------
constexpr int kWalkCols = 64;
constexpr int kWalkRowsPerThread = 64;  // dk <= 256
constexpr int kWalkTB = 16;             // rows of K/V staged per step

template <typename T>
__global__ void __launch_bounds__(kThreads)
generic_state_walk_kernel(const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ state_in,
                          float* __restrict__ state_out, float* __restrict__ chunk_states, int H, int N, int dk,
                          int dv, int chunk, int nchunks, HeadDecay decay) {
  __shared__ float s_k[kWalkTB][256];
  __shared__ float s_v[kWalkTB][kWalkCols];

  const int tid = threadIdx.x;
  const int col = tid & (kWalkCols - 1);
  const int rg = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const float lg = decay.log2g[h];
  const int vcol = blockIdx.y * kWalkCols + col;
  const bool col_ok = vcol < dv;

  float R[kWalkRowsPerThread];
#pragma unroll
  for (int i = 0; i < kWalkRowsPerThread; ++i) {
    const int r = rg + 4 * i;
    R[i] = (state_in && col_ok && r < dk) ? state_in[(bh * dk + r) * dv + vcol] : 0.f;
  }

  const T* kb = k + bh * static_cast<int64_t>(N) * dk;
  const T* vb = v + bh * static_cast<int64_t>(N) * dv;

  for (int c = 0; c < nchunks; ++c) {
    const int cs = c * chunk;
    const int L = min(chunk, N - cs);
    if (chunk_states) {
      float* dst = chunk_states + ((bh * nchunks + c) * dk) * static_cast<int64_t>(dv);
#pragma unroll
      for (int i = 0; i < kWalkRowsPerThread; ++i) {
        const int r = rg + 4 * i;
        if (col_ok && r < dk) dst[static_cast<int64_t>(r) * dv + vcol] = R[i];
      }
    }
    const float carry = decay_pow(lg, static_cast<float>(L));
#pragma unroll
    for (int i = 0; i < kWalkRowsPerThread; ++i) R[i] *= carry;

    for (int t0 = 0; t0 < L; t0 += kWalkTB) {
      __syncthreads();
      for (int e = tid; e < kWalkTB * dk; e += kThreads) {
        const int tt = e / dk, kk = e % dk;
        const int t = t0 + tt;
        s_k[tt][kk] = (t < L) ? Elem<T>::load(kb, static_cast<int64_t>(cs + t) * dk + kk) : 0.f;
      }
      for (int e = tid; e < kWalkTB * kWalkCols; e += kThreads) {
        const int tt = e / kWalkCols, cc = e % kWalkCols;
        const int t = t0 + tt;
        const int vc = blockIdx.y * kWalkCols + cc;
        float x = 0.f;
        if (t < L && vc < dv) {
          x = Elem<T>::load(vb, static_cast<int64_t>(cs + t) * dv + vc) *
              decay_pow(lg, static_cast<float>(L - 1 - t));
        }
        s_v[tt][cc] = x;
      }
      __syncthreads();
#pragma unroll 4
      for (int tt = 0; tt < kWalkTB; ++tt) {
        const float vz = s_v[tt][col];
#pragma unroll
        for (int i = 0; i < kWalkRowsPerThread; ++i) {
          const int r = rg + 4 * i;
          if (r < dk) R[i] = fmaf(s_k[tt][r], vz, R[i]);
        }
      }
    }
  }
  if (state_out) {
#pragma unroll
    for (int i = 0; i < kWalkRowsPerThread; ++i) {
      const int r = rg + 4 * i;
      if (col_ok && r < dk) state_out[(bh * dk + r) * dv + vcol] = R[i];
    }
  }
}

// ---------------------------------------------------------------------------
// Output rows. Grid: B*H*N blocks, block = (b*H + h)*N + n. Thread tid owns columns tid + 256*j (dv <= 1024).
// ---------------------------------------------------------------------------
constexpr int kOutColsPerThread = 4;

template <typename T>
__global__ void __launch_bounds__(kThreads)
generic_chunk_out_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                         const float* __restrict__ chunk_states, int state_for_chunk0, T* __restrict__ o, int H,
                         int N, int dk, int dv, int chunk, int nchunks, HeadDecay decay, GnArgs gn,
                         int accumulate) {
  __shared__ float s_q[256];
  __shared__ float s_w[kThreads];
  __shared__ float s_red[4];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x / N;
  const int n = static_cast<int>(blockIdx.x % N);
  const int h = static_cast<int>(bh % H);
  const float lg = decay.log2g[h];
  const int c = n / chunk;
  const int cs = c * chunk;

  for (int i = tid; i < dk; i += kThreads) s_q[i] = Elem<T>::load(q, (bh * N + n) * dk + i);
  __syncthreads();

  float acc[kOutColsPerThread];
#pragma unroll
  for (int j = 0; j < kOutColsPerThread; ++j) acc[j] = 0.f;

  // Cross-chunk read-out of the state in force before this chunk.
  if (chunk_states && (c > 0 || state_for_chunk0)) {
    const float* R = chunk_states + ((bh * nchunks + c) * dk) * static_cast<int64_t>(dv);
    for (int r = 0; r < dk; ++r) {
      const float qr = s_q[r];
#pragma unroll
      for (int j = 0; j < kOutColsPerThread; ++j) {
        const int col = tid + kThreads * j;
        if (col < dv) acc[j] = fmaf(qr, R[static_cast<int64_t>(r) * dv + col], acc[j]);
      }
    }
    const float xi = decay_pow(lg, static_cast<float>(n - cs + 1));
#pragma unroll
    for (int j = 0; j < kOutColsPerThread; ++j) acc[j] *= xi;
  }

  // Intra-chunk causal part, 256 key rows at a time.
  const T* kb = k + bh * static_cast<int64_t>(N) * dk;
  const T* vb = v + bh * static_cast<int64_t>(N) * dv;
  for (int m0 = cs; m0 <= n; m0 += kThreads) {
    const int m = m0 + tid;
    float w = 0.f;
    if (m <= n) {
      float s = 0.f;
      for (int r = 0; r < dk; ++r) s = fmaf(s_q[r], Elem<T>::load(kb, static_cast<int64_t>(m) * dk + r), s);
      w = s * decay_pow(lg, static_cast<float>(n - m));
    }
    __syncthreads();
    s_w[tid] = w;
    __syncthreads();
    const int cnt = min(kThreads, n - m0 + 1);
    for (int mm = 0; mm < cnt; ++mm) {
      const float wm = s_w[mm];
      const int64_t row = static_cast<int64_t>(m0 + mm) * dv;
#pragma unroll
      for (int j = 0; j < kOutColsPerThread; ++j) {
        const int col = tid + kThreads * j;
        if (col < dv) acc[j] = fmaf(wm, Elem<T>::load(vb, row + col), acc[j]);
      }
    }
  }

  if (gn.enabled) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < kOutColsPerThread; ++j)
      if (tid + kThreads * j < dv) part += acc[j];
    const float mean = block_sum_256(part, s_red) / dv;
    __syncthreads();
    part = 0.f;
#pragma unroll
    for (int j = 0; j < kOutColsPerThread; ++j) {
      if (tid + kThreads * j < dv) {
        const float d = acc[j] - mean;
        part += d * d;
      }
    }
    const float var = block_sum_256(part, s_red) / dv;
    const float rstd = 1.0f / sqrtf(var + gn.eps);
#pragma unroll
    for (int j = 0; j < kOutColsPerThread; ++j) {
      const int col = tid + kThreads * j;
      float y = (acc[j] - mean) * rstd;
      if (gn.weight && col < dv) y *= gn.weight[h * dv + col];
      if (gn.bias && col < dv) y += gn.bias[h * dv + col];
      if (gn.gate && col < dv) y *= swish(Elem<T>::load(static_cast<const T*>(gn.gate), (bh * N + n) * dv + col));
      acc[j] = y;
    }
  }
#pragma unroll
  for (int j = 0; j < kOutColsPerThread; ++j) {
    const int col = tid + kThreads * j;
    if (col < dv) {
      const int64_t at = (bh * N + n) * dv + col;
      Elem<T>::store(o, at, accumulate ? acc[j] + Elem<T>::load(o, at) : acc[j]);
    }
  }
}

}  // namespace

hipError_t launch_generic_state_walk(int dtype, const void* k, const void* v, const float* state_in,
                                     float* state_out, float* chunk_states, const Dims& d, int chunk,
                                     const HeadDecay& decay, hipStream_t stream) {
  const int nchunks = (d.N + chunk - 1) / chunk;
  const dim3 grid(d.B * d.H, (d.dv + kWalkCols - 1) / kWalkCols);
  if (dtype == 0) {
    generic_state_walk_kernel<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(k), static_cast<const float*>(v), state_in, state_out, chunk_states, d.H, d.N,
        d.dk, d.dv, chunk, nchunks, decay);
  } else {
    generic_state_walk_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), state_in, state_out, chunk_states, d.H,
        d.N, d.dk, d.dv, chunk, nchunks, decay);
  }
  return hipGetLastError();
}

hipError_t launch_generic_chunk_out(int dtype, const void* q, const void* k, const void* v,
                                    const float* chunk_states, bool state_for_chunk0, void* o, const Dims& d,
                                    int chunk, const HeadDecay& decay, const GnArgs& gn, bool accumulate,
                                    hipStream_t stream) {
  const int nchunks = (d.N + chunk - 1) / chunk;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(d.B) * d.H * d.N));
  const int acc = accumulate ? 1 : 0;
  if (dtype == 0) {
    generic_chunk_out_kernel<float><<<grid, kThreads, 0, stream>>>(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), chunk_states,
        state_for_chunk0 ? 1 : 0, static_cast<float*>(o), d.H, d.N, d.dk, d.dv, chunk, nchunks, decay, gn, acc);
  } else {
    generic_chunk_out_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        chunk_states, state_for_chunk0 ? 1 : 0, static_cast<uint16_t*>(o), d.H, d.N, d.dk, d.dv, chunk, nchunks,
        decay, gn, acc);
  }
  return hipGetLastError();
}

}  // namespace ret

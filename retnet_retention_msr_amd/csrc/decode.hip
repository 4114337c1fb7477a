// Recurrent decode step of retention ("RetNet - Retentive Network - A
// Successor to Transformer for LLMs", Key Equations, recurrent form):
//   S <- gamma * S + k^T v      (dk x dv outer product, fp32 state, in place)
//   o  = q . S                  (read-out after the update)
// followed by the optional per-head GroupNorm over the dv outputs.
//
// The step moves 8 bytes of state per 4 flops, so it is bound by HBM. Each
// workgroup streams a [dk x 64] column slab of one head's state: a wave covers
// 4 rows x 64 columns per iteration with 16-byte loads and stores (256
// contiguous bytes per row), keeps 4 column partial sums of q . S per lane, and
// the 16 row groups are reduced through LDS at the end. With GroupNorm the
// workgroup walks all column slabs of its head so it sees the whole row.
#include "common.h"
#include "kernels.h"

namespace ret {

namespace {

constexpr int kThreads = 256;
constexpr int kColsPerTile = 64;  // 16 column groups of 4 floats
constexpr int kRowGroups = 16;

// The NR state rows r = ry, ry + 16, ... of one 4-column group: all NR
// 16-byte loads are issued before the first update is written back (about 8%
// faster at B=32 than loading and storing row by row, which keeps fewer bytes
// in flight), then S <- gamma S + k_r v and acc += q_r S.
template <int NR>
__device__ __forceinline__ void update_rows(float* S, int dv, int c0, int ry, float g, const float* s_k,
                                            const float* s_q, const float (&vv)[4], float (&acc)[4]) {
  floatx4* p = reinterpret_cast<floatx4*>(S + static_cast<int64_t>(ry) * dv + c0);
  const int64_t step = static_cast<int64_t>(kRowGroups) * dv / 4;
  floatx4 sv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) sv[i] = p[i * step];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = ry + kRowGroups * i;
    const float kr = s_k[r], qr = s_q[r];
    floatx4 x = sv[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = fmaf(g, x[j], kr * vv[j]);
    p[i * step] = x;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(qr, x[j], acc[j]);
  }
}

template <typename T, bool kFullRow, bool kVec4>
__global__ void __launch_bounds__(kThreads)
decode_step_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   float* __restrict__ state, T* __restrict__ o, int H, int dk, int dv,
                   HeadDecay decay, GnArgs gn) {
  __shared__ float s_q[256];
  __shared__ float s_k[256];
  __shared__ float s_part[kRowGroups][kColsPerTile + 1];
  __shared__ float s_row[kFullRow ? 1024 : 1];
  __shared__ float s_red[4];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int h = static_cast<int>(bh % H);
  const float g = exp2f(decay.log2g[h]);

  for (int i = tid; i < dk; i += kThreads) {
    s_q[i] = Elem<T>::load(q, bh * dk + i);
    s_k[i] = Elem<T>::load(k, bh * dk + i);
  }
  __syncthreads();

  const int cx = tid & 15;   // column group: 4 consecutive columns
  const int ry = tid >> 4;   // row group: rows ry, ry+16, ...
  float* S = state + bh * static_cast<int64_t>(dk) * dv;
  const int ntiles = (dv + kColsPerTile - 1) / kColsPerTile;
  const int t_begin = kFullRow ? 0 : static_cast<int>(blockIdx.y);
  const int t_end = kFullRow ? ntiles : t_begin + 1;

  for (int ct = t_begin; ct < t_end; ++ct) {
    const int c0 = ct * kColsPerTile + cx * 4;
    float vv[4], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = (c0 + j < dv) ? Elem<T>::load(v, bh * dv + c0 + j) : 0.f;

    if (kVec4 && c0 + 3 < dv && dk == kRowGroups * 16) {
      update_rows<16>(S, dv, c0, ry, g, s_k, s_q, vv, acc);
    } else if (kVec4 && c0 + 3 < dv && dk == kRowGroups * 8) {
      update_rows<8>(S, dv, c0, ry, g, s_k, s_q, vv, acc);
    } else if (kVec4 && c0 + 3 < dv) {
#pragma unroll 4
      for (int r = ry; r < dk; r += kRowGroups) {
        float4* p = reinterpret_cast<float4*>(S + static_cast<int64_t>(r) * dv + c0);
        float4 s = *p;
        const float kr = s_k[r], qr = s_q[r];
        s.x = fmaf(g, s.x, kr * vv[0]);
        s.y = fmaf(g, s.y, kr * vv[1]);
        s.z = fmaf(g, s.z, kr * vv[2]);
        s.w = fmaf(g, s.w, kr * vv[3]);
        *p = s;
        acc[0] = fmaf(qr, s.x, acc[0]);
        acc[1] = fmaf(qr, s.y, acc[1]);
        acc[2] = fmaf(qr, s.z, acc[2]);
        acc[3] = fmaf(qr, s.w, acc[3]);
      }
    } else {
      for (int r = ry; r < dk; r += kRowGroups) {
        float* p = S + static_cast<int64_t>(r) * dv;
        const float kr = s_k[r], qr = s_q[r];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (c0 + j < dv) {
            const float s = fmaf(g, p[c0 + j], kr * vv[j]);
            p[c0 + j] = s;
            acc[j] = fmaf(qr, s, acc[j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s_part[ry][cx * 4 + j] = acc[j];
    __syncthreads();
    if (tid < kColsPerTile) {
      const int c = ct * kColsPerTile + tid;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < kRowGroups; ++r) sum += s_part[r][tid];
      if (c < dv) {
        if (kFullRow) s_row[c] = sum;
        else Elem<T>::store(o, bh * dv + c, sum);
      }
    }
    __syncthreads();
  }

  if (kFullRow) {
    // Per-head GroupNorm over the dv outputs: mean, then biased variance.
    float part = 0.f;
    for (int c = tid; c < dv; c += kThreads) part += s_row[c];
    const float mean = block_sum_256(part, s_red) / dv;
    __syncthreads();
    part = 0.f;
    for (int c = tid; c < dv; c += kThreads) {
      const float d = s_row[c] - mean;
      part += d * d;
    }
    const float var = block_sum_256(part, s_red) / dv;
    const float rstd = 1.0f / sqrtf(var + gn.eps);
    for (int c = tid; c < dv; c += kThreads) {
      float y = (s_row[c] - mean) * rstd;
      if (gn.weight) y *= gn.weight[h * dv + c];
      if (gn.bias) y += gn.bias[h * dv + c];
      if (gn.gate) y *= swish(Elem<T>::load(static_cast<const T*>(gn.gate), bh * dv + c));
      Elem<T>::store(o, bh * dv + c, y);
    }
  }
}

template <typename T>
hipError_t launch_typed(const void* q, const void* k, const void* v, float* state, void* o, int B, int H,
                        int dk, int dv, const HeadDecay& decay, const GnArgs& gn, hipStream_t stream) {
  const T* qt = static_cast<const T*>(q);
  const T* kt = static_cast<const T*>(k);
  const T* vt = static_cast<const T*>(v);
  T* ot = static_cast<T*>(o);
  const bool vec4 = (dv % 4) == 0;
  const dim3 block(kThreads);
  if (gn.enabled) {
    const dim3 grid(B * H, 1);
    if (vec4)
      decode_step_kernel<T, true, true><<<grid, block, 0, stream>>>(qt, kt, vt, state, ot, H, dk, dv, decay, gn);
    else
      decode_step_kernel<T, true, false><<<grid, block, 0, stream>>>(qt, kt, vt, state, ot, H, dk, dv, decay, gn);
  } else {
    const dim3 grid(B * H, (dv + kColsPerTile - 1) / kColsPerTile);
    if (vec4)
      decode_step_kernel<T, false, true><<<grid, block, 0, stream>>>(qt, kt, vt, state, ot, H, dk, dv, decay, gn);
    else
      decode_step_kernel<T, false, false><<<grid, block, 0, stream>>>(qt, kt, vt, state, ot, H, dk, dv, decay, gn);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(int dtype, const void* q, const void* k, const void* v, float* state, void* o,
                              int B, int H, int dk, int dv, const HeadDecay& decay, const GnArgs& gn,
                              hipStream_t stream) {
  if (dtype == 0) return launch_typed<float>(q, k, v, state, o, B, H, dk, dv, decay, gn, stream);
  return launch_typed<uint16_t>(q, k, v, state, o, B, H, dk, dv, decay, gn, stream);
}

}  // namespace ret

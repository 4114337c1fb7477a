// Data-movement kernels of the retention backward pass (gfx950).
//
// The gradients of retention are themselves retentions ("RetNet - Retentive
// Network - A Successor to Transformer for LLMs", Key Equations, parallel
// form, differentiated): with dO the output gradient,
//   dQ = retention(query dO, key V, value K)                 (forward in time)
//   dK = reverse-time retention(query V, key dO, value Q)
//   dV = reverse-time retention(query K, key Q, value dO)
// where "reverse-time" is the forward form on token-reversed sequences. The
// host runs each with the chunkwise kernels on operands these kernels prepare
// (token reversal, splitting a width above 256 into parts the MFMA kernels
// take, state transposes and per-head scalings), then sums and un-reverses the
// partial results. All of it is HBM-bound copying.
#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace ret {

namespace {

constexpr int kRowThreads = 256;  // four waves, one source row each
constexpr int kRowsPerBlock = 4;

template <typename T>
struct Vec16;  // 16-byte chunk of T
template <>
struct Vec16<uint16_t> {
  static constexpr int kElems = 8;
};
template <>
struct Vec16<float> {
  static constexpr int kElems = 4;
};

// Up to three destinations of one source row: part p of destination t
// (layout [BH, N, w_p], w_p = part_w except a narrower last part) gets
// columns [p*part_w, p*part_w + w_p) of src row r ([BH, N, D]) at row r or at
// its token reversal within the head. One read of the source feeds them all.
// VEC: every width is a multiple of 16 bytes, copied in 16-byte pieces.
template <typename T>
struct SplitDst {
  T* base[3];
  int part_w[3];
  int64_t part_stride[3];
  int flip[3];
  int count;
};

template <typename T, bool VEC>
__global__ void __launch_bounds__(kRowThreads)
split_rows_kernel(const T* __restrict__ src, SplitDst<T> dst, int64_t rows, int N, int D) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t bh = row / N;
  const int n = static_cast<int>(row - bh * N);
  const T* s = src + row * D;
  if constexpr (VEC) {
    constexpr int E = Vec16<T>::kElems;
    for (int c = lane * E; c < D; c += 64 * E) {
      const uint4 x = *reinterpret_cast<const uint4*>(s + c);
      for (int t = 0; t < dst.count; ++t) {
        const int pw = dst.part_w[t];
        const int p = c / pw, cc = c - p * pw;
        const int w = min(pw, D - p * pw);
        const int nd = dst.flip[t] ? N - 1 - n : n;
        *reinterpret_cast<uint4*>(dst.base[t] + p * dst.part_stride[t] + (bh * N + nd) * static_cast<int64_t>(w) +
                                  cc) = x;
      }
    }
  } else {
    for (int c = lane; c < D; c += 64) {
      const T x = s[c];
      for (int t = 0; t < dst.count; ++t) {
        const int pw = dst.part_w[t];
        const int p = c / pw, cc = c - p * pw;
        const int w = min(pw, D - p * pw);
        const int nd = dst.flip[t] ? N - 1 - n : n;
        dst.base[t][p * dst.part_stride[t] + (bh * N + nd) * static_cast<int64_t>(w) + cc] = x;
      }
    }
  }
}

// dst row r ([BH, N, W]) <- sum over the nparts part buffers (each [BH, N, W],
// part_stride elements apart) of row r or its token reversal, summed in fp32.
template <typename T, bool VEC>
__global__ void __launch_bounds__(kRowThreads)
sum_parts_kernel(const T* __restrict__ parts, T* __restrict__ dst, int64_t rows, int N, int W, int nparts,
                 int64_t part_stride, int flip) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t bh = row / N;
  const int n = static_cast<int>(row - bh * N);
  const int64_t srow = bh * N + (flip ? N - 1 - n : n);
  T* d = dst + row * W;
  if constexpr (VEC && sizeof(T) == 2) {
    for (int c = lane * 8; c < W; c += 64 * 8) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int p = 0; p < nparts; ++p) {
        const uint4 x = *reinterpret_cast<const uint4*>(parts + p * part_stride + srow * W + c);
        const uint32_t wds[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(wds[e] << 16);
          acc[2 * e + 1] += __uint_as_float(wds[e] & 0xffff0000u);
        }
      }
      uint4 y;
      y.x = pack_bf16x2(acc[0], acc[1]);
      y.y = pack_bf16x2(acc[2], acc[3]);
      y.z = pack_bf16x2(acc[4], acc[5]);
      y.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(d + c) = y;
    }
  } else {
    for (int c = lane; c < W; c += 64) {
      float acc = 0.f;
      for (int p = 0; p < nparts; ++p) acc += Elem<T>::load(parts + p * part_stride, srow * W + c);
      Elem<T>::store(d, c, acc);
    }
  }
}

// Per-head scaled copy of fp32 states src [BH, R, C]: dst = fac[h] * src, or,
// with `transpose`, dst part p ([BH, w_p, R], the rows [p*part_w, ..) of the
// transposed state) = fac[h] * src^T. fac == nullptr means 1.
struct HeadFactor {
  float f[kMaxHeads];
};

__global__ void __launch_bounds__(kRowThreads)
state_prep_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t heads, int H, int R, int C,
                  int transpose, int part_w, int64_t part_stride, HeadFactor fac) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kRowThreads + threadIdx.x;
  const int64_t per = static_cast<int64_t>(R) * C;
  if (i >= heads * per) return;
  const int64_t bh = i / per;
  const int rem = static_cast<int>(i - bh * per);
  const int r = rem / C, c = rem - r * C;
  const float x = src[i] * fac.f[bh % H];
  if (!transpose) {
    dst[i] = x;
  } else {
    const int p = c / part_w, cc = c - p * part_w;
    const int w = min(part_w, C - p * part_w);
    dst[p * part_stride + (bh * w + cc) * static_cast<int64_t>(R) + r] = x;
  }
}

bool vec_ok(int esize, int D, int part_w, const void* a, const void* b) {
  return (D * esize) % 16 == 0 && (part_w * esize) % 16 == 0 && reinterpret_cast<uintptr_t>(a) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(b) % 16 == 0;
}

}  // namespace

template <typename T>
hipError_t split_typed(const void* src, const SplitTarget* targets, int ntargets, const Dims& d, int D,
                       hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(d.B) * d.H * d.N;
  if (rows == 0 || ntargets == 0) return hipSuccess;
  SplitDst<T> dst{};
  bool vec = (D * sizeof(T)) % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0;
  for (int t = 0; t < ntargets; ++t) {
    dst.base[t] = static_cast<T*>(targets[t].dst);
    dst.part_w[t] = targets[t].part_w;
    dst.part_stride[t] = targets[t].part_stride;
    dst.flip[t] = targets[t].flip ? 1 : 0;
    vec = vec && (targets[t].part_w * sizeof(T)) % 16 == 0 && reinterpret_cast<uintptr_t>(targets[t].dst) % 16 == 0;
  }
  dst.count = ntargets;
  const dim3 grid(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const T* s = static_cast<const T*>(src);
  if (vec)
    split_rows_kernel<T, true><<<grid, kRowThreads, 0, stream>>>(s, dst, rows, d.N, D);
  else
    split_rows_kernel<T, false><<<grid, kRowThreads, 0, stream>>>(s, dst, rows, d.N, D);
  return hipGetLastError();
}

hipError_t launch_split_rows(int dtype, const void* src, const SplitTarget* targets, int ntargets, const Dims& d,
                             int D, hipStream_t stream) {
  if (ntargets < 0 || ntargets > 3) return hipErrorInvalidValue;
  return dtype == 0 ? split_typed<float>(src, targets, ntargets, d, D, stream)
                    : split_typed<uint16_t>(src, targets, ntargets, d, D, stream);
}

hipError_t launch_sum_parts(int dtype, const void* parts, void* dst, const Dims& d, int W, int nparts,
                            int64_t part_stride, bool flip, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(d.B) * d.H * d.N;
  if (rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const int f = flip ? 1 : 0;
  if (dtype == 0) {
    sum_parts_kernel<float, false><<<grid, kRowThreads, 0, stream>>>(
        static_cast<const float*>(parts), static_cast<float*>(dst), rows, d.N, W, nparts, part_stride, f);
  } else {
    auto s = static_cast<const uint16_t*>(parts);
    auto o = static_cast<uint16_t*>(dst);
    if (vec_ok(2, W, W, parts, dst))
      sum_parts_kernel<uint16_t, true><<<grid, kRowThreads, 0, stream>>>(s, o, rows, d.N, W, nparts, part_stride, f);
    else
      sum_parts_kernel<uint16_t, false><<<grid, kRowThreads, 0, stream>>>(s, o, rows, d.N, W, nparts, part_stride,
                                                                          f);
  }
  return hipGetLastError();
}

hipError_t launch_state_prep(const float* src, float* dst, int B, int H, int R, int C, bool transpose, int part_w,
                             int64_t part_stride, const float* head_factor, hipStream_t stream) {
  HeadFactor fac;
  for (int h = 0; h < kMaxHeads; ++h) fac.f[h] = (head_factor && h < H) ? head_factor[h] : 1.0f;
  const int64_t heads = static_cast<int64_t>(B) * H;
  const int64_t n = heads * R * C;
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + kRowThreads - 1) / kRowThreads));
  state_prep_kernel<<<grid, kRowThreads, 0, stream>>>(src, dst, heads, H, R, C, transpose ? 1 : 0, part_w,
                                                      part_stride, fac);
  return hipGetLastError();
}

}  // namespace ret

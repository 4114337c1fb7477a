// Rotation of the xPos relative position encoding, applied to Q and K before
// retention ("RetNet - Retentive Network - A Successor to Transformer for
// LLMs", Methods: block structure, and Key components, 3. xPos; "RetNet入門",
// the conjugate in the parallel representation). The features of a token,
// taken in pairs (x[2i], x[2i+1]) as complex numbers, are multiplied by
// exp(i n theta_i) at position n:
//   y[2i]   = x[2i] cos(n theta_i) - x[2i+1] sin(n theta_i)
//   y[2i+1] = x[2i] sin(n theta_i) + x[2i+1] cos(n theta_i)
// Q and K rotated alike give real dot products that depend on n - m only.
//
// The pass reads and writes every element once and is bound by HBM. A thread
// takes P pairs of one position (16-byte bf16 accesses at P = 4), forms their
// P angles once and applies them to that position in kHeads heads of Q and of
// K, with all of its loads in flight before the first store; the stores are
// non-temporal. The pass runs at about the rate of a plain device copy of the
// same bytes. An angle is
// n * theta_i in double precision, reduced by the nearest multiple of 2 pi in
// double (positions up to 2^53 stay exact; 2 pi in two parts), then sincosf
// of the remainder in [-pi, pi].
#include "common.h"
#include "kernels.h"

namespace ret {

namespace {

constexpr int kThreadsX = 256;
constexpr int kHeads = 8;  // heads per thread (each of Q and K)
// 2 pi as the nearest double plus the remainder, so that subtracting a whole
// number of turns t leaves an error near t * 1e-32 rather than t * 2.4e-16
// (Cody and Waite's two-constant reduction).
constexpr double kTwoPiHi = 6.283185307179586232;
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

struct XposArgs {
  float theta[kMaxXposPairs];
};

// W 32-bit words per thread and tensor: P pairs of bf16 (W = P) or fp32 (W = 2P).
template <int W>
struct Words {
  uint32_t w[W];
};

template <int W>
__device__ __forceinline__ Words<W> load_words(const void* base, int64_t byte_off) {
  Words<W> r;
  const char* p = static_cast<const char*>(base) + byte_off;
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      const uint4 u = *reinterpret_cast<const uint4*>(p + 4 * i);
      r.w[i] = u.x;
      r.w[i + 1] = u.y;
      r.w[i + 2] = u.z;
      r.w[i + 3] = u.w;
    }
  } else if constexpr (W == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    r.w[0] = u.x;
    r.w[1] = u.y;
  } else {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  return r;
}

// Streaming stores (non-temporal: the rotated tensors are not read again by
// this kernel, measured about 4% faster than ordinary stores).
typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32v2 __attribute__((ext_vector_type(2)));
template <int W>
__device__ __forceinline__ void store_words(void* base, int64_t byte_off, const Words<W>& r) {
  char* p = static_cast<char*>(base) + byte_off;
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      const u32v4 x = {r.w[i], r.w[i + 1], r.w[i + 2], r.w[i + 3]};
      __builtin_nontemporal_store(x, reinterpret_cast<u32v4*>(p + 4 * i));
    }
  } else if constexpr (W == 2) {
    const u32v2 x = {r.w[0], r.w[1]};
    __builtin_nontemporal_store(x, reinterpret_cast<u32v2*>(p));
  } else {
    __builtin_nontemporal_store(r.w[0], reinterpret_cast<uint32_t*>(p));
  }
}

// Rotate the P pairs held in `x` (bf16 pairs: one word per pair; fp32: two).
template <bool BF16, int P, int W>
__device__ __forceinline__ Words<W> rotate(const Words<W>& x, const float (&c)[P], const float (&s)[P]) {
  Words<W> y;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float re, im;
    if constexpr (BF16) {
      re = __uint_as_float(x.w[p] << 16);
      im = __uint_as_float(x.w[p] & 0xffff0000u);
    } else {
      re = __uint_as_float(x.w[2 * p]);
      im = __uint_as_float(x.w[2 * p + 1]);
    }
    const float yr = re * c[p] - im * s[p];
    const float yi = re * s[p] + im * c[p];
    if constexpr (BF16) {
      y.w[p] = pack_bf16x2(yr, yi);
    } else {
      y.w[2 * p] = __float_as_uint(yr);
      y.w[2 * p + 1] = __float_as_uint(yi);
    }
  }
  return y;
}

// Grid: x over blocks of `rows` positions, y over groups of kHeads heads
// (grid-stride when there are more groups than blocks in y). q_out / k_out may
// equal q / k: each element is read and written by the same thread, reads
// first. k == nullptr rotates Q alone.
template <bool BF16, int P>
__global__ void __launch_bounds__(kThreadsX) xpos_kernel(const void* q, const void* k, void* q_out, void* k_out,
                                                          XposArgs th, int BH, int N, int d, int64_t pos0) {
  constexpr int W = BF16 ? P : 2 * P;
  constexpr int kElemBytes = BF16 ? 2 : 4;
  const int groups = d / (2 * P);  // threads per position
  const int rows = kThreadsX / groups;
  const int r = threadIdx.x / groups;
  const int g = threadIdx.x - r * groups;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * rows + r;
  if (r >= rows || n >= N) return;

  const int64_t col_bytes = static_cast<int64_t>(g) * 2 * P * kElemBytes;
  const int ngroups = (BH + kHeads - 1) / kHeads;
  for (int hg = blockIdx.y; hg < ngroups; hg += gridDim.y) {
    const int bh0 = hg * kHeads;
    Words<W> xq[kHeads], xk[kHeads];
#pragma unroll
    for (int j = 0; j < kHeads; ++j) {
      if (bh0 + j >= BH) break;
      const int64_t off = ((static_cast<int64_t>(bh0 + j) * N + n) * d) * kElemBytes + col_bytes;
      xq[j] = load_words<W>(q, off);
      if (k) xk[j] = load_words<W>(k, off);
    }
    // The angles (the same for every head).
    float c[P], s[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const double a = static_cast<double>(pos0 + n) * static_cast<double>(th.theta[g * P + p]);
      const double turns = rint(a * kInvTwoPi);
      const float rem = static_cast<float>(fma(-turns, kTwoPiLo, fma(-turns, kTwoPiHi, a)));
      sincosf(rem, &s[p], &c[p]);
    }
#pragma unroll
    for (int j = 0; j < kHeads; ++j) {
      if (bh0 + j >= BH) break;
      const int64_t off = ((static_cast<int64_t>(bh0 + j) * N + n) * d) * kElemBytes + col_bytes;
      store_words<W>(q_out, off, rotate<BF16, P, W>(xq[j], c, s));
      if (k) store_words<W>(k_out, off, rotate<BF16, P, W>(xk[j], c, s));
    }
  }
}

template <bool BF16, int P>
hipError_t launch(const void* q, const void* k, void* q_out, void* k_out, const XposArgs& th, int BH, int N, int d,
                  int64_t pos0, hipStream_t stream) {
  const int groups = d / (2 * P);
  const int rows = kThreadsX / groups;
  const int64_t gx = (static_cast<int64_t>(N) + rows - 1) / rows;
  const int ngroups = (BH + kHeads - 1) / kHeads;
  const int gy = ngroups < 65535 ? ngroups : 65535;
  if (gx > 0x7fffffff) return hipErrorInvalidConfiguration;
  xpos_kernel<BF16, P><<<dim3(static_cast<unsigned>(gx), gy), kThreadsX, 0, stream>>>(q, k, q_out, k_out, th, BH, N,
                                                                                     d, pos0);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_xpos_rotate(int dtype, const void* q, const void* k, void* q_out, void* k_out, const float* theta,
                              int BH, int N, int d, int64_t pos0, hipStream_t stream) {
  XposArgs th{};
  for (int i = 0; i < d / 2; ++i) th.theta[i] = theta[i];
  // Four pairs per thread (16-byte accesses) when whole groups of 8 features
  // fit the row and every pointer allows 16-byte accesses; else one pair.
  const bool wide = d % 8 == 0 && aligned16(q) && aligned16(q_out) && (!k || (aligned16(k) && aligned16(k_out)));
  const bool bf16 = dtype == 1;
  if (bf16)
    return wide ? launch<true, 4>(q, k, q_out, k_out, th, BH, N, d, pos0, stream)
                : launch<true, 1>(q, k, q_out, k_out, th, BH, N, d, pos0, stream);
  return wide ? launch<false, 4>(q, k, q_out, k_out, th, BH, N, d, pos0, stream)
              : launch<false, 1>(q, k, q_out, k_out, th, BH, N, d, pos0, stream);
}

}  // namespace ret

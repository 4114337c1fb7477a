// C ABI of the retention library: argument validation, planning and launches.
//
// Validation runs entirely on the host and before any HIP call, so invalid or
// unsupported arguments are reported without touching a device. Planning is a
// pure function of the sizes: it picks the MFMA kernels for bf16 shapes they
// cover and the generic vector-ALU kernels otherwise, and it sizes the
// chunkwise workspace.
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "retention.h"

namespace {

using ret::Dims;
using ret::GnArgs;
using ret::HeadDecay;

constexpr size_t kAlign = 256;
constexpr int kMfmaRows = 64;            // MFMA kernels need chunk % 64 == 0
constexpr int64_t kWalkTargetBlocks = 512;  // segment the walk below this many workgroups

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int dtype) { return dtype == RET_F32 || dtype == RET_BF16; }

int check_sizes(int B, int H, int N, int dk, int dv, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || dk <= 0 || dv <= 0) return RET_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return RET_ERR_INVALID_ARG;
  if (H > RETENTION_MAX_HEADS || dk > RETENTION_MAX_DK || dv > RETENTION_MAX_DV) return RET_ERR_UNSUPPORTED;
  // Grid sizes: the generic output kernel launches one block per (b, h, n).
  if (static_cast<int64_t>(B) * H * N >= (int64_t{1} << 31)) return RET_ERR_UNSUPPORTED;
  return RET_OK;
}

int check_gamma(const float* gamma_host, int H, HeadDecay* decay) {
  if (!gamma_host) return RET_ERR_INVALID_ARG;
  for (int h = 0; h < H; ++h) {
    const float g = gamma_host[h];
    if (!std::isfinite(g) || !(g > 0.0f) || !(g < 1.0f)) return RET_ERR_INVALID_ARG;
  }
  if (decay) {
    for (int h = 0; h < RETENTION_MAX_HEADS; ++h)
      decay->log2g[h] = h < H ? static_cast<float>(std::log2(static_cast<double>(gamma_host[h]))) : 0.0f;
  }
  return RET_OK;
}

int check_gn(const retention_gn_t* gn, GnArgs* out) {
  out->enabled = 0;
  out->eps = 0.0f;
  out->weight = nullptr;
  out->bias = nullptr;
  out->gate = nullptr;
  if (!gn) return RET_OK;
  if (!std::isfinite(gn->eps) || gn->eps < 0.0f) return RET_ERR_INVALID_ARG;
  out->enabled = 1;
  out->eps = gn->eps;
  out->weight = gn->weight;
  out->bias = gn->bias;
  out->gate = gn->gate;
  return RET_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? RET_OK : RET_ERR_HIP; }

// Chunkwise execution plan.
struct ChunkPlan {
  bool mfma;
  int nchunks;
  int chunks_per_seg;
  int nseg;
  size_t states_bytes;  // per-chunk states
  size_t seg_bytes;     // segment end states (MFMA path, nseg > 1)
  size_t total;
};

ChunkPlan plan_chunkwise(int B, int H, int N, int dk, int dv, int chunk, int dtype) {
  ChunkPlan p{};
  p.mfma = dtype == RET_BF16 && ret::mfma_supports(dk, dv) && chunk % kMfmaRows == 0;
  p.nchunks = (N + chunk - 1) / chunk;
  const size_t heads = static_cast<size_t>(B) * H;
  const size_t dkdv = static_cast<size_t>(dk) * dv;
  if (p.mfma) {
    const int64_t per_seg = static_cast<int64_t>(heads) * ret::walk_tiles_per_head(heads, dk, dv);
    int64_t want = ret::walk_wide(heads, dk, dv) ? 1 : (kWalkTargetBlocks + per_seg - 1) / per_seg;
    if (want < 1) want = 1;
    if (want > p.nchunks) want = p.nchunks;
    p.chunks_per_seg = static_cast<int>((p.nchunks + want - 1) / want);
    p.nseg = (p.nchunks + p.chunks_per_seg - 1) / p.chunks_per_seg;
    p.states_bytes = align_up(heads * p.nchunks * dkdv * sizeof(uint16_t));
    p.seg_bytes = p.nseg > 1 ? align_up(heads * p.nseg * dkdv * sizeof(float)) : 0;
  } else {
    p.chunks_per_seg = p.nchunks;
    p.nseg = 1;
    p.states_bytes = align_up(heads * p.nchunks * dkdv * sizeof(float));
    p.seg_bytes = 0;
  }
  p.total = p.states_bytes + p.seg_bytes;
  return p;
}

// Shared validation of the chunkwise entry points (no HIP calls).
int check_chunkwise(const float* gamma_host, int B, int H, int N, int dk, int dv, int chunk, int dtype,
                    const retention_gn_t* gn, const void* workspace, size_t workspace_bytes, GnArgs* g,
                    ChunkPlan* plan, HeadDecay* decay) {
  if (chunk <= 0) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  st = check_gn(gn, g);
  if (st != RET_OK) return st;
  *plan = plan_chunkwise(B, H, N, dk, dv, chunk, dtype);
  if (plan->total > 0 && (!workspace || workspace_bytes < plan->total)) return RET_ERR_INVALID_ARG;
  check_gamma(gamma_host, H, decay);
  return RET_OK;
}

hipError_t launch_states(const ChunkPlan& p, const void* k, const void* v, const float* state_in, float* state_out,
                         char* ws, const Dims& d, int chunk, int dtype, const HeadDecay& decay, hipStream_t s) {
  if (p.mfma) {
    uint16_t* states = reinterpret_cast<uint16_t*>(ws);
    float* segs = p.seg_bytes ? reinterpret_cast<float*>(ws + p.states_bytes) : nullptr;
    return ret::launch_mfma_state_walk(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), state_in,
                                       state_out, states, segs, p.chunks_per_seg, d, chunk, decay, s);
  }
  return ret::launch_generic_state_walk(dtype, k, v, state_in, state_out, reinterpret_cast<float*>(ws), d, chunk,
                                        decay, s);
}

hipError_t launch_output(const ChunkPlan& p, const void* q, const void* k, const void* v, void* o, const char* ws,
                         bool state0, const Dims& d, int chunk, int dtype, const HeadDecay& decay, const GnArgs& g,
                         hipStream_t s) {
  if (p.mfma) {
    return ret::launch_mfma_chunk_out(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), reinterpret_cast<const uint16_t*>(ws), state0,
                                      static_cast<uint16_t*>(o), d, chunk, decay, g, s);
  }
  return ret::launch_generic_chunk_out(dtype, q, k, v, reinterpret_cast<const float*>(ws), state0, o, d, chunk,
                                       decay, g, s);
}

}  // namespace

extern "C" {

int retention_abi_version(void) { return RETENTION_ABI_VERSION; }

const char* retention_status_string(int status) {
  switch (status) {
    case RET_OK: return "ok";
    case RET_ERR_INVALID_ARG: return "invalid argument";
    case RET_ERR_UNSUPPORTED: return "unsupported arguments";
    case RET_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int retention_parallel(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B, int H,
                       int N, int dk, int dv, int dtype, const retention_gn_t* gn, void* stream) {
  if (!q || !k || !v || !o) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  GnArgs g;
  st = check_gn(gn, &g);
  if (st != RET_OK) return st;

  HeadDecay decay;
  check_gamma(gamma_host, H, &decay);
  const Dims d{B, H, N, dk, dv};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == RET_BF16 && ret::mfma_supports(dk, dv)) {
    return status_of(ret::launch_mfma_chunk_out(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                                static_cast<const uint16_t*>(v), nullptr, false,
                                                static_cast<uint16_t*>(o), d, N, decay, g, s));
  }
  return status_of(ret::launch_generic_chunk_out(dtype, q, k, v, nullptr, false, o, d, N, decay, g, s));
}

size_t retention_chunkwise_workspace_bytes(int B, int H, int N, int dk, int dv, int chunk, int dtype) {
  if (check_sizes(B, H, N, dk, dv, dtype) != RET_OK || chunk <= 0) return 0;
  return plan_chunkwise(B, H, N, dk, dv, chunk, dtype).total;
}

int retention_chunkwise(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B, int H,
                        int N, int dk, int dv, int chunk, int dtype, const float* state_in, float* state_out,
                        const retention_gn_t* gn, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return RET_ERR_INVALID_ARG;
  GnArgs g;
  ChunkPlan p;
  HeadDecay decay;
  const int st = check_chunkwise(gamma_host, B, H, N, dk, dv, chunk, dtype, gn, workspace, workspace_bytes, &g, &p,
                                 &decay);
  if (st != RET_OK) return st;
  const Dims d{B, H, N, dk, dv};
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (launch_states(p, k, v, state_in, state_out, ws, d, chunk, dtype, decay, s) != hipSuccess) return RET_ERR_HIP;
  return status_of(launch_output(p, q, k, v, o, ws, state_in != nullptr, d, chunk, dtype, decay, g, s));
}

int retention_chunk_states(const void* k, const void* v, const float* gamma_host, int B, int H, int N, int dk,
                           int dv, int chunk, int dtype, const float* state_in, float* state_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!k || !v) return RET_ERR_INVALID_ARG;
  GnArgs g;
  ChunkPlan p;
  HeadDecay decay;
  const int st = check_chunkwise(gamma_host, B, H, N, dk, dv, chunk, dtype, nullptr, workspace, workspace_bytes, &g,
                                 &p, &decay);
  if (st != RET_OK) return st;
  const Dims d{B, H, N, dk, dv};
  return status_of(launch_states(p, k, v, state_in, state_out, static_cast<char*>(workspace), d, chunk, dtype, decay,
                                 static_cast<hipStream_t>(stream)));
}

int retention_chunk_output(const void* q, const void* k, const void* v, const float* gamma_host, void* o, int B,
                           int H, int N, int dk, int dv, int chunk, int dtype, int has_state_in,
                           const retention_gn_t* gn, const void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o) return RET_ERR_INVALID_ARG;
  GnArgs g;
  ChunkPlan p;
  HeadDecay decay;
  const int st = check_chunkwise(gamma_host, B, H, N, dk, dv, chunk, dtype, gn, workspace, workspace_bytes, &g, &p,
                                 &decay);
  if (st != RET_OK) return st;
  const Dims d{B, H, N, dk, dv};
  return status_of(launch_output(p, q, k, v, o, static_cast<const char*>(workspace), has_state_in != 0, d, chunk,
                                 dtype, decay, g, static_cast<hipStream_t>(stream)));
}

int retention_recurrent_step(const void* q, const void* k, const void* v, const float* gamma_host, float* state,
                             void* o, int B, int H, int dk, int dv, int dtype, const retention_gn_t* gn,
                             void* stream) {
  if (!q || !k || !v || !o || !state) return RET_ERR_INVALID_ARG;
  int st = check_sizes(B, H, 1, dk, dv, dtype);
  if (st != RET_OK) return st;
  st = check_gamma(gamma_host, H, nullptr);
  if (st != RET_OK) return st;
  GnArgs g;
  st = check_gn(gn, &g);
  if (st != RET_OK) return st;
  HeadDecay decay;
  check_gamma(gamma_host, H, &decay);
  return status_of(ret::launch_decode_step(dtype, q, k, v, state, o, B, H, dk, dv, decay, g,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

/*
 * retention.h — C ABI of the Multi-Scale Retention library (gfx950 / MI355X).
 *
 * The operator (sources, by page title and section):
 *   "RetNet - Retentive Network - A Successor to Transformer for LLMs"
 *   (irregular6612.github.io blog):
 *     - Key Equations, parallel form: O = (Q K^T (*) D) V with the causal decay
 *       mask D[n][m] = gamma^(n-m) for n >= m and 0 otherwise;
 *     - Key Equations, recurrent form: S_n = gamma S_{n-1} + K_n^T V_n,
 *       o_n = Q_n S_n;
 *     - Key Equations, chunkwise recurrent form: parallel inside a chunk plus
 *       a cross-chunk read-out (Q_[i] (*) xi) R_{i-1} of the carried state;
 *     - Key components, 2. Multi-Scale Retention: each head has its own decay
 *       (the usual schedule is gamma_h = 1 - 2^(-5-h));
 *     - Methods / Key components, 4. block: a GroupNorm follows retention.
 *   jisaku.com RetNet glossary entry: the same definition, 0 < gamma < 1, and
 *   the three computation modes (parallel, recurrent, chunkwise).
 *
 * Conventions shared by every entry point:
 *   - Q, K are [B, H, N, dk] and V, O are [B, H, N, dv], contiguous row-major
 *     device buffers of the element type `dtype` (RET_F32 or RET_BF16). O has
 *     the input's element type; bf16 results are rounded to nearest even.
 *   - A state S is fp32 [B, H, dk, dv], contiguous row-major, dv fastest.
 *     A recurrent step updates the state first and then reads it out, so a
 *     token sees itself with weight 1.
 *   - gamma_host is a HOST array of H floats, each finite with 0 < gamma < 1.
 *     It is read during the call only and may be freed on return.
 *   - gn (optional, NULL = none) asks for the per-head GroupNorm epilogue:
 *     for each (b, h, n) the mean and biased variance over that head's dv
 *     outputs, y = (o - mean) / sqrt(var + eps) * weight[h*dv + c] + bias[h*dv + c].
 *     weight and bias are device fp32 [H*dv] and may each be NULL (identity).
 *   - gn->gate (optional, NULL = none) adds the swish gate of the gated MSR
 *     block ("RetNet - Retentive Network ...", Key components, 4. block:
 *     GroupNorm with swish gating; "RetNet入門" (news.ainew.jp), Multi-Scale
 *     Retention (MSR): the normalised head outputs times the gated branch):
 *     the stored output is y * swish(g) with swish(g) = g / (1 + exp(-g)),
 *     where g is the gate's element at the same position. The gate is a device
 *     buffer of the input's element type laid out like O ([B, H, N, dv]; one
 *     token [B, H, dv] for the recurrent step), read only. It holds the gate
 *     branch's pre-activation (its projection is the caller's). It must not
 *     alias O.
 *   - stream is a hipStream_t (NULL = the default stream). All work is
 *     enqueued on it and the call returns without synchronising. RET_OK means
 *     "validated and launched"; a fault inside a kernel surfaces on the next
 *     synchronising HIP call of the caller.
 *   - Ownership: the caller owns every buffer. The library allocates no
 *     device memory. Its only mutable global state is a per-device cache of
 *     occupancy figures (how many workgroups of a kernel fit the GPU at
 *     once), filled on first use through atomic stores and never changed
 *     afterwards; calls on different streams do not interfere except through
 *     buffers the caller shares.
 *   - O must not share bytes with Q, K or V, nor a gate with O, nor the
 *     recurrent step's state with its token vectors: the kernels write while
 *     other workgroups still read. Such calls are refused with
 *     RET_ERR_INVALID_ARG (the ranges are checked, the pointers never
 *     dereferenced on the host). No entry point throws; all report status.
 *
 * Status codes:
 *   RET_OK (0), RET_ERR_INVALID_ARG (-1): a required pointer is NULL, a size
 *   is <= 0, chunk <= 0, a gamma is not in (0, 1), dtype is unknown, or the
 *   workspace is too small; RET_ERR_UNSUPPORTED (-2): valid arguments outside
 *   what the kernels implement (for example H > RETENTION_MAX_HEADS or dk
 *   above RETENTION_MAX_DK); RET_ERR_HIP (-3): the HIP runtime reported an
 *   error for a launch. Invalid or unsupported arguments are detected before
 *   any HIP call is made. A chunk length at or above N means one chunk (all
 *   such lengths give the same result).
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RETENTION_ABI_VERSION 4
#define RETENTION_MAX_HEADS 256
#define RETENTION_MAX_DK 256
#define RETENTION_MAX_DV 1024
/* Workspace bytes retention_chunkwise_noalloc can provide from its own scratch. */
#define RETENTION_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)64 << 20)

enum retention_dtype { RET_F32 = 0, RET_BF16 = 1 };

enum retention_status {
  RET_OK = 0,
  RET_ERR_INVALID_ARG = -1,
  RET_ERR_UNSUPPORTED = -2,
  RET_ERR_HIP = -3
};

typedef struct retention_gn_t {
  float eps;            /* added to the variance; must be >= 0 and finite */
  const float* weight;  /* device fp32 [H*dv], or NULL for 1 */
  const float* bias;    /* device fp32 [H*dv], or NULL for 0 */
  const void* gate;     /* device, O's type and layout, or NULL for no gate */
} retention_gn_t;

/* RETENTION_ABI_VERSION of the built library. */
int retention_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* retention_status_string(int status);

/*
 * Parallel form ("RetNet - Retentive Network ...", Key Equations, parallel
 * form; jisaku.com glossary, parallel mode): for every (b, h),
 *   o_n = sum_{m <= n} gamma_h^(n-m) (q_n . k_m) v_m,
 * then the optional GroupNorm. The N x N decay mask is never materialised.
 */
int retention_parallel(const void* q, const void* k, const void* v,
                       const float* gamma_host, void* o,
                       int B, int H, int N, int dk, int dv, int dtype,
                       const retention_gn_t* gn, void* stream);

/*
 * Bytes of device workspace retention_chunkwise needs for these sizes
 * (a pure function of its arguments; 0 for invalid sizes). Where the
 * single-pass kernel applies (bf16, dk 128 or 256, dv a multiple of 256 up to
 * 1024, chunk 64 or 128 after clamping to N) it is the GroupNorm exchange,
 * 2 KiB per (head, 256-column v tile), when there are at least 192 such
 * pairs. With fewer, each sequence is cut into nseg segments of whole chunks
 * (nseg = ceil(256 / pairs), at most chunks / 4; used when pairs * nseg >=
 * 192), walked in parallel from states a first pass computes: 2 KiB per
 * (head, segment, v tile), plus the segments' fp32 end states
 * (B*H*nseg*dk*dv*4 bytes) and room for a copy of state_in (B*H*dk*dv*4),
 * each part rounded up to 256 bytes. Otherwise it holds a state per chunk
 * (the two-stage path, retention_chunk_stages_workspace_bytes).
 */
size_t retention_chunkwise_workspace_bytes(int B, int H, int N, int dk, int dv,
                                           int chunk, int dtype);

/*
 * Bytes of device workspace the two stage entry points below need: the bf16
 * (fp32 for fp32 inputs) state carried into every chunk, plus segment end
 * states when the walk is cut into segments.
 */
size_t retention_chunk_stages_workspace_bytes(int B, int H, int N, int dk, int dv,
                                              int chunk, int dtype);

/*
 * Chunkwise recurrent form ("RetNet - Retentive Network ...", Key Equations,
 * chunkwise recurrent form and Key components, 1. Retention; jisaku.com
 * glossary, chunkwise mode). With chunk length C, chunk i covers rows
 * [i*C, min(i*C + C, N)) of length L (the last chunk may be shorter); for
 * local row j, xi_j = gamma^(j+1) and zeta_j = gamma^(L-1-j):
 *   O_[i] = (Q_[i] K_[i]^T (*) D_L) V_[i] + diag(xi) Q_[i] R_{i-1}
 *   R_i   = gamma^L R_{i-1} + K_[i]^T diag(zeta) V_[i]
 * with R_{-1} = state_in (NULL: zeros). state_out (NULL: not written)
 * receives R of the last chunk and may alias state_in. The result equals the
 * parallel and recurrent forms up to rounding. workspace must hold at least
 * retention_chunkwise_workspace_bytes(...) bytes (it may be NULL when that is
 * 0); its contents on entry do not matter and are clobbered.
 */
int retention_chunkwise(const void* q, const void* k, const void* v,
                        const float* gamma_host, void* o,
                        int B, int H, int N, int dk, int dv, int chunk, int dtype,
                        const float* state_in, float* state_out,
                        const retention_gn_t* gn,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * retention_chunkwise for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, results and status codes as
 * retention_chunkwise, without the workspace: the library takes it from a
 * device array of its own (RETENTION_NOALLOC_MAX_WORKSPACE_BYTES, 64 MiB per
 * GPU, held from the library's load until the process ends; its address is
 * looked up once per device on the first call there). Calls whose
 * retention_chunkwise_workspace_bytes(...) exceeds that size return
 * RET_ERR_UNSUPPORTED. The call allocates nothing. All calls on one GPU share
 * that GPU's array: calls that overlap in time on one GPU (different streams
 * not ordered by the caller) race and give undefined results; the contents
 * one call leaves are never read by the next.
 */
int retention_chunkwise_noalloc(const void* q, const void* k, const void* v,
                                const float* gamma_host, void* o,
                                int B, int H, int N, int dk, int dv, int chunk, int dtype,
                                const float* state_in, float* state_out,
                                const retention_gn_t* gn, void* stream);

/*
 * The two stages of retention_chunkwise, for callers that want the chunk
 * states themselves or time the stages separately. Same page and formulas as
 * retention_chunkwise; R_{i-1} is the state carried into chunk i.
 *
 * retention_chunk_states: computes R_{i-1} for every chunk i (R_{-1} =
 * state_in, or zeros when state_in is NULL) into the workspace, and the state
 * after the last chunk into state_out (NULL: not written; it may alias
 * state_in). Reads k and v only.
 *
 * retention_chunk_output: computes O from q, k, v and the chunk states that
 * retention_chunk_states left in the workspace for the same B, H, N, dk, dv,
 * chunk and dtype; has_state_in must be non-zero exactly when that call had a
 * state_in. Applies the optional GroupNorm.
 *
 * The workspace (at least retention_chunk_stages_workspace_bytes(...) bytes)
 * is opaque; its contents are only meaningful between these two calls.
 */
int retention_chunk_states(const void* k, const void* v, const float* gamma_host,
                           int B, int H, int N, int dk, int dv, int chunk, int dtype,
                           const float* state_in, float* state_out,
                           void* workspace, size_t workspace_bytes, void* stream);

int retention_chunk_output(const void* q, const void* k, const void* v,
                           const float* gamma_host, void* o,
                           int B, int H, int N, int dk, int dv, int chunk, int dtype,
                           int has_state_in, const retention_gn_t* gn,
                           const void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent decode step ("RetNet - Retentive Network ...", Key
 * Equations, recurrent form; jisaku.com glossary, recurrent mode):
 *   state <- gamma_h * state + k^T v   (in place, fp32 [B, H, dk, dv])
 *   o      = q . state                 (then the optional GroupNorm)
 * q, k are [B, H, dk] (one token), v and o are [B, H, dv], of type dtype.
 * state is required.
 */
int retention_recurrent_step(const void* q, const void* k, const void* v,
                             const float* gamma_host, float* state, void* o,
                             int B, int H, int dk, int dv, int dtype,
                             const retention_gn_t* gn, void* stream);

/*
 * xPos rotation of Q and K, the prologue of retention ("RetNet - Retentive
 * Network ...", Methods: block structure (xPos applied to Q and K) and Key
 * components, 3. xPos; "RetNet入門", the conjugate in the parallel
 * representation). The pages name a complex rotation by position and give no
 * formula; this takes the features of a token in pairs (x[2i], x[2i+1]) as
 * complex numbers and multiplies pair i of position n by
 * exp(1j * (pos0 + n) * theta_i):
 *   y[2i]   = x[2i] cos(a) - x[2i+1] sin(a),   a = (pos0 + n) * theta_i
 *   y[2i+1] = x[2i] sin(a) + x[2i+1] cos(a)
 * so that rotated queries and keys have real dot products that depend on
 * the positions only through n - m. The decay half of xPos is the
 * retention's own gamma^(n-m). theta_host holds d/2 finite angles (radians
 * per position; any schedule, chosen by the caller) and is read before the
 * call returns. q and k are [B, H, N, d] of type dtype; q_out and k_out have
 * the same shape and type and may be q and k themselves (in place) but must
 * not otherwise overlap any of the four buffers. k may be NULL (then k_out
 * must be NULL too): q alone is rotated. pos0 >= 0 is the position of row 0
 * (a decode step passes its token's position with N = 1); pos0 + N must not
 * exceed 2^53. d must be even, 2 <= d <= RETENTION_MAX_DK. Every pointer must
 * be aligned to a pair of elements (4 bytes for bf16, 8 for fp32). Angles are
 * formed and reduced modulo 2 pi in double precision, then the sine and
 * cosine are taken in float. Status: RET_ERR_INVALID_ARG for null or
 * misaligned pointers, partial overlaps, odd d, non-finite angles or pos0
 * out of range; RET_ERR_UNSUPPORTED for d above RETENTION_MAX_DK.
 */
int retention_xpos_rotate(const void* q, const void* k, void* q_out, void* k_out,
                          const float* theta_host, int B, int H, int N, int d,
                          long long pos0, int dtype, void* stream);

/*
 * Backward pass of retention: gradients with respect to q, k, v and the
 * starting state, for training ("RetNet - Retentive Network ...", Key
 * Equations: the parallel and chunkwise forms are the training forms; the
 * pages print no gradients). The forward map is the chunkwise form above
 * without GroupNorm or gate (a caller with those back-propagates through them
 * first) together with the state it leaves:
 *   O   = (Q K^T (*) D) V + diag(gamma^(n+1)) Q S0
 *   S_N = K^T diag(gamma^(N-1-m)) V + gamma^N S0
 * Given grad_o = dL/dO ([B, H, N, dv], the input type) and grad_state_out =
 * dL/dS_N (fp32 [B, H, dk, dv], NULL = 0), it writes
 *   grad_q = dA K + diag(gamma^(n+1)) grad_o S0^T        with A = Q K^T (*) D,
 *   grad_k = dA^T Q + diag(gamma^(N-1-m)) V dS_N^T            dA = (grad_o V^T) (*) D
 *   grad_v = A^T grad_o + diag(gamma^(N-1-m)) K dS_N
 *   grad_state_in = Q^T diag(gamma^(n+1)) grad_o + gamma^N dS_N   (fp32; NULL: not written)
 * grad_q, grad_k ([B, H, N, dk]) and grad_v ([B, H, N, dv]) have the input
 * type and must not share bytes with any input or with each other
 * (RET_ERR_INVALID_ARG). state_in (fp32, NULL = zeros) is the S0
 * of the forward call. Each gradient is evaluated as a retention of its own
 * (grad_q forward in time; grad_k and grad_v over the token-reversed sequence)
 * with the chunkwise kernels at the given chunk; a width above 256 is split
 * into parts whose results are summed. For bf16 with the chunk a multiple of
 * 64 (after clamping), dk 256 and dv a multiple of 256 (at most 1024), with at least
 * 192 (head, 256-column) units in each launch, the three retentions run on
 * the single-pass kernel reading the inputs in place (reverse order, row
 * pitch; one launch for grad_v, one per 256-wide part for grad_q and grad_k
 * together, the later parts adding to the first in fp32 before rounding; each
 * part's sum is rounded to the input type before the next adds to it, so
 * where the parts of an element cancel its error is set by the parts'
 * magnitudes, about 2^-9 of each in bf16, not by the result's) and
 * the workspace holds four fp32 state buffers and the exchange words;
 * otherwise the operands are first copied (reversed, split) into the
 * workspace. With grad_state_out given, every
 * gamma must be a normal float (>= FLT_MIN, about 1.2e-38): the final-state
 * gradient is divided by gamma on its way in, and RET_ERR_UNSUPPORTED is
 * returned otherwise. workspace must hold
 * retention_chunkwise_backward_workspace_bytes(...) bytes (contents on entry
 * do not matter and are clobbered). Same status codes as the other entry
 * points.
 */
size_t retention_chunkwise_backward_workspace_bytes(int B, int H, int N, int dk, int dv,
                                                    int chunk, int dtype);

int retention_chunkwise_backward(const void* q, const void* k, const void* v, const void* grad_o,
                                 const float* gamma_host, void* grad_q, void* grad_k, void* grad_v,
                                 int B, int H, int N, int dk, int dv, int chunk, int dtype,
                                 const float* state_in, const float* grad_state_out,
                                 float* grad_state_in, void* workspace, size_t workspace_bytes,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_H */

/*
 * la.h - C ABI of a gfx950 (MI355X) library for bidirectional (non-causal)
 * linear attention, forward and backward.
 *
 * The operation (Flash Bi-directional Linear Attention README: intro, and
 * "Update" 2024-12-28 for simple_la, "Update" 2024-12-30 for the backward).
 * Per batch b and head h, with Q, K in R^{T x D}, V in R^{T x Dv} and
 * phi(x) = elu(x) + 1 (x + 1 for x > 0, e^x otherwise; LA_PHI_RELU and
 * LA_PHI_IDENTITY select relu(x) or x instead):
 *     S = sum_t phi(k_t) v_t^T          (D x Dv, S[i][j])
 *     z = sum_t phi(k_t)                (D)
 *     O_t = phi(q_t) S / (phi(q_t) . z + eps)      normalised (default)
 *     O_t = phi(q_t) S                              simple_la (LA_SIMPLE)
 * The backward returns dQ, dK, dV, the vector-Jacobian product of
 * L = sum(O * dO) with eps held constant.
 *
 * Layout. q, k, dq, dk are dense row-major [B, H, T, D] arrays and v, o,
 * dout, dv dense row-major [B, H, T, Dv] arrays of `dtype` elements (the last
 * dimension contiguous), each 16-byte aligned; with LA_LAYOUT_BTHD in flags
 * they are [B, T, H, D] and [B, T, H, Dv] instead (each row still contiguous,
 * heads interleaved token by token). With la_problem.strides set, every
 * tensor has its own batch, head and token strides instead (strided views,
 * such as the Q, K and V of a packed [B, T, 3, H, D] projection, need no
 * copy). `state` is fp32: B*H blocks of S (D*Dv floats, S[i][j] at
 * i*Dv + j) followed by B*H blocks of z (D floats); la_state_bytes() gives
 * its size.
 *
 * Ownership. The caller allocates and owns all device memory: tensors, state
 * and workspace. The library never allocates, frees, synchronises or prints.
 * Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 * the call returns without waiting.
 *
 * Workspace. `ws` must be at least la_workspace_bytes() bytes and 256-byte
 * aligned; its contents need no initialisation. It carries the partial sums
 * of the split-T reductions, the backward state (dS, dz) from la_bwd_dq to
 * la_bwd_dkv, and the forward state when la_fwd is given state == NULL.
 * Calls that overlap in time (different streams, no ordering) must use
 * different workspaces.
 *
 * Errors. Every argument is checked before any HIP call, so a call that
 * returns a validation error has enqueued nothing. LA_ERR_DEVICE reports a
 * HIP launch error. Nothing is thrown across the ABI.
 *
 * Numerics. Inputs are read in `dtype`; phi is evaluated in fp32; matrix
 * products run on MFMA with fp32 accumulation (16-bit operands for f16/bf16,
 * fp32 operands for f32); S, z and their gradients are kept in fp32; outputs
 * are rounded to nearest-even into `dtype`. For f16 the fp32 states are
 * scaled by an exact power of two before they become f16 operands and unscaled
 * in fp32 afterwards. Results are bit-identical across runs for identical
 * inputs, problem and device: the work split is a pure function of the shape
 * and every reduction runs in a fixed order (no floating-point atomics).
 */
#ifndef LA_H_
#define LA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_VERSION 9

typedef enum {
    LA_F32 = 0,
    LA_F16 = 1,
    LA_BF16 = 2
} la_dtype;

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL = 1,       /* a required pointer is NULL                      */
    LA_ERR_SHAPE = 2,      /* B, H or T negative; B*H > 2^24; head too large  */
    LA_ERR_DTYPE = 3,      /* dtype not one of la_dtype                       */
    LA_ERR_HEAD_DIM = 4,   /* D, Dv not in {32, 64, 96, 128} nor both 256     */
    LA_ERR_FLAGS = 5,      /* unknown bit in flags, or two feature maps       */
    LA_ERR_EPS = 6,        /* eps negative or not finite                      */
    LA_ERR_WORKSPACE = 7,  /* ws_bytes below la_workspace_bytes()             */
    LA_ERR_ALIGN = 8,      /* a tensor is not 16-byte aligned, ws not 256     */
    LA_ERR_ALIAS = 9,      /* an output overlaps an input or another output   */
    LA_ERR_DEVICE = 10,    /* HIP reported an error on launch                 */
    LA_ERR_SCALE = 11,     /* scale not finite                                */
    LA_ERR_SCRATCH = 12,   /* la_fwd_noalloc: the problem needs more than
                              LA_NOALLOC_SCRATCH_BYTES of scratch             */
    LA_ERR_STRIDE = 13     /* a stride is negative or not a multiple of 16
                              bytes, rows overlap, or an output's rows overlap
                              each other                                      */
} la_status;

/* Drop the denominator: simple_la (FBi-LA README, "Update" 2024-12-28). */
#define LA_SIMPLE 0x1u
/* Tensors are [B, T, H, D] rather than [B, H, T, D]. */
#define LA_LAYOUT_BTHD 0x2u
/* Feature map (at most one; default elu(x) + 1). relu: phi'(0) = 0. With the
 * identity map the normalised denominator phi(q) . z + eps can vanish or
 * change sign; that is the caller's to avoid (simple_la has none). */
#define LA_PHI_RELU 0x4u
#define LA_PHI_IDENTITY 0x8u
/* Causal (autoregressive) attention: token t attends to tokens s <= t,
 *     O_t = phi(q_t) S_t / (phi(q_t) . z_t + eps),  S_t = sum_{s<=t} phi(k_s) v_s^T,
 * z_t = sum_{s<=t} phi(k_s) (flash-linear-attention README, "Different forms
 * of linear attention"). Accepted by la_fwd and la_bwd for every dtype and
 * every D, Dv in {32, 64, 96, 128} (not 256: LA_ERR_HEAD_DIM). f16 and bf16
 * run scans on 16-bit MFMA operands (a head size of 32 or 96 padded to 64 or
 * 128 inside the kernel, the padding never read from or written to memory);
 * fp32 runs scans on fp32 operands.
 * la_fwd's `state` receives the full-sequence S, z, summed over the causal
 * segments in a fixed order: bit-identical to the non-causal call's except at
 * 16-bit D = Dv = 64, whose causal form sums twice as many segments as the
 * non-causal call sums slices (the same values up to the order of the fp32
 * additions). la_bwd does not read `state`. The step calls return
 * LA_ERR_FLAGS with it. la_workspace_bytes counts the causal backward's
 * scratch when the flag is set. */
#define LA_CAUSAL 0x10u
/* With LA_CAUSAL, in la_bwd: `ws` already holds the causal segment prefixes
 * (the exclusive prefix sums of S and z over the segments) that a la_fwd
 * call wrote into it for the same problem (every other field and flag equal)
 * and the same K and V, and nothing has written to `ws` since. la_bwd then
 * reads them from there instead of recomputing them, skipping one pass over
 * K and V (the state reduction and prefix kernels). The workspace works like
 * a reserve space that the forward fills for the backward. The library cannot
 * check the contract: a workspace that does not hold those prefixes gives
 * wrong gradients without an error. la_fwd ignores the bit (it always leaves
 * the prefixes in `ws`), so one problem serves both calls. Without LA_CAUSAL,
 * in la_fwd_noalloc (whose prefixes stay in its own scratch) and in the step
 * calls: LA_ERR_FLAGS. */
#define LA_REUSE_PREFIX 0x20u

/* Strides of one tensor, in elements: element f of token t of head h of
 * batch b sits at base + b*batch + h*head + t*token + f (the D or Dv features
 * of a row are contiguous). */
typedef struct {
    int64_t batch, head, token;
} la_tensor_strides;

/* The strides of every tensor a call may touch; a call reads only the
 * entries of the tensors it takes (la_fwd: q, k, v, o; la_bwd: q, k, v, dout,
 * dq, dk, dv; the step calls their own). Requirements, per tensor used
 * (LA_ERR_STRIDE otherwise): every stride >= 0 and a multiple of 16 bytes;
 * token >= the row width (D or Dv), so rows do not overlap; one head's rows
 * addressable with 32-bit offsets, (T + 1024) * token * elt < 2^31; and for
 * outputs (o, dq, dk, dv) rows that no other (b, h, t) of the same tensor
 * overlaps: taking the dimensions of extent > 1 by increasing stride, each
 * stride at least the span of the ones before it (row width first). Inputs
 * may overlap each other (q, k, v of one packed buffer) and may repeat rows
 * across heads (head = 0). Outputs must not overlap any other buffer of the
 * call, compared by the byte ranges they span. */
typedef struct {
    la_tensor_strides q, k, v, o, dout, dq, dk, dv;
} la_strides;

/* Problem description shared by every call. B, H, T >= 0 (a zero size is an
 * empty problem: nothing to compute, LA_OK), B*H <= 2^24. D is the head size
 * of Q and K (and of dQ, dK), Dv that of V (and of O, dO, dV); 0 in Dv stands
 * for Dv = D. Each of D and Dv is 32, 64, 96 or 128, in any combination, or
 * both are 256 (f16 and bf16 only; not with LA_CAUSAL).
 * eps >= 0 and finite (used only in normalised mode). One head of each tensor
 * must span less than 2^31 bytes, addressed with 32-bit offsets: with
 * M = max(D, Dv), T * M * elt < 2^31 in [B, H, T, *]; (T + 1024) * H * M * elt
 * < 2^31 in [B, T, H, *], where a head's rows are H * M elements apart at most
 * (the 1024 rows keep the offsets of the padded blocks past a slice below 2^31
 * too). elt is the element size.
 * scale (optional) multiplies the query feature: phi(q) is replaced by
 * scale * phi(q) in every formula, as flash-linear-attention's kernels scale
 * the feature-mapped query (the pages give no scale; 0 or 1 leaves the method
 * as stated). In normalised mode this equals eps / scale with no scale; in
 * simple mode it multiplies O and the three gradients. Any finite value; a
 * non-finite one gives LA_ERR_SCALE. The struct is zero-initialisable: a
 * zero scale stands for 1, NULL strides for the dense layout. */
typedef struct {
    int64_t B, H, T, D;
    int64_t Dv;      /* head size of V, O, dO, dV; 0 means D */
    int32_t dtype;   /* la_dtype */
    uint32_t flags;  /* LA_SIMPLE, LA_LAYOUT_BTHD, one of LA_PHI_RELU, LA_PHI_IDENTITY, LA_CAUSAL */
    float eps;
    float scale;     /* multiplies phi(q); 0 stands for 1 (see below)     */
    const la_strides* strides;  /* NULL: dense, as LA_LAYOUT_BTHD says; else
                                   every tensor's strides (LA_LAYOUT_BTHD must
                                   then be clear: LA_ERR_FLAGS) */
} la_problem;

/* Library version (LA_VERSION of the build). */
int la_version(void);

/* Static string naming a status code; never NULL. */
const char* la_status_str(int status);

/* Bytes of the fp32 state: B*H*(D*Dv + D)*4. 0 for an invalid problem. */
size_t la_state_bytes(const la_problem* p);

/* Bytes of workspace that la_fwd, la_bwd and the step calls below need for
 * this problem (the largest of them). 0 for an invalid problem. */
size_t la_workspace_bytes(const la_problem* p);

/* How a problem's tokens are split across workgroups, per step: a pure
 * function of the problem (shape, dtype, flags), the same for every call. The
 * split-T reduction of the forward (steps 1-3; with LA_CAUSAL also the scan
 * segments) cuts each head into P slices of L tokens, the backward's Q side
 * (steps 5-6) into PB slices of LB tokens; the output (step 4) and the
 * backward's K/V side (step 7) run NQ and NK workgroups per head, which take
 * the head's token rounds in turn, about LQ and LK tokens each. The method
 * itself names no split (any split gives the same S, z up to rounding order);
 * this is for logs and benchmarks. */
typedef struct {
    int64_t P, L, PB, LB, NQ, LQ, NK, LK;
} la_split;

/* Fills *out for a valid problem and returns LA_OK; otherwise returns the
 * validation error (LA_ERR_NULL when p or out is NULL) and leaves *out as it
 * was. Makes no HIP call. */
int la_split_of(const la_problem* p, la_split* out);

/* Forward: O (and the state S, z) from Q, K, V (Flash Bi-directional Linear
 * Attention README: the introduction names the operation, "Update"
 * 2024-12-28 its simple_la form, and the Benchmarks table times this call as
 * its fwd column; with LA_CAUSAL, flash-linear-attention README, "Different
 * forms of linear attention"). Runs la_fwd_state, then
 * la_fwd_output. `state` may be NULL when the caller does not keep it; the
 * workspace then holds it. With LA_CAUSAL: the state reduction per token
 * segment, exclusive prefixes of the segment states, then one chunked scan
 * per segment that writes O. */
int la_fwd(const la_problem* p, const void* q, const void* k, const void* v,
           void* o, void* state, void* ws, size_t ws_bytes, void* stream);

/* Backward (Flash Bi-directional Linear Attention README, "Update"
 * 2024-12-30, which names the backward, and the Benchmarks table's bwd
 * column; the pages print no gradient formula, so the gradients are those of
 * the forward's formulas by the chain rule): dQ, dK, dV from Q, K, V, dO and
 * the state la_fwd wrote (the
 * state is required: S and z are not recomputed). Runs la_bwd_dq, then
 * la_bwd_dkv. With LA_CAUSAL: the vector-Jacobian product of sum(O * dO)
 * through the recurrent form (eps held constant); `state` is not read and may
 * be NULL. The segment states and their exclusive prefixes are recomputed
 * from K, V (or, with LA_REUSE_PREFIX, read from the workspace the forward
 * left them in), a forward-order chunked scan per segment writes dQ and keeps
 * 1/den and c per token in the workspace, exclusive suffixes of its
 * per-segment sums follow, and a reverse-order scan writes dK and dV. */
int la_bwd(const la_problem* p, const void* q, const void* k, const void* v,
           const void* dout, const void* state, void* dq, void* dk, void* dv,
           void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch that la_fwd_noalloc uses (64 MiB). */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. la_fwd with the same
 * problem and buffers, computing the same bits, except that the split
 * partials go into a static device array of LA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU from the moment its code loads there until the
 * process ends, instead of a caller workspace. `state` is required here
 * (LA_ERR_NULL without it). The call allocates and frees nothing, and
 * issues no memset: every scratch byte it reads it has written earlier in the
 * same call. A problem that needs more scratch than the array holds gets
 * LA_ERR_SCRATCH and enqueues nothing. A problem needs B*H*P*(D*Dv + D)*4
 * bytes when the planner splits each head into P > 1 token slices, none when
 * P = 1 (as soon as B*H fills the state kernel's grid of 512 to 2048
 * workgroups); every 16-bit problem with D and Dv up to 96 and every fp32
 * problem with D and Dv up to 64 fits, and so do B8-H16-T16384-D64 (4.3 MB;
 * 8.5 MB causal) and B8-H32-T8192-D128 (33.8 MB). The scratch is
 * shared by every la_fwd_noalloc call on a GPU: calls that may overlap in time
 * on one GPU (different streams with no ordering between them, or different
 * host threads) race on it; calls in one stream's order do not. The current
 * device must be the stream's device. The first call on each device looks up
 * the array's address there (no allocation); make that first call outside
 * graph capture. */
int la_fwd_noalloc(const la_problem* p, const void* q, const void* k, const void* v, void* o,
                   void* state, void* stream);

/* ---- The steps of the path, one call each (la_fwd and la_bwd are exactly
 * these calls in order). ---- */

/* Steps 1-3 (the S and z sums of the forward, Flash Bi-directional Linear
 * Attention README, introduction): phi on K, split-T reduction of each head's token range into
 * partial (S, z) on MFMA, then a fixed-order sum of the partials into
 * `state` (non-NULL here). */
int la_fwd_state(const la_problem* p, const void* k, const void* v, void* state,
                 void* ws, size_t ws_bytes, void* stream);

/* Step 4 (the forward's output, Flash Bi-directional Linear Attention README,
 * introduction, and "Update" 2024-12-28 for simple_la):
 * O_t = phi(q_t) S / (phi(q_t) . z + eps) (or phi(q_t) S) from a
 * complete state. Needs no workspace. */
int la_fwd_output(const la_problem* p, const void* q, const void* state, void* o,
                  void* stream);

/* Steps 5-6 (first half of the backward, Flash Bi-directional Linear
 * Attention README, "Update" 2024-12-30): dQ, and the backward state dS = sum_t phi(q_t) (dO_t/den_t)^T,
 * dz = sum_t c_t phi(q_t) (simple_la: dS = phi(Q)^T dO, dz = 0), reduced split-T
 * with a fixed-order combine into the workspace. */
int la_bwd_dq(const la_problem* p, const void* q, const void* dout, const void* state,
              void* dq, void* ws, size_t ws_bytes, void* stream);

/* Step 7 (second half of the backward, same passage):
 * dK = (dS v_t + dz) * phi'(k_t), dV_t = dS^T phi(k_t) (dS is D x Dv), reading the
 * backward state that la_bwd_dq left in the same workspace. */
int la_bwd_dkv(const la_problem* p, const void* k, const void* v, void* dk, void* dv,
               void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H_ */

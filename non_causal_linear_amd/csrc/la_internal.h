// Internal interface between the C-ABI layer (la_api.cpp) and the kernels
// (la_kernels.hip). Not installed; no HIP types leak into include/la.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Where the rows of head bh = b H + h of one tensor live, in elements: the
// head's row 0 at (bh / H) sb + (bh % H) sh, consecutive rows rs apart, the
// row's D elements contiguous.
//   [B, H, T, D]: sb = H T D, sh = T D, rs = D
//   [B, T, H, D]: sb = T H D, sh = D,   rs = H D
//   strided views: the caller's batch, head and token strides
struct Layout {
    int64_t H = 1, sb = 0, sh = 0, rs = 0;
};

// The layout of each tensor of a call: rows of Q, K, dQ, dK hold DK elements,
// rows of V, O, dO, dV hold DV. Dense [B, H, T, D] or [B, T, H, D] unless the
// caller gave strides.
struct Layouts {
    Layout q, k, v, o, dout, dq, dk, dv;
};

// Work split for one problem. Every field is a pure function of
// (B*H, T, DK, DV, dtype), so the summation order, and with it every output
// bit, depends only on the shape.
struct Plan {
    int64_t BH = 0, T = 0;
    int DK = 0, DV = 0, dtype = 0;
    bool simple = false;
    // normalised: eps / scale; simple_la: the query scale (1 without one).
    // Either way the kernels' one float folds the optional query scale.
    float eps = 0.f;
    int fm = 0;  // feature map: 0 elu + 1, 1 relu, 2 identity
    // causal backward: the segment prefixes are already in the workspace
    bool reuse_prefix = false;
    Layouts lay;
    // state reduction (fwd steps 1-3): P slices of L tokens per head
    int P = 1;
    int64_t L = 0;
    // backward Q side (steps 5-6): PB slices of LB tokens per head
    int PB = 1;
    int64_t LB = 0;
    // output (step 4): NQ chunks of LQ tokens per head
    int NQ = 1;
    int64_t LQ = 0;
    // backward K/V side (step 7): NK chunks of LK tokens per head
    int NK = 1;
    int64_t LK = 0;
    // workspace carving (byte offsets)
    size_t off_part = 0, off_dstate = 0, off_fstate = 0;
    // causal backward (LA_CAUSAL): the per-segment (G, g) sums, w and c^ per
    // token, and one exponent per 64-token chunk (nche chunks per segment)
    size_t off_cgpart = 0, off_cwc = 0, off_ces = 0;
    int nche = 0;
    size_t ws_bytes = 0;
};

// How a kernel wants its tokens split: pieces are multiples of `gran` tokens
// (the last one ragged) and the grid should come close to `target_wgs`
// workgroups (what fits resident on the 256 CUs of the chip at once).
struct SplitCfg {
    int64_t gran;
    int64_t target_wgs;
    int64_t max_len = 0;  // if set, more pieces until each holds at most this many tokens
};
// kStepCausalState: the state reduction whose slices are the causal scans'
// segments (the scans run one workgroup per segment, so they want more of them
// than the bidirectional reduction does).
enum Step { kStepState = 0, kStepOutput = 1, kStepBwdQ = 2, kStepBwdKV = 3, kStepCausalState = 4 };

// The launchers of one compilation unit of la_kernels.hip: one element type
// and one DK, every DV (dispatched on Plan::DV). split_config gives the
// token split each step's kernel wants for that DV.
struct KernelSet {
    hipError_t (*fwd_state)(const Plan& p, const void* k, const void* v, float* state, void* ws,
                            hipStream_t s);
    hipError_t (*fwd_output)(const Plan& p, const void* q, const float* state, void* o, hipStream_t s);
    hipError_t (*bwd_dq)(const Plan& p, const void* q, const void* dout, const float* state, void* dq,
                         void* ws, hipStream_t s);
    hipError_t (*bwd_dkv)(const Plan& p, const void* k, const void* v, void* dk, void* dv, void* ws,
                          hipStream_t s);
    SplitCfg (*split_config)(int step, int DV);
    // causal forward (LA_CAUSAL): 16-bit elements, DK and DV in {64, 128}
    hipError_t (*fwd_causal)(const Plan& p, const void* q, const void* k, const void* v, void* o, float* state,
                             void* ws, hipStream_t s);
    // causal backward (LA_CAUSAL), same element types and sizes
    hipError_t (*bwd_causal)(const Plan& p, const void* q, const void* k, const void* v, const void* dout,
                             void* dq, void* dk, void* dv, void* ws, hipStream_t s);
};

// Bytes of the static device scratch of la_fwd_noalloc (LA_NOALLOC_SCRATCH_BYTES).
constexpr size_t kScratchBytes = size_t(64) << 20;

// Device address of that scratch on the current device, looked up with
// hipGetSymbolAddress on the first call per device and kept (la_scratch.hip).
hipError_t scratch_device_ptr(void** out);

// One unit per (la_dtype, DK): kernel_set_<dtype>_<DK>(). DK = 256 exists for
// the 16-bit types only, with DV = 256.
#define LA_KERNEL_UNITS(X) \
    X(0, 32) X(0, 64) X(0, 96) X(0, 128) X(1, 32) X(1, 64) X(1, 96) X(1, 128) \
    X(2, 32) X(2, 64) X(2, 96) X(2, 128) X(1, 256) X(2, 256)
#define LA_DECLARE_UNIT(dt, dk) const KernelSet* kernel_set_##dt##_##dk();
LA_KERNEL_UNITS(LA_DECLARE_UNIT)
#undef LA_DECLARE_UNIT

}  // namespace la

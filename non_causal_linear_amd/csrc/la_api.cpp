// C ABI of the library (declared in include/la.h): argument checks, the work
// planner, workspace carving and the launch sequence of each entry point.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "la.h"
#include "la_internal.h"

namespace {

// Shortest token slice worth a workgroup of its own.
constexpr int64_t kMinSlice = 256;
// Largest B*H accepted (grid sizes stay below 2^31).
constexpr int64_t kMaxHeads = int64_t(1) << 24;
// One head's rows are addressed through a buffer descriptor with 32-bit
// offsets: a head's span must stay below 2^31 bytes. In [B, T, H, D] the
// span is counted with kRowSlack more rows, which covers the padded blocks a
// workgroup may address past the end of its slice.
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - 1;
constexpr int64_t kRowSlack = 1024;
// Largest token count, and the largest caller stride (elements): keeps every
// product of sizes and strides in the checks far from 64-bit overflow.
constexpr int64_t kMaxTokens = int64_t(1) << 40;
constexpr int64_t kMaxStride = int64_t(1) << 46;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Split T tokens of each of BH heads into P pieces of L tokens (L a multiple of
// the kernel's granularity, last piece ragged): P is the largest power of two
// with BH*P within the kernel's target grid and pieces of at least kMinSlice
// tokens. Pure function of the shape.
void split(int64_t BH, int64_t T, la::SplitCfg cfg, int& P, int64_t& L) {
    if (T <= 0 || BH <= 0) {
        P = 1;
        L = 0;
        return;
    }
    const int64_t gran = cfg.gran;
    const int64_t want = std::max<int64_t>(1, cdiv(cfg.target_wgs, BH));
    const int64_t maxp = std::max<int64_t>(1, T / kMinSlice);
    int64_t p = 1;
    while (p * 2 <= want && p * 2 <= maxp) p *= 2;
    while (cfg.max_len > 0 && cdiv(T, p) > cfg.max_len && p * 2 <= maxp) p *= 2;
    L = cdiv(cdiv(T, p), gran) * gran;
    P = static_cast<int>(cdiv(T, L));
}

bool head_size_ok(int64_t d) { return d == 32 || d == 64 || d == 96 || d == 128; }

// Head size of V, O, dO and dV (0 in la_problem stands for D).
int64_t dv_of(const la_problem* p) { return p->Dv ? p->Dv : p->D; }

la_status check_problem(const la_problem* p) {
    if (!p) return LA_ERR_NULL;
    if (p->dtype != LA_F32 && p->dtype != LA_F16 && p->dtype != LA_BF16) return LA_ERR_DTYPE;
    if (p->D == 256 || dv_of(p) == 256) {
        // the wide kernels: both sizes 256, 16-bit elements
        if (p->D != dv_of(p) || p->dtype == LA_F32) return LA_ERR_HEAD_DIM;
    } else if (!head_size_ok(p->D) || !head_size_ok(dv_of(p))) {
        return LA_ERR_HEAD_DIM;
    }
    if (p->B < 0 || p->H < 0 || p->T < 0) return LA_ERR_SHAPE;
    if (p->B > kMaxHeads || p->H > kMaxHeads || p->B * p->H > kMaxHeads) return LA_ERR_SHAPE;
    if (p->flags & ~(LA_SIMPLE | LA_LAYOUT_BTHD | LA_PHI_RELU | LA_PHI_IDENTITY | LA_CAUSAL | LA_REUSE_PREFIX))
        return LA_ERR_FLAGS;
    // the prefixes to reuse are those of the causal form
    if ((p->flags & LA_REUSE_PREFIX) && !(p->flags & LA_CAUSAL)) return LA_ERR_FLAGS;
    if ((p->flags & LA_PHI_RELU) && (p->flags & LA_PHI_IDENTITY)) return LA_ERR_FLAGS;
    if (p->strides && (p->flags & LA_LAYOUT_BTHD)) return LA_ERR_FLAGS;
    if (p->T > kMaxTokens) return LA_ERR_SHAPE;
    const int64_t row_bytes = std::max(p->D, dv_of(p)) * (p->dtype == LA_F32 ? 4 : 2);
    if (p->strides) {
        // checked per tensor by the calls (check_strides)
    } else if (p->flags & LA_LAYOUT_BTHD) {
        if (p->H > 0 && p->T + kRowSlack > kMaxHeadBytes / (p->H * row_bytes)) return LA_ERR_SHAPE;
    } else if (p->T > kMaxHeadBytes / row_bytes) {
        return LA_ERR_SHAPE;
    }
    if (!(p->eps >= 0.f) || !isfinite(p->eps)) return LA_ERR_EPS;
    if (!isfinite(p->scale)) return LA_ERR_SCALE;
    return LA_OK;
}

size_t elem_bytes(int dtype) { return dtype == LA_F32 ? 4 : 2; }

// The tensors of the path. Rows of Q, K, dQ, dK hold D elements, rows of V,
// O, dO, dV hold Dv.
enum Tensor { kQ, kK, kV, kO, kDO, kDQ, kDK, kDV };

int64_t width(const la_problem* p, Tensor t) {
    return (t == kV || t == kO || t == kDO || t == kDV) ? dv_of(p) : p->D;
}

const la_tensor_strides& given_strides(const la_strides* s, Tensor t) {
    switch (t) {
        case kQ: return s->q;
        case kK: return s->k;
        case kV: return s->v;
        case kO: return s->o;
        case kDO: return s->dout;
        case kDQ: return s->dq;
        case kDK: return s->dk;
        default: return s->dv;
    }
}

// Where tensor t's rows live: the caller's strides, else the dense layout the
// flags name.
la::Layout layout_of(const la_problem* p, Tensor t) {
    la::Layout L;
    L.H = p->H > 0 ? p->H : 1;
    const int64_t W = width(p, t);
    if (p->strides) {
        const la_tensor_strides& g = given_strides(p->strides, t);
        L.sb = g.batch;
        L.sh = g.head;
        L.rs = g.token;
    } else if (p->flags & LA_LAYOUT_BTHD) {
        L.sb = p->T * p->H * W;
        L.sh = W;
        L.rs = p->H * W;
    } else {
        L.sb = p->H * p->T * W;
        L.sh = p->T * W;
        L.rs = W;
    }
    return L;
}

// Bytes from the tensor's base to the end of its last element (0 when empty);
// the strides have passed check_strides, so this fits easily in 64 bits.
size_t span_bytes(const la_problem* p, Tensor t) {
    if (p->B == 0 || p->H == 0 || p->T == 0) return 0;
    const la::Layout L = layout_of(p, t);
    const __int128 e = __int128(p->B - 1) * L.sb + __int128(p->H - 1) * L.sh + __int128(p->T - 1) * L.rs + width(p, t);
    return size_t(e * __int128(elem_bytes(p->dtype)));
}

// Caller strides of tensor t (nothing to check for the dense layouts, which
// check_problem covered): non-negative, 16-byte multiples, rows at least a
// row wide, one head addressable with 32-bit offsets (kRowSlack rows of
// padded blocks included), a span well inside 64 bits; and for an output,
// rows that no other (b, h, t) of the tensor overlaps.
la_status check_strides(const la_problem* p, Tensor t, bool output) {
    if (!p->strides) return LA_OK;
    const la::Layout L = layout_of(p, t);
    const int64_t W = width(p, t), elt = static_cast<int64_t>(elem_bytes(p->dtype));
    const int64_t st[3] = {L.rs, L.sh, L.sb};
    for (int64_t x : st)
        if (x < 0 || x > kMaxStride || (x * elt) % 16 != 0) return LA_ERR_STRIDE;
    if (L.rs < W) return LA_ERR_STRIDE;
    if (L.rs * elt > kMaxHeadBytes / (p->T + kRowSlack)) return LA_ERR_STRIDE;
    if (!output) return LA_OK;
    // dimensions of extent > 1 by increasing stride: each stride must clear
    // the span of those before it, which makes every row its own
    struct Dim {
        int64_t extent, stride;
    } d[3] = {{p->T, L.rs}, {p->H, L.sh}, {p->B, L.sb}};
    std::sort(d, d + 3, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
    __int128 span = W;
    for (const Dim& x : d) {
        if (x.extent <= 1) continue;
        if (__int128(x.stride) < span) return LA_ERR_STRIDE;
        span += __int128(x.stride) * (x.extent - 1);
    }
    return LA_OK;
}

// check_strides over the tensors of one call: ins read, outs written.
la_status check_all_strides(const la_problem* p, std::initializer_list<Tensor> ins,
                            std::initializer_list<Tensor> outs) {
    for (Tensor t : ins)
        if (la_status st = check_strides(p, t, false); st != LA_OK) return st;
    for (Tensor t : outs)
        if (la_status st = check_strides(p, t, true); st != LA_OK) return st;
    return LA_OK;
}

// What the causal forward supports, on a problem check_problem accepted.
la_status check_causal(const la_problem* p) {
    // every dtype and head size except 256 (the wide kernels have no causal form)
    if (p->D == 256 || dv_of(p) == 256) return LA_ERR_HEAD_DIM;
    return LA_OK;
}

// Entry points other than la_fwd do not take LA_CAUSAL.
la_status check_not_causal(const la_problem* p) {
    return (p->flags & LA_CAUSAL) ? LA_ERR_FLAGS : LA_OK;
}

// The kernels of one (dtype, DK); the problem has been checked.
const la::KernelSet* kernel_set(int dtype, int DK) {
#define LA_PICK_UNIT(dt, dk) \
    if (dtype == dt && DK == dk) return la::kernel_set_##dt##_##dk();
    LA_KERNEL_UNITS(LA_PICK_UNIT)
#undef LA_PICK_UNIT
    return nullptr;
}

la::Plan make_plan(const la_problem* p) {
    la::Plan pl;
    pl.BH = p->B * p->H;
    pl.T = p->T;
    pl.DK = static_cast<int>(p->D);
    pl.DV = static_cast<int>(dv_of(p));
    pl.dtype = p->dtype;
    pl.simple = (p->flags & LA_SIMPLE) != 0;
    // The query scale s folds into one number the kernels already take:
    // normalised, s phi(q) S / (s phi(q) . z + eps) = phi(q) S / (phi(q) . z + eps / s);
    // simple_la, the output (and every gradient) is s times the unscaled one.
    const float qscale = p->scale == 0.f ? 1.f : p->scale;
    pl.eps = pl.simple ? qscale : p->eps / qscale;
    pl.fm = (p->flags & LA_PHI_RELU) ? 1 : (p->flags & LA_PHI_IDENTITY) ? 2 : 0;
    pl.reuse_prefix = (p->flags & LA_REUSE_PREFIX) != 0;
    pl.lay.q = layout_of(p, kQ);
    pl.lay.k = layout_of(p, kK);
    pl.lay.v = layout_of(p, kV);
    pl.lay.o = layout_of(p, kO);
    pl.lay.dout = layout_of(p, kDO);
    pl.lay.dq = layout_of(p, kDQ);
    pl.lay.dk = layout_of(p, kDK);
    pl.lay.dv = layout_of(p, kDV);
    const la::KernelSet* ks = kernel_set(pl.dtype, pl.DK);
    const bool causal = (p->flags & LA_CAUSAL) != 0;
    split(pl.BH, pl.T, ks->split_config(causal ? la::kStepCausalState : la::kStepState, pl.DV), pl.P, pl.L);
    split(pl.BH, pl.T, ks->split_config(la::kStepBwdQ, pl.DV), pl.PB, pl.LB);
    split(pl.BH, pl.T, ks->split_config(la::kStepOutput, pl.DV), pl.NQ, pl.LQ);
    split(pl.BH, pl.T, ks->split_config(la::kStepBwdKV, pl.DV), pl.NK, pl.LK);
    const size_t E = size_t(pl.DK) * pl.DV + pl.DK;  // floats per (S, z) block
    const int maxp = std::max(pl.P, pl.PB);
    const size_t part = maxp > 1 ? align256(size_t(pl.BH) * maxp * E * 4) : 0;
    const size_t st = align256(size_t(pl.BH) * E * 4);
    pl.off_part = 0;
    pl.off_dstate = part;
    pl.off_fstate = pl.off_dstate + st;
    pl.ws_bytes = pl.off_fstate + st;
    if (causal) {
        // 64-token chunks per segment, rounded up to even (the scans walk chunk pairs)
        pl.nche = static_cast<int>(((pl.L + 63) / 64 + 1) / 2 * 2);
        pl.off_cgpart = pl.ws_bytes;
        pl.off_cwc = pl.off_cgpart + (pl.P > 1 ? align256(size_t(pl.BH) * pl.P * E * 4) : 0);
        pl.off_ces = pl.off_cwc + align256(size_t(pl.BH) * pl.T * 8);
        pl.ws_bytes = pl.off_ces + align256(size_t(pl.BH) * pl.P * pl.nche * 4);
    }
    return pl;
}

struct Span {
    const void* ptr;
    size_t bytes;
};

bool overlaps(Span a, Span b) {
    if (!a.ptr || !b.ptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.ptr), y = reinterpret_cast<uintptr_t>(b.ptr);
    return x < y + b.bytes && y < x + a.bytes;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// Checks pointers of one call. ins/outs: tensors ([B,H,T,D]); outs must not
// overlap anything else listed; every listed pointer must be non-NULL when its
// span is non-empty.
la_status check_buffers(std::initializer_list<Span> ins, std::initializer_list<Span> outs,
                        std::initializer_list<uintptr_t> ins_align, std::initializer_list<uintptr_t> outs_align) {
    auto ia = ins_align.begin();
    for (const Span& s : ins) {
        if (s.bytes && !s.ptr) return LA_ERR_NULL;
        if (s.bytes && !aligned(s.ptr, *ia)) return LA_ERR_ALIGN;
        ++ia;
    }
    auto oa = outs_align.begin();
    for (const Span& s : outs) {
        if (s.bytes && !s.ptr) return LA_ERR_NULL;
        if (s.bytes && !aligned(s.ptr, *oa)) return LA_ERR_ALIGN;
        ++oa;
    }
    for (const Span* o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlaps(*o, i)) return LA_ERR_ALIAS;
        for (const Span* o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(*o, *o2)) return LA_ERR_ALIAS;
    }
    return LA_OK;
}

la_status device_status(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_DEVICE; }

}  // namespace

extern "C" {

int la_version(void) { return LA_VERSION; }

const char* la_status_str(int s) {
    switch (s) {
        case LA_OK: return "LA_OK";
        case LA_ERR_NULL: return "LA_ERR_NULL: required pointer is NULL";
        case LA_ERR_SHAPE: return "LA_ERR_SHAPE: B, H or T negative or too large";
        case LA_ERR_DTYPE: return "LA_ERR_DTYPE: unknown dtype";
        case LA_ERR_HEAD_DIM: return "LA_ERR_HEAD_DIM: D and Dv must be 32, 64, 96 or 128, or both 256 (16-bit)";
        case LA_ERR_FLAGS: return "LA_ERR_FLAGS: unknown flag bit or two feature maps";
        case LA_ERR_EPS: return "LA_ERR_EPS: eps must be finite and >= 0";
        case LA_ERR_SCALE: return "LA_ERR_SCALE: scale must be finite";
        case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace smaller than la_workspace_bytes()";
        case LA_ERR_ALIGN: return "LA_ERR_ALIGN: tensors need 16-byte, workspace 256-byte alignment";
        case LA_ERR_ALIAS: return "LA_ERR_ALIAS: an output overlaps another buffer";
        case LA_ERR_DEVICE: return "LA_ERR_DEVICE: HIP launch error";
        case LA_ERR_STRIDE: return "LA_ERR_STRIDE: a stride is negative, not a 16-byte multiple, or rows overlap";
        case LA_ERR_SCRATCH: return "LA_ERR_SCRATCH: the problem needs more than LA_NOALLOC_SCRATCH_BYTES of scratch";
        default: return "unknown la_status";
    }
}

size_t la_state_bytes(const la_problem* p) {
    if (check_problem(p) != LA_OK) return 0;
    return size_t(p->B * p->H) * size_t(p->D * dv_of(p) + p->D) * 4;
}

size_t la_workspace_bytes(const la_problem* p) {
    if (check_problem(p) != LA_OK) return 0;
    return make_plan(p).ws_bytes;
}

int la_split_of(const la_problem* p, la_split* out) {
    if (!p || !out) return LA_ERR_NULL;
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if ((p->flags & LA_CAUSAL) && (st = check_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    *out = la_split{pl.P, pl.L, pl.PB, pl.LB, pl.NQ, pl.LQ, pl.NK, pl.LK};
    return LA_OK;
}

int la_fwd_state(const la_problem* p, const void* k, const void* v, void* state, void* ws,
                 size_t ws_bytes, void* stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if ((st = check_not_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kK, kV}, {})) != LA_OK) return st;
    const size_t sb = la_state_bytes(p);
    if (pl.BH > 0 && !state) return LA_ERR_NULL;
    if (ws_bytes < pl.ws_bytes) return LA_ERR_WORKSPACE;
    st = check_buffers({{k, span_bytes(p, kK)}, {v, span_bytes(p, kV)}}, {{state, sb}, {ws, pl.ws_bytes}}, {16, 16}, {16, 256});
    if (st != LA_OK) return st;
    if (pl.BH == 0) return LA_OK;
    return device_status(kernel_set(pl.dtype, pl.DK)->fwd_state(pl, k, v, static_cast<float*>(state), ws,
                                              static_cast<hipStream_t>(stream)));
}

int la_fwd_output(const la_problem* p, const void* q, const void* state, void* o, void* stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if ((st = check_not_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kQ}, {kO})) != LA_OK) return st;
    const size_t sb = la_state_bytes(p);
    st = check_buffers({{q, span_bytes(p, kQ)}, {state, sb}}, {{o, span_bytes(p, kO)}}, {16, 16}, {16});
    if (st != LA_OK) return st;
    if (pl.BH == 0 || pl.T == 0) return LA_OK;
    return device_status(kernel_set(pl.dtype, pl.DK)->fwd_output(pl, q, static_cast<const float*>(state), o,
                                               static_cast<hipStream_t>(stream)));
}

int la_fwd(const la_problem* p, const void* q, const void* k, const void* v, void* o, void* state,
           void* ws, size_t ws_bytes, void* stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    const bool causal = (p->flags & LA_CAUSAL) != 0;
    if (causal && (st = check_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kQ, kK, kV}, {kO})) != LA_OK) return st;
    const size_t sb = la_state_bytes(p);
    if (ws_bytes < pl.ws_bytes) return LA_ERR_WORKSPACE;
    st = check_buffers({{q, span_bytes(p, kQ)}, {k, span_bytes(p, kK)}, {v, span_bytes(p, kV)}}, {{o, span_bytes(p, kO)}, {state, state ? sb : 0}, {ws, pl.ws_bytes}},
                       {16, 16, 16}, {16, 16, 256});
    if (st != LA_OK) return st;
    if (pl.BH == 0) return LA_OK;
    float* stp = state ? static_cast<float*>(state)
                       : reinterpret_cast<float*>(static_cast<char*>(ws) + pl.off_fstate);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (causal) return device_status(kernel_set(pl.dtype, pl.DK)->fwd_causal(pl, q, k, v, o, stp, ws, s));
    st = device_status(kernel_set(pl.dtype, pl.DK)->fwd_state(pl, k, v, stp, ws, s));
    if (st != LA_OK || pl.T == 0) return st;
    return device_status(kernel_set(pl.dtype, pl.DK)->fwd_output(pl, q, stp, o, s));
}

int la_fwd_noalloc(const la_problem* p, const void* q, const void* k, const void* v, void* o, void* state,
                   void* stream) {
    static_assert(LA_NOALLOC_SCRATCH_BYTES == la::kScratchBytes, "scratch size in la.h and the library differ");
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    // its prefixes stay in the library's scratch, where no la_bwd can find them
    if (p->flags & LA_REUSE_PREFIX) return LA_ERR_FLAGS;
    const bool causal = (p->flags & LA_CAUSAL) != 0;
    if (causal && (st = check_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kQ, kK, kV}, {kO})) != LA_OK) return st;
    const size_t sb = la_state_bytes(p);
    if (pl.BH > 0 && !state) return LA_ERR_NULL;
    st = check_buffers({{q, span_bytes(p, kQ)}, {k, span_bytes(p, kK)}, {v, span_bytes(p, kV)}}, {{o, span_bytes(p, kO)}, {state, sb}}, {16, 16, 16}, {16, 16});
    if (st != LA_OK) return st;
    // the forward's only scratch: the split partials, at offset 0 (off_part)
    const size_t need = pl.P > 1 ? size_t(pl.BH) * pl.P * (size_t(pl.DK) * pl.DV + pl.DK) * 4 : 0;
    if (need > la::kScratchBytes) return LA_ERR_SCRATCH;
    if (pl.BH == 0) return LA_OK;
    void* ws = nullptr;
    if (la::scratch_device_ptr(&ws) != hipSuccess) return LA_ERR_DEVICE;
    float* stp = static_cast<float*>(state);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (causal) return device_status(kernel_set(pl.dtype, pl.DK)->fwd_causal(pl, q, k, v, o, stp, ws, s));
    st = device_status(kernel_set(pl.dtype, pl.DK)->fwd_state(pl, k, v, stp, ws, s));
    if (st != LA_OK || pl.T == 0) return st;
    return device_status(kernel_set(pl.dtype, pl.DK)->fwd_output(pl, q, stp, o, s));
}

int la_bwd_dq(const la_problem* p, const void* q, const void* dout, const void* state, void* dq,
              void* ws, size_t ws_bytes, void* stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if ((st = check_not_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kQ, kDO}, {kDQ})) != LA_OK) return st;
    const size_t sb = la_state_bytes(p);
    if (pl.BH > 0 && !state) return LA_ERR_NULL;
    if (ws_bytes < pl.ws_bytes) return LA_ERR_WORKSPACE;
    st = check_buffers({{q, span_bytes(p, kQ)}, {dout, span_bytes(p, kDO)}, {state, sb}}, {{dq, span_bytes(p, kDQ)}, {ws, pl.ws_bytes}}, {16, 16, 16},
                       {16, 256});
    if (st != LA_OK) return st;
    if (pl.BH == 0 || pl.T == 0) return LA_OK;
    return device_status(kernel_set(pl.dtype, pl.DK)->bwd_dq(pl, q, dout, static_cast<const float*>(state), dq, ws,
                                           static_cast<hipStream_t>(stream)));
}

int la_bwd_dkv(const la_problem* p, const void* k, const void* v, void* dk, void* dv, void* ws,
               size_t ws_bytes, void* stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if ((st = check_not_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kK, kV}, {kDK, kDV})) != LA_OK) return st;
    if (ws_bytes < pl.ws_bytes) return LA_ERR_WORKSPACE;
    const bool work = pl.BH > 0 && pl.T > 0;
    if (work && !ws) return LA_ERR_NULL;
    st = check_buffers({{k, span_bytes(p, kK)}, {v, span_bytes(p, kV)}, {ws, work ? pl.ws_bytes : 0}},
                       {{dk, span_bytes(p, kDK)}, {dv, span_bytes(p, kDV)}},
                       {16, 16, 256}, {16, 16});
    if (st != LA_OK) return st;
    if (!work) return LA_OK;
    return device_status(kernel_set(pl.dtype, pl.DK)->bwd_dkv(pl, k, v, dk, dv, ws, static_cast<hipStream_t>(stream)));
}

int la_bwd(const la_problem* p, const void* q, const void* k, const void* v, const void* dout,
           const void* state, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    const bool causal = (p->flags & LA_CAUSAL) != 0;
    if (causal && (st = check_causal(p)) != LA_OK) return st;
    const la::Plan pl = make_plan(p);
    if ((st = check_all_strides(p, {kQ, kK, kV, kDO}, {kDQ, kDK, kDV})) != LA_OK) return st;
    const size_t sb = causal ? 0 : la_state_bytes(p);  // the causal backward does not read the state
    if (pl.BH > 0 && !state && !causal) return LA_ERR_NULL;
    if (ws_bytes < pl.ws_bytes) return LA_ERR_WORKSPACE;
    st = check_buffers({{q, span_bytes(p, kQ)}, {k, span_bytes(p, kK)}, {v, span_bytes(p, kV)}, {dout, span_bytes(p, kDO)}, {state, sb}},
                       {{dq, span_bytes(p, kDQ)}, {dk, span_bytes(p, kDK)}, {dv, span_bytes(p, kDV)}, {ws, pl.ws_bytes}}, {16, 16, 16, 16, 16},
                       {16, 16, 16, 256});
    if (st != LA_OK) return st;
    if (pl.BH == 0 || pl.T == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (causal)
        return device_status(kernel_set(pl.dtype, pl.DK)->bwd_causal(pl, q, k, v, dout, dq, dk, dv, ws, s));
    st = device_status(kernel_set(pl.dtype, pl.DK)->bwd_dq(pl, q, dout, static_cast<const float*>(state), dq, ws, s));
    if (st != LA_OK) return st;
    return device_status(kernel_set(pl.dtype, pl.DK)->bwd_dkv(pl, k, v, dk, dv, ws, s));
}

}  // extern "C"

// gdr2_api.hip -- the C ABI of include/gdr2.h: host-side validation, workspace
// sizing and dispatch to the kernel launchers.  Every check runs before any
// launch; a failed check launches nothing and leaves the outputs untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "gdr2.h"
#include "gdr2_internal.h"

namespace {

thread_local char tl_error[512] = "";

gdr2_status fail(gdr2_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(tl_error, sizeof(tl_error), fmt, ap);
    va_end(ap);
    return s;
}

bool debug_sync()
{
    static const bool on = [] {
        const char* e = std::getenv("GDR2_DEBUG");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

gdr2_status hip_check(hipError_t e, hipStream_t stream, const char* what)
{
    if (e == hipSuccess && debug_sync())
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(GDR2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return GDR2_OK;
}

// Product of non-negative sizes with overflow detection.
bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    return !__builtin_mul_overflow(a, b, out);
}

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, int64_t bytes)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(const Range& a, const Range& b)
{
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t elt_bytes(int32_t dtype) { return dtype == GDR2_BF16 ? 2 : 4; }

// Checks shared by both entry points; fills the byte sizes of each tensor.
gdr2_status check_common(int64_t rows, int64_t Dk, int64_t Dv, int32_t dtype, int32_t bw,
                         int32_t ww, int32_t gw)
{
    if (rows < 0)
        return fail(GDR2_ERR_INVALID_ARG, "negative size");
    if (Dk <= 0 || Dv <= 0)
        return fail(GDR2_ERR_INVALID_ARG, "Dk and Dv must be positive (got %lld, %lld)",
                    (long long)Dk, (long long)Dv);
    if (dtype != GDR2_F32 && dtype != GDR2_BF16)
        return fail(GDR2_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (!(bw == 1 || bw == Dk))
        return fail(GDR2_ERR_INVALID_ARG, "b_width must be 1 or Dk (got %d)", bw);
    if (!(ww == 1 || ww == Dv))
        return fail(GDR2_ERR_INVALID_ARG, "w_width must be 1 or Dv (got %d)", ww);
    if (!(gw == 1 || gw == Dk))
        return fail(GDR2_ERR_INVALID_ARG, "g_width must be 1 or Dk (got %d)", gw);
    if (Dk != Dv || (Dk != 64 && Dk != 128))
        return fail(GDR2_ERR_UNSUPPORTED, "supported head dims: Dk == Dv in {64, 128} (got %lld, %lld)",
                    (long long)Dk, (long long)Dv);
    return GDR2_OK;
}

struct TokenTensors {
    const void* q;
    const void* k;
    const void* v;
    const void* b;
    const void* w;
    const float* g;
    const void* o;
};

// Null, alignment and overlap checks for the per-token tensors of `rows`
// token-heads.  `extra` are further output ranges (states).
gdr2_status check_token_ptrs(const TokenTensors& t, int64_t rows, int64_t Dk, int64_t Dv,
                             int32_t dtype, int32_t bw, int32_t ww, int32_t gw,
                             Range* outs, int n_outs)
{
    int64_t e = elt_bytes(dtype), nq, nv, nb, nw, ng;
    if (!mul_ok(rows, Dk * e, &nq) || !mul_ok(rows, Dv * e, &nv) || !mul_ok(rows, bw * e, &nb) ||
        !mul_ok(rows, ww * e, &nw) || !mul_ok(rows, gw * 4, &ng))
        return fail(GDR2_ERR_INVALID_ARG, "tensor size overflows int64");
    const struct {
        const char* name;
        const void* p;
        int64_t bytes;
    } ins[] = {{"q", t.q, nq}, {"k", t.k, nq}, {"v", t.v, nv}, {"b", t.b, nb},
               {"w", t.w, nw}, {"g", t.g, ng}, {"o", t.o, nv}};
    for (const auto& x : ins) {
        if (!x.p)
            return fail(GDR2_ERR_INVALID_ARG, "%s is NULL", x.name);
        if (!aligned16(x.p))
            return fail(GDR2_ERR_INVALID_ARG, "%s is not 16-byte aligned", x.name);
    }
    Range o = range("o", t.o, nv);
    for (int i = 0; i < 6; ++i) {
        Range r = range(ins[i].name, ins[i].p, ins[i].bytes);
        if (overlaps(o, r))
            return fail(GDR2_ERR_INVALID_ARG, "o overlaps input %s", ins[i].name);
        for (int j = 0; j < n_outs; ++j)
            if (overlaps(outs[j], r))
                return fail(GDR2_ERR_INVALID_ARG, "%s overlaps input %s", outs[j].name, ins[i].name);
    }
    for (int j = 0; j < n_outs; ++j)
        if (overlaps(outs[j], o))
            return fail(GDR2_ERR_INVALID_ARG, "%s overlaps o", outs[j].name);
    return GDR2_OK;
}

gdr2_status validate_forward(const gdr2_fwd_args* a, int64_t* state_bytes, bool with_workspace = true)
{
    if (!a)
        return fail(GDR2_ERR_INVALID_ARG, "args is NULL");
    if (a->B < 0 || a->T < 0 || a->H < 0)
        return fail(GDR2_ERR_INVALID_ARG, "B, T, H must be >= 0");
    int64_t bh, rows;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->T, &rows))
        return fail(GDR2_ERR_INVALID_ARG, "B*T*H overflows int64");
    gdr2_status s = check_common(rows, a->Dk, a->Dv, a->dtype, a->b_width, a->w_width, a->g_width);
    if (s != GDR2_OK)
        return s;
    if (a->algo != GDR2_ALGO_AUTO && a->algo != GDR2_ALGO_STAGED && a->algo != GDR2_ALGO_SEGMENTED &&
        a->algo != GDR2_ALGO_FUSED)
        return fail(GDR2_ERR_INVALID_ARG, "unknown algo %d", a->algo);
    if (a->stage != GDR2_STAGE_ALL && a->stage != GDR2_STAGE_PREP && a->stage != GDR2_STAGE_STATE)
        return fail(GDR2_ERR_INVALID_ARG, "unknown stage %d", a->stage);
    if (a->prologue & ~(GDR2_PROLOGUE_NORM_QK | GDR2_PROLOGUE_GATES))
        return fail(GDR2_ERR_INVALID_ARG, "unknown prologue bits 0x%x", a->prologue);
    if (a->chunk != 32 && a->chunk != 64)
        return fail(GDR2_ERR_UNSUPPORTED, "supported chunk sizes: 32, 64 (got %d)", a->chunk);
    if (a->algo == GDR2_ALGO_FUSED && !gdr2::fused_supported(*a))
        return fail(GDR2_ERR_UNSUPPORTED, "GDR2_ALGO_FUSED supports bf16 inputs only");
    if (a->algo == GDR2_ALGO_FUSED && a->stage != GDR2_STAGE_ALL)
        return fail(GDR2_ERR_UNSUPPORTED, "GDR2_ALGO_FUSED has no stages (stage must be GDR2_STAGE_ALL)");
    int64_t nchunks = (a->T + a->chunk - 1) / a->chunk, groups;
    if (!mul_ok(bh, nchunks, &groups) || groups > (int64_t)INT32_MAX)
        return fail(GDR2_ERR_UNSUPPORTED, "too many chunks for one launch");
    if (!mul_ok(bh, a->Dk * a->Dv * 4, state_bytes))
        return fail(GDR2_ERR_INVALID_ARG, "state size overflows int64");
    int64_t ck_bytes;
    if (!mul_ok(*state_bytes, nchunks, &ck_bytes))
        return fail(GDR2_ERR_INVALID_ARG, "S_chunks size overflows int64");
    Range S0 = range("S0", a->S0, *state_bytes), So = range("S_out", a->S_out, *state_bytes);
    Range Sc = range("S_chunks", a->S_chunks, ck_bytes);
    if (a->S_chunks) {
        if (!aligned16(a->S_chunks))
            return fail(GDR2_ERR_INVALID_ARG, "S_chunks must be 16-byte aligned");
        if (overlaps(Sc, S0) || overlaps(Sc, So))
            return fail(GDR2_ERR_INVALID_ARG, "S_chunks overlaps S0 / S_out");
    }
    if ((a->S0 && !aligned16(a->S0)) || (a->S_out && !aligned16(a->S_out)))
        return fail(GDR2_ERR_INVALID_ARG, "S0 / S_out must be 16-byte aligned");
    if (a->S0 && a->S_out && a->S0 != a->S_out && overlaps(S0, So))
        return fail(GDR2_ERR_INVALID_ARG, "S_out partially overlaps S0 (only exact aliasing is allowed)");
    if (rows > 0) {
        TokenTensors t{a->q, a->k, a->v, a->b, a->w, a->g, a->o};
        Range outs[2];
        int n_outs = 0;
        if (a->S_out)
            outs[n_outs++] = So;
        if (a->S_chunks)
            outs[n_outs++] = Sc;
        s = check_token_ptrs(t, rows, a->Dk, a->Dv, a->dtype, a->b_width, a->w_width, a->g_width,
                             outs, n_outs);
        if (s != GDR2_OK)
            return s;
        // S0 is an input as well: o must not overlap it.
        if (overlaps(range("o", a->o, rows * a->Dv * elt_bytes(a->dtype)), S0))
            return fail(GDR2_ERR_INVALID_ARG, "o overlaps input S0");
        size_t need = with_workspace ? gdr2::staged_workspace_bytes(*a) : 0;
        if (need > 0) {
            if (!a->workspace || a->workspace_bytes < need)
                return fail(GDR2_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                            a->workspace ? a->workspace_bytes : (size_t)0);
            if (!aligned16(a->workspace))
                return fail(GDR2_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
            Range ws = range("workspace", a->workspace, (int64_t)need);
            const int64_t e = elt_bytes(a->dtype);
            const Range others[] = {range("q", a->q, rows * a->Dk * e), range("k", a->k, rows * a->Dk * e),
                                    range("v", a->v, rows * a->Dv * e), range("b", a->b, rows * a->b_width * e),
                                    range("w", a->w, rows * a->w_width * e), range("g", a->g, rows * a->g_width * 4),
                                    S0, So, Sc, range("o", a->o, rows * a->Dv * e)};
            for (const auto& r : others)
                if (overlaps(ws, r))
                    return fail(GDR2_ERR_INVALID_ARG, "workspace overlaps %s", r.name);
        }
    }
    return GDR2_OK;
}

// The chunked backward: every check of the forward's inputs plus the
// gradient buffers.  Outputs may overlap nothing, except that dS0 may be the
// same pointer as dS_final.
gdr2_status validate_backward(const gdr2_bwd_args* a)
{
    if (!a)
        return fail(GDR2_ERR_INVALID_ARG, "args is NULL");
    if (a->B < 0 || a->T < 0 || a->H < 0)
        return fail(GDR2_ERR_INVALID_ARG, "B, T, H must be >= 0");
    int64_t bh, rows;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->T, &rows))
        return fail(GDR2_ERR_INVALID_ARG, "B*T*H overflows int64");
    gdr2_status s = check_common(rows, a->Dk, a->Dv, a->dtype, a->b_width, a->w_width, a->g_width);
    if (s != GDR2_OK)
        return s;
    if (a->prologue & ~(GDR2_PROLOGUE_NORM_QK | GDR2_PROLOGUE_GATES))
        return fail(GDR2_ERR_INVALID_ARG, "unknown prologue bits 0x%x", a->prologue);
    if (a->chunk != 64)
        return fail(GDR2_ERR_UNSUPPORTED, "the backward supports chunk 64 only (got %d)", a->chunk);
    if (a->algo != GDR2_ALGO_AUTO && a->algo != GDR2_ALGO_STAGED && a->algo != GDR2_ALGO_SEGMENTED)
        return fail(GDR2_ERR_INVALID_ARG, "unknown algo %d", a->algo);
    if (a->reserved != 0)
        return fail(GDR2_ERR_INVALID_ARG, "reserved must be 0");
    const int64_t nchunks = (a->T + 63) / 64;
    int64_t nrec, state_bytes, ck_bytes;
    // the widest launch has four workgroups per chunk record
    if (!mul_ok(bh, nchunks, &nrec) || nrec > (int64_t)INT32_MAX / 4)
        return fail(GDR2_ERR_UNSUPPORTED, "too many chunks for one launch");
    if (!mul_ok(bh, a->Dk * a->Dv * 4, &state_bytes) || !mul_ok(state_bytes, nchunks, &ck_bytes))
        return fail(GDR2_ERR_INVALID_ARG, "state size overflows int64");
    if (bh == 0)
        return GDR2_OK;
    const int64_t e = elt_bytes(a->dtype);
    int64_t tmp;
    if (!mul_ok(rows, a->Dk * 4, &tmp) || !mul_ok(rows, a->Dv * 4, &tmp))
        return fail(GDR2_ERR_INVALID_ARG, "tensor size overflows int64");
    const int64_t nk = rows * a->Dk, nv = rows * a->Dv;
    const Range ins[] = {range("q", a->q, nk * e), range("k", a->k, nk * e), range("v", a->v, nv * e),
                         range("b", a->b, rows * a->b_width * e), range("w", a->w, rows * a->w_width * e),
                         range("g", a->g, rows * a->g_width * 4), range("S_chunks", a->S_chunks, ck_bytes),
                         range("dO", a->dO, nv * e), range("dS_final", a->dS_final, state_bytes)};
    const Range outs[] = {range("dq", a->dq, nk * 4), range("dk", a->dk, nk * 4), range("dv", a->dv, nv * 4),
                          range("db", a->db, rows * a->b_width * 4), range("dw", a->dw, rows * a->w_width * 4),
                          range("dg", a->dg, rows * a->g_width * 4), range("dS0", a->dS0, state_bytes)};
    const int n_ins = 9, n_outs = 7;
    const bool need_tokens = rows > 0;
    for (int i = 0; i < n_ins; ++i) {
        const bool optional = i == 8 || (!need_tokens && i < 8);
        if (!ins[i].lo && !optional)
            return fail(GDR2_ERR_INVALID_ARG, "%s is NULL", ins[i].name);
        if (ins[i].lo && (ins[i].lo & 15u))
            return fail(GDR2_ERR_INVALID_ARG, "%s is not 16-byte aligned", ins[i].name);
    }
    for (int i = 0; i < n_outs; ++i) {
        const bool optional = i == 6 || !need_tokens;
        if (!outs[i].lo && !optional)
            return fail(GDR2_ERR_INVALID_ARG, "%s is NULL", outs[i].name);
        if (outs[i].lo && (outs[i].lo & 15u))
            return fail(GDR2_ERR_INVALID_ARG, "%s is not 16-byte aligned", outs[i].name);
    }
    for (int i = 0; i < n_outs; ++i) {
        for (int j = 0; j < n_ins; ++j) {
            const bool alias = i == 6 && j == 8 && outs[i].lo == ins[j].lo;
            if (!alias && overlaps(outs[i], ins[j]))
                return fail(GDR2_ERR_INVALID_ARG, "%s overlaps input %s", outs[i].name, ins[j].name);
        }
        for (int j = i + 1; j < n_outs; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(GDR2_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    const size_t need = gdr2::backward_workspace_bytes(*a);
    if (need > 0) {
        if (!a->workspace || a->workspace_bytes < need)
            return fail(GDR2_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                        a->workspace ? a->workspace_bytes : (size_t)0);
        if (!aligned16(a->workspace))
            return fail(GDR2_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
        const Range ws = range("workspace", a->workspace, (int64_t)need);
        for (const auto& r : ins)
            if (overlaps(ws, r))
                return fail(GDR2_ERR_INVALID_ARG, "workspace overlaps %s", r.name);
        for (const auto& r : outs)
            if (overlaps(ws, r))
                return fail(GDR2_ERR_INVALID_ARG, "workspace overlaps %s", r.name);
    }
    return GDR2_OK;
}

}  // namespace

namespace gdr2 {

gdr2_status check_forward_args(const gdr2_fwd_args* a)
{
    int64_t state_bytes = 0;
    return validate_forward(a, &state_bytes, false);
}

gdr2_status set_error(gdr2_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(tl_error, sizeof(tl_error), fmt, ap);
    va_end(ap);
    return s;
}

}  // namespace gdr2

extern "C" {

size_t gdr2_forward_workspace_size(const gdr2_fwd_args* a)
{
    if (!a || a->B < 0 || a->T < 0 || a->H < 0)
        return 0;
    int64_t bh, rows;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->T, &rows) || rows == 0)
        return 0;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128) || (a->chunk != 32 && a->chunk != 64) ||
        (a->dtype != GDR2_F32 && a->dtype != GDR2_BF16) ||
        (a->algo != GDR2_ALGO_AUTO && a->algo != GDR2_ALGO_STAGED && a->algo != GDR2_ALGO_SEGMENTED &&
         a->algo != GDR2_ALGO_FUSED))
        return 0;
    return gdr2::staged_workspace_bytes(*a);
}

gdr2_status gdr2_forward_chunked(const gdr2_fwd_args* a, void* stream_)
{
    int64_t state_bytes = 0;
    gdr2_status s = validate_forward(a, &state_bytes);
    if (s != GDR2_OK)
        return s;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (a->B * a->H == 0)
        return GDR2_OK;
    if (a->T == 0) {
        if (!a->S_out || a->S_out == a->S0)
            return GDR2_OK;
        return hip_check(gdr2::launch_state_copy(a->S0, a->S_out, state_bytes / 4, stream), stream,
                         "state copy");
    }
    if (gdr2::forward_algo(*a) == GDR2_ALGO_FUSED)
        return hip_check(gdr2::launch_forward_fused(*a, stream), stream, "chunked forward (fused)");
    return hip_check(gdr2::launch_forward_staged(*a, stream), stream, "chunked forward");
}

size_t gdr2_backward_workspace_size(const gdr2_bwd_args* a)
{
    if (!a || a->B < 0 || a->T < 0 || a->H < 0)
        return 0;
    int64_t bh, rows;
    if (!mul_ok(a->B, a->H, &bh) || !mul_ok(bh, a->T, &rows) || rows == 0)
        return 0;
    if (a->Dk != a->Dv || (a->Dk != 64 && a->Dk != 128) || a->chunk != 64 ||
        (a->dtype != GDR2_F32 && a->dtype != GDR2_BF16))
        return 0;
    return gdr2::backward_workspace_bytes(*a);
}

gdr2_status gdr2_backward_chunked(const gdr2_bwd_args* a, void* stream_)
{
    gdr2_status s = validate_backward(a);
    if (s != GDR2_OK)
        return s;
    if (a->B * a->H == 0)
        return GDR2_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    return hip_check(gdr2::launch_backward(*a, stream), stream, "chunked backward");
}

gdr2_status gdr2_decode_step(const gdr2_decode_args* a, void* stream_)
{
    if (!a)
        return fail(GDR2_ERR_INVALID_ARG, "args is NULL");
    if (a->N < 0 || a->H < 0)
        return fail(GDR2_ERR_INVALID_ARG, "N, H must be >= 0");
    int64_t rows, state_bytes;
    if (!mul_ok(a->N, a->H, &rows))
        return fail(GDR2_ERR_INVALID_ARG, "N*H overflows int64");
    gdr2_status s = check_common(rows, a->Dk, a->Dv, a->dtype, a->b_width, a->w_width, a->g_width);
    if (s != GDR2_OK)
        return s;
    if (a->prologue & ~(GDR2_PROLOGUE_NORM_QK | GDR2_PROLOGUE_GATES))
        return fail(GDR2_ERR_INVALID_ARG, "unknown prologue bits 0x%x", a->prologue);
    if (a->reserved != 0)
        return fail(GDR2_ERR_INVALID_ARG, "reserved field must be 0");
    if (rows > (int64_t)INT32_MAX)
        return fail(GDR2_ERR_UNSUPPORTED, "too many states for one launch");
    if (!mul_ok(rows, a->Dk * a->Dv * 4, &state_bytes))
        return fail(GDR2_ERR_INVALID_ARG, "state size overflows int64");
    if (rows == 0)
        return GDR2_OK;
    if (!a->state)
        return fail(GDR2_ERR_INVALID_ARG, "state is NULL");
    if (!aligned16(a->state))
        return fail(GDR2_ERR_INVALID_ARG, "state is not 16-byte aligned");
    TokenTensors t{a->q, a->k, a->v, a->b, a->w, a->g, a->o};
    Range outs[1] = {range("state", a->state, state_bytes)};
    s = check_token_ptrs(t, rows, a->Dk, a->Dv, a->dtype, a->b_width, a->w_width, a->g_width, outs, 1);
    if (s != GDR2_OK)
        return s;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    return hip_check(gdr2::launch_decode(*a, stream), stream, "decode step");
}

const char* gdr2_status_string(gdr2_status s)
{
    switch (s) {
    case GDR2_OK: return "ok";
    case GDR2_ERR_INVALID_ARG: return "invalid argument";
    case GDR2_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDR2_ERR_WORKSPACE: return "workspace missing or too small";
    case GDR2_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* gdr2_last_error(void) { return tl_error; }

int gdr2_abi_version(void) { return GDR2_ABI_VERSION; }

}  // extern "C"

// libselscan C ABI: argument checks, launch planning, workspace, launches.
// Every check runs before the first HIP call, so argument errors are
// reported without touching the device (and are testable without a GPU).
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "../../include/selscan.h"
#include "common.hpp"
#include "launch.hpp"

using namespace selscan;

namespace selscan {
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t st);
}

namespace {

constexpr int kVersion = 10500;  // 1.5.0

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};
Span span(const void* p, int64_t bytes) {
    Span s;
    if (p && bytes > 0) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + uintptr_t(bytes);
    }
    return s;
}
bool overlaps(const Span& a, const Span& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Sizes in elements of the tensors of a call; false on overflow.
struct Sizes {
    int64_t seq;    // batch * dim * L        (x, delta, z, y)
    int64_t bc;     // batch * N * L          (B, C)
    int64_t param;  // dim * N                (A)
    int64_t state;  // batch * dim * N        (states)
    int64_t rows;   // batch * dim
};
bool sizes(const selscan_dims_t& d, int64_t L, Sizes* s) {
    int64_t t;
    if (!mul_ok(d.batch, d.dim, &s->rows)) return false;
    if (!mul_ok(s->rows, L, &s->seq) || !mul_ok(s->seq, 4, &t)) return false;
    if (!mul_ok(d.batch, d.dstate, &t) || !mul_ok(t, L, &s->bc) || !mul_ok(s->bc, 4, &t)) return false;
    if (!mul_ok(d.dim, d.dstate, &s->param)) return false;
    if (!mul_ok(s->rows, d.dstate, &s->state) || !mul_ok(s->state, 4, &t)) return false;
    // launch geometry limits: 64-row blocks per grid, 4 lanes per row for the step
    if (s->rows > (int64_t(1) << 36)) return false;
    return true;
}

int check_common(const selscan_dims_t* dims, bool fwd) {
    if (!dims) return SELSCAN_ERR_NULL;
    if (dims->batch < 0 || dims->dim < 0 || dims->dstate < 0 || (fwd && dims->seqlen < 0))
        return SELSCAN_ERR_DIMS;
    if (dims->dtype != SELSCAN_F32 && dims->dtype != SELSCAN_BF16) return SELSCAN_ERR_DTYPE;
    if (dims->dstate != kN) return SELSCAN_ERR_DSTATE;
    return SELSCAN_OK;
}

// Launch plan of a forward call (shared by the call and the workspace query).
// `four_only`: the call asks for checkpoints or the fused convolution, which
// only the 4-wave kernels provide, so the 8-wave choice below is skipped.
int make_plan(const selscan_dims_t* dims, int32_t segments, int32_t groups, int32_t variant,
              bool four_only, FwdPlan* plan) {
    const int64_t L = dims->seqlen;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    *plan = FwdPlan{};
    plan->groups = groups ? groups : 4;
    plan->vec = (L * es) % 16 == 0;
    const int64_t row_blocks = (dims->dim + kWave - 1) / kWave;
    const int64_t nblocks = row_blocks * dims->batch;
    if (variant == 0 && groups == 0 && segments == 0 && !four_only && L % 4 == 0) {
        // The warp-specialised kernel where it measured faster (L 2048 sweeps
        // of batch x d_inner, whole call; fp32 32..1024 row blocks, bf16
        // 48..1024, and long rows with few blocks): fp32 below 1024 blocks
        // (e.g. 192 blocks: 159 against 197 us; 320: 270 against 302; 48 in
        // segments: 85 against 95); bf16 at 160-256 blocks (192: 175 against
        // 203 us) - elsewhere the per-wave kernel's 16-byte bf16 loads win
        // (512 blocks: 294 against 319 us).
        const bool f32 = dims->dtype == SELSCAN_F32;
        if (f32 ? nblocks < 1024 : (nblocks >= 160 && nblocks <= 256)) {
            plan->ws = true;
            if (nblocks < 160) {
                // few blocks: segments (the rule below), operand prefetch
                plan->groups = 4;
                plan->pref = true;
            } else if (f32 && nblocks < 256) {
                // one block per CU: 8 scan waves (two per SIMD), one pass
                plan->groups = 8;
                plan->pref = true;
                segments = 1;
            } else {
                plan->groups = 4;
                segments = 1;
            }
        }
    }
    if (variant >= 2) {
        // the warp-specialised kernel: whole 4-token vectors per row
        if (L % 4 != 0 || four_only) return SELSCAN_ERR_CONFIG;
        plan->ws = true;
        plan->pref = variant == 3;
        if (groups == 0) plan->groups = nblocks <= 256 ? 8 : 4;
    }
    // 8 waves of 2 states per block in one pass, at 160 (fp32) or 208 (bf16)
    // to 256 row blocks. With 4 waves such a grid holds one wave per SIMD (a
    // block per CU); with 8 it holds two, which hide each other's latency,
    // still one block per CU (its LDS). Measured, L 2048, against the 4-wave
    // plan: fp32 191 vs 205-211 us at 192 blocks (segmented), 190 vs 243 at
    // 256; bf16 187 vs 207 at 256, equal at 192 (segmented); worse for both
    // at 128 blocks (segmented 4-wave plans win) and at 512.
    const int64_t blocks = row_blocks * dims->batch;
    const int64_t g8_from = dims->dtype == SELSCAN_F32 ? 160 : 208;
    if (!plan->ws && groups == 0 && segments == 0 && variant < 2 && !four_only && blocks >= g8_from &&
        blocks <= 256) {
        plan->groups = 8;
        plan->segments = 1;
        plan->seg_len = L;
        return SELSCAN_OK;
    }
    // (the specialised kernel counts like 4 waves per block: 4 or 8 scan
    // waves sharing a block's rows)
    const int64_t waves = row_blocks * dims->batch * (plan->ws ? 4 : plan->groups);
    int64_t S = segments;
    if (S == 0) {
        // Segmenting adds a state pass (about 0.7 of an output pass) over all
        // but the last segment, so it pays only when the one-pass grid leaves
        // SIMDs (1024 of them, two resident waves each) idle. Below 512 waves,
        // aim at two waves per SIMD (2048). Between 512 and 832 the counts
        // below were the fastest of 1..6 in a sweep (L 2048, bf16): a grid
        // just over one round of 2048 waves leaves a small, slow last round,
        // so 3 segments at 640 waves (1,920) but 5 at 704 or 768. From 832
        // waves on, one pass was fastest.
        S = 1;
        if (L >= 16 * kChunk) {
            if (waves < 512) S = (2048 + waves - 1) / waves;
            else if (waves <= 544) S = 4;
            else if (waves <= 682) S = 3;
            else if (waves < 832) S = 5;
            const int64_t max_by_len = L / (8 * kChunk);
            if (S > max_by_len) S = max_by_len;
            if (S < 1) S = 1;
        }
    }
    if (S > 1 && L > 0) {
        int64_t seg_len = (L + S - 1) / S;
        seg_len = (seg_len + kChunk - 1) / kChunk * kChunk;
        S = (L + seg_len - 1) / seg_len;
        plan->seg_len = seg_len;
    } else {
        S = 1;
        plan->seg_len = L;
    }
    plan->segments = int32_t(S);
    if (int64_t(plan->segments) * row_blocks * dims->batch > INT32_MAX) return SELSCAN_ERR_DIMS;
    return SELSCAN_OK;
}

int check_opts(const selscan_fwd_opts_t& o) {
    if (o.segments < 0 || o.segments > 65536) return SELSCAN_ERR_CONFIG;
    if (o.groups != 0 && o.groups != 1 && o.groups != 2 && o.groups != 4 && o.groups != 8)
        return SELSCAN_ERR_CONFIG;
    if (o.ckpt && o.groups != 0 && o.groups != 4) return SELSCAN_ERR_CONFIG;  // 4 waves store them
    // the convolution in front: 4 waves, not with checkpoints, its other inputs only with taps
    if (o.conv_w && ((o.groups != 0 && o.groups != 4) || o.ckpt)) return SELSCAN_ERR_CONFIG;
    if (o.variant < 0 || o.variant > 3) return SELSCAN_ERR_CONFIG;
    // the specialised kernel: 4 or 8 scan waves, no checkpoints, no convolution
    if (o.variant >= 2 && ((o.groups != 0 && o.groups != 4 && o.groups != 8) || o.ckpt || o.conv_w))
        return SELSCAN_ERR_CONFIG;
    if (!o.conv_w && (o.conv_b || o.conv_x_prev || o.conv_x_last)) return SELSCAN_ERR_CONFIG;
    return SELSCAN_OK;
}

int check_fwd_dims(const selscan_dims_t* dims, Sizes* sz) {
    int rc = check_common(dims, true);
    if (rc != SELSCAN_OK) return rc;
    // The kernels address B/C rows with 32-bit offsets of up to N*L elements.
    if (dims->seqlen >= (int64_t(1) << 27)) return SELSCAN_ERR_DIMS;
    if (!sizes(*dims, dims->seqlen, sz)) return SELSCAN_ERR_DIMS;
    return SELSCAN_OK;
}

// Measurement hook state (selscan_timing_*). One pair of events per launch.
struct Timing {
    bool on = false;
    int32_t used = 0;
    std::vector<hipEvent_t> ev;  // 2 per launch, created once, kept for reuse
};
Timing g_timing;

// The next unused event pair, or nulls when not timing or full.
void next_events(hipEvent_t* b, hipEvent_t* e) {
    *b = *e = nullptr;
    if (!g_timing.on || 2 * size_t(g_timing.used + 1) > g_timing.ev.size()) return;
    *b = g_timing.ev[2 * g_timing.used];
    *e = g_timing.ev[2 * g_timing.used + 1];
    ++g_timing.used;
}

// The no-allocation forward's scratch: a file-scope device array, one copy per
// GPU, held until the process ends. Host code never uses the array's name as
// an address (on the host it is only a stand-in for the symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(SELSCAN_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchTable {
    std::mutex m;
    void* ptr[64] = {};  // per device ordinal; null until looked up
};
ScratchTable g_scratch;

// The current device's copy of the scratch array, or null on failure.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch.m);
    if (!g_scratch.ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch.ptr[dev] = p;
    }
    return g_scratch.ptr[dev];
}

// noalloc: the workspace is the device's scratch array (SELSCAN_ERR_SCRATCH
// when the call needs more); nothing is allocated.
int fwd_impl(const void* x, const void* delta, const float* A, const void* B, const void* C,
             const float* D, const void* z, const float* dt_bias, void* y, float* last_state,
             const selscan_dims_t* dims, const selscan_fwd_opts_t* opts, void* stream,
             bool noalloc = false) {
    Sizes sz;
    int rc = check_fwd_dims(dims, &sz);
    if (rc != SELSCAN_OK) return rc;
    const selscan_fwd_opts_t o = opts ? *opts : selscan_fwd_opts_t{};
    rc = check_opts(o);
    if (rc != SELSCAN_OK) return rc;
    const int64_t L = dims->seqlen;
    // A tensor with no elements may come with a null pointer (torch gives one).
    if ((sz.seq > 0 && (!x || !delta || !y)) || (sz.bc > 0 && (!B || !C)) || (sz.param > 0 && !A))
        return SELSCAN_ERR_NULL;
    for (const void* p : {x, delta, (const void*)A, B, C, (const void*)D, z, (const void*)dt_bias, (const void*)y,
                          (const void*)last_state, (const void*)o.h0, (const void*)o.ckpt,
                          (const void*)o.conv_w, (const void*)o.conv_b, (const void*)o.conv_x_prev,
                          (const void*)o.conv_x_last})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    if (o.workspace && (reinterpret_cast<uintptr_t>(o.workspace) & 255u)) return SELSCAN_ERR_CONFIG;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    const Span out_y = span(y, sz.seq * es), out_s = span(last_state, sz.state * 4);
    const Span ins[] = {span(x, sz.seq * es),      span(delta, sz.seq * es), span(z, sz.seq * es),
                        span(B, sz.bc * es),       span(C, sz.bc * es),      span(A, sz.param * 4),
                        span(D, dims->dim * 4),    span(dt_bias, dims->dim * 4)};
    for (const Span& s : ins)
        if (overlaps(s, out_y) || overlaps(s, out_s)) return SELSCAN_ERR_ALIAS;
    if (overlaps(out_y, out_s)) return SELSCAN_ERR_ALIAS;
    // h0 may be last_state itself (each row's state is read before it is
    // written), but no other overlap with an output.
    const Span in_h0 = span(o.h0, sz.state * 4);
    if (overlaps(in_h0, out_y)) return SELSCAN_ERR_ALIAS;
    if (overlaps(in_h0, out_s) && static_cast<const void*>(o.h0) != static_cast<const void*>(last_state))
        return SELSCAN_ERR_ALIAS;
    // checkpoints: an output of ceil(L/16) states per row
    int64_t ck_bytes = 0;
    if (o.ckpt && !mul_ok((L + 15) / 16, sz.state * 4, &ck_bytes)) return SELSCAN_ERR_DIMS;
    const Span out_c = span(o.ckpt, ck_bytes);
    for (const Span& s : ins)
        if (overlaps(s, out_c)) return SELSCAN_ERR_ALIAS;
    if (overlaps(out_c, out_y) || overlaps(out_c, out_s) || overlaps(out_c, in_h0))
        return SELSCAN_ERR_ALIAS;
    // the convolution: x_last is an output (it may be x_prev itself)
    const Span in_cw = span(o.conv_w, dims->dim * 16), in_cb = span(o.conv_b, dims->dim * 4);
    const Span in_cp = span(o.conv_x_prev, sz.rows * 12), out_cl = span(o.conv_x_last, sz.rows * 12);
    for (const Span& s : {in_cw, in_cb, in_cp})
        if (overlaps(s, out_y) || overlaps(s, out_s) || overlaps(s, out_c)) return SELSCAN_ERR_ALIAS;
    for (const Span& s : ins)
        if (overlaps(s, out_cl)) return SELSCAN_ERR_ALIAS;
    if (overlaps(out_cl, out_y) || overlaps(out_cl, out_s) || overlaps(out_cl, in_h0) ||
        overlaps(out_cl, in_cw) || overlaps(out_cl, in_cb))
        return SELSCAN_ERR_ALIAS;
    if (overlaps(out_cl, in_cp) &&
        static_cast<const void*>(o.conv_x_last) != static_cast<const void*>(o.conv_x_prev))
        return SELSCAN_ERR_ALIAS;

    FwdPlan plan{};
    rc = make_plan(dims, o.segments, o.groups, o.variant, o.ckpt || o.conv_w, &plan);
    if (rc != SELSCAN_OK) return rc;
    FwdShape shape{dims->batch, L, dims->dim, dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32};
    const size_t ws_bytes = (sz.rows > 0 && L > 0) ? fwd_workspace_bytes(shape, plan) : 0;
    if (o.workspace && o.workspace_bytes < ws_bytes) return SELSCAN_ERR_CONFIG;
    if (o.workspace) {
        // the workspace must be nobody else's memory
        const Span w = span(o.workspace, int64_t(ws_bytes));
        for (const Span& s : ins)
            if (overlaps(s, w)) return SELSCAN_ERR_ALIAS;
        for (const Span& s : {out_y, out_s, in_h0, out_c, in_cw, in_cb, in_cp, out_cl})
            if (overlaps(s, w)) return SELSCAN_ERR_ALIAS;
    }
    if (noalloc && ws_bytes > kScratchBytes) return SELSCAN_ERR_SCRATCH;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (sz.rows == 0) return SELSCAN_OK;
    if (L == 0) {
        if (o.conv_x_last) {  // no new inputs: the last three are the previous ones
            const hipError_t e = o.conv_x_prev ? launch_copy_f32(o.conv_x_last, o.conv_x_prev, sz.rows * 3, st)
                                               : launch_fill_zero(o.conv_x_last, sz.rows * 3, st);
            if (e != hipSuccess) return SELSCAN_ERR_LAUNCH;
        }
        if (!last_state) return SELSCAN_OK;
        const hipError_t e = o.h0 ? launch_copy_f32(last_state, o.h0, sz.state, st)
                                  : launch_fill_zero(last_state, sz.state, st);
        return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
    }

    FwdTensors t{x, delta, z, A, B, C, D, dt_bias, y, last_state, o.h0, o.ckpt,
                 o.conv_w, o.conv_b, o.conv_x_prev, o.conv_x_last};
    void* ws = o.workspace;
    if (noalloc) {
        // every byte of the workspace that a kernel reads is written first by
        // an earlier kernel of the same call, so no clearing is needed
        ws = scratch_for_current_device();
        if (!ws) return SELSCAN_ERR_LAUNCH;
    }
    next_events(&plan.ev_begin, &plan.ev_end);
    const bool own = ws == nullptr;
    if (own) {
        if (hipMallocAsync(&ws, ws_bytes, st) != hipSuccess || !ws) {
            (void)hipGetLastError();
            return SELSCAN_ERR_ALLOC;
        }
    }
    const hipError_t e = launch_fwd(t, shape, plan, ws, st);
    if (own) (void)hipFreeAsync(ws, st);
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

// Segments of a backward call (the reverse sweep runs 4 waves per 64-row
// block, two blocks per CU); a segmented call adds a state pass and a carry
// sweep, each over all but one segment, which cost less against the reverse
// pass than the forward's state pass does against its output pass, so
// segments pay up to larger grids. Below 512 waves: two waves per SIMD;
// from 512 to 1279 the fastest counts of a sweep (L 2048, bf16); from 1280
// waves on, one sweep.
void bwd_segments(const selscan_dims_t* dims, int32_t requested, int32_t* segments,
                  int64_t* seg_len) {
    const int64_t L = dims->seqlen;
    const int64_t waves = (dims->dim + kWave - 1) / kWave * dims->batch * 4;
    int64_t S = requested;
    if (S == 0) {
        S = 1;
        if (L >= 16 * kChunk) {
            if (waves < 512) S = (2048 + waves - 1) / waves;
            else if (waves <= 544) S = 4;
            else if (waves < 736) S = 5;
            else if (waves < 960) S = 6;
            else if (waves < 1152) S = 2;
            else if (waves < 1280) S = 3;
            const int64_t max_by_len = L / (8 * kChunk);
            if (S > max_by_len) S = max_by_len;
            if (S < 1) S = 1;
        }
    }
    *seg_len = L;
    if (S > 1 && L > 0) {
        int64_t len = (L + S - 1) / S;
        len = (len + kChunk - 1) / kChunk * kChunk;
        S = (L + len - 1) / len;
        *seg_len = S > 1 ? len : L;
    }
    *segments = int32_t(S > 1 ? S : 1);
}

}  // namespace

extern "C" {

int selscan_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, void* y, float* last_state,
                const selscan_dims_t* dims, void* stream) {
    return fwd_impl(x, delta, A, B, C, D, z, dt_bias, y, last_state, dims, nullptr, stream);
}

int selscan_fwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* dt_bias, void* y,
                   float* last_state, const selscan_dims_t* dims,
                   const selscan_fwd_opts_t* opts, void* stream) {
    return fwd_impl(x, delta, A, B, C, D, z, dt_bias, y, last_state, dims, opts, stream);
}

int selscan_fwd_noalloc(const void* x, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        void* y, float* last_state, const selscan_dims_t* dims, void* stream) {
    return fwd_impl(x, delta, A, B, C, D, z, dt_bias, y, last_state, dims, nullptr, stream, true);
}

int selscan_fwd_workspace_size(const selscan_dims_t* dims, const selscan_fwd_opts_t* opts,
                               uint64_t* bytes) {
    if (!bytes) return SELSCAN_ERR_NULL;
    Sizes sz;
    int rc = check_fwd_dims(dims, &sz);
    if (rc != SELSCAN_OK) return rc;
    const selscan_fwd_opts_t o = opts ? *opts : selscan_fwd_opts_t{};
    rc = check_opts(o);
    if (rc != SELSCAN_OK) return rc;
    FwdPlan plan{};
    rc = make_plan(dims, o.segments, o.groups, o.variant, o.ckpt || o.conv_w, &plan);
    if (rc != SELSCAN_OK) return rc;
    FwdShape shape{dims->batch, dims->seqlen, dims->dim,
                   dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32};
    *bytes = (sz.rows > 0 && dims->seqlen > 0) ? fwd_workspace_bytes(shape, plan) : 0;
    return SELSCAN_OK;
}

int selscan_step(float* state, const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, void* y,
                 const selscan_dims_t* dims, void* stream) {
    return selscan_step_ex(state, x, delta, A, B, C, D, z, y, dims, nullptr, stream);
}

int selscan_step_ex(float* state, const void* x, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, void* y,
                    const selscan_dims_t* dims, const selscan_step_opts_t* opts, void* stream) {
    int rc = check_common(dims, false);
    if (rc != SELSCAN_OK) return rc;
    Sizes sz;
    if (!sizes(*dims, 1, &sz)) return SELSCAN_ERR_DIMS;
    const selscan_step_opts_t o = opts ? *opts : selscan_step_opts_t{};
    if ((o.conv_b && !o.conv_w) || (o.conv_w && !o.conv_state && sz.rows > 0) ||
        (o.conv_state && !o.conv_w))
        return SELSCAN_ERR_CONFIG;
    // A tensor with no elements may come with a null pointer (torch gives one).
    if ((sz.rows > 0 && (!state || !x || !delta || !y)) || (dims->batch > 0 && (!B || !C)) ||
        (sz.param > 0 && !A))
        return SELSCAN_ERR_NULL;
    for (const void* p : {(const void*)state, x, delta, (const void*)A, B, C, (const void*)D, z, (const void*)y,
                          (const void*)o.conv_w, (const void*)o.conv_b, (const void*)o.conv_state})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    const Span out_y = span(y, sz.rows * es), io_s = span(state, sz.state * 4),
               io_c = span(o.conv_state, sz.rows * 12);
    const Span ins[] = {span(x, sz.rows * es), span(delta, sz.rows * es), span(z, sz.rows * es),
                        span(B, dims->batch * kN * es), span(C, dims->batch * kN * es),
                        span(A, sz.param * 4), span(D, dims->dim * 4),
                        span(o.conv_w, dims->dim * 16), span(o.conv_b, dims->dim * 4)};
    for (const Span& s : ins)
        if (overlaps(s, out_y) || overlaps(s, io_s) || overlaps(s, io_c)) return SELSCAN_ERR_ALIAS;
    if (overlaps(out_y, io_s) || overlaps(out_y, io_c) || overlaps(io_s, io_c)) return SELSCAN_ERR_ALIAS;
    if (sz.rows == 0) return SELSCAN_OK;
    StepTensors t{state, x, delta, A, B, C, D, z, y, o.conv_w, o.conv_b, o.conv_state};
    hipEvent_t eb, ee;
    next_events(&eb, &ee);
    const hipError_t e = launch_step(t, dims->batch, dims->dim,
                                     dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32,
                                     static_cast<hipStream_t>(stream), eb, ee);
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

int selscan_timing_start(int32_t capacity) {
    if (capacity < 1 || capacity > 65536) return SELSCAN_ERR_CONFIG;
    while (g_timing.ev.size() < 2 * size_t(capacity)) {
        hipEvent_t ev;
        if (hipEventCreate(&ev) != hipSuccess) {
            (void)hipGetLastError();
            return SELSCAN_ERR_LAUNCH;
        }
        g_timing.ev.push_back(ev);
    }
    g_timing.on = true;
    g_timing.used = 0;
    return SELSCAN_OK;
}

int selscan_timing_stop(double* total_ms, int32_t* launches) {
    if (!total_ms || !launches) return SELSCAN_ERR_NULL;
    if (!g_timing.on) return SELSCAN_ERR_CONFIG;
    g_timing.on = false;
    double sum = 0.0;
    for (int32_t i = 0; i < g_timing.used; ++i) {
        float ms = 0.0f;
        if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess) {
            (void)hipGetLastError();
            return SELSCAN_ERR_LAUNCH;
        }
        sum += ms;
    }
    *total_ms = sum;
    *launches = g_timing.used;
    return SELSCAN_OK;
}

int selscan_bwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* dt_bias, const void* dy, void* dx,
                void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddt_bias,
                const selscan_dims_t* dims, void* stream) {
    return selscan_bwd_ex(x, delta, A, B, C, D, z, dt_bias, dy, dx, ddelta, dA, dB, dC, dD, dz,
                          ddt_bias, dims, nullptr, stream);
}

int selscan_bwd_ex(const void* x, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* dt_bias, const void* dy, void* dx,
                   void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                   float* ddt_bias, const selscan_dims_t* dims, const selscan_bwd_opts_t* opts,
                   void* stream) {
    const selscan_bwd_opts_t o = opts ? *opts : selscan_bwd_opts_t{};
    if (o.workspace && (reinterpret_cast<uintptr_t>(o.workspace) & 255u)) return SELSCAN_ERR_CONFIG;
    if (o.segments < 0 || o.segments > 65536) return SELSCAN_ERR_CONFIG;
    Sizes sz;
    int rc = check_fwd_dims(dims, &sz);
    if (rc != SELSCAN_OK) return rc;
    int64_t ck_bytes = 0;
    if (o.ckpt && !mul_ok((dims->seqlen + 15) / 16, sz.state * 4, &ck_bytes)) rc = SELSCAN_ERR_DIMS;
    if (rc != SELSCAN_OK) return rc;
    const int64_t L = dims->seqlen;
    if ((sz.seq > 0 && (!x || !delta || !dy || !dx || !ddelta)) || (sz.bc > 0 && (!B || !C || !dB || !dC)) ||
        (sz.param > 0 && (!A || !dA)))
        return SELSCAN_ERR_NULL;
    if (z && sz.seq > 0 && !dz) return SELSCAN_ERR_NULL;
    if (!z && dz) return SELSCAN_ERR_NULL;  // dz has no meaning without a gate
    for (const void* p : {x, delta, (const void*)A, B, C, (const void*)D, z, (const void*)dt_bias, dy,
                          (const void*)dx, (const void*)ddelta, (const void*)dA, (const void*)dB,
                          (const void*)dC, (const void*)dD, (const void*)dz, (const void*)ddt_bias,
                          (const void*)o.h0, (const void*)o.dlast_state, (const void*)o.dh0,
                          (const void*)o.ckpt})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    const Span outs[] = {span(dx, sz.seq * es), span(ddelta, sz.seq * es), span(dz, sz.seq * es),
                         span(dB, sz.bc * es),  span(dC, sz.bc * es),     span(dA, sz.param * 4),
                         span(dD, dims->dim * 4), span(ddt_bias, dims->dim * 4),
                         span(o.dh0, sz.state * 4)};
    const Span ins[] = {span(x, sz.seq * es), span(delta, sz.seq * es), span(z, sz.seq * es),
                        span(dy, sz.seq * es), span(B, sz.bc * es),     span(C, sz.bc * es),
                        span(A, sz.param * 4), span(D, dims->dim * 4),  span(dt_bias, dims->dim * 4),
                        span(o.h0, sz.state * 4), span(o.dlast_state, sz.state * 4),
                        span(o.ckpt, ck_bytes)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span& s : ins)
            if (overlaps(s, outs[i])) return SELSCAN_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlaps(outs[i], outs[j])) return SELSCAN_ERR_ALIAS;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (sz.rows == 0 || L == 0) {  // no terms: the per-channel sums are zero
        if (launch_fill_zero(dA, sz.param, st) != hipSuccess) return SELSCAN_ERR_LAUNCH;
        if (dD && launch_fill_zero(dD, dims->dim, st) != hipSuccess) return SELSCAN_ERR_LAUNCH;
        if (ddt_bias && launch_fill_zero(ddt_bias, dims->dim, st) != hipSuccess) return SELSCAN_ERR_LAUNCH;
        // the final state is h0 itself: its gradient passes straight through
        if (o.dh0) {
            const hipError_t e = o.dlast_state ? launch_copy_f32(o.dh0, o.dlast_state, sz.state, st)
                                               : launch_fill_zero(o.dh0, sz.state, st);
            if (e != hipSuccess) return SELSCAN_ERR_LAUNCH;
        }
        return SELSCAN_OK;
    }
    int32_t segments = 1;
    int64_t seg_len = L;
    bwd_segments(dims, o.segments, &segments, &seg_len);
    if ((L + 15) / 16 * ((dims->dim + kWave - 1) / kWave) > INT32_MAX ||
        ((dims->dim + kWave - 1) / kWave) * dims->batch * segments > INT32_MAX)
        return SELSCAN_ERR_DIMS;
    const size_t ws_bytes = bwd_workspace_bytes(dims->batch, L, dims->dim, segments, o.ckpt != nullptr);
    if (o.workspace) {
        if (o.workspace_bytes < ws_bytes) return SELSCAN_ERR_CONFIG;
        const Span w = span(o.workspace, int64_t(ws_bytes));
        for (const Span& s : outs)
            if (overlaps(s, w)) return SELSCAN_ERR_ALIAS;
        for (const Span& s : ins)
            if (overlaps(s, w)) return SELSCAN_ERR_ALIAS;
    }
    void* ws = o.workspace;
    const bool own = ws == nullptr;
    if (own && (hipMallocAsync(&ws, ws_bytes, st) != hipSuccess || !ws)) {
        (void)hipGetLastError();
        return SELSCAN_ERR_ALLOC;
    }
    BwdTensors t{x,  delta, A,  B,  C,  D,  z,        dt_bias, dy,
                 dx, ddelta, dA, dB, dC, dD, dz, ddt_bias, o.h0, o.dlast_state, o.dh0, o.ckpt};
    const hipError_t e = launch_bwd(t, dims->batch, L, dims->dim,
                                    dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32,
                                    segments, seg_len, ws, st);
    if (own) (void)hipFreeAsync(ws, st);
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

int selscan_bwd_workspace_size(const selscan_dims_t* dims, const selscan_bwd_opts_t* opts,
                               uint64_t* bytes) {
    if (!bytes) return SELSCAN_ERR_NULL;
    Sizes sz;
    const int rc = check_fwd_dims(dims, &sz);
    if (rc != SELSCAN_OK) return rc;
    const selscan_bwd_opts_t o = opts ? *opts : selscan_bwd_opts_t{};
    if (o.segments < 0 || o.segments > 65536) return SELSCAN_ERR_CONFIG;
    *bytes = 0;
    if (sz.rows == 0 || dims->seqlen == 0) return SELSCAN_OK;
    int32_t segments = 1;
    int64_t seg_len = dims->seqlen;
    bwd_segments(dims, o.segments, &segments, &seg_len);
    *bytes = bwd_workspace_bytes(dims->batch, dims->seqlen, dims->dim, segments, o.ckpt != nullptr);
    return SELSCAN_OK;
}

int selscan_ssd_fwd(const void* x, const void* delta, const float* A, const void* B, const void* C,
                    const float* D, const float* dt_bias, void* y, float* last_state,
                    const selscan_ssd_dims_t* dims, void* stream) {
    return selscan_ssd_fwd_ex(x, delta, A, B, C, D, dt_bias, nullptr, y, last_state, dims, stream);
}

int selscan_ssd_fwd_ex(const void* x, const void* delta, const float* A, const void* B,
                       const void* C, const float* D, const float* dt_bias, const float* h0,
                       void* y, float* last_state, const selscan_ssd_dims_t* dims, void* stream) {
    if (!dims) return SELSCAN_ERR_NULL;
    if (dims->batch < 0 || dims->seqlen < 0 || dims->heads < 0 || dims->headdim < 0 || dims->dstate < 0)
        return SELSCAN_ERR_DIMS;
    if (dims->dtype != SELSCAN_BF16) return SELSCAN_ERR_DTYPE;
    if (dims->headdim != 64 || (dims->dstate != 64 && dims->dstate != 128)) return SELSCAN_ERR_DSTATE;
    if (dims->seqlen >= (int64_t(1) << 27)) return SELSCAN_ERR_DIMS;
    int64_t bl, seq, bh, st, t;
    if (!mul_ok(dims->batch, dims->seqlen, &bl) || !mul_ok(bl, dims->heads * 64, &seq) ||
        !mul_ok(seq, 4, &t) || !mul_ok(dims->batch, dims->heads, &bh) ||
        !mul_ok(bh, 64 * dims->dstate, &st) || !mul_ok(st, 4, &t) || bh > (int64_t(1) << 31) ||
        dims->heads > (int64_t(1) << 20))
        return SELSCAN_ERR_DIMS;
    const int64_t nc = (dims->seqlen + 63) / 64;
    if (bh * nc > INT32_MAX) return SELSCAN_ERR_DIMS;
    const int64_t nbc = bl * dims->dstate;  // elements of B, C
    if ((seq > 0 && (!x || !y)) || (bl * dims->heads > 0 && !delta) || (nbc > 0 && (!B || !C)) ||
        (dims->heads > 0 && !A))
        return SELSCAN_ERR_NULL;
    for (const void* p : {x, delta, (const void*)A, B, C, (const void*)D, (const void*)dt_bias, (const void*)y,
                          (const void*)last_state, (const void*)h0})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const Span oy = span(y, seq * 2), os = span(last_state, st * 4);
    // h0 may be last_state itself (each (b, h) reads it before writing it)
    const Span ih = span(h0, st * 4);
    if (overlaps(ih, oy)) return SELSCAN_ERR_ALIAS;
    if (overlaps(ih, os) && static_cast<const void*>(h0) != static_cast<const void*>(last_state))
        return SELSCAN_ERR_ALIAS;
    const Span ins[] = {span(x, seq * 2), span(delta, bl * dims->heads * 2), span(A, dims->heads * 4),
                        span(B, nbc * 2), span(C, nbc * 2), span(D, dims->heads * 4),
                        span(dt_bias, dims->heads * 4)};
    for (const Span& s : ins)
        if (overlaps(s, oy) || overlaps(s, os)) return SELSCAN_ERR_ALIAS;
    if (overlaps(oy, os)) return SELSCAN_ERR_ALIAS;
    hipStream_t stm = static_cast<hipStream_t>(stream);
    if (bh == 0) return SELSCAN_OK;
    if (dims->seqlen == 0) {
        if (!last_state) return SELSCAN_OK;
        const hipError_t e = h0 ? launch_copy_f32(last_state, h0, st, stm) : launch_fill_zero(last_state, st, stm);
        return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
    }
    SsdTensors tt{x, delta, A, B, C, D, dt_bias, y, last_state, h0};
    const hipError_t e = launch_ssd(tt, dims->batch, dims->seqlen, dims->heads, dims->dstate, stm);
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

int selscan_ssd_step(float* state, const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* D, const float* dt_bias, void* y,
                     const selscan_ssd_dims_t* dims, void* stream) {
    if (!dims) return SELSCAN_ERR_NULL;
    if (dims->batch < 0 || dims->heads < 0 || dims->headdim < 0 || dims->dstate < 0)
        return SELSCAN_ERR_DIMS;
    if (dims->dtype != SELSCAN_BF16) return SELSCAN_ERR_DTYPE;
    if (dims->headdim != 64 || (dims->dstate != 64 && dims->dstate != 128)) return SELSCAN_ERR_DSTATE;
    int64_t bh, xe, st, t, bn;
    if (!mul_ok(dims->batch, dims->heads, &bh) || !mul_ok(bh, 64, &xe) ||
        !mul_ok(xe, dims->dstate, &st) || !mul_ok(st, 4, &t) || !mul_ok(dims->batch, dims->dstate, &bn) ||
        bh > INT32_MAX)
        return SELSCAN_ERR_DIMS;
    if (bh > 0 && (!state || !x || !delta || !A || !y)) return SELSCAN_ERR_NULL;
    if (bn > 0 && (!B || !C)) return SELSCAN_ERR_NULL;
    for (const void* p : {(const void*)state, x, delta, (const void*)A, B, C, (const void*)D,
                          (const void*)dt_bias, (const void*)y})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const Span os = span(state, st * 4), oy = span(y, xe * 2);
    const Span ins[] = {span(x, xe * 2), span(delta, bh * 2), span(A, dims->heads * 4), span(B, bn * 2),
                        span(C, bn * 2), span(D, dims->heads * 4), span(dt_bias, dims->heads * 4)};
    for (const Span& s : ins)
        if (overlaps(s, oy) || overlaps(s, os)) return SELSCAN_ERR_ALIAS;
    if (overlaps(oy, os)) return SELSCAN_ERR_ALIAS;
    if (bh == 0) return SELSCAN_OK;
    SsdStepTensors tt{state, x, delta, A, B, C, D, dt_bias, y};
    const hipError_t e = launch_ssd_step(tt, dims->batch, dims->heads, dims->dstate,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

int selscan_conv1d(const void* x, const float* w, const float* bias, const float* x_prev,
                   void* out, float* x_last, const selscan_dims_t* dims, void* stream) {
    if (!dims) return SELSCAN_ERR_NULL;
    if (dims->batch < 0 || dims->dim < 0 || dims->seqlen < 0) return SELSCAN_ERR_DIMS;
    if (dims->dtype != SELSCAN_F32 && dims->dtype != SELSCAN_BF16) return SELSCAN_ERR_DTYPE;
    int64_t rows, seq, t;
    if (!mul_ok(dims->batch, dims->dim, &rows) || !mul_ok(rows, dims->seqlen, &seq) ||
        !mul_ok(seq, 4, &t) || !mul_ok(rows, 12, &t) || !mul_ok(dims->dim, 16, &t))
        return SELSCAN_ERR_DIMS;
    // grid: one thread per 16-byte vector, blocks of 256, at most 2^32 blocks
    if (rows > (int64_t(1) << 36) || seq >= (int64_t(1) << 42)) return SELSCAN_ERR_DIMS;
    if ((seq > 0 && (!x || !out)) || (dims->dim > 0 && !w)) return SELSCAN_ERR_NULL;
    for (const void* p : {x, (const void*)w, (const void*)bias, (const void*)x_prev, (const void*)out,
                          (const void*)x_last})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    const Span o = span(out, seq * es), xl = span(x_last, rows * 12);
    const Span ins[] = {span(x, seq * es), span(w, dims->dim * 16), span(bias, dims->dim * 4)};
    for (const Span& s : ins)
        if (overlaps(s, o) || overlaps(s, xl)) return SELSCAN_ERR_ALIAS;
    if (overlaps(o, xl)) return SELSCAN_ERR_ALIAS;
    const Span xp = span(x_prev, rows * 12);
    if (overlaps(xp, o)) return SELSCAN_ERR_ALIAS;
    if (overlaps(xp, xl) && static_cast<const void*>(x_prev) != static_cast<const void*>(x_last))
        return SELSCAN_ERR_ALIAS;
    if (rows == 0) return SELSCAN_OK;
    ConvTensors ct{x, w, bias, x_prev, out, x_last};
    const hipError_t e = launch_conv(ct, rows, dims->seqlen, dims->dim,
                                     dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

int selscan_conv1d_bwd(const void* x, const float* w, const float* bias, const float* x_prev,
                       const void* dout, void* dx, float* dw, float* dbias, float* dx_prev,
                       const selscan_dims_t* dims, void* stream) {
    if (!dims) return SELSCAN_ERR_NULL;
    if (dims->batch < 0 || dims->dim < 0 || dims->seqlen < 0) return SELSCAN_ERR_DIMS;
    if (dims->dtype != SELSCAN_F32 && dims->dtype != SELSCAN_BF16) return SELSCAN_ERR_DTYPE;
    int64_t rows, seq, t;
    if (!mul_ok(dims->batch, dims->dim, &rows) || !mul_ok(rows, dims->seqlen, &seq) ||
        !mul_ok(seq, 4, &t) || !mul_ok(rows, 12, &t) || !mul_ok(dims->dim, 16, &t))
        return SELSCAN_ERR_DIMS;
    const DType dt = dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32;
    const ConvBwdPlan plan = conv_bwd_plan(dims->batch, dims->seqlen, dims->dim, dt);
    const int64_t nparts = int64_t(plan.bgroups) * plan.pieces;
    if (dims->dim * nparts > INT32_MAX) return SELSCAN_ERR_DIMS;
    if ((seq > 0 && (!x || !dout || !dx)) || (dims->dim > 0 && (!w || !dw))) return SELSCAN_ERR_NULL;
    for (const void* p : {x, (const void*)w, (const void*)bias, (const void*)x_prev, dout, (const void*)dx,
                          (const void*)dw, (const void*)dbias, (const void*)dx_prev})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    const Span outs[] = {span(dx, seq * es), span(dw, dims->dim * 16), span(dbias, dims->dim * 4),
                         span(dx_prev, rows * 12)};
    const Span ins[] = {span(x, seq * es), span(w, dims->dim * 16), span(bias, dims->dim * 4),
                        span(x_prev, rows * 12), span(dout, seq * es)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Span& s : ins)
            if (overlaps(s, outs[i])) return SELSCAN_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
            if (overlaps(outs[i], outs[j])) return SELSCAN_ERR_ALIAS;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dims->dim == 0) return SELSCAN_OK;
    if (rows == 0 || dims->seqlen == 0) {  // no terms
        if (launch_fill_zero(dw, dims->dim * 4, st) != hipSuccess) return SELSCAN_ERR_LAUNCH;
        if (dbias && launch_fill_zero(dbias, dims->dim, st) != hipSuccess) return SELSCAN_ERR_LAUNCH;
        if (dx_prev && launch_fill_zero(dx_prev, rows * 3, st) != hipSuccess) return SELSCAN_ERR_LAUNCH;
        return SELSCAN_OK;
    }
    void* part = nullptr;
    if (hipMallocAsync(&part, size_t(dims->dim) * nparts * 5 * sizeof(float), st) != hipSuccess || !part) {
        (void)hipGetLastError();
        return SELSCAN_ERR_ALLOC;
    }
    ConvBwdTensors ct{x, w, bias, x_prev, dout, dx, dw, dbias, dx_prev};
    const hipError_t e = launch_conv_bwd(ct, dims->batch, dims->seqlen, dims->dim, dt,
                                         static_cast<float*>(part), plan, st);
    (void)hipFreeAsync(part, st);
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

int selscan_conv1d_step(float* conv_state, const void* x, const float* w, const float* bias,
                        void* out, const selscan_dims_t* dims, void* stream) {
    if (!dims) return SELSCAN_ERR_NULL;
    if (dims->batch < 0 || dims->dim < 0) return SELSCAN_ERR_DIMS;
    if (dims->dtype != SELSCAN_F32 && dims->dtype != SELSCAN_BF16) return SELSCAN_ERR_DTYPE;
    int64_t rows, t;
    if (!mul_ok(dims->batch, dims->dim, &rows) || !mul_ok(rows, 12, &t) || !mul_ok(dims->dim, 16, &t))
        return SELSCAN_ERR_DIMS;
    if (rows > (int64_t(1) << 36)) return SELSCAN_ERR_DIMS;
    if (rows > 0 && (!conv_state || !x || !out || !w)) return SELSCAN_ERR_NULL;
    for (const void* p : {(const void*)conv_state, x, (const void*)w, (const void*)bias, (const void*)out})
        if (!aligned16(p)) return SELSCAN_ERR_ALIGN;
    const int64_t es = dims->dtype == SELSCAN_BF16 ? 2 : 4;
    const Span o = span(out, rows * es), st = span(conv_state, rows * 12);
    const Span ins[] = {span(x, rows * es), span(w, dims->dim * 16), span(bias, dims->dim * 4)};
    for (const Span& s : ins)
        if (overlaps(s, o) || overlaps(s, st)) return SELSCAN_ERR_ALIAS;
    if (overlaps(o, st)) return SELSCAN_ERR_ALIAS;
    if (rows == 0) return SELSCAN_OK;
    ConvStepTensors ct{conv_state, x, w, bias, out};
    const hipError_t e = launch_conv_step(ct, rows, dims->dim,
                                          dims->dtype == SELSCAN_BF16 ? DType::BF16 : DType::F32,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SELSCAN_OK : SELSCAN_ERR_LAUNCH;
}

const char* selscan_strerror(int code) {
    switch (code) {
        case SELSCAN_OK: return "ok";
        case SELSCAN_ERR_NULL: return "a required pointer is NULL";
        case SELSCAN_ERR_DIMS: return "a size is negative or too large";
        case SELSCAN_ERR_DSTATE: return "unsupported dstate (this version supports 16)";
        case SELSCAN_ERR_DTYPE: return "unsupported dtype";
        case SELSCAN_ERR_LAUNCH: return "kernel launch failed";
        case SELSCAN_ERR_ALLOC: return "workspace allocation failed";
        case SELSCAN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case SELSCAN_ERR_ALIAS: return "an output overlaps an input or another output";
        case SELSCAN_ERR_CONFIG: return "options out of range, or workspace too small or misaligned";
        case SELSCAN_ERR_SCRATCH:
            return "the call needs more workspace than the no-allocation scratch holds";
        default: return "unknown error code";
    }
}

int selscan_version(void) { return kVersion; }

}  // extern "C"

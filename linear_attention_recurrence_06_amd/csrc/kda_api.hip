// C ABI of libkda.so: argument validation, workspace sizing and dispatch.
// See include/kda.h for the contract.  Nothing here reads device memory or
// synchronises; every launch goes on the caller's stream.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/kda.h"
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
template <typename T, int D> hipError_t launch_prep(const PrefillArgs&, hipStream_t);
template <typename T, int D> hipError_t launch_recur(const PrefillArgs&, hipStream_t);
template <int D> hipError_t launch_fused(const PrefillArgs&, hipStream_t);

namespace {

hipError_t launch_prep_any(const PrefillArgs& a, hipStream_t s) {
    if (a.bf16) return a.d == 128 ? launch_prep<bf16, 128>(a, s) : launch_prep<bf16, 64>(a, s);
    return a.d == 128 ? launch_prep<float, 128>(a, s) : launch_prep<float, 64>(a, s);
}

hipError_t launch_recur_any(const PrefillArgs& a, hipStream_t s) {
    if (a.bf16) return a.d == 128 ? launch_recur<bf16, 128>(a, s) : launch_recur<bf16, 64>(a, s);
    return a.d == 128 ? launch_recur<float, 128>(a, s) : launch_recur<float, 64>(a, s);
}

// The library's second stream on the current device (default priority, not
// synchronising with the null stream), created on first use and kept until the
// process ends.
hipError_t aux_stream(hipStream_t* out) {
    static std::mutex mu;
    static hipStream_t streams[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!streams[dev]) {
        e = hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking);
        if (e != hipSuccess) {
            streams[dev] = nullptr;
            return e;
        }
    }
    *out = streams[dev];
    return hipSuccess;
}

// Chunks per pipeline segment (at least) and segments per call (at least and
// at most).  Each segment restarts the recurrence's chains and the first
// segment's preparation runs alone, so short segments or few of them cost more
// than the overlap saves (measured: 8,192 tokens x 16 heads in 2 segments +13%,
// 32,768 x 16 in 8 segments +3%; 2^20 x 16 in 16 segments -9%).
constexpr int64_t kSegChunks = 1024;
constexpr int kMinSegments = 4;
constexpr int kMaxSegments = 16;

// Segments for a pipelined call, or 0 for one launch of each kernel.  One
// sequence whose recurrence workgroups (one per head and 16-column tile) leave
// compute units idle: the preparation of later chunks then runs on those units
// while the recurrence works through earlier ones.
int pipeline_segments(const PrefillArgs& a) {
    if (a.n_seqs != 1 || a.total_tokens <= 0 || a.compute_units <= 0) return 0;
    if ((int64_t)a.n_heads * (a.d / 16) >= a.compute_units) return 0;
    const int64_t nch = (a.total_tokens + 63) / 64;
    if (nch < kMinSegments * kSegChunks) return 0;
    return (int)std::min<int64_t>(kMaxSegments, nch / kSegChunks);
}

// Pipelined prefill of one sequence in S segments of chunks.  The preparation
// of segment i goes on the library's second stream, the recurrence over
// segment i on the caller's stream after an event that marks the preparation
// done; the fp32 state passes between segments through `state` (the caller's
// final state, or the workspace).  The caller's stream has every launch of the
// call behind it when this returns, so its later work is ordered after all of
// them, and the second stream starts only after the caller's earlier work.
hipError_t launch_prefill_pipelined(const PrefillArgs& a0, hipStream_t s, int S, float* state) {
    const int64_t nch = (a0.total_tokens + 63) / 64;
    hipStream_t s2;
    hipError_t e = aux_stream(&s2);
    if (e != hipSuccess) return e;
    hipEvent_t ev[kMaxSegments + 1];
    int made = 0;
    for (; made <= S; ++made)
        if ((e = hipEventCreateWithFlags(&ev[made], hipEventDisableTiming)) != hipSuccess) break;
    if (e == hipSuccess) e = hipEventRecord(ev[S], s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s2, ev[S], 0);
    int recorded = 0;  // K1 segments launched and marked on the second stream
    for (int i = 0; i < S && e == hipSuccess; ++i) {
        PrefillArgs a = a0;
        a.slot_begin = nch * i / S;
        a.slot_end = i == S - 1 ? -1 : nch * (i + 1) / S;
        a.prep_setup = i == 0;
        if ((e = launch_prep_any(a, s2)) == hipSuccess && (e = hipEventRecord(ev[i], s2)) == hipSuccess)
            recorded = i + 1;
    }
    for (int i = 0; i < S && e == hipSuccess; ++i) {
        if ((e = hipStreamWaitEvent(s, ev[i], 0)) != hipSuccess) break;
        PrefillArgs a = a0;
        a.chunk_begin = nch * i / S;
        a.chunk_end = nch * (i + 1) / S;
        a.initial_state = i == 0 ? a0.initial_state : state;
        a.final_state = i == S - 1 ? a0.final_state : state;
        e = launch_recur_any(a, s);
    }
    // after a failure, still keep the caller's stream behind everything the
    // second stream has queued, so no work of this call outlives it there
    if (e != hipSuccess && recorded > 0) (void)hipStreamWaitEvent(s, ev[recorded - 1], 0);
    // (events still pending are released once they complete)
    for (int i = 0; i < made; ++i) {
        const hipError_t d = hipEventDestroy(ev[i]);
        if (e == hipSuccess) e = d;
    }
    return e;
}

}  // namespace

bool fused_path(const PrefillArgs& a) {
    // the fused kernel covers the plain recurrence in bf16: per-channel gate,
    // no front end, output gate or checkpoints, the whole call in one launch;
    // it writes the outputs in 16-byte pieces
    if (!a.bf16 || a.scalar_g || a.out_gate != 0 || a.fe.active() || a.ckpt_interval > 0) return false;
    if ((reinterpret_cast<uintptr_t>(a.out) & 15) != 0) return false;
    if (a.total_tokens <= 0 || a.slot_begin != 0 || a.slot_end != -1 || a.chunk_begin != 0 ||
        a.chunk_end != INT64_MAX)
        return false;
    const char* env = std::getenv("KDA_PREFILL_PATH");
    if (env && (std::strcmp(env, "split") == 0 || std::strcmp(env, "segmented") == 0)) return false;
    if (env && std::strcmp(env, "fused") == 0) return true;
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    const int64_t per = a.d == 128 ? kFusedCUsPerChain : kFusedCUsPerChain64;
    return a.compute_units > 0 && chains * per >= (int64_t)a.compute_units;
}

int segmented_segments(const PrefillArgs& a) {
    // the fused kernel's plain recurrence at d = 128, the whole call
    if (!a.bf16 || a.d != 128 || a.scalar_g || a.out_gate != 0 || a.fe.active() ||
        a.ckpt_interval > 0)
        return 0;
    if ((reinterpret_cast<uintptr_t>(a.out) & 15) != 0) return 0;
    if (a.total_tokens <= 0 || a.n_seqs < 1 || a.slot_begin != 0 || a.slot_end != -1 ||
        a.chunk_begin != 0 || a.chunk_end != INT64_MAX)
        return 0;
    // (the scan's grid: eight workgroups per chain)
    if ((int64_t)a.n_seqs * a.n_heads > (int64_t{1} << 24)) return 0;
    const char* env = std::getenv("KDA_PREFILL_PATH");
    const bool forced = env && std::strcmp(env, "segmented") == 0;
    if (env && (std::strcmp(env, "split") == 0 || std::strcmp(env, "fused") == 0)) return 0;
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    const int64_t seq_chunks = (a.total_tokens / a.n_seqs + 63) / 64;
    const int64_t cus = a.compute_units > 0 ? a.compute_units : 256;
    // one chain per CU in each pass, with segments of at least kSegMinChunks
    // (the kernel's placement: P of ceil(7 C / (7 P + 8)) chunks after the first)
    int64_t P = std::min<int64_t>(kSegMaxSegments, std::max<int64_t>(1, cus / chains));
    while (P >= 2 && (7 * seq_chunks + 7 * P + 7) / (7 * P + 8) < kSegMinChunks) --P;
    if (const char* ps = std::getenv("KDA_PREFILL_SEGMENTS")) {
        const long v = std::strtol(ps, nullptr, 10);
        if (v >= 1 && v <= kSegMaxSegments) P = std::min<int64_t>(v, seq_chunks);
    }
    if (P < 2) return 0;
    // automatically: the segment chains fill three quarters of the device,
    // or there are at least kSegManySegments, or the fused kernel would take
    // the call with a chain per CU at most (a third of the device or more)
    if (!forced && (a.compute_units <= 0 ||
                    (chains * P * 4 < (int64_t)a.compute_units * 3 && P < kSegManySegments &&
                     chains * kFusedCUsPerChain < (int64_t)a.compute_units)))
        return 0;
    // its arrays fit in the record area the split path would use
    if (segmented_scratch_bytes(a, (int)P) > a.layout.records_bytes()) return 0;
    return (int)P;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    if (const int P = segmented_segments(a)) return launch_segmented(a, P, s);
    if (fused_path(a))
        return a.d == 128 ? launch_fused<128>(a, s) : launch_fused<64>(a, s);
    // under stream capture the call stays on the caller's stream: no library
    // stream or events enter the caller's graph (the results are the same)
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e0 = hipStreamIsCapturing(s, &cap);
    if (e0 != hipSuccess) return e0;
    const int S = (cap == hipStreamCaptureStatusNone && !a.no_pipeline) ? pipeline_segments(a) : 0;
    if (S >= 2) {
        float* state = a.final_state ? a.final_state
                                     : reinterpret_cast<float*>(a.workspace + a.layout.state_offset());
        return launch_prefill_pipelined(a, s, S, state);
    }
    hipError_t e = launch_prep_any(a, s);
    if (e != hipSuccess) return e;
    return launch_recur_any(a, s);
}
}  // namespace kda

namespace {

// Compute units of the current device, queried once per device (a benign race:
// every thread stores the same value).
hipError_t compute_units(int32_t* out) {
    static std::atomic<int32_t> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) {
        const int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) n = 1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    *out = n;
    return hipSuccess;
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, a + bytes};
}
bool overlap(Range a, Range b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

// Shared descriptor checks.  `prefill` selects the prefill-only rules.
kda_status check_dims(const kda_dims* d, bool prefill) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->num_seqs < 0 || d->num_heads < 1 || d->total_tokens < 0) return KDA_ERR_INVALID_ARG;
    // (per-chunk buffer ranges are 32-bit: 64 token rows of H * d elements)
    if (d->num_heads > 65536) return KDA_ERR_UNSUPPORTED;
    if (d->io_dtype != KDA_BF16 && d->io_dtype != KDA_FP32) return KDA_ERR_UNSUPPORTED;
    if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128)) return KDA_ERR_UNSUPPORTED;
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (d->gate != KDA_GATE_CHANNEL && d->gate != KDA_GATE_HEAD) return KDA_ERR_INVALID_ARG;
    if (prefill) {
        if (d->chunk != 0 && d->chunk != 64) return KDA_ERR_UNSUPPORTED;
        if (d->total_tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    } else {
        if (d->total_tokens != d->num_seqs) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

size_t elt_bytes(const kda_dims* d) { return d->io_dtype == KDA_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int kda_version(void) { return 1 * 10000 + 2 * 100 + 0; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

size_t kda_prefill_workspace_bytes(const kda_dims* d) {
    if (check_dims(d, true) != KDA_OK) return 0;
    if (d->num_seqs == 0) return 256;
    return kda::make_layout(d->d_k, (int)elt_bytes(d), d->total_tokens, d->num_seqs,
                            d->num_heads, true)
        .total();
}

}  // extern "C"

namespace {

// Arguments of a plain call with these sizes on the current device, as far
// as the path choice reads them (false: a descriptor the library rejects, or
// a device that cannot be queried).
bool plain_call_args(const kda_dims* d, int32_t packed, kda::PrefillArgs& a) {
    if (check_dims(d, true) != KDA_OK) return false;
    a = kda::PrefillArgs{};  // (no options, no checkpoints: zero)
    a.total_tokens = d->total_tokens;
    a.n_seqs = d->num_seqs;
    a.n_heads = d->num_heads;
    a.d = d->d_k;
    a.bf16 = d->io_dtype == KDA_BF16;
    a.scalar_g = d->gate == KDA_GATE_HEAD;
    a.scale = d->scale;
    a.l2norm = d->qk_l2norm;
    a.fe = kda::FrontEnd{};
    // stand-ins the choice looks at only for being null or 16-byte aligned
    a.out = reinterpret_cast<void*>(uintptr_t{256});
    a.cu_seqlens = packed ? reinterpret_cast<const int32_t*>(uintptr_t{256}) : nullptr;
    a.layout = kda::make_layout(d->d_k, (int)elt_bytes(d), d->total_tokens, d->num_seqs,
                                d->num_heads, true);
    return compute_units(&a.compute_units) == hipSuccess;
}

// Workspace bytes the path of a call uses: the index areas (fused kernel),
// those and the state maps (segmented), or all of ws_need, the two-kernel
// path's records and pipeline state.
size_t path_workspace_bytes(const kda::PrefillArgs& a, size_t ws_need) {
    if (a.n_seqs == 0 || a.total_tokens == 0) return ws_need;
    if (const int seg = kda::segmented_segments(a))
        return a.layout.records_offset() + kda::segmented_scratch_bytes(a, seg);
    return kda::fused_path(a) ? a.layout.records_offset() : ws_need;
}

}  // namespace

extern "C" {

size_t kda_prefill_path_workspace_bytes(const kda_dims* d, int32_t packed) {
    kda::PrefillArgs a;
    if (!plain_call_args(d, packed, a)) return 0;
    return path_workspace_bytes(a, kda_prefill_workspace_bytes(d));
}

int32_t kda_prefill_path(const kda_dims* d, int32_t packed, int32_t* segments) {
    kda::PrefillArgs a;
    if (!plain_call_args(d, packed, a)) return -1;
    int32_t seg = 0, path = KDA_PATH_SPLIT;
    if (d->num_seqs > 0 && d->total_tokens > 0) {
        if ((seg = kda::segmented_segments(a)) > 0) {
            path = KDA_PATH_SEGMENTED;
        } else if (kda::fused_path(a)) {
            path = KDA_PATH_FUSED;
        } else if ((seg = kda::pipeline_segments(a)) >= 2) {
            path = KDA_PATH_PIPELINED;
        } else {
            seg = 0;
        }
    }
    if (segments) *segments = seg;
    return path;
}

int32_t kda_prefill_pipeline_segments(const kda_dims* d) {
    int32_t seg = 0;
    const int32_t path = kda_prefill_path(d, 0, &seg);
    if (path < 0) return -1;
    return path == KDA_PATH_PIPELINED ? seg : 0;
}

}  // extern "C"

// ------------------------------------------------------------------ no allocation
// The workspace of kda_chunk_prefill_noalloc: one array per device, allocated
// when the library is loaded there and held until the process ends.  Host
// code never uses this name as an address: kernels get the per-device address
// from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

// Front-end checks shared by prefill and decode (need_g: there are tokens,
// so a decay gate must come from g or the low-rank factors).  Fills `fe`
// (inactive when f is NULL).
kda_status check_front_end(const kda_dims* d, const kda_front_end* f, const void* g,
                           bool need_g, kda::FrontEnd& fe) {
    fe = kda::FrontEnd();
    if (!f) return (g || !need_g) ? KDA_OK : KDA_ERR_INVALID_ARG;
    if (f->conv_width < 0 || f->conv_width > 4 || f->conv_silu < 0 || f->conv_silu > 1 ||
        f->reserved != 0)
        return KDA_ERR_INVALID_ARG;
    const int r = f->gate_rank;
    if (r != 0 && r != 32 && r != 64 && r != 96 && r != 128) return KDA_ERR_INVALID_ARG;
    if (f->conv_width > 0 && !f->conv_weight) return KDA_ERR_INVALID_ARG;
    if (r > 0 && (g || (need_g && (!f->gate_a || !f->gate_b)) || d->gate == KDA_GATE_HEAD))
        return KDA_ERR_INVALID_ARG;
    if (r == 0 && !g && need_g) return KDA_ERR_INVALID_ARG;
    const bool states = f->conv_width > 1;
    const void* v16[] = {f->conv_width > 0 ? f->conv_weight : nullptr,
                         states ? f->conv_state_in : nullptr,
                         states ? f->conv_state_out : nullptr, r > 0 ? f->gate_a : nullptr,
                         r > 0 ? f->gate_b : nullptr};
    for (const void* p : v16)
        if (p && !aligned_to(p, 16)) return KDA_ERR_MISALIGNED;
    if (r > 0 && f->gate_bias && !aligned_to(f->gate_bias, 4)) return KDA_ERR_MISALIGNED;
    fe.conv_w = f->conv_width;
    fe.silu = f->conv_width > 0 ? f->conv_silu : 0;
    fe.conv_weight = f->conv_width > 0 ? f->conv_weight : nullptr;
    fe.state_in = states ? f->conv_state_in : nullptr;
    fe.state_out = states ? f->conv_state_out : nullptr;
    fe.rank = r;
    fe.gate_a = r > 0 ? f->gate_a : nullptr;
    fe.gate_b = r > 0 ? f->gate_b : nullptr;
    fe.gate_bias = r > 0 ? f->gate_bias : nullptr;
    return KDA_OK;
}

// Byte ranges of the front end's inputs and of its state output.
struct FrontEndRanges {
    Range in[5];  // weight, state in, a, b, bias
    Range state_out;
};
FrontEndRanges front_end_ranges(const kda_dims* d, const kda::FrontEnd& fe, int64_t T) {
    const size_t E = elt_bytes(d);
    const int64_t N = d->num_seqs, H = d->num_heads, D = d->d_k;
    const size_t wb = (size_t)3 * H * fe.conv_w * D * E;
    const size_t cb = fe.conv_w > 1 ? (size_t)N * 3 * (fe.conv_w - 1) * H * D * E : 0;
    FrontEndRanges r;
    r.in[0] = fe.conv_weight ? range_of(fe.conv_weight, wb) : Range{0, 0};
    r.in[1] = fe.state_in ? range_of(fe.state_in, cb) : Range{0, 0};
    r.in[2] = fe.gate_a ? range_of(fe.gate_a, (size_t)T * fe.rank * E) : Range{0, 0};
    r.in[3] = fe.gate_b ? range_of(fe.gate_b, (size_t)H * D * fe.rank * E) : Range{0, 0};
    r.in[4] = fe.gate_bias ? range_of(fe.gate_bias, (size_t)H * D * 4) : Range{0, 0};
    r.state_out = fe.state_out ? range_of(fe.state_out, cb) : Range{0, 0};
    return r;
}


// Device address of `scratch` on the current device, looked up once per device
// with that device current.
hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

// Shared body of the prefill entry points.
kda_status prefill_impl(const kda_dims* d, const void* q, const void* k, const void* v,
                        const void* g, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, void* out, float* final_state,
                        const kda_prefill_options& o, void* workspace, size_t workspace_bytes,
                        void* stream, bool noalloc = false) {
    kda_status st = check_dims(d, true);
    if (st != KDA_OK) return st;
    const int64_t T = d->total_tokens, N = d->num_seqs, H = d->num_heads, D = d->d_k;
    const int32_t interval = o.checkpoint_interval, out_gate = o.out_gate;
    float* checkpoints = o.checkpoints;
    const void* out_gate_z = o.out_gate_z;
    if (interval < 0) return KDA_ERR_INVALID_ARG;
    if (out_gate < KDA_OUT_GATE_NONE || out_gate > KDA_OUT_GATE_HEAD) return KDA_ERR_INVALID_ARG;
    if (N == 0) return T == 0 ? KDA_OK : KDA_ERR_INVALID_ARG;
    if (!cu_seqlens && T % N != 0) return KDA_ERR_INVALID_ARG;
    kda::FrontEnd fe;
    st = check_front_end(d, o.front_end, g, T > 0, fe);
    if (st != KDA_OK) return st;
    if (T > 0 && (!q || !k || !v || !beta || !out)) return KDA_ERR_INVALID_ARG;
    if (interval > 0 && !checkpoints) return KDA_ERR_INVALID_ARG;
    if (out_gate != KDA_OUT_GATE_NONE && T > 0 && !out_gate_z) return KDA_ERR_INVALID_ARG;
    // q, k, v, g rows and the workspace are read with 16-byte vector accesses;
    // beta, out and the states element by element
    const uintptr_t E_al = d->io_dtype == KDA_BF16 ? 2 : 4;
    const bool sg = d->gate == KDA_GATE_HEAD;
    const void* vec_ptrs[] = {q, k, v, sg ? nullptr : g, workspace};
    for (const void* p : vec_ptrs)
        if (p && !aligned_to(p, 16)) return KDA_ERR_MISALIGNED;
    const void* elt_ptrs[] = {beta, out, sg ? g : nullptr, out_gate ? out_gate_z : nullptr};
    for (const void* p : elt_ptrs)
        if (p && !aligned_to(p, E_al)) return KDA_ERR_MISALIGNED;
    const void* f32_ptrs[] = {initial_state, final_state, cu_seqlens, checkpoints};
    for (const void* p : f32_ptrs)
        if (p && !aligned_to(p, 4)) return KDA_ERR_MISALIGNED;
    // the workspace: too small for any path, or for the two-kernel path where
    // that is the only one the call can take, is rejected without asking the
    // device; the path-specific size is checked once the path is known
    const size_t ws_need = kda_prefill_workspace_bytes(d);
    const bool two_kernel_only = d->io_dtype != KDA_BF16 || sg || interval > 0 ||
                                 out_gate != KDA_OUT_GATE_NONE || fe.active();
    const kda::PrefillLayout lay = kda::make_layout((int)D, (int)elt_bytes(d), T, N, H, true);
    if (workspace && (workspace_bytes < lay.records_offset() ||
                      (two_kernel_only && workspace_bytes < ws_need)))
        return KDA_ERR_WORKSPACE;

    // overlaps: no output may touch an input or another output; final_state
    // may equal initial_state exactly
    const size_t E = elt_bytes(d);
    const size_t qb = (size_t)T * H * D * E, bb = (size_t)T * H * E, sb = (size_t)N * H * D * D * 4;
    const size_t gb = sg ? bb : qb;
    const FrontEndRanges fr = front_end_ranges(d, fe, T);
    const Range r_out = range_of(out, qb);
    const Range r_z = out_gate != KDA_OUT_GATE_NONE
                          ? range_of(out_gate_z, out_gate == KDA_OUT_GATE_HEAD ? bb : qb)
                          : Range{0, 0};
    const Range r_ws = workspace ? range_of(workspace, workspace_bytes) : Range{0, 0};
    const Range r_s0 = initial_state ? range_of(initial_state, sb) : Range{0, 0};
    const Range r_cu = cu_seqlens ? range_of(cu_seqlens, (size_t)(N + 1) * 4) : Range{0, 0};
    const Range ins[] = {range_of(q, qb), range_of(k, qb), range_of(v, qb),
                         g ? range_of(g, gb) : Range{0, 0}, range_of(beta, bb), r_s0, r_cu, r_z,
                         fr.in[0], fr.in[1], fr.in[2], fr.in[3], fr.in[4]};
    const Range r_fin = final_state ? range_of(final_state, sb) : Range{0, 0};
    Range r_ck{0, 0};
    if (interval > 0 && !cu_seqlens) {
        // equal lengths: the checkpoint count is known here, so check its buffer too
        const int64_t C = kda_checkpoint_count(d, nullptr, interval);
        r_ck = range_of(checkpoints, (size_t)C * H * D * D * 4);
    }
    // the workspace is written by the kernels: it may touch no input
    for (const Range& r : ins)
        if (overlap(r_ws, r)) return KDA_ERR_INVALID_ARG;
    if (T > 0) {
        // outputs against inputs (final_state == initial_state is allowed)
        const Range outs[] = {r_out, r_fin, r_ck, fr.state_out};
        for (int oi = 0; oi < 4; ++oi)
            for (const Range& r : ins) {
                if (oi == 1 && initial_state == final_state && r.lo == r_s0.lo && r.hi == r_s0.hi)
                    continue;
                if (overlap(outs[oi], r)) return KDA_ERR_INVALID_ARG;
            }
        // outputs against each other and the workspace
        for (int a = 0; a < 4; ++a) {
            if (overlap(outs[a], r_ws)) return KDA_ERR_INVALID_ARG;
            for (int b = a + 1; b < 4; ++b)
                if (overlap(outs[a], outs[b])) return KDA_ERR_INVALID_ARG;
        }
    } else {
        // no tokens: only the final states and the conv states are written
        if (final_state && initial_state && initial_state != final_state && overlap(r_fin, r_s0))
            return KDA_ERR_INVALID_ARG;
        const Range touched[] = {r_fin, fr.state_out};
        for (const Range& r : touched)
            if (overlap(r, r_ws) || overlap(r, fr.in[1]) || overlap(r, r_cu))
                return KDA_ERR_INVALID_ARG;
        if (overlap(r_fin, fr.state_out) || overlap(fr.state_out, r_s0)) return KDA_ERR_INVALID_ARG;
    }

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.initial_state = initial_state;
    a.cu_seqlens = cu_seqlens;
    a.out = out;
    a.final_state = final_state;
    a.workspace = static_cast<unsigned char*>(workspace);
    a.total_tokens = T;
    a.n_seqs = (int32_t)N;
    a.n_heads = (int32_t)H;
    a.d = (int32_t)D;
    a.bf16 = d->io_dtype == KDA_BF16;
    a.scalar_g = sg;
    a.scale = d->scale;
    a.l2norm = d->qk_l2norm;
    a.ckpt_interval = interval;
    a.checkpoints = checkpoints;
    a.out_gate = out_gate;
    a.out_gate_z = out_gate_z;
    a.fe = fe;
    a.layout = lay;
    // a call that can only take the two-kernel path (fp32 I/O, or the per-head
    // gate) is sized without asking the device
    if (noalloc && two_kernel_only && ws_need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    if (compute_units(&a.compute_units) != hipSuccess) return KDA_ERR_HIP;
    if (workspace && workspace_bytes < path_workspace_bytes(a, ws_need)) return KDA_ERR_WORKSPACE;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (noalloc) {
        // the library's per-device array (its address is found only now, after
        // every argument has been checked); one stream, no library events
        if (path_workspace_bytes(a, ws_need) > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
        void* ws = nullptr;
        if (scratch_address(&ws) != hipSuccess) return KDA_ERR_HIP;
        a.workspace = static_cast<unsigned char*>(ws);
        a.no_pipeline = true;
        const hipError_t e = kda::launch_prefill(a, hs);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (workspace) {
        const hipError_t e = kda::launch_prefill(a, hs);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // no workspace given: a stream-ordered allocation on the caller's stream,
    // freed on it after the last launch (not while the stream is being
    // captured: a graph needs a caller-owned workspace)
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(hs, &cap) != hipSuccess) return KDA_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return KDA_ERR_WORKSPACE;
    // (the fused path keeps its records in LDS and needs only the index areas;
    // the segmented path adds its state maps)
    void* ws = nullptr;
    if (hipMallocAsync(&ws, path_workspace_bytes(a, ws_need), hs) != hipSuccess) return KDA_ERR_HIP;
    a.workspace = static_cast<unsigned char*>(ws);
    const hipError_t e = kda::launch_prefill(a, hs);
    const hipError_t f = hipFreeAsync(ws, hs);
    return (e == hipSuccess && f == hipSuccess) ? KDA_OK : KDA_ERR_HIP;
}

const kda_prefill_options kNoPrefillOptions = {0, KDA_OUT_GATE_NONE, nullptr, nullptr, nullptr};
const kda_decode_options kNoDecodeOptions = {KDA_OUT_GATE_NONE, 0, nullptr, nullptr};

}  // namespace

extern "C" {

kda_status kda_chunk_prefill(const kda_dims* d, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, const float* initial_state,
                             const int32_t* cu_seqlens, void* out, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                        kNoPrefillOptions, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_prefill_ex(const kda_dims* d, const void* q, const void* k, const void* v,
                                const void* g, const void* beta, const float* initial_state,
                                const int32_t* cu_seqlens, void* out, float* final_state,
                                const kda_prefill_options* o, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                        o ? *o : kNoPrefillOptions, workspace, workspace_bytes, stream);
}

int64_t kda_checkpoint_count(const kda_dims* d, const int32_t* host_cu_seqlens,
                             int32_t checkpoint_interval) {
    if (check_dims(d, true) != KDA_OK || checkpoint_interval < 1) return -1;
    const int64_t N = d->num_seqs, T = d->total_tokens;
    if (N == 0) return 0;
    if (!host_cu_seqlens && T % N != 0) return -1;
    int64_t count = 0;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t len = host_cu_seqlens
                                ? (int64_t)host_cu_seqlens[n + 1] - host_cu_seqlens[n]
                                : T / N;
        if (len < 0) return -1;
        const int64_t c = (len + 63) / 64;
        if (c > 0) count += (c - 1) / checkpoint_interval;
    }
    return count;
}

kda_status kda_chunk_prefill_checkpoints(const kda_dims* d, const void* q, const void* k,
                                         const void* v, const void* g, const void* beta,
                                         const float* initial_state,
                                         const int32_t* cu_seqlens, void* out,
                                         float* final_state, int32_t checkpoint_interval,
                                         float* checkpoints, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (checkpoint_interval < 1) return KDA_ERR_INVALID_ARG;
    kda_prefill_options o = kNoPrefillOptions;
    o.checkpoint_interval = checkpoint_interval;
    o.checkpoints = checkpoints;
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, o,
                        workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" kda_status kda_chunk_prefill_noalloc(const kda_dims* d, const void* q, const void* k,
                                                const void* v, const void* g, const void* beta,
                                                const float* initial_state,
                                                const int32_t* cu_seqlens, void* out,
                                                float* final_state, void* stream) {
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                        kNoPrefillOptions, nullptr, 0, stream, /*noalloc=*/true);
}

static kda_status decode_impl(const kda_dims* d, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, float* state_inout, void* out,
                              const kda_decode_options& o, void* stream) {
    kda_status st = check_dims(d, false);
    if (st != KDA_OK) return st;
    const int32_t out_gate = o.out_gate;
    const void* out_gate_z = o.out_gate_z;
    if (out_gate < KDA_OUT_GATE_NONE || out_gate > KDA_OUT_GATE_HEAD || o.reserved != 0)
        return KDA_ERR_INVALID_ARG;
    const int64_t N = d->num_seqs, H = d->num_heads, D = d->d_k;
    if (N == 0) return KDA_OK;
    kda::FrontEnd fe;
    st = check_front_end(d, o.front_end, g, true, fe);
    if (st != KDA_OK) return st;
    if (!q || !k || !v || !beta || !state_inout || !out) return KDA_ERR_INVALID_ARG;
    if (out_gate != KDA_OUT_GATE_NONE && !out_gate_z) return KDA_ERR_INVALID_ARG;
    if (out_gate != KDA_OUT_GATE_NONE && !aligned_to(out_gate_z, d->io_dtype == KDA_BF16 ? 2 : 4))
        return KDA_ERR_MISALIGNED;
    // the state is streamed with 16-byte accesses; token vectors element by element
    const uintptr_t E_al = d->io_dtype == KDA_BF16 ? 2 : 4;
    if (!aligned_to(state_inout, 16)) return KDA_ERR_MISALIGNED;
    const void* ptrs[] = {q, k, v, g, beta, out};
    for (const void* p : ptrs)
        if (p && !aligned_to(p, E_al)) return KDA_ERR_MISALIGNED;
    const size_t E = elt_bytes(d);
    const size_t qb = (size_t)N * H * D * E, bb = (size_t)N * H * E, sb = (size_t)N * H * D * D * 4;
    const size_t gb = d->gate == KDA_GATE_HEAD ? bb : qb;
    const FrontEndRanges fr = front_end_ranges(d, fe, N);
    const Range r_out = range_of(out, qb);
    const Range r_state = range_of(state_inout, sb);
    const Range r_z = out_gate != KDA_OUT_GATE_NONE
                          ? range_of(out_gate_z, out_gate == KDA_OUT_GATE_HEAD ? bb : qb)
                          : Range{0, 0};
    const Range ins[] = {range_of(q, qb), range_of(k, qb), range_of(v, qb),
                         g ? range_of(g, gb) : Range{0, 0}, range_of(beta, bb), r_z,
                         fr.in[0], fr.in[2], fr.in[3], fr.in[4], fr.in[1]};
    constexpr int kInsNoState = 10;  // every input but the conv state
    // out: no overlap with anything; the state: only itself; the conv state:
    // only the input conv state, and only exactly
    for (const Range& r : ins)
        if (overlap(r_out, r) || overlap(r_state, r)) return KDA_ERR_INVALID_ARG;
    if (overlap(r_out, r_state)) return KDA_ERR_INVALID_ARG;
    if (fe.state_out) {
        for (int i = 0; i < kInsNoState; ++i)
            if (overlap(fr.state_out, ins[i])) return KDA_ERR_INVALID_ARG;
        if (overlap(fr.state_out, r_out) || overlap(fr.state_out, r_state))
            return KDA_ERR_INVALID_ARG;
        if (fe.state_in && fe.state_in != fe.state_out && overlap(fr.state_out, fr.in[1]))
            return KDA_ERR_INVALID_ARG;
    }

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.state = state_inout;
    a.out = out;
    a.n_seqs = (int32_t)N;
    a.n_heads = (int32_t)H;
    a.d = (int32_t)D;
    a.bf16 = d->io_dtype == KDA_BF16;
    a.scalar_g = d->gate == KDA_GATE_HEAD;
    a.out_gate = out_gate;
    a.out_gate_z = out_gate_z;
    a.fe = fe;
    a.scale = d->scale;
    a.l2norm = d->qk_l2norm;
    hipError_t e = kda::launch_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}


extern "C" {

kda_status kda_decode_step(const kda_dims* d, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, float* state_inout, void* out,
                           void* stream) {
    return decode_impl(d, q, k, v, g, beta, state_inout, out, kNoDecodeOptions, stream);
}

kda_status kda_decode_step_ex(const kda_dims* d, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, float* state_inout, void* out,
                              const kda_decode_options* o, void* stream) {
    return decode_impl(d, q, k, v, g, beta, state_inout, out, o ? *o : kNoDecodeOptions,
                       stream);
}

}  // extern "C"

// C ABI of libkda.so: argument validation, workspace sizing and dispatch.
// See include/kda.h for the contract.  Nothing here reads device memory or
// synchronises; every launch goes on the caller's stream.
#include <atomic>

#include "../../include/kda.h"
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
template <typename T, int D> hipError_t launch_prep(const PrefillArgs&, hipStream_t);
template <typename T, int D> hipError_t launch_recur(const PrefillArgs&, hipStream_t);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
    hipError_t e;
    if (a.bf16 && a.d == 128) {
        if ((e = launch_prep<bf16, 128>(a, s)) != hipSuccess) return e;
        return launch_recur<bf16, 128>(a, s);
    }
    if (a.bf16 && a.d == 64) {
        if ((e = launch_prep<bf16, 64>(a, s)) != hipSuccess) return e;
        return launch_recur<bf16, 64>(a, s);
    }
    if ((e = launch_prep<float, 64>(a, s)) != hipSuccess) return e;
    return launch_recur<float, 64>(a, s);
}
}  // namespace kda

namespace {

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
    if (d->io_dtype != KDA_BF16 && d->io_dtype != KDA_FP32) return KDA_ERR_UNSUPPORTED;
    if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128)) return KDA_ERR_UNSUPPORTED;
    if (d->qk_l2norm != 0 && d->qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (d->gate != KDA_GATE_CHANNEL && d->gate != KDA_GATE_HEAD) return KDA_ERR_INVALID_ARG;
    if (prefill) {
        if (d->chunk != 0 && d->chunk != 64) return KDA_ERR_UNSUPPORTED;
        // fp32 I/O keeps fp32 operand tiles in LDS; at d = 128 they exceed it
        if (d->io_dtype == KDA_FP32 && d->d_k == 128) return KDA_ERR_UNSUPPORTED;
        if (d->total_tokens > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    } else {
        if (d->total_tokens != d->num_seqs) return KDA_ERR_INVALID_ARG;
    }
    return KDA_OK;
}

size_t elt_bytes(const kda_dims* d) { return d->io_dtype == KDA_BF16 ? 2 : 4; }

// Compute units of the current device, queried once per device.
int current_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

}  // namespace

extern "C" {

int kda_version(void) { return 1 * 10000 + 1 * 100 + 0; }

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

// Shared body of the prefill entry points (interval 0: no checkpoints;
// out_gate 0: no output gate).
kda_status prefill_impl(const kda_dims* d, const void* q, const void* k, const void* v,
                        const void* g, const void* beta, const float* initial_state,
                        const int32_t* cu_seqlens, void* out, float* final_state,
                        int32_t interval, float* checkpoints, int32_t out_gate,
                        const void* out_gate_z, void* workspace, size_t workspace_bytes,
                        void* stream) {
    kda_status st = check_dims(d, true);
    if (st != KDA_OK) return st;
    const int64_t T = d->total_tokens, N = d->num_seqs, H = d->num_heads, D = d->d_k;
    if (interval < 0) return KDA_ERR_INVALID_ARG;
    if (out_gate < KDA_OUT_GATE_NONE || out_gate > KDA_OUT_GATE_HEAD) return KDA_ERR_INVALID_ARG;
    if (N == 0) return T == 0 ? KDA_OK : KDA_ERR_INVALID_ARG;
    if (!cu_seqlens && T % N != 0) return KDA_ERR_INVALID_ARG;
    if (T > 0 && (!q || !k || !v || !g || !beta || !out)) return KDA_ERR_INVALID_ARG;
    if (interval > 0 && !checkpoints) return KDA_ERR_INVALID_ARG;
    if (out_gate != KDA_OUT_GATE_NONE && T > 0 && !out_gate_z) return KDA_ERR_INVALID_ARG;
    if (!workspace) return KDA_ERR_WORKSPACE;
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
    if (workspace_bytes < kda_prefill_workspace_bytes(d)) return KDA_ERR_WORKSPACE;

    // overlaps: out must not touch any input; final_state may equal initial_state exactly
    const size_t E = elt_bytes(d);
    const size_t qb = (size_t)T * H * D * E, bb = (size_t)T * H * E, sb = (size_t)N * H * D * D * 4;
    const size_t gb = sg ? bb : qb;
    const Range r_out = range_of(out, qb);
    const Range ins[] = {range_of(q, qb), range_of(k, qb), range_of(v, qb), range_of(g, gb),
                         range_of(beta, bb),
                         initial_state ? range_of(initial_state, sb) : Range{0, 0},
                         cu_seqlens ? range_of(cu_seqlens, (size_t)(N + 1) * 4) : Range{0, 0},
                         range_of(workspace, workspace_bytes)};
    if (T > 0)
        for (const Range& r : ins)
            if (overlap(r_out, r)) return KDA_ERR_INVALID_ARG;
    const Range r_z = out_gate != KDA_OUT_GATE_NONE
                          ? range_of(out_gate_z, out_gate == KDA_OUT_GATE_HEAD ? bb : qb)
                          : Range{0, 0};
    if (T > 0 && overlap(r_out, r_z)) return KDA_ERR_INVALID_ARG;
    if (final_state) {
        const Range r_fin = range_of(final_state, sb);
        if (initial_state && initial_state != final_state &&
            overlap(r_fin, range_of(initial_state, sb)))
            return KDA_ERR_INVALID_ARG;
        const Range others[] = {range_of(q, qb), range_of(k, qb), range_of(v, qb),
                                range_of(g, gb), range_of(beta, bb), r_out, r_z,
                                range_of(workspace, workspace_bytes)};
        for (const Range& r : others)
            if (overlap(r_fin, r)) return KDA_ERR_INVALID_ARG;
    }
    if (interval > 0 && !cu_seqlens) {
        // equal lengths: the checkpoint count is known here, so check its buffer too
        const int64_t C = kda_checkpoint_count(d, nullptr, interval);
        const Range r_ck = range_of(checkpoints, (size_t)C * H * D * D * 4);
        const Range all[] = {range_of(q, qb), range_of(k, qb), range_of(v, qb),
                             range_of(g, gb), range_of(beta, bb), r_out, r_z,
                             initial_state ? range_of(initial_state, sb) : Range{0, 0},
                             final_state ? range_of(final_state, sb) : Range{0, 0},
                             range_of(workspace, workspace_bytes)};
        for (const Range& r : all)
            if (overlap(r_ck, r)) return KDA_ERR_INVALID_ARG;
    }

    kda::PrefillArgs a;
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
    a.layout = kda::make_layout((int)D, (int)E, T, N, H, true);
    a.cu_count = current_cu_count();
    hipError_t e = kda::launch_prefill(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill(const kda_dims* d, const void* q, const void* k, const void* v,
                             const void* g, const void* beta, const float* initial_state,
                             const int32_t* cu_seqlens, void* out, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state, 0,
                        nullptr, KDA_OUT_GATE_NONE, nullptr, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_prefill_ex(const kda_dims* d, const void* q, const void* k, const void* v,
                                const void* g, const void* beta, const float* initial_state,
                                const int32_t* cu_seqlens, void* out, float* final_state,
                                const kda_prefill_options* o, void* workspace,
                                size_t workspace_bytes, void* stream) {
    const kda_prefill_options none = {0, KDA_OUT_GATE_NONE, nullptr, nullptr};
    if (!o) o = &none;
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                        o->checkpoint_interval, o->checkpoints, o->out_gate, o->out_gate_z,
                        workspace, workspace_bytes, stream);
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
    return prefill_impl(d, q, k, v, g, beta, initial_state, cu_seqlens, out, final_state,
                        checkpoint_interval, checkpoints, KDA_OUT_GATE_NONE, nullptr, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

static kda_status decode_impl(const kda_dims* d, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, float* state_inout, void* out,
                              int32_t out_gate, const void* out_gate_z, void* stream) {
    kda_status st = check_dims(d, false);
    if (st != KDA_OK) return st;
    if (out_gate < KDA_OUT_GATE_NONE || out_gate > KDA_OUT_GATE_HEAD) return KDA_ERR_INVALID_ARG;
    const int64_t N = d->num_seqs, H = d->num_heads, D = d->d_k;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state_inout || !out) return KDA_ERR_INVALID_ARG;
    if (out_gate != KDA_OUT_GATE_NONE && !out_gate_z) return KDA_ERR_INVALID_ARG;
    if (out_gate != KDA_OUT_GATE_NONE && !aligned_to(out_gate_z, d->io_dtype == KDA_BF16 ? 2 : 4))
        return KDA_ERR_MISALIGNED;
    // the state is streamed with 16-byte accesses; token vectors element by element
    const uintptr_t E_al = d->io_dtype == KDA_BF16 ? 2 : 4;
    if (!aligned_to(state_inout, 16)) return KDA_ERR_MISALIGNED;
    const void* ptrs[] = {q, k, v, g, beta, out};
    for (const void* p : ptrs)
        if (!aligned_to(p, E_al)) return KDA_ERR_MISALIGNED;
    const size_t E = elt_bytes(d);
    const size_t qb = (size_t)N * H * D * E, bb = (size_t)N * H * E, sb = (size_t)N * H * D * D * 4;
    const size_t gb = d->gate == KDA_GATE_HEAD ? bb : qb;
    const Range r_out = range_of(out, qb);
    const Range ins[] = {range_of(q, qb), range_of(k, qb), range_of(v, qb), range_of(g, gb),
                         range_of(beta, bb), range_of(state_inout, sb)};
    for (const Range& r : ins)
        if (overlap(r_out, r)) return KDA_ERR_INVALID_ARG;
    const Range r_z = out_gate != KDA_OUT_GATE_NONE
                          ? range_of(out_gate_z, out_gate == KDA_OUT_GATE_HEAD ? bb : qb)
                          : Range{0, 0};
    if (overlap(r_out, r_z)) return KDA_ERR_INVALID_ARG;
    const Range r_state = range_of(state_inout, sb);
    for (int i = 0; i < 5; ++i)
        if (overlap(r_state, ins[i])) return KDA_ERR_INVALID_ARG;
    if (overlap(r_state, r_z)) return KDA_ERR_INVALID_ARG;

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
    a.scale = d->scale;
    a.l2norm = d->qk_l2norm;
    hipError_t e = kda::launch_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}


extern "C" {

kda_status kda_decode_step(const kda_dims* d, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, float* state_inout, void* out,
                           void* stream) {
    return decode_impl(d, q, k, v, g, beta, state_inout, out, KDA_OUT_GATE_NONE, nullptr,
                       stream);
}

kda_status kda_decode_step_ex(const kda_dims* d, const void* q, const void* k, const void* v,
                              const void* g, const void* beta, float* state_inout, void* out,
                              int32_t out_gate, const void* out_gate_z, void* stream) {
    return decode_impl(d, q, k, v, g, beta, state_inout, out, out_gate, out_gate_z, stream);
}

}  // extern "C"

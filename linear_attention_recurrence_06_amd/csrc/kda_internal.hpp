// Host-side interface between the C ABI (kda_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// epsilon inside the L2-norm square root: x / sqrt(sum x^2 + eps)
constexpr float kL2Eps = 1e-6f;

// Largest grid y dimension a launch uses (the runtime's documented limit);
// launches split longer ranges.
constexpr int64_t kMaxGridY = 65535;

// Front end ahead of the recurrence: short causal convolution of the raw q,
// k, v (width conv_w, 0 = none; tap conv_w-1 is the current token; optional
// SiLU) and the low-rank decay gate g = -softplus(a b^T + bias) (rank 0 = g
// given).  Layouts: weight [3, H, W, d], states [N, 3, W-1, H, d], a [T, r],
// b [H, d, r], bias [H, d] fp32.
struct FrontEnd {
    int conv_w = 0;
    int silu = 0;
    const void* conv_weight = nullptr;
    const void* state_in = nullptr;
    void* state_out = nullptr;
    int rank = 0;
    const void* gate_a = nullptr;
    const void* gate_b = nullptr;
    const float* gate_bias = nullptr;
    bool active() const { return conv_w > 0 || rank > 0; }
};

struct DecodeArgs {
    const void *q, *k, *v, *g, *beta;
    float* state;
    void* out;
    int32_t n_seqs, n_heads, d;
    bool bf16;
    bool scalar_g;               // g is [N, H] (one decay per head) instead of [N, H, d]
    float scale;
    int l2norm;
    int out_gate;                // 0 none, 1 z [N, H, d], 2 z [N, H]: out = o * sigmoid(z)
    const void* out_gate_z;
    FrontEnd fe;
};

// Workspace for one prefill call: a chunk index (packed sequences only; first chunk slot of each
// sequence, int32 [N+1]), a checkpoint index (first checkpoint of each
// sequence, int32 [N+1]), one descriptor per chunk slot (first token and
// length, int32 x 2; length 0 marks an unused slot), then one record per
// (chunk slot, head) with the factors the recurrence kernel consumes, stored head-major
// (all chunk slots of head 0, then head 1, ...) so that one head's chain of
// chunks is one contiguous stream.  Record layout, E = element size
// of the I/O type, all matrices in MFMA fragment order:
//   W    64 x D   (A order)   W = T Diag(beta) Khat
//   Qh   64 x D   (A order)   Qhat = q * exp(gamma)
//   M    64 x 64  (A order)   inclusive-lower Q K decay products (the two
//                             fragment tiles of rows 0..31, columns 32..63 are
//                             all zero; they are neither written nor read)
//   Kt   D  x 64  (A order)   Kprime^T, Kprime = k * exp(gamma_C - gamma)
//   U    64 x D   (C order)   U = T Diag(beta) V
//   gC   D fp32               exp(gamma_C)
struct PrefillLayout {
    int d;
    int elt;               // bytes per I/O element
    int64_t slots;         // chunk slots (upper bound on the chunk count)
    int64_t heads;
    size_t index_bytes;    // chunk index, padded to 256 B (checkpoint index: the same)
    size_t desc_bytes;     // chunk-slot descriptors, padded to 256 B
    size_t rec_bytes;      // bytes per (slot, head) record
    size_t off_w, off_q, off_m, off_kt, off_u, off_gc;
    __host__ __device__ size_t ckidx_offset() const { return index_bytes; }
    __host__ __device__ size_t desc_offset() const { return 2 * index_bytes; }
    __host__ __device__ size_t records_offset() const { return 2 * index_bytes + desc_bytes; }
    size_t state_bytes;    // fp32 state of every chain between pipeline segments (one sequence)
    size_t records_bytes() const { return rec_bytes * (size_t)slots * (size_t)heads; }
    size_t state_offset() const { return records_offset() + records_bytes(); }
    size_t total() const { return state_offset() + state_bytes; }
};

inline PrefillLayout make_layout(int d, int elt, int64_t total_tokens, int64_t n_seqs,
                                 int64_t heads, bool varlen) {
    PrefillLayout L;
    L.d = d;
    L.elt = elt;
    L.heads = heads;
    if (varlen || n_seqs == 0) {
        L.slots = (total_tokens + 63) / 64 + n_seqs;
    } else {
        const int64_t len = total_tokens / n_seqs;
        L.slots = n_seqs * ((len + 63) / 64);
    }
    L.index_bytes = (((size_t)(n_seqs + 1) * 4 + 255) / 256) * 256;
    L.desc_bytes = (((size_t)L.slots * 8 + 255) / 256) * 256;
    size_t o = 0;
    L.off_w = o;  o += (size_t)64 * d * elt;
    L.off_q = o;  o += (size_t)64 * d * elt;
    L.off_m = o;  o += (size_t)64 * 64 * elt;
    L.off_kt = o; o += (size_t)d * 64 * elt;
    L.off_u = o;  o += (size_t)64 * d * elt;
    L.off_gc = o; o += (size_t)d * 4;
    L.rec_bytes = o;
    L.state_bytes = n_seqs == 1 ? (size_t)heads * d * d * 4 : 0;
    return L;
}

struct PrefillArgs {
    const void *q, *k, *v, *g, *beta;
    const float* initial_state;
    const int32_t* cu_seqlens;   // may be null: equal lengths
    void* out;
    float* final_state;          // may be null
    unsigned char* workspace;
    int64_t total_tokens;
    int32_t n_seqs, n_heads, d;
    bool bf16;
    bool scalar_g;               // g is [T, H] (one decay per head) instead of [T, H, d]
    float scale;
    int l2norm;
    int32_t ckpt_interval;       // 0: no checkpoints
    float* checkpoints;          // [C, H, d, d] when ckpt_interval > 0
    int out_gate;                // 0 none, 1 z [T, H, d], 2 z [T, H]: out = o * sigmoid(z)
    const void* out_gate_z;
    FrontEnd fe;
    PrefillLayout layout;
    // Part of the work one launch pair covers (the whole call by default): the
    // preparation kernel takes chunk slots [slot_begin, slot_end) and runs the
    // index / descriptor / conv-state kernels only with prep_setup; the
    // recurrence takes chunks [chunk_begin, chunk_end) of every chain, reading
    // initial_state and writing final_state at that range's ends.
    int64_t slot_begin = 0, slot_end = -1;
    bool prep_setup = true;
    int64_t chunk_begin = 0, chunk_end = INT64_MAX;
    int32_t compute_units = 0;   // of the launching device (0: unknown, no pipeline)
    bool no_pipeline = false;    // one stream only: no library stream or events
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// A prefill the segmented path does not take runs the fused kernel
// (persistent workgroups working through whole (sequence, head) chains)
// instead of the preparation and recurrence kernels once it has at least one
// chain per kFusedCUsPerChain compute units (d = 128; per two at d = 64).
// Measured at d = 128 against the two-kernel time (256 CUs): 8,192-token
// sequences, 64 chains 1.15x, 86 chains 0.86x, 128 chains 0.73x, 256 chains
// 0.42x; 65,536-token sequences, 80 chains 0.95x, 96 chains 0.86x, 112 chains
// 0.68x.  At d = 64, 128 chains 0.94x.
constexpr int64_t kFusedCUsPerChain = 3;
constexpr int64_t kFusedCUsPerChain64 = 2;

// Whether the fused kernel takes a call the segmented path does not.  The
// environment variable KDA_PREFILL_PATH=split or =fused overrides the choice
// where the fused kernel applies (=segmented rules it out).
bool fused_path(const PrefillArgs& a);

// Segmented prefill of long chains (d = 128, bf16, plain options): with P
// chains per sequence and head in each pass, every sequence is cut (by the
// kernel, from cu_seqlens) into P + 1 segments; a first pass runs segment 0
// with its outputs and forms the state maps of segments 1..P-1 from the zero
// state and from the identity, a scan composes the maps into the start states
// of segments 2..P, and a second pass runs segments 1..P with their outputs.
// segmented_segments gives P, or 0 where the path does not apply or would not
// pay (KDA_PREFILL_PATH=segmented forces it where it applies, and
// KDA_PREFILL_SEGMENTS=<P> sets P).  Its three [N (P + 1), H, d, d] fp32
// arrays take segmented_scratch_bytes of the workspace's record area.
int segmented_segments(const PrefillArgs& a);
size_t segmented_scratch_bytes(const PrefillArgs& a, int P);
hipError_t launch_segmented(const PrefillArgs& a, int P, hipStream_t stream);
// P is one chain per compute unit in each pass, at most kSegMaxSegments,
// lowered until segments 1..P hold at least kSegMinChunks chunks.  The path is
// taken automatically with P >= 2 whose chains fill three quarters of the
// device, or with kSegManySegments or more, or where the fused kernel would
// take the call (it then runs a chain per CU at most).  Measured at d = 128 on
// 256 CUs, time against the best other path: 2^20 tokens x 16 heads 0.53x
// (two-kernel); 8,192 tokens x 96 heads (P = 2) 0.83x and 2^16 x 96 heads
// 0.73x (fused); 8,192 x 32 heads (P = 8, 14-chunk segments) 0.87x and x 64
// heads (P = 4) 0.70x (two-kernel); 4,096 x 32 heads (P = 8, 7-chunk
// segments) 1.16x and 2,048 x 128 heads (P = 2, 11 chunks) 1.16x (not taken).
constexpr int64_t kSegMinChunks = 12;
constexpr int kSegMaxSegments = 64;
constexpr int64_t kSegManySegments = 16;

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace kda

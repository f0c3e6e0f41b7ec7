/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * The operation.  Kimi Delta Attention (KDA) keeps, per sequence and head, one
 * fixed-size state matrix S (d_k x d_v, fp32) in place of a key/value list
 * that grows with every token (the x.com post mirrored as "one matrix replaced
 * the KV cache", its opening post).  Each token first
 * predicts from the memory, then writes only the difference between the
 * incoming value and the prediction; a learned retention alpha (per key
 * channel, so channels forget on different timescales) and an update strength
 * beta control it ("From KV Cache to Depth Attention: The Bottlenecks Kimi K3
 * Had to Break", Technical Details, Kimi Delta Attention bullet; "Kimi K3: The
 * Manos, The Mythos, The Legendos", bullet on KDA as online learning with a
 * diagonal gate).  Queries and keys are L2-normalised (same page, bullet on
 * stability details).  Written out, with alpha_t = exp(g_t), g_t <= 0:
 *
 *     q_t <- scale * q_t / sqrt(|q_t|^2 + eps),  k_t <- k_t / sqrt(|k_t|^2 + eps)
 *     S_t  = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t  = S_t^T q_t
 *
 * with eps = 1e-6.  Prefill runs this over whole (optionally packed) sequences
 * with linear cost, decode advances one token per sequence at a cost that does
 * not depend on the position ("Kimi K3: The Manos, The Mythos, The Legendos",
 * bullet on chunked prefill and constant-cost decode).
 *
 * Layouts (all row-major, contiguous, token-major):
 *   q, k, g : [T_total, H, d_k]      v, out : [T_total, H, d_v]
 *   beta    : [T_total, H]           (g: [T_total, H] with KDA_GATE_HEAD)
 *   states  : [N, H, d_k, d_v] fp32; S[i][j], i = key channel, j = value
 *             channel (fastest)
 *   cu_seqlens : int32 [N + 1], cu[0] = 0, non-decreasing, cu[N] = T_total
 * q, k, v, g, beta and out share one element type (kda_dims.io_dtype): bf16
 * (raw 16-bit bfloat16 bit patterns) or fp32.  States are always fp32.
 *
 * Ownership: the caller allocates and owns every buffer it passes (device
 * memory).  The library allocates device memory only for a prefill given no
 * workspace (stream-ordered on the call's stream, freed there by the end of
 * the call), and holds one array per device for kda_chunk_prefill_noalloc.
 *
 * Asynchrony: every call only enqueues work on `stream` (a hipStream_t, or
 * NULL for the null stream) and returns without synchronising.  A fault in a
 * kernel surfaces at the caller's next synchronisation.
 *
 * Errors: every call returns a kda_status and never throws.  Validation uses
 * only the descriptor and pointer values (no device reads, no sync):
 * NULL required pointers, unsupported sizes or dtypes, misaligned pointers,
 * undersized workspace, forbidden overlaps.  Alignment: prefill q, k, v, g
 * (per-channel gate) and the workspace 16 bytes; the decode state 16 bytes;
 * every other pointer its element size.  The contents of
 * cu_seqlens and the value ranges (g <= 0, -inf allowed; 0 <= beta <= 1) are
 * preconditions the library does not check.
 *
 * Thread safety and determinism: calls are reentrant.  The library's only
 * state is, per device, the compute-unit count (queried once, cached
 * atomically), the second stream of the pipelined prefill (see
 * kda_chunk_prefill; created once under a lock) and the device array of
 * kda_chunk_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES, allocated when the
 * library is loaded on a device), all kept until the process ends.  The
 * fused prefill kernel hands out (sequence, head) chains through a device
 * counter, but a chain's arithmetic does not depend on which workgroup runs
 * it, and no other kernel uses atomics: identical inputs and sizes give
 * bitwise identical results (a pipelined call included).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* NULL required pointer, bad count, bad overlap   */
    KDA_ERR_UNSUPPORTED = 2, /* head size, chunk size or dtype not implemented  */
    KDA_ERR_MISALIGNED = 3,  /* a pointer is not aligned as its access needs    */
    KDA_ERR_WORKSPACE = 4,   /* workspace too small (or none while capturing)    */
    KDA_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed       */
} kda_status;

typedef enum {
    KDA_BF16 = 0, /* bfloat16 inputs and outputs, fp32 state, bf16 MFMA with fp32 accumulation */
    KDA_FP32 = 1  /* fp32 inputs and outputs, fp32 state, fp32 MFMA                            */
} kda_dtype;

/* Shape of the forget gate g.  KDA's retention is a diagonal matrix, one decay
 * per key channel; the scalar forget gate it refines keeps one decay per token
 * and head ("Kimi K3: The Manos, The Mythos, The Legendos", bullet on KDA as
 * online learning: gating adds a forget gate, KDA makes it diagonal). */
typedef enum {
    KDA_GATE_CHANNEL = 0, /* g [T_total, H, d_k] (decode: [N, H, d_k]): KDA          */
    KDA_GATE_HEAD = 1     /* g [T_total, H] (decode: [N, H]): one decay shared by all
                             key channels, alpha_t = exp(g_t) times the identity     */
} kda_gate;

/* Problem descriptor (host memory, read during the call only). */
typedef struct {
    int64_t total_tokens; /* T_total: length of the packed token axis (decode: = num_seqs) */
    int32_t num_seqs;     /* N >= 1; without cu_seqlens, N equal-length sequences back to back */
    int32_t num_heads;    /* H >= 1                                                       */
    int32_t d_k, d_v;     /* supported: (64, 64) and (128, 128)                            */
    int32_t chunk;        /* prefill chunk length: 0 (default) or 64                      */
    int32_t io_dtype;     /* kda_dtype                                                    */
    float scale;          /* multiplies q after its L2 normalisation (1.0 for plain KDA)  */
    int32_t qk_l2norm;    /* 1: the library L2-normalises q and k; 0: used as given        */
    int32_t gate;         /* kda_gate: layout of g (KDA_GATE_CHANNEL unless stated)       */
} kda_dims;

/* Bytes of device workspace kda_chunk_prefill needs for these sizes (0 on a
 * descriptor the library would reject).  The workspace holds the per-chunk
 * factors the chunk-prep kernel hands to the recurrence kernel and, for a
 * single sequence (num_seqs == 1), one fp32 state per head for a pipelined call
 * (see kda_chunk_prefill). */
size_t kda_prefill_workspace_bytes(const kda_dims* dims);

/* Chunked prefill over packed sequences.
 *
 * Sequence n is tokens cu_seqlens[n] <= t < cu_seqlens[n+1] (cu_seqlens NULL:
 * T_total / num_seqs tokens each, T_total must divide evenly).  Each sequence
 * starts from initial_state[n] (NULL: zero state), writes out[t] for each of
 * its tokens, and ends with final_state[n] (NULL: not written).
 *
 *   q, k, v, g, beta : device, read-only, io_dtype, layouts above
 *   initial_state    : device fp32 [N,H,d_k,d_v] or NULL
 *   cu_seqlens       : device int32 [N+1] or NULL
 *   out              : device io_dtype [T_total,H,d_v]; must not overlap any input
 *   final_state      : device fp32 [N,H,d_k,d_v] or NULL; may be the very same
 *                      pointer as initial_state (each sequence-head reads its
 *                      slot before writing it), any other overlap is rejected
 *   workspace        : device, 16-byte aligned, at least the bytes the call's
 *                      path uses (kda_prefill_path_workspace_bytes; the
 *                      options of kda_chunk_prefill_ex and checkpoints take
 *                      the two-kernel path), and kda_prefill_workspace_bytes(dims)
 *                      is enough for every path; must not overlap any other buffer;
 *                      contents on entry are ignored and on return are
 *                      unspecified.  NULL: the library allocates it with
 *                      hipMallocAsync on stream and frees it there with
 *                      hipFreeAsync after the call's last launch
 *                      (KDA_ERR_WORKSPACE while stream is being captured into
 *                      a graph: a captured call needs a caller-owned workspace)
 *   stream           : hipStream_t (as void*), NULL for the null stream
 *
 * Supported: d_k = d_v in {64, 128} with bf16 or fp32 I/O; T_total <= 2^31 - 1
 * tokens and num_heads <= 65536 (larger: KDA_ERR_UNSUPPORTED).
 *
 * Streams.  Every launch is ordered after the caller's earlier work on stream,
 * and the caller's later work on stream is ordered after every launch of the
 * call.  One long sequence (num_seqs == 1, at least 4 * 1024 chunks of 64
 * tokens) whose recurrence leaves compute units idle (num_heads * d_v / 16
 * below the device's compute units) is pipelined: the chunk preparation of
 * later segments runs on a second stream that the library creates on the
 * current device at its first such call (default priority, non-blocking, kept
 * until the process ends), joined to stream by events, while the recurrence
 * works through earlier segments on stream.  The results are bitwise those of
 * the unpipelined path.  A call on a stream that is being captured into a graph
 * is not pipelined: it launches only on that stream.  Concurrent calls on one
 * device share the second stream; each call's own events keep its launches
 * ordered.
 *
 * Kernels.  A call with bf16 I/O, d = 128, a per-channel gate, out aligned to
 * 16 bytes and no options of kda_chunk_prefill_ex or checkpoints is
 * segmented where that pays.  With P (sequence, head) chains per compute unit
 * in each pass -- CUs / chains, at most 64, lowered until the segments hold at
 * least 12 chunks for sequences of the average length -- each sequence is cut
 * into P + 1 segments of whole chunks (a short sequence may leave segments
 * empty): a first pass of the fused kernel below runs segment 0 with its
 * outputs and forms the state maps S_end = M S_start + b of segments 1..P-1 (b
 * from the zero state, M from the identity with v taken as zero), a scan
 * kernel composes the maps in order into the start states of segments 2..P,
 * and a second pass runs segments 1..P with their outputs (three [N (P + 1),
 * H, d, d] fp32 arrays in the workspace's record area).  It is taken with P of
 * at least 2 whose chains fill three quarters of the compute units, with P of
 * 16 or more, or where the fused kernel would take the call.  Otherwise a
 * call with many chains -- at least a third of the device's compute units at
 * d = 128, half at d = 64 -- under the same conditions (bf16 also at d = 64)
 * runs one fused kernel: persistent workgroups take whole chains, longest
 * sequences first, and step through each 64-token chunk as four 16-token
 * sub-chunks with the chunk's operands in LDS, so only the inputs, the outputs
 * and the states touch HBM; it uses only the first two index areas of the
 * workspace.  Every other call runs the preparation and recurrence kernels,
 * which hand per-chunk records through the workspace.  The paths compute the
 * same recurrence with the same operand precision but round in a different
 * order, so their results agree to the accuracy below, not bit for bit.  The
 * environment variable KDA_PREFILL_PATH (read at each call) set to "split",
 * "fused" or "segmented" overrides the choice where that path applies, and
 * KDA_PREFILL_SEGMENTS=<P> (2 to 64) sets P for a segmented call.
 *
 * Accuracy: bf16 I/O uses bf16 MFMA operands with fp32 accumulation and an
 * fp32 state; fp32 I/O uses fp32 MFMA throughout.  Any g <= 0 is handled:
 * inside a 64-token chunk the decay ratios are factored around 16-token block
 * boundaries with every factor at most 1, except on the diagonal blocks, whose
 * factored form is used only while a block's decay in every channel stays
 * within 2^64; a block past that has its diagonal products formed exactly
 * from per-pair decay ratios that are all at most 1.  A token's retention is
 * floored at 2^-128 (g >= -88.7), a difference no fp32 result can show.
 */
kda_status kda_chunk_prefill(const kda_dims* dims, const void* q, const void* k,
                             const void* v, const void* g, const void* beta,
                             const float* initial_state, const int32_t* cu_seqlens,
                             void* out, float* final_state, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Segments a kda_chunk_prefill with these sizes (cu_seqlens NULL) is
 * pipelined into on the current device, outside stream capture (see Streams
 * at kda_chunk_prefill): 0 for one launch of each kernel or another path
 * (kda_prefill_path), S >= 4 for S segments, -1 for a descriptor the library
 * would reject or a device that cannot be queried.  Reads no device memory. */
int32_t kda_prefill_pipeline_segments(const kda_dims* dims);

/* The kernels a plain kda_chunk_prefill with these sizes runs on the current
 * device (see Kernels at kda_chunk_prefill), outside stream capture, with
 * cu_seqlens given (packed != 0) or NULL and out aligned to 16 bytes; the
 * environment overrides of that paragraph apply.  *segments (when not NULL)
 * receives the pipeline's segment count, or P of a segmented call (P + 1
 * segments; 0 for the other paths).  Returns -1
 * for a descriptor the library would reject or a device that cannot be
 * queried.  Reads no device memory.  A diagnostic, for benchmarks and tests. */
typedef enum {
    KDA_PATH_SPLIT = 0,      /* preparation + recurrence kernels, one launch each */
    KDA_PATH_PIPELINED = 1,  /* the same, pipelined over segments of one sequence */
    KDA_PATH_FUSED = 2,      /* the fused kernel, whole chains */
    KDA_PATH_SEGMENTED = 3   /* segment maps, their scan, then the segments again */
} kda_prefill_path_kind;
int32_t kda_prefill_path(const kda_dims* dims, int32_t packed, int32_t* segments);

/* Bytes of workspace a plain kda_chunk_prefill with these sizes uses on the
 * current device, for the path kda_prefill_path reports with the same
 * arguments: the fused kernel only the index areas (4 (N + 1) bytes twice and
 * 8 bytes per 64-token chunk of every sequence, each area rounded up to 256
 * bytes), a segmented call those and its 3 N (P + 1) H d^2 fp32 state maps, the
 * other paths kda_prefill_workspace_bytes(dims).  Never more than
 * kda_prefill_workspace_bytes(dims); 0 where kda_prefill_path returns -1.
 * Reads no device memory. */
size_t kda_prefill_path_workspace_bytes(const kda_dims* dims, int32_t packed);

/* Number of intermediate states kda_chunk_prefill_checkpoints writes: for each
 * sequence of c = ceil(len / 64) chunks, floor((c - 1) / checkpoint_interval)
 * (none for an empty sequence).  host_cu_seqlens is HOST memory, int32 [N + 1]
 * (NULL: N equal lengths, as in kda_chunk_prefill).  Returns -1 when the
 * descriptor or the interval (must be >= 1) is invalid. */
int64_t kda_checkpoint_count(const kda_dims* dims, const int32_t* host_cu_seqlens,
                             int32_t checkpoint_interval);

/* Chunked prefill that also records intermediate states, so that a later call
 * can resume any sequence from a saved prefix instead of recomputing it.  A
 * fixed-size state is overwritten as the sequence advances, so reusing an
 * earlier prefix needs a snapshot taken before it changes ("Kimi K3: The Manos,
 * The Mythos, The Legendos", Context: the serving engine keeps selected state
 * checkpoints).
 *
 * Same arguments, rules and results as kda_chunk_prefill, plus:
 *   checkpoint_interval : >= 1; one checkpoint every checkpoint_interval
 *                         chunks (64 * checkpoint_interval tokens) of each sequence
 *   checkpoints         : device fp32 [C, H, d_k, d_v] with C =
 *                         kda_checkpoint_count(dims, cu_seqlens on the host,
 *                         checkpoint_interval), 4-byte aligned, required when
 *                         C > 0.  The checkpoints of sequence n follow those of
 *                         sequences 0..n-1; its j-th (j = 0, 1, ...) is the state
 *                         after its first 64 * checkpoint_interval * (j + 1) tokens,
 *                         for every such boundary strictly inside the sequence (the
 *                         state at its end is final_state).  It is bitwise the
 *                         final state of a prefill of that prefix alone.  Must not
 *                         overlap any other buffer.
 * A boundary that is not a multiple of 64 tokens (a prompt boundary) is served
 * by ending a sequence there: final_state is exact at any length, and a prefill
 * started from it continues exactly.
 */
kda_status kda_chunk_prefill_checkpoints(const kda_dims* dims, const void* q, const void* k,
                                         const void* v, const void* g, const void* beta,
                                         const float* initial_state,
                                         const int32_t* cu_seqlens, void* out,
                                         float* final_state, int32_t checkpoint_interval,
                                         float* checkpoints, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Output gate, fused into the output write: out = o * sigmoid(z) with z a
 * caller-supplied pre-activation ("Kimi K3: The Manos, The Mythos, The
 * Legendos", bullet on stability details: a per-head output forget gate).  z
 * has out's element type and either out's layout (one gate per value channel
 * of each head) or [T_total, H] (decode: [N, H]; one gate per token and head). */
typedef enum {
    KDA_OUT_GATE_NONE = 0,
    KDA_OUT_GATE_CHANNEL = 1, /* z [T_total, H, d_v] */
    KDA_OUT_GATE_HEAD = 2     /* z [T_total, H]      */
} kda_out_gate;

/* Front end fused ahead of the recurrence ("Kimi K3: The Manos, The Mythos,
 * The Legendos", bullet on stability details: short convolutions on q, k and
 * v for local dependencies, and low-rank decay gates).  With a front end the
 * q, k and v handed to the call are the raw projections, and the library
 * forms, per sequence, for x in (q, k, v) and every head h and channel c,
 *
 *     x'_t[h][c] = sum_{j < W} conv_weight[x][h][j][c] * x_{t-(W-1)+j}[h][c]
 *
 * (tap W-1 is the current token; tokens before a sequence's start are the
 * rows of conv_state_in, or zero without it), then SiLU(x') = x' sigmoid(x')
 * if conv_silu; and, with gate_rank r > 0,
 *
 *     g_t[h][c] = -softplus(sum_{j < r} gate_a[t][j] gate_b[h][c][j] + gate_bias[h][c])
 *
 * in place of a g argument (which must then be NULL).  The recurrence runs on
 * x' and g exactly as it runs on given q, k, v, g; x' and g stay in fp32 on
 * chip and never reach memory.  conv_width 0 means no convolution (and no
 * SiLU).  The computed g may take any value <= 0, as a given g may.
 *
 * conv_state_* hold, per sequence, the W-1 raw rows before the sequence
 * (in) and the last W-1 raw rows of the sequence (out; for a sequence shorter
 * than W-1 they continue from its input rows), so a later call continues the
 * convolution exactly.  In prefill conv_state_out must not overlap any other
 * buffer; in decode it may be the same pointer as conv_state_in (advanced in
 * place). */
typedef struct {
    int32_t conv_width;        /* 0 (none) or W = 1..4                                   */
    int32_t conv_silu;         /* 0 or 1                                                 */
    const void* conv_weight;   /* [3, H, W, d] io_dtype (q, k, v filters), 16-byte aligned */
    const void* conv_state_in; /* [N, 3, W-1, H, d] io_dtype, 16-byte aligned, nullable   */
    void* conv_state_out;      /* [N, 3, W-1, H, d] io_dtype, 16-byte aligned, nullable   */
    int32_t gate_rank;         /* 0 (g is given) or r in {32, 64, 96, 128}               */
    int32_t reserved;          /* must be 0                                              */
    const void* gate_a;        /* [T_total, r] io_dtype (decode: [N, r]), 16-byte aligned */
    const void* gate_b;        /* [H, d_k, r] io_dtype, 16-byte aligned                  */
    const float* gate_bias;    /* [H, d_k] fp32, nullable (zero)                         */
} kda_front_end;

/* Options of kda_chunk_prefill_ex; all-zero means none (kda_chunk_prefill). */
typedef struct {
    int32_t checkpoint_interval; /* 0, or as in kda_chunk_prefill_checkpoints            */
    int32_t out_gate;            /* kda_out_gate                                          */
    float* checkpoints;          /* as in kda_chunk_prefill_checkpoints (interval > 0)    */
    const void* out_gate_z;      /* device, io_dtype, required unless KDA_OUT_GATE_NONE;
                                    element-size aligned; read only; must not overlap
                                    out, final_state or checkpoints                      */
    const kda_front_end* front_end; /* nullable: q, k, v (and g) as given                */
} kda_prefill_options;

/* Chunked prefill with options: checkpoints (see kda_chunk_prefill_checkpoints),
 * the output gate and/or the front end.  opts NULL means none.  Same
 * arguments, rules and results as kda_chunk_prefill otherwise; with an output
 * gate, out holds the gated outputs (states and checkpoints are unchanged by
 * it); with a front end, q, k, v are the raw projections (see kda_front_end).
 * Errors: KDA_ERR_INVALID_ARG for an out_gate outside kda_out_gate, a NULL
 * out_gate_z with a gate (T_total > 0), z overlapping an output, a front end
 * with conv_width outside 0..4, conv_silu outside 0..1, a NULL conv_weight
 * with W > 0, a gate_rank other than 0, 32, 64, 96, 128, nonzero reserved
 * fields, gate_rank > 0 with a non-NULL g, NULL gate factors or
 * KDA_GATE_HEAD, or a conv_state_out overlapping another buffer;
 * KDA_ERR_MISALIGNED for a z not aligned to its element size or a front-end
 * tensor not 16-byte aligned (gate_bias: 4). */
kda_status kda_chunk_prefill_ex(const kda_dims* dims, const void* q, const void* k,
                                const void* v, const void* g, const void* beta,
                                const float* initial_state, const int32_t* cu_seqlens,
                                void* out, float* final_state, const kda_prefill_options* opts,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Options of kda_decode_step_ex; all-zero means none (kda_decode_step). */
typedef struct {
    int32_t out_gate;            /* kda_out_gate                                          */
    int32_t reserved;            /* must be 0                                             */
    const void* out_gate_z;      /* as in kda_prefill_options with N in place of T_total;
                                    must not overlap out or state_inout                   */
    const kda_front_end* front_end; /* nullable; gate_a is [N, r]                         */
} kda_decode_options;

/* One decode step with options: the output gate and/or the front end.  opts
 * NULL means none.  Errors as for kda_decode_step, plus those listed for the
 * options at kda_chunk_prefill_ex. */
kda_status kda_decode_step_ex(const kda_dims* dims, const void* q, const void* k,
                              const void* v, const void* g, const void* beta,
                              float* state_inout, void* out, const kda_decode_options* opts,
                              void* stream);

/* One decode step: one new token for each of N sequences.
 *
 * dims->total_tokens must equal dims->num_seqs.  q, k, g [N,H,d_k], v [N,H,d_v],
 * beta [N,H] (io_dtype); state_inout fp32 [N,H,d_k,d_v] is advanced in place by
 * one token; out [N,H,d_v] (io_dtype) receives o = S_t^T q_t.  Each
 * (sequence, head) state is read once and written once.  out must not overlap
 * any input or the state.
 */
kda_status kda_decode_step(const kda_dims* dims, const void* q, const void* k,
                           const void* v, const void* g, const void* beta,
                           float* state_inout, void* out, void* stream);

/* Bytes of the per-device array kda_chunk_prefill_noalloc uses as its
 * workspace (320 MiB: the 8,192-token, 32-head, d = 128 bf16 prefill needs
 * 294 MiB). */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)320 << 20)

/* Chunked prefill that allocates nothing, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments (without the workspace), rules and
 * results as kda_chunk_prefill.  Its workspace is a device array of the
 * library, KDA_NOALLOC_SCRATCH_BYTES on each device, allocated when the library
 * is loaded on that device and held until the process ends; its address is
 * looked up once per device on the first call there.  The call never uses the
 * second stream of the pipelined prefill (no library stream or event) and
 * calls no allocating routine.
 * Errors: as kda_chunk_prefill, plus KDA_ERR_WORKSPACE when the path the
 * call takes needs more than KDA_NOALLOC_SCRATCH_BYTES
 * (kda_prefill_path_workspace_bytes).
 * Every call on one device shares that device's array: calls that may run at
 * the same time on one device (different streams without ordering between
 * them) race and corrupt each other's results; order them on one stream.  The
 * array's contents are not preserved between calls (nothing needs to start at
 * zero). */
kda_status kda_chunk_prefill_noalloc(const kda_dims* dims, const void* q, const void* k,
                                     const void* v, const void* g, const void* beta,
                                     const float* initial_state, const int32_t* cu_seqlens,
                                     void* out, float* final_state, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_status_string(kda_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */

// KDA chunked recurrence on gfx950.
//
// For each chunk, in order, starting from the state S at the chunk start
// (the chunk form of the delta rule with a diagonal gate; see kda_prep.hip):
//     u   = U - W S                      (deltas of the chunk's tokens)
//     O   = Qhat S + M u                 (outputs, written to `out`)
//     S  <- Diag(Gamma_C) S + Kprime^T u (state at the chunk end)
// which is the sequential part of the linear-cost chunked prefill ("Kimi K3:
// The Manos, The Mythos, The Legendos", bullet on the two-kernel chunked
// design; update rule of "From KV Cache to Depth Attention: The Bottlenecks
// Kimi K3 Had to Break", Technical Details, KDA bullet).
//
// Parallel split: value columns of S evolve independently (every product above
// acts on S column by column), so one workgroup owns one (sequence, head,
// NT-column tile) chain and keeps that d_k x NT slice of the fp32 state in
// registers for the whole sequence.  Tiles of one (sequence, head) are put on
// the same XCD (blockIdx % 8 selects the XCD) so the W / Qhat / M / Kprime^T
// they all read come from one L2.
//
// Eight waves, two per SIMD.  Wave w works on token block b = w % 4:
//   waves 0-3 compute u = U - W S for block b and publish it (transposed) in LDS;
//   waves 4-7 compute Qhat S for block b and, once u is published, add M u and
//   write the outputs;
//   the state rows are split in 16-row blocks over waves 0..d_k/16-1, each
//   applying Diag(Gamma_C) and adding Kprime^T u to its rows, then publishing
//   the I/O-typed copy of its rows (the MFMA operand of the next chunk).
// No operand of a chunk is used by two waves, so every wave streams its own
// operands from the workspace straight into registers, three chunks ahead (three
// register buffers in rotation; loads are never predicated, so the compiler
// counts the outstanding loads exactly).  Two barriers per chunk.
//
// The eight tiles of a head read the same records at about the same time, so
// each record would arrive from HBM with every tile waiting on it.  Each
// workgroup therefore also touches its eighth (1/ntiles) of the record one chunk
// beyond those in flight, one 128-byte line per lane, which brings the record
// into L2 before the full loads ask for it.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int D, int NT>
struct RecurSmem {
    static constexpr int P = 16 / sizeof(T);
    T ST[NT][D + P];   // I/O-typed copy of S, transposed: [value column][key row]
    T UT[NT][64 + P];  // u, transposed: [value column][token]
};

struct RecurParams {
    const int32_t* cu;
    unsigned char* ws;
    const float* init;
    float* fin;
    void* out;
    float* ckpt;            // checkpoints [C, H, d, d] (checkpointing variant only)
    const void* og_z;       // output-gate pre-activation (gated variant only)
    int64_t total_tokens;
    int32_t n_seqs, n_heads, ntiles;
    int32_t ckpt_interval;  // chunks between checkpoints (checkpointing variant only)
    int32_t og_per_head;    // gated variant: 1 z [T, H], 0 z [T, H, d]
    int64_t chunk_begin;    // chunks [chunk_begin, chunk_end) of every chain; init is the
    int64_t chunk_end;      // state before chunk_begin, fin the state after the range
    PrefillLayout L;
};

// One chunk's operands as held by one wave.
template <typename T, int D, int NT>
struct WaveOps {
    static constexpr int NKS = D / 32;  // 32-deep steps over d_k
    static constexpr int NB = NT / 16;
    typedef T V4 __attribute__((ext_vector_type(4)));
    Frag<T> A[NKS];   // W (waves 0-3) or Qhat (waves 4-7) rows of token block b
    Frag<T> Mf[2];    // M rows of token block b (waves 4-7)
    V4 U[NB];         // U of token block b, this tile (waves 0-3)
    Frag<T> Kt[2];    // Kprime^T rows of this wave's state row block
    f32x4 gc;         // Gamma_C of this wave's state rows (4 per lane)
    uint32_t pf;      // one word of a later chunk's record (L2 prefetch; never used)
    uint32_t zpf;     // one element of a later chunk's output-gate rows (the same)

    // Loads for the phase-one operands (A, and U or M) of record `rec`.
    __device__ __forceinline__ void load_front(const unsigned char* rec, const PrefillLayout& L,
                                               bool uwave, int b, int tile, int lane) {
        const T* a = reinterpret_cast<const T*>(rec + (uwave ? L.off_w : L.off_q));
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) A[ks] = load_frag<T>(a + ((b * NKS + ks) * kWave + lane) * 8);
        if (uwave) {
            const T* u = reinterpret_cast<const T*>(rec + L.off_u);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                U[nb] = *reinterpret_cast<const V4*>(
                    u + ((b * (D / 16) + tile * NB + nb) * kWave + lane) * 4);
        }
    }
    // Loads for the phase-two operands: Kprime^T and Gamma_C of state row block
    // rb, and M (waves 4-7).
    __device__ __forceinline__ void load_back(const unsigned char* rec, const PrefillLayout& L,
                                              bool uwave, int b, int rb, int lane) {
        const T* k = reinterpret_cast<const T*>(rec + L.off_kt);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) Kt[ks] = load_frag<T>(k + ((rb * 2 + ks) * kWave + lane) * 8);
        gc = *reinterpret_cast<const f32x4*>(rec + L.off_gc + (16 * rb + 4 * (lane >> 4)) * 4);
        if (!uwave) {
            const T* m = reinterpret_cast<const T*>(rec + L.off_m);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks == 0 || b >= 2)  // tokens 32.. of blocks 0 and 1 are above the diagonal
                    Mf[ks] = load_frag<T>(m + ((b * 2 + ks) * kWave + lane) * 8);
        }
    }
};

// Per-wave constants of one chain.
struct WaveCtx {
    const unsigned char* rec0;  // record of the chain's first chunk
    size_t rec_bytes;
    int64_t last;               // index of the sequence's last chunk
    int64_t rlast;              // index of the last chunk of this launch's range
    int64_t s_begin;            // first token of the sequence
    int64_t s_len;
    int64_t H;
    int h, col0, tile, w, lane, b, rb;
    int64_t ck0;                // first checkpoint of the sequence
    uint32_t pf_off;            // byte offset of this lane's prefetch line in a record
    uint32_t zpf_off;           // byte offset (in a chunk's z rows) of this lane's z line
    bool zpf_wave;              // the wave that touches z lines ahead (gated variant)
    bool uwave, has_rows;
    __device__ __forceinline__ const unsigned char* rec(int64_t kc) const {
        return rec0 + (size_t)min(kc, rlast) * rec_bytes;
    }
};

// One chunk: consume `ops` (chunk kc), then refill it with chunk kc + NBUF.
// CK: also store the state after every ckpt_interval-th chunk (a checkpoint).
// OG: write out = o * sigmoid(z) (the output gate).
template <typename T, int D, int NT, int NBUF, int PF, bool CK, bool OG>
__device__ __forceinline__ void recur_step(RecurSmem<T, D, NT>& sm, f32x4 (&S)[NT / 16],
                                           WaveOps<T, D, NT>& ops, const RecurParams& p,
                                           const WaveCtx& c, int64_t kc) {
    constexpr int NKS = D / 32;
    constexpr int NB = NT / 16;
    typedef T V4 __attribute__((ext_vector_type(4)));
    const int lane = c.lane;
    const int Lc = (int)min((int64_t)64, c.s_len - 64 * kc);
    const int64_t tok0 = c.s_begin + 64 * kc;

    // Output-gate pre-activations of this chunk's rows, requested before any
    // other load of the step: a load completes only after every load issued
    // before it, so z asked for here is not held up by the operand refills
    // below.  Rows past the sequence's end read as zero (range-checked).  Each
    // is held as its own 32-bit word (16-bit values zero-extended by the load):
    // packing two 16-bit values into one register needs them at once, which
    // would wait for every load in flight, the refills of later chunks included.
    uint32_t zv[NB][4];
    if constexpr (OG) {
        if (!c.uwave) {
            const int64_t zs = p.og_per_head ? c.H : c.H * D;  // elements between tokens
            const int64_t zw = p.og_per_head ? 1 : D;
            const __amdgpu_buffer_rsrc_t zr = make_rsrc(
                reinterpret_cast<const T*>(p.og_z) + (tok0 * c.H + c.h) * zw,
                (uint32_t)(((int64_t)(Lc - 1) * zs + zw) * (int64_t)sizeof(T)));
            const uint32_t zrow = (uint32_t)(zs * (int64_t)sizeof(T));
            const uint32_t zcol = p.og_per_head ? 0u : (uint32_t)sizeof(T);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int col = c.col0 + 16 * nb + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * c.b + 4 * (lane >> 4) + e;
                    const uint32_t off = (uint32_t)row * zrow + (uint32_t)col * zcol;
                    if constexpr (sizeof(T) == 2)
                        zv[nb][e] = (uint32_t)__builtin_bit_cast(uint16_t, buffer_load<uint16_t>(zr, off));
                    else
                        zv[nb][e] = __builtin_bit_cast(uint32_t, buffer_load<float>(zr, off));
                }
            }
        }
    }

    // ---- phase one: A S for token block b (A = W or Qhat)
    Frag<T> Sb[NKS][NB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            Sb[ks][nb] = load_frag<T>(&sm.ST[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) mma(acc[nb], ops.A[ks], Sb[ks][nb]);
    }
    if (c.uwave) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            V4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(to_f32(ops.U[nb][e]) - acc[nb][e]);
            *reinterpret_cast<V4*>(&sm.UT[16 * nb + (lane & 15)][16 * c.b + 4 * (lane >> 4)]) = x;
        }
    }
    ops.load_front(c.rec(kc + NBUF), p.L, c.uwave, c.b, c.tile, lane);
    __syncthreads();

    // ---- phase two: state rows, then M u and the outputs
    Frag<T> Ub[2][NB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            Ub[ks][nb] = load_frag<T>(&sm.UT[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
    if (c.has_rows) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            S[nb] *= ops.gc;
            mma(S[nb], ops.Kt[0], Ub[0][nb]);
            mma(S[nb], ops.Kt[1], Ub[1][nb]);
            V4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(S[nb][e]);
            *reinterpret_cast<V4*>(&sm.ST[16 * nb + (lane & 15)][16 * c.rb + 4 * (lane >> 4)]) = x;
        }
        if constexpr (CK) {
            // state after chunk kc, when kc + 1 is a multiple of the interval and
            // the sequence goes on
            // (chunk counts fit 32 bits: 32-bit division is far cheaper than 64-bit)
            const uint32_t k1 = (uint32_t)kc + 1, iv = (uint32_t)p.ckpt_interval;
            if (k1 % iv == 0 && kc < c.last) {
                const int64_t idx = c.ck0 + (int64_t)(k1 / iv) - 1;
                float* dst = p.ckpt + ((idx * c.H + c.h) * D) * D;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int col = c.col0 + 16 * nb + (lane & 15);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(int64_t)(16 * c.rb + 4 * (lane >> 4) + e) * D + col] = S[nb][e];
                }
            }
        }
    }
    if (!c.uwave) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            mma(acc[nb], ops.Mf[0], Ub[0][nb]);
            if (c.b >= 2) mma(acc[nb], ops.Mf[1], Ub[1][nb]);
        }
    }
    ops.load_back(c.rec(kc + NBUF), p.L, c.uwave, c.b, c.rb, lane);
    if constexpr (PF > 0) {
        // touch this workgroup's share of the record PF chunks beyond the
        // last one requested, so that its lines are in L2 when all tiles ask
        asm volatile("" ::"v"(ops.pf));
        ops.pf = *reinterpret_cast<const uint32_t*>(c.rec(kc + NBUF + PF) + c.pf_off);
    }
    if constexpr (OG && sizeof(T) == 2) {
        // touch this workgroup's share of the z lines of chunk kc + 2, so that
        // the z loads at the start of that step hit L2 (bf16 only: the fp32
        // variant has no registers to spare for it)
        if (c.zpf_wave && kc + 2 <= c.last) {
            asm volatile("" ::"v"(ops.zpf));
            const int L2c = (int)min((int64_t)64, c.s_len - 64 * (kc + 2));
            const int64_t zs = p.og_per_head ? c.H : c.H * D;
            const int64_t zw = p.og_per_head ? 1 : D;
            const __amdgpu_buffer_rsrc_t zr = make_rsrc(
                reinterpret_cast<const T*>(p.og_z) + ((tok0 + 128) * c.H + c.h) * zw,
                (uint32_t)(((int64_t)(L2c - 1) * zs + zw) * (int64_t)sizeof(T)));
            ops.zpf = (uint32_t)__builtin_bit_cast(
                uint16_t, buffer_load<uint16_t>(zr, c.zpf_off));
        }
    }
    if (!c.uwave) {
        if constexpr (OG) {
            // the gate's arithmetic needs only z: pin it here, after the refills
            // are issued (an empty asm that redefines z, ordered after every
            // memory access above), so the scheduler cannot hoist it, and the
            // wait for z, up to the z loads
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) asm volatile("" : "+v"(zv[nb][e])::"memory");
        }
        T* outp = reinterpret_cast<T*>(p.out);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = c.col0 + 16 * nb + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * c.b + 4 * (lane >> 4) + e;
                float o = acc[nb][e];
                if constexpr (OG) {
                    // (a bf16 value is the high half of its fp32 word)
                    const float z = __uint_as_float(sizeof(T) == 2 ? zv[nb][e] << 16 : zv[nb][e]);
                    o *= __builtin_amdgcn_rcpf(1.f + __expf(-z));
                }
                if (row < Lc) outp[((tok0 + row) * c.H + c.h) * D + col] = from_f32<T>(o);
            }
        }
    }
    __syncthreads();
}

template <typename T, int D, int NT, int NBUF, int PF, bool CK, bool OG>
__global__ __launch_bounds__(512) void recur_kernel(RecurParams p) {
    constexpr int NB = NT / 16;
    __shared__ RecurSmem<T, D, NT> sm;

    const int t = threadIdx.x;
    const int bid = blockIdx.x;
    const int chain = 8 * ((bid >> 3) / p.ntiles) + (bid & 7);
    const int tile = (bid >> 3) % p.ntiles;
    if (chain >= p.n_seqs * p.n_heads) return;

    WaveCtx c;
    c.w = t >> 6;
    c.lane = t & 63;
    c.b = c.w & 3;
    c.uwave = c.w < 4;
    c.rb = c.w;
    c.has_rows = c.w < D / 16;
    c.tile = tile;
    c.col0 = tile * NT;
    c.H = p.n_heads;
    const int n = chain / p.n_heads;
    c.h = chain % p.n_heads;
    const int64_t each = p.n_seqs ? p.total_tokens / p.n_seqs : 0;
    c.s_begin = p.cu ? (int64_t)p.cu[n] : (int64_t)n * each;
    c.s_len = p.cu ? (int64_t)p.cu[n + 1] - c.s_begin : each;
    const int64_t nch = (c.s_len + 63) / 64;
    c.last = nch > 0 ? nch - 1 : 0;
    // this launch's chunks; records past the range (possibly not yet written)
    // are never read: the operand refills clamp to its last chunk
    const int64_t kb = min(p.chunk_begin, nch), ke = min(p.chunk_end, nch);
    c.rlast = ke > kb ? ke - 1 : 0;
    c.rec_bytes = p.L.rec_bytes;
    // first chunk slot and first checkpoint of the sequence: from the chunk
    // index for packed sequences, by arithmetic for equal lengths
    int64_t slot0, ck0 = 0;
    if (p.cu) {
        slot0 = reinterpret_cast<const int32_t*>(p.ws)[n];
        if (CK) ck0 = reinterpret_cast<const int32_t*>(p.ws + p.L.ckidx_offset())[n];
    } else {
        slot0 = (int64_t)n * nch;
        if (CK) ck0 = (int64_t)n * (nch > 0 ? (nch - 1) / p.ckpt_interval : 0);
    }
    c.rec0 = p.ws + p.L.records_offset() + ((size_t)c.h * p.L.slots + slot0) * p.L.rec_bytes;
    c.ck0 = ck0;
    const int lane = c.lane;
    {
        // prefetch share: lines [tile * per, (tile + 1) * per) of each record,
        // one 128-byte line per lane (lanes past the share repeat its first line)
        const uint32_t lines = (uint32_t)((p.L.rec_bytes + 127) / 128);
        const uint32_t per = (lines + p.ntiles - 1) / p.ntiles;
        const uint32_t i = (uint32_t)t < per ? (uint32_t)t : 0u;
        const uint32_t line = min((uint32_t)tile * per + i, lines - 1);
        c.pf_off = line * 128;
    }
    {
        // z prefetch share (gated variant): (row, 128-byte part) pairs i = tile +
        // ntiles * lane of a chunk's 64 z rows, one per lane of wave 4 (lanes past
        // the share repeat the first pair)
        const int zrow_bytes = (int)((p.og_per_head ? 1 : D) * sizeof(T));
        const int J = (zrow_bytes + 127) / 128;
        const int per = (64 * J + p.ntiles - 1) / p.ntiles;
        const int l = lane < per ? lane : 0;
        const int i = min(tile + p.ntiles * l, 64 * J - 1);
        const int64_t zs = p.og_per_head ? c.H : c.H * D;
        c.zpf_off = (uint32_t)((i / J) * zs * (int64_t)sizeof(T) + (i % J) * 128);
        c.zpf_wave = OG && c.w == 4;
    }
    // waves without state rows (d_k = 64) read the rows of block 0 in load_back
    // and never use them
    if (!c.has_rows) c.rb = 0;

    // state rows 16*rb .. 16*rb+15 of this tile's columns (waves with rows only)
    f32x4 S[NB];
    const int64_t sbase = ((int64_t)n * c.H + c.h) * D * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = c.col0 + 16 * nb + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * c.rb + 4 * (lane >> 4) + e;
            S[nb][e] = (p.init && c.has_rows) ? p.init[sbase + (int64_t)row * D + col] : 0.f;
        }
    }
    if (c.has_rows) {
        typedef T V4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            V4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(S[nb][e]);
            *reinterpret_cast<V4*>(&sm.ST[16 * nb + (lane & 15)][16 * c.rb + 4 * (lane >> 4)]) = x;
        }
    }
    __syncthreads();

    if (ke > kb) {
        // NBUF named register buffers (an array of them defeats register
        // promotion); chunk kb + j is consumed from buffer j % NBUF
        static_assert(NBUF >= 2 && NBUF <= 5, "prefetch depth");
        WaveOps<T, D, NT> b0, b1, b2, b3, b4;
        auto prime = [&](WaveOps<T, D, NT>& b, int64_t k) {
            b.load_front(c.rec(k), p.L, c.uwave, c.b, tile, lane);
            b.load_back(c.rec(k), p.L, c.uwave, c.b, c.rb, lane);
            if constexpr (PF > 0) b.pf = *reinterpret_cast<const uint32_t*>(c.rec(k + NBUF) + c.pf_off);
        };
        prime(b0, kb);
        prime(b1, kb + 1);
        if constexpr (NBUF > 2) prime(b2, kb + 2);
        if constexpr (NBUF > 3) prime(b3, kb + 3);
        if constexpr (NBUF > 4) prime(b4, kb + 4);
        int64_t kc = kb;
        for (; kc + NBUF <= ke; kc += NBUF) {
            recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b0, p, c, kc);
            recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b1, p, c, kc + 1);
            if constexpr (NBUF > 2) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b2, p, c, kc + 2);
            if constexpr (NBUF > 3) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b3, p, c, kc + 3);
            if constexpr (NBUF > 4) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b4, p, c, kc + 4);
        }
        if (kc < ke) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b0, p, c, kc);
        if constexpr (NBUF > 2)
            if (kc + 1 < ke) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b1, p, c, kc + 1);
        if constexpr (NBUF > 3)
            if (kc + 2 < ke) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b2, p, c, kc + 2);
        if constexpr (NBUF > 4)
            if (kc + 3 < ke) recur_step<T, D, NT, NBUF, PF, CK, OG>(sm, S, b3, p, c, kc + 3);
    }

    if (p.fin && c.has_rows) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = c.col0 + 16 * nb + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * c.rb + 4 * (lane >> 4) + e;
                p.fin[sbase + (int64_t)row * D + col] = S[nb][e];
            }
        }
    }
}

// Chunks whose operands are in flight ahead of the one being consumed (fp32
// operands at d = 128 take twice the registers of bf16 ones: two chunks).
template <typename T, int D>
constexpr int kRecurDepth = (sizeof(T) == 4 && D == 128) ? 2 : 3;
// Chunks beyond those in flight whose records are touched early (L2 prefetch).
constexpr int kRecurPrefetch = 1;

// Column-tile width.  Every tile of a chain streams the same W, Qhat, M and
// Kprime^T, so wider tiles read fewer operand bytes per column but give fewer
// workgroups: 64 columns once that still leaves ~8 workgroups per CU (measured
// -4% per call on 64 packed sequences x 32 heads against 32 columns; not with
// the output gate), 32 while that leaves ~2, 16 otherwise.
static int pick_tile(int64_t chains, int d, bool wide_ok, bool gated) {
    if (wide_ok && !gated && chains * (d / 64) >= 2048) return 64;
    if (wide_ok && chains * (d / 32) >= 512) return 32;
    return 16;
}

template <typename T, int D, int NT>
static hipError_t launch_nt(const PrefillArgs& a, hipStream_t stream) {
    RecurParams p;
    p.cu = a.cu_seqlens;
    p.ws = a.workspace;
    p.init = a.initial_state;
    p.fin = a.final_state;
    p.out = a.out;
    p.ckpt = a.checkpoints;
    p.ckpt_interval = a.ckpt_interval;
    p.og_z = a.out_gate_z;
    p.og_per_head = a.out_gate == 2 ? 1 : 0;
    p.total_tokens = a.total_tokens;
    p.n_seqs = a.n_seqs;
    p.n_heads = a.n_heads;
    p.ntiles = D / NT;
    p.chunk_begin = a.chunk_begin;
    p.chunk_end = a.chunk_end;
    p.L = a.layout;
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    const int64_t groups = (chains + 7) / 8;
    const int64_t grid = 8 * p.ntiles * groups;
    const dim3 gd((unsigned)grid), bd(512);
    constexpr int B = kRecurDepth<T, D>, F = kRecurPrefetch;
    const bool ck = a.ckpt_interval > 0, og = a.out_gate != 0;
    if (!ck && !og)
        hipLaunchKernelGGL((recur_kernel<T, D, NT, B, F, false, false>), gd, bd, 0, stream, p);
    else if (ck && !og)
        hipLaunchKernelGGL((recur_kernel<T, D, NT, B, F, true, false>), gd, bd, 0, stream, p);
    else if constexpr (NT <= 32) {
        // (the gated kernels hold one z word per output element: at 64 columns
        // they would spill, so gated calls never take 64-column tiles)
        if (!ck)
            hipLaunchKernelGGL((recur_kernel<T, D, NT, B, F, false, true>), gd, bd, 0, stream, p);
        else
            hipLaunchKernelGGL((recur_kernel<T, D, NT, B, F, true, true>), gd, bd, 0, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_recur(const PrefillArgs& a, hipStream_t stream) {
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    if (chains == 0) return hipSuccess;
    if constexpr (sizeof(T) == 2) {
        const int nt = pick_tile(chains, D, true, a.out_gate != 0);
        if (nt == 64) return launch_nt<T, D, 64>(a, stream);
        if (nt == 32) return launch_nt<T, D, 32>(a, stream);
    }
    return launch_nt<T, D, 16>(a, stream);
}

template hipError_t launch_recur<bf16, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<float, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<float, 128>(const PrefillArgs&, hipStream_t);

}  // namespace kda

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
// Per chunk, wave w computes u and Qhat S for the 16 tokens of block w; u goes
// through LDS (transposed, as MFMA B operand); then every wave advances its 32
// (d_k = 128) or 16 (d_k = 64) state rows and adds M u to its outputs.  The
// fp32 master state never leaves registers; the I/O-typed copy used as MFMA
// operand is rewritten to LDS once per chunk.  Operands are requested two
// chunks ahead (three register buffers in rotation).
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int D, int NT>
struct RecurSmem {
    static constexpr int P = 16 / sizeof(T);
    T ST[NT][D + P];   // S tile, transposed: [value column][key row]
    T UT[NT][64 + P];  // u tile, transposed: [value column][token]
};

struct RecurParams {
    const int32_t* cu;
    unsigned char* ws;
    const float* init;
    float* fin;
    void* out;
    int64_t total_tokens;
    int32_t n_seqs, n_heads, ntiles;
    PrefillLayout L;
};

// One chunk's operands for one wave: token block w (16 tokens) for u and O,
// key rows 64/4*w.. (D/4 rows) for the state update.
template <typename T, int D, int NT>
struct ChunkOperands {
    static constexpr int NKS = D / 32;
    static constexpr int NB = NT / 16;
    static constexpr int RBW = D / 64;
    typedef T V4 __attribute__((ext_vector_type(4)));
    Frag<T> W[NKS];      // W rows of token block w
    Frag<T> Q[NKS];      // Qhat rows of token block w
    Frag<T> Mf[2];       // M rows of token block w
    Frag<T> Kt[RBW][2];  // Kprime^T rows owned by this wave
    V4 U[NB];            // U, token block w, this tile's columns (accumulator layout)
    f32x4 gC[RBW];       // Gamma_C for this wave's key rows

    __device__ __forceinline__ void load(const unsigned char* rec, const PrefillLayout& L, int w,
                                         int lane, int col0) {
        const T* Wg = reinterpret_cast<const T*>(rec + L.off_w);
        const T* Qg = reinterpret_cast<const T*>(rec + L.off_q);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            W[ks] = load_frag<T>(Wg + ((int64_t)(w * NKS + ks) * kWave + lane) * 8);
            Q[ks] = load_frag<T>(Qg + ((int64_t)(w * NKS + ks) * kWave + lane) * 8);
        }
        const T* Mg = reinterpret_cast<const T*>(rec + L.off_m);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            Mf[ks] = load_frag<T>(Mg + ((int64_t)(w * 2 + ks) * kWave + lane) * 8);
        const T* Kg = reinterpret_cast<const T*>(rec + L.off_kt);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                Kt[rb][ks] = load_frag<T>(Kg + ((int64_t)((RBW * w + rb) * 2 + ks) * kWave + lane) * 8);
        const T* Ug = reinterpret_cast<const T*>(rec + L.off_u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            U[nb] = *reinterpret_cast<const V4*>(
                Ug + corder_index(16 * w + 4 * (lane >> 4), col0 + 16 * nb + (lane & 15), D));
        const float* gcg = reinterpret_cast<const float*>(rec + L.off_gc);
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
            gC[rb] = *reinterpret_cast<const f32x4*>(gcg + 16 * (RBW * w + rb) + 4 * (lane >> 4));
    }
};

// Write the I/O-typed copy of this wave's state rows into the LDS operand tile.
template <typename T, int D, int NT>
__device__ __forceinline__ void put_state(RecurSmem<T, D, NT>& sm,
                                          const f32x4 (&S)[D / 64][NT / 16], int w, int lane) {
    typedef T V4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int rb = 0; rb < D / 64; ++rb)
#pragma unroll
        for (int nb = 0; nb < NT / 16; ++nb) {
            V4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(S[rb][nb][e]);
            *reinterpret_cast<V4*>(
                &sm.ST[16 * nb + (lane & 15)][16 * ((D / 64) * w + rb) + 4 * (lane >> 4)]) = x;
        }
}

// One chunk: u = U - W S, O = Qhat S + M u, S <- Diag(Gamma_C) S + Kprime^T u.
template <typename T, int D, int NT>
__device__ __forceinline__ void recur_step(RecurSmem<T, D, NT>& sm, f32x4 (&S)[D / 64][NT / 16],
                                           const ChunkOperands<T, D, NT>& c, T* outp,
                                           int64_t tok0, int Lc, int64_t H, int h, int col0,
                                           int w, int lane) {
    constexpr int NKS = D / 32;
    constexpr int NB = NT / 16;
    constexpr int RBW = D / 64;
    typedef T V4 __attribute__((ext_vector_type(4)));
    Frag<T> Sb[NKS][NB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            Sb[ks][nb] = load_frag<T>(&sm.ST[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
    f32x4 accO[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        f32x4 au = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            mma(au, c.W[ks], Sb[ks][nb]);
            mma(ao, c.Q[ks], Sb[ks][nb]);
        }
        accO[nb] = ao;
        V4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(to_f32(c.U[nb][e]) - au[e]);
        *reinterpret_cast<V4*>(&sm.UT[16 * nb + (lane & 15)][16 * w + 4 * (lane >> 4)]) = x;
    }
    __syncthreads();
    Frag<T> Ub[2][NB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            Ub[ks][nb] = load_frag<T>(&sm.UT[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            S[rb][nb] *= c.gC[rb];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma(S[rb][nb], c.Kt[rb][ks], Ub[ks][nb]);
        }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) mma(accO[nb], c.Mf[ks], Ub[ks][nb]);
        const int col = col0 + 16 * nb + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * w + 4 * (lane >> 4) + e;
            if (row < Lc) outp[((tok0 + row) * H + h) * D + col] = from_f32<T>(accO[nb][e]);
        }
    }
    put_state<T, D, NT>(sm, S, w, lane);
    __syncthreads();
}

template <typename T, int D, int NT>
__global__ __launch_bounds__(256) void recur_kernel(RecurParams p) {
    constexpr int NB = NT / 16;
    constexpr int RBW = D / 64;
    __shared__ RecurSmem<T, D, NT> sm;

    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int b = blockIdx.x;
    const int chain = 8 * ((b >> 3) / p.ntiles) + (b & 7);
    const int tile = (b >> 3) % p.ntiles;
    const int64_t H = p.n_heads;
    if (chain >= p.n_seqs * p.n_heads) return;
    const int n = chain / p.n_heads, h = chain % p.n_heads;
    const int64_t each = p.n_seqs ? p.total_tokens / p.n_seqs : 0;
    const int64_t s_begin = p.cu ? (int64_t)p.cu[n] : (int64_t)n * each;
    const int64_t s_len = p.cu ? (int64_t)p.cu[n + 1] - s_begin : each;
    const int32_t* cf = reinterpret_cast<const int32_t*>(p.ws);
    const int64_t slot0 = cf[n];
    const int64_t nch = (s_len + 63) / 64;
    const int col0 = tile * NT;

    // initial state slice -> registers (fp32) and LDS (operand copy)
    f32x4 S[RBW][NB];
    const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int col = col0 + 16 * nb + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * (RBW * w + rb) + 4 * (lane >> 4) + e;
                S[rb][nb][e] = p.init ? p.init[sbase + (int64_t)row * D + col] : 0.f;
            }
        }
    put_state<T, D, NT>(sm, S, w, lane);

    const size_t rec_stride = p.L.rec_bytes * (size_t)H;
    const unsigned char* rec0 =
        p.ws + p.L.records_offset() + (size_t)(slot0 * H + h) * p.L.rec_bytes;
    T* outp = reinterpret_cast<T*>(p.out);
    // three operand buffers in rotation: chunk kc's operands are requested at
    // the start of chunk kc-2, so two chunks of compute cover their latency
    ChunkOperands<T, D, NT> b0, b1, b2;
    if (nch > 0) b0.load(rec0, p.L, w, lane, col0);
    if (nch > 1) b1.load(rec0 + rec_stride, p.L, w, lane, col0);
    __syncthreads();
    auto tok = [&](int64_t kc) { return s_begin + 64 * kc; };
    auto len = [&](int64_t kc) { return (int)min((int64_t)64, s_len - 64 * kc); };
    for (int64_t kc = 0; kc < nch; kc += 3) {
        if (kc + 2 < nch) b2.load(rec0 + (size_t)(kc + 2) * rec_stride, p.L, w, lane, col0);
        recur_step<T, D, NT>(sm, S, b0, outp, tok(kc), len(kc), H, h, col0, w, lane);
        if (kc + 1 < nch) {
            if (kc + 3 < nch) b0.load(rec0 + (size_t)(kc + 3) * rec_stride, p.L, w, lane, col0);
            recur_step<T, D, NT>(sm, S, b1, outp, tok(kc + 1), len(kc + 1), H, h, col0, w, lane);
        }
        if (kc + 2 < nch) {
            if (kc + 4 < nch) b1.load(rec0 + (size_t)(kc + 4) * rec_stride, p.L, w, lane, col0);
            recur_step<T, D, NT>(sm, S, b2, outp, tok(kc + 2), len(kc + 2), H, h, col0, w, lane);
        }
    }

    if (p.fin) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int col = col0 + 16 * nb + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * (RBW * w + rb) + 4 * (lane >> 4) + e;
                    p.fin[sbase + (int64_t)row * D + col] = S[rb][nb][e];
                }
            }
    }
}

// Column-tile width: the widest tile that still gives at least ~2 workgroups
// per CU; 16 otherwise (fewest columns per chain, most chains).
static int pick_tile(int64_t chains, int d) {
    if (chains * (d / 32) >= 512) return 32;
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
    p.total_tokens = a.total_tokens;
    p.n_seqs = a.n_seqs;
    p.n_heads = a.n_heads;
    p.ntiles = D / NT;
    p.L = a.layout;
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    const int64_t groups = (chains + 7) / 8;
    const int64_t grid = 8 * p.ntiles * groups;
    hipLaunchKernelGGL((recur_kernel<T, D, NT>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_recur(const PrefillArgs& a, hipStream_t stream) {
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    if (chains == 0) return hipSuccess;
    if (pick_tile(chains, D) == 32) return launch_nt<T, D, 32>(a, stream);
    return launch_nt<T, D, 16>(a, stream);
}

template hipError_t launch_recur<bf16, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<float, 64>(const PrefillArgs&, hipStream_t);

}  // namespace kda

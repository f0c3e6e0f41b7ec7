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
    static constexpr int E = sizeof(T);
    static constexpr int NB = NT / 16;
    // one chunk's operands, laid out as in the workspace record:
    // W | Qhat | M | Kprime^T (contiguous), this tile's U, Gamma_C
    static constexpr int CORE = (192 * D + 64 * 64) * E;
    static constexpr int UBYTES = 4 * NB * 256 * E;
    static constexpr int SLOT = CORE + UBYTES + D * 4;
    T ST[NT][D + P];   // S tile, transposed: [value column][key row]
    T UT[NT][64 + P];  // u tile, transposed: [value column][token]
    alignas(16) unsigned char slot[2][SLOT];
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

// Loader side: one chunk's operands staged in the loader waves' registers
// (16-byte vectors; every loader thread always issues the same loads, so the
// compiler can count outstanding loads exactly).
template <typename T, int D, int NT>
struct Staging {
    typedef RecurSmem<T, D, NT> SM;
    static constexpr int NCORE = SM::CORE / 16 / 256;
    static constexpr int NU = SM::UBYTES / 16;        // U vectors (this tile)
    static constexpr int NG = D / 4;                   // Gamma_C vectors
    static constexpr int NX = (NU + NG + 255) / 256;   // extra vectors per loader
    static_assert(NCORE * 16 * 256 == SM::CORE, "core must split evenly over 256 loaders");
    u32x4 core[NCORE];
    u32x4 extra[NX];

    // source / destination byte offsets of extra vector x (index x < NU + NG)
    __device__ __forceinline__ static void extra_offsets(const PrefillLayout& L, int x, int tile,
                                                         int& src, int& dst) {
        constexpr int E = SM::E;
        constexpr int NB = SM::NB;
        constexpr int per_rb = NB * 256 * E / 16;  // vectors of one 16-row block of this tile's U
        if (x < NU) {
            const int rb = x / per_rb, v = x % per_rb;
            src = (int)L.off_u + ((rb * (D / 16) + tile * NB) * 256) * E + v * 16;
            dst = SM::CORE + rb * NB * 256 * E + v * 16;
        } else {
            const int v = min(x - NU, NG - 1);
            src = (int)L.off_gc + v * 16;
            dst = SM::CORE + SM::UBYTES + v * 16;
        }
    }
    __device__ __forceinline__ void load(const unsigned char* rec, int lt, const int (&src)[NX]) {
#pragma unroll
        for (int i = 0; i < NCORE; ++i)
            core[i] = *reinterpret_cast<const u32x4*>(rec + (size_t)(i * 256 + lt) * 16);
#pragma unroll
        for (int i = 0; i < NX; ++i) extra[i] = *reinterpret_cast<const u32x4*>(rec + src[i]);
    }
    __device__ __forceinline__ void store(unsigned char* slot, int lt, const int (&dst)[NX],
                                          const bool (&has)[NX]) const {
#pragma unroll
        for (int i = 0; i < NCORE; ++i)
            *reinterpret_cast<u32x4*>(slot + (i * 256 + lt) * 16) = core[i];
#pragma unroll
        for (int i = 0; i < NX; ++i)
            if (has[i]) *reinterpret_cast<u32x4*>(slot + dst[i]) = extra[i];
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

// One chunk for compute wave w (token block w; key rows D/4*w..):
// u = U - W S, O = Qhat S + M u, S <- Diag(Gamma_C) S + Kprime^T u,
// with every operand read from the chunk's LDS slot.
template <typename T, int D, int NT>
__device__ __forceinline__ void recur_step(RecurSmem<T, D, NT>& sm, f32x4 (&S)[D / 64][NT / 16],
                                           const unsigned char* slot, T* outp, int64_t tok0,
                                           int Lc, int64_t H, int h, int col0, int w, int lane) {
    typedef RecurSmem<T, D, NT> SM;
    constexpr int NKS = D / 32;
    constexpr int NB = NT / 16;
    constexpr int RBW = D / 64;
    constexpr int E = SM::E;
    typedef T V4 __attribute__((ext_vector_type(4)));
    const T* Wl = reinterpret_cast<const T*>(slot);
    const T* Ql = reinterpret_cast<const T*>(slot + 64 * D * E);
    const T* Ml = reinterpret_cast<const T*>(slot + 128 * D * E);
    const T* Kl = reinterpret_cast<const T*>(slot + (128 * D + 64 * 64) * E);
    const T* Ul = reinterpret_cast<const T*>(slot + SM::CORE);
    const float* Gl = reinterpret_cast<const float*>(slot + SM::CORE + SM::UBYTES);

    Frag<T> Sb[NKS][NB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            Sb[ks][nb] = load_frag<T>(&sm.ST[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
    f32x4 accO[NB];
    {
        Frag<T> Wf[NKS], Qf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            Wf[ks] = load_frag<T>(Wl + ((w * NKS + ks) * kWave + lane) * 8);
            Qf[ks] = load_frag<T>(Ql + ((w * NKS + ks) * kWave + lane) * 8);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            f32x4 au = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                mma(au, Wf[ks], Sb[ks][nb]);
                mma(ao, Qf[ks], Sb[ks][nb]);
            }
            accO[nb] = ao;
            const V4 U = *reinterpret_cast<const V4*>(Ul + ((w * NB + nb) * kWave + lane) * 4);
            V4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = from_f32<T>(to_f32(U[e]) - au[e]);
            *reinterpret_cast<V4*>(&sm.UT[16 * nb + (lane & 15)][16 * w + 4 * (lane >> 4)]) = x;
        }
    }
    __syncthreads();
    Frag<T> Ub[2][NB];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            Ub[ks][nb] = load_frag<T>(&sm.UT[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        const Frag<T> k0 = load_frag<T>(Kl + (((RBW * w + rb) * 2 + 0) * kWave + lane) * 8);
        const Frag<T> k1 = load_frag<T>(Kl + (((RBW * w + rb) * 2 + 1) * kWave + lane) * 8);
        const f32x4 g = *reinterpret_cast<const f32x4*>(Gl + 16 * (RBW * w + rb) + 4 * (lane >> 4));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            S[rb][nb] *= g;
            mma(S[rb][nb], k0, Ub[0][nb]);
            mma(S[rb][nb], k1, Ub[1][nb]);
        }
    }
    const Frag<T> m0 = load_frag<T>(Ml + ((w * 2 + 0) * kWave + lane) * 8);
    const Frag<T> m1 = load_frag<T>(Ml + ((w * 2 + 1) * kWave + lane) * 8);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        mma(accO[nb], m0, Ub[0][nb]);
        mma(accO[nb], m1, Ub[1][nb]);
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

// 512 threads: waves 0-3 compute, waves 4-7 load.  Both sides pass the same
// 1 + 2 * nch barriers.  Chunk kc's operands sit in LDS slot kc % 2; the
// loaders write slot (kc+1) % 2 while the compute waves work on chunk kc, and
// keep chunks kc+2 and kc+3 in flight in their registers.
template <typename T, int D, int NT>
__global__ __launch_bounds__(512) void recur_kernel(RecurParams p) {
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
    const int64_t last = nch > 0 ? nch - 1 : 0;
    const unsigned char* rec0 =
        p.ws + p.L.records_offset() + ((size_t)h * p.L.slots + slot0) * p.L.rec_bytes;
    auto rec = [&](int64_t kc) { return rec0 + (size_t)min(kc, last) * p.L.rec_bytes; };

    if (w >= 4) {
        // ------------------------------------------------------------ loaders
        typedef Staging<T, D, NT> ST_;
        const int lt = t - 256;
        int src_x[ST_::NX], dst_x[ST_::NX];
        bool has_x[ST_::NX];
#pragma unroll
        for (int i = 0; i < ST_::NX; ++i) {
            const int x = lt + 256 * i;
            has_x[i] = x < ST_::NU + ST_::NG;
            ST_::extra_offsets(p.L, has_x[i] ? x : ST_::NU, tile, src_x[i], dst_x[i]);
        }
        ST_ s0, s1;
        if (nch > 0) {
            s0.load(rec(0), lt, src_x);
            s0.store(sm.slot[0], lt, dst_x, has_x);
            s1.load(rec(1), lt, src_x);
            s0.load(rec(2), lt, src_x);
        }
        __syncthreads();
        int64_t kc = 0;
        for (; kc + 2 <= nch; kc += 2) {
            s1.store(sm.slot[1], lt, dst_x, has_x);  // chunk kc+1
            s1.load(rec(kc + 3), lt, src_x);
            __syncthreads();
            __syncthreads();
            s0.store(sm.slot[0], lt, dst_x, has_x);  // chunk kc+2
            s0.load(rec(kc + 4), lt, src_x);
            __syncthreads();
            __syncthreads();
        }
        if (kc < nch) {
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ---------------------------------------------------------------- compute
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
    __syncthreads();
    T* outp = reinterpret_cast<T*>(p.out);
    for (int64_t kc = 0; kc < nch; ++kc)
        recur_step<T, D, NT>(sm, S, sm.slot[kc & 1], outp, s_begin + 64 * kc,
                             (int)min((int64_t)64, s_len - 64 * kc), H, h, col0, w, lane);

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
static int pick_tile(int64_t chains, int d, bool wide_ok) {
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
    p.total_tokens = a.total_tokens;
    p.n_seqs = a.n_seqs;
    p.n_heads = a.n_heads;
    p.ntiles = D / NT;
    p.L = a.layout;
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    const int64_t groups = (chains + 7) / 8;
    const int64_t grid = 8 * p.ntiles * groups;
    hipLaunchKernelGGL((recur_kernel<T, D, NT>), dim3((unsigned)grid), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_recur(const PrefillArgs& a, hipStream_t stream) {
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    if (chains == 0) return hipSuccess;
    // fp32 operands fill LDS at 16 columns already
    if constexpr (sizeof(T) == 2)
        if (pick_tile(chains, D, true) == 32) return launch_nt<T, D, 32>(a, stream);
    return launch_nt<T, D, 16>(a, stream);
}

template hipError_t launch_recur<bf16, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_recur<float, 64>(const PrefillArgs&, hipStream_t);

}  // namespace kda

// KDA chunk preparation on gfx950 (one workgroup per (chunk, head)).
//
// Inside one chunk of C = 64 tokens that starts from state S0, write gamma_r for
// the inclusive cumulative sum of g over the chunk's tokens (per key channel)
// and Gamma_r = exp(gamma_r).  The delta rule with a diagonal gate ("From KV
// Cache to Depth Attention: The Bottlenecks Kimi K3 Had to Break", Technical
// Details, KDA bullet) then unrolls over the chunk as
//     (I + A) u = Diag(beta) (V - Khat S0),  A[s][j] = beta_s sum_c k_s k_j e^(gamma_s - gamma_j)  (j < s)
//     u = U - W S0,  W = T Diag(beta) Khat,  U = T Diag(beta) V,  T = (I + A)^-1
//     O = Qhat S0 + M u,   M[r][j] = sum_c q_r k_j e^(gamma_r - gamma_j)  (j <= r)
//     S_C = Diag(Gamma_C) S0 + Kprime^T u
// with Khat = K Gamma, Qhat = Q Gamma, Kprime = K e^(gamma_C - gamma) -- the
// chunk-wise WY form of the delta rule extended to a per-channel gate, which
// gives the linear-cost chunked prefill of "Kimi K3: The Manos, The Mythos,
// The Legendos" (bullet on the two-kernel chunked design).  This kernel makes
// everything that does not depend on S0: W, U, Qhat, M, Kprime^T and
// Gamma_C, in the layouts the recurrence kernel reads.
//
// Decay factoring.  The chunk is cut into four 16-token blocks.  With rho_R the
// log-decay at the last token of block R (rho_-1 = 0), every exponential is of
// a non-positive number except on the diagonal blocks:
//     E_r = e^(gamma_r - rho_{R-1}),  F_r = e^(rho_R - gamma_r)        (both <= 1)
//     block (R, J<R):  e^(gamma_r - gamma_j) = E_r * e^(rho_{R-1} - rho_J) * F_j
//     block (R, R):    e^(gamma_r - gamma_j) = (E_r / sqrt(D_R)) (F_j / sqrt(D_R)),  D_R = e^(rho_R - rho_{R-1})
// so the products run on MFMA from three decayed copies of q and k (E-, E- and
// F-scaled).  On diagonal blocks the factors stay within e^(+-40) when every
// g >= -5, the documented accuracy range.
//
// Steps (256 threads = 4 waves; wave w owns tokens 16w..16w+15 = block w):
//   P0 load q, k, v, g, beta; L2-normalise q, k; cumulative sum of g per block
//      (in-thread, then across the wave), block totals exchanged through LDS;
//   P1 decay factors; E/F-scaled tiles to LDS; Qhat, Kprime^T, Gamma_C out;
//   P2 A and M blocks on MFMA (A row block w, M row block 3-w per wave);
//   P3 T = (I + A)^-1: the four 16x16 diagonal inverses by forward substitution
//      (one lane per column), then block rows 1..3 by T_RJ = -T_RR sum_K A_RK T_KJ
//      on fp32 MFMA;
//   P4 W and U on MFMA; U, M, W out.
#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

template <typename T, int N>
__device__ __forceinline__ void load_n(const T* p, float (&x)[N]) {
    typedef T V __attribute__((ext_vector_type(N)));
    const V v = *reinterpret_cast<const V*>(p);
#pragma unroll
    for (int j = 0; j < N; ++j) x[j] = to_f32(v[j]);
}

template <typename T, int N>
__device__ __forceinline__ void store_n(T* p, const float (&x)[N]) {
    typedef T V __attribute__((ext_vector_type(N)));
    V v;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = from_f32<T>(x[j]);
    *reinterpret_cast<V*>(p) = v;
}

// acc += A(16x16) * B(16x16), fp32 operands read from LDS (row-major strides).
__device__ __forceinline__ void mm16_lds(f32x4& acc, const float* A, int lda, const float* B,
                                         int ldb) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float a = A[(l & 15) * lda + 4 * m + (l >> 4)];
        const float b = B[(4 * m + (l >> 4)) * ldb + (l & 15)];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
}

template <typename T, int D>
struct PrepSmem {
    static constexpr int P = 16 / sizeof(T);  // 16-byte row padding
    float A[64][65];          // beta-scaled strictly-lower A
    T M[64][64 + P];          // inclusive-lower Q K decay products
    float tau[4][D];          // per-block total log-decay
    float beta[64];
    union {
        struct {
            T KE[64][D + P];
            T QE[64][D + P];
            T KF[64][D + P];
        } a;
        struct {
            T BK[D][64 + P];  // (Diag(beta) Khat)^T
            T BV[D][64 + P];  // (Diag(beta) V)^T
            float Tf[64][65];
            T Tb[64][64 + P];
            float X[4][16][17];
        } b;
        struct {
            T Wst[64][D + P]; // W staging (aliases BK after its last use)
        } c;
    } u;
};

struct PrepParams {
    const void *q, *k, *v, *g, *beta;
    const int32_t* cu;
    unsigned char* ws;
    int64_t total_tokens;
    int32_t n_seqs, n_heads;
    float scale;
    int l2norm;
    PrefillLayout L;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
    constexpr int CPT = D / 16;  // channels per thread in the row layout
    constexpr int NKS = D / 32;  // 32-deep k-steps over the channels
    __shared__ PrepSmem<T, D> sm;

    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int rg = t >> 4, cg = t & 15, grp = lane >> 4;
    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t H = p.n_heads;
    const int32_t* cf = reinterpret_cast<const int32_t*>(p.ws);
    const int N = p.n_seqs;
    if (slot >= cf[N]) return;
    // sequence owning this chunk slot: largest n with cf[n] <= slot
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cf[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    const int n = lo;
    const int64_t each = N ? p.total_tokens / N : 0;
    const int64_t s_begin = p.cu ? (int64_t)p.cu[n] : (int64_t)n * each;
    const int64_t s_end = p.cu ? (int64_t)p.cu[n + 1] : s_begin + each;
    const int64_t t0 = s_begin + 64 * (slot - cf[n]);
    const int Lc = (int)min((int64_t)64, s_end - t0);

    unsigned char* rec = p.ws + p.L.index_bytes + (size_t)(slot * H + h) * p.L.rec_bytes;

    // ---------------------------------------------------------------- P0
    const T* qg = (const T*)p.q;
    const T* kg = (const T*)p.k;
    const T* vg = (const T*)p.v;
    const T* gg = (const T*)p.g;
    float qf[4][CPT], kf[4][CPT], gf[4][CPT], vf[4][CPT];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        if (r < Lc) {
            const int64_t off = ((t0 + r) * H + h) * D + CPT * cg;
            load_n<T, CPT>(qg + off, qf[i]);
            load_n<T, CPT>(kg + off, kf[i]);
            load_n<T, CPT>(gg + off, gf[i]);
            load_n<T, CPT>(vg + off, vf[i]);
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) qf[i][c] = kf[i][c] = gf[i][c] = vf[i][c] = 0.f;
        }
    }
    float bt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        bt[i] = (r < Lc) ? to_f32(((const T*)p.beta)[(t0 + r) * H + h]) : 0.f;
        if (cg == 0) sm.beta[r] = bt[i];
    }
    // L2 norms over the 16 lanes that share a row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            sq += qf[i][c] * qf[i][c];
            sk += kf[i][c] * kf[i][c];
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
            sq += xor_shfl(sq, m);
            sk += xor_shfl(sk, m);
        }
        const float rq = (p.l2norm ? 1.0f / sqrtf(sq + kL2Eps) : 1.0f) * p.scale;
        const float rk = p.l2norm ? 1.0f / sqrtf(sk + kL2Eps) : 1.0f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            qf[i][c] *= rq;
            kf[i][c] *= rk;
        }
    }
    // cumulative log-decay inside the 16-token block: in-thread, then across
    // the four 4-row groups of the wave (inclusive scan, then shift by one group)
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        gf[1][c] += gf[0][c];
        gf[2][c] += gf[1][c];
        gf[3][c] += gf[2][c];
        const float tot = gf[3][c];
        float incl = tot;
        float x = __shfl_up(incl, 16, kWave);
        if (grp >= 1) incl += x;
        x = __shfl_up(incl, 32, kWave);
        if (grp >= 2) incl += x;
        float ex = __shfl_up(incl, 16, kWave);
        if (grp == 0) ex = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) gf[i][c] += ex;
        const float tau = __shfl(gf[3][c], 48 + cg, kWave);  // block total = last row
        if (grp == 0) sm.tau[w][CPT * cg + c] = tau;
    }
    __syncthreads();

    // ---------------------------------------------------------------- P1
    float tauR[CPT], rho_prev[CPT], rho_after[CPT], gamC[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        float tv[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) tv[R] = sm.tau[R][CPT * cg + c];
        tauR[c] = tv[w];
        float before = 0.f, after = 0.f;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            if (R < w) before += tv[R];
            if (R > w) after += tv[R];
        }
        rho_prev[c] = before;   // log-decay from the chunk start to this block's start
        rho_after[c] = after;   // log-decay from this block's end to the chunk end
        gamC[c] = ((tv[0] + tv[1]) + tv[2]) + tv[3];
    }
    float Gs[CPT], Kp[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        Gs[c] = __expf(rho_prev[c]);
        Kp[c] = __expf(rho_after[c]);
    }
    T* Qg = reinterpret_cast<T*>(rec + p.L.off_q);
    T* Ktg = reinterpret_cast<T*>(rec + p.L.off_kt);
    float bK[4][CPT], bV[4][CPT];
    float kpT[CPT][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * rg + i;
        float ke[CPT], qe[CPT], kfv[CPT], qh[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float E = __expf(gf[i][c]);
            const float F = __expf(tauR[c] - gf[i][c]);
            ke[c] = kf[i][c] * E;
            qe[c] = qf[i][c] * E;
            kfv[c] = kf[i][c] * F;
            qh[c] = qe[c] * Gs[c];
            bK[i][c] = bt[i] * ke[c] * Gs[c];
            bV[i][c] = bt[i] * vf[i][c];
            kpT[c][i] = kfv[c] * Kp[c];
        }
        store_n<T, CPT>(&sm.u.a.KE[r][CPT * cg], ke);
        store_n<T, CPT>(&sm.u.a.QE[r][CPT * cg], qe);
        store_n<T, CPT>(&sm.u.a.KF[r][CPT * cg], kfv);
        store_n<T, CPT>(Qg + aorder_index(r, CPT * cg, D), qh);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) store_n<T, 4>(Ktg + aorder_index(CPT * cg + c, 4 * rg, 64), kpT[c]);
    if (rg == 0) {
        float* gC = reinterpret_cast<float*>(rec + p.L.off_gc);
#pragma unroll
        for (int c = 0; c < CPT; ++c) gC[CPT * cg + c] = __expf(gamC[c]);
    }
    __syncthreads();

    // ---------------------------------------------------------------- P2
    // block (R, J): isA -> A (rows from KE, beta-scaled, strict), else M (rows from QE, inclusive)
    auto block = [&](bool isA, int R, int J) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (J <= R) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = 32 * ks + 8 * (lane >> 4);
                Frag<T> a = load_frag<T>(isA ? &sm.u.a.KE[16 * R + (lane & 15)][c0]
                                             : &sm.u.a.QE[16 * R + (lane & 15)][c0]);
                Frag<T> b = load_frag<T>(&sm.u.a.KF[16 * J + (lane & 15)][c0]);
                if (J == R) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float f = __expf(-0.5f * sm.tau[R][c0 + j]);
                        a.v[j] = from_f32<T>(to_f32(a.v[j]) * f);
                        b.v[j] = from_f32<T>(to_f32(b.v[j]) * f);
                    }
                } else if (J < R - 1) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float s = 0.f;
                        for (int m = J + 1; m < R; ++m) s += sm.tau[m][c0 + j];
                        b.v[j] = from_f32<T>(to_f32(b.v[j]) * __expf(s));
                    }
                }
                mma(acc, a, b);
            }
        }
        const int col = lane & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * (lane >> 4) + e;
            float val = acc[e];
            if (isA) {
                val *= sm.beta[16 * R + row];
                if (J > R || (J == R && col >= row)) val = 0.f;
                sm.A[16 * R + row][16 * J + col] = val;
            } else {
                if (J > R || (J == R && col > row)) val = 0.f;
                sm.M[16 * R + row][16 * J + col] = from_f32<T>(val);
            }
        }
    };
    for (int J = 0; J < 4; ++J) block(true, w, J);
    for (int J = 0; J < 4; ++J) block(false, 3 - w, J);
    __syncthreads();

    // ---------------------------------------------------------------- P3
    // transposed beta*Khat and beta*V tiles (the B operands of W and U)
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        float xk[4], xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xk[i] = bK[i][c];
            xv[i] = bV[i][c];
        }
        store_n<T, 4>(&sm.u.b.BK[CPT * cg + c][4 * rg], xk);
        store_n<T, 4>(&sm.u.b.BV[CPT * cg + c][4 * rg], xv);
    }
    if (w == 0) {
        // diagonal 16x16 blocks of (I + A)^-1: lane = (block, column), forward substitution
        const int R = lane >> 4, j = lane & 15;
        float colv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc += sm.A[16 * R + i][16 * R + kk] * colv[kk];
            colv[i] = (i == j) ? 1.f : ((i < j) ? 0.f : -acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.u.b.Tf[16 * R + i][16 * R + j] = colv[i];
    }
    __syncthreads();
    for (int R = 1; R < 4; ++R) {
        if (w < R) {
            const int J = w;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < R; ++K)
                mm16_lds(x, &sm.A[16 * R][16 * K], 65, &sm.u.b.Tf[16 * K][16 * J], 65);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.b.X[w][4 * (lane >> 4) + e][lane & 15] = -x[e];
        }
        __syncthreads();
        if (w < R) {
            const int J = w;
            f32x4 tt = {0.f, 0.f, 0.f, 0.f};
            mm16_lds(tt, &sm.u.b.Tf[16 * R][16 * R], 65, &sm.u.b.X[w][0][0], 17);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.b.Tf[16 * R + 4 * (lane >> 4) + e][16 * J + (lane & 15)] = tt[e];
        }
        __syncthreads();
    }
    for (int idx = t; idx < 64 * 64; idx += 256) {
        const int r = idx >> 6, c = idx & 63;
        sm.u.b.Tb[r][c] = from_f32<T>(c <= r ? sm.u.b.Tf[r][c] : 0.f);
    }
    __syncthreads();

    // ---------------------------------------------------------------- P4
    {
        const int R = w;
        const int nks = (R >= 2) ? 2 : 1;  // T[R][J] = 0 for blocks J > R
        Frag<T> ta[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks < nks) ta[ks] = load_frag<T>(&sm.u.b.Tb[16 * R + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
        f32x4 accW[D / 16];
        T* Ug = reinterpret_cast<T*>(rec + p.L.off_u);
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
            f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks < nks) {
                    const Frag<T> bk = load_frag<T>(&sm.u.b.BK[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
                    const Frag<T> bv = load_frag<T>(&sm.u.b.BV[16 * nb + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
                    mma(aw, ta[ks], bk);
                    mma(au, ta[ks], bv);
                }
            }
            accW[nb] = aw;
            float uv[4] = {au[0], au[1], au[2], au[3]};
            store_n<T, 4>(Ug + corder_index(16 * R + 4 * (lane >> 4), 16 * nb + (lane & 15), D), uv);
        }
        T* Mg = reinterpret_cast<T*>(rec + p.L.off_m);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const Frag<T> f = load_frag<T>(&sm.M[16 * w + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
            store_frag<T>(Mg + ((int64_t)(w * 2 + ks) * kWave + lane) * 8, f);
        }
        __syncthreads();  // every wave is done with BK / BV
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.u.c.Wst[16 * R + 4 * (lane >> 4) + e][16 * nb + (lane & 15)] = from_f32<T>(accW[nb][e]);
        __syncthreads();
        T* Wg = reinterpret_cast<T*>(rec + p.L.off_w);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const Frag<T> f = load_frag<T>(&sm.u.c.Wst[16 * w + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
            store_frag<T>(Wg + ((int64_t)(w * NKS + ks) * kWave + lane) * 8, f);
        }
    }
}

// Chunk index: cf[n] = first chunk slot of sequence n, cf[N] = number of chunks.
// One workgroup; sequences are processed 256 at a time with a running carry.
__global__ __launch_bounds__(256) void chunk_index_kernel(const int32_t* __restrict__ cu,
                                                          int32_t n_seqs, int64_t total_tokens,
                                                          int32_t* __restrict__ cf) {
    __shared__ int32_t s_scan[256];
    const int t = threadIdx.x;
    const int64_t each = n_seqs ? total_tokens / n_seqs : 0;
    int32_t carry = 0;
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + t;
        int32_t c = 0;
        if (n < n_seqs) {
            const int64_t len = cu ? (int64_t)cu[n + 1] - cu[n] : each;
            c = (int32_t)((len + 63) / 64);
        }
        s_scan[t] = c;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t x = (t >= off) ? s_scan[t - off] : 0;
            __syncthreads();
            s_scan[t] += x;
            __syncthreads();
        }
        if (n < n_seqs) cf[n] = carry + s_scan[t] - c;
        carry += s_scan[255];
        __syncthreads();
    }
    if (t == 0) cf[n_seqs] = carry;
}

template <typename T, int D>
hipError_t launch_prep(const PrefillArgs& a, hipStream_t stream) {
    PrepParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta;
    p.cu = a.cu_seqlens;
    p.ws = a.workspace;
    p.total_tokens = a.total_tokens;
    p.n_seqs = a.n_seqs;
    p.n_heads = a.n_heads;
    p.scale = a.scale;
    p.l2norm = a.l2norm;
    p.L = a.layout;
    hipLaunchKernelGGL((chunk_index_kernel), dim3(1), dim3(256), 0, stream, a.cu_seqlens,
                       a.n_seqs, a.total_tokens, reinterpret_cast<int32_t*>(a.workspace));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.total_tokens == 0) return hipSuccess;
    hipLaunchKernelGGL((prep_kernel<T, D>), dim3((unsigned)a.layout.slots, (unsigned)a.n_heads),
                       dim3(256), 0, stream, p);
    return hipGetLastError();
}

template hipError_t launch_prep<bf16, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<float, 64>(const PrefillArgs&, hipStream_t);

}  // namespace kda

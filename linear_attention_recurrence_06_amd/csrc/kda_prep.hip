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
//     block (R, R):    e^(gamma_r - gamma_j) = (E_r / D_R) F_j,  D_R = e^(rho_R - rho_{R-1})
// so the products run on MFMA from three decayed copies of q and k (E-, E- and
// F-scaled).  On diagonal blocks 1/D_R stays below e^80 (and F_j above e^-80)
// when every g >= -5, the documented accuracy range.
//
// Work split: a persistent grid (one workgroup per CU) walks the (chunk slot,
// head) items; each workgroup loads the next item's raw rows while it computes
// the current one, and the item after that's descriptor one step earlier, so
// global-memory latency overlaps the arithmetic.
//
// Steps per item (256 threads = 4 waves; wave w owns tokens 16w..16w+15 = block w):
//   P0 L2-normalise q, k; cumulative sum of g per block (in-thread, then across
//      the wave); block totals through LDS, then a per-channel table of every
//      block-level decay factor (16 x d_k exponentials per chunk);
//   P1 element decay factors; E/F-scaled tiles to LDS; Qhat, Kprime^T, Gamma_C out;
//   P2 A and M blocks on MFMA (row block w of both per wave);
//   P3 T = (I + A)^-1: the four 16x16 diagonal inverses by forward substitution
//      (one lane per column), then block rows 1..3 by T_RJ = -T_RR sum_K A_RK T_KJ
//      on fp32 MFMA;
//   P4 W and U on MFMA; U, M, W out.
#include <algorithm>

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
    float A[64][68];          // beta-scaled strictly-lower A (16-byte aligned rows)
    T M[64][64 + P];          // inclusive-lower Q K decay products
    float tau[4][D];          // per-block total log-decay
    // per-channel decay factors, rows: 0-3 e^(-tau_R); 4 e^(tau_1); 5 e^(tau_1+tau_2);
    // 6 e^(tau_2); 7-10 e^(rho_{R-1}) (chunk start -> block R start); 11-14
    // e^(rho_3 - rho_R) (block R end -> chunk end); 15 e^(rho_3) = Gamma_C
    float fac[16][D];
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

// Row block R of A (beta-scaled, strictly lower) and of M (inclusive lower):
// for every column block J <= R the K-side operand (KF rows of block J) is
// loaded once and feeds both products, so each wave runs two independent MFMA
// chains; blocks J > R are zero.
template <typename T, int D>
__device__ __forceinline__ void decay_row_block(PrepSmem<T, D>& sm, int R, int lane) {
    constexpr int NKS = D / 32;
    Frag<T> ke[NKS], qe[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * (lane >> 4);
        ke[ks] = load_frag<T>(&sm.u.a.KE[16 * R + (lane & 15)][c0]);
        qe[ks] = load_frag<T>(&sm.u.a.QE[16 * R + (lane & 15)][c0]);
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        f32x4 acc_a = {0.f, 0.f, 0.f, 0.f}, acc_m = {0.f, 0.f, 0.f, 0.f};
        if (J <= R) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = 32 * ks + 8 * (lane >> 4);
                Frag<T> b = load_frag<T>(&sm.u.a.KF[16 * J + (lane & 15)][c0]);
                Frag<T> a = ke[ks], q = qe[ks];
                if (J == R) {
                    // diagonal block: e^(gamma_r - gamma_j) = E_r F_j / D_R, on the row side
                    const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sm.fac[R][c0]);
                    const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sm.fac[R][c0 + 4]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float f = j < 4 ? f0[j] : f1[j - 4];
                        a.v[j] = from_f32<T>(to_f32(a.v[j]) * f);
                        q.v[j] = from_f32<T>(to_f32(q.v[j]) * f);
                    }
                } else if (J < R - 1) {
                    const int row = (R == 2) ? 4 : 5 + J;  // e^(rho_{R-1} - rho_J)
                    const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sm.fac[row][c0]);
                    const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sm.fac[row][c0 + 4]);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        b.v[j] = from_f32<T>(to_f32(b.v[j]) * (j < 4 ? f0[j] : f1[j - 4]));
                }
                mma(acc_a, a, b);
                mma(acc_m, q, b);
            }
        }
        const int col = lane & 15;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * (lane >> 4) + e;
            float va = acc_a[e] * sm.beta[16 * R + row];
            float vm = acc_m[e];
            if (J > R || (J == R && col >= row)) va = 0.f;
            if (J > R || (J == R && col > row)) vm = 0.f;
            sm.A[16 * R + row][16 * J + col] = va;
            sm.M[16 * R + row][16 * J + col] = from_f32<T>(vm);
        }
    }
}

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

// (first token, length) of a chunk slot; length 0 marks an unused slot.
__device__ __forceinline__ int2 slot_desc(const PrepParams& p, int64_t slot) {
    if (p.cu) return reinterpret_cast<const int2*>(p.ws + p.L.index_bytes)[slot];
    const int64_t N = p.n_seqs;
    const int64_t each = p.total_tokens / N;
    const int64_t per = (each + 63) / 64;
    if (per == 0 || slot >= per * N) return make_int2(0, 0);
    const int64_t n = slot / per, kc = slot - n * per;
    return make_int2((int)(n * each + 64 * kc), (int)min((int64_t)64, each - 64 * kc));
}

// One thread's share of a chunk's raw input rows (rows 4*rg..4*rg+3, channels
// CPT*cg..+CPT-1), kept in the I/O type so the next item's rows can be in
// flight while the current item computes.
template <typename T, int D>
struct RawRows {
    static constexpr int CPT = D / 16;
    typedef T V __attribute__((ext_vector_type(CPT)));
    V q[4], k[4], g[4], v[4];
    T b[4];

    // Rows past the chunk's length are loaded from its first row (always a
    // valid token) and zeroed by the caller, so the loads are never predicated
    // and the compiler can keep the next item's rows in flight.
    __device__ __forceinline__ void load(const PrepParams& p, int2 d, int h, int rg, int cg) {
        const int64_t H = p.n_heads;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            const int64_t row = (int64_t)d.x + (r < d.y ? r : 0);
            const int64_t off = (row * H + h) * D + CPT * cg;
            q[i] = *reinterpret_cast<const V*>((const T*)p.q + off);
            k[i] = *reinterpret_cast<const V*>((const T*)p.k + off);
            g[i] = *reinterpret_cast<const V*>((const T*)p.g + off);
            v[i] = *reinterpret_cast<const V*>((const T*)p.v + off);
            b[i] = ((const T*)p.beta)[row * H + h];
        }
    }
};

// Everything for one (chunk slot, head) item whose raw rows are already in
// registers (converted to fp32).  Ends with a barrier so the next item may
// reuse the shared memory.
template <typename T, int D>
__device__ __forceinline__ void prep_item(const PrepParams& p, PrepSmem<T, D>& sm, int64_t slot,
                                          int h, float (&qf)[4][D / 16], float (&kf)[4][D / 16],
                                          float (&gf)[4][D / 16], const float (&vf)[4][D / 16],
                                          const float (&bt)[4]) {
    constexpr int CPT = D / 16;  // channels per thread in the row layout
    constexpr int NKS = D / 32;  // 32-deep k-steps over the channels
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int rg = t >> 4, cg = t & 15, grp = lane >> 4;
    unsigned char* rec = p.ws + p.L.records_offset() + ((size_t)h * p.L.slots + slot) * p.L.rec_bytes;

    // ---------------------------------------------------------------- P0
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (cg == 0) sm.beta[4 * rg + i] = bt[i];
    // L2 norms over the 16 lanes that share a row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            sq += qf[i][c] * qf[i][c];
            sk += kf[i][c] * kf[i][c];
        }
        sq = row16_sum(sq);
        sk = row16_sum(sk);
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
        float incl = gf[3][c];
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
    // per-channel table of the block-level decay factors (16 x D exponentials):
    // thread t owns channel t % D and rows t / D + (256 / D) * i
    {
        constexpr int RSTEP = 256 / D;
        const int c = t % D, r0 = t / D;
        const float t0 = sm.tau[0][c], t1 = sm.tau[1][c], t2 = sm.tau[2][c], t3 = sm.tau[3][c];
        const float x[16] = {-t0, -t1, -t2, -t3,
                             t1, t1 + t2, t2,
                             0.f, t0, t0 + t1, (t0 + t1) + t2,
                             (t1 + t2) + t3, t2 + t3, t3, 0.f,
                             ((t0 + t1) + t2) + t3};
#pragma unroll
        for (int i = 0; i < 16 / RSTEP; ++i) {
            const int row = r0 + RSTEP * i;
            float v = x[0];
#pragma unroll
            for (int k = 1; k < 16; ++k) v = (row == k) ? x[k] : v;
            sm.fac[row][c] = __expf(v);
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P1
    T* Qg = reinterpret_cast<T*>(rec + p.L.off_q);
    T* Ktg = reinterpret_cast<T*>(rec + p.L.off_kt);
    float bK[4][CPT], bV[4][CPT];
    float kpT[CPT][4];
    float tauR[CPT], Gs[CPT], Kp[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        tauR[c] = sm.tau[w][CPT * cg + c];
        Gs[c] = sm.fac[7 + w][CPT * cg + c];
        Kp[c] = sm.fac[11 + w][CPT * cg + c];
    }
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
        for (int c = 0; c < CPT; ++c) gC[CPT * cg + c] = sm.fac[15][CPT * cg + c];
    }
    __syncthreads();

    // ---------------------------------------------------------------- P2
    decay_row_block<T, D>(sm, w, lane);
    __syncthreads();

    // ---------------------------------------------------------------- P3
    // transposed beta*Khat and beta*V tiles (the B operands of W and U).  Lane
    // (rg, cg) holds 4 tokens x CPT channels; at write step j it stores channel
    // (j + cg) % CPT, so the 16 lanes of a token group spread over the banks
    // (a plain channel order puts them on two bank positions).  The rotation is
    // a barrel shift of packed token quadruples across the channel index.
    {
        typedef T V4 __attribute__((ext_vector_type(4)));
        V4 rk[CPT], rv[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rk[c][i] = from_f32<T>(bK[i][c]);
                rv[c][i] = from_f32<T>(bV[i][c]);
            }
        }
#pragma unroll
        for (int sh = 1; sh < CPT; sh <<= 1) {
            const bool on = (cg & sh) != 0;
            V4 tk[CPT], tv[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                tk[j] = on ? rk[(j + sh) % CPT] : rk[j];
                tv[j] = on ? rv[(j + sh) % CPT] : rv[j];
            }
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                rk[j] = tk[j];
                rv[j] = tv[j];
            }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = CPT * cg + ((j + cg) % CPT);
            *reinterpret_cast<V4*>(&sm.u.b.BK[c][4 * rg]) = rk[j];
            *reinterpret_cast<V4*>(&sm.u.b.BV[c][4 * rg]) = rv[j];
        }
    }
    if (w == 0) {
        // diagonal 16x16 blocks of (I + A)^-1: lane = (block, column), forward
        // substitution; every row of A_RR is read with 16-byte loads up front
        const int R = lane >> 4, j = lane & 15;
        float arow[16][16];
#pragma unroll
        for (int i = 1; i < 16; ++i)
#pragma unroll
            for (int q4 = 0; q4 < (i + 3) / 4; ++q4) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.A[16 * R + i][16 * R + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) arow[i][4 * q4 + e] = a4[e];
            }
        float colv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc += arow[i][kk] * colv[kk];
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
                mm16_lds(x, &sm.A[16 * R][16 * K], 68, &sm.u.b.Tf[16 * K][16 * J], 65);
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
    {
        // thread t converts row t / 4, columns 16 * (t % 4) .. +15 (zero above the diagonal)
        const int r = t >> 2, c0 = 16 * (t & 3);
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = (c0 + j <= r) ? sm.u.b.Tf[r][c0 + j] : 0.f;
        float lo[8], hi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            lo[j] = x[j];
            hi[j] = x[8 + j];
        }
        store_frag<T>(&sm.u.b.Tb[r][c0], make_frag<T>(lo));
        store_frag<T>(&sm.u.b.Tb[r][c0 + 8], make_frag<T>(hi));
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
    __syncthreads();  // the next item overwrites the shared tiles
}

// Persistent driver: item = slot * H + head; workgroup b takes items b, b + G, ...
template <typename T, int D>
__global__ __launch_bounds__(256) void prep_kernel(PrepParams p) {
    constexpr int CPT = D / 16;
    __shared__ PrepSmem<T, D> sm;
    const int t = threadIdx.x;
    const int rg = t >> 4, cg = t & 15;
    const int64_t H = p.n_heads;
    const int64_t items = p.L.slots * H;
    const int64_t G = gridDim.x;
    int64_t item = blockIdx.x;
    if (item >= items) return;
    // (slot, head) of item, item + G, item + 2G, stepped without 64-bit divisions
    const int gh = (int)(G % H);
    const int64_t gs = G / H;
    auto advance = [&](int64_t& s, int& hh) {
        s += gs;
        hh += gh;
        if (hh >= H) {
            hh -= (int)H;
            s += 1;
        }
    };
    int64_t s0 = item / H;
    int h0 = (int)(item % H);
    int64_t s1 = s0, s2;
    int h1 = h0, h2;
    advance(s1, h1);
    s2 = s1;
    h2 = h1;
    advance(s2, h2);

    RawRows<T, D> raw;
    int2 d_cur = slot_desc(p, s0);
    int2 d_nxt = item + G < items ? slot_desc(p, s1) : make_int2(0, 0);
    raw.load(p, d_cur, h0, rg, cg);
    for (; item < items; item += G) {
        const int2 d = d_cur;
        float qf[4][CPT], kf[4][CPT], gf[4][CPT], vf[4][CPT], bt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = 4 * rg + i < d.y;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                qf[i][c] = ok ? to_f32(raw.q[i][c]) : 0.f;
                kf[i][c] = ok ? to_f32(raw.k[i][c]) : 0.f;
                gf[i][c] = ok ? to_f32(raw.g[i][c]) : 0.f;
                vf[i][c] = ok ? to_f32(raw.v[i][c]) : 0.f;
            }
            bt[i] = ok ? to_f32(raw.b[i]) : 0.f;
        }
        // next item's rows go in flight now (past the last item: the current one
        // again, never used); the descriptor after it one step earlier
        const bool more = item + G < items;
        raw.load(p, more ? d_nxt : d, more ? h1 : h0, rg, cg);
        const int2 d_nn = item + 2 * G < items ? slot_desc(p, s2) : make_int2(0, 0);
        if (d.y > 0) prep_item<T, D>(p, sm, s0, h0, qf, kf, gf, vf, bt);
        d_cur = d_nxt;
        d_nxt = d_nn;
        s0 = s1; h0 = h1;
        s1 = s2; h1 = h2;
        advance(s2, h2);
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

// Chunk-slot descriptors for packed sequences: desc[s] = (first token, length)
// of chunk slot s (length 0 for slots past the last chunk).
__global__ __launch_bounds__(256) void chunk_desc_kernel(const int32_t* __restrict__ cu,
                                                         int32_t n_seqs,
                                                         const int32_t* __restrict__ cf,
                                                         int64_t slots, int2* __restrict__ desc) {
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (s >= slots) return;
    if (s >= cf[n_seqs]) {
        desc[s] = make_int2(0, 0);
        return;
    }
    int lo = 0, hi = n_seqs - 1;  // largest n with cf[n] <= s
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cf[mid] <= s) lo = mid; else hi = mid - 1;
    }
    const int64_t t0 = (int64_t)cu[lo] + 64 * (s - cf[lo]);
    desc[s] = make_int2((int)t0, (int)min((int64_t)64, (int64_t)cu[lo + 1] - t0));
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
    int32_t* cf = reinterpret_cast<int32_t*>(a.workspace);
    hipLaunchKernelGGL((chunk_index_kernel), dim3(1), dim3(256), 0, stream, a.cu_seqlens,
                       a.n_seqs, a.total_tokens, cf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.total_tokens == 0) return hipSuccess;
    if (a.cu_seqlens) {
        const unsigned nb = (unsigned)((a.layout.slots + 255) / 256);
        hipLaunchKernelGGL((chunk_desc_kernel), dim3(nb), dim3(256), 0, stream, a.cu_seqlens,
                           a.n_seqs, cf, a.layout.slots,
                           reinterpret_cast<int2*>(a.workspace + a.layout.index_bytes));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t items = a.layout.slots * a.n_heads;
    const int64_t grid = std::min<int64_t>(items, (int64_t)a.cu_count);
    hipLaunchKernelGGL((prep_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template hipError_t launch_prep<bf16, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<float, 64>(const PrefillArgs&, hipStream_t);

}  // namespace kda

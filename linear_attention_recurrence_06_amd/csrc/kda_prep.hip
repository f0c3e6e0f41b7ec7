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
//     block (R, R):    e^(gamma_r - gamma_j) = E_r (F_j / D_R),  D_R = e^(rho_R - rho_{R-1})
// so the products run on MFMA from three decayed copies of q and k (E-, E- and
// F-scaled), the middle factor and 1/D_R applied per channel to the F-scaled
// operand.  Off the diagonal every factor is at most 1.  On a diagonal block
// F_j / D_R can reach 1/D_R, so the factored form is used only while every
// channel's block decay keeps 1/D_R <= 2^64; a block past that is computed
// exactly instead, from its raw rows, with every factor at most 1: a pair
// (r, j), j < r, of one 16-token block is split at the first bisection level
// that separates them (halves of 8, 4, 2, 1 tokens), and with b the last token
// of the left half at that level,
//     e^(gamma_r - gamma_j) = e^(gamma_r - gamma_b) * e^(gamma_b - gamma_j),
// both factors <= 1.  Each level is one masked MFMA product of row-scaled and
// column-scaled copies of the block's rows, so any g <= 0 is handled.  Per-token
// decay is floored at 2^-128 (g log2 e >= -128): a smaller retention makes no
// difference to any fp32 result, and the floor bounds the in-block sums.
//
// Work split: one workgroup of 512 threads (8 waves) per (chunk slot, head);
// the shared tiles fit in 80 KB, so two workgroups share a CU and one's
// arithmetic covers the other's memory and barrier waits.
// Thread t holds tokens 2*(t/16), +1 and channels (d_k/16)*(t%16).. of the
// chunk's rows; wave w holds tokens 8w..8w+7 (half of 16-token block w/2).
//   P0 L2-normalise q, k; cumulative sum of g inside each 16-token block (in
//      thread, across the wave's four lane rows, then across the two waves of a
//      block through LDS); a per-channel table of every block-level decay
//      factor (16 x d_k exponentials per chunk);
//   P1 element decay factors; E/F-scaled tiles to LDS; Qhat, Kprime^T, Gamma_C out;
//   P2 the ten lower 16x16 blocks of A and M on MFMA, spread over the waves;
//      A stays in LDS, M goes out;
//   P3 T = (I + A)^-1 in place of A: the four 16x16 diagonal inverses by forward
//      substitution (one lane per column), then block rows 1..3 by
//      T_RJ = -T_RR sum_K A_RK T_KJ on fp32 MFMA;
//   P4 U = (T Diag(beta)) V and W^T = Khat^T (T Diag(beta))^T on MFMA, each
//      written straight from the accumulators in the layout the recurrence reads.
#include <algorithm>
#include <cstddef>
#include <type_traits>

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

// One 16-token block's rows for the exact diagonal products: normalised q and
// k (in the I/O type, as the MFMA reads them) and the in-block cumulative
// log2-decay (fp32).
template <typename T, int D>
struct ExactRows {
    static constexpr int P = 16 / sizeof(T);
    T q[16][D + P];
    T k[16][D + P];
    float g[16][D + 4];
};

// Largest per-channel log2-decay of a 16-token block that the factored
// diagonal products take (1/D_R <= 2^64); larger ones take the exact path.
constexpr float kFactoredMaxLog2Decay = 64.f;
// Floor of a token's log2-decay (retention >= 2^-128).
constexpr float kMinLog2Decay = -128.f;

template <typename T, int D>
struct PrepSmem {
    static constexpr int P = 16 / sizeof(T);  // 16-byte row padding
    float A[64][68];  // beta-scaled strictly-lower A, then T = (I + A)^-1 in place
    union {
        float wsum[8][D];  // P0: per-wave sums of g
        struct {
            T KE[64][D + P];
            T QE[64][D + P];
            T KF[64][D + P];
        } a;
        struct {
            T BK[D][64 + P];  // Khat^T
            T BV[D][64 + P];  // V^T
            T Tb[64][64 + P];  // T Diag(beta)
            float X[4][16][17];
        } b;
        struct {
            float wsum[8][D];     // the same words as wsum above
            union {
                float G[64][D + 4];  // front end: the low-rank gate's pre-activations
                struct {
                    T A[64][64 + P];  // 64 ranks of the chunk's gate rows a
                    T B[D][64 + P];   // the same ranks of the head's b
                } st;
            };
        } fe;
    } u;
    int exact[4];     // block R's diagonal products take the exact path
    float tau[4][D];  // per-block total log-decay
    // per-channel decay factors, rows: 0-3 e^(-tau_R); 4 e^(tau_1); 5 e^(tau_1+tau_2);
    // 6 e^(tau_2); 7-10 e^(rho_{R-1}) (chunk start -> block R start); 11-14
    // e^(rho_3 - rho_R) (block R end -> chunk end); 15 e^(rho_3) = Gamma_C
    float fac[16][D];
    float beta[64];
    // Between P0 and P1 on the exact path, A and u (adjacent, both unused then)
    // hold the chunk's rows as four 16-token blocks.
    __device__ ExactRows<T, D>* stage() { return reinterpret_cast<ExactRows<T, D>*>(&A[0][0]); }
};

// Block (R, J), J <= R, of A (beta-scaled, strictly lower; to LDS) and of M
// (inclusive lower; to the record).  Both products share the K-side operand,
// the F-scaled rows of block J, scaled per channel by 1/D_R on the diagonal and
// by e^(rho_{R-1} - rho_J) when J < R - 1.  M is formed transposed, so each lane
// ends with four consecutive columns of one row and writes them in A order.
template <typename T, int D>
__device__ __forceinline__ void decay_block(PrepSmem<T, D>& sm, T* Mg, int R, int J, int lane) {
    constexpr int NKS = D / 32;
    const int frow = (J == R) ? R : (J < R - 1 ? (R == 2 ? 4 : 5 + J) : -1);
    f32x4 acc_a = {0.f, 0.f, 0.f, 0.f}, acc_m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 32 * ks + 8 * (lane >> 4);
        const Frag<T> ke = load_frag<T>(&sm.u.a.KE[16 * R + (lane & 15)][c0]);
        const Frag<T> qe = load_frag<T>(&sm.u.a.QE[16 * R + (lane & 15)][c0]);
        Frag<T> b = load_frag<T>(&sm.u.a.KF[16 * J + (lane & 15)][c0]);
        if (frow >= 0) {
            const f32x4 f0 = *reinterpret_cast<const f32x4*>(&sm.fac[frow][c0]);
            const f32x4 f1 = *reinterpret_cast<const f32x4*>(&sm.fac[frow][c0 + 4]);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                b.v[j] = from_f32<T>(to_f32(b.v[j]) * (j < 4 ? f0[j] : f1[j - 4]));
        }
        mma(acc_a, ke, b);  // A[r][j]: r in block R (rows), j in block J (columns)
        mma(acc_m, b, qe);  // M^T[j][r]
    }
    const int col = lane & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int row = 4 * (lane >> 4) + e;
        float va = acc_a[e] * sm.beta[16 * R + row];
        if (J == R && col >= row) va = 0.f;
        sm.A[16 * R + row][16 * J + col] = va;
    }
    float m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * (lane >> 4) + i;
        m[i] = (J == R && j > col) ? 0.f : acc_m[i];
    }
    store_n<T, 4>(Mg + aorder_index(16 * R + col, 16 * J + 4 * (lane >> 4), 64), m);
}

// Waves per SIMD the preparation kernels are built for: two workgroups of 8
// waves per CU (at most 128 VGPRs, 80 KB of LDS each), except fp32 I/O at
// d = 128, whose fp32 tiles take 129 KB of LDS: one workgroup per CU, which
// may then use 256 VGPRs.
template <typename T, int D>
constexpr int kPrepWavesPerSimd = (sizeof(T) == 4 && D == 128) ? 2 : 4;

// Front end of the preparation (kernel argument): the short convolution of the
// raw q, k, v and the low-rank decay gate.
struct PrepFE {
    int conv_w, silu, rank, scalar_g;
    const void* weight;    // [3, H, W, D]
    const void* state_in;  // [N, 3, W-1, H, D] or null (zeros)
    const void* a;         // [T, r]
    const void* b;         // [H, D, r]
    const float* bias;     // [H, D] or null
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
    PrepFE fe;
    int64_t slot_begin;  // first chunk slot of this launch (grid row y: slot slot_begin + y)
};

// (first token, length) of a chunk slot; length 0 marks an unused slot.
__device__ __forceinline__ int2 slot_desc(const PrepParams& p, int64_t slot) {
    if (p.cu) return reinterpret_cast<const int2*>(p.ws + p.L.desc_offset())[slot];
    // equal lengths: T < 2^31, so every quantity here fits 32 bits
    const uint32_t N = (uint32_t)p.n_seqs;
    const uint32_t each = (uint32_t)(p.total_tokens / N);
    const uint32_t per = (each + 63) / 64;
    const uint32_t s = (uint32_t)slot;
    if (per == 0 || s >= per * N) return make_int2(0, 0);
    const uint32_t n = s / per, kc = s - n * per;
    return make_int2((int)(n * each + 64 * kc), (int)min(64u, each - 64 * kc));
}

// Exclusive prefix over the four 16-lane rows of a wave of x (lanes in the same
// column of different rows), and the wave total, with cross-row lane swaps.
__device__ __forceinline__ void wave_rows_scan(float x, int row, float& excl, float& total) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s1 = x + ((row & 1) ? __uint_as_float(a[0]) : 0.f);  // rows (0,1), (2,3) inclusive
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(s1), __float_as_uint(s1), false, false);
    const float pt = (row & 1) ? s1 : __uint_as_float(b[1]);          // pair total
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(pt), __float_as_uint(pt), false, false);
    const float incl = s1 + (row >= 2 ? __uint_as_float(c[0]) : 0.f);
    total = pt + (row >= 2 ? __uint_as_float(c[0]) : __uint_as_float(c[1]));
    excl = incl - x;
}

// Exchange of one 32-bit word with the lane 16 (row) or 32 (half) away: the
// swap instructions hand the even row's (lower half's) value to the odd row
// (upper half) in the first result and the other way round in the second.
__device__ __forceinline__ uint32_t xchg_row(uint32_t x, bool odd_row) {
    const auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return odd_row ? s[0] : s[1];
}
__device__ __forceinline__ uint32_t xchg_half(uint32_t x, bool upper) {
    const auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return upper ? s[0] : s[1];
}

// Kprime^T store.  The four lane rows of a wave hold token pairs 0..3 of the
// wave's token octet for the same CPT channels; a 4 x 4 transpose of
// (channel-group) units across the rows, in two swap stages, leaves lane row
// r with all 8 tokens of its channels, so each lane writes whole 16-byte
// fragment runs (instead of CPT scattered 4-byte pieces).
template <typename T, int CPT>
__device__ __forceinline__ void store_kt(T* Ktg, const float (&kp)[CPT][2], int cg, int w,
                                         int lrow) {
    constexpr int WPC = sizeof(T) / 2;   // 32-bit words per channel's token pair
    constexpr int NW = CPT * WPC, US = NW / 4, CHU = US / WPC;
    typedef T V2 __attribute__((ext_vector_type(2)));
    uint32_t wd[NW];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        if constexpr (WPC == 1) {
            wd[c] = __builtin_bit_cast(uint32_t, V2{from_f32<T>(kp[c][0]), from_f32<T>(kp[c][1])});
        } else {
            wd[2 * c] = __float_as_uint(kp[c][0]);
            wd[2 * c + 1] = __float_as_uint(kp[c][1]);
        }
    }
    const bool odd = lrow & 1, up = lrow >= 2;
    // stage 1: keep the units k with k % 2 == row % 2, trade the others with row ^ 1
    uint32_t lo[2][US], hi[2][US];  // rows (row & ~1) and (row | 1)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < US; ++u) {
            const uint32_t keep = odd ? wd[(2 * j + 1) * US + u] : wd[2 * j * US + u];
            const uint32_t got = xchg_row(odd ? wd[2 * j * US + u] : wd[(2 * j + 1) * US + u], odd);
            lo[j][u] = odd ? got : keep;
            hi[j][u] = odd ? keep : got;
        }
    // stage 2: keep the units k == row, trade k == row ^ 2 with row ^ 2
    uint32_t fin[4][US];  // by source row 0..3
#pragma unroll
    for (int u = 0; u < US; ++u) {
        const uint32_t klo = up ? lo[1][u] : lo[0][u], khi = up ? hi[1][u] : hi[0][u];
        const uint32_t glo = xchg_half(up ? lo[0][u] : lo[1][u], up);
        const uint32_t ghi = xchg_half(up ? hi[0][u] : hi[1][u], up);
        fin[0][u] = up ? glo : klo;
        fin[1][u] = up ? ghi : khi;
        fin[2][u] = up ? klo : glo;
        fin[3][u] = up ? khi : ghi;
    }
    // lane row r now holds unit r: channels CPT cg + CHU r .. of tokens 8w .. 8w+7
#pragma unroll
    for (int ch = 0; ch < CHU; ++ch) {
        uint32_t x[4 * WPC];
#pragma unroll
        for (int row = 0; row < 4; ++row)
#pragma unroll
            for (int v = 0; v < WPC; ++v) x[row * WPC + v] = fin[row][ch * WPC + v];
        u32x4* dst = reinterpret_cast<u32x4*>(Ktg + aorder_index(CPT * cg + CHU * lrow + ch, 8 * w, 64));
#pragma unroll
        for (int q = 0; q < WPC; ++q) dst[q] = u32x4{x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
    }
}

// One thread's share of a chunk's raw rows: tokens 2rg, 2rg+1, channels
// (d_k/16) cg.. of q, k, g, v, and beta, in the I/O type.  Rows past the chunk's
// length read as zeros (buffer range check), so the loads are never predicated.
// SG: the gate is one value per token and head (g [T, H]) instead of one per
// key channel; it is then used as a per-channel gate with equal channels.
template <typename T, int D, bool SG>
struct RawRows {
    static constexpr int CPT = D / 16;
    typedef T V __attribute__((ext_vector_type(CPT)));
    V q[2], k[2], g[2], v[2];
    T b[2], gs[2];
    __device__ __forceinline__ void load(const PrepParams& p, int2 d, int h, int rg, int cg) {
        const int64_t H = p.n_heads;
        const uint32_t E = sizeof(T);
        const uint32_t rstride = (uint32_t)(H * D) * E;  // bytes between tokens
        const uint32_t span = (uint32_t)(d.y - 1) * rstride + D * E;
        const int64_t first = ((int64_t)d.x * H + h) * D;
        const auto rq = make_rsrc((const T*)p.q + first, span);
        const auto rk = make_rsrc((const T*)p.k + first, span);
        const auto rgg = SG ? make_rsrc((const T*)p.g + (int64_t)d.x * H + h,
                                        (uint32_t)((d.y - 1) * H + 1) * E)
                            : make_rsrc((const T*)p.g + first, span);
        const auto rv = make_rsrc((const T*)p.v + first, span);
        const auto rb = make_rsrc((const T*)p.beta + (int64_t)d.x * H + h,
                                  (uint32_t)((d.y - 1) * H + 1) * E);
        // v is issued last: it is first used after the other rows, so waiting
        // for them does not wait for it
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t r = 2 * rg + i;
            const uint32_t off = r * rstride + CPT * cg * E;
            q[i] = buffer_load<V>(rq, off);
            k[i] = buffer_load<V>(rk, off);
            if constexpr (SG)
                gs[i] = buffer_load<T>(rgg, r * (uint32_t)H * E);
            else
                g[i] = buffer_load<V>(rgg, off);
            b[i] = buffer_load<T>(rb, r * (uint32_t)H * E);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the v loads behind the others
#pragma unroll
        for (int i = 0; i < 2; ++i)
            v[i] = buffer_load<V>(rv, (2 * rg + i) * rstride + CPT * cg * E);
    }
};

// One thread's share of a chunk's rows as the preparation consumes them:
// tokens 2rg, 2rg+1, channels (d_k/16) cg.. of q, k, g (fp32, g in natural
// units), v (in the I/O type) and beta.
template <typename T, int D>
struct ItemRows {
    static constexpr int CPT = D / 16;
    typedef T V __attribute__((ext_vector_type(CPT)));
    float q[2][CPT], k[2][CPT], g[2][CPT], b[2];
    V v[2];
};

template <typename T, int D, bool SG>
__device__ __forceinline__ void rows_from_raw(const RawRows<T, D, SG>& raw, ItemRows<T, D>& r) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            r.q[i][c] = to_f32(raw.q[i][c]);
            r.k[i][c] = to_f32(raw.k[i][c]);
            r.g[i][c] = to_f32(SG ? raw.gs[i] : raw.g[i][c]);
        }
        r.b[i] = to_f32(raw.b[i]);
        r.v[i] = raw.v[i];
    }
}

// Diagonal block (R, R) of A and M computed exactly (see the decay factoring
// above) from the block's rows xr, by one wave.  Lane l holds token
// t = l % 16 in both operand positions (A-operand rows and B-operand columns
// are both lane % 16) and channel octet l / 16 of each 32-deep step.  At level
// L (half size h = 16 >> L) a token in the right half of its 2h-group is a row
// scaled by e^(gamma_t - gamma_b) and a token in the left half a column scaled
// by e^(gamma_b - gamma_t); the level's product is kept only for its own pairs.
// Level 0 is the diagonal r = j of M (factor 1).  M goes to the record; the
// beta-scaled A values are returned (row 4 (l / 16) + e, column l % 16).
template <typename T, int D>
__device__ __forceinline__ void exact_diag_block(const ExactRows<T, D>& xr, const float* beta,
                                                 T* Mg, int R, int lane, float (&a_out)[4]) {
    constexpr int NKS = D / 32;
    const int tk = lane & 15, oc = lane >> 4;
    // every pair belongs to exactly one level, so each level's masked product
    // is selected into the result rather than added
    f32x4 ta = {0.f, 0.f, 0.f, 0.f}, tm = {0.f, 0.f, 0.f, 0.f};
    // (loops kept rolled: this path runs while the caller's rows are live)
#pragma unroll 1
    for (int L = 0; L <= 4; ++L) {
        const int h = L == 0 ? 0 : (16 >> L);
        const int within = L == 0 ? 0 : (tk & (2 * h - 1));
        const bool right = L > 0 && within >= h;
        const int b = L == 0 ? tk : tk - within + h - 1;  // reference token
        f32x4 aa = {0.f, 0.f, 0.f, 0.f}, am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int ks = 0; ks < NKS; ++ks) {
            const int c0 = 32 * ks + 8 * oc;
            // per-channel factor of this token at this level (1 at level 0)
            float f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float gt = xr.g[tk][c0 + j], gb = xr.g[b][c0 + j];
                // gamma decreases along the block, so the exponent is <= 0 (the
                // clamp absorbs rounding in the cumulative sums)
                f[j] = exp2_hw(fminf(right ? gt - gb : gb - gt, 0.f));
            }
            float x[8];
            load8_f32<T>(&xr.k[tk][c0], x);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] *= f[j];
            const Frag<T> fk = make_frag<T>(x);  // k scaled by this token's factor
            const Frag<T> zero = make_frag<T>({0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f});
            load8_f32<T>(&xr.q[tk][c0], x);
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] *= f[j];
            const Frag<T> fq = make_frag<T>(x);
            // rows r carry the right-half tokens, columns j the left-half ones
            // (level 0: every token in both places, for M's diagonal)
            const bool as_row = L == 0 || right, as_col = L == 0 || !right;
            if (L > 0) mma(aa, as_row ? fk : zero, as_col ? fk : zero);  // A[r][j]
            mma(am, as_col ? fk : zero, as_row ? fq : zero);              // M^T[j][r]
        }
        // keep the level's own pairs: accumulator element e is (4 oc + e, tk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int hi = 4 * oc + e;  // row of the accumulator tile
            // A: (r, j) = (hi, tk); M^T: (j, r) = (hi, tk)
            bool inA, inM;
            if (L == 0) {
                inA = false;
                inM = hi == tk;
            } else {
                const int m2 = 2 * h - 1, sh = 5 - L;
                inA = (hi >> sh) == (tk >> sh) && (hi & m2) >= h && (tk & m2) < h;
                inM = (hi >> sh) == (tk >> sh) && (tk & m2) >= h && (hi & m2) < h;
            }
            ta[e] = inA ? aa[e] : ta[e];
            tm[e] = inM ? am[e] : tm[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * oc + e;
        a_out[e] = ta[e] * beta[16 * R + r];
    }
    const float m[4] = {tm[0], tm[1], tm[2], tm[3]};
    store_n<T, 4>(Mg + aorder_index(16 * R + tk, 16 * R + 4 * oc, 64), m);
}

// Everything for one (chunk slot, head) item whose rows are in `rows`.
template <typename T, int D>
__device__ __forceinline__ void prep_item(const PrepParams& p, PrepSmem<T, D>& sm, int64_t slot,
                                          int h, const ItemRows<T, D>& rows) {
    constexpr int CPT = D / 16;  // channels per thread in the row layout
    typedef T V2 __attribute__((ext_vector_type(2)));
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int rg = t >> 4, cg = t & 15, lrow = lane >> 4;
    const int Rb = w >> 1;  // 16-token block of this thread's rows
    unsigned char* rec = p.ws + p.L.records_offset() + ((size_t)h * p.L.slots + slot) * p.L.rec_bytes;

    // g is taken in base-2 units (g log2 e) from here on, floored at kMinLog2Decay
    float qf[2][CPT], kf[2][CPT], gf[2][CPT], bt[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            qf[i][c] = rows.q[i][c];
            kf[i][c] = rows.k[i][c];
            gf[i][c] = fmaxf(rows.g[i][c] * 1.4426950408889634f, kMinLog2Decay);
        }
        bt[i] = rows.b[i];
    }

    // ---------------------------------------------------------------- P0
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (cg == 0) sm.beta[2 * rg + i] = bt[i];
    if (t < 4) sm.exact[t] = 0;
    // L2 norms over the 16 lanes that share a row
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            sq += qf[i][c] * qf[i][c];
            sk += kf[i][c] * kf[i][c];
        }
        sq = row16_sum(sq);
        sk = row16_sum(sk);
        const float rq = (p.l2norm ? __builtin_amdgcn_rsqf(sq + kL2Eps) : 1.0f) * p.scale;
        const float rk = p.l2norm ? __builtin_amdgcn_rsqf(sk + kL2Eps) : 1.0f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            qf[i][c] *= rq;
            kf[i][c] *= rk;
        }
    }
    // cumulative log-decay inside the 16-token block: in-thread over the two
    // rows, across the wave's four lane rows, then across the block's two waves
    float excl[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        gf[1][c] += gf[0][c];
        float total;
        wave_rows_scan(gf[1][c], lrow, excl[c], total);
        if (lrow == 0) sm.u.wsum[w][CPT * cg + c] = total;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const float add = excl[c] + ((w & 1) ? sm.u.wsum[w - 1][CPT * cg + c] : 0.f);
        gf[0][c] += add;
        gf[1][c] += add;
    }
    // per-channel table of the block-level decay factors (16 x D exponentials):
    // thread t owns channel t % D and rows t / D + (512 / D) * i, one row per wave
    // and step, so each exponent is a signed sum of a run of block totals with
    // coefficients known to the whole wave
    {
        constexpr int RSTEP = 512 / D;
        const int c = t % D;
        const int rbase = __builtin_amdgcn_readfirstlane(t / D);
        float tb[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) tb[R] = sm.u.wsum[2 * R][c] + sm.u.wsum[2 * R + 1][c];
        if (rbase == 0) {
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                sm.tau[R][c] = tb[R];
                if (-tb[R] > kFactoredMaxLog2Decay) sm.exact[R] = 1;
            }
        }
#pragma unroll
        for (int i = 0; i < 16 / RSTEP; ++i) {
            const int row = rbase + RSTEP * i;
            int lo, hi;  // the run of blocks summed; empty when lo > hi
            if (row < 4) { lo = row; hi = row; }                  // e^(-tau_R)
            else if (row < 7) { lo = row == 6 ? 2 : 1; hi = row == 4 ? 1 : 2; }
            else if (row < 11) { lo = 0; hi = row - 8; }          // e^(rho_{R-1})
            else if (row < 15) { lo = row - 10; hi = 3; }         // e^(rho_3 - rho_R)
            else { lo = 0; hi = 3; }                              // Gamma_C
            const float sg = row < 4 ? -1.f : 1.f;
            float arg = 0.f;
#pragma unroll
            for (int R = 0; R < 4; ++R) arg += (lo <= R && R <= hi ? sg : 0.f) * tb[R];
            // (rows 0-3 serve only the factored diagonal blocks, whose decay is
            // at most kFactoredMaxLog2Decay; the clamp keeps the others finite)
            sm.fac[row][c] = exp2_hw(row < 4 ? fminf(arg, kFactoredMaxLog2Decay) : arg);
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P0x
    // diagonal blocks past the factored range: every thread parks its rows in
    // the staging area (so they are not live meanwhile), wave R computes block
    // R exactly, and the rows are read back.  q and k come back rounded to the
    // I/O type, as every MFMA operand made from them is.
    // (read as wave-uniform values, so the branches below are scalar)
    const int xmask = __builtin_amdgcn_readfirstlane(
        (sm.exact[0] ? 1 : 0) | (sm.exact[1] ? 2 : 0) | (sm.exact[2] ? 4 : 0) | (sm.exact[3] ? 8 : 0));
    const int wu = __builtin_amdgcn_readfirstlane(w);
    if (xmask) {
        typedef PrepSmem<T, D> Smem;
        static_assert(offsetof(Smem, u) == sizeof(float) * 64 * 68 &&
                          4 * sizeof(ExactRows<T, D>) <= sizeof(float) * 64 * 68 + sizeof(sm.u),
                      "the staging area must fit A and u");
        ExactRows<T, D>& xr = sm.stage()[Rb];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 2 * rg + i - 16 * Rb;
            store_n<T, CPT>(&xr.q[r][CPT * cg], qf[i]);
            store_n<T, CPT>(&xr.k[r][CPT * cg], kf[i]);
            *reinterpret_cast<f32x4*>(&xr.g[r][CPT * cg]) = f32x4{gf[i][0], gf[i][1], gf[i][2], gf[i][3]};
            if constexpr (CPT == 8)
                *reinterpret_cast<f32x4*>(&xr.g[r][CPT * cg + 4]) =
                    f32x4{gf[i][4], gf[i][5], gf[i][6], gf[i][7]};
        }
        __syncthreads();
        float xa[4] = {0.f, 0.f, 0.f, 0.f};
        if (wu < 4 && ((xmask >> wu) & 1))
            exact_diag_block<T, D>(sm.stage()[wu], sm.beta, reinterpret_cast<T*>(rec + p.L.off_m),
                                   wu, lane, xa);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 2 * rg + i - 16 * Rb;
            load_n<T, CPT>(&xr.q[r][CPT * cg], qf[i]);
            load_n<T, CPT>(&xr.k[r][CPT * cg], kf[i]);
#pragma unroll
            for (int c = 0; c < CPT; ++c) gf[i][c] = xr.g[r][CPT * cg + c];
        }
        __syncthreads();
        if (wu < 4 && ((xmask >> wu) & 1)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.A[16 * wu + 4 * (lane >> 4) + e][16 * wu + (lane & 15)] = xa[e];
        }
    }

    // ---------------------------------------------------------------- P1
    T* Qg = reinterpret_cast<T*>(rec + p.L.off_q);
    T* Ktg = reinterpret_cast<T*>(rec + p.L.off_kt);
    // Khat and V of the two rows, per channel, as packed words (the rotation
    // below moves whole words)
    typedef typename std::conditional<sizeof(T) == 2, uint32_t, uint64_t>::type W2;
    W2 rk[CPT], rv[CPT];
    float kpT[CPT][2];
    float tauR[CPT], Gs[CPT], Kp[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        tauR[c] = sm.tau[Rb][CPT * cg + c];
        Gs[c] = sm.fac[7 + Rb][CPT * cg + c];
        Kp[c] = sm.fac[11 + Rb][CPT * cg + c];
    }
    V2 kh[CPT];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 2 * rg + i;
        float ke[CPT], qe[CPT], kfv[CPT], qh[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float E = exp2_hw(gf[i][c]);
            const float F = exp2_hw(tauR[c] - gf[i][c]);
            ke[c] = kf[i][c] * E;
            qe[c] = qf[i][c] * E;
            kfv[c] = kf[i][c] * F;
            qh[c] = qe[c] * Gs[c];
            kh[c][i] = from_f32<T>(ke[c] * Gs[c]);
            kpT[c][i] = kfv[c] * Kp[c];
        }
        store_n<T, CPT>(&sm.u.a.KE[r][CPT * cg], ke);
        store_n<T, CPT>(&sm.u.a.QE[r][CPT * cg], qe);
        store_n<T, CPT>(&sm.u.a.KF[r][CPT * cg], kfv);
        store_n<T, CPT>(Qg + aorder_index(r, CPT * cg, D), qh);
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) rk[c] = __builtin_bit_cast(W2, kh[c]);
    store_kt<T, CPT>(Ktg, kpT, cg, w, lrow);
    if (rg == 0) {
        float* gC = reinterpret_cast<float*>(rec + p.L.off_gc);
#pragma unroll
        for (int c = 0; c < CPT; ++c) gC[CPT * cg + c] = sm.fac[15][CPT * cg + c];
    }
    __syncthreads();

    // ---------------------------------------------------------------- P2
    {
        T* Mg = reinterpret_cast<T*>(rec + p.L.off_m);
        // waves 0-6: blocks (0,0) (1,1) (2,2) (3,3) (2,0) (3,0) (3,1), which all
        // scale their K-side operand; wave 7: (1,0) (2,1) (3,2), which do not.
        // Waves 0 and 5 also write the zero blocks (0,1) and (2,3) of M, which
        // share 16 x 32 fragment tiles with nonzero blocks; the tiles of blocks
        // (0..1, 2..3) are all zero and are never read, so never written.
        if (w < 7) {
            const int R = (0x3323210 >> (4 * w)) & 15;
            const int J = (0x1003210 >> (4 * w)) & 15;
            // (diagonal blocks on the exact path were written in P0x)
            if (wu >= 4 || !((xmask >> wu) & 1)) decay_block<T, D>(sm, Mg, R, J, lane);
            if (w == 0 || w == 5) {
                const int zR = w == 0 ? 0 : 2, zJ = w == 0 ? 1 : 3;
                const float z[4] = {0.f, 0.f, 0.f, 0.f};
                store_n<T, 4>(Mg + aorder_index(16 * zR + (lane & 15), 16 * zJ + 4 * (lane >> 4), 64), z);
            }
        } else {
            for (int R = 1; R < 4; ++R) decay_block<T, D>(sm, Mg, R, R - 1, lane);
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P3
    // transposed Khat and V tiles (the operands of W^T and U).  Lane (rg, cg)
    // holds 2 tokens x CPT channels and stores each channel's token pair at
    // token octet (rg / 4) ^ (cg % 8): an XOR swizzle by channel group, undone
    // by the readers, that spreads the 16 lanes of a token group over the banks
    // (without it they all land on one bank).  V is first used here, so its
    // loads have had P0-P2 to arrive.
    {
        const int col = 8 * ((rg >> 2) ^ (cg & 7)) + 2 * (rg & 3);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            rv[c] = __builtin_bit_cast(W2, V2{rows.v[0][c], rows.v[1][c]});
            *reinterpret_cast<W2*>(&sm.u.b.BK[CPT * cg + c][col]) = rk[c];
            *reinterpret_cast<W2*>(&sm.u.b.BV[CPT * cg + c][col]) = rv[c];
        }
    }
    if (w == 0) {
        // diagonal 16x16 blocks of (I + A)^-1, in place: lane = (block, column),
        // forward substitution; every row of A_RR is read (16-byte loads) before
        // the wave writes any column of T_RR
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
        for (int i = 0; i < 16; ++i) sm.A[16 * R + i][16 * R + j] = colv[i];
    }
    __syncthreads();
    // block rows 1..3: wave J forms T_RJ = -T_RR sum_{K=J}^{R-1} A_RK T_KJ; the
    // sums are taken before any T_RJ replaces A_RJ
    for (int R = 1; R < 4; ++R) {
        if (w < R) {
            const int J = w;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < R; ++K)
                mm16_lds(x, &sm.A[16 * R][16 * K], 68, &sm.A[16 * K][16 * J], 68);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.u.b.X[w][4 * (lane >> 4) + e][lane & 15] = -x[e];
        }
        __syncthreads();
        if (w < R) {
            const int J = w;
            f32x4 tt = {0.f, 0.f, 0.f, 0.f};
            mm16_lds(tt, &sm.A[16 * R][16 * R], 68, &sm.u.b.X[w][0][0], 17);
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.A[16 * R + 4 * (lane >> 4) + e][16 * J + (lane & 15)] = tt[e];
        }
        __syncthreads();
    }
    {
        // thread t converts row t / 8, columns 8 * (t % 8) .. +7 of T Diag(beta)
        // (zero above the diagonal)
        const int r = t >> 3, c0 = 8 * (t & 7);
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (c0 + j <= r) ? sm.A[r][c0 + j] * sm.beta[c0 + j] : 0.f;
        store_frag<T>(&sm.u.b.Tb[r][c0], make_frag<T>(x));
    }
    __syncthreads();

    // ---------------------------------------------------------------- P4
    {
        const int R = w & 3;
        const int nks = (R >= 2) ? 2 : 1;  // T[r][j] = 0 for j in blocks past R
        Frag<T> ta[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks < nks) ta[ks] = load_frag<T>(&sm.u.b.Tb[16 * R + (lane & 15)][32 * ks + 8 * (lane >> 4)]);
        T* Ug = reinterpret_cast<T*>(rec + p.L.off_u);
        T* Wg = reinterpret_cast<T*>(rec + p.L.off_w);
        constexpr int NBW = D / 32;  // column tiles per wave
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            const int nb = (w >> 2) * NBW + i;
            f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks < nks) {
                    // token octet 4 ks + lane / 16 of channel row n, swizzled as stored
                    const int n = 16 * nb + (lane & 15);
                    const int c0 = 8 * ((4 * ks + (lane >> 4)) ^ ((n / CPT) & 7));
                    const Frag<T> bk = load_frag<T>(&sm.u.b.BK[n][c0]);
                    const Frag<T> bv = load_frag<T>(&sm.u.b.BV[n][c0]);
                    mma(aw, bk, ta[ks]);  // W^T[n][r]
                    mma(au, ta[ks], bv);  // U[r][n]
                }
            }
            const float uv[4] = {au[0], au[1], au[2], au[3]};
            store_n<T, 4>(Ug + corder_index(16 * R + 4 * (lane >> 4), 16 * nb + (lane & 15), D), uv);
            const float wv[4] = {aw[0], aw[1], aw[2], aw[3]};
            store_n<T, 4>(Wg + aorder_index(16 * R + (lane & 15), 16 * nb + 4 * (lane >> 4), D), wv);
        }
    }
}

// ------------------------------------------------------------------ front end
// One thread's raw rows for the front end: tokens 2rg-3 .. 2rg+1 of the chunk
// (the three before its own two feed the convolution) of q, k, v, and its two
// rows of g (when given) and beta.  Rows outside [sequence start, chunk end)
// read as zeros; for a sequence's first chunk the rows before it come from the
// conv state.
template <typename T, int D>
struct FeRaw {
    static constexpr int CPT = D / 16;
    typedef T V __attribute__((ext_vector_type(CPT)));
    V x[3][5];
    V g[2];
    T gs[2], b[2];
    __device__ __forceinline__ void load(const PrepParams& p, int2 d, int64_t n, int64_t s_begin,
                                         int h, int rg, int cg) {
        const int64_t H = p.n_heads;
        const uint32_t E = sizeof(T);
        const uint32_t rstride = (uint32_t)(H * D) * E;
        const uint32_t col = CPT * cg * E;
        const int64_t tb = max((int64_t)d.x - 3, s_begin);  // first token in range
        const uint32_t span = (uint32_t)((d.x + d.y - 1 - tb) * rstride) + D * E;
        const int64_t first = (tb * H + h) * D;
        const T* src[3] = {(const T*)p.q, (const T*)p.k, (const T*)p.v};
#pragma unroll
        for (int xi = 0; xi < 3; ++xi) {
            const auto r = make_rsrc(src[xi] + first, span);
#pragma unroll
            for (int m = 0; m < 5; ++m) {
                // rows before tb take an offset far past the range (read as zero)
                const int64_t rel = (int64_t)d.x + 2 * rg - 3 + m - tb;
                const uint32_t off = rel < 0 ? kFarOffset : (uint32_t)rel * rstride + col;
                x[xi][m] = buffer_load<V>(r, off);
            }
        }
        const uint32_t cspan = (uint32_t)(d.y - 1) * rstride + D * E;
        const int64_t cfirst = ((int64_t)d.x * H + h) * D;
        const auto rb = make_rsrc((const T*)p.beta + (int64_t)d.x * H + h,
                                  (uint32_t)((d.y - 1) * H + 1) * E);
#pragma unroll
        for (int i = 0; i < 2; ++i) b[i] = buffer_load<T>(rb, (2 * rg + i) * (uint32_t)H * E);
        if (p.fe.rank == 0) {
            if (p.fe.scalar_g) {
                const auto rg1 = make_rsrc((const T*)p.g + (int64_t)d.x * H + h,
                                           (uint32_t)((d.y - 1) * H + 1) * E);
#pragma unroll
                for (int i = 0; i < 2; ++i) gs[i] = buffer_load<T>(rg1, (2 * rg + i) * (uint32_t)H * E);
            } else {
                const auto rgc = make_rsrc((const T*)p.g + cfirst, cspan);
#pragma unroll
                for (int i = 0; i < 2; ++i) g[i] = buffer_load<V>(rgc, (2 * rg + i) * rstride + col);
            }
        }
        const int W = p.fe.conv_w;
        if (W > 1 && p.fe.state_in && d.x == s_begin) {
            // first chunk: token 2rg-3+m < 0 is row (W-1) + (2rg-3+m) of the state
            const uint32_t sspan = (uint32_t)((W - 2) * H * D + D) * E;
#pragma unroll
            for (int xi = 0; xi < 3; ++xi) {
                const auto r = make_rsrc((const T*)p.fe.state_in +
                                             ((n * 3 + xi) * (W - 1) * H + h) * D,
                                         sspan);
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    const int o = 2 * rg - 3 + m;
                    const int j = (W - 1) + o;
                    const uint32_t off = (o < 0 && j >= 0) ? (uint32_t)j * rstride + col : kFarOffset;
                    const V sv = buffer_load<V>(r, off);
                    if (o < 0) x[xi][m] = sv;
                }
            }
        }
    }
};

// The front end's rows: the convolution (and SiLU) of q, k, v, and g given or
// from the low-rank projection.  Rows past the chunk's length are zero, as
// without a front end.
template <typename T, int D, int KS>
__device__ __forceinline__ void fe_rows(const PrepParams& p, PrepSmem<T, D>& sm, int2 d, int h,
                                        const FeRaw<T, D>& raw, ItemRows<T, D>& r) {
    constexpr int CPT = D / 16;
    typedef T V __attribute__((ext_vector_type(CPT)));
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int rg = t >> 4, cg = t & 15;
    const int64_t H = p.n_heads;
    const int W = p.fe.conv_w;
    const bool live[2] = {2 * rg < d.y, 2 * rg + 1 < d.y};

    // ---- short convolution: tap j' of 4 (tap j' - (4 - W) of the filter)
    // multiplies row i + j' for output row i
    float y[3][2][CPT];
#pragma unroll
    for (int xi = 0; xi < 3; ++xi) {
        if (W == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int c = 0; c < CPT; ++c) y[xi][i][c] = to_f32(raw.x[xi][3 + i][c]);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int c = 0; c < CPT; ++c) y[xi][i][c] = 0.f;
            // the W taps of this head's filter; taps 0 .. 3-W of the four read zero
            const auto rw = make_rsrc((const T*)p.fe.weight + ((int64_t)(xi * H + h) * W) * D,
                                      (uint32_t)(W * D * sizeof(T)));
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                const int tap = jp - (4 - W);
                const uint32_t off =
                    tap < 0 ? kFarOffset : (uint32_t)((tap * D + CPT * cg) * sizeof(T));
                const V wv = buffer_load<V>(rw, off);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int c = 0; c < CPT; ++c)
                        y[xi][i][c] += to_f32(wv[c]) * to_f32(raw.x[xi][i + jp][c]);
            }
            if (p.fe.silu) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int c = 0; c < CPT; ++c)
                        y[xi][i][c] *= __builtin_amdgcn_rcpf(1.f + __expf(-y[xi][i][c]));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            r.q[i][c] = live[i] ? y[0][i][c] : 0.f;
            r.k[i][c] = live[i] ? y[1][i][c] : 0.f;
            r.v[i][c] = from_f32<T>(live[i] ? y[2][i][c] : 0.f);
        }
        // rounded and packed here: left to the compiler, the conversion sinks
        // to v's use in P3 and keeps twice the registers alive until then
        // (measured: 0 spills instead of 6 up to rank 64; with the rank > 64
        // gate's longer product the early packing costs more than it saves)
        if constexpr (KS <= 2) asm volatile("" : "+v"(r.v[i]));
        r.b[i] = to_f32(raw.b[i]);
    }

    // ---- decay gate
    if (p.fe.rank == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int c = 0; c < CPT; ++c)
                r.g[i][c] = to_f32(p.fe.scalar_g ? raw.gs[i] : raw.g[i][c]);
        return;
    }
    // G = a b_h^T on MFMA.  The chunk's gate rows a [64 x R] and the head's b
    // [D x R] go through LDS 64 ranks at a time, so each element is loaded once
    // per workgroup (from registers, each token tile would be fetched by two
    // waves and each channel tile by four).  Wave w forms token tile w % 4
    // against channel tiles (D/32) (w / 4) .. +D/32-1; the pre-activations then
    // go to LDS over the staging area, and each thread takes its rows.
    {
        constexpr int NTW = D / 32;
        const int R = p.fe.rank;
        const int tb = w & 3;
        const uint32_t E = sizeof(T);
        // rows of a past the chunk and ranks past R read zero (range-checked);
        // R is a multiple of 32, so an 8-rank octet is wholly in or out
        const auto ra = make_rsrc((const T*)p.fe.a + (int64_t)d.x * R, (uint32_t)(d.y * R) * E);
        const auto rbm = make_rsrc((const T*)p.fe.b + (int64_t)h * D * R, (uint32_t)(D * R) * E);
        f32x4 acc[NTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pc = 0; pc < KS / 2; ++pc) {
            {
                const int row = t >> 3, k = 64 * pc + 8 * (t & 7);
                store_frag<T>(&sm.u.fe.st.A[row][8 * (t & 7)],
                              buffer_load_frag<T>(ra, k < R ? (uint32_t)(row * R + k) * E : kFarOffset));
            }
#pragma unroll
            for (int j = 0; j < D / 64; ++j) {
                const int i = t + 512 * j, row = i >> 3, k = 64 * pc + 8 * (i & 7);
                store_frag<T>(&sm.u.fe.st.B[row][8 * (i & 7)],
                              buffer_load_frag<T>(rbm, k < R ? (uint32_t)(row * R + k) * E : kFarOffset));
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int k0 = 32 * ks + 8 * (lane >> 4);
                const Frag<T> af = load_frag<T>(&sm.u.fe.st.A[16 * tb + (lane & 15)][k0]);
#pragma unroll
                for (int i = 0; i < NTW; ++i) {
                    const int ct = NTW * (w >> 2) + i;
                    mma(acc[i], af, load_frag<T>(&sm.u.fe.st.B[16 * ct + (lane & 15)][k0]));
                }
            }
            __syncthreads();
        }
        // the bias at this thread's channels, all requested at once (range-checked
        // loads with no branch; a missing bias reads zero)
        const auto rbias = make_rsrc(p.fe.bias ? (const void*)(p.fe.bias + (int64_t)h * D)
                                               : (const void*)p.fe.b,
                                     p.fe.bias ? (uint32_t)(D * 4) : 0u);
        float bias[NTW];
#pragma unroll
        for (int i = 0; i < NTW; ++i)
            bias[i] = buffer_load<float>(rbias, (uint32_t)(16 * (NTW * (w >> 2) + i) + (lane & 15)) * 4);
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const int ch = 16 * (NTW * (w >> 2) + i) + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.u.fe.G[16 * tb + 4 * (lane >> 4) + e][ch] = acc[i][e] + bias[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float z = sm.u.fe.G[2 * rg + i][CPT * cg + c];
            // g = -softplus(z) = -(max(z, 0) + log(1 + e^-|z|))
            const float gv = -(fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z))));
            r.g[i][c] = live[i] ? gv : 0.f;
        }
    }
}

// Sequence index and first token of the sequence that holds token `tok`.
__device__ __forceinline__ void seq_of_token(const PrepParams& p, int64_t tok, int64_t& n,
                                             int64_t& s_begin) {
    if (!p.cu) {
        const int64_t each = p.total_tokens / p.n_seqs;
        n = tok / each;
        s_begin = n * each;
        return;
    }
    int lo = 0, hi = p.n_seqs - 1;  // largest n with cu[n] <= tok
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.cu[mid] <= tok) lo = mid; else hi = mid - 1;
    }
    n = lo;
    s_begin = p.cu[lo];
}

// The preparation with the front end: raw q, k, v, and g given or low-rank.
template <typename T, int D, int KS>
__global__ __launch_bounds__(512, (kPrepWavesPerSimd<T, D>)) void prep_fe_kernel(PrepParams p) {
    __shared__ PrepSmem<T, D> sm;
    const int t = threadIdx.x;
    // 2-D grid (head, chunk slot); the linear workgroup order is slot-major,
    // so head h runs on XCD h mod 8 when H is a multiple of 8
    const int h = blockIdx.x;
    const int64_t slot = p.slot_begin + blockIdx.y;
    const int2 d = slot_desc(p, slot);
    if (d.y <= 0) return;
    int64_t n, s_begin;
    seq_of_token(p, d.x, n, s_begin);
    ItemRows<T, D> rows;
    {
        FeRaw<T, D> raw;
        raw.load(p, d, n, s_begin, h, t >> 4, t & 15);
        fe_rows<T, D, KS>(p, sm, d, h, raw, rows);
    }
    prep_item<T, D>(p, sm, slot, h, rows);
}

// Each sequence's final conv state: its last W-1 raw rows of q, k, v (rows
// before the sequence's start continue from the input state, or are zero).
// One workgroup per (sequence, tensor, state row); threads over H*D elements.
template <typename T, int D>
__global__ __launch_bounds__(256) void conv_state_kernel(PrepParams p, void* state_out) {
    const int W = p.fe.conv_w;
    const int64_t blk = blockIdx.x;  // ((n * 3 + x) * (W - 1)) + j
    const int j = (int)(blk % (W - 1));
    const int64_t nx = blk / (W - 1);
    const int x = (int)(nx % 3);
    const int64_t n = nx / 3;
    const int64_t HD = (int64_t)p.n_heads * D;
    int64_t s_begin, len;
    if (p.cu) {
        s_begin = p.cu[n];
        len = (int64_t)p.cu[n + 1] - s_begin;
    } else {
        len = p.total_tokens / p.n_seqs;
        s_begin = n * len;
    }
    const int64_t rel = len - (W - 1) + j;  // token of state row j, from the sequence start
    const T* src = x == 0 ? (const T*)p.q : (x == 1 ? (const T*)p.k : (const T*)p.v);
    const T* st = (const T*)p.fe.state_in;
    T* dst = (T*)state_out + blk * HD;
    for (int64_t e = threadIdx.x; e < HD; e += 256) {
        T val = from_f32<T>(0.f);
        if (rel >= 0)
            val = src[(s_begin + rel) * HD + e];
        else if (st)
            val = st[(nx * (W - 1) + (j + len)) * HD + e];
        dst[e] = val;
    }
}

// One (chunk slot, head) item per workgroup; two workgroups share a CU (80 KB
// of LDS and at most 128 VGPRs each; fp32 at d = 128: one per CU).
template <typename T, int D, bool SG>
__global__ __launch_bounds__(512, (kPrepWavesPerSimd<T, D>)) void prep_kernel(PrepParams p) {
    __shared__ PrepSmem<T, D> sm;
    const int t = threadIdx.x;
    // 2-D grid (head, chunk slot), one workgroup per item
    const int h = blockIdx.x;
    const int64_t slot = p.slot_begin + blockIdx.y;
    const int2 d = slot_desc(p, slot);
    if (d.y <= 0) return;
    RawRows<T, D, SG> raw;
    raw.load(p, d, h, t >> 4, t & 15);
    ItemRows<T, D> rows;
    rows_from_raw<T, D, SG>(raw, rows);
    prep_item<T, D>(p, sm, slot, h, rows);
}

// Chunk index: cf[n] = first chunk slot of sequence n, cf[N] = number of chunks;
// with checkpoints every `interval` chunks also ck[n] = first checkpoint of
// sequence n (floor((chunks - 1) / interval) per non-empty sequence).  One
// workgroup; sequences are processed 256 at a time with running carries.
__global__ __launch_bounds__(256) void chunk_index_kernel(const int32_t* __restrict__ cu,
                                                          int32_t n_seqs, int64_t total_tokens,
                                                          int32_t* __restrict__ cf,
                                                          int32_t* __restrict__ ck,
                                                          int32_t interval) {
    __shared__ int32_t s_scan[2][256];
    const int t = threadIdx.x;
    const int64_t each = n_seqs ? total_tokens / n_seqs : 0;
    int32_t carry = 0, ccarry = 0;
    for (int base = 0; base < n_seqs; base += 256) {
        const int n = base + t;
        int32_t c = 0, kc = 0;
        if (n < n_seqs) {
            const int64_t len = cu ? (int64_t)cu[n + 1] - cu[n] : each;
            c = (int32_t)((len + 63) / 64);
            kc = (interval > 0 && c > 0) ? (c - 1) / interval : 0;
        }
        s_scan[0][t] = c;
        s_scan[1][t] = kc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t x = (t >= off) ? s_scan[0][t - off] : 0;
            const int32_t y = (t >= off) ? s_scan[1][t - off] : 0;
            __syncthreads();
            s_scan[0][t] += x;
            s_scan[1][t] += y;
            __syncthreads();
        }
        if (n < n_seqs) {
            cf[n] = carry + s_scan[0][t] - c;
            ck[n] = ccarry + s_scan[1][t] - kc;
        }
        carry += s_scan[0][255];
        ccarry += s_scan[1][255];
        __syncthreads();
    }
    if (t == 0) {
        cf[n_seqs] = carry;
        ck[n_seqs] = ccarry;
    }
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
    const int64_t s_end = a.slot_end < 0 ? a.layout.slots : a.slot_end;
    p.slot_begin = a.slot_begin;
    int32_t* cf = reinterpret_cast<int32_t*>(a.workspace);
    int32_t* ck = reinterpret_cast<int32_t*>(a.workspace + a.layout.ckidx_offset());
    hipError_t e;
    if (a.prep_setup && a.cu_seqlens) {
        // equal lengths need no index: the recurrence derives it
        hipLaunchKernelGGL((chunk_index_kernel), dim3(1), dim3(256), 0, stream, a.cu_seqlens,
                           a.n_seqs, a.total_tokens, cf, ck, a.ckpt_interval);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.prep_setup && a.fe.active() && a.fe.conv_w > 1 && a.fe.state_out) {
        // final conv states (also for sequences without tokens)
        p.fe = PrepFE{a.fe.conv_w, a.fe.silu, a.fe.rank, a.scalar_g ? 1 : 0, a.fe.conv_weight,
                      a.fe.state_in, a.fe.gate_a, a.fe.gate_b, a.fe.gate_bias};
        const int64_t blocks = (int64_t)a.n_seqs * 3 * (a.fe.conv_w - 1);
        hipLaunchKernelGGL((conv_state_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, p, a.fe.state_out);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (a.total_tokens == 0) return hipSuccess;
    if (a.prep_setup && a.cu_seqlens) {
        const unsigned nb = (unsigned)((a.layout.slots + 255) / 256);
        hipLaunchKernelGGL((chunk_desc_kernel), dim3(nb), dim3(256), 0, stream, a.cu_seqlens,
                           a.n_seqs, cf, a.layout.slots,
                           reinterpret_cast<int2*>(a.workspace + a.layout.desc_offset()));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t nslots = s_end - a.slot_begin;
    if (nslots <= 0) return hipSuccess;
    if (a.fe.active())
        p.fe = PrepFE{a.fe.conv_w, a.fe.silu, a.fe.rank, a.scalar_g ? 1 : 0, a.fe.conv_weight,
                      a.fe.state_in, a.fe.gate_a, a.fe.gate_b, a.fe.gate_bias};
    // grid (head, chunk slot), at most kMaxGridY slots per launch
    for (int64_t s0 = 0; s0 < nslots; s0 += kMaxGridY) {
        p.slot_begin = a.slot_begin + s0;
        const dim3 grid((unsigned)a.n_heads, (unsigned)std::min<int64_t>(kMaxGridY, nslots - s0));
        if (a.fe.active()) {
            // ranks up to 64 take two 32-deep steps of the gate's product, larger ones four
            if (a.fe.rank <= 64)
                hipLaunchKernelGGL((prep_fe_kernel<T, D, 2>), grid, dim3(512), 0, stream, p);
            else
                hipLaunchKernelGGL((prep_fe_kernel<T, D, 4>), grid, dim3(512), 0, stream, p);
        } else if (a.scalar_g) {
            hipLaunchKernelGGL((prep_kernel<T, D, true>), grid, dim3(512), 0, stream, p);
        } else {
            hipLaunchKernelGGL((prep_kernel<T, D, false>), grid, dim3(512), 0, stream, p);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template hipError_t launch_prep<bf16, 128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<bf16, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<float, 64>(const PrefillArgs&, hipStream_t);
template hipError_t launch_prep<float, 128>(const PrefillArgs&, hipStream_t);

}  // namespace kda

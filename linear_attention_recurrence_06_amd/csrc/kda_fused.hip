// Fused KDA prefill on gfx950 for calls with many (sequence, head) chains.
//
// The two-kernel path hands a record per (chunk, head) from the preparation
// kernel to the recurrence kernel through HBM, and the record is larger than
// the chunk's inputs.  With many chains no chain needs more than one workgroup,
// so here persistent workgroups take whole chains (longest sequences first) and
// keep everything but the inputs, the outputs and the states on chip.
//
// Sub-chunk form.  The delta rule with a diagonal gate ("From KV Cache to
// Depth Attention: The Bottlenecks Kimi K3 Had to Break", Technical Details,
// KDA bullet) is unrolled here over blocks of 16 tokens, so the chunk-wise WY
// form that gives the linear-cost chunked prefill ("Kimi K3: The Manos, The
// Mythos, The Legendos", bullet on the two-kernel chunked design) runs with
// the block as its chunk.  In base-2 units (lambda = g log2 e, floored at -128
// per token), with Gamma_t the inclusive cumulative lambda of token t inside
// its block, tau the block total, and qhat, khat the normalised rows:
//     Ke = khat 2^Gamma,  Qe = qhat 2^Gamma,  K' = khat 2^(tau - Gamma)   (all factors <= 1)
//     A[i][j] = beta_i sum_c khat_i khat_j 2^(Gamma_i - Gamma_j)   (j < i)
//     M[i][j] =        sum_c qhat_i khat_j 2^(Gamma_i - Gamma_j)   (j <= i)
//     u = T Diag(beta) (V - Ke S),  T = (I + A)^-1
//     O = Qe S + M u,   S <- Diag(2^tau) S + K'^T u
// A chunk of 64 tokens is four such steps.  Compared with the 64-token form of
// the two-kernel path this drops the blocks of A and M off the 16 x 16
// diagonal, the blocked inverse and the W and U products, and the recurrence
// takes one more small product (T Diag(beta) times V - Ke S) per block.
//
// Diagonal products.  A and M factor as Ke_i . (K'_j 2^-tau) while every
// channel's block decay keeps 2^-tau <= 2^64; past that they are taken exactly
// by bisection levels (halves of 8, 4, 2, 1 tokens; with b the last token of
// the left half, 2^(Gamma_i - Gamma_j) = 2^(Gamma_i - Gamma_b) 2^(Gamma_b -
// Gamma_j), both factors <= 1), one masked product per level.
//
// Inverse.  N = Diag(beta) A is strictly lower and 16 x 16, so N^16 = 0 and
//     T = (I - N)(I + N^2)(I + N^4)(I + N^8),
// eight fp32 16 x 16 products on MFMA inside one wave, no LDS traffic.
//
// Layout.  A preparation wave takes one 16-token block over all its channels,
// lane (t, g) = (lane % 16, lane / 16) holding token t of the block and
// channels 32 ks + 8 g + {0..7} of each 32-channel slice ks (one 16-byte load
// per row and slice), which is the K order of every 16 x 16 x 32 product over
// channels.  The state's key channels are placed in its 16-row tiles to match:
// row 4 g + e of tile 2 ks holds channel 32 ks + 8 g + e, of tile 2 ks + 1
// channel 32 ks + 8 g + 4 + e, so the state rows a lane holds as accumulator
// are, as they stand, its B operand: no state data moves between lanes.  K'^T is transposed into that
// row order by a product with a 0/1 selector operand.  A recurrence wave owns
// 16 (d = 64) or 32 (d = 128) value columns of the fp32 state and needs no
// other wave's state; the block's operands come from the record in LDS.
//
// Kernels.  At d = 64 (fused_kernel) the four waves of a workgroup prepare a
// chunk's four blocks, meet at a barrier, then run its recurrence on 16 value
// columns each.  At d = 128 (fused_ws_kernel) four waves only prepare and four
// only run the recurrence, one chunk behind, on the same SIMDs.
//
// Segmented prefill (launch_segmented).  For few long chains the sequences are
// cut into segments whose (segment, head) chains fill the device.  The
// recurrence is affine in the state, so over a segment S_end = M S_start + b:
// one variant of fused_ws_kernel forms b (from the zero state) and M (from the
// identity, v taken as zero) together, each recurrence wave carrying four
// state tiles and no outputs, segment_scan_kernel composes the maps in order
// into every segment's start state, and fused_ws_kernel runs the segments
// again from those states for the outputs.
#include <algorithm>
#include <atomic>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr float kSubFactoredMax = 64.f;  // largest block log2-decay of the factored products
constexpr float kSubMinLog2 = -128.f;    // floor of a token's log2-decay
constexpr float kLog2e = 1.4426950408889634f;

// Key channel held by row 4 g + e of state tile rt (see Layout).
__device__ __forceinline__ int state_channel(int rt, int g, int e) {
    return 32 * (rt >> 1) + 8 * g + 4 * (rt & 1) + e;
}

// The value of lane 15 of this lane's 16-lane row (DPP row_newbcast:15).
__device__ __forceinline__ float row_last(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xf, 0xf, false));
}
// Operands of one 64-token chunk (four 16-token blocks), in MFMA lane order.
template <int D>
struct SubRecord {
    static constexpr int NKS = D / 32, NCT = D / 16;
    bf16x8 ke[4][NKS][kWave];  // Ke (A operand of Ke S, channel order above)
    bf16x8 qe[4][NKS][kWave];  // Qe
    bf16x4 kt[4][NCT][kWave];  // K'^T, in the state's row tiles (A operand, K = tokens)
    bf16x4 tb[4][kWave];       // T Diag(beta)
    bf16x4 m[4][kWave];        // M
    f32x4 gend[4][D / 4];      // 2^tau per channel (channel order)
};

// LDS of the d = 64 kernel (fused_kernel).
template <int D>
struct FusedSmem {
    // row padding of the token x channel tiles: rows 8 banks apart, so the
    // recurrence's column reads (4 rows x 16 columns) hit 32 distinct banks
    static constexpr int TP = 16;
    SubRecord<D> rec;
    bf16 vt[64][D + TP];  // the chunk's V rows
    bf16 ot[64][D + TP];  // the chunk's outputs, written out by the next chunk
    int next;             // the chain this workgroup takes next
};

struct FusedParams {
    const bf16 *q, *k, *v, *g, *beta;
    const int32_t* cu;      // [N + 1] or null (equal lengths)
    const float* init;      // [N, H, D, D] or null (zero state)
    float* fin;             // [N, H, D, D] or null
    bf16* out;              // [T, H, D]
    const int32_t* order;   // sequences longest first, or null (natural order)
    int32_t* counter;       // chains handed out so far (zeroed before the launch)
    int64_t total_tokens;
    int32_t n_seqs, n_heads;
    float scale;
    int l2norm;
    // segmented passes: seg_per_seq chains (parts) per sequence and head,
    // n_seqs counting parts; the segments are placed by seg_bounds from each
    // sequence's length (cu, or equal lengths)
    int32_t seg_per_seq = 1;
    float* fin2 = nullptr;  // the first pass's linear parts M (fin takes b)
    float* st = nullptr;    // segment start states
};

__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// Two packed conversions (element-wise ones became four single conversions
// and two permutes where the result feeds a 16x16x16 product).
__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& x) { return from_f32x4<bf16>(x); }
__device__ __forceinline__ bf16x8 to_bf16x8(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
    return r;
}

// X^T Y for 16 x 16 fp32 matrices held in accumulator layout (lane (n, g)
// holds rows 4 g .. 4 g + 3 of column n): the K index of step s is 4 g + s, so
// each lane feeds its own element s of both.
__device__ __forceinline__ f32x4 mm_tn(const f32x4& X, const f32x4& Y) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[s], Y[s], acc, 0, 0, 0);
    return acc;
}

// T^T for T = (I + N)^-1, N strictly lower 16 x 16, from N and N^T.
__device__ __forceinline__ f32x4 unit_lower_inverse_t(const f32x4& N, const f32x4& Nt, int n16,
                                                      int g) {
    const f32x4 N2 = mm_tn(Nt, N), N2t = mm_tn(N, Nt);
    const f32x4 N4 = mm_tn(N2t, N2), N4t = mm_tn(N2, N2t);
    const f32x4 N8 = mm_tn(N4t, N4);
    f32x4 G;
#pragma unroll
    for (int e = 0; e < 4; ++e) G[e] = (4 * g + e == n16) ? 1.f : 0.f;
    G = G - Nt + N2t - mm_tn(N2, Nt);  // (I + N2^T)(I - N^T)
    G += mm_tn(N4, G);                 // (I + N4^T) G
    G += mm_tn(N8, G);                 // (I + N8^T) G
    return G;
}

// Exact diagonal products of one block at bisection level L (0: the diagonal
// of M): P = fk fk^T and Q = fk fq^T over this lane's channels, with fk, fq the
// rows scaled by this token's factor at the level.
__device__ __forceinline__ void exact_level(int L, int n16, int g, const float (&kh)[2][8],
                                            const float (&qh)[2][8], const float (&gam)[2][8],
                                            f32x4& P, f32x4& Q) {
    const int h = L == 0 ? 0 : (16 >> L);
    const int within = L == 0 ? 0 : (n16 & (2 * h - 1));
    const bool right = L > 0 && within >= h;
    const int b = L == 0 ? n16 : n16 - within + h - 1;  // reference token
    P = f32x4{0.f, 0.f, 0.f, 0.f};
    Q = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        float fk[8], fq[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float gb = __shfl(gam[kk][i], b + 16 * g, kWave);
            // gamma decreases along the block, so the exponent is <= 0 (the clamp
            // absorbs rounding in the sums); level 0 has factor 1
            const float f =
                L == 0 ? 1.f : exp2_hw(fminf(right ? gam[kk][i] - gb : gb - gam[kk][i], 0.f));
            fk[i] = kh[kk][i] * f;
            fq[i] = qh[kk][i] * f;
        }
        const bf16x8 a = to_bf16x8(fk), c = to_bf16x8(fq);
        P = mfma32(a, a, P);
        Q = mfma32(a, c, Q);
    }
}

// Where one chunk's rows of head h lie: a load past row Lc - 1 reads zero
// (Lc = 0: every load reads zero and none touches memory).
template <int D>
struct ChunkRange {
    int64_t ebase;      // element offset of (first token, head h, channel 0)
    uint32_t rowb;      // bytes per token row (all heads)
    uint32_t nbytes;    // bytes from ebase to the end of row Lc - 1 of head h
    __device__ ChunkRange(int64_t tok0, int Lc, int64_t H, int h)
        : ebase((tok0 * H + h) * D),
          rowb((uint32_t)(H * D * 2)),
          nbytes(Lc > 0 ? (uint32_t)(((int64_t)(Lc - 1) * H * D + D) * 2) : 0u) {}
};

// One chunk's inputs for one lane of the d = 64 kernel: q, k, g, v of token
// 16 w + lane % 16 over the lane's 8 channels of each of the two slices, and beta (kept
// zero-extended in a register of its own: packing 16-bit values would need the
// load to have landed at the point of packing).
struct ChunkRows {
    bf16x8 q[2], k[2], g[2], v[2];
    uint32_t beta;
};

// fp32 value of a zero-extended bf16
__device__ __forceinline__ float bf16_bits_f32(uint32_t x) { return __uint_as_float(x << 16); }

// PART selects what is loaded: 0 q and k, 1 g and beta, 2 v, -1 everything
// (the refill for the next chunk is spread over the recurrence, so its
// requests do not all queue at one point).
template <int D, int PART = -1>
__device__ __forceinline__ void load_chunk_rows(const FusedParams& p, int64_t tok0, int Lc, int h,
                                                int w, int lane, ChunkRows& r) {
    constexpr bool QK = PART < 0 || PART == 0, GB = PART < 0 || PART == 1, V = PART < 0 || PART == 2;
    static_assert(D == 64, "two 32-channel slices");
    const int n16 = lane & 15, g = lane >> 4, R = w;
    const int64_t H = p.n_heads;
    const ChunkRange<D> c(tok0, Lc, H, h);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(
        p.beta + tok0 * H + h, Lc > 0 ? (uint32_t)(((int64_t)(Lc - 1) * H + 1) * 2) : 0u);
    const uint32_t roff = (uint32_t)(16 * R + n16) * c.rowb;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const uint32_t off = roff + (uint32_t)(32 * kk + 8 * g) * 2;
        if constexpr (QK) {
            r.q[kk] = buffer_load<bf16x8>(rq, off);
            r.k[kk] = buffer_load<bf16x8>(rk, off);
        }
        if constexpr (GB) r.g[kk] = buffer_load<bf16x8>(rg, off);
        if constexpr (V) r.v[kk] = buffer_load<bf16x8>(rv, off);
    }
    if constexpr (GB) r.beta = buffer_load<uint16_t>(rb, (uint32_t)(16 * R + n16) * (uint32_t)H * 2);
}

// Writes the outputs of a chunk (first token tok0, Lc rows) from the LDS tile:
// one 16-byte store per 8 columns of a row.
template <int D>
__device__ __forceinline__ void flush_outputs(const FusedParams& p, const FusedSmem<D>& sm,
                                              int t, int64_t tok0, int Lc, int h) {
    constexpr int PIECES = 64 * D / 8, THREADS = D * 4;
    static_assert(PIECES % THREADS == 0, "whole passes over the tile");
#pragma unroll
    for (int it = 0; it < PIECES / THREADS; ++it) {
        const int i = t + it * THREADS;
        const int row = i / (D / 8), c8 = i % (D / 8);
        if (row < Lc)
            *reinterpret_cast<bf16x8*>(p.out + ((tok0 + row) * p.n_heads + h) * D + 8 * c8) =
                *reinterpret_cast<const bf16x8*>(&sm.ot[row][8 * c8]);
    }
}

// One 64-token chunk of one chain: the preparation writes the chunk's record
// to LDS, then every wave runs the recurrence over the four blocks on its 16
// value columns of S, leaving the outputs in the LDS tile.  `rows` holds the
// chunk's inputs and is refilled with those of the next chunk (none when
// next_len = 0) once the preparation has read them, spread over the inverse
// and the recurrence so the loads overlap them (every wait of a chunk is then
// for data asked for a chunk earlier: loads and stores share one in-order
// counter).  The previous chunk's outputs (prev_len > 0) are written out once
// every wave is past its recurrence.  `lane` is the lane index (passed in, so
// the caller can hand over a copy the compiler cannot see through).
template <int D>
__device__ __forceinline__ void fused_chunk(const FusedParams& p, FusedSmem<D>& sm,
                                            f32x4 (&S)[D / 16], int w, int lane, int64_t tok0,
                                            int Lc, int h, ChunkRows& rows, int next_len,
                                            int64_t prev_tok0, int prev_len) {
    static_assert(D == 64, "one wave per block over all its channels");
    constexpr int NKS = D / 32, NCT = D / 16;
    const int n16 = lane & 15, g = lane >> 4, col = 16 * w + n16;
    const int R = w;  // preparation: block

    // ---- preparation, block R; lane token 16 R + n16
    const bf16x8(&qv)[2] = rows.q;
    const bf16x8(&kv)[2] = rows.k;
    const bf16x8(&gv)[2] = rows.g;
    const float bt = bf16_bits_f32(rows.beta);
    const int t = 64 * w + lane;
    // every wave is past the previous chunk's recurrence (the barrier that
    // ended it): its outputs leave the tile and the V tile is free
    if (prev_len > 0) flush_outputs<D>(p, sm, t, prev_tok0, prev_len, h);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        *reinterpret_cast<bf16x8*>(&sm.vt[16 * R + n16][32 * kk + 8 * g]) = rows.v[kk];

    // in-block cumulative log2-decay: a scan over the 16 lanes of each row
    float gam[2][8], tau[2][8];
    float sq = 0.f, sk = 0.f;
    bool big = false;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x = fmaxf(to_f32(gv[kk][i]) * kLog2e, kSubMinLog2);
            x += dpp<0x111>(x);  // row_shr:1
            x += dpp<0x112>(x);  // row_shr:2
            x += dpp<0x114>(x);  // row_shr:4
            x += dpp<0x118>(x);  // row_shr:8
            gam[kk][i] = x;
            tau[kk][i] = __shfl(x, lane | 15, kWave);
            big |= -tau[kk][i] > kSubFactoredMax;
            const float qx = to_f32(qv[kk][i]), kx = to_f32(kv[kk][i]);
            sq += qx * qx;
            sk += kx * kx;
        }
    sq += xor_shfl(sq, 16);
    sq += xor_shfl(sq, 32);
    sk += xor_shfl(sk, 16);
    sk += xor_shfl(sk, 32);
    const int ex = __builtin_amdgcn_readfirstlane(__ballot(big) != 0ull ? 1 : 0);
    const float rqs = (p.l2norm ? __builtin_amdgcn_rsqf(sq + kL2Eps) : 1.f) * p.scale;
    const float rks = p.l2norm ? __builtin_amdgcn_rsqf(sk + kL2Eps) : 1.f;

    // 0/1 selectors for the K'^T tiles: output column n (state row n of tile
    // 2 ks or 2 ks + 1) takes channel state_channel(2 ks (+ 1), n / 4, n % 4),
    // element n % 4 (lo) or 4 + n % 4 (hi) of lane group n / 4
    bf16x8 sel_lo, sel_hi;
    {
        const uint32_t one = (g == (n16 >> 2)) ? 0x3F80u : 0u;  // bf16 1.0
        const uint32_t w0 = (n16 & 2) ? 0u : one << (16 * (n16 & 1));
        const uint32_t w1 = (n16 & 2) ? one << (16 * (n16 & 1)) : 0u;
        sel_lo = __builtin_bit_cast(bf16x8, u32x4{w0, w1, 0u, 0u});
        sel_hi = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, w0, w1});
    }
    f32x4 Aa = {0.f, 0.f, 0.f, 0.f}, Ata = Aa, Mta = Aa;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int ks = kk;
        float ke[8], qe[8], kf[8], kfs[8], T[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float kh = to_f32(kv[kk][i]) * rks;
            const float qh = to_f32(qv[kk][i]) * rqs;
            const float E = exp2_hw(gam[kk][i]);
            // (past the factored range G may overflow; the products that use it
            // are then skipped and K' is redone below)
            const float G = exp2_hw(-gam[kk][i]);
            T[i] = __shfl(E, lane | 15, kWave);  // 2^tau, from the block's last token
            ke[i] = kh * E;
            qe[i] = qh * E;
            kfs[i] = kh * G;
            // K' = khat 2^(tau - Gamma); past the factored range it is redone below
            kf[i] = kfs[i] * T[i];
        }
        const bf16x8 KE = to_bf16x8(ke), QE = to_bf16x8(qe), KF = to_bf16x8(kf);
        sm.rec.ke[R][ks][lane] = KE;
        sm.rec.qe[R][ks][lane] = QE;
        if (!ex) {
            const bf16x8 KS = to_bf16x8(kfs);
            Aa = mfma32(KE, KS, Aa);    // A[i][j] / beta_i
            Ata = mfma32(KS, KE, Ata);  // its transpose
            Mta = mfma32(KS, QE, Mta);  // M^T
        }
        // K'^T tiles 2 ks, 2 ks + 1 (products with the selectors)
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        sm.rec.kt[R][2 * ks][lane] = to_bf16x4(mfma32(KF, sel_lo, z));
        sm.rec.kt[R][2 * ks + 1][lane] = to_bf16x4(mfma32(KF, sel_hi, z));
        if (n16 == 0) {
            sm.rec.gend[R][8 * ks + 2 * g] = f32x4{T[0], T[1], T[2], T[3]};
            sm.rec.gend[R][8 * ks + 2 * g + 1] = f32x4{T[4], T[5], T[6], T[7]};
        }
    }
    if (ex) {
        float kh[2][8], qh[2][8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kh[kk][i] = to_f32(kv[kk][i]) * rks;
                qh[kk][i] = to_f32(qv[kk][i]) * rqs;
            }
        // every pair (i, j) belongs to exactly one level: select, not add
#pragma unroll 1
        for (int L = 0; L <= 4; ++L) {
            f32x4 P, Q;
            exact_level(L, n16, g, kh, qh, gam, P, Q);
            const int sh = 5 - L, m2 = (32 >> L) - 1, hh = 16 >> L;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                if (L == 0) {
                    Mta[e] = r == n16 ? Q[e] : Mta[e];
                } else {
                    const bool same = (r >> sh) == (n16 >> sh);
                    // (i, j) = (r, n16) and (n16, r): i in the right half, j in the left
                    const bool a_rn = same && (r & m2) >= hh && (n16 & m2) < hh;
                    const bool a_nr = same && (n16 & m2) >= hh && (r & m2) < hh;
                    Aa[e] = a_rn ? P[e] : Aa[e];
                    Ata[e] = a_nr ? P[e] : Ata[e];
                    Mta[e] = a_nr ? Q[e] : Mta[e];
                }
            }
        }
        // K' from its own exponent: 2^tau may be far below 2^-64 here
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ks = kk;
            float kf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) kf[i] = kh[kk][i] * exp2_hw(tau[kk][i] - gam[kk][i]);
            const bf16x8 KF = to_bf16x8(kf);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            sm.rec.kt[R][2 * ks][lane] = to_bf16x4(mfma32(KF, sel_lo, z));
            sm.rec.kt[R][2 * ks + 1][lane] = to_bf16x4(mfma32(KF, sel_hi, z));
            if (n16 == 0) {
                sm.rec.gend[R][8 * ks + 2 * g] = f32x4{exp2_hw(tau[kk][0]), exp2_hw(tau[kk][1]),
                                                       exp2_hw(tau[kk][2]), exp2_hw(tau[kk][3])};
                sm.rec.gend[R][8 * ks + 2 * g + 1] = f32x4{exp2_hw(tau[kk][4]), exp2_hw(tau[kk][5]),
                                                           exp2_hw(tau[kk][6]), exp2_hw(tau[kk][7])};
            }
        }
    }
    // the rows are read: refill them with the next chunk's (q and k now, the
    // rest during the recurrence)
    load_chunk_rows<D, 0>(p, tok0 + 64, next_len, h, w, lane, rows);
    {
        f32x4 N, Nt, Mt, bi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            bi[e] = __shfl(bt, r, kWave);  // beta of token r
            N[e] = n16 < r ? Aa[e] * bi[e] : 0.f;
            Nt[e] = r < n16 ? Ata[e] * bt : 0.f;
            Mt[e] = r <= n16 ? Mta[e] : 0.f;
        }
        const f32x4 Tt = unit_lower_inverse_t(N, Nt, n16, g);
        sm.rec.tb[R][lane] = to_bf16x4(Tt * bi);
        sm.rec.m[R][lane] = to_bf16x4(Mt);
    }
    __syncthreads();  // the record is complete


    // ---- recurrence over the four blocks, value columns of this wave
#pragma unroll
    for (int Rb = 0; Rb < 4; ++Rb) {
        bf16x8 Sb[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Sb[ks][e] = (bf16)S[2 * ks][e];
                Sb[ks][4 + e] = (bf16)S[2 * ks + 1][e];
            }
        f32x4 X = {0.f, 0.f, 0.f, 0.f}, O = X;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            X = mfma32(sm.rec.ke[Rb][ks][lane], Sb[ks], X);
            O = mfma32(sm.rec.qe[Rb][ks][lane], Sb[ks], O);
        }
        f32x4 Yf;
#pragma unroll
        for (int e = 0; e < 4; ++e) Yf[e] = to_f32(sm.vt[16 * Rb + 4 * g + e][col]) - X[e];
        const bf16x4 u = to_bf16x4(mfma16(sm.rec.tb[Rb][lane], to_bf16x4(Yf), f32x4{0.f, 0.f, 0.f, 0.f}));
        O = mfma16(sm.rec.m[Rb][lane], u, O);
        const bf16x4 ob = to_bf16x4(O);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.ot[16 * Rb + 4 * g + e][col] = ob[e];
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt)
            S[rt] = mfma16(sm.rec.kt[Rb][rt][lane], u,
                           S[rt] * sm.rec.gend[Rb][state_channel(rt, g, 0) / 4]);
        if (Rb == 0) load_chunk_rows<D, 1>(p, tok0 + 64, next_len, h, w, lane, rows);
        if (Rb == 1) load_chunk_rows<D, 2>(p, tok0 + 64, next_len, h, w, lane, rows);
    }
    // every wave is past its recurrence before the next chunk writes the record
    __syncthreads();
}

// A workgroup of four waves (d = 64) works on one chain at a time; persistent,
// chains handed out through `counter` in `order`.  Every workgroup takes
// chains until the counter passes the last one, so all of them finish.
template <int D>
__global__ __launch_bounds__(D * 4, 2) void fused_kernel(FusedParams p) {
    static_assert(D == 64, "d = 128 takes fused_ws_kernel");
    constexpr int NCT = D / 16;
    __shared__ FusedSmem<D> sm;
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n16 = lane & 15, g = lane >> 4, col = 16 * w + n16;
    const int64_t H = p.n_heads;
    const int64_t chains = (int64_t)p.n_seqs * H;
    for (;;) {
        if (t == 0) sm.next = atomicAdd(p.counter, 1);
        __syncthreads();
        const int64_t ci = sm.next;
        __syncthreads();  // every thread has read `next` before it is written again
        if (ci >= chains) break;
        const int64_t si = ci / H;
        const int h = (int)(ci - si * H);
        const int64_t n = p.order ? (int64_t)p.order[si] : si;
        int64_t s_begin, s_len;
        if (p.cu) {
            s_begin = p.cu[n];
            s_len = (int64_t)p.cu[n + 1] - s_begin;
        } else {
            s_len = p.total_tokens / p.n_seqs;
            s_begin = n * s_len;
        }
        // this lane's state: key channels state_channel(rt, g, e), value column col
        const int64_t sbase = (n * H + h) * D * D;
        f32x4 S[NCT];
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[rt][e] = p.init ? p.init[sbase + (int64_t)state_channel(rt, g, e) * D + col] : 0.f;
        // the state's loads complete here, once per chain: left pending, their
        // first use inside the chunk loop would wait for every load in flight
#pragma unroll
        for (int rt = 0; rt < NCT; ++rt) asm volatile("" : "+v"(S[rt]));
        const int64_t nch = (s_len + 63) / 64;
        ChunkRows rows;
        load_chunk_rows<D>(p, s_begin, (int)min((int64_t)64, s_len), h, w, lane, rows);
        int64_t prev_tok0 = 0;
        int prev_len = 0;
        for (int64_t kc = 0; kc < nch; ++kc) {
            // a copy of the lane index the compiler cannot see through: the
            // chunk's index arithmetic is redone per chunk instead of hoisted
            // out of this loop and held in registers across it
            int lane_c = lane;
            asm volatile("" : "+v"(lane_c));
            const int64_t rest = s_len - 64 * kc;  // tokens from this chunk on
            const int len = (int)min((int64_t)64, rest);
            fused_chunk<D>(p, sm, S, w, lane_c, s_begin + 64 * kc, len, h, rows,
                           (int)max((int64_t)0, min((int64_t)64, rest - 64)), prev_tok0, prev_len);
            prev_tok0 = s_begin + 64 * kc;
            prev_len = len;
        }
        __syncthreads();  // the last chunk's outputs are complete
        if (prev_len > 0) flush_outputs<D>(p, sm, t, prev_tok0, prev_len, h);
        if (p.fin) {
#pragma unroll
            for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.fin[sbase + (int64_t)state_channel(rt, g, e) * D + col] = S[rt][e];
        }
    }
}

// ------------------------------------------------------------ specialised waves
//
// At d = 128 the workgroup holds two kinds of waves.  Four preparation waves,
// one per 16-token block and each over all the block's channels, write the
// record of chunk i while four recurrence waves, 32 value columns each, run
// chunk i - 1 from the other record buffer.  One of each shares a SIMD, so
// the hardware fills one's waits with the other's work, and they meet once per
// chunk, at the barrier after which record i is complete and record i - 1 is
// free.  A recurrence wave loads its own V columns, runs its two 16-column
// tiles through each block together (one read of each record operand serves
// both), writes the outputs over the V rows they replace and sends them out
// with 16-byte stores.

template <int D>
struct WsSmem {
    static constexpr int TPV = 8;  // V rows 4 banks apart
    SubRecord<D> rec[2];
    bf16 vt[64][D + TPV];          // V of the chunk under recurrence, then its outputs
    int next;
};

// Waves per workgroup: preparation (one per block), recurrence.
template <int D>
constexpr int kWsPrep = 4;
template <int D>
constexpr int kWsRec = D / 32;

// A preparation wave's inputs: q, k, g of token 16 R + lane % 16 over the
// lane's 8 channels of each of the D / 32 slices (channels 32 ks + 8 (lane /
// 16) ..), and beta (zero-extended, as in ChunkRows).
template <int D>
struct BlockRows {
    bf16x8 q[D / 32], k[D / 32], g[D / 32];
    uint32_t beta;
};

// PART 0: q and k, 1: g and beta, -1 all; rows past Lc read zero.  QROWS false:
// no q (a pass that writes no outputs).
template <int D, int PART = -1, bool QROWS = true>
__device__ __forceinline__ void ws_load_rows(const FusedParams& p, int64_t tok0, int Lc, int h,
                                             int R, int lane, BlockRows<D>& r) {
    constexpr bool QK = PART < 0 || PART == 0, GB = PART < 0 || PART == 1;
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t H = p.n_heads;
    const ChunkRange<D> c(tok0, Lc, H, h);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + c.ebase, c.nbytes);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(
        p.beta + tok0 * H + h, Lc > 0 ? (uint32_t)(((int64_t)(Lc - 1) * H + 1) * 2) : 0u);
    const uint32_t roff = (uint32_t)(16 * R + n16) * c.rowb;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const uint32_t off = roff + (uint32_t)(32 * ks + 8 * g) * 2;
        if constexpr (QK) {
            if constexpr (QROWS) r.q[ks] = buffer_load<bf16x8>(rq, off);
            r.k[ks] = buffer_load<bf16x8>(rk, off);
        }
        if constexpr (GB) r.g[ks] = buffer_load<bf16x8>(rg, off);
    }
    if constexpr (GB) r.beta = buffer_load<uint16_t>(rb, (uint32_t)(16 * R + n16) * (uint32_t)H * 2);
}

// Preparation of block R of one chunk (first token tok0) into `rec`, by one
// wave over all the block's channels; the same arithmetic as fused_chunk, the
// two channel halves' partial products summed in the same order.  `rows` holds
// the block's inputs and is refilled with the next chunk's (next_len tokens)
// once read.  QROWS false: the record's Qe and M are not formed (no outputs).
template <int D, bool QROWS = true>
__device__ __forceinline__ void ws_prep(const FusedParams& p, SubRecord<D>& rec, int R, int lane,
                                        int64_t tok0, int h, BlockRows<D>& rows, int next_len) {
    static_assert(D == 128, "two channel halves of two slices");
    const int n16 = lane & 15, g = lane >> 4;
    const float bt = bf16_bits_f32(rows.beta);

    // in-block cumulative log2-decay: a scan over the 16 lanes of each row;
    // [half][slice in half][channel]
    float gam[2][2][8];
    float sq[2] = {0.f, 0.f}, sk[2] = {0.f, 0.f};
    bool big = false;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float x = fmaxf(to_f32(rows.g[2 * hf + kk][i]) * kLog2e, kSubMinLog2);
                x += dpp<0x111>(x);  // row_shr:1
                x += dpp<0x112>(x);  // row_shr:2
                x += dpp<0x114>(x);  // row_shr:4
                x += dpp<0x118>(x);  // row_shr:8
                gam[hf][kk][i] = x;
                // the block's total decay sits in its last lane
                big |= n16 == 15 && -x > kSubFactoredMax;
            }
    // g and beta are read: request the next chunk's
    ws_load_rows<D, 1, QROWS>(p, tok0 + 64, next_len, h, R, lane, rows);
    // the norms' sums of squares, two channels per step (bf16 pairs)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (QROWS) {
                    const bf16x2 qx = {rows.q[2 * hf + kk][2 * i], rows.q[2 * hf + kk][2 * i + 1]};
                    sq[hf] = __builtin_amdgcn_fdot2_f32_bf16(qx, qx, sq[hf], false);
                }
                const bf16x2 kx = {rows.k[2 * hf + kk][2 * i], rows.k[2 * hf + kk][2 * i + 1]};
                sk[hf] = __builtin_amdgcn_fdot2_f32_bf16(kx, kx, sk[hf], false);
            }
        sq[hf] += xor_shfl(sq[hf], 16);
        sq[hf] += xor_shfl(sq[hf], 32);
        sk[hf] += xor_shfl(sk[hf], 16);
        sk[hf] += xor_shfl(sk[hf], 32);
    }
    const int ex = __builtin_amdgcn_readfirstlane(__ballot(big) != 0ull ? 1 : 0);
    const float rqs = (p.l2norm ? __builtin_amdgcn_rsqf(sq[0] + sq[1] + kL2Eps) : 1.f) * p.scale;
    const float rks = p.l2norm ? __builtin_amdgcn_rsqf(sk[0] + sk[1] + kL2Eps) : 1.f;

    bf16x8 sel_lo, sel_hi;  // 0/1 selectors for the K'^T tiles (as in fused_chunk)
    {
        const uint32_t one = (g == (n16 >> 2)) ? 0x3F80u : 0u;  // bf16 1.0
        const uint32_t w0 = (n16 & 2) ? 0u : one << (16 * (n16 & 1));
        const uint32_t w1 = (n16 & 2) ? one << (16 * (n16 & 1)) : 0u;
        sel_lo = __builtin_bit_cast(bf16x8, u32x4{w0, w1, 0u, 0u});
        sel_hi = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, w0, w1});
    }
    f32x4 Aa[2], Ata[2], Mta[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        Aa[hf] = Ata[hf] = Mta[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ks = 2 * hf + kk;
            float ke[8], qe[8], kf[8], kfs[8], E[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float kh = to_f32(rows.k[ks][i]) * rks;
                const float qh = QROWS ? to_f32(rows.q[ks][i]) * rqs : 0.f;
                E[i] = exp2_hw(gam[hf][kk][i]);
                // (past the factored range G may overflow; the products that use
                // it are then skipped and K' is redone below)
                const float G = exp2_hw(-gam[hf][kk][i]);
                ke[i] = kh * E[i];
                qe[i] = qh * E[i];
                kfs[i] = kh * G;
                // K' = khat 2^(tau - Gamma), 2^tau from the block's last token
                kf[i] = kfs[i] * __shfl(E[i], lane | 15, kWave);
            }
            const bf16x8 KE = to_bf16x8(ke), QE = to_bf16x8(qe), KF = to_bf16x8(kf);
            rec.ke[R][ks][lane] = KE;
            if constexpr (QROWS) rec.qe[R][ks][lane] = QE;
            if (!ex) {
                const bf16x8 KS = to_bf16x8(kfs);
                Aa[hf] = mfma32(KE, KS, Aa[hf]);    // A[i][j] / beta_i
                Ata[hf] = mfma32(KS, KE, Ata[hf]);  // its transpose
                if constexpr (QROWS) Mta[hf] = mfma32(KS, QE, Mta[hf]);  // M^T
            }
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            rec.kt[R][2 * ks][lane] = to_bf16x4(mfma32(KF, sel_lo, z));
            rec.kt[R][2 * ks + 1][lane] = to_bf16x4(mfma32(KF, sel_hi, z));
            if (n16 == 15) {  // the block's last token: E = 2^tau
                rec.gend[R][8 * ks + 2 * g] = f32x4{E[0], E[1], E[2], E[3]};
                rec.gend[R][8 * ks + 2 * g + 1] = f32x4{E[4], E[5], E[6], E[7]};
            }
        }
    }
    if (ex) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float kh[2][8], qh[2][8], tau[2][8];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    kh[kk][i] = to_f32(rows.k[2 * hf + kk][i]) * rks;
                    qh[kk][i] = QROWS ? to_f32(rows.q[2 * hf + kk][i]) * rqs : 0.f;
                    tau[kk][i] = row_last(gam[hf][kk][i]);
                }
            Aa[hf] = Ata[hf] = Mta[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
            // every pair (i, j) belongs to exactly one level: select, not add
#pragma unroll 1
            for (int L = 0; L <= 4; ++L) {
                f32x4 P, Q;
                exact_level(L, n16, g, kh, qh, gam[hf], P, Q);
                const int sh = 5 - L, m2 = (32 >> L) - 1, hh = 16 >> L;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    if (L == 0) {
                        Mta[hf][e] = r == n16 ? Q[e] : Mta[hf][e];
                    } else {
                        const bool same = (r >> sh) == (n16 >> sh);
                        // (i, j) = (r, n16) and (n16, r): i in the right half, j in the left
                        const bool a_rn = same && (r & m2) >= hh && (n16 & m2) < hh;
                        const bool a_nr = same && (n16 & m2) >= hh && (r & m2) < hh;
                        Aa[hf][e] = a_rn ? P[e] : Aa[hf][e];
                        Ata[hf][e] = a_nr ? P[e] : Ata[hf][e];
                        Mta[hf][e] = a_nr ? Q[e] : Mta[hf][e];
                    }
                }
            }
            // K' from its own exponent: 2^tau may be far below 2^-64 here
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ks = 2 * hf + kk;
                float kf[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) kf[i] = kh[kk][i] * exp2_hw(tau[kk][i] - gam[hf][kk][i]);
                const bf16x8 KF = to_bf16x8(kf);
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                rec.kt[R][2 * ks][lane] = to_bf16x4(mfma32(KF, sel_lo, z));
                rec.kt[R][2 * ks + 1][lane] = to_bf16x4(mfma32(KF, sel_hi, z));
                if (n16 == 0) {
                    rec.gend[R][8 * ks + 2 * g] = f32x4{exp2_hw(tau[kk][0]), exp2_hw(tau[kk][1]),
                                                        exp2_hw(tau[kk][2]), exp2_hw(tau[kk][3])};
                    rec.gend[R][8 * ks + 2 * g + 1] = f32x4{exp2_hw(tau[kk][4]), exp2_hw(tau[kk][5]),
                                                            exp2_hw(tau[kk][6]), exp2_hw(tau[kk][7])};
                }
            }
        }
    }
    // q and k are read: request the next chunk's
    ws_load_rows<D, 0, QROWS>(p, tok0 + 64, next_len, h, R, lane, rows);
    {
        const f32x4 As = Aa[0] + Aa[1], Ats = Ata[0] + Ata[1], Ms = Mta[0] + Mta[1];
        f32x4 N, Nt, Mt, bi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            bi[e] = __shfl(bt, r, kWave);  // beta of token r
            N[e] = n16 < r ? As[e] * bi[e] : 0.f;
            Nt[e] = r < n16 ? Ats[e] * bt : 0.f;
            Mt[e] = r <= n16 ? Ms[e] : 0.f;
        }
        const f32x4 Tt = unit_lower_inverse_t(N, Nt, n16, g);
        rec.tb[R][lane] = to_bf16x4(Tt * bi);
        if constexpr (QROWS) rec.m[R][lane] = to_bf16x4(Mt);
    }
}

// One 16-token block of the recurrence on NT 16-column tiles of a recurrence
// wave (tile c: value column 32 wr + 16 (c % 2) + lane % 16 of its state):
// operands from `rec`; tiles c < NV take V from `vt`, the others V = 0 (the
// linear part of a state map).  OUT: the outputs of tiles 0 and 1 replace the
// block's V rows in `vt`.  Every record operand read serves all NT tiles.
template <int D, int TPV, bool OUT, int NT, int NV>
__device__ __forceinline__ void ws_block(const SubRecord<D>& rec, bf16 (&vt)[64][D + TPV],
                                         f32x4 (&S)[NT][D / 16], int wr, int lane, int Rb) {
    static_assert(!OUT || (NT == 2 && NV == 2), "outputs only for two V tiles");
    constexpr int NKS = D / 32, NCT = D / 16;
    const int n16 = lane & 15, g = lane >> 4;
    // X = Ke S (and O = Qe S): the state as B operands (tile c, rows 32 ks ..
    // 32 ks + 31), two tiles converted up front, four step by step (fewer
    // registers live)
    f32x4 X[NT], O[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) X[c] = O[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NT == 2) {
        bf16x8 Sb[NT][NKS];
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Sb[c][ks][e] = (bf16)S[c][2 * ks][e];
                    Sb[c][ks][4 + e] = (bf16)S[c][2 * ks + 1][e];
                }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 a = rec.ke[Rb][ks][lane];
#pragma unroll
            for (int c = 0; c < NT; ++c) X[c] = mfma32(a, Sb[c][ks], X[c]);
            if constexpr (OUT) {
                const bf16x8 b = rec.qe[Rb][ks][lane];
#pragma unroll
                for (int c = 0; c < NT; ++c) O[c] = mfma32(b, Sb[c][ks], O[c]);
            }
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            bf16x8 Sb[NT];
#pragma unroll
            for (int c = 0; c < NT; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Sb[c][e] = (bf16)S[c][2 * ks][e];
                    Sb[c][4 + e] = (bf16)S[c][2 * ks + 1][e];
                }
            const bf16x8 a = rec.ke[Rb][ks][lane];
#pragma unroll
            for (int c = 0; c < NT; ++c) X[c] = mfma32(a, Sb[c], X[c]);
        }
    }
    const bf16x4 tb = rec.tb[Rb][lane];
    const bf16x4 m = OUT ? rec.m[Rb][lane] : bf16x4{};
    bf16x4 u[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int col = 32 * wr + 16 * (c % 2) + n16;
        f32x4 Yf;
#pragma unroll
        for (int e = 0; e < 4; ++e) Yf[e] = (c < NV ? to_f32(vt[16 * Rb + 4 * g + e][col]) : 0.f) - X[c][e];
        u[c] = to_bf16x4(mfma16(tb, to_bf16x4(Yf), f32x4{0.f, 0.f, 0.f, 0.f}));
        if constexpr (OUT) {
            O[c] = mfma16(m, u[c], O[c]);
            const bf16x4 ob = to_bf16x4(O[c]);
#pragma unroll
            for (int e = 0; e < 4; ++e) vt[16 * Rb + 4 * g + e][col] = ob[e];
        }
    }
#pragma unroll
    for (int rt = 0; rt < NCT; ++rt) {
        const bf16x4 a = rec.kt[Rb][rt][lane];
        const f32x4 gd = rec.gend[Rb][state_channel(rt, g, 0) / 4];
#pragma unroll
        for (int c = 0; c < NT; ++c) S[c][rt] = mfma16(a, u[c], S[c][rt] * gd);
    }
}

// A recurrence wave's V columns of one chunk (Lc rows): lane piece j is row
// 16 j + lane / 4, columns 32 wr + 8 (lane % 4) ..; rows past Lc read zero.
template <int D>
__device__ __forceinline__ void ws_load_v(const FusedParams& p, int64_t tok0, int Lc, int h,
                                          int wr, int lane, bf16x8 (&v)[4]) {
    const ChunkRange<D> c(tok0, Lc, p.n_heads, h);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + c.ebase, c.nbytes);
    const uint32_t cb = (uint32_t)(32 * wr + 8 * (lane & 3)) * 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = buffer_load<bf16x8>(rv, (uint32_t)(16 * j + (lane >> 2)) * c.rowb + cb);
}

// The same pieces of the outputs from `vt` to HBM; rows past Lc are dropped
// by the range check of the stores.
template <int D, int TPV>
__device__ __forceinline__ void ws_flush(const FusedParams& p, const bf16 (&vt)[64][D + TPV],
                                         int64_t tok0, int Lc, int h, int wr, int lane) {
    const ChunkRange<D> c(tok0, Lc, p.n_heads, h);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.out + c.ebase, c.nbytes);
    const int c8 = 32 * wr + 8 * (lane & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * j + (lane >> 2);
        const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(&vt[r][c8]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o8), ro,
                                               (int)((uint32_t)r * c.rowb + (uint32_t)c8 * 2), 0, 0);
    }
}

// Placement of a sequence's segments in a segmented call with Q chains per
// sequence and head in each pass (Q + 1 segments): of its C chunks, segments
// 1..Q take l = ceil(7 C / (7 Q + 8)) each (the last ones shorter or empty)
// and segment 0 the a = max(0, C - Q l) before them, about 8/7 of l.
// Segment 0 runs with its outputs in the first pass beside the maps of
// segments 1..Q-1, whose chains take about 8/7 as long per chunk.
__device__ __forceinline__ void seg_bounds(int64_t seq_len, int Q, int s, int64_t& begin,
                                           int64_t& len) {
    const int64_t C = (seq_len + 63) / 64;
    const int64_t l = (7 * C + 7 * Q + 7) / (7 * Q + 8);
    const int64_t a = max((int64_t)0, C - Q * l);
    const int64_t c0 = s == 0 ? 0 : min(C, a + (int64_t)(s - 1) * l);
    const int64_t c1 = s == 0 ? a : min(C, a + (int64_t)s * l);
    begin = 64 * c0;
    len = max((int64_t)0, min(64 * c1, seq_len) - 64 * c0);
}

// One chain through fused_ws_kernel: tokens [s_begin, s_begin + s_len) of
// head h, from the state `init` (null: zero) to `fin` (null: not written),
// each the chain's [D, D] fp32 state.  OUT: the outputs are written.  MAPS
// (without OUT): the chain's state map instead, each recurrence wave carrying
// two tiles of b, from the zero state with V, to `fin` and two of M, from the
// identity with V = 0, to `fin2` (init unused).
template <int D, bool OUT, bool MAPS>
__device__ __forceinline__ void ws_chain(const FusedParams& p, WsSmem<D>& sm, int w, int lane,
                                         int h, int64_t s_begin, int64_t s_len,
                                         const float* __restrict__ init, float* __restrict__ fin,
                                         float* __restrict__ fin2) {
    static_assert(!(OUT && MAPS), "a map pass writes no outputs");
    constexpr int NCT = D / 16, TPV = WsSmem<D>::TPV;
    constexpr int NT = MAPS ? 4 : 2;  // 16-column state tiles per recurrence wave
    constexpr int NV = 2;             // of which the first NV see V
    const int64_t nch = (s_len + 63) / 64;
    const auto len_of = [&](int64_t kc) {
        return (int)max((int64_t)0, min((int64_t)64, s_len - 64 * kc));
    };
    if (w < kWsPrep<D>) {
        // block w of chunk kc into record kc % 2, a barrier after each,
        // then one for the last chunk's recurrence
        if (nch > 0) {
            BlockRows<D> rows;
            ws_load_rows<D, -1, OUT>(p, s_begin, len_of(0), h, w, lane, rows);
            for (int64_t kc = 0; kc < nch; ++kc) {
                // a copy of the lane index the compiler cannot see
                // through: the chunk's index arithmetic is redone per
                // chunk instead of held in registers across the loop
                int lane_c = lane;
                asm volatile("" : "+v"(lane_c));
                ws_prep<D, OUT>(p, sm.rec[kc & 1], w, lane_c, s_begin + 64 * kc, h, rows,
                                len_of(kc + 1));
                __syncthreads();
            }
            __syncthreads();
        }
    } else {
        const int wr = w - kWsPrep<D>;
        const int n16 = lane & 15, g = lane >> 4;
        // this lane's state: key channels state_channel(rt, g, e), value
        // column 32 wr + 16 (c % 2) + n16 of tile c
        f32x4 S[NT][NCT];
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int rt = 0; rt < NCT; ++rt) S[c][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the M tiles start from the identity
#pragma unroll
        for (int c = NV; c < NT; ++c)
#pragma unroll
            for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[c][rt][e] = state_channel(rt, g, e) == 32 * wr + 16 * (c % 2) + n16 ? 1.f : 0.f;
        if (!MAPS && init) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[c][rt][e] = init[(int64_t)state_channel(rt, g, e) * D + 32 * wr + 16 * c + n16];
        }
        // the state's loads complete here, once per chain
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
            for (int rt = 0; rt < NCT; ++rt) asm volatile("" : "+v"(S[c][rt]));
        if (nch > 0) {
            bf16x8 v[4];
            ws_load_v<D>(p, s_begin, len_of(0), h, wr, lane, v);
            // step 0: nothing to run; V of chunk 0 to the tile
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<bf16x8*>(&sm.vt[16 * j + (lane >> 2)][32 * wr + 8 * (lane & 3)]) = v[j];
            ws_load_v<D>(p, s_begin + 64, len_of(1), h, wr, lane, v);
            __syncthreads();
            // step kc: the recurrence of chunk kc - 1 from record (kc - 1) % 2
            for (int64_t kc = 1; kc <= nch; ++kc) {
                int lane_c = lane;
                asm volatile("" : "+v"(lane_c));
                const SubRecord<D>& rec = sm.rec[(kc - 1) & 1];
#pragma unroll
                for (int Rb = 0; Rb < 4; ++Rb)
                    ws_block<D, TPV, OUT, NT, NV>(rec, sm.vt, S, wr, lane_c, Rb);
                if constexpr (OUT)
                    ws_flush<D, TPV>(p, sm.vt, s_begin + 64 * (kc - 1), len_of(kc - 1), h, wr, lane_c);
                if (kc < nch) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<bf16x8*>(
                            &sm.vt[16 * j + (lane_c >> 2)][32 * wr + 8 * (lane_c & 3)]) = v[j];
                    ws_load_v<D>(p, s_begin + 64 * (kc + 1), len_of(kc + 1), h, wr, lane_c, v);
                }
                __syncthreads();
            }
        }
        if (fin) {
#pragma unroll
            for (int c = 0; c < NT; ++c) {
                float* f = c < 2 ? fin : fin2;
#pragma unroll
                for (int rt = 0; rt < NCT; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        f[(int64_t)state_channel(rt, g, e) * D + 32 * wr + 16 * (c % 2) + n16] = S[c][rt][e];
            }
        }
    }
}

// Chains of fused_ws_kernel.  kWsPlain: (sequence, head) pairs, states p.init
// and p.fin [N, H, D, D].  The segmented prefill's two passes, chains (part,
// head) with p.seg_per_seq = Q parts per sequence (p.n_seqs counts parts):
// kWsSegFirst, part 0 runs segment 0 with its outputs from p.init to start
// state slot 1 of p.st, and part k >= 1 forms the map of segment k, b to p.fin
// and M to p.fin2; kWsSegOut, part k runs segment k + 1 with its outputs from
// start slot k + 1 of p.st, and the last part writes the final state to p.fin
// [N, H, D, D].  p.st, p.fin and p.fin2 of the first pass are [N (Q + 1), H,
// D, D], slot s of sequence n at n (Q + 1) + s.
enum WsKind { kWsPlain = 0, kWsSegFirst = 1, kWsSegOut = 2 };

template <int D, int KIND = kWsPlain>
__global__ __launch_bounds__(64 * (kWsPrep<D> + kWsRec<D>), 1) void fused_ws_kernel(FusedParams p) {
    __shared__ WsSmem<D> sm;
    const int t = threadIdx.x, lane0 = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t H = p.n_heads;
    const int64_t chains = (int64_t)p.n_seqs * H;
    constexpr int64_t DD = (int64_t)D * D;
    for (;;) {
        if (t == 0) sm.next = atomicAdd(p.counter, 1);
        __syncthreads();
        const int64_t ci = sm.next;
        __syncthreads();  // every thread has read `next` before it is written again
        if (ci >= chains) break;
        const int64_t si = ci / H;
        const int h = (int)(ci - si * H);
        // a copy of the lane index the compiler cannot see through: what the
        // chain derives from it is computed per chain, not hoisted out of the
        // chain loop and held (or spilled) for the whole kernel
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        if constexpr (KIND == kWsPlain) {
            const int64_t n = p.order ? (int64_t)p.order[si] : si;
            int64_t s_begin, s_len;
            if (p.cu) {
                s_begin = p.cu[n];
                s_len = (int64_t)p.cu[n + 1] - s_begin;
            } else {
                s_len = p.total_tokens / p.n_seqs;
                s_begin = n * s_len;
            }
            const int64_t sb = (n * H + h) * DD;
            ws_chain<D, true, false>(p, sm, w, lane, h, s_begin, s_len, p.init ? p.init + sb : nullptr,
                                     p.fin ? p.fin + sb : nullptr, nullptr);
        } else {
            const int Q = p.seg_per_seq;
            const int64_t seq = si / Q;
            const int s = (int)(si - seq * Q) + (KIND == kWsSegOut ? 1 : 0);
            int64_t seq_begin, seq_len;
            if (p.cu) {
                seq_begin = p.cu[seq];
                seq_len = (int64_t)p.cu[seq + 1] - seq_begin;
            } else {
                seq_len = p.total_tokens / (p.n_seqs / Q);
                seq_begin = seq * seq_len;
            }
            int64_t b, len;
            seg_bounds(seq_len, Q, s, b, len);
            const int64_t sb = (seq * H + h) * DD;                      // [N, H, D, D]
            const auto slot = [&](int k) { return ((seq * (Q + 1) + k) * H + h) * DD; };
            if constexpr (KIND == kWsSegFirst) {
                if (s == 0)
                    ws_chain<D, true, false>(p, sm, w, lane, h, seq_begin + b, len,
                                             p.init ? p.init + sb : nullptr, p.st + slot(1), nullptr);
                else
                    ws_chain<D, false, true>(p, sm, w, lane, h, seq_begin + b, len, nullptr,
                                             p.fin + slot(s), p.fin2 + slot(s));
            } else {
                ws_chain<D, true, false>(p, sm, w, lane, h, seq_begin + b, len, p.st + slot(s),
                                         (s == Q && p.fin) ? p.fin + sb : nullptr, nullptr);
            }
        }
    }
}

// Whether the launcher takes the specialised-wave kernel.
template <int D>
constexpr bool kSpecialised = D == 128;

// Largest number of sequences the order kernel sorts (in LDS); past it the
// chains go in their natural order.
constexpr int kOrderSortMax = 2048;

// Zeroes the chain counter (and a second one when not null) and writes the
// sequences in order of decreasing length (ties by index): a bitonic sort of
// (length, index) keys in LDS by one workgroup of 1024 threads, two keys each.
__global__ __launch_bounds__(1024) void chain_order_kernel(const int32_t* __restrict__ cu,
                                                           int32_t n_seqs,
                                                           int32_t* __restrict__ order,
                                                           int32_t* __restrict__ counter,
                                                           int32_t* __restrict__ counter2) {
    __shared__ uint64_t key[kOrderSortMax];
    const int t = threadIdx.x;
    if (t == 0) *counter = 0;
    if (t == 1 && counter2) *counter2 = 0;
    if (!cu || n_seqs > kOrderSortMax) {
        for (int i = t; i < n_seqs; i += 1024) order[i] = i;
        return;
    }
    // ascending keys: (0xffffffff - length) << 32 | index; padding sorts last
    for (int i = t; i < kOrderSortMax; i += 1024) {
        uint64_t k = ~0ull;
        if (i < n_seqs) {
            const uint32_t len = (uint32_t)(cu[i + 1] - cu[i]);
            k = ((uint64_t)(0xffffffffu - len) << 32) | (uint32_t)i;
        }
        key[i] = k;
    }
    __syncthreads();
    for (int size = 2; size <= kOrderSortMax; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = t; i < kOrderSortMax; i += 1024) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool up = (i & size) == 0;
                    const uint64_t a = key[i], c = key[j];
                    if ((a > c) == up) {
                        key[i] = c;
                        key[j] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    for (int i = t; i < n_seqs; i += 1024) order[i] = (int32_t)(key[i] & 0xffffffffu);
}

// Composition of the segments' state maps (segmented prefill).  A segment p
// of a sequence maps its start state to its end state as S_end = M_p S_start +
// b_p (the recurrence is affine in the state, linear in its key rows); M_p is
// the segment run from the identity with V = 0, b_p the segment run from the
// zero state.  One workgroup per (16-column tile, head, sequence), the eight
// tiles of a (sequence, head) on one XCD so that they read M_p from one L2
// (workgroup b: chain 8 (b / 64) + b % 8, tile (b / 8) % 8), walks
// segments p0 .. p0 + cnt - 1 in order, S <- M_p S + b_p from the state
// `init` (zero when null), storing the state before each segment to `start`
// and the one after the last to `fin` (when not null).  Maps and starts are
// [sequence * slots + p][H][D][D] fp32; init and fin hold a [H][D][D] block
// every init_stride and fin_stride elements.
//
// Each step is a 128 x 128 by 128 x 16 product on fp32 MFMA (16x16x4): wave w
// takes rows 32 w .. 32 w + 31 (two row tiles); lane (r, kg) = (lane % 16,
// lane / 16) feeds, at product step 4 i + e, A = M[row r][16 i + 4 kg + e]
// and B = S[16 i + 4 kg + e][column r], so the 32 steps cover every k.  The tile's state
// sits transposed in LDS (St[column][k]) for the B operands; the A operands
// of the next segment's M, and its b, are loaded while the current one is
// multiplied.  The summation order is fixed, so the result does not depend
// on the launch.
template <int D>
__global__ __launch_bounds__(256) void segment_scan_kernel(
    const float* __restrict__ init, int64_t init_stride, const float* __restrict__ Mm,
    const float* __restrict__ bm, float* __restrict__ start, float* __restrict__ fin,
    int64_t fin_stride, int32_t n_seqs, int32_t H, int32_t slots, int32_t p0, int32_t cnt) {
    static_assert(D == 128, "four waves of two 16-row tiles; eight column tiles");
    constexpr int SP = D + 4;  // row pitch of the transposed tile (floats)
    __shared__ __align__(16) float St[16][SP];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, r = lane & 15, kg = lane >> 4;
    const int64_t b = blockIdx.x;
    const int64_t chain = 8 * (b / 64) + b % 8;
    if (chain >= (int64_t)n_seqs * H) return;  // (the whole workgroup: no barrier is skipped)
    const int64_t n = chain / H, h = chain % H;
    const int col0 = 16 * (int)((b / 8) % 8);
    // this lane's output elements: rows 32 w + 16 j + 4 kg + v, column col0 + r
    const auto out_off = [&](int j, int v) { return (int64_t)(32 * w + 16 * j + 4 * kg + v) * D + col0 + r; };
    const auto map_base = [&](int p) { return ((n * slots + p) * H + h) * D * D; };
    f32x4 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[j][v] = init ? init[n * init_stride + h * D * D + out_off(j, v)] : 0.f;
    // A operands of segment p: M_p[32 w + 16 j + r][16 i + 4 kg .. 16 i + 4 kg + 3]
    // for i = 0..7 (the four lanes of a row read 64 contiguous bytes per load),
    // and this lane's elements of b_p
    const auto load_m = [&](int p, float4 (&m)[2][8], f32x4 (&bb)[2]) {
        const float* base = Mm + map_base(p);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float4* row = reinterpret_cast<const float4*>(base + (int64_t)(32 * w + 16 * j + r) * D);
#pragma unroll
            for (int i = 0; i < 8; ++i) m[j][i] = row[4 * i + kg];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) bb[j][v] = bm[map_base(p) + out_off(j, v)];
    };
    // segment p with its operands in (m, bb), the next segment's loaded into
    // (mn, bn) meanwhile; the two sets alternate, so no loaded value is
    // copied (a copy would wait for the load in the middle of the products)
    const auto step = [&](int p, const float4 (&m)[2][8], const f32x4 (&bb)[2], float4 (&mn)[2][8],
                          f32x4 (&bn)[2]) {
        const int64_t mb = map_base(p);
        // the state before segment p: to `start`, and transposed into LDS
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int v = 0; v < 4; ++v) start[mb + out_off(j, v)] = acc[j][v];
            *reinterpret_cast<f32x4*>(&St[r][32 * w + 16 * j + 4 * kg]) = acc[j];
        }
        if (p + 1 < p0 + cnt) load_m(p + 1, mn, bn);
        __syncthreads();
        // B operands: S[16 i + 4 kg .. 16 i + 4 kg + 3][column r]
        float4 Sb[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) Sb[i] = *reinterpret_cast<const float4*>(&St[r][16 * i + 4 * kg]);
        __syncthreads();  // every wave has its B operands; St is free for the next step
        // four independent accumulators per row tile (accumulator q takes the
        // k of steps i = 2 q and 2 q + 1), so the products do not wait on one
        // another; summed in a fixed order
        f32x4 c[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) c[j][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4& cq = c[j][i / 2];
                cq = __builtin_amdgcn_mfma_f32_16x16x4f32(m[j][i].x, Sb[i].x, cq, 0, 0, 0);
                cq = __builtin_amdgcn_mfma_f32_16x16x4f32(m[j][i].y, Sb[i].y, cq, 0, 0, 0);
                cq = __builtin_amdgcn_mfma_f32_16x16x4f32(m[j][i].z, Sb[i].z, cq, 0, 0, 0);
                cq = __builtin_amdgcn_mfma_f32_16x16x4f32(m[j][i].w, Sb[i].w, cq, 0, 0, 0);
            }
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = bb[j] + ((c[j][0] + c[j][1]) + (c[j][2] + c[j][3]));
    };
    float4 Ma[2][8], Mb[2][8];
    f32x4 ba[2], bb2[2];
    if (cnt > 0) load_m(p0, Ma, ba);
    int p = p0;
    for (; p + 1 < p0 + cnt; p += 2) {
        step(p, Ma, ba, Mb, bb2);
        step(p + 1, Mb, bb2, Ma, ba);
    }
    if (p < p0 + cnt) step(p, Ma, ba, Mb, bb2);
    if (fin) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) fin[n * fin_stride + h * D * D + out_off(j, v)] = acc[j][v];
    }
}

// Resident workgroups per CU of the fused kernel for D (queried once per process; the
// answer depends only on the kernel's resources and the gfx950 CU).
template <int D>
hipError_t fused_blocks_per_cu(int* out) {
    static std::atomic<int> cached{0};
    int c = cached.load(std::memory_order_relaxed);
    if (c <= 0) {
        hipError_t e;
        if constexpr (kSpecialised<D>)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, fused_ws_kernel<D, kWsPlain>,
                                                             64 * (kWsPrep<D> + kWsRec<D>), 0);
        else
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, fused_kernel<D>, D * 4, 0);
        if (e != hipSuccess) return e;
        if (c <= 0) c = 1;
        cached.store(c, std::memory_order_relaxed);
    }
    *out = c;
    return hipSuccess;
}

}  // namespace

template <int D>
hipError_t launch_fused(const PrefillArgs& a, hipStream_t stream) {
    if (!a.bf16 || a.d != D) return hipErrorInvalidValue;
    FusedParams fp;
    fp.q = static_cast<const bf16*>(a.q);
    fp.k = static_cast<const bf16*>(a.k);
    fp.v = static_cast<const bf16*>(a.v);
    fp.g = static_cast<const bf16*>(a.g);
    fp.beta = static_cast<const bf16*>(a.beta);
    fp.cu = a.cu_seqlens;
    fp.init = a.initial_state;
    fp.fin = a.final_state;
    fp.out = static_cast<bf16*>(a.out);
    fp.total_tokens = a.total_tokens;
    fp.n_seqs = a.n_seqs;
    fp.n_heads = a.n_heads;
    fp.scale = a.scale;
    fp.l2norm = a.l2norm;
    // the chain counter and the order live in the workspace's two index areas
    int32_t* order = reinterpret_cast<int32_t*>(a.workspace + a.layout.ckidx_offset());
    fp.counter = reinterpret_cast<int32_t*>(a.workspace);
    fp.order = a.cu_seqlens ? order : nullptr;
    hipLaunchKernelGGL(chain_order_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens,
                       a.n_seqs, order, fp.counter, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int per_cu = 1;
    if ((e = fused_blocks_per_cu<D>(&per_cu)) != hipSuccess) return e;
    const int64_t chains = (int64_t)a.n_seqs * a.n_heads;
    const int64_t cus = a.compute_units > 0 ? a.compute_units : 256;
    const int grid = (int)std::min<int64_t>(chains, cus * per_cu);
    if constexpr (kSpecialised<D>)
        hipLaunchKernelGGL((fused_ws_kernel<D, kWsPlain>), dim3(grid), dim3(64 * (kWsPrep<D> + kWsRec<D>)), 0,
                           stream, fp);
    else
        hipLaunchKernelGGL((fused_kernel<D>), dim3(grid), dim3(D * 4), 0, stream, fp);
    return hipGetLastError();
}

template hipError_t launch_fused<128>(const PrefillArgs&, hipStream_t);
template hipError_t launch_fused<64>(const PrefillArgs&, hipStream_t);

size_t segmented_scratch_bytes(const PrefillArgs& a, int P) {
    // b, M and the start states of P + 1 segments per sequence and head
    return 3 * (size_t)a.n_seqs * (P + 1) * a.n_heads * a.d * a.d * sizeof(float);
}

hipError_t launch_segmented(const PrefillArgs& a, int P, hipStream_t stream) {
    constexpr int D = 128;
    if (!a.bf16 || a.d != D || P < 2) return hipErrorInvalidValue;
    const int64_t N = a.n_seqs, H = a.n_heads;
    // P chains per sequence and head in each pass, P + 1 segments (placed by
    // seg_bounds in the kernel, from each sequence's length)
    const int64_t slots = P + 1;
    const size_t map_elems = (size_t)N * slots * H * D * D;
    float* Mm = reinterpret_cast<float*>(a.workspace + a.layout.records_offset());
    float* bm = Mm + map_elems;
    float* st = bm + map_elems;
    FusedParams fp;
    fp.q = static_cast<const bf16*>(a.q);
    fp.k = static_cast<const bf16*>(a.k);
    fp.v = static_cast<const bf16*>(a.v);
    fp.g = static_cast<const bf16*>(a.g);
    fp.beta = static_cast<const bf16*>(a.beta);
    fp.cu = a.cu_seqlens;
    fp.order = nullptr;
    fp.total_tokens = a.total_tokens;
    fp.n_seqs = (int32_t)(N * P);
    fp.n_heads = (int32_t)H;
    fp.scale = a.scale;
    fp.l2norm = a.l2norm;
    fp.seg_per_seq = P;
    fp.st = st;
    fp.out = static_cast<bf16*>(a.out);
    int per_cu = 1;
    hipError_t e = fused_blocks_per_cu<D>(&per_cu);
    if (e != hipSuccess) return e;
    const int64_t cus = a.compute_units > 0 ? a.compute_units : 256;
    const int grid = (int)std::min<int64_t>(N * P * H, cus * per_cu);
    const dim3 block(64 * (kWsPrep<D> + kWsRec<D>));
    // one chain counter per pass (the first two ints of the index area),
    // both zeroed by one launch
    int32_t* const counters = reinterpret_cast<int32_t*>(a.workspace);
    hipLaunchKernelGGL(chain_order_kernel, dim3(1), dim3(1024), 0, stream, nullptr, 0, nullptr,
                       counters, counters + 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // segment 0 with its outputs, from the initial state to start slot 1,
    // beside the maps of segments 1..P-1 (b from the zero state, M from the
    // identity with V = 0)
    fp.init = a.initial_state;
    fp.fin = bm;
    fp.fin2 = Mm;
    fp.counter = counters;
    hipLaunchKernelGGL((fused_ws_kernel<D, kWsSegFirst>), dim3(grid), block, 0, stream, fp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // the start states of segments 2..P from that of segment 1
    const int64_t scan_blocks = 64 * ((N * H + 7) / 8);
    hipLaunchKernelGGL((segment_scan_kernel<D>), dim3((unsigned)scan_blocks), dim3(256), 0, stream,
                       st + H * D * D, slots * H * D * D, Mm, bm, st, st + P * H * D * D,
                       slots * H * D * D, (int32_t)N, (int32_t)H, (int32_t)slots, 1, P - 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // segments 1..P with their outputs; the last writes the final state
    fp.init = nullptr;
    fp.fin = a.final_state;
    fp.fin2 = nullptr;
    fp.counter = counters + 1;
    hipLaunchKernelGGL((fused_ws_kernel<D, kWsSegOut>), dim3(grid), block, 0, stream, fp);
    return hipGetLastError();
}

}  // namespace kda

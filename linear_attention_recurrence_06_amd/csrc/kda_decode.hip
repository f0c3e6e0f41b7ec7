// KDA decode step on gfx950: one token per sequence, state advanced in place.
//
// Per (sequence, head) the step is, with qb, kb the L2-normalised q, k and
// alpha = exp(g) (retention per key channel, or one value for all channels
// with the per-head gate):
//     S' = Diag(alpha) S;  vh = S'^T kb;  y = S'^T qb       (one pass over S)
//     delta = beta (v - vh);  S = S' + kb delta^T;  o = y + (qb . kb) delta
// The second form of o follows from o = (S' + kb delta^T)^T qb, so the state
// is read once and written once ("Kimi K3: The Manos, The Mythos, The
// Legendos", bullet on decode cost constant in sequence length; the update is
// the delta rule with a diagonal gate of "From KV Cache to Depth Attention:
// The Bottlenecks Kimi K3 Had to Break", Technical Details, KDA bullet).
//
// Work split: one workgroup of NTH threads per (sequence, head) (512; 256 for
// the front-end step at D = 64).  Thread t owns value columns 4*(t % (D/4)) ..
// +3 of rows (t / (D/4)) + (NTH/(D/4)) * m, so each wave reads and writes whole
// 512-byte (D=128) state rows with 16-byte accesses, every lane keeps its
// D*D/NTH state values in registers between the
// read and the write, and the read-outs reduce over row groups with one
// cross-lane step inside the wave and one LDS exchange across the waves.
// The kernel is bound by HBM: 2 * 4 * D*D bytes of state per unit.
#include <algorithm>

#include "kda_common.hpp"
#include "kda_internal.hpp"

namespace kda {

// Front end of one decode step (kernel argument): the short convolution of the
// raw q, k, v against each sequence's conv state, advanced in place, and the
// low-rank decay gate.
struct DecodeFE {
    int conv_w, silu, rank;
    const void* weight;     // [3, H, W, d]
    const void* state_in;   // [N, 3, W-1, H, d] or null (zeros)
    void* state_out;        // [N, 3, W-1, H, d] or null; may equal state_in
    const void* a;          // [N, r]
    const void* b;          // [H, d, r]
    const float* bias;      // [H, d] or null
};

// Front-end operands of N consecutive elements of one tensor of one unit:
// the raw token values, the filter taps aligned to the last four tokens (tap
// jp - (4 - W) of the W; the first 4 - W read zero), and the conv-state rows
// aligned the same way (row jp - (4 - W) of the W - 1; rows that do not exist,
// or all of them without an input state, read zero).  All loads are issued
// together with no branch on their values, so one wait covers them.
template <typename T, int N>
struct FeOps {
    typedef T V __attribute__((ext_vector_type(N)));
    V raw, w[4], hist[3];
};

template <typename T, int D, int N>
__device__ __forceinline__ void fe_load(const DecodeFE& fe, const T* raw, int x, int64_t n, int h,
                                        int H, int i0, FeOps<T, N>& f) {
    typedef typename FeOps<T, N>::V V;
    const uint32_t E = sizeof(T);
    const int W = fe.conv_w;
    // (token rows need only element alignment: one load per element)
#pragma unroll
    for (int c = 0; c < N; ++c) f.raw[c] = raw[i0 + c];
    if (W == 0) return;  // no convolution: the raw values pass through
    const auto rw = make_rsrc(reinterpret_cast<const T*>(fe.weight) + (int64_t)(x * H + h) * W * D,
                              (uint32_t)(W * D) * E);
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) {
        const int tap = jp - (4 - W);
        f.w[jp] = buffer_load<V>(rw, tap < 0 ? kFarOffset : (uint32_t)(tap * D + i0) * E);
    }
    const bool has = fe.state_in != nullptr && W > 1;
    const auto rs = make_rsrc(
        has ? reinterpret_cast<const T*>(fe.state_in) + ((n * 3 + x) * (W - 1) * H + h) * D
            : reinterpret_cast<const T*>(fe.weight),
        has ? (uint32_t)(((W - 2) * H * D + D) * E) : 0u);
#pragma unroll
    for (int jp = 0; jp < 3; ++jp) {
        const int j = jp - (4 - W);
        f.hist[jp] = buffer_load<V>(rs, j < 0 ? kFarOffset : (uint32_t)(j * H * D + i0) * E);
    }
}

// The convolution of the loaded operands (then SiLU if asked), and the conv
// state advanced by one token: row j takes old row j + 1, the last row the raw
// value.  The caller is the only reader and writer of these elements' state,
// and every row was read before any is written, so the state may be advanced
// in place.
template <typename T, int D, int N>
__device__ __forceinline__ void fe_apply(const DecodeFE& fe, const FeOps<T, N>& f, int x, int64_t n,
                                         int h, int H, int i0, float (&y)[N]) {
    typedef typename FeOps<T, N>::V V;
    const int W = fe.conv_w;
    if (W == 0) {
#pragma unroll
        for (int c = 0; c < N; ++c) y[c] = to_f32(f.raw[c]);
        return;
    }
#pragma unroll
    for (int c = 0; c < N; ++c) {
        float acc = to_f32(f.w[3][c]) * to_f32(f.raw[c]);
#pragma unroll
        for (int jp = 0; jp < 3; ++jp) acc += to_f32(f.w[jp][c]) * to_f32(f.hist[jp][c]);
        y[c] = fe.silu ? acc * __builtin_amdgcn_rcpf(1.f + __expf(-acc)) : acc;
    }
    if (fe.state_out) {
        T* so = reinterpret_cast<T*>(fe.state_out) + ((n * 3 + x) * (W - 1) * H + h) * D + i0;
#pragma unroll
        for (int jp = 0; jp < 3; ++jp) {
            const int j = jp - (4 - W);
            if (j >= 0)
                *reinterpret_cast<V*>(so + (int64_t)j * H * D) = jp < 2 ? f.hist[jp + 1] : f.raw;
        }
    }
}

// FE: raw q, k, v go through the front end (and g, unless given, comes from
// the low-rank gate); GR: the largest gate rank the instantiation serves (64
// or 128), which sizes the gate's loads.
template <typename T, int D, bool FE, int GR, int NTH, bool OG>
__global__ __launch_bounds__(NTH) void decode_kernel(const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     const T* __restrict__ g,
                                                     const T* __restrict__ beta,
                                                     float* __restrict__ S,
                                                     T* __restrict__ out, float scale,
                                                     int l2norm, int scalar_g, int out_gate,
                                                     const T* __restrict__ og_z, int H,
                                                     DecodeFE fe) {
    constexpr int TPR = D / 4;       // threads per state row
    constexpr int RG = NTH / TPR;    // row groups
    constexpr int NW = NTH / kWave;  // waves
    constexpr int RPT = D / RG;      // rows per thread
    constexpr int EPL = D / kWave;   // vector elements per lane in the norm pass
    constexpr int TPC = NTH / D;     // gate: threads per channel
    constexpr int NJ = GR / TPC / 8; // gate: fragments per thread
    static_assert(RPT * RG == D && EPL * kWave == D, "bad decode tiling");
    // the gate's per-thread rank slice (rank / TPC, rank >= 32) must be whole fragments
    static_assert(!FE || (32 / TPC) % 8 == 0, "front-end gate slice below one fragment");

    // a 2-D grid (head, sequence): N * H workgroups of NTH threads would pass the
    // 32-bit dispatch size in one dimension
    const int64_t unit = (int64_t)blockIdx.y * H + blockIdx.x;  // = n * H + h
    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;
    const int cq = t % TPR, rg = t / TPR;
    const T* qu = q + unit * D;
    const T* ku = k + unit * D;
    const int64_t n = unit / H;
    const int h = (int)(unit - n * H);

    __shared__ float s_q[D], s_k[D], s_a[D], s_v[FE ? D : 1], s_qk;
    __shared__ float s_red[NW][TPR][8];

    // 0. front end: its operands are requested before the state, so their
    // arithmetic can start while the state streams in.  Wave 0 takes q and k
    // (elements EPL*lane ..), its first TPR lanes (row group 0) v (elements
    // 4*cq ..); every thread loads its share of the gate's products.
    FeOps<T, EPL> fq, fk;
    FeOps<T, 4> fv;
    Frag<T> ga[NJ], gb[NJ];
    float gbias = 0.f;
    if constexpr (FE) {
        if (wave == 0) {
            fe_load<T, D, EPL>(fe, qu, 0, n, h, H, EPL * lane, fq);
            fe_load<T, D, EPL>(fe, ku, 1, n, h, H, EPL * lane, fk);
        }
        if (rg == 0) fe_load<T, D, 4>(fe, v + unit * D, 2, n, h, H, 4 * cq, fv);
        if (fe.rank > 0) {
            // channel c = t / TPC, ranks [part * slice, (part + 1) * slice);
            // fragments past the slice read zero (the resources are uniform over
            // the workgroup: a lane-dependent base would make the compiler loop
            // over the lanes' descriptors)
            const int c = t / TPC, part = t % TPC;
            const int R = fe.rank, slice = R / TPC;
            const uint32_t E = sizeof(T);
            const auto ra = make_rsrc(reinterpret_cast<const T*>(fe.a) + n * R, (uint32_t)R * E);
            const auto rb = make_rsrc(reinterpret_cast<const T*>(fe.b) + (int64_t)h * D * R,
                                      (uint32_t)(D * R) * E);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bool in = 8 * j < slice;
                const uint32_t kk = (uint32_t)(part * slice + 8 * j);
                ga[j] = buffer_load_frag<T>(ra, in ? kk * E : kFarOffset);
                gb[j] = buffer_load_frag<T>(rb, in ? ((uint32_t)c * R + kk) * E : kFarOffset);
            }
            if (fe.bias) gbias = fe.bias[h * D + c];
        }
    }

    // OG: the output-gate pre-activations of this thread's outputs (row group 0),
    // requested before the state so that their latency hides under its stream
    // (asked for after it, they held each workgroup up by an HBM round trip at
    // its end: 175.5 against 161.6 us per step)
    T zraw[4] = {};
    if constexpr (OG) {
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) zraw[j] = out_gate == 2 ? og_z[unit] : og_z[unit * D + 4 * cq + j];
        }
    }

    // 1. stream the state in (all loads in flight before any arithmetic on it).
    // Ordinary loads, non-temporal stores: measured 11% faster than with
    // non-temporal loads as well
    float* Su = S + unit * (int64_t)(D * D);
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = *reinterpret_cast<const f32x4*>(Su + (int64_t)(rg + RG * m) * D + 4 * cq);

    // 2. token vectors
    const float b = to_f32(beta[unit]);
    float qk, vj[4];
    if constexpr (FE) {
        if (wave == 0) {
            float qv[EPL], kv[EPL];
            fe_apply<T, D, EPL>(fe, fq, 0, n, h, H, EPL * lane, qv);
            fe_apply<T, D, EPL>(fe, fk, 1, n, h, H, EPL * lane, kv);
            float ssq = 0.f, ssk = 0.f, sqk = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                ssq += qv[e] * qv[e];
                ssk += kv[e] * kv[e];
                sqk += qv[e] * kv[e];
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                ssq += xor_shfl(ssq, m);
                ssk += xor_shfl(ssk, m);
                sqk += xor_shfl(sqk, m);
            }
            const float rq = l2norm ? 1.0f / sqrtf(ssq + kL2Eps) : 1.0f;
            const float rk = l2norm ? 1.0f / sqrtf(ssk + kL2Eps) : 1.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int i = EPL * lane + e;
                s_q[i] = qv[e] * rq * scale;
                s_k[i] = kv[e] * rk;
            }
            if (lane == 0) s_qk = sqk * rq * rk * scale;
        }
        if (rg == 0) {
            float vv[4];
            fe_apply<T, D, 4>(fe, fv, 2, n, h, H, 4 * cq, vv);
#pragma unroll
            for (int j = 0; j < 4; ++j) s_v[4 * cq + j] = vv[j];
        }
        if (fe.rank > 0) {
            // low-rank decay gate g = -softplus(a[n] . b[h][c] + bias[h][c]): the
            // TPC threads of channel c sum their slices with lane swaps
            const int c = t / TPC, part = t % TPC;
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int m = 0; m < 8; ++m) z += to_f32(ga[j].v[m]) * to_f32(gb[j].v[m]);
#pragma unroll
            for (int off = 1; off < TPC; off <<= 1) z += xor_shfl(z, off);
            if (part == 0) {
                z += gbias;
                s_a[c] = __expf(-(fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)))));
            }
        } else if (wave == 0) {
            // g given: read last, since waiting on it also waits for the state
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int i = EPL * lane + e;
                s_a[i] = __expf(to_f32(scalar_g ? g[unit] : g[unit * D + i]));
            }
        }
        __syncthreads();
        qk = s_qk;
#pragma unroll
        for (int j = 0; j < 4; ++j) vj[j] = s_v[4 * cq + j];
    } else {
        // every wave computes the norms itself (no barrier needed for them)
        float qv[EPL], kv[EPL];
        float ssq = 0.f, ssk = 0.f, sqk = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            qv[e] = to_f32(qu[lane + kWave * e]);
            kv[e] = to_f32(ku[lane + kWave * e]);
            ssq += qv[e] * qv[e];
            ssk += kv[e] * kv[e];
            sqk += qv[e] * kv[e];
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            ssq += xor_shfl(ssq, m);
            ssk += xor_shfl(ssk, m);
            sqk += xor_shfl(sqk, m);
        }
        const float rq = l2norm ? 1.0f / sqrtf(ssq + kL2Eps) : 1.0f;
        const float rk = l2norm ? 1.0f / sqrtf(ssk + kL2Eps) : 1.0f;
        qk = sqk * rq * rk * scale;   // (scale * qb) . kb
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int i = lane + kWave * e;
                s_q[i] = qv[e] * rq * scale;
                s_k[i] = kv[e] * rk;
                s_a[i] = __expf(to_f32(scalar_g ? g[unit] : g[unit * D + i]));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) vj[j] = to_f32(v[unit * D + 4 * cq + j]);
        __syncthreads();
    }

    // 3. decay the rows and accumulate both read-outs
    f32x4 vh = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        s[m] *= s_a[i];
        vh += s_k[i] * s[m];
        y += s_q[i] * s[m];
    }
    // 4. reduce over the row groups: inside the wave, then across waves
#pragma unroll
    for (int off = TPR; off < kWave; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vh[j] += xor_shfl(vh[j], off);
            y[j] += xor_shfl(y[j], off);
        }
    }
    if (lane < TPR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_red[wave][cq][j] = vh[j];
            s_red[wave][cq][4 + j] = y[j];
        }
    }
    __syncthreads();
    float d[4], o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float vhat = 0.f, yy = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) {
            vhat += s_red[w2][cq][j];
            yy += s_red[w2][cq][4 + j];
        }
        d[j] = b * (vj[j] - vhat);
        o[j] = yy + qk * d[j];
    }
    // 5. write the difference and stream the state out
    const f32x4 dv = {d[0], d[1], d[2], d[3]};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        s[m] += s_k[i] * dv;
        __builtin_nontemporal_store(
            s[m], reinterpret_cast<f32x4*>(Su + (int64_t)(rg + RG * m) * D + 4 * cq));
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float oj = o[j];
            if constexpr (OG) {  // out = o * sigmoid(z), z per value channel or per head
                const float zz = to_f32(zraw[j]);
                oj *= __builtin_amdgcn_rcpf(1.f + __expf(-zz));
            }
            out[unit * D + 4 * cq + j] = from_f32<T>(oj);
        }
    }
}

// Threads per (sequence, head) workgroup.  The plain step: eight waves, each
// lane holding D*D/512 state values (32 at D = 128); measured 163 us per step
// against 167.5 us with four waves, on 256 sequences x 32 heads.  The
// front-end step: eight waves at D = 128 (rank 128: 193 against 206 us; rank
// 64: no change), four at D = 64, because its gate gives each of the NTH/D
// threads of a channel a whole number of 8-rank fragments only when
// NTH/D <= 32/8 at every rank (32 and up).
constexpr int kDecodeThreads = 512;
template <int D>
constexpr int kDecodeThreadsFE = D == 128 ? 512 : 256;

template <typename T, int D, bool FE, int GR, int NTH>
static hipError_t launch_one(const DecodeArgs& a, const DecodeFE& fe, hipStream_t stream) {
    // grid (head, sequence), at most kMaxGridY sequences per launch
    const int64_t H = a.n_heads;
    for (int64_t n0 = 0; n0 < a.n_seqs; n0 += kMaxGridY) {
        const dim3 grid((unsigned)H, (unsigned)std::min<int64_t>(kMaxGridY, a.n_seqs - n0));
        const int64_t th = n0 * H, td = th * D;  // token-head and element offsets
        DecodeFE f = fe;
        if (f.a) f.a = (const T*)f.a + n0 * f.rank;
        if (f.state_in) f.state_in = (const T*)f.state_in + n0 * 3 * (f.conv_w - 1) * H * D;
        if (f.state_out) f.state_out = (T*)f.state_out + n0 * 3 * (f.conv_w - 1) * H * D;
        const T* g = (const T*)a.g + (a.g ? (a.scalar_g ? th : td) : 0);
        const T* z = (const T*)a.out_gate_z + (a.out_gate_z ? (a.out_gate == 2 ? th : td) : 0);
        if (a.out_gate)
            hipLaunchKernelGGL((decode_kernel<T, D, FE, GR, NTH, true>), grid, dim3(NTH), 0, stream,
                               (const T*)a.q + td, (const T*)a.k + td, (const T*)a.v + td, g,
                               (const T*)a.beta + th, a.state + td * D, (T*)a.out + td, a.scale,
                               a.l2norm, a.scalar_g ? 1 : 0, a.out_gate, z, a.n_heads, f);
        else
            hipLaunchKernelGGL((decode_kernel<T, D, FE, GR, NTH, false>), grid, dim3(NTH), 0, stream,
                               (const T*)a.q + td, (const T*)a.k + td, (const T*)a.v + td, g,
                               (const T*)a.beta + th, a.state + td * D, (T*)a.out + td, a.scale,
                               a.l2norm, a.scalar_g ? 1 : 0, a.out_gate, z, a.n_heads, f);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int D>
static hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    const int64_t units = (int64_t)a.n_seqs * a.n_heads;
    if (units == 0) return hipSuccess;
    DecodeFE fe{a.fe.conv_w, a.fe.silu,     a.fe.rank,  a.fe.conv_weight, a.fe.state_in,
                a.fe.state_out, a.fe.gate_a, a.fe.gate_b, a.fe.gate_bias};
    if (a.fe.active() && a.fe.rank > 64)
        return launch_one<T, D, true, 128, kDecodeThreadsFE<D>>(a, fe, stream);
    if (a.fe.active())
        return launch_one<T, D, true, 64, kDecodeThreadsFE<D>>(a, fe, stream);
    return launch_one<T, D, false, 64, kDecodeThreads>(a, fe, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.bf16) {
        return a.d == 128 ? launch<bf16, 128>(a, stream) : launch<bf16, 64>(a, stream);
    }
    return a.d == 128 ? launch<float, 128>(a, stream) : launch<float, 64>(a, stream);
}

}  // namespace kda

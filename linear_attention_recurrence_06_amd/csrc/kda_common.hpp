// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// Element types: bf16 I/O uses clang's __bf16 (float -> bf16 lowers to the
// hardware round-to-nearest-even v_cvt_pk_bf16_f32 on gfx950); fp32 I/O uses
// float.  Matrix products use the 16x16 MFMA family with fp32 accumulators:
//   bf16: v_mfma_f32_16x16x32_bf16, one instruction per 32-deep step;
//   fp32: v_mfma_f32_16x16x4_f32, eight instructions per 32-deep step.
//
// Fragment conventions (one wave64, a 16x16 output tile):
//   A operand (16 rows x 32 k): lane l holds row (l % 16), k = 8*(l/16) + j, j = 0..7
//   B operand (32 k x 16 cols): lane l holds col (l % 16), k = 8*(l/16) + j
//   C/D accumulator (16 x 16):  lane l holds col (l % 16), rows 4*(l/16) + i, i = 0..3
// A and B assign k to (lane group, element) identically, which is all the sum
// over k needs.  The D layout is the documented one for the 16x16 family and
// is checked on the device by the test suite.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kChunk = 64;   // tokens per chunk
constexpr int kSub = 16;     // rows per MFMA tile / decay sub-block

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Two floats as one word of two bf16 (one packed conversion; element-wise
// conversions into a vector can become single conversions and permutes).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
template <typename T> struct Vec4 { typedef T type __attribute__((ext_vector_type(4))); };
// Four floats as a 4-vector of T (bf16: two packed conversions).
template <typename T>
__device__ __forceinline__ typename Vec4<T>::type from_f32x4(const f32x4& x) {
    if constexpr (sizeof(T) == 2)
        return __builtin_bit_cast(typename Vec4<T>::type, u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])});
    else
        return x;
}

// ---------------------------------------------------------------- 8-element vectors
// Frag<T>: 8 consecutive elements of T held by one lane (16 B for bf16, 32 B for fp32).
template <typename T> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
};
template <> struct Frag<float> {
    f32x8 v;
};

template <typename T>
__device__ __forceinline__ Frag<T> load_frag(const T* p);
template <>
__device__ __forceinline__ Frag<bf16> load_frag<bf16>(const bf16* p) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
}
template <>
__device__ __forceinline__ Frag<float> load_frag<float>(const float* p) {
    Frag<float> f;
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = q[0], b = q[1];
    f.v = f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

template <typename T>
__device__ __forceinline__ void store_frag(T* p, const Frag<T>& f);
template <>
__device__ __forceinline__ void store_frag<bf16>(bf16* p, const Frag<bf16>& f) {
    *reinterpret_cast<bf16x8*>(p) = f.v;
}
template <>
__device__ __forceinline__ void store_frag<float>(float* p, const Frag<float>& f) {
    f32x4* q = reinterpret_cast<f32x4*>(p);
    q[0] = f32x4{f.v[0], f.v[1], f.v[2], f.v[3]};
    q[1] = f32x4{f.v[4], f.v[5], f.v[6], f.v[7]};
}

// Build a fragment from 8 fp32 values (rounding once to T).
template <typename T>
__device__ __forceinline__ Frag<T> make_frag(const float (&x)[8]) {
    Frag<T> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = from_f32<T>(x[j]);
    return f;
}

// Read 8 consecutive T as fp32.
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&x)[8]) {
    Frag<T> f = load_frag<T>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = to_f32(f.v[j]);
}

// ---------------------------------------------------------------- MFMA
// acc += A(16x32) * B(32x16) with the fragment conventions above.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float xor_shfl(float x, int m) { return __shfl_xor(x, m, kWave); }

// DPP move within each 16-lane row (ctrl: quad_perm 0x00-0xff, row_ror:n = 0x120 + n).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of each DPP row, result in every lane of the row.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x124>(x);  // row_ror:4
    x += dpp<0x128>(x);  // row_ror:8
    return x;
}

// ---------------------------------------------------------------- buffer access
// Raw buffer resource over [base, base + bytes): the hardware range check makes
// a load at a byte offset at or past `bytes` return zeros (no memory access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Load a V (8, 16 or 32 bytes, or one 2- or 4-byte element) at byte offset `off`
// (32 bytes: two 16-byte loads).
template <typename V>
__device__ __forceinline__ V buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (sizeof(V) == 32) {
        struct Pair {
            u32x4 lo, hi;
        };
        const Pair x{__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0)),
                     __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, 0))};
        return __builtin_bit_cast(V, x);
    } else if constexpr (sizeof(V) == 16) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    } else if constexpr (sizeof(V) == 8) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    } else if constexpr (sizeof(V) == 4) {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    } else {
        static_assert(sizeof(V) == 2, "buffer_load: 2, 4, 8 or 16 bytes");
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
    }
}

// A buffer offset past every range used here (and far from wrapping), for
// loads that must read zero.
constexpr uint32_t kFarOffset = 0x80000000u;

// Fragment (8 consecutive elements) at byte offset `off` of a buffer; past the
// range it reads zeros.
template <typename T>
__device__ __forceinline__ Frag<T> buffer_load_frag(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        f.v = buffer_load<bf16x8>(r, off);
    } else {
        const f32x4 lo = buffer_load<f32x4>(r, off), hi = buffer_load<f32x4>(r, off + 16);
        f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return f;
}

// 2^x on the hardware exponential unit.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Fragment-ordered storage ("A order"): a rows x kdim matrix stored as 16x32
// tiles, each tile as 64 lanes x 8 elements in A-operand lane order, so one
// wave loads a whole MFMA operand with one contiguous 16-byte (bf16) or
// 32-byte (fp32) access per lane.
__device__ __forceinline__ int64_t aorder_index(int row, int col, int kdim) {
    const int rb = row >> 4, ks = col >> 5;
    const int lane = (row & 15) + 16 * ((col & 31) >> 3);
    return ((int64_t)(rb * (kdim >> 5) + ks) * kWave + lane) * 8 + (col & 7);
}

// Accumulator-ordered storage ("C order") of a rows x ncols matrix: 16x16 tiles,
// each as 64 lanes x 4 elements in accumulator lane order.
__device__ __forceinline__ int64_t corder_index(int row, int col, int ncols) {
    const int rb = row >> 4, nb = col >> 4;
    const int lane = (col & 15) + 16 * ((row & 15) >> 2);
    return ((int64_t)(rb * (ncols >> 4) + nb) * kWave + lane) * 4 + (row & 3);
}

}  // namespace kda

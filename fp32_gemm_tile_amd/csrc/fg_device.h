// Device-side helpers shared by the GEMM kernels: buffer resources, guarded
// loads/stores, and the workgroup-to-tile mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fg_kernels.h"

namespace fg {

typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format,
// no swizzle, no stride).
constexpr int32_t kBufferWord3 = 0x00020000;

// A raw buffer over [base, base + bytes) of any element type (clamped as
// make_rsrc below).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_bytes(const void* base,
                                                                  int64_t bytes) {
    if (bytes < 0) bytes = 0;
    if (bytes > 0xFFFFFFFFll) bytes = 0xFFFFFFFFll;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(uint32_t)bytes, kBufferWord3);
}

// A raw buffer over [base, base + records_bytes). Loads whose byte offset is
// at or past the end return 0 and stores there are dropped by the hardware;
// the kernels still predicate every access themselves, so this is only a
// safety net that keeps any index error inside the caller's matrix.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base,
                                                            int64_t extent_floats) {
    int64_t bytes = extent_floats * 4;
    if (bytes < 0) bytes = 0;
    if (bytes > 0xFFFFFFFFll) bytes = 0xFFFFFFFFll;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0,
                                             (int)(uint32_t)bytes, kBufferWord3);
}

__device__ __forceinline__ f4 ld4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ float ld1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
__device__ __forceinline__ void st4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}
// 128-bit store with the non-temporal cache hint (nt): results of a GEMM are
// written once and not read again by the kernel.
__device__ __forceinline__ void st4_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 2);
}
__device__ __forceinline__ void st1(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 0);
}
__device__ __forceinline__ f2 ld2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
}
__device__ __forceinline__ void st2_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 2);
}
__device__ __forceinline__ void st2(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}

// Four consecutive floats starting at element `e` of a row whose valid length
// is `len` (elements at or past `len` read as 0). `off` is the byte offset of
// element e. vec: the row start and e are 16-byte aligned, so a 128-bit load
// is allowed when all four are in range.
__device__ __forceinline__ f4 ld4_guard(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                        int e, int len, bool vec) {
    f4 v = {0.f, 0.f, 0.f, 0.f};
    if (vec && e + 3 < len) return ld4(r, off);
    if (e + 0 < len) v[0] = ld1(r, off);
    if (e + 1 < len) v[1] = ld1(r, off + 4);
    if (e + 2 < len) v[2] = ld1(r, off + 8);
    if (e + 3 < len) v[3] = ld1(r, off + 12);
    return v;
}

// Barrier after this wave's LDS writes have completed, without the memory
// fence of __syncthreads() (which would also wait for every outstanding global
// load). gfx9 s_waitcnt encoding: lgkmcnt = 0, vmcnt and expcnt at maximum.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
}

// erf(x) for binary32, branch free: formula 7.1.26 of Abramowitz and Stegun,
// "Handbook of Mathematical Functions" (after Hastings),
//     erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//     t = 1 / (1 + p z),  z >= 0,
// whose absolute error is at most 1.5e-7, applied to |x| with the sign put
// back (erf is odd). With the binary32 rounding of these few operations the
// result stays within about 4e-7 of erf(x). The library erff branches on the
// size of |x|, which diverges across a wavefront in an epilogue.
__device__ __forceinline__ float erf_as7126(float x) {
    const float z = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.f));
    float poly = fmaf(t, 1.061405429f, -1.453152027f);
    poly = fmaf(t, poly, 1.421413741f);
    poly = fmaf(t, poly, -0.284496736f);
    poly = fmaf(t, poly, 0.254829592f);
    poly *= t;
    const float e = 1.f - poly * __expf(-z * z);
    return copysignf(e, x);
}

// Fused-epilogue activation in binary32. relu keeps NaN (x < 0 is false for
// it); gelu is the erf form x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2; silu is
// x * sigma(x) = x / (1 + exp(-x)), which tends to -0 for very negative x (exp
// overflows to inf and its reciprocal is 0). Hardware reciprocal and exp2
// (about 1 ulp each) keep both short and branch free.
template <int ACT>
__device__ __forceinline__ float activate_t(float x) {
    if constexpr (ACT == ACT_RELU) return x < 0.f ? 0.f : x;
    else if constexpr (ACT == ACT_GELU)
        return 0.5f * x * (1.f + erf_as7126(x * 0.70710678118654752f));
    else if constexpr (ACT == ACT_SILU) return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
    else return x;
}

// The same with the activation chosen at run time (per element).
__device__ __forceinline__ float activate(float x, int act) {
    if (act == ACT_RELU) return activate_t<ACT_RELU>(x);
    if (act == ACT_GELU) return activate_t<ACT_GELU>(x);
    if (act == ACT_SILU) return activate_t<ACT_SILU>(x);
    return x;
}

// Compile-time activation tag, for code that picks the activation once and
// runs a loop specialised for it.
template <int A>
struct ActTag {
    static constexpr int value = A;
};

// Scale factor alpha * r_i * c_j of element (i, j) under FLAG_EPI.
__device__ __forceinline__ float epi_scale(const GemmParams& p, int64_t i, int64_t j) {
    float s = p.alpha;
    if (p.row_scale) s *= p.row_scale[i];
    if (p.col_scale) s *= p.col_scale[j];
    return s;
}

// act(o + u_i + w_j) of element (i, j) under FLAG_EPI.
__device__ __forceinline__ float epi_finish(const GemmParams& p, float o, int64_t i, int64_t j) {
    if (p.row_bias) o += p.row_bias[i];
    if (p.col_bias) o += p.col_bias[j];
    return activate(o, p.act);
}

// Quantised codes of a final binary32 value (the formats of fg_quant):
//   bf16: the bfloat16 nearest to x, ties to even, computed on the bit
//         pattern (adding 0x7FFF plus the kept half's lowest bit carries into
//         the upper half exactly when the dropped half is above the tie, or at
//         it with an odd upper half; infinities stay, overflow carries into
//         the exponent and gives infinity); every NaN becomes 0x7FC0.
//   int8_row: clamp(round_half_even(x * s), -128, 127) on the binary32
//         product; NaN gives 0.
__device__ __forceinline__ uint32_t bf16_code(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t int8_code(float x, float s) {
    float y = __builtin_rintf(x * s);
    y = (y == y) ? y : 0.f;  // NaN
    y = fminf(fmaxf(y, -128.f), 127.f);
    return (uint32_t)(int32_t)y & 0xFFu;
}
__device__ __forceinline__ uint32_t quant_code(const GemmParams& p, float x, float s) {
    return p.qkind == QUANT_BF16 ? bf16_code(x) : int8_code(x, s);
}

// Q(i, j) of the final value v (plain global store; the callers' i < M,
// j < N keep it inside the caller's Q).
__device__ __forceinline__ void quant_store1(const GemmParams& p, int64_t i, int64_t j, float v) {
    const int64_t e = i * p.ldq + j;
    if (p.qkind == QUANT_BF16)
        static_cast<uint16_t*>(p.qout)[e] = (uint16_t)bf16_code(v);
    else
        static_cast<uint8_t*>(p.qout)[e] = (uint8_t)int8_code(v, p.qscale[i]);
}

// C element (i, j) from its plain product sum `acc` and its old value (read
// only when beta != 0), with or without the fused epilogue; with FLAG_QUANT
// the quantised code of the result is stored to Q(i, j) as well (QUANT: the
// caller's kernel takes quantised calls; the vector-ALU kernel, whose 64
// accumulators per thread went to scratch memory with that code beside its
// stores, does not).
template <bool QUANT = true>
__device__ __forceinline__ float epilogue_value(const GemmParams& p, float acc, float cin,
                                                bool beta0, int64_t i, int64_t j) {
    if (p.flags & FLAG_EPI) {
        float o = epi_scale(p, i, j) * acc;
        if (!beta0) o += p.beta * cin;
        o = epi_finish(p, o, i, j);
        if constexpr (QUANT)
            if (p.flags & FLAG_QUANT) quant_store1(p, i, j, o);
        return o;
    }
    float o = p.alpha * acc;
    if (!beta0) o += p.beta * cin;
    return o;
}

// Tile id -> (tile_m, tile_n) in grouped raster order: tiles are visited in
// bands of `group_m` tile rows, column by column inside a band, so that a run
// of consecutive ids covers a compact block of C (few distinct A row-panels
// and B column-panels).
__device__ __forceinline__ void tile_coords(int L, const GemmParams& p, int& tm, int& tn) {
    const int per_group = p.group_m * p.tiles_n;
    const int g = L / per_group;
    const int first_m = g * p.group_m;
    int gm = p.tiles_m - first_m;
    if (gm > p.group_m) gm = p.group_m;
    const int r = L - g * per_group;
    tm = first_m + r % gm;
    tn = r / gm;
}

// Workgroup id -> tile id (returned) and (tile_m, tile_n).
//
// XCD remap: consecutive workgroup ids are handed to the 8 XCDs in turn, and
// each XCD has its own L2. Renumbering so that XCD x receives the contiguous
// range [x*G/8, (x+1)*G/8) makes the tiles that run together on one XCD
// neighbours in the raster order, so they share operand panels in that XCD's
// L2. A launch covers tile ids [p.tile_base, p.tile_base + nblocks).
__device__ __forceinline__ int map_tile(int bid, int nblocks, const GemmParams& p, int& tm,
                                        int& tn) {
    int L = bid;
    if ((p.flags & FLAG_XCD_REMAP) && (nblocks % 8) == 0)
        L = (bid % 8) * (nblocks / 8) + bid / 8;
    L += p.tile_base;
    tile_coords(L, p, tm, tn);
    return L;
}

}  // namespace fg

// Device helpers shared by the libsanta kernels (gfx950, 64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "santa_internal.h"

namespace santa {
namespace dev {

constexpr int kBlock = 256;            // threads per block of every 256-thread kernel
constexpr int kWaves = kBlock / 64;
constexpr float kNegInfF = -INFINITY;

using bf16_t = uint16_t;               // bfloat16 bit pattern

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

// 16 bytes of cache -> 8 bfloat16 or 4 float32 values, exactly.
__device__ __forceinline__ void unpack(const uint4 v, float *f, bf16_t) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack(const uint4 v, float *f, float) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

template <typename KV> struct KVTraits;
template <> struct KVTraits<bf16_t> { static constexpr int kPerChunk = 8; };
template <> struct KVTraits<float> { static constexpr int kPerChunk = 4; };

__device__ __forceinline__ uint4 ld16(const void *ptr) {
    return *reinterpret_cast<const uint4 *>(ptr);
}

// 16 bytes read once by the whole call (K/V tiles): a non-temporal load
// (streaming cache policy), so the streamed tiles do not push other data out
// of the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *ptr) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(ptr));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// float64 -> bfloat16 in one rounding, ties to even. The spacing of bfloat16
// values near |x| = f 2^e (f in [0.5, 1)) is 2^(e-8), or the subnormal step
// 2^-133 below 2^-126; scaling by it is exact and rint rounds to the nearest
// integer with ties to even.
__device__ __forceinline__ bf16_t f64_to_bf16(double x) {
    if (x != x) return bf16_t(0x7fc0);
    const bf16_t sign = signbit(x) ? bf16_t(0x8000) : bf16_t(0);
    const double ax = fabs(x);
    if (ax == 0.0) return sign;
    int e;
    (void)frexp(ax, &e);
    const int qe = (e - 1 < -126) ? -133 : e - 8;
    const double r = ldexp(rint(ldexp(ax, -qe)), qe);
    if (r > 0x1.fep127) return bf16_t(sign | 0x7f80);
    return bf16_t(sign | (__float_as_uint(float(r)) >> 16));   // r is a bfloat16 value: exact
}

__device__ __forceinline__ void store_rounded(bf16_t *dst, double x) { *dst = f64_to_bf16(x); }
__device__ __forceinline__ void store_rounded(float *dst, double x) { *dst = float(x); }   // IEEE RNE

// Page tile layout of the cache (one tile per (page, KV head), T * d elements).
// A tile is cut into chunks of C = min(T, 32) tokens, C * d elements each.
// Inside a chunk, keys are stored as d / 32 slabs of [C tokens][32 channels]
// and values channel-major as [d][C tokens]. Both offsets are in elements
// from the start of the tile.
__host__ __device__ __forceinline__ int chunk_tokens(int T) { return T < 32 ? T : 32; }
__host__ __device__ __forceinline__ int k_offset(int tok, int ch, int T, int d) {
    const int C = chunk_tokens(T);
    return (tok / C) * (C * d) + (ch >> 5) * (C * 32) + (tok % C) * 32 + (ch & 31);
}
__host__ __device__ __forceinline__ int v_offset(int tok, int ch, int T, int d) {
    const int C = chunk_tokens(T);
    return (tok / C) * (C * d) + ch * C + tok % C;
}

__device__ __forceinline__ int clamp_len(int L, int max_len) {
    return L < 0 ? 0 : (L > max_len ? max_len : L);
}
__device__ __forceinline__ int64_t clamp_page(int32_t pg, int64_t num_pages) {
    return pg < 0 ? 0 : (pg >= num_pages ? num_pages - 1 : int64_t(pg));
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): each round takes the 64-bit products of counter
// words 0 and 2 with two fixed multipliers and forms (hi1 ^ c1 ^ k0, lo1,
// hi0 ^ c3 ^ k1, lo0); the key is bumped by two Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
        const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// Block-wide max of one double per thread (256-thread blocks).
__device__ __forceinline__ double block_max(double v, double *red) {
    for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = red[0];
    for (int i = 1; i < kWaves; ++i) r = fmax(r, red[i]);
    return r;
}

// Exclusive prefix sum of one double per thread, in thread order.
__device__ __forceinline__ double block_exclusive_sum(double v, double *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    double excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    double base = 0.0;
    for (int i = 0; i < wave; ++i) base += red[i];
    return base + excl;
}

inline santa_status launched() {
    return hipGetLastError() == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

}  // namespace dev
}  // namespace santa

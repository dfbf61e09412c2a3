// Canonical fp32 scalar functions for the router, device side.
//
// The router's integer decisions (which k experts a token goes to) are taken
// on fp32 scores, the precision the pages prescribe for the router (CS336
// lecture 4 notes, section 11: router computed in float32).  To make those
// decisions reproducible bit for bit, every score is computed by one fixed
// sequence of IEEE operations:
//   * e^x: Cody-Waite reduction x = n ln2 + r, n = rint(x log2 e), r by two
//     fmas against ln 2 split into a 17-bit head and a tail; e^r by the
//     Taylor series to degree 7 in Horner form; scaling by 2^n through the
//     exponent field; x < -87 gives 0 and x > 88 gives +inf;
//   * ln x: x = m 2^e with m in [sqrt(1/2), sqrt(2)]; ln m = 2 atanh(s),
//     s = (m-1)/(m+1), odd series to s^13 in Horner form in s^2;
//   * ln(1+y): y - y^2/2 below 2^-12, else ln(u) * (y / (u-1)), u = 1+y;
//   * softplus(t) = ln(1+e^t), with t for t > 15 and e^t for t < -15;
//   * sigmoid(z) = 1 / (1 + e^-z);
//   * sin/cos on [0, 2 pi]: quadrant by rint(theta 2/pi), two-fma reduction
//     against split pi/2, Taylor to degree 9 / 8, quadrant rotation;
// all with correctly rounded fp32 division and square root (hipcc's default
// for fp32 '/' and sqrtf) and no fp contraction (this header is compiled
// with -ffp-contract=off; every fma below is explicit).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace canon {

__device__ __forceinline__ float expc(float x) {
    if (x != x) return x;
    if (x > 88.0f) return __builtin_inff();
    if (x < -87.0f) return 0.0f;
    const float n = __builtin_rintf(x * 0x1.715476p+0f);
    float r = __builtin_fmaf(-n, 0x1.62e400p-1f, x);
    r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int ni = (int)n;
    return p * __uint_as_float((uint32_t)(ni + 127) << 23);
}

__device__ __forceinline__ float logc(float x) {
    if (x != x) return x;
    if (x < 0.0f) return __builtin_nanf("");
    if (x == 0.0f) return -__builtin_inff();
    if (x == __builtin_inff()) return x;
    int adj = 0;
    if (x < 0x1p-126f) { x = x * 0x1p+23f; adj = -23; }
    const uint32_t u = __float_as_uint(x);
    int e = (int)(u >> 23) - 127 + adj;
    float m = __uint_as_float((u & 0x007fffffu) | 0x3f800000u);
    if (m > 0x1.6a09e6p+0f) { m = m * 0.5f; e += 1; }
    const float s = (m - 1.0f) / (m + 1.0f);
    const float s2 = s * s;
    float q = 0x1.3b13b2p-4f;
    q = __builtin_fmaf(q, s2, 0x1.745d18p-4f);
    q = __builtin_fmaf(q, s2, 0x1.c71c72p-4f);
    q = __builtin_fmaf(q, s2, 0x1.24924ap-3f);
    q = __builtin_fmaf(q, s2, 0x1.99999ap-3f);
    q = __builtin_fmaf(q, s2, 0x1.555556p-2f);
    q = __builtin_fmaf(q, s2, 1.0f);
    const float lm = (2.0f * s) * q;
    const float ef = (float)e;
    return __builtin_fmaf(ef, 0x1.62e400p-1f, __builtin_fmaf(ef, 0x1.7f7d1cp-20f, lm));
}

__device__ __forceinline__ float log1pc(float y) {
    if (y < 0x1p-12f && y > -0x1p-12f) return __builtin_fmaf(-0.5f * y, y, y);
    const float u = 1.0f + y;
    return logc(u) * (y / (u - 1.0f));
}

__device__ __forceinline__ float softplusc(float t) {
    if (t > 15.0f) return t;
    if (t < -15.0f) return expc(t);
    return log1pc(expc(t));
}

__device__ __forceinline__ float sigmoidc(float z) { return 1.0f / (1.0f + expc(-z)); }

__device__ __forceinline__ void sincosc(float th, float* so, float* co) {
    const float q = __builtin_rintf(th * 0x1.45f306p-1f);
    float r = __builtin_fmaf(-q, 0x1.921fb6p+0f, th);
    r = __builtin_fmaf(-q, -0x1.777a5cp-25f, r);
    const float r2 = r * r;
    float ps = 0x1.71de3ap-19f;
    ps = __builtin_fmaf(ps, r2, -0x1.a01a02p-13f);
    ps = __builtin_fmaf(ps, r2, 0x1.111112p-7f);
    ps = __builtin_fmaf(ps, r2, -0x1.555556p-3f);
    const float sr = __builtin_fmaf(r2 * r, ps, r);
    float pc = 0x1.a01a02p-16f;
    pc = __builtin_fmaf(pc, r2, -0x1.6c16c2p-10f);
    pc = __builtin_fmaf(pc, r2, 0x1.555556p-5f);
    pc = __builtin_fmaf(pc, r2, -0.5f);
    const float cr = __builtin_fmaf(pc, r2, 1.0f);
    switch (((int)q) & 3) {
        case 0: *so = sr; *co = cr; break;
        case 1: *so = cr; *co = -sr; break;
        case 2: *so = -sr; *co = -cr; break;
        default: *so = -cr; *co = sr; break;
    }
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64 multiplies by 0xD2511F53 / 0xCD9E8D57, high halves xored with the
// other counter words and the key, key bumped by 0x9E3779B9 / 0xBB67AE85.
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t lo0 = 0xD2511F53u * c[0];
        const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]);
        const uint32_t lo1 = 0xCD9E8D57u * c[2];
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]);
        const uint32_t n0 = hi1 ^ c[1] ^ k0;
        const uint32_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// Standard normal for flat element i = t*E + e of the noise matrix: one
// Philox block per group of four elements, counter (i>>2, offset), key seed;
// Box-Muller on words (0,1) for elements 0,1 and (2,3) for elements 2,3,
// cosine branch for even elements, sine branch for odd ones.
__device__ __forceinline__ float normalc(uint64_t seed, uint64_t offset, uint64_t i) {
    const uint64_t g = i >> 2;
    uint32_t c[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const int j = (int)(i & 3u);
    const uint32_t w0 = j < 2 ? c[0] : c[2];
    const uint32_t w1 = j < 2 ? c[1] : c[3];
    const float u1 = (float)((w0 >> 8) + 1u) * 0x1p-24f;
    const float u2 = (float)(w1 >> 8) * 0x1p-24f;
    const float rad = __builtin_sqrtf(-2.0f * logc(u1));
    const float th = 0x1.921fb6p+2f * u2;
    float s, co;
    sincosc(th, &s, &co);
    return (j & 1) ? rad * s : rad * co;
}

// Hash-routing key of flat element i = u*E + e (token id u, expert e): the
// top 24 bits of Philox word i & 3 of block (i>>2, offset) under key seed,
// as an exact fp32 integer in [0, 2^24).
__device__ __forceinline__ float hash_keyc(uint64_t seed, uint64_t offset, uint64_t i) {
    const uint64_t g = i >> 2;
    uint32_t c[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const int j = (int)(i & 3u);
    const uint32_t w = j == 0 ? c[0] : (j == 1 ? c[1] : (j == 2 ? c[2] : c[3]));
    return (float)(w >> 8);
}

// Total order on fp32 scores: larger first, -0 == +0, NaN below -inf.
__device__ __forceinline__ int32_t order_key(float f) {
    if (f != f) return (int32_t)0x80000000;
    if (f == 0.0f) return 0;
    const int32_t i = __float_as_int(f);
    return i >= 0 ? i : (i ^ 0x7fffffff);
}

}  // namespace canon
}  // namespace moe

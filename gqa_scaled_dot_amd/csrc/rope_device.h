// Device side of the rotary position embedding (graph protocol op catalogue,
// op `rope`): the turn of one channel pair by position * invFreq[i], used by
// the standalone rope kernel, the rotate-then-write cache kernel and the
// attention kernels' q loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {

// cos and sin of pos * invf, each times af. The angle is reduced modulo pi/2
// in double precision (the product of a position below 2^31 and an f32 is
// exact or within one double rounding, and pi/2 is carried in two doubles), so
// large positions lose nothing; sin and cos of the reduced angle
// (|x| <= pi/4) are their Taylor series to x^11 and x^12, whose truncation
// error there is below 1e-11, evaluated in f32.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, float invf, float af, float& c, float& s) {
    const double a = (double)pos * (double)invf;
    const double k = rint(a * 0.63661977236758134308);  // 2/pi
    double r = fma(-k, 1.5707963267948966, a);          // pi/2, leading double
    r = fma(-k, 6.123233995736766e-17, r);              // pi/2, the rest
    const float x = (float)r;
    const float x2 = x * x;
    // Horner with explicit fmas, so every caller rounds the same way.
    float ps = fmaf(x2, -1.0f / 39916800.0f, 1.0f / 362880.0f);
    ps = fmaf(x2, ps, -1.0f / 5040.0f);
    ps = fmaf(x2, ps, 1.0f / 120.0f);
    ps = fmaf(x2, ps, -1.0f / 6.0f);
    ps = fmaf(x2, ps, 1.0f);
    const float sp = x * ps;
    float pc = fmaf(x2, 1.0f / 479001600.0f, -1.0f / 3628800.0f);
    pc = fmaf(x2, pc, 1.0f / 40320.0f);
    pc = fmaf(x2, pc, -1.0f / 720.0f);
    pc = fmaf(x2, pc, 1.0f / 24.0f);
    pc = fmaf(x2, pc, -0.5f);
    const float cp = fmaf(x2, pc, 1.0f);
    const int quadrant = (int)((int64_t)k & 3);
    float sv, cv;
    if (quadrant == 0) {
        sv = sp;
        cv = cp;
    } else if (quadrant == 1) {
        sv = cp;
        cv = -sp;
    } else if (quadrant == 2) {
        sv = -sp;
        cv = -cp;
    } else {
        sv = -cp;
        cv = sp;
    }
    c = cv * af;
    s = sv * af;
}

// Where channel d of a head gets its turn: the frequency index, the channel
// it pairs with, and the sign of that channel's sine term. Channels from rd
// on pass through (rot = false, partner = d).
struct RopeTap {
    int i;
    int partner;
    float sgn;
    bool rot;
};

__device__ __forceinline__ RopeTap rope_tap(const RopeArgs& ra, int d) {
    RopeTap tp;
    tp.rot = d < ra.rd;
    if (!tp.rot) {
        tp.i = 0;
        tp.partner = d;
        tp.sgn = 0.0f;
    } else if (ra.interleaved) {
        tp.i = d >> 1;
        tp.partner = d ^ 1;
        tp.sgn = (d & 1) ? 1.0f : -1.0f;
    } else {
        const int half = ra.rd >> 1;
        const bool first = d < half;
        tp.i = first ? d : d - half;
        tp.partner = first ? d + half : d - half;
        tp.sgn = first ? -1.0f : 1.0f;
    }
    return tp;
}

// The turned value of a channel x whose pair partner is xp, at position pos,
// with invf = inv_freq[tp.i]: first of a pair a cos - b sin, second
// b cos + a sin.
__device__ __forceinline__ float rope_turn(const RopeArgs& ra, const RopeTap& tp, float x, float xp, float invf,
                                           int64_t pos) {
    if (!tp.rot) return x;
    float c, s;
    rope_cos_sin(pos, invf, ra.af, c, s);
    return fmaf(tp.sgn * xp, s, x * c);
}

// Channel d of one head (row `head`, head_dim channels) after the turn at
// position pos.
__device__ __forceinline__ float rope_channel(const RopeArgs& ra, const float* head, int d, int64_t pos) {
    const RopeTap tp = rope_tap(ra, d);
    return rope_turn(ra, tp, head[d], head[tp.partner], ra.inv_freq[tp.i], pos);
}

// Channels d0..d0+3 of one head after the turn (d0 a multiple of 4).
__device__ __forceinline__ float4 rope_channels4(const RopeArgs& ra, const float* head, int d0, int64_t pos) {
    float4 o;
    o.x = rope_channel(ra, head, d0, pos);
    o.y = rope_channel(ra, head, d0 + 1, pos);
    o.z = rope_channel(ra, head, d0 + 2, pos);
    o.w = rope_channel(ra, head, d0 + 3, pos);
    return o;
}

}  // namespace attn

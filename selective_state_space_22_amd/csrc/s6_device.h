// s6_device.h -- gfx950 device numerics for the selective scan (S6).
//
// Everything here is fp32 on the VALU.  Transcendentals go straight to the
// hardware base-2 instructions (v_exp_f32, v_log_f32, v_rcp_f32), which on
// gfx950 issue at half the rate of an FMA and do not overlap with it, so every
// formula below is arranged to spend as few of them as possible.
//
// Mathematics: "Mamba 状态空间模型原理与 Transformer 对比" (kb.agiseed.tech),
//   section 2.1 eq. (2)  zero-order hold, per diagonal entry A_n:
//                        Abar = e^{dt A_n},  Bbar = (e^{dt A_n} - 1)/A_n * B_n
//   eq. (3a)/(3b)        h_t = Abar h_{t-1} + Bbar x_t,  y_t = C_t . h_t
//   section 3.2          dt = softplus(raw dt + per-channel bias)
//   Figure 3 caption     SiLU gate on the SSM branch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s6 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Below this |dt*A_n*log2(e)| the input weight uses the two-term series of
// (e^x - 1)/x; above it, (Abar - 1)/A_n.  At |x| = 6.4e-3 both branches have a
// relative error near 7e-6: x^2/6 for the series, ~0.74 ulp / |x| for the
// cancellation in Abar - 1 (0.74 ulp is v_exp_f32's measured error).
constexpr float kPhiSeriesX2 = 6.4e-3f * kLog2e;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// I/O element access for the two supported layouts of the per-token tensors.
__device__ __forceinline__ float load_io(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_io(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store_io(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_io(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^{-|v|}).
// log1p(e) for e in (0, 1]: w = 1 + e is rounded; c = e - (w - 1) is that
// rounding error exactly (w - 1 is exact by Sterbenz), and
// log1p(e) = ln(w) + ln(1 + c/w) ~= ln(w) + c with error below 2^-24 * e.
// v_log_f32 keeps ~1e-7 relative accuracy for w near 1 (measured).
__device__ __forceinline__ float softplus(float v) {
  float e = ex2(-fabsf(v) * kLog2e);
  float w = 1.0f + e;
  float c = e - (w - 1.0f);
  return fmaxf(v, 0.0f) + __builtin_fmaf(lg2(w), kLn2, c);
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}); saturates without NaN.
__device__ __forceinline__ float silu(float z) { return z * rcp(1.0f + ex2(-z * kLog2e)); }

// Input weight of eq. (2) for one state: beta = dt * (e^x - 1)/x with x = dt*A_n,
// returned together with Abar = e^x.  x2 = x*log2(e).
//   |x2| <  kPhiSeriesX2 : beta = dt + dt^2 * A_n / 2       (series, error <= x^2/6)
//   otherwise            : beta = (Abar - 1) / A_n           (error <= 0.74ulp/|x|)
// For A_n = 0 the first branch is always taken (x = 0) and gives beta = dt.
__device__ __forceinline__ float input_weight(float abar, float x2, float dt, float dt2, float ka, float ah) {
  float big = __builtin_fmaf(abar, ka, -ka);
  float small = __builtin_fmaf(dt2, ah, dt);
  return fabsf(x2) < kPhiSeriesX2 ? small : big;
}

// Input weight for dt >= 0 (dt from softplus), in three instructions and no
// branch.  With x = dt*A_n, beta = dt * f(x), f(x) = (e^x - 1)/x = integral over
// s in [0, 1] of e^{s x}.  The integrand is convex in s, so the trapezoid rule
// bounds the integral from above: f(x) <= (1 + e^x)/2 for every x, and
//     U = dt * (1 + Abar) / 2 >= beta,   U - beta = dt * (x^2/12 + O(x^3)).
// The quotient (Abar - 1)/A_n is accurate for large |x| but not near 0, where
// the rounding error of Abar becomes a relative error ~ulp/|x|.  Adding a margin
// m that covers that error, q = (Abar - 1)/A_n + m (formed with one rounding as
// Abar * ka + kc, kc = -ka + m), makes q >= beta as well, so the smaller of the
// two upper bounds is the closer one:
//     beta ~= min(q, U),  relative error <= min(x^2/12, 2 m |A_n| / |x|).
// v_exp_f32 is within 1 ulp (0.74 measured), so for A_n < 0 (Abar <= 1) one ulp
// of ka, at least 2^-24 |ka|, covers it; for A_n > 0 (Abar >= 1, where the ulp
// doubles) two ulps do.  In an fp32 emulation with Abar anywhere within 1 ulp of
// 2^x2, the error stays below 1.4e-5 for A_n < 0 (2e-5 for A_n > 0), the same
// bound as the guarded form, with a mean upward bias near 1e-6 where |x| > 1e-3.
// For dt < 0 the trapezoid bound turns into a lower bound, so callers that cannot
// rule out a negative dt use input_weight above.
// 1/A_n for the bracket form, finite for every A_n (an A_n of 0 takes U, which is
// then dt exactly, because q = ka + kc is huge).
__device__ __forceinline__ float bracket_ka(float a) {
  const float r = a == 0.0f ? 3.4028235e38f : rcp(a);
  return fminf(fmaxf(r, -3.4028235e38f), 3.4028235e38f);
}
// -ka moved toward +infinity by one ulp (ka < 0) or two (ka > 0).  A ka too small
// to matter (|A_n| beyond 1e37, where dt A_n overflows anyway) keeps no margin, so
// that the bit step never crosses zero.
__device__ __forceinline__ float bracket_kc(float ka) {
  const float v = -ka;
  const uint32_t b = __float_as_uint(v);
  return v > 0.0f ? __uint_as_float(b + 1u) : (v < -1.0e-37f ? __uint_as_float(b - 2u) : v);
}
__device__ __forceinline__ float input_weight_pos(float abar, float dth, float ka, float kc) {
  return fminf(__builtin_fmaf(abar, ka, kc), __builtin_fmaf(abar, dth, dth));
}

// Per-(channel, state) constants derived from A once per launch.
template <int N>
struct ChanConst {
  float a2[N];  // A_n * log2(e): exponent of Abar in base 2 per unit dt
  float ka[N];  // 1 / A_n (finite: bracket_ka)
  float ah[N];  // A_n / 2: second series term of (e^x - 1)/x times dt (guarded form)
  float kc[N];  // offset of the bracket form's quotient
  __device__ __forceinline__ void set(int n, float a) {
    a2[n] = a * kLog2e;
    ka[n] = bracket_ka(a);  // the guarded form never selects its quotient for A_n = 0
    ah[n] = 0.5f * a;
    kc[n] = bracket_kc(ka[n]);
  }
  __device__ __forceinline__ void load(const float* A_row) {
#pragma unroll
    for (int n = 0; n < N; ++n) set(n, A_row[n]);
  }
};

// Per-token, per-channel front end: dt and the quantities shared by all N states.
struct TokenFront {
  float dt;   // discretisation step
  float dt2;  // dt^2, for the series branch of the guarded input weight
  float dth;  // dt / 2, for the bracket form
  bool pos;   // dt comes from softplus (never negative): the bracket form applies
};

__device__ __forceinline__ TokenFront make_front(float raw, float bias, bool do_softplus) {
  TokenFront f;
  float v = raw + bias;
  f.dt = do_softplus ? softplus(v) : v;
  f.dt2 = f.dt * f.dt;
  f.dth = 0.5f * f.dt;
  f.pos = do_softplus;
  return f;
}

__device__ __forceinline__ float input_weight_of(const TokenFront& f, float abar, float x2, float ka, float ah,
                                                 float kc) {
  return f.pos ? input_weight_pos(abar, f.dth, ka, kc) : input_weight(abar, x2, f.dt, f.dt2, ka, ah);
}

// One token of eq. (3a) for all N states of one channel, followed by the
// eq. (3b) readout from the updated state.  Bt/Ct hold B_t and C_t.
template <int N>
__device__ __forceinline__ float token_step(const ChanConst<N>& cc, const TokenFront& f, float x, const float* Bt,
                                            const float* Ct, float (&h)[N]) {
  float y = 0.0f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x2 = f.dt * cc.a2[n];
    float abar = ex2(x2);
    float beta = input_weight_of(f, abar, x2, cc.ka[n], cc.ah[n], cc.kc[n]);
    h[n] = __builtin_fmaf(abar, h[n], beta * (Bt[n] * x));
    y = __builtin_fmaf(Ct[n], h[n], y);
  }
  return y;
}

// Same recurrence without the readout (chunk aggregates).
template <int N>
__device__ __forceinline__ void token_step_state(const ChanConst<N>& cc, const TokenFront& f, float x, const float* Bt,
                                                 float (&h)[N]) {
#pragma unroll
  for (int n = 0; n < N; ++n) {
    float x2 = f.dt * cc.a2[n];
    float abar = ex2(x2);
    float beta = input_weight_of(f, abar, x2, cc.ka[n], cc.ah[n], cc.kc[n]);
    h[n] = __builtin_fmaf(abar, h[n], beta * (Bt[n] * x));
  }
}

// ---------------------------------------------------------------- complex A
//
// The complex row A_n = -1/2 + n i of the page's A-initialisation ablation
// (section 6.5), with dt, x, B and C real: eq. (2) over the complex numbers,
//     Abar = e^{dt Re A} (cos(dt Im A) + i sin(dt Im A)),  beta = (Abar - 1)/A_n,
// and the output reads Re(C . h).
//
// A state with slow decay multiplies by nearly the same Abar for thousands of
// tokens, so any bias in Abar grows linearly in the state.  The hardware
// v_sin_f32 / v_cos_f32 (errors up to ~3e-7, ~5 ulp) measured four times the
// error budget of an fp32 scan this way; sin and cos are therefore evaluated
// here from their Taylor series (about 1 ulp), with fewer terms when a wave's
// angles of the token are all small.  Below |dt A_n| = 0.02 the input
// weight is the series dt (1 + x/2 + x^2/6) (truncation <= |x|^3/24 < 4e-7);
// above it the quotient, whose cancellation costs err(Abar)/|x| < 1e-5.
constexpr float kCplxSeriesX2 = 0.02f * 0.02f;
constexpr float kQuarterPi = 0.78539816339744831f;
constexpr float k2OverPi = 0.63661977236758134f;
constexpr float kHalfPiHi = 1.57079637050628662f;    // float(pi/2)
constexpr float kHalfPiLo = -4.37113900018624e-8f;   // pi/2 - kHalfPiHi

constexpr float kTinyAngle = 0.25f;

// sin r and cos r for |r| <= 1/4: Taylor series through r^7 and r^6
// (truncation below 1e-11 and 4e-10).
__device__ __forceinline__ void sincos_tiny(float r, float& s, float& c) {
  const float r2 = r * r;
  float ps = __builtin_fmaf(r2, -1.0f / 5040.0f, 1.0f / 120.0f);
  ps = __builtin_fmaf(r2, ps, -1.0f / 6.0f);
  s = __builtin_fmaf(r * r2, ps, r);
  float pc = __builtin_fmaf(r2, -1.0f / 720.0f, 1.0f / 24.0f);
  pc = __builtin_fmaf(r2, pc, -0.5f);
  c = __builtin_fmaf(r2, pc, 1.0f);
}

// sin r and cos r for |r| <= pi/4: Taylor series through r^9 and r^10
// (truncation below 2e-9 and 6e-11).
__device__ __forceinline__ void sincos_small(float r, float& s, float& c) {
  const float r2 = r * r;
  float ps = __builtin_fmaf(r2, 1.0f / 362880.0f, -1.0f / 5040.0f);
  ps = __builtin_fmaf(r2, ps, 1.0f / 120.0f);
  ps = __builtin_fmaf(r2, ps, -1.0f / 6.0f);
  s = __builtin_fmaf(r * r2, ps, r);
  float pc = __builtin_fmaf(r2, -1.0f / 3628800.0f, 1.0f / 40320.0f);
  pc = __builtin_fmaf(r2, pc, -1.0f / 720.0f);
  pc = __builtin_fmaf(r2, pc, 1.0f / 24.0f);
  pc = __builtin_fmaf(r2, pc, -0.5f);
  c = __builtin_fmaf(r2, pc, 1.0f);
}

// sin a and cos a: a = k pi/2 + r with |r| <= pi/4 (pi/2 in two parts, each
// product exact inside the FMA), then the quadrant k mod 4 swaps and negates.
// Accurate while k pi/2 stays far inside fp32's range of exact products
// (|a| up to about 1e5 radians).
__device__ __forceinline__ void sincos_any(float a, float& s, float& c) {
  const float k = __builtin_rintf(a * k2OverPi);
  float r = __builtin_fmaf(-k, kHalfPiHi, a);
  r = __builtin_fmaf(-k, kHalfPiLo, r);
  float sr, cr;
  sincos_small(r, sr, cr);
  const int q = (int)k;
  const float ss = (q & 1) ? cr : sr;
  const float cc = (q & 1) ? sr : cr;
  s = (q & 2) ? -ss : ss;
  c = ((q + 1) & 2) ? -cc : cc;
}

// Per-state constants of a complex A_n.
struct CplxA {
  float re, im;  // A_n
  float kr, ki;  // 1 / A_n = conj(A_n) / |A_n|^2 (inf/NaN for A_n = 0: never selected)
  float m2;      // |A_n|^2
  __device__ __forceinline__ void load(float r, float i) {
    re = r;
    im = i;
    m2 = __builtin_fmaf(r, r, i * i);
    const float inv = rcp(m2);
    kr = r * inv;
    ki = -i * inv;
  }
};

// Angle ranges of the sin/cos evaluation: |dt Im A_n| <= 1/4, <= pi/4, any.
enum AngleTier { kAngleTiny = 0, kAngleSmall = 1, kAngleAny = 2 };

// One token of eq. (3a) for one complex state: h = Abar h + beta * bx, bx = B_t,n x_t.
// TIER: the range the caller has checked |dt Im A_n| to be in.
template <int TIER>
__device__ __forceinline__ void cplx_update(const CplxA& a, float dt, float dt2, float bx, float& hr, float& hi) {
  const float xr = dt * a.re, xi = dt * a.im;
  const float mag = ex2(xr * kLog2e);
  float sn, cs;
  if (TIER == kAngleTiny) sincos_tiny(xi, sn, cs);
  else if (TIER == kAngleSmall) sincos_small(xi, sn, cs);
  else sincos_any(xi, sn, cs);
  const float abr = mag * cs, abi = mag * sn;
  // (Abar - 1) / A
  const float er = abr - 1.0f;
  const float gr = __builtin_fmaf(er, a.kr, -abi * a.ki);
  const float gi = __builtin_fmaf(er, a.ki, abi * a.kr);
  // dt (1 + x (1/2 + x/6))
  const float qr = __builtin_fmaf(xr, 1.0f / 6.0f, 0.5f), qi = xi * (1.0f / 6.0f);
  const float tr = __builtin_fmaf(xr, qr, __builtin_fmaf(-xi, qi, 1.0f));
  const float ti = __builtin_fmaf(xr, qi, xi * qr);
  const bool small = dt2 * a.m2 < kCplxSeriesX2;
  const float br = small ? dt * tr : gr;
  const float bi = small ? dt * ti : gi;
  const float nr = __builtin_fmaf(abr, hr, __builtin_fmaf(-abi, hi, br * bx));
  const float ni = __builtin_fmaf(abr, hi, __builtin_fmaf(abi, hr, bi * bx));
  hr = nr;
  hi = ni;
}

// The smallest tier that holds for every active lane's angles dt |Im A_n|
// (maxim: the lane's largest |Im A_n|); one decision per wave and token.
__device__ __forceinline__ int wave_angle_tier(float dt, float maxim) {
  const float m = dt * maxim;
  if (__all(m <= kTinyAngle)) return kAngleTiny;
  if (__all(m <= kQuarterPi)) return kAngleSmall;
  return kAngleAny;
}

// e^{A_n s} for a sum s of dt (chunk carries).
__device__ __forceinline__ void cplx_decay(const CplxA& a, float s, float& pr, float& pi) {
  const float mag = ex2(s * a.re * kLog2e);
  float sn, cs;
  sincos_any(s * a.im, sn, cs);
  pr = mag * cs;
  pi = mag * sn;
}

// Epilogue of one (token, channel): skip term, then the SiLU gate.
__device__ __forceinline__ float epilogue(float y, float x, float dskip, bool has_z, float zv) {
  y = __builtin_fmaf(dskip, x, y);
  return has_z ? y * silu(zv) : y;
}

}  // namespace s6

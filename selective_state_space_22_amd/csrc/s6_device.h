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

// Per-(channel, state) constants derived from A once per launch.
template <int N>
struct ChanConst {
  float a2[N];  // A_n * log2(e): exponent of Abar in base 2 per unit dt
  float ka[N];  // 1 / A_n
  float ah[N];  // A_n / 2: second series term of (e^x - 1)/x times dt
  __device__ __forceinline__ void load(const float* A_row) {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float a = A_row[n];
      a2[n] = a * kLog2e;
      ka[n] = rcp(a);  // v_rcp_f32 (<1 ulp); inf for A_n = 0, never selected (see input_weight)
      ah[n] = 0.5f * a;
    }
  }
};

// Per-token, per-channel front end: dt and the quantities shared by all N states.
struct TokenFront {
  float dt;   // discretisation step
  float dt2;  // dt^2, for the series branch of the input weight
};

__device__ __forceinline__ TokenFront make_front(float raw, float bias, bool do_softplus) {
  TokenFront f;
  float v = raw + bias;
  f.dt = do_softplus ? softplus(v) : v;
  f.dt2 = f.dt * f.dt;
  return f;
}

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
    float beta = input_weight(abar, x2, f.dt, f.dt2, cc.ka[n], cc.ah[n]);
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
    float beta = input_weight(abar, x2, f.dt, f.dt2, cc.ka[n], cc.ah[n]);
    h[n] = __builtin_fmaf(abar, h[n], beta * (Bt[n] * x));
  }
}

// Epilogue of one (token, channel): skip term, then the SiLU gate.
__device__ __forceinline__ float epilogue(float y, float x, float dskip, bool has_z, float zv) {
  y = __builtin_fmaf(dskip, x, y);
  return has_z ? y * silu(zv) : y;
}

}  // namespace s6

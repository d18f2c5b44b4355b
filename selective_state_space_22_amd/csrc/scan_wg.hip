// scan_wg.hip -- workgroup-cooperative forward selective scan on gfx950.
//
// A workgroup owns one (batch row, block of 64 channels) at a time: lane l of
// every wave is channel block*64 + l, and the W waves split the N states of
// those channels (S = N/W states per wave, kept in VGPRs).  Each token still
// costs one v_exp_f32 per (channel, state), but the work per token is spread
// over W waves, so a (batch*D)-sized problem fills W times more SIMDs than a
// lane-owns-all-states mapping.
//
// Per 16-token tile (one LDS barrier per tile, LDS slots rotating):
//   front   (token j handled by wave j % W): dt = softplus(raw + bias), its
//           square, the input x and the gate z go to LDS; all threads stage
//           B_t and C_t of the tile (shared by all channels: page section 3.2)
//           into LDS.
//   scan    every wave advances its S states over the tile's tokens
//           (eq. (2) discretisation, eq. (3a) recurrence) and writes its partial
//           readout sum_s C_t[s] h_t[s] (eq. (3b)) to LDS.
//   epilogue (token j by wave j % W): y = sum of the W partials, then
//           y + Dskip x, times SiLU(z), one store per (token, channel).
// Global loads for tile k+2 are issued while tile k is computed; every access
// goes through a bounds-checked buffer resource based at the chunk, so tails
// need no branches (out-of-range reads return zero, stores are dropped).
//
// Sequence length is cut into chunks.  In the chained mode the chunks of a
// channel block run in order on whichever workgroup takes them: a persistent
// grid takes work items from a ticket counter in chunk-major order, waits
// until the previous chunk of its channel block has published its end state,
// continues from that state and publishes its own.  A ticket is only handed
// to a running workgroup, and a chunk's predecessor always has a smaller
// ticket, so every wait ends.  In the split mode (few channel blocks, long
// sequences) the chunks run independently in two passes with a carry pass in
// between (the associative composition of chunk aggregates).
#include <cstdlib>

#include "s6_device.h"
#include "s6_internal.h"

namespace s6 {
namespace {

#ifndef S6_SCAN_AHEAD
#define S6_SCAN_AHEAD 1
#endif
#ifndef S6_WG_TILE
#define S6_WG_TILE 16
#endif
#ifndef S6_WG_PER_CU
#define S6_WG_PER_CU 1
#endif
#ifndef S6_WG_SLOTS
#define S6_WG_SLOTS 2
#endif
constexpr int kSlots = S6_WG_SLOTS;  // LDS slots of front-end data (2 or 3)
constexpr int kScanAhead = S6_SCAN_AHEAD;  // tokens of LDS operands read ahead in the scan loop
constexpr int32_t kBufferDword3 = 0x00020000;  // raw (untyped) buffer access on the gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;  // offset beyond every buffer: loads 0, stores dropped

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferDword3);
}

// One I/O element through a buffer resource (bounds-checked by the hardware).
template <typename IO>
struct BufIo;
template <>
struct BufIo<uint16_t> {
  static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw << 16); }
  static __device__ __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
  }
};
template <>
struct BufIo<float> {
  static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw); }
  static __device__ __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
  }
};

// Wait for every outstanding vector-memory access (the item's constants and
// initial state), so that later waits only have to cover the tile prefetches.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDtSlices = 8;  // 64-byte K slices of the fused dt projection kept in registers

// One 64-byte K slice of the dt projection on the matrix cores (16 x 16 output tile).
template <typename IO>
__device__ __forceinline__ f32x4 dt_mfma(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 dt_mfma<uint16_t>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
template <>
__device__ __forceinline__ f32x4 dt_mfma<float>(u32x4 a, u32x4 b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

// POS: dt is known to be non-negative (it comes from softplus), so the input
// weight takes the bracket form (input_weight_pos); otherwise the guarded form.
template <typename IO, int N, int W, int T, int MODE, bool FDT, bool CPLX, bool POS>
struct WgScan {
  static constexpr int S = N / W;                 // states per wave
  static constexpr int CF = CPLX ? 2 : 1;         // floats per state (complex A: re, im)
  static constexpr int CS = CPLX ? S : 1;         // sizes of the complex-only register arrays
  static constexpr int TW = T / W;                // front-end / epilogue tokens per wave per tile
  static constexpr int NT = 64 * W;               // threads
  // B/C of a tile: 2TN elements.  With at least one per thread, the first half
  // of the waves stage B and the second half C, BCV consecutive elements per
  // thread; with fewer (short tiles), the first 2TN/64 waves stage one each.
  static constexpr bool kBcSparse = 2 * T * N < NT;
  static constexpr int BCV = kBcSparse ? 1 : 2 * T * N / NT;  // B/C elements staged per thread per tile
  static_assert(N % W == 0 && T % W == 0 && W % 2 == 0, "tile shape");
  static_assert(kBcSparse ? (T * N) % 64 == 0 : ((2 * T * N) % NT == 0 && N % BCV == 0), "B/C staging");
  static constexpr bool kOut = MODE != kModeAgg;
  static constexpr uint32_t kIo = sizeof(IO);

  // Buffers of tile k: fr and bc in slot k % kSlots, yp in slot k % 2.  With
  // three slots, iteration k runs front(k+1), epilogue(k-1), scan(k), then the
  // tile's one barrier.  Race-free: front(k+1) overwrites the fr/bc slot of
  // tile k-2, whose last readers (scan(k-2), epilogue(k-2)) finished before the
  // barrier of iteration k-1; scan(k) overwrites the yp slot of tile k-2, last
  // read by epilogue(k-2) before that same barrier; epilogue(k-1) reads what
  // scan(k-1) wrote before the barrier of iteration k-1.  With two slots the
  // epilogue of k-1 runs first (see run_item).
  static constexpr int BCW = (2 * S + 3) / 4 * 4;  // bc row per (token, wave), padded to float4

  struct Lds {
    float4 fr[kSlots][T][64];                    // (dt, dt / 2 (POS) or dt^2, x, z) per (token, channel)
    __attribute__((aligned(16))) float bc[kSlots][T][W][BCW];  // per token and wave: B of its states, then C
    float yp[kOut ? 2 : 1][T][W][64];            // partial readouts
    float sdt[W][64];                            // split mode: partial sums of dt
    float raw[FDT ? 2 : 1][T][64];               // fused dt projection: raw dt per (token, channel)
    int item[2];
    int poison;  // chained mode: the wait for this item's carry-in gave up
  };

  struct Regs {  // raw prefetched global data of one tile
    uint32_t dl[TW], uu[TW], zz[TW];
    uint32_t bcv[BCV];
  };

  const WgArgs& A;
  Lds& sm;
  const int lane, w;
  // current item
  int64_t b, d, t0, t1;
  bool dvalid;
  uint32_t chan_off;  // byte offset of this lane's channel in a token row (out of range if d >= D)
  __amdgpu_buffer_rsrc_t r_u, r_dl, r_z, r_out, r_B, r_C;
  // fused dt projection: waves 0..3 own channels 16w..16w+15 of the block
  static_assert(!FDT || T == 16, "fused dt projection works on 16-token tiles");
  __amdgpu_buffer_rsrc_t r_dtl, r_wdt;
  u32x4 wdt[kDtSlices], dta[kDtSlices];
  int nks;
  // per-state constants of the input weight: A_n log2(e), then 1/A_n and the
  // bracket form's offset (POS) or 1/A_n and A_n / 2
  float a2[S], ka[S], k2[S], h[S];
  CplxA ca[CS];  // complex A: per-state constants; h holds Re h, hq Im h
  float hq[CS];
  float maxim;   // complex A: largest |Im A_n| of this wave's states
  float bias, dskip;
  float dsum, dcomp;  // compensated sum of dt (split mode, first pass)

  // The wave index is made a scalar (readfirstlane) so that everything derived
  // from it -- which states a wave owns, which of B/C it stages -- stays uniform.
  __device__ WgScan(const WgArgs& a, Lds& s)
      : A(a), sm(s), lane(threadIdx.x & 63), w(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {}

  __device__ __forceinline__ int tile_valid(int k) const {
    const int64_t tk = t0 + (int64_t)k * T;
    const int64_t r = t1 - tk;
    return r <= 0 ? 0 : (r >= T ? T : (int)r);
  }

  // Global loads of tile k.  Unconditional: rows past the chunk and lanes past D
  // are out of the buffers' range and read as zero.
  __device__ __forceinline__ void load(Regs& r, int k) const {
    const uint32_t row = (uint32_t)(A.s.D * kIo);
    const uint32_t base = chan_off + (uint32_t)(k * T + w) * row;  // one vector add per tile
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const uint32_t off = base + (uint32_t)(W * i) * row;
      if (!FDT) r.dl[i] = BufIo<IO>::load(r_dl, off);
      r.uu[i] = BufIo<IO>::load(r_u, off);
      if (kOut) r.zz[i] = BufIo<IO>::load(r_z, off);
    }
    if (kBcSparse) {
      const int q = (w * 64) / (T * N);  // 0: B, 1: C, >= 2: nothing (uniform per wave)
      const __amdgpu_buffer_rsrc_t rbc = q == 0 ? r_B : r_C;
      const int e = w * 64 + lane - q * (T * N);
      r.bcv[0] = BufIo<IO>::load(rbc, q < 2 ? (uint32_t)(k * T * N + e) * kIo : kOutOfRange);
    } else {
      // The first half of the waves stage B, the second half C (uniform per wave).
      const __amdgpu_buffer_rsrc_t rbc = w < W / 2 ? r_B : r_C;
#pragma unroll
      for (int v = 0; v < BCV; ++v) {
        const int e = ((w % (W / 2)) * 64 + lane) * BCV + v;  // element of the tile's B (or C) block
        r.bcv[v] = BufIo<IO>::load(rbc, (uint32_t)(k * T * N + e) * kIo);
      }
    }
  }

  // Fused dt projection.  Operands straight from global memory in the MFMA
  // layout (lane l: row l % 16, the 16 bytes at offset 16 (l / 16) of each
  // 64-byte K slice); K slices past R and rows past the chunk or D read zero.
  // Waves 0..3 project dt for every tile.  (Alternating tiles between the two
  // groups of four waves measured slower: the extra registers cost more than
  // the balance gains.)
  __device__ __forceinline__ bool dt_group(int) const { return w < 4; }
  __device__ __forceinline__ void load_dt(int k) {
    if (!FDT || !dt_group(k)) return;
    const uint32_t ldb = (uint32_t)(A.s.ldr * kIo);
    const uint32_t rbytes = (uint32_t)(A.s.R * kIo);
    const uint32_t row = (uint32_t)(k * T + (lane & 15));
#pragma unroll
    for (int ks = 0; ks < kDtSlices; ++ks) {
      const uint32_t kb = (uint32_t)ks * 64u + 16u * (lane >> 4);
      dta[ks] = __builtin_amdgcn_raw_buffer_load_b128(r_dtl, ks < nks && kb < rbytes ? row * ldb + kb : kOutOfRange,
                                                      0, 0);
    }
  }
  // raw dt of tile k's 16 tokens for channels 16w..16w+15 into raw slot k & 1
  __device__ __forceinline__ f32x4 mfma_dt() const {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kDtSlices; ++ks)
      if (ks < nks) acc = dt_mfma<IO>(dta[ks], wdt[ks], acc);
    return acc;
  }
  __device__ __forceinline__ void store_dt(const f32x4& acc, int k) {
    if (!FDT || !dt_group(k)) return;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) sm.raw[k & 1][4 * (lane >> 4) + rr][16 * (w & 3) + (lane & 15)] = acc[rr];
  }

  // Front end of tile k into slot f3 of fr and bc.
  __device__ __forceinline__ void front(const Regs& r, int k, int f3) {
    const int nv = tile_valid(k);
    const bool sp = A.s.softplus != 0;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int j = w + W * i;
      const float x = BufIo<IO>::widen(r.uu[i]);
      const float raw = FDT ? sm.raw[k & 1][j][lane] : BufIo<IO>::widen(r.dl[i]);
      TokenFront f = make_front(raw, bias, sp);
      sm.fr[f3][j][lane] = make_float4(f.dt, POS ? 0.5f * f.dt : f.dt2, x, kOut ? BufIo<IO>::widen(r.zz[i]) : 0.0f);
      if (MODE == kModeAgg) {  // Kahan sum of dt over this wave's valid tokens
        const float yk = (j < nv ? f.dt : 0.0f) - dcomp;
        const float tk = dsum + yk;
        dcomp = (tk - dsum) - yk;
        dsum = tk;
      }
    }
    if (kBcSparse) {
      const int q = (w * 64) / (T * N);
      if (q < 2) {
        const int e = w * 64 + lane - q * (T * N);
        const int j = e / N, n = e % N;
        sm.bc[f3][j][n / S][q * S + n % S] = BufIo<IO>::widen(r.bcv[0]);
      }
    } else {
      const int c = w < W / 2 ? 0 : 1;
#pragma unroll
      for (int v = 0; v < BCV; ++v) {
        const int e = ((w % (W / 2)) * 64 + lane) * BCV + v;
        const int j = e / N, n = e % N;
        sm.bc[f3][j][n / S][c * S + n % S] = BufIo<IO>::widen(r.bcv[v]);
      }
    }
  }

  struct Tok {  // LDS operands of one token for this lane and wave
    float4 fv;   // dt, dt^2, x, z
    float bc[BCW];
  };

  __device__ __forceinline__ void read_tok(Tok& t, int f3, int j) const {
    // a 16-byte read although the scan uses three components: a 12-byte LDS
    // read costs about twice the cycles of a 16-byte one on gfx950 (measured)
    t.fv = sm.fr[f3][j][lane];
    asm volatile("" : "+v"(t.fv.w));
#pragma unroll
    for (int q = 0; q < BCW; q += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(&sm.bc[f3][j][w][q]);
      t.bc[q] = v4.x;
      t.bc[q + 1] = v4.y;
      t.bc[q + 2] = v4.z;
      t.bc[q + 3] = v4.w;
    }
  }

  // Complex A: one token for this wave's S states with the sin/cos of one angle tier.
  template <int TIER>
  __device__ __forceinline__ float cstep(const Tok& t) {
    float y = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      cplx_update<TIER>(ca[s], t.fv.x, t.fv.y, t.bc[s] * t.fv.z, h[s], hq[s]);
      if (kOut) y = __builtin_fmaf(t.bc[S + s], h[s], y);
    }
    return y;
  }

  // One token of the recurrence for this wave's S states (eq. (2), (3a)) and
  // its partial readout sum_s C_t[s] h_t[s] (eq. (3b)).
  __device__ __forceinline__ void step(const Tok& t, int y2, int j) {
    float y = 0.0f;
    if constexpr (CPLX) {
      const int tier = wave_angle_tier(t.fv.x, maxim);
      if (tier == kAngleTiny) y = cstep<kAngleTiny>(t);
      else if (tier == kAngleSmall) y = cstep<kAngleSmall>(t);
      else y = cstep<kAngleAny>(t);
      if (kOut) sm.yp[y2][j][w][lane] = y;
      return;
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float x2 = t.fv.x * a2[s];
      const float abar = ex2(x2);
      const float beta = POS ? input_weight_pos(abar, t.fv.y, ka[s], k2[s])
                             : input_weight(abar, x2, t.fv.x, t.fv.y, ka[s], k2[s]);
      h[s] = __builtin_fmaf(abar, h[s], beta * (t.bc[s] * t.fv.z));
      if (kOut) y = __builtin_fmaf(t.bc[S + s], h[s], y);
    }
    if (kOut) sm.yp[y2][j][w][lane] = y;
  }

  // Recurrence over tile k from slot f3; partial readouts to yp slot y2.
  // Full tiles are unrolled (constant LDS offsets) with the next token's
  // operands read before the current token is computed.
  __device__ __forceinline__ void scan(int k, int f3, int y2) {
    const int nv = tile_valid(k);
    if (nv == T) {
      // operands of the next kScanAhead tokens are in flight while a token is computed
      constexpr int P = kScanAhead < T ? kScanAhead : T;
      Tok t[P + 1];
#pragma unroll
      for (int j = 0; j < P; ++j) read_tok(t[j], f3, j);
#pragma unroll
      for (int j = 0; j < T; ++j) {
        if (j + P < T) read_tok(t[(j + P) % (P + 1)], f3, j + P);
        step(t[j % (P + 1)], y2, j);
      }
    } else {
      for (int j = 0; j < nv; ++j) {
        Tok t;
        read_tok(t, f3, j);
        step(t, y2, j);
      }
    }
  }

  // Readout sum, skip, gate and store for this wave's tokens of tile k
  // (rows past the chunk and lanes past D fall outside the output buffer).
  __device__ __forceinline__ void epilogue(int k, int f3, int y2) {
    if (!kOut) return;
    const bool has_z = A.s.z != nullptr;
    const uint32_t row = (uint32_t)(A.s.D * kIo);
    const uint32_t base = chan_off + (uint32_t)(k * T + w) * row;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int j = w + W * i;
      float y = sm.yp[y2][j][0][lane];
#pragma unroll
      for (int q = 1; q < W; ++q) y += sm.yp[y2][j][q][lane];
      const float4 fv = sm.fr[f3][j][lane];
      const float o = s6::epilogue(y, fv.z, dskip, has_z, fv.w);
      BufIo<IO>::store(o, r_out, base + (uint32_t)(W * i) * row);
    }
  }

  // This wave's S states from / to p, the address of the first of them in a
  // state array (N floats, or N (re, im) pairs, per channel).
  __device__ __forceinline__ void get_state(const float* p) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      h[s] = p[s * CF];
      if constexpr (CPLX) hq[s] = p[s * CF + 1];
    }
  }
  __device__ __forceinline__ void put_state(float* p) const {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      p[s * CF] = h[s];
      if constexpr (CPLX) p[s * CF + 1] = hq[s];
    }
  }

  __device__ void run_item(int chain, int g) {
    const int G = A.s.nchunks;
    b = chain / A.blocks_per_row;
    d = (int64_t)(chain % A.blocks_per_row) * 64 + lane;
    dvalid = d < A.s.D;
    t0 = (int64_t)g * A.s.chunk_len;
    t1 = t0 + A.s.chunk_len < A.s.L ? t0 + A.s.chunk_len : A.s.L;
    // an aggregate may skip the part of its chunk that cannot reach the chunk's end
    if (MODE == kModeAgg && A.s.agg_start)
      t0 += A.s.agg_start[((size_t)b * G + g) * A.blocks_per_row + chain % A.blocks_per_row];
    chan_off = dvalid ? (uint32_t)(d * kIo) : kOutOfRange;
    {
      const size_t row0 = ((size_t)b * A.s.L + t0);
      const uint32_t span = (uint32_t)((t1 - t0) * A.s.D * kIo);
      const uint32_t bspan = (uint32_t)((t1 - t0) * N * kIo);
      r_u = make_rsrc(static_cast<const IO*>(A.s.u) + row0 * A.s.D, span);
      r_dl = make_rsrc(static_cast<const IO*>(A.s.delta) + row0 * A.s.D, span);
      r_z = make_rsrc(A.s.z ? static_cast<const IO*>(A.s.z) + row0 * A.s.D : static_cast<const IO*>(A.s.u),
                      A.s.z ? span : 0u);
      r_out = make_rsrc(static_cast<const IO*>(A.s.out) + row0 * A.s.D, kOut ? span : 0u);
      r_B = make_rsrc(static_cast<const IO*>(A.s.B) + row0 * N, bspan);
      r_C = make_rsrc(static_cast<const IO*>(A.s.C) + row0 * N, bspan);
      if (FDT) {
        r_dtl = make_rsrc(static_cast<const IO*>(A.s.dtlow) + row0 * A.s.ldr, (uint32_t)((t1 - t0) * A.s.ldr * kIo));
        const int64_t c0 = (d - lane) + 16 * (w & 3);  // first channel of this wave's group
        const int64_t rows = A.s.D - c0 < 16 ? (A.s.D - c0 > 0 ? A.s.D - c0 : 0) : 16;
        r_wdt = make_rsrc(static_cast<const IO*>(A.s.Wdt) + c0 * A.s.R, (uint32_t)(rows * A.s.R * kIo));
        nks = (int)((A.s.R * kIo + 63) / 64);
        if (w < 4) {
          const uint32_t rbytes = (uint32_t)(A.s.R * kIo);
#pragma unroll
          for (int ks = 0; ks < kDtSlices; ++ks) {
            const uint32_t kb = (uint32_t)ks * 64u + 16u * (lane >> 4);
            wdt[ks] = __builtin_amdgcn_raw_buffer_load_b128(
                r_wdt, ks < nks && kb < rbytes ? (uint32_t)((lane & 15) * A.s.R * kIo) + kb : kOutOfRange, 0, 0);
          }
        }
      }
    }
    const int nstate0 = w * S;
    if constexpr (CPLX) {
      maxim = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const size_t k = ((size_t)d * N + nstate0 + s) * 2;
        ca[s].load(dvalid ? A.s.A[k] : -1.0f, dvalid ? A.s.A[k + 1] : 0.0f);
        maxim = fmaxf(maxim, fabsf(ca[s].im));
      }
    } else {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const float a = dvalid ? A.s.A[d * N + nstate0 + s] : -1.0f;
        a2[s] = a * kLog2e;
        ka[s] = POS ? bracket_ka(a) : rcp(a);
        k2[s] = POS ? bracket_kc(ka[s]) : 0.5f * a;
      }
    }
    bias = (dvalid && A.s.bias) ? A.s.bias[d] : 0.0f;
    dskip = (dvalid && A.s.dskip) ? A.s.dskip[d] : 0.0f;
    dsum = 0.0f;
    dcomp = 0.0f;

    // state entering the chunk
#pragma unroll
    for (int s = 0; s < S; ++s) h[s] = 0.0f;
#pragma unroll
    for (int s = 0; s < CS; ++s) hq[s] = 0.0f;
    if (MODE == kModeChained) {
      if (g == 0) {
        if (A.s.h0 && dvalid) get_state(A.s.h0 + (((size_t)b * A.s.D + d) * N + nstate0) * CF);
      } else {
        if (threadIdx.x == 0) {
          // Bounded wait for the previous chunk's end state.  Giving up sets the
          // device's status word and poisons this chunk's state with NaN, so the
          // rest of the channel block's outputs cannot pass for valid ones.
          bool ok = A.spin_limit > 0;
          uint32_t spins = 0;
          while (ok && __hip_atomic_load(A.flags + chain, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)g) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins >= A.spin_limit) ok = false;
          }
          if (!ok) __hip_atomic_store(A.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sm.poison = ok ? 0 : 1;
        }
        // Thread 0's acquire load (which invalidates this CU's caches) is
        // ordered before the other waves' reads of the carry by the barrier.
        __syncthreads();
        get_state(A.carry + (((size_t)chain * 64 + lane) * N + nstate0) * CF);
        if (sm.poison) {
#pragma unroll
          for (int s = 0; s < S; ++s) h[s] = __builtin_nanf("");
#pragma unroll
          for (int s = 0; s < CS; ++s) hq[s] = __builtin_nanf("");
        }
      }
    } else if (MODE == kModeOut) {
      if (dvalid) get_state(A.s.agg_h + ((((size_t)b * G + g) * A.s.D + d) * N + nstate0) * CF);
    }
    wait_vmem();

    // tile pipeline: global loads one tile ahead, LDS slots rotating
    const int ntiles = (int)((t1 - t0 + T - 1) / T);
    Regs r;
    if (FDT) {  // raw dt of tiles 0 and 1, operands of tile 2 in flight
      load_dt(0);
      if (dt_group(0)) store_dt(mfma_dt(), 0);
      load_dt(1);
      if (dt_group(1)) store_dt(mfma_dt(), 1);
      load_dt(2);
    }
    load(r, 0);
    if (FDT) __syncthreads();
    front(r, 0, 0);
    load(r, 1);
    __syncthreads();
    // The epilogue of tile k-1 runs in the same barrier interval as the scan
    // of tile k: it reads the yp slot of k-1 (next written by the scan of k+1,
    // after this interval's barrier) and the fr slot of k-1 (next written by
    // the front end of k+2, also after it).
    static_assert(!FDT || kSlots == 2, "fused dt projection uses the two-slot pipeline");
    if (kSlots == 3) {
      int f3 = 0;   // slot of tile k
      int f3p = 2;  // slot of tile k - 1
      for (int k = 0; k < ntiles; ++k) {
        const int f3n = f3 == 2 ? 0 : f3 + 1;
        front(r, k + 1, f3n);
        load(r, k + 2);
        if (k > 0) epilogue(k - 1, f3p, (k - 1) & 1);
        scan(k, f3, k & 1);
        __syncthreads();
        f3p = f3;
        f3 = f3n;
      }
      if (ntiles > 0) epilogue(ntiles - 1, f3p, (ntiles - 1) & 1);
    } else {
      // Two slots: the epilogue of tile k-1 reads its fr entries before the
      // front end of tile k+1 overwrites that slot.  Both touch only the
      // entries of this wave's own tokens (token j belongs to wave j % W), so
      // program order within the wave is enough; the scans read all entries
      // of a slot only in the interval after its front end, past a barrier.
      for (int k = 0; k < ntiles; ++k) {
        const int f2 = k & 1;
        if (k > 0) epilogue(k - 1, f2 ^ 1, f2 ^ 1);
        front(r, k + 1, f2 ^ 1);
        // fused dt projection of tile k+2: issued before the scan, its result
        // (raw slot k & 1, last read by front(k) before the previous barrier)
        // stored after it, so the matrix cores run while the VALU scans
        f32x4 acc;
        if (FDT && dt_group(k + 2)) acc = mfma_dt();
        load(r, k + 2);
        load_dt(k + 3);
        scan(k, f2, f2);
        if (FDT) store_dt(acc, k + 2);
        __syncthreads();
      }
      if (ntiles > 0) epilogue(ntiles - 1, (ntiles - 1) & 1, (ntiles - 1) & 1);
    }

    // publish the chunk's end
    if (MODE == kModeChained) {
      if (g < G - 1) {
        put_state(A.carry + (((size_t)chain * 64 + lane) * N + nstate0) * CF);
        // Every wave's carry stores complete (reach L2) before the barrier;
        // thread 0's release store then writes the L2 back once for all of
        // them before the flag becomes visible.
        wait_vmem();
        __syncthreads();
        if (threadIdx.x == 0)
          __hip_atomic_store(A.flags + chain, (uint32_t)(g + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else if (A.s.last && dvalid) {
        put_state(A.s.last + (((size_t)b * A.s.D + d) * N + nstate0) * CF);
      }
    } else if (MODE == kModeAgg) {
      const size_t base = ((size_t)b * G + g) * A.s.D + d;
      if (dvalid) put_state(A.s.agg_h + (base * N + nstate0) * CF);
      sm.sdt[w][lane] = dsum;
      __syncthreads();
      if (w == 0 && dvalid) {
        float tot = 0.0f;
#pragma unroll
        for (int q = 0; q < W; ++q) tot += sm.sdt[q][lane];
        A.s.agg_s[base] = tot;
      }
    } else {  // kModeOut
      if (g == G - 1 && A.s.last && dvalid) put_state(A.s.last + (((size_t)b * A.s.D + d) * N + nstate0) * CF);
    }
  }
};

// The launch bound's second value is the waves per SIMD the registers must
// allow: the workgroups per CU that LDS admits (S6_WG_PER_CU on 16-token tiles,
// twice that on 8-token tiles) times W waves, over the CU's 4 SIMDs.
template <int W, int T>
constexpr int wg_waves_per_simd() {
  constexpr int v = (T < 16 ? 2 : 1) * S6_WG_PER_CU * W / 4;
  return v > 1 ? v : 1;
}

template <typename IO, int N, int W, int T, int MODE, bool FDT, bool CPLX, bool POS>
__global__ __launch_bounds__(64 * W, (wg_waves_per_simd<W, T>())) void scan_wg_kernel(WgArgs a) {
  using K = WgScan<IO, N, W, T, MODE, FDT, CPLX, POS>;
  __shared__ typename K::Lds sm;
  K k(a, sm);
  for (int round = 0;; ++round) {
    if (threadIdx.x == 0) sm.item[round & 1] = (int)atomicAdd(a.ticket, 1u);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(sm.item[round & 1]);
    if (item >= a.nitems) break;
    k.run_item(item % a.chains, item / a.chains);
  }
}

// Clears the work ticket and the chained-mode flags of a call.  The words are
// cleared with agent-scope atomic stores, like every later access to them (the
// ticket's atomic adds, the flags' release stores and acquire polls), so that no
// XCD can read a value of the previous call that a plain store left in another
// XCD's L2; this does not depend on the cache write-back between the two kernels,
// which a replayed graph may arrange differently from a stream.
__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) __hip_atomic_store(p + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// T: tokens per tile of the chained mode and of the split mode's first pass;
// TO: of the split mode's output pass.
template <typename IO, int N, int W, int T, int TO, bool FDT, bool CPLX, bool POS>
hipError_t launch_wg_t(const ScanArgs& s, const ScanPlan& p, void* ws, hipStream_t st) {
  constexpr int CF = CPLX ? 2 : 1;
  uint8_t* base = static_cast<uint8_t*>(ws);
  WgArgs a;
  a.s = s;
  a.blocks_per_row = (int32_t)((s.D + 63) / 64);
  a.chains = (int32_t)(s.batch * a.blocks_per_row);
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(base);
  a.err = wait_status_ptr();
  if (a.err == nullptr) return hipErrorInvalidSymbol;
  a.spin_limit = (uint32_t)option(kOptSpinLimit);
  a.flags = ctrl + 64;
  const int64_t ctrl_words = (int64_t)(p.ws_ctrl / 4);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((ctrl_words + 255) / 256)), dim3(256), 0, st, ctrl,
                     ctrl_words);
  const dim3 block(64 * W);
  if (!p.split) {
    a.ticket = ctrl;
    a.carry = reinterpret_cast<float*>(base + p.ws_ctrl);
    a.nitems = a.chains * p.nchunks;
    hipLaunchKernelGGL((scan_wg_kernel<IO, N, W, T, kModeChained, FDT, CPLX, POS>), dim3(p.grid), block, 0, st, a);
  } else {
    a.s.agg_h = reinterpret_cast<float*>(base + p.ws_ctrl);
    a.s.agg_s = a.s.agg_h + (size_t)s.batch * p.nchunks * s.D * N * CF;
    int32_t* start = reinterpret_cast<int32_t*>(a.s.agg_s + (size_t)s.batch * p.nchunks * s.D);
    if (!CPLX && launch_agg_start(a.s, sizeof(IO) == 2 ? kIoBF16 : kIoF32, N, start, st)) a.s.agg_start = start;
    a.carry = nullptr;
    a.ticket = ctrl;
    a.nitems = a.chains * (p.nchunks - 1);
    const unsigned g1 = (unsigned)(a.nitems < p.grid ? a.nitems : p.grid);
    hipLaunchKernelGGL((scan_wg_kernel<IO, N, W, T, kModeAgg, FDT, CPLX, POS>), dim3(g1), block, 0, st, a);
    const hipError_t ce = CPLX ? launch_cplx_carry(a.s, N, st) : launch_chunk_carry(a.s, N, st);
    if (ce != hipSuccess) return ce;
    a.ticket = ctrl + 1;
    a.nitems = a.chains * p.nchunks;
    const unsigned g2 = (unsigned)(a.nitems < p.grid_out ? a.nitems : p.grid_out);
    hipLaunchKernelGGL((scan_wg_kernel<IO, N, W, TO, kModeOut, FDT, CPLX, POS>), dim3(g2), block, 0, st, a);
  }
  return hipGetLastError();
}

template <typename IO, int N, int W, int T>
hipError_t launch_wg_fdt(const ScanArgs& s, const ScanPlan& p, bool cplx, void* ws, hipStream_t st) {
  if (p.tile_out != T && (p.tile_out != 8 || !p.split || cplx || s.dtlow)) return hipErrorInvalidValue;
  if (cplx) return s.dtlow ? hipErrorInvalidValue : launch_wg_t<IO, N, W, T, T, false, true, false>(s, p, ws, st);
  const bool pos = s.softplus != 0;
  if (s.dtlow) {
    if constexpr (T == 16) {
      return pos ? launch_wg_t<IO, N, W, T, T, true, false, true>(s, p, ws, st)
                 : launch_wg_t<IO, N, W, T, T, true, false, false>(s, p, ws, st);
    }
    return hipErrorInvalidValue;
  }
  if constexpr (T != 8) {
    if (p.tile_out == 8) {
      return pos ? launch_wg_t<IO, N, W, T, 8, false, false, true>(s, p, ws, st)
                 : launch_wg_t<IO, N, W, T, 8, false, false, false>(s, p, ws, st);
    }
  }
  return pos ? launch_wg_t<IO, N, W, T, T, false, false, true>(s, p, ws, st)
             : launch_wg_t<IO, N, W, T, T, false, false, false>(s, p, ws, st);
}

}  // namespace

// The chained-mode waits' status word of each device (a copy per GPU).
__device__ uint32_t s6_wait_status;

uint32_t* wait_status_ptr() {
  constexpr int kMaxDevices = 64;
  static uint32_t* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(s6_wait_status)) != hipSuccess) return nullptr;
    addr[dev] = static_cast<uint32_t*>(p);
  }
  return addr[dev];
}

hipError_t take_wait_status(hipStream_t stream, uint32_t* value) {
  *value = 0;
  uint32_t* p = wait_status_ptr();
  if (p == nullptr) return hipErrorInvalidSymbol;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  e = hipMemcpy(value, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  if (*value != 0) {
    const uint32_t zero = 0;
    e = hipMemcpy(p, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
  }
  return e;
}

bool wg_supported(int64_t N) { return N == 16 || N == 8; }
int wg_waves(int64_t N) {
  if (N == 16 && option(kOptWgWaves) == 4) return 4;
  return N == 16 ? 8 : 4;
}
int wg_tile(int64_t) { return S6_WG_TILE; }

bool fused_dt_supported(int64_t N, int64_t R, int io) {
  const int64_t e = io == kIoBF16 ? 2 : 4;
  return wg_supported(N) && S6_WG_TILE == 16 && R >= 1 && (R * e) % 16 == 0 && R * e <= 64 * kDtSlices;
}

hipError_t launch_scan_wg(const ScanArgs& s, const ScanPlan& p, int io, int N, void* ws, hipStream_t st, bool cplx) {
  const bool bf = io == kIoBF16;
  if (N == 16 && p.waves == 8)
    return bf ? launch_wg_fdt<uint16_t, 16, 8, S6_WG_TILE>(s, p, cplx, ws, st)
              : launch_wg_fdt<float, 16, 8, S6_WG_TILE>(s, p, cplx, ws, st);
  if (N == 16 && p.waves == 4)
    return bf ? launch_wg_fdt<uint16_t, 16, 4, S6_WG_TILE>(s, p, cplx, ws, st)
              : launch_wg_fdt<float, 16, 4, S6_WG_TILE>(s, p, cplx, ws, st);
  if (N == 8)
    return bf ? launch_wg_fdt<uint16_t, 8, 4, S6_WG_TILE>(s, p, cplx, ws, st)
              : launch_wg_fdt<float, 8, 4, S6_WG_TILE>(s, p, cplx, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace s6

// scan_wp.hip -- wave-private forward selective scan on gfx950 (real diagonal A).
//
// One wave owns CW = 64 / P whole channels of one batch row for a whole
// sequence (or one chunk of it): the P = N / 2 lanes of a channel hold two of
// its states each (lane l: channel l / P of the wave, states 2 (l % P) and
// 2 (l % P) + 1), so the wave never waits for another wave.  Everything it needs
// for a tile of T tokens goes through its own LDS, in program order:
//   front    lane l computes dt = softplus(raw + bias), dt^2, x and z for the
//            T / P tokens l / CW + P i of channel l % CW into the fr slot; the
//            B_t / C_t elements it loaded (shared by all channels:
//            "Mamba 状态空间模型原理与 Transformer 对比", section 3.2) go to the bc
//            slot as (B, B, C, C) per token and state pair;
//   scan     every lane advances its two states over the tile (section 2.1
//            eq. (2) discretisation, eq. (3a) recurrence) and writes its partial
//            readout C_t,2g h_t,2g + C_t,2g+1 h_t,2g+1 (eq. (3b)) to yp;
//   epilogue lane l sums the P partials of its tokens in state order, adds
//            Dskip x, multiplies by SiLU(z) and makes one store per (token, channel).
// The expanded (batch, L, D, N) state never leaves VGPRs (section 4.1).
//
// A workgroup is one wave.  Its LDS (12 KB for N = 16) lets twelve waves, three
// per SIMD, share a CU, which is what hides the latencies of the per-token chains
// (exp, select, recurrence FMA) and of LDS.  The P waves of a 64-channel block
// read and write the same 128-byte lines of every token row; workgroup ids are
// mapped so that they run on one XCD (ids are dealt to the XCDs in turn) and
// share its L2.
//
// Sequences too long for the number of channel blocks to fill the GPU are cut
// into chunks processed in two passes (the parallel scan over chunks of
// section 4.1): chunk end states from zero with the chunk's sum of dt, a carry
// pass composing them (the chunk's product of Abar is e^{A sum dt} because A
// does not vary in time), then every chunk again from its exact carry-in.
// Global loads run two tiles ahead through bounds-checked buffer resources based
// at the chunk, so tails need no branches.
#include <utility>

#include "s6_device.h"
#include "s6_internal.h"

namespace s6 {
namespace {

#ifndef S6_WP_TILE
#define S6_WP_TILE 16  // tokens per tile (N = 8)
#endif
#ifndef S6_WP_TILE16
#define S6_WP_TILE16 16  // tokens per tile (N = 16)
#endif
#ifndef S6_WP_BATCH
#define S6_WP_BATCH 2  // tokens whose input terms are computed together in the scan
#endif
#ifndef S6_WP_TREE
#define S6_WP_TREE 0  // 1: pairwise sum of the partial readouts
#endif
#ifndef S6_WP_WGW
#define S6_WP_WGW 1  // waves per workgroup (a divisor of N / 2); each owns its channels
#endif
#ifndef S6_WP_LDAUX
#define S6_WP_LDAUX 0  // cache policy bits of the per-token row loads
#endif
#ifndef S6_WP_STAUX
#define S6_WP_STAUX 0  // cache policy bits of the output stores
#endif
#ifndef S6_WP_PD
#define S6_WP_PD 4  // tiles of global loads in flight per wave (N = 16)
#endif
#ifndef S6_WP_YPSINGLE
#define S6_WP_YPSINGLE 1  // partial readouts stored one token at a time
#endif
#ifndef S6_WP_WPE
#define S6_WP_WPE 3  // occupancy hint: waves per SIMD
#endif

constexpr int32_t kWpBufferDword3 = 0x00020000;  // raw (untyped) buffer access on the gfx9 family
constexpr uint32_t kWpOutOfRange = 0x80000000u;  // offset beyond every buffer: loads 0, stores dropped

// Passes of the wave-private engine.
enum WpMode { kWpFull = 0, kWpAgg = 1, kWpOut = 2 };

struct WpArgs {
  ScanArgs s;
  int32_t nblk;   // 64-channel blocks per batch row
  int32_t units;  // (chunk, batch row, block) units of this launch
};

// Values that are the same in every lane, kept in scalar registers (the
// compiler cannot always prove it, and a buffer resource in vector registers
// costs a loop over the lanes at every access).
__device__ __forceinline__ uint32_t wp_uniform(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ const char* wp_uniform(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = wp_uniform((uint32_t)v), hi = wp_uniform((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(lo | (hi << 32));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wp_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kWpBufferDword3);
}

// A 16-byte LDS read whose fourth component the caller does not use: the empty
// asm keeps the compiler from narrowing it to a 12-byte read, which costs about
// twice the LDS cycles of a 16-byte one on gfx950 (measured).
#ifndef S6_WP_READ16
#define S6_WP_READ16 0
#endif
__device__ __forceinline__ float4 lds_read16(const float4* p) {
  float4 v = *p;
  if (S6_WP_READ16) asm volatile("" : "+v"(v.w));
  return v;
}

// Orders this wave's LDS accesses across the phases of a tile: its lanes
// exchange data through LDS, which serves one wave's accesses in order, so only
// the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <typename IO>
struct WpIo;
template <>
struct WpIo<uint16_t> {
  static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, S6_WP_LDAUX);
  }
  static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw << 16); }
  static __device__ __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, S6_WP_STAUX);
  }
};
template <>
struct WpIo<float> {
  static __device__ __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, S6_WP_LDAUX);
  }
  static __device__ __forceinline__ float widen(uint32_t raw) { return __uint_as_float(raw); }
  static __device__ __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, S6_WP_STAUX);
  }
};

typedef unsigned int wp_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int wp_u32x4 __attribute__((ext_vector_type(4)));

// K consecutive dwords at byte offset off (buffer loads of 4, 8 or 16 bytes).
template <int K>
__device__ __forceinline__ void load_dwords(uint32_t (&w)[K], __amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (K == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (K == 2) {
    const wp_u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v.x;
    w[1] = v.y;
  } else {
    static_assert(K % 4 == 0, "B/C staging width");
#pragma unroll
    for (int q = 0; q < K; q += 4) {
      const wp_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * (q / 4), 0, 0);
      w[q] = v.x;
      w[q + 1] = v.y;
      w[q + 2] = v.z;
      w[q + 3] = v.w;
    }
  }
}

template <typename IO, int N, int T, int MODE, bool SP>
struct WpScan {
  static constexpr int S = 2;            // states per lane
  static constexpr int P = N / S;        // lanes per channel = waves per 64-channel block
  static constexpr int CW = 64 / P;      // channels per wave
  static constexpr int TQ = T / P;       // front-end / epilogue tokens per lane per tile
  static constexpr int NQ = T * P / 64;  // (token, state pair) B/C chunks staged per lane per tile
  static constexpr uint32_t kIo = sizeof(IO);
  static constexpr int DPC = 2 * (int)kIo / 4;  // dwords of B (or C) per chunk: a state pair
  static_assert(N % S == 0 && T % P == 0 && (T * P) % 64 == 0 && T % 2 == 0, "tile shape");
  // the phases of a tile need at least two parts: the epilogue of a part reads
  // partial readouts that the scan of the next part leaves alone
  static_assert(T / P >= 2, "at least two token slots per lane and tile");
  static_assert(P == 8 || P == 4, "partial-readout layout");
  static constexpr bool kOut = MODE != kWpAgg;
  // Partial readouts of one token: P floats per channel, 64 per row.  For P = 8
  // the two 16-byte halves of a channel are swapped for channels 4..7, and odd
  // rows are rotated by half a row (position ^ 32), so that the epilogue's
  // 16-byte reads (lane = channel, eight or sixteen lanes of two consecutive
  // rows per LDS cycle) and the scan's 4-byte writes touch distinct banks
  // without padding: 12 KB of LDS per wave, so that twelve waves fit a CU.
  static constexpr int YS = 64;
  static __device__ __forceinline__ int ypos(int c, int g) {
    if constexpr (P == 8) return 4 * (2 * c + ((g >> 2) ^ ((c >> 2) & 1))) + (g & 3);
    return 4 * c + g;
  }

  struct Lds {
    float4 fr[2][T][CW];             // (dt, dt / 2 (softplus) or dt^2, x, z) per (token, channel)
    float4 bc[2][T][P];              // (B_2g, B_2g+1, C_2g, C_2g+1) per (token, state pair g)
    float yp[kOut ? T : 1][YS];      // partial readouts per token (layout: ypos)
    float sdt[MODE == kWpAgg ? 64 : 1];  // chunk sums of dt per lane
  };

  struct Regs {  // raw prefetched global data of one tile
    uint32_t dl[TQ], uu[TQ], zz[TQ];
    uint32_t bw[NQ][DPC], cw[NQ][DPC];
  };

  const WpArgs& A;
  Lds& sm;
  const int lane;
  const int sc, sg;  // scan lane: channel within the wave, state pair
  const int fc, fq;  // front / epilogue lane: channel within the wave, first token in the tile
  int64_t b, t0, t1;
  int g;
  int64_t dscan, dfront;
  uint32_t row_bytes;  // one token row of u, delta, z, out in bytes
  // Byte offset of token slot i of a tile (token fq + P i, the front lane's
  // channel) from the tile's first row; out of range for channels >= D.
  uint32_t voff[TQ];
  uint32_t bc_off;  // this lane's B / C chunks from the tile's first row
  int yo0, yo1;     // this lane's partial-readout position in even / odd token rows
  // Chunk bases and spans in bytes; each tile gets buffer resources based at its
  // first row, so that the tile's position costs scalar instructions only and
  // rows past the chunk still fall outside the resource.
  const char *p_u, *p_dl, *p_z, *p_out, *p_B, *p_C;
  uint32_t span, zspan, ospan, bspan;
  // per-state constants of the input weight: A_n log2(e), then (dt from softplus,
  // never negative) the bracket form's 1/A_n and offset, else 1/A_n and A_n / 2
  float a2[S], ka[S], k2[S], h[S];
  float bias, dskip;
  float dsum, dcomp;  // compensated sum of dt (first pass of the split scan)

  __device__ WpScan(const WpArgs& a, Lds& s)
      : A(a),
        sm(s),
        lane(threadIdx.x & 63),
        sc((threadIdx.x & 63) / P),
        sg((threadIdx.x & 63) % P),
        fc((threadIdx.x & 63) % CW),
        fq((threadIdx.x & 63) / CW) {
    yo0 = ypos(sc, sg);
    yo1 = P == 8 ? yo0 ^ 32 : yo0;
  }

  __device__ __forceinline__ int tile_valid(int k) const {
    const int64_t tk = t0 + (int64_t)k * T;
    const int64_t r = t1 - tk;
    return r <= 0 ? 0 : (r >= T ? T : (int)r);
  }

  // Global loads of tile k (rows past the chunk and channels past D read zero).
  // B / C: lane l stages the chunks NQ l + q of the tile, chunk = (token, state
  // pair), i.e. the state pair's two elements, contiguous in memory.
  // Buffer resource of tile k of a tensor whose chunk starts at base and spans span bytes.
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t span, uint32_t off) {
    // spans are below 2^31: a signed difference clamped at zero (scalar max, where
    // an unsigned saturating subtraction would be a vector instruction)
    const int32_t left = (int32_t)span - (int32_t)off;
    return wp_rsrc(base + off, (uint32_t)(left > 0 ? left : 0));
  }

  __device__ __forceinline__ void load(Regs& r, int k) const {
    const uint32_t toff = (uint32_t)(k * T) * row_bytes;
    const __amdgpu_buffer_rsrc_t r_dl = tile_rsrc(p_dl, span, toff), r_u = tile_rsrc(p_u, span, toff);
    const __amdgpu_buffer_rsrc_t r_z = tile_rsrc(p_z, zspan, toff);
#pragma unroll
    for (int i = 0; i < TQ; ++i) {
      r.dl[i] = WpIo<IO>::load(r_dl, voff[i]);
      r.uu[i] = WpIo<IO>::load(r_u, voff[i]);
      if (kOut) r.zz[i] = WpIo<IO>::load(r_z, voff[i]);
    }
    // this lane's NQ chunks are consecutive (chunks NQ l .. NQ l + NQ - 1): one load per tensor
    {
      uint32_t bw[NQ * DPC], cw[NQ * DPC];
      const uint32_t bt = (uint32_t)(k * T * N) * kIo;
      load_dwords<NQ * DPC>(bw, tile_rsrc(p_B, bspan, bt), bc_off);
      if (kOut) load_dwords<NQ * DPC>(cw, tile_rsrc(p_C, bspan, bt), bc_off);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < DPC; ++e) {
          r.bw[q][e] = bw[q * DPC + e];
          if (kOut) r.cw[q][e] = cw[q * DPC + e];
        }
    }
  }

  // Front end of token slot i (token fq + P i) of tile k into slot f.
  __device__ __forceinline__ void front_part(const Regs& r, int k, int f, int i) {
    const int j = fq + P * i;
    const float x = WpIo<IO>::widen(r.uu[i]);
    const float raw = WpIo<IO>::widen(r.dl[i]) + bias;
    const float dt = SP ? softplus(raw) : raw;
    sm.fr[f][j][fc] = make_float4(dt, SP ? 0.5f * dt : dt * dt, x, kOut ? WpIo<IO>::widen(r.zz[i]) : 0.0f);
    if (MODE == kWpAgg) {  // Kahan sum of dt over this lane's valid tokens
      const float yk = (j < tile_valid(k) ? dt : 0.0f) - dcomp;
      const float tk = dsum + yk;
      dcomp = (tk - dsum) - yk;
      dsum = tk;
    }
  }

  // B / C of a tile into slot f as (B, B, C, C) per (token, state pair).
  __device__ __forceinline__ void stage_bc(const Regs& r, int f) {
    float4* bc = &sm.bc[f][0][0];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float b0, b1, c0 = 0.0f, c1 = 0.0f;
      if constexpr (kIo == 2) {
        b0 = bf16_lo(r.bw[q][0]);
        b1 = bf16_hi(r.bw[q][0]);
        if (kOut) {
          c0 = bf16_lo(r.cw[q][0]);
          c1 = bf16_hi(r.cw[q][0]);
        }
      } else {
        b0 = __uint_as_float(r.bw[q][0]);
        b1 = __uint_as_float(r.bw[q][1]);
        if (kOut) {
          c0 = __uint_as_float(r.cw[q][0]);
          c1 = __uint_as_float(r.cw[q][1]);
        }
      }
      bc[NQ * lane + q] = make_float4(b0, b1, c0, c1);
    }
  }

  // Partial readout of token row j.  One 4-byte store per token: the row's
  // position is then an immediate offset (paired stores of two rows would need
  // an address computed per pair).
  __device__ __forceinline__ void yp_store(int j, float v) {
#if S6_WP_YPSINGLE
    *(volatile __attribute__((address_space(3))) float*)(&sm.yp[j][(j & 1) ? yo1 : yo0]) = v;
#else
    sm.yp[j][(j & 1) ? yo1 : yo0] = v;
#endif
  }

  // BT tokens at a time: their input terms (Abar, beta B x) first, then the
  // recurrence steps and partial readouts, so a wave has independent work in flight.
  template <int BT>
  __device__ __forceinline__ void stepb(const float4 (&fv)[BT], const float4 (&bv)[BT], int j) {
    float ab[BT][S], in[BT][S];
#pragma unroll
    for (int q = 0; q < BT; ++q)
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const float x2 = fv[q].x * a2[s];
        ab[q][s] = ex2(x2);
        const float beta = SP ? input_weight_pos(ab[q][s], fv[q].y, ka[s], k2[s])
                              : input_weight(ab[q][s], x2, fv[q].x, fv[q].y, ka[s], k2[s]);
        in[q][s] = beta * ((s == 0 ? bv[q].x : bv[q].y) * fv[q].z);
      }
#pragma unroll
    for (int q = 0; q < BT; ++q) {
      h[0] = __builtin_fmaf(ab[q][0], h[0], in[q][0]);
      h[1] = __builtin_fmaf(ab[q][1], h[1], in[q][1]);
      if (kOut) yp_store(j + q, __builtin_fmaf(bv[q].w, h[1], bv[q].z * h[0]));
    }
  }

  __device__ __forceinline__ void step1(const float4& fv, const float4& bv, int j) {
    float y = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float x2 = fv.x * a2[s];
      const float abar = ex2(x2);
      const float beta = SP ? input_weight_pos(abar, fv.y, ka[s], k2[s])
                            : input_weight(abar, x2, fv.x, fv.y, ka[s], k2[s]);
      h[s] = __builtin_fmaf(abar, h[s], beta * ((s == 0 ? bv.x : bv.y) * fv.z));
      y = s == 0 ? bv.z * h[0] : __builtin_fmaf(bv.w, h[1], y);
    }
    if (kOut) yp_store(j, y);
  }

  // Recurrence over rows [P p, P p + P) of a full tile in slot f; partial readouts to yp.
  __device__ __forceinline__ void scan_part(int f, int p) {
    constexpr int BT = S6_WP_BATCH;
    static_assert(P % BT == 0, "scan batch");
    const int j0 = P * p;
    float4 fv[BT], bv[BT], fn[BT], bn[BT];
#pragma unroll
    for (int q = 0; q < BT; ++q) {
      fv[q] = lds_read16(&sm.fr[f][j0 + q][sc]);
      bv[q] = sm.bc[f][j0 + q][sg];
    }
#pragma unroll
    for (int j = j0; j < j0 + P; j += BT) {
      if (j + BT < j0 + P) {
#pragma unroll
        for (int q = 0; q < BT; ++q) {
          fn[q] = lds_read16(&sm.fr[f][j + BT + q][sc]);
          bn[q] = sm.bc[f][j + BT + q][sg];
        }
      }
      stepb<BT>(fv, bv, j);
      if (j + BT < j0 + P) {
#pragma unroll
        for (int q = 0; q < BT; ++q) {
          fv[q] = fn[q];
          bv[q] = bn[q];
        }
      }
    }
  }

  // The same rows of a partial tile with nv valid tokens.
  __device__ __forceinline__ void scan_part_tail(int f, int p, int nv) {
    const int j1 = P * p + P < nv ? P * p + P : nv;
    for (int j = P * p; j < j1; ++j) step1(lds_read16(&sm.fr[f][j][sc]), sm.bc[f][j][sg], j);
  }

  // Readout sum, skip, gate and store of token slot i (token fq + P i) of tile k
  // (rows past the chunk and channels past D fall outside the output buffer).
  __device__ __forceinline__ void epi_part(int k, int f, int i) {
    if (!kOut) return;
    const int j = fq + P * i;
    const float4* row = reinterpret_cast<const float4*>(&sm.yp[j][0]);
    const int sw = P == 8 ? 32 * (j & 1) : 0;
    const float4 lo = row[(ypos(fc, 0) ^ sw) / 4];
    float y = ((lo.x + lo.y) + lo.z) + lo.w;  // the P partials in state order
    if constexpr (P == 8) {
      const float4 hi = row[(ypos(fc, 4) ^ sw) / 4];
      y = (((y + hi.x) + hi.y) + hi.z) + hi.w;
    }
    const float4 fv = lds_read16(&sm.fr[f][j][fc]);
    const float o = s6::epilogue(y, fv.z, dskip, A.s.z != nullptr, fv.w);
    WpIo<IO>::store(o, tile_rsrc(p_out, ospan, (uint32_t)(k * T) * row_bytes), voff[i]);
  }

  // Raw global data of PD tiles is in flight per wave (a ring of registers): the
  // loads must cover the HBM latency, and a wave's requests are small (16-byte
  // pieces of token rows), so only many in flight at once keep HBM busy.
  static constexpr int PD = N == 16 ? S6_WP_PD : 2;

  // One tile k (full when FULL, else nv valid tokens) with the front end of tile
  // k+1 (raw data in ring slot RS) and the epilogue of tile k-1's last rows,
  // phased so that every LDS round trip has other work between its write and
  // its read: for each part p of P rows, scan(k, p); epilogue of the part before
  // (tile k-1's last part when p = 0); front end of tile k+1's part p.  Then the
  // slot is refilled with tile k+1+PD.
  template <bool FULL, int RS>
  __device__ __forceinline__ void tile(Regs (&ring)[PD], int k, int nv) {
    const int f = k & 1;
    Regs& r = ring[RS];
#pragma unroll
    for (int p = 0; p < TQ; ++p) {
      wave_lds_order();
      if (FULL) scan_part(f, p);
      else scan_part_tail(f, p, nv);
      wave_lds_order();
      if (p == 0) {
        if (k > 0) epi_part(k - 1, f ^ 1, TQ - 1);
      } else {
        epi_part(k, f, p - 1);
      }
      wave_lds_order();
      front_part(r, k + 1, f ^ 1, p);
      if (p == 0) stage_bc(r, f ^ 1);
    }
    load(r, k + 1 + PD);
  }

  // PD consecutive full tiles from k (a multiple of PD): tile k+i reads ring slot (i+1) % PD.
  template <int... I>
  __device__ __forceinline__ void tiles_full(Regs (&ring)[PD], int k, std::integer_sequence<int, I...>) {
    (tile<true, (I + 1) % PD>(ring, k + I, T), ...);
  }
  // The rem <= PD tiles from k, full or not.
  template <int... I>
  __device__ __forceinline__ void tiles_tail(Regs (&ring)[PD], int k, int rem, std::integer_sequence<int, I...>) {
    ((rem > I ? tile<false, (I + 1) % PD>(ring, k + I, tile_valid(k + I)) : void()), ...);
  }

  // This lane's two states from / to p, the first of them in a state array.
  __device__ __forceinline__ void get_state(const float* p) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    h[0] = v.x;
    h[1] = v.y;
  }
  __device__ __forceinline__ void put_state(float* p) const {
    *reinterpret_cast<float2*>(p) = make_float2(h[0], h[1]);
  }

  // unit: (chunk, batch row, 64-channel block) in that order of significance; kw: wave of the block
  __device__ void run(int unit, int kw) {
    const int G = A.s.nchunks;
    const int nb = A.nblk;
    g = MODE == kWpFull ? 0 : unit / (int)(A.s.batch * nb);
    b = (unit / nb) % A.s.batch;
    const int64_t d0 = (int64_t)(unit % nb) * 64 + CW * kw;
    dscan = d0 + sc;
    dfront = d0 + fc;
    const bool svalid = dscan < A.s.D, fvalid = dfront < A.s.D;
    t0 = (int64_t)g * A.s.chunk_len;
    t1 = t0 + A.s.chunk_len < A.s.L ? t0 + A.s.chunk_len : A.s.L;
    // an aggregate may skip the part of its chunk that cannot reach the chunk's end
    if (MODE == kWpAgg && A.s.agg_start) t0 += A.s.agg_start[((size_t)b * G + g) * nb + unit % nb];
    row_bytes = wp_uniform((uint32_t)(A.s.D * kIo));
    {
      const uint32_t chan_off = fvalid ? (uint32_t)(dfront * kIo) : kWpOutOfRange;
#pragma unroll
      for (int i = 0; i < TQ; ++i) voff[i] = chan_off + (uint32_t)(fq + P * i) * row_bytes;
      bc_off = (uint32_t)(2 * NQ * lane) * kIo;
      const size_t row0 = ((size_t)b * A.s.L + t0);
      span = (uint32_t)((t1 - t0) * A.s.D * kIo);
      bspan = (uint32_t)((t1 - t0) * N * kIo);
      zspan = A.s.z ? span : 0u;
      ospan = kOut ? span : 0u;
      p_u = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.u) + row0 * A.s.D));
      p_dl = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.delta) + row0 * A.s.D));
      p_z = A.s.z ? wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.z) + row0 * A.s.D)) : p_u;
      p_out = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.out) + row0 * A.s.D));
      p_B = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.B) + row0 * N));
      p_C = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.C) + row0 * N));
      span = wp_uniform(span);
      bspan = wp_uniform(bspan);
      zspan = wp_uniform(zspan);
      ospan = wp_uniform(ospan);
    }
    const int n0 = S * sg;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float a = svalid ? A.s.A[dscan * N + n0 + s] : -1.0f;
      a2[s] = a * kLog2e;
      ka[s] = SP ? bracket_ka(a) : rcp(a);
      k2[s] = SP ? bracket_kc(ka[s]) : 0.5f * a;
      h[s] = 0.0f;
    }
    bias = (fvalid && A.s.bias) ? A.s.bias[dfront] : 0.0f;
    dskip = (fvalid && A.s.dskip) ? A.s.dskip[dfront] : 0.0f;
    dsum = 0.0f;
    dcomp = 0.0f;
    // state entering the chunk
    if (MODE == kWpFull) {
      if (A.s.h0 && svalid) get_state(A.s.h0 + ((size_t)b * A.s.D + dscan) * N + n0);
    } else if (MODE == kWpOut) {
      if (svalid) get_state(A.s.agg_h + (((size_t)b * G + g) * A.s.D + dscan) * N + n0);
    }
    // tile pipeline: global loads PD tiles ahead, two fr / bc slots
    const int ntiles = (int)((t1 - t0 + T - 1) / T);
    const int nfull = (int)((t1 - t0) / T);
    Regs ring[PD];
#pragma unroll
    for (int q = 0; q < PD; ++q) load(ring[q], q);
#pragma unroll
    for (int i = 0; i < TQ; ++i) front_part(ring[0], 0, 0, i);
    stage_bc(ring[0], 0);
    load(ring[0], PD);
    int k = 0;
    for (; k + PD <= nfull; k += PD) tiles_full(ring, k, std::make_integer_sequence<int, PD>{});
    tiles_tail(ring, k, ntiles - k, std::make_integer_sequence<int, PD>{});  // the last (up to PD) tiles
    wave_lds_order();
    if (ntiles > 0) epi_part(ntiles - 1, (ntiles - 1) & 1, TQ - 1);

    // the chunk's end
    if (MODE == kWpFull) {
      if (A.s.last && svalid) put_state(A.s.last + ((size_t)b * A.s.D + dscan) * N + n0);
    } else if (MODE == kWpAgg) {
      if (svalid) put_state(A.s.agg_h + (((size_t)b * G + g) * A.s.D + dscan) * N + n0);
      // dt sum of the front lane's channel over its P lanes (fq = 0 .. P-1), in order
      sm.sdt[lane] = dsum;
      wave_lds_order();
      if (fq == 0 && fvalid) {
        float tot = 0.0f;
#pragma unroll
        for (int q = 0; q < P; ++q) tot += sm.sdt[fc + CW * q];
        A.s.agg_s[((size_t)b * G + g) * A.s.D + dfront] = tot;
      }
    } else {  // kWpOut
      if (g == G - 1 && A.s.last && svalid) put_state(A.s.last + ((size_t)b * A.s.D + dscan) * N + n0);
    }
  }
};

// WGW waves per workgroup, each on its own channels.  Workgroup ids go to the
// XCDs in turn (id % 8); the P waves of a unit get workgroup ids that are
// consecutive among one XCD's ids (for WGW = P, one workgroup is one unit).
template <typename IO, int N, int T, int MODE, bool SP>
__global__ __launch_bounds__(64 * S6_WP_WGW, S6_WP_WPE) void scan_wp_kernel(WpArgs a) {
  using K = WpScan<IO, N, T, MODE, SP>;
  constexpr int WGW = S6_WP_WGW < K::P ? S6_WP_WGW : K::P;
  constexpr int WPU = K::P / WGW;  // workgroups per unit
  static_assert(K::P % WGW == 0, "waves per workgroup");
  __shared__ typename K::Lds sm[WGW];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int id = blockIdx.x;
  const int m = id >> 3;
  const int unit = WPU == 1 ? id : (m / WPU) * 8 + (id & 7);
  if (unit >= a.units) return;
  K k(a, sm[wv]);
  k.run(unit, (WPU == 1 ? 0 : (m % WPU)) * WGW + wv);
}

template <typename IO, int N, int MODE>
void launch_wp_pass(const WpArgs& a, hipStream_t st) {
  constexpr int WGW = S6_WP_WGW < N / 2 ? S6_WP_WGW : N / 2;
  constexpr int WPU = (N / 2) / WGW;
  const unsigned grid = WPU == 1 ? (unsigned)a.units : (unsigned)((a.units + 7) / 8 * 8 * WPU);
  if (a.s.softplus)
    hipLaunchKernelGGL((scan_wp_kernel<IO, N, (N == 16 ? S6_WP_TILE16 : S6_WP_TILE), MODE, true>), dim3(grid), dim3(64 * WGW), 0, st, a);
  else
    hipLaunchKernelGGL((scan_wp_kernel<IO, N, (N == 16 ? S6_WP_TILE16 : S6_WP_TILE), MODE, false>), dim3(grid), dim3(64 * WGW), 0, st, a);
}

template <typename IO>
hipError_t launch_wp_mixed(const ScanArgs& s, int32_t wp1_units, hipStream_t st);

template <typename IO, int N>
hipError_t launch_wp_t(const ScanArgs& s, const ScanPlan& p, void* ws, hipStream_t st) {
  if (p.wp1_units > 0) return (N == 16 && !p.split) ? launch_wp_mixed<IO>(s, p.wp1_units, st) : hipErrorInvalidValue;
  WpArgs a;
  a.s = s;
  a.nblk = (int32_t)((s.D + 63) / 64);
  const int32_t rows = (int32_t)(s.batch * a.nblk);
  if (!p.split) {
    a.units = rows;
    launch_wp_pass<IO, N, kWpFull>(a, st);
  } else {
    a.s.agg_h = static_cast<float*>(ws);
    a.s.agg_s = a.s.agg_h + (size_t)s.batch * p.nchunks * s.D * N;
    int32_t* start = reinterpret_cast<int32_t*>(a.s.agg_s + (size_t)s.batch * p.nchunks * s.D);
    if (launch_agg_start(a.s, sizeof(IO) == 2 ? kIoBF16 : kIoF32, N, start, st)) a.s.agg_start = start;
    a.units = rows * (p.nchunks - 1);
    launch_wp_pass<IO, N, kWpAgg>(a, st);
    const hipError_t ce = launch_chunk_carry(a.s, N, st);
    if (ce != hipSuccess) return ce;
    a.units = rows * p.nchunks;
    launch_wp_pass<IO, N, kWpOut>(a, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- one state per lane (N = 16)
//
// A second layout for mixed launches.  A wave owns 4 channels of one batch row
// for the whole sequence: the 16 lanes of row r (lanes 16r .. 16r+15, one DPP
// row) hold the 16 states of channel r, one each, so its work is half a
// two-states-per-lane wave's.  Lane 16r + j also owns token j of every 16-token
// tile of channel r: it loads delta, u and z, computes dt, and after the scan
// sums the row's 16 partial readouts of that token (eq. (3b)) in state order,
// adds Dskip x, multiplies by SiLU(z) and makes the store.  The scan of token j
// reads dt and x from lane 16r + j of its own row with a DPP row broadcast
// (row_newbcast:j), which the compiler folds into the multiplies that use them;
// B_t and C_t (shared by all channels, section 3.2) are staged once per tile in
// LDS as (B, C) pairs per state.  The guarded input weight's series branch is
// written dt (1 + x ln2 / 2) with x = dt A log2(e), the same value as
// dt + dt^2 A / 2, so that dt enters it only through a multiply.
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf,
                                                               false));
}

template <typename IO, bool SP>
struct Wp1Scan {
  static constexpr int N = 16, T = 16, CW1 = 4;
  static constexpr int PD = 3;  // tiles of global loads in flight
  static constexpr uint32_t kIo = sizeof(IO);
  static constexpr int KB = (int)kIo;  // dwords of B (or C) a lane stages per tile: four elements
  // Partial readouts: 64 floats per token (channel-major), rows 68 floats apart so
  // that the epilogue's 16-byte reads of consecutive tokens touch distinct banks.
  static constexpr int YS = 68;
  static constexpr float kHalfLn2 = 0.5f * kLn2;

  struct Lds {
    float2 bc[T][N];  // (B, C) per (token, state)
    float yp[T][YS];  // partial readouts per (token, channel * 16 + state)
  };
  struct Regs {  // raw prefetched global data of one tile: this lane's token, its four B / C elements
    uint32_t dl, uu, zz;
    uint32_t bw[KB], cw[KB];
  };

  const WpArgs& A;
  Lds& sm;
  const int lane, r, n;  // channel within the wave (row), state = token of the row's front lane
  int64_t L;
  uint32_t row_bytes, voff, bc_off;
  const char *p_u, *p_dl, *p_z, *p_out, *p_B, *p_C;
  uint32_t span, zspan, bspan;
  float a2, ka, kc, h, bias, dskip;
  float fdt, fdh, fx, fz;  // front end of this lane's token of the current tile (fdh = dt / 2)

  __device__ Wp1Scan(const WpArgs& a, Lds& s)
      : A(a), sm(s), lane(threadIdx.x & 63), r((threadIdx.x & 63) >> 4), n(threadIdx.x & 15) {}

  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, uint32_t span, uint32_t off) {
    const int32_t left = (int32_t)span - (int32_t)off;
    return wp_rsrc(base + off, (uint32_t)(left > 0 ? left : 0));
  }

  __device__ __forceinline__ void load(Regs& g, int k) const {
    const uint32_t toff = (uint32_t)(k * T) * row_bytes;
    g.dl = WpIo<IO>::load(tile_rsrc(p_dl, span, toff), voff);
    g.uu = WpIo<IO>::load(tile_rsrc(p_u, span, toff), voff);
    g.zz = WpIo<IO>::load(tile_rsrc(p_z, zspan, toff), voff);
    const uint32_t bt = (uint32_t)(k * T * N) * kIo;
    load_dwords<KB>(g.bw, tile_rsrc(p_B, bspan, bt), bc_off);
    load_dwords<KB>(g.cw, tile_rsrc(p_C, bspan, bt), bc_off);
  }

  __device__ __forceinline__ void front(const Regs& g) {
    fx = WpIo<IO>::widen(g.uu);
    fz = WpIo<IO>::widen(g.zz);
    const float raw = WpIo<IO>::widen(g.dl) + bias;
    fdt = SP ? softplus(raw) : raw;
    fdh = 0.5f * fdt;
  }

  // B / C of a tile: lane l stages elements 4l .. 4l+3 of the (token, state)
  // block, i.e. token l / 4, states 4 (l % 4) .. 4 (l % 4) + 3.
  __device__ __forceinline__ void stage_bc(const Regs& g) {
    float bv[4], cv[4];
    if constexpr (kIo == 2) {
      bv[0] = bf16_lo(g.bw[0]);
      bv[1] = bf16_hi(g.bw[0]);
      bv[2] = bf16_lo(g.bw[1]);
      bv[3] = bf16_hi(g.bw[1]);
      cv[0] = bf16_lo(g.cw[0]);
      cv[1] = bf16_hi(g.cw[0]);
      cv[2] = bf16_lo(g.cw[1]);
      cv[3] = bf16_hi(g.cw[1]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bv[q] = __uint_as_float(g.bw[q]);
        cv[q] = __uint_as_float(g.cw[q]);
      }
    }
    float4* dst = reinterpret_cast<float4*>(&sm.bc[lane >> 2][4 * (lane & 3)]);
    dst[0] = make_float4(bv[0], cv[0], bv[1], cv[1]);
    dst[1] = make_float4(bv[2], cv[2], bv[3], cv[3]);
  }

  // Input terms of token J (eq. (2)): Abar and beta B x for this lane's state.
  template <int J>
  __device__ __forceinline__ void input_terms(const float2 v, float& ab, float& in) const {
    const float x2 = row_bcast<J>(fdt) * a2;
    ab = ex2(x2);
    float beta;
    if constexpr (SP) {  // bracket form (dt >= 0), its bound written (dt / 2)(1 + Abar): dt through a multiply
      beta = fminf(__builtin_fmaf(ab, ka, kc), row_bcast<J>(fdh) * (1.0f + ab));
    } else {
      const float big = __builtin_fmaf(ab, ka, -ka);
      const float small = row_bcast<J>(fdt) * __builtin_fmaf(x2, kHalfLn2, 1.0f);
      beta = fabsf(x2) < kPhiSeriesX2 ? small : big;
    }
    in = beta * (row_bcast<J>(fx) * v.x);
  }
  // Tokens J and J+1: both tokens' input terms, then the two recurrence steps
  // (eq. (3a)) and partial readouts C h (eq. (3b)) to LDS.
  template <int J>
  __device__ __forceinline__ void pair(const float2 (&v)[T]) {
    float ab0, in0, ab1, in1;
    input_terms<J>(v[J], ab0, in0);
    input_terms<J + 1>(v[J + 1], ab1, in1);
    h = __builtin_fmaf(ab0, h, in0);
    sm.yp[J][lane] = v[J].y * h;
    h = __builtin_fmaf(ab1, h, in1);
    sm.yp[J + 1][lane] = v[J + 1].y * h;
  }
  template <int J>
  __device__ __forceinline__ void single(const float2 (&v)[T]) {
    float ab, in;
    input_terms<J>(v[J], ab, in);
    h = __builtin_fmaf(ab, h, in);
    sm.yp[J][lane] = v[J].y * h;
  }
  template <int... P>
  __device__ __forceinline__ void pairs(const float2 (&v)[T], std::integer_sequence<int, P...>) {
    (pair<2 * P>(v), ...);
  }
  template <int... J>
  __device__ __forceinline__ void singles(const float2 (&v)[T], int nv, std::integer_sequence<int, J...>) {
    ((J < nv ? single<J>(v) : void()), ...);
  }
  // The tile's 16 tokens (the first nv of them when not FULL); the (B, C) pairs
  // of all 16 are read from LDS first, so the reads' latency is paid once.
  template <bool FULL>
  __device__ __forceinline__ void scan(int nv) {
    float2 v[T];
#pragma unroll
    for (int j = 0; j < T; ++j) v[j] = sm.bc[j][n];
    if (FULL) pairs(v, std::make_integer_sequence<int, T / 2>{});
    else singles(v, nv, std::make_integer_sequence<int, T>{});
  }

  // This lane's token of tile k: the 16 partials in state order, skip, gate, store.
  __device__ __forceinline__ void epilogue(int k) {
    const float4* row = reinterpret_cast<const float4*>(&sm.yp[n][16 * r]);
    const float4 p0 = row[0], p1 = row[1], p2 = row[2], p3 = row[3];
    float y = ((p0.x + p0.y) + p0.z) + p0.w;
    y = (((y + p1.x) + p1.y) + p1.z) + p1.w;
    y = (((y + p2.x) + p2.y) + p2.z) + p2.w;
    y = (((y + p3.x) + p3.y) + p3.z) + p3.w;
    const float o = s6::epilogue(y, fx, dskip, A.s.z != nullptr, fz);
    WpIo<IO>::store(o, tile_rsrc(p_out, span, (uint32_t)(k * T) * row_bytes), voff);
  }

  // Tile k (full when FULL) from ring slot RS, then that slot refilled with tile k + PD.
  template <bool FULL, int RS>
  __device__ __forceinline__ void tile(Regs (&ring)[PD], int k, int nv) {
    front(ring[RS]);
    stage_bc(ring[RS]);
    load(ring[RS], k + PD);
    wave_lds_order();
    scan<FULL>(nv);
    wave_lds_order();
    epilogue(k);
    wave_lds_order();
  }
  template <int... I>
  __device__ __forceinline__ void tiles_full(Regs (&ring)[PD], int k, std::integer_sequence<int, I...>) {
    (tile<true, I>(ring, k + I, T), ...);
  }
  template <int... I>
  __device__ __forceinline__ void tiles_tail(Regs (&ring)[PD], int k, int ntiles, std::integer_sequence<int, I...>) {
    ((k + I < ntiles ? tile<false, I>(ring, k + I, (int)(L - (int64_t)(k + I) * T < T ? L - (int64_t)(k + I) * T : T))
                     : void()),
     ...);
  }

  // unit: (batch row, 64-channel block); kw: the wave's group of 4 channels in the block
  __device__ void run(int unit, int kw) {
    const int nb = A.nblk;
    const int64_t b = unit / nb;
    L = A.s.L;
    const int64_t d = (int64_t)(unit % nb) * 64 + CW1 * kw + r;
    const bool valid = d < A.s.D;
    row_bytes = wp_uniform((uint32_t)(A.s.D * kIo));
    voff = valid ? (uint32_t)(d * kIo) + (uint32_t)n * row_bytes : kWpOutOfRange;
    bc_off = (uint32_t)(4 * lane) * kIo;
    const size_t row0 = (size_t)b * A.s.L;
    span = wp_uniform((uint32_t)(A.s.L * A.s.D * kIo));
    bspan = wp_uniform((uint32_t)(A.s.L * N * kIo));
    zspan = A.s.z ? span : 0u;
    p_u = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.u) + row0 * A.s.D));
    p_dl = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.delta) + row0 * A.s.D));
    p_z = A.s.z ? wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.z) + row0 * A.s.D)) : p_u;
    p_out = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.out) + row0 * A.s.D));
    p_B = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.B) + row0 * N));
    p_C = wp_uniform(reinterpret_cast<const char*>(static_cast<const IO*>(A.s.C) + row0 * N));
    const float a = valid ? A.s.A[d * N + n] : -1.0f;
    a2 = a * kLog2e;
    ka = SP ? bracket_ka(a) : rcp(a);
    kc = bracket_kc(ka);
    bias = (valid && A.s.bias) ? A.s.bias[d] : 0.0f;
    dskip = (valid && A.s.dskip) ? A.s.dskip[d] : 0.0f;
    h = (A.s.h0 && valid) ? A.s.h0[((size_t)b * A.s.D + d) * N + n] : 0.0f;
    const int ntiles = (int)((L + T - 1) / T);
    const int nfull = (int)(L / T);
    Regs ring[PD];
#pragma unroll
    for (int q = 0; q < PD; ++q) load(ring[q], q);
    int k = 0;
    for (; k + PD <= nfull; k += PD) tiles_full(ring, k, std::make_integer_sequence<int, PD>{});
    tiles_tail(ring, k, ntiles, std::make_integer_sequence<int, PD>{});
    if (A.s.last && valid) A.s.last[((size_t)b * A.s.D + d) * N + n] = h;
  }
};

// Mixed launch (N = 16, unchunked): the first units2 (batch row, block) units run
// with two states per lane (8 waves each), the rest with one state per lane (16
// waves of half the work each).  With the split chosen so that the launch has 2
// or 3 waves per SIMD (1024 SIMDs), the workgroups dealt last, the one-state
// waves, fill the SIMDs that a launch of two-state waves alone leaves a wave
// short.  Workgroup ids of both parts are mapped XCD by XCD as in scan_wp_kernel.
template <typename IO, bool SP>
__global__ __launch_bounds__(64, 3) void scan_wp_mixed_kernel(WpArgs a, int32_t units2, int32_t grid2) {
  using K2 = WpScan<IO, 16, S6_WP_TILE16, kWpFull, SP>;
  using K1 = Wp1Scan<IO, SP>;
  __shared__ union {
    typename K2::Lds two;
    typename K1::Lds one;
  } sm;
  const int id = blockIdx.x;
  if (id < grid2) {
    const int m = id >> 3;
    const int unit = (m / K2::P) * 8 + (id & 7);
    if (unit >= units2) return;
    K2 k(a, sm.two);
    k.run(unit, m % K2::P);
  } else {
    const int i1 = id - grid2;
    const int m = i1 >> 3;
    const int unit = units2 + (m / 16) * 8 + (i1 & 7);
    if (unit >= a.units) return;
    K1 k(a, sm.one);
    k.run(unit, m % 16);
  }
}

template <typename IO>
hipError_t launch_wp_mixed(const ScanArgs& s, int32_t wp1_units, hipStream_t st) {
  WpArgs a;
  a.s = s;
  a.nblk = (int32_t)((s.D + 63) / 64);
  a.units = (int32_t)(s.batch * a.nblk);
  const int32_t units2 = a.units - wp1_units;
  if (units2 < 0 || wp1_units < 0) return hipErrorInvalidValue;
  // both parts' grids are whole multiples of 8 (one id per XCD in turn)
  const int32_t grid2 = (units2 + 7) / 8 * 8 * 8;
  const int32_t grid1 = (wp1_units + 7) / 8 * 8 * 16;
  if (s.softplus)
    hipLaunchKernelGGL((scan_wp_mixed_kernel<IO, true>), dim3((unsigned)(grid2 + grid1)), dim3(64), 0, st, a, units2,
                       grid2);
  else
    hipLaunchKernelGGL((scan_wp_mixed_kernel<IO, false>), dim3((unsigned)(grid2 + grid1)), dim3(64), 0, st, a, units2,
                       grid2);
  return hipGetLastError();
}

}  // namespace

int wp_tile() { return S6_WP_TILE > S6_WP_TILE16 ? S6_WP_TILE : S6_WP_TILE16; }

hipError_t launch_scan_wp(const ScanArgs& s, const ScanPlan& p, int io, int N, void* ws, hipStream_t st) {
  const bool bf = io == kIoBF16;
  if (N == 16) return bf ? launch_wp_t<uint16_t, 16>(s, p, ws, st) : launch_wp_t<float, 16>(s, p, ws, st);
  if (N == 8) return bf ? launch_wp_t<uint16_t, 8>(s, p, ws, st) : launch_wp_t<float, 8>(s, p, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace s6

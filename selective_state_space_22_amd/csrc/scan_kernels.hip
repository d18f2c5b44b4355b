// scan_kernels.hip -- forward selective scan on gfx950.
//
// Layout (row-major): u, delta, z, out (batch, L, D); B, C (batch, L, N);
// A (D, N); bias, Dskip (D); h0, last_state (batch, D, N).
//
// Mapping: one lane owns one channel d of one batch row and keeps its N
// states in VGPRs for the whole chunk; the 64 lanes of a wave are 64
// consecutive channels, so the per-token loads of u/delta/z and the store of
// out are 64 consecutive elements, and B_t/C_t (shared by all channels,
// "Mamba 状态空间模型原理与 Transformer 对比", section 3.2) are wave-uniform
// scalar loads.  The expanded state (batch, L, D, N) never leaves registers
// (section 4.1: only the (batch, L, D) output returns to HBM).
//
// When batch*D alone cannot fill the GPU, L is cut into chunks (the parallel
// scan of section 4.1, over chunks): each chunk except the last runs the
// recurrence from a zero state and keeps only its end state b_g and the sum
// of dt over the chunk; a carry pass composes them in order with the
// associative step h_in(g+1) = e^{A * sum dt_g} h_in(g) + b_g (the product of
// the chunk's Abar is e^{A * sum dt} because A does not vary in time); the
// output pass then reruns every chunk from its exact carry-in.
#include <cstdlib>

#include "s6_device.h"
#include "s6_internal.h"

namespace s6 {

template <typename IO, int N>
struct BCLoader;

// bf16, even N: N/2 wave-uniform 32-bit words per token.
template <int N>
struct BCLoader<uint16_t, N> {
  static __device__ __forceinline__ void load(const uint16_t* __restrict__ p, float (&v)[N]) {
    if constexpr (N % 2 == 0) {
      const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
      for (int j = 0; j < N / 2; ++j) {
        uint32_t x = w[j];
        v[2 * j] = bf16_lo(x);
        v[2 * j + 1] = bf16_hi(x);
      }
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) v[n] = bf16_to_f32(p[n]);
    }
  }
};

template <int N>
struct BCLoader<float, N> {
  static __device__ __forceinline__ void load(const float* __restrict__ p, float (&v)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = p[n];
  }
};

// Chunk end states from a zero start (all chunks but the last).
template <typename IO, int N>
__global__ __launch_bounds__(256) void scan_chunk_state_kernel(ScanArgs a) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t g = blockIdx.z;
  if (d >= a.D) return;
  const int64_t L = a.L, D = a.D;
  const IO* __restrict__ u = static_cast<const IO*>(a.u);
  const IO* __restrict__ dl = static_cast<const IO*>(a.delta);
  const IO* __restrict__ Bp = static_cast<const IO*>(a.B);
  const float bias = a.bias ? a.bias[d] : 0.0f;
  ChanConst<N> cc;
  cc.load(a.A + d * N);
  float h[N];
#pragma unroll
  for (int n = 0; n < N; ++n) h[n] = 0.0f;
  float s = 0.0f, sc = 0.0f;  // compensated sum of dt
  const int64_t t0 = g * a.chunk_len;
  const int64_t t1 = t0 + a.chunk_len < L ? t0 + a.chunk_len : L;
  const bool sp = a.softplus != 0;
  for (int64_t t = t0; t < t1; ++t) {
    const size_t i = ((size_t)b * L + t) * D + d;
    float Bt[N];
    BCLoader<IO, N>::load(Bp + ((size_t)b * L + t) * N, Bt);
    TokenFront f = make_front(load_io(dl, i), bias, sp);
    token_step_state<N>(cc, f, load_io(u, i), Bt, h);
    float yk = f.dt - sc;  // Kahan summation of dt
    float tk = s + yk;
    sc = (tk - s) - yk;
    s = tk;
  }
  const size_t base = ((size_t)b * a.nchunks + g) * D + d;
#pragma unroll
  for (int n = 0; n < N; ++n) a.agg_h[base * N + n] = h[n];
  a.agg_s[base] = s;
}

// Carry pass: one lane per (batch, channel, state), sequential over chunks.
// On exit agg_h[b, g, d, n] holds the state entering chunk g.
template <int N>
__global__ __launch_bounds__(256) void scan_carry_kernel(ScanArgs a) {
  const int64_t lane = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t D = a.D;
  if (lane >= a.batch * D * N) return;
  const int64_t n = lane % N;
  const int64_t d = (lane / N) % D;
  const int64_t b = lane / (N * D);
  const float a2 = a.A[d * N + n] * kLog2e;
  float carry = a.h0 ? a.h0[lane] : 0.0f;
  const int G = a.nchunks;
  // chunks in groups of 16: the group's loads are issued together (they do not depend
  // on the chain), then the chain runs through them in order
  constexpr int kBatch = 16;
  for (int g0 = 0; g0 < G - 1; g0 += kBatch) {
    float sv[kBatch], hv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (g0 + u < G - 1) {
        const size_t base = ((size_t)b * G + g0 + u) * D + d;
        sv[u] = a.agg_s[base];
        hv[u] = a.agg_h[base * N + n];
      }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (g0 + u < G - 1) {
        const size_t base = ((size_t)b * G + g0 + u) * D + d;
        const float decay = ex2(a2 * sv[u]);
        a.agg_h[base * N + n] = carry;
        carry = __builtin_fmaf(decay, carry, hv[u]);
      }
  }
  a.agg_h[(((size_t)b * G + (G - 1)) * D + d) * N + n] = carry;
}

// ---------------------------------------------------------------- aggregate starts
//
// A state entering token t of chunk g reaches the chunk's end multiplied by the
// product of Abar over tokens t..end, e^{A_n S(t)} with S(t) the sum of dt over
// those tokens (eq. (2); A does not vary in time).  With dt >= 0 (softplus) and
// A_n log2(e) S(t) <= -200 for every state of every channel of a 64-channel
// block, that factor is below 2^-200: whatever the chunk holds before t moves
// its end state by less than 2^-200 of that state's size, far below fp32
// rounding.  The aggregate pass then starts at t from zero, and its sum of dt
// (over t..end) makes the carry pass's factor e^{A_n sum dt} underflow to zero,
// so the state entering the chunk is dropped as well, by the same bound.  Only
// with softplus: dt >= 0 keeps the aggregate's own sum of dt (which the carry
// uses) at or above the sum tested here, up to rounding; without it nothing is
// skipped.
// One wave per (batch row, chunk, block) walks back from the chunk's end a tile
// of 16 tokens at a time and records the latest tile start where the bound holds
// for the whole block (0 if it never does).  The walk sums max(raw + bias, 0),
// a lower bound of dt = softplus(raw + bias), so the bound it tests is the
// stronger one, at a few instructions per token; the loads of eight tiles are
// issued together (one wave per SIMD at most: the walk is latency-bound).
constexpr float kAggSkipExp2 = -200.0f;
constexpr int kAggStartTile = 16;
constexpr int kAggStartGroup = 8;  // tiles whose loads are in flight together

template <typename IO>
__global__ __launch_bounds__(64) void agg_start_kernel(ScanArgs a, int32_t N, int32_t nblk, int32_t* start) {
  constexpr int T = kAggStartTile;
  constexpr int GT = kAggStartGroup;
  const int G = a.nchunks;
  const int64_t unit = blockIdx.x;  // (batch row, chunk < G - 1, block), block fastest
  const int64_t blk = unit % nblk;
  const int64_t g = (unit / nblk) % (G - 1);
  const int64_t b = unit / ((int64_t)nblk * (G - 1));
  const int64_t d = blk * 64 + threadIdx.x;
  const bool dv = d < a.D;
  // the channel's slowest decay: the largest A_n log2(e)
  float amax = -__builtin_inff();
  if (dv)
    for (int n = 0; n < N; ++n) amax = fmaxf(amax, a.A[d * N + n] * kLog2e);
  const float bias = (dv && a.bias) ? a.bias[d] : 0.0f;
  // chunks before the last hold chunk_len tokens, a multiple of the tile (checked
  // at the launch): every tile is whole
  const int ntiles = (int)(a.chunk_len / T);
  const IO* chunk = static_cast<const IO*>(a.delta) + ((size_t)b * a.L + (size_t)g * a.chunk_len) * a.D;
  // element offsets of the tile's 16 rows in this lane's channel (lanes past D read channel 0)
  uint32_t off[T];
#pragma unroll
  for (int j = 0; j < T; ++j) off[j] = (uint32_t)(j * a.D + (dv ? d : 0));
  float S = 0.0f;  // lower bound of the sum of dt from the current tile's start to the chunk's end
  int32_t s0 = 0;
  // tiles kg, kg - 1, ..., kg - GT + 1 (those >= 1: a start at tile 0 skips nothing)
  for (int kg = ntiles - 1; kg >= 1 && s0 == 0; kg -= GT) {
    float v[GT][T];
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      const IO* rows = chunk + (size_t)(kg - q > 0 ? kg - q : 0) * T * a.D;
#pragma unroll
      for (int j = 0; j < T; ++j) v[q][j] = load_io(rows, off[j]);
    }
#pragma unroll
    for (int q = 0; q < GT; ++q) {
      const int k = kg - q;
      if (k < 1) break;
      float ts = 0.0f;
#pragma unroll
      for (int j = 0; j < T; ++j) ts += fmaxf(v[q][j] + bias, 0.0f);
      S += ts;
      if (__all(!dv || amax * S <= kAggSkipExp2)) {
        s0 = k * T;
        break;
      }
    }
  }
  if (threadIdx.x == 0) start[((size_t)b * G + g) * nblk + blk] = s0;
}

size_t agg_start_bytes(int64_t batch, int64_t nchunks, int64_t D) {
  return (size_t)batch * nchunks * ((D + 63) / 64) * sizeof(int32_t);
}

bool launch_agg_start(const ScanArgs& a, int io, int N, int32_t* start, hipStream_t s) {
  // dt >= 0 only with softplus; the fused dt projection has no delta to read
  if (option(kOptAggSkip) == 0 || a.softplus == 0 || a.dtlow != nullptr || start == nullptr || a.nchunks < 2 ||
      a.chunk_len % kAggStartTile != 0 || a.chunk_len * a.D > 0x7fffffff)
    return false;
  const int32_t nblk = (int32_t)((a.D + 63) / 64);
  const int64_t units = a.batch * (int64_t)(a.nchunks - 1) * nblk;
  if (units <= 0 || units > 0x7fffffff) return false;
  if (io == kIoBF16)
    hipLaunchKernelGGL(agg_start_kernel<uint16_t>, dim3((unsigned)units), dim3(64), 0, s, a, (int32_t)N, nblk, start);
  else
    hipLaunchKernelGGL(agg_start_kernel<float>, dim3((unsigned)units), dim3(64), 0, s, a, (int32_t)N, nblk, start);
  return true;
}

// Output pass: every chunk from its carry-in (or h0 / zero when unchunked).
template <typename IO, int N>
__global__ __launch_bounds__(256) void scan_output_kernel(ScanArgs a) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t g = blockIdx.z;
  if (d >= a.D) return;
  const int64_t L = a.L, D = a.D;
  const IO* __restrict__ u = static_cast<const IO*>(a.u);
  const IO* __restrict__ dl = static_cast<const IO*>(a.delta);
  const IO* __restrict__ zp = static_cast<const IO*>(a.z);
  const IO* __restrict__ Bp = static_cast<const IO*>(a.B);
  const IO* __restrict__ Cp = static_cast<const IO*>(a.C);
  IO* __restrict__ out = static_cast<IO*>(a.out);
  const float bias = a.bias ? a.bias[d] : 0.0f;
  const float dskip = a.dskip ? a.dskip[d] : 0.0f;
  ChanConst<N> cc;
  cc.load(a.A + d * N);
  float h[N];
  if (a.nchunks > 1) {
    const float* src = a.agg_h + (((size_t)b * a.nchunks + g) * D + d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = src[n];
  } else if (a.h0) {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = a.h0[((size_t)b * D + d) * N + n];
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = 0.0f;
  }
  const int64_t t0 = g * a.chunk_len;
  const int64_t t1 = t0 + a.chunk_len < L ? t0 + a.chunk_len : L;
  const bool sp = a.softplus != 0;
  const bool has_z = zp != nullptr;
  for (int64_t t = t0; t < t1; ++t) {
    const size_t i = ((size_t)b * L + t) * D + d;
    float Bt[N], Ct[N];
    BCLoader<IO, N>::load(Bp + ((size_t)b * L + t) * N, Bt);
    BCLoader<IO, N>::load(Cp + ((size_t)b * L + t) * N, Ct);
    const float x = load_io(u, i);
    TokenFront f = make_front(load_io(dl, i), bias, sp);
    float y = token_step<N>(cc, f, x, Bt, Ct, h);
    const float zv = has_z ? load_io(zp, i) : 0.0f;
    store_io(out, i, epilogue(y, x, dskip, has_z, zv));
  }
  if (a.last && g == a.nchunks - 1) {
#pragma unroll
    for (int n = 0; n < N; ++n) a.last[((size_t)b * D + d) * N + n] = h[n];
  }
}

bool dstate_supported(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

namespace {


size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

#ifndef S6_WG_PER_CU
#define S6_WG_PER_CU 1
#endif
constexpr int64_t kCus = 256;                          // compute units of an MI355X
constexpr int64_t kGridMax = kCus * S6_WG_PER_CU;      // persistent workgroups
constexpr int64_t kChainedMinChains = 128;  // below this many channel blocks, long sequences use two passes

// cf: floats per state (1 real, 2 complex), for the workspace size.
ScanPlan plan_lane(int64_t batch, int64_t L, int64_t D, int64_t N, int cf = 1) {
  ScanPlan p{};
  p.engine = kEngineLane;
  p.block = D >= 256 ? 256 : (int32_t)(((D + 63) / 64) * 64);
  if (p.block < 64) p.block = 64;
  // Waves of the unchunked scan; cut L until about two waves per SIMD
  // (1024 SIMDs on 256 CUs), keeping chunks of at least 256 tokens.
  const int64_t waves = batch * ((D + 63) / 64);
  const int64_t target = 2048;
  int64_t g = waves > 0 ? (target + waves - 1) / waves : 1;
  int64_t gmax = L / 256 > 1 ? L / 256 : 1;
  if (gmax > 65535) gmax = 65535;
  if (g > gmax) g = gmax;
  if (g < 1) g = 1;
  p.chunk_len = L > 0 ? (L + g - 1) / g : 0;
  p.nchunks = (int32_t)(p.chunk_len > 0 ? (L + p.chunk_len - 1) / p.chunk_len : 1);
  if (p.nchunks < 1) p.nchunks = 1;
  p.ws_ctrl = 0;
  p.ws_bytes = p.nchunks > 1 ? (size_t)batch * p.nchunks * D * (N * cf + 1) * sizeof(float) : 0;
  return p;
}

#ifndef S6_WG_SPLIT_ITEMS
#define S6_WG_SPLIT_ITEMS 512
#endif

ScanPlan plan_wg(int64_t batch, int64_t L, int64_t D, int64_t N, int cf = 1, bool fdt = false) {
  ScanPlan p{};
  p.engine = kEngineWg;
  p.waves = wg_waves(N);
  const int64_t T = wg_tile(N);
  const int64_t chains = batch * ((D + 63) / 64);
  const int64_t tiles = (L + T - 1) / T;
  // A chunk's token rows, plus the up to four tiles the pipeline reads past its
  // end, must span less than 2^31 bytes: buffer offsets are 32-bit and the
  // out-of-range offset 2^31 must never wrap back into range.
  int64_t cap = ((int64_t)0x7fffffff / (D * 4) - 4 * T) / T * T;
  if (cap < T) cap = T;
  if (chains >= kChainedMinChains || tiles < 32) {
    // Chained chunks.  With more channel blocks than workgroups, chunks of
    // about 1024 tokens let the persistent grid balance the blocks.
    p.split = 0;
    int64_t chunk = L;
    if (chains > kCus) chunk = option(kOptChunk) > 0 ? option(kOptChunk) : 1024;
    chunk = ((chunk + T - 1) / T) * T;
    if (chunk > cap) chunk = cap;
    if (chunk >= L) chunk = L;
    p.chunk_len = chunk;
    p.nchunks = (int32_t)((L + chunk - 1) / chunk);
    p.grid = (int32_t)(chains < kGridMax ? chains : kGridMax);
    p.tile_out = (int32_t)T;
    p.grid_out = p.grid;
    p.ws_ctrl = round_up(256 + 4 * (size_t)chains, 256);
    p.ws_bytes = p.ws_ctrl + (size_t)chains * 64 * N * cf * sizeof(float);
  } else {
    // Two passes over independent chunks: about S6_WG_SPLIT_ITEMS work items.
    p.split = 1;
    int64_t g = (S6_WG_SPLIT_ITEMS + chains - 1) / chains;
    if (g > tiles / 4) g = tiles / 4;
    if (g < 2) g = 2;
    int64_t chunk = (L + g - 1) / g;
    chunk = ((chunk + T - 1) / T) * T;
    if (chunk > cap) chunk = cap;
    p.chunk_len = chunk;
    p.nchunks = (int32_t)((L + chunk - 1) / chunk);
    p.grid = (int32_t)kGridMax;
    // The output pass of a real scan runs on 8-token tiles: half the LDS, so two
    // workgroups share a CU (the projected-dt front end needs 16-token tiles).
    p.tile_out = (cf == 1 && !fdt && T == 16) ? 8 : (int32_t)T;
    p.grid_out = p.tile_out < T ? 2 * p.grid : p.grid;
    p.ws_ctrl = 256;
    // then the aggregate starts (real A only)
    p.ws_bytes = p.ws_ctrl + (size_t)batch * p.nchunks * D * (N * cf + 1) * sizeof(float) +
                 (cf == 1 ? agg_start_bytes(batch, p.nchunks, D) : 0);
  }
  return p;
}

}  // namespace

// Wave-private engine: one wave per (batch row, CW channels) for the whole
// sequence; long sequences over few channels are cut into chunks (two passes)
// until about 2.5 waves per SIMD result.
#ifndef S6_WP_MIXED
#define S6_WP_MIXED 1  // 0: no mixed launches of two- and one-state-per-lane waves
#endif
#ifndef S6_WP_SPLIT_WAVES
#define S6_WP_SPLIT_WAVES 2560  // waves the chunked scan aims for (2.5 per SIMD)
#endif
constexpr int64_t kWpSplitBelow = 1024;  // waves of the unchunked scan below which L is cut
constexpr int64_t kWpTargetWaves = S6_WP_SPLIT_WAVES;

ScanPlan plan_wp(int64_t batch, int64_t L, int64_t D, int64_t N, bool mixed) {
  ScanPlan p{};
  p.engine = kEngineWp;
  p.waves = (int32_t)(N / 2);
  const int64_t T = wp_tile();
  const int64_t waves = batch * ((D + 63) / 64) * (N / 2);
  const int64_t tiles = (L + T - 1) / T;
  // A chunk's token rows (of u, delta, z, out and of B, C), plus the tiles the
  // pipeline reads past its end (at most five), must span less than 2^31 bytes:
  // buffer offsets are 32-bit and the out-of-range offset 2^31 must never wrap
  // back into range.
  int64_t cap = ((int64_t)0x7fffffff / ((D > N ? D : N) * 4) - 8 * T) / T * T;
  if (cap < T) cap = T;
  int64_t g = 1;
  if (waves < kWpSplitBelow && tiles >= 8) {
    g = (kWpTargetWaves + waves - 1) / waves;
    if (g > tiles / 4) g = tiles / 4;
    if (g < 2) g = 2;
  }
  int64_t chunk = (L + g - 1) / g;
  chunk = ((chunk + T - 1) / T) * T;
  if (chunk > cap) chunk = cap;
  if (chunk >= L) chunk = L;
  p.chunk_len = chunk;
  p.nchunks = (int32_t)((L + chunk - 1) / chunk);
  p.split = p.nchunks > 1;
  // Unchunked N = 16 with more than 1024 but fewer than 3072 waves: part of the
  // (batch row, block) units run with one state per lane (twice the waves, half
  // the work each), so that the launch has 2 or 3 waves on every SIMD.
  const int64_t units = batch * ((D + 63) / 64);
  if (S6_WP_MIXED && mixed && !p.split && N == 16) {
    if (units > 128 && units < 256) p.wp1_units = (int32_t)(256 - units);
    else if (units > 256 && units < 384) p.wp1_units = (int32_t)(384 - units);
  }
  p.ws_ctrl = 0;
  p.ws_bytes = p.split ? (size_t)batch * p.nchunks * D * (N + 1) * sizeof(float) + agg_start_bytes(batch, p.nchunks, D)
                       : 0;
  return p;
}

ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N, bool mixed) {
  const int64_t engine = option(kOptEngine);
  if (wg_supported(N) && batch > 0 && L > 0 && D > 0 && engine != 1) {
    if (engine == 3) return plan_wp(batch, L, D, N, mixed);
    // Long sequences over few channel blocks (two passes over chunks) run faster
    // on the workgroup engine, whose waves load whole 128-byte lines of a token row.
    if (engine == 0) {
      const ScanPlan p = plan_wp(batch, L, D, N, mixed);
      if (!p.split) return p;
    }
    return plan_wg(batch, L, D, N);
  }
  return plan_lane(batch, L, D, N);
}

ScanPlan plan_scan_fused_dt(int64_t batch, int64_t L, int64_t D, int64_t N) {
  if (wg_supported(N) && batch > 0 && L > 0 && D > 0) return plan_wg(batch, L, D, N, 1, true);
  return plan_lane(batch, L, D, N);
}

ScanPlan plan_scan_complex(int64_t batch, int64_t L, int64_t D, int64_t N) {
  // The real scan's plans; carries and chunk aggregates hold N complex states.
  if (wg_supported(N) && batch > 0 && L > 0 && D > 0 && option(kOptEngine) != 1) return plan_wg(batch, L, D, N, 2);
  return plan_lane(batch, L, D, N, 2);
}

template <typename IO, int N>
static hipError_t launch_scan_t(const ScanArgs& a, const ScanPlan& p, hipStream_t s) {
  const int block = p.block;
  const dim3 grid_c((unsigned)((a.D + block - 1) / block), (unsigned)a.batch, (unsigned)p.nchunks);
  if (p.nchunks > 1) {
    const dim3 grid_a((unsigned)((a.D + block - 1) / block), (unsigned)a.batch, (unsigned)(p.nchunks - 1));
    hipLaunchKernelGGL((scan_chunk_state_kernel<IO, N>), grid_a, dim3(block), 0, s, a);
    const int64_t lanes = a.batch * a.D * N;
    hipLaunchKernelGGL((scan_carry_kernel<N>), dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((scan_output_kernel<IO, N>), grid_c, dim3(block), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chunk_carry(const ScanArgs& a, int N, hipStream_t s) {
  const int64_t lanes = a.batch * a.D * N;
  const dim3 grid((unsigned)((lanes + 255) / 256));
  switch (N) {
    case 1: hipLaunchKernelGGL((scan_carry_kernel<1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((scan_carry_kernel<2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((scan_carry_kernel<4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((scan_carry_kernel<8>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((scan_carry_kernel<16>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

template <typename IO>
static hipError_t launch_scan_io(const ScanArgs& a, const ScanPlan& p, int N, hipStream_t s) {
  switch (N) {
    case 1: return launch_scan_t<IO, 1>(a, p, s);
    case 2: return launch_scan_t<IO, 2>(a, p, s);
    case 4: return launch_scan_t<IO, 4>(a, p, s);
    case 8: return launch_scan_t<IO, 8>(a, p, s);
    case 16: return launch_scan_t<IO, 16>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

// L == 0: no output; the final state is the initial one.
__global__ __launch_bounds__(256) void scan_empty_kernel(float* last, const float* h0, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) last[i] = h0 ? h0[i] : 0.0f;
}

hipError_t launch_scan(const ScanArgs& in, const ScanPlan& p, int io, int N, void* workspace, hipStream_t s) {
  if (in.batch == 0 || in.D == 0) return hipSuccess;
  if (in.L == 0) {
    if (!in.last) return hipSuccess;
    const int64_t count = in.batch * in.D * N;
    hipLaunchKernelGGL(scan_empty_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, in.last, in.h0, count);
    return hipGetLastError();
  }
  ScanArgs a = in;
  a.chunk_len = p.chunk_len;
  a.nchunks = p.nchunks;
  if (p.engine == kEngineWp) return a.dtlow ? hipErrorInvalidValue : launch_scan_wp(a, p, io, N, workspace, s);
  if (p.engine == kEngineWg) return launch_scan_wg(a, p, io, N, workspace, s);
  a.agg_h = static_cast<float*>(workspace);
  a.agg_s = p.ws_bytes > 0 ? a.agg_h + (size_t)a.batch * p.nchunks * a.D * N : nullptr;
  return io == kIoBF16 ? launch_scan_io<uint16_t>(a, p, N, s) : launch_scan_io<float>(a, p, N, s);
}

// ----------------------------------------------------------------- decode

// One token for every (batch, channel), N = 1 and 2: lane = channel d of batch
// row blockIdx.y, all N states read and written in place.  B_t and C_t
// of the row are shared by the row's channels (page section 3.2): they are read
// once per wave through the scalar cache (whole dwords through the constant
// address space: the kernel never writes them), A as float4.
template <typename IO, int N>
__global__ __launch_bounds__(256) void state_update_kernel(StepArgs a) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = blockIdx.y;
  float Bt[N], Ct[N], h[N];
  if constexpr (sizeof(IO) == 2 && N % 2 == 0) {
    using CW = __attribute__((address_space(4))) const uint32_t;
    const CW* Bw = (const CW*)(static_cast<const uint32_t*>(a.B)) + b * (N / 2);
    const CW* Cw = (const CW*)(static_cast<const uint32_t*>(a.C)) + b * (N / 2);
#pragma unroll
    for (int q = 0; q < N / 2; ++q) {
      const uint32_t wb = Bw[q], wc = Cw[q];
      Bt[2 * q] = bf16_lo(wb);
      Bt[2 * q + 1] = bf16_hi(wb);
      Ct[2 * q] = bf16_lo(wc);
      Ct[2 * q + 1] = bf16_hi(wc);
    }
  } else if constexpr (sizeof(IO) == 4) {
    using CF = __attribute__((address_space(4))) const float;
    const CF* Bf = (const CF*)(static_cast<const float*>(a.B)) + b * N;
    const CF* Cf = (const CF*)(static_cast<const float*>(a.C)) + b * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      Bt[n] = Bf[n];
      Ct[n] = Cf[n];
    }
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) {
      Bt[n] = load_io(static_cast<const IO*>(a.B) + b * N, n);
      Ct[n] = load_io(static_cast<const IO*>(a.C) + b * N, n);
    }
  }
  if (d >= a.D) return;
  const int64_t idx = b * a.D + d;
  float* __restrict__ st = a.state + (size_t)idx * N;
  ChanConst<N> cc;
  if constexpr (N % 4 == 0) {
    float av[N];
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      const float4 v = reinterpret_cast<const float4*>(st)[j];
      h[4 * j] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
      const float4 q = reinterpret_cast<const float4*>(a.A + d * N)[j];
      av[4 * j] = q.x; av[4 * j + 1] = q.y; av[4 * j + 2] = q.z; av[4 * j + 3] = q.w;
    }
#pragma unroll
    for (int n = 0; n < N; ++n) cc.set(n, av[n]);
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = st[n];
    cc.load(a.A + d * N);
  }
  const float x = load_io(static_cast<const IO*>(a.u), idx);
  TokenFront f = make_front(load_io(static_cast<const IO*>(a.delta), idx), a.bias ? a.bias[d] : 0.0f, a.softplus != 0);
  float y = token_step<N>(cc, f, x, Bt, Ct, h);
  const bool has_z = a.z != nullptr;
  const float zv = has_z ? load_io(static_cast<const IO*>(a.z), idx) : 0.0f;
  store_io(static_cast<IO*>(a.out), idx, epilogue(y, x, a.dskip ? a.dskip[d] : 0.0f, has_z, zv));
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int j = 0; j < N / 4; ++j)
      reinterpret_cast<float4*>(st)[j] = make_float4(h[4 * j], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]);
  } else {
#pragma unroll
    for (int n = 0; n < N; ++n) st[n] = h[n];
  }
}

// The same step with four states per lane (N = 4, 8, 16): the N / 4 lanes of a
// channel are adjacent, so a wave's state loads and stores cover one
// contiguous 1 KB run per instruction (a lane that owned all N states would
// read them as N / 4 float4s at a 4 N-byte lane stride).  Each lane evaluates
// the channel's front end itself (dt, x and z are per channel, read by all its
// lanes at one address); the readout is summed over the channel's lanes with
// quad lane swaps.
#ifndef S6_DECODE_ROUNDS
#define S6_DECODE_ROUNDS 2  // channel groups per lane (their loads are issued together)
#endif
#ifndef S6_DECODE_NT
#define S6_DECODE_NT 3  // non-temporal state loads (bit 0) and stores (bit 1)
#endif
typedef float dec_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 dec_load_state(const float* p) {
  const dec_f32x4 v = (S6_DECODE_NT & 1) ? __builtin_nontemporal_load(reinterpret_cast<const dec_f32x4*>(p))
                                   : *reinterpret_cast<const dec_f32x4*>(p);
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void dec_store_state(float* p, float a, float b, float c, float d) {
  const dec_f32x4 v = {a, b, c, d};
  if (S6_DECODE_NT & 2) __builtin_nontemporal_store(v, reinterpret_cast<dec_f32x4*>(p));
  else *reinterpret_cast<dec_f32x4*>(p) = v;
}

// SP: softplus on (a compile-time flag, so that only one input-weight form is built).
template <typename IO, int N, bool SP>
__global__ __launch_bounds__(256) void state_update_vec_kernel(StepArgs a) {
  constexpr int LPC = N / 4;      // lanes per channel
  constexpr int CPB = 256 / LPC;  // channels per block and round
  constexpr int R = S6_DECODE_ROUNDS;
  static_assert(N % 4 == 0 && LPC <= 4, "four states per lane");
  const int q = threadIdx.x % LPC;
  const int64_t b = blockIdx.y;
  const int n0 = 4 * q;
  float Bt[4], Ct[4];
  if constexpr (sizeof(IO) == 2) {
    const uint2 wb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.B) + b * N + n0);
    const uint2 wc = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.C) + b * N + n0);
    Bt[0] = bf16_lo(wb.x); Bt[1] = bf16_hi(wb.x); Bt[2] = bf16_lo(wb.y); Bt[3] = bf16_hi(wb.y);
    Ct[0] = bf16_lo(wc.x); Ct[1] = bf16_hi(wc.x); Ct[2] = bf16_lo(wc.y); Ct[3] = bf16_hi(wc.y);
  } else {
    const float4 vb = *reinterpret_cast<const float4*>(static_cast<const float*>(a.B) + b * N + n0);
    const float4 vc = *reinterpret_cast<const float4*>(static_cast<const float*>(a.C) + b * N + n0);
    Bt[0] = vb.x; Bt[1] = vb.y; Bt[2] = vb.z; Bt[3] = vb.w;
    Ct[0] = vc.x; Ct[1] = vc.y; Ct[2] = vc.z; Ct[3] = vc.w;
  }
  // every round's loads first
  int64_t d[R];
  bool ok[R];
  float4 hv[R], qa[R];
  float xr[R], dr[R], zr[R];
  const bool has_z = a.z != nullptr;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    d[r] = ((int64_t)blockIdx.x * R + r) * CPB + threadIdx.x / LPC;
    ok[r] = d[r] < a.D;  // whole channels (all LPC lanes of a channel) agree
    const int64_t dd = ok[r] ? d[r] : 0;
    const int64_t idx = b * a.D + dd;
    hv[r] = ok[r] ? dec_load_state(a.state + (size_t)idx * N + n0) : make_float4(0.f, 0.f, 0.f, 0.f);
    qa[r] = *reinterpret_cast<const float4*>(a.A + dd * N + n0);
    xr[r] = load_io(static_cast<const IO*>(a.u), idx);
    dr[r] = load_io(static_cast<const IO*>(a.delta), idx);
    zr[r] = has_z ? load_io(static_cast<const IO*>(a.z), idx) : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t dd = ok[r] ? d[r] : 0;
    const int64_t idx = b * a.D + dd;
    float h[4] = {hv[r].x, hv[r].y, hv[r].z, hv[r].w};
    const float av[4] = {qa[r].x, qa[r].y, qa[r].z, qa[r].w};
    ChanConst<4> cc;
#pragma unroll
    for (int n = 0; n < 4; ++n) cc.set(n, av[n]);
    const TokenFront f = make_front(dr[r], a.bias ? a.bias[dd] : 0.0f, SP);
    float y = token_step<4>(cc, f, xr[r], Bt, Ct, h);
    // sum over the channel's lanes: (q0 + q1) + (q2 + q3), the same in every lane
    if constexpr (LPC >= 2) y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0xB1, 0xf, 0xf, false));
    if constexpr (LPC == 4) y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x4E, 0xf, 0xf, false));
    if (ok[r]) {
      dec_store_state(a.state + (size_t)idx * N + n0, h[0], h[1], h[2], h[3]);
      if (q == 0)
        store_io(static_cast<IO*>(a.out), idx, epilogue(y, xr[r], a.dskip ? a.dskip[dd] : 0.0f, has_z, zr[r]));
    }
  }
}

template <typename IO, int N>
static void launch_step_vec(const StepArgs& a, hipStream_t s) {
  constexpr int CPB = 256 / (N / 4) * S6_DECODE_ROUNDS;  // channels per block
  const dim3 grid((unsigned)((a.D + CPB - 1) / CPB), (unsigned)a.batch);
  if (a.softplus)
    hipLaunchKernelGGL((state_update_vec_kernel<IO, N, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((state_update_vec_kernel<IO, N, false>), grid, dim3(256), 0, s, a);
}

template <typename IO>
static hipError_t launch_step_io(const StepArgs& a, int N, hipStream_t s) {
  const dim3 grid((unsigned)((a.D + 255) / 256), (unsigned)a.batch);
  switch (N) {
    case 1: hipLaunchKernelGGL((state_update_kernel<IO, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((state_update_kernel<IO, 2>), grid, dim3(256), 0, s, a); break;
    case 4: launch_step_vec<IO, 4>(a, s); break;
    case 8: launch_step_vec<IO, 8>(a, s); break;
    case 16: launch_step_vec<IO, 16>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs& a, int io, int N, hipStream_t s) {
  if (a.batch == 0 || a.D == 0) return hipSuccess;
  return io == kIoBF16 ? launch_step_io<uint16_t>(a, N, s) : launch_step_io<float>(a, N, s);
}

}  // namespace s6

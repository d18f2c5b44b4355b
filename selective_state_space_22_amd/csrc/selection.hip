// selection.hip -- the selection front end of the selective scan on gfx950:
// the per-token B_t, C_t and the raw dt are linear functions of the token
// ("Mamba 状态空间模型原理与 Transformer 对比", kb.agiseed.tech, section 3.2:
// s_B(x) = Linear_N(x), s_C(x) = Linear_N(x), s_dt(x) = a projection of x of a
// small size, broadcast to the D channels; the dt projection size is the
// subject of the page's Δ-projection ablation table).  With rank R:
//     xdbl  = x W_x^T                (M x (R + 2N)),  M = batch * L
//     B, C  = columns R.. and R+N.. of xdbl
//     delta = xdbl[:, :R] W_dt^T     (M x D)          (bias and softplus follow in the scan)
// Both products are dense contractions, so they run on the matrix cores:
// v_mfma_f32_16x16x32_bf16 for bf16 I/O, v_mfma_f32_16x16x4_f32 for fp32 I/O,
// fp32 accumulation in both cases.
//
// GEMM kernel (C = A B^T, A: M x K, B: N x K, both K-contiguous, 16-byte
// aligned rows): 128 x 128 output blocks, operands staged through LDS with
// coalesced loads, fp32 accumulation, results leaving through LDS as 16-byte
// row segments; every global access is bounds-checked by a buffer resource
// (rows past M or N and K past the end read as zero, stores past the edges are
// dropped).  A long K with few output columns (x W_x^T) is split over
// workgroups into fp32 parts, summed in a fixed order by the kernel that also
// rounds and splits xdbl.  Shapes whose rows are not 16-byte aligned take a
// plain VALU kernel instead.
#include <cstdlib>
#include <type_traits>

#include "s6_device.h"
#include "s6_internal.h"

namespace s6 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int32_t kBufferDword3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferDword3);
}

template <typename T>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, float v);
template <>
__device__ __forceinline__ void store_elem<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
}
template <>
__device__ __forceinline__ void store_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// One K slice of 64 bytes per row: 32 bf16 (one MFMA) or 16 fp32 (four MFMAs).
template <typename T>
struct Mfma;
template <>
struct Mfma<uint16_t> {
  static constexpr int kSlice = 32;  // elements per 64-byte slice
  static __device__ __forceinline__ f32x4 step(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  static constexpr int kSlice = 16;
  static __device__ __forceinline__ f32x4 step(u32x4 a, u32x4 b, f32x4 c) {
    // lanes 16q..16q+15 hold K offsets 4q..4q+3 of the slice; MFMA e takes element e
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

struct GemmArgs {
  const void* A;  // M x K, row stride lda (elements)
  const void* B;  // N x K, row stride ldb
  void* C;        // M x N, row stride ldc
  int64_t M, N, K, lda, ldb, ldc;
  int64_t split_stride = 0;  // split K (parts > 1): part z covers stages [z*sps, (z+1)*sps), output at C + z*split_stride
  int32_t sps = 0;
  int32_t parts = 1;
  int32_t act = 0;  // 1: SiLU of every output element (applied in fp32 before rounding)
  // large-product kernel: one fp32 256 x 256 slot per workgroup for the halves of the
  // blocks of a last, at most half-filled round, split in K (null: no split)
  float* part = nullptr;
  // large-product kernel: the output columns from n2 on (n2 a multiple of its block
  // width) go to C2 instead, as columns 0 .. N - n2 - 1 with the same row stride and
  // without the activation (null: every column to C)
  void* C2 = nullptr;
  int64_t n2 = 0;
};

// 128 x 128 output block per workgroup of 2 x 2 waves (4 x 4 tiles of 16 x 16
// each).  K advances in stages of 128 bytes per row (64 bf16 / 32 fp32): the
// A and B stage tiles (128 rows x 128 bytes each) are read with coalesced
// 16-byte loads (8 adjacent lanes per row), stored to LDS (double buffered,
// chunks XOR-swizzled by row against bank conflicts, see stage_off), and each
// wave reads its MFMA operands from LDS (lane l: row l % 16, bytes 16 (l / 16)
// of a 64-byte half-stage).  Global loads run three stages ahead of the
// multiplication, through a ring of registers: with two workgroups per CU that
// keeps ~190 KB per CU in flight, enough to cover HBM latency at full bandwidth.
constexpr int kGemmBM = 128;
constexpr int kStageBytes = 128;                  // K bytes per row per stage
// LDS stage layout: 128-byte rows, the 16-byte chunk c of row r stored at chunk
// c ^ ((r >> 1) & 7).  The 16 lanes of a quarter-wave then touch 64 distinct
// banks both when they store two rows (8 chunks each) and when they read one
// chunk of 16 consecutive rows as MFMA operands.
__device__ __forceinline__ uint32_t stage_off(uint32_t row, uint32_t chunk) {
  return row * kStageBytes + 16u * (chunk ^ ((row >> 1) & 7u));
}

template <typename IN, typename OUT>
__global__ __launch_bounds__(256, 2) void gemm_nt_mfma_kernel(GemmArgs g) {
  constexpr int TM = 4, TN = 4;
  constexpr uint32_t E = sizeof(IN);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 1, wn = w & 1;
  // XCD-aware block order.  Consecutive workgroup ids go to the 8 XCDs in turn,
  // each with its own L2.  The column blocks of one (row block, K part) group,
  // which all read the same rows of A, get ids congruent mod 8 and 8 apart:
  // they run on one XCD at about the same time and read A once into its L2.
  const int nbn = (int)((g.N + kGemmBM - 1) / kGemmBM);
  const int64_t groups = ((g.M + kGemmBM - 1) / kGemmBM) * g.parts;
  const int64_t id = blockIdx.x;
  const int64_t round = id / (8 * nbn), rem = id % (8 * nbn);
  const int64_t grp = round * 8 + rem % 8;
  if (grp >= groups) return;
  const int col_blk = (int)(rem / 8);
  const int64_t row_blk = grp % ((g.M + kGemmBM - 1) / kGemmBM);
  const int part = (int)(grp / ((g.M + kGemmBM - 1) / kGemmBM));
  const int64_t bm0 = row_blk * kGemmBM;
  const int64_t bn0 = (int64_t)col_blk * kGemmBM;
  const int64_t mrows = g.M - bm0 < kGemmBM ? g.M - bm0 : kGemmBM;
  const int64_t nrows = g.N - bn0 < kGemmBM ? g.N - bn0 : kGemmBM;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(static_cast<const IN*>(g.A) + bm0 * g.lda,
                                              (uint32_t)(((mrows - 1) * g.lda + g.K) * E));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const IN*>(g.B) + bn0 * g.ldb,
                                              (uint32_t)(((nrows - 1) * g.ldb + g.K) * E));
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kGemmBM * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kGemmBM * kStageBytes];

  // global -> register share of one stage: 4 loads per operand per thread
  const int t = threadIdx.x;
  const int lrow = t >> 3;             // 0..31, + 32 v
  const uint32_t lbyte = (t & 7) * 16u;
  const uint32_t kbytes = (uint32_t)(g.K * E);
  u32x4 ga[3][4], gb[3][4];  // register ring: stage s lives in slot (s - first) % 3
  const int all = (int)((kbytes + kStageBytes - 1) / kStageBytes);
  const int first = g.parts > 1 ? part * g.sps : 0;
  const int nst = g.parts > 1 ? (all - first < g.sps ? all - first : g.sps) : all;
  auto gload = [&](int stage, auto slot) {
    constexpr int R = decltype(slot)::value;
    const uint32_t kb = (uint32_t)stage * kStageBytes + lbyte;
    const bool in = stage < first + nst && kb < kbytes;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t row = lrow + 32 * v;
      ga[R][v] = __builtin_amdgcn_raw_buffer_load_b128(ra, in ? (uint32_t)(row * g.lda * E) + kb : kOutOfRange, 0, 0);
      gb[R][v] = __builtin_amdgcn_raw_buffer_load_b128(rb, in ? (uint32_t)(row * g.ldb * E) + kb : kOutOfRange, 0, 0);
    }
  };
  auto lstore = [&](int buf, auto slot) {
    constexpr int R = decltype(slot)::value;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t o = stage_off(lrow + 32 * v, lbyte / 16);
      *reinterpret_cast<u32x4*>(&lds_a[buf][o]) = ga[R][v];
      *reinterpret_cast<u32x4*>(&lds_b[buf][o]) = gb[R][v];
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int r16 = lane & 15, q = lane >> 4;
  // Stage k of this launch (global stage first + k): multiply it from LDS
  // buffer k & 1, move stage k + 1 from its register slot to the other buffer,
  // then reuse stage k's slot (stored to LDS one step earlier) for stage k + 3.
  auto step = [&](int k, auto next_slot, auto own_slot) {
    const int buf = k & 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // two 64-byte halves of the stage
      u32x4 a[TM], b[TN];
      const uint32_t chunk = 4u * h + q;
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const u32x4*>(&lds_a[buf][stage_off(wm * 64 + 16 * i + r16, chunk)]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const u32x4*>(&lds_b[buf][stage_off(wn * 64 + 16 * j + r16, chunk)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<IN>::step(a[i], b[j], acc[i][j]);
    }
    if (k + 1 < nst) lstore(buf ^ 1, next_slot);
    gload(first + k + 3, own_slot);
    __syncthreads();
  };
  gload(first, S0{});
  gload(first + 1, S1{});
  gload(first + 2, S2{});
  lstore(0, S0{});
  __syncthreads();
  for (int k = 0; k < nst; k += 3) {
    step(k, S1{}, S0{});
    if (k + 1 < nst) step(k + 1, S2{}, S1{});
    if (k + 2 < nst) step(k + 2, S0{}, S2{});
  }

  // Output: each 16-row strip of a wave's 64 x 64 tile goes through LDS (fp32,
  // reusing the stage buffers after the last barrier), then every lane writes
  // 16 contiguous bytes of one row.
  OUT* cbase = static_cast<OUT*>(g.C) + (g.parts > 1 ? (int64_t)part * g.split_stride : 0);
  const int64_t m0 = bm0 + wm * 64, n0 = bn0 + wn * 64;
  const int64_t wrows = g.M - m0 < 64 ? (g.M - m0 > 0 ? g.M - m0 : 0) : 64;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(cbase + m0 * g.ldc, (uint32_t)(wrows > 0 ? ((wrows - 1) * g.ldc + g.N) * sizeof(OUT) : 0));
  const bool vec_ok = (g.ldc * sizeof(OUT)) % 16 == 0 && (reinterpret_cast<uintptr_t>(cbase) & 15u) == 0;
  float(*st)[68] = reinterpret_cast<float(*)[68]>(&lds_a[0][0] + w * 16 * 68 * 4);
  constexpr int EPV = 16 / sizeof(OUT);  // output elements per 16-byte store
  constexpr int LPR = 64 / EPV;          // lanes per row
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[4 * q + r][16 * j + r16] = acc[i][j][r];
    __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave execute in order
#pragma unroll
    for (int e0 = 0; e0 < 16 * LPR; e0 += 64) {
      const int e = e0 + lane;
      const int row = e / LPR, c0 = (e % LPR) * EPV;
      const int64_t grow = 16 * i + row;  // relative to m0
      const int64_t gcol = n0 + c0;
      float v[EPV];
#pragma unroll
      for (int k4 = 0; k4 < EPV / 4; ++k4) {  // 16-byte reads (rows of 68 floats, 16-byte aligned)
        const float4 f = *reinterpret_cast<const float4*>(&st[row][c0 + 4 * k4]);
        v[4 * k4] = f.x;
        v[4 * k4 + 1] = f.y;
        v[4 * k4 + 2] = f.z;
        v[4 * k4 + 3] = f.w;
      }
      if (g.act)
#pragma unroll
        for (int kk = 0; kk < EPV; ++kk) v[kk] = silu(v[kk]);
      if (vec_ok && gcol + EPV <= g.N) {
        const uint32_t off = (uint32_t)((grow * g.ldc + gcol) * sizeof(OUT));
        u32x4 pk;
        if constexpr (sizeof(OUT) == 2) {
          pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          pk.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
          pk.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
        } else {
          pk = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        }
        __builtin_amdgcn_raw_buffer_store_b128(pk, rc, grow < wrows ? off : kOutOfRange, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < EPV; ++kk) {
          const uint32_t off =
              gcol + kk < g.N ? (uint32_t)((grow * g.ldc + gcol + kk) * sizeof(OUT)) : kOutOfRange;
          store_elem<OUT>(rc, grow < wrows ? off : kOutOfRange, v[kk]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Short K (at most KS 64-byte slices per row: the dt projection, K = dt rank).
// The general kernel spends most of its time waiting for the first operands of
// each output block here, since a block has only a few K stages.  Instead each
// wave keeps the B operands of one 64-column strip in registers for the whole
// launch and streams 32-row chunks of A straight into the MFMA layout (lane l:
// row l % 16, the 16 bytes at 16 (l / 16) of each 64-byte slice), the next
// chunk's loads in flight while the current one is multiplied.  The four waves
// of a workgroup take four adjacent strips of the same row chunks, so the A rows
// (small, L2-resident) are fetched once per workgroup, and the workgroups that
// share row chunks get ids congruent mod 8 (one XCD).  Results leave through a
// per-wave LDS strip as 16-byte row segments.
constexpr int kShortRows = 32;  // rows per chunk

template <typename IN, typename OUT, int KS>
__global__ __launch_bounds__(256, 2) void gemm_nt_shortk_kernel(GemmArgs g, int chunks_per_wg) {
  constexpr uint32_t E = sizeof(IN);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int ncg = (int)((g.N + 255) / 256);
  const int64_t nchunks = (g.M + kShortRows - 1) / kShortRows;
  const int64_t nrg = (nchunks + chunks_per_wg - 1) / chunks_per_wg;
  const int64_t id = blockIdx.x;
  const int64_t round = id / (8 * ncg), rem = id % (8 * ncg);
  const int64_t rg = round * 8 + rem % 8;
  if (rg >= nrg) return;
  const int64_t n0 = (rem / 8) * 256 + 64 * w;  // this wave's column strip
  const int64_t c0 = rg * chunks_per_wg;
  const int64_t c1 = c0 + chunks_per_wg < nchunks ? c0 + chunks_per_wg : nchunks;
  const uint32_t kbytes = (uint32_t)(g.K * E);

  // B operands of the strip, for the whole launch
  const int64_t nrows = g.N - n0 < 64 ? (g.N - n0 > 0 ? g.N - n0 : 0) : 64;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(static_cast<const IN*>(g.B) + (nrows > 0 ? n0 : 0) * g.ldb,
                                              (uint32_t)(nrows > 0 ? ((nrows - 1) * g.ldb + g.K) * E : 0));
  u32x4 b[4][KS];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t kb = (uint32_t)(64 * ks + 16 * q);
      b[j][ks] = __builtin_amdgcn_raw_buffer_load_b128(
          rb, kb < kbytes ? (uint32_t)((16 * j + r16) * g.ldb * E) + kb : kOutOfRange, 0, 0);
    }

  // A rows of this workgroup's chunks
  const int64_t arow0 = c0 * kShortRows;
  const int64_t arows = (g.M < c1 * kShortRows ? g.M : c1 * kShortRows) - arow0;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(static_cast<const IN*>(g.A) + arow0 * g.lda, (uint32_t)(((arows - 1) * g.lda + g.K) * E));
  auto aload = [&](u32x4 (&a)[2][KS], int64_t c) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t kb = (uint32_t)(64 * ks + 16 * q);
        const int64_t row = (c - c0) * kShortRows + 16 * i + r16;  // < arows unless past M (then out of range)
        a[i][ks] = __builtin_amdgcn_raw_buffer_load_b128(
            ra, c < c1 && kb < kbytes ? (uint32_t)(row * g.lda * E) + kb : kOutOfRange, 0, 0);
      }
  };

  // output strip staging: 32 rows x 64 columns of fp32 per wave; rows of 68 floats
  // (16-byte aligned): the tile writes below hit 64 distinct banks, and the 16-byte
  // read-back of 8 lanes (one row's 32-byte pieces) 32 distinct banks
  __shared__ __attribute__((aligned(16))) float stage[4][kShortRows][68];
  float(*st)[68] = stage[w];
  const bool vec_ok = (g.ldc * sizeof(OUT)) % 16 == 0 && (reinterpret_cast<uintptr_t>(g.C) & 15u) == 0;
  constexpr int EPV = 16 / sizeof(OUT);  // output elements per 16-byte store
  constexpr int LPR = 64 / EPV;          // lanes per row
  OUT* cbase = static_cast<OUT*>(g.C);

  u32x4 a[2][KS], an[2][KS];
  aload(a, c0);
  for (int64_t c = c0; c < c1; ++c) {
    aload(an, c + 1);
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[i][j] = Mfma<IN>::step(a[i][ks], b[j][ks], acc[i][j]);
      }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[16 * i + 4 * q + r][16 * j + r16] = acc[i][j][r];
    __builtin_amdgcn_wave_barrier();  // LDS accesses of one wave execute in order
    const int64_t m0 = c * kShortRows;
    const int64_t wrows = g.M - m0 < kShortRows ? g.M - m0 : kShortRows;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(cbase + m0 * g.ldc, (uint32_t)(((wrows - 1) * g.ldc + g.N) * sizeof(OUT)));
#pragma unroll
    for (int e0 = 0; e0 < kShortRows * LPR; e0 += 64) {
      const int e = e0 + lane;
      const int row = e / LPR, cc = (e % LPR) * EPV;
      const int64_t gcol = n0 + cc;
      float v[EPV];
#pragma unroll
      for (int k4 = 0; k4 < EPV / 4; ++k4) {
        const float4 f = *reinterpret_cast<const float4*>(&st[row][cc + 4 * k4]);
        v[4 * k4] = f.x;
        v[4 * k4 + 1] = f.y;
        v[4 * k4 + 2] = f.z;
        v[4 * k4 + 3] = f.w;
      }
      if (g.act)
#pragma unroll
        for (int kk = 0; kk < EPV; ++kk) v[kk] = silu(v[kk]);
      if (vec_ok && gcol + EPV <= g.N) {
        const uint32_t off = (uint32_t)((row * g.ldc + gcol) * sizeof(OUT));
        u32x4 pk;
        if constexpr (sizeof(OUT) == 2) {
          pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          pk.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
          pk.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
        } else {
          pk = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        }
        __builtin_amdgcn_raw_buffer_store_b128(pk, rc, row < wrows ? off : kOutOfRange, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < EPV; ++kk) {
          const uint32_t off = gcol + kk < g.N ? (uint32_t)((row * g.ldc + gcol + kk) * sizeof(OUT)) : kOutOfRange;
          store_elem<OUT>(rc, row < wrows ? off : kOutOfRange, v[kk]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a[i][ks] = an[i][ks];
  }
}

// Large products (the block's input and output projections): 256 x 256 output
// blocks of 8 waves, two per SIMD, each wave owning 128 x 64 (8 x 4 tiles of 16 x 16,
// accumulators in AGPRs).  K advances in stages of 128 bytes per row, one cache
// line: operands go from global memory straight into LDS with buffer loads that
// carry the lds bit (lane i of a load writes the 16 bytes at 16 i of its 1 KB
// destination, so one load moves 8 rows x 128 bytes); such loads of whole lines move
// 1.7x the bytes per unit time of loads of half lines.  A stage is 512 rows x 128
// bytes = 64 KB and LDS holds two: while stage p is multiplied (in two halves of 64
// bytes of K), stage p + 1 lands.  Row r's 16-byte chunk c sits at chunk
// c ^ ((r >> 1) & 7): the MFMA operand reads (lane l: row l % 16, chunk 4h + l / 16)
// then run at the rate of plain 1 KB reads.
constexpr int kBigBM = 256;     // rows of A (and of B) per output block
constexpr int kBigStage = 128;  // K bytes per row per stage
constexpr int kBigBufs = 2;
constexpr int kBigThreads = 512;
constexpr int64_t kBigCus = 256;  // compute units of an MI355X: the kernel's grid

__device__ __forceinline__ uint32_t big_off(uint32_t row, uint32_t chunk) {
  return row * kBigStage + 16u * (chunk ^ ((row >> 1) & 7u));
}

// s_waitcnt with vmcnt = n and lgkmcnt = 0 (expcnt not waited for).
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0070);
}

template <typename IN, typename OUT>
__global__ __launch_bounds__(kBigThreads) void gemm_nt_big_kernel(GemmArgs g) {
  constexpr int TM = 8, TN = 4;  // 16 x 16 tiles of a wave: 128 rows x 64 columns
  constexpr uint32_t E = sizeof(IN);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int r16 = lane & 15, q = lane >> 4;
  // Output blocks.  The grid is one workgroup per CU (a multiple of 8) and each
  // workgroup works through several blocks.  Workgroup ids go to the 8 XCDs in turn
  // (id mod 8): XCD x owns the contiguous range of blocks [x per_xcd, (x + 1) per_xcd),
  // and its workgroup j takes blocks x per_xcd + j, + j + G / 8, ..., so at any time
  // the XCD's workgroups hold consecutive blocks.  Blocks are numbered in groups 8 row
  // blocks high, so consecutive blocks share rows of A or of B through the XCD's L2.
  // When the XCD's last round is at most half full (rem blocks for G / 8 workgroups),
  // its blocks are split in K instead: workgroup j takes half j / rem of block
  // j % rem and writes fp32 partial sums to its slot of g.part, which
  // big_fixup_kernel adds up (so no workgroup idles for a whole block).
  const int64_t nbn = (g.N + kBigBM - 1) / kBigBM;
  const int64_t nbm = (g.M + kBigBM - 1) / kBigBM;
  const int64_t ntiles = nbm * nbn;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t wpx = gridDim.x / 8;
  const int64_t xcd = blockIdx.x % 8;
  const int64_t jw = blockIdx.x / 8;
  const int64_t xbeg = xcd * per_xcd;
  const int64_t xend = (xcd + 1) * per_xcd < ntiles ? (xcd + 1) * per_xcd : ntiles;
  const int64_t nx = xend > xbeg ? xend - xbeg : 0;  // blocks of this XCD
  const int64_t rounds = nx / wpx, rem = nx % wpx;
  const bool split = g.part != nullptr && rem > 0 && 2 * rem <= wpx;
  const int nfull = (int)rounds + (!split && jw < rem ? 1 : 0);
  const bool has_half = split && jw < 2 * rem;
  const int ntl = nfull + (has_half ? 1 : 0);  // items (blocks or halves) of this workgroup
  if (ntl == 0) return;
  auto tile_of = [&](int u) -> int64_t {
    return u < nfull ? xbeg + jw + (int64_t)u * wpx : xbeg + rounds * wpx + jw % (rem > 0 ? rem : 1);
  };
  auto origin = [&](int u, int64_t& bm0, int64_t& bn0) {
    const int64_t t = tile_of(u);
    constexpr int64_t kGroup = 8;
    const int64_t grp = t / (kGroup * nbn);
    const int64_t rows_in_grp = nbm - grp * kGroup < kGroup ? nbm - grp * kGroup : kGroup;
    const int64_t in_grp = t - grp * kGroup * nbn;
    bm0 = (grp * kGroup + in_grp % rows_in_grp) * kBigBM;
    bn0 = (in_grp / rows_in_grp) * kBigBM;
  };
  // LDS rows 0..255: A; rows 256..511: B.
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBigBufs][2 * kBigBM * kBigStage];

  const uint32_t kbytes = (uint32_t)(g.K * E);
  const int nst = (int)((kbytes + kBigStage - 1) / kBigStage);  // stages per block
  // Each XCD takes the K stages in its own rotated order, starting at stage x nst / 8:
  // the workgroups of one XCD keep one order (they share stages through its L2), while
  // the XCDs, which share HBM and the Infinity Cache, do not all ask for the same
  // columns of K at the same time.
  const uint32_t krot = (uint32_t)((xcd * nst) / 8);
  auto kstage = [&](int st) -> uint32_t {
    const uint32_t v = (uint32_t)st + krot;
    return v >= (uint32_t)nst ? v - (uint32_t)nst : v;
  };
  // stages [s_begin, s_end) of item u: a half takes the first nh stages or the rest
  const int nh = (nst + 1) / 2;
  const int half_no = has_half ? (int)(jw / rem) : 0;
  auto s_begin = [&](int u) { return u == nfull && half_no == 1 ? nh : 0; };
  auto s_end = [&](int u) { return u == nfull && half_no == 0 ? nh : nst; };
  // The loads run through the workgroup's blocks as one stream of K stages: the
  // stages of its next block follow those of the current one in the ring, so the
  // next block's first stages land while the current one finishes and is written.
  // Load cursor: stage ds of block du, with that block's buffer resources; past the
  // last block, loads past every row (read as zero).  DMA share of this wave per
  // stage: rows 32 w .. 32 w + 31 of A and of B, four loads of 8 rows each.  Lane i
  // of a load lands at row base + i / 8, physical chunk i % 8, so it fetches the
  // logical chunk (i % 8) ^ ((row >> 1) & 7).
  const uint32_t lrow = (uint32_t)(lane >> 3), lch = (uint32_t)(lane & 7);
  const uint32_t ldaE = (uint32_t)(g.lda * E), ldbE = (uint32_t)(g.ldb * E);
  int du = 0, ds = 0;
  __amdgpu_buffer_rsrc_t ra = make_rsrc(g.A, 0), rb = make_rsrc(g.B, 0);
  auto load_block = [&](int u) {
    if (u >= ntl) return;
    int64_t bm0, bn0;
    origin(u, bm0, bn0);
    const int64_t mrows = g.M - bm0 < kBigBM ? g.M - bm0 : kBigBM;
    const int64_t nrows = g.N - bn0 < kBigBM ? g.N - bn0 : kBigBM;
    ra = make_rsrc(static_cast<const IN*>(g.A) + bm0 * g.lda, (uint32_t)(((mrows - 1) * g.lda + g.K) * E));
    rb = make_rsrc(static_cast<const IN*>(g.B) + bn0 * g.ldb, (uint32_t)(((nrows - 1) * g.ldb + g.K) * E));
  };
  // Load n (0..7) of this wave for the cursor's stage: rows 32 w + 8 m + (0..7) of A
  // (n = 2m) or of B (n = 2m + 1).  Row r = 32 w + 8 m + lrow has the swizzle
  // (r >> 1) & 7 = (lrow >> 1) ^ 4 (m & 1): two per-lane chunk offsets serve all loads.
  const uint32_t la = lrow * ldaE, lb = lrow * ldbE;
  const uint32_t ch0 = 16u * (lch ^ (lrow >> 1)), ch1 = 16u * (lch ^ ((lrow >> 1) ^ 4u));
  auto dma_one = [&](int buf, int n) {
    const uint32_t m = (uint32_t)(n >> 1);
    const uint32_t ch = (m & 1) ? ch1 : ch0;
    const uint32_t kb = kstage(ds) * kBigStage + ch;
    // past K or past the last block: an offset past every row, read as zero
    const uint32_t cut = kb < kbytes && du < ntl ? 0u : kOutOfRange;
    const uint32_t r0 = (uint32_t)(32 * w) + 8u * m;  // first row of the load
    if (n & 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, &lds[buf][(kBigBM + r0) * kBigStage], 16,
                                               (r0 * ldbE + lb + kb) | cut, 0, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, &lds[buf][r0 * kBigStage], 16, (r0 * ldaE + la + kb) | cut, 0, 0,
                                               0);
  };
  auto next_load = [&] {
    if (du < ntl && ++ds == s_end(du)) {
      ++du;
      ds = du < ntl ? s_begin(du) : 0;
      load_block(du);
    }
  };
  // A barrier without a memory fence: a fence here would make every wave wait for
  // all of its loads in flight (they write LDS); instead each wave waits for its
  // loads of the stage it is about to read (vmcnt) before the barrier.  The signal
  // fences keep the compiler from moving LDS accesses across it.
  auto stage_barrier = [] {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  // Operand fragments of half h (64 bytes of K) of a stage.
  auto read_a = [&](int buf, int i, int h) {
    return *reinterpret_cast<const u32x4*>(&lds[buf][big_off(wm * 128 + 16 * i + r16, 4 * h + q)]);
  };
  auto read_b = [&](int buf, int j, int h) {
    return *reinterpret_cast<const u32x4*>(&lds[buf][big_off(kBigBM + wn * 64 + 16 * j + r16, 4 * h + q)]);
  };
  // acc += (a b^T)^T on one 16 x 16 tile: the B fragment goes in as the first MFMA
  // operand, so lane (q, r) holds the outputs (row r, columns 4q .. 4q + 3) of the tile,
  // which it stores as one 8- or 16-byte segment.  For bf16 the MFMA is written out so
  // that its accumulator is tied to its result register: the compiler's own form may
  // put the result in another AGPR quad, which across the K loop turns into a rotation
  // of the accumulators through VGPRs at every stage.  The "memory" clobber keeps the
  // LDS reads where they are written, between the MFMAs.
  auto mma = [](f32x4& c, const u32x4& a, const u32x4& b) {
    if constexpr (sizeof(IN) == 2)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a) : "memory");
    else
      c = Mfma<IN>::step(b, a, c);
  };

  f32x4 acc[TM][TN];
  auto clear = [&] {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  };
  clear();

  // Output of block u straight from the accumulators: tile (i, j) of the wave gives
  // lane (q, r) the 4 columns 16 j + 4 q .. + 3 of row 16 i + r; rows and columns past
  // the edges are dropped.
  OUT* cbase = static_cast<OUT*>(g.C);
  // 32-bit offsets: a per-lane part (row r, columns 4q..) and a uniform part per tile.
  // The lane index is counted afresh here (v_mbcnt, in a volatile statement the
  // compiler cannot hoist), so that nothing per-lane is kept live across the K loop.
  const uint32_t ldcB = (uint32_t)(g.ldc * (int64_t)sizeof(OUT));
  auto write_block = [&](int u) {
    uint32_t ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int r16 = (int)(ln & 15), q = (int)(ln >> 4);
    const uint32_t lane_off = (uint32_t)r16 * ldcB + (uint32_t)(4 * q * (int)sizeof(OUT));
    int64_t bm0, bn0;
    origin(u, bm0, bn0);
    // the block's output: its columns of C, or of C2 past n2
    const bool second = g.C2 != nullptr && bn0 >= g.n2;
    OUT* const cb = second ? static_cast<OUT*>(g.C2) : cbase;
    const int64_t ncols = second ? g.N - g.n2 : (g.C2 != nullptr ? g.n2 : g.N);
    const bool act = g.act != 0 && !second;
    const int64_t m0 = bm0 + wm * 128, n0 = (second ? bn0 - g.n2 : bn0) + wn * 64;
    const int64_t wrows = g.M - m0 < 128 ? (g.M - m0 > 0 ? g.M - m0 : 0) : 128;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(
        cb + (wrows > 0 ? m0 : 0) * g.ldc, (uint32_t)(wrows > 0 ? ((wrows - 1) * g.ldc + ncols) * sizeof(OUT) : 0));
    // the last MFMAs' results must be written before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const int wr = (int)wrows;                     // rows of this wave's part inside M
    const int cl = (int)(ncols - n0) - 4 * q;      // columns left for this lane's segments
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const bool row_ok = 16 * i + r16 < wr;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t off = lane_off + (uint32_t)(16 * i) * ldcB + (uint32_t)((n0 + 16 * j) * (int64_t)sizeof(OUT));
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = act ? silu(acc[i][j][r]) : acc[i][j][r];
        // N and ldc are multiples of 4 and C is aligned to a segment (see big_ok)
        const uint32_t o = row_ok && 16 * j < cl ? off : kOutOfRange;
        if constexpr (sizeof(OUT) == 2) {
          u32x2 pk;
          pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(pk, rc, o, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}, rc, o, 0,
              0);
        }
      }
    }
  };

  // A half block's fp32 partial sums, to this workgroup's slot of g.part (256 x 256,
  // row-major, whole: the edges are dropped when the halves are added up).
  auto write_partial = [&] {
    uint32_t ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const uint32_t r16 = ln & 15, q = ln >> 4;
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(g.part + (size_t)blockIdx.x * kBigBM * kBigBM, (uint32_t)(kBigBM * kBigBM * sizeof(float)));
    const uint32_t lane_off = ((uint32_t)(wm * 128) + r16) * (kBigBM * 4) + ((uint32_t)(wn * 64) + 4 * q) * 4;
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(acc[i][j][0]), __float_as_uint(acc[i][j][1]), __float_as_uint(acc[i][j][2]),
                  __float_as_uint(acc[i][j][3])},
            rp, lane_off + (uint32_t)(16 * i * kBigBM * 4 + 16 * j * 4), 0, 0);
  };

  // Stage p of the stream in two halves of 64 bytes of K, with the operands of the
  // current half in registers (read during the previous half):
  // - first half: 32 MFMAs, and the second half's operands read from stage p's buffer
  //   between them;
  // - second half: once this wave's loads of stage p + 1 have landed and every wave has
  //   passed the barrier (each wave waits for its LDS reads before it), stage p + 1 is
  //   readable and stage p's buffer is read by no one, so the loads of stage p + 2 go
  //   there, spread over the MFMAs, while the first half of stage p + 1 is read between
  //   them.
  // Rows 0..5 of the tiles read, once a[i] is spent, the next half's fragment i of A
  // into a[i] itself; rows 0..3 read fragment i of B into nb[i] after their first
  // MFMA, rows 4 and 5 the A fragments 6 and 7 into na.  The last read is two rows
  // before the end, so the wait for all of them before the next barrier is short.
  int pbuf = 0;  // buffer of stage p; stage p + 1 in the other
  auto half = [&](int h, u32x4 (&a)[TM], const u32x4 (&b)[TN], u32x4 (&nb)[TN]) {
    const int nbuf = h == 0 ? pbuf : pbuf ^ 1;
    if (h == 1) {
      wait_vm_lgkm0<0>();
      stage_barrier();
    }
    u32x4 na[2];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        mma(acc[i][j], a[i], b[j]);
        if (j == 0 && i < TN) nb[i] = read_b(nbuf, i, h ^ 1);
        if (j == 0 && (i == 4 || i == 5)) na[i - 4] = read_a(nbuf, i + 2, h ^ 1);
        // the loads of stage p + 2, one per 4 MFMAs
        if (h == 1 && j == 2) dma_one(pbuf, i);
      }
      if (i < 6) a[i] = read_a(nbuf, i, h ^ 1);
    }
    a[6] = na[0];
    a[7] = na[1];
    if (h == 1) {
      next_load();
      pbuf ^= 1;
    }
  };

  u32x4 a[TM], b0[TN], b1[TN];
  ds = s_begin(0);
  load_block(0);
#pragma unroll 1
  for (int k = 0; k < kBigBufs; ++k) {
#pragma unroll
    for (int n = 0; n < 8; ++n) dma_one(k, n);
    next_load();
  }
  wait_vm_lgkm0<8>();
  stage_barrier();
#pragma unroll
  for (int i = 0; i < TM; ++i) a[i] = read_a(0, i, 0);
#pragma unroll
  for (int j = 0; j < TN; ++j) b0[j] = read_b(0, j, 0);
  for (int u = 0; u < ntl; ++u) {
    for (int k = s_begin(u); k < s_end(u); ++k) {
      half(0, a, b0, b1);
      half(1, a, b1, b0);
    }
    if (u < nfull) write_block(u);
    else write_partial();
    clear();
  }
  // every load in flight (the zero stages past the end) lands before the workgroup ends
  wait_vm_lgkm0<0>();
}

// The blocks that gemm_nt_big_kernel split in K, added up: workgroup b takes rows
// 16 (b % 16) .. + 15 of XCD x's split block r (x = (b / 16) % 8, r = b / 128), whose
// halves are in the slots of workgroups 8 r + x and 8 (r + rem) + x of the big kernel's
// grid of G; it applies the SiLU where asked and stores 4 outputs at a time (N and ldc
// are multiples of 4 and C is aligned to 4 outputs, see big_ok).
template <typename OUT>
__global__ __launch_bounds__(256) void big_fixup_kernel(GemmArgs g, int64_t grid) {
  const int64_t nbn = (g.N + kBigBM - 1) / kBigBM;
  const int64_t nbm = (g.M + kBigBM - 1) / kBigBM;
  const int64_t ntiles = nbm * nbn;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t wpx = grid / 8;
  const int64_t strip = blockIdx.x % 16, xcd = (blockIdx.x / 16) % 8, r = blockIdx.x / 128;
  const int64_t xbeg = xcd * per_xcd;
  const int64_t xend = (xcd + 1) * per_xcd < ntiles ? (xcd + 1) * per_xcd : ntiles;
  const int64_t nx = xend > xbeg ? xend - xbeg : 0;
  const int64_t rounds = nx / wpx, rem = nx % wpx;
  if (!(rem > 0 && 2 * rem <= wpx && r < rem)) return;
  const int64_t t = xbeg + rounds * wpx + r;
  constexpr int64_t kGroup = 8;
  const int64_t grp = t / (kGroup * nbn);
  const int64_t rows_in_grp = nbm - grp * kGroup < kGroup ? nbm - grp * kGroup : kGroup;
  const int64_t in_grp = t - grp * kGroup * nbn;
  const int64_t bm0 = (grp * kGroup + in_grp % rows_in_grp) * kBigBM;
  const int64_t bn0 = (in_grp / rows_in_grp) * kBigBM;
  const bool second = g.C2 != nullptr && bn0 >= g.n2;  // columns past n2 go to C2
  const int64_t ncols = second ? g.N - g.n2 : (g.C2 != nullptr ? g.n2 : g.N);
  const int64_t cn0 = second ? bn0 - g.n2 : bn0;
  const bool act = g.act != 0 && !second;
  const float4* p0 = reinterpret_cast<const float4*>(g.part + (size_t)(8 * r + xcd) * kBigBM * kBigBM);
  const float4* p1 = reinterpret_cast<const float4*>(g.part + (size_t)(8 * (r + rem) + xcd) * kBigBM * kBigBM);
  OUT* c = static_cast<OUT*>(second ? g.C2 : g.C);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = (int)strip * 16 * (kBigBM / 4) + k * 256 + (int)threadIdx.x;  // float4 index in the block
    const int64_t row = bm0 + e / (kBigBM / 4), col = cn0 + (e % (kBigBM / 4)) * 4;
    if (row >= g.M || col >= ncols) continue;
    const float4 x = p0[e], y = p1[e];
    float v[4] = {x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w};
    if (act)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = silu(v[i]);
    OUT* dst = c + row * g.ldc + col;
    if constexpr (sizeof(OUT) == 2) {
      u32x2 pk;
      pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<u32x2*>(dst) = pk;
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Any alignment: one thread per output element, K FMAs.
template <typename IN, typename OUT>
__global__ void gemm_nt_valu_kernel(GemmArgs g) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= g.M * g.N) return;
  const int64_t m = i / g.N, n = i % g.N;
  const IN* a = static_cast<const IN*>(g.A) + m * g.lda;
  const IN* b = static_cast<const IN*>(g.B) + n * g.ldb;
  float acc = 0.0f;
  for (int64_t k = 0; k < g.K; ++k) acc = __builtin_fmaf(load_io(a, k), load_io(b, k), acc);
  store_io(static_cast<OUT*>(g.C), (size_t)(m * g.ldc + n), g.act ? silu(acc) : acc);
}

// Sum of the split-K parts of x W_x^T, rounded once to the I/O type: the
// first R columns to xdbl (input of the dt projection), the next N to B, the
// last N to C.
template <typename IO>
__global__ void xproj_reduce_kernel(const float* part, int64_t parts, int64_t M, int64_t R, int64_t N, IO* xdbl,
                                    int64_t ldx, IO* B, IO* C) {
  const int64_t W = R + 2 * N;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (m, c)
  if (i >= M * W) return;
  const int64_t m = i / W, c = i % W;
  float v = 0.0f;
  for (int64_t z = 0; z < parts; ++z) v += part[z * M * W + i];
  if (c < R) store_io(xdbl, (size_t)(m * ldx + c), v);
  else if (c < R + N) store_io(B, (size_t)(m * N + c - R), v);
  else store_io(C, (size_t)(m * N + c - R - N), v);
}

size_t xdbl_bytes(int64_t batch, int64_t L, int64_t R, int64_t N, size_t e) {
  (void)N;
  return ((size_t)batch * L * ((R + 7) / 8 * 8) * e + 255) / 256 * 256;
}

template <typename IN>
bool mfma_ok(const GemmArgs& g) {
  constexpr int64_t VEC = 16 / sizeof(IN);
  return g.K % VEC == 0 && g.lda % VEC == 0 && g.ldb % VEC == 0 && (reinterpret_cast<uintptr_t>(g.A) & 15u) == 0 &&
         (reinterpret_cast<uintptr_t>(g.B) & 15u) == 0;
}

// C (OUT) = A B^T.  128 x 128 per workgroup of 2 x 2 waves of 4 x 4 tiles, two
// K slices in flight; with parts > 1, K is split into parts and part z is
// written (fp32) at C + z * split_stride.
template <typename IN, typename OUT, int KS>
hipError_t launch_shortk(const GemmArgs& g, hipStream_t st) {
  const int64_t nchunks = (g.M + kShortRows - 1) / kShortRows;
  const int64_t ncg = (g.N + 255) / 256;
  // about four workgroups per CU over the launch, at least one chunk each
  int64_t per = nchunks * ncg / 1024;
  if (per < 1) per = 1;
  const int64_t nrg = (nchunks + per - 1) / per;
  const int64_t blocks = (nrg + 7) / 8 * 8 * ncg;  // whole groups of 8 (ids past the last row group exit)
  hipLaunchKernelGGL((gemm_nt_shortk_kernel<IN, OUT, KS>), dim3((unsigned)blocks), dim3(256), 0, st, g, (int)per);
  return hipGetLastError();
}

// Slices of 64 bytes per row that the short-K kernel is instantiated for: with
// two workgroups per CU a wave has 256 VGPRs, which hold the B strip, two A
// chunks and the accumulators up to six slices (384 bytes: dt rank 192 in bf16).
constexpr int kShortMaxSlices = 6;

template <typename IN, typename OUT>
hipError_t gemm_nt_short(const GemmArgs& g, int ks, hipStream_t st) {
  switch (ks) {
    case 1: return launch_shortk<IN, OUT, 1>(g, st);
    case 2: return launch_shortk<IN, OUT, 2>(g, st);
    case 3: return launch_shortk<IN, OUT, 3>(g, st);
    case 4: return launch_shortk<IN, OUT, 4>(g, st);
    case 5: return launch_shortk<IN, OUT, 5>(g, st);
    case 6: return launch_shortk<IN, OUT, 6>(g, st);
    default: return hipErrorInvalidValue;
  }
}

// The large-block kernel pays off once both output dimensions fill several of
// its 256 x 256 blocks and K spans a few stages.
template <typename IN>
bool big_ok(const GemmArgs& g, size_t out_bytes) {
  const int64_t e = sizeof(IN);
  // row offsets inside a 256-row block must stay below the out-of-range bit
  const bool offsets = 256 * g.lda * e + g.K * e < (int64_t)kOutOfRange && 256 * g.ldb * e + g.K * e < (int64_t)kOutOfRange;
  // each lane stores 4 consecutive outputs of a row as one aligned segment
  const bool segments = g.N % 4 == 0 && g.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(g.C) % (4 * out_bytes) == 0;
  // a second output starts at a block edge and is aligned like the first
  const bool second = g.C2 == nullptr ||
                      (g.n2 > 0 && g.n2 < g.N && g.n2 % kBigBM == 0 && reinterpret_cast<uintptr_t>(g.C2) % (4 * out_bytes) == 0);
  return g.M >= 1024 && g.N >= 512 && g.K * e >= 1024 && offsets && segments && second &&
         option(kOptGemmGeneral) == 0;
}

template <typename IN, typename OUT>
hipError_t gemm_nt(GemmArgs g, hipStream_t st, int parts = 1) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  if (mfma_ok<IN>(g) && parts == 1 && big_ok<IN>(g, sizeof(OUT))) {
    const int64_t nbn = (g.N + kBigBM - 1) / kBigBM;
    const int64_t nbm = (g.M + kBigBM - 1) / kBigBM;
    // one workgroup per CU (the LDS holds one), in 8 equal XCD shares
    const int64_t blocks = nbm * nbn < kBigCus ? (nbm * nbn + 7) / 8 * 8 : kBigCus;
    hipLaunchKernelGGL((gemm_nt_big_kernel<IN, OUT>), dim3((unsigned)blocks), dim3(kBigThreads), 0, st, g);
    if (g.part != nullptr) {  // any XCD with a split last round?
      const int64_t ntiles = nbm * nbn, per_xcd = (ntiles + 7) / 8, wpx = blocks / 8;
      bool any = false;
      for (int64_t x = 0; x < 8; ++x) {
        const int64_t lo = x * per_xcd, hi = (x + 1) * per_xcd < ntiles ? (x + 1) * per_xcd : ntiles;
        const int64_t rem = (hi > lo ? hi - lo : 0) % wpx;
        any = any || (rem > 0 && 2 * rem <= wpx);
      }
      // 16 row strips of each possible split block: 8 XCDs x wpx / 2 blocks
      if (any)
        hipLaunchKernelGGL((big_fixup_kernel<OUT>), dim3((unsigned)(16 * 8 * (wpx / 2))), dim3(256), 0, st, g, blocks);
    }
    return hipGetLastError();
  }
  if (g.C2 != nullptr) return hipErrorInvalidValue;  // only the large-product kernel routes columns
  const int ks = (int)((g.K * (int64_t)sizeof(IN) + 63) / 64);
  if (mfma_ok<IN>(g) && parts == 1 && ks <= kShortMaxSlices && option(kOptGemmGeneral) == 0)
    return gemm_nt_short<IN, OUT>(g, ks, st);
  if (mfma_ok<IN>(g)) {
    const int all = (int)((g.K * (int64_t)sizeof(IN) + kStageBytes - 1) / kStageBytes);
    g.sps = (all + parts - 1) / parts;
    g.parts = parts;
    const int64_t nbn = (g.N + kGemmBM - 1) / kGemmBM;
    const int64_t groups = ((g.M + kGemmBM - 1) / kGemmBM) * parts;
    const int64_t blocks = (groups + 7) / 8 * 8 * nbn;  // whole groups of 8 (ids past the last group exit)
    hipLaunchKernelGGL((gemm_nt_mfma_kernel<IN, OUT>), dim3((unsigned)blocks), dim3(256), 0, st, g);
  } else {
    // the vector path never splits: part 0 holds the whole sum (callers pass parts = 1 then)
    const int64_t n = g.M * g.N;
    hipLaunchKernelGGL((gemm_nt_valu_kernel<IN, OUT>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

// Split of K for x W_x^T (few output columns, long K): enough workgroups for
// one full round of the chip, two per CU (measured on the Mamba-3B layer:
// 1, 2, 4 and 8 parts took 88, 70, 76 and 89 us, the summing kernel 8-22 us).
int xproj_parts(int64_t M, int64_t W, int64_t K, int esize) {
  const int64_t tiles = ((M + 127) / 128) * ((W + 127) / 128);
  const int64_t stages = (K * esize + kStageBytes - 1) / kStageBytes;
  int parts = 1;
  while (parts < 8 && tiles * parts < 512 && stages / (parts * 2) >= 8) parts *= 2;
  return parts;
}

template <typename IO>
hipError_t launch_selection_t(const SelArgs& s, hipStream_t st) {
  const int64_t M = s.batch * s.L;
  const int64_t W = s.R + 2 * s.N;
  IO* xdbl = static_cast<IO*>(s.xdbl);
  float* part = reinterpret_cast<float*>(static_cast<uint8_t*>(s.xdbl) + xdbl_bytes(s.batch, s.L, s.R, s.N, sizeof(IO)));
  GemmArgs g1{s.x, s.Wx, part, M, W, s.D, s.D, s.D, W};
  g1.split_stride = M * W;
  const int parts = mfma_ok<IO>(g1) ? xproj_parts(M, W, s.D, sizeof(IO)) : 1;
  hipError_t e = gemm_nt<IO, float>(g1, st, parts);
  if (e != hipSuccess) return e;
  const int64_t n = M * W;
  hipLaunchKernelGGL((xproj_reduce_kernel<IO>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     (int64_t)parts, M, s.R, s.N, xdbl, s.ldx, static_cast<IO*>(s.Bout), static_cast<IO*>(s.Cout));
  if (!s.delta) return hipGetLastError();  // dt projection fused into the scan
  GemmArgs g2{xdbl, s.Wdt, s.delta, M, s.D, s.R, s.ldx, s.R, s.D};
  return gemm_nt<IO, IO>(g2, st);
}

}  // namespace

int64_t selection_ld(int64_t R, int64_t N) { return (R + 7) / 8 * 8; }

size_t selection_ws_bytes(int64_t batch, int64_t L, int64_t R, int64_t N, int io) {
  const size_t e = io == kIoBF16 ? 2 : 4;
  const int64_t M = batch * L, W = R + 2 * N;
  // xdbl (first R columns, padded rows), then up to 8 fp32 split-K parts of x W_x^T
  return xdbl_bytes(batch, L, R, N, e) + ((size_t)8 * M * W * 4 + 255) / 256 * 256;
}

hipError_t launch_selection(const SelArgs& s, int io, hipStream_t st) {
  return io == kIoBF16 ? launch_selection_t<uint16_t>(s, st) : launch_selection_t<float>(s, st);
}

size_t gemm_nt_part_bytes() { return (size_t)kBigCus * kBigBM * kBigBM * sizeof(float); }

hipError_t launch_gemm_nt(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                          int64_t ldb, int64_t ldc, int io, int act, float* part, hipStream_t st) {
  GemmArgs g{A, B, C, M, N, K, lda, ldb, ldc};
  g.act = act;
  g.part = part;
  return io == kIoBF16 ? gemm_nt<uint16_t, uint16_t>(g, st) : gemm_nt<float, float>(g, st);
}

template <typename IO>
hipError_t gemm_nt_pair_t(const GemmArgs& g, hipStream_t st) {
  if (mfma_ok<IO>(g) && big_ok<IO>(g, sizeof(IO))) return gemm_nt<IO, IO>(g, st);
  // two launches: the first n2 rows of B into C, the rest into C2
  GemmArgs g1 = g, g2 = g;
  g1.C2 = g2.C2 = nullptr;
  g1.N = g.n2;
  g2.B = static_cast<const IO*>(g.B) + g.n2 * g.ldb;
  g2.C = g.C2;
  g2.N = g.N - g.n2;
  g2.act = 0;
  hipError_t e = gemm_nt<IO, IO>(g1, st);
  return e == hipSuccess ? gemm_nt<IO, IO>(g2, st) : e;
}

hipError_t launch_gemm_nt_pair(const void* A, const void* B, void* C, void* C2, int64_t M, int64_t N1, int64_t N2,
                               int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int io, int act, float* part,
                               hipStream_t st) {
  if (N1 <= 0 || N2 <= 0) return hipErrorInvalidValue;
  GemmArgs g{A, B, C, M, N1 + N2, K, lda, ldb, ldc};
  g.act = act;
  g.part = part;
  g.C2 = C2;
  g.n2 = N1;
  return io == kIoBF16 ? gemm_nt_pair_t<uint16_t>(g, st) : gemm_nt_pair_t<float>(g, st);
}

}  // namespace s6

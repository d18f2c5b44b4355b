// s6_internal.h -- host-side plan and launcher declarations shared by the
// C-ABI layer (api.cpp) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace s6 {

enum IoType { kIoF32 = 0, kIoBF16 = 1 };

// Process-wide tuning options (the mamba_option values of the C ABI).  They are
// read by the plans, so a workspace size depends on the shape and on them.
enum Option {
  kOptEngine = 1,       // forward engine: 0 automatic, 1 lane, 2 workgroup, 3 wave-private
  kOptChunk = 2,        // tokens per chunk of the workgroup engine's chained mode (0: 1024)
  kOptWgWaves = 3,      // waves of the workgroup engine for N = 16 (0: 8, or 4)
  kOptFusedDt = 4,      // 1: mamba_ssm_fwd projects dt inside the scan
  kOptBwdChunk = 5,     // tokens per chunk of the backward (0: automatic)
  kOptGemmGeneral = 6,  // 1: only the general GEMM kernel
  kOptSpinLimit = 7,    // polls of a chained-mode wait before it gives up (0: give up at once)
  kOptAggSkip = 8,      // 1: chunk aggregates skip what decays below 2^-200 before the chunk end
  kOptCount = 9
};
int64_t option(int key);

// Sticky per-device status word of the chained-mode waits (nonzero: some wait
// gave up since the last read); kernels write it through this device address.
uint32_t* wait_status_ptr();
// Synchronise the stream, then read and clear the current device's status word.
hipError_t take_wait_status(hipStream_t stream, uint32_t* value);

// Arguments of one forward scan; pointers are device pointers.
struct ScanArgs {
  const void* u;
  const void* delta;
  const float* bias;   // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* dskip;  // may be null
  const void* z;       // may be null
  const float* h0;     // may be null
  void* out;
  float* last;         // may be null
  float* agg_h;        // workspace: (batch, nchunks, D, N) chunk states / carries
  float* agg_s;        // workspace: (batch, nchunks, D) chunk sums of dt
  int64_t batch, L, D;
  int64_t chunk_len;
  int32_t nchunks;
  int32_t softplus;
  // Fused dt projection (workgroup engine only): when dtlow is set, the raw dt
  // is dtlow[token, :R] . Wdt[channel, :R] computed on the matrix cores and
  // `delta` is not read.  dtlow: (batch*L, ldr), Wdt: (D, R), both I/O type.
  const void* dtlow = nullptr;
  const void* Wdt = nullptr;
  int64_t R = 0, ldr = 0;
  // Two-pass scans: first token of each chunk aggregate, relative to the
  // chunk's first token, per (batch, chunk, 64-channel block); null: every
  // aggregate starts at its chunk's first token.
  const int32_t* agg_start = nullptr;
};

// Largest dt rank the fused projection keeps in registers (eight 64-byte K slices).
bool fused_dt_supported(int64_t N, int64_t R, int io);

struct StepArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* bias;
  const float* A;
  const void* B;
  const void* C;
  const float* dskip;
  const void* z;
  void* out;
  int64_t batch, D;
  int32_t softplus;
};

// Engines of the forward scan.
enum Engine {
  kEngineLane = 0,  // one lane owns all N states of a channel (any supported N)
  kEngineWg = 1,    // a workgroup owns 64 channels, its waves split the N states (N = 8, 16)
  kEngineWp = 2,    // a workgroup owns 64 channels, each wave whole channels, two states per lane (N = 8, 16)
};

// Modes of the workgroup engine.
enum WgMode {
  kModeChained = 0,  // chunks of a channel block run in order, carried through the workspace
  kModeAgg = 1,      // chunk end states from zero and chunk sums of dt (first pass of the split scan)
  kModeOut = 2,      // outputs of every chunk from precomputed carry-ins (second pass)
};

// Arguments of the workgroup engine on top of the scan arguments.
struct WgArgs {
  ScanArgs s;
  uint32_t* ticket;   // work counter of this launch (zeroed before the launch)
  uint32_t* flags;    // chained mode: chunks finished per channel block (zeroed before the launch)
  uint32_t* err;      // the device's wait status word: set when a wait gives up (never expected)
  uint32_t spin_limit;  // polls of a wait before it gives up; 0: give up at once (testing)
  float* carry;       // chained mode: (chains, 64, N) state handed from chunk to chunk
  int32_t chains;     // batch * blocks_per_row: independent (batch row, 64-channel block) pairs
  int32_t blocks_per_row;
  int32_t nitems;     // work items of this launch
};

// Execution plan of a forward scan, a pure function of the shape.
struct ScanPlan {
  int32_t engine;     // Engine
  int32_t split;      // workgroup engine: 0 chained, 1 two passes (aggregates, carry, outputs)
  int32_t waves;      // workgroup engine: waves per workgroup
  int32_t nchunks;    // L is cut into this many chunks of chunk_len tokens
  int64_t chunk_len;
  int32_t block;      // lane engine: threads per workgroup (64 channels per wave)
  int32_t grid;       // workgroup engine: persistent workgroups
  int32_t tile_out;   // workgroup engine, two passes: tokens per tile of the output pass
  int32_t grid_out;   // workgroup engine, two passes: persistent workgroups of the output pass
  int32_t wp1_units;  // wave-private engine, unchunked N = 16: the last wp1_units (batch row, 64-channel
                      // block) units run with one state per lane in the same launch (0: none)
  size_t ws_ctrl;     // bytes of counters and flags at the start of the workspace
  size_t ws_bytes;    // workspace the plan needs in total (0 when nothing is needed)
};

// mixed: whether an unchunked N = 16 scan may use the mixed launch (two- and
// one-state-per-lane waves).  It is the faster launch when scans run back to back,
// and the slower one right after the selection GEMMs (mamba_ssm_fwd and the block
// pass false).
ScanPlan plan_scan(int64_t batch, int64_t L, int64_t D, int64_t N, bool mixed = true);
// Plan of a scan whose dt is projected inside the workgroup engine (ScanArgs::dtlow).
ScanPlan plan_scan_fused_dt(int64_t batch, int64_t L, int64_t D, int64_t N);

// Workgroup engine (scan_wg.hip).
// cplx: complex A (A, h0, last and the carries hold (re, im) pairs), no fused dt projection.
hipError_t launch_scan_wg(const ScanArgs& a, const ScanPlan& p, int io, int N, void* workspace, hipStream_t stream,
                          bool cplx = false);
bool wg_supported(int64_t N);
int wg_waves(int64_t N);
int wg_tile(int64_t N);

// Wave-private engine (scan_wp.hip): real A, N = 8 or 16, the workgroup engine's plans.
hipError_t launch_scan_wp(const ScanArgs& a, const ScanPlan& p, int io, int N, void* workspace, hipStream_t stream);
int wp_tile();

bool dstate_supported(int64_t N);

// Complex diagonal A (scan_complex.hip): A, h0 and last are (.., N, 2) re/im
// float; agg_h is (batch, nchunks, D, N, 2).  The plans are those of the real
// scan with two floats per state.
ScanPlan plan_scan_complex(int64_t batch, int64_t L, int64_t D, int64_t N);
hipError_t launch_scan_complex(const ScanArgs& a, const ScanPlan& p, int io, int N, void* workspace,
                               hipStream_t stream);
// One decode token with complex A: state is (batch, D, N, 2), A (D, N, 2).
hipError_t launch_step_complex(const StepArgs& a, int io, int N, hipStream_t stream);
// Carry pass over complex (batch, chunk, D, N, 2) chunk aggregates.
hipError_t launch_cplx_carry(const ScanArgs& a, int N, hipStream_t stream);

// ---------------------------------------------------------------- backward (scan_bwd.hip)

constexpr int kBwdTile = 8;  // tokens per tile of the backward passes

// Arguments of one backward scan; pointers are device pointers.
struct BwdArgs {
  const void* u;
  const void* delta;
  const float* bias;   // may be null
  const float* A;
  const void* B;
  const void* C;
  const float* dskip;  // may be null
  const void* z;       // may be null
  const float* h0;     // may be null
  const void* dout;
  const float* dlast;  // may be null
  void* du;
  void* ddelta;
  float* dA;
  void* dB;
  void* dC;
  float* dDskip;       // may be null
  void* dz;            // may be null
  float* dbias;        // may be null
  float* dh0;          // may be null
  // workspace
  float* hs;    // (batch, G, N, D) chunk end state from zero, then the state entering the chunk
  float* gq;    // (batch, G, N, D) chunk gradient aggregate, then the gradient arriving at the chunk end
  float* sdt;   // (batch, G, D) sum of dt over the chunk
  float* srel;  // (batch, G, tpc, N, D) state at each tile start, relative to a zero chunk start
  float* cdt;   // (batch, G, tpc, D) sum of dt from the chunk start to each tile start
  float* pbc;   // (batch, nblk, L, 2, N) per-block partial dB (0) and dC (1)
  float* pA;    // (batch * G, N, D) per-chunk partial dA
  float* pD;    // (batch * G, 2, D) per-chunk partial dDskip (0) and bias gradient (1)
  int64_t batch, L, D;
  int64_t chunk_len;
  int32_t nchunks, tpc, nblk;
  int32_t softplus;
};

struct BwdPlan {
  int64_t chunk_len;
  int32_t nchunks, tpc, nblk;
  size_t off_hs, off_gq, off_sdt, off_srel, off_cdt, off_pbc, off_pA, off_pD;
  size_t ws_bytes;
};

BwdPlan plan_bwd(int64_t batch, int64_t L, int64_t D, int64_t N);
hipError_t launch_bwd(const BwdArgs& a, int io, int N, hipStream_t stream);

// ---------------------------------------------------------------- selection projections (selection.hip)

// xdbl = x W_x^T (M x (R+2N), row stride ldx), B/C = its last 2N columns, delta = xdbl[:, :R] W_dt^T.
struct SelArgs {
  const void* x;    // (M, D)
  const void* Wx;   // (R + 2N, D)
  const void* Wdt;  // (D, R)
  void* delta;      // (M, D); null: only xdbl, B and C (the scan projects dt itself)
  void* Bout;       // (M, N)
  void* Cout;       // (M, N)
  void* xdbl;       // workspace (M, ldx)
  int64_t batch, L, D, N, R, ldx;
};

int64_t selection_ld(int64_t R, int64_t N);
size_t selection_ws_bytes(int64_t batch, int64_t L, int64_t R, int64_t N, int io);
hipError_t launch_selection(const SelArgs& s, int io, hipStream_t stream);
// C (I/O type) = A B^T, A: M x K, B: N x K (row strides lda, ldb, ldc); act = 1
// applies SiLU to every output element before rounding.  part: scratch of
// gemm_nt_part_bytes() for the large-product kernel's K-split last round (may be
// null: no split).
size_t gemm_nt_part_bytes();
hipError_t launch_gemm_nt(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int64_t lda,
                          int64_t ldb, int64_t ldc, int io, int act, float* part, hipStream_t stream);
// Two products with a common A: C = act(A B[0:N1]^T) and C2 = A B[N1:N1+N2]^T (the rows
// of B consecutive, C and C2 with row stride ldc), one launch where the large-product
// kernel takes the pair, else two.
hipError_t launch_gemm_nt_pair(const void* A, const void* B, void* C, void* C2, int64_t M, int64_t N1, int64_t N2,
                               int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int io, int act, float* part,
                               hipStream_t stream);

// Enqueue the kernels of one scan / one decode step on `stream`.
hipError_t launch_scan(const ScanArgs& a, const ScanPlan& p, int io, int N, void* workspace, hipStream_t stream);
// Carry pass over (batch, chunk, D, N) chunk aggregates (both engines' split modes).
hipError_t launch_chunk_carry(const ScanArgs& a, int N, hipStream_t stream);
// Start tokens of the chunk aggregates of a two-pass scan (ScanArgs::agg_start):
// (batch, nchunks, ceil(D / 64)) int32 in `start`.  Returns false (and launches
// nothing) where every aggregate must start at its chunk's first token.
size_t agg_start_bytes(int64_t batch, int64_t nchunks, int64_t D);
bool launch_agg_start(const ScanArgs& a, int io, int N, int32_t* start, hipStream_t stream);
hipError_t launch_step(const StepArgs& a, int io, int N, hipStream_t stream);

}  // namespace s6

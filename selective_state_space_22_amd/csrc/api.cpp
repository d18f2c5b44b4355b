// api.cpp -- the C ABI declared in include/mamba_mi355x.h.
//
// Every entry point validates its arguments on the host before it touches
// the HIP runtime, then enqueues kernels on the caller's stream and returns.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mamba_mi355x.h"
#include "s6_internal.h"

namespace {

bool debug_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("MAMBA_MI355X_DEBUG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

int fail(int status, const char* where, const char* what) {
  if (debug_enabled()) std::fprintf(stderr, "[mamba_mi355x] %s: %s (%s)\n", where, mamba_status_string(status), what);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------------ options

constexpr int64_t kDefaultSpinLimit = int64_t(1) << 24;

int64_t env_value(const char* name, int64_t dflt) {
  const char* v = std::getenv(name);
  if (!v || !v[0]) return dflt;
  char* end = nullptr;
  const long long x = std::strtoll(v, &end, 10);
  return (end && *end == 0 && x >= 0) ? (int64_t)x : dflt;
}

// The options start from the environment once, when the library is first used.
struct Options {
  std::atomic<int64_t> v[s6::kOptCount];
  Options() {
    int64_t engine = 0;
    if (const char* e = std::getenv("MAMBA_MI355X_ENGINE")) {
      if (!std::strcmp(e, "lane")) engine = 1;
      else if (!std::strcmp(e, "wg")) engine = 2;
      else if (!std::strcmp(e, "wp")) engine = 3;
    }
    if (env_value("MAMBA_MI355X_LANE_ENGINE", 0) == 1) engine = 1;
    if (env_value("MAMBA_MI355X_WG_ENGINE", 0) == 1) engine = 2;
    for (auto& x : v) x.store(0);
    v[s6::kOptEngine].store(engine);
    v[s6::kOptChunk].store(env_value("MAMBA_MI355X_CHUNK", 0));
    v[s6::kOptWgWaves].store(env_value("MAMBA_MI355X_WG_WAVES", 0));
    v[s6::kOptFusedDt].store(env_value("MAMBA_MI355X_FUSED_DT", 0) == 1 ? 1 : 0);
    v[s6::kOptBwdChunk].store(env_value("MAMBA_MI355X_BWD_CHUNK", 0));
    v[s6::kOptGemmGeneral].store(std::getenv("MAMBA_MI355X_GEMM_GENERAL") ? 1 : 0);
    const int64_t spin = env_value("MAMBA_MI355X_SPIN_LIMIT", kDefaultSpinLimit);
    v[s6::kOptSpinLimit].store(spin <= 0xffffffffll ? spin : kDefaultSpinLimit);
    v[s6::kOptAggSkip].store(env_value("MAMBA_MI355X_AGG_SKIP", 1) == 0 ? 0 : 1);
  }
};

Options& options() {
  static Options o;
  return o;
}

bool option_valid(int key, int64_t value) {
  switch (key) {
    case s6::kOptEngine: return value >= 0 && value <= 3;
    case s6::kOptChunk: return value >= 0 && value <= (int64_t(1) << 30);
    case s6::kOptWgWaves: return value == 0 || value == 4 || value == 8;
    case s6::kOptFusedDt: return value == 0 || value == 1;
    case s6::kOptBwdChunk: return value >= 0 && value <= (int64_t(1) << 30);
    case s6::kOptGemmGeneral: return value == 0 || value == 1;
    case s6::kOptSpinLimit: return value >= 0 && value <= 0xffffffffll;
    case s6::kOptAggSkip: return value == 0 || value == 1;
    default: return false;
  }
}

constexpr int64_t kMaxBatch = 65535;
constexpr int64_t kMaxDim = int64_t(1) << 22;

// Shape and dtype checks shared by the entry points (MAMBA_OK if usable).
int check_shape(const char* where, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io) {
  if (io != MAMBA_IO_F32 && io != MAMBA_IO_BF16) return fail(MAMBA_ERR_DTYPE, where, "io_dtype");
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate <= 0) return fail(MAMBA_ERR_DIM, where, "negative or zero size");
  if (batch > kMaxBatch) return fail(MAMBA_ERR_DIM, where, "batch > 65535");
  if (dim > kMaxDim) return fail(MAMBA_ERR_DIM, where, "dim > 4194304");
  if (!s6::dstate_supported(dstate)) return fail(MAMBA_ERR_UNSUPPORTED, where, "dstate");
  // element counts must fit comfortably in 63 bits
  const double n = (double)batch * (double)(seqlen > 0 ? seqlen : 1) * (double)(dim > 0 ? dim : 1) * (double)dstate;
  if (n > 4.0e18) return fail(MAMBA_ERR_DIM, where, "tensor too large");
  return MAMBA_OK;
}

struct PtrCheck {
  const char* where;
  int status = MAMBA_OK;
  // A tensor that must be present when `needed`; any present pointer must be aligned.
  void req(const void* p, bool needed, const char* name) {
    if (status != MAMBA_OK) return;
    if (!p && needed) status = fail(MAMBA_ERR_NULL, where, name);
    else if (p && !aligned16(p)) status = fail(MAMBA_ERR_ALIGN, where, name);
  }
  void opt(const void* p, const char* name) { req(p, false, name); }
};

// Validation and launch shared by the real and complex decode steps.
int state_update(bool cplx, const char* where, int64_t batch, int64_t dim, int64_t dstate, int io_dtype,
                 float* state, const void* u, const void* delta, const float* delta_bias, const float* A,
                 const void* B, const void* C, const float* Dskip, const void* z, int delta_softplus, void* out,
                 void* stream) {
  int st = check_shape(where, batch, 1, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  const bool any = batch > 0 && dim > 0;
  PtrCheck pc{where};
  pc.req(state, any, "state");
  pc.req(u, any, "u");
  pc.req(delta, any, "delta");
  pc.req(A, any, "A");
  pc.req(B, any, "B");
  pc.req(C, any, "C");
  pc.req(out, any, "out");
  pc.opt(delta_bias, "delta_bias");
  pc.opt(Dskip, "Dskip");
  pc.opt(z, "z");
  if (pc.status != MAMBA_OK) return pc.status;
  if (!any) return MAMBA_OK;
  s6::StepArgs a;
  a.state = state;
  a.u = u;
  a.delta = delta;
  a.bias = delta_bias;
  a.A = A;
  a.B = B;
  a.C = C;
  a.dskip = Dskip;
  a.z = z;
  a.out = out;
  a.batch = batch;
  a.D = dim;
  a.softplus = delta_softplus != 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = cplx ? s6::launch_step_complex(a, io_dtype, (int)dstate, s) : s6::launch_step(a, io_dtype, (int)dstate, s);
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e));
  return MAMBA_OK;
}

}  // namespace

namespace s6 {
int64_t option(int key) { return key > 0 && key < kOptCount ? options().v[key].load() : 0; }
}  // namespace s6

extern "C" {

int mamba_version(void) { return 200; }

int mamba_set_option(int option, int64_t value) {
  if (!option_valid(option, value)) return fail(MAMBA_ERR_OPTION, "mamba_set_option", "option or value");
  options().v[option].store(value);
  return MAMBA_OK;
}

int64_t mamba_get_option(int option) {
  if (option <= 0 || option >= s6::kOptCount) return -1;
  return options().v[option].load();
}

int mamba_stream_status(void* stream) {
  uint32_t v = 0;
  const hipError_t e = s6::take_wait_status(static_cast<hipStream_t>(stream), &v);
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, "mamba_stream_status", hipGetErrorString(e));
  return v != 0 ? fail(MAMBA_ERR_TIMEOUT, "mamba_stream_status", "a chained-chunk wait gave up") : MAMBA_OK;
}

const char* mamba_status_string(int status) {
  switch (status) {
    case MAMBA_OK: return "ok";
    case MAMBA_ERR_NULL: return "a required pointer is NULL";
    case MAMBA_ERR_DIM: return "invalid size";
    case MAMBA_ERR_UNSUPPORTED: return "unsupported dstate (supported: 1, 2, 4, 8, 16)";
    case MAMBA_ERR_DTYPE: return "invalid io_dtype";
    case MAMBA_ERR_WORKSPACE: return "workspace missing or too small";
    case MAMBA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MAMBA_ERR_HIP: return "HIP kernel launch failed";
    case MAMBA_ERR_TIMEOUT: return "a wait between sequence chunks gave up; outputs after it are NaN";
    case MAMBA_ERR_OPTION: return "unknown option or invalid option value";
    default: return "unknown status";
  }
}

size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype) {
  if (check_shape("mamba_scan_fwd_workspace_size", batch, seqlen, dim, dstate, io_dtype) != MAMBA_OK) return 0;
  return s6::plan_scan(batch, seqlen, dim, dstate).ws_bytes;
}

int mamba_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                   const void* u, const void* delta, const float* delta_bias, const float* A,
                   const void* B, const void* C, const float* Dskip, const void* z,
                   int delta_softplus, const float* h0,
                   void* out, float* last_state,
                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* where = "mamba_scan_fwd";
  int st = check_shape(where, batch, seqlen, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  const bool tokens = batch > 0 && seqlen > 0 && dim > 0;
  const bool chans = batch > 0 && dim > 0;
  PtrCheck pc{where};
  pc.req(u, tokens, "u");
  pc.req(delta, tokens, "delta");
  pc.req(A, tokens, "A");
  pc.req(B, tokens, "B");
  pc.req(C, tokens, "C");
  pc.req(out, tokens, "out");
  pc.opt(delta_bias, "delta_bias");
  pc.opt(Dskip, "Dskip");
  pc.opt(z, "z");
  pc.opt(h0, "h0");
  pc.opt(last_state, "last_state");
  pc.opt(workspace, "workspace");
  if (pc.status != MAMBA_OK) return pc.status;
  if (!chans) return MAMBA_OK;
  const s6::ScanPlan plan = s6::plan_scan(batch, seqlen, dim, dstate);
  if (tokens && plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(MAMBA_ERR_WORKSPACE, where, "workspace");
  s6::ScanArgs a;
  a.u = u;
  a.delta = delta;
  a.bias = delta_bias;
  a.A = A;
  a.B = B;
  a.C = C;
  a.dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.out = out;
  a.last = last_state;
  a.agg_h = nullptr;
  a.agg_s = nullptr;
  a.batch = batch;
  a.L = seqlen;
  a.D = dim;
  a.chunk_len = plan.chunk_len;
  a.nchunks = plan.nchunks;
  a.softplus = delta_softplus != 0;
  hipError_t e = s6::launch_scan(a, plan, io_dtype, (int)dstate, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e));
  return MAMBA_OK;
}

size_t mamba_scan_fwd_complex_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                             int io_dtype) {
  if (check_shape("mamba_scan_fwd_complex_workspace_size", batch, seqlen, dim, dstate, io_dtype) != MAMBA_OK)
    return 0;
  return s6::plan_scan_complex(batch, seqlen, dim, dstate).ws_bytes;
}

int mamba_scan_fwd_complex(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                           const void* u, const void* delta, const float* delta_bias, const float* A,
                           const void* B, const void* C, const float* Dskip, const void* z,
                           int delta_softplus, const float* h0,
                           void* out, float* last_state,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const char* where = "mamba_scan_fwd_complex";
  int st = check_shape(where, batch, seqlen, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  const bool tokens = batch > 0 && seqlen > 0 && dim > 0;
  const bool chans = batch > 0 && dim > 0;
  PtrCheck pc{where};
  pc.req(u, tokens, "u");
  pc.req(delta, tokens, "delta");
  pc.req(A, tokens, "A");
  pc.req(B, tokens, "B");
  pc.req(C, tokens, "C");
  pc.req(out, tokens, "out");
  pc.opt(delta_bias, "delta_bias");
  pc.opt(Dskip, "Dskip");
  pc.opt(z, "z");
  pc.opt(h0, "h0");
  pc.opt(last_state, "last_state");
  pc.opt(workspace, "workspace");
  if (pc.status != MAMBA_OK) return pc.status;
  if (!chans) return MAMBA_OK;
  const s6::ScanPlan plan = s6::plan_scan_complex(batch, seqlen, dim, dstate);
  if (tokens && plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(MAMBA_ERR_WORKSPACE, where, "workspace");
  s6::ScanArgs a;
  a.u = u;
  a.delta = delta;
  a.bias = delta_bias;
  a.A = A;
  a.B = B;
  a.C = C;
  a.dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.out = out;
  a.last = last_state;
  a.agg_h = nullptr;
  a.agg_s = nullptr;
  a.batch = batch;
  a.L = seqlen;
  a.D = dim;
  a.chunk_len = plan.chunk_len;
  a.nchunks = plan.nchunks;
  a.softplus = delta_softplus != 0;
  hipError_t e =
      s6::launch_scan_complex(a, plan, io_dtype, (int)dstate, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e));
  return MAMBA_OK;
}

int mamba_state_update(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float* state,
                       const void* u, const void* delta, const float* delta_bias, const float* A,
                       const void* B, const void* C, const float* Dskip, const void* z,
                       int delta_softplus, void* out, void* stream) {
  return state_update(false, "mamba_state_update", batch, dim, dstate, io_dtype, state, u, delta, delta_bias, A, B,
                      C, Dskip, z, delta_softplus, out, stream);
}

int mamba_state_update_complex(int64_t batch, int64_t dim, int64_t dstate, int io_dtype, float* state,
                               const void* u, const void* delta, const float* delta_bias, const float* A,
                               const void* B, const void* C, const float* Dskip, const void* z,
                               int delta_softplus, void* out, void* stream) {
  return state_update(true, "mamba_state_update_complex", batch, dim, dstate, io_dtype, state, u, delta, delta_bias,
                      A, B, C, Dskip, z, delta_softplus, out, stream);
}

size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype) {
  if (check_shape("mamba_scan_bwd_workspace_size", batch, seqlen, dim, dstate, io_dtype) != MAMBA_OK) return 0;
  return s6::plan_bwd(batch, seqlen, dim, dstate).ws_bytes;
}

int mamba_scan_bwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                   const void* u, const void* delta, const float* delta_bias, const float* A,
                   const void* B, const void* C, const float* Dskip, const void* z,
                   int delta_softplus, const float* h0,
                   const void* dout, const float* dlast_state,
                   void* du, void* ddelta, float* dA, void* dB, void* dC,
                   float* dDskip, void* dz, float* ddelta_bias, float* dh0,
                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* where = "mamba_scan_bwd";
  int st = check_shape(where, batch, seqlen, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  const bool tokens = batch > 0 && seqlen > 0 && dim > 0;
  const bool chans = batch > 0 && dim > 0;
  PtrCheck pc{where};
  pc.req(u, tokens, "u");
  pc.req(delta, tokens, "delta");
  pc.req(A, tokens, "A");
  pc.req(B, tokens, "B");
  pc.req(C, tokens, "C");
  pc.req(dout, tokens, "dout");
  pc.req(du, tokens, "du");
  pc.req(ddelta, tokens, "ddelta");
  pc.req(dA, dim > 0, "dA");
  pc.req(dB, tokens, "dB");
  pc.req(dC, tokens, "dC");
  pc.opt(delta_bias, "delta_bias");
  pc.opt(Dskip, "Dskip");
  pc.opt(z, "z");
  pc.opt(h0, "h0");
  pc.opt(dlast_state, "dlast_state");
  pc.opt(dDskip, "dDskip");
  pc.opt(dz, "dz");
  pc.opt(ddelta_bias, "ddelta_bias");
  pc.opt(dh0, "dh0");
  pc.opt(workspace, "workspace");
  if (pc.status != MAMBA_OK) return pc.status;
  if (dim == 0) return MAMBA_OK;
  const s6::BwdPlan plan = s6::plan_bwd(batch, seqlen, dim, dstate);
  if (tokens && (!workspace || workspace_bytes < plan.ws_bytes))
    return fail(MAMBA_ERR_WORKSPACE, where, "workspace");
  s6::BwdArgs a{};
  a.u = u;
  a.delta = delta;
  a.bias = delta_bias;
  a.A = A;
  a.B = B;
  a.C = C;
  a.dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.dout = dout;
  a.dlast = dlast_state;
  a.du = du;
  a.ddelta = ddelta;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dDskip = dDskip;
  a.dz = dz;
  a.dbias = ddelta_bias;
  a.dh0 = dh0;
  if (tokens) {
    uint8_t* w = static_cast<uint8_t*>(workspace);
    a.hs = reinterpret_cast<float*>(w + plan.off_hs);
    a.gq = reinterpret_cast<float*>(w + plan.off_gq);
    a.sdt = reinterpret_cast<float*>(w + plan.off_sdt);
    a.srel = reinterpret_cast<float*>(w + plan.off_srel);
    a.cdt = reinterpret_cast<float*>(w + plan.off_cdt);
    a.pbc = reinterpret_cast<float*>(w + plan.off_pbc);
    a.pA = reinterpret_cast<float*>(w + plan.off_pA);
    a.pD = reinterpret_cast<float*>(w + plan.off_pD);
  }
  a.batch = chans ? batch : 0;
  a.L = seqlen;
  a.D = dim;
  a.chunk_len = plan.chunk_len;
  a.nchunks = plan.nchunks;
  a.tpc = plan.tpc;
  a.nblk = plan.nblk;
  a.softplus = delta_softplus != 0;
  hipError_t e = s6::launch_bwd(a, io_dtype, (int)dstate, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e));
  return MAMBA_OK;
}

size_t mamba_selection_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                          int64_t dt_rank, int io_dtype) {
  if (check_shape("mamba_selection_fwd_workspace_size", batch, seqlen, dim, dstate, io_dtype) != MAMBA_OK) return 0;
  if (dt_rank < 1 || dt_rank > kMaxDim) return 0;
  return s6::selection_ws_bytes(batch, seqlen, dt_rank, dstate, io_dtype);
}

int mamba_selection_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t dt_rank, int io_dtype,
                        const void* x, const void* W_x, const void* W_dt, void* delta, void* B, void* C,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const char* where = "mamba_selection_fwd";
  int st = check_shape(where, batch, seqlen, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  if (dt_rank < 1 || dt_rank > kMaxDim) return fail(MAMBA_ERR_DIM, where, "dt_rank");
  const bool tokens = batch > 0 && seqlen > 0;
  PtrCheck pc{where};
  pc.req(x, tokens && dim > 0, "x");
  pc.req(W_x, tokens && dim > 0, "W_x");
  pc.req(W_dt, tokens && dim > 0, "W_dt");
  pc.req(delta, tokens && dim > 0, "delta");
  pc.req(B, tokens, "B");
  pc.req(C, tokens, "C");
  pc.opt(workspace, "workspace");
  if (pc.status != MAMBA_OK) return pc.status;
  if (!tokens) return MAMBA_OK;
  const size_t need = s6::selection_ws_bytes(batch, seqlen, dt_rank, dstate, io_dtype);
  if (!workspace || workspace_bytes < need) return fail(MAMBA_ERR_WORKSPACE, where, "workspace");
  s6::SelArgs a{x, W_x, W_dt, delta, B, C, workspace, batch, seqlen, dim, dstate, dt_rank,
                s6::selection_ld(dt_rank, dstate)};
  hipError_t e = s6::launch_selection(a, io_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e));
  return MAMBA_OK;
}

size_t mamba_ssm_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t dt_rank,
                                    int io_dtype) {
  if (check_shape("mamba_ssm_fwd_workspace_size", batch, seqlen, dim, dstate, io_dtype) != MAMBA_OK) return 0;
  if (dt_rank < 1 || dt_rank > kMaxDim) return 0;
  const size_t e = io_dtype == MAMBA_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)batch * seqlen;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al(tok * dim * e) + 2 * al(tok * dstate * e) + s6::selection_ws_bytes(batch, seqlen, dt_rank, dstate, io_dtype) +
         al(std::max(s6::plan_scan(batch, seqlen, dim, dstate, false).ws_bytes,
                     s6::plan_scan_fused_dt(batch, seqlen, dim, dstate).ws_bytes));
}

int mamba_ssm_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t dt_rank, int io_dtype,
                  const void* x, const void* z, const void* W_x, const void* W_dt, const float* dt_bias,
                  const float* A, const float* Dskip, int delta_softplus, const float* h0,
                  void* out, float* last_state, void* workspace, size_t workspace_bytes, void* stream) {
  const char* where = "mamba_ssm_fwd";
  int st = check_shape(where, batch, seqlen, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  if (dt_rank < 1 || dt_rank > kMaxDim) return fail(MAMBA_ERR_DIM, where, "dt_rank");
  const bool tokens = batch > 0 && seqlen > 0 && dim > 0;
  PtrCheck pc{where};
  pc.req(x, tokens, "x");
  pc.req(W_x, tokens, "W_x");
  pc.req(W_dt, tokens, "W_dt");
  pc.req(A, tokens, "A");
  pc.req(out, tokens, "out");
  pc.opt(z, "z");
  pc.opt(dt_bias, "dt_bias");
  pc.opt(Dskip, "Dskip");
  pc.opt(h0, "h0");
  pc.opt(last_state, "last_state");
  pc.opt(workspace, "workspace");
  if (pc.status != MAMBA_OK) return pc.status;
  if (batch == 0 || dim == 0) return MAMBA_OK;
  const size_t need = mamba_ssm_fwd_workspace_size(batch, seqlen, dim, dstate, dt_rank, io_dtype);
  if (tokens && (!workspace || workspace_bytes < need)) return fail(MAMBA_ERR_WORKSPACE, where, "workspace");
  const size_t e = io_dtype == MAMBA_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)batch * seqlen;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* w = static_cast<uint8_t*>(workspace);
  void* delta = w;
  void* Bm = w + al(tok * dim * e);
  void* Cm = w + al(tok * dim * e) + al(tok * dstate * e);
  void* xdbl = w + al(tok * dim * e) + 2 * al(tok * dstate * e);
  void* scan_ws = static_cast<uint8_t*>(xdbl) + s6::selection_ws_bytes(batch, seqlen, dt_rank, dstate, io_dtype);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // Opt-in (MAMBA_MI355X_FUSED_DT=1): the workgroup engine projects dt itself
  // on the matrix cores (no delta tensor).  Off by default: the scan is
  // VALU-bound and the extra per-tile work there costs about what the separate
  // dt projection GEMM does.
  const bool fused = tokens && s6::wg_supported(dstate) && s6::fused_dt_supported(dstate, dt_rank, io_dtype) &&
                     aligned16(W_dt) && s6::option(s6::kOptFusedDt) == 1;
  // The scan here follows the selection GEMMs, where the mixed launch measured
  // slower than the plain one (Mamba-3B layer: 0.64 against 0.57 ms of scan).
  const s6::ScanPlan plan = fused ? s6::plan_scan_fused_dt(batch, seqlen, dim, dstate)
                                  : s6::plan_scan(batch, seqlen, dim, dstate, false);
  if (tokens) {
    s6::SelArgs sa{x, W_x, W_dt, fused ? nullptr : delta, Bm, Cm, xdbl, batch, seqlen, dim, dstate, dt_rank,
                   s6::selection_ld(dt_rank, dstate)};
    hipError_t e1 = s6::launch_selection(sa, io_dtype, hs);
    if (e1 != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e1));
  }
  s6::ScanArgs a{};
  a.u = x;
  a.delta = delta;
  a.bias = dt_bias;
  a.A = A;
  a.B = Bm;
  a.C = Cm;
  a.dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.out = out;
  a.last = last_state;
  a.batch = batch;
  a.L = seqlen;
  a.D = dim;
  a.chunk_len = plan.chunk_len;
  a.nchunks = plan.nchunks;
  a.softplus = delta_softplus != 0;
  if (fused) {
    a.delta = nullptr;
    a.dtlow = xdbl;
    a.Wdt = W_dt;
    a.R = dt_rank;
    a.ldr = s6::selection_ld(dt_rank, dstate);
  }
  hipError_t e2 = s6::launch_scan(a, plan, io_dtype, (int)dstate, tokens ? scan_ws : nullptr, hs);
  if (e2 != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(e2));
  return MAMBA_OK;
}

size_t mamba_block_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_model, int64_t dim, int64_t dstate,
                                      int64_t dt_rank, int io_dtype) {
  if (check_shape("mamba_block_fwd_workspace_size", batch, seqlen, dim, dstate, io_dtype) != MAMBA_OK) return 0;
  if (d_model < 1 || d_model > kMaxDim || dt_rank < 1 || dt_rank > kMaxDim) return 0;
  const size_t e = io_dtype == MAMBA_IO_BF16 ? 2 : 4;
  const size_t tok = (size_t)batch * seqlen;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  // x, z, y, the projections' split-K partial blocks, then the selective SSM's workspace
  return 3 * al(tok * dim * e) + al(s6::gemm_nt_part_bytes()) +
         mamba_ssm_fwd_workspace_size(batch, seqlen, dim, dstate, dt_rank, io_dtype);
}

int mamba_block_fwd(int64_t batch, int64_t seqlen, int64_t d_model, int64_t dim, int64_t dstate, int64_t dt_rank,
                    int io_dtype, const void* hidden, const void* W_in, const void* W_x, const void* W_dt,
                    const float* dt_bias, const float* A, const float* Dskip, const void* W_out, int delta_softplus,
                    const float* h0, void* out, float* last_state, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* where = "mamba_block_fwd";
  int st = check_shape(where, batch, seqlen, dim, dstate, io_dtype);
  if (st != MAMBA_OK) return st;
  if (d_model < 1 || d_model > kMaxDim) return fail(MAMBA_ERR_DIM, where, "d_model");
  if (dt_rank < 1 || dt_rank > kMaxDim) return fail(MAMBA_ERR_DIM, where, "dt_rank");
  const bool tokens = batch > 0 && seqlen > 0 && dim > 0;
  PtrCheck pc{where};
  pc.req(hidden, tokens, "hidden");
  pc.req(W_in, tokens, "W_in");
  pc.req(W_x, tokens, "W_x");
  pc.req(W_dt, tokens, "W_dt");
  pc.req(A, tokens, "A");
  pc.req(W_out, tokens, "W_out");
  pc.req(out, tokens, "out");
  pc.opt(dt_bias, "dt_bias");
  pc.opt(Dskip, "Dskip");
  pc.opt(h0, "h0");
  pc.opt(last_state, "last_state");
  pc.opt(workspace, "workspace");
  if (pc.status != MAMBA_OK) return pc.status;
  if (batch == 0 || dim == 0) return MAMBA_OK;
  const size_t need = mamba_block_fwd_workspace_size(batch, seqlen, d_model, dim, dstate, dt_rank, io_dtype);
  if (tokens && (!workspace || workspace_bytes < need)) return fail(MAMBA_ERR_WORKSPACE, where, "workspace");
  const size_t e = io_dtype == MAMBA_IO_BF16 ? 2 : 4;
  const int64_t M = batch * seqlen;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* w = static_cast<uint8_t*>(workspace);
  void* x = tokens ? w : nullptr;
  void* z = tokens ? w + al((size_t)M * dim * e) : nullptr;
  void* y = tokens ? w + 2 * al((size_t)M * dim * e) : nullptr;
  float* part = tokens ? reinterpret_cast<float*>(w + 3 * al((size_t)M * dim * e)) : nullptr;
  const size_t head = 3 * al((size_t)M * dim * e) + al(s6::gemm_nt_part_bytes());
  void* ssm_ws = tokens ? w + head : nullptr;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t he = hipSuccess;
  if (tokens) {
    // input projection: SSM branch (first dim rows of W_in) through SiLU, gate branch plain
    he = s6::launch_gemm_nt_pair(hidden, W_in, x, z, M, dim, dim, d_model, d_model, d_model, dim, io_dtype, 1, part,
                                 hs);
    if (he != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(he));
  }
  st = mamba_ssm_fwd(batch, seqlen, dim, dstate, dt_rank, io_dtype, x, z, W_x, W_dt, dt_bias, A, Dskip,
                     delta_softplus, h0, y, last_state, ssm_ws,
                     tokens ? workspace_bytes - head : 0, stream);
  if (st != MAMBA_OK) return st;
  if (tokens) {
    he = s6::launch_gemm_nt(y, W_out, out, M, d_model, dim, dim, dim, d_model, io_dtype, 0, part, hs);
    if (he != hipSuccess) return fail(MAMBA_ERR_HIP, where, hipGetErrorString(he));
  }
  return MAMBA_OK;
}

}  // extern "C"

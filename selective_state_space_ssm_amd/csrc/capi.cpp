// Host side of the C ABI declared in include/ssm_scan.h: argument checks
// (all before any HIP call), plan selection, two-pass workspace, launches.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "ssm_kernels.h"
#include "ssm_scan.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SSM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [p, p + n) of a possibly-null pointer.
struct Range {
  uintptr_t lo, hi;
  bool valid;
};
Range range_of(const void* p, uint64_t bytes) {
  Range r;
  r.valid = p != nullptr && bytes > 0;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + bytes;
  return r;
}
bool overlap(const Range& a, const Range& b) { return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi; }

// x*y with an overflow check against 2^62.
bool mul_ok(int64_t x, int64_t y, int64_t* out) {
  const int64_t lim = int64_t(1) << 62;
  if (x < 0 || y < 0) return false;
  if (x != 0 && y > lim / x) return false;
  *out = x * y;
  return true;
}

constexpr int64_t kCUs = 256;      // MI355X: 256 CUs of 4 SIMDs
constexpr int64_t kMaxChunks = 65535;
constexpr int64_t kMinChunk = 1024;
constexpr int64_t kGroup = 16;     // channels per workgroup
// Longest L: 16 rows of float32 (the rows of one workgroup, or the d_state
// rows of B or C) stay below 2^32 bytes with room for the read-ahead.
constexpr int64_t kMaxL = ((int64_t(1) << 32) - 4096) / (16 * 4);

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Plan choice, measured on MI355X with the five benchmark workloads.
//  * States per lane S: the workgroup covers 16 channels x 16 states with
//    4/S wavefronts.  Four states per lane spend the fewest issue slots per
//    state-step (fewest partial sums to add) and win when every SIMD still
//    gets two or more wavefronts (six or more workgroups per CU).  With fewer
//    channels, two states per lane double the wavefronts; one state per lane
//    would triple them but doubles the LDS traffic per state-step, which
//    measured slower at every benchmark shape.
//  * Carry vs two-pass: the carry plan keeps one state vector per (channel,
//    state) in registers for the whole length.  With fewer workgroups than
//    CUs and a long sequence, the two-pass plan splits L into K chunks
//    ([Scan page] §2.2: chunk aggregates, a scan over the K chunk totals,
//    then the fix-up) so that about eight workgroups run per CU.
int states_for(int64_t wgs) { return wgs >= 6 * kCUs ? 4 : 2; }

// Backward states per lane, measured on MI355X: four once every SIMD gets
// two or more one-wavefront workgroups (the 1.4B shape: 2048 groups); one
// (four wavefronts per group) when there are fewer groups than SIMDs (the
// 130m shape: 768 groups, three wavefronts per SIMD), where latency hiding
// outweighs the extra cross-row sums; two in between.
int bwd_states_for(int64_t groups) { return groups >= 8 * kCUs ? 4 : (groups >= 4 * kCUs ? 2 : 1); }

//  * L-parallel plan: workgroups of 4 channels whose tiles are cut into 16
//    time segments, so a problem gets batch*d_inner wavefronts whatever L
//    ([Scan page] §2.1, §3.2, §3.3).  Measured against the carry plan, it
//    wins below 2.5 channel groups per CU (b=2 d=4096 L=2048: 103 vs 126 us;
//    b=4 d=1536 L=2048: 82 vs 128 us; b=1 d=1536 L=512: 14 vs 28 us) and
//    loses above (the 130m shape, 12288 channels: 175 vs 124 us for the mixed
//    plan), where each lane's own chain is cheaper per step than fold,
//    scan and refold.  Against the two-pass plan it wins once its wavefronts
//    are at least 3/4 of the two-pass plan's (d=2048 L=65536: 786 vs 869 us;
//    d=768 L=2048: 22 vs 97 us) and loses below (d=512 L=65536: 570 vs
//    235 us).  Tiles are 256 steps, so L below 512 keeps the other plans.
constexpr int64_t kLparMinL = 512;

void choose(int64_t batch, int64_t dim, int64_t dstate, int64_t L, int* plan, int* S_out, int64_t* chunk_out,
            bool lpar_ok = true) {
  (void)dstate;
  const int64_t groups = batch * ceil_div(dim, kGroup);
  int64_t chunk = L;
  int pl = SSM_PLAN_CARRY;
  int S = states_for(groups);
  // about three channel groups per CU: one two-group block (S = 2) and one
  // one-group block (S = 1) per CU give every SIMD three chains per lane,
  // where S = 2 alone leaves half of the SIMDs with twice the work of the rest
  if (groups >= 5 * kCUs / 2 && groups < 4 * kCUs && ceil_div(dim, kGroup) >= 3) {
    pl = SSM_PLAN_MIXED;
    S = 0;
  }
  if (groups < kCUs && L >= 2 * kMinChunk) {
    int64_t K = ceil_div(8 * kCUs, groups);
    if (K > L / kMinChunk) K = L / kMinChunk;
    if (K > kMaxChunks) K = kMaxChunks;
    if (K >= 2) {
      // whole groups of four 32-step tiles: the bfloat16 one-wave kernels
      // run their tiles four at a time (identity tiles fill a chunk up)
      chunk = ceil_div(ceil_div(L, K), 128) * 128;
      pl = SSM_PLAN_TWOPASS;
      S = states_for(groups * ceil_div(L, chunk));
    }
  }
  if (lpar_ok && groups < 5 * kCUs / 2 && L >= kLparMinL) {
    const int64_t lpar_waves = batch * dim;
    const int64_t tp_waves = pl == SSM_PLAN_TWOPASS ? groups * ceil_div(L, chunk) * (4 / S) : 0;
    if (4 * lpar_waves >= 3 * tp_waves) {
      pl = SSM_PLAN_LPAR;
      S = ssm::kLparStates;
      chunk = L;
    }
  }
  if (plan) *plan = pl;
  if (S_out) *S_out = S;
  if (chunk_out) *chunk_out = chunk;
}

int check_sizes(int64_t batch, int64_t dim, int64_t dstate, int64_t L) {
  if (batch <= 0 || dim <= 0 || dstate <= 0 || L <= 0)
    return fail(SSM_EINVAL, "sizes must be positive (batch=%lld d_inner=%lld d_state=%lld L=%lld)",
                (long long)batch, (long long)dim, (long long)dstate, (long long)L);
  if (dstate > 16) return fail(SSM_EUNSUPPORTED, "d_state=%lld > 16 is not supported", (long long)dstate);
  if (batch > 65535) return fail(SSM_EUNSUPPORTED, "batch=%lld > 65535 is not supported", (long long)batch);
  if (L > kMaxL)
    return fail(SSM_EUNSUPPORTED, "L=%lld exceeds %lld (a workgroup's 16 rows are addressed with 32-bit byte offsets)",
                (long long)L, (long long)kMaxL);
  int64_t bd, bdl, bnl;
  if (!mul_ok(batch, dim, &bd) || !mul_ok(bd, L, &bdl) || !mul_ok(batch * dstate, L, &bnl) || bdl > (int64_t(1) << 60))
    return fail(SSM_EINVAL, "tensor sizes overflow");
  return SSM_OK;
}

// Where the two-pass workspace comes from: nullptr = stream-ordered
// allocation per call; otherwise a fixed region of `bytes` whose device
// address `get` returns (called only after every argument has been checked).
struct FixedWorkspace {
  size_t bytes;
  hipError_t (*get)(void** ptr);
};

int scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* delta_bias, int delta_softplus, const float* h0, void* y,
                  float* last_state, float* chunk_states, int64_t state_chunk, int64_t batch, int64_t dim,
                  int64_t dstate, int64_t L, int dtype, int plan, int S_req, int64_t chunk_req, const float* conv_w, const float* conv_b,
                  int conv_k, void* u_out, void* stream, const FixedWorkspace* fixed_ws = nullptr) {
  g_err.clear();
  if (!u || !delta || !A || !B || !C || !y)
    return fail(SSM_EINVAL, "u, delta, A, B, C and y must not be NULL");
  if (int rc = check_sizes(batch, dim, dstate, L)) return rc;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  if (delta_softplus != 0 && delta_softplus != 1) return fail(SSM_EINVAL, "delta_softplus must be 0 or 1");
  if (plan != SSM_PLAN_AUTO && plan != SSM_PLAN_CARRY && plan != SSM_PLAN_TWOPASS && plan != SSM_PLAN_MIXED &&
      plan != SSM_PLAN_LPAR)
    return fail(SSM_EINVAL, "unknown plan %d", plan);
  if (S_req != 0 && S_req != 1 && S_req != 2 && S_req != 4)
    return fail(SSM_EINVAL, "states_per_lane must be 0, 1, 2 or 4 (got %d)", S_req);
  if (chunk_req < 0 || chunk_req % 64 != 0) return fail(SSM_EINVAL, "chunk must be 0 or a positive multiple of 64");
  if (chunk_states != nullptr && (state_chunk <= 0 || state_chunk % ssm::rows_time_tile() != 0))
    return fail(SSM_EINVAL, "state_chunk must be a positive multiple of %d when chunk_states is given",
                ssm::rows_time_tile());
  if (conv_w == nullptr && (conv_b != nullptr || u_out != nullptr))
    return fail(SSM_EINVAL, "conv_b and u_out need conv_w");
  if (conv_w != nullptr && (conv_k < 1 || conv_k > 4))
    return fail(SSM_EUNSUPPORTED, "conv_k must be 1 to 4 (got %d)", conv_k);
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, y, last_state, chunk_states, conv_w, conv_b, u_out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");

  const uint64_t es = dtype == SSM_F32 ? 4 : 2;
  const uint64_t nbdl = uint64_t(batch) * dim * L, nbnl = uint64_t(batch) * dstate * L;
  const uint64_t nstate = uint64_t(batch) * dim * dstate;
  const uint64_t nsc = chunk_states ? uint64_t((L + state_chunk - 1) / state_chunk) : 0;
  const Range rin[] = {range_of(u, nbdl * es), range_of(delta, nbdl * es), range_of(z, nbdl * es),
                       range_of(B, nbnl * es), range_of(C, nbnl * es), range_of(A, uint64_t(dim) * dstate * 4),
                       range_of(D, uint64_t(dim) * 4), range_of(delta_bias, uint64_t(dim) * 4),
                       range_of(h0, nstate * 4), range_of(conv_w, uint64_t(dim) * (conv_w ? conv_k : 0) * 4),
                       range_of(conv_b, uint64_t(dim) * 4)};
  const Range ry = range_of(y, nbdl * es);
  const Range rl = range_of(last_state, nstate * 4);
  const Range rc = range_of(chunk_states, nsc * nstate * 4);
  const Range ru = range_of(u_out, nbdl * es);
  for (const Range& r : rin)
    if (overlap(ry, r) || overlap(rl, r) || overlap(rc, r) || overlap(ru, r))
      return fail(SSM_EINVAL, "outputs must not overlap inputs");
  if (overlap(ry, rl) || overlap(ry, rc) || overlap(rl, rc) || overlap(ru, ry) || overlap(ru, rl) || overlap(ru, rc))
    return fail(SSM_EINVAL, "outputs overlap each other");

  int pl, S;
  int64_t chunk;
  // a forced plan takes the states per lane and chunk of the choice among
  // the other plans
  choose(batch, dim, dstate, L, &pl, &S, &chunk, plan == SSM_PLAN_AUTO);
  if (plan != SSM_PLAN_AUTO) pl = plan;
  if (S_req) S = S_req;
  if (S == 0) S = 2;  // states per lane of a carry or two-pass plan forced over a mixed choice
  if (pl == SSM_PLAN_TWOPASS) {
    if (chunk_req)
      chunk = chunk_req;
    else if (chunk >= L)  // two-pass forced where auto would not split: two chunks
      chunk = ceil_div(ceil_div(L, 2), 64) * 64;
    if (chunk >= L) pl = SSM_PLAN_CARRY;  // a single chunk is the carry plan
  }

  ssm::FwdArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.y = y; a.last_state = last_state; a.h_init = nullptr; a.agg_p = nullptr; a.agg_h = nullptr;
  a.h0 = h0; a.chunk_states = chunk_states; a.state_chunk = chunk_states ? state_chunk : 0;
  a.batch = batch; a.dim = dim; a.dstate = dstate; a.L = L; a.softplus = delta_softplus;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_k = conv_w ? conv_k : 0; a.u_out = u_out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SSM_BF16;

  if (pl == SSM_PLAN_MIXED) {
    a.chunk = L;
    // one two-group block per three groups, the rest one-group blocks; with
    // fewer than three groups (a forced mixed plan) every block has one group
    const int64_t gd = ceil_div(dim, kGroup);
    hipError_t e = ssm::launch_mixed_full(a, bf16, gd / 3, 1, st);
    if (e != hipSuccess) return hip_fail(e, "selective-scan launch");
    return SSM_OK;
  }
  if (pl == SSM_PLAN_LPAR) {
    a.chunk = L;
    hipError_t e = ssm::launch_lpar(a, bf16, st);
    if (e != hipSuccess) return hip_fail(e, "selective-scan launch");
    return SSM_OK;
  }
  if (pl == SSM_PLAN_CARRY) {
    a.chunk = L;
    hipError_t e = ssm::launch_rows_full(a, bf16, S, 1, st);
    if (e != hipSuccess) return hip_fail(e, "selective-scan launch");
    return SSM_OK;
  }

  const int64_t K = ceil_div(L, chunk);
  if (K > kMaxChunks) return fail(SSM_EUNSUPPORTED, "%lld chunks exceed the limit of %lld", (long long)K,
                                  (long long)kMaxChunks);
  const int64_t rows = batch * dstate * dim;
  const size_t per = sizeof(float) * static_cast<size_t>(rows) * static_cast<size_t>(K);
  void* ws = nullptr;
  hipError_t e;
  if (fixed_ws != nullptr) {
    if (3 * per > fixed_ws->bytes)
      return fail(SSM_EUNSUPPORTED,
                  "the two-pass workspace of %zu bytes (%lld chunks) exceeds the %zu-byte scratch of the "
                  "no-allocation entry point", 3 * per, (long long)K, fixed_ws->bytes);
    e = fixed_ws->get(&ws);
    if (e != hipSuccess) return hip_fail(e, "no-allocation scratch lookup");
  } else {
    e = hipMallocAsync(&ws, 3 * per, st);
    if (e == hipErrorOutOfMemory) return fail(SSM_ENOMEM, "two-pass workspace of %zu bytes", 3 * per);
    if (e != hipSuccess) return hip_fail(e, "two-pass workspace allocation");
  }
  float* agg_p = static_cast<float*>(ws);
  float* agg_h = agg_p + rows * K;
  float* h_init = agg_h + rows * K;
  a.chunk = chunk;
  a.agg_p = agg_p;
  a.agg_h = agg_h;
  e = ssm::launch_rows_agg(a, bf16, S, K - 1, st);
  if (e == hipSuccess) e = ssm::launch_combine(agg_p, agg_h, h0, h_init, batch, dim, dstate, K, st);
  if (e == hipSuccess) {
    a.agg_p = nullptr;
    a.agg_h = nullptr;
    a.h_init = h_init;
    e = ssm::launch_rows_full(a, bf16, S, K, st);
  }
  hipError_t ef = fixed_ws != nullptr ? hipSuccess : hipFreeAsync(ws, st);
  if (e != hipSuccess) return hip_fail(e, "two-pass launch");
  if (ef != hipSuccess) return hip_fail(ef, "two-pass workspace release");
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int delta_softplus, void* y, float* last_state,
                 int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype, void* stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, nullptr, y, last_state, nullptr, 0, batch,
                       d_inner, d_state, L, dtype, SSM_PLAN_AUTO, 0, 0, nullptr, nullptr, 0, nullptr, stream);
}

int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                         const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                         float* last_state, int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype,
                         void* stream) {
  static const FixedWorkspace scratch{ssm::kNoAllocScratchBytes, &ssm::noalloc_scratch};
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, nullptr, y, last_state, nullptr, 0, batch,
                       d_inner, d_state, L, dtype, SSM_PLAN_AUTO, 0, 0, nullptr, nullptr, 0, nullptr, stream,
                       &scratch);
}

int ssm_scan_fwd_plan(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                      float* last_state, int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype,
                      int plan, int states_per_lane, int64_t chunk, void* stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, nullptr, y, last_state, nullptr, 0, batch,
                       d_inner, d_state, L, dtype, plan, states_per_lane, chunk, nullptr, nullptr, 0, nullptr, stream);
}

int ssm_scan_fwd_states(const void* u, const void* delta, const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* delta_bias, int delta_softplus, const float* h0,
                        void* y, float* last_state, float* chunk_states, int64_t state_chunk, int64_t batch,
                        int64_t d_inner, int64_t d_state, int64_t L, int dtype, int plan, void* stream) {
  return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, y, last_state, chunk_states,
                       state_chunk, batch, d_inner, d_state, L, dtype, plan, 0, 0, nullptr, nullptr, 0, nullptr,
                       stream);
}

int ssm_scan_fwd_conv(const void* x, const float* conv_w, const float* conv_b, int conv_k, const void* delta,
                      const float* A, const void* B, const void* C, const float* D, const void* z,
                      const float* delta_bias, int delta_softplus, const float* h0, void* y, float* last_state,
                      void* u_out, float* chunk_states, int64_t state_chunk, int64_t batch, int64_t d_inner,
                      int64_t d_state, int64_t L, int dtype, int plan, void* stream) {
  g_err.clear();
  if (!conv_w) return fail(SSM_EINVAL, "conv_w must not be NULL");
  return scan_fwd_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, y, last_state, chunk_states,
                       state_chunk, batch, d_inner, d_state, L, dtype, plan, 0, 0, conv_w, conv_b, conv_k, u_out,
                       stream);
}

int ssm_scan_plan_for(int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype, int* plan,
                      int* states_per_lane, int64_t* chunk) {
  g_err.clear();
  if (int rc = check_sizes(batch, d_inner, d_state, L)) return rc;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  choose(batch, d_inner, d_state, L, plan, states_per_lane, chunk);
  return SSM_OK;
}

int ssm_step(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
             const void* z, const float* delta_bias, int delta_softplus, const float* state_in, float* state_out,
             void* y, int64_t batch, int64_t d_inner, int64_t d_state, int dtype, void* stream) {
  g_err.clear();
  if (!u || !delta || !A || !B || !C || !state_in || !state_out || !y)
    return fail(SSM_EINVAL, "u, delta, A, B, C, state_in, state_out and y must not be NULL");
  if (int rc = check_sizes(batch, d_inner, d_state, 1)) return rc;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  if (delta_softplus != 0 && delta_softplus != 1) return fail(SSM_EINVAL, "delta_softplus must be 0 or 1");
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, state_in, state_out, y};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");
  const uint64_t es = dtype == SSM_F32 ? 4 : 2;
  const uint64_t nbd = uint64_t(batch) * d_inner, nbn = uint64_t(batch) * d_state;
  const uint64_t nstate = nbd * d_state;
  const Range rin[] = {range_of(u, nbd * es), range_of(delta, nbd * es), range_of(z, nbd * es),
                       range_of(B, nbn * es), range_of(C, nbn * es), range_of(A, uint64_t(d_inner) * d_state * 4),
                       range_of(D, uint64_t(d_inner) * 4), range_of(delta_bias, uint64_t(d_inner) * 4)};
  const Range ry = range_of(y, nbd * es);
  const Range rsi = range_of(state_in, nstate * 4), rso = range_of(state_out, nstate * 4);
  for (const Range& r : rin)
    if (overlap(ry, r) || overlap(rso, r) || overlap(rsi, r))
      return fail(SSM_EINVAL, "y, state_in and state_out must not overlap the other inputs");
  if (overlap(ry, rso) || overlap(ry, rsi)) return fail(SSM_EINVAL, "y overlaps the state");
  if (state_in != state_out && overlap(rsi, rso))
    return fail(SSM_EINVAL, "state_out must equal state_in or be disjoint from it");
  ssm::StepArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.state_in = state_in; a.state_out = state_out; a.y = y;
  a.batch = batch; a.dim = d_inner; a.dstate = d_state; a.softplus = delta_softplus;
  hipError_t e = ssm::launch_step(a, dtype == SSM_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "recurrent step launch");
  return SSM_OK;
}

}  // extern "C"

namespace {

int scan_bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                  const void* z, const float* delta_bias, int delta_softplus, const float* h0,
                  const float* chunk_states, int64_t state_chunk, const void* dy, const float* dlast, void* du,
                  void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                  int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype, int states_per_lane,
                  const float* conv_w, const float* conv_b, int conv_k, float* dconv_w, float* dconv_b,
                  void* stream) {
  g_err.clear();
  if (!u || !delta || !A || !B || !C || !chunk_states || !dy || !du || !ddelta || !dA || !dB || !dC)
    return fail(SSM_EINVAL, "u, delta, A, B, C, chunk_states, dy, du, ddelta, dA, dB and dC must not be NULL");
  if ((z != nullptr) != (dz != nullptr)) return fail(SSM_EINVAL, "dz must be given if and only if z is");
  if (int rc = check_sizes(batch, d_inner, d_state, L)) return rc;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  if (delta_softplus != 0 && delta_softplus != 1) return fail(SSM_EINVAL, "delta_softplus must be 0 or 1");
  if (state_chunk <= 0 || state_chunk % ssm::rows_time_tile() != 0 || state_chunk > ssm::kBwdMaxChunk)
    return fail(SSM_EINVAL, "state_chunk must be a positive multiple of %d and at most %d (got %lld)",
                ssm::rows_time_tile(), ssm::kBwdMaxChunk, (long long)state_chunk);
  if (states_per_lane != 0 && states_per_lane != 1 && states_per_lane != 2 && states_per_lane != 4)
    return fail(SSM_EINVAL, "states_per_lane must be 0, 1, 2 or 4 (got %d)", states_per_lane);
  if (conv_w != nullptr && (conv_k < 1 || conv_k > 4))
    return fail(SSM_EUNSUPPORTED, "conv_k must be 1 to 4 (got %d)", conv_k);
  if (conv_w != nullptr && dconv_w == nullptr) return fail(SSM_EINVAL, "dconv_w must not be NULL");
  const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, chunk_states, dy, dlast,
                        du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, conv_w, conv_b, dconv_w, dconv_b};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");
  const uint64_t es = dtype == SSM_F32 ? 4 : 2;
  const uint64_t K = uint64_t(ceil_div(L, state_chunk));
  const uint64_t nbdl = uint64_t(batch) * d_inner * L, nbnl = uint64_t(batch) * d_state * L;
  const uint64_t nbdn = uint64_t(batch) * d_inner * d_state, ndn = uint64_t(d_inner) * d_state;
  const Range rin[] = {range_of(u, nbdl * es), range_of(delta, nbdl * es), range_of(z, nbdl * es),
                       range_of(dy, nbdl * es), range_of(B, nbnl * es), range_of(C, nbnl * es),
                       range_of(A, ndn * 4), range_of(D, uint64_t(d_inner) * 4),
                       range_of(delta_bias, uint64_t(d_inner) * 4), range_of(h0, nbdn * 4),
                       range_of(chunk_states, K * nbdn * 4), range_of(dlast, nbdn * 4),
                       range_of(conv_w, uint64_t(d_inner) * (conv_w ? conv_k : 0) * 4),
                       range_of(conv_b, uint64_t(d_inner) * 4)};
  const Range rout[] = {range_of(du, nbdl * es), range_of(ddelta, nbdl * es), range_of(dz, nbdl * es),
                        range_of(dA, ndn * 4), range_of(dB, nbnl * 4), range_of(dC, nbnl * 4),
                        range_of(dD, uint64_t(d_inner) * 4), range_of(ddelta_bias, uint64_t(d_inner) * 4),
                        range_of(dh0, nbdn * 4), range_of(dconv_w, uint64_t(d_inner) * (conv_w ? conv_k : 0) * 4),
                        range_of(dconv_b, uint64_t(d_inner) * 4)};
  for (size_t i = 0; i < sizeof(rout) / sizeof(rout[0]); ++i) {
    for (const Range& r : rin)
      if (overlap(rout[i], r)) return fail(SSM_EINVAL, "gradient outputs must not overlap any input");
    for (size_t j = i + 1; j < sizeof(rout) / sizeof(rout[0]); ++j)
      if (overlap(rout[i], rout[j])) return fail(SSM_EINVAL, "gradient outputs must not overlap each other");
  }
  const int64_t groups = batch * ceil_div(d_inner, kGroup);
  int S = states_per_lane != 0 ? states_per_lane : bwd_states_for(groups);
  // with the conv in front, four states per lane run out of registers
  // (spills) and LDS (occupancy): two measured faster at the 1.4B shape
  if (states_per_lane == 0 && conv_w != nullptr && S == 4) S = 2;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // every output that the kernel sums into with atomics, cleared by one launch
  ssm::ZeroList zl{};
  auto clear = [&](float* q, int64_t n) {
    if (q != nullptr && n > 0) {
      zl.p[zl.count] = q;
      zl.n[zl.count] = n;
      ++zl.count;
    }
  };
  clear(dA, int64_t(ndn));
  clear(dB, int64_t(nbnl));
  clear(dC, int64_t(nbnl));
  clear(dD, d_inner);
  clear(ddelta_bias, d_inner);
  if (conv_w) {
    clear(dconv_w, d_inner * conv_k);
    clear(dconv_b, d_inner);
  }
  hipError_t e = ssm::launch_zero(zl, st);
  if (e != hipSuccess) return hip_fail(e, "gradient clear launch");
  ssm::BwdArgs a{};
  a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.h0 = h0; a.chunk_states = chunk_states; a.dy = dy; a.dlast = dlast;
  a.du = du; a.ddelta = ddelta; a.dz = dz; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dbias = ddelta_bias;
  a.dh0 = dh0;
  a.batch = batch; a.dim = d_inner; a.dstate = d_state; a.L = L; a.state_chunk = state_chunk;
  a.softplus = delta_softplus;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_k = conv_w ? conv_k : 0; a.dconv_w = dconv_w; a.dconv_b = dconv_b;
  e = ssm::launch_bwd(a, dtype == SSM_BF16, S, st);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C, const float* D,
                 const void* z, const float* delta_bias, int delta_softplus, const float* h0,
                 const float* chunk_states, int64_t state_chunk, const void* dy, const float* dlast, void* du,
                 void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, float* ddelta_bias, float* dh0,
                 int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype, int states_per_lane,
                 void* stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, chunk_states, state_chunk, dy, dlast,
                       du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, batch, d_inner, d_state, L, dtype,
                       states_per_lane, nullptr, nullptr, 0, nullptr, nullptr, stream);
}

int ssm_scan_bwd_conv(const void* x, const float* conv_w, const float* conv_b, int conv_k, const void* delta,
                      const float* A, const void* B, const void* C, const float* D, const void* z,
                      const float* delta_bias, int delta_softplus, const float* h0, const float* chunk_states,
                      int64_t state_chunk, const void* dy, const float* dlast, void* dx, float* dconv_w,
                      float* dconv_b, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                      float* ddelta_bias, float* dh0, int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                      int dtype, int states_per_lane, void* stream) {
  g_err.clear();
  if (!conv_w) return fail(SSM_EINVAL, "conv_w must not be NULL");
  return scan_bwd_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, chunk_states, state_chunk, dy, dlast,
                       dx, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0, batch, d_inner, d_state, L, dtype,
                       states_per_lane, conv_w, conv_b, conv_k, dconv_w, dconv_b, stream);
}

int ssm_step_conv(const void* x, const float* conv_w, const float* conv_b, int conv_k, const float* conv_state_in,
                  float* conv_state_out, const void* delta, const float* A, const void* B, const void* C,
                  const float* D, const void* z, const float* delta_bias, int delta_softplus, const float* state_in,
                  float* state_out, void* y, void* u_out, int64_t batch, int64_t d_inner, int64_t d_state, int dtype,
                  void* stream) {
  g_err.clear();
  if (!x || !conv_w || !delta || !A || !B || !C || !state_in || !state_out || !y)
    return fail(SSM_EINVAL, "x, conv_w, delta, A, B, C, state_in, state_out and y must not be NULL");
  if (int rc = check_sizes(batch, d_inner, d_state, 1)) return rc;
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  if (delta_softplus != 0 && delta_softplus != 1) return fail(SSM_EINVAL, "delta_softplus must be 0 or 1");
  if (conv_k < 1 || conv_k > 4) return fail(SSM_EUNSUPPORTED, "conv_k must be 1 to 4 (got %d)", conv_k);
  if (conv_k > 1 && (!conv_state_in || !conv_state_out))
    return fail(SSM_EINVAL, "conv_state_in and conv_state_out must not be NULL when conv_k > 1");
  const void* ptrs[] = {x, conv_w, conv_b, conv_state_in, conv_state_out, delta, A, B, C, D, z, delta_bias,
                        state_in, state_out, y, u_out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");
  const uint64_t es = dtype == SSM_F32 ? 4 : 2;
  const uint64_t nbd = uint64_t(batch) * d_inner, nbn = uint64_t(batch) * d_state;
  const uint64_t nstate = nbd * d_state, ncs = nbd * uint64_t(conv_k - 1);
  const Range rin[] = {range_of(x, nbd * es), range_of(delta, nbd * es), range_of(z, nbd * es),
                       range_of(B, nbn * es), range_of(C, nbn * es), range_of(A, uint64_t(d_inner) * d_state * 4),
                       range_of(D, uint64_t(d_inner) * 4), range_of(delta_bias, uint64_t(d_inner) * 4),
                       range_of(conv_w, uint64_t(d_inner) * conv_k * 4), range_of(conv_b, uint64_t(d_inner) * 4)};
  const Range ry = range_of(y, nbd * es), ru = range_of(u_out, nbd * es);
  const Range rsi = range_of(state_in, nstate * 4), rso = range_of(state_out, nstate * 4);
  const Range rci = range_of(conv_state_in, ncs * 4), rco = range_of(conv_state_out, ncs * 4);
  for (const Range& r : rin)
    if (overlap(ry, r) || overlap(ru, r) || overlap(rso, r) || overlap(rsi, r) || overlap(rco, r) || overlap(rci, r))
      return fail(SSM_EINVAL, "outputs and states must not overlap the other inputs");
  const Range outs[] = {ry, ru, rso, rco};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(SSM_EINVAL, "outputs overlap each other");
  if (overlap(ry, rsi) || overlap(ry, rci) || overlap(ru, rsi) || overlap(ru, rci) || overlap(rso, rci) ||
      overlap(rco, rsi))
    return fail(SSM_EINVAL, "outputs overlap a state input");
  if (state_in != state_out && overlap(rsi, rso))
    return fail(SSM_EINVAL, "state_out must equal state_in or be disjoint from it");
  if (conv_state_in != conv_state_out && overlap(rci, rco))
    return fail(SSM_EINVAL, "conv_state_out must equal conv_state_in or be disjoint from it");
  ssm::StepArgs a{};
  a.u = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
  a.state_in = state_in; a.state_out = state_out; a.y = y;
  a.batch = batch; a.dim = d_inner; a.dstate = d_state; a.softplus = delta_softplus;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_k = conv_k; a.conv_state_in = conv_state_in;
  a.conv_state_out = conv_state_out; a.u_out = u_out;
  hipError_t e = ssm::launch_step(a, dtype == SSM_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "recurrent step launch");
  return SSM_OK;
}

int ssm_out_proj(const void* y, const void* W, void* out, int64_t batch, int64_t d_inner, int64_t d_model,
                 int64_t L, int dtype, void* stream) {
  g_err.clear();
  if (!y || !W || !out) return fail(SSM_EINVAL, "y, W and out must not be NULL");
  if (batch <= 0 || d_inner <= 0 || d_model <= 0 || L <= 0)
    return fail(SSM_EINVAL, "sizes must be positive (batch=%lld d_inner=%lld d_model=%lld L=%lld)",
                (long long)batch, (long long)d_inner, (long long)d_model, (long long)L);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  const void* ptrs[] = {y, W, out};
  for (const void* q : ptrs)
    if (!aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");
  const int64_t es = dtype == SSM_F32 ? 4 : 2;
  const int64_t lim = int64_t(1) << 31;
  int64_t yrow, wsz, orow, tmp;
  if (!mul_ok(d_inner, L, &tmp) || !mul_ok(tmp, es, &yrow) || yrow >= lim || !mul_ok(d_model, d_inner, &tmp) ||
      !mul_ok(tmp, es, &wsz) || wsz >= lim || !mul_ok(L, d_model, &tmp) || !mul_ok(tmp, es, &orow) || orow >= lim)
    return fail(SSM_EUNSUPPORTED, "a batch row of y or out, or W, reaches 2^31 bytes");
  int64_t ybytes, obytes;
  if (!mul_ok(yrow, batch, &ybytes) || !mul_ok(orow, batch, &obytes)) return fail(SSM_EINVAL, "tensor sizes overflow");
  if (ssm::proj_tiles(dtype == SSM_BF16, batch, d_model, L) >= lim)
    return fail(SSM_EUNSUPPORTED, "too many output tiles for one launch");
  const Range ry = range_of(y, uint64_t(ybytes)), rw = range_of(W, uint64_t(wsz)), ro = range_of(out, uint64_t(obytes));
  if (overlap(ro, ry) || overlap(ro, rw)) return fail(SSM_EINVAL, "out must not overlap y or W");
  ssm::ProjArgs a{y, W, out, batch, d_inner, d_model, L};
  hipError_t e = ssm::launch_out_proj(a, dtype == SSM_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "out-projection launch");
  return SSM_OK;
}

int ssm_out_proj_bwd(const void* y, const void* W, const void* dout, void* dy, void* dW, int64_t batch,
                     int64_t d_inner, int64_t d_model, int64_t L, int dtype, void* stream) {
  g_err.clear();
  if (!y || !W || !dout) return fail(SSM_EINVAL, "y, W and dout must not be NULL");
  if (!dy && !dW) return fail(SSM_EINVAL, "at least one of dy and dW must be given");
  if (batch <= 0 || d_inner <= 0 || d_model <= 0 || L <= 0)
    return fail(SSM_EINVAL, "sizes must be positive (batch=%lld d_inner=%lld d_model=%lld L=%lld)",
                (long long)batch, (long long)d_inner, (long long)d_model, (long long)L);
  if (dtype != SSM_F32 && dtype != SSM_BF16) return fail(SSM_EUNSUPPORTED, "dtype %d is not supported", dtype);
  const void* ptrs[] = {y, W, dout, dy, dW};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");
  const int64_t es = dtype == SSM_F32 ? 4 : 2;
  const int64_t lim = int64_t(1) << 31;
  int64_t yrow, wsz, orow, w4, tmp;
  if (!mul_ok(d_inner, L, &tmp) || !mul_ok(tmp, es, &yrow) || yrow >= lim || !mul_ok(d_model, d_inner, &tmp) ||
      !mul_ok(tmp, es, &wsz) || !mul_ok(tmp, 4, &w4) || w4 >= lim || !mul_ok(L, d_model, &tmp) ||
      !mul_ok(tmp, es, &orow) || orow >= lim)
    return fail(SSM_EUNSUPPORTED, "a batch row of y or dout, or W in float32, reaches 2^31 bytes");
  int64_t ybytes, obytes;
  if (!mul_ok(yrow, batch, &ybytes) || !mul_ok(orow, batch, &obytes)) return fail(SSM_EINVAL, "tensor sizes overflow");
  ssm::ProjBwdArgs a{y, W, dout, dy, dW, batch, d_inner, d_model, L};
  const bool bf16 = dtype == SSM_BF16;
  if (ssm::proj_bwd_tiles(bf16, a) >= lim) return fail(SSM_EUNSUPPORTED, "too many output tiles for one launch");
  const Range ins[] = {range_of(y, uint64_t(ybytes)), range_of(W, uint64_t(wsz)), range_of(dout, uint64_t(obytes))};
  const Range rdy = range_of(dy, uint64_t(ybytes)), rdw = range_of(dW, uint64_t(wsz));
  for (const Range& r : ins)
    if (overlap(rdy, r) || overlap(rdw, r)) return fail(SSM_EINVAL, "dy and dW must not overlap y, W or dout");
  if (overlap(rdy, rdw)) return fail(SSM_EINVAL, "dy and dW overlap");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t wbytes = ssm::proj_bwd_workspace_bytes(bf16, a);
  void* ws = nullptr;
  if (wbytes > 0) {
    hipError_t e = hipMallocAsync(&ws, wbytes, st);
    if (e == hipErrorOutOfMemory) return fail(SSM_ENOMEM, "dW split workspace of %zu bytes", wbytes);
    if (e != hipSuccess) return hip_fail(e, "dW split workspace allocation");
  }
  hipError_t e = ssm::launch_out_proj_bwd(a, bf16, static_cast<float*>(ws), wbytes, st);
  hipError_t ef = ws ? hipFreeAsync(ws, st) : hipSuccess;
  if (e != hipSuccess) return hip_fail(e, "out-projection backward launch");
  if (ef != hipSuccess) return hip_fail(ef, "dW split workspace release");
  return SSM_OK;
}

int affine_scan(const float* a, const float* b, float* out_a, float* out_b, int64_t rows, int64_t L,
                void* stream) {
  g_err.clear();
  if (!a || !b || !out_b) return fail(SSM_EINVAL, "a, b and out_b must not be NULL");
  if (rows <= 0 || L <= 0) return fail(SSM_EINVAL, "rows and L must be positive");
  int64_t n;
  if (!mul_ok(rows, L, &n) || n > (int64_t(1) << 60)) return fail(SSM_EINVAL, "tensor sizes overflow");
  const void* ptrs[] = {a, b, out_a, out_b};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(SSM_EINVAL, "every pointer must be 16-byte aligned");
  const uint64_t bytes = uint64_t(n) * 4;
  const Range ra = range_of(a, bytes), rb = range_of(b, bytes), roa = range_of(out_a, bytes),
              rob = range_of(out_b, bytes);
  if (overlap(roa, rob)) return fail(SSM_EINVAL, "out_a and out_b overlap");
  if (!(out_b == b) && (overlap(rob, ra) || overlap(rob, rb)))
    return fail(SSM_EINVAL, "out_b must equal b or be disjoint from the inputs");
  if (out_a && !(out_a == a) && (overlap(roa, ra) || overlap(roa, rb)))
    return fail(SSM_EINVAL, "out_a must equal a or be disjoint from the inputs");
  if (out_b == b && overlap(rob, ra)) return fail(SSM_EINVAL, "a and b overlap");
  hipError_t e = ssm::launch_affine_scan(a, b, out_a, out_b, rows, L, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "affine_scan launch");
  return SSM_OK;
}

int affine_scan_order(int* items_per_lane, int* lanes, int* waves, int* chunk) {
  if (items_per_lane) *items_per_lane = ssm::kAffT;
  if (lanes) *lanes = ssm::kAffLanes;
  if (waves) *waves = ssm::kAffW;
  if (chunk) *chunk = ssm::kAffChunk;
  return SSM_OK;
}

const char* ssm_last_error(void) { return g_err.c_str(); }

}  // extern "C"

// Internal interface between the host C ABI (capi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

enum { kFull = 0, kAgg = 1 };

// Arguments of the row-layout selective-scan kernel (by value).
struct FwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // nullable
  const void* z;            // nullable: no gate
  const float* bias;        // nullable
  void* y;                  // kFull
  float* last_state;        // kFull, nullable
  const float* h_init;      // kFull: [K][b][n][d] chunk start states, nullable (zero)
  const float* h0;          // [b][d][n] start state of the sequence, nullable (zero)
  float* chunk_states;      // kFull: [b][Ks][d][n] states at every state_chunk boundary, nullable
  int64_t state_chunk;      // steps per chunk_states entry (multiple of the time tile)
  float* agg_p;             // kAgg: [K][b][n][d] chunk decay products
  float* agg_h;             // kAgg: [K][b][n][d] chunk end states from zero
  int64_t batch, dim, dstate, L;
  int64_t chunk;            // steps per chunk (grid z); = L for one chunk
  int softplus;
  const float* conv_w;      // nullable: [d][conv_k] causal conv1d in front (u then holds x)
  const float* conv_b;      // [d] nullable
  int conv_k;               // 1..4 taps
  void* u_out;              // nullable: [b][d][L] silu(conv1d(x)), kFull only
};

// Sizes and flags of one row-layout launch (by value).
struct CsSizes {
  int64_t batch, dim, dstate, L;
  int64_t chunk;
  int64_t state_chunk;   // chunk_states spacing (0: none)
  int softplus;
  int convk;             // conv1d taps (0: no conv)
};

// S = states per lane (1, 2 or 4); a workgroup is 16 channels x 16 states
// in 4/S wavefronts.
size_t rows_smem_bytes(int S, int mode);
int rows_time_tile();
hipError_t launch_rows_full(const FwdArgs& a, bool bf16, int S, int64_t nchunks, hipStream_t st);
hipError_t launch_rows_agg(const FwdArgs& a, bool bf16, int S, int64_t nchunks, hipStream_t st);
// Mixed launch: per batch row, `pairs` blocks of two groups at S = 2 and the
// remaining groups at S = 1 (one group per block).
hipError_t launch_mixed_full(const FwdArgs& a, bool bf16, int64_t pairs, int64_t nchunks, hipStream_t st);
// h0: [batch][dim][dstate] start state or null; rows = batch*dstate*dim.
// With kCombScanMinChunks or more chunks the carry runs as a blocked scan.
constexpr int64_t kCombScanMinChunks = 64;
hipError_t launch_combine(const float* agg_p, const float* agg_h, const float* h0, float* h_init, int64_t batch,
                          int64_t dim, int64_t dstate, int64_t K, hipStream_t st);

// One recurrent step (decode) for every (batch, channel).
struct StepArgs {
  const void* u;        // [b][d]
  const void* delta;    // [b][d]
  const float* A;       // [d][n]
  const void* B;        // [b][n]
  const void* C;        // [b][n]
  const float* D;       // [d] nullable
  const void* z;        // [b][d] nullable
  const float* bias;    // [d] nullable
  const float* state_in;  // [b][d][n]
  float* state_out;       // [b][d][n], may equal state_in
  void* y;              // [b][d]
  int64_t batch, dim, dstate;
  int softplus;
  const float* conv_w;          // nullable: [d][conv_k] conv1d in front (u then holds x_t)
  const float* conv_b;          // [d] nullable
  int conv_k;                   // 1..4
  const float* conv_state_in;   // [b][d][conv_k-1]
  float* conv_state_out;        // [b][d][conv_k-1], may equal conv_state_in
  void* u_out;                  // [b][d] nullable
};
hipError_t launch_step(const StepArgs& a, bool bf16, hipStream_t st);

// Gradients of the selective scan by chunked recomputation from the states
// the forward kept at every state_chunk boundary.
struct BwdArgs {
  const void* u;              // [b][d][L]
  const void* delta;          // [b][d][L]
  const float* A;             // [d][n]
  const void* B;              // [b][n][L]
  const void* C;              // [b][n][L]
  const float* D;             // [d] nullable
  const void* z;              // [b][d][L] nullable: no gate
  const float* bias;          // [d] nullable
  const float* h0;            // [b][d][n] nullable (zero)
  const float* chunk_states;  // [b][K][d][n], entry k = state after step min((k+1)*sc, L) - 1
  const void* dy;             // [b][d][L]
  const float* dlast;         // [b][d][n] nullable (zero)
  void* du;                   // [b][d][L]
  void* ddelta;               // [b][d][L]
  void* dz;                   // [b][d][L], iff z
  float* dA;                  // [d][n], accumulated: zeroed by the caller of launch_bwd
  float* dB;                  // [b][n][L], accumulated
  float* dC;                  // [b][n][L], accumulated
  float* dD;                  // [d] nullable, accumulated
  float* dbias;               // [d] nullable, accumulated
  float* dh0;                 // [b][d][n] nullable, written
  int64_t batch, dim, dstate, L;
  int64_t state_chunk;        // sc: multiple of the backward tile, at most kBwdMaxChunk
  int softplus;
  const float* conv_w;        // nullable: [d][conv_k] conv1d in front (u then holds x, du receives dx)
  const float* conv_b;        // [d] nullable
  int conv_k;                 // 1..4
  float* dconv_w;             // [d][conv_k], accumulated
  float* dconv_b;             // [d] nullable, accumulated
};
constexpr int kBwdTile = 16;       // steps per backward tile
constexpr int kBwdMaxChunk = 512;  // largest state_chunk (LDS holds one state per tile of a chunk)
size_t bwd_smem_bytes(int S, int64_t state_chunk, bool conv);
hipError_t launch_bwd(const BwdArgs& a, bool bf16, int S, hipStream_t st);
// Fill n floats with zero (a kernel, not a memset).
// Float buffers to clear with one launch (n[i] elements at p[i]; count of
// them used, at most kZeroBufs).
constexpr int kZeroBufs = 8;
struct ZeroList {
  float* p[kZeroBufs];
  int64_t n[kZeroBufs];
  int count;
};
hipError_t launch_zero(const ZeroList& z, hipStream_t st);

// L-parallel single-pass forward (ssm_lpar.hip): workgroups of 4 channels x
// all states of one batch row; each tile is 16 segments of kLparSegSteps
// steps, one per lane of a row of 16.  Takes every field of `a` that the
// carry plan takes: u (or x with the conv), delta, A, B, C, D, z, bias, h0,
// y, last_state, chunk_states / state_chunk (a multiple of 32) and the conv
// front (conv_w, conv_b, conv_k, u_out).
constexpr int kLparStates = 4;     // states per lane (16/kLparStates wavefronts)
constexpr int kLparSegSteps = 16;
hipError_t launch_lpar(const FwdArgs& a, bool bf16, hipStream_t st);

// Fixed per-device scratch of the entry point that allocates nothing
// (noalloc.hip): its size in bytes, and its device address on the current
// device (looked up once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
hipError_t noalloc_scratch(void** ptr);

// affine_scan association-order constants and launcher
constexpr int kAffT = 8;      // items per lane
constexpr int kAffLanes = 64; // lanes per wave
constexpr int kAffW = 4;      // waves per block
constexpr int kAffChunk = kAffT * kAffLanes * kAffW;
hipError_t launch_affine_scan(const float* a, const float* b, float* oa, float* ob, int64_t rows, int64_t L,
                              hipStream_t st);

// Output projection out[b][t][m] = sum_k W[m][k] y[b][k][t] on the matrix
// cores (bfloat16 or float32 storage, float32 accumulation).
struct ProjArgs {
  const void* y;     // [batch][d_inner][L]
  const void* w;     // [d_model][d_inner]
  void* out;         // [batch][L][d_model]
  int64_t batch, d_inner, d_model, L;
};
hipError_t launch_out_proj(const ProjArgs& a, bool bf16, hipStream_t st);
// workgroups of one launch
int64_t proj_tiles(bool bf16, int64_t batch, int64_t d_model, int64_t L);

// Gradients of the output projection for dout [batch][L][d_model]:
// dy[b][k][t] = sum_m W[m][k] dout[b][t][m], dW[m][k] = sum_{b,t}
// dout[b][t][m] y[b][k][t].  dy or dw may be null (not computed).  dW may
// split its sum over the batch rows into float32 partials in `work`
// (proj_bwd_workspace_bytes; the split is skipped when work is null).
struct ProjBwdArgs {
  const void* y;      // [batch][d_inner][L]
  const void* w;      // [d_model][d_inner]
  const void* dout;   // [batch][L][d_model]
  void* dy;           // [batch][d_inner][L], nullable
  void* dw;           // [d_model][d_inner], nullable
  int64_t batch, d_inner, d_model, L;
};
size_t proj_bwd_workspace_bytes(bool bf16, const ProjBwdArgs& a);
int64_t proj_bwd_tiles(bool bf16, const ProjBwdArgs& a);
hipError_t launch_out_proj_bwd(const ProjBwdArgs& a, bool bf16, float* work, size_t work_bytes, hipStream_t st);

}  // namespace ssm

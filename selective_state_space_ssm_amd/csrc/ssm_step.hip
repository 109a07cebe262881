// One recurrent step of the selective scan for every (batch, channel) on
// gfx950: the decode-time form of the recurrence ([Mamba-2 page]
// "Mamba (part 2): parallel scan and hardware-aware optimisation", §7 on
// constant-time recurrent inference; [Scan page] "Hardware-aware parallel
// associative scan for Mamba", §1.2 for the step itself):
//     Delta = softplus(delta + bias) (or delta + bias)
//     h_n   = exp(Delta * A[d,n]) * h_n + Delta * B[b,n] * u
//     y     = sum_n C[b,n] * h_n + D[d] * u,   y *= silu(z)
//
// Layout and mapping: the state is [b][d][n] float32.  Each channel owns four
// consecutive lanes (a DPP quad); lane q of the quad carries states
// [4q, 4q+4) as one float4, so a wave covers 16 channels and every state
// load and store is a coalesced 16-byte access.  The four partial sums of
// C . h meet by two DPP quad permutations; lane 0 of the quad stores y.
// The step is bound by the state's HBM traffic (read and write 8*n bytes
// per channel); Delta and the gate are recomputed by the four lanes of a
// quad, which costs nothing next to that.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct F32S {
  using T = float;
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};

struct BF16S {
  using T = uint16_t;
  static __device__ __forceinline__ float ld(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
  static __device__ __forceinline__ void st(uint16_t* p, float v) {
    *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // round to nearest even
  }
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

// quad_perm DPP controls: swap neighbours, swap pairs
constexpr int kQuadSwap1 = 0xB1;  // [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;  // [2, 3, 0, 1]

// every lane of a quad takes lane J's value
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), J | (J << 2) | (J << 4) | (J << 6), 0xf,
                                                    0xf, false));
}

// lane q of a quad takes lane q+1's value (lane 3 its own)
__device__ __forceinline__ float quad_shift_down(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 1 | (2 << 2) | (3 << 4) | (3 << 6), 0xf,
                                                    0xf, false));
}

__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap2, 0xf, 0xf, false));
  return v;
}

}  // namespace

// Grid: one thread per (channel, quad), 256 threads (64 channels) per block.
// VEC4: d_state is a multiple of 4 (float4 state and B/C accesses).
// CONV: u comes from the causal conv1d + SiLU over the window (conv state,
// x_t): the conv state [b][d][K-1] holds the K-1 previous inputs, oldest
// first; u = silu(conv_b + sum_k conv_w[k] window[k]) and the window shifted
// by one (x_t in, the oldest out) is written back.  The four lanes of a
// channel all read the state before lane 0 writes it (the stored values
// depend on the loaded ones), so the update may be in place.
template <typename IO>
struct StepDev {
  const typename IO::T* u;  // x with CONV
  const typename IO::T* dlt;
  const float* A;
  const typename IO::T* B;
  const typename IO::T* C;
  const float* D;
  const typename IO::T* z;
  const float* bias;
  const float* state_in;
  float* state_out;
  typename IO::T* y;
  const float* conv_w;
  const float* conv_b;
  const float* cs_in;
  float* cs_out;
  typename IO::T* u_out;
  int64_t batch, dim, N;
  int softplus, conv_k;
};

template <typename IO, bool VEC4, bool CONV>
__global__ __launch_bounds__(256) void ssm_step_kernel(StepDev<IO> a) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t dim = a.dim, N = a.N;
  const int64_t ch = gid >> 2;  // (b, d) flattened, d fastest
  const int q = static_cast<int>(gid & 3);
  const bool valid = ch < a.batch * dim;
  const int64_t chc = valid ? ch : 0;
  const int64_t b = chc / dim;
  const int64_t d = chc - b * dim;

  // Every load first: the state (the bulk of the traffic) and the step's
  // inputs are in flight together, and only then are the conv state and
  // the SSM state stored (the stores may overwrite what was loaded: the
  // update may be in place).
  const int64_t n0 = 4 * q;
  const bool has_states = valid && n0 < N;
  const int64_t so = ch * N + n0;
  float h[4], bv[4], cv[4], av[4];
  if (has_states) {
    if constexpr (VEC4) {
      // the state is read and written once per step: non-temporal
      const f32x4v hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(a.state_in + so));
      const float4 hs = make_float4(hv[0], hv[1], hv[2], hv[3]);
      const float4 as = *reinterpret_cast<const float4*>(a.A + d * N + n0);
      h[0] = hs.x; h[1] = hs.y; h[2] = hs.z; h[3] = hs.w;
      av[0] = as.x; av[1] = as.y; av[2] = as.z; av[3] = as.w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bv[e] = IO::ld(a.B + b * N + n0 + e);
        cv[e] = IO::ld(a.C + b * N + n0 + e);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = n0 + e < N;
        h[e] = ok ? a.state_in[so + e] : 0.0f;
        av[e] = ok ? a.A[d * N + n0 + e] : 0.0f;
        bv[e] = ok ? IO::ld(a.B + b * N + n0 + e) : 0.0f;
        cv[e] = ok ? IO::ld(a.C + b * N + n0 + e) : 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = av[e] = bv[e] = cv[e] = 0.0f;
  }
  const float x = IO::ld(a.dlt + chc) + (a.bias != nullptr ? a.bias[d] : 0.0f);
  const float Dd = a.D != nullptr ? a.D[d] : 0.0f;
  const float zz = a.z != nullptr ? IO::ld(a.z + chc) : 0.0f;

  float uu;
  if constexpr (CONV) {
    const int K = a.conv_k;
    // lane q of the quad holds conv state element q (q < K-1): the channel's
    // K-1 floats are read and written by neighbouring lanes, coalesced over
    // the wave; the four lanes see the whole window through DPP broadcasts.
    const float xt = IO::ld(a.u + chc);
    const bool own = valid && q < K - 1;
    const float sq = own ? a.cs_in[chc * (K - 1) + q] : 0.0f;
    float pre = a.conv_b != nullptr ? a.conv_b[d] : 0.0f;
    const float* w = a.conv_w + d * K;
    float wk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wk[j] = j < K ? w[j] : 0.0f;
    const float s0 = quad_bcast<0>(sq), s1 = quad_bcast<1>(sq), s2 = quad_bcast<2>(sq);
    // window oldest first: state[0 .. K-2], then x_t
    if (K >= 2) pre = __builtin_fmaf(wk[0], s0, pre);
    if (K >= 3) pre = __builtin_fmaf(wk[1], s1, pre);
    if (K >= 4) pre = __builtin_fmaf(wk[2], s2, pre);
    pre = __builtin_fmaf(wk[K - 1], xt, pre);
    uu = pre * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * pre));
    // the window moves by one: element q takes element q+1, the last x_t
    const float next = quad_shift_down(sq);
    if (own) a.cs_out[chc * (K - 1) + q] = (q < K - 2) ? next : xt;
    if (valid && q == 0 && a.u_out != nullptr) IO::st(a.u_out + chc, uu);
  } else {
    uu = IO::ld(a.u + chc);
  }
  // Delta in log2 units (dt2) and in natural units (dt): softplus(x) =
  // ln2 * softplus2(x log2 e), accurate as e^x -> 0
  const float x2 = x * kLog2e;
  const float dt2 = a.softplus ? dev::softplus2(x2) : x2;
  const float dt = a.softplus ? dt2 * dev::kLn2 : x;
  const float dtu = dt * uu;

  float part = 0.0f;
  if (has_states) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = __builtin_fmaf(__builtin_amdgcn_exp2f(dt2 * av[e]), h[e], dtu * bv[e]);
      part = __builtin_fmaf(cv[e], h[e], part);
    }
    if constexpr (VEC4) {
      const f32x4v hw = {h[0], h[1], h[2], h[3]};
      __builtin_nontemporal_store(hw, reinterpret_cast<f32x4v*>(a.state_out + so));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + e < N) a.state_out[so + e] = h[e];
    }
  }
  const float tot = quad_sum(part);
  if (valid && q == 0) {
    float yv = tot + Dd * uu;
    if (a.z != nullptr) yv *= zz * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * zz));
    IO::st(a.y + chc, yv);
  }
}

template <typename IO>
static hipError_t launch_step_t(const StepArgs& h, hipStream_t st) {
  using T = typename IO::T;
  StepDev<IO> a;
  a.u = static_cast<const T*>(h.u); a.dlt = static_cast<const T*>(h.delta); a.A = h.A;
  a.B = static_cast<const T*>(h.B); a.C = static_cast<const T*>(h.C); a.D = h.D;
  a.z = static_cast<const T*>(h.z); a.bias = h.bias; a.state_in = h.state_in; a.state_out = h.state_out;
  a.y = static_cast<T*>(h.y); a.conv_w = h.conv_w; a.conv_b = h.conv_b; a.cs_in = h.conv_state_in;
  a.cs_out = h.conv_state_out; a.u_out = static_cast<T*>(h.u_out);
  a.batch = h.batch; a.dim = h.dim; a.N = h.dstate; a.softplus = h.softplus; a.conv_k = h.conv_w ? h.conv_k : 0;
  const int64_t threads = h.batch * h.dim * 4;
  const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
  };
  const bool vec4 = h.dstate % 4 == 0;
  if (h.conv_w != nullptr) return vec4 ? run(ssm_step_kernel<IO, true, true>) : run(ssm_step_kernel<IO, false, true>);
  return vec4 ? run(ssm_step_kernel<IO, true, false>) : run(ssm_step_kernel<IO, false, false>);
}

hipError_t launch_step(const StepArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? launch_step_t<BF16S>(a, st) : launch_step_t<F32S>(a, st);
}

}  // namespace ssm

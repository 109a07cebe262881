// Selective-scan forward kernels for gfx950 (MI355X, CDNA4).
//
// Pages cited:
//   [Scan page]    "Hardware-aware parallel associative scan for Mamba"
//                  (http://www.pwwt.cn/news/6375169/)
//   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
//                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
//
// What runs where
// ---------------
// One workgroup owns 64 channels (one per lane) of one batch row and G
// wavefronts; wavefront g carries states [g*S, g*S+S) of every channel, so a
// lane holds S states of the recurrence h_n = a_n h_n + b_n in registers and
// never writes h or the pairs (a, b) to memory ([Scan page] §2.2, the
// channel-parallel, time-serial mapping, and §2.3 on fusing the
// discretisation into the scan; [Mamba-2 page] §3-§4).
//
// Time is processed in tiles of TT steps.  Per tile:
//   prep  (all waves): coalesced vector loads of u, delta (and z) along L,
//         Delta = softplus(delta + bias) kept in log2 units, Delta*u; both
//         go to LDS.  The loads of the next tile are issued before the
//         recurrence of this one, so HBM latency overlaps compute.
//   recur (wave g):   a = exp2(Delta2 * A[d,n]), b = (Delta*u) * B[n,t],
//         h = fma(a, h, b), partial y += C[n,t] * h over the wave's states.
//         B and C are the same for all 64 lanes: they are read with scalar
//         loads into SGPRs and used as the scalar operand of v_mul / v_fmac,
//         so the shared [b, n, L] rows cost neither VGPRs nor LDS bandwidth.
//   epi   (all waves): y = sum of the G partial sums + D*u, times silu(z),
//         rounded to the storage type, coalesced vector stores.
// Exp is v_exp_f32 (2^x): A is used unscaled because Delta is kept as
// Delta2 = Delta*log2(e); Delta*u is formed from Delta2*ln(2).
//
// Modes (template MODE):
//   kFull: start from zero or from a per-chunk start state, emit y over
//          [chunk*k, chunk*(k+1)), and last_state from the chunk that ends at L.
//   kAgg:  start from zero, emit only the chunk aggregate
//          (P_n = exp2(A_n * sum Delta2), H_n = h_n at the chunk end),
//          i.e. the chunk total (A^(k), B^(k)) of [Scan page] §2.2 / §3.3.
// The combine kernel then runs h_init^(k) = A^(k-1) h_init^(k-1) + B^(k-1)
// ([Scan page] §3.3 fix-up) over the K chunks of every (b, n, d).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_kernels.h"

namespace ssm {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTT = 32;          // steps per tile
constexpr int kCH = 64;          // channels per workgroup (= lanes)
constexpr int kRow = kTT + 4;    // LDS row stride in floats (conflict-free b128)
constexpr int kQ4 = kTT / 4;     // 4-step groups per tile row
constexpr int kSlots = kCH * kQ4;

// ---------------------------------------------------------------- storage
struct F32 {
  using T = float;
  static __device__ __forceinline__ float4 ld4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  static __device__ __forceinline__ float ld1(const float* p) { return *p; }
  static __device__ __forceinline__ void st4(float* p, float4 v) {
    *reinterpret_cast<float4*>(p) = v;
  }
  static __device__ __forceinline__ void st1(float* p, float v) { *p = v; }
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct BF16 {
  using T = uint16_t;
  static __device__ __forceinline__ float4 ld4(const uint16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y));
  }
  static __device__ __forceinline__ float ld1(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
  static __device__ __forceinline__ uint16_t cvt(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));  // v_cvt_pk_bf16_f32, RNE
  }
  static __device__ __forceinline__ void st4(uint16_t* p, float4 v) {
    uint2 w;
    w.x = static_cast<uint32_t>(cvt(v.x)) | (static_cast<uint32_t>(cvt(v.y)) << 16);
    w.y = static_cast<uint32_t>(cvt(v.z)) | (static_cast<uint32_t>(cvt(v.w)) << 16);
    *reinterpret_cast<uint2*>(p) = w;
  }
  static __device__ __forceinline__ void st1(uint16_t* p, float v) { *p = cvt(v); }
};

__device__ __forceinline__ float get(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}
__device__ __forceinline__ void set(float4& v, int j, float x) {
  if (j == 0) v.x = x; else if (j == 1) v.y = x; else if (j == 2) v.z = x; else v.w = x;
}

// Delta in log2 units from raw delta: x2 = (delta + bias) * log2(e);
// softplus(x) * log2(e) = log2(1 + 2^x2) ([Scan page] §1.2 softplus), taken
// as x2 itself above 64 where 2^-x2 is below float32 resolution.  The
// compare-and-select form keeps NaN inputs NaN and maps -inf to exactly 0.
__device__ __forceinline__ float delta2(float dl, float bias2, bool softplus) {
  const float x2 = __builtin_fmaf(dl, kLog2e, bias2);
  if (!softplus) return x2;
  const float sp = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(x2));
  return x2 > 64.0f ? x2 : sp;
}

// silu(z) = z / (1 + e^-z) ([Mamba-2 page] §4.1 SiLU gate).
__device__ __forceinline__ float silu(float zz) {
  return zz * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * zz));
}

}  // namespace

// --------------------------------------------------------------------------
// Broadcast of one step's B or C value: B and C for 16 consecutive steps sit
// in one VGPR, lane j of every row of 16 lanes holding step j.  DPP
// row_newbcast:j (gfx90a and later) hands lane j's value to its whole row as
// the src0 operand of the consuming v_mul / v_fmac, at no extra instruction.
// --------------------------------------------------------------------------
// x * bcast16<J>(c) and acc += bcast16<J>(c) * h as single v_mul_f32_dpp /
// v_fmac_f32_dpp instructions, written out so that every mode gets the fused
// form (the compiler folds a separate broadcast into v_mul only when both sit
// in one basic block, and never into v_fmac).  Hazard: a DPP source must not
// have been written by a VALU instruction in the two preceding instructions;
// c is only ever written by memory loads, which tests/test_isa_hazards.py
// checks on the generated ISA.
template <int J>
__device__ __forceinline__ float mul_bcast16(float c, float x) {
  float r;
  asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=v"(r)
      : "v"(c), "v"(x), "n"(J));
  return r;
}

template <int J>
__device__ __forceinline__ void fmac_bcast16(float& acc, float c, float h) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "+v"(acc)
      : "v"(c), "v"(h), "n"(J));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// --------------------------------------------------------------------------
// Channel-serial kernel.  Template: storage IO, states per wave S, waves G,
// mode, and GATED (z present).  Grid: x = channel block (64 channels),
// y = batch row, z = chunk.  Every pointer is a separate __restrict__
// parameter: the caller guarantees that outputs overlap no input.
//
// Two code paths share the registers and LDS layout:
//  * fast: a full block of 64 channels, whole tiles, L % 4 == 0.  The loop
//    body is straight-line (next-tile prefetches use clamped addresses
//    instead of branches), so the compiler can count outstanding memory
//    operations exactly and wait only for the ones each step consumes.
//  * generic: any tail tile, a partial channel block or unaligned L; loads
//    and stores element by element with bounds checks, no prefetch.
// --------------------------------------------------------------------------
template <typename IO, int S, int G, int MODE, bool GATED>
__global__ __launch_bounds__(64 * G) void ssm_cs_kernel(
    const typename IO::T* __restrict__ u, const typename IO::T* __restrict__ dlt,
    const float* __restrict__ Ag, const typename IO::T* __restrict__ Bg, const typename IO::T* __restrict__ Cg,
    const float* __restrict__ Dg, const typename IO::T* __restrict__ zg, const float* __restrict__ biasg,
    typename IO::T* __restrict__ yg, float* __restrict__ last_state, const float* __restrict__ h_init,
    float* __restrict__ agg_p, float* __restrict__ agg_h, CsSizes p) {
  using T = typename IO::T;
  constexpr int kThreads = 64 * G;
  constexpr int kSPT = (kSlots + kThreads - 1) / kThreads;  // prep/epilogue slots per thread
  constexpr bool kEvenSlots = (kSlots % kThreads) == 0;
  constexpr int kH = kTT / 16;                               // 16-step halves per tile
  constexpr bool kGate = GATED && MODE == kFull;
  constexpr int kNS = S * G;                                 // state rows staged per tile
  constexpr int kBCq = 2 * kNS * kQ4;                        // 4-step B/C groups per tile
  constexpr int kBCPT = (kBCq + kThreads - 1) / kThreads;    // ... per thread

  extern __shared__ float smem[];
  float* sDt = smem;                 // [64][kRow]  Delta2
  float* sDu = sDt + kCH * kRow;     // [64][kRow]  Delta * u
  float* sBC = sDu + kCH * kRow;     // [2][kNS][kTT] B and C of the tile, float32 (fast path)
  float* sY = sBC + 2 * kNS * kTT;   // [G][64][kRow] partial y (kFull only)

  const int tid = threadIdx.x;
  // the wave index as an SGPR keeps every per-wave quantity uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t dim = p.dim, L = p.L, N = p.dstate;
  const int64_t d0 = static_cast<int64_t>(blockIdx.x) * kCH;
  const int64_t b = blockIdx.y;
  const int64_t k = blockIdx.z;
  const int64_t t_begin = k * p.chunk;
  const int64_t t_end = (t_begin + p.chunk < L) ? t_begin + p.chunk : L;
  const bool softplus = p.softplus != 0;

  // ---- recurrence registers: S states of channel d0 + lane
  const int64_t d = d0 + lane;
  const bool dvalid = d < dim;
  float h[S], An[S];
  const T* Brow[S];
  const T* Crow[S];
  bool svalid[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = static_cast<int64_t>(wave) * S + s;
    svalid[s] = n < N;                                   // uniform per wave
    const int64_t nn = svalid[s] ? n : 0;
    An[s] = (svalid[s] && dvalid) ? Ag[d * N + nn] : 0.0f;
    h[s] = 0.0f;
    if (MODE == kFull && h_init != nullptr && svalid[s] && dvalid)
      h[s] = h_init[((k * p.batch + b) * N + nn) * dim + d];
    Brow[s] = Bg + (b * N + nn) * L;
    Crow[s] = Cg + (b * N + nn) * L;
  }
  float dsum = 0.0f;  // kAgg: sum of Delta2 over the chunk

  // ---- prep/epilogue slots of this thread: (row, 4-step group)
  float bias2[kSPT], Dd[kSPT];
#pragma unroll
  for (int j = 0; j < kSPT; ++j) {
    const int q = tid + j * kThreads;
    const int64_t dd = d0 + q / kQ4;
    const bool ok = q < kSlots && dd < dim;
    bias2[j] = (ok && biasg) ? biasg[dd] * kLog2e : 0.0f;
    Dd[j] = (ok && Dg) ? Dg[dd] : 0.0f;
  }

  const float* rowDt = sDt + lane * kRow;
  const float* rowDu = sDu + lane * kRow;
  float* rowY = sY + (wave * kCH + lane) * kRow;

  // Reduce the G partial sums of one slot, add D*u, gate, store (fast path).
  auto epilogue_slot = [&](int j, int64_t t0, float4 uu, float4 zz, bool vec) {
    const int q = tid + j * kThreads;
    const int r = q / kQ4;
    const int c4 = (q % kQ4) * 4;
    float4 acc = *reinterpret_cast<const float4*>(sY + r * kRow + c4);
#pragma unroll
    for (int g = 1; g < G; ++g) {
      const float4 v = *reinterpret_cast<const float4*>(sY + (g * kCH + r) * kRow + c4);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float yv = __builtin_fmaf(Dd[j], get(uu, e), get(acc, e));
      if (kGate) yv = yv * silu(get(zz, e));
      set(out, e, yv);
    }
    const int64_t dd = d0 + r;
    const int64_t t = t0 + c4;
    const int64_t off = (b * dim + dd) * L + t;
    if (vec) {
      IO::st4(yg + off, out);
    } else if (dd < dim) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t + e < t_end) IO::st1(yg + off + e, get(out, e));
    }
  };

  // ======================== fast path ========================
  const bool fast = (L % 4 == 0) && (d0 + kCH <= dim) && kEvenSlots;
  const int64_t n_fast = fast ? (t_end - t_begin) / kTT : 0;
  const int64_t t_fast_end = t_begin + n_fast * kTT;
  if (n_fast > 0) {
    // raw inputs of the next tile, prefetched one tile ahead
    float4 ru[kSPT], rd[kSPT], rz[kSPT], rbc[kBCPT];
    auto fetch = [&](int64_t t0) {
#pragma unroll
      for (int j = 0; j < kSPT; ++j) {
        const int q = tid + j * kThreads;
        const int64_t off = (b * dim + d0 + q / kQ4) * L + t0 + (q % kQ4) * 4;
        ru[j] = IO::ld4(u + off);
        rd[j] = IO::ld4(dlt + off);
        if (kGate) rz[j] = IO::ld4(zg + off);
      }
      // B then C rows of every staged state; rows past d_state read row 0
      // and are zeroed when written to LDS.  Every thread issues its loads
      // (surplus threads re-read a valid group) so that the number of memory
      // operations in flight is the same on every path.
#pragma unroll
      for (int j = 0; j < kBCPT; ++j) {
        const int q = (tid + j * kThreads) % kBCq;
        const int row = q / kQ4;                    // 0..2*kNS-1
        const int n = row % kNS;
        const T* base = (row < kNS) ? Bg : Cg;
        const int64_t nn = (n < N) ? n : 0;
        rbc[j] = IO::ld4(base + (b * N + nn) * L + t0 + (q % kQ4) * 4);
      }
    };

    float4 pu[kSPT], pz[kSPT];  // u, z of the tile whose epilogue is pending

    // ---- prep: Delta2, Delta*u, B, C of the tile in registers into LDS
    auto prep = [&]() {
#pragma unroll
      for (int j = 0; j < kSPT; ++j) {
        const int q = tid + j * kThreads;
        const int r = q / kQ4;
        const int c4 = (q % kQ4) * 4;
        float4 dt, du;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v2 = delta2(get(rd[j], e), bias2[j], softplus);
          set(dt, e, v2);
          set(du, e, (v2 * kLn2) * get(ru[j], e));
        }
        *reinterpret_cast<float4*>(sDt + r * kRow + c4) = dt;
        *reinterpret_cast<float4*>(sDu + r * kRow + c4) = du;
        pu[j] = ru[j];
        pz[j] = rz[j];
      }
#pragma unroll
      for (int j = 0; j < kBCPT; ++j) {
        const int q = tid + j * kThreads;
        if (kBCq % kThreads != 0 && q >= kBCq) continue;
        const int row = q / kQ4;
        const bool ok = (row % kNS) < N && (MODE == kFull || row < kNS);
        *reinterpret_cast<float4*>(sBC + row * kTT + (q % kQ4) * 4) =
            ok ? rbc[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };

    // ---- recurrence of one tile from LDS
    auto recur = [&]() {
      float4 dq[kQ4], uq[kQ4];
      float bc[S][kH], cc[S][kH];  // lane l: step 16*half + (l & 15) of state wave*S+s
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int hh = 0; hh < kH; ++hh) {
          const int n = wave * S + s;
          bc[s][hh] = sBC[n * kTT + 16 * hh + (lane & 15)];
          cc[s][hh] = (MODE == kFull) ? sBC[(kNS + n) * kTT + 16 * hh + (lane & 15)] : 0.0f;
        }
#pragma unroll
      for (int g4 = 0; g4 < kQ4; ++g4) {
        dq[g4] = *reinterpret_cast<const float4*>(rowDt + g4 * 4);
        uq[g4] = *reinterpret_cast<const float4*>(rowDu + g4 * 4);
      }
      static_for<0, kH>([&](auto HH) {
        constexpr int hh = decltype(HH)::value;
        float4 y4;
        static_for<0, 16>([&](auto JJ) {
          constexpr int j = decltype(JJ)::value;
          constexpr int st = hh * 16 + j;
          const float dt = get(dq[st / 4], st % 4);
          const float du = get(uq[st / 4], st % 4);
          float yv = 0.0f;
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const float a = __builtin_amdgcn_exp2f(dt * An[s]);
            h[s] = __builtin_fmaf(a, h[s], mul_bcast16<j>(bc[s][hh], du));
            if (MODE == kFull) {
              if (s == 0)
                yv = mul_bcast16<j>(cc[s][hh], h[s]);
              else
                fmac_bcast16<j>(yv, cc[s][hh], h[s]);
            }
          }
          if (MODE == kAgg) dsum += dt;
          set(y4, j % 4, yv);
          if (MODE == kFull && j % 4 == 3) *reinterpret_cast<float4*>(rowY + st - 3) = y4;
        });
      });
    };

    auto epilogue = [&](int64_t t0) {
      if (MODE == kFull) {
#pragma unroll
        for (int j = 0; j < kSPT; ++j) epilogue_slot(j, t0, pu[j], pz[j], true);
      }
    };

    // Tile 0 is peeled and every later iteration starts with the previous
    // tile's epilogue: the loop is entered from both sides with the same
    // memory operations outstanding (the prefetched loads are the newest),
    // so waits are counted exactly and never include the y stores.
    fetch(t_begin);
    prep();
    fetch(n_fast > 1 ? t_begin + kTT : t_begin);
    __syncthreads();
    recur();
    __syncthreads();
    for (int64_t it = 1; it < n_fast; ++it) {
      const int64_t t0 = t_begin + it * kTT;
      const int64_t tn = (it + 1 < n_fast) ? t0 + kTT : t0;
      epilogue(t0 - kTT);
      prep();
      fetch(tn);
      __syncthreads();
      recur();
      __syncthreads();
    }
    epilogue(t_fast_end - kTT);
  }

  // ======================== generic path ========================
  for (int64_t t0 = t_fast_end; t0 < t_end; t0 += kTT) {
    const int nsteps = static_cast<int>((t_end - t0 < kTT) ? (t_end - t0) : kTT);
    float4 pu[kSPT], pz[kSPT];
#pragma unroll
    for (int j = 0; j < kSPT; ++j) {
      const int q = tid + j * kThreads;
      pu[j] = pz[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q >= kSlots) continue;
      const int r = q / kQ4;
      const int c4 = (q % kQ4) * 4;
      const int64_t dd = d0 + r;
      const int64_t t = t0 + c4;
      float4 dt = make_float4(0.f, 0.f, 0.f, 0.f), du = dt;
      if (dd < dim) {
        const int64_t off = (b * dim + dd) * L + t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (t + e < t_end) {
            const float uu = IO::ld1(u + off + e);
            const float v2 = delta2(IO::ld1(dlt + off + e), bias2[j], softplus);
            set(dt, e, v2);
            set(du, e, (v2 * kLn2) * uu);
            set(pu[j], e, uu);
            if (kGate) set(pz[j], e, IO::ld1(zg + off + e));
          }
        }
      }
      *reinterpret_cast<float4*>(sDt + r * kRow + c4) = dt;
      *reinterpret_cast<float4*>(sDu + r * kRow + c4) = du;
    }
    __syncthreads();
    for (int e = 0; e < nsteps; ++e) {
      const float dt = rowDt[e], du = rowDu[e];
      float yv = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const float bv = svalid[s] ? IO::ld1(Brow[s] + t0 + e) : 0.0f;
        const float cv = (MODE == kFull && svalid[s]) ? IO::ld1(Crow[s] + t0 + e) : 0.0f;
        const float a = __builtin_amdgcn_exp2f(dt * An[s]);
        h[s] = __builtin_fmaf(a, h[s], du * bv);
        if (MODE == kFull) yv = (s == 0) ? cv * h[s] : __builtin_fmaf(cv, h[s], yv);
      }
      if (MODE == kAgg) dsum += dt;
      if (MODE == kFull) rowY[e] = yv;
    }
    __syncthreads();
    if (MODE == kFull) {
#pragma unroll
      for (int j = 0; j < kSPT; ++j) {
        const int q = tid + j * kThreads;
        if (q >= kSlots) continue;
        if (t0 + (q % kQ4) * 4 >= t_end) continue;
        epilogue_slot(j, t0, pu[j], pz[j], false);
      }
    }
    __syncthreads();
  }

  // ---- chunk end: final state or chunk aggregate
  if (!dvalid) return;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (!svalid[s]) continue;
    const int64_t n = static_cast<int64_t>(wave) * S + s;
    if (MODE == kFull) {
      if (last_state != nullptr && t_end == L) last_state[(b * dim + d) * N + n] = h[s];
    } else {
      const int64_t o = ((k * p.batch + b) * N + n) * dim + d;
      agg_p[o] = __builtin_amdgcn_exp2f(dsum * An[s]);
      agg_h[o] = h[s];
    }
  }
}

// --------------------------------------------------------------------------
// Chunk combine: for every (b, n, d), run the carry over the K chunk totals,
//   h_init^(0) = 0,  h_init^(k) = P^(k-1) h_init^(k-1) + H^(k-1)
// ([Scan page] §3.3 fix-up), writing h_init for k = 0..K-1.  One thread per
// (b, n, d); d is contiguous, so every access is coalesced.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ssm_combine_kernel(const float* __restrict__ agg_p,
                                                          const float* __restrict__ agg_h,
                                                          float* __restrict__ h_init, int64_t rows,
                                                          int64_t K) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  float hv = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    h_init[k * rows + i] = hv;
    if (k + 1 < K) hv = __builtin_fmaf(agg_p[k * rows + i], hv, agg_h[k * rows + i]);
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
size_t cs_smem_bytes(int S, int G, int mode) {
  return sizeof(float) * (static_cast<size_t>(kCH) * kRow * (2 + (mode == kFull ? G : 0)) +
                          static_cast<size_t>(2) * S * G * kTT);
}

int cs_time_tile() { return kTT; }

template <typename IO, int S, int G, int MODE, bool GATED>
static hipError_t launch_cs_v(const FwdArgs& a, int64_t nchunks, hipStream_t st) {
  using T = typename IO::T;
  const dim3 grid(static_cast<unsigned>((a.dim + kCH - 1) / kCH), static_cast<unsigned>(a.batch),
                  static_cast<unsigned>(nchunks));
  const size_t smem = cs_smem_bytes(S, G, MODE);
  auto kern = ssm_cs_kernel<IO, S, G, MODE, GATED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  CsSizes sz;
  sz.batch = a.batch; sz.dim = a.dim; sz.dstate = a.dstate; sz.L = a.L; sz.chunk = a.chunk; sz.softplus = a.softplus;
  hipLaunchKernelGGL(kern, grid, dim3(64 * G), smem, st, static_cast<const T*>(a.u), static_cast<const T*>(a.delta),
                     a.A, static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.D, static_cast<const T*>(a.z),
                     a.bias, static_cast<T*>(a.y), a.last_state, a.h_init, a.agg_p, a.agg_h, sz);
  return hipGetLastError();
}

template <typename IO, int S, int G, int MODE>
static hipError_t launch_cs(const FwdArgs& a, int64_t nchunks, hipStream_t st) {
  if (MODE == kFull && a.z != nullptr) return launch_cs_v<IO, S, G, MODE, true>(a, nchunks, st);
  return launch_cs_v<IO, S, G, MODE, false>(a, nchunks, st);
}

template <typename IO, int MODE>
static hipError_t dispatch_sg(const FwdArgs& a, int S, int G, int64_t nchunks, hipStream_t st) {
#define SSM_CASE(SS, GG) \
  if (S == SS && G == GG) return launch_cs<IO, SS, GG, MODE>(a, nchunks, st);
  SSM_CASE(2, 1) SSM_CASE(2, 2) SSM_CASE(2, 4) SSM_CASE(2, 8)
  SSM_CASE(4, 1) SSM_CASE(4, 2) SSM_CASE(4, 4)
  SSM_CASE(8, 1) SSM_CASE(8, 2)
#undef SSM_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_cs_full(const FwdArgs& a, bool bf16, int S, int G, int64_t nchunks, hipStream_t st) {
  return bf16 ? dispatch_sg<BF16, kFull>(a, S, G, nchunks, st) : dispatch_sg<F32, kFull>(a, S, G, nchunks, st);
}

hipError_t launch_cs_agg(const FwdArgs& a, bool bf16, int S, int G, int64_t nchunks, hipStream_t st) {
  return bf16 ? dispatch_sg<BF16, kAgg>(a, S, G, nchunks, st) : dispatch_sg<F32, kAgg>(a, S, G, nchunks, st);
}

hipError_t launch_combine(const float* agg_p, const float* agg_h, float* h_init, int64_t rows, int64_t K,
                          hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>((rows + 255) / 256);
  hipLaunchKernelGGL(ssm_combine_kernel, dim3(blocks), dim3(256), 0, st, agg_p, agg_h, h_init, rows, K);
  return hipGetLastError();
}

}  // namespace ssm

// L-parallel selective-scan forward for gfx950 (MI355X, CDNA4): a single
// pass for problems with few channels and long sequences, where one
// time-serial chain per lane leaves most SIMDs idle.
//
// Pages cited:
//   [Scan page]    "Hardware-aware parallel associative scan for Mamba"
//                  (http://www.pwwt.cn/news/6375169/)
//   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
//                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
//
// What runs where
// ---------------
// A workgroup owns 4 channels of one batch row and all (up to 16) states of
// them, in 16/S wavefronts: wave w carries states S*w .. S*w+S-1, S per lane
// (S = 4 and KS = 16 as built: four wavefronts, 256-step tiles).  Lane
// (r, j) of a wave (row r = lane / 16, j = lane % 16) holds channel c0 + r
// over time segment j of the current tile: the tile of 16*KS steps is cut
// into 16 segments of KS steps, one per lane of the row.  Per tile:
//   prep  (every thread): with the conv in front, u = silu(causal conv1d
//         of x) from x and the 3 steps before each thread's slot (stored
//         when asked for); Delta2 = softplus(delta + bias) in log2 units and
//         Delta*u of the tile's 4 channels, and B and C of its 16 states,
//         into LDS (float32); D*u and silu(z) stay in registers for the
//         epilogue.  The global loads are issued right after: B and C of
//         the next tile (read by every workgroup of the batch row, mostly
//         L2 hits) and u, delta, z of the tile after it (two register sets,
//         the loop unrolled by two), so that the HBM reads have two tiles
//         to arrive.
//   fold  (every lane, thread-serial over its KS steps and four states):
//         a = exp2(Delta2 * A), b = (Delta*u) * B, kept in registers, and
//         the segment's pair (P, H): P = prod a = exp2(A * sum Delta2), H =
//         the state at the segment end when it starts from zero
//         ([Scan page] §2.1, the serial pass inside a block; §2.2, the
//         chunk aggregate).
//   scan  (per row of 16 lanes): inclusive scan of the 16 segment pairs
//         under (P2, H2) o (P1, H1) = (P2 P1, P2 H1 + H2) in four
//         Hillis-Steele levels (shifts 1, 2, 4, 8) with DPP row_shr as the
//         operand of v_fmac / v_mul ([Scan page] §3.2, the warp-level scan;
//         §2.1, Hillis-Steele).  Lanes whose source lies before the row
//         keep their value: the identity pair.
//   carry: the state entering segment j is P_{<j} h_in + H_{<j}, composed
//         from the inclusive pair of segment j-1 and the tile's carry-in
//         ([Scan page] §3.3, the cross-chunk fix-up, at tile level).
//   refold (every lane): h = fma(a, h, b) again from that state over the
//         kept pairs, with the partial output sum over the lane's states of
//         C[n,t] * h into LDS; the state after segment 15 is the next
//         tile's carry-in (DPP row_newbcast:15).
//   epi   (every thread): y = sum of the waves' partials + D*u, times
//         silu(z), rounded to the storage type and stored.
// Chunk states (the checkpoints of the chunked recompute, [Mamba-2 page]
// §4.3): every state_chunk boundary is a multiple of 32 steps, so it falls on
// the end of a segment, whose lane holds that state after its refold and
// stores it.  Which segments of a tile end on a boundary is one 16-bit mask,
// worked out by the scalar unit per tile.  The last entry, the state after
// step L - 1, is the final carry, stored with last_state.
// Two barriers per tile: prep | fold-scan-refold | epilogue + next prep.
// Steps past L get Delta2 = 0, Delta*u = 0 and B = C = 0 (the identity
// step, a = 1, b = 0); channels past d_inner and states past d_state read
// zero (A = 0, B = C = 0) and are never stored.
//
// Cost against the time-serial plans: the fold and refold together issue
// about 7 VALU slots per state-step (mul, exp at half rate, mul, fma; then
// fma, fma) plus 0.5 for the scan at KS = 16, against 6 for one time-serial
// pass; in exchange every problem gets batch*d_inner wavefronts whatever its
// length, and it replaces the two full recurrences (and two reads of the
// inputs) of the two-pass plan where the channels alone cannot fill the
// chip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {

using namespace dev;

namespace {

constexpr int kLpCh = 4;           // channels per workgroup (rows of a wave)
constexpr int kLpSeg = 16;         // time segments per tile (lanes of a row)

// One Hillis-Steele level over the rows of 16 lanes: lane j with j >= SH
// becomes (P_{j-SH}, H_{j-SH}) composed before its own (P_j, H_j):
// H_j += H_{j-SH} * P_j, then P_j *= P_{j-SH}.  Lanes j < SH have no
// source in their row and are not written (bound_ctrl off), which is the
// identity pair.  The s_nop covers the DPP read-after-VALU-write hazard
// (two wait states) for values written just before the block.
template <int SH>
__device__ __forceinline__ void scan_level(float& H, float& P) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %1 row_shr:%2 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %1, %1 row_shr:%2 row_mask:0xf bank_mask:0xf"
      : "+v"(H), "+v"(P)
      : "n"(SH));
}

// Lane j of every row of 16 gets x of lane j - 1; lane 0 keeps `old`.
__device__ __forceinline__ float row_shr1_or(float old, float x) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mov_b32_dpp %0, %1 row_shr:1 row_mask:0xf bank_mask:0xf"
      : "+v"(old)
      : "v"(x));
  return old;
}

// x of lane 15 of every row of 16, to the whole row.
__device__ __forceinline__ float row_last(float x) {
  float r;
  asm volatile(
      "s_nop 1\n\t"
      "v_mov_b32_dpp %0, %1 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "=v"(r)
      : "v"(x));
  return r;
}

__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// A buffer offset past every resource of the kernel (their sizes stay below
// 2^30 bytes): a store there is dropped by the range check.
constexpr uint32_t kDropOffset = 0xFFFFFF00u;

}  // namespace

template <typename IO>
struct LparArgs {
  const typename IO::T* u;
  const typename IO::T* dlt;
  const float* Ag;
  const typename IO::T* Bg;
  const typename IO::T* Cg;
  const float* Dg;      // nullable
  const typename IO::T* zg;  // nullable (GATED false)
  const float* biasg;   // nullable
  typename IO::T* yg;
  float* last_state;    // nullable
  const float* h0;      // nullable
  float* chunk_states;  // nullable: [b][nsc][d][n]
  const float* convw;   // CONV: [d][K] causal conv1d weights (u then points at x)
  const float* convb;   // CONV: [d] conv bias, nullable
  typename IO::T* uo;   // CONV: [b][d][L] silu(conv1d(x)) output, nullable
};

struct LparSizes {
  int64_t batch, dim, dstate, L;
  int64_t nsc;          // chunk_states entries per batch row (0: none)
  int sc;               // steps per entry, a multiple of 2*KS (0: none)
  int softplus;
  int convk;            // CONV: conv1d taps, 1..4
};

// Template: storage IO, S states per lane (2 or 4: 16/S wavefronts), KS steps
// per segment (tile = 16*KS steps), GATED (z present), VEC (L is a multiple
// of 8: vector loads and stores), CS (chunk states kept), CONV (u =
// silu(causal conv1d of x) computed in prep from x, [Mamba-2 page] §4.1).
template <typename IO, int S, int KS, bool GATED, bool VEC, bool CS, bool CONV>
__global__ __launch_bounds__(1024 / S, 2) void ssm_lpar_kernel(LparArgs<IO> args, LparSizes p) {
  using T = typename IO::T;
  using Buf = typename BufOf<IO>::type;
  constexpr uint32_t ES = sizeof(T);
  constexpr int W = 16 / S;                // wavefronts (state groups)
  constexpr int NT = 64 * W;               // threads
  constexpr int TT = kLpSeg * KS;          // steps per tile
  constexpr int SS = KS + 4;               // LDS floats per segment (staggers the segments' banks)
  constexpr int RS = kLpSeg * SS;          // LDS floats per channel or state row of a tile
  constexpr int V = kLpCh * TT / NT;       // prep / epilogue steps per thread
  constexpr int TPC = NT / kLpCh;          // prep / epilogue threads per channel
  constexpr int NBC = 2 * 16 * kLpSeg / NT;  // B/C (state, segment) slots per thread
  static_assert(S == 2 || S == 4, "S");
  static_assert(KS % 4 == 0 && V >= 1 && KS % V == 0 && NBC >= 1, "tiling");
  extern __shared__ float smem[];
  float* sDt = smem;                 // [kLpCh][RS]  Delta2
  float* sDu = sDt + kLpCh * RS;     // [kLpCh][RS]  Delta * u
  float* sB = sDu + kLpCh * RS;      // [16][RS]
  float* sC = sB + 16 * RS;          // [16][RS]
  float* sY = sC + 16 * RS;          // [W][kLpCh][RS] partial y per wave

  const T* __restrict__ u = args.u;
  const T* __restrict__ dlt = args.dlt;
  const T* __restrict__ zg = args.zg;
  T* __restrict__ yg = args.yg;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane >> 4;
  const int j = lane & 15;
  const int64_t dim = p.dim, L = p.L, N = p.dstate;
  const int Li = static_cast<int>(L);
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kLpCh;
  const int64_t b = blockIdx.y;
  const bool softplus = p.softplus != 0;
  // waves whose four states all lie past d_state have nothing to scan
  const int WA = static_cast<int>((N + S - 1) / S);

  // ---- scan registers: channel c0 + r, states 4*wave + s
  const int64_t d = c0 + r;
  const bool dvalid = d < dim;
  float An[S], carry[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = static_cast<int64_t>(wave) * S + s;
    const bool ok = dvalid && n < N;
    An[s] = ok ? args.Ag[d * N + n] : 0.0f;
    carry[s] = (ok && args.h0 != nullptr) ? args.h0[(b * dim + d) * N + n] : 0.0f;
  }

  // ---- prep / epilogue slot: channel pc, steps [pt, pt + V) of the tile
  const int pc = tid / TPC;
  const int pt = (tid % TPC) * V;
  const int pidx = pc * RS + (pt / KS) * SS + (pt % KS);
  const int64_t pd = c0 + pc;
  const bool pvalid = pd < dim;
  const float bias2 = (pvalid && args.biasg != nullptr) ? args.biasg[pd] * kLog2e : 0.0f;
  const float Dd = (pvalid && args.Dg != nullptr) ? args.Dg[pd] : 0.0f;
  // CONV: the K taps right-aligned in w4 (w4[3] multiplies x_t, w4[3-j]
  // multiplies x_{t-j}); x before step 0 is zero
  float w4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float cbias = 0.0f;
  if constexpr (CONV) {
    const int K = p.convk;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (pvalid && jj >= 4 - K) w4[jj] = args.convw[pd * K + (jj - (4 - K))];
    cbias = (pvalid && args.convb != nullptr) ? args.convb[pd] : 0.0f;
  }

  // Buffer resources over the workgroup's rows of u, delta, z, y and over
  // batch row b of B and C: channels past d_inner and states past d_state
  // lie past the resource's size, so they read zero and their stores drop.
  const int64_t rows_here = (dim - c0) < kLpCh ? (dim - c0) : kLpCh;
  const int64_t row0 = (b * dim + c0) * L;
  const uint32_t in_bytes = static_cast<uint32_t>(rows_here * L * ES);
  const Rsrc rU = make_rsrc(u + row0, in_bytes);
  const Rsrc rD = make_rsrc(dlt + row0, in_bytes);
  const Rsrc rZ = make_rsrc(GATED ? zg + row0 : u + row0, in_bytes);
  const Rsrc rY = make_rsrc(yg + row0, in_bytes);
  // CONV: silu(conv1d(x)) out, when asked for (else an empty resource: the
  // stores still issue, and drop)
  const bool uo_on = CONV && args.uo != nullptr;
  const Rsrc rUO = make_rsrc(uo_on ? args.uo + row0 : yg + row0, uo_on ? in_bytes : 0u);
  const uint32_t bc_bytes = static_cast<uint32_t>(N * L * ES);
  const Rsrc rB = make_rsrc(args.Bg + b * N * L, bc_bytes);
  const Rsrc rC = make_rsrc(args.Cg + b * N * L, bc_bytes);
  const uint32_t poff = static_cast<uint32_t>((pc * L + pt) * ES);
  // B/C slots q = tid + i*NT: B for q < 256, else C (the same for a whole
  // wave), state bn = (q % 256) / 16, segment bj = q % 16 (KS steps)
  uint32_t bcoff[NBC];
  int bidx[NBC], bj[NBC];
  bool bcis_c[NBC];
#pragma unroll
  for (int i = 0; i < NBC; ++i) {
    const int q = tid + i * NT;
    bcis_c[i] = __builtin_amdgcn_readfirstlane((wave * 64 + i * NT) / 256) != 0;
    const int bn = (q & 255) >> 4;
    bj[i] = q & 15;
    bcoff[i] = static_cast<uint32_t>((bn * L + bj[i] * KS) * ES);
    bidx[i] = bn * RS + bj[i] * SS;
  }

  constexpr int RW = VEC ? Buf::template kWords<V> : V;
  constexpr int KC = KS < 8 ? KS : 8;  // B/C elements per load (at most 8 bfloat16 in one b128)
  constexpr int BW = VEC ? (KS / KC) * Buf::template kWords<KC> : KS;
  constexpr int HW = CONV ? 3 : 1;  // CONV: x at the 3 steps before the slot
  // float32 rows of u, delta, z and y are read or written once, by this
  // workgroup alone: non-temporal (long -0.2% to -0.8%, interleaved, on two
  // machines); B and C, which every workgroup of the batch row reads, keep
  // the default policy
  constexpr int kNT = std::is_same<IO, F32>::value ? kCacheNT : 0;
  struct UDRegs {
    uint32_t wu[RW], wd[RW], wz[RW];
    uint32_t wh[HW];
  };
  struct BCRegs {
    uint32_t wbc[NBC][BW];
  };
  auto load_ud = [&](UDRegs& R, int t0) {
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if (!GATED) {
#pragma unroll
      for (int e = 0; e < RW; ++e) R.wz[e] = 0u;
    }
    if constexpr (CONV) {
      // x at steps pt-3 .. pt-1 (halo_offset: never below zero; prep
      // zeroes the steps before 0)
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) Buf::template ldw<1>(rU, halo_offset(poff + toff, (3 - jj) * ES), &R.wh[jj]);
    } else {
      R.wh[0] = 0u;
    }
    if constexpr (VEC) {
      Buf::template ldw<V, kNT>(rU, poff + toff, R.wu);
      Buf::template ldw<V, kNT>(rD, poff + toff, R.wd);
      if (GATED) Buf::template ldw<V, kNT>(rZ, poff + toff, R.wz);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Buf::template ldw<1>(rU, poff + toff + e * ES, &R.wu[e]);
        Buf::template ldw<1>(rD, poff + toff + e * ES, &R.wd[e]);
        if (GATED) Buf::template ldw<1>(rZ, poff + toff + e * ES, &R.wz[e]);
      }
    }
  };
  auto load_bc = [&](BCRegs& R, int t0) {
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if constexpr (VEC) {
#pragma unroll
      for (int q = 0; q < NBC; ++q)
#pragma unroll
        for (int i = 0; i < KS; i += KC)
          Buf::template ldw<KC>(bcis_c[q] ? rC : rB, bcoff[q] + toff + i * ES,
                                R.wbc[q] + (i / KC) * Buf::template kWords<KC>);
    } else {
#pragma unroll
      for (int q = 0; q < NBC; ++q)
#pragma unroll
        for (int e = 0; e < KS; ++e) Buf::template ldw<1>(bcis_c[q] ? rC : rB, bcoff[q] + toff + e * ES, &R.wbc[q][e]);
    }
  };

  float nDu[V], nG[V];
  auto prep = [&](UDRegs& R, BCRegs& RB, int t0) {
    // the loaded words are pinned so that no conversion moves ahead of here
#pragma unroll
    for (int e = 0; e < RW; ++e) asm volatile("" : "+v"(R.wu[e]), "+v"(R.wd[e]), "+v"(R.wz[e]));
#pragma unroll
    for (int jj = 0; jj < HW; ++jj) asm volatile("" : "+v"(R.wh[jj]));
#pragma unroll
    for (int q = 0; q < NBC; ++q)
#pragma unroll
      for (int e = 0; e < BW; ++e) asm volatile("" : "+v"(RB.wbc[q][e]));
    float ru[V], rd[V], rz[V], rbc[NBC][KS];
    if constexpr (VEC) {
      Buf::template unpack<V>(R.wu, ru);
      Buf::template unpack<V>(R.wd, rd);
      Buf::template unpack<V>(R.wz, rz);
#pragma unroll
      for (int q = 0; q < NBC; ++q) Buf::template unpack<KS>(RB.wbc[q], rbc[q]);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Buf::template unpack<1>(&R.wu[e], &ru[e]);
        Buf::template unpack<1>(&R.wd[e], &rd[e]);
        Buf::template unpack<1>(&R.wz[e], &rz[e]);
      }
#pragma unroll
      for (int q = 0; q < NBC; ++q)
#pragma unroll
        for (int e = 0; e < KS; ++e) Buf::template unpack<1>(&RB.wbc[q][e], &rbc[q][e]);
    }
    if constexpr (CONV) {
      // u_t = silu(bias + sum_j w4[j] x_{t-3+j}); the same stores on every
      // tile (steps past L to the dropping offset, as in the epilogue)
      float xs[V + 3];
#pragma unroll
      for (int jj = 0; jj < 3; ++jj) {
        float v;
        Buf::template unpack<1>(&R.wh[jj], &v);
        xs[jj] = t0 + pt - 3 + jj >= 0 ? v : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < V; ++e) xs[3 + e] = ru[e];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float pre = cbias;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pre = __builtin_fmaf(w4[jj], xs[e + jj], pre);
        ru[e] = silu(pre);
      }
      const uint32_t toff = static_cast<uint32_t>(t0) * ES;
      if constexpr (VEC) {
        Buf::template st<V>(rUO, t0 + pt < Li ? poff + toff : kDropOffset, ru);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e)
          Buf::template st<1>(rUO, t0 + pt + e < Li ? poff + toff + e * ES : kDropOffset, &ru[e]);
      }
    }
    // whole tiles take no per-element masks; softplus is one uniform branch
    float dt[V], du[V];
    auto delta_steps = [&](auto SP, bool whole) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const bool ok = whole || t0 + pt + e < Li;
        const float uu = ok ? ru[e] : 0.0f;
        const float v2 = delta2c<decltype(SP)::value>(rd[e], bias2);
        dt[e] = ok ? v2 : 0.0f;
        du[e] = (dt[e] * kLn2) * uu;
        nDu[e] = Dd * uu;
        nG[e] = GATED ? silu(rz[e]) : 1.0f;
      }
    };
    const bool whole = t0 + TT <= Li;
    if (whole) {
      if (softplus) delta_steps(std::true_type{}, true); else delta_steps(std::false_type{}, true);
    } else {
      if (softplus) delta_steps(std::true_type{}, false); else delta_steps(std::false_type{}, false);
#pragma unroll
      for (int q = 0; q < NBC; ++q)
#pragma unroll
        for (int e = 0; e < KS; ++e) rbc[q][e] = t0 + bj[q] * KS + e < Li ? rbc[q][e] : 0.0f;
    }
    F32::template st<V>(sDt + pidx, dt);
    F32::template st<V>(sDu + pidx, du);
#pragma unroll
    for (int q = 0; q < NBC; ++q) F32::template st<KS>((bcis_c[q] ? sC : sB) + bidx[q], rbc[q]);
  };

  auto epilogue = [&](int t0) {
    float yv[V];
#pragma unroll
    for (int e = 0; e < V; ++e) yv[e] = nDu[e];
    for (int w = 0; w < WA; ++w) {
      float part[V];
      F32::template ld<V>(sY + w * kLpCh * RS + pidx, part);
#pragma unroll
      for (int e = 0; e < V; ++e) yv[e] += part[e];
    }
#pragma unroll
    for (int e = 0; e < V; ++e) yv[e] *= nG[e];
    // The same stores on every tile (steps past L go to an offset past the
    // resource, where the store is dropped), so that the wait for the next
    // tile's loads can count the stores issued after them and need not wait
    // for the stores themselves.  With VEC, L is a multiple of 8 and a
    // thread's V steps lie all before or all past L.
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if constexpr (VEC) {
      Buf::template st<V, kNT>(rY, t0 + pt < Li ? poff + toff : kDropOffset, yv);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        Buf::template st<1>(rY, t0 + pt + e < Li ? poff + toff + e * ES : kDropOffset, &yv[e]);
    }
  };

  // ---- fold, scan and refold of one tile by wave `wave` (states 4*wave ..)
  const float* rowDt = sDt + r * RS + j * SS;
  const float* rowDu = sDu + r * RS + j * SS;
  const float* rowB = sB + wave * S * RS + j * SS;
  const float* rowC = sC + wave * S * RS + j * SS;
  float* rowY = sY + (wave * kLpCh + r) * RS + j * SS;
  const int sc = p.sc;
  // bmask: bit i set when segment i of the tile ends on a chunk boundary;
  // kb: the boundaries before the tile (t0 / sc)
  auto save_states = [&](const float* h, int t0, uint32_t bmask, int kb) {
    if constexpr (!CS) return;
    // the last entry (state after step L - 1) is the final carry, stored
    // after the loop with last_state
    const bool at = ((bmask >> j) & 1u) != 0 && t0 + (j + 1) * KS < Li && dvalid;
    if (!at) return;
    const int64_t k = kb + __builtin_popcount(bmask & ((2u << j) - 1u)) - 1;
    float* dst = args.chunk_states + ((b * p.nsc + k) * dim + d) * N + static_cast<int64_t>(wave) * S;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (static_cast<int64_t>(wave) * S + s < N) dst[s] = h[s];
  };
  auto scan_tile = [&](int t0, uint32_t bmask, int kb) {
    float a[KS][S], bb[KS][S], H[S], P[S];
    float dsum = 0.0f;
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) {
      const float4 dt4 = lds4(rowDt + 4 * q);
      const float4 du4 = lds4(rowDu + 4 * q);
      float4 B4[S];
#pragma unroll
      for (int s = 0; s < S; ++s) B4[s] = lds4(rowB + s * RS + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q + e;
        const float x = get(dt4, e);
        const float du = get(du4, e);
        dsum += x;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          a[i][s] = __builtin_amdgcn_exp2f(x * An[s]);
          bb[i][s] = du * get(B4[s], e);
          H[s] = i == 0 ? bb[i][s] : __builtin_fmaf(a[i][s], H[s], bb[i][s]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) P[s] = __builtin_amdgcn_exp2f(An[s] * dsum);
#pragma unroll
    for (int s = 0; s < S; ++s) scan_level<1>(H[s], P[s]);
#pragma unroll
    for (int s = 0; s < S; ++s) scan_level<2>(H[s], P[s]);
#pragma unroll
    for (int s = 0; s < S; ++s) scan_level<4>(H[s], P[s]);
#pragma unroll
    for (int s = 0; s < S; ++s) scan_level<8>(H[s], P[s]);
    float h[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float hend = __builtin_fmaf(P[s], carry[s], H[s]);
      h[s] = row_shr1_or(carry[s], hend);
    }
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) {
      float4 C4[S];
#pragma unroll
      for (int s = 0; s < S; ++s) C4[s] = lds4(rowC + s * RS + 4 * q);
      float yq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q + e;
        float y = 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          h[s] = __builtin_fmaf(a[i][s], h[s], bb[i][s]);
          y = s == 0 ? get(C4[s], e) * h[s] : __builtin_fmaf(get(C4[s], e), h[s], y);
        }
        yq[e] = y;
      }
      *reinterpret_cast<float4*>(rowY + 4 * q) = make_float4(yq[0], yq[1], yq[2], yq[3]);
    }
    save_states(h, t0, bmask, kb);
#pragma unroll
    for (int s = 0; s < S; ++s) carry[s] = row_last(h[s]);
  };

  // The loads are issued on every tile, the last ones included (reads past
  // L return words of the next row or zero past the resource, and prep never
  // uses them), so that no branch makes the wait for them conservative.
  // The first loads go out in the order of every later tile (u/delta/z of
  // tile 0, B/C of tile 0, then u/delta/z of tile 1: the scheduling barriers
  // keep the compiler from interleaving them), followed by as many stores
  // as one epilogue issues (dropped, past the resource): the wait at the top
  // of the loop then sees the same count of memory operations after each
  // set of loads on entry as on every later pair of tiles, so it waits for
  // the loads only.
  UDRegs U0, U1;
  BCRegs RB;
  load_ud(U0, 0);
  load_bc(RB, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_ud(U1, TT);
  __builtin_amdgcn_sched_barrier(0);
  {
    float zero[V];
#pragma unroll
    for (int e = 0; e < V; ++e) zero[e] = 0.0f;
    if constexpr (VEC) {
      Buf::template st<V>(rY, kDropOffset, zero);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) Buf::template st<1>(rY, kDropOffset, &zero[e]);
    }
  }
  int nxt = sc;  // steps from t0 to the next chunk boundary (1 .. sc)
  int kb = 0;
  // A tile that starts at or past L (the second of the last pair when the
  // tile count is odd) is all identity steps: its prep, loads and (dropped)
  // stores still run, so that every tile issues the same memory operations,
  // but its scan is skipped (the carry would come out unchanged).
  auto tile = [&](UDRegs& U, int t0) {
    prep(U, RB, t0);
    load_bc(RB, t0 + TT);
    load_ud(U, t0 + 2 * TT);
    uint32_t bmask = 0;
    const int kb_tile = kb;
    if constexpr (CS) {
      for (; nxt <= TT; nxt += sc, ++kb) bmask |= 1u << (nxt / KS - 1);
      nxt -= TT;
    }
    __syncthreads();
    if (wave < WA && t0 < Li) scan_tile(t0, bmask, kb_tile);
    __syncthreads();
    epilogue(t0);
  };
  for (int t0 = 0; t0 < Li; t0 += 2 * TT) {
    tile(U0, t0);
    tile(U1, t0 + TT);
  }

  if (wave < WA && j == 0 && dvalid) {
    // the last chunk-state entry is the final state, bit for bit last_state
    float* last_cs = CS ? args.chunk_states + ((b * p.nsc + p.nsc - 1) * dim + d) * N : nullptr;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t n = static_cast<int64_t>(wave) * S + s;
      if (n >= N) continue;
      if (args.last_state != nullptr) args.last_state[(b * dim + d) * N + n] = carry[s];
      if (last_cs != nullptr) last_cs[n] = carry[s];
    }
  }
}

template <typename IO, int S, int KS, bool GATED, bool VEC, bool CS, bool CONV>
static hipError_t launch_lpar_v(const FwdArgs& a, hipStream_t st) {
  using T = typename IO::T;
  constexpr int RS = kLpSeg * (KS + 4);
  const size_t smem = sizeof(float) * static_cast<size_t>(RS) * (2 * kLpCh + 2 * 16 + (16 / S) * kLpCh);
  LparArgs<IO> g;
  g.u = static_cast<const T*>(a.u); g.dlt = static_cast<const T*>(a.delta); g.Ag = a.A;
  g.Bg = static_cast<const T*>(a.B); g.Cg = static_cast<const T*>(a.C); g.Dg = a.D;
  g.zg = static_cast<const T*>(a.z); g.biasg = a.bias; g.yg = static_cast<T*>(a.y);
  g.last_state = a.last_state; g.h0 = a.h0; g.chunk_states = a.chunk_states;
  g.convw = a.conv_w; g.convb = a.conv_b; g.uo = static_cast<T*>(a.u_out);
  LparSizes sz;
  sz.batch = a.batch; sz.dim = a.dim; sz.dstate = a.dstate; sz.L = a.L; sz.softplus = a.softplus;
  sz.convk = CONV ? a.conv_k : 0;
  if (CONV && (a.conv_w == nullptr || a.conv_k < 1 || a.conv_k > 4)) return hipErrorInvalidValue;
  const bool cs = a.chunk_states != nullptr && a.state_chunk > 0;
  if (cs && a.state_chunk % (2 * KS) != 0) return hipErrorInvalidValue;
  // a spacing of L or more has no boundary before step L; any multiple of 32
  // past L then stands for it and fits an int
  sz.sc = cs ? static_cast<int>(a.state_chunk <= a.L ? a.state_chunk : (a.L / 32 + 1) * 32) : 0;
  sz.nsc = cs ? (a.L + a.state_chunk - 1) / a.state_chunk : 0;
  const dim3 grid(static_cast<unsigned>((a.dim + kLpCh - 1) / kLpCh), static_cast<unsigned>(a.batch));
  auto kern = ssm_lpar_kernel<IO, S, KS, GATED, VEC, CS, CONV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(1024 / S), smem, st, g, sz);
  return hipGetLastError();
}

template <typename IO, bool CS, bool CONV>
static hipError_t dispatch_lpar(const FwdArgs& a, hipStream_t st) {
  constexpr int S = kLparStates, KS = kLparSegSteps;
  const bool vec = a.L % 8 == 0;
  if (a.z != nullptr)
    return vec ? launch_lpar_v<IO, S, KS, true, true, CS, CONV>(a, st)
               : launch_lpar_v<IO, S, KS, true, false, CS, CONV>(a, st);
  return vec ? launch_lpar_v<IO, S, KS, false, true, CS, CONV>(a, st)
             : launch_lpar_v<IO, S, KS, false, false, CS, CONV>(a, st);
}

template <typename IO>
static hipError_t dispatch_lpar(const FwdArgs& a, hipStream_t st) {
  // the chunk-state stores (and their per-tile mask) and the conv front are
  // compiled in only where they are asked for
  const bool cs = a.chunk_states != nullptr && a.state_chunk > 0;
  if (a.conv_w != nullptr) return cs ? dispatch_lpar<IO, true, true>(a, st) : dispatch_lpar<IO, false, true>(a, st);
  return cs ? dispatch_lpar<IO, true, false>(a, st) : dispatch_lpar<IO, false, false>(a, st);
}

hipError_t launch_lpar(const FwdArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? dispatch_lpar<BF16>(a, st) : dispatch_lpar<F32>(a, st);
}

}  // namespace ssm

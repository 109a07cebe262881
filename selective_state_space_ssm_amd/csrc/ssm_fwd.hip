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
// A workgroup owns 16 channels of one batch row and all (up to 16) states of
// them.  Its W = 4/S wavefronts are split into rows of 16 lanes: lane `col`
// of a row is channel c0 + col, and row `row` of wave `w` carries the S
// states n = (4w + row)*S + s of that channel.  The recurrence
// h_n = a_n h_n + b_n therefore runs time-serially in registers, one
// (channel, state) chain per lane slot, and neither h nor the pairs (a, b)
// are written to memory ([Scan page] §2.2, the channel-parallel,
// time-serial mapping, and §2.3 on fusing the discretisation into the scan;
// [Mamba-2 page] §3-§4).  Sixteen channels per workgroup (not 64) give
// batch*d_inner/16 workgroups, enough for every CU of the chip at the
// 130m-like shape (768 workgroups, three per CU, three waves per SIMD with
// one state per lane), and S trades lanes for registers where channels are
// plentiful.
//
// Time is processed in tiles of kTT steps, with two barriers per tile:
//   recur (every lane): a = exp2(Delta2 * A[d,n]), b = (Delta*u) * B[n,t],
//         h = fma(a, h, b), partial y = sum over the lane's S states of
//         C[n,t] * h, written to LDS per (row group, channel, step).
//         B and C of step t for the row's state sit in one VGPR (lane j of
//         the row holds step j of a 16-step half tile) and reach the whole
//         row through DPP row_newbcast as an operand of v_mul / v_fmac.
//   epi   (every thread, V steps of one channel): y = sum of the 4W partial
//         sums + D*u, times silu(z); rounded to the storage type, stored.
//   prep  (every thread, V steps of one channel, next tile): Delta2 =
//         softplus(delta + bias) in log2 units and Delta*u into LDS; B and C
//         of the tile (float32) into LDS.  The global loads run two tiles
//         ahead in two register sets (bfloat16 one-wave groups: four sets,
//         a 128-byte line's two halves loaded together), issued after the
//         epilogue.  One-wave groups also vote on whether the tile is an
//         identity tile (all Delta2 and Delta*u zero, B finite), whose
//         recurrence then reduces to the partial sums.
// Exp is v_exp_f32 (2^x): A is used unscaled because Delta is kept as
// Delta2 = Delta*log2(e); Delta*u is formed from Delta2*ln(2).
//
// Steps past the end of the chunk (ragged last tile) and channels or states
// past the problem size get Delta2 = 0, Delta*u = 0 and B = C = 0: the
// identity step (a = 1, b = 0) of [Scan page] §2.1, so the registers need
// no masking and only the stores are guarded.
//
// Modes (template MODE):
//   kFull: start from zero, from the caller's h0 or from a per-chunk start
//          state, emit y over [chunk*k, chunk*(k+1)), last_state from the
//          chunk that ends at L, and optionally the state after every tile
//          that ends a state chunk (the checkpoints of the Mamba-2 page's
//          §4.3 chunked recomputation).
//   kAgg:  start from zero, emit only the chunk aggregate
//          (P_n = exp2(A_n * sum Delta2), H_n = h_n at the chunk end),
//          i.e. the chunk total (A^(k), B^(k)) of [Scan page] §2.2 / §3.3.
// The combine kernel then runs h_init^(k) = A^(k-1) h_init^(k-1) + B^(k-1)
// ([Scan page] §3.3 fix-up) over the K chunks of every (b, n, d).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {

using namespace dev;

namespace {

constexpr int kTT = 32;          // steps per tile
constexpr int kCG = 16;          // channels per workgroup (= lanes per row)
constexpr int kNS = 16;          // state slots per workgroup (d_state <= 16)
constexpr int kRow = kTT + 4;    // LDS row stride in floats (float4 rows, staggered banks)

}  // namespace

// --------------------------------------------------------------------------
// One 16-channel group of the row layout, run by 4/S wavefronts of the
// block (block-local thread `tid`, wave `wave`), over channels [c0, c0+16)
// of batch row b and chunk k, with its LDS at `smem`.  Template: storage
// IO, states per lane S (1, 2, 4), mode, GATED (z present), VEC (L is a
// multiple of 8: vector loads and stores), CONV (u = silu(causal conv1d of
// x) computed in prep from x and the conv weights, [Mamba-2 page] §4.1).  Every wave of the block calls
// __syncthreads() in the same sequence (all groups of a block have the same
// tile count).  Pointers: the caller guarantees that outputs overlap no
// input.
// --------------------------------------------------------------------------
template <typename IO>
struct RowArgs {
  const typename IO::T* u;
  const typename IO::T* dlt;
  const float* Ag;
  const typename IO::T* Bg;
  const typename IO::T* Cg;
  const float* Dg;
  const typename IO::T* zg;
  const float* biasg;
  typename IO::T* yg;
  float* last_state;
  const float* h_init;
  const float* h0;
  float* chunk_states;
  float* agg_p;
  float* agg_h;
  const float* convw;      // CONV: [d][K] causal conv1d weights (u then points at x)
  const float* convb;      // CONV: [d] conv bias, nullable
  typename IO::T* uo;      // CONV: [b][d][L] silu(conv1d(x)) output, nullable
};

template <typename IO, int S, int MODE, bool GATED, bool VEC, bool CONV>
__device__ __forceinline__ void rows_group(const RowArgs<IO>& args, const CsSizes& p, float* smem, int tid,
                                           int wave, int64_t c0, int64_t b, int64_t k) {
  using T = typename IO::T;
  const T* __restrict__ u = args.u;
  const T* __restrict__ dlt = args.dlt;
  const float* __restrict__ Ag = args.Ag;
  const T* __restrict__ Bg = args.Bg;
  const T* __restrict__ Cg = args.Cg;
  const float* __restrict__ Dg = args.Dg;
  const T* __restrict__ zg = args.zg;
  const float* __restrict__ biasg = args.biasg;
  T* __restrict__ yg = args.yg;
  float* __restrict__ last_state = args.last_state;
  const float* __restrict__ h_init = args.h_init;
  const float* __restrict__ h0 = args.h0;
  float* __restrict__ chunk_states = args.chunk_states;
  float* __restrict__ agg_p = args.agg_p;
  float* __restrict__ agg_h = args.agg_h;
  constexpr int W = 4 / S;                 // wavefronts
  constexpr int NT = 64 * W;               // threads
  constexpr int NG = 4 * W;                // partial-sum groups (rows of all waves)
  constexpr int V = kCG * kTT / NT;        // prep / epilogue steps per thread
  constexpr int TPC = kTT / V;             // prep / epilogue threads per channel
  constexpr int BCQ = 2 * kNS * kTT / 4 / NT;  // B/C float4 groups per thread
  constexpr bool kGate = GATED && MODE == kFull;
  static_assert(S == 1 || S == 2 || S == 4, "S");
  static_assert(V * NT == kCG * kTT && BCQ * NT * 4 == 2 * kNS * kTT, "tiling");

  float* sDt = smem;                  // [16][kRow]  Delta2
  float* sDu = sDt + kCG * kRow;      // [16][kRow]  Delta * u
  float* sBC = sDu + kCG * kRow;      // [2][16][kTT] B rows, then C rows (float32), swizzled (bc_col)
  float* sP = sBC + 2 * kNS * kTT;    // [NG][16][kRow] partial y (kFull only)

  const int lane = tid & 63;
  const int row = lane >> 4;
  const int col = lane & 15;
  const int64_t dim = p.dim, L = p.L, N = p.dstate;
  // time indices fit in 32 bits (the host rejects L >= 2^31)
  const int Li = static_cast<int>(L);
  const int t_begin = static_cast<int>(k * p.chunk);
  const int t_end = (p.chunk < Li - t_begin) ? t_begin + static_cast<int>(p.chunk) : Li;
  const bool softplus = p.softplus != 0;

  // ---- recurrence registers: S states of channel c0 + col
  const int grp = wave * 4 + row;
  const int64_t d = c0 + col;
  const bool dvalid = d < dim;
  float h[S], An[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = static_cast<int64_t>(grp) * S + s;
    const bool ok = dvalid && n < N;
    An[s] = ok ? Ag[d * N + n] : 0.0f;
    h[s] = 0.0f;
    // start state: the chunk start state of the two-pass plan (which already
    // includes h0), else h0 for the single-chunk plans; the aggregate pass
    // always starts from zero
    if (MODE == kFull && ok) {
      if (h_init != nullptr)
        h[s] = h_init[((k * p.batch + b) * N + n) * dim + d];
      else if (h0 != nullptr)
        h[s] = h0[(b * dim + d) * N + n];
    }
  }
  float dsum = 0.0f;  // kAgg: sum of Delta2 over the chunk

  // ---- prep / epilogue slot of this thread: channel pc, steps [pt, pt + V)
  using Buf = typename BufOf<IO>::type;
  constexpr uint32_t ES = sizeof(T);
  const int pc = tid / TPC;
  const int pt = (tid % TPC) * V;
  const int64_t pd = c0 + pc;
  const bool pvalid = pd < dim;
  const float bias2 = (pvalid && biasg != nullptr) ? biasg[pd] * kLog2e : 0.0f;
  const float Dd = (pvalid && Dg != nullptr) ? Dg[pd] : 0.0f;

  // Buffer resources over this workgroup's rows of u, delta, z, y (its
  // channels of batch row b) and over batch row b of B and C.  Channels
  // past d_inner and states past d_state lie past the resource's size: they
  // read as zero and their writes are dropped.  Byte offsets fit in 32 bits
  // (the host bounds 16 * L * element size).
  const int64_t rows_left = dim - c0;  // may be <= 0 for a padding group of a mixed block
  const int64_t rows_here = rows_left < 0 ? 0 : (rows_left < kCG ? rows_left : kCG);
  const int64_t row0 = (b * dim + (rows_here > 0 ? c0 : 0)) * L;
  const uint32_t in_bytes = static_cast<uint32_t>(rows_here * L * ES);
  const Rsrc rU = make_rsrc(u + row0, in_bytes);
  const Rsrc rD = make_rsrc(dlt + row0, in_bytes);
  const Rsrc rZ = make_rsrc(kGate ? zg + row0 : u + row0, in_bytes);
  const Rsrc rY = make_rsrc(MODE == kFull ? yg + row0 : u + row0, in_bytes);
  const uint32_t bc_bytes = static_cast<uint32_t>(N * L * ES);
  const Rsrc rB = make_rsrc(Bg + b * N * L, bc_bytes);
  const Rsrc rC = make_rsrc(Cg + b * N * L, bc_bytes);
  const uint32_t poff = static_cast<uint32_t>((pc * L + pt) * ES);

  // B/C slots of this thread: group q = tid + i*NT covers 4 steps of state n
  // of B (first 128 groups) or C; the tensor is the same for a whole wave.
  uint32_t bcoff[BCQ];
  bool bcis_c[BCQ];
#pragma unroll
  for (int i = 0; i < BCQ; ++i) {
    const int q = tid + i * NT;
    bcis_c[i] = __builtin_amdgcn_readfirstlane((wave * 64 + i * NT) / (kNS * kTT / 4)) != 0;
    const int n = (q / (kTT / 4)) % kNS;
    bcoff[i] = static_cast<uint32_t>((n * L + (q % (kTT / 4)) * 4) * ES);
  }

  // Raw inputs of one tile (32-bit words as loaded), a whole tile of
  // recurrence ahead of use.  The loads are straight-line code (reads past a
  // row run into the next row or past the resource, both harmless); prep
  // pins the words, converts them and zeroes whatever lies past the chunk,
  // so nothing touches a loaded register before prep.
  // words per tile row slice and per B/C group: packed (VEC) or one per element
  constexpr int RW = VEC ? Buf::template kWords<V> : V;
  constexpr int BW = VEC ? Buf::template kWords<4> : 4;
  constexpr int HW = CONV ? 3 : 0;  // conv halo: the 3 steps before the slot
  // float32 rows of u, delta, z and y are each read or written once and
  // belong to this group alone: non-temporal (130m -2%, interleaved).  The
  // bfloat16 kernels keep the default policy, which measured faster for
  // them (1.4B +1.2% with it), and B and C, which every group of the batch
  // row reads, always do.
  constexpr int kNT = std::is_same<IO, F32>::value ? kCacheNT : 0;
  struct TileRegs {
    uint32_t wu[RW], wd[RW], wz[RW];
    uint32_t wh[HW > 0 ? HW : 1];
    uint32_t wbc[BCQ][BW];
    int t0;  // first step of the tile the words hold
  };

  auto load_tile = [&](TileRegs& R, int t0) {
    uint32_t* wu = R.wu;
    uint32_t* wd = R.wd;
    uint32_t* wz = R.wz;
    auto& wbc = R.wbc;
    R.t0 = t0;
    if (!kGate) {
#pragma unroll
      for (int e = 0; e < RW; ++e) wz[e] = 0u;
    }
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if constexpr (CONV) {
      // x at steps pt-3 .. pt-1 of the tile (halo_offset: never below zero;
      // prep zeroes the steps before 0)
#pragma unroll
      for (int j = 0; j < HW; ++j) Buf::template ldw<1>(rU, halo_offset(poff + toff, (HW - j) * ES), &R.wh[j]);
    }
    if constexpr (VEC) {
      Buf::template ldw<V, kNT>(rU, poff + toff, wu);
      Buf::template ldw<V, kNT>(rD, poff + toff, wd);
      if (kGate) Buf::template ldw<V, kNT>(rZ, poff + toff, wz);
#pragma unroll
      for (int i = 0; i < BCQ; ++i) Buf::template ldw<4>(bcis_c[i] ? rC : rB, bcoff[i] + toff, wbc[i]);
    } else {
      // one element per load; the words then hold float32 bits (F32) or a
      // bfloat16 in their high half (BF16), as ldw<1> returns them
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Buf::template ldw<1>(rU, poff + toff + e * ES, &wu[e]);
        Buf::template ldw<1>(rD, poff + toff + e * ES, &wd[e]);
        if (kGate) Buf::template ldw<1>(rZ, poff + toff + e * ES, &wz[e]);
      }
#pragma unroll
      for (int i = 0; i < BCQ; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Buf::template ldw<1>(bcis_c[i] ? rC : rB, bcoff[i] + toff + e * ES, &wbc[i][e]);
    }
  };

  // Convert the pinned words of the tile to float32.
  float ru[V], rd[V], rz[V];
  float4 rbc[BCQ];
  auto unpack_tile = [&](TileRegs& R) {
    uint32_t* wu = R.wu;
    uint32_t* wd = R.wd;
    uint32_t* wz = R.wz;
    auto& wbc = R.wbc;
#pragma unroll
    for (int e = 0; e < RW; ++e) asm volatile("" : "+v"(wu[e]), "+v"(wd[e]), "+v"(wz[e]));
#pragma unroll
    for (int j = 0; j < HW; ++j) asm volatile("" : "+v"(R.wh[j]));
#pragma unroll
    for (int i = 0; i < BCQ; ++i)
#pragma unroll
      for (int e = 0; e < BW; ++e) asm volatile("" : "+v"(wbc[i][e]));
    if constexpr (VEC) {
      Buf::template unpack<V>(wu, ru);
      Buf::template unpack<V>(wd, rd);
      Buf::template unpack<V>(wz, rz);
#pragma unroll
      for (int i = 0; i < BCQ; ++i) {
        float v[4];
        Buf::template unpack<4>(wbc[i], v);
        rbc[i] = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Buf::template unpack<1>(&wu[e], &ru[e]);
        Buf::template unpack<1>(&wd[e], &rd[e]);
        Buf::template unpack<1>(&wz[e], &rz[e]);
      }
#pragma unroll
      for (int i = 0; i < BCQ; ++i) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Buf::template unpack<1>(&wbc[i][e], &v[e]);
        rbc[i] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  };

  // LDS position of B/C float4 group q (state n = (q / 8) % 16, steps
  // 4 (q % 8) .. + 3, B for q < 128 and C after): the two 16-step halves of
  // a state's row are swapped for states of odd lane rows (row group n / S
  // odd), so that the two rows of 16 lanes that a 32-lane half of a wave
  // reads in one LDS access land in different banks (32 banks of 4 bytes).
  auto bc_slot = [&](int q) {
    const int n = (q / (kTT / 4)) % kNS;
    const int t = (q % (kTT / 4)) * 4;
    return (q / (kTT / 4)) * kTT + (t ^ (16 * ((n / S) & 1)));
  };

  // D*u and silu(z) of the tile just prepared (n*) and of the tile whose
  // epilogue is pending (c*).  Prep computes them from the loaded registers,
  // so no loaded value is ever copied: a copy would let the compiler keep the
  // next tile's load in another register and wait for it at the loop's end.
  float nDu[V], nG[V];
  float cDu[V], cG[V];
  // Identity tiles (one-wave groups, full pass): a tile whose Delta2 and
  // Delta*u are all exactly zero and whose B is finite leaves every state
  // unchanged (a = exp2(0) = 1, b = 0 * B = 0), so its recurrence reduces to
  // the partial sums C.h.  Prep decides it for the tile it prepares (one OR
  // per step over the bits of Delta2 and Delta*u, a wave vote, and only when
  // that vote says zero the finiteness of B); the recurrence takes it from
  // cur_live.  Varlen padding (Delta = 0 past each length) makes such tiles.
  // A must be finite as well (checked once).
  constexpr bool kSkip = (W == 1) && MODE == kFull && !CONV;
  bool next_live = true, cur_live = true;
  // a non-finite A makes exp2(0 * A) NaN: such a group never skips
  bool a_finite = true;
  if constexpr (kSkip) {
    float za = 0.0f;
#pragma unroll
    for (int s = 0; s < S; ++s) za = __builtin_fmaf(An[s], 0.0f, za);
    a_finite = __builtin_amdgcn_ballot_w64((__float_as_uint(za) & 0x7fffffffu) != 0u) == 0u;
  }

  // ---- prep: Delta2, Delta*u, B, C of the tile held in registers into LDS.
  // In the ragged last tile, steps past the chunk become identity steps
  // (Delta2 = Delta*u = 0, B = C = 0).  Channels past d_inner read u = 0
  // (so Delta*u = 0) and their lanes have A = 0 (so a = 1): their state
  // stays zero without a mask.
  // Pin nDu / nG into VGPRs where prep computes them, so the compiler cannot
  // sink their products past the next load of the same registers.
  auto pin = [&]() {
#pragma unroll
    for (int e = 0; e < V; ++e) asm volatile("" : "+v"(nDu[e]), "+v"(nG[e]));
  };

  // ---- causal conv1d + SiLU in front of the scan (CONV): with K taps
  // right-aligned in w4 (w4[3] multiplies x_t, w4[3-j] multiplies x_{t-j}),
  // u_t = silu(bias + sum_j w4[j] x_{t-3+j}), x before step 0 being zero.
  // u replaces the loaded x in ru; with an output it is also stored.
  float w4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float cbias = 0.0f;
  if constexpr (CONV) {
    const int K = p.convk;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (pvalid && j >= 4 - K) w4[j] = args.convw[pd * K + (j - (4 - K))];
    cbias = (pvalid && args.convb != nullptr) ? args.convb[pd] : 0.0f;
  }
  const Rsrc rUO = make_rsrc(CONV && MODE == kFull && args.uo != nullptr ? args.uo + row0 : u + row0,
                             CONV && MODE == kFull && args.uo != nullptr ? in_bytes : 0u);
  auto conv_front = [&](TileRegs& R, int r_t0) {
    float xs[V + 3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      float v;
      Buf::template unpack<1>(&R.wh[j], &v);
      xs[j] = (r_t0 + pt - 3 + j >= 0) ? v : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) xs[3 + e] = ru[e];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float pre = cbias;
#pragma unroll
      for (int j = 0; j < 4; ++j) pre = __builtin_fmaf(w4[j], xs[e + j], pre);
      ru[e] = silu(pre);
    }
    const uint32_t toff = static_cast<uint32_t>(r_t0) * ES;
    if (VEC && r_t0 + kTT <= t_end) {
      Buf::template st<V>(rUO, poff + toff, ru);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (r_t0 + pt + e < t_end) Buf::template st<1>(rUO, poff + toff + e * ES, &ru[e]);
    }
  };
  auto prep = [&](TileRegs& R) {
    unpack_tile(R);
    const int r_t0 = R.t0;
    if constexpr (CONV) conv_front(R, r_t0);
    float dt[V], du[V];
    // softplus is one uniform branch around straight-line code per element
    auto delta_full = [&](auto SP) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float v2 = delta2c<decltype(SP)::value>(rd[e], bias2);
        dt[e] = v2;
        du[e] = (v2 * kLn2) * ru[e];
        nDu[e] = Dd * ru[e];
        nG[e] = kGate ? silu(rz[e]) : 1.0f;
      }
    };
    auto delta_part = [&](auto SP) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const bool ok = r_t0 + pt + e < t_end;
        const float uu = ok ? ru[e] : 0.0f;
        const float v2 = ok ? delta2c<decltype(SP)::value>(rd[e], bias2) : 0.0f;
        dt[e] = v2;
        du[e] = (v2 * kLn2) * uu;
        nDu[e] = Dd * uu;
        nG[e] = (kGate && ok) ? silu(rz[e]) : 1.0f;
      }
    };
    if (r_t0 + kTT <= t_end) {
      if (softplus) delta_full(std::true_type{}); else delta_full(std::false_type{});
      pin();
      F32::template st<V>(sDt + pc * kRow + pt, dt);
      F32::template st<V>(sDu + pc * kRow + pt, du);
#pragma unroll
      for (int i = 0; i < BCQ; ++i) *reinterpret_cast<float4*>(sBC + bc_slot(tid + i * NT)) = rbc[i];
    } else {
      if (softplus) delta_part(std::true_type{}); else delta_part(std::false_type{});
      pin();
      F32::template st<V>(sDt + pc * kRow + pt, dt);
      F32::template st<V>(sDu + pc * kRow + pt, du);
#pragma unroll
      for (int i = 0; i < BCQ; ++i) {
        const int q = tid + i * NT;
        const int t = r_t0 + (q % (kTT / 4)) * 4;
        float4 v = rbc[i];
        v.x = t < t_end ? v.x : 0.0f;
        v.y = t + 1 < t_end ? v.y : 0.0f;
        v.z = t + 2 < t_end ? v.z : 0.0f;
        v.w = t + 3 < t_end ? v.w : 0.0f;
        *reinterpret_cast<float4*>(sBC + bc_slot(q)) = v;
      }
    }
    if constexpr (kSkip) {
      uint32_t acc = 0u;
#pragma unroll
      for (int e = 0; e < V; ++e) acc |= __float_as_uint(dt[e]) | __float_as_uint(du[e]);
      bool live = !a_finite || __builtin_amdgcn_ballot_w64((acc & 0x7fffffffu) != 0u) != 0u;
      if (!live) {
        // 0 * B is zero for a finite B and NaN otherwise (the loaded words
        // past the chunk end can only make a tile live, which is always safe)
        float zb = 0.0f;
#pragma unroll
        for (int i = 0; i < BCQ; ++i) {
          if (bcis_c[i]) continue;
          zb = __builtin_fmaf(rbc[i].x, 0.0f, zb);
          zb = __builtin_fmaf(rbc[i].y, 0.0f, zb);
          zb = __builtin_fmaf(rbc[i].z, 0.0f, zb);
          zb = __builtin_fmaf(rbc[i].w, 0.0f, zb);
        }
        live = __builtin_amdgcn_ballot_w64((__float_as_uint(zb) & 0x7fffffffu) != 0u) != 0u;
      }
      next_live = live;
    }
  };

  // ---- recurrence of one tile from LDS
  // Its LDS operands: B and C of the tile's step for each lane (both 16-step
  // halves) and the Delta2 / Delta*u rows of each half.  In a one-wave
  // workgroup (S = 4) they are read ahead of the arithmetic: the first
  // half's rows and B, C right after the wave's own prep (the epilogue and
  // the loads cover their latency), the second half's before the first is
  // computed; such a workgroup also needs no barrier, since one wave's LDS
  // accesses run in program order (1.4B -1.8%, varlen -0.4%).  With several
  // waves per group the rows are read where the half starts (reading ahead
  // there cost 1.4% at 130m).  bc and cc are only ever written by these LDS
  // loads (they are DPP sources, see mul_bcast16).
  constexpr bool kPre = (W == 1);
  const float* rowDt = sDt + col * kRow;
  const float* rowDu = sDu + col * kRow;
  float* rowP = sP + (grp * kCG + col) * kRow;
  float bc[S][2], cc[S][2];  // lane j of the row: step 16*half + j of state grp*S+s
  float4 dqh[2][4], uqh[2][4];
  auto read_bc = [&]() {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int n = grp * S + s;
        const int tt = (16 * hh) ^ (16 * (grp & 1));
        bc[s][hh] = sBC[n * kTT + tt + col];
        cc[s][hh] = (MODE == kFull) ? sBC[(kNS + n) * kTT + tt + col] : 0.0f;
      }
  };
  auto read_half = [&](int hh) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      dqh[hh][g4] = *reinterpret_cast<const float4*>(rowDt + 16 * hh + g4 * 4);
      uqh[hh][g4] = *reinterpret_cast<const float4*>(rowDu + 16 * hh + g4 * 4);
    }
  };
  auto recur = [&]() {
    if constexpr (kPre) {
      read_half(1);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      read_bc();
    }
    if (kSkip && !cur_live) {
      // identity tile: the states stay; only the partial sums C.h
      static_for<0, 2>([&](auto HH) {
        constexpr int hh = decltype(HH)::value;
        float y4[4];
        static_for<0, 16>([&](auto JJ) {
          constexpr int j = decltype(JJ)::value;
          float yv = 0.0f;
#pragma unroll
          for (int s = 0; s < S; ++s) {
            if (s == 0)
              yv = mul_bcast16<j>(cc[s][hh], h[s]);
            else
              fmac_bcast16<j>(yv, cc[s][hh], h[s]);
          }
          y4[j % 4] = yv;
          if (j % 4 == 3)
            *reinterpret_cast<float4*>(rowP + 16 * hh + j - 3) = make_float4(y4[0], y4[1], y4[2], y4[3]);
        });
      });
      return;
    }
    static_for<0, 2>([&](auto HH) {
      constexpr int hh = decltype(HH)::value;
      if constexpr (!kPre) read_half(hh);
      float4 (&dq)[4] = dqh[hh];
      float4 (&uq)[4] = uqh[hh];
      float y4[4];
      static_for<0, 16>([&](auto JJ) {
        constexpr int j = decltype(JJ)::value;
        // The aggregate pass has no LDS store every four steps to bound how
        // far the scheduler hoists the exps of later steps (it then runs out
        // of registers): an empty asm that takes this group's Delta values
        // and the state after the previous group orders the groups.
        if constexpr (MODE == kAgg && j % 4 == 0) {
          asm volatile("" : "+v"(dq[j / 4].x), "+v"(dq[j / 4].y), "+v"(dq[j / 4].z), "+v"(dq[j / 4].w));
          asm volatile("" : "+v"(uq[j / 4].x), "+v"(uq[j / 4].y), "+v"(uq[j / 4].z), "+v"(uq[j / 4].w));
#pragma unroll
          for (int s = 0; s < S; ++s) asm volatile("" : "+v"(h[s]));
        }
        const float dt = get(dq[j / 4], j % 4);
        const float du = get(uq[j / 4], j % 4);
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
        y4[j % 4] = yv;
        if (MODE == kFull && j % 4 == 3)
          *reinterpret_cast<float4*>(rowP + 16 * hh + j - 3) = make_float4(y4[0], y4[1], y4[2], y4[3]);

      });
    });
  };

  // ---- epilogue of the tile at t0: sum partials, D skip, gate, store
  // bfloat16 vector stores of two tiles at once (see the epilogue)
  constexpr bool kPairStores = std::is_same<IO, BF16>::value && VEC && V >= 2;
  uint32_t yhold[kPairStores ? V / 2 : 1];
  auto store_words = [&](uint32_t off, const uint32_t* w) {
    if constexpr (V == 2) {
      __builtin_amdgcn_raw_buffer_store_b32(w[0], rY, off, 0, 0);
    } else if constexpr (V == 4) {
      u32x2 x;
      x.x = w[0]; x.y = w[1];
      __builtin_amdgcn_raw_buffer_store_b64(x, rY, off, 0, 0);
    } else {
      u32x4 x;
      x.x = w[0]; x.y = w[1]; x.z = w[2]; x.w = w[3];
      __builtin_amdgcn_raw_buffer_store_b128(x, rY, off, 0, 0);
    }
  };
  auto epilogue = [&](int t0, auto PARC) {
    constexpr int PAR = decltype(PARC)::value;  // tile parity within the unrolled pair
    float acc[V];
    F32::template ld<V>(sP + pc * kRow + pt, acc);
#pragma unroll
    for (int gg = 1; gg < NG; ++gg) {
      float v[V];
      F32::template ld<V>(sP + (gg * kCG + pc) * kRow + pt, v);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += v[e];
    }
    float out[V];
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = kGate ? (acc[e] + cDu[e]) * cG[e] : acc[e] + cDu[e];
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if constexpr (kPairStores) {
      // bfloat16: a tile's row slice is 64 bytes, half of a 128-byte line.
      // The first tile of a pair keeps its packed outputs in registers and
      // the second stores both halves back to back, so each line reaches
      // the L2 whole rather than as two halves a tile apart.
      if (PAR == 0 && t0 + kTT <= t_end) {
#pragma unroll
        for (int e = 0; e < V / 2; ++e) yhold[e] = BF16::cvt2(out[2 * e], out[2 * e + 1]);
        return;
      }
      if (PAR == 1 && t0 <= t_end) store_words(poff + toff - kTT * ES, yhold);
    }
    if (VEC && t0 + kTT <= t_end) {
      Buf::template st<V, kNT>(rY, poff + toff, out);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (t0 + pt + e < t_end) Buf::template st<1>(rY, poff + toff + e * ES, &out[e]);
    }
  };

  // Per tile: recurrence | barrier | prep of the next tile, epilogue of this
  // tile, loads of the tile two ahead | barrier.  Two register sets (A for
  // even tiles, B for odd ones) keep two tiles of loads in flight, which the
  // HBM latency under load needs; the loop is unrolled by two so each set
  // stays in fixed registers.  Prep, epilogue and loads run unconditionally
  // (past the chunk they read harmless words and prepare identity steps that
  // nothing stores): a conditional load would make the compiler copy its
  // result at the join and wait for it there.  An odd tile count runs one
  // extra all-identity tile.
  // bfloat16 in a one-wave group: a tile's row slice is 64 bytes, half of a
  // 128-byte line, and the two halves of a line, loaded a tile apart, met in
  // the L2 only when the line survived that long: with row strides of a
  // power of two (L = 8192: 16 KB) the lines of all rows fall into the same
  // few L2 sets and the varlen shape fetched 1.33x its input bytes (1.04x at
  // L = 8256).  Such groups load a line's two halves together instead: four
  // register sets (A, B, then A2, B2: tiles 4i .. 4i+3), refilled two at a
  // time, the loop unrolled by four; the last loads run up to seven tiles
  // ahead and 0 to 3 all-identity tiles close the chunk.
  constexpr bool kPairLoads = std::is_same<IO, BF16>::value && VEC && S == 4 && !CONV;
  const int ntiles = (t_end - t_begin + kTT - 1) / kTT;
  TileRegs A, B, A2, B2;
  load_tile(A, t_begin);
  load_tile(B, t_begin + kTT);
  if constexpr (kPairLoads) {
    load_tile(A2, t_begin + 2 * kTT);
    load_tile(B2, t_begin + 3 * kTT);
  }
  prep(A);
  if constexpr (kPre) {
    read_bc();
    read_half(0);
  }
#pragma unroll
  for (int e = 0; e < V; ++e) {
    cDu[e] = nDu[e];
    cG[e] = nG[e];
  }
  cur_live = next_live;
  if constexpr (!kPairLoads) load_tile(A, t_begin + 2 * kTT);
  // A one-wave workgroup needs no barrier: its LDS accesses run in program
  // order.
  if constexpr (!kPre) __syncthreads();
  // State after the tile [t0, t0 + kTT) when it ends a state chunk (or the
  // sequence): the checkpoint of the Mamba-2 page §4.3 chunked recompute.
  const int sc = static_cast<int>(p.state_chunk);
  const int64_t nsc = sc > 0 ? (L + sc - 1) / sc : 0;
  auto save_states = [&](int t0) {
    if (MODE != kFull || chunk_states == nullptr || t0 >= t_end) return;
    const int te = t0 + kTT;
    int64_t kc = -1;
    if (te <= Li && te % sc == 0)
      kc = te / sc - 1;
    else if (te >= Li && t_end == Li)
      kc = nsc - 1;
    if (kc < 0 || !dvalid) return;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t n = static_cast<int64_t>(grp) * S + s;
      if (n < N) chunk_states[((b * nsc + kc) * dim + d) * N + n] = h[s];
    }
  };
  auto half_step = [&](int t0, TileRegs& next, auto PARC, auto&& loads) {
    // With two or more states per lane the recurrence is a long VALU stream
    // while the other waves of the SIMD sit in the latency-bound prep and
    // epilogue: raising this wave's issue priority for the recurrence keeps
    // the VALU fed (measured: -10% on the 1.4B-like shape).  With one state
    // per lane it measured neutral to slightly worse.
    if constexpr (S >= 2) __builtin_amdgcn_s_setprio(1);
    recur();
    if constexpr (S >= 2) __builtin_amdgcn_s_setprio(0);
    save_states(t0);
    if constexpr (!kPre) __syncthreads();
    prep(next);
    if constexpr (kPre) {
      read_bc();
      read_half(0);
    }
    if (MODE == kFull) epilogue(t0, PARC);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      cDu[e] = nDu[e];
      cG[e] = nG[e];
    }
    cur_live = next_live;
    loads();
    if constexpr (!kPre) __syncthreads();
  };
  constexpr std::integral_constant<int, 0> kEven{};
  constexpr std::integral_constant<int, 1> kOdd{};
  if constexpr (kPairLoads) {
#pragma unroll 1
    for (int it = 0; it < ntiles; it += 4) {
      const int t0 = t_begin + it * kTT;
      half_step(t0, B, kEven, [&] {
        load_tile(A, t0 + 4 * kTT);
        load_tile(B, t0 + 5 * kTT);
      });
      half_step(t0 + kTT, A2, kOdd, [] {});
      half_step(t0 + 2 * kTT, B2, kEven, [&] {
        load_tile(A2, t0 + 6 * kTT);
        load_tile(B2, t0 + 7 * kTT);
      });
      half_step(t0 + 3 * kTT, A, kOdd, [] {});
    }
  } else {
#pragma unroll 1
    for (int it = 0; it < ntiles; it += 2) {
      const int t0 = t_begin + it * kTT;
      half_step(t0, B, kEven, [&] { load_tile(B, t0 + 3 * kTT); });
      half_step(t0 + kTT, A, kOdd, [&] { load_tile(A, t0 + 4 * kTT); });
    }
  }

  // ---- chunk end: final state or chunk aggregate
  if (!dvalid) return;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = static_cast<int64_t>(grp) * S + s;
    if (n >= N) continue;
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
// Kernels.
//  ssm_rows_kernel: one 16-channel group per block.  Grid: x = channel
//    group, y = batch row, z = chunk; block 64 * (4 / S) threads.
//  ssm_mixed_kernel: blocks of 256 threads of two kinds, so that a CU that
//    holds one of each gives every SIMD three (channel, state) chains per
//    lane: blocks [0, nA) run two groups at two states per lane (waves 0-1
//    and 2-3), blocks [nA, nA + nB) one group at one state per lane.  Grid:
//    x = nA + nB (all two-group blocks first, so that consecutive launches
//    of each kind spread over the CUs), z = chunk.  Per batch row,
//    groups [0, 2*pairs) belong to two-group blocks and the rest to
//    one-group blocks.
// --------------------------------------------------------------------------
template <typename IO, int S, int MODE, bool GATED, bool VEC, bool CONV>
__global__ __launch_bounds__(256 / S, 2) void ssm_rows_kernel(RowArgs<IO> args, CsSizes p) {
  extern __shared__ float smem[];
  // One-wave workgroups (S = 4): reserving VGPR 175 keeps every such
  // instantiation at 176 or more VGPRs, so a SIMD holds at most two of these
  // waves.  A third resident wave (what 150 VGPRs would allow) made a
  // 5120-workgroup bfloat16 launch (16 x 5120 x 16 x 8192) 25% slower, with
  // 50% more instruction-wait cycles and the same VALU count; a cap through
  // LDS size does not help, as it limits waves per CU, not per SIMD.
  if constexpr (S == 4) asm volatile("" ::: "v175");
  const int tid = threadIdx.x;
  // the wave index as an SGPR keeps every per-wave quantity uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dispatched round-robin over the 8 XCDs, each with its
  // own L2.  The (group, batch row, chunk) order is remapped so that each
  // XCD takes a contiguous range of it, channel groups fastest: an XCD then
  // works on a few batch rows (or chunks) at a time, whose B and C stay in
  // its L2 for all of their channel groups.
  const int64_t X = gridDim.x, Y = gridDim.y;
  const int64_t G = X * Y * gridDim.z;
  const int64_t pid = blockIdx.x + X * (blockIdx.y + Y * static_cast<int64_t>(blockIdx.z));
  const int64_t q = G / 8, r = G % 8, xcd = pid % 8, slot = pid / 8;
  const int64_t logical = xcd * q + (xcd < r ? xcd : r) + slot;
  rows_group<IO, S, MODE, GATED, VEC, CONV>(args, p, smem, tid, wave, (logical % X) * kCG, (logical / X) % Y,
                                            logical / (X * Y));
}

struct MixedSizes {
  int64_t pairs;    // two-group blocks per batch row
  int64_t singles;  // one-group blocks per batch row
};

template <typename IO, int MODE, bool GATED, bool VEC, bool CONV>
__global__ __launch_bounds__(256, 2) void ssm_mixed_kernel(RowArgs<IO> args, CsSizes p, MixedSizes m,
                                                           int smem_pair_floats) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nA = p.batch * m.pairs;
  int64_t x = blockIdx.x;
  if (gridDim.z == 1) {
    // XCD-contiguous ranges within each kind of block (the two-group blocks
    // are dispatched first, then the one-group blocks): an XCD then works on
    // whole batch rows, whose B and C stay in its L2, and still gets as many
    // blocks of each kind as the others
    const int64_t nB = p.batch * m.singles;
    const int64_t xcd = x % 8;
    if (x < nA) {
      const int64_t q = nA / 8, r = nA % 8;
      x = xcd * q + (xcd < r ? xcd : r) + x / 8;
    } else {
      const int64_t first = nA + (xcd - nA % 8 + 8) % 8;
      int64_t off = 0;
      for (int64_t xx = 0; xx < xcd; ++xx) {
        const int64_t o = (xx - nA % 8 + 8) % 8;
        off += o < nB ? (nB - o + 7) / 8 : 0;
      }
      x = nA + off + (x - first) / 8;
    }
  }
  if (x < nA) {
    const int sub = wave >> 1;
    const int64_t b = x / m.pairs;
    const int64_t g = 2 * (x % m.pairs) + sub;
    rows_group<IO, 2, MODE, GATED, VEC, CONV>(args, p, smem + sub * smem_pair_floats, tid - 128 * sub, wave & 1,
                                              g * kCG, b, blockIdx.z);
  } else {
    const int64_t q = x - nA;
    const int64_t b = q / m.singles;
    const int64_t g = 2 * m.pairs + q % m.singles;
    rows_group<IO, 1, MODE, GATED, VEC, CONV>(args, p, smem, tid, wave, g * kCG, b, blockIdx.z);
  }
}

// --------------------------------------------------------------------------
// Chunk combine: for every (b, n, d), run the carry over the K chunk totals,
//   h_init^(0) = h0 (zero if absent),  h_init^(k) = P^(k-1) h_init^(k-1) + H^(k-1)
// ([Scan page] §3.3 fix-up), writing h_init for k = 0..K-1.  One thread per
// (b, n, d); d is contiguous, so every access is coalesced.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ssm_combine_kernel(const float* __restrict__ agg_p,
                                                          const float* __restrict__ agg_h,
                                                          const float* __restrict__ h0,
                                                          float* __restrict__ h_init, int64_t batch, int64_t dim,
                                                          int64_t dstate, int64_t K) {
  const int64_t rows = batch * dstate * dim;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  // row i = (b, n, d) with d fastest; h0 is [b][d][n]
  const int64_t d = i % dim;
  const int64_t n = (i / dim) % dstate;
  const int64_t b = i / (dim * dstate);
  float hv = h0 != nullptr ? h0[(b * dim + d) * dstate + n] : 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    h_init[k * rows + i] = hv;
    if (k + 1 < K) hv = __builtin_fmaf(agg_p[k * rows + i], hv, agg_h[k * rows + i]);
  }
}

// --------------------------------------------------------------------------
// Chunk combine for many chunks: the scan over the K chunk totals of
// [Scan page] §3.3 as a blocked scan.  A workgroup takes 64 consecutive
// rows (b, n, d); its 16 wavefronts split K into 16 segments (lane = row,
// so every access is coalesced).  Each lane folds its segment's totals
// (P, H) in chunk order, the segment totals meet in LDS and each lane
// composes h0 with the totals of the segments before its own, in segment
// order, then walks its segment again writing h_init^(k).  Depth K/16 + 16
// instead of K.
// --------------------------------------------------------------------------
constexpr int kCombRows = 64;
constexpr int kCombSegs = 16;

__global__ __launch_bounds__(kCombRows * kCombSegs) void ssm_combine_scan_kernel(
    const float* __restrict__ agg_p, const float* __restrict__ agg_h, const float* __restrict__ h0,
    float* __restrict__ h_init, int64_t batch, int64_t dim, int64_t dstate, int64_t K) {
  __shared__ float sP[kCombSegs][kCombRows], sH[kCombSegs][kCombRows];
  const int64_t rows = batch * dstate * dim;
  const int lane = threadIdx.x & (kCombRows - 1);
  const int seg = threadIdx.x / kCombRows;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kCombRows + lane;
  const bool valid = i < rows;
  // segment seg covers chunks [k0, k1) (chunk K-1's total is never needed)
  const int64_t per = (K + kCombSegs - 1) / kCombSegs;
  const int64_t k0 = seg * per;
  const int64_t k1 = (k0 + per < K) ? k0 + per : K;
  float P = 1.0f, H = 0.0f;
  if (valid) {
    for (int64_t k = k0; k < k1 && k + 1 < K; ++k) {
      const float p = agg_p[k * rows + i], hh = agg_h[k * rows + i];
      H = __builtin_fmaf(p, H, hh);
      P = p * P;
    }
  }
  sP[seg][lane] = P;
  sH[seg][lane] = H;
  __syncthreads();
  if (!valid) return;
  // start state of the segment: h0, then the totals of segments 0 .. seg-1
  const int64_t d = i % dim;
  const int64_t n = (i / dim) % dstate;
  const int64_t b = i / (dim * dstate);
  float hv = h0 != nullptr ? h0[(b * dim + d) * dstate + n] : 0.0f;
  for (int s = 0; s < seg; ++s) hv = __builtin_fmaf(sP[s][lane], hv, sH[s][lane]);
  for (int64_t k = k0; k < k1; ++k) {
    h_init[k * rows + i] = hv;
    if (k + 1 < K) hv = __builtin_fmaf(agg_p[k * rows + i], hv, agg_h[k * rows + i]);
  }
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
size_t rows_smem_bytes(int S, int mode) {
  const int W = 4 / S;
  return sizeof(float) * (static_cast<size_t>(2) * kCG * kRow + static_cast<size_t>(2) * kNS * kTT +
                          (mode == kFull ? static_cast<size_t>(4 * W) * kCG * kRow : 0));
}

int rows_time_tile() { return kTT; }

template <typename IO>
static RowArgs<IO> row_args(const FwdArgs& a) {
  using T = typename IO::T;
  RowArgs<IO> r;
  r.u = static_cast<const T*>(a.u); r.dlt = static_cast<const T*>(a.delta); r.Ag = a.A;
  r.Bg = static_cast<const T*>(a.B); r.Cg = static_cast<const T*>(a.C); r.Dg = a.D;
  r.zg = static_cast<const T*>(a.z); r.biasg = a.bias; r.yg = static_cast<T*>(a.y);
  r.last_state = a.last_state; r.h_init = a.h_init; r.h0 = a.h0; r.chunk_states = a.chunk_states;
  r.agg_p = a.agg_p; r.agg_h = a.agg_h;
  r.convw = a.conv_w; r.convb = a.conv_b; r.uo = static_cast<T*>(a.u_out);
  return r;
}

static CsSizes cs_sizes(const FwdArgs& a) {
  CsSizes sz;
  sz.batch = a.batch; sz.dim = a.dim; sz.dstate = a.dstate; sz.L = a.L; sz.chunk = a.chunk; sz.softplus = a.softplus;
  sz.state_chunk = a.chunk_states != nullptr ? a.state_chunk : 0;
  sz.convk = a.conv_w != nullptr ? a.conv_k : 0;
  return sz;
}

template <typename IO, int S, int MODE, bool GATED, bool VEC, bool CONV>
static hipError_t launch_rows_v(const FwdArgs& a, int64_t nchunks, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.dim + kCG - 1) / kCG), static_cast<unsigned>(a.batch),
                  static_cast<unsigned>(nchunks));
  const size_t smem = rows_smem_bytes(S, MODE);
  auto kern = ssm_rows_kernel<IO, S, MODE, GATED, VEC, CONV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(256 / S), smem, st, row_args<IO>(a), cs_sizes(a));
  return hipGetLastError();
}

template <typename IO, int MODE, bool GATED, bool VEC, bool CONV>
static hipError_t launch_mixed_v(const FwdArgs& a, int64_t pairs, int64_t nchunks, hipStream_t st) {
  const int64_t groups = (a.dim + kCG - 1) / kCG;
  MixedSizes m;
  m.pairs = pairs;
  m.singles = groups - 2 * pairs;
  const size_t pair_bytes = rows_smem_bytes(2, MODE);
  const size_t smem = (2 * pair_bytes > rows_smem_bytes(1, MODE)) ? 2 * pair_bytes : rows_smem_bytes(1, MODE);
  const dim3 grid(static_cast<unsigned>(a.batch * (m.pairs + m.singles)), 1, static_cast<unsigned>(nchunks));
  auto kern = ssm_mixed_kernel<IO, MODE, GATED, VEC, CONV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(256), smem, st, row_args<IO>(a), cs_sizes(a), m,
                     static_cast<int>(pair_bytes / sizeof(float)));
  return hipGetLastError();
}

template <typename IO, int MODE, bool CONV>
static hipError_t dispatch_mixed_c(const FwdArgs& a, int64_t pairs, int64_t nchunks, hipStream_t st) {
  const bool vec = a.L % 8 == 0;
  if constexpr (MODE == kFull) {
    if (a.z != nullptr)
      return vec ? launch_mixed_v<IO, MODE, true, true, CONV>(a, pairs, nchunks, st)
                 : launch_mixed_v<IO, MODE, true, false, CONV>(a, pairs, nchunks, st);
  }
  return vec ? launch_mixed_v<IO, MODE, false, true, CONV>(a, pairs, nchunks, st)
             : launch_mixed_v<IO, MODE, false, false, CONV>(a, pairs, nchunks, st);
}

template <typename IO, int MODE>
static hipError_t dispatch_mixed(const FwdArgs& a, int64_t pairs, int64_t nchunks, hipStream_t st) {
  return a.conv_w != nullptr ? dispatch_mixed_c<IO, MODE, true>(a, pairs, nchunks, st)
                             : dispatch_mixed_c<IO, MODE, false>(a, pairs, nchunks, st);
}

template <typename IO, int S, int MODE, bool CONV>
static hipError_t dispatch_flags_c(const FwdArgs& a, int64_t nchunks, hipStream_t st) {
  const bool vec = a.L % 8 == 0;
  if constexpr (MODE == kFull) {
    if (a.z != nullptr)
      return vec ? launch_rows_v<IO, S, MODE, true, true, CONV>(a, nchunks, st)
                 : launch_rows_v<IO, S, MODE, true, false, CONV>(a, nchunks, st);
  }
  return vec ? launch_rows_v<IO, S, MODE, false, true, CONV>(a, nchunks, st)
             : launch_rows_v<IO, S, MODE, false, false, CONV>(a, nchunks, st);
}

template <typename IO, int S, int MODE>
static hipError_t dispatch_flags(const FwdArgs& a, int64_t nchunks, hipStream_t st) {
  return a.conv_w != nullptr ? dispatch_flags_c<IO, S, MODE, true>(a, nchunks, st)
                             : dispatch_flags_c<IO, S, MODE, false>(a, nchunks, st);
}

template <typename IO, int MODE>
static hipError_t dispatch_s(const FwdArgs& a, int S, int64_t nchunks, hipStream_t st) {
  if (S == 1) return dispatch_flags<IO, 1, MODE>(a, nchunks, st);
  if (S == 2) return dispatch_flags<IO, 2, MODE>(a, nchunks, st);
  if (S == 4) return dispatch_flags<IO, 4, MODE>(a, nchunks, st);
  return hipErrorInvalidValue;
}

hipError_t launch_rows_full(const FwdArgs& a, bool bf16, int S, int64_t nchunks, hipStream_t st) {
  return bf16 ? dispatch_s<BF16, kFull>(a, S, nchunks, st) : dispatch_s<F32, kFull>(a, S, nchunks, st);
}

hipError_t launch_rows_agg(const FwdArgs& a, bool bf16, int S, int64_t nchunks, hipStream_t st) {
  return bf16 ? dispatch_s<BF16, kAgg>(a, S, nchunks, st) : dispatch_s<F32, kAgg>(a, S, nchunks, st);
}

hipError_t launch_mixed_full(const FwdArgs& a, bool bf16, int64_t pairs, int64_t nchunks, hipStream_t st) {
  return bf16 ? dispatch_mixed<BF16, kFull>(a, pairs, nchunks, st) : dispatch_mixed<F32, kFull>(a, pairs, nchunks, st);
}

hipError_t launch_combine(const float* agg_p, const float* agg_h, const float* h0, float* h_init, int64_t batch,
                          int64_t dim, int64_t dstate, int64_t K, hipStream_t st) {
  const int64_t rows = batch * dstate * dim;
  if (K >= kCombScanMinChunks) {
    const unsigned blocks = static_cast<unsigned>((rows + kCombRows - 1) / kCombRows);
    hipLaunchKernelGGL(ssm_combine_scan_kernel, dim3(blocks), dim3(kCombRows * kCombSegs), 0, st, agg_p, agg_h, h0,
                       h_init, batch, dim, dstate, K);
    return hipGetLastError();
  }
  const unsigned blocks = static_cast<unsigned>((rows + 255) / 256);
  hipLaunchKernelGGL(ssm_combine_kernel, dim3(blocks), dim3(256), 0, st, agg_p, agg_h, h0, h_init, batch, dim, dstate,
                     K);
  return hipGetLastError();
}

}  // namespace ssm

// Selective-scan backward kernel for gfx950 (MI355X, CDNA4): the gradients
// of every input by chunked recomputation.
//
// Pages cited:
//   [Scan page]    "Hardware-aware parallel associative scan for Mamba"
//                  (http://www.pwwt.cn/news/6375169/)
//   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
//                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
//
// Method.  The forward keeps only the state at every chunk boundary; the
// backward visits the chunks from last to first, re-runs each chunk forward
// from its boundary state to get the states inside it, and walks the chunk
// back ([Scan page] §4.2 on recomputation in training; [Mamba-2 page] §4.3,
// the chunked recomputation with the L = 12, chunk 4 example).  With s_t the
// sum before the gate and g_t = dLoss/dh_t, the reverse walk computes
//     gs_t   = dy_t silu(z_t)            (dy_t without a gate)
//     g_t    = C_t gs_t + a_{t+1} g_{t+1}     (g after the last step = dlast)
//     dB_t  += g_t Delta_t u_t,  dC_t += gs_t h_t     (summed over channels)
//     dA    += g_t a_t h_{t-1} Delta_t            (summed over batch and time)
//     du_t   = D gs_t + Delta_t sum_n g_t B_t
//     dDelta = u_t sum_n g_t B_t + sum_n g_t a_t h_{t-1} A
//     dz_t   = dy_t s_t silu'(z_t),  ddelta = dDelta softplus'(x) = dDelta sigmoid(x)
// i.e. the chain rule through the recurrence h_t = a_t h_{t-1} + b_t of
// [Scan page] §1.2.
//
// What runs where
// ---------------
// The row layout of the forward kernel: a workgroup owns 16 channels of one
// batch row and all (up to 16) states; lane `col` of a row is channel
// c0 + col and row `row` of wave `w` carries states (4w + row)*S + s.  Time
// runs in tiles of 16 steps.  For each chunk:
//   phase 1: the chunk forward over all its tiles but the last, keeping the
//            state at every tile start in LDS (lane-private slots);
//   phase 2: its tiles from last to first, each in two barrier intervals:
//     compute (every lane): the tile forward again from its start state,
//            keeping h_t (and a_t with two states per lane) of the 16 steps in
//            registers, with the partial sums C.h; then the 16 steps back.
//            Sums over the lane's states are finished across the wave's
//            four rows with the gfx950 lane swaps (v_permlane32_swap,
//            v_permlane16_swap: four values summed over four rows in three
//            swaps and three adds) and left in LDS per (wave, channel, step).
//            dB and dC, sums over the row's 16 channels, go through a DPP
//            reduce-scatter (after four butterfly stages lane j of a row holds
//            the sum for one step of its state; the first two stages use
//            bank-masked DPP adds), fed step by step so that each stage's
//            pair is ready as soon as its second half is, and leave the
//            workgroup as one atomic add per (state, step).
//     epilogue + prep (every thread, V steps of one channel): du, ddelta,
//            dz of this tile from the LDS sums; then Delta2, Delta*u, gs, B
//            and C of the tile before into LDS, whose global loads were issued
//            a tile ahead.
// Exp and the step arithmetic are those of the forward kernel (a =
// exp2(Delta2 A), b = B (Delta2 ln2 u), h = fma(a, h, b)), so the states
// recomputed from a chunk boundary written by the forward repeat the
// forward's values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {

using namespace dev;

namespace {

constexpr int kBT = kBwdTile;   // steps per tile (16: one DPP row of steps)
constexpr int kCG = 16;         // channels per workgroup
constexpr int kNS = 16;         // state slots per workgroup
constexpr int kBR = kBT + 4;    // LDS row stride in floats (float4 rows, staggered banks)
constexpr int kXR = kBR + 20;   // CONV: LDS row of pre (kBR) then x at steps -3 .. 15 (and padding)

// DPP lane patterns within a row of 16 lanes (lane l reads the lane named)
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]: l ^ 1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]: l ^ 2
constexpr int kRowRor4 = 0x124;   // row_ror:4: (l - 4) mod 16
constexpr int kRowRor8 = 0x128;   // row_ror:8: (l - 8) mod 16 = l ^ 8

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Butterfly stages of the reduce-scatter.  Of a pair (lo, hi) of values
// whose index differs in this stage's bit, lanes whose selector bit is set
// end with hi summed with their partner's hi, the others with lo summed with
// their partner's lo.  Stages 1 and 2 select on lane bits 2 and 3, i.e. on
// the DPP bank (four consecutive lanes): all lanes add lo, then a
// bank-masked add overwrites the selected banks with hi (two instructions;
// s_nop 1 gives the two wait states a DPP read needs after a VALU write of
// its source).  Stages 3 and 4 select on bits 0 and 1 with v_cndmask (three
// instructions).
__device__ __forceinline__ float rs_stage1(float lo, float hi) {
  float out = lo + dpp_f<kRowRor4>(lo);
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:4 row_mask:0xf bank_mask:0xa"
      : "+v"(out)
      : "v"(hi));
  return out;
}
__device__ __forceinline__ float rs_stage2(float lo, float hi) {
  float out = lo + dpp_f<kRowRor8>(lo);
  asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "+v"(out)
      : "v"(hi));
  return out;
}
template <int CTRL>
__device__ __forceinline__ float rs_stage_sel(float lo, float hi, bool sel_hi) {
  const float keep = sel_hi ? hi : lo;
  const float send = sel_hi ? lo : hi;
  return keep + dpp_f<CTRL>(send);
}

// Reduce-scatter of 16 values over the 16 lanes of a row, fed one value at a
// time: value number P (P = 0..15 in the order produced) has index P, and
// stage k (k = 1..4) combines indices that differ in bit k-1, selecting on
// lane bit 2, 3, 0, 1 with the partner lane (l - 4) mod 16, l ^ 8, l ^ 1,
// l ^ 2.  Each partner agrees with the lane on every earlier selector bit
// and differs in this one; after stage 2 a lane's values are summed over
// the four lanes that share its bits 0 and 1, after stage 4 over all 16, so
// lane l holds the full sum of value number
// rs_value(l) = bit2(l) + 2 bit3(l) + 4 bit0(l) + 8 bit1(l).
// Both halves of every pair are consecutive in production order, so at most
// one value waits per stage.
__device__ __forceinline__ int rs_value(int l) {
  return ((l >> 2) & 1) | (((l >> 3) & 1) << 1) | ((l & 1) << 2) | (((l >> 1) & 1) << 3);
}

struct RsTree {
  float p0, p1, p2, p3, out;
};

template <int P>
__device__ __forceinline__ void rs_push(RsTree& t, float x, const bool (&sel)[2]) {
  if constexpr ((P & 1) == 0) {
    t.p0 = x;
  } else {
    const float y1 = rs_stage1(t.p0, x);
    if constexpr (((P >> 1) & 1) == 0) {
      t.p1 = y1;
    } else {
      const float y2 = rs_stage2(t.p1, y1);
      if constexpr (((P >> 2) & 1) == 0) {
        t.p2 = y2;
      } else {
        const float y3 = rs_stage_sel<kQuadSwap1>(t.p2, y2, sel[0]);
        if constexpr (((P >> 3) & 1) == 0)
          t.p3 = y3;
        else
          t.out = rs_stage_sel<kQuadSwap2>(t.p3, y3, sel[1]);
      }
    }
  }
}

// Sum over the four rows (16 lanes each) of a wave of four values at once:
// row r of the result holds the four-row sum of x_{o(r)}, o = (0, 2, 1, 3).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; v_permlane16_swap exchanges the odd rows of the
// first with the even rows of the second.
__device__ __forceinline__ float xrow_sum4(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  const float p = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x2), __float_as_uint(x3), false, false);
  const float q = __uint_as_float(c[0]) + __uint_as_float(c[1]);
  const auto e = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(q), false, false);
  return __uint_as_float(e[0]) + __uint_as_float(e[1]);
}

template <typename IO>
struct BwdDev {
  const typename IO::T* u;
  const typename IO::T* dlt;
  const typename IO::T* Bg;
  const typename IO::T* Cg;
  const typename IO::T* zg;
  const typename IO::T* dy;
  const float* Ag;
  const float* Dg;
  const float* biasg;
  const float* h0;
  const float* cst;    // chunk states [b][K][d][n]
  const float* dlast;
  typename IO::T* du;
  typename IO::T* ddelta;
  typename IO::T* dz;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dbias;
  float* dh0;
  const float* convw;   // CONV: [d][K] conv1d weights (u then points at x, du at dx)
  const float* convb;   // CONV: [d] nullable
  float* dconvw;        // CONV: [d][K], accumulated
  float* dconvb;        // CONV: [d] nullable, accumulated
};

struct BwdSz {
  int64_t batch, dim, dstate, L, sc;
  int softplus;
  int convk;
};

}  // namespace

// S: states per lane (1, 2 or 4); workgroup = 16 channels x 16 states in
// 4/S wavefronts; grid (ceil(d_inner/16), batch).  With S <= 2 the tile's a_t
// are kept in registers; with S = 4 they are recomputed on the way back (the
// registers for them are not there).
// CONV: the scan's input is u = silu(pre), pre = conv_b + sum_j w4[j] x_{t-3+j}
// (the causal conv1d in front, K <= 4 taps right-aligned in w4), recomputed
// from x like the forward; the epilogue turns du into dpre = du silu'(pre),
// adds dpre x into dconv_w and dpre into dconv_b, and leaves dpre in LDS;
// dx_t = sum_j w4[j] dpre_{t+3-j} of a tile is formed after the next tile's
// prep barrier, when the dpre of the tile and of the one after it (the
// previous tile processed) are both in LDS.
template <typename IO, int S, bool GATED, bool VEC, bool CONV>
__global__ __launch_bounds__(256 / S, S == 1 ? 3 : 2) void ssm_bwd_kernel(BwdDev<IO> a, BwdSz p) {
  using T = typename IO::T;
  using Buf = typename BufOf<IO>::type;
  constexpr int W = 4 / S;
  constexpr int NT = 64 * W;
  constexpr int V = kCG * kBT / NT;             // prep / epilogue steps per thread
  constexpr int TPC = kBT / V;                  // prep / epilogue threads per channel
  constexpr int BCG = 2 * kNS * kBT / 4;        // B/C float4 groups per tile
  constexpr int BCQ = (BCG + NT - 1) / NT;       // per thread (the first BCG threads with S = 1)
  constexpr bool kKeepA = S <= 2;
  constexpr uint32_t ES = sizeof(T);
  static_assert(S == 1 || S == 2 || S == 4, "S");
  static_assert(V * NT == kCG * kBT && BCG % 64 == 0, "tiling");

  extern __shared__ float smem[];
  float* sDt = smem;                    // [16][kBR] Delta2
  float* sDu = sDt + kCG * kBR;         // [16][kBR] Delta*u
  float* sGs = sDu + kCG * kBR;         // [16][kBR] gs
  float* sBC = sGs + kCG * kBR;         // [2][16 n][16 t] B then C
  float* sX = sBC + 2 * kNS * kBT;      // [W][3][16][kBR] four-row sums: s, r, w
  float* sDP = sX + W * 3 * kCG * kBR;  // CONV: [2][16][kBR] dpre of two consecutive tiles
  float* sPX = sDP + (CONV ? 2 * kCG * kBR : 0);  // CONV: [2][16][kXR] pre (kBR) and x (3 + kBT) of a tile
  float* sCk = sPX + (CONV ? 2 * kCG * kXR : 0);  // [tiles][16 n][16 c] tile start states

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row = lane >> 4;
  const int col = lane & 15;
  const int grp = wave * 4 + row;
  const int64_t b = blockIdx.y;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kCG;
  const int64_t dim = p.dim, L = p.L, N = p.dstate;
  const int Li = static_cast<int>(L);
  const bool softplus = p.softplus != 0;

  // ---- chains of this lane: channel c0 + col, states grp*S + s
  const int64_t d = c0 + col;
  const bool dvalid = d < dim;
  float An[S], g[S], anext[S], dAacc[S];
  bool ok[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t n = static_cast<int64_t>(grp) * S + s;
    ok[s] = dvalid && n < N;
    An[s] = ok[s] ? a.Ag[d * N + n] : 0.0f;
    g[s] = (ok[s] && a.dlast != nullptr) ? a.dlast[(b * dim + d) * N + n] : 0.0f;
    anext[s] = 1.0f;
    dAacc[s] = 0.0f;
  }

  // ---- prep / epilogue cell of this thread: channel pc, steps [pt, pt + V)
  const int pc = tid / TPC;
  const int pt = (tid % TPC) * V;
  const int64_t pd = c0 + pc;
  const bool pvalid = pd < dim;
  const float bias2 = (pvalid && a.biasg != nullptr) ? a.biasg[pd] * kLog2e : 0.0f;
  const float Dd = (pvalid && a.Dg != nullptr) ? a.Dg[pd] : 0.0f;
  float dDacc = 0.0f, dbacc = 0.0f;

  // ---- buffer resources (reads past a resource return zero, writes past it
  // are dropped); byte offsets fit in 32 bits (the host bounds 16 * L * 4)
  const int64_t rows_left = dim - c0;
  const int64_t rows_here = rows_left < kCG ? rows_left : kCG;
  const int64_t row0 = (b * dim + c0) * L;
  const uint32_t in_bytes = static_cast<uint32_t>(rows_here * L * ES);
  const Rsrc rU = make_rsrc(a.u + row0, in_bytes);
  const Rsrc rD = make_rsrc(a.dlt + row0, in_bytes);
  const Rsrc rZ = make_rsrc(GATED ? a.zg + row0 : a.u + row0, in_bytes);
  const Rsrc rY = make_rsrc(a.dy + row0, in_bytes);
  const Rsrc rOU = make_rsrc(a.du + row0, in_bytes);
  const Rsrc rOD = make_rsrc(a.ddelta + row0, in_bytes);
  const Rsrc rOZ = make_rsrc(GATED ? a.dz + row0 : a.du + row0, GATED ? in_bytes : 0u);
  const uint32_t bc_bytes = static_cast<uint32_t>(N * L * ES);
  const Rsrc rB = make_rsrc(a.Bg + b * N * L, bc_bytes);
  const Rsrc rC = make_rsrc(a.Cg + b * N * L, bc_bytes);
  const uint32_t poff = static_cast<uint32_t>((pc * L + pt) * ES);

  // B/C groups of this thread: group q = tid + i*NT (q < BCG; whole waves
  // have a group or none) covers 4 steps of state (q/4) % 16 of B (q < 64)
  // or C; its LDS slot is sBC + 4q.
  uint32_t bcoff[BCQ];
  bool bcis_c[BCQ], bchas[BCQ];
#pragma unroll
  for (int i = 0; i < BCQ; ++i) {
    const int q = tid + i * NT;
    const int q0 = __builtin_amdgcn_readfirstlane(wave * 64 + i * NT);
    bchas[i] = q0 < BCG;
    bcis_c[i] = q0 >= kNS * kBT / 4;
    const int n = (q / (kBT / 4)) % kNS;
    bcoff[i] = static_cast<uint32_t>((n * L + (q % (kBT / 4)) * 4) * ES);
  }

  // ---- raw words of one tile, loaded a tile ahead of their use
  constexpr int RW = VEC ? Buf::template kWords<V> : V;
  constexpr int BW = VEC ? Buf::template kWords<4> : 4;
  constexpr int HW = CONV ? 3 : 1;  // conv halo: the 3 steps before the slot
  struct TileRegs {
    uint32_t wu[RW], wd[RW], wz[RW], wy[RW];
    uint32_t wh[HW];
    uint32_t wbc[BCQ][BW];
  };
  // FULL: also z, dy and C (phase 2); otherwise u, delta and B only.
  auto load_tile = [&](TileRegs& R, int t0, auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if constexpr (CONV) {
      // x at steps pt-3 .. pt-1 (halo_offset: never below zero; the conv
      // front zeroes the steps before 0)
#pragma unroll
      for (int j = 0; j < 3; ++j) Buf::template ldw<1>(rU, halo_offset(poff + toff, (3 - j) * ES), &R.wh[j]);
    }
    if constexpr (VEC) {
      Buf::template ldw<V>(rU, poff + toff, R.wu);
      Buf::template ldw<V>(rD, poff + toff, R.wd);
      if constexpr (FULL) {
        if constexpr (GATED) Buf::template ldw<V>(rZ, poff + toff, R.wz);
        Buf::template ldw<V>(rY, poff + toff, R.wy);
      }
#pragma unroll
      for (int i = 0; i < BCQ; ++i)
        if (bchas[i] && (FULL || !bcis_c[i])) Buf::template ldw<4>(bcis_c[i] ? rC : rB, bcoff[i] + toff, R.wbc[i]);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Buf::template ldw<1>(rU, poff + toff + e * ES, &R.wu[e]);
        Buf::template ldw<1>(rD, poff + toff + e * ES, &R.wd[e]);
        if constexpr (FULL) {
          if constexpr (GATED) Buf::template ldw<1>(rZ, poff + toff + e * ES, &R.wz[e]);
          Buf::template ldw<1>(rY, poff + toff + e * ES, &R.wy[e]);
        }
      }
#pragma unroll
      for (int i = 0; i < BCQ; ++i)
        if (bchas[i] && (FULL || !bcis_c[i]))
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Buf::template ldw<1>(bcis_c[i] ? rC : rB, bcoff[i] + toff + e * ES, &R.wbc[i][e]);
    }
  };

  auto unpack = [&](uint32_t* w, float* o) {
    if constexpr (VEC) {
      Buf::template unpack<V>(w, o);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) Buf::template unpack<1>(&w[e], &o[e]);
    }
  };
  auto unpack_bc = [&](TileRegs& R, int i) {
    float v[4];
    if constexpr (VEC) {
      Buf::template unpack<4>(R.wbc[i], v);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) Buf::template unpack<1>(&R.wbc[i][e], &v[e]);
    }
    return make_float4(v[0], v[1], v[2], v[3]);
  };

  // ---- conv front (CONV): u = silu(pre) from x and the halo
  float w4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float cbias = 0.0f;
  float dcw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dcb = 0.0f;
  if constexpr (CONV) {
    const int Kc = p.convk;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (pvalid && j >= 4 - Kc) w4[j] = a.convw[pd * Kc + (j - (4 - Kc))];
    cbias = (pvalid && a.convb != nullptr) ? a.convb[pd] : 0.0f;
  }
  // xs[0..V+2] = x at steps pt-3 .. pt+V-1 of the tile; ru <- u, pre kept
  auto conv_front = [&](TileRegs& R, int t0, float* ru, float* xs, float* pre) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      float v;
      Buf::template unpack<1>(&R.wh[j], &v);
      xs[j] = (t0 + pt - 3 + j >= 0) ? v : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < V; ++e) xs[3 + e] = ru[e];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float pr = cbias;
#pragma unroll
      for (int j = 0; j < 4; ++j) pr = __builtin_fmaf(w4[j], xs[e + j], pr);
      pre[e] = pr;
      ru[e] = silu(pr);
    }
  };

  // ---- phase-1 prep: Delta2 and Delta*u of a whole tile, and B, into LDS
  auto prep1 = [&](TileRegs& R, int t0) {
    float ru[V], rd[V], dt[V], du[V];
    unpack(R.wu, ru);
    unpack(R.wd, rd);
    if constexpr (CONV) {
      float xs[V + 3], pre[V];
      conv_front(R, t0, ru, xs, pre);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float v2 = delta2(rd[e], bias2, softplus);
      dt[e] = v2;
      du[e] = (v2 * kLn2) * ru[e];
    }
    F32::template st<V>(sDt + pc * kBR + pt, dt);
    F32::template st<V>(sDu + pc * kBR + pt, du);
#pragma unroll
    for (int i = 0; i < BCQ; ++i)
      if (bchas[i] && !bcis_c[i]) *reinterpret_cast<float4*>(sBC + (tid + i * NT) * 4) = unpack_bc(R, i);
  };

  // ---- phase-2 prep; e* keep what the epilogue of the same tile needs
  float eu[V], edn[V], esig[V], egs[V], ee[V];
  auto prep2 = [&](TileRegs& R, int t0, int t_end) {
    float ru[V], rd[V], rz[V], ry[V], dt[V], du[V], gsv[V];
    unpack(R.wu, ru);
    unpack(R.wd, rd);
    unpack(R.wy, ry);
    if constexpr (GATED) unpack(R.wz, rz);
    if constexpr (CONV) {
      // pre and x of the tile go to LDS for the epilogue (slot by tile parity)
      float xs[V + 3], pre[V];
      conv_front(R, t0, ru, xs, pre);
      float* row = sPX + ((t0 / kBT) & 1) * kCG * kXR + pc * kXR;
#pragma unroll
      for (int e = 0; e < V; ++e) row[pt + e] = pre[e];
#pragma unroll
      for (int e = 0; e < V; ++e) row[kBR + 3 + pt + e] = xs[3 + e];
      if (pt == 0) {
#pragma unroll
        for (int j = 0; j < 3; ++j) row[kBR + j] = xs[j];
      }
    }
    const bool full = t0 + kBT <= t_end;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      // past the end of the sequence a read runs into the next row: zero it
      const bool in = full || t0 + pt + e < t_end;
      const float uu = in ? ru[e] : 0.0f;
      const float yy = in ? ry[e] : 0.0f;
      const float x2 = __builtin_fmaf(rd[e], kLog2e, bias2);
      const float v2 = in ? delta2(rd[e], bias2, softplus) : 0.0f;
      dt[e] = v2;
      edn[e] = v2 * kLn2;
      du[e] = edn[e] * uu;
      // softplus'(x) = sigmoid(x) = 1 / (1 + 2^-x2)
      esig[e] = softplus ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x2)) : 1.0f;
      eu[e] = uu;
      if constexpr (GATED) {
        const float zz = rz[e];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * zz));
        gsv[e] = yy * (zz * sg);
        // d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))
        ee[e] = yy * (sg * (1.0f + zz * (1.0f - sg)));
      } else {
        gsv[e] = yy;
        ee[e] = 0.0f;
      }
      egs[e] = gsv[e];
    }
    F32::template st<V>(sDt + pc * kBR + pt, dt);
    F32::template st<V>(sDu + pc * kBR + pt, du);
    F32::template st<V>(sGs + pc * kBR + pt, gsv);
#pragma unroll
    for (int i = 0; i < BCQ; ++i) {
      if (!bchas[i]) continue;
      const int q = tid + i * NT;
      float4 v = unpack_bc(R, i);
      if (!full) {
        const int t = t0 + (q % (kBT / 4)) * 4;
        v.x = t < t_end ? v.x : 0.0f;
        v.y = t + 1 < t_end ? v.y : 0.0f;
        v.z = t + 2 < t_end ? v.z : 0.0f;
        v.w = t + 3 < t_end ? v.w : 0.0f;
      }
      *reinterpret_cast<float4*>(sBC + q * 4) = v;
    }
  };

  const float* rowDt = sDt + col * kBR;
  const float* rowDu = sDu + col * kBR;
  const float* rowGs = sGs + col * kBR;
  float* xw = sX + wave * 3 * kCG * kBR;  // this wave's four-row sums
  const int xo = ((row & 1) << 1) | (row >> 1);
  // LDS slot of this lane's state s at tile start i: sCk[(i*16 + grp*S + s)*16 + col]
  float* myCk = sCk + (grp * S) * kCG + col;

  // ---- phase 1: the tile forward, state only
  auto recur1 = [&](float (&h)[S]) {
    float bc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) bc[s] = sBC[(grp * S + s) * kBT + col];
    static_for<0, 4>([&](auto G) {
      constexpr int g4 = decltype(G)::value;
      const float4 dq = *reinterpret_cast<const float4*>(rowDt + 4 * g4);
      const float4 uq = *reinterpret_cast<const float4*>(rowDu + 4 * g4);
      static_for<0, 4>([&](auto JJ) {
        constexpr int jj = decltype(JJ)::value;
        constexpr int j = 4 * g4 + jj;
        const float dt = get(dq, jj);
        const float du = get(uq, jj);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const float av = __builtin_amdgcn_exp2f(dt * An[s]);
          h[s] = __builtin_fmaf(av, h[s], mul_bcast16<j>(bc[s], du));
        }
      });
    });
  };

  // ---- phase 2 compute of one tile
  const bool sel[2] = {(col & 1) != 0, (col & 2) != 0};
  auto compute = [&](const float (&hst)[S], int t0, int t_end, bool last_tile_of_seq) {
    float bc[S], cc[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      bc[s] = sBC[(grp * S + s) * kBT + col];
      cc[s] = sBC[(kNS + grp * S + s) * kBT + col];
    }
    // forward again: h_t (and a_t) of the 16 steps, partial C.h
    float hs[kBT][S];
    float as[kKeepA ? kBT : 1][S];
    {
      float hc[S];
#pragma unroll
      for (int s = 0; s < S; ++s) hc[s] = hst[s];
      static_for<0, 4>([&](auto G) {
        constexpr int g4 = decltype(G)::value;
        const float4 dq = *reinterpret_cast<const float4*>(rowDt + 4 * g4);
        const float4 uq = *reinterpret_cast<const float4*>(rowDu + 4 * g4);
        float y4[4];
        static_for<0, 4>([&](auto JJ) {
          constexpr int jj = decltype(JJ)::value;
          constexpr int j = 4 * g4 + jj;
          const float dt = get(dq, jj);
          const float du = get(uq, jj);
          float yp = 0.0f;
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const float av = __builtin_amdgcn_exp2f(dt * An[s]);
            if constexpr (kKeepA) as[j][s] = av;
            hc[s] = __builtin_fmaf(av, hc[s], mul_bcast16<j>(bc[s], du));
            hs[j][s] = hc[s];
            if (s == 0)
              yp = mul_bcast16<j>(cc[s], hc[s]);
            else
              fmac_bcast16<j>(yp, cc[s], hc[s]);
          }
          y4[jj] = yp;
        });
        xw[(0 * kCG + col) * kBR + 4 * g4 + xo] = xrow_sum4(y4[0], y4[1], y4[2], y4[3]);
      });
    }
    // back over the 16 steps
    RsTree tb[S], tc[S];
    float rprev = 0.0f, wprev = 0.0f;
    float4 dq, uq, gq;
    static_for<0, kBT>([&](auto PP) {
      constexpr int P = decltype(PP)::value;
      constexpr int j = kBT - 1 - P;
      if constexpr (j % 4 == 3) {
        dq = *reinterpret_cast<const float4*>(rowDt + j - 3);
        uq = *reinterpret_cast<const float4*>(rowDu + j - 3);
        gq = *reinterpret_cast<const float4*>(rowGs + j - 3);
      }
      const float dt = get(dq, j % 4);
      const float du = get(uq, j % 4);
      const float gs = get(gq, j % 4);
      float rp = 0.0f, wp = 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        float av;
        if constexpr (kKeepA)
          av = as[j][s];
        else
          av = __builtin_amdgcn_exp2f(dt * An[s]);
        g[s] = __builtin_fmaf(anext[s], g[s], mul_bcast16<j>(cc[s], gs));
        const float hp = (j > 0) ? hs[j > 0 ? j - 1 : 0][s] : hst[s];
        const float qa = (g[s] * hp) * av;
        dAacc[s] = __builtin_fmaf(qa, dt, dAacc[s]);
        if (s == 0) {
          wp = qa * An[s];
          rp = mul_bcast16<j>(bc[s], g[s]);
        } else {
          wp = __builtin_fmaf(qa, An[s], wp);
          fmac_bcast16<j>(rp, bc[s], g[s]);
        }
        rs_push<P>(tb[s], g[s] * du, sel);
        rs_push<P>(tc[s], gs * hs[j][s], sel);
        anext[s] = av;
      }
      if constexpr ((P & 1) == 0) {
        rprev = rp;
        wprev = wp;
      } else {
        // rows 0..3 get r_{j+1}, r_j, w_{j+1}, w_j
        const float v = xrow_sum4(rprev, wprev, rp, wp);
        const int q = row < 2 ? 1 : 2;
        const int step = (row & 1) ? j : j + 1;
        xw[(q * kCG + col) * kBR + step] = v;
      }
    });
    // dB, dC of this tile: lane col holds value number rs_value(col), the
    // value produced at step 15 - rs_value(col)
    const int tl = t0 + kBT - 1 - rs_value(col);
    if (tl < t_end) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int64_t n = static_cast<int64_t>(grp) * S + s;
        if (n < N) {
          unsafeAtomicAdd(a.dB + (b * N + n) * L + tl, tb[s].out);
          unsafeAtomicAdd(a.dC + (b * N + n) * L + tl, tc[s].out);
        }
      }
    }
    // gradient of the start state of the sequence: dh0 = a_0 g_0
    if (last_tile_of_seq && a.dh0 != nullptr) {
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (ok[s]) a.dh0[(b * dim + d) * N + grp * S + s] = anext[s] * g[s];
    }
  };

  // ---- epilogue of one tile
  auto epilogue = [&](int t0, int t_end) {
    float sv[V], rv[V], wv[V];
    F32::template ld<V>(sX + (0 * kCG + pc) * kBR + pt, sv);
    F32::template ld<V>(sX + (1 * kCG + pc) * kBR + pt, rv);
    F32::template ld<V>(sX + (2 * kCG + pc) * kBR + pt, wv);
#pragma unroll
    for (int w = 1; w < W; ++w) {
      float s2[V], r2[V], w2[V];
      const float* base = sX + w * 3 * kCG * kBR;
      F32::template ld<V>(base + (0 * kCG + pc) * kBR + pt, s2);
      F32::template ld<V>(base + (1 * kCG + pc) * kBR + pt, r2);
      F32::template ld<V>(base + (2 * kCG + pc) * kBR + pt, w2);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        sv[e] += s2[e];
        rv[e] += r2[e];
        wv[e] += w2[e];
      }
    }
    float odu[V], odd[V], odz[V];
    const bool full = t0 + kBT <= t_end;
    float* dp = sDP + ((t0 / kBT) & 1) * kCG * kBR + pc * kBR + pt;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float sfull = __builtin_fmaf(Dd, eu[e], sv[e]);
      odu[e] = __builtin_fmaf(Dd, egs[e], edn[e] * rv[e]);
      const float ddt = __builtin_fmaf(eu[e], rv[e], wv[e]);
      odd[e] = ddt * esig[e];
      odz[e] = sfull * ee[e];
      if (full || t0 + pt + e < t_end) {
        dDacc = __builtin_fmaf(egs[e], eu[e], dDacc);
        dbacc += odd[e];
      }
      if constexpr (CONV) {
        // dpre = du silu'(pre), silu'(p) = sig(p) (1 + p (1 - sig(p))); zero past the end
        const float* row = sPX + ((t0 / kBT) & 1) * kCG * kXR + pc * kXR;
        const float pr = row[pt + e];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * pr));
        const float dpr = (full || t0 + pt + e < t_end) ? odu[e] * (sg * (1.0f + pr * (1.0f - sg))) : 0.0f;
        dp[e] = dpr;
        dcb += dpr;
#pragma unroll
        for (int j = 0; j < 4; ++j) dcw[j] = __builtin_fmaf(dpr, row[kBR + pt + e + j], dcw[j]);
      }
    }
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if (VEC && full) {
      if constexpr (!CONV) Buf::template st<V>(rOU, poff + toff, odu);
      Buf::template st<V>(rOD, poff + toff, odd);
      if constexpr (GATED) Buf::template st<V>(rOZ, poff + toff, odz);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (t0 + pt + e < t_end) {
          if constexpr (!CONV) Buf::template st<1>(rOU, poff + toff + e * ES, &odu[e]);
          Buf::template st<1>(rOD, poff + toff + e * ES, &odd[e]);
          if constexpr (GATED) Buf::template st<1>(rOZ, poff + toff + e * ES, &odz[e]);
        }
    }
  };

  // ---- dx of the tile at t0 (CONV): dx_t = sum_j w4[j] dpre_{t+3-j}, the
  // dpre of this tile in its parity slot of sDP and of the tile after it in
  // the other (zero after the end of the sequence)
  auto conv_dx = [&](int t0) {
    const float* cur = sDP + ((t0 / kBT) & 1) * kCG * kBR + pc * kBR;
    const float* nxt = sDP + (((t0 / kBT) & 1) ^ 1) * kCG * kBR + pc * kBR;
    float dv[V + 3];
#pragma unroll
    for (int e = 0; e < V + 3; ++e) {
      const int q = pt + e;
      dv[e] = q < kBT ? cur[q] : nxt[q - kBT];
    }
    float dx[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(w4[j], dv[e + 3 - j], acc);
      dx[e] = acc;
    }
    const uint32_t toff = static_cast<uint32_t>(t0) * ES;
    if (VEC && t0 + kBT <= Li) {
      Buf::template st<V>(rOU, poff + toff, dx);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (t0 + pt + e < Li) Buf::template st<1>(rOU, poff + toff + e * ES, &dx[e]);
    }
  };
  if constexpr (CONV) {
    for (int i = tid; i < 2 * kCG * kBR; i += NT) sDP[i] = 0.0f;
  }
  int prev_t0 = -1;

  // ---- chunks from last to first
  const int sc = static_cast<int>(p.sc);
  const int K = (Li + sc - 1) / sc;
  TileRegs R;
  using kPart = std::integral_constant<bool, false>;
  using kFullLoad = std::integral_constant<bool, true>;
  // The first tile of the last chunk is loaded here; the first tile of every
  // earlier chunk (always a whole chunk, so phase 1 runs) during the last tile
  // of the chunk after it, and phase 2's first tile during phase 1's last.
  {
    const int cs = (K - 1) * sc;
    if (Li - cs > kBT)
      load_tile(R, cs, kPart{});
    else
      load_tile(R, cs, kFullLoad{});
  }
#pragma unroll 1
  for (int k = K - 1; k >= 0; --k) {
    const int cs = k * sc;
    const int ce = (sc < Li - cs) ? cs + sc : Li;
    const int nt = (ce - cs + kBT - 1) / kBT;
    // state at the chunk start: h0 (or zero) for the first chunk, else the
    // boundary state the forward kept after step cs - 1
    float h[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t n = static_cast<int64_t>(grp) * S + s;
      float v = 0.0f;
      if (ok[s]) {
        if (k > 0)
          v = a.cst[((b * K + (k - 1)) * dim + d) * N + n];
        else if (a.h0 != nullptr)
          v = a.h0[(b * dim + d) * N + n];
      }
      h[s] = v;
      myCk[s * kCG] = v;
    }
    // phase 1: states at the start of tiles 1 .. nt-1 (all full tiles)
#pragma unroll 1
    for (int i = 0; i + 1 < nt; ++i) {
      prep1(R, cs + i * kBT);
      if (i + 2 < nt)
        load_tile(R, cs + (i + 1) * kBT, kPart{});
      else
        load_tile(R, cs + (nt - 1) * kBT, kFullLoad{});
      __syncthreads();
      recur1(h);
#pragma unroll
      for (int s = 0; s < S; ++s) myCk[((i + 1) * kNS + s) * kCG] = h[s];
      __syncthreads();
    }
    // phase 2: tiles from last to first
#pragma unroll 1
    for (int i = nt - 1; i >= 0; --i) {
      const int t0 = cs + i * kBT;
      prep2(R, t0, ce);
      if (i > 0)
        load_tile(R, t0 - kBT, kFullLoad{});
      else if (k > 0)
        load_tile(R, cs - sc, kPart{});
      __syncthreads();
      if constexpr (CONV) {
        if (prev_t0 >= 0) conv_dx(prev_t0);
      }
      float hst[S];
#pragma unroll
      for (int s = 0; s < S; ++s) hst[s] = myCk[(i * kNS + s) * kCG];
      compute(hst, t0, ce, k == 0 && i == 0);
      __syncthreads();
      epilogue(t0, ce);
      prev_t0 = t0;
    }
  }
  if constexpr (CONV) {
    __syncthreads();
    conv_dx(prev_t0);
  }

  // ---- sums over batch rows and time: one atomic add per lane / thread
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (ok[s]) unsafeAtomicAdd(a.dA + d * N + grp * S + s, dAacc[s] * kLn2);
  if (pvalid) {
    if (a.dD != nullptr) unsafeAtomicAdd(a.dD + pd, dDacc);
    if (a.dbias != nullptr) unsafeAtomicAdd(a.dbias + pd, dbacc);
    if constexpr (CONV) {
      const int Kc = p.convk;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j >= 4 - Kc) unsafeAtomicAdd(a.dconvw + pd * Kc + (j - (4 - Kc)), dcw[j]);
      if (a.dconvb != nullptr) unsafeAtomicAdd(a.dconvb + pd, dcb);
    }
  }
}

// Clears up to kZeroBufs float buffers in one launch: grid row y clears
// buffer y with a grid-stride loop over x.
__global__ __launch_bounds__(256) void ssm_zero_kernel(ZeroList z) {
  float* __restrict__ p = z.p[blockIdx.y];
  const int64_t n = z.n[blockIdx.y];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

size_t bwd_smem_bytes(int S, int64_t state_chunk, bool conv) {
  const int W = 4 / S;
  const int64_t tiles = (state_chunk + kBT - 1) / kBT;
  return sizeof(float) * static_cast<size_t>(3 * kCG * kBR + 2 * kNS * kBT + W * 3 * kCG * kBR +
                                             (conv ? 2 * kCG * (kBR + kXR) : 0) + tiles * kNS * kCG);
}

template <typename IO, int S, bool GATED, bool VEC, bool CONV>
static hipError_t launch_bwd_t(const BwdArgs& h, hipStream_t st) {
  using T = typename IO::T;
  BwdDev<IO> a;
  a.u = static_cast<const T*>(h.u);
  a.dlt = static_cast<const T*>(h.delta);
  a.Bg = static_cast<const T*>(h.B);
  a.Cg = static_cast<const T*>(h.C);
  a.zg = static_cast<const T*>(h.z);
  a.dy = static_cast<const T*>(h.dy);
  a.Ag = h.A;
  a.Dg = h.D;
  a.biasg = h.bias;
  a.h0 = h.h0;
  a.cst = h.chunk_states;
  a.dlast = h.dlast;
  a.du = static_cast<T*>(h.du);
  a.ddelta = static_cast<T*>(h.ddelta);
  a.dz = static_cast<T*>(h.dz);
  a.dA = h.dA;
  a.dB = h.dB;
  a.dC = h.dC;
  a.dD = h.dD;
  a.dbias = h.dbias;
  a.dh0 = h.dh0;
  a.convw = h.conv_w;
  a.convb = h.conv_b;
  a.dconvw = h.dconv_w;
  a.dconvb = h.dconv_b;
  const BwdSz p{h.batch, h.dim, h.dstate, h.L, h.state_chunk, h.softplus, h.conv_w ? h.conv_k : 0};
  const dim3 grid(static_cast<unsigned>((h.dim + kCG - 1) / kCG), static_cast<unsigned>(h.batch));
  hipLaunchKernelGGL((ssm_bwd_kernel<IO, S, GATED, VEC, CONV>), grid, dim3(256 / S),
                     bwd_smem_bytes(S, h.state_chunk, CONV), st, a, p);
  return hipGetLastError();
}

template <typename IO, int S, bool CONV>
static hipError_t launch_bwd_c(const BwdArgs& h, hipStream_t st) {
  const bool vec = h.L % 8 == 0;
  if (h.z != nullptr)
    return vec ? launch_bwd_t<IO, S, true, true, CONV>(h, st) : launch_bwd_t<IO, S, true, false, CONV>(h, st);
  return vec ? launch_bwd_t<IO, S, false, true, CONV>(h, st) : launch_bwd_t<IO, S, false, false, CONV>(h, st);
}

template <typename IO, int S>
static hipError_t launch_bwd_s(const BwdArgs& h, hipStream_t st) {
  return h.conv_w != nullptr ? launch_bwd_c<IO, S, true>(h, st) : launch_bwd_c<IO, S, false>(h, st);
}

hipError_t launch_bwd(const BwdArgs& h, bool bf16, int S, hipStream_t st) {
  if (bf16) {
    if (S == 4) return launch_bwd_s<BF16, 4>(h, st);
    return S == 2 ? launch_bwd_s<BF16, 2>(h, st) : launch_bwd_s<BF16, 1>(h, st);
  }
  if (S == 4) return launch_bwd_s<F32, 4>(h, st);
  return S == 2 ? launch_bwd_s<F32, 2>(h, st) : launch_bwd_s<F32, 1>(h, st);
}

hipError_t launch_zero(const ZeroList& z, hipStream_t st) {
  if (z.count <= 0) return hipSuccess;
  if (z.count > kZeroBufs) return hipErrorInvalidValue;
  int64_t most = 0;
  for (int i = 0; i < z.count; ++i) most = z.n[i] > most ? z.n[i] : most;
  int64_t blocks = (most + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ssm_zero_kernel, dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(z.count)), dim3(256),
                     0, st, z);
  return hipGetLastError();
}

}  // namespace ssm

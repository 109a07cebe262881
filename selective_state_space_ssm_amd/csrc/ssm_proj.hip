// Output projection after the gated scan, on the matrix cores of gfx950:
//
//   out[b, t, m] = sum_k W[m, k] * y[b, k, t]
//
// ([Mamba-2 page] §4.1 lists this Linear last in the fused chain: Conv1D,
// SSM, SiLU gate, Linear.)  Unlike the scan it is a dense contraction over
// d_inner, so it runs as MFMA tiles with float32 accumulation.
//
// Layout.  y is [b][d_inner][L] as the scan writes it (L contiguous), W is
// [d_model][d_inner] (d_inner contiguous), out is [b][L][d_model] (token
// major, the layout of the residual stream).  y is read in place: no
// transposed copy is made in HBM.
//
// Tiling.  A workgroup of 256 threads (4 wavefronts in a 2 x 2 grid) owns a
// BM (d_model) x BN (token) tile of one batch row and walks d_inner in steps
// of BK values (128 bytes: 64 bfloat16 or 32 float32).  Each step stages the
// W slice [BM][BK] and the y slice [BK][BN] into LDS, the y slice transposed
// to [token][k] on the way in (an E x E register transpose per thread, E =
// values per 16 bytes), so that both MFMA operands read E consecutive k of
// one row with one 128-bit LDS read.  Each wavefront owns (BM/2) x (BN/2):
// a TI x TJ grid of 16 x 16 MFMA tiles.  Two LDS buffers: the next step's
// global loads are issued before this step's MFMAs and written to the other
// buffer after them, with one barrier per step.
//
//   bfloat16: v_mfma_f32_16x16x32_bf16, BM = BN = 256 (TI = TJ = 8, 256
//             accumulators per lane, one workgroup per CU, 128 KB of LDS)
//   float32:  v_mfma_f32_16x16x4_f32,   BM = BN = 128 (TI = TJ = 4), the k
//             order inside a 16-value step permuted identically for both
//             operands so that each lane reads 4 consecutive k at once
//
// LDS rows are 128 bytes (8 chunks of 16 bytes) without padding; chunk c of
// row r sits at position c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7.  The MFMA
// operand reads (16 consecutive rows, one chunk) and the transposing y writes
// (rows E apart, one chunk) then both spread every 8 lanes over the 8 chunk
// positions, i.e. over all banks.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order is
// remapped so that each XCD takes a contiguous range of tiles, d_model tiles
// fastest: the workgroups that share a y slice share one L2.
//
// Bounds.  Global accesses go through buffer resources (one per batch row
// for y and out): an out-of-range offset reads zero and drops a write.  Rows
// or columns past the edge of the problem get such an offset, so partial
// tiles load zeros (contributing nothing to the sums) and store nothing.
//
// Pages cited:
//   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
//                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
#include <hip/hip_runtime.h>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource (sizes are < 2^31)

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <typename IO>
struct ProjCfg;
template <>
struct ProjCfg<F32> {
  static constexpr int E = 4;     // values per 16-byte chunk
  static constexpr int TI = 4;    // 16 x 16 tiles per wavefront along d_model
  static constexpr int TJ = 4;    // ... along tokens
  static constexpr int ES = 4;    // bytes per value
};
template <>
struct ProjCfg<BF16> {
  static constexpr int E = 8;
  static constexpr int TI = 8;
  static constexpr int TJ = 8;
  static constexpr int ES = 2;
};

struct ProjDev {
  const char* y;
  const char* w;
  char* out;
  int64_t batch, K, M, L;   // K = d_inner, M = d_model
};

template <typename IO>
constexpr int proj_bm() { return 32 * ProjCfg<IO>::TI; }
template <typename IO>
constexpr int proj_bn() { return 32 * ProjCfg<IO>::TJ; }
template <typename IO>
constexpr size_t proj_lds_bytes() { return size_t(2) * (proj_bm<IO>() + proj_bn<IO>()) * 128; }

// 8 bfloat16 values -> MFMA operand
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

template <typename IO, bool VEC>
__global__ void __launch_bounds__(kPThreads, 1) ssm_out_proj_kernel(ProjDev p) {
  using C = ProjCfg<IO>;
  constexpr int E = C::E, TI = C::TI, TJ = C::TJ, ES = C::ES;
  constexpr int BM = proj_bm<IO>(), BN = proj_bn<IO>(), BK = 8 * E;
  constexpr int NW = BM / 32;                   // W chunks per thread per step
  static_assert(BN / E == 32, "one E x E block of y per thread per step");

  extern __shared__ uint4 lds[];                // [2][BM + BN][8] chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- tile of this workgroup (XCD-contiguous order, d_model tiles fastest)
  const int64_t nm = (p.M + BM - 1) / BM, nl = (p.L + BN - 1) / BN;
  const int64_t G = static_cast<int64_t>(gridDim.x);
  const int64_t pid = blockIdx.x, q = G / 8, r = G % 8, xcd = pid % 8, slot = pid / 8;
  const int64_t logical = xcd * q + (xcd < r ? xcd : r) + slot;
  const int64_t mt = logical % nm, rest = logical / nm;
  const int64_t lt = rest % nl, b = rest / nl;
  const int64_t m0 = mt * BM, l0 = lt * BN;

  const uint32_t ybytes = static_cast<uint32_t>(p.K * p.L * ES);
  const Rsrc ry = make_rsrc(p.y + b * p.K * p.L * ES, ybytes);
  const Rsrc rw = make_rsrc(p.w, static_cast<uint32_t>(p.M * p.K * ES));
  const Rsrc ro = make_rsrc(p.out + b * p.L * p.M * ES, static_cast<uint32_t>(p.L * p.M * ES));

  // ---- per-thread load roles
  // W: chunk c of rows (tid >> 3) + 32 i;  y: k-group kg (E rows), token group tg (E tokens)
  const int wc = tid & 7, wr0 = tid >> 3;
  const int tg = tid & 31, kg = tid >> 5;
  const int64_t ytok = l0 + tg * E;

  uint4 wreg[NW];
  uint4 yreg[E];

  // 32-bit byte offsets: a per-thread base plus uniform steps.  Every valid
  // offset is below 2^31; invalid ones are replaced by kOOB before use.
  const uint32_t wstride = static_cast<uint32_t>(p.K * ES);          // bytes per W row
  const uint32_t ystride = static_cast<uint32_t>(p.L * ES);          // bytes per y row
  const int64_t wm0 = m0 + wr0;
  const uint32_t wbase = static_cast<uint32_t>(wm0 * wstride + wc * E * ES);
  const uint32_t ybase = static_cast<uint32_t>(kg * E * static_cast<int64_t>(ystride) + ytok * ES);
  const int wrows_ok = wm0 >= p.M ? 0 : static_cast<int>((p.M - wm0 + 31) / 32);   // valid i < this

  auto load_w_chunk = [&](int i, int64_t k0) -> uint4 {
    const int64_t k = k0 + wc * E;
    const uint32_t off = wbase + static_cast<uint32_t>(i * 32) * wstride + static_cast<uint32_t>(k0 * ES);
    if constexpr (VEC) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, (i < wrows_ok && k < p.K) ? off : kOOB, 0, 0);
      return make_uint4(v.x, v.y, v.z, v.w);
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t oe = (i < wrows_ok && k + e < p.K) ? off + e * ES : kOOB;
        if constexpr (ES == 4) {
          w[e] = __builtin_amdgcn_raw_buffer_load_b32(rw, oe, 0, 0);
        } else {
          const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(rw, oe, 0, 0);
          w[e >> 1] |= (e & 1) ? (h << 16) : h;
        }
      }
      return make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto load_y_row = [&](int rr, int64_t k0) -> uint4 {
    const int64_t k = k0 + kg * E + rr;
    const uint32_t off = ybase + static_cast<uint32_t>(rr) * ystride + static_cast<uint32_t>(k0 * ystride);
    if constexpr (VEC) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ry, (k < p.K && ytok < p.L) ? off : kOOB, 0, 0);
      return make_uint4(v.x, v.y, v.z, v.w);
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t oe = (k < p.K && ytok + e < p.L) ? off + e * ES : kOOB;
        if constexpr (ES == 4) {
          w[e] = __builtin_amdgcn_raw_buffer_load_b32(ry, oe, 0, 0);
        } else {
          const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(ry, oe, 0, 0);
          w[e >> 1] |= (e & 1) ? (h << 16) : h;
        }
      }
      return make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto load_global = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NW; ++i) wreg[i] = load_w_chunk(i, k0);
#pragma unroll
    for (int rr = 0; rr < E; ++rr) yreg[rr] = load_y_row(rr, k0);
  };
  // registers -> LDS buffer `buf`: W rows as they are, y as [token][k]
  auto store_lds = [&](int buf) {
    uint4* sw = lds + buf * (BM + BN) * 8;
    uint4* sy = sw + BM * 8;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int row = wr0 + 32 * i;
      sw[row * 8 + (wc ^ swz(row))] = wreg[i];
    }
    if constexpr (ES == 2) {
      // 8 k-rows of 8 tokens -> 8 tokens of 8 k (k pairs packed low, high)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pw = j >> 1;
        uint32_t o[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const uint32_t lo = reinterpret_cast<const uint32_t*>(&yreg[2 * qd])[pw];
          const uint32_t hi = reinterpret_cast<const uint32_t*>(&yreg[2 * qd + 1])[pw];
          o[qd] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int row = tg * 8 + j;
        sy[row * 8 + (kg ^ swz(row))] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
      // 4 k-rows of 4 tokens -> 4 tokens of 4 k
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = tg * 4 + j;
        const uint4 v = make_uint4(reinterpret_cast<const uint32_t*>(&yreg[0])[j],
                                   reinterpret_cast<const uint32_t*>(&yreg[1])[j],
                                   reinterpret_cast<const uint32_t*>(&yreg[2])[j],
                                   reinterpret_cast<const uint32_t*>(&yreg[3])[j]);
        sy[row * 8 + (kg ^ swz(row))] = v;
      }
    }
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA operand reads.  Lane reads row (lane & 15) + 16 i of its wavefront's
  // half at chunk 4 s + (lane >> 4).  With the swizzle above the chunk
  // position of (step s, subtile i) is qpos ^ 4 s ^ 2 (i & 3), qpos a lane
  // constant, so four per-lane byte offsets serve every read and the 16-row
  // steps are immediate offsets.
  const int lgrp = lane >> 4;
  int loff[4];
  {
    const int qpos = lgrp ^ (lane & 7) ^ ((lane >> 3) & 1);
#pragma unroll
    for (int x = 0; x < 4; ++x) loff[x] = (lane & 15) * 128 + 16 * (qpos ^ (2 * x));
  }
  // both k-steps' fragments are read first (the reads overlap each other and
  // the first MFMAs wait only for their own operands), then 2 x TI x TJ MFMAs
  auto compute = [&](int buf) {
    const char* abase = reinterpret_cast<const char*>(lds + buf * (BM + BN) * 8) + wm * (BM / 2) * 128;
    const char* bbase = reinterpret_cast<const char*>(lds + buf * (BM + BN) * 8) + BM * 128 + wn * (BN / 2) * 128;
    uint4 fa[2][TI], fb[2][TJ];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
        fa[s][i] = *reinterpret_cast<const uint4*>(abase + loff[((4 * s) ^ (2 * (i & 3))) >> 1] + 2048 * i);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        fb[s][j] = *reinterpret_cast<const uint4*>(bbase + loff[((4 * s) ^ (2 * (j & 3))) >> 1] + 2048 * j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (ES == 2) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(fa[s][i]), as_bf16x8(fb[s][j]), acc[i][j],
                                                                0, 0, 0);
      } else {
        // the 16 k of a step: lane group g holds k = 4 g + e of its chunk;
        // MFMA e takes element e of both operands (the same k on both sides)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __uint_as_float(reinterpret_cast<const uint32_t*>(&fa[s][i])[e]),
                  __uint_as_float(reinterpret_cast<const uint32_t*>(&fb[s][j])[e]), acc[i][j], 0, 0, 0);
      }
    }
  };

  const int64_t nk = (p.K + BK - 1) / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int64_t it = 0; it < nk; ++it) {
    const bool more = it + 1 < nk;
    if (more) load_global((it + 1) * BK);
    compute(static_cast<int>(it & 1));
    if (more) store_lds(static_cast<int>((it + 1) & 1));
    __syncthreads();
  }

  // ---- epilogue: lane holds d_model rows 4*lgrp + v of column (lane & 15)
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * i + 4 * lgrp;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t t = l0 + wn * (BN / 2) + 16 * j + (lane & 15);
      const f32x4 v = acc[i][j];
      if constexpr (VEC) {
        const uint32_t off = (t < p.L && m < p.M) ? static_cast<uint32_t>(t * p.M + m) * ES : kOOB;
        if constexpr (ES == 4) {
          u32x4 w;
          w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
          w.z = __float_as_uint(v[2]); w.w = __float_as_uint(v[3]);
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
        } else {
          u32x2 w;
          w.x = BF16::cvt(v[0]) | (BF16::cvt(v[1]) << 16);
          w.y = BF16::cvt(v[2]) | (BF16::cvt(v[3]) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (t < p.L && m + e < p.M) ? static_cast<uint32_t>(t * p.M + m + e) * ES : kOOB;
          if constexpr (ES == 4)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), ro, off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(BF16::cvt(v[e])), ro, off, 0, 0);
        }
      }
    }
  }
}

template <typename IO, bool VEC>
hipError_t launch_proj_t(const ProjArgs& h, hipStream_t st) {
  constexpr int BM = proj_bm<IO>(), BN = proj_bn<IO>();
  ProjDev p{static_cast<const char*>(h.y), static_cast<const char*>(h.w), static_cast<char*>(h.out), h.batch,
            h.d_inner, h.d_model, h.L};
  const int64_t tiles = ((h.d_model + BM - 1) / BM) * ((h.L + BN - 1) / BN) * h.batch;
  const size_t smem = proj_lds_bytes<IO>();
  auto kern = ssm_out_proj_kernel<IO, VEC>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(kPThreads), smem, st, p);
  return hipGetLastError();
}

}  // namespace

int64_t proj_tiles(bool bf16, int64_t batch, int64_t d_model, int64_t L) {
  const int64_t bm = bf16 ? proj_bm<BF16>() : proj_bm<F32>();
  const int64_t bn = bf16 ? proj_bn<BF16>() : proj_bn<F32>();
  return ((d_model + bm - 1) / bm) * ((L + bn - 1) / bn) * batch;
}

hipError_t launch_out_proj(const ProjArgs& h, bool bf16, hipStream_t st) {
  const int64_t E = bf16 ? 8 : 4;
  const bool vec = h.d_inner % E == 0 && h.L % E == 0 && h.d_model % 4 == 0;
  if (bf16) return vec ? launch_proj_t<BF16, true>(h, st) : launch_proj_t<BF16, false>(h, st);
  return vec ? launch_proj_t<F32, true>(h, st) : launch_proj_t<F32, false>(h, st);
}

}  // namespace ssm

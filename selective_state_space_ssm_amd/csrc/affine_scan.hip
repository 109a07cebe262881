// Bare inclusive scan of affine pairs on gfx950 ([Scan page] "Hardware-aware
// parallel associative scan for Mamba" (pwwt.cn/news/6375169), §1.2 monoid,
// §2.1 scans, §2.2 chunking, §3.2-§3.3 in-block scan and chunk carry).
//
// A pair (a, b) is h -> a*h + b; (a2,b2) o (a1,b1) = (a2*a1, fma(a2, b1, b2)).
// One block (4 wavefronts) scans one row, chunk by chunk (chunk = 64*4*8
// steps), carrying the composed prefix from chunk to chunk.  Inside a chunk:
//   1. thread-serial: every lane folds its 8 consecutive items in registers;
//   2. wave64 scan of the 64 lane totals with DPP: row_shr 1, 2, 4, 8 inside
//      each row of 16 lanes, then row_bcast:15 and row_bcast:31 across rows
//      (lanes without a partner compose with the identity (1, 0), which the
//      DPP "old" operand supplies);
//   3. exclusive lane prefix by wave_shr:1;
//   4. the 4 wave totals meet in LDS; each wave folds the carry with the
//      totals of the waves before it, in order;
//   5. each lane re-folds its items from its start state and writes every
//      prefix, coalesced (8 consecutive floats per lane).
// The order is fixed and documented in the public header so that results
// are reproducible bit for bit and can be replayed on the CPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_kernels.h"

namespace ssm {
namespace {

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROWMASK, 0xf, false));
}

// (P, H) <- (P, H) o (partner), partner = identity where DPP gives none.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void hs_round(float& P, float& H) {
  const float tp = dpp<CTRL, ROWMASK>(1.0f, P);
  const float th = dpp<CTRL, ROWMASK>(0.0f, H);
  H = __builtin_fmaf(P, th, H);
  P = P * tp;
}

constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

}  // namespace

__global__ __launch_bounds__(kAffLanes * kAffW) void affine_scan_kernel(const float* a,
                                                                         const float* b,
                                                                         float* oa, float* ob, int64_t rows,
                                                                         int64_t L, int vec) {
  __shared__ float sP[kAffW], sH[kAffW];
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* ar = a + r * L;
    const float* br = b + r * L;
    float* oar = oa ? oa + r * L : nullptr;
    float* obr = ob + r * L;
    float cP = 1.0f, cH = 0.0f;
    for (int64_t base = 0; base < L; base += kAffChunk) {
      const int64_t i0 = base + static_cast<int64_t>(w * kAffLanes + l) * kAffT;
      float av[kAffT], bv[kAffT];
      if (vec && i0 + kAffT <= L) {
#pragma unroll
        for (int q = 0; q < kAffT / 4; ++q) {
          const float4 x = *reinterpret_cast<const float4*>(ar + i0 + 4 * q);
          const float4 y = *reinterpret_cast<const float4*>(br + i0 + 4 * q);
          av[4 * q] = x.x; av[4 * q + 1] = x.y; av[4 * q + 2] = x.z; av[4 * q + 3] = x.w;
          bv[4 * q] = y.x; bv[4 * q + 1] = y.y; bv[4 * q + 2] = y.z; bv[4 * q + 3] = y.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kAffT; ++j) {
          const bool in = i0 + j < L;
          av[j] = in ? ar[i0 + j] : 1.0f;
          bv[j] = in ? br[i0 + j] : 0.0f;
        }
      }
      // 1. thread-serial fold from the first item
      float P = av[0], H = bv[0];
#pragma unroll
      for (int j = 1; j < kAffT; ++j) {
        H = __builtin_fmaf(av[j], H, bv[j]);
        P = av[j] * P;
      }
      // 2. wave64 inclusive scan of lane totals
      hs_round<kRowShr1, 0xf>(P, H);
      hs_round<kRowShr2, 0xf>(P, H);
      hs_round<kRowShr4, 0xf>(P, H);
      hs_round<kRowShr8, 0xf>(P, H);
      hs_round<kRowBcast15, 0xa>(P, H);
      hs_round<kRowBcast31, 0xc>(P, H);
      // 3. exclusive prefix: lane l-1's inclusive value
      const float eP = dpp<kWaveShr1, 0xf>(1.0f, P);
      const float eH = dpp<kWaveShr1, 0xf>(0.0f, H);
      // 4. cross-wave combine through LDS
      if (l == kAffLanes - 1) {
        sP[w] = P;
        sH[w] = H;
      }
      __syncthreads();
      float aP = cP, aH = cH;
      for (int v = 0; v < w; ++v) {
        const float tp = sP[v], th = sH[v];
        aH = __builtin_fmaf(tp, aH, th);
        aP = tp * aP;
      }
      float stP = eP * aP;
      float stH = __builtin_fmaf(eP, aH, eH);
      if (l == 0) {
        stP = aP;
        stH = aH;
      }
#pragma unroll
      for (int v = 0; v < kAffW; ++v) {
        const float tp = sP[v], th = sH[v];
        cH = __builtin_fmaf(tp, cH, th);
        cP = tp * cP;
      }
      __syncthreads();
      // 5. re-fold from the start state and write every prefix
      float outA[kAffT], outB[kAffT];
#pragma unroll
      for (int j = 0; j < kAffT; ++j) {
        stH = __builtin_fmaf(av[j], stH, bv[j]);
        stP = av[j] * stP;
        outA[j] = stP;
        outB[j] = stH;
      }
      if (vec && i0 + kAffT <= L) {
#pragma unroll
        for (int q = 0; q < kAffT / 4; ++q) {
          *reinterpret_cast<float4*>(obr + i0 + 4 * q) =
              make_float4(outB[4 * q], outB[4 * q + 1], outB[4 * q + 2], outB[4 * q + 3]);
          if (oar)
            *reinterpret_cast<float4*>(oar + i0 + 4 * q) =
                make_float4(outA[4 * q], outA[4 * q + 1], outA[4 * q + 2], outA[4 * q + 3]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kAffT; ++j) {
          if (i0 + j < L) {
            obr[i0 + j] = outB[j];
            if (oar) oar[i0 + j] = outA[j];
          }
        }
      }
    }
  }
}

hipError_t launch_affine_scan(const float* a, const float* b, float* oa, float* ob, int64_t rows, int64_t L,
                              hipStream_t st) {
  const int64_t cap = 1 << 20;
  const unsigned blocks = static_cast<unsigned>(rows < cap ? rows : cap);
  const int vec = (L % 4 == 0) ? 1 : 0;
  hipLaunchKernelGGL(affine_scan_kernel, dim3(blocks), dim3(kAffLanes * kAffW), 0, st, a, b, oa, ob, rows, L,
                     vec);
  return hipGetLastError();
}

}  // namespace ssm

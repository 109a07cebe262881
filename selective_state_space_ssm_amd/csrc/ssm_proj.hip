// Output projection after the gated scan, and its gradients, on the matrix
// cores of gfx950:
//
//   out[b, t, m] = sum_k W[m, k] * y[b, k, t]                     (forward)
//   dy[b, k, t]  = sum_m W[m, k] * dout[b, t, m]                  (grad of y)
//   dW[m, k]     = sum_{b, t} dout[b, t, m] * y[b, k, t]          (grad of W)
//
// ([Mamba-2 page] §4.1 lists this Linear last in the fused chain: Conv1D,
// SSM, SiLU gate, Linear.)  Unlike the scan these are dense contractions, so
// they run as MFMA tiles with float32 accumulation.
//
// One kernel serves all three.  It computes C^T = A B, i.e.
//
//   out[n][m] = sum_k A[m][k] * B[k][n]
//
// with A row-major [M][K] (K contiguous), B row-major [K][N] (N contiguous)
// and out row-major [N][M] (M contiguous), for `batch` independent outputs
// (each operand with its own batch stride, 0 = shared) and, inside one
// output, a sum over `nseg` segments of K (each operand with its own segment
// stride).  With y [b][d_inner][L], W [d_model][d_inner], dout
// [b][L][d_model]:
//
//   forward  A = W,       B = y[b],     M = d_model, N = L,       K = d_inner
//   dy       A = dout[b], B = W,        M = L,       N = d_inner, K = d_model
//   dW       A = y[b],    B = dout[b],  M = d_inner, N = d_model, K = L, the
//            batch rows being the segments summed
//
// so every operand is read in place, in the layout the rest of the block
// keeps it in.
//
// Tiling.  A workgroup of 256 threads (4 wavefronts in a 2 x 2 grid) owns a
// BM (M) x BN (N) tile and walks K in steps of BK values (128 bytes: 64
// bfloat16 or 32 float32).  Each step stages the A slice [BM][BK] and the B
// slice [BK][BN] into LDS, B transposed to [n][k] on the way in (an E x E
// register transpose per thread, E = values per 16 bytes), so that both MFMA
// operands read E consecutive k of one row with one 128-bit LDS read.  Each
// wavefront owns (BM/2) x (BN/2): a TI x TJ grid of 16 x 16 MFMA tiles.  Two
// LDS buffers: the next step's global loads are issued before this step's
// MFMAs and written to the other buffer after them, one barrier per step.
//
//   bfloat16: v_mfma_f32_16x16x32_bf16, BM = BN = 256 (TI = TJ = 8, 256
//             accumulators per lane, one workgroup per CU, 128 KB of LDS)
//   float32:  v_mfma_f32_16x16x4_f32,   BM = BN = 128 (TI = TJ = 4), the k
//             order inside a 16-value step permuted identically for both
//             operands so that each lane reads 4 consecutive k at once
//
// bfloat16 with every size a multiple of 8 (the block's shapes) takes a
// second kernel, ssm_proj_dma_kernel, with the same tiles and results bit
// for bit, whose staging costs no registers: both operands go from HBM
// straight into LDS (16-byte buffer loads with the LDS as destination), four
// 32-k stages deep, and B stays in its own [k][n] layout in LDS.  The B
// fragments are read with gfx950's transposing LDS read (ds_read_b64_tr_b16):
// lane s of each 16-lane group reads 4 consecutive n of k-row s / 4, and the
// read hands lane i the 4 k values of column i.  Each step reads the next
// step's fragments before its own MFMAs.
//
// When the output tiles alone would leave CUs idle (dW: d_model x d_inner
// tiles only), the segments are split over `nsplit` workgroups per tile;
// each writes a float32 partial and a second kernel sums the partials in a
// fixed order (the result is the same from run to run).
//
// LDS rows are 128 bytes (8 chunks of 16 bytes) without padding; chunk c of
// row r sits at position c ^ swz(r), swz(r) = (r ^ (r >> 3)) & 7.  The MFMA
// operand reads (16 consecutive rows, one chunk) and the transposing B
// writes (rows E apart, one chunk) then both spread every 8 lanes over the 8
// chunk positions.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the tile order is
// remapped so that each XCD takes a contiguous range of tiles, M tiles
// fastest: the workgroups that share a B slice share one L2.
//
// Bounds.  Global accesses go through buffer resources (one per operand,
// batch and segment): an out-of-range offset reads zero and drops a write.
// Rows or columns past the edge of the problem get such an offset, so
// partial tiles load zeros (contributing nothing to the sums) and store
// nothing.
//
// Pages cited:
//   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
//                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ssm_device.h"
#include "ssm_kernels.h"

namespace ssm {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;    // an offset past every resource (sizes are < 2^31)
constexpr int64_t kFillWorkgroups = 512;  // split the segments until about this many workgroups

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <typename IO>
struct ProjCfg;
template <>
struct ProjCfg<F32> {
  static constexpr int E = 4;     // values per 16-byte chunk
  static constexpr int TI = 4;    // 16 x 16 tiles per wavefront along M
  static constexpr int TJ = 4;    // ... along N
  static constexpr int ES = 4;    // bytes per value
};
template <>
struct ProjCfg<BF16> {
  static constexpr int E = 8;
  static constexpr int TI = 8;
  static constexpr int TJ = 8;
  static constexpr int ES = 2;
};

// One launch: out[bt][n][m] = sum over segments s and k of
// A[bt][s][m][k] * B[bt][s][k][n].  Strides in elements.
struct GemmDev {
  const char* a;
  const char* b;
  char* out;        // IO-typed output, or (PART) float32 partials [batch][nsplit][N][M]
  int64_t M, N, K;
  int64_t lda, ldb, ldo;
  int64_t a_batch, b_batch, o_batch;
  int64_t a_seg, b_seg;
  int64_t nseg, spp;    // segments, segments per split
  int64_t nsplit, batch;
};

template <typename IO>
constexpr int proj_bm() { return 32 * ProjCfg<IO>::TI; }
template <typename IO>
constexpr int proj_bn() { return 32 * ProjCfg<IO>::TJ; }
template <typename IO>
constexpr size_t proj_lds_bytes() { return size_t(2) * (proj_bm<IO>() + proj_bn<IO>()) * 128; }

// 8 bfloat16 values -> MFMA operand
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

template <typename IO, bool VEC, bool PART>
__global__ void __launch_bounds__(kPThreads, 1) ssm_proj_gemm_kernel(GemmDev p) {
  using C = ProjCfg<IO>;
  constexpr int E = C::E, TI = C::TI, TJ = C::TJ, ES = C::ES;
  constexpr int BM = proj_bm<IO>(), BN = proj_bn<IO>(), BK = 8 * E;
  constexpr int NW = BM / 32;                   // A chunks per thread per step
  static_assert(BN / E == 32, "one E x E block of B per thread per step");

  extern __shared__ uint4 lds[];                // [2][BM + BN][8] chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- tile of this workgroup (XCD-contiguous order, M tiles fastest)
  const int64_t nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
  const int64_t G = static_cast<int64_t>(gridDim.x);
  const int64_t pid = blockIdx.x, q = G / 8, r = G % 8, xcd = pid % 8, slot = pid / 8;
  const int64_t logical = xcd * q + (xcd < r ? xcd : r) + slot;
  const int64_t mt = logical % nm;
  int64_t rest = logical / nm;
  const int64_t nt = rest % nn;
  rest /= nn;
  const int64_t split = rest % p.nsplit, bt = rest / p.nsplit;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t seg0 = split * p.spp;
  const int64_t seg1 = (seg0 + p.spp < p.nseg) ? seg0 + p.spp : p.nseg;

  // ---- per-thread load roles
  // A: chunk c of rows (tid >> 3) + 32 i;  B: k-group kg (E rows), n group tg (E columns)
  const int wc = tid & 7, wr0 = tid >> 3;
  const int tg = tid & 31, kg = tid >> 5;
  const int64_t bcol = n0 + tg * E;

  uint4 areg[NW];
  uint4 breg[E];

  // 32-bit byte offsets: a per-thread base plus uniform steps.  Every valid
  // offset is below 2^31; invalid ones are replaced by kOOB before use.
  const uint32_t astride = static_cast<uint32_t>(p.lda * ES);        // bytes per A row
  const uint32_t bstride = static_cast<uint32_t>(p.ldb * ES);        // bytes per B row
  const int64_t am0 = m0 + wr0;
  const uint32_t abase = static_cast<uint32_t>(am0 * astride + wc * E * ES);
  const uint32_t bbase = static_cast<uint32_t>(kg * E * static_cast<int64_t>(bstride) + bcol * ES);
  const int arows_ok = am0 >= p.M ? 0 : static_cast<int>((p.M - am0 + 31) / 32);   // valid i < this
  const bool bcol_ok = bcol < p.N;
  const uint32_t abytes = static_cast<uint32_t>(p.M * p.lda * ES);
  const uint32_t bbytes = static_cast<uint32_t>(p.K * p.ldb * ES);

  auto krem_of = [&](int64_t k0) -> int {   // values of K left from k0, clamped to [-1, BK]
    const int64_t rr = p.K - k0;
    return rr < 0 ? -1 : (rr > BK ? BK : static_cast<int>(rr));
  };
  // The steps of this workgroup walk K in BK steps within a segment, then
  // the next segment; (cur_seg, cur_k0) is the next step to load, advanced
  // by one step per load (no 64-bit division in the loop).
  const int64_t ksteps = (p.K + BK - 1) / BK;
  const int64_t nsteps = (seg1 - seg0) * ksteps;
  int64_t cur_seg = seg0, cur_k0 = 0;
  auto load_global = [&]() {
    const int64_t seg = cur_seg;
    const int64_t k0 = cur_k0;
    cur_k0 += BK;
    if (cur_k0 >= ksteps * BK) {
      cur_k0 = 0;
      ++cur_seg;
    }
    const Rsrc ra = make_rsrc(p.a + (bt * p.a_batch + seg * p.a_seg) * ES, abytes);
    const Rsrc rb = make_rsrc(p.b + (bt * p.b_batch + seg * p.b_seg) * ES, bbytes);
    const int krem = krem_of(k0);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t off = abase + static_cast<uint32_t>(i * 32) * astride + static_cast<uint32_t>(k0 * ES);
      if constexpr (VEC) {
        const bool ok = (i < arows_ok) & (wc * E < krem);
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? off : kOOB, 0, 0);
        areg[i] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool ok = (i < arows_ok) & (wc * E + e < krem);
          const uint32_t oe = ok ? off + e * ES : kOOB;
          if constexpr (ES == 4) {
            w[e] = __builtin_amdgcn_raw_buffer_load_b32(ra, oe, 0, 0);
          } else {
            const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(ra, oe, 0, 0);
            w[e >> 1] |= (e & 1) ? (h << 16) : h;
          }
        }
        areg[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < E; ++rr) {
      const uint32_t off = bbase + static_cast<uint32_t>(rr) * bstride + static_cast<uint32_t>(k0 * p.ldb * ES);
      if constexpr (VEC) {
        const bool ok = (kg * E + rr < krem) & bcol_ok;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rb, ok ? off : kOOB, 0, 0);
        breg[rr] = make_uint4(v.x, v.y, v.z, v.w);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool ok = (kg * E + rr < krem) & (bcol + e < p.N);
          const uint32_t oe = ok ? off + e * ES : kOOB;
          if constexpr (ES == 4) {
            w[e] = __builtin_amdgcn_raw_buffer_load_b32(rb, oe, 0, 0);
          } else {
            const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(rb, oe, 0, 0);
            w[e >> 1] |= (e & 1) ? (h << 16) : h;
          }
        }
        breg[rr] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };
  // registers -> LDS buffer `buf`: A rows as they are, B as [n][k]
  auto store_lds = [&](int buf) {
    uint4* sa = lds + buf * (BM + BN) * 8;
    uint4* sb = sa + BM * 8;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int row = wr0 + 32 * i;
      sa[row * 8 + (wc ^ swz(row))] = areg[i];
    }
    if constexpr (ES == 2) {
      // 8 k-rows of 8 columns -> 8 columns of 8 k (k pairs packed low, high)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pw = j >> 1;
        uint32_t o[4];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const uint32_t lo = reinterpret_cast<const uint32_t*>(&breg[2 * qd])[pw];
          const uint32_t hi = reinterpret_cast<const uint32_t*>(&breg[2 * qd + 1])[pw];
          o[qd] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int row = tg * 8 + j;
        sb[row * 8 + (kg ^ swz(row))] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
      // 4 k-rows of 4 columns -> 4 columns of 4 k
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = tg * 4 + j;
        const uint4 v = make_uint4(reinterpret_cast<const uint32_t*>(&breg[0])[j],
                                   reinterpret_cast<const uint32_t*>(&breg[1])[j],
                                   reinterpret_cast<const uint32_t*>(&breg[2])[j],
                                   reinterpret_cast<const uint32_t*>(&breg[3])[j]);
        sb[row * 8 + (kg ^ swz(row))] = v;
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
    const char* fa_base = reinterpret_cast<const char*>(lds + buf * (BM + BN) * 8) + wm * (BM / 2) * 128;
    const char* fb_base = reinterpret_cast<const char*>(lds + buf * (BM + BN) * 8) + BM * 128 + wn * (BN / 2) * 128;
    uint4 fa[2][TI], fb[2][TJ];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
        fa[s][i] = *reinterpret_cast<const uint4*>(fa_base + loff[((4 * s) ^ (2 * (i & 3))) >> 1] + 2048 * i);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        fb[s][j] = *reinterpret_cast<const uint4*>(fb_base + loff[((4 * s) ^ (2 * (j & 3))) >> 1] + 2048 * j);
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

  if (nsteps > 0) {
    load_global();
    store_lds(0);
  }
  __syncthreads();
  for (int64_t s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) load_global();
    compute(static_cast<int>(s & 1));
    if (more) store_lds(static_cast<int>((s + 1) & 1));
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*lgrp + v (M) of column (lane & 15) (N)
  const Rsrc ro = PART ? make_rsrc(p.out + ((bt * p.nsplit + split) * p.N * p.M) * 4,
                                   static_cast<uint32_t>(p.N * p.M * 4))
                       : make_rsrc(p.out + bt * p.o_batch * ES, static_cast<uint32_t>(p.N * p.ldo * ES));
  const int64_t ldo = PART ? p.M : p.ldo;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * i + 4 * lgrp;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
      const f32x4 v = acc[i][j];
      if constexpr (PART) {
        // float32 partial, dense [N][M]; M % 4 == 0 on this path
        const uint32_t off = (n < p.N && m < p.M) ? static_cast<uint32_t>(n * ldo + m) * 4 : kOOB;
        u32x4 w;
        w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
        w.z = __float_as_uint(v[2]); w.w = __float_as_uint(v[3]);
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
      } else if constexpr (VEC) {
        const uint32_t off = (n < p.N && m < p.M) ? static_cast<uint32_t>(n * ldo + m) * ES : kOOB;
        if constexpr (ES == 4) {
          u32x4 w;
          w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
          w.z = __float_as_uint(v[2]); w.w = __float_as_uint(v[3]);
          __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
        } else {
          u32x2 w;
          w.x = BF16::cvt2(v[0], v[1]);
          w.y = BF16::cvt2(v[2], v[3]);
          __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t off = (n < p.N && m + e < p.M) ? static_cast<uint32_t>(n * ldo + m + e) * ES : kOOB;
          if constexpr (ES == 4)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), ro, off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(BF16::cvt(v[e])), ro, off, 0, 0);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// bfloat16, every size a multiple of 8: the operands DMA'd into LDS.
//
// Stage layout (32 KB): A [256 m][32 k] in 64-byte rows whose 16-byte chunk
// c sits at position c ^ ((m >> 1) & 3); B [32 k][256 n] in 512-byte rows
// whose chunk c sits at c ^ swz_kn(k).  With 32 banks of 4 bytes, both keep
// the fragment reads free of bank conflicts (counted: zero): any 8
// consecutive lanes of an A read (one chunk of 8 consecutive rows) and any
// 16 consecutive lanes of a transposing B read (4 k-rows x 32 bytes) cover
// 128 distinct bytes of the bank space.
// A DMA load writes 16 bytes per lane at block base + 16 lane, so the
// swizzle is applied by choosing which global chunk each lane fetches.
// --------------------------------------------------------------------------
constexpr int kDmaBK = 32;                       // k per stage
constexpr int kDmaStages = 4;                    // stages in LDS (three in flight)
constexpr int kDmaA = 256 * kDmaBK * 2;          // A bytes per stage
constexpr int kDmaStage = 2 * kDmaA;             // A + B bytes per stage
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz_kn(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

// Buffer descriptor words for dma16: base, stride 0, size in bytes.
__device__ __forceinline__ u32x4 dma_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d.x = static_cast<uint32_t>(a);
  d.y = static_cast<uint32_t>(a >> 32) & 0xffffu;
  d.z = bytes;
  d.w = static_cast<uint32_t>(kRsrcWord3);
  return d;
}

// 16 bytes per lane from the buffer at byte offset voff (past the size:
// zeros) into LDS at lds + 16 * lane.  Written as inline asm so that the
// compiler does not count it: it would otherwise wait for every load in
// flight before the next LDS read, which undoes the pipeline.  The kernel
// waits for these loads itself (vmcnt before the barrier of the step that
// reads the stage, and all of them before the workgroup ends).  M0 holds
// the LDS address; one wait state separates its write from the load that
// reads it.  Nothing else in the kernel uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4& d, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(d)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <bool PART>
__global__ void __launch_bounds__(kPThreads, 1) ssm_proj_dma_kernel(GemmDev p) {
  constexpr int BM = 256, BN = 256, BK = kDmaBK, TI = 8, TJ = 8, ES = 2;
  __shared__ __attribute__((aligned(1024))) char stg[kDmaStages][kDmaStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // ---- tile of this workgroup (as in ssm_proj_gemm_kernel)
  const int64_t nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
  const int64_t G = static_cast<int64_t>(gridDim.x);
  const int64_t pid = blockIdx.x, q8 = G / 8, r8 = G % 8, xcd = pid % 8, slot = pid / 8;
  const int64_t logical = xcd * q8 + (xcd < r8 ? xcd : r8) + slot;
  const int64_t mt = logical % nm;
  int64_t rest = logical / nm;
  const int64_t nt = rest % nn;
  rest /= nn;
  const int64_t split = rest % p.nsplit, bt = rest / p.nsplit;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t seg0 = split * p.spp;
  const int64_t seg1 = (seg0 + p.spp < p.nseg) ? seg0 + p.spp : p.nseg;

  // ---- DMA roles: 1 KB blocks q = wave + 4 i (i < 4) of each operand per
  // stage.  A block q: rows 16 q + lane / 4, position lane & 3.  B block q:
  // k-rows 2 q + lane / 32, position lane & 31.  Offsets at k0 = 0.
  const uint32_t astride = static_cast<uint32_t>(p.lda * ES), bstride = static_cast<uint32_t>(p.ldb * ES);
  uint32_t a_off[4], b_off[4];
  int a_k[4], b_k[4];
  bool a_ok[4], b_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = wave + 4 * i;
    const int ra = 16 * q + (lane >> 2);
    const int ca = (lane & 3) ^ ((ra >> 1) & 3);
    a_ok[i] = m0 + ra < p.M;
    a_k[i] = 8 * ca;
    a_off[i] = static_cast<uint32_t>((m0 + ra) * astride) + static_cast<uint32_t>(8 * ca * ES);
    const int rb = 2 * q + (lane >> 5);
    const int cb = (lane & 31) ^ swz_kn(rb);
    b_ok[i] = n0 + 8 * cb < p.N;
    b_k[i] = rb;
    b_off[i] = static_cast<uint32_t>(rb) * bstride + static_cast<uint32_t>((n0 + 8 * cb) * ES);
  }
  const uint32_t abytes = static_cast<uint32_t>(p.M * p.lda * ES);
  const uint32_t bbytes = static_cast<uint32_t>(p.K * p.ldb * ES);
  const int64_t ksteps = (p.K + BK - 1) / BK;
  const int64_t nsteps = (seg1 - seg0) * ksteps;
  // Per-lane offsets relative to the stage's k0, past the buffer for rows
  // and columns outside the problem.
  uint32_t a_v[4], b_v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_v[i] = a_ok[i] ? a_off[i] : kOOB;
    b_v[i] = b_ok[i] ? b_off[i] : kOOB;
  }
  // The stages are issued in order.  The scalar cursor holds the next
  // stage's k0 and segment, and the byte address of A and B at that k0 with
  // the bytes left from there: the descriptors advance by one stage with
  // scalar adds, so a whole stage needs no per-lane address arithmetic.  A
  // stage past the end is still issued with an empty buffer (every load
  // reads zeros), so that every step issues the same number of loads and
  // one vmcnt value serves every wait.
  int64_t cur_seg = seg0, cur_k0 = 0;
  uint64_t a_addr = reinterpret_cast<uint64_t>(p.a + (bt * p.a_batch + seg0 * p.a_seg) * ES);
  uint64_t b_addr = reinterpret_cast<uint64_t>(p.b + (bt * p.b_batch + seg0 * p.b_seg) * ES);
  uint32_t a_rec = abytes, b_rec = bbytes;
  auto issue = [&](auto KS, bool live) {
    const u32x4 ra = dma_desc(reinterpret_cast<const void*>(a_addr), live ? a_rec : 0u);
    const u32x4 rb = dma_desc(reinterpret_cast<const void*>(b_addr), live ? b_rec : 0u);
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)stg[decltype(KS)::value]));
    const int64_t left = p.K - cur_k0;
    if (!live || left >= BK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = wave + 4 * i;
        dma16(ra, a_v[i], base + q * 1024);
        dma16(rb, b_v[i], base + kDmaA + q * 1024);
      }
    } else {
      // the last stage of a segment with K % 32 != 0: k past K reads zeros
      const int krem = static_cast<int>(left);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = wave + 4 * i;
        dma16(ra, a_k[i] < krem ? a_v[i] : kOOB, base + q * 1024);
        dma16(rb, b_k[i] < krem ? b_v[i] : kOOB, base + kDmaA + q * 1024);
      }
    }
    if (live) {
      cur_k0 += BK;
      a_addr += static_cast<uint64_t>(BK * ES);
      a_rec -= static_cast<uint32_t>(BK * ES);
      b_addr += static_cast<uint64_t>(BK) * bstride;
      b_rec -= static_cast<uint32_t>(BK) * bstride;
      if (cur_k0 >= ksteps * BK) {
        cur_k0 = 0;
        ++cur_seg;
        a_addr = reinterpret_cast<uint64_t>(p.a + (bt * p.a_batch + cur_seg * p.a_seg) * ES);
        b_addr = reinterpret_cast<uint64_t>(p.b + (bt * p.b_batch + cur_seg * p.b_seg) * ES);
        a_rec = abytes;
        b_rec = bbytes;
      }
    }
  };

  // ---- fragments: A lane reads row wm*128 + 16 i + (lane & 15), chunk
  // lane >> 4 (k 8 (lane >> 4) ..); B lane 16 g + s reads k-row 8 g + s / 4
  // (+ 4 for k 8 g + 4 ..) at n = wn*128 + 16 j + 4 (s & 3)
  const int a_lo = (wm * 128 + (lane & 15)) * 64 + 16 * ((lane >> 4) ^ (((lane & 15) >> 1) & 3));
  const int kB = 8 * (lane >> 4) + ((lane & 15) >> 2);
  int b_lo[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
    b_lo[j] = kB * 512 + 16 * (wn * 16 + ((2 * j) ^ swz_kn(kB)) + ((lane >> 1) & 1)) + 8 * (lane & 1);

  struct Frag {
    uint4 a[TI], b[TJ];
  };
  auto read_a = [&](auto KS, Frag& f) {
    const char* sa = stg[decltype(KS)::value];
#pragma unroll
    for (int i = 0; i < TI; ++i) f.a[i] = *reinterpret_cast<const uint4*>(sa + a_lo + 1024 * i);
  };
  auto read_b = [&](auto KS, Frag& f) {
    const char* sb = stg[decltype(KS)::value] + kDmaA;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sb + b_lo[j]));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(sb + b_lo[j] + 4 * 512));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      f.b[j] = make_uint4(l2.x, l2.y, h2.x, h2.y);
    }
  };
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mfma_rows = [&](const Frag& f, auto I0) {   // MFMA rows I0, I0 + 1
#pragma unroll
    for (int i = decltype(I0)::value; i < decltype(I0)::value + 2; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.a[i]), as_bf16x8(f.b[j]), acc[i][j], 0, 0, 0);
  };

  // ---- pipeline.  Step s: wait until stage s + 1 has landed (8 loads per
  // wave per stage, so vmcnt(8) leaves only stage s + 2 in flight) and until
  // this wave's reads issued at step s - 1 are done (lgkmcnt(0)); barrier
  // (no fence: a release fence would wait for every load in flight); then
  // step s's 64 MFMAs in four groups, with the refill of the stage read at
  // step s - 1 (stage s + 3) and the reads of step s + 1's fragments issued
  // between the groups.  (The inline-asm loads keep the compiler from
  // moving the MFMAs across them, so this order is the issue order.)
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  constexpr int kWait16 = 0 | (7 << 4) | (0 << 8) | (1 << 14);   // vmcnt(16) lgkmcnt(0)
  constexpr int kWait8 = 8 | (7 << 4) | (0 << 8);                // vmcnt(8) lgkmcnt(0)
  using R0 = std::integral_constant<int, 0>;
  using R2 = std::integral_constant<int, 2>;
  using R4 = std::integral_constant<int, 4>;
  using R6 = std::integral_constant<int, 6>;
  Frag F0, F1;
  issue(S0{}, 0 < nsteps);
  issue(S1{}, 1 < nsteps);
  issue(S2{}, 2 < nsteps);
  __builtin_amdgcn_s_waitcnt(kWait16);
  asm volatile("s_barrier" ::: "memory");
  read_a(S0{}, F0);
  read_b(S0{}, F0);
  auto step = [&](auto KR, auto KN, Frag& cur, Frag& nxt, int64_t s) {
    __builtin_amdgcn_s_waitcnt(kWait8);
    asm volatile("s_barrier" ::: "memory");
    mfma_rows(cur, R0{});
    issue(KR, s + 3 < nsteps);
    mfma_rows(cur, R2{});
    read_a(KN, nxt);
    mfma_rows(cur, R4{});
    read_b(KN, nxt);
    mfma_rows(cur, R6{});
  };
  for (int64_t s = 0; s < nsteps; s += 4) {
    step(S3{}, S1{}, F0, F1, s);
    if (s + 1 < nsteps) step(S0{}, S2{}, F1, F0, s + 1);
    if (s + 2 < nsteps) step(S1{}, S3{}, F0, F1, s + 2);
    if (s + 3 < nsteps) step(S2{}, S0{}, F1, F0, s + 3);
  }
  // no load into LDS may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: lane holds rows 4*lgrp + v (M) of column (lane & 15) (N)
  const int lgrp = lane >> 4;
  const Rsrc ro = PART ? make_rsrc(p.out + ((bt * p.nsplit + split) * p.N * p.M) * 4,
                                   static_cast<uint32_t>(p.N * p.M * 4))
                       : make_rsrc(p.out + bt * p.o_batch * ES, static_cast<uint32_t>(p.N * p.ldo * ES));
  const int64_t ldo = PART ? p.M : p.ldo;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * i + 4 * lgrp;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
      const f32x4 v = acc[i][j];
      if constexpr (PART) {
        const uint32_t off = (n < p.N && m < p.M) ? static_cast<uint32_t>(n * ldo + m) * 4 : kOOB;
        u32x4 w;
        w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
        w.z = __float_as_uint(v[2]); w.w = __float_as_uint(v[3]);
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
      } else {
        const uint32_t off = (n < p.N && m < p.M) ? static_cast<uint32_t>(n * ldo + m) * ES : kOOB;
        u32x2 w;
        w.x = BF16::cvt2(v[0], v[1]);
        w.y = BF16::cvt2(v[2], v[3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
      }
    }
  }
}

// out[bt][n][m] = sum_{s < nsplit} part[bt][s][n][m], summed in split order;
// four consecutive m per thread (M % 4 == 0 on the split path).
template <typename IO>
__global__ void __launch_bounds__(256) ssm_proj_reduce_kernel(const float* __restrict__ part, char* out, int64_t N,
                                                              int64_t M, int64_t ldo, int64_t o_batch,
                                                              int64_t nsplit, int64_t batch) {
  using T = typename IO::T;
  const int64_t per = N * M / 4;
  const int64_t total = per * batch;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t bt = i / per, e4 = (i % per) * 4;
    const int64_t n = e4 / M, m = e4 % M;
    const float4* src = reinterpret_cast<const float4*>(part + bt * nsplit * N * M + e4);
    float4 s = src[0];
    for (int64_t k = 1; k < nsplit; ++k) {
      const float4 v = src[k * per];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const float o[4] = {s.x, s.y, s.z, s.w};
    IO::template st<4>(reinterpret_cast<T*>(out) + bt * o_batch + n * ldo + m, o);
  }
}

template <typename IO, bool VEC, bool PART>
hipError_t launch_gemm_t(const GemmDev& p, hipStream_t st) {
  constexpr int BM = proj_bm<IO>(), BN = proj_bn<IO>();
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN) * p.nsplit * p.batch;
  if constexpr (VEC && std::is_same<IO, BF16>::value) {
    // every size a multiple of 8, and lda = K and ldb = N in every
    // contraction: each 16-byte chunk a DMA load fetches is whole and aligned
    hipLaunchKernelGGL(ssm_proj_dma_kernel<PART>, dim3(static_cast<unsigned>(tiles)), dim3(kPThreads), 0, st, p);
    return hipGetLastError();
  } else {
    const size_t smem = proj_lds_bytes<IO>();
    auto kern = ssm_proj_gemm_kernel<IO, VEC, PART>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(tiles)), dim3(kPThreads), smem, st, p);
    return hipGetLastError();
  }
}

template <typename IO>
int64_t tiles_of(const GemmDev& p) {
  return ((p.M + proj_bm<IO>() - 1) / proj_bm<IO>()) * ((p.N + proj_bn<IO>() - 1) / proj_bn<IO>()) * p.batch;
}

// Segments per split for a contraction: more than one workgroup per tile
// only when the segments can be split, the tiles alone leave the chip idle,
// and M allows the float32 partials' vector stores.  Returns spp (= nseg:
// no split).
template <typename IO>
int64_t split_spp(const GemmDev& p) {
  if (p.nseg <= 1 || p.M % 4 != 0) return p.nseg;
  const int64_t tiles = tiles_of<IO>(p);
  int64_t want = (kFillWorkgroups + tiles - 1) / tiles;
  if (want > p.nseg) want = p.nseg;
  if (want <= 1) return p.nseg;
  return (p.nseg + want - 1) / want;
}

template <typename IO>
int64_t split_floats_of(const GemmDev& p) {
  const int64_t spp = split_spp<IO>(p);
  if (spp >= p.nseg) return 0;
  return ((p.nseg + spp - 1) / spp) * p.batch * p.N * p.M;
}

// One contraction: split its segments over workgroups (float32 partials in
// `work`, then the fixed-order sum) when that pays and the workspace is
// there; else one workgroup per tile writes out directly.
template <typename IO>
hipError_t run_gemm(GemmDev p, float* work, int64_t work_floats, hipStream_t st) {
  const int64_t E = ProjCfg<IO>::E;
  const bool vec = p.K % E == 0 && p.N % E == 0 && p.M % 4 == 0;
  const int64_t need = split_floats_of<IO>(p);
  if (need == 0 || work == nullptr || need > work_floats) {
    p.spp = p.nseg;
    p.nsplit = 1;
    return vec ? launch_gemm_t<IO, true, false>(p, st) : launch_gemm_t<IO, false, false>(p, st);
  }
  p.spp = split_spp<IO>(p);
  p.nsplit = (p.nseg + p.spp - 1) / p.spp;
  char* out = p.out;
  p.out = reinterpret_cast<char*>(work);
  hipError_t e = vec ? launch_gemm_t<IO, true, true>(p, st) : launch_gemm_t<IO, false, true>(p, st);
  if (e != hipSuccess) return e;
  const int64_t n4 = p.batch * p.N * p.M / 4;
  const int64_t blocks = n4 / 256 + 1 < 4096 ? n4 / 256 + 1 : 4096;
  hipLaunchKernelGGL(ssm_proj_reduce_kernel<IO>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st,
                     static_cast<const float*>(work), out, p.N, p.M, p.ldo, p.o_batch, p.nsplit, p.batch);
  return hipGetLastError();
}

GemmDev forward_desc(const ProjArgs& h) {
  GemmDev p{};
  p.a = static_cast<const char*>(h.w);
  p.b = static_cast<const char*>(h.y);
  p.out = static_cast<char*>(h.out);
  p.M = h.d_model; p.N = h.L; p.K = h.d_inner;
  p.lda = h.d_inner; p.ldb = h.L; p.ldo = h.d_model;
  p.a_batch = 0; p.b_batch = h.d_inner * h.L; p.o_batch = h.L * h.d_model;
  p.a_seg = 0; p.b_seg = 0;
  p.nseg = 1; p.spp = 1; p.nsplit = 1; p.batch = h.batch;
  return p;
}

GemmDev dy_desc(const ProjBwdArgs& h) {
  GemmDev p{};
  p.a = static_cast<const char*>(h.dout);
  p.b = static_cast<const char*>(h.w);
  p.out = static_cast<char*>(h.dy);
  p.M = h.L; p.N = h.d_inner; p.K = h.d_model;
  p.lda = h.d_model; p.ldb = h.d_inner; p.ldo = h.L;
  p.a_batch = h.L * h.d_model; p.b_batch = 0; p.o_batch = h.d_inner * h.L;
  p.a_seg = 0; p.b_seg = 0;
  p.nseg = 1; p.spp = 1; p.nsplit = 1; p.batch = h.batch;
  return p;
}

GemmDev dw_desc(const ProjBwdArgs& h) {
  GemmDev p{};
  p.a = static_cast<const char*>(h.y);
  p.b = static_cast<const char*>(h.dout);
  p.out = static_cast<char*>(h.dw);
  p.M = h.d_inner; p.N = h.d_model; p.K = h.L;
  p.lda = h.L; p.ldb = h.d_model; p.ldo = h.d_inner;
  p.a_batch = 0; p.b_batch = 0; p.o_batch = 0;
  p.a_seg = h.d_inner * h.L; p.b_seg = h.L * h.d_model;
  p.nseg = h.batch; p.spp = h.batch; p.nsplit = 1; p.batch = 1;
  return p;
}

}  // namespace

int64_t proj_tiles(bool bf16, int64_t batch, int64_t d_model, int64_t L) {
  const int64_t bm = bf16 ? proj_bm<BF16>() : proj_bm<F32>();
  const int64_t bn = bf16 ? proj_bn<BF16>() : proj_bn<F32>();
  return ((d_model + bm - 1) / bm) * ((L + bn - 1) / bn) * batch;
}

int64_t proj_bwd_tiles(bool bf16, const ProjBwdArgs& h) {
  const GemmDev a = dy_desc(h), b = dw_desc(h);
  const int64_t ta = bf16 ? tiles_of<BF16>(a) : tiles_of<F32>(a);
  const int64_t tb = (bf16 ? tiles_of<BF16>(b) : tiles_of<F32>(b)) * h.batch;
  return ta > tb ? ta : tb;
}

size_t proj_bwd_workspace_bytes(bool bf16, const ProjBwdArgs& h) {
  if (h.dw == nullptr) return 0;
  const GemmDev p = dw_desc(h);
  return sizeof(float) * static_cast<size_t>(bf16 ? split_floats_of<BF16>(p) : split_floats_of<F32>(p));
}

hipError_t launch_out_proj(const ProjArgs& h, bool bf16, hipStream_t st) {
  const GemmDev p = forward_desc(h);
  return bf16 ? run_gemm<BF16>(p, nullptr, 0, st) : run_gemm<F32>(p, nullptr, 0, st);
}

hipError_t launch_out_proj_bwd(const ProjBwdArgs& h, bool bf16, float* work, size_t work_bytes, hipStream_t st) {
  const int64_t wf = static_cast<int64_t>(work_bytes / sizeof(float));
  if (h.dy != nullptr) {
    const GemmDev p = dy_desc(h);
    const hipError_t e = bf16 ? run_gemm<BF16>(p, nullptr, 0, st) : run_gemm<F32>(p, nullptr, 0, st);
    if (e != hipSuccess) return e;
  }
  if (h.dw != nullptr) {
    const GemmDev p = dw_desc(h);
    const hipError_t e = bf16 ? run_gemm<BF16>(p, work, wf, st) : run_gemm<F32>(p, work, wf, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ssm

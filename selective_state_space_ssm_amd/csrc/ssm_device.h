// Device-side building blocks shared by the selective-scan kernels for
// gfx950: float32 / bfloat16 storage conversions, buffer-resource loads and
// stores, the softplus and SiLU forms used on the path, and the DPP row
// broadcast that feeds one lane's value to its row of 16 lanes as an operand.
//
// Pages cited:
//   [Scan page]    "Hardware-aware parallel associative scan for Mamba"
//                  (http://www.pwwt.cn/news/6375169/)
//   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
//                  optimisation" (scwacadex.pages.dev, blog8_mamba_parallel_scan)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssm {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- storage
// Loads and stores of V consecutive elements (V = 1, 2, 4 or 8) of the
// storage type, converted to / from float32.
struct F32 {
  using T = float;
  template <int V>
  static __device__ __forceinline__ void ld(const float* p, float* o) {
    if constexpr (V == 1) {
      o[0] = *p;
    } else if constexpr (V == 2) {
      const float2 v = *reinterpret_cast<const float2*>(p);
      o[0] = v.x; o[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + i);
        o[i] = v.x; o[i + 1] = v.y; o[i + 2] = v.z; o[i + 3] = v.w;
      }
    }
  }
  template <int V>
  static __device__ __forceinline__ void st(float* p, const float* v) {
    if constexpr (V == 1) {
      *p = v[0];
    } else if constexpr (V == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
#pragma unroll
      for (int i = 0; i < V; i += 4)
        *reinterpret_cast<float4*>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    }
  }
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct BF16 {
  using T = uint16_t;
  static __device__ __forceinline__ uint32_t cvt(float f) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));  // RNE
  }
  // two values rounded to nearest even and packed (lo in bits 0-15): one
  // v_cvt_pk_bf16_f32 on gfx950 instead of two conversions, a shift and an or
  static __device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
    f32x2 v;
    v.x = lo;
    v.y = hi;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
  template <int V>
  static __device__ __forceinline__ void ld(const uint16_t* p, float* o) {
    if constexpr (V == 1) {
      o[0] = __uint_as_float(static_cast<uint32_t>(*p) << 16);
    } else if constexpr (V == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      o[0] = bf_lo(w); o[1] = bf_hi(w);
    } else if constexpr (V == 4) {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
    } else {
      const uint4 w = *reinterpret_cast<const uint4*>(p);
      o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
      o[4] = bf_lo(w.z); o[5] = bf_hi(w.z); o[6] = bf_lo(w.w); o[7] = bf_hi(w.w);
    }
  }
  template <int V>
  static __device__ __forceinline__ void st(uint16_t* p, const float* v) {
    if constexpr (V == 1) {
      *p = static_cast<uint16_t>(cvt(v[0]));
    } else if constexpr (V == 2) {
      *reinterpret_cast<uint32_t*>(p) = cvt2(v[0], v[1]);
    } else if constexpr (V == 4) {
      *reinterpret_cast<uint2*>(p) = make_uint2(cvt2(v[0], v[1]), cvt2(v[2], v[3]));
    } else {
      *reinterpret_cast<uint4*>(p) =
          make_uint4(cvt2(v[0], v[1]), cvt2(v[2], v[3]),
                     cvt2(v[4], v[5]), cvt2(v[6], v[7]));
    }
  }
};

// Buffer-resource access (raw buffer loads and stores).  A resource holds
// a base address and a byte size in SGPRs; every access gives a 32-bit byte
// offset, and a read past the size returns zero while a write past it is
// dropped, so no address is ever clamped or masked in VGPRs.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 family: 32-bit untyped data format

// Cache policy of a buffer access (the AUX argument of ldw / st): kCacheNT
// marks it non-temporal, for data read or written once that other
// workgroups do not share (gfx950's nt bit).
constexpr int kCacheNT = 2;

// Byte offset `back` bytes before offset `off`, saturated at zero (one
// v_sub_u32 with clamp).  For the conv halo: a slot before the start of
// the buffer then reads word 0, whose value the caller discards (the step
// is before 0).  A wrapped offset would not be safe: the compiler may
// merge the halo with the neighbouring loads and address those as the
// wrapped base plus an immediate, and the range check does not wrap, so
// they would read zero.
__device__ __forceinline__ uint32_t halo_offset(uint32_t off, uint32_t back) {
  return __builtin_elementwise_sub_sat(off, back);
}

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

struct BufF32 {
  // raw 32-bit words of V elements, and their conversion to float32
  template <int V>
  static constexpr int kWords = V;
  template <int V, int AUX = 0>
  static __device__ __forceinline__ void ldw(Rsrc r, uint32_t off, uint32_t* w) {
    if constexpr (V == 1) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
    } else if constexpr (V == 2) {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
      w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, AUX);
        w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
      }
    }
  }
  template <int V>
  static __device__ __forceinline__ void unpack(const uint32_t* w, float* o) {
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = __uint_as_float(w[e]);
  }
  template <int V>
  static __device__ __forceinline__ void ld(Rsrc r, uint32_t off, float* o) {
    if constexpr (V == 1) {
      o[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    } else if constexpr (V == 2) {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      o[0] = __uint_as_float(w.x); o[1] = __uint_as_float(w.y);
    } else {
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * i, 0, 0);
        o[i] = __uint_as_float(w.x); o[i + 1] = __uint_as_float(w.y);
        o[i + 2] = __uint_as_float(w.z); o[i + 3] = __uint_as_float(w.w);
      }
    }
  }
  template <int V, int AUX = 0>
  static __device__ __forceinline__ void st(Rsrc r, uint32_t off, const float* v) {
    if constexpr (V == 1) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, off, 0, AUX);
    } else if constexpr (V == 2) {
      u32x2 w;
      w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
      __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, AUX);
    } else {
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        u32x4 w;
        w.x = __float_as_uint(v[i]); w.y = __float_as_uint(v[i + 1]);
        w.z = __float_as_uint(v[i + 2]); w.w = __float_as_uint(v[i + 3]);
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off + 4 * i, 0, AUX);
      }
    }
  }
};

struct BufBF16 {
  template <int V>
  static constexpr int kWords = (V + 1) / 2;
  template <int V, int AUX = 0>
  static __device__ __forceinline__ void ldw(Rsrc r, uint32_t off, uint32_t* w) {
    if constexpr (V == 1) {
      w[0] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX)) << 16;
    } else if constexpr (V == 2) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
    } else if constexpr (V == 4) {
      const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
      w[0] = x.x; w[1] = x.y;
    } else {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    }
  }
  // V == 1 words hold the element in their high half already
  template <int V>
  static __device__ __forceinline__ void unpack(const uint32_t* w, float* o) {
    if constexpr (V == 1) {
      o[0] = __uint_as_float(w[0]);
    } else {
#pragma unroll
      for (int e = 0; e < V; e += 2) {
        o[e] = bf_lo(w[e / 2]);
        o[e + 1] = bf_hi(w[e / 2]);
      }
    }
  }
  template <int V>
  static __device__ __forceinline__ void ld(Rsrc r, uint32_t off, float* o) {
    if constexpr (V == 1) {
      o[0] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
    } else if constexpr (V == 2) {
      const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
      o[0] = bf_lo(w); o[1] = bf_hi(w);
    } else if constexpr (V == 4) {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
    } else {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
      o[0] = bf_lo(w.x); o[1] = bf_hi(w.x); o[2] = bf_lo(w.y); o[3] = bf_hi(w.y);
      o[4] = bf_lo(w.z); o[5] = bf_hi(w.z); o[6] = bf_lo(w.w); o[7] = bf_hi(w.w);
    }
  }
  template <int V, int AUX = 0>
  static __device__ __forceinline__ void st(Rsrc r, uint32_t off, const float* v) {
    if constexpr (V == 1) {
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(BF16::cvt(v[0])), r, off, 0, AUX);
    } else if constexpr (V == 2) {
      __builtin_amdgcn_raw_buffer_store_b32(BF16::cvt2(v[0], v[1]), r, off, 0, AUX);
    } else if constexpr (V == 4) {
      u32x2 w;
      w.x = BF16::cvt2(v[0], v[1]);
      w.y = BF16::cvt2(v[2], v[3]);
      __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, AUX);
    } else {
      u32x4 w;
      w.x = BF16::cvt2(v[0], v[1]);
      w.y = BF16::cvt2(v[2], v[3]);
      w.z = BF16::cvt2(v[4], v[5]);
      w.w = BF16::cvt2(v[6], v[7]);
      __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, AUX);
    }
  }
};

template <typename IO> struct BufOf;
template <> struct BufOf<F32> { using type = BufF32; };
template <> struct BufOf<BF16> { using type = BufBF16; };

__device__ __forceinline__ float get(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// softplus in log2 units: log2(1 + 2^x2) = max(x2, 0) + log2(1 + e) with
// e = 2^-|x2| in (0, 1] ([Scan page] §1.2: Delta is made positive with
// softplus).  w = 1 + e is rounded; c = e - (w - 1) is that rounding error
// exactly (w - 1 is exact for w in [1, 2], and e and w - 1 are within a
// factor of two of each other or w - 1 is 0), and log2(1 + e) =
// log2(w) + c / (w ln 2) + O(c^2).  Taking c / w as c leaves an error below
// 2^-24 of the result, so the value keeps float32 relative precision as
// 2^x2 -> 0, where log2(1 + 2^x2) alone rounds to 0 (x2 below about -24,
// i.e. delta + bias below about -16.6) and loses digits well before.
// NaN stays NaN; -inf gives exactly 0 and +inf gives +inf.
__device__ __forceinline__ float softplus2(float x2) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x2));
  const float w = 1.0f + e;
  const float c = e - (w - 1.0f);
  return __builtin_fmaf(c, kLog2e, __builtin_amdgcn_logf(w)) + __builtin_fmaxf(x2, 0.0f);
}

// Delta in log2 units from raw delta: x2 = (delta + bias) * log2(e), and
// softplus(x) * log2(e) = softplus2(x2).
__device__ __forceinline__ float delta2(float dl, float bias2, bool softplus) {
  const float x2 = __builtin_fmaf(dl, kLog2e, bias2);
  return softplus ? softplus2(x2) : x2;
}

// delta2 with the softplus flag known at compile time (no branch per element).
template <bool SP>
__device__ __forceinline__ float delta2c(float dl, float bias2) {
  const float x2 = __builtin_fmaf(dl, kLog2e, bias2);
  if constexpr (SP) return softplus2(x2);
  return x2;
}

// silu(z) = z / (1 + e^-z) ([Mamba-2 page] §4.1 SiLU gate).
__device__ __forceinline__ float silu(float zz) {
  return zz * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * zz));
}

// --------------------------------------------------------------------------
// Broadcast of one step's B or C value: B and C for 16 consecutive steps sit
// in one VGPR, lane j of every row of 16 lanes holding step j of that row's
// state.  DPP row_newbcast:j (gfx90a and later) hands lane j's value to its
// whole row as the src0 operand of the consuming v_mul / v_fmac, at no extra
// instruction.  Written out as inline asm so that every mode gets the fused
// form (the compiler folds a separate broadcast into v_mul only when both
// sit in one basic block, and never into v_fmac).  Hazard: a DPP source
// must not have been written by a VALU instruction in the two preceding
// instructions; c is only ever written by LDS loads, which
// tests/test_isa_hazards.py checks on the generated ISA.
// --------------------------------------------------------------------------
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

}  // namespace dev
}  // namespace ssm

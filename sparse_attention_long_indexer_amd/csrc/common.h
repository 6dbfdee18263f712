// Device helpers shared by the DSA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace dsa {

// Raise a kernel's dynamic-LDS limit once per device (the attribute is held
// per device).  `done` is the caller's bit set of devices already configured;
// concurrent first calls may both set it, which is harmless.
inline hipError_t set_lds_limit_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kIdxDim = 128;
constexpr int kWave = 64;
constexpr int64_t kMaxGridY = 65535;  // blocks along a grid's y (and z) extent

// ---- number formats ------------------------------------------------------

// OCP e4m3fn code -> float (exact): E=0 subnormal M*2^-9, else (8+M)*2^(E-10).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = (e == 0) ? ldexpf((float)m, -9) : ldexpf((float)(8u + m), (int)e - 10);
  return (c & 0x80u) ? -mag : mag;
}

// double -> e4m3fn code, round to nearest (ties to even mantissa), saturating
// at 448; zero (either sign) encodes as +0.  The grid step for |x| in
// [2^e, 2^(e+1)) is 2^(e-3) (e >= -6), 2^-9 below 2^-6; scaling by a power of
// two is exact, so rint() performs the only rounding.
__device__ __forceinline__ uint32_t f64_to_e4m3_rne_sat(double x) {
  const uint32_t sign = signbit(x) ? 0x80u : 0u;
  double a = fabs(x);
  if (!(a > 0.0)) return 0u;
  if (a >= 448.0) return sign | 0x7Eu;
  int ex;
  frexp(a, &ex);                       // a = f * 2^ex, f in [0.5, 1)
  int e = ex - 1;
  if (e < -6) e = -6;
  double n = rint(ldexp(a, 3 - e));    // grid steps, exact scaling
  if (n == 0.0) return 0u;
  double v = ldexp(n, e - 3);          // rounded magnitude (<= 448)
  int ev;
  frexp(v, &ev);
  ev -= 1;
  uint32_t code;
  if (ev < -6) {
    code = (uint32_t)ldexp(v, 9);                        // subnormal mantissa
  } else {
    code = ((uint32_t)(ev + 7) << 3) | ((uint32_t)ldexp(v, 3 - ev) - 8u);
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite here)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
}

// two floats -> packed fp16 pair (round to nearest even), and four packed
// fp16 values back to floats
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 v2h __attribute__((ext_vector_type(2)));
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2h));
}
__device__ __forceinline__ v4f unpack_f16x4(v2i p) {
  typedef _Float16 v4h __attribute__((ext_vector_type(4)));
  return __builtin_convertvector(__builtin_bit_cast(v4h, p), v4f);
}

// Order-preserving map of a float score to uint32 (larger score -> larger
// key); -0.0 is folded onto +0.0 so that zeros tie.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- MFMA wrappers ------------------------------------------------------

// 16x16x128 e4m3 x e4m3 -> fp32 (both operand formats code 0 = FP8 E4M3,
// no block scaling).  Lane l supplies 32 bytes of row / column (l % 16);
// lane group l / 16 selects the quarter of the 128-wide reduction; the
// result lane l holds rows 4*(l/16) .. +3 of column l % 16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 -> fp32; lane l supplies 8 values of row / column (l % 16)
// for reduction slice l / 16; result layout as above.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8s& a, const v8s& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16((v8bf)a, (v8bf)b, c, 0, 0, 0);
}

// 32x32x16 bf16 -> fp32; lane l supplies 8 values of row / column (l % 32)
// for reduction slice l / 32; result register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8s& a, const v8s& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16((v8bf)a, (v8bf)b, c, 0, 0, 0);
}

// ---- wave helpers --------------------------------------------------------

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48)
// with the row-swap permutes (VALU, no LDS round trip)
__device__ __forceinline__ float rows_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (VALU only): rows of 16 first, then row 0's total into row 1,
// row 2's into row 3, and lane 31's into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// The same pattern for max / min of unsigned values, read back from lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return ~wave_max_u32(~v);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), 63);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}


// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global access (vmcnt(0)), which would stall on
// direct-to-LDS gathers issued for later tiles; their completion is instead
// awaited explicitly with s_waitcnt vmcnt before the barrier that publishes
// the tile.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier; lgkmcnt(0) completes this wave's LDS accesses.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited on
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace dsa

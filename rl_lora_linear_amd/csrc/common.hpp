// Shared device/host helpers for the gfx950 kernels of the LoRA hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "lora_mi355x.h"

namespace lora {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
__device__ __forceinline__ float bf2f_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 (quiet NaN preserved).
// fp32 -> bf16 round-to-nearest-even on the gfx950 conversion unit
// (v_cvt_pk_bf16_f32, two values per instruction; NaN stays NaN).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const f32x2_hw v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw));
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Split fp32 values into hi + lo bf16 parts (hi = RNE(x), lo = RNE(x - hi)).
// hi + lo carries ~16 significant bits, so a product with an exact bf16 operand
// accumulated by MFMA in fp32 loses ~2^-16 relative instead of 2^-8.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}
// Two values at once: hi = packed RNE(a), RNE(b); lo = packed residuals.
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2bf(a, b);
  lo = pack2bf(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  union { uint4 u; bf16x8 b; } c;
  c.u = v;
  return c.b;
}

// ---------------------------------------------------------------- SwiGLU
// silu(z) = z * sigmoid(z), in fp32 from bf16 inputs, one rounding per output.
// Shared by the elementwise kernels and the GEMM epilogues, so every path
// produces the same bits.  sigmoid uses the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32, ~1 ulp each): exp2 of a large argument is +inf and
// its reciprocal 0, so both tails are exact.
__device__ __forceinline__ float swiglu_sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}
// h = silu(g) * u
__device__ __forceinline__ uint16_t swiglu_fwd1(uint16_t g, uint16_t u) {
  const float z = bf2f(g);
  const float sl = z * swiglu_sigmoid(z);
  return f2bf(sl * bf2f(u));
}
// dg = dh * u * silu'(g), du = dh * silu(g)
__device__ __forceinline__ void swiglu_bwd1(uint16_t dh, uint16_t g, uint16_t u, uint16_t& dg,
                                            uint16_t& du) {
  const float z = bf2f(g), uu = bf2f(u), d = bf2f(dh);
  const float sg = swiglu_sigmoid(z);
  const float sl = z * sg;
  dg = f2bf(d * uu * (sg * (1.f + z * (1.f - sg))));
  du = f2bf(d * sl);
}
__device__ __forceinline__ uint16_t lo16(uint32_t w) { return (uint16_t)(w & 0xFFFFu); }
__device__ __forceinline__ uint16_t hi16(uint32_t w) { return (uint16_t)(w >> 16); }
__device__ __forceinline__ uint32_t pk16(uint16_t a, uint16_t b) { return a | ((uint32_t)b << 16); }
// 8 packed bf16 at once
__device__ __forceinline__ uint4 swiglu_fwd8(uint4 g, uint4 u) {
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t h[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    h[q] = pk16(swiglu_fwd1(lo16(gw[q]), lo16(uw[q])), swiglu_fwd1(hi16(gw[q]), hi16(uw[q])));
  return make_uint4(h[0], h[1], h[2], h[3]);
}
__device__ __forceinline__ void swiglu_bwd8(uint4 dh, uint4 g, uint4 u, uint4& dg, uint4& du) {
  const uint32_t dw[4] = {dh.x, dh.y, dh.z, dh.w}, gw[4] = {g.x, g.y, g.z, g.w},
                 uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t a[4], b[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint16_t g0, u0, g1, u1;
    swiglu_bwd1(lo16(dw[q]), lo16(gw[q]), lo16(uw[q]), g0, u0);
    swiglu_bwd1(hi16(dw[q]), hi16(gw[q]), hi16(uw[q]), g1, u1);
    a[q] = pk16(g0, g1);
    b[q] = pk16(u0, u1);
  }
  dg = make_uint4(a[0], a[1], a[2], a[3]);
  du = make_uint4(b[0], b[1], b[2], b[3]);
}

// ---------------------------------------------------------------- LDS transposing read
// ds_read_b64_tr_b16: in each 16-lane group, lane 4q + j addresses row t0 + q,
// columns 4j..4j+3 of a row-major bf16 tile; lane i of the group receives
// column i of rows t0..t0+3.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 tr_read(const uint4* base, uint32_t byte_off) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)(
                                                     (__attribute__((address_space(3))) void*)base) +
                                                 byte_off));
  union { s16x4 s; uint2 u; } c;
  c.s = v;
  return c.u;
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- status
__device__ __forceinline__ void set_flag(int32_t* status, int32_t bit) {
  // vector-memory atomic OR into the sticky status word
  __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- LDS swizzle
// For LDS tiles whose rows hold eight 16-byte chunks: chunk c of row r lives at
// physical chunk c ^ lds_sw(r), lds_sw(r) = (r & 7) ^ ((r >> 3) & 1).  The
// 16-byte reads of 16 consecutive rows at one logical chunk then land in 16
// distinct (row parity, chunk) slots -- conflict-free whether the LDS serves 8
// or 16 lanes of a ds_read_b128 per clock (gfx950 serves 16; with plain (r & 7)
// rows r and r + 8 collide).
__device__ __forceinline__ int lds_sw(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// ---------------------------------------------------------------- misc
__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Binary search: largest a in [0, n) with pre[a] <= i (pre non-decreasing, pre[0] = 0).
__device__ __forceinline__ int find_bucket(const int32_t* pre, int n, int32_t i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same search by a whole wave (all 64 lanes active, i uniform): 64 samples
// of the range per round, and the highest lane whose sample is <= i narrows it
// to one sample interval -- one dependent load per factor of 64 of n (two for
// n <= 4096) instead of one per halving.
__device__ __forceinline__ int find_bucket_wave(const int32_t* pre, int n, int32_t i) {
  const int lane = (int)(threadIdx.x & 63);
  int lo = 0, end = n;   // pre[lo] <= i; the answer lies in [lo, end)
  while (end - lo > 64) {
    const int step = (end - lo + 63) / 64;
    const int j = lo + lane * step;
    const uint64_t m = __ballot(j < end && pre[j] <= i);
    const int k = 63 - __clzll(m);   // lane 0 samples pre[lo] <= i, so m != 0
    lo += k * step;
    end = min(end, lo + step);
  }
  const int j = lo + lane;
  const uint64_t m = __ballot(j < end && pre[j] <= i);
  return lo + 63 - __clzll(m);
}

}  // namespace lora

// ---------------------------------------------------------------- host side
namespace lora_host {

void set_error(const char* fmt, ...);
lora_status hip_check(hipError_t e, const char* what);
lora_status launch_check(const char* what);
// Compute units of the current device (queried once per device).
int device_cus();

// Kernel timing hooks (no-ops unless lora_timing_enable(1)).
void timer_begin(int timer, hipStream_t s);
void timer_end(int timer, hipStream_t s);

struct Carve {
  char* base;
  size_t used;
  size_t cap;
  explicit Carve(void* b, size_t c) : base((char*)b), used(0), cap(c) {}
  template <typename T>
  T* take(size_t count) {
    used = (size_t)lora::align_up((int64_t)used, 256);
    T* p = base ? (T*)(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
  bool fits() const { return used <= cap; }
};

}  // namespace lora_host

#define TRY_HIP(expr)                                               \
  do {                                                              \
    lora_status _hs = lora_host::hip_check((expr), #expr);          \
    if (_hs != LORA_OK) return _hs;                                 \
  } while (0)

#define LORA_ARG_CHECK(cond, ...)                       \
  do {                                                  \
    if (!(cond)) {                                      \
      lora_host::set_error(__VA_ARGS__);                \
      return LORA_E_INVALID_ARG;                        \
    }                                                   \
  } while (0)

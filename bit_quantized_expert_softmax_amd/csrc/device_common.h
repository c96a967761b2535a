// Device helpers shared by the libmoedecode kernels (gfx950, wave64).
//
// Activation vectors are carried into the int4 GEMVs as "digit planes": each
// group of 32 consecutive fp32 values gets one scale sc = max|x| / kQmax and
// a signed integer q = rint(x / sc) with |q| <= kQmax, written in balanced
// base 16 as q = d0 + 16 d1 + 256 d2 + 4096 d3 with every digit in -8..7.
// Digit d of elements [8p, 8p+8) of the group is packed into one 32-bit word
// (element 8p+i in bits 4i..4i+3), the same order in which the weight bytes
// hold their nibbles. One v_dot8_i32_i4 then multiplies 8 signed weight
// nibbles by 8 signed digits and accumulates in int32, so a 16-byte weight
// chunk (32 nibbles, exactly one quantisation group) costs 16 dot8 and a
// handful of scalar ops, with no nibble unpacking at all. The weight side is
// exact; the activation side is rounded to 16 bits relative to its group's
// largest magnitude (error <= max|x_g| / (2 kQmax) per element).
//
// The digits need no digit-by-digit loop: for |q| <= 0x7777 every nibble of
// q + 0x8888 is d_i + 8 (no borrow leaves a nibble), so the two's complement
// digit nibbles d_i & 15 are the nibbles of (q + 0x8888) ^ 0x8888.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 32;
// Largest |q| whose balanced base-16 expansion has d3 in -8..7 on both signs
// (0x7777).
constexpr int kQmax = 30583;

// The 4 digit nibbles of q (|q| <= kQmax), digit d in bits 4d..4d+3.
__device__ __forceinline__ uint32_t digit_nibbles(int q) {
  return (static_cast<uint32_t>(q + 0x8888) ^ 0x8888u) & 0xFFFFu;
}
constexpr int kWave = 64;

// Digit planes of one group: 4 positions x uint4 (digit words 0..3).
struct DigitGroup {
  uint4 p[4];
};

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot8(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Sum over L consecutive lanes (L a power of two <= 64); every lane of the
// L-lane segment receives the total.
template <int L>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <int L>
__device__ __forceinline__ double seg_sum_f64(double v) {
#pragma unroll
  for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Cross-lane moves through DPP (no LDS traffic). CTRL is the DPP control:
// quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), quad_perm [2,3,0,1] = 0x4E (lane ^ 2),
// row_half_mirror = 0x141 (mirror within 8 lanes), row_mirror = 0x140
// (mirror within 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b & 0xffffffffll), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// Sum over aligned segments of L lanes (L = 4, 8, 16, 32 or 64); every lane of
// a segment receives the segment total. Within 16 lanes the steps are DPP.
template <int L, class T>
__device__ __forceinline__ T dpp_sum(T v) {
  v += dpp<0xB1>(v);
  if (L >= 4) v += dpp<0x4E>(v);
  if (L >= 8) v += dpp<0x141>(v);
  if (L >= 16) v += dpp<0x140>(v);
  if (L >= 32) v += __shfl_xor(v, 16, kWave);
  if (L >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Sum over the whole wave, in every lane: DPP within each 16-lane row, then
// the four row sums through lane reads (a fixed order, no LDS shuffles).
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_sum<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ double wave_sum(double v) {
  v = dpp_sum<16>(v);
  double r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffll), 16 * i);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 16 * i);
    r[i] = __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
  }
  return (r[0] + r[1]) + (r[2] + r[3]);
}

// GELU, tanh form: z/2 * (1 + tanh(u)), u = sqrt(2/pi) * (z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)) (the same function: (1 + tanh u) / 2 is the
// logistic function of 2u) with the hardware exp2 and reciprocal, a few
// units in the last place from the exact value; large |z| give z or -0.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float u = k0 * (z + k1 * z * z * z);
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);  // exp(-2u) = 2^(-2u log2 e)
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Quantise two groups of 32 values to digit planes; called by a whole wave.
// Lanes 0-31 take group g0, lanes 32-63 group g0+1 (skipped when >= ng).
// v is the lane's value (already loaded); writes dig[g] and sc[g]. COHERENT:
// with agent-scope stores, for readers in other blocks of the same launch.
template <bool COHERENT = false>
__device__ __forceinline__ void quant_pair_of_groups(float v, int g0, int ng, DigitGroup* dig,
                                                     float* sc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int g = g0 + (lane >> 5);
  const int i = lane & 31;
  // max over the 32 lanes: DPP within 16 lanes, one shuffle across (max and
  // OR below are exact, so the order of the steps does not matter)
  float m = fabsf(v);
  m = fmaxf(m, dpp<0xB1>(m));
  m = fmaxf(m, dpp<0x4E>(m));
  m = fmaxf(m, dpp<0x141>(m));
  m = fmaxf(m, dpp<0x140>(m));
  m = fmaxf(m, __shfl_xor(m, 16, kWave));
  const float inv = m > 0.f ? static_cast<float>(kQmax) / m : 0.f;
  int q = static_cast<int>(rintf(v * inv));
  q = q > kQmax ? kQmax : (q < -kQmax ? -kQmax : q);
  const uint32_t nb = digit_nibbles(q);
  const int sh = 4 * (i & 7);
  uint32_t w0 = (nb & 15u) << sh;
  uint32_t w1 = ((nb >> 4) & 15u) << sh;
  uint32_t w2 = ((nb >> 8) & 15u) << sh;
  uint32_t w3 = (nb >> 12) << sh;
  // OR over each aligned 8 lanes: quads, then the mirrored quad
  w0 |= dpp<0xB1>(w0);
  w1 |= dpp<0xB1>(w1);
  w2 |= dpp<0xB1>(w2);
  w3 |= dpp<0xB1>(w3);
  w0 |= dpp<0x4E>(w0);
  w1 |= dpp<0x4E>(w1);
  w2 |= dpp<0x4E>(w2);
  w3 |= dpp<0x4E>(w3);
  w0 |= dpp<0x141>(w0);
  w1 |= dpp<0x141>(w1);
  w2 |= dpp<0x141>(w2);
  w3 |= dpp<0x141>(w3);
  if (g < ng) {
    if (COHERENT) {
      if ((i & 7) == 0) {
        uint32_t* p = reinterpret_cast<uint32_t*>(&dig[g].p[i >> 3]);
        __hip_atomic_store(p, w0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p + 1, w1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p + 2, w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p + 3, w3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (i == 0) __hip_atomic_store(sc + g, m / static_cast<float>(kQmax), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if ((i & 7) == 0) dig[g].p[i >> 3] = make_uint4(w0, w1, w2, w3);
      if (i == 0) sc[g] = m / static_cast<float>(kQmax);
    }
  }
}

// Integer dot of one 16-byte weight chunk (32 nibbles) with one digit group:
// returns sum_i nibble_i * q_i exactly (|result| < 2^24).
__device__ __forceinline__ int chunk_dot(const uint4 w, const DigitGroup& x) {
  int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  a0 = sdot8(w.x, x.p[0].x, a0);
  a1 = sdot8(w.x, x.p[0].y, a1);
  a2 = sdot8(w.x, x.p[0].z, a2);
  a3 = sdot8(w.x, x.p[0].w, a3);
  a0 = sdot8(w.y, x.p[1].x, a0);
  a1 = sdot8(w.y, x.p[1].y, a1);
  a2 = sdot8(w.y, x.p[1].z, a2);
  a3 = sdot8(w.y, x.p[1].w, a3);
  a0 = sdot8(w.z, x.p[2].x, a0);
  a1 = sdot8(w.z, x.p[2].y, a1);
  a2 = sdot8(w.z, x.p[2].z, a2);
  a3 = sdot8(w.z, x.p[2].w, a3);
  a0 = sdot8(w.w, x.p[3].x, a0);
  a1 = sdot8(w.w, x.p[3].y, a1);
  a2 = sdot8(w.w, x.p[3].z, a2);
  a3 = sdot8(w.w, x.p[3].w, a3);
  return a0 + 16 * a1 + 256 * a2 + 4096 * a3;
}

__device__ __forceinline__ float h2f(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// Streaming 16-byte load of weight bytes (read once per call).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_w16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming 16-byte store (data not read again by this kernel).
__device__ __forceinline__ void store_nt16(uint4* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Barrier of a block that keeps its vector loads in flight. __syncthreads()
// orders memory with a fence whose lowering waits for every outstanding
// vector load, loads meant for later work included, which would drain a
// prefetch. Here each wave has already waited (by data dependence or an
// explicit s_waitcnt) for its own loads whose LDS data the others read next,
// waits for its own LDS accesses (lgkmcnt 0), then meets the others; the empty
// asm statements keep the compiler from moving memory accesses across,
// sched_barrier keeps the scheduler from moving instructions.
__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only (vmcnt 63, expcnt 7: no wait)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace moe

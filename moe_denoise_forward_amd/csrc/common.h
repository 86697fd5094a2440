// Device-side helpers shared by the libdgmoe kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dgmoe.h"

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

#define DG_WAVE 64

template <typename T, typename S>
__device__ __forceinline__ T bitcast(S s) {
  static_assert(sizeof(T) == sizeof(S), "bitcast size");
  return __builtin_bit_cast(T, s);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)bitcast<_Float16>(b);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return bitcast<float>((uint32_t)b << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = bitcast<uint32_t>(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A lane's view of another lane of its row of 16 (DPP, no LDS crossbar).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// Sum within each row of 16 lanes, in every lane of the row: swap neighbours,
// swap pairs, mirror halves of 8, mirror the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += bitcast<float>(dpp32<0xB1>(bitcast<uint32_t>(v)));   // quad_perm [1,0,3,2]
  v += bitcast<float>(dpp32<0x4E>(bitcast<uint32_t>(v)));   // quad_perm [2,3,0,1]
  v += bitcast<float>(dpp32<0x141>(bitcast<uint32_t>(v)));  // row_half_mirror
  v += bitcast<float>(dpp32<0x140>(bitcast<uint32_t>(v)));  // row_mirror
  return v;
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return bitcast<float>(__builtin_amdgcn_readlane(bitcast<int>(v), lane));
}
// Wave-wide sum as a uniform value: the four row sums added in a fixed order,
// so the result is the same on every run.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// One Q4G64 word (8 consecutive inputs, layout of include/dgmoe.h) -> 8 fp16
// weights, each RNE(scale * q + bias) with a single rounding.
//
// The nibble pairs (0,1) and (4,5) sit in the low nibble of each 16-bit half
// after an optional >> 8; OR-ing 0x6400 (fp16 1024.0) makes the half exactly
// 1024 + q.  Pairs (2,3) and (6,7) sit in bits 4..7 of each half; OR-ing 0x5400
// (fp16 64.0, whose mantissa step at bit 4 is 1.0) makes it exactly 64 + q.
// Subtracting the magic is exact, and one packed fma applies scale and bias.
__device__ __forceinline__ half8_t dequant_q4_word(uint32_t v, half2_t s2, half2_t b2) {
  const half2_t m1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2_t m64 = {(_Float16)64.0f, (_Float16)64.0f};
  // (v & mask) | magic is one v_bitop3_b32 (truth table 0xEA = (a & b) | c)
  uint32_t v8 = v >> 8;
  half2_t q01 = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v, 0x000F000Fu, 0x64006400u, 0xEA)) - m1024;
  half2_t q23 = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v, 0x00F000F0u, 0x54005400u, 0xEA)) - m64;
  half2_t q45 = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v8, 0x000F000Fu, 0x64006400u, 0xEA)) - m1024;
  half2_t q67 = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v8, 0x00F000F0u, 0x54005400u, 0xEA)) - m64;
  half2_t w01 = __builtin_elementwise_fma(q01, s2, b2);
  half2_t w23 = __builtin_elementwise_fma(q23, s2, b2);
  half2_t w45 = __builtin_elementwise_fma(q45, s2, b2);
  half2_t w67 = __builtin_elementwise_fma(q67, s2, b2);
  half8_t r = {w01[0], w01[1], w23[0], w23[1], w45[0], w45[1], w67[0], w67[1]};
  return r;
}

// Eight Q8G64 codes (two little-endian words, inputs in byte order) -> 8
// fp16 weights, each RNE(scale * q + bias) with a single rounding: v_perm
// puts each code byte under the high byte 0x64, which makes the fp16 half
// exactly 1024 + q; subtracting 1024 is exact and one packed fma applies scale
// and bias.
__device__ __forceinline__ half8_t dequant_q8_pair(uint32_t lo, uint32_t hi, half2_t s2, half2_t b2) {
  const half2_t m1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  // selector bytes: 0..3 the code word, 4 the constant's 0x64
  const half2_t q01 = bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - m1024;
  const half2_t q23 = bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - m1024;
  const half2_t q45 = bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - m1024;
  const half2_t q67 = bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - m1024;
  const half2_t w01 = __builtin_elementwise_fma(q01, s2, b2);
  const half2_t w23 = __builtin_elementwise_fma(q23, s2, b2);
  const half2_t w45 = __builtin_elementwise_fma(q45, s2, b2);
  const half2_t w67 = __builtin_elementwise_fma(q67, s2, b2);
  half8_t r = {w01[0], w01[1], w23[0], w23[1], w45[0], w45[1], w67[0], w67[1]};
  return r;
}

// One Q6G32 word (the low 4 bits of 8 codes, Q4G64 word layout) and its high
// bits (hw: the high two bits of input 2p + t at bits 2p + 16t) -> 8 fp16
// weights, each RNE(scale * q + bias) with a single rounding: both parts of
// every code are expanded exactly with the magic numbers of dequant_q4_word,
// joined exactly (q = 16 hi + lo <= 63) and one packed fma applies scale and
// bias.
__device__ __forceinline__ half8_t dequant_q6_word(uint32_t v, uint32_t hw, half2_t s2, half2_t b2) {
  const half2_t m1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2_t m64 = {(_Float16)64.0f, (_Float16)64.0f};
  const half2_t k16 = {(_Float16)16.0f, (_Float16)16.0f};
  const uint32_t v8 = v >> 8;
  half2_t q[4];
  q[0] = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v, 0x000F000Fu, 0x64006400u, 0xEA)) - m1024;
  q[1] = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v, 0x00F000F0u, 0x54005400u, 0xEA)) - m64;
  q[2] = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v8, 0x000F000Fu, 0x64006400u, 0xEA)) - m1024;
  q[3] = bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(v8, 0x00F000F0u, 0x54005400u, 0xEA)) - m64;
  half8_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const half2_t hi =
        bitcast<half2_t>(__builtin_amdgcn_bitop3_b32(hw >> (2 * p), 0x00030003u, 0x64006400u, 0xEA)) - m1024;
    const half2_t w = __builtin_elementwise_fma(__builtin_elementwise_fma(hi, k16, q[p]), s2, b2);
    r[2 * p] = w[0];
    r[2 * p + 1] = w[1];
  }
  return r;
}

// One word of 4-bit E2M1 codes (the Q4G64 word layout: input 2p + t at bits
// 4p + 16t) -> 8 fp16 weights e2m1(code) * s2.  v_perm looks each code's
// magnitude up in an 8-byte table of fp16 high bytes (0, .5, 1, 1.5, 2, 3, 4,
// 6), the sign bit is or-ed in, and a second v_perm places each byte over a
// zero low byte; every E2M1 value is exact in fp16.  The low nibbles of the
// four bytes are inputs 0, 4, 1, 5 and the high nibbles inputs 2, 6, 3, 7.
__device__ __forceinline__ half8_t dequant_fp4_word(uint32_t v, half2_t s2) {
  const uint32_t tlo = 0x3E3C3800u, thi = 0x46444240u;
  const uint32_t e = __builtin_amdgcn_perm(thi, tlo, v & 0x07070707u) | ((v << 4) & 0x80808080u);
  const uint32_t o = __builtin_amdgcn_perm(thi, tlo, (v >> 4) & 0x07070707u) | (v & 0x80808080u);
  const half2_t w01 = bitcast<half2_t>(__builtin_amdgcn_perm(e, e, 0x020C000Cu)) * s2;
  const half2_t w23 = bitcast<half2_t>(__builtin_amdgcn_perm(o, o, 0x020C000Cu)) * s2;
  const half2_t w45 = bitcast<half2_t>(__builtin_amdgcn_perm(e, e, 0x030C010Cu)) * s2;
  const half2_t w67 = bitcast<half2_t>(__builtin_amdgcn_perm(o, o, 0x030C010Cu)) * s2;
  half8_t r = {w01[0], w01[1], w23[0], w23[1], w45[0], w45[1], w67[0], w67[1]};
  return r;
}

// An E4M3 scale byte (sign 0) -> its exact fp16 value: its exponent and
// mantissa bits placed in fp16's (bits 7..13) read 2^-8 times the value, for
// subnormals too; multiplying by 256 is exact.
__device__ __forceinline__ _Float16 e4m3_half(uint32_t byte) {
  return bitcast<_Float16>((uint16_t)((byte & 0x7Fu) << 7)) * (_Float16)256.0f;
}

__device__ __forceinline__ uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// A workgroup barrier that orders LDS accesses only: the vector memory loads
// in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 8 bf16 values (as 4 uint32) -> 8 fp16 (RNE of each value).
__device__ __forceinline__ half8_t bf16x8_to_half8(uint4 v) {
  half8_t r;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)bitcast<float>(w[i] << 16);
    r[2 * i + 1] = (_Float16)bitcast<float>(w[i] & 0xFFFF0000u);
  }
  return r;
}

// Data passed between workgroups of one launch (counters, stamps, logits,
// partial tiles) is written and read with agent-scope relaxed atomic accesses,
// which are coherent across the XCDs' L2 caches without a cache write-back
// or invalidate; a writer waits until all of its stores have completed
// (vmcnt(0)) before the barrier that precedes its arrival.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Record error kind `kind` for the call with this stamp (see the sync region
// in kernels.h); every writer of one call writes the same value.
__device__ __forceinline__ void flag_error(uint32_t* sync, int kind, uint64_t stamp) {
  st_agent((uint64_t*)(sync + 4) + kind, stamp);
}
__device__ __forceinline__ void drain_then_sync() {
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt, lgkmcnt all zero: this wave's stores are done
  __syncthreads();
}

// GELU, tanh form: 0.5 g (1 + tanh u) with u = sqrt(2/pi) (g + 0.044715 g^3),
// evaluated as the identical g / (1 + exp(-2u)), exp(-2u) = 2^(-2u log2 e) on
// the hardware exp2, then one hardware reciprocal (both within an ulp or so;
// the result is rounded to fp16 next).  No branch: large |u| saturates through
// exp2's inf / 0 to -0 / g.  Every operation is an explicitly rounded one (no
// contraction into fma), so each inlined copy -- one per accumulator position
// in a GEMM epilogue -- computes bit-identical results and a row's output
// never depends on where in a tile it sits.
__device__ __forceinline__ float gelu_tanh(float g) {
  const float c = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float g3 = __fmul_rn(__fmul_rn(g, g), g);
  const float t = __fmul_rn(c, __fadd_rn(g, __fmul_rn(0.044715f, g3)));
  return __fmul_rn(g, __builtin_amdgcn_rcpf(__fadd_rn(1.0f, __builtin_amdgcn_exp2f(t))));
}

// Device-side building blocks for the KDA kernels on gfx950 (CDNA4):
// 64-lane wavefront matrix-core (MFMA) wrappers, DPP row scans, and
// element conversions. Everything here is wave-level and header-only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kChunk = 16;  // tokens per chunk (one MFMA tile edge)

// ---- element conversions -------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Input element loads: T is float (fp32 inputs) or uint16_t (bf16 bits).
template <typename T> __device__ __forceinline__ float load_in(const T* p, size_t i);
template <> __device__ __forceinline__ float load_in<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

// An input element as loaded (float, or bf16 bits) -> float.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t b) { return bf16_bits_to_f32(b); }

// Four consecutive input elements starting at p[i] (i a multiple of 4).
template <typename T> __device__ __forceinline__ void load_in4(const T* p, size_t i, float out[4]);
template <> __device__ __forceinline__ void load_in4<float>(const float* p, size_t i, float out[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p + i);
  out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
}
template <> __device__ __forceinline__ void load_in4<uint16_t>(const uint16_t* p, size_t i, float out[4]) {
  const uint2 x = *reinterpret_cast<const uint2*>(p + i);
  out[0] = __uint_as_float(x.x << 16);
  out[1] = __uint_as_float(x.x & 0xffff0000u);
  out[2] = __uint_as_float(x.y << 16);
  out[3] = __uint_as_float(x.y & 0xffff0000u);
}

// Unpack four input elements loaded as one vector (float4 for fp32 inputs,
// two dwords of bf16 bit pairs for bf16 inputs).
__device__ __forceinline__ void unpack4(const float4& x, float out[4]) {
  out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
}
__device__ __forceinline__ void unpack4(const uint2& x, float out[4]) {
  out[0] = __uint_as_float(x.x << 16);
  out[1] = __uint_as_float(x.x & 0xffff0000u);
  out[2] = __uint_as_float(x.y << 16);
  out[3] = __uint_as_float(x.y & 0xffff0000u);
}

// Access at a wavefront-uniform base plus a 32-bit per-lane byte offset. This
// is the shape the backend emits as a scalar-base global access (base in
// SGPRs, offset in one VGPR), with no 64-bit per-lane address arithmetic.
template <typename T>
__device__ __forceinline__ T ld_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ void st_at(void* base, uint32_t byte_off, T x) {
  *reinterpret_cast<T*>(reinterpret_cast<char*>(base) + byte_off) = x;
}
__device__ __forceinline__ float ld_in_at(const float* base, uint32_t byte_off) {
  return ld_at<float>(base, byte_off);
}
__device__ __forceinline__ float ld_in_at(const uint16_t* base, uint32_t byte_off) {
  return bf16_bits_to_f32(ld_at<uint16_t>(base, byte_off));
}
__device__ __forceinline__ void st_out_at(float* base, uint32_t byte_off, float x) {
  st_at<float>(base, byte_off, x);
}
__device__ __forceinline__ void st_out_at(uint16_t* base, uint32_t byte_off, float x) {
  st_at<uint16_t>(base, byte_off, f32_to_bf16_bits(x));
}

// Four consecutive outputs at a uniform base plus a per-lane byte offset (16
// bytes for fp32, 8 bytes of bf16 for bf16 outputs).
__device__ __forceinline__ void st_out4_at(float* base, uint32_t byte_off, f32x4 x) {
  st_at<f32x4>(base, byte_off, x);
}
__device__ __forceinline__ void st_out4_at(uint16_t* base, uint32_t byte_off, f32x4 x) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t w = {static_cast<uint32_t>(f32_to_bf16_bits(x[0])) |
                         (static_cast<uint32_t>(f32_to_bf16_bits(x[1])) << 16),
                     static_cast<uint32_t>(f32_to_bf16_bits(x[2])) |
                         (static_cast<uint32_t>(f32_to_bf16_bits(x[3])) << 16)};
  st_at<u32x2_t>(base, byte_off, w);
}

template <typename T> __device__ __forceinline__ void store_out(T* p, size_t i, float x);
template <> __device__ __forceinline__ void store_out<float>(float* p, size_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, size_t i, float x) {
  p[i] = f32_to_bf16_bits(x);
}

// Log-decay floor: clamp to [-5, 0] with comparisons, so NaN stays NaN.
__device__ __forceinline__ float clamp_decay(float x) {
  return x < -5.0f ? -5.0f : (x > 0.0f ? 0.0f : x);
}

// Per-channel log-decay from the g input. GATE 0: g is the log-decay itself
// (floored at -5, capped at 0). GATE 1: g is a raw gate logit x and the
// log-decay is the sigmoid scaled to the floor, -5 / (1 + e^-x), a lower-
// bounded sigmoid decay whose retention never drops below e^-5 ("Kimi K3
// goes trillion-scale with sparse MoE efficiency" subtitles, cue 14; "K3 tech
// report" podcast, the decay-bound exchange). The clamp then only passes NaN.
template <int GATE>
__device__ __forceinline__ float gate_decay(float x) {
  if constexpr (GATE == 1) {
    return clamp_decay(-5.0f / (1.0f + __expf(-x)));
  } else {
    return clamp_decay(x);
  }
}

// ---- DPP row scans (a row is 16 consecutive lanes) -----------------------

template <int kCtrl>
__device__ __forceinline__ float dpp_move(float x) {
  // Lanes whose source falls outside the row receive 0.0f.
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

// Inclusive prefix sum over the 16 lanes of each row (lane r gets sum of
// lanes 0..r of its row): Hillis-Steele with row_shr:1,2,4,8.
__device__ __forceinline__ float row_inclusive_prefix_sum(float x) {
  x += dpp_move<0x111>(x);
  x += dpp_move<0x112>(x);
  x += dpp_move<0x114>(x);
  x += dpp_move<0x118>(x);
  return x;
}

// Lane 15 of each row broadcast to the whole row (row_newbcast:15): the value
// at a chunk's last token, e.g. e^gamma from e^Gamma_r.
__device__ __forceinline__ float row_broadcast_last(float x) { return dpp_move<0x15F>(x); }

// ---- MFMA wrappers (16x16 output tiles, fp32 accumulate) -----------------
// Output layout for every 16x16 tile: lane l holds rows 4*(l/16)+i, i=0..3,
// of column l%16. Operand layouts (checked on gfx950): 16x16x16 f16 lane l
// holds A[l%16][4*(l/16)+i] and B[4*(l/16)+i][l%16]; 16x16x32 f16/bf16 holds
// A[l%16][8*(l/16)+j] and B[8*(l/16)+j][l%16]; 16x16x4 f32 holds A[l%16][l/16]
// and B[l/16][l%16].
// On gfx950 an accumulator written by one MFMA shape and read as the
// accumulator input of a different shape (16x16x16 <-> 16x16x32) needs about
// six wait states that the compiler does not insert (the later MFMA then sees
// stale elements). Chains of one shape are interlocked by the hardware, so
// every accumulation chain in these kernels uses a single shape.

__device__ __forceinline__ f32x4 mma_16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_16x16x16_f16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda

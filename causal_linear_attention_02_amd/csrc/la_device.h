// Device-side building blocks for the linear-attention kernels (gfx950 / CDNA4).
//
// Matrix products run on the 32x32 MFMA shape. One "K-block" is 16 values of
// the contraction index; an operand fragment holds, for each lane l, 8 values
// of that block: rows/columns (l % 32) and contraction indices 8*(l/32)+0..7.
//   bf16 operands: one v_mfma_f32_32x32x16_bf16 per K-block;
//   fp32 operands: eight v_mfma_f32_32x32x2_f32 per K-block, issue j taking
//                  contraction index 8*(l/32)+j (the same fragment layout).
// Accumulator tile (32x32 fp32): lane l, register r holds
//   row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
//
// An accumulator tile T becomes an operand fragment with lanes indexing T's
// columns and the registers indexing T's rows (acc_to_frag): the lower half
// of the wave holds rows 0-3 of each group of 8 and the upper half rows 4-7,
// so one v_permlane32_swap per register pair completes the 8 contiguous rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;      // tokens per chunk (two 32-row MFMA tiles)
constexpr float kEps = 1e-6f;   // denominator clamp: y = num / max(den, eps)


// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));  // RNE
}

__device__ __forceinline__ float round_bf16(float a) {
  return bf16_bits_to_f32(pack_bf16x2(a, 0.f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// Raw buffer access: a wave-uniform descriptor (base, size in bytes) and a
// per-lane 32-bit byte offset. Loads past `bytes` return zero and stores past
// it are dropped by the hardware range check.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}
// Non-temporal forms (cache-policy bit NT) for data a kernel touches once:
// measured on the long-context prefill, they keep these streams from
// evicting lines that a later pass reuses and shorten the state pass by ~25%.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kNonTemporal));
}
__device__ __forceinline__ void buf_store16_nt(__amdgpu_buffer_rsrc_t r, int voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kNonTemporal);
}

// 8 consecutive input elements -> fp32
template <typename IN> struct In8;
template <> struct In8<__bf16> {
  using raw = u32x4;  // 16 bytes
  __device__ static void to_f32(const raw& r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(r[i] << 16);
      x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
  __device__ static raw load(const void* p) { return *reinterpret_cast<const raw*>(p); }
  __device__ static raw bload(__amdgpu_buffer_rsrc_t r, int voff) { return buf_load16(r, voff); }
  __device__ static raw bload_nt(__amdgpu_buffer_rsrc_t r, int voff) { return buf_load16_nt(r, voff); }
  __device__ static raw zero() { return raw{0, 0, 0, 0}; }
  __device__ static raw neg_inf() { return raw{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u}; }
};
template <> struct In8<float> {
  struct raw { f32x4 a, b; };  // 32 bytes
  __device__ static void to_f32(const raw& r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = r.a[i]; x[4 + i] = r.b[i]; }
  }
  __device__ static raw load(const void* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    return raw{q[0], q[1]};
  }
  __device__ static raw bload(__amdgpu_buffer_rsrc_t r, int voff) {
    return raw{__builtin_bit_cast(f32x4, buf_load16(r, voff)), __builtin_bit_cast(f32x4, buf_load16(r, voff + 16))};
  }
  __device__ static raw bload_nt(__amdgpu_buffer_rsrc_t r, int voff) {
    return raw{__builtin_bit_cast(f32x4, buf_load16_nt(r, voff)),
               __builtin_bit_cast(f32x4, buf_load16_nt(r, voff + 16))};
  }
  __device__ static raw zero() { return raw{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
  __device__ static raw neg_inf() {
    const float n = -__builtin_inff();
    return raw{f32x4{n, n, n, n}, f32x4{n, n, n, n}};
  }
};

// ---------------------------------------------------------------------------
// Feature maps (fp32 math)
// ---------------------------------------------------------------------------
// elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) for x <= 0.
// Written as max(x, 0) + min(exp(x), 1): for x > 0 that is x + 1, for x <= 0
// it is exp(x). The min is the clamp output modifier of the hardware exp2 and
// the max is the NaN-propagating maximum, so NaN stays NaN and exp(-inf) = 0.
__device__ __forceinline__ float phi_elu1(float x) {
  const float e = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * 1.4426950408889634f), 0.f, 1.f);
  return __builtin_elementwise_maximum(x, 0.f) + e;
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles. Rows of RB bytes; 16-byte units are permuted per row so
// that both 16-byte row-fragment reads (16 consecutive rows, same unit) and
// transposed reads (4 consecutive rows, 4 consecutive units) hit distinct
// bank groups.
// ---------------------------------------------------------------------------
template <int RB>
__device__ __forceinline__ int swz(int row) {
  if constexpr (RB <= 64) return (row >> 2) & 3;
  else if constexpr (RB == 128) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else if constexpr (RB == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  // rows of 32 or more units: row bit 4 also picks the upper half of 32
  // units, so that the 32 rows of one MFMA tile read at one column land in
  // 32 different units (the transposed reads, 4 rows within a 16-row block,
  // see the same permutation as above)
  else return ((row & 3) << 2) | ((row >> 2) & 3) | (row & 16);
}

template <int RB>
__device__ __forceinline__ int tile_off(int row, int byte) {
  return row * RB + ((((byte >> 4) ^ swz<RB>(row))) << 4) + (byte & 15);
}

// ---------------------------------------------------------------------------
// Operand policies
// ---------------------------------------------------------------------------
template <typename OP> struct Ops;

template <> struct Ops<__bf16> {
  using frag = bf16x8;
  static constexpr int kBytes = 2;

  __device__ static __forceinline__ void mma(f32x16& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ static __forceinline__ frag zero() { return frag{}; }

  // Rows = lane % 32 + row0, contraction index k0 + 8*(lane/32) + 0..7.
  template <int RB>
  __device__ static __forceinline__ frag load_rows(const uint8_t* tile, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const int row = row0 + (l & 31);
    const int byte = (k0 + 8 * (l >> 5)) * 2;
    return *reinterpret_cast<const frag*>(tile + tile_off<RB>(row, byte));
  }
  // Transposed: lane l gets column col0 + lane % 32 of rows j0 + 8*(lane/32) + 0..7.
  template <int RB>
  __device__ static __forceinline__ frag load_cols(const uint8_t* tile, int j0, int col0) {
    const int l = threadIdx.x & 63;
    const int g = l >> 4, t = l & 15;
    const int rbase = j0 + 8 * (g >> 1) + (t >> 2);
    const int col = col0 + 16 * (g & 1) + 4 * (t & 3);
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint8_t* p0 = tile + tile_off<RB>(rbase, col * 2);
    const uint8_t* p1 = tile + tile_off<RB>(rbase + 4, col * 2);
    s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    u32x2 a = __builtin_bit_cast(u32x2, r0), b = __builtin_bit_cast(u32x2, r1);
    u32x4 v = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(frag, v);
  }
  // Accumulator tile -> fragment for K-block kb (rows 16kb..16kb+15).
  __device__ static __forceinline__ frag from_acc(const f32x16& c, int kb) {
    uint32_t a0 = pack_bf16x2(c[8 * kb + 0], c[8 * kb + 1]);
    uint32_t a1 = pack_bf16x2(c[8 * kb + 2], c[8 * kb + 3]);
    uint32_t b0 = pack_bf16x2(c[8 * kb + 4], c[8 * kb + 5]);
    uint32_t b1 = pack_bf16x2(c[8 * kb + 6], c[8 * kb + 7]);
    auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
    return __builtin_bit_cast(frag, v);
  }
  // fp32 value of element i of a fragment
  __device__ static __forceinline__ float elem(const frag& f, int i) { return (float)f[i]; }
  // store 8 fp32 values (already feature-mapped) into a tile row chunk
  template <int RB>
  __device__ static __forceinline__ void store8(uint8_t* tile, int row, int k0, const float (&x)[8]) {
    u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
               pack_bf16x2(x[6], x[7])};
    *reinterpret_cast<u32x4*>(tile + tile_off<RB>(row, k0 * 2)) = v;
  }
};

template <> struct Ops<float> {
  using frag = f32x8;
  static constexpr int kBytes = 4;

  __device__ static __forceinline__ void mma(f32x16& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
  }
  __device__ static __forceinline__ frag zero() { return frag{}; }

  template <int RB>
  __device__ static __forceinline__ frag load_rows(const uint8_t* tile, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const int row = row0 + (l & 31);
    const int byte = (k0 + 8 * (l >> 5)) * 4;
    f32x4 a = *reinterpret_cast<const f32x4*>(tile + tile_off<RB>(row, byte));
    f32x4 b = *reinterpret_cast<const f32x4*>(tile + tile_off<RB>(row, byte + 16));
    return frag{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  template <int RB>
  __device__ static __forceinline__ frag load_cols(const uint8_t* tile, int j0, int col0) {
    const int l = threadIdx.x & 63;
    const int col = col0 + (l & 31);
    const int r0 = j0 + 8 * (l >> 5);
    frag f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) f[jj] = *reinterpret_cast<const float*>(tile + tile_off<RB>(r0 + jj, col * 4));
    return f;
  }
  __device__ static __forceinline__ frag from_acc(const f32x16& c, int kb) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[8 * kb + i]),
                                                __float_as_uint(c[8 * kb + 4 + i]), false, false);
      f[i] = __uint_as_float(s[0]);
      f[4 + i] = __uint_as_float(s[1]);
    }
    return f;
  }
  __device__ static __forceinline__ float elem(const frag& f, int i) { return f[i]; }
  template <int RB>
  __device__ static __forceinline__ void store8(uint8_t* tile, int row, int k0, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, k0 * 4)) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, k0 * 4 + 16)) = f32x4{x[4], x[5], x[6], x[7]};
  }
};

// s_waitcnt vmcnt(0): wait for every outstanding vector memory operation.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Range guard of the chunked decay and gated kernels. They scale the rows of
// a 64-token chunk by up to gamma^-32 (or alpha^-32 per feature), which stays
// within 2^64 only for gamma, alpha in [1/4, 1]. A value outside that range
// (NaN included) becomes NaN, so every output that depends on it is NaN, and
// raises the device status flag that the host reports (la_device_status).
// The flag is set by a vector atomic from one lane.
// ---------------------------------------------------------------------------
constexpr float kMinFactor = 0.25f;
constexpr float kMinLogFactor = -1.3862944f;   // log(1/4), rounded toward -inf in fp32

__device__ __forceinline__ void raise_status(int* flag) {
  if (flag) atomicOr(flag, 1);
}

// log2(gamma) for gamma in [1/4, 1]; NaN (and the flag, from thread 0) otherwise.
__device__ __forceinline__ float decay_log2(float g, int* flag) {
  if (g >= kMinFactor && g <= 1.f) return __log2f(g);
  if (threadIdx.x == 0) raise_status(flag);
  return __builtin_nanf("");
}

// A log-gate in [log(1/4), 0] as given; NaN (and the flag) otherwise.
__device__ __forceinline__ float checked_log_gate(float x, int* flag) {
  if (x >= kMinLogFactor && x <= 0.f) return x;
  raise_status(flag);
  return __builtin_nanf("");
}

// Exchange with the lane 32 positions away (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // lanes 0-31 receive the upper half's value in s[1]; lanes 32-63 the lower half's in s[0]
  return __uint_as_float((threadIdx.x & 32) ? s[0] : s[1]);
}

}  // namespace la

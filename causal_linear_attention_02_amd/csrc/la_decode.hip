// Recurrent decode step of kernelized linear attention on gfx950.
//
// One new token per (batch, head) ("Linear Attention", marovi.ai, "Forma
// recurrente e inferencia autorregresiva"; "Linear Transformer (Transformers
// are RNNs)", "La formulación recurrente paso a paso"):
//   S <- S + phi(k) v^T,  z <- z + phi(k),  y = phi(q)^T S / phi(q).z
// (the state is updated first, so the new token attends to itself).
//
// The identity map uses q and k as they are.
// Random features: phi(x) = exp(W x~ - |x~|^2/2) / sqrt(m), x~ = d^(-1/4) x
// ("Linear Attention", "Mapas de características"), computed per head in fp32
// from W (m x d, fp32; rounded to bf16 for bf16 inputs) before the state
// update.
//
// The step is a pure stream over the fp32 state: every state element is read
// once and written once. Each head's DF x D state is covered by TPH threads,
// each owning a 4-column group (one 16-byte vector) of DF/R rows, so one load
// instruction of a head covers R consecutive rows = TPH * 16 contiguous
// bytes. All state loads are issued before any arithmetic.
#include "la_device.h"
#include "la_kernels.h"

namespace la {

template <int D, int DF>
struct DecodeShape {
  static constexpr int TPH = (DF * D / 64 > 64) ? DF * D / 64 : 64;  // threads per head
  static constexpr int HPB = 256 / TPH;                               // heads per block
  static constexpr int CG = D / 4;                                    // 16-byte column groups
  static constexpr int R = TPH / CG;                                  // row groups
  static constexpr int RPT = DF / R;                                  // rows per thread
  static constexpr int WPH = TPH / 64;                                // waves per head
  static_assert(TPH % CG == 0 && DF % R == 0, "decode tiling");
};

template <typename IN> __device__ __forceinline__ float load_elem(const void* p, long long i);
template <> __device__ __forceinline__ float load_elem<__bf16>(const void* p, long long i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_elem<float>(const void* p, long long i) {
  return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int D, int DF, typename IN, int FM>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  using SH = DecodeShape<D, DF>;
  __shared__ float s_phiq[SH::HPB][DF];
  __shared__ float s_phik[SH::HPB][DF];
  __shared__ float s_v[SH::HPB][D];
  __shared__ f32x4 s_num[SH::HPB][SH::R][SH::CG];
  __shared__ float s_den[SH::HPB][SH::WPH];
  __shared__ float s_x[FM == kPerformer ? SH::HPB : 1][FM == kPerformer ? 2 * D : 1];

  const int hb = threadIdx.x / SH::TPH;      // head within block
  const int t = threadIdx.x % SH::TPH;       // thread within head
  const long long head = (long long)blockIdx.x * SH::HPB + hb;
  const bool valid = head < a.BH;
  const int cg = t % SH::CG, rg = t / SH::CG;

  // state loads first (the bulk of the traffic)
  float* Sh = a.S + head * (DF * D);
  f32x4 Sv[SH::RPT];
  if (valid) {
#pragma unroll
    for (int i = 0; i < SH::RPT; ++i)
      Sv[i] = *reinterpret_cast<const f32x4*>(Sh + (long long)(rg + SH::R * i) * D + 4 * cg);
  }
  // token features
  if constexpr (FM == kElu1) {
    if (valid) {
      for (int e = t; e < D; e += SH::TPH) {
        const long long off = head * D + e;
        s_phiq[hb][e] = phi_elu1(load_elem<IN>(a.q, off));
        s_phik[hb][e] = phi_elu1(load_elem<IN>(a.k, off));
        s_v[hb][e] = load_elem<IN>(a.v, off);
      }
    }
  } else if constexpr (FM == kIdentity) {
    if (valid) {
      for (int e = t; e < D; e += SH::TPH) {
        const long long off = head * D + e;
        s_phiq[hb][e] = load_elem<IN>(a.q, off);
        s_phik[hb][e] = load_elem<IN>(a.k, off);
        s_v[hb][e] = load_elem<IN>(a.v, off);
      }
    }
  } else {
    if (valid) {
      for (int e = t; e < D; e += SH::TPH) {
        const long long off = head * D + e;
        s_x[hb][e] = load_elem<IN>(a.q, off);
        s_x[hb][D + e] = load_elem<IN>(a.k, off);
        s_v[hb][e] = load_elem<IN>(a.v, off);
      }
    }
    __syncthreads();
    if (valid) {
      float nq = 0.f, nk = 0.f;
      for (int e = 0; e < D; ++e) {
        nq += s_x[hb][e] * s_x[hb][e];
        nk += s_x[hb][D + e] * s_x[hb][D + e];
      }
      const float A = sqrtf(sqrtf(1.0f / (float)D)) * 1.4426950408889634f;
      const float c = 1.4426950408889634f * 0.5f / sqrtf((float)D);
      const float Bm = 0.5f * __log2f((float)DF);
      for (int f = t; f < DF; f += SH::TPH) {
        const float* wr = a.W + (long long)f * D;
        float uq = 0.f, uk = 0.f;
#pragma unroll 4
        for (int e = 0; e < D; e += 4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(wr + e);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // bf16 inputs project with W in bf16, as the chunked forward does
            const float wj = sizeof(IN) == 2 ? round_bf16(w4[j]) : w4[j];
            uq += wj * s_x[hb][e + j];
            uk += wj * s_x[hb][D + e + j];
          }
        }
        s_phiq[hb][f] = __builtin_amdgcn_exp2f(A * uq - c * nq - Bm);
        s_phik[hb][f] = __builtin_amdgcn_exp2f(A * uk - c * nk - Bm);
      }
    }
  }
  __syncthreads();

  // decay ("Linear Attention", "Variantes y extensiones"): S <- gamma S + phi(k) v^T, z alike
  const float gm = (a.gamma && valid) ? a.gamma[head % a.H] : 1.f;
  // z <- gamma z + phi(k); partial phi(q).z
  float dpart = 0.f;
  if (valid) {
    for (int c = t; c < DF; c += SH::TPH) {
      const float gz = a.lgate ? gm * __builtin_amdgcn_exp2f(a.lgate[head * DF + c] * 1.4426950408889634f) : gm;
      const float zn = gz * a.z[head * DF + c] + s_phik[hb][c];
      a.z[head * DF + c] = zn;
      dpart += s_phiq[hb][c] * zn;
    }
  }
  dpart = wave_sum(dpart);
  if ((t & 63) == 0) s_den[hb][t >> 6] = dpart;

  // S <- S + phi(k) v^T; numerator phi(q)^T S over this thread's rows
  const f32x4 v4 = valid ? *reinterpret_cast<const f32x4*>(&s_v[hb][4 * cg]) : f32x4{0, 0, 0, 0};
  f32x4 num = {0, 0, 0, 0};
  if (valid) {
#pragma unroll
    for (int i = 0; i < SH::RPT; ++i) {
      const int r = rg + SH::R * i;
      const float pk = s_phik[hb][r], pq = s_phiq[hb][r];
      // gated: per-feature gate exp(lgate) of this row of S
      const float gr = a.lgate ? gm * __builtin_amdgcn_exp2f(a.lgate[head * DF + r] * 1.4426950408889634f) : gm;
      f32x4 s = Sv[i];
      s[0] = gr * s[0] + pk * v4[0];
      s[1] = gr * s[1] + pk * v4[1];
      s[2] = gr * s[2] + pk * v4[2];
      s[3] = gr * s[3] + pk * v4[3];
      *reinterpret_cast<f32x4*>(Sh + (long long)r * D + 4 * cg) = s;
      num[0] += pq * s[0];
      num[1] += pq * s[1];
      num[2] += pq * s[2];
      num[3] += pq * s[3];
    }
  }
  s_num[hb][rg][cg] = num;
  __syncthreads();

  if (valid && rg == 0) {
    f32x4 acc = s_num[hb][0][cg];
#pragma unroll
    for (int g = 1; g < SH::R; ++g) {
      const f32x4 o = s_num[hb][g][cg];
      acc[0] += o[0];
      acc[1] += o[1];
      acc[2] += o[2];
      acc[3] += o[3];
    }
    float inv = 1.f;
    if (a.normalize) {
      float den = 0.f;
#pragma unroll
      for (int wv = 0; wv < SH::WPH; ++wv) den += s_den[hb][wv];
      inv = 1.f / fmaxf(den, kEps);
    }
    const long long off = head * D + 4 * cg;
    if constexpr (sizeof(IN) == 2) {
      uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + off);
      o[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
      o[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + off) =
          f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    }
  }
}

template <int D, int DF, typename IN, int FM>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  using SH = DecodeShape<D, DF>;
  const int blocks = (a.BH + SH::HPB - 1) / SH::HPB;
  hipLaunchKernelGGL((decode_step_kernel<D, DF, IN, FM>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename IN>
static hipError_t decode_typed(const DecodeArgs& a, int D, int DF, int fmap, hipStream_t st) {
  if (fmap == kElu1) {
    switch (D) {
      case 32: return launch_decode<32, 32, IN, kElu1>(a, st);
      case 64: return launch_decode<64, 64, IN, kElu1>(a, st);
      case 128: return launch_decode<128, 128, IN, kElu1>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (fmap == kIdentity) {
    if (DF != D) return hipErrorInvalidValue;
    switch (D) {
      case 32: return launch_decode<32, 32, IN, kIdentity>(a, st);
      case 64: return launch_decode<64, 64, IN, kIdentity>(a, st);
      case 128: return launch_decode<128, 128, IN, kIdentity>(a, st);
    }
    return hipErrorInvalidValue;
  }
#define LA_PERF_CASE(d, m) \
  if (D == d && DF == m) return launch_decode<d, m, IN, kPerformer>(a, st);
  LA_PERF_CASE(32, 64) LA_PERF_CASE(32, 128)
  LA_PERF_CASE(64, 64) LA_PERF_CASE(64, 128) LA_PERF_CASE(64, 256)
  LA_PERF_CASE(128, 64) LA_PERF_CASE(128, 128)
#undef LA_PERF_CASE
  return hipErrorInvalidValue;
}

hipError_t decode_dispatch(const DecodeArgs& a, int D, int DF, int fmap, int dtype, hipStream_t st) {
  if (dtype == 1) return decode_typed<__bf16>(a, D, DF, fmap, st);
  return decode_typed<float>(a, D, DF, fmap, st);
}

// ---------------------------------------------------------------------------
// Plain state copy (N = 0 forward with a state hand-off): S_out <- S_in or 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_state_kernel(const float* S_in, const float* z_in, float* S_out,
                                                         float* z_out, long long nS, long long nz) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < nS && S_out) S_out[i] = S_in ? S_in[i] : 0.f;
  if (i < nz && z_out) z_out[i] = z_in ? z_in[i] : 0.f;
}

hipError_t copy_state_dispatch(const float* S_in, const float* z_in, float* S_out, float* z_out, long long nS,
                               long long nz, hipStream_t st) {
  const long long n = nS > nz ? nS : nz;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, S_in, z_in, S_out,
                     z_out, nS, nz);
  return hipGetLastError();
}

}  // namespace la

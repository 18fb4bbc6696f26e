// Standalone feature-map kernel: phi applied row-wise to a [rows][D] matrix.
//
// elu+1 ("Linear Transformer (Transformers are RNNs)", "La función ELU + 1"):
// elementwise, x + 1 for x > 0 and exp(x) for x <= 0, computed in fp32 and
// written in the requested output precision. It is the same device function
// the prefill and decode kernels apply to their tiles.
#include "la_device.h"
#include "la_kernels.h"

namespace la {

template <typename OUT> __device__ __forceinline__ void store8_out(void* p, long long off, const float (&x)[8]);
template <> __device__ __forceinline__ void store8_out<__bf16>(void* p, long long off, const float (&x)[8]) {
  u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p) + off) = v;
}
template <> __device__ __forceinline__ void store8_out<float>(void* p, long long off, const float (&x)[8]) {
  f32x4* q = reinterpret_cast<f32x4*>(static_cast<float*>(p) + off);
  q[0] = f32x4{x[0], x[1], x[2], x[3]};
  q[1] = f32x4{x[4], x[5], x[6], x[7]};
}

template <typename IN, typename OUT>
__global__ __launch_bounds__(256) void fmap_elu1_kernel(FmapArgs a, long long pieces) {
  for (long long p = (long long)blockIdx.x * 256 + threadIdx.x; p < pieces; p += (long long)gridDim.x * 256) {
    float x[8];
    In8<IN>::to_f32(In8<IN>::load(static_cast<const IN*>(a.x) + 8 * p), x);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = phi_elu1(x[i]);
    store8_out<OUT>(a.phi, 8 * p, x);
  }
}

template <typename IN, typename OUT>
static hipError_t launch_fmap_elu(const FmapArgs& a, int D, hipStream_t st) {
  const long long pieces = a.rows * D / 8;
  if (pieces == 0) return hipSuccess;
  long long blocks = (pieces + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((fmap_elu1_kernel<IN, OUT>), dim3((unsigned)blocks), dim3(256), 0, st, a, pieces);
  return hipGetLastError();
}

hipError_t fmap_dispatch(const FmapArgs& a, int D, int DF, int fmap, int in_dtype, int out_dtype, hipStream_t st) {
  (void)DF;
  if (fmap != kElu1) return hipErrorInvalidValue;
  if (in_dtype == 1 && out_dtype == 1) return launch_fmap_elu<__bf16, __bf16>(a, D, st);
  if (in_dtype == 1 && out_dtype == 0) return launch_fmap_elu<__bf16, float>(a, D, st);
  if (in_dtype == 0 && out_dtype == 1) return launch_fmap_elu<float, __bf16>(a, D, st);
  return launch_fmap_elu<float, float>(a, D, st);
}

}  // namespace la

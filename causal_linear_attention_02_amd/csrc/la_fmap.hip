// Standalone feature-map kernels: phi applied row-wise to a [rows][D] matrix.
//
// elu+1 ("Linear Transformer (Transformers are RNNs)", "La función ELU + 1"):
// elementwise, the same device function the prefill and decode kernels use.
// The identity map ("Linear Attention", "Mapas de características") is the
// same kernel without the map: a copy in the requested precision.
//
// Positive random features ("Linear Attention", marovi.ai, "Mapas de
// características"): phi(x) = exp(W x~ - |x~|^2 / 2) / sqrt(m), x~ = d^(-1/4) x,
// W of shape m x d. Per 64-row tile the projection U^T = W X^T runs on MFMA
// (bf16 operands for bf16 inputs, W rounded to bf16; fp32 operands for fp32
// inputs), then phi = 2^(A u - B_row) with A = d^(-1/4) log2(e) and
// B_row = log2(e) d^(-1/2) |x_row|^2 / 2 + log2(m) / 2. Output tiles are staged
// in LDS and stored as whole rows.
#include <type_traits>

#include "la_device.h"
#include "la_kernels.h"

namespace la {

constexpr int kCUs = 256;  // compute units of one MI355X

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

// elementwise maps: elu+1 or the identity (a precision-converting copy)
template <typename IN, typename OUT, int FM>
__global__ __launch_bounds__(256) void fmap_elementwise_kernel(FmapArgs a, long long pieces) {
  for (long long p = (long long)blockIdx.x * 256 + threadIdx.x; p < pieces; p += (long long)gridDim.x * 256) {
    float x[8];
    In8<IN>::to_f32(In8<IN>::load(static_cast<const IN*>(a.x) + 8 * p), x);
    if constexpr (FM == kElu1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = phi_elu1(x[i]);
    }
    store8_out<OUT>(a.phi, 8 * p, x);
  }
}

// ---------------------------------------------------------------------------
// Random-feature map. Block = 256 threads, one 64-row tile per block.
// ---------------------------------------------------------------------------
template <int D, int DF, typename OP>
struct PerfTile {
  static constexpr int RBX = D * Ops<OP>::kBytes;    // X tile rows
  static constexpr int RBW = D * Ops<OP>::kBytes;    // W rows
  static constexpr int XB = 64 * RBX;
  static constexpr int WB = DF * RBW;
};

// Stage W (fp32, [DF][D]) into LDS in operand precision.
template <int D, int DF, typename OP>
__device__ __forceinline__ void stage_W(const float* W, uint8_t* sW) {
  constexpr int RBW = PerfTile<D, DF, OP>::RBW;
  for (int p = threadIdx.x; p < DF * D / 8; p += 256) {
    const int row = p / (D / 8), col = 8 * (p % (D / 8));
    const f32x4 a = *reinterpret_cast<const f32x4*>(W + (long long)row * D + col);
    const f32x4 b = *reinterpret_cast<const f32x4*>(W + (long long)row * D + col + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    Ops<OP>::template store8<RBW>(sW, row, col, x);
  }
}

// Projection of one staged 64-row X tile: the accumulator for feature block
// fb and row block rb holds U^T[f][row] = sum_e W[f][e] X[row][e].
template <int D, int DF, typename OP>
__device__ __forceinline__ f32x16 project_tile(const uint8_t* sW, const uint8_t* sX, int fb, int rb) {
  using P = PerfTile<D, DF, OP>;
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < D / 16; ++kb)
    Ops<OP>::mma(acc, Ops<OP>::template load_rows<P::RBW>(sW, 32 * fb, 16 * kb),
                 Ops<OP>::template load_rows<P::RBX>(sX, 32 * rb, 16 * kb));
  return acc;
}

// Each block stages W once and then walks 64-row tiles blockIdx.x,
// blockIdx.x + gridDim.x, ...; the rows of the next tile are loaded into
// registers while the current tile is projected.
template <int D, int DF, typename IN, typename OUT, typename OP>
__global__ __launch_bounds__(256) void fmap_perf_kernel(FmapArgs a) {
  using P = PerfTile<D, DF, OP>;
  constexpr int RBO = DF * (int)sizeof(OUT);
  constexpr int RL = D / 8;           // threads per X row
  constexpr int XP = 64 * RL / 256;   // X pieces per thread
  static_assert(XP >= 1 && 64 * RL == 256 * XP, "X tile geometry");
  __shared__ __attribute__((aligned(16))) uint8_t sX[P::XB];
  __shared__ __attribute__((aligned(16))) uint8_t sW[P::WB];
  __shared__ __attribute__((aligned(16))) uint8_t sO[64 * RBO];
  __shared__ float sB[64];
  const long long ntiles = (a.rows + 63) / 64;
  const float s2 = 1.0f / sqrtf((float)D);                 // (d^(-1/4))^2
  const float A = sqrtf(sqrtf(1.0f / (float)D)) * 1.4426950408889634f;
  const float Bm = 0.5f * __log2f((float)DF);
  const IN* xg = static_cast<const IN*>(a.x);

  // rows of tile t held by this thread (rows past the end read as zero)
  typename In8<IN>::raw xr[XP];
  auto load_x = [&](long long t) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = threadIdx.x + 256 * i;
      const long long row = 64 * t + p / RL;
      xr[i] = row < a.rows ? In8<IN>::load(xg + row * D + 8 * (p % RL)) : In8<IN>::zero();
    }
  };
  if ((long long)blockIdx.x < ntiles) load_x(blockIdx.x);
  stage_W<D, DF, OP>(a.W, sW);

  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, li = l & 31;
  for (long long t = blockIdx.x; t < ntiles; t += gridDim.x) {
    // X tile and |x|^2 of each row
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = threadIdx.x + 256 * i;
      const int row = p / RL, col = 8 * (p % RL);
      float v[8];
      In8<IN>::to_f32(xr[i], v);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
#pragma unroll
      for (int m = 1; m < RL; m <<= 1) ss += __shfl_xor(ss, m, 64);
      if ((p % RL) == 0) sB[row] = 1.4426950408889634f * 0.5f * s2 * ss + Bm;
      Ops<OP>::template store8<P::RBX>(sX, row, col, v);
    }
    __syncthreads();
    if (t + gridDim.x < ntiles) load_x(t + gridDim.x);

    for (int u = w; u < (DF / 32) * 2; u += 4) {
      const int fb = u >> 1, rb = u & 1;
      const f32x16 acc = project_tile<D, DF, OP>(sW, sX, fb, rb);
      const int row = 32 * rb + li;
      const float b = sB[row];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = 32 * fb + 8 * g + 4 * h;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = __builtin_amdgcn_exp2f(A * acc[4 * g + j] - b);
        if constexpr (sizeof(OUT) == 2) {
          *reinterpret_cast<u32x2*>(sO + tile_off<RBO>(row, f * 2)) =
              u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        } else {
          *reinterpret_cast<f32x4*>(sO + tile_off<RBO>(row, f * 4)) = f32x4{y[0], y[1], y[2], y[3]};
        }
      }
    }
    __syncthreads();
    const int valid = (int)min(64LL, a.rows - 64 * t);
    uint8_t* o = reinterpret_cast<uint8_t*>(static_cast<OUT*>(a.phi) + 64 * t * DF);
    constexpr int OPR = RBO / 16;  // 16-byte pieces per output row
    for (int p = threadIdx.x; p < 64 * OPR; p += 256) {
      const int row = p / OPR, cb = 16 * (p % OPR);
      if (row < valid)
        *reinterpret_cast<u32x4*>(o + (long long)row * RBO + cb) =
            *reinterpret_cast<const u32x4*>(sO + tile_off<RBO>(row, cb));
    }
  }
}

template <typename IN, typename OUT, int FM>
static hipError_t launch_fmap_elementwise(const FmapArgs& a, int D, hipStream_t st) {
  const long long pieces = a.rows * D / 8;
  if (pieces == 0) return hipSuccess;
  long long blocks = (pieces + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((fmap_elementwise_kernel<IN, OUT, FM>), dim3((unsigned)blocks), dim3(256), 0, st, a, pieces);
  return hipGetLastError();
}

template <int FM>
static hipError_t fmap_elementwise_dispatch(const FmapArgs& a, int D, int in_dtype, int out_dtype, hipStream_t st) {
  if (in_dtype == 1 && out_dtype == 1) return launch_fmap_elementwise<__bf16, __bf16, FM>(a, D, st);
  if (in_dtype == 1 && out_dtype == 0) return launch_fmap_elementwise<__bf16, float, FM>(a, D, st);
  if (in_dtype == 0 && out_dtype == 1) return launch_fmap_elementwise<float, __bf16, FM>(a, D, st);
  return launch_fmap_elementwise<float, float, FM>(a, D, st);
}

template <int D, int DF, typename IN, typename OUT>
static hipError_t launch_fmap_perf(const FmapArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  using OP = typename std::conditional<sizeof(IN) == 2, __bf16, float>::type;
  using P = PerfTile<D, DF, OP>;
  // blocks that fit on the chip at once (LDS-limited), each walking several tiles
  constexpr int kLds = P::XB + P::WB + 64 * DF * (int)sizeof(OUT) + 256;
  constexpr int kPerCU = (160 * 1024) / kLds < 1 ? 1 : ((160 * 1024) / kLds > 4 ? 4 : (160 * 1024) / kLds);
  long long blocks = (a.rows + 63) / 64;
  if (blocks > (long long)kCUs * kPerCU) blocks = (long long)kCUs * kPerCU;
  hipLaunchKernelGGL((fmap_perf_kernel<D, DF, IN, OUT, OP>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename IN, typename OUT>
static hipError_t fmap_perf_dispatch(const FmapArgs& a, int D, int DF, hipStream_t st) {
#define LA_PERF_CASE(d, m) \
  if (D == d && DF == m) return launch_fmap_perf<d, m, IN, OUT>(a, st);
  LA_PERF_CASE(32, 64) LA_PERF_CASE(32, 128)
  LA_PERF_CASE(64, 64) LA_PERF_CASE(64, 128) LA_PERF_CASE(64, 256)
  LA_PERF_CASE(128, 64) LA_PERF_CASE(128, 128)
#undef LA_PERF_CASE
  return hipErrorInvalidValue;
}

hipError_t fmap_dispatch(const FmapArgs& a, int D, int DF, int fmap, int in_dtype, int out_dtype, hipStream_t st) {
  if (fmap == kElu1) return fmap_elementwise_dispatch<kElu1>(a, D, in_dtype, out_dtype, st);
  if (fmap == kIdentity) return fmap_elementwise_dispatch<kIdentity>(a, D, in_dtype, out_dtype, st);
  if (in_dtype == 1 && out_dtype == 1) return fmap_perf_dispatch<__bf16, __bf16>(a, D, DF, st);
  if (in_dtype == 1 && out_dtype == 0) return fmap_perf_dispatch<__bf16, float>(a, D, DF, st);
  if (in_dtype == 0 && out_dtype == 1) return fmap_perf_dispatch<float, __bf16>(a, D, DF, st);
  return fmap_perf_dispatch<float, float>(a, D, DF, st);
}

}  // namespace la

// Random-feature linear attention with the feature map fused into the chunked
// passes ("Linear Attention", marovi.ai, "Mapas de características" for the
// map; "Entrenamiento: forma paralela" for the blockwise form).
//
//   phi(x) = exp(W x~ - |x~|^2 / 2) / sqrt(m),   x~ = d^(-1/4) x,   W: m x d
//
// Each chunk's raw q and k rows are read once and projected on MFMA inside the
// pass (U^T = W X^T, bf16 operands, fp32 accumulation); phi = 2^(A u - B_row)
// with A = d^(-1/4) log2(e) and B_row = log2(e) d^(-1/2) |x_row|^2 / 2 +
// log2(m) / 2 goes straight into LDS as bf16, so the m-wide features never
// reach HBM.
//
// d = 64, bf16 inputs, causal.
//   state pass : local (S, z) of every segment but the last -> workspace
//                (8 waves for m >= 128, else 4; each holds one feature slice
//                of S for 32 value columns)
//   carry scan : the exclusive prefix over segments (la_prefill.hip)
//   output pass: each segment walks its chunks from its carried prefix
//                (8 waves, two per SIMD)
// In the output pass wave w < 4 holds S[fh*m/2 .. fh*m/2 + m/2)[32 cb .. 32 cb + 32)
// in MFMA accumulators (fh = w >> 1, cb = w & 1) and finishes query rows
// [32 fh, 32 fh + 32) x value columns [32 cb, 32 cb + 32) of every chunk; the
// read-out over the other feature half comes from wave w ^ 2 and the in-chunk
// term from a score wave, both through LDS.
// Layouts as in the other passes: q, k, v, out [BH][N][64]; S [BH][m][64];
// z [BH][m].
#include "la_device.h"
#include "la_kernels.h"

namespace la {
namespace {

constexpr int kPD = 64;  // head dimension of the fused kernels
using B16 = Ops<__bf16>;

template <int DF>
struct PfL {
  static constexpr int RBF = DF * 2;       // phi tile rows, bf16
  static constexpr int RBV = kPD * 2;      // v and W rows, bf16
  static constexpr int NT = DF / 64;       // S tiles per wave (m/2 features)
  static constexpr int NFB = DF / 32;      // 32-feature blocks
  static constexpr int NG = DF / 4;        // column-sum groups of 4 features
  static_assert(NT >= 1 && NG <= 256, "geometry");
};

// W (fp32 [DF][64], bf16-representable values) -> LDS rows in bf16
template <int DF, int NTH>
__device__ __forceinline__ void pf_stage_W(const float* W, uint8_t* sW) {
  for (int p = threadIdx.x; p < DF * kPD / 8; p += NTH) {
    const int row = p >> 3, col = 8 * (p & 7);
    const f32x4 a = *reinterpret_cast<const f32x4*>(W + row * kPD + col);
    const f32x4 b = *reinterpret_cast<const f32x4*>(W + row * kPD + col + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    B16::template store8<PfL<DF>::RBV>(sW, row, col, x);
  }
}

// Raw rows [row0, row0 + 32) of a chunk as the B operand of U^T = W X^T:
// lane l gets x[row0 + l % 32][16 kb + 8 (l / 32) + 0..7] for kb = 0..3.
// Rows past the descriptor's range read as zero. Each 128-byte row is read
// by four instructions (and by two waves), so these loads keep the default
// cache policy: with the non-temporal hint the output pass took 13% longer.
__device__ __forceinline__ void pf_load_x(u32x4 (&xr)[4], __amdgpu_buffer_rsrc_t r, int row0) {
  const int l = threadIdx.x & 63;
  const int off = (row0 + (l & 31)) * kPD * 2 + 16 * (l >> 5);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) xr[kb] = buf_load16(r, off + 32 * kb);
}

// v of one chunk: 512 / NTH 16-byte pieces per thread (rows p / 8, bytes 16 (p % 8))
template <int NTH>
__device__ __forceinline__ void pf_load_v(u32x4 (&vr)[512 / NTH], __amdgpu_buffer_rsrc_t r) {
#pragma unroll
  for (int i = 0; i < 512 / NTH; ++i) {
    const int p = threadIdx.x + NTH * i;
    vr[i] = buf_load16_nt(r, (p >> 3) * kPD * 2 + 16 * (p & 7));
  }
}
template <int NTH>
__device__ __forceinline__ void pf_store_v(const u32x4 (&vr)[512 / NTH], uint8_t* sV) {
#pragma unroll
  for (int i = 0; i < 512 / NTH; ++i) {
    const int p = threadIdx.x + NTH * i;
    *reinterpret_cast<u32x4*>(sV + tile_off<kPD * 2>(p >> 3, 16 * (p & 7))) = vr[i];
  }
}

// B_row of the lane's row: log2(e) d^(-1/2) |x|^2 / 2 + log2(m) / 2
__device__ __forceinline__ float pf_row_bias(const u32x4 (&xr)[4], float bm) {
  float ss = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(xr[kb][j] << 16), hi = __uint_as_float(xr[kb][j] & 0xffff0000u);
      ss += lo * lo + hi * hi;
    }
  ss += xor32(ss);
  return 1.4426950408889634f * 0.0625f * ss + bm;  // d^(-1/2) / 2 = 1/16 at d = 64
}

// U^T block for features [32 fb, 32 fb + 32): lane holds the lane's row and
// features 32 fb + 8 g + 4 (l / 32) + i in element 4 g + i
template <int DF>
__device__ __forceinline__ f32x16 pf_project(const uint8_t* sW, const u32x4 (&xr)[4], int fb) {
  f32x16 acc = {};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    B16::mma(acc, B16::template load_rows<PfL<DF>::RBV>(sW, 32 * fb, 16 * kb), __builtin_bit_cast(bf16x8, xr[kb]));
  return acc;
}

constexpr float kPfA = 1.4426950408889634f * 0.35355339059327373f;  // log2(e) * 64^(-1/4)

// phi of one projected block -> LDS tile row `row` (bf16); zero: the row is
// past the end of the sequence and gets phi = 0
template <int DF>
__device__ __forceinline__ void pf_phi_store(const f32x16& u, float b, bool zero, uint8_t* tile, int row, int fb) {
  const int h = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int f = 32 * fb + 8 * g + 4 * h;
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = zero ? 0.f : __builtin_amdgcn_exp2f(kPfA * u[4 * g + j] - b);
    *reinterpret_cast<u32x2*>(tile + tile_off<PfL<DF>::RBF>(row, f * 2)) =
        u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  }
}

// column sums of rows [sl * SLR, sl * SLR + SLR) of a phi tile for features
// [4 grp, 4 grp + 4), added into cs; NTH threads, NTH / (DF / 4) row slices
template <int DF, int NTH>
__device__ __forceinline__ void pf_colsum(const uint8_t* tile, float (&cs)[4]) {
  using L = PfL<DF>;
  constexpr int SLR = 64 / (NTH / L::NG);
  const int grp = threadIdx.x % L::NG, sl = threadIdx.x / L::NG;
#pragma unroll
  for (int r = 0; r < SLR; ++r) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(tile + tile_off<L::RBF>(sl * SLR + r, grp * 8));
    cs[0] += __uint_as_float(v[0] << 16);
    cs[1] += __uint_as_float(v[0] & 0xffff0000u);
    cs[2] += __uint_as_float(v[1] << 16);
    cs[3] += __uint_as_float(v[1] & 0xffff0000u);
  }
}

// NT accumulator tiles of S held by one wave: element r of tile t is
// S[f0 + 32 t + 8 (r / 4) + 4 (l / 32) + r % 4][32 cb + l % 32]
template <int NT>
__device__ __forceinline__ void pf_load_S(f32x16 (&st)[NT], const float* Sp, int f0, int cb) {
  const int l = threadIdx.x & 63, h = l >> 5, li = l & 31;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = f0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
      st[t][r] = Sp ? Sp[(long long)f * kPD + 32 * cb + li] : 0.f;
    }
}
template <int NT>
__device__ __forceinline__ void pf_add_S(f32x16 (&st)[NT], const float* Sp, int f0, int cb) {
  const int l = threadIdx.x & 63, h = l >> 5, li = l & 31;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = f0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
      st[t][r] += Sp[(long long)f * kPD + 32 * cb + li];
    }
}
template <int NT>
__device__ __forceinline__ void pf_store_S(const f32x16 (&st)[NT], float* Sp, int f0, int cb) {
  const int l = threadIdx.x & 63, h = l >> 5, li = l & 31;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = f0 + 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
      Sp[(long long)f * kPD + 32 * cb + li] = st[t][r];
    }
}

// S[f0 .., 32 cb ..] += phi(K)^T V over the chunk's 64 rows
template <int DF, int NT>
__device__ __forceinline__ void pf_update_S(f32x16 (&st)[NT], const uint8_t* sK, const uint8_t* sV, int f0, int cb) {
  using L = PfL<DF>;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    // one k-block at a time: keeps the operand fragments in flight (and the
    // registers they take) bounded
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 vf = B16::template load_cols<L::RBV>(sV, 16 * kb, 32 * cb);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      B16::mma(st[t], B16::template load_cols<L::RBF>(sK, 16 * kb, f0 + 32 * t), vf);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// State pass: grid (BH, segments - 1), NW waves (8 for m >= 128, else 4).
// Wave w maps rows [32 (w & 1), +32) of the chunk's k for feature slice
// w >> 1 (m / (NW / 2) features) and holds S[slice features][32 (w & 1), +32).
// ---------------------------------------------------------------------------
template <int DF, int NW>
struct PsL {
  using L = PfL<DF>;
  static constexpr int NTH = 64 * NW;
  static constexpr int FS = DF / (NW / 2);   // features per slice
  static constexpr int NTS = FS / 32;        // S tiles (and projected blocks) per wave
  static constexpr int NSL = NTH / L::NG;    // column-sum row slices
  static constexpr int K_OFF = DF * L::RBV;
  static constexpr int V_OFF = K_OFF + 64 * L::RBF;
  static constexpr int ZP_OFF = V_OFF + 64 * L::RBV;
  static constexpr int BYTES = ZP_OFF + NSL * DF * 4;
  static_assert(NTS >= 1 && FS % 32 == 0, "feature slices of whole 32-feature blocks");
  static_assert(BYTES <= 80 * 1024, "two blocks per compute unit");
};

template <int DF, int NW>
__global__ __launch_bounds__(64 * NW) void pf_state_kernel(FwdArgs a) {
  using L = PfL<DF>;
  using Q = PsL<DF, NW>;
  constexpr int NTH = Q::NTH;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Q::BYTES];
  uint8_t* sW = smem;
  uint8_t* sK = smem + Q::K_OFF;
  uint8_t* sV = smem + Q::V_OFF;
  float* zp = reinterpret_cast<float*>(smem + Q::ZP_OFF);
  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg_state;
  const int n = max(0, min(c0 + a.chunks_per_seg_state, a.nchunks) - c0);
  const long long base = (long long)bh * a.N;
  const __bf16* k = static_cast<const __bf16*>(a.k);
  const __bf16* v = static_cast<const __bf16*>(a.v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, li = l & 31;
  const int rb = w & 1, sl = w >> 1;  // rows [32 rb, +32); feature slice [sl FS, +FS)
  const int cb = w & 1;               // S columns [32 cb, +32)
  const float bm = 0.5f * __log2f((float)DF);

  u32x4 xr[4], vr[512 / NTH];
  auto rsrc = [&](const __bf16* p, int c) {
    return make_rsrc(p + (base + 64LL * c) * kPD, (unsigned)(min(64, a.N - 64 * c) * kPD * 2));
  };
  if (n > 0) {
    pf_load_x(xr, rsrc(k, c0), 32 * rb);
    pf_load_v<NTH>(vr, rsrc(v, c0));
  }
  pf_stage_W<DF, NTH>(a.W, sW);
  f32x16 st[Q::NTS];
#pragma unroll
  for (int t = 0; t < Q::NTS; ++t) st[t] = f32x16{};
  float cs[4] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  for (int it = 0; it < n; ++it) {
    const int c = c0 + it;
    const int valid = min(64, a.N - 64 * c);
    const float b = pf_row_bias(xr, bm);
    const bool past = 32 * rb + li >= valid;
#pragma unroll
    for (int j = 0; j < Q::NTS; ++j) {
      const int fb = sl * Q::NTS + j;
      pf_phi_store<DF>(pf_project<DF>(sW, xr, fb), b, past, sK, 32 * rb + li, fb);
    }
    pf_store_v<NTH>(vr, sV);
    if (it + 1 < n) {
      pf_load_x(xr, rsrc(k, c + 1), 32 * rb);
      pf_load_v<NTH>(vr, rsrc(v, c + 1));
    }
    __syncthreads();
    pf_update_S<DF, Q::NTS>(st, sK, sV, sl * Q::FS, cb);
    pf_colsum<DF, NTH>(sK, cs);
    __syncthreads();
  }

  float* out = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
  pf_store_S<Q::NTS>(st, out, sl * Q::FS, cb);
  {
    const int grp = threadIdx.x % L::NG, zs = threadIdx.x / L::NG;
    *reinterpret_cast<f32x4*>(zp + zs * DF + 4 * grp) = f32x4{cs[0], cs[1], cs[2], cs[3]};
  }
  __syncthreads();
  if (threadIdx.x < DF) {
    float s = 0.f;
#pragma unroll
    for (int zs = 0; zs < Q::NSL; ++zs) s += zp[zs * DF + threadIdx.x];
    out[DF * kPD + threadIdx.x] = s;
  }
}

// ---------------------------------------------------------------------------
// Output pass: grid (BH, segments), 512 threads (two waves per SIMD). Per
// chunk, two barriers:
//   1. all waves map the chunk: waves 0-3 q, waves 4-7 k; wave w takes rows
//      [32 (w & 1), +32) and features [((w >> 1) & 1) m/2, +m/2); every
//      thread stages one piece of v. After the barrier all threads store the
//      previous chunk's output tile as whole rows.
//   2. state waves 0-3 (fh, cb): read-out of both row blocks over their
//      feature half (the other row block handed to wave w ^ 2), S update;
//      score waves 4-7 (r, cb): masked scores of row block r, their product
//      with v[:, 32 cb, +32), the in-chunk denominator and phi(q_i) . z over
//      half of the features; all threads: column sums of phi(K)
//   3. after the second barrier, state wave (fh, cb) adds the hand-overs,
//      normalizes and writes rows [32 fh, +32) x columns [32 cb, +32) into the
//      LDS output tile, and z moves on; then it maps the next chunk, while the
//      score waves may already be mapping theirs (nothing of steps 1-2 is read
//      in step 3).
// ---------------------------------------------------------------------------
template <int DF>
struct PoL {
  using L = PfL<DF>;
  static constexpr int NSL = 512 / L::NG;                 // column-sum row slices
  static constexpr int W_OFF = 0;
  static constexpr int Q_OFF = W_OFF + DF * L::RBV;
  static constexpr int K_OFF = Q_OFF + 64 * L::RBF;
  static constexpr int V_OFF = K_OFF + 64 * L::RBF;
  static constexpr int R_OFF = V_OFF + 64 * L::RBV;       // read-out hand-over [4 waves][4][64 lanes] f32x4
  static constexpr int A_OFF = R_OFF + 4 * 64 * 16 * 4;   // score-wave products with v, same layout
  static constexpr int ZP_OFF = A_OFF + 4 * 64 * 16 * 4;  // column-sum partials [NSL][DF]
  static constexpr int Z_OFF = ZP_OFF + NSL * DF * 4;     // running z [2][DF]
  static constexpr int DEN_OFF = Z_OFF + 2 * DF * 4;      // phi(q_i) . z per feature half [2][64]
  static constexpr int DP_OFF = DEN_OFF + 2 * 64 * 4;     // in-chunk denominators [64]
  static constexpr int Y_OFF = DP_OFF + 64 * 4;           // output tile [64][64] bf16
  static constexpr int BYTES = Y_OFF + 64 * L::RBV;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ void pf_put16(float* base, int slot, const f32x16& x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<f32x4*>(base + ((slot * 4 + j) * 64 + l) * 4) = f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
}
__device__ __forceinline__ void pf_add16(const float* base, int slot, f32x16& x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 o = *reinterpret_cast<const f32x4*>(base + ((slot * 4 + j) * 64 + l) * 4);
    x[4 * j] += o[0];
    x[4 * j + 1] += o[1];
    x[4 * j + 2] += o[2];
    x[4 * j + 3] += o[3];
  }
}

template <int DF>
__global__ __launch_bounds__(512) void pf_output_kernel(FwdArgs a) {
  using L = PfL<DF>;
  using O = PoL<DF>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[O::BYTES];
  uint8_t* sW = smem + O::W_OFF;
  uint8_t* sQ = smem + O::Q_OFF;
  uint8_t* sK = smem + O::K_OFF;
  uint8_t* sV = smem + O::V_OFF;
  float* sR = reinterpret_cast<float*>(smem + O::R_OFF);
  float* sA = reinterpret_cast<float*>(smem + O::A_OFF);
  float* zp = reinterpret_cast<float*>(smem + O::ZP_OFF);
  float* sZ = reinterpret_cast<float*>(smem + O::Z_OFF);
  float* sDen = reinterpret_cast<float*>(smem + O::DEN_OFF);
  float* sDp = reinterpret_cast<float*>(smem + O::DP_OFF);
  uint8_t* sY = smem + O::Y_OFF;

  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int n = max(0, min(c0 + a.chunks_per_seg, a.nchunks) - c0);
  const long long base = (long long)bh * a.N;
  const __bf16* q = static_cast<const __bf16*>(a.q);
  const __bf16* k = static_cast<const __bf16*>(a.k);
  const __bf16* v = static_cast<const __bf16*>(a.v);
  __bf16* out = static_cast<__bf16*>(a.out);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, li = l & 31;
  // mapping roles
  const bool qwave = w < 4;
  const int rb = w & 1, ph = (w >> 1) & 1;
  // chunk roles: state waves (fh, cb), score waves (r, cb)
  const bool swave = w < 4;
  const int fh = (w >> 1) & 1, cb = w & 1;
  const float bm = 0.5f * __log2f((float)DF);

  const float* Sinit;
  const float* zinit;
  if (a.init_from_ws) {
    const float* s = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
    Sinit = s;
    zinit = s + DF * kPD;
  } else {
    Sinit = a.S_in ? a.S_in + (long long)bh * DF * kPD : nullptr;
    zinit = a.z_in ? a.z_in + (long long)bh * DF : nullptr;
  }

  u32x4 xr[4], vr[1];
  auto rsrc = [&](const __bf16* p, int c) {
    return make_rsrc(p + (base + 64LL * c) * kPD, (unsigned)(min(64, a.N - 64 * c) * kPD * 2));
  };
  if (n > 0) {
    pf_load_x(xr, rsrc(qwave ? q : k, c0), 32 * rb);
    pf_load_v<512>(vr, rsrc(v, c0));
  }
  pf_stage_W<DF, 512>(a.W, sW);
  if (threadIdx.x < DF) {
    float z0 = zinit ? zinit[threadIdx.x] : 0.f;
    if (a.init_sum_ws)  // local sums of the segments before this one
      for (int j = 0; j < seg; ++j) z0 += a.ws[((long long)bh * a.ws_slots + j) * a.state_elems + DF * kPD + threadIdx.x];
    sZ[threadIdx.x] = z0;
  }

  // 1. feature map of chunk it (all waves), then the loads of chunk it + 1
  auto map_chunk = [&](int it) {
    const int c = c0 + it;
    const int valid = min(64, a.N - 64 * c);
    const float b = pf_row_bias(xr, bm);
    const int row = 32 * rb + li;
    if (qwave) {
#pragma unroll 1
      for (int j = 0; j < L::NFB / 2; ++j) {
        const int fb = ph * (L::NFB / 2) + j;
        pf_phi_store<DF>(pf_project<DF>(sW, xr, fb), b, false, sQ, row, fb);
      }
    } else {
      const bool past = row >= valid;
#pragma unroll 1
      for (int j = 0; j < L::NFB / 2; ++j) {
        const int fb = ph * (L::NFB / 2) + j;
        pf_phi_store<DF>(pf_project<DF>(sW, xr, fb), b, past, sK, row, fb);
      }
    }
    pf_store_v<512>(vr, sV);
    if (it + 1 < n) {
      pf_load_x(xr, rsrc(qwave ? q : k, c + 1), 32 * rb);
      pf_load_v<512>(vr, rsrc(v, c + 1));
    }
  };
  // the output tile of chunk it (staged in sY) as whole rows, one 16-byte
  // piece per thread; rows past the end are dropped by the range check
  auto flush_y = [&](int it) {
    const int c = c0 + it;
    const auto ro = make_rsrc(out + (base + 64LL * c) * kPD, (unsigned)(min(64, a.N - 64 * c) * kPD * 2));
    const int p = threadIdx.x;
    buf_store16_nt(ro, (p >> 3) * kPD * 2 + 16 * (p & 7),
                   *reinterpret_cast<const u32x4*>(sY + tile_off<kPD * 2>(p >> 3, 16 * (p & 7))));
  };
  // column sums of the chunk's phi(K), partials over row slices
  auto colsum = [&]() {
    float cs[4] = {0.f, 0.f, 0.f, 0.f};
    pf_colsum<DF, 512>(sK, cs);
    const int grp = threadIdx.x % L::NG, sl = threadIdx.x / L::NG;
    *reinterpret_cast<f32x4*>(zp + sl * DF + 4 * grp) = f32x4{cs[0], cs[1], cs[2], cs[3]};
  };

  // The two roles run separate loops with the same three barriers per chunk,
  // so that the state tiles take registers in the state waves only.
  if (swave) {
    f32x16 st[L::NT];
    pf_load_S<L::NT>(st, Sinit, fh * (DF / 2), cb);
    if (a.init_sum_ws)
      for (int j = 0; j < seg; ++j)
        pf_add_S<L::NT>(st, a.ws + ((long long)bh * a.ws_slots + j) * a.state_elems, fh * (DF / 2), cb);
    __syncthreads();
    for (int it = 0; it < n; ++it) {
      map_chunk(it);
      __syncthreads();
      if (it > 0) flush_y(it - 1);
      // ---- 2. read-out over the wave's feature half, then the S update ----
      f32x16 num;
      {
        f32x16 R0 = {}, R1 = {};
#pragma unroll
        for (int t = 0; t < L::NT; ++t)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const bf16x8 sf = B16::from_acc(st[t], kb2);
            const int f0 = fh * (DF / 2) + 32 * t + 16 * kb2;
            B16::mma(R0, sf, B16::template load_rows<L::RBF>(sQ, 0, f0));
            B16::mma(R1, sf, B16::template load_rows<L::RBF>(sQ, 32, f0));
          }
        // row block 1 - fh goes to state wave w ^ 2, which finishes it
        pf_put16(sR, w, fh ? R0 : R1);
        num = fh ? R1 : R0;
      }
      pf_update_S<DF, L::NT>(st, sK, sV, fh * (DF / 2), cb);
      colsum();
      __syncthreads();
      // ---- 3. finish rows [32 fh, +32) x columns [32 cb, +32); move z on ----
      pf_add16(sR, w ^ 2, num);
      pf_add16(sA, 2 * fh + cb, num);
      const int i = 32 * fh + li;
      float inv = 1.f;
      if (a.normalize) inv = 1.f / fmaxf(sDp[i] + sDen[i] + sDen[64 + i], kEps);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<u32x2*>(sY + tile_off<kPD * 2>(i, (32 * cb + 8 * g + 4 * h) * 2)) =
            u32x2{pack_bf16x2(num[4 * g] * inv, num[4 * g + 1] * inv),
                  pack_bf16x2(num[4 * g + 2] * inv, num[4 * g + 3] * inv)};
      if (threadIdx.x < DF) {  // state waves hold threads 0..255 >= DF - 1
        const float* zc = sZ + (it & 1) * DF;
        float s = zc[threadIdx.x];
#pragma unroll
        for (int sl = 0; sl < O::NSL; ++sl) s += zp[sl * DF + threadIdx.x];
        sZ[((it + 1) & 1) * DF + threadIdx.x] = s;
      }
    }
    __syncthreads();  // the last output tile is complete
    if (n > 0) flush_y(n - 1);
    if (a.S_out && seg == a.nseg - 1) {
      pf_store_S<L::NT>(st, a.S_out + (long long)bh * DF * kPD, fh * (DF / 2), cb);
      if (threadIdx.x < DF) a.z_out[(long long)bh * DF + threadIdx.x] = sZ[(n & 1) * DF + threadIdx.x];
    }
  } else {
    __syncthreads();
    const int r = fh;  // query row block of this score wave
    for (int it = 0; it < n; ++it) {
      map_chunk(it);
      __syncthreads();
      if (it > 0) flush_y(it - 1);
      // ---- 2. A[j][i] for keys j of block 0 (and block 1 when r = 1) and
      // queries i of block r; lane holds query i = 32 r + li ----
      f32x16 Aa = {}, Ab = {};
#pragma unroll 4
      for (int kb = 0; kb < DF / 16; ++kb) {
        const bf16x8 bq = B16::template load_rows<L::RBF>(sQ, 32 * r, 16 * kb);
        B16::mma(Aa, B16::template load_rows<L::RBF>(sK, 0, 16 * kb), bq);
        if (r) B16::mma(Ab, B16::template load_rows<L::RBF>(sK, 32, 16 * kb), bq);
      }
      float dpart = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int jt = 8 * (e >> 2) + 4 * h + (e & 3);
        const bool keep = jt <= li;
        if (r) {
          Ab[e] = keep ? Ab[e] : 0.f;
          dpart += Aa[e] + Ab[e];
        } else {
          Aa[e] = keep ? Aa[e] : 0.f;
          dpart += Aa[e];
        }
      }
      dpart += xor32(dpart);
      if (cb == 0 && h == 0) sDp[32 * r + li] = dpart;
      {
        // phi(q_i) . z for the rows of block r over features
        // [cb m/2 + h m/4, +m/4) (bf16 phi(q) from LDS), halves added across
        // lanes l and l ^ 32; z after the previous chunk
        const float* zc = sZ + (it & 1) * DF;
        const int i = 32 * r + li, f0 = cb * (DF / 2) + h * (DF / 4);
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < DF / 32; ++u) {
          const u32x4 qv = *reinterpret_cast<const u32x4*>(sQ + tile_off<L::RBF>(i, (f0 + 8 * u) * 2));
          const f32x4 z0 = *reinterpret_cast<const f32x4*>(zc + f0 + 8 * u);
          const f32x4 z1 = *reinterpret_cast<const f32x4*>(zc + f0 + 8 * u + 4);
          dot += __uint_as_float(qv[0] << 16) * z0[0] + __uint_as_float(qv[0] & 0xffff0000u) * z0[1] +
                 __uint_as_float(qv[1] << 16) * z0[2] + __uint_as_float(qv[1] & 0xffff0000u) * z0[3] +
                 __uint_as_float(qv[2] << 16) * z1[0] + __uint_as_float(qv[2] & 0xffff0000u) * z1[1] +
                 __uint_as_float(qv[3] << 16) * z1[2] + __uint_as_float(qv[3] & 0xffff0000u) * z1[3];
        }
        dot += xor32(dot);
        if (h == 0) sDen[cb * 64 + i] = dot;
      }
      f32x16 av = {};
#pragma unroll
      for (int kbj = 0; kbj < 2; ++kbj)
        B16::mma(av, B16::template load_cols<L::RBV>(sV, 16 * kbj, 32 * cb), B16::from_acc(Aa, kbj));
      if (r) {
#pragma unroll
        for (int kbj = 0; kbj < 2; ++kbj)
          B16::mma(av, B16::template load_cols<L::RBV>(sV, 32 + 16 * kbj, 32 * cb), B16::from_acc(Ab, kbj));
      }
      pf_put16(sA, w - 4, av);
      colsum();
      __syncthreads();
    }
    __syncthreads();  // the last output tile is complete
    if (n > 0) flush_y(n - 1);
  }
}

template <int DF>
hipError_t launch_pf(const FwdArgs& a, const ScanArgs& s, hipStream_t st, hipEvent_t* ev) {
  constexpr int NW = DF >= 128 ? 8 : 4;
  if (a.run_state_pass)
    hipLaunchKernelGGL((pf_state_kernel<DF, NW>), dim3(a.BH, a.nseg_state), dim3(64 * NW), 0, st, a);
  if (ev) (void)hipEventRecord(ev[1], st);
  if (a.run_scan) {
    const hipError_t e = scan_dispatch(s, st);
    if (e != hipSuccess) return e;
  }
  if (ev) (void)hipEventRecord(ev[2], st);
  hipLaunchKernelGGL(pf_output_kernel<DF>, dim3(a.BH, a.nseg), dim3(512), 0, st, a);
  if (ev) (void)hipEventRecord(ev[3], st);
  return hipGetLastError();
}

}  // namespace

bool perf_fused_supported(int D, int DF, int dtype, bool causal, bool decay) {
  return D == kPD && (DF == 64 || DF == 128 || DF == 256) && dtype == 1 && causal && !decay;
}

hipError_t perf_fused_dispatch(const FwdArgs& a, const ScanArgs& s, int DF, hipStream_t st, hipEvent_t* ev) {
  switch (DF) {
    case 64: return launch_pf<64>(a, s, st, ev);
    case 128: return launch_pf<128>(a, s, st, ev);
    case 256: return launch_pf<256>(a, s, st, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace la

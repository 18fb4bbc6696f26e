// Gated linear attention on gfx950: the chunked causal forward with a
// per-token, per-channel gate on the feature dimension.
//
// "Linear Attention" (marovi.ai), "Variantes y extensiones", GLA item: the
// scalar decay is replaced by a gate that depends on the data. Read here as
//   S_t = diag(alpha_t) S_{t-1} + phi(k_t) v_t^T,  z_t = alpha_t * z_{t-1} + phi(k_t),
//   y_t = phi(q_t)^T S_t / max(phi(q_t).z_t, eps)   (or the numerator alone),
// with the gates given as log-gates lg = log(alpha) in [-log 4, 0].
//
// Blockwise ("Entrenamiento: forma paralela"): inside a chunk of 64 tokens
// let lam_r = lg_0 + ... + lg_r (per channel, in-chunk prefix). Key j enters
// row i through channel f with weight exp(lam_if - lam_jf) (j <= i), the
// state carried into the chunk with exp(lam_if), and the chunk moves it on
// as S <- diag(exp(lam_63)) S + sum_j diag(exp(lam_63 - lam_j)) phi(k_j) v_j^T.
// With c = 32 the output pass stages
//   Qh[r][f] = phi(q_r)_f exp(lam_rf - lam_cf),  Kh[r][f] = phi(k_r)_f exp(lam_cf - lam_rf),
// so Qh Kh^T carries exactly those weights, and it scales the carried state
// by exp(lam_c) before the readout (the carried term of row i is
// Qh_i . diag(exp(lam_c)) S) and by exp(lam_63 - lam_c) after adding Kh^T V.
// With alpha >= 1/4 no factor exceeds exp(32 log 4) = 2^64.
//
// Passes (the forward's segment split, P segments of whole chunks):
//   gla_state_kernel : local (S, z) of every segment but the last, relative to
//                      the segment's end, and the segment's total log-gate
//   carry scan       : P_{s+1} = diag(exp(total_s)) P_s + local_s (la_prefill.hip)
//   gla_output_kernel: every segment from its carried state
// All waves load and stage (no producer/consumer split); d' = d.
#include "la_device.h"
#include "la_kernels.h"

namespace la {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kCenter = 32;

template <int FM>
__device__ __forceinline__ float gphi(float x) {
  if constexpr (FM == kElu1) return phi_elu1(x);
  else return x;
}
__device__ __forceinline__ float exp_nat(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

template <typename IN, typename OP, int RB>
__device__ __forceinline__ void put_raw_g(uint8_t* tile, int row, int col, const typename In8<IN>::raw& r) {
  static_assert(sizeof(IN) == sizeof(OP), "raw staging needs matching element types");
  if constexpr (sizeof(IN) == 2) {
    *reinterpret_cast<u32x4*>(tile + tile_off<RB>(row, col * 2)) = r;
  } else {
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4)) = r.a;
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4 + 16)) = r.b;
  }
}

// sum over the lanes of a wave that share lane % RL
template <int RL>
__device__ __forceinline__ float colsum_lanes(float x) {
#pragma unroll
  for (int s = RL; s < 64; s <<= 1) x += __shfl_xor(x, s, 64);
  return x;
}

// In-chunk prefix of the log-gates: lam[r][f] = lg_0f + ... + lg_rf for the
// 64 rows of the chunk (fp32). The gate tile is loaded in 16-byte row pieces
// into lam; then NT/D threads per channel scan it in place, each over
// 64*D/NT consecutive rows, and add the totals of the rows before theirs.
// Rows past the end of the sequence load as 0 (buffer range check), so lam
// stays at its last value there. tot: NT/D x D scratch. Three barriers.
// A log-gate outside [log(1/4), 0] becomes NaN (checked_log_gate), so the
// prefix of its channel is NaN from its row on, and raises the status flag.
template <int D, int NT>
__device__ __forceinline__ void gate_prefix(const float* lg, long long row0, int valid, float* lam, float* tot,
                                            int* flag) {
  constexpr int NQ = NT / D, RPQ = 64 / NQ, NPC = 16 * D / NT;  // pieces of 4 per thread
  const int t = threadIdx.x, col = t % D, qt = t / D;
  const auto R = make_rsrc(lg + row0 * D, (unsigned)(valid * D * 4));
  f32x4 p[NPC];
#pragma unroll
  for (int i = 0; i < NPC; ++i) p[i] = __builtin_bit_cast(f32x4, buf_load16(R, (t + NT * i) * 16));
#pragma unroll
  for (int i = 0; i < NPC; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) p[i][e] = checked_log_gate(p[i][e], flag);
    *reinterpret_cast<f32x4*>(lam + 4 * (t + NT * i)) = p[i];
  }
  __syncthreads();
  float run = 0.f;
  for (int r = 0; r < RPQ; ++r) {
    float* x = lam + (qt * RPQ + r) * D + col;
    run += *x;
    *x = run;
  }
  tot[qt * D + col] = run;
  __syncthreads();
  float off = 0.f;
  for (int q2 = 0; q2 < qt; ++q2) off += tot[q2 * D + col];
  if (qt > 0) {
    for (int r = 0; r < RPQ; ++r) lam[(qt * RPQ + r) * D + col] += off;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// State pass: local state of every segment with a successor, relative to the
// segment's end: S_loc = sum_j diag(exp(Lam_end - Lam_j)) phi(k_j) v_j^T (z
// alike), and the segment's total log-gate per channel (lfac[bh][seg][f]).
// Per chunk S <- diag(exp(lam_63)) S + Kt^T V with Kt[r] = phi(k_r) exp(lam_63 - lam_r) <= phi(k_r).
// grid = (BH, P - 1), block = 2*D threads; wave w owns S[:, 32w:32w+32].
// ---------------------------------------------------------------------------
template <int D, typename OP, typename IN, int FM>
__global__ __launch_bounds__(D * 2) void gla_state_kernel(GatedArgs g) {
  using Frag = typename Ops<OP>::frag;
  constexpr int NW = D / 32, NT = 2 * D, RL = D / 8;
  constexpr int RB = D * Ops<OP>::kBytes, TB = 64 * RB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TB];
  __shared__ __attribute__((aligned(16))) float lam[64 * D];
  __shared__ float tot[(NT / D) * D];
  __shared__ float zsum[NW][D];
  __shared__ float f63[D];  // per channel exp(lam_63)
  uint8_t* sK = smem;
  uint8_t* sV = smem + TB;
  const FwdArgs& a = g.f;
  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg_state;
  const int n = max(0, min(c0 + a.chunks_per_seg_state, a.nchunks) - c0);
  const int t = threadIdx.x, w = t >> 6, l = t & 63, h = l >> 5, li = l & 31;
  const long long base = (long long)bh * a.N;
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  const int col = 8 * (t % RL);

  f32x16 S[NW];
#pragma unroll
  for (int fb = 0; fb < NW; ++fb) S[fb] = f32x16{};
  float zr[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float ltot = 0.f;  // thread t < D: the segment's total log-gate of channel t
  for (int m = 0; m < n; ++m) {
    const int c = c0 + m;
    const int valid = min(64, a.N - 64 * c);
    const long long row0 = base + 64LL * c;
    const unsigned bytes = (unsigned)(valid * D * (int)sizeof(IN));
    const auto Rk = make_rsrc(k + row0 * D, bytes);
    const auto Rv = make_rsrc(v + row0 * D, bytes);
    typename In8<IN>::raw rk[4], rv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = ((t / RL + 16 * i) * D + col) * (int)sizeof(IN);
      rk[i] = In8<IN>::bload(Rk, o);
      rv[i] = In8<IN>::bload(Rv, o);
    }
    gate_prefix<D, NT>(g.log_gates, row0, valid, lam, tot, g.f.status_flag);
    float l63[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      l63[e] = lam[63 * D + col + e];
      zr[e] *= exp_nat(l63[e]);
    }
    if (t < D) {
      ltot += lam[63 * D + t];
      f63[t] = exp_nat(lam[63 * D + t]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t / RL + 16 * i;
      float x[8];
      In8<IN>::to_f32(rk[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = row < valid ? gphi<FM>(x[e]) * exp_nat(l63[e] - lam[row * D + col + e]) : 0.f;
        zr[e] += x[e];
      }
      Ops<OP>::template store8<RB>(sK, row, col, x);
      put_raw_g<IN, OP, RB>(sV, row, col, rv[i]);
    }
    __syncthreads();
    // S <- diag(exp(lam_63)) S + Kt^T V
#pragma unroll
    for (int fb = 0; fb < NW; ++fb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[fb][r] *= f63[32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const Frag vf = Ops<OP>::template load_cols<RB>(sV, 16 * kb, 32 * w);
#pragma unroll
      for (int fb = 0; fb < NW; ++fb) Ops<OP>::mma(S[fb], Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * fb), vf);
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) zr[e] = colsum_lanes<RL>(zr[e]);
  if (l < RL) {
#pragma unroll
    for (int e = 0; e < 8; ++e) zsum[w][col + e] = zr[e];
  }
  __syncthreads();
  float* st = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
#pragma unroll
  for (int fb = 0; fb < NW; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st[(long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li] = S[fb][r];
  for (int f = t; f < D; f += NT) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += zsum[ww][f];
    st[D * D + f] = s;
  }
  if (t < D) g.lfac[((long long)bh * a.nseg + seg) * D + t] = ltot;
}

// ---------------------------------------------------------------------------
// Output pass. grid = (BH, P), block = 4*D threads: wave (ib, w) handles
// query rows [32 ib, 32 ib + 32) of the chunk and value columns [32 w,
// 32 w + 32), keeping S[:, 32w:32w+32] (rows = features) in accumulators;
// threads t < D keep z_t.
// ---------------------------------------------------------------------------
template <int D, typename OP, typename IN, int FM>
__global__ __launch_bounds__(D * 4) void gla_output_kernel(GatedArgs g) {
  using Frag = typename Ops<OP>::frag;
  constexpr int NW = D / 32, NT = 4 * D, RL = D / 8, NWAVE = NT / 64;
  constexpr int RB = D * Ops<OP>::kBytes, TB = 64 * RB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * TB];
  __shared__ __attribute__((aligned(16))) float lam[64 * D];
  __shared__ float tot[(NT / D) * D];
  __shared__ float zpart[NWAVE][D];
  __shared__ __attribute__((aligned(16))) float zc[D];  // exp(lam_c) z of the state entering the chunk
  __shared__ float fc[D], fe[D];                         // per channel: exp(lam_c), exp(lam_63 - lam_c)
  uint8_t* sQ = smem;
  uint8_t* sK = smem + TB;
  uint8_t* sV = smem + 2 * TB;
  const FwdArgs& a = g.f;
  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int n = max(0, min(c0 + a.chunks_per_seg, a.nchunks) - c0);
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, h = l >> 5, li = l & 31;
  const int ib = wave / NW, w = wave % NW;
  const long long base = (long long)bh * a.N;
  const IN* q = static_cast<const IN*>(a.q);
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  IN* out = static_cast<IN*>(a.out);
  const int col = 8 * (t % RL);

  const float* Sinit;
  const float* zinit;
  if (a.init_from_ws) {
    Sinit = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
    zinit = Sinit + D * D;
  } else {
    Sinit = a.S_in ? a.S_in + (long long)bh * D * D : nullptr;
    zinit = a.z_in ? a.z_in + (long long)bh * D : nullptr;
  }
  f32x16 S[NW];
#pragma unroll
  for (int fb = 0; fb < NW; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      S[fb][r] = Sinit ? Sinit[(long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li] : 0.f;
  float zreg = (t < D && zinit) ? zinit[t] : 0.f;

  for (int m = 0; m < n; ++m) {
    const int c = c0 + m;
    const int valid = min(64, a.N - 64 * c);
    const long long row0 = base + 64LL * c;
    const unsigned bytes = (unsigned)(valid * D * (int)sizeof(IN));
    const auto Rq = make_rsrc(q + row0 * D, bytes);
    const auto Rk = make_rsrc(k + row0 * D, bytes);
    const auto Rv = make_rsrc(v + row0 * D, bytes);
    typename In8<IN>::raw rq[2], rk[2], rv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int o = ((t / RL + 32 * i) * D + col) * (int)sizeof(IN);
      rq[i] = In8<IN>::bload(Rq, o);
      rk[i] = In8<IN>::bload(Rk, o);
      rv[i] = In8<IN>::bload(Rv, o);
    }
    gate_prefix<D, NT>(g.log_gates, row0, valid, lam, tot, g.f.status_flag);
    // stage Qh, Kh (rows past the end: 0), V; column sums of Kh
    float lc[8], cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lc[e] = lam[kCenter * D + col + e];
      cs[e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = t / RL + 32 * i;
      float xq[8], xk[8];
      In8<IN>::to_f32(rq[i], xq);
      In8<IN>::to_f32(rk[i], xk);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = exp_nat(lam[row * D + col + e] - lc[e]);
        xq[e] = gphi<FM>(xq[e]) * f;
        xk[e] = row < valid ? gphi<FM>(xk[e]) * __builtin_amdgcn_rcpf(f) : 0.f;
        cs[e] += xk[e];
      }
      Ops<OP>::template store8<RB>(sQ, row, col, xq);
      Ops<OP>::template store8<RB>(sK, row, col, xk);
      put_raw_g<IN, OP, RB>(sV, row, col, rv[i]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = colsum_lanes<RL>(cs[e]);
    if (l < RL) {
#pragma unroll
      for (int e = 0; e < 8; ++e) zpart[wave][col + e] = cs[e];
    }
    __syncthreads();
    // z: the carried part exp(lam_c) z for this chunk's readout, then the
    // state leaving it, exp(lam_63 - lam_c) (exp(lam_c) z + colsum Kh)
    if (t < D) {
      float s = 0.f;
#pragma unroll
      for (int ww = 0; ww < NWAVE; ++ww) s += zpart[ww][t];
      const float lct = lam[kCenter * D + t];
      const float ec = exp_nat(lct), ee = exp_nat(lam[63 * D + t] - lct);
      fc[t] = ec;
      fe[t] = ee;
      const float zcar = ec * zreg;
      zc[t] = zcar;
      zreg = ee * (zcar + s);
    }
    __syncthreads();
    // S' = diag(exp(lam_c)) S
#pragma unroll
    for (int fb = 0; fb < NW; ++fb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[fb][r] *= fc[32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)];

    // scores A[j][i] for the wave's query rows (key blocks 0..ib), numerator
    f32x16 num = {};
    float den = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      if (jb > ib) break;
      f32x16 A = {};
      // partial unroll: full unrolling hoists every fragment load and spills
#pragma unroll 2
      for (int kb = 0; kb < D / 16; ++kb)
        Ops<OP>::mma(A, Ops<OP>::template load_rows<RB>(sK, 32 * jb, 16 * kb),
                     Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 16 * kb));
      if (jb == ib) {
#pragma unroll
        for (int r = 0; r < 16; ++r) A[r] = 8 * (r >> 2) + 4 * h + (r & 3) <= li ? A[r] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) den += A[r];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Ops<OP>::mma(num, Ops<OP>::template load_cols<RB>(sV, 32 * jb + 16 * kk, 32 * w), Ops<OP>::from_acc(A, kk));
    }
#pragma unroll
    for (int fb = 0; fb < NW; ++fb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        Ops<OP>::mma(num, Ops<OP>::from_acc(S[fb], kk), Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 32 * fb + 16 * kk));
    // carried denominator Qh_i . zc over this lane half's features
    const int irow = 32 * ib + li;
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {  // D/2 features per lane half, 4 at a time
      const int f0 = (D / 2) * h + 4 * u;
      float x[4];
      if constexpr (sizeof(OP) == 2) {
        const u32x2 p = *reinterpret_cast<const u32x2*>(sQ + tile_off<RB>(irow, f0 * 2));
        x[0] = __uint_as_float(p[0] << 16);
        x[1] = __uint_as_float(p[0] & 0xffff0000u);
        x[2] = __uint_as_float(p[1] << 16);
        x[3] = __uint_as_float(p[1] & 0xffff0000u);
      } else {
        const f32x4 p = *reinterpret_cast<const f32x4*>(sQ + tile_off<RB>(irow, f0 * 4));
        x[0] = p[0];
        x[1] = p[1];
        x[2] = p[2];
        x[3] = p[3];
      }
      const f32x4 zz = *reinterpret_cast<const f32x4*>(zc + f0);
      den += x[0] * zz[0] + x[1] * zz[1] + x[2] * zz[2] + x[3] * zz[3];
    }
    den += xor32(den);
    const float inv = a.normalize ? 1.f / fmaxf(den, kEps) : 1.f;
    if (irow < valid) {
      IN* o = out + (row0 + irow) * D + 32 * w + 4 * h;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float y0 = num[4 * gq] * inv, y1 = num[4 * gq + 1] * inv;
        const float y2 = num[4 * gq + 2] * inv, y3 = num[4 * gq + 3] * inv;
        if constexpr (sizeof(IN) == 2) {
          *reinterpret_cast<u32x2*>(o + 8 * gq) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        } else {
          *reinterpret_cast<f32x4*>(o + 8 * gq) = f32x4{y0, y1, y2, y3};
        }
      }
    }
    // S <- diag(exp(lam_63 - lam_c)) (S' + Kh^T V)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const Frag vf = Ops<OP>::template load_cols<RB>(sV, 16 * kb, 32 * w);
#pragma unroll
      for (int fb = 0; fb < NW; ++fb) Ops<OP>::mma(S[fb], Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * fb), vf);
    }
#pragma unroll
    for (int fb = 0; fb < NW; ++fb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[fb][r] *= fe[32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)];
    __syncthreads();
  }
  if (a.S_out && seg == a.nseg - 1) {
    if (ib == 0) {
#pragma unroll
      for (int fb = 0; fb < NW; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          a.S_out[(long long)bh * D * D + (long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li] =
              S[fb][r];
    }
    if (t < D) a.z_out[(long long)bh * D + t] = zreg;
  }
}

template <int D, typename T, int FM>
hipError_t launch_gated(const GatedArgs& g, const ScanArgs& s, hipStream_t st) {
  if (g.f.run_state_pass)
    hipLaunchKernelGGL((gla_state_kernel<D, T, T, FM>), dim3(g.f.BH, g.f.nseg_state), dim3(2 * D), 0, st, g);
  if (g.f.run_scan) {
    const hipError_t e = scan_dispatch(s, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gla_output_kernel<D, T, T, FM>), dim3(g.f.BH, g.f.nseg), dim3(4 * D), 0, st, g);
  return hipGetLastError();
}

template <typename T, int FM>
hipError_t gated_d(const GatedArgs& g, const ScanArgs& s, int D, hipStream_t st) {
  switch (D) {
    case 32: return launch_gated<32, T, FM>(g, s, st);
    case 64: return launch_gated<64, T, FM>(g, s, st);
    case 128: return launch_gated<128, T, FM>(g, s, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gated_dispatch(const GatedArgs& g, const ScanArgs& s, int D, int fmap, int dtype, hipStream_t st) {
  if (dtype == 1) {
    if (fmap == kElu1) return gated_d<__bf16, kElu1>(g, s, D, st);
    if (fmap == kIdentity) return gated_d<__bf16, kIdentity>(g, s, D, st);
  } else {
    if (fmap == kElu1) return gated_d<float, kElu1>(g, s, D, st);
    if (fmap == kIdentity) return gated_d<float, kIdentity>(g, s, D, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace la

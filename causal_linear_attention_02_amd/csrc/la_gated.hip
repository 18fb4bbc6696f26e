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
// With c = 31 (lam_c is the first half's total) the output pass stages
//   Qh[r][f] = phi(q_r)_f exp(lam_rf - lam_cf),  Kh[r][f] = phi(k_r)_f exp(lam_cf - lam_rf),
// so Qh Kh^T carries exactly those weights, and it scales the carried state
// by exp(lam_c) before the readout (the carried term of row i is
// Qh_i . diag(exp(lam_c)) S) and by exp(lam_63 - lam_c) after adding Kh^T V.
// With alpha >= 1/4 no factor exceeds exp(32 log 4) = 2^64.
//
// Passes (each sequence split into P segments of whole chunks; d' = d):
//   gla_state_kernel : local (S, z) of every segment but the last, relative to
//                      the segment's end, and the segment's total log-gate
//   carry scan       : P_{s+1} = diag(exp(total_s)) P_s + local_s (la_prefill.hip)
//   gla_output_kernel: every segment from its carried state; producer waves
//                      stage the gated q, k tiles while consumer waves run
//                      the previous chunk's products. Where the split needs
//                      two rounds of workgroups it takes two of the state
//                      pass's segments at a time (GatedArgs::seg_stride).
// Both passes load the next chunk while they stage the current one.
#include "la_device.h"
#include "la_kernels.h"

namespace la {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int FM>
__device__ __forceinline__ float gphi(float x) {
  if constexpr (FM == kElu1) return phi_elu1(x);
  else return x;
}
__device__ __forceinline__ float exp_nat(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Cross-lane moves of the gate layout below: DPP inside a 16-lane row and
// the gfx950 row swaps between rows run on the vector ALU, where a shuffle
// through ds_bpermute costs an LDS round trip and its address arithmetic.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kRowShr = 0x110;  // + s: the value of lane l - s of the same row (0 before the row's start)
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kMirror = 0x140;
constexpr int kRor4 = 0x124;
constexpr int kRor8 = 0x128;
// the value of lane l ^ 16
__device__ __forceinline__ float xor16(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // even rows receive the odd row above in s[1]; odd rows the even row below in s[0]
  return __uint_as_float((threadIdx.x & 16) ? s[0] : s[1]);
}
// 4 consecutive input elements: raw form (one buffer load) and fp32
template <typename IN> struct In4;
template <> struct In4<__bf16> {
  using raw = u32x2;  // 8 bytes
  __device__ static raw bload(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
  }
  __device__ static void to_f32(const raw& r, float (&x)[4]) {
    x[0] = __uint_as_float(r[0] << 16);
    x[1] = __uint_as_float(r[0] & 0xffff0000u);
    x[2] = __uint_as_float(r[1] << 16);
    x[3] = __uint_as_float(r[1] & 0xffff0000u);
  }
};
template <> struct In4<float> {
  using raw = f32x4;  // 16 bytes
  __device__ static raw bload(__amdgpu_buffer_rsrc_t r, int voff) { return __builtin_bit_cast(f32x4, buf_load16(r, voff)); }
  __device__ static void to_f32(const raw& r, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = r[i];
  }
};

// 4 fp32 values of a row (columns col .. col+3) into a swizzled operand tile
template <typename OP, int RB>
__device__ __forceinline__ void store4(uint8_t* tile, int row, int col, const float (&x)[4]) {
  if constexpr (sizeof(OP) == 2) {
    *reinterpret_cast<u32x2*>(tile + tile_off<RB>(row, col * 2)) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  } else {
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4)) = f32x4{x[0], x[1], x[2], x[3]};
  }
}
// The same, and x becomes the values as the tile holds them (bf16: rounded)
template <typename OP, int RB>
__device__ __forceinline__ void store4_held(uint8_t* tile, int row, int col, float (&x)[4]) {
  if constexpr (sizeof(OP) == 2) {
    const u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *reinterpret_cast<u32x2*>(tile + tile_off<RB>(row, col * 2)) = pk;
    x[0] = __uint_as_float(pk[0] << 16);
    x[1] = __uint_as_float(pk[0] & 0xffff0000u);
    x[2] = __uint_as_float(pk[1] << 16);
    x[3] = __uint_as_float(pk[1] & 0xffff0000u);
  } else {
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4)) = f32x4{x[0], x[1], x[2], x[3]};
  }
}

// Thread layout of the gated passes' loads and staging: NT threads over a
// 64 x D chunk. Thread t holds channels [4 g, 4 g + 4) of the R consecutive
// rows [R j, R j + R) (row block j of channel group g). A wave holds GW = R
// channel groups of all J row blocks, lane l = g % GW + GW j: the 16 lanes of
// a DPP row then hold 16 / GW row blocks of 4 GW consecutive channels, so a
// load of those lanes covers 2 (or 4) row pieces of 64 (or 32) bytes rather
// than 8 (or 16) pieces of 16. The in-chunk prefix of the log-gates is a sum
// in registers over R rows and a scan over the J lanes of the group, GW apart.
template <int D, int NT>
struct GMap {
  static constexpr int CG = D / 4, J = NT / CG, R = 64 / J, GW = R;
  static constexpr int PR = 16 / GW;  // row blocks of a group in one DPP row
  static_assert(NT % 64 == 0 && CG == NT / 64 * GW && (J == 8 || J == 16), "gate layout");
  __device__ static int group(int t) { return (t >> 6) * GW + (t & 63) % GW; }
  __device__ static int block(int t) { return (t & 63) / GW; }
};

// The value rows need no gate, so they take a layout of their own: thread t
// holds the 16-byte units i NT + t (i < NU) of the chunk's rows, so that a
// wave's load covers whole rows. Unit i goes out with row i EVERY of the gate
// layout.
template <int D, int NT, typename IN>
struct VMap {
  static constexpr int UPR = D * (int)sizeof(IN) / 16;  // 16-byte units per row
  static constexpr int NU = 64 * UPR / NT;              // units per thread
  static constexpr int EVERY = GMap<D, NT>::R / NU;
  static_assert(NU >= 1 && NU * NT == 64 * UPR && GMap<D, NT>::R % NU == 0, "value layout");
};

// Registers of one chunk: log-gates, k (and q) in the gate layout, v in its own.
template <int D, int NT, typename IN, bool Q>
struct GSet {
  static constexpr int R = GMap<D, NT>::R;
  f32x4 lg[R];
  typename In4<IN>::raw q[Q ? R : 1], k[R];
  u32x4 v[VMap<D, NT, IN>::NU];
};

// Loads of the chunk at rows [row0, row0 + valid); rows past `valid` read as
// zero through the descriptors' range check (log-gate 0: the prefix stays at
// its last value there). `valid` must be wave-uniform.
struct GRsrc {
  __amdgpu_buffer_rsrc_t g, q, k, v;
};
template <int D, typename IN>
__device__ __forceinline__ GRsrc grsrc(const float* lg, const IN* q, const IN* k, const IN* v, long long row0,
                                       int valid) {
  const unsigned eb = (unsigned)(valid * D * (int)sizeof(IN));
  return GRsrc{make_rsrc(lg + row0 * D, (unsigned)(valid * D * 4)), make_rsrc(q ? q + row0 * D : q, eb),
               make_rsrc(k + row0 * D, eb), make_rsrc(v + row0 * D, eb)};
}
// row e of the thread's rows
template <int D, int NT, typename IN, bool Q>
__device__ __forceinline__ void gload_row(GSet<D, NT, IN, Q>& s, const GRsrc& r, int e, int t) {
  using M = GMap<D, NT>;
  const int gi = M::group(t), j = M::block(t);
  const int el = (M::R * j + e) * D + 4 * gi;
  s.lg[e] = __builtin_bit_cast(f32x4, buf_load16(r.g, el * 4));
  if constexpr (Q) s.q[e] = In4<IN>::bload(r.q, el * (int)sizeof(IN));
  s.k[e] = In4<IN>::bload(r.k, el * (int)sizeof(IN));
  using V = VMap<D, NT, IN>;
  if (e % V::EVERY == 0) s.v[e / V::EVERY] = buf_load16(r.v, 16 * ((e / V::EVERY) * NT + t));
}
// Row e's share of the value units into the swizzled value tile
template <int D, int NT, typename IN, int RB, bool Q>
__device__ __forceinline__ void stage_v(uint8_t* sV, const GSet<D, NT, IN, Q>& s, int e, int t) {
  using V = VMap<D, NT, IN>;
  static_assert(RB == 16 * V::UPR, "value tile rows hold the input rows");
  if (e % V::EVERY == 0) {
    const int u = (e / V::EVERY) * NT + t;
    *reinterpret_cast<u32x4*>(sV + tile_off<RB>(u / V::UPR, 16 * (u % V::UPR))) = s.v[e / V::EVERY];
  }
}
template <int D, int NT, typename IN, bool Q>
__device__ __forceinline__ void gload(GSet<D, NT, IN, Q>& s, const float* lg, const IN* q, const IN* k, const IN* v,
                                      long long row0, int valid, int t) {
  const GRsrc r = grsrc<D, IN>(lg, q, k, v, row0, valid);
#pragma unroll
  for (int e = 0; e < GMap<D, NT>::R; ++e) gload_row<D, NT, IN, Q>(s, r, e, t);
}

// In-chunk prefix of the log-gates, in place: p[e][c] becomes
// lam = lg_0 + ... + lg_r at row r = R j + e, channel 4 g + c (fp32); every
// lane of the group also gets lam at rows 31 and 63 (half and whole). A
// log-gate outside [log(1/4), 0] becomes NaN (checked_log_gate), so the
// prefix of its channel is NaN from its row on, and raises the status flag.
// The thread's values are checked at once through their NaN-propagating
// minimum and maximum; only a thread holding a bad one checks them one by one.
template <int D, int NT, int NR>
__device__ __forceinline__ void gate_scan(f32x4 (&p)[NR], int* flag, int t, f32x4& half, f32x4& whole) {
  using M = GMap<D, NT>;
  static_assert(NR == M::R, "rows per thread");
  float mn = p[0][0], mx = p[0][0];
#pragma unroll
  for (int e = 0; e < M::R; ++e)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mn = __builtin_elementwise_minimum(mn, p[e][c]);
      mx = __builtin_elementwise_maximum(mx, p[e][c]);
    }
  if (!(mn >= kMinLogFactor && mx <= 0.f)) {
#pragma unroll
    for (int e = 0; e < M::R; ++e)
#pragma unroll
      for (int c = 0; c < 4; ++c) p[e][c] = checked_log_gate(p[e][c], flag);
  }
#pragma unroll
  for (int e = 1; e < M::R; ++e) p[e] += p[e - 1];
  // the sum of the group's row blocks before this one: first over the
  // blocks in this lane's DPP row (GW lanes apart), then over the rows before
  // it (the row totals through the row swaps). A row shift gives 0 where its
  // source lies before the row's start, which masks the first blocks; no
  // shift sits under a lane condition (a DPP read from a lane that the
  // condition switched off would read nothing).
  const int row = (t >> 4) & 3;
  f32x4 off;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float x = p[M::R - 1][c];
    float ex, tot;
    if constexpr (M::PR == 2) {
      ex = dpp<kRowShr + 8>(x);
      tot = x + dpp<kRor8>(x);
    } else {
      float inc = x + dpp<kRowShr + 4>(x);
      inc += dpp<kRowShr + 8>(inc);
      ex = dpp<kRowShr + 4>(inc);
      tot = x + dpp<kRor4>(x);
      tot += dpp<kRor8>(tot);
    }
    const float below = xor16(tot);         // rows 1, 3: the total of rows 0, 2
    const float pair = tot + below;         // rows 0+1 or 2+3
    const float other = xor32(pair);        // rows 2, 3: the total of rows 0+1
    off[c] = ex + ((row & 1) ? below : 0.f) + ((row & 2) ? other : 0.f);
    half[c] = (row & 2) ? other : pair;     // rows 0+1: row blocks 0 .. J/2 - 1
    whole[c] = pair + other;
  }
#pragma unroll
  for (int e = 0; e < M::R; ++e) p[e] += off;
}

// sum over the J row blocks of a channel group (lanes GW apart)
template <int J>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(J == 8 || J == 16, "gate layout");
  if constexpr (J == 16) x += dpp<kRor4>(x);
  x += dpp<kRor8>(x);
  x += xor16(x);
  return x + xor32(x);
}
// sum over the channel groups of a wave that hold the same rows (GW = 64 / J
// consecutive lanes)
template <int J>
__device__ __forceinline__ float across_groups(float x) {
  static_assert(J == 8 || J == 16, "gate layout");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  if constexpr (J == 8) x += dpp<kHalfMirror>(x);
  return x;
}

// ---------------------------------------------------------------------------
// State pass: local state of every segment with a successor, relative to the
// segment's end: S_loc = sum_j diag(exp(Lam_end - Lam_j)) phi(k_j) v_j^T (z
// alike), and the segment's total log-gate per channel (lfac[bh][seg][f]).
// Per chunk S <- diag(exp(lam_63)) S + Kt^T V with Kt[r] = phi(k_r) exp(lam_63 - lam_r) <= phi(k_r).
// grid = (BH, P - 1), block = 2*D threads; wave w owns S[:, 32w:32w+32].
// The next chunk's rows are loaded while this one is staged (row by row, in
// the registers just freed) and multiplied; two LDS buffers leave one
// barrier per chunk.
// ---------------------------------------------------------------------------
// two workgroups per CU where the LDS holds two (bf16 tiles)
template <int D, typename OP, typename IN, int FM>
__global__ __launch_bounds__(D * 2, (sizeof(IN) == 2 ? 2 : 1)) void gla_state_kernel(GatedArgs g) {
  constexpr int NW = D / 32, NT = 2 * D;
  using M = GMap<D, NT>;
  constexpr int R = M::R, J = M::J;
  constexpr int RB = D * Ops<OP>::kBytes, TB = 64 * RB;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2 * TB];
  __shared__ __attribute__((aligned(16))) float f63[2][D];  // per channel exp(lam_63)
  const FwdArgs& a = g.f;
  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg_state;
  const int n = max(0, min(c0 + a.chunks_per_seg_state, a.nchunks) - c0);
  const int t = threadIdx.x, w = t >> 6, l = t & 63, h = l >> 5, li = l & 31;
  const int gi = M::group(t), j = M::block(t);
  const long long base = (long long)bh * a.N;
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);

  f32x16 S[NW];
#pragma unroll
  for (int fb = 0; fb < NW; ++fb) S[fb] = f32x16{};
  float zr[4] = {0.f, 0.f, 0.f, 0.f};    // this lane's rows' part of z, channels 4 gi + c
  float ltot[4] = {0.f, 0.f, 0.f, 0.f};  // the segment's total log-gate, channels 4 gi + c

  auto load = [&](int m, GSet<D, NT, IN, false>& s) {
    const int c = min(c0 + m, a.nchunks - 1);
    const int valid = __builtin_amdgcn_readfirstlane(m < n ? min(64, a.N - 64 * c) : 0);
    gload<D, NT, IN, false>(s, g.log_gates, nullptr, k, v, base + 64LL * c, valid, t);
  };
  GSet<D, NT, IN, false> cur;
  auto step = [&](int m) {
    const int valid = __builtin_amdgcn_readfirstlane(min(64, a.N - 64 * (c0 + m)));
    // chunk m + 1 (none past the segment): each row's registers take its
    // row as soon as they are staged, so its loads go out during the staging
    const int cn = min(c0 + m + 1, a.nchunks - 1);
    const int vn = __builtin_amdgcn_readfirstlane(m + 1 < n ? min(64, a.N - 64 * cn) : 0);
    const GRsrc nr = grsrc<D, IN>(g.log_gates, static_cast<const IN*>(nullptr), k, v, base + 64LL * cn, vn);
    uint8_t* sK = smem[m & 1];
    uint8_t* sV = sK + TB;
    float* fb63 = f63[m & 1];
    f32x4 l31, l63;
    gate_scan<D, NT>(cur.lg, a.status_flag, t, l31, l63);
    f32x4 e63;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ltot[c] += l63[c];
      e63[c] = exp_nat(l63[c]);
      zr[c] *= e63[c];
    }
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int row = R * j + e;
      // rows past the end (zero k and log-gates: finite products) times 0,
      // without a branch around the exponentials
      const float keep = row < valid ? 1.f : 0.f;
      float x[4];
      In4<IN>::to_f32(cur.k[e], x);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[c] = gphi<FM>(x[c]) * exp_nat(l63[c] - cur.lg[e][c]) * keep;
        zr[c] += x[c];
      }
      store4<OP, RB>(sK, row, 4 * gi, x);
      stage_v<D, NT, IN, RB>(sV, cur, e, t);
      gload_row<D, NT, IN, false>(cur, nr, e, t);
    }
    if (j == 0) *reinterpret_cast<f32x4*>(fb63 + 4 * gi) = e63;
    __syncthreads();
    // S <- diag(exp(lam_63)) S + Kt^T V
#pragma unroll
    for (int fb = 0; fb < NW; ++fb)
#pragma unroll
      for (int r = 0; r < 16; ++r) S[fb][r] *= fb63[32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const auto vf = Ops<OP>::template load_cols<RB>(sV, 16 * kb, 32 * w);
#pragma unroll
      for (int fb = 0; fb < NW; ++fb) Ops<OP>::mma(S[fb], Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * fb), vf);
    }
  };
  load(0, cur);
  for (int m = 0; m < n; ++m) step(m);
  float* st = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
#pragma unroll
  for (int fb = 0; fb < NW; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st[(long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li] = S[fb][r];
#pragma unroll
  for (int c = 0; c < 4; ++c) zr[c] = group_sum<J>(zr[c]);
  if (j == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      st[D * D + 4 * gi + c] = zr[c];
      g.lfac[((long long)bh * g.lfac_stride + seg) * D + 4 * gi + c] = ltot[c];
    }
  }
}

// ---------------------------------------------------------------------------
// Output pass. grid = (BH, P), block = 64 (NW + NWP) threads in two roles:
//   producers (NWP waves): load chunk m + 1 while they stage chunk m: the
//     in-chunk gate prefix, Qh and Kh, V, the column sums of Kh (the lanes of
//     channel group g keep z of channels [4 g, 4 g + 4)), the factors
//     exp(lam_c) and exp(lam_63 - lam_c), and each producer wave's part of
//     the carried denominator Qh_i . exp(lam_c) z of every row;
//   consumers (D/32 waves): wave w keeps S[:, 32w:32w+32] (rows = features)
//     in accumulators and, for both 32-row blocks of chunk m - 1, forms the
//     scores, both numerator terms and the denominator, writes the output
//     rows and moves S on.
// Step it: the producers stage chunk it while the consumers compute chunk
// it - 1 from the other LDS buffer; one barrier per step hands them over
// (two where one buffer is all that fits).
// ---------------------------------------------------------------------------
// Producer waves of the output pass: two per consumer wave where the
// registers allow it (d <= 64: the producers' vector work is the longer
// chain), one at d = 128 (three waves per SIMD would leave the consumers too
// few registers; measured 900 against 746 us on B1 H16 N65536).
template <int D>
constexpr int gla_producer_waves() { return (D == 128 ? 1 : 2) * D / 32; }
template <int D>
constexpr int gla_output_threads() { return 64 * (D / 32 + gla_producer_waves<D>()); }

template <int D, typename OP, typename IN, int FM>
__global__ __launch_bounds__(gla_output_threads<D>()) void gla_output_kernel(GatedArgs g) {
  constexpr int NW = D / 32;       // consumer waves = value blocks = feature blocks
  constexpr int NWP = gla_producer_waves<D>();
  // consumer loops unrolled where the registers allow it (one producer wave
  // per consumer wave)
  constexpr int UNR = NWP == NW ? 2 : 1, UNR4 = NWP == NW ? 4 : 1;
  constexpr int NTP = 64 * NWP;    // producer threads
  using M = GMap<D, NTP>;
  constexpr int R = M::R, J = M::J;
  constexpr int RB = D * Ops<OP>::kBytes, TB = 64 * RB;
  // output staging: each consumer wave's 32 x 32 block of a row block, rows
  // padded by 16 bytes (the lanes of one write then fall in distinct banks)
  constexpr int YRS = 32 * (int)sizeof(IN) + 16, YST = NW * 32 * YRS;
  constexpr int NBUF = 2 * (3 * TB + 2 * D * 4 + NWP * 64 * 4) + YST <= 160 * 1024 ? 2 : 1;
  // Two register sets of prefetched rows where they fit (bf16): the next
  // chunk's loads go out before this one is staged. With one set they go out
  // after it, during the consumers' products.
  constexpr int PSETS = sizeof(IN) == 2 && D <= 64 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF][3 * TB];
  // per buffer and channel: exp(lam_c) and exp(lam_63 - lam_c)
  __shared__ __attribute__((aligned(16))) float fac[NBUF][2][D];
  // per buffer: each producer wave's part of the carried denominator of every row
  __shared__ float dpart[NBUF][NWP][64];
  __shared__ __attribute__((aligned(16))) uint8_t ystage[YST];
  const FwdArgs& a = g.f;
  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int n = max(0, min(c0 + a.chunks_per_seg, a.nchunks) - c0);
  const int t = threadIdx.x, l = t & 63, h = l >> 5, li = l & 31;
  // the wave index in a scalar register: the role branches stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const long long base = (long long)bh * a.N;
  const IN* q = static_cast<const IN*>(a.q);
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  IN* out = static_cast<IN*>(a.out);

  const float* Sinit;
  const float* zinit;
  if (a.init_from_ws) {
    Sinit = a.ws + ((long long)bh * a.ws_slots + seg * g.seg_stride) * a.state_elems;
    zinit = Sinit + D * D;
  } else {
    Sinit = a.S_in ? a.S_in + (long long)bh * D * D : nullptr;
    zinit = a.z_in ? a.z_in + (long long)bh * D : nullptr;
  }

  if (wave >= NW) {
    // ------------------------------------------------------------ producers
    const int p = t - 64 * NW, pw = wave - NW;
    const int gi = M::group(p), j = M::block(p);
    float zreg[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) zreg[c] = zinit ? zinit[4 * gi + c] : 0.f;
    auto rsrc_of = [&](int m) {
      const int c = min(c0 + m, a.nchunks - 1);
      const int valid = __builtin_amdgcn_readfirstlane(m < n ? min(64, a.N - 64 * c) : 0);
      return grsrc<D, IN>(g.log_gates, q, k, v, base + 64LL * c, valid);
    };
    auto load = [&](int m, GSet<D, NTP, IN, true>& s) {
      const GRsrc r = rsrc_of(m);
#pragma unroll
      for (int e = 0; e < R; ++e) gload_row<D, NTP, IN, true>(s, r, e, p);
    };
    // With one register set (PSETS == 1) each row's registers take the same
    // row of chunk m + 1 as soon as it is staged: the next chunk's loads go
    // out during the staging rather than after it.
    auto stage = [&](int m, GSet<D, NTP, IN, true>& cur) {
      const GRsrc nr = rsrc_of(m + 1);
      const int valid = __builtin_amdgcn_readfirstlane(min(64, a.N - 64 * (c0 + m)));
      uint8_t* sQ = smem[m % NBUF];
      uint8_t* sK = sQ + TB;
      uint8_t* sV = sK + TB;
      // lam_c = lam_31 (the first half's total), lam_63 (the chunk's)
      f32x4 lc, l63;
      gate_scan<D, NTP>(cur.lg, a.status_flag, p, lc, l63);
      float cs[4] = {0.f, 0.f, 0.f, 0.f};
      // the carried part exp(lam_c) z for this chunk's readout (its dot
      // products with the staged Qh rows form the carried denominator)
      f32x4 ec, ee, zcar;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ec[c] = exp_nat(lc[c]);
        zcar[c] = ec[c] * zreg[c];
      }
      float dq[R];
#pragma unroll
      for (int e = 0; e < R; ++e) {
        const int row = R * j + e;
        const float keep = row < valid ? 1.f : 0.f;  // key rows past the end, without a branch
        float xq[4], xk[4];
        In4<IN>::to_f32(cur.q[e], xq);
        In4<IN>::to_f32(cur.k[e], xk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float f = exp_nat(cur.lg[e][c] - lc[c]);
          xq[c] = gphi<FM>(xq[c]) * f;
          xk[c] = gphi<FM>(xk[c]) * __builtin_amdgcn_rcpf(f) * keep;
          cs[c] += xk[c];
        }
        store4_held<OP, RB>(sQ, row, 4 * gi, xq);  // xq: Qh as the operand holds it
        store4<OP, RB>(sK, row, 4 * gi, xk);
        stage_v<D, NTP, IN, RB>(sV, cur, e, p);
        dq[e] = xq[0] * zcar[0] + xq[1] * zcar[1] + xq[2] * zcar[2] + xq[3] * zcar[3];
        if constexpr (PSETS == 1) gload_row<D, NTP, IN, true>(cur, nr, e, p);
      }
      // the wave's GW channel groups (consecutive lanes) hold the same rows
#pragma unroll
      for (int e = 0; e < R; ++e) dq[e] = across_groups<J>(dq[e]);
      if (l % M::GW == 0) {
#pragma unroll
        for (int e = 0; e < R; ++e) dpart[m % NBUF][pw][R * j + e] = dq[e];
      }
      // the state leaving the chunk, exp(lam_63 - lam_c) (exp(lam_c) z + colsum Kh)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cs[c] = group_sum<J>(cs[c]);
        ee[c] = exp_nat(l63[c] - lc[c]);
        zreg[c] = ee[c] * (zcar[c] + cs[c]);
      }
      if (j == 0) {
        *reinterpret_cast<f32x4*>(&fac[m % NBUF][0][4 * gi]) = ec;
        *reinterpret_cast<f32x4*>(&fac[m % NBUF][1][4 * gi]) = ee;
      }
    };
    // step it: stage chunk it (if any) and load chunk it + 1; one barrier
    // (two with one buffer: the consumers first finish chunk it - 1)
    auto pstep = [&](int it, GSet<D, NTP, IN, true>& cur, GSet<D, NTP, IN, true>& nxt) {
      if constexpr (PSETS == 2) load(it + 1, nxt);
      if constexpr (NBUF == 1) __syncthreads();
      if (it < n) stage(it, cur);
      __syncthreads();
    };
    if constexpr (PSETS == 2) {
      GSet<D, NTP, IN, true> A, B;
      load(0, A);
      for (int it = 0; it <= n; it += 2) {
        pstep(it, A, B);
        if (it + 1 <= n) pstep(it + 1, B, A);
      }
    } else {
      GSet<D, NTP, IN, true> A;
      load(0, A);
      for (int it = 0; it <= n; ++it) pstep(it, A, A);
    }
    if (a.S_out && seg == a.nseg - 1 && j == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) a.z_out[(long long)bh * D + 4 * gi + c] = zreg[c];
    }
  } else {
    // ------------------------------------------------------------ consumers
    const int w = wave;
    f32x16 S[NW];
#pragma unroll
    for (int fb = 0; fb < NW; ++fb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        S[fb][r] = Sinit ? Sinit[(long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li] : 0.f;
    auto compute = [&](int m) {
      const int valid = __builtin_amdgcn_readfirstlane(min(64, a.N - 64 * (c0 + m)));
      const long long row0 = base + 64LL * (c0 + m);
      const uint8_t* sQ = smem[m % NBUF];
      const uint8_t* sK = sQ + TB;
      const uint8_t* sV = sK + TB;
      const float* fc = fac[m % NBUF][0];
      const float* fe = fac[m % NBUF][1];
      // S' = diag(exp(lam_c)) S
#pragma unroll
      for (int fb = 0; fb < NW; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[fb][r] *= fc[32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll UNR
      for (int rb = 0; rb < 2; ++rb) {
        // scores A[j][i] of query block rb (key blocks 0..rb), numerator
        f32x16 num = {};
        float den = 0.f;
#pragma unroll UNR
        for (int jb = 0; jb <= rb; ++jb) {
          f32x16 A = {};
          // partial unroll: full unrolling hoists every fragment load
#pragma unroll 2
          for (int kb = 0; kb < D / 16; ++kb)
            Ops<OP>::mma(A, Ops<OP>::template load_rows<RB>(sK, 32 * jb, 16 * kb),
                         Ops<OP>::template load_rows<RB>(sQ, 32 * rb, 16 * kb));
          if (jb == rb) {
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
            Ops<OP>::mma(num, Ops<OP>::from_acc(S[fb], kk),
                         Ops<OP>::template load_rows<RB>(sQ, 32 * rb, 32 * fb + 16 * kk));
        // carried denominator: the producer waves' parts (added by one lane half)
        const int irow = 32 * rb + li;
        if (h == 0) {
#pragma unroll
          for (int ww = 0; ww < NWP; ++ww) den += dpart[m % NBUF][ww][irow];
        }
        den += xor32(den);
        const float inv = a.normalize ? 1.f / fmaxf(den, kEps) : 1.f;
        // lane (li, h) holds row li, columns 8 gq + 4 h + 0..3 of the wave's
        // 32: written to the wave's LDS block and read back by rows, so that
        // every store covers whole 32-column row pieces (rows past the end
        // fall outside the descriptor's range)
        uint8_t* ys = ystage + w * 32 * YRS;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const float y0 = num[4 * gq] * inv, y1 = num[4 * gq + 1] * inv;
          const float y2 = num[4 * gq + 2] * inv, y3 = num[4 * gq + 3] * inv;
          uint8_t* yp = ys + li * YRS + (8 * gq + 4 * h) * (int)sizeof(IN);
          if constexpr (sizeof(IN) == 2)
            *reinterpret_cast<u32x2*>(yp) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
          else
            *reinterpret_cast<f32x4*>(yp) = f32x4{y0, y1, y2, y3};
        }
        // the block is the wave's own: its LDS operations complete in order,
        // so the fences only keep the compiler from moving the reads above
        // the writes (and, after the stores, the next block's writes above
        // these reads)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
          constexpr int UPR = 2 * (int)sizeof(IN);  // 16-byte units per row piece
          constexpr int RPP = 64 / UPR;             // rows per pass of the wave
          const auto ro = make_rsrc(out + row0 * D, (unsigned)(valid * D * (int)sizeof(IN)));
#pragma unroll
          for (int i = 0; i < 32 / RPP; ++i) {
            const int rr = RPP * i + l / UPR, u = l % UPR;
            buf_store16_nt(ro, ((32 * rb + rr) * D + 32 * w) * (int)sizeof(IN) + 16 * u,
                           *reinterpret_cast<const u32x4*>(ys + rr * YRS + 16 * u));
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      // S <- diag(exp(lam_63 - lam_c)) (S' + Kh^T V)
#pragma unroll UNR4
      for (int kb = 0; kb < 4; ++kb) {
        const auto vf = Ops<OP>::template load_cols<RB>(sV, 16 * kb, 32 * w);
#pragma unroll
        for (int fb = 0; fb < NW; ++fb)
          Ops<OP>::mma(S[fb], Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * fb), vf);
      }
#pragma unroll
      for (int fb = 0; fb < NW; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[fb][r] *= fe[32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)];
    };
    // step it: chunk it - 1 (if any); the producers' barriers, one or two a step
    for (int it = 0; it <= n; ++it) {
      if (it >= 1) compute(it - 1);
      if constexpr (NBUF == 1) __syncthreads();
      __syncthreads();
    }
    if (a.S_out && seg == a.nseg - 1) {
#pragma unroll
      for (int fb = 0; fb < NW; ++fb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          a.S_out[(long long)bh * D * D + (long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li] =
              S[fb][r];
    }
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
  hipLaunchKernelGGL((gla_output_kernel<D, T, T, FM>), dim3(g.f.BH, g.f.nseg), dim3(gla_output_threads<D>()), 0, st,
                     g);
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

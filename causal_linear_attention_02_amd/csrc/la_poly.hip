// Degree-2 polynomial feature map ("Linear Attention", "Mapas de
// características", polynomial bullet): phi(x) = (1, x, x (x) x), truncated
// at degree 2 with unit coefficients and the d x d block row-major, so that
// phi(q).phi(k) = 1 + q.k + (q.k)^2 and d' = 1 + d + d^2 (1057 at d = 32,
// 4161 at d = 64). State rows: 0 the constant, 1 + b the linear part,
// 1 + d + a d + b the quadratic part.
//
// Chunked forward. The quadratic part of the state, S2[a][b][e] =
// sum_j k_ja k_jb v_je (d^3 floats, 1 MB per head at d = 64), never leaves
// the compute units: it is split over the workgroups of one (batch, head) by
// value-column block E (32 columns) and by a range of a, and every wave
// keeps four 32 x 32 fp32 tiles S2[a][32bb..][32E..] in accumulators for the
// whole sequence. Per chunk a wave reads out
//   y_i[E] += sum_a q_ia (sum_b q_ib S2[a][b][E])     (MFMA over b, q_ia on the result)
// and updates
//   S2[a][b][E] += sum_j k_jb (k_ja v_j[E])            (MFMA over j, k_ja on the values).
// The low-degree state (S0 = sum v, S1 = sum k v^T) and the normalizer state
// (n, z1 = sum k, Z2 = sum k k^T) are small; they sit in LDS in the first
// two workgroups of each value block, where a few waves read them out and
// update them beside their own tiles, and form the in-chunk part with the
// kernel applied to the scores, A_ij = 1 + s_ij + s_ij^2 (j <= i). So a head
// takes exactly NE * NA workgroups, one per compute unit. Every workgroup
// walks the chunks in order and writes its partial numerators (fp32) to the
// workspace, and some write partial denominators; a last kernel sums the
// partials and divides. Non-causal: every chunk updates first, then every
// chunk reads out the total.
#include "la_device.h"
#include "la_kernels.h"

namespace la {
namespace {

template <int D>
struct PolyCfg {
  static constexpr int NW = D / 8;      // waves per workgroup (4 at d = 32, 8 at d = 64)
  static constexpr int NT = 64 * NW;    // threads: one 8-element piece of a 64-row chunk each
  static constexpr int NBB = D / 32;    // 32-row b-blocks per a
  static constexpr int NE = D / 32;     // 32-column value blocks
  static constexpr int APW = 4 / NBB;   // a values per wave (four tiles)
  static constexpr int APB = NW * APW;  // a values per workgroup
  static constexpr int NA = D / APB;    // workgroups per value block
  static constexpr int DP = 1 + D + D * D;
  // in-chunk part: its own workgroup (hb = 2) with one score tile per wave
  // when there are more than two workgroups per value block; else it shares
  // workgroup 0 and one wave takes both tiles of the second row block, whose
  // row sums then need no extra denominator slot
  static constexpr bool SPLIT = NA > 2;
  static constexpr int NDEN = 1 + NE + (SPLIT ? 1 : 0);
  static_assert(NA * APB == D && 4 * NE == NW, "tiling of the state");
};

template <typename OP> struct MkFrag;
template <> struct MkFrag<__bf16> {
  __device__ static bf16x8 make(const float (&x)[8]) {
    u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
               pack_bf16x2(x[6], x[7])};
    return __builtin_bit_cast(bf16x8, v);
  }
};
template <> struct MkFrag<float> {
  __device__ static f32x8 make(const float (&x)[8]) {
    return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  }
};

// row of accumulator register r for lane half hh (column = lane % 32)
__device__ __forceinline__ int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

template <int D, typename OP, typename IN, bool CAUSAL>
__global__ __launch_bounds__(PolyCfg<D>::NT) void poly_chunk_kernel(PolyArgs a) {
  using C = PolyCfg<D>;
  using Frag = typename Ops<OP>::frag;
  constexpr int RB = D * Ops<OP>::kBytes;  // operand tile row bytes
  constexpr int TB = 64 * RB;
  constexpr int TS = 68;                   // row stride (floats) of the transposed fp32 tiles
  constexpr int TTB = D * TS * 4;
  constexpr int RL = D / 8;
  constexpr int NB = C::NBB;
  // operand tiles Q, K; fp32 feature-major tiles Q^T, K^T, V^T; the waves'
  // partial outputs; the low-degree state tiles (fp32, accumulator layout)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TB + 3 * TTB + C::NW * 2048 * 4 + (NB + 1) * 4096];
  uint8_t* sQ = smem;
  uint8_t* sK = smem + TB;
  float* sQt = reinterpret_cast<float*>(smem + 2 * TB);  // [feature][row]
  float* sKt = sQt + D * TS;
  float* sVt = sKt + D * TS;
  f32x4* red = reinterpret_cast<f32x4*>(sVt + D * TS);   // [wave][2][4 register groups][64 lanes] of f32x4
  f32x4* lowst = red + C::NW * 512;                       // [tile][4 register groups][64 lanes] of f32x4

  const int bh = blockIdx.x, blk = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, hh = l >> 5, li = l & 31;
  const int E = blk % C::NE, hb = blk / C::NE;
  const int a0 = hb * C::APB + w * C::APW;
  const long long base = (long long)bh * a.N;
  const long long SD = (long long)bh * C::DP;  // first state row of this (batch, head)
  const long long BHN = (long long)a.BH * a.N;
  const IN* q = static_cast<const IN*>(a.q);
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  float* part = a.part + ((long long)hb * a.BH + bh) * a.N * D;

  // Every thread moves one 8-element piece of q, k and v per chunk: loaded
  // into registers one chunk ahead (fetch), then written (put) into the
  // swizzled operand tiles and, transposed and in fp32, into the
  // feature-major tiles.
  using Raw = typename In8<IN>::raw;
  struct Piece {
    Raw q, k, v;
  };
  const int prow = t / RL, pc0 = 8 * (t % RL);
  auto fetch = [&](int c) -> Piece {
    Piece pc;
    const bool live = c < a.nchunks && prow < min(64, a.N - 64 * c);
    const long long off = live ? (base + 64LL * c + prow) * D + pc0 : 0;
    pc.q = live ? In8<IN>::load(q + off) : In8<IN>::zero();
    pc.k = live ? In8<IN>::load(k + off) : In8<IN>::zero();
    pc.v = live ? In8<IN>::load(v + off) : In8<IN>::zero();
    return pc;
  };
  Piece cur = fetch(0);
  auto put = [&]() {
    float xq[8], xk[8], xv[8];
    In8<IN>::to_f32(cur.q, xq);
    In8<IN>::to_f32(cur.k, xk);
    In8<IN>::to_f32(cur.v, xv);
    Ops<OP>::template store8<RB>(sQ, prow, pc0, xq);
    Ops<OP>::template store8<RB>(sK, prow, pc0, xk);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sQt[(pc0 + e) * TS + prow] = xq[e];
      sKt[(pc0 + e) * TS + prow] = xk[e];
      sVt[(pc0 + e) * TS + prow] = xv[e];
    }
  };
  // chunk c into LDS, and the loads of chunk c + 1 issued
  auto stage = [&](int c) {
    if (c == 0) cur = fetch(0);
    put();
    __syncthreads();
    cur = fetch(c + 1);
  };
  // value operand: V[j][e] for this lane's column e = 32 E + lane % 32 and
  // rows j = j0 + 8 (lane / 32) + 0..7, optionally scaled per row
  auto vfrag = [&](int j0, const float* scale) -> Frag {
    const float* vt = sVt + (32 * E + li) * TS + j0 + 8 * hh;
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(vt), v1 = *reinterpret_cast<const f32x4*>(vt + 4);
    float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    if (scale) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(scale + j0 + 8 * hh);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(scale + j0 + 8 * hh + 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] *= s0[u];
        x[4 + u] *= s1[u];
      }
    }
    return MkFrag<OP>::make(x);
  };
  Frag ones;
  {
    const float o[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    ones = MkFrag<OP>::make(o);
  }
  auto ld_tile = [&](int ti) {
    f32x16 x;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 y = lowst[(ti * 4 + g) * 64 + l];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[4 * g + u] = y[u];
    }
    return x;
  };
  auto st_tile = [&](int ti, const f32x16& x) {
#pragma unroll
    for (int g = 0; g < 4; ++g) lowst[(ti * 4 + g) * 64 + l] = f32x4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
  };

  // quadratic state: tile (ia, bb) at ia * NB + bb, rows b = 32 bb + ..,
  // columns e = 32 E + .. of S2[a0 + ia]
  f32x16 ST[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int av = a0 + tt / NB, bb = tt % NB;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      ST[tt][r] = a.S_in ? a.S_in[(SD + 1 + D + av * D + 32 * bb + acc_row(r, hh)) * D + 32 * E + li] : 0.f;
  }
  // Low-degree state, in LDS. Workgroups hb = 0 hold S1[:, E] (tiles 0..NB-1,
  // rows b) and S0[E] (tile NB, every row equal); workgroups hb = 1 hold
  // Z2[:, E] (tiles 0..NB-1, rows b, columns c = 32 E + ..) and z1[E]
  // (tile NB, rows c, every column equal). Wave w <= NB fills tile w.
  const bool lnum = hb == 0, lden = hb == 1;
  if ((lnum || lden) && w <= NB) {
    f32x16 x;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = acc_row(r, hh);
      float val = 0.f;
      if (lnum && a.S_in) val = w < NB ? a.S_in[(SD + 1 + 32 * w + rr) * D + 32 * E + li] : a.S_in[SD * D + 32 * E + li];
      if (lden && a.z_in) val = w < NB ? a.z_in[SD + 1 + D + (32 * w + rr) * D + 32 * E + li] : a.z_in[SD + 1 + 32 * E + rr];
      x[r] = val;
    }
    st_tile(w, x);
  }
  float n_prev = a.z_in ? a.z_in[SD] : 0.f;  // tokens before the current chunk (and the carried count)

  auto update = [&](int c) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag kc[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) kc[bb] = Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * bb);
#pragma unroll
      for (int ia = 0; ia < C::APW; ++ia) {
        const Frag vb = vfrag(16 * kb, sKt + (a0 + ia) * TS);  // k_ja v_je
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) Ops<OP>::mma(ST[ia * NB + bb], kc[bb], vb);
      }
    }
    // low-degree updates, one tile per wave on the last waves
    __builtin_amdgcn_sched_barrier(0);
    const int u = C::NW - 1 - w;
    if ((lnum || lden) && u <= NB) {
      f32x16 x = ld_tile(u);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (lnum) {
          const Frag vb = vfrag(16 * kb, nullptr);
          if (u < NB)
            Ops<OP>::mma(x, Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * u), vb);  // S1[b][e] += k_jb v_je
          else
            Ops<OP>::mma(x, ones, vb);  // S0[e] += v_je
        } else {
          const Frag kcb = Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * E);
          if (u < NB)
            Ops<OP>::mma(x, Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * u), kcb);  // Z2[b][c] += k_jb k_jc
          else
            Ops<OP>::mma(x, kcb, ones);  // z1[c] += k_jc
        }
      }
      st_tile(u, x);
    }
    n_prev += (float)min(64, a.N - 64 * c);
  };

  auto readout = [&](int c, bool intra) {
    const int valid = min(64, a.N - 64 * c);
    // Low-degree read-outs first (waves 0..1 of workgroups hb = 0 and 1, and
    // the in-chunk waves), while the output tiles are not yet live: the
    // numerator part lands in lo (row block lo_ib) and seeds this wave's
    // output tile.
    f32x16 lo = {};
    int lo_ib = -1;
    {
      const int ib = w;
      if (lnum && w < 2) {
        // S0[E] + q_i . S1[:, E]
        f32x16 acc = ld_tile(NB);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          const f32x16 s1 = ld_tile(bb);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            Ops<OP>::mma(acc, Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 32 * bb + 16 * kk),
                         Ops<OP>::from_acc(s1, kk));
        }
        lo = acc;
        lo_ib = ib;
      }
    }
    // In-chunk part A V[:, E], A_ij = 1 + s_ij + s_ij^2 on keys j <= i, score
    // tiles (ib, jb) of this wave; the row sums (plus the carried count, on
    // the tiles jb = 0) form denominator slot 0, or slot 1 + NE for tile (1, 1)
    // when it has a wave of its own.
    {
      int ib = -1, jb0 = 0, njb = 1;
      if constexpr (C::SPLIT) {
        if (hb == 2 && w < 3) {
          ib = w == 0 ? 0 : 1;
          jb0 = w == 2 ? 1 : 0;
        }
      } else {
        if (hb == 0 && (w == 2 || w == 3)) {
          ib = w - 2;
          njb = ib + 1;
        }
      }
      if (ib >= 0) {
        float dsum = 0.f;
        f32x16 acc = {};
        if (intra) {
          for (int jb = jb0; jb < jb0 + njb; ++jb) {
            f32x16 Sc = {};
#pragma unroll
            for (int kb = 0; kb < D / 16; ++kb)
              Ops<OP>::mma(Sc, Ops<OP>::template load_rows<RB>(sK, 32 * jb, 16 * kb),
                           Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 16 * kb));
            // Sc[j][i] = k_j . q_i
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const bool keep = jb < ib || acc_row(r, hh) <= li;
              const float sv = Sc[r];
              const float A = keep ? 1.f + sv + sv * sv : 0.f;
              Sc[r] = A;
              dsum += A;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              Ops<OP>::mma(acc, Ops<OP>::from_acc(Sc, kk), vfrag(32 * jb + 16 * kk, nullptr));
          }
          lo = acc;
          lo_ib = ib;
        }
        dsum += xor32(dsum);
        if (E == 0 && a.normalize && hh == 0) {  // the other value blocks repeat these tiles
          const bool own = C::SPLIT && jb0 == 1;  // tile (1, 1) alone: slot 1 + NE
          const long long slot = own ? (1 + C::NE) * BHN : 0;
          const int i = 32 * ib + li;
          if (i < valid) a.den[slot + base + 64LL * c + i] = (own ? 0.f : n_prev) + dsum;
          if (own && li < valid) a.den[slot + base + 64LL * c + li] = 0.f;  // rows 0..31 of that slot
        }
      }
    }
    if (lden && w < 2 && a.normalize) {
      // phi(q_i) . (z1, Z2) over feature block E: sum_c q_ic (z1_c + sum_b Z2[b][c] q_ib)
      const int ib = w;
      f32x16 acc = ld_tile(NB);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const f32x16 z2 = ld_tile(bb);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          Ops<OP>::mma(acc, Ops<OP>::from_acc(z2, kk), Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 32 * bb + 16 * kk));
      }
      const int i = 32 * ib + li;
      // q_ic for c = 32 E + acc_row(r, hh): four groups of four consecutive
      // features of row i of the operand tile (the same values as Q^T)
      float p = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int byte = (32 * E + 8 * g + 4 * hh) * Ops<OP>::kBytes;  // inside one 16-byte unit
        float qc[4];
        if constexpr (sizeof(OP) == 2) {
          const u32x2 r = *reinterpret_cast<const u32x2*>(sQ + tile_off<RB>(i, byte));
          qc[0] = __uint_as_float(r[0] << 16);
          qc[1] = __uint_as_float(r[0] & 0xffff0000u);
          qc[2] = __uint_as_float(r[1] << 16);
          qc[3] = __uint_as_float(r[1] & 0xffff0000u);
        } else {
          const f32x4 r = *reinterpret_cast<const f32x4*>(sQ + tile_off<RB>(i, byte));
#pragma unroll
          for (int u = 0; u < 4; ++u) qc[u] = r[u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) p += qc[u] * acc[4 * g + u];
      }
      p += xor32(p);
      if (hh == 0 && i < valid) a.den[(1 + E) * BHN + base + 64LL * c + i] = p;
    }
    f32x16 Y[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      Y[0][r] = lo_ib == 0 ? lo[r] : 0.f;
      Y[1][r] = lo_ib == 1 ? lo[r] : 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ia = 0; ia < C::APW; ++ia) {
      Frag bf[NB][2];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) bf[bb][kk] = Ops<OP>::from_acc(ST[ia * NB + bb], kk);
      // both row blocks at once: two independent accumulation chains
      f32x16 R[2] = {};
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int ib = 0; ib < 2; ++ib)
            Ops<OP>::mma(R[ib], Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 32 * bb + 16 * kk), bf[bb][kk]);
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const float* qa = sQt + (a0 + ia) * TS + 32 * ib + 4 * hh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(qa + 8 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) Y[ib][4 * g + u] += qv[u] * R[ib][4 * g + u];
        }
      }
    }
    // sum the waves' tiles and store the partial (the next writes to red
    // come after the next chunk's staging barrier; the low-degree state is
    // updated only after this barrier)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        red[((w * 2 + ib) * 4 + g) * 64 + l] = f32x4{Y[ib][4 * g], Y[ib][4 * g + 1], Y[ib][4 * g + 2], Y[ib][4 * g + 3]};
    __syncthreads();
    // slot x = (ib, g, lane): four rows 32 ib + 8 g + 4 (lane / 32) + 0..3 of column lane % 32
    for (int x = t; x < 512; x += C::NT) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ww = 0; ww < C::NW; ++ww) s += red[ww * 512 + x];
      const int ib = x >> 8, g = (x >> 6) & 3, ll = x & 63;
      const int row0 = 32 * ib + 8 * g + 4 * (ll >> 5);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (row0 + u < valid) part[(64LL * c + row0 + u) * D + 32 * E + (ll & 31)] = s[u];
    }
  };

  if constexpr (CAUSAL) {
    for (int c = 0; c < a.nchunks; ++c) {
      stage(c);
      readout(c, true);  // the state of the chunks before this one
      update(c);
      __syncthreads();
    }
  } else {
    for (int c = 0; c < a.nchunks; ++c) {
      stage(c);
      update(c);
      __syncthreads();
    }
    for (int c = 0; c < a.nchunks; ++c) {
      stage(c);
      readout(c, false);
      __syncthreads();
    }
  }
  if (a.S_out) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int av = a0 + tt / NB, bb = tt % NB;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        a.S_out[(SD + 1 + D + av * D + 32 * bb + acc_row(r, hh)) * D + 32 * E + li] = ST[tt][r];
    }
    if ((lnum || lden) && w <= NB) {
      const f32x16 x = ld_tile(w);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = acc_row(r, hh);
        if (lnum) {
          if (w < NB)
            a.S_out[(SD + 1 + 32 * w + rr) * D + 32 * E + li] = x[r];
          else if (r == 0 && hh == 0)
            a.S_out[SD * D + 32 * E + li] = x[0];
        } else {
          if (w < NB)
            a.z_out[SD + 1 + D + (32 * w + rr) * D + 32 * E + li] = x[r];
          else if (li == 0)
            a.z_out[SD + 1 + 32 * E + rr] = x[r];
        }
      }
    }
    if (lden && E == 0 && t == 0) a.z_out[SD] = n_prev;
  }
}

// y = (sum of the partial numerators) / max(den, eps), four outputs per thread
template <typename IN>
__global__ __launch_bounds__(256) void poly_finalize_kernel(PolyArgs a, int D, int nslots, int nden) {
  const long long total = (long long)a.BH * a.N * D;
  const long long e0 = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
  if (e0 >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(a.part + e0);
  for (int sl = 1; sl < nslots; ++sl) s += *reinterpret_cast<const f32x4*>(a.part + sl * total + e0);
  if (a.normalize) {
    const long long row = e0 / D, rows = (long long)a.BH * a.N;
    float den = a.den[row];
    for (int sl = 1; sl < nden; ++sl) den += a.den[sl * rows + row];
    s *= 1.f / fmaxf(den, kEps);
  }
  IN* out = static_cast<IN*>(a.out) + e0;
  if constexpr (sizeof(IN) == 2) {
    *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  } else {
    *reinterpret_cast<f32x4*>(out) = s;
  }
}

// phi of row x at feature f (x in LDS, fp32)
__device__ __forceinline__ float poly_phi(const float* x, int D, int f) {
  if (f == 0) return 1.f;
  if (f <= D) return x[f - 1];
  const int g = f - 1 - D;
  return x[g / D] * x[g % D];
}

// Decode step: one workgroup per (batch, head). Thread t owns value column
// t % D of state rows r = t / D, t / D + 256 / D, ... (coalesced rows) and
// normalizer entries t, t + 256, ...
template <int D, typename IN>
__global__ __launch_bounds__(256) void poly_decode_kernel(DecodeArgs a) {
  constexpr int DP = 1 + D + D * D, NG = 256 / D;
  __shared__ float sq[D], sk[D], sv[D];
  __shared__ float rn[NG][D], rd[256];
  const int bh = blockIdx.x, t = threadIdx.x;
  if (t < D) {
    const long long o = (long long)bh * D + t;
    if constexpr (sizeof(IN) == 2) {
      sq[t] = (float)static_cast<const __bf16*>(a.q)[o];
      sk[t] = (float)static_cast<const __bf16*>(a.k)[o];
      sv[t] = (float)static_cast<const __bf16*>(a.v)[o];
    } else {
      sq[t] = static_cast<const float*>(a.q)[o];
      sk[t] = static_cast<const float*>(a.k)[o];
      sv[t] = static_cast<const float*>(a.v)[o];
    }
  }
  __syncthreads();
  const int e = t % D, g = t / D;
  float* S = a.S + (long long)bh * DP * D;
  float num = 0.f;
  const float ve = sv[e];
  for (int r = g; r < DP; r += NG) {
    const float s = S[(long long)r * D + e] + poly_phi(sk, D, r) * ve;
    S[(long long)r * D + e] = s;
    num += poly_phi(sq, D, r) * s;
  }
  float* z = a.z + (long long)bh * DP;
  float den = 0.f;
  for (int r = t; r < DP; r += 256) {
    const float zz = z[r] + poly_phi(sk, D, r);
    z[r] = zz;
    den += poly_phi(sq, D, r) * zz;
  }
  rn[g][e] = num;
  rd[t] = den;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) rd[t] += rd[t + s];
    __syncthreads();
  }
  if (t < D) {
    float y = 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) y += rn[gg][t];
    if (a.normalize) y /= fmaxf(rd[0], kEps);
    const long long o = (long long)bh * D + t;
    if constexpr (sizeof(IN) == 2)
      static_cast<__bf16*>(a.out)[o] = (__bf16)y;
    else
      static_cast<float*>(a.out)[o] = y;
  }
}

// phi(x) rows materialized: one thread per output element
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void poly_fmap_kernel(FmapArgs a, int D) {
  const long long DP = 1 + D + (long long)D * D;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.rows * DP) return;
  const long long row = idx / DP;
  const int f = (int)(idx % DP);
  const TI* x = static_cast<const TI*>(a.x) + row * D;
  float y;
  if (f == 0) {
    y = 1.f;
  } else if (f <= D) {
    y = (float)x[f - 1];
  } else {
    const int gg = f - 1 - D;
    y = (float)x[gg / D] * (float)x[gg % D];
  }
  static_cast<TO*>(a.phi)[idx] = (TO)y;
}

template <int D, typename OP, typename IN>
hipError_t launch_poly(const PolyArgs& a, bool causal, hipStream_t st) {
  using C = PolyCfg<D>;
  const dim3 grid(a.BH, C::NE * C::NA), block(C::NT);
  if (causal)
    hipLaunchKernelGGL((poly_chunk_kernel<D, OP, IN, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((poly_chunk_kernel<D, OP, IN, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n4 = (long long)a.BH * a.N * D / 4;
  hipLaunchKernelGGL((poly_finalize_kernel<IN>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a, D,
                     C::NA, C::NDEN);
  return hipGetLastError();
}

}  // namespace

int poly_partials(int D) { return D == 32 ? PolyCfg<32>::NA : PolyCfg<64>::NA; }
int poly_den_slots(int D) { return D == 32 ? PolyCfg<32>::NDEN : PolyCfg<64>::NDEN; }

hipError_t poly_forward_dispatch(const PolyArgs& a, int D, int dtype, bool causal, hipStream_t st) {
  const bool bf = dtype == 1;
  if (D == 32) return bf ? launch_poly<32, __bf16, __bf16>(a, causal, st) : launch_poly<32, float, float>(a, causal, st);
  if (D == 64) return bf ? launch_poly<64, __bf16, __bf16>(a, causal, st) : launch_poly<64, float, float>(a, causal, st);
  return hipErrorInvalidValue;
}

hipError_t poly_decode_dispatch(const DecodeArgs& a, int D, int dtype, hipStream_t st) {
  const bool bf = dtype == 1;
  if (D == 32) {
    if (bf) hipLaunchKernelGGL((poly_decode_kernel<32, __bf16>), dim3(a.BH), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((poly_decode_kernel<32, float>), dim3(a.BH), dim3(256), 0, st, a);
  } else if (D == 64) {
    if (bf) hipLaunchKernelGGL((poly_decode_kernel<64, __bf16>), dim3(a.BH), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((poly_decode_kernel<64, float>), dim3(a.BH), dim3(256), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t poly_fmap_dispatch(const FmapArgs& a, int D, int in_dtype, int out_dtype, hipStream_t st) {
  const long long n = a.rows * (1 + D + (long long)D * D);
  const dim3 grid((unsigned)((n + 255) / 256));
  const bool bi = in_dtype == 1, bo = out_dtype == 1;
  if (bi && bo) hipLaunchKernelGGL((poly_fmap_kernel<__bf16, __bf16>), grid, dim3(256), 0, st, a, D);
  else if (bi) hipLaunchKernelGGL((poly_fmap_kernel<__bf16, float>), grid, dim3(256), 0, st, a, D);
  else if (bo) hipLaunchKernelGGL((poly_fmap_kernel<float, __bf16>), grid, dim3(256), 0, st, a, D);
  else hipLaunchKernelGGL((poly_fmap_kernel<float, float>), grid, dim3(256), 0, st, a, D);
  return hipGetLastError();
}

}  // namespace la

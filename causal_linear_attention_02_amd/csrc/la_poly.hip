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
// One more workgroup per (batch, head) holds the low-degree state
// (S0 = sum v, S1 = sum k v^T), the normalizer state (n, z1 = sum k,
// Z2 = sum k k^T) and forms the in-chunk part with the kernel applied to the
// scores, A_ij = 1 + s_ij + s_ij^2 (j <= i). Every workgroup walks the chunks
// in order and writes its partial numerators (fp32) to the workspace; the
// low-degree workgroup also writes the denominators. A last kernel sums the
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
  constexpr int VB = TB > TTB ? TB : TTB;  // sV (low-degree workgroup) and sVt (the others) share it
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TB + 2 * TTB + VB + C::NW * 2048 * 4];
  __shared__ float dint[64], dpart[C::NE][64];
  uint8_t* sQ = smem;
  uint8_t* sK = smem + TB;
  float* sQt = reinterpret_cast<float*>(smem + 2 * TB);  // [feature][row]
  float* sKt = sQt + D * TS;
  uint8_t* sV = smem + 2 * TB + 2 * TTB;
  float* sVt = reinterpret_cast<float*>(sV);
  float* red = reinterpret_cast<float*>(smem + 2 * TB + 2 * TTB + VB);  // [wave][2][16 registers][64 lanes]

  const int bh = blockIdx.x, blk = blockIdx.y;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, hh = l >> 5, li = l & 31;
  const bool low = blk == C::NE * C::NA;
  const long long base = (long long)bh * a.N;
  const long long SD = (long long)bh * C::DP;  // first state row of this (batch, head)
  const IN* q = static_cast<const IN*>(a.q);
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);

  // Every thread moves one 8-element piece of q, k and v per chunk: loaded
  // into registers one chunk ahead (fetch), then written (put) into the
  // swizzled operand tiles and, transposed and in fp32, into the
  // feature-major tiles (v: the operand tile in the low-degree workgroup,
  // the transposed one in the others).
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
    if (low) Ops<OP>::template store8<RB>(sV, prow, pc0, xv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sQt[(pc0 + e) * TS + prow] = xq[e];
      sKt[(pc0 + e) * TS + prow] = xk[e];
      if (!low) sVt[(pc0 + e) * TS + prow] = xv[e];
    }
  };
  // chunk c into LDS, and the loads of chunk c + 1 issued
  auto stage = [&](int c) {
    if (c == 0) cur = fetch(0);
    put();
    __syncthreads();
    cur = fetch(c + 1);
  };

  if (!low) {
    // ------------------------------------------------------------------
    // quadratic part: value block E, a in [a0, a0 + APW) for this wave
    // ------------------------------------------------------------------
    const int E = blk % C::NE, hb = blk / C::NE;
    const int a0 = hb * C::APB + w * C::APW;
    float* part = a.part + ((long long)(1 + hb) * a.BH + bh) * a.N * D;
    f32x16 ST[4];  // tile (ia, bb) at ia * NBB + bb: rows b = 32 bb + .., columns e = 32 E + ..
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int av = a0 + tt / C::NBB, bb = tt % C::NBB;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ST[tt][r] = a.S_in ? a.S_in[(SD + 1 + D + av * D + 32 * bb + acc_row(r, hh)) * D + 32 * E + li] : 0.f;
    }
    auto update = [&]() {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Frag kc[C::NBB];
#pragma unroll
        for (int bb = 0; bb < C::NBB; ++bb) kc[bb] = Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * bb);
        const float* vt = sVt + (32 * E + li) * TS + 16 * kb + 8 * hh;
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(vt), v1 = *reinterpret_cast<const f32x4*>(vt + 4);
#pragma unroll
        for (int ia = 0; ia < C::APW; ++ia) {
          const float* kt = sKt + (a0 + ia) * TS + 16 * kb + 8 * hh;
          const f32x4 k0 = *reinterpret_cast<const f32x4*>(kt), k1 = *reinterpret_cast<const f32x4*>(kt + 4);
          const float x[8] = {v0[0] * k0[0], v0[1] * k0[1], v0[2] * k0[2], v0[3] * k0[3],
                              v1[0] * k1[0], v1[1] * k1[1], v1[2] * k1[2], v1[3] * k1[3]};
          const Frag vb = MkFrag<OP>::make(x);
#pragma unroll
          for (int bb = 0; bb < C::NBB; ++bb) Ops<OP>::mma(ST[ia * C::NBB + bb], kc[bb], vb);
        }
      }
    };
    auto readout = [&](int c) {
      const int valid = min(64, a.N - 64 * c);
      f32x16 Y[2] = {};
#pragma unroll
      for (int ia = 0; ia < C::APW; ++ia) {
        Frag bf[C::NBB][2];
#pragma unroll
        for (int bb = 0; bb < C::NBB; ++bb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) bf[bb][kk] = Ops<OP>::from_acc(ST[ia * C::NBB + bb], kk);
        // both row blocks at once: two independent accumulation chains
        f32x16 R[2] = {};
#pragma unroll
        for (int bb = 0; bb < C::NBB; ++bb)
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
      // come after the next chunk's staging barrier)
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[((w * 2 + ib) * 16 + r) * 64 + l] = Y[ib][r];
      __syncthreads();
      for (int x = t; x < 2048; x += C::NT) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < C::NW; ++ww) s += red[ww * 2048 + x];
        const int ib = x >> 10, r = (x >> 6) & 15, ll = x & 63;
        const int row = 32 * ib + acc_row(r, ll >> 5);
        if (row < valid) part[(64LL * c + row) * D + 32 * E + (ll & 31)] = s;
      }
    };
    if constexpr (CAUSAL) {
      for (int c = 0; c < a.nchunks; ++c) {
        stage(c);
        readout(c);  // the state of the chunks before this one
        update();
        __syncthreads();
      }
    } else {
      for (int c = 0; c < a.nchunks; ++c) {
        stage(c);
        update();
        __syncthreads();
      }
      for (int c = 0; c < a.nchunks; ++c) {
        stage(c);
        readout(c);
        __syncthreads();
      }
    }
    if (a.S_out) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int av = a0 + tt / C::NBB, bb = tt % C::NBB;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          a.S_out[(SD + 1 + D + av * D + 32 * bb + acc_row(r, hh)) * D + 32 * E + li] = ST[tt][r];
      }
    }
    return;
  }

  // --------------------------------------------------------------------
  // low-degree workgroup. Waves 0 .. 2NE-1 ("num"): row block ib, value
  // block E; they hold S1[:, E] (rows b) and S0[E] (every row of X equal).
  // Waves 2NE .. 4NE-1 ("den"): row block ib, feature block Cb; they hold
  // Z2[:, Cb] (rows b) and z1[Cb] (X: rows c, every column equal).
  // --------------------------------------------------------------------
  const bool numw = w < 2 * C::NE;
  const int wr = numw ? w : w - 2 * C::NE;
  const int ib = wr / C::NE, E = wr % C::NE;  // E: value block (num) or feature block (den)
  float* part = a.part + (long long)bh * a.N * D;
  Frag ones;
  {
    const float o[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    ones = MkFrag<OP>::make(o);
  }
  f32x16 T[C::NBB], X;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = acc_row(r, hh);
#pragma unroll
    for (int bb = 0; bb < C::NBB; ++bb) {
      if (numw)
        T[bb][r] = a.S_in ? a.S_in[(SD + 1 + 32 * bb + rr) * D + 32 * E + li] : 0.f;
      else
        T[bb][r] = a.z_in ? a.z_in[SD + 1 + D + (32 * bb + rr) * D + 32 * E + li] : 0.f;
    }
    X[r] = numw ? (a.S_in ? a.S_in[SD * D + 32 * E + li] : 0.f) : (a.z_in ? a.z_in[SD + 1 + 32 * E + rr] : 0.f);
  }
  float n_prev = a.z_in ? a.z_in[SD] : 0.f;

  auto update = [&](int c) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const Frag cf = numw ? Ops<OP>::template load_cols<RB>(sV, 16 * kb, 32 * E)
                           : Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * E);
#pragma unroll
      for (int bb = 0; bb < C::NBB; ++bb) Ops<OP>::mma(T[bb], Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * bb), cf);
      if (numw)
        Ops<OP>::mma(X, ones, cf);  // S0[e] += sum_j v_je in every row
      else
        Ops<OP>::mma(X, cf, ones);  // z1[c] += sum_j k_jc in every column
    }
    n_prev += (float)min(64, a.N - 64 * c);
  };
  // numerator (num waves) or normalizer partials (den waves) of chunk c
  auto readout = [&](int c, bool intra) {
    const int valid = min(64, a.N - 64 * c);
    f32x16 acc = X;
#pragma unroll
    for (int bb = 0; bb < C::NBB; ++bb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag qf = Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 32 * bb + 16 * kk);
        if (numw)
          Ops<OP>::mma(acc, qf, Ops<OP>::from_acc(T[bb], kk));  // [i][e] += sum_b q_ib S1[b][e]
        else
          Ops<OP>::mma(acc, Ops<OP>::from_acc(T[bb], kk), qf);  // [c][i] += sum_b Z2[b][c] q_ib
      }
    if (numw) {
      float dsum = 0.f;
      if (intra) {
        for (int jb = 0; jb <= ib; ++jb) {
          f32x16 Sc = {};
#pragma unroll
          for (int kb = 0; kb < D / 16; ++kb)
            Ops<OP>::mma(Sc, Ops<OP>::template load_rows<RB>(sK, 32 * jb, 16 * kb),
                         Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 16 * kb));
          // Sc[j][i] = k_j.q_i -> kernel 1 + s + s^2 on keys j <= i
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool keep = jb < ib || acc_row(r, hh) <= li;
            const float s = Sc[r];
            const float A = keep ? 1.f + s + s * s : 0.f;
            Sc[r] = A;
            dsum += A;
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            Ops<OP>::mma(acc, Ops<OP>::from_acc(Sc, kk),
                         Ops<OP>::template load_cols<RB>(sV, 32 * jb + 16 * kk, 32 * E));
        }
      }
      if (E == 0) {
        dsum += xor32(dsum);
        if (hh == 0) dint[32 * ib + li] = dsum;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = 32 * ib + acc_row(r, hh);
        if (i < valid) part[(64LL * c + i) * D + 32 * E + li] = acc[r];
      }
    } else {
      // phi(q_i) . (z1, Z2) over this feature block: sum_c q_ic (z1_c + sum_b Z2[b][c] q_ib)
      const int i = 32 * ib + li;
      float p = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) p += sQt[(32 * E + acc_row(r, hh)) * TS + i] * acc[r];
      p += xor32(p);
      if (hh == 0) dpart[E][i] = p;
    }
    __syncthreads();
    if (!numw && E == 0 && hh == 0 && a.normalize) {
      const int i = 32 * ib + li;
      if (i < valid) {
        float den = n_prev + (intra ? dint[i] : 0.f);
#pragma unroll
        for (int cb = 0; cb < C::NE; ++cb) den += dpart[cb][i];
        a.den[base + 64LL * c + i] = den;
      }
    }
  };

  if constexpr (CAUSAL) {
    for (int c = 0; c < a.nchunks; ++c) {
      stage(c);
      readout(c, true);
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
  if (a.S_out && ib == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = acc_row(r, hh);
#pragma unroll
      for (int bb = 0; bb < C::NBB; ++bb) {
        if (numw)
          a.S_out[(SD + 1 + 32 * bb + rr) * D + 32 * E + li] = T[bb][r];
        else
          a.z_out[SD + 1 + D + (32 * bb + rr) * D + 32 * E + li] = T[bb][r];
      }
      if (numw) {
        if (r == 0 && hh == 0) a.S_out[SD * D + 32 * E + li] = X[0];
      } else if (li == 0) {
        a.z_out[SD + 1 + 32 * E + rr] = X[r];
      }
    }
    if (!numw && E == 0 && l == 0) a.z_out[SD] = n_prev;
  }
}

// y = (sum of the partial numerators) / max(den, eps), four outputs per thread
template <typename IN>
__global__ __launch_bounds__(256) void poly_finalize_kernel(PolyArgs a, int D, int nslots) {
  const long long total = (long long)a.BH * a.N * D;
  const long long e0 = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
  if (e0 >= total) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(a.part + e0);
  for (int sl = 1; sl < nslots; ++sl) s += *reinterpret_cast<const f32x4*>(a.part + sl * total + e0);
  if (a.normalize) s *= 1.f / fmaxf(a.den[e0 / D], kEps);
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
  const dim3 grid(a.BH, C::NE * C::NA + 1), block(C::NT);
  if (causal)
    hipLaunchKernelGGL((poly_chunk_kernel<D, OP, IN, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((poly_chunk_kernel<D, OP, IN, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n4 = (long long)a.BH * a.N * D / 4;
  hipLaunchKernelGGL((poly_finalize_kernel<IN>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a, D,
                     C::NA + 1);
  return hipGetLastError();
}

}  // namespace

int poly_partials(int D) { return D == 32 ? PolyCfg<32>::NA + 1 : PolyCfg<64>::NA + 1; }

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

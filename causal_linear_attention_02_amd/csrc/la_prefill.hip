// Chunked kernelized linear attention on gfx950.
//
// Definitions ("Linear Attention", marovi.ai, "Reformulación con núcleos"):
//   y_i = phi(q_i)^T S / phi(q_i)^T z,  S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j)
// with the causal sums taken over j <= i ("Forma recurrente e inferencia
// autorregresiva"), computed blockwise ("Entrenamiento: forma paralela"): the
// sequence is cut into chunks of 64 tokens; inside a chunk the masked
// quadratic form, across chunks the running state (S, z).
//
// Sequence parallelism on one GPU: each (batch, head) sequence is split into
// P segments of whole chunks.
//   state pass : every segment's local sums (S_loc, z_loc)         -> workspace
//                (the chunk's keys split across waves, partials added at the end)
//   carry scan : exclusive prefix over segments (+ initial state)  -> workspace
//   output pass: every segment starts from its prefix and walks its chunks
// The non-causal form reuses the state pass, a total-sum scan and the output
// pass without the intra-chunk term.
//
// Output pass workgroup = D/32 consumer waves + D/32 producer waves (two per
// SIMD at d = 128, so vector work and matrix work overlap):
//   producers: global loads one chunk ahead (two register sets), the feature
//     map, LDS staging, the running z (column sums of phi(K)) and the
//     cross-chunk denominator phi(q_i).z of every row;
//   consumers: consumer wave w owns value columns [32w, 32w+32) and keeps
//     S[:, 32w:32w+32] in fp32 MFMA accumulators; it forms the masked scores,
//     both numerator terms, normalizes, stores y and updates S.
// Layouts: q, k, v, out are [BH][N][D]; S is [BH][DF][D] (row = feature,
// column = value dim); z is [BH][DF].
#include "la_device.h"
#include "la_kernels.h"

namespace la {

// ---------------------------------------------------------------------------
// Staging geometry of NPT threads over a 64-row chunk (NPT = 2*D producers in
// the output pass; the state pass's whole block). Feature-side rows (phi(Q),
// phi(K); DF values) are covered by RLF = DF/8 threads each, so thread p
// holds pieces i = 0..NQ-1 at row p/RLF + RSF*i, columns 8*(p % RLF); value
// rows (D values) by RLV = D/8 threads, pieces i = 0..NV-1 at row
// p/RLV + RSV*i. Threads with equal p % RLF share feature columns.
// ---------------------------------------------------------------------------
template <int D, int DF, int NPT = 2 * D>
struct Stage {
  static constexpr int NP = NPT;
  static constexpr int RLF = DF / 8, RSF = NP / RLF, NQ = 64 / RSF;
  static constexpr int RLV = D / 8, RSV = NP / RLV, NV = 64 / RSV;
  static_assert(NP % RLF == 0 && 64 % RSF == 0 && NQ >= 1 && NQ <= 16, "staging geometry");
  static_assert(NP % RLV == 0 && 64 % RSV == 0 && NV >= 1 && NV <= 16, "staging geometry");
  // register sets for the loads in flight. Two, for every head dimension:
  // against three, the long-context prefill ran 1% faster at d = 128, 3-4%
  // at d = 32 and 64, and 16% with many 4096-token sequences (B32 H32) at
  // d = 32 and 64 (the decay variants, whose scaling needs registers, had
  // kept two all along)
  static constexpr int NSET = 2;
  template <bool DECAY>
  static constexpr int nset() { return NSET; }
};

template <int D, int DF, typename IN, int NPT = 2 * D>
struct Pref {
  typename In8<IN>::raw q[Stage<D, DF, NPT>::NQ], k[Stage<D, DF, NPT>::NQ], v[Stage<D, DF, NPT>::NV];
};

template <int D, int DF, typename IN, int NPT = 2 * D>
struct Voff {
  static constexpr bool kSame = DF == D;  // then feature and value pieces coincide
  int f[Stage<D, DF, NPT>::NQ];                    // byte offsets of the feature-side pieces
  int v_[kSame ? 1 : Stage<D, DF, NPT>::NV];       // byte offsets of the value pieces
  __device__ __forceinline__ explicit Voff(int p) {
    using G = Stage<D, DF, NPT>;
#pragma unroll
    for (int i = 0; i < G::NQ; ++i)
      f[i] = ((p / G::RLF + G::RSF * i) * DF + 8 * (p % G::RLF)) * (int)sizeof(IN);
    if constexpr (!kSame) {
#pragma unroll
      for (int i = 0; i < G::NV; ++i)
        v_[i] = ((p / G::RLV + G::RSV * i) * D + 8 * (p % G::RLV)) * (int)sizeof(IN);
    }
  }
  __device__ __forceinline__ int v(int i) const {
    if constexpr (kSame) return f[i];
    else return v_[i];
  }
};

// Loads of one chunk (rows [row_base, row_base + valid)); rows past the end
// read as zero through the descriptor's range check. q and k rows have DF
// elements, v rows D.
template <int D, int DF, typename IN, bool LQ, bool LKV, int NPT>
__device__ __forceinline__ void prod_load(Pref<D, DF, IN, NPT>& pf, const Voff<D, DF, IN, NPT>& vo, const IN* q,
                                          const IN* k, const IN* v, long long row_base, int valid) {
  using G = Stage<D, DF, NPT>;
  const unsigned fbytes = (unsigned)(valid * DF * (int)sizeof(IN));
  const unsigned vbytes = (unsigned)(valid * D * (int)sizeof(IN));
#pragma unroll
  for (int i = 0; i < G::NQ; ++i) {
    if constexpr (LQ) pf.q[i] = In8<IN>::bload_nt(make_rsrc(q + row_base * DF, fbytes), vo.f[i]);
    if constexpr (LKV) pf.k[i] = In8<IN>::bload_nt(make_rsrc(k + row_base * DF, fbytes), vo.f[i]);
  }
  if constexpr (LKV) {
#pragma unroll
    for (int i = 0; i < G::NV; ++i) pf.v[i] = In8<IN>::bload_nt(make_rsrc(v + row_base * D, vbytes), vo.v(i));
  }
}

// Marks the registers of a prefetched chunk as read without touching them.
// A step that does not stage its chunk calls this, so that every load is
// retired on every path through a step: the wait-count analysis then needs no
// conservative drain of the loads still in flight at the loop's back edge.
template <typename R> __device__ __forceinline__ void touch(const R& r) {
  if constexpr (sizeof(R) == 16) {
    asm volatile("" ::"v"(r));
  } else {
    asm volatile("" ::"v"(r.a));
    asm volatile("" ::"v"(r.b));
  }
}
template <int D, int DF, typename IN, bool LQ, bool LKV, int NPT>
__device__ __forceinline__ void retire(const Pref<D, DF, IN, NPT>& pf) {
#pragma unroll
  for (int i = 0; i < Stage<D, DF, NPT>::NQ; ++i) {
    if constexpr (LQ) touch(pf.q[i]);
    if constexpr (LKV) touch(pf.k[i]);
  }
  if constexpr (LKV) {
#pragma unroll
    for (int i = 0; i < Stage<D, DF, NPT>::NV; ++i) touch(pf.v[i]);
  }
}

// Key rows past the end of the sequence become -inf (elu+1: phi = 0 there)
// or 0 (pre-mapped features), so they add nothing to the scores, S or z.
// Branch-free, so every step has the same instruction stream.
template <int D, int DF, typename IN, int FM, int NPT>
__device__ __forceinline__ void mask_tail_keys(Pref<D, DF, IN, NPT>& pf, int p, int valid) {
  using G = Stage<D, DF, NPT>;
  const auto fill = FM == kElu1 ? In8<IN>::neg_inf() : In8<IN>::zero();
#pragma unroll
  for (int i = 0; i < G::NQ; ++i) {
    const bool past = p / G::RLF + G::RSF * i >= valid;
    if constexpr (sizeof(IN) == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pf.k[i][j] = past ? fill[j] : pf.k[i][j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf.k[i].a[j] = past ? fill.a[j] : pf.k[i].a[j];
        pf.k[i].b[j] = past ? fill.b[j] : pf.k[i].b[j];
      }
    }
  }
}

template <typename IN, typename OP, int RB>
__device__ __forceinline__ void store_raw(uint8_t* tile, int row, int col, const typename In8<IN>::raw& r) {
  static_assert(sizeof(IN) == sizeof(OP), "raw staging needs matching element types");
  if constexpr (sizeof(IN) == 2) {
    *reinterpret_cast<u32x4*>(tile + tile_off<RB>(row, col * 2)) = r;
  } else {
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4)) = r.a;
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4 + 16)) = r.b;
  }
}

template <int FM>
__device__ __forceinline__ float fmap_in_stage(float x) {
  if constexpr (FM == kElu1) return phi_elu1(x);
  else return x;  // features already mapped by the random-feature kernel
}

// Feature map + LDS writes for one chunk.
// Accumulates, per piece i, dp[i] = sum_e phi(q)[i][e] * z[e] (if LQ) and the
// column sums of phi(k) over the thread's rows in cs (if LKV).
template <int D, int DF, typename IN, typename OP, int FM, bool LQ, bool LKV, int NPT>
__device__ __forceinline__ void prod_stage(const Pref<D, DF, IN, NPT>& pf, int p, uint8_t* sQ, uint8_t* sK,
                                           uint8_t* sV, const float (&z)[8], float (&dp)[Stage<D, DF, NPT>::NQ],
                                           float (&cs)[8]) {
  using G = Stage<D, DF, NPT>;
  constexpr int RBF = DF * Ops<OP>::kBytes, RBV = D * Ops<OP>::kBytes;
  const int fcol = 8 * (p % G::RLF);
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = 0.f;
#pragma unroll
  for (int i = 0; i < G::NQ; ++i) {
    const int row = p / G::RLF + G::RSF * i;
    float x[8];
    if constexpr (LQ) {
      In8<IN>::to_f32(pf.q[i], x);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = fmap_in_stage<FM>(x[e]);
        d += x[e] * z[e];
      }
      dp[i] = d;
      Ops<OP>::template store8<RBF>(sQ, row, fcol, x);
    }
    if constexpr (LKV) {
      In8<IN>::to_f32(pf.k[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = fmap_in_stage<FM>(x[e]);
        cs[e] += x[e];
      }
      Ops<OP>::template store8<RBF>(sK, row, fcol, x);
      // equal widths: value piece i sits at the same row and column, and
      // storing it here frees its registers early
      if constexpr (DF == D) store_raw<IN, OP, RBV>(sV, row, fcol, pf.v[i]);
    }
  }
  if constexpr (LKV && DF != D) {
#pragma unroll
    for (int i = 0; i < G::NV; ++i) store_raw<IN, OP, RBV>(sV, p / G::RLV + G::RSV * i, 8 * (p % G::RLV), pf.v[i]);
  }
}

// Piecewise forms of prod_load / mask_tail_keys / prod_stage for the output
// pass, which interleaves the loads of the next chunk with the staging of the
// current one piece by piece, so that each wave's memory requests spread over
// the whole step instead of leaving in one burst after the barrier.
struct ChunkRsrc {
  __amdgpu_buffer_rsrc_t q, k, v;
};
template <int D, int DF, typename IN>
__device__ __forceinline__ ChunkRsrc chunk_rsrc(const IN* q, const IN* k, const IN* v, long long row_base,
                                                int valid) {
  const unsigned fbytes = (unsigned)(valid * DF * (int)sizeof(IN));
  const unsigned vbytes = (unsigned)(valid * D * (int)sizeof(IN));
  return ChunkRsrc{make_rsrc(q + row_base * DF, fbytes), make_rsrc(k + row_base * DF, fbytes),
                   make_rsrc(v + row_base * D, vbytes)};
}

// phi(q) piece i (times the row scale sc when SC): LDS tile row, and
// dp = phi(q) . z over the piece's columns
template <int D, int DF, typename IN, typename OP, int FM, bool SC>
__device__ __forceinline__ float stage_q_piece(const typename In8<IN>::raw& r, int p, int i, uint8_t* sQ,
                                               const float (&z)[8], float sc) {
  using G = Stage<D, DF>;
  float x[8];
  In8<IN>::to_f32(r, x);
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = fmap_in_stage<FM>(x[e]);
    if constexpr (SC) x[e] *= sc;
    d += x[e] * z[e];
  }
  Ops<OP>::template store8<DF * Ops<OP>::kBytes>(sQ, p / G::RLF + G::RSF * i, 8 * (p % G::RLF), x);
  return d;
}

// phi(k) piece i (rows past `valid` masked to phi = 0; times the row scale sc
// when SC): LDS tile row, column sums into cs
template <int D, int DF, typename IN, typename OP, int FM, bool SC, int NPT = 2 * D>
__device__ __forceinline__ void stage_k_piece(typename In8<IN>::raw r, int p, int i, int valid, uint8_t* sK,
                                              float (&cs)[8], float sc) {
  using G = Stage<D, DF, NPT>;
  const int row = p / G::RLF + G::RSF * i;
  const auto fill = FM == kElu1 ? In8<IN>::neg_inf() : In8<IN>::zero();
  const bool past = row >= valid;
  if constexpr (sizeof(IN) == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = past ? fill[j] : r[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.a[j] = past ? fill.a[j] : r.a[j];
      r.b[j] = past ? fill.b[j] : r.b[j];
    }
  }
  float x[8];
  In8<IN>::to_f32(r, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = fmap_in_stage<FM>(x[e]);
    if constexpr (SC) x[e] *= sc;
    cs[e] += x[e];
  }
  Ops<OP>::template store8<DF * Ops<OP>::kBytes>(sK, row, 8 * (p % G::RLF), x);
}

// ---------------------------------------------------------------------------
// Decay ("Linear Attention", "Variantes y extensiones", RetNet item):
// S_t = gamma S_{t-1} + phi(k_t) v_t^T, z alike. Inside a chunk, row r of
// phi(Q) is staged times gamma^(r-32) and row r of phi(K) times gamma^(32-r),
// so the chunk's score matrix carries gamma^(r_i - r_j). Running states are
// kept as gamma^-31 times the true ones; then one chunk moves them on as
// S' <- gamma^64 S' + K^T V with the scaled keys, and the carried term of row
// r_i, gamma^(r_i+1) phi(q_i) S, is (scaled q_i) . (gamma^64 S'). With
// gamma >= 1/4 no scale exceeds 2^64. gamma^64 is formed as gamma^32
// squared: below gamma = 0.2552 it is a denormal (2^-128 at gamma = 1/4),
// and the state it moves on is then 2^-126 or less of the chunk's own
// terms. The running normalizers take gamma^32 twice.
// ---------------------------------------------------------------------------
constexpr int kDecayCenter = 32;
constexpr int kDecayFrame = kChunk - 1 - kDecayCenter;  // 31
__device__ __forceinline__ float gpow(float lg, float n) { return __builtin_amdgcn_exp2f(lg * n); }

// DPP lane moves within rows of 16 lanes (quad_perm, mirrors, rotations).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor8 = 0x128;

// Sum over the RL lanes that share one row (aligned groups of RL lanes).
template <int RL>
__device__ __forceinline__ float row_reduce(float x) {
  if constexpr (RL >= 2) x += dpp_mov<kDppQuadXor1>(x);
  if constexpr (RL >= 4) x += dpp_mov<kDppQuadXor2>(x);
  if constexpr (RL >= 8) x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (RL >= 16) x += dpp_mov<kDppMirror>(x);
  if constexpr (RL >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}
// Sum over the lanes of a wave that share lane % RL.
template <int RL>
__device__ __forceinline__ float col_reduce(float x) {
  if constexpr (RL <= 4) x += dpp_mov<kDppRor4>(x);
  if constexpr (RL <= 8) x += dpp_mov<kDppRor8>(x);
  if constexpr (RL <= 32) x += xor32(x);
  if constexpr (RL <= 16) x += __shfl_xor(x, 16, 64);
  return x;
}

// Load this wave's state tiles (accumulator layout): rows = features
// 32cb + ..., columns = value dims 32w + lane%32.
template <int D, int DF>
__device__ __forceinline__ void load_state_tiles(f32x16 (&S)[DF / 32], const float* Sp, int w) {
  const int l = threadIdx.x & 63, h = l >> 5, li = l & 31;
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * cb + 8 * (r >> 2) + 4 * h + (r & 3);
      S[cb][r] = Sp ? Sp[(long long)c * D + 32 * w + li] : 0.f;
    }
}

template <int D, int DF>
__device__ __forceinline__ void add_state_tiles(f32x16 (&S)[DF / 32], const float* Sp, int w) {
  const int l = threadIdx.x & 63, h = l >> 5, li = l & 31;
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * cb + 8 * (r >> 2) + 4 * h + (r & 3);
      S[cb][r] += Sp[(long long)c * D + 32 * w + li];
    }
}

template <int D, int DF>
__device__ __forceinline__ void store_state_tiles(const f32x16 (&S)[DF / 32], float* Sp, int w) {
  const int l = threadIdx.x & 63, h = l >> 5, li = l & 31;
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * cb + 8 * (r >> 2) + 4 * h + (r & 3);
      Sp[(long long)c * D + 32 * w + li] = S[cb][r];
    }
}

// ---------------------------------------------------------------------------
// State pass: local (S, z) of every segment. NW = D/32 value blocks times KS
// key splits: wave w = nw + NW ks owns value columns [32 nw, 32 nw + 32) of
// S and, of every 64-row chunk, the 16-key blocks kb = ks, ks + KS, ..; all
// threads stage. The KS partial states are added through LDS at the end.
// Splitting the keys gives every SIMD two waves at d = 64 and 128 (one wave
// per SIMD runs its VALU staging at about half the SIMD's rate).
// HILO (bf16 operands, for the gradient passes): phi(K) enters S as hi + lo
// bf16 tiles, so S carries phi(k) to about 2^-16 instead of 2^-9 (the
// gradient with respect to q magnifies that rounding where phi(k) varies
// little over the keys).
// grid = (BH, P), block = StateGeo<D, HILO>::NT threads.
// ---------------------------------------------------------------------------
// The hi + lo-keys variant keeps one key split: the gradient passes launch
// twice as many segments, which already puts two of its workgroups on every
// compute unit (with eight waves per block only one would fit).
template <int D, bool HILO = false>
struct StateGeo {
  static constexpr int NW = D / 32;                           // value blocks
  static constexpr int KS = HILO ? 1 : D == 128 ? 2 : 4;      // key splits (4 key blocks per chunk)
  static constexpr int NT = 64 * NW * KS;                     // 512 threads at d = 64 and 128, 256 at d = 32
  static constexpr int KPW = 4 / KS;                          // key blocks per wave and chunk
};

template <int D, int DF, typename OP, typename IN, int FM, bool DECAY, bool HILO = false>
__global__ __launch_bounds__((StateGeo<D, HILO>::NT), (HILO ? 2 : 1)) void state_pass_kernel(FwdArgs a) {
  using Frag = typename Ops<OP>::frag;
  using SG = StateGeo<D, HILO>;
  constexpr int NT = SG::NT, NW = SG::NW, KS = SG::KS, NWT = NW * KS;
  using G = Stage<D, DF, NT>;
  static_assert(!HILO || (sizeof(OP) == 2 && DF == D), "hi + lo keys: bf16 operands, d' = d");
  constexpr int RBF = DF * Ops<OP>::kBytes;
  constexpr int RBV = D * Ops<OP>::kBytes;
  constexpr int KB = 64 * RBF, VB = 64 * RBV, BUF = KB + VB + (HILO ? KB : 0);
  constexpr int NS = G::template nset<DECAY>();  // register sets in the load rotation
  // two staged chunks when they fit; otherwise one, with an extra barrier.
  // The hi + lo-keys variant stages one: two of its larger buffers would
  // leave room for one workgroup per CU, one buffer for two.
  constexpr int NB = (!HILO && 2 * BUF + NWT * DF * 4 <= 160 * 1024) ? 2 : 1;
  // the end of the pass reuses the buffers for one key split's partial states
  constexpr int RED = NW * DF * 128;
  constexpr int SMEM = NB * BUF > RED ? NB * BUF : RED;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ float zsum[NWT][DF];

  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg_state;
  const int c1 = min(c0 + a.chunks_per_seg_state, a.nchunks);
  const long long base = (long long)bh * a.N;
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  const int p = threadIdx.x, l = p & 63;
  const int wv = __builtin_amdgcn_readfirstlane(p >> 6);
  const int w = wv % NW, ks = wv / NW;  // value block, key split

  f32x16 S[DF / 32];
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb) S[cb] = f32x16{};
  float zr[8], cs[8], dp[G::NQ];
#pragma unroll
  for (int e = 0; e < 8; ++e) zr[e] = 0.f;
  const Voff<D, DF, IN, NT> vo(p);
  const float lg = DECAY ? decay_log2(a.gamma[bh % a.H], a.status_flag) : 0.f;
  const float gH = DECAY ? gpow(lg, kChunk / 2) : 1.f;  // gamma^32; a chunk moves states on by gH^2

  // every load is issued (with zero size past the segment) so that all
  // iterations have the same memory instruction stream
  const int nch = c1 - c0;
  auto load = [&](Pref<D, DF, IN, NT>& pf, int m) {
    const int c = c0 + m;
    const int valid = m < nch ? min(64, a.N - 64 * c) : 0;
    prod_load<D, DF, IN, false, true>(pf, vo, nullptr, k, v, base + 64LL * min(c, a.nchunks - 1), valid);
  };
  auto stage = [&](Pref<D, DF, IN, NT>& pf, int m) {
    const int c = c0 + m;
    mask_tail_keys<D, DF, IN, FM>(pf, p, min(64, a.N - 64 * c));
    uint8_t* sK = smem + (NB == 2 ? (m & 1) : 0) * BUF;
    if constexpr (DECAY) {
      // scaled keys (see the decay note above); v pieces raw
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] = 0.f;
      if constexpr (HILO) {
        uint8_t* sKl = sK + KB + VB;
#pragma unroll
        for (int i = 0; i < G::NQ; ++i) {
          const int row = p / G::RLF + G::RSF * i, col = 8 * (p % G::RLF);
          const float sc = gpow(lg, kDecayCenter - row);
          float x[8], lo[8];
          In8<IN>::to_f32(pf.k[i], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = fmap_in_stage<FM>(x[e]) * sc;
            cs[e] += x[e];
            lo[e] = x[e] - round_bf16(x[e]);
          }
          Ops<OP>::template store8<RBF>(sK, row, col, x);
          Ops<OP>::template store8<RBF>(sKl, row, col, lo);
        }
      } else {
#pragma unroll
        for (int i = 0; i < G::NQ; ++i)
          stage_k_piece<D, DF, IN, OP, FM, true, NT>(pf.k[i], p, i, 64, sK, cs,
                                                     gpow(lg, kDecayCenter - (p / G::RLF + G::RSF * i)));
      }
#pragma unroll
      for (int i = 0; i < G::NV; ++i)
        store_raw<IN, OP, RBV>(sK + KB, p / G::RLV + G::RSV * i, 8 * (p % G::RLV), pf.v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) zr[e] = gH * (gH * zr[e]) + cs[e];
    } else if constexpr (HILO) {
      uint8_t* sKl = sK + KB + VB;
#pragma unroll
      for (int i = 0; i < G::NQ; ++i) {
        const int row = p / G::RLF + G::RSF * i, col = 8 * (p % G::RLF);
        float x[8], lo[8];
        In8<IN>::to_f32(pf.k[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = fmap_in_stage<FM>(x[e]);
          zr[e] += x[e];
          lo[e] = x[e] - round_bf16(x[e]);
        }
        Ops<OP>::template store8<RBF>(sK, row, col, x);
        Ops<OP>::template store8<RBF>(sKl, row, col, lo);
        store_raw<IN, OP, RBV>(sK + KB, row, col, pf.v[i]);
      }
    } else {
      prod_stage<D, DF, IN, OP, FM, false, true>(pf, p, nullptr, sK, sK + KB, zr, dp, cs);
#pragma unroll
      for (int e = 0; e < 8; ++e) zr[e] += cs[e];
    }
  };
  // iteration m: multiply the wave's key blocks of chunk m (in LDS), stage
  // chunk m+1, and keep the loads of the following chunk(s) in flight
  auto mult = [&](int m) {
    const uint8_t* sK = smem + (NB == 2 ? (m & 1) : 0) * BUF;
    const uint8_t* sV = sK + KB;
    if constexpr (DECAY) {
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb) S[cb] *= gH * gH;
    }
    Frag Vf[SG::KPW];
#pragma unroll
    for (int j = 0; j < SG::KPW; ++j) Vf[j] = Ops<OP>::template load_cols<RBV>(sV, 16 * (ks + KS * j), 32 * w);
#pragma unroll
    for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
      for (int j = 0; j < SG::KPW; ++j) {
        const int kb = ks + KS * j;
        Ops<OP>::mma(S[cb], Ops<OP>::template load_cols<RBF>(sK, 16 * kb, 32 * cb), Vf[j]);
        if constexpr (HILO) Ops<OP>::mma(S[cb], Ops<OP>::template load_cols<RBF>(sV + VB, 16 * kb, 32 * cb), Vf[j]);
      }
  };
  // iteration m multiplies chunk m (LDS), stages chunk m+1 (registers) and
  // issues the loads of chunk m+NSET into the set chunk m occupied
  // The rotation of register sets runs whole (iteration count rounded up to
  // a multiple of NSET); iterations past the segment multiply nothing and
  // only retire their (empty) loads.
  auto iter = [&](int m, Pref<D, DF, IN, NT>& ld, Pref<D, DF, IN, NT>& st) {
    load(ld, m + NS);
    if (m < nch) mult(m);
    if constexpr (NB == 1) __syncthreads();
    if (m + 1 < nch) stage(st, m + 1);
    else retire<D, DF, IN, false, true>(st);
    __syncthreads();
  };
  static_assert(NS == 2, "two register sets rotate");
  const int nround = (nch + NS - 1) / NS * NS;
  {
    Pref<D, DF, IN, NT> pA, pB;
    load(pA, 0);
    load(pB, 1);
    if (nch > 0) stage(pA, 0);
    else retire<D, DF, IN, false, true>(pA);
    __syncthreads();
    for (int m = 0; m < nround; m += 2) {
      iter(m, pA, pB);
      iter(m + 1, pB, pA);
    }
  }
  // z: reduce the per-thread column sums over rows (lanes, then waves)
#pragma unroll
  for (int e = 0; e < 8; ++e) zr[e] = col_reduce<G::RLF>(zr[e]);
  if (l < G::RLF) {
#pragma unroll
    for (int e = 0; e < 8; ++e) zsum[wv][8 * l + e] = zr[e];
  }
  // S: the key splits ks = 1 .. KS-1 hand their partial tiles to ks = 0, one
  // split at a time, through the (now idle) staging buffers
  f32x4* red = reinterpret_cast<f32x4*>(smem);
#pragma unroll
  for (int r = 1; r < KS; ++r) {
    __syncthreads();
    if (ks == r) {
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          red[((w * (DF / 32) + cb) * 4 + g) * 64 + l] = f32x4{S[cb][4 * g], S[cb][4 * g + 1], S[cb][4 * g + 2], S[cb][4 * g + 3]};
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = red[((w * (DF / 32) + cb) * 4 + g) * 64 + l];
#pragma unroll
          for (int e = 0; e < 4; ++e) S[cb][4 * g + e] += x[e];
        }
    }
  }
  __syncthreads();
  float* st = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
  const float fr = DECAY ? gpow(lg, kDecayFrame) : 1.f;  // back from the scaled frame
  if (ks == 0) {
    if constexpr (DECAY) {
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb) S[cb] *= fr;
    }
    store_state_tiles<D, DF>(S, st, w);
  }
  for (int c = p; c < DF; c += NT) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWT; ++ww) s += zsum[ww][c];
    st[DF * D + c] = fr * s;
  }
}

// ---------------------------------------------------------------------------
// Carry scan: ws[bh][p] <- init + sum_{p' < p} ws[bh][p']  (exclusive), and
// the total into ws[bh][P] (and S_out/z_out) when requested.
// grid = (BH, ceil(state_elems/1024)), block = 256.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void carry_scan_kernel(ScanArgs a) {
  // four consecutive state elements per thread (the state size d'(d+1) is a
  // multiple of 4 and every slot starts 16-byte aligned); the loads of up to
  // kScanBatch segments are issued before their dependent adds and stores
  const int e = 4 * (blockIdx.y * 256 + threadIdx.x);
  const int bh = blockIdx.x;
  if (e >= a.state_elems) return;
  const int sdd = a.DF * a.D;
  f32x4 run = {0.f, 0.f, 0.f, 0.f};
  if (e < sdd) {
    if (a.S_in) run = *reinterpret_cast<const f32x4*>(a.S_in + (long long)bh * sdd + e);
  } else {
    if (a.z_in) run = *reinterpret_cast<const f32x4*>(a.z_in + (long long)bh * a.DF + (e - sdd));
  }
  float* col = a.ws + (long long)bh * a.ws_slots * a.state_elems + e;
  const long long st = a.state_elems;
  // decay: each combined segment of seg_len tokens multiplies what precedes it by gamma^seg_len
  const float g = a.gamma ? gpow(decay_log2(a.gamma[bh % a.H], a.status_flag), (float)a.seg_len) : 1.f;
  constexpr int kScanBatch = 32;
  for (int p0 = 0; p0 < a.P; p0 += kScanBatch) {
    const int cnt = min(kScanBatch, a.P - p0);
    f32x4 t[kScanBatch];
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j)
      if (j < cnt) t[j] = *reinterpret_cast<const f32x4*>(col + (p0 + j) * st);
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      if (j < cnt) {
        if (a.exclusive) *reinterpret_cast<f32x4*>(col + (p0 + j) * st) = run;
        f32x4 gf = {g, g, g, g};
        if (a.lfac) {  // gated: per-channel factor of the combined segment (row of S, or entry of z)
          const float* lf = a.lfac + ((long long)bh * a.lfac_stride + p0 + j) * a.DF;
          if (e < sdd) {
            const float x = gpow(lf[e / a.D] * 1.4426950408889634f, 1.f);
            gf = f32x4{x, x, x, x};
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) gf[u] = gpow(lf[e - sdd + u] * 1.4426950408889634f, 1.f);
          }
        }
        run[0] = gf[0] * run[0] + t[j][0];
        run[1] = gf[1] * run[1] + t[j][1];
        run[2] = gf[2] * run[2] + t[j][2];
        run[3] = gf[3] * run[3] + t[j][3];
      }
    }
  }
  if (a.write_total) *reinterpret_cast<f32x4*>(col + a.P * st) = run;
  if (e < sdd) {
    if (a.S_out) *reinterpret_cast<f32x4*>(a.S_out + (long long)bh * sdd + e) = run;
  } else {
    if (a.z_out) *reinterpret_cast<f32x4*>(a.z_out + (long long)bh * a.DF + (e - sdd)) = run;
  }
}

// ---------------------------------------------------------------------------
// Output pass.
// CAUSAL: y_i = [sum_{j<=i in chunk} w_ij v_j + phi(q_i)^T S_prev] / [..]
// otherwise: y_i = phi(q_i)^T S / phi(q_i)^T z with the total (S, z).
// grid = (BH, P), block = 2 * 64 * D/32 threads (consumers, then producers).
// ---------------------------------------------------------------------------
template <int D, int DF, typename OP, typename IN, bool CAUSAL>
struct OutLayout {
  static constexpr int NWC = D / 32, NWP = D / 32;
  static constexpr int RBF = DF * Ops<OP>::kBytes;
  static constexpr int RBV = D * Ops<OP>::kBytes;
  static constexpr int QB = 64 * RBF, KB = CAUSAL ? 64 * RBF : 0, VB = CAUSAL ? 64 * RBV : 0;
  static constexpr int BUF = QB + KB + VB;
  static constexpr int DEN = 2 * 64 * 4;                         // den_inter, double-buffered
  static constexpr int ZP = CAUSAL ? 2 * NWP * DF * 4 : 0;       // colsum partials, double-buffered
  // two staged chunks when they fit in LDS; otherwise one, with an extra
  // barrier per step so the producers wait for the consumers
  static constexpr int NB = (2 * BUF + DEN + ZP <= 160 * 1024) ? 2 : 1;
  static constexpr int NBAR = NB == 2 ? 1 : 2;
  // output tiles go through LDS (double-buffered) and the producers store
  // them as whole rows one step later, when that fits
  static constexpr int RBY = D * (int)sizeof(IN);
  static constexpr int YB1 = 64 * RBY;
  static constexpr bool YS = NB * BUF + DEN + ZP + 2 * YB1 <= 160 * 1024;
  static constexpr int YB = YS ? 2 * YB1 : 0;
  static constexpr int BYTES = NB * BUF + DEN + ZP + YB;
};

template <int D, int DF, typename OP, typename IN, int FM, bool CAUSAL, bool DECAY>
__global__ __launch_bounds__(D * 4) void output_pass_kernel(FwdArgs a) {
  static_assert(!DECAY || CAUSAL, "decay is defined for the causal form only");
  using Frag = typename Ops<OP>::frag;
  using L = OutLayout<D, DF, OP, IN, CAUSAL>;
  using G = Stage<D, DF>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[L::BYTES];
  float* dbuf = reinterpret_cast<float*>(smem + L::NB * L::BUF);
  float* zpart = reinterpret_cast<float*>(smem + L::NB * L::BUF + L::DEN);
  uint8_t* ybuf = smem + L::NB * L::BUF + L::DEN + L::ZP;
  constexpr int LAST = L::YS ? 1 : 0;  // extra step in which the last output tile is stored

  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int n = max(0, min(c0 + a.chunks_per_seg, a.nchunks) - c0);
  // Producer steps IT0 .. itend-1, whole rotations of the register sets. The
  // first NSET-1 steps (negative) only issue the loads of chunks 0..NSET-2, so
  // the loop is entered with no loads in flight and the wait counts inside it
  // follow the steady state alone. Steps past n + LAST only retire empty loads.
  constexpr int NS = Stage<D, DF>::template nset<DECAY>();
  constexpr int IT0 = -(NS - 1);
  const int itend = IT0 + (n + LAST + 1 - IT0 + NS - 1) / NS * NS;
  const long long base = (long long)bh * a.N;
  const IN* q = static_cast<const IN*>(a.q);
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  IN* out = static_cast<IN*>(a.out);
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, li = l & 31;
  const bool producer = wave >= L::NWC;
  const int p = threadIdx.x - 64 * L::NWC;     // producer thread index
  const int pw = wave - L::NWC;                // producer wave index
  const int cw = wave;                         // consumer wave = value-column block

  // decay: per-head gamma, the per-chunk factor and the factor of the final
  // state (scaled frame back to the true one, and a partial last chunk of
  // vl rows moved on by gamma^vl instead of gamma^64)
  const float lg = DECAY ? decay_log2(a.gamma[bh % a.H], a.status_flag) : 0.f;
  const float gH = DECAY ? gpow(lg, kChunk / 2) : 1.f;  // gamma^32; a chunk moves states on by gH^2
  const int vl = a.N - kChunk * (a.nchunks - 1);
  const float fout = DECAY ? gpow(lg, kDecayFrame + vl - kChunk) : 1.f;
  const float fin = DECAY ? gpow(lg, -kDecayFrame) : 1.f;

  const float* Sinit;
  const float* zinit;
  if (a.init_from_ws) {
    const float* st = a.ws + ((long long)bh * a.ws_slots + (CAUSAL ? seg : a.ws_total_slot)) * a.state_elems;
    Sinit = st;
    zinit = st + DF * D;
  } else {
    Sinit = a.S_in ? a.S_in + (long long)bh * DF * D : nullptr;
    zinit = a.z_in ? a.z_in + (long long)bh * DF : nullptr;
  }

  if (producer) {
    // ------------------------------------------------------------------
    // producers: chunk `it` is loaded NSET-1 steps before step it stages it
    // ------------------------------------------------------------------
    // The producers are the critical path; a producer and a consumer wave
    // share each SIMD, and the raised priority lets the producer's VALU and
    // memory instructions issue first (about 3% on the long-context shape).
    __builtin_amdgcn_s_setprio(1);
    float zrun[8], dp[G::NQ], cs[8];
    const int cr = 8 * (p % G::RLF);
    const Voff<D, DF, IN> vo(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) zrun[e] = zinit ? fin * zinit[cr + e] : 0.f;
    if constexpr (CAUSAL && !DECAY) {
      if (a.init_sum_ws) {  // the carried normalizer: local sums of the segments before this one
#pragma unroll 4
        for (int j = 0; j < seg; ++j) {
          const float* zj = a.ws + ((long long)bh * a.ws_slots + j) * a.state_elems + DF * D + cr;
#pragma unroll
          for (int e = 0; e < 8; ++e) zrun[e] += zj[e];
        }
      }
    }
    // Drain that load now: otherwise the wait-count analysis carries it
    // around the loop and waits for every outstanding prefetch each step.
    wait_vmem_all();
    // every load and store below is issued in every step (zero size when out
    // of range), so the wait counts are the same on every path


    // step `it` stores the output tile of chunk it-2, stages chunk it (held
    // in `cur`) and issues the loads of chunk it+NSET-1 into `nxt`
    // Step `it` stores the output tile of chunk it-2, stages chunk it (held
    // in `cur`) and loads chunk it+NSET-1 into `nxt`, piece by piece.
    constexpr int NSLOT = G::NQ > 4 ? G::NQ : 4;
    auto pstep = [&](int it, Pref<D, DF, IN>& cur, Pref<D, DF, IN>& nxt) {
      const bool stg = it >= 0 && it < n;
      const int cs_ = c0 + it;                       // chunk staged in this step
      const int vs = stg ? min(64, a.N - 64 * cs_) : 0;
      const int ln = it + NS - 1;                    // chunk loaded in this step
      const int cl = c0 + ln;
      const ChunkRsrc rl = chunk_rsrc<D, DF, IN>(q, k, v, base + 64LL * min(cl, a.nchunks - 1),
                                                 ln < n ? min(64, a.N - 64 * cl) : 0);
      const int cy = c0 + max(0, min(it - 2, n - 1));  // chunk whose output tile is stored
      const int vy = (it >= 2 && it - 2 < n) ? min(64, a.N - 64 * cy) : 0;
      const auto ro = make_rsrc(out + (base + 64LL * cy) * D, (unsigned)(vy * D * (int)sizeof(IN)));
      const uint8_t* yb = ybuf + (it & 1) * L::YB1;
      uint8_t* sQ = smem + (L::NB == 2 ? (it & 1) : 0) * L::BUF;
      uint8_t* sK = sQ + L::QB;
      uint8_t* sV = sK + L::KB;
      if constexpr (CAUSAL) {
        // z_{it-1} = z_{it-2} + column sums of chunk it-1 (all producer waves)
        if (stg && it >= 1) {
          const float* zp = zpart + ((it - 1) & 1) * L::NWP * DF;
#pragma unroll
          for (int ww = 0; ww < L::NWP; ++ww) {
            const f32x4 z0 = *reinterpret_cast<const f32x4*>(zp + ww * DF + cr);
            const f32x4 z1 = *reinterpret_cast<const f32x4*>(zp + ww * DF + cr + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              zrun[e] = (ww == 0 ? gH * (gH * zrun[e]) : zrun[e]) + z0[e];
              zrun[4 + e] = (ww == 0 ? gH * (gH * zrun[4 + e]) : zrun[4 + e]) + z1[e];
            }
          }
        }
      }
      if constexpr (L::NB == 1) __syncthreads();  // consumers are done with the buffer
      // decay: the carried normalizer moved on by gamma^64 before the dot
      // product with the scaled q rows (the two scales would overflow apart)
      float zs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        zs[e] = gH * (gH * zrun[e]);
        cs[e] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < NSLOT; ++i) {
        if (i < 4) {
          if constexpr (L::YS) {
            const int row = p / G::RLV + 16 * i, col = 8 * (p % G::RLV);
            if constexpr (sizeof(IN) == 2) {
              buf_store16_nt(ro, vo.v(i), *reinterpret_cast<const u32x4*>(yb + tile_off<L::RBY>(row, col * 2)));
            } else {
              buf_store16_nt(ro, vo.v(i), *reinterpret_cast<const u32x4*>(yb + tile_off<L::RBY>(row, col * 4)));
              buf_store16_nt(ro, vo.v(i) + 16,
                             *reinterpret_cast<const u32x4*>(yb + tile_off<L::RBY>(row, col * 4 + 16)));
            }
          }
        }
        if (i < G::NQ) {
          nxt.q[i] = In8<IN>::bload_nt(rl.q, vo.f[i]);
          if constexpr (CAUSAL) nxt.k[i] = In8<IN>::bload(rl.k, vo.f[i]);
        }
        if constexpr (CAUSAL) {
          if (i < 4) nxt.v[i] = In8<IN>::bload(rl.v, vo.v(i));
        }
        if (stg) {
          if (i < G::NQ) {
            const int row = p / G::RLF + G::RSF * i;
            dp[i] = stage_q_piece<D, DF, IN, OP, FM, DECAY>(cur.q[i], p, i, sQ, zs,
                                                            DECAY ? gpow(lg, row - kDecayCenter) : 1.f);
            if constexpr (CAUSAL)
              stage_k_piece<D, DF, IN, OP, FM, DECAY>(cur.k[i], p, i, vs, sK, cs,
                                                      DECAY ? gpow(lg, kDecayCenter - row) : 1.f);
          }
          if constexpr (CAUSAL) {
            if (i < 4) store_raw<IN, OP, L::RBV>(sV, p / G::RLV + 16 * i, 8 * (p % G::RLV), cur.v[i]);
          }
        }
      }
      if (stg) {
        if constexpr (CAUSAL) {
          // publish this chunk's column sums of phi(K)
#pragma unroll
          for (int e = 0; e < 8; ++e) cs[e] = col_reduce<G::RLF>(cs[e]);
          if (l < G::RLF) {
            float* zw = zpart + (it & 1) * L::NWP * DF + pw * DF + cr;
            *reinterpret_cast<f32x4*>(zw) = f32x4{cs[0], cs[1], cs[2], cs[3]};
            *reinterpret_cast<f32x4*>(zw + 4) = f32x4{cs[4], cs[5], cs[6], cs[7]};
          }
        }
        // cross-chunk denominator phi(q_i).z_{it-1} for the thread's rows
        if (a.normalize) {
          float* db = dbuf + (it & 1) * 64;
#pragma unroll
          for (int i = 0; i < G::NQ; ++i) {
            const float s = row_reduce<G::RLF>(dp[i]);
            if ((p % G::RLF) == 0) db[p / G::RLF + G::RSF * i] = s;
          }
        }
      } else {
        retire<D, DF, IN, true, CAUSAL>(cur);
        if constexpr (CAUSAL) if (it == n) {
          // final z = z_{n-2} + column sums of the last chunk
          const float* zp = zpart + ((it - 1) & 1) * L::NWP * DF;
#pragma unroll
          for (int e = 0; e < 8; ++e) zrun[e] = gH * (gH * zrun[e]);
#pragma unroll
          for (int ww = 0; ww < L::NWP; ++ww)
#pragma unroll
            for (int e = 0; e < 8; ++e) zrun[e] += zp[ww * DF + cr + e];
        }
      }
      __syncthreads();
    };
    // whole rotations of the register sets; the steps past n + LAST only
    // retire their empty loads (the consumers run as many barriers)
    // chunk c is held in the set that step c - NSET + 1 loads and step c stages
    static_assert(NS == 2, "two register sets rotate");
    {
      Pref<D, DF, IN> pA, pB;
      for (int it = IT0; it < itend; it += 2) {
        pstep(it, pA, pB);
        pstep(it + 1, pB, pA);
      }
    }
    if constexpr (CAUSAL) {
      if (a.S_out && seg == a.nseg - 1 && p < G::RLF) {
        float* zo = a.z_out + (long long)bh * DF + cr;
#pragma unroll
        for (int e = 0; e < 8; ++e) zo[e] = fout * zrun[e];
      }
    }
  } else {
    // ------------------------------------------------------------------
    // consumers: chunk it-1 in step it
    // ------------------------------------------------------------------
    f32x16 S[DF / 32];
    load_state_tiles<D, DF>(S, Sinit, cw);
    if constexpr (CAUSAL && !DECAY) {
      if (a.init_sum_ws) {  // the carried state: local sums of the segments before this one
#pragma unroll 4
        for (int j = 0; j < seg; ++j)
          add_state_tiles<D, DF>(S, a.ws + ((long long)bh * a.ws_slots + j) * a.state_elems, cw);
      }
    }
    if constexpr (DECAY) {  // entering the first chunk: moved on by gamma^64 in the scaled frame
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb) S[cb] = ((S[cb] * fin) * gH) * gH;
    }
    Frag Sf_const[CAUSAL ? 1 : DF / 16];
    if constexpr (!CAUSAL) {
#pragma unroll
      for (int kb = 0; kb < DF / 16; ++kb) Sf_const[kb] = Ops<OP>::from_acc(S[kb >> 1], kb & 1);
    }
    for (int bar = 0; bar < L::NBAR * (1 - IT0); ++bar) __syncthreads();  // producer steps IT0 .. 0
    for (int it = 1; it < itend; ++it) {
      if (it > n) {  // the producers store the last tile, or idle
        for (int bar = 0; bar < L::NBAR; ++bar) __syncthreads();
        continue;
      }
      const int c = c0 + it - 1;
      const int b = L::NB == 2 ? ((it - 1) & 1) : 0;
      const uint8_t* sQ = smem + b * L::BUF;
      const uint8_t* sK = sQ + L::QB;
      const uint8_t* sV = sK + L::KB;
      const int valid = min(64, a.N - 64 * c);
      f32x16 num0 = {}, num1 = {};
      float dpart0 = 0.f, dpart1 = 0.f;
      Frag Vf[4];
      if constexpr (CAUSAL) {
        f32x16 A00 = {}, A01 = {}, A11 = {};
#pragma unroll
        for (int kb = 0; kb < DF / 16; ++kb) {
          const Frag bq0 = Ops<OP>::template load_rows<L::RBF>(sQ, 0, 16 * kb);
          const Frag bq1 = Ops<OP>::template load_rows<L::RBF>(sQ, 32, 16 * kb);
          const Frag k0 = Ops<OP>::template load_rows<L::RBF>(sK, 0, 16 * kb);
          const Frag k1 = Ops<OP>::template load_rows<L::RBF>(sK, 32, 16 * kb);
          Ops<OP>::mma(A00, k0, bq0);
          Ops<OP>::mma(A01, k0, bq1);
          Ops<OP>::mma(A11, k1, bq1);
          const Frag sf = Ops<OP>::from_acc(S[kb >> 1], kb & 1);
          Ops<OP>::mma(num0, sf, bq0);
          Ops<OP>::mma(num1, sf, bq1);
        }

        // causal mask on the diagonal tiles (keep j <= i) and the in-chunk
        // part of the denominator
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jt = 8 * (r >> 2) + 4 * h + (r & 3);
          const bool keep = jt <= li;
          A00[r] = keep ? A00[r] : 0.f;
          A11[r] = keep ? A11[r] : 0.f;
          dpart0 += A00[r];
          dpart1 += A01[r] + A11[r];
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Vf[kb] = Ops<OP>::template load_cols<L::RBV>(sV, 16 * kb, 32 * cw);
#pragma unroll
        for (int kbj = 0; kbj < 2; ++kbj) {
          Ops<OP>::mma(num0, Vf[kbj], Ops<OP>::from_acc(A00, kbj));
          Ops<OP>::mma(num1, Vf[kbj], Ops<OP>::from_acc(A01, kbj));
          Ops<OP>::mma(num1, Vf[2 + kbj], Ops<OP>::from_acc(A11, kbj));
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < DF / 16; ++kb) {
          Ops<OP>::mma(num0, Sf_const[kb], Ops<OP>::template load_rows<L::RBF>(sQ, 0, 16 * kb));
          Ops<OP>::mma(num1, Sf_const[kb], Ops<OP>::template load_rows<L::RBF>(sQ, 32, 16 * kb));
        }
      }
      // normalize and store: lane holds y[i = 32ib + li][e = 32cw + 8(r/4) + 4h + r%4]
      const float* db = dbuf + ((it - 1) & 1) * 64;
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const f32x16& nm = ib ? num1 : num0;
        float inv = 1.f;
        if (a.normalize) {
          const float dp = ib ? dpart1 : dpart0;
          const float den = dp + xor32(dp) + db[32 * ib + li];
          inv = 1.f / fmaxf(den, kEps);
        }
        const int i = 32 * ib + li;
        if constexpr (L::YS) {
          uint8_t* yb = ybuf + ((it - 1) & 1) * L::YB1;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float y0 = nm[4 * g + 0] * inv, y1 = nm[4 * g + 1] * inv;
            const float y2 = nm[4 * g + 2] * inv, y3 = nm[4 * g + 3] * inv;
            const int e = 32 * cw + 8 * g + 4 * h;
            if constexpr (sizeof(IN) == 2) {
              *reinterpret_cast<u32x2*>(yb + tile_off<L::RBY>(i, e * 2)) =
                  u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
            } else {
              *reinterpret_cast<f32x4*>(yb + tile_off<L::RBY>(i, e * 4)) = f32x4{y0, y1, y2, y3};
            }
          }
        } else if (i < valid) {
          const long long rowoff = (base + 64LL * c + i) * D + 32 * cw + 4 * h;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float y0 = nm[4 * g + 0] * inv, y1 = nm[4 * g + 1] * inv;
            const float y2 = nm[4 * g + 2] * inv, y3 = nm[4 * g + 3] * inv;
            if constexpr (sizeof(IN) == 2) {
              *reinterpret_cast<u32x2*>(out + rowoff + 8 * g) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
            } else {
              *reinterpret_cast<f32x4*>(out + rowoff + 8 * g) = f32x4{y0, y1, y2, y3};
            }
          }
        }
      }
      if constexpr (CAUSAL) {
#pragma unroll
        for (int cb = 0; cb < DF / 32; ++cb)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            Ops<OP>::mma(S[cb], Ops<OP>::template load_cols<L::RBF>(sK, 16 * kb, 32 * cb), Vf[kb]);
        if constexpr (DECAY) {  // the state as the next chunk's rows see it: moved on by gamma^64
          if (it < n) {
#pragma unroll
            for (int cb = 0; cb < DF / 32; ++cb) S[cb] *= gH * gH;
          }
        }
      }
      for (int bar = 0; bar < L::NBAR; ++bar) __syncthreads();
    }
    if constexpr (CAUSAL) {
      if (a.S_out && seg == a.nseg - 1) {
        if constexpr (DECAY) {
#pragma unroll
          for (int cb = 0; cb < DF / 32; ++cb) S[cb] *= fout;
        }
        store_state_tiles<D, DF>(S, a.S_out + (long long)bh * DF * D, cw);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (one instantiation per supported shape)
// ---------------------------------------------------------------------------
template <int D, int DF, typename OP, typename IN, int FM, bool DECAY>
static hipError_t launch_prefill_t(const FwdArgs& a, const ScanArgs& s, bool causal, hipStream_t st,
                                   hipEvent_t* ev) {
  // ev[0] is recorded by the caller (before any feature-map kernels)
  if (a.run_state_pass) {
    constexpr bool kHiloOk = sizeof(OP) == 2 && DF == D;
    if (kHiloOk && a.hilo_keys)
      hipLaunchKernelGGL((state_pass_kernel<D, DF, OP, IN, FM, DECAY, kHiloOk>), dim3(a.BH, a.nseg_state),
                         dim3(StateGeo<D, kHiloOk>::NT), 0, st, a);
    else
      hipLaunchKernelGGL((state_pass_kernel<D, DF, OP, IN, FM, DECAY>), dim3(a.BH, a.nseg_state),
                         dim3(StateGeo<D>::NT), 0, st, a);
  }
  if (ev) (void)hipEventRecord(ev[1], st);
  if (a.run_scan) {
    hipLaunchKernelGGL(carry_scan_kernel, dim3(s.BH, (s.state_elems / 4 + 255) / 256), dim3(256), 0, st, s);
  }
  if (ev) (void)hipEventRecord(ev[2], st);
  if (a.skip_output) return hipGetLastError();
  if (causal) {
    hipLaunchKernelGGL((output_pass_kernel<D, DF, OP, IN, FM, true, DECAY>), dim3(a.BH, a.nseg), dim3(D * 4), 0, st,
                       a);
  } else {
    if constexpr (DECAY) return hipErrorInvalidValue;
    else
      hipLaunchKernelGGL((output_pass_kernel<D, DF, OP, IN, FM, false, false>), dim3(a.BH, a.nseg), dim3(D * 4), 0,
                         st, a);
  }
  if (ev) (void)hipEventRecord(ev[3], st);
  return hipGetLastError();
}

template <int D, int DF, typename OP, typename IN, int FM>
static hipError_t launch_prefill(const FwdArgs& a, const ScanArgs& s, bool causal, bool decay, hipStream_t st,
                                 hipEvent_t* ev) {
  if (decay) return launch_prefill_t<D, DF, OP, IN, FM, true>(a, s, causal, st, ev);
  return launch_prefill_t<D, DF, OP, IN, FM, false>(a, s, causal, st, ev);
}

template <typename T>
static hipError_t prefill_typed(const FwdArgs& a, const ScanArgs& s, int D, int DF, int fmap, bool causal, bool decay,
                                hipStream_t st, hipEvent_t* ev) {
  if (fmap == kElu1) {
    switch (D) {
      case 32: return launch_prefill<32, 32, T, T, kElu1>(a, s, causal, decay, st, ev);
      case 64: return launch_prefill<64, 64, T, T, kElu1>(a, s, causal, decay, st, ev);
      case 128: return launch_prefill<128, 128, T, T, kElu1>(a, s, causal, decay, st, ev);
    }
    return hipErrorInvalidValue;
  }
#define LA_PRE_CASE(d, m) \
  if (D == d && DF == m) return launch_prefill<d, m, T, T, kIdentity>(a, s, causal, decay, st, ev);
  LA_PRE_CASE(32, 32) LA_PRE_CASE(32, 64) LA_PRE_CASE(32, 128)
  LA_PRE_CASE(64, 64) LA_PRE_CASE(64, 128) LA_PRE_CASE(64, 256)
  LA_PRE_CASE(128, 64) LA_PRE_CASE(128, 128)
#undef LA_PRE_CASE
  return hipErrorInvalidValue;
}

hipError_t scan_dispatch(const ScanArgs& s, hipStream_t st) {
  hipLaunchKernelGGL(carry_scan_kernel, dim3(s.BH, (s.state_elems / 4 + 255) / 256), dim3(256), 0, st, s);
  return hipGetLastError();
}

hipError_t prefill_dispatch(const FwdArgs& a, const ScanArgs& s, int D, int DF, int fmap, int dtype, bool causal,
                            bool decay, hipStream_t st, hipEvent_t* ev) {
  if (fmap != kElu1 && fmap != kIdentity) return hipErrorInvalidValue;
  if (decay && !causal) return hipErrorInvalidValue;
  if (dtype == 1) return prefill_typed<__bf16>(a, s, D, DF, fmap, causal, decay, st, ev);
  return prefill_typed<float>(a, s, D, DF, fmap, causal, decay, st, ev);
}

}  // namespace la

// Gradients of causal chunked linear attention on gfx950.
//
// "Linear Attention" (marovi.ai), "Entrenamiento: forma paralela", motivates
// the blockwise form by training; the pages print no gradient formulas.
// Differentiating y_i = num_i / max(den_i, eps), num_i = sum_{j<=i}
// (phi(q_i).phi(k_j)) v_j, den_i = sum_{j<=i} phi(q_i).phi(k_j) (plus an
// initial state), with the output cotangents dY, gives per token
//   D_i = max(den_i, eps),  g_i = dY_i / D_i,  h_i = -(dY_i . num_i) / D_i^2
//   (h_i = 0 when den_i < eps; without normalization g = dY, h = 0)
//   d phi(q_i) = sum_{j<=i} phi(k_j) (g_i.v_j + h_i)        [= S_i g_i + z_i h_i]
//   d phi(k_j) = sum_{i>=j} phi(q_i) (g_i.v_j + h_i)        [= R_j v_j + r_j]
//   dv_j       = sum_{i>=j} (phi(q_i).phi(k_j)) g_i        [= R_j^T phi(k_j)]
// with the suffix states R_j = dS_N + sum_{i>=j} phi(q_i) g_i^T and
// r_j = dz_N + sum_{i>=j} phi(q_i) h_i, and dq, dk through phi'
// (elu+1: phi' = 1 for x > 0, exp(x) otherwise, i.e. min(phi(x), 1)).
//
// Passes (each (batch, head) sequence split into P segments of whole chunks
// for the state passes and scans; the dq and dk/dv passes take seg_stride
// (1 or 2) of those at a time):
//   forward state pass + carry scan : state (S, z) entering every segment
//   dq pass      : per chunk, in order: scores, value products, numerator and
//                  denominator terms -> D_i, h_i (kept per token), dq
//   r-state pass : per segment, local sums of phi(q_i) g_i^T and phi(q_i) h_i
//   carry scan   : suffix sums (slots in reverse segment order), seeded with
//                  the final-state cotangents; the total is dS_in, dz_in
//   dk/dv pass   : per chunk, in reverse order, from the segment's suffix state
// Matrix products on the 32x32 MFMA shape (la_device.h): acc[m][n] +=
// sum_k a[m][k] b[n][k], the a-fragment's lanes give the rows m and the
// b-fragment's lanes the columns n of the accumulator.
#include "la_device.h"
#include "la_kernels.h"

namespace la {
namespace {

template <int FM>
__device__ __forceinline__ float bphi(float x) {
  if constexpr (FM == kElu1) return phi_elu1(x);
  else return x;
}
// phi'(x) from phi(x): elu+1 -> min(phi, 1); identity -> 1
template <int FM>
__device__ __forceinline__ float bdphi(float f) {
  if constexpr (FM == kElu1) return fminf(f, 1.f);
  else return 1.f;
}

template <typename IN, typename OP, int RB>
__device__ __forceinline__ void put_raw(uint8_t* tile, int row, int col, const typename In8<IN>::raw& r) {
  static_assert(sizeof(IN) == sizeof(OP), "raw staging needs matching element types");
  if constexpr (sizeof(IN) == 2) {
    *reinterpret_cast<u32x4*>(tile + tile_off<RB>(row, col * 2)) = r;
  } else {
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4)) = r.a;
    *reinterpret_cast<f32x4*>(tile + tile_off<RB>(row, col * 4 + 16)) = r.b;
  }
}

// four consecutive operand values of one tile row, as fp32
template <typename OP, int RB>
__device__ __forceinline__ void lds_read4(const uint8_t* tile, int row, int col, float* x) {
  if constexpr (sizeof(OP) == 2) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(tile + tile_off<RB>(row, col * 2));
    x[0] = __uint_as_float(u[0] << 16);
    x[1] = __uint_as_float(u[0] & 0xffff0000u);
    x[2] = __uint_as_float(u[1] << 16);
    x[3] = __uint_as_float(u[1] & 0xffff0000u);
  } else {
    const f32x4 f = *reinterpret_cast<const f32x4*>(tile + tile_off<RB>(row, col * 4));
    x[0] = f[0];
    x[1] = f[1];
    x[2] = f[2];
    x[3] = f[3];
  }
}

// Lane (li, h) holds y[4 g + c] = row `row`, column col0 + 8 g + 4 h + c of
// a wave's 32-column block (the accumulator layout) of a chunk whose rows
// start at `chunk`. bf16: one swap with the other lane half gives each lane
// 8 consecutive columns (16 p + 8 h ..), so each of its two stores covers 32
// bytes of every row rather than 16. Rows at or past `valid` fall outside
// the descriptor's range. Every lane calls it (the swap pairs lanes l and
// l ^ 32, which hold the same row).
template <typename IN, int D>
__device__ __forceinline__ void store_block_rows(IN* chunk, int valid, int row, int col0, const float (&y)[16]) {
  const auto r = make_rsrc(chunk, (unsigned)(valid * D * (int)sizeof(IN)));
  const int h = (threadIdx.x >> 5) & 1;
  if constexpr (sizeof(IN) == 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int b = 8 * p;
      const uint32_t x0 = pack_bf16x2(y[b], y[b + 1]), x1 = pack_bf16x2(y[b + 2], y[b + 3]);
      const uint32_t z0 = pack_bf16x2(y[b + 4], y[b + 5]), z1 = pack_bf16x2(y[b + 6], y[b + 7]);
      const auto s0 = __builtin_amdgcn_permlane32_swap(x0, z0, false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(x1, z1, false, false);
      buf_store16(r, (row * D + col0 + 16 * p + 8 * h) * 2, u32x4{s0[0], s1[0], s0[1], s1[1]});
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      buf_store16(r, (row * D + col0 + 8 * g + 4 * h) * 4,
                  __builtin_bit_cast(u32x4, f32x4{y[4 * g], y[4 * g + 1], y[4 * g + 2], y[4 * g + 3]}));
  }
}

// operand fragment holding x[0..7] as its 8 contraction values (every lane)
template <typename OP>
__device__ __forceinline__ typename Ops<OP>::frag frag8(const float (&x)[8]) {
  if constexpr (sizeof(OP) == 2) {
    const u32x4 u = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7])};
    return __builtin_bit_cast(typename Ops<OP>::frag, u);
  } else {
    return typename Ops<OP>::frag{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  }
}

// An accumulator block as two bf16 fragments hi + lo (x = hi + lo to within
// 2^-16 |x|): for products whose result is a small difference of large
// terms. Same lane layout as Ops<__bf16>::from_acc.
__device__ __forceinline__ void frag_hilo(const f32x16& c, int kb, bf16x8& hi, bf16x8& lo) {
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = c[8 * kb + 2 * i], x1 = c[8 * kb + 2 * i + 1];
    ph[i] = pack_bf16x2(x0, x1);
    pl[i] = pack_bf16x2(x0 - __uint_as_float(ph[i] << 16), x1 - __uint_as_float(ph[i] & 0xffff0000u));
  }
  // elements 0-3 of the block are rows 0-3 (this half) and 4-7 rows 8-11 of
  // the group of 16; the swap completes 8 contiguous rows per lane half
  auto h0 = __builtin_amdgcn_permlane32_swap(ph[0], ph[2], false, false);
  auto h1 = __builtin_amdgcn_permlane32_swap(ph[1], ph[3], false, false);
  auto l0 = __builtin_amdgcn_permlane32_swap(pl[0], pl[2], false, false);
  auto l1 = __builtin_amdgcn_permlane32_swap(pl[1], pl[3], false, false);
  hi = __builtin_bit_cast(bf16x8, u32x4{h0[0], h1[0], h0[1], h1[1]});
  lo = __builtin_bit_cast(bf16x8, u32x4{l0[0], l1[0], l0[1], l1[1]});
}

// sum over the lanes of a wave that share lane % RL
template <int RL>
__device__ __forceinline__ float lane_colsum(float x) {
#pragma unroll
  for (int s = RL; s < 64; s <<= 1) x += __shfl_xor(x, s, 64);
  return x;
}

// One chunk of q, k, v, dy as raw 16-byte pieces: 4*D threads, two pieces
// per tile each, rows t/(D/8) and t/(D/8) + 32, columns 8 (t % (D/8)).
// bf16 chunks go straight from HBM into LDS while the previous chunk's
// products run (below); fp32 chunks are loaded into registers just before
// staging (two sets of fp32 tiles do not fit in LDS at d = 128).
template <typename IN>
constexpr bool kDma = sizeof(IN) == 2;

template <int D, typename IN>
struct Chunk4 {
  typename In8<IN>::raw q[2], k[2], v[2], y[2];
  f32x2 rs[2];  // per-token (1 / D_i, h_i) of the two rows (dk/dv pass)
};

template <int D, typename IN, bool RS>
__device__ __forceinline__ void load_chunk4(Chunk4<D, IN>& ck, const BwdArgs& a, long long row0, int valid) {
  constexpr int RL = D / 8;
  const int t = threadIdx.x;
  const unsigned bytes = (unsigned)(valid * D * (int)sizeof(IN));
  const long long off = row0 * D;
  const auto Rq = make_rsrc(static_cast<const IN*>(a.q) + off, bytes);
  const auto Rk = make_rsrc(static_cast<const IN*>(a.k) + off, bytes);
  const auto Rv = make_rsrc(static_cast<const IN*>(a.v) + off, bytes);
  const auto Ry = make_rsrc(static_cast<const IN*>(a.dy) + off, bytes);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = t / RL + 32 * i;
    const int o = (row * D + 8 * (t % RL)) * (int)sizeof(IN);
    ck.q[i] = In8<IN>::bload(Rq, o);
    ck.k[i] = In8<IN>::bload(Rk, o);
    ck.v[i] = In8<IN>::bload(Rv, o);
    ck.y[i] = In8<IN>::bload(Ry, o);
    if constexpr (RS) {
      ck.rs[i] = row < valid ? *reinterpret_cast<const f32x2*>(a.rowstats + 2 * (row0 + row)) : f32x2{0.f, 0.f};
    }
  }
}

// A bf16 tile of a 64-token chunk loaded straight into LDS, no registers
// involved: 4*D threads = D/16 waves, two 1 KB blocks of the swizzled tile
// per wave. The hardware puts lane l's 16 bytes of block b at LDS bytes
// 1024 b + 16 l, so that lane fetches the 16-byte unit of the global row that
// the swizzle maps to that place. Rows past the descriptor's range (the end
// of the sequence) arrive as zeros.
template <int D>
__device__ __forceinline__ int dma_off(int i) {
  return (2 * (threadIdx.x >> 6) + i) * 1024 + 16 * (threadIdx.x & 63);
}
//
// The transfer is written as inline assembly: the compiler cannot tell which
// LDS bytes a transfer writes, and for the builtin form it waits for every
// outstanding transfer before the next LDS read, which would serialize the
// load of chunk m+1 with the products of chunk m. Here the kernels order the
// transfers themselves: a full vector-memory wait and a barrier before any
// wave reads the set they filled.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds_wave_base, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)lds_wave_base));
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
template <int D>
__device__ __forceinline__ void dma_tile(uint8_t* tile, __amdgpu_buffer_rsrc_t r) {
  constexpr int RB = 2 * D;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int o = dma_off<D>(i);
    const int row = o / RB;
    const int u = ((o % RB) >> 4) ^ swz<RB>(row);
    dma16(r, tile + (o & ~1023), row * RB + 16 * u);
  }
}

// elementwise phi (rows at or past `valid`: 0 when MASK) on 8 bf16 values in place
template <int FM, bool MASK>
__device__ __forceinline__ u32x4 phi_bf16x8(u32x4 r, bool live, float sc = 1.f) {
  float x[8];
  In8<__bf16>::to_f32(r, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (!MASK || live) ? bphi<FM>(x[e]) * sc : 0.f;
  return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

// phi of 8 bf16 values as hi + lo bf16 (rows at or past `valid`: 0)
template <int FM>
__device__ __forceinline__ void phi_bf16x8_hilo(u32x4 r, bool live, u32x4& hi, u32x4& lo, float sc = 1.f) {
  float x[8];
  In8<__bf16>::to_f32(r, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = live ? bphi<FM>(x[e]) * sc : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    lo[i] = pack_bf16x2(x[2 * i] - __uint_as_float(hi[i] << 16), x[2 * i + 1] - __uint_as_float(hi[i] & 0xffff0000u));
  }
}

// Decay (per-head gamma): gamma^n as exp2(n log2 gamma).
struct Decay {
  float lg = 0.f;
  __device__ __forceinline__ float pw(float n) const { return __builtin_amdgcn_exp2f(lg * n); }
};
template <bool DECAY>
__device__ __forceinline__ Decay decay_of(const BwdArgs& a, int bh) {
  Decay d;
  if constexpr (DECAY) d.lg = decay_log2(a.gamma[bh % a.H], a.status_flag);
  return d;
}

// ---------------------------------------------------------------------------
// dq pass. grid = (BH, P), block = 4*D threads: wave (ib, w) handles query
// rows [32 ib, 32 ib + 32) of the chunk and features [32 w, 32 w + 32). Each
// wave keeps S^T (rows = value dims, columns = its features) and z over its
// features in fp32 accumulators; the two waves of one feature block hold
// the same state.
// Precision: d phi(q_i) = sum_j phi(k_j) (v_j - y_i).g_i is a small
// difference of large sums when phi(k) varies little over the keys (q, k of
// small norm: phi(k) = 1 + a small part), and one bf16 rounding of phi(k)
// loses a large share of that small part. With bf16 operands phi(K) enters
// the S and z updates and the in-chunk product as hi + lo tiles, and S the
// product with dY as hi + lo fragments.
// Decay (DECAY): rows r of the chunk stage phi(q) gamma^(r-32) and phi(k)
// gamma^(32-r) (the scores then carry gamma^(r_i-r_j)); the carried terms
// (S dy and z) enter scaled by gamma^33 (so that row i gets gamma^(r_i+1)),
// the result of row i is scaled by gamma^(r_i-32), and the state moves on as
// gamma^31 (gamma^33 S + Kh^T V) = gamma^64 S + sum_j gamma^(63-r_j) phi(k_j) v_j^T.
// ---------------------------------------------------------------------------
template <int D, typename OP, typename IN, int FM, bool DECAY>
__global__ __launch_bounds__(D * 4) void bwd_dq_kernel(BwdArgs a) {
  using Frag = typename Ops<OP>::frag;
  constexpr int NW = D / 32;
  constexpr int RB = D * Ops<OP>::kBytes;
  constexpr int TB = 64 * RB;
  constexpr int RL = D / 8;
  constexpr bool DMA = kDma<IN>;
  // one set of tiles phi(Q), phi(K), V, dY per chunk; with DMA two sets, the
  // next chunk landing in one while the other is multiplied, and the low
  // part of phi(K)
  constexpr bool HILO = sizeof(OP) == 2;
  static_assert(!HILO || DMA, "bf16 operands take the transfer path, which also writes the low part of phi(K)");
  __shared__ __attribute__((aligned(16))) uint8_t smem[(DMA ? 2 : 1) * 4 * TB + (HILO ? TB : 0)];
  __shared__ float red[2][NW][32][2];  // per row block and feature block: (phi(q).z, phi(q).(S dy)) partials

  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int n = max(0, min(c0 + a.chunks_per_seg, a.nchunks) - c0);
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, h = l >> 5, li = l & 31;
  const int ib = wave / NW, w = wave % NW;
  const long long base = (long long)bh * a.N;
  IN* dq = static_cast<IN*>(a.dq);
  const Decay dc = decay_of<DECAY>(a, bh);

  const float* Sp;
  const float* zp;
  if (a.init_from_ws) {
    Sp = a.ws_fwd + ((long long)bh * a.fwd_slots + seg * a.seg_stride) * a.state_elems;
    zp = Sp + D * D;
  } else {
    Sp = a.S_in ? a.S_in + (long long)bh * D * D : nullptr;
    zp = a.z_in ? a.z_in + (long long)bh * D : nullptr;
  }
  f32x16 ST[NW], Z;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
    for (int eb = 0; eb < NW; ++eb) ST[eb][r] = Sp ? Sp[(long long)(32 * w + li) * D + 32 * eb + rr] : 0.f;
    Z[r] = zp ? zp[32 * w + rr] : 0.f;
  }
  Frag ones;
  {
    float o[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    ones = frag8<OP>(o);
  }

  auto issue = [&](int m) {  // DMA of chunk c0 + m into set m & 1
    const int c = c0 + m;
    const unsigned bytes = (unsigned)(min(64, a.N - 64 * c) * D * 2);
    const long long off = (base + 64LL * c) * D;
    uint8_t* t0 = smem + (m & 1) * 4 * TB;
    dma_tile<D>(t0, make_rsrc(static_cast<const IN*>(a.q) + off, bytes));
    dma_tile<D>(t0 + TB, make_rsrc(static_cast<const IN*>(a.k) + off, bytes));
    dma_tile<D>(t0 + 2 * TB, make_rsrc(static_cast<const IN*>(a.v) + off, bytes));
    dma_tile<D>(t0 + 3 * TB, make_rsrc(static_cast<const IN*>(a.dy) + off, bytes));
  };
  if constexpr (DMA) {
    if (n > 0) issue(0);
  }
  for (int m = 0; m < n; ++m) {
    const int c = c0 + m;
    const int valid = min(64, a.N - 64 * c);
    uint8_t* sQ = smem + (DMA ? (m & 1) : 0) * 4 * TB;
    uint8_t* sK = sQ + TB;
    uint8_t* sV = sQ + 2 * TB;
    uint8_t* sY = sQ + 3 * TB;
    uint8_t* sKl = smem + (DMA ? 2 : 1) * 4 * TB;  // low part of phi(K) (HILO)
    if constexpr (DMA) {
      // chunk m has landed (every wave's transfers, then the barrier); phi in place
      wait_vmem_all();
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int o = dma_off<D>(i);
        const int row = o / RB;
        const bool live = row < valid;
        u32x4* pq = reinterpret_cast<u32x4*>(sQ + o);
        u32x4* pk = reinterpret_cast<u32x4*>(sK + o);
        *pq = phi_bf16x8<FM, false>(*pq, live, DECAY ? dc.pw(row - 32) : 1.f);
        u32x4 khi, klo;
        phi_bf16x8_hilo<FM>(*pk, live, khi, klo, DECAY ? dc.pw(32 - row) : 1.f);
        *pk = khi;
        *reinterpret_cast<u32x4*>(sKl + o) = klo;
      }
      __syncthreads();
      if (m + 1 < n) issue(m + 1);
    } else {
      Chunk4<D, IN> ck;
      load_chunk4<D, IN, false>(ck, a, base + 64LL * c, valid);
      // stage phi(Q), phi(K) (rows past the end: 0), V, dY
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = t / RL + 32 * i, col = 8 * (t % RL);
        float x[8];
        In8<IN>::to_f32(ck.q[i], x);
        const float sq = DECAY ? dc.pw(row - 32) : 1.f, sk = DECAY ? dc.pw(32 - row) : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bphi<FM>(x[e]) * sq;
        Ops<OP>::template store8<RB>(sQ, row, col, x);
        In8<IN>::to_f32(ck.k[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = row < valid ? bphi<FM>(x[e]) * sk : 0.f;
        Ops<OP>::template store8<RB>(sK, row, col, x);
        put_raw<IN, OP, RB>(sV, row, col, ck.v[i]);
        put_raw<IN, OP, RB>(sY, row, col, ck.y[i]);
      }
      __syncthreads();
    }

    // scores A[j][i] = phi(k_j).phi(q_i) and value products P[j][i] = v_j.dy_i
    // for the wave's query rows i: the diagonal key block (d) and, for the
    // second row block, the first key block (o)
    // (each score tile is reduced into the row sums as soon as it is formed)
    f32x16 Pd = {}, Po = {};
    float den = 0.f, dyn = 0.f;
    {
      f32x16 Ad = {};
#pragma unroll 4
      for (int kb = 0; kb < D / 16; ++kb) {
        Ops<OP>::mma(Ad, Ops<OP>::template load_rows<RB>(sK, 32 * ib, 16 * kb),
                     Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 16 * kb));
        Ops<OP>::mma(Pd, Ops<OP>::template load_rows<RB>(sV, 32 * ib, 16 * kb),
                     Ops<OP>::template load_rows<RB>(sY, 32 * ib, 16 * kb));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool keep = 8 * (r >> 2) + 4 * h + (r & 3) <= li;
        const float x = keep ? Ad[r] : 0.f;
        den += x;
        dyn += x * Pd[r];
      }
    }
    if (ib) {
      f32x16 Ao = {};
#pragma unroll 4
      for (int kb = 0; kb < D / 16; ++kb) {
        Ops<OP>::mma(Ao, Ops<OP>::template load_rows<RB>(sK, 0, 16 * kb),
                     Ops<OP>::template load_rows<RB>(sQ, 32 * ib, 16 * kb));
        Ops<OP>::mma(Po, Ops<OP>::template load_rows<RB>(sV, 0, 16 * kb),
                     Ops<OP>::template load_rows<RB>(sY, 32 * ib, 16 * kb));
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        den += Ao[r];
        dyn += Ao[r] * Po[r];
      }
    }
    // T[f][i] = sum_e S[f][e] dy_i[e] over the wave's features. With bf16
    // operands S enters as hi + lo: T / D_i and h_i z cancel down to
    // sum_j phi(k_j) (v_j - y_i).g_i, which is much smaller than either term
    // when phi(k) varies little over the keys, and a single bf16 rounding of
    // S would be magnified by that ratio.
    f32x16 T = {};
#pragma unroll
    for (int eb = 0; eb < NW; ++eb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag yf = Ops<OP>::template load_rows<RB>(sY, 32 * ib, 32 * eb + 16 * kk);
        if constexpr (sizeof(OP) == 2) {
          bf16x8 hi, lo;
          frag_hilo(ST[eb], kk, hi, lo);
          Ops<OP>::mma(T, hi, yf);
          Ops<OP>::mma(T, lo, yf);
        } else {
          Ops<OP>::mma(T, Ops<OP>::from_acc(ST[eb], kk), yf);
        }
      }
    const float g33 = DECAY ? dc.pw(33) : 1.f;
    if constexpr (DECAY) T *= g33;
    // in-chunk parts (keys j <= i) of den_i and dy_i.num_i: both lane halves
    den += xor32(den);
    dyn += xor32(dyn);
    // carried parts over the wave's features: phi(q_i).z and phi(q_i).T_i
    const int irow = 32 * ib + li;
    float fq[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) lds_read4<OP, RB>(sQ, irow, 32 * w + 8 * g + 4 * h, &fq[4 * g]);
    float pden = 0.f, pdyn = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pden += fq[r] * Z[r];
      pdyn += fq[r] * T[r];
    }
    if constexpr (DECAY) pden *= g33;
    pden += xor32(pden);
    pdyn += xor32(pdyn);
    if (h == 0) {
      red[ib][w][li][0] = pden;
      red[ib][w][li][1] = pdyn;
    }
    __syncthreads();
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      den += red[ib][ww][li][0];
      dyn += red[ib][ww][li][1];
    }
    float inv = 1.f, hh = 0.f;
    if (a.normalize) {
      const float Dn = fmaxf(den, kEps);
      inv = 1.f / Dn;
      hh = den >= kEps ? -dyn * inv * inv : 0.f;
    }
    // B[j][i] = g_i.v_j + h_i (keys j <= i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool keep = 8 * (r >> 2) + 4 * h + (r & 3) <= li;
      Pd[r] = keep ? Pd[r] * inv + hh : 0.f;
      Po[r] = Po[r] * inv + hh;
    }
    // d phi(q_i)[f] = T[f][i] / D_i + h_i z_f + sum_j phi(k_j)[f] B[j][i]
#pragma unroll
    for (int r = 0; r < 16; ++r) T[r] = T[r] * inv + (DECAY ? hh * g33 : hh) * Z[r];
    // (bf16: phi(K) and B both as hi + lo; the lo x lo term is below 2^-16)
    auto intra = [&](const f32x16& Bt, int j0) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag kf = Ops<OP>::template load_cols<RB>(sK, j0 + 16 * kk, 32 * w);
        if constexpr (HILO) {
          bf16x8 bh, bl;
          frag_hilo(Bt, kk, bh, bl);
          Ops<OP>::mma(T, kf, bh);
          Ops<OP>::mma(T, kf, bl);
          Ops<OP>::mma(T, Ops<OP>::template load_cols<RB>(sKl, j0 + 16 * kk, 32 * w), bh);
        } else {
          Ops<OP>::mma(T, kf, Ops<OP>::from_acc(Bt, kk));
        }
      }
    };
    intra(Pd, 32 * ib);
    if (ib) intra(Po, 0);
    {
      // decay: the row's factor gamma^(r-32), and phi(q) back from the staged row
      const float fr = DECAY ? dc.pw(irow - 32) : 1.f, fb = DECAY ? dc.pw(32 - irow) : 1.f;
      float y[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) y[r] = fr * T[r] * bdphi<FM>(fb * fq[r]);
      store_block_rows<IN, D>(dq + (base + 64LL * c) * D, valid, irow, 32 * w, y);
      if (irow < valid && w == 0 && h == 0)
        *reinterpret_cast<f32x2*>(a.rowstats + 2 * (base + 64LL * c + irow)) = f32x2{inv, hh};
    }
    if constexpr (DECAY) {
#pragma unroll
      for (int eb = 0; eb < NW; ++eb) ST[eb] *= g33;
      Z *= g33;
    }
    // S^T += V^T phi(K), z += column sums of phi(K)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const Frag kf = Ops<OP>::template load_cols<RB>(sK, 16 * kb, 32 * w);
      const Frag kl = HILO ? Ops<OP>::template load_cols<RB>(sKl, 16 * kb, 32 * w) : kf;
#pragma unroll
      for (int eb = 0; eb < NW; ++eb) {
        const Frag vf = Ops<OP>::template load_cols<RB>(sV, 16 * kb, 32 * eb);
        Ops<OP>::mma(ST[eb], vf, kf);
        if constexpr (HILO) Ops<OP>::mma(ST[eb], vf, kl);
      }
      Ops<OP>::mma(Z, kf, ones);
      if constexpr (HILO) Ops<OP>::mma(Z, kl, ones);
    }
    if constexpr (DECAY) {  // gamma^31 (gamma^33 S + Kh^T V): the state after the chunk
      const float g31 = dc.pw(31);
#pragma unroll
      for (int eb = 0; eb < NW; ++eb) ST[eb] *= g31;
      Z *= g31;
    }
    // the single set is restaged next; with two sets the next chunk's
    // barriers already order these reads before that set is refilled
    if constexpr (!DMA) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// r-state pass: per segment R_loc = sum_i phi(q_i) g_i^T, r_loc = sum_i
// phi(q_i) h_i into ws_rev slot P-1-seg (decay: weighted gamma^(i - s0 + 1),
// relative to the row before the segment, s0 its first token). grid = (BH, P), block = 2*D
// threads; wave w keeps R[:, 32w:32w+32] (rows = features). Staging threads
// hold pieces at rows t/(D/8) + 16 i, i = 0..3.
// ---------------------------------------------------------------------------
template <int D, typename OP, typename IN, int FM, bool DECAY>
__global__ __launch_bounds__(D * 2) void bwd_rstate_kernel(BwdArgs a) {
  constexpr int NW = D / 32;
  constexpr int RB = D * Ops<OP>::kBytes;
  constexpr int TB = 64 * RB;
  constexpr int RL = D / 8;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TB];
  __shared__ float rsum[NW][D];
  uint8_t* sQ = smem;
  uint8_t* sG = smem + TB;

  const int bh = blockIdx.x, seg = blockIdx.y;  // a state-pass segment
  const int c0 = seg * a.chunks_per_seg_state;
  const int n = max(0, min(c0 + a.chunks_per_seg_state, a.nchunks) - c0);
  const int t = threadIdx.x, w = t >> 6, l = t & 63, h = l >> 5, li = l & 31;
  const long long base = (long long)bh * a.N;
  const IN* q = static_cast<const IN*>(a.q);
  const IN* dy = static_cast<const IN*>(a.dy);
  const Decay dc = decay_of<DECAY>(a, bh);

  f32x16 R[NW];
#pragma unroll
  for (int fb = 0; fb < NW; ++fb) R[fb] = f32x16{};
  float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int col = 8 * (t % RL);
  for (int mm = 0; mm < n; ++mm) {
    const int m = DECAY ? n - 1 - mm : mm;  // decay: chunks from the last, the sums moved on by gamma^64
    const int c = c0 + m;
    const int valid = min(64, a.N - 64 * c);
    const unsigned bytes = (unsigned)(valid * D * (int)sizeof(IN));
    const long long row0 = base + 64LL * c;
    const auto Rq = make_rsrc(q + row0 * D, bytes);
    const auto Ry = make_rsrc(dy + row0 * D, bytes);
    typename In8<IN>::raw rq[4], ry[4];
    f32x2 rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t / RL + 16 * i;
      const int o = (row * D + col) * (int)sizeof(IN);
      rq[i] = In8<IN>::bload(Rq, o);
      ry[i] = In8<IN>::bload(Ry, o);
      rs[i] = row < valid ? *reinterpret_cast<const f32x2*>(a.rowstats + 2 * (row0 + row)) : f32x2{0.f, 0.f};
    }
    if constexpr (DECAY) {
      const float g32 = dc.pw(32);
#pragma unroll
      for (int fb = 0; fb < NW; ++fb) R[fb] = (R[fb] * g32) * g32;
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] = (cs[e] * g32) * g32;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = t / RL + 16 * i;
      const float sq = DECAY ? dc.pw(row + 1) : 1.f;  // decay: relative to the row before the chunk
      float x[8];
      In8<IN>::to_f32(rq[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = row < valid ? bphi<FM>(x[e]) * sq : 0.f;
        cs[e] += x[e] * rs[i][1];
      }
      Ops<OP>::template store8<RB>(sQ, row, col, x);
      In8<IN>::to_f32(ry[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= rs[i][0];
      Ops<OP>::template store8<RB>(sG, row, col, x);
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const auto gf = Ops<OP>::template load_cols<RB>(sG, 16 * kb, 32 * w);
#pragma unroll
      for (int fb = 0; fb < NW; ++fb) Ops<OP>::mma(R[fb], Ops<OP>::template load_cols<RB>(sQ, 16 * kb, 32 * fb), gf);
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = lane_colsum<RL>(cs[e]);
  if (l < RL) {
#pragma unroll
    for (int e = 0; e < 8; ++e) rsum[w][col + e] = cs[e];
  }
  __syncthreads();
  float* st = a.ws_rev + ((long long)bh * (a.nseg_state + 1) + (a.nseg_state - 1 - seg)) * a.state_elems;
  // decay: the last segment also carries the final-state cotangents, which
  // reach the row before the segment with gamma^(N - s0)
  const bool seed = DECAY && a.dS_out && seg == a.nseg_state - 1;
  const float fs = seed ? dc.pw((float)(a.N - 64 * c0)) : 0.f;
  const float* sS = seed ? a.dS_out + (long long)bh * D * D : nullptr;
  const float* sz = seed ? a.dz_out + (long long)bh * D : nullptr;
#pragma unroll
  for (int fb = 0; fb < NW; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const long long ix = (long long)(32 * fb + 8 * (r >> 2) + 4 * h + (r & 3)) * D + 32 * w + li;
      st[ix] = R[fb][r] + (seed ? fs * sS[ix] : 0.f);
    }
  for (int f = t; f < D; f += 2 * D) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += rsum[ww][f];
    st[D * D + f] = s + (seed ? fs * sz[f] : 0.f);
  }
}

// ---------------------------------------------------------------------------
// dk/dv pass. grid = (BH, P), block = 4*D threads, chunks of the segment in
// reverse order, starting from the cotangent of the state leaving the
// segment (ws_rev slot P-1-seg).
//   waves 0..NW-1 (value block w): R[:, 32w:32w+32] (rows = features), the
//     scores A[i][j] = phi(q_i).phi(k_j) of the chunk, dv for value dims
//     [32w, 32w+32);
//   waves NW..2NW-1 (feature block w): R^T[:, 32w:32w+32] (rows = value
//     dims), r over the block's features, B[i][j] = g_i.v_j + h_i, dk for
//     features [32w, 32w+32).
// Tiles: phi(Q), phi(K), V, a "Y" tile and a "Qs" tile, with a per-row
// scale sI: bf16 keeps Y = raw dY, Qs = phi(Q) / D_i and sI = 1 / D_i, so
// the 1/D_i scaling happens in fp32 (B = (dy_i.v_j) sI_i + h_i, and the
// scores times sI_i for dv): g_i.v_j and -h_i cancel where v_j is close to
// the output y_i, and a product with g rounded to bf16 would leave that
// rounding in dk. fp32 keeps Y = G = dY / D_i, Qs = phi(Q) and sI = 1.
// Decay (DECAY): rows stage phi(q) gamma^(r-32) and phi(k) gamma^(32-r);
// the suffix state of a chunk of v valid rows is kept relative to its last
// valid row, enters as gamma^(v-33) R (row j then gets gamma^(v-1-r_j) R
// through the staged keys), the dk of row j is scaled by gamma^(32-r_j), and
// the state moves to the previous chunk as gamma^33 (gamma^(v-33) R + Qs^T Y).
// ---------------------------------------------------------------------------
template <int D, typename OP, typename IN, int FM, bool DECAY>
__global__ __launch_bounds__(D * 4) void bwd_dkv_kernel(BwdArgs a) {
  using Frag = typename Ops<OP>::frag;
  constexpr int NW = D / 32;
  constexpr int RB = D * Ops<OP>::kBytes;
  constexpr int TB = 64 * RB;
  constexpr int RL = D / 8;
  constexpr bool DMA = kDma<IN>;
  // DMA: two sets of q, k, v, dY tiles (the next chunk lands in one while the
  // other is multiplied) and the Qs tile; otherwise one set (Y = G, Qs = phi(Q))
  __shared__ __attribute__((aligned(16))) uint8_t smem[(DMA ? 9 : 4) * TB];
  __shared__ __attribute__((aligned(16))) float sH[64];
  __shared__ __attribute__((aligned(16))) float sI[64];

  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int n = max(0, min(c0 + a.chunks_per_seg, a.nchunks) - c0);
  const int t = threadIdx.x, wave = t >> 6, l = t & 63, h = l >> 5, li = l & 31;
  const bool vgroup = wave < NW;
  const int w = vgroup ? wave : wave - NW;
  const long long base = (long long)bh * a.N;
  IN* dk = static_cast<IN*>(a.dk);
  IN* dv = static_cast<IN*>(a.dv);
  const Decay dc = decay_of<DECAY>(a, bh);
  // decay: the last segment starts from the final-state cotangents (the
  // reverse scan carries no seed then)
  const bool seed = DECAY && a.dS_out && seg == a.nseg - 1;
  const float* sS = seed ? a.dS_out + (long long)bh * D * D : nullptr;
  const float* sz = seed ? a.dz_out + (long long)bh * D : nullptr;

  const int last = min(seg * a.seg_stride + a.seg_stride - 1, a.nseg_state - 1);  // its last state-pass segment
  const float* Rp = a.ws_rev + ((long long)bh * (a.nseg_state + 1) + (a.nseg_state - 1 - last)) * a.state_elems;
  f32x16 RS[NW], rK;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
    for (int b = 0; b < NW; ++b) {
      const long long ix = vgroup ? (long long)(32 * b + rr) * D + 32 * w + li : (long long)(32 * w + li) * D + 32 * b + rr;
      RS[b][r] = Rp[ix] + (seed ? sS[ix] : 0.f);
    }
    rK[r] = vgroup ? 0.f : Rp[D * D + 32 * w + rr] + (seed ? sz[32 * w + rr] : 0.f);
  }

  uint8_t* sQs = smem + 8 * TB;  // DMA only
  f32x2 rs[2];                    // DMA: (1 / D_i, h_i) of the rows of the thread's two units
  auto issue = [&](int m) {       // DMA of chunk c0 + m into set m & 1, and its row statistics
    const int c = c0 + m;
    const int valid = min(64, a.N - 64 * c);
    const unsigned bytes = (unsigned)(valid * D * 2);
    const long long row0 = base + 64LL * c;
    const long long off = row0 * D;
    uint8_t* t0 = smem + (m & 1) * 4 * TB;
    dma_tile<D>(t0, make_rsrc(static_cast<const IN*>(a.q) + off, bytes));
    dma_tile<D>(t0 + TB, make_rsrc(static_cast<const IN*>(a.k) + off, bytes));
    dma_tile<D>(t0 + 2 * TB, make_rsrc(static_cast<const IN*>(a.v) + off, bytes));
    dma_tile<D>(t0 + 3 * TB, make_rsrc(static_cast<const IN*>(a.dy) + off, bytes));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = dma_off<D>(i) / RB;
      rs[i] = row < valid ? *reinterpret_cast<const f32x2*>(a.rowstats + 2 * (row0 + row)) : f32x2{0.f, 0.f};
    }
  };
  if constexpr (DMA) {
    if (n > 0) issue(n - 1);
  }
  for (int m = n - 1; m >= 0; --m) {
    const int c = c0 + m;
    const int valid = min(64, a.N - 64 * c);
    uint8_t* sQ = smem + (DMA ? (m & 1) : 0) * 4 * TB;
    uint8_t* sK = sQ + TB;
    uint8_t* sV = sQ + 2 * TB;
    uint8_t* sY = sQ + 3 * TB;
    uint8_t* sQq = DMA ? sQs : sQ;
    if constexpr (DMA) {
      // chunk m has landed: phi in place (rows past the end: 0), Qs = phi(Q) / D_i
      wait_vmem_all();
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int o = dma_off<D>(i);
        const int row = o / RB;
        const bool live = row < valid;
        u32x4* pq = reinterpret_cast<u32x4*>(sQ + o);
        u32x4* pk = reinterpret_cast<u32x4*>(sK + o);
        // phi(q) in fp32 once: the tile gets it rounded to bf16, Qs = phi(q) / D_i
        // is rounded once from the fp32 value (not from the rounded phi)
        float x[8];
        In8<__bf16>::to_f32(*pq, x);
        const float sq = DECAY ? dc.pw(row - 32) : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = live ? bphi<FM>(x[e]) * sq : 0.f;
        *pq = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7])};
        *pk = phi_bf16x8<FM, true>(*pk, live, DECAY ? dc.pw(32 - row) : 1.f);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= rs[i][0];
        *reinterpret_cast<u32x4*>(sQs + o) = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                   pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        if ((o % RB) == 0) {
          sH[row] = rs[i][1];
          sI[row] = rs[i][0];
        }
      }
      __syncthreads();
      if (m > 0) issue(m - 1);
    } else {
      Chunk4<D, IN> ck;
      load_chunk4<D, IN, true>(ck, a, base + 64LL * c, valid);
      // stage phi(Q), phi(K) (rows past the end: 0), V, G = dY / D_i, h
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = t / RL + 32 * i, col = 8 * (t % RL);
        const bool live = row < valid;
        float x[8];
        const float sq = DECAY ? dc.pw(row - 32) : 1.f, sk = DECAY ? dc.pw(32 - row) : 1.f;
        In8<IN>::to_f32(ck.q[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = live ? bphi<FM>(x[e]) * sq : 0.f;
        Ops<OP>::template store8<RB>(sQ, row, col, x);
        In8<IN>::to_f32(ck.k[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = live ? bphi<FM>(x[e]) * sk : 0.f;
        Ops<OP>::template store8<RB>(sK, row, col, x);
        put_raw<IN, OP, RB>(sV, row, col, ck.v[i]);
        In8<IN>::to_f32(ck.y[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= ck.rs[i][0];
        Ops<OP>::template store8<RB>(sY, row, col, x);
        if (col == 0) {
          sH[row] = ck.rs[i][1];
          sI[row] = 1.f;
        }
      }
      __syncthreads();
    }

    if constexpr (DECAY) {  // the suffix state as this chunk's rows see it: gamma^(v-33) R
      const float fa = dc.pw(valid - 33);
#pragma unroll
      for (int b = 0; b < NW; ++b) RS[b] *= fa;
      rK *= fa;
    }
    if (vgroup) {
      // dv_j[e] = sum_{i>=j} G[i][e] A[i][j] + sum_f R[f][e] phi(k_j)[f], with the
      // scores A[i][j] of (query block, key block) (0,0), (1,0), (1,1), j <= i,
      // formed one tile at a time
      f32x16 V0 = {}, V1 = {};
#pragma unroll
      for (int tI = 0; tI < 3; ++tI) {
        const int qb = tI == 0 ? 0 : 1, kbk = tI == 2 ? 1 : 0;
        f32x16 A = {};
// partial unroll: full unrolling hoists every fragment load and spills
#pragma unroll 2
        for (int kb = 0; kb < D / 16; ++kb)
          Ops<OP>::mma(A, Ops<OP>::template load_rows<RB>(sQ, 32 * qb, 16 * kb),
                       Ops<OP>::template load_rows<RB>(sK, 32 * kbk, 16 * kb));
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 iq = *reinterpret_cast<const f32x4*>(sI + 32 * qb + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool keep = qb != kbk || li <= 8 * g + 4 * h + e;
            A[4 * g + e] = keep ? A[4 * g + e] * iq[e] : 0.f;
          }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          Ops<OP>::mma(kbk ? V1 : V0, Ops<OP>::template load_cols<RB>(sY, 32 * qb + 16 * kk, 32 * w),
                       Ops<OP>::from_acc(A, kk));
      }
#pragma unroll
      for (int fb = 0; fb < NW; ++fb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const Frag rf = Ops<OP>::from_acc(RS[fb], kk);
          Ops<OP>::mma(V0, rf, Ops<OP>::template load_rows<RB>(sK, 0, 32 * fb + 16 * kk));
          Ops<OP>::mma(V1, rf, Ops<OP>::template load_rows<RB>(sK, 32, 32 * fb + 16 * kk));
        }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const f32x16& Vt = jb ? V1 : V0;
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) y[r] = Vt[r];
        store_block_rows<IN, D>(dv + (base + 64LL * c) * D, valid, 32 * jb + li, 32 * w, y);
      }
      // R += phi(Q)^T G = Qs^T Y over the chunk
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const Frag gf = Ops<OP>::template load_cols<RB>(sY, 16 * kb, 32 * w);
#pragma unroll
        for (int fb = 0; fb < NW; ++fb) Ops<OP>::mma(RS[fb], Ops<OP>::template load_cols<RB>(sQq, 16 * kb, 32 * fb), gf);
      }
    } else {
      // d phi(k_j)[f] = sum_{i>=j} phi(q_i)[f] B[i][j] + sum_e R[f][e] v_j[e] + r_f,
      // with B[i][j] = g_i.v_j + h_i of (query block, key block) (0,0), (1,0),
      // (1,1), j <= i, formed one tile at a time
      f32x16 K0 = rK, K1 = rK;
#pragma unroll
      for (int tI = 0; tI < 3; ++tI) {
        const int qb = tI == 0 ? 0 : 1, kbk = tI == 2 ? 1 : 0;
        f32x16 Bt = {};
// partial unroll: full unrolling hoists every fragment load and spills
#pragma unroll 2
        for (int kb = 0; kb < D / 16; ++kb)
          Ops<OP>::mma(Bt, Ops<OP>::template load_rows<RB>(sY, 32 * qb, 16 * kb),
                       Ops<OP>::template load_rows<RB>(sV, 32 * kbk, 16 * kb));
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 hq = *reinterpret_cast<const f32x4*>(sH + 32 * qb + 8 * g + 4 * h);
          const f32x4 iq = *reinterpret_cast<const f32x4*>(sI + 32 * qb + 8 * g + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool keep = qb != kbk || li <= 8 * g + 4 * h + e;
            Bt[4 * g + e] = keep ? Bt[4 * g + e] * iq[e] + hq[e] : 0.f;
          }
        }
        // B enters as hi + lo fragments with bf16 operands: sum_i phi(q_i) B[i][j]
        // is a sum of terms of both signs that can cancel far below its terms
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const Frag qf = Ops<OP>::template load_cols<RB>(sQ, 32 * qb + 16 * kk, 32 * w);
          if constexpr (sizeof(OP) == 2) {
            bf16x8 bh, bl;
            frag_hilo(Bt, kk, bh, bl);
            Ops<OP>::mma(kbk ? K1 : K0, qf, bh);
            Ops<OP>::mma(kbk ? K1 : K0, qf, bl);
          } else {
            Ops<OP>::mma(kbk ? K1 : K0, qf, Ops<OP>::from_acc(Bt, kk));
          }
        }
      }
      // R^T v_j: with bf16 operands R enters as hi + lo fragments. The
      // product is a dot product over value dims of both signs and can be far
      // smaller than its terms. With R and B rounded to bf16, rows of dk on the
      // long-context workload were off by up to ~3%; a CPU emulation of the
      // pass's rounding puts the worst row at ~0.8% of its 64-token block's
      // RMS row norm with both as hi + lo (Qs stays bf16: no room in LDS for
      // a lo tile at d = 128).
#pragma unroll
      for (int eb = 0; eb < NW; ++eb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const Frag v0 = Ops<OP>::template load_rows<RB>(sV, 0, 32 * eb + 16 * kk);
          const Frag v1 = Ops<OP>::template load_rows<RB>(sV, 32, 32 * eb + 16 * kk);
          if constexpr (sizeof(OP) == 2) {
            bf16x8 rh, rl;
            frag_hilo(RS[eb], kk, rh, rl);
            Ops<OP>::mma(K0, rh, v0);
            Ops<OP>::mma(K0, rl, v0);
            Ops<OP>::mma(K1, rh, v1);
            Ops<OP>::mma(K1, rl, v1);
          } else {
            const Frag rf = Ops<OP>::from_acc(RS[eb], kk);
            Ops<OP>::mma(K0, rf, v0);
            Ops<OP>::mma(K1, rf, v1);
          }
        }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const f32x16& Kt = jb ? K1 : K0;
        const int j = 32 * jb + li;
        // decay: the row's factor gamma^(32-r), and phi(k) back from the staged row
        const float fr = DECAY ? dc.pw(32 - j) : 1.f, fb = DECAY ? dc.pw(j - 32) : 1.f;
        float y[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float fk[4];
          lds_read4<OP, RB>(sK, j, 32 * w + 8 * g + 4 * h, fk);
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) y[4 * g + cc] = fr * Kt[4 * g + cc] * bdphi<FM>(fb * fk[cc]);
        }
        store_block_rows<IN, D>(dk + (base + 64LL * c) * D, valid, j, 32 * w, y);
      }
      // R^T += G^T phi(Q), r += phi(Q)^T h over the chunk
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const Frag qf = Ops<OP>::template load_cols<RB>(sQ, 16 * kb, 32 * w);
        const Frag qsf = DMA ? Ops<OP>::template load_cols<RB>(sQq, 16 * kb, 32 * w) : qf;
#pragma unroll
        for (int eb = 0; eb < NW; ++eb) Ops<OP>::mma(RS[eb], Ops<OP>::template load_cols<RB>(sY, 16 * kb, 32 * eb), qsf);
        const f32x4 ha = *reinterpret_cast<const f32x4*>(sH + 16 * kb + 8 * h);
        const f32x4 hb = *reinterpret_cast<const f32x4*>(sH + 16 * kb + 8 * h + 4);
        const float hv[8] = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
        Ops<OP>::mma(rK, qf, frag8<OP>(hv));
      }
    }
    if constexpr (DECAY) {  // on to the previous chunk: gamma^33 (gamma^(v-33) R + Qs^T Y)
      const float g33 = dc.pw(33);
#pragma unroll
      for (int b = 0; b < NW; ++b) RS[b] *= g33;
      rK *= g33;
    }
    // the single set is restaged next; with two sets the next chunk's
    // barriers already order these reads before that set is refilled
    if constexpr (!DMA) __syncthreads();
  }
}

template <int D, typename T, int FM, bool DECAY>
hipError_t launch_backward(const FwdArgs& fa, const ScanArgs& fs, const BwdArgs& b, const ScanArgs& rs, int dtype,
                           hipStream_t st) {
  if (fa.run_state_pass || fa.run_scan) {
    FwdArgs f = fa;
    f.skip_output = 1;
    f.hilo_keys = 1;  // S carries phi(k) to ~2^-16 (the dq pass needs it; see there)
    const hipError_t e = prefill_dispatch(f, fs, D, D, FM, dtype, true, DECAY, st, nullptr);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, T, T, FM, DECAY>), dim3(b.BH, b.nseg), dim3(4 * D), 0, st, b);
  hipLaunchKernelGGL((bwd_rstate_kernel<D, T, T, FM, DECAY>), dim3(b.BH, b.nseg_state), dim3(2 * D), 0, st, b);
  const hipError_t e = scan_dispatch(rs, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkv_kernel<D, T, T, FM, DECAY>), dim3(b.BH, b.nseg), dim3(4 * D), 0, st, b);
  return hipGetLastError();
}

template <typename T, int FM, bool DECAY>
hipError_t backward_d(const FwdArgs& fa, const ScanArgs& fs, const BwdArgs& b, const ScanArgs& rs, int D, int dtype,
                      hipStream_t st) {
  switch (D) {
    case 32: return launch_backward<32, T, FM, DECAY>(fa, fs, b, rs, dtype, st);
    case 64: return launch_backward<64, T, FM, DECAY>(fa, fs, b, rs, dtype, st);
    case 128: return launch_backward<128, T, FM, DECAY>(fa, fs, b, rs, dtype, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int FM>
hipError_t backward_dd(const FwdArgs& fa, const ScanArgs& fs, const BwdArgs& b, const ScanArgs& rs, int D, int dtype,
                       bool decay, hipStream_t st) {
  return decay ? backward_d<T, FM, true>(fa, fs, b, rs, D, dtype, st) : backward_d<T, FM, false>(fa, fs, b, rs, D, dtype, st);
}

}  // namespace

hipError_t backward_dispatch(const FwdArgs& fa, const ScanArgs& fs, const BwdArgs& b, const ScanArgs& rs, int D,
                             int fmap, int dtype, bool decay, hipStream_t st) {
  if (dtype == 1) {
    if (fmap == kElu1) return backward_dd<__bf16, kElu1>(fa, fs, b, rs, D, dtype, decay, st);
    if (fmap == kIdentity) return backward_dd<__bf16, kIdentity>(fa, fs, b, rs, D, dtype, decay, st);
  } else {
    if (fmap == kElu1) return backward_dd<float, kElu1>(fa, fs, b, rs, D, dtype, decay, st);
    if (fmap == kIdentity) return backward_dd<float, kIdentity>(fa, fs, b, rs, D, dtype, decay, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace la

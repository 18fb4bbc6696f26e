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
//   carry scan : exclusive prefix over segments (+ initial state)  -> workspace
//   output pass: every segment starts from its prefix and walks its chunks
// The non-causal form reuses the state pass, a total-sum scan and the output
// pass without the intra-chunk term.
//
// Wave w of a workgroup owns value columns [32w, 32w+32): it keeps the fp32
// state S[:, 32w:32w+32] in MFMA accumulators and produces those output
// columns. Layouts: q, k, v, out are [BH][N][D]; S is [BH][DF][D] (row c =
// feature, column e = value dim); z is [BH][DF].
#include "la_device.h"
#include "la_kernels.h"

namespace la {

// One chunk's worth of raw rows held in registers between issue and staging.
template <int D, typename IN>
struct Prefetch {
  static constexpr int kPer = 4;  // 8-element pieces per thread per tensor (64*D/8 / (64*D/32))
  typename In8<IN>::raw q[kPer], k[kPer], v[kPer];
};

template <int D, int NT>
__device__ __forceinline__ void piece_of(int p, int& row, int& col8) {
  row = p / (D / 8);
  col8 = (p % (D / 8)) * 8;
}

// Issue global loads of rows [t0, t0 + valid) of one chunk (zeros beyond).
template <int D, typename IN, bool LOADQ, bool LOADKV>
__device__ __forceinline__ void issue_loads(Prefetch<D, IN>& pf, const IN* q, const IN* k, const IN* v,
                                            long long row_base, int valid) {
  constexpr int NT = D * 2;  // threads: 64 * (D/32)
#pragma unroll
  for (int i = 0; i < Prefetch<D, IN>::kPer; ++i) {
    const int p = threadIdx.x + i * NT;
    int row, col;
    piece_of<D, NT>(p, row, col);
    if (row < valid) {
      const long long off = (row_base + row) * D + col;
      if constexpr (LOADQ) pf.q[i] = In8<IN>::load(q + off);
      if constexpr (LOADKV) {
        pf.k[i] = In8<IN>::load(k + off);
        pf.v[i] = In8<IN>::load(v + off);
      }
    } else {
      if constexpr (LOADQ) pf.q[i] = In8<IN>::zero();
      if constexpr (LOADKV) {
        pf.k[i] = In8<IN>::zero();
        pf.v[i] = In8<IN>::zero();
      }
    }
  }
}

// Apply the feature map and write one chunk into LDS (phi(Q), phi(K), V).
// Rows beyond `valid` get phi = 0 and v = 0, so they add nothing to any sum.
template <int D, typename IN, typename OP, bool LOADQ, bool LOADKV>
__device__ __forceinline__ void stage_chunk(const Prefetch<D, IN>& pf, uint8_t* sQ, uint8_t* sK,
                                            uint8_t* sV, int valid) {
  constexpr int NT = D * 2;
  constexpr int RB = D * Ops<OP>::kBytes;
#pragma unroll
  for (int i = 0; i < Prefetch<D, IN>::kPer; ++i) {
    const int p = threadIdx.x + i * NT;
    int row, col;
    piece_of<D, NT>(p, row, col);
    const bool ok = row < valid;
    float x[8];
    if constexpr (LOADQ) {
      In8<IN>::to_f32(pf.q[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ok ? phi_elu1(x[e]) : 0.f;
      Ops<OP>::template store8<RB>(sQ, row, col, x);
    }
    if constexpr (LOADKV) {
      In8<IN>::to_f32(pf.k[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ok ? phi_elu1(x[e]) : 0.f;
      Ops<OP>::template store8<RB>(sK, row, col, x);
      In8<IN>::to_f32(pf.v[i], x);
      Ops<OP>::template store8<RB>(sV, row, col, x);
    }
  }
}

// Load this wave's state tiles (accumulator layout) and its copy of z.
template <int D, int DF>
__device__ __forceinline__ void load_state(f32x16 (&S)[DF / 32], float (&zc)[DF / 32], const float* Sp,
                                           const float* zp) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6, h = l >> 5, li = l & 31;
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * cb + 8 * (r >> 2) + 4 * h + (r & 3);
      S[cb][r] = Sp ? Sp[(long long)c * D + 32 * w + li] : 0.f;
    }
    zc[cb] = zp ? zp[32 * cb + li] : 0.f;
  }
}

template <int D, int DF>
__device__ __forceinline__ void store_state(const f32x16 (&S)[DF / 32], const float (&zc)[DF / 32], float* Sp,
                                            float* zp) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6, h = l >> 5, li = l & 31;
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 32 * cb + 8 * (r >> 2) + 4 * h + (r & 3);
      Sp[(long long)c * D + 32 * w + li] = S[cb][r];
    }
    if (w == 0 && h == 0) zp[32 * cb + li] = zc[cb];
  }
}

// S[:, e-block] += phi(K)^T V over one staged chunk; zc (per lane: feature
// 32cb + lane%32, this half's tokens) += column sums of phi(K).
template <int D, int DF, typename OP>
__device__ __forceinline__ void state_update(f32x16 (&S)[DF / 32], float (&zpart)[DF / 32], const uint8_t* sK,
                                             const uint8_t* sV, const typename Ops<OP>::frag (&Vf)[4]) {
  constexpr int RBF = DF * Ops<OP>::kBytes;
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {  // 64 tokens = 4 blocks of 16
      typename Ops<OP>::frag Kt = Ops<OP>::template load_cols<RBF>(sK, 16 * kb, 32 * cb);
      Ops<OP>::mma(S[cb], Kt, Vf[kb]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) zpart[cb] += Ops<OP>::elem(Kt, jj);
    }
  }
}

// ---------------------------------------------------------------------------
// State pass: local (S, z) of every segment.
// grid = (BH, P), block = 64 * D/32 threads.
// ---------------------------------------------------------------------------
template <int D, int DF, typename OP, typename IN>
__global__ __launch_bounds__(D * 2) void state_pass_kernel(FwdArgs a) {
  constexpr int RBF = DF * Ops<OP>::kBytes;
  constexpr int RBV = D * Ops<OP>::kBytes;
  constexpr int KBYTES = 64 * RBF, VBYTES = 64 * RBV;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (KBYTES + VBYTES)];
  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg_state;
  const int c1 = min(c0 + a.chunks_per_seg_state, a.nchunks);
  const long long base = (long long)bh * a.N;
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;

  f32x16 S[DF / 32];
  float zc[DF / 32];
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb) {
    S[cb] = f32x16{};
    zc[cb] = 0.f;
  }
  Prefetch<D, IN> pf;
  if (c0 < c1) {
    issue_loads<D, IN, false, true>(pf, nullptr, k, v, base + 64LL * c0, min(64, a.N - 64 * c0));
    stage_chunk<D, IN, OP, false, true>(pf, nullptr, smem, smem + KBYTES, min(64, a.N - 64 * c0));
  }
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) & 1;
    uint8_t* sK = smem + buf * (KBYTES + VBYTES);
    uint8_t* sV = sK + KBYTES;
    const bool more = c + 1 < c1;
    const int nvalid = more ? min(64, a.N - 64 * (c + 1)) : 0;
    if (more) issue_loads<D, IN, false, true>(pf, nullptr, k, v, base + 64LL * (c + 1), nvalid);
    typename Ops<OP>::frag Vf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Vf[kb] = Ops<OP>::template load_cols<RBV>(sV, 16 * kb, 32 * w);
    state_update<D, DF, OP>(S, zc, sK, sV, Vf);
    if (more) {
      uint8_t* nK = smem + (buf ^ 1) * (KBYTES + VBYTES);
      stage_chunk<D, IN, OP, false, true>(pf, nullptr, nK, nK + KBYTES, nvalid);
    }
    __syncthreads();
  }
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb) zc[cb] += xor32(zc[cb]);
  (void)l;
  float* st = a.ws + ((long long)bh * a.ws_slots + seg) * a.state_elems;
  store_state<D, DF>(S, zc, st, st + DF * D);
}

// ---------------------------------------------------------------------------
// Carry scan: ws[bh][p] <- init + sum_{p' < p} ws[bh][p']  (exclusive), and
// the total into ws[bh][P] (and S_out/z_out) when requested.
// grid = (BH, ceil(state_elems/256)), block = 256.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void carry_scan_kernel(ScanArgs a) {
  const int e = blockIdx.y * 256 + threadIdx.x;
  const int bh = blockIdx.x;
  if (e >= a.state_elems) return;
  const int sdd = a.DF * a.D;
  float run = 0.f;
  if (e < sdd) {
    if (a.S_in) run = a.S_in[(long long)bh * sdd + e];
  } else {
    if (a.z_in) run = a.z_in[(long long)bh * a.DF + (e - sdd)];
  }
  float* col = a.ws + (long long)bh * a.ws_slots * a.state_elems + e;
  for (int p = 0; p < a.P; ++p) {
    const float t = col[(long long)p * a.state_elems];
    if (a.exclusive) col[(long long)p * a.state_elems] = run;
    run += t;
  }
  if (a.write_total) col[(long long)a.P * a.state_elems] = run;
  if (e < sdd) {
    if (a.S_out) a.S_out[(long long)bh * sdd + e] = run;
  } else {
    if (a.z_out) a.z_out[(long long)bh * a.DF + (e - sdd)] = run;
  }
}

// ---------------------------------------------------------------------------
// Output pass.
// CAUSAL: y_i = [sum_{j<=i in chunk} w_ij v_j + phi(q_i)^T S_prev] / [..]
// otherwise: y_i = phi(q_i)^T S / phi(q_i)^T z with the total (S, z).
// grid = (BH, P), block = 64 * D/32 threads.
// ---------------------------------------------------------------------------
template <int D, int DF, typename OP, typename IN, bool CAUSAL>
__global__ __launch_bounds__(D * 2) void output_pass_kernel(FwdArgs a) {
  using Frag = typename Ops<OP>::frag;
  constexpr int NW = D / 32;
  constexpr int RBF = DF * Ops<OP>::kBytes;
  constexpr int RBV = D * Ops<OP>::kBytes;
  constexpr int QBYTES = 64 * RBF, KBYTES = CAUSAL ? 64 * RBF : 0, VBYTES = CAUSAL ? 64 * RBV : 0;
  constexpr int BUF = QBYTES + KBYTES + VBYTES;
  // double-buffer the staged chunk when two copies fit in LDS
  constexpr int NBUF = (2 * BUF + NW * DF * 4 <= 160 * 1024) ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * BUF + NW * DF * 4];
  float* zbuf = reinterpret_cast<float*>(smem + NBUF * BUF) + (threadIdx.x >> 6) * DF;

  const int bh = blockIdx.x, seg = blockIdx.y;
  const int c0 = seg * a.chunks_per_seg;
  const int c1 = min(c0 + a.chunks_per_seg, a.nchunks);
  const long long base = (long long)bh * a.N;
  const IN* q = static_cast<const IN*>(a.q);
  const IN* k = static_cast<const IN*>(a.k);
  const IN* v = static_cast<const IN*>(a.v);
  IN* out = static_cast<IN*>(a.out);
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6, h = l >> 5, li = l & 31;

  // ---- starting state ----
  f32x16 S[DF / 32];
  float zc[DF / 32];
  {
    const float* Sp;
    const float* zp;
    if (a.init_from_ws) {
      const float* st = a.ws + ((long long)bh * a.ws_slots + (CAUSAL ? seg : a.ws_total_slot)) * a.state_elems;
      Sp = st;
      zp = st + DF * D;
    } else {
      Sp = a.S_in ? a.S_in + (long long)bh * DF * D : nullptr;
      zp = a.z_in ? a.z_in + (long long)bh * DF : nullptr;
    }
    load_state<D, DF>(S, zc, Sp, zp);
  }
  // every wave keeps its own copy of z in LDS (read back by feature index)
#pragma unroll
  for (int cb = 0; cb < DF / 32; ++cb)
    if (h == 0) zbuf[32 * cb + li] = zc[cb];
  // non-causal: the state never changes; convert it once
  Frag Sf_const[CAUSAL ? 1 : DF / 16];
  if constexpr (!CAUSAL) {
#pragma unroll
    for (int kb = 0; kb < DF / 16; ++kb) Sf_const[kb] = Ops<OP>::from_acc(S[kb >> 1], kb & 1);
  }

  Prefetch<D, IN> pf;
  if (c0 < c1) {
    const int nv = min(64, a.N - 64 * c0);
    issue_loads<D, IN, true, CAUSAL>(pf, q, k, v, base + 64LL * c0, nv);
    stage_chunk<D, IN, OP, true, CAUSAL>(pf, smem, smem + QBYTES, smem + QBYTES + KBYTES, nv);
  }
  __syncthreads();

  for (int c = c0; c < c1; ++c) {
    const int buf = NBUF == 2 ? ((c - c0) & 1) : 0;
    uint8_t* sQ = smem + buf * BUF;
    uint8_t* sK = sQ + QBYTES;
    uint8_t* sV = sK + KBYTES;
    const int valid = min(64, a.N - 64 * c);
    const bool more = c + 1 < c1;
    const int nvalid = more ? min(64, a.N - 64 * (c + 1)) : 0;
    if (more) issue_loads<D, IN, true, CAUSAL>(pf, q, k, v, base + 64LL * (c + 1), nvalid);

    // phi(Q) fragments (B operand: contraction = feature, columns = query rows)
    Frag Bq[2][DF / 16];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int kb = 0; kb < DF / 16; ++kb) Bq[ib][kb] = Ops<OP>::template load_rows<RBF>(sQ, 32 * ib, 16 * kb);

    f32x16 num[2] = {f32x16{}, f32x16{}};
    float dpart[2] = {0.f, 0.f};
    Frag Vf[4];
    if constexpr (CAUSAL) {
      // scores A^T[j][i] = phi(k_j).phi(q_i) for tile pairs (jb, ib) with jb <= ib
      f32x16 A00 = {}, A01 = {}, A11 = {};
#pragma unroll
      for (int kb = 0; kb < DF / 16; ++kb) {
        Frag k0 = Ops<OP>::template load_rows<RBF>(sK, 0, 16 * kb);
        Frag k1 = Ops<OP>::template load_rows<RBF>(sK, 32, 16 * kb);
        Ops<OP>::mma(A00, k0, Bq[0][kb]);
        Ops<OP>::mma(A01, k0, Bq[1][kb]);
        Ops<OP>::mma(A11, k1, Bq[1][kb]);
      }
      // causal mask on the diagonal tiles (keep j <= i), rounding to the
      // operand precision, and the within-chunk part of the denominator
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jt = 8 * (r >> 2) + 4 * h + (r & 3);
        const bool keep = jt <= li;
        float x00 = keep ? A00[r] : 0.f, x11 = keep ? A11[r] : 0.f, x01 = A01[r];
        if constexpr (sizeof(OP) == 2) {
          x00 = round_bf16(x00);
          x11 = round_bf16(x11);
          x01 = round_bf16(x01);
        }
        A00[r] = x00;
        A11[r] = x11;
        A01[r] = x01;
        dpart[0] += x00;
        dpart[1] += x01 + x11;
      }
      // V^T fragments (rows = value columns of this wave, contraction = token)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Vf[kb] = Ops<OP>::template load_cols<RBV>(sV, 16 * kb, 32 * w);
      // intra-chunk numerator: num^T[e][i] += sum_j V^T[e][j] A^T[j][i]
#pragma unroll
      for (int kbj = 0; kbj < 2; ++kbj) {
        Ops<OP>::mma(num[0], Vf[kbj], Ops<OP>::from_acc(A00, kbj));
        Ops<OP>::mma(num[1], Vf[kbj], Ops<OP>::from_acc(A01, kbj));
        Ops<OP>::mma(num[1], Vf[2 + kbj], Ops<OP>::from_acc(A11, kbj));
      }
    }
    // inter-chunk numerator: num^T[e][i] += sum_c S^T[e][c] phi(Q)^T[c][i]
#pragma unroll
    for (int kb = 0; kb < DF / 16; ++kb) {
      Frag Sf;
      if constexpr (CAUSAL) Sf = Ops<OP>::from_acc(S[kb >> 1], kb & 1);
      else Sf = Sf_const[kb];
      Ops<OP>::mma(num[0], Sf, Bq[0][kb]);
      Ops<OP>::mma(num[1], Sf, Bq[1][kb]);
    }
    // denominator: phi(q_i).z over this lane's half of the features
    if (a.normalize) {
#pragma unroll
      for (int kb = 0; kb < DF / 16; ++kb) {
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(zbuf + 16 * kb + 8 * h);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(zbuf + 16 * kb + 8 * h + 4);
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          float s = 0.f;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) s += Ops<OP>::elem(Bq[ib][kb], jj) * z0[jj];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) s += Ops<OP>::elem(Bq[ib][kb], 4 + jj) * z1[jj];
          dpart[ib] += s;
        }
      }
    }
    // normalize and store: lane holds y[i = 32ib + li][e = 32w + 8(r/4) + 4h + r%4]
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      float inv = 1.f;
      if (a.normalize) {
        const float den = dpart[ib] + xor32(dpart[ib]);
        inv = 1.f / fmaxf(den, kEps);
      }
      const int i = 32 * ib + li;
      if (i < valid) {
        const long long rowoff = (base + 64LL * c + i) * D + 32 * w + 4 * h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float y0 = num[ib][4 * g + 0] * inv, y1 = num[ib][4 * g + 1] * inv;
          const float y2 = num[ib][4 * g + 2] * inv, y3 = num[ib][4 * g + 3] * inv;
          if constexpr (sizeof(IN) == 2) {
            *reinterpret_cast<u32x2*>(out + rowoff + 8 * g) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
          } else {
            *reinterpret_cast<f32x4*>(out + rowoff + 8 * g) = f32x4{y0, y1, y2, y3};
          }
        }
      }
    }
    if constexpr (CAUSAL) {
      // state update and z for the next chunk
      float zp[DF / 32];
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb) zp[cb] = 0.f;
      state_update<D, DF, OP>(S, zp, sK, sV, Vf);
#pragma unroll
      for (int cb = 0; cb < DF / 32; ++cb) {
        zc[cb] += zp[cb] + xor32(zp[cb]);
        if (h == 0) zbuf[32 * cb + li] = zc[cb];
      }
    }
    if (more) {
      if constexpr (NBUF == 1) __syncthreads();
      uint8_t* nQ = smem + (NBUF == 2 ? (buf ^ 1) : 0) * BUF;
      stage_chunk<D, IN, OP, true, CAUSAL>(pf, nQ, nQ + QBYTES, nQ + QBYTES + KBYTES, nvalid);
    }
    __syncthreads();
  }
  if constexpr (CAUSAL) {
    if (a.S_out && seg == a.nseg - 1) {
      store_state<D, DF>(S, zc, a.S_out + (long long)bh * DF * D, a.z_out + (long long)bh * DF);
    }
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (one instantiation per supported shape)
// ---------------------------------------------------------------------------
template <int D, int DF, typename OP, typename IN>
static hipError_t launch_prefill(const FwdArgs& a, const ScanArgs& s, bool causal, hipStream_t st,
                                 hipEvent_t* ev) {
  const dim3 block(D * 2);
  if (ev) (void)hipEventRecord(ev[0], st);
  if (a.run_state_pass) {
    hipLaunchKernelGGL((state_pass_kernel<D, DF, OP, IN>), dim3(a.BH, a.nseg_state), block, 0, st, a);
  }
  if (ev) (void)hipEventRecord(ev[1], st);
  if (a.run_scan) {
    hipLaunchKernelGGL(carry_scan_kernel, dim3(s.BH, (s.state_elems + 255) / 256), dim3(256), 0, st, s);
  }
  if (ev) (void)hipEventRecord(ev[2], st);
  if (causal) {
    hipLaunchKernelGGL((output_pass_kernel<D, DF, OP, IN, true>), dim3(a.BH, a.nseg), block, 0, st, a);
  } else {
    hipLaunchKernelGGL((output_pass_kernel<D, DF, OP, IN, false>), dim3(a.BH, a.nseg), block, 0, st, a);
  }
  if (ev) (void)hipEventRecord(ev[3], st);
  return hipGetLastError();
}

hipError_t prefill_dispatch(const FwdArgs& a, const ScanArgs& s, int D, int DF, int fmap, int dtype, bool causal,
                            hipStream_t st, hipEvent_t* ev) {
  if (fmap != kElu1) return hipErrorInvalidValue;
  if (dtype == 1) {  // bf16
    switch (D) {
      case 32: return launch_prefill<32, 32, __bf16, __bf16>(a, s, causal, st, ev);
      case 64: return launch_prefill<64, 64, __bf16, __bf16>(a, s, causal, st, ev);
      case 128: return launch_prefill<128, 128, __bf16, __bf16>(a, s, causal, st, ev);
    }
  } else {
    switch (D) {
      case 32: return launch_prefill<32, 32, float, float>(a, s, causal, st, ev);
      case 64: return launch_prefill<64, 64, float, float>(a, s, causal, st, ev);
      case 128: return launch_prefill<128, 128, float, float>(a, s, causal, st, ev);
    }
  }
  (void)DF;
  return hipErrorInvalidValue;
}

}  // namespace la

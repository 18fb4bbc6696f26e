// Host side of the C ABI declared in include/linattn.h: argument validation,
// work planning (sequence segments, workspace carving) and kernel dispatch.
// Nothing here allocates device memory. The only state kept between calls is
// the address, per device, of the library's device status flag.
#include "linattn.h"

#include <stdint.h>

#include <mutex>

#include "la_kernels.h"

// Raised (set to nonzero) by the chunked decay and gated kernels when a decay
// factor or gate lies outside the range they support; read and cleared by
// la_device_status. One per device: every GPU the library runs on holds its
// own copy, at its own address.
__device__ int la_status_flag;

// Workspace of la_forward_static (callers that cannot allocate): the segment
// states and every other scratch need of la_forward, up to
// LA_STATIC_SCRATCH_BYTES. Each GPU the library runs on holds its own copy
// from the first la_forward_static call on it until the process ends. In host
// code this name is only a stand-in: kernels get the device address that
// static_scratch_ptr() looked up.
static __device__ __align__(256) unsigned char scratch[LA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int* g_flag_addr[kMaxDevices];
void* g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on the first call on each device (that device
// current), kept per device; null when the runtime refuses.
void* static_scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_addr[dev] = p;
  }
  return g_scratch_addr[dev];
}

// Device address of la_status_flag on the current device (looked up once per
// device with that device current), or null when the runtime refuses.
int* status_flag_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_flag_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(la_status_flag)) != hipSuccess) return nullptr;
    g_flag_addr[dev] = static_cast<int*>(p);
  }
  return g_flag_addr[dev];
}

constexpr int kChunk = 64;
// Output/state passes aim for this many workgroups so that every compute unit
// has work even when batch * heads is small (long single sequences). One
// workgroup per compute unit: on the long-context and random-feature
// workloads 256 ran 5-10% faster than 512 or 384, and 128 far slower.
constexpr long long kTargetBlocks = 256;
// The gated forward and the gradient passes keep twice as many: the gated
// forward on the long-context workload took 916 us at 256 against 811 us at 512.
constexpr long long kTargetBlocksWide = 512;
// A segment never gets fewer chunks than this (its carried state costs about
// as much traffic as 64 tokens of q, k, v and out at d' = d).
constexpr int kMinChunksPerSegment = 4;
// Causal forwards whose segment states take at most this many bytes per
// sequence skip the carry scan: each output-pass workgroup adds the local
// sums of the segments before it while loading its initial state. On
// B=4 H=8 N=2048 d=64 (8 segments of 16.6 KB) that removes the scan's launch
// (27.1 -> 23.6 us per call); long sequences (16 states of 66 KB) keep the
// scan, since their last segments would read up to 1 MB of states each.
constexpr size_t kFoldBytes = 256 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, long long abytes, const void* b, long long bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool d_supported(int d) { return d == 32 || d == 64 || d == 128; }

// (d, m) pairs with random-feature kernels.
bool perf_supported(int d, int m) {
  switch (d) {
    case 32: return m == 64 || m == 128;
    case 64: return m == 64 || m == 128 || m == 256;
    case 128: return m == 64 || m == 128;
  }
  return false;
}

// Feature dimension d' for a map, or a negative status.
int feature_dim(const la_feature_map* fm, int d) {
  if (!fm) return LA_ERR_INVALID_ARG;
  if (fm->kind == LA_ELU1 || fm->kind == LA_IDENTITY) return d;
  if (fm->kind == LA_POLY2) return (d == 32 || d == 64) ? 1 + d + d * d : LA_ERR_UNSUPPORTED;
  if (fm->kind == LA_PERFORMER) {
    if (fm->m <= 0 || !fm->W || !aligned16(fm->W)) return LA_ERR_INVALID_ARG;
    if (!perf_supported(d, fm->m)) return LA_ERR_UNSUPPORTED;
    return fm->m;
  }
  return LA_ERR_INVALID_ARG;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
  int nchunks = 0;
  int P = 1, cps = 0;        // output pass
  int Ps = 0, cpss = 0;      // state pass
  int ws_slots = 0;
  bool state_pass = false, scan = false;
  size_t phi_bytes = 0;      // one mapped-feature buffer (random features), fp32-sized
  size_t ws_bytes = 0;       // total: two feature buffers, then the segment states
};

void split(int nchunks, long long BH, int& P, int& cps, long long target = kTargetBlocks) {
  long long want = (target + BH - 1) / BH;
  long long cap = nchunks / kMinChunksPerSegment;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  cps = (int)((nchunks + want - 1) / want);
  P = (nchunks + cps - 1) / cps;
}

Plan make_plan(long long BH, int N, int d, int dfeat, bool causal, bool mapped_inputs,
               long long target = kTargetBlocks) {
  Plan p;
  if (mapped_inputs && N > 0) p.phi_bytes = align256((size_t)BH * N * dfeat * sizeof(float));
  p.nchunks = (N + kChunk - 1) / kChunk;
  const size_t state_bytes = (size_t)(dfeat * d + dfeat) * sizeof(float);
  if (N == 0 || BH == 0) return p;
  split(p.nchunks, BH, p.P, p.cps, target);
  if (causal) {
    if (p.P > 1) {
      p.Ps = p.P - 1;  // the last segment's local sums are never carried
      p.cpss = p.cps;
      p.ws_slots = p.P;
      p.state_pass = true;
      p.scan = true;
    }
  } else {
    split(p.nchunks, BH, p.Ps, p.cpss, target);
    p.ws_slots = p.Ps + 1;
    p.state_pass = true;
    p.scan = true;
  }
  p.ws_bytes = 2 * p.phi_bytes + (size_t)BH * p.ws_slots * state_bytes;
  return p;
}

int status_from_hip(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

// Polynomial map: partial numerators, then the denominators.
size_t poly_part_bytes(long long BH, int N, int d) {
  return align256((size_t)la::poly_partials(d) * BH * N * d * sizeof(float));
}
size_t poly_ws_bytes(long long BH, int N, int d) {
  if (BH == 0 || N == 0) return 0;
  return poly_part_bytes(BH, N, d) + align256((size_t)la::poly_den_slots(d) * BH * N * sizeof(float));
}

}  // namespace

extern "C" {

int la_version(void) { return (0 << 16) | 2; }

int la_device_status(hipStream_t stream) {
  int* flag = status_flag_ptr();
  if (!flag) return LA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return LA_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, flag, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return LA_ERR_HIP;
  if (v == 0) return LA_OK;
  const int zero = 0;
  if (hipMemcpy(flag, &zero, sizeof(int), hipMemcpyHostToDevice) != hipSuccess) return LA_ERR_HIP;
  return LA_ERR_INVALID_ARG;
}

const char* la_status_string(int status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_ERR_INVALID_ARG: return "invalid argument";
    case LA_ERR_UNSUPPORTED: return "unsupported shape or feature map";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t la_forward_workspace_size_dt(int B, int H, int N, int d, const la_feature_map* feature_map, int causal,
                                    int dtype) {
  if (B < 0 || H < 0 || N < 0 || !d_supported(d)) return 0;
  if (dtype != LA_F32 && dtype != LA_BF16) return 0;
  const int dfeat = feature_dim(feature_map, d);
  if (dfeat <= 0) return 0;
  if (feature_map->kind == LA_POLY2) return poly_ws_bytes((long long)B * H, N, d);
  const bool mapped = feature_map->kind == LA_PERFORMER;
  const bool fused = mapped && la::perf_fused_supported(d, dfeat, dtype, causal != 0, false);
  return make_plan((long long)B * H, N, d, dfeat, causal != 0, mapped && !fused).ws_bytes;
}

size_t la_forward_workspace_size(int B, int H, int N, int d, const la_feature_map* feature_map, int causal) {
  const size_t a = la_forward_workspace_size_dt(B, H, N, d, feature_map, causal, LA_F32);
  const size_t b = la_forward_workspace_size_dt(B, H, N, d, feature_map, causal, LA_BF16);
  return a > b ? a : b;
}

}  // extern "C"

namespace {

// The whole forward; gamma (device, [H]) is the per-head decay or null.
// static_ws: the workspace is the library's `scratch` array (la_forward_static);
// workspace / workspace_bytes are then ignored.
int forward_impl(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                 const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
                 const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                 hipStream_t stream, hipEvent_t* events, const float* gamma, bool static_ws = false) {
  if (B < 0 || H < 0 || N < 0) return LA_ERR_INVALID_ARG;
  if (gamma && (causal != 1 || (reinterpret_cast<uintptr_t>(gamma) & 3u) != 0)) return LA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return LA_ERR_INVALID_ARG;
  if (normalize != 0 && normalize != 1) return LA_ERR_INVALID_ARG;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
  if ((S_in == nullptr) != (z_in == nullptr)) return LA_ERR_INVALID_ARG;
  if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
  if (!d_supported(d)) return LA_ERR_UNSUPPORTED;
  const int dfeat = feature_dim(feature_map, d);
  if (dfeat < 0) return dfeat;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 31) - 1) return LA_ERR_UNSUPPORTED;
  const long long esz = dtype == LA_BF16 ? 2 : 4;
  const long long tok_bytes = BH * N * d * esz;
  const long long s_bytes = BH * dfeat * d * 4, z_bytes = BH * dfeat * 4;
  if (S_in && (!aligned16(S_in) || !aligned16(z_in))) return LA_ERR_INVALID_ARG;
  if (S_out && (!aligned16(S_out) || !aligned16(z_out))) return LA_ERR_INVALID_ARG;
  if (S_out && (overlaps(S_out, s_bytes, z_out, z_bytes) || overlaps(S_out, s_bytes, S_in, s_bytes) ||
                overlaps(S_out, s_bytes, z_in, z_bytes) || overlaps(z_out, z_bytes, S_in, s_bytes) ||
                overlaps(z_out, z_bytes, z_in, z_bytes)))
    return LA_ERR_INVALID_ARG;

  if (BH == 0 || N == 0) {
    int st = LA_OK;
    if (BH > 0 && S_out)
      st = status_from_hip(la::copy_state_dispatch(S_in, z_in, S_out, z_out, s_bytes / 4, z_bytes / 4, stream));
    if (st == LA_OK && events) {  // every pass is empty: all four markers at once
      for (int i = 0; i < 4; ++i)
        if (hipEventRecord(events[i], stream) != hipSuccess) return LA_ERR_HIP;
    }
    return st;
  }
  if (!q || !k || !v || !out) return LA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_INVALID_ARG;
  if (overlaps(out, tok_bytes, q, tok_bytes) || overlaps(out, tok_bytes, k, tok_bytes) ||
      overlaps(out, tok_bytes, v, tok_bytes))
    return LA_ERR_INVALID_ARG;
  if (S_out && (overlaps(S_out, s_bytes, q, tok_bytes) || overlaps(S_out, s_bytes, k, tok_bytes) ||
                overlaps(S_out, s_bytes, v, tok_bytes) || overlaps(S_out, s_bytes, out, tok_bytes) ||
                overlaps(z_out, z_bytes, q, tok_bytes) || overlaps(z_out, z_bytes, k, tok_bytes) ||
                overlaps(z_out, z_bytes, v, tok_bytes) || overlaps(z_out, z_bytes, out, tok_bytes)))
    return LA_ERR_INVALID_ARG;
  // the decay factors are read by every pass: no output may overlap them
  if (gamma && (overlaps(out, tok_bytes, gamma, 4LL * H) || overlaps(S_out, s_bytes, gamma, 4LL * H) ||
                overlaps(z_out, z_bytes, gamma, 4LL * H)))
    return LA_ERR_INVALID_ARG;

  if (feature_map->kind == LA_POLY2) {
    if (gamma) return LA_ERR_UNSUPPORTED;
    const size_t need = poly_ws_bytes(BH, N, d);
    if (static_ws) {
      if (need > LA_STATIC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
      if (!(workspace = static_scratch_ptr())) return LA_ERR_HIP;
    } else {
      if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
      const long long wsz = (long long)need;
      if (overlaps(workspace, wsz, out, tok_bytes) || overlaps(workspace, wsz, q, tok_bytes) ||
          overlaps(workspace, wsz, k, tok_bytes) || overlaps(workspace, wsz, v, tok_bytes) ||
          overlaps(workspace, wsz, S_out, s_bytes) || overlaps(workspace, wsz, z_out, z_bytes) ||
          overlaps(workspace, wsz, S_in, s_bytes) || overlaps(workspace, wsz, z_in, z_bytes))
        return LA_ERR_INVALID_ARG;
    }
    if (events && hipEventRecord(events[0], stream) != hipSuccess) return LA_ERR_HIP;
    la::PolyArgs pa{};
    pa.q = q;
    pa.k = k;
    pa.v = v;
    pa.out = out;
    pa.BH = (int)BH;
    pa.N = N;
    pa.nchunks = (N + kChunk - 1) / kChunk;
    pa.normalize = normalize;
    pa.part = static_cast<float*>(workspace);
    pa.den = reinterpret_cast<float*>(static_cast<char*>(workspace) + poly_part_bytes(BH, N, d));
    pa.S_in = S_in;
    pa.z_in = z_in;
    pa.S_out = S_out;
    pa.z_out = z_out;
    const int st = status_from_hip(la::poly_forward_dispatch(pa, d, dtype, causal != 0, stream));
    if (st == LA_OK && events) {  // one pass: the state, scan and output markers coincide at its end
      for (int i = 1; i < 4; ++i)
        if (hipEventRecord(events[i], stream) != hipSuccess) return LA_ERR_HIP;
    }
    return st;
  }
  const bool mapped = feature_map->kind == LA_PERFORMER;
  if (mapped) {
    const long long wb = (long long)dfeat * d * 4;
    if (overlaps(out, tok_bytes, feature_map->W, wb) || overlaps(S_out, s_bytes, feature_map->W, wb) ||
        overlaps(z_out, z_bytes, feature_map->W, wb))
      return LA_ERR_INVALID_ARG;
  }
  // random features in bf16 (non-causal, or causal at d = 64): the
  // projection runs inside the chunked passes and the workspace holds
  // segment states only
  const bool fused = mapped && la::perf_fused_supported(d, dfeat, dtype, causal != 0, gamma != nullptr);
  const Plan p = make_plan(BH, N, d, dfeat, causal != 0, mapped && !fused);
  if (static_ws) {
    if (p.ws_bytes > LA_STATIC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
  } else if (p.ws_bytes > 0) {
    if (!workspace || workspace_bytes < p.ws_bytes) return LA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
    if (overlaps(workspace, (long long)p.ws_bytes, out, tok_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, q, tok_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, k, tok_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, v, tok_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, S_out, s_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, z_out, z_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, S_in, s_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, z_in, z_bytes) ||
        overlaps(workspace, (long long)p.ws_bytes, gamma, 4LL * H) ||
        (mapped && overlaps(workspace, (long long)p.ws_bytes, feature_map->W, (long long)dfeat * d * 4)))
      return LA_ERR_INVALID_ARG;
  }

  int* flag = nullptr;  // looked up after validation: a rejected call makes no HIP call
  if (gamma && !(flag = status_flag_ptr())) return LA_ERR_HIP;
  if (static_ws && p.ws_bytes > 0 && !(workspace = static_scratch_ptr())) return LA_ERR_HIP;
  if (events) {
    if (hipEventRecord(events[0], stream) != hipSuccess) return LA_ERR_HIP;
  }
  char* wsb = static_cast<char*>(workspace);
  const void* qm = q;
  const void* km = k;
  if (mapped && !fused) {
    // random features: phi(q), phi(k) into the workspace, in the operand
    // precision of the chunked passes; those passes then use them as given
    void* fq = wsb;
    void* fk = wsb + p.phi_bytes;
    la::FmapArgs fa{};
    fa.x = q;
    fa.phi = fq;
    fa.rows = BH * N;
    fa.W = feature_map->W;
    hipError_t e = la::fmap_dispatch(fa, d, dfeat, la::kPerformer, dtype, dtype, stream);
    if (e != hipSuccess) return LA_ERR_HIP;
    fa.x = k;
    fa.phi = fk;
    e = la::fmap_dispatch(fa, d, dfeat, la::kPerformer, dtype, dtype, stream);
    if (e != hipSuccess) return LA_ERR_HIP;
    qm = fq;
    km = fk;
  }

  la::FwdArgs a{};
  a.q = qm;
  a.k = km;
  a.v = v;
  a.out = out;
  a.BH = (int)BH;
  a.N = N;
  a.nchunks = p.nchunks;
  a.nseg = p.P;
  a.chunks_per_seg = p.cps;
  a.nseg_state = p.Ps;
  a.chunks_per_seg_state = p.cpss;
  a.run_state_pass = p.state_pass;
  a.run_scan = p.scan;
  a.ws = reinterpret_cast<float*>(wsb + 2 * p.phi_bytes);
  a.ws_slots = p.ws_slots;
  a.ws_total_slot = causal ? 0 : p.Ps;
  a.state_elems = dfeat * d + dfeat;
  a.init_from_ws = p.ws_slots > 0;
  a.S_in = S_in;
  a.z_in = z_in;
  a.S_out = causal ? S_out : nullptr;
  a.z_out = causal ? z_out : nullptr;
  a.normalize = normalize;
  a.W = feature_map->W;
  a.gamma = gamma;
  a.H = H;
  a.status_flag = flag;
  if (causal && !gamma && p.P > 1 && (size_t)p.P * a.state_elems * sizeof(float) <= kFoldBytes) {
    a.init_from_ws = 0;
    a.init_sum_ws = 1;
    a.run_scan = 0;
  }

  la::ScanArgs s{};
  s.ws = a.ws;
  s.ws_slots = p.ws_slots;
  s.state_elems = a.state_elems;
  s.BH = (int)BH;
  s.DF = dfeat;
  s.D = d;
  s.S_in = S_in;
  s.z_in = z_in;
  s.gamma = gamma;
  s.H = H;
  s.status_flag = flag;
  s.seg_len = 64 * p.cps;  // every combined (non-last) segment is whole
  if (causal) {
    s.P = p.P - 1;
    s.exclusive = 1;
    s.write_total = 1;  // prefix of the last segment
  } else {
    s.P = p.Ps;
    s.exclusive = 0;
    s.write_total = 1;
    s.S_out = S_out;
    s.z_out = z_out;
  }
  if (fused) return status_from_hip(la::perf_fused_dispatch(a, s, d, dfeat, causal != 0, stream, events));
  const int kfm = feature_map->kind == LA_ELU1 ? la::kElu1 : la::kIdentity;  // mapped features: identity inside
  return status_from_hip(la::prefill_dispatch(a, s, d, dfeat, kfm, dtype, causal != 0, gamma != nullptr, stream,
                                              events));
}

}  // namespace

extern "C" {

int la_forward_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                  const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
                  const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                  hipStream_t stream, hipEvent_t* events) {
  return forward_impl(q, k, v, out, B, H, N, d, feature_map, causal, normalize, dtype, S_in, z_in, S_out, z_out,
                      workspace, workspace_bytes, stream, events, nullptr);
}

int la_forward_decay(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                     const la_feature_map* feature_map, const float* gamma, int normalize, int dtype,
                     const float* S_in, const float* z_in, float* S_out, float* z_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  if (!gamma) return LA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, out, B, H, N, d, feature_map, 1, normalize, dtype, S_in, z_in, S_out, z_out,
                      workspace, workspace_bytes, stream, nullptr, gamma);
}

int la_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
               const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
               const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  return la_forward_ex(q, k, v, out, B, H, N, d, feature_map, causal, normalize, dtype, S_in, z_in, S_out, z_out,
                       workspace, workspace_bytes, stream, nullptr);
}

int la_forward_static(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                      const la_feature_map* feature_map, int causal, int normalize, int dtype, const float* S_in,
                      const float* z_in, float* S_out, float* z_out, hipStream_t stream) {
  return forward_impl(q, k, v, out, B, H, N, d, feature_map, causal, normalize, dtype, S_in, z_in, S_out, z_out,
                      nullptr, 0, stream, nullptr, nullptr, true);
}

}  // extern "C"

namespace {

int decode_impl(float* S, float* z, const void* q, const void* k, const void* v, void* out, int B, int H, int d,
                const la_feature_map* feature_map, int normalize, int dtype, hipStream_t stream,
                const float* gamma) {
  if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
  if (gamma && (reinterpret_cast<uintptr_t>(gamma) & 3u) != 0) return LA_ERR_INVALID_ARG;
  if (normalize != 0 && normalize != 1) return LA_ERR_INVALID_ARG;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
  if (!d_supported(d)) return LA_ERR_UNSUPPORTED;
  const int dfeat = feature_dim(feature_map, d);
  if (dfeat < 0) return dfeat;
  const long long BH = (long long)B * H;
  if (BH == 0) return LA_OK;
  if (BH > (1LL << 31) - 1) return LA_ERR_UNSUPPORTED;
  if (!S || !z || !q || !k || !v || !out) return LA_ERR_INVALID_ARG;
  if (!aligned16(S) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return LA_ERR_INVALID_ARG;
  const long long esz = dtype == LA_BF16 ? 2 : 4;
  const long long tb = BH * d * esz, sb = BH * dfeat * d * 4, zb = BH * dfeat * 4;
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) || overlaps(out, tb, S, sb) ||
      overlaps(out, tb, z, zb) || overlaps(S, sb, z, zb) || overlaps(S, sb, q, tb) || overlaps(S, sb, k, tb) ||
      overlaps(S, sb, v, tb) || overlaps(z, zb, q, tb) || overlaps(z, zb, k, tb) || overlaps(z, zb, v, tb))
    return LA_ERR_INVALID_ARG;
  if (feature_map->kind == LA_PERFORMER) {
    const long long wb = (long long)dfeat * d * 4;
    if (overlaps(out, tb, feature_map->W, wb) || overlaps(S, sb, feature_map->W, wb) ||
        overlaps(z, zb, feature_map->W, wb))
      return LA_ERR_INVALID_ARG;
  }
  if (gamma && (overlaps(out, tb, gamma, 4LL * H) || overlaps(S, sb, gamma, 4LL * H) ||
                overlaps(z, zb, gamma, 4LL * H)))
    return LA_ERR_INVALID_ARG;
  la::DecodeArgs a{};
  a.S = S;
  a.z = z;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.BH = (int)BH;
  a.normalize = normalize;
  a.W = feature_map->W;
  a.gamma = gamma;
  a.H = H;
  if (feature_map->kind == LA_POLY2) {
    if (gamma) return LA_ERR_UNSUPPORTED;
    return status_from_hip(la::poly_decode_dispatch(a, d, dtype, stream));
  }
  return status_from_hip(la::decode_dispatch(a, d, dfeat, feature_map->kind, dtype, stream));
}

}  // namespace

extern "C" {

int la_decode_step(float* S, float* z, const void* q, const void* k, const void* v, void* out, int B, int H,
                   int d, const la_feature_map* feature_map, int normalize, int dtype, hipStream_t stream) {
  return decode_impl(S, z, q, k, v, out, B, H, d, feature_map, normalize, dtype, stream, nullptr);
}

int la_decode_step_decay(float* S, float* z, const void* q, const void* k, const void* v, void* out, int B, int H,
                         int d, const la_feature_map* feature_map, const float* gamma, int normalize, int dtype,
                         hipStream_t stream) {
  if (!gamma) return LA_ERR_INVALID_ARG;
  return decode_impl(S, z, q, k, v, out, B, H, d, feature_map, normalize, dtype, stream, gamma);
}

int la_feature_map_apply(const void* x, void* phi, long long rows, int d, const la_feature_map* feature_map,
                         int in_dtype, int out_dtype, hipStream_t stream) {
  if (rows < 0) return LA_ERR_INVALID_ARG;
  if ((in_dtype != LA_F32 && in_dtype != LA_BF16) || (out_dtype != LA_F32 && out_dtype != LA_BF16))
    return LA_ERR_INVALID_ARG;
  if (!d_supported(d)) return LA_ERR_UNSUPPORTED;
  const int dfeat = feature_dim(feature_map, d);
  if (dfeat < 0) return dfeat;
  if (rows == 0) return LA_OK;
  if (!x || !phi || !aligned16(x) || !aligned16(phi)) return LA_ERR_INVALID_ARG;
  const long long xb = rows * d * (in_dtype == LA_BF16 ? 2 : 4);
  const long long pb = rows * dfeat * (out_dtype == LA_BF16 ? 2 : 4);
  if (overlaps(x, xb, phi, pb)) return LA_ERR_INVALID_ARG;
  if (feature_map->kind == LA_PERFORMER && overlaps(phi, pb, feature_map->W, (long long)dfeat * d * 4))
    return LA_ERR_INVALID_ARG;
  la::FmapArgs a{};
  a.x = x;
  a.phi = phi;
  a.rows = rows;
  a.W = feature_map->W;
  if (feature_map->kind == LA_POLY2) return status_from_hip(la::poly_fmap_dispatch(a, d, in_dtype, out_dtype, stream));
  return status_from_hip(la::fmap_dispatch(a, d, dfeat, feature_map->kind, in_dtype, out_dtype, stream));
}

}  // extern "C"

namespace {

// Segments of a pass with one workgroup per CU, in state-pass segments: two
// where P state-pass segments per sequence need two rounds of workgroups
// (B*H*P >= 512), else one.
int paired_segments(long long BH, int P) { return (P >= 2 && BH * P >= 2 * kTargetBlocks) ? 2 : 1; }

struct BwdPlan {
  int nchunks = 0, P = 1, cps = 0;
  size_t fwd_bytes = 0, rev_bytes = 0, row_bytes = 0, ws_bytes = 0;
};

BwdPlan make_bwd_plan(long long BH, int N, int d) {
  BwdPlan p;
  if (N == 0 || BH == 0) return p;
  p.nchunks = (N + kChunk - 1) / kChunk;
  split(p.nchunks, BH, p.P, p.cps, kTargetBlocksWide);
  const size_t state_bytes = (size_t)(d * d + d) * sizeof(float);
  p.fwd_bytes = p.P > 1 ? align256((size_t)BH * p.P * state_bytes) : 0;
  p.rev_bytes = align256((size_t)BH * (p.P + 1) * state_bytes);
  p.row_bytes = align256((size_t)BH * N * 2 * sizeof(float));
  p.ws_bytes = p.fwd_bytes + p.rev_bytes + p.row_bytes;
  return p;
}

// Gradient requests support the maps applied inside the kernels (d' = d).
int bwd_map(const la_feature_map* fm, int d) {
  const int dfeat = feature_dim(fm, d);
  if (dfeat < 0) return dfeat;
  return (fm->kind == LA_PERFORMER || fm->kind == LA_POLY2) ? LA_ERR_UNSUPPORTED : LA_OK;
}

}  // namespace

extern "C" {

size_t la_backward_workspace_size(int B, int H, int N, int d, const la_feature_map* feature_map) {
  if (B < 0 || H < 0 || N < 0 || !d_supported(d) || bwd_map(feature_map, d) != LA_OK) return 0;
  return make_bwd_plan((long long)B * H, N, d).ws_bytes;
}

}  // extern "C"

namespace {

// The gradient passes; gamma (device, [H]) is the per-head decay or null.
int backward_impl(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv, int B,
                  int H, int N, int d, const la_feature_map* feature_map, int normalize, int dtype, const float* S_in,
                  const float* z_in, const float* dS_out, const float* dz_out, float* dS_in, float* dz_in,
                  void* workspace, size_t workspace_bytes, hipStream_t stream, const float* gamma) {
  if (B < 0 || H < 0 || N < 0) return LA_ERR_INVALID_ARG;
  if (gamma && (reinterpret_cast<uintptr_t>(gamma) & 3u) != 0) return LA_ERR_INVALID_ARG;
  if (normalize != 0 && normalize != 1) return LA_ERR_INVALID_ARG;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
  if ((S_in == nullptr) != (z_in == nullptr) || (dS_out == nullptr) != (dz_out == nullptr) ||
      (dS_in == nullptr) != (dz_in == nullptr))
    return LA_ERR_INVALID_ARG;
  if (!d_supported(d)) return LA_ERR_UNSUPPORTED;
  const int fs = bwd_map(feature_map, d);
  if (fs != LA_OK) return fs;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 31) - 1) return LA_ERR_UNSUPPORTED;
  const long long esz = dtype == LA_BF16 ? 2 : 4;
  const long long tb = BH * N * d * esz, sb = BH * d * d * 4, zb = BH * d * 4;
  for (const void* p : {(const void*)S_in, (const void*)z_in, (const void*)dS_out, (const void*)dz_out,
                        (const void*)dS_in, (const void*)dz_in})
    if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
  // written state gradients overlap nothing else
  if (dS_in) {
    const void* ro[] = {S_in, z_in, dS_out, dz_out};
    const long long rb[] = {sb, zb, sb, zb};
    if (overlaps(dS_in, sb, dz_in, zb)) return LA_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
      if (overlaps(dS_in, sb, ro[i], rb[i]) || overlaps(dz_in, zb, ro[i], rb[i])) return LA_ERR_INVALID_ARG;
  }
  const BwdPlan p = make_bwd_plan(BH, N, d);
  if (BH == 0 || N == 0) {
    if (BH > 0 && dS_in)
      return status_from_hip(la::copy_state_dispatch(dS_out, dz_out, dS_in, dz_in, sb / 4, zb / 4, stream));
    return LA_OK;
  }
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return LA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return LA_ERR_INVALID_ARG;
  {
    const void* wr[] = {dq, dk, dv, dS_in, dz_in};
    const long long wrb[] = {tb, tb, tb, sb, zb};
    const void* all[] = {q, k, v, dout, S_in, z_in, dS_out, dz_out, dq, dk, dv, dS_in, dz_in};
    const long long allb[] = {tb, tb, tb, tb, sb, zb, sb, zb, tb, tb, tb, sb, zb};
    for (int i = 0; i < 5; ++i) {
      for (int j = 0; j < 13; ++j)
        if (all[j] != wr[i] && overlaps(wr[i], wrb[i], all[j], allb[j])) return LA_ERR_INVALID_ARG;
      if (gamma && overlaps(wr[i], wrb[i], gamma, 4LL * H)) return LA_ERR_INVALID_ARG;
    }
    if (!workspace || workspace_bytes < p.ws_bytes) return LA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
    for (int j = 0; j < 13; ++j)
      if (overlaps(workspace, (long long)p.ws_bytes, all[j], allb[j])) return LA_ERR_INVALID_ARG;
    if (gamma && overlaps(workspace, (long long)p.ws_bytes, gamma, 4LL * H)) return LA_ERR_INVALID_ARG;
  }
  int* flag = nullptr;
  if (gamma && !(flag = status_flag_ptr())) return LA_ERR_HIP;
  char* wsb = static_cast<char*>(workspace);
  float* ws_fwd = reinterpret_cast<float*>(wsb);
  float* ws_rev = reinterpret_cast<float*>(wsb + p.fwd_bytes);
  float* rowstats = reinterpret_cast<float*>(wsb + p.fwd_bytes + p.rev_bytes);
  const int state_elems = d * d + d;

  // forward states entering each segment (as la_forward, causal)
  la::FwdArgs fa{};
  fa.q = q;
  fa.k = k;
  fa.v = v;
  fa.BH = (int)BH;
  fa.N = N;
  fa.nchunks = p.nchunks;
  fa.nseg = p.P;
  fa.chunks_per_seg = p.cps;
  fa.nseg_state = p.P - 1;
  fa.chunks_per_seg_state = p.cps;
  fa.run_state_pass = p.P > 1;
  fa.run_scan = p.P > 1;
  fa.ws = ws_fwd;
  fa.ws_slots = p.P;
  fa.state_elems = state_elems;
  fa.S_in = S_in;
  fa.z_in = z_in;
  fa.normalize = normalize;
  fa.H = H;
  fa.gamma = gamma;
  fa.status_flag = flag;
  la::ScanArgs fsa{};
  fsa.ws = ws_fwd;
  fsa.ws_slots = p.P;
  fsa.state_elems = state_elems;
  fsa.BH = (int)BH;
  fsa.P = p.P - 1;
  fsa.DF = d;
  fsa.D = d;
  fsa.exclusive = 1;
  fsa.write_total = 1;
  fsa.S_in = S_in;
  fsa.z_in = z_in;
  fsa.H = H;
  fsa.seg_len = 64 * p.cps;
  fsa.gamma = gamma;
  fsa.status_flag = flag;

  la::BwdArgs b{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.dy = dout;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.BH = (int)BH;
  b.N = N;
  b.nchunks = p.nchunks;
  // The dq and dk/dv passes (one workgroup per CU) run whole segments of two
  // state-pass segments when the state passes' split needs two rounds of
  // workgroups; the state passes (two workgroups per CU) stay faster at the
  // finer split. Gradients on B1 H16 N65536 d128: 1307-1319 -> 1277-1302 us.
  const int stride = paired_segments(BH, p.P);
  b.nseg = (p.P + stride - 1) / stride;
  b.chunks_per_seg = p.cps * stride;
  b.nseg_state = p.P;
  b.chunks_per_seg_state = p.cps;
  b.seg_stride = stride;
  b.normalize = normalize;
  b.ws_fwd = ws_fwd;
  b.fwd_slots = p.P;
  b.init_from_ws = p.P > 1;
  b.S_in = S_in;
  b.z_in = z_in;
  b.ws_rev = ws_rev;
  b.state_elems = state_elems;
  b.rowstats = rowstats;
  b.gamma = gamma;
  b.H = H;
  b.dS_out = dS_out;
  b.dz_out = dz_out;
  b.status_flag = flag;

  // suffix sums of the segments' gradient states, seeded with dS_out / dz_out
  la::ScanArgs rs{};
  rs.ws = ws_rev;
  rs.ws_slots = p.P + 1;
  rs.state_elems = state_elems;
  rs.BH = (int)BH;
  rs.P = p.P;
  rs.DF = d;
  rs.D = d;
  rs.exclusive = 1;
  rs.write_total = 1;
  // with decay the final-state cotangents enter through the gradient passes
  // (the last segment may be partial, so a whole-segment factor would not fit)
  rs.S_in = gamma ? nullptr : dS_out;
  rs.z_in = gamma ? nullptr : dz_out;
  rs.S_out = dS_in;
  rs.z_out = dz_in;
  rs.H = H;
  rs.seg_len = 64 * p.cps;
  rs.gamma = gamma;
  rs.status_flag = flag;
  const int kfm = feature_map->kind == LA_ELU1 ? la::kElu1 : la::kIdentity;
  return status_from_hip(la::backward_dispatch(fa, fsa, b, rs, d, kfm, dtype, gamma != nullptr, stream));
}

}  // namespace

extern "C" {

int la_backward(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv, int B,
                int H, int N, int d, const la_feature_map* feature_map, int normalize, int dtype, const float* S_in,
                const float* z_in, const float* dS_out, const float* dz_out, float* dS_in, float* dz_in,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return backward_impl(q, k, v, dout, dq, dk, dv, B, H, N, d, feature_map, normalize, dtype, S_in, z_in, dS_out,
                       dz_out, dS_in, dz_in, workspace, workspace_bytes, stream, nullptr);
}

int la_backward_decay(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, const la_feature_map* feature_map, const float* gamma, int normalize,
                      int dtype, const float* S_in, const float* z_in, const float* dS_out, const float* dz_out,
                      float* dS_in, float* dz_in, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!gamma) return LA_ERR_INVALID_ARG;
  return backward_impl(q, k, v, dout, dq, dk, dv, B, H, N, d, feature_map, normalize, dtype, S_in, z_in, dS_out,
                       dz_out, dS_in, dz_in, workspace, workspace_bytes, stream, gamma);
}

}  // extern "C"

namespace {

struct GatedPlan {
  Plan p;
  size_t state_bytes = 0, lfac_bytes = 0, ws_bytes = 0;
};

GatedPlan make_gated_plan(long long BH, int N, int d) {
  GatedPlan g;
  g.p = make_plan(BH, N, d, d, true, false, kTargetBlocksWide);  // the causal split; its workspace holds the segment states
  if (N == 0 || BH == 0) return g;
  g.state_bytes = align256(g.p.ws_bytes);
  g.lfac_bytes = g.p.P > 1 ? align256((size_t)BH * g.p.P * d * sizeof(float)) : 0;
  g.ws_bytes = g.state_bytes + g.lfac_bytes;
  return g;
}

}  // namespace

extern "C" {

size_t la_forward_gated_workspace_size(int B, int H, int N, int d, const la_feature_map* feature_map) {
  if (B < 0 || H < 0 || N < 0 || !d_supported(d) || bwd_map(feature_map, d) != LA_OK) return 0;
  return make_gated_plan((long long)B * H, N, d).ws_bytes;
}

int la_forward_gated(const void* q, const void* k, const void* v, const float* log_gates, void* out, int B, int H,
                     int N, int d, const la_feature_map* feature_map, int normalize, int dtype, const float* S_in,
                     const float* z_in, float* S_out, float* z_out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return LA_ERR_INVALID_ARG;
  if (normalize != 0 && normalize != 1) return LA_ERR_INVALID_ARG;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
  if ((S_in == nullptr) != (z_in == nullptr) || (S_out == nullptr) != (z_out == nullptr)) return LA_ERR_INVALID_ARG;
  if (!d_supported(d)) return LA_ERR_UNSUPPORTED;
  const int fs = bwd_map(feature_map, d);  // maps applied in the kernels (d' = d)
  if (fs != LA_OK) return fs;
  const long long BH = (long long)B * H;
  if (BH > (1LL << 31) - 1) return LA_ERR_UNSUPPORTED;
  const long long esz = dtype == LA_BF16 ? 2 : 4;
  const long long tb = BH * N * d * esz, gb = BH * N * d * 4, sb = BH * d * d * 4, zb = BH * d * 4;
  for (const void* p : {(const void*)S_in, (const void*)z_in, (const void*)S_out, (const void*)z_out})
    if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
  if (S_out) {
    const void* ro[] = {S_in, z_in};
    const long long rb[] = {sb, zb};
    if (overlaps(S_out, sb, z_out, zb)) return LA_ERR_INVALID_ARG;
    for (int i = 0; i < 2; ++i)
      if (overlaps(S_out, sb, ro[i], rb[i]) || overlaps(z_out, zb, ro[i], rb[i])) return LA_ERR_INVALID_ARG;
  }
  if (BH == 0 || N == 0) {
    if (BH > 0 && S_out)
      return status_from_hip(la::copy_state_dispatch(S_in, z_in, S_out, z_out, sb / 4, zb / 4, stream));
    return LA_OK;
  }
  if (!q || !k || !v || !out || !log_gates) return LA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(log_gates))
    return LA_ERR_INVALID_ARG;
  const GatedPlan g = make_gated_plan(BH, N, d);
  {
    const void* all[] = {q, k, v, log_gates, S_in, z_in};
    const long long allb[] = {tb, tb, tb, gb, sb, zb};
    for (int j = 0; j < 6; ++j) {
      if (overlaps(out, tb, all[j], allb[j])) return LA_ERR_INVALID_ARG;
      if (S_out && (overlaps(S_out, sb, all[j], allb[j]) || overlaps(z_out, zb, all[j], allb[j])))
        return LA_ERR_INVALID_ARG;
    }
    if (S_out && (overlaps(S_out, sb, out, tb) || overlaps(z_out, zb, out, tb))) return LA_ERR_INVALID_ARG;
    if (g.ws_bytes > 0) {
      if (!workspace || workspace_bytes < g.ws_bytes) return LA_ERR_WORKSPACE;
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
      const void* any[] = {q, k, v, log_gates, S_in, z_in, out, S_out, z_out};
      const long long anyb[] = {tb, tb, tb, gb, sb, zb, tb, sb, zb};
      for (int j = 0; j < 9; ++j)
        if (overlaps(workspace, (long long)g.ws_bytes, any[j], anyb[j])) return LA_ERR_INVALID_ARG;
    }
  }
  const Plan& p = g.p;
  int* flag = status_flag_ptr();
  if (!flag) return LA_ERR_HIP;
  char* wsb = static_cast<char*>(workspace);
  la::GatedArgs ga{};
  la::FwdArgs& a = ga.f;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.BH = (int)BH;
  a.N = N;
  a.nchunks = p.nchunks;
  // The output pass (one workgroup per CU) runs whole segments of two
  // state-pass segments when the state pass's split needs two rounds of
  // workgroups; the state pass (two workgroups per CU) keeps the finer split.
  const int stride = paired_segments(BH, p.P);
  a.nseg = (p.P + stride - 1) / stride;
  a.chunks_per_seg = p.cps * stride;
  a.nseg_state = p.Ps;
  a.chunks_per_seg_state = p.cpss;
  a.run_state_pass = p.state_pass;
  a.run_scan = p.scan;
  a.ws = reinterpret_cast<float*>(wsb);
  a.ws_slots = p.ws_slots;
  a.state_elems = d * d + d;
  a.init_from_ws = p.ws_slots > 0;
  a.S_in = S_in;
  a.z_in = z_in;
  a.S_out = S_out;
  a.z_out = z_out;
  a.normalize = normalize;
  a.H = H;
  a.status_flag = flag;
  ga.log_gates = log_gates;
  ga.lfac = g.lfac_bytes ? reinterpret_cast<float*>(wsb + g.state_bytes) : nullptr;
  ga.lfac_stride = p.P;
  ga.seg_stride = stride;

  la::ScanArgs s{};
  s.ws = a.ws;
  s.ws_slots = p.ws_slots;
  s.state_elems = a.state_elems;
  s.BH = (int)BH;
  s.P = p.P - 1;
  s.DF = d;
  s.D = d;
  s.exclusive = 1;
  s.write_total = 1;
  s.S_in = S_in;
  s.z_in = z_in;
  s.H = H;
  s.seg_len = 64 * p.cps;
  s.lfac = ga.lfac;
  s.lfac_stride = p.P;
  s.status_flag = flag;
  const int kfm = feature_map->kind == LA_ELU1 ? la::kElu1 : la::kIdentity;
  return status_from_hip(la::gated_dispatch(ga, s, d, kfm, dtype, stream));
}

int la_decode_step_gated(float* S, float* z, const void* q, const void* k, const void* v, const float* log_gate,
                         void* out, int B, int H, int d, const la_feature_map* feature_map, int normalize, int dtype,
                         hipStream_t stream) {
  if (B < 0 || H < 0) return LA_ERR_INVALID_ARG;
  if (normalize != 0 && normalize != 1) return LA_ERR_INVALID_ARG;
  if (dtype != LA_F32 && dtype != LA_BF16) return LA_ERR_INVALID_ARG;
  if (!d_supported(d)) return LA_ERR_UNSUPPORTED;
  const int dfeat = feature_dim(feature_map, d);
  if (dfeat < 0) return dfeat;
  if (feature_map->kind == LA_POLY2) return LA_ERR_UNSUPPORTED;
  const long long BH = (long long)B * H;
  if (BH == 0) return LA_OK;
  if (!log_gate || !aligned16(log_gate)) return LA_ERR_INVALID_ARG;
  const long long tb = BH * d * (dtype == LA_BF16 ? 2 : 4), sb = BH * dfeat * d * 4, zb = BH * dfeat * 4;
  if (overlaps(log_gate, zb, out, tb) || overlaps(log_gate, zb, S, sb) || overlaps(log_gate, zb, z, zb))
    return LA_ERR_INVALID_ARG;
  // the shared decode path with the per-feature gate
  if (!S || !z || !q || !k || !v || !out) return LA_ERR_INVALID_ARG;
  if (!aligned16(S) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return LA_ERR_INVALID_ARG;
  if (BH > (1LL << 31) - 1) return LA_ERR_UNSUPPORTED;
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) || overlaps(out, tb, S, sb) ||
      overlaps(out, tb, z, zb) || overlaps(S, sb, z, zb) || overlaps(S, sb, q, tb) || overlaps(S, sb, k, tb) ||
      overlaps(S, sb, v, tb) || overlaps(z, zb, q, tb) || overlaps(z, zb, k, tb) || overlaps(z, zb, v, tb))
    return LA_ERR_INVALID_ARG;
  if (feature_map->kind == LA_PERFORMER) {
    const long long wb = (long long)dfeat * d * 4;
    if (overlaps(out, tb, feature_map->W, wb) || overlaps(S, sb, feature_map->W, wb) ||
        overlaps(z, zb, feature_map->W, wb))
      return LA_ERR_INVALID_ARG;
  }
  la::DecodeArgs a{};
  a.S = S;
  a.z = z;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.BH = (int)BH;
  a.normalize = normalize;
  a.W = feature_map->W;
  a.H = H;
  a.lgate = log_gate;
  return status_from_hip(la::decode_dispatch(a, d, dfeat, feature_map->kind, dtype, stream));
}

}  // extern "C"

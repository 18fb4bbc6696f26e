// Kernel argument blocks and launch entry points shared by the host API
// (la_api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

namespace la {

enum FeatureMap {
  kElu1 = 0,       // elu(x) + 1 applied in the kernels
  kPerformer = 1,  // positive random features
  kIdentity = 2,   // phi(x) = x: the identity map, or features already mapped by the random-feature kernel
};

// Chunked forward (prefill / non-causal). All pointers are device pointers.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int BH;                  // batch * heads
  int N;                   // tokens per sequence
  int nchunks;             // ceil(N / 64)
  int nseg;                // output-pass segments per sequence
  int chunks_per_seg;      // output-pass chunks per segment
  int nseg_state;          // state-pass segments per sequence
  int chunks_per_seg_state;
  int run_state_pass;
  int run_scan;
  float* ws;               // workspace: [BH][ws_slots][state_elems] fp32
  int ws_slots;
  int ws_total_slot;       // non-causal: slot holding the full-sequence state
  int state_elems;         // DF * D + DF
  int init_from_ws;        // output pass starts from the workspace slot (else S_in/z_in or zero)
  int init_sum_ws;         // causal, no decay: segment s starts from S_in/z_in (or zero) plus the
                           // local sums in slots 0..s-1, added by the output pass itself (no carry scan)
  const float* S_in;       // [BH][DF][D] or null
  const float* z_in;       // [BH][DF] or null
  float* S_out;            // [BH][DF][D] or null (causal: written by the last segment)
  float* z_out;
  int normalize;
  const float* W;          // random-feature projection [DF][D] (fp32) or null
  const float* gamma;      // decay per head [H] (causal only) or null
  int H;                   // heads (gamma index = bh % H)
  int skip_output;         // run the state pass and scan only (segment prefixes for the gradient passes)
  int hilo_keys;           // state pass with phi(K) as hi + lo bf16 (bf16, no decay, d' = d; gradient passes)
  int* status_flag;        // device flag raised when a decay factor or gate is outside the supported range
};

struct ScanArgs {
  float* ws;
  int ws_slots;
  int state_elems;
  int BH;
  int P;            // number of local states to combine (slots 0..P-1)
  int DF, D;
  int exclusive;    // rewrite slots 0..P-1 with exclusive prefixes
  int write_total;  // write the sum into slot P
  const float* S_in;
  const float* z_in;
  float* S_out;     // total state (non-causal only)
  float* z_out;
  const float* gamma;  // decay per head [H] or null: P_{s+1} = gamma^seg_len P_s + L_s
  int H;
  int seg_len;         // tokens per combined segment (all full)
  const float* lfac;   // gated: per-segment, per-channel log factors [BH][lfac_stride][DF] or null:
  int lfac_stride;     //   P_{s+1} = diag(exp(lfac_s)) P_s + L_s
  int* status_flag;    // as FwdArgs::status_flag
};

struct DecodeArgs {
  float* S;         // [BH][DF][D], updated in place
  float* z;         // [BH][DF], updated in place
  const void* q;    // [BH][D]
  const void* k;
  const void* v;
  void* out;        // [BH][D]
  int BH;
  int normalize;
  const float* W;   // [DF][D] or null
  const float* gamma;  // decay per head [H] or null: S <- gamma S + phi(k) v^T
  int H;
  const float* lgate;  // gated: log-gate per head and feature [BH][DF] or null: S <- diag(exp(lgate)) S + ...
};

// Gradient passes (causal; d' = d). Workspace regions: the forward segment
// prefixes (as FwdArgs::ws), the reverse ("suffix") states and two floats per
// token (1 / max(den, eps) and the denominator cotangent).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dy;          // output cotangent [BH][N][D]
  void* dq;
  void* dk;
  void* dv;
  int BH, N, nchunks;
  int nseg, chunks_per_seg;  // segments of the dq and dk/dv passes
  // The state passes (forward states, r-state pass, both scans) split each
  // of those segments into seg_stride (1 or 2) segments of chunks_per_seg_state
  // chunks, nseg_state in all; the state slots below count those.
  int nseg_state, chunks_per_seg_state, seg_stride;
  int normalize;
  const float* ws_fwd;     // [BH][fwd_slots][state_elems]: state entering state-pass segment s (slot s)
  int fwd_slots;
  int init_from_ws;        // else S_in / z_in (or zero) enter the single segment
  const float* S_in;
  const float* z_in;
  float* ws_rev;           // [BH][nseg_state + 1][state_elems]: slot nseg_state-1-s holds state-pass
                           // segment s's sums, then (after the scan) the cotangent of the state leaving it
  int state_elems;         // D * D + D
  float* rowstats;         // [BH][N][2]: 1 / max(den, eps), d loss / d den
  const float* gamma;      // decay per head [H] or null
  int H;
  const float* dS_out;     // decay: cotangents of the final state, added by the passes themselves
  const float* dz_out;
  int* status_flag;        // as FwdArgs::status_flag
};

// Gated linear attention (per-token, per-channel log-gates on the feature
// dimension): the forward's argument block plus the gates and the
// per-segment total log-gates the state pass writes for the scan.
struct GatedArgs {
  FwdArgs f;
  const float* log_gates;  // [BH][N][D] fp32, natural log of the gates, in [-log 4, 0]
  float* lfac;             // [BH][lfac_stride][D] fp32 (workspace): total log-gate of each state-pass segment
  int lfac_stride;
  // output-pass segment s starts where state-pass segment s * seg_stride does
  // (its state in ws slot s * seg_stride); f.nseg, f.chunks_per_seg describe
  // the output pass, f.nseg_state, f.chunks_per_seg_state the state pass
  int seg_stride;
};

// Degree-2 polynomial map (d' = 1 + d + d^2), chunked forward. Workspace:
// partial numerators [poly_partials(D)][BH][N][D] fp32, then partial
// denominators [poly_den_slots(D)][BH][N] fp32.
struct PolyArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int BH, N, nchunks;
  int normalize;
  float* part;
  float* den;
  const float* S_in;  // [BH][d'][D] or null
  const float* z_in;  // [BH][d']
  float* S_out;       // written at the end (causal: final state; non-causal: the total)
  float* z_out;
};

struct FmapArgs {
  const void* x;    // [rows][D]
  void* phi;        // [rows][DF]
  long long rows;
  const float* W;   // [DF][D] or null
};

hipError_t prefill_dispatch(const FwdArgs& a, const ScanArgs& s, int D, int DF, int fmap, int dtype, bool causal,
                            bool decay, hipStream_t st, hipEvent_t* ev);
hipError_t scan_dispatch(const ScanArgs& s, hipStream_t st);
// random features with the projection fused into the chunked passes (bf16):
// state pass, carry scan, then the output pass (causal, d = 64, m in
// {64, 128, 256}) or the read-out against the total (non-causal, every
// supported (d, m) pair)
bool perf_fused_supported(int D, int DF, int dtype, bool causal, bool decay);
hipError_t perf_fused_dispatch(const FwdArgs& a, const ScanArgs& s, int D, int DF, bool causal, hipStream_t st,
                               hipEvent_t* ev);
hipError_t backward_dispatch(const FwdArgs& fa, const ScanArgs& fs, const BwdArgs& b, const ScanArgs& rs, int D,
                             int fmap, int dtype, bool decay, hipStream_t st);
hipError_t gated_dispatch(const GatedArgs& g, const ScanArgs& s, int D, int fmap, int dtype, hipStream_t st);
hipError_t decode_dispatch(const DecodeArgs& a, int D, int DF, int fmap, int dtype, hipStream_t st);
int poly_partials(int D);
int poly_den_slots(int D);
hipError_t poly_forward_dispatch(const PolyArgs& a, int D, int dtype, bool causal, hipStream_t st);
hipError_t poly_decode_dispatch(const DecodeArgs& a, int D, int dtype, hipStream_t st);
hipError_t poly_fmap_dispatch(const FmapArgs& a, int D, int in_dtype, int out_dtype, hipStream_t st);
hipError_t fmap_dispatch(const FmapArgs& a, int D, int DF, int fmap, int in_dtype, int out_dtype, hipStream_t st);
hipError_t copy_state_dispatch(const float* S_in, const float* z_in, float* S_out, float* z_out, long long nS,
                               long long nz, hipStream_t st);

}  // namespace la

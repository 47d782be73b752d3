// gdn_internal.h -- parameter blocks and launcher entry points between the
// host-side C ABI (gdn_api.cpp) and the HIP kernels.  Everything here has
// already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

struct PrepareParams {
  int Hk, Hv, Dk, Dv, K;
  int Cc;
  int N;
  int64_t T;
  const int32_t* cu;      // device [N+1]
  const void* x;          // [T, x_stride] act
  int64_t x_stride;
  const void* a;          // [T, a_stride] act
  int64_t a_stride;
  const void* b;          // [T, b_stride] act
  int64_t b_stride;
  const void* w;          // [Cc, K] act
  const float* A_log;     // [Hv]
  const float* dt_bias;   // [Hv]
  void* conv_pool;        // [S, Cc, W] act; the leading K-1 taps are used
  int W;                  // taps per conv-history row
  int num_slots;
  const int32_t* slots;   // device [N] or null (slot = s)
  const uint8_t* has_init;  // device [N] or null (all 1)
  int l2norm;
  void* q;                // [T, Hk, Dk] qkv
  void* k;                // [T, Hk, Dk] qkv
  void* v;                // [T, Hv, Dv] qkv
  float* g;               // [T, Hv]
  float* beta;            // [T, Hv]
  gdn_dtype act, qkv;
  const int32_t* cu_host;  // host [N+1]: read by the launcher only
};

struct DecodeParams {
  int Hk, Hv, Dk, Dv, K;
  int Cc;
  int B;
  const void* x;
  int64_t x_stride;
  const void* a;
  int64_t a_stride;
  const void* b;
  int64_t b_stride;
  const void* w;
  const float* A_log;
  const float* dt_bias;
  void* conv_pool;        // [S, Cc, W] act; the leading K-1 taps are used
  int W;                  // taps per conv-history row
  void* ssm_pool;         // [S, Hv, Dv, Dk] state
  int num_slots;
  const int32_t* slots;   // device [B]
  float scale;
  void* out;              // [B, Hv, Dv] act
  gdn_dtype act, state;
  // fused output epilogue (gated RMS norm), when gated is set
  int gated;
  const void* gz;         // gate, row b head h at gz[b * gz_stride + h * Dv + j], act
  int64_t gz_stride;
  const void* gw;         // [Dv] act
  float geps;
  int gsig;               // logistic gate instead of silu
};

struct SpecDecodeParams {
  int Hk, Hv, Dk, Dv, K;
  int Cc;
  int N;                  // requests
  int cols;               // slot columns per request (1..8)
  int W;                  // taps per conv-history row, >= (K-1) + (cols-1)
  int64_t T;
  const int32_t* cu;      // device [N+1]
  const void* x;          // [T, x_stride] act
  int64_t x_stride;
  const void* a;
  int64_t a_stride;
  const void* b;
  int64_t b_stride;
  const void* w;          // [Cc, K] act
  const float* A_log;
  const float* dt_bias;
  void* conv_pool;        // [S, Cc, W] act
  void* ssm_pool;         // [S, Hv, Dv, Dk] state
  int num_slots;
  const int32_t* state_idx;     // device [N, cols]
  const int32_t* num_accepted;  // device [N]
  float scale;
  void* out;              // [T, Hv, Dv] act
  gdn_dtype act, state;
};

struct GatedNormParams {
  int T, H, D;
  const void* x;          // [T, H, D] io
  const void* z;          // token t head h at z[t * z_stride + h * D + j], io
  int64_t z_stride;
  const void* w;          // [D] io
  float eps;
  int sig;
  void* out;              // [T, H, D] io
  gdn_dtype io;
};

struct PrefillParams {
  int Hk, Hv, Dk, Dv;
  int N;
  int64_t T;
  const int32_t* cu;      // device [N+1]
  const void* q;          // [T, Hk, Dk] qkv
  const void* k;
  const void* v;          // [T, Hv, Dv] qkv
  const float* g;         // [T, Hv]
  const float* beta;      // [T, Hv]
  void* ssm_pool;         // [S, Hv, Dv, Dk] state
  int num_slots;
  const int32_t* slots;   // device [N] or null
  const uint8_t* has_init;  // device [N] or null
  float scale;
  int l2norm;
  int chunk;
  void* out;              // [T, Hv, Dv] qkv
  void* workspace;
  size_t workspace_bytes;
  int64_t num_chunks;     // sum over sequences of ceil(L / chunk)
  int max_chunks_per_seq;
  gdn_dtype qkv, state;
  // value heads h0 .. h0+hg-1 run in this launch; the workspace holds blocks
  // for those heads only ([chunk][hg]); h0 = 0, hg = Hv for the whole layer
  int h0, hg;
};

struct KdaParams {
  int Hk, Hv, Dk, Dv;
  int N;
  int64_t T;
  const int32_t* cu;      // device [N+1]
  const void* q;          // [T, Hk, Dk] qkv
  const void* k;
  const void* v;          // [T, Hv, Dv] qkv
  const float* g;         // [T, Hv, Dk]: log-decay, or the gate's input when A_log is set
  const float* A_log;     // [Hv] or null
  const float* dt_bias;   // [Hv, Dk] or null
  const float* beta;      // [T, Hv]
  void* ssm_pool;         // [S, Hv, Dv, Dk] state
  int num_slots;
  const int32_t* slots;   // device [N] or null
  const uint8_t* has_init;  // device [N] or null
  float scale;
  int l2norm;
  void* out;              // [T, Hv, Dv] qkv
  gdn_dtype qkv, state;
  // chunked form only
  void* workspace;
  size_t workspace_bytes;
  int64_t num_chunks;     // sum over sequences of ceil(L / 64)
  int max_chunks_per_seq;
};

struct Mamba2Params {
  int H, P, G, N;
  int Nseq;               // sequences (prefill) or rows (decode)
  int64_t T;
  const int32_t* cu;      // device [Nseq+1] (prefill)
  const void* x;          // [T, H, P] act
  const void* dt;         // [T, H] act (raw)
  const void* B;          // [T, G, N] act
  const void* C;          // [T, G, N] act
  const void* z;          // [T, H, P] act or null
  const float* A;         // [H]
  const float* dt_bias;   // [H] or null
  const float* D;         // [H] or [H, P] or null
  int D_per_p;
  int dt_softplus;
  float dt_min, dt_max;
  void* ssm_pool;         // [S, H, P, N] state
  int num_slots;
  const int32_t* slots;   // device [Nseq] (decode: required; prefill: or null)
  const uint8_t* has_init;  // device [Nseq] or null (prefill)
  void* out;              // [T, H, P] act
  gdn_dtype act, state;
  void* workspace;        // prefill
  size_t workspace_bytes;
  int64_t num_chunks;
};

// Each launcher enqueues its kernels on `stream` and returns the HIP status
// of the launch.
hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_decode_spec(const SpecDecodeParams& p, hipStream_t stream);
size_t decode_spec_lds_bytes(int Hk, int Hv, int Dk, int Dv, int cols);
hipError_t launch_gated_rmsnorm(const GatedNormParams& p, hipStream_t stream);
hipError_t launch_kda_recurrent(const KdaParams& p, hipStream_t stream);
hipError_t launch_kda_prefill(const KdaParams& p, hipStream_t stream);
size_t kda_prefill_workspace_bytes(int Hv, int Dk, int Dv, int N, int64_t T, gdn_dtype qkv);
bool kda_chunked_dims(int Dk, int Dv);
hipError_t launch_mamba2_update(const Mamba2Params& p, hipStream_t stream);
hipError_t launch_mamba2_chunk_scan(const Mamba2Params& p, hipStream_t stream);
size_t mamba2_workspace_bytes(int H, int P, int N, int Ns, int64_t T);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
size_t prefill_workspace_bytes(int Hk, int Hv, int Dk, int Dv, int N, int64_t T, int chunk);
// Scratch bytes the chunked prefill needs for ONE value head (0 when the
// shape runs the token-sequential kernel, which needs none).
size_t prefill_workspace_bytes_per_head(int Dk, int Dv, int N, int64_t T);
// The prefill on the library's static scratch (no allocation), value heads in
// groups that fit it; p.workspace is ignored.  The caller has checked that
// one head fits (prefill_workspace_bytes_per_head <= kNoAllocScratchBytes).
hipError_t launch_prefill_noalloc(const PrefillParams& p, hipStream_t stream);
constexpr size_t kNoAllocScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;

}  // namespace gdn

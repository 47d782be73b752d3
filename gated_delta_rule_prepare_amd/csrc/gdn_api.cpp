// gdn_api.cpp -- the C ABI: argument checks on the host, then launches.
//
// The checks follow the pages' contracts: positive dims and Hv divisible by
// Hk ([P3] validate_gated_delta_rule_shape), offsets that start at 0, end at
// T and give every sequence at least one token ([P3]
// recurrent_gated_delta_rule_varlen_f32; [P2] ValidateGdnAttentionMetadata),
// slot indices in range, unique among live rows, -1 the only negative value
// and allowed for decode rows only ([P2] ValidateGdnStateIndices), and the
// dtype sets the layer uses ([P2] GdnPackedDecodeDTypesCompatible,
// ResolveMambaSsmCacheDType).  [P1] = vllm.cpp cpu_ops.cpp, [P2] = vllm.cpp
// qwen3_5.cpp, [P3] = ferrum-kernels cpu.rs.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status ok() {
  g_last_error[0] = '\0';
  return GDN_OK;
}

bool pow2_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

size_t dtype_size(gdn_dtype t) { return t == GDN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdn_status check_dims(const char* fn, const gdn_dims* d) {
  if (d == nullptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dims is null", fn);
  if (d->num_k_heads <= 0 || d->num_v_heads <= 0 || d->head_k_dim <= 0 || d->head_v_dim <= 0 ||
      d->conv_kernel <= 0)
    return fail(GDN_ERR_SHAPE,
                "%s: dims must be positive, got Hk=%d Hv=%d Dk=%d Dv=%d K=%d", fn, d->num_k_heads,
                d->num_v_heads, d->head_k_dim, d->head_v_dim, d->conv_kernel);
  if (d->num_v_heads % d->num_k_heads != 0)
    return fail(GDN_ERR_SHAPE, "%s: value heads %d must be a multiple of key heads %d", fn,
                d->num_v_heads, d->num_k_heads);
  if (!pow2_head_dim(d->head_k_dim) || !pow2_head_dim(d->head_v_dim))
    return fail(GDN_ERR_SHAPE, "%s: head dims must be 16, 32, 64, 128 or 256, got Dk=%d Dv=%d", fn,
                d->head_k_dim, d->head_v_dim);
  if (d->conv_kernel > 4)
    return fail(GDN_ERR_SHAPE, "%s: conv_kernel must be 1..4, got %d", fn, d->conv_kernel);
  const int64_t cc = 2LL * d->num_k_heads * d->head_k_dim + (int64_t)d->num_v_heads * d->head_v_dim;
  if (cc > (1LL << 30)) return fail(GDN_ERR_SHAPE, "%s: too many channels", fn);
  if (d->conv_state_len != 0 && (d->conv_state_len < d->conv_kernel - 1 || d->conv_state_len > 1024))
    return fail(GDN_ERR_SHAPE, "%s: conv_state_len must be 0 or in [K-1, 1024], got %d (K=%d)", fn,
                d->conv_state_len, d->conv_kernel);
  return GDN_OK;
}

// Taps per conv-history row: dims.conv_state_len, 0 meaning K-1.
int conv_row_len(const gdn_dims* d) { return d->conv_state_len ? d->conv_state_len : d->conv_kernel - 1; }

int conv_channels(const gdn_dims* d) {
  return 2 * d->num_k_heads * d->head_k_dim + d->num_v_heads * d->head_v_dim;
}

// Offsets: cu[0] = 0, strictly increasing (no empty sequence), cu[N] = T.
gdn_status check_offsets(const char* fn, int32_t n, int64_t t, const int32_t* cu_host,
                         const int32_t* cu_dev) {
  if (n < 0 || t < 0) return fail(GDN_ERR_SHAPE, "%s: negative sizes N=%d T=%lld", fn, n, (long long)t);
  if (n == 0 || t == 0) {
    if (n != 0 || t != 0)
      return fail(GDN_ERR_SHAPE, "%s: N=%d sequences but T=%lld tokens", fn, n, (long long)t);
    return GDN_OK;
  }
  if (t > INT32_MAX) return fail(GDN_ERR_SHAPE, "%s: T=%lld exceeds int32 offsets", fn, (long long)t);
  if (cu_host == nullptr || cu_dev == nullptr)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens host and device pointers are required", fn);
  if (cu_host[0] != 0 || cu_host[n] != t)
    return fail(GDN_ERR_SHAPE, "%s: cu_seqlens must start at 0 and end at T=%lld, got %d and %d", fn,
                (long long)t, cu_host[0], cu_host[n]);
  for (int32_t s = 0; s < n; ++s)
    if (cu_host[s + 1] <= cu_host[s])
      return fail(GDN_ERR_SHAPE, "%s: sequence %d is empty or offsets decrease (%d..%d)", fn, s,
                  cu_host[s], cu_host[s + 1]);
  return GDN_OK;
}

// Offsets that may repeat (empty sequences): cu[0] = 0, non-decreasing, cu[N] = T.
gdn_status check_offsets_nondecreasing(const char* fn, int32_t n, int64_t t, const int32_t* cu_host,
                                       const int32_t* cu_dev) {
  if (n < 0 || t < 0) return fail(GDN_ERR_SHAPE, "%s: negative sizes N=%d T=%lld", fn, n, (long long)t);
  if (n == 0) {
    if (t != 0) return fail(GDN_ERR_SHAPE, "%s: N=0 sequences but T=%lld tokens", fn, (long long)t);
    return GDN_OK;
  }
  if (t > INT32_MAX) return fail(GDN_ERR_SHAPE, "%s: T=%lld exceeds int32 offsets", fn, (long long)t);
  if (cu_host == nullptr || cu_dev == nullptr)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens host and device pointers are required", fn);
  if (cu_host[0] != 0 || cu_host[n] != t)
    return fail(GDN_ERR_SHAPE, "%s: cu_seqlens must start at 0 and end at T=%lld, got %d and %d", fn,
                (long long)t, cu_host[0], cu_host[n]);
  for (int32_t s = 0; s < n; ++s)
    if (cu_host[s + 1] < cu_host[s])
      return fail(GDN_ERR_SHAPE, "%s: offsets decrease at sequence %d (%d..%d)", fn, s, cu_host[s], cu_host[s + 1]);
  return GDN_OK;
}

// Slots: live slot in [0, num_slots), unique; -1 allowed only if allow_null.
gdn_status check_slots(const char* fn, const int32_t* idx, int32_t n, int32_t num_slots, bool allow_null) {
  std::vector<uint8_t> seen((size_t)(num_slots > 0 ? num_slots : 0), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = idx[i];
    if (s < 0) {
      if (s == -1 && allow_null) continue;
      return fail(GDN_ERR_INDEX, "%s: row %d has slot %d (%s)", fn, i, s,
                  allow_null ? "only -1 may be negative" : "sequences need a live slot");
    }
    if (s >= num_slots)
      return fail(GDN_ERR_INDEX, "%s: row %d slot %d out of range [0, %d)", fn, i, s, num_slots);
    if (seen[(size_t)s]) return fail(GDN_ERR_INDEX, "%s: slot %d used by more than one row", fn, s);
    seen[(size_t)s] = 1;
  }
  return GDN_OK;
}

gdn_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(GDN_ERR_DEVICE, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GDN_ERR_SHAPE: return "shape mismatch";
    case GDN_ERR_INDEX: return "bad slot index";
    case GDN_ERR_DTYPE: return "unsupported dtype";
    case GDN_ERR_WORKSPACE: return "workspace too small";
    case GDN_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* gdn_last_error(void) { return g_last_error; }

int32_t gdn_version(void) { return 140; }

gdn_status gdn_prepare(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                       const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                       const void* mixed_qkv, int64_t mixed_row_stride, const void* a_raw,
                       int64_t a_row_stride, const void* b_raw, int64_t b_row_stride,
                       gdn_dtype act_dtype, const void* conv_weight, const float* A_log,
                       const float* dt_bias, void* conv_state_pool, int32_t num_slots,
                       const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                       const uint8_t* has_initial_state_dev, int32_t apply_qk_l2norm,
                       void* q_out, void* k_out, void* v_out, gdn_dtype qkv_dtype,
                       float* g_out, float* beta_out, void* stream) {
  const char* fn = "gdn_prepare";
  gdn_status st = check_dims(fn, dims);
  if (st != GDN_OK) return st;
  st = check_offsets(fn, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev);
  if (st != GDN_OK) return st;
  if (num_seqs == 0) return ok();
  if (act_dtype != GDN_F32 && act_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: activations must be f32 or bf16", fn);
  if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: q/k/v outputs must be f32 or bf16", fn);
  const int cc = conv_channels(dims);
  const int K = dims->conv_kernel;
  if (!mixed_qkv || !a_raw || !b_raw || !conv_weight || !A_log || !dt_bias || !q_out || !k_out ||
      !v_out || !g_out || !beta_out || (K > 1 && !conv_state_pool))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
  if (mixed_row_stride < cc || a_row_stride < dims->num_v_heads || b_row_stride < dims->num_v_heads)
    return fail(GDN_ERR_SHAPE, "%s: row strides (%lld, %lld, %lld) below widths (%d, %d)", fn,
                (long long)mixed_row_stride, (long long)a_row_stride, (long long)b_row_stride, cc,
                dims->num_v_heads);
  if (!aligned16(mixed_qkv) || (mixed_row_stride * (int64_t)dtype_size(act_dtype)) % 16 != 0 ||
      !aligned16(q_out) || !aligned16(k_out) || !aligned16(v_out))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: mixed_qkv rows and q/k/v outputs must be 16-byte aligned", fn);
  if (!aligned16(conv_weight) || (K > 1 && !aligned16(conv_state_pool)))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: the conv weight and conv-history pool must be 16-byte aligned", fn);
  if ((slot_idx_host == nullptr) != (slot_idx_dev == nullptr))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: pass both slot index copies or neither", fn);
  if (K > 1) {
    if (num_slots <= 0) return fail(GDN_ERR_SHAPE, "%s: num_slots must be positive", fn);
    if (slot_idx_host) {
      st = check_slots(fn, slot_idx_host, num_seqs, num_slots, false);
      if (st != GDN_OK) return st;
    } else if (num_seqs > num_slots) {
      return fail(GDN_ERR_INDEX, "%s: %d sequences but only %d slots", fn, num_seqs, num_slots);
    }
  }
  if (apply_qk_l2norm != 0 && apply_qk_l2norm != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: apply_qk_l2norm must be 0 or 1", fn);

  gdn::PrepareParams p{};
  p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads; p.Dk = dims->head_k_dim; p.Dv = dims->head_v_dim;
  p.K = K; p.Cc = cc; p.N = num_seqs; p.T = total_tokens; p.cu = cu_seqlens_dev;
  p.x = mixed_qkv; p.x_stride = mixed_row_stride; p.a = a_raw; p.a_stride = a_row_stride;
  p.b = b_raw; p.b_stride = b_row_stride; p.w = conv_weight; p.A_log = A_log; p.dt_bias = dt_bias;
  p.conv_pool = conv_state_pool; p.W = conv_row_len(dims); p.num_slots = num_slots; p.slots = slot_idx_dev;
  p.has_init = has_initial_state_dev; p.l2norm = apply_qk_l2norm; p.q = q_out; p.k = k_out; p.v = v_out;
  p.g = g_out; p.beta = beta_out; p.act = act_dtype; p.qkv = qkv_dtype; p.cu_host = cu_seqlens_host;
  return launched(fn, gdn::launch_prepare(p, static_cast<hipStream_t>(stream)));
}

namespace {

struct GateArgs {
  const void* z;
  int64_t z_row_stride;
  const void* weight;
  float eps;
  int32_t sigmoid_gate;
};

bool good_eps(float eps) { return eps == eps && eps >= 0.0f && eps <= 3.0e38f; }

gdn_status decode_common(const char* fn, const gdn_dims* dims, int32_t batch, const void* mixed_qkv,
                         int64_t mixed_row_stride, const void* a_raw, int64_t a_row_stride,
                         const void* b_raw, int64_t b_row_stride, gdn_dtype act_dtype,
                         const void* conv_weight, const float* A_log, const float* dt_bias,
                         void* conv_state_pool, void* ssm_state_pool, gdn_dtype state_dtype,
                         int32_t num_slots, const int32_t* slot_idx_dev, const int32_t* slot_idx_host,
                         float scale, const GateArgs* gate, void* out, void* stream) {
  gdn_status st = check_dims(fn, dims);
  if (st != GDN_OK) return st;
  if (batch < 0) return fail(GDN_ERR_SHAPE, "%s: negative batch %d", fn, batch);
  if (batch == 0) return ok();
  if (act_dtype != GDN_F32 && act_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: activations must be f32 or bf16", fn);
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16 && state_dtype != GDN_F16)
    return fail(GDN_ERR_DTYPE, "%s: state must be f32, bf16 or f16", fn);
  const int cc = conv_channels(dims);
  const int K = dims->conv_kernel;
  if (!mixed_qkv || !a_raw || !b_raw || !conv_weight || !A_log || !dt_bias || !ssm_state_pool ||
      !slot_idx_dev || !out || (K > 1 && !conv_state_pool))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
  if (mixed_row_stride < cc || a_row_stride < dims->num_v_heads || b_row_stride < dims->num_v_heads)
    return fail(GDN_ERR_SHAPE, "%s: row strides below widths", fn);
  if (!aligned16(ssm_state_pool))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: the state pool must be 16-byte aligned", fn);
  if ((int64_t)(dims->num_v_heads / dims->num_k_heads) * dims->head_v_dim > 8192)
    return fail(GDN_ERR_SHAPE, "%s: (Hv/Hk)*Dv must be at most 8192", fn);
  if (num_slots <= 0) return fail(GDN_ERR_SHAPE, "%s: num_slots must be positive", fn);
  if (slot_idx_host) {
    st = check_slots(fn, slot_idx_host, batch, num_slots, true);
    if (st != GDN_OK) return st;
  }
  if (!(scale == scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: scale is NaN", fn);
  if (gate) {
    if (!gate->z || !gate->weight) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
    if (gate->z_row_stride < (int64_t)dims->num_v_heads * dims->head_v_dim)
      return fail(GDN_ERR_SHAPE, "%s: z_row_stride %lld below Hv*Dv", fn, (long long)gate->z_row_stride);
    if (!good_eps(gate->eps)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
    if (gate->sigmoid_gate != 0 && gate->sigmoid_gate != 1)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: sigmoid_gate must be 0 or 1", fn);
  }

  gdn::DecodeParams p{};
  p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads; p.Dk = dims->head_k_dim; p.Dv = dims->head_v_dim;
  p.K = K; p.Cc = cc; p.B = batch; p.x = mixed_qkv; p.x_stride = mixed_row_stride; p.a = a_raw;
  p.a_stride = a_row_stride; p.b = b_raw; p.b_stride = b_row_stride; p.w = conv_weight; p.A_log = A_log;
  p.dt_bias = dt_bias; p.conv_pool = conv_state_pool; p.W = conv_row_len(dims); p.ssm_pool = ssm_state_pool;
  p.num_slots = num_slots;
  p.slots = slot_idx_dev; p.scale = scale; p.out = out; p.act = act_dtype; p.state = state_dtype;
  if (gate) {
    p.gated = 1; p.gz = gate->z; p.gz_stride = gate->z_row_stride; p.gw = gate->weight; p.geps = gate->eps;
    p.gsig = gate->sigmoid_gate;
  }
  return launched(fn, gdn::launch_decode(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

gdn_status gdn_decode(const gdn_dims* dims, int32_t batch, const void* mixed_qkv,
                      int64_t mixed_row_stride, const void* a_raw, int64_t a_row_stride,
                      const void* b_raw, int64_t b_row_stride, gdn_dtype act_dtype,
                      const void* conv_weight, const float* A_log, const float* dt_bias,
                      void* conv_state_pool, void* ssm_state_pool, gdn_dtype state_dtype,
                      int32_t num_slots, const int32_t* slot_idx_dev,
                      const int32_t* slot_idx_host, float scale, void* out, void* stream) {
  return decode_common("gdn_decode", dims, batch, mixed_qkv, mixed_row_stride, a_raw, a_row_stride, b_raw,
                       b_row_stride, act_dtype, conv_weight, A_log, dt_bias, conv_state_pool, ssm_state_pool,
                       state_dtype, num_slots, slot_idx_dev, slot_idx_host, scale, nullptr, out, stream);
}

gdn_status gdn_decode_gated(const gdn_dims* dims, int32_t batch, const void* mixed_qkv,
                            int64_t mixed_row_stride, const void* a_raw, int64_t a_row_stride,
                            const void* b_raw, int64_t b_row_stride, gdn_dtype act_dtype,
                            const void* conv_weight, const float* A_log, const float* dt_bias,
                            void* conv_state_pool, void* ssm_state_pool, gdn_dtype state_dtype,
                            int32_t num_slots, const int32_t* slot_idx_dev,
                            const int32_t* slot_idx_host, float scale, const void* z,
                            int64_t z_row_stride, const void* norm_weight, float eps,
                            int32_t sigmoid_gate, void* out, void* stream) {
  const GateArgs gate{z, z_row_stride, norm_weight, eps, sigmoid_gate};
  return decode_common("gdn_decode_gated", dims, batch, mixed_qkv, mixed_row_stride, a_raw, a_row_stride,
                       b_raw, b_row_stride, act_dtype, conv_weight, A_log, dt_bias, conv_state_pool,
                       ssm_state_pool, state_dtype, num_slots, slot_idx_dev, slot_idx_host, scale, &gate, out,
                       stream);
}

gdn_status gdn_decode_spec(const gdn_dims* dims, int32_t num_reqs, int64_t total_tokens,
                           const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                           const void* mixed_qkv, int64_t mixed_row_stride, const void* a_raw,
                           int64_t a_row_stride, const void* b_raw, int64_t b_row_stride,
                           gdn_dtype act_dtype, const void* conv_weight, const float* A_log,
                           const float* dt_bias, void* conv_state_pool, void* ssm_state_pool,
                           gdn_dtype state_dtype, int32_t num_slots, int32_t num_cols,
                           const int32_t* state_idx_dev, const int32_t* num_accepted_dev,
                           const int32_t* state_idx_host, const int32_t* num_accepted_host,
                           float scale, void* out, void* stream) {
  const char* fn = "gdn_decode_spec";
  gdn_status st = check_dims(fn, dims);
  if (st != GDN_OK) return st;
  st = check_offsets(fn, num_reqs, total_tokens, cu_seqlens_host, cu_seqlens_dev);
  if (st != GDN_OK) return st;
  if (num_reqs == 0) return ok();
  if (act_dtype != GDN_F32 && act_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: activations must be f32 or bf16", fn);
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16 && state_dtype != GDN_F16)
    return fail(GDN_ERR_DTYPE, "%s: state must be f32, bf16 or f16", fn);
  const int K = dims->conv_kernel;
  if (K < 2) return fail(GDN_ERR_SHAPE, "%s: speculative decode needs conv_kernel >= 2, got %d", fn, K);
  if (num_cols < 1 || num_cols > 8)
    return fail(GDN_ERR_SHAPE, "%s: num_cols must be in [1, 8], got %d", fn, num_cols);
  const int W = conv_row_len(dims);
  if (W < (K - 1) + (num_cols - 1))
    return fail(GDN_ERR_SHAPE, "%s: conv rows of %d taps are narrower than (K-1)+(num_cols-1) = %d", fn, W,
                (K - 1) + (num_cols - 1));
  for (int32_t i = 0; i < num_reqs; ++i)
    if (cu_seqlens_host[i + 1] - cu_seqlens_host[i] > num_cols)
      return fail(GDN_ERR_SHAPE, "%s: request %d has %d tokens, more than num_cols=%d", fn, i,
                  cu_seqlens_host[i + 1] - cu_seqlens_host[i], num_cols);
  const int cc = conv_channels(dims);
  if (!mixed_qkv || !a_raw || !b_raw || !conv_weight || !A_log || !dt_bias || !conv_state_pool ||
      !ssm_state_pool || !state_idx_dev || !num_accepted_dev || !out)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
  if (mixed_row_stride < cc || a_row_stride < dims->num_v_heads || b_row_stride < dims->num_v_heads)
    return fail(GDN_ERR_SHAPE, "%s: row strides below widths", fn);
  if (!aligned16(ssm_state_pool))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: the state pool must be 16-byte aligned", fn);
  if (gdn::decode_spec_lds_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_k_dim, dims->head_v_dim,
                                 num_cols) > 64 * 1024)
    return fail(GDN_ERR_SHAPE, "%s: num_cols * (2*Dk + 2*(Hv/Hk)*Dv) too large for one workgroup", fn);
  if (num_slots <= 0) return fail(GDN_ERR_SHAPE, "%s: num_slots must be positive", fn);
  if ((state_idx_host == nullptr) != (num_accepted_host == nullptr))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: pass both index host copies or neither", fn);
  if (state_idx_host) {
    std::vector<uint8_t> seen((size_t)num_slots, 0);
    for (int32_t i = 0; i < num_reqs; ++i) {
      const int32_t acc = num_accepted_host[i];
      if (acc < 1 || acc > num_cols)
        return fail(GDN_ERR_INDEX, "%s: request %d num_accepted %d not in [1, %d]", fn, i, acc, num_cols);
      const int32_t* row = state_idx_host + (int64_t)i * num_cols;
      const bool live = row[acc - 1] >= 0;
      if (live && row[0] < 0)
        return fail(GDN_ERR_INDEX, "%s: request %d is live but its conv slot (column 0) is -1", fn, i);
      for (int32_t c = 0; c < num_cols; ++c) {
        const int32_t s = row[c];
        if (s < -1 || s >= num_slots)
          return fail(GDN_ERR_INDEX, "%s: request %d column %d slot %d out of range [0, %d)", fn, i, c, s, num_slots);
        if (s < 0) continue;
        if (seen[(size_t)s]) return fail(GDN_ERR_INDEX, "%s: slot %d appears more than once", fn, s);
        seen[(size_t)s] = 1;
      }
    }
  }
  if (!(scale == scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: scale is NaN", fn);

  gdn::SpecDecodeParams p{};
  p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads; p.Dk = dims->head_k_dim; p.Dv = dims->head_v_dim;
  p.K = K; p.Cc = cc; p.N = num_reqs; p.cols = num_cols; p.W = W; p.T = total_tokens; p.cu = cu_seqlens_dev;
  p.x = mixed_qkv; p.x_stride = mixed_row_stride; p.a = a_raw; p.a_stride = a_row_stride; p.b = b_raw;
  p.b_stride = b_row_stride; p.w = conv_weight; p.A_log = A_log; p.dt_bias = dt_bias;
  p.conv_pool = conv_state_pool; p.ssm_pool = ssm_state_pool; p.num_slots = num_slots;
  p.state_idx = state_idx_dev; p.num_accepted = num_accepted_dev; p.scale = scale; p.out = out;
  p.act = act_dtype; p.state = state_dtype;
  return launched(fn, gdn::launch_decode_spec(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_gated_rmsnorm(int32_t num_tokens, int32_t num_heads, int32_t head_dim, const void* x,
                             const void* z, int64_t z_row_stride, const void* weight, float eps,
                             int32_t sigmoid_gate, void* out, gdn_dtype io_dtype, void* stream) {
  const char* fn = "gdn_gated_rmsnorm";
  if (num_tokens < 0 || num_heads <= 0)
    return fail(GDN_ERR_SHAPE, "%s: bad sizes T=%d Hv=%d", fn, num_tokens, num_heads);
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(GDN_ERR_SHAPE, "%s: head_dim must be 16, 32, 64, 128 or 256, got %d", fn, head_dim);
  if (io_dtype != GDN_F32 && io_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "%s: io dtype must be f32 or bf16", fn);
  if (num_tokens == 0) return ok();
  if (!x || !z || !weight || !out) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
  if (z_row_stride < (int64_t)num_heads * head_dim)
    return fail(GDN_ERR_SHAPE, "%s: z_row_stride %lld below Hv*Dv", fn, (long long)z_row_stride);
  if (!aligned16(x) || !aligned16(z) || !aligned16(weight) || !aligned16(out) ||
      (z_row_stride * (int64_t)dtype_size(io_dtype)) % 16 != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, z rows, weight and out must be 16-byte aligned", fn);
  if (!good_eps(eps)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
  if (sigmoid_gate != 0 && sigmoid_gate != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: sigmoid_gate must be 0 or 1", fn);
  gdn::GatedNormParams p{};
  p.T = num_tokens; p.H = num_heads; p.D = head_dim; p.x = x; p.z = z; p.z_stride = z_row_stride; p.w = weight;
  p.eps = eps; p.sig = sigmoid_gate; p.out = out; p.io = io_dtype;
  return launched(fn, gdn::launch_gated_rmsnorm(p, static_cast<hipStream_t>(stream)));
}


namespace {

// Checks shared by the KDA entry points; fills p on success.
gdn_status kda_common(const char* fn, const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                      const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* q, const void* k,
                      const void* v, gdn_dtype qkv_dtype, const float* g, const float* A_log, const float* dt_bias,
                      const float* beta, void* ssm_state_pool, gdn_dtype state_dtype, int32_t num_slots,
                      const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                      const uint8_t* has_initial_state_dev, float scale, int32_t use_qk_l2norm, void* out,
                      gdn::KdaParams& p) {
  gdn_status st = check_dims(fn, dims);
  if (st != GDN_OK) return st;
  st = check_offsets_nondecreasing(fn, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev);
  if (st != GDN_OK) return st;
  if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: q/k/v must be f32 or bf16", fn);
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16 && state_dtype != GDN_F16)
    return fail(GDN_ERR_DTYPE, "%s: state must be f32, bf16 or f16", fn);
  if (num_seqs > 0) {
    if (!ssm_state_pool || (total_tokens > 0 && (!q || !k || !v || !g || !beta || !out)))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ssm_state_pool) ||
        !aligned16(g) || !aligned16(dt_bias))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q/k/v/out/state/g/dt_bias must be 16-byte aligned", fn);
    if (dt_bias && !A_log)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dt_bias is only used with A_log", fn);
    if ((slot_idx_host == nullptr) != (slot_idx_dev == nullptr))
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: pass both slot index copies or neither", fn);
    if (num_slots <= 0) return fail(GDN_ERR_SHAPE, "%s: num_slots must be positive", fn);
    if (slot_idx_host) {
      st = check_slots(fn, slot_idx_host, num_seqs, num_slots, false);
      if (st != GDN_OK) return st;
    } else if (num_seqs > num_slots) {
      return fail(GDN_ERR_INDEX, "%s: %d sequences but only %d slots", fn, num_seqs, num_slots);
    }
  }
  if (use_qk_l2norm != 0 && use_qk_l2norm != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: use_qk_l2norm must be 0 or 1", fn);
  if (!(scale == scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: scale is NaN", fn);
  p = gdn::KdaParams{};
  p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads; p.Dk = dims->head_k_dim; p.Dv = dims->head_v_dim;
  p.N = num_seqs; p.T = total_tokens; p.cu = cu_seqlens_dev; p.q = q; p.k = k; p.v = v; p.g = g;
  p.A_log = A_log; p.dt_bias = dt_bias; p.beta = beta; p.ssm_pool = ssm_state_pool; p.num_slots = num_slots;
  p.slots = slot_idx_dev; p.has_init = has_initial_state_dev; p.scale = scale; p.l2norm = use_qk_l2norm;
  p.out = out; p.qkv = qkv_dtype; p.state = state_dtype;
  return GDN_OK;
}

}  // namespace

gdn_status gdn_kda_recurrent(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                             const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* q,
                             const void* k, const void* v, gdn_dtype qkv_dtype, const float* g,
                             const float* A_log, const float* dt_bias, const float* beta, void* ssm_state_pool,
                             gdn_dtype state_dtype, int32_t num_slots, const int32_t* slot_idx_host,
                             const int32_t* slot_idx_dev, const uint8_t* has_initial_state_dev, float scale,
                             int32_t use_qk_l2norm, void* out, void* stream) {
  const char* fn = "gdn_kda_recurrent";
  gdn::KdaParams p;
  const gdn_status st = kda_common(fn, dims, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev, q, k, v,
                                   qkv_dtype, g, A_log, dt_bias, beta, ssm_state_pool, state_dtype, num_slots,
                                   slot_idx_host, slot_idx_dev, has_initial_state_dev, scale, use_qk_l2norm, out, p);
  if (st != GDN_OK) return st;
  if (num_seqs == 0) return ok();
  return launched(fn, gdn::launch_kda_recurrent(p, static_cast<hipStream_t>(stream)));
}

size_t gdn_kda_prefill_workspace_size(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                      int32_t chunk_size, gdn_dtype qkv_dtype) {
  if (check_dims("gdn_kda_prefill_workspace_size", dims) != GDN_OK || num_seqs < 0 || total_tokens < 0) return 0;
  if (chunk_size == 0) chunk_size = 64;
  if (chunk_size != 64 || (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16)) return 0;
  return gdn::kda_prefill_workspace_bytes(dims->num_v_heads, dims->head_k_dim, dims->head_v_dim, num_seqs,
                                          total_tokens, qkv_dtype);
}

gdn_status gdn_kda_prefill_varlen(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                  const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* q,
                                  const void* k, const void* v, gdn_dtype qkv_dtype, const float* g,
                                  const float* A_log, const float* dt_bias, const float* beta, void* ssm_state_pool,
                                  gdn_dtype state_dtype, int32_t num_slots, const int32_t* slot_idx_host,
                                  const int32_t* slot_idx_dev, const uint8_t* has_initial_state_dev, float scale,
                                  int32_t use_qk_l2norm, int32_t chunk_size, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_kda_prefill_varlen";
  gdn::KdaParams p;
  gdn_status st = kda_common(fn, dims, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev, q, k, v, qkv_dtype,
                             g, A_log, dt_bias, beta, ssm_state_pool, state_dtype, num_slots, slot_idx_host,
                             slot_idx_dev, has_initial_state_dev, scale, use_qk_l2norm, out, p);
  if (st != GDN_OK) return st;
  if (chunk_size == 0) chunk_size = 64;
  if (chunk_size != 64) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: chunk_size must be 0 or 64", fn);
  if (num_seqs == 0) return ok();
  const size_t need = gdn::kda_prefill_workspace_bytes(dims->num_v_heads, dims->head_k_dim, dims->head_v_dim,
                                                       num_seqs, total_tokens, qkv_dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  int64_t nchunks = 0;
  int max_chunks = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int c = (cu_seqlens_host[s + 1] - cu_seqlens_host[s] + 63) / 64;
    nchunks += c;
    if (c > max_chunks) max_chunks = c;
  }
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.num_chunks = nchunks;
  p.max_chunks_per_seq = max_chunks;
  return launched(fn, gdn::launch_kda_prefill(p, static_cast<hipStream_t>(stream)));
}

namespace {

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

// Checks shared by the Mamba2 entry points; fills p's common fields.
gdn_status mamba2_common(const char* fn, const gdn_ssm_dims* d, const void* x, const void* dt, const float* A,
                         const void* B, const void* C, const float* D, int32_t D_per_head_dim, const void* z,
                         const gdn_ssm_dt* dtp, gdn_dtype act_dtype, void* state_pool, gdn_dtype state_dtype,
                         int32_t num_slots, void* out, bool any_tokens, gdn::Mamba2Params& p) {
  if (d == nullptr || dtp == nullptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: sdims or dtp is null", fn);
  if (d->num_heads <= 0 || d->head_dim <= 0 || d->num_groups <= 0 || d->num_heads % d->num_groups != 0)
    return fail(GDN_ERR_SHAPE, "%s: need H > 0, P > 0, G > 0 and H a multiple of G, got H=%d P=%d G=%d", fn,
                d->num_heads, d->head_dim, d->num_groups);
  if (!pow2_in(d->state_dim, 16, 256))
    return fail(GDN_ERR_SHAPE, "%s: state_dim must be 16, 32, 64, 128 or 256, got %d", fn, d->state_dim);
  if (act_dtype != GDN_F32 && act_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: activations must be f32 or bf16", fn);
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16 && state_dtype != GDN_F16)
    return fail(GDN_ERR_DTYPE, "%s: state must be f32, bf16 or f16", fn);
  if (!state_pool || !A || (any_tokens && (!x || !dt || !B || !C || !out)))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
  if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(z) || !aligned16(out) || !aligned16(state_pool))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, B, C, z, out and the pool must be 16-byte aligned", fn);
  if (D_per_head_dim != 0 && D_per_head_dim != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: D_per_head_dim must be 0 or 1", fn);
  if (dtp->softplus != 0 && dtp->softplus != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dt softplus flag must be 0 or 1", fn);
  if (!(dtp->dt_min >= 0.0f) || !(dtp->dt_max >= dtp->dt_min))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: need 0 <= dt_min <= dt_max, got %g and %g", fn, dtp->dt_min,
                dtp->dt_max);
  if (num_slots <= 0) return fail(GDN_ERR_SHAPE, "%s: num_slots must be positive", fn);
  p = gdn::Mamba2Params{};
  p.H = d->num_heads; p.P = d->head_dim; p.G = d->num_groups; p.N = d->state_dim;
  p.x = x; p.dt = dt; p.B = B; p.C = C; p.z = z; p.A = A; p.dt_bias = dtp->dt_bias; p.D = D;
  p.D_per_p = D_per_head_dim; p.dt_softplus = dtp->softplus; p.dt_min = dtp->dt_min; p.dt_max = dtp->dt_max;
  p.ssm_pool = state_pool; p.num_slots = num_slots; p.out = out; p.act = act_dtype; p.state = state_dtype;
  return GDN_OK;
}

bool mamba2_chunked_dims(const gdn_ssm_dims* d) {
  return (d->head_dim == 32 || d->head_dim == 64 || d->head_dim == 128) &&
         (d->state_dim == 32 || d->state_dim == 64 || d->state_dim == 128);
}

}  // namespace

gdn_status gdn_mamba2_state_update(const gdn_ssm_dims* sdims, int32_t batch, const void* x, const void* dt,
                                   const float* A, const void* B, const void* C, const float* D,
                                   int32_t D_per_head_dim, const void* z, const gdn_ssm_dt* dtp,
                                   gdn_dtype act_dtype, void* state_pool, gdn_dtype state_dtype,
                                   int32_t num_slots, const int32_t* slot_idx_dev, const int32_t* slot_idx_host,
                                   void* out, void* stream) {
  const char* fn = "gdn_mamba2_state_update";
  if (batch < 0) return fail(GDN_ERR_SHAPE, "%s: negative batch %d", fn, batch);
  gdn::Mamba2Params p;
  gdn_status st = mamba2_common(fn, sdims, x, dt, A, B, C, D, D_per_head_dim, z, dtp, act_dtype, state_pool,
                                state_dtype, num_slots, out, batch > 0, p);
  if (st != GDN_OK) return st;
  if (batch == 0) return ok();
  if (sdims->head_dim > 1024) return fail(GDN_ERR_SHAPE, "%s: head_dim must be at most 1024", fn);
  if (!slot_idx_dev) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: slot_idx_dev is null", fn);
  if (slot_idx_host) {
    st = check_slots(fn, slot_idx_host, batch, num_slots, true);
    if (st != GDN_OK) return st;
  }
  p.Nseq = batch;
  p.T = batch;
  p.slots = slot_idx_dev;
  return launched(fn, gdn::launch_mamba2_update(p, static_cast<hipStream_t>(stream)));
}

size_t gdn_mamba2_workspace_size(const gdn_ssm_dims* sdims, int32_t num_seqs, int64_t total_tokens) {
  if (sdims == nullptr || num_seqs < 0 || total_tokens < 0 || sdims->num_heads <= 0 || !mamba2_chunked_dims(sdims))
    return 0;
  return gdn::mamba2_workspace_bytes(sdims->num_heads, sdims->head_dim, sdims->state_dim, num_seqs, total_tokens);
}

gdn_status gdn_mamba2_chunk_scan(const gdn_ssm_dims* sdims, int32_t num_seqs, int64_t total_tokens,
                                 const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* x,
                                 const void* dt, const float* A, const void* B, const void* C, const float* D,
                                 int32_t D_per_head_dim, const void* z, const gdn_ssm_dt* dtp,
                                 gdn_dtype act_dtype, void* state_pool, gdn_dtype state_dtype, int32_t num_slots,
                                 const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                                 const uint8_t* has_initial_state_dev, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_mamba2_chunk_scan";
  gdn_status st = check_offsets(fn, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev);
  if (st != GDN_OK) return st;
  gdn::Mamba2Params p;
  st = mamba2_common(fn, sdims, x, dt, A, B, C, D, D_per_head_dim, z, dtp, act_dtype, state_pool, state_dtype,
                     num_slots, out, total_tokens > 0, p);
  if (st != GDN_OK) return st;
  if (num_seqs == 0) return ok();
  if (!mamba2_chunked_dims(sdims))
    return fail(GDN_ERR_SHAPE, "%s: head_dim and state_dim must be 32, 64 or 128, got %d and %d", fn,
                sdims->head_dim, sdims->state_dim);
  if ((slot_idx_host == nullptr) != (slot_idx_dev == nullptr))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: pass both slot index copies or neither", fn);
  if (slot_idx_host) {
    st = check_slots(fn, slot_idx_host, num_seqs, num_slots, false);
    if (st != GDN_OK) return st;
  } else if (num_seqs > num_slots) {
    return fail(GDN_ERR_INDEX, "%s: %d sequences but only %d slots", fn, num_seqs, num_slots);
  }
  const size_t need = gdn::mamba2_workspace_bytes(sdims->num_heads, sdims->head_dim, sdims->state_dim, num_seqs,
                                                  total_tokens);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  int64_t nchunks = 0;
  for (int32_t s = 0; s < num_seqs; ++s) nchunks += (cu_seqlens_host[s + 1] - cu_seqlens_host[s] + 63) / 64;
  p.Nseq = num_seqs;
  p.T = total_tokens;
  p.cu = cu_seqlens_dev;
  p.slots = slot_idx_dev;
  p.has_init = has_initial_state_dev;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.num_chunks = nchunks;
  return launched(fn, gdn::launch_mamba2_chunk_scan(p, static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_size(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                  int32_t chunk_size) {
  if (check_dims("gdn_prefill_workspace_size", dims) != GDN_OK || num_seqs < 0 || total_tokens < 0)
    return 0;
  if (chunk_size == 0) chunk_size = 64;
  if (chunk_size != 64) return 0;
  return gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_k_dim,
                                      dims->head_v_dim, num_seqs, total_tokens, chunk_size);
}

}  // extern "C"

namespace {

// gdn_prefill_varlen and its allocation-free variant: the same checks, then
// the launch on the caller's workspace or on the library's static scratch.
gdn_status prefill_entry(const char* fn, const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                         const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev, const void* q,
                         const void* k, const void* v, gdn_dtype qkv_dtype, const float* g, const float* beta,
                         void* ssm_state_pool, gdn_dtype state_dtype, int32_t num_slots,
                         const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                         const uint8_t* has_initial_state_dev, float scale, int32_t use_qk_l2norm,
                         int32_t chunk_size, void* out, void* workspace, size_t workspace_bytes, bool noalloc,
                         void* stream) {

  gdn_status st = check_dims(fn, dims);
  if (st != GDN_OK) return st;
  st = check_offsets(fn, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev);
  if (st != GDN_OK) return st;
  if (num_seqs == 0) return ok();
  if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16)
    return fail(GDN_ERR_DTYPE, "%s: q/k/v must be f32 or bf16", fn);
  if (state_dtype != GDN_F32 && state_dtype != GDN_BF16 && state_dtype != GDN_F16)
    return fail(GDN_ERR_DTYPE, "%s: state must be f32, bf16 or f16", fn);
  if (chunk_size == 0) chunk_size = 64;
  if (chunk_size != 64) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: chunk_size must be 0 or 64", fn);
  if (!q || !k || !v || !g || !beta || !ssm_state_pool || !out)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a required pointer is null", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(ssm_state_pool))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q/k/v/out/state must be 16-byte aligned", fn);
  if ((slot_idx_host == nullptr) != (slot_idx_dev == nullptr))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: pass both slot index copies or neither", fn);
  if (num_slots <= 0) return fail(GDN_ERR_SHAPE, "%s: num_slots must be positive", fn);
  if (slot_idx_host) {
    st = check_slots(fn, slot_idx_host, num_seqs, num_slots, false);
    if (st != GDN_OK) return st;
  } else if (num_seqs > num_slots) {
    return fail(GDN_ERR_INDEX, "%s: %d sequences but only %d slots", fn, num_seqs, num_slots);
  }
  if (use_qk_l2norm != 0 && use_qk_l2norm != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: use_qk_l2norm must be 0 or 1", fn);
  if (!(scale == scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: scale is NaN", fn);
  if (noalloc) {
    const size_t one = gdn::prefill_workspace_bytes_per_head(dims->head_k_dim, dims->head_v_dim, num_seqs,
                                                             total_tokens);
    if (one > gdn::kNoAllocScratchBytes)
      return fail(GDN_ERR_WORKSPACE,
                  "%s: %d sequences of %lld tokens need %zu bytes of scratch per value head; the static scratch "
                  "holds %zu",
                  fn, num_seqs, (long long)total_tokens, one, gdn::kNoAllocScratchBytes);
  } else {
    const size_t need = gdn::prefill_workspace_bytes(dims->num_k_heads, dims->num_v_heads, dims->head_k_dim,
                                                     dims->head_v_dim, num_seqs, total_tokens, chunk_size);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
      return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(GDN_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }

  int64_t nchunks = 0;
  int max_chunks = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int c = (cu_seqlens_host[s + 1] - cu_seqlens_host[s] + chunk_size - 1) / chunk_size;
    nchunks += c;
    if (c > max_chunks) max_chunks = c;
  }
  gdn::PrefillParams p{};
  p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads; p.Dk = dims->head_k_dim; p.Dv = dims->head_v_dim;
  p.N = num_seqs; p.T = total_tokens; p.cu = cu_seqlens_dev; p.q = q; p.k = k; p.v = v; p.g = g;
  p.beta = beta; p.ssm_pool = ssm_state_pool; p.num_slots = num_slots; p.slots = slot_idx_dev;
  p.has_init = has_initial_state_dev; p.scale = scale; p.l2norm = use_qk_l2norm; p.chunk = chunk_size;
  p.out = out; p.workspace = workspace; p.workspace_bytes = workspace_bytes; p.num_chunks = nchunks;
  p.max_chunks_per_seq = max_chunks; p.qkv = qkv_dtype; p.state = state_dtype;
  p.h0 = 0; p.hg = dims->num_v_heads;
  if (noalloc) return launched(fn, gdn::launch_prefill_noalloc(p, static_cast<hipStream_t>(stream)));
  return launched(fn, gdn::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_varlen(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                              const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                              const void* q, const void* k, const void* v, gdn_dtype qkv_dtype,
                              const float* g, const float* beta, void* ssm_state_pool,
                              gdn_dtype state_dtype, int32_t num_slots,
                              const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                              const uint8_t* has_initial_state_dev, float scale,
                              int32_t use_qk_l2norm, int32_t chunk_size, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_entry("gdn_prefill_varlen", dims, num_seqs, total_tokens, cu_seqlens_host, cu_seqlens_dev, q, k,
                       v, qkv_dtype, g, beta, ssm_state_pool, state_dtype, num_slots, slot_idx_host, slot_idx_dev,
                       has_initial_state_dev, scale, use_qk_l2norm, chunk_size, out, workspace, workspace_bytes,
                       false, stream);
}

gdn_status gdn_prefill_varlen_noalloc(const gdn_dims* dims, int32_t num_seqs, int64_t total_tokens,
                                      const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                                      const void* q, const void* k, const void* v, gdn_dtype qkv_dtype,
                                      const float* g, const float* beta, void* ssm_state_pool,
                                      gdn_dtype state_dtype, int32_t num_slots,
                                      const int32_t* slot_idx_host, const int32_t* slot_idx_dev,
                                      const uint8_t* has_initial_state_dev, float scale,
                                      int32_t use_qk_l2norm, int32_t chunk_size, void* out, void* stream) {
  return prefill_entry("gdn_prefill_varlen_noalloc", dims, num_seqs, total_tokens, cu_seqlens_host,
                       cu_seqlens_dev, q, k, v, qkv_dtype, g, beta, ssm_state_pool, state_dtype, num_slots,
                       slot_idx_host, slot_idx_dev, has_initial_state_dev, scale, use_qk_l2norm, chunk_size, out,
                       nullptr, 0, true, stream);
}

}  // extern "C"

// C ABI of the Taylor-attention library: validation, sizing, table export and dispatch.
//
// Everything here is host logic.  Validation happens before any HIP call, so
// an invalid call returns its status without touching the device (and without
// needing one).  The library never allocates, frees or synchronises device
// memory; its global state is the per-device address of the static workspace
// array of taylor_attn_prefill_into_static (set once per device under a mutex)
// and the single-pass prefill's per-call tag counter (prefill_mfma.hip).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/taylor_attn.h"
#include "common.hpp"
#include "backward.hpp"
#include "launch.hpp"
#include "prefill_mfma.hpp"
#include "prefill_wide.hpp"

namespace {

using taylor::Shape;

constexpr int kDefaultChunk = 64;
constexpr long long kMaxGridY = 65535;  // heads are the second grid dimension

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a config and fills `s`; returns a taylor_status.
int check_config(const taylor_config* cfg, Shape* s) {
  if (!cfg) return TAYLOR_ERR_INVALID_ARG;
  if (cfg->n_terms < 1 || cfg->d_k < 1 || cfg->d_v < 1) return TAYLOR_ERR_INVALID_ARG;
  if (cfg->in_dtype != TAYLOR_F32 && cfg->in_dtype != TAYLOR_BF16) return TAYLOR_ERR_INVALID_ARG;
  if (cfg->readout != TAYLOR_READOUT_KERNEL && cfg->readout != TAYLOR_READOUT_CENTERED) return TAYLOR_ERR_INVALID_ARG;
  if (cfg->chunk < 0) return TAYLOR_ERR_INVALID_ARG;
  if (!std::isfinite(cfg->scale)) return TAYLOR_ERR_INVALID_ARG;
  if (cfg->n_terms > taylor::kMaxTerms) return TAYLOR_ERR_UNSUPPORTED;
  if (cfg->d_k > 4096 || cfg->d_v > 65536) return TAYLOR_ERR_INVALID_ARG;
  const long long W = taylor::feature_width_ll(cfg->n_terms, cfg->d_k);
  if (W <= 0 || W > 0x7fffffffLL) return TAYLOR_ERR_INVALID_ARG;
  if (cfg->d_v % 4 != 0) return TAYLOR_ERR_UNSUPPORTED;
  if (s) {
    s->nt = cfg->n_terms;
    s->dk = cfg->d_k;
    s->dv = cfg->d_v;
    s->dtype = cfg->in_dtype;
    s->readout = cfg->readout;
    s->scale = cfg->scale;
    s->W = W;
    s->stride = (W * (cfg->d_v + 1) + 3) / 4 * 4;
  }
  return TAYLOR_OK;
}

int chunk_of(const taylor_config* cfg) { return cfg->chunk == 0 ? kDefaultChunk : cfg->chunk; }

enum class Path { None, Generic, Mfma, Wide };

Path prefill_path(const Shape& s, int C) {
  if (taylor::prefill_wide_has(s.nt, s.dk, s.dv, s.dtype)) return Path::Wide;
  if (taylor::prefill_mfma_has(s.nt, s.dk, s.dv, s.dtype)) return Path::Mfma;
  if (taylor::prefill_generic_has(s.nt, s.dk, s.dv, C)) return Path::Generic;
  return Path::None;
}

// The expanded-softmax readout is compiled for orders 1 and 2 on the matrix-core shapes.
bool centered_ok(const Shape& s) {
  return s.readout != TAYLOR_READOUT_CENTERED || ((s.nt == 2 || s.nt == 3) && s.dk == 16 && s.dv == 64);
}

int supported(const taylor_config* cfg, const Shape& s) {
  const int C = chunk_of(cfg);
  if (C != 64 && C != 128) return TAYLOR_ERR_UNSUPPORTED;
  if (!centered_ok(s)) return TAYLOR_ERR_UNSUPPORTED;
  if (!taylor::decode_has(s.nt, s.dk, s.dv)) return TAYLOR_ERR_UNSUPPORTED;
  if (prefill_path(s, C) == Path::None) return TAYLOR_ERR_UNSUPPORTED;
  return TAYLOR_OK;
}

int check_sizes(int B, int H, int N) {
  if (B < 0 || H < 0 || N < 0) return TAYLOR_ERR_INVALID_ARG;
  if ((long long)B * H > kMaxGridY) return TAYLOR_ERR_UNSUPPORTED;
  return TAYLOR_OK;
}

taylor::SeqMap equal_lengths(int B, int H, int N) { return taylor::SeqMap{nullptr, 0, B, H, N, 0}; }

int64_t ws_bytes(const Shape& s, int C, int BH, const taylor::SeqMap& seq) {
  if (BH == 0 || seq.N == 0 || seq.tokens(BH) == 0) return 0;
  switch (prefill_path(s, C)) {
    case Path::Mfma: return taylor::prefill_mfma_ws_bytes(s, BH, seq);
    case Path::Wide: return taylor::prefill_wide_ws_bytes(s, BH, seq);
    case Path::Generic:
      if (seq.packed) return TAYLOR_ERR_UNSUPPORTED;
      return taylor::prefill_generic_ws_bytes(s, BH, seq.N, C);
    default: return TAYLOR_ERR_UNSUPPORTED;
  }
}

// Ragged batches: sizes, and the sequence map of a call (cu may be null for a workspace query).
int check_varlen(int n_seqs, int H, int max_seqlen, int64_t total_tokens) {
  int rc = check_sizes(n_seqs, H, max_seqlen);
  if (rc != TAYLOR_OK) return rc;
  if (total_tokens < 0 || total_tokens > (int64_t)n_seqs * max_seqlen) return TAYLOR_ERR_INVALID_ARG;
  if (total_tokens * (int64_t)(H > 0 ? H : 1) > (int64_t(1) << 40)) return TAYLOR_ERR_UNSUPPORTED;
  return TAYLOR_OK;
}

taylor::SeqMap packed_map(const int32_t* cu, int n_seqs, int H, int max_seqlen, int64_t total_tokens) {
  return taylor::SeqMap{cu, 1, n_seqs, H, max_seqlen, (long long)total_tokens};
}

int map_launch(int rc) { return rc == 0 ? TAYLOR_OK : rc == -2 ? TAYLOR_ERR_UNSUPPORTED : TAYLOR_ERR_HIP; }

// Shared by the equal-length and ragged prefills once sizes are checked: pointers, workspace and launch.
int prefill_common(const Shape& s, int C, const void* q, const void* k, const void* v, float* o,
                   const float* state_in, float* state, void* workspace, int BH, const taylor::SeqMap& seq,
                   hipStream_t stream) {
  if (!k || !v || !aligned16(k) || !aligned16(v)) return TAYLOR_ERR_INVALID_ARG;
  if (o && (!q || !aligned16(q) || !aligned16(o))) return TAYLOR_ERR_INVALID_ARG;
  if ((state && !aligned16(state)) || (state_in && !aligned16(state_in))) return TAYLOR_ERR_INVALID_ARG;
  const int64_t need = ws_bytes(s, C, BH, seq);
  if (need < 0) return (int)need;
  if (need > 0 && (!workspace || !aligned16(workspace))) return TAYLOR_ERR_INVALID_ARG;
  if ((long long)(seq.N + C - 1) / C > 0x7fffffffLL / 256) return TAYLOR_ERR_UNSUPPORTED;

  taylor::PrefillArgs a{};
  a.s = s;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.state_in = state_in;
  a.state = state;
  a.ws = workspace;
  a.BH = BH;
  a.N = seq.N;
  a.C = C;
  a.seq = seq;
  a.stream = stream;
  switch (prefill_path(s, C)) {
    case Path::Mfma: return map_launch(taylor::prefill_mfma_launch(a));
    case Path::Wide: return map_launch(taylor::prefill_wide_launch(a));
    default: return seq.packed ? TAYLOR_ERR_UNSUPPORTED : map_launch(taylor::prefill_generic_launch(a));
  }
}

// Workspace of taylor_attn_prefill_into_static: a device array of the library's code object, so each
// GPU the library runs on holds its own copy (from the first call there until the process ends).  In
// host code the name `scratch` is a host-side stand-in, never a device address: kernels receive the
// address hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[TAYLOR_STATIC_WORKSPACE_BYTES];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TAYLOR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TAYLOR_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TAYLOR_OK;
}

}  // namespace

extern "C" {

const char* taylor_status_string(int status) {
  switch (status) {
    case TAYLOR_OK: return "TAYLOR_OK";
    case TAYLOR_ERR_INVALID_ARG: return "TAYLOR_ERR_INVALID_ARG: invalid argument";
    case TAYLOR_ERR_UNSUPPORTED: return "TAYLOR_ERR_UNSUPPORTED: no kernel compiled for this configuration";
    case TAYLOR_ERR_HIP: return "TAYLOR_ERR_HIP: HIP runtime error";
  }
  return "unknown taylor_status";
}

int taylor_feature_width(int n_terms, int d_k) {
  if (n_terms < 1 || d_k < 1 || d_k > 4096 || n_terms > 64) return TAYLOR_ERR_INVALID_ARG;
  long long w = 0;
  for (int m = 0; m < n_terms; ++m) {
    w += taylor::binom(d_k + m - 1, m);
    if (w > 0x7fffffffLL || w <= 0) return TAYLOR_ERR_INVALID_ARG;
  }
  return (int)w;
}

int64_t taylor_state_elems(const taylor_config* cfg) {
  Shape s;
  const int rc = check_config(cfg, &s);
  return rc != TAYLOR_OK ? rc : s.W * (cfg->d_v + 1);
}

int64_t taylor_state_stride(const taylor_config* cfg) {
  Shape s;
  const int rc = check_config(cfg, &s);
  return rc != TAYLOR_OK ? rc : s.stride;
}

int taylor_monomial_table(int n_terms, int d_k, int32_t* idx_out, double* coef_out, size_t cap_rows) {
  if (n_terms < 1 || n_terms > taylor::kMaxTerms) return TAYLOR_ERR_INVALID_ARG;
  const int W = taylor_feature_width(n_terms, d_k);
  if (W < 0) return W;
  if (cap_rows < (size_t)W) return TAYLOR_ERR_INVALID_ARG;
  const int width = n_terms - 1 > 1 ? n_terms - 1 : 1;
  taylor::for_each_monomial(n_terms, d_k, [&](int a, int m, const int* t, int af) {
    if (idx_out)
      for (int p = 0; p < width; ++p) idx_out[(size_t)a * width + p] = p < m ? t[p] : -1;
    if (coef_out) coef_out[a] = 1.0 / std::sqrt((double)af);
  });
  return W;
}

int taylor_supported(const taylor_config* cfg) {
  Shape s;
  const int rc = check_config(cfg, &s);
  return rc != TAYLOR_OK ? rc : supported(cfg, s);
}

int taylor_prefill_chunk(const taylor_config* cfg) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  switch (prefill_path(s, chunk_of(cfg))) {
    case Path::Mfma: return taylor::kMfmaChunk;
    case Path::Wide: return taylor::kWideChunk;
    default: return chunk_of(cfg);
  }
}

int64_t taylor_prefill_workspace_bytes(const taylor_config* cfg, int B, int H, int N) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_sizes(B, H, N)) != TAYLOR_OK) return rc;
  return ws_bytes(s, chunk_of(cfg), B * H, equal_lengths(B, H, N));
}

int64_t taylor_prefill_varlen_workspace_bytes(const taylor_config* cfg, int n_seqs, int H, int max_seqlen,
                                              int64_t total_tokens) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_varlen(n_seqs, H, max_seqlen, total_tokens)) != TAYLOR_OK) return rc;
  return ws_bytes(s, chunk_of(cfg), n_seqs * H, packed_map(nullptr, n_seqs, H, max_seqlen, total_tokens));
}

int taylor_state_init(float* state, int B, int H, const taylor_config* cfg, hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = check_sizes(B, H, 0)) != TAYLOR_OK) return rc;
  if ((long long)B * H == 0) return TAYLOR_OK;
  if (!state || !aligned16(state)) return TAYLOR_ERR_INVALID_ARG;
  return map_launch(taylor::state_zero_launch(state, (long long)B * H * s.stride, stream));
}

int taylor_attn_prefill(const void* q, const void* k, const void* v, float* o, float* state, void* workspace, int B,
                        int H, int N, const taylor_config* cfg, hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_sizes(B, H, N)) != TAYLOR_OK) return rc;
  if (!o && !state) return TAYLOR_ERR_INVALID_ARG;
  const int BH = B * H;
  if (BH == 0 || N == 0) return TAYLOR_OK;
  return prefill_common(s, chunk_of(cfg), q, k, v, o, state, state, workspace, BH, equal_lengths(B, H, N), stream);
}

int taylor_attn_prefill_into(const void* q, const void* k, const void* v, float* o, const float* state_in,
                             float* state_out, void* workspace, int B, int H, int N, const taylor_config* cfg,
                             hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_sizes(B, H, N)) != TAYLOR_OK) return rc;
  if (!o && !state_out) return TAYLOR_ERR_INVALID_ARG;
  const long long BH = (long long)B * H;
  if (BH == 0) return TAYLOR_OK;
  if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out))) return TAYLOR_ERR_INVALID_ARG;
  if (state_in && state_out && state_in != state_out) {
    // the two state arrays are the same array or disjoint
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(state_in), b0 = reinterpret_cast<uintptr_t>(state_out);
    const uintptr_t bytes = (uintptr_t)(BH * s.stride) * sizeof(float);
    if (a0 < b0 + bytes && b0 < a0 + bytes) return TAYLOR_ERR_INVALID_ARG;
  }
  if (N == 0) {
    // no tokens: the final state is the incoming one
    if (!state_out || state_out == state_in) return TAYLOR_OK;
    return map_launch(state_in ? taylor::state_copy_launch(state_out, state_in, BH * s.stride, stream)
                               : taylor::state_zero_launch(state_out, BH * s.stride, stream));
  }
  return prefill_common(s, chunk_of(cfg), q, k, v, o, state_in, state_out, workspace, (int)BH, equal_lengths(B, H, N),
                        stream);
}

int taylor_attn_prefill_into_static(const void* q, const void* k, const void* v, float* o, const float* state_in,
                                    float* state_out, int B, int H, int N, const taylor_config* cfg,
                                    hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_sizes(B, H, N)) != TAYLOR_OK) return rc;
  const int BH = B * H;
  const int64_t need = (BH == 0 || N == 0) ? 0 : ws_bytes(s, chunk_of(cfg), BH, equal_lengths(B, H, N));
  if (need < 0) return (int)need;
  if (need > (int64_t)TAYLOR_STATIC_WORKSPACE_BYTES) return TAYLOR_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (need > 0 && (rc = scratch_for_current_device(&ws)) != TAYLOR_OK) return rc;
  return taylor_attn_prefill_into(q, k, v, o, state_in, state_out, ws, B, H, N, cfg, stream);
}

int taylor_attn_prefill_varlen(const void* q, const void* k, const void* v, float* o, float* state, void* workspace,
                               const int32_t* cu_seqlens, int n_seqs, int H, int max_seqlen, int64_t total_tokens,
                               const taylor_config* cfg, hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_varlen(n_seqs, H, max_seqlen, total_tokens)) != TAYLOR_OK) return rc;
  if (!o && !state) return TAYLOR_ERR_INVALID_ARG;
  const int BH = n_seqs * H;
  if (BH == 0 || total_tokens == 0) return TAYLOR_OK;  // every sequence is empty: states unchanged
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return TAYLOR_ERR_INVALID_ARG;
  return prefill_common(s, chunk_of(cfg), q, k, v, o, state, state, workspace, BH,
                        packed_map(cu_seqlens, n_seqs, H, max_seqlen, total_tokens), stream);
}

int taylor_attn_prefill_varlen_into(const void* q, const void* k, const void* v, float* o, const float* state_in,
                                    float* state_out, void* workspace, const int32_t* cu_seqlens, int n_seqs, int H,
                                    int max_seqlen, int64_t total_tokens, const taylor_config* cfg,
                                    hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if ((rc = supported(cfg, s)) != TAYLOR_OK) return rc;
  if ((rc = check_varlen(n_seqs, H, max_seqlen, total_tokens)) != TAYLOR_OK) return rc;
  if (!o && !state_out) return TAYLOR_ERR_INVALID_ARG;
  const long long BH = (long long)n_seqs * H;
  if (BH == 0) return TAYLOR_OK;
  if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out))) return TAYLOR_ERR_INVALID_ARG;
  if (state_in && state_out && state_in != state_out) {
    // the two state arrays are the same array or disjoint
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(state_in), b0 = reinterpret_cast<uintptr_t>(state_out);
    const uintptr_t bytes = (uintptr_t)(BH * s.stride) * sizeof(float);
    if (a0 < b0 + bytes && b0 < a0 + bytes) return TAYLOR_ERR_INVALID_ARG;
  }
  if (total_tokens == 0) {
    // every sequence is empty: each final state is its incoming one
    if (!state_out || state_out == state_in) return TAYLOR_OK;
    return map_launch(state_in ? taylor::state_copy_launch(state_out, state_in, BH * s.stride, stream)
                               : taylor::state_zero_launch(state_out, BH * s.stride, stream));
  }
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return TAYLOR_ERR_INVALID_ARG;
  return prefill_common(s, chunk_of(cfg), q, k, v, o, state_in, state_out, workspace, (int)BH,
                        packed_map(cu_seqlens, n_seqs, H, max_seqlen, total_tokens), stream);
}

int64_t taylor_prefill_backward_workspace_bytes(const taylor_config* cfg, int B, int H, int N) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if (s.readout != TAYLOR_READOUT_KERNEL || !taylor::backward_has(s.nt, s.dk, s.dv)) return TAYLOR_ERR_UNSUPPORTED;
  if ((rc = check_sizes(B, H, N)) != TAYLOR_OK) return rc;
  return taylor::backward_ws_bytes(s, B * H, N);
}

int taylor_attn_prefill_backward(const void* q, const void* k, const void* v, const float* o, const float* g,
                                 const float* state, float* dstate, float* dq, float* dk, float* dv, void* workspace,
                                 int B, int H, int N, const taylor_config* cfg, hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if (s.readout != TAYLOR_READOUT_KERNEL || !taylor::backward_has(s.nt, s.dk, s.dv)) return TAYLOR_ERR_UNSUPPORTED;
  if ((rc = check_sizes(B, H, N)) != TAYLOR_OK) return rc;
  const int BH = B * H;
  if (BH == 0) return TAYLOR_OK;
  if (N == 0) {
    // no tokens: the incoming state's gradient is the final state's; dstate is left as it is
    return TAYLOR_OK;
  }
  const void* need16[] = {q, k, v, o, g, dq, dk, dv};
  for (const void* p : need16)
    if (!p || !aligned16(p)) return TAYLOR_ERR_INVALID_ARG;
  if ((state && !aligned16(state)) || (dstate && !aligned16(dstate))) return TAYLOR_ERR_INVALID_ARG;
  if ((long long)(N + 15) / 16 > 0x7fffffffLL / 256) return TAYLOR_ERR_UNSUPPORTED;
  const long long need = taylor::backward_ws_bytes(s, BH, N);
  if (need > 0 && (!workspace || !aligned16(workspace))) return TAYLOR_ERR_INVALID_ARG;
  taylor::BwdArgs a{};
  a.s = s;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.g = g;
  a.state = state;
  a.dstate = dstate;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws = workspace;
  a.BH = BH;
  a.N = N;
  a.stream = stream;
  return map_launch(taylor::backward_launch(a));
}

int taylor_attn_decode_step(const void* q, const void* k, const void* v, float* o, float* state, int B, int H,
                            const taylor_config* cfg, hipStream_t stream) {
  Shape s;
  int rc = check_config(cfg, &s);
  if (rc != TAYLOR_OK) return rc;
  if (!taylor::decode_has(s.nt, s.dk, s.dv)) return TAYLOR_ERR_UNSUPPORTED;
  if (!centered_ok(s)) return TAYLOR_ERR_UNSUPPORTED;
  if ((rc = check_sizes(B, H, 1)) != TAYLOR_OK) return rc;
  const int BH = B * H;
  if (BH == 0) return TAYLOR_OK;
  if (!q || !k || !v || !o || !state) return TAYLOR_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(state))
    return TAYLOR_ERR_INVALID_ARG;
  taylor::DecodeArgs a{};
  a.s = s;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.state = state;
  a.BH = BH;
  a.stream = stream;
  return map_launch(taylor::decode_launch(a));
}

}  // extern "C"

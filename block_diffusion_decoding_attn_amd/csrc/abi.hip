// C ABI entry points of libfdl: host-side validation, then kernel launches.
// Nothing here allocates device memory or synchronizes with the device.
#include "common.h"
#include "launch.h"

#include <cmath>
#include <mutex>

namespace fdl {

// Scratch of fdl_lm_head_select_noalloc: a file-scope device array (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// must not pass `scratch` itself to a kernel (that is a host-side stand-in):
// its device address is looked up once per device with hipGetSymbolAddress
// and kept per device.
static __device__ __align__(256) char scratch[FDL_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device, with it current).
static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FDL_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FDL_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FDL_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FDL_OK;
}

int dtype_size(int dtype) { return dtype == FDL_F32 ? 4 : 2; }

int check_launch() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? FDL_OK : FDL_E_HIP;
}

// Checks shared by every entry point.
static int check_dims(const fdl_dims* d) {
  if (!d) return FDL_E_INVAL;
  if (d->batch < 1 || d->prompt_len < 0 || d->gen_len < 1 || d->block < 1 || d->sub_block < 1) return FDL_E_INVAL;
  if (d->block % d->sub_block != 0 || d->gen_len % d->block != 0) return FDL_E_INVAL;
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0) return FDL_E_INVAL;
  if (d->head_dim < 1 || d->hidden < 1 || d->vocab < 1) return FDL_E_INVAL;
  if (d->dtype != FDL_F32 && d->dtype != FDL_BF16) return FDL_E_INVAL;
  if (d->attn_mode != FDL_ATTN_BLOCK_CAUSAL && d->attn_mode != FDL_ATTN_DUAL_CACHE) return FDL_E_INVAL;
  // size limits that keep every index inside 32-bit arithmetic where it is used
  const long long cap = (long long)d->prompt_len + d->gen_len;
  if (cap > (1 << 24) || d->vocab > (1 << 28) || d->hidden > (1 << 20)) return FDL_E_UNSUPPORTED;
  if (d->batch > 65535 || d->n_kv_heads > 32767) return FDL_E_UNSUPPORTED;  // grid y/z extents
  if (d->head_dim != 64 && d->head_dim != 128) return FDL_E_UNSUPPORTED;
  return FDL_OK;
}

static int check_select_args(const fdl_dims& d, int32_t rows_per_seq, const uint8_t* masked, const float* tau,
                             int32_t mode, int32_t k, float factor, const int32_t* token_out, const float* conf_out,
                             const uint8_t* commit_out, const int32_t* n_commit) {
  if (rows_per_seq < 1 || rows_per_seq > 256) return FDL_E_INVAL;
  if (!masked || !token_out || !conf_out || !commit_out || !n_commit) return FDL_E_INVAL;
  if (mode == FDL_SELECT_THRESHOLD) {
    if (!tau) return FDL_E_INVAL;
  } else if (mode == FDL_SELECT_TOPK) {
    if (k < 1) return FDL_E_INVAL;
  } else if (mode == FDL_SELECT_FACTOR) {
    if (!(factor > 0.f)) return FDL_E_INVAL;
  } else {
    return FDL_E_INVAL;
  }
  if ((long long)d.batch * rows_per_seq > 65535) return FDL_E_UNSUPPORTED;  // grid y extent
  return FDL_OK;
}

static int check_lm_head_args(const fdl_dims& d, int32_t rows, const void* x, const void* w) {
  if (rows < 1 || !x || !w) return FDL_E_INVAL;
  if (d.dtype == FDL_BF16 && d.hidden % 64 != 0) return FDL_E_UNSUPPORTED;
  if (d.dtype == FDL_F32 && (d.hidden % 4 != 0 || rows > 64)) return FDL_E_UNSUPPORTED;
  if ((long long)rows * d.vocab > (1LL << 40)) return FDL_E_UNSUPPORTED;
  return FDL_OK;
}

// Arguments of the decode loop beyond the dims.
static int check_decode(const fdl_dims& d, const fdl_decode_args* g) {
  if (!g) return FDL_E_INVAL;
  if (!g->w || !g->boost_tok || !g->boost_val || !g->k_cache || !g->v_cache || !g->len || !g->tokens ||
      !g->masked || !g->seq_steps || !g->eos_block || !g->counters)
    return FDL_E_INVAL;
  if (d.prompt_len > 0 && !g->prompt) return FDL_E_INVAL;
  if (g->mask_id < 0 || g->mask_id >= d.vocab || g->eos_id < 0 || g->eos_id >= d.vocab) return FDL_E_INVAL;
  if (!std::isfinite(g->gain)) return FDL_E_INVAL;
  const int nb = d.gen_len / d.block;
  if (g->max_blocks < 0 || g->max_blocks > nb) return FDL_E_INVAL;
  const int S = d.sub_block;
  if (S > 256) return FDL_E_INVAL;
  if ((long long)d.batch * S > 65535) return FDL_E_UNSUPPORTED;  // select grid extent
  if (g->mode == FDL_SELECT_THRESHOLD) {
    if (!g->tau) return FDL_E_INVAL;
  } else if (g->mode == FDL_SELECT_TOPK) {
    if (g->k < 1) return FDL_E_INVAL;
  } else if (g->mode == FDL_SELECT_FACTOR) {
    if (!(g->factor > 0.f)) return FDL_E_INVAL;
  } else {
    return FDL_E_INVAL;
  }
  const int rc = check_lm_head_args(d, d.batch * S, g->w, g->w);
  if (rc != FDL_OK) return rc;
  if ((long long)d.n_q_heads * d.head_dim != d.hidden) return FDL_E_UNSUPPORTED;  // the stand-in model
  if ((d.n_q_heads / d.n_kv_heads) * S > attn_max_rows()) return FDL_E_UNSUPPORTED;
  const bool any = g->trace_meta || g->trace_tokens || g->trace_masked || g->trace_token || g->trace_conf;
  const bool all = g->trace_meta && g->trace_tokens && g->trace_masked && g->trace_token && g->trace_conf;
  if (any && !all) return FDL_E_INVAL;
  if (all) {
    const long long slots = (long long)(g->max_blocks > 0 ? g->max_blocks : nb) * (d.block / S) *
                            decode_slots_per_sub(d, g->mode, g->k);
    if (g->trace_cap < slots) return FDL_E_INVAL;
  }
  return FDL_OK;
}

}  // namespace fdl

using namespace fdl;

#pragma GCC visibility push(default)
extern "C" {

int fdl_version(void) { return 100; }

const char* fdl_strerror(int status) {
  switch (status) {
    case FDL_OK: return "ok";
    case FDL_E_INVAL: return "invalid argument";
    case FDL_E_UNSUPPORTED: return "unsupported argument combination";
    case FDL_E_HIP: return "HIP launch error";
    case FDL_E_WORKSPACE: return "workspace missing or too small";
    case FDL_E_SCRATCH: return "problem needs more than the allocation-free entry point's static scratch";
    default: return "unknown status";
  }
}

int fdl_dims_check(const fdl_dims* dims) { return check_dims(dims); }

size_t fdl_block_attn_workspace_size(const fdl_dims* dims) {
  if (check_dims(dims) != FDL_OK) return 0;
  return attn_workspace_bytes(*dims);
}

int fdl_block_attn(const fdl_dims* dims, int32_t block_idx, int32_t sub_idx, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* prefix_len, const void* k_blk, const void* v_blk, void* out,
                   float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  if (block_idx < 0 || block_idx >= d.gen_len / d.block) return FDL_E_INVAL;
  if (sub_idx < 0 || sub_idx >= d.block / d.sub_block) return FDL_E_INVAL;
  if (!q || !k_cache || !v_cache || !k_blk || !v_blk || !out) return FDL_E_INVAL;
  if ((d.n_q_heads / d.n_kv_heads) * d.sub_block > attn_max_rows()) return FDL_E_UNSUPPORTED;
  return attn_launch(d, block_idx, q, k_cache, v_cache, prefix_len, k_blk, v_blk, out, lse, workspace,
                     workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

int fdl_prefill_attn(const fdl_dims* dims, int32_t q_start, int32_t n_q, int32_t n_keys, int32_t causal,
                     const void* q, const void* k, const void* v, void* out, float* lse, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  if (!q || !k || !v || !out) return FDL_E_INVAL;
  if (n_q < 1 || q_start < 0 || n_keys < 1 || n_keys > d.prompt_len + d.gen_len) return FDL_E_INVAL;
  if (causal != 0 && causal != 1) return FDL_E_INVAL;
  if (d.dtype != FDL_BF16) return FDL_E_UNSUPPORTED;
  if ((long long)q_start + n_q > (1 << 24) || d.n_q_heads > 65535) return FDL_E_UNSUPPORTED;
  return prefill_launch(d, q_start, n_q, n_keys, causal, q, k, v, out, lse, reinterpret_cast<hipStream_t>(stream));
}

int fdl_lm_head(const fdl_dims* dims, int32_t rows, const void* x, const void* w, float* logits, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  if (!logits) return FDL_E_INVAL;
  rc = check_lm_head_args(d, rows, x, w);
  if (rc != FDL_OK) return rc;
  return lm_head_launch(d, rows, x, w, logits, nullptr, reinterpret_cast<hipStream_t>(stream));
}

size_t fdl_conf_select_workspace_size(const fdl_dims* dims, int32_t rows_per_seq) {
  if (check_dims(dims) != FDL_OK || rows_per_seq < 1 || rows_per_seq > 256) return 0;
  return select_workspace_bytes(*dims, rows_per_seq);
}

int fdl_conf_select(const fdl_dims* dims, int32_t rows_per_seq, const float* logits, const uint8_t* masked,
                    const float* tau, int32_t mode, int32_t k, float factor, int32_t* token_out, float* conf_out,
                    uint8_t* commit_out, int32_t* n_commit, int32_t* tokens_inout, uint8_t* masked_inout,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  if (!logits) return FDL_E_INVAL;
  rc = check_select_args(d, rows_per_seq, masked, tau, mode, k, factor, token_out, conf_out, commit_out, n_commit);
  if (rc != FDL_OK) return rc;
  return select_launch(d, rows_per_seq, logits, masked, tau, mode, k, factor, token_out, conf_out, commit_out,
                       n_commit, tokens_inout, masked_inout, workspace, workspace_bytes,
                       reinterpret_cast<hipStream_t>(stream));
}

size_t fdl_lm_head_select_workspace_size(const fdl_dims* dims, int32_t rows_per_seq) {
  if (check_dims(dims) != FDL_OK || rows_per_seq < 1 || rows_per_seq > 256) return 0;
  return partials_workspace_bytes(*dims, rows_per_seq, lm_head_tiles(*dims, dims->batch * rows_per_seq));
}

int fdl_lm_head_select(const fdl_dims* dims, int32_t rows_per_seq, const void* x, const void* w, float* logits,
                       const uint8_t* masked, const float* tau, int32_t mode, int32_t k, float factor,
                       int32_t* token_out, float* conf_out, uint8_t* commit_out, int32_t* n_commit,
                       int32_t* tokens_inout, uint8_t* masked_inout, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  rc = check_select_args(d, rows_per_seq, masked, tau, mode, k, factor, token_out, conf_out, commit_out, n_commit);
  if (rc != FDL_OK) return rc;
  const int rows = d.batch * rows_per_seq;
  rc = check_lm_head_args(d, rows, x, w);
  if (rc != FDL_OK) return rc;
  const int nc = lm_head_tiles(d, rows);
  if (!workspace || workspace_bytes < partials_workspace_bytes(d, rows_per_seq, nc)) return FDL_E_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = lm_head_launch(d, rows, x, w, logits, workspace, st);
  if (rc != FDL_OK) return rc;
  return select_finalize_launch(d, rows_per_seq, workspace, nc, masked, tau, mode, k, factor, token_out, conf_out,
                                commit_out, n_commit, tokens_inout, masked_inout, st);
}

int fdl_lm_head_select_noalloc(const fdl_dims* dims, int32_t rows_per_seq, const void* x, const void* w,
                               float* logits, const uint8_t* masked, const float* tau, int32_t mode, int32_t k,
                               float factor, int32_t* token_out, float* conf_out, uint8_t* commit_out,
                               int32_t* n_commit, int32_t* tokens_inout, uint8_t* masked_inout, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  rc = check_select_args(d, rows_per_seq, masked, tau, mode, k, factor, token_out, conf_out, commit_out, n_commit);
  if (rc != FDL_OK) return rc;
  const int rows = d.batch * rows_per_seq;
  rc = check_lm_head_args(d, rows, x, w);
  if (rc != FDL_OK) return rc;
  const int nc = lm_head_tiles(d, rows);
  const size_t need = partials_workspace_bytes(d, rows_per_seq, nc);
  if (need > FDL_NOALLOC_SCRATCH_BYTES) return FDL_E_SCRATCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FDL_OK) return rc;
  // the partials' row counters are zeroed by the LM-head kernel itself, so
  // nothing of the scratch has to be cleared here
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  rc = lm_head_launch(d, rows, x, w, logits, ws, st);
  if (rc != FDL_OK) return rc;
  return select_finalize_launch(d, rows_per_seq, ws, nc, masked, tau, mode, k, factor, token_out, conf_out,
                                commit_out, n_commit, tokens_inout, masked_inout, st);
}

int fdl_kv_append(const fdl_dims* dims, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  int32_t n_new, int32_t* len, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  if (!k_cache || !v_cache || !k_new || !v_new || !len) return FDL_E_INVAL;
  if (n_new < 1 || n_new > d.prompt_len + d.gen_len) return FDL_E_INVAL;
  return append_launch(d, k_cache, v_cache, k_new, v_new, n_new, len, reinterpret_cast<hipStream_t>(stream));
}

int fdl_kv_write(const fdl_dims* dims, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                 int32_t pos, int32_t n_new, int32_t* len, void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  if (!k_cache || !v_cache || !k_new || !v_new) return FDL_E_INVAL;
  if (n_new < 1 || pos < 0 || (long long)pos + n_new > (long long)d.prompt_len + d.gen_len) return FDL_E_INVAL;
  return write_launch(d, k_cache, v_cache, k_new, v_new, pos, n_new, len, reinterpret_cast<hipStream_t>(stream));
}

size_t fdl_decode_workspace_size(const fdl_dims* dims) {
  if (check_dims(dims) != FDL_OK) return 0;
  return decode_workspace_bytes(*dims);
}

int32_t fdl_decode_step_slots(const fdl_dims* dims, int32_t mode, int32_t k, int32_t max_blocks) {
  if (check_dims(dims) != FDL_OK) return 0;
  const int nb = dims->gen_len / dims->block;
  if (max_blocks < 0 || max_blocks > nb) return 0;
  if (mode != FDL_SELECT_THRESHOLD && mode != FDL_SELECT_TOPK && mode != FDL_SELECT_FACTOR) return 0;
  if (mode == FDL_SELECT_TOPK && k < 1) return 0;
  return (max_blocks > 0 ? max_blocks : nb) * (dims->block / dims->sub_block) *
         decode_slots_per_sub(*dims, mode, k);
}

int fdl_decode(const fdl_dims* dims, const fdl_decode_args* args, void* workspace, size_t workspace_bytes,
               void* stream) {
  int rc = check_dims(dims);
  if (rc != FDL_OK) return rc;
  const fdl_dims& d = *dims;
  rc = check_decode(d, args);
  if (rc != FDL_OK) return rc;
  if (!workspace || workspace_bytes < decode_workspace_bytes(d)) return FDL_E_WORKSPACE;
  return decode_launch(d, *args, workspace, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
#pragma GCC visibility pop

// Internal launchers of libfdl (host side): each validates nothing and only
// enqueues kernels on the given stream.  The C ABI entry points check their
// arguments before calling these; the decode loop calls them with a gate
// word (a kernel whose gate reads 0 does no work).
#pragma once

#include "common.h"

namespace fdl {

size_t attn_workspace_bytes(const fdl_dims& d);
int attn_max_rows();
int attn_launch(const fdl_dims& d, int block_idx, const void* q, const void* kc, const void* vc,
                const int32_t* prefix_len, const void* kb, const void* vb, void* out, float* lse, void* ws,
                size_t ws_bytes, hipStream_t st, const int32_t* gate = nullptr);
int prefill_launch(const fdl_dims& d, int q_start, int n_q, int n_keys, int causal, const void* q, const void* k,
                   const void* v, void* out, float* lse, hipStream_t st);
int lm_head_tiles(const fdl_dims& d, int rows);
// part: null, or a partials workspace laid out for rows / d.batch rows per
// sequence (partials_workspace_bytes), whose counters the launch zeroes
int lm_head_launch(const fdl_dims& d, int rows, const void* x, const void* w, float* logits, void* part,
                   hipStream_t st, const int32_t* gate = nullptr);
int select_finalize_launch(const fdl_dims& d, int R, const void* part, int nc, const uint8_t* masked,
                           const float* tau, int mode, int k, float factor, int32_t* token_out, float* conf_out,
                           uint8_t* commit_out, int32_t* n_commit, int32_t* tokens_inout, uint8_t* masked_inout,
                           hipStream_t st, int state_stride = 0, const int32_t* gate = nullptr);
size_t select_workspace_bytes(const fdl_dims& d, int rows_per_seq);
size_t partials_workspace_bytes(const fdl_dims& d, int rows_per_seq, int nc);
int32_t* partials_counters(void* ws, const fdl_dims& d, int rows_per_seq, int nc);
int select_launch(const fdl_dims& d, int R, const float* logits, const uint8_t* masked, const float* tau, int mode,
                  int k, float factor, int32_t* token_out, float* conf_out, uint8_t* commit_out, int32_t* n_commit,
                  int32_t* tokens_inout, uint8_t* masked_inout, void* ws, size_t ws_bytes, hipStream_t st);
int append_launch(const fdl_dims& d, void* kc, void* vc, const void* kn, const void* vn, int n_new, int32_t* len,
                  hipStream_t st, const int32_t* gate = nullptr);
int write_launch(const fdl_dims& d, void* kc, void* vc, const void* kn, const void* vn, int pos, int n_new,
                 int32_t* len, hipStream_t st);
size_t decode_workspace_bytes(const fdl_dims& d);
int decode_slots_per_sub(const fdl_dims& d, int mode, int k);
int decode_launch(const fdl_dims& d, const fdl_decode_args& g, void* ws, hipStream_t st);

}  // namespace fdl

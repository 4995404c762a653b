// Confidence select with the commit-state update.
//
// Per row ("Fast-dLLM v2: Efficient Block-Diffusion LLM", Inference Pipeline
// Level 2; "Fast-dLLM: Reusing Bidirectional State ...", Algorithm 2 steps
// 1-2): the greedy token is the argmax of the logits (lowest id on equal
// values) and its confidence is its softmax probability,
// 1 / sum_v exp(l_v - l_max).
// Per sequence, over the masked (candidate) rows: Algorithm 2 threshold with
// the single-most-confident fallback, the fixed count of the review
// questions page, or the factor rule of eq 13 / Algorithm 3.
//
// gfx950 design: the logits are an HBM stream of 4 M V bytes.  Kernel 1 splits
// every row into chunks so that thousands of workgroups stream it with 16-byte
// loads, each reducing its chunk to (max, lowest argmax, sum exp(l - max)).
// (The fused LM head writes the same partials from its epilogue instead.)
// Kernel 2 (one workgroup per row) merges a row's partials in a fixed order --
// the result does not depend on scheduling -- and the workgroup that finishes
// a sequence's last row applies the selection rule, then writes the commit set
// and updates tokens/masked.
#include <climits>

#include "common.h"

namespace fdl {

struct SelArgs {
  const float* logits;
  const uint8_t* masked;
  const float* tau;
  int mode, k;
  float factor;
  int32_t* token_out;
  float* conf_out;
  uint8_t* commit_out;
  int32_t* n_commit;
  int32_t* tokens_inout;
  uint8_t* masked_inout;
  f32x4* part;  // [M][NC] (max, sum, argmax bits, 0)
  int B, R, V, NC, chunk;
  int sstride;          // elements between sequences in masked / tokens_inout / masked_inout
  const int32_t* gate;  // decode loop: skip the launch when *gate == 0 (null: always run)
  int32_t* cnt;         // [B] rows finalized per sequence (zeroed by the producer of the partials)
};

template <bool VEC>
__global__ __launch_bounds__(256) void select_partial_kernel(SelArgs a) {
  __shared__ Red sh[4];
  if (gate_closed(a.gate)) return;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.B; i += 256) a.cnt[i] = 0;
  const int row = blockIdx.y, c = blockIdx.x;
  const int v_begin = c * a.chunk;
  const int v_end = min(v_begin + a.chunk, a.V);
  const float* lg = a.logits + size_t(row) * a.V;
  Red r{-INFINITY, 0.f, INT_MAX};
  if (VEC) {
    for (int v = v_begin + threadIdx.x * 4; v < v_end; v += 256 * 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(lg + v);
      push(r, x[0], v);
      push(r, x[1], v + 1);
      push(r, x[2], v + 2);
      push(r, x[3], v + 3);
    }
  } else {
    for (int v = v_begin + threadIdx.x; v < v_end; v += 256) push(r, lg[v], v);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Red b{__shfl_xor(r.m, o, 64), __shfl_xor(r.s, o, 64), __shfl_xor(r.i, o, 64)};
    r = combine(r, b);
  }
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    Red t = sh[0];
    t = combine(t, sh[1]);
    t = combine(t, sh[2]);
    t = combine(t, sh[3]);
    a.part[size_t(row) * a.NC + c] = f32x4{t.m, t.s, __int_as_float(t.i), 0.f};
  }
}

// One workgroup of FIN_NT threads per row.  Phase 1: the row's chunk
// partials are merged, thread j taking chunks j, j + FIN_NT, ... in
// increasing order (all its loads issued together), then a fixed butterfly
// over the wave and a fixed-order combination of the waves: the result does
// not depend on scheduling.  The row's token and confidence are written and
// the row is counted for its sequence (a device-scope counter that the
// producer kernel zeroed).  Phase 2 runs only in the workgroup that counts a
// sequence's last row: one thread per row (R <= 256) applies the rule.
constexpr int FIN_NT = 256;
constexpr int FIN_U = 8;

__global__ __launch_bounds__(FIN_NT) void select_finalize_kernel(SelArgs a) {
  __shared__ Red red_w[FIN_NT / 64];
  __shared__ float conf_s[256];
  __shared__ int cand_s[256];
  __shared__ int red_i[256];
  __shared__ int last_s;
  if (gate_closed(a.gate)) return;
  const int row_g = blockIdx.x;               // b * R + r
  const int b = row_g / a.R;
  const int tid = threadIdx.x;
  {
    const f32x4* prow = a.part + size_t(row_g) * a.NC;
    Red t = red_empty();
    for (int c0 = tid; c0 < a.NC; c0 += FIN_NT * FIN_U) {
      f32x4 p[FIN_U];
#pragma unroll
      for (int u = 0; u < FIN_U; ++u) {
        const int c = c0 + u * FIN_NT;
        p[u] = c < a.NC ? prow[c] : f32x4{-INFINITY, 0.f, __int_as_float(0x7fffffff), 0.f};
      }
#pragma unroll
      for (int u = 0; u < FIN_U; ++u) t = combine(t, unpack_red(p[u]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) t = combine(t, shfl_xor_red(t, o));
    if ((tid & 63) == 0) red_w[tid >> 6] = t;
    __syncthreads();
    if (tid == 0) {
      Red r = red_w[0];
#pragma unroll
      for (int w = 1; w < FIN_NT / 64; ++w) r = combine(r, red_w[w]);
      a.token_out[row_g] = r.i;
      a.conf_out[row_g] = 1.f / r.s;
      // publish the row, then count it; the last row of the sequence applies the rule
      __threadfence();
      const int prev = atomicAdd(&a.cnt[b], 1);
      last_s = prev == a.R - 1;
    }
    __syncthreads();
    if (!last_s) return;
    __threadfence();
  }
  const int r = tid;
  const bool live = r < a.R;
  const size_t row = size_t(b) * a.R + r;
  const size_t srow = size_t(b) * a.sstride + r;  // row in the per-sequence state arrays
  float conf = 0.f;
  int tok = 0, cand = 0;
  if (live) {
    conf = __hip_atomic_load(&a.conf_out[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok = __hip_atomic_load(&a.token_out[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cand = a.masked[srow] != 0;
    conf_s[r] = conf;
  }
  if (r < 256) cand_s[r] = live ? cand : 0;
  __syncthreads();

  // rank among candidates: decreasing confidence, lower row first on ties
  int rank = 0;
  if (live && cand) {
    for (int q = 0; q < a.R; ++q) {
      if (!cand_s[q]) continue;
      const float cq = conf_s[q];
      rank += (cq > conf || (cq == conf && q < r)) ? 1 : 0;
    }
  }
  // block reductions (every thread reaches each barrier)
  auto reduce_sum = [&](int v) {
    red_i[r] = v;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (r < o) red_i[r] += red_i[r + o];
      __syncthreads();
    }
    const int out = red_i[0];
    __syncthreads();
    return out;
  };
  auto reduce_max = [&](int v) {
    red_i[r] = v;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (r < o) red_i[r] = max(red_i[r], red_i[r + o]);
      __syncthreads();
    }
    const int out = red_i[0];
    __syncthreads();
    return out;
  };
  bool sel = false;
  if (a.mode == FDL_SELECT_THRESHOLD) {
    sel = live && cand && conf > a.tau[b];
    const int n_above = reduce_sum(sel ? 1 : 0);
    if (n_above == 0) sel = live && cand && rank == 0;  // fallback: the most confident candidate
  } else if (a.mode == FDL_SELECT_TOPK) {
    sel = live && cand && rank < a.k;
  } else {  // FDL_SELECT_FACTOR
    const int n = rank + 1;
    const bool ok = live && cand && float(n + 1) * (1.f - conf) < a.factor;
    const int best = reduce_max(ok ? n : 0);
    const int nstar = best > 0 ? best : 1;
    sel = live && cand && rank < nstar;
  }
  const int n_sel = reduce_sum(sel ? 1 : 0);
  if (r == 0) {
    a.n_commit[b] = n_sel;
    a.cnt[b] = 0;
  }
  if (live) {
    a.commit_out[row] = sel ? 1 : 0;
    if (sel && a.tokens_inout) a.tokens_inout[srow] = tok;
    if (sel && a.masked_inout) a.masked_inout[srow] = 0;
  }
}

// Many rows (B x R > 64, R a multiple of 8, R <= 64): a workgroup of 1024
// threads merges 8 rows of one sequence, 128 threads per row with sixteen
// partial loads in flight per thread (thread t of a row takes partials t,
// t + 128, ... in increasing order; then a fixed butterfly over the wave and
// the row's two waves in order), writes their tokens and confidences and
// counts itself on the sequence's counter: R / 8 arrivals per counter instead
// of R, since device-scope atomics on one address serialize and each
// arrival's release fence is a write-back of the CU's L2 (measured at 16 x 32
// rows: 25 us per-row, 17 us without the fences, 8 us for the merges alone).
// The workgroup that counts a sequence's last group applies the rule in one
// wave, lane q = row q, with the same decisions as select_finalize_kernel.
constexpr int FGR_NT = 1024, FGR_ROWS = 8, FGR_T = FGR_NT / FGR_ROWS, FGR_U = 16;
static_assert(FGR_T == 128, "two waves per row below");

__global__ __launch_bounds__(FGR_NT) void select_finalize_group_kernel(SelArgs a) {
  __shared__ Red red_w[FGR_NT / 64];
  __shared__ float conf_s[64];
  __shared__ int tok_s[64];
  __shared__ int cand_s[64];
  __shared__ int last_s;
  if (gate_closed(a.gate)) return;
  const int ngrp = a.R / FGR_ROWS;
  const int b = blockIdx.x / ngrp, r0 = (blockIdx.x % ngrp) * FGR_ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = r0 + tid / FGR_T, t = tid % FGR_T;
  {
    const f32x4* prow = a.part + (size_t(b) * a.R + r) * a.NC;
    Red acc = red_empty();
    for (int c0 = t; c0 < a.NC; c0 += FGR_T * FGR_U) {
      f32x4 p[FGR_U];
#pragma unroll
      for (int u = 0; u < FGR_U; ++u) {
        const int c = c0 + u * FGR_T;
        p[u] = c < a.NC ? prow[c] : f32x4{-INFINITY, 0.f, __int_as_float(0x7fffffff), 0.f};
      }
#pragma unroll
      for (int u = 0; u < FGR_U; ++u) acc = combine(acc, unpack_red(p[u]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) acc = combine(acc, shfl_xor_red(acc, o));
    if (lane == 0) red_w[tid >> 6] = acc;
    __syncthreads();
    if (t == 0) {
      const Red res = combine(red_w[tid >> 6], red_w[(tid >> 6) + 1]);
      const size_t row = size_t(b) * a.R + r;
      a.token_out[row] = res.i;
      a.conf_out[row] = 1.f / res.s;
    }
    // the group's rows are written (the barrier waits for every wave's
    // stores); one release and one count for the whole group
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      last_s = atomicAdd(&a.cnt[b], 1) == ngrp - 1;
    }
    __syncthreads();
    if (!last_s) return;
    __threadfence();
  }
  if (tid >= 64) return;
  const int q = tid;
  const bool live = q < a.R;
  const size_t row = size_t(b) * a.R + q;
  const size_t srow = size_t(b) * a.sstride + q;
  float conf = 0.f;
  int tok = 0;
  bool cand = false;
  if (live) {
    conf = __hip_atomic_load(&a.conf_out[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok = __hip_atomic_load(&a.token_out[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    cand = a.masked[srow] != 0;
    conf_s[q] = conf;
    cand_s[q] = cand;
    tok_s[q] = tok;
  }
  __builtin_amdgcn_wave_barrier();
  int rank = 0;  // among candidates: decreasing confidence, lower row first on ties
  if (cand) {
    for (int p = 0; p < a.R; ++p) {
      if (!cand_s[p]) continue;
      const float cp = conf_s[p];
      rank += (cp > conf || (cp == conf && p < q)) ? 1 : 0;
    }
  }
  bool sel = false;
  if (a.mode == FDL_SELECT_THRESHOLD) {
    sel = cand && conf > a.tau[b];
    if (__builtin_amdgcn_ballot_w64(sel) == 0) sel = cand && rank == 0;  // fallback: the most confident candidate
  } else if (a.mode == FDL_SELECT_TOPK) {
    sel = cand && rank < a.k;
  } else {  // FDL_SELECT_FACTOR
    const int n = rank + 1;
    int best = cand && float(n + 1) * (1.f - conf) < a.factor ? n : 0;
    for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o, kWave));
    const int nstar = best > 0 ? best : 1;
    sel = cand && rank < nstar;
  }
  const int n_sel = __builtin_popcountll(__builtin_amdgcn_ballot_w64(sel));
  if (q == 0) {
    a.n_commit[b] = n_sel;
    a.cnt[b] = 0;
  }
  if (live) {
    a.commit_out[row] = sel ? 1 : 0;
    if (sel && a.tokens_inout) a.tokens_inout[srow] = tok_s[q];
    if (sel && a.masked_inout) a.masked_inout[srow] = 0;
  }
}

static void launch_finalize(const SelArgs& a, hipStream_t st) {
  if (a.B * a.R > 64 && a.R % FGR_ROWS == 0 && a.R <= 64)
    hipLaunchKernelGGL(select_finalize_group_kernel, dim3(a.B * (a.R / FGR_ROWS)), dim3(FGR_NT), 0, st, a);
  else
    hipLaunchKernelGGL(select_finalize_kernel, dim3(a.B * a.R), dim3(FIN_NT), 0, st, a);
}

// ---------------------------------------------------------------------------
// host side

static void select_plan(int rows, int V, int& nc, int& chunk) {
  const int target_wg = 2048;
  const int max_nc = (V + 1023) / 1024;
  nc = (target_wg + rows - 1) / rows;
  if (nc > max_nc) nc = max_nc;
  if (nc < 1) nc = 1;
  chunk = ((V + nc - 1) / nc + 1023) / 1024 * 1024;
  nc = (V + chunk - 1) / chunk;
}

// Partials [B*R][nc] (16 bytes each), then the per-sequence row counters.
size_t partials_workspace_bytes(const fdl_dims& d, int rows_per_seq, int nc) {
  const size_t part = size_t(d.batch) * rows_per_seq * nc * sizeof(f32x4);
  return part + (size_t(d.batch) * sizeof(int32_t) + 15) / 16 * 16;
}

int32_t* partials_counters(void* ws, const fdl_dims& d, int rows_per_seq, int nc) {
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) +
                                    size_t(d.batch) * rows_per_seq * nc * sizeof(f32x4));
}

size_t select_workspace_bytes(const fdl_dims& d, int rows_per_seq) {
  int nc, chunk;
  select_plan(d.batch * rows_per_seq, d.vocab, nc, chunk);
  return partials_workspace_bytes(d, rows_per_seq, nc);
}

// Finalize from partials produced elsewhere (the LM head's fused epilogue).
int select_finalize_launch(const fdl_dims& d, int R, const void* part, int nc, const uint8_t* masked,
                           const float* tau, int mode, int k, float factor, int32_t* token_out, float* conf_out,
                           uint8_t* commit_out, int32_t* n_commit, int32_t* tokens_inout, uint8_t* masked_inout,
                           hipStream_t st, int state_stride, const int32_t* gate) {
  SelArgs a;
  a.logits = nullptr; a.masked = masked; a.tau = tau;
  a.mode = mode; a.k = k; a.factor = factor;
  a.token_out = token_out; a.conf_out = conf_out; a.commit_out = commit_out; a.n_commit = n_commit;
  a.tokens_inout = tokens_inout; a.masked_inout = masked_inout;
  a.B = d.batch; a.R = R; a.V = d.vocab;
  a.NC = nc; a.chunk = 0;
  a.sstride = state_stride > 0 ? state_stride : R;
  a.gate = gate;
  a.part = reinterpret_cast<f32x4*>(const_cast<void*>(part));
  a.cnt = partials_counters(const_cast<void*>(part), d, R, nc);
  launch_finalize(a, st);
  return check_launch();
}

int select_launch(const fdl_dims& d, int R, const float* logits, const uint8_t* masked, const float* tau, int mode,
                  int k, float factor, int32_t* token_out, float* conf_out, uint8_t* commit_out, int32_t* n_commit,
                  int32_t* tokens_inout, uint8_t* masked_inout, void* ws, size_t ws_bytes, hipStream_t st) {
  SelArgs a;
  a.logits = logits; a.masked = masked; a.tau = tau;
  a.mode = mode; a.k = k; a.factor = factor;
  a.token_out = token_out; a.conf_out = conf_out; a.commit_out = commit_out; a.n_commit = n_commit;
  a.tokens_inout = tokens_inout; a.masked_inout = masked_inout;
  a.B = d.batch; a.R = R; a.V = d.vocab;
  a.sstride = R;
  a.gate = nullptr;
  select_plan(d.batch * R, d.vocab, a.NC, a.chunk);
  const size_t need = partials_workspace_bytes(d, R, a.NC);
  if (!ws || ws_bytes < need) return FDL_E_WORKSPACE;
  a.part = reinterpret_cast<f32x4*>(ws);
  a.cnt = partials_counters(ws, d, R, a.NC);
  const dim3 grid(a.NC, d.batch * R);
  if ((d.vocab & 3) == 0) hipLaunchKernelGGL(select_partial_kernel<true>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(select_partial_kernel<false>, grid, dim3(256), 0, st, a);
  launch_finalize(a, st);
  return check_launch();
}

}  // namespace fdl

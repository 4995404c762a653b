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
// Kernel 2, the finalize, merges a row's partials in a fixed order -- the
// result does not depend on scheduling -- and applies the selection rule per
// sequence, then writes the commit set and updates tokens/masked: one wave
// per row (the wave that counts a sequence's last row applies the rule) up to
// 256 rows, one workgroup per sequence beyond that, or, for more than 64 rows
// per sequence, one 256-thread workgroup per row.
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

// The selection rule over one sequence's rows in one wave, lane q = row q
// (R <= 64), from every row's confidence and candidate flag in LDS: rank
// among candidates by decreasing confidence, lower row first on ties; then
// the threshold with the single-most-confident fallback, the fixed count, or
// the factor rule -- the decisions of select_finalize_kernel.  Every lane of
// the wave takes part (ballots); lanes q >= R return false.
__device__ __forceinline__ bool wave_rule(const SelArgs& a, int q, bool live, bool cand, float conf, float tau,
                                          const float* conf_s, const int* cand_s) {
  int rank = 0;
  if (live && cand) {
    for (int p = 0; p < a.R; ++p) {
      if (!cand_s[p]) continue;
      const float cp = conf_s[p];
      rank += (cp > conf || (cp == conf && p < q)) ? 1 : 0;
    }
  }
  if (a.mode == FDL_SELECT_THRESHOLD) {
    const bool above = live && cand && conf > tau;
    if (__builtin_amdgcn_ballot_w64(above) != 0) return above;
    return live && cand && rank == 0;  // fallback: the most confident candidate
  }
  if (a.mode == FDL_SELECT_TOPK) return live && cand && rank < a.k;
  // FDL_SELECT_FACTOR
  const int n = rank + 1;
  int best = live && cand && float(n + 1) * (1.f - conf) < a.factor ? n : 0;
  for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o, kWave));
  const int nstar = best > 0 ? best : 1;
  return live && cand && rank < nstar;
}

// One workgroup of 1024 threads per sequence (R <= 64 rows), TPR threads per
// row: no device-scope synchronization at all.  Wave 0 fetches the rule's
// inputs (masked flags, tau) before the partials arrive.  Phase 1: each
// thread merges its share of the row's partials (max and lowest argmax first,
// then one exponential per partial), then a fixed xor butterfly over the
// row's lanes -- every lane ends with the same bits -- and, for rows wider
// than a wave, a fixed combination of the row's waves.  Phase 2: wave 0, lane
// q = row q, applies the rule from LDS, with the decisions of
// select_finalize_kernel.
constexpr int FSQ_NT = 1024, FSQ_U = 16;

// U partials of one thread (empty ones: -inf, 0, INT_MAX) -> (max, lowest
// argmax, sum of s exp(m - max))
template <int U>
__device__ __forceinline__ Red merge_run(const f32x4 (&p)[U]) {
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) mx = fmaxf(mx, p[u][0]);
  int im = INT_MAX;
  float sm = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const Red q = unpack_red(p[u]);
    if (q.m == mx) im = min(im, q.i);
    if (q.s > 0.f) sm += q.s * exp2f((q.m - mx) * kLog2e);
  }
  return Red{mx, sm, im};
}

// xor butterfly over groups of W lanes (W a power of two up to 64)
template <int W>
__device__ __forceinline__ Red butterfly_red(Red r) {
  float mx = r.m;
#pragma unroll
  for (int o = 1; o < W; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  int im = r.m == mx ? r.i : INT_MAX;
#pragma unroll
  for (int o = 1; o < W; o <<= 1) im = min(im, __shfl_xor(im, o, kWave));
  float sm = r.s > 0.f ? r.s * exp2f((r.m - mx) * kLog2e) : 0.f;
#pragma unroll
  for (int o = 1; o < W; o <<= 1) sm += __shfl_xor(sm, o, kWave);
  return Red{mx, sm, im};
}

template <int TPR>
__global__ __launch_bounds__(FSQ_NT) void select_finalize_seq_kernel(SelArgs a) {
  constexpr int ROWS = FSQ_NT / TPR, WPR = TPR > kWave ? TPR / kWave : 1;
  static_assert(ROWS <= 64, "one lane of wave 0 per row in the rule phase");
  __shared__ Red wred[FSQ_NT / kWave];
  __shared__ float conf_s[ROWS];
  __shared__ int tok_s[ROWS];
  __shared__ int cand_s[ROWS];
  if (gate_closed(a.gate)) return;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid / TPR, t = tid % TPR;
  const int q = lane;  // the row of this lane in the rule phase
  const bool live = wave == 0 && q < a.R;
  const size_t srow = size_t(b) * a.sstride + q;
  bool cand = false;
  float tau = 0.f;
  if (live) cand = a.masked[srow] != 0;
  if (wave == 0 && a.mode == FDL_SELECT_THRESHOLD) tau = a.tau[b];

  Red acc = red_empty();
  if (r < a.R) {
    const f32x4* prow = a.part + (size_t(b) * a.R + r) * a.NC;
    for (int c0 = t; c0 < a.NC; c0 += TPR * FSQ_U) {
      f32x4 p[FSQ_U];
#pragma unroll
      for (int u = 0; u < FSQ_U; ++u) {
        const int c = c0 + u * TPR;
        p[u] = c < a.NC ? prow[c] : f32x4{-INFINITY, 0.f, __int_as_float(INT_MAX), 0.f};
      }
      acc = combine(acc, merge_run(p));
    }
  }
  acc = butterfly_red<(TPR < kWave ? TPR : kWave)>(acc);
  if (WPR > 1) {
    if (lane == 0) wred[wave] = acc;
    __syncthreads();
    if (t == 0) {
      Red w = wred[wave];
      for (int j = 1; j < WPR; ++j) w = combine(w, wred[wave + j]);
      acc = w;
    }
  }
  if (t == 0 && r < a.R) {
    conf_s[r] = 1.f / acc.s;
    tok_s[r] = acc.i;
  }
  __syncthreads();
  if (wave != 0) return;

  const size_t row = size_t(b) * a.R + q;
  float conf = 0.f;
  if (live) {
    conf = conf_s[q];
    cand_s[q] = cand;
  }
  __builtin_amdgcn_wave_barrier();
  const bool sel = wave_rule(a, q, live, cand, conf, tau, conf_s, cand_s);
  const int n_sel = __builtin_popcountll(__builtin_amdgcn_ballot_w64(sel));
  if (q == 0) a.n_commit[b] = n_sel;
  if (live) {
    a.token_out[row] = tok_s[q];
    a.conf_out[row] = conf;
    a.commit_out[row] = sel ? 1 : 0;
    if (sel && a.tokens_inout) a.tokens_inout[srow] = tok_s[q];
    if (sel && a.masked_inout) a.masked_inout[srow] = 0;
  }
}

// One wave per row (R <= 64): the row's partials, FRW_U per lane in flight,
// merged as above with one butterfly; lane 0 writes the row's token and
// confidence and counts the row on its sequence's counter (zeroed by the
// producer of the partials), and the wave that counts the sequence's last row
// applies the rule, lane q = row q.  The rule's masked flags and tau are
// fetched at the start by every wave, so the last one only reloads the
// sequence's tokens and confidences.  No workgroup barrier anywhere.
constexpr int FRW_U = 20;

__global__ __launch_bounds__(kWave) void select_finalize_row_kernel(SelArgs a) {
  __shared__ float conf_s[64];
  __shared__ int cand_s[64];
  if (gate_closed(a.gate)) return;
  const int row_g = blockIdx.x;  // b * R + r
  const int b = row_g / a.R;
  const int lane = threadIdx.x;
  const int q = lane;
  const bool live = q < a.R;
  const size_t srow = size_t(b) * a.sstride + q;
  bool cand = false;
  float tau = 0.f;
  if (live) cand = a.masked[srow] != 0;
  if (a.mode == FDL_SELECT_THRESHOLD) tau = a.tau[b];

  Red acc = red_empty();
  const f32x4* prow = a.part + size_t(row_g) * a.NC;
  for (int c0 = lane; c0 < a.NC; c0 += kWave * FRW_U) {
    f32x4 p[FRW_U];
#pragma unroll
    for (int u = 0; u < FRW_U; ++u) {
      const int c = c0 + u * kWave;
      p[u] = c < a.NC ? prow[c] : f32x4{-INFINITY, 0.f, __int_as_float(INT_MAX), 0.f};
    }
    acc = combine(acc, merge_run(p));
  }
  acc = butterfly_red<kWave>(acc);
  int prev = 0;
  if (lane == 0) {
    a.token_out[row_g] = acc.i;
    a.conf_out[row_g] = 1.f / acc.s;
    // publish the row, then count it
    __threadfence();
    prev = atomicAdd(&a.cnt[b], 1);
  }
  prev = __shfl(prev, 0, kWave);
  if (prev != a.R - 1) return;
  __threadfence();

  const size_t row = size_t(b) * a.R + q;
  float conf = 0.f;
  int tok = 0;
  if (live) {
    conf = __hip_atomic_load(&a.conf_out[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tok = __hip_atomic_load(&a.token_out[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    conf_s[q] = conf;
    cand_s[q] = cand;
  }
  __builtin_amdgcn_wave_barrier();
  const bool sel = wave_rule(a, q, live, cand, conf, tau, conf_s, cand_s);
  const int n_sel = __builtin_popcountll(__builtin_amdgcn_ballot_w64(sel));
  if (q == 0) {
    a.n_commit[b] = n_sel;
    a.cnt[b] = 0;
  }
  if (live) {
    a.commit_out[row] = sel ? 1 : 0;
    if (sel && a.tokens_inout) a.tokens_inout[srow] = tok;
    if (sel && a.masked_inout) a.masked_inout[srow] = 0;
  }
}

// Up to 256 rows: one wave per row, so that the partials stream through as
// many CUs as there are rows (measured at 1278 partials per row: 4 x 8 rows
// 8.2 -> 6.5 us, 1 x 32 rows 9.9 -> 8.1 us against the 256-thread per-row
// kernel).  More rows (and R <= 64): one workgroup per sequence, no
// device-scope synchronization (16 x 32 rows of 1188 partials: 21.9 ->
// 12.9 us).  R > 64: the 256-thread per-row kernel.
static void launch_finalize(const SelArgs& a, hipStream_t st) {
  if (a.R > 64) {
    hipLaunchKernelGGL(select_finalize_kernel, dim3(a.B * a.R), dim3(FIN_NT), 0, st, a);
  } else if (a.B * a.R <= 256) {
    hipLaunchKernelGGL(select_finalize_row_kernel, dim3(a.B * a.R), dim3(kWave), 0, st, a);
  } else {
    int rp2 = 1;
    while (rp2 < a.R) rp2 *= 2;
    switch (FSQ_NT / rp2) {  // threads per row
      case 16: hipLaunchKernelGGL(select_finalize_seq_kernel<16>, dim3(a.B), dim3(FSQ_NT), 0, st, a); break;
      case 32: hipLaunchKernelGGL(select_finalize_seq_kernel<32>, dim3(a.B), dim3(FSQ_NT), 0, st, a); break;
      case 64: hipLaunchKernelGGL(select_finalize_seq_kernel<64>, dim3(a.B), dim3(FSQ_NT), 0, st, a); break;
      default: hipLaunchKernelGGL(select_finalize_seq_kernel<128>, dim3(a.B), dim3(FSQ_NT), 0, st, a); break;
    }
  }
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

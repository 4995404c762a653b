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
// Kernel 2 (one workgroup per sequence) merges the chunk partials of each row
// in chunk order -- the result does not depend on scheduling -- and applies
// the selection rule, then writes the commit set and updates tokens/masked.
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
};

struct Red {
  float m, s;
  int i;
};

// merge two (max, sum of exp relative to max, lowest argmax) triples
__device__ __forceinline__ Red combine(Red a, Red b) {
  Red r;
  r.m = fmaxf(a.m, b.m);
  const float ta = a.s > 0.f ? a.s * exp2f((a.m - r.m) * kLog2e) : 0.f;
  const float tb = b.s > 0.f ? b.s * exp2f((b.m - r.m) * kLog2e) : 0.f;
  r.s = ta + tb;
  r.i = (b.m > a.m || (b.m == a.m && b.i < a.i)) ? b.i : a.i;
  return r;
}

__device__ __forceinline__ void push(Red& r, float x, int v) {
  if (x > r.m) {
    r.s = r.s * exp2f((r.m - x) * kLog2e) + 1.f;
    r.m = x;
    r.i = v;
  } else {
    r.s += exp2f((x - r.m) * kLog2e);
  }
}

template <bool VEC>
__global__ __launch_bounds__(256) void select_partial_kernel(SelArgs a) {
  __shared__ Red sh[4];
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

// one workgroup per sequence: each wave merges the chunk partials of rows
// w, w+4, ... (lanes take chunks lane, lane+64, ... in order, then a fixed
// butterfly), then one thread per row (R <= 256) applies the selection rule.
__global__ __launch_bounds__(256) void select_finalize_kernel(SelArgs a) {
  __shared__ float conf_s[256];
  __shared__ int tok_s[256];
  __shared__ int cand_s[256];
  __shared__ int red_i[256];
  const int b = blockIdx.x, r = threadIdx.x;
  const int lane = r & 63, wave = r >> 6;
  for (int row_in = wave; row_in < a.R; row_in += 4) {
    const size_t row = size_t(b) * a.R + row_in;
    Red t{-INFINITY, 0.f, INT_MAX};
    for (int c = lane; c < a.NC; c += 64) {
      const f32x4 p = a.part[row * a.NC + c];
      t = combine(t, Red{p[0], p[1], __float_as_int(p[2])});
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      Red u{__shfl_xor(t.m, o, 64), __shfl_xor(t.s, o, 64), __shfl_xor(t.i, o, 64)};
      t = combine(t, u);
    }
    if (lane == 0) {
      conf_s[row_in] = 1.f / t.s;
      tok_s[row_in] = t.i;
    }
  }
  __syncthreads();
  const bool live = r < a.R;
  const size_t row = size_t(b) * a.R + r;
  float conf = 0.f;
  int tok = 0, cand = 0;
  if (live) {
    conf = conf_s[r];
    tok = tok_s[r];
    cand = a.masked[row] != 0;
    a.token_out[row] = tok;
    a.conf_out[row] = conf;
  }
  cand_s[r] = live ? cand : 0;
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
  bool sel = false;
  if (a.mode == FDL_SELECT_THRESHOLD) {
    const float tau = a.tau[b];
    sel = live && cand && conf > tau;
    red_i[r] = sel ? 1 : 0;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (r < o) red_i[r] += red_i[r + o];
      __syncthreads();
    }
    const int n_above = red_i[0];
    if (n_above == 0) sel = live && cand && rank == 0;  // fallback: the most confident candidate
  } else if (a.mode == FDL_SELECT_TOPK) {
    sel = live && cand && rank < a.k;
  } else {  // FDL_SELECT_FACTOR
    const int n = rank + 1;
    const bool ok = live && cand && float(n + 1) * (1.f - conf) < a.factor;
    red_i[r] = ok ? n : 0;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (r < o) red_i[r] = max(red_i[r], red_i[r + o]);
      __syncthreads();
    }
    const int nstar = red_i[0] > 0 ? red_i[0] : 1;
    sel = live && cand && rank < nstar;
  }
  __syncthreads();
  red_i[r] = sel ? 1 : 0;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (r < o) red_i[r] += red_i[r + o];
    __syncthreads();
  }
  if (r == 0) a.n_commit[b] = red_i[0];
  if (live) {
    a.commit_out[row] = sel ? 1 : 0;
    if (sel && a.tokens_inout) a.tokens_inout[row] = tok;
    if (sel && a.masked_inout) a.masked_inout[row] = 0;
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

size_t select_workspace_bytes(const fdl_dims& d, int rows_per_seq) {
  int nc, chunk;
  select_plan(d.batch * rows_per_seq, d.vocab, nc, chunk);
  return size_t(d.batch) * rows_per_seq * nc * sizeof(f32x4);
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
  select_plan(d.batch * R, d.vocab, a.NC, a.chunk);
  const size_t need = size_t(d.batch) * R * a.NC * sizeof(f32x4);
  if (!ws || ws_bytes < need) return FDL_E_WORKSPACE;
  a.part = reinterpret_cast<f32x4*>(ws);
  const dim3 grid(a.NC, d.batch * R);
  if ((d.vocab & 3) == 0) hipLaunchKernelGGL(select_partial_kernel<true>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(select_partial_kernel<false>, grid, dim3(256), 0, st, a);
  hipLaunchKernelGGL(select_finalize_kernel, dim3(d.batch), dim3(256), 0, st, a);
  return check_launch();
}

}  // namespace fdl

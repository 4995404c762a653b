// Decode loop: a whole generation of a batch with its control on the device.
//
// "Fast-dLLM v2: Efficient Block-Diffusion LLM", Inference Pipeline: blocks
// are generated left to right (Level 1); a block starts fully masked and is
// refined step after step, sub-block by sub-block, until no position is
// masked (Level 2; "Sub-block size as a decoding granularity knob"); its K/V
// then enter the block-level cache (Level 3); a sequence stops once a finished
// block holds EOS, and the batch advances in lock step with padding blocks
// for stopped sequences ("Batch decoding with length padding").  In the v1
// DualCache mode ("Fast-dLLM: Reusing Bidirectional State ...", section 3,
// Algorithm 1) the cache is refreshed at every block start instead of
// appended at its end.
//
// gfx950 design: nothing is read back to the host.  The host enqueues a fixed
// schedule of step slots -- as many per sub-block as the selection rule can
// need -- and a one-workgroup control kernel in front of every slot writes a
// gate word: 1 while some sequence still has a masked row in the active
// sub-block.  Every kernel of the slot (embedding, attention, merge, hidden
// rows, LM head, select) reads that word first and returns at once when it is
// 0, so a finished sub-block costs only the empty launches of its spare slots.
//
// The transformer is a synthetic stand-in whose inputs to each step are
// functions of the current tokens (the weight w doubles as the token
// embedding, H = Hq * d): e(t) = sqrt(H) w[t]; query head h = e(t)[h d, +d);
// key head g = e(t)[g d, +d); value head g = e(t)[H - (Hkv-g) d, +d) reversed;
// hidden row = gain * attention output + beta w[t'] / |w[t']|^2.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace fdl {

// control words at the head of the workspace
enum { C_GATE_BLOCK = 0, C_GATE_STEP = 1, C_STEPS = 2, C_BLOCKS = 3, C_CUR = 4, C_DONE = 5 };

struct DecArgs {
  int32_t* tokens;     // [B][cap]
  uint8_t* masked;     // [B][cap]
  int32_t* len;        // [B]
  int32_t* seq_steps;  // [B]
  int32_t* eos_block;  // [B]
  int32_t* ctl;        // control words, then done[B]
  const int32_t* prompt;
  int B, P, cap, D, S, V, mask_id, eos_id, dual;
};

// 16-byte chunks of float or bfloat16 elements, widened to float
template <typename T>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int E = 4;
  __device__ static void load(const float* p, float* v) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  }
  __device__ static void store(float* p, const float* v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  }
};
template <>
struct Chunk<bf16_t> {
  static constexpr int E = 8;
  __device__ static void load(const bf16_t* p, float* v) {
    const u32x4 u = ld16(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(bf16_t(u[j] & 0xffffu));
      v[2 * j + 1] = bf16_to_f32(bf16_t(u[j] >> 16));
    }
  }
  __device__ static void store(bf16_t* p, const float* v) {
    u32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    st16(p, u);
  }
};

// ---------------------------------------------------------------------------
// control kernels (one workgroup each)

__global__ __launch_bounds__(256) void dec_init_kernel(DecArgs a) {
  const int b = blockIdx.y;
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < a.cap) {
    int t = a.mask_id;
    if (p < a.P) {
      const int u = a.prompt[size_t(b) * a.P + p];
      t = (u >= 0 && u < a.V) ? u : a.mask_id;
    }
    a.tokens[size_t(b) * a.cap + p] = t;
    a.masked[size_t(b) * a.cap + p] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.seq_steps[b] = 0;
    a.eos_block[b] = -1;
    a.ctl[C_DONE + b] = 0;
    a.len[b] = a.dual ? a.cap : a.P;  // DualCache: every position is written by block 0's refresh
    if (b == 0) {
      a.ctl[C_GATE_BLOCK] = 1;
      a.ctl[C_GATE_STEP] = 0;
      a.ctl[C_STEPS] = 0;
      a.ctl[C_BLOCKS] = 0;
      a.ctl[C_CUR] = 0;
    }
  }
}

// Block start: live sequences get D masked positions, stopped ones padding.
__global__ __launch_bounds__(256) void dec_block_begin_kernel(DecArgs a, int blk) {
  int live = 0;
  for (int b = threadIdx.x; b < a.B; b += 256) live |= a.ctl[C_DONE + b] == 0;
  for (int idx = threadIdx.x; idx < a.B * a.D; idx += 256) {
    const int b = idx / a.D, j = idx % a.D;
    const size_t p = size_t(b) * a.cap + a.P + size_t(blk) * a.D + j;
    a.tokens[p] = a.mask_id;
    a.masked[p] = a.ctl[C_DONE + b] == 0 ? 1 : 0;
  }
  live = __syncthreads_or(live);
  if (threadIdx.x == 0) {
    a.ctl[C_GATE_BLOCK] = live;
    a.ctl[C_GATE_STEP] = 0;
    if (live) a.ctl[C_BLOCKS] += 1;
  }
}

// Block end: a live sequence whose finished block holds EOS stops.
__global__ __launch_bounds__(256) void dec_block_end_kernel(DecArgs a, int blk) {
  if (gate_closed(a.ctl + C_GATE_BLOCK)) return;
  for (int b = threadIdx.x; b < a.B; b += 256) {
    if (a.ctl[C_DONE + b]) continue;
    const int32_t* tk = a.tokens + size_t(b) * a.cap + a.P + size_t(blk) * a.D;
    int eos = 0;
    for (int j = 0; j < a.D; ++j) eos |= tk[j] == a.eos_id;
    if (eos) {
      a.ctl[C_DONE + b] = 1;
      a.eos_block[b] = blk;
    }
  }
}

__global__ void dec_finish_kernel(const int32_t* ctl, int32_t* counters) {
  if (threadIdx.x == 0) {
    counters[0] = ctl[C_STEPS];
    counters[1] = ctl[C_BLOCKS];
  }
}

struct TraceArgs {
  int32_t* meta;
  int32_t* tokens;
  uint8_t* masked;
  int32_t* token;
  float* conf;
  int cap;
  const int32_t* tok_out;
  const float* conf_out;
};

__global__ __launch_bounds__(256) void dec_trace_kernel(DecArgs a, TraceArgs t, int blk, int sub) {
  if (gate_closed(a.ctl + C_GATE_STEP)) return;
  const int n = a.ctl[C_CUR];
  if (n < 0 || n >= t.cap) return;
  if (threadIdx.x == 0) {
    t.meta[2 * n] = blk;
    t.meta[2 * n + 1] = sub;
  }
  for (int idx = threadIdx.x; idx < a.B * a.D; idx += 256) {
    const int b = idx / a.D, j = idx % a.D;
    const size_t p = size_t(b) * a.cap + a.P + size_t(blk) * a.D + j;
    const size_t q = (size_t(n) * a.B + b) * a.D + j;
    t.tokens[q] = a.tokens[p];
    t.masked[q] = a.masked[p];
  }
  for (int idx = threadIdx.x; idx < a.B * a.S; idx += 256) {
    const size_t q = size_t(n) * a.B * a.S + idx;
    t.token[q] = t.tok_out[idx];
    t.conf[q] = t.conf_out[idx];
  }
}

// ---------------------------------------------------------------------------
// stand-in model kernels

struct EmbedArgs {
  const void* w;          // [V][H]
  const int32_t* tokens;  // [B][cap]
  int cap, V, H, Hkv, dh, mask_id;
  float scale;            // sqrt(H)
  int pos0;               // embed positions pos0 .. pos0 + gridDim.x - 1 of every sequence
  void* kd;               // K destination [B][Hkv][dcap][dh] at dpos0 + i, or null
  void* vd;               // V destination, same layout, or null
  int dcap, dpos0;
  void* qd;               // Q destination [B][nq][H] for positions qpos0 .. qpos0 + nq - 1, or null
  int qpos0, nq;
  const int32_t* gate;
  // a step slot's embedding also opens the slot: non-null ctl, then the
  // active sub-block's rows start at step_off in every sequence's [cap]
  // masked flags (only live sequences have masked rows)
  int32_t* ctl;
  const uint8_t* masked;
  int32_t* seq_steps;
  int B, S, step_off;
};

// Whether some sequence has a masked row in the active sub-block (the step
// slot's gate); with `count`, also the bookkeeping of an opened slot.  Every
// workgroup of the step's embedding evaluates the gate itself; workgroup
// (0, 0) alone writes the gate word the slot's later kernels read and the
// step counters.
__device__ __forceinline__ bool step_open(const EmbedArgs& a, bool count) {
  __shared__ int any_s;
  if (threadIdx.x < 64) {
    int any = 0;
    for (int b = threadIdx.x; b < a.B; b += 64) {
      const uint8_t* m = a.masked + size_t(b) * a.cap + a.step_off;
      int live = 0;
      for (int i = 0; i < a.S; ++i) live |= m[i];
      if (count && live) a.seq_steps[b] += 1;
      any |= live;
    }
    any = __builtin_amdgcn_ballot_w64(any != 0) != 0;
    if (threadIdx.x == 0) {
      any_s = any;
      if (count) {
        a.ctl[C_GATE_STEP] = any;
        if (any) {
          a.ctl[C_CUR] = a.ctl[C_STEPS];
          a.ctl[C_STEPS] += 1;
        }
      }
    }
  }
  __syncthreads();
  return any_s != 0;
}

// One workgroup per (position, sequence): the token's embedding row is read
// once and scattered to its query, key and (reversed) value slices.
template <typename T>
__global__ __launch_bounds__(256) void sm_embed_kernel(EmbedArgs a) {
  if (a.ctl) {
    if (!step_open(a, blockIdx.x == 0 && blockIdx.y == 0)) return;
  } else if (gate_closed(a.gate)) {
    return;
  }
  typedef Chunk<T> C;
  constexpr int E = C::E;
  const int i = blockIdx.x, b = blockIdx.y;
  const int p = a.pos0 + i;
  int t = a.tokens[size_t(b) * a.cap + p];
  if (t < 0 || t >= a.V) t = a.mask_id;
  const T* wr = reinterpret_cast<const T*>(a.w) + size_t(t) * a.H;
  const int kvw = a.Hkv * a.dh, voff = a.H - kvw;
  const bool has_q = a.qd != nullptr && p >= a.qpos0 && p < a.qpos0 + a.nq;
  T* qd = reinterpret_cast<T*>(a.qd);
  T* kd = reinterpret_cast<T*>(a.kd);
  T* vd = reinterpret_cast<T*>(a.vd);
  for (int c = threadIdx.x; c < a.H / E; c += 256) {
    const int e0 = c * E;
    float v[E];
    C::load(wr + e0, v);
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] *= a.scale;
    if (has_q) C::store(qd + (size_t(b) * a.nq + (p - a.qpos0)) * a.H + e0, v);
    if (kd && e0 < kvw) {
      const int g = e0 / a.dh, j = e0 % a.dh;
      C::store(kd + ((size_t(b) * a.Hkv + g) * a.dcap + a.dpos0 + i) * a.dh + j, v);
    }
    if (vd && e0 >= voff) {
      const int g = (e0 - voff) / a.dh, j = (e0 - voff) % a.dh;
      float r[E];
#pragma unroll
      for (int m = 0; m < E; ++m) r[m] = v[E - 1 - m];
      C::store(vd + ((size_t(b) * a.Hkv + g) * a.dcap + a.dpos0 + i) * a.dh + (a.dh - E - j), r);
    }
  }
}

struct MixArgs {
  const void* o;        // [B*S][H] attention output (heads concatenated)
  const void* w;        // [V][H]
  void* x;              // [B*S][H] hidden rows
  const int32_t* btok;  // [B][L]
  const float* bval;    // [B][L]
  int S, L, V, H, r0;   // r0: generated-position index of the active sub-block's row 0
  float gain;
  const int32_t* gate;
};

// One workgroup per row: |w[t]|^2 by a block reduction, then
// x = gain * o + beta / |w[t]|^2 * w[t].
template <typename T>
__global__ __launch_bounds__(256) void sm_mix_kernel(MixArgs a) {
  if (gate_closed(a.gate)) return;
  typedef Chunk<T> C;
  constexpr int E = C::E;
  __shared__ float red[4];
  const int row = blockIdx.x, b = row / a.S, i = row % a.S;
  const size_t gp = size_t(b) * a.L + a.r0 + i;
  const int t = a.btok[gp];
  const bool boosted = t >= 0 && t < a.V;
  const T* wr = reinterpret_cast<const T*>(a.w) + size_t(boosted ? t : 0) * a.H;
  const T* orow = reinterpret_cast<const T*>(a.o) + size_t(row) * a.H;
  T* xrow = reinterpret_cast<T*>(a.x) + size_t(row) * a.H;
  float ss = 0.f;
  for (int c = threadIdx.x; c < a.H / E; c += 256) {
    float v[E];
    C::load(wr + c * E, v);
#pragma unroll
    for (int j = 0; j < E; ++j) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float coef = (boosted && ss > 0.f) ? a.bval[gp] / ss : 0.f;
  for (int c = threadIdx.x; c < a.H / E; c += 256) {
    float v[E], o[E];
    C::load(wr + c * E, v);
    C::load(orow + c * E, o);
#pragma unroll
    for (int j = 0; j < E; ++j) o[j] = fmaf(a.gain, o[j], coef * v[j]);
    C::store(xrow + c * E, o);
  }
}

// ---------------------------------------------------------------------------
// host side

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct DecLayout {
  size_t ctl, q, kb, vb, o, x, part, attn, tok, conf, commit, ncommit, total;
};

static DecLayout decode_layout(const fdl_dims& d) {
  const size_t es = dtype_size(d.dtype);
  const size_t rows = size_t(d.batch) * d.sub_block;
  DecLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.ctl = take(sizeof(int32_t) * (C_DONE + size_t(d.batch)));
  L.q = take(rows * d.hidden * es);
  L.kb = take(size_t(d.batch) * d.n_kv_heads * d.block * d.head_dim * es);
  L.vb = take(size_t(d.batch) * d.n_kv_heads * d.block * d.head_dim * es);
  L.o = take(rows * d.hidden * es);
  L.x = take(rows * d.hidden * es);
  L.part = take(partials_workspace_bytes(d, d.sub_block, lm_head_tiles(d, d.batch * d.sub_block)));
  L.attn = take(attn_workspace_bytes(d));
  L.tok = take(rows * sizeof(int32_t));
  L.conf = take(rows * sizeof(float));
  L.commit = take(rows);
  L.ncommit = take(size_t(d.batch) * sizeof(int32_t));
  L.total = off;
  return L;
}

size_t decode_workspace_bytes(const fdl_dims& d) { return decode_layout(d).total; }

int decode_slots_per_sub(const fdl_dims& d, int mode, int k) {
  return mode == FDL_SELECT_TOPK ? (d.sub_block + k - 1) / k : d.sub_block;
}

template <typename T>
static void launch_embed(const EmbedArgs& e, int n, int B, hipStream_t st) {
  hipLaunchKernelGGL(sm_embed_kernel<T>, dim3(n, B), dim3(256), 0, st, e);
}

int decode_launch(const fdl_dims& d, const fdl_decode_args& g, void* ws, hipStream_t st) {
  const DecLayout lay = decode_layout(d);
  char* base = reinterpret_cast<char*>(ws);
  int32_t* ctl = reinterpret_cast<int32_t*>(base + lay.ctl);
  void* q = base + lay.q;
  void* kb = base + lay.kb;
  void* vb = base + lay.vb;
  void* o = base + lay.o;
  void* x = base + lay.x;
  void* part = base + lay.part;
  void* attn_ws = base + lay.attn;
  int32_t* tok_out = reinterpret_cast<int32_t*>(base + lay.tok);
  float* conf_out = reinterpret_cast<float*>(base + lay.conf);
  uint8_t* commit_out = reinterpret_cast<uint8_t*>(base + lay.commit);
  int32_t* n_commit = reinterpret_cast<int32_t*>(base + lay.ncommit);
  const int32_t* gate_block = ctl + C_GATE_BLOCK;
  const int32_t* gate_step = ctl + C_GATE_STEP;

  const int B = d.batch, P = d.prompt_len, L = d.gen_len, D = d.block, S = d.sub_block;
  const int cap = P + L, dual = d.attn_mode == FDL_ATTN_DUAL_CACHE;
  const int nblocks = g.max_blocks > 0 ? g.max_blocks : L / D;
  const int slots = decode_slots_per_sub(d, g.mode, g.k);
  const bool bf = d.dtype == FDL_BF16;
  const int nc = lm_head_tiles(d, d.batch * d.sub_block);

  DecArgs a;
  a.tokens = g.tokens; a.masked = g.masked; a.len = g.len; a.seq_steps = g.seq_steps; a.eos_block = g.eos_block;
  a.ctl = ctl; a.prompt = g.prompt;
  a.B = B; a.P = P; a.cap = cap; a.D = D; a.S = S; a.V = d.vocab;
  a.mask_id = g.mask_id; a.eos_id = g.eos_id; a.dual = dual;

  EmbedArgs e;
  e.ctl = nullptr; e.masked = nullptr; e.seq_steps = nullptr; e.B = B; e.S = S; e.step_off = 0;
  e.w = g.w; e.tokens = g.tokens;
  e.cap = cap; e.V = d.vocab; e.H = d.hidden; e.Hkv = d.n_kv_heads; e.dh = d.head_dim; e.mask_id = g.mask_id;
  e.scale = sqrtf(float(d.hidden));
  auto embed = [&](int pos0, int n, void* kd, void* vd, int dcap, int dpos0, void* qd, int qpos0, int nq,
                   const int32_t* gate, int step_off = -1) {
    EmbedArgs ee = e;
    ee.pos0 = pos0; ee.kd = kd; ee.vd = vd; ee.dcap = dcap; ee.dpos0 = dpos0;
    ee.qd = qd; ee.qpos0 = qpos0; ee.nq = nq; ee.gate = gate;
    if (step_off >= 0) ee.ctl = ctl, ee.masked = g.masked, ee.seq_steps = g.seq_steps, ee.step_off = step_off;
    if (bf) launch_embed<bf16_t>(ee, n, B, st);
    else launch_embed<float>(ee, n, B, st);
  };

  MixArgs m;
  m.o = o; m.w = g.w; m.x = x; m.btok = g.boost_tok; m.bval = g.boost_val;
  m.S = S; m.L = L; m.V = d.vocab; m.H = d.hidden; m.gain = g.gain; m.gate = gate_step;

  TraceArgs t;
  t.meta = g.trace_meta; t.tokens = g.trace_tokens; t.masked = g.trace_masked;
  t.token = g.trace_token; t.conf = g.trace_conf; t.cap = g.trace_cap;
  t.tok_out = tok_out; t.conf_out = conf_out;
  const bool trace = g.trace_meta != nullptr;

  hipLaunchKernelGGL(dec_init_kernel, dim3((cap + 255) / 256, B), dim3(256), 0, st, a);
  if (!dual && P > 0) embed(0, P, g.k_cache, g.v_cache, cap, 0, nullptr, 0, 0, nullptr);
  int rc = check_launch();
  if (rc != FDL_OK) return rc;

  for (int blk = 0; blk < nblocks; ++blk) {
    const int bstart = P + blk * D;
    hipLaunchKernelGGL(dec_block_begin_kernel, dim3(1), dim3(256), 0, st, a, blk);
    if (dual) embed(0, cap, g.k_cache, g.v_cache, cap, 0, nullptr, 0, 0, gate_block);  // refresh
    for (int sub = 0; sub < D / S; ++sub) {
      const int r0 = blk * D + sub * S;
      m.r0 = r0;
      for (int it = 0; it < slots; ++it) {
        // the step's embedding opens the slot: the gate of the slot's later
        // kernels and the step counters
        embed(bstart, D, kb, vb, D, 0, q, P + r0, S, gate_step, P + r0);
        rc = attn_launch(d, blk, q, g.k_cache, g.v_cache, nullptr, kb, vb, o, nullptr, attn_ws,
                         attn_workspace_bytes(d), st, gate_step);
        if (rc != FDL_OK) return rc;
        if (bf) hipLaunchKernelGGL(sm_mix_kernel<bf16_t>, dim3(B * S), dim3(256), 0, st, m);
        else hipLaunchKernelGGL(sm_mix_kernel<float>, dim3(B * S), dim3(256), 0, st, m);
        rc = lm_head_launch(d, B * S, x, g.w, nullptr, part, st, gate_step);
        if (rc != FDL_OK) return rc;
        rc = select_finalize_launch(d, S, part, nc, g.masked + P + r0, g.tau, g.mode, g.k, g.factor, tok_out,
                                    conf_out, commit_out, n_commit, g.tokens + P + r0, g.masked + P + r0, st, cap,
                                    gate_step);
        if (rc != FDL_OK) return rc;
        if (trace) hipLaunchKernelGGL(dec_trace_kernel, dim3(1), dim3(256), 0, st, a, t, blk, sub);
      }
    }
    if (!dual) {
      // the finished block's K/V enter the block-level cache
      embed(bstart, D, kb, vb, D, 0, nullptr, 0, 0, gate_block);
      rc = append_launch(d, g.k_cache, g.v_cache, kb, vb, D, g.len, st, gate_block);
      if (rc != FDL_OK) return rc;
    }
    hipLaunchKernelGGL(dec_block_end_kernel, dim3(1), dim3(256), 0, st, a, blk);
    rc = check_launch();
    if (rc != FDL_OK) return rc;
  }
  hipLaunchKernelGGL(dec_finish_kernel, dim3(1), dim3(64), 0, st, ctl, g.counters);
  return check_launch();
}

}  // namespace fdl

// Multi-block attention: many query positions over one K/V sequence, either
// block-causal (the prompt prefill of a block-diffusion model: query position
// p sees every key in its own block and all earlier blocks, the M_BC pattern
// of "Fast-dLLM v2: Efficient Block-Diffusion LLM", Attention Mask Design) or
// fully bidirectional (the per-block refresh of the Fast-dLLM v1 caches,
// "Fast-dLLM: Reusing Bidirectional State ...", Algorithm 1, and the
// PrefixCache recomputation of section 3).  eq 3 of the latter page.
//
// gfx950 design: a workgroup of 4 waves owns 128 consecutive query positions
// of one query head; each wave 32 of them, on 32x32x16 bf16 MFMA in the same
// S^T = K Q^T / O^T = V^T P^T orientation as the block attention kernel, with
// its K/V path: 64-key tiles HBM -> LDS by direct-to-LDS loads (a tile wholly
// below the workgroup's key limit from one wave-uniform base plus per-lane
// offsets), K rows swizzled for conflict-free fragment reads, V^T operands
// from transposing LDS reads, two LDS stages (64 KB at d = 128: two
// workgroups per CU) with the next tile's loads in flight while one is
// consumed.  The workgroup walks the keys its last position may see; each
// lane masks the keys beyond its own position's block.  The work is
// MFMA-bound (AI in the hundreds of flop/B), so heads are not grouped: the G
// query heads of a KV head re-read its K/V from L2.  Two waves per SIMD (two
// workgroups per CU): one wave's softmax overlaps the other's MFMA work,
// which a single wave per SIMD cannot do across its own dependent
// S -> P -> O chain.
#include "common.h"
#include "kv_tiles.h"

namespace fdl {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int B, Hq, Hkv, G, nq, q_start, n_keys, cap, D, causal;
  float scale_log2;
};

constexpr int PF_TK = 64;

template <int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_bf16_kernel(
    PrefillArgs a) {
  typedef bf16_t T;
  constexpr int NW = 4, TK = PF_TK, NS = 2;
  constexpr int ROWB = DH * 2;         // bytes per key row
  constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  constexpr int KPI = 1024 / ROWB;     // key rows per 1 KB load instruction
  constexpr int TILEB = TK * ROWB;     // one K (or V) tile
  constexpr int STB = 2 * TILEB;       // one stage: K tile, then V tile
  constexpr int IPH = TILEB / 1024;    // load instructions per K (or V) tile
  constexpr int IPW = 2 * IPH / NW;    // load instructions per wave per stage
  static_assert(IPH % IPW == 0, "a wave loads only K or only V");
  constexpr int KSTEPS = DH / 16, DT = DH / 32;
  __shared__ __attribute__((aligned(1024))) char smem[NS * STB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int hq = blockIdx.y, b = blockIdx.z;
  const int g = hq / a.G;
  const int qi = blockIdx.x * 128 + wave * 32 + l32;          // this lane's query column
  const bool qok = qi < a.nq;
  const int qi_last = min(a.nq - 1, int(blockIdx.x) * 128 + 127);
  auto key_limit = [&](int pos_index) {
    if (!a.causal) return a.n_keys;
    const int p = a.q_start + pos_index;
    return min(a.n_keys, (p / a.D + 1) * a.D);
  };
  const int k_end = key_limit(qi_last);
  const int lim = qok ? key_limit(qi) : 0;
  const size_t kvbase = (size_t(b) * a.Hkv + g) * a.cap * DH;
  const T* K = reinterpret_cast<const T*>(a.k) + kvbase;
  const T* V = reinterpret_cast<const T*>(a.v) + kvbase;

  // this lane's share of the wave's load instructions (see the block attention)
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool wave_v = wave_s * IPW >= IPH;
  const T* const my_src = pick(wave_v, V, K);
  int ld_row[IPW], ld_lds[IPW];
  uint32_t ld_voff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int i = wave_s * IPW + j - (wave_v ? IPH : 0);
    const int row = KPI * i + lane / CPR;
    const int c = (lane % CPR) ^ (wave_v ? swz_v<DH>(row) : swz_k<DH>(row));
    ld_row[j] = row;
    ld_lds[j] = (wave_v ? TILEB : 0) + i * 1024;
    ld_voff[j] = uint32_t(row * DH + c * 8) * uint32_t(sizeof(T));
  }
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * TK;
    char* sb = smem + (t % NS) * STB;
    if (key0 + TK <= k_end) {
      const char* const tb = reinterpret_cast<const char*>(my_src + size_t(key0) * DH);
#pragma unroll
      for (int j = 0; j < IPW; ++j) load_lds16_s(tb, ld_voff[j], sb + ld_lds[j]);
      return;
    }
    // the last tile: rows past the workgroup's key limit read its last key
    // (their scores are masked)
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int key = min(key0 + ld_row[j], k_end - 1);
      load_lds16(reinterpret_cast<const char*>(my_src + size_t(key) * DH) + (ld_voff[j] - ld_row[j] * ROWB),
                 sb + ld_lds[j]);
    }
  };
  int koff[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + h) ^ swz_k<DH>(l32)) << 4);
  int voff[DT];
  {
    const int grp = lane >> 4, sl = lane & 15, e = sl >> 2, qq = sl & 3;
    const int row = 4 * (grp >> 1) + e;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + 16 * (grp & 1) + 4 * qq;
      voff[dt] = row * ROWB + (((d >> 3) ^ swz_v<DH>(row)) << 4) + (d & 7) * 2;
    }
  }

  u32x4 qf[KSTEPS];
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = -INFINITY;
  float lw[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's share of the row sum, four chains
  const float c = a.scale_log2;

  auto compute_tile = [&](int t) __attribute__((always_inline)) {
    const int key0 = t * TK;
    const char* Ks = smem + (t % NS) * STB;
    const char* Vs = Ks + TILEB;
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(Ks + kt * 32 * ROWB + koff[ks]);
        s[kt] = mfma32x32x16_bf16(kf, qf[ks], s[kt]);
      }
    // keys beyond this lane's position's block (or the sequence) do not exist for it
    if (key0 + TK > lim) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (key0 + kt * 32 + (v / 4) * 8 + h * 4 + (v % 4) >= lim) s[kt][v] = -INFINITY;
    }
    float mq[4];
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int kt = qd >> 1, v0 = (qd & 1) * 8;
      mq[qd] = fmaxf(fmaxf(s[kt][v0], s[kt][v0 + 1]), s[kt][v0 + 2]);
      mq[qd] = fmaxf(fmaxf(mq[qd], s[kt][v0 + 3]), s[kt][v0 + 4]);
      mq[qd] = fmaxf(fmaxf(mq[qd], s[kt][v0 + 5]), s[kt][v0 + 6]);
      mq[qd] = fmaxf(mq[qd], s[kt][v0 + 7]);
    }
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx = xor32_max(mx) * c;
    // lazy rescale (see the block attention kernel); a fully masked tile
    // (mx = -inf) leaves the state untouched
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int w = 0; w < 4; ++w) lw[w] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = mn;
    }
    // a lane that has seen no key yet (only one past the sequence: its
    // scores are all -inf) gets P = 0
    const float mneg = m == -INFINITY ? 0.f : -m;
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 pf;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * q + 2 * w], c, mneg));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][8 * q + 2 * w + 1], c, mneg));
          // (a named value: a bit cast of the vector element pf[w] reads element 0)
          const uint32_t pw = pack_bf16x2(p0, p1);
          pf[w] = pw;
          lw[w] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw), ones, lw[w], false);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const char* vb0 = Vs + (kt * 32 + q * 16) * ROWB + voff[dt];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vb0));
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vb0 + 8 * ROWB));
          const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 vf{lo2[0], lo2[1], hi2[0], hi2[1]};
          o[dt] = mfma32x32x16_bf16(vf, pf, o[dt]);
        }
      }
  };

  const int ntiles = (k_end + TK - 1) / TK;
  issue(0);
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t(b) * a.nq + (qok ? qi : 0)) * a.Hq + hq) * DH;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = qok ? ld16(qp + ks * 16 + 8 * h) : u32x4{0, 0, 0, 0};
  }
  for (int t = 0; t < ntiles; ++t) {
    // this wave's loads of tile t (the only ones in flight) are done; after the
    // barrier every wave's are, and every wave is done with tile t - 1, whose
    // stage the loads of tile t + 1 then refill
    wait_vm<0>();
    bare_barrier();
    if (t + 1 < ntiles) issue(t + 1);
    compute_tile(t);
  }
  const float l = xor32_sum((lw[0] + lw[1]) + (lw[2] + lw[3]));  // both half-waves' shares of the row sum
  if (!qok) return;
  const float inv = 1.f / l;
  T* op = reinterpret_cast<T*>(a.out) + ((size_t(b) * a.nq + qi) * a.Hq + hq) * DH;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 w;
      w[0] = pack_bf16x2(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv);
      w[1] = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + dt * 32 + q4 * 8 + h * 4) = w;
    }
  if (a.lse && h == 0) a.lse[(size_t(b) * a.Hq + hq) * a.nq + qi] = (m + __log2f(l)) * kLn2;
}

int prefill_launch(const fdl_dims& d, int q_start, int n_q, int n_keys, int causal, const void* q, const void* k,
                   const void* v, void* out, float* lse, hipStream_t st) {
  PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.B = d.batch; a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads; a.G = d.n_q_heads / d.n_kv_heads;
  a.nq = n_q; a.q_start = q_start; a.n_keys = n_keys; a.cap = d.prompt_len + d.gen_len; a.D = d.block;
  a.causal = causal;
  a.scale_log2 = kLog2e / sqrtf(float(d.head_dim));
  const dim3 grid((n_q + 127) / 128, d.n_q_heads, d.batch);
  if (d.head_dim == 128) hipLaunchKernelGGL(prefill_attn_bf16_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(prefill_attn_bf16_kernel<64>, grid, dim3(256), 0, st, a);
  return check_launch();
}

}  // namespace fdl

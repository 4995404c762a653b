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
// S^T = K Q^T / O^T = V^T P^T orientation as the block attention kernel.  The
// workgroup walks the keys its last position may see in 64-key tiles staged
// through a double-buffered LDS (V transposed on the way in); each lane masks
// the keys beyond its own position's block.  The work is MFMA-bound (AI in
// the hundreds of flop/B), so heads are not grouped: the G query heads of a
// KV head re-read its K/V from L2.  The register budget is capped at two
// waves per SIMD (two workgroups per CU, 2 x 68 KB of LDS): one wave's
// softmax then overlaps the other's MFMA work, which a single wave per SIMD
// cannot do across its own dependent S -> P -> O chain (measured 1.5-1.75x).
#include "common.h"

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
  constexpr int NT = 256, TK = PF_TK;
  constexpr int KSTEPS = DH / 16, DT = DH / 32;
  constexpr int EPC = 8, CPR = DH / EPC;
  constexpr int KCH = TK * CPR, KCH_T = KCH / NT;
  constexpr int VU = (TK / 4) * CPR, VU_T = (VU + NT - 1) / NT;
  constexpr int KST = DH + 8, VST = TK + 4;
  __shared__ __attribute__((aligned(16))) T Ks[2][TK * KST];
  __shared__ __attribute__((aligned(16))) T Vt[2][DH * VST];

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

  u32x4 qf[KSTEPS];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((size_t(b) * a.nq + (qok ? qi : 0)) * a.Hq + hq) * DH;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = qok ? ld16(qp + ks * 16 + 8 * h) : u32x4{0, 0, 0, 0};
  }
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  u32x4 kreg[KCH_T];
  u32x4 vreg[VU_T][4];
  auto load_tile = [&](int key0) {
#pragma unroll
    for (int c = 0; c < KCH_T; ++c) {
      const int ch = tid + c * NT, key = key0 + ch / CPR;
      kreg[c] = key < k_end ? ld16(K + size_t(key) * DH + (ch % CPR) * EPC) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VU_T; ++u) {
      const int un = tid + u * NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + (un % (TK / 4)) * 4 + e;
        vreg[u][e] = (un < VU && key < k_end) ? ld16(V + size_t(key) * DH + (un / (TK / 4)) * EPC)
                                               : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < KCH_T; ++c) {
      const int ch = tid + c * NT;
      *reinterpret_cast<u32x4*>(&Ks[buf][(ch / CPR) * KST + (ch % CPR) * EPC]) = kreg[c];
    }
#pragma unroll
    for (int u = 0; u < VU_T; ++u) {
      const int un = tid + u * NT;
      if (un >= VU) continue;
      const int k4 = (un % (TK / 4)) * 4, d0 = (un / (TK / 4)) * EPC;
      const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&vreg[u][0]);
      const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&vreg[u][1]);
      const uint16_t* e2 = reinterpret_cast<const uint16_t*>(&vreg[u][2]);
      const uint16_t* e3 = reinterpret_cast<const uint16_t*>(&vreg[u][3]);
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        u32x2 w;
        w[0] = uint32_t(e0[x]) | (uint32_t(e1[x]) << 16);
        w[1] = uint32_t(e2[x]) | (uint32_t(e3[x]) << 16);
        *reinterpret_cast<u32x2*>(&Vt[buf][(d0 + x) * VST + k4]) = w;
      }
    }
  };
  auto compute_tile = [&](int buf, int key0) {
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(&Ks[buf][(kt * 32 + l32) * KST + ks * 16 + 8 * h]);
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
    const float c = a.scale_log2;
    float mx = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
    mx = xor32_max(mx) * c;
    // lazy rescale (see the block attention kernel); a fully masked tile
    // (mx = -inf) leaves the state untouched
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
      const float mn = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = mn;
    }
    float rs = 0.f;
    const float mneg = -m;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[kt][v], c, mneg));
        s[kt][v] = p;
        rs += p;
      }
    rs = xor32_sum(rs);
    l += rs;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 pf;
        pf[0] = pack_bf16x2(s[kt][8 * q + 0], s[kt][8 * q + 1]);
        pf[1] = pack_bf16x2(s[kt][8 * q + 2], s[kt][8 * q + 3]);
        pf[2] = pack_bf16x2(s[kt][8 * q + 4], s[kt][8 * q + 5]);
        pf[3] = pack_bf16x2(s[kt][8 * q + 6], s[kt][8 * q + 7]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T* row = &Vt[buf][(dt * 32 + l32) * VST + kt * 32 + q * 16 + h * 4];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 8);
          o[dt] = mfma32x32x16_bf16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, o[dt]);
        }
      }
  };

  const int ntiles = (k_end + TK - 1) / TK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile((t + 1) * TK);
    compute_tile(buf, t * TK);
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
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

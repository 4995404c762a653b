// Block attention of the active (sub-)block over the block-level KV cache.
//
// Computes eq 3 of "Fast-dLLM: Reusing Bidirectional State and Spending
// Confidence on Parallel Tokens" (softmax(Q K^T / sqrt(d)) V) for the query
// rows of the active block, whose visible keys are the cached prefix plus the
// block's own D positions ("Fast-dLLM v2: Efficient Block-Diffusion LLM",
// Inference-time attention mask, Figure 7b) or, in the v1 DualCache mode,
// additionally the cached suffix (section 3 of the Fast-dLLM review).
//
// gfx950 design
//   * One workgroup per (sequence, KV head, key split).  All G = Hq/Hkv query
//     heads x S query rows of a KV head live in the workgroup, so every K/V
//     byte of a split is read from HBM exactly once per step.
//   * K/V tiles of 64 keys are staged through LDS by 16-byte coalesced loads,
//     prefetched into registers ahead of the MFMA work (two tiles ahead for
//     bf16, one for f32).  V is written to LDS transposed so that the P.V
//     product reads contiguous keys.
//   * S^T = K Q^T and O^T = V^T P^T run on MFMA (32x32x16 bf16, or 16x16x4
//     f32 for f32 data).  In this orientation the score accumulator of a lane
//     is exactly the P operand of the next MFMA (same query column, the same
//     keys under a fixed permutation), and the per-query softmax statistics
//     sit in the lane that owns that query column, so the online-softmax
//     rescale needs no shuffles.
//   * Online softmax in fp32 with exp2 and the log2(e)/sqrt(d) scale folded
//     into the scores.  Splits write (m, l, unnormalized O) partials that a
//     second kernel merges in a fixed order (deterministic).
#include "common.h"

namespace fdl {

constexpr int TK = 64;  // keys per tile

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kb;
  const void* vb;
  const int32_t* prefix_len;
  void* out;
  float* lse;
  float* part_o;   // [nsplit][B][Hq][S][d]      (nsplit > 1)
  float* part_ml;  // [nsplit][B][Hq][S][2]      (m in log2 units, l)
  int B, S, Hq, Hkv, G, cap, D;
  int default_lp;
  int dual;
  int nsplit;
  int split_keys;
  float scale_log2;
  const int32_t* gate;  // decode loop: skip the launch when *gate == 0 (null: always run)
};

template <typename T>
struct Frag;

// bf16: one MFMA consumes 32 k values; a lane holds 8 of them (16 bytes).
template <>
struct Frag<bf16_t> {
  static constexpr int KPI = 32;
  static constexpr int EPL = 8;
  typedef u32x4 type;
  static __device__ __forceinline__ type load(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ type zero() { return u32x4{0, 0, 0, 0}; }
  static __device__ __forceinline__ f32x4 mma(type a, type b, f32x4 c) { return mfma16x16x32_bf16(a, b, c); }
};

// f32: one MFMA consumes 4 k values; a lane holds 1.
template <>
struct Frag<float> {
  static constexpr int KPI = 4;
  static constexpr int EPL = 1;
  typedef float type;
  static __device__ __forceinline__ type load(const float* p) { return *p; }
  static __device__ __forceinline__ type zero() { return 0.f; }
  static __device__ __forceinline__ f32x4 mma(type a, type b, f32x4 c) { return mfma16x16x4_f32(a, b, c); }
};

__device__ __forceinline__ void store4(bf16_t* p, f32x4 v, float s) {
  u32x2 w;
  w[0] = pack_bf16x2(v[0] * s, v[1] * s);
  w[1] = pack_bf16x2(v[2] * s, v[3] * s);
  *reinterpret_cast<u32x2*>(p) = w;
}
__device__ __forceinline__ void store4(float* p, f32x4 v, float s) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0] * s, v[1] * s, v[2] * s, v[3] * s};
}

// f32 data (and the generic 16-row layout): 16x16x4 f32 MFMA.
template <typename T, int DH, int NW, int RB>
__global__ __launch_bounds__(NW * 64) void block_attn_kernel(AttnArgs a) {
  if (gate_closed(a.gate)) return;
  typedef Frag<T> F;
  constexpr int NT = NW * 64;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int CPR = DH / EPC;                // chunks per K/V row
  constexpr int KCH = TK * CPR;                // K chunks per tile
  constexpr int KCH_T = (KCH + NT - 1) / NT;   // per thread
  constexpr int VU = (TK / 4) * CPR;           // V units (4 keys x 1 chunk) per tile
  constexpr int VU_T = (VU + NT - 1) / NT;
  constexpr int KS = DH / F::KPI;              // MFMA k-steps over the head dim
  constexpr int KPAD = EPC;                    // 16 bytes of padding per K row
  constexpr int KST = DH + KPAD;
  constexpr int VPAD = (sizeof(T) == 2) ? 8 : 4;
  constexpr int VST = TK + VPAD;
  constexpr int DT = DH / 16;                  // 16-row tiles of the head dim

  __shared__ __attribute__((aligned(16))) T Ks[2][TK * KST];
  __shared__ __attribute__((aligned(16))) T Vt[2][DH * VST];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;

  int lp = a.default_lp;
  if (a.prefix_len) {
    lp = a.prefix_len[b];
    lp = lp < 0 ? 0 : (lp > a.cap - a.D ? a.cap - a.D : lp);
  }
  const int lk = a.dual ? a.cap : lp + a.D;
  const int k_begin = split * a.split_keys;
  const int k_end = min(k_begin + a.split_keys, lk);
  const int rows = a.G * a.S;
  const size_t pair = size_t(b) * a.Hkv + g;

  const T* kc = reinterpret_cast<const T*>(a.kc) + pair * a.cap * DH;
  const T* vc = reinterpret_cast<const T*>(a.vc) + pair * a.cap * DH;
  const T* kbk = reinterpret_cast<const T*>(a.kb) + pair * a.D * DH;
  const T* vbk = reinterpret_cast<const T*>(a.vb) + pair * a.D * DH;

  if (k_begin >= lk) {  // empty split (per-sequence prefix shorter than the grid assumed)
    for (int r = tid; r < rows; r += NT) {
      const int h = g * a.G + r / a.S, i = r % a.S;
      const size_t row = (size_t(b) * a.Hq + h) * a.S + i;
      float* ml = a.part_ml + (size_t(split) * a.B * a.Hq * a.S + row) * 2;
      ml[0] = -INFINITY;
      ml[1] = 0.f;
    }
    return;
  }

  // --- query fragments (B operand of S^T = K Q^T): lane holds query column l16
  typename F::type qf[RB][KS];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int rb = wave + NW * j;
    const int r = rb * 16 + l16;
    const bool ok = r < rows;
    const T* qp = nullptr;
    if (ok) {
      const int h = g * a.G + r / a.S, i = r % a.S;
      qp = reinterpret_cast<const T*>(a.q) + ((size_t(b) * a.S + i) * a.Hq + h) * DH;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[j][ks] = ok ? F::load(qp + ks * F::KPI + F::EPL * grp) : F::zero();
  }

  f32x4 o[RB][DT];
  float m[RB], l[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[j][dt] = f32x4{0, 0, 0, 0};
  }

  // logical key -> its 16-byte chunk source (prefix cache / block buffer / suffix cache)
  auto key_ptr = [&](const T* cache, const T* blk, int j) -> const T* {
    if (j >= lp && j < lp + a.D) return blk + size_t(j - lp) * DH;
    return cache + size_t(j) * DH;
  };

  // one register stage and two LDS buffers: tile t+1 is in flight while
  // tile t is consumed from LDS; one barrier per tile
  struct Stage {
    u32x4 k[KCH_T];
    u32x4 v[VU_T][4];
  };
  Stage st0;
  auto load_tile = [&](Stage& S_, int key0) {
#pragma unroll
    for (int c = 0; c < KCH_T; ++c) {
      const int ch = tid + c * NT;
      S_.k[c] = u32x4{0, 0, 0, 0};
      if (ch < KCH) {
        const int key = key0 + ch / CPR;
        if (key < k_end) S_.k[c] = ld16(key_ptr(kc, kbk, key) + (ch % CPR) * EPC);
      }
    }
#pragma unroll
    for (int u = 0; u < VU_T; ++u) {
      const int un = tid + u * NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S_.v[u][e] = u32x4{0, 0, 0, 0};
        if (un < VU) {
          const int key = key0 + (un % (TK / 4)) * 4 + e;
          if (key < k_end) S_.v[u][e] = ld16(key_ptr(vc, vbk, key) + (un / (TK / 4)) * EPC);
        }
      }
    }
  };
  auto store_tile = [&](const Stage& S_, int buf) {
#pragma unroll
    for (int c = 0; c < KCH_T; ++c) {
      const int ch = tid + c * NT;
      if (ch < KCH) *reinterpret_cast<u32x4*>(&Ks[buf][(ch / CPR) * KST + (ch % CPR) * EPC]) = S_.k[c];
    }
#pragma unroll
    for (int u = 0; u < VU_T; ++u) {
      const int un = tid + u * NT;
      if (un >= VU) continue;
      const int k4 = (un % (TK / 4)) * 4;
      const int d0 = (un / (TK / 4)) * EPC;
      if constexpr (sizeof(T) == 2) {
        // 4 keys x 8 dims -> 8 rows of V^T, 4 contiguous keys (8 bytes) each
        const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&S_.v[u][0]);
        const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&S_.v[u][1]);
        const uint16_t* e2 = reinterpret_cast<const uint16_t*>(&S_.v[u][2]);
        const uint16_t* e3 = reinterpret_cast<const uint16_t*>(&S_.v[u][3]);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          u32x2 w;
          w[0] = uint32_t(e0[x]) | (uint32_t(e1[x]) << 16);
          w[1] = uint32_t(e2[x]) | (uint32_t(e3[x]) << 16);
          *reinterpret_cast<u32x2*>(&Vt[buf][(d0 + x) * VST + k4]) = w;
        }
      } else {
        // 4 keys x 4 dims -> 4 rows of V^T, 4 contiguous keys (16 bytes) each
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          u32x4 w{S_.v[u][0][x], S_.v[u][1][x], S_.v[u][2][x], S_.v[u][3][x]};
          *reinterpret_cast<u32x4*>(&Vt[buf][(d0 + x) * VST + k4]) = w;
        }
      }
    }
  };

  auto compute_tile = [&](int buf, int key0) {
      // ---- S^T = K Q^T : s[j][kt] holds keys key0 + 16kt + 4grp + v for query column l16
      f32x4 s[RB][4];
#pragma unroll
      for (int j = 0; j < RB; ++j)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[j][kt] = f32x4{0, 0, 0, 0};
      // k-steps outermost so that consecutive MFMAs feed independent accumulators
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const typename F::type kf = F::load(&Ks[buf][(kt * 16 + l16) * KST + ks * F::KPI + F::EPL * grp]);
#pragma unroll
          for (int j = 0; j < RB; ++j) s[j][kt] = F::mma(kf, qf[j][ks], s[j][kt]);
        }
      }

      const bool partial = key0 + TK > k_end;
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float x = s[j][kt][v] * a.scale_log2;
            if (partial && key0 + kt * 16 + grp * 4 + v >= k_end) x = -INFINITY;
            s[j][kt][v] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m[j], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[j] - mn);
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = __builtin_amdgcn_exp2f(s[j][kt][v] - mn);
            s[j][kt][v] = p;
            rs += p;
          }
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        l[j] = l[j] * alpha + rs;
        m[j] = mn;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[j][dt] *= alpha;
      }

      // ---- O^T += V^T P^T
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < TK / 32; ++c) {
          u32x4 pf[RB];
#pragma unroll
          for (int j = 0; j < RB; ++j) {
            pf[j][0] = pack_bf16x2(s[j][2 * c][0], s[j][2 * c][1]);
            pf[j][1] = pack_bf16x2(s[j][2 * c][2], s[j][2 * c][3]);
            pf[j][2] = pack_bf16x2(s[j][2 * c + 1][0], s[j][2 * c + 1][1]);
            pf[j][3] = pack_bf16x2(s[j][2 * c + 1][2], s[j][2 * c + 1][3]);
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const T* row = &Vt[buf][(dt * 16 + l16) * VST + c * 32 + grp * 4];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16);
            const u32x4 vf{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
            for (int j = 0; j < RB; ++j) o[j][dt] = mfma16x16x32_bf16(vf, pf[j], o[j][dt]);
          }
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const float vf = reinterpret_cast<const float*>(Vt[buf])[(dt * 16 + l16) * VST + kt * 16 + grp * 4 + v];
#pragma unroll
              for (int j = 0; j < RB; ++j) o[j][dt] = mfma16x16x4_f32(vf, s[j][kt][v], o[j][dt]);
            }
      }
  };

  const int ntiles = (k_end - k_begin + TK - 1) / TK;
  load_tile(st0, k_begin);
  store_tile(st0, 0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(st0, k_begin + (t + 1) * TK);
    compute_tile(buf, k_begin + t * TK);
    if (t + 1 < ntiles) store_tile(st0, buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds O^T[16dt + 4grp + v][query column l16]
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int r = (wave + NW * j) * 16 + l16;
    if (r >= rows) continue;
    const int h = g * a.G + r / a.S, i = r % a.S;
    const size_t row = (size_t(b) * a.Hq + h) * a.S + i;  // [B][Hq][S] row id
    if (a.nsplit == 1) {
      const float inv = 1.f / l[j];
      T* op = reinterpret_cast<T*>(a.out) + ((size_t(b) * a.S + i) * a.Hq + h) * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store4(op + dt * 16 + grp * 4, o[j][dt], inv);
      if (a.lse && grp == 0) a.lse[row] = (m[j] + __log2f(l[j])) * kLn2;
    } else {
      float* po = a.part_o + (size_t(split) * a.B * a.Hq * a.S + row) * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) store4(po + dt * 16 + grp * 4, o[j][dt], 1.f);
      if (grp == 0) {
        float* ml = a.part_ml + (size_t(split) * a.B * a.Hq * a.S + row) * 2;
        ml[0] = m[j];
        ml[1] = l[j];
      }
    }
  }
}

// bf16 data: 32x32x16 MFMA (on gfx950 twice the rate of 16x16x32).  Each of
// the NW waves owns 32 query rows (NW*32 >= G*S); every wave helps stage the
// K/V tiles.  S^T = K Q^T leaves a lane with 32 scores of its query column
// (lane & 31): keys key0 + 32kt + 8(v/4) + 4h + v%4, h = lane >> 5.  Packed
// 16 at a time, those are exactly the B operand of O^T += V^T P^T under the
// k permutation {4h..4h+3, 8+4h..8+4h+3} of each 16-key chunk, which the V^T
// fragments read with the same permutation.  Row statistics need one
// cross-lane exchange (lane ^ 32).  The running maximum is only moved when a
// tile raises it by more than 2^8 (log2 units 8): p then stays below 256, the
// normalization is unchanged, and the O/l rescale is skipped on most tiles.
// Registers are held to 256 per lane (two waves per SIMD) also for the 4-wave
// form: left to itself the compiler spreads that form over 332 and the copies
// between the two register files cost 5-7% (same results bit for bit).
template <int DH, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void block_attn_bf16_kernel(
    AttnArgs a) {
  if (gate_closed(a.gate)) return;
  constexpr int RB = 1;
  constexpr int KSTEPS = DH / 16, DT = DH / 32;
  typedef bf16_t T;
  constexpr int NT = NW * 64;
  constexpr int EPC = 8, CPR = DH / EPC;
  constexpr int KCH = TK * CPR, KCH_T = (KCH + NT - 1) / NT;
  constexpr int VU = (TK / 4) * CPR, VU_T = (VU + NT - 1) / NT;
  constexpr int KST = DH + 8;   // 272 B rows
  constexpr int VST = TK + 4;   // 136 B rows
  __shared__ __attribute__((aligned(16))) T Ks[2][TK * KST];
  __shared__ __attribute__((aligned(16))) T Vt[2][DH * VST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;

  int lp = a.default_lp;
  if (a.prefix_len) {
    lp = a.prefix_len[b];
    lp = lp < 0 ? 0 : (lp > a.cap - a.D ? a.cap - a.D : lp);
  }
  const int lk = a.dual ? a.cap : lp + a.D;
  const int k_begin = split * a.split_keys;
  const int k_end = min(k_begin + a.split_keys, lk);
  const int rows = a.G * a.S;
  constexpr int row0 = 0, rows_per_rg = NW * RB * 32;
  const size_t pair = size_t(b) * a.Hkv + g;
  const T* kc = reinterpret_cast<const T*>(a.kc) + pair * a.cap * DH;
  const T* vc = reinterpret_cast<const T*>(a.vc) + pair * a.cap * DH;
  const T* kbk = reinterpret_cast<const T*>(a.kb) + pair * a.D * DH;
  const T* vbk = reinterpret_cast<const T*>(a.vb) + pair * a.D * DH;

  if (k_begin >= lk) {
    for (int r = row0 + tid; r < min(rows, row0 + rows_per_rg); r += NT) {
      const int hq = g * a.G + r / a.S, i = r % a.S;
      const size_t row = (size_t(b) * a.Hq + hq) * a.S + i;
      float* ml = a.part_ml + (size_t(split) * a.B * a.Hq * a.S + row) * 2;
      ml[0] = -INFINITY;
      ml[1] = 0.f;
    }
    return;
  }

  u32x4 qf[RB][KSTEPS];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int r = row0 + (wave + NW * j) * 32 + l32;
    const bool ok = r < rows;
    const T* qp = nullptr;
    if (ok) {
      const int hq = g * a.G + r / a.S, i = r % a.S;
      qp = reinterpret_cast<const T*>(a.q) + ((size_t(b) * a.S + i) * a.Hq + hq) * DH;
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[j][ks] = ok ? ld16(qp + ks * 16 + 8 * h) : u32x4{0, 0, 0, 0};
  }
  f32x16 o[RB][DT];
  float m[RB], l[RB];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[j][dt][e] = 0.f;
  }
  auto key_ptr = [&](const T* cache, const T* blk, int j) -> const T* {
    if (j >= lp && j < lp + a.D) return blk + size_t(j - lp) * DH;
    return cache + size_t(j) * DH;
  };
  // two register stages: tile t + 2 is fetched while tile t is computed
  u32x4 kreg[2][KCH_T];
  u32x4 vreg[2][VU_T][4];
  // Per-thread source offsets of the K and V chunks within a tile; a tile that
  // lies wholly inside the cache (no block keys, no key past the split) takes
  // them with a scalar offset, the rest go through the per-key selection.
  int koff[KCH_T], voff[VU_T][4];
#pragma unroll
  for (int c = 0; c < KCH_T; ++c) {
    const int ch = tid + c * NT;
    koff[c] = (ch / CPR) * DH + (ch % CPR) * EPC;
  }
#pragma unroll
  for (int u = 0; u < VU_T; ++u) {
    const int un = tid + u * NT;
#pragma unroll
    for (int e = 0; e < 4; ++e) voff[u][e] = ((un % (TK / 4)) * 4 + e) * DH + (un / (TK / 4)) * EPC;
  }
  auto load_tile = [&](int rs, int key0) {
    const bool fast = key0 + TK <= k_end && (key0 + TK <= lp || key0 >= lp + a.D);
    if (fast) {
      const T* kt = kc + size_t(key0) * DH;
      const T* vt = vc + size_t(key0) * DH;
#pragma unroll
      for (int c = 0; c < KCH_T; ++c)
        if (KCH % NT == 0 || tid + c * NT < KCH) kreg[rs][c] = ld16(kt + koff[c]);
#pragma unroll
      for (int u = 0; u < VU_T; ++u)
        if (VU % NT == 0 || tid + u * NT < VU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) vreg[rs][u][e] = ld16(vt + voff[u][e]);
        }
      return;
    }
#pragma unroll
    for (int c = 0; c < KCH_T; ++c) {
      const int ch = tid + c * NT;
      kreg[rs][c] = u32x4{0, 0, 0, 0};
      if (ch < KCH) {
        const int key = key0 + ch / CPR;
        if (key < k_end) kreg[rs][c] = ld16(key_ptr(kc, kbk, key) + (ch % CPR) * EPC);
      }
    }
#pragma unroll
    for (int u = 0; u < VU_T; ++u) {
      const int un = tid + u * NT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vreg[rs][u][e] = u32x4{0, 0, 0, 0};
        if (un < VU) {
          const int key = key0 + (un % (TK / 4)) * 4 + e;
          if (key < k_end) vreg[rs][u][e] = ld16(key_ptr(vc, vbk, key) + (un / (TK / 4)) * EPC);
        }
      }
    }
  };
  auto store_tile = [&](int rs, int buf) {
#pragma unroll
    for (int c = 0; c < KCH_T; ++c) {
      const int ch = tid + c * NT;
      if (ch < KCH) *reinterpret_cast<u32x4*>(&Ks[buf][(ch / CPR) * KST + (ch % CPR) * EPC]) = kreg[rs][c];
    }
#pragma unroll
    for (int u = 0; u < VU_T; ++u) {
      const int un = tid + u * NT;
      if (un >= VU) continue;
      const int k4 = (un % (TK / 4)) * 4;
      const int d0 = (un / (TK / 4)) * EPC;
      const uint16_t* e0 = reinterpret_cast<const uint16_t*>(&vreg[rs][u][0]);
      const uint16_t* e1 = reinterpret_cast<const uint16_t*>(&vreg[rs][u][1]);
      const uint16_t* e2 = reinterpret_cast<const uint16_t*>(&vreg[rs][u][2]);
      const uint16_t* e3 = reinterpret_cast<const uint16_t*>(&vreg[rs][u][3]);
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
    // S^T = K Q^T: s[j][kt][v] = score of key key0 + 32kt + 8(v/4) + 4h + v%4, query column l32
    f32x16 s[RB][2];
#pragma unroll
    for (int j = 0; j < RB; ++j)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[j][kt][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(&Ks[buf][(kt * 32 + l32) * KST + ks * 16 + 8 * h]);
#pragma unroll
        for (int j = 0; j < RB; ++j) s[j][kt] = mfma32x32x16_bf16(kf, qf[j][ks], s[j][kt]);
      }
    }
    const bool partial = key0 + TK > k_end;
    const float c = a.scale_log2;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      if (partial) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (key0 + kt * 32 + (v / 4) * 8 + h * 4 + (v % 4) >= k_end) s[j][kt][v] = -INFINITY;
      }
      float mx = s[j][0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[j][kt][v]);
      mx = xor32_max(mx) * c;
      // lazy rescale: keep the running reference unless the new maximum
      // exceeds it by more than 8 (log2 units); p then stays below 2^8
      if (__builtin_amdgcn_ballot_w64(mx > m[j] + 8.f) != 0) {
        const float mn = fmaxf(m[j], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[j] - mn);
        l[j] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[j][dt] *= alpha;
        m[j] = mn;
      }
      float rs = 0.f;
      const float mneg = -m[j];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[j][kt][v], c, mneg));
          s[j][kt][v] = p;
          rs += p;
        }
      rs = xor32_sum(rs);
      l[j] += rs;
    }
    // O^T += V^T P^T over 16-key chunks (kt, q)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4 pf[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          pf[j][0] = pack_bf16x2(s[j][kt][8 * q + 0], s[j][kt][8 * q + 1]);
          pf[j][1] = pack_bf16x2(s[j][kt][8 * q + 2], s[j][kt][8 * q + 3]);
          pf[j][2] = pack_bf16x2(s[j][kt][8 * q + 4], s[j][kt][8 * q + 5]);
          pf[j][3] = pack_bf16x2(s[j][kt][8 * q + 6], s[j][kt][8 * q + 7]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T* row = &Vt[buf][(dt * 32 + l32) * VST + kt * 32 + q * 16 + h * 4];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(row);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 8);
          const u32x4 vf{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int j = 0; j < RB; ++j) o[j][dt] = mfma32x32x16_bf16(vf, pf[j], o[j][dt]);
        }
      }
  };

  // tile t lives in register stage t & 1 until it is stored to LDS buffer
  // t & 1; its load is issued two tiles ahead of its use, so two tiles of
  // MFMA work cover its latency
  const int ntiles = (k_end - k_begin + TK - 1) / TK;
  // A wave whose row blocks are all padding (G*S rows short of the NW*32 the
  // workgroup covers) only helps stage the tiles: its scores would never be
  // stored (2-3% off the attention at 56 and 32 rows per KV head).
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: a scalar branch
  bool wave_live = false;
#pragma unroll
  for (int j = 0; j < RB; ++j) wave_live |= row0 + (wave_s + NW * j) * 32 < rows;
  load_tile(0, k_begin);
  if (ntiles > 1) load_tile(1, k_begin + TK);
  store_tile(0, 0);
  __syncthreads();
  // the stage index is a literal at each call (register arrays cannot be
  // indexed at run time without going to scratch), hence the loop by two
  auto step = [&](int t, int buf) {
    if (t + 2 < ntiles) load_tile(buf, k_begin + (t + 2) * TK);  // stage buf held tile t, already in LDS
    if (wave_live) compute_tile(buf, k_begin + t * TK);
    if (t + 1 < ntiles) store_tile(buf ^ 1, buf ^ 1);
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, 0);
    if (t + 1 < ntiles) step(t + 1, 1);
  }
  // epilogue: o[j][dt][v] = O^T[d = 32dt + 8(v/4) + 4h + v%4][query l32]
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int r = row0 + (wave + NW * j) * 32 + l32;
    if (r >= rows) continue;
    const int hq = g * a.G + r / a.S, i = r % a.S;
    const size_t row = (size_t(b) * a.Hq + hq) * a.S + i;
    if (a.nsplit == 1) {
      const float inv = 1.f / l[j];
      T* op = reinterpret_cast<T*>(a.out) + ((size_t(b) * a.S + i) * a.Hq + hq) * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          store4(op + dt * 32 + q4 * 8 + h * 4,
                 f32x4{o[j][dt][4 * q4], o[j][dt][4 * q4 + 1], o[j][dt][4 * q4 + 2], o[j][dt][4 * q4 + 3]}, inv);
      if (a.lse && h == 0) a.lse[row] = (m[j] + __log2f(l[j])) * kLn2;
    } else {
      float* po = a.part_o + (size_t(split) * a.B * a.Hq * a.S + row) * DH;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          store4(po + dt * 32 + q4 * 8 + h * 4,
                 f32x4{o[j][dt][4 * q4], o[j][dt][4 * q4 + 1], o[j][dt][4 * q4 + 2], o[j][dt][4 * q4 + 3]}, 1.f);
      if (h == 0) {
        float* ml = a.part_ml + (size_t(split) * a.B * a.Hq * a.S + row) * 2;
        ml[0] = m[j];
        ml[1] = l[j];
      }
    }
  }
}


// Merge the split partials of every query row in split order.  The loads of
// up to sixteen splits are issued together so that their latencies overlap
// (the partials were written by workgroups on other XCDs and come back from
// beyond L2): one round of memory latency for the usual split counts.
template <typename T, int DH>
__global__ __launch_bounds__(256) void block_attn_merge_kernel(AttnArgs a) {
  if (gate_closed(a.gate)) return;
  constexpr int TPR = DH / 4;  // threads per row, 4 dims each
  constexpr int U = 16;
  const int n_rows = a.B * a.Hq * a.S;
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * 4;
  if (row >= n_rows) return;
  const size_t stride = size_t(n_rows);
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml);
  // splits in rounds of U (one round for U or fewer splits), each round's
  // loads issued together; across rounds the reference maximum is carried
  float mmax = -INFINITY, lsum = 0.f;
  f32x4 acc{0, 0, 0, 0};
  for (int s0 = 0; s0 < a.nsplit; s0 += U) {
    float2 v[U];
    f32x4 po[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + u < a.nsplit;
      v[u] = ok ? ml[(s0 + u) * stride + row] : float2{-INFINITY, 0.f};
      po[u] = ok ? *reinterpret_cast<const f32x4*>(a.part_o + ((s0 + u) * stride + row) * DH + d0)
                 : f32x4{0, 0, 0, 0};
    }
    float rmax = mmax;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v[u].y > 0.f) rmax = fmaxf(rmax, v[u].x);
    if (rmax > mmax) {
      const float alpha = mmax == -INFINITY ? 0.f : exp2f(mmax - rmax);
      lsum *= alpha;
      acc *= alpha;
      mmax = rmax;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!(v[u].y > 0.f)) continue;
      const float w = exp2f(v[u].x - mmax);
      lsum += w * v[u].y;
      acc += w * po[u];
    }
  }
  // row = (b*Hq + h)*S + i  ->  out[b][i][h]
  const int i = row % a.S;
  const int h = (row / a.S) % a.Hq;
  const int b = row / (a.S * a.Hq);
  T* op = reinterpret_cast<T*>(a.out) + ((size_t(b) * a.S + i) * a.Hq + h) * DH + d0;
  store4(op, acc, 1.f / lsum);
  if (a.lse && d0 == 0) a.lse[row] = (mmax + __log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------------------
// host side

struct AttnPlan {
  int nw, rb, nsplit, split_keys;
};

static int n_row_blocks(const fdl_dims& d) { return (d.n_q_heads / d.n_kv_heads * d.sub_block + 15) / 16; }

static AttnPlan plan_for(const fdl_dims& d, int lk) {
  AttnPlan p;
  const int nrb = n_row_blocks(d);
  if (d.dtype == FDL_BF16) p.nw = nrb <= 8 ? 4 : 8, p.rb = 1;   // 32-row blocks, <= 128 / 256 rows
  else if (nrb <= 1) p.nw = 1, p.rb = 1;
  else if (nrb <= 2) p.nw = 2, p.rb = 1;
  else if (nrb <= 4) p.nw = 4, p.rb = 1;
  else if (nrb <= 8) p.nw = 8, p.rb = 1;
  else p.nw = 8, p.rb = 2;
  const int pairs = d.batch * d.n_kv_heads;
  const int tiles = (lk + TK - 1) / TK;
  const int target_wg = 256;                       // one workgroup per CU
  int want = (target_wg + pairs - 1) / pairs;
  // as many splits as fill the chip, down to one tile each: with few KV heads
  // (1.5B/bs1: 2) the splits' tiles are the only parallelism there is
  const int tiles_per_split = (tiles + want - 1) / want;
  p.split_keys = tiles_per_split * TK;
  p.nsplit = (lk + p.split_keys - 1) / p.split_keys;
  return p;
}

// Largest split count any call with these dims can use: plan_for gives
// nsplit = ceil(tiles / tiles_per_split) with tiles_per_split =
// ceil(tiles / want), so nsplit <= min(want, tiles) for every key count up to
// the capacity.
static int max_splits(const fdl_dims& d) {
  const int pairs = d.batch * d.n_kv_heads;
  const int want = (256 + pairs - 1) / pairs;
  const int tiles = (d.prompt_len + d.gen_len + TK - 1) / TK;
  return tiles < want ? tiles : want;
}

size_t attn_workspace_bytes(const fdl_dims& d) {
  const int ns = max_splits(d);
  if (ns <= 1) return 0;
  const size_t rows = size_t(d.batch) * d.n_q_heads * d.sub_block;
  return size_t(ns) * rows * (d.head_dim + 2) * sizeof(float);
}

template <typename T, int DH, int NW, int RB>
static void launch_attn(const AttnArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((block_attn_kernel<T, DH, NW, RB>), grid, dim3(NW * 64), 0, st, a);
}

template <typename T, int DH>
static void launch_merge(const AttnArgs& a, hipStream_t st) {
  const int n_rows = a.B * a.Hq * a.S;
  const int rows_per_block = 256 / (DH / 4);
  hipLaunchKernelGGL((block_attn_merge_kernel<T, DH>), dim3((n_rows + rows_per_block - 1) / rows_per_block),
                     dim3(256), 0, st, a);
}

template <int DH>
static void launch_attn_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  dim3 grid(p.nsplit, a.Hkv, a.B);
  if (p.nw == 8) hipLaunchKernelGGL((block_attn_bf16_kernel<DH, 8>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((block_attn_bf16_kernel<DH, 4>), grid, dim3(256), 0, st, a);
  if (p.nsplit > 1) launch_merge<bf16_t, DH>(a, st);
}

template <int DH>
static void launch_attn_f32(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  dim3 grid(p.nsplit, a.Hkv, a.B);
  if (p.rb == 2) launch_attn<float, DH, 8, 2>(a, grid, st);
  else if (p.nw == 8) launch_attn<float, DH, 8, 1>(a, grid, st);
  else if (p.nw == 4) launch_attn<float, DH, 4, 1>(a, grid, st);
  else if (p.nw == 2) launch_attn<float, DH, 2, 1>(a, grid, st);
  else launch_attn<float, DH, 1, 1>(a, grid, st);
  if (p.nsplit > 1) launch_merge<float, DH>(a, st);
}

int attn_max_rows() { return 256; }

int attn_launch(const fdl_dims& d, int block_idx, const void* q, const void* kc, const void* vc,
                const int32_t* prefix_len, const void* kb, const void* vb, void* out, float* lse,
                void* ws, size_t ws_bytes, hipStream_t st, const int32_t* gate) {
  const int cap = d.prompt_len + d.gen_len;
  const int default_lp = d.prompt_len + block_idx * d.block;
  // grid covers the longest key list any sequence can have at this step
  const int lk = d.attn_mode == FDL_ATTN_DUAL_CACHE ? cap : (prefix_len ? cap : default_lp + d.block);
  const AttnPlan p = plan_for(d, lk);
  AttnArgs a;
  a.q = q; a.kc = kc; a.vc = vc; a.kb = kb; a.vb = vb;
  a.prefix_len = prefix_len;
  a.out = out; a.lse = lse;
  a.B = d.batch; a.S = d.sub_block; a.Hq = d.n_q_heads; a.Hkv = d.n_kv_heads;
  a.G = d.n_q_heads / d.n_kv_heads; a.cap = cap; a.D = d.block;
  a.default_lp = default_lp;
  a.dual = d.attn_mode == FDL_ATTN_DUAL_CACHE;
  a.nsplit = p.nsplit;
  a.split_keys = p.split_keys;
  a.scale_log2 = kLog2e / sqrtf(float(d.head_dim));
  a.part_o = nullptr; a.part_ml = nullptr;
  a.gate = gate;
  if (p.nsplit > 1) {
    const size_t rows = size_t(d.batch) * d.n_q_heads * d.sub_block;
    const size_t need = size_t(p.nsplit) * rows * (d.head_dim + 2) * sizeof(float);
    if (!ws || ws_bytes < need) return FDL_E_WORKSPACE;
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_o + size_t(p.nsplit) * rows * d.head_dim;
  }
  if (d.dtype == FDL_BF16) {
    if (d.head_dim == 128) launch_attn_bf16<128>(a, p, st);
    else launch_attn_bf16<64>(a, p, st);
  } else {
    if (d.head_dim == 128) launch_attn_f32<128>(a, p, st);
    else launch_attn_f32<64>(a, p, st);
  }
  return check_launch();
}

}  // namespace fdl

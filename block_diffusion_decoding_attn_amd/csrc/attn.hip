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
//   * bf16: K/V tiles of 64 keys travel HBM -> LDS by direct-to-LDS loads
//     through a 4-stage ring (no register staging); V^T operands come from
//     transposing LDS reads.  f32 (the tiny workload): register-staged tiles,
//     V transposed on its way into LDS.
//   * S^T = K Q^T and O^T = V^T P^T run on MFMA (32x32x16 bf16, or 16x16x4
//     f32 for f32 data).  In this orientation the score accumulator of a lane
//     is exactly the P operand of the next MFMA (same query column, the same
//     keys under a fixed permutation), and the per-query softmax statistics
//     sit in the lane that owns that query column, so the online-softmax
//     rescale needs no shuffles.
//   * Online softmax in fp32 with exp2 and the log2(e)/sqrt(d) scale folded
//     into the scores.  Splits write (m, l, O) partials that a second kernel
//     merges in a fixed order (deterministic): bf16 data O / l in bf16 pairs
//     per lane of the attention wave; f32 data unnormalized O per query row.
#include "common.h"
#include "kv_tiles.h"

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
  float* part_o;   // nsplit > 1: f32 data [nsplit][B][Hq][S][d]; bf16 data the per-lane partials (attn_pslot)
  float* part_ml;  // f32 data: [nsplit][B][Hq][S][2]      (m in log2 units, l)
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

// ---------------------------------------------------------------------------
// bf16 data (every bf16 workload)
//
// One workgroup per (sequence, KV head, key split); wave w owns query rows
// [32w, 32w + 32) of the KV head's G*S rows on 32x32x16 MFMA (a wave whose
// rows are all padding only helps load).
//
// K/V travel HBM -> LDS by global_load_lds_dwordx4 (no register staging)
// through a ring of NST stages of one 64-key tile each (K tile, then V tile,
// rows of d bf16 stored as they are in memory): up to NST - 1 tiles are in
// flight while one is consumed, with one s_waitcnt + barrier per tile.  A
// 1 KB load instruction fills 1024 / (2d) whole key rows; lane l fetches
// physical 16-byte chunk l % (2d / 16) of its row, which holds the logical
// chunk named by the row's swizzle, so that both kinds of fragment reads
// below are free of LDS bank conflicts.
//
// S^T = K Q^T leaves a lane with 32 scores of its query column (lane & 31):
// keys key0 + 32kt + 8(v/4) + 4h + v%4, h = lane >> 5.  Packed 16 at a time
// they are exactly the B operand of O^T += V^T P^T under the k order
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key chunk; the matching V^T operand
// comes from two transposing LDS reads (ds_read_b64_tr_b16: within each 16
// lanes, lane 4e + q reads four consecutive d of key k0 + e and every lane j
// receives keys k0..k0+3 of column d0 + j), so V is never transposed in
// registers.  Online softmax in fp32 with exp2 and log2(e)/sqrt(d) folded
// into the scores; the running maximum moves only when a tile raises it by
// more than 8 (log2 units), so P < 2^8 and most tiles skip the rescale.  The
// row sum adds the bf16-rounded P that the P.V product uses (v_dot2 of each
// packed pair with (1, 1)), per lane; the two half-waves combine at the end.
//
// Splits: every split writes O / l (bf16 pairs), m and l in the lanes' own
// register layout (coalesced, no transposition); block_attn_bf16_merge_kernel
// combines the splits of each KV head in split order (deterministic).  The
// splits of a KV head are placed on one XCD (workgroups are dealt
// round-robin to the 8 XCDs; the logical id below groups them), so they share
// that XCD's L2 for the block's K/V rows.
constexpr int NST = 4;  // LDS ring stages (tiles)


// Workspace of the bf16 kernel (nsplit > 1): partials of nsplit x KV heads x
// NW waves, each PSLOT x 64 lanes 32-bit words, where a wave's PSLOT = d/4 + 2
// words per lane are its d/2 O^T values divided by the split's row sum l
// (bf16, two per word: each is a convex combination of V rows, so bf16 keeps
// its relative precision), then m and l (fp32).
__host__ __device__ constexpr int attn_pslot(int dh) { return dh / 4 + 2; }

template <int DH, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void block_attn_bf16_kernel(
    AttnArgs a) {
  if (gate_closed(a.gate)) return;
  typedef bf16_t T;
  constexpr int ROWB = DH * 2;         // bytes per key row
  constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  constexpr int KPI = 1024 / ROWB;     // key rows per 1 KB load instruction
  constexpr int TILEB = TK * ROWB;     // one K (or V) tile
  constexpr int STB = 2 * TILEB;       // one stage: K tile, then V tile
  constexpr int IPH = TILEB / 1024;    // load instructions per K (or V) tile
  constexpr int IPW = 2 * IPH / NW;    // load instructions per wave per stage
  static_assert(2 * IPH % NW == 0, "whole load instructions per wave");
  constexpr int KSTEPS = DH / 16, DT = DH / 32;
  __shared__ __attribute__((aligned(1024))) char smem[NST * STB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  // logical workgroup id: the workgroups of one XCD (hardware id % 8) take a
  // contiguous run of ids, split fastest, so a KV head's splits share an L2
  const int nwg = gridDim.x, hw = blockIdx.x;
  const int xcd = hw & 7, k8 = hw >> 3, q8 = nwg >> 3, r8 = nwg & 7;
  const int lid = xcd < r8 ? xcd * (q8 + 1) + k8 : r8 * (q8 + 1) + (xcd - r8) * q8 + k8;
  const int split = lid % a.nsplit, pid = lid / a.nsplit;  // pid = b * Hkv + g
  const int g = pid % a.Hkv, b = pid / a.Hkv;

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
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool wave_live = wave_s * 32 < rows;
  const int r = wave * 32 + l32;  // this lane's query row (column of S^T)

  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m = -INFINITY;
  float lw[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's share of the row sum, in four independent chains

  if (k_begin < lk) {
    // this lane's share of the wave's load instructions.  A wave's IPW
    // instructions all fill the K tile or all the V tile of a stage
    // (IPH is a multiple of IPW); instruction j fills 1 KB at ld_lds[j] with
    // key rows KPI * i .. of the tile, this lane one chunk of row ld_row[j].
    static_assert(IPH % IPW == 0, "a wave loads only K or only V");
    const bool wave_v = wave_s * IPW >= IPH;
    const T* const my_cache = pick(wave_v, vc, kc);
    const T* const my_blk = pick(wave_v, vbk, kbk);
    int ld_row[IPW], ld_elem[IPW], ld_lds[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int i = wave_s * IPW + j - (wave_v ? IPH : 0);
      const int row = KPI * i + lane / CPR;
      const int c = (lane % CPR) ^ (wave_v ? swz_v<DH>(row) : swz_k<DH>(row));
      ld_row[j] = row;
      ld_elem[j] = c * 8;
      ld_lds[j] = (wave_v ? TILEB : 0) + i * 1024;
    }
    uint32_t ld_voff[IPW];  // byte offset of this lane's chunk from its tile's first row
#pragma unroll
    for (int j = 0; j < IPW; ++j) ld_voff[j] = uint32_t(ld_row[j] * DH + ld_elem[j]) * uint32_t(sizeof(T));
    const int ntiles = (k_end - k_begin + TK - 1) / TK;
    u32x4 qf[KSTEPS];  // B operand of S^T = K Q^T: query column l32, d = 16ks + 8h .. + 7
    auto issue = [&](int t) __attribute__((always_inline)) {
      const int key0 = k_begin + t * TK;
      char* sb = smem + (t % NST) * STB;
      const bool fast = key0 + TK <= k_end && (key0 + TK <= lp || key0 >= lp + a.D);
      if (fast) {
        // the whole tile in the cache: one wave-uniform base in SGPRs plus the
        // lane's constant byte offset (no per-lane 64-bit address arithmetic,
        // which was a fifth of the loop's VALU instructions)
        const T* const tb = my_cache + size_t(key0) * DH;
#pragma unroll
        for (int j = 0; j < IPW; ++j) load_lds16_s(tb, ld_voff[j], sb + ld_lds[j]);
        return;
      }
      // the tile holding the block or the split's end: per-lane rows from the
      // cache or the block buffer; keys past the split's end read a valid
      // row, and their scores are masked
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int key = min(key0 + ld_row[j], k_end - 1);
        const bool in_blk = key >= lp && key < lp + a.D;
        const size_t off = size_t(in_blk ? key - lp : key) * DH;  // element offset from my_cache (or my_blk)
        const T* base = pick(in_blk, my_blk, my_cache);
        load_lds16(base + off + ld_elem[j], sb + ld_lds[j]);
      }
    };

    // per-lane LDS byte offsets of the fragment reads (the tile, chunk and
    // stage parts are immediate offsets)
    int koff[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + h) ^ swz_k<DH>(l32)) << 4);
    int voff[DT];
    {
      const int grp = lane >> 4, sl = lane & 15, e = sl >> 2, qq = sl & 3;
      const int row = 4 * (grp >> 1) + e;  // key row within each 16-key chunk (first read)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + 16 * (grp & 1) + 4 * qq;
        voff[dt] = row * ROWB + (((d >> 3) ^ swz_v<DH>(row)) << 4) + (d & 7) * 2;
      }
    }
    const float c = a.scale_log2;

    auto compute = [&](int t) __attribute__((always_inline)) {
      const int key0 = k_begin + t * TK;
      const char* Ks = smem + (t % NST) * STB;
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
      if (key0 + TK > k_end) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (key0 + kt * 32 + (v / 4) * 8 + h * 4 + (v % 4) >= k_end) s[kt][v] = -INFINITY;
      }
      // four independent max chains (a single chain of dependent max3 would
      // expose the VALU latency at every step)
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
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.f) != 0) {
        const float mn = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int w = 0; w < 4; ++w) lw[w] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m = mn;
      }
      const float mneg = -m;
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

    issue(0);
    if (ntiles > 1) issue(1);
    {
      const bool ok = r < rows;
      const T* qp = nullptr;
      if (ok) {
        const int hq = g * a.G + r / a.S, i = r % a.S;
        qp = reinterpret_cast<const T*>(a.q) + ((size_t(b) * a.S + i) * a.Hq + hq) * DH;
      }
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = ok ? ld16(qp + ks * 16 + 8 * h) : u32x4{0, 0, 0, 0};
    }
    // the query fragments (and the first two tiles) have landed before the
    // third tile is issued: the compiler does not count the tile loads, so
    // it must not be left to wait for Q inside the loop
    wait_vm<0>();
    if (ntiles > 2) issue(2);
    for (int t = 0; t < ntiles; ++t) {
      // this wave's loads of tile t are done once at most those of the (up to
      // two) later tiles already issued are in flight; after the barrier every
      // wave's are, and every wave is done with tile t - 1, whose stage the
      // loads of tile t + 3 then refill
      if (t + 2 < ntiles) wait_vm<2 * IPW>();
      else if (t + 1 < ntiles) wait_vm<IPW>();
      else wait_vm<0>();
      bare_barrier();
      if (t + 3 < ntiles) issue(t + 3);
      if (wave_live) compute(t);
    }
  }
  float l = xor32_sum((lw[0] + lw[1]) + (lw[2] + lw[3]));  // both half-waves' shares of the row sum

  // o[dt][v] = O^T[d = 32dt + 8(v/4) + 4h + v%4][query row r]
  auto store_out = [&](const f32x16* oo, float mm, float ll) __attribute__((always_inline)) {
    if (r >= rows) return;
    const int hq = g * a.G + r / a.S, i = r % a.S;
    const float inv = 1.f / ll;
    T* op = reinterpret_cast<T*>(a.out) + ((size_t(b) * a.S + i) * a.Hq + hq) * DH;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4(op + dt * 32 + q4 * 8 + h * 4,
               f32x4{oo[dt][4 * q4], oo[dt][4 * q4 + 1], oo[dt][4 * q4 + 2], oo[dt][4 * q4 + 3]}, inv);
    if (a.lse && h == 0) a.lse[(size_t(b) * a.Hq + hq) * a.S + i] = (mm + __log2f(ll)) * kLn2;
  };

  if (a.nsplit == 1) {
    if (wave_live) store_out(o, m, l);
    return;
  }
  // split partial: this wave's O^T registers divided by l (bf16 pairs), m and
  // l, in the lanes' own layout (word w of every lane in one 256-byte run);
  // merged by block_attn_bf16_merge_kernel.  A split that holds keys has
  // l >= 1 in every row (its largest score contributes exp2(0) at least).
  if (!wave_live) return;
  constexpr int PS = attn_pslot(DH);
  const int npairs = a.B * a.Hkv;
  uint32_t* pp = reinterpret_cast<uint32_t*>(a.part_o) + ((size_t(split) * npairs + pid) * NW + wave) * PS * 64 + lane;
  if (k_begin < lk) {
    const float inv = 1.f / l;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 16; e += 2) pp[(dt * 8 + e / 2) * 64] = pack_bf16x2(o[dt][e] * inv, o[dt][e + 1] * inv);
  }
  pp[(PS - 2) * 64] = __float_as_uint(m);
  pp[(PS - 1) * 64] = __float_as_uint(l);
}

// Merge of the bf16 kernel's split partials: one workgroup per (KV head,
// 32-row block) of d / (2 NE) waves; wave j of it merges the lanes' values
// NE j .. NE j + NE - 1 of the attention wave's O^T registers (stored as O / l
// in bf16 pairs), each split weighted by exp2(m_s - max m) l_s.  Lane =
// (query column, half) exactly as in the attention kernel, so every load is a
// 256-byte run.  The (m, l) and values of up to U splits are fetched in one
// round of loads; splits are combined in split order.  Few splits: NE = 16,
// U = 4, the d / 32 waves of a row block in one workgroup (they share its
// (m, l) loads); many splits: NE = 4, U = 16 (one round), one wave per
// workgroup, so that the loads of few row blocks spread over many CUs.
template <int DH, int NW, int NE, int U, int NWG>
__global__ __launch_bounds__(NWG * 64) void block_attn_bf16_merge_kernel(AttnArgs a) {
  if (gate_closed(a.gate)) return;
  typedef bf16_t T;
  constexpr int PS = attn_pslot(DH), NJ = DH / 2 / NE;  // waves per row block
  const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
  const int blk = blockIdx.x / (NJ / NWG);
  const int j = (threadIdx.x >> 6) + NWG * (blockIdx.x % (NJ / NWG));
  const int wave = blk % NW, pid = blk / NW;
  const int rows = a.G * a.S;
  if (wave * 32 >= rows) return;
  const int g = pid % a.Hkv, b = pid / a.Hkv;
  const int npairs = a.B * a.Hkv;
  float mmax = -INFINITY, lsum = 0.f;
  float acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.f;
  static_assert(NE % 2 == 0, "bf16 pairs");
  for (int s0 = 0; s0 < a.nsplit; s0 += U) {
    float mv[U], lv[U], ov[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = s0 + u < a.nsplit;
      const uint32_t* pp =
          reinterpret_cast<const uint32_t*>(a.part_o) + ((size_t(s0 + u) * npairs + pid) * NW + wave) * PS * 64 + lane;
      mv[u] = ok ? __uint_as_float(pp[(PS - 2) * 64]) : -INFINITY;
      lv[u] = ok ? __uint_as_float(pp[(PS - 1) * 64]) : 0.f;
#pragma unroll
      for (int e = 0; e < NE; e += 2) {
        const uint32_t w = ok ? pp[((NE * j + e) / 2) * 64] : 0u;
        ov[u][e] = __uint_as_float(w << 16);
        ov[u][e + 1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
    float rmax = mmax;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lv[u] > 0.f) rmax = fmaxf(rmax, mv[u]);
    if (rmax > mmax) {  // carry the reference maximum across rounds
      const float alpha = mmax == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mmax - rmax);
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] *= alpha;
      mmax = rmax;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!(lv[u] > 0.f)) continue;  // an empty split wrote no O
      const float w = __builtin_amdgcn_exp2f(mv[u] - mmax) * lv[u];  // the split's weight; its O is O / l
      lsum += w;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] += w * ov[u][e];
    }
  }
  const int r = wave * 32 + l32;
  if (r >= rows) return;
  const int hq = g * a.G + r / a.S, i = r % a.S;
  // value NE*j + e of the lane = O^T[d = 32 dt + 8 (v/4) + 4h + v%4][row r], dt = (NE*j + e) / 16, v = (..) % 16
  T* op = reinterpret_cast<T*>(a.out) + ((size_t(b) * a.S + i) * a.Hq + hq) * DH;
  const float inv = 1.f / lsum;
#pragma unroll
  for (int e4 = 0; e4 < NE; e4 += 4) {
    const int e = NE * j + e4, dt = e / 16, v = e % 16;
    store4(op + dt * 32 + (v / 4) * 8 + h * 4, f32x4{acc[e4], acc[e4 + 1], acc[e4 + 2], acc[e4 + 3]}, inv);
  }
  if (a.lse && h == 0 && j == 0) a.lse[(size_t(b) * a.Hq + hq) * a.S + i] = (mmax + __log2f(lsum)) * kLn2;
}


// f32 data: merge the split partials of every query row in split order.  The
// loads of up to sixteen splits are issued together so that their latencies
// overlap: one round of memory latency for the usual split counts.
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

// bf16: waves of 32 query rows, at least two (the second only loads when the
// KV head has at most 32 rows), a power of two
static int bf16_waves(const fdl_dims& d) {
  const int rows = d.n_q_heads / d.n_kv_heads * d.sub_block;
  return rows <= 64 ? 2 : rows <= 128 ? 4 : 8;
}

static AttnPlan plan_for(const fdl_dims& d, int lk) {
  AttnPlan p;
  const int nrb = n_row_blocks(d);
  if (d.dtype == FDL_BF16) p.nw = bf16_waves(d), p.rb = 1;
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

static size_t bf16_split_bytes(const fdl_dims& d, int nsplit) {
  const int pairs = d.batch * d.n_kv_heads, nw = bf16_waves(d);
  return size_t(nsplit) * pairs * nw * attn_pslot(d.head_dim) * 64 * sizeof(float);
}

size_t attn_workspace_bytes(const fdl_dims& d) {
  const int ns = max_splits(d);
  if (ns <= 1) return 0;
  if (d.dtype == FDL_BF16) return bf16_split_bytes(d, ns);
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

template <int DH, int NW>
static void launch_merge_bf16(const AttnArgs& a, hipStream_t st) {
  const int blocks = NW * a.Hkv * a.B;  // (KV head, 32-row block) pairs
  if (a.nsplit <= 4)
    hipLaunchKernelGGL((block_attn_bf16_merge_kernel<DH, NW, 16, 4, DH / 32>), dim3(blocks), dim3(DH / 32 * 64), 0,
                       st, a);
  else
    hipLaunchKernelGGL((block_attn_bf16_merge_kernel<DH, NW, 4, 16, 1>), dim3(blocks * (DH / 8)), dim3(64), 0, st,
                       a);
}

template <int DH>
static void launch_attn_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  const dim3 grid(p.nsplit * a.Hkv * a.B);  // one workgroup per (KV head, split); see the logical id
  if (p.nw == 8) {
    hipLaunchKernelGGL((block_attn_bf16_kernel<DH, 8>), grid, dim3(512), 0, st, a);
    if (p.nsplit > 1) launch_merge_bf16<DH, 8>(a, st);
  } else if (p.nw == 4) {
    hipLaunchKernelGGL((block_attn_bf16_kernel<DH, 4>), grid, dim3(256), 0, st, a);
    if (p.nsplit > 1) launch_merge_bf16<DH, 4>(a, st);
  } else {
    hipLaunchKernelGGL((block_attn_bf16_kernel<DH, 2>), grid, dim3(128), 0, st, a);
    if (p.nsplit > 1) launch_merge_bf16<DH, 2>(a, st);
  }
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
  if (p.nsplit > 1 && d.dtype == FDL_BF16) {
    if (!ws || ws_bytes < bf16_split_bytes(d, p.nsplit)) return FDL_E_WORKSPACE;
    a.part_o = reinterpret_cast<float*>(ws);  // the split partials (O, m, l per lane)
  } else if (p.nsplit > 1) {
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

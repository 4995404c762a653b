// LM head: logits[M][V] = X[M][H] . W[V][H]^T with fp32 accumulation.
//
// "Fast-dLLM v2: Efficient Block-Diffusion LLM", Inference Pipeline Level 2:
// every position of the active block gets a probability distribution over the
// vocabulary; this kernel produces its logits.
//
// Two regimes on gfx950 (ridge ~312 flop/B for bf16 MFMA at 8 TB/s):
//   * skinny (M <= 64, the per-step rows of one or a few sequences): 2M flop
//     per weight element, far below the ridge, so the kernel is a weight
//     stream: W is read once with coalesced 16-byte non-temporal loads,
//     staged with the matching X slab through LDS, and fed to MFMA
//     (A = W rows, B = X^T).
//   * tiled (M > 64): MFMA-bound; 256 x 256 output tiles per workgroup, K
//     streamed HBM -> LDS by direct-to-LDS loads through two 64-wide slab
//     stages, 32x32x16 bf16 MFMA.
#include "common.h"
#include "launch.h"

namespace fdl {

struct LmArgs {
  const void* x;
  const void* w;
  float* out;    // [M][V] logits, or null (fused select: only partials)
  f32x4* part;   // [M][nc] confidence partials (one per workgroup vocabulary span: skinny span or
                 // 256-row weight tile), or null
  int M, H, V, nc;
  const int32_t* gate;  // decode loop: skip the launch when *gate == 0 (null: always run)
  int32_t* cnt;         // select row counters to zero (with part), or null
  int ncnt;
  int span;             // skinny bf16: vocabulary rows per workgroup (at most 128)
};

// Workgroup 0 zeroes the select's per-sequence row counters for the
// finalize kernel that follows on the stream.
__device__ __forceinline__ void zero_counters(const LmArgs& a) {
  if (a.cnt && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.ncnt; i += blockDim.x) a.cnt[i] = 0;
}

// Fused-select epilogue, shared by the skinny kernels: lane holds
// acc[t][n][e] = logit of vocabulary row vbase + 16t + 4grp + e for column
// m = 16n + l16; rows at or past vend do not count.  Reduce each column over
// the lane's rows (increasing index), then over the 4 lane groups, then over
// the workgroup's waves through LDS, and write the workgroup's partial for
// each row (partial index tile = the workgroup's vocabulary range).
template <int RT, int NTM, int NWAVES>
__device__ __forceinline__ void epilogue_partials(const LmArgs& a, const f32x4 (&acc)[RT][NTM], int vbase, int vend,
                                                  int wave, int l16, int grp, int tile, f32x4 (*red)[NTM * 16]) {
#pragma unroll
  for (int n = 0; n < NTM; ++n) {
    Red r = red_empty();
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = vbase + t * 16 + grp * 4 + e;
        if (v < vend) push(r, acc[t][n][e], v);
      }
    r = combine(r, shfl_xor_red(r, 16));
    r = combine(r, shfl_xor_red(r, 32));
    if (grp == 0) red[wave][n * 16 + l16] = pack_red(r);
  }
  __syncthreads();
  const int m = threadIdx.x;
  if (m < NTM * 16 && m < a.M) {
    Red r = unpack_red(red[0][m]);
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) r = combine(r, unpack_red(red[w][m]));
    a.part[size_t(m) * a.nc + tile] = pack_red(r);
  }
}

// ---------------------------------------------------------------------------
// skinny: a workgroup of WPB waves owns a contiguous range of a.span <= ROWS
// vocabulary rows, [b span, (b + 1) span) for workgroup b.  K is walked
// in slabs of KSLAB: the W slab (ROWS x KSLAB) and the X slab (16 NTM x
// KSLAB) are fetched with 16-byte loads in which 8 consecutive lanes cover one
// row's 128 contiguous bytes (rows past the range are not fetched), the next
// slab is held in registers while the current one is consumed, and both are
// written XOR-swizzled into LDS, from which every wave reads its MFMA
// fragments (A = 16 W rows x 32 k, B = 32 k x 16 X rows).  Staging X in LDS
// once per workgroup keeps the X re-reads off the L2 path (measured: 5.8 TB/s
// against 4.5 TB/s when every wave fetched its own X fragments).
//
// ONEBUF (up to 32 rows): one LDS buffer (22.5 KB, two barriers per slab) and
// at most 96 VGPRs, so that five workgroups fit on a CU and the launch can
// hold up to 1280 workgroups resident at once on MI355X's 256 CUs; the span
// is then V / 1280 rounded up (119 rows for 152064), so every workgroup
// streams the same share of W from its first cycle.  With 128-row tiles
// (1188 for a 152064-row vocabulary) at three per CU the launch ran in two
// rounds, the second one 55% full (measured per workgroup: 7.3 TB/s while
// all slots were busy, 5.5-6 TB/s in the second round).  Otherwise (33-64
// rows) a double-buffered LDS with one barrier.
template <int NTM, int ROWS, int KSLAB, int WPB, bool ONEBUF>
__device__ __forceinline__ void skinny_bf16_body(const LmArgs& a) {
  if (gate_closed(a.gate)) return;
  zero_counters(a);
  constexpr int NT = WPB * 64;
  constexpr int CPR = KSLAB * 2 / 16;        // 16-byte chunks per row of a slab
  constexpr int WCH = ROWS * CPR;            // W chunks per slab
  constexpr int WPER = WCH / NT;
  constexpr int XCH = NTM * 16 * CPR;        // X chunks per slab
  constexpr int XPER = (XCH + NT - 1) / NT;
  constexpr int RPW = ROWS / WPB;            // rows per wave
  constexpr int RT = RPW / 16;
  constexpr int NBUF = ONEBUF ? 1 : 2;
  static_assert(WCH % NT == 0 && RPW % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) u32x4 Ws[NBUF][WCH];
  __shared__ __attribute__((aligned(16))) u32x4 Xs[NBUF][XCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int v0 = min(a.V, int(blockIdx.x) * a.span), v1 = min(a.V, v0 + a.span);
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.w);
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.x);

  // per-thread staging sources (W rows past the range and X rows past M read as zero)
  const bf16_t* wsrc[WPER];
  int wdst[WPER];
  bool wok[WPER];
#pragma unroll
  for (int p = 0; p < WPER; ++p) {
    const int ch = tid + p * NT, row = ch / CPR, c = ch % CPR;
    wok[p] = v0 + row < v1;
    wsrc[p] = W + size_t(wok[p] ? v0 + row : v0) * a.H + c * 8;
    wdst[p] = row * CPR + (c ^ (row % CPR));
  }
  const bf16_t* xsrc[XPER];
  int xdst[XPER];
  bool xok[XPER];
#pragma unroll
  for (int p = 0; p < XPER; ++p) {
    const int ch = tid + p * NT, row = ch / CPR, c = ch % CPR;
    xok[p] = ch < XCH && row < a.M;
    xsrc[p] = X + size_t(xok[p] ? row : 0) * a.H + c * 8;
    xdst[p] = ch < XCH ? row * CPR + (c ^ (row % CPR)) : -1;
  }

  f32x4 acc[RT][NTM];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int n = 0; n < NTM; ++n) acc[t][n] = f32x4{0, 0, 0, 0};

  u32x4 wreg[WPER], xreg[XPER];
  auto gload = [&](int k) {
#pragma unroll
    for (int p = 0; p < WPER; ++p) wreg[p] = wok[p] ? ld16_stream(wsrc[p] + k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < XPER; ++p) xreg[p] = xok[p] ? ld16(xsrc[p] + k) : u32x4{0, 0, 0, 0};
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < WPER; ++p) Ws[buf][wdst[p]] = wreg[p];
#pragma unroll
    for (int p = 0; p < XPER; ++p)
      if (xdst[p] >= 0) Xs[buf][xdst[p]] = xreg[p];
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KSLAB / 32; ++ks) {
      const int c = ks * 4 + grp;
      u32x4 xb[NTM];
#pragma unroll
      for (int n = 0; n < NTM; ++n) {
        const int row = n * 16 + l16;
        xb[n] = Xs[buf][row * CPR + (c ^ (row % CPR))];
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int row = wave * RPW + t * 16 + l16;
        const u32x4 wf = Ws[buf][row * CPR + (c ^ (row % CPR))];
#pragma unroll
        for (int n = 0; n < NTM; ++n) acc[t][n] = mfma16x16x32_bf16(wf, xb[n], acc[t][n]);
      }
    }
  };

  // Workgroup b walks the K slabs starting at slab (5 b) mod nslab: when the
  // row stride is a multiple of the HBM channel interleave (H = 4096: 8 KB)
  // the workgroups in flight would otherwise all read the same low address
  // bits at the same time and queue on a few channels (measured at H = 4096:
  // 255 -> 196 us per call; strides 1, 5, 13, 29 all alike).  The sum order
  // differs per workgroup but is fixed.
  const int nslab = a.H / KSLAB;
  const int rot = int((5u * blockIdx.x) % unsigned(nslab));
  auto kslab = [&](int sl) { return (sl + rot < nslab ? sl + rot : sl + rot - nslab) * KSLAB; };
  gload(kslab(0));
  if (ONEBUF) {
    // the next slab waits in registers and is stored once every wave has
    // finished reading the current one
    for (int sl = 0; sl < nslab; ++sl) {
      if (sl > 0) __syncthreads();
      lstore(0);
      __syncthreads();
      if (sl + 1 < nslab) gload(kslab(sl + 1));
      compute(0);
    }
  } else {
    lstore(0);
    __syncthreads();
    for (int sl = 0; sl < nslab; ++sl) {
      const int buf = sl & 1;
      if (sl + 1 < nslab) gload(kslab(sl + 1));
      compute(buf);
      if (sl + 1 < nslab) lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // lane holds C[vocab v0 + wave*RPW + 16t + 4grp + e][m = 16n + l16]
  if (a.part) {
    __shared__ f32x4 red[WPB][NTM * 16];
    epilogue_partials<RT, NTM, WPB>(a, acc, v0 + wave * RPW, v1, wave, l16, grp, blockIdx.x, red);
  }
  if (!a.out) return;
#pragma unroll
  for (int n = 0; n < NTM; ++n) {
    const int m = n * 16 + l16;
    if (m >= a.M) continue;
    float* orow = a.out + size_t(m) * a.V;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int v = v0 + wave * RPW + t * 16 + grp * 4;
      if (v + 3 < v1 && ((v | a.V) & 3) == 0) {
        *reinterpret_cast<f32x4*>(orow + v) = acc[t][n];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (v + e < v1) orow[v + e] = acc[t][n][e];
      }
    }
  }
}

constexpr int SK_ROWS = 128, SK_KSLAB = 64, SK_WPB = 4;
constexpr int SK_RESIDENT = 1280;  // workgroups resident at once: 5 per CU x 256 CUs

template <int NTM>
__global__ __launch_bounds__(SK_WPB * 64) __attribute__((amdgpu_waves_per_eu(5, 5))) void lm_head_skinny_bf16_one(
    LmArgs a) {
  skinny_bf16_body<NTM, SK_ROWS, SK_KSLAB, SK_WPB, true>(a);
}

template <int NTM>
__global__ __launch_bounds__(SK_WPB * 64) void lm_head_skinny_bf16(LmArgs a) {
  skinny_bf16_body<NTM, SK_ROWS, SK_KSLAB, SK_WPB, false>(a);
}

// f32 data (the small fp32 workload): same wave decomposition on the
// 16x16x4 f32 MFMA, one k value per lane per instruction.
template <int NTM, int RT>
__global__ __launch_bounds__(256) void lm_head_skinny_f32(LmArgs a) {
  if (gate_closed(a.gate)) return;
  zero_counters(a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int v0 = (blockIdx.x * 4 + wave) * RT * 16;
  const float* W = reinterpret_cast<const float*>(a.w);
  const float* X = reinterpret_cast<const float*>(a.x);
  f32x4 acc[RT][NTM];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int n = 0; n < NTM; ++n) acc[t][n] = f32x4{0, 0, 0, 0};
  if (v0 < a.V) {
    for (int k = 0; k < a.H; k += 4) {
      float xa[NTM];
#pragma unroll
      for (int n = 0; n < NTM; ++n) {
        const int m = n * 16 + l16;
        xa[n] = m < a.M ? X[size_t(m) * a.H + k + grp] : 0.f;
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        int row = v0 + t * 16 + l16;
        row = row < a.V ? row : a.V - 1;
        const float wv = W[size_t(row) * a.H + k + grp];
#pragma unroll
        for (int n = 0; n < NTM; ++n) acc[t][n] = mfma16x16x4_f32(wv, xa[n], acc[t][n]);
      }
    }
  }
  if (a.part) {  // a workgroup covers 4 waves x RT*16 = 128 vocabulary rows when RT = 2
    __shared__ f32x4 red[4][NTM * 16];
    epilogue_partials<RT, NTM, 4>(a, acc, v0, a.V, wave, l16, grp, blockIdx.x, red);
  }
  if (!a.out || v0 >= a.V) return;
#pragma unroll
  for (int n = 0; n < NTM; ++n) {
    const int m = n * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = v0 + t * 16 + grp * 4 + e;
        if (v < a.V) a.out[size_t(m) * a.V + v] = acc[t][n][e];
      }
  }
}

// ---------------------------------------------------------------------------
// tiled (M > 64): workgroup tile 256 (vocab) x 256 (rows), 8 waves in a 2 x 4
// grid of 128 x 64 wave tiles (4 x 2 MFMA 32x32x16 tiles each).  K is consumed
// in 64-wide slabs that travel HBM -> LDS by global_load_lds_dwordx4 (no
// register staging) through two 64 KB stages: the next slab's loads are in
// flight while the current slab is consumed, one barrier per slab.  A slab
// row is 128 bytes = 8 chunks of 16; chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7) so that the 32-row fragment reads of a wave are free of
// bank conflicts.  Fragment reads are software-pipelined: the eight MFMAs of
// one 16-wide k-step run while the next k-step's fragments are read (against
// 32-wide slabs in a five-stage ring: 624 -> 561 us for M = 512, half the
// barriers).
constexpr int TB_V = 256, TB_M = 256, TB_K = 64, TB_NST = 2, TB_NWV = 2, TB_NWM = 4;  // 2 x 64 KB of LDS
constexpr int TB_ROWB = TB_K * 2;                          // bytes per row per stage
constexpr int TB_ABYTES = TB_V * TB_ROWB, TB_STB = (TB_V + TB_M) * TB_ROWB;
constexpr int TB_NT = TB_NWV * TB_NWM * 64;
constexpr int TB_IPW = TB_STB / 1024 / (TB_NWV * TB_NWM);  // 1 KB load instructions per wave per stage
constexpr int TB_TV = TB_V / TB_NWV / 32, TB_TM = TB_M / TB_NWM / 32;
static_assert(TB_TV * 32 == 128, "a wave covers half of a 256-row weight tile");

typedef __attribute__((address_space(3))) void lds_void_t;

// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((((N >> 4) & 3) << 14) | (0xF << 8) | (7 << 4) | (N & 15));
}

// (max, sum of exp(x - max), lowest argmax) of the 16 values a lane holds of
// one 32x32 accumulator tile: value e is vocabulary row vb + 8(e/4) + e%4.
// Rows at or past V do not count.
__device__ __forceinline__ Red tile_red(const f32x16 t, int vb, int V) {
  float x[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = vb + (e / 4) * 8 + (e % 4) < V ? t[e] : -INFINITY;
  float mt = x[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) mt = fmaxf(mt, x[e]);
  if (mt == -INFINITY) return red_empty();
  int it = 0;
#pragma unroll
  for (int e = 15; e >= 0; --e)
    if (x[e] == mt) it = vb + (e / 4) * 8 + (e % 4);
  float st = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) st += exp2f((x[e] - mt) * kLog2e);
  return Red{mt, st, it};
}

__global__ __launch_bounds__(TB_NT) void lm_head_tiled_bf16(LmArgs a) {
  if (gate_closed(a.gate)) return;
  zero_counters(a);
  __shared__ __attribute__((aligned(1024))) char smem[TB_NST * TB_STB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  // XCD-aware tile order: workgroups are dealt round-robin to the 8 XCDs, so
  // give each XCD a contiguous run of tiles, row tiles fastest, so that the
  // row tiles sharing a weight tile meet in the same L2.
  const int nvt = (a.V + TB_V - 1) / TB_V, nmt = (a.M + TB_M - 1) / TB_M;
  const int ntiles = nvt * nmt, per_xcd = (ntiles + 7) / 8;
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= ntiles) return;
  const int vt = tile / nmt, mt = tile % nmt;
  const int v0 = vt * TB_V, m0 = mt * TB_M;
  const int wv0 = (wave % TB_NWV) * (TB_TV * 32), wm0 = (wave / TB_NWV) * (TB_TM * 32);
  const bf16_t* W = reinterpret_cast<const bf16_t*>(a.w);
  const bf16_t* X = reinterpret_cast<const bf16_t*>(a.x);

  // Load instruction j of this wave fills stage bytes [kb KB, kb KB + 1 KB):
  // 8 rows of 128 bytes (W rows 0..255, then X rows); lane l writes physical
  // chunk l & 7 of row kb * 8 + l / 8, which holds logical chunk
  // (l & 7) ^ ((row >> 1) & 7).  Rows past V or M read a valid row; their
  // results are never stored.
  const bf16_t* src[TB_IPW];
  int dst[TB_IPW];
#pragma unroll
  for (int j = 0; j < TB_IPW; ++j) {
    const int kb = wave * TB_IPW + j;
    const int rr = kb * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((rr >> 1) & 7);
    if (rr < TB_V) src[j] = W + size_t(min(v0 + rr, a.V - 1)) * a.H + c * 8;
    else src[j] = X + size_t(min(m0 + rr - TB_V, a.M - 1)) * a.H + c * 8;
    dst[j] = kb * 1024;
  }
  // load instructions j0 .. j1 - 1 of this wave's share of a slab
  auto issue_part = [&](int slab, int j0, int j1) __attribute__((always_inline)) {
    char* sb = smem + (slab % TB_NST) * TB_STB;
    const int k0 = slab * TB_K;
#pragma unroll
    for (int j = 0; j < TB_IPW; ++j)
      if (j >= j0 && j < j1) __builtin_amdgcn_global_load_lds(src[j] + k0, (lds_void_t*)(sb + dst[j]), 16, 0, 0);
  };
  auto issue = [&](int slab) __attribute__((always_inline)) { issue_part(slab, 0, TB_IPW); };

  f32x16 acc[TB_TV][TB_TM];
#pragma unroll
  for (int i = 0; i < TB_TV; ++i)
#pragma unroll
    for (int j = 0; j < TB_TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = a.H / TB_K;
  issue(0);
  // the fragments of one 16-wide k-step of a slab
  auto frag = [&](int slab, int ks, u32x4* af, u32x4* bf) __attribute__((always_inline)) {
    const char* sb = smem + (slab % TB_NST) * TB_STB;
    const bf16_t* As = reinterpret_cast<const bf16_t*>(sb);
    const bf16_t* Bs = reinterpret_cast<const bf16_t*>(sb + TB_ABYTES);
    const int c = 2 * ks + half;
#pragma unroll
    for (int i = 0; i < TB_TV; ++i) {
      const int r = wv0 + i * 32 + l32;
      af[i] = *reinterpret_cast<const u32x4*>(As + r * TB_K + 8 * (c ^ ((r >> 1) & 7)));
    }
#pragma unroll
    for (int j = 0; j < TB_TM; ++j) {
      const int r = wm0 + j * 32 + l32;
      bf[j] = *reinterpret_cast<const u32x4*>(Bs + r * TB_K + 8 * (c ^ ((r >> 1) & 7)));
    }
  };
  auto mma = [&](const u32x4* af, const u32x4* bf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TB_TV; ++i)
#pragma unroll
      for (int j = 0; j < TB_TM; ++j) acc[i][j] = mfma32x32x16_bf16(af[i], bf[j], acc[i][j]);
  };
  // a slab has landed once this wave's own loads of it are done and, after
  // the barrier, every wave's
  auto arrive = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  // Each group of eight MFMAs runs while the next k-step's fragments are
  // read.  An explicit LDS wait right after the group (whose MFMAs take
  // hundreds of cycles to issue) completes those reads, so the compiler puts
  // no wait of its own in front of the next group; every loop iteration has
  // the same shape (the last slab is peeled) so its wait counts stay exact.
  constexpr int LGKM0 = 0xC07F;  // s_waitcnt lgkmcnt(0), the other counters untouched
  static_assert(TB_K == 64, "four k-steps per slab below");
  u32x4 a0[TB_TV], b0[TB_TM], a1[TB_TV], b1[TB_TM];
  arrive();
  if (1 < nk) issue(1);
  frag(0, 0, a0, b0);
  __builtin_amdgcn_s_waitcnt(LGKM0);
  // A slab's loads are issued in two parts: a quarter right after the
  // barrier that frees its stage, the rest one MFMA group later.  Issuing all
  // of them at the barrier, where every wave does so at once, fills the CU's
  // memory queue and stalls the waves' MFMA issue behind it (625 -> 605 us
  // for M = 512 run back to back).
  constexpr int EARLY = TB_IPW / 4;
  for (int t = 0; t + 1 < nk; ++t) {
    if (t >= 1) issue_part(t + 1, EARLY, TB_IPW);  // the rest of slab t + 1 (its first part: previous iteration)
    frag(t, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(LGKM0);
    frag(t, 2, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(LGKM0);
    frag(t, 3, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(LGKM0);
    arrive();                       // slab t + 1 has landed everywhere
    if (t + 2 < nk) issue_part(t + 2, 0, EARLY);  // into slab t's stage: every wave read and waited for it above
    frag(t + 1, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(LGKM0);
  }
  frag(nk - 1, 1, a1, b1);
  mma(a0, b0);
  __builtin_amdgcn_s_waitcnt(LGKM0);
  frag(nk - 1, 2, a0, b0);
  mma(a1, b1);
  __builtin_amdgcn_s_waitcnt(LGKM0);
  frag(nk - 1, 3, a1, b1);
  mma(a0, b0);
  __builtin_amdgcn_s_waitcnt(LGKM0);
  mma(a1, b1);

  // lane holds C[vocab 8(e/4) + 4 half + e%4][row l32] of each 32x32 tile.
  // The two waves of a row band (wave % TB_NWV = 0, 1) hold the lower and
  // upper 128 vocabulary rows of the weight tile: the upper one hands its
  // partials over through LDS and the lower one writes the tile's partial,
  // lower rows first (one partial per row and 256-row weight tile).
  if (a.part) {
    Red rr[TB_TM];
#pragma unroll
    for (int j = 0; j < TB_TM; ++j) {
      Red r = red_empty();
#pragma unroll
      for (int i = 0; i < TB_TV; ++i) {
        __builtin_amdgcn_sched_barrier(0);  // one accumulator tile at a time
        r = combine(r, tile_red(acc[i][j], v0 + wv0 + i * 32 + half * 4, a.V));
      }
      rr[j] = combine(r, shfl_xor_red(r, 32));
    }
    static_assert(TB_NWV == 2 && TB_TM * 32 * TB_NWM * 16 <= TB_NST * TB_STB, "partials hand-over in LDS");
    f32x4* xch = reinterpret_cast<f32x4*>(smem);  // [row band][TB_TM * 32 rows]
    __syncthreads();                               // every wave is done with the K slabs
    if (wave % TB_NWV == 1 && half == 0) {
#pragma unroll
      for (int j = 0; j < TB_TM; ++j) xch[(wave / TB_NWV) * (TB_TM * 32) + j * 32 + l32] = pack_red(rr[j]);
    }
    __syncthreads();
    if (wave % TB_NWV == 0 && half == 0) {
#pragma unroll
      for (int j = 0; j < TB_TM; ++j) {
        const Red r = combine(rr[j], unpack_red(xch[(wave / TB_NWV) * (TB_TM * 32) + j * 32 + l32]));
        const int m = m0 + wm0 + j * 32 + l32;
        if (m < a.M) a.part[size_t(m) * a.nc + vt] = pack_red(r);
      }
    }
  }
  if (!a.out) return;
#pragma unroll
  for (int j = 0; j < TB_TM; ++j) {
    const int m = m0 + wm0 + j * 32 + l32;
    if (m >= a.M) continue;
    float* orow = a.out + size_t(m) * a.V;
#pragma unroll
    for (int i = 0; i < TB_TV; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int v = v0 + wv0 + i * 32 + q * 8 + half * 4;
        const f32x4 val{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        if (v + 3 < a.V && (a.V & 3) == 0) {
          *reinterpret_cast<f32x4*>(orow + v) = val;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < a.V) orow[v + e] = val[e];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// host side

// Vocabulary rows per workgroup of the bf16 skinny LM head: up to 32 rows
// with a large vocabulary, V / SK_RESIDENT rounded up (all workgroups
// resident at once), else 128.
static int skinny_span(int V, int rows) {
  if (rows <= 32 && V >= 64 * SK_RESIDENT && V <= SK_ROWS * SK_RESIDENT) return (V + SK_RESIDENT - 1) / SK_RESIDENT;
  return SK_ROWS;
}
static int skinny_workgroups(int V, int rows) {
  const int span = skinny_span(V, rows);
  return (V + span - 1) / span;
}

template <int NTM>
static void launch_skinny_bf16(const LmArgs& args, hipStream_t st) {
  LmArgs a = args;
  a.span = skinny_span(a.V, a.M);
  const dim3 grid(skinny_workgroups(a.V, a.M));
  if constexpr (NTM <= 2) hipLaunchKernelGGL(lm_head_skinny_bf16_one<NTM>, grid, dim3(SK_WPB * 64), 0, st, a);
  else hipLaunchKernelGGL(lm_head_skinny_bf16<NTM>, grid, dim3(SK_WPB * 64), 0, st, a);
}

template <int NTM>
static void launch_skinny_f32(const LmArgs& a, hipStream_t st) {
  constexpr int RT = 2;
  const int waves = (a.V + RT * 16 - 1) / (RT * 16);
  hipLaunchKernelGGL((lm_head_skinny_f32<NTM, RT>), dim3((waves + 3) / 4), dim3(256), 0, st, a);
}

int lm_head_tiles(const fdl_dims& d, int rows) {
  if (d.dtype == FDL_BF16) {
    if (rows <= 64) return skinny_workgroups(d.vocab, rows);
    return (d.vocab + TB_V - 1) / TB_V;  // tiled: one partial per 256-row weight tile
  }
  return (d.vocab + 127) / 128;  // f32: one partial per 128-row vocabulary tile
}

int lm_head_launch(const fdl_dims& d, int rows, const void* x, const void* w, float* logits, void* part,
                   hipStream_t st, const int32_t* gate) {
  LmArgs a{x, w, logits, reinterpret_cast<f32x4*>(part), rows, d.hidden, d.vocab, lm_head_tiles(d, rows), gate,
           nullptr, 0, SK_ROWS};
  if (part) {
    a.cnt = partials_counters(part, d, rows / d.batch, a.nc);
    a.ncnt = d.batch;
  }
  const int ntm = (rows + 15) / 16;
  if (d.dtype == FDL_BF16) {
    switch (ntm) {
      case 1: launch_skinny_bf16<1>(a, st); break;
      case 2: launch_skinny_bf16<2>(a, st); break;
      case 3: launch_skinny_bf16<3>(a, st); break;
      case 4: launch_skinny_bf16<4>(a, st); break;
      default: {
        const int nvt = (a.V + TB_V - 1) / TB_V, nmt = (rows + TB_M - 1) / TB_M;
        hipLaunchKernelGGL(lm_head_tiled_bf16, dim3(8 * ((nvt * nmt + 7) / 8)), dim3(TB_NT), 0, st, a);
      }
    }
  } else {
    if (ntm > 4) return FDL_E_UNSUPPORTED;
    switch (ntm) {
      case 1: launch_skinny_f32<1>(a, st); break;
      case 2: launch_skinny_f32<2>(a, st); break;
      case 3: launch_skinny_f32<3>(a, st); break;
      default: launch_skinny_f32<4>(a, st); break;
    }
  }
  return check_launch();
}

}  // namespace fdl

// KV append: write a finished block's K/V into the block-level cache.
//
// "Fast-dLLM v2: Efficient Block-Diffusion LLM", Inference Pipeline Level 3:
// once a block is fully decoded its K/V are stored and reused unchanged by all
// later blocks.  "Fast-dLLM: Reusing Bidirectional State ...", Algorithm 1:
// the per-block refresh rewrites the cached regions (len = 0, then append all
// P + L positions).
//
// A bitwise copy with 16-byte vector loads and stores.  The append reads its
// position from len[b] on the device and advances it.  When a sequence's new
// K/V fit one workgroup's loop (a block of 32 positions does: 2 * Hkv * 32
// rows), one 512-thread workgroup per sequence copies them and then advances
// len[b] itself after a barrier: one launch, and no copy can see a
// half-updated length.  Larger appends spread the copy over (sequence,
// K|V x head, chunk) workgroups and a second one-thread-per-sequence kernel
// advances len after every copy of the call has been issued on the stream.
#include "common.h"

namespace fdl {

struct AppendArgs {
  void* kc;
  void* vc;
  const void* kn;
  const void* vn;
  int32_t* len;
  int B, Hkv, cap, n_new;
  int row_bytes;  // head_dim * element size
  const int32_t* gate;  // decode loop: skip the launch when *gate == 0 (null: always run)
};

__global__ __launch_bounds__(256) void kv_append_copy_kernel(AppendArgs a) {
  if (gate_closed(a.gate)) return;
  const int b = blockIdx.z;
  const int kv = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
  const int lo = a.len[b];
  if (lo < 0 || lo > a.cap - a.n_new) return;  // would overflow: leave the sequence untouched
  const size_t pair = size_t(b) * a.Hkv + g;
  const char* src = reinterpret_cast<const char*>(kv ? a.vn : a.kn) + pair * a.n_new * size_t(a.row_bytes);
  char* dst = reinterpret_cast<char*>(kv ? a.vc : a.kc) + (pair * a.cap + lo) * size_t(a.row_bytes);
  const size_t n16 = size_t(a.n_new) * a.row_bytes / 16;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    st16(dst + i * 16, ld16(src + i * 16));
}

// One workgroup per sequence: every 16-byte chunk of the sequence's K and V
// rows (2 * Hkv * n_new rows), eight loads in flight per thread, then len[b]
// advances once all of the workgroup's copies are done.
constexpr int kAppendSeqThreads = 512;
constexpr int kAppendSeqUnroll = 8;
constexpr size_t kAppendSeqMaxChunks = size_t(kAppendSeqThreads) * kAppendSeqUnroll * 4;  // 256 KB

__global__ __launch_bounds__(kAppendSeqThreads) void kv_append_seq_kernel(AppendArgs a) {
  if (gate_closed(a.gate)) return;
  const int b = blockIdx.x;
  const int lo = a.len[b];
  if (lo < 0 || lo > a.cap - a.n_new) return;  // would overflow: leave the sequence untouched
  // 32-bit chunk indices (a sequence's new rows are at most kAppendSeqMaxChunks chunks)
  const uint32_t per_row = uint32_t(a.row_bytes) / 16u;   // chunks per K/V row
  const uint32_t per_head = uint32_t(a.n_new) * per_row;  // chunks per (K|V, head)
  const uint32_t total = 2u * uint32_t(a.Hkv) * per_head;
  const char* kn = reinterpret_cast<const char*>(a.kn) + size_t(b) * a.Hkv * per_head * 16;
  const char* vn = reinterpret_cast<const char*>(a.vn) + size_t(b) * a.Hkv * per_head * 16;
  char* kc = reinterpret_cast<char*>(a.kc) + (size_t(b) * a.Hkv * a.cap + lo) * per_row * 16;
  char* vc = reinterpret_cast<char*>(a.vc) + (size_t(b) * a.Hkv * a.cap + lo) * per_row * 16;
  const uint32_t head_stride = uint32_t(a.cap) * per_row;  // chunks between heads in the cache
  for (uint32_t c0 = 0; c0 < total; c0 += kAppendSeqThreads * kAppendSeqUnroll) {
    u32x4 v[kAppendSeqUnroll];
#pragma unroll
    for (int u = 0; u < kAppendSeqUnroll; ++u) {
      const uint32_t c = c0 + u * kAppendSeqThreads + threadIdx.x;
      if (c < total) {
        const uint32_t half = c >= total / 2;                      // 0: K, 1: V
        const uint32_t r = c - half * (total / 2);                  // chunk within K (or V) of the sequence
        v[u] = ld16((half ? vn : kn) + size_t(r) * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < kAppendSeqUnroll; ++u) {
      const uint32_t c = c0 + u * kAppendSeqThreads + threadIdx.x;
      if (c < total) {
        const uint32_t half = (c >= total / 2);
        const uint32_t r = c - half * (total / 2);
        const uint32_t g = r / per_head, rr = r - g * per_head;    // head, chunk within the head's new rows
        st16((half ? vc : kc) + (size_t(g) * head_stride + rr) * 16, v[u]);
      }
    }
  }
  __syncthreads();  // every thread has read len[b] and finished its copies
  if (threadIdx.x == 0) a.len[b] = lo + a.n_new;
}

__global__ void kv_append_len_kernel(int32_t* len, int B, int cap, int n_new, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int lo = len[b];
  if (lo < 0 || lo > cap - n_new) return;
  len[b] = lo + n_new;
}

// Write at a position given by the caller (the refresh: every position from
// 0): the copies do not read len, so workgroup (0, 0, b) sets it directly and
// one launch does the whole step.
__global__ __launch_bounds__(256) void kv_write_kernel(AppendArgs a, int pos) {
  const int b = blockIdx.z;
  const int kv = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
  const size_t pair = size_t(b) * a.Hkv + g;
  const char* src = reinterpret_cast<const char*>(kv ? a.vn : a.kn) + pair * a.n_new * size_t(a.row_bytes);
  char* dst = reinterpret_cast<char*>(kv ? a.vc : a.kc) + (pair * a.cap + pos) * size_t(a.row_bytes);
  const size_t n16 = size_t(a.n_new) * a.row_bytes / 16;
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    st16(dst + i * 16, ld16(src + i * 16));
  if (a.len && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.len[b] = pos + a.n_new;
}

int write_launch(const fdl_dims& d, void* kc, void* vc, const void* kn, const void* vn, int pos, int n_new,
                 int32_t* len, hipStream_t st) {
  AppendArgs a;
  a.kc = kc; a.vc = vc; a.kn = kn; a.vn = vn; a.len = len; a.gate = nullptr;
  a.B = d.batch; a.Hkv = d.n_kv_heads; a.cap = d.prompt_len + d.gen_len; a.n_new = n_new;
  a.row_bytes = d.head_dim * dtype_size(d.dtype);
  const size_t n16 = size_t(n_new) * a.row_bytes / 16;
  int chunks = int((n16 + 255) / 256);
  if (chunks > 64) chunks = 64;
  hipLaunchKernelGGL(kv_write_kernel, dim3(chunks, 2 * d.n_kv_heads, d.batch), dim3(256), 0, st, a, pos);
  return check_launch();
}

int append_launch(const fdl_dims& d, void* kc, void* vc, const void* kn, const void* vn, int n_new, int32_t* len,
                  hipStream_t st, const int32_t* gate) {
  AppendArgs a;
  a.kc = kc; a.vc = vc; a.kn = kn; a.vn = vn; a.len = len; a.gate = gate;
  a.B = d.batch; a.Hkv = d.n_kv_heads; a.cap = d.prompt_len + d.gen_len; a.n_new = n_new;
  a.row_bytes = d.head_dim * dtype_size(d.dtype);
  const size_t n16 = size_t(n_new) * a.row_bytes / 16;
  if (2 * size_t(d.n_kv_heads) * n16 <= kAppendSeqMaxChunks) {
    hipLaunchKernelGGL(kv_append_seq_kernel, dim3(d.batch), dim3(kAppendSeqThreads), 0, st, a);
    return check_launch();
  }
  int chunks = int((n16 + 255) / 256);
  if (chunks > 64) chunks = 64;
  hipLaunchKernelGGL(kv_append_copy_kernel, dim3(chunks, 2 * d.n_kv_heads, d.batch), dim3(256), 0, st, a);
  hipLaunchKernelGGL(kv_append_len_kernel, dim3((d.batch + 255) / 256), dim3(256), 0, st, len, d.batch, a.cap,
                     n_new, gate);
  return check_launch();
}

}  // namespace fdl

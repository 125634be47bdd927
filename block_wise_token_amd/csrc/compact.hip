// Expand kept blocks into token rows and compact hidden states and positions.
//
// [UP] "Top-p selection" paragraph: the selection yields the token indices to keep;
// [UP] "propagation" and "Sparsity Propagation" paragraphs: every later layer
// receives only the surviving tokens; [UP] "scheduler" paragraph: the survivors'
// original positions travel with them.
//
// A block's G rows are consecutive rows of `hidden`, so compaction is a copy of
// whole contiguous runs of G * row_bytes: up_block_dst_kernel assigns each kept
// block its destination row (kept blocks in ascending order per request, requests
// in order), and up_gather_kernel streams the runs with 16-byte loads and stores,
// several workgroups per block.  The row-index list (idx_out) and positions come
// out of the same pass.  Drop composition is a plain gather through idx.
#include "up_internal.h"

namespace up {

__device__ __forceinline__ int64_t wg_sum_i64(int64_t v, int64_t* wsum) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t r = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += wsum[w];
  __syncthreads();
  return r;
}

// Inclusive scan of an int64 over a 1024-thread workgroup; *total gets the sum.
__device__ __forceinline__ int64_t wg_incl_scan_i64(int64_t v, int64_t* wsum, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int64_t pre = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) pre += wsum[w];
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return pre + v;
}

// One workgroup walks every request: validates cu_seqlens and cu_seqlens_out against
// the host totals and the keep flags, and writes per global block its source row,
// length and destination row (-1 when dropped).  hdr->valid = 1 only if all agree.
__global__ __launch_bounds__(1024) void up_block_dst_kernel(
    const uint8_t* __restrict__ keep, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_out, int B, int G, int64_t T_host, int64_t nb_tot_host,
    WsHeader* __restrict__ hdr, int32_t* __restrict__ dst, int32_t* __restrict__ src,
    int32_t* __restrict__ len, int* __restrict__ err) {
  __shared__ int64_t wsum[16];
  const int tid = threadIdx.x;
  int64_t part = 0, neg = 0;
  for (int r = tid; r < B; r += 1024) {
    const int64_t L = (int64_t)cu[r + 1] - cu[r];
    if (L < 0) neg += 1; else part += (L + G - 1) / G;
  }
  const int64_t nbt = wg_sum_i64(part, wsum);
  const int64_t nneg = wg_sum_i64(neg, wsum);
  const bool ok = nneg == 0 && nbt == nb_tot_host && (int64_t)cu[B] == T_host && cu[0] == 0 &&
                  cu_out[0] == 0;
  if (!ok) {
    if (tid == 0) { hdr->valid = 0; atomicOr(err, 1); }
    return;
  }
  bool consistent = true;
  int64_t boff = 0;
  for (int i = 0; i < B; ++i) {
    const int64_t L = (int64_t)cu[i + 1] - cu[i];
    const int64_t nb = (L + G - 1) / G;
    const int64_t tok = cu[i], out0 = cu_out[i];
    int64_t carry = 0;
    for (int64_t base = 0; base < nb; base += 1024) {
      const int64_t b = base + tid;
      const int64_t bl = (b < nb) ? ((L - b * G) < G ? (L - b * G) : G) : 0;
      const bool kept = (b < nb) && keep[boff + b] != 0;
      const int64_t kl = kept ? bl : 0;
      int64_t tot;
      const int64_t inc = wg_incl_scan_i64(kl, wsum, &tot);
      if (b < nb) {
        dst[boff + b] = kept ? (int32_t)(out0 + carry + inc - kl) : -1;
        src[boff + b] = (int32_t)(tok + b * G);
        len[boff + b] = (int32_t)bl;
      }
      carry += tot;
    }
    if ((int64_t)cu_out[i + 1] - out0 != carry) consistent = false;
    boff += nb;
  }
  if (tid == 0) {
    const bool v = consistent && (int64_t)cu_out[B] <= T_host;
    hdr->valid = v ? 1 : 0;
    if (!v) atomicOr(err, 1);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename V>
__device__ __forceinline__ V nt_load(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void nt_store(V v, V* p) { __builtin_nontemporal_store(v, p); }

// Copy kept blocks: workgroup (blk, part) moves its share of block blk's rows.
template <typename V, int NT, int UNROLL>
__global__ __launch_bounds__(NT) void up_gather_kernel(
    const uint8_t* __restrict__ hidden, int64_t row_bytes, const int32_t* __restrict__ pos,
    const WsHeader* __restrict__ hdr, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ src, const int32_t* __restrict__ len, int split,
    int32_t* __restrict__ idx_out, uint8_t* __restrict__ hidden_out,
    int32_t* __restrict__ pos_out) {
  if (hdr->valid != 1) return;
  const int64_t blk = blockIdx.x / split;
  const int part = (int)(blockIdx.x % split);
  const int32_t d = dst[blk];
  if (d < 0) return;
  const int64_t s = src[blk];
  const int n = len[blk];
  const int64_t nvec = (int64_t)n * row_bytes / (int64_t)sizeof(V);
  const int64_t lo = nvec * part / split, hi = nvec * (part + 1) / split;
  const V* sp = reinterpret_cast<const V*>(hidden + s * row_bytes);
  V* dp = reinterpret_cast<V*>(hidden_out + (int64_t)d * row_bytes);
  int64_t v = lo + threadIdx.x;
  for (; v + (UNROLL - 1) * NT < hi; v += UNROLL * NT) {
    V tmp[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) tmp[u] = nt_load(sp + v + u * NT);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) nt_store(tmp[u], dp + v + u * NT);
  }
  for (; v < hi; v += NT) nt_store(nt_load(sp + v), dp + v);
  if (part == 0) {
    for (int t = threadIdx.x; t < n; t += NT) {
      idx_out[d + t] = (int32_t)(s + t);
      if (pos_out) pos_out[d + t] = pos[s + t];
    }
  }
}

// orig_out[r] = prev[idx[r]] for r < *count.
__global__ __launch_bounds__(256) void up_compose_kernel(const int32_t* __restrict__ prev,
                                                         int prev_len,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ count,
                                                         int capacity, int32_t* __restrict__ out,
                                                         int* __restrict__ err) {
  int c = *count;
  if (c > capacity || c < 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, 4);
    c = c < 0 ? 0 : capacity;
  }
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= c) return;
  const int32_t j = idx[r];
  if (j < 0 || j >= prev_len) {
    out[r] = -1;
    atomicOr(err, 2);
  } else {
    out[r] = prev[j];
  }
}

CompactWs compact_ws_layout(int64_t nb_tot) {
  CompactWs L;
  size_t off = 0;
  L.hdr = off; off = align_up(off + sizeof(WsHeader));
  L.dst = off; off = align_up(off + (size_t)nb_tot * 4);
  L.src = off; off = align_up(off + (size_t)nb_tot * 4);
  L.len = off; off = align_up(off + (size_t)nb_tot * 4);
  L.total = off;
  return L;
}

static inline char* wsb(void* ws) { return static_cast<char*>(ws); }

hipError_t launch_block_dst(const uint8_t* keep, const int32_t* cu, const int32_t* cu_out, int B,
                            int G, int64_t T_host, int64_t nb_tot_host, void* ws,
                            const CompactWs& L, int* err, hipStream_t st) {
  hipLaunchKernelGGL(up_block_dst_kernel, dim3(1), dim3(1024), 0, st, keep, cu, cu_out, B, G,
                     T_host, nb_tot_host, reinterpret_cast<WsHeader*>(wsb(ws) + L.hdr),
                     reinterpret_cast<int32_t*>(wsb(ws) + L.dst),
                     reinterpret_cast<int32_t*>(wsb(ws) + L.src),
                     reinterpret_cast<int32_t*>(wsb(ws) + L.len), err);
  return hipGetLastError();
}

hipError_t launch_gather(const void* hidden, int64_t row_bytes, const int32_t* pos, void* ws,
                         const CompactWs& L, int64_t nb_tot, int G, int32_t* idx_out,
                         void* hidden_out, int32_t* pos_out, hipStream_t st) {
  if (nb_tot == 0) return hipSuccess;
  // Many small workgroups (4 KiB each, two 16-byte vectors per lane in flight)
  // stream fastest on MI355X: about 6.5 TB/s read+write for a plain 1 GiB copy.
  constexpr int NT = 128;
  const int64_t blk_bytes = (int64_t)G * row_bytes;
  int64_t split = blk_bytes / 4096;
  if (split < 1) split = 1;
  if (split > 4096) split = 4096;
  if (split > INT32_MAX / nb_tot) split = INT32_MAX / nb_tot > 0 ? INT32_MAX / nb_tot : 1;
  const dim3 grid((unsigned)(nb_tot * split));
  const auto* h = static_cast<const uint8_t*>(hidden);
  auto* ho = static_cast<uint8_t*>(hidden_out);
  const auto* hdr = reinterpret_cast<const WsHeader*>(wsb(ws) + L.hdr);
  const auto* dst = reinterpret_cast<const int32_t*>(wsb(ws) + L.dst);
  const auto* src = reinterpret_cast<const int32_t*>(wsb(ws) + L.src);
  const auto* len = reinterpret_cast<const int32_t*>(wsb(ws) + L.len);
  const uintptr_t al = reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(hidden_out);
  if (row_bytes % 16 == 0 && al % 16 == 0) {
    hipLaunchKernelGGL((up_gather_kernel<u32x4, NT, 2>), grid, dim3(NT), 0, st, h, row_bytes, pos,
                       hdr, dst, src, len, split, idx_out, ho, pos_out);
  } else if (row_bytes % 4 == 0 && al % 4 == 0) {
    hipLaunchKernelGGL((up_gather_kernel<uint32_t, NT, 4>), grid, dim3(NT), 0, st, h, row_bytes,
                       pos, hdr, dst, src, len, split, idx_out, ho, pos_out);
  } else {
    hipLaunchKernelGGL((up_gather_kernel<uint8_t, NT, 4>), grid, dim3(NT), 0, st, h, row_bytes,
                       pos, hdr, dst, src, len, split, idx_out, ho, pos_out);
  }
  return hipGetLastError();
}

hipError_t launch_compose(const int32_t* prev, int prev_len, const int32_t* idx,
                          const int32_t* count, int capacity, int32_t* out, int* err,
                          hipStream_t st) {
  if (capacity == 0) return hipSuccess;
  const unsigned grid = (unsigned)((capacity + 255) / 256);
  hipLaunchKernelGGL(up_compose_kernel, dim3(grid), dim3(256), 0, st, prev, prev_len, idx, count,
                     capacity, out, err);
  return hipGetLastError();
}

}  // namespace up

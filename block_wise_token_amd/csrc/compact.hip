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
// several workgroups per block.  The row-index list (idx_out), the positions and,
// when asked, the composed original indices (orig_out[r] = prev_orig[idx_out[r]])
// come out of the same pass.  up_compose_kernel is the standalone composition: a
// plain gather through idx.
#include "up_dpp.h"
#include "up_internal.h"

#include <mutex>

namespace up {

// One workgroup.  Requests are taken 1024 at a time: their block counts are
// scanned into block offsets (LDS), then the chunk's blocks -- contiguous in the
// global block numbering -- are scanned in rounds of 1024 x 4, thread t taking 4
// consecutive blocks.  A kept block's destination row is the number of kept tokens
// before it in the whole batch, which equals cu_seqlens_out[i] + (kept tokens of
// request i before it) exactly when cu_seqlens_out is the running sum of the kept
// counts -- checked at every request's last block (cu_seqlens_out[i + 1] must equal
// the running sum there).  Each block's request is found by binary search over the
// chunk's offsets, for its source row and length.  Every write is bounded by the host
// block count; hdr->valid = 1 only if all checks pass (the gather does nothing
// otherwise).
constexpr int kDstThreads = 1024;
constexpr int kDstPer = 4;   // consecutive blocks per thread per round

__global__ __launch_bounds__(1024) void up_block_dst_kernel(
    const uint8_t* __restrict__ keep, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_out, int B, int G, int64_t T_host, int64_t nb_tot_host,
    WsHeader* __restrict__ hdr, int32_t* __restrict__ dst, int32_t* __restrict__ src,
    int32_t* __restrict__ len, int* __restrict__ err) {
  __shared__ int64_t wtot[2][16];
  __shared__ int32_t req_boff[kDstThreads];   // chunk-relative first block of each request
  __shared__ int32_t req_tok[kDstThreads];
  __shared__ int32_t req_len[kDstThreads];
  __shared__ int32_t req_oend[kDstThreads];   // cu_seqlens_out[i + 1]
  __shared__ int bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t ends[4] = {0, 0, 0, 0};
  if (tid == 0) {
    bad = 0;
    ends[0] = cu[0];
    ends[1] = cu[B];
    ends[2] = cu_out[0];
    ends[3] = cu_out[B];
  }
  __syncthreads();
  int64_t blk_base = 0;   // global index of the chunk's first block
  int64_t kept_base = 0;  // kept tokens before the chunk
  int par = 0;            // which wtot buffer the next scan uses
  // Exclusive scan of v over the workgroup (in thread order) and its total.
  auto scan = [&](int64_t v, int64_t& total) -> int64_t {
    const uint64_t inc = wave_scan_u64((uint64_t)v);
    if (lane == 63) wtot[par][wave] = (int64_t)inc;
    __syncthreads();
    int64_t pre = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int64_t t = wtot[par][w];
      pre += w < wave ? t : 0;
      all += t;
    }
    par ^= 1;   // the next scan writes the other buffer: one barrier per scan suffices
    total = all;
    return pre + (int64_t)inc - v;
  };
  for (int base = 0; base < B; base += kDstThreads) {
    const int r = base + tid;
    int64_t nb_r = 0;
    if (r < B) {
      const int32_t t0 = cu[r], t1 = cu[r + 1];
      const int64_t Lr = (int64_t)t1 - t0;
      if (Lr < 0) atomicOr(&bad, 1);
      nb_r = Lr > 0 ? (Lr + G - 1) / G : 0;
      const int32_t o0 = cu_out[r], o1 = cu_out[r + 1];
      req_tok[tid] = t0;
      req_len[tid] = Lr > 0 ? (int32_t)Lr : 0;
      req_oend[tid] = o1;
      // An empty request keeps nothing: its two cu_seqlens_out entries must agree.
      if (nb_r == 0 && o1 != o0) atomicOr(&bad, 1);
    }
    int64_t chunk_blocks;
    const int64_t boff = scan(nb_r, chunk_blocks);
    const int nreq = (B - base) < kDstThreads ? (B - base) : kDstThreads;
    if (r < B) req_boff[tid] = (int32_t)(boff < INT32_MAX ? boff : INT32_MAX);
    __syncthreads();
    for (int64_t rb = 0; rb < chunk_blocks; rb += (int64_t)kDstThreads * kDstPer) {
      const int64_t g0 = rb + (int64_t)tid * kDstPer;   // chunk-relative
      // Request of block g0: the last request whose first block is <= g0.
      int lo = 0, hi = nreq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (req_boff[mid] <= g0) lo = mid; else hi = mid - 1;
      }
      int rr = lo;
      int64_t kl[kDstPer];
      int64_t tot = 0;
      {
        int q = rr;
#pragma unroll
        for (int j = 0; j < kDstPer; ++j) {
          const int64_t g = g0 + j;
          kl[j] = 0;
          if (g < chunk_blocks && blk_base + g < nb_tot_host) {
            while (q + 1 < nreq && req_boff[q + 1] <= g) ++q;
            const int64_t b = g - req_boff[q];
            const int64_t L = req_len[q];
            if (keep[blk_base + g] != 0) kl[j] = (L - b * G) < G ? (L - b * G) : G;
          }
          tot += kl[j];
        }
      }
      int64_t round_kept;
      int64_t run = kept_base + scan(tot, round_kept);
      int q = rr;
#pragma unroll
      for (int j = 0; j < kDstPer; ++j) {
        const int64_t g = g0 + j;
        if (g < chunk_blocks && blk_base + g < nb_tot_host) {
          while (q + 1 < nreq && req_boff[q + 1] <= g) ++q;
          const int64_t b = g - req_boff[q];
          const int64_t L = req_len[q];
          const int64_t bl = (L - b * G) < G ? (L - b * G) : G;
          dst[blk_base + g] = kl[j] ? (int32_t)run : -1;
          src[blk_base + g] = (int32_t)(req_tok[q] + b * G);
          len[blk_base + g] = (int32_t)bl;
          run += kl[j];
          // The request's last block: the running sum must be cu_seqlens_out[i + 1].
          if ((b + 1) * G >= L && (int64_t)req_oend[q] != run) atomicOr(&bad, 1);
        }
      }
      kept_base += round_kept;
    }
    blk_base += chunk_blocks;
    __syncthreads();   // before the next chunk overwrites the request tables
  }
  if (tid == 0) {
    const bool v = !bad && ends[0] == 0 && (int64_t)ends[1] == T_host && ends[2] == 0 &&
                   (int64_t)ends[3] <= T_host && blk_base == nb_tot_host;
    hdr->valid = v ? 1 : 0;
    if (!v) atomicOr(err, 1);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The hidden rows are read once: non-temporal loads.  They are written with ordinary
// stores: on MI355X that moves a decision 14 us faster than non-temporal stores (the
// copy itself 319 against 340 us at 128K; part of the write-back then lands in the next
// kernels), while non-temporal loads beat ordinary ones (340 against 346 us).
template <typename V>
__device__ __forceinline__ V nt_load(const V* p) { return __builtin_nontemporal_load(p); }
template <typename V>
__device__ __forceinline__ void row_store(V v, V* p) { *p = v; }

// Copy kept blocks: workgroup (blk, part) moves its share of block blk's rows.
template <typename V, int NT, int UNROLL>
__global__ __launch_bounds__(NT) void up_gather_kernel(
    const uint8_t* __restrict__ hidden, int64_t row_bytes, const int32_t* __restrict__ pos,
    const WsHeader* __restrict__ hdr, const int32_t* __restrict__ dst,
    const int32_t* __restrict__ src, const int32_t* __restrict__ len, int split,
    int32_t* __restrict__ idx_out, uint8_t* __restrict__ hidden_out,
    int32_t* __restrict__ pos_out, const int32_t* __restrict__ prev_orig,
    int32_t* __restrict__ orig_out, int64_t cap, int64_t T_in, int* __restrict__ err) {
  if (hdr->valid != 1) return;
  const int64_t blk = blockIdx.x / split;
  const int part = (int)(blockIdx.x % split);
  const int32_t d = dst[blk];
  if (d < 0) return;
  const int64_t s = src[blk];
  const int n = len[blk];
  // The header says the run table is consistent; a run that would still land outside
  // the outputs (capacity cap rows) or read outside the input (T_in rows) is refused.
  if (n < 0 || s < 0 || (int64_t)d + n > cap || s + n > T_in) {
    if (part == 0 && threadIdx.x == 0) atomicOr(err, 16);
    return;
  }
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
    for (int u = 0; u < UNROLL; ++u) row_store(tmp[u], dp + v + u * NT);
  }
  for (; v < hi; v += NT) row_store(nt_load(sp + v), dp + v);
  if (part == 0) {
    for (int t = threadIdx.x; t < n; t += NT) {
      idx_out[d + t] = (int32_t)(s + t);
      if (pos_out) pos_out[d + t] = pos[s + t];
      if (orig_out) orig_out[d + t] = prev_orig[s + t];   // drop composition, fused
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

// ---------------------------------------------------------------------------
// Run table of up_expand_compact_noalloc: a file-scope device array, one per GPU,
// held until the process ends.  Host code never uses the array's name as an address
// (on the host it is only a stand-in symbol); its device address is looked up once
// per device with hipGetSymbolAddress and that pointer is what the kernels get.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = 256 + 3 * (size_t)kStaticCompactBlocks * 4;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

void* static_compact_scratch(size_t* bytes) {
  *bytes = kStaticScratchBytes;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
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
                         const CompactWs& L, int64_t nb_tot, int G, int64_t T, int32_t* idx_out,
                         void* hidden_out, int32_t* pos_out, const int32_t* prev_orig,
                         int32_t* orig_out, int* err, hipStream_t st) {
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
                       hdr, dst, src, len, split, idx_out, ho, pos_out, prev_orig, orig_out, T, T, err);
  } else if (row_bytes % 4 == 0 && al % 4 == 0) {
    hipLaunchKernelGGL((up_gather_kernel<uint32_t, NT, 4>), grid, dim3(NT), 0, st, h, row_bytes,
                       pos, hdr, dst, src, len, split, idx_out, ho, pos_out, prev_orig, orig_out, T, T, err);
  } else {
    hipLaunchKernelGGL((up_gather_kernel<uint8_t, NT, 4>), grid, dim3(NT), 0, st, h, row_bytes,
                       pos, hdr, dst, src, len, split, idx_out, ho, pos_out, prev_orig, orig_out, T, T, err);
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

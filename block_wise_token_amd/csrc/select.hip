// Top-p / Top-k block selection on the GPU, one workgroup per request.
//
// [UP] "Top-p selection" paragraph: blocks sorted by descending importance are kept
// until their cumulative sum reaches p; [UP] "Triton kernels" paragraph: the
// selection runs on the GPU with no host round trip; [UP] "ablation" paragraph:
// Top-k (a fixed count) is the alternative the ablation compares against.
//
// Order: 64-bit keys (~float bits of the score) << 32 | block index, sorted
// ascending by a bitonic network in LDS, give score descending and ties by the
// lower block index.  The running sum is exact: a float32 in [0, 1] is an integer
// multiple of 2^-149 (below 2^150), so every score is widened to a 192-bit integer
// and the prefix sums are integer adds -- associative, so the parallel scan gives
// the same cut as a sequential exact sum would.  The cut is the first sorted
// position whose running sum reaches p (float32 p widened the same way).
#include "up_internal.h"

namespace up {

struct U192 {
  uint64_t lo, mid, hi;
};

__device__ __forceinline__ U192 u192_zero() { return U192{0, 0, 0}; }

// A score as an exact count of 2^-149 units.  Scores outside [0, 1] are clamped into
// it and NaN counts as 0 (scores produced by up_block_scores are always in [0, 1]).
__device__ __forceinline__ float clamp_score(float s) {
  if (!(s > 0.f)) return 0.f;
  return s > 1.f ? 1.f : s;
}

__device__ __forceinline__ U192 score_units(float s) {
  const uint32_t bits = __float_as_uint(s);
  const uint32_t e = bits >> 23, f = bits & 0x7FFFFFu;
  uint64_t m;
  int sh;
  if (e == 0) { m = f; sh = 0; } else { m = f | 0x800000u; sh = (int)e - 1; }   // sh <= 126
  U192 r = u192_zero();
  if (sh < 64) {
    r.lo = m << sh;
    r.mid = sh ? (m >> (64 - sh)) : 0;
  } else {
    r.mid = m << (sh - 64);
    r.hi = (sh == 64) ? 0 : (m >> (128 - sh));
  }
  return r;
}

__device__ __forceinline__ U192 u192_add(U192 a, U192 b) {
  U192 r;
  r.lo = a.lo + b.lo;
  const uint64_t c0 = r.lo < a.lo;
  const uint64_t t = a.mid + b.mid;
  const uint64_t c1 = t < a.mid;
  r.mid = t + c0;
  const uint64_t c2 = r.mid < t;
  r.hi = a.hi + b.hi + c1 + c2;
  return r;
}

__device__ __forceinline__ bool u192_geq(U192 a, U192 b) {
  if (a.hi != b.hi) return a.hi > b.hi;
  if (a.mid != b.mid) return a.mid > b.mid;
  return a.lo >= b.lo;
}

__device__ __forceinline__ U192 u192_shfl_up(U192 v, int d) {
  U192 r;
  r.lo = __shfl_up(v.lo, d);
  r.mid = __shfl_up(v.mid, d);
  r.hi = __shfl_up(v.hi, d);
  return r;
}

// Sum of an int64 over the workgroup (1024 threads) in a fixed order: a butterfly
// within each wave, then the 16 wave sums in wave order.
__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t* wsum) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t r = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r += wsum[w];
  __syncthreads();
  return r;
}

constexpr int kSelThreads = 1024;
constexpr int kSelMaxPer = kSelectMaxBlocks / kSelThreads;   // sorted positions per thread

__global__ __launch_bounds__(1024) void up_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ cu, int B, int n, int G,
    int mode, float p, int topk, int NP, int64_t T_host, int64_t nb_tot_host,
    uint8_t* __restrict__ keep, int32_t* __restrict__ cu_out, int* __restrict__ err) {
  extern __shared__ uint64_t keys[];            // NP sort keys
  __shared__ int64_t red[kSelThreads / 64];
  __shared__ U192 wave_tot[kSelThreads / 64];
  __shared__ int cut_pos;

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // First global block of this request: sum of the earlier requests' block counts.
  int64_t part = 0;
  for (int r = tid; r < i; r += kSelThreads) {
    const int64_t Lr = (int64_t)cu[r + 1] - cu[r];
    part += Lr > 0 ? (Lr + G - 1) / G : 0;
  }
  const int64_t blk_off = block_sum_i64(part, red);
  const int64_t L = (int64_t)cu[i + 1] - cu[i];
  const int64_t nb = L > 0 ? (L + G - 1) / G : 0;
  const bool bad = (L < 0) || ((int64_t)cu[B] != T_host) || (blk_off + nb > nb_tot_host) ||
                   (nb > NP) || (cu[0] != 0);
  if (bad) {
    if (tid == 0) {
      atomicOr(err, 1);
      cu_out[i + 1] = 0;
    }
    return;
  }
  const int64_t W = L < n ? L : n;
  const int64_t wfirst = (L - W) / G;   // first block holding a window token

  // Sort keys.  Element a of the bitonic network lives in thread a % 1024, slot
  // a / 1024: partners at distance j >= 1024 are in the same thread, partners at
  // 64 <= j < 1024 are exchanged through LDS, partners at j < 64 by wave shuffles.
  const int PER = NP >= kSelThreads ? NP / kSelThreads : 1;
  uint64_t kv[kSelMaxPer];
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q) {
    const int a = q * kSelThreads + tid;
    uint64_t key = ~0ull;
    if (q < PER && a < nb) {
      const float s = clamp_score(scores[blk_off + a]);
      key = ((uint64_t)(~__float_as_uint(s)) << 32) | (uint32_t)a;
    }
    kv[q] = key;
  }
  for (int k = 2; k <= NP; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kSelThreads) {
        const int jj = j / kSelThreads;
        auto cx = [&](int q, int p) {   // q < p: slots q and p of this thread
          const bool up = ((q * kSelThreads + tid) & k) == 0;
          const uint64_t x = kv[q], y = kv[p];
          if ((x > y) == up) { kv[q] = y; kv[p] = x; }
        };
#pragma unroll
        for (int q = 0; q < kSelMaxPer; ++q) {
          if (jj == 1 && !(q & 1) && q + 1 < PER) cx(q, q + 1);
          if (jj == 2 && !(q & 2) && q + 2 < PER) cx(q, q + 2);
          if (jj == 4 && !(q & 4) && q + 4 < PER) cx(q, q + 4);
        }
      } else {
        uint64_t y[kSelMaxPer];
        if (j >= 64) {
#pragma unroll
          for (int q = 0; q < kSelMaxPer; ++q)
            if (q < PER) keys[q * kSelThreads + tid] = kv[q];
          __syncthreads();
#pragma unroll
          for (int q = 0; q < kSelMaxPer; ++q)
            if (q < PER) y[q] = keys[q * kSelThreads + (tid ^ j)];
          __syncthreads();
        } else {
#pragma unroll
          for (int q = 0; q < kSelMaxPer; ++q)
            if (q < PER) y[q] = __shfl_xor(kv[q], j);
        }
#pragma unroll
        for (int q = 0; q < kSelMaxPer; ++q) {
          if (q < PER) {
            const int a = q * kSelThreads + tid;
            const bool lower = (a & j) == 0, up = (a & k) == 0;
            const uint64_t x = kv[q];
            kv[q] = (lower == up) ? (x < y[q] ? x : y[q]) : (x < y[q] ? y[q] : x);
          }
        }
      }
    }
  }
  // Re-distribute: thread t takes PER consecutive sorted positions.
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q)
    if (q < PER) keys[q * kSelThreads + tid] = kv[q];
  __syncthreads();
  U192 seg = u192_zero();
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q) {
    const int pos = tid * PER + q;
    kv[q] = (q < PER && pos < nb) ? keys[pos] : ~0ull;
    if (kv[q] != ~0ull) seg = u192_add(seg, score_units(__uint_as_float(~(uint32_t)(kv[q] >> 32))));
  }

  int64_t kstar = nb;
  if (mode == 1) {
    kstar = topk < nb ? topk : nb;
  } else if (p < 1.0f) {
    // Exclusive prefix of the segment sums: wave scan by shuffles, then wave totals.
    U192 inc = seg;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const U192 o = u192_shfl_up(inc, d);
      if (lane >= d) inc = u192_add(inc, o);
    }
    if (lane == 63) wave_tot[wave] = inc;
    if (tid == 0) cut_pos = 0x7fffffff;
    __syncthreads();
    U192 wpre = u192_zero();
    for (int w = 0; w < wave; ++w) wpre = u192_add(wpre, wave_tot[w]);
    U192 excl = u192_shfl_up(inc, 1);
    if (lane == 0) excl = u192_zero();
    U192 run = u192_add(wpre, excl);
    const U192 P = score_units(p);
#pragma unroll
    for (int q = 0; q < kSelMaxPer; ++q) {
      if (kv[q] != ~0ull) {
        run = u192_add(run, score_units(__uint_as_float(~(uint32_t)(kv[q] >> 32))));
        if (u192_geq(run, P)) {
          atomicMin(&cut_pos, tid * PER + q);
          break;
        }
      }
    }
    __syncthreads();
    if (cut_pos != 0x7fffffff) kstar = cut_pos + 1;
  }

  // Keep flags and kept-token count.
  int64_t cnt = 0;
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q) {
    if (kv[q] != ~0ull) {
      const int pos = tid * PER + q;
      const int64_t b = (int64_t)(uint32_t)kv[q];
      const bool kept = (pos < kstar) || (b >= wfirst);
      keep[blk_off + b] = kept ? 1 : 0;
      if (kept) cnt += (L - b * G) < G ? (L - b * G) : G;
    }
  }
  const int64_t total = block_sum_i64(cnt, red);
  if (tid == 0) cu_out[i + 1] = (int32_t)total;
}

// In-place inclusive scan of the per-request kept counts in cu_out[1..B]; cu_out[0] = 0.
__global__ __launch_bounds__(1024) void up_select_finalize_kernel(int32_t* __restrict__ cu_out,
                                                                  int B) {
  __shared__ int64_t buf[1024];
  __shared__ int64_t carry;
  const int tid = threadIdx.x;
  if (tid == 0) { carry = 0; cu_out[0] = 0; }
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    const int idx = base + tid;
    buf[tid] = idx < B ? cu_out[idx + 1] : 0;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int64_t v = tid >= d ? buf[tid - d] : 0;
      __syncthreads();
      buf[tid] += v;
      __syncthreads();
    }
    if (idx < B) cu_out[idx + 1] = (int32_t)(carry + buf[tid]);
    __syncthreads();
    if (tid == 1023) carry += buf[1023];
    __syncthreads();
  }
}

hipError_t launch_select(const float* scores, const int32_t* cu, int B, int n, int G, int mode,
                         float p, int topk, int nb_max, int64_t T_host, int64_t nb_tot_host,
                         uint8_t* keep, int32_t* cu_out, int* err, hipStream_t st) {
  if (B == 0) return hipSuccess;
  int NP = 1;
  while (NP < nb_max) NP <<= 1;
  const size_t lds = (size_t)(NP > kSelThreads ? NP : kSelThreads) * sizeof(uint64_t);
  hipLaunchKernelGGL(up_select_kernel, dim3(B), dim3(kSelThreads), lds, st, scores, cu, B, n, G,
                     mode, p, topk, NP, T_host, nb_tot_host, keep, cu_out, err);
  return hipGetLastError();
}

hipError_t launch_select_finalize(int32_t* cu_out, int B, hipStream_t st) {
  hipLaunchKernelGGL(up_select_finalize_kernel, dim3(1), dim3(1024), 0, st, cu_out, B);
  return hipGetLastError();
}

}  // namespace up

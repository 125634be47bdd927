// Top-p / Top-k block selection on the GPU, one workgroup per request.
//
// [UP] "Top-p selection" paragraph: blocks sorted by descending importance are kept
// until their cumulative sum reaches p; [UP] "Triton kernels" paragraph: the
// selection runs on the GPU with no host round trip; [UP] "ablation" paragraph:
// Top-k (a fixed count) is the alternative the ablation compares against.
//
// Order: score descending, ties by the lower block index.  The kept set is the
// shortest prefix of that order whose exact running sum reaches p, so it is fixed
// by one key, the cut: the (score, index) of the last kept block.  Nothing is
// sorted.  The cut's score is found by a radix select over the float bits (a score
// in [0, 1] has 30 significant bits: 7 exponent bits, 23 fraction bits), four
// passes from the top: the exponent, then fraction digits of 8, 8 and 7 bits.  Each
// pass histograms the candidates still in play by digit -- a count and an exact sum
// per bin, spread over eight copies against LDS atomic contention -- and takes the
// first bin, walking digits downwards, whose cumulative sum reaches what is left of p.
//
// Sums are exact integers.  A float32 in [0, 1] is M * 2^sh units of 2^-149, with M
// its 24-bit significand and sh = max(exponent - 1, 0).  The first digit fixes the
// exponent, so a first-pass bin total is (sum of M) << sh, compared as a 192-bit
// integer; after that every candidate shares sh and the remainder of p is carried
// as a 64-bit count of 2^sh units.  Integer sums are order-independent, so the cut
// equals the one a sequential exact running sum over the sorted order gives.
// Among the blocks whose score equals the cut score (ties), the remainder decides
// how many are kept, taken in ascending block index.
#include "up_dpp.h"
#include "up_internal.h"

namespace up {

struct U192 {
  uint64_t lo, mid, hi;
};

__device__ __forceinline__ U192 u192_zero() { return U192{0, 0, 0}; }

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

// a - b for a >= b.
__device__ __forceinline__ U192 u192_sub(U192 a, U192 b) {
  U192 r;
  r.lo = a.lo - b.lo;
  const uint64_t b0 = a.lo < b.lo;
  const uint64_t t = a.mid - b.mid;
  const uint64_t b1 = a.mid < b.mid;
  r.mid = t - b0;
  const uint64_t b2 = t < b0;
  r.hi = a.hi - b.hi - b1 - b2;
  return r;
}

__device__ __forceinline__ bool u192_geq(U192 a, U192 b) {
  if (a.hi != b.hi) return a.hi > b.hi;
  if (a.mid != b.mid) return a.mid > b.mid;
  return a.lo >= b.lo;
}

// x << sh for x < 2^64 and 0 <= sh <= 127.
__device__ __forceinline__ U192 u192_shl(uint64_t x, int sh) {
  U192 r = u192_zero();
  if (sh == 0) {
    r.lo = x;
  } else if (sh < 64) {
    r.lo = x << sh;
    r.mid = x >> (64 - sh);
  } else if (sh == 64) {
    r.mid = x;
  } else if (sh < 128) {
    r.mid = x << (sh - 64);
    r.hi = x >> (128 - sh);
  }
  return r;
}

// ceil(a / 2^sh) for 0 <= sh <= 127, when the result is known to be below 2^64.
__device__ __forceinline__ uint64_t u192_shr_ceil(U192 a, int sh) {
  uint64_t q;
  bool rem;
  if (sh == 0) {
    q = a.lo;
    rem = false;
  } else if (sh < 64) {
    q = (a.lo >> sh) | (a.mid << (64 - sh));
    rem = (a.lo << (64 - sh)) != 0;
  } else if (sh == 64) {
    q = a.mid;
    rem = a.lo != 0;
  } else {
    q = (a.mid >> (sh - 64)) | (a.hi << (128 - sh));
    rem = a.lo != 0 || (a.mid << (128 - sh)) != 0;
  }
  return q + (rem ? 1 : 0);
}

__device__ __forceinline__ U192 u192_shfl_up(U192 v, int d) {
  U192 r;
  r.lo = __shfl_up(v.lo, d);
  r.mid = __shfl_up(v.mid, d);
  r.hi = __shfl_up(v.hi, d);
  return r;
}

// Float bits of a score clamped into [0, 1] (NaN counts as 0); scores produced by
// up_block_scores are always in [0, 1].  The bits are below 2^30.
__device__ __forceinline__ uint32_t score_bits(float s) {
  if (!(s > 0.f)) return 0u;
  return __float_as_uint(s > 1.f ? 1.f : s);
}

// Significand M and shift sh of float bits u: the value is M * 2^sh units of 2^-149.
__device__ __forceinline__ uint32_t sig_of(uint32_t u) {
  const uint32_t e = u >> 23, f = u & 0x7FFFFFu;
  return e ? (f | 0x800000u) : f;
}
__device__ __forceinline__ int shift_of_exp(uint32_t e) { return e ? (int)e - 1 : 0; }

template <int CTRL, int ROWMASK>
__device__ __forceinline__ U192 dpp_in192(U192 v) {
  return U192{dpp_in64<CTRL, ROWMASK>(v.lo), dpp_in64<CTRL, ROWMASK>(v.mid),
              dpp_in64<CTRL, ROWMASK>(v.hi)};
}

__device__ __forceinline__ U192 wave_scan_u192(U192 v) {
  v = u192_add(v, dpp_in192<0x111, 0xf>(v));
  v = u192_add(v, dpp_in192<0x112, 0xf>(v));
  v = u192_add(v, dpp_in192<0x114, 0xf>(v));
  v = u192_add(v, dpp_in192<0x118, 0xf>(v));
  v = u192_add(v, dpp_in192<0x142, 0xa>(v));
  v = u192_add(v, dpp_in192<0x143, 0xc>(v));
  return v;
}

constexpr int kSelPer = 16;                      // most candidate slots per thread
constexpr int kBins = 256;                       // digits of at most 8 bits
constexpr int kCopies = 8;                       // lane l adds into histogram copy l % 8
constexpr uint32_t kAbsent = 0xFFFFFFFFu;        // no block in this slot
static_assert(kSelectMaxBlocks <= 1024 * kSelPer, "select slots");

// Digit passes over the 30 score bits: the exponent (bits 29..23), then the
// fraction in 8, 8 and 7 bits.
__device__ __forceinline__ int digit_shift(int pass) {
  return pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
}

template <int NW>
struct SelLds {
  uint32_t cnt[kBins * kCopies];
  uint64_t sum[kBins * kCopies];
  U192 wtot192[NW];
  uint64_t wtot64[NW];
  uint32_t wtot32[NW];
  int64_t red[NW];
  uint32_t tie_cnt[kSelPer * NW];
  uint32_t tie_pre[kSelPer * NW];
  int64_t dtot[kSelPer * NW];   // fused decision: kept tokens per (slot, wave)
  double red64[NW];             // fused decision: wave sums of the block masses
  int win;            // (thread) index of the bin holding the cut, from the top
  uint32_t prefix;    // cut digits found so far
  uint64_t rem;       // remainder of p in units of 2^sh of the cut's exponent
  uint32_t rem_k;     // remainder of the count (Top-k)
  uint32_t ties;      // blocks whose score equals the cut score
  uint32_t full;      // the cut's score bits, when a pass leaves one candidate
  int keep_all;
};

// Inclusive scans over the workgroup in thread order: DPP within each wave, then
// the totals of the lower waves (read as independent LDS loads).
template <int NW, typename Lds>
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, Lds& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_u32(v);
  if (lane == 63) S.wtot32[wave] = v;
  __syncthreads();
  uint32_t pre = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = S.wtot32[w];
    pre += w < wave ? t : 0u;
  }
  return pre + v;
}
template <int NW, typename Lds>
__device__ __forceinline__ uint64_t block_scan_u64(uint64_t v, Lds& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_u64(v);
  if (lane == 63) S.wtot64[wave] = v;
  __syncthreads();
  uint64_t pre = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t t = S.wtot64[w];
    pre += w < wave ? t : 0ull;
  }
  return pre + v;
}
template <int NW, typename Lds>
__device__ __forceinline__ U192 block_scan_u192(U192 v, Lds& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_u192(v);
  if (lane == 63) S.wtot192[wave] = v;
  __syncthreads();
  U192 pre = u192_zero();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const U192 t = S.wtot192[w];
    if (w < wave) pre = u192_add(pre, t);
  }
  return u192_add(pre, v);
}
// Sum over the workgroup, the same value in every thread (integer: order-free).
template <int NW, typename Lds>
__device__ __forceinline__ int64_t block_sum_i64(int64_t v, Lds& S) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = (int64_t)wave_scan_u64((uint64_t)v);
  if (lane == 63) S.red[wave] = v;
  __syncthreads();
  int64_t r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += S.red[w];
  return r;
}

// NT threads per request; block a of the request lives in slot a / NT of thread a % NT,
// PER slots per thread (the launch takes the fewest that hold the request: every phase
// loops over the slots, so empty ones cost time).
//
// FUSED (NT = 256, requests of at most 4096 blocks): the kernel also does the
// normalisation and the block destinations of the compaction, so the decision needs
// neither the normalise nor the block-destination launch.  It reads the float64 block
// masses, sums them in the order the normalise kernel uses (per thread over blocks tid,
// tid + 256, ..., then the lanes by butterfly, then the four waves in order) so the
// float32 scores it writes are bit-identical, selects on them, and writes each block's
// destination row, source row and length.  One request (direct): absolute
// destinations and the compaction header's valid flag.  Several: destinations relative
// to the request's first output row, each block's request index and the kept count
// (-1 when a check failed); up_select_finalize_fused_kernel completes them.
template <int NT, int PER, bool FUSED>
__global__ __launch_bounds__(NT) void up_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ cu, int B, int n, int G,
    int mode, float p, int topk, int64_t T_host, int64_t nb_tot_host, int direct,
    uint8_t* __restrict__ keep, int32_t* __restrict__ cu_out, int* __restrict__ err,
    FusedDecision fd) {
  constexpr int NW = NT / 64;
  constexpr int MAXB = NT * PER;
  static_assert(PER >= 1 && PER <= kSelPer, "slots per thread");
  __shared__ SelLds<NW> S;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // A single request starts at block 0 and has the host's block count, so its scores
  // are fetched before cu_seqlens is back; the device values are checked after.
  uint32_t u[PER];
  int64_t blk_off = 0;
  if constexpr (FUSED) {
    if (fd.shdr->valid != 1) {   // the score pass did not run: no masses to select on
      if (tid == 0) {
        if (direct) {
          fd.chdr->valid = 0;
          cu_out[0] = 0;
          cu_out[1] = 0;
        } else {
          cu_out[i + 1] = -1;   // the fused finalize then writes nothing
        }
      }
      return;
    }
    // One request: its blocks start at 0, host's count.  Several: the score plan's
    // offsets (valid: the header says the plan matches the host totals).
    int64_t mnb = nb_tot_host;
    if (!direct) {
      blk_off = fd.splan[i].blk_off;
      mnb = fd.splan[i].nb;
    }
    double mv[PER];
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int64_t a = (int64_t)q * NT + tid;
      mv[q] = a < mnb ? fd.mass[blk_off + a] : 0.0;
      part += mv[q];
    }
#pragma unroll
    for (int dd = 32; dd > 0; dd >>= 1) part += __shfl_xor(part, dd);
    if (lane == 0) S.red64[wave] = part;
    __syncthreads();
    const double tot = (S.red64[0] + S.red64[1]) + (S.red64[2] + S.red64[3]);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int64_t a = (int64_t)q * NT + tid;
      if (a < mnb) {
        const float sc = (float)(mv[q] / tot);
        fd.scores[blk_off + a] = sc;
        u[q] = __float_as_uint(sc);
      } else {
        u[q] = kAbsent;
      }
    }
  } else if (direct) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int64_t a = (int64_t)q * NT + tid;
      u[q] = a < nb_tot_host ? __float_as_uint(scores[a]) : kAbsent;
    }
  } else {
    // First global block of this request: sum of the earlier requests' block counts.
    int64_t part = 0;
    for (int r = tid; r < i; r += NT) {
      const int64_t Lr = (int64_t)cu[r + 1] - cu[r];
      part += Lr > 0 ? (Lr + G - 1) / G : 0;
    }
    blk_off = block_sum_i64<NW>(part, S);
  }
  const int64_t cu_lo = cu[i];
  const int64_t L = (int64_t)cu[i + 1] - cu_lo;
  const int64_t nb = L > 0 ? (L + G - 1) / G : 0;
  const bool bad = (L < 0) || ((int64_t)cu[B] != T_host) || (blk_off + nb > nb_tot_host) ||
                   (nb > MAXB) || (cu[0] != 0);
  if (bad) {
    if (tid == 0) {
      atomicOr(err, 1);
      cu_out[i + 1] = (FUSED && !direct) ? -1 : 0;
      if (direct) cu_out[0] = 0;
      if (FUSED && direct) fd.chdr->valid = 0;
    }
    return;
  }
  if (!direct && !FUSED) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int64_t a = (int64_t)q * NT + tid;
      u[q] = a < nb ? __float_as_uint(scores[blk_off + a]) : kAbsent;
    }
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int64_t a = (int64_t)q * NT + tid;
    u[q] = a < nb ? score_bits(__uint_as_float(u[q])) : kAbsent;
  }
  const int64_t W = L < n ? L : n;
  const int64_t wfirst = (L - W) / G;   // first block holding a window token

  // How many of the top blocks the cut keeps, as a target the passes narrow down.
  const int64_t kcount = mode == 1 ? (topk < nb ? topk : nb) : nb;
  const bool all = mode == 1 ? (kcount >= nb) : !(p < 1.0f);
  const bool none = mode == 1 && kcount == 0;
  if (tid == 0) {
    S.keep_all = all ? 1 : 0;
    S.prefix = 0;
    S.rem_k = (uint32_t)kcount;
    S.rem = 0;
    S.ties = 0;
  }
  __syncthreads();
  uint32_t ustar = kAbsent;   // the cut's score bits
  uint32_t jtie = 0;          // ties at the cut score that are kept
  const int copy = lane & (kCopies - 1);

  if (!all && !none && nb > 0) {
    bool early = false;   // a pass left a single candidate
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int dsh = digit_shift(pass);
      for (int e = tid; e < kBins * kCopies; e += NT) {
        S.cnt[e] = 0;
        S.sum[e] = 0;
      }
      if (tid == 0) S.win = kBins;
      __syncthreads();
      const uint32_t pre = S.prefix;
      const int hsh = pass == 0 ? 30 : digit_shift(pass - 1);   // bits above this digit
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const uint32_t x = u[q];
        if (x != kAbsent && (pass == 0 || (x >> hsh) == pre)) {
          const uint32_t dg = (x >> dsh) & ((1u << (hsh - dsh)) - 1u);
          atomicAdd(&S.cnt[dg * kCopies + copy], 1u);
          if (mode == 0)
            atomicAdd((unsigned long long*)&S.sum[dg * kCopies + copy],
                      (unsigned long long)sig_of(x));
        }
      }
      __syncthreads();
      // Thread t looks at digit kBins-1-t: ascending threads walk digits downwards.
      const int dg = kBins - 1 - tid;
      uint32_t c = 0;
      uint64_t m = 0;
      if (dg >= 0) {
#pragma unroll
        for (int k = 0; k < kCopies; ++k) {
          c += S.cnt[dg * kCopies + k];
          if (mode == 0) m += S.sum[dg * kCopies + k];
        }
      }
      // The winning bin is read into a register right after the barrier that follows
      // the atomicMin: thread 0 resets S.win at the start of the next pass, which it can
      // reach once every wave has passed the pass's last barrier, so S.win must not be
      // read after that barrier.
      int win = kBins;
      if (mode == 0) {
        if (pass == 0) {
          const int sh = shift_of_exp((uint32_t)(dg >= 0 ? dg : 0));   // the digit is the exponent
          const U192 v = u192_shl(m, sh);
          const U192 inc = block_scan_u192<NW>(v, S);
          // P: p as units of 2^-149 (p is a float32 in (0, 1)).
          const uint32_t pb = __float_as_uint(p);
          const U192 P = u192_shl(sig_of(pb), shift_of_exp(pb >> 23));
          if (c > 0 && u192_geq(inc, P)) atomicMin(&S.win, tid);
          __syncthreads();
          win = S.win;
          if (tid == win) {
            // What is left of p after every block of a higher exponent, in 2^sh units.
            S.rem = u192_shr_ceil(u192_sub(P, u192_sub(inc, v)), sh);
            S.prefix = (uint32_t)dg;
            S.ties = c;
          }
        } else {
          const uint64_t inc = block_scan_u64<NW>(m, S);
          const uint64_t target = S.rem;
          if (c > 0 && inc >= target) atomicMin(&S.win, tid);
          __syncthreads();
          win = S.win;
          if (tid == win) {
            S.rem = target - (inc - m);
            S.prefix = (pre << (hsh - dsh)) | (uint32_t)dg;
            S.ties = c;
          }
        }
      } else {
        const uint32_t inc = block_scan_u32<NW>(c, S);
        const uint32_t target = S.rem_k;
        if (c > 0 && inc >= target) atomicMin(&S.win, tid);
        __syncthreads();
        win = S.win;
        if (tid == win) {
          S.rem_k = target - (inc - c);
          S.prefix = pass == 0 ? (uint32_t)dg : ((pre << (hsh - dsh)) | (uint32_t)dg);
          S.ties = c;
        }
      }
      __syncthreads();
      if (pass == 0 && win == kBins) {
        // Every running sum stays below p: all blocks are kept.
        if (tid == 0) S.keep_all = 1;
        __syncthreads();
        break;
      }
      // One candidate left in the winning bin: it is the cut (the remainder it has to
      // meet is at most its own value, so one tie is kept), and the later passes would
      // only recover its remaining digits.  S.ties and S.prefix are written by the next
      // pass's winner only after that pass's first barrier, which every wave reaches
      // after these reads; the branch is the same in every wave.
      if (pass < 3 && S.ties == 1) {
        const uint32_t pfx = S.prefix;
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (u[q] != kAbsent && (u[q] >> dsh) == pfx) S.full = u[q];
        __syncthreads();
        early = true;
        break;
      }
    }
    if (!S.keep_all) {
      ustar = early ? S.full : S.prefix;
      if (mode == 0) {
        // The remainder is met by j ties of value sig(ustar) * 2^sh each.
        const uint64_t t = sig_of(ustar);
        const uint64_t r = S.rem;
        jtie = t == 0 ? 1u : (uint32_t)((r + t - 1) / t);
        if (jtie == 0) jtie = 1;
      } else {
        jtie = S.rem_k;
      }
    }
  }
  const bool keep_all = S.keep_all != 0;
  const uint32_t ties = S.ties;

  // When the cut splits a run of ties, rank them in ascending block index: slot-major,
  // then wave, then lane, which is the order a = q * NT + tid.
  uint32_t tie_rank[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) tie_rank[q] = 0;
  if (ustar != kAbsent && jtie < ties) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const uint64_t msk = __ballot(u[q] == ustar);
      tie_rank[q] = (uint32_t)__popcll(msk & ((1ull << lane) - 1));
      if (lane == 0) S.tie_cnt[q * NW + wave] = (uint32_t)__popcll(msk);
    }
    __syncthreads();
    if (wave == 0) {
      // Exclusive scan of the PER * NW tie counts, E per lane.
      constexpr int E = (PER * NW + 63) / 64;
      uint32_t loc[E], sl = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int idx = lane * E + e;
        loc[e] = idx < PER * NW ? S.tie_cnt[idx] : 0u;
        sl += loc[e];
      }
      uint32_t run = wave_scan_u32(sl) - sl;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int idx = lane * E + e;
        if (idx < PER * NW) S.tie_pre[idx] = run;
        run += loc[e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) tie_rank[q] += S.tie_pre[q * NW + wave];
  }

  // Keep flags and kept-token count.
  int64_t cnt = 0;
  uint32_t kl[FUSED ? PER : 1];   // fused: kept tokens of each slot's block (<= G)
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const uint32_t x = u[q];
    if constexpr (FUSED) kl[q] = 0;
    if (x != kAbsent) {
      const int64_t b = (int64_t)q * NT + tid;
      bool kept = keep_all || b >= wfirst;
      if (!kept && ustar != kAbsent)
        kept = x > ustar || (x == ustar && tie_rank[q] < jtie);
      keep[blk_off + b] = kept ? 1 : 0;
      if (kept) {
        const int64_t bl = (L - b * G) < G ? (L - b * G) : G;
        cnt += bl;
        if constexpr (FUSED) kl[q] = (uint32_t)bl;
      }
    }
  }
  const int64_t total = block_sum_i64<NW>(cnt, S);
  if (tid == 0) {
    cu_out[i + 1] = (int32_t)total;
    if (direct) cu_out[0] = 0;
  }
  if constexpr (FUSED) {
    // Destination of block b = kept tokens of blocks 0..b-1.  Blocks are slot-major
    // (b = q NT + tid): a wave scan per slot, then the slot and wave totals.
    uint32_t incl[PER];   // within a wave: at most 64 blocks of <= 1024 tokens
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      incl[q] = wave_scan_u32(kl[q]);
      if (lane == 63) S.dtot[q * NW + wave] = (int64_t)incl[q];
    }
    __syncthreads();
    int64_t before = 0;   // kept tokens of all earlier slots
    bool dst_bad = false;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      int64_t pre = before, slot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int64_t t = S.dtot[q * NW + w];
        pre += w < wave ? t : 0;
        slot += t;
      }
      const int64_t b = (int64_t)q * NT + tid;
      if (b < nb) {
        // Relative to the request's first output row (one request: absolute).
        const int64_t dd = pre + (int64_t)(incl[q] - kl[q]);
        // A kept run must lie inside the kept-token count (which is at most T).
        if (kl[q] && (dd < 0 || dd + kl[q] > total)) dst_bad = true;
        fd.dst[blk_off + b] = kl[q] ? (int32_t)dd : -1;
        fd.src[blk_off + b] = (int32_t)(cu_lo + b * G);
        fd.len[blk_off + b] = (int32_t)((L - b * G) < G ? (L - b * G) : G);
        if (!direct) fd.rq[blk_off + b] = i;
      }
      before += slot;
    }
    // The slot totals must add up to the kept count, and every run must fit; only
    // then may the gather use the destinations.
    const int64_t nbad = block_sum_i64<NW>((dst_bad || before != total) ? 1 : 0, S);
    if (tid == 0) {
      const bool ok = nbad == 0 && total <= T_host;
      if (direct) {
        fd.chdr->valid = ok ? 1 : 0;
      } else if (!ok) {
        cu_out[i + 1] = -1;   // the fused finalize refuses the batch
      }
      if (!ok) atomicOr(err, 1);
    }
  }
}

// Requests of at most 256 blocks (block a in thread a): instead of the digit passes,
// every block finds its rank in the order (score descending, index ascending) by
// comparing itself with each block of the request, the scores are placed in rank
// order in LDS, and one exact integer scan over that order gives each rank the sum
// of the scores ranked before it.  The block at rank r is in the shortest prefix that
// reaches p exactly when that sum is still below p (Top-k: when r < k), which is the
// cut the digit passes find, so both give the same keep flags.
constexpr int kSmallSelBlocks = 256;

__global__ __launch_bounds__(kSmallSelBlocks) void up_select_small_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ cu, int B, int n, int G,
    int mode, float p, int topk, int64_t T_host, int64_t nb_tot_host, int direct,
    uint8_t* __restrict__ keep, int32_t* __restrict__ cu_out, int* __restrict__ err) {
  constexpr int NT = kSmallSelBlocks, NW = NT / 64;
  struct Lds {
    uint32_t u[NT];          // score bits by block
    uint32_t sorted[NT];     // score bits by rank
    uint8_t keep_rank[NT];   // kept, by rank
    U192 wtot192[NW];
    int64_t red[NW];
  };
  __shared__ Lds S;
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  int64_t blk_off = 0;
  if (!direct) {
    int64_t part = 0;
    for (int r = tid; r < i; r += NT) {
      const int64_t Lr = (int64_t)cu[r + 1] - cu[r];
      part += Lr > 0 ? (Lr + G - 1) / G : 0;
    }
    blk_off = block_sum_i64<NW>(part, S);
  }
  const int64_t L = (int64_t)cu[i + 1] - cu[i];
  const int64_t nb = L > 0 ? (L + G - 1) / G : 0;
  const bool bad = (L < 0) || ((int64_t)cu[B] != T_host) || (blk_off + nb > nb_tot_host) ||
                   (nb > NT) || (cu[0] != 0);
  if (bad) {
    if (tid == 0) {
      atomicOr(err, 1);
      cu_out[i + 1] = 0;
      if (direct) cu_out[0] = 0;
    }
    return;
  }
  const bool mine = tid < nb;
  const uint32_t u = mine ? score_bits(scores[blk_off + tid]) : 0u;
  S.u[tid] = u;
  __syncthreads();
  uint32_t rank = 0;
  if (mine) {
    for (int j = 0; j < (int)nb; ++j) {
      const uint32_t x = S.u[j];
      rank += (x > u || (x == u && j < tid)) ? 1u : 0u;
    }
    S.sorted[rank] = u;
  }
  __syncthreads();
  // Thread r holds rank r: the exact sum of the scores ranked before it, in units of
  // 2^-149 (a score in [0, 1] is its significand times 2^sh, see sig_of).
  const bool have = tid < nb;
  const uint32_t x = have ? S.sorted[tid] : 0u;
  const U192 v = have ? u192_shl(sig_of(x), shift_of_exp(x >> 23)) : u192_zero();
  const U192 incl = block_scan_u192<NW>(v, S);
  const U192 before = u192_sub(incl, v);
  if (have) {
    bool k;
    if (mode == 1) {
      k = (int64_t)tid < (int64_t)topk;
    } else if (!(p < 1.0f)) {
      k = true;
    } else {
      const uint32_t pb = __float_as_uint(p);
      const U192 P = u192_shl(sig_of(pb), shift_of_exp(pb >> 23));
      k = !u192_geq(before, P);
    }
    S.keep_rank[tid] = k ? 1 : 0;
  }
  __syncthreads();
  const int64_t W = L < n ? L : n;
  const int64_t wfirst = (L - W) / G;   // first block holding a window token
  int64_t cnt = 0;
  if (mine) {
    const bool kept = S.keep_rank[rank] != 0 || (int64_t)tid >= wfirst;
    keep[blk_off + tid] = kept ? 1 : 0;
    if (kept) cnt = (L - (int64_t)tid * G) < G ? (L - (int64_t)tid * G) : G;
  }
  const int64_t total = block_sum_i64<NW>(cnt, S);
  if (tid == 0) {
    cu_out[i + 1] = (int32_t)total;
    if (direct) cu_out[0] = 0;
  }
}

// In-place inclusive scan of the per-request kept counts in cu_out[1..B]; cu_out[0] = 0.
__global__ __launch_bounds__(1024) void up_select_finalize_kernel(int32_t* __restrict__ cu_out,
                                                                  int B) {
  struct FinLds {
    uint64_t wtot64[16];
  };
  __shared__ FinLds S;
  const int tid = threadIdx.x;
  if (tid == 0) cu_out[0] = 0;
  // Counts 1024 at a time: wave scans, then the lower waves' totals.
  int64_t carry = 0;   // the same in every thread
  for (int base = 0; base < B; base += 1024) {
    const int idx = base + tid;
    const int64_t c = idx < B ? cu_out[idx + 1] : 0;
    const uint64_t inc = block_scan_u64<16>((uint64_t)c, S);
    if (idx < B) cu_out[idx + 1] = (int32_t)(carry + (int64_t)inc);
    uint64_t round = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) round += S.wtot64[w];
    carry += (int64_t)round;
    __syncthreads();   // the next round rewrites S
  }
}

// The fused decision over several requests: scan the per-request kept counts the
// select workgroups left in cu_out[1..B] into cu_seqlens_out, then make every kept
// block's destination absolute (its request's first output row plus its destination
// within the request) and write the compaction header.  A request whose checks failed
// left -1: then cu_seqlens_out is all zeros and the header invalid (the gather moves
// nothing).
__global__ __launch_bounds__(1024) void up_select_finalize_fused_kernel(
    int32_t* __restrict__ cu_out, int B, int64_t T_host, int64_t nb_tot_host, int* __restrict__ err,
    FusedDecision fd) {
  constexpr int kOffs = 4096;   // request offsets kept in LDS for packs below this size
  struct FinLds {
    uint64_t wtot64[16];
  };
  __shared__ FinLds S;
  __shared__ int32_t offs[kOffs];
  const int tid = threadIdx.x;
  const bool lds_offs = B < kOffs;
  if (tid == 0) {
    cu_out[0] = 0;   // request 0's first output row (read below)
    if (lds_offs) offs[0] = 0;
  }
  // Counts 1024 at a time: wave scans, then the lower waves' totals.
  bool bad_c = false;
  int64_t carry = 0;   // the same in every thread
  for (int base = 0; base < B; base += 1024) {
    const int idx = base + tid;
    const int64_t c = idx < B ? cu_out[idx + 1] : 0;
    if (c < 0) bad_c = true;
    const uint64_t inc = block_scan_u64<16>((uint64_t)(c < 0 ? 0 : c), S);
    if (idx < B) {
      const int32_t o = (int32_t)(carry + (int64_t)inc);
      cu_out[idx + 1] = o;
      if (lds_offs) offs[idx + 1] = o;
    }
    uint64_t round = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) round += S.wtot64[w];
    carry += (int64_t)round;
    __syncthreads();   // the next round rewrites S
  }
  const int64_t total = carry;
  const bool ok_counts = !__syncthreads_or(bad_c ? 1 : 0) && total <= T_host;
  // Absolute destinations; a run must fit inside the kept count.  A thread takes four
  // blocks at a time, their loads issued together.
  bool run_bad = false;
  if (ok_counts) {
    constexpr int U = 4;
    for (int64_t b0 = tid; b0 < nb_tot_host; b0 += U * 1024) {
      int32_t d[U], r[U], ln[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t b = b0 + (int64_t)u * 1024;
        const bool in = b < nb_tot_host;
        d[u] = in ? fd.dst[b] : -1;
        r[u] = in ? fd.rq[b] : 0;
        ln[u] = in ? fd.len[b] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (d[u] < 0) continue;
        if (r[u] < 0 || r[u] >= B) { run_bad = true; continue; }
        const int64_t ad = (int64_t)(lds_offs ? offs[r[u]] : cu_out[r[u]]) + d[u];
        if (ad + ln[u] > total) run_bad = true;
        fd.dst[b0 + (int64_t)u * 1024] = (int32_t)ad;
      }
    }
  }
  const int any = __syncthreads_or(run_bad ? 1 : 0);
  const bool ok = ok_counts && !any;
  if (!ok) {
    for (int idx = tid; idx <= B; idx += 1024) cu_out[idx] = 0;
  }
  if (tid == 0) {
    fd.chdr->valid = ok ? 1 : 0;
    if (!ok) atomicOr(err, 1);
  }
}

// Slots per thread of a 256-thread select for a request of nb blocks: the fewest of
// 1, 2, 4, 8, 16 that hold it (nb <= 256 * kSelPer).
static int sel_slots(int64_t nb) {
  int per = 1;
  while (per < kSelPer && (int64_t)256 * per < nb) per *= 2;
  return per;
}

template <bool FUSED>
static void launch_select256(int per, int B, hipStream_t st, const float* scores,
                             const int32_t* cu, int n, int G, int mode, float p, int topk,
                             int64_t T_host, int64_t nb_tot_host, int direct, uint8_t* keep,
                             int32_t* cu_out, int* err, const FusedDecision& fd) {
#define UP_SEL_LAUNCH(P)                                                                   \
  hipLaunchKernelGGL((up_select_kernel<256, P, FUSED>), dim3(B), dim3(256), 0, st, scores, \
                     cu, B, n, G, mode, p, topk, T_host, nb_tot_host, direct, keep, cu_out,  \
                     err, fd)
  switch (per) {
    case 1: UP_SEL_LAUNCH(1); break;
    case 2: UP_SEL_LAUNCH(2); break;
    case 4: UP_SEL_LAUNCH(4); break;
    case 8: UP_SEL_LAUNCH(8); break;
    default: UP_SEL_LAUNCH(kSelPer); break;
  }
#undef UP_SEL_LAUNCH
}

hipError_t launch_select(const float* scores, const int32_t* cu, int B, int n, int G, int mode,
                         float p, int topk, int nb_max, int64_t T_host, int64_t nb_tot_host,
                         uint8_t* keep, int32_t* cu_out, int* err, hipStream_t st) {
  if (B == 0) return hipSuccess;
  // One request: its count is cu_out[1] itself, no scan launch needed.
  const int direct = B == 1 ? 1 : 0;
  const FusedDecision none{};
  if (nb_max <= kSmallSelBlocks) {
    hipLaunchKernelGGL(up_select_small_kernel, dim3(B), dim3(kSmallSelBlocks), 0, st, scores, cu,
                       B, n, G, mode, p, topk, T_host, nb_tot_host, direct, keep, cu_out, err);
  } else if (nb_max <= 256 * kSelPer) {
    launch_select256<false>(sel_slots(nb_max), B, st, scores, cu, n, G, mode, p, topk, T_host,
                            nb_tot_host, direct, keep, cu_out, err, none);
  } else {
    hipLaunchKernelGGL((up_select_kernel<1024, kSelPer, false>), dim3(B), dim3(1024), 0, st,
                       scores, cu, B, n, G, mode, p, topk, T_host, nb_tot_host, direct, keep,
                       cu_out, err, none);
  }
  return hipGetLastError();
}

hipError_t launch_select_fused(const int32_t* cu, int B, int n, int G, float p, int nb_max,
                               int64_t T_host, int64_t nb_tot_host, uint8_t* keep,
                               int32_t* cu_out, int* err, const FusedDecision& fd,
                               hipStream_t st) {
  static_assert(kFusedSelectMaxBlocks <= 256 * kSelPer, "fused select slots");
  if (B < 1 || nb_max > kFusedSelectMaxBlocks) return hipErrorInvalidValue;
  launch_select256<true>(sel_slots(nb_max), B, st, nullptr, cu, n, G, 0, p, 0, T_host,
                         nb_tot_host, B == 1 ? 1 : 0, keep, cu_out, err, fd);
  if (B > 1)
    hipLaunchKernelGGL(up_select_finalize_fused_kernel, dim3(1), dim3(1024), 0, st, cu_out, B,
                       T_host, nb_tot_host, err, fd);
  return hipGetLastError();
}

hipError_t launch_select_finalize(int32_t* cu_out, int B, hipStream_t st) {
  if (B == 1) return hipSuccess;   // written by the select kernel
  hipLaunchKernelGGL(up_select_finalize_kernel, dim3(1), dim3(1024), 0, st, cu_out, B);
  return hipGetLastError();
}

}  // namespace up

// Block scores on CDNA4 (gfx950).
//
// What is computed ([UP] "drop" and "block-wise estimation" paragraphs; [CP] causal
// mask over absolute positions): for every window row (query head h, window row j
// at absolute position t) the softmax over keys 0..t of scale * q.k, summed over
// heads, rows and the G keys of each block, normalised per request.
//
// How: one pass over the keys on the matrix cores instead of the two-pass
// max-then-sum that an online softmax usually takes.  For each (row, block) the
// kernel keeps the block-local maximum m_b and the block-local sum
// l_b = sum_{k in b} 2^(x_k - m_b) (x = logit * scale * log2 e).  Row statistics
// (m, l) follow by the usual online-softmax merge, and a block's mass is
// sum_rows 2^(m_b - m) * l_b / l -- the same quantity, rearranged.  This reads K
// once and runs Q K^T once, half the matrix-core work and key traffic of two passes.
//
// Kernels (all launched on the caller's stream, in this order):
//   up_score_plan_kernel     per-request offsets from the device cu_seqlens, checked
//                            against the host-derived totals
//   up_score_partial_kernel  Q K^T on bf16 MFMA (32x32x16), per-(row, block) block sums
//                            and per-(row, key chunk) merged statistics
//   up_row_stats_kernel      merge chunk statistics into per-row (m, 1 / l), and each
//                            (row, chunk)'s weight of its block sums
//   up_block_mass_kernel     per-block mass, float64 sums in a fixed order
//   up_normalize_kernel      per-request normalisation to scores that sum to one
// (up_block_mass_pairs_kernel serves the attention's fused form, whose row statistics
// come from the attention kernel itself.)
#include "up_dpp.h"
#include "up_internal.h"

#include <math.h>

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

static constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax merge of (m, s) into (M, S), both in log2 units: afterwards
// S * 2^M = S_old * 2^M_old + s * 2^m.  An empty side has m = -inf, s = 0.
__device__ __forceinline__ void merge_ml(float& M, float& S, float m, float s) {
  if (m > M) {
    S = S * fast_exp2(M - m) + s;   // M = -inf gives 0 * 0 + s
    M = m;
  } else if (m != kNegInf) {
    S += s * fast_exp2(m - M);
  }
}

// Number of requests whose work items end at or before x, i.e. the request holding
// work item x.  Every lane of the wave must call it (wave-wide ballot).
__device__ __forceinline__ int request_of_item(const ReqPlan* __restrict__ plan, int B, int x) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  for (int base = 0; base < B; base += 64) {
    const int i = base + lane;
    const bool pred = (i < B) && (plan[i].item_end <= x);
    cnt += __popcll(__ballot(pred));
  }
  return cnt;
}

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------
// One workgroup of kPlanThreads; requests are taken kPlanThreads at a time, thread t
// planning request base + t, and the per-request counts are scanned into offsets
// (DPP within each wave, the wave totals through LDS, a carry between rounds).
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void up_score_plan_kernel(
    const int32_t* __restrict__ cu, ScoreShape s, Totals host, WsHeader* __restrict__ hdr,
    ReqPlan* __restrict__ plan, int* __restrict__ err) {
  constexpr int NW = kPlanThreads / 64;
  constexpr int NV = 6;   // scanned quantities: W, nb, items, ml, cs, pm
  __shared__ int64_t wtot[NV][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gs = s.Hq / s.Hkv;
  // Every check is one workgroup vote at the end, so the first and last entries of
  // cu_seqlens are read together with the requests' own.
  bool bad = tid == 0 && cu[0] != 0;
  const int32_t cu_end = tid == 0 ? cu[s.B] : 0;
  int64_t carry[NV] = {0, 0, 0, 0, 0, 0};
  for (int base = 0; base < s.B; base += kPlanThreads) {
    const int i = base + tid;
    int64_t v[NV] = {0, 0, 0, 0, 0, 0};
    ReqPlan p{};
    if (i < s.B) {
      const int32_t a = cu[i], b = cu[i + 1];
      int64_t L = (int64_t)b - a;
      if (L < 0) { bad = true; L = 0; }
      const int64_t W = L < s.n ? L : s.n;
      const int64_t nb = (L + s.G - 1) / s.G;
      const int64_t R = gs * W;
      const int64_t nrt = (R + s.rows_wg - 1) / s.rows_wg;
      const int cbs = stat_chunk_blocks(nb, s.Hkv * nrt);
      const int64_t nch = (nb + cbs - 1) / cbs;
      const int cps = chunks_per_item(cbs, nch, s.TB);
      v[0] = W;
      v[1] = nb;
      v[2] = (nch + cps - 1) / cps * s.Hkv * nrt;
      v[3] = nb * s.Hkv * R;
      v[4] = nch * s.Hkv * R;
      v[5] = nb * s.Hkv * nrt;
      p.tok_off = a; p.L = (int32_t)L; p.W = (int32_t)W; p.nb = (int32_t)nb;
      p.nch = (int32_t)nch; p.cbs = cbs; p.cps = cps;
    }
    int64_t inc[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      inc[q] = (int64_t)wave_scan_u64((uint64_t)v[q]);
      if (lane == 63) wtot[q][wave] = inc[q];
    }
    __syncthreads();
    int64_t pre[NV], tot[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      pre[q] = carry[q];
      tot[q] = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int64_t t = wtot[q][w];
        pre[q] += w < wave ? t : 0;
        tot[q] += t;
      }
    }
    __syncthreads();   // the next round overwrites wtot
    if (i < s.B) {
      p.win_off = (int32_t)(pre[0] + inc[0] - v[0]);
      p.blk_off = (int32_t)(pre[1] + inc[1] - v[1]);
      p.item_end = (int32_t)(pre[2] + inc[2]);            // inclusive
      p.ml_off = pre[3] + inc[3] - v[3];
      p.cs_off = pre[4] + inc[4] - v[4];
      p.pm_off = pre[5] + inc[5] - v[5];
      plan[i] = p;
    }
#pragma unroll
    for (int q = 0; q < NV; ++q) carry[q] += tot[q];
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (tid == 0) {
    const bool ok = !any_bad && (int64_t)cu_end == host.T && carry[0] == host.win_rows &&
                    carry[1] == host.nb_tot && carry[2] == host.items &&
                    carry[3] == host.ml_pairs && carry[4] == host.cs_pairs &&
                    carry[5] == host.pm_parts;
    hdr->valid = ok ? 1 : 0;
    if (!ok) atomicOr(err, 1);
  }
}

// ---------------------------------------------------------------------------
// Partial statistics on the matrix cores
//
// Workgroup = NW waves = one (request, kv head g, query-row tile, work item: a run of
// the request's statistics chunks, see stat_chunk_blocks).  Each
// wave holds QT tiles of 32 query rows of kv head g's group in VGPRs as the B
// operand (rows r = j * gs + hh: window row j, head g*gs + hh).  Keys stream through
// a ring of NS LDS stages of 64 keys: each stage is copied straight from global
// memory into LDS (global_load_lds_dwordx4, no VGPR round trip) by all lanes, NS-2
// stages ahead of use, and one barrier per stage publishes it and frees the slot the
// previous stage used.  Rows are unpadded; their 16-byte granules are XOR-swizzled
// so A-operand reads are free of bank conflicts.  Keys are the A operand, so
// S^T = K Q^T lands with one query per lane column: lane l and lane l^32 together
// hold the 32 keys of a half-stage for query l%32.
//
// The keys are processed in halves of 32: the MFMAs of half h+1 are issued between
// the exp/sum instructions of half h, on two accumulator sets.  The main loop is
// unrolled over the ring so every LDS offset is a compile-time constant.
//
// Softmax statistics: one running reference Rs per query (log2 units), the same in
// both lanes of the query, and each lane's sums l = sum 2^(x - Rs) over its keys of
// the current block and statistics chunk.  Any reference gives the same (reference,
// sum) value, so there is no per-block max pass; only when a half's sum leaves
// [0, 2^64] (overflow, or the unset reference of a statistics chunk's first half)
// does the wave rebase the affected queries on the pair's maximum (a wave-uniform
// branch, rare).  At a block end the partner lane's sum is added with
// v_permlane32_swap and one lane stores (Rs, l_b); at a statistics chunk's end its
// sums are stored likewise and the reference is reset, so every stored value depends
// only on the keys of its own chunk, whatever work item the chunk ran in.
//
// The head dimension is contracted in a permuted order that both operands share:
// lane half h, k-step s holds d-elements [h*D/2 + 8s, h*D/2 + 8s + 8), so every
// lane reads one contiguous D-byte run per row.
// ---------------------------------------------------------------------------

constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64

// Lanes l and l^32 hold the two key halves of one query.  v_permlane32_swap(x, x)
// returns x of the low lane in [0] and of the high lane in [1], in both lanes.
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);   // same operand order in both lanes
}
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// K rows live in LDS without padding; 16-byte granules of a row are XOR-swizzled
// so that the 16 lanes of an LDS read phase (16 consecutive keys, same granule)
// hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_swizzle(int key) {
  return (D / 8 >= 16) ? (key & 15) : ((key >> 1) & 7);
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane i of the wave writes LDS bytes [m0 + 16 i, m0 + 16 i + 16) and reads 16 bytes
// at a wave-uniform 64-bit base (held in SGPRs) plus its own 32-bit byte offset, so a
// lane spends no vector instructions on 64-bit address arithmetic.  Issued from
// inline assembly so that the compiler does not drain every outstanding load at the
// next LDS read; completion is awaited explicitly (vmcnt) before the barrier that
// publishes a stage.  NTL marks the copies non-temporal: the d = 256 pass reads twice
// the key bytes per flop of d = 128, and with non-temporal copies its decision step is
// faster (the pass 171-174 -> 139-140 us, the next compaction 293 -> 317 us, the step
// 497 -> 489 us at 128K tokens); at d = 128 the same policy made the step slower, so
// only the d = 256 instances take it.
template <bool NTL = false>
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t voff, uint32_t m0) {
  // readfirstlane returns a signed int: both halves go through uint32_t before they
  // are widened, so the low word is zero-extended, never sign-extended.
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t sa = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (NTL)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(reinterpret_cast<const void*>(sa)),
                 "{m0}"(m0)
                 : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(reinterpret_cast<const void*>(sa)),
                 "{m0}"(m0)
                 : "memory");
}

// Wait until at most n vector-memory operations of this wave are outstanding and all
// LDS operations are done, then barrier.  n is a small constant known per call site.
__device__ __forceinline__ void wait_vm_lgkm_barrier(int n) {
  // s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
#define UP_WAIT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (0 << 8))
  switch (n) {
    case 0: UP_WAIT(0); break;
    case 1: UP_WAIT(1); break;
    case 2: UP_WAIT(2); break;
    case 3: UP_WAIT(3); break;
    case 4: UP_WAIT(4); break;
    case 5: UP_WAIT(5); break;
    case 6: UP_WAIT(6); break;
    case 7: UP_WAIT(7); break;
    case 8: UP_WAIT(8); break;
    case 9: UP_WAIT(9); break;
    case 10: UP_WAIT(10); break;
    case 11: UP_WAIT(11); break;
    case 12: UP_WAIT(12); break;
    case 13: UP_WAIT(13); break;
    case 14: UP_WAIT(14); break;
    case 15: UP_WAIT(15); break;
    default: UP_WAIT(0); break;
  }
#undef UP_WAIT
  asm volatile("s_barrier" ::: "memory");
}

// LSE = true: the given-lse pass.  Each query's reference is its own log-sum-exp
// (row_lse * log2 e), so 2^(x - Rs) are the softmax probabilities themselves and no
// rebase ever happens; at a block end the workgroup sums the block's probabilities
// (DPP within each wave, then the waves through LDS at the chunk end) and writes one
// float partial per (block, kv head, row tile) to pm instead of per-row statistics.
//
// PAGED = true: keys come from a paged cache kmat = [num_pages][page][Hkv][D] through
// the request's row of the block table (pages of 2^lps tokens, lps >= 4).  A 64-key
// stage spans at most four pages; their indices are wave-uniform scalar loads made
// one stage ahead.  Table slots are clamped to the row and page indices outside
// [0, num_pages) read page 0 and raise error bit 8, so no input reaches memory out of
// bounds.
template <int D, int QT, int NS, int NW, bool LSE, bool PAGED>
__global__ __launch_bounds__(64 * NW, 8 / NW) void up_score_partial_kernel(
    const uint16_t* __restrict__ qwin, const uint16_t* __restrict__ kmat,
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq, int Hkv,
    int G, float c, float* __restrict__ ml, float* __restrict__ mref, int32_t* __restrict__ crb,
    float2* __restrict__ cs,
    const float* __restrict__ row_lse, float* __restrict__ pm,
    const int32_t* __restrict__ btab, int max_pages, int lps, int64_t num_pages,
    int* __restrict__ err) {
  constexpr int NT = 64 * NW;
  constexpr int UK = 64;               // keys per LDS stage (two 32-key halves)
  constexpr int RB = 2 * D;            // LDS bytes per key row
  constexpr int SB = UK * RB;          // LDS bytes per stage
  constexpr int SPT = SB / (NT * 16);  // 16-byte DMA copies per lane per stage
  constexpr int DS = D / 16;           // MFMA k-steps over the head dimension
  constexpr int ROWS = NW * QT * 32;   // query rows per workgroup
  constexpr int EPS = 16 / DS;         // softmax elements per tile per k-step
  static_assert(SB % (NT * 16) == 0, "stage must be a whole number of DMA rounds");
  static_assert((NS - 2) * SPT <= 15, "vmcnt wait range");
  static_assert((NS & (NS - 1)) == 0, "ring length must be a power of two");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * SB];
  __shared__ float blk_acc[LSE ? kMaxChunkBlocks * NW : 1];   // per (block, wave) sums

  if (hdr->valid != 1) return;
  const int x = blockIdx.x;
  const int i = request_of_item(plan, B, x);
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  const int gs = Hq / Hkv;
  const int R = gs * pr.W;
  const int nrt = (R + ROWS - 1) / ROWS;
  int xl = x - (i > 0 ? plan[i - 1].item_end : 0);
  const int g = xl % Hkv;
  xl /= Hkv;
  const int rt = xl % nrt;
  const int it = xl / nrt;              // work item within the (request, kv head, row tile)
  const int ch0 = it * pr.cps;          // its first statistics chunk

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int row0 = rt * ROWS + wave * (QT * 32);

  // Query operand, resident for the whole chunk.
  bf16x8 qreg[QT][DS];
  int qpos[QT];
  float lse_ref[QT];   // given-lse pass: the row's log-sum-exp in log2 units (+inf: no row)
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int r = row0 + t * 32 + l32;
    lse_ref[t] = __builtin_inff();
    if (r < R) {
      const int j = r / gs, hh = r - j * gs;
      const int64_t qrow = (int64_t)(pr.win_off + j) * Hq + g * gs + hh;
      const uint16_t* src = qwin + qrow * D + half * (D / 2);
#pragma unroll
      for (int s = 0; s < DS; ++s) qreg[t][s] = *reinterpret_cast<const bf16x8*>(src + s * 8);
      qpos[t] = pr.L - pr.W + j;
      if (LSE) lse_ref[t] = row_lse[qrow] * 1.4426950408889634f;
    } else {
#pragma unroll
      for (int s = 0; s < DS; ++s) qreg[t][s] = bf16x8{};
      qpos[t] = -1;   // inactive row: every key masked in masked halves, never stored
    }
  }
  // Q is in registers before any K copy is issued: the waits below count K copies only.
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)

  const int b0 = ch0 * pr.cbs;
  const int b1 = min(pr.nb, b0 + pr.cps * pr.cbs);
  const int k0 = b0 * G;
  const int kend = min(b1 * G, pr.L);
  const int nh = (kend - k0 + 31) / 32;          // 32-key halves in this chunk
  const int nst = (nh + 1) / 2;                  // LDS stages
  const int64_t kstride = (int64_t)Hkv * D;
  const uint16_t* kbase =
      PAGED ? kmat + (int64_t)g * D : kmat + ((int64_t)pr.tok_off * Hkv + g) * D;
  const int32_t* trow = PAGED ? btab + (int64_t)i * max_pages : nullptr;
  bool bad_page = false;
  // A wave's copy q of a stage fetches 1024 bytes: 1024 / RB consecutive keys, aligned
  // to their count (2, 4 or 8), so inside one page (pages hold at least 16 keys; keys
  // past the request read its last key, still inside that page).  Its page index is
  // therefore wave-uniform: one scalar load per copy, made one stage ahead.
  int pf_stage = -1;
  int pf_pg[SPT];
  auto load_pages = [&](int st, int (&pg)[SPT]) {
    const int ks = k0 + st * UK;
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
      const int key0 = __builtin_amdgcn_readfirstlane((q * NT * 16 + wave * 1024) / RB);
      const int slot =
          __builtin_amdgcn_readfirstlane(min(min(ks + key0, pr.L - 1) >> lps, max_pages - 1));
      int p = trow[slot];
      if (p < 0 || (int64_t)p >= num_pages) { bad_page = true; p = 0; }
      pg[q] = p;
    }
  };
  const int fast_limit = pr.L - pr.W;   // keys <= this are visible to every window row
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8*)lds;   // LDS byte address

  // Per-lane constants: where this lane's DMA copies come from and land, and where its
  // A-operand reads are (granule half*DS+s of key l32, swizzled; key 32+l32 is 32 rows on).
  // Byte offsets are 32-bit: a stage spans 64 keys of kstride2 bytes (the host keeps
  // 64 * kstride2 below 2^31).
  const uint32_t kstride2 = (uint32_t)(kstride * 2);
  uint32_t dma_voff[SPT];   // from the stage's first key (full stages, contiguous keys)
  uint32_t dma_gran[SPT];   // the swizzled 16-byte granule within the key's row
  uint32_t dma_loff[SPT];
  int dma_key[SPT];
#pragma unroll
  for (int q = 0; q < SPT; ++q) {
    const int o = q * NT * 16 + tid * 16;
    const int key = o / RB;
    const int p = ((o % RB) / 16) ^ k_swizzle<D>(key);
    dma_key[q] = key;
    dma_gran[q] = (uint32_t)p * 16;
    dma_voff[q] = (uint32_t)key * kstride2 + dma_gran[q];
    dma_loff[q] = q * NT * 16 + wave * 1024;   // wave-uniform
  }
  uint32_t rd_off[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) rd_off[s] = l32 * RB + 16 * ((half * DS + s) ^ k_swizzle<D>(l32));

  // Issue the DMA copies of stage st into ring slot st % NS.  Keys past the request read
  // its last key instead (they are masked); nothing is read out of bounds.
  auto stage_issue = [&](int st) {
    const int ks = k0 + st * UK;
    const uint32_t sbase = lds_base + (uint32_t)((st & (NS - 1)) * SB);
    if constexpr (PAGED) {
      int pg[SPT];
      if (pf_stage == st) {
#pragma unroll
        for (int q = 0; q < SPT; ++q) pg[q] = pf_pg[q];
      } else {
        load_pages(st, pg);
      }
      const int pmask = (1 << lps) - 1;
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        const int kabs = min(ks + dma_key[q], pr.L - 1);
        lds_dma16_s(kbase + ((int64_t)pg[q] << lps) * kstride,
                    (uint32_t)(kabs & pmask) * kstride2 + dma_gran[q],
                    __builtin_amdgcn_readfirstlane(sbase + dma_loff[q]));
      }
      // The next stage's page indices, in flight while this stage's copies are.
      if (st + 1 < nst) {
        load_pages(st + 1, pf_pg);
        pf_stage = st + 1;
      }
      return;
    }
    const uint16_t* gb = kbase + (int64_t)ks * kstride;
    if (ks + UK <= pr.L) {
#pragma unroll
      for (int q = 0; q < SPT; ++q)
        lds_dma16_s<D == 256>(gb, dma_voff[q], __builtin_amdgcn_readfirstlane(sbase + dma_loff[q]));
    } else {
#pragma unroll
      for (int q = 0; q < SPT; ++q) {
        const int kabs = min(ks + dma_key[q], pr.L - 1);
        lds_dma16_s<D == 256>(gb, (uint32_t)(kabs - ks) * kstride2 + dma_gran[q],
                    __builtin_amdgcn_readfirstlane(sbase + dma_loff[q]));
      }
    }
  };
  // Make stage st visible: wait for its copies (later stages may stay in flight),
  // barrier, then refill the slot freed by stage st-1 with stage st+NS-1.
  auto stage_enter = [&](int st) {
    const int later = min(NS - 2, nst - 1 - st);   // stages issued after st
    wait_vm_lgkm_barrier(later * SPT);
    if (st + NS - 1 <= nst - 1) stage_issue(st + NS - 1);
  };

  // Softmax state.  Rs is one reference per query, identical in the two lanes that
  // hold the query's keys; lblk / Lch are each lane's sums over its own keys of the
  // current block / chunk, relative to Rs.
  float Rs[QT], lblk[QT], Lch[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    Rs[t] = LSE ? lse_ref[t] : kNegInf;
    lblk[t] = 0.f;
    Lch[t] = 0.f;
  }
  const int t_st = (QT == 2) ? half : 0;          // the tile this lane stores
  const int r_st = row0 + t_st * 32 + l32;
  const bool st_ok = (QT == 2 || half == 0) && (r_st < R);

  int hcnt = G / 32;   // halves left in the current block
  // Blocks end one at a time in order: the item-relative index of the next block to
  // end, and (full pass) where its (m, l) pair goes, advanced by one block per end.
  int blk_rel = 0;
  int ccnt = pr.cbs;   // blocks left in the current statistics chunk
  int chk = ch0;       // the current statistics chunk
  int64_t ml_at = st_ok ? pr.ml_off + ((int64_t)b0 * Hkv + g) * R + r_st : -1;
  const int64_t ml_step = (int64_t)Hkv * R;
  // The stored block sums of a chunk are relative to the chunk's final reference, except
  // that a rebase of a set reference in mid-chunk leaves the blocks ended before it
  // relative to the reference they ended under: the storing lane then writes that
  // reference to mref for those blocks, and keeps in first_cur the first block of the
  // chunk (chunk-relative) that ends under the current reference, stored with the
  // chunk's statistics.  ml_chunk: where block 0 of the current chunk goes.
  int first_cur = 0;
  int64_t ml_chunk = ml_at;
  f32x16 acc0[QT], acc1[QT];
  float pend_v = 0.f;   // block sum waiting to be stored
  int64_t pend_i = -1;
  auto flush_pending = [&]() {
    if (pend_i >= 0) ml[pend_i] = pend_v;
    pend_i = -1;
  };

  // MFMAs of half h into acc (LDS slot offset `so` bytes, runtime or constant).
  auto mfma_half = [&](uint32_t so, f32x16 (&acc)[QT]) {
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(lds + so + rd_off[s]);
#pragma unroll
      for (int t = 0; t < QT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[t][s], s == 0 ? f32x16{} : acc[t],
                                                         0, 0, 0);
    }
  };

  // Sum of 2^(x - Rs) over a lane's 16 values (masked keys give 0), even/odd partials.
  auto half_sums = [&](f32x16 (&acc)[QT], float (&sum)[QT]) {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        a0 += fast_exp2(fmaf(acc[t][e], c, -Rs[t]));
        a1 += fast_exp2(fmaf(acc[t][e + 1], c, -Rs[t]));
      }
      sum[t] = a0 + a1;
    }
  };

  // Apply the causal mask to half h's values (keys past a row's position -> -inf).
  auto mask_half = [&](int h, f32x16 (&acc)[QT]) {
    const int key0 = k0 + h * 32;
#pragma unroll
    for (int t = 0; t < QT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // 32x32 MFMA result layout: register e of lane l holds row
        // 8*(e/4) + 4*(l/32) + e%4 (the key) and column l%32 (the query).
        const int key = key0 + 8 * (e >> 2) + 4 * half + (e & 3);
        if (key > qpos[t]) acc[t][e] = kNegInf;
      }
  };

  // Rebase the reference of every query whose half left [0, 2^64] (a sum overflowed,
  // or the reference was unset) on the pair's maximum over this half; runs for the
  // whole wave, the lanes whose sums were fine get the same sums back.
  auto rebase = [&](f32x16 (&acc)[QT], float (&nl)[QT]) {
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float mx = kNegInf;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[t][e]);
      mx = pair_max(mx);
      if (mx == kNegInf) { nl[t] = lblk[t]; continue; }   // no visible key for this query
      const float rn = fmaxf(Rs[t], mx * c);
      if constexpr (!LSE) {
        if (t == t_st && st_ok && Rs[t] != kNegInf && rn != Rs[t]) {
          // blocks of this chunk that ended under the old reference keep it
          const int ended = pr.cbs - ccnt;
          for (int j = first_cur; j < ended; ++j) mref[ml_chunk + (int64_t)j * ml_step] = Rs[t];
          first_cur = ended;
        }
      }
      const float sc = fast_exp2(Rs[t] - rn);            // Rs = -inf gives 0 (sums were 0)
      lblk[t] *= sc;
      Lch[t] *= sc;
      Rs[t] = rn;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        a0 += fast_exp2(fmaf(acc[t][e], c, -rn));
        a1 += fast_exp2(fmaf(acc[t][e + 1], c, -rn));
      }
      nl[t] = lblk[t] + (a0 + a1);
    }
  };

  // Accumulate half h's sums; handle block ends.
  auto finish_half = [&](int h, f32x16 (&acc)[QT], const float (&sum)[QT]) {
    if constexpr (LSE) {
      // Probabilities already: accumulate; at a block end sum over the wave's 64 lanes
      // (all its queries and keys) and leave the wave's total in LDS.
#pragma unroll
      for (int t = 0; t < QT; ++t) lblk[t] += sum[t];
      if (--hcnt == 0 || h == nh - 1) {
        hcnt = G / 32;
        const int bl = blk_rel++;   // chunk-relative block
        float v = lblk[0];
#pragma unroll
        for (int t = 1; t < QT; ++t) v += lblk[t];
#pragma unroll
        for (int t = 0; t < QT; ++t) lblk[t] = 0.f;
        v = wave_scan_f32(v);
        if (lane == 63) blk_acc[bl * NW + wave] = v;
      }
      return;
    }
    float nl[QT];
    bool bad = false;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      nl[t] = lblk[t] + sum[t];
      bad = bad || !(nl[t] <= kSumLimit);
    }
    if (__ballot(bad) != 0) rebase(acc, nl);   // wave-uniform branch, rare
#pragma unroll
    for (int t = 0; t < QT; ++t) lblk[t] = nl[t];
    if (--hcnt == 0 || h == nh - 1) {
      hcnt = G / 32;
      float lst = 0.f;
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const float lp = pair_sum(lblk[t]);   // same value in both lanes
        if (t == t_st) lst = lp;
        Lch[t] += lblk[t];
        lblk[t] = 0.f;
      }
      // The store is issued after the next stage barrier (flush_pending).
      flush_pending();   // a block ended since the last barrier (G < 64): store it now
      pend_v = lst;
      pend_i = ml_at;
      if (st_ok) ml_at += ml_step;
      if (--ccnt == 0 || h == nh - 1) {
        // End of a statistics chunk: store its merged pair (the two lanes of a query
        // share the reference; add their sums), then restart the reference so the next
        // chunk's statistics depend on its own keys only.
        float mc = 0.f, lc = 0.f;
#pragma unroll
        for (int t = 0; t < QT; ++t) {
          const float lp = pair_sum(Lch[t]);
          if (t == t_st) { mc = Rs[t]; lc = lp; }
          Rs[t] = kNegInf;
          Lch[t] = 0.f;
        }
        if (st_ok) {
          const int64_t ci = pr.cs_off + ((int64_t)chk * Hkv + g) * R + r_st;
          cs[ci] = make_float2(lc > 0.f ? mc : kNegInf, lc);
          crb[ci] = first_cur;
        }
        ++chk;
        ccnt = pr.cbs;
        first_cur = 0;
        ml_chunk = ml_at;
      }
    }
  };

  // Fast step (half h and h+1 unmasked, h+1 < nh): MFMAs of h+1 from LDS slot offset
  // `so` interleaved with the exp-and-sum of h.
  auto step_fast = [&](int h, uint32_t so, f32x16 (&cur)[QT], f32x16 (&nxt)[QT]) {
    float part[QT][2];
    // All A operands of half h+1 are requested up front, in the order the MFMAs use
    // them (one scheduling region per read), so MFMA s waits for read s only.
    bf16x8 a[DS];
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
      a[ks] = *reinterpret_cast<const bf16x8*>(lds + so + rd_off[ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < DS; ++ks) {
#pragma unroll
      for (int t = 0; t < QT; ++t)
        nxt[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qreg[t][ks],
                                                         ks == 0 ? f32x16{} : nxt[t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < QT; ++t)
#pragma unroll
        for (int q = 0; q < EPS; ++q) {
          const int e = ks * EPS + q;
          const float v = fast_exp2(fmaf(cur[t][e], c, -Rs[t]));
          if (e < 2) part[t][e] = v; else part[t][e & 1] += v;
        }
    }
    float sum[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) sum[t] = part[t][0] + part[t][1];
    finish_half(h, cur, sum);
  };

  // Generic step: any half (masked or the chunk's last), runtime LDS slot.
  auto step_generic = [&](int h, f32x16 (&cur)[QT], f32x16 (&nxt)[QT]) {
    const bool more = h + 1 < nh;
    if (more && ((h + 1) & 1) == 0) {
      stage_enter((h + 1) / 2);
      flush_pending();
    }
    if (more) mfma_half((uint32_t)((((h + 1) / 2) & (NS - 1)) * SB + ((h + 1) & 1) * 32 * RB), nxt);
    if (k0 + h * 32 + 31 > fast_limit) mask_half(h, cur);
    float sum[QT];
    half_sums(cur, sum);
    finish_half(h, cur, sum);
  };

  // Prologue: stages 0 .. NS-2 in flight, stage 0 published, MFMAs of half 0.
  for (int st = 0; st <= NS - 2 && st < nst; ++st) stage_issue(st);
  stage_enter(0);
  mfma_half(0, acc0);

  // Main loop, unrolled over the ring: halves h .. h+2NS-1 (stages h/2 .. h/2+NS-1, ring
  // slots 0 .. NS-1) when every one of them and the next half are unmasked.
  int h = 0;
  while (h + 2 * NS < nh && k0 + (h + 2 * NS) * 32 + 31 <= fast_limit) {
#pragma unroll
    for (int j = 0; j < 2 * NS; ++j) {
      f32x16 (&cur)[QT] = (j & 1) ? acc1 : acc0;
      f32x16 (&nxt)[QT] = (j & 1) ? acc0 : acc1;
      if ((j & 1) == 1) {
        stage_enter((h + j + 1) / 2);
        flush_pending();
      }
      step_fast(h + j, (uint32_t)((((j + 1) / 2) & (NS - 1)) * SB + ((j + 1) & 1) * 32 * RB), cur, nxt);
    }
    h += 2 * NS;
  }
  // Tail: pairs of halves with static accumulator parity (h is even here).
  for (; h < nh; h += 2) {
    step_generic(h, acc0, acc1);
    if (h + 1 >= nh) break;
    step_generic(h + 1, acc1, acc0);
  }

  flush_pending();
  // Each wave checks only the page indices of its own copies: every wave reports.
  if (PAGED && bad_page && (tid & 63) == 0) atomicOr(err, 8);
  if constexpr (LSE) {
    // Block partials of this (kv head, row tile): the waves' totals in wave order.
    __syncthreads();
    for (int b = tid; b < b1 - b0; b += NT) {
      float v = blk_acc[b * NW];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += blk_acc[b * NW + w];
      pm[pr.pm_off + (int64_t)(g * nrt + rt) * pr.nb + b0 + b] = v;   // part-major
    }
  }
}

// ---------------------------------------------------------------------------
// Row statistics and chunk weights.
//
// The score kernel leaves, per (row, block), the block's sum l_b relative to the
// reference of its statistics chunk (the chunk's final reference Rc, stored with the
// chunk's statistics), except for the blocks that ended before a mid-chunk rebase, whose
// reference is in mref; per (row, chunk) first_cur says which blocks those are.  Here
// every (request, kv head, row)'s chunks are merged into (M, 1 / L), and every (row,
// chunk) gets the weight w = 2^(Rc - M) / L that turns its block sums into
// probabilities: w = -1 - first_cur (negative) for a (row, chunk) with a mid-chunk
// rebase, whose terms the block-mass kernel forms one by one.
// Output layout: rs[win_off*Hq + g*R + r] (the request's Hq*W rows, g-major); the
// weights in the chunk statistics' layout.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_of_row(const ReqPlan* __restrict__ plan, int B, int Hq,
                                              int64_t x) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)(plan[mid].win_off + plan[mid].W) * Hq <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Workgroup = 64 rows (one per lane) x 16 waves; wave w merges chunks w, w+16, ...
// of its lane's row in that order, wave 0 merges the 16 partial results in wave order,
// then wave w writes the weights of the same chunks.  The row's plan entry is read
// while the header's flag is in flight (a lone request needs no search; every index
// stays inside the plan) and used only once the flag says the plan is valid; a wave
// issues up to four chunks' loads at once and keeps its first four for the weights.
__global__ __launch_bounds__(1024) void up_row_stats_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq, int Hkv,
    const float2* __restrict__ cs, const int32_t* __restrict__ crb, float2* __restrict__ rs,
    float* __restrict__ wt, int64_t total_rows, float* __restrict__ row_lse) {
  __shared__ float2 part[16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t x = (int64_t)blockIdx.x * 64 + lane;
  const int valid = hdr->valid;
  int i = B;
  ReqPlan pr{};
  if (B == 1) {
    pr = plan[0];
    i = x < total_rows ? 0 : 1;
  } else if (x < total_rows) {
    i = request_of_row(plan, B, Hq, x);
    if (i < B) pr = plan[i];
  }
  if (valid != 1) return;
  float M = kNegInf, S = 0.f;
  int64_t lse_at = -1;   // the row's index in the [sum W, Hq] window-row layout
  int64_t c0 = -1;       // the row's pair of chunk 0; chunk chk at c0 + chk * cstep
  int64_t cstep = 0;
  int nch = 0;
  float rc0[4];          // the reference and rebase mark of chunks wave + 16 q
  int fc0[4];
  if (i < B) {
    const int gs = Hq / Hkv;
    const int R = gs * pr.W;
    const int64_t local = x - (int64_t)pr.win_off * Hq;   // = g*R + r
    const int g = (int)(local / R), r = (int)(local % R);
    lse_at = (int64_t)(pr.win_off + r / gs) * Hq + g * gs + r % gs;
    c0 = pr.cs_off + (int64_t)g * R + r;
    cstep = (int64_t)Hkv * R;
    nch = pr.nch;
    for (int base = wave; base < nch; base += 64) {
      float2 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chk = base + 16 * q;
        v[q] = chk < nch ? cs[c0 + chk * cstep] : make_float2(kNegInf, 0.f);
        if (base == wave) fc0[q] = chk < nch ? crb[c0 + chk * cstep] : 0;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (base + 16 * q < nch) merge_ml(M, S, v[q].x, v[q].y);
        if (base == wave) rc0[q] = v[q].x;
      }
    }
  }
  part[wave][lane] = make_float2(M, S);
  __syncthreads();
  if (wave == 0 && c0 >= 0) {
    float Mt = kNegInf, St = 0.f;
    for (int w = 0; w < 16; ++w) merge_ml(Mt, St, part[w][lane].x, part[w][lane].y);
    const float2 st = make_float2(Mt, St > 0.f ? 1.f / St : 0.f);   // (row max, 1 / row sum)
    rs[x] = st;
    part[0][lane] = st;
    // Natural-log log-sum-exp of the row's scaled logits: (M + log2 l) * ln 2.
    if (row_lse) row_lse[lse_at] = (Mt + log2f(St)) * 0.6931471805599453f;
  }
  __syncthreads();
  if (c0 >= 0) {
    const float2 st = part[0][lane];
    auto weight = [&](int fc, float rc) {
      return fc > 0 ? -1.f - (float)fc : fast_exp2(rc - st.x) * st.y;
    };
    for (int base = wave; base < nch; base += 64) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t chk = base + 16 * q;
        if (chk >= nch) continue;
        const int64_t ci = c0 + chk * cstep;
        wt[ci] = base == wave ? weight(fc0[q], rc0[q]) : weight(crb[ci], cs[ci].x);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Block masses.  mass[b] = sum_{g, r} l_b(r) w_c(r) over the block's Hq * W (row)
// terms, c the block's statistics chunk: each term in float32, summed in float64 in a
// fixed order (per thread over its terms, the terms of rebased (row, chunk)s after the
// others, then the workgroup).  One workgroup per global block.  (A
// last-workgroup-normalises variant needs an agent-scope release per workgroup, an L2
// writeback on every XCD, which costs far more than the separate normalisation launch.)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_of_block(const ReqPlan* __restrict__ plan, int B,
                                                int64_t x) {
  int lo = 0, hi = B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)plan[mid].blk_off + plan[mid].nb <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Sum over a 256-thread workgroup in a fixed order (butterfly within each wave, then
// the four wave sums in order); every thread gets the same value.
__device__ __forceinline__ double wg256_sum_f64(double v, double* red) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void up_block_mass_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq,
    const float* __restrict__ lb, const float* __restrict__ mref, const float* __restrict__ wt,
    const float2* __restrict__ cs, const float2* __restrict__ rs, double* __restrict__ mass) {
  __shared__ double red[4];
  const int64_t blk = blockIdx.x;
  // The plan entry is read while the header's flag is in flight (a lone request needs no
  // search; every index stays inside the plan) and used only once the flag says the
  // plan is valid.
  const int valid = hdr->valid;
  const int i = B == 1 ? 0 : request_of_block(plan, B, blk);
  ReqPlan pr{};
  if (i < B) pr = plan[i];
  if (valid != 1 || i >= B) return;
  const int64_t b = blk - pr.blk_off;
  const int64_t c = b / pr.cbs;                    // the block's statistics chunk
  const int j = (int)(b - c * pr.cbs);             // its index within the chunk
  const int64_t terms = (int64_t)Hq * pr.W;        // Hkv * R
  const int64_t lo = pr.ml_off + b * terms;        // the block's sums (and mref)
  const int64_t wo = pr.cs_off + c * terms;        // its chunk's weights (and statistics)
  const float* lrow = lb + lo;
  const float* wrow = wt + wo;
  constexpr int U = 4;
  double acc = 0.0;
  float wmin = 0.f;
  if ((terms & 3) == 0 && ((lo | wo) & 3) == 0) {
    // four terms per 16-byte load; thread t takes quads t, t + 256, ... in order
    const float4* l4 = reinterpret_cast<const float4*>(lrow);
    const float4* w4 = reinterpret_cast<const float4*>(wrow);
    const int64_t quads = terms >> 2;
    int64_t e = threadIdx.x;
    auto add4 = [&](float4 l, float4 w) {
      wmin = fminf(wmin, fminf(fminf(w.x, w.y), fminf(w.z, w.w)));
      acc += (double)(l.x * fmaxf(w.x, 0.f));
      acc += (double)(l.y * fmaxf(w.y, 0.f));
      acc += (double)(l.z * fmaxf(w.z, 0.f));
      acc += (double)(l.w * fmaxf(w.w, 0.f));
    };
    for (; e + (U - 1) * 256 < quads; e += U * 256) {
      float4 v[U], w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u] = l4[e + u * 256];
        w[u] = w4[e + u * 256];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) add4(v[u], w[u]);
    }
    for (; e < quads; e += 256) add4(l4[e], w4[e]);
  } else {
    for (int64_t e = threadIdx.x; e < terms; e += 256) {
      const float w = wrow[e];
      wmin = fminf(wmin, w);
      acc += (double)(lrow[e] * fmaxf(w, 0.f));
    }
  }
  if (__syncthreads_or(wmin < 0.f)) {
    // Rows whose chunk had a mid-chunk rebase (rare): each term with the reference its
    // block ended under, in the thread's order.
    const float2* srow = rs + (int64_t)pr.win_off * Hq;
    for (int64_t e = threadIdx.x; e < terms; e += 256) {
      const float w = wrow[e];
      if (!(w < 0.f)) continue;
      const int fc = (int)(-w) - 1;   // first block under the chunk's final reference
      const float ref = j < fc ? mref[lo + e] : cs[wo + e].x;
      const float2 st = srow[e];
      acc += (double)(lrow[e] * fast_exp2(ref - st.x) * st.y);
    }
  }
  const double tot = wg256_sum_f64(acc, red);
  if (threadIdx.x == 0) mass[blk] = tot;
}

// The attention's fused form: mass[b] = sum_{g, r} l_b * 2^(m_b - M) * (1 / l) from
// (reference, sum) pairs per (row, block) and the row statistics (M, 1 / l).
__global__ __launch_bounds__(256) void up_block_mass_pairs_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq,
    const float2* __restrict__ ml, const float2* __restrict__ rs, double* __restrict__ mass) {
  __shared__ double red[4];
  if (hdr->valid != 1) return;
  const int64_t blk = blockIdx.x;
  const int i = request_of_block(plan, B, blk);
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  const int64_t b = blk - pr.blk_off;
  const int64_t terms = (int64_t)Hq * pr.W;           // Hkv * R
  const float2* mrow = ml + pr.ml_off + b * terms;
  const float2* rrow = rs + (int64_t)pr.win_off * Hq;
  constexpr int U = 8;
  double acc = 0.0;
  if ((terms & 1) == 0 && (((uintptr_t)mrow | (uintptr_t)rrow) & 15) == 0) {
    // two consecutive terms per 16-byte load; thread t sums terms 2t, 2t + 1, then
    // those 512 on, in that order
    const float4* m4 = reinterpret_cast<const float4*>(mrow);
    const float4* r4 = reinterpret_cast<const float4*>(rrow);
    const int64_t pairs = terms >> 1;
    int64_t e = threadIdx.x;
    for (; e + (U - 1) * 256 < pairs; e += U * 256) {
      float4 v[U], w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u] = m4[e + u * 256];
        w[u] = r4[e + u * 256];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc += (double)(v[u].y * fast_exp2(v[u].x - w[u].x) * w[u].y);
        acc += (double)(v[u].w * fast_exp2(v[u].z - w[u].z) * w[u].w);
      }
    }
    for (; e < pairs; e += 256) {
      const float4 v = m4[e], w = r4[e];
      acc += (double)(v.y * fast_exp2(v.x - w.x) * w.y);
      acc += (double)(v.w * fast_exp2(v.z - w.z) * w.w);
    }
  } else {
    int64_t e = threadIdx.x;
    for (; e + (U - 1) * 256 < terms; e += U * 256) {
      float2 v[U], w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u] = mrow[e + u * 256];
        w[u] = rrow[e + u * 256];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc += (double)(v[u].y * fast_exp2(v[u].x - w[u].x) * w[u].y);
    }
    for (; e < terms; e += 256) {
      const float2 v = mrow[e], w = rrow[e];
      acc += (double)(v.y * fast_exp2(v.x - w.x) * w.y);
    }
  }
  const double tot = wg256_sum_f64(acc, red);
  if (threadIdx.x == 0) mass[blk] = tot;
}

// ---------------------------------------------------------------------------
// Normalise: scores[b] = mass[b] / sum of the request's masses.  One workgroup
// per request; the sum has a fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void up_normalize_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B,
    const double* __restrict__ mass, float* __restrict__ scores) {
  __shared__ double red[4];
  if (hdr->valid != 1) return;
  const int i = blockIdx.x;
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  double acc = 0.0;
  for (int b = threadIdx.x; b < pr.nb; b += 256) acc += mass[pr.blk_off + b];
  const double tot = wg256_sum_f64(acc, red);
  for (int b = threadIdx.x; b < pr.nb; b += 256)
    scores[pr.blk_off + b] = (float)(mass[pr.blk_off + b] / tot);
}

// ---------------------------------------------------------------------------
// Given-lse pass: scores[b] = (sum of the block's partials over kv heads and row
// tiles) / (the request's total), float64 sums in a fixed order.  One workgroup per
// request.  Partials are part-major ([Hkv * nrt][nb]), so the loads of one part are
// coalesced across blocks and the parts of a block are independent loads; the
// masses of the first kFinMass blocks stay in LDS for the second sweep.
// ---------------------------------------------------------------------------
constexpr int kFinThreads = 1024;
constexpr int kFinMass = 4096;

__global__ __launch_bounds__(kFinThreads) void up_lse_finalize_kernel(
    const WsHeader* __restrict__ hdr, const ReqPlan* __restrict__ plan, int B, int Hq, int Hkv,
    int rows_wg, const float* __restrict__ pm, float* __restrict__ scores) {
  __shared__ double mass_lds[kFinMass];
  __shared__ double red[kFinThreads / 64];
  if (hdr->valid != 1) return;
  const int i = blockIdx.x;
  if (i >= B) return;
  const ReqPlan pr = plan[i];
  const int R = (Hq / Hkv) * pr.W;
  const int parts = Hkv * ((R + rows_wg - 1) / rows_wg);
  const float* base = pm + pr.pm_off;
  const int64_t nb = pr.nb;
  auto mass = [&](int64_t b) {
    double m0 = 0.0, m1 = 0.0, m2 = 0.0, m3 = 0.0;
    int q = 0;
    for (; q + 3 < parts; q += 4) {
      m0 += (double)base[(int64_t)q * nb + b];
      m1 += (double)base[(int64_t)(q + 1) * nb + b];
      m2 += (double)base[(int64_t)(q + 2) * nb + b];
      m3 += (double)base[(int64_t)(q + 3) * nb + b];
    }
    for (; q < parts; ++q) m0 += (double)base[(int64_t)q * nb + b];
    return (m0 + m1) + (m2 + m3);
  };
  double acc = 0.0;
  for (int64_t b = threadIdx.x; b < nb; b += kFinThreads) {
    const double m = mass(b);
    if (b < kFinMass) mass_lds[b] = m;
    acc += m;
  }
  // Fixed-order sum: butterfly within each wave, then the wave sums in order.
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  double tot = 0.0;
  for (int w = 0; w < kFinThreads / 64; ++w) tot += red[w];
  for (int64_t b = threadIdx.x; b < nb; b += kFinThreads)
    scores[pr.blk_off + b] = (float)((b < kFinMass ? mass_lds[b] : mass(b)) / tot);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
ScoreWs score_ws_layout(int B, const Totals& t) {
  ScoreWs L;
  size_t off = align_up(sizeof(WsHeader));
  L.plan = off; off = align_up(off + (size_t)B * sizeof(ReqPlan));
  L.ml = off;   off = align_up(off + (size_t)t.ml_pairs * sizeof(float2));
  L.cs = off;   off = align_up(off + (size_t)t.cs_pairs * sizeof(float2));
  L.crb = off;  off = align_up(off + (size_t)t.cs_pairs * sizeof(int32_t));
  L.wt = off;   off = align_up(off + (size_t)t.cs_pairs * sizeof(float));
  L.rs = off;   off = align_up(off + (size_t)t.rows * sizeof(float2));
  L.mass = off; off = align_up(off + (size_t)t.nb_tot * sizeof(double));
  L.total = off;
  return L;
}

ScoreLseWs score_lse_ws_layout(int B, const Totals& t) {
  ScoreLseWs L;
  size_t off = align_up(sizeof(WsHeader));
  L.plan = off; off = align_up(off + (size_t)B * sizeof(ReqPlan));
  L.pm = off;   off = align_up(off + (size_t)t.pm_parts * sizeof(float));
  L.total = off;
  return L;
}

static inline char* wsb(void* ws) { return static_cast<char*>(ws); }

hipError_t launch_score_plan(const int32_t* cu, const ScoreShape& s, const Totals& t, void* ws,
                             size_t plan_off, int* err, hipStream_t st) {
  hipLaunchKernelGGL(up_score_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, cu, s, t,
                     reinterpret_cast<WsHeader*>(wsb(ws)),
                     reinterpret_cast<ReqPlan*>(wsb(ws) + plan_off), err);
  return hipGetLastError();
}

// Inputs and outputs of one launch of the score kernel (the unused ones are null).
struct PartialOut {
  size_t plan_off;
  float* ml;      // per (row, block) block sums
  float* mref;    // per (row, block) references of blocks ended before a mid-chunk rebase
  int32_t* crb;   // per (row, chunk) first block under the chunk's final reference
  float2* cs;
  const float* row_lse;
  float* pm;
  PagedK pk;
};

template <int D, int QT, int NS, int NW, bool LSE, bool PAGED>
static hipError_t launch_partial_t(const void* qwin, const void* k, const ScoreShape& s,
                                   const Totals& t, void* ws, const PartialOut& o, float c,
                                   hipStream_t st) {
  static_assert(NW * QT * 32 == score_rows_wg(D), "row tile of the kernel and of the plan");
  hipLaunchKernelGGL((up_score_partial_kernel<D, QT, NS, NW, LSE, PAGED>),
                     dim3((unsigned)t.items), dim3(64 * NW), 0,
                     st, static_cast<const uint16_t*>(qwin), static_cast<const uint16_t*>(k),
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + o.plan_off), s.B, s.Hq, s.Hkv,
                     s.G, c, o.ml, o.mref, o.crb, o.cs, o.row_lse, o.pm, o.pk.table, o.pk.max_pages,
                     o.pk.log2_page, o.pk.num_pages, o.pk.err);
  return hipGetLastError();
}

template <bool LSE, bool PAGED>
static hipError_t launch_partial_d(const void* qwin, const void* k, const ScoreShape& s,
                                   const Totals& t, void* ws, const PartialOut& o, float c,
                                   hipStream_t st) {
  if (t.items == 0) return hipSuccess;
  switch (s.d) {
    case 64: return launch_partial_t<64, 2, 8, 8, LSE, PAGED>(qwin, k, s, t, ws, o, c, st);
    case 128: return launch_partial_t<128, 2, 4, 8, LSE, PAGED>(qwin, k, s, t, ws, o, c, st);
    case 256: return launch_partial_t<256, 1, 4, 8, LSE, PAGED>(qwin, k, s, t, ws, o, c, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score_partial(const void* qwin, const void* k, const ScoreShape& s,
                                const Totals& t, void* ws, const ScoreWs& L, float c,
                                const PagedK* paged, hipStream_t st) {
  // The pair region holds the block sums in its first half and mref in its second.
  float* lb = reinterpret_cast<float*>(wsb(ws) + L.ml);
  PartialOut o{L.plan, lb, lb + t.ml_pairs, reinterpret_cast<int32_t*>(wsb(ws) + L.crb),
               reinterpret_cast<float2*>(wsb(ws) + L.cs), nullptr, nullptr, PagedK{}};
  if (paged) {
    o.pk = *paged;
    return launch_partial_d<false, true>(qwin, k, s, t, ws, o, c, st);
  }
  return launch_partial_d<false, false>(qwin, k, s, t, ws, o, c, st);
}

hipError_t launch_score_partial_lse(const void* qwin, const void* k, const float* row_lse,
                                    const ScoreShape& s, const Totals& t, void* ws,
                                    const ScoreLseWs& L, float c, const PagedK* paged,
                                    hipStream_t st) {
  PartialOut o{L.plan, nullptr, nullptr, nullptr, nullptr, row_lse,
               reinterpret_cast<float*>(wsb(ws) + L.pm), PagedK{}};
  if (paged) {
    o.pk = *paged;
    return launch_partial_d<true, true>(qwin, k, s, t, ws, o, c, st);
  }
  return launch_partial_d<true, false>(qwin, k, s, t, ws, o, c, st);
}

hipError_t launch_lse_finalize(const ScoreShape& s, const Totals& t, void* ws,
                               const ScoreLseWs& L, float* scores, hipStream_t st) {
  if (s.B == 0 || t.nb_tot == 0) return hipSuccess;
  hipLaunchKernelGGL(up_lse_finalize_kernel, dim3(s.B), dim3(kFinThreads), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq, s.Hkv,
                     s.rows_wg, reinterpret_cast<const float*>(wsb(ws) + L.pm), scores);
  return hipGetLastError();
}

hipError_t launch_row_stats(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                            float* row_lse, hipStream_t st) {
  if (t.rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((t.rows + 63) / 64);
  hipLaunchKernelGGL(up_row_stats_kernel, dim3(grid), dim3(1024), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq, s.Hkv,
                     reinterpret_cast<const float2*>(wsb(ws) + L.cs),
                     reinterpret_cast<const int32_t*>(wsb(ws) + L.crb),
                     reinterpret_cast<float2*>(wsb(ws) + L.rs),
                     reinterpret_cast<float*>(wsb(ws) + L.wt), t.rows, row_lse);
  return hipGetLastError();
}

hipError_t launch_block_mass(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                             hipStream_t st) {
  if (t.nb_tot == 0) return hipSuccess;
  // the pair region holds the block sums in its first half and mref in its second
  const float* lb = reinterpret_cast<const float*>(wsb(ws) + L.ml);
  hipLaunchKernelGGL(up_block_mass_kernel, dim3((unsigned)t.nb_tot), dim3(256), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq, lb,
                     lb + t.ml_pairs, reinterpret_cast<const float*>(wsb(ws) + L.wt),
                     reinterpret_cast<const float2*>(wsb(ws) + L.cs),
                     reinterpret_cast<const float2*>(wsb(ws) + L.rs),
                     reinterpret_cast<double*>(wsb(ws) + L.mass));
  return hipGetLastError();
}

hipError_t launch_block_mass_pairs(const ScoreShape& s, const Totals& t, void* ws,
                                   const ScoreWs& L, hipStream_t st) {
  if (t.nb_tot == 0) return hipSuccess;
  hipLaunchKernelGGL(up_block_mass_pairs_kernel, dim3((unsigned)t.nb_tot), dim3(256), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B, s.Hq,
                     reinterpret_cast<const float2*>(wsb(ws) + L.ml),
                     reinterpret_cast<const float2*>(wsb(ws) + L.rs),
                     reinterpret_cast<double*>(wsb(ws) + L.mass));
  return hipGetLastError();
}

hipError_t launch_normalize(const ScoreShape& s, const Totals& t, void* ws, const ScoreWs& L,
                            float* scores, hipStream_t st) {
  if (s.B == 0 || t.nb_tot == 0) return hipSuccess;
  hipLaunchKernelGGL(up_normalize_kernel, dim3(s.B), dim3(256), 0, st,
                     reinterpret_cast<const WsHeader*>(wsb(ws)),
                     reinterpret_cast<const ReqPlan*>(wsb(ws) + L.plan), s.B,
                     reinterpret_cast<const double*>(wsb(ws) + L.mass), scores);
  return hipGetLastError();
}

}  // namespace up

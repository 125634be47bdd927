// Index arithmetic of the attention kernels (consumer.hip: the 8-wave kernel W8 and
// the 4-wave kernel W4): which request, heads and token tiles a workgroup and its
// waves take, where every global-to-LDS copy reads and lands, and where every operand
// read and output store goes.  The kernels call these functions and nothing else for
// their addresses; a host replay (tests/attn_replay.cpp, built with g++) calls the same
// functions for every workgroup, wave, lane and stage of a launch and checks each
// access against its buffer, the ring's stage hand-over and the operand layouts.
#pragma once
#include <cstdint>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define UP_HD __host__ __device__ __forceinline__
#else
#define UP_HD inline
#endif

namespace up {
namespace attn {

// Largest Hkv of the 8-wave kernel (per-head LDS slots of the layout pass's key norms).
constexpr int kMaxKvHeads = 256;
// The 8-wave kernel serves d = 64 and 128 up to kMaxKvHeads kv heads.
constexpr bool w8_serves(int d, int Hkv) { return (d == 64 || d == 128) && Hkv <= kMaxKvHeads; }

// Request holding padded row / tile x: the largest i in [0, B) with off[i] <= x
// (empty requests share their successor's offset and are skipped).  off[B] > x.
UP_HD int request_of(const int32_t* off, int B, int64_t x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// 16-byte granule swizzles.  The LDS serves a 16-byte read to 16 lanes per clock over
// 64 banks; the 16 lanes of a group read 16 consecutive rows at one logical granule,
// which the XOR spreads over 16 distinct bank groups: by row & 15 for K rows of 256
// bytes or more, by (row >> 1) & 7 for 128-byte rows (odd rows sit half a bank cycle
// further on).
template <int D>
UP_HD int k_swz(int key) {
  return (D / 8 >= 16) ? (key & 15) : ((key >> 1) & 7);
}
UP_HD int v128_swz(int row) { return (row >> 1) & 7; }
// V^T rows of 64 bytes (32 tokens): granule g of row r sits at g ^ ((r >> 2) & 3), which
// spreads the 16 rows one 16-lane group reads over all 64 banks.
UP_HD int v64_swz(int row) { return (row >> 2) & 3; }

// Token stored at position t of the transposed v: inside each 16-token group bits 2
// and 3 are swapped, so that the 8 keys a lane half contracts in one MFMA step (the
// P^T register layout) are 8 adjacent positions.  (An involution.)
UP_HD int swap_bits23(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// Eight waves (two per SIMD) share one ring of NS stages of 64 keys: the K tile
// [64][D] (row bytes KRB) and the V^T tile [D][64] (row bytes 128).  A (query head,
// 64-token tile) pair is two waves of 32 query rows.
template <int D>
struct W8 {
  static constexpr int NW = 8, NT = 64 * NW, NS = 4, UK = 64;
  static constexpr int DS = D / 16;        // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;        // 32-row tiles of O^T
  static constexpr int KRB = 2 * D;        // K tile row bytes
  static constexpr int KB = UK * KRB;      // K tile bytes
  static constexpr int VRB = 2 * UK;       // V^T tile row bytes
  static constexpr int VB = D * VRB;       // V^T tile bytes
  static constexpr int SB = KB + VB;       // stage bytes
  static constexpr int KSPT = KB / (NT * 16);   // 16-byte copies per lane per stage, K
  static constexpr int VSPT = VB / (NT * 16);   // and V^T
  static constexpr int SPT = KSPT + VSPT;
  static_assert(KB % (NT * 16) == 0 && VB % (NT * 16) == 0, "whole copy rounds");
  static_assert(2 * SPT < 64, "vmcnt range");
  static_assert(NS * SB <= 160 * 1024, "LDS");

  // Copy q of a stage, thread tid: 16 bytes land at stage byte q NT 16 + 16 tid (the
  // wave's base below plus 16 per lane) and come from this element offset, counted
  // from the stage's first K row (K) or from its first token of V^T row 0 (V^T).
  UP_HD static int k_src(int q, int tid) {
    const int o = q * NT * 16 + tid * 16;
    const int key = o / KRB;
    const int gr = ((o % KRB) / 16) ^ k_swz<D>(key);
    return key * D + gr * 8;
  }
  UP_HD static int64_t v_src(int q, int tid, int64_t Rp) {
    const int o = q * NT * 16 + tid * 16;
    const int row = o / VRB;
    const int gr = ((o % VRB) / 16) ^ v128_swz(row);
    return (int64_t)row * Rp + gr * 8;
  }
  // Stage byte of lane 0's 16 bytes for copy q of a wave (the M0 base of the copy).
  UP_HD static uint32_t k_dst(int q, int wave) { return (uint32_t)(q * NT * 16 + wave * 1024); }
  UP_HD static uint32_t v_dst(int q, int wave) {
    return (uint32_t)(KB + q * NT * 16 + wave * 1024);
  }
  // Operand reads, stage bytes.  K: row tile kt (keys 32 kt + l32) adds kt 32 KRB;
  // lane half h, k-step s reads d-elements [h D/2 + 8 s, +8).
  UP_HD static uint32_t k_rd(int l32, int half, int s) {
    return (uint32_t)(l32 * KRB + 16 * ((half * DS + s) ^ k_swz<D>(l32)));
  }
  // V^T: granule j (tokens [8 j, 8 j + 8) of the stage in stored order) of row l32;
  // row tile dt of the head dimension adds dt 32 VRB (dt 32 leaves the swizzle alone).
  UP_HD static uint32_t v_rd(int l32, int j) {
    return (uint32_t)(KB + l32 * VRB + 16 * (j ^ v128_swz(l32)));
  }
};

// Four waves (one per SIMD at d = 256) share one ring of NS stages of 32 keys: the K
// tile [32][D] and the V^T tile [D][32] (row bytes 64).  Each wave holds one query head's
// 32-token tile.
template <int D>
struct W4 {
  static constexpr int NW = 4, NT = 64 * NW, NS = 4, UK = 32;
  static constexpr int DS = D / 16;        // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;        // 32-row tiles of O^T
  static constexpr int KRB = 2 * D;        // K tile row bytes
  static constexpr int KB = UK * KRB;      // K tile bytes
  static constexpr int VRB = 2 * UK;       // V^T tile row bytes
  static constexpr int VB = D * VRB;       // V^T tile bytes
  static constexpr int SB = KB + VB;       // stage bytes
  static constexpr int KSPT = KB / (NT * 16);   // 16-byte copies per lane per stage, K
  static constexpr int VSPT = VB / (NT * 16);   // and V^T
  static constexpr int SPT = KSPT + VSPT;
  static_assert(KB % (NT * 16) == 0 && VB % (NT * 16) == 0, "whole copy rounds");
  static_assert(2 * SPT < 64, "vmcnt range");
  static_assert(NS * SB <= 160 * 1024, "LDS");

  // Copy q of a stage, thread tid: as in W8 (element offsets from the stage's first K
  // row, or from its first token of V^T row 0).
  UP_HD static int k_src(int q, int tid) {
    const int o = q * NT * 16 + tid * 16;
    const int key = o / KRB;
    const int gr = ((o % KRB) / 16) ^ k_swz<D>(key);
    return key * D + gr * 8;
  }
  UP_HD static int64_t v_src(int q, int tid, int64_t Rp) {
    const int o = q * NT * 16 + tid * 16;
    const int row = o / VRB;
    const int gr = ((o % VRB) / 16) ^ v64_swz(row);
    return (int64_t)row * Rp + gr * 8;
  }
  UP_HD static uint32_t k_dst(int q, int wave) { return (uint32_t)(q * NT * 16 + wave * 1024); }
  UP_HD static uint32_t v_dst(int q, int wave) {
    return (uint32_t)(KB + q * NT * 16 + wave * 1024);
  }
  // Operand reads, stage bytes: K row l32 (the stage's key l32), lane half h, k-step s
  // reads d-elements [h D/2 + 8 s, +8); V^T granule j of row l32 (row tile dt adds
  // dt 32 VRB).
  UP_HD static uint32_t k_rd(int l32, int half, int s) {
    return (uint32_t)(l32 * KRB + 16 * ((half * DS + s) ^ k_swz<D>(l32)));
  }
  UP_HD static uint32_t v_rd(int l32, int j) {
    return (uint32_t)(KB + l32 * VRB + 16 * (j ^ v64_swz(l32)));
  }
};

// Launch layouts of the tile slots (blockIdx.y).  A request's slots are its workgroup
// tiles, heaviest (last) first; tp is the prefix of the requests' slot counts.  With
// window block statistics, the first k_i slots of request i hold its window rows (wp is
// the prefix of k_i): one launch takes those (kSlotsWindow) and another the rest
// (kSlotsRest); kSlotsAll takes every slot.
constexpr int kSlotsAll = 0, kSlotsWindow = 1, kSlotsRest = 2;

// Slot by of a launch in the given layout -> request i and slot j of the request.
UP_HD void slot_of(int mode, int by, int B, const int32_t* tp, const int32_t* wp, int& i,
                   int& j) {
  if (mode == kSlotsAll) {
    i = request_of(tp, B, by);
    j = by - tp[i];
  } else if (mode == kSlotsWindow) {
    i = request_of(wp, B, by);
    j = by - wp[i];
  } else {
    // the rest: request i's slots start at tp[i] - wp[i] and skip its k_i window slots
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tp[mid] - wp[mid] <= by) lo = mid;
      else hi = mid - 1;
    }
    i = lo;
    j = by - (tp[i] - wp[i]) + (wp[i + 1] - wp[i]);
  }
}

// Workgroup (blockIdx.x = kv head x query-head quad, blockIdx.y = tile slot).
struct Wg {
  int g, quad, i, L, wt, ntile, tile0, nst;
  int64_t pbase;
};
UP_HD Wg wg_of(int bx, int by, int Hq, int Hkv, int HQ, int TT, int B, const int32_t* cu,
               const int32_t* po, const int32_t* tp, int mode = kSlotsAll,
               const int32_t* wp = nullptr, int tile_shift = 6) {
  Wg w;
  const int gsz = Hq / Hkv, quads = gsz / HQ;
  w.g = bx / quads;
  w.quad = bx - w.g * quads;
  int j = 0;
  slot_of(mode, by, B, tp, wp, w.i, j);
  w.L = cu[w.i + 1] - cu[w.i];
  const int nwt = tp[w.i + 1] - tp[w.i];
  w.wt = nwt - 1 - j;   // heaviest tile first
  w.ntile = (w.L + (1 << tile_shift) - 1) >> tile_shift;   // tiles of the request
  w.tile0 = w.wt * TT;
  w.nst = w.tile0 + TT < w.ntile ? w.tile0 + TT : w.ntile;   // key stages of the workgroup
  w.pbase = po[w.i];
  return w;
}

// A wave's query head, 64-token tile (its diagonal stage) and which 32 rows of it.
struct Wv {
  int head, tw, sub;
  bool act;
};
UP_HD Wv wave_of(const Wg& w, int wave, int Hq, int Hkv, int HQ) {
  Wv v;
  const int gsz = Hq / Hkv;
  const int pair = wave >> 1;
  v.sub = wave & 1;
  v.head = w.g * gsz + w.quad * HQ + pair % HQ;
  v.tw = w.tile0 + pair / HQ;
  v.act = v.tw < w.ntile;
  return v;
}
// Request-local token of a wave's query row (lane column l32).
UP_HD int query_token(const Wv& v, int l32) { return v.tw * 64 + v.sub * 32 + l32; }

// The 4-wave kernel's waves: query head HQ-major within the quad, one 32-token tile
// each (wg_of with tile_shift 5).
UP_HD Wv wave4_of(const Wg& w, int wave, int Hq, int Hkv, int HQ) {
  Wv v;
  const int gsz = Hq / Hkv;
  v.sub = 0;
  v.head = w.g * gsz + w.quad * HQ + wave % HQ;
  v.tw = w.tile0 + wave / HQ;
  v.act = v.tw < w.ntile;
  return v;
}
UP_HD int query_token4(const Wv& v, int l32) { return v.tw * 32 + l32; }
template <int D>
UP_HD int64_t q_src4(const Wg& w, const Wv& v, int l32, int half, int64_t Rp) {
  return ((int64_t)v.head * Rp + w.pbase + v.tw * 32 + l32) * D + half * (D / 2);
}
// Element offsets of the 32-key K and V^T stage st of kv head g.
template <int D>
UP_HD int64_t k_stage4(const Wg& w, int st, int64_t Rp) {
  return ((int64_t)w.g * Rp + w.pbase) * D + (int64_t)st * 32 * D;
}
template <int D>
UP_HD int64_t v_stage4(const Wg& w, int st, int64_t Rp) {
  return (int64_t)w.g * D * Rp + w.pbase + (int64_t)st * 32;
}
template <int D>
UP_HD int64_t out_index4(const int32_t* cu, const Wg& w, const Wv& v, int l32, int Hq, int dv) {
  return (((int64_t)cu[w.i] + query_token4(v, l32)) * Hq + v.head) * D + dv;
}
// Element offset of a query row's operand in the rotated copy qr [Hq][Rp][D].
template <int D>
UP_HD int64_t q_src(const Wg& w, const Wv& v, int l32, int half, int64_t Rp) {
  return ((int64_t)v.head * Rp + w.pbase + query_token(v, l32)) * D + half * (D / 2);
}
// Key of register e of lane half h in half-step hs of a 32x32 MFMA result (row
// 8 (e / 4) + 4 h + e % 4 of the tile).
UP_HD int acc_key(int hs, int e, int half) { return hs * 32 + 8 * (e >> 2) + 4 * half + (e & 3); }
// Element offsets of the K and V^T stage st of kv head g in kr [Hkv][Rp][D] and
// vt [Hkv][D][Rp].
template <int D>
UP_HD int64_t k_stage(const Wg& w, int st, int64_t Rp) {
  return ((int64_t)w.g * Rp + w.pbase + (int64_t)st * 64) * D;
}
template <int D>
UP_HD int64_t v_stage(const Wg& w, int st, int64_t Rp) {
  return (int64_t)w.g * D * Rp + w.pbase + (int64_t)st * 64;
}
// Entry of the key-norm table kn [Hkv][Rp / 64] for stage st.
UP_HD int64_t kn_index(const Wg& w, int st, int64_t Rp) {
  return (int64_t)w.g * (Rp / 64) + (w.pbase >> 6) + st;
}
// Element offset of output dims [dv, dv + 4) of a query row in out [R][Hq][D].
template <int D>
UP_HD int64_t out_index(const int32_t* cu, const Wg& w, const Wv& v, int l32, int Hq, int dv) {
  return (((int64_t)cu[w.i] + query_token(v, l32)) * Hq + v.head) * D + dv;
}

// Window-row block statistics (the attention's fused form of the block scores).  The
// window is the last W = min(n, L) tokens of a request; window row wr of query head
// head (kv head g, gs = Hq / Hkv query heads per kv head) is term
// g gs W + wr gs + (head - g gs) of the request's [Hkv][gs W] rows.
UP_HD int64_t win_term(int g, int gs, int W, int wr, int head) {
  return (int64_t)g * gs * W + (int64_t)wr * gs + (head - g * gs);
}
// A wave's 32-key half-step hs closes a G-key block at its end, or is the wave's last.
UP_HD bool stats_flush(int hs, int last, int G) { return ((hs + 1) * 32) % G == 0 || hs == last; }
UP_HD int stats_block(int hs, int G) { return (hs * 32) / G; }
// First block wholly after a wave whose last half-step is `last`.
UP_HD int stats_tail_first(int last, int G) { return ((last + 1) * 32 - 1) / G + 1; }

}  // namespace attn
}  // namespace up
